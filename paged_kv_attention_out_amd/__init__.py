"""Attention over a paged KV cache for AMD MI355X (gfx950).

The compute lives in libpkv.so (HIP kernels behind the C ABI of
include/pkv.h); this package holds its build script, a thin ctypes binding
and the seeded input generators used by the tests and the benchmark.
"""

from ._lib import (  # noqa: F401
    DecodeGraphs,
    PKVError,
    decode_workspace,
    lib,
    pkv_decode_split_tokens,
    pkv_decode_graphs_create,
    pkv_decode_graphs_workspace_bytes,
    pkv_decode_metadata,
    pkv_decode_multi_workspace_bytes,
    pkv_decode_step,
    pkv_decode_step_noalloc,
    pkv_decode_step_noalloc_max_bytes,
    pkv_decode_workspace_bytes,
    pkv_paged_attn_decode,
    pkv_paged_attn_decode_multi,
    pkv_paged_attn_decode_shared,
    pkv_paged_attn_decode_shared_workspace_bytes,
    pkv_paged_attn_prefill,
    pkv_prefill_metadata,
    pkv_prefill_workspace_bytes,
    pkv_ref_stream_read,
    prefill_workspace,
    pkv_store_kv,
    strerror,
    version,
)

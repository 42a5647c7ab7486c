"""Thin ctypes binding of libpkv.so (declared in include/pkv.h).

The functions carry the C names and only marshal arguments: torch tensors
become device pointers, the current torch stream becomes the hipStream_t,
and a non-zero status becomes a ``PKVError``.  Every step of the
computation runs in the HIP kernels of libpkv.so; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOSPACE, PKV_EHIP = 0, 1, 2, 3, 4

# Exported symbols and their C signatures, in header order.
_c_void_p, _i32, _i64, _f32, _size = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_store_kv": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                    _c_void_p, _i64, _i32, _i32, _c_void_p]),
    "pkv_decode_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_split_tokens": (_i32, [_i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _c_void_p, _i32, _c_void_p, _i32, _i32,
        _i32, _i32, _i32, _f32, _i32, _c_void_p, _c_void_p, _size, _c_void_p]),
    "pkv_paged_attn_prefill": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p, _i32,
        _i64, _c_void_p, _i32, _i32, _i32, _i32, _f32, _c_void_p, _c_void_p, _size,
        _c_void_p]),
    "pkv_prefill_workspace_bytes": (_size, []),
    "pkv_prefill_metadata": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _c_void_p, _i32, _i32,
                                             _i32, _c_void_p, _c_void_p, _c_void_p]),
    "pkv_decode_metadata": (ctypes.c_int, [_c_void_p, _i32, _c_void_p, _i32, _i32, _c_void_p,
                                            _c_void_p]),
    "pkv_decode_step": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_void_p,
        _c_void_p, _size, _c_void_p]),
    "pkv_decode_step_noalloc": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _c_void_p,
        _c_void_p]),
    "pkv_decode_step_noalloc_max_bytes": (_size, []),
    "pkv_paged_attn_decode_shared": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32,
        _i32, _i32, _f32, _i32, _c_void_p, _c_void_p, _size, _c_void_p]),
    "pkv_paged_attn_decode_shared_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                             _i32]),
    "pkv_decode_graphs_workspace_bytes": (_size, [_c_void_p, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_graphs_create": (ctypes.c_int, [
        _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i32, _i64, _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _f32, _c_void_p,
        _c_void_p, _size, ctypes.POINTER(ctypes.c_void_p)]),
    "pkv_decode_graphs_replay": (ctypes.c_int, [_c_void_p, _i32, _c_void_p,
                                                 ctypes.POINTER(ctypes.c_int32)]),
    "pkv_decode_graphs_destroy": (None, [_c_void_p]),
    "pkv_decode_multi_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode_multi": (ctypes.c_int, [
        _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i64, _c_void_p, _i32, _c_void_p, _i32,
        _i32, _i32, _i32, _i32, _f32, _i32, _c_void_p, _c_void_p, _size, _c_void_p]),
    # include/pkv_ref.h: the streaming-read reference (measurement only)
    "pkv_ref_stream_sink_words": (_size, [_i32]),
    "pkv_ref_stream_read": (ctypes.c_int, [_c_void_p, _size, _i32, _c_void_p, _c_void_p]),
}

_LIB: Optional[ctypes.CDLL] = None


class PKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libpkv.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_attention_out_amd.build`"
                " (there is no non-HIP fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def strerror(status: int) -> str:
    return lib().pkv_strerror(status).decode()


def version() -> str:
    return lib().pkv_version().decode()


def _check(status: int, where: str):
    if status != PKV_OK:
        raise PKVError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t: torch.Tensor, expected, name: str) -> None:
    """Raise ValueError unless ``t`` has ``len(expected)`` dimensions whose
    sizes equal the non-None entries of ``expected``."""
    if t.dim() != len(expected) or any(e is not None and int(s) != int(e)
                                       for s, e in zip(t.shape, expected)):
        shown = tuple("*" if e is None else int(e) for e in expected)
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shown}")


def _pool_shape(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_pages, page_size, Hkv, d) of the K pool; V must have the same."""
    _shape(k_cache, (None, None, None, None), "k_cache")
    _shape(v_cache, tuple(k_cache.shape), "v_cache")
    return tuple(int(x) for x in k_cache.shape)


def _table_rows(page_table: torch.Tensor, num_seqs: int) -> None:
    _shape(page_table, (None, None), "page_table")
    if page_table.shape[0] < num_seqs:
        raise ValueError(f"page_table has {page_table.shape[0]} rows for {num_seqs} sequences")


def _numel(t: torch.Tensor, n: int, name: str, at_least: bool = False) -> None:
    if t.dim() != 1 or (t.numel() < n if at_least else t.numel() != n):
        want = f"at least {n}" if at_least else f"{n}"
        raise ValueError(f"{name} must be 1-D with {want} entries, has shape {tuple(t.shape)}")


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def pkv_store_kv(k_new: torch.Tensor, v_new: torch.Tensor, out_loc: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Scatter k_new/v_new ``[T, Hkv, d]`` into pool rows ``out_loc``."""
    _, _, hkv, hd = _pool_shape(k_cache, v_cache)
    _numel(out_loc, out_loc.numel(), "out_loc")
    _shape(k_new, (out_loc.numel(), hkv, hd), "k_new")
    _shape(v_new, (out_loc.numel(), hkv, hd), "v_new")
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, n)
    _dev(out_loc, torch.int32, "out_loc")
    T = out_loc.numel()
    Hkv, d = k_cache.shape[-2], k_cache.shape[-1]
    slots = k_cache.numel() // (Hkv * d)
    _check(lib().pkv_store_kv(_ptr(k_new), _ptr(v_new), _ptr(out_loc), T, _ptr(k_cache),
                              _ptr(v_cache), slots, Hkv, d, _stream(k_cache)), "pkv_store_kv")


def pkv_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                               head_dim: int, max_seq_len: int, split_tokens: int = 0) -> int:
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 max_seq_len, split_tokens))


def pkv_decode_split_tokens(num_seqs: int, num_kv_heads: int, max_seq_len: int,
                            split_tokens: int = 0) -> int:
    return int(lib().pkv_decode_split_tokens(num_seqs, num_kv_heads, max_seq_len, split_tokens))


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                     split_tokens=0, device="cuda") -> Optional[torch.Tensor]:
    """A zero-filled workspace of the size the decode call needs (or None)."""
    nbytes = pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_seq_len, split_tokens)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace,
                         q_dims: int = 3):
    """Shapes of a decode call checked against each other before any launch
    (q ``[B, Hq, d]``, or ``[B, q_len, Hq, d]`` for multi-token decode)."""
    _shape(q, (None,) * q_dims, "q")
    B, hq, d = int(q.shape[0]), int(q.shape[-2]), int(q.shape[-1])
    _, _, hkv, hd = _pool_shape(k_cache, v_cache)
    if hd != d:
        raise ValueError(f"k_cache head_dim {hd} differs from q head_dim {d}")
    if hkv == 0 or hq % hkv != 0:
        raise ValueError(f"{hq} query heads are not a multiple of {hkv} KV heads")
    _table_rows(page_table, B)
    _numel(seq_lens, B, "seq_lens")
    if out is not None:
        _shape(out, tuple(q.shape), "out")
    if workspace is not None and (not workspace.is_cuda or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    return B, hkv, d


def pkv_paged_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                          softmax_scale: float, out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          split_tokens: int = 0) -> torch.Tensor:
    """Decode attention; q ``[B, Hq, d]`` -> out ``[B, Hq, d]`` (bf16)."""
    _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace)
    _dev(q, torch.bfloat16, "q")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(page_table, torch.int32, "page_table")
    _dev(seq_lens, torch.int32, "seq_lens")
    B, Hq, d = q.shape
    num_pages, ps, Hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, d, max_seq_len, split_tokens, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), ps, num_pages, _ptr(page_table),
        page_table.shape[1], _ptr(seq_lens), B, max_seq_len, Hq, Hkv, d, softmax_scale,
        split_tokens, _ptr(out), _ptr(workspace), ws_bytes, _stream(q)), "pkv_paged_attn_decode")
    return out


def pkv_decode_step(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    out_loc: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                    softmax_scale: float, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None,
                    split_tokens: int = 0) -> torch.Tensor:
    """Store the new token's K/V rows and run decode attention in one call."""
    B, hkv, d = _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace)
    _shape(k_new, (B, hkv, d), "k_new")
    _shape(v_new, (B, hkv, d), "v_new")
    _numel(out_loc, B, "out_loc")
    for t, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                    (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, name)
    for t, name in ((out_loc, "out_loc"), (page_table, "page_table"), (seq_lens, "seq_lens")):
        _dev(t, torch.int32, name)
    B, Hq, d = q.shape
    num_pages, ps, Hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if workspace is None:
        workspace = decode_workspace(B, Hq, Hkv, d, max_seq_len, split_tokens, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_step(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out_loc), _ptr(k_cache), _ptr(v_cache), ps,
        num_pages, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, max_seq_len, Hq,
        Hkv, d, softmax_scale, split_tokens, _ptr(out), _ptr(workspace), ws_bytes, _stream(q)),
        "pkv_decode_step")
    return out


def pkv_decode_step_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            out_loc: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                            softmax_scale: float, out: torch.Tensor,
                            split_tokens: int = 0) -> torch.Tensor:
    """pkv_decode_step with the library's fixed scratch instead of a
    workspace; the caller passes ``out`` (nothing is allocated)."""
    B, hkv, d = _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, None)
    _shape(k_new, (B, hkv, d), "k_new")
    _shape(v_new, (B, hkv, d), "v_new")
    _numel(out_loc, B, "out_loc")
    for t, name in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                    (v_cache, "v_cache"), (out, "out")):
        _dev(t, torch.bfloat16, name)
    for t, name in ((out_loc, "out_loc"), (page_table, "page_table"), (seq_lens, "seq_lens")):
        _dev(t, torch.int32, name)
    Hq = q.shape[1]
    num_pages, ps = k_cache.shape[0], k_cache.shape[1]
    _check(lib().pkv_decode_step_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out_loc), _ptr(k_cache), _ptr(v_cache), ps,
        num_pages, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, max_seq_len, Hq,
        hkv, d, softmax_scale, split_tokens, _ptr(out), _stream(q)), "pkv_decode_step_noalloc")
    return out


def pkv_decode_step_noalloc_max_bytes() -> int:
    return int(lib().pkv_decode_step_noalloc_max_bytes())


def pkv_paged_attn_decode_shared_workspace_bytes(num_seqs: int, num_q_heads: int,
                                                 num_kv_heads: int, head_dim: int,
                                                 max_seq_len: int, max_shared_len: int,
                                                 split_tokens: int = 0) -> int:
    return int(lib().pkv_paged_attn_decode_shared_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len, max_shared_len,
        split_tokens))


def pkv_paged_attn_decode_shared(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 page_table: torch.Tensor, seq_lens: torch.Tensor,
                                 max_seq_len: int, cu_groups: torch.Tensor,
                                 shared_lens: torch.Tensor, max_group_size: int,
                                 max_shared_len: int, softmax_scale: float,
                                 out: Optional[torch.Tensor] = None,
                                 k_new: Optional[torch.Tensor] = None,
                                 v_new: Optional[torch.Tensor] = None,
                                 out_loc: Optional[torch.Tensor] = None,
                                 workspace: Optional[torch.Tensor] = None,
                                 split_tokens: int = 0) -> torch.Tensor:
    """Decode (with the new token's store when k_new/v_new/out_loc are
    given) over requests grouped by shared prefix: group g is requests
    cu_groups[g] .. cu_groups[g+1]-1, sharing their first shared_lens tokens."""
    B, hkv, d = _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace)
    _shape(cu_groups, (None,), "cu_groups")
    if cu_groups.numel() < 2:
        raise ValueError("cu_groups needs at least two entries")
    _numel(shared_lens, B, "shared_lens")
    if k_new is not None:
        _shape(k_new, (B, hkv, d), "k_new")
        _shape(v_new, (B, hkv, d), "v_new")
        _numel(out_loc, B, "out_loc")
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            _dev(t, torch.bfloat16, name)
        _dev(out_loc, torch.int32, "out_loc")
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, torch.bfloat16, name)
    for t, name in ((page_table, "page_table"), (seq_lens, "seq_lens"), (cu_groups, "cu_groups"),
                    (shared_lens, "shared_lens")):
        _dev(t, torch.int32, name)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if workspace is None:
        nbytes = pkv_paged_attn_decode_shared_workspace_bytes(
            B, q.shape[1], hkv, d, max_seq_len, max_shared_len, split_tokens)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    num_pages, ps = k_cache.shape[0], k_cache.shape[1]
    _check(lib().pkv_paged_attn_decode_shared(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out_loc), _ptr(k_cache), _ptr(v_cache), ps,
        num_pages, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), B, max_seq_len,
        _ptr(cu_groups), _ptr(shared_lens), cu_groups.numel() - 1, max_group_size,
        max_shared_len, q.shape[1], hkv, d, softmax_scale, split_tokens, _ptr(out),
        _ptr(workspace), ws_bytes, _stream(q)), "pkv_paged_attn_decode_shared")
    return out


def _buckets(buckets):
    arr = (ctypes.c_int32 * len(buckets))(*[int(b) for b in buckets])
    return arr, len(buckets)


def pkv_decode_graphs_workspace_bytes(buckets, num_q_heads: int, num_kv_heads: int,
                                      head_dim: int, max_seq_len: int) -> int:
    arr, n = _buckets(buckets)
    return int(lib().pkv_decode_graphs_workspace_bytes(arr, n, num_q_heads, num_kv_heads,
                                                       head_dim, max_seq_len))


class DecodeGraphs:
    """Handle of pkv_decode_graphs_create: one captured decode step per
    batch-size bucket over fixed buffers sized for the largest bucket.  The
    buffers (and the workspace) are kept referenced for the graphs' life."""

    def __init__(self, handle, buckets, keep):
        self._handle = handle
        self.buckets = sorted(int(b) for b in buckets)
        self._keep = keep

    def replay(self, num_seqs: int, stream=None) -> int:
        """Replay the smallest bucket >= num_seqs on the current stream (or
        ``stream``); returns the bucket used.  Rows num_seqs .. bucket-1 of
        seq_lens must hold padding (<= 0)."""
        used = ctypes.c_int32(0)
        s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        _check(lib().pkv_decode_graphs_replay(self._handle, num_seqs, s, ctypes.byref(used)),
               "pkv_decode_graphs_replay")
        return int(used.value)

    def destroy(self) -> None:
        if self._handle is not None:
            lib().pkv_decode_graphs_destroy(self._handle)
            self._handle = None
            self._keep = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def pkv_decode_graphs_create(buckets, q: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, page_table: torch.Tensor,
                             seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float,
                             out: torch.Tensor, k_new: Optional[torch.Tensor] = None,
                             v_new: Optional[torch.Tensor] = None,
                             out_loc: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None) -> DecodeGraphs:
    """Capture the decode step (fused store when k_new/v_new/out_loc are
    given) once per bucket over fixed buffers sized for the largest bucket;
    ``workspace`` None uses the library's fixed scratch."""
    B, hkv, d = _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace)
    if B < max(int(b) for b in buckets):
        raise ValueError(f"buffers hold {B} rows, fewer than the largest bucket")
    fused = k_new is not None
    if fused:
        _shape(k_new, (B, hkv, d), "k_new")
        _shape(v_new, (B, hkv, d), "v_new")
        _numel(out_loc, B, "out_loc")
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            _dev(t, torch.bfloat16, name)
        _dev(out_loc, torch.int32, "out_loc")
    for t, name in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _dev(t, torch.bfloat16, name)
    for t, name in ((page_table, "page_table"), (seq_lens, "seq_lens")):
        _dev(t, torch.int32, name)
    arr, n = _buckets(buckets)
    handle = ctypes.c_void_p()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    num_pages, ps = k_cache.shape[0], k_cache.shape[1]
    _check(lib().pkv_decode_graphs_create(
        arr, n, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out_loc), _ptr(k_cache), _ptr(v_cache),
        ps, num_pages, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), max_seq_len,
        q.shape[1], hkv, d, softmax_scale, _ptr(out), _ptr(workspace), ws_bytes,
        ctypes.byref(handle)), "pkv_decode_graphs_create")
    keep = (q, k_new, v_new, out_loc, k_cache, v_cache, page_table, seq_lens, out, workspace)
    return DecodeGraphs(handle, buckets, keep)


def pkv_decode_multi_workspace_bytes(num_seqs: int, q_len: int, num_q_heads: int,
                                     num_kv_heads: int, head_dim: int, max_seq_len: int,
                                     split_tokens: int = 0) -> int:
    return int(lib().pkv_decode_multi_workspace_bytes(num_seqs, q_len, num_q_heads,
                                                       num_kv_heads, head_dim, max_seq_len,
                                                       split_tokens))


def pkv_paged_attn_decode_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                page_table: torch.Tensor, seq_lens: torch.Tensor,
                                max_seq_len: int, softmax_scale: float,
                                out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None,
                                split_tokens: int = 0) -> torch.Tensor:
    """Multi-token decode; q ``[B, q_len, Hq, d]`` -> out ``[B, q_len, Hq, d]``
    (bf16); query token t of request r sits at position seq_lens[r] - q_len + t."""
    _check_decode_shapes(q, k_cache, v_cache, page_table, seq_lens, out, workspace, q_dims=4)
    _dev(q, torch.bfloat16, "q")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(page_table, torch.int32, "page_table")
    _dev(seq_lens, torch.int32, "seq_lens")
    B, L, Hq, d = q.shape
    num_pages, ps, Hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    if workspace is None:
        nbytes = pkv_decode_multi_workspace_bytes(B, L, Hq, Hkv, d, max_seq_len, split_tokens)
        if nbytes:
            workspace = torch.zeros(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_multi(
        _ptr(q), L, _ptr(k_cache), _ptr(v_cache), ps, num_pages, _ptr(page_table),
        page_table.shape[1], _ptr(seq_lens), B, max_seq_len, Hq, Hkv, d, softmax_scale,
        split_tokens, _ptr(out), _ptr(workspace), ws_bytes, _stream(q)),
        "pkv_paged_attn_decode_multi")
    return out


def pkv_prefill_metadata(seq_lens: torch.Tensor, prefix_lens: torch.Tensor,
                         page_table: torch.Tensor, page_size: int, max_tokens: int,
                         cu_seqlens_q: Optional[torch.Tensor] = None,
                         out_loc: Optional[torch.Tensor] = None):
    """cu_seqlens_q ``[B+1]`` and out_loc ``[max_tokens]`` of a prefill batch."""
    _numel(seq_lens, seq_lens.numel(), "seq_lens")
    _numel(prefix_lens, seq_lens.numel(), "prefix_lens")
    _table_rows(page_table, seq_lens.numel())
    if cu_seqlens_q is not None:
        _numel(cu_seqlens_q, seq_lens.numel() + 1, "cu_seqlens_q", at_least=True)
    if out_loc is not None:
        _numel(out_loc, max_tokens, "out_loc", at_least=True)
    for t, name in ((seq_lens, "seq_lens"), (prefix_lens, "prefix_lens"),
                    (page_table, "page_table")):
        _dev(t, torch.int32, name)
    B = seq_lens.numel()
    if cu_seqlens_q is None:
        cu_seqlens_q = torch.empty(B + 1, dtype=torch.int32, device=seq_lens.device)
    if out_loc is None:
        out_loc = torch.empty(max(max_tokens, 1), dtype=torch.int32, device=seq_lens.device)
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    _dev(out_loc, torch.int32, "out_loc")
    _check(lib().pkv_prefill_metadata(
        _ptr(seq_lens), _ptr(prefix_lens), B, _ptr(page_table), page_table.shape[1], page_size,
        max_tokens, _ptr(cu_seqlens_q), _ptr(out_loc), _stream(seq_lens)),
        "pkv_prefill_metadata")
    return cu_seqlens_q, out_loc


def pkv_decode_metadata(seq_lens: torch.Tensor, page_table: torch.Tensor, page_size: int,
                        out_loc: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out_loc ``[B]``: the slot of each sequence's newest token."""
    _numel(seq_lens, seq_lens.numel(), "seq_lens")
    _table_rows(page_table, seq_lens.numel())
    if out_loc is not None:
        _numel(out_loc, seq_lens.numel(), "out_loc", at_least=True)
    _dev(seq_lens, torch.int32, "seq_lens")
    _dev(page_table, torch.int32, "page_table")
    B = seq_lens.numel()
    if out_loc is None:
        out_loc = torch.empty(max(B, 1), dtype=torch.int32, device=seq_lens.device)
    _dev(out_loc, torch.int32, "out_loc")
    _check(lib().pkv_decode_metadata(_ptr(seq_lens), B, _ptr(page_table), page_table.shape[1],
                                     page_size, _ptr(out_loc), _stream(seq_lens)),
           "pkv_decode_metadata")
    return out_loc


def pkv_ref_stream_read(src: torch.Tensor, blocks: int,
                        sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One plain streaming read of ``src`` (contiguous device memory, a
    multiple of 16 bytes) by ``blocks`` workgroups; returns the sink (one
    word per wavefront).  A bandwidth reference, not part of the path."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    words = int(lib().pkv_ref_stream_sink_words(blocks))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _numel(sink, words, "sink", at_least=True)
    _dev(sink, torch.int32, "sink")
    _check(lib().pkv_ref_stream_read(_ptr(src), nbytes, blocks, _ptr(sink), _stream(src)),
           "pkv_ref_stream_read")
    return sink


def pkv_prefill_workspace_bytes() -> int:
    return int(lib().pkv_prefill_workspace_bytes())


_PREFILL_WS = {}


def prefill_workspace(device: torch.device, stream: int) -> torch.Tensor:
    """A zeroed prefill workspace for one (device, stream).

    Every prefill call leaves its workspace zeroed again, so one buffer serves
    all calls that are ordered on that stream."""
    key = (device.index, stream)
    ws = _PREFILL_WS.get(key)
    if ws is None:
        ws = torch.zeros(pkv_prefill_workspace_bytes(), dtype=torch.uint8, device=device)
        _PREFILL_WS[key] = ws
    return ws


def pkv_paged_attn_prefill(q: torch.Tensor, cu_seqlens_q: torch.Tensor,
                           prefix_lens: torch.Tensor, max_q_len: int, max_seq_len: int,
                           k_cache: torch.Tensor, v_cache: torch.Tensor,
                           page_table: torch.Tensor, softmax_scale: float,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal prefill with prefix; q ``[T, Hq, d]`` -> out ``[T, Hq, d]``.

    ``workspace`` (uint8, zero before its first use) defaults to one buffer
    per (device, stream)."""
    _shape(q, (None, None, None), "q")
    _, _, hkv, hd = _pool_shape(k_cache, v_cache)
    if hd != q.shape[-1]:
        raise ValueError(f"k_cache head_dim {hd} differs from q head_dim {q.shape[-1]}")
    if hkv == 0 or q.shape[1] % hkv != 0:
        raise ValueError(f"{q.shape[1]} query heads are not a multiple of {hkv} KV heads")
    _numel(prefix_lens, prefix_lens.numel(), "prefix_lens")
    _numel(cu_seqlens_q, prefix_lens.numel() + 1, "cu_seqlens_q")
    _table_rows(page_table, prefix_lens.numel())
    if out is not None:
        _shape(out, tuple(q.shape), "out")
    _dev(q, torch.bfloat16, "q")
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(page_table, torch.int32, "page_table")
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q")
    _dev(prefix_lens, torch.int32, "prefix_lens")
    T, Hq, d = q.shape
    num_pages, ps, Hkv, _ = k_cache.shape
    B = prefix_lens.numel()
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.bfloat16, "out")
    stream = _stream(q)
    if workspace is None:
        workspace = prefill_workspace(q.device, stream)
    _dev(workspace, torch.uint8, "workspace")
    _check(lib().pkv_paged_attn_prefill(
        _ptr(q), _ptr(cu_seqlens_q), _ptr(prefix_lens), B, T, max_q_len, max_seq_len,
        _ptr(k_cache), _ptr(v_cache), ps, num_pages, _ptr(page_table), page_table.shape[1], Hq,
        Hkv, d, softmax_scale, _ptr(out), _ptr(workspace), workspace.numel(), stream),
        "pkv_paged_attn_prefill")
    return out

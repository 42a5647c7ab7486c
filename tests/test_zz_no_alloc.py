"""pkv_decode_step_noalloc -- the decode step for callers that cannot
allocate (its split partials go to the library's fixed per-GPU scratch) --
against pkv_decode_step with a caller workspace, through the C ABI: the
outputs and the pools must be bit-identical (same kernels, same split), and
within tolerance of the oracle, on two calls in a row, the second with a
smaller batch (the scratch keeps the first call's partials)."""

import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools

pytestmark = pytest.mark.gpu


def _both(w, split):
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    out_a = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale,
                                split_tokens=split)
    ka, va = w.k_cache.clone(), w.v_cache.clone()
    w.k_cache.copy_(k0)
    w.v_cache.copy_(v0)
    out_b = torch.full_like(w.q, 3.0)
    pkv.pkv_decode_step_noalloc(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale, out=out_b,
                                split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(ka.view(torch.int16), w.k_cache.view(torch.int16))
    assert torch.equal(va.view(torch.int16), w.v_cache.view(torch.int16))
    return assert_close(f64(out_b), ref, "no-alloc decode step")


@pytest.mark.parametrize("split", [0, 64])
def test_noalloc_decode_step_matches_workspace_call(split):
    assert pkv.pkv_decode_step_noalloc_max_bytes() == 32 << 20
    big = inputs.make_workload("llama_decode", device="cuda")
    small = inputs.build_decode(5, 16, 4, 128, 32, [1, 17, 300, 999, 2000], seed=91,
                                device="cuda", store_new=True)
    for name, w in (("llama_decode", big), ("5 requests, d=128", small)):
        need = pkv.pkv_decode_workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                              w.head_dim, w.max_seq_len, split)
        print(f"no-alloc step: {name}, split {split}, scratch use {need} bytes", flush=True)
        assert 0 < need <= pkv.pkv_decode_step_noalloc_max_bytes()
        print(_both(w, split))

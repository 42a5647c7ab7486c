"""The README's Python example, run as written on small batches and checked
against the oracle."""

import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools

pytestmark = pytest.mark.gpu


def test_readme_decode_step():
    B, Hq, Hkv, d = 6, 8, 2, 64
    w = inputs.build_decode(B, Hq, Hkv, d, 16, [1, 40, 300, 17, 1000, 64], seed=401,
                            device="cuda", store_new=True)
    ref_pools = host_pools(w)
    q, k_new, v_new, out_loc = w.q, w.k_new, w.v_new, w.out_loc
    k_cache, v_cache, page_table, seq_lens = w.k_cache, w.v_cache, w.page_table, w.seq_lens
    max_seq_len, scale = w.max_seq_len, w.scale

    ws = pkv.decode_workspace(B, Hq, Hkv, d, max_seq_len)
    out = pkv.pkv_decode_step(q, k_new, v_new, out_loc, k_cache, v_cache,
                              page_table, seq_lens, max_seq_len, scale, workspace=ws)
    torch.cuda.synchronize()
    ref = orc.decode(inputs.bf16_bits(w.q), *ref_pools, w.page_table_np, w.seq_lens_np, w.scale)
    print(assert_close(f64(out), ref, "readme decode step"))


def test_readme_prefill():
    w = inputs.build_prefill(3, 8, 2, 64, 16, [0, 37, 500], [70, 1, 130], seed=402,
                             device="cuda")
    ref_pools = host_pools(w)  # (the oracle's own store of the new rows)
    seq_lens = (w.prefix_lens + (w.cu_seqlens_q[1:] - w.cu_seqlens_q[:-1])).to(torch.int32)
    prefix_lens, page_table, page_size, T = w.prefix_lens, w.page_table, w.page_size, w.num_tokens
    k_new, v_new, k_cache, v_cache = w.k_new, w.v_new, w.k_cache, w.v_cache
    q, max_q_len, max_seq_len, scale = w.q, w.max_q_len, w.max_seq_len, w.scale

    cu, out_loc = pkv.pkv_prefill_metadata(seq_lens, prefix_lens, page_table, page_size, T)
    pkv.pkv_store_kv(k_new, v_new, out_loc, k_cache, v_cache)
    out = pkv.pkv_paged_attn_prefill(q, cu, prefix_lens, max_q_len, max_seq_len,
                                     k_cache, v_cache, page_table, scale)
    torch.cuda.synchronize()
    assert torch.equal(cu, w.cu_seqlens_q)
    assert torch.equal(out_loc[:T], w.out_loc)
    ref = orc.prefill_dense(inputs.bf16_bits(w.q), w.cu_seqlens_q.cpu().numpy(), w.prefix_lens_np,
                            *ref_pools, w.page_table_np, w.scale)
    print(assert_close(f64(out), ref, "readme prefill"))

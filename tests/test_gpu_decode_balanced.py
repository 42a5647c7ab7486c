"""Single-token decode of batches that need several rounds of units, with
the automatic split: the work is shared evenly by one round of workgroups
(pieces cut at 16-token boundaries, a partial per piece, merged per
request).  Every element of every live request against the oracle, empty
and negative lengths give zero rows, and the fused step keeps the pools
bit-exact.  Each batch needs at least four times more units than a round
of the GPU's resident waves holds, so the launch takes the balanced path."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from gpu_helpers import assert_close, compact, f64, host_pools
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

pytestmark = pytest.mark.gpu

# Units of max-length requests at or above 4 x 4096 (eight rounds of the
# 2,048 decode waves resident on this GPU) always take several rounds.
MAX_RESIDENT_WAVES = 4096


def _lengths(B, lo, hi, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    special = [0, 0, 7, 16, 17, 1]  # empty (the second made negative), short, block edges
    lens[1:1 + len(special)] = special
    return lens


def _check(w, out):
    got = f64(out)
    lens = w.seq_lens.cpu().numpy()
    live = [r for r in range(w.num_seqs) if lens[r] > 0]
    for r in range(w.num_seqs):
        if lens[r] <= 0:
            assert np.array_equal(got[r], np.zeros_like(got[r])), f"request {r} not zero"
    errs = []
    for i in range(0, len(live), 16):
        reqs = live[i:i + 16]
        kc, vc, table = compact(w, reqs)
        ref = orc.decode(inputs.bf16_bits(w.q)[reqs], kc, vc, table, lens[reqs], w.scale)
        errs.append(assert_close(got[reqs], ref, f"requests {reqs[0]}.."))
    return errs


CASES = [
    # B, hq, hkv, d, page_size, lengths lo..hi
    (96, 32, 8, 64, 16, 2000, 12000),
    (100, 16, 8, 128, 256, 1000, 9000),
    (48, 8, 1, 128, 32, 20000, 60000),
    (200, 4, 2, 64, 64, 100, 6000),
    (40, 16, 4, 64, 128, 4000, 30000),
    (256, 8, 8, 64, 16, 2000, 12000),   # one query head per KV head, the most requests
]


@pytest.mark.parametrize("B,hq,hkv,d,ps,lo,hi", CASES)
def test_balanced_decode(B, hq, hkv, d, ps, lo, hi):
    lens = _lengths(B, lo, hi, seed=B + hq + d + ps)
    split = pkv.pkv_decode_split_tokens(B, hkv, int(lens.max()))
    # units of max-length requests at the host split, over KV heads: beyond
    # four rounds of any resident wave count, so no one-round launch
    worst = B * (-(-int(lens.max()) // split)) * hkv
    assert worst >= 4 * MAX_RESIDENT_WAVES, "batch too small for several rounds"
    units = worst
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=B + d, device="cuda")
    w.seq_lens[2] = -3  # a negative length reads nothing and gives a zero row
    print(f"balanced: B={B} hq{hq} hkv{hkv} d{d} ps{ps} lens {lo}..{hi} split {split} "
          f"units {units}", flush=True)
    out = pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                    w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    print("max/mean err per 16 requests", _check(w, out))
    # deterministic: a second call gives the same bits
    out2 = pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                     w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_balanced_decode_step_fused_store():
    B, hq, hkv, d, ps = 96, 32, 8, 64, 16
    lens = _lengths(B, 2000, 12000, seed=5)
    lens[1], lens[2] = 1, 5  # every request of a step has its new token
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=9, device="cuda", store_new=True)
    kc_ref, vc_ref = host_pools(w)  # pools after the oracle's store
    out = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                              w.page_table, w.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(inputs.bf16_bits(w.k_cache), kc_ref), "K pool differs from the store"
    assert np.array_equal(inputs.bf16_bits(w.v_cache), vc_ref), "V pool differs from the store"
    print("max/mean err per 16 requests", _check(w, out))


def test_split_launch_beyond_256_requests():
    """257 requests: more than the balanced launch keeps in registers, so the
    split launch runs the several rounds; same checks."""
    B, hq, hkv, d, ps = 257, 16, 8, 64, 16
    lens = _lengths(B, 500, 3000, seed=257)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=17, device="cuda")
    w.seq_lens[2] = -3
    out = pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                    w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    print("max/mean err per 16 requests", _check(w, out))


def test_balanced_step_noalloc_and_graph_match_the_workspace_call():
    """A multi-round decode step through the fixed scratch and through a
    captured graph gives the same bits as the call with a workspace."""
    B, hq, hkv, d, ps = 100, 16, 8, 128, 256
    lens = np.random.default_rng(3).integers(1000, 9001, size=B).astype(np.int32)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=21, device="cuda", store_new=True)
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()

    def restore():
        w.k_cache.copy_(k0)
        w.v_cache.copy_(v0)

    ws = pkv.decode_workspace(B, hq, hkv, d, w.max_seq_len)
    out_a = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale, workspace=ws)
    ka = w.k_cache.clone()
    restore()
    out_b = torch.full_like(w.q, 3.0)
    pkv.pkv_decode_step_noalloc(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale, out=out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(ka.view(torch.int16), w.k_cache.view(torch.int16))
    out_g = torch.empty_like(w.q)
    gws = torch.zeros(pkv.pkv_decode_graphs_workspace_bytes([B], hq, hkv, d, w.max_seq_len),
                      dtype=torch.uint8, device="cuda")
    graphs = pkv.pkv_decode_graphs_create([B], w.q, w.k_cache, w.v_cache, w.page_table,
                                          w.seq_lens, w.max_seq_len, w.scale, out_g,
                                          k_new=w.k_new, v_new=w.v_new, out_loc=w.out_loc,
                                          workspace=gws)
    try:
        for _ in range(3):
            restore()
            out_g.fill_(7.0)
            torch.cuda.synchronize()
            assert graphs.replay(B) == B
            torch.cuda.synchronize()
            assert torch.equal(out_a.view(torch.int16), out_g.view(torch.int16))
            assert torch.equal(ka.view(torch.int16), w.k_cache.view(torch.int16))
    finally:
        graphs.destroy()
    print("max/mean err per 16 requests", _check(w, out_a))

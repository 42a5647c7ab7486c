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

MAX_RESIDENT_WAVES = 4096  # above any round of the decode kernels on this GPU


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
]


@pytest.mark.parametrize("B,hq,hkv,d,ps,lo,hi", CASES)
def test_balanced_decode(B, hq, hkv, d, ps, lo, hi):
    lens = _lengths(B, lo, hi, seed=B + hq + d + ps)
    split = pkv.pkv_decode_split_tokens(B, hkv, int(lens.max()))
    # units of max-length requests at the host split, over KV heads: beyond
    # four rounds of any resident wave count, so no one-round launch
    worst = B * (-(-int(lens.max()) // split)) * hkv
    assert worst > 4 * MAX_RESIDENT_WAVES, "batch too small for several rounds"
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

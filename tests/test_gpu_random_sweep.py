"""Seeded random sweep of the attention entry points against the float64
oracle: head groupings, head sizes, page sizes, batch sizes, ragged and
degenerate lengths, automatic and explicit splits, the fused decode step
and multi-token drafts drawn at random, every output element compared.
Each case prints its parameters before it runs."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as orc
import paged_kv_attention_out_amd as pkv
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools, run_decode, run_prefill, run_store

pytestmark = pytest.mark.gpu

N_DECODE = 192
N_MULTI = 96
N_PREFILL = 80


def _heads(rng):
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    return g * hkv, hkv, int(rng.choice([64, 128])), int(rng.choice([16, 32, 64, 128, 256]))


def _lengths(rng, B, lo=1):
    kind = rng.random(B)
    n = np.where(kind < 0.3, rng.integers(1, 65, B),
                 np.where(kind < 0.8, rng.integers(65, 1501, B), rng.integers(1501, 5001, B)))
    return [max(int(x), lo) for x in n]


def _split(rng):
    return 0 if rng.random() < 0.5 else 16 * int(rng.integers(1, 129))


def _decode_case(i):
    rng = np.random.default_rng(5000 + i)
    hq, hkv, d, ps = _heads(rng)
    B = int(rng.integers(1, 25)) if rng.random() < 0.8 else int(rng.integers(64, 201))
    lens = _lengths(rng, B)
    if B > 64:  # keep the oracle's work bounded
        lens = [min(x, 600) for x in lens]
    step = bool(rng.random() < 0.5)
    if not step and B > 1 and rng.random() < 0.3:
        lens[int(rng.integers(0, B))] = 0  # an empty request gets a zero row
    return hq, hkv, d, ps, lens, _split(rng), step


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    hq, hkv, d, ps, lens, split, step = _decode_case(i)
    print(f"random decode {i}: hq={hq} hkv={hkv} d={d} ps={ps} B={len(lens)} "
          f"sum={sum(lens)} split={split} step={step}", flush=True)
    w = inputs.build_decode(len(lens), hq, hkv, d, ps, lens, seed=6000 + i, device="cuda",
                            store_new=step)
    kc, vc = host_pools(w)
    live = [r for r, n in enumerate(lens) if n > 0]
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                     requests=live)
    if step:
        out = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                  w.page_table, w.seq_lens, w.max_seq_len, w.scale,
                                  split_tokens=split)
    else:
        out = run_decode(w, split_tokens=split)
    torch.cuda.synchronize()
    got = f64(out)
    print(i, assert_close(got, ref, f"random decode {i}"))
    for r, n in enumerate(lens):
        if n == 0:
            assert (got[r] == 0).all(), f"request {r} without keys must get zeros"
    if step:
        # the new rows landed in their slots, bit for bit
        kf = w.k_cache.view(-1, hkv, d)[w.out_loc.long()]
        assert torch.equal(kf.view(torch.int16), w.k_new.view(torch.int16))


def _multi_case(i):
    rng = np.random.default_rng(7000 + i)
    hq, hkv, d, ps = _heads(rng)
    q_len = int(rng.integers(2, 17))
    B = int(rng.integers(1, 17))
    lens = _lengths(rng, B)
    if rng.random() < 0.3:
        lens[0] = int(rng.integers(1, q_len + 1))  # a context no longer than the draft
    return hq, hkv, d, ps, q_len, lens, _split(rng)


@pytest.mark.parametrize("i", range(N_MULTI))
def test_random_decode_multi(i):
    hq, hkv, d, ps, q_len, lens, split = _multi_case(i)
    print(f"random multi {i}: hq={hq} hkv={hkv} d={d} ps={ps} q_len={q_len} B={len(lens)} "
          f"sum={sum(lens)} split={split}", flush=True)
    w = inputs.build_decode(len(lens), hq, hkv, d, ps, lens, seed=8000 + i, device="cuda",
                            q_len=q_len)
    kc, vc = host_pools(w)
    ref = orc.decode_multi(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np,
                           w.scale)
    out = pkv.pkv_paged_attn_decode_multi(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                          w.max_seq_len, w.scale, split_tokens=split)
    torch.cuda.synchronize()
    print(i, assert_close(f64(out), ref, f"random multi {i}"))


def _prefill_case(i):
    rng = np.random.default_rng(9000 + i)
    hq, hkv, d, ps = _heads(rng)
    while hq > 16:  # keep the oracle's dense products small
        hkv //= 2
        hq //= 2
    B = int(rng.integers(1, 7))
    prefix = [int(x) for x in rng.integers(0, 1501, B)]
    qlens = [int(x) for x in rng.integers(0, 301, B)]
    if rng.random() < 0.3:
        prefix[0] = 0
    if sum(qlens) == 0:
        qlens[-1] = 1
    return hq, hkv, d, ps, prefix, qlens


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill(i):
    hq, hkv, d, ps, prefix, qlens = _prefill_case(i)
    print(f"random prefill {i}: hq={hq} hkv={hkv} d={d} ps={ps} prefix={prefix} "
          f"qlens={qlens}", flush=True)
    w = inputs.build_prefill(len(prefix), hq, hkv, d, ps, prefix, qlens, seed=10000 + i,
                             device="cuda")
    kc, vc = host_pools(w)
    ref = orc.prefill_dense(inputs.bf16_bits(w.q), w.cu_seqlens_q.cpu().numpy(),
                            w.prefix_lens_np, kc, vc, w.page_table_np, w.scale)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(i, assert_close(f64(out), ref, f"random prefill {i}"))


N_SHARED = 32
N_LARGE = 16


def _shared_case(i):
    rng = np.random.default_rng(11000 + i)
    hq, hkv, d, ps = _heads(rng)
    groups = [(int(rng.integers(1, 41)), int(rng.integers(0, 1501)))
              for _ in range(int(rng.integers(1, 5)))]
    return hq, hkv, d, ps, groups, bool(rng.random() < 0.5), _split(rng)


@pytest.mark.parametrize("i", range(N_SHARED))
def test_random_decode_shared(i):
    from test_gpu_decode_shared import _grouped, _run
    hq, hkv, d, ps, groups, store, split = _shared_case(i)
    print(f"random shared {i}: hq={hq} hkv={hkv} d={d} ps={ps} groups={groups} "
          f"store={store} split={split}", flush=True)
    w, cu, shared, max_group, max_shared = _grouped(hq, hkv, d, ps, groups, 12000 + i, store)
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
    out = _run(w, cu, shared, max_group, max_shared, split)
    torch.cuda.synchronize()
    print(i, assert_close(f64(out), ref, f"random shared {i}"))


def _large_case(i):
    # Batches long enough to need several rounds of units (the balanced
    # launch when it applies); a random subset of requests is compared.
    rng = np.random.default_rng(13000 + i)
    hq, hkv, d, ps = _heads(rng)
    hkv = max(hkv, 2)
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(64, 257))
    lens = [int(x) for x in rng.integers(1, 8193, B)]
    lens[int(rng.integers(0, B))] = 8192
    for r in rng.choice(B, size=min(3, B), replace=False):
        lens[int(r)] = int(rng.choice([0, 1, 16, 17]))
    reqs = sorted(int(r) for r in rng.choice(B, size=24, replace=False))
    return hq, hkv, d, ps, lens, reqs, bool(rng.random() < 0.5)


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_decode_large(i):
    hq, hkv, d, ps, lens, reqs, step = _large_case(i)
    if step:
        lens = [max(n, 1) for n in lens]
    print(f"random large {i}: hq={hq} hkv={hkv} d={d} ps={ps} B={len(lens)} "
          f"sum={sum(lens)} step={step}", flush=True)
    w = inputs.build_decode(len(lens), hq, hkv, d, ps, lens, seed=14000 + i, device="cuda",
                            store_new=step)
    kc, vc = host_pools(w)
    live = [r for r in reqs if lens[r] > 0]
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                     requests=live)
    if step:
        out = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                  w.page_table, w.seq_lens, w.max_seq_len, w.scale)
    else:
        out = run_decode(w)
    torch.cuda.synchronize()
    got = f64(out)
    print(i, assert_close(got, ref, f"random large {i}"))
    for r in reqs:
        if lens[r] == 0:
            assert (got[r] == 0).all(), f"request {r} without keys must get zeros"

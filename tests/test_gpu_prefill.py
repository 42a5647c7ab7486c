"""Causal prefill with prefix on the GPU against the float64 oracle.

Small cases cover every (head_dim, group) instantiation, empty requests,
one-token requests, ragged query tiles and prefixes that are not page
multiples; the chunked-prefill workload runs at full size (store, then
attention) and is compared on every element.  Invariants: page
permutation (bit-exact), determinism, one visible key returns its V row
exactly, decode == one-row prefill (two different kernels, within
tolerance)."""

import numpy as np
import pytest
import torch

from oracle import paged_attention as orc
import paged_kv_attention_out_amd as pkv
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools, run_decode, run_prefill, run_store

pytestmark = pytest.mark.gpu

# (Hq, Hkv, d, ps, prefix_lens, q_lens)
CASES = [
    (4, 2, 64, 16, [0, 5, 37], [1, 70, 130]),
    (8, 2, 64, 16, [100, 0], [64, 200]),
    (8, 8, 64, 32, [0, 3], [300, 17]),
    (16, 2, 64, 16, [10, 0], [40, 33]),
    (4, 4, 128, 256, [0, 600], [129, 50]),
    (8, 4, 128, 16, [20, 0, 0], [0, 45, 160]),
    (16, 4, 128, 64, [64, 7], [100, 1]),
    (8, 2, 64, 128, [1000, 0, 255], [65, 257, 2]),
    (16, 2, 128, 16, [3, 0, 70], [90, 40, 17]),     # 8 query heads per KV head, 16-row tiles
    (8, 1, 128, 32, [50], [33]),
    (8, 2, 64, 64, [70, 0, 5], [200, 64, 1]),      # 64-row pages: one page per key tile
]


def _ids(c):
    return f"hq{c[0]}-hkv{c[1]}-d{c[2]}-ps{c[3]}-P{'_'.join(map(str, c[4]))}"


def _oracle(w, heads=None):
    kc, vc = host_pools(w)
    return orc.prefill_dense(inputs.bf16_bits(w.q), w.cu_seqlens_q.cpu().numpy(),
                             w.prefix_lens_np, kc, vc, w.page_table_np, w.scale, heads=heads)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_prefill_small(case):
    hq, hkv, d, ps, prefix, qlens = case
    print(f"prefill case {_ids(case)} qlens={qlens}", flush=True)
    w = inputs.build_prefill(len(prefix), hq, hkv, d, ps, prefix, qlens,
                             seed=sum(prefix) + sum(qlens) + d, device="cuda")
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    assert_close(f64(out), ref, _ids(case))


def test_prefill_chunked_workload():
    """The chunked-prefill batch at full size (16 requests, ~15K new tokens
    over prefixes of up to 1024): store, then attention; every element of
    all 32 query heads against the oracle."""
    w = inputs.make_workload("chunked_prefill", device="cuda")
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    got = f64(out)
    print("chunked_prefill max/mean err", assert_close(got, ref, "chunked_prefill"))
    assert np.isfinite(got).all()


def test_prefill_page_permutation_and_determinism():
    w = inputs.build_prefill(3, 8, 2, 64, 16, [30, 0, 300], [200, 64, 1], seed=31,
                             device="cuda")
    run_store(w)
    a = run_prefill(w).clone()
    b = run_prefill(w).clone()
    perm = torch.randperm(w.num_pages, generator=torch.Generator().manual_seed(6)).cuda()
    k2 = torch.empty_like(w.k_cache)
    v2 = torch.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    w.k_cache, w.v_cache = k2, v2
    w.page_table = perm.to(torch.int32)[w.page_table.long()]
    c = run_prefill(w)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_prefill_single_key_returns_v_exactly():
    w = inputs.build_prefill(2, 8, 2, 64, 16, [0, 0], [1, 1], seed=32, device="cuda")
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    for t in range(2):
        for h in range(8):
            assert torch.equal(out[t, h].view(torch.int16), w.v_new[t, h // 4].view(torch.int16))


def test_decode_equals_one_row_prefill():
    w = inputs.build_decode(4, 16, 8, 128, 16, [1, 100, 1000, 4097], seed=33, device="cuda")
    dec = f64(run_decode(w, split_tokens=256))
    w.kind = "prefill"
    pre = f64(run_prefill(w))
    torch.cuda.synchronize()
    assert np.abs(dec - pre).max() <= 2e-2
    assert np.abs(dec - pre).mean() <= 2e-3


def test_prefill_workspace_returns_to_zero():
    """The work counter goes back to zero at the end of every call, so one
    workspace serves calls of any size in a row (more and fewer work items
    than resident blocks)."""
    ws = torch.zeros(pkv.pkv_prefill_workspace_bytes(), dtype=torch.uint8, device="cuda")
    shapes = [(1, 4, 4, 64, 16, [3], [5]),                       # one work item
              (3, 8, 2, 64, 16, [40, 0, 300], [500, 64, 1]),
              (2, 8, 1, 128, 32, [0, 9], [700, 31])]
    for i, (B, hq, hkv, d, ps, prefix, qlens) in enumerate(shapes):
        print(f"workspace call {i}: hq={hq} hkv={hkv} d={d} qlens={qlens}", flush=True)
        w = inputs.build_prefill(B, hq, hkv, d, ps, prefix, qlens, seed=50 + i, device="cuda")
        ref = _oracle(w)
        run_store(w)
        out = pkv.pkv_paged_attn_prefill(w.q, w.cu_seqlens_q, w.prefix_lens, w.max_q_len,
                                         w.max_seq_len, w.k_cache, w.v_cache, w.page_table,
                                         w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, f"call {i} left the counter non-zero"
        assert_close(f64(out), ref, f"workspace call {i}")


def _shifted(w, q_add=0.0, k_add=0.0, k_outlier_frac=0.0, scale=None, seed=0):
    """Host workload with shifted q / K values (NaN poison stays NaN) and
    optionally a fraction of K rows (pool and new rows) scaled by 8."""
    g = torch.Generator().manual_seed(seed)
    w.q = (w.q.float() + q_add).to(torch.bfloat16)
    for name in ("k_cache", "k_new"):
        t = getattr(w, name).float() + k_add
        if k_outlier_frac:
            rows = t.view(-1, t.shape[-1])
            pick = torch.rand(rows.shape[0], generator=g) < k_outlier_frac
            rows[pick] *= 8.0
        setattr(w, name, t.to(torch.bfloat16))
    if scale is not None:
        w.scale = scale
    return w.to("cuda")


@pytest.mark.parametrize("kind", ["large_scale_outliers", "all_scores_negative"])
def test_prefill_extreme_scores(kind):
    # The kernel keeps each column's softmax reference point in bf16 and
    # moves it only when a tile's maximum exceeds it by more than 8: large
    # scores (coarse bf16 spacing of the reference, frequent moves) and
    # uniformly very negative scores (reference far below 0) both exercise it.
    w = inputs.build_prefill(3, 8, 2, 64, 16, [200, 0, 37], [150, 300, 64], seed=61)
    if kind == "large_scale_outliers":
        w = _shifted(w, k_outlier_frac=0.02, scale=1.0, seed=62)
    else:
        w = _shifted(w, q_add=3.0, k_add=-3.0)
    print(f"prefill extreme scores: {kind}", flush=True)
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(kind, assert_close(f64(out), ref, kind))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [0.125, 1.0])
def test_prefill_late_score_jump(scale, d):
    # Keys of the first tiles score near 0 and a few later keys score far
    # above them (+23 in base 2 at scale 1/8, +184 at scale 1: 2^184 is not
    # an fp32 number).  The running reference point of the softmax must move
    # on those tiles before any of their probabilities is accumulated.
    w = inputs.build_prefill(2, 8, 2, d, 16, [400, 0], [100, 200], seed=71)
    g = torch.Generator().manual_seed(72)
    w.q = torch.ones_like(w.q.float()).to(torch.bfloat16)
    w.k_cache = (w.k_cache.float() * 0.1).to(torch.bfloat16)
    w.k_new = (w.k_new.float() * 0.1).to(torch.bfloat16)
    kc = w.k_cache.view(-1, w.num_kv_heads, w.head_dim)
    ps = w.page_size
    for pos, kvh in [(100, 0), (250, 1), (399, 0), (399, 1), (77, 1)]:
        slot = int(w.page_table_np[0, pos // ps]) * ps + pos % ps
        kc[slot, kvh] = 2.0 + 0.01 * torch.randn(w.head_dim, generator=g)
    w.scale = scale
    w = w.to("cuda")
    print(f"prefill late score jump: scale {scale}, head_dim {d}", flush=True)
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(scale, assert_close(f64(out), ref, f"late score jump, scale {scale}"))


@pytest.mark.parametrize("B", [64, 70])
def test_prefill_many_requests(B):
    # Work items are handed out longest first (key range of each query tile)
    # for up to 64 requests and query tile by query tile beyond; both orders
    # must cover every tile exactly once, with empty requests in between.
    rng = np.random.default_rng(80 + B)
    prefix = [int(x) for x in rng.integers(0, 300, B)]
    qlens = [int(x) for x in rng.integers(0, 140, B)]
    qlens[3] = 0
    w = inputs.build_prefill(B, 8, 2, 64, 16, prefix, qlens, seed=81 + B, device="cuda")
    print(f"prefill many requests: B={B} tokens={w.num_tokens}", flush=True)
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(B, assert_close(f64(out), ref, f"{B} requests"))


def test_prefill_long_prefix_query_tile_order():
    # 8 query heads per KV head at head_dim 128 give 16-position query tiles;
    # with a 17,000-token prefix the levels of the longest-first walk exceed
    # its bound, so the items go query tile by query tile instead.
    w = inputs.build_prefill(2, 16, 2, 128, 16, [17000, 5], [40, 33], seed=91, device="cuda")
    print(f"prefill long prefix: max_seq_len={w.max_seq_len}", flush=True)
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(assert_close(f64(out), ref, "long prefix"))


@pytest.mark.parametrize("prefix", [[30000, 20000, 10], [40000, 30000, 5]],
                         ids=["3136_pages", "4386_pages"])
def test_prefill_long_prefixes(prefix):
    # Head_dim 64, longest-first order over several hundred levels: long
    # cached prefixes with few new tokens, thousands of page numbers per
    # call, and a near-empty request beside them.
    qlens = [40, 70, 30]
    w = inputs.build_prefill(3, 8, 2, 64, 16, prefix, qlens, seed=93 + prefix[0], device="cuda")
    pages = sum(-(-(p + q) // 16) for p, q in zip(prefix, qlens))
    print(f"prefill long prefixes: pages={pages}", flush=True)
    ref = _oracle(w)
    run_store(w)
    out = run_prefill(w)
    torch.cuda.synchronize()
    print(pages, assert_close(f64(out), ref, f"long prefixes, {pages} pages"))


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_pool_beyond_2gib(d):
    # Pools of up to 2 GiB are read with buffer loads at 32-bit offsets,
    # larger ones with 64-bit addresses.  The same batch, its pages moved to
    # the far end of a 2.46 GB pool, gives the same bits as in its own small
    # pool, and stays within tolerance of the oracle.
    hq, hkv, ps = 8, 2, 16
    w = inputs.build_prefill(2, hq, hkv, d, ps, [100, 37], [70, 130], seed=97 + d, device="cuda")
    ref = _oracle(w)
    run_store(w)
    small = run_prefill(w).clone()
    page_bytes = ps * hkv * d * 2
    big_pages = (2**31 + 2**29) // page_bytes
    n_small = w.k_cache.shape[0]
    shift = big_pages - n_small
    kb = torch.empty((big_pages, ps, hkv, d), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    kb[shift:].copy_(w.k_cache)
    vb[shift:].copy_(w.v_cache)
    table = (w.page_table + shift).contiguous()
    print(f"prefill pool beyond 2 GiB: d={d} pages={big_pages} shift={shift}", flush=True)
    big = pkv.pkv_paged_attn_prefill(w.q, w.cu_seqlens_q, w.prefix_lens, w.max_q_len,
                                     w.max_seq_len, kb, vb, table, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(big.view(torch.int16), small.view(torch.int16))
    print(d, assert_close(f64(big), ref, "pool beyond 2 GiB"))
    del kb, vb
    torch.cuda.empty_cache()

"""Paged decode attention on the GPU against the float64 oracle.

Small cases compare every output element; the full-size workloads compare
every element of every request (tiny, Llama- and Qwen-shaped), and for the
long-context batch every request on the query heads of one KV head each
(all eight KV heads covered).  Invariants: physical page
permutation (bit-exact), run-to-run determinism (bit-exact), independence
of the split length (within tolerance), a single visible token returns its
V row exactly, zero query gives the mean of V, empty requests give zeros,
and one workspace serves calls of any shape."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, compact, f64, host_pools, run_decode, run_store

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, d, ps, seq_lens, split_tokens) -- every (d, g) instantiation,
# tails of every length class, several splits per request
CASES = [
    (3, 4, 4, 64, 16, [1, 17, 64], 0),
    (5, 8, 4, 64, 16, [15, 16, 100, 333, 1000], 64),
    (2, 8, 2, 64, 32, [2000, 77], 128),
    (4, 16, 8, 128, 256, [1, 255, 256, 1500], 0),
    (4, 16, 8, 128, 256, [700, 2000, 513, 20], 256),
    (3, 8, 8, 128, 16, [40, 1, 300], 32),
    (2, 8, 2, 128, 64, [911, 16], 16),
    (3, 2, 1, 64, 128, [129, 4000, 3], 0),
    (3, 16, 2, 64, 16, [1, 300, 2000], 0),         # 8 query heads per KV head
    (3, 32, 4, 128, 32, [17, 900, 3000], 128),
]


def _ids(c):
    return f"B{c[0]}-hq{c[1]}-hkv{c[2]}-d{c[3]}-ps{c[4]}-split{c[6]}"


def _oracle(w, requests=None, heads=None):
    kc, vc = host_pools(w)
    return orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                      requests=requests, heads=heads)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_small(case):
    B, hq, hkv, d, ps, lens, split = case
    print(f"decode case {_ids(case)} lens={lens}", flush=True)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=sum(lens) + d, device="cuda",
                            store_new=True)
    ref = _oracle(w)                    # host copies taken before any kernel runs
    run_store(w)
    out = run_decode(w, split_tokens=split)
    torch.cuda.synchronize()
    assert_close(f64(out), ref, _ids(case))


def test_decode_tiny_workload():
    w = inputs.make_workload("tiny_decode", device="cuda")
    out = run_decode(w)
    torch.cuda.synchronize()
    assert_close(f64(out), _oracle(w), "tiny_decode")


def test_decode_llama_workload():
    w = inputs.make_workload("llama_decode")          # generated on the host, then copied
    ref = _oracle(w)
    w = w.to("cuda")
    run_store(w)
    out = run_decode(w)
    torch.cuda.synchronize()
    print("llama_decode max/mean err", assert_close(f64(out), ref, "llama_decode"))


def test_decode_qwen_workload_every_request():
    """Qwen-shaped batch (128 requests up to 8192 tokens, 256-row pages):
    every element of every request against the oracle, 16 requests at a
    time."""
    w = inputs.make_workload("qwen_decode", device="cuda")
    out = run_decode(w)
    torch.cuda.synchronize()
    got = f64(out)
    errs = []
    for r0 in range(0, w.num_seqs, 16):
        reqs = list(range(r0, min(r0 + 16, w.num_seqs)))
        kc, vc, table = compact(w, reqs)
        ref = orc.decode(inputs.bf16_bits(w.q)[reqs], kc, vc, table, w.seq_lens_np[reqs],
                         w.scale)
        errs.append(assert_close(got[reqs], ref, f"qwen_decode requests {r0}.."))
    print("qwen_decode max/mean err per 16 requests", errs)


def test_decode_long_workload_every_request():
    """Long-context batch (16 requests of 32K-131K tokens, 1% of K rows x8):
    every request against the oracle, one request at a time, on the two
    query heads of one KV head (request r: KV head r % 8, so all eight KV
    heads are covered twice)."""
    w = inputs.make_workload("long_decode", device="cuda")
    out = run_decode(w)
    torch.cuda.synchronize()
    got = f64(out)
    g, d = w.group, w.head_dim
    for r in range(w.num_seqs):
        kvh = r % w.num_kv_heads
        kc, vc, table = compact(w, [r], kv_head=kvh)
        q = inputs.bf16_bits(w.q)[[r]][:, kvh * g:(kvh + 1) * g]
        ref = orc.decode(q, kc, vc, table, w.seq_lens_np[[r]], w.scale)
        print(f"long_decode request {r} (n={int(w.seq_lens_np[r])}, KV head {kvh})",
              assert_close(got[[r]][:, kvh * g:(kvh + 1) * g], ref, f"long_decode r{r}"),
              flush=True)


@pytest.mark.parametrize("hq,hkv,d,ps,lens,split", [
    (4, 2, 128, 256, [32800, 16500, 300], 16400),  # split 1 starts 16 rows into page 64
    (8, 2, 64, 32, [4200, 2064, 2065], 2064),       # split 1 starts 16 rows into page 64
    (4, 2, 64, 64, [9000, 4113], 4112),
    (8, 4, 128, 128, [20000], 2064),
])
def test_decode_split_starting_inside_a_page(hq, hkv, d, ps, lens, split):
    """Splits whose first token is not the first row of a page and that span
    more than 63 pages: every window must end on a page boundary."""
    print(f"split inside a page: ps={ps} split={split} lens={lens}", flush=True)
    w = inputs.build_decode(len(lens), hq, hkv, d, ps, lens, seed=split + ps, device="cuda",
                            store_new=True)
    ref = _oracle(w)
    run_store(w)
    out = run_decode(w, split_tokens=split)
    torch.cuda.synchronize()
    print(assert_close(f64(out), ref, f"ps {ps} split {split}"))


def test_decode_automatic_split_not_a_page_multiple():
    """1024 requests x 8 KV heads with max_seq_len 40000 and 256-row pages:
    the host's automatic split (20000 tokens) is not a multiple of the page
    size, so the long requests' second splits start inside a page."""
    B, hq, hkv, d, ps = 1024, 8, 8, 64, 256
    rng = np.random.default_rng(1024)
    lens = rng.integers(1, 257, size=B).astype(np.int32)
    long_reqs = [3, 500, 1023]
    lens[long_reqs] = [40000, 36500, 39999]
    split = pkv.pkv_decode_split_tokens(B, hkv, 40000)
    assert split % ps != 0, split
    print(f"automatic split {split} at ps {ps}", flush=True)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=1025, device="cuda")
    out = run_decode(w)
    torch.cuda.synchronize()
    reqs = long_reqs + [0, 1, 700]
    kc, vc, table = compact(w, reqs)
    ref = orc.decode(inputs.bf16_bits(w.q)[reqs], kc, vc, table, w.seq_lens_np[reqs], w.scale)
    print(assert_close(f64(out)[reqs], ref, "automatic split"))


def test_decode_page_permutation_is_bit_exact():
    w = inputs.build_decode(4, 8, 2, 64, 16, [300, 1, 77, 1024], seed=21, device="cuda")
    a = run_decode(w, split_tokens=64).clone()
    perm = torch.randperm(w.num_pages, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(len(perm))
    k2 = torch.empty_like(w.k_cache)
    v2 = torch.empty_like(w.v_cache)
    k2[perm.cuda()] = w.k_cache
    v2[perm.cuda()] = w.v_cache
    w.k_cache, w.v_cache = k2, v2
    w.page_table = perm.cuda().to(torch.int32)[w.page_table.long()]
    b = run_decode(w, split_tokens=64)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_deterministic_and_split_invariant():
    w = inputs.build_decode(3, 16, 8, 128, 16, [3000, 999, 2048], seed=22, device="cuda")
    ref = _oracle(w)
    outs = {}
    for split in (16, 48, 256, 1024, 0):
        a = run_decode(w, split_tokens=split).clone()
        b = run_decode(w, split_tokens=split).clone()
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), split
        assert_close(f64(a), ref, f"split {split}")
        outs[split] = f64(a)
    for s, o in outs.items():
        assert np.abs(o - outs[0]).max() <= 2e-2, s


def test_decode_single_token_returns_v_exactly():
    w = inputs.build_decode(3, 8, 2, 64, 16, [1, 1, 1], seed=23, device="cuda")
    out = run_decode(w)
    torch.cuda.synchronize()
    v = w.v_cache.view(-1, 2, 64)
    for r in range(3):
        slot = int(w.page_table_np[r, 0]) * 16
        for h in range(8):
            assert torch.equal(out[r, h].view(torch.int16), v[slot, h // 4].view(torch.int16))


def test_decode_zero_query_is_mean_of_v():
    w = inputs.build_decode(2, 4, 2, 128, 16, [37, 500], seed=24, device="cuda")
    w.q.zero_()
    out = run_decode(w, split_tokens=64)
    torch.cuda.synchronize()
    kc, vc = host_pools(w)
    for r in range(2):
        V = orc.bf16_to_f64(vc.reshape(-1, 2, 128)[orc.request_slots(
            w.page_table_np[r], int(w.seq_lens_np[r]), 16)])
        for h in range(4):
            ref = V[:, h // 2].mean(axis=0)
            assert np.abs(f64(out[r, h]) - ref).max() <= 2e-2


def test_decode_empty_request_gives_zeros():
    w = inputs.build_decode(3, 8, 2, 64, 16, [50, 1, 70], seed=25, device="cuda")
    w.seq_lens[1] = 0
    out = torch.full_like(w.q, 7.0)
    run_decode(w, out=out, split_tokens=16)
    torch.cuda.synchronize()
    assert (out[1] == 0).all()
    w.seq_lens_np = w.seq_lens_np.copy()
    w.seq_lens_np[1] = 1
    ref = _oracle(w, requests=[0, 2])
    assert_close(f64(out), ref, "empty request")


def test_decode_workspace_reuse_across_shapes():
    """One workspace, filled with garbage, serves calls of different shapes."""
    ws = torch.full((pkv.pkv_decode_workspace_bytes(4, 8, 4, 64, 1500, 64),), 0x7F,
                    dtype=torch.uint8, device="cuda")
    a = inputs.build_decode(4, 8, 4, 64, 16, [900, 33, 1500, 16], seed=26, device="cuda")
    b = inputs.build_decode(2, 8, 4, 64, 16, [700, 1200], seed=27, device="cuda")
    for w in (a, b, a):
        out = run_decode(w, split_tokens=64, workspace=ws)
        torch.cuda.synchronize()
        assert_close(f64(out), _oracle(w), "reuse")


STEP_CASES = [
    (4, 32, 8, 64, 16, [1, 17, 300, 2048], 0),      # one-token request; new token in a full chunk
    (3, 16, 8, 128, 256, [256, 513, 4000], 0),
    (5, 8, 2, 64, 32, [16, 48, 95, 1000, 64], 64),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"B{c[0]}-hq{c[1]}-hkv{c[2]}-d{c[3]}-ps{c[4]}")
def test_decode_step_equals_store_then_decode(case):
    """pkv_decode_step (one launch) against pkv_store_kv + pkv_paged_attn_decode:
    bit-identical output and pools, and within tolerance of the oracle."""
    B, hq, hkv, d, ps, lens, split = case
    print(f"decode step case {case}", flush=True)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=77 + d + B, device="cuda",
                            store_new=True)
    ref = _oracle(w)
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    run_store(w)
    out_a = run_decode(w, split_tokens=split).clone()
    ka, va = w.k_cache.clone(), w.v_cache.clone()
    w.k_cache.copy_(k0)
    w.v_cache.copy_(v0)
    out_b = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale,
                                split_tokens=split)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    assert torch.equal(ka.view(torch.int16), w.k_cache.view(torch.int16))
    assert torch.equal(va.view(torch.int16), w.v_cache.view(torch.int16))
    assert_close(f64(out_b), ref, "decode step")


def test_decode_step_llama_workload():
    w = inputs.make_workload("llama_decode", device="cuda")
    reqs = [0, 7, 33, 63]
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                     requests=reqs)
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    run_store(w)
    out_a = run_decode(w).clone()
    w.k_cache.copy_(k0)
    w.v_cache.copy_(v0)
    out_b = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    print("llama decode step max/mean err", assert_close(f64(out_b), ref, "llama step"))


def test_shared_prefix_decode_workload():
    """Requests whose page tables alias one cached 1024-token prefix
    (prefix caching): the kernels read the shared pages once per request and
    per KV head, like any other page."""
    w = inputs.make_workload("shared_prefix_decode", device="cuda")
    reqs = [0, 21, 42, 63]
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                     requests=reqs)
    out = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                              w.page_table, w.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    print("shared prefix max/mean err", assert_close(f64(out), ref, "shared prefix"))


def _shift_decode(w, q_add=0.0, k_add=0.0, k_outlier_frac=0.0, scale=None, seed=0):
    """Host decode workload with shifted q / K values (NaN poison stays NaN),
    optionally a fraction of K rows scaled by 8, and another softmax scale."""
    g = torch.Generator().manual_seed(seed)
    w.q = (w.q.float() + q_add).to(torch.bfloat16)
    for name in ("k_cache", "k_new"):
        t = getattr(w, name)
        if t is None:
            continue
        t = t.float() + k_add
        if k_outlier_frac:
            rows = t.view(-1, t.shape[-1])
            pick = torch.rand(rows.shape[0], generator=g) < k_outlier_frac
            rows[pick] *= 8.0
        setattr(w, name, t.to(torch.bfloat16))
    if scale is not None:
        w.scale = scale
    return w.to("cuda")


@pytest.mark.parametrize("kind", ["large_scale_outliers", "all_scores_negative"])
@pytest.mark.parametrize("q_len", [1, 4])
def test_decode_extreme_scores(kind, q_len):
    # Large scores (softmax_scale 1.0 with x8 key outliers: a near one-hot
    # softmax, frequent moves of the running max) and uniformly very negative
    # scores, through the split path (several splits per request + merge).
    lens = [37, 700, 1500]
    w = inputs.build_decode(3, 16, 4, 64, 16, lens, seed=71 + q_len, q_len=q_len,
                            store_new=q_len == 1)
    if kind == "large_scale_outliers":
        w = _shift_decode(w, k_outlier_frac=0.02, scale=1.0, seed=72)
    else:
        w = _shift_decode(w, q_add=3.0, k_add=-3.0)
    print(f"decode extreme scores: {kind} q_len={q_len}", flush=True)
    kc, vc = host_pools(w)
    if q_len == 1:
        ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
        run_store(w)
        out = run_decode(w, split_tokens=128)
    else:
        ref = orc.decode_multi(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np,
                               w.scale)
        out = pkv.pkv_paged_attn_decode_multi(w.q, w.k_cache, w.v_cache, w.page_table,
                                              w.seq_lens, w.max_seq_len, w.scale,
                                              split_tokens=128)
    torch.cuda.synchronize()
    print(kind, q_len, assert_close(f64(out), ref, kind))


@pytest.mark.parametrize("B,hq,hkv,d,lo,hi,q_len", [
    (250, 32, 8, 64, 50, 300, 1),     # the device's split choice reads four chunks of 64 lengths
    (100, 32, 8, 64, 100, 600, 1),
    (100, 32, 8, 64, 100, 600, 2),
    (100, 16, 8, 128, 50, 900, 1),    # eight KV heads per workgroup at head_dim 128
    (65, 16, 4, 128, 300, 2000, 1),   # four per workgroup; lengths in two chunks of 64
    (256, 8, 2, 64, 16, 400, 1),      # two per workgroup; the largest batch the device splits
    (130, 32, 8, 64, 10, 500, 4),
])
def test_decode_device_chosen_split(B, hq, hkv, d, lo, hi, q_len):
    # With the automatic split, batches that need few rounds of resident
    # waves get a split chosen on the device from the actual lengths (here
    # longer than the host's); the merge reads the split the split kernel
    # recorded.  An empty and a negative length are among them (both give
    # zeros).  Parity against the oracle on every element.
    rng = np.random.default_rng(B + hi + q_len + d)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    lens[3] = 0
    w = inputs.build_decode(B, hq, hkv, d, 16, lens, seed=int(B + q_len + d), device="cuda",
                            q_len=q_len)
    w.seq_lens[5] = -7
    kc, vc = host_pools(w)
    print(f"device-chosen split: B={B} hq{hq} hkv{hkv} d{d} lens {lo}..{hi} q_len={q_len} "
          f"host split {pkv.pkv_decode_split_tokens(B, hkv, w.max_seq_len)}", flush=True)
    live = [r for r in range(B) if r not in (3, 5)]
    if q_len == 1:
        ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                         requests=live)
        ws = pkv.decode_workspace(B, hq, hkv, d, w.max_seq_len)
        out = pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                        w.max_seq_len, w.scale, workspace=ws)
    else:
        ref = orc.decode_multi(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np,
                               w.scale)
        ws = torch.zeros(pkv.pkv_decode_multi_workspace_bytes(B, q_len, hq, hkv, d,
                                                              w.max_seq_len),
                         dtype=torch.uint8, device="cuda")
        out = pkv.pkv_paged_attn_decode_multi(w.q, w.k_cache, w.v_cache, w.page_table,
                                              w.seq_lens, w.max_seq_len, w.scale, workspace=ws)
    torch.cuda.synchronize()
    # the split the kernels used is recorded in the workspace's first 256 bytes
    used = int(ws[:256].view(torch.int32)[0].item())
    host = pkv.pkv_decode_split_tokens(B, hkv, w.max_seq_len)
    assert used >= host and used % 16 == 0, (used, host)
    got = f64(out)
    for r in (3, 5):
        assert np.array_equal(got[r], np.zeros_like(got[r]))
        ref[r] = 0.0
    assert_close(got, ref, f"B{B}")


def test_decode_merge_of_many_splits():
    # A few long requests with more splits than the merge fetches ahead.
    lens = np.array([100, 5000, 40, 3000], np.int32)
    w = inputs.build_decode(4, 32, 8, 64, 16, lens, seed=83, device="cuda", store_new=True)
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
    print(f"many splits: host split {pkv.pkv_decode_split_tokens(4, 8, w.max_seq_len)}", flush=True)
    run_store(w)
    out = run_decode(w)
    torch.cuda.synchronize()
    assert_close(f64(out), ref, "many splits")


@pytest.mark.parametrize("split", [64, 128])
def test_decode_unit_order_many_requests(split):
    """Blocks take the full-length splits of all requests first and each
    request's short last split after them.  300 requests (five chunks of 64
    lengths, the last one read past the first 256) with lengths that are
    exact multiples of the split, one token past one, empty and negative,
    at an explicit split: every element against the oracle."""
    B, hq, hkv, d, ps = 300, 8, 2, 64, 16
    rng = np.random.default_rng(split + 5)
    lens = rng.integers(1, 400, size=B).astype(np.int32)
    lens[::7] = split * rng.integers(1, 5, size=len(lens[::7]))   # whole splits only
    lens[3::11] = split + 1                                        # one token into a split
    lens[5] = 0
    lens[290] = 0
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=int(split + B), device="cuda")
    w.seq_lens[9] = -4
    print(f"unit order: B={B} split={split}", flush=True)
    kc, vc = host_pools(w)
    live = [r for r in range(B) if r not in (5, 9, 290)]
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale,
                     requests=live)
    out = run_decode(w, split_tokens=split)
    torch.cuda.synchronize()
    got = f64(out)
    for r in (5, 9, 290):
        assert np.array_equal(got[r], np.zeros_like(got[r]))
        ref[r] = 0.0
    assert_close(got, ref, f"unit order split {split}")

"""Device-resident values that the host cannot check, out of range.

Page tables get out-of-range entries inside some requests' used pages:
negative ids, ids at and past the pool's page count, ids beyond 2^24 and
INT32_MAX.  The kernels keep every access inside the pools.  Decode windows
read page 0 for such ids.  The prefill and prefix-pass fetches clamp them to
the last page.  The prefill's buffer loads at 32-bit offsets read zeros past
the pool, or other rows of the pool for ids of 2^24 and more (their offsets
wrap).

Lengths get values beyond max_seq_len and below zero; the kernels clamp
them to [0, max_seq_len].  Shared-prefix lengths are cut to
[0, max_shared_len].

In every case the other requests' outputs are unchanged bit for bit, and the
pools are unchanged.  What an affected request gets is unspecified and not
compared."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from paged_kv_attention_out_amd import inputs

from gpu_helpers import run_prefill, run_store

pytestmark = pytest.mark.gpu


def _bad_ids(num_pages):
    return [-1, -2**31, num_pages, num_pages + 7, 2**24 + 3, 2**31 - 1]


def _poison_table(table, used, requests, num_pages):
    """Copy of ``table`` with the first, a middle and the last used page of
    each listed request replaced by out-of-range ids."""
    bad = _bad_ids(num_pages)
    t = table.clone()
    k = 0
    for r in requests:
        n = int(used[r])
        for i in sorted({0, n // 2, n - 1}):
            t[r, i] = bad[k % len(bad)]
            k += 1
    return t


def _same_rows(a, b, rows, where):
    for r in rows:
        assert torch.equal(a[r].view(torch.int16), b[r].view(torch.int16)), f"{where}: row {r}"


def _pages_used(w):
    return (w.seq_lens_np.astype(np.int64) + w.page_size - 1) // w.page_size


@pytest.mark.parametrize("kind", ["split", "balanced", "multi", "step"])
def test_decode_invalid_page_ids(kind):
    if kind == "balanced":
        # several rounds of units: the automatic split takes the balanced launch
        B, lo, hi = 96, 2000, 12000
    else:
        B, lo, hi = 24, 100, 1500
    hq, hkv, d, ps = 32, 8, 64, 16
    rng = np.random.default_rng(41)
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    q_len = 4 if kind == "multi" else 1
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=43, device="cuda",
                            store_new=kind == "step", q_len=q_len)
    bad_reqs = [3, 10, 17]
    print(f"invalid page ids, decode {kind}: B={B} lens {lo}..{hi} poisoned {bad_reqs}",
          flush=True)

    def call(table):
        if kind == "multi":
            return pkv.pkv_paged_attn_decode_multi(w.q, w.k_cache, w.v_cache, table, w.seq_lens,
                                                   w.max_seq_len, w.scale)
        if kind == "step":
            return pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                       table, w.seq_lens, w.max_seq_len, w.scale)
        return pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, table, w.seq_lens,
                                         w.max_seq_len, w.scale)

    clean = call(w.page_table).clone()
    torch.cuda.synchronize()
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    table = _poison_table(w.page_table, _pages_used(w), bad_reqs, w.num_pages)
    got = call(table)
    torch.cuda.synchronize()
    _same_rows(got, clean, [r for r in range(B) if r not in bad_reqs], f"decode {kind}")
    # the step stores the same new rows again; nothing else writes the pools
    assert torch.equal(w.k_cache.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(w.v_cache.view(torch.int16), v0.view(torch.int16))


def test_decode_shared_invalid_page_ids():
    from test_gpu_decode_shared import _grouped, _run
    hq, hkv, d, ps = 32, 8, 64, 16
    groups = [(6, 300), (5, 500), (4, 0)]
    w, cu, shared, max_group, max_shared = _grouped(hq, hkv, d, ps, groups, 47, False)
    clean = _run(w, cu, shared, max_group, max_shared).clone()
    torch.cuda.synchronize()
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    # Group 0's shared pages (read by the prefix pass from its first member's
    # row) and a private page of the second member of group 1.
    table = w.page_table.clone()
    bad = _bad_ids(w.num_pages)
    for i, page in enumerate([0, 9, 18]):
        table[0, page] = bad[i]
    used1 = int(_pages_used(w)[7])
    table[7, used1 - 1] = bad[4]
    table[7, -(-500 // ps)] = bad[5]  # its first private page
    w.page_table = table
    print(f"invalid page ids, shared decode: groups {groups}", flush=True)
    got = _run(w, cu, shared, max_group, max_shared)
    torch.cuda.synchronize()
    affected = set(range(0, 6)) | {7}
    _same_rows(got, clean, [r for r in range(w.num_seqs) if r not in affected], "shared decode")
    assert torch.equal(w.k_cache.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(w.v_cache.view(torch.int16), v0.view(torch.int16))


def _prefill_rows(w, requests):
    cu = w.cu_seqlens_q.cpu().numpy()
    return [t for r in requests for t in range(int(cu[r]), int(cu[r + 1]))]


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_invalid_page_ids(d):
    # pools below 2 GiB: rows are fetched by range-checked buffer loads
    hq, hkv, ps = 8, 2, 16
    prefix, qlens = [100, 300, 0, 50], [70, 130, 40, 200]
    w = inputs.build_prefill(4, hq, hkv, d, ps, prefix, qlens, seed=53 + d, device="cuda")
    run_store(w)
    clean = run_prefill(w).clone()
    torch.cuda.synchronize()
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    bad_reqs = [1, 3]
    w.page_table = _poison_table(w.page_table, _pages_used(w), bad_reqs, w.num_pages)
    print(f"invalid page ids, prefill d={d}: poisoned {bad_reqs}", flush=True)
    got = run_prefill(w)
    torch.cuda.synchronize()
    _same_rows(got, clean, _prefill_rows(w, [0, 2]), f"prefill d={d}")
    assert torch.equal(w.k_cache.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(w.v_cache.view(torch.int16), v0.view(torch.int16))


def test_prefill_invalid_page_ids_pool_beyond_2gib():
    # pools beyond 2 GiB: rows are fetched at 64-bit addresses with the page
    # clamped to the pool's last
    hq, hkv, d, ps = 8, 2, 64, 16
    w = inputs.build_prefill(3, hq, hkv, d, ps, [120, 0, 64], [90, 60, 33], seed=59,
                             device="cuda")
    run_store(w)
    page_bytes = ps * hkv * d * 2
    big_pages = (2**31 + 2**29) // page_bytes
    shift = big_pages - w.k_cache.shape[0]
    kb = torch.empty((big_pages, ps, hkv, d), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    kb[shift:].copy_(w.k_cache)
    vb[shift:].copy_(w.v_cache)
    table = (w.page_table + shift).contiguous()

    def call(t):
        return pkv.pkv_paged_attn_prefill(w.q, w.cu_seqlens_q, w.prefix_lens, w.max_q_len,
                                          w.max_seq_len, kb, vb, t, w.scale)

    clean = call(table).clone()
    torch.cuda.synchronize()
    bad = _poison_table(table, _pages_used(w), [1], big_pages)
    print(f"invalid page ids, prefill pool beyond 2 GiB: pages={big_pages}", flush=True)
    got = call(bad)
    torch.cuda.synchronize()
    _same_rows(got, clean, _prefill_rows(w, [0, 2]), "prefill, pool beyond 2 GiB")
    assert torch.equal(kb[shift:].view(torch.int16), w.k_cache.view(torch.int16))
    del kb, vb
    torch.cuda.empty_cache()


def test_decode_lengths_beyond_max_seq_len():
    # Lengths above max_seq_len read max_seq_len tokens; with a fixed split
    # every other request keeps its splits and its bits.
    B, hq, hkv, d, ps = 24, 32, 8, 64, 16
    lens = np.random.default_rng(61).integers(100, 1500, size=B).astype(np.int32)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=67, device="cuda")
    print("out-of-range lengths, decode", flush=True)

    def call(seq_lens):
        return pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, seq_lens,
                                         w.max_seq_len, w.scale, split_tokens=256)

    clean = call(w.seq_lens).clone()
    bad = w.seq_lens.clone()
    bad[5] = w.max_seq_len + 999
    bad[9] = 2**31 - 1
    got = call(bad)
    torch.cuda.synchronize()
    _same_rows(got, clean, [r for r in range(B) if r not in (5, 9)], "decode lengths")


def test_prefill_prefix_lengths_out_of_range():
    # A prefix beyond max_seq_len - (new tokens) is cut to it and a negative
    # one read as 0; the other requests keep their bits.
    hq, hkv, d, ps = 8, 2, 64, 16
    prefix, qlens = [100, 300, 0, 50], [70, 130, 40, 200]
    w = inputs.build_prefill(4, hq, hkv, d, ps, prefix, qlens, seed=71, device="cuda")
    run_store(w)
    clean = run_prefill(w).clone()
    w.prefix_lens = w.prefix_lens.clone()
    w.prefix_lens[0] = 2**31 - 1  # read as 430 - 70 keys before its new tokens
    w.prefix_lens[3] = -5
    print("out-of-range prefix lengths, prefill", flush=True)
    got = run_prefill(w)
    torch.cuda.synchronize()
    _same_rows(got, clean, _prefill_rows(w, [1, 2]), "prefill prefix lengths")


def test_decode_shared_lengths_out_of_range():
    # Shared lengths above max_shared_len or below zero are cut to
    # [0, max_shared_len]: each request's partials stay inside the workspace
    # sized for max_shared_len (a guard after it stays untouched), and the
    # requests with valid lengths keep their bits.
    from test_gpu_decode_shared import _grouped
    hq, hkv, d, ps = 32, 8, 64, 16
    groups = [(6, 300), (5, 500), (4, 0)]
    w, cu, shared, max_group, max_shared = _grouped(hq, hkv, d, ps, groups, 73, False)
    B = w.num_seqs
    need = pkv.pkv_paged_attn_decode_shared_workspace_bytes(B, hq, hkv, d, w.max_seq_len,
                                                            max_shared, 256)
    guard = 1 << 20
    ws = torch.full((need + guard,), 0x5A, dtype=torch.uint8, device="cuda")

    def call(sh):
        return pkv.pkv_paged_attn_decode_shared(
            w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.max_seq_len, cu, sh,
            max_group, max_shared, w.scale, workspace=ws[:need], split_tokens=256)

    clean = call(shared).clone()
    bad = shared.clone()
    bad[6] = 2**31 - 1   # the first member of group 1: its pass reads max_shared_len
    bad[12] = 2**31 - 1  # group 2 shares nothing; these two claim more
    bad[14] = 2**31 - 1
    bad[13] = -5
    print(f"out-of-range shared lengths: groups {groups}, workspace {need} bytes", flush=True)
    got = call(bad)
    torch.cuda.synchronize()
    affected = set(range(6, 11)) | {12, 13, 14}
    _same_rows(got, clean, [r for r in range(B) if r not in affected], "shared lengths")
    assert (ws[need:] == 0x5A).all(), "a partial landed past the workspace"

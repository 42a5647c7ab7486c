"""Host-side checks of the seeded input generators (no GPU, no oracle math)."""

import numpy as np
import pytest
import torch

from paged_kv_attention_out_amd import inputs


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_lengths_follow_recipe(name):
    cfg = inputs.WORKLOADS[name]
    a = inputs.draw_lengths(name)
    b = inputs.draw_lengths(name)
    if cfg["kind"] == "decode":
        assert np.array_equal(a, b)  # seeded
        lo, hi = cfg["len_range"]
        assert len(a) == cfg["num_seqs"] and a.min() >= lo and a.max() <= hi
    else:
        (p, q), (p2, q2) = a, b
        assert np.array_equal(p, p2) and np.array_equal(q, q2)
        assert p.min() >= cfg["prefix_range"][0] and p.max() <= cfg["prefix_range"][1]
        assert q.min() >= cfg["new_range"][0] and q.max() <= cfg["new_range"][1]
        assert q.sum() <= cfg["max_new_total"]


def _check_pages(w):
    ps = w.page_size
    owned = []
    for r in range(w.num_seqs):
        k = (int(w.seq_lens_np[r]) + ps - 1) // ps
        row = w.page_table_np[r]
        assert (row[:k] >= 0).all() and (row[:k] < w.poison_page).all()
        assert (row[k:] == w.poison_page).all()
        owned.extend(row[:k].tolist())
    assert len(owned) == len(set(owned)), "a physical page is owned twice"


def test_tiny_decode_layout():
    w = inputs.make_workload("tiny_decode")
    assert w.num_pages == 17 and w.poison_page == 16 and w.width == 4
    assert w.seq_lens_np.tolist() == [64]
    _check_pages(w)
    assert sorted(w.page_table_np[0].tolist()) == sorted(set(w.page_table_np[0].tolist()))
    k = w.k_cache.float()
    assert torch.isnan(k[16]).all()                    # poison page
    used = set(w.page_table_np[0].tolist())
    for p in range(16):
        assert torch.isnan(k[p]).all() != (p in used)  # unowned pages are NaN


def test_decode_store_slots():
    w = inputs.build_decode(5, 4, 2, 16, 16, [1, 16, 17, 40, 33], seed=3, store_new=True)
    _check_pages(w)
    ps = 16
    for r in range(5):
        n = int(w.seq_lens_np[r])
        slot = int(w.out_loc_np[r])
        assert slot // ps == w.page_table_np[r, (n - 1) // ps] and slot % ps == (n - 1) % ps
        # the slot about to be written is NaN before the store
        assert torch.isnan(w.k_cache.view(-1, 2, 16)[slot].float()).all()
    assert len(set(w.out_loc_np.tolist())) == 5


def test_prefill_slots_and_cu():
    w = inputs.build_prefill(3, 4, 2, 16, 16, [0, 5, 31], [7, 1, 20], seed=4)
    _check_pages(w)
    assert w.cu_seqlens_q.tolist() == [0, 7, 8, 28]
    assert len(w.out_loc_np) == 28 and len(set(w.out_loc_np.tolist())) == 28
    assert tuple(w.k_new.shape) == (28, 2, 16) and tuple(w.q.shape) == (28, 4, 16)
    ps = 16
    t = 0
    for r in range(3):
        for i in range(int(w.q_lens_np[r])):
            pos = int(w.prefix_lens_np[r]) + i
            s = int(w.out_loc_np[t])
            assert s // ps == w.page_table_np[r, pos // ps] and s % ps == pos % ps
            t += 1
    # cached prefix rows are finite, tail rows are NaN
    flat = w.k_cache.view(-1, 2, 16).float()
    for r in range(3):
        n = int(w.seq_lens_np[r])
        for pos in range(int(w.prefix_lens_np[r])):
            s = int(w.page_table_np[r, pos // ps]) * ps + pos % ps
            assert torch.isfinite(flat[s]).all()
        for pos in range(n, -(-n // ps) * ps):
            s = int(w.page_table_np[r, pos // ps]) * ps + pos % ps
            assert torch.isnan(flat[s]).all()


def test_outliers_are_exact_powers():
    w = inputs.build_decode(2, 4, 2, 16, 16, [300, 200], seed=5, outlier_frac=0.05)
    w0 = inputs.build_decode(2, 4, 2, 16, 16, [300, 200], seed=5, outlier_frac=0.0)
    a = w.k_cache.float().view(-1, 16)
    b = w0.k_cache.float().view(-1, 16)
    fin = torch.isfinite(b).all(dim=1)
    ratio_rows = ((a[fin] != b[fin]).any(dim=1))
    assert ratio_rows.sum() > 0
    assert torch.equal(a[fin][ratio_rows], b[fin][ratio_rows] * 8)


def test_shared_prefix_pages_alias_and_the_rest_are_private():
    w = inputs.make_workload("shared_prefix_decode")
    t, ps = w.page_table_np, w.page_size
    shared = inputs.WORKLOADS["shared_prefix_decode"]["shared_prefix"] // ps
    assert (t[:, :shared] == t[0, :shared]).all()
    need = (w.seq_lens_np + ps - 1) // ps
    private = np.concatenate([t[r, shared:need[r]] for r in range(w.num_seqs)])
    assert len(np.unique(private)) == len(private)
    assert not np.isin(private, t[0, :shared]).any()
    assert not np.isin(w.out_loc_np // ps, t[0, :shared]).any()  # new tokens in private pages


def test_multi_token_decode_inputs():
    w = inputs.build_decode(3, 8, 2, 16, 16, [2, 40, 17], seed=21, q_len=4)
    _check_pages(w)
    assert tuple(w.q.shape) == (3, 4, 8, 16)
    assert w.q_lens_np.tolist() == [4, 4, 4] and w.num_tokens == 12
    assert w.prefix_lens_np.tolist() == [0, 36, 13]
    # every owned position, the new tokens included, holds finite K/V
    for r in range(3):
        for t in range(int(w.seq_lens_np[r])):
            row = w.k_cache[w.page_table_np[r, t // 16], t % 16]
            assert torch.isfinite(row.float()).all()
    # q_len = 1 keeps the single-token layout and random stream
    a = inputs.build_decode(3, 8, 2, 16, 16, [2, 40, 17], seed=21)
    b = inputs.build_decode(3, 8, 2, 16, 16, [2, 40, 17], seed=21, q_len=1)
    assert torch.equal(a.q, b.q) and tuple(a.q.shape) == (3, 8, 16)
    with pytest.raises(AssertionError):
        inputs.build_decode(3, 8, 2, 16, 16, [2, 40, 17], seed=21, q_len=2, store_new=True)

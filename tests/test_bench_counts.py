"""The benchmark's counting rules (algorithmic bytes and FLOPs behind every
GB/s and TFLOP/s figure) against brute-force counts on small batches."""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from paged_kv_attention_out_amd import inputs  # noqa: E402


def test_prefill_flops_counts_causal_visible_pairs():
    w = inputs.build_prefill(3, 8, 2, 64, 16, [0, 37, 5], [70, 1, 130], seed=501)
    pairs = 0
    for r in range(w.num_seqs):
        P, L = int(w.prefix_lens_np[r]), int(w.q_lens_np[r])
        for i in range(L):          # new token i sits at position P + i
            for j in range(P + L):  # keys of the request
                pairs += j <= P + i
    # QK^T and PV: 2 * d multiply-adds per (query head, visible pair)
    assert bench.prefill_flops(w) == pairs * w.num_q_heads * 2 * 2 * w.head_dim


def test_decode_bytes_counts_every_row_once_per_kv_head():
    w = inputs.build_decode(4, 8, 2, 64, 16, [1, 17, 300, 64], seed=502)
    kv = q = meta = 0
    for r in range(w.num_seqs):
        n = int(w.seq_lens_np[r])
        for _t in range(n):
            kv += 2 * w.num_kv_heads * w.head_dim * 2  # K and V row slices, bf16
        q += 2 * w.num_q_heads * w.head_dim * 2       # q row in, out row back
        meta += 4 * -(-n // w.page_size) + 4          # page ids and the length
    assert bench.decode_bytes(w) == kv + q + meta


def test_store_bytes():
    w = inputs.build_decode(3, 8, 2, 64, 16, [5, 20, 33], seed=503, store_new=True)
    T = w.k_new.shape[0]
    # read k_new and v_new, write the same rows, read out_loc
    assert bench.store_bytes(w) == T * (2 * 2 * w.num_kv_heads * w.head_dim * 2 + 4)


def test_unique_kv_bytes_counts_shared_rows_once():
    # two requests whose first two pages are the same physical pages
    w = inputs.build_decode(2, 4, 1, 64, 16, [40, 50], seed=504)
    table = w.page_table_np.copy()
    table[1, :2] = table[0, :2]
    w.page_table_np = table
    rows = set()
    for r in range(2):
        n = int(w.seq_lens_np[r])
        for t in range(n):
            rows.add((int(table[r, t // 16]), t % 16))
    assert bench.unique_kv_bytes(w) == len(rows) * w.num_kv_heads * w.head_dim * 2 * 2
    assert len(rows) < int(w.seq_lens_np.sum())

"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same bytes, compare."""

from __future__ import annotations

import numpy as np
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

# Attention tolerance on bf16 inputs with fp32 accumulation, against the
# float64 oracle: max |err| and mean |err| over the compared elements.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> float64 host array (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, where: str = ""):
    mask = ~np.isnan(ref)
    assert mask.any(), "nothing to compare"
    g, r = got[mask], ref[mask]
    assert np.isfinite(g).all(), f"{where}: non-finite output"
    err = np.abs(g - r)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{where}: max|err| {mx:.3e} mean|err| {mean:.3e}"
    return mx, mean


def run_store(w: inputs.Workload):
    if w.k_new is not None:
        pkv.pkv_store_kv(w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache)


def run_decode(w: inputs.Workload, split_tokens: int = 0, out=None, workspace=None):
    return pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                     w.max_seq_len, w.scale, out=out, workspace=workspace,
                                     split_tokens=split_tokens)


def run_prefill(w: inputs.Workload, out=None):
    return pkv.pkv_paged_attn_prefill(w.q, w.cu_seqlens_q, w.prefix_lens, max(w.max_q_len, 1),
                                      max(w.max_seq_len, 1), w.k_cache, w.v_cache, w.page_table,
                                      w.scale, out=out)


def host_pools(w: inputs.Workload, stored: bool = True):
    """Host bit copies of the pools, with the oracle's store applied."""
    kc, vc = inputs.bf16_bits(w.k_cache), inputs.bf16_bits(w.v_cache)
    if stored and w.k_new is not None:
        kc, vc = orc.store_kv(kc, vc, inputs.bf16_bits(w.k_new), inputs.bf16_bits(w.v_new),
                              w.out_loc_np)
    return kc, vc


def compact(w: inputs.Workload, requests, kv_head=None):
    """Host bit copies of just the given requests' pages (gathered with torch
    indexing on the device), with a page table renumbered to match.  With
    ``kv_head`` only that KV head's slice of each row is kept (a pool of one
    KV head)."""
    ps = w.page_size
    rows, tables = [], []
    nxt = 0
    for r in requests:
        k = (int(w.seq_lens_np[r]) + ps - 1) // ps
        pages = w.page_table_np[r, :k]
        rows.append(pages)
        tables.append(np.arange(nxt, nxt + k, dtype=np.int32))
        nxt += k
    idx = torch.from_numpy(np.concatenate(rows).astype(np.int64)).to(w.k_cache.device)
    heads = slice(None) if kv_head is None else slice(kv_head, kv_head + 1)
    kc = inputs.bf16_bits(w.k_cache[idx][:, :, heads].contiguous())
    vc = inputs.bf16_bits(w.v_cache[idx][:, :, heads].contiguous())
    W = max(len(t) for t in tables)
    table = np.zeros((len(requests), W), np.int32)
    for i, t in enumerate(tables):
        table[i, :len(t)] = t
    return kc, vc, table

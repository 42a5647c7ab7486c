#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the hot path over one batch: the KV scatter of the
step's new rows (store_kv) followed by paged decode attention, on the
Llama-3.2-1B-shaped decode batch (64 requests, 32 query / 8 KV heads,
head_dim 64, page_size 16, seq_lens uniform in [128, 2048]).  The batch is
replicated R times in HBM and the steps rotate over the replicas, so the
timed working set (>= 1 GiB) cannot stay in the 256 MB Infinity Cache.

Prints ONE JSON line.  ``value`` is algorithmic bytes per step (K/V read
once per KV head, q, out, page table, seq_lens, plus store_kv's reads and
writes) over wall-clock time per step.  ``roofline`` is for the decode
kernel alone, timed with HIP events on its launch stream.  ``also`` holds
the same measurement for the other workloads: Qwen3-0.6B-shaped decode,
long-context decode, and chunked prefill (TFLOP/s against the bf16 MFMA
peak).  ``cpu_baseline`` is the float64 CPU oracle on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
MIN_WORKING_SET = 1 << 30
MIN_WARM_S = 0.25  # seconds of back-to-back calls before any timed pass
METRIC = "paged decode attn HBM GB/s (% peak) + causal prefill attn TFLOP/s (% peak)"
PRIMARY = "llama_decode"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---- algorithmic work --------------------------------------------------------

def decode_bytes(w) -> int:
    n = w.seq_lens_np.astype(np.int64)
    ps = w.page_size
    kv = int(n.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * w.num_tokens * w.num_q_heads * w.head_dim * 2   # q_len query rows per request
    meta = int(((n + ps - 1) // ps).sum()) * 4 + 4 * w.num_seqs
    return kv + qo + meta


def store_bytes(w) -> int:
    if w.k_new is None:
        return 0
    T = w.k_new.shape[0]
    return 2 * T * w.num_kv_heads * w.head_dim * 2 * 2 + 4 * T


def unique_kv_bytes(w) -> int:
    """K/V bytes of the distinct pool rows a decode batch reads (pages shared
    between requests counted once)."""
    ps = w.page_size
    rows = set()
    for r in range(w.num_seqs):
        n = int(w.seq_lens_np[r])
        pages = w.page_table_np[r, :(n + ps - 1) // ps]
        for i, pg in enumerate(pages):
            rows.add((int(pg), min(ps, n - i * ps)))
    tokens = {}
    for pg, cnt in rows:
        tokens[pg] = max(tokens.get(pg, 0), cnt)
    return sum(tokens.values()) * w.num_kv_heads * w.head_dim * 2 * 2


def prefill_flops(w) -> int:
    L = w.q_lens_np.astype(np.int64)
    P = w.prefix_lens_np.astype(np.int64)
    pairs = int((L * P + L * (L + 1) // 2).sum())
    return 4 * w.head_dim * w.num_q_heads * pairs


def prefill_bytes(w) -> int:
    n = w.seq_lens_np.astype(np.int64)
    kv = int(n.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * w.num_tokens * w.num_q_heads * w.head_dim * 2
    return kv + qo


def source_digest(path: str) -> str:
    """sha256 of a kernel source with comments and blank space removed, so a
    change to comments alone does not invalidate counters taken on it."""
    import hashlib
    import re

    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(line.strip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(text.encode()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode call measured with rocprofv3 counters
    (profiles/traffic.txt), or None when the kernel source has changed since
    the counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        wl, src, sha, fetch, write = line.split()
        if wl != workload:
            continue
        try:
            cur = source_digest(os.path.join(root, src))
        except OSError:
            return None
        return int(fetch) + int(write) if cur.startswith(sha) else None
    return None


# ---- GPU timing ----------------------------------------------------------------

def _replicate(w, R):
    import copy

    reps = [w]
    for _ in range(R - 1):
        c = copy.copy(w)
        for f in ("q", "k_cache", "v_cache", "page_table", "seq_lens", "prefix_lens",
                  "cu_seqlens_q", "k_new", "v_new", "out_loc"):
            t = getattr(w, f)
            setattr(c, f, None if t is None else t.clone())
        reps.append(c)
    return reps


def segment_trace(path: str, gap_ms: float = 20.0):
    """Print per-workload statistics of the attention and store kernels in a
    rocprofv3 kernel-trace CSV of this script: the workloads run one after
    another, separated by input generation, so dispatches of one kernel
    more than gap_ms apart start a new segment (segments follow the order
    in which main() times the workloads)."""
    import collections
    import csv

    by = collections.defaultdict(list)
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            by[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    keep = ("prefill_kernel", "decode_split_kernel", "decode_combine_kernel",
            "decode_balanced_kernel", "decode_combine_balanced_kernel", "decode_split_prefix_kernel",
            "store_kv_kernel")
    for name, v in by.items():
        short = next((k for k in keep if k in name), None)
        if short is None:
            continue
        tmpl = name[name.find(short) + len(short):].split("(")[0]
        v.sort()
        segs, cur = [], [v[0]]
        for a, b in zip(v, v[1:]):
            if b[0] - a[1] > gap_ms * 1e6:
                segs.append(cur)
                cur = []
            cur.append(b)
        segs.append(cur)
        for i, sg in enumerate(segs):
            d = sorted((e - s0) / 1e3 for s0, e in sg)
            print(f"{short + tmpl:34s} segment {i}: calls {len(d):6d}  mean {sum(d) / len(d):9.2f} us"
                  f"  median {d[len(d) // 2]:9.2f}  min {d[0]:9.2f}  max {d[-1]:9.2f}")


def warm_up(step, warmup: int, min_s: float = MIN_WARM_S):
    """Run step(i) for the requested warm-up steps, then more until min_s
    seconds of back-to-back calls have run, so the timed passes see the GPU
    at its steady clocks (a short burst times a compute-bound kernel while
    the clocks are still ramping up).  min_s = 0: exactly `warmup` steps."""
    import torch

    t_w = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t_w < min_s:
        step(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_workload(name: str, steps: int, warmup: int, split_tokens: int = 0,
                  fused_store: bool = True, via_prefill: bool = False,
                  min_warm_s: float = MIN_WARM_S, read_once: bool = False):
    """Time one workload's attention call.  A multi-token decode workload runs
    pkv_paged_attn_decode_multi, or with ``via_prefill`` the same batch through
    pkv_paged_attn_prefill (q_len new tokens after a cached prefix of n - q_len).
    ``read_once``: the shared-prefix workload through pkv_paged_attn_decode_shared
    (one group of all requests, the shared prefix read once per KV head)."""
    import torch

    import paged_kv_attention_out_amd as pkv
    from paged_kv_attention_out_amd import inputs

    lib = pkv.lib()
    w = inputs.make_workload(name, device="cuda", poison=False)
    is_multi = w.kind == "decode" and w.q.dim() == 4
    if via_prefill:
        assert is_multi
        w.q = w.q.reshape(w.num_tokens, w.num_q_heads, w.head_dim)
        w.kind = "prefill"
    is_decode = w.kind == "decode"
    L = w.q.shape[1] if is_multi and is_decode else 1
    work_bytes = decode_bytes(w) if is_decode else prefill_bytes(w)
    R = max(1, min(64, math.ceil(MIN_WORKING_SET / max(work_bytes, 1))))
    reps = _replicate(w, R)
    stream = torch.cuda.current_stream().cuda_stream
    B, Hq, Hkv, d, ps = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    split = pkv.pkv_decode_split_tokens(B, Hkv, w.max_seq_len, split_tokens) if is_decode else 0
    ws = pkv.decode_workspace(B, Hq, Hkv, d, w.max_seq_len, split_tokens) if is_decode else None
    if L > 1:
        nb = pkv.pkv_decode_multi_workspace_bytes(B, L, Hq, Hkv, d, w.max_seq_len, split_tokens)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda") if nb else None
    if not is_decode:
        ws = torch.zeros(pkv.pkv_prefill_workspace_bytes(), dtype=torch.uint8, device="cuda")
    shared_len = inputs.WORKLOADS[name].get("shared_prefix", 0)
    if read_once:
        nb = pkv.pkv_paged_attn_decode_shared_workspace_bytes(B, Hq, Hkv, d, w.max_seq_len,
                                                              shared_len, split_tokens)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        cu_g = torch.tensor([0, B], dtype=torch.int32, device="cuda")
        sh_l = torch.full((B,), shared_len, dtype=torch.int32, device="cuda")
    if is_decode and ws is not None and ws.numel() >= 256:
        # the split kernel writes the split it used to the first word; the
        # balanced launch (no fixed split) leaves this marker
        ws[:4].view(torch.int32).fill_(-1)
    ws_ptr, ws_bytes = (0, 0) if ws is None else (ws.data_ptr(), ws.numel())

    # Pre-marshalled C calls: the timed loop only enqueues.
    calls = []
    for c in reps:
        out = torch.empty_like(c.q)
        st = None
        if c.k_new is not None:
            st = (c.k_new.data_ptr(), c.v_new.data_ptr(), c.out_loc.data_ptr(),
                  c.k_new.shape[0], c.k_cache.data_ptr(), c.v_cache.data_ptr(),
                  c.k_cache.shape[0] * ps, Hkv, d, stream)
        if read_once:
            at = (c.q.data_ptr(), c.k_new.data_ptr(), c.v_new.data_ptr(), c.out_loc.data_ptr(),
                  c.k_cache.data_ptr(), c.v_cache.data_ptr(), ps, c.num_pages,
                  c.page_table.data_ptr(), c.page_table.shape[1], c.seq_lens.data_ptr(), B,
                  w.max_seq_len, cu_g.data_ptr(), sh_l.data_ptr(), 1, B, shared_len, Hq, Hkv,
                  d, w.scale, split_tokens, out.data_ptr(), ws_ptr, ws_bytes, stream)
            st = None
        elif is_decode and st is not None and fused_store:
            # one call: the new rows are written to the pool by the decode kernel
            at = (c.q.data_ptr(), c.k_new.data_ptr(), c.v_new.data_ptr(), c.out_loc.data_ptr(),
                  c.k_cache.data_ptr(), c.v_cache.data_ptr(), ps, c.num_pages,
                  c.page_table.data_ptr(), c.page_table.shape[1], c.seq_lens.data_ptr(), B,
                  w.max_seq_len, Hq, Hkv, d, w.scale, split_tokens, out.data_ptr(), ws_ptr,
                  ws_bytes, stream)
            st = None
        elif L > 1:
            at = (c.q.data_ptr(), L, c.k_cache.data_ptr(), c.v_cache.data_ptr(), ps,
                  c.num_pages, c.page_table.data_ptr(), c.page_table.shape[1],
                  c.seq_lens.data_ptr(), B, w.max_seq_len, Hq, Hkv, d, w.scale, split_tokens,
                  out.data_ptr(), ws_ptr, ws_bytes, stream)
        elif is_decode:
            at = (c.q.data_ptr(), c.k_cache.data_ptr(), c.v_cache.data_ptr(), ps, c.num_pages,
                  c.page_table.data_ptr(), c.page_table.shape[1], c.seq_lens.data_ptr(), B,
                  w.max_seq_len, Hq, Hkv, d, w.scale, split_tokens, out.data_ptr(), ws_ptr,
                  ws_bytes, stream)
        else:
            at = (c.q.data_ptr(), c.cu_seqlens_q.data_ptr(), c.prefix_lens.data_ptr(), B,
                  w.num_tokens, w.max_q_len, w.max_seq_len, c.k_cache.data_ptr(),
                  c.v_cache.data_ptr(), ps, c.num_pages, c.page_table.data_ptr(),
                  c.page_table.shape[1], Hq, Hkv, d, w.scale, out.data_ptr(), ws_ptr, ws_bytes,
                  stream)
        calls.append((st, at, out))
    f_store = lib.pkv_store_kv
    fused = is_decode and w.k_new is not None and fused_store
    f_attn = (lib.pkv_paged_attn_decode_shared if read_once else
              lib.pkv_decode_step if fused else
              lib.pkv_paged_attn_decode_multi if L > 1 else
              lib.pkv_paged_attn_decode if is_decode else lib.pkv_paged_attn_prefill)

    def step(i, ev=None):
        st, at, _ = calls[i % R]
        if st is not None and f_store(*st) != 0:
            raise RuntimeError("pkv_store_kv failed")
        if ev is not None:
            ev[0].record()
        if f_attn(*at) != 0:
            raise RuntimeError("attention call failed")
        if ev is not None:
            ev[1].record()

    warm_up(step, warmup, min_warm_s)
    # Whole-step throughput: K steps between two synchronisations, nothing
    # else enqueued.
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Per-call GPU time: a second pass with HIP events around each attention
    # call on the launch stream.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    for i in range(steps):
        step(i, events[i])
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in events]
    for _, _, out in calls:
        if not torch.isfinite(out.float()).all():
            raise RuntimeError(f"{name}: non-finite output")
    if R > 1 and not torch.equal(calls[0][2], calls[1][2]):
        raise RuntimeError(f"{name}: replicas disagree")
    # the split the kernels used: recorded by the split kernel in the first
    # word of the decode workspace (the device may pick a longer one); the
    # balanced launch shares each KV head's blocks evenly instead
    launch = None
    if is_decode and ws is not None and ws.numel() >= 256:
        rec = int(ws[:4].view(torch.int32)[0].item())
        split, launch = (None, "balanced") if rec < 0 else (rec, "split")
    res = dict(workload=w, replicas=R, split=split, launch=launch, fused=fused,
               ms_per_step=(t1 - t0) * 1e3 / steps,
               kernel_ms_mean=float(np.mean(kernel_ms)), kernel_ms_median=float(np.median(kernel_ms)),
               kernel_ms_min=float(np.min(kernel_ms)))
    return res


def time_store(name: str, steps: int, warmup: int):
    """store_kv alone on a workload's new rows (events around each call)."""
    import torch

    import paged_kv_attention_out_amd as pkv
    from paged_kv_attention_out_amd import inputs

    lib = pkv.lib()
    w = inputs.make_workload(name, device="cuda", poison=False)
    T = w.k_new.shape[0]
    nbytes = store_bytes(w)
    R = max(1, min(64, math.ceil(MIN_WORKING_SET / max(nbytes, 1))))
    stream = torch.cuda.current_stream().cuda_stream
    calls = []
    for _ in range(R):   # distinct source rows per replica; the pool is shared
        kn, vn = w.k_new.clone(), w.v_new.clone()
        calls.append((kn, vn, (kn.data_ptr(), vn.data_ptr(), w.out_loc.data_ptr(), T,
                               w.k_cache.data_ptr(), w.v_cache.data_ptr(),
                               w.k_cache.shape[0] * w.page_size, w.num_kv_heads, w.head_dim,
                               stream)))
    f = lib.pkv_store_kv
    warm_up(lambda i: f(*calls[i % R][2]), warmup)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        if f(*calls[i % R][2]) != 0:
            raise RuntimeError("pkv_store_kv failed")
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # device time per call: a captured graph of back-to-back calls (the
    # events above also time the host's launch rate when a call is short)
    per_graph = 20
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for i in range(per_graph):
            if f(*(calls[i % R][2][:-1] + (cs,))) != 0:
                raise RuntimeError("pkv_store_kv failed")
    g.replay()
    torch.cuda.synchronize()
    reps = max(5, steps // per_graph)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    dev_ms = e0.elapsed_time(e1) / (reps * per_graph)
    del g
    return {"rows": T, "us_mean": round(ms * 1e3, 2), "bytes": nbytes,
            "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "device_us_per_call": round(dev_ms * 1e3, 2),
            "device_GB/s": round(nbytes / (dev_ms * 1e-3) / 1e9, 1)}


def time_graph_buckets(name: str, steps: int, warmup: int,
                       buckets=(1, 2, 4, 8, 16, 32, 64)):
    """The decode step captured once per batch-size bucket with
    pkv_decode_graphs_create over the workload's buffers (sized for the
    largest bucket), replayed with the first `b` requests live and the rest
    padded (length 0).  Per bucket: the same live batch as an eager
    pkv_decode_step call, and the graph replay, each timed back to back by
    wall clock (host + device) and with HIP events on the stream around each
    call (device time).  The buffers are not replicated: every bucket's
    working set is at most the workload's (~150 MB for the Llama-shaped
    batch), for eager and graph alike."""
    import ctypes

    import torch

    import paged_kv_attention_out_amd as pkv
    from paged_kv_attention_out_amd import inputs

    lib = pkv.lib()
    w = inputs.make_workload(name, device="cuda", poison=False)
    B, Hq, Hkv, d, ps = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    buckets = [b for b in buckets if b <= B]
    nb = pkv.pkv_decode_graphs_workspace_bytes(buckets, Hq, Hkv, d, w.max_seq_len)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(w.q)
    lens = w.seq_lens.clone()
    graphs = pkv.pkv_decode_graphs_create(buckets, w.q, w.k_cache, w.v_cache, w.page_table,
                                          w.seq_lens, w.max_seq_len, w.scale, out,
                                          k_new=w.k_new, v_new=w.v_new, out_loc=w.out_loc,
                                          workspace=ws)
    stream = torch.cuda.current_stream().cuda_stream
    used = ctypes.c_int32(0)
    res = {}
    try:
        for b in buckets:
            w.seq_lens.copy_(lens)
            w.seq_lens[b:] = 0           # padding rows: the dummy request
            torch.cuda.synchronize()
            at = (w.q.data_ptr(), w.k_new.data_ptr(), w.v_new.data_ptr(), w.out_loc.data_ptr(),
                  w.k_cache.data_ptr(), w.v_cache.data_ptr(), ps, w.num_pages,
                  w.page_table.data_ptr(), w.page_table.shape[1], w.seq_lens.data_ptr(), b,
                  w.max_seq_len, Hq, Hkv, d, w.scale, 0, out.data_ptr(), ws.data_ptr(),
                  ws.numel(), stream)

            def eager(_i):
                if lib.pkv_decode_step(*at) != 0:
                    raise RuntimeError("pkv_decode_step failed")

            def replay(_i):
                if lib.pkv_decode_graphs_replay(graphs._handle, b, stream,
                                                ctypes.byref(used)) != 0:
                    raise RuntimeError("graph replay failed")

            rec = {"live": b, "bytes": int(decode_bytes_rows(w, b))}
            for kind, fn in (("eager", eager), ("graph", replay)):
                warm_up(fn, warmup)
                t0 = time.perf_counter()
                for i in range(steps):
                    fn(i)
                torch.cuda.synchronize()
                rec[f"{kind}_us_per_step"] = round((time.perf_counter() - t0) * 1e6 / steps, 2)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(steps)]
                for i in range(steps):
                    ev[i][0].record()
                    fn(i)
                    ev[i][1].record()
                torch.cuda.synchronize()
                rec[f"{kind}_gpu_us"] = round(float(np.mean([a.elapsed_time(e) for a, e in ev]))
                                              * 1e3, 2)
            if used.value != b:
                raise RuntimeError(f"bucket {b}: replay used bucket {used.value}")
            res[str(b)] = rec
    finally:
        graphs.destroy()
        w.seq_lens.copy_(lens)
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("graph replay: non-finite output")
    return res


def decode_bytes_rows(w, rows: int) -> int:
    """decode_bytes of the first `rows` requests of a decode workload, plus
    their store_kv rows."""
    n = w.seq_lens_np[:rows].astype(np.int64)
    ps = w.page_size
    kv = int(n.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = 2 * rows * w.num_q_heads * w.head_dim * 2
    meta = int(((n + ps - 1) // ps).sum()) * 4 + 4 * rows
    st = 2 * rows * w.num_kv_heads * w.head_dim * 2 * 2 + 4 * rows if w.k_new is not None else 0
    return kv + qo + meta + st


def time_metadata(steps: int):
    """The device-side metadata builders on the chunked-prefill and
    Llama-decode batches (events around each call)."""
    import torch

    import paged_kv_attention_out_amd as pkv
    from paged_kv_attention_out_amd import inputs

    res = {}
    wp = inputs.make_workload("chunked_prefill", device="cuda", poison=False)
    wd = inputs.make_workload("llama_decode", device="cuda", poison=False)
    cu = torch.empty_like(wp.cu_seqlens_q)
    loc_p = torch.empty_like(wp.out_loc)
    loc_d = torch.empty_like(wd.out_loc)
    calls = {
        "prefill_metadata": lambda: pkv.pkv_prefill_metadata(
            wp.seq_lens, wp.prefix_lens, wp.page_table, wp.page_size, wp.num_tokens,
            cu_seqlens_q=cu, out_loc=loc_p),
        "decode_metadata": lambda: pkv.pkv_decode_metadata(wd.seq_lens, wd.page_table,
                                                           wd.page_size, out_loc=loc_d),
    }
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        # Events around single calls of a few-microsecond kernel time the
        # host's launch rate; device time per call comes from a captured
        # graph of back-to-back calls, replayed between two events.
        per_graph = 20
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        reps = max(5, steps // per_graph)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"us_mean": round(float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3,
                                      2),
                     "device_us_per_call": round(e0.elapsed_time(e1) * 1e3 / (reps * per_graph),
                                                 2)}
        del g
    res["prefill_metadata"]["tokens"] = wp.num_tokens
    res["decode_metadata"]["requests"] = wd.num_seqs
    if not (torch.equal(cu, wp.cu_seqlens_q) and torch.equal(loc_p, wp.out_loc)
            and torch.equal(loc_d, wd.out_loc)):
        raise RuntimeError("metadata builders disagree with the workloads")
    return res


def decode_step_bytes(name: str) -> int:
    """decode_bytes + store_bytes of a named decode workload, from its
    lengths alone (no pool is built)."""
    from paged_kv_attention_out_amd import inputs

    cfg = inputs.WORKLOADS[name]
    n = inputs.draw_lengths(name).astype(np.int64)
    B, ps = cfg["num_seqs"], cfg["page_size"]
    hkv, hq, d, ql = cfg["num_kv_heads"], cfg["num_q_heads"], cfg["head_dim"], cfg.get("q_len", 1)
    kv = int(n.sum()) * hkv * d * 2 * 2
    qo = 2 * B * ql * hq * d * 2
    meta = int(((n + ps - 1) // ps).sum()) * 4 + 4 * B
    store = 2 * B * hkv * d * 2 * 2 + 4 * B if cfg["store_new"] else 0
    return kv + qo + meta + store


STREAM_BLOCKS = (1024, 2048, 4096, 8192)


def stream_reference(steps: int):
    """The device's plain streaming-read rate over each decode workload's
    step bytes: the library's reference read (`pkv_ref_stream_read`, one
    contiguous pass, 16-byte loads, eight in flight per thread) at several
    grid sizes, rotating over replicas so the working set (>= 1 GiB) exceeds
    the 256 MB Infinity Cache; mean per-call time by HIP events after a
    0.25 s warm-up.  torch's reduction and copy over the Llama-shaped step
    bytes are listed beside it.  A reference for the decode kernels'
    bandwidth, not part of the hot path."""
    import torch

    import paged_kv_attention_out_amd as pkv

    def timed(call):
        warm_up(call, 5)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            call(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3

    res = {}
    for name in ("llama_decode", "qwen_decode", "long_decode"):
        nbytes = decode_step_bytes(name) // 16 * 16
        R = max(1, math.ceil(MIN_WORKING_SET / nbytes))
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(R)]
        sink = torch.empty(int(pkv.lib().pkv_ref_stream_sink_words(max(STREAM_BLOCKS))),
                           dtype=torch.int32, device="cuda")
        out = {"bytes": nbytes, "replicas": R, "by_blocks": {}}
        for blocks in STREAM_BLOCKS:
            us = timed(lambda i: pkv.pkv_ref_stream_read(bufs[i % R], blocks, sink))
            out["by_blocks"][blocks] = {"us_mean": round(us, 2),
                                        "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        best = min(out["by_blocks"], key=lambda k: out["by_blocks"][k]["us_mean"])
        out["best"] = dict(out["by_blocks"][best], blocks=best)
        if name == PRIMARY:
            n = nbytes // 4
            f = [b.view(torch.float32)[:n] for b in bufs]
            dst = torch.empty_like(f[0])
            for kind in ("sum", "copy"):
                call = (lambda i: f[i % R].sum()) if kind == "sum" else \
                    (lambda i: dst.copy_(f[i % R]))
                us = timed(call)
                moved = n * 4 * (1 if kind == "sum" else 2)
                out["torch_" + kind] = {"us_mean": round(us, 2), "bytes": moved,
                                        "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
            del f, dst
        res[name] = out
        del bufs, sink
        torch.cuda.empty_cache()
    return res


# ---- CPU baseline (the oracle) ------------------------------------------------

def _host_request(w, r):
    """Host bf16 bits of request r's pages (gathered on the device) and its
    page-table row renumbered to them."""
    import torch

    from paged_kv_attention_out_amd import inputs

    ps = w.page_size
    n = int(w.seq_lens_np[r])
    k = max((n + ps - 1) // ps, 1)
    pages = torch.from_numpy(w.page_table_np[r, :k].astype(np.int64)).to(w.k_cache.device)
    return (inputs.bf16_bits(w.k_cache[pages]), inputs.bf16_bits(w.v_cache[pages]),
            np.arange(k, dtype=np.int32)[None])


def cpu_baseline(name: str, budget_s: float):
    """The float64 CPU oracle on a bounded sample of a workload: requests are
    taken in order (whole passes over the batch when it is small) until
    budget_s of oracle time has run.  Decode: store_kv of the request's new
    row (if any) and decode, in GB/s under the same counting rule as the GPU
    line.  Prefill: store_kv of the request's new rows and the causal prefill
    of all its rows and heads, in TFLOP/s of causal-visible pairs and new
    tokens/s.  Only the oracle calls are timed (host copies of the inputs
    are not)."""
    import torch

    from oracle import paged_attention as orc
    from paged_kv_attention_out_amd import inputs

    w = inputs.make_workload(name, device="cuda", poison=False)
    small = w.k_cache.numel() * 2 <= (1 << 30)   # keep host copies for later passes
    cache = {}
    q_all = inputs.bf16_bits(w.q)
    kn_all = None if w.k_new is None else inputs.bf16_bits(w.k_new)
    vn_all = None if w.v_new is None else inputs.bf16_bits(w.v_new)
    is_decode = w.kind == "decode"
    multi = is_decode and w.q.dim() == 4
    ps, hkv, d = w.page_size, w.num_kv_heads, w.head_dim
    done_bytes = done_flops = done_tokens = 0
    reqs = 0
    wall = cpu = 0.0
    r = 0
    while wall < budget_s and (r < w.num_seqs or small):
        rr = r % w.num_seqs
        kc, vc, row = cache[rr] if rr in cache else _host_request(w, rr)
        if small:
            cache[rr] = (kc, vc, row)
        n = int(w.seq_lens_np[rr])
        if is_decode:
            if kn_all is not None:
                slot = int(orc.slot_of(row[0], n - 1, ps))
                args = (kn_all[rr:rr + 1], vn_all[rr:rr + 1], np.array([slot], np.int32))
            c0, t0 = time.process_time(), time.perf_counter()
            kc2, vc2 = (orc.store_kv(kc, vc, *args) if kn_all is not None else (kc, vc))
            if multi:
                orc.decode_multi(q_all[rr:rr + 1], kc2, vc2, row, w.seq_lens_np[rr:rr + 1],
                                 w.scale)
            else:
                orc.decode(q_all[rr:rr + 1], kc2, vc2, row, w.seq_lens_np[rr:rr + 1], w.scale)
            wall += time.perf_counter() - t0
            cpu += time.process_time() - c0
            L = w.q.shape[1] if multi else 1
            done_bytes += (n * hkv * d * 2 * 2 + 2 * L * w.num_q_heads * d * 2 +
                           ((n + ps - 1) // ps) * 4 + 4 +
                           (2 * hkv * d * 2 * 2 + 4 if kn_all is not None else 0))
        else:
            s0, s1 = int(w.cu_seqlens_q[rr]), int(w.cu_seqlens_q[rr + 1])
            L, P = s1 - s0, int(w.prefix_lens_np[rr])
            slots = np.array([orc.slot_of(row[0], P + i, ps) for i in range(L)], np.int32)
            c0, t0 = time.process_time(), time.perf_counter()
            kc2, vc2 = orc.store_kv(kc, vc, kn_all[s0:s1], vn_all[s0:s1], slots)
            orc.prefill_dense(q_all[s0:s1], np.array([0, L], np.int32),
                              np.array([P], np.int32), kc2, vc2, row, w.scale)
            wall += time.perf_counter() - t0
            cpu += time.process_time() - c0
            done_flops += 4 * d * w.num_q_heads * (L * P + L * (L + 1) // 2)
            done_tokens += L
        reqs += 1
        r += 1
    cores = len(os.sched_getaffinity(0))
    what = ("store_kv + causal prefill" if not is_decode else
            ("store_kv + " if kn_all is not None else "") +
            (f"{w.q.shape[1]}-token decode" if multi else "decode"))
    rec = {"kind": "oracle", "cores": max(1, round(cpu / max(wall, 1e-9))),
           "sample": f"{reqs} request(s) of the {name} batch ({w.num_seqs} per batch), "
                     f"{what}, "
                     f"float64 NumPy, {cores} host cores available; {wall:.1f} s of oracle time"}
    if is_decode:
        rec.update(value=round(done_bytes / wall / 1e9, 4), unit="GB/s")
    else:
        rec.update(value=round(done_flops / wall / 1e12, 6), unit="TFLOP/s",
                   tokens_per_s=round(done_tokens / wall, 1))
    del w
    torch.cuda.empty_cache()
    return rec


# ---- main ------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default=PRIMARY)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--separate-store", action="store_true",
                    help="time pkv_store_kv + pkv_paged_attn_decode instead of pkv_decode_step")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for the primary workload (half that for "
                         "each other workload)")
    ap.add_argument("--only", default="", metavar="WORKLOAD",
                    help="only time one named workload (for profiler runs of a single "
                         "kernel), print its timing as JSON and exit")
    ap.add_argument("--read-once", action="store_true",
                    help="with --only shared_prefix_decode: time pkv_paged_attn_decode_shared "
                         "(the shared prefix read once per KV head)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (a known "
                         "byte count for scaling HBM traffic counters) and exit")
    ap.add_argument("--stream-ref", action="store_true",
                    help="only time torch's own read kernels (a float32 sum, a device "
                         "copy) over buffers of the Llama-shaped decode step's size and of "
                         "1 GiB, rotating over replicas of >= 1 GiB, as a reference for what "
                         "a plain stream over the same bytes costs, print JSON and exit")
    ap.add_argument("--segment-trace", default=None, metavar="CSV",
                    help="only summarise a rocprofv3 kernel-trace CSV of this script per "
                         "workload (no GPU use) and exit")
    args = ap.parse_args()
    if args.segment_trace:
        segment_trace(args.segment_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_out_amd as pkv

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 5}))
        return
    if args.stream_ref:
        print(json.dumps(stream_reference(args.steps)))
        return
    if args.only:
        r = time_workload(args.only, args.steps, args.warmup, args.split_tokens,
                          read_once=args.read_once)
        wa = r["workload"]
        rec = {"workload": args.only, "kernel_us_mean": round(r["kernel_ms_mean"] * 1e3, 2),
               "ms_per_step": round(r["ms_per_step"], 5), "replicas": r["replicas"]}
        if wa.kind == "decode":
            rec["bytes_per_launch"] = decode_bytes(wa) + (store_bytes(wa) if r["fused"] else 0)
        else:
            rec["flops_per_launch"] = prefill_flops(wa)
        print(json.dumps(rec))
        return
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} CUs={props.multi_processor_count} "
        f"arch={getattr(props, 'gcnArchName', '?')} lib={pkv.version()}")

    # the primary line: exactly --warmup untimed steps, then exactly --steps
    r = time_workload(args.workload, args.steps, args.warmup, args.split_tokens,
                      fused_store=not args.separate_store, min_warm_s=0.0)
    w = r["workload"]
    if w.kind != "decode":
        raise SystemExit("the primary line is a decode workload")
    step_bytes = decode_bytes(w) + store_bytes(w)
    value = step_bytes / (r["ms_per_step"] * 1e-3) / 1e9
    # bytes of the timed call: with the fused step it also moves the new rows
    call_bytes = step_bytes if r["fused"] else decode_bytes(w)
    achieved = call_bytes / (r["kernel_ms_mean"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "num_seqs": w.num_seqs,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size,
                   "seq_lens_sum": int(w.seq_lens_np.sum()), "seed": w.seed,
                   "replicas": r["replicas"], "split_tokens": r["split"], "launch": r["launch"],
                   "step": ("pkv_decode_step (store_kv fused into paged decode)" if r["fused"]
                            else "pkv_store_kv + pkv_paged_attn_decode"),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.workload),
                     "kernel": ("decode step call (decode_split_kernel with the fused store + "
                                "decode_combine_kernel)" if r["fused"] else
                                "decode call (decode_split_kernel + decode_combine_kernel)"),
                     "kernel_us_mean": round(r["kernel_ms_mean"] * 1e3, 2),
                     "kernel_us_median": round(r["kernel_ms_median"] * 1e3, 2),
                     "bytes_per_launch": call_bytes},
    }
    if not args.no_also:
        also = {}
        for name in ("qwen_decode", "long_decode", "chunked_prefill", "shared_prefix_decode"):
            torch.cuda.empty_cache()
            steps = max(10, args.steps // 10)
            a = time_workload(name, steps, max(3, args.warmup // 4))
            wa = a["workload"]
            if wa.kind == "decode":
                call_b = decode_bytes(wa) + (store_bytes(wa) if a["fused"] else 0)
                gbs = call_b / (a["kernel_ms_mean"] * 1e-3) / 1e9
                also[name] = {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                              "kernel_us_mean": round(a["kernel_ms_mean"] * 1e3, 2),
                              "ms_per_step": round(a["ms_per_step"], 4),
                              "tokens_per_s": round(wa.num_seqs / (a["ms_per_step"] * 1e-3), 1),
                              "split_tokens": a["split"], "launch": a["launch"],
                              "replicas": a["replicas"]}
                if name == "shared_prefix_decode":
                    # counting rule: shared pages count once per request; the
                    # distinct K/V bytes of the batch are far fewer
                    ub = unique_kv_bytes(wa)
                    also[name]["unique_kv_bytes"] = ub
                    also[name]["unique_GB/s"] = round(ub / (a["kernel_ms_mean"] * 1e-3) / 1e9, 1)
                    # the same step with the shared prefix read once per KV head
                    # (pkv_paged_attn_decode_shared)
                    torch.cuda.empty_cache()
                    b = time_workload(name, steps, max(3, args.warmup // 4), read_once=True)
                    ro_s = b["kernel_ms_mean"] * 1e-3
                    also[name]["read_once"] = {
                        "kernel_us_mean": round(b["kernel_ms_mean"] * 1e3, 2),
                        "ms_per_step": round(b["ms_per_step"], 4),
                        "GB/s": round(call_b / ro_s / 1e9, 1),
                        "unique_GB/s": round(ub / ro_s / 1e9, 1),
                        "unique_frac": round(ub / ro_s / 1e9 / HBM_PEAK_GBS, 4),
                        "tokens_per_s": round(wa.num_seqs / (b["ms_per_step"] * 1e-3), 1)}
                    del b
            else:
                tf = prefill_flops(wa) / (a["kernel_ms_mean"] * 1e-3) / 1e12
                also[name] = {"TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                              "kernel_us_mean": round(a["kernel_ms_mean"] * 1e3, 2),
                              "ms_per_step": round(a["ms_per_step"], 4),
                              "tokens_per_s": round(wa.num_tokens / (a["ms_per_step"] * 1e-3), 1),
                              "flops": prefill_flops(wa), "replicas": a["replicas"]}
            del a, wa
        also["store_kv"] = {n: time_store(n, max(20, args.steps // 5), 3)
                            for n in ("llama_decode", "chunked_prefill")}
        also["decode_graph_buckets"] = time_graph_buckets(args.workload,
                                                          max(20, args.steps // 5),
                                                          max(3, args.warmup // 20))
        also["metadata"] = time_metadata(max(20, args.steps // 5))
        # multi-token decode (4 draft tokens per request), and the same batch
        # through the prefill kernel for comparison
        torch.cuda.empty_cache()
        a = time_workload("spec_decode", max(10, args.steps // 10), max(3, args.warmup // 4))
        wa = a["workload"]
        gbs = decode_bytes(wa) / (a["kernel_ms_mean"] * 1e-3) / 1e9
        also["spec_decode"] = {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                               "kernel_us_mean": round(a["kernel_ms_mean"] * 1e3, 2),
                               "ms_per_step": round(a["ms_per_step"], 4),
                               "query_tokens_per_s":
                                   round(wa.num_tokens / (a["ms_per_step"] * 1e-3), 1),
                               "split_tokens": a["split"], "launch": a["launch"],
                              "replicas": a["replicas"]}
        del a, wa
        torch.cuda.empty_cache()
        a = time_workload("spec_decode", max(10, args.steps // 10), max(3, args.warmup // 4),
                          via_prefill=True)
        also["spec_decode"]["via_prefill_kernel_us_mean"] = round(a["kernel_ms_mean"] * 1e3, 2)
        del a
        line["also"] = also
        line["tokens_per_s"] = round(w.num_seqs / (r["ms_per_step"] * 1e-3), 1)
    if not args.no_cpu_baseline:
        del r, w
        torch.cuda.empty_cache()
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_budget)
        if "also" in line:
            for name in ("qwen_decode", "long_decode", "chunked_prefill",
                         "shared_prefix_decode", "spec_decode"):
                line["also"][name]["cpu_baseline"] = cpu_baseline(name, args.cpu_budget / 2)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

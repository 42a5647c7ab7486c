"""The decode step and the prefill call captured in a HIP graph and replayed.

The pages capture the decode step in CUDA graphs and replay it with new
batch contents in fixed buffers (mini-sglang "Engine Class", CUDA graph
capture; miniVLLM "Engine Architecture", prepare_decode and capture of
decode batches).  Every entry point here is stream-ordered, allocates
nothing, records no memset, and reads lengths and tables from device memory,
so one capture serves any batch whose sizes stay within the captured
bounds.  Each replay is checked against the float64 oracle of the contents
copied in just before it, and against an eager call on the same contents
(bit-exact: the kernels are deterministic)."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools

pytestmark = pytest.mark.gpu

B, HQ, HKV, D, PS = 8, 32, 8, 64, 16
MAX_LEN = 1024                     # captured bound on every request's length
WIDTH = MAX_LEN // PS
POOL = 8 * WIDTH + 8               # the same pool size for every batch


def _decode_batch(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, MAX_LEN + 1, size=B).astype(np.int32)
    return inputs.build_decode(B, HQ, HKV, D, PS, lens, seed=seed, device="cuda",
                               pool_pages=POOL, width=WIDTH, store_new=True)


def _static_like(w):
    names = ("q", "k_cache", "v_cache", "page_table", "seq_lens", "k_new", "v_new", "out_loc")
    return {n: torch.empty_like(getattr(w, n)) for n in names}


def _load(static, w):
    for n, t in static.items():
        t.copy_(getattr(w, n))


def test_decode_step_graph_replays():
    batches = [_decode_batch(300 + i) for i in range(3)]
    refs = []
    for w in batches:
        kc, vc = host_pools(w)
        refs.append(orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np,
                               w.scale))
    st = _static_like(batches[0])
    out = torch.empty_like(st["q"])
    ws = pkv.decode_workspace(B, HQ, HKV, D, MAX_LEN)
    scale = batches[0].scale

    def step():
        pkv.pkv_store_kv(st["k_new"], st["v_new"], st["out_loc"], st["k_cache"], st["v_cache"])
        pkv.pkv_paged_attn_decode(st["q"], st["k_cache"], st["v_cache"], st["page_table"],
                                  st["seq_lens"], MAX_LEN, scale, out=out, workspace=ws)

    _load(st, batches[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                      # first launch outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    _load(st, batches[0])
    with torch.cuda.graph(graph):
        step()
    for rep in range(2):
        for i, w in enumerate(batches):
            print(f"decode graph replay {rep}.{i}: lens {w.seq_lens_np.tolist()}", flush=True)
            _load(st, w)
            graph.replay()
            torch.cuda.synchronize()
            got = out.clone()
            assert_close(f64(got), refs[i], f"replay {rep}.{i}")
            _load(st, w)            # eager call on the same contents
            step()
            torch.cuda.synchronize()
            assert torch.equal(got, out), f"replay {rep}.{i} differs from the eager call"


def test_prefill_graph_replays_and_counter_resets():
    rng = np.random.default_rng(7)
    batches = []
    for i in range(3):
        prefix = rng.integers(0, 300, size=4).astype(np.int32)
        qlens = rng.integers(1, 200, size=4).astype(np.int32)
        batches.append(inputs.build_prefill(4, HQ, HKV, D, PS, prefix, qlens, seed=400 + i,
                                            device="cuda", pool_pages=4 * 32 + 4, width=32))
    T = 200 * 4
    refs = []
    for w in batches:
        kc, vc = host_pools(w)
        refs.append(orc.prefill_dense(inputs.bf16_bits(w.q), w.cu_seqlens_q.cpu().numpy(),
                                      w.prefix_lens_np, kc, vc, w.page_table_np, w.scale))
    # static buffers sized for T tokens; each batch fills its first num_tokens rows
    w0 = batches[0]
    st = {n: torch.empty_like(getattr(w0, n))
          for n in ("k_cache", "v_cache", "page_table", "prefix_lens", "cu_seqlens_q")}
    q_s = torch.zeros((T, HQ, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q_s)
    ws = torch.zeros(pkv.pkv_prefill_workspace_bytes(), dtype=torch.uint8, device="cuda")
    scale = w0.scale

    def load(w):
        for n, t in st.items():
            t.copy_(getattr(w, n))
        q_s.zero_()
        q_s[:w.num_tokens].copy_(w.q)
        out.zero_()
        # the new tokens' rows go into the pool before the call (the store
        # path is exercised by the decode graph)
        pkv.pkv_store_kv(w.k_new, w.v_new, w.out_loc, st["k_cache"], st["v_cache"])

    def call():
        pkv.pkv_paged_attn_prefill(q_s, st["cu_seqlens_q"], st["prefix_lens"], 200, 500,
                                   st["k_cache"], st["v_cache"], st["page_table"], scale,
                                   out=out, workspace=ws)

    load(w0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(2):
        for i, w in enumerate(batches):
            print(f"prefill graph replay {rep}.{i}: q_lens {np.diff(w.cu_seqlens_q.cpu().numpy()).tolist()}",
                  flush=True)
            load(w)
            graph.replay()
            torch.cuda.synchronize()
            assert int(ws.count_nonzero()) == 0, "the work counter must be zero after a replay"
            got = out[:w.num_tokens].clone()
            assert_close(f64(got), refs[i], f"prefill replay {rep}.{i}")
            load(w)
            call()
            torch.cuda.synchronize()
            assert torch.equal(got, out[:w.num_tokens]), "replay differs from the eager call"


# ---- graphs per batch-size bucket, padded with the dummy request ----------

BUCKETS = [1, 2, 4, 8, 16, 32, 64]
GB_MAX, GB_LEN, GB_WIDTH = 64, 1024, 64
GB_POOL = GB_MAX * GB_WIDTH + 8


def _bucket_batch(live, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, GB_LEN + 1, size=live).astype(np.int32)
    return inputs.build_decode(live, HQ, HKV, D, PS, lens, seed=seed, device="cuda",
                               pool_pages=GB_POOL, width=GB_WIDTH, store_new=True)


@pytest.mark.parametrize("workspace", ["caller", "fixed scratch"])
def test_decode_graph_buckets_with_padding(workspace):
    """pkv_decode_graphs_create captures the decode step for buckets
    1, 2, 4, ..., 64 (largest first) over fixed 64-row buffers; each step
    copies its batch into the first rows, pads the rest with the dummy request
    (length 0, the spare page, no slot), and replays the smallest bucket that
    holds it.  Checked per replay: the bucket chosen, the live rows against
    the oracle (store, then attention), zeros in the padded rows, rows past
    the bucket untouched, and the pools bit-exact: only the live requests'
    new slots change."""
    dev = "cuda"
    st = {
        "q": torch.zeros(GB_MAX, HQ, D, dtype=torch.bfloat16, device=dev),
        "k_new": torch.zeros(GB_MAX, HKV, D, dtype=torch.bfloat16, device=dev),
        "v_new": torch.zeros(GB_MAX, HKV, D, dtype=torch.bfloat16, device=dev),
        "out_loc": torch.full((GB_MAX,), -1, dtype=torch.int32, device=dev),
        "page_table": torch.zeros(GB_MAX, GB_WIDTH, dtype=torch.int32, device=dev),
        "seq_lens": torch.zeros(GB_MAX, dtype=torch.int32, device=dev),
        "k_cache": torch.zeros(GB_POOL + 1, PS, HKV, D, dtype=torch.bfloat16, device=dev),
        "v_cache": torch.zeros(GB_POOL + 1, PS, HKV, D, dtype=torch.bfloat16, device=dev),
    }
    out = torch.zeros(GB_MAX, HQ, D, dtype=torch.bfloat16, device=dev)
    ws = None
    if workspace == "caller":
        nb = pkv.pkv_decode_graphs_workspace_bytes(BUCKETS, HQ, HKV, D, GB_LEN)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(D)
    graphs = pkv.pkv_decode_graphs_create(
        BUCKETS, st["q"], st["k_cache"], st["v_cache"], st["page_table"], st["seq_lens"],
        GB_LEN, scale, out, k_new=st["k_new"], v_new=st["v_new"], out_loc=st["out_loc"],
        workspace=ws)
    try:
        for rep in range(2):
            for i, live in enumerate([1, 2, 3, 5, 9, 17, 33, 64, 48]):
                w = _bucket_batch(live, seed=500 + 10 * rep + i)
                kc, vc = host_pools(w)
                ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np,
                                 w.scale)
                # fixed buffers: the batch in the first rows, the dummy request after
                for n in ("q", "k_new", "v_new", "out_loc", "page_table", "seq_lens"):
                    st[n][:live].copy_(getattr(w, n))
                st["q"][live:].zero_()
                st["k_new"][live:].zero_()
                st["v_new"][live:].zero_()
                st["out_loc"][live:] = -1
                st["seq_lens"][live:] = 0
                st["page_table"][live:] = w.poison_page
                st["k_cache"].copy_(w.k_cache)
                st["v_cache"].copy_(w.v_cache)
                out.fill_(5.0)
                bucket = graphs.replay(live)
                torch.cuda.synchronize()
                expect = min(b for b in BUCKETS if b >= live)
                print(f"graph buckets ({workspace}) rep {rep}: {live} live -> bucket {bucket}",
                      flush=True)
                assert bucket == expect
                got = f64(out)
                assert_close(got[:live], ref, f"{live} live in bucket {bucket}")
                assert np.array_equal(got[live:bucket], np.zeros_like(got[live:bucket]))
                assert (got[bucket:] == 5.0).all(), "rows past the bucket were written"
                assert np.array_equal(inputs.bf16_bits(st["k_cache"]), kc)
                assert np.array_equal(inputs.bf16_bits(st["v_cache"]), vc)
    finally:
        graphs.destroy()


def test_decode_graph_bucket_limits():
    st = _static_like(_decode_batch(301))
    out = torch.empty_like(st["q"])
    graphs = pkv.pkv_decode_graphs_create(
        [2, 8], st["q"], st["k_cache"], st["v_cache"], st["page_table"], st["seq_lens"],
        MAX_LEN, 0.125, out, k_new=st["k_new"], v_new=st["v_new"], out_loc=st["out_loc"])
    try:
        assert graphs.replay(0) == 0              # nothing to do
        with pytest.raises(pkv.PKVError):
            graphs.replay(9)                      # above the largest bucket
        torch.cuda.synchronize()
    finally:
        graphs.destroy()

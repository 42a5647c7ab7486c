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

"""Multi-token decode (q_len new tokens per request, causal among them) on
the GPU against the float64 oracle.

Cases cover every (head_dim, query heads per KV head) pair, query tiles of
2, 4, 8 and 16 tokens, drafts wider than one block (several query slices per
KV head), drafts whose length is not a power of two, splits that start past
the first draft token's last visible key, contexts shorter than the draft
(rows with no visible key are zero) and empty requests.  With q_len = 1 the
call is bit-identical to plain decode."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, d, ps, seq_lens, q_len, split_tokens)
CASES = [
    (4, 8, 2, 64, 16, [2, 17, 64, 300], 2, 0),
    (4, 8, 2, 64, 16, [4, 33, 129, 1000], 4, 16),
    (3, 8, 2, 64, 16, [5, 81, 700], 5, 32),        # 2 slices of 4, one padded column
    (3, 8, 2, 64, 32, [3, 8, 1500], 8, 64),        # context shorter than the draft
    (2, 16, 4, 64, 16, [16, 900], 16, 0),          # 4 slices
    (3, 8, 4, 128, 16, [97, 3, 450], 3, 16),       # g = 2, tile 4; splits past the limit
    (3, 8, 4, 128, 256, [8, 300, 2000], 8, 256),   # g = 2, tile 8
    (2, 8, 4, 128, 64, [12, 777], 12, 48),         # g = 2, 2 slices of 8
    (3, 4, 4, 64, 16, [16, 200, 1111], 16, 0),     # g = 1, tile 16
    (3, 4, 4, 128, 128, [7, 130, 513], 7, 128),    # g = 1, tile 8
    (4, 16, 16, 64, 16, [1, 2, 3, 4], 4, 0),       # every request shorter than or equal to q_len
    (3, 16, 2, 64, 16, [2, 90, 1200], 2, 64),      # g = 8, tile 2
    (3, 32, 4, 128, 32, [5, 333, 900], 5, 0),      # g = 8, 3 slices of 2, one padded column
]


def _ids(c):
    return f"B{c[0]}-hq{c[1]}-hkv{c[2]}-d{c[3]}-ps{c[4]}-L{c[6]}-split{c[7]}"


def _oracle(w, seq_lens=None):
    kc, vc = host_pools(w)
    lens = w.seq_lens_np if seq_lens is None else seq_lens
    return orc.decode_multi(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, lens, w.scale)


def _run(w, split=0, out=None, workspace=None):
    return pkv.pkv_paged_attn_decode_multi(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                           w.max_seq_len, w.scale, out=out,
                                           workspace=workspace, split_tokens=split)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_decode_multi_small(case):
    B, hq, hkv, d, ps, lens, L, split = case
    print(f"decode_multi case {_ids(case)} lens={lens}", flush=True)
    w = inputs.build_decode(B, hq, hkv, d, ps, lens, seed=sum(lens) + 7 * L + d, device="cuda",
                            q_len=L)
    ref = _oracle(w)
    out = _run(w, split)
    torch.cuda.synchronize()
    got = f64(out)
    assert_close(got, ref, _ids(case))
    # rows whose position is negative are exactly zero
    for r, n in enumerate(lens):
        if n < L:
            assert np.array_equal(got[r, :L - n], np.zeros_like(got[r, :L - n]))


def test_decode_multi_empty_request_gives_zeros():
    w = inputs.build_decode(3, 8, 2, 64, 16, [50, 70, 90], seed=31, device="cuda", q_len=4)
    lens = w.seq_lens_np.copy()
    lens[1] = 0
    w.seq_lens[1] = 0
    ref = _oracle(w, lens)
    print("decode_multi empty request", flush=True)
    out = _run(w, 16)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.array_equal(got[1], np.zeros_like(got[1]))
    assert_close(got, ref, "empty request")


@pytest.mark.parametrize("hq,hkv,d,ps", [(32, 8, 64, 16), (16, 8, 128, 256), (8, 8, 64, 32)])
def test_decode_multi_one_token_is_decode(hq, hkv, d, ps):
    lens = [1, 31, 600, 2048]
    w = inputs.build_decode(4, hq, hkv, d, ps, lens, seed=41 + d, device="cuda")
    print(f"decode_multi q_len=1 vs decode hq{hq} hkv{hkv} d{d}", flush=True)
    a = pkv.pkv_paged_attn_decode(w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                  w.max_seq_len, w.scale, split_tokens=128)
    q4 = w.q.reshape(4, 1, hq, d)
    b = pkv.pkv_paged_attn_decode_multi(q4, w.k_cache, w.v_cache, w.page_table, w.seq_lens,
                                        w.max_seq_len, w.scale, split_tokens=128)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.reshape(4, hq, d).view(torch.int16))


def test_decode_multi_deterministic_and_split_independent():
    w = inputs.build_decode(6, 32, 8, 64, 16, [300, 1, 2048, 999, 64, 1500], seed=51,
                            device="cuda", q_len=8)
    ref = _oracle(w)
    print("decode_multi determinism / splits", flush=True)
    a = _run(w, 0)
    b = _run(w, 0)
    c = _run(w, 16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_close(f64(a), ref, "auto split")
    assert_close(f64(c), ref, "split 16")


def test_spec_decode_workload():
    w = inputs.make_workload("spec_decode", device="cuda")
    assert tuple(w.q.shape) == (64, 4, 32, 64)
    ref = _oracle(w)
    print(f"spec_decode workload lens {w.seq_lens_np.min()}..{w.seq_lens_np.max()}", flush=True)
    ws = torch.zeros(pkv.pkv_decode_multi_workspace_bytes(64, 4, 32, 8, 64, w.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    out = _run(w, 0, workspace=ws)
    torch.cuda.synchronize()
    mx, mean = assert_close(f64(out), ref, "spec_decode")
    print(f"spec_decode max|err| {mx:.3e} mean|err| {mean:.3e}", flush=True)

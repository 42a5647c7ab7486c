"""Pins for the CPU oracle, checked against things other than itself.

* a library routine: torch's scaled_dot_product_attention in float64 on
  unpaged inputs that the test pages itself;
* brute force with scalar Python arithmetic on tiny inputs;
* closed forms (q = 0 gives the mean of the visible V rows, constant V
  returns that row, one visible key returns its V row, two keys give the
  logistic weights, a huge scale gives the arg-max row);
* invariants (physical page permutation, GQA as MHA with repeated K/V
  heads, chunked prefill vs. one long prefill, decode as a one-row prefill,
  multi-token decode with one token as decode);
* the pages' one worked value: cu_seqlens_q = [0, 5, 8, 12];
* planted mistakes: each plausible slip in the oracle must trip a pin.
"""

import inspect
import json
import math
import os
import textwrap

import numpy as np
import pytest
import torch

from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# helpers (test side; they page contiguous data with their own loops)
# --------------------------------------------------------------------------

def _rand_bits(rng, shape):
    """bf16 bit patterns of N(0,1) draws (round to nearest even via torch)."""
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_t64(bits):
    """Widen bf16 bits with torch (a path independent of the oracle's)."""
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)


class Case:
    """Contiguous per-request K/V, paged into a shuffled pool by the test."""

    def __init__(self, seed, Hq, Hkv, d, ps, prefix, qlens, pool_extra=3):
        rng = np.random.default_rng(seed)
        self.Hq, self.Hkv, self.d, self.ps = Hq, Hkv, d, ps
        self.prefix = np.asarray(prefix, np.int32)
        self.qlens = np.asarray(qlens, np.int32)
        self.n = self.prefix + self.qlens
        B = len(self.n)
        need = [(int(n) + ps - 1) // ps for n in self.n]
        pool = sum(need) + pool_extra
        perm = rng.permutation(pool)
        W = max(need) if need else 1
        self.table = np.full((B, W), pool, np.int32)   # pool = spare page id
        self.k_cache = np.full((pool + 1, ps, Hkv, d), 0x7FC0, np.uint16)  # NaN
        self.v_cache = self.k_cache.copy()
        self.K, self.V = [], []
        off = 0
        for r in range(B):
            n = int(self.n[r])
            K = _rand_bits(rng, (n, Hkv, d))
            V = _rand_bits(rng, (n, Hkv, d))
            pages = perm[off:off + need[r]]
            off += need[r]
            self.table[r, :need[r]] = pages
            for t in range(n):
                self.k_cache[pages[t // ps], t % ps] = K[t]
                self.v_cache[pages[t // ps], t % ps] = V[t]
            self.K.append(K)
            self.V.append(V)
        T = int(self.qlens.sum())
        self.q = _rand_bits(rng, (T, Hq, d))
        self.cu = np.concatenate([[0], np.cumsum(self.qlens)]).astype(np.int32)
        self.scale = 1.0 / math.sqrt(d)

    def oracle_prefill(self):
        return orc.prefill(self.q, self.cu, self.prefix, self.k_cache,
                           self.v_cache, self.table, self.scale)

    def oracle_prefill_dense(self, heads=None):
        return orc.prefill_dense(self.q, self.cu, self.prefix, self.k_cache,
                                 self.v_cache, self.table, self.scale, heads=heads)

    def sdpa(self):
        """torch SDPA (float64) on the contiguous data, GQA by repetition."""
        g = self.Hq // self.Hkv
        out = np.full((len(self.q), self.Hq, self.d), np.nan)
        for r in range(len(self.n)):
            s0, s1 = self.cu[r], self.cu[r + 1]
            L, P, n = s1 - s0, int(self.prefix[r]), int(self.n[r])
            if L == 0:
                continue
            q = _bits_to_t64(self.q[s0:s1]).permute(1, 0, 2)          # [Hq, L, d]
            k = _bits_to_t64(self.K[r]).permute(1, 0, 2).repeat_interleave(g, 0)
            v = _bits_to_t64(self.V[r]).permute(1, 0, 2).repeat_interleave(g, 0)
            mask = torch.ones(L, n, dtype=torch.bool).tril(diagonal=P)
            o = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=mask, scale=self.scale)
            out[s0:s1] = o.permute(1, 0, 2).numpy()
        return out


# --------------------------------------------------------------------------
# pin checks, written as plain functions so the planted-mistake test can
# run them against a broken oracle
# --------------------------------------------------------------------------

def pin_store_kv_is_index_assignment():
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 1 << 16, size=(9, 16, 2, 8), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(9, 16, 2, 8), dtype=np.uint16)
    T = 40
    loc = rng.choice(9 * 16, size=T, replace=False).astype(np.int32)
    kn = rng.integers(0, 1 << 16, size=(T, 2, 8), dtype=np.uint16)
    vn = rng.integers(0, 1 << 16, size=(T, 2, 8), dtype=np.uint16)
    k2, v2 = orc.store_kv(kc, vc, kn, vn, loc)
    ek, ev = kc.reshape(-1, 2, 8).copy(), vc.reshape(-1, 2, 8).copy()
    ek[loc] = kn
    ev[loc] = vn
    assert np.array_equal(k2.reshape(-1, 2, 8), ek)
    assert np.array_equal(v2.reshape(-1, 2, 8), ev)
    assert np.array_equal(kc.reshape(-1, 2, 8)[loc], kc.reshape(-1, 2, 8)[loc])  # input untouched


def pin_vs_sdpa(g=2, d=16, ps=16, seed=3):
    c = Case(seed, Hq=2 * g, Hkv=2, d=d, ps=ps, prefix=[0, 5, 17, 33],
             qlens=[7, 1, 20, 4])
    got = c.oracle_prefill()
    ref = c.sdpa()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_decode_vs_sdpa(seed=4):
    c = Case(seed, Hq=8, Hkv=2, d=32, ps=16, prefix=[0, 15, 16, 40], qlens=[1, 1, 1, 1])
    got = orc.decode(c.q.reshape(4, 8, 32), c.k_cache, c.v_cache, c.table, c.n, c.scale)
    ref = c.sdpa().reshape(4, 8, 32)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_zero_query_is_mean_of_visible_v():
    c = Case(5, Hq=4, Hkv=2, d=8, ps=16, prefix=[3, 0], qlens=[5, 9])
    c.q[:] = 0
    got = c.oracle_prefill()
    for r in range(2):
        Vr = _bits_to_t64(c.V[r]).numpy()
        for i in range(int(c.qlens[r])):
            row = c.cu[r] + i
            vis = int(c.prefix[r]) + i + 1
            for h in range(4):
                exp = Vr[:vis, h // 2].mean(axis=0)
                np.testing.assert_allclose(got[row, h], exp, rtol=1e-12, atol=1e-14)


def pin_constant_v_returns_row():
    c = Case(6, Hq=4, Hkv=2, d=8, ps=16, prefix=[0, 11], qlens=[6, 3])
    rowval = _rand_bits(np.random.default_rng(60), (2, 8))
    for r in range(2):
        c.V[r][:] = rowval[None]
    # re-page V with the constant rows
    for r in range(2):
        for t in range(int(c.n[r])):
            c.v_cache[c.table[r, t // 16], t % 16] = rowval
    got = c.oracle_prefill()
    exp = _bits_to_t64(rowval).numpy()
    for h in range(4):
        np.testing.assert_allclose(got[:, h], np.broadcast_to(exp[h // 2], got[:, h].shape),
                                   rtol=1e-14, atol=0)


def pin_single_visible_key_returns_v():
    c = Case(7, Hq=2, Hkv=1, d=8, ps=16, prefix=[0], qlens=[1])
    got = orc.decode(c.q.reshape(1, 2, 8), c.k_cache, c.v_cache, c.table, c.n, c.scale)
    exp = _bits_to_t64(c.V[0][0]).numpy()
    assert np.array_equal(got[0, 0], exp[0]) and np.array_equal(got[0, 1], exp[0])


def pin_two_keys_logistic():
    c = Case(8, Hq=2, Hkv=2, d=8, ps=16, prefix=[1], qlens=[1])
    got = orc.decode(c.q.reshape(1, 2, 8), c.k_cache, c.v_cache, c.table, c.n, c.scale)
    q = _bits_to_t64(c.q[0]).numpy()
    K = _bits_to_t64(c.K[0]).numpy()
    V = _bits_to_t64(c.V[0]).numpy()
    for h in range(2):
        s0 = float(q[h] @ K[0, h]) * c.scale
        s1 = float(q[h] @ K[1, h]) * c.scale
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        exp = (1 - w1) * V[0, h] + w1 * V[1, h]
        np.testing.assert_allclose(got[0, h], exp, rtol=1e-12, atol=1e-14)


def pin_large_scale_is_argmax():
    c = Case(9, Hq=2, Hkv=1, d=16, ps=16, prefix=[30], qlens=[1])
    big = 1e4
    got = orc.decode(c.q.reshape(1, 2, 16), c.k_cache, c.v_cache, c.table, c.n, big)
    q = _bits_to_t64(c.q[0]).numpy()
    K = _bits_to_t64(c.K[0]).numpy()
    V = _bits_to_t64(c.V[0]).numpy()
    for h in range(2):
        s = K[:, 0] @ q[h]
        top = np.argsort(s)[-2:]
        assert (s[top[1]] - s[top[0]]) * big > 60  # the winner dominates
        np.testing.assert_allclose(got[0, h], V[top[1], 0], rtol=1e-12, atol=1e-12)


def pin_brute_force_scalar(seed=10):
    c = Case(seed, Hq=4, Hkv=2, d=4, ps=16, prefix=[2, 0], qlens=[3, 2])
    got = c.oracle_prefill()
    for r in range(2):
        q = _bits_to_t64(c.q[c.cu[r]:c.cu[r + 1]]).tolist()
        K = _bits_to_t64(c.K[r]).tolist()
        V = _bits_to_t64(c.V[r]).tolist()
        for i in range(int(c.qlens[r])):
            for h in range(4):
                kvh = h // 2
                vis = int(c.prefix[r]) + i + 1
                sc = [sum(q[i][h][e] * K[j][kvh][e] for e in range(4)) * c.scale
                      for j in range(vis)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                exp = [sum(w[j] * V[j][kvh][e] for j in range(vis)) / tot for e in range(4)]
                np.testing.assert_allclose(got[c.cu[r] + i, h], exp, rtol=1e-12, atol=1e-14)


def pin_page_permutation_invariance():
    w = inputs.build_prefill(3, 4, 2, 16, 16, [5, 0, 20], [9, 33, 4], seed=11)
    args = _wl_np(w)
    args["kc"], args["vc"] = orc.store_kv(args["kc"], args["vc"], inputs.bf16_bits(w.k_new),
                                          inputs.bf16_bits(w.v_new), w.out_loc_np)
    base = orc.prefill(args["q"], args["cu"], args["prefix"], args["kc"], args["vc"],
                       args["table"], w.scale)
    rng = np.random.default_rng(12)
    P = args["kc"].shape[0]
    perm = rng.permutation(P)            # new id of old page p is perm[p]
    kc2 = np.empty_like(args["kc"])
    vc2 = np.empty_like(args["vc"])
    kc2[perm] = args["kc"]
    vc2[perm] = args["vc"]
    table2 = perm[args["table"]].astype(np.int32)
    got = orc.prefill(args["q"], args["cu"], args["prefix"], kc2, vc2, table2, w.scale)
    assert np.isfinite(base).all()
    assert np.array_equal(base, got)


def pin_gqa_is_repeated_mha():
    c = Case(13, Hq=8, Hkv=2, d=8, ps=16, prefix=[4], qlens=[6])
    got = c.oracle_prefill()
    g = 4
    kc = np.repeat(c.k_cache, g, axis=2)
    vc = np.repeat(c.v_cache, g, axis=2)
    mha = orc.prefill(c.q, c.cu, c.prefix, kc, vc, c.table, c.scale)
    np.testing.assert_allclose(got, mha, rtol=0, atol=0)


def pin_chunked_prefill_matches_full():
    c = Case(14, Hq=4, Hkv=2, d=8, ps=16, prefix=[0], qlens=[40])
    full = c.oracle_prefill()
    # same pool, same request, but the first 25 tokens count as cached prefix
    cu = np.array([0, 15], np.int32)
    part = orc.prefill(c.q[25:], cu, np.array([25], np.int32), c.k_cache,
                       c.v_cache, c.table, c.scale)
    np.testing.assert_allclose(part, full[25:], rtol=1e-13, atol=1e-15)


def pin_decode_is_one_row_prefill():
    w = inputs.build_decode(3, 4, 2, 16, 16, [1, 17, 50], seed=15)
    a = _wl_np(w)
    dec = orc.decode(a["q"], a["kc"], a["vc"], a["table"], w.seq_lens_np, w.scale)
    assert np.isfinite(dec).all()
    pre = orc.prefill(a["q"], np.arange(4, dtype=np.int32), w.seq_lens_np - 1,
                      a["kc"], a["vc"], a["table"], w.scale)
    np.testing.assert_allclose(dec, pre, rtol=0, atol=0)


def pin_golden_cu_seqlens():
    with open(os.path.join(GOLDEN, "cu_seqlens_example.json")) as f:
        ex = json.load(f)
    c = Case(16, Hq=2, Hkv=1, d=8, ps=16, prefix=[0, 0, 0], qlens=ex["q_lens"])
    assert c.cu.tolist() == ex["cu_seqlens_q"]
    got = orc.prefill(c.q, np.array(ex["cu_seqlens_q"], np.int32), c.prefix,
                      c.k_cache, c.v_cache, c.table, c.scale)
    np.testing.assert_allclose(got, c.sdpa(), rtol=1e-12, atol=1e-12)


def pin_decode_multi_vs_sdpa(seed=17):
    L = 4
    c = Case(seed, Hq=8, Hkv=2, d=16, ps=16, prefix=[0, 12, 29, 60], qlens=[L] * 4)
    got = orc.decode_multi(c.q.reshape(4, L, 8, 16), c.k_cache, c.v_cache, c.table, c.n,
                           c.scale)
    np.testing.assert_allclose(got, c.sdpa().reshape(4, L, 8, 16), rtol=1e-12, atol=1e-12)


def pin_decode_multi_one_token_is_decode(seed=18):
    c = Case(seed, Hq=4, Hkv=2, d=8, ps=16, prefix=[0, 7, 31], qlens=[1, 1, 1])
    one = orc.decode_multi(c.q.reshape(3, 1, 4, 8), c.k_cache, c.v_cache, c.table, c.n,
                           c.scale)
    dec = orc.decode(c.q.reshape(3, 4, 8), c.k_cache, c.v_cache, c.table, c.n, c.scale)
    assert np.isfinite(dec).all()
    np.testing.assert_allclose(one[:, 0], dec, rtol=0, atol=0)


def pin_decode_multi_short_context(seed=19):
    # 3 tokens in the pool but 5 query rows: rows 0 and 1 would sit at
    # positions -2 and -1 and see nothing (zeros); rows 2..4 are the three
    # tokens' causal attention; an empty request is all zero.
    c = Case(seed, Hq=4, Hkv=2, d=8, ps=16, prefix=[0], qlens=[3])
    extra = _rand_bits(np.random.default_rng(190), (2, 4, 8))
    q = np.concatenate([extra, c.q])[None]
    lens = c.n.copy()
    got = orc.decode_multi(q, c.k_cache, c.v_cache, c.table, lens, c.scale)
    assert np.array_equal(got[0, :2], np.zeros((2, 4, 8)))
    np.testing.assert_allclose(got[0, 2:], c.sdpa(), rtol=1e-12, atol=1e-12)
    empty = orc.decode_multi(q, c.k_cache, c.v_cache, c.table, np.array([0], np.int32),
                             c.scale)
    assert np.array_equal(empty, np.zeros_like(empty))


# ---- prefill_dense: the block-at-a-time form every GPU prefill test uses ----

def pin_prefill_dense_vs_sdpa(g=2, d=16, ps=16, seed=30):
    # ragged requests, prefixes that are not page multiples, an empty request
    c = Case(seed, Hq=2 * g, Hkv=2, d=d, ps=ps, prefix=[0, 5, 17, 33, 9],
             qlens=[7, 1, 20, 0, 4])
    np.testing.assert_allclose(c.oracle_prefill_dense(), c.sdpa(), rtol=1e-12, atol=1e-12)


def pin_prefill_dense_heads_subset(seed=31):
    # asked-for heads match SDPA; every other head stays NaN
    c = Case(seed, Hq=8, Hkv=2, d=8, ps=16, prefix=[3, 0], qlens=[12, 30])
    got = c.oracle_prefill_dense(heads=[1, 6])
    ref = c.sdpa()
    np.testing.assert_allclose(got[:, [1, 6]], ref[:, [1, 6]], rtol=1e-12, atol=1e-12)
    assert np.isnan(got[:, [0, 2, 3, 4, 5, 7]]).all()


def pin_prefill_dense_brute_force_scalar(seed=32):
    c = Case(seed, Hq=4, Hkv=2, d=4, ps=16, prefix=[2, 0, 5], qlens=[3, 2, 0])
    got = c.oracle_prefill_dense()
    for r in range(3):
        q = _bits_to_t64(c.q[c.cu[r]:c.cu[r + 1]]).tolist()
        K = _bits_to_t64(c.K[r]).tolist()
        V = _bits_to_t64(c.V[r]).tolist()
        for i in range(int(c.qlens[r])):
            for h in range(4):
                kvh = h // 2
                vis = int(c.prefix[r]) + i + 1
                sc = [sum(q[i][h][e] * K[j][kvh][e] for e in range(4)) * c.scale
                      for j in range(vis)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                tot = sum(w)
                exp = [sum(w[j] * V[j][kvh][e] for j in range(vis)) / tot for e in range(4)]
                np.testing.assert_allclose(got[c.cu[r] + i, h], exp, rtol=1e-12, atol=1e-14)


def pin_prefill_dense_zero_query_is_mean(seed=33):
    # q = 0: row i of request r is the mean of V rows 0 .. prefix_r + i
    c = Case(seed, Hq=4, Hkv=2, d=8, ps=16, prefix=[3, 0, 16], qlens=[5, 9, 17])
    c.q[:] = 0
    got = c.oracle_prefill_dense()
    for r in range(3):
        Vr = _bits_to_t64(c.V[r]).numpy()
        for i in range(int(c.qlens[r])):
            vis = int(c.prefix[r]) + i + 1
            for h in range(4):
                np.testing.assert_allclose(got[c.cu[r] + i, h], Vr[:vis, h // 2].mean(axis=0),
                                           rtol=1e-12, atol=1e-14)


def pin_prefill_dense_chunked_matches_full(seed=34):
    c = Case(seed, Hq=4, Hkv=2, d=8, ps=16, prefix=[0], qlens=[40])
    full = c.oracle_prefill_dense()
    part = orc.prefill_dense(c.q[25:], np.array([0, 15], np.int32), np.array([25], np.int32),
                             c.k_cache, c.v_cache, c.table, c.scale)
    np.testing.assert_allclose(part, full[25:], rtol=1e-13, atol=1e-15)


def pin_prefill_dense_single_key_returns_v(seed=35):
    c = Case(seed, Hq=2, Hkv=1, d=8, ps=16, prefix=[0], qlens=[1])
    got = c.oracle_prefill_dense()
    exp = _bits_to_t64(c.V[0][0]).numpy()
    assert np.array_equal(got[0, 0], exp[0]) and np.array_equal(got[0, 1], exp[0])


def pin_prefill_dense_page_permutation_invariance(seed=36):
    w = inputs.build_prefill(3, 4, 2, 16, 16, [5, 0, 20], [9, 33, 4], seed=seed)
    a = _wl_np(w)
    a["kc"], a["vc"] = orc.store_kv(a["kc"], a["vc"], inputs.bf16_bits(w.k_new),
                                    inputs.bf16_bits(w.v_new), w.out_loc_np)
    base = orc.prefill_dense(a["q"], a["cu"], a["prefix"], a["kc"], a["vc"], a["table"],
                             w.scale)
    perm = np.random.default_rng(seed).permutation(a["kc"].shape[0])
    kc2 = np.empty_like(a["kc"])
    vc2 = np.empty_like(a["vc"])
    kc2[perm] = a["kc"]
    vc2[perm] = a["vc"]
    got = orc.prefill_dense(a["q"], a["cu"], a["prefix"], kc2, vc2,
                            perm[a["table"]].astype(np.int32), w.scale)
    assert np.isfinite(base).all()
    assert np.array_equal(base, got)


def _wl_np(w):
    return dict(q=inputs.bf16_bits(w.q), kc=inputs.bf16_bits(w.k_cache),
                vc=inputs.bf16_bits(w.v_cache), table=w.page_table_np,
                cu=w.cu_seqlens_q.numpy(), prefix=w.prefix_lens_np)


PINS = [pin_store_kv_is_index_assignment, pin_vs_sdpa, pin_decode_vs_sdpa,
        pin_zero_query_is_mean_of_visible_v, pin_constant_v_returns_row,
        pin_single_visible_key_returns_v, pin_two_keys_logistic,
        pin_large_scale_is_argmax, pin_brute_force_scalar,
        pin_page_permutation_invariance, pin_gqa_is_repeated_mha,
        pin_chunked_prefill_matches_full, pin_decode_is_one_row_prefill,
        pin_golden_cu_seqlens, pin_decode_multi_vs_sdpa,
        pin_decode_multi_one_token_is_decode, pin_decode_multi_short_context,
        pin_prefill_dense_vs_sdpa, pin_prefill_dense_heads_subset,
        pin_prefill_dense_brute_force_scalar, pin_prefill_dense_zero_query_is_mean,
        pin_prefill_dense_chunked_matches_full, pin_prefill_dense_single_key_returns_v,
        pin_prefill_dense_page_permutation_invariance]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("g,d,ps", [(1, 64, 16), (2, 128, 256), (4, 64, 16), (4, 8, 32),
                                    (8, 64, 16), (8, 128, 32)])
def test_vs_sdpa_shapes(g, d, ps):
    pin_vs_sdpa(g=g, d=d, ps=ps, seed=100 + g + d + ps)
    pin_prefill_dense_vs_sdpa(g=g, d=d, ps=ps, seed=200 + g + d + ps)


def test_bf16_widening_exact():
    x = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3FC0],
                 np.uint16)
    got = orc.bf16_to_f64(x)
    exp = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 2.0 ** -133, 3.3895313892515355e38, 1.5]
    assert np.array_equal(got[:6], exp[:6])
    assert got[6] == exp[6] and got[7] == exp[7] and got[8] == exp[8]
    assert np.isnan(orc.bf16_to_f64(np.array([0x7FC0], np.uint16)))[0]


# --------------------------------------------------------------------------
# planted mistakes: every one of these slips must make some pin fail
# --------------------------------------------------------------------------

def _wrong_slots(row, n, ps):                      # page and offset swapped
    pos = np.arange(n, dtype=np.int64)
    return pos % ps * ps + row[pos // ps].astype(np.int64)


def _wrong_head(h, hq, hkv):                       # interleaved instead of grouped
    return h % hkv


def _wrong_visible(first, rows, keys):             # off by one on the diagonal
    r = first + np.arange(rows)[:, None]
    return np.arange(keys)[None, :] < r


def _wrong_visible_open(first, rows, keys):        # no causal mask at all
    return np.ones((rows, keys), bool)


def _make_wrong_attend(kind):
    def attend(q, k, v, first, scale):
        s = q @ k.T
        if kind != "no_scale":
            s = s * scale
        s = np.where(orc.visible(first, q.shape[0], k.shape[0]), s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        if kind == "col_norm":
            e = np.where(np.isfinite(s), e, 0)
            return (e / np.maximum(e.sum(axis=0, keepdims=True), 1e-300)) @ v
        if kind == "transposed_k":
            s2 = (q @ k[:, ::-1].T) * scale
            s2 = np.where(orc.visible(first, q.shape[0], k.shape[0]), s2, -np.inf)
            e = np.exp(s2 - s2.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)) @ v
    return attend


def _wrong_store(kc, vc, kn, vn, loc):             # K and V rows swapped
    return orc.__dict__["_real_store"](kc, vc, vn, kn, loc)


MUTANTS = {
    "slots_swapped": ("request_slots", _wrong_slots),
    "head_interleaved": ("kv_head_of", _wrong_head),
    "mask_off_by_one": ("visible", _wrong_visible),
    "mask_missing": ("visible", _wrong_visible_open),
    "scale_dropped": ("attend", _make_wrong_attend("no_scale")),
    "softmax_wrong_axis": ("attend", _make_wrong_attend("col_norm")),
    "keys_reversed": ("attend", _make_wrong_attend("transposed_k")),
    "store_k_v_swapped": ("store_kv", _wrong_store),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(orc.__dict__, "_real_store", orc.store_kv)
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # a failed assertion or a crash both count
            caught.append(pin.__name__)
    assert caught, f"no pin notices the planted mistake {name}"


# Mistakes planted in the text of one oracle function, the way a slip would
# be typed: ``old`` becomes ``new`` in that function's source, the function
# is recompiled against the oracle module's names and swapped in, and at
# least one pin must fail.  These reach functions (prefill_dense, decode,
# decode_multi) whose arithmetic the helper-level mutants above do not touch.
SOURCE_MUTANTS = {
    "dense_mask_off_by_one": ("prefill_dense", "P, scale)", "P + 1, scale)"),
    "dense_mask_one_early": ("prefill_dense", "P, scale)", "P - 1, scale)"),
    "dense_prefix_ignored": ("prefill_dense", "P = int(prefix_lens[r])", "P = 0"),
    "dense_heads_interleaved": ("prefill_dense", "kv_head_of(h, Hq, Hkv)", "h % Hkv"),
    "dense_scale_dropped": ("prefill_dense", "P, scale)", "P, 1.0)"),
    "dense_k_v_swapped": ("prefill_dense", "kr[:, kvh], vr[:, kvh]",
                          "vr[:, kvh], kr[:, kvh]"),
    "dense_heads_ignored": ("prefill_dense", "(range(Hq) if heads is None else heads)",
                            "range(Hq)"),
    "decode_position_one_early": ("decode", "n - 1, scale)", "n - 2, scale)"),
    "decode_last_key_dropped": ("decode", "attend(qr[h][None, :], kr[:, kvh], vr[:, kvh]",
                                "attend(qr[h][None, :], kr[:-1, kvh], vr[:-1, kvh]"),
    "prefill_row_one_late": ("prefill", "P + int(i), scale)", "P + int(i) + 1, scale)"),
    "multi_mask_off_by_one": ("decode_multi", "first + t0, scale)", "first + t0 + 1, scale)"),
    "multi_first_position": ("decode_multi", "first = n - L ", "first = n - L + 1 "),
}


def _source_mutant(name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(orc, name)))
    assert old in src, f"{name} no longer contains {old!r}: update the planted mistake"
    namespace = dict(orc.__dict__)
    exec(compile(src.replace(old, new, 1), f"<planted mistake in {name}>", "exec"), namespace)
    return namespace[name]


@pytest.mark.parametrize("mutant", sorted(SOURCE_MUTANTS))
def test_planted_source_mistake_is_caught(mutant, monkeypatch):
    name, old, new = SOURCE_MUTANTS[mutant]
    monkeypatch.setattr(orc, name, _source_mutant(name, old, new))
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # a failed assertion or a crash both count
            caught.append(pin.__name__)
    assert caught, f"no pin notices the planted mistake {mutant}"


# ---- step metadata (prepare_prefill / prepare_decode) -------------------------

def test_prefill_metadata_golden_cu_seqlens():
    """The pages' example: three sequences with 5, 3 and 4 new tokens give
    cu_seqlens_q = [0, 5, 8, 12]."""
    g = json.load(open(os.path.join(GOLDEN, "cu_seqlens_example.json")))
    lens = np.array(g["q_lens"], np.int32)
    table = np.zeros((len(lens), 4), np.int32)
    cu, slots = orc.prefill_metadata(lens, np.zeros_like(lens), table, 16)
    assert cu.tolist() == g["cu_seqlens_q"]
    assert len(slots) == cu[-1]


def test_metadata_hand_example():
    """Page row [7, 2], page size 4: positions 3, 4, 5 sit in page 7 row 3
    (slot 31), then page 2 rows 0, 1 (slots 8, 9)."""
    table = np.array([[7, 2], [5, 0]], np.int32)
    cu, slots = orc.prefill_metadata([6, 2], [3, 0], table, 4)
    assert cu.tolist() == [0, 3, 5]
    assert slots.tolist() == [31, 8, 9, 20, 21]
    assert orc.decode_slots([6, 0], table, 4).tolist() == [9, -1]
    # a position past the row's pages has no slot
    assert orc.decode_slots([9], table[:1], 4).tolist() == [-1]
    # more cached tokens than tokens: nothing new
    cu, slots = orc.prefill_metadata([3], [5], table[:1], 4)
    assert cu.tolist() == [0, 0] and len(slots) == 0


def test_metadata_matches_the_generators():
    """The input generators place new tokens with their own slot code; the
    oracle's metadata must name the same slots."""
    w = inputs.build_decode(5, 8, 2, 64, 16, [1, 17, 300, 2048, 64], seed=3, store_new=True)
    assert np.array_equal(orc.decode_slots(w.seq_lens_np, w.page_table_np, 16), w.out_loc_np)
    w = inputs.build_prefill(3, 8, 2, 64, 32, [0, 40, 33], [70, 1, 200], seed=4)
    cu, slots = orc.prefill_metadata(w.seq_lens_np, w.prefix_lens_np, w.page_table_np, 32)
    assert np.array_equal(cu, w.cu_seqlens_q.numpy())
    assert np.array_equal(slots, w.out_loc_np)

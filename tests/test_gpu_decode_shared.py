"""Decode over requests that share cached prefixes, with every shared
prefix read once per group (pkv_paged_attn_decode_shared), against the
float64 oracle of plain decode on the same page tables.

Cases: the shared-prefix workload (64 requests sharing a 1024-token prefix,
with the new token's store), several groups per batch with different shared
lengths (one not a multiple of the page size, one of zero, a group of one),
a group wider than one query tile of the shared pass, every (head_dim,
query heads per KV head) pair, explicit and automatic splits, and requests
whose whole context is the shared prefix."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import assert_close, f64, host_pools

pytestmark = pytest.mark.gpu


def _grouped(hq, hkv, d, ps, groups, seed, store):
    """A decode batch whose group members alias their group's first member's
    first pages for the shared tokens.  groups: list of (members, shared)."""
    rng = np.random.default_rng(seed)
    lens, shared = [], []
    for members, sh in groups:
        k = -(-sh // ps)
        lo = k * ps + 1 if store else max(sh, 1)
        for i in range(members):
            # (without the store, the first request of a group may end exactly
            # at its shared prefix)
            n = sh if (not store and sh > 0 and i == 0) else lo + int(rng.integers(0, 700))
            lens.append(max(n, 1))
            shared.append(sh)
    B = len(lens)
    w = inputs.build_decode(B, hq, hkv, d, ps, np.array(lens, np.int32), seed=seed,
                            device="cuda", store_new=store)
    table = w.page_table_np.copy()
    cu = [0]
    for members, sh in groups:
        first = cu[-1]
        k = -(-sh // ps)
        for m in range(first, first + members):
            table[m, :k] = table[first, :k]
        cu.append(first + members)
    w.page_table_np = table
    w.page_table = torch.from_numpy(table).cuda()
    return (w, torch.tensor(cu, dtype=torch.int32, device="cuda"),
            torch.tensor(shared, dtype=torch.int32, device="cuda"),
            max(m for m, _ in groups), max(sh for _, sh in groups))


def _run(w, cu, shared, max_group, max_shared, split=0):
    store = w.k_new is not None
    return pkv.pkv_paged_attn_decode_shared(
        w.q, w.k_cache, w.v_cache, w.page_table, w.seq_lens, w.max_seq_len, cu, shared,
        max_group, max_shared, w.scale, k_new=w.k_new if store else None,
        v_new=w.v_new if store else None, out_loc=w.out_loc if store else None,
        split_tokens=split)


def test_shared_prefix_workload():
    """64 Llama-shaped requests sharing a 1024-token prefix, with the store of
    each request's new token: every element against the oracle, the pools
    bit-exact, and within tolerance of pkv_decode_step (which streams the
    prefix once per request)."""
    w = inputs.make_workload("shared_prefix_decode", device="cuda")
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
    k0, v0 = w.k_cache.clone(), w.v_cache.clone()
    cu = torch.tensor([0, w.num_seqs], dtype=torch.int32, device="cuda")
    shared = torch.full((w.num_seqs,), 1024, dtype=torch.int32, device="cuda")
    out = _run(w, cu, shared, w.num_seqs, 1024)
    torch.cuda.synchronize()
    got = f64(out)
    print("shared prefix workload", assert_close(got, ref, "shared prefix workload"))
    assert np.array_equal(inputs.bf16_bits(w.k_cache), kc)
    assert np.array_equal(inputs.bf16_bits(w.v_cache), vc)
    w.k_cache.copy_(k0)
    w.v_cache.copy_(v0)
    plain = pkv.pkv_decode_step(w.q, w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache,
                                w.page_table, w.seq_lens, w.max_seq_len, w.scale)
    torch.cuda.synchronize()
    assert np.abs(got - f64(plain)).max() <= 2e-2


# (Hq, Hkv, d, ps, groups as (members, shared tokens), store, split)
CASES = [
    (32, 8, 64, 16, [(3, 256), (1, 0), (6, 512), (70, 100)], True, 0),
    (32, 8, 64, 16, [(5, 1024), (2, 64)], False, 64),
    (16, 8, 128, 256, [(4, 512), (4, 768)], True, 0),
    (16, 8, 128, 256, [(4, 512), (4, 768)], False, 256),
    (16, 2, 64, 32, [(5, 320), (2, 0)], False, 0),        # 8 query heads per KV head
    (4, 4, 128, 64, [(3, 128), (2, 640)], True, 128),      # one query head per KV head
    (8, 4, 64, 16, [(40, 2000)], False, 0),                 # long prefix, 16 key splits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"hq{c[0]}-hkv{c[1]}-d{c[2]}-ps{c[3]}-"
                         f"g{len(c[4])}-{'store' if c[5] else 'plain'}-split{c[6]}")
def test_shared_groups(case):
    hq, hkv, d, ps, groups, store, split = case
    print(f"shared groups {case}", flush=True)
    w, cu, shared, mg, ms = _grouped(hq, hkv, d, ps, groups, seed=hq + d + ps + len(groups),
                                     store=store)
    kc, vc = host_pools(w)
    ref = orc.decode(inputs.bf16_bits(w.q), kc, vc, w.page_table_np, w.seq_lens_np, w.scale)
    out = _run(w, cu, shared, mg, ms, split)
    torch.cuda.synchronize()
    print(assert_close(f64(out), ref, f"groups {groups}"))
    if store:
        assert np.array_equal(inputs.bf16_bits(w.k_cache), kc)
        assert np.array_equal(inputs.bf16_bits(w.v_cache), vc)

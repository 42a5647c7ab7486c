"""Device-side step metadata against the oracle, bit-exact: prefill
cu_seqlens_q and slot_mapping (miniVLLM "Engine Architecture",
prepare_prefill) and the decode step's slot_mapping (prepare_decode)."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

pytestmark = pytest.mark.gpu


def _table(rng, B, width, pool):
    return rng.permutation(pool)[:B * width].reshape(B, width).astype(np.int32)


@pytest.mark.parametrize("B,ps,width,seed", [(1, 16, 4, 1), (7, 16, 40, 2), (33, 48, 9, 3),
                                              (300, 256, 3, 4),
                                              (2500, 16, 3, 8)])   # three chunks of the scan
def test_prefill_metadata_matches_oracle(B, ps, width, seed):
    rng = np.random.default_rng(seed)
    table = _table(rng, B, width, B * width + 50)
    seq = rng.integers(0, width * ps + 1, size=B).astype(np.int32)
    pre = (seq * rng.random(B)).astype(np.int32)
    pre[::5] = seq[::5] + 3          # more cached than present: no new token
    seq[::7] = 0                     # empty requests
    cu_ref, slots_ref = orc.prefill_metadata(seq, pre, table, ps)
    total = int(cu_ref[-1])
    print(f"B={B} ps={ps} total new tokens {total}", flush=True)
    dev = lambda a: torch.from_numpy(a).cuda()
    for cap in (total, max(total // 2, 0)):
        out_loc = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
        cu, out_loc = pkv.pkv_prefill_metadata(dev(seq), dev(pre), dev(table), ps, cap,
                                               out_loc=out_loc)
        torch.cuda.synchronize()
        assert np.array_equal(cu.cpu().numpy(), cu_ref)
        got = out_loc.cpu().numpy()
        assert np.array_equal(got[:cap], slots_ref[:cap])
        if cap < out_loc.numel():
            assert (got[cap:] == -7).all(), "entries past max_tokens must not be written"


@pytest.mark.parametrize("B,ps,width,seed", [(1, 16, 4, 5), (64, 16, 128, 6), (129, 32, 7, 7)])
def test_decode_metadata_matches_oracle(B, ps, width, seed):
    rng = np.random.default_rng(seed)
    table = _table(rng, B, width, B * width + 10)
    seq = rng.integers(0, width * ps + 3, size=B).astype(np.int32)   # some past the row
    seq[::9] = 0                                                     # padding rows
    ref = orc.decode_slots(seq, table, ps)
    got = pkv.pkv_decode_metadata(torch.from_numpy(seq).cuda(), torch.from_numpy(table).cuda(),
                                  ps)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy()[:B], ref)


def test_metadata_feeds_the_workloads():
    """The built metadata equals what the workload generators hand to the
    kernels (the chunked-prefill and Llama-decode batches)."""
    w = inputs.make_workload("chunked_prefill", device="cuda")
    cu, out_loc = pkv.pkv_prefill_metadata(w.seq_lens, w.prefix_lens, w.page_table,
                                           w.page_size, w.num_tokens)
    torch.cuda.synchronize()
    assert torch.equal(cu, w.cu_seqlens_q)
    assert torch.equal(out_loc, w.out_loc)
    w = inputs.make_workload("llama_decode", device="cuda")
    out_loc = pkv.pkv_decode_metadata(w.seq_lens, w.page_table, w.page_size)
    torch.cuda.synchronize()
    assert torch.equal(out_loc, w.out_loc)


@pytest.mark.parametrize("B", [5, 1100])  # the one-launch builder and the chunked scan
def test_prefill_metadata_huge_lengths(B):
    """Lengths near INT32_MAX (device values the host does not check): the
    counts are summed with saturation, so cu_seqlens stays non-negative and
    non-decreasing, every slot written lies below max_tokens, and the tokens
    before the first huge request (and that request's first ones) get their
    exact slots."""
    rng = np.random.default_rng(91 + B)
    ps, width = 16, 6
    table = _table(rng, B, width, B * width + 20)
    seq = rng.integers(0, width * ps + 1, size=B).astype(np.int32)
    pre = np.zeros(B, np.int32)
    big = [1, 2] if B == 5 else [600, 1050]
    seq[big[0]] = 2**31 - 1
    seq[big[1]] = 2**31 - 1
    pre[big[1]] = 10
    if B == 5:
        seq[4], pre[4] = -2**31, 2**31 - 1  # no new token
    head = big[0]  # requests before the first huge one are exact
    cu_head, slots_head = orc.prefill_metadata(seq[:head], pre[:head], table[:head], ps)
    start = int(cu_head[-1])
    cap = start + 100
    # the first 100 tokens of the huge request, at positions 0..99 of its row
    slots_big = [orc.slot_of(table[head], t, ps) for t in range(100)]
    dev = lambda a: torch.from_numpy(a).cuda()
    out_loc = torch.full((cap + 8,), -7, dtype=torch.int32, device="cuda")
    print(f"huge lengths: B={B} huge requests {big} max_tokens {cap}", flush=True)
    cu, out_loc = pkv.pkv_prefill_metadata(dev(seq), dev(pre), dev(table), ps, cap,
                                           out_loc=out_loc)
    torch.cuda.synchronize()
    cu = cu.cpu().numpy().astype(np.int64)
    got = out_loc.cpu().numpy()
    assert np.array_equal(cu[:head + 1], cu_head)
    assert (cu >= 0).all() and (np.diff(cu) >= 0).all()
    assert cu[head + 1] == 2**31 - 1  # saturated from the first huge count on
    assert np.array_equal(got[:start], slots_head)
    assert np.array_equal(got[start:cap], np.array(slots_big, np.int32))
    assert (got[cap:] == -7).all(), "entries past max_tokens must not be written"

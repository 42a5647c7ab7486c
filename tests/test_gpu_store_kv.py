"""store_kv on the GPU: bit-exact against the oracle's index assignment over
the WHOLE pool (rows that must not change included)."""

import numpy as np
import pytest
import torch

import paged_kv_attention_out_amd as pkv
from oracle import paged_attention as orc
from paged_kv_attention_out_amd import inputs

from gpu_helpers import host_pools

pytestmark = pytest.mark.gpu


def _check(w):
    kc0, vc0 = host_pools(w, stored=False)
    ek, ev = orc.store_kv(kc0, vc0, inputs.bf16_bits(w.k_new), inputs.bf16_bits(w.v_new),
                          w.out_loc_np)
    pkv.pkv_store_kv(w.k_new, w.v_new, w.out_loc, w.k_cache, w.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(inputs.bf16_bits(w.k_cache), ek)
    assert np.array_equal(inputs.bf16_bits(w.v_cache), ev)


@pytest.mark.parametrize("name", ["llama_decode", "chunked_prefill"])
def test_store_kv_workload(name):
    print(f"store_kv workload={name}", flush=True)
    w = inputs.make_workload(name, device="cuda")
    _check(w)


@pytest.mark.parametrize("hkv,d,ps", [(1, 8, 16), (2, 64, 16), (8, 128, 256), (3, 24, 32)])
def test_store_kv_shapes(hkv, d, ps):
    print(f"store_kv hkv={hkv} d={d} ps={ps}", flush=True)
    w = inputs.build_prefill(3, hkv, hkv, d, ps, [0, 17, 5], [33, 1, 300], seed=hkv + d + ps,
                             device="cuda")
    _check(w)


def test_store_kv_skips_out_of_range_slots():
    w = inputs.build_prefill(2, 2, 2, 64, 16, [0, 3], [20, 9], seed=7, device="cuda")
    kc0, vc0 = host_pools(w, stored=False)
    loc = w.out_loc_np.copy()
    nslots = w.num_pages * w.page_size
    loc[3] = -1
    loc[10] = nslots          # one past the end
    loc[11] = 2 ** 31 - 1
    keep = np.ones(len(loc), bool)
    keep[[3, 10, 11]] = False
    ek, ev = orc.store_kv(kc0, vc0, inputs.bf16_bits(w.k_new)[keep],
                          inputs.bf16_bits(w.v_new)[keep], loc[keep])
    pkv.pkv_store_kv(w.k_new, w.v_new, torch.from_numpy(loc).cuda(), w.k_cache, w.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(inputs.bf16_bits(w.k_cache), ek)
    assert np.array_equal(inputs.bf16_bits(w.v_cache), ev)


def test_store_kv_empty_is_noop():
    w = inputs.build_prefill(1, 2, 2, 64, 16, [4], [8], seed=8, device="cuda")
    before = inputs.bf16_bits(w.k_cache)
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    pkv.pkv_store_kv(e, e, torch.empty(0, dtype=torch.int32, device="cuda"), w.k_cache,
                     w.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(inputs.bf16_bits(w.k_cache), before)

"""The Python binding checks tensor shapes against each other before any
launch: a mismatch would make a kernel read or write outside a buffer, so it
must raise ValueError on the host.  These run on the CPU: the shape checks
come before the device checks, and a call whose shapes agree fails only on
the device check (no kernel is launched here)."""

import pytest
import torch

import paged_kv_attention_out_amd as pkv

bf, i32 = torch.bfloat16, torch.int32


def _decode_args(B=4, hq=8, hkv=2, d=64, pages=10, ps=16, width=8):
    return dict(q=torch.zeros(B, hq, d, dtype=bf),
                k_cache=torch.zeros(pages, ps, hkv, d, dtype=bf),
                v_cache=torch.zeros(pages, ps, hkv, d, dtype=bf),
                page_table=torch.zeros(B, width, dtype=i32),
                seq_lens=torch.ones(B, dtype=i32))


def _decode(**over):
    a = _decode_args()
    a.update(over)
    return pkv.pkv_paged_attn_decode(a["q"], a["k_cache"], a["v_cache"], a["page_table"],
                                     a["seq_lens"], 100, 0.125, out=a.get("out"))


@pytest.mark.parametrize("over,msg", [
    (dict(k_cache=torch.zeros(10, 16, 2, 128, dtype=bf),
          v_cache=torch.zeros(10, 16, 2, 128, dtype=bf)), "head_dim"),
    (dict(v_cache=torch.zeros(10, 16, 2, 32, dtype=bf)), "v_cache"),
    (dict(v_cache=torch.zeros(9, 16, 2, 64, dtype=bf)), "v_cache"),
    (dict(k_cache=torch.zeros(160, 2, 64, dtype=bf)), "k_cache"),
    (dict(q=torch.zeros(4, 7, 64, dtype=bf)), "multiple"),
    (dict(seq_lens=torch.ones(3, dtype=i32)), "seq_lens"),
    (dict(page_table=torch.zeros(3, 8, dtype=i32)), "page_table"),
    (dict(page_table=torch.zeros(32, dtype=i32)), "page_table"),
    (dict(out=torch.zeros(4, 8, 32, dtype=bf)), "out"),
])
def test_decode_shape_mismatch(over, msg):
    with pytest.raises(ValueError, match=msg):
        _decode(**over)


def test_decode_consistent_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        _decode()


def _step(**over):
    a = _decode_args()
    a.update(dict(k_new=torch.zeros(4, 2, 64, dtype=bf), v_new=torch.zeros(4, 2, 64, dtype=bf),
                  out_loc=torch.zeros(4, dtype=i32)))
    a.update(over)
    return pkv.pkv_decode_step(a["q"], a["k_new"], a["v_new"], a["out_loc"], a["k_cache"],
                               a["v_cache"], a["page_table"], a["seq_lens"], 100, 0.125)


@pytest.mark.parametrize("over,msg", [
    (dict(k_new=torch.zeros(3, 2, 64, dtype=bf)), "k_new"),
    (dict(v_new=torch.zeros(4, 4, 64, dtype=bf)), "v_new"),
    (dict(k_new=torch.zeros(4, 2, 128, dtype=bf)), "k_new"),
    (dict(out_loc=torch.zeros(5, dtype=i32)), "out_loc"),
])
def test_decode_step_shape_mismatch(over, msg):
    with pytest.raises(ValueError, match=msg):
        _step(**over)


def test_decode_multi_shape_mismatch():
    a = _decode_args()
    with pytest.raises(ValueError, match="q has shape"):
        pkv.pkv_paged_attn_decode_multi(a["q"], a["k_cache"], a["v_cache"], a["page_table"],
                                        a["seq_lens"], 100, 0.125)
    q4 = torch.zeros(4, 3, 8, 64, dtype=bf)
    with pytest.raises(ValueError, match="out"):
        pkv.pkv_paged_attn_decode_multi(q4, a["k_cache"], a["v_cache"], a["page_table"],
                                        a["seq_lens"], 100, 0.125,
                                        out=torch.zeros(4, 8, 64, dtype=bf))


@pytest.mark.parametrize("over,msg", [
    (dict(k_new=torch.zeros(5, 2, 64, dtype=bf)), "k_new"),
    (dict(v_new=torch.zeros(6, 2, 32, dtype=bf)), "v_new"),
    (dict(v_cache=torch.zeros(10, 16, 2, 128, dtype=bf)), "v_cache"),
    (dict(out_loc=torch.zeros(6, 1, dtype=i32)), "out_loc"),
])
def test_store_kv_shape_mismatch(over, msg):
    a = dict(k_new=torch.zeros(6, 2, 64, dtype=bf), v_new=torch.zeros(6, 2, 64, dtype=bf),
             out_loc=torch.zeros(6, dtype=i32), k_cache=torch.zeros(10, 16, 2, 64, dtype=bf),
             v_cache=torch.zeros(10, 16, 2, 64, dtype=bf))
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        pkv.pkv_store_kv(a["k_new"], a["v_new"], a["out_loc"], a["k_cache"], a["v_cache"])


@pytest.mark.parametrize("over,msg", [
    (dict(cu=torch.zeros(5, dtype=i32)), "cu_seqlens_q"),
    (dict(prefix=torch.zeros(2, dtype=i32)), "cu_seqlens_q"),
    (dict(table=torch.zeros(2, 8, dtype=i32)), "page_table"),
    (dict(kc=torch.zeros(10, 16, 2, 128, dtype=bf), vc=torch.zeros(10, 16, 2, 128, dtype=bf)),
     "head_dim"),
    (dict(q=torch.zeros(20, 7, 64, dtype=bf)), "multiple"),
    (dict(out=torch.zeros(21, 8, 64, dtype=bf)), "out"),
])
def test_prefill_shape_mismatch(over, msg):
    a = dict(q=torch.zeros(20, 8, 64, dtype=bf), cu=torch.zeros(4, dtype=i32),
             prefix=torch.zeros(3, dtype=i32), kc=torch.zeros(10, 16, 2, 64, dtype=bf),
             vc=torch.zeros(10, 16, 2, 64, dtype=bf), table=torch.zeros(3, 8, dtype=i32))
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        pkv.pkv_paged_attn_prefill(a["q"], a["cu"], a["prefix"], 10, 100, a["kc"], a["vc"],
                                   a["table"], 0.125, out=a.get("out"))


def test_metadata_shape_mismatch():
    seq = torch.ones(4, dtype=i32)
    with pytest.raises(ValueError, match="prefix_lens"):
        pkv.pkv_prefill_metadata(seq, torch.zeros(3, dtype=i32), torch.zeros(4, 2, dtype=i32),
                                 16, 8)
    with pytest.raises(ValueError, match="page_table"):
        pkv.pkv_prefill_metadata(seq, torch.zeros(4, dtype=i32), torch.zeros(3, 2, dtype=i32),
                                 16, 8)
    with pytest.raises(ValueError, match="cu_seqlens_q"):
        pkv.pkv_prefill_metadata(seq, torch.zeros(4, dtype=i32), torch.zeros(4, 2, dtype=i32),
                                 16, 8, cu_seqlens_q=torch.zeros(4, dtype=i32))
    with pytest.raises(ValueError, match="out_loc"):
        pkv.pkv_prefill_metadata(seq, torch.zeros(4, dtype=i32), torch.zeros(4, 2, dtype=i32),
                                 16, 8, out_loc=torch.zeros(7, dtype=i32))
    with pytest.raises(ValueError, match="out_loc"):
        pkv.pkv_decode_metadata(seq, torch.zeros(4, 2, dtype=i32), 16,
                                out_loc=torch.zeros(3, dtype=i32))

"""The C ABI on the host: the library loads, exports what include/*.h
declares, and rejects bad arguments before anything is enqueued.

Every call here fails host-side validation, so no kernel is ever launched
(the fake device pointers below are never dereferenced)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

import paged_kv_attention_out_amd as pkv
from paged_kv_attention_out_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
FAKE = 1 << 20  # 16-byte aligned, never dereferenced: every call below fails validation


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("pkv_store_kv", "pkv_paged_attn_decode", "pkv_paged_attn_prefill",
              "pkv_decode_workspace_bytes", "pkv_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = pkv.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(_lib.SIGNATURES) == set(_declared())


def test_strerror_and_version():
    assert pkv.strerror(0) == "success"
    for s in range(1, 5):
        assert pkv.strerror(s) and pkv.strerror(s) != "unknown status"
    assert pkv.strerror(99) == "unknown status"
    assert "gfx950" in pkv.version()


def _store(**kw):
    a = dict(k_new=FAKE, v_new=FAKE, out_loc=FAKE, T=4, kc=FAKE, vc=FAKE, slots=64, hkv=8,
             d=64, stream=None)
    a.update(kw)
    return pkv.lib().pkv_store_kv(a["k_new"], a["v_new"], a["out_loc"], a["T"], a["kc"],
                                  a["vc"], a["slots"], a["hkv"], a["d"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), 1), (dict(out_loc=None), 1), (dict(kc=None), 1),
    (dict(T=-1), 1), (dict(slots=0), 1), (dict(hkv=0), 1), (dict(d=12), 1),
    (dict(k_new=FAKE + 8), 1), (dict(vc=FAKE + 2), 1),
    (dict(T=0, k_new=None, v_new=None, out_loc=None), 0),
])
def test_store_kv_validation(kw, status):
    assert _store(**kw) == status


def _decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ps=16, pages=100, pt=FAKE, stride=128, seq=FAKE, B=4,
             maxlen=2048, hq=32, hkv=8, d=64, scale=0.125, split=0, out=FAKE, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return pkv.lib().pkv_paged_attn_decode(
        a["q"], a["kc"], a["vc"], a["ps"], a["pages"], a["pt"], a["stride"], a["seq"], a["B"],
        a["maxlen"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["out"], a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(pt=None), 1), (dict(seq=None), 1), (dict(out=None), 1),
    (dict(B=-1), 1), (dict(hq=30), 1), (dict(hkv=0), 1), (dict(maxlen=0), 1),
    (dict(scale=0.0), 1), (dict(scale=-1.0), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(stride=127), 1), (dict(pages=0), 1),
    (dict(split=8), 1), (dict(split=17), 1), (dict(split=70000), 1), (dict(q=FAKE + 4), 1),
    (dict(ps=24), 2), (dict(ps=8), 2), (dict(ps=512), 2), (dict(d=96), 2), (dict(d=256), 2),
    (dict(hq=128), 2),                      # 16 query heads per KV head
    (dict(wsb=100, ws=FAKE), 3),            # needs a workspace, too small
    (dict(B=0), 0),
])
def test_decode_validation(kw, status):
    assert _decode(**kw) == status


def _step(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, loc=FAKE, kc=FAKE, vc=FAKE, ps=16, pages=100, pt=FAKE,
             stride=128, seq=FAKE, B=4, maxlen=2048, hq=32, hkv=8, d=64, scale=0.125, split=0,
             out=FAKE, ws=None, wsb=0, stream=None)
    a.update(kw)
    return pkv.lib().pkv_decode_step(
        a["q"], a["kn"], a["vn"], a["loc"], a["kc"], a["vc"], a["ps"], a["pages"], a["pt"],
        a["stride"], a["seq"], a["B"], a["maxlen"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["split"], a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), 1), (dict(vn=None), 1), (dict(loc=None), 1), (dict(kn=FAKE + 8), 1),
    (dict(vn=FAKE + 2), 1), (dict(q=None), 1), (dict(d=96), 2), (dict(hq=128), 2),
    (dict(wsb=100, ws=FAKE), 3), (dict(B=0, kn=None, vn=None, loc=None), 0),
])
def test_decode_step_validation(kw, status):
    assert _step(**kw) == status


def _noalloc(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, loc=FAKE, kc=FAKE, vc=FAKE, ps=16, pages=100, pt=FAKE,
             stride=128, seq=FAKE, B=4, maxlen=2048, hq=32, hkv=8, d=64, scale=0.125, split=0,
             out=FAKE, stream=None)
    a.update(kw)
    return pkv.lib().pkv_decode_step_noalloc(
        a["q"], a["kn"], a["vn"], a["loc"], a["kc"], a["vc"], a["ps"], a["pages"], a["pt"],
        a["stride"], a["seq"], a["B"], a["maxlen"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["split"], a["out"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), 1), (dict(loc=None), 1), (dict(q=None), 1), (dict(hq=30), 1),
    (dict(d=96), 2), (dict(hq=128), 2),
    # partials beyond the fixed scratch: rejected before anything is enqueued
    (dict(B=4096, maxlen=131072, stride=8192, hq=32, hkv=8, d=128, split=16), 3),
    (dict(B=0, kn=None, vn=None, loc=None), 0),
])
def test_decode_step_noalloc_validation(kw, status):
    assert _noalloc(**kw) == status


def test_decode_step_noalloc_scratch_size():
    cap = pkv.pkv_decode_step_noalloc_max_bytes()
    assert cap == 32 << 20
    # the named decode batches fit the scratch at their automatic split
    for B, hq, hkv, d, maxlen in ((64, 32, 8, 64, 2048), (128, 16, 8, 128, 8192),
                                  (16, 16, 8, 128, 131072)):
        assert 0 < pkv.pkv_decode_workspace_bytes(B, hq, hkv, d, maxlen) <= cap


def _shared(**kw):
    a = dict(q=FAKE, kn=None, vn=None, loc=None, kc=FAKE, vc=FAKE, ps=16, pages=100, pt=FAKE,
             stride=128, seq=FAKE, B=4, maxlen=2048, cu=FAKE, sh=FAKE, G=2, maxg=3, maxsh=1024,
             hq=32, hkv=8, d=64, scale=0.125, split=0, out=FAKE, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return pkv.lib().pkv_paged_attn_decode_shared(
        a["q"], a["kn"], a["vn"], a["loc"], a["kc"], a["vc"], a["ps"], a["pages"], a["pt"],
        a["stride"], a["seq"], a["B"], a["maxlen"], a["cu"], a["sh"], a["G"], a["maxg"],
        a["maxsh"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["out"], a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), 1), (dict(sh=None), 1), (dict(G=0), 1), (dict(G=5), 1), (dict(G=-1), 1),
    (dict(maxg=5), 1), (dict(maxg=-1), 1), (dict(maxsh=4096), 1), (dict(maxsh=-16), 1),
    (dict(q=None), 1), (dict(hq=30), 1), (dict(kn=FAKE), 1),   # part of the store missing
    (dict(d=96), 2), (dict(hq=128), 2), (dict(wsb=100), 3),
    (dict(B=0, G=0, maxg=0, cu=None, sh=None), 0),
])
def test_decode_shared_validation(kw, status):
    assert _shared(**kw) == status


def test_decode_shared_workspace_size():
    plain = pkv.pkv_decode_workspace_bytes(64, 32, 8, 64, 2048)
    shared = pkv.pkv_paged_attn_decode_shared_workspace_bytes(64, 32, 8, 64, 2048, 1024)
    assert shared > plain   # 16 more partial slots per (request, KV head) for the prefix splits
    # no prefix splits: the split partials alone (plain decode may reserve
    # more, for the rows of its balanced launch)
    none = pkv.pkv_paged_attn_decode_shared_workspace_bytes(64, 32, 8, 64, 2048, 0)
    assert 0 < none <= plain
    assert pkv.pkv_paged_attn_decode_shared_workspace_bytes(64, 32, 8, 64, 2048, 4096) == 0


def test_decode_graphs_validation():
    lib = pkv.lib()
    arr = (ctypes.c_int32 * 3)(1, 2, 4)
    h = ctypes.c_void_p(123)

    def create(buckets=arr, n=3, ws=FAKE, wsb=1 << 30, out_ptr=ctypes.byref(h), hq=32, kn=FAKE):
        return lib.pkv_decode_graphs_create(buckets, n, FAKE, kn, FAKE, FAKE, FAKE, FAKE, 16,
                                            100, FAKE, 128, FAKE, 2048, hq, 8, 64, 0.125, FAKE,
                                            ws, wsb, out_ptr)

    assert create(out_ptr=None) == 1
    assert create(buckets=None) == 1 and h.value is None     # handle cleared on error
    assert create(n=0) == 1
    assert create(n=65) == 1
    assert create(buckets=(ctypes.c_int32 * 3)(1, 2, 2)) == 1  # duplicate bucket
    assert create(buckets=(ctypes.c_int32 * 2)(0, 4), n=2) == 1
    assert create(hq=30) == 1
    assert create(kn=None) == 1                                 # part of the fused store missing
    assert create(wsb=100) == 3                                 # workspace too small
    n = lib.pkv_decode_graphs_workspace_bytes(arr, 3, 32, 8, 64, 2048)
    assert n == max(pkv.pkv_decode_workspace_bytes(b, 32, 8, 64, 2048) for b in (1, 2, 4))
    used = ctypes.c_int32(7)
    assert lib.pkv_decode_graphs_replay(None, 1, None, ctypes.byref(used)) == 1
    assert used.value == 0
    lib.pkv_decode_graphs_destroy(None)


def _multi(**kw):
    a = dict(q=FAKE, L=4, kc=FAKE, vc=FAKE, ps=16, pages=100, pt=FAKE, stride=128, seq=FAKE,
             B=4, maxlen=2048, hq=32, hkv=8, d=64, scale=0.125, split=0, out=FAKE, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return pkv.lib().pkv_paged_attn_decode_multi(
        a["q"], a["L"], a["kc"], a["vc"], a["ps"], a["pages"], a["pt"], a["stride"], a["seq"],
        a["B"], a["maxlen"], a["hq"], a["hkv"], a["d"], a["scale"], a["split"], a["out"],
        a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), 1), (dict(L=17), 1), (dict(L=-3), 1), (dict(q=None), 1), (dict(out=None), 1),
    (dict(seq=None), 1), (dict(scale=0.0), 1), (dict(hq=30), 1), (dict(split=24), 1),
    (dict(q=FAKE + 2), 1), (dict(d=96), 2), (dict(hq=128), 2), (dict(ps=24), 2),
    (dict(wsb=100, ws=FAKE), 3), (dict(ws=FAKE + 64, wsb=1 << 30), 1),
    (dict(B=0), 0), (dict(B=0, L=16), 0),
])
def test_decode_multi_validation(kw, status):
    assert _multi(**kw) == status


def test_decode_multi_workspace_sizes():
    # q_len = 1 needs what plain decode needs
    for args in ((64, 32, 8, 64, 2048), (16, 16, 16, 128, 4096), (1, 4, 2, 64, 64)):
        B, hq, hkv, d, maxlen = args
        assert pkv.pkv_decode_multi_workspace_bytes(B, 1, hq, hkv, d, maxlen) == \
            pkv.pkv_decode_workspace_bytes(B, hq, hkv, d, maxlen)
    one = pkv.pkv_decode_multi_workspace_bytes(64, 1, 32, 8, 64, 2048)
    four = pkv.pkv_decode_multi_workspace_bytes(64, 4, 32, 8, 64, 2048)
    assert 4 * one - 3 * 256 <= four <= 4 * one   # every array grows by q_len (256-B rounding)
    assert pkv.pkv_decode_multi_workspace_bytes(64, 0, 32, 8, 64, 2048) == 0
    assert pkv.pkv_decode_multi_workspace_bytes(64, 17, 32, 8, 64, 2048) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(seq=None), 1), (dict(pre=None), 1), (dict(pt=None), 1), (dict(cu=None), 1),
    (dict(loc=None), 1), (dict(B=-1), 1), (dict(maxt=-1), 1), (dict(stride=0), 1),
    (dict(ps=0), 1), (dict(B=0, seq=None), 0),
])
def test_prefill_metadata_validation(kw, status):
    a = dict(seq=FAKE, pre=FAKE, B=4, pt=FAKE, stride=8, ps=16, maxt=100, cu=FAKE, loc=FAKE)
    a.update(kw)
    assert pkv.lib().pkv_prefill_metadata(a["seq"], a["pre"], a["B"], a["pt"], a["stride"],
                                          a["ps"], a["maxt"], a["cu"], a["loc"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(seq=None), 1), (dict(pt=None), 1), (dict(loc=None), 1), (dict(B=-1), 1),
    (dict(stride=0), 1), (dict(ps=-16), 1), (dict(B=0, seq=None), 0),
])
def test_decode_metadata_validation(kw, status):
    a = dict(seq=FAKE, B=4, pt=FAKE, stride=8, ps=16, loc=FAKE)
    a.update(kw)
    assert pkv.lib().pkv_decode_metadata(a["seq"], a["B"], a["pt"], a["stride"], a["ps"],
                                         a["loc"], None) == status


def test_decode_workspace_sizes():
    # one split per request: no workspace
    assert pkv.pkv_decode_workspace_bytes(1, 4, 2, 64, 64) == 0
    assert pkv.pkv_decode_split_tokens(1, 2, 64) == 64
    n = pkv.pkv_decode_workspace_bytes(64, 32, 8, 64, 2048)
    s = pkv.pkv_decode_split_tokens(64, 8, 2048)
    nsm = -(-2048 // s)
    assert nsm > 1
    assert n >= 2 * 64 * 8 * nsm * 4 * 4 + 64 * 8 * nsm * 4 * 64 * 4  # (m, l) + o per split
    assert pkv.pkv_decode_split_tokens(64, 8, 2048, 48) == 48
    assert pkv.pkv_decode_split_tokens(64, 8, 2048, 40) == 0   # not a multiple of 16
    assert pkv.pkv_decode_workspace_bytes(64, 30, 8, 64, 2048) == 0  # invalid grouping


def _prefill(**kw):
    a = dict(q=FAKE, cu=FAKE, prefix=FAKE, B=4, T=100, maxq=50, maxlen=1000, kc=FAKE, vc=FAKE,
             ps=16, pages=100, pt=FAKE, stride=64, hq=32, hkv=8, d=64, scale=0.125, out=FAKE,
             ws=FAKE, wsb=256, stream=None)
    a.update(kw)
    return pkv.lib().pkv_paged_attn_prefill(
        a["q"], a["cu"], a["prefix"], a["B"], a["T"], a["maxq"], a["maxlen"], a["kc"], a["vc"],
        a["ps"], a["pages"], a["pt"], a["stride"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(prefix=None), 1), (dict(out=None), 1),
    (dict(ws=None), 1), (dict(ws=FAKE + 4), 1), (dict(wsb=0), 3), (dict(wsb=255), 3),
    (dict(B=0), 1), (dict(B=-2), 1), (dict(T=-1), 1), (dict(maxq=0), 1), (dict(maxlen=0), 1),
    (dict(hq=33), 1), (dict(scale=0.0), 1), (dict(stride=62), 1), (dict(pages=0), 1),
    (dict(kc=FAKE + 8), 1),
    (dict(ps=48), 2), (dict(d=80), 2), (dict(hq=128), 2), (dict(d=128, hq=256), 2),
    (dict(T=0, q=None), 0),
])
def test_prefill_validation(kw, status):
    assert _prefill(**kw) == status


def test_prefill_workspace_size():
    assert 4 <= pkv.pkv_prefill_workspace_bytes() <= 4096


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


@pytest.mark.parametrize("src,nbytes,blocks,sink,status", [
    (FAKE, 1 << 20, 0, FAKE, 1), (FAKE, 1 << 20, (1 << 20) + 1, FAKE, 1),
    (None, 1 << 20, 64, FAKE, 1), (FAKE, 1 << 20, 64, None, 1),
    (FAKE + 8, 1 << 20, 64, FAKE, 1), (FAKE, (1 << 20) + 8, 64, FAKE, 1),
    (None, 0, 64, None, 0),
])
def test_ref_stream_read_validation(src, nbytes, blocks, sink, status):
    assert pkv.lib().pkv_ref_stream_read(src, nbytes, blocks, sink, None) == status


def test_ref_stream_sink_words():
    lib = pkv.lib()
    assert lib.pkv_ref_stream_sink_words(0) == 0
    assert lib.pkv_ref_stream_sink_words(-3) == 0
    assert lib.pkv_ref_stream_sink_words(10) == 40

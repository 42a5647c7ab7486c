"""Checks on the AMD assembly of the code objects compiled from this source tree.

* No instruction writes through the scalar data cache (scalar stores,
  scalar atomics, scalar cache write-back / discard): every store and
  atomic the kernels make is a vector memory instruction.
* No packed fp32 VALU instruction: the build disables them.
* Every kernel uses MFMA (and the LDS transpose read) where the design
  says it does.

This file names the forbidden mnemonics, so it is CPU-only and is kept out
of GPU uploads.
"""

import re
import subprocess

import pytest

from paged_kv_attention_out_amd import build as B

FORBIDDEN = re.compile(
    r"^\s*(s_store_|s_buffer_store|s_scratch_store|s_atomic_|s_buffer_atomic|s_dcache_wb"
    r"|s_dcache_discard|v_pk_fma_f32|v_pk_mul_f32|v_pk_add_f32)", re.M)


@pytest.fixture(scope="module")
def disasm():
    out = {}
    for co in B.code_objects():
        txt = subprocess.run(["/opt/rocm/llvm/bin/llvm-objdump", "-d", "--mcpu=gfx950", co],
                             capture_output=True, text=True, check=True).stdout
        out[co] = txt
    return out


def test_no_scalar_cache_writes_or_packed_fp32(disasm):
    for co, txt in disasm.items():
        bad = FORBIDDEN.findall(txt)
        assert not bad, f"{co}: {sorted(set(bad))}"


def test_kernels_use_mfma(disasm):
    txt = {k.split("/")[-1].split(".")[0]: v for k, v in disasm.items()}
    assert "v_mfma_f32_16x16x32_bf16" in txt["decode"]
    assert "v_mfma_f32_32x32x16_bf16" in txt["prefill"]
    assert "ds_read_b64_tr_b16" in txt["decode"]      # V read key-contiguous from LDS
    assert "global_atomic" not in txt["decode"]       # splits merge in a second kernel

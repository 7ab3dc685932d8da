"""The LDS-poisoning debug build differs from the product build exactly by its
poison stores: compiled to gfx950 assembly here (no GPU needed), a kernel of
the debug build carries the entry fill of its LDS (one more barrier) and a
poison store before every direct-to-LDS load, and the product build has none
of them.  The GPU side of the check is tests/test_lds_poison_gpu.py."""
import os
import re
import subprocess

import pytest

from sparse_mla_attention_fwd_amd import build as B


def _asm(tmp_path, poison):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path / ("p.s" if poison else "c.s")
    cmd = [cc, *B.compile_flags(poison), "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, "smla_fwd_bf16_persist.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _count(asm, op):
    return len(re.findall(r"^\s+" + op + r"\b", asm, flags=re.M))


def test_debug_build_adds_only_poison_stores(tmp_path):
    prod, dbg = _asm(tmp_path, False), _asm(tmp_path, True)
    dma = _count(prod, "buffer_load_dwordx4") + _count(prod, "buffer_load_dword")
    assert dma > 0
    # one 16-byte (or 4-byte, index ring) poison store per direct-to-LDS load
    extra = (_count(dbg, "ds_write_b128") - _count(prod, "ds_write_b128")) + \
            (_count(dbg, "ds_write_b32") - _count(prod, "ds_write_b32"))
    assert extra >= dma
    # the entry fill ends with one more workgroup barrier
    assert _count(dbg, "s_barrier") == _count(prod, "s_barrier") + 1
    # the arithmetic is the same: as many MFMAs and exponentials
    for op in ("v_mfma_f32_16x16x32_bf16", "v_exp_f32"):
        assert _count(dbg, op) == _count(prod, op), op

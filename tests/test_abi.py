"""C-ABI checks that need no GPU: the library loads, exports every function
include/smla.h declares, validates arguments on the host (returning a status
and enqueuing nothing) and plans the named workloads as documented."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from sparse_mla_attention_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(smla_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = _declared_functions()
    assert declared, "no declarations parsed"
    assert sorted(declared) == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.smla_abi_version() == _lib.ABI_VERSION


@pytest.mark.parametrize("struct,cname", [(_lib.smla_fwd_params, "smla_fwd_params"),
                                          (_lib.smla_paged_kv, "smla_paged_kv")])
def test_struct_layouts_match_header(tmp_path, struct, cname):
    """Every field offset of the ctypes mirrors equals the C compiler's."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler to read the header's layout")
    fields = [f for f, _ in struct._fields_]
    src = tmp_path / "off.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "smla.h"\nint main(void){\n'
                   + f'printf("%zu\\n", sizeof({cname}));\n'
                   + "".join(f'printf("%zu\\n", offsetof({cname}, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "off"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(struct)
    assert got[1:] == [getattr(struct, f).offset for f in fields]


FAKE = 1 << 20   # 16-byte aligned fake device addresses: never dereferenced on failure paths

# The entry points that enqueue work (smla_fwd, smla_fwd_paged, smla_fwd_tune)
# are called with the fake addresses only where no GPU is visible: should a
# check ever regress there, the launch fails for want of a device instead of
# running a kernel on unmapped addresses.  Rejection itself is checked through
# the calls that share the same validation and never launch (smla_fwd_plan and
# the workspace queries); the checks that only the launching calls make
# (workspace size and alignment) are covered with real device buffers in
# tests/test_abi_gpu.py.
NO_GPU = torch.cuda.device_count() == 0


def _params(**kw):
    p = _lib.smla_fwd_params()
    p.s_q, p.h_q, p.d_qk, p.d_v, p.topk, p.s_kv = 4, 16, 576, 512, 128, 2048
    p.sm_scale = 1 / 24
    p.q, p.q_stride_token, p.q_stride_head = FAKE, 16 * 576, 576
    p.kv, p.kv_stride_row, p.kv_format = FAKE * 2, 576, 0
    p.indices, p.indices_stride_token = FAKE * 3, 128
    p.out, p.out_stride_token, p.out_stride_head = FAKE * 4, 16 * 512, 512
    p.lse, p.lse_stride_token = FAKE * 5, 16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("field,value,status", [
    ("d_qk", 512, _lib.SMLA_ERR_UNSUPPORTED),
    ("d_v", 576, _lib.SMLA_ERR_UNSUPPORTED),
    ("h_q", 24, _lib.SMLA_ERR_UNSUPPORTED),
    ("h_q", 256, _lib.SMLA_ERR_UNSUPPORTED),
    ("s_q", -1, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("topk", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("s_kv", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("s_kv", 1 << 31, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("sm_scale", float("nan"), _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("q", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("lse", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("q", FAKE + 8, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("q_stride_head", 575, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("kv_stride_row", 580, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("out_stride_token", 512, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("lse_stride_token", 8, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("kv_format", 7, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("b_topk", 48, _lib.SMLA_ERR_UNSUPPORTED),
    ("num_splits", -2, _lib.SMLA_ERR_INVALID_ARGUMENT),
])
def test_invalid_arguments_are_rejected_on_the_host(field, value, status):
    lib = _lib.load()
    p = _params(**{field: value})
    ns, bt = ctypes.c_int32(), ctypes.c_int32()
    assert lib.smla_fwd_plan(ctypes.byref(p), ctypes.byref(ns), ctypes.byref(bt)) == status
    assert _lib.last_error() != ""
    n = ctypes.c_size_t(123)
    assert lib.smla_fwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    if NO_GPU:
        assert lib.smla_fwd(ctypes.byref(p), None) == status


def test_null_params_and_status_strings():
    lib = _lib.load()
    assert lib.smla_fwd(None, None) == _lib.SMLA_ERR_INVALID_ARGUMENT
    for s in range(5):
        assert lib.smla_status_string(s).decode()
    assert lib.smla_status_string(99).decode() == "unknown status"


def test_empty_batch_is_a_no_op():
    lib = _lib.load()
    p = _params(s_q=0, q=0, kv=0, indices=0, out=0, lse=0)
    assert lib.smla_fwd(ctypes.byref(p), None) == _lib.SMLA_OK


def test_workspace_required_for_split_plans():
    lib = _lib.load()
    p = _params(num_splits=3)
    assert _lib.smla_fwd_plan(p) == (3, 32)
    need = _lib.smla_fwd_workspace_size(p)
    parts = 4 * 3 * 16
    # fp32 lse per part (256-byte aligned), then the bf16 output of every part
    assert need == parts * 512 * 2 + ((parts * 4 + 255) // 256) * 256
    if NO_GPU:
        assert lib.smla_fwd(ctypes.byref(p), None) == _lib.SMLA_ERR_WORKSPACE
        p.workspace, p.workspace_bytes = FAKE * 6, need - 1
        assert lib.smla_fwd(ctypes.byref(p), None) == _lib.SMLA_ERR_WORKSPACE


@pytest.mark.parametrize("name,splits", [("tiny", None), ("prefill", 1), ("causal", 1), ("decode", 4),
                                         ("decode_fp8", None), ("decode_fp4", None),
                                         ("decode_paged", 4)])
def test_plans_of_named_workloads(name, splits):
    import workloads
    w = workloads.WORKLOADS[name]
    fp8 = w.kv_format == "fp8"
    fmt = {"bf16": 0, "fp8": 1, "fp4": 2}[w.kv_format]
    p = _params(s_q=w.s_q, h_q=w.h_q, topk=w.topk, s_kv=w.s_kv, num_splits=w.num_splits,
                q_stride_token=w.h_q * 576, out_stride_token=w.h_q * 512, lse_stride_token=w.h_q,
                indices_stride_token=w.topk, kv_format=fmt,
                kv_stride_row={"bf16": 576, "fp8": 640, "fp4": 320}[w.kv_format])
    ns, bt = _lib.smla_fwd_plan(p)
    if splits is not None:
        assert ns == splits
    assert bt in (32, 64)
    cap = _lib.MAX_SLOTS_PER_SPLIT_FP8 if fp8 else _lib.MAX_SLOTS_PER_SPLIT
    assert (w.topk + ns - 1) // ns <= cap


def test_b_topk_128_is_a_bf16_block_size():
    """B_TOPK 128 is accepted for bf16 KV (planned as asked, no block-count
    workspace) and refused for the quantised formats."""
    p = _params(topk=2048, indices_stride_token=2048, num_splits=1, b_topk=128)
    assert _lib.smla_fwd_plan(p) == (1, 128)
    assert _lib.smla_fwd_workspace_size(p) == 0
    for fmt, row in ((1, 640), (2, 320)):
        p = _params(kv_format=fmt, kv_stride_row=row, topk=1024, indices_stride_token=1024, b_topk=128)
        with pytest.raises(_lib.SmlaError):
            _lib.smla_fwd_plan(p)


def test_topk_beyond_one_split_needs_more_parts():
    p = _params(topk=5000, indices_stride_token=5000, num_splits=2)
    with pytest.raises(_lib.SmlaError):
        _lib.smla_fwd_plan(p)
    p.num_splits = 0
    ns, _ = _lib.smla_fwd_plan(p)
    assert ns >= 3


def test_fp8_plan_limits():
    p = _params(kv_format=1, kv_stride_row=640, topk=2048, indices_stride_token=2048, num_splits=1)
    with pytest.raises(_lib.SmlaError):
        _lib.smla_fwd_plan(p)          # 2048 slots exceed one fp8 part
    p.num_splits = 2
    assert _lib.smla_fwd_plan(p) == (2, 32)
    p.b_topk = 64
    with pytest.raises(_lib.SmlaError):
        _lib.smla_fwd_plan(p)
    p.b_topk, p.kv_stride_row = 0, 600
    with pytest.raises(_lib.SmlaError):
        _lib.smla_fwd_plan(p)


def test_pack_fp8_rows_host():
    rng = np.random.default_rng(0)
    codes = torch.from_numpy(rng.integers(0, 256, (7, 576), dtype=np.uint8))
    scales = torch.from_numpy(rng.random((7, 5), dtype=np.float32))
    packed = _lib.smla_pack_fp8_kv_host(codes, scales)
    assert packed.shape == (7, 640)
    assert torch.equal(packed[:, :576], codes)
    assert torch.equal(packed[:, 576:596].contiguous().view(torch.float32), scales)
    assert torch.all(packed[:, 596:] == 0)


def _paged(**kw):
    g = _lib.smla_paged_kv()
    g.block_table, g.block_table_stride_token, g.table_width, g.page_size = FAKE * 7, 32, 32, 64
    for k, v in kw.items():
        setattr(g, k, v)
    return g


@pytest.mark.parametrize("field,value,status", [
    ("page_size", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("page_size", 3, _lib.SMLA_ERR_INVALID_ARGUMENT),        # s_kv 2048 is not whole pages of 3
    ("table_width", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("table_width", 1 << 30, _lib.SMLA_ERR_UNSUPPORTED),     # logical positions past int32
    ("block_table", 0, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("block_table", FAKE + 2, _lib.SMLA_ERR_INVALID_ARGUMENT),
    ("block_table_stride_token", -1, _lib.SMLA_ERR_INVALID_ARGUMENT),
])
def test_paged_arguments_are_rejected_on_the_host(field, value, status):
    lib = _lib.load()
    p = _params()
    g = _paged(**{field: value})
    n = ctypes.c_size_t(123)
    assert lib.smla_fwd_paged_workspace_size(ctypes.byref(p), ctypes.byref(g), ctypes.byref(n)) == status
    assert _lib.last_error() != ""
    if NO_GPU:
        assert lib.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == status


def test_paged_workspace_and_null_paged():
    lib = _lib.load()
    p = _params()
    n = ctypes.c_size_t(123)
    assert lib.smla_fwd_paged_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == \
        _lib.SMLA_ERR_INVALID_ARGUMENT
    if NO_GPU:
        assert lib.smla_fwd_paged(ctypes.byref(p), None, None) == _lib.SMLA_ERR_INVALID_ARGUMENT
    g = _paged()
    # translated indices first (s_q * topk int32, 256-byte rounded), then the split region
    p.num_splits = 1
    assert _lib.smla_fwd_paged_workspace_size(p, g) == 4 * 128 * 4
    p.num_splits = 3
    assert _lib.smla_fwd_paged_workspace_size(p, g) == 4 * 128 * 4 + _lib.smla_fwd_workspace_size(p)
    if NO_GPU:
        assert lib.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == _lib.SMLA_ERR_WORKSPACE
    p.s_q = 0
    assert lib.smla_fwd_paged(ctypes.byref(p), ctypes.byref(g), None) == _lib.SMLA_OK


def test_fp4_plan_limits_and_strides():
    p = _params(kv_format=2, kv_stride_row=320, topk=2048, indices_stride_token=2048, num_splits=1)
    assert _lib.smla_fwd_plan(p) == (1, 32)       # 2048 slots fit one fp4 part
    p.b_topk = 64
    with pytest.raises(_lib.SmlaError):
        _lib.smla_fwd_plan(p)
    p.b_topk = 0
    for bad in (304, 328):                        # shorter than a row / not 16-byte aligned
        p.kv_stride_row = bad
        with pytest.raises(_lib.SmlaError):
            _lib.smla_fwd_plan(p)


def test_pack_fp4_rows_host():
    rng = np.random.default_rng(1)
    codes = torch.from_numpy(rng.integers(0, 16, (5, 576), dtype=np.uint8))
    scales = torch.from_numpy(rng.random((5, 5), dtype=np.float32))
    packed = _lib.smla_pack_fp4_kv_host(codes, scales)
    assert packed.shape == (5, 320)
    c = codes.numpy()
    assert np.array_equal(packed[:, :288].numpy(), (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8))
    assert torch.equal(packed[:, 288:308].contiguous().view(torch.float32), scales)
    assert torch.all(packed[:, 308:] == 0)
    bad = codes.clone()
    bad[2, 7] = 16
    with pytest.raises(_lib.SmlaError):
        _lib.smla_pack_fp4_kv_host(bad, scales)


def test_tune_arguments_and_workspace():
    lib = _lib.load()
    p = _params(h_q=128, q_stride_token=128 * 576, out_stride_token=128 * 512, lse_stride_token=128,
                topk=512, indices_stride_token=512)
    need = _lib.smla_fwd_tune_workspace_size(p)
    # at least the workspace of every explicit split count it tries
    for ns in (1, 2, 4, 8, 16, 32):
        p.num_splits = ns
        assert need >= _lib.smla_fwd_workspace_size(p)
    ns, bt, us = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    args = (ctypes.byref(ns), ctypes.byref(bt), ctypes.byref(us))
    # rejected on the host before any HIP call
    assert lib.smla_fwd_tune(ctypes.byref(p), None, 0, *args) == _lib.SMLA_ERR_INVALID_ARGUMENT
    assert lib.smla_fwd_tune(ctypes.byref(p), None, 10, None, ctypes.byref(bt), None) == \
        _lib.SMLA_ERR_INVALID_ARGUMENT
    if NO_GPU:
        assert lib.smla_fwd_tune(ctypes.byref(p), None, 10, *args) == _lib.SMLA_ERR_WORKSPACE
    bad = _params(h_q=24)
    assert lib.smla_fwd_tune(ctypes.byref(bad), None, 10, *args) == _lib.SMLA_ERR_UNSUPPORTED
    # nothing to time: the planner's plan, no HIP call
    empty = _params(s_q=0, q=0, kv=0, indices=0, out=0, lse=0)
    assert lib.smla_fwd_tune(ctypes.byref(empty), None, 10, *args) == _lib.SMLA_OK
    assert (ns.value, bt.value) == _lib.smla_fwd_plan(empty)


def test_static_scratch_size_and_oversized_plans():
    """The header's scratch size is the binding's; a plan whose split partials
    exceed it is refused before anything is enqueued."""
    text = open(HEADER).read()
    m = re.search(r"#define SMLA_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.STATIC_SCRATCH_BYTES
    lib = _lib.load()
    p = _params(s_q=256, h_q=128, topk=2048, indices_stride_token=2048, num_splits=16,
                q_stride_token=128 * 576, out_stride_token=128 * 512, lse_stride_token=128)
    assert _lib.smla_fwd_workspace_size(p) > _lib.STATIC_SCRATCH_BYTES
    if NO_GPU:
        assert lib.smla_fwd_static_scratch(ctypes.byref(p), None) == _lib.SMLA_ERR_WORKSPACE
        assert "static scratch" in _lib.last_error()
        bad = _params(h_q=24)
        assert lib.smla_fwd_static_scratch(ctypes.byref(bad), None) == _lib.SMLA_ERR_UNSUPPORTED


def test_schedule_planning():
    """The planner runs the grid; single-split pipelined plans in the 32-bit
    window take one int32 block count per token of workspace (computed ahead);
    the persistent schedule runs when asked for and is refused where it is not
    built."""
    big = dict(s_q=4096, h_q=64, topk=2048, s_kv=65536, indices_stride_token=2048,
               q_stride_token=64 * 576, out_stride_token=64 * 512, lse_stride_token=64)
    p = _params(**big)
    assert _lib.smla_fwd_schedule(p) == _lib.SMLA_SCHEDULE_GRID
    assert _lib.smla_fwd_plan(p) == (1, 32)
    assert _lib.smla_fwd_workspace_size(p) == 4096 * 4
    p = _params(**big, schedule=_lib.SMLA_SCHEDULE_PERSISTENT)
    assert _lib.smla_fwd_schedule(p) == _lib.SMLA_SCHEDULE_PERSISTENT
    assert _lib.smla_fwd_workspace_size(p) == 4096 * 4
    p = _params(**dict(big, s_kv=4_000_000))                # beyond the 32-bit window: no counts
    assert _lib.smla_fwd_workspace_size(p) == 0
    p = _params(**dict(big, topk=512, indices_stride_token=512), num_splits=1)   # short split
    assert _lib.smla_fwd_workspace_size(p) == 0
    p = _params(**dict(big, s_q=3), schedule=_lib.SMLA_SCHEDULE_PERSISTENT, persistent_workgroups=2)
    assert _lib.smla_fwd_schedule(p) == _lib.SMLA_SCHEDULE_PERSISTENT
    assert _lib.smla_fwd_workspace_size(p) == 256
    for bad in (dict(h_q=128, q_stride_token=128 * 576, out_stride_token=128 * 512, lse_stride_token=128),
                dict(topk=1000, indices_stride_token=1000), dict(b_topk=64), dict(num_splits=2),
                dict(kv_format=1, kv_stride_row=640), dict(s_kv=4_000_000)):
        p = _params(**dict(big, **bad), schedule=_lib.SMLA_SCHEDULE_PERSISTENT)
        with pytest.raises(_lib.SmlaError):
            _lib.smla_fwd_schedule(p)
    for field, value in (("schedule", 3), ("schedule", -1), ("persistent_workgroups", -1),
                         ("persistent_workgroups", 1 << 16)):
        p = _params(**{field: value})
        with pytest.raises(_lib.SmlaError):
            _lib.smla_fwd_plan(p)


def test_poison_debug_library_loads_with_the_same_exports():
    """The LDS-poisoning debug build (tests/test_lds_poison_gpu.py) exports the
    same ABI, and switching the binding to it restores the product library."""
    before = _lib.load()
    with _lib.library(_lib.POISON_LIB_PATH) as dbg:
        assert dbg is not before
        for name in _declared_functions():
            assert hasattr(dbg, name), name
        assert dbg.smla_abi_version() == _lib.ABI_VERSION
        assert _lib.load() is dbg
    assert _lib.load() is before

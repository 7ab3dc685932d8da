"""The Python binding's tensor checks (no GPU): everything the C ABI cannot
see from plain pointers -- devices, the dtypes and shapes of the outputs,
innermost strides, the index table's shape -- is rejected before a pointer
reaches the library.  Tensors on the ``meta`` device stand in for device
tensors (they carry shapes, strides and a device, and no memory)."""
import pytest
import torch

import sparse_mla_attention_fwd_amd as smla

META = torch.device("meta")


def _ok(**over):
    s_q, h_q, topk = 3, 16, 40
    t = dict(q=torch.empty((s_q, h_q, 576), dtype=torch.bfloat16, device=META),
             kv=torch.empty((100, 576), dtype=torch.bfloat16, device=META),
             indices=torch.empty((s_q, topk), dtype=torch.int32, device=META),
             out=torch.empty((s_q, h_q, 512), dtype=torch.bfloat16, device=META),
             lse=torch.empty((s_q, h_q), dtype=torch.float32, device=META))
    t.update(over)
    return t


def _check(fmt=smla.SMLA_KV_BF16, **over):
    t = _ok(**over)
    smla.check_tensors(t["q"], t["kv"], t["indices"], fmt, out=t["out"], lse=t["lse"],
                       workspace=t.get("workspace"), block_table=t.get("block_table"))


def test_consistent_tensors_pass():
    _check()
    _check(fmt=smla.SMLA_KV_FP8_E4M3, kv=torch.empty((100, 640), dtype=torch.uint8, device=META))
    _check(fmt=smla.SMLA_KV_FP4_E2M1, kv=torch.empty((100, 320), dtype=torch.uint8, device=META))
    big = torch.empty((3, 24, 640), dtype=torch.bfloat16, device=META)
    _check(q=big[:, 4:20, :576])                       # head-sliced view, unit inner stride


@pytest.mark.parametrize("name,value", [
    ("kv", torch.empty((100, 576), dtype=torch.bfloat16)),                     # host KV
    ("indices", torch.empty((3, 40), dtype=torch.int32)),                      # host indices
    ("out", torch.empty((3, 16, 512), dtype=torch.bfloat16)),                  # host out
    ("workspace", torch.empty(1024, dtype=torch.uint8)),                       # host workspace
    ("block_table", torch.zeros((3, 4), dtype=torch.int32)),                   # host block table
])
def test_tensor_on_another_device_is_rejected(name, value):
    with pytest.raises(ValueError, match="device"):
        _check(**{name: value})


def test_quantised_rows_packed_on_the_host_are_rejected():
    """pack_fp8_kv without device= returns host rows: handing them to the
    gather would fault the GPU, so the binding refuses them."""
    host_rows = torch.zeros((100, 640), dtype=torch.uint8)
    with pytest.raises(ValueError, match="device"):
        _check(fmt=smla.SMLA_KV_FP8_E4M3, kv=host_rows)


@pytest.mark.parametrize("over", [
    dict(out=torch.empty((3, 16, 512), dtype=torch.float32, device=META)),     # fp32 out
    dict(out=torch.empty((3, 16, 576), dtype=torch.bfloat16, device=META)),    # d_qk-wide out
    dict(out=torch.empty((3, 8, 512), dtype=torch.bfloat16, device=META)),     # too few heads
    dict(lse=torch.empty((3, 16), dtype=torch.bfloat16, device=META)),         # bf16 lse
    dict(lse=torch.empty((3, 16), dtype=torch.float64, device=META)),          # fp64 lse
    dict(lse=torch.empty((3, 32), dtype=torch.float32, device=META)[:, ::2]),  # strided heads
    dict(indices=torch.empty((120,), dtype=torch.int32, device=META)),         # 1-D indices
    dict(indices=torch.empty((4, 40), dtype=torch.int32, device=META)),        # wrong s_q
    dict(q=torch.empty((3, 16, 1152), dtype=torch.bfloat16, device=META)[..., ::2]),   # strided q
    dict(kv=torch.empty((100, 1152), dtype=torch.bfloat16, device=META)[:, ::2]),      # strided kv
    dict(out=torch.empty((3, 16, 1024), dtype=torch.bfloat16, device=META)[..., ::2]),  # strided out
    dict(kv=torch.empty((100, 512), dtype=torch.bfloat16, device=META)),       # rows too short
])
def test_bad_shapes_strides_and_dtypes_are_rejected(over):
    with pytest.raises(ValueError):
        _check(**over)


@pytest.mark.parametrize("fmt,over", [
    (smla.SMLA_KV_BF16, dict(q=torch.empty((3, 16, 576), dtype=torch.float16, device=META))),
    (smla.SMLA_KV_BF16, dict(kv=torch.empty((100, 576), dtype=torch.float32, device=META))),
    (smla.SMLA_KV_FP8_E4M3, dict(kv=torch.empty((100, 576), dtype=torch.bfloat16, device=META))),
    (smla.SMLA_KV_BF16, dict(indices=torch.empty((3, 40), dtype=torch.int64, device=META))),
])
def test_bad_input_dtypes_are_rejected(fmt, over):
    with pytest.raises(TypeError):
        _check(fmt=fmt, **over)


def test_host_query_is_rejected_before_any_library_call():
    q = torch.zeros((1, 16, 576), dtype=torch.bfloat16)
    kv = torch.zeros((10, 576), dtype=torch.bfloat16)
    idx = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        smla.sparse_mla_fwd(q, kv, idx, 1 / 24)
    with pytest.raises(ValueError, match="GPU"):
        smla.tune_plan(q, kv, idx, 1 / 24)

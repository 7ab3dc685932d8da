"""ctypes binding of libsmla.so (include/smla.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no fallback: if the library is missing the import fails.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime before libsmla binds to it)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmla.so")
# The LDS-poisoning debug build (same ABI; tests of races and unwritten LDS)
POISON_LIB_PATH = os.path.join(HERE, "libsmla_poison.so")

SMLA_OK = 0
SMLA_ERR_INVALID_ARGUMENT = 1
SMLA_ERR_UNSUPPORTED = 2
SMLA_ERR_WORKSPACE = 3
SMLA_ERR_HIP = 4
SMLA_SCHEDULE_AUTO = 0
SMLA_SCHEDULE_GRID = 1
SMLA_SCHEDULE_PERSISTENT = 2
SMLA_KV_BF16 = 0
SMLA_KV_FP8_E4M3 = 1
SMLA_KV_FP4_E2M1 = 2
D_QK = 576
D_V = 512
FP8_GROUP = 128
FP8_NUM_GROUPS = 5
FP8_ROW_BYTES = 640
FP4_ROW_BYTES = 320
MAX_SLOTS_PER_SPLIT = 2048
MAX_SLOTS_PER_SPLIT_FP8 = 1536

# Every symbol include/smla.h declares.
EXPORTS = ("smla_fwd_plan", "smla_fwd_schedule", "smla_fwd_workspace_size", "smla_fwd", "smla_fwd_static_scratch",
           "smla_fwd_paged_workspace_size",
           "smla_fwd_paged", "smla_fwd_tune_workspace_size", "smla_fwd_tune", "smla_pack_fp8_kv_host",
           "smla_pack_fp4_kv_host", "smla_status_string", "smla_last_error", "smla_abi_version")
ABI_VERSION = 6
STATIC_SCRATCH_BYTES = 64 << 20


class smla_fwd_params(ctypes.Structure):
    _fields_ = [
        ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32), ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("topk", ctypes.c_int32), ("s_kv", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_stride_token", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("kv", ctypes.c_void_p), ("kv_stride_row", ctypes.c_int64), ("kv_format", ctypes.c_int32),
        ("indices", ctypes.c_void_p), ("indices_stride_token", ctypes.c_int64),
        ("out", ctypes.c_void_p), ("out_stride_token", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("lse_stride_token", ctypes.c_int64),
        ("num_splits", ctypes.c_int32), ("b_topk", ctypes.c_int32),
        ("schedule", ctypes.c_int32), ("persistent_workgroups", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class smla_paged_kv(ctypes.Structure):
    _fields_ = [
        ("block_table", ctypes.c_void_p), ("block_table_stride_token", ctypes.c_int64),
        ("table_width", ctypes.c_int32), ("page_size", ctypes.c_int32),
    ]


class SmlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_mla_attention_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(smla_fwd_params)
    lib.smla_fwd_plan.argtypes = [P, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.smla_fwd_plan.restype = ctypes.c_int
    lib.smla_fwd_schedule.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.smla_fwd_schedule.restype = ctypes.c_int
    lib.smla_fwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.smla_fwd_workspace_size.restype = ctypes.c_int
    lib.smla_fwd.argtypes = [P, ctypes.c_void_p]
    lib.smla_fwd.restype = ctypes.c_int
    lib.smla_fwd_static_scratch.argtypes = [P, ctypes.c_void_p]
    lib.smla_fwd_static_scratch.restype = ctypes.c_int
    G = ctypes.POINTER(smla_paged_kv)
    lib.smla_fwd_paged_workspace_size.argtypes = [P, G, ctypes.POINTER(ctypes.c_size_t)]
    lib.smla_fwd_paged_workspace_size.restype = ctypes.c_int
    lib.smla_fwd_paged.argtypes = [P, G, ctypes.c_void_p]
    lib.smla_fwd_paged.restype = ctypes.c_int
    lib.smla_fwd_tune_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.smla_fwd_tune_workspace_size.restype = ctypes.c_int
    I32 = ctypes.POINTER(ctypes.c_int32)
    lib.smla_fwd_tune.argtypes = [P, ctypes.c_void_p, ctypes.c_int32, I32, I32, ctypes.POINTER(ctypes.c_float)]
    lib.smla_fwd_tune.restype = ctypes.c_int
    lib.smla_pack_fp8_kv_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.smla_pack_fp8_kv_host.restype = ctypes.c_int
    lib.smla_pack_fp4_kv_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.smla_pack_fp4_kv_host.restype = ctypes.c_int
    lib.smla_status_string.argtypes = [ctypes.c_int32]
    lib.smla_status_string.restype = ctypes.c_char_p
    lib.smla_last_error.argtypes = []
    lib.smla_last_error.restype = ctypes.c_char_p
    lib.smla_abi_version.argtypes = []
    lib.smla_abi_version.restype = ctypes.c_int32
    if lib.smla_abi_version() != ABI_VERSION:
        raise ImportError(f"libsmla ABI version {lib.smla_abi_version()} != {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


@contextlib.contextmanager
def library(path: str):
    """Inside the block every call of this binding goes to the library at
    ``path`` (another build of the same ABI, such as POISON_LIB_PATH); the
    library loaded before is restored afterwards."""
    global _lib
    saved = _lib
    _lib = None
    try:
        yield load(path)
    finally:
        _lib = saved


def status_string(status: int) -> str:
    return load().smla_status_string(status).decode()


def last_error() -> str:
    return load().smla_last_error().decode()


def _check(status: int):
    if status != SMLA_OK:
        raise SmlaError(status, last_error())


def smla_fwd_plan(params: smla_fwd_params) -> tuple[int, int]:
    ns, bt = ctypes.c_int32(), ctypes.c_int32()
    _check(load().smla_fwd_plan(ctypes.byref(params), ctypes.byref(ns), ctypes.byref(bt)))
    return ns.value, bt.value


def smla_fwd_schedule(params: smla_fwd_params) -> int:
    """SMLA_SCHEDULE_GRID or SMLA_SCHEDULE_PERSISTENT: the schedule the library
    would run."""
    v = ctypes.c_int32()
    _check(load().smla_fwd_schedule(ctypes.byref(params), ctypes.byref(v)))
    return v.value


def smla_fwd_workspace_size(params: smla_fwd_params) -> int:
    n = ctypes.c_size_t()
    _check(load().smla_fwd_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def smla_fwd(params: smla_fwd_params, stream: int | None = None):
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(load().smla_fwd(ctypes.byref(params), ctypes.c_void_p(stream)))


def smla_fwd_static_scratch(params: smla_fwd_params, stream: int | None = None):
    """smla_fwd with the split partials in the library's per-device static
    scratch (no workspace, no allocation)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(load().smla_fwd_static_scratch(ctypes.byref(params), ctypes.c_void_p(stream)))


def smla_fwd_paged_workspace_size(params: smla_fwd_params, paged: smla_paged_kv) -> int:
    n = ctypes.c_size_t()
    _check(load().smla_fwd_paged_workspace_size(ctypes.byref(params), ctypes.byref(paged), ctypes.byref(n)))
    return n.value


def smla_fwd_paged(params: smla_fwd_params, paged: smla_paged_kv, stream: int | None = None):
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    _check(load().smla_fwd_paged(ctypes.byref(params), ctypes.byref(paged), ctypes.c_void_p(stream)))


def smla_fwd_tune_workspace_size(params: smla_fwd_params) -> int:
    n = ctypes.c_size_t()
    _check(load().smla_fwd_tune_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def smla_fwd_tune(params: smla_fwd_params, iterations: int = 10,
                  stream: int | None = None) -> tuple[int, int, float]:
    """Time the candidate plans; returns (num_splits, b_topk, microseconds)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ns, bt, us = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    _check(load().smla_fwd_tune(ctypes.byref(params), ctypes.c_void_p(stream), int(iterations),
                                ctypes.byref(ns), ctypes.byref(bt), ctypes.byref(us)))
    return ns.value, bt.value, us.value


def make_paged(block_table: torch.Tensor, page_size: int) -> smla_paged_kv:
    """smla_paged_kv for an int32 block table [s_q, table_width]."""
    g = smla_paged_kv()
    g.block_table = block_table.data_ptr()
    g.block_table_stride_token = block_table.stride(0)
    g.table_width = block_table.shape[1]
    g.page_size = int(page_size)
    return g


def smla_pack_fp8_kv_host(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """Pack host uint8 codes [rows, 576] and float32 scales [rows, 5] into
    640-byte fp8 KV rows (a host uint8 tensor [rows, 640])."""
    codes = codes.contiguous()
    scales = scales.to(torch.float32).contiguous()
    assert codes.dtype == torch.uint8 and codes.dim() == 2 and codes.shape[1] == D_QK
    assert scales.shape == (codes.shape[0], FP8_NUM_GROUPS)
    rows = codes.shape[0]
    packed = torch.empty((rows, FP8_ROW_BYTES), dtype=torch.uint8)
    _check(load().smla_pack_fp8_kv_host(codes.data_ptr(), scales.data_ptr(), rows, packed.data_ptr()))
    return packed


def smla_pack_fp4_kv_host(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """Pack host uint8 E2M1 codes [rows, 576] (one 4-bit code per byte) and
    float32 scales [rows, 5] into 320-byte fp4 KV rows (a host uint8 tensor
    [rows, 320])."""
    codes = codes.contiguous()
    scales = scales.to(torch.float32).contiguous()
    assert codes.dtype == torch.uint8 and codes.dim() == 2 and codes.shape[1] == D_QK
    assert scales.shape == (codes.shape[0], FP8_NUM_GROUPS)
    rows = codes.shape[0]
    packed = torch.empty((rows, FP4_ROW_BYTES), dtype=torch.uint8)
    _check(load().smla_pack_fp4_kv_host(codes.data_ptr(), scales.data_ptr(), rows, packed.data_ptr()))
    return packed


def make_params(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                out: torch.Tensor, lse: torch.Tensor, *, kv_format: int = SMLA_KV_BF16,
                s_kv: int | None = None, num_splits: int = 0, b_topk: int = 0, schedule: int = 0,
                persistent_workgroups: int = 0) -> smla_fwd_params:
    """Fill smla_fwd_params from tensors (no checks beyond shapes: the library
    validates everything else)."""
    s_q, h_q, d_qk = q.shape
    p = smla_fwd_params()
    p.s_q, p.h_q, p.d_qk, p.d_v = s_q, h_q, d_qk, out.shape[-1]
    p.topk = indices.shape[1]
    p.s_kv = kv.shape[0] if s_kv is None else s_kv
    p.sm_scale = float(sm_scale)
    p.q, p.q_stride_token, p.q_stride_head = q.data_ptr(), q.stride(0), q.stride(1)
    p.kv = kv.data_ptr()
    p.kv_stride_row = kv.stride(0) * (kv.element_size() if kv_format != SMLA_KV_BF16 else 1)
    p.kv_format = kv_format
    p.indices, p.indices_stride_token = indices.data_ptr(), indices.stride(0)
    p.out, p.out_stride_token, p.out_stride_head = out.data_ptr(), out.stride(0), out.stride(1)
    p.lse, p.lse_stride_token = lse.data_ptr(), lse.stride(0)
    p.num_splits, p.b_topk = num_splits, b_topk
    p.schedule, p.persistent_workgroups = schedule, persistent_workgroups
    return p

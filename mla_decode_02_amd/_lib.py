"""ctypes binding for libmla_decode.so (C ABI: include/mla_decode.h).

Argument marshalling only: shape / dtype / device checks that the C side
cannot make (it only sees pointers), pointer extraction, the current HIP
stream, and -- when the caller passes none -- a workspace of the size the
library asks for, with its arrival-counter region zeroed as the C ABI requires
(kept per device and stream and reused by that stream's later calls, so a call
without a workspace allocates only when it needs a larger one). No arithmetic
of the operation happens here.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_DECODE_LIBRARY=phases loads the measurement build of the same sources,
# whose kernels record phase timestamps (include/mla_decode_phases.h); only
# bench.py --phases sets it. Otherwise the decode library is loaded.
PHASES = os.environ.get("MLA_DECODE_LIBRARY", "") == "phases"
LIB_PATH = os.path.join(_HERE, "libmla_decode_phases.so" if PHASES else "libmla_decode.so")

NUM_HEADS, QK_DIM, V_DIM = 16, 576, 512
KV_BF16, KV_FP8_E4M3, KV_MXFP4 = 0, 1, 2
FLAG_FORCE_SPLIT, FLAG_FORCE_PERSISTENT, FLAG_MIXED_LENGTHS, FLAG_COMBINE_LAUNCH = 0x1, 0x2, 0x4, 0x8
FLAG_ROW_PER_WG = 0x10  # several-query-token calls: one query row per workgroup
WORKSPACE_COUNTER_BYTES = 65536  # leading workspace bytes that hold the arrival counters (zero between calls)
FLAG_SPLITS_SHIFT, FLAG_GRID_SHIFT = 8, 16
Q_SCALE_STATIC, Q_SCALE_DYNAMIC = 0, 1

_EXPORTS = ("mla_decode", "mla_decode_rows", "mla_decode_noalloc", "mla_decode_paged", "mla_decode_q8", "mla_decode_mtp", "mla_decode_plan",
            "mla_decode_mtp_plan",
            "mla_decode_workspace_size", "mla_decode_q8_workspace_size", "mla_decode_mtp_workspace_size",
            "mla_quantize_q8_debug", "mla_dequant_debug", "mla_hbm_read_probe", "mla_status_string",
            "mla_source_digest")


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mla_status_string(status)} (status {status})")
        self.status = status


class _Plan(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("num_splits", ctypes.c_int), ("grid", ctypes.c_int),
                ("num_partials", ctypes.c_int), ("combine", ctypes.c_int), ("rows_per_wg", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


@dataclass(frozen=True)
class PlanInfo:
    mode: int            # 0 split-K, 1 persistent
    num_splits: int
    grid: int
    num_partials: int
    combine: int         # 0 none, 1 combine launch, 2 merged by the last-arriving split workgroup
    workspace_bytes: int
    rows_per_wg: int = 1  # query rows each stage-1 workgroup carries


def new_workspace(nbytes: int, device, poison: bool = False):
    """A decode workspace of nbytes: the arrival-counter region zeroed (the C ABI
    requires it once; calls leave it zero). poison fills the rest with NaN, so a
    read of a partial that no workgroup wrote would show in the output."""
    ws = torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    if poison and ws.numel() > WORKSPACE_COUNTER_BYTES:
        ws[WORKSPACE_COUNTER_BYTES:].view(torch.float32).fill_(float("nan"))
    return ws


# Workspaces of the calls made without one, one per (device, stream): calls on a
# stream run in order and each leaves the arrival-counter region zero, so a
# stream's workspace is reused by its next call; it grows when a call needs more.
_STREAM_WORKSPACES = {}


def _stream_workspace(nbytes: int, device):
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(device).cuda_stream)
    ws = _STREAM_WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(nbytes, device)
        _STREAM_WORKSPACES[key] = ws
    return ws


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mla_decode_02_amd/build.py` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name in _EXPORTS:
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}")
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, ctypes.c_float, vp, sz, i32, vp]
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, ctypes.c_float, i32, vp]
    lib.mla_decode_rows.restype = i32
    lib.mla_decode_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i32, ctypes.c_float, vp, sz, i32, vp]
    lib.mla_decode_paged.restype = i32
    lib.mla_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i64, i32, ctypes.c_float, vp, sz, i32,
                                     vp]
    lib.mla_decode_q8.restype = i32
    lib.mla_decode_q8.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, vp, vp, i32, i64, i32, ctypes.c_float, vp, sz,
                                  i32, vp]
    lib.mla_decode_q8_workspace_size.restype = sz
    lib.mla_decode_q8_workspace_size.argtypes = [i32, i64, i32, i32, i32]
    lib.mla_quantize_q8_debug.restype = i32
    lib.mla_quantize_q8_debug.argtypes = [vp, i32, vp, i32, vp, vp, sz, vp]
    lib.mla_decode_mtp.restype = i32
    lib.mla_decode_mtp.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, i32, i64, i32,
                                   ctypes.c_float, vp, sz, i32, vp]
    lib.mla_decode_mtp_workspace_size.restype = sz
    lib.mla_decode_mtp_workspace_size.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.mla_decode_mtp_plan.restype = i32
    lib.mla_decode_mtp_plan.argtypes = [i32, i32, i32, i64, i32, i32, ctypes.POINTER(_Plan)]
    lib.mla_decode_plan.restype = i32
    lib.mla_decode_plan.argtypes = [i32, i64, i32, i32, ctypes.POINTER(_Plan)]
    lib.mla_decode_workspace_size.restype = sz
    lib.mla_decode_workspace_size.argtypes = [i32, i64, i32, i32]
    lib.mla_dequant_debug.restype = i32
    lib.mla_dequant_debug.argtypes = [i32, vp, vp, i64, i32, vp, vp]
    lib.mla_hbm_read_probe.restype = i32
    lib.mla_hbm_read_probe.argtypes = [vp, sz, vp]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [i32]
    lib.mla_source_digest.restype = ctypes.c_char_p
    lib.mla_source_digest.argtypes = []
    if PHASES:
        if not hasattr(lib, "mla_phase_buffers"):
            raise ImportError(f"{LIB_PATH} is not the measurement build (no mla_phase_buffers)")
        lib.mla_phase_buffers.restype = i32
        lib.mla_phase_buffers.argtypes = [vp, vp]
    # A library built from other sources than the ones beside it (an edit not
    # followed by a build) would run kernels that are not the tree's: refuse it.
    built = lib.mla_source_digest().decode()
    if all(os.path.exists(p) for p in _build.SOURCES):
        tree = _build.source_digest()
        if built != tree:
            raise ImportError(
                f"{LIB_PATH} was built from sources with digest {built}, the tree's are {tree}: "
                "rebuild it with `python mla_decode_02_amd/build.py`")
    return lib


_lib = _load()


def mla_status_string(status: int) -> str:
    return _lib.mla_status_string(int(status)).decode()


def mla_phase_buffers(stage1, combine) -> None:
    """Measurement build only: the int64 device tensors the next launches write
    their phase timestamps into (include/mla_decode_phases.h), or None."""
    if not PHASES:
        raise RuntimeError("phase timestamps need the measurement build (MLA_DECODE_LIBRARY=phases)")
    for t in (stage1, combine):
        _need(t is None or (t.is_cuda and t.dtype == torch.int64 and t.is_contiguous()),
              "phase buffers must be contiguous int64 device tensors")
    rc = _lib.mla_phase_buffers(_ptr(stage1), _ptr(combine))
    if rc != 0:
        raise MlaError(rc, "mla_phase_buffers")


def mla_source_digest() -> str:
    """Digest of the sources the loaded library was compiled from."""
    return _lib.mla_source_digest().decode()


def flags_for(splits: int | None = None, persistent: bool | None = None, grid: int | None = None) -> int:
    """Compose the flags word: force split-K with `splits`, or persistent with `grid` workgroups."""
    f = 0
    if persistent:
        f |= FLAG_FORCE_PERSISTENT
        if grid:
            f |= (int(grid) & 0xFFF) << FLAG_GRID_SHIFT
    elif splits:
        f |= FLAG_FORCE_SPLIT | ((int(splits) & 0xFF) << FLAG_SPLITS_SHIFT)
    return f


def mla_decode_plan(batch: int, total_kv: int, kv_dtype: int, flags: int = 0) -> PlanInfo:
    p = _Plan()
    rc = _lib.mla_decode_plan(int(batch), int(total_kv), int(kv_dtype), int(flags), ctypes.byref(p))
    if rc != 0:
        raise MlaError(rc, "mla_decode_plan")
    return PlanInfo(p.mode, p.num_splits, p.grid, p.num_partials, p.combine, p.workspace_bytes, p.rows_per_wg)


def mla_decode_mtp_plan(batch: int, total_q: int, total_kv: int, kv_dtype: int, flags: int = 0,
                        uni_q_len: int = 0) -> PlanInfo:
    """The launch plan of mla_decode_mtp (include/mla_decode.h, mla_decode_mtp_plan)."""
    p = _Plan()
    rc = _lib.mla_decode_mtp_plan(int(batch), int(total_q), int(uni_q_len), int(total_kv), int(kv_dtype), int(flags),
                                  ctypes.byref(p))
    if rc != 0:
        raise MlaError(rc, "mla_decode_mtp_plan")
    return PlanInfo(p.mode, p.num_splits, p.grid, p.num_partials, p.combine, p.workspace_bytes, p.rows_per_wg)


def mla_decode_workspace_size(batch: int, total_kv: int, kv_dtype: int, flags: int = 0) -> int:
    return int(_lib.mla_decode_workspace_size(int(batch), int(total_kv), int(kv_dtype), int(flags)))


def mla_decode_q8_workspace_size(batch: int, total_kv: int, kv_dtype: int, flags: int = 0,
                                 q_scale_mode: int = Q_SCALE_DYNAMIC) -> int:
    return int(_lib.mla_decode_q8_workspace_size(int(batch), int(total_kv), int(kv_dtype), int(flags),
                                                 int(q_scale_mode)))


def mla_decode_mtp_workspace_size(batch: int, total_q: int, total_kv: int, kv_dtype: int, flags: int = 0,
                                  uni_q_len: int = 0) -> int:
    return int(_lib.mla_decode_mtp_workspace_size(int(batch), int(total_q), int(uni_q_len), int(total_kv),
                                                  int(kv_dtype), int(flags)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_kv(kv, kv_scales, kv_dtype):
    _need(kv.is_cuda and kv.is_contiguous(), "kv must be a contiguous device tensor")
    if kv_dtype == KV_BF16:
        _need(kv.dtype == torch.bfloat16 and kv.dim() == 2 and kv.shape[1] == QK_DIM, "bf16 kv must be [rows, 576]")
        _need(kv_scales is None, "bf16 kv takes no scales")
    elif kv_dtype == KV_FP8_E4M3:
        _need(kv.dtype in (torch.uint8, torch.float8_e4m3fn) and kv.dim() == 2 and kv.shape[1] == QK_DIM,
              "fp8 kv must be uint8/float8_e4m3fn [rows, 576]")
        _need(kv_scales is not None and kv_scales.is_cuda and kv_scales.dtype == torch.float32
              and kv_scales.numel() >= 1, "fp8 kv needs a device fp32 scale tensor")
    elif kv_dtype == KV_MXFP4:
        _need(kv.dtype == torch.uint8 and kv.dim() == 2 and kv.shape[1] == QK_DIM // 2, "mxfp4 kv must be uint8 [rows, 288]")
        _need(kv_scales is not None and kv_scales.is_cuda and kv_scales.is_contiguous()
              and kv_scales.dtype in (torch.uint8, torch.float8_e8m0fnu)
              and tuple(kv_scales.shape) == (kv.shape[0], QK_DIM // 32), "mxfp4 scales must be uint8 [rows, 18]")
    else:
        raise ValueError(f"unknown kv_dtype {kv_dtype}")


def mla_decode(q, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, total_kv: int, kv_dtype: int,
               sm_scale: float = 0.0, workspace=None, flags: int = 0, kv_rows: int | None = None):
    """Enqueue MLA decode on the current stream of q's device (see include/mla_decode.h).

    q [B,16,576] bf16, kv / kv_scales per kv_dtype, kv_indptr [B+1] int32,
    kv_indices [total_kv] int32, out [B,16,512] bf16, lse [B,16] fp32 or None.
    total_kv is the host copy of kv_indptr[B]. kv_rows is the cache's row
    count for mla_decode_rows (None: kv's own, 0: unknown, i.e. mla_decode).
    Returns the workspace used.
    """
    B = int(kv_indptr.shape[0]) - 1
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and tuple(q.shape) == (B, NUM_HEADS, QK_DIM),
          "q must be contiguous bf16 [batch, 16, 576]")
    _check_kv(kv, kv_scales, kv_dtype)
    _need(kv_indptr.is_cuda and kv_indptr.dtype == torch.int32 and kv_indptr.is_contiguous(),
          "kv_indptr must be a contiguous device int32 tensor")
    _need(kv_indices.is_cuda and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous()
          and kv_indices.numel() >= total_kv, "kv_indices must be a contiguous device int32 tensor of >= total_kv")
    _need(out.is_cuda and out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (B, NUM_HEADS, V_DIM),
          "out must be contiguous bf16 [batch, 16, 512]")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, NUM_HEADS),
              "lse must be contiguous fp32 [batch, 16]")
    need = mla_decode_workspace_size(B, total_kv, kv_dtype, flags)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rows = _kv_rows(kv, kv_rows)
    rc = _lib.mla_decode_rows(_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices), _ptr(out),
                              _ptr(lse), B, int(total_kv), rows, int(kv_dtype), float(sm_scale), _ptr(workspace),
                              ws_bytes, int(flags), _stream(q.device))
    if rc != 0:
        raise MlaError(rc, "mla_decode")
    return workspace


def mla_decode_noalloc(q, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, total_kv: int, kv_dtype: int,
                       sm_scale: float = 0.0, flags: int = 0):
    """Enqueue mla_decode_noalloc (see include/mla_decode.h): mla_decode without a
    workspace, its partials in the library's fixed per-device scratch array. Nothing is
    allocated, here or in the library. Calls that may overlap on one device race."""
    B = int(kv_indptr.shape[0]) - 1
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and tuple(q.shape) == (B, NUM_HEADS, QK_DIM),
          "q must be contiguous bf16 [batch, 16, 576]")
    _check_kv(kv, kv_scales, kv_dtype)
    _need(kv_indptr.is_cuda and kv_indptr.dtype == torch.int32 and kv_indptr.is_contiguous(),
          "kv_indptr must be a contiguous device int32 tensor")
    _need(kv_indices.is_cuda and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous()
          and kv_indices.numel() >= total_kv, "kv_indices must be a contiguous device int32 tensor of >= total_kv")
    _need(out.is_cuda and out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (B, NUM_HEADS, V_DIM),
          "out must be contiguous bf16 [batch, 16, 512]")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, NUM_HEADS),
              "lse must be contiguous fp32 [batch, 16]")
    rc = _lib.mla_decode_noalloc(_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices), _ptr(out),
                                 _ptr(lse), B, int(total_kv), int(kv_dtype), float(sm_scale), int(flags),
                                 _stream(q.device))
    if rc != 0:
        raise MlaError(rc, "mla_decode_noalloc")


def _kv_rows(kv, kv_rows):
    """The cache row count passed to mla_decode_rows: kv's leading dimension
    unless the caller gives one (0 turns the early row requests off; more rows
    than kv holds are refused, since the kernels may read below that bound)."""
    if kv_rows is None:
        return int(kv.shape[0])
    _need(0 <= int(kv_rows) <= int(kv.shape[0]), "kv_rows must lie in [0, kv.shape[0]]")
    return int(kv_rows)


def mla_decode_paged(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse=None, *, page_size: int,
                     total_kv: int, kv_dtype: int, sm_scale: float = 0.0, workspace=None, flags: int = 0):
    """Enqueue MLA decode over a paged cache (see include/mla_decode.h, mla_decode_paged).

    kv rows grouped in pages of page_size rows ([pages * page_size, ...] as for
    mla_decode); kv_indptr [B+1] int32 into kv_indices (page ids);
    kv_last_page_len [B] int32 (tokens in each sequence's last page);
    total_kv is the host total token count. Returns the workspace used.
    """
    B = int(kv_indptr.shape[0]) - 1
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and tuple(q.shape) == (B, NUM_HEADS, QK_DIM),
          "q must be contiguous bf16 [batch, 16, 576]")
    _check_kv(kv, kv_scales, kv_dtype)
    _need(kv.shape[0] % max(int(page_size), 1) == 0, "kv rows must be a whole number of pages")
    _need(kv_indptr.is_cuda and kv_indptr.dtype == torch.int32 and kv_indptr.is_contiguous(),
          "kv_indptr must be a contiguous device int32 tensor")
    _need(kv_indices.is_cuda and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous(),
          "kv_indices must be a contiguous device int32 tensor")
    if page_size > 1:
        _need(kv_last_page_len is not None and kv_last_page_len.is_cuda and kv_last_page_len.dtype == torch.int32
              and kv_last_page_len.is_contiguous() and kv_last_page_len.numel() == B,
              "kv_last_page_len must be a contiguous device int32 tensor [batch]")
    _need(out.is_cuda and out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (B, NUM_HEADS, V_DIM),
          "out must be contiguous bf16 [batch, 16, 512]")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, NUM_HEADS),
              "lse must be contiguous fp32 [batch, 16]")
    plan_flags = flags | (FLAG_FORCE_SPLIT if page_size > 1 else 0)
    need = mla_decode_workspace_size(B, total_kv, kv_dtype, plan_flags)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.mla_decode_paged(_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices),
                               _ptr(kv_last_page_len), int(page_size), _ptr(out), _ptr(lse), B, int(total_kv),
                               int(kv_dtype), float(sm_scale), _ptr(workspace), ws_bytes, int(flags),
                               _stream(q.device))
    if rc != 0:
        raise MlaError(rc, "mla_decode_paged")
    return workspace


def prepare_decode(q, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, total_kv: int, kv_dtype: int,
                   sm_scale: float = 0.0, workspace=None, flags: int = 0, kv_rows: int | None = None):
    """Check and marshal the arguments once; return a zero-argument callable that
    enqueues the same mla_decode call (through mla_decode_rows, kv_rows as for
    mla_decode) on the current stream (for serving loops and timing, where
    per-call Python checks would dominate). The tensors must stay alive and in
    place while the callable is used."""
    ws = mla_decode(q, kv, kv_scales, kv_indptr, kv_indices, out, lse, total_kv=total_kv, kv_dtype=kv_dtype,
                    sm_scale=sm_scale, workspace=workspace, flags=flags, kv_rows=kv_rows)
    B = int(kv_indptr.shape[0]) - 1
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    args = (_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices), _ptr(out), _ptr(lse), B,
            int(total_kv), _kv_rows(kv, kv_rows), int(kv_dtype), float(sm_scale), _ptr(ws), ws_bytes, int(flags),
            _stream(q.device))
    fn = _lib.mla_decode_rows
    keep = (q, kv, kv_scales, kv_indptr, kv_indices, out, lse, ws)

    def call():
        rc = fn(*args)
        if rc != 0:
            raise MlaError(rc, "mla_decode")
        return keep

    return call


def prepare_decode_paged(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse=None, *,
                         page_size: int, total_kv: int, kv_dtype: int, sm_scale: float = 0.0, workspace=None,
                         flags: int = 0):
    """prepare_decode for mla_decode_paged: checks once (one checked call),
    then returns a zero-argument callable that enqueues the same call."""
    ws = mla_decode_paged(q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, page_size=page_size,
                          total_kv=total_kv, kv_dtype=kv_dtype, sm_scale=sm_scale, workspace=workspace, flags=flags)
    B = int(kv_indptr.shape[0]) - 1
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    args = (_ptr(q), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len),
            int(page_size), _ptr(out), _ptr(lse), B, int(total_kv), int(kv_dtype), float(sm_scale), _ptr(ws),
            ws_bytes, int(flags), _stream(q.device))
    fn = _lib.mla_decode_paged
    keep = (q, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, ws)

    def call():
        rc = fn(*args)
        if rc != 0:
            raise MlaError(rc, "mla_decode_paged")
        return keep

    return call


def mla_dequant_debug(kv, kv_scales, kv_dtype: int, path: int = 0, out=None):
    """Decode every physical cache row to fp32 [rows, 576] with the kernels' decode routines.

    path 0: score-operand decode for all columns; path 1: value-operand decode
    (transposed LDS reads) for columns 0..511.
    """
    _check_kv(kv, kv_scales, kv_dtype)
    rows = int(kv.shape[0])
    if out is None:
        out = torch.empty((rows, QK_DIM), dtype=torch.float32, device=kv.device)
    _need(out.is_cuda and out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (rows, QK_DIM),
          "out must be contiguous fp32 [rows, 576]")
    rc = _lib.mla_dequant_debug(int(kv_dtype), _ptr(kv), _ptr(kv_scales), rows, int(path), _ptr(out),
                                _stream(kv.device))
    if rc != 0:
        raise MlaError(rc, "mla_dequant_debug")
    return out


def _check_q_scale(q_scale, q_scale_mode):
    _need(q_scale_mode in (Q_SCALE_STATIC, Q_SCALE_DYNAMIC), f"unknown q_scale_mode {q_scale_mode}")
    _need(q_scale is not None and q_scale.is_cuda and q_scale.dtype == torch.float32 and q_scale.numel() >= 1,
          "q_scale must be a device fp32 tensor of >= 1 element")


def mla_decode_q8(q, q_scale, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, q_scale_mode: int,
                  total_kv: int, kv_dtype: int, kv_last_page_len=None, page_size: int = 1, sm_scale: float = 0.0,
                  workspace=None, flags: int = 0):
    """Enqueue MLA decode with an fp8-quantised query (see include/mla_decode.h, mla_decode_q8).

    q [B,16,576] bf16 (quantised inside the call); q_scale device fp32 [1]: read
    (Q_SCALE_STATIC) or written (Q_SCALE_DYNAMIC). The cache arguments are those
    of mla_decode_paged (page_size 1: those of mla_decode). Returns the workspace.
    """
    B = int(kv_indptr.shape[0]) - 1
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and tuple(q.shape) == (B, NUM_HEADS, QK_DIM),
          "q must be contiguous bf16 [batch, 16, 576]")
    _check_q_scale(q_scale, q_scale_mode)
    _check_kv(kv, kv_scales, kv_dtype)
    _need(kv.shape[0] % max(int(page_size), 1) == 0, "kv rows must be a whole number of pages")
    _need(kv_indptr.is_cuda and kv_indptr.dtype == torch.int32 and kv_indptr.is_contiguous(),
          "kv_indptr must be a contiguous device int32 tensor")
    _need(kv_indices.is_cuda and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous(),
          "kv_indices must be a contiguous device int32 tensor")
    if page_size > 1:
        _need(kv_last_page_len is not None and kv_last_page_len.is_cuda and kv_last_page_len.dtype == torch.int32
              and kv_last_page_len.is_contiguous() and kv_last_page_len.numel() == B,
              "kv_last_page_len must be a contiguous device int32 tensor [batch]")
    else:
        _need(kv_indices.numel() >= total_kv, "kv_indices must hold >= total_kv entries")
    _need(out.is_cuda and out.dtype == torch.bfloat16 and out.is_contiguous() and tuple(out.shape) == (B, NUM_HEADS, V_DIM),
          "out must be contiguous bf16 [batch, 16, 512]")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, NUM_HEADS),
              "lse must be contiguous fp32 [batch, 16]")
    plan_flags = flags | (FLAG_FORCE_SPLIT if page_size > 1 else 0)
    need = mla_decode_q8_workspace_size(B, total_kv, kv_dtype, plan_flags, q_scale_mode)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.mla_decode_q8(_ptr(q), _ptr(q_scale), int(q_scale_mode), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr),
                            _ptr(kv_indices), _ptr(kv_last_page_len), int(page_size), _ptr(out), _ptr(lse), B,
                            int(total_kv), int(kv_dtype), float(sm_scale), _ptr(workspace), ws_bytes, int(flags),
                            _stream(q.device))
    if rc != 0:
        raise MlaError(rc, "mla_decode_q8")
    return workspace


def prepare_decode_q8(q, q_scale, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, q_scale_mode: int,
                      total_kv: int, kv_dtype: int, kv_last_page_len=None, page_size: int = 1,
                      sm_scale: float = 0.0, workspace=None, flags: int = 0):
    """prepare_decode for mla_decode_q8: checks once (one checked call), then
    returns a zero-argument callable that enqueues the same call."""
    ws = mla_decode_q8(q, q_scale, kv, kv_scales, kv_indptr, kv_indices, out, lse, q_scale_mode=q_scale_mode,
                       total_kv=total_kv, kv_dtype=kv_dtype, kv_last_page_len=kv_last_page_len,
                       page_size=page_size, sm_scale=sm_scale, workspace=workspace, flags=flags)
    B = int(kv_indptr.shape[0]) - 1
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    args = (_ptr(q), _ptr(q_scale), int(q_scale_mode), _ptr(kv), _ptr(kv_scales), _ptr(kv_indptr), _ptr(kv_indices),
            _ptr(kv_last_page_len), int(page_size), _ptr(out), _ptr(lse), B, int(total_kv), int(kv_dtype),
            float(sm_scale), _ptr(ws), ws_bytes, int(flags), _stream(q.device))
    fn = _lib.mla_decode_q8
    keep = (q, q_scale, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, ws)

    def call():
        rc = fn(*args)
        if rc != 0:
            raise MlaError(rc, "mla_decode_q8")
        return keep

    return call


def mla_quantize_q8_debug(q, q_scale, q_scale_mode: int, codes=None, workspace=None):
    """The query quantisation of mla_decode_q8 on its own: e4m3fn codes uint8 [B,16,576]
    (q_scale read for Q_SCALE_STATIC, written for Q_SCALE_DYNAMIC). Returns codes."""
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous() and q.dim() == 3
          and tuple(q.shape[1:]) == (NUM_HEADS, QK_DIM), "q must be contiguous bf16 [batch, 16, 576]")
    _check_q_scale(q_scale, q_scale_mode)
    B = int(q.shape[0])
    if codes is None:
        codes = torch.empty((B, NUM_HEADS, QK_DIM), dtype=torch.uint8, device=q.device)
    _need(codes.is_cuda and codes.dtype == torch.uint8 and codes.is_contiguous()
          and tuple(codes.shape) == (B, NUM_HEADS, QK_DIM), "codes must be contiguous uint8 [batch, 16, 576]")
    if workspace is None and q_scale_mode == Q_SCALE_DYNAMIC:
        workspace = torch.empty(1024, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.mla_quantize_q8_debug(_ptr(q), B, _ptr(q_scale), int(q_scale_mode), _ptr(codes), _ptr(workspace),
                                    ws_bytes, _stream(q.device))
    if rc != 0:
        raise MlaError(rc, "mla_quantize_q8_debug")
    return codes


def _mtp_args(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, total_q, uni_q_len,
              causal, total_kv, kv_dtype, page_size, sm_scale, workspace, flags):
    B = int(kv_indptr.shape[0]) - 1
    _need(q.is_cuda and q.dtype == torch.bfloat16 and q.is_contiguous()
          and tuple(q.shape) == (total_q, NUM_HEADS, QK_DIM), "q must be contiguous bf16 [total_q, 16, 576]")
    if uni_q_len:
        _need(int(uni_q_len) * B == int(total_q), "uniform query length: total_q must be batch * uni_q_len")
    else:
        _need(qo_indptr is not None and qo_indptr.is_cuda and qo_indptr.dtype == torch.int32
              and qo_indptr.is_contiguous() and qo_indptr.numel() == B + 1,
              "qo_indptr must be a contiguous device int32 tensor [batch + 1]")
    _check_kv(kv, kv_scales, kv_dtype)
    _need(kv.shape[0] % max(int(page_size), 1) == 0, "kv rows must be a whole number of pages")
    _need(kv_indptr.is_cuda and kv_indptr.dtype == torch.int32 and kv_indptr.is_contiguous(),
          "kv_indptr must be a contiguous device int32 tensor")
    _need(kv_indices.is_cuda and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous(),
          "kv_indices must be a contiguous device int32 tensor")
    if page_size > 1:
        _need(kv_last_page_len is not None and kv_last_page_len.is_cuda and kv_last_page_len.dtype == torch.int32
              and kv_last_page_len.is_contiguous() and kv_last_page_len.numel() == B,
              "kv_last_page_len must be a contiguous device int32 tensor [batch]")
    _need(out.is_cuda and out.dtype == torch.bfloat16 and out.is_contiguous()
          and tuple(out.shape) == (total_q, NUM_HEADS, V_DIM), "out must be contiguous bf16 [total_q, 16, 512]")
    if lse is not None:
        _need(lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
              and tuple(lse.shape) == (total_q, NUM_HEADS), "lse must be contiguous fp32 [total_q, 16]")
    need = mla_decode_mtp_workspace_size(B, total_q, total_kv, kv_dtype, flags, uni_q_len)
    if workspace is None and need > 0:
        workspace = _stream_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(qo_indptr), int(total_q), int(uni_q_len), int(bool(causal)), _ptr(kv), _ptr(kv_scales),
            _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len), int(page_size), _ptr(out), _ptr(lse), B,
            int(total_kv), int(kv_dtype), float(sm_scale), _ptr(workspace), ws_bytes, int(flags), _stream(q.device))
    return args, workspace


def mla_decode_mtp(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, total_q: int,
                   causal: bool, total_kv: int, kv_dtype: int, uni_q_len: int = 0, kv_last_page_len=None,
                   page_size: int = 1, sm_scale: float = 0.0, workspace=None, flags: int = 0):
    """Enqueue MLA decode with several query tokens per sequence (see include/mla_decode.h,
    mla_decode_mtp). q [total_q,16,576] bf16, qo_indptr [B+1] int32 (may be None when
    uni_q_len > 0), out [total_q,16,512], lse [total_q,16]. Returns the workspace used."""
    args, ws = _mtp_args(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, total_q,
                         uni_q_len, causal, total_kv, kv_dtype, page_size, sm_scale, workspace, flags)
    rc = _lib.mla_decode_mtp(*args)
    if rc != 0:
        raise MlaError(rc, "mla_decode_mtp")
    return ws


def prepare_decode_mtp(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, out, lse=None, *, total_q: int,
                       causal: bool, total_kv: int, kv_dtype: int, uni_q_len: int = 0, kv_last_page_len=None,
                       page_size: int = 1, sm_scale: float = 0.0, workspace=None, flags: int = 0):
    """prepare_decode for mla_decode_mtp: checks once (one checked call), then
    returns a zero-argument callable that enqueues the same call."""
    ws = mla_decode_mtp(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, out, lse, total_q=total_q, causal=causal,
                        total_kv=total_kv, kv_dtype=kv_dtype, uni_q_len=uni_q_len, kv_last_page_len=kv_last_page_len,
                        page_size=page_size, sm_scale=sm_scale, workspace=workspace, flags=flags)
    args, _ = _mtp_args(q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, total_q,
                        uni_q_len, causal, total_kv, kv_dtype, page_size, sm_scale, ws, flags)
    fn = _lib.mla_decode_mtp
    keep = (q, qo_indptr, kv, kv_scales, kv_indptr, kv_indices, kv_last_page_len, out, lse, ws)

    def call():
        rc = fn(*args)
        if rc != 0:
            raise MlaError(rc, "mla_decode_mtp")
        return keep

    return call


def mla_hbm_read_probe(buf):
    """Enqueue the library's streaming read of a device tensor (measurement aid; see
    include/mla_decode.h). Its size in bytes must be a multiple of 16."""
    _need(buf.is_cuda and buf.is_contiguous(), "buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    rc = _lib.mla_hbm_read_probe(_ptr(buf), nbytes, _stream(buf.device))
    if rc != 0:
        raise MlaError(rc, "mla_hbm_read_probe")

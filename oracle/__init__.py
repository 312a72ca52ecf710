"""CPU fp64 oracle for single-token MLA decode -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path (the HIP library and its Python binding) never
imports, links or calls it, and the oracle never touches the HIP library: the
two share no code.

The arithmetic lives in ``mla_oracle.c`` (plain C, fp64, no fast-math); this
module only marshals numpy arrays through ctypes. What the oracle computes is
the plain definition of the operation on the amd-mixed-mla pages (submission
593653, ``_bmm_reference``):

    s_j  = sm_scale * sum_d q[h, d] * x_j[d]          (576 dims, sm_scale = 1/24)
    out  = sum_j softmax(s)_j * x_j[0:512],  lse = logsumexp_j s_j   (natural log)

over the dequantised cache rows x_j = dequant(kv[kv_indices[kv_indptr[b] + j]]).
Decoders follow submission 754939 (``_dq4``, the e8m0 scale loop of ``mla_s1``)
and the e4m3fn format of ``quantize_fp8``.

Parity pins for every function here are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

KV_BF16, KV_FP8, KV_MXFP4 = 0, 1, 2
NUM_HEADS, DQK, DV = 16, 576, 512
SM_SCALE = 1.0 / 24.0  # 1/sqrt(576)

ROUTE_MAIN, ROUTE_BRUTE, ROUTE_SPLIT = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    alt = os.environ.get("MLA_ORACLE_LIB")  # a planted-mistake build (tests only)
    if alt:
        lib = ctypes.CDLL(alt)
    else:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_bf16_value.restype = ctypes.c_float
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    for name in ("oracle_e4m3fn_value", "oracle_e2m1_value", "oracle_e8m0_value"):
        f = getattr(lib, name)
        f.restype = ctypes.c_float
        f.argtypes = [ctypes.c_uint8]
    lib.oracle_dequant_rows.restype = ctypes.c_int
    lib.oracle_dequant_rows.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p]
    lib.oracle_mla_decode.restype = ctypes.c_int
    lib.oracle_mla_decode.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_mla_decode_q8.restype = ctypes.c_int
    lib.oracle_mla_decode_q8.argtypes = [
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_mla_decode_mtp.restype = ctypes.c_int
    lib.oracle_mla_decode_mtp.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_e4m3fn_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
    lib.oracle_quantize_q_fp8.restype = ctypes.c_int
    lib.oracle_quantize_q_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.oracle_expand_pages.restype = ctypes.c_int
    lib.oracle_expand_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
    lib.oracle_mla_decode_paged.restype = ctypes.c_int
    lib.oracle_mla_decode_paged.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p,
    ]
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16_value(bits: int) -> float:
    return float(_load().oracle_bf16_value(bits))


def e4m3fn_value(code: int) -> float:
    return float(_load().oracle_e4m3fn_value(code))


def e2m1_value(nibble: int) -> float:
    return float(_load().oracle_e2m1_value(nibble))


def e8m0_value(code: int) -> float:
    return float(_load().oracle_e8m0_value(code))


def dequant_rows(kv_dtype: int, kv: np.ndarray, scales: np.ndarray | None) -> np.ndarray:
    """Decode every physical row of the cache to float32 [rows, 576]."""
    kv = np.ascontiguousarray(kv)
    rows = kv.shape[0]
    if scales is not None:
        scales = np.ascontiguousarray(scales)
    out = np.empty((rows, DQK), dtype=np.float32)
    rc = _load().oracle_dequant_rows(kv_dtype, _ptr(kv), _ptr(scales), rows, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_dequant_rows: invalid argument")
    return out


def mla_decode(q_bits: np.ndarray, kv_dtype: int, kv: np.ndarray, scales: np.ndarray | None,
               kv_indptr: np.ndarray, kv_indices: np.ndarray, sm_scale: float = SM_SCALE,
               batches=None, route: int = ROUTE_MAIN, nsplit: int = 1, form: int = 0,
               nthreads: int = 0):
    """Reference MLA decode. Returns (out [n,16,512] f64, lse [n,16] f64).

    ``batches`` restricts the computation to those batch ids (sampled parity at
    full size); rows of the result follow that list.
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv = np.ascontiguousarray(kv)
    scales = None if scales is None else np.ascontiguousarray(scales)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    batch = kv_indptr.shape[0] - 1
    if batches is None:
        blist = None
        n = batch
    else:
        blist = np.ascontiguousarray(np.asarray(batches, dtype=np.int32))
        n = blist.shape[0]
    out = np.zeros((n, NUM_HEADS, DV), dtype=np.float64)
    lse = np.zeros((n, NUM_HEADS), dtype=np.float64)
    rc = _load().oracle_mla_decode(
        _ptr(q_bits), kv_dtype, _ptr(kv), _ptr(scales), _ptr(kv_indptr),
        _ptr(kv_indices) if kv_indices.size else None, batch, float(sm_scale),
        _ptr(blist), n, route, nsplit, form, nthreads, _ptr(out), _ptr(lse),
    )
    if rc != 0:
        raise ValueError("oracle_mla_decode: invalid argument")
    return out, lse


def mla_decode_q8(q_codes: np.ndarray, q_scale: float, kv_dtype: int, kv: np.ndarray, scales: np.ndarray | None,
                  kv_indptr: np.ndarray, kv_indices: np.ndarray, sm_scale: float = SM_SCALE, batches=None,
                  route: int = ROUTE_MAIN, nsplit: int = 1, form: int = 0, nthreads: int = 0):
    """Reference MLA decode with an fp8 query: e4m3fn codes [B,16,576] and one
    fp32 scale (query element = binary32 code value * q_scale). Returns
    (out [n,16,512] f64, lse [n,16] f64) as mla_decode."""
    q_codes = np.ascontiguousarray(q_codes, dtype=np.uint8)
    kv = np.ascontiguousarray(kv)
    scales = None if scales is None else np.ascontiguousarray(scales)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    batch = kv_indptr.shape[0] - 1
    if batches is None:
        blist = None
        n = batch
    else:
        blist = np.ascontiguousarray(np.asarray(batches, dtype=np.int32))
        n = blist.shape[0]
    out = np.zeros((n, NUM_HEADS, DV), dtype=np.float64)
    lse = np.zeros((n, NUM_HEADS), dtype=np.float64)
    rc = _load().oracle_mla_decode_q8(
        _ptr(q_codes), float(np.float32(q_scale)), kv_dtype, _ptr(kv), _ptr(scales), _ptr(kv_indptr),
        _ptr(kv_indices) if kv_indices.size else None, batch, float(sm_scale),
        _ptr(blist), n, route, nsplit, form, nthreads, _ptr(out), _ptr(lse),
    )
    if rc != 0:
        raise ValueError("oracle_mla_decode_q8: invalid argument")
    return out, lse


def mla_decode_mtp(q: np.ndarray, qo_indptr: np.ndarray, causal: bool, kv_dtype: int, kv: np.ndarray,
                   scales: np.ndarray | None, kv_indptr: np.ndarray, kv_indices: np.ndarray, sm_scale: float = SM_SCALE,
                   rows=None, route: int = ROUTE_MAIN, nthreads: int = 0):
    """Reference MLA decode with several query tokens per sequence: q bf16 bits
    [total_q, 16, 576], qo_indptr [B+1]; causal as in oracle_mla_decode_mtp.
    Returns (out [n,16,512] f64, lse [n,16] f64) for the listed query rows (all by default)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kv = np.ascontiguousarray(kv)
    scales = None if scales is None else np.ascontiguousarray(scales)
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    batch = kv_indptr.shape[0] - 1
    if rows is None:
        rlist, n = None, int(qo_indptr[batch])
    else:
        rlist = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n = rlist.shape[0]
    out = np.zeros((n, NUM_HEADS, DV), dtype=np.float64)
    lse = np.zeros((n, NUM_HEADS), dtype=np.float64)
    rc = _load().oracle_mla_decode_mtp(
        _ptr(q), _ptr(qo_indptr), int(bool(causal)), kv_dtype, _ptr(kv), _ptr(scales), _ptr(kv_indptr),
        _ptr(kv_indices) if kv_indices.size else None, batch, float(sm_scale), _ptr(rlist), n, route, nthreads,
        _ptr(out), _ptr(lse),
    )
    if rc != 0:
        raise ValueError("oracle_mla_decode_mtp: invalid argument")
    return out, lse


def expand_pages(page_indptr: np.ndarray, page_ids: np.ndarray, last_page_len: np.ndarray | None, page_size: int):
    """Token-level tables of a paged cache (oracle_expand_pages): returns
    (tok_indptr int32 [B+1], tok_rows int32 [T]) with the cache row of every
    token, sequence by sequence, in token order."""
    page_indptr = np.ascontiguousarray(page_indptr, dtype=np.int32)
    page_ids = np.ascontiguousarray(page_ids, dtype=np.int32)
    last = None if last_page_len is None else np.ascontiguousarray(last_page_len, dtype=np.int32)
    batch = page_indptr.shape[0] - 1
    cap = int(page_indptr[batch]) * int(page_size)
    tok_indptr = np.zeros(batch + 1, dtype=np.int32)
    tok_rows = np.zeros(max(cap, 1), dtype=np.int32)
    rc = _load().oracle_expand_pages(_ptr(page_indptr), _ptr(page_ids) if page_ids.size else None, _ptr(last),
                                     int(page_size), batch, _ptr(tok_indptr), _ptr(tok_rows), cap)
    if rc != 0:
        raise ValueError("oracle_expand_pages: invalid argument")
    return tok_indptr, tok_rows[:int(tok_indptr[batch])].copy()


def mla_decode_paged(q_bits: np.ndarray, kv_dtype: int, kv: np.ndarray, scales: np.ndarray | None,
                     page_indptr: np.ndarray, page_ids: np.ndarray, last_page_len: np.ndarray | None,
                     page_size: int, sm_scale: float = SM_SCALE, batches=None, nthreads: int = 0):
    """Reference MLA decode over a paged cache (oracle_mla_decode_paged): the
    oracle expands the pages itself. Returns (out [n,16,512] f64, lse [n,16] f64)."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv = np.ascontiguousarray(kv)
    scales = None if scales is None else np.ascontiguousarray(scales)
    page_indptr = np.ascontiguousarray(page_indptr, dtype=np.int32)
    page_ids = np.ascontiguousarray(page_ids, dtype=np.int32)
    last = None if last_page_len is None else np.ascontiguousarray(last_page_len, dtype=np.int32)
    batch = page_indptr.shape[0] - 1
    if batches is None:
        blist, n = None, batch
    else:
        blist = np.ascontiguousarray(np.asarray(batches, dtype=np.int32))
        n = blist.shape[0]
    out = np.zeros((n, NUM_HEADS, DV), dtype=np.float64)
    lse = np.zeros((n, NUM_HEADS), dtype=np.float64)
    rc = _load().oracle_mla_decode_paged(
        _ptr(q_bits), kv_dtype, _ptr(kv), _ptr(scales), _ptr(page_indptr), _ptr(page_ids) if page_ids.size else None,
        _ptr(last), int(page_size), batch, float(sm_scale), _ptr(blist), n, nthreads, _ptr(out), _ptr(lse),
    )
    if rc != 0:
        raise ValueError("oracle_mla_decode_paged: invalid argument")
    return out, lse


Q_SCALE_STATIC = 0
Q_SCALE_DYNAMIC = 1


def e4m3fn_encode(x: float) -> int:
    """Nearest e4m3fn code of a binary32 value (ties to even)."""
    return int(_load().oracle_e4m3fn_encode(float(np.float32(x))))


def quantize_q_fp8(q_bits: np.ndarray, scale: float | None = None):
    """Per-tensor fp8 quantisation of a bf16 query (bits, any shape).

    scale None: dynamic, scale = max(absmax, 1e-12) / 448 in fp32. Otherwise the
    static fp32 scale. Returns (codes uint8 of q's shape, scale float32 [1])."""
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    codes = np.empty(q_bits.shape, dtype=np.uint8)
    sc = np.array([0.0 if scale is None else scale], dtype=np.float32)
    mode = Q_SCALE_DYNAMIC if scale is None else Q_SCALE_STATIC
    rc = _load().oracle_quantize_q_fp8(_ptr(q_bits), q_bits.size, mode, _ptr(sc), _ptr(codes))
    if rc != 0:
        raise ValueError("oracle_quantize_q_fp8: invalid argument")
    return codes, sc


def max_threads() -> int:
    return int(_load().oracle_max_threads())

"""Seeded synthetic inputs for MLA decode (shared by tests, smoke check and bench).

This module only *produces* inputs: random bf16 queries and cache rows, the
fp8 / MXFP4 encodings of those rows, and the paging arrays. It holds none of
the attention arithmetic and no decoder; both the HIP library and the CPU
oracle consume exactly the codes produced here.

Workload recipe (the pages' leaderboard generator is not available, so these
stand in for it):
  * q ~ N(0, 1) drawn first, then the cache rows ~ N(0, 1), both as float32 from
    numpy's PCG64 ``default_rng(seed)`` and rounded to bf16 (RNE). The pages
    state that q is standard normal (submission 593653, module comment on the
    static Q scale).
  * fp8 cache: one per-tensor fp32 scale = absmax / 448 and codes
    RNE_e4m3fn(clamp(x / scale, +-448)) of the bf16-rounded rows, computed in
    fp32 (submission 754939, ``quantize_fp8``).
  * MXFP4 cache: per token and 32-element block, the OCP MX v1.0 recipe: shared
    exponent floor(log2(absmax)) - 2, e8m0 code = exponent + 127, elements
    rounded to nearest-even on the e2m1 grid and saturated at +-6; an all-zero
    block gets code 127. Two elements per byte, even element in the low nibble
    (submission 754939, V loop of ``mla_s1``).
  * Paging: page size 1, ``kv_indptr`` = prefix sums of the sequence lengths,
    ``kv_indices`` = arange (as on the pages) or a seeded permutation.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

KV_BF16, KV_FP8, KV_MXFP4 = 0, 1, 2
KV_NAMES = {KV_BF16: "bf16", KV_FP8: "fp8", KV_MXFP4: "mxfp4"}
NUM_HEADS, DQK, DV = 16, 576, 512
MX_BLOCK = 32
FP8_MAX = 448.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_fp8_per_tensor(x: np.ndarray):
    """Per-tensor e4m3fn codes and fp32 scale (absmax / 448), fp32 arithmetic."""
    import torch  # torch's CPU float -> float8_e4m3fn cast rounds to nearest-even

    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.float32(max(float(np.max(np.abs(x))), 1e-12))
    scale = np.float32(amax / np.float32(FP8_MAX))
    y = np.clip(x / scale, -FP8_MAX, FP8_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, np.array([scale], dtype=np.float32)


# e2m1 magnitude grid and the nearest-even decision points between neighbours.
# Ties go to the code with an even mantissa bit (codes 0, 2, 4, 6).
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def _round_e2m1_magnitude(a: np.ndarray) -> np.ndarray:
    """Nearest-even e2m1 code (0..7) for non-negative float32 magnitudes, saturating."""
    code = np.zeros(a.shape, dtype=np.uint8)
    # (lower bound, inclusive?) for each code 1..7: value rounds to code k when it
    # is above the midpoint to k-1 (or equal, if k is even).
    mids = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) * 0.5
    for k in range(1, 8):
        m = mids[k - 1]
        if k % 2 == 0:
            code = np.where(a >= m, np.uint8(k), code)
        else:
            code = np.where(a > m, np.uint8(k), code)
    return code


def quantize_mxfp4(x: np.ndarray):
    """OCP MXFP4 codes: packed nibbles [T, 288] uint8 and e8m0 scales [T, 18] uint8."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    blocks = x.reshape(T, DQK // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, e = np.frexp(amax)  # amax = f * 2^e with f in [0.5, 1): floor(log2 amax) = e - 1
    shared = (e.astype(np.int32) - 1) - 2
    shared = np.clip(shared, -127, 127)
    shared = np.where(amax == 0, 0, shared)
    scale_codes = (shared + 127).astype(np.uint8)
    y = blocks / np.ldexp(np.float32(1.0), shared)[..., None].astype(np.float32)
    mag = _round_e2m1_magnitude(np.abs(y).astype(np.float32))
    sign = (np.signbit(y) & (mag > 0)).astype(np.uint8)
    nib = (mag | (sign << 3)).reshape(T, DQK)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scale_codes)


@dataclass
class Case:
    """One MLA decode workload: host arrays in the library's layouts."""

    kv_dtype: int
    q: np.ndarray            # uint16 bf16 bits [B, 16, 576]
    kv: np.ndarray           # bf16 bits [rows, 576] (uint16) | fp8 codes [rows, 576] | fp4 [rows, 288]
    kv_scales: np.ndarray | None  # None | float32 [1] | uint8 [rows, 18]
    kv_indptr: np.ndarray    # int32 [B + 1]
    kv_indices: np.ndarray   # int32 [T]
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def total_kv(self) -> int:
        return int(self.kv_indptr[-1])

    def kv_bytes(self) -> int:
        """Algorithmic cache bytes one decode reads: codes + scales of every referenced token."""
        T = self.total_kv
        per_tok = {KV_BF16: 2 * DQK, KV_FP8: DQK, KV_MXFP4: DQK // 2 + DQK // MX_BLOCK}[self.kv_dtype]
        return T * per_tok + (4 if self.kv_dtype == KV_FP8 else 0)

    def total_bytes(self) -> int:
        """KV + scales + kv_indices + kv_indptr + q + out (bf16) + lse (fp32); a paged
        cache reads one kv_indices entry per page plus kv_last_page_len."""
        B, T = self.batch, self.total_kv
        paged = self.meta.get("paged")
        index_bytes = 4 * T if paged is None else 4 * (int(paged["kv_indptr"][-1]) + B)
        return (self.kv_bytes() + index_bytes + 4 * (B + 1) + 2 * B * NUM_HEADS * DQK
                + 2 * B * NUM_HEADS * DV + 4 * B * NUM_HEADS)


def make_case(batch: int, kv_lens, kv_dtype: int, seed: int, shuffle: bool = False,
              extra_rows: int = 0, pool_rows: int = 0) -> Case:
    """Build a seeded workload.

    kv_lens: an int (uniform length) or a sequence of per-batch lengths.
    shuffle: use a seeded permutation of the physical rows as kv_indices.
    extra_rows: physical rows beyond the ones referenced (never read).
    pool_rows: if > 0 and smaller than the cache, draw and quantise that many
        rows and repeat them to fill the cache (physical rows stay distinct
        in memory; used for the largest shapes, where drawing every row on the
        host would take minutes).
    """
    if np.isscalar(kv_lens):
        lens = np.full(batch, int(kv_lens), dtype=np.int64)
    else:
        lens = np.asarray(kv_lens, dtype=np.int64)
        assert lens.shape == (batch,)
    indptr = np.zeros(batch + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(lens)
    T = int(indptr[-1])
    rows = T + int(extra_rows)
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((batch, NUM_HEADS, DQK), dtype=np.float32))
    drawn = min(rows, pool_rows) if pool_rows > 0 else rows
    kv_f32 = rng.standard_normal((drawn, DQK), dtype=np.float32)
    kv_bits = f32_to_bf16_bits(kv_f32)
    del kv_f32
    if kv_dtype == KV_BF16:
        kv, scales = kv_bits, None
    elif kv_dtype == KV_FP8:
        kv, scales = quantize_fp8_per_tensor(bf16_bits_to_f32(kv_bits))
    elif kv_dtype == KV_MXFP4:
        kv, scales = quantize_mxfp4(bf16_bits_to_f32(kv_bits))
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype}")
    if drawn < rows:  # repeat the pool: row r holds pool row r % drawn
        reps = -(-rows // drawn)
        kv = np.ascontiguousarray(np.tile(kv, (reps, 1))[:rows])
        if kv_dtype == KV_MXFP4:
            scales = np.ascontiguousarray(np.tile(scales, (reps, 1))[:rows])
    if shuffle:
        indices = rng.permutation(rows)[:T].astype(np.int32)
    else:
        indices = np.arange(T, dtype=np.int32)
    return Case(kv_dtype, q, kv, scales, indptr.astype(np.int32), indices,
                meta={"batch": batch, "seed": seed, "shuffle": shuffle, "kv_dtype": KV_NAMES[kv_dtype]})


def make_mtp_query(q_lens, seed: int):
    """Query for several tokens per sequence (multi-token decode): bf16 bits
    [total_q, 16, 576] ~ N(0, 1) and qo_indptr [B + 1] with q_lens[b] query
    tokens in sequence b."""
    lens = np.asarray(q_lens, dtype=np.int64)
    qo = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    qo[1:] = np.cumsum(lens)
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((int(qo[-1]), NUM_HEADS, DQK), dtype=np.float32))
    return q, qo.astype(np.int32)


def make_paged_case(batch: int, kv_lens, kv_dtype: int, page_size: int, seed: int, shuffle: bool = True,
                    extra_pages: int = 0):
    """A seeded workload over a paged cache: each sequence's tokens fill whole
    pages of `page_size` rows except the last one; the physical pages are a
    seeded permutation (or the identity). Returns (case, paged): `paged` holds
    the page table (page-level kv_indptr, kv_indices = page ids, and
    kv_last_page_len); `case` carries the query, the cache of every physical
    page, and the token-level kv_indptr (prefix sums of the lengths). Which
    cache row a token reads is the method's paging rule, so it is not written
    here: case.kv_indices is empty, and the oracle expands the page table
    itself (oracle.expand_pages)."""
    if np.isscalar(kv_lens):
        lens = np.full(batch, int(kv_lens), dtype=np.int64)
    else:
        lens = np.asarray(kv_lens, dtype=np.int64)
        assert lens.shape == (batch,)
    npages = (lens + page_size - 1) // page_size
    page_indptr = np.zeros(batch + 1, dtype=np.int64)
    page_indptr[1:] = np.cumsum(npages)
    total_pages = int(page_indptr[-1])
    phys_pages = total_pages + int(extra_pages)
    base = make_case(batch, 0, kv_dtype, seed, extra_rows=phys_pages * page_size)  # q and every physical row
    rng = np.random.default_rng(seed + 7919)
    page_ids = (rng.permutation(phys_pages)[:total_pages] if shuffle else np.arange(total_pages)).astype(np.int64)
    tok_indptr = np.zeros(batch + 1, dtype=np.int64)
    tok_indptr[1:] = np.cumsum(lens)
    last = np.where(npages > 0, lens - (npages - 1) * page_size, 0)
    paged = {"page_size": page_size, "kv_indptr": page_indptr.astype(np.int32),
             "kv_indices": page_ids.astype(np.int32), "kv_last_page_len": last.astype(np.int32)}
    case = Case(kv_dtype, base.q, base.kv, base.kv_scales, tok_indptr.astype(np.int32), np.zeros(0, np.int32),
                meta={"batch": batch, "seed": seed, "page_size": page_size, "kv_dtype": KV_NAMES[kv_dtype],
                      "paged": paged})
    return case, paged


# The five measured workloads (batch x kv_len, KV format, seed).
WORKLOADS = {
    "bf16_b4_kv1024": dict(batch=4, kv_lens=1024, kv_dtype=KV_BF16, seed=0),
    "fp8_b32_kv1024": dict(batch=32, kv_lens=1024, kv_dtype=KV_FP8, seed=1),
    "fp8_b4_kv8192": dict(batch=4, kv_lens=8192, kv_dtype=KV_FP8, seed=2),
    "fp8_b64_kv8192": dict(batch=64, kv_lens=8192, kv_dtype=KV_FP8, seed=3),
    "mxfp4_b32_kv8192": dict(batch=32, kv_lens=8192, kv_dtype=KV_MXFP4, seed=4),
}


# The pages' full benchmark grid: batch {4, 32, 64, 256} x kv_len {1024, 8192}
# x each KV format (timed by `bench.py --sweep`; caches beyond 64K rows repeat a
# 64K-row seeded pool).
SWEEP_POOL_ROWS = 65536
SWEEP = {
    f"{KV_NAMES[fmt]}_b{b}_kv{L}": dict(batch=b, kv_lens=L, kv_dtype=fmt, seed=100 + 10 * fmt + i,
                                          pool_rows=SWEEP_POOL_ROWS)
    for fmt in (KV_BF16, KV_FP8, KV_MXFP4)
    for i, (b, L) in enumerate((b, L) for b in (4, 32, 64, 256) for L in (1024, 8192))
}


# Paged caches in the pages' configuration for kv >= 8192 (8-row pages).
PAGED = {
    "fp8_b64_kv8192_page8": dict(batch=64, kv_lens=8192, kv_dtype=KV_FP8, page_size=8, seed=3),
    "mxfp4_b32_kv8192_page8": dict(batch=32, kv_lens=8192, kv_dtype=KV_MXFP4, page_size=8, seed=4),
}


def ragged_lens(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded per-sequence lengths, uniform in [lo, hi] (a mixed-length decode batch)."""
    return np.random.default_rng(seed).integers(lo, hi + 1, size=batch)


# Mixed-length batches with the same mean length as the 8192-token shapes:
# lengths uniform in [256, 16128].
RAGGED = {
    "fp8_b64_ragged": dict(batch=64, kv_lens=ragged_lens(64, 256, 16128, 7), kv_dtype=KV_FP8, seed=7,
                           pool_rows=SWEEP_POOL_ROWS),
    "mxfp4_b32_ragged": dict(batch=32, kv_lens=ragged_lens(32, 256, 16128, 8), kv_dtype=KV_MXFP4, seed=8,
                             pool_rows=SWEEP_POOL_ROWS),
}


def make_workload(name: str) -> Case:
    """A named workload; for the paged ones the page-level arrays are in meta['paged']."""
    if name in PAGED:
        c, _ = make_paged_case(**PAGED[name])
    elif name in RAGGED:
        c = make_case(**RAGGED[name])
    else:
        c = make_case(**(WORKLOADS[name] if name in WORKLOADS else SWEEP[name]))
    c.meta["workload"] = name
    return c

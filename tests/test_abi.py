"""Host-side checks of the C ABI (no GPU needed): exports, planner, validation.

Every entry point declared in include/mla_decode.h must be exported by the
built library. Argument validation happens on the host before any device call,
so every error code except MLA_ERR_UNSUPPORTED / MLA_ERR_HIP is reachable here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def mla():
    import mla_decode_02_amd

    return mla_decode_02_amd


@pytest.fixture(scope="module")
def raw_lib(mla):
    return ctypes.CDLL(mla.LIB_PATH)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(mla_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("mla_decode", "mla_decode_rows", "mla_decode_paged", "mla_decode_q8", "mla_decode_mtp", "mla_decode_plan",
              "mla_decode_workspace_size", "mla_decode_q8_workspace_size", "mla_decode_mtp_workspace_size", "mla_decode_mtp_plan",
              "mla_quantize_q8_debug", "mla_dequant_debug", "mla_hbm_read_probe", "mla_decode_noalloc",
              "mla_status_string", "mla_source_digest"):
        assert n in names


def test_library_is_built_from_the_tree_sources(mla, raw_lib):
    """The library records the digest of the sources it was compiled from; the
    loaded one must be the tree's (importing the package refuses any other)."""
    import mla_decode_02_amd.build as build

    f = raw_lib.mla_source_digest
    f.restype = ctypes.c_char_p
    f.argtypes = []
    assert f().decode() == build.source_digest() == mla.mla_source_digest()


def test_phase_stamps_only_in_the_measurement_build(mla, raw_lib):
    """The decode library records no timestamps and does not export the phase
    buffers; the measurement build of the same sources does, with the same digest."""
    import mla_decode_02_amd.build as build

    assert not hasattr(raw_lib, "mla_phase_buffers")
    assert not mla.PHASES and mla.LIB_PATH.endswith("libmla_decode.so")
    ph = ctypes.CDLL(build.PHASES_LIB)
    assert hasattr(ph, "mla_phase_buffers")
    ph.mla_source_digest.restype = ctypes.c_char_p
    assert ph.mla_source_digest().decode() == mla.mla_source_digest()


def test_source_digest_follows_every_source_file(tmp_path, monkeypatch):
    """A change to any one source file (kernel, planner, planner header, C ABI
    header) changes the digest."""
    import mla_decode_02_amd.build as build

    copies = []
    for i, src in enumerate(build.SOURCES):
        dst = tmp_path / f"{i}_{os.path.basename(src)}"
        dst.write_bytes(open(src, "rb").read())
        copies.append(str(dst))
    monkeypatch.setattr(build, "SOURCES", copies)
    base = build.source_digest()
    assert base == build.source_digest()
    for path in copies:
        data = open(path, "rb").read()
        with open(path, "wb") as f:
            f.write(data + b" ")
        assert build.source_digest() != base, path
        with open(path, "wb") as f:
            f.write(data)
    assert build.source_digest() == base


def test_library_exports_every_declared_symbol(raw_lib):
    for name in _declared_functions():
        assert hasattr(raw_lib, name), name


def test_hbm_read_probe_validation(raw_lib):
    """The streaming-read measurement aid checks its arguments on the host (no launch)."""
    f = raw_lib.mla_hbm_read_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, 0, None) == 0           # nothing to read
    assert f(None, 64, None) == -1         # null buffer
    assert f(ctypes.c_void_p(24), 64, None) == -1   # misaligned
    assert f(ctypes.c_void_p(256), 40, None) == -1  # not a multiple of 16


def test_noalloc_refuses_plans_beyond_its_scratch(raw_lib, mla):
    """mla_decode_noalloc refuses a plan whose workspace exceeds its fixed scratch before any
    device call (so this runs without a GPU)."""
    f = raw_lib.mla_decode_noalloc
    f.restype = ctypes.c_int
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_int64, i32, ctypes.c_float, i32, vp]
    A = ctypes.c_void_p(256)
    limit = 32 << 20
    flags = mla.flags_for(splits=2)
    assert mla.mla_decode_workspace_size(1100, 1100 * 2048, 1, flags) > limit
    assert f(A, A, A, A, A, A, None, 1100, 1100 * 2048, 1, 0.0, flags, None) == -3
    assert mla.mla_decode_workspace_size(500, 500 * 2048, 1, flags) <= limit
    assert f(A, A, A, A, A, A, None, 0, 0, 1, 0.0, 0, None) == 0        # empty batch: a no-op
    assert f(A, A, A, A, A, A, None, -1, 0, 1, 0.0, 0, None) == -1      # invalid sizes


def test_status_strings(mla):
    assert mla.mla_status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert mla.mla_status_string(code) not in ("ok", "unknown status")
    assert mla.mla_status_string(-99) == "unknown status"


WORKLOADS = [(4, 1024), (32, 1024), (4, 8192), (64, 8192), (32, 8192), (256, 1024), (256, 8192), (1, 1), (7, 13)]


@pytest.mark.parametrize("B,L", WORKLOADS)
@pytest.mark.parametrize("kv_dtype", [0, 1, 2])
def test_heuristic_plan_invariants(mla, B, L, kv_dtype):
    p = mla.mla_decode_plan(B, B * L, kv_dtype)
    assert p.mode in (0, 1)
    if p.mode == 0:
        assert 1 <= p.num_splits <= 64
        assert p.grid == p.num_splits * B
        # the last-arriving split merges up to 4 splits, or up to 8 on the bf16 and fp8 caches (from bf16
        # partials); more merge in a combine launch
        S = p.num_splits
        merged = S <= 4 or (S <= 8 and kv_dtype != 2)
        assert p.combine == (0 if S == 1 else 2 if merged else 1)
        assert p.num_partials == (p.num_splits * B if p.num_splits > 1 else 0)
    else:
        assert 1 <= p.grid <= 4095 and p.num_partials == p.grid + B - 1 and p.combine == 1
    expect = 0
    if p.num_partials:
        o = p.num_partials * 16 * 512 * 4
        lse = p.num_partials * 16 * 4
        expect = mla.WORKSPACE_COUNTER_BYTES + -(-o // 256) * 256 + -(-lse // 256) * 256
    assert p.workspace_bytes == expect
    assert mla.mla_decode_workspace_size(B, B * L, kv_dtype) == expect


def test_heuristic_fills_the_chip_for_the_measured_shapes(mla):
    # Stage-1 workgroups fit one (bf16) or two (fp8, MXFP4) per compute unit:
    # the grid is a whole number of workgroups per CU, up to that many.
    for fmt, per_cu in [(0, 1), (1, 2), (2, 2)]:
        for B, L in [(32, 1024), (4, 8192), (64, 8192), (32, 8192), (256, 1024)]:
            p = mla.mla_decode_plan(B, B * L, fmt)
            assert p.grid % 256 == 0 and 256 <= p.grid <= 256 * per_cu, (fmt, B, L, p)


def test_short_sequences_take_one_step_per_workgroup(mla):
    # 4 x 1k: one workgroup per compute unit with one 32-token step each beats
    # fewer, longer workgroups (the fill rule alone gives 8 splits)
    for fmt in (0, 1, 2):
        p = mla.mla_decode_plan(4, 4 * 1024, fmt)
        assert (p.mode, p.num_splits, p.grid) == (0, 32, 128), (fmt, p)
    # long sequences keep the fill rule
    assert mla.mla_decode_plan(64, 64 * 8192, 1).num_splits == 8
    assert mla.mla_decode_plan(32, 32 * 8192, 2).num_splits == 16


def test_forced_plans(mla):
    p = mla.mla_decode_plan(4, 4000, 1, mla.flags_for(splits=7))
    assert (p.mode, p.num_splits, p.grid, p.num_partials) == (0, 7, 28, 28)
    p = mla.mla_decode_plan(4, 4000, 1, mla.flags_for(splits=1))
    assert (p.num_splits, p.combine, p.workspace_bytes) == (1, 0, 0)
    p = mla.mla_decode_plan(4, 4000, 2, mla.flags_for(persistent=True, grid=37))
    assert (p.mode, p.grid, p.num_partials, p.combine) == (1, 37, 40, 1)
    p = mla.mla_decode_plan(4, 4000, 2, mla.flags_for(persistent=True))
    assert p.mode == 1 and p.grid == 4000 // 128  # at least 128 tokens per workgroup


def test_mixed_lengths_hint_selects_persistent(mla):
    hint = mla.FLAG_MIXED_LENGTHS
    p = mla.mla_decode_plan(64, 560343, 1, hint)
    assert p.mode == 1 and p.grid == mla.mla_decode_plan(64, 560343, 1, mla.flags_for(persistent=True)).grid
    assert p.num_partials == p.grid + 64 - 1 and p.combine == 1
    # a forced split count or split-K wins over the hint; a tiny batch ignores it
    assert mla.mla_decode_plan(64, 560343, 1, hint | mla.flags_for(splits=8)).mode == 0
    assert mla.mla_decode_plan(64, 560343, 1, hint | mla.FLAG_FORCE_SPLIT).mode == 0
    assert mla.mla_decode_plan(2, 100, 1, hint).mode == 0
    # calls that always plan split-K accept the hint and stay split-K
    assert mla.mla_decode_mtp_workspace_size(32, 64, 32 * 8192, 1, hint) == \
        mla.mla_decode_mtp_workspace_size(32, 64, 32 * 8192, 1, 0)


@pytest.mark.parametrize("args", [
    (-1, 10, 1, 0),            # negative batch
    (2, -1, 1, 0),             # negative total
    (2, 2 ** 31, 1, 0),        # total beyond int32 indices
    (2, 10, 3, 0),             # unknown format
    (2, 10, 1, 0x3),           # both forcing flags
    (2, 10, 1, 1 << 30),       # unknown flag bit
])
def test_plan_rejects_invalid(mla, args):
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_plan(*args)
    assert e.value.status == -1
    assert mla.mla_decode_workspace_size(*args) == 0


def test_empty_batch_plan(mla):
    p = mla.mla_decode_plan(0, 0, 1)
    assert p.grid == 0 and p.workspace_bytes == 0


# ---------------------------------------------------------------- validation


def _call(raw_lib, q=16, kv=16, sc=16, indptr=16, indices=16, out=16, lse=None, batch=2, total=64, dtype=1,
          ws=None, ws_bytes=0, flags=0):
    f = raw_lib.mla_decode
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_float, vp,
                  ctypes.c_size_t, ctypes.c_int, vp]
    return f(q, kv, sc, indptr, indices, out, lse, batch, total, dtype, 0.0, ws, ws_bytes, flags, None)


# Pointers are never dereferenced on the host; validation fails before any use.
A = 0x10000


def test_null_and_misaligned_pointers(raw_lib):
    assert _call(raw_lib, q=None, kv=A, sc=A, indptr=A, indices=A, out=A) == -1
    assert _call(raw_lib, q=A, kv=None, sc=A, indptr=A, indices=A, out=A) == -1
    assert _call(raw_lib, q=A, kv=A, sc=None, indptr=A, indices=A, out=A) == -1       # fp8 needs a scale
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=None, indices=A, out=A) == -1
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=None, out=A) == -1       # total > 0 needs indices
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=None) == -1
    assert _call(raw_lib, q=A + 2, kv=A, sc=A, indptr=A, indices=A, out=A) == -1      # q not 16-byte aligned
    assert _call(raw_lib, q=A, kv=A + 8, sc=A, indptr=A, indices=A, out=A) == -1      # kv not 16-byte aligned
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A + 2, indices=A, out=A) == -1
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=A, lse=A + 1) == -1
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=A, dtype=7) == -1


def test_workspace_too_small(raw_lib, mla):
    need = mla.mla_decode_workspace_size(2, 64, 1, mla.flags_for(splits=4))
    assert need > 0
    f = mla.flags_for(splits=4)
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=A, ws=None, ws_bytes=0, flags=f) == -3
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=A, ws=A, ws_bytes=need - 1, flags=f) == -3
    assert _call(raw_lib, q=A, kv=A, sc=A, indptr=A, indices=A, out=A, ws=A + 4, ws_bytes=need, flags=f) == -1


def _call_paged(raw_lib, last=A, page_size=8, flags=0, batch=2, total=64):
    f = raw_lib.mla_decode_paged
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, vp]
    return f(A, A, A, A, A, last, page_size, A, None, batch, total, 1, 0.0, None, 0, flags, None)


def test_paged_validation(raw_lib, mla):
    assert _call_paged(raw_lib, page_size=0) == -1
    assert _call_paged(raw_lib, page_size=-3) == -1
    assert _call_paged(raw_lib, page_size=(1 << 16) + 1) == -1
    assert _call_paged(raw_lib, last=None) == -1                    # page_size > 1 needs last-page lengths
    assert _call_paged(raw_lib, last=A + 2) == -1                   # misaligned
    assert _call_paged(raw_lib, flags=mla.flags_for(persistent=True)) == -1
    # paged calls plan split-K: without a workspace a multi-split plan reports it
    assert _call_paged(raw_lib, flags=mla.flags_for(splits=4)) == -3
    assert _call_paged(raw_lib, batch=0, total=0) == 0


def _call_q8(raw_lib, q_scale=A, mode=1, page_size=1, last=None, flags=0, batch=2, total=64, ws=None, ws_bytes=0):
    f = raw_lib.mla_decode_q8
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, vp]
    return f(A, q_scale, mode, A, A, A, A, last, page_size, A, None, batch, total, 1, 0.0, ws, ws_bytes, flags, None)


def test_q8_validation(raw_lib, mla):
    assert _call_q8(raw_lib, mode=2) == -1
    assert _call_q8(raw_lib, mode=-1) == -1
    assert _call_q8(raw_lib, q_scale=None) == -1
    assert _call_q8(raw_lib, q_scale=A + 2) == -1
    assert _call_q8(raw_lib, page_size=0) == -1
    assert _call_q8(raw_lib, page_size=8, last=None) == -1
    assert _call_q8(raw_lib, page_size=8, last=A, flags=mla.flags_for(persistent=True)) == -1
    # the dynamic scale needs its partial maxima even when the plan needs no partials
    assert mla.mla_decode_workspace_size(2, 64, 1, mla.flags_for(splits=1)) == 0
    assert _call_q8(raw_lib, flags=mla.flags_for(splits=1)) == -3
    assert _call_q8(raw_lib, mode=0, q_scale=None, batch=0, total=0) == 0


def test_q8_workspace_size(mla):
    for flags in (0, mla.flags_for(splits=1), mla.flags_for(splits=8), mla.flags_for(persistent=True, grid=100)):
        base = mla.mla_decode_workspace_size(32, 32 * 1024, 1, flags)
        assert mla.mla_decode_q8_workspace_size(32, 32 * 1024, 1, flags, mla.Q_SCALE_STATIC) == base
        dyn = mla.mla_decode_q8_workspace_size(32, 32 * 1024, 1, flags, mla.Q_SCALE_DYNAMIC)
        # the partial maxima follow the plan's bytes and never start inside the counter region
        assert dyn - 1024 == max((base + 255) // 256 * 256, mla.WORKSPACE_COUNTER_BYTES)
    assert mla.mla_decode_q8_workspace_size(32, 1024, 1, 0, 7) == 0


def test_q8_dynamic_maxima_stay_out_of_the_counter_region(mla):
    """A plan without split partials needs no workspace of its own; the dynamic scale's
    1 KiB of partial maxima then lies right after the arrival-counter region, so a later
    merging call on the same buffer still finds every counter zero."""
    one = mla.flags_for(splits=1)
    assert mla.mla_decode_workspace_size(4, 4 * 300, 1, one) == 0
    assert mla.mla_decode_q8_workspace_size(4, 4 * 300, 1, one, mla.Q_SCALE_DYNAMIC) == \
        mla.WORKSPACE_COUNTER_BYTES + 1024
    assert mla.mla_decode_q8_workspace_size(4, 4 * 300, 1, one, mla.Q_SCALE_STATIC) == 0


def test_quantize_q8_debug_validation(raw_lib):
    f = raw_lib.mla_quantize_q8_debug
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, vp, vp, ctypes.c_size_t, vp]
    assert f(A, 2, A, 3, A, A, 1024, None) == -1
    assert f(A, -1, A, 0, A, None, 0, None) == -1
    assert f(A + 2, 2, A, 0, A, None, 0, None) == -1
    assert f(A, 2, None, 0, A, None, 0, None) == -1
    assert f(A, 2, A, 1, A, None, 0, None) == -3
    assert f(A, 2, A, 1, A, A, 1023, None) == -3
    assert f(A, 0, None, 0, None, None, 0, None) == 0


def _call_mtp(raw_lib, qo=A, total_q=4, uni=2, causal=1, page_size=1, last=None, flags=0, batch=2, total=64,
              ws=None, ws_bytes=0):
    f = raw_lib.mla_decode_mtp
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp,
                  ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, vp]
    return f(A, qo, total_q, uni, causal, A, A, A, A, last, page_size, A, None, batch, total, 1, 0.0, ws, ws_bytes,
             flags, None)


def test_mtp_validation(raw_lib, mla):
    assert _call_mtp(raw_lib, causal=2) == -1
    assert _call_mtp(raw_lib, uni=3) == -1                          # total_q != batch * uni_q_len
    assert _call_mtp(raw_lib, uni=-1) == -1
    assert _call_mtp(raw_lib, total_q=-1, uni=0) == -1
    assert _call_mtp(raw_lib, uni=0, qo=None) == -1                 # ragged needs qo_indptr
    assert _call_mtp(raw_lib, uni=0, qo=A + 2) == -1
    assert _call_mtp(raw_lib, flags=mla.flags_for(persistent=True)) == -1
    assert _call_mtp(raw_lib, page_size=8, last=None) == -1
    assert _call_mtp(raw_lib, flags=mla.flags_for(splits=4)) == -3  # partials need a workspace
    assert _call_mtp(raw_lib, total_q=0, uni=0, qo=None) == 0       # no query rows: a no-op
    assert _call_mtp(raw_lib, batch=0, total=0, total_q=0, uni=0) == 0


def test_mtp_plan_is_split_over_rows(mla):
    # 32 sequences x 2 query tokens plan like 64 single-token sequences of the same length
    assert mla.mla_decode_mtp_workspace_size(32, 64, 32 * 1024, 1, 0) == \
        mla.mla_decode_workspace_size(64, 64 * 1024, 1, mla.FLAG_FORCE_SPLIT)
    assert mla.mla_decode_mtp_workspace_size(4, 8, 4 * 8192, 1, mla.flags_for(splits=5)) == \
        mla.mla_decode_workspace_size(8, 8 * 8192, 1, mla.flags_for(splits=5))
    assert mla.mla_decode_mtp_workspace_size(4, 8, 4 * 8192, 1, mla.flags_for(persistent=True)) == 0
    # the uniform count changes nothing off the bf16 cache
    for fmt in (1, 2):
        assert mla.mla_decode_mtp_plan(32, 64, 32 * 1024, fmt, 0, 2) == mla.mla_decode_mtp_plan(32, 64, 32 * 1024, fmt)
        assert mla.mla_decode_mtp_plan(32, 64, 32 * 1024, fmt).rows_per_wg == 1


def test_mtp_plan_pairs_rows_on_the_bf16_cache(mla):
    """bf16 cache, uniform count n >= 2: workgroups carry row pairs, planned like batch x ceil(n / 2)
    sequences; partials and counters stay per query row."""
    for n in (2, 3, 4, 5):
        B, L = 16, 1024
        p = mla.mla_decode_mtp_plan(B, B * n, B * L, 0, 0, n)
        pairs = B * ((n + 1) // 2)
        single = mla.mla_decode_plan(pairs, pairs * L, 0, mla.FLAG_FORCE_SPLIT)
        assert p.rows_per_wg == 2 and p.mode == 0
        assert p.num_splits == single.num_splits and p.grid == single.grid == p.num_splits * pairs
        s = p.num_splits
        assert p.num_partials == (s * B * n if s > 1 else 0)
        assert p.combine == (0 if s == 1 else 2 if s <= 4 else 1)
        assert p.workspace_bytes == mla.mla_decode_mtp_workspace_size(B, B * n, B * L, 0, 0, n)
        assert p.workspace_bytes >= (mla.WORKSPACE_COUNTER_BYTES + p.num_partials * 16 * 513 * 4 if s > 1 else 0)
    # the headline shape: 64 x 8192, two tokens -> the single-token plan's grid
    p = mla.mla_decode_mtp_plan(64, 128, 64 * 8192, 0, 0, 2)
    one = mla.mla_decode_plan(64, 64 * 8192, 0)
    assert (p.rows_per_wg, p.num_splits, p.grid, p.combine) == (2, one.num_splits, one.grid, one.combine)
    assert p.num_partials == 2 * one.num_partials
    # one row per workgroup: on request, for one token, and for ragged counts
    assert mla.mla_decode_mtp_plan(16, 32, 16 * 1024, 0, mla.FLAG_ROW_PER_WG, 2).rows_per_wg == 1
    assert mla.mla_decode_mtp_plan(16, 16, 16 * 1024, 0, 0, 1).rows_per_wg == 1
    assert mla.mla_decode_mtp_plan(16, 32, 16 * 1024, 0, 0, 0).rows_per_wg == 1
    # forced splits and the combine launch carry over; a count that does not match is rejected
    p = mla.mla_decode_mtp_plan(3, 9, 3000, 0, mla.flags_for(splits=3) | mla.FLAG_COMBINE_LAUNCH, 3)
    assert (p.rows_per_wg, p.num_splits, p.grid, p.combine, p.num_partials) == (2, 3, 18, 1, 27)
    with pytest.raises(mla.MlaError):
        mla.mla_decode_mtp_plan(3, 10, 3000, 0, 0, 3)
    assert mla.mla_decode_mtp_workspace_size(3, 10, 3000, 0, 0, 3) == 0


def test_batch_zero_is_a_noop(raw_lib):
    assert _call(raw_lib, q=None, kv=None, sc=None, indptr=None, indices=None, out=None, batch=0, total=0) == 0


def test_dequant_debug_validation(raw_lib):
    f = raw_lib.mla_dequant_debug
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int64, ctypes.c_int, vp, vp]
    assert f(5, A, A, 4, 0, A, None) == -1
    assert f(1, A, None, 4, 0, A, None) == -1
    assert f(1, A, A, -1, 0, A, None) == -1
    assert f(1, A, A, 4, 2, A, None) == -1
    assert f(1, A + 8, A, 4, 0, A, None) == -1
    assert f(1, A, A, 0, 0, A, None) == 0


# ---------------------------------------------------------------- persistent partition


def _shares(T, G):
    return [(p * T // G, (p + 1) * T // G) for p in range(G)]


@pytest.mark.parametrize("seed", range(20))
def test_persistent_partition_slots(seed):
    """Workgroup p covers [floor(pT/G), floor((p+1)T/G)); it writes one partial per
    sequence it touches into slot p + b. Slots are unique, below G + B - 1, and the
    combine's owner formula floor(((t + 1) G - 1) / T) names the share holding t."""
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 300, size=B) * (rng.random(B) > 0.2)
    indptr = np.concatenate([[0], np.cumsum(lens)])
    T = int(indptr[-1])
    if T == 0:
        return
    G = int(rng.integers(1, 300))
    slots = set()
    covered = np.zeros(T, dtype=int)
    for p, (g0, g1) in enumerate(_shares(T, G)):
        for b in range(B):
            t0, t1 = max(g0, indptr[b]), min(g1, indptr[b + 1])
            if t0 < t1:
                assert p + b not in slots
                slots.add(p + b)
                covered[t0:t1] += 1
    assert np.all(covered == 1)
    assert max(slots) < G + B - 1 + 1
    for t in range(0, T, max(1, T // 50)):
        p = ((t + 1) * G - 1) // T
        g0, g1 = _shares(T, G)[p]
        assert g0 <= t < g1


@pytest.mark.parametrize("L,S", [(0, 3), (1, 8), (31, 2), (33, 2), (1024, 8), (8192, 64), (100, 7), (5, 64)])
def test_split_ranges_cover_tokens_once(L, S):
    """Split s covers [min(L, s*chunk), min(L, s*chunk + chunk)), chunk = ceil(L/S)
    rounded up to the 32-token wave step."""
    chunk = -(-(-(-L // S)) // 32) * 32 if L else 0
    covered = np.zeros(L, dtype=int)
    for s in range(S):
        t0 = min(L, s * chunk)
        t1 = min(L, t0 + chunk)
        covered[t0:t1] += 1
    assert np.all(covered == 1)


def test_plan_merge_rule(mla):
    """Split-K plans of 2..4 splits merge in the last-arriving split workgroup
    (combine = 2) unless MLA_FLAG_COMBINE_LAUNCH asks for the combine launch, and
    so do 5..8 splits on the bf16 and fp8 caches; more splits, MXFP4 plans of more
    than 4, or more query rows than the counter region holds, use the launch.
    The partials always start after the counter region."""
    for s in range(1, 10):
        p = mla.mla_decode_plan(8, 8 * 4096, 1, mla.flags_for(splits=s))
        assert p.combine == (0 if s == 1 else 2 if s <= 8 else 1)
        m = mla.mla_decode_plan(8, 8 * 4096, 2, mla.flags_for(splits=s))
        assert m.combine == (0 if s == 1 else 2 if s <= 4 else 1)
        q = mla.mla_decode_plan(8, 8 * 4096, 1, mla.flags_for(splits=s) | mla.FLAG_COMBINE_LAUNCH)
        assert q.combine == (0 if s == 1 else 1)
        assert q.workspace_bytes == p.workspace_bytes
        if s > 1:
            assert p.workspace_bytes > mla.WORKSPACE_COUNTER_BYTES + s * 8 * 16 * 512 * 4
    # 5..8 splits merge in stage 1 (bf16 partials) on the bf16 and fp8 caches, short splits included
    for s in range(5, 10):
        for L in (1, 32 * s - 1, 1024 * s, 8192):
            for fmt in (0, 1):
                p = mla.mla_decode_plan(8, 8 * L, fmt, mla.flags_for(splits=s))
                assert p.combine == (2 if s <= 8 else 1), (s, L, fmt)
                f = mla.flags_for(splits=s) | mla.FLAG_COMBINE_LAUNCH
                assert mla.mla_decode_plan(8, 8 * L, fmt, f).combine == 1
    assert mla.mla_decode_plan(64, 64 * 8192, 1, 0).combine == 2  # the 8-split fp8 64 x 8192 plan
    assert mla.mla_decode_plan(8, 8 * 8192, 0, mla.flags_for(splits=8)).combine == 2  # bf16 too
    assert mla.mla_decode_plan(8, 8 * 8192, 2, mla.flags_for(splits=8)).combine == 1  # not MXFP4
    rows = mla.WORKSPACE_COUNTER_BYTES // 4
    assert mla.mla_decode_plan(rows, rows * 64, 1, mla.flags_for(splits=2)).combine == 2
    assert mla.mla_decode_plan(rows + 1, (rows + 1) * 64, 1, mla.flags_for(splits=2)).combine == 1
    # several query tokens: the rows are the query tokens
    assert mla.mla_decode_mtp_workspace_size(4, 16, 4 * 1024, 1, mla.flags_for(splits=3)) == \
        mla.mla_decode_workspace_size(16, 16 * 1024, 1, mla.flags_for(splits=3))


def test_rows_validation(raw_lib):
    """mla_decode_rows rejects a negative cache row count on the host, before any launch."""
    f = raw_lib.mla_decode_rows
    f.restype = ctypes.c_int
    vp = ctypes.c_void_p
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_float, vp, ctypes.c_size_t, ctypes.c_int, vp]
    assert f(A, A, A, A, A, A, None, 2, 64, -1, 1, 0.0, None, 0, 0, None) == -1
    assert f(A, A, A, A, A, A, None, 0, 0, -1, 1, 0.0, None, 0, 0, None) == 0   # batch 0: a no-op, as mla_decode


def test_short_splits_take_one_workgroup_per_cu_merged(mla):
    """Where the plan at two workgroups per CU would need the combine launch, short
    splits on a batch that fills the chip at one workgroup per CU with at most 4
    splits take that plan, merged by the last-arriving split (MXFP4 64 x 1k: 4 merged
    splits, not 8 with the launch). On the bf16 and fp8 caches 8 splits merge in
    stage 1 themselves (fp8 64 x 1k and 32 x 1k: 8 merged). MLA_FLAG_COMBINE_LAUNCH
    keeps the 8-split plan; long splits keep two workgroups per CU (64 x 8k: 8), and
    batches that one workgroup per CU cannot fill within 4 splits keep their plan
    (MXFP4 32 x 1k: 8 with the launch)."""
    p = mla.mla_decode_plan(64, 64 * 1024, 2)
    assert (p.num_splits, p.combine) == (4, 2)
    p = mla.mla_decode_plan(64, 64 * 1024, 2, mla.FLAG_COMBINE_LAUNCH)
    assert (p.num_splits, p.combine) == (8, 1)
    p = mla.mla_decode_plan(64, 64 * 1024, 1)
    assert (p.num_splits, p.combine) == (8, 2)
    p = mla.mla_decode_plan(64, 64 * 1024, 1, mla.FLAG_COMBINE_LAUNCH)
    assert (p.num_splits, p.combine) == (8, 1)
    assert mla.mla_decode_plan(64, 64 * 8192, 1).num_splits == 8
    assert mla.mla_decode_plan(64, 64 * 8192, 2).num_splits == 8
    p = mla.mla_decode_plan(32, 32 * 1024, 1)
    assert (p.num_splits, p.combine) == (8, 2)
    p = mla.mla_decode_plan(32, 32 * 1024, 2)
    assert (p.num_splits, p.combine) == (8, 1)
    p = mla.mla_decode_plan(256, 256 * 1024, 1)
    assert (p.num_splits, p.combine) == (2, 2)

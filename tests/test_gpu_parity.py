"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Tolerances: every output element within 2e-2 absolute + 2e-2 relative of the
oracle and every lse within 1e-3 absolute (the stated acceptance band), plus a
tighter internal gate on the outputs, because the acceptance band alone would
miss a wrong softmax scale. The gate is the worst-case error of the kernel's
arithmetic: the probabilities enter the P.V product rounded to bf16 (relative
error <= 2^-8 each) and the output is rounded to bf16 (<= 2^-8 |out|), so

    |gpu - oracle| <= 2^-8 (sum_j p_j |V_j[d]| + |oracle|) + 1e-4

with p_j the exact softmax weights (computed here in fp64 from the decoded rows
and the oracle's lse) and 1e-4 for the fp32 accumulation.
Decoding is checked bit-exactly against the oracle's decoders.
"""
import math

import numpy as np
import pytest

import synthetic as syn
from helpers import set_one_hot

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL, RTOL, LSE_TOL = 2e-2, 2e-2, 1e-3
U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand)
GATE_SLACK = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def mla(dev):
    import mla_decode_02_amd

    return mla_decode_02_amd


@pytest.fixture(scope="module")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def to_dev(case, dev):
    q = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if case.kv_dtype == syn.KV_BF16:
        kv = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        kv = torch.from_numpy(case.kv).to(dev)
    sc = None if case.kv_scales is None else torch.from_numpy(case.kv_scales).to(dev)
    return dict(q=q, kv=kv, kv_scales=sc, kv_indptr=torch.from_numpy(case.kv_indptr).to(dev),
                kv_indices=torch.from_numpy(case.kv_indices).to(dev))


def new_workspace(mla, case, dev, flags=0, nan_fill=True):
    """Workspace for one plan: arrival counters zeroed (the C ABI requires it) and,
    by default, the partials NaN-filled so that an unwritten partial surfaces as NaN
    (their contents need no initialisation)."""
    plan = mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, flags)
    if not plan.workspace_bytes:
        return None
    return mla.new_workspace(plan.workspace_bytes, dev, poison=nan_fill)


def run_gpu(mla, case, dev, flags=0, sm_scale=0.0, with_lse=True, nan_workspace=True, ws=None):
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev) if with_lse else None
    if ws is None:
        ws = new_workspace(mla, case, dev, flags, nan_fill=nan_workspace)
    mla.mla_decode(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse,
                   total_kv=case.total_kv, kv_dtype=case.kv_dtype, sm_scale=sm_scale, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), (lse.cpu().numpy().astype(np.float64) if with_lse else None)


def check(got, ref, name=""):
    go, gl = got
    ro, rl = ref[0], ref[1]
    assert not np.any(np.isnan(go)), f"{name}: NaN in output"
    err = np.abs(go - ro)
    rms = float(np.sqrt(np.mean(ro ** 2))) if ro.size else 0.0
    print(f"{name}: max |gpu - oracle| {err.max() if err.size else 0.0:.3e}, "
          f"err / rms(out) {(err.max() / rms) if rms > 0 else 0.0:.3e}")
    bad = err > ATOL + RTOL * np.abs(ro)
    assert not np.any(bad), f"{name}: {bad.sum()} outputs outside the band, max err {err.max():.3e}"
    if len(ref) > 2:
        allow = U_BF16 * (ref[2] + np.abs(ro)) + GATE_SLACK
        print(f"{name}: largest |gpu - oracle| / rounding bound {float((err / allow).max()) if err.size else 0.0:.3f}")
        over = err > allow
        if np.any(over):
            i = np.unravel_index(np.argmax(err - allow), err.shape)
            raise AssertionError(f"{name}: {over.sum()} outputs above the rounding bound; worst at {i}: "
                                 f"gpu {go[i]:.6f} oracle {ro[i]:.6f} bound {allow[i]:.2e}")
    if gl is not None:
        fin = np.isfinite(rl)
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl)), f"{name}: -inf lse pattern differs"
        if fin.any():
            lerr = np.abs(gl[fin] - rl[fin]).max()
            assert lerr <= LSE_TOL, f"{name}: lse error {lerr:.3e}"
    return float(err.max())


def weighted_abs_v(orc, case, batches, lse, sm_scale):
    """sum_j p_j |V_j[d]| per (sequence, head, column), p_j = exp(s_j - lse) in fp64."""
    res = np.zeros((len(batches), 16, 512))
    for i, b in enumerate(batches):
        s0, s1 = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        if s1 == s0:
            continue
        rows = case.kv_indices[s0:s1]
        sc = case.kv_scales[rows] if case.kv_dtype == syn.KV_MXFP4 else case.kv_scales
        x = orc.dequant_rows(case.kv_dtype, case.kv[rows], sc).astype(np.float64)
        q = syn.bf16_bits_to_f32(case.q[b]).astype(np.float64)
        p = np.exp((q @ x.T) * sm_scale - lse[i][:, None])
        res[i] = p @ np.abs(x[:, :512])
    return res


def oracle_ref(orc, case, batches=None, sm_scale=1.0 / 24.0):
    """Oracle outputs, lse, and the per-element rounding bound term sum_j p_j |V_j[d]|."""
    o, l = orc.mla_decode(case.q, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                          sm_scale=sm_scale, batches=batches)
    blist = list(range(case.batch)) if batches is None else list(batches)
    return o, l, weighted_abs_v(orc, case, blist, l, sm_scale)


def oracle_tokens(orc, case, paged):
    """The paged workload with the token tables of the oracle's own page expansion
    (oracle.expand_pages); the input generator writes none."""
    import dataclasses

    ti, tr = orc.expand_pages(paged["kv_indptr"], paged["kv_indices"], paged["kv_last_page_len"], paged["page_size"])
    assert np.array_equal(ti, case.kv_indptr), "page table and sequence lengths disagree"
    return dataclasses.replace(case, kv_indptr=ti, kv_indices=tr)


def oracle_ref_paged(orc, case, paged, batches=None, sm_scale=1.0 / 24.0):
    """Oracle outputs and lse of a paged workload through the oracle's paged route (which
    expands the pages itself), with the rounding-bound term over the same tokens."""
    o, l = orc.mla_decode_paged(case.q, case.kv_dtype, case.kv, case.kv_scales, paged["kv_indptr"],
                                paged["kv_indices"], paged["kv_last_page_len"], paged["page_size"],
                                sm_scale=sm_scale, batches=batches)
    blist = list(range(case.batch)) if batches is None else list(batches)
    return o, l, weighted_abs_v(orc, oracle_tokens(orc, case, paged), blist, l, sm_scale)


DTYPES = [syn.KV_BF16, syn.KV_FP8, syn.KV_MXFP4]


# ------------------------------------------------------------------ decode, bit-exact

def _f32_equal(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return nan | (a.view(np.uint32) == b.view(np.uint32))


@pytest.mark.parametrize("path", [0, 1])
def test_dequant_fp8_all_codes_bit_exact(mla, orc, dev, path):
    rng = np.random.default_rng(0)
    rows = 70
    codes = rng.integers(0, 256, size=(rows, 576)).astype(np.uint8)
    codes[0, :256] = np.arange(256, dtype=np.uint8)
    codes[1, 256:512] = np.arange(256, dtype=np.uint8)
    codes[2, 320:576] = np.arange(256, dtype=np.uint8)  # covers the RoPE columns too
    for scale in (1.0, 0.0123456, 7.5):
        s = np.array([scale], np.float32)
        got = mla.mla_dequant_debug(torch.from_numpy(codes).to(dev), torch.from_numpy(s).to(dev), 1, path=path)
        ref = orc.dequant_rows(1, codes, s)
        ok = _f32_equal(got.cpu().numpy(), ref)
        assert ok.all(), f"scale {scale} path {path}: {np.argwhere(~ok)[:5]}"


@pytest.mark.parametrize("path", [0, 1])
def test_dequant_mxfp4_all_code_scale_pairs_bit_exact(mla, orc, dev, path):
    rng = np.random.default_rng(1)
    rows = 256 + 37
    nib = rng.integers(0, 16, size=(rows, 576)).astype(np.uint8)
    nib[:256, 0:16] = np.arange(16, dtype=np.uint8)[None, :]
    nib[:256, 48:64] = np.arange(16, dtype=np.uint8)[None, ::-1]
    nib[:256, 560:576] = np.arange(16, dtype=np.uint8)[None, :]
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0, 256, size=(rows, 18)).astype(np.uint8)
    scales[:256, 0] = np.arange(256, dtype=np.uint8)   # every scale code x every nibble, block 0
    scales[:256, 1] = np.arange(256, dtype=np.uint8)[::-1]
    scales[:256, 17] = np.arange(256, dtype=np.uint8)  # RoPE block
    got = mla.mla_dequant_debug(torch.from_numpy(packed).to(dev), torch.from_numpy(scales).to(dev), 2, path=path)
    ref = orc.dequant_rows(2, packed, scales)
    ok = _f32_equal(got.cpu().numpy(), ref)
    assert ok.all(), f"path {path}: {np.argwhere(~ok)[:5]}"


@pytest.mark.parametrize("path", [0, 1])
def test_dequant_bf16_bit_exact(mla, orc, dev, path):
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 65536, size=(45, 576)).astype(np.uint16)
    kv = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    got = mla.mla_dequant_debug(kv, None, 0, path=path)
    ref = orc.dequant_rows(0, bits, None)
    assert _f32_equal(got.cpu().numpy(), ref).all()


# ------------------------------------------------------------------ attention parity, small sizes

@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_ragged_shuffled_default_plan(mla, orc, dev, kv_dtype):
    lens = [1, 37, 100, 0, 16, 33, 513, 64]
    case = syn.make_case(len(lens), lens, kv_dtype, seed=20 + kv_dtype, shuffle=True, extra_rows=11)
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), "ragged")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("splits", [1, 2, 3, 8, 64])
def test_forced_splits(mla, orc, dev, kv_dtype, splits):
    lens = [300, 7, 1030]
    case = syn.make_case(3, lens, kv_dtype, seed=30 + splits, shuffle=True)
    check(run_gpu(mla, case, dev, flags=mla.flags_for(splits=splits)), oracle_ref(orc, case), f"splits={splits}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("grid", [1, 5, 64, 300])
def test_persistent_grid(mla, orc, dev, kv_dtype, grid):
    lens = [300, 0, 7, 1030, 1, 64]
    case = syn.make_case(len(lens), lens, kv_dtype, seed=40 + grid, shuffle=True)
    check(run_gpu(mla, case, dev, flags=mla.flags_for(persistent=True, grid=grid)), oracle_ref(orc, case),
          f"persistent grid={grid}")


@pytest.mark.parametrize("grid", [97, 512])
def test_persistent_many_sequences(mla, orc, dev, grid):
    """More sequences than a workgroup's threads (the first-sequence count runs over several chunks), with empty
    sequences; shares start inside, at and across sequence boundaries."""
    rng = np.random.default_rng(611)
    lens = rng.integers(0, 60, size=600)
    lens[::7] = 0
    case = syn.make_case(600, lens, syn.KV_FP8, seed=612, shuffle=True)
    got_o, got_l = run_gpu(mla, case, dev, flags=mla.flags_for(persistent=True, grid=grid))
    sample = sorted({0, 1, 7, 299, 300, 301, 511, 598, 599} | set(range(250, 262)))
    check((got_o[sample], got_l[sample]), oracle_ref(orc, case, batches=sample), f"600 sequences grid={grid}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 32, 33, 63, 65, 127, 129, 1000])
def test_lengths_single_sequence(mla, orc, dev, kv_dtype, L):
    case = syn.make_case(1, L, kv_dtype, seed=50 + L, shuffle=True, extra_rows=3)
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), f"L={L}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_long_sequence_several_index_windows(mla, orc, dev, kv_dtype):
    case = syn.make_case(2, [9000, 4500], kv_dtype, seed=60, shuffle=True)
    check(run_gpu(mla, case, dev, flags=mla.flags_for(splits=1)), oracle_ref(orc, case), "one split")
    check(run_gpu(mla, case, dev, flags=mla.flags_for(persistent=True, grid=1)), oracle_ref(orc, case), "grid 1")
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), "default")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("lens,splits", [
    ([256] * 4, 0),       # equal lengths: every split keeps its guessed first index window
    ([256] * 4, 3),
    ([3000] * 2, 1),      # kept first window, the later windows read as usual
    ([0, 600], 0),        # total a multiple of batch but lengths differ: guesses rejected, one range empty
    ([100, 500], 2),
    ([1, 2, 3, 2], 0),    # only the last sequence sits where the guess puts it
])
def test_equal_length_index_guess(mla, orc, dev, kv_dtype, lens, splits):
    """Split-K requests the first index window of sequence b at entry b * total / batch
    before kv_indptr arrives; kept or rejected, the result is the oracle's (shuffled
    rows, so a wrongly kept window would attend the wrong tokens)."""
    case = syn.make_case(len(lens), lens, kv_dtype, seed=71, shuffle=True)
    flags = mla.flags_for(splits=splits) if splits else 0
    check(run_gpu(mla, case, dev, flags), oracle_ref(orc, case), f"lens {lens} splits {splits}")


@pytest.mark.parametrize("kv_dtype", [syn.KV_FP8, syn.KV_MXFP4])
@pytest.mark.parametrize("lens", [[5000, 37, 2600], [33, 64, 95, 1], [4097] * 2])
def test_split_grids_around_one_per_cu(mla, orc, dev, kv_dtype, lens):
    """The same batch under split grids from a few workgroups to just over one per compute
    unit: odd and even step counts, empty and one-step ranges, several index windows."""
    case = syn.make_case(len(lens), lens, kv_dtype, seed=72, shuffle=True)
    ref = oracle_ref(orc, case)
    for splits in (1, 3, 85, 86):  # grids 3..258 workgroups for three sequences
        if splits * case.batch > 512:
            continue
        check(run_gpu(mla, case, dev, mla.flags_for(splits=splits)), ref, f"lens {lens} splits {splits}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_all_sequences_empty(mla, orc, dev, kv_dtype):
    case = syn.make_case(3, [0, 0, 0], kv_dtype, seed=61, extra_rows=4)
    for flags in (0, mla.flags_for(splits=4), mla.flags_for(persistent=True, grid=3)):
        o, l = run_gpu(mla, case, dev, flags=flags)
        assert np.all(o == 0) and np.all(np.isneginf(l))


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_without_lse_and_custom_scale(mla, orc, dev, kv_dtype):
    case = syn.make_case(3, [40, 200, 5], kv_dtype, seed=62, shuffle=True)
    got = run_gpu(mla, case, dev, with_lse=False)
    ref = oracle_ref(orc, case)
    check(got, (ref[0], None, ref[2]), "no lse")
    sc = 1.0 / math.sqrt(512.0)
    check(run_gpu(mla, case, dev, sm_scale=sc), oracle_ref(orc, case, sm_scale=sc), "sm_scale")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_one_hot_scores(mla, orc, dev, kv_dtype):
    """q = 1440 e_col: score 60 for one token, 0 for the others (pins the scale)."""
    for col in (3, 540):
        case = syn.make_case(1, 300, kv_dtype, seed=63, shuffle=True)
        set_one_hot(case, 123, col)
        case.q[:] = 0
        case.q[:, :, col] = 0x44B4
        got = run_gpu(mla, case, dev)
        ref = oracle_ref(orc, case)
        check(got, ref, f"one-hot col {col}")
        assert abs(got[1][0, 0] - 60.0) < 1e-3


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_rope_only_query(mla, orc, dev, kv_dtype):
    case = syn.make_case(2, [77, 300], kv_dtype, seed=64, shuffle=True)
    case.q[:, :, :512] = 0
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), "rope only")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_deterministic(mla, dev, kv_dtype):
    case = syn.make_case(4, [1000, 3000, 5, 700], kv_dtype, seed=65, shuffle=True)
    a = run_gpu(mla, case, dev)
    b = run_gpu(mla, case, dev, nan_workspace=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_workspace_reused_across_calls_and_plans(mla, orc, dev, kv_dtype):
    """One workspace, NaN-filled once, serves a run of calls with different split
    counts, persistent grids and batch sizes in a row (stale partials of an earlier
    call are never read)."""
    big = syn.make_case(5, [900, 40, 2500, 0, 333], kv_dtype, seed=66, shuffle=True)
    small = syn.make_case(2, [129, 64], kv_dtype, seed=67, shuffle=True)
    plans = [(big, mla.flags_for(splits=8)), (big, mla.flags_for(splits=3)), (small, 0),
             (big, mla.flags_for(persistent=True, grid=64)), (small, mla.flags_for(splits=64)), (big, 0),
             (big, mla.flags_for(splits=8))]
    need = max(mla.mla_decode_workspace_size(c.batch, c.total_kv, c.kv_dtype, f) for c, f in plans)
    ws = mla.new_workspace(need, dev, poison=True)
    refs = {id(big): oracle_ref(orc, big), id(small): oracle_ref(orc, small)}
    for i, (c, f) in enumerate(plans):
        check(run_gpu(mla, c, dev, flags=f, ws=ws), refs[id(c)], f"call {i} flags={f:#x}")


def test_large_scores_rescale_path(mla, orc, dev):
    """Scores that grow along the sequence force the running-max rescale repeatedly."""
    case = syn.make_case(1, 2000, syn.KV_BF16, seed=66)
    x = syn.bf16_bits_to_f32(case.kv).copy()
    x[:, 0] = np.linspace(-4, 4, x.shape[0], dtype=np.float32)
    case.kv = syn.f32_to_bf16_bits(x)
    case.q[:, :, 0] = syn.f32_to_bf16_bits(np.full((1, 16), 96.0, np.float32))[0]
    check(run_gpu(mla, case, dev, flags=mla.flags_for(splits=1)), oracle_ref(orc, case), "rescale")


# ------------------------------------------------------------------ full-size workloads, sampled

@pytest.mark.parametrize("name", list(syn.WORKLOADS))
def test_full_size_workload(mla, orc, dev, name):
    """Full-size workloads in the benchmark's launch configuration (default plan), every
    sequence compared with the oracle."""
    case = syn.make_workload(name)
    print(f"{name}: plan {mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, 0)}", flush=True)
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), name)


# The pages' whole shape grid (batch {4, 32, 64, 256} x kv_len {1024, 8192} x format), at
# full size and in the default plan; caches beyond 64K rows repeat a seeded 64K-row pool.
# Every sequence is compared, except on the 256 x 8192 shapes (2M tokens), where 32
# sequences spread over the batch are.
def _sweep_sample(B, L):
    if B * L <= 256 * 1024:
        return None
    return sorted({int(x) for x in np.linspace(0, B - 1, 32)})


@pytest.mark.parametrize("name", list(syn.SWEEP))
def test_sweep_shape(mla, orc, dev, name):
    case = syn.make_workload(name)
    print(f"{name}: plan {mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, 0)}", flush=True)
    got_o, got_l = run_gpu(mla, case, dev, nan_workspace=False)
    sample = _sweep_sample(case.batch, int(case.kv_indptr[1]))
    if sample is None:
        check((got_o, got_l), oracle_ref(orc, case), name)
    else:
        check((got_o[sample], got_l[sample]), oracle_ref(orc, case, batches=sample), name)


@pytest.mark.parametrize("name", list(syn.RAGGED))
@pytest.mark.parametrize("hint", [False, True])
def test_mixed_length_workload_sampled(mla, orc, dev, name, hint):
    """Full-size mixed-length batches, default plan (split-K) and with the mixed-lengths hint (persistent)."""
    case = syn.make_workload(name)
    flags = mla.FLAG_MIXED_LENGTHS if hint else 0
    assert mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, flags).mode == (1 if hint else 0)
    check(run_gpu(mla, case, dev, flags=flags, nan_workspace=False), oracle_ref(orc, case), f"{name} hint={hint}")


# ------------------------------------------------------------------ paged cache

def run_gpu_paged(mla, case, paged, dev, flags=0):
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    ps = paged["page_size"]
    plan_flags = flags | (mla.FLAG_FORCE_SPLIT if ps > 1 else 0)
    need = mla.mla_decode_workspace_size(B, case.total_kv, case.kv_dtype, plan_flags)
    ws = None
    if need:
        ws = mla.new_workspace(need, dev, poison=True)
    mla.mla_decode_paged(t["q"], t["kv"], t["kv_scales"], torch.from_numpy(paged["kv_indptr"]).to(dev),
                         torch.from_numpy(paged["kv_indices"]).to(dev),
                         torch.from_numpy(paged["kv_last_page_len"]).to(dev), out, lse, page_size=ps,
                         total_kv=case.total_kv, kv_dtype=case.kv_dtype, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("page_size", [2, 3, 8, 16, 64])
def test_paged_cache(mla, orc, dev, kv_dtype, page_size):
    """Ragged lengths with partial last pages, an empty sequence, shuffled physical pages."""
    lens = [1, 0, page_size, 3 * page_size + 1, 333, 1030]
    case, paged = syn.make_paged_case(len(lens), lens, kv_dtype, page_size, seed=70 + page_size, extra_pages=5)
    check(run_gpu_paged(mla, case, paged, dev), oracle_ref_paged(orc, case, paged), f"page_size={page_size}")


@pytest.mark.parametrize("splits", [1, 5])
def test_paged_cache_forced_splits(mla, orc, dev, splits):
    lens = [300, 7, 1030]
    case, paged = syn.make_paged_case(3, lens, syn.KV_FP8, 8, seed=80 + splits)
    check(run_gpu_paged(mla, case, paged, dev, flags=mla.flags_for(splits=splits)),
          oracle_ref_paged(orc, case, paged), f"splits={splits}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_page_size_one_is_mla_decode(mla, dev, kv_dtype):
    """Page size 1 through mla_decode_paged gives bitwise the result of mla_decode."""
    case = syn.make_case(4, [1000, 3, 700, 0], kv_dtype, seed=85, shuffle=True)
    paged = {"page_size": 1, "kv_indptr": case.kv_indptr, "kv_indices": case.kv_indices,
             "kv_last_page_len": np.zeros(case.batch, np.int32)}
    a = run_gpu(mla, case, dev)
    b = run_gpu_paged(mla, case, paged, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_paged_equal_length_index_guess(mla, orc, dev, kv_dtype):
    """With equal lengths that are whole pages of a power-of-two size, stage 1 stages
    each split's first page entries before kv_indptr arrives, guessing sequence b's
    pages to start at entry b * Lu / page_size, and expands them into rows once the
    guess is confirmed. Kept (equal lengths; one index window and several), rejected
    (the same total over unequal lengths, an empty sequence among them) and not made
    (a page size that is no power of two; a length that is not whole pages): every
    result within the oracle's bounds, on shuffled physical pages."""
    cases = [("kept", [2048] * 4, 8, 0), ("kept, split", [2048] * 4, 8, 3), ("kept, windows", [4608] * 2, 16, 1),
             ("kept, big pages", [1024] * 3, 64, 0), ("rejected", [128, 0, 192, 192], 8, 0),
             ("rejected, split", [256, 512, 0, 256], 8, 3), ("no power of two", [1200] * 3, 12, 0),
             ("not whole pages", [100] * 4, 8, 0)]
    for name, lens, ps, splits in cases:
        case, paged = syn.make_paged_case(len(lens), lens, kv_dtype, ps, seed=90 + ps + splits, extra_pages=3)
        flags = mla.flags_for(splits=splits) if splits else 0
        check(run_gpu_paged(mla, case, paged, dev, flags=flags), oracle_ref_paged(orc, case, paged),
              f"{name}, page_size={ps}")


@pytest.mark.parametrize("name", list(syn.PAGED))
def test_paged_full_size_page8(mla, orc, dev, name):
    """The pages' paged configuration for kv >= 8192: 8-row pages over shuffled physical
    pages, full size, default split plan, every sequence compared with the oracle's paged
    route."""
    case = syn.make_workload(name)
    paged = case.meta["paged"]
    check(run_gpu_paged(mla, case, paged, dev), oracle_ref_paged(orc, case, paged), name)


# ---------------------------------------------------------------------------
# Split partials merged by the last-arriving split workgroup (plan combine = 2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kv_dtype", [syn.KV_BF16, syn.KV_FP8, syn.KV_MXFP4])
def test_merge_in_stage1_against_oracle_and_combine_launch(mla, orc, dev, kv_dtype):
    """Split counts of the fp32-partial merge (2..4), of the bf16-partial one (5, 8: bf16
    and fp8 caches; MXFP4 takes the combine launch) and one beyond both (9), on ragged,
    shuffled sequences with an empty one and ones shorter than the splits: the
    merged result within the oracle's bounds, the same as the combine launch's
    up to the merge's rounding, and the arrival counters back to zero after each
    call (the next call depends on it)."""
    case = syn.make_case(6, [700, 1, 0, 2048, 33, 515], kv_dtype, seed=91, shuffle=True)
    ref = oracle_ref(orc, case)
    for splits in (2, 3, 4, 5, 8, 9):
        f = mla.flags_for(splits=splits)
        plan = mla.mla_decode_plan(case.batch, case.total_kv, kv_dtype, f)
        assert plan.combine == (2 if splits <= 4 or (splits <= 8 and kv_dtype != syn.KV_MXFP4) else 1)
        ws = new_workspace(mla, case, dev, f)
        a = run_gpu(mla, case, dev, flags=f, ws=ws)
        check(a, ref, f"merge in stage 1, {splits} splits")
        counters = ws[: mla.WORKSPACE_COUNTER_BYTES]
        assert int(torch.count_nonzero(counters)) == 0, "arrival counters not left at zero"
        b = run_gpu(mla, case, dev, flags=f | mla.FLAG_COMBINE_LAUNCH)
        check(b, ref, f"combine launch, {splits} splits")
        assert np.abs(a[0] - b[0]).max() <= 2 * U_BF16 * max(np.abs(b[0]).max(), 1e-3)
        fin = np.isfinite(b[1])
        assert np.array_equal(np.isneginf(a[1]), np.isneginf(b[1]))
        assert np.abs(a[1][fin] - b[1][fin]).max() <= 1e-5


@pytest.mark.parametrize("kv_dtype", [syn.KV_BF16, syn.KV_FP8])
@pytest.mark.parametrize("lens", [[12000, 9000, 0, 12500], [20000, 13000, 3, 0], [700, 33, 1500, 256]])
def test_merge_bf16_partials_5_to_8_splits(mla, orc, dev, kv_dtype, lens):
    """5..8 splits (bf16 and fp8 caches) merge in the last-arriving split from bf16
    partials on the MFMA, all in one round: within the oracle's bounds, the same as
    the combine launch up to the partials' rounding, the counters back at zero, and
    ten queued calls on one workspace bitwise equal. Long and short splits; sequences
    of 3 and 0 tokens leave most or all of their splits empty."""
    case = syn.make_case(4, lens, kv_dtype, seed=95, shuffle=True)
    ref = oracle_ref(orc, case)
    for splits in (5, 6, 7, 8):
        f = mla.flags_for(splits=splits)
        assert mla.mla_decode_plan(case.batch, case.total_kv, kv_dtype, f).combine == 2
        ws = new_workspace(mla, case, dev, f)
        a = run_gpu(mla, case, dev, flags=f, ws=ws)
        check(a, ref, f"bf16-partial merge, {splits} splits")
        assert int(torch.count_nonzero(ws[: mla.WORKSPACE_COUNTER_BYTES])) == 0, "arrival counters not left at zero"
        b = run_gpu(mla, case, dev, flags=f | mla.FLAG_COMBINE_LAUNCH)
        assert np.abs(a[0] - b[0]).max() <= 2 * U_BF16 * max(np.abs(b[0]).max(), 1e-3)
        fin = np.isfinite(b[1])
        assert np.array_equal(np.isneginf(a[1]), np.isneginf(b[1]))
        assert np.abs(a[1][fin] - b[1][fin]).max() <= 1e-5
        for _ in range(10):
            c = run_gpu(mla, case, dev, flags=f, ws=ws)
            assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


@pytest.mark.parametrize("kv_dtype", [syn.KV_FP8, syn.KV_MXFP4])
def test_merge_in_stage1_back_to_back_calls_bitwise(mla, dev, kv_dtype):
    """The merge reads the partials in slot order whichever split arrives last,
    so repeated calls give bitwise-identical results. 40 calls are queued back to
    back on one workspace (each call's counters are reset by its own last
    arrivals before the next call starts), each writing its own output buffers;
    a partial read before it was complete, or a counter left behind, would change
    some bits."""
    case = syn.make_case(48, [1024] * 40 + [300, 7, 0, 4000, 1024, 64, 1025, 2], kv_dtype, seed=92, shuffle=True)
    t = to_dev(case, dev)
    B = case.batch
    f = mla.flags_for(splits=4)
    assert mla.mla_decode_plan(B, case.total_kv, kv_dtype, f).combine == 2
    ws = new_workspace(mla, case, dev, f)
    outs = [torch.empty((B, 16, 512), dtype=torch.bfloat16, device=dev) for _ in range(40)]
    lses = [torch.empty((B, 16), dtype=torch.float32, device=dev) for _ in range(40)]
    for o, l in zip(outs, lses):
        mla.mla_decode(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], o, l,
                       total_kv=case.total_kv, kv_dtype=kv_dtype, workspace=ws, flags=f)
    torch.cuda.synchronize()
    for i in range(1, 40):
        assert torch.equal(outs[i].view(torch.int16), outs[0].view(torch.int16)), f"call {i}: output bits differ"
        assert torch.equal(lses[i].view(torch.int32), lses[0].view(torch.int32)), f"call {i}: lse bits differ"
    assert int(torch.count_nonzero(ws[: mla.WORKSPACE_COUNTER_BYTES])) == 0


def test_mxfp4_split_query_wide_range(mla, orc, dev):
    """On the MXFP4 cache the bf16 query enters the scores as two e4m3fn code sets
    with per-32-element e8m0 scales. Its weak spot is a block whose elements span
    a wide range (the small ones keep fewer bits), so the query here has
    magnitudes 2^-24 .. 2^3 inside every block, all-zero blocks, blocks with one
    nonzero element and a block at the top of the range: the result stays within
    the same bounds as the oracle's exact bf16 query (the acceptance band, the
    rounding gate and lse within 1e-3)."""
    case = syn.make_case(3, [500, 64, 1000], syn.KV_MXFP4, seed=93, shuffle=True)
    rng = np.random.default_rng(94)
    q = rng.standard_normal(case.q.shape).astype(np.float32)
    q *= np.exp2(rng.integers(-24, 4, size=case.q.shape)).astype(np.float32)
    q[0, 0, :32] = 0.0                      # an all-zero block
    q[1, 3, 64:96] = 0.0
    q[1, 3, 70] = 2.5                       # one nonzero element in a block
    q[2, 15, 544:576] = 0.0                 # the last RoPE block: one tiny element
    q[2, 15, 575] = 2.0 ** -20
    q[2, 7, 0:32] = rng.standard_normal(32).astype(np.float32) * 60.0  # large block, scores of order 10
    case.q = syn.f32_to_bf16_bits(q)
    ref = oracle_ref(orc, case)
    check(run_gpu(mla, case, dev), ref, "MXFP4, wide-range query")
    check(run_gpu(mla, case, dev, flags=mla.flags_for(persistent=True, grid=7)), ref, "MXFP4, wide-range query, persistent")


# ---------------------------------------------------------------------------
# Early gathers of the rows a contiguous cache would hold (mla_decode_rows)
# ---------------------------------------------------------------------------
def _run_rows(mla, case, dev, kv_rows, flags=0):
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    mla.mla_decode(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse,
                   total_kv=case.total_kv, kv_dtype=case.kv_dtype, flags=flags, kv_rows=kv_rows)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()


def _with_indices(case, indices, rows=None):
    """The case with kv_indices replaced (and the cache cut to `rows` rows)."""
    import dataclasses
    kv, sc = case.kv, case.kv_scales
    if rows is not None:
        kv = kv[:rows]
        if case.kv_dtype == syn.KV_MXFP4:
            sc = sc[:rows]
    return dataclasses.replace(case, kv=np.ascontiguousarray(kv), kv_scales=sc,
                               kv_indices=np.ascontiguousarray(indices, dtype=np.int32))


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_early_gathers_match_the_plain_call(mla, orc, dev, kv_dtype):
    """With the cache size known, stage 1 requests the rows a contiguous cache
    holds before kv_indices arrives (split plans: with equal lengths, before
    kv_indptr too; the persistent grid: each share's first rows of a sequence),
    and keeps them only where kv_indices agrees. Whatever the indices, the
    result is bit-identical to the call without early requests (kv_rows = 0),
    on split plans and on persistent grids whose shares start inside
    sequences, and within the oracle's bounds:
    contiguous indices (all kept), shuffled (all gathered again), contiguous
    but for a few entries in the first steps of some ranges (only those waves
    gather again), and a cache with fewer rows than tokens (indices repeat;
    guessed rows beyond the cache are clamped below it)."""
    B, L = 6, 700
    base = syn.make_case(B, [L] * B, kv_dtype, seed=95)
    T = base.total_kv
    rng = np.random.default_rng(96)
    contiguous = np.arange(T, dtype=np.int32)
    shuffled = rng.permutation(T).astype(np.int32)
    patched = contiguous.copy()
    for pos in (0, 5, 33, 700 + 17, 3 * 700 + 64, 5 * 700 + 2):
        patched[pos] = int(rng.integers(0, T))
    small = 1000
    repeating = (np.arange(T) % small).astype(np.int32)
    cases = [("contiguous", _with_indices(base, contiguous)), ("shuffled", _with_indices(base, shuffled)),
             ("patched", _with_indices(base, patched)), ("repeating", _with_indices(base, repeating, rows=small))]
    for name, case in cases:
        ref = oracle_ref(orc, case)
        for flags in (0, mla.flags_for(splits=3), mla.flags_for(splits=1),
                      mla.flags_for(persistent=True, grid=5), mla.flags_for(persistent=True, grid=64)):
            early = _run_rows(mla, case, dev, None, flags)
            plain = _run_rows(mla, case, dev, 0, flags)
            assert np.array_equal(early[0], plain[0]), f"{name} flags={flags:#x}: out differs from the plain call"
            assert np.array_equal(early[1], plain[1]), f"{name} flags={flags:#x}: lse differs from the plain call"
        check(run_gpu(mla, case, dev), ref, f"early gathers, {name}")


def test_early_gathers_unequal_lengths(mla, orc, dev):
    """Lengths that differ: the split plan's guessed range is rejected once
    kv_indptr arrives and its early requests are dropped; the persistent grid's
    requests (each share's first rows, contiguous here) are kept. Either way
    the result equals the plain call's."""
    case = syn.make_case(5, [700, 700, 0, 2000, 33], syn.KV_FP8, seed=97)
    case = _with_indices(case, np.arange(case.total_kv, dtype=np.int32))
    for flags in (0, mla.flags_for(persistent=True, grid=7), mla.flags_for(persistent=True, grid=40)):
        a = _run_rows(mla, case, dev, None, flags)
        b = _run_rows(mla, case, dev, 0, flags)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"flags={flags:#x}"
    check(run_gpu(mla, case, dev), oracle_ref(orc, case), "early gathers, unequal lengths")
    with pytest.raises(ValueError):  # a bound beyond the cache tensor is refused before any launch
        _run_rows(mla, case, dev, int(case.kv.shape[0]) + 1)


def test_merge_in_stage1_two_streams(mla, dev):
    """Two streams run merged-split calls at the same time, each on its own
    workspace (the C ABI orders calls that share one): every result equals the
    same call run alone, bit for bit, so concurrent kernels do not disturb each
    other's arrival counters or coherent partials."""
    cases = [syn.make_case(24, [1024] * 20 + [77, 0, 900, 3000], syn.KV_FP8, seed=98, shuffle=True),
             syn.make_case(16, [512] * 16, syn.KV_MXFP4, seed=99)]
    flags = mla.flags_for(splits=3)
    setups = []
    for c in cases:
        t = to_dev(c, dev)
        assert mla.mla_decode_plan(c.batch, c.total_kv, c.kv_dtype, flags).combine == 2
        ws = new_workspace(mla, c, dev, flags)
        ref_o = torch.empty((c.batch, 16, 512), dtype=torch.bfloat16, device=dev)
        ref_l = torch.empty((c.batch, 16), dtype=torch.float32, device=dev)
        mla.mla_decode(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], ref_o, ref_l,
                       total_kv=c.total_kv, kv_dtype=c.kv_dtype, workspace=ws, flags=flags)
        setups.append((c, t, ws, ref_o, ref_l))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    outs = [[], []]
    for _ in range(15):
        for k, (c, t, ws, _, _) in enumerate(setups):
            with torch.cuda.stream(streams[k]):
                o = torch.empty((c.batch, 16, 512), dtype=torch.bfloat16, device=dev)
                l = torch.empty((c.batch, 16), dtype=torch.float32, device=dev)
                mla.mla_decode(t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], o, l,
                               total_kv=c.total_kv, kv_dtype=c.kv_dtype, workspace=ws, flags=flags)
                outs[k].append((o, l))
    torch.cuda.synchronize()
    for k, (c, _, ws, ref_o, ref_l) in enumerate(setups):
        for i, (o, l) in enumerate(outs[k]):
            assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), f"stream {k} call {i}: out differs"
            assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), f"stream {k} call {i}: lse differs"
        assert int(torch.count_nonzero(ws[: mla.WORKSPACE_COUNTER_BYTES])) == 0


# ---------------------------------------------------------------------------
# The mla_decode export itself (the Python binding calls mla_decode_rows)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("flags_kind", ["default", "one", "merged3", "merged8", "combine8", "persistent"])
def test_mla_decode_export_through_ctypes(mla, orc, dev, kv_dtype, flags_kind):
    """mla_decode called through ctypes with raw device pointers, in every merge form,
    against the oracle and bit for bit against the binding's call (mla_decode_rows)."""
    import ctypes

    flags = {"default": 0, "one": mla.flags_for(splits=1), "merged3": mla.flags_for(splits=3),
             "merged8": mla.flags_for(splits=8), "combine8": mla.flags_for(splits=8) | mla.FLAG_COMBINE_LAUNCH,
             "persistent": mla.flags_for(persistent=True, grid=40)}[flags_kind]
    case = syn.make_case(5, [640, 1, 0, 333, 2048], kv_dtype, seed=620 + kv_dtype, shuffle=True, extra_rows=9)
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    ws = new_workspace(mla, case, dev, flags)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_int64, i32, ctypes.c_float, vp,
                               ctypes.c_size_t, i32, vp]
    rc = lib.mla_decode(p(t["q"]), p(t["kv"]), p(t["kv_scales"]), p(t["kv_indptr"]), p(t["kv_indices"]), p(out),
                             p(lse), B, case.total_kv, kv_dtype, ctypes.c_float(0.0), p(ws),
                             0 if ws is None else ws.numel(), flags, stream)
    assert rc == 0, mla.mla_status_string(rc)
    torch.cuda.synchronize()
    got = (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64))
    check(got, oracle_ref(orc, case), f"mla_decode export {flags_kind}")
    again = run_gpu(mla, case, dev, flags=flags)
    assert np.array_equal(got[0], again[0]) and np.array_equal(got[1], again[1])

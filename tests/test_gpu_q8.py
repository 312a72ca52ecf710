"""GPU parity of the fp8-query entry point (mla_decode_q8) against the oracle.

The query codes are a decision taken in binary32 on both sides (one IEEE
division, a clamp, round to nearest even), so the kernel's codes and its
dynamic scale are compared bit-exactly with the oracle's quantiser
(mla_quantize_q8_debug runs the kernels' own routines). The attention is then
compared with the oracle's fp8-query attention under the same bands and the
same internal rounding gate as the bf16-query path: the query enters the score
MFMAs exactly (as codes), so the error analysis is unchanged.
"""
import numpy as np
import pytest

import synthetic as syn
from test_gpu_parity import DTYPES, check, oracle_tokens, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


STATIC_SCALE = 6.0 / 448.0  # the pages' static query scale (absmax 6 over the fp8 maximum)


def _decoded_q(codes, scale):
    c = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    return (c * torch.tensor(np.float32(scale))).to(torch.float64).numpy()


def q8_ref(orc, case, scale=None, batches=None, sm_scale=1.0 / 24.0):
    """Oracle: quantise (static `scale`, or dynamic), attend with the decoded query.
    Returns (out, lse, gate term sum_j p_j |V_j[d]|) and the quantiser's (codes, scale)."""
    codes, sc = orc.quantize_q_fp8(case.q, scale=scale)
    o, l = orc.mla_decode_q8(codes, float(sc[0]), case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr,
                             case.kv_indices, sm_scale=sm_scale, batches=batches)
    blist = list(range(case.batch)) if batches is None else list(batches)
    qd = _decoded_q(codes, sc[0])
    w = np.zeros((len(blist), 16, 512))
    for i, b in enumerate(blist):
        s0, s1 = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        if s1 == s0:
            continue
        rows = case.kv_indices[s0:s1]
        ksc = case.kv_scales[rows] if case.kv_dtype == syn.KV_MXFP4 else case.kv_scales
        x = orc.dequant_rows(case.kv_dtype, case.kv[rows], ksc).astype(np.float64)
        p = np.exp((qd[b] @ x.T) * sm_scale - l[i][:, None])
        w[i] = p @ np.abs(x[:, :512])
    return (o, l, w), (codes, sc)


def run_q8(mla, case, dev, mode, scale=None, flags=0, paged=None, sm_scale=0.0, ws=None):
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    q_scale = torch.tensor([scale if scale is not None else float("nan")], dtype=torch.float32, device=dev)
    ps = 1 if paged is None else paged["page_size"]
    if paged is None:
        indptr, indices, last = t["kv_indptr"], t["kv_indices"], None
    else:
        indptr = torch.from_numpy(paged["kv_indptr"]).to(dev)
        indices = torch.from_numpy(paged["kv_indices"]).to(dev)
        last = torch.from_numpy(paged["kv_last_page_len"]).to(dev)
    if ws is None:
        plan_flags = flags | (mla.FLAG_FORCE_SPLIT if ps > 1 else 0)
        need = mla.mla_decode_q8_workspace_size(B, case.total_kv, case.kv_dtype, plan_flags, mode)
        if need:
            ws = mla.new_workspace(need, dev, poison=True)
    mla.mla_decode_q8(t["q"], q_scale, t["kv"], t["kv_scales"], indptr, indices, out, lse, q_scale_mode=mode,
                      total_kv=case.total_kv, kv_dtype=case.kv_dtype, kv_last_page_len=last, page_size=ps,
                      sm_scale=sm_scale, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            q_scale.cpu().numpy())


# ------------------------------------------------------------------ the quantiser, bit-exact

def _all_finite_bf16_query():
    """Every finite bf16 value, tiled into whole [B, 16, 576] sequences."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(syn.bf16_bits_to_f32(bits))]
    per = 16 * 576
    B = -(-bits.size // per)
    q = np.resize(bits, B * per)
    return q.reshape(B, 16, 576)


# 2^-90 and 2^85 lie outside the range where the kernels use the FMA-corrected
# reciprocal; they take the IEEE division instead.
@pytest.mark.parametrize("scale", [1.0, 0.0133928571, STATIC_SCALE, 3.0e-5, 0.7390851, 2.0 ** -90, 2.0 ** 85])
def test_quantiser_static_all_bf16_values(mla, orc, dev, scale):
    q = _all_finite_bf16_query()
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    sc = torch.tensor([scale], dtype=torch.float32, device=dev)
    got = mla.mla_quantize_q8_debug(qt, sc, mla.Q_SCALE_STATIC).cpu().numpy()
    ref, _ = orc.quantize_q_fp8(q, scale=scale)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, f"{bad.size} codes differ; first: q bits {q.ravel()[bad[0]]:#06x} " \
                          f"gpu {got.ravel()[bad[0]]:#04x} oracle {ref.ravel()[bad[0]]:#04x}"


@pytest.mark.parametrize("B", [1, 5, 300])
def test_quantiser_dynamic_scale_and_codes(mla, orc, dev, B):
    case = syn.make_case(B, [1] * B, syn.KV_BF16, seed=400 + B)
    qt = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(dev)
    sc = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    got = mla.mla_quantize_q8_debug(qt, sc, mla.Q_SCALE_DYNAMIC).cpu().numpy()
    ref, rsc = orc.quantize_q_fp8(case.q)
    assert sc.cpu().numpy()[0] == rsc[0]
    assert np.array_equal(got, ref)


def test_quantiser_dynamic_zero_query(mla, orc, dev):
    qt = torch.zeros((3, 16, 576), dtype=torch.bfloat16, device=dev)
    sc = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    got = mla.mla_quantize_q8_debug(qt, sc, mla.Q_SCALE_DYNAMIC).cpu().numpy()
    _, rsc = orc.quantize_q_fp8(np.zeros((3, 16, 576), np.uint16))
    assert sc.cpu().numpy()[0] == rsc[0] and not got.any()


# ------------------------------------------------------------------ attention with the fp8 query

@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("mode", [0, 1])
def test_q8_ragged_default_plan(mla, orc, dev, kv_dtype, mode):
    case = syn.make_case(5, [1, 77, 0, 300, 1029], kv_dtype, seed=410 + kv_dtype, shuffle=True, extra_rows=11)
    scale = STATIC_SCALE if mode == 0 else None
    ref, (_, rsc) = q8_ref(orc, case, scale=scale)
    go, gl, gsc = run_q8(mla, case, dev, mode, scale=scale)
    check((go, gl), ref, f"q8 mode={mode}")
    if mode == 1:
        assert gsc[0] == rsc[0]


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("splits", [1, 3, 64])
def test_q8_forced_splits(mla, orc, dev, kv_dtype, splits):
    case = syn.make_case(3, [700, 33, 2100], kv_dtype, seed=420 + splits, shuffle=True)
    ref, _ = q8_ref(orc, case)
    go, gl, _ = run_q8(mla, case, dev, 1, flags=mla.flags_for(splits=splits))
    check((go, gl), ref, f"q8 splits={splits}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("grid", [1, 7, 300])
def test_q8_persistent(mla, orc, dev, kv_dtype, grid):
    """Persistent partition, including grids with empty shares (workgroup 0 still publishes the scale)."""
    case = syn.make_case(4, [5, 0, 130, 64], kv_dtype, seed=430 + grid)
    ref, (_, rsc) = q8_ref(orc, case)
    go, gl, gsc = run_q8(mla, case, dev, 1, flags=mla.flags_for(persistent=True, grid=grid))
    check((go, gl), ref, f"q8 persistent grid={grid}")
    assert gsc[0] == rsc[0]


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_paged(mla, orc, dev, kv_dtype):
    lens = [1, 0, 8, 25, 1030]
    case, paged = syn.make_paged_case(len(lens), lens, kv_dtype, 8, seed=440 + kv_dtype, extra_pages=3)
    ref, _ = q8_ref(orc, oracle_tokens(orc, case, paged), scale=STATIC_SCALE)  # the oracle expands the pages
    go, gl, _ = run_q8(mla, case, dev, 0, scale=STATIC_SCALE, paged=paged)
    check((go, gl), ref, "q8 paged")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_custom_sm_scale_and_clamped_query(mla, orc, dev, kv_dtype):
    """A static scale small enough that part of the query saturates at +-448."""
    case = syn.make_case(2, [200, 41], kv_dtype, seed=450 + kv_dtype)
    scale, sm = 1.0 / 256.0, 0.03
    ref, (codes, _) = q8_ref(orc, case, scale=scale, sm_scale=sm)
    assert ((codes & 0x7F) == 0x7E).any()
    go, gl, _ = run_q8(mla, case, dev, 0, scale=scale, sm_scale=sm)
    check((go, gl), ref, "q8 clamped")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_static_equals_dynamic_with_the_same_scale(mla, orc, dev, kv_dtype):
    case = syn.make_case(3, [500, 12, 90], kv_dtype, seed=460 + kv_dtype)
    _, rsc = orc.quantize_q_fp8(case.q)
    a = run_q8(mla, case, dev, 1)
    b = run_q8(mla, case, dev, 0, scale=float(rsc[0]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["fp8_b32_kv1024", "fp8_b64_kv8192", "mxfp4_b32_kv8192", "bf16_b4_kv1024"])
def test_q8_full_size_sampled(mla, orc, dev, name):
    """Full-size workloads, default plan, dynamic scale; the oracle computes a sample of sequences
    (the dynamic scale is over the whole query, as on the GPU)."""
    case = syn.make_workload(name)
    go, gl, gsc = run_q8(mla, case, dev, 1)
    B = case.batch
    sample = sorted({0, B - 1, B // 2})
    ref, (_, rsc) = q8_ref(orc, case, batches=sample)
    assert gsc[0] == rsc[0]
    check((go[sample], gl[sample]), ref, f"q8 {name}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_scale_outside_fast_range_through_attention(mla, orc, dev, kv_dtype):
    """A static scale of 2^-90 takes the kernels' IEEE-division fallback inside stage 1; the query saturates."""
    case = syn.make_case(2, [150, 33], kv_dtype, seed=470 + kv_dtype)
    scale = 2.0 ** -90
    ref, (codes, _) = q8_ref(orc, case, scale=scale, sm_scale=2.0 ** 80)
    assert ((codes & 0x7F) == 0x7E).mean() > 0.9
    go, gl, _ = run_q8(mla, case, dev, 0, scale=scale, sm_scale=2.0 ** 80)
    check((go, gl), ref, "q8 slow division")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_prepared_q8_call_matches_direct_call(mla, dev, kv_dtype):
    """prepare_decode_q8 (the benchmark's marshalled call) gives bitwise the direct call's result."""
    case = syn.make_case(3, [700, 20, 1500], kv_dtype, seed=480 + kv_dtype)
    t = to_dev(case, dev)
    outs = []
    for prepared in (False, True):
        out = torch.empty((3, 16, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((3, 16), dtype=torch.float32, device=dev)
        qs = torch.empty(1, dtype=torch.float32, device=dev)
        kw = dict(q_scale_mode=mla.Q_SCALE_DYNAMIC, total_kv=case.total_kv, kv_dtype=kv_dtype)
        args = (t["q"], qs, t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse)
        if prepared:
            call = mla.prepare_decode_q8(*args, **kw)
            out.fill_(float("nan"))
            call()
        else:
            mla.mla_decode_q8(*args, **kw)
        torch.cuda.synchronize()
        outs.append((out.float().cpu().numpy(), lse.cpu().numpy(), qs.item()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert outs[0][2] == outs[1][2]


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_dynamic_single_split_then_merged_call_on_one_workspace(mla, orc, dev, kv_dtype):
    """A dynamic-scale call whose plan has one split (no partials) writes its partial
    maxima after the arrival-counter region: a merging call (3 splits) on the same
    workspace afterwards finds every counter zero, merges, and leaves them zero."""
    case = syn.make_case(4, [300, 45, 0, 260], kv_dtype, seed=470 + kv_dtype, shuffle=True)
    one, three = mla.flags_for(splits=1), mla.flags_for(splits=3)
    assert mla.mla_decode_plan(4, case.total_kv, kv_dtype, three).combine == 2
    need = max(mla.mla_decode_q8_workspace_size(4, case.total_kv, kv_dtype, f, mla.Q_SCALE_DYNAMIC)
               for f in (one, three))
    ws = mla.new_workspace(need, dev, poison=True)
    ref, (_, rsc) = q8_ref(orc, case)
    for flags in (one, three, one, three):
        go, gl, gsc = run_q8(mla, case, dev, 1, flags=flags, ws=ws)
        check((go, gl), ref, f"q8 dynamic flags={flags:#x}")
        assert gsc[0] == rsc[0]
        counters = ws[:mla.WORKSPACE_COUNTER_BYTES].view(torch.int32)
        assert int(torch.count_nonzero(counters)) == 0, "arrival counters left non-zero"

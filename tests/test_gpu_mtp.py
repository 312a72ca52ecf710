"""GPU parity of mla_decode_mtp (several query tokens per sequence) against the oracle.

Same bands and internal rounding gate as the single-token path: each query row is
an independent softmax over the cache tokens it sees (all of its sequence, or the
causal prefix), so the error analysis per row is unchanged.
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


def mtp_ref(orc, case, q, qo, causal, rows=None, sm_scale=1.0 / 24.0):
    """Oracle rows plus the gate term sum_j p_j |V_j[d]| over the tokens each row sees."""
    o, l = orc.mla_decode_mtp(q, qo, causal, case.kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                              sm_scale=sm_scale, rows=rows)
    rlist = list(range(int(qo[-1]))) if rows is None else list(rows)
    w = np.zeros((len(rlist), 16, 512))
    for i, r in enumerate(rlist):
        b = int(np.searchsorted(qo, r, side="right")) - 1
        n, t = int(qo[b + 1] - qo[b]), r - int(qo[b])
        s0, s1 = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        vis = (s1 - s0) - n + 1 + t if causal else s1 - s0
        vis = max(0, min(s1 - s0, vis))
        if vis == 0:
            continue
        idx = case.kv_indices[s0:s0 + vis]
        ksc = case.kv_scales[idx] if case.kv_dtype == syn.KV_MXFP4 else case.kv_scales
        x = orc.dequant_rows(case.kv_dtype, case.kv[idx], ksc).astype(np.float64)
        qr = syn.bf16_bits_to_f32(q[r]).astype(np.float64)
        p = np.exp((qr @ x.T) * sm_scale - l[i][:, None])
        w[i] = p @ np.abs(x[:, :512])
    return o, l, w


def run_mtp(mla, case, q, qo, dev, causal, uni=0, flags=0, paged=None, ws_nan=True):
    t = to_dev(case, dev)
    TQ = q.shape[0]
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.full((TQ, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((TQ, 16), float("nan"), dtype=torch.float32, device=dev)
    qo_t = None if uni else torch.from_numpy(qo).to(dev)
    ps = 1 if paged is None else paged["page_size"]
    if paged is None:
        indptr, indices, last = t["kv_indptr"], t["kv_indices"], None
    else:
        indptr = torch.from_numpy(paged["kv_indptr"]).to(dev)
        indices = torch.from_numpy(paged["kv_indices"]).to(dev)
        last = torch.from_numpy(paged["kv_last_page_len"]).to(dev)
    need = mla.mla_decode_mtp_workspace_size(case.batch, TQ, case.total_kv, case.kv_dtype, flags, uni)
    ws = None
    if need:
        ws = mla.new_workspace(need, dev, poison=ws_nan)
    mla.mla_decode_mtp(qt, qo_t, t["kv"], t["kv_scales"], indptr, indices, out, lse, total_q=TQ, causal=causal,
                       total_kv=case.total_kv, kv_dtype=case.kv_dtype, uni_q_len=uni, kv_last_page_len=last,
                       page_size=ps, workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
def test_mtp_ragged(mla, orc, dev, kv_dtype, causal):
    """Ragged query counts, an empty sequence, and a sequence shorter than its query count."""
    lens = [40, 0, 2, 700, 1029]
    qlens = [3, 2, 3, 1, 4]
    case = syn.make_case(5, lens, kv_dtype, seed=500 + kv_dtype, shuffle=True, extra_rows=7)
    q, qo = syn.make_mtp_query(qlens, seed=510 + kv_dtype)
    check(run_mtp(mla, case, q, qo, dev, causal), mtp_ref(orc, case, q, qo, causal), f"mtp causal={causal}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("qlen", [2, 4])
def test_mtp_uniform(mla, orc, dev, kv_dtype, qlen):
    case = syn.make_case(3, [300, 64, 1100], kv_dtype, seed=520 + qlen)
    q, qo = syn.make_mtp_query([qlen] * 3, seed=530 + qlen)
    check(run_mtp(mla, case, q, qo, dev, True, uni=qlen), mtp_ref(orc, case, q, qo, True), f"mtp uni={qlen}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_mtp_uniform_equals_ragged_indptr(mla, dev, kv_dtype):
    """The same uniform query counts given as uni_q_len or through qo_indptr give identical results
    (one query row per workgroup in both: on the bf16 cache the uniform call would pair rows)."""
    case = syn.make_case(4, [100, 33, 512, 7], kv_dtype, seed=540)
    q, qo = syn.make_mtp_query([3] * 4, seed=541)
    a = run_mtp(mla, case, q, qo, dev, True, uni=3, flags=mla.FLAG_ROW_PER_WG)
    b = run_mtp(mla, case, q, qo, dev, True, uni=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_mtp_single_token_is_mla_decode(mla, dev, kv_dtype):
    """One query token per sequence: bitwise the result of mla_decode with the same split plan."""
    from test_gpu_parity import run_gpu

    case = syn.make_case(4, [1000, 3, 700, 0], kv_dtype, seed=550, shuffle=True)
    qo = np.arange(5, dtype=np.int32)
    f = mla.flags_for(splits=4)
    a = run_gpu(mla, case, dev, flags=f)
    b = run_mtp(mla, case, case.q, qo, dev, True, uni=1, flags=f)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("splits", [1, 3, 64])
def test_mtp_forced_splits(mla, orc, dev, splits):
    case = syn.make_case(2, [900, 130], syn.KV_FP8, seed=560 + splits)
    q, qo = syn.make_mtp_query([2, 3], seed=561)
    check(run_mtp(mla, case, q, qo, dev, True, flags=mla.flags_for(splits=splits)),
          mtp_ref(orc, case, q, qo, True), f"mtp splits={splits}")


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_mtp_paged(mla, orc, dev, kv_dtype):
    lens = [17, 8, 300]
    case, paged = syn.make_paged_case(3, lens, kv_dtype, 8, seed=570 + kv_dtype, extra_pages=2)
    q, qo = syn.make_mtp_query([2, 4, 3], seed=571)
    # reference over the oracle's own expansion of the page table
    check(run_mtp(mla, case, q, qo, dev, True, paged=paged), mtp_ref(orc, oracle_tokens(orc, case, paged), q, qo, True),
          "mtp paged")


def test_mtp_many_sequences_ragged(mla, orc, dev):
    """More sequences than one workgroup's threads: the row-to-sequence count runs over several chunks."""
    rng = np.random.default_rng(580)
    B = 600
    lens = rng.integers(0, 40, size=B)
    qlens = rng.integers(0, 4, size=B)
    case = syn.make_case(B, lens, syn.KV_FP8, seed=581)
    q, qo = syn.make_mtp_query(qlens, seed=582)
    go, gl = run_mtp(mla, case, q, qo, dev, True)
    TQ = q.shape[0]
    sample = sorted({0, 1, TQ // 3, TQ // 2, TQ - 2, TQ - 1} | set(range(int(qo[B // 2]), int(qo[B // 2 + 2]))))
    check((go[sample], gl[sample]), mtp_ref(orc, case, q, qo, True, rows=sample), "mtp 600 sequences")


@pytest.mark.parametrize("name,qlen", [("fp8_b32_kv1024", 2), ("fp8_b64_kv8192", 2), ("mxfp4_b32_kv8192", 4)])
def test_mtp_full_size_sampled(mla, orc, dev, name, qlen):
    """Full-size caches with qlen causal query tokens per sequence, default plan; sampled rows."""
    case = syn.make_workload(name)
    q, qo = syn.make_mtp_query([qlen] * case.batch, seed=590 + qlen)
    go, gl = run_mtp(mla, case, q, qo, dev, True, uni=qlen, ws_nan=False)
    TQ = q.shape[0]
    sample = sorted({0, 1, qlen - 1, TQ // 2, TQ - qlen, TQ - 1})
    check((go[sample], gl[sample]), mtp_ref(orc, case, q, qo, True, rows=sample), f"mtp {name} q{qlen}")


def test_prepared_mtp_call_matches_direct_call(mla, dev):
    """prepare_decode_mtp (the benchmark's marshalled call) gives bitwise the direct call's result."""
    case = syn.make_case(3, [700, 20, 1500], syn.KV_FP8, seed=595)
    q, qo = syn.make_mtp_query([2, 2, 2], seed=596)
    t = to_dev(case, dev)
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    outs = []
    for prepared in (False, True):
        out = torch.empty((6, 16, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((6, 16), dtype=torch.float32, device=dev)
        kw = dict(total_q=6, causal=True, total_kv=case.total_kv, kv_dtype=syn.KV_FP8, uni_q_len=2)
        args = (qt, None, t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse)
        if prepared:
            call = mla.prepare_decode_mtp(*args, **kw)
            out.fill_(float("nan"))
            call()
        else:
            mla.mla_decode_mtp(*args, **kw)
        torch.cuda.synchronize()
        outs.append((out.float().cpu().numpy(), lse.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_mtp_one_token_ragged_indptr_matches_uniform(mla, dev, kv_dtype):
    """One query token per sequence through a ragged qo_indptr equals the uniform count of one."""
    case = syn.make_case(5, [33, 0, 900, 64, 2], kv_dtype, seed=597)
    qo = np.arange(6, dtype=np.int32)
    a = run_mtp(mla, case, case.q, qo, dev, True, uni=1)
    b = run_mtp(mla, case, case.q, qo, dev, False, uni=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- two query rows per workgroup (bf16 cache, uniform query count >= 2) ----

@pytest.mark.parametrize("qlen", [2, 3, 4, 5])
@pytest.mark.parametrize("causal", [False, True])
def test_mtp_pairs(mla, orc, dev, qlen, causal):
    """Row pairs on the bf16 cache: odd counts (a last row alone), sequences shorter than the
    query count (the earlier row of a pair sees nothing), an empty sequence, ragged cache lengths
    across tile and step boundaries."""
    lens = [300, 0, 1, 2, 64, 1100, 33]
    case = syn.make_case(len(lens), lens, syn.KV_BF16, seed=600 + qlen, shuffle=True, extra_rows=5)
    q, qo = syn.make_mtp_query([qlen] * len(lens), seed=610 + qlen)
    assert mla.mla_decode_mtp_plan(case.batch, q.shape[0], case.total_kv, syn.KV_BF16, 0, qlen).rows_per_wg == 2
    check(run_mtp(mla, case, q, qo, dev, causal, uni=qlen), mtp_ref(orc, case, q, qo, causal),
          f"mtp pairs q{qlen} causal={causal}")


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 8, 64])
def test_mtp_pairs_forced_splits(mla, orc, dev, splits):
    """Every merge form: one split (final rows), 2-4 splits (merged per row by the last-arriving
    split workgroup), more (combine launch); splits past a short sequence's end are empty."""
    case = syn.make_case(3, [900, 130, 5], syn.KV_BF16, seed=620 + splits)
    q, qo = syn.make_mtp_query([3] * 3, seed=621)
    f = mla.flags_for(splits=splits)
    p = mla.mla_decode_mtp_plan(3, 9, case.total_kv, syn.KV_BF16, f, 3)
    assert p.rows_per_wg == 2 and p.num_splits == splits and p.grid == splits * 3 * 2
    check(run_mtp(mla, case, q, qo, dev, True, uni=3, flags=f), mtp_ref(orc, case, q, qo, True),
          f"mtp pairs splits={splits}")


def test_mtp_pairs_combine_launch(mla, orc, dev):
    """Two to four splits merged by the combine launch instead of in stage 1."""
    case = syn.make_case(2, [700, 260], syn.KV_BF16, seed=630)
    q, qo = syn.make_mtp_query([2, 2], seed=631)
    f = mla.flags_for(splits=3) | mla.FLAG_COMBINE_LAUNCH
    assert mla.mla_decode_mtp_plan(2, 4, case.total_kv, syn.KV_BF16, f, 2).combine == 1
    check(run_mtp(mla, case, q, qo, dev, True, uni=2, flags=f), mtp_ref(orc, case, q, qo, True), "mtp pairs combine")


def test_mtp_pairs_paged(mla, orc, dev):
    lens = [17, 8, 300, 1]
    case, paged = syn.make_paged_case(4, lens, syn.KV_BF16, 8, seed=640, extra_pages=2)
    q, qo = syn.make_mtp_query([3] * 4, seed=641)
    check(run_mtp(mla, case, q, qo, dev, True, uni=3, paged=paged),
          mtp_ref(orc, oracle_tokens(orc, case, paged), q, qo, True), "mtp pairs paged")


def test_mtp_pairs_repeated_calls_bitwise(mla, dev):
    """Queued calls on one workspace (the stage-1 merge's counters reused) are bit-identical."""
    case = syn.make_case(4, [600, 90, 1000, 3], syn.KV_BF16, seed=650)
    q, qo = syn.make_mtp_query([2] * 4, seed=651)
    f = mla.flags_for(splits=4)
    assert mla.mla_decode_mtp_plan(4, 8, case.total_kv, syn.KV_BF16, f, 2).combine == 2
    ref = run_mtp(mla, case, q, qo, dev, True, uni=2, flags=f)
    t = to_dev(case, dev)
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    ws = mla.new_workspace(mla.mla_decode_mtp_workspace_size(4, 8, case.total_kv, syn.KV_BF16, f, 2), dev)
    outs = []
    for _ in range(20):
        out = torch.empty((8, 16, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((8, 16), dtype=torch.float32, device=dev)
        mla.mla_decode_mtp(qt, None, t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse, total_q=8,
                           causal=True, total_kv=case.total_kv, kv_dtype=syn.KV_BF16, uni_q_len=2, workspace=ws,
                           flags=f)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert int(ws[:mla.WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0
    for out, lse in outs:
        assert np.array_equal(out.float().cpu().numpy(), ref[0]) and np.array_equal(lse.cpu().numpy(), ref[1])


def test_mtp_pairs_full_size_sampled(mla, orc, dev):
    """bf16 64 x 8192 with two causal query tokens per sequence, default plan (row pairs);
    rows sampled across the batch."""
    case = syn.make_workload("bf16_b64_kv8192")
    q, qo = syn.make_mtp_query([2] * case.batch, seed=660)
    assert mla.mla_decode_mtp_plan(case.batch, q.shape[0], case.total_kv, syn.KV_BF16, 0, 2).rows_per_wg == 2
    go, gl = run_mtp(mla, case, q, qo, dev, True, uni=2, ws_nan=False)
    TQ = q.shape[0]
    sample = sorted({0, 1, 2, 63, 64, TQ // 2 + 1, TQ - 2, TQ - 1})
    check((go[sample], gl[sample]), mtp_ref(orc, case, q, qo, True, rows=sample), "mtp pairs bf16 64x8192 q2")

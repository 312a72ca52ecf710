"""Pins for the CPU oracle: each check ties it to something other than itself.

- decoders: exhaustive against torch's own CPU dtype conversions (float8_e4m3fn,
  float8_e8m0fnu) and the OCP e2m1 table (tests/golden);
- attention core: torch fp64 scaled_dot_product_attention (a library special
  case), naive brute force, closed forms (uniform scores, one token, one-hot),
  invariants (probabilities sum to 1, gather permutation, duplicate tokens);
- split + combine: all three merge forms against the single pass.

A plausible mistake in the oracle -- a dropped RoPE term, a wrong scale, a wrong
V slice, a transposed nibble order, a wrong log base -- fails at least one test
here (tests/test_oracle_mutations.py plants such mistakes and checks that).
"""
import math
import os

import numpy as np
import pytest
import torch

import synthetic as syn
from helpers import set_one_hot as _set_one_hot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 16), float(b)))
    return rows


def _same_f32(a, b):
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(both_nan | (a.view(np.uint32) == b.view(np.uint32))))


# --------------------------------------------------------------------------- decoders


def test_e4m3fn_exhaustive_vs_torch(oracle_mod):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle_mod.e4m3fn_value(c) for c in range(256)], dtype=np.float32)
    assert _same_f32(got, ref)


def test_e4m3fn_golden_points(oracle_mod):
    for code, val in _read_table("e4m3fn_points.txt"):
        got = oracle_mod.e4m3fn_value(code)
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e8m0_exhaustive_vs_torch(oracle_mod):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    got = np.array([oracle_mod.e8m0_value(c) for c in range(256)], dtype=np.float32)
    assert _same_f32(got, ref)
    assert oracle_mod.e8m0_value(127) == 1.0


def test_e2m1_table(oracle_mod):
    table = _read_table("e2m1_table.txt")
    assert len(table) == 16
    for nib, val in table:
        got = oracle_mod.e2m1_value(nib)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(nib)


def _e2m1_ref():
    return np.array([v for _, v in _read_table("e2m1_table.txt")], dtype=np.float32)


def test_mxfp4_rows_all_code_scale_pairs(oracle_mod):
    """Every (nibble, e8m0) pair, both nibble positions, every scale column."""
    e2m1 = _e2m1_ref()
    e8m0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    rng = np.random.default_rng(7)
    rows = 256
    nib = rng.integers(0, 16, size=(rows, 576)).astype(np.uint8)
    # make sure every nibble value meets every scale code in both nibble positions
    nib[:, 0:16] = np.arange(16, dtype=np.uint8)[None, :]
    nib[:, 16:32] = np.arange(16, dtype=np.uint8)[::-1][None, :]
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(0, 256, size=(rows, 18)).astype(np.uint8)
    scales[:, 0] = np.arange(256, dtype=np.uint8)
    got = oracle_mod.dequant_rows(syn.KV_MXFP4, packed, scales)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = (e2m1[nib] * e8m0[scales][:, np.arange(576) // 32]).astype(np.float32)
    assert _same_f32(got, ref)


def test_fp8_rows_vs_torch(oracle_mod):
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(64, 576)).astype(np.uint8)
    codes[0, :256] = np.arange(256, dtype=np.uint8)
    for scale in (1.0, 0.0123456, 3.0e-3, 7.5):
        s = np.array([scale], dtype=np.float32)
        got = oracle_mod.dequant_rows(syn.KV_FP8, codes, s)
        ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(s[0])).numpy()
        assert _same_f32(got, ref)


def test_bf16_rows_exact(oracle_mod):
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 65536, size=(8, 576)).astype(np.uint16)
    got = oracle_mod.dequant_rows(syn.KV_BF16, bits, None)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    assert _same_f32(got, ref)


# --------------------------------------------------------------------------- attention

DTYPES = [syn.KV_BF16, syn.KV_FP8, syn.KV_MXFP4]


def _decoded_torch(case, oracle_mod):
    """Decoded physical rows as fp64; bf16/fp8 via torch conversions, MXFP4 via the pinned decoder."""
    if case.kv_dtype == syn.KV_BF16:
        x = torch.from_numpy(case.kv.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    elif case.kv_dtype == syn.KV_FP8:
        x = torch.from_numpy(case.kv).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(case.kv_scales[0])
    else:
        x = torch.from_numpy(oracle_mod.dequant_rows(case.kv_dtype, case.kv, case.kv_scales))
    return x.to(torch.float64)


def _q64(case):
    return torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _sdpa_ref(case, oracle_mod, sm_scale=1.0 / 24.0, q=None):
    x = _decoded_torch(case, oracle_mod)
    q = _q64(case) if q is None else q
    outs, lses = [], []
    for b in range(case.batch):
        s, e = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        rows = torch.from_numpy(case.kv_indices[s:e].astype(np.int64))
        K = x[rows]                  # [L, 576]
        V = K[:, :512].contiguous()  # first 512 columns of the same rows
        qb = q[b]                    # [16, 576]
        if e == s:
            outs.append(torch.zeros(16, 512, dtype=torch.float64))
            lses.append(torch.full((16,), -math.inf, dtype=torch.float64))
            continue
        o = torch.nn.functional.scaled_dot_product_attention(
            qb[None, :, None, :], K[None, None].expand(1, 16, -1, -1), V[None, None].expand(1, 16, -1, -1),
            scale=sm_scale)
        outs.append(o[0, :, 0, :])
        lses.append(torch.logsumexp((qb @ K.T) * sm_scale, dim=1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_attention_vs_torch_sdpa(oracle_mod, kv_dtype):
    case = syn.make_case(4, [1, 5, 37, 0], kv_dtype, seed=11, shuffle=True, extra_rows=9)
    out, lse = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    ref_o, ref_l = _sdpa_ref(case, oracle_mod)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_custom_sm_scale_vs_sdpa(oracle_mod, kv_dtype):
    case = syn.make_case(2, [9, 3], kv_dtype, seed=12)
    sc = 1.0 / math.sqrt(512.0)
    out, lse = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                                     sm_scale=sc)
    ref_o, ref_l = _sdpa_ref(case, oracle_mod, sm_scale=sc)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_brute_matches_main(oracle_mod, kv_dtype):
    case = syn.make_case(3, [1, 7, 20], kv_dtype, seed=5, shuffle=True)
    a = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    b = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                              route=oracle_mod.ROUTE_BRUTE)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("form", [0, 1, 2])
def test_split_combine_equals_single_pass(oracle_mod, kv_dtype, form):
    L = 29
    case = syn.make_case(2, [L, 6], kv_dtype, seed=6)
    ref = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    for nsplit in (1, 2, 3, 7, L, L + 5):  # L + 5 leaves empty pieces
        got = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                                    route=oracle_mod.ROUTE_SPLIT, nsplit=nsplit, form=form)
        np.testing.assert_allclose(got[0], ref[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got[1], ref[1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_zero_query_is_uniform_average(oracle_mod, kv_dtype):
    """q = 0: every score is 0, so out = mean of V rows and lse = ln L exactly."""
    L = 23
    case = syn.make_case(1, L, kv_dtype, seed=8, shuffle=True, extra_rows=4)
    case.q[:] = 0
    out, lse = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    x = _decoded_torch(case, oracle_mod).numpy()[case.kv_indices]
    np.testing.assert_allclose(out[0], np.broadcast_to(x[:, :512].mean(axis=0), (16, 512)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(L), rtol=0, atol=1e-14)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_single_token(oracle_mod, kv_dtype):
    """L = 1: out = V_0, lse = s_0."""
    case = syn.make_case(1, 1, kv_dtype, seed=9, shuffle=True, extra_rows=3)
    out, lse = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    x = _decoded_torch(case, oracle_mod).numpy()[case.kv_indices[0]]
    q = _q64(case).numpy()[0]
    np.testing.assert_allclose(out[0], np.broadcast_to(x[:512], (16, 512)), rtol=0, atol=0)
    np.testing.assert_allclose(lse[0], (q @ x) / 24.0, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("col", [0, 540])  # a no-RoPE column and a RoPE column
def test_one_hot_selects_single_row(oracle_mod, kv_dtype, col):
    """q = 1440 e_col (exact in bf16): s_j* = 1440/24 = 60, all other s = 0."""
    L, j_star = 41, 17
    case = syn.make_case(1, L, kv_dtype, seed=10, shuffle=True)
    _set_one_hot(case, j_star, col)
    case.q[:] = 0
    case.q[:, :, col] = 0x44B4  # 1440.0 in bf16
    out, lse = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    x = _decoded_torch(case, oracle_mod).numpy()[case.kv_indices]
    assert x[j_star, col] == 1.0 and np.count_nonzero(x[:, col]) == 1
    w_other = math.exp(-60.0)
    expect = (x[j_star, :512] + w_other * (x[:, :512].sum(axis=0) - x[j_star, :512])) / (1 + (L - 1) * w_other)
    np.testing.assert_allclose(out[0], np.broadcast_to(expect, (16, 512)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0], 60.0 + math.log1p((L - 1) * w_other), rtol=0, atol=1e-13)


def test_rope_columns_contribute(oracle_mod):
    """q_nope = 0, q_rope != 0: the result must differ from the uniform average."""
    case = syn.make_case(1, 64, syn.KV_BF16, seed=13)
    case.q[:, :, :512] = 0
    out, lse = oracle_mod.mla_decode(case.q, syn.KV_BF16, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    x = _decoded_torch(case, oracle_mod).numpy()
    assert np.max(np.abs(out[0] - x[:, :512].mean(axis=0))) > 1e-3
    assert np.all(np.abs(lse[0] - math.log(64)) > 1e-4)
    ref_o, ref_l = _sdpa_ref(case, oracle_mod)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)


def test_probabilities_sum_to_one(oracle_mod):
    """V = all ones and random RoPE columns: out = sum_j p_j = 1."""
    case = syn.make_case(2, [50, 3], syn.KV_BF16, seed=14)
    case.kv[:, :512] = 0x3F80
    out, _ = oracle_mod.mla_decode(case.q, syn.KV_BF16, case.kv, None, case.kv_indptr, case.kv_indices)
    assert np.max(np.abs(out - 1.0)) <= 1e-14


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_gather_permutation_invariance(oracle_mod, kv_dtype):
    case = syn.make_case(2, [13, 30], kv_dtype, seed=15)
    ref = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    perm = np.random.default_rng(1).permutation(case.kv.shape[0])
    inv = np.argsort(perm)
    kv2 = case.kv[perm]  # physical row r of kv2 is old row perm[r]
    sc2 = case.kv_scales[perm] if kv_dtype == syn.KV_MXFP4 else case.kv_scales
    idx2 = inv[case.kv_indices].astype(np.int32)
    got = oracle_mod.mla_decode(case.q, kv_dtype, kv2, sc2, case.kv_indptr, idx2)
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(got[1], ref[1], rtol=1e-14, atol=1e-14)


def test_duplicate_index_equals_duplicate_row(oracle_mod):
    case = syn.make_case(1, 10, syn.KV_BF16, seed=16)
    idx = np.concatenate([case.kv_indices, case.kv_indices[[3]]]).astype(np.int32)
    kv_dup = np.concatenate([case.kv, case.kv[[3]]])
    a = oracle_mod.mla_decode(case.q, 0, case.kv, None, np.array([0, 11], np.int32), idx)
    b = oracle_mod.mla_decode(case.q, 0, kv_dup, None, np.array([0, 11], np.int32), np.arange(11, dtype=np.int32))
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-16)
    c = oracle_mod.mla_decode(case.q, 0, case.kv, None, np.array([0, 10], np.int32), case.kv_indices)
    assert np.max(np.abs(a[0] - c[0])) > 1e-6


def test_empty_sequence(oracle_mod):
    case = syn.make_case(3, [4, 0, 2], syn.KV_FP8, seed=17)
    out, lse = oracle_mod.mla_decode(case.q, 1, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[[0, 2]]))


def test_batch_subset_matches_full(oracle_mod):
    case = syn.make_case(5, [3, 8, 1, 0, 6], syn.KV_MXFP4, seed=18, shuffle=True)
    full = oracle_mod.mla_decode(case.q, 2, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    sub = oracle_mod.mla_decode(case.q, 2, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                                batches=[4, 1])
    np.testing.assert_array_equal(sub[0], full[0][[4, 1]])
    np.testing.assert_array_equal(sub[1], full[1][[4, 1]])


# --------------------------------------------------------------------------- fp8 query

def _q8_decoded_torch(codes, scale):
    """fp8 query decoded with torch: e4m3fn -> fp32, one fp32 multiply by the scale, widened to fp64."""
    c = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    return (c * torch.tensor(np.float32(scale), dtype=torch.float32)).to(torch.float64)


def _torch_quant(q_bits, scale):
    """(q / scale).clamp(-448, 448) cast to e4m3fn, all in torch fp32 (its CPU cast rounds to nearest even)."""
    q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16).to(torch.float32)
    y = (q / torch.tensor(np.float32(scale), dtype=torch.float32)).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = syn.bf16_bits_to_f32(bits)
    return bits[np.isfinite(v)]


def test_e4m3fn_encode_exhaustive_bf16_vs_torch(oracle_mod):
    """Every finite bf16 value (all e4m3 midpoints are among them, so every tie is hit) through the
    quantiser with scale 1: codes equal torch's clamped cast bit for bit."""
    bits = _all_finite_bf16()
    codes, _ = oracle_mod.quantize_q_fp8(bits, scale=1.0)
    np.testing.assert_array_equal(codes, _torch_quant(bits, 1.0))


def test_e4m3fn_encode_ties_and_points(oracle_mod):
    assert oracle_mod.e4m3fn_encode(1.0) == 0x38
    assert oracle_mod.e4m3fn_encode(1.0625) == 0x38          # midpoint of 1 and 1.125 -> even mantissa
    assert oracle_mod.e4m3fn_encode(1.1875) == 0x3A          # midpoint of 1.125 and 1.25 -> even mantissa
    assert oracle_mod.e4m3fn_encode(-448.0) == 0xFE
    assert oracle_mod.e4m3fn_encode(2.0 ** -10) == 0x00      # half the smallest subnormal 2^-9 -> zero (even)
    assert oracle_mod.e4m3fn_encode(3 * 2.0 ** -10) == 0x02  # between 1 and 2 subnormal steps -> even
    assert oracle_mod.e4m3fn_encode(-0.0) == 0x80


@pytest.mark.parametrize("scale", [0.0133928571, 6.0 / 448.0, 0.5])
def test_quantize_static_vs_torch(oracle_mod, scale):
    case = syn.make_case(3, [2, 3, 4], syn.KV_BF16, seed=35)
    codes, sc = oracle_mod.quantize_q_fp8(case.q, scale=scale)
    assert sc[0] == np.float32(scale)
    np.testing.assert_array_equal(codes, _torch_quant(case.q, scale))


def test_quantize_dynamic_scale(oracle_mod):
    case = syn.make_case(4, [2, 3, 4, 5], syn.KV_BF16, seed=36)
    codes, sc = oracle_mod.quantize_q_fp8(case.q)
    q = syn.bf16_bits_to_f32(case.q)
    assert sc[0] == np.float32(np.abs(q).max()) / np.float32(448.0)
    np.testing.assert_array_equal(codes, _torch_quant(case.q, sc[0]))
    # the largest magnitude maps to the top of the range
    assert (codes & 0x7F).max() == 0x7E


def test_quantize_dynamic_zero_query(oracle_mod):
    codes, sc = oracle_mod.quantize_q_fp8(np.zeros((2, 16, 576), dtype=np.uint16))
    assert sc[0] == np.float32(1e-12) / np.float32(448.0)
    assert not codes.any()


def test_quantize_rejects_bad_static_scale(oracle_mod):
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            oracle_mod.quantize_q_fp8(np.zeros(4, dtype=np.uint16), scale=bad)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_vs_torch_sdpa(oracle_mod, kv_dtype):
    """fp8 query with a scale that is not a power of two, so the fp32 rounding of code * scale matters."""
    case = syn.make_case(3, [1, 23, 40], kv_dtype, seed=31, shuffle=True, extra_rows=5)
    codes, scale = oracle_mod.quantize_q_fp8(case.q)
    assert float(scale[0]) != 2.0 ** round(math.log2(float(scale[0])))
    out, lse = oracle_mod.mla_decode_q8(codes, float(scale[0]), kv_dtype, case.kv, case.kv_scales,
                                        case.kv_indptr, case.kv_indices)
    ref_o, ref_l = _sdpa_ref(case, oracle_mod, q=_q8_decoded_torch(codes, scale[0]))
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_l, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_q8_exact_scale_equals_bf16_query(oracle_mod, kv_dtype):
    """With a power-of-two scale every decoded query element (3 mantissa bits) is a bf16 value, so the
    fp8-query route must reproduce the bf16-query route on those bf16 bits exactly."""
    case = syn.make_case(2, [17, 6], kv_dtype, seed=32)
    rng = np.random.default_rng(33)
    codes = rng.integers(0, 256, size=case.q.shape, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C                       # no NaN codes
    scale = 2.0 ** -5
    qf = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * scale
    qbits = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert torch.equal(torch.from_numpy(qbits.view(np.int16)).view(torch.bfloat16).to(torch.float32), qf)
    a = oracle_mod.mla_decode_q8(codes, scale, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    b = oracle_mod.mla_decode(qbits, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------- several query tokens

def _mtp_sdpa_ref(case, q_bits, qo, causal, oracle_mod, sm_scale=1.0 / 24.0):
    """torch fp64 SDPA per sequence with an explicit visibility mask (bottom-right causal or none)."""
    x = _decoded_torch(case, oracle_mod)
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    outs, lses = [], []
    for b in range(case.batch):
        s, e = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        r0, r1 = int(qo[b]), int(qo[b + 1])
        n, L = r1 - r0, e - s
        K = x[torch.from_numpy(case.kv_indices[s:e].astype(np.int64))]
        for t in range(n):
            vis = L - n + 1 + t if causal else L
            vis = max(0, min(L, vis))
            qt = q[r0 + t]                                    # [16, 576]
            if vis == 0:
                outs.append(torch.zeros(16, 512, dtype=torch.float64))
                lses.append(torch.full((16,), -math.inf, dtype=torch.float64))
                continue
            mask = torch.zeros(1, 1, 1, L, dtype=torch.bool)
            mask[..., :vis] = True
            o = torch.nn.functional.scaled_dot_product_attention(
                qt[None, :, None, :], K[None, None].expand(1, 16, -1, -1),
                K[:, :512].contiguous()[None, None].expand(1, 16, -1, -1), attn_mask=mask, scale=sm_scale)
            outs.append(o[0, :, 0, :])
            lses.append(torch.logsumexp((qt @ K[:vis].T) * sm_scale, dim=1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("causal", [False, True])
def test_mtp_vs_torch_sdpa_masked(oracle_mod, kv_dtype, causal):
    """Ragged query counts (1..4, one sequence shorter than its query count) against masked SDPA."""
    case = syn.make_case(4, [9, 2, 30, 17], kv_dtype, seed=41, shuffle=True, extra_rows=3)
    q, qo = syn.make_mtp_query([1, 3, 2, 4], seed=42)
    out, lse = oracle_mod.mla_decode_mtp(q, qo, causal, kv_dtype, case.kv, case.kv_scales, case.kv_indptr,
                                         case.kv_indices)
    ref_o, ref_l = _mtp_sdpa_ref(case, q, qo, causal, oracle_mod)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(lse), ~fin)
    np.testing.assert_allclose(lse[fin], ref_l[fin], rtol=1e-13, atol=1e-12)
    if causal:
        assert (~fin).any()   # the 2-token sequence with 3 query tokens: its first query sees nothing


def test_mtp_causal_first_query_sees_one_row(oracle_mod):
    """n query tokens over n cache tokens, causal: query 0 sees only row 0, so its output is that row's V."""
    case = syn.make_case(1, [5], syn.KV_BF16, seed=43)
    q, qo = syn.make_mtp_query([5], seed=44)
    out, lse = oracle_mod.mla_decode_mtp(q, qo, True, syn.KV_BF16, case.kv, None, case.kv_indptr, case.kv_indices)
    v0 = syn.bf16_bits_to_f32(case.kv[case.kv_indices[0]])[:512].astype(np.float64)
    assert np.array_equal(out[0], np.broadcast_to(v0, (16, 512)))


@pytest.mark.parametrize("causal", [False, True])
def test_mtp_brute_matches_main(oracle_mod, causal):
    case = syn.make_case(2, [12, 7], syn.KV_FP8, seed=45)
    q, qo = syn.make_mtp_query([3, 2], seed=46)
    a = oracle_mod.mla_decode_mtp(q, qo, causal, syn.KV_FP8, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    b = oracle_mod.mla_decode_mtp(q, qo, causal, syn.KV_FP8, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices,
                                  route=oracle_mod.ROUTE_BRUTE)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-13)


def test_mtp_row_subset(oracle_mod):
    case = syn.make_case(3, [4, 11, 6], syn.KV_MXFP4, seed=47)
    q, qo = syn.make_mtp_query([2, 2, 2], seed=48)
    full = oracle_mod.mla_decode_mtp(q, qo, True, syn.KV_MXFP4, case.kv, case.kv_scales, case.kv_indptr,
                                     case.kv_indices)
    sub = oracle_mod.mla_decode_mtp(q, qo, True, syn.KV_MXFP4, case.kv, case.kv_scales, case.kv_indptr,
                                    case.kv_indices, rows=[5, 0, 3])
    assert np.array_equal(sub[0], full[0][[5, 0, 3]]) and np.array_equal(sub[1], full[1][[5, 0, 3]])


# --------------------------------------------------------------------------- paged cache


def _read_paged_example():
    """tests/golden/paged_example.txt: (page_size, page_indptr, page_ids, last_page_len, expected rows per sequence)."""
    ps, pages, last, rows = None, [], [], []
    with open(os.path.join(GOLDEN, "paged_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("page_size"):
                ps = int(line.split()[1])
                continue
            assert line.startswith("seq")
            a, b, c = line[3:].split("|")
            pages.append([int(x) for x in a.split()])
            last.append(int(b))
            rows.append([int(x) for x in c.split()])
    indptr = np.zeros(len(pages) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum([len(p) for p in pages])
    ids = np.array([x for p in pages for x in p], dtype=np.int32)
    return ps, indptr, ids, np.array(last, dtype=np.int32), rows


def test_paged_expansion_worked_example(oracle_mod):
    """The oracle's page expansion reproduces the hand-worked token rows (a partial last
    page, an empty sequence, a page shared by two sequences)."""
    ps, indptr, ids, last, rows = _read_paged_example()
    tok_indptr, tok_rows = oracle_mod.expand_pages(indptr, ids, last, ps)
    assert tok_indptr.tolist() == [0] + np.cumsum([len(r) for r in rows]).tolist()
    assert tok_rows.tolist() == [x for r in rows for x in r]


@pytest.mark.parametrize("kv_dtype", [syn.KV_BF16, syn.KV_FP8, syn.KV_MXFP4])
def test_paged_decode_worked_example(oracle_mod, kv_dtype):
    """The paged route on the worked example equals the plain route over the hand-written
    token rows, bit for bit."""
    ps, indptr, ids, last, rows = _read_paged_example()
    B = len(rows)
    case = syn.make_case(B, 0, kv_dtype, seed=61, extra_rows=6 * ps)
    tok_indptr = np.zeros(B + 1, dtype=np.int32)
    tok_indptr[1:] = np.cumsum([len(r) for r in rows])
    tok_rows = np.array([x for r in rows for x in r], dtype=np.int32)
    o1, l1 = oracle_mod.mla_decode_paged(case.q, kv_dtype, case.kv, case.kv_scales, indptr, ids, last, ps)
    o2, l2 = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, tok_indptr, tok_rows)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isneginf(l1[1]).all() and not o1[1].any()  # the empty sequence


@pytest.mark.parametrize("kv_dtype", [syn.KV_FP8, syn.KV_MXFP4])
def test_paged_page_size_one_is_the_plain_route(oracle_mod, kv_dtype):
    """With one row per page the page table is the token table: the paged route equals
    oracle_mla_decode on the same arrays (kv_last_page_len is not read)."""
    case = syn.make_case(4, [7, 0, 30, 1], kv_dtype, seed=62, shuffle=True, extra_rows=5)
    o1, l1 = oracle_mod.mla_decode_paged(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr,
                                         case.kv_indices, None, 1)
    o2, l2 = oracle_mod.mla_decode(case.q, kv_dtype, case.kv, case.kv_scales, case.kv_indptr, case.kv_indices)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_paged_expansion_counts_and_rejects(oracle_mod):
    """Token count = (pages - 1) * page_size + last_page_len per non-empty sequence; a last
    page length outside 1..page_size is refused."""
    rng = np.random.default_rng(63)
    ps = 16
    npages = rng.integers(0, 6, size=9)
    last = np.where(npages > 0, rng.integers(1, ps + 1, size=9), 0).astype(np.int32)
    indptr = np.zeros(10, dtype=np.int32)
    indptr[1:] = np.cumsum(npages)
    ids = rng.permutation(200)[:indptr[-1]].astype(np.int32)
    tok_indptr, tok_rows = oracle_mod.expand_pages(indptr, ids, last, ps)
    want = np.where(npages > 0, (npages - 1) * ps + last, 0)
    assert np.diff(tok_indptr).tolist() == want.tolist()
    assert all(r // ps in set(ids.tolist()) for r in tok_rows.tolist())
    bad = last.copy()
    bad[np.argmax(npages > 0)] = ps + 1
    with pytest.raises(ValueError):
        oracle_mod.expand_pages(indptr, ids, bad, ps)

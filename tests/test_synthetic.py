"""The seeded input generator: determinism, shapes and the quantisers' invariants.

Decoding here goes through torch's own conversions or the pinned e2m1 table,
never through the HIP library.
"""
import numpy as np
import pytest
import torch

import synthetic as syn

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=np.float32)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-39, 65504.0], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(syn.f32_to_bf16_bits(x), ref)
    r = np.random.default_rng(0).standard_normal(100000, dtype=np.float32)
    ref = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(syn.f32_to_bf16_bits(r), ref)


@pytest.mark.parametrize("kv_dtype", [0, 1, 2])
def test_seeded_determinism_and_shapes(kv_dtype):
    a = syn.make_case(3, [5, 0, 9], kv_dtype, seed=42, shuffle=True, extra_rows=2)
    b = syn.make_case(3, [5, 0, 9], kv_dtype, seed=42, shuffle=True, extra_rows=2)
    for x, y in ((a.q, b.q), (a.kv, b.kv), (a.kv_indices, b.kv_indices), (a.kv_indptr, b.kv_indptr)):
        np.testing.assert_array_equal(x, y)
    assert a.q.shape == (3, 16, 576) and a.q.dtype == np.uint16
    assert list(a.kv_indptr) == [0, 5, 5, 14]
    assert a.kv_indices.shape == (14,) and len(set(a.kv_indices.tolist())) == 14
    rows = 16
    if kv_dtype == 0:
        assert a.kv.shape == (rows, 576) and a.kv_scales is None
    elif kv_dtype == 1:
        assert a.kv.shape == (rows, 576) and a.kv_scales.shape == (1,) and a.kv_scales.dtype == np.float32
    else:
        assert a.kv.shape == (rows, 288) and a.kv_scales.shape == (rows, 18)
    c = syn.make_case(3, [5, 0, 9], kv_dtype, seed=43, shuffle=True, extra_rows=2)
    assert not np.array_equal(a.q, c.q)


def test_fp8_quantiser_recipe():
    x = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(
        np.random.default_rng(1).standard_normal((512, 576), dtype=np.float32)))
    codes, scale = syn.quantize_fp8_per_tensor(x)
    assert scale.dtype == np.float32
    assert scale[0] == np.float32(np.float32(np.max(np.abs(x))) / np.float32(448.0))
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.max(np.abs(vals)) == 448.0           # absmax maps to the largest code
    assert not np.any(np.isnan(vals))
    y = x / scale[0]
    normal = np.abs(y) >= 2.0 ** -6
    rel = np.abs(vals[normal] - y[normal]) / np.abs(y[normal])
    assert np.max(rel) <= 2.0 ** -4                 # half an ulp of a 3-bit mantissa


def test_mxfp4_quantiser_recipe():
    x = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(
        np.random.default_rng(2).standard_normal((256, 576), dtype=np.float32)))
    x[0, :32] = 0.0                                  # all-zero block
    packed, scales = syn.quantize_mxfp4(x)
    assert packed.shape == (256, 288) and scales.shape == (256, 18)
    nib = np.empty((256, 576), dtype=np.uint8)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    assert scales[0, 0] == 127 and np.all(nib[0, :32] == 0)
    blocks = x.reshape(256, 18, 32)
    amax = np.abs(blocks).max(axis=2)
    nz = amax > 0
    expect = np.floor(np.log2(amax[nz])).astype(np.int32) - 2 + 127
    np.testing.assert_array_equal(scales[nz].astype(np.int32), expect)
    e8 = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float32).numpy()
    dec = E2M1[nib] * np.repeat(e8, 32, axis=1)
    mag = np.abs(E2M1[nib]).reshape(256, 18, 32)
    assert np.all(mag.max(axis=2)[nz] >= 4.0)        # the block max lands in [4, 6]
    # error bound: half a grid step at the element's magnitude, or saturation above 6
    y = (x.reshape(256, 18, 32) / np.repeat(e8, 32, axis=1).reshape(256, 18, 32)).reshape(256, 576)
    grid_step = np.where(np.abs(y) < 2, 0.5, np.where(np.abs(y) < 4, 1.0, 2.0))
    err = np.abs(dec - x) / np.repeat(e8, 32, axis=1)
    ok = (err <= grid_step / 2 + 1e-6) | (np.abs(y) > 6)
    assert np.all(ok)


def test_mxfp4_ties_round_to_even():
    # one block with a neutral scale: amax 4 -> floor(log2 4) - 2 = 0 -> scale code 127
    v = np.zeros((1, 576), dtype=np.float32)
    v[0, :10] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, 6.5]
    packed, scales = syn.quantize_mxfp4(v)
    assert scales[0, 0] == 127
    nib = np.empty(576, dtype=np.uint8)
    nib[0::2] = packed[0] & 0xF
    nib[1::2] = packed[0] >> 4
    assert list(E2M1[nib[:9]]) == [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 0.0]


def test_workload_bytes():
    c = syn.make_case(4, 16, syn.KV_FP8, seed=0)
    assert c.kv_bytes() == 64 * 576 + 4
    c = syn.make_case(4, 16, syn.KV_MXFP4, seed=0)
    assert c.kv_bytes() == 64 * (288 + 18)


@pytest.mark.parametrize("page_size", [1, 2, 8, 13])
def test_paged_case_page_table(page_size):
    """The page table of a paged workload: whole pages but the last, a last-page
    length in 1..page_size, each physical page used once; the generator writes
    no token-to-row expansion (the oracle expands the pages itself)."""
    lens = [0, 1, page_size, 2 * page_size + 1, 37]
    case, pg = syn.make_paged_case(len(lens), lens, syn.KV_FP8, page_size, seed=9, extra_pages=3)
    assert list(np.diff(case.kv_indptr)) == lens
    assert case.kv_indices.size == 0 and case.meta["paged"] is pg
    assert case.kv.shape[0] % page_size == 0
    ids = pg["kv_indices"]
    assert len(set(ids.tolist())) == len(ids)  # each physical page used once
    assert ids.max() < case.kv.shape[0] // page_size
    for b, L in enumerate(lens):
        np_b = pg["kv_indptr"][b + 1] - pg["kv_indptr"][b]
        assert np_b == -(-L // page_size)
        if L:
            assert 1 <= pg["kv_last_page_len"][b] <= page_size
            assert (np_b - 1) * page_size + pg["kv_last_page_len"][b] == L


def test_mtp_query_layout():
    q, qo = syn.make_mtp_query([2, 0, 3], seed=5)
    assert q.shape == (5, 16, 576) and q.dtype == np.uint16
    assert qo.tolist() == [0, 2, 2, 5] and qo.dtype == np.int32
    q2, _ = syn.make_mtp_query([2, 0, 3], seed=5)
    assert np.array_equal(q, q2)

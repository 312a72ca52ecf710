"""mla_decode_noalloc (the entry point that allocates nothing) through the C ABI.

Its split partials and arrival counters live in the library's fixed per-device
scratch array instead of a caller workspace. It runs the same plan and kernels
as mla_decode, so its output must equal mla_decode's bit for bit (and the
oracle within the parity bands), call after call on the shared scratch: here a
large input, then a smaller one, in every merge form.
"""
import ctypes

import numpy as np
import pytest

import synthetic as syn
from test_gpu_parity import DTYPES, check, oracle_ref, run_gpu, to_dev

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


@pytest.fixture(scope="module")
def noalloc(mla):
    lib = ctypes.CDLL(mla.LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    f = lib.mla_decode_noalloc
    f.restype = i32
    f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_int64, i32, ctypes.c_float, i32, vp]
    return f


def run_noalloc(f, case, dev, flags):
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = f(p(t["q"]), p(t["kv"]), p(t["kv_scales"]), p(t["kv_indptr"]), p(t["kv_indices"]), p(out), p(lse), B,
           case.total_kv, case.kv_dtype, ctypes.c_float(0.0), flags, stream)
    assert rc == 0, f"mla_decode_noalloc returned {rc}"
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kv_dtype", DTYPES)
@pytest.mark.parametrize("plan", ["default", "merged3", "combine8", "merged8", "persistent"])
def test_noalloc_equals_mla_decode_large_then_small(mla, orc, dev, noalloc, kv_dtype, plan):
    flags = {"default": 0, "merged3": mla.flags_for(splits=3),
             "combine8": mla.flags_for(splits=8) | mla.FLAG_COMBINE_LAUNCH, "merged8": mla.flags_for(splits=8),
             "persistent": mla.flags_for(persistent=True, grid=64)}[plan]
    big = syn.make_case(6, [3000, 1, 0, 777, 5000, 64], kv_dtype, seed=700 + kv_dtype, shuffle=True, extra_rows=3)
    if plan == "merged8":  # 8 splits: merged in stage 1 from bf16 partials (bf16 and fp8 caches)
        big = syn.make_case(4, [12000, 9000, 0, 12500], kv_dtype, seed=720 + kv_dtype, shuffle=True, extra_rows=3)
        assert mla.mla_decode_plan(big.batch, big.total_kv, kv_dtype, flags).combine == (1 if kv_dtype == syn.KV_MXFP4
                                                                                          else 2)
    small = syn.make_case(3, [100, 0, 40], kv_dtype, seed=710 + kv_dtype)
    for name, case in (("large", big), ("small", small)):
        print(f"noalloc {plan} {syn.KV_NAMES[kv_dtype]} {name}: plan "
              f"{mla.mla_decode_plan(case.batch, case.total_kv, kv_dtype, flags)}", flush=True)
        got = run_noalloc(noalloc, case, dev, flags)
        ref = run_gpu(mla, case, dev, flags=flags)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), f"{name}: differs from mla_decode"
        check(got, oracle_ref(orc, case), f"noalloc {plan} {name}")

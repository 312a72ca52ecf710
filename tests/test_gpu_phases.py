"""The measurement build (phase timestamps, include/mla_decode_phases.h) on the GPU.

It is the decode library's sources compiled with MLA_PHASE_STAMPS=1. Loaded with
ctypes beside the decode library, it must give bit-identical results to it and
write every stamp of every workgroup, in phase order.
"""
import ctypes
import os

import numpy as np
import pytest

import synthetic as syn
from test_gpu_parity import new_workspace, run_gpu, to_dev

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
def phases_lib(mla):
    import mla_decode_02_amd.build as build

    assert os.path.exists(build.PHASES_LIB), "build the measurement library with mla_decode_02_amd/build.py"
    lib = ctypes.CDLL(build.PHASES_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.mla_source_digest.restype = ctypes.c_char_p
    assert lib.mla_source_digest().decode() == mla.mla_source_digest()
    lib.mla_phase_buffers.restype = i32
    lib.mla_phase_buffers.argtypes = [vp, vp]
    lib.mla_decode.restype = i32
    lib.mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_int64, i32, ctypes.c_float, vp,
                               ctypes.c_size_t, i32, vp]
    yield lib
    lib.mla_phase_buffers(None, None)


@pytest.mark.parametrize("flags_kind", ["combine8", "merged8", "merged3", "one"])
def test_phase_stamps_ordered_and_results_identical(mla, dev, phases_lib, flags_kind):
    flags = {"combine8": mla.flags_for(splits=8) | mla.FLAG_COMBINE_LAUNCH, "merged8": mla.flags_for(splits=8),
             "merged3": mla.flags_for(splits=3), "one": mla.flags_for(splits=1)}[flags_kind]
    case = syn.make_case(6, [700, 33, 1500, 256, 1, 999], syn.KV_FP8, seed=680, shuffle=True)
    plan = mla.mla_decode_plan(case.batch, case.total_kv, case.kv_dtype, flags)
    t = to_dev(case, dev)
    B = case.batch
    out = torch.full((B, 16, 512), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, 16), float("nan"), dtype=torch.float32, device=dev)
    st = torch.zeros(plan.grid * 8, dtype=torch.int64, device=dev)
    comb = torch.zeros(64 * B * 2, dtype=torch.int64, device=dev)
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())  # noqa: E731
    assert phases_lib.mla_phase_buffers(p(st), p(comb)) == 0
    ws = new_workspace(mla, case, dev, flags)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = phases_lib.mla_decode(p(t["q"]), p(t["kv"]), p(t["kv_scales"]), p(t["kv_indptr"]), p(t["kv_indices"]),
                               p(out), p(lse), B, case.total_kv, case.kv_dtype, ctypes.c_float(0.0), p(ws),
                               0 if ws is None else ws.numel(), flags, stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert phases_lib.mla_phase_buffers(None, None) == 0
    got = (out.float().cpu().numpy(), lse.cpu().numpy())
    ref = run_gpu(mla, case, dev, flags=flags)
    assert np.array_equal(got[0], ref[0].astype(np.float32)) and np.array_equal(got[1], ref[1].astype(np.float32))
    s = st.view(-1, 8).cpu().numpy()
    # a split past its sequence's end (t0 = s * chunk >= L) attends no tokens and has no phase 2
    S = plan.num_splits
    lens = np.diff(case.kv_indptr)
    chunks = ((lens + S - 1) // S + 31) // 32 * 32
    empty = sum(int(np.sum(np.arange(S) * c >= L)) for L, c in zip(lens, chunks))
    assert int(np.sum(s[:, 2] == 0)) == empty
    cols = [0, 1, 3, 4, 5]
    assert np.all(s[:, cols] > 0), "a stage-1 workgroup left a phase unstamped"
    assert np.all(np.diff(s[:, cols], axis=1) >= 0), "stage-1 phases out of order"
    att = s[:, 2] > 0
    assert np.all(s[att, 1] <= s[att, 2]) and np.all(s[att, 2] <= s[att, 3])
    c = comb.view(-1, 2).cpu().numpy()
    if plan.combine == 1:
        n = 16 * 4 * B // 8  # combine workgroups of the 8-split plan (8 items each)
        assert np.all(c[:n] > 0) and np.all(c[n:] == 0)
        assert np.all(c[:n, 1] >= c[:n, 0])
        assert c[:n, 0].min() >= s[:, 0].min()
    else:
        assert np.all(c == 0)

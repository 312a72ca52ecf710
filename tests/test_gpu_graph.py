"""The decode calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, synchronises nothing and clears nothing with
memsets, so a captured call is the same launches on the captured pointers.
Each replay is compared bitwise with an eager call on the same inputs; between
replays the program runs other eager work and changes the query in place, so
a replay that reused stale results would show.
"""
import numpy as np
import pytest

import synthetic as syn
from test_gpu_parity import DTYPES, to_dev

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


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("merge", ["launch", "merged3", "merged8"])
@pytest.mark.parametrize("kv_dtype", DTYPES)
def test_captured_decode_replays(mla, dev, kv_dtype, merge):
    """A captured call replays bit-identically to eager calls, with the combine
    launch (default plan here), with the partials merged by the last-arriving
    split (3 splits; its arrival counters are reset inside the kernel), and with
    8 long splits merged there from bf16 partials (bf16 and fp8 caches)."""
    if merge == "merged8" and kv_dtype == syn.KV_MXFP4:
        pytest.skip("MXFP4 merges 8 splits in the combine launch")
    lens = [12000, 9000, 0, 12500] if merge == "merged8" else [1000, 3, 700, 0, 2000, 64]
    case = syn.make_case(len(lens), lens, kv_dtype, seed=620 + kv_dtype, shuffle=True)
    t = to_dev(case, dev)
    B = case.batch
    flags = {"launch": 0, "merged3": mla.flags_for(splits=3), "merged8": mla.flags_for(splits=8)}[merge]
    assert mla.mla_decode_plan(B, case.total_kv, kv_dtype, flags).combine == (1 if merge == "launch" else 2)
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, 16), dtype=torch.float32, device=dev)
    ws = mla.new_workspace(mla.mla_decode_workspace_size(B, case.total_kv, kv_dtype, flags), dev)
    args = (t["q"], t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], out, lse)
    kw = dict(total_kv=case.total_kv, kv_dtype=kv_dtype, workspace=ws, flags=flags)
    g = _capture(lambda: mla.mla_decode(*args, **kw))
    rng = np.random.default_rng(621)
    other = syn.make_case(2, [300, 40], kv_dtype, seed=622)
    for i in range(4):
        # eager reference on the current inputs, into separate outputs
        ro = torch.empty_like(out)
        rl = torch.empty_like(lse)
        mla.mla_decode(args[0], *args[1:5], ro, rl, total_kv=case.total_kv, kv_dtype=kv_dtype, flags=flags)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ro.view(torch.int16)), f"replay {i}: out differs"
        assert torch.equal(lse, rl), f"replay {i}: lse differs"
        # unrelated eager work, then a new query in place for the next replay
        to = to_dev(other, dev)
        o2 = torch.empty((2, 16, 512), dtype=torch.bfloat16, device=dev)
        mla.mla_decode(to["q"], to["kv"], to["kv_scales"], to["kv_indptr"], to["kv_indices"], o2, None,
                       total_kv=other.total_kv, kv_dtype=kv_dtype)
        torch.cuda.synchronize()
        qn = syn.f32_to_bf16_bits(rng.standard_normal((B, 16, 576), dtype=np.float32))
        args[0].copy_(torch.from_numpy(qn.view(np.int16)).view(torch.bfloat16))


def test_captured_fp8_query_dynamic_scale_replays(mla, dev):
    """Three launches per call (partial maxima, stage 1, combine) and the scale written by the kernels."""
    case = syn.make_case(5, [900, 33, 2500, 1, 400], syn.KV_MXFP4, seed=630, shuffle=True)
    t = to_dev(case, dev)
    B = case.batch
    out = torch.empty((B, 16, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, 16), dtype=torch.float32, device=dev)
    qs = torch.empty(1, dtype=torch.float32, device=dev)
    need = mla.mla_decode_q8_workspace_size(B, case.total_kv, syn.KV_MXFP4, 0, mla.Q_SCALE_DYNAMIC)
    ws = mla.new_workspace(need, dev)
    kw = dict(q_scale_mode=mla.Q_SCALE_DYNAMIC, total_kv=case.total_kv, kv_dtype=syn.KV_MXFP4)
    g = _capture(lambda: mla.mla_decode_q8(t["q"], qs, t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"],
                                           out, lse, workspace=ws, **kw))
    rng = np.random.default_rng(631)
    for i in range(4):
        ro, rl, rs = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(qs)
        mla.mla_decode_q8(t["q"], rs, t["kv"], t["kv_scales"], t["kv_indptr"], t["kv_indices"], ro, rl, **kw)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        qs.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ro.view(torch.int16)), f"replay {i}: out differs"
        assert torch.equal(lse, rl) and torch.equal(qs, rs), f"replay {i}: lse or scale differs"
        qn = syn.f32_to_bf16_bits(rng.standard_normal((B, 16, 576), dtype=np.float32) * (1 + i))
        t["q"].copy_(torch.from_numpy(qn.view(np.int16)).view(torch.bfloat16))

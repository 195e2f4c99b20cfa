"""dpsgd_step_noalloc (the step on the library's per-device scratch, for callers that cannot
allocate) against dpsgd_step on a caller workspace: the same kernels, so the same inputs must give
bitwise the same norms, factors and noised sums, on two calls in a row whose second input is
smaller, on the direct (stored blocks, fused tail), Gram and dense-GEMM paths; a nonfinite record
reports through status_out and a following call resets it; plans too large for the scratch are
refused before any launch."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
from _helpers import host_inputs, to_device  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def _run(plan, w, dA, dG, n, noalloc, flags=0, seed=5, step=2):
    out = [torch.full((a * b,), float("nan"), dtype=torch.float32, device=DEV) for a, b in w.layers]
    nrm = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=DEV)
    cf = torch.full((max(n, 1),), -1.0, dtype=torch.float32, device=DEV)
    if noalloc:
        st = torch.full((1,), 0x7777, dtype=torch.int32, device=DEV)
        dp.step_noalloc(plan, dA, dG, out, w.C, w.sigma, seed, step, n_records=n, flags=flags,
                        norms_out=nrm, clip_out=cf, status_out=st)
        torch.cuda.synchronize()
        status = int(st.cpu().numpy()[0])
    else:
        ws = plan.workspace(DEV)
        dp.step(plan, dA, dG, out, ws, w.C, w.sigma, seed, step, n_records=n, flags=flags,
                norms_out=nrm, clip_out=cf)
        status = 0 if dp.status(plan, ws) == dp.OK else 1
    return {"n": nrm.cpu().numpy()[:n], "c": cf.cpu().numpy()[:n], "status": status,
            "out": [o.cpu().numpy() for o in out]}


def _same(a, b):
    assert a["status"] == b["status"] == 0
    assert np.array_equal(a["n"], b["n"]) and np.array_equal(a["c"], b["c"])
    for x, y in zip(a["out"], b["out"]):
        assert np.array_equal(x, y)


CASES = [
    ("direct fp32, stored blocks", datagen.reduced(2), dp.PATH_AUTO),
    ("direct bf16 LoRA", datagen.reduced(3), dp.PATH_AUTO),
    ("Gram + dense GEMM bf16", datagen.reduced(4), dp.PATH_AUTO),
    ("Gram fp32", datagen.reduced(2), dp.PATH_GRAM),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_noalloc_matches_step_two_calls(idx):
    label, w, path = CASES[idx]
    say("noalloc", label)
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T, path)
    assert plan.ws_bytes <= 64 << 20
    As, Gs = host_inputs(w)
    dA = [to_device(a, DEV) for a in As]
    dG = [to_device(g, DEV) for g in Gs]
    # first call: the whole batch; second call: fewer records (a smaller input), same scratch
    for n in (w.B, w.B - 2):
        ref = _run(plan, w, dA, dG, n, noalloc=False)
        got = _run(plan, w, dA, dG, n, noalloc=True)
        _same(ref, got)
    # then a smaller plan (fewer, narrower layers) on the same scratch
    w2 = w.with_(layers=w.layers[:1], layer_names=w.layer_names[:1], B=2, logical_B=2)
    plan2 = dp.Plan(w2.layers, w2.dtype, w2.B, w2.T, path)
    A2, G2 = host_inputs(w2)
    d2A = [to_device(a, DEV) for a in A2]
    d2G = [to_device(g, DEV) for g in G2]
    _same(_run(plan2, w2, d2A, d2G, 2, noalloc=False), _run(plan2, w2, d2A, d2G, 2, noalloc=True))


def test_noalloc_virtual_batch_and_status():
    """Two physical batches accumulated on the scratch, noise once, against the caller-workspace
    path; a NaN record sets status_out and leaves out untouched; the next call without
    ACCUMULATE resets it."""
    w = datagen.reduced(5)
    say("noalloc virtual batch")
    plan = dp.Plan(w.layers, w.dtype, w.B, w.T)
    ws = plan.workspace(DEV)
    res = {}
    for noalloc in (False, True):
        out = [torch.empty(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
        for p in range(2):
            As, Gs = host_inputs(w, first=p * w.B, n=w.B)
            dA = [to_device(a, DEV) for a in As]
            dG = [to_device(g, DEV) for g in Gs]
            flags = dp.NO_NOISE | (dp.ACCUMULATE if p else 0)
            if noalloc:
                dp.step_noalloc(plan, dA, dG, out, w.C, w.sigma, 0, 0, flags=flags)
            else:
                dp.step(plan, dA, dG, out, ws, w.C, w.sigma, 0, 0, flags=flags)
        dp.noise(plan, out, w.C, w.sigma, 0, 0, ws=None if noalloc else ws)
        torch.cuda.synchronize()
        res[noalloc] = [o.cpu().numpy() for o in out]
    for x, y in zip(res[False], res[True]):
        assert np.array_equal(x, y)
    # a NaN input: status_out nonzero, out untouched
    As, Gs = host_inputs(w)
    As[0] = As[0].copy()
    As[0][1, 2, :] = np.uint16(0x7FC0)          # bf16 NaN
    dA = [to_device(a, DEV) for a in As]
    dG = [to_device(g, DEV) for g in Gs]
    out = [torch.full((a * b,), 3.0, dtype=torch.float32, device=DEV) for a, b in w.layers]
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    dp.step_noalloc(plan, dA, dG, out, w.C, w.sigma, 0, 0, status_out=st)
    torch.cuda.synchronize()
    assert int(st.cpu().numpy()[0]) != 0
    assert all(np.all(o.cpu().numpy() == 3.0) for o in out)
    As, Gs = host_inputs(w)
    dA = [to_device(a, DEV) for a in As]
    dp.step_noalloc(plan, dA, dG, out, w.C, w.sigma, 0, 0, status_out=st)
    torch.cuda.synchronize()
    assert int(st.cpu().numpy()[0]) == 0


def test_noalloc_refuses_large_and_segment_plans():
    lib = dp.load()
    big = dp.Plan([(768, 8), (8, 768)] * 24, dp.DTYPE_F32, 4096, 128)
    assert big.ws_bytes > 64 << 20
    args = dp.StepArgs(1, None, None, None, None, 1.0, 1.0, 0, 0, 0, None, None, None, 0.0, 1.0)
    assert lib.dpsgd_step_noalloc(big.handle, ctypes.byref(args), None, None) == dp.ERR_INVALID_ARG
    seg = dp.Plan([(8, 8)], dp.DTYPE_F32, 2, 4, segments=True)
    assert lib.dpsgd_step_noalloc(seg.handle, ctypes.byref(args), None, None) == dp.ERR_INVALID_ARG


def test_noalloc_step_in_a_hip_graph():
    """The use the entry point is for: the whole step (norms, clip factors, the fused sum + noise or
    the GEMM sum, the status copy) captured once into a HIP graph, which no allocation may enter,
    then replayed on new inputs copied into the same buffers, with eager steps and
    synchronisations between the replays; every replay equals the eager dpsgd_step on a caller
    workspace bit for bit."""
    for w, sp in ((datagen.reduced(2), dp.SUM_AUTO), (datagen.reduced(3), dp.SUM_GEMM)):
        say("noalloc graph", w.name, sp)
        plan = dp.Plan(w.layers, w.dtype, w.B, w.T, dp.PATH_AUTO, sp)
        As, Gs = host_inputs(w)
        dA = [to_device(a, DEV) for a in As]
        dG = [to_device(g, DEV) for g in Gs]
        out = [torch.zeros(a * b, dtype=torch.float32, device=DEV) for a, b in w.layers]
        nrm = torch.zeros(w.B, dtype=torch.float32, device=DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        cap = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            dp.step_noalloc(plan, dA, dG, out, w.C, w.sigma, 9, 4, norms_out=nrm, status_out=st,
                            stream=cap)
        for k in range(3):
            A2, G2 = host_inputs(w, first=w.B * (k + 1), n=w.B)
            for d, h in zip(dA + dG, A2 + G2):
                d.copy_(to_device(h, DEV))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = ([o.cpu().numpy().copy() for o in out], nrm.cpu().numpy().copy(), int(st.cpu().numpy()[0]))
            ref = _run(plan, w, dA, dG, w.B, noalloc=False, seed=9, step=4)
            assert got[2] == 0 and ref["status"] == 0
            assert np.array_equal(got[1], ref["n"])
            for x, y in zip(got[0], ref["out"]):
                assert np.array_equal(x, y)
        del g

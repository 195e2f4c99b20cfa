"""C-ABI checks that need no GPU: the library loads and exports every function include/dpsgd.h
declares; plan construction validates its inputs and chooses paths as documented; every argument
error of the compute entry points is returned before any launch (on a machine without a GPU a
launch would surface as DPSGD_ERR_HIP instead)."""
import ctypes
import os
import re
import subprocess

import pytest

import differentially_private_amd as dp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dpsgd.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dpsgd_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert len(names) >= 15
    lib = dp.load()
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.check_output(["nm", "-D", "--defined-only", dp.LIB_PATH], text=True)
    exported = set(re.findall(r"\bT (dpsgd_\w+)", dyn))
    assert set(names) <= exported
    assert set(names) == set(dp.EXPORTS)


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_error_strings():
    lib = dp.load()
    for code in (dp.OK, dp.ERR_INVALID_ARG, dp.ERR_UNSUPPORTED, dp.ERR_NONFINITE, dp.ERR_HIP, 99):
        assert lib.dpsgd_error_string(code)


@pytest.mark.parametrize("kw,code", [
    (dict(layers=[(0, 8)]), dp.ERR_INVALID_ARG),
    (dict(layers=[(8, -1)]), dp.ERR_INVALID_ARG),
    (dict(layers=[]), dp.ERR_INVALID_ARG),
    (dict(dtype=7), dp.ERR_UNSUPPORTED),
    (dict(max_records=0), dp.ERR_INVALID_ARG),
    (dict(max_records=70000), dp.ERR_INVALID_ARG),
    (dict(tokens=0), dp.ERR_INVALID_ARG),
    (dict(path_policy=9), dp.ERR_UNSUPPORTED),
    (dict(sum_policy=-1), dp.ERR_UNSUPPORTED),
    (dict(layers=[(2**30, 2**30)], max_records=65535, tokens=2**30), dp.ERR_INVALID_ARG),
])
def test_plan_validation(kw, code):
    args = dict(layers=[(8, 8)], dtype=dp.DTYPE_F32, max_records=4, tokens=4, path_policy=0,
                sum_policy=0)
    args.update(kw)
    with pytest.raises(dp.DpsgdError) as e:
        dp.Plan(args["layers"], args["dtype"], args["max_records"], args["tokens"],
                args["path_policy"], args["sum_policy"])
    assert e.value.code == code


def test_path_choice_rule():
    """Gram iff T^2 < d_in*d_out; a tie takes the direct path."""
    p = dp.Plan([(64, 32), (768, 8), (4096, 4096), (16, 16), (17, 16)], dp.DTYPE_F32, 2, 16)
    assert [p.layer_info(l)[0] for l in range(5)] == [dp.PATH_GRAM, dp.PATH_GRAM, dp.PATH_GRAM,
                                                       dp.PATH_DIRECT, dp.PATH_GRAM]
    p = dp.Plan([(768, 8), (4096, 16)], dp.DTYPE_BF16, 2, 512)
    assert [p.layer_info(l)[0] for l in range(2)] == [dp.PATH_DIRECT, dp.PATH_DIRECT]
    f = dp.Plan([(64, 32)], dp.DTYPE_F32, 2, 4, dp.PATH_DIRECT)
    assert f.layer_info(0)[0] == dp.PATH_DIRECT


def test_sum_strategy_rule_and_workspace():
    # LoRA layers: keeping gradient blocks (8 B/param) beats re-reading T*(d_in+d_out) inputs
    p = dp.Plan([(4096, 16), (16, 4096)] * 128, dp.DTYPE_BF16, 256, 512)
    assert p.layer_info(0) == (dp.PATH_DIRECT, dp.SUM_STORED)
    assert p.n_params == 16777216
    assert p.ws_bytes >= 256 * 16777216 * 4
    # dense layers on the Gram path always re-read A and G
    p = dp.Plan([(4096, 4096)] * 4, dp.DTYPE_BF16, 64, 256)
    assert p.layer_info(0) == (dp.PATH_GRAM, dp.SUM_GEMM)
    assert p.ws_bytes < 64 << 20
    p = dp.Plan([(768, 8)], dp.DTYPE_F32, 16, 128, dp.PATH_AUTO, dp.SUM_GEMM)
    assert p.layer_info(0)[1] == dp.SUM_GEMM


class _Dummy:
    """Fake device pointers: validation must reject before anything touches them."""
    def __init__(self, v):
        self.v = v

    def data_ptr(self):
        return self.v


W = _Dummy(1 << 20)      # 256-byte aligned fake workspace
P = _Dummy(1 << 21)


@pytest.fixture
def plan():
    return dp.Plan([(8, 8), (8, 4)], dp.DTYPE_F32, 4, 4)


def _step(plan, **kw):
    a = dict(A=[P, P], G=[P, P], out=[P, P], ws=W, C=1.0, sigma=1.0, seed=0, step_idx=0,
             n_records=4, flags=0, stream=0, params=None, lr=0.01, normalizer=16.0)
    a.update(kw)
    return dp.step(plan, a["A"], a["G"], a["out"], a["ws"], a["C"], a["sigma"], a["seed"],
                   a["step_idx"], n_records=a["n_records"], flags=a["flags"], stream=a["stream"],
                   params=a["params"], lr=a["lr"], normalizer=a["normalizer"])


@pytest.mark.parametrize("kw", [dict(C=0.0), dict(C=-1.0), dict(C=float("nan")), dict(C=float("inf")),
                                dict(sigma=-0.1), dict(sigma=float("nan")), dict(n_records=5),
                                dict(n_records=-1), dict(ws=None), dict(ws=_Dummy((1 << 20) + 16)),
                                dict(flags=8), dict(out=[P, None]), dict(A=[P, None]),
                                dict(G=None)])
def test_step_rejects_before_launch(plan, kw):
    with pytest.raises(dp.DpsgdError) as e:
        _step(plan, **kw)
    assert e.value.code == dp.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(flags=dp.DESCENT), dict(params=[P, None]),
                                dict(params=[P, P], lr=float("nan")), dict(params=[P, P], lr=float("inf")),
                                dict(params=[P, P], normalizer=0.0), dict(params=[P, P], normalizer=-1.0),
                                dict(params=[P, P], normalizer=float("inf")),
                                dict(params=[P, P], lr=1e300, normalizer=1e-10),
                                dict(params=[P, P], lr=1e38, normalizer=1e-3),
                                dict(params=[P, P], flags=dp.NO_NOISE)])
def test_descent_rejects_before_launch(plan, kw):
    """The descent step needs one parameter buffer per layer, a finite learning rate, a finite
    normaliser > 0 whose quotient fits fp32, and the noise (an update without it would release
    the un-noised sum)."""
    with pytest.raises(dp.DpsgdError) as e:
        _step(plan, **kw)
    assert e.value.code == dp.ERR_INVALID_ARG
    for bad in (dict(params=[P, None]), dict(params=[P, P], normalizer=0.0),
                dict(params=[P, P], lr=float("nan"))):
        k = dict(params=[P, P], lr=0.01, normalizer=16.0)
        k.update(bad)
        with pytest.raises(dp.DpsgdError) as e:
            dp.noise(plan, [P, P], 1.0, 1.0, 0, 0, ws=W, stream=0, **k)
        assert e.value.code == dp.ERR_INVALID_ARG


def test_phase_entry_points_reject_before_launch(plan):
    lib = dp.load()
    with pytest.raises(dp.DpsgdError):
        dp.norms(plan, 4, 1, 3, [P, P], [P, P], W, stream=0)        # layer range
    with pytest.raises(dp.DpsgdError):
        dp.norms(plan, 4, 0, 2, [P, None], [P, P], W, stream=0)
    with pytest.raises(dp.DpsgdError):
        dp.clip(plan, 4, -2.0, W, stream=0)
    with pytest.raises(dp.DpsgdError):
        dp.clipped_sum(plan, 4, 0, 2, [P, P], [P, P], None, [P, None], W, stream=0)
    with pytest.raises(dp.DpsgdError):
        dp.noise(plan, [P, P], 1.0, float("inf"), 0, 0, stream=0)
    with pytest.raises(dp.DpsgdError):
        dp.layer_norm2(plan, 9, 0, 2, W, P, stream=0)
    assert lib.dpsgd_plan_layer_info(None, 0, None, None) == dp.ERR_INVALID_ARG
    assert lib.dpsgd_status(None, None, None) == dp.ERR_INVALID_ARG
    assert lib.dpsgd_philox_raw(0, 0, 0, 4, None, None) == dp.ERR_INVALID_ARG
    assert lib.dpsgd_philox_raw(0, 0, 2**64 - 2, 4, ctypes.c_void_p(P.v), None) == dp.ERR_INVALID_ARG
    assert lib.dpsgd_plan_num_params(None) == -1
    assert b"layer" in lib.dpsgd_last_error() or lib.dpsgd_last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(dp, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(dp, "_lib", None)
    with pytest.raises(RuntimeError):
        dp.load()


def test_segment_offsets_rejected_before_copy():
    """dpsgd_ws_segments checks the plan flag, the record count and every segment length
    (offsets[0] = 0, non-decreasing, each at most `tokens` rows) before anything is copied."""
    seg_plan = dp.Plan([(8, 8)], dp.DTYPE_F32, 3, 4, segments=True)
    fixed = dp.Plan([(8, 8)], dp.DTYPE_F32, 3, 4)
    for plan_, offs in ((fixed, [0, 2, 4]), (seg_plan, [1, 2, 4]), (seg_plan, [0, 3, 2]),
                        (seg_plan, [0, 5]), (seg_plan, [0, 1, 2, 3, 4]), (seg_plan, [0, 4, 9])):
        with pytest.raises(dp.DpsgdError) as e:
            dp.ws_segments(plan_, W, offs, stream=0)
        assert e.value.code == dp.ERR_INVALID_ARG, offs
    with pytest.raises(dp.DpsgdError) as e:
        dp.ws_segments(seg_plan, None, [0, 1], stream=0)
    assert e.value.code == dp.ERR_INVALID_ARG


def test_unknown_plan_flags_rejected():
    lib = dp.load()
    layers = (dp.LayerShape * 1)(dp.LayerShape(8, 8))
    desc = dp.PlanDesc(1, layers, dp.DTYPE_F32, 4, 4, dp.PATH_AUTO, dp.SUM_AUTO, 2)
    h, ws = ctypes.c_void_p(), ctypes.c_size_t()
    assert lib.dpsgd_plan_create(ctypes.byref(desc), ctypes.byref(h), ctypes.byref(ws)) == dp.ERR_INVALID_ARG


def test_i8_entry_points_reject_before_launch():
    """The INT8 forward's argument errors are returned on the host (no GPU is touched)."""
    lib = dp.load()
    assert dp.i8_pitch(4) == 64 and dp.i8_pitch(768) == 768 and dp.i8_pitch(770) == 832
    assert dp.i8_pitch(0) == 0 and dp.i8_pitch(32769) == 0
    for args in [(-1, 1, 8), (8, 0, 8), (8, 1, 0), (8, 1, 32769), (1 << 20, 1, 4096)]:
        with pytest.raises(dp.DpsgdError) as e:
            dp.I8Plan(*args)
        assert e.value.code == dp.ERR_INVALID_ARG
    plan = dp.I8Plan(64, 4, 128)
    assert plan.ws_bytes > 64 * 128
    fake_ws = 1 << 40          # never dereferenced: every case below fails validation first
    bad_offsets = [[1, 4], [0, 5, 3], [0, 65], [0] * 6]
    for off in bad_offsets:
        with pytest.raises(dp.DpsgdError):
            dp.i8_set_records(plan, fake_ws, off, stream=0)
    ok = dict(n_rows=8, n_records=2, A=fake_ws, k=64, wq=fake_ws, w_scale=fake_ws, n_out=16,
              tau=6.0, Y=fake_ws, stream=0)
    for change in [dict(n_rows=65), dict(n_records=5), dict(n_records=0), dict(k=129), dict(k=0),
                   dict(tau=float("nan")), dict(A=0), dict(wq=0), dict(Y=0), dict(wq=fake_ws + 8),
                   dict(n_out=-1)]:
        kw = dict(ok, **change)
        with pytest.raises(dp.DpsgdError) as e:
            dp.i8_forward(plan, fake_ws + (1 if change == {} else 0), **kw)
        assert e.value.code == dp.ERR_INVALID_ARG
    with pytest.raises(dp.DpsgdError):
        dp.i8_forward(plan, fake_ws + 16, **ok)       # misaligned workspace
    for args in [(fake_ws, 4, 0, fake_ws, fake_ws), (fake_ws, -1, 8, fake_ws, fake_ws),
                 (0, 4, 8, fake_ws, fake_ws)]:
        with pytest.raises(dp.DpsgdError):
            dp.i8_quantize_weight(*args, stream=0)
    assert lib.dpsgd_i8_pitch(64) == 64


def test_hbm_read_rejects_before_launch():
    """The streaming-read measurement aid checks its arguments on the host (no GPU is touched)."""
    fake = 1 << 40          # never dereferenced: every case below fails validation first
    for buf, nbytes, sink in [(0, 16, fake), (fake, 16, 0), (fake, 0, fake), (fake, -16, fake),
                              (fake, 24, fake), (fake + 8, 16, fake)]:
        with pytest.raises(dp.DpsgdError) as e:
            dp.hbm_read(buf, nbytes, sink, stream=0)
        assert e.value.code == dp.ERR_INVALID_ARG

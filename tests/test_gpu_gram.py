"""GPU parity of the Gram-path ghost norms of bf16 layers against the oracle.

With rows 16-byte aligned and d_in, d_out multiples of 32, records of at most 256 tokens take the
one-workgroup-per-record kernel (off-diagonal 64-token block pairs and pairs of diagonal blocks
as wavefronts) and longer ones the 128-token block-pair kernel; these cases put T off every block
multiple (5, 8, 50, 129, 150, 200, 257, 300, 384: records no longer than one 8-row copy, one, three
and four 64-token blocks, where three leaves a diagonal wavefront with a single block, and two or
three 128-token blocks), give 1 to 17 records
(more than 8 spread a layer's block pairs over workgroup ids of every XCD), and mix layer shapes,
with widths that are odd multiples of 32 (a half feature step) and multiples of 64.
Per-layer squared norms are compared with the oracle (relative 2e-3, bf16 inputs) and with the
direct path on the same data; integer inputs small enough for exact fp32 sums are compared bit
for bit.  Misaligned rows take the register kernel and must agree as well.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import datagen  # noqa: E402
import differentially_private_amd as dp  # noqa: E402
import oracle  # noqa: E402
from _helpers import TOL, host_inputs, max_rel, to_device  # noqa: E402
from datagen import BF16  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def layer_norm2(shapes, T, B, As, Gs, path, shift=False):
    plan = dp.Plan(shapes, BF16, B, T, path)
    ws = plan.workspace(DEV)

    def up(x):
        if not shift:
            return to_device(x, DEV)
        t = to_device(x.reshape(-1), DEV)
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        buf[1:].copy_(t)
        return buf[1:]
    dA = [up(a) for a in As]
    dG = [up(g) for g in Gs]
    dp.ws_init(plan, ws)
    dp.norms(plan, B, 0, len(shapes), dA, dG, ws)
    out = torch.empty(len(shapes) * B, dtype=torch.float32, device=DEV)
    dp.layer_norm2(plan, B, 0, len(shapes), ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(len(shapes), B).astype(np.float64)


@pytest.mark.parametrize("T,shapes,B", [
    (50, ((32, 64), (96, 32)), 3),
    (5, ((32, 64), (64, 96)), 4),
    (8, ((96, 32),), 3),
    (128, ((64, 64),), 9),
    (150, ((64, 96), (96, 32)), 4),
    (129, ((32, 64),), 3),
    (200, ((64, 96), (32, 32)), 5),
    (256, ((128, 256),), 17),
    (300, ((32, 64), (64, 32)), 2),
    (257, ((64, 96),), 3),
    (384, ((96, 160), (256, 64)), 9),
    (64, ((512, 512),), 1),
])
def test_gram_norms_against_oracle(T, shapes, B):
    w = datagen.Workload(name="gram", layers=shapes, layer_names=tuple("l%d" % i for i in range(len(shapes))),
                         dtype=BF16, B=B, logical_B=B, T=T, C=1.0, sigma=0.0, data_seed=300 + T + B)
    say("gram", T, shapes, B)
    As, Gs = host_inputs(w)
    want = np.stack([oracle.layer_norm2(a, g) for a, g in zip(As, Gs)])
    got = layer_norm2(shapes, T, B, As, Gs, dp.PATH_GRAM)
    direct = layer_norm2(shapes, T, B, As, Gs, dp.PATH_DIRECT)
    e, ed = max_rel(got, want), max_rel(direct, want)
    say(f"  gram {e:.2e} direct {ed:.2e}")
    assert e <= TOL[BF16] and ed <= TOL[BF16]


def test_gram_integer_exact():
    """Entries in {-1, 0, 1}, T = 50, d <= 64: every Gram entry, product and sum is an integer
    below 2^24, so the per-layer squared norms equal the oracle's exactly."""
    rng = np.random.default_rng(21)
    shapes, T, B = ((64, 32), (32, 64)), 50, 4

    def bits(x):
        return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    As = [bits(rng.integers(-1, 2, size=(B, T, a))) for a, _ in shapes]
    Gs = [bits(rng.integers(-1, 2, size=(B, T, b))) for _, b in shapes]
    want = np.stack([oracle.layer_norm2(a, g) for a, g in zip(As, Gs)])
    got = layer_norm2(shapes, T, B, As, Gs, dp.PATH_GRAM)
    assert np.array_equal(got, want), (got, want)


def test_gram_misaligned_rows_match():
    """Rows one element past a 16-byte boundary take the register kernel: same norms within
    tolerance of the oracle."""
    shapes, T, B = ((64, 96),), 200, 3
    w = datagen.Workload(name="gram_shift", layers=shapes, layer_names=("l0",), dtype=BF16, B=B,
                         logical_B=B, T=T, C=1.0, sigma=0.0, data_seed=4321)
    As, Gs = host_inputs(w)
    want = np.stack([oracle.layer_norm2(a, g) for a, g in zip(As, Gs)])
    got = layer_norm2(shapes, T, B, As, Gs, dp.PATH_GRAM, shift=True)
    assert max_rel(got, want) <= TOL[BF16]

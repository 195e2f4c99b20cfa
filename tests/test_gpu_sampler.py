"""GPU parity of the Poisson sampler against the oracle: inclusion decisions are integer
comparisons of Philox words, so the mask, the index list and the count must be bit-identical."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import differentially_private_amd as dp  # noqa: E402
from oracle import accountant as acc  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def gpu_sample(seed, step, q, n, with_mask=True):
    idx = torch.full((max(n, 1),), -1, dtype=torch.int64, device=DEV)
    cnt = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    ws = torch.empty(dp.poisson_ws_bytes(n) // 8, dtype=torch.int64, device=DEV)
    mask = torch.full((max(n, 4) + 4,), 7, dtype=torch.uint8, device=DEV) if with_mask else None
    dp.poisson_sample(seed, step, q, n, idx, cnt, ws, mask=mask)
    torch.cuda.synchronize()
    c = int(cnt.item())
    return (idx.cpu().numpy()[:c], c, mask.cpu().numpy()[:n] if with_mask else None,
            idx.cpu().numpy())


@pytest.mark.parametrize("seed,step,q,n", [(0, 0, 0.01, 1_000_000), (7, 3, 0.5, 4097), (7, 4, 0.5, 4097),
                                           (2**64 - 1, 2**40, 0.25, 1023), (5, 1, 0.0, 5000),
                                           (5, 1, 1.0, 5001), (9, 9, 0.999, 3), (1, 2, 0.37, 0),
                                           (11, 0, 0.03, 3_000_001),
                                           # more workgroup counts than the scan has threads: each
                                           # scan thread takes a run of them
                                           (13, 2, 0.05, 5_000_001), (17, 8, 0.01, 2**25 + 3)])
def test_sampler_matches_oracle(seed, step, q, n):
    print("sampler", seed, step, q, n, flush=True)
    idx, c, mask, raw = gpu_sample(seed, step, q, n)
    want = acc.poisson_sample(seed, step, q, n)
    assert c == int(want.sum())
    assert np.array_equal(idx, np.nonzero(want)[0])
    assert np.array_equal(mask.astype(bool), want)
    if c < len(raw) and n > 0:
        assert (raw[c:] == -1).all()       # nothing written past the count


def test_sampler_without_mask_and_repeat():
    a = gpu_sample(3, 5, 0.2, 100_000, with_mask=False)
    b = gpu_sample(3, 5, 0.2, 100_000, with_mask=False)
    assert a[1] == b[1] and np.array_equal(a[0], b[0])

"""The seeded input generator: determinism, window consistency, gather == fill, moments."""
import numpy as np

import datagen


def test_fill_deterministic_and_windowed():
    w = datagen.reduced(2)
    a = datagen.host_tensor(w, 1, 0)
    b = datagen.host_tensor(w, 1, 0)
    assert np.array_equal(a, b)
    part = datagen.host_tensor(w, 1, 0, first=2, n=2)
    assert np.array_equal(part, a[2:4])
    # other layer / tensor / seed give other values
    assert not np.array_equal(datagen.host_tensor(w, 2, 0)[:, :, :8], a[:, :, :8])
    assert not np.array_equal(datagen.host_tensor(w, 0, 1)[:, :, :8], datagen.host_tensor(w, 0, 0)[:, :, :8])


def test_gather_matches_fill_bf16_with_heavy_records():
    w = datagen.reduced(3)
    x = datagen.bf16_bits_to_f32(datagen.host_tensor(w, 0, 0))
    rng = np.random.default_rng(0)
    rec = rng.integers(0, w.B, 200)
    tok = rng.integers(0, w.T, 200)
    col = rng.integers(0, 4096, 200)
    g = datagen.gather(w, 0, 0, rec, tok, col)
    assert np.array_equal(g, x[rec, tok, col])


def test_moments_and_heavy_tails():
    w = datagen.workload(2)
    a = datagen.host_tensor(w, 0, 0, n=4)
    assert abs(a.mean()) < 5e-3 and abs(a.std() - 1) < 5e-3
    w3 = datagen.reduced(3)          # heavy_every = 3: records 0 and 3 are Student-t(3)
    x = datagen.bf16_bits_to_f32(datagen.host_tensor(w3, 0, 0))
    light = x[[1, 2, 4]]
    heavy = x[[0, 3]]
    assert abs(light.std() - 0.02) < 1e-3
    assert heavy.std() > 1.3 * light.std()          # t(3) has variance 3
    assert np.abs(heavy).max() > 8 * np.abs(light).max() / 5


def test_workload_shapes():
    w2 = datagen.workload(2)
    assert w2.n_params == 294912 and w2.n_layers == 48
    w3 = datagen.workload(3)
    assert w3.n_params == 16777216 and w3.n_layers == 256
    assert abs(w3.input_bytes_per_batch() - 275.95e9) < 0.01e9
    w4 = datagen.workload(4)
    assert w4.n_params == 67108864
    w5 = datagen.workload(5)
    assert w5.n_params == 393216 and w5.n_phys == 16

"""The seeded input generator (host side): determinism, random access, moments."""
import numpy as np

from synth import synth


def test_deterministic_and_random_access():
    a = synth.generate(7, 3, 40, 96, *synth.DIST_MOE)
    b = synth.generate(7, 3, 40, 96, *synth.DIST_MOE)
    assert np.array_equal(a, b)
    sub = synth.generate(7, 3, 40, 96, *synth.DIST_MOE, rows=[5, 17, 39], cols=[0, 33, 95])
    assert np.array_equal(sub, a[np.ix_([5, 17, 39], [0, 33, 95])])
    assert not np.array_equal(a, synth.generate(7, 4, 40, 96, *synth.DIST_MOE))


def test_moments():
    z = synth._irwin_hall12(synth.stream_key(1, 2), np.arange(400000))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01 and np.abs(z).max() <= 6.0
    y = np.linspace(-4, 4, 4001)
    assert np.max(np.abs(synth.exp_det(y) / np.exp(y) - 1.0)) < 1e-14
    w = synth.generate(9, 1, 512, 256, 1.0, 0.0, 0.0, 1.0)
    f = (w.astype(np.uint32) << 16).view(np.float32)
    assert abs(f.std() - 1.0) < 0.02


def test_outlier_rate():
    w = synth.generate(11, 1, 256, 1024, 1.0, 0.0, 0.01, 1000.0)
    f = np.abs((w.astype(np.uint32) << 16).view(np.float32))
    rate = (f > 10.0).mean()
    assert 0.007 < rate < 0.013

"""Pins of oracle.norm.rms_norm (the fused pre-attention norm, Runway
Characters paper §4.4): a library routine (torch's float64 rms_norm), closed
forms and invariants."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle.norm import rms_norm


def test_matches_torch_rms_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 128)) * rng.uniform(0.01, 30, size=(7, 3, 1))
    w = rng.uniform(0.5, 1.5, size=128)
    for eps in (1e-6, 1e-2):
        ref = F.rms_norm(torch.from_numpy(x), (128,), weight=torch.from_numpy(w), eps=eps).numpy()
        assert np.max(np.abs(rms_norm(x, w, eps) - ref)) < 1e-13


def test_closed_forms():
    d = 64
    # alternating +-a: mean square a^2, so with eps = 0 every entry is +-1 times w
    a = 3.25
    x = np.tile([a, -a], d // 2)
    w = np.arange(1, d + 1) / 8.0
    np.testing.assert_allclose(rms_norm(x, w, 0.0), np.tile([1.0, -1.0], d // 2) * w, rtol=0, atol=1e-15)
    # unit weights, eps = 0: every row comes out with mean square exactly 1
    rng = np.random.default_rng(1)
    y = rms_norm(rng.standard_normal((5, d)) * 7.0, np.ones(d), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-14)
    # eps enters inside the root: a zero row stays zero, a row of ones scales by 1/sqrt(1 + eps)
    assert not rms_norm(np.zeros(d), np.ones(d), 1e-6).any()
    np.testing.assert_allclose(rms_norm(np.ones(d), np.ones(d), 0.25), 1 / np.sqrt(1.25), rtol=1e-15)


def test_scale_invariance_and_row_independence():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2, 32))
    w = rng.uniform(0.5, 2.0, size=32)
    base = rms_norm(x, w, 0.0)
    np.testing.assert_allclose(rms_norm(x * 1e3, w, 0.0), base, rtol=1e-13)
    # each (token, head) row is normalized on its own: scaling one row leaves the others
    x2 = x.copy()
    x2[1, 0] *= 50.0
    y2 = rms_norm(x2, w, 0.0)
    assert np.array_equal(np.delete(y2.reshape(8, 32), 2, axis=0), np.delete(base.reshape(8, 32), 2, axis=0))

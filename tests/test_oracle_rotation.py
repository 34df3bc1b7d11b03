"""Pins for the oracle's Walsh-Hadamard rotation before MXFP4 (CPU only).

The rotation is the alternative to promotion that the pages name for
handling outliers (reading R34)."""

import numpy as np
import pytest
from scipy.linalg import hadamard

import mxq_inputs
from oracle import attention as A
from oracle import formats as F


@pytest.mark.parametrize("D", [32, 64, 128])
def test_fast_transform_equals_the_sylvester_matrix(D):
    # small integers: every butterfly sum is exact, so the transform equals
    # the matrix product exactly and only the final scaling rounds
    x = np.random.default_rng(D).integers(-9, 10, size=(5, D)).astype(np.float32)
    want = ((x.astype(np.float64) @ hadamard(D)).astype(np.float32) * np.float32(1 / np.sqrt(D))).astype(np.float32)
    assert np.array_equal(F.hadamard_rotate(x), want)


def test_rotation_is_orthonormal():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    y = rng.standard_normal((4, 128)).astype(np.float32)
    rx, ry = F.hadamard_rotate(x), F.hadamard_rotate(y)
    assert np.allclose(F.hadamard_rotate(rx), x, atol=1e-5)             # H/sqrt(D) is its own inverse
    assert np.allclose((rx * ry).sum(-1), (x * y).sum(-1), rtol=1e-5, atol=1e-4)  # dot products kept


def test_an_outlier_channel_is_spread_over_the_row():
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 37] = 20.0
    r = F.hadamard_rotate(x)
    assert np.allclose(np.abs(r), 20.0 / np.sqrt(128), rtol=1e-6)


def test_rotation_cuts_the_low_bit_error_on_outlier_channels():
    """Q/K with outlier channels x20 (the workload recipe): all-low-bit
    attention over rotated operands is much closer to exact attention."""
    cfg = mxq_inputs.make_prefill("llama8b", N=512, n_valid=512, Hq=4, Hkv=1, B=1)
    args = (cfg["q"], cfg["k"], cfg["v"], 512, 128, 64, True)
    exact = A.attn_exact_ref(cfg["q"], cfg["k"], cfg["v"], 512, True)
    plain, _ = A.attn_mixed_ref(*args, mode=A.MODE_ALL_LOWBIT)
    rot, _ = A.attn_mixed_ref(*args, mode=A.MODE_ALL_LOWBIT, rotate=True)
    e_plain = np.linalg.norm(plain - exact) / np.linalg.norm(exact)
    e_rot = np.linalg.norm(rot - exact) / np.linalg.norm(exact)
    assert e_rot < 0.7 * e_plain, (e_rot, e_plain)

"""Pins for the oracle's sign diagonal and Walsh-Hadamard rotation (CPU only)."""

import json
import os

import numpy as np
import pytest
from scipy.linalg import hadamard as scipy_hadamard

from oracle import rotation as rot
from oracle import signs as sg

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


@pytest.mark.parametrize("d", [2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester(d):
    """Our popcount-parity H equals scipy's Sylvester construction."""
    np.testing.assert_array_equal(rot.hadamard(d), scipy_hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [8, 128, 256])
def test_butterflies_equal_dense_matrix(d):
    """The in-place stages of [Spec] 'Hadamard Transform Detail' compute H x."""
    eye = np.eye(d)
    y, _ = rot.fwht_stages(eye)
    np.testing.assert_array_equal(y, scipy_hadamard(d).astype(np.float64))


def test_orthogonality_and_self_inverse():
    d = 128
    H = rot.hadamard(d)
    np.testing.assert_array_equal(H @ H.T, d * np.eye(d))
    np.testing.assert_allclose((H / np.sqrt(d)) @ (H / np.sqrt(d)), np.eye(d), atol=1e-14)


def test_flop_counts_printed_on_spec():
    g = GOLDEN["fwht_flops_d128"]
    _, ops = rot.fwht_stages(np.zeros(128))
    assert ops == g["fwht"] == 128 * 7
    assert 128 * 128 == g["dense"]


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_is_orthogonal(d):
    s = sg.signs(42, d)
    R = np.stack([rot.forward64(e, s) for e in np.eye(d)], axis=1)
    np.testing.assert_allclose(R @ R.T, np.eye(d), atol=1e-13)
    Rt = np.stack([rot.inverse64(e, s) for e in np.eye(d)], axis=1)
    np.testing.assert_allclose(Rt, R.T, atol=1e-14)
    x = np.random.default_rng(1).standard_normal(d)
    np.testing.assert_allclose(np.linalg.norm(rot.forward64(x, s)), np.linalg.norm(x), rtol=1e-14)
    np.testing.assert_allclose(rot.inverse64(rot.forward64(x, s), s), x, atol=1e-13)


def test_signs_applied_before_transform():
    """[Spec] 'As-Built Notes': R e_i = s_i H[:, i] / sqrt(d) (signs first).  Signs
    applied after H would give s * H[:, i] / sqrt(d) instead."""
    d = 128
    s = sg.signs(42, d)
    H = rot.hadamard(d)
    for i in (0, 5, 77):
        e = np.zeros(d)
        e[i] = 1.0
        np.testing.assert_allclose(rot.forward64(e, s), s[i] * H[:, i] / np.sqrt(d), atol=1e-15)


def test_blockwise_d256_uses_sign_slices():
    d = 256
    s = sg.signs(7, d)
    x = np.random.default_rng(2).standard_normal(d)
    y = rot.forward64(x, s)
    H = rot.hadamard(128) / np.sqrt(128)
    np.testing.assert_allclose(y[:128], H @ (s[:128] * x[:128]), atol=1e-13)
    np.testing.assert_allclose(y[128:], H @ (s[128:] * x[128:]), atol=1e-13)


def test_canonical_f32_stages_close_to_f64():
    x = np.random.default_rng(3).standard_normal((64, 128)).astype(np.float32)
    y32 = rot.fwht_stages_f32(x)
    y64, _ = rot.fwht_stages(x.astype(np.float64))
    np.testing.assert_allclose(y32, y64, rtol=0, atol=1e-5 * np.max(np.abs(y64)))


def test_splitmix64_published_first_output():
    """SplitMix64 from state 0: first output 0xE220A8397B1DCDAF (reference C of
    Steele, Lea and Flood's generator as distributed with Vigna's xoshiro code)."""
    assert sg.splitmix64(0, 1)[0] == 0xE220A8397B1DCDAF


def test_signs_deterministic_and_balanced():
    a = sg.signs(42, 128)
    b = sg.signs(42, 128)
    assert a.dtype == np.int8 and set(np.unique(a)) <= {-1, 1}
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, sg.signs(43, 128))
    neg = np.mean([np.mean(sg.signs(seed, 128) < 0) for seed in range(200)])
    assert abs(neg - 0.5) < 0.01

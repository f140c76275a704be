"""Pins of the whole-vector mode ([Spec] "Step 1": one d x d rotation with d =
head_dim; "Step 2": one codebook per (head_dim, bits)) at d = 256."""

import numpy as np
import pytest

from oracle import codebook as o_cb
from oracle import codec
from oracle import rotation
from oracle import signs as o_signs

SEED = 42
D = 256


def test_whole_rotation_is_the_dense_signed_hadamard():
    s = o_signs.signs(SEED, D)
    R = rotation.hadamard(D) * s[None, :].astype(float) / np.sqrt(D)
    x = np.random.default_rng(0).standard_normal((4, D))
    np.testing.assert_allclose(rotation.forward64_whole(x, s), x @ R.T, atol=1e-12)
    np.testing.assert_allclose(R @ R.T, np.eye(D), atol=1e-12)
    np.testing.assert_allclose(rotation.inverse64_whole(rotation.forward64_whole(x, s), s), x,
                               atol=1e-12)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_whole_encode_matches_fp64_math_mode(bits):
    """Canonical fp32 codes equal the fp64 codes of the dense rotation, except for
    rare adjacent flips next to a boundary; likewise the fp16 norms."""
    x = np.random.default_rng(bits).standard_normal((2000, D)).astype(np.float32)
    s = o_signs.signs(SEED, D)
    b, _ = o_cb.codebook(bits, D)
    codes, n16, _ = codec.encode_mse_whole(x, s, b)
    x64 = x.astype(np.float64)
    R = rotation.hadamard(D) * s[None, :].astype(float) / np.sqrt(D)
    n = np.linalg.norm(x64, axis=-1)
    u64 = (x64 @ R.T) / n[:, None]
    c64 = np.searchsorted(b.astype(np.float64), u64, side="left")
    diff = codes.astype(int) - c64
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 3
    # the fp16 norm is RN16 of the fp32 norm: equal to RN16 of the fp64 norm except
    # where the two round apart (rare)
    assert np.count_nonzero(n16 != n.astype(np.float16)) <= 3


@pytest.mark.parametrize("bits", [2, 4])
def test_whole_roundtrip_mse_is_the_d256_distortion(bits):
    """R is orthogonal, so u is uniform on the 256-sphere: the round-trip MSE is
    d * D of the d = 256 codebook under the exact sphere marginal (d - 3) / 2."""
    x = np.random.default_rng(10 + bits).standard_normal((2048, D)).astype(np.float32)
    s = o_signs.signs(SEED, D)
    b, c = o_cb.codebook(bits, D)
    codes, n16, _ = codec.encode_mse_whole(x, s, b)
    xh = codec.decode_mse_whole(codes, n16, s, c)
    mse = np.mean(np.sum((xh - x) ** 2, -1)) / np.mean(np.sum(x.astype(float) ** 2, -1))
    want = D * o_cb.distortion(b, c, m=(D - 3) / 2)
    assert abs(mse / want - 1) < 0.03, (mse, want)


def test_whole_mode_beats_the_blocked_mode_at_equal_bits():
    """The d = 256 codebook fits the 256-dimensional marginal: its round-trip MSE is
    no worse than two 128-blocks with the d = 128 codebook (which also store two
    norms), within sampling noise."""
    x = np.random.default_rng(5).standard_normal((4096, D)).astype(np.float32)
    s = o_signs.signs(SEED, D)
    b2, c2 = o_cb.codebook(2, D)
    cw, nw, _ = codec.encode_mse_whole(x, s, b2)
    ew = np.mean(np.sum((codec.decode_mse_whole(cw, nw, s, c2) - x) ** 2, -1))
    b1, c1 = o_cb.codebook(2, 128)
    cb_, nb, _ = codec.encode_mse(x, s, b1)
    eb = np.mean(np.sum((codec.decode_mse(cb_, nb, s, c1) - x) ** 2, -1))
    assert ew <= eb * 1.01, (ew, eb)


def test_whole_zero_vector():
    b, c = o_cb.codebook(3, D)
    codes, n16, u = codec.encode_mse_whole(np.zeros((2, D), np.float32), o_signs.signs(SEED, D), b)
    assert np.all(n16 == 0) and np.all(u == 0) and np.all(codes == 3)

"""Pins of the whole-vector mode at a head_dim d that is not a power of two ([Spec]
"Hadamard Transform Detail": zero-pad to d' = the next power of two, transform,
and drop the padding again after the inverse).  The codes are those of the d'
transform with the d' codebook; one norm per vector.

The oracle runs the padded vector through its butterflies; the pins below use the
dense d' x d' matrix built from the Sylvester definition instead, restricted to the
first d columns, the exact distribution of a padded rotated coordinate, and the
orthogonality of the transform."""

import numpy as np
import pytest

from oracle import codebook as o_cb
from oracle import codec
from oracle import rotation
from oracle import signs as o_signs

SEED = 42
DIMS = [80, 96, 120, 136, 192, 200, 248]


def _dense_columns(d):
    """A = (H_d' diag(s) / sqrt(d'))[:, :d]: the padded transform as a d' x d matrix."""
    dp = codec.pow2_length(d)
    s = o_signs.signs(SEED, dp)
    R = rotation.hadamard(dp) * s[None, :].astype(float) / np.sqrt(dp)
    return R[:, :d], s, dp


def test_pow2_length():
    got = [codec.pow2_length(d) for d in (1, 2, 3, 80, 96, 127, 128, 129, 192, 255, 256)]
    assert got == [1, 2, 4, 128, 128, 128, 128, 256, 256, 256, 256]


@pytest.mark.parametrize("d", DIMS)
def test_padded_transform_has_orthonormal_columns(d):
    """A^T A = I_d: the padded transform keeps the norm, so one norm per vector is
    the norm of the d inputs, and the exact inverse returns zeros in the padding."""
    A, s, dp = _dense_columns(d)
    np.testing.assert_allclose(A.T @ A, np.eye(d), atol=1e-12)
    x = np.random.default_rng(d).standard_normal((8, d))
    y = rotation.forward64_whole(codec.pad_pow2(x), s)
    np.testing.assert_allclose(y, x @ A.T, atol=1e-12)
    back = rotation.inverse64_whole(y, s)
    np.testing.assert_allclose(back[:, :d], x, atol=1e-12)
    assert np.max(np.abs(back[:, d:])) < 1e-12


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d", DIMS)
def test_padded_encode_matches_the_dense_fp64_codes(d, bits):
    """Canonical fp32 codes of the padded vector equal searchsorted of the fp64 dense
    u = A x / |x| in the d' table, except for rare adjacent flips at a boundary; the
    fp16 norm is RN16 of the fp64 norm of the d inputs except in rare rounding cases."""
    A, s, dp = _dense_columns(d)
    x = np.random.default_rng(100 + d + bits).standard_normal((1500, d)).astype(np.float32)
    b, _ = o_cb.codebook(bits, dp)
    codes, n16, _ = codec.encode_mse_whole(x, s, b)
    assert codes.shape == (1500, dp) and n16.shape == (1500,)
    x64 = x.astype(np.float64)
    n = np.linalg.norm(x64, axis=-1)
    c64 = np.searchsorted(b.astype(np.float64), (x64 @ A.T) / n[:, None], side="left")
    diff = codes.astype(int) - c64
    assert np.all(np.abs(diff) <= 1) and np.count_nonzero(diff) <= 3
    assert np.count_nonzero(n16 != n.astype(np.float16)) <= 3


@pytest.mark.parametrize("d", [96, 192])
def test_padded_decode_is_the_dense_transpose(d):
    """x_hat = A^T (n16 c[code]): the first d outputs of the inverse d' transform."""
    A, s, dp = _dense_columns(d)
    rng = np.random.default_rng(d)
    b, c = o_cb.codebook(3, dp)
    codes = rng.integers(0, 8, (20, dp)).astype(np.uint8)
    n16 = rng.uniform(0.5, 4.0, 20).astype(np.float16)
    want = (c.astype(np.float64)[codes] * n16.astype(np.float64)[:, None]) @ A
    got = codec.decode_mse_whole(codes, n16, s, c, head_dim=d)
    assert got.shape == (20, d)
    np.testing.assert_allclose(got, want, atol=1e-12)


def _padded_coordinate_mse(b, c, d, dp):
    """E (u - Q(u))^2 for one rotated coordinate of a padded isotropic vector:
    u = a w with a = sqrt(d / d') and w distributed as one coordinate of a uniform
    unit d-vector (density prop. to (1 - w^2)^((d-3)/2)).  In w the quantizer has
    boundaries b / a and values c / a, so the error is a^2 times their distortion."""
    a = np.sqrt(d / dp)
    return a * a * o_cb.distortion(np.asarray(b, np.float64) / a,
                                   np.asarray(c, np.float64) / a, m=(d - 3) / 2)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("d", [96, 192])
def test_padded_rotated_domain_mse_is_the_scaled_marginal_distortion(d, bits):
    """For x ~ N(0, I_d) the rotated vector is A x with |A x| = |x|, and each row of
    A has squared length d / d', so a rotated coordinate over |x| is sqrt(d / d')
    times a unit-d-vector coordinate, independent of |x|.  The error of the full
    d' decode against the padded input (the rotated-domain error, by
    orthogonality) is then d' times the distortion of that law."""
    dp = codec.pow2_length(d)
    s = o_signs.signs(SEED, dp)
    x = np.random.default_rng(7 * d + bits).standard_normal((4096, d)).astype(np.float32)
    b, c = o_cb.codebook(bits, dp)
    codes, n16, _ = codec.encode_mse_whole(x, s, b)
    full = codec.decode_mse_whole(codes, n16, s, c)
    err = np.mean(np.sum((full - codec.pad_pow2(x).astype(np.float64)) ** 2, -1))
    rel = err / np.mean(np.sum(x.astype(np.float64) ** 2, -1))
    want = dp * _padded_coordinate_mse(b, c, d, dp)
    assert abs(rel / want - 1) < 0.03, (rel, want)
    # dropping the padding projects the error: the d outputs never do worse
    xh = codec.decode_mse_whole(codes, n16, s, c, head_dim=d)
    assert np.mean(np.sum((xh - x) ** 2, -1)) <= err


@pytest.mark.parametrize("d", [96, 192])
def test_padded_coordinates_fit_the_d_prime_table(d):
    """A padded rotated coordinate has variance 1/d' (not 1/d), so the d' table
    quantizes it with less error than the table built for d itself."""
    dp = codec.pow2_length(d)
    bp, cp = o_cb.codebook(4, dp)
    bd, cd = o_cb.codebook(4, d)
    assert _padded_coordinate_mse(bp, cp, d, dp) < _padded_coordinate_mse(bd, cd, d, dp)


def test_padded_zero_vector():
    b, c = o_cb.codebook(3, 256)
    s = o_signs.signs(SEED, 256)
    codes, n16, u = codec.encode_mse_whole(np.zeros((2, 192), np.float32), s, b)
    assert codes.shape == (2, 256) and np.all(n16 == 0) and np.all(u == 0)
    assert np.all(codes == 3)
    assert np.all(codec.decode_mse_whole(codes, n16, s, c, head_dim=192) == 0)

"""Pins of the oracle's encoder variants ([turboq] "Encode pipeline"): the second
sign vector s2 applied after the normalized butterflies (step 2), and the
corrected norm grp_norm / recon_norm (step 4).  Each is checked against what the
mathematics fixes, not against a retyped formula."""

import numpy as np
import pytest

from oracle import attention as o_att
from oracle import codebook as o_cb
from oracle import codec
from oracle import rotation
from oracle import signs as o_signs

SEED = 42


def _x(n, d=128, seed=0):
    return np.random.default_rng(seed).standard_normal((n, d)).astype(np.float32)


def test_second_signs_are_a_fresh_pm1_vector():
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    assert set(np.unique(s2)) <= {-1, 1}
    assert not np.array_equal(s1, s2)
    assert 40 <= int(np.sum(s2 < 0)) <= 88
    np.testing.assert_array_equal(o_signs.signs2(SEED, 128), s2)      # deterministic
    assert not np.array_equal(o_signs.signs2(SEED + 1, 128), s2)


def test_two_sign_rotation_is_the_orthogonal_matrix_d2_h_d1():
    """forward64 with s2 equals the dense D2 H D1 / sqrt(128) (built from the
    Sylvester matrix), is orthogonal, and inverse64 is its transpose."""
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    R = np.diag(s2.astype(float)) @ rotation.hadamard(128) @ np.diag(s1.astype(float))
    R /= np.sqrt(128)
    x = np.random.default_rng(1).standard_normal((5, 128))
    np.testing.assert_allclose(rotation.forward64(x, s1, s2), x @ R.T, atol=1e-12)
    np.testing.assert_allclose(R @ R.T, np.eye(128), atol=1e-12)
    np.testing.assert_allclose(rotation.inverse64(rotation.forward64(x, s1, s2), s1, s2), x,
                               atol=1e-12)


def test_all_plus_second_signs_reduce_to_one_sign():
    x = _x(64)
    s1 = o_signs.signs(SEED, 128)
    b, c = o_cb.codebook(3)
    one = codec.encode_mse(x, s1, b)
    two = codec.encode_mse(x, s1, b, np.ones(128, np.int8))
    for a, z in zip(one, two):
        np.testing.assert_array_equal(a, z)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_second_signs_mirror_codes_through_the_symmetric_codebook(bits):
    """u(two-sign) = s2 * u(one-sign) exactly, and the Lloyd-Max table is mirror
    symmetric, so where s2 = -1 the code becomes L - 1 - code (no exact ties in
    continuous data); where s2 = +1 it is unchanged."""
    x = _x(200, seed=bits)
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    b, c = o_cb.codebook(bits)
    L = 1 << bits
    one, n1, u1 = codec.encode_mse(x, s1, b)
    two, n2, u2 = codec.encode_mse(x, s1, b, s2)
    np.testing.assert_array_equal(u2, u1 * s2.astype(np.float32))
    np.testing.assert_array_equal(n1, n2)
    flip = np.broadcast_to(s2 < 0, one.shape)
    np.testing.assert_array_equal(two[flip], L - 1 - one[flip].astype(int))
    np.testing.assert_array_equal(two[~flip], one[~flip])


@pytest.mark.parametrize("bits", [2, 4])
def test_two_sign_roundtrip_mse_matches_codebook_distortion(bits):
    """R is orthogonal, so R x of a Gaussian x is Gaussian and the round-trip MSE is
    d * D of the codebook under the sphere marginal, as for one sign vector."""
    x = _x(1024, seed=10 + bits)
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    b, c = o_cb.codebook(bits)
    codes, n16, _ = codec.encode_mse(x, s1, b, s2)
    xh = codec.decode_mse(codes, n16, s1, c, s2)
    mse = np.mean(np.sum((xh - x) ** 2, axis=-1)) / np.mean(np.sum(x.astype(float) ** 2, -1))
    want = 128 * o_cb.distortion(b, c, m=(128 - 3) / 2)
    assert abs(mse / want - 1) < 0.03, (mse, want)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_corrected_norm_restores_the_input_norm(bits):
    """Step 4: with the stored norm n / ||c[codes]||, the decoded block's norm is the
    input norm up to the fp16 rounding of the stored value (|ratio - 1| <= 2^-11);
    without it the decoded norm is n * ||c[codes]||, short by the codebook's
    distortion (about sqrt(1 - d D))."""
    x = _x(500, seed=20 + bits)
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    b, c = o_cb.codebook(bits)
    n_in = np.linalg.norm(x.astype(np.float64), axis=-1)
    for s2_ in (None, s2):
        codes, nc, _ = codec.encode_mse(x, s1, b, s2_, c, norm_correct=True)
        xh = codec.decode_mse(codes, nc, s1, c, s2_)
        ratio = np.linalg.norm(xh, axis=-1) / n_in
        assert np.max(np.abs(ratio - 1)) <= 2.0 ** -11
        codes_p, npl, _ = codec.encode_mse(x, s1, b, s2_)
        np.testing.assert_array_equal(codes_p, codes)      # the codes do not change
        plain = np.linalg.norm(codec.decode_mse(codes_p, npl, s1, c, s2_), axis=-1) / n_in
        short = np.sqrt(1 - 128 * o_cb.distortion(b, c, m=(128 - 3) / 2))
        assert abs(np.mean(plain) / short - 1) < 0.01, (np.mean(plain), short)


def test_corrected_norm_equals_fp64_quotient_up_to_fp16_rounding():
    """The canonical fp32 quotient rounds to the same fp16 as the fp64 quotient
    ||x|| / ||c[codes]|| except in rare fp16 rounding ties."""
    x = _x(4000, seed=7)
    s1 = o_signs.signs(SEED, 128)
    b, c = o_cb.codebook(4)
    codes, nc, _ = codec.encode_mse(x, s1, b, None, c, norm_correct=True)
    r64 = np.linalg.norm(np.asarray(c, np.float32).astype(np.float64)[codes], axis=-1)
    q64 = (np.linalg.norm(x.astype(np.float64), axis=-1) / r64).astype(np.float16)
    assert np.count_nonzero(q64 != nc[..., 0]) <= 4


def test_zero_block_with_corrected_norm_is_zero():
    x = np.zeros((2, 128), np.float32)
    b, c = o_cb.codebook(2)
    codes, nc, _ = codec.encode_mse(x, o_signs.signs(SEED, 128), b, None, c, norm_correct=True)
    assert np.all(nc == 0) and np.all(codes == 1)


def test_two_sign_fused_attention_equals_bruteforce():
    """<q, R^T k'> = <R q, k'> for R = D2 H D1 / sqrt(128) as well: the fused
    rotated-domain attention equals softmax(q K_hat^T) V_hat on the decoded cache."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T = 2, 4, 2, 37
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    bk, ck = o_cb.codebook(4)
    bv, cv = o_cb.codebook(2)
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    kc, kn, _ = codec.encode_mse(k, s1, bk, s2, ck, norm_correct=True)
    vc, vn, _ = codec.encode_mse(v, s1, bv, s2, cv, norm_correct=True)
    kp, vp = codec.pack(kc, 4), codec.pack(vc, 2)
    q = rng.standard_normal((B, Hq, 128))
    lens = [T, 20]
    a = o_att.attend_fused(q, kp, kn, vp, vn, lens, 4, 2, ck, cv, s1, 0.09, s2=s2)
    z = o_att.attend_bruteforce(q, kp, kn, vp, vn, lens, 4, 2, ck, cv, s1, 0.09, s2=s2)
    np.testing.assert_allclose(a, z, atol=1e-12)
    # and the second sign vector matters: the one-sign attention differs
    w = o_att.attend_fused(q, kp, kn, vp, vn, lens, 4, 2, ck, cv, s1, 0.09)
    assert np.max(np.abs(w - a)) > 1e-2


def test_u8_second_signs_match_the_rotation():
    x = _x(50, seed=8)
    s1, s2 = o_signs.signs(SEED, 128), o_signs.signs2(SEED, 128)
    codes, sc = codec.encode_u8(x, s1, s2)
    xh = codec.decode_u8(codes, sc, s1, s2)
    rel = np.linalg.norm(xh - x, axis=-1) / np.linalg.norm(x.astype(float), axis=-1)
    assert np.max(rel) < 0.01          # 8-bit grid, about 0.3 % typical
    wrong = codec.decode_u8(codes, sc, s1)
    assert np.min(np.linalg.norm(wrong - x, axis=-1) / np.linalg.norm(x, axis=-1)) > 0.5

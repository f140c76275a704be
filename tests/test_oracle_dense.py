"""Pins of the dense-rotation oracle (oracle/dense.py) against what the mathematics
fixes, independently of the oracle's own formulas:

* the Box-Muller normals have the moments of N(0, 1) and are uncorrelated;
* R is orthogonal, and R^T G is upper triangular with a positive diagonal (the
  characterization of the sign-fixed QR factor), computed here by a plain
  Gram-Schmidt of G's columns in fp64;
* the codes are the nearest centroids of u = R x / ||x|| (Lloyd-Max boundaries are
  the midpoints between neighbouring centroids), checked by brute force;
* orthogonality makes the decode error exactly n ||u - c[codes]||;
* the round-trip mean squared error matches the codebook's distortion for dim d;
* the stored norm is the same canonical fp32 norm as the whole-vector mode's.
"""

import numpy as np
import pytest

from oracle import codebook as o_cb
from oracle import codec
from oracle import dense


def test_normals_moments():
    z = dense.normals(42, 200_000, 256)
    assert abs(z.mean()) < 0.01
    assert abs(z.var() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05                  # Gaussian kurtosis
    assert abs(np.corrcoef(z[0::2], z[1::2])[0, 1]) < 0.01     # the pair's two normals


def _gram_schmidt(g):
    q = np.zeros_like(g)
    for k in range(g.shape[1]):
        v = g[:, k].copy()
        for i in range(k):
            v -= (q[:, i] @ g[:, k]) * q[:, i]
        q[:, k] = v / np.linalg.norm(v)
    return q


@pytest.mark.parametrize("d", [24, 96, 160])
def test_rotation_is_the_sign_fixed_qr_factor(d):
    r = dense.dense_rotation(42, d)
    assert np.max(np.abs(r @ r.T - np.eye(d))) < 1e-12
    assert np.max(np.abs(r.T @ r - np.eye(d))) < 1e-12
    g = dense.normals(42, d * d, 2 * d).reshape(d, d)
    t = r.T @ g
    assert np.max(np.abs(np.tril(t, -1))) < 1e-9
    assert np.all(np.diag(t) > 0)
    # classical Gram-Schmidt of G's columns gives the same Q (positive diagonal)
    assert np.max(np.abs(_gram_schmidt(g) - r)) < 1e-8


def test_rotation_depends_on_seed_and_dim():
    a, b = dense.dense_rotation(42, 96), dense.dense_rotation(42, 96)
    assert np.array_equal(a, b)
    assert np.max(np.abs(a - dense.dense_rotation(43, 96))) > 0.1
    assert dense.dense_rotation(42, 160).shape == (160, 160)


@pytest.mark.parametrize("d,bits", [(96, 4), (96, 2), (160, 3), (40, 4)])
def test_codes_are_nearest_centroids_and_decode_error(d, bits):
    rng = np.random.default_rng(d + bits)
    x = rng.standard_normal((300, d)).astype(np.float32) * rng.uniform(0.1, 10, (300, 1)).astype(np.float32)
    b, c = o_cb.codebook(bits, d)
    r32 = dense.rotation_f32(42, d)
    codes, n16, u = dense.encode_dense(x, r32, b)
    # u is R x / n (fp64), and the code is the nearest centroid of u
    n = codec.norm_f32(codec.pad_pow2(x)).astype(np.float64)
    np.testing.assert_allclose(u, (x.astype(np.float64) @ r32.astype(np.float64).T) / n[:, None],
                               rtol=1e-12, atol=1e-15)
    c64 = np.asarray(c, np.float32).astype(np.float64)
    near = np.argmin(np.abs(u[..., None] - c64[None, None, :]), axis=-1)
    assert np.mean(near != codes) < 1e-4          # only ties of the fp32 midpoints
    # R orthogonal (to fp32 rounding): ||x_hat - x|| = n16 ||c[codes] - u n / n16||
    xh = dense.decode_dense(codes, n16, r32, c)
    lhs = np.linalg.norm(xh - x.astype(np.float64) @ (r32.astype(np.float64).T @ r32.astype(np.float64)).T, axis=-1)
    rhs = np.linalg.norm(c64[codes] * n16.astype(np.float64)[:, None] - u * n[:, None], axis=-1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-9)


@pytest.mark.parametrize("d,bits", [(96, 4), (160, 2)])
def test_roundtrip_mse_matches_distortion(d, bits):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4000, d)).astype(np.float32)
    b, c = o_cb.codebook(bits, d)
    r32 = dense.rotation_f32(42, d)
    codes, n16, _ = dense.encode_dense(x, r32, b)
    xh = dense.decode_dense(codes, n16, r32, c)
    rel = np.sum((xh - x) ** 2, axis=-1) / np.sum(x.astype(np.float64) ** 2, axis=-1)
    # per-coordinate distortion of the dim-d codebook, times d coordinates
    want = d * o_cb.distortion(b, c, o_cb.m_sphere(d))
    assert abs(rel.mean() / want - 1.0) < 0.05


def test_norm_matches_whole_vector_mode():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 96)).astype(np.float32)
    b, _ = o_cb.codebook(4, 96)
    _, n_dense, _ = dense.encode_dense(x, dense.rotation_f32(42, 96), b)
    bw, _ = o_cb.codebook(4, 128)
    from oracle import signs
    _, n_whole, _ = codec.encode_mse_whole(x, signs.signs(42, 128), bw)
    assert np.array_equal(n_dense.view(np.uint16), n_whole.view(np.uint16))


def test_pack_dense_pads_with_code_zero():
    codes = np.arange(96, dtype=np.uint8).reshape(1, 96) % 16
    p = dense.pack_dense(codes, 4)
    assert p.shape == (1, 1, 64)
    back = codec.unpack(p, 4)
    assert np.array_equal(back[0, :96], codes[0]) and np.all(back[0, 96:] == 0)


def _dense_cache(rng, B, H, T, d, bits, r32):
    x = rng.standard_normal((B, H, T, d)).astype(np.float32)
    b, c = o_cb.codebook(bits, d)
    codes, norms, _ = dense.encode_dense(x.reshape(-1, d), r32, b)
    return codes.reshape(B, H, T, d), norms.reshape(B, H, T), c


def test_attend_dense_is_the_fused_rotated_domain_attention():
    """softmax(scale q K^T) V over decoded vectors equals the fused form computed in the
    rotated domain (q' = R q, scores n <q', c[code]>, o' = sum p n c[code], out = R^T o'):
    the identity <q, R^T k'> = <R q, k'>.  A transposed R or a wrong GQA map breaks it."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, T, d = 2, 6, 3, 37, 40
    r = dense.rotation_f32(42, d)
    kc, kn, ck = _dense_cache(rng, B, Hkv, T, d, 4, r)
    vc, vn, cv = _dense_cache(rng, B, Hkv, T, d, 2, r)
    q = rng.standard_normal((B, Hq, d))
    lens = [37, 20]
    scale = 1 / np.sqrt(d)
    got = dense.attend_dense(q, kc, kn, vc, vn, lens, r, ck, cv, scale)
    r64 = r.astype(np.float64)
    ckf, cvf = np.asarray(ck, np.float32).astype(np.float64), np.asarray(cv, np.float32).astype(np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            n = lens[b]
            qr = r64 @ q[b, h]
            s = np.array([scale * float(kn[b, g, t]) * (ckf[kc[b, g, t]] @ qr) for t in range(n)])
            p = np.exp(s - s.max())
            p /= p.sum()
            o_rot = sum(p[t] * float(vn[b, g, t]) * cvf[vc[b, g, t]] for t in range(n))
            np.testing.assert_allclose(got[b, h], r64.T @ o_rot, rtol=0, atol=1e-12)


def test_attend_dense_special_cases():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, T, d = 3, 4, 2, 9, 24
    r = dense.rotation_f32(5, d)
    kc, kn, ck = _dense_cache(rng, B, Hkv, T, d, 3, r)
    vc, vn, cv = _dense_cache(rng, B, Hkv, T, d, 3, r)
    q = rng.standard_normal((B, Hq, d))
    v_hat = dense.decode_dense(vc, vn, r, cv)
    # length 0 -> zeros; a length past T -> the whole cache; length 1 -> the decoded value
    out = dense.attend_dense(q, kc, kn, vc, vn, [0, T + 50, 1], r, ck, cv, 0.3)
    assert np.all(out[0] == 0.0)
    np.testing.assert_array_equal(out[1], dense.attend_dense(q, kc, kn, vc, vn, [0, T, 1], r, ck,
                                                             cv, 0.3)[1])
    for h in range(Hq):
        np.testing.assert_allclose(out[2, h], v_hat[2, h // 2, 0], rtol=0, atol=1e-12)
    # identical keys -> uniform weights -> the mean of the decoded values
    kc2 = np.broadcast_to(kc[:, :, :1], kc.shape).copy()
    kn2 = np.broadcast_to(kn[:, :, :1], kn.shape).copy()
    out = dense.attend_dense(q, kc2, kn2, vc, vn, [T, T, T], r, ck, cv, 0.3)
    for b in range(B):
        for h in range(Hq):
            np.testing.assert_allclose(out[b, h], v_hat[b, h // 2].mean(axis=0), rtol=0, atol=1e-12)
    # query head h reads KV head h // 2: zero norms on KV head 0 zero heads 0 and 1 only
    vn0 = vn.copy()
    vn0[:, 0] = 0
    out = dense.attend_dense(q, kc, kn, vc, vn0, [T, T, T], r, ck, cv, 0.3)
    assert np.all(out[:, :2] == 0.0) and np.all(np.abs(out[:, 2:]).sum(axis=-1) > 0)

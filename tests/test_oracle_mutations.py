"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each test patches one plausible error into the oracle and checks that a pin that
does not share the oracle's code fails on the patched version.
"""

import numpy as np
from scipy.linalg import hadamard as scipy_hadamard

from oracle import attention as att
from oracle import codebook as cbm
from oracle import codec
from oracle import rotation as rot
from oracle import signs as sg


def test_dropped_fwht_stage_is_caught(monkeypatch):
    real = rot.fwht_stages

    def short(x, dtype=np.float64):
        y = np.array(x, dtype=dtype, copy=True)
        d = y.shape[-1]
        length = 1
        while length < d // 2:          # stops one stage early
            shaped = y.reshape(y.shape[:-1] + (d // (2 * length), 2, length))
            u, v = shaped[..., 0, :], shaped[..., 1, :]
            y = np.stack((u + v, u - v), axis=-2).reshape(y.shape)
            length <<= 1
        return y, 0

    monkeypatch.setattr(rot, "fwht_stages", short)
    y, _ = rot.fwht_stages(np.eye(128))
    assert not np.array_equal(y, scipy_hadamard(128).astype(np.float64))
    monkeypatch.setattr(rot, "fwht_stages", real)


def test_wrong_sign_placement_is_caught():
    d = 128
    s = sg.signs(42, d).astype(np.float64)
    H = rot.hadamard(d) / np.sqrt(d)
    e = np.zeros(d)
    e[3] = 1.0
    after = s * (H @ e)                    # D applied after H
    assert not np.allclose(after, s[3] * H[:, 3])
    np.testing.assert_allclose(rot.forward64(e, s), s[3] * H[:, 3], atol=1e-15)


def test_cell_midpoint_instead_of_conditional_mean_is_caught(monkeypatch):
    """Replacing the centroid (conditional mean) by the cell midpoint breaks the
    printed turboq2 centroids."""
    def midpoint_moment(a, b, m):
        return 0.5 * (np.asarray(a) + np.asarray(b)) * cbm._mass(a, b, m)

    monkeypatch.setattr(cbm, "_first_moment", midpoint_moment)
    _, c = cbm.codebook(2, 128)
    assert not np.array_equal(np.round(c.astype(np.float64), 3), [-0.133, -0.040, 0.040, 0.133])


def test_upper_tie_rule_is_caught():
    """Ties must go to the lower level: a value equal to a boundary."""
    b, _ = cbm.codebook(4)
    u = b[10:11]
    assert np.searchsorted(b, u, side="left")[0] == 10
    assert np.searchsorted(b, u, side="right")[0] == 11


def test_transposed_attention_operand_is_caught():
    """Using the value codes for the scores (a swapped operand) breaks the brute-force pin."""
    rng = np.random.default_rng(0)
    d, T = 128, 9
    s = sg.signs(42, d)
    bk, ck = cbm.codebook(4)
    kc, kn, _ = codec.encode_mse(rng.standard_normal((1, 1, T, d)).astype(np.float32), s, bk)
    vc, vn, _ = codec.encode_mse(rng.standard_normal((1, 1, T, d)).astype(np.float32), s, bk)
    kc, vc = codec.pack(kc, 4), codec.pack(vc, 4)
    q = rng.standard_normal((1, 1, d))
    good = att.attend_bruteforce(q, kc, kn, vc, vn, [T], 4, 4, ck, ck, s, 0.3)
    swapped = att.attend_fused(q, vc, vn, vc, vn, [T], 4, 4, ck, ck, s, 0.3)
    assert np.max(np.abs(good - swapped)) > 1e-3


def test_second_signs_before_the_transform_are_caught(monkeypatch):
    """Applying s2 before the butterflies (with s1) instead of after them breaks the
    dense D2 H D1 pin."""
    s1, s2 = sg.signs(42, 128), sg.signs2(42, 128)
    real = rot.forward64

    def early(x, s, s2_=None):
        s_comb = np.asarray(s, np.float64) * (1.0 if s2_ is None else np.asarray(s2_, np.float64))
        return real(x, s_comb)

    monkeypatch.setattr(rot, "forward64", early)
    R = np.diag(s2.astype(float)) @ rot.hadamard(128) @ np.diag(s1.astype(float)) / np.sqrt(128)
    x = np.random.default_rng(0).standard_normal((3, 128))
    assert not np.allclose(rot.forward64(x, s1, s2), x @ R.T, atol=1e-9)


def test_corrected_norm_with_the_fp16_input_norm_is_caught():
    """Dividing the fp16-rounded norm (instead of n32) by ||c[codes]|| and rounding
    again misses the fp64 quotient in far more than a few blocks."""
    x = np.random.default_rng(7).standard_normal((4000, 128)).astype(np.float32)
    s1 = sg.signs(42, 128)
    b, c = cbm.codebook(4)
    codes, n16, _ = codec.encode_mse(x, s1, b)
    r32 = codec.norm_f32(np.asarray(c, np.float32)[codes.reshape(-1, 1, 128)])
    wrong = (n16.astype(np.float32) / r32).astype(np.float16)
    r64 = np.linalg.norm(np.asarray(c, np.float32).astype(np.float64)[codes], axis=-1)
    q64 = (np.linalg.norm(x.astype(np.float64), axis=-1) / r64).astype(np.float16)
    assert np.count_nonzero(q64 != wrong[..., 0]) > 40


def test_dense_rotation_without_sign_fix_is_caught(monkeypatch):
    """Dropping the column sign fix of the QR factor breaks the positive-diagonal
    characterization the dense-rotation pin checks."""
    from oracle import dense

    def unfixed(seed, d):
        g = dense.normals(seed, d * d, 2 * d).reshape(d, d)
        q, _ = np.linalg.qr(g)
        return q

    monkeypatch.setattr(dense, "dense_rotation", unfixed)
    d = 96
    r = dense.dense_rotation(42, d)
    g = dense.normals(42, d * d, 2 * d).reshape(d, d)
    assert not np.all(np.diag(r.T @ g) > 0)


def test_dense_rotation_transposed_in_encode_is_caught():
    """Multiplying by R^T instead of R changes u (R is not symmetric)."""
    from oracle import dense
    d = 96
    r32 = dense.rotation_f32(42, d)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((8, d)).astype(np.float32)
    b, _ = cbm.codebook(4, d)
    _, _, u = dense.encode_dense(x, r32, b)
    n = codec.norm_f32(codec.pad_pow2(x)).astype(np.float64)
    wrong = (x.astype(np.float64) @ r32.astype(np.float64)) / n[:, None]
    assert np.max(np.abs(u - wrong)) > 1e-3


def test_dense_attention_with_a_transposed_decode_is_caught(monkeypatch):
    """Decoding with R instead of R^T breaks the fused-form identity the dense
    attention pin checks (scores <q, K^> against n <R q, c[code]>)."""
    from oracle import codebook as o_cb
    from oracle import dense
    d = 16
    r = dense.rotation_f32(42, d)
    rng = np.random.default_rng(0)
    b, c = o_cb.codebook(4, d)
    kc, kn, _ = dense.encode_dense(rng.standard_normal((1, d)).astype(np.float32), r, b)
    q = rng.standard_normal(d)

    def transposed(codes, norms16, r32, centroids):
        cc = np.asarray(centroids, np.float32).astype(np.float64)
        v = cc[np.asarray(codes)] * np.asarray(norms16, np.float16).astype(np.float64)[..., None]
        return v @ np.asarray(r32, np.float64).T          # R v instead of R^T v

    monkeypatch.setattr(dense, "decode_dense", transposed)
    k_hat = dense.decode_dense(kc, kn, r, c)
    fused = float(kn[0]) * (np.asarray(c, np.float32).astype(np.float64)[kc[0]] @ (r.astype(np.float64) @ q))
    assert abs(float(k_hat[0] @ q) - fused) > 1e-6

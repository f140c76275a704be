"""Pins for the oracle's encoder, decoder, packing and the 8-bit variant (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import codebook as cbm
from oracle import codec
from oracle import rotation as rot
from oracle import signs as sg

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
S128 = sg.signs(42, 128)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_unpack_every_value_at_every_position(bits):
    L = 1 << bits
    pos = np.arange(128)
    codes = np.stack([(pos + v) % L for v in range(L)]).astype(np.uint8)  # [L, 128]
    packed = codec.pack(codes, bits)
    assert packed.shape == (L, 1, codec.code_bytes(bits))
    np.testing.assert_array_equal(codec.unpack(packed, bits), codes)


def test_pack_bit_order_lsb_first():
    c = np.zeros(128, np.uint8)
    c[:4] = [0, 1, 2, 3]
    assert codec.pack(c, 2)[0, 0] == 0b11100100
    c4 = np.zeros(128, np.uint8)
    c4[:2] = [0x3, 0xA]
    assert codec.pack(c4, 4)[0, 0] == 0xA3
    c3 = np.zeros(128, np.uint8)
    c3[0], c3[1], c3[9] = 5, 2, 4        # 5 = 0b101, 4 = 0b100
    p3 = codec.pack(c3, 3)[0]
    assert p3[0] == 0b1001 and p3[2] == 0        # low planes of codes 0 and 1
    assert p3[32] == 0b1 and p3[33] == 0b10      # high bits of code 0 and code 9


def test_block_sizes_against_pages():
    g = GOLDEN["block_bytes_qk128"]
    # our blocks: codes + one fp16 norm; turboq4 also stores a second fp16 field
    assert codec.code_bytes(2) + 2 == g["turboq2"]
    assert codec.code_bytes(3) + 2 == g["turboq3"]
    assert codec.code_bytes(4) + 2 + g["turboq4_extra_fp16_fields"] == g["turboq4"]
    assert codec.code_bytes(8) + 2 == g["turboq8"]
    for name, bits in (("turboq2", 2), ("turboq3", 3), ("turboq8", 8)):
        assert (codec.code_bytes(bits) + 2) * 8 / 128 == g["bpw"][name]
    m = GOLDEN["memory_per_token_layer"]
    assert 16 * codec.code_bytes(4) == m["k4v2_16h"]["keys"]
    assert 16 * codec.code_bytes(2) == m["k4v2_16h"]["values"]
    assert 32 * codec.code_bytes(4) == m["k4v2_32h"]["keys"]
    assert 32 * codec.code_bytes(2) == m["k4v2_32h"]["values"]
    assert 16 * codec.code_bytes(3) == m["k3v2_16h"]["keys"]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_zero_vector(bits):
    b, c = cbm.codebook(bits)
    codes, n, _ = codec.encode_mse(np.zeros((3, 128), np.float32), S128, b)
    assert np.all(codes == (1 << bits) // 2 - 1) and np.all(n == 0)
    np.testing.assert_array_equal(codec.decode_mse(codes, n, S128, c)[0] * 0.0, np.zeros(128))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unit_basis_vector_by_hand(bits):
    """x = t e_i: R x = t s_i H[:, i]/sqrt(128), so u_k = s_i H[k, i] / sqrt(128) and
    each code is the level of +-1/sqrt(128) read off the boundaries by hand."""
    b, c = cbm.codebook(bits)
    H = rot.hadamard(128)
    for i, t in ((0, 3.0), (17, 0.25)):
        x = np.zeros(128, np.float32)
        x[i] = t
        codes, n, _ = codec.encode_mse(x, S128, b)
        assert n[0] == np.float16(t)
        a = np.float32(1.0) / np.float32(np.sqrt(128.0))
        up = int(np.sum(b < a))
        dn = int(np.sum(b < -a))
        expect = np.where(S128[i] * H[:, i] > 0, up, dn)
        np.testing.assert_array_equal(codes, expect)


def test_norm_canonical_vs_fp64():
    x = np.random.default_rng(0).standard_normal((20000, 128)).astype(np.float32)
    n32 = codec.norm_f32(x)
    n64 = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=1))
    assert np.max(np.abs(n32 / n64 - 1)) < 4e-7
    mismatch = np.mean(n32.astype(np.float16) != n64.astype(np.float16))
    assert mismatch < 2e-3


def test_norm_pairwise_order_is_bit0_first():
    """Sum order is part of the canonical definition: a case where left-to-right and
    pairwise (bit 0 first) sums differ in fp32."""
    x = np.zeros(128, np.float32)
    x[0], x[2], x[3] = np.float32(4096.0), np.float32(1.0), np.float32(1.0)
    q = x * x
    pair = (q[0] + q[1]) + (q[2] + q[3])
    assert codec.norm_f32(x[None])[0] == np.sqrt(pair + np.float32(0))
    seq = np.float32(0)
    for v in q:
        seq = np.float32(seq + v)
    assert pair != seq


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_canonical_codes_vs_math_mode(bits):
    """fp32 canonical codes differ from fp64 math-mode codes only at decision
    boundaries (adjacent levels) and rarely."""
    b, _ = cbm.codebook(bits)
    x = np.random.default_rng(1).standard_normal((8192, 128)).astype(np.float32)
    c32, _, _ = codec.encode_mse(x, S128, b)
    c64, _ = codec.encode_mse_f64(x, S128, b)
    diff = c32.astype(int) - c64.astype(int)
    assert np.all(np.abs(diff) <= 1)
    assert np.mean(diff != 0) < 1e-5


@pytest.mark.parametrize("bits", [2, 4])
def test_power_of_two_scale_equivariance(bits):
    b, _ = cbm.codebook(bits)
    x = np.random.default_rng(2).standard_normal((256, 128)).astype(np.float32)
    c0, n0, _ = codec.encode_mse(x, S128, b)
    for k in (-6, 5):
        c1, n1, _ = codec.encode_mse(x * np.float32(2.0 ** k), S128, b)
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(n1.astype(np.float32),
                                      (n0.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16).astype(np.float32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_roundtrip_mse_matches_codebook_distortion(bits):
    """For Gaussian x, R x / ||x|| is uniform on the sphere and independent of ||x||,
    so E||x - x_hat||^2 / E||x||^2 = d * D(sphere marginal)."""
    b, c = cbm.codebook(bits)
    x = np.random.default_rng(3).standard_normal((16384, 128)).astype(np.float32)
    codes, n, _ = codec.encode_mse(x, S128, b)
    xh = codec.decode_mse(codes, n, S128, c)
    ratio = np.sum((x - xh) ** 2) / np.sum(x.astype(np.float64) ** 2)
    expect = 128 * cbm.distortion(b, c, cbm.m_sphere(128))
    assert abs(ratio / expect - 1) < 0.015


def test_encode_is_deterministic_from_seed():
    b, _ = cbm.codebook(4)
    x = np.random.default_rng(4).standard_normal((64, 256)).astype(np.float32)
    s = sg.signs(99, 256)
    a = codec.encode_mse(x, s, b)
    z = codec.encode_mse(x, sg.signs(99, 256), b)
    np.testing.assert_array_equal(a[0], z[0])
    assert not np.array_equal(a[0], codec.encode_mse(x, sg.signs(100, 256), b)[0])


def test_all_same_and_extreme_magnitudes():
    b, c = cbm.codebook(4)
    for val in (1.0, 1e-3, 5000.0):   # norm stays inside the fp16 range
        x = np.full((1, 128), val, np.float32)
        codes, n, _ = codec.encode_mse(x, S128, b)
        xh = codec.decode_mse(codes, n, S128, c)
        assert np.linalg.norm(xh - x) / np.linalg.norm(x) < 0.2
    # below the fp16 range the stored norm is 0 and the block decodes to zero,
    # while the codes still carry the direction (the fp32 norm is nonzero)
    x = np.full((1, 128), 1e-20, np.float32)
    codes, n, _ = codec.encode_mse(x, S128, b)
    assert n[0] == 0 and not np.all(codes == 7)
    assert np.all(codec.decode_mse(codes, n, S128, c) == 0)


def test_u8_variant_error_bounds():
    s = sg.signs(42, 256)
    x = np.random.default_rng(5).standard_normal((2048, 256)).astype(np.float32)
    codes, sc = codec.encode_u8(x, s)
    y = rot.forward64(x.astype(np.float64), s).reshape(2048, 2, 128)
    yh = ((codes.astype(np.float64).reshape(2048, 2, 128) - 127.5) / 127.5
          * sc.astype(np.float64)[..., None])
    s64 = sc.astype(np.float64)[..., None]
    assert np.all(np.abs(yh - y) <= s64 / 255 * (1 + 1e-3) + np.abs(y) * 2e-3)
    # the largest |y| of each block decodes to +-s16 (the grid end points)
    imax = np.argmax(np.abs(y), axis=-1)
    ext = np.take_along_axis(codes.reshape(2048, 2, 128), imax[..., None], -1)[..., 0]
    assert np.mean((ext == 0) | (ext == 255)) > 0.99
    # uniform-grid MSE ~ step^2 / 12
    step = 2 * s64 / 255
    ratio = np.mean((yh - y) ** 2) / np.mean(step ** 2 / 12)
    assert 0.9 < ratio < 1.1
    xh = codec.decode_u8(codes, sc, s)
    np.testing.assert_allclose(xh, rot.inverse64(yh.reshape(2048, 256), s), atol=1e-12)


def test_u8_zero_block():
    codes, sc = codec.encode_u8(np.zeros((1, 128), np.float32), S128)
    assert np.all(codes == 128) and sc[0] == 0


def test_round_bf16_ties_and_library_agreement():
    """Ties go to the even 8-bit significand; on fp32 inputs the result equals an
    independent bf16 conversion (torch's round-to-nearest-even cast)."""
    import torch
    assert codec.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert codec.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert codec.round_bf16(np.array([-(1.0 + 2.0 ** -7 + 2.0 ** -20)]))[0] == -(1.0 + 2.0 ** -7)
    assert codec.round_bf16(np.array([0.0]))[0] == 0.0
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 3.0
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(codec.round_bf16(x.astype(np.float64)), want)

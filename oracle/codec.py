"""TurboQuant MSE encoder / decoder and bit packing (oracle; test infrastructure).

Pipeline per 128-element block, in the order of [Spec] "Overview" and "As-Built
Notes" and [turboq] "Encode pipeline" steps 1-3:

1. norm n = ||x||_2 of the block, stored as fp16 ([turboq] "Block structures":
   every block carries an fp16 norm);
2. rotate: h = H (s * x) (butterflies of [Spec] "Hadamard Transform Detail");
3. scale to the unit sphere: u = h / (sqrt(128) n)  ([Spec] "As-Built Notes":
   normalize by the L2 norm, the mapping the Beta codebook is built for);
4. bucketize: code_i = #{j : b_j < u_i}  ([Spec] Step 2: binary search in the
   boundaries gives the level index; ties go to the lower level);
5. pack ([Spec] "Step 3: Packing"; [turboq] "Block structures").

Canonical fp32 arithmetic (the bits the GPU must reproduce; the pages fix no
operation order, so this is this implementation's reading):

* x is widened exactly to fp32 (bf16 and fp32 inputs);
* q_i = RN32(x_i * x_i); the 128 squares are summed pairwise, combining index bit
  0 first, then bit 1, ..., bit 6 (level k adds partial sums whose indices differ
  in bit k);  n32 = RN32(sqrt(ss)) (correctly rounded);  stored norm RN16(n32);
* h = the fp32 butterflies of s * x in stage order len = 1, 2, ..., 64 (no scale);
* g = RN32(c / n32) with c = RN32(1/sqrt(128)), and g = 0 when n32 == 0;
* u_i = RN32(h_i * g);  code_i = #{j : b_j < u_i} with the fp32 boundaries.

Decode ([Spec] "Overview": look up reconstruction values, then rotate back) in
fp64:  x_hat = s * (H (n16 * c[code])) / sqrt(128), with n16 the stored fp16 norm.

Bit layouts per 128-block (LSB first inside each byte; the pages draw the fields
[v0:2][v1:2].. without naming an end, read here as least-significant first):

* 2 bits: 32 bytes, byte k = sum_j code[4k + j] << 2j;
* 3 bits: 48 bytes, split planes as in [turboq] block_turboq3_0: bytes 0..31 hold
  the low two bits in the 2-bit layout, bytes 32..47 the high bit,
  byte 32 + k = sum_j ((code[8k + j] >> 2) & 1) << j;
* 4 bits: 64 bytes, byte k = code[2k] | code[2k + 1] << 4;
* 8 bits: 128 bytes, byte k = code[k].

8-bit variant ([turboq] "At a glance", turboq8): the FWHT rotation followed by a
uniform 256-level grid, centroid[i] = (i - 127.5)/127.5, with a per-block absmax
scale.  Canonical fp32 reading (scale kept as fp16 in the norm slot):

* h as above;  a = max_i |h_i|;  s16 = RN16(RN32(a * c));  s32 = fp32(s16);
* G = RN32(K8 / s32) with K8 = RN32(c * 127.5), and G = 0 when s32 == 0;
* t_i = RN32(h_i * G);  w_i = RN32(t_i + 127.5);
  code_i = clamp(round_half_even(w_i), 0, 255);
* decode: y_hat_i = s32 (code_i - 127.5) / 127.5, then x_hat = R^T y_hat.
"""

from __future__ import annotations

import numpy as np

from .rotation import QK, fwht_stages, fwht_stages_f32, forward64, inverse64, inverse64_whole

C_SCALE = np.float32(1.0 / np.sqrt(128.0))
K8 = np.float32(C_SCALE * np.float32(127.5))

CODE_BYTES = {2: 32, 3: 48, 4: 64, 8: 128}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of fp64 values, returned as fp64: 8
    significant bits, fp32's exponent range (the bulk restore of the LMCache page
    "TurboQuant Serde Backend" writes bf16 KV; values here are normal numbers)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def code_bytes(bits: int) -> int:
    """Packed bytes per 128-element block."""
    return CODE_BYTES[bits]


def _blocks(x: np.ndarray) -> np.ndarray:
    d = x.shape[-1]
    assert d % QK == 0
    return x.reshape(x.shape[:-1] + (d // QK, QK))


def _sign_blocks(s: np.ndarray, d: int) -> np.ndarray:
    return np.asarray(s, np.float32).reshape(d // QK, QK)


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(u16, np.uint32) << 16).view(np.float32)


def norm_f32(xb: np.ndarray) -> np.ndarray:
    """Canonical fp32 norm of each 128-block (last axis): pairwise, bit 0 first."""
    q = xb * xb
    while q.shape[-1] > 1:
        q = q[..., 0::2] + q[..., 1::2]
    return np.sqrt(q[..., 0])


def encode_mse(x: np.ndarray, s: np.ndarray, boundaries: np.ndarray,
               s2: np.ndarray | None = None, centroids: np.ndarray | None = None,
               norm_correct: bool = False):
    """Canonical fp32 encode.  x: float32 [..., d].  Returns (codes uint8 [..., d],
    norms float16 [..., d/128], u float32 [..., d]).

    s2: the second sign vector ([turboq] "Encode pipeline" step 2): h_i becomes
    s2_i h_i (an exact sign change) before the scaling.
    norm_correct ([turboq] "Encode pipeline" step 4): the stored norm is
    RN16(RN32(n32 / r32)) with r32 the canonical fp32 norm of the block's centroid
    values c[code_i] (same pairwise order as the input norm), so the decoded block
    has the input's norm up to the fp16 rounding of the stored value."""
    x = np.asarray(x)
    assert x.dtype == np.float32
    d = x.shape[-1]
    xb = _blocks(x)
    xs = xb * _sign_blocks(s, d)
    n32 = norm_f32(xb)
    h = fwht_stages_f32(xs)
    if s2 is not None:
        h = h * _sign_blocks(s2, d)
    g = np.zeros_like(n32)
    np.divide(C_SCALE, n32, out=g, where=n32 > 0)
    u = h * g[..., None]
    codes = np.searchsorted(np.asarray(boundaries, np.float32), u, side="left")
    stored = n32
    if norm_correct:
        cv = np.asarray(centroids, np.float32)[codes]
        r32 = norm_f32(cv)
        stored = np.zeros_like(n32)
        np.divide(n32, r32, out=stored, where=r32 > 0)
    return (codes.astype(np.uint8).reshape(x.shape), stored.astype(np.float16),
            u.reshape(x.shape))


def encode_mse_f64(x: np.ndarray, s: np.ndarray, boundaries: np.ndarray):
    """fp64 "math mode" encode (used only to bound the canonical-mode flip rate)."""
    x64 = np.asarray(x, np.float64)
    d = x64.shape[-1]
    y = _blocks(forward64(x64, s))
    n = np.sqrt(np.sum(_blocks(x64) ** 2, axis=-1))
    u = np.where(n[..., None] > 0, y / np.where(n > 0, n, 1.0)[..., None], 0.0)
    codes = np.searchsorted(np.asarray(boundaries, np.float64), u, side="left")
    return codes.astype(np.uint8).reshape(x64.shape[:-1] + (d,)), n


def decode_mse(codes: np.ndarray, norms16: np.ndarray, s: np.ndarray,
               centroids: np.ndarray, s2: np.ndarray | None = None) -> np.ndarray:
    """fp64 decode: x_hat = s * (H (s2 * n16 * c[code])) / sqrt(128), per block (s2
    omitted: all ones)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    c = np.asarray(centroids, np.float32).astype(np.float64)
    n = np.asarray(norms16, np.float16).astype(np.float64)
    v = _blocks(c[codes]) * n[..., None]
    return inverse64(v.reshape(codes.shape), s, s2)


def pow2_length(d: int) -> int:
    """Transform length of a head_dim-d vector: d itself when a power of two, else
    the next power of two ([Spec] "Hadamard Transform Detail": a head_dim that is not
    a power of two is zero-padded to the next one, transformed, and the padding is
    dropped again after the inverse)."""
    n = 1
    while n < d:
        n <<= 1
    return n


def pad_pow2(x: np.ndarray) -> np.ndarray:
    """x [..., d] zero-padded to [..., pow2_length(d)] (same dtype)."""
    x = np.asarray(x)
    d = x.shape[-1]
    dp = pow2_length(d)
    if dp == d:
        return x
    out = np.zeros(x.shape[:-1] + (dp,), x.dtype)
    out[..., :d] = x
    return out


def encode_mse_whole(x: np.ndarray, s: np.ndarray, boundaries: np.ndarray):
    """Canonical fp32 encode with one rotation over the whole vector and the codebook
    of dimension d = head_dim ([Spec] "Step 1" and "Step 2": R is d x d, one codebook
    per (head_dim, bits)).  A head_dim that is not a power of two is zero-padded to
    d' = the next power of two first, and the transform, the codebook and the codes
    are those of length d' (s has d' signs).  One norm per vector (the padding adds
    nothing to it).

    n32 = RN32(sqrt(pairwise sum of RN32(x_i^2))) over index bits 0 .. log2(d') - 1;
    h = fp32 butterflies of s * x in stage order 1, 2, ..., d'/2; g = RN32(c / n32)
    with c = RN32(1/sqrt(d')) (0 when n32 == 0); u = RN32(h * g);
    code = #{j : b_j < u}.  Returns (codes uint8 [..., d'], norms fp16 [...], u)."""
    x = np.asarray(x)
    assert x.dtype == np.float32
    x = pad_pow2(x)
    d = x.shape[-1]
    n32 = norm_f32(x)
    h, _ = fwht_stages(x * np.asarray(s, np.float32), dtype=np.float32)
    c_d = np.float32(1.0 / np.sqrt(float(d)))
    g = np.zeros_like(n32)
    np.divide(c_d, n32, out=g, where=n32 > 0)
    u = h * g[..., None]
    codes = np.searchsorted(np.asarray(boundaries, np.float32), u, side="left")
    return codes.astype(np.uint8), n32.astype(np.float16), u


def decode_mse_whole(codes: np.ndarray, norms16: np.ndarray, s: np.ndarray,
                     centroids: np.ndarray, head_dim: int | None = None) -> np.ndarray:
    """fp64 decode of the whole-vector mode: x_hat = s * H_d' (n16 * c[code]) / sqrt(d')
    over the d' codes, then the first head_dim coordinates (the padding is dropped;
    head_dim defaults to d')."""
    c = np.asarray(centroids, np.float32).astype(np.float64)
    n = np.asarray(norms16, np.float16).astype(np.float64)
    x = inverse64_whole(c[np.asarray(codes)] * n[..., None], s)
    return x if head_dim is None else x[..., :head_dim]


def encode_u8(x: np.ndarray, s: np.ndarray, s2: np.ndarray | None = None):
    """Canonical fp32 8-bit encode.  Returns (codes uint8 [..., d], scales fp16);
    s2 as for ``encode_mse``."""
    x = np.asarray(x)
    assert x.dtype == np.float32
    d = x.shape[-1]
    xs = _blocks(x) * _sign_blocks(s, d)
    h = fwht_stages_f32(xs)
    if s2 is not None:
        h = h * _sign_blocks(s2, d)
    a = np.max(np.abs(h), axis=-1)
    s16 = (a * C_SCALE).astype(np.float16)
    s32 = s16.astype(np.float32)
    G = np.zeros_like(s32)
    np.divide(K8, s32, out=G, where=s32 > 0)
    t = h * G[..., None]
    w = t + np.float32(127.5)
    codes = np.clip(np.rint(w), 0, 255).astype(np.uint8)
    return codes.reshape(x.shape), s16


def decode_u8(codes: np.ndarray, scales16: np.ndarray, s: np.ndarray,
              s2: np.ndarray | None = None) -> np.ndarray:
    """fp64 decode of the 8-bit variant."""
    codes = np.asarray(codes)
    sc = np.asarray(scales16, np.float16).astype(np.float64)
    y = (_blocks(codes.astype(np.float64)) - 127.5) / 127.5 * sc[..., None]
    return inverse64(y.reshape(codes.shape), s, s2)


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [..., d] (d multiple of 128) into bytes [..., d/128, cb]."""
    c = _blocks(np.asarray(codes, np.uint8)).astype(np.uint32)
    if bits == 2:
        q = c.reshape(c.shape[:-1] + (32, 4))
        out = q[..., 0] | q[..., 1] << 2 | q[..., 2] << 4 | q[..., 3] << 6
    elif bits == 4:
        q = c.reshape(c.shape[:-1] + (64, 2))
        out = q[..., 0] | q[..., 1] << 4
    elif bits == 3:
        lo = pack((c & 3).reshape(codes.shape), 2)
        hb = ((c >> 2) & 1).reshape(c.shape[:-1] + (16, 8))
        hi = np.zeros(hb.shape[:-1], np.uint32)
        for j in range(8):
            hi |= hb[..., j] << j
        return np.concatenate((lo, hi.astype(np.uint8)), axis=-1)
    elif bits == 8:
        out = c
    else:
        raise ValueError(f"unsupported bits {bits}")
    return out.astype(np.uint8)


def unpack(packed: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of ``pack``: bytes [..., nblk, cb] -> codes [..., nblk * 128]."""
    p = np.asarray(packed, np.uint8).astype(np.uint32)
    lead = p.shape[:-2]
    nblk = p.shape[-2]
    if bits == 2:
        out = np.stack([(p >> (2 * j)) & 3 for j in range(4)], axis=-1)
    elif bits == 4:
        out = np.stack([p & 15, p >> 4], axis=-1)
    elif bits == 3:
        lo = unpack(p[..., :32], 2).reshape(lead + (nblk, QK))
        hb = np.stack([(p[..., 32:48] >> j) & 1 for j in range(8)], axis=-1)
        out = lo | (hb.reshape(lead + (nblk, QK)) << 2)
    elif bits == 8:
        out = p
    else:
        raise ValueError(f"unsupported bits {bits}")
    return out.reshape(lead + (nblk * QK,)).astype(np.uint8)

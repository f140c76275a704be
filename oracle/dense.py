"""Dense random orthogonal rotation for head_dims that are not a power of two
(oracle; test infrastructure).

[Spec] "Hadamard Transform Detail": for a head_dim that is not a power of two the page
offers, besides zero-padding to the next power of two, a dense random orthogonal
matrix.  [Spec] "Step 1: Random Orthogonal Rotation": a fixed d x d orthogonal R,
generated once from a seed and reused for every vector; rotate(x) = R x.

Readings (the pages name no generator):

* Gaussian entries: SplitMix64 seeded with the rotation seed, continuing after the
  2 d draws of the two sign vectors (draw index 2 d onwards); draws z1, z2 of a pair
  give the uniforms u1 = ((z1 >> 11) + 1/2) 2^-53 (in (0, 1)) and u2 = (z2 >> 11) 2^-53,
  and the Box-Muller transform (Box and Muller, 1958) gives two standard normals
  r cos(2 pi u2) and r sin(2 pi u2) with r = sqrt(-2 ln u1).  G[i][j] is normal
  number i d + j.
* R = Q of the QR decomposition G = Q T, with the signs of Q's columns chosen so
  that T has a positive diagonal (this makes R Haar-distributed and unique).
* The device path uses R rounded to fp32; so does this module's encode.
* Codes: u = (R x) / ||x|| against the codebook of dimension d, code = #{j : b_j < u},
  computed here in fp64; the norm is the canonical fp32 norm of the whole vector
  (``codec.norm_f32`` over the vector zero-padded to a power of two), stored as fp16.
* Layout: the d codes of a vector fill ceil(d / 128) packed 128-element blocks, the
  positions past d holding code 0; one norm per vector.
* Attention over such a cache ([Spec] "Optimization: Fused dequant-dot" with this R):
  the plain definition, softmax(scale q K^T) V over the decoded keys and values
  K^ = decode_dense(K), V^ = decode_dense(V), in fp64 (a length is clamped to
  [0, T]; length 0 gives zeros; query head h reads KV head h / (Hq / Hkv)).
"""

from __future__ import annotations

import numpy as np

from . import codec
from .signs import splitmix64


def normals(seed: int, n: int, offset: int) -> np.ndarray:
    """n standard normals (fp64) from SplitMix64 draws offset, offset + 1, ...,
    two per pair of draws (Box-Muller)."""
    pairs = (n + 1) // 2
    z = np.array(splitmix64(seed, offset + 2 * pairs)[offset:], dtype=np.uint64)
    u1 = ((z[0::2] >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    u2 = (z[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * pairs)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n]


def dense_rotation(seed: int, d: int) -> np.ndarray:
    """The d x d orthogonal matrix R (fp64): Q of G = Q T with T's diagonal positive."""
    g = normals(seed, d * d, 2 * d).reshape(d, d)
    q, t = np.linalg.qr(g)
    sgn = np.where(np.diag(t) < 0, -1.0, 1.0)
    return q * sgn[None, :]


def rotation_f32(seed: int, d: int) -> np.ndarray:
    """R rounded to fp32 (what the device path multiplies by)."""
    return dense_rotation(seed, d).astype(np.float32)


def encode_dense(x: np.ndarray, r32: np.ndarray, boundaries: np.ndarray):
    """x float32 [..., d], r32 float32 [d, d].  Returns (codes uint8 [..., d],
    norms fp16 [...], u fp64 [..., d]) with u = (R x) / n32 in fp64."""
    x = np.asarray(x)
    assert x.dtype == np.float32
    n32 = codec.norm_f32(codec.pad_pow2(x))
    y = x.astype(np.float64) @ np.asarray(r32, np.float64).T
    n = n32.astype(np.float64)
    u = np.zeros_like(y)
    np.divide(y, n[..., None], out=u, where=n[..., None] > 0)
    b = np.asarray(boundaries, np.float32).astype(np.float64)
    codes = np.searchsorted(b, u, side="left")
    return codes.astype(np.uint8), n32.astype(np.float16), u


def decode_dense(codes: np.ndarray, norms16: np.ndarray, r32: np.ndarray,
                 centroids: np.ndarray) -> np.ndarray:
    """fp64 x_hat = R^T (n16 * c[code]) over the d codes of each vector."""
    c = np.asarray(centroids, np.float32).astype(np.float64)
    n = np.asarray(norms16, np.float16).astype(np.float64)
    v = c[np.asarray(codes)] * n[..., None]
    return v @ np.asarray(r32, np.float64)


def pack_dense(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., d] -> packed [..., ceil(d / 128), cb] with code 0 past d."""
    d = codes.shape[-1]
    dp = -(-d // 128) * 128
    full = np.zeros(codes.shape[:-1] + (dp,), np.uint8)
    full[..., :d] = codes
    return codec.pack(full, bits)


def attend_dense(q: np.ndarray, k_codes: np.ndarray, k_norms16: np.ndarray,
                 v_codes: np.ndarray, v_norms16: np.ndarray, lens, r32: np.ndarray,
                 k_centroids: np.ndarray, v_centroids: np.ndarray, scale: float) -> np.ndarray:
    """q [B, Hq, d]; codes [B, Hkv, T, d] (unpacked), norms fp16 [B, Hkv, T] ->
    out fp64 [B, Hq, d] = softmax(scale q K^T) V with K^ = decode_dense(K),
    V^ = decode_dense(V)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv, T = k_codes.shape[1], k_codes.shape[2]
    k_hat = decode_dense(k_codes, k_norms16, r32, k_centroids)   # [B, Hkv, T, d]
    v_hat = decode_dense(v_codes, v_norms16, r32, v_centroids)
    out = np.zeros((B, Hq, d))
    grp = Hq // Hkv
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), T))
        if n == 0:
            continue
        for h in range(Hq):
            g = h // grp
            s = scale * (k_hat[b, g, :n] @ q[b, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            out[b, h] = p @ v_hat[b, g, :n]
    return out

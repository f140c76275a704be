"""Randomized Walsh-Hadamard rotation (oracle; test infrastructure).

[Spec] "Step 1: Random Orthogonal Rotation" and "Hadamard Transform Detail": the
Walsh-Hadamard matrix H is applied in place by butterflies, stage lengths
1, 2, 4, ..., d/2, each pair (x[i+j], x[i+j+len]) becoming (u + v, u - v), and the
result is scaled by 1/sqrt(d).  [Spec] "As-Built Notes" puts the signs before the
transform: R x = H (D x) / sqrt(d).  The exact inverse is R^T = D H / sqrt(d)
(H / sqrt(d) is symmetric and its own inverse, D is its own inverse).

The transform is applied per QK = 128 block ([turboq] "Block structures": every
block covers 128 elements; head_dim must be a multiple of 128), with block j of a
longer vector using the slice s[128 j : 128 (j + 1)] of the sign vector.

Two arithmetic modes:

* ``hadamard`` / ``forward64`` / ``inverse64``: fp64 "math" mode;
* ``fwht_stages_f32``: the canonical fp32 butterflies in the stage order above,
  without the 1/sqrt(d) factor (the codec applies scaling itself).
"""

from __future__ import annotations

import numpy as np

QK = 128


def hadamard(d: int) -> np.ndarray:
    """Sylvester Walsh-Hadamard matrix, H[i, j] = (-1)^popcount(i & j), fp64."""
    idx = np.arange(d)
    parity = np.zeros((d, d), dtype=np.int64)
    a = idx[:, None] & idx[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 1, -1.0, 1.0)


def fwht_stages(x: np.ndarray, dtype=np.float64) -> tuple[np.ndarray, int]:
    """Butterfly transform over the last axis (length a power of two), in ``dtype``.

    Stage ``len`` pairs index i with i + len inside each run of 2*len elements and
    writes (u + v, u - v).  Returns (H x, number of butterfly add/sub operations).
    """
    y = np.array(x, dtype=dtype, copy=True)
    d = y.shape[-1]
    ops = 0
    length = 1
    while length < d:
        shaped = y.reshape(y.shape[:-1] + (d // (2 * length), 2, length))
        u = shaped[..., 0, :]
        v = shaped[..., 1, :]
        top = u + v
        bot = u - v
        y = np.stack((top, bot), axis=-2).reshape(y.shape)
        ops += d
        length <<= 1
    return y, ops


def fwht_stages_f32(x: np.ndarray) -> np.ndarray:
    """Canonical fp32 butterflies (no scaling) over the last axis of length 128."""
    assert x.dtype == np.float32 and x.shape[-1] == QK
    y, _ = fwht_stages(x, dtype=np.float32)
    return y


def _blocked(x: np.ndarray):
    d = x.shape[-1]
    assert d % QK == 0, "head_dim must be a multiple of 128"
    return x.reshape(x.shape[:-1] + (d // QK, QK))


def forward64(x: np.ndarray, s: np.ndarray, s2: np.ndarray | None = None) -> np.ndarray:
    """R x = H (s * x) / sqrt(128), blockwise per 128 elements, in fp64.  With a
    second sign vector ([turboq] "Encode pipeline" step 2): R x = s2 * H (s * x) /
    sqrt(128)."""
    xb = _blocked(np.asarray(x, np.float64) * np.asarray(s, np.float64))
    y, _ = fwht_stages(xb, np.float64)
    y = (y / np.sqrt(QK)).reshape(np.shape(x))
    return y if s2 is None else y * np.asarray(s2, np.float64)


def inverse64(y: np.ndarray, s: np.ndarray, s2: np.ndarray | None = None) -> np.ndarray:
    """R^T y = s * (H y) / sqrt(128), blockwise per 128 elements, in fp64 (with a
    second sign vector: s * H (s2 * y) / sqrt(128), the transpose of the above)."""
    y = np.asarray(y, np.float64)
    if s2 is not None:
        y = y * np.asarray(s2, np.float64)
    yb = _blocked(y)
    h, _ = fwht_stages(yb, np.float64)
    return (h / np.sqrt(QK)).reshape(np.shape(y)) * np.asarray(s, np.float64)


def forward64_whole(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """One transform over the whole vector ([Spec] "Step 1": R is d x d with d =
    head_dim, a power of two): R x = H_d (s * x) / sqrt(d), fp64."""
    x = np.asarray(x, np.float64) * np.asarray(s, np.float64)
    y, _ = fwht_stages(x, np.float64)
    return y / np.sqrt(x.shape[-1])


def inverse64_whole(y: np.ndarray, s: np.ndarray) -> np.ndarray:
    """R^T y = s * H_d y / sqrt(d) over the whole vector, fp64."""
    y = np.asarray(y, np.float64)
    h, _ = fwht_stages(y, np.float64)
    return h / np.sqrt(y.shape[-1]) * np.asarray(s, np.float64)

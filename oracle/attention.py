"""Decode attention over the packed cache (oracle; test infrastructure).

[Spec] "Optimization: Fused dequant-dot": pre-rotate the query once, take the dot
product of the rotated query with the centroid look-ups of each cached key (no
inverse transform per cached vector, because <q, R^T k'> = <R q, k'>), accumulate
the softmax-weighted centroid look-ups of the values in the rotated domain, and
inverse-rotate the output once.  [Rotor] "The QJL Estimator Formula" writes the
same first term as norm * sum_d(Q_rot[d] * centroids[idx[s, d]]); the QJL term is
not part of this path.

``attend_fused`` computes exactly that in fp64:

    q' = R q;  s_t = scale * sum_blk nK[t, blk] <q'_blk, cK[codeK_t, blk]>;
    p = softmax(s over t < len);  o' = sum_t p_t nV[t, blk] cV[codeV_t, blk];
    o = R^T o'.

Readings: the GQA head map is g = floor(h / (Hq / Hkv)) (not on the pages); a
sequence of length 0 gives an all-zero output; the scale is a caller argument
(1/sqrt(128) for the pages' workloads).

``attend_bruteforce`` is the plain definition softmax(scale q K_hat^T) V_hat on the
decoded cache (``codec.decode_mse``), used to pin ``attend_fused``.

Every function takes an optional second sign vector s2 ([turboq] "Encode pipeline"
step 2: R = D2 H D1 / sqrt(128)); the rotated-domain identity holds for any
orthogonal R, so the fused form is unchanged apart from the rotation.

``append_attend`` is [Spec] "Attention with TurboQuant cache": quantize the new K
and V vectors into the cache at their positions, then attend with the
full-precision query over the cached positions.  Positions map to cache slots
modulo the cache length ([Spec] "Integration Points": circular addressing
cache_pos = pos % max_seq), so a full ring holds the last max_seq tokens.
"""

from __future__ import annotations

import numpy as np

from .codec import decode_mse, encode_mse, pack, unpack
from .rotation import QK, forward64, inverse64


def _softmax64(s: np.ndarray) -> np.ndarray:
    m = np.max(s)
    e = np.exp(s - m)
    return e / np.sum(e)


def attend_fused(q, k_codes, k_norms, v_codes, v_norms, seq_lens, k_bits, v_bits,
                 k_centroids, v_centroids, s, scale, heads=None, s2=None):
    """fp64 fused rotated-domain attention.

    q: [B, Hq, d] (any float dtype), k_codes/v_codes: [B, Hkv, T, nblk, cb] uint8,
    k_norms/v_norms: [B, Hkv, T, nblk] float16, seq_lens: [B] ints.
    ``heads`` optionally restricts the computation to a list of (b, h) pairs; the
    rows not computed are left at zero.  Returns out [B, Hq, d] float64.
    """
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    grp = Hq // Hkv
    nblk = d // QK
    ck = np.asarray(k_centroids, np.float32).astype(np.float64)
    cv = np.asarray(v_centroids, np.float32).astype(np.float64)
    out = np.zeros((B, Hq, d), np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    cache = {}
    for b, h in heads:
        L = int(seq_lens[b])
        if L == 0:
            continue
        g = h // grp
        if (b, g) not in cache:
            kc = ck[unpack(k_codes[b, g, :L], k_bits)].reshape(L, nblk, QK)
            vc = cv[unpack(v_codes[b, g, :L], v_bits)].reshape(L, nblk, QK)
            kn = np.asarray(k_norms[b, g, :L], np.float16).astype(np.float64)
            vn = np.asarray(v_norms[b, g, :L], np.float16).astype(np.float64)
            cache = {(b, g): (kc, vc, kn, vn)}
        kc, vc, kn, vn = cache[(b, g)]
        qr = forward64(q[b, h], s, s2).reshape(nblk, QK)
        dots = np.einsum("tjc,jc->tj", kc, qr)
        scores = scale * np.sum(kn * dots, axis=-1)
        p = _softmax64(scores)
        o_rot = np.einsum("t,tj,tjc->jc", p, vn, vc)
        out[b, h] = inverse64(o_rot.reshape(d), s, s2)
    return out


def attend_fused_counted(q, k_codes, k_norms, v_codes, v_norms, counts, k_bits, v_bits,
                         k_centroids, v_centroids, s, scale, s2=None):
    """fp64 fused attention of one sequence and KV head over a cache given as distinct
    tokens with multiplicities (test infrastructure for caches too long to unpack).

    A cache in which token j occurs counts[j] times has the softmax of [Spec]
    "Optimization: Fused dequant-dot" over all its slots, so token j's weight is
    counts[j] * exp(s_j - m) / sum_i counts[i] * exp(s_i - m): the same steps as
    ``attend_fused`` with each exponential multiplied by its count.

    q: [G, d] (the query heads of the KV head); k_codes/v_codes: [n, nblk, cb] uint8;
    k_norms/v_norms: [n, nblk] float16; counts: [n] non-negative integers.
    Returns out [G, d] float64.
    """
    q = np.asarray(q, np.float64)
    G, d = q.shape
    nblk = d // QK
    n = k_codes.shape[0]
    w = np.asarray(counts, np.float64)
    kc = np.asarray(k_centroids, np.float32).astype(np.float64)[unpack(k_codes, k_bits)]
    vc = np.asarray(v_centroids, np.float32).astype(np.float64)[unpack(v_codes, v_bits)]
    kc, vc = kc.reshape(n, nblk, QK), vc.reshape(n, nblk, QK)
    kn = np.asarray(k_norms, np.float16).astype(np.float64).reshape(n, nblk)
    vn = np.asarray(v_norms, np.float16).astype(np.float64).reshape(n, nblk)
    out = np.zeros((G, d), np.float64)
    live = w > 0
    if not np.any(live):
        return out
    for h in range(G):
        qr = forward64(q[h], s, s2).reshape(nblk, QK)
        scores = scale * np.sum(kn * np.einsum("tjc,jc->tj", kc, qr), axis=-1)
        m = np.max(scores[live])
        e = np.where(live, w * np.exp(np.where(live, scores - m, 0.0)), 0.0)
        p = e / np.sum(e)
        o_rot = np.einsum("t,tj,tjc->jc", p, vn, vc)
        out[h] = inverse64(o_rot.reshape(d), s, s2)
    return out


def attend_bruteforce(q, k_codes, k_norms, v_codes, v_norms, seq_lens, k_bits, v_bits,
                      k_centroids, v_centroids, s, scale, s2=None):
    """softmax(scale * q K_hat^T) V_hat on the decoded cache, fp64 (tiny inputs)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            g = h // grp
            kh = decode_mse(unpack(k_codes[b, g, :L], k_bits), k_norms[b, g, :L], s,
                            k_centroids, s2)
            vh = decode_mse(unpack(v_codes[b, g, :L], v_bits), v_norms[b, g, :L], s,
                            v_centroids, s2)
            p = _softmax64(scale * (kh @ q[b, h]))
            out[b, h] = p @ vh
    return out


def append_attend(q, k_new, v_new, pos, k_codes, k_norms, v_codes, v_norms, k_bits, v_bits,
                  k_boundaries, k_centroids, v_boundaries, v_centroids, s, scale, s2=None,
                  norm_correct=False):
    """Append then attend (fp64 attention; canonical fp32 encode).

    q: [B, Hq, d]; k_new/v_new: [B, Hkv, n_new, d] float32; pos: [B] position of the
    first new token of each sequence; caches as in ``attend_fused`` with T slots.
    Token i of sequence b is encoded into slot (pos[b] + i) mod T; the attention then
    covers the min(pos[b] + n_new, T) filled slots (softmax and the weighted sum do
    not depend on slot order).  The caches are updated in place.
    Returns (out [B, Hq, d] float64, seq_lens [B]).
    """
    k_new = np.asarray(k_new, np.float32)
    v_new = np.asarray(v_new, np.float32)
    B, Hkv, n_new, d = k_new.shape
    T = k_codes.shape[2]
    kc, kn, _ = encode_mse(k_new, s, k_boundaries, s2, k_centroids, norm_correct)
    vc, vn, _ = encode_mse(v_new, s, v_boundaries, s2, v_centroids, norm_correct)
    kp, vp = pack(kc, k_bits), pack(vc, v_bits)
    for b in range(B):
        for i in range(n_new):
            slot = (int(pos[b]) + i) % T
            k_codes[b, :, slot] = kp[b, :, i]
            v_codes[b, :, slot] = vp[b, :, i]
            k_norms[b, :, slot] = kn[b, :, i]
            v_norms[b, :, slot] = vn[b, :, i]
    lens = np.array([min(int(pos[b]) + n_new, T) for b in range(B)], np.int64)
    out = attend_fused(q, k_codes, k_norms, v_codes, v_norms, lens, k_bits, v_bits,
                       k_centroids, v_centroids, s, scale, s2=s2)
    return out, lens


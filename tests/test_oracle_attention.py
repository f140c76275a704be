"""Pins for the oracle's fused decode attention (CPU only)."""

import json
import os

import numpy as np
import pytest

import workloads
from oracle import attention as att
from oracle import codebook as cbm
from oracle import codec
from oracle import signs as sg

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def _cache(kx, vx, s, kb, vb):
    """Encode K/V [B, Hkv, T, d] float32 into packed codes and fp16 norms."""
    bk, _ = cbm.codebook(kb)
    bv, _ = cbm.codebook(vb)
    kc, kn, _ = codec.encode_mse(kx, s, bk)
    vc, vn, _ = codec.encode_mse(vx, s, bv)
    return codec.pack(kc, kb), kn, codec.pack(vc, vb), vn


@pytest.mark.parametrize("d,kb,vb", [(128, 4, 2), (256, 3, 3), (128, 4, 4)])
def test_fused_equals_bruteforce(d, kb, vb):
    rng = np.random.default_rng(0)
    B, Hq, Hkv, T = 2, 4, 2, 37
    s = sg.signs(42, d)
    kx = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    vx = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    q = rng.standard_normal((B, Hq, d)).astype(np.float32)
    kc, kn, vc, vn = _cache(kx, vx, s, kb, vb)
    lens = np.array([T, 11])
    ck = cbm.codebook(kb)[1]
    cv = cbm.codebook(vb)[1]
    scale = 1 / np.sqrt(d)
    a = att.attend_fused(q, kc, kn, vc, vn, lens, kb, vb, ck, cv, s, scale)
    b = att.attend_bruteforce(q, kc, kn, vc, vn, lens, kb, vb, ck, cv, s, scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_single_token_and_identical_keys_and_empty():
    rng = np.random.default_rng(1)
    d = 128
    s = sg.signs(42, d)
    kx = np.repeat(rng.standard_normal((1, 1, 1, d)), 5, axis=2).astype(np.float32)
    vx = rng.standard_normal((1, 1, 5, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    kc, kn, vc, vn = _cache(kx, vx, s, 4, 2)
    ck, cv = cbm.codebook(4)[1], cbm.codebook(2)[1]
    vhat = codec.decode_mse(codec.unpack(vc[0, 0], 2), vn[0, 0], s, cv)
    one = att.attend_fused(q, kc, kn, vc, vn, [1], 4, 2, ck, cv, s, 0.1)
    np.testing.assert_allclose(one[0, 0], vhat[0], atol=1e-12)
    allk = att.attend_fused(q, kc, kn, vc, vn, [5], 4, 2, ck, cv, s, 0.1)
    np.testing.assert_allclose(allk[0, 0], vhat.mean(axis=0), atol=1e-12)
    zero = att.attend_fused(q, kc, kn, vc, vn, [0], 4, 2, ck, cv, s, 0.1)
    assert np.all(zero == 0)


def test_gqa_head_mapping():
    """Query head h reads KV head floor(h / (Hq/Hkv)): duplicating a KV head's data
    into every group gives identical outputs for heads with the same query."""
    rng = np.random.default_rng(2)
    d, T = 128, 20
    s = sg.signs(3, d)
    kx = rng.standard_normal((1, 2, T, d)).astype(np.float32)
    vx = rng.standard_normal((1, 2, T, d)).astype(np.float32)
    qh = rng.standard_normal(d).astype(np.float32)
    q = np.tile(qh, (1, 4, 1))
    kc, kn, vc, vn = _cache(kx, vx, s, 4, 4)
    ck = cbm.codebook(4)[1]
    o = att.attend_fused(q, kc, kn, vc, vn, [T], 4, 4, ck, ck, s, 0.2)
    np.testing.assert_allclose(o[0, 0], o[0, 1], atol=0)
    np.testing.assert_allclose(o[0, 2], o[0, 3], atol=0)
    assert np.max(np.abs(o[0, 0] - o[0, 2])) > 1e-3


def _cosine_study(kx, vx, qs, kb, vb):
    s = sg.signs(workloads.ROTATION_SEED, 128)
    T = kx.shape[0]
    kc, kn, vc, vn = _cache(kx[None, None], vx[None, None], s, kb, vb)
    ck, cv = cbm.codebook(kb)[1], cbm.codebook(vb)[1]
    q = qs[None].astype(np.float32)
    scale = 1 / np.sqrt(128)
    oq = att.attend_fused(q, kc, kn, vc, vn, [T], kb, vb, ck, cv, s, scale)[0]
    cos = []
    for i, qq in enumerate(qs.astype(np.float64)):
        sc = scale * (kx.astype(np.float64) @ qq)
        p = np.exp(sc - sc.max())
        p /= p.sum()
        ref = p @ vx.astype(np.float64)
        cos.append(ref @ oq[i] / np.linalg.norm(ref) / np.linalg.norm(oq[i]))
    return float(np.mean(cos))


@pytest.mark.parametrize("kb,vb,key,lo,hi", [
    (4, 2, "k4v2_gaussian", 0.92, 0.95),
    (4, 3, "k4v3_gaussian", 0.97, 0.99),
    (4, 4, "k4v4_gaussian", 0.985, 1.0),
])
def test_quality_matches_spec_table_gaussian(kb, vb, key, lo, hi):
    """[Spec] 'Measured quality': attention-output cosine FP vs compressed (statistical
    soft check over 20 seeded queries, T = 1024, scale 1/sqrt(128))."""
    k, v, _ = workloads.tiny_inputs()
    qs = np.random.default_rng(100).standard_normal((20, 128))
    c = _cosine_study(k, v, qs, kb, vb)
    assert lo <= c <= hi, (c, GOLDEN["attention_cosine"][key])


def test_quality_matches_spec_table_correlated():
    import torch
    w = workloads.WORKLOADS["llama_layer"]
    k, v = workloads.make_kv(w, "cpu", tokens=1024, batch=1)
    k = k[0, 0].to(torch.float32).numpy()
    v = v[0, 0].to(torch.float32).numpy()
    qs = np.random.default_rng(101).standard_normal((20, 128))
    c = _cosine_study(k, v, qs, 4, 2)
    assert 0.96 <= c <= 0.99, (c, GOLDEN["attention_cosine"]["k4v2_correlated"])


def _empty_cache(B, Hkv, T, d, kb, vb):
    nblk = d // 128
    return (np.zeros((B, Hkv, T, nblk, codec.code_bytes(kb)), np.uint8),
            np.zeros((B, Hkv, T, nblk), np.float16),
            np.zeros((B, Hkv, T, nblk, codec.code_bytes(vb)), np.uint8),
            np.zeros((B, Hkv, T, nblk), np.float16))


def test_append_first_token_gives_its_value():
    """pos 0 into an empty cache: one cached token, so every head returns its V_hat."""
    rng = np.random.default_rng(3)
    d, s = 128, sg.signs(42, 128)
    bk, ck = cbm.codebook(4)
    bv, cv = cbm.codebook(2)
    kc, kn, vc, vn = _empty_cache(1, 2, 16, d, 4, 2)
    kx = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    vx = rng.standard_normal((1, 2, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out, lens = att.append_attend(q, kx, vx, [0], kc, kn, vc, vn, 4, 2, bk, ck, bv, cv, s, 0.1)
    assert list(lens) == [1]
    for h in range(4):
        g = h // 2
        vhat = codec.decode_mse(codec.unpack(vc[0, g, :1], 2), vn[0, g, :1], s, cv)[0]
        np.testing.assert_allclose(out[0, h], vhat, atol=1e-12)
    # slot 0 holds exactly the packed encoding of the new vectors
    ref_k, ref_kn, _ = codec.encode_mse(kx, s, bk)
    np.testing.assert_array_equal(kc[0, :, 0], codec.pack(ref_k, 4)[0, :, 0])
    np.testing.assert_array_equal(kn[0, :, 0], ref_kn[0, :, 0])


@pytest.mark.parametrize("n_new", [1, 3])
def test_append_ring_equals_attention_over_last_tokens(n_new):
    """Appending a stream of tokens into a ring of T slots, then attending, equals
    brute-force attention over the last T tokens encoded into a plain cache (the
    circular addressing keeps exactly those, in some slot order)."""
    rng = np.random.default_rng(4)
    d, T, Hkv, Hq, total = 128, 7, 2, 4, 23
    s = sg.signs(42, d)
    bk, ck = cbm.codebook(4)
    bv, cv = cbm.codebook(3)
    kx = rng.standard_normal((1, Hkv, total, d)).astype(np.float32)
    vx = rng.standard_normal((1, Hkv, total, d)).astype(np.float32)
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    ring = _empty_cache(1, Hkv, T, d, 4, 3)
    pos = 0
    while pos < total:
        n = min(n_new, total - pos)
        out, lens = att.append_attend(q, kx[:, :, pos:pos + n], vx[:, :, pos:pos + n], [pos],
                                      *ring, 4, 3, bk, ck, bv, cv, s, 0.09)
        pos += n
        assert list(lens) == [min(pos, T)]
    kc, kn, vc, vn = _cache(kx[:, :, total - T:], vx[:, :, total - T:], s, 4, 3)
    ref = att.attend_bruteforce(q, kc, kn, vc, vn, [T], 4, 3, ck, cv, s, 0.09)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_append_per_sequence_positions():
    """Each sequence appends at its own position; a sequence that has not wrapped
    attends over pos + n_new tokens, one that has wrapped over all T slots."""
    rng = np.random.default_rng(5)
    d, T, Hkv, Hq = 128, 9, 1, 2
    s = sg.signs(42, d)
    bk, ck = cbm.codebook(4)
    bv, cv = cbm.codebook(2)
    kc, kn, vc, vn = _empty_cache(2, Hkv, T, d, 4, 2)
    hist_k = rng.standard_normal((2, Hkv, T, d)).astype(np.float32)
    hist_v = rng.standard_normal((2, Hkv, T, d)).astype(np.float32)
    pk, pkn, pv, pvn = _cache(hist_k, hist_v, s, 4, 2)
    kc[:], kn[:], vc[:], vn[:] = pk, pkn, pv, pvn
    kx = rng.standard_normal((2, Hkv, 2, d)).astype(np.float32)
    vx = rng.standard_normal((2, Hkv, 2, d)).astype(np.float32)
    q = rng.standard_normal((2, Hq, d)).astype(np.float32)
    out, lens = att.append_attend(q, kx, vx, [3, 17], kc, kn, vc, vn, 4, 2, bk, ck, bv, cv, s,
                                  0.09)
    assert list(lens) == [5, 9]
    # sequence 0: history slots 0-2, new tokens in slots 3-4
    k0 = np.concatenate([hist_k[0:1, :, :3], kx[0:1]], axis=2)
    v0 = np.concatenate([hist_v[0:1, :, :3], vx[0:1]], axis=2)
    # sequence 1: positions 17, 18 -> slots 8, 0; the other slots keep the history
    k1 = hist_k[1:2].copy()
    v1 = hist_v[1:2].copy()
    k1[:, :, 8], k1[:, :, 0] = kx[1, :, 0], kx[1, :, 1]
    v1[:, :, 8], v1[:, :, 0] = vx[1, :, 0], vx[1, :, 1]
    for b, (kk, vv, L) in enumerate(((k0, v0, 5), (k1, v1, 9))):
        c = _cache(kk, vv, s, 4, 2)
        ref = att.attend_bruteforce(q[b:b + 1], *c, [L], 4, 2, ck, cv, s, 0.09)
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3)])
def test_counted_equals_repeated_cache(kb, vb):
    """The multiset form equals attend_fused on the cache with every distinct token
    written out counts[j] times (in any slot order), and zero counts drop a token."""
    rng = np.random.default_rng(7)
    d, n, G = 128, 6, 4
    s = sg.signs(42, d)
    kx = (rng.standard_normal((1, 1, n, d)) * rng.uniform(0.5, 4.0, (1, 1, n, 1))).astype(np.float32)
    vx = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    q = rng.standard_normal((1, G, d)).astype(np.float32)
    kc, kn, vc, vn = _cache(kx, vx, s, kb, vb)
    ck, cv = cbm.codebook(kb)[1], cbm.codebook(vb)[1]
    counts = np.array([3, 1, 0, 7, 2, 5])
    idx = rng.permutation(np.repeat(np.arange(n), counts))
    full = att.attend_fused(q, kc[:, :, idx], kn[:, :, idx], vc[:, :, idx], vn[:, :, idx],
                            [idx.size], kb, vb, ck, cv, s, 0.3)
    got = att.attend_fused_counted(q[0], kc[0, 0], kn[0, 0], vc[0, 0], vn[0, 0], counts, kb, vb,
                                   ck, cv, s, 0.3)
    np.testing.assert_allclose(got, full[0], rtol=0, atol=1e-12)
    assert np.all(att.attend_fused_counted(q[0], kc[0, 0], kn[0, 0], vc[0, 0], vn[0, 0],
                                           np.zeros(n), kb, vb, ck, cv, s, 0.3) == 0)

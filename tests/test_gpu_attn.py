"""GPU parity of fa_tq_attn_decode against the fp64 CPU oracle (MI355X).

The packed cache the kernel reads is always produced without the HIP path: by the
oracle's own encoder, or (for the largest workloads) drawn directly as seeded
random codes and fp16 norms.  The oracle evaluates the same packed cache.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as o_att
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import ATTN_MAX_ABS, bf16_to_f32, say

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _oracle_cache(x32: np.ndarray, bits: int, seed: int = SEED):
    """x32 [B, H, T, 128] -> (packed [B, H, T, 1, cb] uint8, norms f16 [B, H, T, 1])."""
    b, _ = o_cb.codebook(bits)
    c, n, _ = codec.encode_mse(x32, o_signs.signs(seed, 128), b)
    return codec.pack(c, bits), n


def _random_cache(B, H, T, bits, seed):
    """Seeded random packed codes and fp16 norms (norms ~ 11.3 * lognormal(0, 0.3))."""
    rng = np.random.default_rng(seed)
    cbytes = {2: 32, 3: 48, 4: 64}[bits]
    packed = rng.integers(0, 256, size=(B, H, T, 1, cbytes), dtype=np.uint8)
    norms = (11.3 * np.exp(0.3 * rng.standard_normal((B, H, T, 1)))).astype(np.float16)
    return packed, norms


def _run(fa, q, kp, kn, vp, vn, lens, kb, vb, scale, heads=None, where="", flags=0):
    torch = _torch()
    dev = "cuda"
    ck, cv = fa.codebook_init(128, kb), fa.codebook_init(128, vb)
    qt = torch.from_numpy(q).to(dev) if isinstance(q, np.ndarray) else q
    out = fa.attn_decode(ck, cv, SEED, qt, torch.from_numpy(kp).to(dev),
                         torch.from_numpy(kn.view(np.int16)).to(dev),
                         torch.from_numpy(vp).to(dev), torch.from_numpy(vn.view(np.int16)).to(dev),
                         torch.tensor(lens, dtype=torch.int32, device=dev), scale, flags=flags)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    q32 = bf16_to_f32(qt) if qt.dtype == torch.bfloat16 else qt.cpu().numpy()
    ref = o_att.attend_fused(q32, kp, kn, vp, vn, lens, kb, vb, o_cb.codebook(kb)[1],
                             o_cb.codebook(vb)[1], o_signs.signs(SEED, 128), scale, heads=heads)
    if heads is not None:
        sel = tuple(np.array(heads).T)
        got, ref = got[sel], ref[sel]
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    say(f"{where}: max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS, f"{where}: {err}"
    return err


@pytest.mark.parametrize("flags", [0, "valu"])
def test_attn_lengths_outside_the_cache_are_clamped(gpu_lib, flags):
    """seq_lens is device data the host cannot check: a negative length gives zeros and a
    length past t_max attends over the whole cache (the oracle on the clamped lengths)."""
    torch = _torch()
    B, Hq, Hkv, T = 3, 8, 2, 300
    rng = np.random.default_rng(17)
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(torch.bfloat16)
    kp, kn = _oracle_cache(k, 4)
    vp, vn = _oracle_cache(v, 2)
    dev = "cuda"
    ck, cv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 2)
    fl = gpu_lib.ATTN_VECTOR_ALU if flags == "valu" else 0
    out = gpu_lib.attn_decode(ck, cv, SEED, q.cuda(), torch.from_numpy(kp).to(dev),
                              torch.from_numpy(kn.view(np.int16)).to(dev),
                              torch.from_numpy(vp).to(dev),
                              torch.from_numpy(vn.view(np.int16)).to(dev),
                              torch.tensor([-5, T + 1000, 2**31 - 1], dtype=torch.int32,
                                           device=dev), 1 / np.sqrt(128), flags=fl)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = o_att.attend_fused(bf16_to_f32(q), kp, kn, vp, vn, [0, T, T], 4, 2,
                             o_cb.codebook(4)[1], o_cb.codebook(2)[1], o_signs.signs(SEED, 128),
                             1 / np.sqrt(128))
    assert np.all(got[0] == 0.0)
    err = float(np.max(np.abs(got - ref)))
    say(f"clamped lengths ({flags}): max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS


def test_attn_tiny_workload(gpu_lib):
    k, v, q = workloads.tiny_inputs()
    kp, kn = _oracle_cache(k.reshape(1, 1, 1024, 128), 4)
    vp, vn = _oracle_cache(v.reshape(1, 1, 1024, 128), 2)
    _run(gpu_lib, q.reshape(1, 1, 128), kp, kn, vp, vn, [1024], 4, 2, 1 / np.sqrt(128),
         where="tiny")


@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3), (4, 4), (2, 3), (3, 4), (2, 2), (4, 3)])
@pytest.mark.parametrize("B,Hq,Hkv,T,lens", [
    (3, 8, 2, 333, [333, 0, 1]),
    (2, 4, 4, 1000, [1000, 517]),
    (1, 32, 2, 700, [700]),
    (2, 6, 3, 2100, [64, 2099]),
    (1, 40, 5, 300, [300]),
    (2, 5, 1, 129, [129, 77]),
    (1, 12, 4, 257, [257]),       # groups of 3
    (2, 14, 2, 300, [31, 300]),   # groups of 7
    (1, 24, 2, 200, [199]),       # groups of 12: two workgroups of 6 per KV head
    (2, 32, 2, 400, [400, 123]),  # groups of 16: two workgroups of 8
    (2, 32, 1, 300, [300, 57]),   # one KV head (groups of 32): four workgroups of 8
    (1, 64, 1, 200, [200]),       # groups of 64: eight workgroups of 8
    (1, 22, 2, 150, [150]),       # groups of 11: eleven workgroups of 1
])
def test_attn_ragged(gpu_lib, kb, vb, B, Hq, Hkv, T, lens):
    torch = _torch()
    say(f"attn ragged K{kb}V{vb} B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens}")
    rng = np.random.default_rng(kb * 10 + vb + T)
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32) * rng.uniform(0.2, 3.0, (1, Hkv, 1, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(torch.bfloat16)
    kp, kn = _oracle_cache(k, kb)
    vp, vn = _oracle_cache(v, vb)
    _run(gpu_lib, q.cuda(), kp, kn, vp, vn, lens, kb, vb, 1 / np.sqrt(128), where="ragged")


@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3), (4, 4)])
@pytest.mark.parametrize("B,Hq,Hkv,T,lens", [(2, 32, 8, 1500, [1500, 901]), (1, 4, 4, 300, [257]),
                                             (1, 24, 2, 200, [199]), (2, 32, 2, 300, [300, 41])])
def test_attn_vector_alu_kernels(gpu_lib, kb, vb, B, Hq, Hkv, T, lens):
    """FA_TQ_ATTN_VECTOR_ALU: the vector-ALU kernels (group sizes up to 16) against the
    same oracle."""
    torch = _torch()
    say(f"attn vector-ALU K{kb}V{vb} B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens}")
    rng = np.random.default_rng(kb * 100 + vb + T)
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(torch.bfloat16)
    kp, kn = _oracle_cache(k, kb)
    vp, vn = _oracle_cache(v, vb)
    _run(gpu_lib, q.cuda(), kp, kn, vp, vn, lens, kb, vb, 1 / np.sqrt(128), where="valu",
         flags=gpu_lib.ATTN_VECTOR_ALU)


def test_attn_fp32_query_and_scales(gpu_lib):
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T = 2, 8, 8, 257
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    kp, kn = _oracle_cache(k, 4)
    vp, vn = _oracle_cache(v, 2)
    for scale in (1 / np.sqrt(128), 0.5, 1e-3):
        _run(gpu_lib, q, kp, kn, vp, vn, [T, 100], 4, 2, scale, where=f"scale {scale}")


def test_attn_seq_len_clamped_to_t_max(gpu_lib):
    rng = np.random.default_rng(4)
    T = 130
    k = rng.standard_normal((1, 1, T, 128)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, 128)).astype(np.float32)
    q = rng.standard_normal((1, 2, 128)).astype(np.float32)
    kp, kn = _oracle_cache(k, 4)
    vp, vn = _oracle_cache(v, 4)
    torch = _torch()
    ck = gpu_lib.codebook_init(128, 4)
    args = [torch.from_numpy(a).cuda() for a in (kp, kn.view(np.int16), vp, vn.view(np.int16))]
    big = gpu_lib.attn_decode(ck, ck, SEED, torch.from_numpy(q).cuda(), *args,
                              torch.tensor([10 ** 6], dtype=torch.int32, device="cuda"), 0.1)
    ref = gpu_lib.attn_decode(ck, ck, SEED, torch.from_numpy(q).cuda(), *args,
                              torch.tensor([T], dtype=torch.int32, device="cuda"), 0.1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(big.cpu().numpy(), ref.cpu().numpy())


def test_attn_llama_layer_full(gpu_lib):
    """Llama-3-8B-shaped layer at full size (32768 tokens, 32/8 heads, K4/V2): the
    oracle encodes the whole bf16 cache; all 32 heads compared."""
    torch = _torch()
    w = workloads.WORKLOADS["llama_layer"]
    say("attn llama_layer full")
    k, v = workloads.make_kv(w, "cuda")
    q = workloads.make_q(w, "cuda")
    kp, kn = _oracle_cache(bf16_to_f32(k), w.k_bits)
    vp, vn = _oracle_cache(bf16_to_f32(v), w.v_bits)
    del k, v
    _run(gpu_lib, q, kp, kn, vp, vn, [w.tokens], w.k_bits, w.v_bits, 1 / np.sqrt(128),
         where="llama_layer")


def test_attn_batched_full_sampled(gpu_lib):
    """Batched workload at full size (16 x 8192, K3/V3, lengths in [4096, 8192])."""
    w = workloads.WORKLOADS["batched"]
    say("attn batched full")
    kp, kn = _random_cache(w.batch, w.n_kv_heads, w.tokens, w.k_bits, 31)
    vp, vn = _random_cache(w.batch, w.n_kv_heads, w.tokens, w.v_bits, 32)
    lens = workloads.make_seq_lens(w)
    q = workloads.make_q(w, "cuda")
    heads = [(b, h) for b in (0, 7, 15) for h in (0, 5, 31)]
    _run(gpu_lib, q, kp, kn, vp, vn, lens, w.k_bits, w.v_bits, 1 / np.sqrt(128), heads=heads,
         where="batched")


def test_attn_long_context_full_sampled(gpu_lib):
    """Long-context workload at full size (4 x 131072, K4/V4)."""
    w = workloads.WORKLOADS["long_context"]
    say("attn long_context full")
    kp, kn = _random_cache(w.batch, w.n_kv_heads, w.tokens, w.k_bits, 41)
    vp, vn = _random_cache(w.batch, w.n_kv_heads, w.tokens, w.v_bits, 42)
    lens = workloads.make_seq_lens(w)
    q = workloads.make_q(w, "cuda")
    heads = [(0, 0), (1, 9), (2, 20), (3, 31)]   # four (sequence, KV head) slices
    _run(gpu_lib, q, kp, kn, vp, vn, lens, w.k_bits, w.v_bits, 1 / np.sqrt(128), heads=heads,
         where="long_context")


def test_attn_largest_t_max(gpu_lib):
    """The largest t_max of the matrix-core path (2^25 - 1 slots: K4 code rows of
    2 GiB - 64 B, byte offsets near 2^31).  Every slot holds a cold key (codes 0)
    except three hot ones (codes 15) at slots 0, 2^24 + 5 and t_max - 1; with key
    norms of 60000 and a query along the hot direction the cold slots' softmax
    weights are exactly zero in fp32 and in fp64, so the output is the oracle's
    attention over the three hot slots (their values random codes and norms)."""
    from oracle import rotation
    torch = _torch()
    fa = gpu_lib
    T = (1 << 25) - 1
    hot = [0, (1 << 24) + 5, T - 1]
    say(f"attn largest t_max={T}")
    dev = "cuda"
    kp = torch.zeros((1, 1, T, 1, 64), dtype=torch.uint8, device=dev)
    kn = torch.full((1, 1, T, 1), 60000.0, dtype=torch.float16, device=dev).view(torch.int16)
    vp = torch.zeros((1, 1, T, 1, 32), dtype=torch.uint8, device=dev)
    vn = torch.full((1, 1, T, 1), 1.0, dtype=torch.float16, device=dev).view(torch.int16)
    rng = np.random.default_rng(5)
    hv = rng.integers(0, 256, (3, 32), dtype=np.uint8)
    hn = (1.0 + rng.random(3)).astype(np.float16)
    for i, t in enumerate(hot):
        kp[0, 0, t] = 0xFF
        vp[0, 0, t, 0] = torch.from_numpy(hv[i]).to(dev)
        vn[0, 0, t, 0] = int(hn[i:i + 1].view(np.int16)[0])
    s = o_signs.signs(SEED, 128)
    q = rotation.inverse64(np.full((1, 4, 128), 0.1), s).astype(np.float32)   # R q = 0.1
    scale = 1 / np.sqrt(128)
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    out = fa.attn_decode(ck, cv, SEED, torch.from_numpy(q).to(dev), kp, kn, vp, vn,
                         torch.tensor([T], dtype=torch.int32, device=dev), scale)
    torch.cuda.synchronize()
    kp3 = np.full((1, 1, 3, 1, 64), 0xFF, np.uint8)
    kn3 = np.full((1, 1, 3, 1), 60000.0, np.float16)
    ref = o_att.attend_fused(q, kp3, kn3, hv.reshape(1, 1, 3, 1, 32), hn.reshape(1, 1, 3, 1),
                             [3], 4, 2, o_cb.codebook(4)[1], o_cb.codebook(2)[1], s, scale)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    say(f"largest t_max: max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS


def test_attn_sink_and_faint_tail(gpu_lib):
    """Value weights far below one next to a dominant token, over a long stream.

    t_max = 2^25 - 1 slots of one KV head with 4 query heads (K4/V2).  Slot 0 is a
    sink (the highest score); slots 1 .. 65535 hold keys whose softmax weights
    relative to the sink are log-spread over [1e-7, 1e-5] (61 distinct key norms
    in turn), all with the same value codes (the largest centroid in every
    element, a sign-coherent value row) and value norm 1, so rounding of their
    weights cannot cancel; every later slot has a key pointing away from the query
    (weight 0 in fp32, below 1e-120 in fp64).  Each wave of the first split streams
    thousands of these faint tokens after the sink, the case where a one-signed
    rounding of small weights would add up.  The reference is the oracle's fused
    attention over the distinct tokens with their multiplicities.

    A weight rounding biased toward zero (fp16 halves of p * n_V cut to the fp16
    subnormal step) loses about 2.5e-3 here (CPU emulation); round-to-nearest halves
    in the normal range leave the fp32 accumulation of ~1024 MFMA tile sums per wave
    onto a sink-sized accumulator (at most ~2^-24 of it per addition, 6e-5 relative
    in all, 7e-4 on these outputs of magnitude 12).  The test asks for half the
    contract's tolerance."""
    from oracle import rotation
    torch = _torch()
    fa = gpu_lib
    T, C, P = (1 << 25) - 1, 1 << 16, 61
    scale = 1 / np.sqrt(128)
    ck4, cv2 = o_cb.codebook(4)[1], o_cb.codebook(2)[1]
    a = np.array([0.1, 0.1, 0.08, 0.12])          # q'_h = a_h * (1, ..., 1)
    kfac = scale * 128 * float(ck4[15])           # score per unit key norm and unit a
    n_sink = 100.0
    p_want = np.exp(np.linspace(np.log(1e-7), np.log(1e-5), P))
    n_cold = (n_sink + np.log(p_want) / (kfac * a[0])).astype(np.float16)
    say(f"attn sink + faint tail: t_max={T}, {C - 1} faint slots, key norms "
        f"{float(n_cold.min()):.2f}..{float(n_cold.max()):.2f}")
    dev = "cuda"
    kp = torch.full((1, 1, T, 1, 64), 0xFF, dtype=torch.uint8, device=dev)
    kp[0, 0, C:] = 0
    kn = torch.full((1, 1, T, 1), 1000.0, dtype=torch.float16, device=dev)
    kn[0, 0, 0, 0] = n_sink
    reps = -(-(C - 1) // P)
    kn[0, 0, 1:C, 0] = torch.from_numpy(np.tile(n_cold, reps)[:C - 1]).to(dev)
    vp = torch.full((1, 1, T, 1, 32), 0xFF, dtype=torch.uint8, device=dev)
    vn = torch.full((1, 1, T, 1), 1.0, dtype=torch.float16, device=dev)
    vn[0, 0, 0, 0] = 8.0
    s = o_signs.signs(SEED, 128)
    q = rotation.inverse64(a[:, None] * np.ones((4, 128)), s).astype(np.float32)[None]
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    out = fa.attn_decode(ck, cv, SEED, torch.from_numpy(q).to(dev), kp, kn.view(torch.int16),
                         vp, vn.view(torch.int16),
                         torch.tensor([T], dtype=torch.int32, device=dev), scale)
    torch.cuda.synchronize()
    del kp, kn, vp, vn
    # distinct tokens: sink, the P faint keys, the far key
    counts = np.concatenate([[1], np.bincount(np.arange(C - 1) % P, minlength=P), [T - C]])
    dk = np.full((P + 2, 1, 64), 0xFF, np.uint8)
    dk[-1] = 0
    dkn = np.concatenate([[n_sink], n_cold, [1000.0]]).astype(np.float16).reshape(-1, 1)
    dv = np.full((P + 2, 1, 32), 0xFF, np.uint8)
    dvn = np.ones((P + 2, 1), np.float16)
    dvn[0] = 8.0
    ref = o_att.attend_fused_counted(q[0], dk, dkn, dv, dvn, counts, 4, 2, ck4, cv2, s, scale)
    err = float(np.max(np.abs(out.cpu().numpy()[0] - ref)))
    say(f"sink + faint tail: max abs err {err:.3e} (|out| max {np.max(np.abs(ref)):.2f})")
    assert err <= ATTN_MAX_ABS, err
    assert err <= ATTN_MAX_ABS / 2, f"no margin left: {err}"


@pytest.mark.parametrize("kb,vb", [(4, 2), (2, 4), (3, 4), (4, 4)])
def test_attn_long_splits_deep_prefetch(gpu_lib, kb, vb):
    """Splits long enough that every wave streams more than 16 super tiles (the kernels
    then keep three super tiles of codes in flight instead of one): 4 sequences x 8 KV
    heads x 40000 slots (chunks of 5120 tokens), ragged lengths, seeded random codes;
    the query heads of four (sequence, KV head) slices against the fused fp64
    attention."""
    torch = _torch()
    B, Hq, Hkv, T = 4, 16, 8, 40000
    lens = [40000, 38001, 20003, 4097]
    say(f"attn deep prefetch K{kb}V{vb}")
    kp, kn = _random_cache(B, Hkv, T, kb, 100 + kb)
    vp, vn = _random_cache(B, Hkv, T, vb, 200 + vb)
    rng = np.random.default_rng(kb * 10 + vb)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(torch.bfloat16)
    grp = Hq // Hkv
    heads = [(b, g * grp + i) for b, g in ((0, 3), (1, 0), (2, 5), (3, 7)) for i in range(grp)]
    _run(gpu_lib, q.cuda(), kp, kn, vp, vn, lens, kb, vb, 1 / np.sqrt(128), heads=heads,
         where=f"deep prefetch K{kb}V{vb}")

"""GPU parity of fa_tq_attn_append (append into a ring cache, then attend) against
the CPU oracle's append_attend (MI355X).

The cache history is written by the oracle's own encoder (or drawn as seeded random
codes at full size); the new K/V vectors are encoded by both sides from the same
inputs.  Cache contents after the call are compared byte for byte (codes may differ
only by the contract's adjacent-level flips), outputs within the attention bound.
"""

import numpy as np
import pytest

import workloads
from oracle import attention as o_att
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import ATTN_MAX_ABS, bf16_to_f32, compare_codes, compare_norms, say

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _history(B, H, T, bits, rng):
    """Oracle-encoded history [B, H, T, 1, cb] from N(0, 1) float32 vectors."""
    x = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    b, _ = o_cb.codebook(bits)
    c, n, _ = codec.encode_mse(x, o_signs.signs(SEED, 128), b)
    return codec.pack(c, bits), n


def _step(fa, q, kx, vx, pos, caches, kb, vb, scale, where):
    """One append call on the GPU and in the oracle; caches = numpy (kp, kn, vp, vn)
    (updated in place by the oracle) and their device copies."""
    torch = _torch()
    (kp, kn, vp, vn), dev = caches
    ck, cv = fa.codebook_init(128, kb), fa.codebook_init(128, vb)
    out = fa.attn_append(ck, cv, SEED, torch.from_numpy(q).cuda(), torch.from_numpy(kx).cuda(),
                         torch.from_numpy(vx).cuda(),
                         torch.tensor(pos, dtype=torch.int32, device="cuda"), *dev, scale)
    torch.cuda.synchronize()
    ref, lens = o_att.append_attend(q, kx, vx, pos, kp, kn, vp, vn, kb, vb,
                                    o_cb.codebook(kb)[0], o_cb.codebook(kb)[1],
                                    o_cb.codebook(vb)[0], o_cb.codebook(vb)[1],
                                    o_signs.signs(SEED, 128), scale)
    T = kp.shape[2]
    for name, g, o, bits in (("k", dev[0], kp, kb), ("v", dev[2], vp, vb)):
        compare_codes(g.cpu().numpy().reshape(-1, o.shape[-1]),
                      codec.unpack(o.reshape(-1, 1, o.shape[-1]), bits).reshape(-1, 128), bits,
                      f"{where} {name} cache")
    compare_norms(dev[1].cpu().numpy(), kn, f"{where} k norms")
    compare_norms(dev[3].cpu().numpy(), vn, f"{where} v norms")
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    say(f"{where}: lens {list(lens)} T {T} max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS, f"{where}: {err}"


def _device(fa, kp, kn, vp, vn):
    torch = _torch()
    return (torch.from_numpy(kp.copy()).cuda(), torch.from_numpy(kn.view(np.int16).copy()).cuda(),
            torch.from_numpy(vp.copy()).cuda(), torch.from_numpy(vn.view(np.int16).copy()).cuda())


@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3), (4, 4), (2, 4), (3, 2)])
@pytest.mark.parametrize("n_new", [1, 3])
def test_append_positions_and_wrap(gpu_lib, kb, vb, n_new):
    """Three sequences: one early in the cache, one ending on the last slot, one that
    wraps around the ring within this call."""
    rng = np.random.default_rng(100 + kb * 10 + vb + n_new)
    B, Hq, Hkv, T = 3, 8, 2, 96
    kp, kn = _history(B, Hkv, T, kb, rng)
    vp, vn = _history(B, Hkv, T, vb, rng)
    caches = ((kp, kn, vp, vn), _device(gpu_lib, kp, kn, vp, vn))
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    kx = rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32)
    vx = rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32)
    pos = [5, T - n_new, 2 * T - 1]
    _step(gpu_lib, q, kx, vx, pos, caches, kb, vb, 1 / np.sqrt(128), f"wrap K{kb}V{vb} n{n_new}")


def test_append_token_stream_into_ring(gpu_lib):
    """Decode loop: 40 single-token appends into a 16-slot ring, checked every step."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, T = 2, 8, 2, 16
    kb, vb = 4, 2
    nb = {2: 32, 3: 48, 4: 64}
    kp = np.zeros((B, Hkv, T, 1, nb[kb]), np.uint8)
    vp = np.zeros((B, Hkv, T, 1, nb[vb]), np.uint8)
    kn = np.zeros((B, Hkv, T, 1), np.float16)
    vn = np.zeros((B, Hkv, T, 1), np.float16)
    caches = ((kp, kn, vp, vn), _device(gpu_lib, kp, kn, vp, vn))
    for step in range(40):
        q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
        kx = rng.standard_normal((B, Hkv, 1, 128)).astype(np.float32)
        vx = rng.standard_normal((B, Hkv, 1, 128)).astype(np.float32)
        _step(gpu_lib, q, kx, vx, [step, step + 3], caches, kb, vb, 1 / np.sqrt(128),
              f"stream step {step}")


def test_append_bf16_strided_new_tokens(gpu_lib):
    """bf16 new K/V given as a slice of a wider tensor (non-contiguous head and token
    strides) and a bf16 query."""
    torch = _torch()
    rng = np.random.default_rng(9)
    B, Hq, Hkv, T = 2, 4, 2, 40
    kp, kn = _history(B, Hkv, T, 4, rng)
    vp, vn = _history(B, Hkv, T, 4, rng)
    dev = _device(gpu_lib, kp, kn, vp, vn)
    wide_k = torch.randn((B, Hkv + 1, 5, 256), dtype=torch.float32).to(torch.bfloat16)
    wide_v = torch.randn((B, Hkv + 1, 5, 256), dtype=torch.float32).to(torch.bfloat16)
    kx, vx = wide_k[:, 1:, 1:3, 128:], wide_v[:, :Hkv, 2:4, :128]
    q = torch.randn((B, Hq, 128), dtype=torch.float32).to(torch.bfloat16)
    ck, cv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 4)
    pos = [7, 39]
    out = gpu_lib.attn_append(ck, cv, SEED, q.cuda(), kx.cuda(), vx.cuda(),
                              torch.tensor(pos, dtype=torch.int32, device="cuda"), *dev, 0.1)
    torch.cuda.synchronize()
    bk, c4 = o_cb.codebook(4)
    ref, _ = o_att.append_attend(bf16_to_f32(q), bf16_to_f32(kx), bf16_to_f32(vx), pos, kp, kn,
                                 vp, vn, 4, 4, bk, c4, bk, c4, o_signs.signs(SEED, 128), 0.1)
    compare_codes(dev[0].cpu().numpy().reshape(-1, 64),
                  codec.unpack(kp.reshape(-1, 1, 64), 4).reshape(-1, 128), 4, "bf16 k cache")
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    say(f"append bf16 strided: max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS


def test_append_rejects_before_writing(gpu_lib):
    """n_new > t_max and a bad group size are rejected and leave the cache untouched."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(11)
    B, Hkv, T = 1, 2, 8
    kp, kn = _history(B, Hkv, T, 4, rng)
    vp, vn = _history(B, Hkv, T, 2, rng)
    dev = _device(fa, kp, kn, vp, vn)
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    for Hq, n_new in ((4, T + 1), (3, 1)):
        q = torch.randn((B, Hq, 128), device="cuda")
        kx = torch.randn((B, Hkv, n_new, 128), device="cuda")
        with pytest.raises(fa.FaTqError):
            fa.attn_append(ck, cv, SEED, q, kx, kx.clone(), pos, *dev, 0.1)
    torch.cuda.synchronize()
    assert np.array_equal(dev[0].cpu().numpy(), kp)
    assert np.array_equal(dev[2].cpu().numpy(), vp)


def test_append_llama_layer_full(gpu_lib):
    """Llama-3-8B-shaped layer (32/8 heads, 32768 slots, K4/V2): one decode token
    appended at the last slot, then one at position 32768 + 1234 (slot 1234);
    the cache is seeded random codes, outputs checked on sampled heads."""
    torch = _torch()
    fa = gpu_lib
    w = workloads.WORKLOADS["llama_layer"]
    B, Hq, Hkv, T = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens
    rng = np.random.default_rng(12)
    kp = rng.integers(0, 256, size=(B, Hkv, T, 1, 64), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(B, Hkv, T, 1, 32), dtype=np.uint8)
    kn = (11.3 * np.exp(0.3 * rng.standard_normal((B, Hkv, T, 1)))).astype(np.float16)
    vn = (11.3 * np.exp(0.3 * rng.standard_normal((B, Hkv, T, 1)))).astype(np.float16)
    dev = _device(fa, kp, kn, vp, vn)
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    bk, c4 = o_cb.codebook(4)
    bv, c2 = o_cb.codebook(2)
    s = o_signs.signs(SEED, 128)
    heads = [(0, 0), (0, 13), (0, 31)]
    for pos in (T - 1, T + 1234):
        kx = torch.randn((B, Hkv, 1, 128), dtype=torch.float32).to(torch.bfloat16)
        vx = torch.randn((B, Hkv, 1, 128), dtype=torch.float32).to(torch.bfloat16)
        q = torch.randn((B, Hq, 128), dtype=torch.float32).to(torch.bfloat16)
        out = fa.attn_append(ck, cv, SEED, q.cuda(), kx.cuda(), vx.cuda(),
                             torch.tensor([pos], dtype=torch.int32, device="cuda"), *dev,
                             1 / np.sqrt(128))
        torch.cuda.synchronize()
        # oracle: encode the new token into its slot, then attend on sampled heads
        k32, v32 = bf16_to_f32(kx), bf16_to_f32(vx)
        kc, kno, _ = codec.encode_mse(k32, s, bk)
        vc, vno, _ = codec.encode_mse(v32, s, bv)
        slot = pos % T
        kp[:, :, slot], kn[:, :, slot] = codec.pack(kc, 4)[:, :, 0], kno[:, :, 0]
        vp[:, :, slot], vn[:, :, slot] = codec.pack(vc, 2)[:, :, 0], vno[:, :, 0]
        ref = o_att.attend_fused(bf16_to_f32(q), kp, kn, vp, vn, [T], 4, 2, c4, c2, s,
                                 1 / np.sqrt(128), heads=heads)
        got = out.cpu().numpy()
        sel = tuple(np.array(heads).T)
        err = float(np.max(np.abs(got[sel] - ref[sel])))
        assert np.array_equal(dev[0][:, :, slot].cpu().numpy(), kp[:, :, slot])
        assert np.array_equal(dev[3][:, :, slot].cpu().numpy().view(np.float16), vn[:, :, slot])
        say(f"append llama pos {pos} (slot {slot}): max abs err {err:.3e}")
        assert err <= ATTN_MAX_ABS


def test_append_graph_replay_matches_eager(gpu_lib):
    """A captured append call, replayed with new positions, tokens and queries written
    into its input buffers between replays, matches the same calls made eagerly on a
    twin cache (every replay compared: output, codes and norms)."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(13)
    B, Hq, Hkv, T = 2, 8, 2, 64
    kp, kn = _history(B, Hkv, T, 4, rng)
    vp, vn = _history(B, Hkv, T, 2, rng)
    graph_cache, eager_cache = _device(fa, kp, kn, vp, vn), _device(fa, kp, kn, vp, vn)
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    q = torch.zeros((B, Hq, 128), device="cuda")
    kx = torch.zeros((B, Hkv, 1, 128), device="cuda")
    vx = torch.zeros((B, Hkv, 1, 128), device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, 128), device="cuda")
    ws = fa.attn_workspace(B, Hq, Hkv, T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attn_append_call(ck, cv, SEED, q, kx, vx, pos, *eager_cache, 0.09, out, ws)()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager_cache[0].copy_(graph_cache[0]), eager_cache[1].copy_(graph_cache[1])
    eager_cache[2].copy_(graph_cache[2]), eager_cache[3].copy_(graph_cache[3])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.attn_append_call(ck, cv, SEED, q, kx, vx, pos, *graph_cache, 0.09, out, ws)()
    for step, p in enumerate([[3, 70], [4, 71], [63, 127], [64, 200]]):
        qn = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).cuda()
        kn_ = torch.from_numpy(rng.standard_normal((B, Hkv, 1, 128)).astype(np.float32)).cuda()
        vn_ = torch.from_numpy(rng.standard_normal((B, Hkv, 1, 128)).astype(np.float32)).cuda()
        pn = torch.tensor(p, dtype=torch.int32, device="cuda")
        ref = fa.attn_append(ck, cv, SEED, qn, kn_, vn_, pn, *eager_cache, 0.09)
        torch.cuda.synchronize()
        q.copy_(qn), kx.copy_(kn_), vx.copy_(vn_), pos.copy_(pn)
        graph.replay()
        torch.cuda.synchronize()
        say(f"graph replay {step} pos {p}")
        assert torch.equal(out, ref), f"replay {step}: output differs from the eager call"
        for g, e in zip(graph_cache, eager_cache):
            assert torch.equal(g, e), f"replay {step}: cache differs from the eager call"

"""GPU parity of the dense-rotation encode and decode (head_dims that are not a power
of two) against the CPU oracle (oracle/dense.py).

Encode: the GPU encodes seeded inputs with the library's rotation matrix; codes are
compared with the oracle's encode of the same values (fp64 product, so a code next to
a decision boundary may differ by one level: the flip budget), norms bit for bit.
Decode: the oracle encodes and packs; the GPU decodes those codes; the result is
compared with the oracle's fp64 decode (relative L2 error per vector).
"""

import numpy as np
import pytest

import workloads
from oracle import codebook as o_cb
from oracle import codec
from oracle import dense
from tests.gpu_helpers import ATTN_MAX_ABS, DECODE_REL_L2, bf16_to_f32, compare_norms, say, FLIP_BUDGET

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _check_codes(gpu_codes, oracle_codes, bits, d, where):
    """gpu_codes [N, nblk, cb] packed, oracle_codes [N, d]: adjacent flips within the
    budget, code 0 past d, bytes equal when nothing flips."""
    n = gpu_codes.shape[0]
    g = codec.unpack(gpu_codes, bits).astype(np.int64)          # [N, nblk * 128]
    assert np.all(g[:, d:] == 0), f"{where}: nonzero code past head_dim"
    diff = g[:, :d] - oracle_codes.astype(np.int64)
    assert np.all(np.abs(diff) <= 1), f"{where}: non-adjacent code mismatch"
    flips = int(np.count_nonzero(diff))
    assert flips <= max(1, FLIP_BUDGET * diff.size), f"{where}: {flips} flips in {diff.size}"
    if flips == 0:
        np.testing.assert_array_equal(gpu_codes, dense.pack_dense(oracle_codes, bits).reshape(gpu_codes.shape))
    return flips


@pytest.mark.parametrize("d", [40, 70, 96, 100, 160, 192])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dense_encode(gpu_lib, d, bits, dtype):
    torch = _torch()
    say(f"dense encode d={d} bits={bits} {dtype}")
    rng = np.random.default_rng(d * 10 + bits)
    B, H, T = 2, 3, 257
    x = rng.standard_normal((B, H, T, d)).astype(np.float32)
    x *= rng.uniform(0.05, 20.0, (B, H, T, 1)).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    if dtype == "bf16":
        xt = xt.to(torch.bfloat16)
    x32 = bf16_to_f32(xt) if dtype == "bf16" else x
    cb = gpu_lib.codebook_init(d, bits)
    r = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).cuda()
    codes, norms = gpu_lib.encode_dense(cb, r, xt)
    torch.cuda.synchronize()
    b, _ = o_cb.codebook(bits, d)
    oc, on, _ = dense.encode_dense(x32.reshape(-1, d), dense.rotation_f32(SEED, d), b)
    flips = _check_codes(codes.cpu().numpy().reshape(B * H * T, -1, codes.shape[-1]), oc, bits, d,
                         f"dense d={d} bits={bits} {dtype}")
    compare_norms(norms.cpu().numpy(), on, f"dense d={d} norms")
    say(f"dense d={d} bits={bits} {dtype}: {flips} flips")


def test_dense_encode_positions_and_strides(gpu_lib):
    """t0 positions (some past t_max: skipped), a strided input view."""
    torch = _torch()
    d, bits, B, H, T, t_max = 96, 4, 3, 2, 50, 64
    rng = np.random.default_rng(5)
    big = torch.from_numpy(rng.standard_normal((B, T, H, 128)).astype(np.float32)).cuda()
    x = big[..., :d].permute(0, 2, 1, 3)               # [B, H, T, d], strides (T*H*128, 128, H*128)
    t0 = torch.tensor([0, 10, 40], dtype=torch.int32, device="cuda")
    cb = gpu_lib.codebook_init(d, bits)
    r = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).cuda()
    codes, norms = gpu_lib.dense_cache_buffers(B, H, t_max, d, bits)
    codes.fill_(0xAB)
    norms.fill_(0x1234)
    gpu_lib.encode_dense(cb, r, x, t_max=t_max, t0=t0, codes=codes, norms=norms)
    torch.cuda.synchronize()
    b, _ = o_cb.codebook(bits, d)
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    x32 = x.cpu().numpy()
    for bi, start in enumerate([0, 10, 40]):
        n_in = min(T, t_max - start)
        oc, on, _ = dense.encode_dense(np.ascontiguousarray(x32[bi, :, :n_in]).reshape(-1, d),
                                       dense.rotation_f32(SEED, d), b)
        _check_codes(gc[bi, :, start:start + n_in].reshape(H * n_in, 1, -1), oc, bits, d, "positions")
        compare_norms(gn[bi, :, start:start + n_in], on, "positions")
        # slots before the start and after the last position are untouched
        assert np.all(gc[bi, :, :start] == 0xAB) and np.all(gc[bi, :, start + n_in:] == 0xAB)


@pytest.mark.parametrize("d,bits", [(40, 4), (70, 3), (96, 2), (100, 4), (160, 3), (192, 4), (192, 2)])
def test_dense_decode(gpu_lib, d, bits):
    torch = _torch()
    say(f"dense decode d={d} bits={bits}")
    rng = np.random.default_rng(d + 100 * bits)
    B, H, T = 2, 2, 300
    x = rng.standard_normal((B, H, T, d)).astype(np.float32) * 3.0
    b, c = o_cb.codebook(bits, d)
    r32 = dense.rotation_f32(SEED, d)
    oc, on, _ = dense.encode_dense(x.reshape(-1, d), r32, b)
    packed = dense.pack_dense(oc, bits).reshape(B, H, T, -1, codec.code_bytes(bits))
    norms = on.reshape(B, H, T).view(np.int16)
    ref = dense.decode_dense(oc, on, r32, c).reshape(B, H, T, d)
    cb = gpu_lib.codebook_init(d, bits)
    r = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).cuda()
    ct, nt = torch.from_numpy(packed).cuda(), torch.from_numpy(norms).cuda()
    out = gpu_lib.decode_dense(cb, r, ct, nt, d).cpu().numpy()
    err = np.linalg.norm(out - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    assert float(err.max()) <= DECODE_REL_L2, float(err.max())
    # bf16 output: the fp32 result rounded to nearest even
    outb = gpu_lib.decode_dense(cb, r, ct, nt, d, out_dtype=torch.bfloat16)
    want = torch.from_numpy(out).cuda().to(torch.bfloat16)
    assert torch.equal(outb.view(torch.int16), want.view(torch.int16))
    # a sub-range of tokens
    part = gpu_lib.decode_dense(cb, r, ct, nt, d, n_tokens=7).cpu().numpy()
    np.testing.assert_array_equal(part, out[:, :, :7])


def test_dense_prefill_slice_sampled(gpu_lib):
    """The first 192 channels of a prefill-shaped slice (8 x 8 x 4096 vectors, bf16 AR(1)
    rho 0.9), all encoded on the GPU, 32768 sampled vectors compared with the oracle."""
    torch = _torch()
    w = workloads.WORKLOADS["prefill"]
    k, _ = workloads.make_kv(w, "cuda", tokens=4096, batch=8)
    x = k[..., :192].contiguous()
    del k
    d, bits = 192, 4
    cb = gpu_lib.codebook_init(d, bits)
    r = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).cuda()
    codes, norms = gpu_lib.encode_dense(cb, r, x)
    torch.cuda.synchronize()
    nvec = x.shape[0] * x.shape[1] * x.shape[2]
    pick = np.sort(np.random.default_rng(1).choice(nvec, 32768, replace=False))
    idx = torch.from_numpy(pick).cuda()
    xs = x.reshape(nvec, d).index_select(0, idx)
    gc = codes.reshape(nvec, -1, codes.shape[-1]).index_select(0, idx).cpu().numpy()
    gn = norms.reshape(nvec).index_select(0, idx).cpu().numpy()
    b, _ = o_cb.codebook(bits, d)
    oc, on, _ = dense.encode_dense(bf16_to_f32(xs), dense.rotation_f32(SEED, d), b)
    flips = _check_codes(gc, oc, bits, d, "prefill dense")
    compare_norms(gn, on, "prefill dense")
    say(f"prefill dense d=192: {flips} flips in {oc.size} codes")


@pytest.mark.parametrize("d", [37, 40, 70, 96, 128])
@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3), (4, 4)])
@pytest.mark.parametrize("flags", [0, "valu"])
def test_dense_attention(gpu_lib, d, kb, vb, flags):
    """Attention over oracle-encoded dense caches (ragged lengths, a zero length, GQA
    groups of 4) against the fp64 definition over the decoded vectors."""
    torch = _torch()
    say(f"dense attention d={d} K{kb}V{vb} {flags or 'mfma'}")
    B, Hq, Hkv, T = 3, 8, 2, 300
    lens = [300, 0, 129]
    rng = np.random.default_rng(d * 100 + kb * 10 + vb)
    k = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    k *= rng.uniform(0.3, 3.0, (1, Hkv, 1, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, d)).astype(np.float32)
    r32 = dense.rotation_f32(SEED, d)
    bk, ck = o_cb.codebook(kb, d)
    bv, cv = o_cb.codebook(vb, d)
    kc, kn, _ = dense.encode_dense(k.reshape(-1, d), r32, bk)
    vc, vn, _ = dense.encode_dense(v.reshape(-1, d), r32, bv)
    kc, vc = kc.reshape(B, Hkv, T, d), vc.reshape(B, Hkv, T, d)
    kn, vn = kn.reshape(B, Hkv, T), vn.reshape(B, Hkv, T)
    dev = "cuda"
    kp = torch.from_numpy(dense.pack_dense(kc, kb).reshape(B, Hkv, T, 1, -1)).to(dev)
    vp = torch.from_numpy(dense.pack_dense(vc, vb).reshape(B, Hkv, T, 1, -1)).to(dev)
    q = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(torch.bfloat16)
    scale = 1 / np.sqrt(d)
    rot = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).to(dev)
    out = gpu_lib.attn_decode_dense(
        gpu_lib.codebook_init(d, kb), gpu_lib.codebook_init(d, vb), rot, q.to(dev), kp,
        torch.from_numpy(kn.view(np.int16)).to(dev), vp, torch.from_numpy(vn.view(np.int16)).to(dev),
        torch.tensor(lens, dtype=torch.int32, device=dev), scale,
        flags=gpu_lib.ATTN_VECTOR_ALU if flags == "valu" else 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = dense.attend_dense(bf16_to_f32(q), kc, kn, vc, vn, lens, r32, ck, cv, scale)
    assert np.all(got[1] == 0.0)
    err = float(np.max(np.abs(got - ref)))
    say(f"dense attention d={d} K{kb}V{vb}: max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS


def test_dense_attention_llama_full(gpu_lib):
    """Attention over dense-rotation caches at the llama layer's full size, in the launch
    the benchmark times (1 x 32 query / 8 KV heads x 32768 tokens, head_dim 128, K4/V2,
    MFMA kernels): the GPU encodes the caches; for KV heads 0 and 5 (query heads 0-3
    and 20-23) the output equals the fp64 definition over those caches' decoded
    vectors."""
    torch = _torch()
    w = workloads.WORKLOADS["llama_layer"]
    B, Hq, Hkv, T, d = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens, w.head_dim
    say("dense attention llama full")
    k, v = workloads.make_kv(w, "cuda")
    q = workloads.make_q(w, "cuda")
    lens_np = workloads.make_seq_lens(w)
    lens = torch.from_numpy(lens_np).cuda()
    scale = 1 / np.sqrt(d)
    cbk, cbv = gpu_lib.codebook_init(d, w.k_bits), gpu_lib.codebook_init(d, w.v_bits)
    rot = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).cuda()
    kc, kn = gpu_lib.encode_dense(cbk, rot, k)
    vc, vn = gpu_lib.encode_dense(cbv, rot, v)
    del k, v
    out = gpu_lib.attn_decode_dense(cbk, cbv, rot, q, kc, kn, vc, vn, lens, scale)
    torch.cuda.synchronize()
    G = Hq // Hkv
    heads = [0, 5]
    qh = [h for g in heads for h in range(g * G, (g + 1) * G)]
    sel = torch.tensor(heads, device="cuda")
    kcodes = codec.unpack(kc.index_select(1, sel).cpu().numpy(), w.k_bits)[..., :d]
    vcodes = codec.unpack(vc.index_select(1, sel).cpu().numpy(), w.v_bits)[..., :d]
    knorm = kn.index_select(1, sel).cpu().numpy().view(np.float16)
    vnorm = vn.index_select(1, sel).cpu().numpy().view(np.float16)
    _, ck = o_cb.codebook(w.k_bits, d)
    _, cv = o_cb.codebook(w.v_bits, d)
    qs = bf16_to_f32(q[:, qh])
    ref = dense.attend_dense(qs, kcodes, knorm, vcodes, vnorm, lens_np,
                             dense.rotation_f32(SEED, d), ck, cv, scale)
    got = out[:, qh].cpu().numpy()
    err = float(np.max(np.abs(got - ref)))
    say(f"dense attention llama full (KV heads {heads}): max abs err {err:.3e}")
    assert err <= ATTN_MAX_ABS


def test_dense_attention_graph_replays(gpu_lib):
    """The dense-attention call (query kernel, attention kernels, output kernel) captured
    in a HIP graph: every replay, with eager work and synchronizations between them,
    equals the eager result bit for bit."""
    torch = _torch()
    d, B, Hq, Hkv, T = 96, 2, 8, 2, 200
    dev = "cuda"
    rng = np.random.default_rng(3)
    cbk, cbv = gpu_lib.codebook_init(d, 4), gpu_lib.codebook_init(d, 2)
    rot = torch.from_numpy(gpu_lib.rotation_dense(SEED, d)).to(dev)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, T, d)).astype(np.float32)).to(dev)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, T, d)).astype(np.float32)).to(dev)
    kc, kn = gpu_lib.encode_dense(cbk, rot, k)
    vc, vn = gpu_lib.encode_dense(cbv, rot, v)
    q = torch.from_numpy(rng.standard_normal((B, Hq, d)).astype(np.float32)).to(dev)
    lens = torch.tensor([200, 77], dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(gpu_lib.attn_dense_workspace_bytes(B, Hq, Hkv, T), dtype=torch.uint8,
                     device=dev)
    eager = gpu_lib.attn_decode_dense(cbk, cbv, rot, q, kc, kn, vc, vn, lens, 0.1).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call = gpu_lib.attn_decode_dense_call(cbk, cbv, rot, q, kc, kn, vc, vn, lens, 0.1, out, ws)
        call()
    for i in range(3):
        out.fill_(float(i) - 7.0)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"

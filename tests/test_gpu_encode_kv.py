"""GPU parity of fa_tq_encode_kv (the keys and values of the same tokens in one call)
against the CPU oracle, and bit for bit against two fa_tq_encode_ex calls."""

import numpy as np
import pytest

import workloads
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import bf16_to_f32, compare_codes, compare_norms, say

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _oracle_encode(x32: np.ndarray, bits: int, seed: int):
    """x32 [..., d] float32 -> (codes [..., nblk, 128], norms f16 [..., nblk])."""
    d = x32.shape[-1]
    s = o_signs.signs(seed, d)
    if bits == 8:
        c, n = codec.encode_u8(x32, s)
    else:
        b, _ = o_cb.codebook(bits)
        c, n, _ = codec.encode_mse(x32, s, b)
    return c.reshape(x32.shape[:-1] + (d // 128, 128)), n


def _filled_cache(fa, B, H, t_max, d, bits, dev, flags=0):
    codes, norms = fa.cache_buffers(B, H, t_max, d, bits, dev, flags)
    codes.fill_(0xAB)
    norms.fill_(0x1234)
    return codes, norms


def _same(a, b, where):
    torch = _torch()
    for x, y, what in zip(a, b, ("codes", "norms")):
        assert torch.equal(x, y), f"{where}: {what} differ from the separate encode"


@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3), (2, 4), (4, 4), (4, 8), (8, 2)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_encode_kv_matches_oracle(gpu_lib, kb, vb, dtype):
    """Ragged sizes (333 tokens, two blocks per vector), per-sequence offsets t0 into a
    longer cache: every written block equals the oracle's, the slots outside [t0, t0 +
    T) keep their contents, and both caches equal those of two separate encodes (8-bit
    pairs take two launches, the others one)."""
    torch = _torch()
    say(f"encode_kv K{kb}V{vb} {dtype}")
    B, H, T, d, t_max = 2, 3, 333, 256, 400
    t0 = [0, 41]
    g = torch.Generator(device="cuda").manual_seed(kb * 10 + vb)
    k = torch.randn((B, H, T, d), generator=g, device="cuda")
    v = torch.randn((B, H, T, d), generator=g, device="cuda") * 3.0
    if dtype == "bf16":
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    cbk, cbv = gpu_lib.codebook_init(128, kb), gpu_lib.codebook_init(128, vb)
    t0_dev = torch.tensor(t0, dtype=torch.int32, device="cuda")
    kc = _filled_cache(gpu_lib, B, H, t_max, d, kb, "cuda")
    vc = _filled_cache(gpu_lib, B, H, t_max, d, vb, "cuda")
    gpu_lib.encode_kv(cbk, cbv, SEED, k, v, t_max=t_max, t0=t0_dev, k_cache=kc, v_cache=vc)
    ks = _filled_cache(gpu_lib, B, H, t_max, d, kb, "cuda")
    vs = _filled_cache(gpu_lib, B, H, t_max, d, vb, "cuda")
    gpu_lib.encode(cbk, SEED, k, t_max=t_max, t0=t0_dev, codes=ks[0], norms=ks[1])
    gpu_lib.encode(cbv, SEED, v, t_max=t_max, t0=t0_dev, codes=vs[0], norms=vs[1])
    torch.cuda.synchronize()
    _same(kc, ks, "keys")
    _same(vc, vs, "values")
    for x, bits, (codes, norms) in ((k, kb, kc), (v, vb, vc)):
        x32 = bf16_to_f32(x) if x.dtype == torch.bfloat16 else x.cpu().numpy()
        oc, on = _oracle_encode(np.ascontiguousarray(x32), bits, SEED)
        gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
        for b in range(B):
            sl = slice(t0[b], t0[b] + T)
            where = f"encode_kv K{kb}V{vb} {dtype} bits {bits} seq {b}"
            compare_codes(gc[b, :, sl].reshape(-1, gc.shape[-1]), oc[b].reshape(-1, 128), bits,
                          where)
            compare_norms(gn[b, :, sl], on[b], where)
            outside = np.ones(t_max, bool)
            outside[sl] = False
            assert np.all(gc[b, :, outside] == 0xAB), where


@pytest.mark.parametrize("flags", ["two_signs+nc", "whole"])
def test_encode_kv_variant_flags(gpu_lib, flags):
    """The encoder variants through the joint call equal two fa_tq_encode_ex calls with
    the same flags: the second sign vector with the corrected norm (one launch), and
    the whole-vector mode with head_dim 192 zero-padded to 256 (two launches)."""
    torch = _torch()
    say(f"encode_kv flags {flags}")
    if flags == "whole":
        fl, d = gpu_lib.WHOLE_VECTOR, 192
        cbk, cbv = gpu_lib.codebook_init(256, 4), gpu_lib.codebook_init(256, 2)
    else:
        fl, d = gpu_lib.TWO_SIGNS | gpu_lib.NORM_CORRECT, 128
        cbk, cbv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 2)
    B, H, T = 3, 2, 517
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.randn((B, H, T, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, T, d), generator=g, device="cuda").to(torch.bfloat16)
    kc, vc = gpu_lib.encode_kv(cbk, cbv, SEED, k, v, flags=fl)
    ks = gpu_lib.encode(cbk, SEED, k, flags=fl)
    vs = gpu_lib.encode(cbv, SEED, v, flags=fl)
    torch.cuda.synchronize()
    _same(kc, ks, f"keys {flags}")
    _same(vc, vs, f"values {flags}")


def test_encode_kv_strided_layouts(gpu_lib):
    """K and V with layouts of their own (token-major slices of larger tensors, one of
    them with the heads interleaved): each cache equals its separate encode."""
    torch = _torch()
    say("encode_kv strided")
    g = torch.Generator(device="cuda").manual_seed(9)
    big_k = torch.randn((2, 4, 300, 256), generator=g, device="cuda").to(torch.bfloat16)
    big_v = torch.randn((2, 300, 4, 128), generator=g, device="cuda").to(torch.bfloat16)
    k = big_k[:, 1:3, 7:207, 128:256]
    v = big_v[:, 50:250, 2:4, :].permute(0, 2, 1, 3)
    assert not k.is_contiguous() and not v.is_contiguous()
    cbk, cbv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 3)
    kc, vc = gpu_lib.encode_kv(cbk, cbv, SEED, k, v, t_max=256)
    ks = gpu_lib.encode(cbk, SEED, k, t_max=256)
    vs = gpu_lib.encode(cbv, SEED, v, t_max=256)
    torch.cuda.synchronize()
    for (a, b), (c, e) in ((kc, ks), (vc, vs)):
        assert torch.equal(a[:, :, :200], c[:, :, :200])
        assert torch.equal(b[:, :, :200], e[:, :, :200])


def test_encode_kv_empty_is_noop(gpu_lib):
    """Zero tokens (or sequences, or heads) is an OK no-op that writes nothing."""
    torch = _torch()
    cbk, cbv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 2)
    for shape in ((2, 3, 0, 128), (0, 3, 5, 128), (2, 0, 5, 128)):
        k = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        kc = _filled_cache(gpu_lib, shape[0], shape[1], 8, 128, 4, "cuda")
        vc = _filled_cache(gpu_lib, shape[0], shape[1], 8, 128, 2, "cuda")
        gpu_lib.encode_kv(cbk, cbv, SEED, k, k.clone(), t_max=8, k_cache=kc, v_cache=vc)
        torch.cuda.synchronize()
        assert torch.all(kc[0] == 0xAB) and torch.all(vc[0] == 0xAB)


def test_encode_kv_llama_layer_full(gpu_lib):
    """Llama-3-8B-shaped layer at full size in the bench's launch (1 x 8 KV heads x
    32768 tokens, K4/V2 in one launch): both caches equal the separate encodes bit for
    bit, and a seeded sample of 16384 vectors of each equals the oracle."""
    torch = _torch()
    w = workloads.WORKLOADS["llama_layer"]
    say("encode_kv llama_layer full")
    k, v = workloads.make_kv(w, "cuda")
    cbk, cbv = gpu_lib.codebook_init(128, w.k_bits), gpu_lib.codebook_init(128, w.v_bits)
    kc, vc = gpu_lib.encode_kv(cbk, cbv, SEED, k, v)
    ks = gpu_lib.encode(cbk, SEED, k)
    vs = gpu_lib.encode(cbv, SEED, v)
    torch.cuda.synchronize()
    _same(kc, ks, "llama keys")
    _same(vc, vs, "llama values")
    nvec = w.batch * w.n_kv_heads * w.tokens
    rng = np.random.default_rng(11)
    idx = torch.from_numpy(np.sort(rng.choice(nvec, 16384, replace=False))).cuda()
    for x, bits, (codes, norms) in ((k, w.k_bits, kc), (v, w.v_bits, vc)):
        xs = x.reshape(nvec, w.head_dim).index_select(0, idx)
        gc = codes.reshape(nvec, -1).index_select(0, idx).cpu().numpy()
        gn = norms.reshape(nvec, -1).index_select(0, idx).cpu().numpy()
        oc, on = _oracle_encode(bf16_to_f32(xs), bits, SEED)
        compare_codes(gc, oc.reshape(-1, 128), bits, f"llama encode_kv {bits}")
        compare_norms(gn, on, f"llama encode_kv {bits}")


def test_encode_kv_graph_replays(gpu_lib):
    """The joint encode captured in a HIP graph: every replay, with eager work and
    synchronizations between them and the caches overwritten before each, equals the
    eager result bit for bit."""
    torch = _torch()
    say("encode_kv graph replays")
    B, H, T, d = 2, 4, 700, 128
    g = torch.Generator(device="cuda").manual_seed(21)
    k = torch.randn((B, H, T, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, T, d), generator=g, device="cuda").to(torch.bfloat16)
    cbk, cbv = gpu_lib.codebook_init(128, 4), gpu_lib.codebook_init(128, 2)
    ek, ev = gpu_lib.encode_kv(cbk, cbv, SEED, k, v)
    kc = gpu_lib.cache_buffers(B, H, T, d, 4, "cuda")
    vc = gpu_lib.cache_buffers(B, H, T, d, 2, "cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call = gpu_lib.encode_kv_call(cbk, cbv, SEED, k, v, *kc, *vc)
        call()
    for i in range(3):
        for t in (*kc, *vc):
            t.fill_(i + 1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(kc, ek, f"keys, replay {i}")
        _same(vc, ev, f"values, replay {i}")

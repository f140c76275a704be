"""GPU parity of fa_tq_encode / fa_tq_decode against the CPU oracle (MI355X)."""

import numpy as np
import pytest

import workloads
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import (DECODE_REL_L2, bf16_to_f32, compare_codes, compare_norms,
                               say)

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


def _check_encode(fa, x, bits, seed=SEED, t_max=None, t0=None, where=""):
    """Encode x (torch [B,H,T,d]) on the GPU and compare every block with the oracle."""
    torch = _torch()
    B, H, T, d = x.shape
    cb = fa.codebook_init(128, bits)
    t_max = T if t_max is None else t_max
    codes, norms = fa.cache_buffers(B, H, t_max, d, bits, x.device)
    codes.fill_(0xAB)
    norms.fill_(0x1234)
    t0_dev = None if t0 is None else torch.tensor(t0, dtype=torch.int32, device=x.device)
    fa.encode(cb, seed, x, t_max=t_max, t0=t0_dev, codes=codes, norms=norms)
    torch.cuda.synchronize()
    x32 = bf16_to_f32(x) if x.dtype == torch.bfloat16 else x.detach().cpu().numpy()
    oc, on = _oracle_encode(np.ascontiguousarray(x32), bits, seed)
    gc = codes.cpu().numpy()
    gn = norms.cpu().numpy()
    offs = [0] * B if t0 is None else t0
    flips = 0
    for b in range(B):
        sl = slice(offs[b], offs[b] + T)
        flips += compare_codes(gc[b, :, sl].reshape(-1, gc.shape[-1]), oc[b].reshape(-1, 128),
                               bits, where)
        compare_norms(gn[b, :, sl], on[b], where)
        # cache positions outside [t0, t0 + T) are untouched
        untouched = np.ones(t_max, bool)
        untouched[sl] = False
        assert np.all(gc[b, :, untouched] == 0xAB), where
    return flips


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 256])
def test_encode_ragged(gpu_lib, bits, dtype, d):
    torch = _torch()
    say(f"encode ragged bits={bits} dtype={dtype} d={d}")
    g = torch.Generator(device="cuda").manual_seed(bits * 100 + d)
    x = torch.randn((2, 3, 333, d), generator=g, device="cuda")
    x = x.to(torch.bfloat16) if dtype == "bf16" else x
    _check_encode(gpu_lib, x, bits, where=f"ragged {bits} {dtype} {d}")


def test_encode_tiny_workload(gpu_lib):
    """Tiny workload: fp32 K and V [1024, 128], K4/V2, rotation seed 42."""
    torch = _torch()
    k, v, _ = workloads.tiny_inputs()
    say("encode tiny K4/V2")
    for arr, bits in ((k, 4), (v, 2)):
        x = torch.from_numpy(arr).reshape(1, 1, 1024, 128).cuda()
        assert _check_encode(gpu_lib, x, bits, where=f"tiny {bits}") == 0


def test_encode_strided_and_offsets(gpu_lib):
    """Non-contiguous input (a token/head slice of a larger tensor), per-sequence
    cache offsets t0, and t_max beyond the written range."""
    torch = _torch()
    say("encode strided + t0")
    g = torch.Generator(device="cuda").manual_seed(7)
    big = torch.randn((3, 5, 400, 256), generator=g, device="cuda").to(torch.bfloat16)
    x = big[:, 1:4, 10:107, 128:256]
    assert not x.is_contiguous()
    _check_encode(gpu_lib, x, 4, t_max=300, t0=[0, 150, 203], where="strided")


def test_encode_edge_values(gpu_lib):
    """Zero vectors, all-equal vectors, tiny values whose squares are subnormal or
    vanish, large values near the fp16 norm limit, and exact boundary ties."""
    torch = _torch()
    say("encode edge values")
    rows = [np.zeros(128), np.full(128, 0.5), np.full(128, -3.0), np.full(128, 1e-20),
            np.full(128, 3e-23), np.full(128, 5000.0), np.full(128, 6e4)]
    x = np.zeros(128)
    x[5] = 1e-30
    rows.append(x)
    x = np.zeros(128)
    x[0], x[1] = 7.0, -7.0
    rows.append(x)
    rng = np.random.default_rng(0)
    rows += list(rng.standard_normal((8, 128)) * np.array([1e-19, 1e-10, 1e10, 1e15, 1e-3, 1, 10, 100])[:, None])
    arr = np.stack(rows).astype(np.float32)
    for bits in (2, 3, 4, 8):
        xt = torch.from_numpy(arr).reshape(1, 1, -1, 128).cuda()
        _check_encode(gpu_lib, xt, bits, where=f"edge f32 {bits}")
        xb = xt.to(torch.bfloat16)
        _check_encode(gpu_lib, xb, bits, where=f"edge bf16 {bits}")


def test_encode_empty_is_noop(gpu_lib):
    torch = _torch()
    cb = gpu_lib.codebook_init(128, 4)
    x = torch.zeros((1, 1, 0, 128), device="cuda", dtype=torch.bfloat16)
    codes, norms = gpu_lib.cache_buffers(1, 1, 4, 128, 4)
    codes.fill_(7)
    gpu_lib.encode(cb, SEED, x, t_max=4, codes=codes, norms=norms)
    torch.cuda.synchronize()
    assert bool((codes == 7).all())


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_decode_every_code_at_every_position(gpu_lib, bits):
    """Unpack: oracle-packed blocks holding every level at every position decode to
    the oracle's fp64 reconstruction within relative L2 1e-5."""
    torch = _torch()
    say(f"decode all codes bits={bits}")
    L = 1 << bits
    pos = np.arange(128)
    codes = np.stack([(pos * 7 + v) % L for v in range(L)]).astype(np.uint8)
    codes = np.concatenate([codes, codes[:, ::-1]], axis=0)
    n = codes.shape[0]
    rng = np.random.default_rng(bits)
    norms = rng.uniform(0.01, 300.0, n).astype(np.float16)
    norms[0] = 0
    packed = codec.pack(codes, bits)
    cb = gpu_lib.codebook_init(128, bits)
    out = gpu_lib.decode(cb, SEED, torch.from_numpy(packed).cuda(),
                         torch.from_numpy(norms.view(np.int16)).reshape(n, 1).cuda(), 128)
    s = o_signs.signs(SEED, 128)
    if bits == 8:
        ref = codec.decode_u8(codes, norms.reshape(n, 1), s)
    else:
        ref = codec.decode_mse(codes, norms.reshape(n, 1), s, o_cb.codebook(bits)[1])
    got = out.cpu().numpy().reshape(n, 128)
    err = np.linalg.norm(got - ref, axis=1)
    scale = np.linalg.norm(ref, axis=1)
    assert np.all(err <= DECODE_REL_L2 * scale + 1e-30)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_encode_decode_roundtrip_d256(gpu_lib, bits):
    """GPU decode of the oracle's own packing of a d=256 batch (two sign slices)."""
    torch = _torch()
    say(f"decode d256 bits={bits}")
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((257, 256)).astype(np.float32)
    c, n = _oracle_encode(x, bits, SEED)
    packed = codec.pack(c.reshape(257, 256), bits)
    cb = gpu_lib.codebook_init(128, bits)
    out = gpu_lib.decode(cb, SEED, torch.from_numpy(packed).cuda(),
                         torch.from_numpy(n.view(np.int16)).cuda(), 256).cpu().numpy()
    s = o_signs.signs(SEED, 256)
    if bits == 8:
        ref = codec.decode_u8(c.reshape(257, 256), n, s)
    else:
        ref = codec.decode_mse(c.reshape(257, 256), n, s, o_cb.codebook(bits)[1])
    err = np.linalg.norm(out - ref, axis=1)
    assert np.all(err <= DECODE_REL_L2 * np.linalg.norm(ref, axis=1))


def test_encode_llama_layer_full(gpu_lib):
    """Llama-3-8B-shaped layer at full size: K4 and V2 for all 2 x 262144 blocks."""
    torch = _torch()
    w = workloads.WORKLOADS["llama_layer"]
    say("encode llama_layer full")
    k, v = workloads.make_kv(w, "cuda")
    total = 0
    for x, bits in ((k, w.k_bits), (v, w.v_bits)):
        total += _check_encode(gpu_lib, x, bits, where=f"llama {bits}")
    say(f"llama_layer flips: {total}")


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_encode_prefill_full_sampled(gpu_lib, bits):
    """Prefill workload at full size ([32, 8, 65536, 256] bf16): encode everything on
    the GPU, compare a seeded sample of 131072 vectors with the oracle."""
    torch = _torch()
    w = workloads.WORKLOADS["prefill"]
    say(f"encode prefill full bits={bits}")
    shape = (w.batch, w.n_kv_heads, w.tokens, w.head_dim)
    x = workloads.ar1(shape, w.rho, 5, "cuda")
    cb = gpu_lib.codebook_init(128, bits)
    codes, norms = gpu_lib.encode(cb, SEED, x)
    torch.cuda.synchronize()
    rng = np.random.default_rng(bits)
    nvec = w.batch * w.n_kv_heads * w.tokens
    pick = np.sort(rng.choice(nvec, 131072, replace=False))
    idx = torch.from_numpy(pick).cuda()
    xs = x.reshape(nvec, w.head_dim).index_select(0, idx)
    gc = codes.reshape(nvec, -1).index_select(0, idx).cpu().numpy()
    gn = norms.reshape(nvec, -1).index_select(0, idx).cpu().numpy()
    del codes, norms, x
    oc, on = _oracle_encode(bf16_to_f32(xs), bits, SEED)
    cbytes = gpu_lib.code_bytes(bits)
    compare_codes(gc.reshape(-1, cbytes), oc.reshape(-1, 128), bits, f"prefill {bits}")
    compare_norms(gn, on, f"prefill {bits}")


@pytest.mark.parametrize("bits", [4, 8])
def test_encode_and_restore_largest_row(gpu_lib, bits):
    """The largest (batch, head) row the library accepts: 8388607 bf16 tokens of
    head_dim 128 (2 GiB - 256 B of input in one row, byte offsets near 2^31).  Tokens
    sampled over the whole row, the last ones included, are compared with the oracle,
    and restored to bf16 (fa_tq_decode_kv) within the decode bound; one more token is
    rejected."""
    torch = _torch()
    fa = gpu_lib
    T = (1 << 31) // 256 - 1
    say(f"encode largest row bits={bits} tokens={T}")
    g = torch.Generator(device="cuda").manual_seed(77 + bits)
    x = torch.empty((1, 1, T, 128), dtype=torch.bfloat16, device="cuda")
    for s0 in range(0, T, 1 << 22):   # fill in slices (fp32 draws, then bf16)
        s1 = min(T, s0 + (1 << 22))
        x[0, 0, s0:s1] = torch.randn((s1 - s0, 128), generator=g, device="cuda").to(torch.bfloat16)
    cb = fa.codebook_init(128, bits)
    codes, norms = fa.encode(cb, SEED, x)
    torch.cuda.synchronize()
    rng = np.random.default_rng(bits)
    pick = np.unique(np.concatenate([rng.choice(T, 2000, replace=False),
                                     np.arange(T - 64, T), np.arange(64)]))
    idx = torch.from_numpy(pick).cuda()
    xs = x[0, 0].index_select(0, idx)
    gc = codes[0, 0].index_select(0, idx).cpu().numpy()
    gn = norms[0, 0].index_select(0, idx).cpu().numpy()
    oc, on = _oracle_encode(bf16_to_f32(xs), bits, SEED)
    cbytes = fa.code_bytes(bits)
    compare_codes(gc.reshape(-1, cbytes), oc.reshape(-1, 128), bits, "largest row")
    compare_norms(gn, on, "largest row")
    # restore the whole row to bf16, check the sampled tokens against the fp64 decode
    out = fa.decode_kv(cb, SEED, codes, norms)
    torch.cuda.synchronize()
    got = bf16_to_f32(out[0, 0].index_select(0, idx)).astype(np.float64)
    s = o_signs.signs(SEED, 128)
    oc2, on2 = oc.reshape(-1, 128), np.asarray(on).reshape(-1, 1)
    ref = (codec.decode_u8(oc2, on2, s) if bits == 8 else
           codec.decode_mse(oc2, on2, s, o_cb.codebook(bits)[1])).reshape(got.shape)
    rel = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    assert rel.max() < 4e-3, rel.max()   # bf16 output: ~2^-9 relative per element
    del out, codes, norms
    with pytest.raises(fa.FaTqError):
        fa.encode(cb, SEED, torch.empty((1, 1, T + 1, 128), dtype=torch.bfloat16, device="cuda"))

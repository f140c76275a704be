"""GPU parity of fa_tq_decode_kv (bulk restore of a packed cache to a bf16 or fp32
K/V tensor in a caller-given layout) against the CPU oracle (MI355X).

Rules: the fp32 output is the same arithmetic as fa_tq_decode (compared bit for
bit) and within the decode bound of the fp64 oracle; each bf16 output is the
round-to-nearest-even bf16 of a value within the fp32 error bound of the fp64
oracle value.
"""

import numpy as np
import pytest

import workloads
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import DECODE_REL_L2, bf16_to_f32, say

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _random_cache(B, H, T, nblk, bits, rng):
    """Seeded packed cache: random code bytes, fp16 norms ~ 11.3 * lognormal(0, 0.3)."""
    cb = codec.code_bytes(bits)
    codes = rng.integers(0, 256, size=(B, H, T, nblk, cb), dtype=np.uint8)
    norms = (11.3 * np.exp(0.3 * rng.standard_normal((B, H, T, nblk)))).astype(np.float16)
    return codes, norms


def _oracle_decode(codes, norms, bits, d):
    """fp64 decode of a packed cache [B, H, T, nblk, cb] -> [B, H, T, d]."""
    s = o_signs.signs(SEED, d)
    c = codec.unpack(codes, bits)
    if bits == 8:
        return codec.decode_u8(c, norms, s)
    return codec.decode_mse(c, norms, s, o_cb.codebook(bits)[1])


def _check_bf16(got_bf16, x64, where):
    """got: numpy float32 (widened bf16); x64: fp64 oracle values.  Rounding is
    monotonic, so a bf16 of some fp32 value within err of x lies between the bf16
    roundings of x - err and x + err; err = 1e-6 * the vector's largest |x| bounds
    the fp32 decode error (about 1e-7 relative in L2)."""
    err = 1e-6 * np.max(np.abs(x64), axis=-1, keepdims=True)
    lo, hi = codec.round_bf16(x64 - err), codec.round_bf16(x64 + err)
    off = (got_bf16 < lo) | (got_bf16 > hi)
    idx = np.argwhere(off)[:6]
    detail = [(float(x64[tuple(i)]), float(got_bf16[tuple(i)])) for i in idx]
    assert not np.any(off), f"{where}: {int(off.sum())} bf16 outputs off (x, got): {detail}"
    exact = int(np.count_nonzero(got_bf16 == codec.round_bf16(x64)))
    say(f"{where}: bf16 {exact} of {got_bf16.size} equal to the nearest bf16 of the fp64 value")


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [128, 256])
def test_decode_kv_fp32_equals_flat_decode(gpu_lib, bits, d):
    """Contiguous fp32 restore == fa_tq_decode (same arithmetic, bit for bit) and
    within the decode bound of the oracle."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(20 + bits + d)
    B, H, T = 2, 3, 77
    codes, norms = _random_cache(B, H, T, d // 128, bits, rng)
    cb = fa.codebook_init(128, bits)
    gc = torch.from_numpy(codes).cuda()
    gn = torch.from_numpy(norms.view(np.int16)).cuda()
    out = fa.decode_kv(cb, SEED, gc, gn, out_dtype=torch.float32)
    flat = fa.decode(cb, SEED, gc, gn, d)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(-1), flat.reshape(-1))
    x64 = _oracle_decode(codes, norms, bits, d)
    g = out.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(g - x64, axis=-1) / np.maximum(np.linalg.norm(x64, axis=-1), 1e-30)
    say(f"decode_kv fp32 bits={bits} d={d}: max rel L2 {rel.max():.2e}")
    assert rel.max() <= DECODE_REL_L2


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_decode_kv_bf16_lmcache_layout(gpu_lib, bits):
    """Restore into the LMCache tensor [2][layers][tokens][hidden]: K and V of one
    layer, heads interleaved along the hidden axis, only the first n_tokens slots."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(40 + bits)
    H, T, n_tok, L, d = 4, 64, 50, 3, 128
    lm = torch.full((2, L, n_tok, H * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    cb = fa.codebook_init(128, bits)
    layer = 1
    for kv in range(2):
        codes, norms = _random_cache(1, H, T, 1, bits, rng)
        view = lm[kv, layer].view(n_tok, H, d).permute(1, 0, 2).unsqueeze(0)
        fa.decode_kv(cb, SEED, torch.from_numpy(codes).cuda(),
                     torch.from_numpy(norms.view(np.int16)).cuda(), n_tokens=n_tok, out=view)
        torch.cuda.synchronize()
        got = bf16_to_f32(view).astype(np.float64)
        x64 = _oracle_decode(codes[:, :, :n_tok], norms[:, :, :n_tok], bits, d)
        _check_bf16(got, x64, f"lmcache bits={bits} kv={kv}")
    # the other layers are untouched
    others = torch.cat([lm[:, :layer], lm[:, layer + 1:]], dim=1)
    assert torch.isnan(others.float()).all()


def test_decode_kv_empty_and_rejects(gpu_lib):
    torch = _torch()
    fa = gpu_lib
    cb = fa.codebook_init(128, 4)
    codes = torch.zeros((1, 2, 8, 1, 64), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((1, 2, 8, 1), dtype=torch.int16, device="cuda")
    out = torch.full((1, 2, 0, 128), 1.0, dtype=torch.bfloat16, device="cuda")
    fa.decode_kv(cb, SEED, codes, norms, n_tokens=0, out=out)   # no-op
    with pytest.raises(fa.FaTqError):
        fa.decode_kv(cb, SEED, codes, norms, n_tokens=9)
    wide = torch.empty((1, 2, 8, 132), dtype=torch.bfloat16, device="cuda")[..., :128]
    with pytest.raises(fa.FaTqError):   # token stride 132 is not a multiple of 8
        fa.decode_kv(cb, SEED, codes, norms, out=wide)


def test_decode_kv_llama_layer_sampled(gpu_lib):
    """Llama-3-8B-shaped K cache (8 heads x 32768 slots, K4) encoded on the GPU,
    restored to bf16; sampled tokens compared with the oracle decode."""
    torch = _torch()
    fa = gpu_lib
    w = workloads.WORKLOADS["llama_layer"]
    k, _ = workloads.make_kv(w, "cuda")
    cb = fa.codebook_init(128, w.k_bits)
    codes, norms = fa.encode(cb, SEED, k)
    out = fa.decode_kv(cb, SEED, codes, norms)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(w.tokens, 256, replace=False))
    heads = [0, 3, 7]
    c = codes.cpu().numpy()[:, heads][:, :, toks]
    n = norms.cpu().numpy().view(np.float16)[:, heads][:, :, toks]
    x64 = _oracle_decode(c, n, w.k_bits, 128)
    got = bf16_to_f32(out[:, heads][:, :, toks]).astype(np.float64)
    _check_bf16(got, x64, "llama K4 bf16 restore")


def test_flat_decode_beyond_one_row(gpu_lib):
    """fa_tq_decode of more vectors than one launch row holds (its fp32 output spans
    more than 2 GiB at head_dim 128: 2^31 / 512 B = 4194303 vectors per row): the
    vectors around the row boundary, the first and the last decode as the oracle
    does; a second, shorter call into the same output leaves the rest untouched."""
    torch = _torch()
    fa = gpu_lib
    bits, d = 4, 128
    per_row = ((1 << 31) - 1) // (d * 4)
    n = per_row + 1001
    rng = np.random.default_rng(77)
    gc = torch.randint(0, 256, (n, 1, 64), dtype=torch.uint8, device="cuda")
    n16 = (11.3 * np.exp(0.3 * rng.standard_normal((n, 1)))).astype(np.float16)
    gn = torch.from_numpy(n16.view(np.int16)).cuda()
    cb = fa.codebook_init(128, bits)
    out = fa.decode(cb, SEED, gc, gn, d)
    torch.cuda.synchronize()
    idx = np.array([0, 1, per_row - 2, per_row - 1, per_row, per_row + 1, n - 2, n - 1])
    ti = torch.from_numpy(idx).cuda()
    codes = gc[ti].cpu().numpy()
    x64 = _oracle_decode(codes.reshape(1, 1, -1, 1, 64), n16[idx].reshape(1, 1, -1, 1), bits, d)
    g = out[ti].cpu().numpy().astype(np.float64).reshape(x64.shape)
    rel = np.linalg.norm(g - x64, axis=-1) / np.linalg.norm(x64, axis=-1)
    assert rel.max() <= DECODE_REL_L2, rel
    # a shorter call (one row) rewrites only its own vectors
    ref_tail = out[per_row:].clone()
    out2 = fa.decode(cb, SEED, gc[:1000], gn[:1000], d, out=out[:1000])
    torch.cuda.synchronize()
    assert out2.data_ptr() == out.data_ptr()
    assert torch.equal(out[per_row:], ref_tail)
    say(f"flat decode of {n} vectors: max rel L2 {rel.max():.2e} at the sampled vectors")

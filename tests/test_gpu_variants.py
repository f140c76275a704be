"""GPU parity of the encoder variants of [turboq] "Encode pipeline" (second sign
vector s2, corrected norm) through encode, decode, attention and append, against
the CPU oracle (MI355X).  Same rules as the base path: codes exact up to the
adjacent-flip budget, norms bit-exact, decode relative L2 <= 1e-5, attention max
abs error <= 2e-3 against the fp64 oracle on the same packed cache."""

import numpy as np
import pytest

import workloads
from oracle import attention as o_att
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import (ATTN_MAX_ABS, DECODE_REL_L2, bf16_to_f32, compare_codes,
                               compare_norms, say)

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _signs(d, two):
    return o_signs.signs(SEED, d), (o_signs.signs2(SEED, d) if two else None)


def _oracle_encode(x32, bits, two, nc):
    d = x32.shape[-1]
    s1, s2 = _signs(d, two)
    if bits == 8:
        c, n = codec.encode_u8(x32, s1, s2)
    else:
        b, cent = o_cb.codebook(bits)
        c, n, _ = codec.encode_mse(x32, s1, b, s2, cent, nc)
    return c.reshape(x32.shape[:-1] + (d // 128, 128)), n


def _compare_encoded(codes, norms, oc, on, x32, bits, nc, where):
    """Codes within the flip budget, norms bit-exact.  An adjacent flip (u exactly on
    a boundary, where the mirrored code of the second sign vector and the code of -u
    differ) changes ||c[codes]||, so with the corrected norm the norms are compared
    with the oracle's quotient for the GPU's own codes."""
    gc = codes.cpu().numpy().reshape(-1, codes.shape[-1])
    flips = compare_codes(gc, oc.reshape(-1, 128), bits, where)
    if nc and flips:
        gcodes = codec.unpack(gc.reshape(-1, 1, gc.shape[-1]), bits).reshape(oc.shape)
        n32 = codec.norm_f32(np.ascontiguousarray(x32).reshape(oc.shape))
        r32 = codec.norm_f32(o_cb.codebook(bits)[1][gcodes])
        on = np.where(r32 > 0, n32 / np.where(r32 > 0, r32, 1), 0).astype(np.float16)
    compare_norms(norms.cpu().numpy(), on, where)
    return flips


def _flags(fa, two, nc):
    return (fa.TWO_SIGNS if two else 0) | (fa.NORM_CORRECT if nc else 0)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("two,nc", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_encode_variants(gpu_lib, bits, two, nc, dtype):
    torch = _torch()
    fa = gpu_lib
    g = torch.Generator(device="cuda").manual_seed(bits * 7 + two * 3 + nc)
    x = torch.randn((2, 3, 301, 256), generator=g, device="cuda")
    x = x.to(torch.bfloat16) if dtype == "bf16" else x
    cb = fa.codebook_init(128, bits)
    if bits == 8 and nc:
        # the corrected norm is defined for the 2-4 bit codebooks: rejected before
        # any launch, the cache left as it was
        codes, norms = fa.cache_buffers(2, 3, 301, 256, 8, x.device)
        codes.fill_(0x5A)
        with pytest.raises(fa.FaTqError) as err:
            fa.encode(cb, SEED, x, codes=codes, norms=norms, flags=_flags(fa, two, nc))
        torch.cuda.synchronize()
        assert err.value.status == fa.FA_TQ_EUNSUPPORTED
        assert torch.all(codes == 0x5A)
        return
    codes, norms = fa.encode(cb, SEED, x, flags=_flags(fa, two, nc))
    torch.cuda.synchronize()
    x32 = bf16_to_f32(x) if dtype == "bf16" else x.cpu().numpy()
    oc, on = _oracle_encode(np.ascontiguousarray(x32), bits, two, nc)
    where = f"encode bits={bits} two={two} nc={nc} {dtype}"
    flips = _compare_encoded(codes, norms, oc, on, x32, bits, nc, where)
    say(f"{where}: {flips} adjacent flips")


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_decode_two_signs(gpu_lib, bits):
    """Decode of an oracle-encoded two-sign cache (fp32 restore) vs the fp64 oracle."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(50 + bits)
    x = rng.standard_normal((2, 3, 45, 256)).astype(np.float32)
    oc, on = _oracle_encode(x, bits, True, bits != 8)
    packed = codec.pack(oc.reshape(x.shape), bits)
    cb = fa.codebook_init(128, bits)
    out = fa.decode_kv(cb, SEED, torch.from_numpy(packed).cuda(),
                       torch.from_numpy(on.view(np.int16)).cuda(), out_dtype=torch.float32,
                       flags=fa.TWO_SIGNS)
    torch.cuda.synchronize()
    s1, s2 = _signs(256, True)
    if bits == 8:
        ref = codec.decode_u8(oc.reshape(x.shape), on, s1, s2)
    else:
        ref = codec.decode_mse(oc.reshape(x.shape), on, s1, o_cb.codebook(bits)[1], s2)
    g = out.cpu().numpy().astype(np.float64)
    rel = np.linalg.norm(g - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    say(f"decode two-sign bits={bits}: max rel L2 {rel.max():.2e}")
    assert rel.max() <= DECODE_REL_L2
    # bf16 restore: the round-to-nearest-even of the same fp32 decode
    ob = fa.decode_kv(cb, SEED, torch.from_numpy(packed).cuda(),
                      torch.from_numpy(on.view(np.int16)).cuda(), out_dtype=torch.bfloat16,
                      flags=fa.TWO_SIGNS)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_to_f32(ob), codec.round_bf16(g).astype(np.float32))


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 2)])
@pytest.mark.parametrize("kb,vb", [(4, 2), (3, 3)])
def test_attention_two_signs(gpu_lib, Hq, Hkv, kb, vb):
    """Attention over a cache encoded with both variants (the corrected norms are
    just stored norms to attention); group 4 runs the MFMA kernel, group 16 the VALU
    one."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(60 + Hkv + kb)
    B, T = 2, 700
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    kc, kn = _oracle_encode(k, kb, True, True)
    vc, vn = _oracle_encode(v, vb, True, True)
    kp, vp = codec.pack(kc.reshape(k.shape), kb), codec.pack(vc.reshape(v.shape), vb)
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    lens = np.array([T, 333], np.int32)
    ck, cv = fa.codebook_init(128, kb), fa.codebook_init(128, vb)
    out = fa.attn_decode(ck, cv, SEED, torch.from_numpy(q).cuda(), torch.from_numpy(kp).cuda(),
                         torch.from_numpy(kn.view(np.int16)).cuda(), torch.from_numpy(vp).cuda(),
                         torch.from_numpy(vn.view(np.int16)).cuda(),
                         torch.from_numpy(lens).cuda(), 1 / np.sqrt(128), flags=fa.TWO_SIGNS)
    torch.cuda.synchronize()
    s1, s2 = _signs(128, True)
    ref = o_att.attend_fused(q, kp, kn, vp, vn, lens, kb, vb, o_cb.codebook(kb)[1],
                             o_cb.codebook(vb)[1], s1, 1 / np.sqrt(128), s2=s2)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    say(f"attention two-sign Hq={Hq} Hkv={Hkv} K{kb}V{vb}: max abs {err:.2e}")
    assert err <= ATTN_MAX_ABS


def test_append_with_variants(gpu_lib):
    """Append then attend with both flags, against the oracle's append_attend."""
    torch = _torch()
    fa = gpu_lib
    rng = np.random.default_rng(70)
    B, Hq, Hkv, T, n_new = 2, 8, 2, 64, 2
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    kc, kn = _oracle_encode(k, 4, True, True)
    vc, vn = _oracle_encode(v, 2, True, True)
    kp, vp = codec.pack(kc.reshape(k.shape), 4), codec.pack(vc.reshape(v.shape), 2)
    dev = [torch.from_numpy(a.copy()).cuda() for a in (kp, kn.view(np.int16), vp, vn.view(np.int16))]
    q = rng.standard_normal((B, Hq, 128)).astype(np.float32)
    kx = rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32)
    vx = rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32)
    pos = [10, T - 1]
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    out = fa.attn_append(ck, cv, SEED, torch.from_numpy(q).cuda(), torch.from_numpy(kx).cuda(),
                         torch.from_numpy(vx).cuda(), torch.tensor(pos, dtype=torch.int32,
                                                                   device="cuda"),
                         *dev, 1 / np.sqrt(128), flags=fa.TWO_SIGNS | fa.NORM_CORRECT)
    torch.cuda.synchronize()
    s1, s2 = _signs(128, True)
    bk, c4 = o_cb.codebook(4)
    bv, c2 = o_cb.codebook(2)
    ref, _ = o_att.append_attend(q, kx, vx, pos, kp, kn, vp, vn, 4, 2, bk, c4, bv, c2, s1,
                                 1 / np.sqrt(128), s2=s2, norm_correct=True)
    compare_codes(dev[0].cpu().numpy().reshape(-1, 64),
                  codec.unpack(kp.reshape(-1, 1, 64), 4).reshape(-1, 128), 4, "append k")
    compare_norms(dev[1].cpu().numpy(), kn, "append k norms")
    compare_norms(dev[3].cpu().numpy(), vn, "append v norms")
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    say(f"append with variants: max abs {err:.2e}")
    assert err <= ATTN_MAX_ABS


def test_encode_variants_llama_layer_full(gpu_lib):
    """The llama-layer K cache (8 x 32768 bf16 vectors, K4) with both variants,
    every block compared with the oracle."""
    torch = _torch()
    fa = gpu_lib
    w = workloads.WORKLOADS["llama_layer"]
    k, _ = workloads.make_kv(w, "cuda")
    cb = fa.codebook_init(128, 4)
    codes, norms = fa.encode(cb, SEED, k, flags=fa.TWO_SIGNS | fa.NORM_CORRECT)
    torch.cuda.synchronize()
    x32 = np.ascontiguousarray(bf16_to_f32(k))
    oc, on = _oracle_encode(x32, 4, True, True)
    flips = _compare_encoded(codes, norms, oc, on, x32, 4, True, "llama K4 variants")
    say(f"llama K4 two-sign + corrected norm: {flips} adjacent flips in {oc.size}")

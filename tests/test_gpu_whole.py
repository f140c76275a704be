"""GPU parity of the whole-vector mode (FA_TQ_WHOLE_VECTOR: one rotation over
head_dim, the codebook of that dimension, one norm per vector) against the CPU
oracle (MI355X): codes exact up to the adjacent-flip budget, norms bit-exact,
decode relative L2 <= 1e-5 against the fp64 oracle."""

import numpy as np
import pytest

import workloads
from oracle import codebook as o_cb
from oracle import codec
from oracle import signs as o_signs
from tests.gpu_helpers import DECODE_REL_L2, bf16_to_f32, compare_codes, compare_norms, say

pytestmark = pytest.mark.gpu
SEED = workloads.ROTATION_SEED


def _torch():
    import torch
    return torch


def _check(fa, x, bits, where, t_max=None, t0=None):
    """Encode x [B, H, T, d] in the whole-vector mode (d zero-padded to the transform
    length d' when it is not 128 or 256), compare codes and norms with the oracle,
    then decode back (fp32, the first d outputs) against the fp64 oracle decode."""
    torch = _torch()
    B, H, T, d = x.shape
    dp = fa.whole_length(d)
    cb = fa.codebook_init(dp, bits)
    t_max = T if t_max is None else t_max
    codes, norms = fa.cache_buffers(B, H, t_max, d, bits, x.device, flags=fa.WHOLE_VECTOR)
    assert codes.shape[3] == dp // 128 and norms.shape[3] == 1
    codes.fill_(0xAB)
    t0d = None if t0 is None else torch.tensor(t0, dtype=torch.int32, device=x.device)
    fa.encode(cb, SEED, x, t_max=t_max, t0=t0d, codes=codes, norms=norms, flags=fa.WHOLE_VECTOR)
    torch.cuda.synchronize()
    x32 = np.ascontiguousarray(bf16_to_f32(x) if x.dtype == torch.bfloat16 else x.cpu().numpy())
    b, c = o_cb.codebook(bits, dp)
    oc, on, _ = codec.encode_mse_whole(x32, o_signs.signs(SEED, dp), b)
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    offs = [0] * B if t0 is None else t0
    flips = 0
    for bb in range(B):
        sl = slice(offs[bb], offs[bb] + T)
        flips += compare_codes(gc[bb, :, sl].reshape(-1, gc.shape[-1]),
                               oc[bb].reshape(-1, 128), bits, where)
        compare_norms(gn[bb, :, sl], on[bb], where)
        rest = np.ones(t_max, bool)
        rest[sl] = False
        assert np.all(gc[bb, :, rest] == 0xAB), where
    # decode back (fp32) against the fp64 oracle decode of the oracle's codes
    out = fa.decode_kv(cb, SEED, codes, norms, out_dtype=torch.float32, flags=fa.WHOLE_VECTOR,
                       head_dim=d)
    torch.cuda.synchronize()
    assert out.shape[-1] == d
    g = out.cpu().numpy().astype(np.float64)
    for bb in range(B):
        sl = slice(offs[bb], offs[bb] + T)
        ref = codec.decode_mse_whole(codec.unpack(gc[bb, :, sl], bits), gn[bb, :, sl, 0].view(np.float16),
                                     o_signs.signs(SEED, dp), c, head_dim=d)
        rel = np.linalg.norm(g[bb, :, sl] - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
        assert rel.max() <= DECODE_REL_L2, (where, rel.max())
    say(f"{where}: {flips} adjacent flips")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [128, 256])
def test_whole_encode_decode(gpu_lib, bits, dtype, d):
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(bits * 11 + d)
    x = torch.randn((2, 3, 257, d), generator=g, device="cuda")
    x = x.to(torch.bfloat16) if dtype == "bf16" else x
    _check(gpu_lib, x, bits, f"whole bits={bits} {dtype} d={d}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [72, 96, 120, 136, 192, 248])
def test_whole_padded_encode_decode(gpu_lib, bits, dtype, d):
    """head_dim not a power of two: zero-padded to 128 or 256 for the transform."""
    torch = _torch()
    g = torch.Generator(device="cuda").manual_seed(bits * 13 + d)
    x = torch.randn((2, 3, 131, d), generator=g, device="cuda")
    x = x.to(torch.bfloat16) if dtype == "bf16" else x
    _check(gpu_lib, x, bits, f"whole padded bits={bits} {dtype} d={d}")


@pytest.mark.parametrize("d", [96, 192])
def test_whole_padded_reads_and_writes_only_head_dim(gpu_lib, d):
    """The padding is zeros, not the memory after the vector: an input that is the
    first d channels of a wider tensor whose other channels hold NaN encodes as the
    contiguous copy does, and decoding into the first d channels of a wider output
    leaves the other channels untouched (bf16 and fp32 outputs)."""
    torch = _torch()
    fa = gpu_lib
    dp = fa.whole_length(d)
    wide = torch.full((2, 3, 70, 320), float("nan"), device="cuda", dtype=torch.bfloat16)
    wide[..., :d] = torch.randn((2, 3, 70, d), device="cuda").to(torch.bfloat16)
    x = wide[..., :d]
    cb = fa.codebook_init(dp, 4)
    c1, n1 = fa.encode(cb, SEED, x, flags=fa.WHOLE_VECTOR)
    c2, n2 = fa.encode(cb, SEED, x.contiguous(), flags=fa.WHOLE_VECTOR)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(n1, n2)
    assert not torch.isnan(n1.view(torch.float16)).any()
    for dt in (torch.bfloat16, torch.float32):
        ref = fa.decode_kv(cb, SEED, c1, n1, out_dtype=dt, flags=fa.WHOLE_VECTOR, head_dim=d)
        big = torch.full((2, 3, 70, 328), 7.0, device="cuda", dtype=dt)
        fa.decode_kv(cb, SEED, c1, n1, out=big[..., 8:8 + d], flags=fa.WHOLE_VECTOR)
        torch.cuda.synchronize()
        assert torch.equal(big[..., 8:8 + d], ref)
        assert torch.all(big[..., :8] == 7) and torch.all(big[..., 8 + d:] == 7)


def test_whole_positions_and_strides(gpu_lib):
    """Start positions per sequence and a non-contiguous input (a slice of a wider
    tensor)."""
    torch = _torch()
    wide = torch.randn((2, 4, 90, 512), device="cuda").to(torch.bfloat16)
    x = wide[:, 1:3, 5:85, 128:384]
    _check(gpu_lib, x, 4, "whole strided", t_max=200, t0=[7, 120])


def test_whole_blocked_mode_differs_only_by_codebook_and_rotation(gpu_lib):
    """At d = 128 the whole-vector mode and the blocked mode are the same transform
    and the same table: identical codes and norms."""
    torch = _torch()
    fa = gpu_lib
    x = torch.randn((1, 2, 100, 128), device="cuda").to(torch.bfloat16)
    cb = fa.codebook_init(128, 3)
    c1, n1 = fa.encode(cb, SEED, x)
    c2, n2 = fa.encode(cb, SEED, x, flags=fa.WHOLE_VECTOR)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(n1, n2)


def test_whole_prefill_slice_sampled(gpu_lib):
    """Prefill-shaped slice (4 x 8 x 65536 tokens, head_dim 256, bf16 AR(1)), 4-bit,
    sampled vectors compared with the oracle."""
    torch = _torch()
    fa = gpu_lib
    w = workloads.WORKLOADS["prefill"]
    k, v = workloads.make_kv(w, "cuda", batch=4)
    del v
    cb = fa.codebook_init(256, 4)
    codes, norms = fa.encode(cb, SEED, k, flags=fa.WHOLE_VECTOR)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    toks = torch.from_numpy(np.sort(rng.choice(k.shape[2], 512, replace=False)))
    xs = np.ascontiguousarray(bf16_to_f32(k[:, :, toks]))
    b, c = o_cb.codebook(4, 256)
    oc, on, _ = codec.encode_mse_whole(xs, o_signs.signs(SEED, 256), b)
    gc = codes[:, :, toks].cpu().numpy()
    flips = compare_codes(gc.reshape(-1, 64), oc.reshape(-1, 128), 4, "prefill whole")
    compare_norms(norms[:, :, toks].cpu().numpy(), on, "prefill whole")
    say(f"prefill slice whole-vector: {flips} flips in {oc.size}")


@pytest.mark.parametrize("bits", [2, 4])
def test_whole_decode_bf16_is_rounded_fp32(gpu_lib, bits):
    """head_dim 256 whole-vector decode to bf16 is the round-to-nearest-even of the
    fp32 decode (the same arithmetic, rounded at the store), in a strided output."""
    torch = _torch()
    fa = gpu_lib
    x = torch.randn((2, 3, 77, 256), device="cuda").to(torch.bfloat16)
    cb = fa.codebook_init(256, bits)
    codes, norms = fa.encode(cb, SEED, x, flags=fa.WHOLE_VECTOR)
    f32 = fa.decode_kv(cb, SEED, codes, norms, out_dtype=torch.float32, flags=fa.WHOLE_VECTOR)
    wide = torch.zeros((2, 3, 77, 384), dtype=torch.bfloat16, device="cuda")
    out = wide[..., 64:320]
    fa.decode_kv(cb, SEED, codes, norms, out=out, flags=fa.WHOLE_VECTOR)
    torch.cuda.synchronize()
    want = codec.round_bf16(f32.cpu().numpy().astype(np.float64))
    np.testing.assert_array_equal(bf16_to_f32(out), want.astype(np.float32))
    assert torch.all(wide[..., :64] == 0) and torch.all(wide[..., 320:] == 0)

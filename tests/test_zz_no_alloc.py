"""fa_tq_attn_decode_noalloc (no workspace: the split partials live in the library's
per-GPU scratch array) against fa_tq_attn_decode with a caller workspace, through the
C ABI: same kernels, so the outputs must be identical bit for bit, and within the
attention tolerance of the fp64 oracle.  Two calls in a row, the second smaller
(the array keeps the first call's partials)."""

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


def _case(B, Hq, Hkv, T, lens, kb, vb, seed):
    import torch
    rng = np.random.default_rng(seed)
    s = o_signs.signs(SEED, 128)
    k = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32) * 2.0
    v = rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)
    kc, kn, _ = codec.encode_mse(k, s, o_cb.codebook(kb)[0])
    vc, vn, _ = codec.encode_mse(v, s, o_cb.codebook(vb)[0])
    kp, vp = codec.pack(kc, kb), codec.pack(vc, vb)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(torch.bfloat16)
    dev = "cuda"
    t = dict(q=q.to(dev), kp=torch.from_numpy(kp).to(dev),
             kn=torch.from_numpy(kn.view(np.int16)).to(dev), vp=torch.from_numpy(vp).to(dev),
             vn=torch.from_numpy(vn.view(np.int16)).to(dev),
             lens=torch.tensor(lens, dtype=torch.int32, device=dev))
    ref = o_att.attend_fused(bf16_to_f32(q), kp, kn, vp, vn, lens, kb, vb, o_cb.codebook(kb)[1],
                             o_cb.codebook(vb)[1], s, 1 / np.sqrt(128))
    return t, ref


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    import torch
    fa = gpu_lib
    for (B, Hq, Hkv, T, lens, kb, vb, seed) in ((2, 32, 8, 3000, [3000, 1711], 4, 2, 1),
                                                 (1, 8, 2, 333, [300], 3, 3, 2)):
        say(f"noalloc B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens} K{kb}V{vb}")
        t, ref = _case(B, Hq, Hkv, T, lens, kb, vb, seed)
        ck, cv = fa.codebook_init(128, kb), fa.codebook_init(128, vb)
        args = (t["q"], t["kp"], t["kn"], t["vp"], t["vn"], t["lens"], 1 / np.sqrt(128))
        out_ws = fa.attn_decode(ck, cv, SEED, *args)
        out_na = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        fa.attn_decode_noalloc(ck, cv, SEED, *args, out_na)
        torch.cuda.synchronize()
        got = out_na.cpu().numpy()
        assert np.array_equal(got, out_ws.cpu().numpy()), "differs from the workspace call"
        err = float(np.max(np.abs(got - ref)))
        say(f"  bit-equal to the workspace call; max abs err vs oracle {err:.3e}")
        assert err <= ATTN_MAX_ABS

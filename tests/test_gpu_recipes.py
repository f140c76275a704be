"""GPU parity on the batched and long-context input recipes at full size.

* The GPU encodes the whole K and V caches of the batched recipe (N(0, 1) with 1 % of
  (head, channel) pairs scaled x20, K3/V3) and of the long-context recipe (AR(1)
  rho = 0.95 with lognormal channel scales, K4/V4); sampled (sequence, KV head)
  slices, every token of them, are compared with the oracle's encode of the same
  bf16 values (codes within the flip budget, fp16 norms bit-exact).  The batched
  sample includes the KV heads that hold the x20 channels.
* Attention runs on caches of the full shapes whose sampled slices hold the
  oracle's encode of the recipe inputs (the other slices are zero and not compared):
  the query heads of the sampled slices are compared with the fp64 oracle.
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


def _oracle_slice(x32: np.ndarray, bits: int):
    """x32 [T, 128] float32 -> (packed [T, 1, cb] uint8, norms f16 [T, 1], codes [T, 128])."""
    b, _ = o_cb.codebook(bits)
    c, n, _ = codec.encode_mse(x32, o_signs.signs(SEED, 128), b)
    return codec.pack(c, bits).reshape(x32.shape[0], 1, -1), n.reshape(-1, 1), c


def _outlier_heads(x):
    """KV heads of sequence 0 ordered by their largest |value| (largest first)."""
    m = x[0].abs().amax(dim=(1, 2)).float().cpu().numpy()
    return [int(h) for h in np.argsort(-m)]


def _slices(name, x):
    """Four (sequence, KV head) slices; for the batched recipe the two KV heads with
    the largest values (the x20 channels) and two others."""
    if name == "batched":
        hs = _outlier_heads(x)
        return [(0, hs[0]), (7, hs[1]), (11, hs[4]), (15, hs[-1])]
    return [(0, 0), (1, 5), (2, 2), (3, 7)]


@pytest.mark.parametrize("name", ["batched", "long_context"])
def test_encode_recipe_full_sampled(gpu_lib, name):
    torch = _torch()
    w = workloads.WORKLOADS[name]
    say(f"encode recipe {name} full")
    k, v = workloads.make_kv(w, "cuda")
    for tag, x, bits in (("K", k, w.k_bits), ("V", v, w.v_bits)):
        cb = gpu_lib.codebook_init(128, bits)
        codes, norms = gpu_lib.encode(cb, SEED, x)
        torch.cuda.synchronize()
        flips = 0
        for b, h in _slices(name, x):
            where = f"{name} {tag}{bits} slice ({b}, {h})"
            say(where)
            op, on, oc = _oracle_slice(bf16_to_f32(x[b, h]), bits)
            gc = codes[b, h].cpu().numpy()
            gn = norms[b, h].cpu().numpy()
            flips += compare_codes(gc.reshape(-1, gc.shape[-1]), oc, bits, where)
            compare_norms(gn, on, where)
        say(f"{name} {tag}{bits}: {flips} flips in the sampled slices")
        del codes, norms


@pytest.mark.parametrize("name", ["batched", "long_context"])
def test_attn_recipe_caches(gpu_lib, name):
    torch = _torch()
    w = workloads.WORKLOADS[name]
    say(f"attn recipe {name}")
    B, Hq, Hkv, T = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens
    grp = Hq // Hkv
    k, v = workloads.make_kv(w, "cuda")
    q = workloads.make_q(w, "cuda")
    lens = workloads.make_seq_lens(w)
    cbk, cbv = gpu_lib.code_bytes(w.k_bits), gpu_lib.code_bytes(w.v_bits)
    kp = np.zeros((B, Hkv, T, 1, cbk), np.uint8)
    vp = np.zeros((B, Hkv, T, 1, cbv), np.uint8)
    kn = np.zeros((B, Hkv, T, 1), np.float16)
    vn = np.zeros((B, Hkv, T, 1), np.float16)
    sl = _slices(name, k)
    for b, h in sl:
        kp[b, h], kn[b, h], _ = _oracle_slice(bf16_to_f32(k[b, h]), w.k_bits)
        vp[b, h], vn[b, h], _ = _oracle_slice(bf16_to_f32(v[b, h]), w.v_bits)
    del k, v
    dev = "cuda"
    ck, cv = gpu_lib.codebook_init(128, w.k_bits), gpu_lib.codebook_init(128, w.v_bits)
    out = gpu_lib.attn_decode(ck, cv, SEED, q, torch.from_numpy(kp).to(dev),
                              torch.from_numpy(kn.view(np.int16)).to(dev),
                              torch.from_numpy(vp).to(dev),
                              torch.from_numpy(vn.view(np.int16)).to(dev),
                              torch.tensor(lens, dtype=torch.int32, device=dev),
                              1 / np.sqrt(128))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    heads = [(b, g * grp + i) for b, g in sl for i in range(grp)]
    ref = o_att.attend_fused(bf16_to_f32(q), kp, kn, vp, vn, lens, w.k_bits, w.v_bits,
                             o_cb.codebook(w.k_bits)[1], o_cb.codebook(w.v_bits)[1],
                             o_signs.signs(SEED, 128), 1 / np.sqrt(128), heads=heads)
    sel = tuple(np.array(heads).T)
    err = float(np.max(np.abs(got[sel] - ref[sel])))
    say(f"{name}: attention on recipe caches, max abs err {err:.3e} over {len(heads)} heads")
    assert err <= ATTN_MAX_ABS

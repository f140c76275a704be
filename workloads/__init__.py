"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds none of the method's arithmetic: it only draws random tensors.
Both the HIP-path tests/bench and the oracle take their inputs from here.

Recipes (all draws are float64/float32 normals from a seeded generator, cast to
bf16 round-to-nearest-even through float32 where a bf16 tensor is asked for):

* ``tiny``: K, V [1024, 128] fp32 ~ N(0, 1) from ``numpy.random.default_rng(0)``
  drawn in the order K, V, then q [128]; rotation seed 42; K4/V2.
* ``llama_layer``: K, V [1, 8, 32768, 128] bf16 AR(1) over tokens with rho = 0.9
  (x_0 = e_0, x_t = rho x_{t-1} + sqrt(1 - rho^2) e_t), each (head, channel)
  multiplied by an independent lognormal(0, 1) scale (separately for K and V);
  q [1, 32, 128] bf16 ~ N(0, 1); K4/V2.
* ``batched``: K, V [16, 8, 8192, 128] bf16 N(0, 1) with 10 (head, channel) pairs
  (1 % of 8 x 128, drawn without replacement, shared over the batch) scaled x20;
  seq_lens ~ uniform integers in [4096, 8192]; q [16, 32, 128]; K3/V3.
* ``long_context``: K, V [4, 8, 131072, 128] bf16 AR(1) rho = 0.95 with lognormal
  channel scales; q [4, 32, 128]; K4/V4.
* ``prefill``: K, V [32, 8, 65536, 256] bf16 AR(1) rho = 0.9 (no channel scales);
  encode only (K4, V2 and the 8-bit variant).

Large tensors are generated with torch on the requested device (a CPU run and a GPU
run of the same recipe draw different, but each seeded, streams); the AR(1)
recurrence is evaluated chunk by chunk in closed form.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROTATION_SEED = 42


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    tokens: int
    head_dim: int
    k_bits: int
    v_bits: int
    kind: str          # "gauss", "ar1", "outlier"
    rho: float = 0.0
    channel_scales: bool = False
    var_lens: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 1024, 128, 4, 2, "gauss"),
    "llama_layer": Workload("llama_layer", 1, 32, 8, 32768, 128, 4, 2, "ar1", 0.9, True),
    "batched": Workload("batched", 16, 32, 8, 8192, 128, 3, 3, "outlier", var_lens=True),
    "long_context": Workload("long_context", 4, 32, 8, 131072, 128, 4, 4, "ar1", 0.95, True),
    "prefill": Workload("prefill", 32, 8, 8, 65536, 256, 4, 2, "ar1", 0.9, False),
}


def tiny_inputs():
    """(K [1024,128] f32, V [1024,128] f32, q [128] f32) from default_rng(0)."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((1024, 128)).astype(np.float32)
    v = rng.standard_normal((1024, 128)).astype(np.float32)
    q = rng.standard_normal(128).astype(np.float32)
    return k, v, q


def _torch():
    import torch
    return torch


def _gen(seed: int, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def ar1(shape, rho: float, seed: int, device="cpu", channel_scales: bool = False,
        chunk: int = 256, dtype=None):
    """AR(1)-over-tokens tensor of shape [B, H, T, D], returned in ``dtype`` (bf16).

    Recurrence x_0 = e_0, x_t = rho x_{t-1} + sqrt(1 - rho^2) e_t over the T axis,
    evaluated per chunk of ``chunk`` tokens as x_chunk = M e_chunk + rho^(j+1) x_prev
    with M[j, k] = rho^(j-k) (k <= j).  Channel scales are lognormal(0, 1) per (H, D).
    """
    torch = _torch()
    dtype = dtype or torch.bfloat16
    B, H, T, D = shape
    g = _gen(seed, device)
    sigma = math.sqrt(1.0 - rho * rho)
    scales = None
    if channel_scales:
        scales = torch.exp(torch.randn((H, D), generator=g, device=device,
                                       dtype=torch.float32))
    out = torch.empty((B, H, T, D), dtype=dtype, device=device)
    C = min(chunk, T)
    j = torch.arange(C, device=device, dtype=torch.float64)
    M = torch.tril(rho ** (j[:, None] - j[None, :]).clamp(min=0)).to(torch.float32)
    carry = (rho ** (j + 1)).to(torch.float32)
    prev = torch.zeros((B, H, 1, D), device=device, dtype=torch.float32)
    for t0 in range(0, T, C):
        c = min(C, T - t0)
        e = torch.randn((B, H, c, D), generator=g, device=device, dtype=torch.float32)
        e = e * sigma
        if t0 == 0:
            e[:, :, 0, :] = e[:, :, 0, :] / sigma
        x = torch.matmul(M[:c, :c], e) + carry[:c, None] * prev
        prev = x[:, :, c - 1:c, :]
        if scales is not None:
            x = x * scales[None, :, None, :]
        out[:, :, t0:t0 + c, :] = x.to(dtype)
    return out


def gaussian_outliers(shape, seed: int, device="cpu", frac: float = 0.01,
                      factor: float = 20.0, dtype=None):
    """N(0,1) tensor [B, H, T, D] with round(frac*H*D) (head, channel) pairs x factor."""
    torch = _torch()
    dtype = dtype or torch.bfloat16
    B, H, T, D = shape
    g = _gen(seed, device)
    n_out = int(round(frac * H * D))
    pick = torch.randperm(H * D, generator=_gen(seed + 7777, "cpu"))[:n_out]
    mult = torch.ones(H * D, dtype=torch.float32)
    mult[pick] = factor
    mult = mult.reshape(H, D).to(device)
    out = torch.empty((B, H, T, D), dtype=dtype, device=device)
    for b in range(B):
        x = torch.randn((H, T, D), generator=g, device=device, dtype=torch.float32)
        out[b] = (x * mult[:, None, :]).to(dtype)
    return out


def gaussian(shape, seed: int, device="cpu", dtype=None):
    torch = _torch()
    dtype = dtype or torch.bfloat16
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device,
                       dtype=torch.float32).to(dtype)


def seq_lens_uniform(batch: int, lo: int, hi: int, seed: int):
    """int32 numpy array of per-sequence lengths, uniform integers in [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def make_kv(w: Workload, device="cpu", tokens: int | None = None, batch: int | None = None,
            seed: int = 0):
    """(K, V) bf16 tensors [B, Hkv, T, D] for workload ``w`` (optionally shrunk)."""
    T = tokens or w.tokens
    B = batch or w.batch
    shape = (B, w.n_kv_heads, T, w.head_dim)
    if w.kind == "ar1":
        k = ar1(shape, w.rho, seed * 10 + 1, device, w.channel_scales)
        v = ar1(shape, w.rho, seed * 10 + 2, device, w.channel_scales)
    elif w.kind == "outlier":
        k = gaussian_outliers(shape, seed * 10 + 1, device)
        v = gaussian_outliers(shape, seed * 10 + 2, device)
    else:
        k = gaussian(shape, seed * 10 + 1, device)
        v = gaussian(shape, seed * 10 + 2, device)
    return k, v


def make_q(w: Workload, device="cpu", batch: int | None = None, seed: int = 0):
    B = batch or w.batch
    return gaussian((B, w.n_q_heads, w.head_dim), seed * 10 + 3, device)


def make_seq_lens(w: Workload, tokens: int | None = None, batch: int | None = None,
                  seed: int = 0):
    T = tokens or w.tokens
    B = batch or w.batch
    if w.var_lens:
        return seq_lens_uniform(B, T // 2, T, seed * 10 + 4)
    return np.full(B, T, np.int32)

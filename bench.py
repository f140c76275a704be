"""Benchmark of the TurboQuant MSE KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in
HBM: encode the bf16 K cache (K4), encode the bf16 V cache (V2), then single-query
decode attention over the packed cache just written.  The workload is the
Llama-3-8B-shaped layer: 1 x 32768 tokens, 32 query / 8 KV heads, head_dim 128.

Prints one JSON line.  ``value`` = algorithmic bytes of a step / step time (GB/s).
Algorithmic bytes: encode = input bytes + packed code bytes + 2-byte norm per
128-block; attention = per (sequence, token, KV head) the K and V code bytes and
the two norms, plus the query and output.  Buffers rotate over several copies so
that consecutive steps do not hit the 256 MB last-level cache with the previous
step's data.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn packed-KV GB/s + encode vectors/s, % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama_layer")
    p.add_argument("--copies", type=int, default=4, help="input/cache copies rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-reps", type=int, default=50)
    return p.parse_args()


def enc_bytes(n_blocks: int, in_bytes: int, bits: int) -> int:
    cb = {2: 32, 3: 48, 4: 64, 8: 128}[bits]
    return n_blocks * (in_bytes + cb + 2)


def attn_bytes(lens, hkv, hq, kb, vb) -> int:
    cbk = {2: 32, 3: 48, 4: 64}[kb]
    cbv = {2: 32, 3: 48, 4: 64}[vb]
    per_tok = hkv * (cbk + cbv + 4)
    return int(np.sum(lens)) * per_tok + len(lens) * hq * 128 * (2 + 4)


def time_events(fn, reps: int) -> float:
    """Average ms per call of ``fn`` over ``reps`` back-to-back calls (HIP events on
    the current stream, which is the stream the library launches on)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def cpu_baseline(w, seed: int, n_slices: int | None = None, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on ``n_slices`` (batch, KV head) slices of the workload
    (default: all of them): encode their K and V blocks in canonical fp32 and run fp64
    attention for their query heads; repeated until ``min_seconds`` have passed."""
    n_slices = n_slices or w.n_kv_heads
    import torch
    from threadpoolctl import threadpool_limits

    import workloads
    from oracle import attention as o_att
    from oracle import codebook as o_cb
    from oracle import codec
    from oracle import signs as o_signs

    T = w.tokens
    k, v = workloads.make_kv(w, "cpu", batch=1)
    q = workloads.make_q(w, "cpu", batch=1)
    k32 = k[:, :n_slices].to(torch.float32).numpy()
    v32 = v[:, :n_slices].to(torch.float32).numpy()
    grp = w.n_q_heads // w.n_kv_heads
    q32 = q[:, :grp * n_slices].to(torch.float32).numpy()
    s = o_signs.signs(seed, 128)
    bk, ck = o_cb.codebook(w.k_bits)
    bv, cv = o_cb.codebook(w.v_bits)
    reps, t_enc, t_att = 0, 0.0, 0.0
    with threadpool_limits(limits=1):
        while reps == 0 or (t_enc + t_att < min_seconds and reps < 50):
            t0 = time.perf_counter()
            kc, kn, _ = codec.encode_mse(k32, s, bk)
            vc, vn, _ = codec.encode_mse(v32, s, bv)
            kp, vp = codec.pack(kc, w.k_bits), codec.pack(vc, w.v_bits)
            t1 = time.perf_counter()
            o_att.attend_fused(q32, kp, kn, vp, vn, [T], w.k_bits, w.v_bits, ck, cv, s,
                               1 / np.sqrt(128))
            t2 = time.perf_counter()
            t_enc += t1 - t0
            t_att += t2 - t1
            reps += 1
    nbytes = (enc_bytes(n_slices * T, 256, w.k_bits) + enc_bytes(n_slices * T, 256, w.v_bits)
              + attn_bytes([T], n_slices, grp * n_slices, w.k_bits, w.v_bits))
    per = (t_enc + t_att) / reps
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_slices} of the {w.n_kv_heads} KV heads of the workload: encode "
                      f"{n_slices * T} K and V blocks each (canonical fp32) + fp64 attention "
                      f"for their {grp * n_slices} query heads; "
                      f"mean of {reps} repetitions: encode {t_enc / reps:.2f} s, attention "
                      f"{t_att / reps:.2f} s; numpy, one thread",
            "seconds": round(t_enc + t_att, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import kv_cache_vector_fa_amd as fa
    import workloads

    fa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.WORKLOADS[args.workload]
    seed = workloads.ROTATION_SEED
    B, Hq, Hkv, T, d = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens, w.head_dim
    R = max(1, args.copies)
    k, v = workloads.make_kv(w, "cuda")
    q = workloads.make_q(w, "cuda")
    lens_np = workloads.make_seq_lens(w)
    lens = torch.from_numpy(lens_np).cuda()
    ks = [k] + [k.clone() for _ in range(R - 1)]
    vs = [v] + [v.clone() for _ in range(R - 1)]
    cbk, cbv = fa.codebook_init(128, w.k_bits), fa.codebook_init(128, w.v_bits)
    caches = [fa.cache_buffers(B, Hkv, T, d, w.k_bits) + fa.cache_buffers(B, Hkv, T, d, w.v_bits)
              for _ in range(R)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = fa.attn_workspace(B, Hq, Hkv, T, d)
    scale = 1 / np.sqrt(d)

    def enc_k(i):
        kc, kn, _, _ = caches[i % R]
        fa.encode(cbk, seed, ks[i % R], codes=kc, norms=kn)

    def enc_v(i):
        _, _, vc, vn = caches[i % R]
        fa.encode(cbv, seed, vs[i % R], codes=vc, norms=vn)

    def attn(i):
        kc, kn, vc, vn = caches[i % R]
        fa.attn_decode(cbk, cbv, seed, q, kc, kn, vc, vn, lens, scale, out=out, workspace=ws)

    def step(i):
        enc_k(i)
        enc_v(i)
        attn(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(step, args.steps)
    wall = time.perf_counter() - t0

    nblk = B * Hkv * T * (d // 128)
    b_ek = enc_bytes(nblk, 256, w.k_bits)
    b_ev = enc_bytes(nblk, 256, w.v_bits)
    b_at = attn_bytes(lens_np, Hkv, Hq, w.k_bits, w.v_bits)
    step_bytes = b_ek + b_ev + b_at

    reps = args.kernel_reps
    kern = {}
    for name, fn, nbytes, vecs in (("encode_k", enc_k, b_ek, nblk), ("encode_v", enc_v, b_ev, nblk),
                                   ("attn_decode", attn, b_at, None)):
        fn(0)
        kms = time_events(fn, reps)
        rec = {"us": round(kms * 1e3, 3), "algorithmic_bytes": nbytes,
               "gbps": round(nbytes / (kms * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(nbytes / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if vecs:
            rec["vectors_per_s"] = round(vecs / (d // 128) / (kms * 1e-3), 1)
        kern[name] = rec
    dom = max(kern, key=lambda n: kern[n]["us"])
    roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["gbps"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[dom]["frac_hbm_peak"], "traffic": None}

    rec = {
        "metric": METRIC,
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; bf16 AR(1) rho 0.9 with lognormal channel scales)",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "tokens": T, "head_dim": d, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "step": "encode K + encode V + decode attention", "copies": R},
        "step_algorithmic_bytes": step_bytes,
        "wall_s_timed": round(wall, 3),
        "kernels": kern,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, seed)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the TurboQuant MSE KV-cache hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in
HBM: encode the bf16 K cache (K4) and the bf16 V cache (V2) in one call
(fa_tq_encode_kv: one launch whose workgroups split between the two), then
single-query decode attention over the packed cache just written.  The workload is the
Llama-3-8B-shaped layer: 1 x 32768 tokens, 32 query / 8 KV heads, head_dim 128.

Prints one JSON line.  ``value`` = algorithmic bytes of a step / step time (GB/s).
Algorithmic bytes: encode = input bytes + packed code bytes + 2-byte norm per
128-block; attention = per (sequence, token, KV head) the K and V code bytes and
the two norms, plus the query and output.  Inputs rotate over 12 copies (an encode
streams about 84 MB, so a copy comes back only after 11 other encodes of its phase,
over 900 MB of traffic) and packed caches over 32 copies (the attention phase cycles
through 840 MB), so no call finds its data in the 256 MB last-level cache.

The K timed steps run in rounds of R steps, phase by phase within a round: R encodes
of K and V back to back, then R attentions, step i's attention reading the cache
copy its encode wrote (every copy holds the same codes).  HIP events at the phase boundaries (on the stream the library launches on)
give each kernel's mean launch-to-launch time without the dispatch of a different
kernel in between, the figure rocprofv3's kernel durations are compared with; the
rounds spread every kernel over the whole timed region, so a clock change on the
box does not land on one kernel only.  The ``roofline.traffic``
figure is read from the committed rocprofv3 counter summary in ``profiles/`` when
the kernel's source file still has the hash recorded there, else it is null.

Other modes:
  --calibrate-copy        before the steps, copy a 256 MiB buffer 5 times (the
                          plain copy whose counters calibrate FETCH_SIZE/WRITE_SIZE);
  --summarize-rocprof DIR print per-kernel means of a rocprofv3 CSV directory
                          (kernel_stats or counter_collection) and exit;
  --cpu-baseline-only     the bounded CPU-oracle baseline of the step alone (no GPU;
                          the GPU run starts it as a child process);
  --cpu-baseline-full     the CPU oracle on every workload at full size (prefill: a
                          stated subset), one worker and N worker processes (no GPU).

Each kernel's per-call distribution (median, p10, p90) comes from a separate pass of
60 calls, each between its own pair of HIP events (``per_call``: steady state, back to
back over the rotating copies), and a cold-HBM pass (``cold_hbm``): a 1 GiB write
before each call, then the call alone between its events; the step figures above
are means over back-to-back calls.  ``attn_decode_graph`` times the attention as a HIP graph of
32 calls over the cache copies (GPU time per call without host launch gaps), and
``attn_decode_vector_alu`` the same calls on the vector-ALU attention kernels
(FA_TQ_ATTN_VECTOR_ALU) for comparison with the matrix-core ones.

After the timed steps (outside them), ``restore_bf16`` times fa_tq_decode_kv restoring
the K cache to bf16 in the LMCache layout, ``encode_k_variants`` the K encode with the
second sign vector and corrected norm, ``prefill_encode_d256`` a head_dim-256 encode in
the whole-vector and blocked modes (and head_dim 192 zero-padded to 256 in the
whole-vector mode, or with the dense random orthogonal rotation),
``attention_other_workloads`` decode attention on the batched
and long-context workloads, and ``append_decode`` reports the decode-loop call
fa_tq_attn_append: one new token per sequence quantized into the full cache (ring
slot), then attention over all T_max slots.  Eight such calls with distinct
positions are captured in one HIP graph and replayed, so the figure is GPU time per
call without host launch gaps.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn packed-KV GB/s + encode vectors/s, % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0
ROUND = 10   # timed steps per round (see the module docstring)
CSRC = os.path.join(ROOT, "kv_cache_vector_fa_amd", "csrc")
# kernel name prefix (as rocprofv3 reports it) -> source file that defines it
KERNEL_SOURCE = {"encode_kernel": "codec.hip", "encode_pair_kernel": "codec.hip",
                 "attn_mfma_kernel": "attn_mfma.hip",
                 "attn_merge_splits_kernel": "attn_mfma.hip", "attn_split_kernel": "attn.hip",
                 "attn_merge_kernel": "attn.hip", "decode_kv_kernel": "codec.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "llama_layer_pmc_traffic.txt")
CALIB_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="llama_layer")
    p.add_argument("--copies", type=int, default=12, help="input copies rotated per step")
    p.add_argument("--cache-copies", type=int, default=32, help="packed-cache copies rotated")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-append", action="store_true", help="skip the append_decode figure")
    p.add_argument("--no-cold-hbm", action="store_true",
                   help="skip the cold-HBM pass (profiled runs: kernel averages of steady-state "
                        "calls only)")
    p.add_argument("--calibrate-copy", action="store_true")
    p.add_argument("--summarize-rocprof", metavar="DIR")
    p.add_argument("--cpu-baseline-only", action="store_true")
    p.add_argument("--cpu-baseline-full", action="store_true")
    p.add_argument("--prefill-only", action="store_true",
                   help="run only the prefill-slice encode figures (whole-vector, blocked, "
                        "8-bit, padded and dense-rotation head_dim 192) and print them")
    p.add_argument("--workers", type=int, default=0,
                   help="CPU-oracle worker processes (default: os.cpu_count(), at most 16)")
    return p.parse_args()


def enc_bytes(n_blocks: int, in_bytes: int, bits: int) -> int:
    cb = {2: 32, 3: 48, 4: 64, 8: 128}[bits]
    return n_blocks * (in_bytes + cb + 2)


def attn_bytes(lens, hkv, hq, kb, vb) -> int:
    cbk = {2: 32, 3: 48, 4: 64}[kb]
    cbv = {2: 32, 3: 48, 4: 64}[vb]
    per_tok = hkv * (cbk + cbv + 4)
    return int(np.sum(lens)) * per_tok + len(lens) * hq * 128 * (2 + 4)


def source_hash(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_kernel(name: str) -> str:
    n = name.split("(anonymous namespace)::")[-1]
    n = re.sub(r"^void ", "", n)
    return n.split("(")[0].strip()


def summarize_rocprof(d: str) -> None:
    """Per-kernel means of the rocprofv3 CSV files in ``d``."""
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# {os.path.basename(f)}: kernel | calls | average_ns | min_ns | max_ns")
        for r in csv.DictReader(open(f)):
            print(f"{short_kernel(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                  f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
        dur = {}
        for r in csv.DictReader(open(f)):
            if "Kernel_Name" in r and "Start_Timestamp" in r and "End_Timestamp" in r:
                dur.setdefault(short_kernel(r["Kernel_Name"]), []).append(
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        print(f"# {os.path.basename(f)}: kernel | dispatches | p10_ns | median_ns | p90_ns")
        for k, v in dur.items():
            p10, p50, p90 = np.percentile(v, [10, 50, 90])
            print(f"{k} | {len(v)} | {p10:.0f} | {p50:.0f} | {p90:.0f}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg, disp = {}, {}
        for r in csv.DictReader(open(f)):
            k = short_kernel(r["Kernel_Name"])
            agg.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
            agg[k][r["Counter_Name"]] += float(r["Counter_Value"])
            disp.setdefault(k, set()).add(r["Dispatch_Id"])
        print(f"# {os.path.basename(f)}: kernel | dispatches | counter=mean per dispatch")
        for k, cs in agg.items():
            n = len(disp[k])
            print(f"{k} | {n} | " + " ".join(f"{c}={v / n:.6g}" for c, v in sorted(cs.items())))


def traffic_for(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, or None
    when it is absent or the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals, hashes = {}, {}
    for line in open(TRAFFIC_FILE):
        f = [x.strip() for x in line.split("|")]
        if f[0] == "source_sha256" and len(f) == 3:
            hashes[f[1]] = f[2]
        elif f[0] == "traffic" and len(f) >= 3:
            vals[f[1]] = float(f[2])
    src = next((v for p, v in KERNEL_SOURCE.items() if kernel.startswith(p)), None)
    if kernel not in vals or src is None or hashes.get(src) != source_hash(src):
        return None
    return vals[kernel]


def per_call_distribution(calls, n=60) -> dict:
    """Median, p10 and p90 (us) of n single calls, each between its own pair of HIP
    events on the current stream (calls rotate over the given list)."""
    import torch
    for c in calls[:4]:
        c()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        calls[i % len(calls)]()
        e1.record()
    torch.cuda.synchronize()
    us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"median_us": round(float(p50), 3), "p10_us": round(float(p10), 3),
            "p90_us": round(float(p90), 3), "calls": n}


def attention_graph(fa, cbk, cbv, seed, q, caches, lens, scale, out, ws, nbytes, flags=0,
                    n_calls=32, replays=10) -> dict:
    """GPU time per attention call from replays of a HIP graph of n_calls calls over
    the cache copies (no host launch gaps), with the given variant flags."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls = [fa.attn_decode_call(cbk, cbv, seed, q, *c, lens, scale, out, ws, flags=flags)
                 for c in caches]
        for i in range(n_calls):
            calls[i % len(calls)]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls = [fa.attn_decode_call(cbk, cbv, seed, q, *c, lens, scale, out, ws, flags=flags)
                 for c in caches]
        for i in range(n_calls):
            calls[i % len(calls)]()
    graph.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    us = float(np.median(per))
    gbs = nbytes / (us * 1e-6) / 1e9
    p10, p90 = np.percentile(per, [10, 90])
    return {"us": round(us, 3), "p10_us": round(float(p10), 3), "p90_us": round(float(p90), 3),
            "gbps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": f"median over {replays} replays of a HIP graph of {n_calls} calls"}


def large_groups(fa, seed) -> dict:
    """Decode attention at group sizes above the matrix-core tile's 8 query heads (the
    group split over workgroups per KV head, each reading that KV head's codes): 1 x 8
    KV heads x 32768 slots with 128 query heads (G = 16; also on the vector-ALU
    kernels) and 4 x 1 KV head x 65536 slots with 32 query heads (multi-query, G = 32).
    K4/V2 caches of seeded random codes with unit norms, copies over >= 768 MB, HIP
    graph per call; algorithmic bytes count the cache once."""
    import torch
    res = {}
    gen = torch.Generator(device="cuda").manual_seed(seed)
    cbk, cbv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    for name, (B, Hq, Hkv, T) in (("g16", (1, 128, 8, 32768)), ("mqa_g32", (4, 32, 1, 65536))):
        lens_np = np.full(B, T, np.int32)
        nbytes = attn_bytes(lens_np, Hkv, Hq, 4, 2)
        copies = max(1, -(-768_000_000 // nbytes))
        caches = []
        for _ in range(copies):
            kc, kn = fa.cache_buffers(B, Hkv, T, 128, 4)
            vc, vn = fa.cache_buffers(B, Hkv, T, 128, 2)
            kc.random_(0, 256, generator=gen)
            vc.random_(0, 256, generator=gen)
            kn.fill_(0x3C00)   # fp16 1.0
            vn.fill_(0x3C00)
            caches.append((kc, kn, vc, vn))
        q = torch.randn((B, Hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
        lens = torch.from_numpy(lens_np).cuda()
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        ws = fa.attn_workspace(B, Hq, Hkv, T, 128)
        rec = attention_graph(fa, cbk, cbv, seed, q, caches, lens, 1 / np.sqrt(128), out, ws,
                              nbytes)
        rec["shape"] = f"{B} x {Hkv} KV heads x {T} slots, {Hq} query heads (G = {Hq // Hkv})"
        rec["copies"] = copies
        if Hq // Hkv <= 16:
            rec["vector_alu"] = attention_graph(fa, cbk, cbv, seed, q, caches, lens,
                                                1 / np.sqrt(128), out, ws, nbytes,
                                                flags=fa.ATTN_VECTOR_ALU, n_calls=4, replays=3)
        res[name] = rec
        del caches, ws
    return res


def cold_hbm(calls, n=20, flush_bytes=1 << 30) -> dict:
    """Cold-HBM time per call: before each call a 1 GiB scratch buffer is written (the
    last-level cache then holds none of the call's data), and only the call itself lies
    between its pair of HIP events.  Median, p10, p90 over n calls."""
    import torch
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    us = []
    for i in range(n):
        scratch.fill_(i & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"median_us": round(float(p50), 3), "p10_us": round(float(p10), 3),
            "p90_us": round(float(p90), 3), "calls": n, "flush": "1 GiB write before each call"}


def append_decode(fa, w, cbk, cbv, seed, q, cache, out, ws, scale, replays=20) -> dict:
    """GPU time per fa_tq_attn_append call (one token per sequence, full cache),
    from replays of a HIP graph holding eight calls at distinct positions."""
    import torch
    B, Hq, Hkv, T, d = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens, w.head_dim
    P = 8
    g = torch.Generator(device="cpu").manual_seed(1234)
    new = [(torch.randn((B, Hkv, 1, d), generator=g).to(torch.bfloat16).cuda(),
            torch.randn((B, Hkv, 1, d), generator=g).to(torch.bfloat16).cuda()) for _ in range(P)]
    pos = [torch.full((B,), T - 1 + i, dtype=torch.int32, device="cuda") for i in range(P)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls = [fa.attn_append_call(cbk, cbv, seed, q, new[i][0], new[i][1], pos[i], *cache,
                                     scale, out, ws) for i in range(P)]
        for c in calls:     # eager warm-up on the capture stream
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls = [fa.attn_append_call(cbk, cbv, seed, q, new[i][0], new[i][1], pos[i], *cache,
                                     scale, out, ws) for i in range(P)]
        for c in calls:
            c()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * P)
    kb, vb = fa.code_bytes(w.k_bits), fa.code_bytes(w.v_bits)
    nbytes = (B * Hkv * 256 * 2 + B * Hkv * (kb + vb + 4)
              + attn_bytes(np.full(B, T), Hkv, Hq, w.k_bits, w.v_bits))
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us_per_call": round(us, 3), "new_tokens_per_sequence": 1, "attended_slots": T,
            "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "timing": "HIP graph of 8 calls"}


def restore_bf16(fa, w, cbk, seed, caches, reps=64) -> dict:
    """GPU time of fa_tq_decode_kv restoring the whole K cache to bf16 in the LMCache
    layout [tokens][heads * head_dim] (the serde restore path), over the rotating
    cache copies of the step."""
    import torch
    B, Hkv, T, d = w.batch, w.n_kv_heads, w.tokens, w.head_dim
    lm = torch.empty((B, T, Hkv * d), dtype=torch.bfloat16, device="cuda")
    view = lm.view(B, T, Hkv, d).permute(0, 2, 1, 3)
    calls = [fa.decode_kv_call(cbk, seed, c[0], c[1], view) for c in caches]
    for call in calls:
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nblk = B * Hkv * T * (d // 128)
    nbytes = nblk * (fa.code_bytes(w.k_bits) + 2 + 256)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "what": "packed K cache -> bf16 [tokens][heads*head_dim]"}


def dense_attention(fa, w, seed, k, v, q, lens, lens_np, scale) -> dict:
    """Decode attention over dense-rotation caches of the same layer shape (head_dim
    128, K4/V2): the keys and values encoded with the dense rotation, cloned to copies
    holding more than 768 MB of attention bytes, calls rotating over them; a small
    kernel maps the query into the attention kernels' frame and the merge applies R^T
    (fa_tq_attn_decode_dense)."""
    import torch
    B, Hq, Hkv, T, d = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens, w.head_dim
    cbk, cbv = fa.codebook_init(d, w.k_bits), fa.codebook_init(d, w.v_bits)
    rot = torch.from_numpy(fa.rotation_dense(seed, d)).cuda()
    kc, kn = fa.encode_dense(cbk, rot, k)
    vc, vn = fa.encode_dense(cbv, rot, v)
    nbytes = attn_bytes(lens_np, Hkv, Hq, w.k_bits, w.v_bits)
    copies = max(1, -(-768_000_000 // nbytes))
    caches = [(kc, kn, vc, vn)] + [tuple(t.clone() for t in (kc, kn, vc, vn))
                                   for _ in range(copies - 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.attn_dense_workspace_bytes(B, Hq, Hkv, T), dtype=torch.uint8,
                     device="cuda")
    # a HIP graph of 32 calls (each: query kernel, attention kernels, output kernel),
    # replayed; the calls are created inside the capture (on its stream)
    n_calls = 32
    for i in range(4):
        fa.attn_decode_dense(cbk, cbv, rot, q, *caches[i % copies], lens, scale, out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls = [fa.attn_decode_dense_call(cbk, cbv, rot, q, *caches[i % copies], lens, scale,
                                           out, ws) for i in range(n_calls)]
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    times = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(10):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    us = float(np.median(times))
    gbs = nbytes / (us * 1e-6) / 1e9
    res = {"us": round(us, 2), "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "copies": copies,
           "timing": f"median over 10 replays of a HIP graph of {n_calls} calls"}
    del g, calls
    del caches, kc, kn, vc, vn, ws
    return res


def encode_separate(enc_k, enc_v, K, C, nblk, w) -> dict:
    """The step's encodes as two calls (fa_tq_encode of K, then of V), timed like the
    step: rounds of R encodes of K, then R of V, over the same copies."""
    import torch
    for i in range(4):
        enc_k[i % C]()
        enc_v[i % C]()
    rounds = [(s0, min(K, s0 + ROUND)) for s0 in range(0, K, ROUND)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(rounds) + 1)]
    torch.cuda.synchronize()
    for r, (s0, s1) in enumerate(rounds):
        for j, c in enumerate((enc_k, enc_v)):
            ev[2 * r + j].record()
            for i in range(s0, s1):
                c[i % C]()
    ev[-1].record()
    torch.cuda.synchronize()
    out = {}
    for j, (name, bits) in enumerate((("encode_k", w.k_bits), ("encode_v", w.v_bits))):
        us = sum(ev[2 * r + j].elapsed_time(ev[2 * r + j + 1]) for r in range(len(rounds))) \
            * 1e3 / K
        nb = enc_bytes(nblk, 256, bits)
        gbs = nb / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 3), "algorithmic_bytes": nb, "gbps": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    out["sum_us"] = round(out["encode_k"]["us"] + out["encode_v"]["us"], 3)
    return out


def encode_variants(fa, w, cbk, seed, ks, caches, reps=20) -> dict:
    """GPU time of the K encode with the second sign vector and the corrected norm
    (fa_tq_encode_ex), over the same rotating input and cache copies as the step."""
    import torch
    flags = fa.TWO_SIGNS | fa.NORM_CORRECT
    calls = [fa.encode_call(cbk, seed, k, c[0], c[1], flags=flags) for k, c in zip(ks, caches)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nblk = w.batch * w.n_kv_heads * w.tokens * (w.head_dim // 128)
    nbytes = enc_bytes(nblk, 256, w.k_bits)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 3), "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "flags": "two signs + corrected norm"}


def prefill_whole(fa, seed, reps=10) -> dict:
    """Encode of a prefill-shaped K slice (8 x 8 KV heads x 16384 tokens, head_dim 256,
    bf16 AR(1) rho 0.9, 512 MiB: larger than the last-level cache) with 4-bit codes,
    in the whole-vector mode (one 256-point rotation, the d = 256 codebook, one norm
    per vector) and in the blocked mode (two 128-blocks), for comparison; the blocked
    8-bit uniform grid (turboq8); and the first 192 channels of the same vectors (a
    contiguous head_dim-192 tensor) in the whole-vector mode, zero-padded to 256, and
    with the dense random orthogonal rotation (``dense_d192``)."""
    import torch
    import workloads
    w = workloads.WORKLOADS["prefill"]
    k, v = workloads.make_kv(w, "cuda", tokens=16384, batch=8)
    del v
    B, H, T, d = k.shape
    out = {}
    cb256 = fa.codebook_init(256, 4)
    for mode, cb, flags in (("whole", cb256, fa.WHOLE_VECTOR),
                            ("blocked", fa.codebook_init(128, 4), 0),
                            ("blocked_8bit", fa.codebook_init(128, 8), 0),
                            ("whole_padded_d192", cb256, fa.WHOLE_VECTOR)):
        x = k[..., :192].contiguous() if mode == "whole_padded_d192" else k
        d = x.shape[-1]
        codes, norms = fa.cache_buffers(B, H, T, d, cb.bits, flags=flags)
        nnorm = norms.shape[-1]
        call = fa.encode_call(cb, seed, x, codes, norms, flags=flags)
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nvec = B * H * T
        nbytes = nvec * (2 * d + codes.shape[-2] * fa.code_bytes(cb.bits) + 2 * nnorm)
        gbs = nbytes / (us * 1e-6) / 1e9
        # round trip on the GPU over the first sequence (8 heads x 16384 vectors):
        # mean ||x - x^||^2 / ||x||^2 per vector, x^ restored by fa_tq_decode_kv in fp32
        xr = fa.decode_kv(cb, seed, codes[:1].contiguous(), norms[:1].contiguous(),
                          out_dtype=torch.float32, flags=flags, head_dim=d)
        x0 = x[:1].float()
        rel = ((x0 - xr) ** 2).sum(-1) / (x0 ** 2).sum(-1).clamp_min(1e-30)
        out[mode] = {"us": round(us, 1), "vectors_per_s": round(nvec / (us * 1e-6), 1),
                     "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "roundtrip_rel_mse": float(rel.mean().item()),
                     "roundtrip_vectors": int(rel.numel())}
        del xr, x0, rel
        del codes, norms, x
    # the same first 192 channels with the dense random orthogonal rotation (the other
    # option for a head_dim that is not a power of two): d^2 multiply-adds per vector
    x = k[..., :192].contiguous()
    d = 192
    cb = fa.codebook_init(d, 4)
    rot = torch.from_numpy(fa.rotation_dense(seed, d)).cuda()
    codes, norms = fa.encode_dense(cb, rot, x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fa.encode_dense(cb, rot, x, codes=codes, norms=norms)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nvec = B * H * T
    nbytes = nvec * (2 * d + codes.shape[-2] * fa.code_bytes(4) + 2)
    gbs = nbytes / (us * 1e-6) / 1e9
    # matrix-core work as executed: the hi and lo halves of R, 2 d^2 flops each
    tflops = 2 * 2 * d * d * nvec / (us * 1e-6) / 1e12
    # restore of the whole slice to bf16 (R^T times the centroids' hi and lo halves)
    xb = torch.empty_like(x)
    fa.decode_dense(cb, rot, codes, norms, d, out=xb)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fa.decode_dense(cb, rot, codes, norms, d, out=xb)
    e1.record()
    torch.cuda.synchronize()
    dus = e0.elapsed_time(e1) * 1e3 / reps
    dbytes = nvec * (codes.shape[-2] * fa.code_bytes(4) + 2 + 2 * d)
    del xb
    xr = fa.decode_dense(cb, rot, codes[:1].contiguous(), norms[:1].contiguous(), d)
    x0 = x[:1].float()
    rel = ((x0 - xr) ** 2).sum(-1) / (x0 ** 2).sum(-1).clamp_min(1e-30)
    out["dense_d192"] = {"us": round(us, 1), "vectors_per_s": round(nvec / (us * 1e-6), 1),
                         "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                         "mfma_tflops": round(tflops, 1),
                         "frac_mfma_fp16_peak": round(tflops / 2500.0, 4),
                         "decode_bf16_us": round(dus, 1),
                         "decode_bf16_gbps": round(dbytes / (dus * 1e-6) / 1e9, 1),
                         "roundtrip_rel_mse": float(rel.mean().item()),
                         "roundtrip_vectors": int(rel.numel())}
    del codes, norms, x, xr, x0, rel
    del k
    return out


def other_attention(fa, seed, reps=20) -> dict:
    """GPU time of fa_tq_attn_decode on the batched workload (16 sequences x 8 KV heads,
    8192 slots, lengths 4096..8192, K3/V3) and the long-context one (4 x 8 x 131072,
    K4/V4): caches encoded from the seeded inputs, calls rotating over enough cache
    copies (at least 768 MB of attention bytes) that the working set exceeds the
    256 MB last-level cache."""
    import torch
    import workloads
    out = {}
    for name in ("batched", "long_context"):
        w = workloads.WORKLOADS[name]
        B, Hq, Hkv, T, d = w.batch, w.n_q_heads, w.n_kv_heads, w.tokens, w.head_dim
        k, v = workloads.make_kv(w, "cuda")
        q = workloads.make_q(w, "cuda")
        lens_np = workloads.make_seq_lens(w)
        lens = torch.from_numpy(lens_np).cuda()
        cbk, cbv = fa.codebook_init(128, w.k_bits), fa.codebook_init(128, w.v_bits)
        kc, kn = fa.encode(cbk, seed, k)
        vc, vn = fa.encode(cbv, seed, v)
        enc = {}
        for tag, cb, x, c, n_ in (("encode_k", cbk, k, kc, kn), ("encode_v", cbv, v, vc, vn)):
            call = fa.encode_call(cb, seed, x, c, n_)
            call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                call()
            e1.record()
            torch.cuda.synchronize()
            eus = e0.elapsed_time(e1) * 1e3 / 3
            nblk = B * Hkv * T
            eb = enc_bytes(nblk, 256, cb.bits)
            enc[tag] = {"us": round(eus, 1), "vectors_per_s": round(nblk / (eus * 1e-6), 1),
                        "algorithmic_bytes": int(eb), "gbps": round(eb / eus / 1e3, 1),
                        "frac_hbm_peak": round(eb / eus / 1e3 / HBM_PEAK_GBS, 4)}
        del k, v
        nbytes = attn_bytes(lens_np, Hkv, Hq, w.k_bits, w.v_bits)
        copies = max(1, -(-768_000_000 // nbytes))
        caches = [(kc, kn, vc, vn)] + [tuple(t.clone() for t in (kc, kn, vc, vn))
                                       for _ in range(copies - 1)]
        o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        ws = fa.attn_workspace(B, Hq, Hkv, T, d)
        calls = [fa.attn_decode_call(cbk, cbv, seed, q, *c, lens, 1 / np.sqrt(d), o, ws)
                 for c in caches]
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 1), "algorithmic_bytes": int(nbytes), "gbps": round(gbs, 1),
                     "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "cache_copies": copies,
                     "shape": f"{B}x{Hkv}x{T} K{w.k_bits}/V{w.v_bits}, {Hq} query heads",
                     "per_call": per_call_distribution(calls, 30),
                     "graph": attention_graph(fa, cbk, cbv, seed, q, caches, lens,
                                              1 / np.sqrt(d), o, ws, nbytes,
                                              n_calls=max(8, len(caches)), replays=5),
                     **enc}
        del caches, kc, kn, vc, vn, ws, o
    return out


# ---------------------------------------------------------------- CPU-oracle baseline
# Work units are independent (sequence, KV head) slices (prefill: (layer, KV head));
# the N-worker runs fork processes that share the parent's input arrays.  Nothing here
# touches the GPU: the GPU run starts this leg as a child process.
_UNITS: dict = {}


def _cpu_info(workers: int) -> dict:
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{dep.get('name')} {dep.get('version')}"
    except Exception:   # noqa: BLE001 - numpy builds differ in what they report
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "workers": workers,
            "numpy": np.__version__, "blas": blas}


def _default_workers() -> int:
    # one GPU's share of the host: at most 16 processes
    return max(1, min(os.cpu_count() or 1, 16))


def _unit_attention(u: int):
    """Oracle work of unit u of the workload in _UNITS: encode its K and V vectors
    (canonical fp32), pack them, fp64 attention for its query heads."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as o_att
    from oracle import codec
    W = _UNITS
    b, g = divmod(u, W["hkv"])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k32 = W["k"][b, g][None, None]
        v32 = W["v"][b, g][None, None]
        kc, kn, _ = codec.encode_mse(k32, W["s"], W["bk"])
        vc, vn, _ = codec.encode_mse(v32, W["s"], W["bv"])
        kp, vp = codec.pack(kc, W["kb"]), codec.pack(vc, W["vb"])
        t1 = time.perf_counter()
        q = W["q"][b, g * W["grp"]:(g + 1) * W["grp"]][None]
        o_att.attend_fused(q, kp, kn, vp, vn, [int(W["lens"][b])], W["kb"], W["vb"], W["ck"],
                           W["cv"], W["s"], 1 / np.sqrt(128))
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def _unit_prefill(u: int):
    """Oracle encode of unit u = (layer, KV head) of the prefill subset: K4 one d=256
    rotation per vector, V2 in 128-blocks, and the 8-bit grid in 128-blocks."""
    from threadpoolctl import threadpool_limits

    from oracle import codec
    W = _UNITS
    li, g = divmod(u, W["hkv"])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        k32, v32 = W["k"][li, g], W["v"][li, g]
        codec.encode_mse_whole(k32, W["s256"], W["bk256"])
        t1 = time.perf_counter()
        vc, _, _ = codec.encode_mse(v32, W["s256"], W["bv"])
        codec.pack(vc, 2)
        t2 = time.perf_counter()
        codec.encode_u8(k32, W["s256"])
        t3 = time.perf_counter()
    return t1 - t0, t2 - t1, t3 - t2


def _run_units(fn, n_units: int, workers: int):
    """Wall time of fn over all units: one process (workers == 1) or a fork pool."""
    t0 = time.perf_counter()
    if workers == 1:
        parts = [fn(u) for u in range(n_units)]
    else:
        import multiprocessing as mp
        with mp.get_context("fork").Pool(workers) as pool:
            parts = pool.map(fn, range(n_units), chunksize=1)
    return time.perf_counter() - t0, np.sum(np.array(parts), axis=0)


def _load_attention_units(w, seed: int, n_slices: int | None = None):
    import torch

    import workloads
    from oracle import codebook as o_cb
    from oracle import signs as o_signs
    if w.name == "tiny":
        k, v, q = workloads.tiny_inputs()
        k, v, q = k[None, None], v[None, None], q[None, None].astype(np.float64)
        lens = np.array([k.shape[2]])
    else:
        kt, vt = workloads.make_kv(w, "cpu")
        k = kt.to(torch.float32).numpy()
        v = vt.to(torch.float32).numpy()
        del kt, vt
        q = workloads.make_q(w, "cpu").to(torch.float32).numpy().astype(np.float64)
        lens = workloads.make_seq_lens(w)
    bk, ck = o_cb.codebook(w.k_bits)
    bv, cv = o_cb.codebook(w.v_bits)
    _UNITS.clear()
    _UNITS.update(k=k, v=v, q=q, lens=lens, s=o_signs.signs(seed, 128), bk=bk, ck=ck, bv=bv,
                  cv=cv, kb=w.k_bits, vb=w.v_bits, hkv=w.n_kv_heads,
                  grp=w.n_q_heads // w.n_kv_heads)
    n_units = k.shape[0] * k.shape[1]
    return n_units if n_slices is None else min(n_slices, n_units)


def _attention_record(w, n_units: int, workers: int, reps: int = 1) -> dict:
    """Oracle throughput over the first n_units slices: encode K and V of each slice
    and fp64 attention for its query heads; bytes as the GPU path counts them."""
    lens = _UNITS["lens"]
    hkv = _UNITS["hkv"]
    T = _UNITS["k"].shape[2]
    units_b = [u // hkv for u in range(n_units)]
    tok = int(sum(T for _ in units_b))
    att_tok = int(sum(int(lens[b]) for b in units_b))
    enc_b = enc_bytes(tok, 256, w.k_bits) + enc_bytes(tok, 256, w.v_bits)
    cbk, cbv = {2: 32, 3: 48, 4: 64}[w.k_bits], {2: 32, 3: 48, 4: 64}[w.v_bits]
    att_b = att_tok * (cbk + cbv + 4) + n_units * _UNITS["grp"] * 128 * (2 + 4)
    wall, parts = 0.0, np.zeros(2)
    for _ in range(reps):
        wl, pt = _run_units(_unit_attention, n_units, workers)
        wall += wl
        parts += pt
    wall /= reps
    parts /= reps
    return {"value": round((enc_b + att_b) / wall / 1e9, 4), "unit": "GB/s",
            "cores": min(workers, n_units),
            "seconds": round(wall, 3),
            "encode_vectors_per_cpu_s": round(2 * tok / float(parts[0]), 1),
            "cpu_s_encode": round(float(parts[0]), 3), "cpu_s_attention": round(float(parts[1]), 3),
            "units": n_units, "algorithmic_bytes": int(enc_b + att_b), "repetitions": reps}


def cpu_baseline(seed: int, workers: int) -> dict:
    """The oracle as it stands, on the step's workload (all 8 KV-head slices of the
    Llama-shaped layer: encode K and V, fp64 attention): one worker, then N worker
    processes over the slices."""
    import workloads
    w = workloads.WORKLOADS["llama_layer"]
    n = _load_attention_units(w, seed)
    one = _attention_record(w, n, 1, reps=3)
    many = _attention_record(w, n, workers, reps=5)
    rec = dict(many)
    rec.update({"kind": "oracle",
                "sample": f"the whole step workload ({n} (sequence, KV head) slices x "
                          f"{w.tokens} tokens): encode K and V (canonical fp32) + fp64 "
                          f"attention for {w.n_q_heads} query heads; numpy, "
                          f"{min(workers, n)} worker processes, one slice each (mean of 5 "
                          f"runs; single_worker: one process, mean of 3 runs)",
                "single_worker": one})
    rec.update(_cpu_info(workers))
    return rec


def cpu_baseline_full(seed: int, workers: int) -> dict:
    """The oracle on every workload: configs tiny, llama_layer, batched and
    long_context at full size, and the prefill encode on layers {0, 31}, all 8 KV
    heads, tokens [0, 8192); each with one worker and with N worker processes."""
    import torch

    import workloads
    from oracle import codebook as o_cb
    from oracle import signs as o_signs
    out = {"info": _cpu_info(workers)}
    for name in ("tiny", "llama_layer", "batched", "long_context"):
        w = workloads.WORKLOADS[name]
        t0 = time.perf_counter()
        n = _load_attention_units(w, seed)
        gen = time.perf_counter() - t0
        out[name] = {"1_worker": _attention_record(w, n, 1),
                     f"{workers}_workers": _attention_record(w, n, workers),
                     "input_generation_s": round(gen, 1)}
        print(f"# cpu oracle {name}: {out[name]}", file=sys.stderr, flush=True)
    w = workloads.WORKLOADS["prefill"]
    T = 8192
    kt, vt = workloads.make_kv(w, "cpu", tokens=T)
    k = kt[[0, w.batch - 1]].to(torch.float32).numpy()
    v = vt[[0, w.batch - 1]].to(torch.float32).numpy()
    del kt, vt
    bk256, _ = o_cb.codebook(4, 256)
    bv, _ = o_cb.codebook(2)
    _UNITS.clear()
    _UNITS.update(k=k, v=v, s256=o_signs.signs(seed, 256),
                  bk256=bk256, bv=bv, hkv=w.n_kv_heads)
    n = 2 * w.n_kv_heads
    nvec = n * T
    rec = {}
    for nw in (1, workers):
        wall, parts = _run_units(_unit_prefill, n, nw)
        rec[f"{nw}_worker" + ("s" if nw > 1 else "")] = {
            "seconds": round(wall, 3), "cores": nw,
            "vectors_per_s_all_three": round(3 * nvec / wall, 1),
            "cpu_s": {"k4_whole_d256": round(float(parts[0]), 3),
                      "v2_blocked": round(float(parts[1]), 3),
                      "k8_blocked": round(float(parts[2]), 3)},
            "vectors_per_s_k4_whole_d256_1core": round(nvec / float(parts[0]), 1)}
    out["prefill_subset"] = {"subset": f"layers 0 and {w.batch - 1}, {w.n_kv_heads} KV heads, "
                                       f"tokens [0, {T}), head_dim 256", **rec}
    return out


def _cpu_baseline_child(workers: int) -> dict:
    """Run the bounded CPU baseline in a child process (the GPU process never forks)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
           "--workers", str(workers)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    workers = args.workers or _default_workers()
    if args.cpu_baseline_only or args.cpu_baseline_full:
        import workloads
        seed = workloads.ROTATION_SEED
        res = cpu_baseline_full(seed, workers) if args.cpu_baseline_full else \
            cpu_baseline(seed, workers)
        print(json.dumps(res), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import kv_cache_vector_fa_amd as fa
    import workloads

    fa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.prefill_only:
        print(json.dumps({"prefill_encode_d256": prefill_whole(fa, workloads.ROTATION_SEED)}),
              flush=True)
        return
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
    C = max(R, args.cache_copies)
    caches = [fa.cache_buffers(B, Hkv, T, d, w.k_bits) + fa.cache_buffers(B, Hkv, T, d, w.v_bits)
              for _ in range(C)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = fa.attn_workspace(B, Hq, Hkv, T, d)
    scale = 1 / np.sqrt(d)
    # arguments marshalled once per buffer copy: a launch costs one ctypes call
    # step i: input copy i % R, cache copy i % C
    enc_kv = [fa.encode_kv_call(cbk, cbv, seed, ks[i % R], vs[i % R], *caches[i])
              for i in range(C)]
    attn = [fa.attn_decode_call(cbk, cbv, seed, q, *caches[i], lens, scale, out, ws)
            for i in range(C)]
    names = ("encode_kv", "attn_decode")
    calls = (enc_kv, attn)
    # the same encodes as two calls (fa_tq_encode of K, then of V), timed beside the step
    enc_k = [fa.encode_call(cbk, seed, ks[i % R], caches[i][0], caches[i][1]) for i in range(C)]
    enc_v = [fa.encode_call(cbv, seed, vs[i % R], caches[i][2], caches[i][3]) for i in range(C)]

    for i in range(args.warmup):
        for c in calls:
            c[i % C]()
    K = args.steps
    rounds = [(s0, min(K, s0 + ROUND)) for s0 in range(0, K, ROUND)]
    P = len(calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(P * len(rounds) + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r, (s0, s1) in enumerate(rounds):
        for j, c in enumerate(calls):
            ev[P * r + j].record()
            for i in range(s0, s1):
                c[i % C]()
    ev[-1].record()
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[-1]) / K
    kms = [sum(ev[P * r + j].elapsed_time(ev[P * r + j + 1]) for r in range(len(rounds))) / K
           for j in range(P)]

    nblk = B * Hkv * T * (d // 128)
    nbytes = (enc_bytes(nblk, 256, w.k_bits) + enc_bytes(nblk, 256, w.v_bits),
              attn_bytes(lens_np, Hkv, Hq, w.k_bits, w.v_bits))
    step_bytes = sum(nbytes)
    kern = {}
    for name, km, nb in zip(names, kms, nbytes):
        gbs = nb / (km * 1e-3) / 1e9
        rec = {"us": round(km * 1e3, 3), "algorithmic_bytes": nb, "gbps": round(gbs, 1),
               "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        if name.startswith("encode"):   # key and value vectors
            rec["vectors_per_s"] = round(2 * nblk / (d // 128) / (km * 1e-3), 1)
        kern[name] = rec
    dom = max(kern, key=lambda n: kern[n]["us"])
    kname = {"encode_kv": f"encode_pair_kernel<{w.k_bits}, {w.v_bits}, true, false, false>"}.get(
        dom, dom)
    traffic = traffic_for(kname)
    roof = {"kernel": kname, "bound": "hbm", "achieved": kern[dom]["gbps"],
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kern[dom]["frac_hbm_peak"],
            "traffic": None if traffic is None else round(traffic)}

    rec = {
        "metric": METRIC,
        "value": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; bf16 AR(1) rho 0.9 with lognormal channel scales)",
        "config": {"workload": w.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": Hkv,
                   "tokens": T, "head_dim": d, "k_bits": w.k_bits, "v_bits": w.v_bits,
                   "step": "encode K and V (one call) + decode attention", "copies": R,
                   "cache_copies": C},
        "step_algorithmic_bytes": step_bytes,
        "wall_s_timed": round(wall, 4),
        "host_us_per_step": round(t_host / K * 1e6, 1),
        "kernels": kern,
        "roofline": roof,
    }
    rec["encode_separate"] = encode_separate(enc_k, enc_v, K, C, nblk, w)
    sep = dict(zip(names, calls), encode_k=enc_k, encode_v=enc_v)
    rec["per_call"] = {n: per_call_distribution(c) for n, c in sep.items()}
    if not args.no_cold_hbm:
        rec["cold_hbm"] = {n: cold_hbm(c) for n, c in sep.items()}
    rec["attn_decode_graph"] = attention_graph(fa, cbk, cbv, seed, q, caches, lens, scale, out,
                                               ws, nbytes[1])
    rec["attn_decode_vector_alu"] = attention_graph(fa, cbk, cbv, seed, q, caches, lens, scale,
                                                    out, ws, nbytes[1], flags=fa.ATTN_VECTOR_ALU)
    if not args.no_append:
        rec["append_decode"] = append_decode(fa, w, cbk, cbv, seed, q, caches[0], out, ws, scale)
        rec["restore_bf16"] = restore_bf16(fa, w, cbk, seed, caches)
        rec["encode_k_variants"] = encode_variants(fa, w, cbk, seed, ks, caches)
        rec["attn_decode_dense_d128"] = dense_attention(fa, w, seed, k, v, q, lens, lens_np,
                                                        scale)
        rec["prefill_encode_d256"] = prefill_whole(fa, seed)
        rec["attention_other_workloads"] = other_attention(fa, seed)
        rec["attention_large_groups"] = large_groups(fa, seed)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = _cpu_baseline_child(workers)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Host-side pins of the benchmark's measurement arithmetic (no device): the
algorithmic byte counts of the llama-layer step, the one-GPU contract of the
command line, and the rule that HBM traffic is reported only while the kernel
source still has the hash the counters were taken with."""

import json
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_encode_bytes_of_the_llama_layer():
    """262144 blocks of bf16 input (256 B) with 4-bit codes (64 B) and an fp16 norm:
    84,410,368 B for K; 2-bit values 76,021,760 B."""
    assert bench.enc_bytes(262144, 256, 4) == 84_410_368
    assert bench.enc_bytes(262144, 256, 2) == 76_021_760
    assert bench.enc_bytes(1, 512, 8) == 512 + 128 + 2


def test_attention_bytes_of_the_llama_layer():
    """32768 tokens x 8 KV heads x (64 + 32 + 2 + 2) B of packed cache, plus the bf16
    query and the fp32 output of 32 heads."""
    assert bench.attn_bytes(np.array([32768]), 8, 32, 4, 2) == 26_214_400 + 32 * 128 * 6
    # ragged lengths count only the valid tokens
    assert bench.attn_bytes(np.array([10, 0, 5]), 2, 4, 3, 3) == 15 * 2 * 100 + 3 * 4 * 128 * 6


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_traffic_only_while_the_source_matches(monkeypatch):
    """The committed counters name the encoder's source hash: with the hash as it is
    the traffic is a positive byte count near the algorithmic bytes; with any other
    hash it is withheld."""
    name = "encode_kernel<4, true, false, false, false>"
    t = bench.traffic_for(name)
    if t is not None:   # counters taken with the current source
        assert 0.9 * 84_410_368 < t < 1.2 * 84_410_368
    monkeypatch.setattr(bench, "source_hash", lambda _: "0" * 16)
    assert bench.traffic_for(name) is None
    assert bench.traffic_for("no_such_kernel") is None

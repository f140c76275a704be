"""Shared helpers for the GPU parity tests (comparison rules of the contract).

Rules: packed bytes and fp16 norm bits exact; quantization codes exact except at
most 1e-5 of them may be adjacent-level flips; decoded vectors relative L2 error
<= 1e-5 against the fp64 oracle; attention max abs error <= 2e-3 against the fp64
oracle on the same packed cache.
"""

import sys

import numpy as np

from oracle import codec

FLIP_BUDGET = 1e-5
DECODE_REL_L2 = 1e-5
ATTN_MAX_ABS = 2e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_to_f32(t):
    """torch bf16 tensor (any device) -> numpy float32 (exact widening)."""
    import torch
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16).astype(np.uint32).__lshift__(16).view(np.float32)


def compare_codes(gpu_packed: np.ndarray, oracle_codes: np.ndarray, bits: int, where=""):
    """gpu_packed [N, cb] bytes, oracle_codes [N, 128] ints.  Returns flip count."""
    n = gpu_packed.shape[0]
    g = codec.unpack(gpu_packed.reshape(n, 1, -1), bits).astype(np.int64)
    o = oracle_codes.reshape(n, 128).astype(np.int64)
    diff = g - o
    assert np.all(np.abs(diff) <= 1), f"{where}: non-adjacent code mismatch"
    flips = int(np.count_nonzero(diff))
    assert flips <= FLIP_BUDGET * diff.size, f"{where}: {flips} flips in {diff.size} codes"
    if flips == 0:
        np.testing.assert_array_equal(gpu_packed.reshape(n, -1),
                                      codec.pack(oracle_codes.reshape(n, 128), bits).reshape(n, -1))
    return flips


def compare_norms(gpu_norms_i16: np.ndarray, oracle_norms_f16: np.ndarray, where=""):
    g = np.asarray(gpu_norms_i16).view(np.uint16).reshape(-1)
    o = np.asarray(oracle_norms_f16, np.float16).view(np.uint16).reshape(-1)
    bad = np.count_nonzero(g != o)
    assert bad == 0, f"{where}: {bad} of {g.size} fp16 norms differ"

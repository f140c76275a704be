"""The random +/-1 sign diagonal D of the rotation (oracle; test infrastructure).

[Spec] "Step 1: Random Orthogonal Rotation": D is a diagonal of random +1/-1 signs,
one head_dim-element array generated once from a seed and reused for all tokens,
heads and layers ([Spec] "API", Lifecycle: the seed determines the rotation).

The pages do not name the generator.  Reading: SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014), seeded with the
64-bit seed; the i-th draw gives s_i = -1 when its top bit is set, else +1, for
i = 0 .. head_dim - 1.  This is a convention of this implementation; the pages pin
no particular sequence (parity of the sequence itself is unpinned by the pages).
"""

from __future__ import annotations

import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def splitmix64(seed: int, n: int) -> list[int]:
    """First n outputs of SplitMix64 started at state ``seed`` (Python ints, exact)."""
    state = seed & _MASK
    out = []
    for _ in range(n):
        state = (state + _GAMMA) & _MASK
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK
        out.append(z ^ (z >> 31))
    return out


def signs(seed: int, head_dim: int) -> np.ndarray:
    """int8 array of +1/-1, s_i = -1 iff bit 63 of the i-th SplitMix64 draw is set."""
    draws = splitmix64(seed, head_dim)
    return np.array([-1 if (z >> 63) else 1 for z in draws], dtype=np.int8)


def signs2(seed: int, head_dim: int) -> np.ndarray:
    """The second fixed +/-1 vector of [turboq] "Encode pipeline" step 2 (applied
    after the normalized butterflies).  Reading: the next head_dim draws of the same
    SplitMix64 stream, i.e. draws head_dim .. 2 head_dim - 1, sign from the top bit."""
    draws = splitmix64(seed, 2 * head_dim)[head_dim:]
    return np.array([-1 if (z >> 63) else 1 for z in draws], dtype=np.int8)

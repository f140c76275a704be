"""CPU oracle for the TurboQuant MSE KV-cache path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP path is
checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``kv_cache_vector_fa_amd``) never imports, links or calls anything here, and this
package imports nothing from the product path: the two share no code.

Pages cited (by title and section):

* [Spec]    "TurboQuant KV Cache Compression -- Spec" (Foundry attention module).
* [turboq]  "TurboQuant KV Cache (turboq2 / turboq3 / turboq4)" (llama.cpp fork docs).
* [Rotor]   "RotorQuant KV Cache Compression" (only the MSE score term is used).

Modules:

* ``codebook``  -- Lloyd-Max levels for the rotated-coordinate density.
* ``signs``     -- the random +/-1 diagonal drawn from the seed.
* ``rotation``  -- Walsh-Hadamard transform (fp64 math mode and canonical fp32 stages).
* ``codec``     -- norm, bucketize, bit-pack, decode, and the 8-bit variant.
* ``attention`` -- fused rotated-domain decode attention and its brute-force check.
* ``dense``     -- the dense random orthogonal rotation for head_dims that are not a
                 power of two, and its encode / decode.

Arithmetic modes: fp64 "math" mode for invariants and the attention reference, and
"canonical fp32" mode (numpy float32, IEEE round-to-nearest-even, no fused
multiply-add, a fixed operation order) which defines the exact code and norm bits.
"""

from . import codebook, signs, rotation, codec, attention, dense  # noqa: F401

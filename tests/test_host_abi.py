"""Host-side checks of the C ABI (CPU only: no device compute is called here).

The library must load, export every function ``include/fa_tq.h`` declares, build
the same codebooks and signs as the oracle (two independent implementations), and
reject bad arguments before touching the device.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_fa_amd as fa
from oracle import codebook as o_cb
from oracle import signs as o_signs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return fa.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "fa_tq.h")).read()
    return sorted(set(re.findall(r"\b(fa_tq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert len(declared) >= 8
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(fa.exported_symbols()) == declared


@pytest.mark.parametrize("dim", [64, 96, 128, 160, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_matches_oracle_exactly(lib, dim, bits):
    """C++ (incomplete-beta quadrature) and oracle (Gauss-Legendre) tables agree
    bit for bit in fp32."""
    cb = fa.codebook_init(dim, bits)
    b, c = cb.arrays()
    ob, oc = o_cb.codebook(bits, dim)
    assert cb.dim == dim and cb.bits == bits and cb.levels == 1 << bits
    np.testing.assert_array_equal(b, ob)
    np.testing.assert_array_equal(c, oc)


def test_codebook_8bit_is_grid(lib):
    cb = fa.codebook_init(128, 8)
    assert cb.levels == 256 and all(x == 0 for x in cb.boundaries) and all(x == 0 for x in cb.centroids)


@pytest.mark.parametrize("seed", [0, 42, 2 ** 63 + 5])
def test_signs_match_oracle(lib, seed):
    np.testing.assert_array_equal(fa.signs(seed, 256), o_signs.signs(seed, 256))


def test_code_bytes_and_workspace(lib):
    assert [fa.code_bytes(b) for b in (2, 3, 4, 8)] == [32, 48, 64, 128]
    assert fa.code_bytes(5) == -1
    ws = fa.attn_workspace_bytes(1, 32, 8, 32768)
    assert ws > 0 and ws % 4 == 0
    assert fa.attn_workspace_bytes(1, 30, 8, 100) == 0      # 30 % 8 != 0
    assert fa.attn_workspace_bytes(1, 32, 8, 100, 256) == 0  # head_dim 256 unsupported


def _err(fn, *args):
    with pytest.raises(fa.FaTqError) as ei:
        fn(*args)
    return ei.value.status


def test_codebook_init_rejects_bad_arguments(lib):
    assert _err(fa.codebook_init, 128, 5) == fa.FA_TQ_EINVAL
    assert _err(fa.codebook_init, 2, 4) == fa.FA_TQ_EINVAL
    assert _err(fa.codebook_init, 1024, 4) == fa.FA_TQ_EINVAL
    assert lib.fa_tq_codebook_init(128, 4, None) == fa.FA_TQ_EINVAL


def _encode_raw(lib, cb, head_dim, x_ptr, dtype, layout, B, H, T, t_max, codes, norms):
    return lib.fa_tq_encode(ctypes.byref(cb), 42, head_dim, ctypes.c_void_p(x_ptr), dtype,
                            layout, B, H, T, None, t_max, ctypes.c_void_p(codes),
                            ctypes.c_void_p(norms), None)


def test_encode_validation_before_launch(lib):
    """Every rejected call returns before any HIP call (no device is needed)."""
    cb = fa.codebook_init(128, 4)
    lay = fa.Layout(8 * 128, 8 * 128, 128)
    A = 1 << 20  # any 16-byte aligned non-null value; never dereferenced on rejection
    assert _encode_raw(lib, cb, 100, A, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    assert _encode_raw(lib, cb, 128, A + 4, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    assert _encode_raw(lib, cb, 128, 0, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    bad = fa.Layout(8 * 128, 8 * 128, 100)
    assert _encode_raw(lib, cb, 128, A, 1, bad, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    assert _encode_raw(lib, cb, 128, A, 1, lay, 1, 1, 5, 4, A, A) == fa.FA_TQ_EINVAL
    assert _encode_raw(lib, cb, 128, A, 7, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EUNSUPPORTED
    assert _encode_raw(lib, cb, 128, A, 1, lay, -1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    # zero-sized work is an OK no-op (no launch)
    assert _encode_raw(lib, cb, 128, 0, 1, lay, 0, 1, 1, 1, 0, 0) == fa.FA_TQ_OK
    # a tampered codebook is rejected
    bad_cb = fa.codebook_init(128, 4)
    bad_cb.boundaries[3] = bad_cb.boundaries[2]
    assert _encode_raw(lib, bad_cb, 128, A, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    bad_cb = fa.codebook_init(128, 4)
    bad_cb.dim = 256
    assert _encode_raw(lib, bad_cb, 128, A, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    bad_cb = fa.codebook_init(128, 4)
    bad_cb.levels = 8
    assert _encode_raw(lib, bad_cb, 128, A, 1, lay, 1, 1, 1, 1, A, A) == fa.FA_TQ_EINVAL
    assert "levels" in lib.fa_tq_last_error().decode()


def _encode_kv_raw(lib, ck, cv, flags=0, k=1 << 20, v=1 << 20, B=1, T=1, t_max=1,
                   kcodes=1 << 20, vnorms=1 << 20, head_dim=128):
    P = ctypes.c_void_p
    lay = fa.Layout(256, 256, 256)
    return lib.fa_tq_encode_kv(ctypes.byref(ck), ctypes.byref(cv), 42, flags, head_dim, P(k),
                               P(v), fa.FA_TQ_BF16, lay, lay, B, 1, T, None, t_max, P(kcodes),
                               P(1 << 20), P(1 << 20), P(vnorms), None)


def test_encode_kv_validation_before_launch(lib):
    """fa_tq_encode_kv checks both halves before anything is launched (no device is
    needed): a bad value codebook, a misaligned V input, an odd V norms pointer, a NULL
    K cache, too many tokens, unknown flags; empty work is an OK no-op."""
    c4, c2 = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    A = 1 << 20
    bad = fa.codebook_init(128, 2)
    bad.boundaries[1] = bad.boundaries[0]
    assert _encode_kv_raw(lib, c4, bad) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, v=A + 4) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, vnorms=A + 1) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, kcodes=0) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, T=5, t_max=4) == fa.FA_TQ_EINVAL
    assert "fa_tq_encode_kv" in lib.fa_tq_last_error().decode()
    assert _encode_kv_raw(lib, c4, c2, flags=8) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, head_dim=100) == fa.FA_TQ_EINVAL
    assert _encode_kv_raw(lib, c4, c2, B=0) == fa.FA_TQ_OK
    assert _encode_kv_raw(lib, c4, c2, T=0) == fa.FA_TQ_OK


def test_encode_kv_binding_rejects_mismatched_inputs(lib):
    """The binding refuses V of another shape or dtype than K, and caches of the wrong
    shape (CPU tensors: the checks run before the device check)."""
    import torch
    cbk, cbv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    k = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16)
    kc = fa.cache_buffers(1, 2, 8, 128, 4, "cpu")
    vc = fa.cache_buffers(1, 2, 8, 128, 2, "cpu")
    with pytest.raises(ValueError):
        fa.encode_kv_call(cbk, cbv, 42, k, torch.zeros((1, 2, 9, 128), dtype=torch.bfloat16),
                          *kc, *vc)
    with pytest.raises(ValueError):
        fa.encode_kv_call(cbk, cbv, 42, k, k.float(), *kc, *vc)
    with pytest.raises(ValueError):   # the V cache sized for 4-bit codes
        fa.encode_kv_call(cbk, cbv, 42, k, k.clone(), *kc, *kc)


def _attn_raw(lib, ck, cv, hd, B, Hq, Hkv, T, ws_bytes, ptr=1 << 20):
    P = ctypes.c_void_p(ptr)
    return lib.fa_tq_attn_decode(ctypes.byref(ck), ctypes.byref(cv), 42, hd, P, 1, P, P, P, P,
                                 P, B, Hq, Hkv, T, 0.0884, P, P, ws_bytes, None)


def test_attn_validation_before_launch(lib):
    ck, cv = fa.codebook_init(128, 4), fa.codebook_init(128, 2)
    big = 1 << 40
    assert _attn_raw(lib, ck, cv, 128, 1, 30, 8, 64, big) == fa.FA_TQ_EINVAL
    assert _attn_raw(lib, ck, cv, 256, 1, 32, 8, 64, big) == fa.FA_TQ_EUNSUPPORTED
    # group size 32: the matrix-core kernels take it (split over workgroups), the
    # vector-ALU kernels do not
    P = ctypes.c_void_p(1 << 20)
    assert lib.fa_tq_attn_decode_ex(ctypes.byref(ck), ctypes.byref(cv), 42, fa.ATTN_VECTOR_ALU,
                                    128, P, 1, P, P, P, P, P, 1, 64, 2, 64, 0.0884, P, P, big,
                                    None) == fa.FA_TQ_EUNSUPPORTED
    assert "vector-ALU" in lib.fa_tq_last_error().decode()
    assert fa.attn_workspace_bytes(1, 64, 2, 64) > 0
    assert fa.attn_workspace_bytes(2, 64, 1, 1000) >= 2 * 64 * 130 * 4
    assert _attn_raw(lib, ck, cv, 128, 1, 32, 8, 64, 16) == fa.FA_TQ_EINVAL   # workspace
    assert _attn_raw(lib, ck, cv, 128, 1, 32, 8, 64, big, ptr=(1 << 20) + 8) == fa.FA_TQ_EINVAL
    c8 = fa.codebook_init(128, 8)
    assert _attn_raw(lib, c8, cv, 128, 1, 32, 8, 64, big) == fa.FA_TQ_EUNSUPPORTED
    assert _attn_raw(lib, ck, cv, 128, 0, 32, 8, 64, big) == fa.FA_TQ_OK


def _encode_ex_raw(lib, cb, flags, B=1, ptr=1 << 20, head_dim=128):
    P = ctypes.c_void_p(ptr)
    lay = fa.Layout(256, 256, 256)
    return lib.fa_tq_encode_ex(ctypes.byref(cb), 42, flags, head_dim, P, fa.FA_TQ_BF16, lay, B,
                               1, 1, None, 1, P, P, None)


def test_variant_flags_validated_before_launch(lib):
    """Unknown flags, the corrected norm with the 8-bit grid, and the two-sign
    rotation with a codebook that is not mirror symmetric are rejected (no device
    needed); valid flags with an empty batch are an OK no-op."""
    c4, c8 = fa.codebook_init(128, 4), fa.codebook_init(128, 8)
    assert _encode_ex_raw(lib, c4, 8) == fa.FA_TQ_EINVAL
    # whole-vector mode: no other flag, head_dim 128/256, codebook of that dimension
    assert _encode_ex_raw(lib, c4, fa.WHOLE_VECTOR | fa.TWO_SIGNS) == fa.FA_TQ_EUNSUPPORTED
    assert _encode_ex_raw(lib, c8, fa.WHOLE_VECTOR) == fa.FA_TQ_EUNSUPPORTED
    assert _encode_ex_raw(lib, c8, fa.NORM_CORRECT) == fa.FA_TQ_EUNSUPPORTED
    b = np.array(c4.boundaries[:15], np.float32)
    c = np.array(c4.centroids[:16], np.float32)
    c[3] *= 1.01                                    # still ascending, no longer symmetric
    skew = fa.codebook_from_arrays(4, b, c)
    assert _encode_ex_raw(lib, skew, fa.TWO_SIGNS) == fa.FA_TQ_EUNSUPPORTED
    assert "mirror" in lib.fa_tq_last_error().decode()
    assert _encode_ex_raw(lib, c4, fa.TWO_SIGNS | fa.NORM_CORRECT, B=0) == fa.FA_TQ_OK
    P = ctypes.c_void_p(1 << 20)
    # decode and attention accept only the rotation flag
    lay = fa.Layout(0, 128, 128)
    assert lib.fa_tq_decode_kv(ctypes.byref(c4), 42, fa.NORM_CORRECT, 128, P, P, 1, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay, None) == fa.FA_TQ_EINVAL
    c2 = fa.codebook_init(128, 2)
    assert lib.fa_tq_attn_decode_ex(ctypes.byref(c4), ctypes.byref(c2), 42, fa.WHOLE_VECTOR, 128,
                                    P, 1, P, P, P, P, P, 1, 32, 8, 64, 0.088, P, P, 1 << 40,
                                    None) == fa.FA_TQ_EUNSUPPORTED
    c256 = fa.codebook_init(256, 4)
    lay256 = fa.Layout(0, 256, 256)
    assert lib.fa_tq_decode_kv(ctypes.byref(c4), 42, fa.WHOLE_VECTOR, 256, P, P, 1, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay256, None) == fa.FA_TQ_EINVAL   # dim 128 table
    assert lib.fa_tq_decode_kv(ctypes.byref(c256), 42, fa.WHOLE_VECTOR, 512, P, P, 1, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay256, None) == fa.FA_TQ_EUNSUPPORTED
    assert lib.fa_tq_attn_decode_ex(ctypes.byref(c4), ctypes.byref(c2), 42, fa.NORM_CORRECT, 128,
                                    P, 1, P, P, P, P, P, 1, 32, 8, 64, 0.088, P, P, 1 << 40,
                                    None) == fa.FA_TQ_EINVAL


def test_whole_vector_head_dims_validated(lib):
    """Whole-vector mode: head_dim in (64, 256] and a multiple of 8, padded to 128 or
    256 with the codebook of that length; other head_dims, or a padded head_dim
    without the flag, are rejected before any launch (batch 0: an OK no-op)."""
    W = fa.WHOLE_VECTOR
    c128, c256, c192 = (fa.codebook_init(n, 4) for n in (128, 256, 192))
    for d, cb in ((72, c128), (96, c128), (120, c128), (136, c256), (192, c256), (248, c256)):
        assert _encode_ex_raw(lib, cb, W, B=0, head_dim=d) == fa.FA_TQ_OK, d
    assert _encode_ex_raw(lib, c192, W, B=0, head_dim=192) == fa.FA_TQ_EINVAL   # dim 192 table
    assert "256" in lib.fa_tq_last_error().decode()
    assert _encode_ex_raw(lib, c256, W, B=0, head_dim=96) == fa.FA_TQ_EINVAL    # 96 pads to 128
    for d in (64, 100, 260, 384):
        assert _encode_ex_raw(lib, c256, W, B=0, head_dim=d) == fa.FA_TQ_EUNSUPPORTED, d
    assert _encode_ex_raw(lib, c128, 0, B=0, head_dim=192) == fa.FA_TQ_EINVAL
    P = ctypes.c_void_p(1 << 20)
    lay = fa.Layout(0, 256, 256)
    assert lib.fa_tq_decode_kv(ctypes.byref(c256), 42, W, 200, P, P, 0, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay, None) == fa.FA_TQ_OK
    assert lib.fa_tq_decode_kv(ctypes.byref(c128), 42, W, 200, P, P, 0, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay, None) == fa.FA_TQ_EINVAL
    assert lib.fa_tq_decode_kv(ctypes.byref(c256), 42, 0, 200, P, P, 0, 1, 1, 1, P,
                               fa.FA_TQ_BF16, lay, None) == fa.FA_TQ_EINVAL


def test_padded_cache_shapes_in_the_binding(lib):
    """cache_buffers sizes a padded whole-vector cache by the transform length, and
    decode_kv refuses a cache whose block count does not fit head_dim (no device)."""
    import torch
    codes, norms = fa.cache_buffers(2, 3, 5, 192, 4, device="cpu", flags=fa.WHOLE_VECTOR)
    assert tuple(codes.shape) == (2, 3, 5, 2, 64) and tuple(norms.shape) == (2, 3, 5, 1)
    codes, norms = fa.cache_buffers(2, 3, 5, 96, 2, device="cpu", flags=fa.WHOLE_VECTOR)
    assert tuple(codes.shape) == (2, 3, 5, 1, 32) and tuple(norms.shape) == (2, 3, 5, 1)
    cb = fa.codebook_init(128, 2)
    with pytest.raises(ValueError):
        fa.decode_kv(cb, 42, codes, norms, flags=fa.WHOLE_VECTOR, head_dim=192)
    with pytest.raises(ValueError):
        fa.decode_kv(cb, 42, codes, norms, head_dim=96)   # blocked mode: 96 is no block count
    out = torch.empty((2, 3, 5, 200), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.decode_kv_call(cb, 42, codes, norms, out, flags=fa.WHOLE_VECTOR)


def test_decode_kv_rejects_an_output_row_of_2_gib(lib):
    """fa_tq_decode_kv addresses one (batch, head) row of output with 32-bit byte
    offsets: an output whose token stride makes one row span 2 GiB or more is
    rejected before any launch (no device needed)."""
    cb = fa.codebook_init(128, 4)
    P = ctypes.c_void_p(1 << 20)
    big = fa.Layout(0, 128, 1 << 29)   # 3 tokens of bf16 at 1 GiB apart
    assert lib.fa_tq_decode_kv(ctypes.byref(cb), 42, 0, 128, P, P, 1, 1, 3, 3, P,
                               fa.FA_TQ_BF16, big, None) == fa.FA_TQ_EUNSUPPORTED
    assert "2 GiB" in lib.fa_tq_last_error().decode()


def _attn_args(B=2, Hq=8, Hkv=2, T=64, kb=4, vb=2):
    """CPU tensors with the shapes attn_decode_call expects (no device is touched:
    every check runs before the library call)."""
    import torch
    t = dict(
        q=torch.zeros((B, Hq, 128), dtype=torch.bfloat16),
        k_codes=torch.zeros((B, Hkv, T, 1, fa.code_bytes(kb)), dtype=torch.uint8),
        k_norms=torch.zeros((B, Hkv, T, 1), dtype=torch.int16),
        v_codes=torch.zeros((B, Hkv, T, 1, fa.code_bytes(vb)), dtype=torch.uint8),
        v_norms=torch.zeros((B, Hkv, T, 1), dtype=torch.int16),
        seq_lens=torch.full((B,), T, dtype=torch.int32),
        out=torch.zeros((B, Hq, 128), dtype=torch.float32),
        workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    return t


def _call_attn(t, kb=4, vb=2):
    cbk, cbv = fa.codebook_init(128, kb), fa.codebook_init(128, vb)
    return fa.attn_decode_call(cbk, cbv, 42, t["q"], t["k_codes"], t["k_norms"], t["v_codes"],
                               t["v_norms"], t["seq_lens"], 0.1, t["out"], t["workspace"])


@pytest.mark.parametrize("case", ["int64_lens", "short_v_cache", "v_heads", "q_strided",
                                  "out_dtype", "k_norms_f32", "cpu_tensors"])
def test_attn_binding_rejects_bad_tensors(lib, case):
    """The binding checks dtype, shape and contiguity of every tensor before any
    launch (an int64 length array would be read as int32 pairs; a smaller value
    cache would be addressed with the key cache's sizes)."""
    import torch
    t = _attn_args()
    if case == "int64_lens":
        t["seq_lens"] = t["seq_lens"].to(torch.int64)
    elif case == "short_v_cache":
        t["v_codes"], t["v_norms"] = t["v_codes"][:, :, :32], t["v_norms"][:, :, :32]
    elif case == "v_heads":
        t["v_codes"], t["v_norms"] = t["v_codes"][:, :1].contiguous(), t["v_norms"][:, :1].contiguous()
    elif case == "q_strided":
        t["q"] = torch.zeros((2, 16, 128), dtype=torch.bfloat16)[:, ::2]
    elif case == "out_dtype":
        t["out"] = t["out"].to(torch.bfloat16)
    elif case == "k_norms_f32":
        t["k_norms"] = t["k_norms"].to(torch.float32)
    with pytest.raises(ValueError):
        _call_attn(t)


def test_encode_and_decode_binding_reject_bad_buffers(lib):
    import torch
    cb = fa.codebook_init(128, 4)
    x = torch.zeros((1, 2, 16, 128), dtype=torch.bfloat16)
    codes = torch.zeros((1, 2, 16, 1, 64), dtype=torch.uint8)
    norms = torch.zeros((1, 2, 16, 1), dtype=torch.int16)
    with pytest.raises(ValueError):   # codes sized for 2-bit rows
        fa.encode_call(cb, 42, x, codes[..., :32].contiguous(), norms)
    with pytest.raises(ValueError):   # fewer cache slots than tokens x t_max claims
        fa.encode_call(cb, 42, x, codes, norms, t_max=32)
    with pytest.raises(ValueError):   # t0 of the wrong dtype
        fa.encode_call(cb, 42, x, codes, norms, t0=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError):   # CPU tensors never reach the library
        fa.encode_call(cb, 42, x, codes, norms)
    with pytest.raises(ValueError):   # norms for fewer vectors than codes
        fa.decode(cb, 42, codes, norms[:, :, :8].contiguous(), 128)
    with pytest.raises(ValueError):   # an output of the wrong dtype
        fa.decode(cb, 42, codes, norms, 128, out=torch.zeros((1, 2, 16, 128), dtype=torch.bfloat16))


def test_dense_attention_rejections_before_launch(lib):
    """fa_tq_attn_decode_dense refuses before any launch (fake device pointers are never
    dereferenced)."""
    fake = ctypes.c_void_p(1 << 20)
    B, Hq, Hkv, T = 2, 8, 2, 64
    need = lib.fa_tq_attn_dense_workspace_bytes(B, Hq, Hkv, T)
    assert need >= 2 * B * Hq * 128 * 4 + fa.attn_workspace_bytes(B, Hq, Hkv, T)
    assert lib.fa_tq_attn_dense_workspace_bytes(B, 7, 2, T) == 0      # Hq % Hkv != 0

    def call(cbk, cbv, d, flags=0, ws_bytes=need, hq=Hq, rot=fake):
        return lib.fa_tq_attn_decode_dense(ctypes.byref(cbk), ctypes.byref(cbv), rot, d, flags,
                                           fake, fa.FA_TQ_BF16, fake, fake, fake, fake, fake, B,
                                           hq, Hkv, T, 0.1, fake, fake, ws_bytes, None)
    c96, c96v = fa.codebook_init(96, 4), fa.codebook_init(96, 2)
    c160 = fa.codebook_init(160, 4)
    assert call(c160, c160, 160) == fa.FA_TQ_EUNSUPPORTED           # more than one block
    assert call(fa.codebook_init(128, 4), c96v, 96) == fa.FA_TQ_EINVAL   # codebook dim
    assert call(c96, c96v, 96, flags=fa.TWO_SIGNS) == fa.FA_TQ_EINVAL
    assert call(c96, c96v, 96, ws_bytes=need - 256) == fa.FA_TQ_EINVAL
    assert call(c96, c96v, 96, hq=7) == fa.FA_TQ_EINVAL
    assert call(c96, fa.codebook_init(96, 8), 96) == fa.FA_TQ_EUNSUPPORTED   # 8-bit grid
    # the query kernel stages R with 16-byte loads: a 4-byte aligned R is refused
    assert call(c96, c96v, 96, rot=ctypes.c_void_p((1 << 20) + 4)) == fa.FA_TQ_EINVAL


def test_dense_binding_rejects_bad_buffers(lib):
    """The dense-rotation binding checks every tensor before the library sees it (CPU
    tensors: the checks run before the device check)."""
    import torch
    d = 96
    cb = fa.codebook_init(d, 4)
    x = torch.zeros((2, 2, 16, d), dtype=torch.bfloat16)
    rot = torch.zeros((d, d), dtype=torch.float32)
    codes = torch.zeros((2, 2, 16, 1, 64), dtype=torch.uint8)
    norms = torch.zeros((2, 2, 16), dtype=torch.int16)
    with pytest.raises(ValueError):   # t0 not contiguous (every other int32 of a longer row)
        fa.encode_dense(cb, rot, x, codes=codes, norms=norms,
                        t0=torch.zeros(4, dtype=torch.int32)[::2])
    with pytest.raises(ValueError):   # a rotation of another size
        fa.encode_dense(cb, torch.zeros((d + 1, d + 1)), x, codes=codes, norms=norms)
    with pytest.raises(ValueError):   # codes of 2-bit rows for a 4-bit codebook
        fa.encode_dense(cb, rot, x, codes=codes[..., :32].contiguous(), norms=norms)
    with pytest.raises(ValueError):   # norms as float
        fa.decode_dense(cb, rot, codes, norms.float(), d)
    with pytest.raises(ValueError):   # codes for a wider head_dim
        fa.decode_dense(cb, rot, torch.zeros((2, 2, 16, 2, 64), dtype=torch.uint8), norms, d)
    with pytest.raises(ValueError):   # CPU tensors never reach the library
        fa.encode_dense(cb, rot, x, codes=codes, norms=norms)


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """Partials larger than the scratch array are refused before any device call
    (the pointers below are never dereferenced)."""
    B, Hq, Hkv, T = 512, 32, 8, 128
    assert fa.attn_workspace_bytes(B, Hq, Hkv, T) > fa.NOALLOC_SCRATCH_BYTES
    cb = fa.codebook_init(128, 4)
    fake = ctypes.c_void_p(1 << 20)
    st = lib.fa_tq_attn_decode_noalloc(ctypes.byref(cb), ctypes.byref(cb), 42, 0, 128, fake,
                                       fa.FA_TQ_BF16, fake, fake, fake, fake, fake, B, Hq, Hkv,
                                       T, 0.1, fake, None)
    assert st == fa.FA_TQ_EUNSUPPORTED
    assert "scratch" in lib.fa_tq_last_error().decode()


@pytest.mark.parametrize("dim", [24, 96, 160, 192, 250])
def test_dense_rotation_matches_oracle(lib, dim):
    """fa_tq_rotation_dense (C++ Householder) and the oracle (numpy QR) give the same
    fp32 matrix: two independent implementations of the sign-fixed QR factor."""
    from oracle import dense
    out = fa.rotation_dense(42, dim)
    ref = dense.rotation_f32(42, dim)
    assert np.max(np.abs(out.astype(np.float64) - ref.astype(np.float64))) <= 2 ** -23
    assert np.count_nonzero(out != ref) <= dim * dim // 1000


def test_dense_rejections_before_launch(lib):
    ctypes_cb = fa.codebook_init(96, 4)
    lay = fa.Layout(0, 0, 96)
    x = ctypes.c_void_p(256)
    rot = ctypes.c_void_p(4096)
    codes = ctypes.c_void_p(4096)
    norms = ctypes.c_void_p(4096)
    # head_dim past the dense limit
    cb300 = fa.codebook_init(300, 4)
    assert lib.fa_tq_encode_dense(ctypes.byref(cb300), rot, 300, x, fa.FA_TQ_BF16, lay, 1, 1, 1,
                                  None, 1, codes, norms, None) == fa.FA_TQ_EUNSUPPORTED
    # codebook built for another dim
    cb128 = fa.codebook_init(128, 4)
    assert lib.fa_tq_encode_dense(ctypes.byref(cb128), rot, 96, x, fa.FA_TQ_BF16, lay, 1, 1, 1,
                                  None, 1, codes, norms, None) == fa.FA_TQ_EINVAL
    # no rotation
    assert lib.fa_tq_encode_dense(ctypes.byref(ctypes_cb), None, 96, x, fa.FA_TQ_BF16, lay, 1, 1,
                                  1, None, 1, codes, norms, None) == fa.FA_TQ_EINVAL
    # the 8-bit grid has no dense form
    cb8 = fa.codebook_init(96, 8)
    assert lib.fa_tq_decode_dense(ctypes.byref(cb8), rot, 96, codes, norms, 1, 1, 1, 1,
                                  ctypes.c_void_p(4096), fa.FA_TQ_F32, lay, None) != fa.FA_TQ_OK
    # n_tokens > t_max on decode
    assert lib.fa_tq_decode_dense(ctypes.byref(ctypes_cb), rot, 96, codes, norms, 1, 1, 5, 4,
                                  ctypes.c_void_p(4096), fa.FA_TQ_F32, lay, None) == fa.FA_TQ_EINVAL
    assert lib.fa_tq_rotation_dense(42, 1, ctypes.c_void_p(4096)) == fa.FA_TQ_EINVAL
    # two boundaries in one cell of the encoder's 1024-cell grid over [-1, 1] (0 and
    # 0.001: distinct cells of the blocked encoder's table, one cell of the grid)
    close = fa.codebook_init(96, 4)
    assert close.boundaries[7] == 0.0
    close.boundaries[8] = 0.001
    assert lib.fa_tq_encode_dense(ctypes.byref(close), rot, 96, x, fa.FA_TQ_BF16, lay, 1, 1, 1,
                                  None, 1, codes, norms, None) == fa.FA_TQ_EUNSUPPORTED
    # 2^31 vectors in one call
    assert lib.fa_tq_encode_dense(ctypes.byref(ctypes_cb), rot, 96, x, fa.FA_TQ_BF16, lay,
                                  1 << 16, 1 << 8, 1 << 7, None, 1 << 7, codes, norms,
                                  None) == fa.FA_TQ_EUNSUPPORTED
    assert lib.fa_tq_decode_dense(ctypes.byref(ctypes_cb), rot, 96, codes, norms, 1 << 16,
                                  1 << 8, 1 << 7, 1 << 7, ctypes.c_void_p(4096), fa.FA_TQ_F32,
                                  lay, None) == fa.FA_TQ_EUNSUPPORTED

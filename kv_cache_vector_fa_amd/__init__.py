"""MI355X (gfx950) TurboQuant MSE KV-cache path: Python binding of ``libfa_tq.so``.

The functions here have the names of the C ABI in ``include/fa_tq.h`` and only
marshal arguments: torch tensors supply device memory and the current HIP stream;
every step of the path runs in the library's HIP kernels.  There is no fallback:
if the library is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_TQ_LIB names another build of the library (e.g. the AddressSanitizer host build)
LIB_PATH = os.environ.get("FA_TQ_LIB") or os.path.join(_HERE, "libfa_tq.so")

FA_TQ_OK, FA_TQ_EINVAL, FA_TQ_EUNSUPPORTED, FA_TQ_EHIP = 0, 1, 2, 3
FA_TQ_F32, FA_TQ_BF16 = 0, 1
QK = 128

_lib = None


class FaTqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa_tq status {status}: {message}")
        self.status = status


class Codebook(ctypes.Structure):
    """Mirror of ``fa_tq_codebook``."""
    _fields_ = [("dim", ctypes.c_int32), ("bits", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("boundaries", ctypes.c_float * 15), ("centroids", ctypes.c_float * 16)]

    def arrays(self):
        L = self.levels
        if self.bits == 8:
            return np.zeros(0, np.float32), np.zeros(0, np.float32)
        return (np.array(self.boundaries[:L - 1], np.float32),
                np.array(self.centroids[:L], np.float32))


class Layout(ctypes.Structure):
    """Mirror of ``fa_tq_layout`` (element strides of batch, head, token)."""
    _fields_ = [("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_t", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGS = {
    "fa_tq_codebook_init": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(Codebook)]),
    "fa_tq_signs": (ctypes.c_int, [ctypes.c_uint64, ctypes.c_int32, _P]),
    "fa_tq_code_bytes": (ctypes.c_int32, [ctypes.c_int32]),
    "fa_tq_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 5),
    "fa_tq_last_error": (ctypes.c_char_p, []),
    "fa_tq_encode": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.c_uint64, ctypes.c_int32,
                                    _P, ctypes.c_int, Layout, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _P, ctypes.c_int32, _P, _P, _P]),
    "fa_tq_encode_ex": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.c_uint64, ctypes.c_uint32,
                                       ctypes.c_int32, _P, ctypes.c_int, Layout, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                                       _P]),
    "fa_tq_encode_kv": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.POINTER(Codebook),
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, _P, _P,
                                       ctypes.c_int, Layout, Layout, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                                       _P, _P, _P]),
    "fa_tq_decode_kv": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.c_uint64, ctypes.c_uint32,
                                       ctypes.c_int32, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int, Layout,
                                       _P]),
    "fa_tq_decode": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.c_uint64, ctypes.c_int32,
                                    _P, _P, ctypes.c_int64, _P, _P]),
    "fa_tq_attn_decode": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.POINTER(Codebook),
                                         ctypes.c_uint64, ctypes.c_int32, _P, ctypes.c_int,
                                         _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P,
                                         _P, ctypes.c_size_t, _P]),
    "fa_tq_attn_append": (ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.POINTER(Codebook),
                                         ctypes.c_uint64, ctypes.c_int32, _P, ctypes.c_int,
                                         _P, _P, ctypes.c_int, Layout, Layout, ctypes.c_int32,
                                         _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P,
                                         _P, ctypes.c_size_t, _P]),
}
# fa_tq_attn_decode_ex without the workspace pointer and size.
_SIGS["fa_tq_attn_decode_noalloc"] = (
    ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.POINTER(Codebook), ctypes.c_uint64,
                   ctypes.c_uint32, ctypes.c_int32, _P, ctypes.c_int, _P, _P, _P, _P, _P,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_float, _P, _P])
NOALLOC_SCRATCH_BYTES = 8 << 20   # FA_TQ_NOALLOC_SCRATCH_BYTES
# Dense random orthogonal rotation (head_dims that are not a power of two).
_SIGS["fa_tq_rotation_dense"] = (ctypes.c_int, [ctypes.c_uint64, ctypes.c_int32, _P])
_SIGS["fa_tq_encode_dense"] = (
    ctypes.c_int, [ctypes.POINTER(Codebook), _P, ctypes.c_int32, _P, ctypes.c_int, Layout,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P, _P,
                   _P])
_SIGS["fa_tq_decode_dense"] = (
    ctypes.c_int, [ctypes.POINTER(Codebook), _P, ctypes.c_int32, _P, _P, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int, Layout,
                   _P])
_SIGS["fa_tq_attn_dense_workspace_bytes"] = (ctypes.c_size_t, [ctypes.c_int32] * 4)
_SIGS["fa_tq_attn_decode_dense"] = (
    ctypes.c_int, [ctypes.POINTER(Codebook), ctypes.POINTER(Codebook), _P, ctypes.c_int32,
                   ctypes.c_uint32, _P, ctypes.c_int, _P, _P, _P, _P, _P, ctypes.c_int32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _P, _P,
                   ctypes.c_size_t, _P])
DENSE_MAX_HEAD_DIM = 192
DENSE_ATTN_MAX_HEAD_DIM = 128
# The _ex entry points take the variant flags right after the seed.
for _name in ("fa_tq_attn_decode", "fa_tq_attn_append"):
    _r, _a = _SIGS[_name]
    _SIGS[_name + "_ex"] = (_r, _a[:3] + [ctypes.c_uint32] + _a[3:])

TWO_SIGNS = 1       # FA_TQ_TWO_SIGNS: R = D2 H D1 / sqrt(128)
NORM_CORRECT = 2    # FA_TQ_NORM_CORRECT: stored norm n / ||c[codes]|| (encode)
WHOLE_VECTOR = 4    # FA_TQ_WHOLE_VECTOR: one rotation over head_dim, one norm per vector
ATTN_VECTOR_ALU = 8  # FA_TQ_ATTN_VECTOR_ALU: the vector-ALU attention kernels (groups up to 16)


def _with_flags(lib, name, args, flags, seed_at):
    """The plain entry point for flags 0, else its _ex form with the flags right after
    the seed (argument ``seed_at``)."""
    if not flags:
        return getattr(lib, name), args
    k = seed_at + 1
    return getattr(lib, name + "_ex"), args[:k] + (ctypes.c_uint32(flags),) + args[k:]


def load(path: str | None = None):
    """Load ``libfa_tq.so`` (built by ``kv_cache_vector_fa_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != FA_TQ_OK:
        raise FaTqError(status, _lib.fa_tq_last_error().decode())


def exported_symbols():
    return list(_SIGS)


# --------------------------------------------------------------------------- host

def codebook_init(dim: int, bits: int) -> Codebook:
    lib = load()
    cb = Codebook()
    _check(lib.fa_tq_codebook_init(dim, bits, ctypes.byref(cb)))
    return cb


def codebook_from_arrays(bits: int, boundaries=None, centroids=None, dim: int = QK) -> Codebook:
    """A ``Codebook`` filled from explicit tables (e.g. tables built elsewhere)."""
    cb = Codebook()
    cb.dim, cb.bits, cb.levels = dim, bits, 1 << bits
    if bits != 8:
        for i, v in enumerate(np.asarray(boundaries, np.float32)):
            cb.boundaries[i] = float(v)
        for i, v in enumerate(np.asarray(centroids, np.float32)):
            cb.centroids[i] = float(v)
    return cb


def signs(seed: int, head_dim: int) -> np.ndarray:
    lib = load()
    out = np.zeros(head_dim, np.int8)
    _check(lib.fa_tq_signs(seed, head_dim, out.ctypes.data))
    return out


def rotation_dense(seed: int, dim: int) -> np.ndarray:
    """The dense rotation R (fp32 [dim, dim], row-major) of ``fa_tq_rotation_dense``."""
    lib = load()
    out = np.zeros((dim, dim), np.float32)
    _check(lib.fa_tq_rotation_dense(seed, dim, out.ctypes.data))
    return out


def code_bytes(bits: int) -> int:
    return int(load().fa_tq_code_bytes(bits))


def attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, head_dim=QK) -> int:
    return int(load().fa_tq_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, head_dim))


# ------------------------------------------------------------------------- device

def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_TQ_BF16
    if t.dtype == torch.float32:
        return FA_TQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def whole_length(head_dim: int) -> int:
    """Transform length of the whole-vector mode: head_dim zero-padded to 128 or 256."""
    return QK if head_dim <= QK else 2 * QK


def cache_buffers(batch, n_kv_heads, t_max, head_dim, bits, device="cuda", flags: int = 0):
    """Allocate (codes, norms) for the packed SoA cache layout (with WHOLE_VECTOR:
    whole_length(head_dim) / 128 code blocks and one norm per vector)."""
    import torch
    whole = bool(flags & WHOLE_VECTOR)
    nblk = (whole_length(head_dim) if whole else head_dim) // QK
    codes = torch.empty((batch, n_kv_heads, t_max, nblk, code_bytes(bits)), dtype=torch.uint8,
                        device=device)
    norms = torch.empty((batch, n_kv_heads, t_max, 1 if whole else nblk), dtype=torch.int16,
                        device=device)
    return codes, norms


def encode(cb: Codebook, seed: int, x, t_max: int | None = None, t0=None, codes=None,
           norms=None, stream=None, flags: int = 0):
    """Encode x [B, Hkv, T, d] (bf16/fp32, channel stride 1) into the packed cache."""
    B, H, T, d = x.shape
    t_max = T if t_max is None else t_max
    if codes is None or norms is None:
        codes, norms = cache_buffers(B, H, t_max, d, cb.bits, x.device, flags)
    encode_call(cb, seed, x, codes, norms, t_max, t0, stream, flags)()
    return codes, norms


def decode(cb: Codebook, seed: int, codes, norms, head_dim: int, out=None, stream=None):
    """Decode packed blocks; codes [..., nblk, cb] -> float32 [..., head_dim]."""
    import torch
    lib = load()
    nblk = head_dim // QK
    cbytes = code_bytes(cb.bits)
    if head_dim % QK or codes.dim() < 2 or tuple(codes.shape[-2:]) != (nblk, cbytes) or \
            codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError(f"codes: expected contiguous uint8 [..., {nblk}, {cbytes}], got "
                         f"{codes.dtype} {tuple(codes.shape)}")
    n_vec = codes.numel() // (nblk * cbytes)
    if norms.dtype != torch.int16 or not norms.is_contiguous() or norms.numel() != n_vec * nblk:
        raise ValueError(f"norms: expected {n_vec * nblk} contiguous int16 (fp16 bits), got "
                         f"{norms.dtype} {tuple(norms.shape)}")
    if out is None:
        out = torch.empty(tuple(codes.shape[:-2]) + (head_dim,), dtype=torch.float32,
                          device=codes.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != n_vec * head_dim:
        raise ValueError(f"out: expected {n_vec * head_dim} contiguous float32, got "
                         f"{out.dtype} {tuple(out.shape)}")
    _same_device(codes, norms, out)
    _check(lib.fa_tq_decode(ctypes.byref(cb), seed, head_dim, _ptr(codes), _ptr(norms), n_vec,
                            _ptr(out), _stream(stream)))
    return out


def _expect_blocks(nblk, head_dim, flags):
    want = (whole_length(head_dim) if flags & WHOLE_VECTOR else head_dim) // QK
    if nblk != want:
        raise ValueError(f"a cache of {nblk} blocks per vector for head_dim {head_dim}")


def decode_kv(cb: Codebook, seed: int, codes, norms, n_tokens: int | None = None, out=None,
              out_dtype=None, stream=None, flags: int = 0, head_dim: int | None = None):
    """Restore a packed cache [B, Hkv, T_max, nblk, cb] to a K or V tensor: tokens
    [0, n_tokens) of every row into out [B, Hkv, n_tokens, head_dim] (any strides
    with channel stride 1, bf16 or float32; bf16 by default).  head_dim defaults to
    out's last size, else nblk * 128 (a padded whole-vector cache needs it)."""
    import torch
    lib = load()
    B, H, t_max, nblk, cbytes = codes.shape
    d = head_dim or (out.shape[3] if out is not None else nblk * QK)
    _expect_blocks(nblk, d, flags)
    n_tokens = t_max if n_tokens is None else n_tokens
    if cbytes != code_bytes(cb.bits):
        raise ValueError(f"code rows of {cbytes} bytes for {cb.bits}-bit codes")
    nnorm = 1 if flags & WHOLE_VECTOR else nblk
    if not codes.is_contiguous() or tuple(norms.shape) != (B, H, t_max, nnorm) or \
            not norms.is_contiguous():
        raise ValueError("codes/norms must be the contiguous packed cache")
    if out is None:
        out = torch.empty((B, H, n_tokens, d), dtype=out_dtype or torch.bfloat16,
                          device=codes.device)
    if tuple(out.shape) != (B, H, n_tokens, d) or out.stride(3) != 1:
        raise ValueError(f"out {tuple(out.shape)} for a cache of {tuple(codes.shape)}")
    lay = Layout(out.stride(0), out.stride(1), out.stride(2))
    _check(lib.fa_tq_decode_kv(ctypes.byref(cb), seed, flags, d, _ptr(codes), _ptr(norms), B,
                               H, n_tokens, t_max, _ptr(out), _dtype_code(out), lay,
                               _stream(stream)))
    return out


def decode_kv_call(cb: Codebook, seed: int, codes, norms, out, n_tokens: int | None = None,
                   stream=None, flags: int = 0):
    """``decode_kv`` with its arguments marshalled once (see ``encode_call``)."""
    lib = load()
    B, H, t_max, nblk, cbytes = codes.shape
    d = out.shape[3]
    _expect_blocks(nblk, d, flags)
    n_tokens = t_max if n_tokens is None else n_tokens
    if tuple(out.shape) != (B, H, n_tokens, d) or out.stride(3) != 1:
        raise ValueError(f"out {tuple(out.shape)} for a cache of {tuple(codes.shape)}")
    lay = Layout(out.stride(0), out.stride(1), out.stride(2))
    args = (ctypes.byref(cb), ctypes.c_uint64(seed), ctypes.c_uint32(flags), ctypes.c_int32(d),
            _ptr(codes), _ptr(norms), ctypes.c_int32(B), ctypes.c_int32(H),
            ctypes.c_int32(n_tokens), ctypes.c_int32(t_max), _ptr(out),
            ctypes.c_int(_dtype_code(out)), lay, _stream(stream))
    fn = lib.fa_tq_decode_kv
    keep = (cb, codes, norms, out)

    def call():
        _check(fn(*args))
        return keep
    return call


def attn_workspace(batch, n_q_heads, n_kv_heads, t_max, head_dim=QK, device="cuda"):
    """A workspace for ``attn_decode`` / ``attn_append`` (reusable by later calls in
    order on one stream)."""
    import torch
    need = attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, head_dim)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


def attn_decode(cb_k: Codebook, cb_v: Codebook, seed: int, q, k_codes, k_norms, v_codes,
                v_norms, seq_lens, scale: float, out=None, workspace=None, stream=None,
                flags: int = 0):
    """Single-query decode attention.  q [B, Hq, d]; caches [B, Hkv, T_max, nblk, cb]."""
    import torch
    B, Hq, d = q.shape
    Hkv, t_max = k_codes.shape[1], k_codes.shape[2]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = attn_workspace(B, Hq, Hkv, t_max, d, q.device)
    attn_decode_call(cb_k, cb_v, seed, q, k_codes, k_norms, v_codes, v_norms, seq_lens, scale,
                     out, workspace, stream, flags)()
    return out


def _same_device(*ts):
    """Every tensor on one GPU (the kernels take raw device addresses)."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1 or next(iter(devs)).type != "cuda":
        raise ValueError(f"tensors must share one GPU device, got {sorted(map(str, devs))}")


def attn_decode_noalloc(cb_k: Codebook, cb_v: Codebook, seed: int, q, k_codes, k_norms,
                        v_codes, v_norms, seq_lens, scale: float, out, stream=None,
                        flags: int = 0):
    """``attn_decode`` through fa_tq_attn_decode_noalloc: no workspace, the split
    partials go to the library's per-GPU scratch array (calls that overlap on one
    GPU race).  ``out`` [B, Hq, d] float32 must be given (nothing is allocated)."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    Hkv, t_max = k_codes.shape[1], k_codes.shape[2]
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _expect(seq_lens, (B,), torch.int32, "seq_lens")
    _expect_cache(k_codes, k_norms, B, Hkv, t_max, d, cb_k.bits, "k cache")
    _expect_cache(v_codes, v_norms, B, Hkv, t_max, d, cb_v.bits, "v cache")
    _expect(out, (B, Hq, d), torch.float32, "out")
    _same_device(q, seq_lens, k_codes, k_norms, v_codes, v_norms, out)
    _check(lib.fa_tq_attn_decode_noalloc(
        ctypes.byref(cb_k), ctypes.byref(cb_v), ctypes.c_uint64(seed), ctypes.c_uint32(flags),
        ctypes.c_int32(d), _ptr(q), ctypes.c_int(_dtype_code(q)), _ptr(k_codes),
        _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), _ptr(seq_lens), ctypes.c_int32(B),
        ctypes.c_int32(Hq), ctypes.c_int32(Hkv), ctypes.c_int32(t_max), ctypes.c_float(scale),
        _ptr(out), _stream(stream)))
    return out


def _expect(t, shape, dtype, name):
    """Shape/dtype/contiguity check of a device buffer the kernels index densely."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} (contiguous={t.is_contiguous()})")


def _expect_cache(codes, norms, B, H, t_max, d, bits, name):
    import torch
    nblk = d // QK
    _expect(codes, (B, H, t_max, nblk, code_bytes(bits)), torch.uint8, f"{name} codes")
    _expect(norms, (B, H, t_max, nblk), torch.int16, f"{name} norms")


def attn_append(cb_k: Codebook, cb_v: Codebook, seed: int, q, k_new, v_new, pos, k_codes,
                k_norms, v_codes, v_norms, scale: float, out=None, workspace=None, stream=None,
                flags: int = 0):
    """Append k_new/v_new [B, Hkv, n_new, d] at positions pos [B] (slot = position mod
    T_max) into the packed caches, then decode attention for q [B, Hq, d]."""
    import torch
    B, Hq, d = q.shape
    Hkv, t_max = k_new.shape[1], k_codes.shape[2]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = attn_workspace(B, Hq, Hkv, t_max, d, q.device)
    attn_append_call(cb_k, cb_v, seed, q, k_new, v_new, pos, k_codes, k_norms, v_codes,
                     v_norms, scale, out, workspace, stream, flags)()
    return out


# ------------------------------------------------------------ prepared device calls

def encode_call(cb: Codebook, seed: int, x, codes, norms, t_max: int | None = None, t0=None,
                stream=None, flags: int = 0):
    """``encode`` with its arguments marshalled once: returns a callable that launches
    fa_tq_encode on the same tensors (for tight loops where per-call Python work
    would dominate the kernel)."""
    import torch
    lib = load()
    B, H, T, d = x.shape
    if x.stride(3) != 1:
        raise ValueError("channel stride must be 1")
    t_max = T if t_max is None else t_max
    whole = bool(flags & WHOLE_VECTOR)
    nblk = (whole_length(d) if whole else d) // QK
    if not whole and d % QK:
        raise ValueError(f"head_dim {d} is not a multiple of {QK}")
    _expect(codes, (B, H, t_max, nblk, code_bytes(cb.bits)), torch.uint8, "codes")
    _expect(norms, (B, H, t_max, 1 if whole else nblk), torch.int16, "norms")
    if t0 is not None:
        _expect(t0, (B,), torch.int32, "t0")
    _same_device(x, codes, norms, t0)
    args = (ctypes.byref(cb), ctypes.c_uint64(seed), ctypes.c_int32(d), _ptr(x),
            ctypes.c_int(_dtype_code(x)), Layout(x.stride(0), x.stride(1), x.stride(2)),
            ctypes.c_int32(B), ctypes.c_int32(H), ctypes.c_int32(T), _ptr(t0),
            ctypes.c_int32(t_max), _ptr(codes), _ptr(norms), _stream(stream))
    fn, args = _with_flags(lib, "fa_tq_encode", args, flags, 1)
    keep = (cb, x, codes, norms, t0)

    def call():
        _check(fn(*args))
        return keep
    return call


def encode_kv_call(cb_k: Codebook, cb_v: Codebook, seed: int, k, v, k_codes, k_norms, v_codes,
                   v_norms, t_max: int | None = None, t0=None, stream=None, flags: int = 0):
    """``encode_kv`` with its arguments marshalled once (see ``encode_call``)."""
    import torch
    lib = load()
    B, H, T, d = k.shape
    if tuple(v.shape) != (B, H, T, d) or v.dtype != k.dtype:
        raise ValueError(f"v: expected {k.dtype} {(B, H, T, d)}, got {v.dtype} {tuple(v.shape)}")
    if k.stride(3) != 1 or v.stride(3) != 1:
        raise ValueError("channel stride must be 1")
    t_max = T if t_max is None else t_max
    whole = bool(flags & WHOLE_VECTOR)
    nblk = (whole_length(d) if whole else d) // QK
    if not whole and d % QK:
        raise ValueError(f"head_dim {d} is not a multiple of {QK}")
    for name, cb, c, n in (("k", cb_k, k_codes, k_norms), ("v", cb_v, v_codes, v_norms)):
        _expect(c, (B, H, t_max, nblk, code_bytes(cb.bits)), torch.uint8, f"{name}_codes")
        _expect(n, (B, H, t_max, 1 if whole else nblk), torch.int16, f"{name}_norms")
    if t0 is not None:
        _expect(t0, (B,), torch.int32, "t0")
    _same_device(k, v, k_codes, k_norms, v_codes, v_norms, t0)
    args = (ctypes.byref(cb_k), ctypes.byref(cb_v), ctypes.c_uint64(seed), ctypes.c_uint32(flags),
            ctypes.c_int32(d), _ptr(k), _ptr(v), ctypes.c_int(_dtype_code(k)),
            Layout(k.stride(0), k.stride(1), k.stride(2)),
            Layout(v.stride(0), v.stride(1), v.stride(2)), ctypes.c_int32(B), ctypes.c_int32(H),
            ctypes.c_int32(T), _ptr(t0), ctypes.c_int32(t_max), _ptr(k_codes), _ptr(k_norms),
            _ptr(v_codes), _ptr(v_norms), _stream(stream))
    fn = lib.fa_tq_encode_kv
    keep = (cb_k, cb_v, k, v, k_codes, k_norms, v_codes, v_norms, t0)

    def call():
        _check(fn(*args))
        return keep
    return call


def encode_kv(cb_k: Codebook, cb_v: Codebook, seed: int, k, v, t_max: int | None = None,
              t0=None, k_cache=None, v_cache=None, stream=None, flags: int = 0):
    """Encode K and V [B, Hkv, T, d] of the same tokens in one call (fa_tq_encode_kv);
    returns ((k_codes, k_norms), (v_codes, v_norms)), bit for bit those of ``encode``."""
    B, H, T, d = k.shape
    t_max = T if t_max is None else t_max
    if k_cache is None:
        k_cache = cache_buffers(B, H, t_max, d, cb_k.bits, k.device, flags)
    if v_cache is None:
        v_cache = cache_buffers(B, H, t_max, d, cb_v.bits, v.device, flags)
    encode_kv_call(cb_k, cb_v, seed, k, v, *k_cache, *v_cache, t_max, t0, stream, flags)()
    return k_cache, v_cache


def attn_decode_call(cb_k: Codebook, cb_v: Codebook, seed: int, q, k_codes, k_norms, v_codes,
                     v_norms, seq_lens, scale: float, out, workspace, stream=None,
                     flags: int = 0):
    """``attn_decode`` with its arguments marshalled once (see ``encode_call``)."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    Hkv, t_max = k_codes.shape[1], k_codes.shape[2]
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _expect(seq_lens, (B,), torch.int32, "seq_lens")
    _expect_cache(k_codes, k_norms, B, Hkv, t_max, d, cb_k.bits, "k cache")
    _expect_cache(v_codes, v_norms, B, Hkv, t_max, d, cb_v.bits, "v cache")
    _expect(out, (B, Hq, d), torch.float32, "out")
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_device(q, seq_lens, k_codes, k_norms, v_codes, v_norms, out, workspace)
    args = (ctypes.byref(cb_k), ctypes.byref(cb_v), ctypes.c_uint64(seed), ctypes.c_int32(d),
            _ptr(q), ctypes.c_int(_dtype_code(q)), _ptr(k_codes), _ptr(k_norms),
            _ptr(v_codes), _ptr(v_norms), _ptr(seq_lens), ctypes.c_int32(B),
            ctypes.c_int32(Hq), ctypes.c_int32(Hkv), ctypes.c_int32(t_max),
            ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(stream))
    fn, args = _with_flags(lib, "fa_tq_attn_decode", args, flags, 2)
    keep = (cb_k, cb_v, q, k_codes, k_norms, v_codes, v_norms, seq_lens, out, workspace)

    def call():
        _check(fn(*args))
        return keep
    return call



def attn_append_call(cb_k: Codebook, cb_v: Codebook, seed: int, q, k_new, v_new, pos, k_codes,
                     k_norms, v_codes, v_norms, scale: float, out, workspace, stream=None,
                     flags: int = 0):
    """``attn_append`` with its arguments marshalled once (see ``encode_call``)."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    _, Hkv, n_new, _ = k_new.shape
    t_max = k_codes.shape[2]
    if k_new.dtype != v_new.dtype or k_new.stride(3) != 1 or v_new.stride(3) != 1:
        raise ValueError("k_new and v_new need one dtype and channel stride 1")
    if tuple(v_new.shape) != tuple(k_new.shape) or k_new.shape[0] != B or k_new.shape[3] != d:
        raise ValueError(f"k_new {tuple(k_new.shape)}, v_new {tuple(v_new.shape)} for q "
                         f"{tuple(q.shape)}")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _expect(pos, (B,), torch.int32, "pos")
    _expect_cache(k_codes, k_norms, B, Hkv, t_max, d, cb_k.bits, "k cache")
    _expect_cache(v_codes, v_norms, B, Hkv, t_max, d, cb_v.bits, "v cache")
    _expect(out, (B, Hq, d), torch.float32, "out")
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_device(q, k_new, v_new, pos, k_codes, k_norms, v_codes, v_norms, out, workspace)
    args = (ctypes.byref(cb_k), ctypes.byref(cb_v), ctypes.c_uint64(seed), ctypes.c_int32(d),
            _ptr(q), ctypes.c_int(_dtype_code(q)), _ptr(k_new), _ptr(v_new),
            ctypes.c_int(_dtype_code(k_new)),
            Layout(k_new.stride(0), k_new.stride(1), k_new.stride(2)),
            Layout(v_new.stride(0), v_new.stride(1), v_new.stride(2)), ctypes.c_int32(n_new),
            _ptr(pos), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms),
            ctypes.c_int32(B), ctypes.c_int32(Hq), ctypes.c_int32(Hkv), ctypes.c_int32(t_max),
            ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(stream))
    fn, args = _with_flags(lib, "fa_tq_attn_append", args, flags, 2)
    keep = (cb_k, cb_v, q, k_new, v_new, pos, k_codes, k_norms, v_codes, v_norms, out, workspace)

    def call():
        _check(fn(*args))
        return keep
    return call


def dense_cache_buffers(batch, n_kv_heads, t_max, head_dim, bits, device="cuda"):
    """(codes, norms) of a dense-rotation cache: [B, Hkv, T_max, ceil(d/128), cb] uint8
    and one fp16 norm per vector [B, Hkv, T_max] (int16 bits)."""
    import torch
    nblk = -(-head_dim // QK)
    codes = torch.zeros((batch, n_kv_heads, t_max, nblk, code_bytes(bits)), dtype=torch.uint8,
                        device=device)
    norms = torch.zeros((batch, n_kv_heads, t_max), dtype=torch.int16, device=device)
    return codes, norms


def encode_dense(cb: Codebook, rotation, x, t_max: int | None = None, t0=None, codes=None,
                 norms=None, stream=None):
    """Encode x [B, Hkv, T, d] (bf16/fp32, channel stride 1) with the dense rotation
    (``rotation``: device fp32 [d, d] from ``rotation_dense``)."""
    import torch
    lib = load()
    B, H, T, d = x.shape
    t_max = T if t_max is None else t_max
    if codes is None or norms is None:
        codes, norms = dense_cache_buffers(B, H, t_max, d, cb.bits, x.device)
    nblk = -(-d // QK)
    _expect(codes, (B, H, t_max, nblk, code_bytes(cb.bits)), torch.uint8, "codes")
    _expect(norms, (B, H, t_max), torch.int16, "norms")
    _expect(rotation, (d, d), torch.float32, "rotation")
    if x.stride(3) != 1:
        raise ValueError("x: channel stride must be 1")
    if t0 is not None:
        _expect(t0, (B,), torch.int32, "t0")
    _same_device(x, codes, norms, rotation, *([t0] if t0 is not None else []))
    lay = Layout(x.stride(0), x.stride(1), x.stride(2))
    _check(lib.fa_tq_encode_dense(ctypes.byref(cb), _ptr(rotation), d, _ptr(x), _dtype_code(x),
                                  lay, B, H, T, _ptr(t0), t_max, _ptr(codes), _ptr(norms),
                                  _stream(stream)))
    return codes, norms


def attn_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max) -> int:
    return int(load().fa_tq_attn_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max))


def attn_decode_dense_call(cb_k: Codebook, cb_v: Codebook, rotation, q, k_codes, k_norms,
                           v_codes, v_norms, seq_lens, scale: float, out, workspace,
                           flags: int = 0, stream=None):
    """``attn_decode_dense`` with its arguments checked and marshalled once (see
    ``encode_call``)."""
    import torch
    lib = load()
    B, Hq, d = q.shape
    Hkv, t_max = k_codes.shape[1], k_codes.shape[2]
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _expect(seq_lens, (B,), torch.int32, "seq_lens")
    _expect(rotation, (d, d), torch.float32, "rotation")
    for name, c, n, cb in (("k", k_codes, k_norms, cb_k), ("v", v_codes, v_norms, cb_v)):
        _expect(c, (B, Hkv, t_max, -(-d // QK), code_bytes(cb.bits)), torch.uint8, f"{name} codes")
        _expect(n, (B, Hkv, t_max), torch.int16, f"{name} norms")
    _expect(out, (B, Hq, d), torch.float32, "out")
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_device(q, seq_lens, rotation, k_codes, k_norms, v_codes, v_norms, out, workspace)
    args = (ctypes.byref(cb_k), ctypes.byref(cb_v), _ptr(rotation), ctypes.c_int32(d),
            ctypes.c_uint32(flags), _ptr(q), ctypes.c_int(_dtype_code(q)), _ptr(k_codes),
            _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), _ptr(seq_lens), ctypes.c_int32(B),
            ctypes.c_int32(Hq), ctypes.c_int32(Hkv), ctypes.c_int32(t_max),
            ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(stream))
    fn = lib.fa_tq_attn_decode_dense
    keep = (cb_k, cb_v, rotation, q, k_codes, k_norms, v_codes, v_norms, seq_lens, out,
            workspace)

    def call():
        _check(fn(*args))
        return keep
    return call


def attn_decode_dense(cb_k: Codebook, cb_v: Codebook, rotation, q, k_codes, k_norms, v_codes,
                      v_norms, seq_lens, scale: float, out=None, workspace=None, flags: int = 0,
                      stream=None):
    """Decode attention over dense-rotation caches (``encode_dense``, head_dim <= 128):
    q [B, Hq, d] (bf16/fp32), caches [B, Hkv, T_max, 1, cb] with norms [B, Hkv, T_max];
    returns out [B, Hq, d] float32."""
    import torch
    B, Hq, d = q.shape
    Hkv, t_max = k_codes.shape[1], k_codes.shape[2]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(attn_dense_workspace_bytes(B, Hq, Hkv, t_max), 16),
                                dtype=torch.uint8, device=q.device)
    attn_decode_dense_call(cb_k, cb_v, rotation, q, k_codes, k_norms, v_codes, v_norms,
                           seq_lens, scale, out, workspace, flags, stream)()
    return out


def decode_dense(cb: Codebook, rotation, codes, norms, head_dim: int, n_tokens: int | None = None,
                 out=None, out_dtype=None, stream=None):
    """Restore a dense-rotation cache to out [B, Hkv, n_tokens, head_dim] (fp32 by
    default, or bf16; channel stride 1)."""
    import torch
    lib = load()
    B, H, t_max, nblk, cbytes = codes.shape
    n_tokens = t_max if n_tokens is None else n_tokens
    if nblk != -(-head_dim // QK) or cbytes != code_bytes(cb.bits):
        raise ValueError("codes: not a dense-rotation cache of this head_dim and bit width")
    _expect(codes, (B, H, t_max, nblk, cbytes), torch.uint8, "codes")
    _expect(norms, (B, H, t_max), torch.int16, "norms")
    _expect(rotation, (head_dim, head_dim), torch.float32, "rotation")
    if out is None:
        out = torch.empty((B, H, n_tokens, head_dim), dtype=out_dtype or torch.float32,
                          device=codes.device)
    if tuple(out.shape) != (B, H, n_tokens, head_dim) or out.stride(3) != 1:
        raise ValueError(f"out {tuple(out.shape)} for a cache of {tuple(codes.shape)}")
    _same_device(codes, norms, rotation, out)
    lay = Layout(out.stride(0), out.stride(1), out.stride(2))
    _check(lib.fa_tq_decode_dense(ctypes.byref(cb), _ptr(rotation), head_dim, _ptr(codes),
                                  _ptr(norms), B, H, n_tokens, t_max, _ptr(out), _dtype_code(out),
                                  lay, _stream(stream)))
    return out

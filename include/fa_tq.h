/*
 * fa_tq.h -- C ABI of the MI355X (gfx950) TurboQuant MSE KV-cache library.
 *
 * Pages cited by title and section:
 *   [Spec]   "TurboQuant KV Cache Compression -- Spec"
 *   [turboq] "TurboQuant KV Cache (turboq2 / turboq3 / turboq4)"
 *
 * Every symbol has C linkage.  No C++ exception, abort or torch type crosses this
 * boundary: pointers are plain host or device addresses and sizes are integers.
 *
 * Ownership: the caller allocates and frees every buffer.  The library keeps no
 * device state and allocates nothing on the device; device entry points are
 * asynchronous on the caller's stream (a hipStream_t passed as void*, NULL = the
 * null stream) and never synchronize the host.
 *
 * Errors: arguments are checked on the host before any launch.  A non-OK status
 * launches nothing and leaves a message readable with fa_tq_last_error() (per host
 * thread).  FA_TQ_EINVAL: a bad size, pointer, alignment or table; FA_TQ_EUNSUPPORTED:
 * a valid combination the library has no kernel for; FA_TQ_EHIP: the HIP runtime
 * reported an error at launch.  Faults inside a kernel surface at the caller's next
 * synchronization, as for any HIP kernel.
 *
 * Packed-cache layout (structure of arrays; QK = 128-element blocks, nblk = d/128):
 *   codes[B][Hkv][T_max][nblk][cb]   uint8, cb = fa_tq_code_bytes(bits)
 *   norms[B][Hkv][T_max][nblk]       uint16 holding IEEE binary16 bits
 * Bits inside a block are packed least-significant first: 2-bit 4 codes per byte;
 * 3-bit as two planes (32 bytes of low two bits, then 16 bytes of the high bit);
 * 4-bit 2 codes per byte; 8-bit one code per byte ([Spec] "Step 3: Packing";
 * [turboq] "Block structures").  Every code row starts on a 16-byte boundary.
 */
#ifndef FA_TQ_H
#define FA_TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_TQ_QK 128          /* elements per block ([turboq] "Block structures") */
#define FA_TQ_MAX_HEAD_DIM 2048

typedef enum {
    FA_TQ_OK = 0,
    FA_TQ_EINVAL = 1,
    FA_TQ_EUNSUPPORTED = 2,
    FA_TQ_EHIP = 3
} fa_tq_status;

typedef enum { FA_TQ_F32 = 0, FA_TQ_BF16 = 1 } fa_tq_dtype;

/*
 * Variant flags of the _ex entry points ([turboq] "Encode pipeline"):
 *   FA_TQ_TWO_SIGNS: the rotation is R = D2 H D1 / sqrt(128) (step 2: a second fixed
 *     +/-1 vector after the normalized butterflies); D1 holds draws 0 .. head_dim-1
 *     of the seed's SplitMix64 stream (as fa_tq_signs), D2 draws head_dim ..
 *     2 head_dim - 1.  Encode, decode and attention of one cache must agree on it.
 *     Encoding with bits 2-4 needs a mirror-symmetric codebook (as fa_tq_codebook_init
 *     builds): the sign change of D2 is applied as the mirrored code.
 *   FA_TQ_NORM_CORRECT (encode only, bits 2-4): store grp_norm / recon_norm (step 4),
 *     recon_norm being the norm of the block's centroid values c[code_i] (fp32,
 *     squares summed pairwise as for the input norm), so a decoded block keeps its
 *     input norm up to the fp16 rounding of the stored value.
 *   FA_TQ_WHOLE_VECTOR (encode and fa_tq_decode_kv only; no other flag): [Spec]
 *     "Step 1"/"Step 2" read literally, one rotation R = D H_d' / sqrt(d') over the
 *     whole head_dim d with a codebook built for dim = d', and one fp16 norm per
 *     vector: norms[B][Hkv][T_max] instead of [B][Hkv][T_max][nblk].  d' = d for d
 *     = 128 or 256; any other d in (64, 256] that is a multiple of 8 is zero-padded
 *     to d' = 128 or 256, the next power of two ([Spec] "Hadamard Transform
 *     Detail"): the codes are those of all d' transformed elements (nblk = d'/128),
 *     the signs D are draws 0 .. d'-1, and decoding keeps the first d outputs of the
 *     inverse.  The codes are packed per consecutive 128 elements exactly as the
 *     blocked layout.  Arithmetic as the blocked mode over d' elements (squares
 *     summed over index bits 0, 1, ... in order, the padding adding zeros;
 *     butterflies in stage order 1 .. d'/2, c = fp32(1/sqrt(d'))).
 *   FA_TQ_ATTN_VECTOR_ALU (fa_tq_attn_decode_ex and fa_tq_attn_decode_noalloc only):
 *     run the vector-ALU attention kernels instead of the matrix-core kernels (group
 *     sizes n_q_heads / n_kv_heads up to 16), e.g. to compare the two; the result is
 *     the same computation ([Spec] "Optimization: Fused dequant-dot") under the same
 *     accuracy bound.
 * Entry points without _ex use flags 0.
 */
#define FA_TQ_TWO_SIGNS 1u
#define FA_TQ_NORM_CORRECT 2u
#define FA_TQ_WHOLE_VECTOR 4u
#define FA_TQ_ATTN_VECTOR_ALU 8u

/*
 * Scalar quantizer for one 128-element block ([Spec] "Step 2: Lloyd-Max Scalar
 * Quantization": bits, levels, boundaries[15], centroids[16]; plus the dimension
 * the table was built for).  Plain data, owned by the caller, passed by pointer
 * and copied into the kernel arguments.  For bits 2..4 the code of a rotated,
 * normalized coordinate u is #{j : boundaries[j] < u} and its value centroids[code].
 * bits == 8 selects the uniform 256-level grid of [turboq] "At a glance" (turboq8):
 * the arrays are unused and must be zero.
 */
typedef struct {
    int32_t dim;            /* 128 (per QK block); d' (128 or 256) for FA_TQ_WHOLE_VECTOR */
    int32_t bits;           /* 2, 3, 4, or 8 */
    int32_t levels;         /* 1 << bits */
    float boundaries[15];   /* levels - 1 used, strictly ascending */
    float centroids[16];    /* levels used, ascending */
} fa_tq_codebook;

/* Element strides of the (batch, head, token) axes of an input tensor; the channel
 * stride is 1.  Each stride must be a multiple of 8 elements. */
typedef struct {
    int64_t stride_b;
    int64_t stride_h;
    int64_t stride_t;
} fa_tq_layout;

/*
 * Lloyd-Max quantizer for the density of a rotated, L2-normalized coordinate,
 * proportional to (1 - y^2)^(dim/2 - 1) on [-1, 1] (the Beta(d/2, d/2) law of
 * [Spec] "Step 1"/"Step 2", with [Spec] "As-Built Notes" L2 normalization),
 * built as in [Spec] "Codebook Generation": uniform start, centroids = conditional
 * means, boundaries = midpoints, iterated to convergence (|change| < 1e-12) in fp64
 * and stored as fp32.  dim in [4, 512] (FA_TQ_EINVAL outside); bits in {2, 3, 4, 8}
 * (8: grid, arrays zeroed).  Host only: pure, deterministic, touches no device.
 */
fa_tq_status fa_tq_codebook_init(int32_t dim, int32_t bits, fa_tq_codebook *out);

/*
 * The random +/-1 diagonal of the rotation ([Spec] "Step 1": one head_dim array
 * generated from the seed, shared by K, V, all heads and layers).  out[i] = -1 when
 * bit 63 of the i-th output of SplitMix64 seeded with `seed` is set, else +1.
 * Host only.  out: host array of head_dim int8.
 */
fa_tq_status fa_tq_signs(uint64_t seed, int32_t head_dim, int8_t *out);

/* Packed bytes per 128-element block: 32, 48, 64, 128 for bits 2, 3, 4, 8; -1 else. */
int32_t fa_tq_code_bytes(int32_t bits);

/* Bytes of device workspace fa_tq_attn_decode needs for these sizes (0 on bad sizes). */
size_t fa_tq_attn_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t t_max, int32_t head_dim);

/* Text describing the last non-OK status on the calling host thread. */
const char *fa_tq_last_error(void);

/*
 * Encode ([Spec] "Overview" and "As-Built Notes"; [turboq] "Encode pipeline" steps
 * 1-3): for every 128-block of every vector x[b][h][t][:] (t < n_tokens):
 *   norm n = ||x_blk||, stored as fp16 in norms;
 *   u = H (s * x_blk) / (sqrt(128) n)   (signs s from `seed`, block j uses s[128j..]);
 *   code_i = #{j : boundaries[j] < u_i}, packed into codes.
 * bits == 8: codes of the uniform grid with the block's absmax scale in norms.
 * Arithmetic is fp32 in a fixed order, so codes and norms are reproducible bit for
 * bit: squares summed pairwise over index bits 0..6; sqrt and division correctly
 * rounded; butterflies in stage order 1, 2, ..., 64; u_i = h_i * (c / n) with
 * c = fp32(1/sqrt(128)).
 *   x: device, dtype x_dtype, element (b,h,t,c) at b*stride_b + h*stride_h +
 *      t*stride_t + c; 16-byte aligned.
 *   t0: device int32[batch] first cache position per sequence, or NULL for 0.
 *      Vector t goes to cache position t0[b] + t; positions >= t_max are skipped.
 *   codes, norms: device, SoA layout above with T_max = t_max, Hkv = n_kv_heads.
 * batch, n_kv_heads or n_tokens == 0 is an OK no-op.
 */
fa_tq_status fa_tq_encode(const fa_tq_codebook *cb, uint64_t seed, int32_t head_dim,
                          const void *x, fa_tq_dtype x_dtype, fa_tq_layout x_layout,
                          int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                          const int32_t *t0, int32_t t_max,
                          uint8_t *codes, uint16_t *norms, void *stream);

/* fa_tq_encode with variant flags (FA_TQ_TWO_SIGNS, FA_TQ_NORM_CORRECT, or
 * FA_TQ_WHOLE_VECTOR alone; in the last, codes hold nblk = d'/128 blocks per
 * vector and x holds head_dim elements). */
fa_tq_status fa_tq_encode_ex(const fa_tq_codebook *cb, uint64_t seed, uint32_t flags,
                             int32_t head_dim, const void *x, fa_tq_dtype x_dtype,
                             fa_tq_layout x_layout, int32_t batch, int32_t n_kv_heads,
                             int32_t n_tokens, const int32_t *t0, int32_t t_max,
                             uint8_t *codes, uint16_t *norms, void *stream);

/*
 * The keys and the values of the same tokens in one call (one rotation from the seed
 * for both, [Spec] "Step 1: Random Orthogonal Rotation"; each with its own bit width,
 * [Spec] "As-Built Notes", K4/V2 by default): codes and norms
 * equal to fa_tq_encode_ex of k with cb_k and of v with cb_v, bit for bit.  Both
 * inputs share x_dtype, head_dim, the sizes, t0 and t_max; each has its own layout
 * and cache.  With 2-4 bit codebooks and no FA_TQ_WHOLE_VECTOR both run in one
 * launch (workgroups split between them), else as two launches.  Every argument of
 * both halves is checked before anything is launched; errors as fa_tq_encode_ex.
 */
fa_tq_status fa_tq_encode_kv(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                             uint64_t seed, uint32_t flags, int32_t head_dim, const void *k,
                             const void *v, fa_tq_dtype x_dtype, fa_tq_layout k_layout,
                             fa_tq_layout v_layout, int32_t batch, int32_t n_kv_heads,
                             int32_t n_tokens, const int32_t *t0, int32_t t_max,
                             uint8_t *k_codes, uint16_t *k_norms, uint8_t *v_codes,
                             uint16_t *v_norms, void *stream);

/*
 * Decode ([Spec] "Overview": look up reconstruction values, then rotate back; the
 * exact inverse R^T = D H / sqrt(d)):  x_hat = s * (H (n16 * c[code])) / sqrt(128)
 * per block (bits 8: c[code] = (code - 127.5)/127.5 times the block scale).
 *   codes: device [n_vec][nblk][cb]; norms: device [n_vec][nblk];
 *   out: device float [n_vec][head_dim], 16-byte aligned.
 */
fa_tq_status fa_tq_decode(const fa_tq_codebook *cb, uint64_t seed, int32_t head_dim,
                          const uint8_t *codes, const uint16_t *norms, int64_t n_vec,
                          float *out, void *stream);

/*
 * Bulk restore of a packed cache to a plain K or V tensor (the decompression path
 * of the LMCache page "TurboQuant Serde Backend": compressed bytes back to the
 * original KV layout for storage reuse; no attention).  Every block of tokens
 * t < n_tokens of every (b, h) row is decoded as fa_tq_decode does and written to
 * out at element (b, h, t, c) = b*stride_b + h*stride_h + t*stride_t + c, as fp32 or
 * as bf16 (round to nearest even of the fp32 result).  The LMCache tensor
 * [2][num_layers][num_tokens][hidden] of one (K or V, layer) pair is the layout
 * stride_h = head_dim, stride_t = hidden with batch 1.
 *   codes, norms: device, SoA layout above (T_max = t_max, Hkv = n_kv_heads).
 *   out: device, 16-byte aligned; strides non-negative multiples of 8 elements.
 * flags: 0, FA_TQ_TWO_SIGNS or FA_TQ_WHOLE_VECTOR (how the cache was encoded; in
 * the last, codes hold d'/128 blocks per vector and head_dim elements are written).
 * batch, n_kv_heads or n_tokens == 0 is an OK no-op; n_tokens <= t_max.
 */
fa_tq_status fa_tq_decode_kv(const fa_tq_codebook *cb, uint64_t seed, uint32_t flags,
                             int32_t head_dim, const uint8_t *codes, const uint16_t *norms,
                             int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                             int32_t t_max, void *out, fa_tq_dtype out_dtype,
                             fa_tq_layout out_layout, void *stream);

/*
 * Dense random orthogonal rotation ([Spec] "Hadamard Transform Detail": for a
 * head_dim that is not a power of two, the alternative to zero-padding; [Spec] "Step 1:
 * Random Orthogonal Rotation": a fixed d x d orthogonal R from the seed, rotate(x) =
 * R x).  G[i][j] is standard normal number i*dim + j from the seed's SplitMix64
 * stream, continuing after the 2*dim draws of the two sign vectors (draws 2*dim,
 * 2*dim + 1, ...): draws z1, z2 give u1 = ((z1 >> 11) + 1/2) 2^-53, u2 = (z2 >> 11)
 * 2^-53 and the Box-Muller pair r cos(2 pi u2), r sin(2 pi u2), r = sqrt(-2 ln u1).
 * R is the Q factor of G = Q T with T's diagonal positive (fp64), rounded to fp32.
 *   out: host, float[dim * dim], R row-major (R[i][j] at out[i*dim + j]).
 *   dim in [2, 512] (FA_TQ_EINVAL outside).
 */
fa_tq_status fa_tq_rotation_dense(uint64_t seed, int32_t dim, float *out);

/*
 * Encode with the dense rotation: per vector x (head_dim elements, bf16 or fp32),
 * n = the fp32 norm of x (squares summed pairwise over index bits 0, 1, ... of x
 * zero-padded to a power of two), stored as fp16; codes of u = (R x) / n against cb
 * (code = #{j : b_j < u_j}).  The head_dim codes fill ceil(head_dim / 128) packed
 * 128-element blocks (the blocked byte layout; code 0 past head_dim); one norm per
 * vector: norms[B][Hkv][T_max].
 *   cb: a 2-4 bit codebook built for dim = head_dim whose adjacent boundaries are
 *   more than 2/1024 apart (they must fall in distinct cells of the encoder's uniform
 *   1024-cell grid over [-1, 1]; FA_TQ_EUNSUPPORTED otherwise; every Lloyd-Max table
 *   for head_dim <= 192 qualifies); rotation: device, R as written by
 *   fa_tq_rotation_dense (fp32 row-major, 16-byte aligned, owned by the caller).
 *   head_dim in [4, 192] (FA_TQ_EUNSUPPORTED outside).  x: device, element
 *   (b, h, t, c) at b*stride_b + h*stride_h + t*stride_t + c (non-negative strides),
 *   aligned to its element size (16-byte aligned rows with head_dim % 8 == 0 take the
 *   fast path).  t0 / t_max / codes / norms as fa_tq_encode, except that positions
 *   outside [0, t_max) are skipped (no ring).  At most 2^31 - 1 vectors per call
 *   (FA_TQ_EUNSUPPORTED otherwise).
 * The product R x runs on fp16 matrix instructions with R split into two fp16 halves
 * (about 22 significant bits; an fp32 input is split the same way) and fp32
 * accumulation, so a code next to a decision boundary can differ from an exact
 * evaluation by one level.
 */
fa_tq_status fa_tq_encode_dense(const fa_tq_codebook *cb, const float *rotation,
                                int32_t head_dim, const void *x, fa_tq_dtype x_dtype,
                                fa_tq_layout x_layout, int32_t batch, int32_t n_kv_heads,
                                int32_t n_tokens, const int32_t *t0, int32_t t_max,
                                uint8_t *codes, uint16_t *norms, void *stream);

/*
 * Decode of a dense-rotation cache: x_hat = n16 * (R^T c[code]) over the head_dim
 * codes of each vector (R and the centroids split into two fp16 halves each, fp32
 * accumulation: about 2^-21 relative), tokens t < n_tokens of every row written to
 * out at (b, h, t, c) as fp32 or bf16 (round to nearest even); out aligned to its
 * element size, non-negative strides.  n_tokens <= t_max; at most 2^31 - 1 vectors
 * per call (FA_TQ_EUNSUPPORTED otherwise).
 */
fa_tq_status fa_tq_decode_dense(const fa_tq_codebook *cb, const float *rotation,
                                int32_t head_dim, const uint8_t *codes, const uint16_t *norms,
                                int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                                int32_t t_max, void *out, fa_tq_dtype out_dtype,
                                fa_tq_layout out_layout, void *stream);

/*
 * Single-query decode attention over a dense-rotation cache written by
 * fa_tq_encode_dense ([Spec] "Optimization: Fused dequant-dot" with the dense R of
 * "Hadamard Transform Detail"): per (b, query head h), g = h / (n_q_heads / n_kv_heads):
 *   q' = R q;  s_t = scale * n_K[t] * <q', c_K[code_K[t]]>  for t < seq_lens[b];
 *   p = softmax(s);  o' = sum_t p_t n_V[t] c_V[code_V[t]];  out = R^T o'.
 * The coordinates past head_dim (code 0 in the cache) do not enter: q' is zero there and
 * out takes the first head_dim coordinates of o'.  The attention kernels run in their
 * own Walsh-Hadamard frame R_w: a small kernel maps the query in as R_w^-1 (R q); the
 * MFMA kernels' merge then writes R^T o' directly, the vector-ALU kernels' result y
 * leaves through a second small kernel as R^T (R_w y).  Accuracy is that of
 * fa_tq_attn_decode_ex.
 *   cb_k, cb_v: 2-4 bit codebooks of dim head_dim; rotation: as fa_tq_encode_dense;
 *   head_dim in [4, 128] (FA_TQ_EUNSUPPORTED above: the cache then has more than one
 *   128-element block per vector).  q: device [batch][n_q_heads][head_dim] of q_dtype
 *   (bf16 or fp32); k/v codes: [batch][n_kv_heads][t_max][1][code bytes]; norms:
 *   [batch][n_kv_heads][t_max] (one per vector); seq_lens: device [batch] int32,
 *   clamped to [0, t_max]; out: device fp32 [batch][n_q_heads][head_dim].
 *   flags: 0 or FA_TQ_ATTN_VECTOR_ALU.  workspace: device, 16-byte aligned, at least
 *   fa_tq_attn_dense_workspace_bytes(...) bytes, contents on entry do not matter.
 *   Errors as fa_tq_attn_decode_ex.
 */
size_t fa_tq_attn_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t t_max);
fa_tq_status fa_tq_attn_decode_dense(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                                     const float *rotation, int32_t head_dim, uint32_t flags,
                                     const void *q, fa_tq_dtype q_dtype,
                                     const uint8_t *k_codes, const uint16_t *k_norms,
                                     const uint8_t *v_codes, const uint16_t *v_norms,
                                     const int32_t *seq_lens, int32_t batch, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t t_max, float scale, float *out,
                                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * Single-query decode attention over the packed cache ([Spec] "Optimization: Fused
 * dequant-dot"): per (b, query head h), with g = h / (n_q_heads / n_kv_heads):
 *   q' = R q;  s_t = scale * n_K[t] * <q', c_K[code_K[t]]>  for t < seq_lens[b];
 *   p = softmax(s);  o' = sum_t p_t n_V[t] c_V[code_V[t]];  out = R^T o'.
 * seq_lens[b] == 0 gives zeros.  Accumulation in fp32.
 *   q: device [batch][n_q_heads][head_dim] of q_dtype.
 *   k_codes/k_norms/v_codes/v_norms: device, SoA layout above.
 *   seq_lens: device int32[batch], each in [0, t_max] (larger values are clamped).
 *   out: device float [batch][n_q_heads][head_dim].
 *   workspace: device, >= fa_tq_attn_workspace_bytes(...), 16-byte aligned.  It
 *   holds per-split partial results (m, l and the unnormalized rotated output per
 *   split of the sequence); its contents on entry do not matter.  Calls that run
 *   concurrently must not share a workspace; calls in order on one stream may.
 * The library supports head_dim == 128, key/value bits in {2, 3, 4}, any group size
 * n_q_heads / n_kv_heads (the matrix-core kernels take up to 8 query heads per
 * workgroup: a larger group of G heads is split over the smallest r dividing G with
 * G / r <= 8 workgroups per KV head, each reading that KV head's codes, e.g. r = 2
 * for G = 16 and 4 for G = 32; the vector-ALU kernels take G <= 16), and
 * t_max < 33554432 (one cache row below 2 GiB).
 */
fa_tq_status fa_tq_attn_decode(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                               uint64_t seed, int32_t head_dim,
                               const void *q, fa_tq_dtype q_dtype,
                               const uint8_t *k_codes, const uint16_t *k_norms,
                               const uint8_t *v_codes, const uint16_t *v_norms,
                               const int32_t *seq_lens, int32_t batch,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t t_max,
                               float scale, float *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* fa_tq_attn_decode with flags: FA_TQ_TWO_SIGNS (the cache's rotation) and/or
 * FA_TQ_ATTN_VECTOR_ALU (the kernel family). */
fa_tq_status fa_tq_attn_decode_ex(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                                  uint64_t seed, uint32_t flags, int32_t head_dim,
                                  const void *q, fa_tq_dtype q_dtype,
                                  const uint8_t *k_codes, const uint16_t *k_norms,
                                  const uint8_t *v_codes, const uint16_t *v_norms,
                                  const int32_t *seq_lens, int32_t batch, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t t_max, float scale, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the per-GPU scratch array of fa_tq_attn_decode_noalloc (8 MiB). */
#define FA_TQ_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * fa_tq_attn_decode_ex without the workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus workspace and
 * workspace_bytes), same kernels and results as fa_tq_attn_decode_ex; the per-split
 * partial results go to a scratch array of FA_TQ_NOALLOC_SCRATCH_BYTES bytes that
 * the library holds in the memory of each GPU it runs on until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Sizes whose partials (fa_tq_attn_workspace_bytes) exceed the array are rejected
 *   with FA_TQ_EUNSUPPORTED, before anything is launched.
 *   The array of the current device is used; its device address is looked up once
 *   per device, on the first call on that device (make that first call outside
 *   graph capture).
 *   Every call on one GPU shares its array, which keeps the last call's contents:
 *   calls that can overlap on one GPU (several streams or host threads) race and
 *   give wrong results; calls in order on one stream are safe.
 */
fa_tq_status fa_tq_attn_decode_noalloc(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                                       uint64_t seed, uint32_t flags, int32_t head_dim,
                                       const void *q, fa_tq_dtype q_dtype,
                                       const uint8_t *k_codes, const uint16_t *k_norms,
                                       const uint8_t *v_codes, const uint16_t *v_norms,
                                       const int32_t *seq_lens, int32_t batch,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t t_max,
                                       float scale, float *out, void *stream);

/*
 * Append, then attend ([Spec] "Attention with TurboQuant cache": the cached-attention
 * call quantizes the current K and V into the cache, then attends with the full-
 * precision query; [Spec] "Integration Points": circular addressing, cache position
 * = pos % max_seq).  In one call, on `stream`:
 *   1. encode k_new[b][h][i][:] and v_new[b][h][i][:] (i < n_new) as fa_tq_encode
 *      does, into cache slot (pos[b] + i) % t_max of sequence b;
 *   2. decode attention as fa_tq_attn_decode with seq_lens[b] = min(pos[b] + n_new,
 *      t_max): every filled slot (a full ring holds the last t_max tokens; the
 *      result does not depend on slot order).
 *   q, out, workspace: as for fa_tq_attn_decode; k_new, v_new: device, kv_dtype, with
 *      the element strides of k_layout / v_layout (channel stride 1), 16-byte aligned.
 *   pos: device int32[batch], positions >= 0 (a negative position stores nothing and
 *      clamps the attended length at 0).
 *   codebooks: bits 2, 3 or 4 for keys and values; head_dim 128.
 *   1 <= n_new <= t_max (two new tokens never share a slot); every argument is
 *   checked before anything is written to the cache.
 */
fa_tq_status fa_tq_attn_append(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                               uint64_t seed, int32_t head_dim,
                               const void *q, fa_tq_dtype q_dtype,
                               const void *k_new, const void *v_new, fa_tq_dtype kv_dtype,
                               fa_tq_layout k_layout, fa_tq_layout v_layout,
                               int32_t n_new, const int32_t *pos,
                               uint8_t *k_codes, uint16_t *k_norms,
                               uint8_t *v_codes, uint16_t *v_norms,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t t_max, float scale, float *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* fa_tq_attn_append with variant flags: FA_TQ_TWO_SIGNS (encode and attention) and
 * FA_TQ_NORM_CORRECT (the new tokens' stored norms). */
fa_tq_status fa_tq_attn_append_ex(const fa_tq_codebook *cb_k, const fa_tq_codebook *cb_v,
                                  uint64_t seed, uint32_t flags, int32_t head_dim,
                                  const void *q, fa_tq_dtype q_dtype,
                                  const void *k_new, const void *v_new, fa_tq_dtype kv_dtype,
                                  fa_tq_layout k_layout, fa_tq_layout v_layout,
                                  int32_t n_new, const int32_t *pos,
                                  uint8_t *k_codes, uint16_t *k_norms,
                                  uint8_t *v_codes, uint16_t *v_norms,
                                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t t_max, float scale, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_TQ_H */

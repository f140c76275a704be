// Internal declarations shared by the host front-end and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "fa_tq.h"

namespace fatq {

constexpr int QK = FA_TQ_QK;
constexpr int MAX_BLK = FA_TQ_MAX_HEAD_DIM / FA_TQ_QK;

// Sign diagonal as bit masks in the quad layout used by the block kernels: four
// lanes own one 128-block, lane q holding chunks q, q+4, q+8, q+12 of 8 elements,
// so element e = 8 (q + 4 k) + i.  Bit (8 k + i) of w[j][q] is set when the sign
// of element 128 j + e is -1.
struct SignWords {
  uint32_t w[MAX_BLK][4];
  // The second sign vector s2 of the two-sign rotation R = D2 H D1 / sqrt(128)
  // ([turboq] "Encode pipeline" step 2), same layout; two == 0: s2 = all +1.
  uint32_t w2[MAX_BLK][4];
  int32_t two;
};

// Codebook as the kernels read it (uniform kernel arguments).  For the 2-4 bit
// codebooks the host also derives what the encoder's cell table needs: the biased
// exponent range [emin, emax] of the nonzero boundaries, and the entries of the
// cells outside that range, which hold no boundary: (threshold, base, c[base]^2,
// c[base + 1]^2) as fp32 bits for positive cells below the range, negative cells
// below it, positive cells above it, negative cells above it, and the cell of +0.
struct KTable {
  float b[15];   // boundaries (nb used, +inf after them)
  float c[16];   // centroids
  int32_t nb;    // levels - 1
  int32_t bits;
  uint32_t emin, emax;
  uint32_t cell_out[5][4];
};

// fp32 nearest to 1/sqrt(128) (the scale of [Spec] Step 1), and the 8-bit grid
// constant fp32(kInvSqrtQK * 127.5).
constexpr float kInvSqrtQK = static_cast<float>(0.08838834764831845);
constexpr float kGrid8 = kInvSqrtQK * 127.5f;

struct EncodeLaunch {
  const void* x;
  int64_t sb, sh, st;   // element strides
  int32_t batch, heads, tokens, nblk, t_max;
  const int32_t* t0;     // first cache position per sequence, or null (0)
  int32_t ring;          // positions map to slots modulo t_max (append into a ring)
  uint8_t* codes;
  uint16_t* norms;
  int32_t x_is_bf16;
  int32_t t_step;        // token stride of one quad (set by the launcher from its grid)
  int32_t dim;           // input elements per vector (head_dim); below QK * nblk, the
                         // rest of the transform's input is zero padding
};

// norm_correct: store n / ||c[codes]|| ([turboq] "Encode pipeline" step 4; bits 2-4).
// whole: whole-vector mode ([Spec] "Step 1": one rotation over the transform length
// QK * nblk = 128 or 256, one norm per vector, norms[rows][t_max]; codes as the
// blocked layout).  dim < QK * nblk (whole mode only): the vector is zero-padded to
// the transform length ([Spec] "Hadamard Transform Detail").
hipError_t launch_encode(const EncodeLaunch& a, const KTable& tab, const SignWords& sw,
                         bool norm_correct, bool whole, hipStream_t stream);
// The keys and the values of one append (same shape, 2-4 bit tables, blocked mode) in
// one launch.
hipError_t launch_encode_pair(const EncodeLaunch& ak, const KTable& tk, const EncodeLaunch& av,
                              const KTable& tv, const SignWords& sw, bool norm_correct,
                              bool append, hipStream_t stream);
// Decode of tokens [0, tokens) of `rows` cache rows of t_max slots each (row =
// b * heads + h) into out[b][h][t][:] at element strides (sb, sh, st).
struct DecodeLaunch {
  const uint8_t* codes;
  const uint16_t* norms;
  int64_t rows, tokens, t_max;
  int32_t heads, nblk;
  void* out;
  int64_t sb, sh, st;
  int32_t out_bf16;
  int32_t dim;   // output elements per vector; below QK * nblk (whole mode only) the
                 // transform's last outputs are the padding, not stored
};

hipError_t launch_decode(const DecodeLaunch& d, const KTable& tab, const SignWords& sw,
                         bool whole, hipStream_t stream);

// Dense random orthogonal rotation ([Spec] "Hadamard Transform Detail", the option for
// head_dims that are not a power of two): encode and decode with a d x d fp32 matrix R
// (row-major, device memory), d <= kDenseMax; codes of the d coordinates in
// nblk = ceil(d / 128) blocks (code 0 past d), one fp16 norm per vector.
constexpr int kDenseMax = 192;
// cells of the dense encoder's bucketize grid over [-1, 1] (see dense_grid_cell)
constexpr int kDenseGrid = 1024;

struct DenseLaunch {
  const void* x;
  int64_t sb, sh, st;   // element strides
  int32_t batch, heads, tokens, t_max, dim, nblk;
  const int32_t* t0;    // first cache position per sequence, or null (0)
  const float* rot;
  uint8_t* codes;
  uint16_t* norms;      // [rows][t_max]
  int32_t x_is_bf16;
  int32_t vec;          // x 16-byte aligned, strides of 16 bytes, d % 8 == 0: 16-byte loads
};

struct DenseDecodeLaunch {
  const uint8_t* codes;
  const uint16_t* norms;
  const float* rot;
  int64_t rows, tokens, t_max;
  int32_t heads, dim, nblk;
  void* out;
  int64_t sb, sh, st;
  int32_t out_bf16;
  int32_t vec;          // out 16-byte aligned, strides multiples of 4 elements: 8/16-byte stores
};

// Attention over a dense-rotation cache (head_dim <= 128) runs the attention kernels in
// their own Walsh-Hadamard frame R_w = c H D (D = diag(signs), c = fp32(1/sqrt(128))):
// the query enters as q~ = R_w^-1 (R q) and the result y leaves as R^T (R_w y).
constexpr int kDenseAttnMax = QK;

struct DenseAttnLaunch {
  const void* q;        // [batch][hq][dim], bf16 or fp32
  int32_t q_is_bf16;
  const float* rot;     // R, [dim][dim] row-major
  int32_t batch, hq, dim;
  float* qt;            // q~, [batch][hq][128] fp32
  const float* y;       // attention result in the frame, [batch][hq][128] fp32
  float* out;           // [batch][hq][dim] fp32
  uint32_t signs[4];    // bit i % 32 of word i / 32: element i of D is -1
};

hipError_t launch_dense_attn_query(const DenseAttnLaunch& a, hipStream_t stream);
hipError_t launch_dense_attn_out(const DenseAttnLaunch& a, hipStream_t stream);

hipError_t launch_dense_encode(const DenseLaunch& a, const KTable& tab, hipStream_t stream);
hipError_t launch_dense_decode(const DenseDecodeLaunch& a, const KTable& tab,
                               hipStream_t stream);

struct AttnLaunch {
  const void* q;
  int32_t q_is_bf16;
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  const int32_t* seq_lens;   // tokens per sequence, or (when pos is set)
  const int32_t* pos;        //   min(pos[b] + n_new, t_max)
  int32_t n_new;
  const int32_t* lens;       // set by the launchers: pos ? pos : seq_lens,
  int32_t len_add;           //   and pos ? n_new : 0 (one load per sequence)
  int32_t batch, hq, hkv, t_max;
  float scale;
  float* out;
  void* workspace;
  int32_t n_split, chunk;
  // MFMA family only: workgroups per KV head, each taking hq / (hkv * kv_div) query heads
  int32_t kv_div = 1;
  // MFMA family only: when set, the merge writes out[b][h][0 .. dense_dim) = R^T o with
  // R = dense_rot (row-major dense_dim x dense_dim) in place of the inverse rotation
  // (attention over a dense-rotation cache)
  const float* dense_rot = nullptr;
  int32_t dense_dim = 0;
};

// Split-KV partitioning used by both the workspace query and the launch.
void attn_partition(int32_t batch, int32_t hkv, int32_t t_max, int32_t* n_split,
                    int32_t* chunk);
size_t attn_workspace_bytes(int32_t batch, int32_t hq, int32_t n_split);

hipError_t launch_attn(const AttnLaunch& a, const KTable& tk, const KTable& tv,
                       const SignWords& sw, hipStream_t stream);

// MFMA path: up to 8 query heads per workgroup; a larger group of a KV head is split
// over attn_mfma_groups(hq, hkv) workgroups (the partition then counts hkv times that).
int32_t attn_mfma_groups(int32_t hq, int32_t hkv);
void attn_mfma_partition(int32_t batch, int32_t hkv, int32_t t_max, int32_t* n_split,
                         int32_t* chunk);
size_t attn_mfma_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t n_split);
hipError_t launch_attn_mfma(const AttnLaunch& a, const KTable& tk, const KTable& tv,
                            const SignWords& sw, hipStream_t stream);

}  // namespace fatq

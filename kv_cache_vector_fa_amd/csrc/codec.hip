// Encode and decode kernels for gfx950 (compiled with -ffp-contract=off: the
// encoder's fp32 operation order defines the code and norm bits).
//
// Pages cited: [Spec] "TurboQuant KV Cache Compression -- Spec";
//              [turboq] "TurboQuant KV Cache (turboq2 / turboq3 / turboq4)".
//
// Work layout ("quad"): four consecutive lanes own one 128-element block.  Lane
// q = lane & 3 holds the 8-element chunks c = q, q+4, q+8, q+12, i.e. element
// e = 8 (q + 4 k) + i lives in register v[k][i].  Index bits 0-2 of e are in-lane
// (i), bits 3-4 are the lane bits (q), bits 5-6 are in-lane (k).  With this map
// a bf16 block is read as four 16-byte loads per lane, every 4-lane group reading
// 64 contiguous bytes, and the butterfly stages 1, 2, 4, 32, 64 of [Spec] "Hadamard
// Transform Detail" are in-lane while stages 8 and 16 exchange with lane q^1, q^2.

#include <hip/hip_fp16.h>

#include <type_traits>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

constexpr int kThreads = 256;
#ifndef FATQ_ENCODE_THREADS
#define FATQ_ENCODE_THREADS 256
#endif
constexpr int kEncThreads = FATQ_ENCODE_THREADS;

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float flip_sign(float x, uint32_t bit) {
  return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

// Keeps x as a materialized fp32 value: stops the compiler from fusing the fp32
// rounding of a product into a following conversion (e.g. one fp16 rounding of
// a*b instead of rounding to fp32 first, which the canonical arithmetic requires).
__device__ __forceinline__ float fp32_value(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void bfly(float& a, float& b) {
  const float u = a, v = b;
  a = u + v;
  b = u - v;
}

template <int BITS>
constexpr int code_bytes_of() {
  return BITS == 2 ? 32 : BITS == 3 ? 48 : BITS == 4 ? 64 : 128;
}

// ---------------------------------------------------------------------------
// Bucketize by cell table.  A cell is the set of fp32 values sharing the top 11
// bits (sign, exponent, two leading mantissa bits), so cell index = bits >> 21 and
// cells are contiguous intervals.  Adjacent Lloyd-Max boundaries of the 2-4 bit
// tables are more than 1.25x apart (the host checks that no two boundaries share a
// cell), so a cell contains at most one boundary and
//     code(u) = base[cell] + (u > thr[cell]),
// with base = #{j : b_j < smallest value of the cell} and thr = b[base] (+inf when
// base = L - 1).  One 8-byte LDS read and one compare per coordinate reproduce
// code = #{j : b_j < u} exactly, ties included ([Spec] "Step 2": the boundaries
// are the decision thresholds).
constexpr int kCellShift = 21;
constexpr uint32_t kCells = 1u << (32 - kCellShift);   // 2048 cells, 16 KB of LDS
constexpr uint32_t kNegCell = kCells / 2;

// Workgroup barrier ordering LDS only: unlike __syncthreads() it does not wait for
// outstanding global loads, so a prefetch issued before it stays in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Entry of cell c: (threshold, base) or, for the corrected norm, (threshold, base,
// c[base]^2, c[base + 1]^2) so that the chosen code's squared centroid comes with the
// compare.
__device__ __forceinline__ void set_cell(uint2* cells, uint32_t c, uint4 e) {
  cells[c] = make_uint2(e.x, e.y);
}
__device__ __forceinline__ void set_cell(uint4* cells, uint32_t c, uint4 e) { cells[c] = e; }

// Fill the 2048 cells.  Cells whose exponent lies outside [emin, emax] (the nonzero
// boundaries' range) hold no boundary and take one of four host-made entries by
// sign and side; the few inside it, and the +0 cell, count the boundaries below
// their smallest member.  Everything read from the codebook is uniform, so it
// arrives in one batch of scalar loads.
template <typename Cell>
__device__ __forceinline__ void fill_cells(Cell* cells, const KTable& t) {
  float b[15], c[16];
#pragma unroll
  for (int m = 0; m < 15; ++m) b[m] = t.b[m];   // +inf past the last boundary
#pragma unroll
  for (int m = 0; m < 16; ++m) c[m] = t.c[m];
  const uint32_t emin = t.emin, emax = t.emax;
  auto out = [&](int k) {
    return make_uint4(t.cell_out[k][0], t.cell_out[k][1], t.cell_out[k][2], t.cell_out[k][3]);
  };
  const uint4 below_pos = out(0), below_neg = out(1), above_pos = out(2), above_neg = out(3);
  for (uint32_t cc = threadIdx.x; cc < kCells; cc += blockDim.x) {
    const uint32_t e = (cc >> 2) & 0xFFu;
    const bool neg = cc >= kNegCell;
    uint4 ent;
    if ((e >= emin && e <= emax) || cc == 0) {
      const uint32_t lo = cc << kCellShift;
      const float umin = __uint_as_float(neg ? (lo | ((1u << kCellShift) - 1u)) : lo);
      // boundaries ascend: the last one below umin fixes base, threshold and centroids
      uint32_t base = 0;
      float thr = b[0], c0 = c[0], c1 = c[1];
#pragma unroll
      for (int m = 0; m < 15; ++m) {
        const bool below = b[m] < umin;
        base += below ? 1u : 0u;
        thr = below ? (m + 1 < 15 ? b[m + 1] : INFINITY) : thr;
        c0 = below ? c[m + 1] : c0;
        c1 = below ? c[m + 2 < 16 ? m + 2 : 15] : c1;
      }
      ent = make_uint4(__float_as_uint(thr), base, __float_as_uint(c0 * c0),
                       __float_as_uint(c1 * c1));
    } else {
      const uint4 lo = neg ? below_neg : below_pos, hi = neg ? above_neg : above_pos;
      ent = e < emin ? lo : hi;
    }
    set_cell(cells, cc, ent);
  }
}

// Codes of 8 coordinates y[0..7] (u_i = y_i * g) as LSB-first fields of width W
// (Horner from the last coordinate, so y[0] lands in the lowest field).
template <int W>
__device__ __forceinline__ uint32_t bucketize8(const float (&y)[8], float g,
                                               const uint2* cells) {
  uint32_t acc = 0;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    const float u = y[i] * g;
    const uint32_t off = (__float_as_uint(u) >> (kCellShift - 3)) & ((kCells - 1u) << 3);
    const uint2 cell = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(cells) + off);
    acc = (acc << W) + cell.y + (u > __uint_as_float(cell.x) ? 1u : 0u);
  }
  return acc;
}

// As bucketize8, also returning the canonical fp32 sum of c[code_i]^2 over the 8
// coordinates (pairwise: index bit 0, then 1, then 2).
template <int W>
__device__ __forceinline__ uint32_t bucketize8_sq(const float (&y)[8], float g,
                                                  const uint4* cells, float& sq) {
  uint32_t acc = 0;
  float c2[8];
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    const float u = y[i] * g;
    const uint32_t off = (__float_as_uint(u) >> (kCellShift - 4)) & ((kCells - 1u) << 4);
    const uint4 cell = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(cells) + off);
    const bool up = u > __uint_as_float(cell.x);
    acc = (acc << W) + cell.y + (up ? 1u : 0u);
    c2[i] = __uint_as_float(up ? cell.w : cell.z);
  }
  sq = ((c2[0] + c2[1]) + (c2[2] + c2[3])) + ((c2[4] + c2[5]) + (c2[6] + c2[7]));
  return acc;
}

// Mirror masks of the second sign vector: with a mirror-symmetric codebook,
// code(-u) = L - 1 - code(u) (up to u exactly on a boundary), so the sign change of
// coordinate i becomes an XOR of its code field with L - 1.  Field width W, 8
// coordinates of chunk byte `bits8` (bit i: coordinate i is negated).
template <int W>
__device__ __forceinline__ uint32_t mirror_mask(uint32_t bits8, uint32_t fieldmask) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m |= ((bits8 >> i) & 1u) * (fieldmask << (W * i));
  return m;
}

// Cross-lane butterfly stage on one 8-element chunk: v <- v + mu * v(partner), the
// partner chosen by the DPP quad permutation.  With mu = +1 in the lower lane of the
// pair and -1 in the upper one this is (a + b, -(a - b)): the upper lane keeps the
// negated difference, and the sign is tracked by the caller.  fma(x, +-1, y) rounds
// exactly like y +- x.  The s_nop pairs cover the 2-wait-state hazard of a DPP read
// of a VGPR written by the preceding VALU instruction (before the block) and of a
// DPP instruction after it reading these results.
template <int CTRL>
__device__ __forceinline__ void xstage(float (&v)[8], float mu) {
  static_assert(CTRL == 0xB1 || CTRL == 0x4E, "quad permutation");
  if constexpr (CTRL == 0xB1) {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
          "+v"(v[6]), "+v"(v[7])
        : "v"(mu));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1"
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
          "+v"(v[6]), "+v"(v[7])
        : "v"(mu));
  }
}

// Add the value of lane q ^ 1 (CTRL 0xB1) or q ^ 2 (0x4E) within the quad.
template <int CTRL>
__device__ __forceinline__ float quad_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float quad_max(float x) {
  return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false)));
}

// Whole-vector mode, head_dim 256: the butterfly stage between the vector's two
// 128-blocks.  Their quads are adjacent and the second holds its chunks in reversed
// lane order, so lane i and lane 7 - i of a half row hold the same chunk of the two
// blocks: row_half_mirror is the partner.  v <- v + mu * v(partner) as in xstage.
__device__ __forceinline__ void xstage_mirror(float (&v)[8], float mu) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),
        "+v"(v[6]), "+v"(v[7])
      : "v"(mu));
}
__device__ __forceinline__ float mirror_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
}

// One block's input in the quad layout: raw words (bf16: 4 x 16 B per lane; fp32:
// 8 x 16 B per lane).
template <bool BF16>
struct RawBlock {
  uint4 w[BF16 ? 4 : 8];
};

// Raw buffer resources (per-row base, byte range).  An access whose offset is at or
// beyond the range is dropped by the hardware (stores) or returns zeros (loads), so
// lanes without work use offset kOOB instead of a branch: with no divergent control
// flow around memory operations the compiler can wait for exactly the loads it needs.
constexpr int32_t kRsrcWord3 = 0x00020000;   // raw dword-format buffer on gfx9
constexpr uint32_t kOOB = 0x80000000u;        // every range is below 2^31 (host check)
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRsrcWord3);
}

// One block's input in the quad layout from byte offset `off` of resource r.
// dead[k] is 0, or kOOB for a chunk that lies in the zero padding of a vector: or-ed
// into its offset (every in-range offset is below 2^31) it makes the load return
// zeros without reading past the vector.
template <bool BF16>
__device__ __forceinline__ void load_raw(Rsrc r, uint32_t off, int q, const uint32_t (&dead)[4],
                                         RawBlock<BF16>& b) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      b.w[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                             r, (off + 16 * (q + 4 * k)) | dead[k], 0, 0));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t o = (off + 32 * (q + 4 * k)) | dead[k];
      b.w[2 * k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
      b.w[2 * k + 1] =
          __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, 0));
    }
  }
}

// Stores of one encoded block (same count and kinds as the encoder's), all to
// offset kOOB, so they are dropped.
template <int BITS>
__device__ __forceinline__ void dummy_stores(Rsrc rc, Rsrc rn) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t o = kOOB + 64 * k;   // distinct offsets: no store is merged away
    if constexpr (BITS == 8) {
      __builtin_amdgcn_raw_buffer_store_b32(0u, rc, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(0u, rc, o + 4, 0, 0);
    } else if constexpr (BITS == 4) {
      __builtin_amdgcn_raw_buffer_store_b32(0u, rc, o, 0, 0);
    } else if constexpr (BITS == 2) {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), rc, o, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), rc, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(0), rc, o + 32, 0, 0);
    }
  }
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), rn, kOOB, 0, 0);
}

// Sign-flip (s * x) and widen to fp32; also return the canonical sum of squares of
// this lane's 4 chunks (levels 0-2 of the pairwise tree, index bits 0-2): each square
// rounded to fp32, then added.
// smask[k][m]: bit 15 / bit 31 flip the low / high bf16 of word m of chunk k.
template <bool BF16>
__device__ __forceinline__ void widen(const RawBlock<BF16>& r, const uint32_t (&smask)[16],
                                      uint32_t sbits, float (&x)[4][8], float (&p)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float s[4];
    if constexpr (BF16) {
      const uint32_t d[4] = {r.w[k].x, r.w[k].y, r.w[k].z, r.w[k].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t f = d[m] ^ smask[4 * k + m];
        const float lo = __uint_as_float(f << 16), hi = __uint_as_float(f & 0xffff0000u);
        x[k][2 * m] = lo;
        x[k][2 * m + 1] = hi;
        // a bf16 square is exact in fp32 (for |x| >= 2^-63), so one fma is
        // RN32(RN32(lo^2) + RN32(hi^2))
        s[m] = __builtin_fmaf(hi, hi, lo * lo);
      }
    } else {
      const uint4 a = r.w[2 * k], b = r.w[2 * k + 1];
      const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        x[k][i] = __uint_as_float(d[i] ^ (((sbits >> (8 * k + i)) & 1u) << 31));
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float a0 = x[k][2 * m] * x[k][2 * m], a1 = x[k][2 * m + 1] * x[k][2 * m + 1];
        s[m] = a0 + a1;
      }
    }
    p[k] = (s[0] + s[1]) + (s[2] + s[3]);
  }
}

// Encode: one quad per 128-block.  Grid (gx, gy): blockIdx.y strides over the
// (batch, head) rows, and quad f of the x-grid over the rows' (token, block)
// pairs; the x-stride is a multiple of nblk, so a quad keeps one block index j
// (one sign slice) for the whole kernel.  The next block's input is loaded while
// the current one is processed.
// WV: whole-vector mode for head_dim 256 ([Spec] "Step 1", one 256-point transform;
// nblk = 2): the two quads of a vector also run the last butterfly stage between
// them, share one norm (and store it once) and scale by RN32(1/16).
// PAD: a.dim < QK * nblk; the chunks at or past a.dim load as zeros.
template <int BITS, bool BF16, bool NC, bool WV, bool PAD>
__device__ __forceinline__ void encode_body(const EncodeLaunch& a, const KTable& tab,
                                            const SignWords& sw) {
  static_assert(!WV || (BITS != 8 && !NC), "whole-vector mode: 2-4 bit codebooks");
  static_assert(!PAD || (BITS != 8 && !NC), "padding: whole-vector mode only");
  constexpr int CB = code_bytes_of<BITS>();
  typedef typename std::conditional<NC, uint4, uint2>::type Cell;
  __shared__ Cell cells[BITS == 8 ? 1 : kCells];
  const uint32_t f0 = blockIdx.x * (kEncThreads / 4) + (threadIdx.x >> 2);
  const uint32_t nblk = static_cast<uint32_t>(a.nblk);
  const int j = static_cast<int>(f0 % nblk);
  // chunk index of the lane (reversed in a whole vector's second quad, see xstage_mirror)
  const int q = WV && (j & 1) ? 3 - static_cast<int>(threadIdx.x & 3) : threadIdx.x & 3;
  const int t_first = static_cast<int>(f0 / nblk);
  const int t_step = a.t_step;   // gridDim.x * quads per workgroup / nblk
  const int rows = a.batch * a.heads;
  constexpr uint32_t ES = BF16 ? 2 : 4;   // input element bytes
  const uint32_t xbytes = static_cast<uint32_t>(((a.tokens - 1) * a.st + a.dim) * ES);
  const uint32_t cbytes = static_cast<uint32_t>(a.t_max) * a.nblk * CB;
  const uint32_t nbytes = static_cast<uint32_t>(a.t_max) * a.nblk * 2;
  struct Row {
    Rsrc rx, rc, rn;
    int tbase;
  };
  auto open_row = [&](int row) {
    const int b = row / a.heads;
    const int h = row - b * a.heads;
    Row r;
    r.tbase = a.t0 ? a.t0[b] : 0;
    r.rx = make_rsrc(static_cast<const char*>(a.x) + (b * a.sb + h * a.sh) * ES, xbytes);
    const int64_t crow = static_cast<int64_t>(row) * a.t_max * a.nblk;
    r.rc = make_rsrc(a.codes + crow * CB, cbytes);
    // one norm per block, or per vector in the whole-vector mode
    r.rn = WV ? make_rsrc(a.norms + static_cast<int64_t>(row) * a.t_max, nbytes / 2)
              : make_rsrc(a.norms + crow, nbytes);
    return r;
  };
  // byte offset of block (t, j) in the input row; kOOB past the last token
  auto xoff = [&](int t) {
    return t < a.tokens ? static_cast<uint32_t>((t * a.st + QK * j) * ES) : kOOB;
  };

  // The per-lane sign words (kernel arguments read through vector loads) and the
  // first block's input go out before the cell table is filled; nothing waits for
  // them until the fill is done.
  int row = blockIdx.y;
  if (row >= rows) return;   // uniform over the workgroup
  const uint32_t sbits = sw.w[j][q];
  const uint32_t s2bits = sw.two ? sw.w2[j][q] : 0u;
  uint32_t dead[4] = {0u, 0u, 0u, 0u};
  if constexpr (PAD) {
#pragma unroll
    for (int k = 0; k < 4; ++k) dead[k] = QK * j + 8 * (q + 4 * k) >= a.dim ? kOOB : 0u;
  }
  Row R = open_row(row);
  int t = t_first;
  RawBlock<BF16> ba, bb;
  load_raw<BF16>(R.rx, xoff(t), q, dead, ba);
  if constexpr (BITS != 8) {
    fill_cells(cells, tab);
    lds_barrier();
  }

  uint32_t smask[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    smask[i] = (((sbits >> (2 * i)) & 1u) << 15) | (((sbits >> (2 * i + 1)) & 1u) << 31);
  // mu of the two cross-lane stages, and the sign the lane's results carry after them
  const float mu1 = (q & 1) ? -1.0f : 1.0f;
  const float mu2 = (q & 2) ? -1.0f : 1.0f;
  const uint32_t carried = (((q ^ (q >> 1)) & 1u) ^ (WV ? (j & 1) : 0)) << 31;
  const float mu3 = (j & 1) ? -1.0f : 1.0f;   // the stage between the two blocks (WV)
  constexpr float c_scale = WV ? 0.0625f : kInvSqrtQK;   // RN32(1/sqrt(d))
  // second sign vector: code mirror masks per chunk (zero without it)
  uint32_t mirror[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t b8 = (s2bits >> (8 * k)) & 0xFFu;
    mirror[k] = BITS == 2 ? mirror_mask<2>(b8, 3u) : BITS == 3 ? mirror_mask<4>(b8, 7u)
                                                              : mirror_mask<4>(b8, 15u);
  }


  auto process = [&](const RawBlock<BF16>& cur, int t) {
    float x[4][8], p[4];
    widen<BF16>(cur, smask, sbits, x, p);
    // canonical norm: levels 3-4 across the quad, 5-6 across chunks
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = quad_add<0xB1>(p[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k) p[k] = quad_add<0x4E>(p[k]);
    float ss = (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (WV) ss = mirror_add(ss);   // level 7: the vector's two blocks
    const float n32 = __builtin_sqrtf(ss);
    // Walsh-Hadamard butterflies, stages 1, 2, 4 (in-chunk), 8, 16 (across the
    // quad), 32, 64 (across chunks), and 128 across the two quads of a whole vector
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bfly(x[k][0], x[k][1]); bfly(x[k][2], x[k][3]);
      bfly(x[k][4], x[k][5]); bfly(x[k][6], x[k][7]);
      bfly(x[k][0], x[k][2]); bfly(x[k][1], x[k][3]);
      bfly(x[k][4], x[k][6]); bfly(x[k][5], x[k][7]);
      bfly(x[k][0], x[k][4]); bfly(x[k][1], x[k][5]);
      bfly(x[k][2], x[k][6]); bfly(x[k][3], x[k][7]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) xstage<0xB1>(x[k], mu1);
#pragma unroll
    for (int k = 0; k < 4; ++k) xstage<0x4E>(x[k], mu2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bfly(x[0][i], x[1][i]);
      bfly(x[2][i], x[3][i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bfly(x[0][i], x[2][i]);
      bfly(x[1][i], x[3][i]);
    }
    if constexpr (WV) {
#pragma unroll
      for (int k = 0; k < 4; ++k) xstage_mirror(x[k], mu3);
    }

    // position tbase + t, or its ring slot; 0 <= tbase + t < 2^32 when tbase >= 0
    int64_t tt = static_cast<int64_t>(R.tbase) + t;
    if (a.ring && tt >= 0)
      tt = static_cast<uint32_t>(tt) % static_cast<uint32_t>(a.t_max);
    const bool valid = t < a.tokens && tt >= 0 && tt < a.t_max;
    const uint32_t cblk = static_cast<uint32_t>(tt * a.nblk + j);
    const uint32_t co = valid ? cblk * CB : kOOB;
    uint16_t nbits;
    if constexpr (BITS == 8) {
      // turboq8 grid: per-block absmax scale, codes round((y / s) * 127.5 + 127.5)
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[k][i]));
      amax = quad_max<0xB1>(amax);
      amax = quad_max<0x4E>(amax);
      const __half s16 = __float2half_rn(fp32_value(amax * kInvSqrtQK));
      const float s32 = __half2float(s16);
      const float G = __uint_as_float(__float_as_uint(s32 > 0.0f ? kGrid8 / s32 : 0.0f) ^ carried);
      nbits = __half_as_ushort(s16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t8 = x[k][i] * ((s2bits >> (8 * k + i)) & 1u ? -G : G);
          const float w = t8 + 127.5f;
          code[i] = static_cast<uint32_t>(fminf(fmaxf(rintf(w), 0.0f), 255.0f));
        }
        const uint32_t lo = code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24;
        const uint32_t hi = code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24;
        const uint32_t o = co + 8 * (q + 4 * k);
        __builtin_amdgcn_raw_buffer_store_b32(lo, R.rc, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(hi, R.rc, o + 4, 0, 0);
      }
    } else {
      const float g0 = n32 > 0.0f ? c_scale / n32 : 0.0f;
      const float g = __uint_as_float(__float_as_uint(g0) ^ carried);
      float sq[4];
      auto codes8 = [&](int k) {
        constexpr int W = BITS == 2 ? 2 : 4;
        if constexpr (NC) return bucketize8_sq<W>(x[k], g, cells, sq[k]) ^ mirror[k];
        else return bucketize8<W>(x[k], g, cells) ^ mirror[k];
      };
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c = q + 4 * k;
        if constexpr (BITS == 4) {
          __builtin_amdgcn_raw_buffer_store_b32(codes8(k), R.rc, co + 4 * c, 0, 0);
        } else if constexpr (BITS == 2) {
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(codes8(k)), R.rc,
                                                co + 2 * c, 0, 0);
        } else {
          // 3-bit codes in nibbles, then the two planes of [turboq] block_turboq3_0
          const uint32_t w = codes8(k);
          uint32_t lo = w & 0x33333333u;
          lo = (lo | (lo >> 2)) & 0x0F0F0F0Fu;
          lo = (lo | (lo >> 4)) & 0x00FF00FFu;
          lo = (lo | (lo >> 8)) & 0x0000FFFFu;
          uint32_t hi = (w >> 2) & 0x11111111u;
          hi = (hi | (hi >> 3)) & 0x03030303u;
          hi = (hi | (hi >> 6)) & 0x000F000Fu;
          hi = (hi | (hi >> 12)) & 0xFFu;
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(lo), R.rc, co + 2 * c, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(hi), R.rc, co + 32 + c, 0, 0);
        }
      }
      if constexpr (NC) {
        // corrected norm n / ||c[codes]||: squared centroids summed in the input
        // norm's order (bits 0-2 in the chunk, 3-4 across the quad, 5-6 across chunks)
#pragma unroll
        for (int k = 0; k < 4; ++k) sq[k] = quad_add<0xB1>(sq[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k) sq[k] = quad_add<0x4E>(sq[k]);
        const float r32 = __builtin_sqrtf((sq[0] + sq[1]) + (sq[2] + sq[3]));
        nbits = __half_as_ushort(__float2half_rn(r32 > 0.0f ? n32 / r32 : 0.0f));
      } else {
        nbits = __half_as_ushort(__float2half_rn(n32));
      }
    }
    const uint32_t nidx = WV ? static_cast<uint32_t>(tt) : cblk;
    __builtin_amdgcn_raw_buffer_store_b16(
        nbits, R.rn, valid && q == 0 && (!WV || j == 0) ? 2 * nidx : kOOB, 0, 0);
  };
  // Ping-pong buffers: block t + t_step loads while block t is processed.  The trip
  // count is uniform over the wavefront (lane 0 holds its smallest t); lanes past the
  // last token load zeros and store nothing.
  // The stores of one block go to offsets past every range here (dropped by the
  // hardware) after the first load: the loop is then entered with the same
  // outstanding-memory pattern as every later iteration (loads, then that block's
  // stores), so the compiler's wait before each block covers only its own loads.
  // The scheduling barriers keep each prefetch ahead of the block it overlaps.
  for (;;) {
    dummy_stores<BITS>(R.rc, R.rn);
    while (__builtin_amdgcn_readfirstlane(t) < a.tokens) {
      load_raw<BF16>(R.rx, xoff(t + t_step), q, dead, bb);
      __builtin_amdgcn_sched_barrier(0);
      process(ba, t);
      t += t_step;
      if (__builtin_amdgcn_readfirstlane(t) >= a.tokens) break;
      load_raw<BF16>(R.rx, xoff(t + t_step), q, dead, ba);
      __builtin_amdgcn_sched_barrier(0);
      process(bb, t);
      t += t_step;
    }
    row += gridDim.y;
    if (row >= rows) break;
    R = open_row(row);
    t = t_first;
    load_raw<BF16>(R.rx, xoff(t), q, dead, ba);
  }
}

template <int BITS, bool BF16, bool NC, bool WV, bool PAD>
__global__ void __launch_bounds__(kEncThreads) encode_kernel(EncodeLaunch a, KTable tab,
                                                          SignWords sw) {
  encode_body<BITS, BF16, NC, WV, PAD>(a, tab, sw);
}

// The keys and the values of the same tokens in one launch (the same grid over the same
// shape): blockIdx.z = 0 encodes the keys, 1 the values.  APPEND only names the
// instantiation, so that the few-token encodes of an append and the joint encodes of
// whole caches show apart in kernel statistics.
template <int KB, int VB, bool BF16, bool NC, bool APPEND>
__global__ void __launch_bounds__(kEncThreads) encode_pair_kernel(EncodeLaunch ak, KTable tk,
                                                               EncodeLaunch av, KTable tv,
                                                               SignWords sw) {
  if (blockIdx.z == 0)
    encode_body<KB, BF16, NC, false, false>(ak, tk, sw);
  else
    encode_body<VB, BF16, NC, false, false>(av, tv, sw);
}

// Raw code words of one block for the lane's chunks q + 4k, and its norm, as loaded:
// a[k] the chunk's codes (4-bit: 4 bytes, 2/3-bit: the 2-bit plane's 2 bytes, 8-bit:
// the first 4 bytes), b[k] the 3-bit high plane byte or the second 4 bytes of an
// 8-bit chunk; n the fp16 norm bits.
template <int BITS>
struct RawCodes {
  uint32_t a[4];
  uint32_t b[BITS == 3 || BITS == 8 ? 4 : 1];
  uint32_t n;
};

// Loads of one block (byte offset co of its code row in rc, norm byte offset no in
// rn; kOOB for slots without work: zeros, nothing read).
template <int BITS>
__device__ __forceinline__ void load_codes(Rsrc rc, Rsrc rn, uint32_t co, uint32_t no, int q,
                                           RawCodes<BITS>& r) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t c = static_cast<uint32_t>(q + 4 * k);
    if constexpr (BITS == 4) {
      r.a[k] = __builtin_amdgcn_raw_buffer_load_b32(rc, co + 4 * c, 0, 0);
    } else if constexpr (BITS == 2) {
      r.a[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, co + 2 * c, 0, 0);
    } else if constexpr (BITS == 3) {
      r.a[k] = __builtin_amdgcn_raw_buffer_load_b16(rc, co + 2 * c, 0, 0);
      r.b[k] = __builtin_amdgcn_raw_buffer_load_b8(rc, co + 32 + c, 0, 0);
    } else {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(rc, co + 8 * c, 0, 0);
      r.a[k] = w[0];
      r.b[k] = w[1];
    }
  }
  r.n = __builtin_amdgcn_raw_buffer_load_b16(rn, no, 0, 0);
}

// The 8 codes of the lane's chunk k of an 8-bit row (one byte per code); 2-, 3- and
// 4-bit codes index the decoder's centroid table by byte or element pair.
template <int BITS>
__device__ __forceinline__ void chunk_codes(const RawCodes<BITS>& r, int k, uint32_t (&code)[8]) {
  static_assert(BITS == 8, "2-4 bit codes are looked up by byte or pair");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    code[i] = (r.a[k] >> (8 * i)) & 255u;
    code[4 + i] = (r.b[k] >> (8 * i)) & 255u;
  }
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Stores of one decoded block (same count and kinds as the decoder's), all to
// offset kOOB, so they are dropped.
template <bool BF16_OUT>
__device__ __forceinline__ void dummy_out_stores(Rsrc ro) {
#pragma unroll
  for (int k = 0; k < (BF16_OUT ? 4 : 8); ++k)
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, ro, kOOB + 16 * k, 0, 0);
}

// Decode: x_hat = s * (H (n * c[code])) / sqrt(128), one quad per block, in the
// encoder's layout: grid (gx, gy), blockIdx.y over the (batch, head) rows and block
// slots f = (token, block j) of a row strided by gridDim.x * 64 (a multiple of nblk, so
// a quad keeps its j and its sign words).  Ping-pong register sets: the next block's
// codes and norm load while the current block is transformed and stored.  Memory
// operations go through buffer resources; slots past the row's last token (and, with
// PAD, the padding chunks) use offset kOOB: they load zeros and store nothing,
// without divergent control flow, and every iteration leaves the same pattern of
// outstanding loads and stores, so the wait before a block covers only its own
// loads.  The two cross-lane stages are DPP multiply-adds as in the encoder: the
// upper lane of a pair keeps the negated difference, a sign folded into the final
// scale.  WV: whole vectors of head_dim 256 (nblk = 2): one norm per vector, the
// second quad's chunks in reversed lane order and the stage between the vector's two
// blocks by row_half_mirror, scale 1/16.
// PAD: d.dim < QK * nblk; the chunks at or past d.dim (the padding) are not stored.
// TWO: the two-sign rotation (otherwise s2 = +1 and its flips are compiled out).
template <int BITS, bool BF16_OUT, bool WV, bool PAD, bool TWO>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeLaunch d, KTable tab,
                                                          SignWords sw) {
  static_assert(!WV || BITS != 8, "whole-vector mode: 2-4 bit codebooks");
  static_assert(!PAD || BITS != 8, "padding: whole-vector mode only");
  static_assert(!TWO || (!WV && !PAD), "the whole-vector mode has one sign vector");
  constexpr int CB = code_bytes_of<BITS>();
  constexpr uint32_t OES = BF16_OUT ? 2 : 4;   // output element bytes
  // Centroid table in LDS.  4-bit codes: entry r (one code byte) holds the two
  // centroids (c[r & 15], c[r >> 4]); 2-bit: entry r holds the four centroids of the
  // byte's fields; 3-bit: entry r of 64 holds the centroids of an element pair whose
  // low bits are r & 15 (two 2-bit fields) and high bits r >> 4 (two 1-bit fields).
  constexpr int TW = BITS == 2 ? 4 : 2;   // floats per entry
  constexpr int TN = BITS == 3 ? 64 : 256;   // entries
  __shared__ __attribute__((aligned(16))) float ctab[BITS == 8 ? 1 : TN * TW];
  static_assert(kThreads == 256, "one table entry per thread");
  if constexpr (BITS == 4 || BITS == 2) {
    const uint32_t r = threadIdx.x;
#pragma unroll
    for (int m = 0; m < TW; ++m) ctab[TW * r + m] = tab.c[(r >> (8 / TW * m)) & ((1u << BITS) - 1)];
  } else if constexpr (BITS == 3) {
    const uint32_t r = threadIdx.x;
    if (r < 64) {
      ctab[2 * r] = tab.c[(r & 3) | ((r >> 2) & 4)];
      ctab[2 * r + 1] = tab.c[((r >> 2) & 3) | ((r >> 3) & 4)];
    }
  }
  __syncthreads();
  const int64_t rows = d.rows;
  int64_t row = blockIdx.y;
  if (row >= rows) return;   // uniform over the workgroup
  const uint32_t nblk = static_cast<uint32_t>(d.nblk);
  const uint32_t f0 = blockIdx.x * (kThreads / 4) + (threadIdx.x >> 2);
  const uint32_t fstep = gridDim.x * (kThreads / 4);
  const int j = static_cast<int>(f0 % nblk);
  const int q = WV && (j & 1) ? 3 - static_cast<int>(threadIdx.x & 3) : threadIdx.x & 3;
  const uint32_t sbits = sw.w[j][q];
  const uint32_t s2bits = TWO ? sw.w2[j][q] : 0u;   // R^T = D1 H D2 / sqrt(128)
  const float mu1 = (q & 1) ? -1.0f : 1.0f;
  const float mu2 = (q & 2) ? -1.0f : 1.0f;
  const float mu3 = (j & 1) ? -1.0f : 1.0f;
  const uint32_t carried = (((q ^ (q >> 1)) & 1u) ^ (WV ? (j & 1) : 0)) << 31;
  constexpr float c_scale = WV ? 0.0625f : kInvSqrtQK;   // RN32(1/sqrt(d))
  const float scale = __uint_as_float(__float_as_uint(c_scale) ^ carried);
  // store offset of the lane's chunk k relative to its block (or kOOB in the padding)
  uint32_t cofs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t e = QK * j + 8 * (q + 4 * k);
    cofs[k] = PAD && static_cast<int>(e) >= d.dim ? kOOB : e * OES;
  }
  // The host keeps a row's decoded codes, its norms and its output span below 2^31
  // bytes, so every offset below is a 32-bit value and kOOB lies past every range.
  const uint32_t tokens = static_cast<uint32_t>(d.tokens);
  const uint32_t per_row = tokens * nblk;
  const uint32_t nnorm = WV ? tokens : per_row;
  const uint32_t obytes =
      static_cast<uint32_t>(((d.tokens - 1) * d.st + static_cast<int64_t>(d.dim)) * OES);
  const uint32_t st_bytes = static_cast<uint32_t>(d.st) * OES;   // token stride of out
  // the quad's slots are f = t * nblk + j for its tokens t = t_first, + t_step, ...
  const uint32_t t_first = f0 / nblk, t_step = fstep / nblk;
  struct Row {
    Rsrc rc, rn, ro;
  };
  auto open_row = [&](int64_t r) {
    const int64_t b = r / d.heads, h = r - b * d.heads;
    Row R;
    R.rc = make_rsrc(d.codes + r * d.t_max * nblk * CB, per_row * CB);
    R.rn = make_rsrc(d.norms + r * d.t_max * (WV ? 1 : nblk), 2 * nnorm);
    R.ro = make_rsrc(static_cast<char*>(d.out) + (b * d.sb + h * d.sh) * OES, obytes);
    return R;
  };
  auto load = [&](const Row& R, uint32_t t, RawCodes<BITS>& raw) {
    const bool live = t < tokens;
    const uint32_t f = t * nblk + j;
    load_codes<BITS>(R.rc, R.rn, live ? f * CB : kOOB, live ? 2 * (WV ? t : f) : kOOB, q, raw);
  };
  auto process = [&](const Row& R, const RawCodes<BITS>& raw, uint32_t t) {
    const float n = __half2float(__ushort_as_half(static_cast<uint16_t>(raw.n)));
    float v[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float cv[8];   // centroid values of the chunk's 8 codes
      if constexpr (BITS == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float2 e = reinterpret_cast<const float2*>(ctab)[(raw.a[k] >> (8 * m)) & 255u];
          cv[2 * m] = e.x;
          cv[2 * m + 1] = e.y;
        }
      } else if constexpr (BITS == 2) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const float4 e = reinterpret_cast<const float4*>(ctab)[(raw.a[k] >> (8 * m)) & 255u];
          cv[4 * m] = e.x;
          cv[4 * m + 1] = e.y;
          cv[4 * m + 2] = e.z;
          cv[4 * m + 3] = e.w;
        }
      } else if constexpr (BITS == 3) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // elements 2m, 2m + 1: low bits from the 2-bit plane, high bits from the
          // 1-bit plane ([turboq] block_turboq3_0)
          const uint32_t r = ((raw.a[k] >> (4 * m)) & 15u) | (((raw.b[k] >> (2 * m)) & 3u) << 4);
          const float2 e = reinterpret_cast<const float2*>(ctab)[r];
          cv[2 * m] = e.x;
          cv[2 * m + 1] = e.y;
        }
      } else {
        uint32_t code[8];
        chunk_codes<BITS>(raw, k, code);
#pragma unroll
        for (int i = 0; i < 8; ++i) cv[i] = static_cast<float>(code[i]) - 127.5f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float r = BITS == 8 ? cv[i] * (n / 127.5f) : n * cv[i];
        v[k][i] = flip_sign(r, (s2bits >> (8 * k + i)) & 1u);
      }
    }
    // butterflies: stages 1, 2, 4 in-chunk, 8, 16 across the quad, 32, 64 across
    // chunks, and 128 across a whole vector's two quads
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bfly(v[k][0], v[k][1]); bfly(v[k][2], v[k][3]);
      bfly(v[k][4], v[k][5]); bfly(v[k][6], v[k][7]);
      bfly(v[k][0], v[k][2]); bfly(v[k][1], v[k][3]);
      bfly(v[k][4], v[k][6]); bfly(v[k][5], v[k][7]);
      bfly(v[k][0], v[k][4]); bfly(v[k][1], v[k][5]);
      bfly(v[k][2], v[k][6]); bfly(v[k][3], v[k][7]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) xstage<0xB1>(v[k], mu1);
#pragma unroll
    for (int k = 0; k < 4; ++k) xstage<0x4E>(v[k], mu2);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bfly(v[0][i], v[1][i]);
      bfly(v[2][i], v[3][i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bfly(v[0][i], v[2][i]);
      bfly(v[1][i], v[3][i]);
    }
    if constexpr (WV) {
#pragma unroll
      for (int k = 0; k < 4; ++k) xstage_mirror(v[k], mu3);
    }
    // byte offset of the block's token row; kOOB for a slot past the row
    const uint32_t tb = t < tokens ? t * st_bytes : kOOB;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = flip_sign(v[k][i] * scale, (sbits >> (8 * k + i)) & 1u);
      // past every range when either part is kOOB (the sum alone may wrap)
      const uint32_t o = (tb + cofs[k]) | ((tb | cofs[k]) & kOOB);
      if constexpr (BF16_OUT) {
        // v_cvt_pk_bf16_f32: two fp32 to bf16, round to nearest even
        uint32_t w[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          w[m] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                                  f2{r[2 * m], r[2 * m + 1]}, bf16x2));
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, R.ro, o, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]),
                  __float_as_uint(r[3])}, R.ro, o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4{__float_as_uint(r[4]), __float_as_uint(r[5]), __float_as_uint(r[6]),
                  __float_as_uint(r[7])}, R.ro, o + 16, 0, 0);
      }
    }
  };
  Row R = open_row(row);
  uint32_t t = t_first;
  RawCodes<BITS> ra, rb;
  load(R, t, ra);
  // Ping-pong over the row's slots (lane 0 holds the wavefront's smallest slot, so
  // the trip count is uniform); the stores of a block placed before the first one
  // (dropped) give the loop entry the same outstanding-memory pattern as later
  // iterations.
  for (;;) {
    dummy_out_stores<BF16_OUT>(R.ro);
    while (__builtin_amdgcn_readfirstlane(t) < tokens) {
      load(R, t + t_step, rb);
      __builtin_amdgcn_sched_barrier(0);
      process(R, ra, t);
      t += t_step;
      if (__builtin_amdgcn_readfirstlane(t) >= tokens) break;
      load(R, t + t_step, ra);
      __builtin_amdgcn_sched_barrier(0);
      process(R, rb, t);
      t += t_step;
    }
    row += gridDim.y;
    if (row >= rows) break;
    R = open_row(row);
    t = t_first;
    load(R, t, ra);
  }
}


// Encode grid: y over (batch, head) rows, x over the quads of a row; about
// kEncodeWGs workgroups in total, x a multiple of what keeps 64 * x divisible by
// nblk (so each quad keeps one block index j).
#ifndef FATQ_ENCODE_WGS
#define FATQ_ENCODE_WGS 1024
#endif
constexpr int64_t kEncodeWGs = FATQ_ENCODE_WGS;
// the workgroup budget of each half (keys, values) of an encode of both
#ifndef FATQ_ENCODE_PAIR_WGS
#define FATQ_ENCODE_PAIR_WGS FATQ_ENCODE_WGS
#endif
constexpr int64_t kEncodePairWGs = FATQ_ENCODE_PAIR_WGS;

dim3 encode_grid(const EncodeLaunch& a, int64_t wgs = kEncodeWGs) {
  const int64_t rows = static_cast<int64_t>(a.batch) * a.heads;
  const int64_t per_row = static_cast<int64_t>(a.tokens) * a.nblk;
  const int64_t wg_row = (per_row + kEncThreads / 4 - 1) / (kEncThreads / 4);
  const int64_t gy = rows < 65535 ? rows : 65535;
  int64_t gx = wgs / gy;
  if (gx > wg_row) gx = wg_row;
  if (gx < 1) gx = 1;
  int64_t g = kEncThreads / 4, n = a.nblk;   // r = nblk / gcd(quads per WG, nblk)
  while (n != 0) {
    const int64_t t = g % n;
    g = n;
    n = t;
  }
  const int64_t r = a.nblk / g;
  gx = (gx + r - 1) / r * r;
  return dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy));
}

}  // namespace

hipError_t launch_encode(const EncodeLaunch& a, const KTable& tab, const SignWords& sw,
                         bool norm_correct, bool whole, hipStream_t stream) {
  const dim3 grid = encode_grid(a), block(kEncThreads);
  EncodeLaunch la = a;
  la.t_step = static_cast<int32_t>(grid.x * (kEncThreads / 4) / a.nblk);
#define FATQ_ENC(B, F, N, W, P) \
  hipLaunchKernelGGL((encode_kernel<B, F, N, W, P>), grid, block, 0, stream, la, tab, sw)
#define FATQ_ENC_BITS(F, N)                            \
  switch (tab.bits) {                                  \
    case 2: FATQ_ENC(2, F, N, false, false); break;    \
    case 3: FATQ_ENC(3, F, N, false, false); break;    \
    case 4: FATQ_ENC(4, F, N, false, false); break;    \
    default: FATQ_ENC(8, F, false, false, false); break; \
  }
#define FATQ_ENC_WV(F, W, P)                        \
  switch (tab.bits) {                               \
    case 2: FATQ_ENC(2, F, false, W, P); break;     \
    case 3: FATQ_ENC(3, F, false, W, P); break;     \
    default: FATQ_ENC(4, F, false, W, P); break;    \
  }
#define FATQ_ENC_WHOLE(F)                                          \
  if (a.nblk == 2) {                                               \
    if (pad) { FATQ_ENC_WV(F, true, true) } else { FATQ_ENC_WV(F, true, false) } \
  } else {                                                         \
    FATQ_ENC_WV(F, false, true)                                    \
  }
  // unpadded head_dim 128 in the whole-vector mode is the blocked encode itself
  const bool pad = a.dim != QK * a.nblk;
  if (pad && !whole) return hipErrorInvalidValue;
  if (whole && (a.nblk == 2 || pad)) {
    if (a.x_is_bf16) { FATQ_ENC_WHOLE(true) } else { FATQ_ENC_WHOLE(false) }
  } else if (a.x_is_bf16) {
    if (norm_correct) { FATQ_ENC_BITS(true, true) } else { FATQ_ENC_BITS(true, false) }
  } else {
    if (norm_correct) { FATQ_ENC_BITS(false, true) } else { FATQ_ENC_BITS(false, false) }
  }
#undef FATQ_ENC_WHOLE
#undef FATQ_ENC_WV
#undef FATQ_ENC_BITS
#undef FATQ_ENC
  return hipGetLastError();
}

hipError_t launch_encode_pair(const EncodeLaunch& ak, const KTable& tk, const EncodeLaunch& av,
                              const KTable& tv, const SignWords& sw, bool norm_correct,
                              bool append, hipStream_t stream) {
  if (ak.batch != av.batch || ak.heads != av.heads || ak.tokens != av.tokens ||
      ak.nblk != av.nblk || ak.x_is_bf16 != av.x_is_bf16 || ak.dim != QK * ak.nblk ||
      av.dim != QK * av.nblk || tk.bits == 8 || tv.bits == 8)
    return hipErrorInvalidValue;
  const dim3 g2 = encode_grid(ak, kEncodePairWGs), grid(g2.x, g2.y, 2), block(kEncThreads);
  EncodeLaunch lk = ak, lv = av;
  lk.t_step = lv.t_step = static_cast<int32_t>(grid.x * (kEncThreads / 4) / ak.nblk);
#define FATQ_PAIR(K, V, F, N)                                                              \
  hipLaunchKernelGGL((append ? encode_pair_kernel<K, V, F, N, true>                        \
                             : encode_pair_kernel<K, V, F, N, false>),                     \
                     grid, block, 0, stream, lk, tk, lv, tv, sw)
#define FATQ_PAIR_V(K, F, N)                     \
  switch (tv.bits) {                             \
    case 2: FATQ_PAIR(K, 2, F, N); break;        \
    case 3: FATQ_PAIR(K, 3, F, N); break;        \
    default: FATQ_PAIR(K, 4, F, N); break;       \
  }
#define FATQ_PAIR_KV(F, N)                       \
  switch (tk.bits) {                             \
    case 2: FATQ_PAIR_V(2, F, N) break;          \
    case 3: FATQ_PAIR_V(3, F, N) break;          \
    default: FATQ_PAIR_V(4, F, N) break;         \
  }
  if (ak.x_is_bf16) {
    if (norm_correct) { FATQ_PAIR_KV(true, true) } else { FATQ_PAIR_KV(true, false) }
  } else {
    if (norm_correct) { FATQ_PAIR_KV(false, true) } else { FATQ_PAIR_KV(false, false) }
  }
#undef FATQ_PAIR_KV
#undef FATQ_PAIR_V
#undef FATQ_PAIR
  return hipGetLastError();
}

// Decode grid: y over the rows, x over the block slots of a row (about kDecodeWGs
// workgroups in total, so that a quad loops over several blocks and its loads run
// one block ahead), x a multiple of what keeps 64 * x divisible by nblk.
#ifndef FATQ_DECODE_WGS
#define FATQ_DECODE_WGS 2048
#endif
constexpr int64_t kDecodeWGs = FATQ_DECODE_WGS;

dim3 decode_grid(const DecodeLaunch& d) {
  const int64_t gy = d.rows < 65535 ? d.rows : 65535;
  const int64_t per_row = d.tokens * d.nblk;
  const int64_t wg_row = (per_row + kThreads / 4 - 1) / (kThreads / 4);
  int64_t gx = kDecodeWGs / gy;
  if (gx > wg_row) gx = wg_row;
  if (gx < 1) gx = 1;
  int64_t g = kThreads / 4, n = d.nblk;
  while (n != 0) {
    const int64_t t = g % n;
    g = n;
    n = t;
  }
  const int64_t r = d.nblk / g;
  gx = (gx + r - 1) / r * r;
  return dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy > 0 ? gy : 1));
}

hipError_t launch_decode(const DecodeLaunch& d, const KTable& tab, const SignWords& sw,
                         bool whole, hipStream_t stream) {
  const dim3 grid = decode_grid(d), block(kThreads);
#define FATQ_DEC(B, F, W, P, T) \
  hipLaunchKernelGGL((decode_kernel<B, F, W, P, T>), grid, block, 0, stream, d, tab, sw)
#define FATQ_DEC_BITS(F, T)                            \
  switch (tab.bits) {                                  \
    case 2: FATQ_DEC(2, F, false, false, T); break;    \
    case 3: FATQ_DEC(3, F, false, false, T); break;    \
    case 4: FATQ_DEC(4, F, false, false, T); break;    \
    default: FATQ_DEC(8, F, false, false, T); break;   \
  }
#define FATQ_DEC_WV(F, W, P)                       \
  switch (tab.bits) {                              \
    case 2: FATQ_DEC(2, F, W, P, false); break;    \
    case 3: FATQ_DEC(3, F, W, P, false); break;    \
    default: FATQ_DEC(4, F, W, P, false); break;   \
  }
#define FATQ_DEC_WHOLE(F)                                          \
  if (d.nblk == 2) {                                               \
    if (pad) { FATQ_DEC_WV(F, true, true) } else { FATQ_DEC_WV(F, true, false) } \
  } else {                                                         \
    FATQ_DEC_WV(F, false, true)                                    \
  }
  const bool pad = d.dim != QK * d.nblk;
  if (pad && !whole) return hipErrorInvalidValue;
  if (whole && sw.two) return hipErrorInvalidValue;
  if (whole && (d.nblk == 2 || pad)) {
    if (d.out_bf16) { FATQ_DEC_WHOLE(true) } else { FATQ_DEC_WHOLE(false) }
  } else if (sw.two) {
    if (d.out_bf16) { FATQ_DEC_BITS(true, true) } else { FATQ_DEC_BITS(false, true) }
  } else {
    if (d.out_bf16) { FATQ_DEC_BITS(true, false) } else { FATQ_DEC_BITS(false, false) }
  }
#undef FATQ_DEC_WHOLE
#undef FATQ_DEC_WV
#undef FATQ_DEC_BITS
#undef FATQ_DEC
  return hipGetLastError();
}

}  // namespace fatq

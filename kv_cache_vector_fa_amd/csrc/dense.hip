// Encode and decode with a dense random orthogonal rotation, for head_dims that are not
// a power of two (gfx950).
//
// Page cited: [Spec] "TurboQuant KV Cache Compression -- Spec", "Hadamard Transform
// Detail" (for a head_dim that is not a power of two: a dense random orthogonal matrix
// instead of padding to the next power of two) and "Step 1: Random Orthogonal
// Rotation" (rotate(x) = R x with a fixed d x d orthogonal R from the seed).
//
// The rotation of a batch of vectors is a dense product, Y = R X (d x d times d x N),
// so it runs on v_mfma_f32_16x16x32_f16: A = a 16 x 32 tile of R (outputs x channels),
// B = a 32 x 16 tile of X (channels x vectors), D = 16 outputs of 16 vectors.
//
// Accuracy (every fp16 product exact in the fp32 accumulator):
//  * R is held in LDS as two fp16 matrices, 2^14 R = hi + lo (hi the nearest fp16, lo
//    the nearest fp16 of the exact fp32 remainder): about 22 significant bits, and both
//    halves fp16 normal numbers unless |R_ij| is below about 2^-17;
//  * an input vector is scaled by the power of two 2^k that puts its fp32 norm n in
//    [2^14, 2^15) (so every |x_i| 2^k < 2^15); a scaled bf16 value of magnitude at
//    least 2^-17 (every |x_i| >= 2^-31 n) is then an exact fp16 number, and a smaller
//    one is off by at most 2^-25 (2^-39 n before scaling).  An fp32 input is split like
//    R (two fp16 halves, three products per tile);
//  * Y = (2^14 R)(2^k X) accumulates in fp32; u = Y / (2^(14 + k) n) with one fp32
//    multiply by RN(1 / (2^(14+k) n)), which is RN(1 / n) 2^-(14+k) whenever 1 / n is a
//    normal number, so u = RN(y RN(1 / n)) for the rotated coordinate y.
// The norm n is the canonical fp32 norm of the vector zero-padded to a power of two
// (squares summed pairwise over index bits 0, 1, ...: bits 0-2 in-lane, bits 3-4
// across the four row groups of the B layout, bits 5-7 over the k-steps), stored as
// fp16 (for bf16 inputs each pair of exact squares is added by one fma).  Codes are
// #{j : b_j < u}, read from a table of 1024 cells of a uniform grid over [-1, 1] (one
// LDS read and one compare: see grid_cell); the d codes of a vector fill
// ceil(d / 128) packed blocks, code 0 past d.
//
// Decode is the transpose: A = R^T tiles (2^14 R^T = hi + lo in LDS), B = the centroids
// of the codes (2^14 c = hi + lo, looked up in LDS per code byte as ready B operand
// pieces), three products per tile, then x = acc * (n16 2^-28).
//
// Work layout: one workgroup of eight waves per compute unit (the two R halves take up
// to 150 KB of LDS, the encoder's grid table 8 KB more); a wave processes 16 NV vectors
// per pass, holds them in registers as B operands for the whole pass, issues the next
// pass's loads, and loops over the output tiles (16 rows of R), reading each A operand
// from LDS once for NV products.  LDS rows are padded by 16 bytes, so the 16 lanes of a
// row group reading 16 rows at one column hit 16 distinct 4-bank groups.

#include <type_traits>

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kDW = 8;                  // waves per workgroup
constexpr int kDT = 64 * kDW;
constexpr int kNS = kDenseMax / 32;     // k-steps of 32 channels at the largest head_dim
constexpr int kNO = kDenseMax / 16;     // output tiles of 16 at the largest head_dim
constexpr int kRowH = kDenseMax + 8;    // fp16 per LDS row of R (16 bytes of padding)
constexpr int kRShift = 14;             // R and the centroids are scaled by 2^14 (exact)
// 16-vector tiles per wave pass (two: with the next pass's inputs in flight the
// registers hold no more; three or four measured slower)
constexpr int kNV = 2;

template <int B>
constexpr int dense_cbytes() { return B == 2 ? 32 : B == 3 ? 48 : 64; }

// Bucketize grid: cell(u) = clamp(floor(fma(u, G/2, G/2)), 0, G - 1), monotone in u, so
// with at most one boundary per cell, code = #{b_j : cell(b_j) < cell(u)} + (u > b*)
// where b* is the boundary in u's cell (+inf if none) -- the exact count #{j : b_j < u}.
__device__ __forceinline__ int grid_cell(float u) {
  const float f = __builtin_amdgcn_fmed3f(__builtin_fmaf(u, 0.5f * kDenseGrid, 0.5f * kDenseGrid),
                                          0.0f, static_cast<float>(kDenseGrid - 1));
  // f is in [0, G - 1] (or NaN, which the conversion turns into 0): truncation is floor
  return static_cast<int>(f);
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(_Float16 x, _Float16 y) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  h2 v = {x, y};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^14 r = hi + lo, hi the nearest fp16, lo the nearest fp16 of the exact remainder
__device__ __forceinline__ void split14(float r, _Float16& hi, _Float16& lo) {
  const float s = __builtin_amdgcn_ldexpf(r, kRShift);
  hi = static_cast<_Float16>(s);
  lo = static_cast<_Float16>(s - static_cast<float>(hi));
}

// Values of the lane pairs (l, l ^ 16) and then (l, l ^ 32): v_permlane16_swap with
// both operands equal returns the even row of a pair in its first result and the odd
// row in its second on every lane of the pair (permlane32_swap: the low and high
// halves of the wave).
__device__ __forceinline__ void rows16(uint32_t v, uint32_t& even, uint32_t& odd) {
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  even = p[0];
  odd = p[1];
}
__device__ __forceinline__ void halves32(uint32_t v, uint32_t& low, uint32_t& high) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  low = p[0];
  high = p[1];
}

// sum over the four row groups: index bit 3 (lanes l, l ^ 16), then bit 4
__device__ __forceinline__ float sum_groups(float t) {
  uint32_t e, o;
  rows16(__float_as_uint(t), e, o);
  t = __uint_as_float(e) + __uint_as_float(o);
  halves32(__float_as_uint(t), e, o);
  return __uint_as_float(e) + __uint_as_float(o);
}

struct VecPos {
  int64_t row;   // b * heads + h
  int t;         // token index within the call
  int b, h;
  bool live;
};

// position of vector gv (< 2^31 vectors per call, checked by the host): 32-bit division
__device__ __forceinline__ VecPos vec_pos(int64_t gv, int64_t nvec, int tokens, int heads) {
  VecPos p;
  p.live = gv < nvec;
  const uint32_t v = static_cast<uint32_t>(p.live ? gv : 0);
  const uint32_t row = v / static_cast<uint32_t>(tokens);
  p.row = row;
  p.t = static_cast<int>(v - row * static_cast<uint32_t>(tokens));
  p.b = static_cast<int>(row / static_cast<uint32_t>(heads));
  p.h = static_cast<int>(row - static_cast<uint32_t>(p.b) * static_cast<uint32_t>(heads));
  return p;
}

// the 8 elements of a 16-byte (bf16) or 32-byte (fp32) chunk as fp32
template <bool F32>
__device__ __forceinline__ void unpack8(const uint4 (&w)[F32 ? 2 : 1], float (&v)[8]) {
  if constexpr (F32) {
    const uint32_t ws[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[F32].x, w[F32].y, w[F32].z, w[F32].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(ws[e]);
  } else {
    const uint32_t ws[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[2 * m] = __uint_as_float(ws[m] << 16);
      v[2 * m + 1] = __uint_as_float(ws[m] & 0xFFFF0000u);
    }
  }
}

template <int BITS, bool F32, int NS, bool VEC>
__global__ void __launch_bounds__(kDT, 1) dense_encode_kernel(DenseLaunch a, KTable tab) {
  constexpr int NV = kNV;
  constexpr int CB = dense_cbytes<BITS>();
  __shared__ __attribute__((aligned(16))) _Float16 rh[kNO * 16 * kRowH];
  __shared__ __attribute__((aligned(16))) _Float16 rl[kNO * 16 * kRowH];
  __shared__ uint2 gt[kDenseGrid];   // per grid cell: {boundary in the cell or +inf, base code}
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.dim, no = (d + 15) >> 4;

  // 2^14 R (row i = output i, column j = input j) as fp16 hi / lo, zero past d
  const int rows = no * 16;
  for (int c = tid; c < rows * (kDenseMax / 8); c += kDT) {
    const int i = c / (kDenseMax / 8), j0 = (c - i * (kDenseMax / 8)) * 8;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int j = j0 + 2 * m;
      const float r0 = i < d && j < d ? a.rot[i * d + j] : 0.0f;
      const float r1 = i < d && j + 1 < d ? a.rot[i * d + j + 1] : 0.0f;
      _Float16 h0, l0, h1, l1;
      split14(r0, h0, l0);
      split14(r1, h1, l1);
      hw[m] = pack2(h0, h1);
      lw[m] = pack2(l0, l1);
    }
    *reinterpret_cast<uint4*>(rh + i * kRowH + j0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(rl + i * kRowH + j0) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  // the grid table (the host checked that no cell holds two boundaries)
  for (int c = tid; c < kDenseGrid; c += kDT) {
    uint32_t base = 0u;
    float thr = __builtin_inff();
#pragma unroll
    for (int q = 0; q < 15; ++q) {
      if (q < tab.nb) {
        const int cq = grid_cell(tab.b[q]);
        base += cq < c ? 1u : 0u;
        thr = cq == c ? tab.b[q] : thr;
      }
    }
    gt[c] = make_uint2(__float_as_uint(thr), base);
  }
  __syncthreads();

  const int64_t nvec = static_cast<int64_t>(a.batch) * a.heads * a.tokens;
  const int64_t per = 16 * NV;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * kDW * per;
  const int nblk = a.nblk;
  // ---- inputs as B operands (lane: vector 16 nv + n, channels 32 s + 8 g .. + 7).
  //      VEC (16-byte aligned rows, d a multiple of 8): every 16-byte load of a pass is
  //      issued before any is used, and the next pass's loads are issued before this
  //      pass's products (their latency hides behind them).  A k-step inside the vector
  //      for every lane loads at a fixed offset from the lane's row pointer (a lane
  //      without a vector points into the first vector, whose chunk at that offset
  //      exists); a k-step reaching past d redirects the lanes past d to the first chunk
  //      and zeroes them.  Otherwise: element loads at an index clamped into the vector,
  //      zeros selected outside it.
  constexpr int RW = F32 ? 2 : 1;   // 16-byte words per 8 elements
  constexpr int64_t ES = F32 ? 4 : 2;
  const char* x0 = static_cast<const char*>(a.x);
  uint4 raw[NV][NS][RW];
  auto load_raw = [&](int64_t v0) {
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const VecPos p = vec_pos(v0 + 16 * nv + n, nvec, a.tokens, a.heads);
      const int64_t base = p.live ? p.b * a.sb + p.h * a.sh + static_cast<int64_t>(p.t) * a.st : 0;
      const char* row = x0 + (base + 8 * g) * ES;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint4* src;
        if (32 * s + 32 <= d) {
          src = reinterpret_cast<const uint4*>(row + 32 * s * ES);
        } else {
          const bool ok = 32 * s + 8 * g < d;
          src = reinterpret_cast<const uint4*>(ok ? row + 32 * s * ES : x0);
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) raw[nv][s][r] = src[r];
      }
    }
  };
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kDW + wave) * per;
  if constexpr (VEC) {
    if (first < nvec) load_raw(first);
  }
  for (int64_t v0 = first; v0 < nvec; v0 += gstride) {
    int64_t base[NV], slot[NV];
    bool live[NV];
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const VecPos p = vec_pos(v0 + 16 * nv + n, nvec, a.tokens, a.heads);
      live[nv] = p.live;
      base[nv] = p.live ? p.b * a.sb + p.h * a.sh + static_cast<int64_t>(p.t) * a.st : 0;
      const int64_t pos = static_cast<int64_t>(a.t0 ? a.t0[p.live ? p.b : 0] : 0) + p.t;
      slot[nv] = p.live && pos >= 0 && pos < a.t_max ? p.row * a.t_max + pos : -1;
    }
    if constexpr (VEC) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (32 * s + 32 > d) {
          const bool ok = 32 * s + 8 * g < d;
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
            for (int r = 0; r < RW; ++r) {
              raw[nv][s][r].x = ok ? raw[nv][s][r].x : 0u;
              raw[nv][s][r].y = ok ? raw[nv][s][r].y : 0u;
              raw[nv][s][r].z = ok ? raw[nv][s][r].z : 0u;
              raw[nv][s][r].w = ok ? raw[nv][s][r].w : 0u;
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int i0 = 32 * s + 8 * g;
          uint32_t w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = i0 + e;
            const int64_t at = base[nv] + (j < d ? j : d - 1);
            uint32_t t;
            if constexpr (F32)
              t = __float_as_uint(static_cast<const float*>(a.x)[at]);
            else
              t = static_cast<const uint16_t*>(a.x)[at];
            w[e] = live[nv] && j < d ? t : 0u;
          }
          if constexpr (F32) {
            raw[nv][s][0] = make_uint4(w[0], w[1], w[2], w[3]);
            raw[nv][s][RW - 1] = make_uint4(w[4], w[5], w[6], w[7]);
          } else {
            raw[nv][s][0] = make_uint4(w[0] | w[1] << 16, w[2] | w[3] << 16, w[4] | w[5] << 16,
                                       w[6] | w[7] << 16);
          }
        }
        // one vector tile's loads in flight at a time (bounds the registers they hold)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    h8 xh[NV][NS], xl[F32 ? NV : 1][NS];
    float gs[NV];
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      float part[8];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
        unpack8<F32>(raw[nv][s], v);
        float p2[4];   // level 0 of the tree: q[2m] + q[2m + 1], q = RN(x^2)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if constexpr (F32) {
            p2[m] = v[2 * m] * v[2 * m] + v[2 * m + 1] * v[2 * m + 1];
          } else {
            // a bf16 square is exact in fp32 (q = x^2), so one fma gives RN(q0 + q1)
            p2[m] = __builtin_fmaf(v[2 * m], v[2 * m], v[2 * m + 1] * v[2 * m + 1]);
          }
        }
        part[s] = sum_groups((p2[0] + p2[1]) + (p2[2] + p2[3]));
      }
#pragma unroll
      for (int s = NS; s < 8; ++s) part[s] = 0.0f;
      const float ss = ((part[0] + part[1]) + (part[2] + part[3])) +
                       ((part[4] + part[5]) + (part[6] + part[7]));
      const float n32 = __builtin_sqrtf(ss);
      // 2^k puts n (>= every |x_i|, up to the rounding of fp32 squares) in [2^14, 2^15)
      const int k = 141 - static_cast<int>((__float_as_uint(n32) >> 23) & 0xFFu);
      gs[nv] = n32 > 0.0f ? 1.0f / __builtin_amdgcn_ldexpf(n32, kRShift + k) : 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float v[8];
        unpack8<F32>(raw[nv][s], v);
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float s0 = __builtin_amdgcn_ldexpf(v[2 * m], k);
          const float s1 = __builtin_amdgcn_ldexpf(v[2 * m + 1], k);
          const _Float16 h0 = static_cast<_Float16>(s0), h1 = static_cast<_Float16>(s1);
          wh[m] = pack2(h0, h1);
          if constexpr (F32) {
            wl[m] = pack2(static_cast<_Float16>(s0 - static_cast<float>(h0)),
                          static_cast<_Float16>(s1 - static_cast<float>(h1)));
          }
        }
        xh[nv][s] = __builtin_bit_cast(h8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
        if constexpr (F32) xl[nv][s] = __builtin_bit_cast(h8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
      }
      if (g == 0 && slot[nv] >= 0) a.norms[slot[nv]] = __half_as_ushort(__float2half_rn(n32));
    }

    if constexpr (VEC) {
      if (v0 + gstride < nvec) load_raw(v0 + gstride);
    }
    // ---- output tiles: 16 rows of R against the NV vector tiles
    uint8_t* dstv[NV];   // each vector's packed codes (slot 0 for a vector not stored)
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) dstv[nv] = a.codes + (slot[nv] < 0 ? 0 : slot[nv]) * nblk * CB;
    for (int o = 0; o < no; ++o) {
      // fp32 inputs: the hi x hi products in acc, the cross products in acc2 (two
      // independent chains per tile); bf16 inputs: NV chains of acc
      f4 acc[NV], acc2[F32 ? NV : 1];
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) acc[nv] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int nv = 0; nv < (F32 ? NV : 1); ++nv) acc2[nv] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      const _Float16* ph = rh + (16 * o + n) * kRowH + 8 * g;
      const _Float16* pl = rl + (16 * o + n) * kRowH + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const h8 ah = *reinterpret_cast<const h8*>(ph + 32 * s);
        const h8 al = *reinterpret_cast<const h8*>(pl + 32 * s);
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) acc[nv] = mfma(ah, xh[nv][s], acc[nv]);
        if constexpr (F32) {
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) acc2[nv] = mfma(al, xh[nv][s], acc2[nv]);
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) acc2[nv] = mfma(ah, xl[nv][s], acc2[nv]);
        } else {
#pragma unroll
          for (int nv = 0; nv < NV; ++nv) acc[nv] = mfma(al, xh[nv][s], acc[nv]);
        }
      }
      if constexpr (F32) {
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) acc[nv] += acc2[F32 ? nv : 0];
      }
      // lane (g, n) holds outputs 16 o + 4 g + i of vector 16 nv + n; code 0 past d
      const int i0 = 16 * o + 4 * g;
      float u[NV][4];
      uint2 ge[NV][4];
#pragma unroll
      for (int nv = 0; nv < NV; ++nv)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u[nv][i] = acc[nv][i] * gs[nv];
          ge[nv][i] = gt[grid_cell(u[nv][i])];
        }
      uint32_t cc[NV][4];
#pragma unroll
      for (int nv = 0; nv < NV; ++nv)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cc[nv][i] = ge[nv][i].y + (u[nv][i] > __uint_as_float(ge[nv][i].x) ? 1u : 0u);
      if (16 * o + 16 > d) {
#pragma unroll
        for (int nv = 0; nv < NV; ++nv)
#pragma unroll
          for (int i = 0; i < 4; ++i) cc[nv][i] = i0 + i < d ? cc[nv][i] : 0u;
      }
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) {
        const uint32_t (&c)[4] = cc[nv];
        uint8_t* dst = dstv[nv];
        const bool store = slot[nv] >= 0;
        if constexpr (BITS == 4) {
          // word w of the vector: codes 8 w .. 8 w + 7, low nibble first; rows 2 w' and
          // 2 w' + 1 of tile o make word 2 o + w'
          const uint32_t h = c[0] | c[1] << 4 | c[2] << 8 | c[3] << 12;
          uint32_t he, ho;
          rows16(h, he, ho);
          if (store && (g & 1) == 0)
            reinterpret_cast<uint32_t*>(dst)[2 * o + (g >> 1)] = he | ho << 16;
        } else if constexpr (BITS == 2) {
          // word o: codes 16 o .. 16 o + 15, 2 bits each
          const uint32_t b = c[0] | c[1] << 2 | c[2] << 4 | c[3] << 6;
          uint32_t be, bo, lo, hi;
          rows16(b, be, bo);
          halves32(be | bo << 8, lo, hi);
          if (store && g == 0) reinterpret_cast<uint32_t*>(dst)[o] = lo | hi << 16;
        } else {
          // 3-bit ([turboq] block_turboq3_0): block o / 8 holds 32 bytes of low 2-bit
          // fields (word o % 8 for this tile) and then 16 bytes of high bits (bytes
          // 2 (o % 8) and 2 (o % 8) + 1)
          const uint32_t b = (c[0] & 3u) | (c[1] & 3u) << 2 | (c[2] & 3u) << 4 | (c[3] & 3u) << 6;
          const uint32_t t = (c[0] >> 2) | (c[1] >> 2) << 1 | (c[2] >> 2) << 2 | (c[3] >> 2) << 3;
          uint32_t be, bo, te, to, lo, hi, tlo, thi;
          rows16(b, be, bo);
          rows16(t, te, to);
          halves32(be | bo << 8, lo, hi);
          halves32(te | to << 4, tlo, thi);
          if (store && g == 0) {
            uint8_t* blk = dst + (o >> 3) * CB;
            reinterpret_cast<uint32_t*>(blk)[o & 7] = lo | hi << 16;
            reinterpret_cast<uint16_t*>(blk + 32)[o & 7] = static_cast<uint16_t>(tlo | thi << 8);
          }
        }
      }
    }
    // ---- code 0 in the tiles past the last output tile, up to the end of the blocks
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      if (slot[nv] < 0 || g != 0) continue;
      uint8_t* dst = dstv[nv];
      for (int o = no; o < 8 * nblk; ++o) {
        if constexpr (BITS == 4) {
          reinterpret_cast<uint2*>(dst)[o] = make_uint2(0u, 0u);
        } else if constexpr (BITS == 2) {
          reinterpret_cast<uint32_t*>(dst)[o] = 0u;
        } else {
          uint8_t* blk = dst + (o >> 3) * CB;
          reinterpret_cast<uint32_t*>(blk)[o & 7] = 0u;
          reinterpret_cast<uint16_t*>(blk + 32)[o & 7] = 0u;
        }
      }
    }
  }
}

// B operand pieces of 8 codes: hi and lo halves of 2^14 c[code] for the code bytes.
// 4-bit: entry per code byte (two codes): {hi pair, lo pair}; 2-bit: entry per byte
// (four codes): {hi quad, lo quad}; 3-bit: entry per pair of codes indexed by the pair's
// two low-bit fields and two high bits: {hi pair, lo pair}.
template <int BITS>
constexpr int ctab_entries() { return BITS == 3 ? 64 : 256; }

template <int BITS, int NS>
__global__ void __launch_bounds__(kDT, 1) dense_decode_kernel(DenseDecodeLaunch a, KTable tab) {
  constexpr int NV = kNV;
  constexpr int CB = dense_cbytes<BITS>();
  __shared__ __attribute__((aligned(16))) _Float16 rh[kNO * 16 * kRowH];
  __shared__ __attribute__((aligned(16))) _Float16 rl[kNO * 16 * kRowH];
  // 2-bit: {hi quad, lo quad} per code byte; 3/4-bit: {hi pair, lo pair}
  typedef typename std::conditional<BITS == 2, uint4, uint2>::type CT;
  __shared__ __attribute__((aligned(16))) CT ct[ctab_entries<BITS>()];
  __shared__ float cs[16];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.dim, no = (d + 15) >> 4;

  // 2^14 R^T (row j = output j, column i = code coordinate i) as fp16 hi / lo
  const int rows = no * 16;
  for (int c = tid; c < rows * (kDenseMax / 8); c += kDT) {
    const int j = c % rows, i0 = (c / rows) * 8;
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = i0 + 2 * m;
      const float r0 = j < d && i < d ? a.rot[i * d + j] : 0.0f;
      const float r1 = j < d && i + 1 < d ? a.rot[(i + 1) * d + j] : 0.0f;
      _Float16 h0, l0, h1, l1;
      split14(r0, h0, l0);
      split14(r1, h1, l1);
      hw[m] = pack2(h0, h1);
      lw[m] = pack2(l0, l1);
    }
    *reinterpret_cast<uint4*>(rh + j * kRowH + i0) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4*>(rl + j * kRowH + i0) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) cs[q] = tab.c[q];
  }
  __syncthreads();
  for (int e = tid; e < ctab_entries<BITS>(); e += kDT) {
    _Float16 h[4], l[4];
    int nc;
    if constexpr (BITS == 4) {
      split14(cs[e & 15], h[0], l[0]);
      split14(cs[e >> 4], h[1], l[1]);
      nc = 2;
    } else if constexpr (BITS == 2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) split14(cs[(e >> (2 * m)) & 3], h[m], l[m]);
      nc = 4;
    } else {
      split14(cs[(e & 3) | ((e >> 4) & 1) << 2], h[0], l[0]);
      split14(cs[((e >> 2) & 3) | ((e >> 5) & 1) << 2], h[1], l[1]);
      nc = 2;
    }
    (void)nc;
    if constexpr (BITS == 2)
      ct[e] = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(l[0], l[1]), pack2(l[2], l[3]));
    else
      ct[e] = make_uint2(pack2(h[0], h[1]), pack2(l[0], l[1]));
  }
  __syncthreads();

  const int64_t nvec = a.rows * a.tokens;
  const int64_t per = 16 * NV;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * kDW * per;
  const int nblk = a.nblk;
  // ---- codes and norms of a pass: every load issued before any is used (lanes without
  //      a vector read slot 0); the codes of k-steps past d lie inside the vector's
  //      blocks and meet zero columns of R^T.  The next pass's loads are issued before
  //      this pass's products, so their latency hides behind them.
  uint32_t cw[NV][NS], ch[BITS == 3 ? NV : 1][NS];
  uint16_t nraw[NV];
  auto load_pass = [&](int64_t v0) {
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const VecPos p = vec_pos(v0 + 16 * nv + n, nvec, static_cast<int>(a.tokens), a.heads);
      const int64_t slot = p.live ? p.row * a.t_max + p.t : 0;
      nraw[nv] = a.norms[slot];
      const uint8_t* row = a.codes + slot * nblk * CB;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int i0 = 32 * s + 8 * g;   // 8 codes i0 .. i0 + 7 (within one block)
        if constexpr (BITS == 4) {
          cw[nv][s] = *reinterpret_cast<const uint32_t*>(row + (i0 >> 1));
        } else if constexpr (BITS == 2) {
          cw[nv][s] = *reinterpret_cast<const uint16_t*>(row + (i0 >> 2));
        } else {
          const uint8_t* blk = row + (i0 >> 7) * CB;
          const int e = i0 & 127;
          cw[nv][s] = *reinterpret_cast<const uint16_t*>(blk + (e >> 2));
          ch[BITS == 3 ? nv : 0][s] = blk[32 + (e >> 3)];
        }
      }
    }
  };
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * kDW + wave) * per;
  if (first < nvec) load_pass(first);
  for (int64_t v0 = first; v0 < nvec; v0 += gstride) {
    float sc[NV];
    int64_t obase[NV];
    bool live[NV];
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      const VecPos p = vec_pos(v0 + 16 * nv + n, nvec, static_cast<int>(a.tokens), a.heads);
      live[nv] = p.live;
      obase[nv] = p.b * a.sb + p.h * a.sh + static_cast<int64_t>(p.t) * a.st;
    }
    h8 bh[NV][NS], bl[NV][NS];
#pragma unroll
    for (int nv = 0; nv < NV; ++nv) {
      sc[nv] = live[nv] ? __builtin_amdgcn_ldexpf(__half2float(__ushort_as_half(nraw[nv])), -2 * kRShift)
                        : 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        uint4 eh, el;
        const uint32_t w = cw[nv][s];
        if constexpr (BITS == 4) {
          uint2 e[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) e[m] = ct[(w >> (8 * m)) & 0xFFu];
          eh = make_uint4(e[0].x, e[1].x, e[2].x, e[3].x);
          el = make_uint4(e[0].y, e[1].y, e[2].y, e[3].y);
        } else if constexpr (BITS == 2) {
          const uint4 e0 = ct[w & 0xFFu], e1 = ct[w >> 8];
          eh = make_uint4(e0.x, e0.y, e1.x, e1.y);
          el = make_uint4(e0.z, e0.w, e1.z, e1.w);
        } else {
          const uint32_t hb = ch[BITS == 3 ? nv : 0][s];
          uint2 t[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) t[m] = ct[((w >> (4 * m)) & 15u) | ((hb >> (2 * m)) & 3u) << 4];
          eh = make_uint4(t[0].x, t[1].x, t[2].x, t[3].x);
          el = make_uint4(t[0].y, t[1].y, t[2].y, t[3].y);
        }
        bh[nv][s] = __builtin_bit_cast(h8, eh);
        bl[nv][s] = __builtin_bit_cast(h8, el);
      }
    }
    if (v0 + gstride < nvec) load_pass(v0 + gstride);
    for (int o = 0; o < no; ++o) {
      f4 acc[NV], acc2[NV];
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) {
        acc[nv] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        acc2[nv] = f4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      const _Float16* ph = rh + (16 * o + n) * kRowH + 8 * g;
      const _Float16* pl = rl + (16 * o + n) * kRowH + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const h8 ah = *reinterpret_cast<const h8*>(ph + 32 * s);
        const h8 al = *reinterpret_cast<const h8*>(pl + 32 * s);
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) acc[nv] = mfma(ah, bh[nv][s], acc[nv]);
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) acc2[nv] = mfma(al, bh[nv][s], acc2[nv]);
#pragma unroll
        for (int nv = 0; nv < NV; ++nv) acc2[nv] = mfma(ah, bl[nv][s], acc2[nv]);
      }
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) acc[nv] += acc2[nv];
      const int j0 = 16 * o + 4 * g;   // outputs j0 .. j0 + 3 of vector 16 nv + n
#pragma unroll
      for (int nv = 0; nv < NV; ++nv) {
        if (!live[nv]) continue;
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = acc[nv][i] * sc[nv];
        if (a.out_bf16) {
          __hip_bfloat16* out = static_cast<__hip_bfloat16*>(a.out) + obase[nv] + j0;
          if (a.vec && j0 + 4 <= d) {
            uint32_t w[2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
              w[m] = static_cast<uint32_t>(__bfloat16_as_ushort(__float2bfloat16(x[2 * m]))) |
                     static_cast<uint32_t>(__bfloat16_as_ushort(__float2bfloat16(x[2 * m + 1]))) << 16;
            *reinterpret_cast<uint2*>(out) = make_uint2(w[0], w[1]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (j0 + i < d) out[i] = __float2bfloat16(x[i]);
          }
        } else {
          float* out = static_cast<float*>(a.out) + obase[nv] + j0;
          if (a.vec && j0 + 4 <= d) {
            *reinterpret_cast<float4*>(out) = make_float4(x[0], x[1], x[2], x[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (j0 + i < d) out[i] = x[i];
          }
        }
      }
    }
  }
}

// ---- attention over a dense-rotation cache: the query into the attention kernels'
// Walsh-Hadamard frame, and (after the vector-ALU kernels, whose merge leaves the
// result in that frame) the result out of it.  One workgroup per (sequence, query
// head); thread i owns element i of the 128-point frame.

__device__ __forceinline__ bool frame_sign(const DenseAttnLaunch& a, int i) {
  return (a.signs[i >> 5] >> (i & 31)) & 1u;
}

// y <- H y over the 128 elements in LDS (butterflies of strides 1 .. 64); threads with
// on == false only take part in the barriers
__device__ __forceinline__ void hadamard128(float* y, int i, bool on) {
#pragma unroll
  for (int L = 1; L < QK; L <<= 1) {
    float own = 0.0f, other = 0.0f;
    if (on) {
      own = y[i];
      other = y[i ^ L];
    }
    __syncthreads();
    if (on) y[i] = (i & L) ? other - own : own + other;
    __syncthreads();
  }
}

// q~ = R_w^-1 (R q) = D H (R q) / (128 c): R q zero-padded to 128, then H, the scale
// (1 / (128 c) = c up to the rounding of c) and the signs.  Wave w takes rows 32 w ..
// 32 w + 31 of R; lane l reads columns l and l + 64 of each (coalesced, all 64 loads in
// flight together; indexes clamped into R, the columns past d meet zeros of q, the rows
// past d are dropped), then a halving exchange over the lane bits 5 .. 1 leaves lanes
// 2r and 2r + 1 with row 32 w + r summed over 32 lanes, and one more exchange over
// bit 0 completes the sum.
// One halving step over lane bit 2S: of its 2S row partials v[0 .. 2S), a lane keeps
// the upper half when that bit is set (else the lower one), sends the other half to
// its partner and adds what it receives: v[0 .. S) then hold the kept rows summed over
// both lanes.
template <int S>
__device__ __forceinline__ void halve_rows(float* v, int lane) {
  const bool up = lane & (2 * S);
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const float send = up ? v[j] : v[j + S];
    const float keep = up ? v[j + S] : v[j];
    v[j] = keep + __shfl_xor(send, 2 * S);
  }
}

constexpr int kQueryThreads = 256;
__global__ void __launch_bounds__(kQueryThreads) dense_attn_query_kernel(DenseAttnLaunch a) {
  __shared__ float y[QK];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x, d = a.dim;
  const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform
  const int64_t row = static_cast<int64_t>(b) * a.hq + h;
  float q0 = 0.0f, q1 = 0.0f;
  if (a.q_is_bf16) {
    const uint16_t* qb = static_cast<const uint16_t*>(a.q) + row * d;
    if (lane < d) q0 = __uint_as_float(static_cast<uint32_t>(qb[lane]) << 16);
    if (lane + 64 < d) q1 = __uint_as_float(static_cast<uint32_t>(qb[lane + 64]) << 16);
  } else {
    const float* qf = static_cast<const float*>(a.q) + row * d;
    if (lane < d) q0 = qf[lane];
    if (lane + 64 < d) q1 = qf[lane + 64];
  }
  const uint32_t c0 = min(lane, d - 1), c1 = min(lane + 64, d - 1);
  float r0[32], r1[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float* rr = a.rot + min(32 * w + j, d - 1) * d;
    r0[j] = rr[c0];
    r1[j] = rr[c1];
  }
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = __builtin_fmaf(r1[j], q1, r0[j] * q0);
  halve_rows<16>(v, lane);
  halve_rows<8>(v, lane);
  halve_rows<4>(v, lane);
  halve_rows<2>(v, lane);
  halve_rows<1>(v, lane);
  const float sum = v[0] + __shfl_xor(v[0], 1);
  const int r = 32 * w + (lane >> 1);
  if ((lane & 1) == 0 && r < QK) y[r] = r < d ? sum : 0.0f;
  __syncthreads();
  hadamard128(y, t, t < QK);
  if (t < QK) {
    const float v2 = y[t] * kInvSqrtQK;
    a.qt[row * QK + t] = frame_sign(a, t) ? -v2 : v2;
  }
}

// out = R^T (R_w y) = R^T (c H (D y)): the first d elements of the frame's result
// (the others carry the centroids of the code-0 padding and are zeroed before the
// product).  Thread i reads column min(i, d - 1) of R, coalesced across the threads,
// all loads issued at once.
__global__ void __launch_bounds__(QK) dense_attn_out_kernel(DenseAttnLaunch a) {
  __shared__ float y[QK];
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x, d = a.dim;
  const int64_t row = static_cast<int64_t>(b) * a.hq + h;
  const float* c = a.rot + min(i, d - 1);
  float rv[QK];
#pragma unroll
  for (int k = 0; k < QK; ++k) rv[k] = c[static_cast<int64_t>(min(k, d - 1)) * d];
  const float v = a.y[row * QK + i];
  y[i] = frame_sign(a, i) ? -v : v;
  __syncthreads();
  hadamard128(y, i, true);
  y[i] = i < d ? y[i] * kInvSqrtQK : 0.0f;
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < QK; ++k) acc = __builtin_fmaf(rv[k], y[k], acc);
  if (i < d) a.out[row * d + i] = acc;
}

int dense_grid(int64_t nvec, int per_wave) {
  const int64_t per = static_cast<int64_t>(kDW) * per_wave;
  const int64_t want = (nvec + per - 1) / per;
  return static_cast<int>(want < 256 ? (want > 0 ? want : 1) : 256);
}

}  // namespace

template <int BITS, bool F32>
void enc_ns(const DenseLaunch& a, const KTable& tab, dim3 grid, hipStream_t stream) {
  const dim3 block(kDT);
  if (!(a.vec && a.dim % 8 == 0))
    hipLaunchKernelGGL((dense_encode_kernel<BITS, F32, kNS, false>), grid, block, 0, stream, a, tab);
  else if (a.dim <= 64)
    hipLaunchKernelGGL((dense_encode_kernel<BITS, F32, 2, true>), grid, block, 0, stream, a, tab);
  else if (a.dim <= 128)
    hipLaunchKernelGGL((dense_encode_kernel<BITS, F32, 4, true>), grid, block, 0, stream, a, tab);
  else
    hipLaunchKernelGGL((dense_encode_kernel<BITS, F32, kNS, true>), grid, block, 0, stream, a, tab);
}

template <int BITS>
void dec_ns(const DenseDecodeLaunch& a, const KTable& tab, dim3 grid, hipStream_t stream) {
  const dim3 block(kDT);
  if (a.dim <= 64)
    hipLaunchKernelGGL((dense_decode_kernel<BITS, 2>), grid, block, 0, stream, a, tab);
  else if (a.dim <= 128)
    hipLaunchKernelGGL((dense_decode_kernel<BITS, 4>), grid, block, 0, stream, a, tab);
  else
    hipLaunchKernelGGL((dense_decode_kernel<BITS, kNS>), grid, block, 0, stream, a, tab);
}

hipError_t launch_dense_encode(const DenseLaunch& a, const KTable& tab, hipStream_t stream) {
  const int64_t nvec = static_cast<int64_t>(a.batch) * a.heads * a.tokens;
  const dim3 grid(dense_grid(nvec, 16 * kNV));
  if (a.x_is_bf16) {
    switch (tab.bits) {
      case 2: enc_ns<2, false>(a, tab, grid, stream); break;
      case 3: enc_ns<3, false>(a, tab, grid, stream); break;
      default: enc_ns<4, false>(a, tab, grid, stream); break;
    }
  } else {
    switch (tab.bits) {
      case 2: enc_ns<2, true>(a, tab, grid, stream); break;
      case 3: enc_ns<3, true>(a, tab, grid, stream); break;
      default: enc_ns<4, true>(a, tab, grid, stream); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_dense_attn_query(const DenseAttnLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(dense_attn_query_kernel, dim3(a.hq, a.batch), dim3(kQueryThreads), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_dense_attn_out(const DenseAttnLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(dense_attn_out_kernel, dim3(a.hq, a.batch), dim3(QK), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const DenseDecodeLaunch& a, const KTable& tab,
                               hipStream_t stream) {
  const dim3 grid(dense_grid(a.rows * a.tokens, 16 * kNV));
  switch (tab.bits) {
    case 2: dec_ns<2>(a, tab, grid, stream); break;
    case 3: dec_ns<3>(a, tab, grid, stream); break;
    default: dec_ns<4>(a, tab, grid, stream); break;
  }
  return hipGetLastError();
}

}  // namespace fatq

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

#include "fa_tq_internal.h"

namespace fatq {
namespace {

constexpr int kThreads = 256;

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

// Butterfly across lanes: the lower lane of the pair keeps u + v, the upper one
// v_lower - v_upper (the same (u + v, u - v) pair, computed in the owning lane).
__device__ __forceinline__ float xbfly(float x, int mask, bool upper) {
  const float p = __shfl_xor(x, mask, 64);
  return upper ? (p - x) : (x + p);
}

// Unscaled Walsh-Hadamard transform of one block in quad layout, stage order
// len = 1, 2, 4, 8, 16, 32, 64.
__device__ __forceinline__ void fwht_quad(float (&v)[4][8], int q) {
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
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[k][i] = xbfly(v[k][i], 1, q & 1);
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) v[k][i] = xbfly(v[k][i], 2, (q & 2) != 0);
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
}

// Canonical fp32 norm: squares summed pairwise over index bits 0, 1, ..., 6.
__device__ __forceinline__ float norm_quad(const float (&x)[4][8]) {
  float p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = x[k][i] * x[k][i];
    const float a0 = s[0] + s[1], a1 = s[2] + s[3], a2 = s[4] + s[5], a3 = s[6] + s[7];
    const float b0 = a0 + a1, b1 = a2 + a3;
    p[k] = b0 + b1;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = p[k] + __shfl_xor(p[k], 1, 64);
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = p[k] + __shfl_xor(p[k], 2, 64);
  const float c0 = p[0] + p[1], c1 = p[2] + p[3];
  return __builtin_sqrtf(c0 + c1);
}

template <bool BF16>
__device__ __forceinline__ void load_block(const void* base, int64_t off, int q,
                                           float (&x)[4][8]) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    uint4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = p[q + 4 * k];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t d[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[k][2 * m] = __uint_as_float(d[m] << 16);
        x[k][2 * m + 1] = __uint_as_float(d[m] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    float4 w[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      w[2 * k] = p[2 * (q + 4 * k)];
      w[2 * k + 1] = p[2 * (q + 4 * k) + 1];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k][0] = w[2 * k].x; x[k][1] = w[2 * k].y; x[k][2] = w[2 * k].z; x[k][3] = w[2 * k].w;
      x[k][4] = w[2 * k + 1].x; x[k][5] = w[2 * k + 1].y;
      x[k][6] = w[2 * k + 1].z; x[k][7] = w[2 * k + 1].w;
    }
  }
}

// Pack the 8 codes of chunk c of one block and store them at the packed row
// ([Spec] "Step 3: Packing", least-significant field first; 3 bits as the split
// planes of [turboq] block_turboq3_0).
template <int BITS>
__device__ __forceinline__ void store_chunk(uint8_t* row, int c, const uint32_t (&code)[8]) {
  if constexpr (BITS == 4) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= code[i] << (4 * i);
    reinterpret_cast<uint32_t*>(row)[c] = w;
  } else if constexpr (BITS == 2) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= code[i] << (2 * i);
    reinterpret_cast<uint16_t*>(row)[c] = static_cast<uint16_t>(w);
  } else if constexpr (BITS == 3) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo |= (code[i] & 3u) << (2 * i);
      hi |= ((code[i] >> 2) & 1u) << i;
    }
    reinterpret_cast<uint16_t*>(row)[c] = static_cast<uint16_t>(lo);
    row[32 + c] = static_cast<uint8_t>(hi);
  } else {
    uint2 w;
    w.x = code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24;
    w.y = code[4] | code[5] << 8 | code[6] << 16 | code[7] << 24;
    reinterpret_cast<uint2*>(row)[c] = w;
  }
}

template <int BITS>
__device__ __forceinline__ void load_chunk(const uint8_t* row, int c, uint32_t (&code)[8]) {
  if constexpr (BITS == 4) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = (w >> (4 * i)) & 15u;
  } else if constexpr (BITS == 2) {
    const uint32_t w = reinterpret_cast<const uint16_t*>(row)[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = (w >> (2 * i)) & 3u;
  } else if constexpr (BITS == 3) {
    const uint32_t lo = reinterpret_cast<const uint16_t*>(row)[c];
    const uint32_t hi = row[32 + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = ((lo >> (2 * i)) & 3u) | (((hi >> i) & 1u) << 2);
  } else {
    const uint2 w = reinterpret_cast<const uint2*>(row)[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      code[i] = (w.x >> (8 * i)) & 255u;
      code[4 + i] = (w.y >> (8 * i)) & 255u;
    }
  }
}

template <int BITS>
constexpr int code_bytes_of() {
  return BITS == 2 ? 32 : BITS == 3 ? 48 : BITS == 4 ? 64 : 128;
}

// Encode: one quad per 128-block, grid-stride over blocks.  The number of quads in
// the grid is a multiple of nblk, so each quad keeps one sign slice j.
template <int BITS, bool BF16>
__global__ void __launch_bounds__(kThreads) encode_kernel(EncodeLaunch a, KTable tab,
                                                          SignWords sw) {
  constexpr int CB = code_bytes_of<BITS>();
  const int q = threadIdx.x & 3;
  const int64_t quad0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 2;
  const int64_t nquad = (static_cast<int64_t>(gridDim.x) * kThreads) >> 2;
  const int64_t total = static_cast<int64_t>(a.batch) * a.heads * a.tokens * a.nblk;
  const int j = static_cast<int>(quad0 % a.nblk);
  const uint32_t sbits = sw.w[j][q];

  for (int64_t blk = quad0; blk < total; blk += nquad) {
    int64_t v = blk / a.nblk;
    const int t = static_cast<int>(v % a.tokens);
    v /= a.tokens;
    const int h = static_cast<int>(v % a.heads);
    const int b = static_cast<int>(v / a.heads);
    const int tt = (a.t0 ? a.t0[b] : 0) + t;
    if (tt < 0 || tt >= a.t_max) continue;
    const int64_t xoff = b * a.sb + h * a.sh + t * a.st + static_cast<int64_t>(QK) * j;

    float x[4][8];
    load_block<BF16>(a.x, xoff, q, x);
    const float n32 = norm_quad(x);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[k][i] = flip_sign(x[k][i], (sbits >> (8 * k + i)) & 1u);
    fwht_quad(x, q);

    const int64_t row = ((static_cast<int64_t>(b) * a.heads + h) * a.t_max + tt) * a.nblk + j;
    uint8_t* crow = a.codes + row * CB;
    uint16_t nbits;
    if constexpr (BITS == 8) {
      // turboq8 grid: per-block absmax scale, codes round((y / s) * 127.5 + 127.5)
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[k][i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const __half s16 = __float2half_rn(fp32_value(amax * kInvSqrtQK));
      const float s32 = __half2float(s16);
      const float G = s32 > 0.0f ? kGrid8 / s32 : 0.0f;
      nbits = __half_as_ushort(s16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t8 = x[k][i] * G;
          const float w = t8 + 127.5f;
          code[i] = static_cast<uint32_t>(fminf(fmaxf(rintf(w), 0.0f), 255.0f));
        }
        store_chunk<8>(crow, q + 4 * k, code);
      }
    } else {
      const float g = n32 > 0.0f ? kInvSqrtQK / n32 : 0.0f;
      nbits = __half_as_ushort(__float2half_rn(n32));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t code[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u = x[k][i] * g;
          uint32_t cnt = 0;
#pragma unroll
          for (int m = 0; m < (1 << BITS) - 1; ++m) cnt += tab.b[m] < u ? 1u : 0u;
          code[i] = cnt;
        }
        store_chunk<BITS>(crow, q + 4 * k, code);
      }
    }
    if (q == 0) a.norms[row] = nbits;
  }
}

// Decode: x_hat = s * (H (n * c[code])) / sqrt(128), one quad per block.
template <int BITS>
__global__ void __launch_bounds__(kThreads) decode_kernel(const uint8_t* codes,
                                                          const uint16_t* norms,
                                                          int64_t nblocks, int nblk, float* out,
                                                          KTable tab, SignWords sw) {
  constexpr int CB = code_bytes_of<BITS>();
  __shared__ float cent[16];
  if (threadIdx.x < 16) cent[threadIdx.x] = tab.c[threadIdx.x];
  __syncthreads();
  const int q = threadIdx.x & 3;
  const int64_t quad0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 2;
  const int64_t nquad = (static_cast<int64_t>(gridDim.x) * kThreads) >> 2;
  const int j = static_cast<int>(quad0 % nblk);
  const uint32_t sbits = sw.w[j][q];
  for (int64_t blk = quad0; blk < nblocks; blk += nquad) {
    const uint8_t* crow = codes + blk * CB;
    const float n = __half2float(__ushort_as_half(norms[blk]));
    float v[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t code[8];
      load_chunk<BITS>(crow, q + 4 * k, code);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (BITS == 8)
          v[k][i] = (static_cast<float>(code[i]) - 127.5f) * (n / 127.5f);
        else
          v[k][i] = n * cent[code[i]];
      }
    }
    fwht_quad(v, q);
    float4* o = reinterpret_cast<float4*>(out + blk * QK);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        r[i] = flip_sign(v[k][i] * kInvSqrtQK, (sbits >> (8 * k + i)) & 1u);
      const int c = q + 4 * k;
      o[2 * c] = make_float4(r[0], r[1], r[2], r[3]);
      o[2 * c + 1] = make_float4(r[4], r[5], r[6], r[7]);
    }
  }
}

int grid_for(int64_t blocks) {
  const int64_t quads_per_wg = kThreads / 4;
  int64_t g = (blocks + quads_per_wg - 1) / quads_per_wg;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_encode(const EncodeLaunch& a, const KTable& tab, const SignWords& sw,
                         hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(a.batch) * a.heads * a.tokens * a.nblk;
  const dim3 grid(grid_for(total)), block(kThreads);
#define FATQ_ENC(B, F) \
  hipLaunchKernelGGL((encode_kernel<B, F>), grid, block, 0, stream, a, tab, sw)
  if (a.x_is_bf16) {
    switch (tab.bits) {
      case 2: FATQ_ENC(2, true); break;
      case 3: FATQ_ENC(3, true); break;
      case 4: FATQ_ENC(4, true); break;
      default: FATQ_ENC(8, true); break;
    }
  } else {
    switch (tab.bits) {
      case 2: FATQ_ENC(2, false); break;
      case 3: FATQ_ENC(3, false); break;
      case 4: FATQ_ENC(4, false); break;
      default: FATQ_ENC(8, false); break;
    }
  }
#undef FATQ_ENC
  return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* codes, const uint16_t* norms, int64_t n_vec,
                         int32_t nblk, float* out, const KTable& tab, const SignWords& sw,
                         hipStream_t stream) {
  const int64_t nblocks = n_vec * nblk;
  const dim3 grid(grid_for(nblocks)), block(kThreads);
  switch (tab.bits) {
    case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, codes, norms, nblocks, nblk, out, tab, sw); break;
    case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, codes, norms, nblocks, nblk, out, tab, sw); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, codes, norms, nblocks, nblk, out, tab, sw); break;
    default: hipLaunchKernelGGL(decode_kernel<8>, grid, block, 0, stream, codes, norms, nblocks, nblk, out, tab, sw); break;
  }
  return hipGetLastError();
}

}  // namespace fatq

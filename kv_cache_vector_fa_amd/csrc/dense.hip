// Encode and decode with a dense random orthogonal rotation, for head_dims that are not
// a power of two (gfx950).
//
// Page cited: [Spec] "TurboQuant KV Cache Compression -- Spec", "Hadamard Transform
// Detail" (for a head_dim that is not a power of two: a dense random orthogonal matrix
// instead of padding to the next power of two) and "Step 1: Random Orthogonal
// Rotation" (rotate(x) = R x with a fixed d x d orthogonal R from the seed).
//
// The rotation is a d x d matrix-vector product per vector (d^2 multiply-adds instead
// of the Walsh-Hadamard transform's d log2 d adds), d <= 192 so that R fits in LDS.
// Work layout: one workgroup per compute unit (4 waves) loops over groups of 4
// vectors per wave.  Encode: R^T in LDS (rt[j][i] = R[i][j], so the lanes of one
// wave read consecutive words for a fixed j); a wave stages its 4 input vectors in
// LDS as fp32 [j][v] (one 16-byte broadcast read per j) and each lane accumulates the
// outputs i = lane, lane + 64, lane + 128 of the 4 vectors in fp32, j ascending.
// The norm is the canonical fp32 norm of the vector zero-padded to a power of two
// (squares summed pairwise over index bits 0, 1, ...: bits 0-5 across the lanes,
// bits 6-7 in-lane).  Codes u = y / n against the boundaries of the dim-d codebook
// (code = #{j : b_j < u}); the codes of the d coordinates fill ceil(d / 128) packed
// blocks, code 0 past d; one fp16 norm per vector.  Decode is the transpose: R in
// LDS (r[i][j]), the values n16 * c[code_i] staged as fp32 [i][v].

#include <hip/hip_bf16.h>
#include <hip/hip_fp16.h>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

constexpr int kDWaves = 4;
constexpr int kDThreads = 64 * kDWaves;
constexpr int kDV = 4;   // vectors per wave per pass

template <int B>
constexpr int dense_cbytes() { return B == 2 ? 32 : B == 3 ? 48 : 64; }

// LDS visibility of one wave's own writes to its later reads (no other wave shares
// the region): wait for the wave's LDS operations, then a wave-level barrier.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, bool bf16) {
  if (bf16) {
    const uint16_t h = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
  return static_cast<const float*>(base)[idx];
}

// One 16-byte LDS word per (j, lane group) of the staging area: [j][v] fp32.
struct Stage {
  float v[kDV];
};

template <int BITS>
__global__ void __launch_bounds__(kDThreads) dense_encode_kernel(DenseLaunch a, KTable tab) {
  __shared__ float rt[kDenseMax * kDenseMax];
  __shared__ __attribute__((aligned(16))) Stage xs[kDWaves][kDenseMax];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.dim;
  const int nk = (d + 63) >> 6;   // outputs per lane: i = lane + 64 k, k < nk
  // R^T into LDS (R row-major in global memory)
  for (int e = tid; e < d * d; e += kDThreads) {
    const int i = e / d, j = e - i * d;
    rt[j * d + i] = a.rot[e];
  }
  __syncthreads();

  constexpr int CB = dense_cbytes<BITS>();
  const int64_t nvec = static_cast<int64_t>(a.batch) * a.heads * a.tokens;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * kDWaves * kDV;
  for (int64_t v0 = (static_cast<int64_t>(blockIdx.x) * kDWaves + wave) * kDV; v0 < nvec;
       v0 += gstride) {
    // ---- stage the 4 vectors (fp32) and their canonical norms
    float n32[kDV];
    int64_t slot[kDV];   // cache slot index (row * t_max + position), -1: nothing stored
#pragma unroll
    for (int v = 0; v < kDV; ++v) {
      const int64_t gv = v0 + v;
      const bool live = gv < nvec;
      int64_t row = 0;
      int t = 0;
      if (live) {
        row = gv / a.tokens;
        t = static_cast<int>(gv - row * a.tokens);
      }
      const int b = static_cast<int>(row / a.heads), h = static_cast<int>(row - (row / a.heads) * a.heads);
      const int64_t base = live ? b * a.sb + h * a.sh + static_cast<int64_t>(t) * a.st : 0;
      float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        float x = 0.0f;
        if (live && j < d) x = load_elem(a.x, base + j, a.x_is_bf16);
        if (j < d) xs[wave][j].v[v] = x;
        s[k] = x * x;
      }
      // canonical pairwise sum: index bits 0-5 across lanes (a + b == b + a in fp32),
      // then bits 6 and 7 in-lane (s[3] is the zero padding)
#pragma unroll
      for (int L = 1; L < 64; L <<= 1) {
#pragma unroll
        for (int k = 0; k < 3; ++k) s[k] = s[k] + __shfl_xor(s[k], L, 64);
      }
      const float ss = (s[0] + s[1]) + (s[2] + s[3]);
      n32[v] = __builtin_sqrtf(ss);
      const int64_t pos = static_cast<int64_t>(a.t0 ? a.t0[live ? b : 0] : 0) + t;
      slot[v] = live && pos >= 0 && pos < a.t_max ? row * a.t_max + pos : -1;
    }
    wave_lds_sync();
    // ---- y = R x for the 4 vectors: y[k][v] for output i = lane + 64 k
    float y[3][kDV];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int v = 0; v < kDV; ++v) y[k][v] = 0.0f;
#pragma unroll 4
    for (int j = 0; j < d; ++j) {
      const Stage xv = xs[wave][j];
      const float* rj = rt + j * d + lane;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < nk) {
          const float r = lane + 64 * k < d ? rj[64 * k] : 0.0f;
#pragma unroll
          for (int v = 0; v < kDV; ++v) y[k][v] = __builtin_fmaf(r, xv.v[v], y[k][v]);
        }
      }
    }
    wave_lds_sync();   // every lane is done with xs before it is reused for the codes
    // ---- codes into LDS (one byte per coordinate, 0 past d), then packed and stored
    uint8_t* cs = reinterpret_cast<uint8_t*>(&xs[wave][0]);   // [v][256] bytes
#pragma unroll
    for (int v = 0; v < kDV; ++v) {
      const float g = n32[v] > 0.0f ? 1.0f / n32[v] : 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = lane + 64 * k;
        uint32_t code = 0;
        if (k < 3 && i < d) {
          const float u = y[k][v] * g;
          // the boundaries past nb are +inf (never below u)
#pragma unroll
          for (int q = 0; q < 15; ++q) code += u > tab.b[q] ? 1u : 0u;
        }
        cs[v * 256 + i] = static_cast<uint8_t>(code);
      }
    }
    wave_lds_sync();
    const int nblk = a.nblk;
#pragma unroll
    for (int v = 0; v < kDV; ++v) {
      if (slot[v] < 0) continue;   // uniform over the wave
      uint8_t* dst = a.codes + slot[v] * nblk * CB;
      const uint8_t* src = cs + v * 256;
      if constexpr (BITS == 4) {
        // word w (16 per block): codes 8w .. 8w + 7, low nibble first
        for (int w = lane; w < 16 * nblk; w += 64) {
          uint32_t word = 0;
#pragma unroll
          for (int m = 0; m < 8; ++m) word |= static_cast<uint32_t>(src[8 * w + m]) << (4 * m);
          reinterpret_cast<uint32_t*>(dst)[w] = word;
        }
      } else if constexpr (BITS == 2) {
        // word w (8 per block): codes 16w .. 16w + 15, 2 bits each
        for (int w = lane; w < 8 * nblk; w += 64) {
          uint32_t word = 0;
#pragma unroll
          for (int m = 0; m < 16; ++m) word |= static_cast<uint32_t>(src[16 * w + m]) << (2 * m);
          reinterpret_cast<uint32_t*>(dst)[w] = word;
        }
      } else {
        // 3-bit ([turboq] block_turboq3_0): per block 32 bytes of low 2-bit fields
        // (4 per byte), then 16 bytes of high bits (8 per byte); words of 4 bytes
        for (int w = lane; w < 12 * nblk; w += 64) {
          const int blk = w / 12, r = w - blk * 12;
          const uint8_t* c = src + 128 * blk;
          uint32_t word = 0;
          if (r < 8) {
#pragma unroll
            for (int m = 0; m < 16; ++m) word |= static_cast<uint32_t>(c[16 * r + m] & 3u) << (2 * m);
          } else {
#pragma unroll
            for (int m = 0; m < 32; ++m)
              word |= static_cast<uint32_t>((c[32 * (r - 8) + m] >> 2) & 1u) << m;
          }
          reinterpret_cast<uint32_t*>(dst + blk * CB)[r] = word;
        }
      }
      if (lane == 0) a.norms[slot[v]] = __half_as_ushort(__float2half_rn(n32[v]));
    }
    wave_lds_sync();   // the codes are read before the next pass stages its vectors
  }
}

template <int BITS>
__global__ void __launch_bounds__(kDThreads) dense_decode_kernel(DenseDecodeLaunch a, KTable tab) {
  __shared__ float r[kDenseMax * kDenseMax];
  __shared__ __attribute__((aligned(16))) Stage vs[kDWaves][kDenseMax];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.dim;
  const int nk = (d + 63) >> 6;
  for (int e = tid; e < d * d; e += kDThreads) r[e] = a.rot[e];
  __syncthreads();

  constexpr int CB = dense_cbytes<BITS>();
  const int64_t nvec = a.rows * a.tokens;
  const int64_t gstride = static_cast<int64_t>(gridDim.x) * kDWaves * kDV;
  for (int64_t v0 = (static_cast<int64_t>(blockIdx.x) * kDWaves + wave) * kDV; v0 < nvec;
       v0 += gstride) {
    int64_t obase[kDV];
    bool live[kDV];
#pragma unroll
    for (int v = 0; v < kDV; ++v) {
      const int64_t gv = v0 + v;
      live[v] = gv < nvec;
      const int64_t row = live[v] ? gv / a.tokens : 0;
      const int64_t t = live[v] ? gv - row * a.tokens : 0;
      const int64_t slot = row * a.t_max + t;
      const int b = static_cast<int>(row / a.heads), h = static_cast<int>(row - (row / a.heads) * a.heads);
      obase[v] = b * a.sb + h * a.sh + t * a.st;
      const uint8_t* src = a.codes + slot * a.nblk * CB;
      const float n = live[v] ? __half2float(__ushort_as_half(a.norms[slot])) : 0.0f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int i = lane + 64 * k;
        if (i < d) {
          uint32_t code = 0;
          if (live[v]) {
            const int blk = i >> 7, e = i & 127;
            const uint8_t* c = src + blk * CB;
            if constexpr (BITS == 4) code = (c[e >> 1] >> (4 * (e & 1))) & 15u;
            else if constexpr (BITS == 2) code = (c[e >> 2] >> (2 * (e & 3))) & 3u;
            else code = ((c[e >> 2] >> (2 * (e & 3))) & 3u) | (((c[32 + (e >> 3)] >> (e & 7)) & 1u) << 2);
          }
          vs[wave][i].v[v] = live[v] ? n * tab.c[code] : 0.0f;
        }
      }
    }
    wave_lds_sync();
    float x[3][kDV];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int v = 0; v < kDV; ++v) x[k][v] = 0.0f;
    // x_hat[j] = sum_i R[i][j] * (n c[code_i]), j = lane + 64 k, i ascending
#pragma unroll 4
    for (int i = 0; i < d; ++i) {
      const Stage cv = vs[wave][i];
      const float* ri = r + i * d + lane;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        if (k < nk) {
          const float rr = lane + 64 * k < d ? ri[64 * k] : 0.0f;
#pragma unroll
          for (int v = 0; v < kDV; ++v) x[k][v] = __builtin_fmaf(rr, cv.v[v], x[k][v]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < kDV; ++v) {
      if (!live[v]) continue;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int j = lane + 64 * k;
        if (j < d) {
          if (a.out_bf16) {
            const __hip_bfloat16 o = __float2bfloat16(x[k][v]);
            static_cast<__hip_bfloat16*>(a.out)[obase[v] + j] = o;
          } else {
            static_cast<float*>(a.out)[obase[v] + j] = x[k][v];
          }
        }
      }
    }
    wave_lds_sync();   // vs is read before the next pass overwrites it
  }
}

int dense_grid(int64_t nvec) {
  const int64_t per = static_cast<int64_t>(kDWaves) * kDV;
  const int64_t want = (nvec + per - 1) / per;
  return static_cast<int>(want < 256 ? (want > 0 ? want : 1) : 256);
}

}  // namespace

hipError_t launch_dense_encode(const DenseLaunch& a, const KTable& tab, hipStream_t stream) {
  const int64_t nvec = static_cast<int64_t>(a.batch) * a.heads * a.tokens;
  const dim3 grid(dense_grid(nvec)), block(kDThreads);
  switch (tab.bits) {
    case 2: hipLaunchKernelGGL(dense_encode_kernel<2>, grid, block, 0, stream, a, tab); break;
    case 3: hipLaunchKernelGGL(dense_encode_kernel<3>, grid, block, 0, stream, a, tab); break;
    default: hipLaunchKernelGGL(dense_encode_kernel<4>, grid, block, 0, stream, a, tab); break;
  }
  return hipGetLastError();
}

hipError_t launch_dense_decode(const DenseDecodeLaunch& a, const KTable& tab,
                               hipStream_t stream) {
  const dim3 grid(dense_grid(a.rows * a.tokens)), block(kDThreads);
  switch (tab.bits) {
    case 2: hipLaunchKernelGGL(dense_decode_kernel<2>, grid, block, 0, stream, a, tab); break;
    case 3: hipLaunchKernelGGL(dense_decode_kernel<3>, grid, block, 0, stream, a, tab); break;
    default: hipLaunchKernelGGL(dense_decode_kernel<4>, grid, block, 0, stream, a, tab); break;
  }
  return hipGetLastError();
}

}  // namespace fatq

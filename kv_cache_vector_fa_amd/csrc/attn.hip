// Decode attention over the packed cache, gfx950.
//
// Page cited: [Spec] "TurboQuant KV Cache Compression -- Spec", section
// "Optimization: Fused dequant-dot": rotate the query once, dot it with centroid
// look-ups of the cached keys (never inverse-rotating a cached vector), accumulate
// the weighted value look-ups in the rotated domain, inverse-rotate the output once.
//
// Two kernels per call:
//   attn_split_kernel  grid (ceil(n_split / 4), Hkv, B), 4 waves per workgroup; wave w
//                      owns split s = 4 blockIdx.x + w, i.e. tokens
//                      [s * chunk, min(len, (s + 1) * chunk)) of KV head g, for all
//                      query heads of the group.  It keeps an online softmax and writes
//                      the partial (m, l, o') of each head to the workspace.
//   attn_merge_kernel  grid (Hq, B): log-sum-exp merge of the splits, 1/l, inverse
//                      rotation R^T = D H / sqrt(128), fp32 output.
// Scores are kept in base 2: s2 = s * log2(e), so exp() becomes exp2().

#include <hip/hip_fp16.h>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 64;        // tokens per wave tile
constexpr int kMaxGroup = 16;    // query heads per KV head
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

template <int BITS>
constexpr int cbytes() {
  return BITS == 2 ? 32 : BITS == 3 ? 48 : 64;
}

// Codes of elements 16*sl .. 16*sl + 15 of one packed 128-block.
template <int BITS>
__device__ __forceinline__ void codes16(const uint8_t* row, int sl, uint32_t (&c)[16]) {
  if constexpr (BITS == 4) {
    const uint2 w = reinterpret_cast<const uint2*>(row)[sl];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      c[i] = (w.x >> (4 * i)) & 15u;
      c[8 + i] = (w.y >> (4 * i)) & 15u;
    }
  } else if constexpr (BITS == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(row)[sl];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = (w >> (2 * i)) & 3u;
  } else {
    const uint32_t lo = reinterpret_cast<const uint32_t*>(row)[sl];
    const uint32_t hi = reinterpret_cast<const uint16_t*>(row + 32)[sl];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = ((lo >> (2 * i)) & 3u) | (((hi >> i) & 1u) << 2);
  }
}

// Codes of elements 2p and 2p + 1 of one packed 128-block.
template <int BITS>
__device__ __forceinline__ void codes2(const uint8_t* row, int p, uint32_t& c0, uint32_t& c1) {
  if constexpr (BITS == 4) {
    const uint32_t w = row[p];
    c0 = w & 15u;
    c1 = w >> 4;
  } else if constexpr (BITS == 2) {
    const uint32_t w = row[p >> 1] >> (4 * (p & 1));
    c0 = w & 3u;
    c1 = (w >> 2) & 3u;
  } else {
    const uint32_t lo = row[p >> 1] >> (4 * (p & 1));
    const uint32_t hi = row[32 + (p >> 2)] >> (2 * (p & 3));
    c0 = (lo & 3u) | ((hi & 1u) << 2);
    c1 = ((lo >> 2) & 3u) | (((hi >> 1) & 1u) << 2);
  }
}

__device__ __forceinline__ bool sign_neg(const SignWords& sw, int e) {
  const int q = (e >> 3) & 3, k = e >> 5, i = e & 7;
  return (sw.w[0][q] >> (8 * k + i)) & 1u;
}
// The second sign vector s2 (R = D2 H D1 / sqrt(128)); +1 everywhere without it.
__device__ __forceinline__ bool sign2_neg(const SignWords& sw, int e) {
  const int q = (e >> 3) & 3, k = e >> 5, i = e & 7;
  return sw.two && ((sw.w2[0][q] >> (8 * k + i)) & 1u);
}

template <int KB, int VB>
__global__ void __launch_bounds__(kWaves * 64) attn_split_kernel(AttnLaunch a, KTable tk,
                                                                 KTable tv, SignWords sw) {
  constexpr int KCB = cbytes<KB>(), VCB = cbytes<VB>();
  __shared__ float qr[kMaxGroup][QK];
  __shared__ float centk[16], centv[16];
  __shared__ float wt[kWaves][kMaxGroup][kTile];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kWaves][kTile][VCB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = a.hq / a.hkv;

  // Rotate the group's queries once: q' = s2 * H (s * q) / sqrt(128).
  if (tid < 16) {
    centk[tid] = tk.c[tid];
    centv[tid] = tv.c[tid];
  }
  for (int idx = tid; idx < G * QK; idx += kWaves * 64) {
    const int h = idx / QK, e = idx % QK;
    const int64_t qo = (static_cast<int64_t>(b) * a.hq + g * G + h) * QK + e;
    float v = a.q_is_bf16
                  ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(a.q)[qo]) << 16)
                  : static_cast<const float*>(a.q)[qo];
    qr[h][e] = sign_neg(sw, e) ? -v : v;
  }
  __syncthreads();
  for (int len = 1; len < QK; len <<= 1) {
    for (int idx = tid; idx < G * (QK / 2); idx += kWaves * 64) {
      const int h = idx / (QK / 2), p = idx % (QK / 2);
      const int i = (p / len) * 2 * len + (p % len);
      const float u = qr[h][i], v = qr[h][i + len];
      qr[h][i] = u + v;
      qr[h][i + len] = u - v;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < G * QK; idx += kWaves * 64)
    qr[idx / QK][idx % QK] *= sign2_neg(sw, idx % QK) ? -kInvSqrtQK : kInvSqrtQK;
  __syncthreads();

  const int split = blockIdx.x * kWaves + wave;
  if (split >= a.n_split) return;
  const int64_t len64 = a.pos ? static_cast<int64_t>(a.pos[b]) + a.n_new : a.seq_lens[b];
  const int len = len64 < 0 ? 0 : (len64 > a.t_max ? a.t_max : static_cast<int>(len64));
  const int t_begin = split * a.chunk;
  const int t_end = min(len, t_begin + a.chunk);
  const float sc2 = a.scale * kLog2e;

  const int64_t kv_base = (static_cast<int64_t>(b) * a.hkv + g) * a.t_max;
  const uint8_t* kc = a.k_codes + kv_base * KCB;
  const uint8_t* vc = a.v_codes + kv_base * VCB;
  const uint16_t* kn = a.k_norms + kv_base;
  const uint16_t* vn = a.v_norms + kv_base;

  float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][2];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
    acc[h][0] = acc[h][1] = 0.0f;
  }

  const int tok8 = lane >> 3, sl = lane & 7;
  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    // Scores: 8 lanes per token, each over 16 elements, then a reduction.
    for (int step = 0; step < kTile / 8; ++step) {
      const int tl = step * 8 + tok8;
      const int t = t0 + tl;
      float dot[kMaxGroup];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) dot[h] = 0.0f;
      if (t < t_end) {
        uint32_t c[16];
        codes16<KB>(kc + static_cast<int64_t>(t) * KCB, sl, c);
        float kv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) kv[i] = centk[c[i]];
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h < G) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s += qr[h][16 * sl + i] * kv[i];
            dot[h] = s;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          float s = dot[h];
          s += __shfl_xor(s, 1, 64);
          s += __shfl_xor(s, 2, 64);
          s += __shfl_xor(s, 4, 64);
          if (sl == 0)
            wt[wave][h][tl] = t < t_end ? s * half_bits_to_float(kn[t]) * sc2 : -INFINITY;
        }
      }
    }
    // Stage this tile's value codes: lane = token.
    {
      const int t = t0 + lane;
      if (t < t_end) {
        const uint4* src = reinterpret_cast<const uint4*>(vc + static_cast<int64_t>(t) * VCB);
        uint4* dst = reinterpret_cast<uint4*>(&vt[wave][lane][0]);
#pragma unroll
        for (int k = 0; k < VCB / 16; ++k) dst[k] = src[k];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    // Online softmax over the tile (lane = token).
    const int t = t0 + lane;
    const float nv = t < t_end ? half_bits_to_float(vn[t]) : 0.0f;
    float alpha[kMaxGroup];
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      alpha[h] = 1.0f;
      if (h < G) {
        const float s = wt[wave][h][lane];
        const float mt = wave_max(s);
        const float mn = fmaxf(m[h], mt);
        alpha[h] = exp2f(m[h] - mn);
        const float p = t < t_end ? exp2f(s - mn) : 0.0f;
        l[h] = l[h] * alpha[h] + wave_sum(p);
        m[h] = mn;
        wt[wave][h][lane] = p * nv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // Values: lane owns rotated-domain elements 2*lane, 2*lane + 1.
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      acc[h][0] *= alpha[h];
      acc[h][1] *= alpha[h];
    }
    const int nt = min(kTile, t_end - t0);
    for (int tt = 0; tt < nt; ++tt) {
      uint32_t c0, c1;
      codes2<VB>(&vt[wave][tt][0], lane, c0, c1);
      const float v0 = centv[c0], v1 = centv[c1];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) {
        if (h < G) {
          const float w = wt[wave][h][tt];
          acc[h][0] += w * v0;
          acc[h][1] += w * v1;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  float* ws_o = static_cast<float*>(a.workspace);
  float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * a.n_split * QK;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      const int64_t r = (static_cast<int64_t>(b) * a.hq + g * G + h) * a.n_split + split;
      reinterpret_cast<float2*>(ws_o + r * QK)[lane] = make_float2(acc[h][0], acc[h][1]);
      if (lane == 0) {
        ws_ml[2 * r] = m[h];
        ws_ml[2 * r + 1] = l[h];
      }
    }
  }
}

__global__ void __launch_bounds__(QK) attn_merge_kernel(AttnLaunch a, SignWords sw) {
  __shared__ float o[QK];
  __shared__ float red[QK];
  const int h = blockIdx.x, b = blockIdx.y, e = threadIdx.x;
  const float* ws_o = static_cast<const float*>(a.workspace);
  const float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * a.n_split * QK;
  const int64_t r0 = (static_cast<int64_t>(b) * a.hq + h) * a.n_split;
  float mx = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) mx = fmaxf(mx, ws_ml[2 * (r0 + s)]);
  float num = 0.0f, den = 0.0f;
  if (mx > -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const float ms = ws_ml[2 * (r0 + s)];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - mx);
      den += w * ws_ml[2 * (r0 + s) + 1];
      num += w * ws_o[(r0 + s) * QK + e];
    }
  }
  const float oe = den > 0.0f ? num / den : 0.0f;
  o[e] = sign2_neg(sw, e) ? -oe : oe;
  __syncthreads();
  for (int len = 1; len < QK; len <<= 1) {
    float u = 0.0f, v = 0.0f;
    int i = 0;
    if (e < QK / 2) {
      i = (e / len) * 2 * len + (e % len);
      u = o[i];
      v = o[i + len];
    }
    __syncthreads();
    if (e < QK / 2) {
      o[i] = u + v;
      o[i + len] = u - v;
    }
    __syncthreads();
  }
  const float r = o[e] * kInvSqrtQK;
  a.out[(static_cast<int64_t>(b) * a.hq + h) * QK + e] = sign_neg(sw, e) ? -r : r;
  (void)red;
}

}  // namespace

void attn_partition(int32_t batch, int32_t hkv, int32_t t_max, int32_t* n_split,
                    int32_t* chunk) {
  const int64_t units = static_cast<int64_t>(batch > 0 ? batch : 1) * hkv;
  const int64_t want_waves = 4096;
  int64_t ns = (want_waves + units - 1) / units;
  const int64_t min_chunk = 256;
  const int64_t max_ns = t_max > 0 ? (t_max + min_chunk - 1) / min_chunk : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int64_t c = t_max > 0 ? (t_max + ns - 1) / ns : kTile;
  c = (c + kTile - 1) / kTile * kTile;
  ns = t_max > 0 ? (t_max + c - 1) / c : 1;
  *n_split = static_cast<int32_t>(ns);
  *chunk = static_cast<int32_t>(c);
}

size_t attn_workspace_bytes(int32_t batch, int32_t hq, int32_t n_split) {
  return static_cast<size_t>(batch) * hq * n_split * (QK + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnLaunch& a, const KTable& tk, const KTable& tv,
                       const SignWords& sw, hipStream_t stream) {
  const dim3 g1((a.n_split + kWaves - 1) / kWaves, a.hkv, a.batch), b1(kWaves * 64);
#define FATQ_ATT(K, V) \
  hipLaunchKernelGGL((attn_split_kernel<K, V>), g1, b1, 0, stream, a, tk, tv, sw)
  switch (tk.bits * 10 + tv.bits) {
    case 22: FATQ_ATT(2, 2); break;
    case 23: FATQ_ATT(2, 3); break;
    case 24: FATQ_ATT(2, 4); break;
    case 32: FATQ_ATT(3, 2); break;
    case 33: FATQ_ATT(3, 3); break;
    case 34: FATQ_ATT(3, 4); break;
    case 42: FATQ_ATT(4, 2); break;
    case 43: FATQ_ATT(4, 3); break;
    default: FATQ_ATT(4, 4); break;
  }
#undef FATQ_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(a.hq, a.batch), dim3(QK), 0, stream, a, sw);
  return hipGetLastError();
}

}  // namespace fatq

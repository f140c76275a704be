// Decode attention over the packed cache with the per-group contractions on MFMA.
//
// Page cited: [Spec] "TurboQuant KV Cache Compression -- Spec", "Optimization:
// Fused dequant-dot": pre-rotate q once, dot it with centroid look-ups of the
// cached keys, accumulate the weighted value look-ups in the rotated domain, and
// inverse-rotate the output once.
//
// For one (sequence b, KV head g) the G = Hq/Hkv query heads share every cached key
// and value, so a 16-token tile costs two dense contractions over the group:
// scores K~ (16 x 128) . Q'^T (128 x G) and values P (G x 16) . V~ (16 x 128).
// Both run on v_mfma_f32_16x16x32_f16 (8 k-steps of 32 slots per product).
//
// Accuracy (fp32 level from fp16 operands, all splits exact in fp32):
//  * every centroid value is split as 4c = hi + lo (fp16 each; the factor 4 is exact
//    and keeps lo in the fp16 normal range).  Four k-slots hold two elements:
//    A = [hi(c_e0), hi(c_e1), lo(c_e0), lo(c_e1)], B = [q_e0, q_e1, q_e0, q_e1];
//  * queries: B columns 0..G-1 hold hi(q'), columns G..2G-1 hold lo(q'); the two
//    score columns of a head are added (q' is scaled by a power of two so |q'| < 1);
//  * values: B = [hi(v_ta), hi(v_tb), lo(v_ta), lo(v_tb)] for two tokens, and the
//    probabilities A = [p_ta, p_tb, p_ta, p_tb] with rows 0..G-1 = hi(p'), rows
//    G..2G-1 = lo(p'); the two output rows of a head are added at the end.
// Every fp16 product is exact in the fp32 accumulator.
//
// Dequantization is a table look-up in LDS returning a ready MFMA operand (8 bytes):
//  * keys: byte of two 4-bit codes -> entry (3- and 2-bit keys are first widened
//    to 4-bit fields in registers);
//  * values: the codes of one element in two tokens -> entry (2-bit: 16 entries;
//    3/4-bit: 256 entries).
// Tables with 256 entries are replicated 16 times and lane L reads copy L % 16, so
// the 16 lanes an LDS cycle serves hit 16 different bank pairs.
//
// Token order inside a 16-token tile is the identity: score row r = 4 qq + j is
// token r, which is the token pair (4qq + j, j = 0..3) lane group qq needs for its
// probability operand, so no cross-lane exchange is needed between the products.
//
// Work layout: grid (n_split, Hkv, B), 4 waves per workgroup; the workgroup owns
// tokens [split*chunk, min(len, (split+1)*chunk)) and wave w takes 32-token super
// tiles w, w+4, ... with the next super tile's codes loaded while the current one
// is processed.  Waves merge in LDS and each workgroup writes one partial
// (m, l, o') per head to the workspace; a second kernel merges the splits,
// divides by l and applies R^T = D H / sqrt(128).  Scores are kept in base 2.
//
// MFMA 16x16x32 f16 operand layout (wave64): A[i][k]: lane i%16 + 16*(k/8), slot
// k%8; B[k][j]: lane j + 16*(k/8), slot k%8; D[i][j]: lane j + 16*(i/4), slot i%4.

#include <hip/hip_fp16.h>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kST = 32;          // tokens per super tile (2 MFMA tiles)
constexpr int kMaxG = 8;         // query heads per KV head on this path
constexpr int kRep = 16;         // replicas of the 256-entry tables
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kCScale = 4.0f;  // centroid pre-scale (exact)

#ifndef FATQ_ATTN_WANT_WG
#define FATQ_ATTN_WANT_WG 768
#endif
#ifndef FATQ_ATTN_MIN_CHUNK
#define FATQ_ATTN_MIN_CHUNK 512
#endif

template <int B>
constexpr int cbytes() { return B == 2 ? 32 : B == 3 ? 48 : 64; }

__device__ __forceinline__ f4 mfma(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 x, _Float16 y) {
  h2 v = {x, y};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ h4 h4_of(uint2 u) { return __builtin_bit_cast(h4, u); }

__device__ __forceinline__ void split_h(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

// Spread 8 two-bit fields (bits 2i..2i+1) to nibbles (bits 4i..4i+1).
__device__ __forceinline__ uint32_t spread2(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return x;
}

// Spread 8 one-bit fields (bit i) to nibbles (bit 4i).
__device__ __forceinline__ uint32_t spread1(uint32_t x) {
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x;
}

// Key codes of elements 32 qq .. 32 qq + 31 of a token as 16 bytes of two 4-bit
// fields (byte i: element 32 qq + 2i in the low nibble, 32 qq + 2i + 1 high).
template <int KB>
__device__ __forceinline__ uint4 load_k32(const uint8_t* row, int qq) {
  if constexpr (KB == 4) {
    return *reinterpret_cast<const uint4*>(row + 16 * qq);
  } else if constexpr (KB == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * qq);
    return make_uint4(spread2(w.x & 0xFFFFu), spread2(w.x >> 16), spread2(w.y & 0xFFFFu),
                      spread2(w.y >> 16));
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * qq);
    const uint32_t h = *reinterpret_cast<const uint32_t*>(row + 32 + 4 * qq);
    return make_uint4(spread2(w.x & 0xFFFFu) | (spread1(h & 0xFFu) << 2),
                      spread2(w.x >> 16) | (spread1((h >> 8) & 0xFFu) << 2),
                      spread2(w.y & 0xFFFFu) | (spread1((h >> 16) & 0xFFu) << 2),
                      spread2(w.y >> 16) | (spread1(h >> 24) << 2));
  }
}

// Value codes of elements 8n .. 8n+7 of a token: 16 bits of 2-bit fields (VB = 2)
// or a word of 4-bit fields (VB = 3, 4).
template <int VB>
__device__ __forceinline__ uint32_t load_v8(const uint8_t* row, int n) {
  if constexpr (VB == 4) {
    return *reinterpret_cast<const uint32_t*>(row + 4 * n);
  } else if constexpr (VB == 2) {
    return *reinterpret_cast<const uint16_t*>(row + 2 * n);
  } else {
    const uint32_t lo = *reinterpret_cast<const uint16_t*>(row + 2 * n);
    const uint32_t hi = row[32 + n];
    return spread2(lo) | (spread1(hi) << 2);
  }
}

// Fill a 256-entry operand table for a byte index of two 4-bit codes (low nibble:
// first element/token, high nibble: second), replicated kRep times, by the 192
// threads t in [0, 192) of waves 1..3.
__device__ __forceinline__ void fill_table256(uint2* tab, const KTable& t, int t3) {
  for (int i = t3; i < 256; i += 192) {
    const int r = i & (kRep - 1);
    const int lo4 = i >> 4;
    _Float16 h0, l0;
    split_h(kCScale * t.c[lo4], h0, l0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      _Float16 h1, l1;
      split_h(kCScale * t.c[k], h1, l1);
      const int byte = lo4 | (k << 4);
      tab[byte * kRep + r] = make_uint2(pack_h2(h0, h1), pack_h2(l0, l1));
    }
  }
}

// In-register Walsh-Hadamard transform (unnormalized) of a 128-block held by a quad
// of lanes: lane q holds elements 8 (q + 4k) + i in v[k][i].  Strides 1, 2, 4 are
// inside a chunk, 8 and 16 across the quad's lanes, 32 and 64 across chunks.
__device__ __forceinline__ void fwht_quad(float (&v)[4][8], int q) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int L = 1; L < 8; L <<= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & L) == 0) {
          const float x = v[k][i], y = v[k][i + L];
          v[k][i] = x + y;
          v[k][i + L] = x - y;
        }
#pragma unroll
  for (int msk = 1; msk <= 2; msk <<= 1) {
    const bool upper = (q & msk) != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __shfl_xor(v[k][i], msk, 64);
        v[k][i] = upper ? p - v[k][i] : v[k][i] + p;
      }
  }
#pragma unroll
  for (int L = 1; L < 4; L <<= 1)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((k & L) == 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = v[k][i], y = v[k + L][i];
          v[k][i] = x + y;
          v[k + L][i] = x - y;
        }
}

// Shift a value down (lane i reads lane i + d) or up (lane i reads lane i - d)
// inside rows of 16 lanes; a compile-time distance becomes one DPP move.
template <int D>
__device__ __forceinline__ float row_down(float x, int d) {
  if constexpr (D > 0)
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x100 + D, 0xF, 0xF, false));
  else
    return __shfl_down(x, d, 16);
}
template <int D>
__device__ __forceinline__ uint32_t row_up(uint32_t x, int d) {
  if constexpr (D > 0)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(x), 0x110 + D, 0xF, 0xF, false));
  else
    return __shfl_up(x, d, 16);
}

// 8 two-bit fields of each of two 16-bit words wa, wb interleaved to nibbles:
// nibble m = (wa field m) | (wb field m) << 2.
__device__ __forceinline__ uint32_t interleave2(uint32_t wa, uint32_t wb) {
  uint32_t x = __builtin_amdgcn_perm(wb, wa, 0x05010400u);   // [wa.b0, wb.b0, wa.b1, wb.b1]
  uint32_t t = ((x >> 4) ^ x) & 0x00F000F0u;
  x ^= t ^ (t << 4);
  t = ((x >> 2) ^ x) & 0x0C0C0C0Cu;
  x ^= t ^ (t << 2);
  return x;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 h8_of(uint2 lo, uint2 hi) {
  uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
  return __builtin_bit_cast(h8, u);
}

// VSH: key and value codebooks are identical, so one operand table serves both.
// GT: the group size G as a compile-time constant (1, 2, 4, 8), or 0 (runtime).
template <int KB, int VB, bool VSH, int GT>
__global__ void __launch_bounds__(kThreads, 2) attn_mfma_kernel(AttnLaunch a, KTable tk,
                                                                KTable tv, SignWords sw) {
  constexpr bool V2 = VB == 2;
  constexpr int KCB = cbytes<KB>(), VCB = cbytes<VB>();
  constexpr int VENT = VSH ? 1 : (V2 ? 16 : 256 * kRep);
  __shared__ uint2 ktab[256 * kRep];            // 32 KB; reused for the wave merge
  __shared__ uint2 vtab_own[VENT];
  __shared__ __attribute__((aligned(16))) float qr[kMaxG][QK];
  __shared__ float qsc;
  __shared__ __attribute__((aligned(16))) float nrm[kWaves][3][kST];
  __shared__ float comb_ml[kWaves][kMaxG][2];
  static_assert(sizeof(ktab) >= sizeof(float) * kWaves * 2 * kMaxG * QK, "merge buffer");
  static_assert(!(VSH && V2), "2-bit values use their own 16-entry table");
  uint2* vtab = VSH ? ktab : vtab_own;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qq = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = GT > 0 ? GT : a.hq / a.hkv;

  // ---- the sequence range, then the first super tile's loads (in flight during setup)
  const int64_t len64 = a.pos ? static_cast<int64_t>(a.pos[b]) + a.n_new : a.seq_lens[b];
  const int len = len64 < 0 ? 0 : (len64 > a.t_max ? a.t_max : static_cast<int>(len64));
  const int c0 = split * a.chunk;
  const int c1 = min(len, c0 + a.chunk);
  const int last = c1 - 1;
  const int64_t kvb = (static_cast<int64_t>(b) * a.hkv + g) * a.t_max;
  const uint8_t* kc = a.k_codes + kvb * KCB;
  const uint8_t* vc = a.v_codes + kvb * VCB;
  const uint16_t* kn = a.k_norms + kvb;
  const uint16_t* vn = a.v_norms + kvb;
  int st = c0 + wave * kST;
  uint4 kw[2];
  uint32_t vw[2][4];
  uint32_t nh = 0;
  auto issue_loads = [&](int s0) {
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      const uint32_t ta = static_cast<uint32_t>(min(s0 + 16 * t4 + n, last));
      kw[t4] = load_k32<KB>(kc + ta * KCB, qq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t tv_ = static_cast<uint32_t>(min(s0 + 16 * t4 + 4 * qq + j, last));
        vw[t4][j] = load_v8<VB>(vc + tv_ * VCB, n);
      }
    }
    const int tcl = min(s0 + (lane & 31), last);
    nh = lane < 32 ? kn[tcl] : vn[tcl];
  };
  if (st < c1) issue_loads(st);

  // ---- wave 0: q' = H (s * q) / sqrt(128) for the G heads in registers (quad h =
  // lanes 4h..4h+3 holds head h, lane q of the quad elements 8 (q + 4k) + i), scaled
  // by a power of two so that |q'| < 1, into LDS.  The other waves fill the tables.
  if (wave == 0) {
    float qx[4][8];
    const int hq_ = lane >> 2, qd = lane & 3;
    const bool act = hq_ < G;
    const int64_t qo = (static_cast<int64_t>(b) * a.hq + g * G + (act ? hq_ : 0)) * QK;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e0 = 8 * (qd + 4 * k);
      if (a.q_is_bf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qo + e0);
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          qx[k][2 * m] = __uint_as_float(d[m] << 16);
          qx[k][2 * m + 1] = __uint_as_float(d[m] & 0xffff0000u);
        }
      } else {
        const float* qf = static_cast<const float*>(a.q) + qo + e0;
        const float4 w0 = *reinterpret_cast<const float4*>(qf);
        const float4 w1 = *reinterpret_cast<const float4*>(qf + 4);
        qx[k][0] = w0.x; qx[k][1] = w0.y; qx[k][2] = w0.z; qx[k][3] = w0.w;
        qx[k][4] = w1.x; qx[k][5] = w1.y; qx[k][6] = w1.z; qx[k][7] = w1.w;
      }
      const uint32_t sb = sw.w[0][qd];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = ((sb >> (8 * k + i)) & 1u) ? -qx[k][i] : qx[k][i];
        qx[k][i] = act ? v : 0.0f;
      }
    }
    fwht_quad(qx, qd);
    float qmax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) qmax = fmaxf(qmax, fabsf(qx[k][i]));
#pragma unroll
    for (int s2 = 32; s2 >= 1; s2 >>= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, s2, 64));
    int qex = 0;
    frexpf(qmax * kInvSqrtQK, &qex);
    const float qs = qmax > 0.0f ? ldexpf(1.0f, qex) : 1.0f;
    const float inv = kInvSqrtQK / qs;
    if (act) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float* dst = &qr[hq_][8 * (qd + 4 * k)];
        *reinterpret_cast<float4*>(dst) =
            make_float4(qx[k][0] * inv, qx[k][1] * inv, qx[k][2] * inv, qx[k][3] * inv);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(qx[k][4] * inv, qx[k][5] * inv, qx[k][6] * inv, qx[k][7] * inv);
      }
    }
    if (lane == 0) qsc = qs;
  } else {
    // ---- operand tables (shared by the four waves), filled by waves 1..3
    const int t3 = tid - 64;
    fill_table256(ktab, tk, t3);
    if constexpr (!VSH) {
      if constexpr (V2) {
        if (t3 < 16) {
          _Float16 h0, l0, h1, l1;
          split_h(kCScale * tv.c[t3 & 3], h0, l0);
          split_h(kCScale * tv.c[t3 >> 2], h1, l1);
          vtab[t3] = make_uint2(pack_h2(h0, h1), pack_h2(l0, l1));
        }
      } else {
        fill_table256(vtab, tv, t3);
      }
    }
  }
  __syncthreads();   // q' and the operand tables are complete
  const float qscale = qsc;

  // ---- B operands of the score product: k-step m covers elements 32qq + 4m .. +3
  h8 bq[8];
  {
    const bool used = n < 2 * G;
    const int h = n < G ? n : (used ? n - G : 0);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 xv = *reinterpret_cast<const float4*>(&qr[h][32 * qq + 4 * m]);
      const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
      _Float16 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        _Float16 hi, lo;
        split_h(xs[i], hi, lo);
        x[i] = n < G ? hi : (used ? lo : _Float16(0));
      }
      bq[m] = h8{x[0], x[1], x[0], x[1], x[2], x[3], x[2], x[3]};
    }
  }
  const float sc2 = a.scale * kLog2e * qscale / kCScale;
  const uint32_t roff = (lane & (kRep - 1)) << 3;      // byte offset of this lane's replica

  float m_run = -INFINITY, l_run = 0.0f;
  f4 o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  for (; st < c1; st += kWaves * kST) {
    // take this super tile's data, start loading the next one
    uint4 kcur[2];
    uint32_t vcur[2][4];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      kcur[t4] = kw[t4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vcur[t4][j] = vw[t4][j];
    }
    const uint32_t ncur = nh;
    if (st + kWaves * kST < c1) issue_loads(st + kWaves * kST);
    // per-token factors through LDS: key scale (0 when masked), key bias (-inf when
    // masked), value scale
    {
      const int t = st + (lane & 31);
      const float nf = __half2float(__ushort_as_half(static_cast<uint16_t>(ncur)));
      if (lane < 32) {
        nrm[wave][0][lane] = t < c1 ? nf * sc2 : 0.0f;
        nrm[wave][1][lane] = t < c1 ? 0.0f : -INFINITY;
      } else {
        nrm[wave][2][lane - 32] = nf * (1.0f / kCScale);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- scores
    float sc[2][4];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
      const uint32_t w4[4] = {kcur[t4].x, kcur[t4].y, kcur[t4].z, kcur[t4].w};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = w4[m >> 1] >> (16 * (m & 1));
        const uint32_t a0 = ((m & 1) ? (w << 7) : (w << 7)) & 0x7F80u;
        const uint32_t a1 = (w >> 1) & 0x7F80u;
        const uint2 e0 = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const uint8_t*>(ktab) + (a0 | roff));
        const uint2 e1 = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const uint8_t*>(ktab) + (a1 | roff));
        acc = mfma32(h8_of(e0, e1), bq[m], acc);
      }
      const float4 f = *reinterpret_cast<const float4*>(&nrm[wave][0][16 * t4 + 4 * qq]);
      const float4 z = *reinterpret_cast<const float4*>(&nrm[wave][1][16 * t4 + 4 * qq]);
      const float fk[4] = {f.x, f.y, f.z, f.w}, zb[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[t4][j] = fmaf(acc[j] + row_down<GT>(acc[j], G), fk[j], zb[j]);
    }
    // ---- online softmax (lanes n < G carry head n; other columns are ignored)
    float mloc = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mnew = fmaxf(m_run, mloc);
    float p[2][4];
    float lsum = 0.0f;
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[t4][j] = __builtin_amdgcn_exp2f(sc[t4][j] - mnew);
        lsum += p[t4][j];
      }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    if (__ballot(mnew > m_run && n < G)) {   // rescale only when a running maximum grew
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float ar = __shfl(alpha, (4 * qq + j) % G, 64);
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m][j] *= ar;
      }
    }
    l_run += lsum;
    m_run = mnew;
    // ---- value product: A = [p_a, p_b, p_a, p_b, p_c, p_d, p_c, p_d] for tokens
    // 4qq..4qq+3; rows < G hi(p'), rows G..2G-1 lo(p') (moved up by G lanes)
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      const float4 f = *reinterpret_cast<const float4*>(&nrm[wave][2][16 * t4 + 4 * qq]);
      const float pv[4] = {p[t4][0] * f.x, p[t4][1] * f.y, p[t4][2] * f.z, p[t4][3] * f.w};
      _Float16 hv[4], lv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split_h(pv[j], hv[j], lv[j]);
      const uint32_t lab = row_up<GT>(pack_h2(lv[0], lv[1]), G);
      const uint32_t lcd = row_up<GT>(pack_h2(lv[2], lv[3]), G);
      const uint32_t pab = n < G ? pack_h2(hv[0], hv[1]) : (n < 2 * G ? lab : 0u);
      const uint32_t pcd = n < G ? pack_h2(hv[2], hv[3]) : (n < 2 * G ? lcd : 0u);
      const h8 ap = __builtin_bit_cast(h8, make_uint4(pab, pab, pcd, pcd));
      if constexpr (V2) {
        const uint32_t zab = interleave2(vcur[t4][0], vcur[t4][1]);
        const uint32_t zcd = interleave2(vcur[t4][2], vcur[t4][3]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t oab = (m == 0 ? (zab << 3) : (zab >> (4 * m - 3))) & 0x78u;
          const uint32_t ocd = (m == 0 ? (zcd << 3) : (zcd >> (4 * m - 3))) & 0x78u;
          const uint2 eab = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(vtab) + oab);
          const uint2 ecd = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(vtab) + ocd);
          o[m] = mfma32(ap, h8_of(eab, ecd), o[m]);
        }
      } else {
        const uint32_t wa = vcur[t4][0], wb = vcur[t4][1], wc = vcur[t4][2], wd = vcur[t4][3];
        const uint32_t ze0 = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
        const uint32_t zo0 = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
        const uint32_t ze1 = (wc & 0x0F0F0F0Fu) | ((wd << 4) & 0xF0F0F0F0u);
        const uint32_t zo1 = ((wc >> 4) & 0x0F0F0F0Fu) | (wd & 0xF0F0F0F0u);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int k = m >> 1;
          const uint32_t z0 = (m & 1) ? zo0 : ze0, z1 = (m & 1) ? zo1 : ze1;
          const uint32_t i0 = (k == 0 ? (z0 << 7) : (z0 >> (8 * k - 7))) & 0x7F80u;
          const uint32_t i1 = (k == 0 ? (z1 << 7) : (z1 >> (8 * k - 7))) & 0x7F80u;
          const uint2 eab = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(vtab) + (i0 | roff));
          const uint2 ecd = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(vtab) + (i1 | roff));
          o[m] = mfma32(ap, h8_of(eab, ecd), o[m]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the four waves in LDS (the key table is no longer needed)
  __syncthreads();
  float* comb_o = reinterpret_cast<float*>(ktab);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * qq + j;
    if (r < 2 * G) {
#pragma unroll
      for (int m = 0; m < 8; ++m) comb_o[(wave * 2 * kMaxG + r) * QK + 8 * n + m] = o[m][j];
    }
  }
  if (qq == 0 && n < G) {
    comb_ml[wave][n][0] = m_run;
    comb_ml[wave][n][1] = l_run;
  }
  __syncthreads();
  float* ws_o = static_cast<float*>(a.workspace);
  float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * a.n_split * QK;
  const int64_t rbase = (static_cast<int64_t>(b) * a.hq + g * G) * a.n_split;
  for (int idx = tid; idx < G * QK; idx += kThreads) {
    const int h = idx >> 7, e = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, comb_ml[w][h][0]);
    float os = 0.0f, ls = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float m_w = comb_ml[w][h][0];
        const float f = m_w > -INFINITY ? __builtin_amdgcn_exp2f(m_w - M) : 0.0f;
        os += f * (comb_o[(w * 2 * kMaxG + h) * QK + e] + comb_o[(w * 2 * kMaxG + G + h) * QK + e]);
        ls += f * comb_ml[w][h][1];
      }
    }
    const int64_t r = rbase + static_cast<int64_t>(h) * a.n_split + split;
    ws_o[r * QK + e] = os;
    if (e == 0) {
      ws_ml[2 * r] = M;
      ws_ml[2 * r + 1] = ls;
    }
  }
}

// Merge the splits of one (b, query head): weights f_s = exp2(m_s - M), output
// (sum_s f_s o'_s) / (sum_s f_s l_s), then R^T = D H / sqrt(128).  256 threads:
// 32 float4 columns x 8 split groups.
__global__ void __launch_bounds__(256) attn_merge_splits_kernel(AttnLaunch a, SignWords sw) {
  __shared__ float fs[1024];
  __shared__ __attribute__((aligned(16))) float part[8][QK];
  __shared__ float red[2];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.n_split;
  const float* ws_o = static_cast<const float*>(a.workspace);
  const float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * ns * QK;
  const int64_t r0 = (static_cast<int64_t>(b) * a.hq + h) * ns;
  if (wave == 0) {
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, ws_ml[2 * (r0 + s)]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) mx = fmaxf(mx, __shfl_xor(mx, k, 64));
    float den = 0.0f;
    for (int s = lane; s < ns; s += 64) {
      const float ms = ws_ml[2 * (r0 + s)];
      const float f = ms > -INFINITY ? __builtin_amdgcn_exp2f(ms - mx) : 0.0f;
      fs[s] = f;
      den += f * ws_ml[2 * (r0 + s) + 1];
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k, 64);
    if (lane == 0) red[0] = den;
  }
  __syncthreads();
  const int e4 = tid & 31, grp = tid >> 5;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = grp; s < ns; s += 8) {
    const float f = fs[s];
    const float4 v = reinterpret_cast<const float4*>(ws_o + (r0 + s) * QK)[e4];
    acc.x += f * v.x;
    acc.y += f * v.y;
    acc.z += f * v.z;
    acc.w += f * v.w;
  }
  reinterpret_cast<float4*>(&part[grp][0])[e4] = acc;
  __syncthreads();
  float num = 0.0f;
  if (tid < QK) {
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) num += part[gi][tid];
  }
  const float den = red[0];
  __syncthreads();
  float* o = &part[0][0];
  if (tid < QK) o[tid] = den > 0.0f ? num / den : 0.0f;
  __syncthreads();
  for (int L = 1; L < QK; L <<= 1) {
    float u = 0.0f, v = 0.0f;
    int i = 0;
    if (tid < QK / 2) {
      i = (tid / L) * 2 * L + (tid % L);
      u = o[i];
      v = o[i + L];
    }
    __syncthreads();
    if (tid < QK / 2) {
      o[i] = u + v;
      o[i + L] = u - v;
    }
    __syncthreads();
  }
  if (tid < QK) {
    const int qd = (tid >> 3) & 3, k = tid >> 5, i = tid & 7;
    const float r = o[tid] * kInvSqrtQK;
    a.out[(static_cast<int64_t>(b) * a.hq + h) * QK + tid] =
        ((sw.w[0][qd] >> (8 * k + i)) & 1u) ? -r : r;
  }
}

}  // namespace

bool attn_mfma_supported(int32_t hq, int32_t hkv) { return hq / hkv <= kMaxG; }

void attn_mfma_partition(int32_t batch, int32_t hkv, int32_t t_max, int32_t* n_split,
                         int32_t* chunk) {
  const int64_t units = static_cast<int64_t>(batch > 0 ? batch : 1) * hkv;
  const int64_t want = FATQ_ATTN_WANT_WG;   // workgroups in flight
  int64_t ns = (want + units - 1) / units;
  const int64_t min_chunk = FATQ_ATTN_MIN_CHUNK;   // tokens per split at least
  const int64_t max_ns = t_max > 0 ? (t_max + min_chunk - 1) / min_chunk : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns > 1024) ns = 1024;
  if (ns < 1) ns = 1;
  int64_t c = t_max > 0 ? (t_max + ns - 1) / ns : kST;
  c = (c + kST - 1) / kST * kST;
  ns = t_max > 0 ? (t_max + c - 1) / c : 1;
  *n_split = static_cast<int32_t>(ns);
  *chunk = static_cast<int32_t>(c);
}

size_t attn_mfma_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t n_split) {
  (void)hkv;
  return static_cast<size_t>(batch) * hq * n_split * (QK + 2) * sizeof(float);
}

template <int GT>
void launch_g(const AttnLaunch& a, const KTable& tk, const KTable& tv, const SignWords& sw,
              hipStream_t stream, bool same) {
  const dim3 g1(a.n_split, a.hkv, a.batch), b1(kThreads);
#define FATQ_ATT(K, V) \
  hipLaunchKernelGGL((attn_mfma_kernel<K, V, false, GT>), g1, b1, 0, stream, a, tk, tv, sw)
#define FATQ_ATS(K) \
  hipLaunchKernelGGL((attn_mfma_kernel<K, K, true, GT>), g1, b1, 0, stream, a, tk, tv, sw)
  if (same) {
    if (tk.bits == 3) FATQ_ATS(3);
    else FATQ_ATS(4);
    return;
  }
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
#undef FATQ_ATS
}

hipError_t launch_attn_mfma(const AttnLaunch& a, const KTable& tk, const KTable& tv,
                            const SignWords& sw, hipStream_t stream) {
  bool same = tk.bits == tv.bits && tv.bits != 2;
  for (int i = 0; same && i < (1 << tk.bits); ++i) same = tk.c[i] == tv.c[i];
  switch (a.hq / a.hkv) {
    case 1: launch_g<1>(a, tk, tv, sw, stream, same); break;
    case 2: launch_g<2>(a, tk, tv, sw, stream, same); break;
    case 4: launch_g<4>(a, tk, tv, sw, stream, same); break;
    case 8: launch_g<8>(a, tk, tv, sw, stream, same); break;
    default: launch_g<0>(a, tk, tv, sw, stream, same); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_splits_kernel, dim3(a.hq, a.batch), dim3(256), 0, stream, a, sw);
  return hipGetLastError();
}

}  // namespace fatq

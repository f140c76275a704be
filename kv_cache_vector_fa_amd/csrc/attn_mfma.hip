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
// Accuracy (about 22 significant bits per product, every fp16 product exact in the
// fp32 accumulator, every fp16 half rounded to nearest):
//  * every centroid value is split as 64c = hi + lo (fp16 each; the factor 64 is exact
//    and keeps lo in the fp16 normal range for every 2-4 bit table of dimension 128).
//    Four k-slots hold two elements: A = [hi(c_e0), hi(c_e1), lo(c_e0), lo(c_e1)],
//    B = [q_e0, q_e1, q_e0, q_e1];
//  * queries: B columns 0..G-1 hold hi(q'), columns G..2G-1 hold lo(q'); the two
//    score columns of a head are added (q' is scaled by a power of two so that
//    2^13 <= max |q'| < 2^14);
//  * values: B = [hi(v_ta), hi(v_tb), lo(v_ta), lo(v_tb)] for two tokens, and the
//    weights A = [w_ta, w_tb, w_ta, w_tb] with rows 0..G-1 = hi(w), rows G..2G-1 =
//    lo(w), w = p * n_V * vs; the two output rows of a head are added at the end.
//    p <= 1, and vs is a power of two per wave, lowered (the accumulator rescaled
//    with it) whenever a super tile holds a value norm n with n * vs > 2^15, so the
//    weights of a wave's stream stay below 2^15 and lo(w) is an fp16 normal number
//    unless w < 2^-3.  The rounding error of one token's weight is then at most
//    2^-22 w + 2^-25 (absolute floor of the fp16 subnormals), i.e. relative to the
//    largest value norm of the stream at most 2^-22 + 2^-40 per token, with no sign
//    bias (round to nearest), and the fp32 normaliser l carries exact p.
// Scores and weights therefore carry fp32-level rounding, not fp16-level.
//
// Dequantization is a table look-up in LDS returning a ready MFMA operand.  One
// 64 KB table has a 256-byte row per index byte r:
//  * bytes [0, 128): key entry r (two 4-bit key codes: low nibble first element),
//    8 bytes replicated 16 times;
//  * bytes [128, 256): value entry r.  2-bit values: r holds the codes of one
//    element in the four tokens of a lane's operand, and the 16-byte entry is that
//    whole operand, replicated 8 times; 3/4-bit values: r holds the codes of one
//    element in two tokens (8 bytes, 16 replicas).  When keys and values share a codebook the value
//    look-ups use the key half.
// A look-up address is one v_perm: (index byte << 8) | replica offset of the lane.
// Lane L reads replica L % 16 (8-byte entries) or L % 8 (16-byte entries), so the
// lanes an LDS cycle serves hit distinct banks.
//
// Token order inside a 16-token tile is the identity: score row r = 4 qq + j is
// token r, which is the token pair (4qq + j, j = 0..3) lane group qq needs for its
// probability operand, so no cross-lane exchange is needed between the products.
//
// Work layout: grid (n_split, Hkv, B), 4 waves per workgroup; the workgroup owns
// tokens [split*chunk, min(len, (split+1)*chunk)) and wave w takes 32-token super
// tiles w, w+4, ... with the next super tile's codes loaded while the current one
// is processed.  Waves merge in LDS and each workgroup writes one partial
// (m, l, o') per head to the workspace; a second kernel merges the splits by
// log-sum-exp, divides by l and applies R^T = D H / sqrt(128).  Scores are in
// base 2.
//
// MFMA 16x16x32 f16 operand layout (wave64): A[i][k]: lane i%16 + 16*(k/8), slot
// k%8; B[k][j]: lane j + 16*(k/8), slot k%8; D[i][j]: lane j + 16*(i/4), slot i%4.

#include <hip/hip_fp16.h>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kST = 32;          // tokens per super tile (2 MFMA tiles)
constexpr int kMaxG = 8;         // query heads per KV head on this path
constexpr int kRow = 256;        // table bytes per index byte
constexpr int kMaxSplit = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kCScale = 64.0f;  // centroid pre-scale (exact)
constexpr float kWMax = 32768.0f;  // bound of the value weights w = p n_V vs
// Raw buffer resources: an access at or beyond the range returns zeros, so loads
// past the sequence need no clamp and lanes without work use offset kOOB.
constexpr int32_t kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;   // every range is below 2^31 (host check)

#ifndef FATQ_ATTN_WANT_WG
#define FATQ_ATTN_WANT_WG 512
#endif
#ifndef FATQ_ATTN_MIN_CHUNK
#define FATQ_ATTN_MIN_CHUNK 512
#endif

template <int B>
constexpr int cbytes() { return B == 2 ? 32 : B == 3 ? 48 : 64; }

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRsrcWord3);
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 x, _Float16 y) {
  h2 v = {x, y};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void split_h(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ h8 h8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(h8, make_uint4(a, b, c, d));
}

// Barrier that orders LDS only: the workgroup's outstanding global loads stay in
// flight (__syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maximum over each row of 16 lanes (every lane of the row gets it).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));    // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f<0x4E>(x));    // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f<0x141>(x));   // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));   // row_mirror
  return x;
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

// Raw code words of one super tile as loaded (widened to 4-bit fields at use).
//  k[t4]: the key codes of elements 32 qq .. 32 qq + 31 of token 16 t4 + n;
//  v[t4][j]: the value codes of elements 8 n .. 8 n + 7 of token 16 t4 + 4 qq + j;
//  nrm: lanes < 32 the key norm, lanes >= 32 the value norm of token lane % 32.
template <int KB, int VB>
struct Codes {
  uint32_t k[2][KB == 4 ? 4 : 3];
  uint32_t v[2][4][VB == 3 ? 2 : 1];
  uint32_t nrm;
};

struct Rows {
  Rsrc kc, vc, kn, vn;
};

template <int KB, int VB>
__device__ __forceinline__ void issue_loads(const Rows& r, Codes<KB, VB>& c, int s0, bool live,
                                            int lane) {
  constexpr uint32_t KCB = cbytes<KB>(), VCB = cbytes<VB>();
  const int n = lane & 15, qq = lane >> 4;
  const uint32_t tk = static_cast<uint32_t>(s0 + n);
  const uint32_t tv = static_cast<uint32_t>(s0 + 4 * qq);
#pragma unroll
  for (int t4 = 0; t4 < 2; ++t4) {
    if constexpr (KB == 4) {
      const uint32_t o = live ? tk * KCB + 16 * qq : kOOB;
      const uint4 w = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r.kc, o + 16 * KCB * t4, 0, 0));
      c.k[t4][0] = w.x; c.k[t4][1] = w.y; c.k[t4][2] = w.z; c.k[t4][3] = w.w;
    } else {
      const uint32_t o = live ? tk * KCB + 8 * qq : kOOB;
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(r.kc, o + 16 * KCB * t4, 0, 0);
      c.k[t4][0] = w[0];
      c.k[t4][1] = w[1];
      if constexpr (KB == 3) {
        const uint32_t oh = live ? tk * KCB + 32 + 4 * qq : kOOB;
        c.k[t4][2] = __builtin_amdgcn_raw_buffer_load_b32(r.kc, oh + 16 * KCB * t4, 0, 0);
      } else {
        c.k[t4][2] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d = (16 * t4 + j) * VCB;
      if constexpr (VB == 4) {
        const uint32_t o = live ? tv * VCB + 4 * n : kOOB;
        c.v[t4][j][0] = __builtin_amdgcn_raw_buffer_load_b32(r.vc, o + d, 0, 0);
      } else {
        const uint32_t o = live ? tv * VCB + 2 * n : kOOB;
        c.v[t4][j][0] = __builtin_amdgcn_raw_buffer_load_b16(r.vc, o + d, 0, 0);
        if constexpr (VB == 3) {
          const uint32_t oh = live ? tv * VCB + 32 + n : kOOB;
          c.v[t4][j][1] = __builtin_amdgcn_raw_buffer_load_b8(r.vc, oh + d, 0, 0);
        }
      }
    }
  }
  const uint32_t on = static_cast<uint32_t>(s0 + (lane & 31)) * 2;
  const uint32_t ok = live && lane < 32 ? on : kOOB;
  const uint32_t ov = live && lane >= 32 ? on : kOOB;
  c.nrm = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r.kn, ok, 0, 0)) |
          static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r.vn, ov, 0, 0));
}

// The key words of one tile as four words of table index bytes (byte i of the 16:
// elements e = 32 qq + 2i and e + 1).  2/4-bit: 4-bit fields, code(e) in the low
// nibble.  3-bit: lo(e) | lo(e + 1) << 2 | hi(e) << 4 | hi(e + 1) << 5 from the
// low-bit plane (lo) and the high-bit plane (hi), the layout of the 3-bit key rows.
template <int KB>
__device__ __forceinline__ void key_fields(const uint32_t (&w)[KB == 4 ? 4 : 3], uint32_t (&f)[4]) {
  if constexpr (KB == 4) {
    f[0] = w[0]; f[1] = w[1]; f[2] = w[2]; f[3] = w[3];
  } else if constexpr (KB == 2) {
    f[0] = spread2(w[0] & 0xFFFFu); f[1] = spread2(w[0] >> 16);
    f[2] = spread2(w[1] & 0xFFFFu); f[3] = spread2(w[1] >> 16);
  } else {
    const uint32_t h = w[2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // the pair (e, e + 1)'s low bits are a nibble of the low plane: bytes 2(m & 1)
      // and 2(m & 1) + 1 of its word go to bytes 0 and 2, then a nibble to a byte
      const uint32_t b0 = 2u * (m & 1);
      const uint32_t y = __builtin_amdgcn_perm(0u, m < 2 ? w[0] : w[1],
                                               0x0C000C00u | ((b0 + 1) << 16) | b0);
      const uint32_t z = (y | (y << 4)) & 0x0F0F0F0Fu;
      // their high bits, a 2-bit field of byte m of the high plane, to bits 4-5
      const uint32_t a = (h >> (8 * m)) & 0xFFu;
      const uint32_t b = (a | (a << 12)) & 0x000F000Fu;
      const uint32_t c = (b | (b << 6)) & 0x03030303u;
      f[m] = z | (c << 4);
    }
  }
}

// Value word of elements 8 n .. 8 n + 7 as 4-bit fields (3/4-bit values).
template <int VB>
__device__ __forceinline__ uint32_t value_fields(const uint32_t (&w)[VB == 3 ? 2 : 1]) {
  if constexpr (VB == 4) return w[0];
  else return spread2(w[0] & 0xFFFFu) | (spread1(w[1] & 0xFFu) << 2);
}

// Four 16-bit words of 2-bit value codes (tokens a, b, c, d; field i = element
// 8n + i) -> index bytes: byte k of e = element 2k, of o = element 2k + 1, each
// (code of a) | (b) << 2 | (c) << 4 | (d) << 6.
__device__ __forceinline__ void quad_index2(uint32_t wa, uint32_t wb, uint32_t wc, uint32_t wd,
                                            uint32_t& e, uint32_t& o) {
  auto pair = [](uint32_t x, uint32_t y) {
    // bytes [x.b0, y.b0, x.b1, y.b1], then nibble k = (x nibble k) | (y nibble k) << 4,
    // then fields reordered within each byte to (x_2k, y_2k, x_2k+1, y_2k+1)
    uint32_t z = __builtin_amdgcn_perm(y, x, 0x05010400u);
    uint32_t t = ((z >> 4) ^ z) & 0x00F000F0u;
    z ^= t ^ (t << 4);
    t = ((z >> 2) ^ z) & 0x0C0C0C0Cu;
    return z ^ t ^ (t << 2);
  };
  const uint32_t ab = pair(wa, wb), cd = pair(wc, wd);
  e = (ab & 0x0F0F0F0Fu) | ((cd << 4) & 0xF0F0F0F0u);
  o = ((ab >> 4) & 0x0F0F0F0Fu) | (cd & 0xF0F0F0F0u);
}

// Table address of index byte k of word z: (byte << 8) | byte `rsel` of lane word R.
template <int K, int RSEL>
__device__ __forceinline__ uint32_t taddr(uint32_t z, uint32_t R) {
  return __builtin_amdgcn_perm(z, R, 0x0C0C0000u | ((4u + K) << 8) | RSEL);
}

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

// Sign of element e of the first 128-block (SignWords quad layout), of s1 and of the
// second sign vector s2 (R = D2 H D1 / sqrt(128); s2 = +1 without it).
__device__ __forceinline__ bool sign_bit(const SignWords& sw, int e) {
  const int c = e >> 3;
  return (sw.w[0][c & 3] >> (8 * (c >> 2) + (e & 7))) & 1u;
}
// Bit of element e in its sign word (the word sw.w[0][(e >> 3) & 3]).
__device__ __forceinline__ bool bit_of(uint32_t word, int e) {
  const int c = e >> 3;
  return (word >> (8 * (c >> 2) + (e & 7))) & 1u;
}
__device__ __forceinline__ bool sign_bit2(const SignWords& sw, int e) {
  const int c = e >> 3;
  return sw.two && ((sw.w2[0][c & 3] >> (8 * (c >> 2) + (e & 7))) & 1u);
}

// Inverse rotation of one head's merged output held as elements 2 lane, 2 lane + 1
// (fp32: s2, unnormalized Walsh-Hadamard, then s1 and 1/sqrt(128)), stored to dst.
__device__ __forceinline__ void rotate_out(float2 o, const SignWords& sw, int lane, float* dst) {
  o.x = sign_bit2(sw, 2 * lane) ? -o.x : o.x;
  o.y = sign_bit2(sw, 2 * lane + 1) ? -o.y : o.y;
  float u = o.x + o.y, v = o.x - o.y;
#pragma unroll
  for (int L = 1; L < 64; L <<= 1) {
    const float pu = __shfl_xor(u, L, 64), pv = __shfl_xor(v, L, 64);
    const bool up = (lane & L) != 0;
    u = up ? pu - u : u + pu;
    v = up ? pv - v : v + pv;
  }
  const float r0 = u * kInvSqrtQK, r1 = v * kInvSqrtQK;
  reinterpret_cast<float2*>(dst)[lane] =
      make_float2(sign_bit(sw, 2 * lane) ? -r0 : r0, sign_bit(sw, 2 * lane + 1) ? -r1 : r1);
}

// VSH: key and value codebooks are identical, so the key entries serve both.
// GT: the group size G as a compile-time constant (1, 2, 4, 8), or 0 (runtime).
template <int KB, int VB, bool VSH, int GT>
__global__ void __launch_bounds__(kThreads, 2) attn_mfma_kernel(AttnLaunch a, KTable tk,
                                                                KTable tv, SignWords sw) {
  constexpr bool V2 = VB == 2;
  __shared__ __attribute__((aligned(16))) uint8_t tab[256 * kRow];   // 64 KB
  __shared__ __attribute__((aligned(16))) uint16_t qhl[17][QK];      // hi, lo, zero rows
  __shared__ __attribute__((aligned(16))) float nrm[kWaves][3][kST];
  __shared__ uint32_t sp[2][16];
  __shared__ float qmx[kMaxG];
  __shared__ float comb_ml[kWaves][kMaxG][2];
  static_assert(sizeof(tab) >= sizeof(float) * kWaves * 2 * kMaxG * QK, "merge buffer");
  static_assert(!(VSH && V2), "2-bit values have their own entries");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, qq = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = GT > 0 ? GT : a.hq / a.hkv;
  constexpr uint32_t KCB = cbytes<KB>(), VCB = cbytes<VB>();

  // ---- loads that need only the kernel arguments go out first (query elements, sign
  // words and centroids, all indexed per lane), so that waiting for them later
  // leaves the code loads in flight: wave w rotates heads w and w + 4; lane holds
  // elements lane and lane + 64 of each
  // (raw bits here; widened after the loads are waited for)
  uint32_t qraw[2][2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const int h = wave + kWaves * hs;
    const int hc = h < G ? h : 0;
    const int64_t qo = (static_cast<int64_t>(b) * a.hq + g * G + hc) * QK;
    if (a.q_is_bf16) {
      const uint16_t* qb = static_cast<const uint16_t*>(a.q) + qo;
      qraw[hs][0] = qb[lane];
      qraw[hs][1] = qb[lane + 64];
    } else {
      const uint32_t* qf = static_cast<const uint32_t*>(a.q) + qo;
      qraw[hs][0] = qf[lane];
      qraw[hs][1] = qf[lane + 64];
    }
  }
  // sign words of elements lane and lane + 64 (the same word; see sign_bit)
  const uint32_t sw1 = sw.w[0][(lane >> 3) & 3], sw2 = sw.w2[0][(lane >> 3) & 3];
  __builtin_amdgcn_sched_barrier(0);

  // ---- the sequence range, then the first super tile's loads (in flight during setup)
  const int64_t len64 = static_cast<int64_t>(a.lens[b]) + a.len_add;
  const int len = len64 < 0 ? 0 : (len64 > a.t_max ? a.t_max : static_cast<int>(len64));
  const int c0 = split * a.chunk;
  const int c1 = min(len, c0 + a.chunk);
  const int64_t kvb = (static_cast<int64_t>(b) * a.hkv + g) * a.t_max;
  const uint32_t ulen = static_cast<uint32_t>(len);
  Rows rows;
  rows.kc = make_rsrc(a.k_codes + kvb * KCB, ulen * KCB);
  rows.vc = make_rsrc(a.v_codes + kvb * VCB, ulen * VCB);
  rows.kn = make_rsrc(a.k_norms + kvb, ulen * 2);
  rows.vn = make_rsrc(a.v_norms + kvb, ulen * 2);
  int st = c0 + wave * kST;
  Codes<KB, VB> buf0, buf1;
  issue_loads<KB, VB>(rows, buf0, st, st < c1, lane);

  // ---- centroid splits, then the operand table (thread r fills row r)
  {
    // centroid tid % 16 of the key (tid < 16) or value codebook, selected from the
    // uniform kernel arguments (straight-line selects: no per-lane argument loads)
    float c = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float ki = tk.c[i], vi = tv.c[i];
      c = (tid & 15) == i ? (tid < 16 ? ki : vi) : c;
    }
    _Float16 hi, lo;
    split_h(kCScale * c, hi, lo);
    if (tid < 32) sp[tid >> 4][tid & 15] = pack_h2(hi, lo);
  }
  lds_barrier();
  if (tid < 256) {
    const int r = tid;
    uint8_t* row = tab + r * kRow;
    // key row r: the codes of its two elements (3-bit rows: see key_fields)
    const uint32_t a0 = sp[0][KB == 3 ? (r & 3) | ((r >> 2) & 4) : r & 15];
    const uint32_t a1 = sp[0][KB == 3 ? ((r >> 2) & 3) | ((r >> 3) & 4) : r >> 4];
    const uint32_t kh = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // hi(c_lo4), hi(c_hi4)
    const uint32_t kl = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // lo(c_lo4), lo(c_hi4)
    const uint4 ke = make_uint4(kh, kl, kh, kl);
    // all 8 slots of a row hold the same value; rotating the slot a step writes by
    // the row index spreads the lanes of one store over all banks
#pragma unroll
    for (int k = 0; k < 8; ++k) reinterpret_cast<uint4*>(row)[(k + r) & 7] = ke;
    if constexpr (V2) {
      const uint32_t va = sp[1][r & 3], vb = sp[1][(r >> 2) & 3];
      const uint32_t vc = sp[1][(r >> 4) & 3], vd = sp[1][r >> 6];
      const uint4 ve = make_uint4(__builtin_amdgcn_perm(vb, va, 0x05040100u),
                                  __builtin_amdgcn_perm(vb, va, 0x07060302u),
                                  __builtin_amdgcn_perm(vd, vc, 0x05040100u),
                                  __builtin_amdgcn_perm(vd, vc, 0x07060302u));
#pragma unroll
      for (int k = 0; k < 8; ++k) reinterpret_cast<uint4*>(row + 128)[(k + r) & 7] = ve;
    } else if constexpr (!VSH) {
      const uint32_t v0 = sp[1][r & 15], v1 = sp[1][r >> 4];
      const uint32_t vh = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
      const uint32_t vl = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
      const uint4 ve = make_uint4(vh, vl, vh, vl);
#pragma unroll
      for (int k = 0; k < 8; ++k) reinterpret_cast<uint4*>(row + 128)[(k + r) & 7] = ve;
    }
  }

  // ---- q' = s2 * H (s * q): stride 64 in-lane, strides 32 .. 1 across lanes; the
  // largest |q'| of each head to LDS
  float qx[2][2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      qx[hs][i] = __uint_as_float(a.q_is_bf16 ? qraw[hs][i] << 16 : qraw[hs][i]);
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    float x0 = bit_of(sw1, lane) ? -qx[hs][0] : qx[hs][0];
    float x1 = bit_of(sw1, lane + 64) ? -qx[hs][1] : qx[hs][1];
    float u = x0 + x1, v = x0 - x1;
#pragma unroll
    for (int L = 32; L >= 1; L >>= 1) {
      const float pu = __shfl_xor(u, L, 64), pv = __shfl_xor(v, L, 64);
      const bool up = (lane & L) != 0;
      u = up ? pu - u : u + pu;
      v = up ? pv - v : v + pv;
    }
    qx[hs][0] = sw.two && bit_of(sw2, lane) ? -u : u;
    qx[hs][1] = sw.two && bit_of(sw2, lane + 64) ? -v : v;
    float mx = fmaxf(fabsf(u), fabsf(v));
#pragma unroll
    for (int s2 = 32; s2 >= 1; s2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s2, 64));
    const int h = wave + kWaves * hs;
    if (lane == 0 && h < G) qmx[h] = mx;
  }
  lds_barrier();   // tables and per-head maxima complete
  float qmax = 0.0f;
  for (int h = 0; h < G; ++h) qmax = fmaxf(qmax, qmx[h]);
  // qscale = 2^e with 2^13 <= max |q'| / qscale < 2^14 (e >= -110: a query that
  // small gives scores of 0 either way, and 1 / qscale stays finite)
  int qex = 0;
  frexpf(qmax * kInvSqrtQK, &qex);
  const float qscale = qmax > 0.0f ? ldexpf(1.0f, max(qex - 14, -110)) : 1.0f;
  {
    const float inv = kInvSqrtQK / qscale;
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int h = wave + kWaves * hs;
      if (h < G) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          _Float16 hi, lo;
          split_h(qx[hs][i] * inv, hi, lo);
          qhl[h][lane + 64 * i] = __builtin_bit_cast(uint16_t, hi);
          qhl[kMaxG + h][lane + 64 * i] = __builtin_bit_cast(uint16_t, lo);
        }
      }
    }
    if (tid < 64) reinterpret_cast<uint32_t*>(&qhl[2 * kMaxG][0])[tid] = 0u;
  }
  lds_barrier();   // q' halves complete

  // ---- B operands of the score product: k-step m covers elements 32qq + 4m .. +3;
  // column n < G: hi(q'_n), G <= n < 2G: lo(q'_{n-G}), else zero
  h8 bq[8];
  {
    const int qrow = n < G ? n : (n < 2 * G ? kMaxG + n - G : 2 * kMaxG);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint2 d = *reinterpret_cast<const uint2*>(&qhl[qrow][32 * qq + 4 * m]);
      bq[m] = h8_of(d.x, d.x, d.y, d.y);
    }
  }
  const float sc2 = a.scale * kLog2e * qscale / kCScale;
  // byte 0: key replica offset, byte 1: value replica offset (+128) of this lane
  const uint32_t R = ((lane & 15) << 3) |
                     ((VSH ? ((lane & 15) << 3) : V2 ? 128 + ((lane & 7) << 4) : 128 + ((lane & 15) << 3)) << 8);

  float m_run = -INFINITY, l_run = 0.0f;
  // value weight scale of this wave's stream; above any value a norm needs, so the
  // first super tile with a nonzero value norm sets it
  float vs = 18446744073709551616.0f;   // 2^64
  f4 o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  auto process = [&](const Codes<KB, VB>& cur, int s0) {
    // per-token factors through LDS: key scale (0 when masked), key bias (-inf when
    // masked), value weight factor n_V * vs
    {
      const int t = s0 + (lane & 31);
      const float nf = __half2float(__ushort_as_half(static_cast<uint16_t>(cur.nrm)));
      // the largest value norm of the super tile (lanes 32..63; past the sequence the
      // loads return 0) bounds every weight p n_V (p <= 1): lower vs, and rescale the
      // accumulator by the same power of two, when it would push a weight past kWMax
      const float rm = row_max16(nf);
      const float vmax = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                   __builtin_bit_cast(int, rm), 32)),
                               __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                   __builtin_bit_cast(int, rm), 48)));
      if (vmax * vs > kWMax) {
        int e = 0;
        frexpf(vmax, &e);                       // vmax < 2^e
        const float vs_new = ldexpf(kWMax, -e);  // vmax * vs_new < 2^15
        const float r = vs_new / vs;            // a power of two
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] *= r;
        vs = vs_new;
      }
      if (lane < 32) {
        nrm[wave][0][lane] = t < c1 ? nf * sc2 : 0.0f;
        nrm[wave][1][lane] = t < c1 ? 0.0f : -INFINITY;
      } else {
        nrm[wave][2][lane - 32] = nf * vs;
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- scores
    float sc[2][4];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      uint32_t f[4];
      key_fields<KB>(cur.k[t4], f);
      f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
      f4 acc1 = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = f[m >> 1];
        uint32_t a0, a1;
        if (m & 1) {
          a0 = taddr<2, 0>(w, R);
          a1 = taddr<3, 0>(w, R);
        } else {
          a0 = taddr<0, 0>(w, R);
          a1 = taddr<1, 0>(w, R);
        }
        const uint2 e0 = *reinterpret_cast<const uint2*>(tab + a0);
        const uint2 e1 = *reinterpret_cast<const uint2*>(tab + a1);
        // two accumulators halve the chain of dependent products
        if (m & 1) acc1 = mfma32(h8_of(e0.x, e0.y, e1.x, e1.y), bq[m], acc1);
        else acc = mfma32(h8_of(e0.x, e0.y, e1.x, e1.y), bq[m], acc);
      }
      acc += acc1;
      const float4 fk = *reinterpret_cast<const float4*>(&nrm[wave][0][16 * t4 + 4 * qq]);
      const float4 zb = *reinterpret_cast<const float4*>(&nrm[wave][1][16 * t4 + 4 * qq]);
      sc[t4][0] = fmaf(acc[0] + row_down<GT>(acc[0], G), fk.x, zb.x);
      sc[t4][1] = fmaf(acc[1] + row_down<GT>(acc[1], G), fk.y, zb.y);
      sc[t4][2] = fmaf(acc[2] + row_down<GT>(acc[2], G), fk.z, zb.z);
      sc[t4][3] = fmaf(acc[3] + row_down<GT>(acc[3], G), fk.w, zb.w);
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
      const float4 fv = *reinterpret_cast<const float4*>(&nrm[wave][2][16 * t4 + 4 * qq]);
      const float pa = p[t4][0] * fv.x, pb = p[t4][1] * fv.y;
      const float pc = p[t4][2] * fv.z, pd = p[t4][3] * fv.w;
      // hi = nearest fp16, lo = nearest fp16 of the exact fp32 remainder
      _Float16 ha, la, hb, lb, hc, lc, hd, ld;
      split_h(pa, ha, la);
      split_h(pb, hb, lb);
      split_h(pc, hc, lc);
      split_h(pd, hd, ld);
      const h2 hab = {ha, hb}, hcd = {hc, hd}, lab2 = {la, lb}, lcd2 = {lc, ld};
      const uint32_t lab = row_up<GT>(__builtin_bit_cast(uint32_t, lab2), G);
      const uint32_t lcd = row_up<GT>(__builtin_bit_cast(uint32_t, lcd2), G);
      const uint32_t pab = n < G ? __builtin_bit_cast(uint32_t, hab) : (n < 2 * G ? lab : 0u);
      const uint32_t pcd = n < G ? __builtin_bit_cast(uint32_t, hcd) : (n < 2 * G ? lcd : 0u);
      const h8 ap = h8_of(pab, pab, pcd, pcd);
      if constexpr (V2) {
        uint32_t ze, zo;
        quad_index2(cur.v[t4][0][0], cur.v[t4][1][0], cur.v[t4][2][0], cur.v[t4][3][0], ze, zo);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t z = (m & 1) ? zo : ze;
          uint32_t ad;
          if ((m >> 1) == 0) ad = taddr<0, 1>(z, R);
          else if ((m >> 1) == 1) ad = taddr<1, 1>(z, R);
          else if ((m >> 1) == 2) ad = taddr<2, 1>(z, R);
          else ad = taddr<3, 1>(z, R);
          const uint4 ev = *reinterpret_cast<const uint4*>(tab + ad);
          o[m] = mfma32(ap, h8_of(ev.x, ev.y, ev.z, ev.w), o[m]);
        }
      } else {
        const uint32_t wa = value_fields<VB>(cur.v[t4][0]), wb = value_fields<VB>(cur.v[t4][1]);
        const uint32_t wc = value_fields<VB>(cur.v[t4][2]), wd = value_fields<VB>(cur.v[t4][3]);
        // byte k of ze: element 2k (tokens a | b << 4); zo: element 2k + 1
        const uint32_t ze0 = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
        const uint32_t zo0 = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
        const uint32_t ze1 = (wc & 0x0F0F0F0Fu) | ((wd << 4) & 0xF0F0F0F0u);
        const uint32_t zo1 = ((wc >> 4) & 0x0F0F0F0Fu) | (wd & 0xF0F0F0F0u);
        constexpr int RS = VSH ? 0 : 1;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t z0 = (m & 1) ? zo0 : ze0, z1 = (m & 1) ? zo1 : ze1;
          uint32_t i0, i1;
          if ((m >> 1) == 0) { i0 = taddr<0, RS>(z0, R); i1 = taddr<0, RS>(z1, R); }
          else if ((m >> 1) == 1) { i0 = taddr<1, RS>(z0, R); i1 = taddr<1, RS>(z1, R); }
          else if ((m >> 1) == 2) { i0 = taddr<2, RS>(z0, R); i1 = taddr<2, RS>(z1, R); }
          else { i0 = taddr<3, RS>(z0, R); i1 = taddr<3, RS>(z1, R); }
          const uint2 eab = *reinterpret_cast<const uint2*>(tab + i0);
          const uint2 ecd = *reinterpret_cast<const uint2*>(tab + i1);
          o[m] = mfma32(ap, h8_of(eab.x, eab.y, ecd.x, ecd.y), o[m]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  constexpr int kStep = kWaves * kST;
  // ---- main loop: two register sets, the next super tile loading while one is used
  while (st < c1) {
    issue_loads<KB, VB>(rows, buf1, st + kStep, st + kStep < c1, lane);
    process(buf0, st);
    st += kStep;
    if (st >= c1) break;
    issue_loads<KB, VB>(rows, buf0, st + kStep, st + kStep < c1, lane);
    process(buf1, st);
    st += kStep;
  }

  // ---- merge the four waves in LDS (the table is no longer needed) and write this
  // split's partial (m, l, o') per head
  __syncthreads();
  float* comb_o = reinterpret_cast<float*>(tab);
  const float ovs = 1.0f / (kCScale * vs);   // a power of two: o' = o / (64 vs)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * qq + j;
    if (r < 2 * G) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        comb_o[(wave * 2 * kMaxG + r) * QK + 8 * n + m] = o[m][j] * ovs;
    }
  }
  if (qq == 0 && n < G) {
    comb_ml[wave][n][0] = m_run;
    comb_ml[wave][n][1] = l_run;
  }
  __syncthreads();
  const int ns = a.n_split;
  float* ws_o = static_cast<float*>(a.workspace);
  float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * ns * QK;
  const int64_t rbase = (static_cast<int64_t>(b) * a.hq + g * G) * ns;
  for (int idx = tid; idx < G * (QK / 4); idx += kThreads) {
    const int h = idx >> 5, e4 = idx & 31;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, comb_ml[w][h][0]);
    float4 os = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float ls = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float m_w = comb_ml[w][h][0];
        const float f = m_w > -INFINITY ? __builtin_amdgcn_exp2f(m_w - M) : 0.0f;
        const float4 hi4 = reinterpret_cast<const float4*>(comb_o + (w * 2 * kMaxG + h) * QK)[e4];
        const float4 lo4 = reinterpret_cast<const float4*>(comb_o + (w * 2 * kMaxG + G + h) * QK)[e4];
        os.x += f * (hi4.x + lo4.x);
        os.y += f * (hi4.y + lo4.y);
        os.z += f * (hi4.z + lo4.z);
        os.w += f * (hi4.w + lo4.w);
        ls += f * comb_ml[w][h][1];
      }
    }
    const int64_t r = rbase + static_cast<int64_t>(h) * ns + split;
    reinterpret_cast<float4*>(ws_o + r * QK)[e4] = os;
    if (e4 == 0) reinterpret_cast<float2*>(ws_ml)[r] = make_float2(M, ls);
  }
}

// Merge the splits of one (b, query head): weights f_s = exp2(m_s - M), output
// (sum_s f_s o'_s) / (sum_s f_s l_s), then R^T = D H / sqrt(128).  256 threads:
// thread (slice, c) folds float4 column c of splits slice, slice + 8, ... eight at a
// time with a running maximum (the eight loads of a chunk are all in flight
// together); the 8 slices are then combined in LDS.
__global__ void __launch_bounds__(256) attn_merge_splits_kernel(AttnLaunch a, SignWords sw) {
  __shared__ __attribute__((aligned(16))) float po[8][QK];
  __shared__ float pm[8], pl[8];
  __shared__ float ov[QK];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int c4 = tid & 31, sl = tid >> 5;
  const int ns = a.n_split;
  const float* ws_o = static_cast<const float*>(a.workspace);
  const float* ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * ns * QK;
  const int64_t r0 = (static_cast<int64_t>(b) * a.hq + h) * ns;
  float mx = -INFINITY, den = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // chunks of 8 splits per thread: all 16 loads issued, then one rescale per chunk
  for (int s0 = sl; s0 < ns; s0 += 64) {
    float2 ml[8];
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = min(s0 + 8 * k, ns - 1);
      ml[k] = reinterpret_cast<const float2*>(ws_ml)[r0 + s];
      v[k] = reinterpret_cast<const float4*>(ws_o + (r0 + s) * QK)[c4];
    }
    __builtin_amdgcn_sched_barrier(0);   // keep the 16 loads ahead of their uses
    float cm = mx;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (s0 + 8 * k >= ns) ml[k].x = -INFINITY;
      cm = fmaxf(cm, ml[k].x);
    }
    // no branch: with every maximum still -inf all weights are 0 and acc stays 0
    const float f0 = mx > -INFINITY ? __builtin_amdgcn_exp2f(mx - cm) : 0.0f;
    acc = make_float4(acc.x * f0, acc.y * f0, acc.z * f0, acc.w * f0);
    den *= f0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float f = ml[k].x > -INFINITY ? __builtin_amdgcn_exp2f(ml[k].x - cm) : 0.0f;
      acc.x += f * v[k].x;
      acc.y += f * v[k].y;
      acc.z += f * v[k].z;
      acc.w += f * v[k].w;
      den += f * ml[k].y;
    }
    mx = cm;
  }
  reinterpret_cast<float4*>(&po[sl][0])[c4] = acc;
  if (c4 == 0) {
    pm[sl] = mx;
    pl[sl] = den;
  }
  __syncthreads();
  if (tid < QK) {
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, pm[k]);
    float num = 0.0f, dsum = 0.0f;
    if (M > -INFINITY) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float f = pm[k] > -INFINITY ? __builtin_amdgcn_exp2f(pm[k] - M) : 0.0f;
        num += f * po[k][tid];
        dsum += f * pl[k];
      }
    }
    ov[tid] = dsum > 0.0f ? num / dsum : 0.0f;
  }
  __syncthreads();
  if (tid < 64) {
    const float2 v = reinterpret_cast<const float2*>(ov)[lane];
    rotate_out(v, sw, lane, a.out + (static_cast<int64_t>(b) * a.hq + h) * QK);
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
  if (ns > kMaxSplit) ns = kMaxSplit;
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
  // shared key/value entries for 4-bit tables (3-bit key rows have their own layout)
  if (same && tk.bits == 4) {
    FATQ_ATS(4);
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

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
//  * queries: B column h < G holds hi(q'_h), column 15 - h holds lo(q'_h) (q' is
//    scaled by a power of two so that 2^13 <= max |q'| < 2^14).  One DPP add of the
//    mirrored lane (row_mirror) gives both lanes h and 15 - h the full score of head h;
//  * values: B = [hi(v_ta), hi(v_tb), lo(v_ta), lo(v_tb)] for two tokens, and the
//    weights A = [w_ta, w_tb, w_ta, w_tb] with row h = hi(w) and row 15 - h = lo(w)
//    of head h, each lane taking the half of its own row (no lane moves); the two
//    output rows of a head are added at the end.  w = p * n_V * vs with p <= 2^8 (see
//    the softmax below) and vs a power of two per wave, lowered (the accumulator
//    rescaled with it) whenever a super tile holds a value norm n with n * vs > 2^7,
//    so every weight stays below 2^15 and lo(w) is an fp16 normal number unless
//    w < 2^-3: a token's weight is off by at most 2^-22 w + 2^-25 (the fp16 subnormal
//    step), relative to the stream's largest weight 2^-22 + 2^-40, with no sign bias.
// The fp32 normaliser l carries the exact p.  What remains is fp32 accumulation.
//
// Online softmax with a lazy reference (base 2): p = 2^(s - m) against a per-head
// reference m that only moves when a super tile holds a score above m + 8 (or on the
// first tile); then m becomes the tile's true maximum and l and the accumulator are
// rescaled.  So p <= 2^8, and the usual path needs no cross-lane maximum or sum:
// each lane keeps the partial l of its own tokens, added across lanes at the end.
//
// Dequantization is a table look-up in LDS returning a ready MFMA operand; the rows
// are laid out so that a wave's look-ups never share an LDS bank (gfx950: 64 banks,
// a ds_read_b64 serves 32 lanes per cycle, a ds_read_b128 16 lanes):
//  * key rows (bytes [0, 64 KB)): one 256-byte row per index byte r, the 8-byte key
//    entry (two 4-bit key codes of r: low nibble first element) replicated 32 times;
//    lane L reads replica L % 32;
//  * value rows (bytes [64 KB, 128 KB)), unless keys and values share a 4-bit
//    codebook (then the key rows serve both): 2-bit values: r holds the codes of one
//    element in the four tokens of a lane's operand and the 16-byte entry is that
//    whole operand, replicated 16 times (lane L reads replica L % 16); 3/4-bit
//    values: r holds the codes of one element in two tokens, an 8-byte entry
//    replicated 32 times.
// A look-up address is one v_perm of the index byte and the lane's replica offset
// (and, for value rows, the 64 KB base held in a byte of the same lane word).
//
// Token order inside a 16-token tile is the identity: score row r = 4 qq + j is
// token r, which is the token the lane group qq needs for its weight operand, so no
// cross-lane exchange is needed between the products.
//
// Work layout: grid (n_split, Hkv, B), 8 waves per workgroup (one workgroup per
// compute unit: the table takes 128 KB of LDS); the workgroup owns tokens
// [split*chunk, min(len, (split+1)*chunk)) and wave w takes 32-token super tiles
// w, w+8, ... with the codes of the next three super tiles (one for 3-bit values) in
// flight while one is processed.  Within a super tile all key look-ups go out before
// the score products, and all value look-ups (they need only the codes) before the
// softmax, so the LDS latency is paid once per phase rather than at every MFMA.
// Waves merge in LDS and each workgroup stores one partial (m, l, o') per head to the
// workspace; a second kernel, one workgroup per (sequence, KV head), merges the splits
// by log-sum-exp, divides by l, applies R^T = D H / sqrt(128) and writes the output.
// (Merging in the split kernel instead, by the last workgroup of a sequence to arrive
// on a counter, measured slower: the device-scope stores, the counter and the loads
// each cost a full memory round trip inside the kernel.)
//
// MFMA 16x16x32 f16 operand layout (wave64): A[i][k]: lane i%16 + 16*(k/8), slot
// k%8; B[k][j]: lane j + 16*(k/8), slot k%8; D[i][j]: lane j + 16*(i/4), slot i%4.

#include <hip/hip_fp16.h>

#include <type_traits>

#include "fa_tq_internal.h"

namespace fatq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

// Super tiles of codes in flight beyond the one processed (2- and 4-bit values): three
// when a wave's share of a split is long, one when it is at most FATQ_ATTN_SHALLOW_TILES
// super tiles (a deep prefetch there only delays every wave's first codes).
#ifndef FATQ_ATTN_DEPTH
#define FATQ_ATTN_DEPTH 3
#endif
#ifndef FATQ_ATTN_SHALLOW_TILES
#define FATQ_ATTN_SHALLOW_TILES 16
#endif
#ifndef FATQ_ATTN_WANT_WG
#define FATQ_ATTN_WANT_WG 256
#endif

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kST = 32;           // tokens per super tile (2 MFMA tiles)
constexpr int kMaxG = 8;          // query heads per KV head on this path
constexpr int kRow = 256;         // table bytes per index byte
constexpr int kVBase = 65536;     // byte offset of the value rows
constexpr int kMaxSplit = 1024;   // splits per (sequence, KV head)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kCScale = 64.0f;  // centroid pre-scale (exact)
constexpr float kTau = 8.0f;      // a score may pass the reference by this (log2) before a rescale
constexpr float kVMax = 128.0f;   // bound of n_V * vs: weights p n_V vs <= 2^8 * 2^7 = 2^15
// Raw buffer resources: an access at or beyond the range returns zeros, so loads
// past the sequence need no clamp and lanes without work use offset kOOB.
constexpr int32_t kRsrcWord3 = 0x00020000;
constexpr uint32_t kOOB = 0x80000000u;   // every range is below 2^31 (host check)

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

// x = hi + lo, hi the nearest fp16, lo the nearest fp16 of the exact fp32 remainder.
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

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, false));
}

// Maximum over each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));    // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f<0x4E>(x));    // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f<0x141>(x));   // row_half_mirror
  x = fmaxf(x, dpp_f<0x140>(x));   // row_mirror
  return x;
}

__device__ __forceinline__ float max8(const float (&x)[2][4]) {
  return fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
               fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
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

// Raw code words of one super tile as loaded.  Every load is a plain 32- or 128-bit
// word and nothing is computed from it here: the words are only read when the super
// tile is processed, so the compiler's wait for them comes there, not at the load.
//  k[t4]: the key codes of elements 32 qq .. 32 qq + 31 of token 16 t4 + n;
//  v[t4][j]: value codes of token 16 t4 + 4 qq + j holding elements 8 n .. 8 n + 7:
//    2-bit: the 32-bit word with the lane's 16 bits in half n & 1; 3-bit: that word of
//    the low-bit plane, then the word of the high-bit plane with the lane's 8 bits in
//    byte n & 3; 4-bit: the lane's own 32 bits;
//  nk / nv: the 32-bit word holding, in half (t + sh) & 1, the key norm (lanes < 32;
//    nk) or the value norm (lanes >= 32; nv) of token t = s0 + lane % 32 (norm rows are
//    read in aligned words from the row start rounded down to 4 bytes; sh = 1 when
//    the row starts 2 bytes past a word).
template <int KB, int VB>
struct Codes {
  uint32_t k[2][KB == 4 ? 4 : 3];
  uint32_t v[2][4][VB == 3 ? 2 : 1];
  uint32_t nk, nv;
};

// One (sequence, KV head) row of the cache: uniform row starts (norm rows aligned down
// to a word), the readable token count, and the lane's constant byte offsets within a
// super tile.  A super tile's loads use buffer resources based at its first token whose
// range ends at the readable count (zero for a tile not loaded), so the per-tile address
// arithmetic is scalar and a lane past the end reads zeros without touching memory.
struct Rows {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint8_t* kn;
  const uint8_t* vn;
  int ntok;        // tokens [0, ntok) are readable
  int ksh, vsh;    // norm rows: tokens of the half-word offset of their start
  int nsh;         // this lane's (ksh for lanes < 32, vsh for lanes >= 32)
  uint32_t ko, ko3, vo, vo3;   // code offsets of the lane in a super tile (3-bit high planes)
  uint32_t okn, ovn;           // norm word offsets (kOOB for the other half of the wave)
};

template <int KB, int VB>
__device__ __forceinline__ void issue_loads(const Rows& r, Codes<KB, VB>& c, int s0, bool live,
                                            int lane) {
  constexpr uint32_t KCB = cbytes<KB>(), VCB = cbytes<VB>();
  // s0 is even (super tiles start at multiples of 32 tokens), so a norm word of the
  // tile starts at word s0 / 2 of the row
  const uint32_t rem = live && s0 < r.ntok ? static_cast<uint32_t>(r.ntok - s0) : 0u;
  const uint32_t nw = live ? static_cast<uint32_t>(max((r.ntok + r.ksh + 1) / 2 - s0 / 2, 0)) : 0u;
  const uint32_t vw = live ? static_cast<uint32_t>(max((r.ntok + r.vsh + 1) / 2 - s0 / 2, 0)) : 0u;
  const Rsrc kc = make_rsrc(r.kc + static_cast<uint32_t>(s0) * KCB, rem * KCB);
  const Rsrc vc = make_rsrc(r.vc + static_cast<uint32_t>(s0) * VCB, rem * VCB);
  const Rsrc kn = make_rsrc(r.kn + 2u * static_cast<uint32_t>(s0), nw * 4u);
  const Rsrc vn = make_rsrc(r.vn + 2u * static_cast<uint32_t>(s0), vw * 4u);
#pragma unroll
  for (int t4 = 0; t4 < 2; ++t4) {
    if constexpr (KB == 4) {
      const uint4 w = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, r.ko + 16 * KCB * t4, 0, 0));
      c.k[t4][0] = w.x; c.k[t4][1] = w.y; c.k[t4][2] = w.z; c.k[t4][3] = w.w;
    } else {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(kc, r.ko + 16 * KCB * t4, 0, 0);
      c.k[t4][0] = w[0];
      c.k[t4][1] = w[1];
      if constexpr (KB == 3) {
        c.k[t4][2] = __builtin_amdgcn_raw_buffer_load_b32(kc, r.ko3 + 16 * KCB * t4, 0, 0);
      } else {
        c.k[t4][2] = 0;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d = (16 * t4 + j) * VCB;
      c.v[t4][j][0] = __builtin_amdgcn_raw_buffer_load_b32(vc, r.vo + d, 0, 0);
      if constexpr (VB == 3)
        c.v[t4][j][1] = __builtin_amdgcn_raw_buffer_load_b32(vc, r.vo3 + d, 0, 0);
    }
  }
  // (two loads with uniform resources, each lane using one: lanes < 32 the key norm
  // word, lanes >= 32 the value norm word)
  c.nk = __builtin_amdgcn_raw_buffer_load_b32(kn, r.okn, 0, 0);
  c.nv = __builtin_amdgcn_raw_buffer_load_b32(vn, r.ovn, 0, 0);
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

// Value word of elements 8 n .. 8 n + 7 as 4-bit fields (3/4-bit values; n = lane % 16).
template <int VB>
__device__ __forceinline__ uint32_t value_fields(const uint32_t (&w)[VB == 3 ? 2 : 1], int n) {
  if constexpr (VB == 4) return w[0];
  else
    return spread2(__builtin_amdgcn_ubfe(w[0], 16 * (n & 1), 16)) |
           (spread1(__builtin_amdgcn_ubfe(w[1], 8 * (n & 3), 8)) << 2);
}

// Four 16-bit groups of 2-bit value codes (tokens a, b, c, d; field i = element
// 8n + i) -> index bytes: byte k of e = element 2k, of o = element 2k + 1, each
// (code of a) | (b) << 2 | (c) << 4 | (d) << 6.
// The words hold the lane's 16 bits in the half that `sel` picks: 0x05010400 (low
// halves) or 0x07030602 (high halves).
__device__ __forceinline__ void quad_index2(uint32_t wa, uint32_t wb, uint32_t wc, uint32_t wd,
                                            uint32_t sel, uint32_t& e, uint32_t& o) {
  auto pair = [sel](uint32_t x, uint32_t y) {
    // bytes [x.b0, y.b0, x.b1, y.b1] of the lane's halves, then nibble k = (x nibble k)
    // | (y nibble k) << 4, then fields reordered within each byte to (x_2k, y_2k,
    // x_2k+1, y_2k+1)
    uint32_t z = __builtin_amdgcn_perm(y, x, sel);
    uint32_t t = ((z >> 4) ^ z) & 0x00F000F0u;
    z ^= t ^ (t << 4);
    t = ((z >> 2) ^ z) & 0x0C0C0C0Cu;
    return z ^ t ^ (t << 2);
  };
  const uint32_t ab = pair(wa, wb), cd = pair(wc, wd);
  e = (ab & 0x0F0F0F0Fu) | ((cd << 4) & 0xF0F0F0F0u);
  o = ((ab >> 4) & 0x0F0F0F0Fu) | (cd & 0xF0F0F0F0u);
}

// Key-row address of index byte K of word z: (byte << 8) | lane's key replica offset
// (byte 0 of the lane word R).
template <int K>
__device__ __forceinline__ uint32_t kaddr(uint32_t z, uint32_t R) {
  return __builtin_amdgcn_perm(z, R, 0x0C0C0000u | ((4u + K) << 8));
}
// Value-row address: kVBase (byte 2 of R) | (byte << 8) | value replica offset (byte 1).
template <int K>
__device__ __forceinline__ uint32_t vaddr(uint32_t z, uint32_t R) {
  return __builtin_amdgcn_perm(z, R, 0x0C020001u | ((4u + K) << 8));
}

// Workspace: the split partials, o' rows [B][Hq][n_split][QK] then (m, l) pairs
// [B][Hq][n_split][2]; for one (sequence, KV head) the pairs j = h * n_split + split of
// its G heads are contiguous in both.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store4(Rsrc r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ void store2(Rsrc r, uint32_t off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
struct Partials {
  Rsrc o, ml;
};
__device__ __forceinline__ Partials unit_partials(const AttnLaunch& a, int b, int g, int G) {
  const int ns = a.n_split, np = G * ns;
  const int64_t rbase = (static_cast<int64_t>(b) * a.hq + g * G) * ns;
  float* const ws_o = static_cast<float*>(a.workspace);
  float* const ws_ml = ws_o + static_cast<int64_t>(a.batch) * a.hq * ns * QK;
  return {make_rsrc(ws_o + rbase * QK, np * QK * 4), make_rsrc(ws_ml + 2 * rbase, np * 8)};
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

// The row (sequence, KV head) at token offset kvb of the cache, tokens [0, ntok)
// readable.  Norm rows are read as aligned words: the start rounded down to 4 bytes
// (1 token earlier when it is 2 bytes past a word) and the range rounded up to whole
// words; a word never crosses a page, so the last one is always readable.
template <int KB, int VB>
__device__ __forceinline__ Rows make_rows(const AttnLaunch& a, int64_t kvb, int ntok, int lane) {
  constexpr uint32_t KCB = cbytes<KB>(), VCB = cbytes<VB>();
  const int n = lane & 15, qq = lane >> 4;
  Rows r;
  r.kc = a.k_codes + kvb * KCB;
  r.vc = a.v_codes + kvb * VCB;
  const uintptr_t ka = reinterpret_cast<uintptr_t>(a.k_norms + kvb);
  const uintptr_t va = reinterpret_cast<uintptr_t>(a.v_norms + kvb);
  r.ksh = static_cast<int>((ka >> 1) & 1);
  r.vsh = static_cast<int>((va >> 1) & 1);
  r.kn = reinterpret_cast<const uint8_t*>(ka & ~uintptr_t{3});
  r.vn = reinterpret_cast<const uint8_t*>(va & ~uintptr_t{3});
  r.ntok = ntok;
  r.nsh = lane < 32 ? r.ksh : r.vsh;
  // key words: token n of the tile, 16 (4-bit) or 8 bytes of quarter qq; value words:
  // token 4 qq of the tile, the word of element 2n (4-bit) or 4 (n >> 1) (2/3-bit)
  r.ko = n * KCB + (KB == 4 ? 16 : 8) * qq;
  r.ko3 = n * KCB + 32 + 4 * qq;
  r.vo = 4 * qq * VCB + (VB == 4 ? 4 * n : 4 * (n >> 1));
  r.vo3 = 4 * qq * VCB + 32 + 4 * (n >> 2);
  r.okn = lane < 32 ? static_cast<uint32_t>(lane + r.ksh) / 2 * 4 : kOOB;
  r.ovn = lane >= 32 ? static_cast<uint32_t>(lane - 32 + r.vsh) / 2 * 4 : kOOB;
  return r;
}

// VSH: key and value codebooks are identical 4-bit tables, so the key rows serve both.
// GT: the group size G as a compile-time constant (1, 2, 4, 8), or 0 (runtime).
template <int KB, int VB, bool VSH, int GT, int DEPTH>
__global__ void __launch_bounds__(kThreads, 1) attn_mfma_kernel(AttnLaunch a, KTable tk,
                                                                KTable tv, SignWords sw) {
  constexpr bool V2 = VB == 2;
  // super tiles of codes in flight beyond the one processed (3-bit values: their larger
  // register sets leave room for one)
  constexpr int kDepth = VB == 3 ? 1 : DEPTH;
  // the rows, and afterwards the waves' partial outputs for the merge in LDS
  constexpr int kMergeBytes = sizeof(float) * kWaves * 2 * kMaxG * QK;
  constexpr int kTab = (VSH ? kVBase : 2 * kVBase) > kMergeBytes ? (VSH ? kVBase : 2 * kVBase)
                                                                  : kMergeBytes;
  __shared__ __attribute__((aligned(16))) uint8_t tab[kTab];
  __shared__ __attribute__((aligned(16))) uint16_t qhl[2 * kMaxG + 1][QK];   // hi, lo, zero rows
  __shared__ __attribute__((aligned(16))) float nrm[kWaves][2][kST];
  __shared__ uint32_t sp[2][16];
  __shared__ float qmx[kMaxG];
  __shared__ float comb_ml[kWaves][kMaxG][2];
  static_assert(!(VSH && V2), "2-bit values have their own entries");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar tile indices
  const int n = lane & 15, qq = lane >> 4;
  // g: the group of G query heads g * G .. g * G + G - 1, all of KV head g / kv_div
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = GT > 0 ? GT : a.hq / (a.hkv * a.kv_div);
  // lanes of column h < G carry hi(q'_h) and row h of the weights (hi), lanes of
  // column 15 - h the lo halves; the other columns are zero (scores) or unused rows
  const bool hi_lane = n < G;
  const bool use = hi_lane || n >= 16 - G;

  // ---- loads that need only the kernel arguments go out first.  The code rows'
  // resources are built before the query loads, so that every kernel argument
  // arrives in one round of scalar loads.
  const int len_raw = a.lens[b];
  const int c0 = split * a.chunk;
  const int ce = min(a.t_max, c0 + a.chunk);
  const int64_t kvb = (static_cast<int64_t>(b) * a.hkv + g / a.kv_div) * a.t_max;
  Rows rows = make_rows<KB, VB>(a, kvb, ce > 0 ? ce : 0, lane);
  // The query: wave w < G rotates head w, lane holding elements lane and lane + 64
  // (raw bits, widened later); one load form for both dtypes (no branch on the dtype
  // argument): a bf16 element is read as the aligned word holding it.
  uint32_t qraw[2];
  {
    const int hc = wave < G ? wave : 0;
    const int64_t qo = (static_cast<int64_t>(b) * a.hq + g * G + hc) * QK;
    const uint32_t es = a.q_is_bf16 ? 2u : 4u;
    const char* qp = static_cast<const char*>(a.q) + qo * es;
    const uint32_t o0 = (static_cast<uint32_t>(lane) * es) & ~3u;
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(qp + o0);
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(qp + o0 + 64 * es);
    const uint32_t sh = a.q_is_bf16 ? (lane & 1) * 16u : 0u;
    qraw[0] = w0 >> sh;
    qraw[1] = w1 >> sh;
  }
  // sign words of elements lane and lane + 64 (the same word; see sign_bit)
  const uint32_t sw1 = sw.w[0][(lane >> 3) & 3], sw2 = sw.w2[0][(lane >> 3) & 3];
  __builtin_amdgcn_sched_barrier(0);

  // ---- the first super tiles' loads go out at once, bounded by the split's chunk
  // (tokens past the sequence are masked when processed), so they need not wait for
  // the sequence length, which arrives while the table is built
  int st = c0 + wave * kST;
  constexpr int kStep = kWaves * kST;
  // ring of kDepth + 1 register sets: the codes of the next kDepth super tiles are
  // in flight while one is processed
  Codes<KB, VB> buf[kDepth + 1];
#pragma unroll
  for (int i = 0; i < kDepth; ++i)
    issue_loads<KB, VB>(rows, buf[i], st + i * kStep, st + i * kStep < ce, lane);

  // ---- centroid splits, then the operand rows (thread r < 256 fills key row r,
  // thread 256 + r value row r)
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
  {
    const int r = tid & 255;
    uint4 e;
    if (tid < 256) {
      // key row r: the codes of its two elements (3-bit rows: see key_fields)
      const uint32_t a0 = sp[0][KB == 3 ? (r & 3) | ((r >> 2) & 4) : r & 15];
      const uint32_t a1 = sp[0][KB == 3 ? ((r >> 2) & 3) | ((r >> 3) & 4) : r >> 4];
      const uint32_t kh = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // hi(c_lo4), hi(c_hi4)
      const uint32_t kl = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // lo(c_lo4), lo(c_hi4)
      e = make_uint4(kh, kl, kh, kl);
    } else if constexpr (V2) {
      const uint32_t va = sp[1][r & 3], vb = sp[1][(r >> 2) & 3];
      const uint32_t vc = sp[1][(r >> 4) & 3], vd = sp[1][r >> 6];
      e = make_uint4(__builtin_amdgcn_perm(vb, va, 0x05040100u),
                     __builtin_amdgcn_perm(vb, va, 0x07060302u),
                     __builtin_amdgcn_perm(vd, vc, 0x05040100u),
                     __builtin_amdgcn_perm(vd, vc, 0x07060302u));
    } else {
      const uint32_t v0 = sp[1][r & 15], v1 = sp[1][r >> 4];
      const uint32_t vh = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
      const uint32_t vl = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
      e = make_uint4(vh, vl, vh, vl);
    }
    if (tid < 256 || (!VSH && tid < 512)) {
      uint8_t* row = tab + (tid < 256 ? 0 : kVBase) + r * kRow;
      // every 16-byte slot of a row holds the same entry; rotating the slot a step
      // per row index spreads the 16 lanes of one store cycle over all banks
#pragma unroll
      for (int k = 0; k < 16; ++k) reinterpret_cast<uint4*>(row)[(k + r) & 15] = e;
    }
  }

  // ---- q' = s2 * H (s * q) of head `wave`: stride 64 in-lane, strides 32 .. 1 across
  // lanes; its largest |q'| to LDS
  float qx0 = __uint_as_float(a.q_is_bf16 ? qraw[0] << 16 : qraw[0]);
  float qx1 = __uint_as_float(a.q_is_bf16 ? qraw[1] << 16 : qraw[1]);
  {
    const float x0 = bit_of(sw1, lane) ? -qx0 : qx0;
    const float x1 = bit_of(sw1, lane + 64) ? -qx1 : qx1;
    float u = x0 + x1, v = x0 - x1;
    // butterflies of strides 32 .. 1 across lanes (the partner lane's value by a swap
    // across the wave halves, an LDS swizzle across rows, DPP within a row)
    auto stage = [&](auto xor_of, int L) {
      const float pu = xor_of(u), pv = xor_of(v);
      const bool up = (lane & L) != 0;
      u = up ? pu - u : u + pu;
      v = up ? pv - v : v + pv;
    };
    stage([](float x) { return __shfl_xor(x, 32, 64); }, 32);
    stage([](float x) {
      return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                                   0x401F));   // xor 16
    }, 16);
    stage([](float x) { return dpp_f<0x128>(x); }, 8);   // row_ror:8 = xor 8 in a row
    stage([lane](float x) {
      const float r = dpp_f<0x114>(x), l = dpp_f<0x104>(x);   // row_shr:4, row_shl:4
      return (lane & 4) ? r : l;
    }, 4);
    stage([](float x) { return dpp_f<0x4E>(x); }, 2);    // quad_perm [2, 3, 0, 1]
    stage([](float x) { return dpp_f<0xB1>(x); }, 1);    // quad_perm [1, 0, 3, 2]
    qx0 = sw.two && bit_of(sw2, lane) ? -u : u;
    qx1 = sw.two && bit_of(sw2, lane + 64) ? -v : v;
    const float rm = row_max16(fmaxf(fabsf(u), fabsf(v)));
    const float mx = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 0)),
                                 __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 16))),
                           fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 32)),
                                 __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 48))));
    if (lane == 0 && wave < G) qmx[wave] = mx;
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
    if (wave < G) {
      _Float16 hi, lo;
      split_h(qx0 * inv, hi, lo);
      qhl[wave][lane] = __builtin_bit_cast(uint16_t, hi);
      qhl[kMaxG + wave][lane] = __builtin_bit_cast(uint16_t, lo);
      split_h(qx1 * inv, hi, lo);
      qhl[wave][lane + 64] = __builtin_bit_cast(uint16_t, hi);
      qhl[kMaxG + wave][lane + 64] = __builtin_bit_cast(uint16_t, lo);
    }
    if (tid < 64) reinterpret_cast<uint32_t*>(&qhl[2 * kMaxG][0])[tid] = 0u;
  }
  lds_barrier();   // q' halves complete

  // ---- B operands of the score product: k-step m covers elements 32qq + 4m .. +3;
  // column h < G: hi(q'_h), column 15 - h: lo(q'_h), else zero
  h8 bq[8];
  {
    const int qrow = hi_lane ? n : (use ? kMaxG + 15 - n : 2 * kMaxG);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint2 d = *reinterpret_cast<const uint2*>(&qhl[qrow][32 * qq + 4 * m]);
      bq[m] = h8_of(d.x, d.x, d.y, d.y);
    }
  }
  const float sc2 = a.scale * kLog2e * qscale / kCScale;
  // ---- the sequence range; later loads are bounded by the sequence length
  const int64_t len64 = static_cast<int64_t>(len_raw) + a.len_add;
  const int len = len64 < 0 ? 0 : (len64 > a.t_max ? a.t_max : static_cast<int>(len64));
  const int c1 = min(len, c0 + a.chunk);
  rows = make_rows<KB, VB>(a, kvb, len, lane);
  // byte 0: key replica offset, byte 1: value replica offset, byte 2: value-row base
  const uint32_t R = ((lane & 31) << 3) | ((V2 ? (lane & 15) << 4 : (lane & 31) << 3) << 8) |
                     (static_cast<uint32_t>(kVBase >> 16) << 16);

  // byte selector of the lane's 16-bit half in the 2-bit value words
  const uint32_t vsel = (n & 1) ? 0x07030602u : 0x05010400u;
  float m_ref = -INFINITY, l_run = 0.0f;
  bool started = false;   // a super tile has set the softmax reference (wave-uniform)
  // value weight scale of this wave's stream; above any value a norm needs, so the
  // first super tile with a nonzero value norm sets it
  float vs = 18446744073709551616.0f;   // 2^64
  f4 o[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) o[m] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  auto process = [&](const Codes<KB, VB>& cur, int s0) {
    // ---- per-token factors through LDS: key scale, value weight factor n_V * vs
    {
      // (0 past the sequence: the first super tiles are loaded to the chunk's end)
      const float nf = s0 + (lane & 31) < c1
                           ? __half2float(__ushort_as_half(static_cast<uint16_t>(
                                 __builtin_amdgcn_ubfe(lane < 32 ? cur.nk : cur.nv,
                                                       16 * ((s0 + lane + rows.nsh) & 1), 16))))
                           : 0.0f;
      // the largest value norm of the super tile (lanes 32..63; past the sequence the
      // loads return 0) bounds every n_V: lower vs, and rescale the accumulator by the
      // same power of two, when n_V * vs would pass kVMax
      // (tested lane by lane; the wave-wide maximum only when some norm passes)
      if (__ballot(lane >= 32 && nf * vs > kVMax)) {
        const float rm = row_max16(lane >= 32 ? nf : 0.0f);
        const float vmax = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 32)),
                                 __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                     __builtin_bit_cast(int, rm), 48)));
        int e = 0;
        frexpf(vmax, &e);                       // vmax < 2^e
        const float vs_new = ldexpf(kVMax, -e);  // vmax * vs_new < kVMax
        const float r = vs_new / vs;            // a power of two
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] *= r;
        vs = vs_new;
      }
      nrm[wave][lane >> 5][lane & 31] = nf * (lane < 32 ? sc2 : vs);
    }
    __builtin_amdgcn_wave_barrier();
    // ---- key look-ups of both tiles, then the score products: sum = the head's full
    // score before the key factor (hi + lo columns)
    uint2 ke[2][16];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      uint32_t f[4];
      key_fields<KB>(cur.k[t4], f);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = f[m >> 1];
        uint32_t a0, a1;
        if (m & 1) {
          a0 = kaddr<2>(w, R);
          a1 = kaddr<3>(w, R);
        } else {
          a0 = kaddr<0>(w, R);
          a1 = kaddr<1>(w, R);
        }
        ke[t4][2 * m] = *reinterpret_cast<const uint2*>(tab + a0);
        ke[t4][2 * m + 1] = *reinterpret_cast<const uint2*>(tab + a1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float sum[2][4];
    float4 fk[2];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint2 e0 = ke[t4][2 * m], e1 = ke[t4][2 * m + 1];
        acc = mfma32(h8_of(e0.x, e0.y, e1.x, e1.y), bq[m], acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[t4][j] = acc[j] + dpp_f<0x140>(acc[j]);   // row_mirror
      fk[t4] = *reinterpret_cast<const float4*>(&nrm[wave][0][16 * t4 + 4 * qq]);
    }
    // ---- value look-ups of both tiles (B operands; they need only the codes), in
    // flight during the softmax
    using VEnt = typename std::conditional<V2, uint4, uint2>::type;
    VEnt ve[2][V2 ? 8 : 16];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      if constexpr (V2) {
        uint32_t ze, zo;
        quad_index2(cur.v[t4][0][0], cur.v[t4][1][0], cur.v[t4][2][0], cur.v[t4][3][0], vsel,
                    ze, zo);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t z = (m & 1) ? zo : ze;
          uint32_t ad;
          if ((m >> 1) == 0) ad = vaddr<0>(z, R);
          else if ((m >> 1) == 1) ad = vaddr<1>(z, R);
          else if ((m >> 1) == 2) ad = vaddr<2>(z, R);
          else ad = vaddr<3>(z, R);
          ve[t4][m] = *reinterpret_cast<const VEnt*>(tab + ad);
        }
      } else {
        const uint32_t wa4 = value_fields<VB>(cur.v[t4][0], n);
        const uint32_t wb4 = value_fields<VB>(cur.v[t4][1], n);
        const uint32_t wc4 = value_fields<VB>(cur.v[t4][2], n);
        const uint32_t wd4 = value_fields<VB>(cur.v[t4][3], n);
        // byte k of ze: element 2k (tokens a | b << 4); zo: element 2k + 1
        const uint32_t ze0 = (wa4 & 0x0F0F0F0Fu) | ((wb4 << 4) & 0xF0F0F0F0u);
        const uint32_t zo0 = ((wa4 >> 4) & 0x0F0F0F0Fu) | (wb4 & 0xF0F0F0F0u);
        const uint32_t ze1 = (wc4 & 0x0F0F0F0Fu) | ((wd4 << 4) & 0xF0F0F0F0u);
        const uint32_t zo1 = ((wc4 >> 4) & 0x0F0F0F0Fu) | (wd4 & 0xF0F0F0F0u);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t z0 = (m & 1) ? zo0 : ze0, z1 = (m & 1) ? zo1 : ze1;
          uint32_t i0, i1;
          if constexpr (VSH) {
            if ((m >> 1) == 0) { i0 = kaddr<0>(z0, R); i1 = kaddr<0>(z1, R); }
            else if ((m >> 1) == 1) { i0 = kaddr<1>(z0, R); i1 = kaddr<1>(z1, R); }
            else if ((m >> 1) == 2) { i0 = kaddr<2>(z0, R); i1 = kaddr<2>(z1, R); }
            else { i0 = kaddr<3>(z0, R); i1 = kaddr<3>(z1, R); }
          } else {
            if ((m >> 1) == 0) { i0 = vaddr<0>(z0, R); i1 = vaddr<0>(z1, R); }
            else if ((m >> 1) == 1) { i0 = vaddr<1>(z0, R); i1 = vaddr<1>(z1, R); }
            else if ((m >> 1) == 2) { i0 = vaddr<2>(z0, R); i1 = vaddr<2>(z1, R); }
            else { i0 = vaddr<3>(z0, R); i1 = vaddr<3>(z1, R); }
          }
          ve[t4][2 * m] = *reinterpret_cast<const VEnt*>(tab + i0);
          ve[t4][2 * m + 1] = *reinterpret_cast<const VEnt*>(tab + i1);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- exponents against the reference: x = s - m_ref (masked tokens -inf)
    float x[2][4];
    const float nm = -m_ref;
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      x[t4][0] = fmaf(sum[t4][0], fk[t4].x, nm);
      x[t4][1] = fmaf(sum[t4][1], fk[t4].y, nm);
      x[t4][2] = fmaf(sum[t4][2], fk[t4].z, nm);
      x[t4][3] = fmaf(sum[t4][3], fk[t4].w, nm);
    }
    const bool partial = s0 + kST > c1;   // uniform: only a stream's last super tile
    if (partial) {
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          x[t4][j] = s0 + 16 * t4 + 4 * qq + j < c1 ? x[t4][j] : -INFINITY;
    }
    // a score above m_ref + kTau (or the first tile, m_ref = -inf: x = +inf) moves the
    // reference to the super tile's true maximum
    // (the test compares the bit patterns as integers: for a positive bound that is the
    // float order, -inf and every negative value fall below it, +inf and NaN above)
    int xm = __builtin_bit_cast(int, x[0][0]);
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
      for (int j = 0; j < 4; ++j) xm = max(xm, __builtin_bit_cast(int, x[t4][j]));
    if (__ballot(use && xm > __builtin_bit_cast(int, kTau))) {
      float sc[2][4];
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) {
        sc[t4][0] = sum[t4][0] * fk[t4].x;
        sc[t4][1] = sum[t4][1] * fk[t4].y;
        sc[t4][2] = sum[t4][2] * fk[t4].z;
        sc[t4][3] = sum[t4][3] * fk[t4].w;
        if (partial) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sc[t4][j] = s0 + 16 * t4 + 4 * qq + j < c1 ? sc[t4][j] : -INFINITY;
        }
      }
      float mt = max8(sc);
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_ref, mt);
      if (started) {   // nothing to rescale before the first super tile
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l_run *= alpha;
        // accumulator row 4 qq + j belongs to head r (r < G) or 15 - r (r >= 16 - G)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * qq + j;
          const float ar = __shfl(alpha, r < G ? r : 15 - r, 64);
#pragma unroll
          for (int m = 0; m < 8; ++m) o[m][j] *= ar;
        }
      }
      started = true;
      m_ref = m_new;
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[t4][j] = sc[t4][j] - m_ref;
    }
    float p[2][4];
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[t4][j] = __builtin_amdgcn_exp2f(x[t4][j]);
        l_run += p[t4][j];
      }
    // ---- value product: A = [w_a, w_b, w_a, w_b, w_c, w_d, w_c, w_d] for tokens
    // 4qq..4qq+3, the hi halves in the rows of lanes h < G, the lo halves in rows 15 - h
#pragma unroll
    for (int t4 = 0; t4 < 2; ++t4) {
      const float4 fv = *reinterpret_cast<const float4*>(&nrm[wave][1][16 * t4 + 4 * qq]);
      const float wa = p[t4][0] * fv.x, wb = p[t4][1] * fv.y;
      const float wc = p[t4][2] * fv.z, wd = p[t4][3] * fv.w;
      _Float16 ha, la, hb, lb, hc, lc, hd, ld;
      split_h(wa, ha, la);
      split_h(wb, hb, lb);
      split_h(wc, hc, lc);
      split_h(wd, hd, ld);
      const uint32_t pab = hi_lane ? pack_h2(ha, hb) : pack_h2(la, lb);
      const uint32_t pcd = hi_lane ? pack_h2(hc, hd) : pack_h2(lc, ld);
      const h8 ap = h8_of(pab, pab, pcd, pcd);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if constexpr (V2) {
          const uint4 ev = ve[t4][m];
          o[m] = mfma32(ap, h8_of(ev.x, ev.y, ev.z, ev.w), o[m]);
        } else {
          const uint2 eab = ve[t4][2 * m], ecd = ve[t4][2 * m + 1];
          o[m] = mfma32(ap, h8_of(eab.x, eab.y, ecd.x, ecd.y), o[m]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- main loop over the ring, kDepth + 1 super tiles per pass: the loads of set
  // i + kDepth go out before set i is processed, every step issuing its loads so that
  // the compiler's count of loads in flight is the same on every path; a super tile
  // past this split's stream is loaded at the out-of-range offset (zeros, no memory
  // access: the tokens after the chunk are the next split's) and not processed (a
  // uniform branch)
  const int n_tiles = st < c1 ? (c1 - st + kStep - 1) / kStep : 0;
  for (int it = 0; it < n_tiles; it += kDepth + 1) {
#pragma unroll
    for (int i = 0; i <= kDepth; ++i) {
      const int sn = st + kDepth * kStep;
      issue_loads<KB, VB>(rows, buf[(i + kDepth) % (kDepth + 1)], sn, sn < c1, lane);
      if (st < c1) process(buf[i], st);
      st += kStep;
    }
  }

  // ---- merge the waves in LDS (the table is no longer needed) and write this
  // split's partial (m, l, o') per head
  __syncthreads();
  float* comb_o = reinterpret_cast<float*>(tab);
  const float ovs = 1.0f / (kCScale * vs);   // a power of two: o' = o / (64 vs)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * qq + j;
    const int slot = r < G ? r : (r >= 16 - G ? kMaxG + 15 - r : -1);
    if (slot >= 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        comb_o[(wave * 2 * kMaxG + slot) * QK + 8 * n + m] = o[m][j] * ovs;
    }
  }
  // the head's l: the lanes of its column in the four row groups
  float lsum = l_run + __shfl_xor(l_run, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (qq == 0 && hi_lane) {
    comb_ml[wave][n][0] = m_ref;
    comb_ml[wave][n][1] = lsum;
  }
  __syncthreads();
  const int ns = a.n_split;
  const Partials pt = unit_partials(a, b, g, G);
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
        const float4 lo4 =
            reinterpret_cast<const float4*>(comb_o + (w * 2 * kMaxG + kMaxG + h) * QK)[e4];
        os.x += f * (hi4.x + lo4.x);
        os.y += f * (hi4.y + lo4.y);
        os.z += f * (hi4.z + lo4.z);
        os.w += f * (hi4.w + lo4.w);
        ls += f * comb_ml[w][h][1];
      }
    }
    const int j = h * ns + split;
    store4(pt.o, (j * QK + 4 * e4) * 4, os);
    if (e4 == 0) store2(pt.ml, j * 8, make_float2(M, ls));
  }
}

// Merge the splits of one (b, query head): weights f_s = exp2(m_s - M), output
// (sum_s f_s o'_s) / (sum_s f_s l_s), then R^T = D H / sqrt(128).  256 threads:
// thread (slice, c) folds float4 column c of splits slice, slice + 8, ... eight at a
// time with a running maximum (the eight loads of a chunk are all in flight
// together); the 8 slices are then combined in LDS.
// DENSE: the codes are those of a dense rotation R (d x d, d <= 128) and the output is
// R^T o over the first d elements; thread (half, i) sums rows 64 half .. 64 half + 63 of
// column i of R, loaded before the partials (row and column indexes clamped into R;
// the rows past d meet zeros of o).
template <bool DENSE>
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
  [[maybe_unused]] float rv[DENSE ? 64 : 1];
  if constexpr (DENSE) {
    const int d = a.dense_dim, col = min(tid & (QK - 1), d - 1), k0 = (tid >> 7) * 64;
#pragma unroll
    for (int m = 0; m < 64; ++m) rv[m] = a.dense_rot[min(k0 + m, d - 1) * d + col];
  }
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
    if constexpr (DENSE) {
      if (tid >= a.dense_dim) ov[tid] = 0.0f;
    }
  }
  __syncthreads();
  if constexpr (DENSE) {
    const int d = a.dense_dim, k0 = (tid >> 7) * 64;
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 64; ++m) acc = __builtin_fmaf(rv[m], ov[k0 + m], acc);
    float* half = &po[0][0];   // rows 0 and 1 of po (their reads ended at the barrier)
    half[tid] = acc;
    __syncthreads();
    if (tid < d) a.out[(static_cast<int64_t>(b) * a.hq + h) * d + tid] = half[tid] + half[tid + QK];
  } else if (tid < 64) {
    const float2 v = reinterpret_cast<const float2*>(ov)[lane];
    rotate_out(v, sw, lane, a.out + (static_cast<int64_t>(b) * a.hq + h) * QK);
  }
}

}  // namespace

// Workgroups per KV head: the smallest r dividing the group size hq / hkv with at most
// kMaxG query heads per workgroup (each of the r reads the KV head's codes).
int32_t attn_mfma_groups(int32_t hq, int32_t hkv) {
  const int32_t G = hq / hkv;
  int32_t r = (G + kMaxG - 1) / kMaxG;
  while (G % r != 0) ++r;
  return r;
}

// Splits per (sequence, KV head) so that the grid holds about FATQ_ATTN_WANT_WG
// workgroups (one per compute unit), each chunk a multiple of a round of super tiles
// (kWaves * kST tokens) so every wave of a full chunk gets the same work.
void attn_mfma_partition(int32_t batch, int32_t hkv, int32_t t_max, int32_t* n_split,
                         int32_t* chunk) {
  constexpr int64_t kRound = kWaves * kST;
  const int64_t units = static_cast<int64_t>(batch > 0 ? batch : 1) * hkv;
  const int64_t want = FATQ_ATTN_WANT_WG;
  int64_t ns = (want + units - 1) / units;
  const int64_t max_ns = t_max > 0 ? (t_max + kRound - 1) / kRound : 1;
  if (ns > max_ns) ns = max_ns;
  if (ns > kMaxSplit) ns = kMaxSplit;
  if (ns < 1) ns = 1;
  int64_t c = t_max > 0 ? (t_max + ns - 1) / ns : kRound;
  c = (c + kRound - 1) / kRound * kRound;
  ns = t_max > 0 ? (t_max + c - 1) / c : 1;
  *n_split = static_cast<int32_t>(ns);
  *chunk = static_cast<int32_t>(c);
}

size_t attn_mfma_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t n_split) {
  return static_cast<size_t>(batch) * hq * n_split * (QK + 2) * sizeof(float);
}

template <int GT>
void launch_g(const AttnLaunch& a, const KTable& tk, const KTable& tv, const SignWords& sw,
              hipStream_t stream, bool same) {
  const dim3 g1(a.n_split, a.hkv * a.kv_div, a.batch), b1(kThreads);
  const bool shallow = a.chunk <= FATQ_ATTN_SHALLOW_TILES * kWaves * kST;
  constexpr int kDeep = FATQ_ATTN_DEPTH;
  // (3-bit values take one super tile in flight either way: one instantiation)
#define FATQ_ATT(K, V)                                                                         \
  if ((V) == 3 || shallow)                                                                    \
    hipLaunchKernelGGL((attn_mfma_kernel<K, V, false, GT, 1>), g1, b1, 0, stream, a, tk, tv,  \
                       sw);                                                                   \
  else                                                                                        \
    hipLaunchKernelGGL((attn_mfma_kernel<K, V, false, GT, (V) == 3 ? 1 : kDeep>), g1, b1, 0,  \
                       stream, a, tk, tv, sw)
#define FATQ_ATS(K)                                                                            \
  if (shallow)                                                                                \
    hipLaunchKernelGGL((attn_mfma_kernel<K, K, true, GT, 1>), g1, b1, 0, stream, a, tk, tv,   \
                       sw);                                                                   \
  else                                                                                        \
    hipLaunchKernelGGL((attn_mfma_kernel<K, K, true, GT, kDeep>), g1, b1, 0, stream, a, tk,   \
                       tv, sw)
  // shared key/value rows for identical 4-bit tables (3-bit key rows have their own layout)
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
  switch (a.hq / (a.hkv * a.kv_div)) {
    case 1: launch_g<1>(a, tk, tv, sw, stream, same); break;
    case 2: launch_g<2>(a, tk, tv, sw, stream, same); break;
    case 4: launch_g<4>(a, tk, tv, sw, stream, same); break;
    case 8: launch_g<8>(a, tk, tv, sw, stream, same); break;
    default: launch_g<0>(a, tk, tv, sw, stream, same); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.dense_rot)
    hipLaunchKernelGGL(attn_merge_splits_kernel<true>, dim3(a.hq, a.batch), dim3(256), 0, stream,
                       a, sw);
  else
    hipLaunchKernelGGL(attn_merge_splits_kernel<false>, dim3(a.hq, a.batch), dim3(256), 0,
                       stream, a, sw);
  return hipGetLastError();
}

}  // namespace fatq

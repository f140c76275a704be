// Host front-end of the C ABI declared in include/fa_tq.h: argument checks, the
// Lloyd-Max codebook builder, the sign diagonal, and kernel launches.
//
// Pages cited: [Spec] "TurboQuant KV Cache Compression -- Spec";
//              [turboq] "TurboQuant KV Cache (turboq2 / turboq3 / turboq4)".

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fa_tq_internal.h"

namespace {

thread_local std::string g_last_error;

fa_tq_status fail(fa_tq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa_tq_status ok() { return FA_TQ_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Lloyd-Max for the density proportional to (1 - y^2)^m on [-1, 1], m = dim/2 - 1
// ([Spec] "Step 2" and "Codebook Generation").  The cell mass is computed from the
// regularized incomplete beta function (continued fraction, modified Lentz), the
// first moment in closed form; only the positive half is iterated and mirrored.

// Continued fraction for I_x(a, b), valid for x < (a + 1) / (a + b + 2).
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  const double qab = a + b, qap = a + 1.0, qam = a - 1.0;
  double c = 1.0;
  double d = 1.0 - qab * x / qap;
  if (std::fabs(d) < tiny) d = tiny;
  d = 1.0 / d;
  double h = d;
  for (int k = 1; k <= 100000; ++k) {
    const double k2 = 2.0 * k;
    double aa = k * (b - k) * x / ((qam + k2) * (a + k2));
    d = 1.0 + aa * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + aa / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    h *= d * c;
    aa = -(a + k) * (qab + k) * x / ((a + k2) * (qap + k2));
    d = 1.0 + aa * d;
    if (std::fabs(d) < tiny) d = tiny;
    c = 1.0 + aa / c;
    if (std::fabs(c) < tiny) c = tiny;
    d = 1.0 / d;
    const double del = d * c;
    h *= del;
    if (std::fabs(del - 1.0) < 1e-16) break;
  }
  return h;
}

// Upper tail of the symmetric law: T(y) = P(Y > y) for y in [0, 1], where
// (1 + Y) / 2 ~ Beta(p, p);  T(y) = I_{(1-y)/2}(p, p).
double upper_tail(double y, double p, double lnB) {
  if (y <= 0.0) return 0.5;
  if (y >= 1.0) return 0.0;
  const double x = 0.5 * (1.0 - y);
  const double front = std::exp(p * std::log(x) + p * std::log1p(-x) - lnB) / p;
  return front * beta_cf(p, p, x);
}

bool lloyd_max(int dim, int bits, float* boundaries, float* centroids) {
  const int L = 1 << bits;
  const int half = L / 2;
  const double m = dim / 2.0 - 1.0;
  const double p = m + 1.0;
  const double lnB = 2.0 * std::lgamma(p) - std::lgamma(2.0 * p);
  const double lnK = (2.0 * m + 1.0) * std::log(2.0) + lnB;  // mass = K * dT
  const double K = std::exp(lnK);
  std::vector<double> pos(half - 1), cent(half), edges(half + 1);
  for (int k = 0; k < half - 1; ++k) pos[k] = 2.0 * (half + 1 + k) / L - 1.0;
  auto centroids_of = [&](const std::vector<double>& bnd) {
    edges[0] = 0.0;
    for (int k = 0; k < half - 1; ++k) edges[k + 1] = bnd[k];
    edges[half] = 1.0;
    for (int j = 0; j < half; ++j) {
      const double a = edges[j], b = edges[j + 1];
      const double f1 = (std::pow(1.0 - a * a, p) - std::pow(1.0 - b * b, p)) / (2.0 * p);
      const double f0 = K * (upper_tail(a, p, lnB) - upper_tail(b, p, lnB));
      cent[j] = f1 / f0;
    }
  };
  for (int it = 0; it < 100000; ++it) {
    centroids_of(pos);
    double delta = 0.0;
    for (int k = 0; k < half - 1; ++k) {
      const double nb = 0.5 * (cent[k] + cent[k + 1]);
      delta = std::fmax(delta, std::fabs(nb - pos[k]));
      pos[k] = nb;
    }
    if (delta < 1e-12) break;
  }
  centroids_of(pos);
  for (int j = 0; j < half; ++j) {
    if (!std::isfinite(cent[j])) return false;
    centroids[half + j] = static_cast<float>(cent[j]);
    centroids[half - 1 - j] = static_cast<float>(-cent[j]);
  }
  boundaries[half - 1] = 0.0f;
  for (int k = 0; k < half - 1; ++k) {
    boundaries[half + k] = static_cast<float>(pos[k]);
    boundaries[half - 2 - k] = static_cast<float>(-pos[k]);
  }
  return true;
}

// SplitMix64 (Steele, Lea and Flood 2014), written from its published definition.
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

void make_signs(uint64_t seed, int head_dim, int8_t* out) {
  SplitMix64 g{seed};
  for (int i = 0; i < head_dim; ++i) out[i] = (g.next() >> 63) ? -1 : 1;
}

// Sign words of s1 (draws 0 .. d-1 of the seed's stream) and, for the two-sign
// rotation, s2 (draws d .. 2d-1).
fatq::SignWords make_sign_words(uint64_t seed, int head_dim, bool two = false) {
  std::vector<int8_t> s(2 * static_cast<size_t>(head_dim));
  make_signs(seed, 2 * head_dim, s.data());
  fatq::SignWords sw;
  std::memset(&sw, 0, sizeof(sw));
  sw.two = two ? 1 : 0;
  for (int j = 0; j < head_dim / fatq::QK; ++j)
    for (int q = 0; q < 4; ++q)
      for (int k = 0; k < 4; ++k)
        for (int i = 0; i < 8; ++i) {
          const int e = fatq::QK * j + 8 * (q + 4 * k) + i;
          if (s[e] < 0) sw.w[j][q] |= 1u << (8 * k + i);
          if (two && s[head_dim + e] < 0) sw.w2[j][q] |= 1u << (8 * k + i);
        }
  return sw;
}

// Whole-vector mode: transform length of a head_dim-d vector, d itself for 128 and
// 256, else the next of the two ([Spec] "Hadamard Transform Detail": a head_dim that
// is not a power of two is zero-padded to the next one).
int32_t whole_length(int32_t head_dim) { return head_dim <= 128 ? 128 : 256; }

// Whole-vector mode: 64 < head_dim <= 256, a multiple of 8 (one 16-byte bf16 chunk),
// and a 2-4 bit codebook.
fa_tq_status check_whole(const fa_tq_codebook* cb, int32_t head_dim, const char* who) {
  if (head_dim <= 64 || head_dim > 256 || head_dim % 8 != 0)
    return fail(FA_TQ_EUNSUPPORTED,
                "%s: whole-vector mode for head_dim in (64, 256], a multiple of 8 (got %d)", who,
                head_dim);
  if (cb && cb->bits == 8)
    return fail(FA_TQ_EUNSUPPORTED, "%s: whole-vector mode needs a 2-4 bit codebook", who);
  return ok();
}

// Flags of the _ex entry points.  Encode takes both; decode and attention take the
// rotation flag only (the corrected norm is a property of the stored norms).
fa_tq_status check_flags(uint32_t flags, uint32_t allowed, const fa_tq_codebook* cb,
                         const char* who) {
  if ((flags & FA_TQ_WHOLE_VECTOR) && !(allowed & FA_TQ_WHOLE_VECTOR))
    return fail(FA_TQ_EUNSUPPORTED, "%s: the whole-vector mode has encode and decode only", who);
  if ((flags & FA_TQ_WHOLE_VECTOR) && (flags & ~FA_TQ_WHOLE_VECTOR))
    return fail(FA_TQ_EUNSUPPORTED, "%s: the whole-vector mode takes no other flag", who);
  if (flags & ~allowed) return fail(FA_TQ_EINVAL, "%s: unknown flags 0x%x", who, flags & ~allowed);
  if ((flags & FA_TQ_NORM_CORRECT) && cb && cb->bits == 8)
    return fail(FA_TQ_EUNSUPPORTED, "%s: the corrected norm needs a 2-4 bit codebook", who);
  if ((flags & FA_TQ_TWO_SIGNS) && cb && cb->bits != 8) {
    // the encoder applies s2 by mirroring codes through the table's symmetry
    const int L = cb->levels;
    bool sym = true;
    for (int j = 0; j + 1 < L; ++j) sym = sym && cb->boundaries[j] == -cb->boundaries[L - 2 - j];
    for (int j = 0; j < L; ++j) sym = sym && cb->centroids[j] == -cb->centroids[L - 1 - j];
    if (!sym)
      return fail(FA_TQ_EUNSUPPORTED,
                  "%s: the two-sign rotation needs a mirror-symmetric codebook", who);
  }
  return ok();
}

// Uniform parameters of the encoder's cell table (see KTable): a cell is the set
// of fp32 values sharing sign, exponent and two leading mantissa bits; the cells
// whose exponent lies outside the nonzero boundaries' range hold no boundary, so
// base = #{j : b_j < any value of the cell} follows from the sign and the side.
void fill_cell_params(fatq::KTable* tab) {
  const int nb = tab->nb;
  for (int j = nb; j < 15; ++j) tab->b[j] = INFINITY;
  uint32_t emin = 0xFFu, emax = 0u, nneg = 0u, nle0 = 0u;
  for (int j = 0; j < nb; ++j) {
    const float bj = tab->b[j];
    uint32_t u;
    std::memcpy(&u, &bj, 4);
    const uint32_t e = (u >> 23) & 0xFFu;
    if (bj != 0.0f) {
      emin = e < emin ? e : emin;
      emax = e > emax ? e : emax;
    }
    nneg += bj < 0.0f ? 1u : 0u;
    nle0 += bj <= 0.0f ? 1u : 0u;
  }
  if (emin > emax) emin = emax = 0;   // no nonzero boundary: only the zero cells count
  tab->emin = emin;
  tab->emax = emax;
  // the +0 cell: #{b_j < +0} = nneg, and its threshold may be a zero boundary
  const uint32_t bases[5] = {nle0, nneg, static_cast<uint32_t>(nb), 0u, nneg};
  for (int k = 0; k < 5; ++k) {
    const uint32_t base = bases[k];
    const float thr = base < static_cast<uint32_t>(nb) ? tab->b[base] : INFINITY;
    const float c0 = tab->c[base], c1 = tab->c[base + 1 < 16 ? base + 1 : 15];
    const float q0 = c0 * c0, q1 = c1 * c1;   // fp32 products, as the kernel's
    std::memcpy(&tab->cell_out[k][0], &thr, 4);
    tab->cell_out[k][1] = base;
    std::memcpy(&tab->cell_out[k][2], &q0, 4);
    std::memcpy(&tab->cell_out[k][3], &q1, 4);
  }
}

fa_tq_status check_codebook(const fa_tq_codebook* cb, const char* what, bool allow8,
                            fatq::KTable* tab, int32_t dim = fatq::QK) {
  if (!cb) return fail(FA_TQ_EINVAL, "%s: codebook pointer is NULL", what);
  if (cb->dim != dim)
    return fail(FA_TQ_EINVAL, "%s: codebook dim %d, expected %d (the transform length)", what,
                cb->dim, dim);
  const int bits = cb->bits;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8))
    return fail(FA_TQ_EINVAL, "%s: bits %d not in {2, 3, 4, 8}", what, bits);
  if (cb->levels != (1 << bits))
    return fail(FA_TQ_EINVAL, "%s: levels %d != 1 << bits (%d)", what, cb->levels, 1 << bits);
  if (bits == 8 && !allow8)
    return fail(FA_TQ_EUNSUPPORTED, "%s: the 8-bit grid is supported by encode/decode only",
                what);
  std::memset(tab, 0, sizeof(*tab));
  tab->bits = bits;
  if (bits == 8) {
    tab->nb = 255;
    return ok();
  }
  const int L = cb->levels;
  tab->nb = L - 1;
  for (int j = 0; j < L - 1; ++j) {
    if (!std::isfinite(cb->boundaries[j]))
      return fail(FA_TQ_EINVAL, "%s: boundary %d is not finite", what, j);
    if (j > 0 && !(cb->boundaries[j] > cb->boundaries[j - 1]))
      return fail(FA_TQ_EINVAL, "%s: boundaries are not strictly ascending at %d", what, j);
    tab->b[j] = cb->boundaries[j];
  }
  // The encoder bucketizes through a table of fp32 cells (values sharing their top
  // 11 bits) that holds at most one boundary per cell.
  for (int j = 0; j + 1 < L - 1; ++j) {
    uint32_t u0, u1;
    std::memcpy(&u0, &cb->boundaries[j], 4);
    std::memcpy(&u1, &cb->boundaries[j + 1], 4);
    if ((u0 >> 21) == (u1 >> 21))
      return fail(FA_TQ_EUNSUPPORTED,
                  "%s: boundaries %d and %d are closer than the encoder's cell resolution "
                  "(ratio <= 1.25)", what, j, j + 1);
  }
  for (int j = 0; j < L; ++j) {
    if (!std::isfinite(cb->centroids[j]))
      return fail(FA_TQ_EINVAL, "%s: centroid %d is not finite", what, j);
    tab->c[j] = cb->centroids[j];
  }
  fill_cell_params(tab);
  return ok();
}

fa_tq_status check_head_dim(int32_t head_dim) {
  if (head_dim <= 0 || head_dim % fatq::QK != 0 || head_dim > FA_TQ_MAX_HEAD_DIM)
    return fail(FA_TQ_EINVAL,
                "head_dim %d must be a positive multiple of 128 and at most %d", head_dim,
                FA_TQ_MAX_HEAD_DIM);
  return ok();
}

fa_tq_status launched(hipError_t e, const char* what) {
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(FA_TQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

fa_tq_status encode_impl(const char* who, const fa_tq_codebook* cb, uint64_t seed,
                         uint32_t flags, int32_t head_dim,
                          const void* x, fa_tq_dtype x_dtype, fa_tq_layout x_layout,
                          int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                          const int32_t* t0, int32_t t_max, uint8_t* codes, uint16_t* norms,
                          void* stream, bool ring, bool check_only = false,
                          fatq::EncodeLaunch* prep = nullptr, fatq::KTable* prep_tab = nullptr,
                          fatq::SignWords* prep_sw = nullptr) {
  fatq::KTable tab;
  const bool whole = (flags & FA_TQ_WHOLE_VECTOR) != 0;
  fa_tq_status st = check_flags(
      flags, FA_TQ_TWO_SIGNS | FA_TQ_NORM_CORRECT | (ring ? 0u : FA_TQ_WHOLE_VECTOR), cb, who);
  if (st != FA_TQ_OK) return st;
  if (whole && (st = check_whole(cb, head_dim, who)) != FA_TQ_OK) return st;
  // transform length: head_dim, or its zero-padded length in the whole-vector mode
  const int32_t dt = whole ? whole_length(head_dim) : head_dim;
  if ((st = check_codebook(cb, who, true, &tab, whole ? dt : fatq::QK)) != FA_TQ_OK)
    return st;
  if (!whole && (st = check_head_dim(head_dim)) != FA_TQ_OK) return st;
  if (batch < 0 || n_kv_heads < 0 || n_tokens < 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: negative size", who);
  if (x_dtype != FA_TQ_F32 && x_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: input dtype %d", who, (int)x_dtype);
  if (batch == 0 || n_kv_heads == 0 || n_tokens == 0) return ok();
  if (!x || !codes || !norms)
    return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if (!aligned16(x) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(norms) & 1u))
    return fail(FA_TQ_EINVAL, "%s: x and codes must be 16-byte aligned, norms 2-byte", who);
  if (x_layout.stride_b % 8 || x_layout.stride_h % 8 || x_layout.stride_t % 8 ||
      x_layout.stride_b < 0 || x_layout.stride_h < 0 || x_layout.stride_t < 0)
    return fail(FA_TQ_EINVAL, "%s: strides must be non-negative multiples of 8", who);
  if (n_tokens > t_max && !t0)
    return fail(FA_TQ_EINVAL, "%s: n_tokens %d > t_max %d", who, n_tokens, t_max);
  // The kernel addresses one (batch, head) row of input, codes and norms with 32-bit
  // byte offsets below 2^31.
  const int64_t esize = x_dtype == FA_TQ_BF16 ? 2 : 4;
  const int64_t xrow = ((static_cast<int64_t>(n_tokens) - 1) * x_layout.stride_t + head_dim) * esize;
  const int64_t crow = static_cast<int64_t>(t_max) * (dt / fatq::QK) * fa_tq_code_bytes(cb->bits);
  if (xrow >= (int64_t{1} << 31) || crow >= (int64_t{1} << 31))
    return fail(FA_TQ_EUNSUPPORTED, "%s: one (batch, head) row spans 2 GiB or more", who);
  if (check_only) return ok();
  fatq::EncodeLaunch a;
  a.x = x;
  a.sb = x_layout.stride_b;
  a.sh = x_layout.stride_h;
  a.st = x_layout.stride_t;
  a.batch = batch;
  a.heads = n_kv_heads;
  a.tokens = n_tokens;
  a.nblk = dt / fatq::QK;
  a.dim = head_dim;
  a.t_max = t_max;
  a.t0 = t0;
  a.ring = ring ? 1 : 0;
  a.codes = codes;
  a.norms = norms;
  a.x_is_bf16 = x_dtype == FA_TQ_BF16;
  const fatq::SignWords sw = make_sign_words(seed, dt, flags & FA_TQ_TWO_SIGNS);
  if (prep) {   // the caller launches (the keys and values of an append together)
    *prep = a;
    *prep_tab = tab;
    *prep_sw = sw;
    return ok();
  }
  return launched(fatq::launch_encode(a, tab, sw, (flags & FA_TQ_NORM_CORRECT) != 0, whole,
                                      static_cast<hipStream_t>(stream)),
                  who);
}

// Split partials of fa_tq_attn_decode_noalloc: one array per GPU the library runs on,
// held until the process ends.  Host code never passes `scratch` itself to a kernel
// (in host code it names a host-side stand-in): it passes the device address that
// hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) uint8_t scratch[FA_TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, resolved once per device.
fa_tq_status scratch_of_current_device(const char* who, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FA_TQ_EHIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_TQ_EUNSUPPORTED, "%s: device index %d >= %d", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FA_TQ_EHIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

// Attention over a dense-rotation cache: on the MFMA kernels the merge writes
// out = R^T o (d elements per head) itself and sets written.
struct DenseOutput {
  const float* rot;
  int32_t dim;
  float* out;
  bool written;
};

fa_tq_status attn_impl(const char* who, const fa_tq_codebook* cb_k,
                       const fa_tq_codebook* cb_v, uint64_t seed, uint32_t flags,
                       int32_t head_dim,
                       const void* q, fa_tq_dtype q_dtype, const uint8_t* k_codes,
                       const uint16_t* k_norms, const uint8_t* v_codes,
                       const uint16_t* v_norms, const int32_t* seq_lens, const int32_t* pos,
                       int32_t n_new, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t t_max, float scale, float* out, void* workspace,
                       size_t workspace_bytes, void* stream, bool check_only = false,
                       int32_t cb_dim = fatq::QK, DenseOutput* dense = nullptr) {
  fatq::KTable tk, tv;
  fa_tq_status st = check_codebook(cb_k, who, false, &tk, cb_dim);
  if (st != FA_TQ_OK) return st;
  if ((st = check_codebook(cb_v, who, false, &tv, cb_dim)) != FA_TQ_OK)
    return st;
  if ((st = check_flags(flags, FA_TQ_TWO_SIGNS | FA_TQ_ATTN_VECTOR_ALU, nullptr, who)) !=
      FA_TQ_OK)
    return st;
  if ((st = check_head_dim(head_dim)) != FA_TQ_OK) return st;
  if (head_dim != fatq::QK)
    return fail(FA_TQ_EUNSUPPORTED, "%s: head_dim %d (the attention kernels take 128)", who,
                head_dim);
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: bad sizes", who);
  if (n_q_heads % n_kv_heads != 0)
    return fail(FA_TQ_EINVAL, "%s: n_q_heads %d not a multiple of n_kv_heads %d", who,
                n_q_heads, n_kv_heads);
  if ((flags & FA_TQ_ATTN_VECTOR_ALU) && n_q_heads / n_kv_heads > 16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: group size %d > 16 on the vector-ALU kernels", who,
                n_q_heads / n_kv_heads);
  if (q_dtype != FA_TQ_F32 && q_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: query dtype %d", who, (int)q_dtype);
  if (!std::isfinite(scale)) return fail(FA_TQ_EINVAL, "%s: scale not finite", who);
  if (batch == 0) return ok();
  if (!q || !k_codes || !k_norms || !v_codes || !v_norms || !(seq_lens || pos) || !out ||
      !workspace)
    return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if (!aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out) || !aligned16(workspace) ||
      !aligned16(q) || (reinterpret_cast<uintptr_t>(k_norms) & 1u) ||
      (reinterpret_cast<uintptr_t>(v_norms) & 1u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(pos) & 3u))
    return fail(FA_TQ_EINVAL, "%s: misaligned pointer", who);
  const size_t need =
      fa_tq_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, head_dim);
  if (workspace_bytes < need)
    return fail(FA_TQ_EINVAL, "%s: workspace %zu bytes < %zu", who, workspace_bytes,
                need);
  if (check_only) return ok();
  fatq::AttnLaunch a;
  a.q = q;
  a.q_is_bf16 = q_dtype == FA_TQ_BF16;
  a.k_codes = k_codes;
  a.k_norms = k_norms;
  a.v_codes = v_codes;
  a.v_norms = v_norms;
  a.seq_lens = seq_lens;
  a.pos = pos;
  a.n_new = n_new;
  a.lens = pos ? pos : seq_lens;
  a.len_add = pos ? n_new : 0;
  a.batch = batch;
  a.hq = n_q_heads;
  a.hkv = n_kv_heads;
  a.t_max = t_max;
  a.scale = scale;
  a.out = out;
  a.workspace = workspace;
  const fatq::SignWords sw = make_sign_words(seed, head_dim, flags & FA_TQ_TWO_SIGNS);
  if (!(flags & FA_TQ_ATTN_VECTOR_ALU)) {
    // the MFMA kernels address one (batch, KV head) row of codes with 32-bit offsets
    if (static_cast<int64_t>(t_max) * 64 >= (int64_t{1} << 31))
      return fail(FA_TQ_EUNSUPPORTED, "%s: t_max %d: a cache row spans 2 GiB or more", who,
                  t_max);
    a.kv_div = fatq::attn_mfma_groups(n_q_heads, n_kv_heads);
    fatq::attn_mfma_partition(batch, n_kv_heads * a.kv_div, t_max, &a.n_split, &a.chunk);
    if (dense) {   // the merge applies R^T and writes the caller's output
      a.dense_rot = dense->rot;
      a.dense_dim = dense->dim;
      a.out = dense->out;
      dense->written = true;
    }
    return launched(fatq::launch_attn_mfma(a, tk, tv, sw, static_cast<hipStream_t>(stream)),
                    who);
  }
  fatq::attn_partition(batch, n_kv_heads, t_max, &a.n_split, &a.chunk);
  return launched(fatq::launch_attn(a, tk, tv, sw, static_cast<hipStream_t>(stream)),
                  who);
}


// Dense random orthogonal rotation ([Spec] "Hadamard Transform Detail": the option for
// head_dims that are not a power of two; "Step 1": a fixed d x d orthogonal R from the
// seed).  The Gaussian matrix G (row-major) takes SplitMix64 draws 2d, 2d + 1, ... of
// the seed's stream (after the two sign vectors' draws) in pairs through the
// Box-Muller transform (Box and Muller, 1958); R is the Q factor of G = Q T by
// Householder reflections in fp64, with the columns' signs chosen so that T has a
// positive diagonal; stored rounded to fp32.
void make_dense_rotation(uint64_t seed, int d, float* out) {
  const size_t n = static_cast<size_t>(d) * d;
  SplitMix64 g{seed};
  for (int i = 0; i < 2 * d; ++i) g.next();
  std::vector<double> a(n + 1);
  const double two_pi = 2.0 * 3.141592653589793;
  for (size_t t = 0; t < n; t += 2) {
    const uint64_t z1 = g.next(), z2 = g.next();
    const double u1 = (static_cast<double>(z1 >> 11) + 0.5) * 0x1p-53;
    const double u2 = static_cast<double>(z2 >> 11) * 0x1p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    a[t] = r * std::cos(two_pi * u2);
    a[t + 1] = r * std::sin(two_pi * u2);   // a has one spare element for odd n
  }
  auto A = [&](int i, int j) -> double& { return a[static_cast<size_t>(i) * d + j]; };
  std::vector<double> v(n, 0.0), diag(d);
  for (int k = 0; k < d; ++k) {
    double* vk = &v[static_cast<size_t>(k) * d];
    double norm = 0.0;
    for (int i = k; i < d; ++i) norm += A(i, k) * A(i, k);
    norm = std::sqrt(norm);
    const double alpha = A(k, k) > 0.0 ? -norm : norm;
    for (int i = k; i < d; ++i) vk[i] = A(i, k);
    vk[k] -= alpha;
    double vn = 0.0;
    for (int i = k; i < d; ++i) vn += vk[i] * vk[i];
    vn = std::sqrt(vn);
    if (vn > 0.0)
      for (int i = k; i < d; ++i) vk[i] /= vn;
    for (int j = k; j < d; ++j) {
      double sdot = 0.0;
      for (int i = k; i < d; ++i) sdot += vk[i] * A(i, j);
      for (int i = k; i < d; ++i) A(i, j) -= 2.0 * sdot * vk[i];
    }
    diag[k] = A(k, k);
  }
  // Q = H_0 H_1 ... H_{d-1}, applied to the identity from the last reflection back
  std::vector<double> q(n, 0.0);
  for (int i = 0; i < d; ++i) q[static_cast<size_t>(i) * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    const double* vk = &v[static_cast<size_t>(k) * d];
    for (int j = 0; j < d; ++j) {
      double sdot = 0.0;
      for (int i = k; i < d; ++i) sdot += vk[i] * q[static_cast<size_t>(i) * d + j];
      for (int i = k; i < d; ++i) q[static_cast<size_t>(i) * d + j] -= 2.0 * sdot * vk[i];
    }
  }
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < d; ++k) {
      const double x = q[static_cast<size_t>(i) * d + k];
      out[static_cast<size_t>(i) * d + k] = static_cast<float>(diag[k] < 0.0 ? -x : x);
    }
}

// Cell of u in the dense encoder's bucketize grid: clamp(floor(fma(u, G/2, G/2)), 0,
// G - 1) in fp32, the same operations as the kernel's, so a boundary's cell here is
// its cell there.
int dense_grid_cell(float u) {
  const float h = 0.5f * fatq::kDenseGrid;
  const float f = std::fmin(std::fmax(std::fmaf(u, h, h), 0.0f),
                            static_cast<float>(fatq::kDenseGrid - 1));
  return static_cast<int>(std::floor(f));
}

// The dense-rotation calls: head_dim in [4, kDenseMax], a 2-4 bit codebook of dim
// head_dim whose boundaries lie in distinct cells of the encoder's grid.
fa_tq_status check_dense(const fa_tq_codebook* cb, const float* rotation, int32_t head_dim,
                         const char* who, fatq::KTable* tab) {
  if (head_dim < 4 || head_dim > fatq::kDenseMax)
    return fail(FA_TQ_EUNSUPPORTED, "%s: head_dim %d not in [4, %d]", who, head_dim,
                fatq::kDenseMax);
  fa_tq_status st = check_codebook(cb, who, false, tab, head_dim);
  if (st != FA_TQ_OK) return st;
  for (int j = 1; j < tab->nb; ++j)
    if (dense_grid_cell(tab->b[j]) == dense_grid_cell(tab->b[j - 1]))
      return fail(FA_TQ_EUNSUPPORTED,
                  "%s: boundaries %d and %d share a cell of the encoder's grid (width 2/%d)",
                  who, j - 1, j, fatq::kDenseGrid);
  if (!rotation) return fail(FA_TQ_EINVAL, "%s: rotation is NULL", who);
  if (!aligned16(rotation)) return fail(FA_TQ_EINVAL, "%s: rotation must be 16-byte aligned", who);
  return ok();
}
}  // namespace

extern "C" {

const char* fa_tq_last_error(void) { return g_last_error.c_str(); }

fa_tq_status fa_tq_rotation_dense(uint64_t seed, int32_t dim, float* out) {
  if (!out) return fail(FA_TQ_EINVAL, "fa_tq_rotation_dense: out is NULL");
  if (dim < 2 || dim > 512)
    return fail(FA_TQ_EINVAL, "fa_tq_rotation_dense: dim %d not in [2, 512]", dim);
  make_dense_rotation(seed, dim, out);
  return ok();
}

fa_tq_status fa_tq_encode_dense(const fa_tq_codebook* cb, const float* rotation,
                                int32_t head_dim, const void* x, fa_tq_dtype x_dtype,
                                fa_tq_layout x_layout, int32_t batch, int32_t n_kv_heads,
                                int32_t n_tokens, const int32_t* t0, int32_t t_max,
                                uint8_t* codes, uint16_t* norms, void* stream) {
  static const char* who = "fa_tq_encode_dense";
  fatq::KTable tab;
  fa_tq_status st = check_dense(cb, rotation, head_dim, who, &tab);
  if (st != FA_TQ_OK) return st;
  if (batch < 0 || n_kv_heads < 0 || n_tokens < 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: negative size", who);
  if (x_dtype != FA_TQ_F32 && x_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: input dtype %d", who, (int)x_dtype);
  if (x_layout.stride_b < 0 || x_layout.stride_h < 0 || x_layout.stride_t < 0)
    return fail(FA_TQ_EINVAL, "%s: negative stride", who);
  if (n_tokens > t_max && !t0)
    return fail(FA_TQ_EINVAL, "%s: n_tokens %d > t_max %d", who, n_tokens, t_max);
  if (static_cast<int64_t>(batch) * n_kv_heads * n_tokens >= (int64_t{1} << 31))
    return fail(FA_TQ_EUNSUPPORTED, "%s: %lld vectors in one call (at most 2^31 - 1)", who,
                static_cast<long long>(static_cast<int64_t>(batch) * n_kv_heads * n_tokens));
  if (batch == 0 || n_kv_heads == 0 || n_tokens == 0) return ok();
  if (!x || !codes || !norms) return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if ((reinterpret_cast<uintptr_t>(x) & (x_dtype == FA_TQ_BF16 ? 1u : 3u)) || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(norms) & 1u))
    return fail(FA_TQ_EINVAL, "%s: misaligned pointer", who);
  fatq::DenseLaunch a;
  a.x = x;
  a.sb = x_layout.stride_b;
  a.sh = x_layout.stride_h;
  a.st = x_layout.stride_t;
  a.batch = batch;
  a.heads = n_kv_heads;
  a.tokens = n_tokens;
  a.t_max = t_max;
  a.dim = head_dim;
  a.nblk = (head_dim + fatq::QK - 1) / fatq::QK;
  a.t0 = t0;
  a.rot = rotation;
  a.codes = codes;
  a.norms = norms;
  a.x_is_bf16 = x_dtype == FA_TQ_BF16;
  {
    const int64_t q = x_dtype == FA_TQ_BF16 ? 8 : 4;   // elements per 16 bytes
    // 16-byte loads of whole 8-element chunks (a lane without a vector reads the
    // first chunk of the input instead)
    a.vec = head_dim % 8 == 0 && aligned16(x) && a.sb % q == 0 && a.sh % q == 0 &&
            a.st % q == 0;
  }
  return launched(fatq::launch_dense_encode(a, tab, static_cast<hipStream_t>(stream)), who);
}

fa_tq_status fa_tq_decode_dense(const fa_tq_codebook* cb, const float* rotation,
                                int32_t head_dim, const uint8_t* codes, const uint16_t* norms,
                                int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                                int32_t t_max, void* out, fa_tq_dtype out_dtype,
                                fa_tq_layout out_layout, void* stream) {
  static const char* who = "fa_tq_decode_dense";
  fatq::KTable tab;
  fa_tq_status st = check_dense(cb, rotation, head_dim, who, &tab);
  if (st != FA_TQ_OK) return st;
  if (batch < 0 || n_kv_heads < 0 || n_tokens < 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: negative size", who);
  if (n_tokens > t_max)
    return fail(FA_TQ_EINVAL, "%s: n_tokens %d > t_max %d", who, n_tokens, t_max);
  if (static_cast<int64_t>(batch) * n_kv_heads * n_tokens >= (int64_t{1} << 31))
    return fail(FA_TQ_EUNSUPPORTED, "%s: %lld vectors in one call (at most 2^31 - 1)", who,
                static_cast<long long>(static_cast<int64_t>(batch) * n_kv_heads * n_tokens));
  if (out_dtype != FA_TQ_F32 && out_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: output dtype %d", who, (int)out_dtype);
  if (out_layout.stride_b < 0 || out_layout.stride_h < 0 || out_layout.stride_t < 0)
    return fail(FA_TQ_EINVAL, "%s: negative stride", who);
  if (batch == 0 || n_kv_heads == 0 || n_tokens == 0) return ok();
  if (!codes || !norms || !out) return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if (!aligned16(codes) || (reinterpret_cast<uintptr_t>(norms) & 1u) ||
      (reinterpret_cast<uintptr_t>(out) & (out_dtype == FA_TQ_BF16 ? 1u : 3u)))
    return fail(FA_TQ_EINVAL, "%s: misaligned pointer", who);
  fatq::DenseDecodeLaunch d;
  d.codes = codes;
  d.norms = norms;
  d.rot = rotation;
  d.rows = static_cast<int64_t>(batch) * n_kv_heads;
  d.tokens = n_tokens;
  d.t_max = t_max;
  d.heads = n_kv_heads;
  d.dim = head_dim;
  d.nblk = (head_dim + fatq::QK - 1) / fatq::QK;
  d.out = out;
  d.sb = out_layout.stride_b;
  d.sh = out_layout.stride_h;
  d.st = out_layout.stride_t;
  d.out_bf16 = out_dtype == FA_TQ_BF16;
  d.vec = aligned16(out) && d.sb % 4 == 0 && d.sh % 4 == 0 && d.st % 4 == 0;
  return launched(fatq::launch_dense_decode(d, tab, static_cast<hipStream_t>(stream)), who);
}

// The attention kernels' own frame for attention over a dense-rotation cache: the
// Walsh-Hadamard rotation of this seed (any seed would do: the frame cancels).
constexpr uint64_t kDenseFrameSeed = 0;

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t fa_tq_attn_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t t_max) {
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || t_max < 0 ||
      n_q_heads % n_kv_heads != 0)
    return 0;
  const size_t attn = fa_tq_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, fatq::QK);
  const size_t frame = align256(static_cast<size_t>(batch) * n_q_heads * fatq::QK * sizeof(float));
  return 2 * frame + attn;
}

fa_tq_status fa_tq_attn_decode_dense(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                                     const float* rotation, int32_t head_dim, uint32_t flags,
                                     const void* q, fa_tq_dtype q_dtype,
                                     const uint8_t* k_codes, const uint16_t* k_norms,
                                     const uint8_t* v_codes, const uint16_t* v_norms,
                                     const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                     int32_t n_kv_heads, int32_t t_max, float scale, float* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  static const char* who = "fa_tq_attn_decode_dense";
  fatq::KTable tk, tv;
  fa_tq_status st = check_dense(cb_k, rotation, head_dim, who, &tk);
  if (st != FA_TQ_OK) return st;
  if ((st = check_dense(cb_v, rotation, head_dim, who, &tv)) != FA_TQ_OK) return st;
  if (head_dim > fatq::kDenseAttnMax)
    return fail(FA_TQ_EUNSUPPORTED, "%s: head_dim %d (attention over a dense cache takes <= %d)",
                who, head_dim, fatq::kDenseAttnMax);
  if ((st = check_flags(flags, FA_TQ_ATTN_VECTOR_ALU, nullptr, who)) != FA_TQ_OK) return st;
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: bad sizes", who);
  if (q_dtype != FA_TQ_F32 && q_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: query dtype %d", who, (int)q_dtype);
  if (batch == 0) return ok();
  if (!q || !out || !workspace) return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if ((reinterpret_cast<uintptr_t>(q) & (q_dtype == FA_TQ_BF16 ? 1u : 3u)) ||
      (reinterpret_cast<uintptr_t>(out) & 3u) || !aligned16(workspace))
    return fail(FA_TQ_EINVAL, "%s: misaligned pointer", who);
  // the frame's query and result first, then the attention call's own workspace (whose
  // size, with every other argument, attn_impl checks)
  const size_t frame = align256(static_cast<size_t>(batch) * n_q_heads * fatq::QK * sizeof(float));
  if (workspace_bytes < 2 * frame)
    return fail(FA_TQ_EINVAL, "%s: workspace %zu bytes < %zu", who, workspace_bytes,
                fa_tq_attn_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max));
  float* qt = static_cast<float*>(workspace);
  float* y = reinterpret_cast<float*>(static_cast<char*>(workspace) + frame);
  void* ws = static_cast<char*>(workspace) + 2 * frame;
  // every check of the attention call itself before anything is launched
  if ((st = attn_impl(who, cb_k, cb_v, kDenseFrameSeed, flags, fatq::QK, qt, FA_TQ_F32, k_codes,
                      k_norms, v_codes, v_norms, seq_lens, nullptr, 0, batch, n_q_heads,
                      n_kv_heads, t_max, scale, y, ws, workspace_bytes - 2 * frame, stream,
                      true, head_dim)) != FA_TQ_OK)
    return st;
  fatq::DenseAttnLaunch a;
  a.q = q;
  a.q_is_bf16 = q_dtype == FA_TQ_BF16;
  a.rot = rotation;
  a.batch = batch;
  a.hq = n_q_heads;
  a.dim = head_dim;
  a.qt = qt;
  a.y = y;
  a.out = out;
  {
    int8_t sg[fatq::QK];
    make_signs(kDenseFrameSeed, fatq::QK, sg);
    for (int w = 0; w < 4; ++w) a.signs[w] = 0;
    for (int i = 0; i < fatq::QK; ++i)
      if (sg[i] < 0) a.signs[i >> 5] |= 1u << (i & 31);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = launched(fatq::launch_dense_attn_query(a, s), who)) != FA_TQ_OK) return st;
  DenseOutput dense{rotation, head_dim, out, false};
  if ((st = attn_impl(who, cb_k, cb_v, kDenseFrameSeed, flags, fatq::QK, qt, FA_TQ_F32, k_codes,
                      k_norms, v_codes, v_norms, seq_lens, nullptr, 0, batch, n_q_heads,
                      n_kv_heads, t_max, scale, y, ws, workspace_bytes - 2 * frame, stream,
                      false, head_dim, &dense)) != FA_TQ_OK)
    return st;
  // the vector-ALU kernels leave the result in the frame: the output kernel maps it back
  return dense.written ? ok() : launched(fatq::launch_dense_attn_out(a, s), who);
}

int32_t fa_tq_code_bytes(int32_t bits) {
  switch (bits) {
    case 2: return 32;
    case 3: return 48;
    case 4: return 64;
    case 8: return 128;
    default: return -1;
  }
}

fa_tq_status fa_tq_signs(uint64_t seed, int32_t head_dim, int8_t* out) {
  if (!out) return fail(FA_TQ_EINVAL, "fa_tq_signs: out is NULL");
  if (head_dim <= 0 || head_dim > (1 << 20))
    return fail(FA_TQ_EINVAL, "fa_tq_signs: head_dim %d out of range", head_dim);
  make_signs(seed, head_dim, out);
  return ok();
}

fa_tq_status fa_tq_codebook_init(int32_t dim, int32_t bits, fa_tq_codebook* out) {
  if (!out) return fail(FA_TQ_EINVAL, "fa_tq_codebook_init: out is NULL");
  if (dim < 4 || dim > 512)
    return fail(FA_TQ_EINVAL, "fa_tq_codebook_init: dim %d not in [4, 512]", dim);
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8))
    return fail(FA_TQ_EINVAL, "fa_tq_codebook_init: bits %d not in {2, 3, 4, 8}", bits);
  std::memset(out, 0, sizeof(*out));
  out->dim = dim;
  out->bits = bits;
  out->levels = 1 << bits;
  if (bits == 8) return ok();
  if (!lloyd_max(dim, bits, out->boundaries, out->centroids))
    return fail(FA_TQ_EINVAL, "fa_tq_codebook_init: iteration did not stay finite");
  return ok();
}

size_t fa_tq_attn_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t t_max, int32_t head_dim) {
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || t_max < 0 || head_dim != fatq::QK ||
      n_q_heads % n_kv_heads != 0)
    return 0;
  // enough for either kernel family (FA_TQ_ATTN_VECTOR_ALU selects the vector-ALU one)
  int32_t n_split = 1, chunk = 0;
  fatq::attn_partition(batch, n_kv_heads, t_max, &n_split, &chunk);
  size_t need = fatq::attn_workspace_bytes(batch, n_q_heads, n_split);
  const int32_t r = fatq::attn_mfma_groups(n_q_heads, n_kv_heads);
  fatq::attn_mfma_partition(batch, n_kv_heads * r, t_max, &n_split, &chunk);
  need = std::max(need, fatq::attn_mfma_workspace_bytes(batch, n_q_heads, n_kv_heads, n_split));
  return need;
}

fa_tq_status fa_tq_encode(const fa_tq_codebook* cb, uint64_t seed, int32_t head_dim,
                          const void* x, fa_tq_dtype x_dtype, fa_tq_layout x_layout,
                          int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                          const int32_t* t0, int32_t t_max, uint8_t* codes, uint16_t* norms,
                          void* stream) {
  return encode_impl("fa_tq_encode", cb, seed, 0, head_dim, x, x_dtype, x_layout, batch,
                     n_kv_heads, n_tokens, t0, t_max, codes, norms, stream, false);
}

fa_tq_status fa_tq_encode_ex(const fa_tq_codebook* cb, uint64_t seed, uint32_t flags,
                             int32_t head_dim, const void* x, fa_tq_dtype x_dtype,
                             fa_tq_layout x_layout, int32_t batch, int32_t n_kv_heads,
                             int32_t n_tokens, const int32_t* t0, int32_t t_max,
                             uint8_t* codes, uint16_t* norms, void* stream) {
  return encode_impl("fa_tq_encode_ex", cb, seed, flags, head_dim, x, x_dtype, x_layout,
                     batch, n_kv_heads, n_tokens, t0, t_max, codes, norms, stream, false);
}

fa_tq_status fa_tq_encode_kv(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                             uint64_t seed, uint32_t flags, int32_t head_dim, const void* k,
                             const void* v, fa_tq_dtype x_dtype, fa_tq_layout k_layout,
                             fa_tq_layout v_layout, int32_t batch, int32_t n_kv_heads,
                             int32_t n_tokens, const int32_t* t0, int32_t t_max,
                             uint8_t* k_codes, uint16_t* k_norms, uint8_t* v_codes,
                             uint16_t* v_norms, void* stream) {
  static const char* who = "fa_tq_encode_kv";
  // both halves are checked before anything is launched
  fa_tq_status st;
  for (int half = 0; half < 2; ++half) {
    if ((st = encode_impl(who, half ? cb_v : cb_k, seed, flags, head_dim, half ? v : k, x_dtype,
                          half ? v_layout : k_layout, batch, n_kv_heads, n_tokens, t0, t_max,
                          half ? v_codes : k_codes, half ? v_norms : k_norms, stream, false,
                          true)) != FA_TQ_OK)
      return st;
  }
  if (batch == 0 || n_kv_heads == 0 || n_tokens == 0) return ok();
  if ((flags & FA_TQ_WHOLE_VECTOR) || cb_k->bits == 8 || cb_v->bits == 8) {
    // the pair kernel takes the blocked 2-4 bit encodes: two launches otherwise
    for (int half = 0; half < 2; ++half) {
      if ((st = encode_impl(who, half ? cb_v : cb_k, seed, flags, head_dim, half ? v : k,
                            x_dtype, half ? v_layout : k_layout, batch, n_kv_heads, n_tokens,
                            t0, t_max, half ? v_codes : k_codes, half ? v_norms : k_norms,
                            stream, false)) != FA_TQ_OK)
        return st;
    }
    return ok();
  }
  fatq::EncodeLaunch ak, av;
  fatq::KTable tk, tv;
  fatq::SignWords sw;
  if ((st = encode_impl(who, cb_k, seed, flags, head_dim, k, x_dtype, k_layout, batch, n_kv_heads,
                        n_tokens, t0, t_max, k_codes, k_norms, stream, false, false, &ak, &tk,
                        &sw)) != FA_TQ_OK ||
      (st = encode_impl(who, cb_v, seed, flags, head_dim, v, x_dtype, v_layout, batch, n_kv_heads,
                        n_tokens, t0, t_max, v_codes, v_norms, stream, false, false, &av, &tv,
                        &sw)) != FA_TQ_OK)
    return st;
  return launched(fatq::launch_encode_pair(ak, tk, av, tv, sw, (flags & FA_TQ_NORM_CORRECT) != 0,
                                           false, static_cast<hipStream_t>(stream)),
                  who);
}

fa_tq_status fa_tq_decode(const fa_tq_codebook* cb, uint64_t seed, int32_t head_dim,
                          const uint8_t* codes, const uint16_t* norms, int64_t n_vec,
                          float* out, void* stream) {
  fatq::KTable tab;
  fa_tq_status st = check_codebook(cb, "fa_tq_decode", true, &tab);
  if (st != FA_TQ_OK) return st;
  if ((st = check_head_dim(head_dim)) != FA_TQ_OK) return st;
  if (n_vec < 0) return fail(FA_TQ_EINVAL, "fa_tq_decode: negative n_vec");
  if (n_vec == 0) return ok();
  if (!codes || !norms || !out) return fail(FA_TQ_EINVAL, "fa_tq_decode: NULL device pointer");
  if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(norms) & 1u))
    return fail(FA_TQ_EINVAL, "fa_tq_decode: codes and out must be 16-byte aligned");
  // The kernel addresses one row of codes and of output with 32-bit byte offsets
  // below 2^31: the vectors go as rows of R vectors each, then one row of the rest.
  const int32_t nblk = head_dim / fatq::QK;
  const int64_t vec_bytes = static_cast<int64_t>(nblk) * fa_tq_code_bytes(cb->bits);
  const int64_t out_bytes = static_cast<int64_t>(head_dim) * sizeof(float);
  const int64_t R = ((int64_t{1} << 31) - 1) / std::max(vec_bytes, out_bytes);
  const fatq::SignWords sw = make_sign_words(seed, head_dim);
  auto launch_rows = [&](int64_t first, int64_t rows, int64_t per) {
    fatq::DecodeLaunch d;
    d.codes = codes + first * vec_bytes;
    d.norms = norms + first * nblk;
    d.rows = rows;
    d.tokens = per;
    d.t_max = per;
    d.heads = 1;
    d.nblk = nblk;
    d.out = out + first * head_dim;
    d.sb = per * head_dim;   // row b starts at vector first + b * per
    d.sh = 0;
    d.st = head_dim;
    d.out_bf16 = 0;
    d.dim = head_dim;
    return launched(fatq::launch_decode(d, tab, sw, false, static_cast<hipStream_t>(stream)),
                    "fa_tq_decode");
  };
  if (n_vec <= R) return launch_rows(0, 1, n_vec);
  const int64_t full = n_vec / R, rem = n_vec - full * R;
  if ((st = launch_rows(0, full, R)) != FA_TQ_OK) return st;
  return rem ? launch_rows(full * R, 1, rem) : ok();
}

fa_tq_status fa_tq_decode_kv(const fa_tq_codebook* cb, uint64_t seed, uint32_t flags,
                             int32_t head_dim, const uint8_t* codes, const uint16_t* norms,
                             int32_t batch, int32_t n_kv_heads, int32_t n_tokens,
                             int32_t t_max, void* out, fa_tq_dtype out_dtype,
                             fa_tq_layout out_layout, void* stream) {
  static const char* who = "fa_tq_decode_kv";
  fatq::KTable tab;
  const bool whole = (flags & FA_TQ_WHOLE_VECTOR) != 0;
  fa_tq_status st = check_flags(flags, FA_TQ_TWO_SIGNS | FA_TQ_WHOLE_VECTOR, nullptr, who);
  if (st != FA_TQ_OK) return st;
  if (whole && (st = check_whole(cb, head_dim, who)) != FA_TQ_OK) return st;
  const int32_t dt = whole ? whole_length(head_dim) : head_dim;   // transform length
  if ((st = check_codebook(cb, who, true, &tab, whole ? dt : fatq::QK)) != FA_TQ_OK)
    return st;
  if (!whole && (st = check_head_dim(head_dim)) != FA_TQ_OK) return st;
  if (batch < 0 || n_kv_heads < 0 || n_tokens < 0 || t_max < 0)
    return fail(FA_TQ_EINVAL, "%s: negative size", who);
  if (n_tokens > t_max)
    return fail(FA_TQ_EINVAL, "%s: n_tokens %d > t_max %d", who, n_tokens, t_max);
  if (static_cast<int64_t>(batch) * n_kv_heads * n_tokens >= (int64_t{1} << 31))
    return fail(FA_TQ_EUNSUPPORTED, "%s: %lld vectors in one call (at most 2^31 - 1)", who,
                static_cast<long long>(static_cast<int64_t>(batch) * n_kv_heads * n_tokens));
  if (out_dtype != FA_TQ_F32 && out_dtype != FA_TQ_BF16)
    return fail(FA_TQ_EUNSUPPORTED, "%s: output dtype %d", who, (int)out_dtype);
  if (out_layout.stride_b % 8 || out_layout.stride_h % 8 || out_layout.stride_t % 8 ||
      out_layout.stride_b < 0 || out_layout.stride_h < 0 || out_layout.stride_t < 0)
    return fail(FA_TQ_EINVAL, "%s: strides must be non-negative multiples of 8", who);
  if (batch == 0 || n_kv_heads == 0 || n_tokens == 0) return ok();
  if (!codes || !norms || !out) return fail(FA_TQ_EINVAL, "%s: NULL device pointer", who);
  if (!aligned16(codes) || !aligned16(out) || (reinterpret_cast<uintptr_t>(norms) & 1u))
    return fail(FA_TQ_EINVAL, "%s: codes and out must be 16-byte aligned, norms 2-byte", who);
  // The kernel addresses the decoded codes and the output of one (batch, head) row
  // with 32-bit byte offsets below 2^31.
  const int64_t oes = out_dtype == FA_TQ_BF16 ? 2 : 4;
  if (static_cast<int64_t>(n_tokens) * (dt / fatq::QK) * fa_tq_code_bytes(cb->bits) >=
          (int64_t{1} << 31) ||
      ((n_tokens - 1) * out_layout.stride_t + head_dim) * oes >= (int64_t{1} << 31))
    return fail(FA_TQ_EUNSUPPORTED,
                "%s: one (batch, head) row of codes or of output spans 2 GiB or more", who);
  fatq::DecodeLaunch d;
  d.codes = codes;
  d.norms = norms;
  d.rows = static_cast<int64_t>(batch) * n_kv_heads;
  d.tokens = n_tokens;
  d.t_max = t_max;
  d.heads = n_kv_heads;
  d.nblk = dt / fatq::QK;
  d.out = out;
  d.sb = out_layout.stride_b;
  d.sh = out_layout.stride_h;
  d.st = out_layout.stride_t;
  d.out_bf16 = out_dtype == FA_TQ_BF16;
  d.dim = head_dim;
  const fatq::SignWords sw = make_sign_words(seed, dt, flags & FA_TQ_TWO_SIGNS);
  return launched(fatq::launch_decode(d, tab, sw, whole, static_cast<hipStream_t>(stream)),
                  who);
}

fa_tq_status fa_tq_attn_decode(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                               uint64_t seed, int32_t head_dim, const void* q,
                               fa_tq_dtype q_dtype, const uint8_t* k_codes,
                               const uint16_t* k_norms, const uint8_t* v_codes,
                               const uint16_t* v_norms, const int32_t* seq_lens,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t t_max, float scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return fa_tq_attn_decode_ex(cb_k, cb_v, seed, 0, head_dim, q, q_dtype, k_codes, k_norms,
                              v_codes, v_norms, seq_lens, batch, n_q_heads, n_kv_heads, t_max,
                              scale, out, workspace, workspace_bytes, stream);
}

fa_tq_status fa_tq_attn_decode_ex(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                                  uint64_t seed, uint32_t flags, int32_t head_dim,
                                  const void* q, fa_tq_dtype q_dtype, const uint8_t* k_codes,
                                  const uint16_t* k_norms, const uint8_t* v_codes,
                                  const uint16_t* v_norms, const int32_t* seq_lens,
                                  int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t t_max, float scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (batch > 0 && !seq_lens) return fail(FA_TQ_EINVAL, "fa_tq_attn_decode: seq_lens is NULL");
  return attn_impl("fa_tq_attn_decode", cb_k, cb_v, seed, flags, head_dim, q, q_dtype,
                   k_codes, k_norms, v_codes, v_norms, seq_lens, nullptr, 0, batch, n_q_heads,
                   n_kv_heads, t_max, scale, out, workspace, workspace_bytes, stream);
}

fa_tq_status fa_tq_attn_decode_noalloc(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                                       uint64_t seed, uint32_t flags, int32_t head_dim,
                                       const void* q, fa_tq_dtype q_dtype,
                                       const uint8_t* k_codes, const uint16_t* k_norms,
                                       const uint8_t* v_codes, const uint16_t* v_norms,
                                       const int32_t* seq_lens, int32_t batch,
                                       int32_t n_q_heads, int32_t n_kv_heads, int32_t t_max,
                                       float scale, float* out, void* stream) {
  static const char* who = "fa_tq_attn_decode_noalloc";
  if (batch > 0 && !seq_lens) return fail(FA_TQ_EINVAL, "%s: seq_lens is NULL", who);
  // every argument checked (with a stand-in workspace address) before the scratch
  // array is looked up or anything is launched
  void* const probe = reinterpret_cast<void*>(uintptr_t{256});
  fa_tq_status st = attn_impl(who, cb_k, cb_v, seed, flags, head_dim, q, q_dtype, k_codes,
                              k_norms, v_codes, v_norms, seq_lens, nullptr, 0, batch, n_q_heads,
                              n_kv_heads, t_max, scale, out, probe,
                              FA_TQ_NOALLOC_SCRATCH_BYTES, stream, true);
  if (st != FA_TQ_OK) {
    const size_t need = fa_tq_attn_workspace_bytes(batch, n_q_heads, n_kv_heads, t_max, head_dim);
    if (need > FA_TQ_NOALLOC_SCRATCH_BYTES)
      return fail(FA_TQ_EUNSUPPORTED,
                  "%s: these sizes need %zu bytes of split partials, more than the %u-byte "
                  "scratch array; use fa_tq_attn_decode with a workspace", who, need,
                  static_cast<unsigned>(FA_TQ_NOALLOC_SCRATCH_BYTES));
    return st;
  }
  if (batch == 0) return ok();
  void* ws = nullptr;
  if ((st = scratch_of_current_device(who, &ws)) != FA_TQ_OK) return st;
  return attn_impl(who, cb_k, cb_v, seed, flags, head_dim, q, q_dtype, k_codes, k_norms,
                   v_codes, v_norms, seq_lens, nullptr, 0, batch, n_q_heads, n_kv_heads, t_max,
                   scale, out, ws, FA_TQ_NOALLOC_SCRATCH_BYTES, stream);
}

fa_tq_status fa_tq_attn_append(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                               uint64_t seed, int32_t head_dim, const void* q,
                               fa_tq_dtype q_dtype, const void* k_new, const void* v_new,
                               fa_tq_dtype kv_dtype, fa_tq_layout k_layout,
                               fa_tq_layout v_layout, int32_t n_new, const int32_t* pos,
                               uint8_t* k_codes, uint16_t* k_norms, uint8_t* v_codes,
                               uint16_t* v_norms, int32_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t t_max, float scale, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return fa_tq_attn_append_ex(cb_k, cb_v, seed, 0, head_dim, q, q_dtype, k_new, v_new,
                              kv_dtype, k_layout, v_layout, n_new, pos, k_codes, k_norms,
                              v_codes, v_norms, batch, n_q_heads, n_kv_heads, t_max, scale, out,
                              workspace, workspace_bytes, stream);
}

fa_tq_status fa_tq_attn_append_ex(const fa_tq_codebook* cb_k, const fa_tq_codebook* cb_v,
                                  uint64_t seed, uint32_t flags, int32_t head_dim,
                                  const void* q, fa_tq_dtype q_dtype, const void* k_new,
                                  const void* v_new, fa_tq_dtype kv_dtype,
                                  fa_tq_layout k_layout, fa_tq_layout v_layout, int32_t n_new,
                                  const int32_t* pos, uint8_t* k_codes, uint16_t* k_norms,
                                  uint8_t* v_codes, uint16_t* v_norms, int32_t batch,
                                  int32_t n_q_heads, int32_t n_kv_heads, int32_t t_max,
                                  float scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  static const char* who = "fa_tq_attn_append";
  if (batch < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || t_max <= 0)
    return fail(FA_TQ_EINVAL, "%s: bad sizes", who);
  if (n_new < 1 || n_new > t_max)
    return fail(FA_TQ_EINVAL, "%s: n_new %d not in [1, t_max %d]", who, n_new, t_max);
  if (batch == 0) return ok();
  if (!pos) return fail(FA_TQ_EINVAL, "%s: pos is NULL", who);
  // Every argument of the three steps is checked before the first launch, so a
  // rejected call leaves the cache untouched.
  // The keys and values of the new tokens are encoded by one launch (blockIdx.z
  // selects K or V), then the attention kernels run.
  fa_tq_status st;
  fatq::EncodeLaunch ak, av;
  fatq::KTable tk, tv;
  fatq::SignWords sw;
  for (bool check_only : {true, false}) {
    if ((st = encode_impl(who, cb_k, seed, flags, head_dim, k_new, kv_dtype, k_layout, batch,
                          n_kv_heads, n_new, pos, t_max, k_codes, k_norms, stream, true,
                          check_only, &ak, &tk, &sw)) != FA_TQ_OK)
      return st;
    if ((st = encode_impl(who, cb_v, seed, flags, head_dim, v_new, kv_dtype, v_layout, batch,
                          n_kv_heads, n_new, pos, t_max, v_codes, v_norms, stream, true,
                          check_only, &av, &tv, &sw)) != FA_TQ_OK)
      return st;
    if (!check_only &&
        (st = launched(fatq::launch_encode_pair(ak, tk, av, tv, sw,
                                                (flags & FA_TQ_NORM_CORRECT) != 0, true,
                                                static_cast<hipStream_t>(stream)),
                       who)) != FA_TQ_OK)
      return st;
    if ((st = attn_impl(who, cb_k, cb_v, seed, flags & FA_TQ_TWO_SIGNS, head_dim, q, q_dtype,
                        k_codes, k_norms, v_codes, v_norms, nullptr, pos, n_new, batch,
                        n_q_heads, n_kv_heads, t_max, scale, out, workspace, workspace_bytes,
                        stream, check_only)) != FA_TQ_OK)
      return st;
  }
  return ok();
}

}  // extern "C"

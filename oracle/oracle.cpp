// Plain fp64 CPU oracle for paged grouped-query attention with head_dim 256.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// CPU-baseline leg of the benchmark may load this library.  It shares no code,
// header or table with the HIP library: it has its own decoders, its own
// argument struct and its own page addressing.
//
// What it computes is the plain definition of attention over a paged KV cache,
// written out once, in fp64, with no tiling, no segments and no online
// rescaling:
//
//   for sequence b, query token t (0 <= t < Lq_b) and query head h:
//     g      = h / (Hq / Hkv)                    (contiguous query-head groups)
//     V_set  = { j : 0 <= j <= Lk_b - Lq_b + t }  (bottom-right causal), or the
//              row's own index list (sparse)
//     K_j, V_j read at page block_table[b][j / P], slot j % P, kv head g
//     s_j    = softmax_scale * q_ds * k_ds * sum_d q[t,h,d] * K_j[d]
//     m      = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j
//     out    = v_ds * sum_j p_j V_j / l,   lse = m + ln l
//
// Sources: the causal rule with cached keys longer than the new queries is the
// one ROCm/ATOM PR #2534 ("asm FP8 FMHA for prefix-hit prefill ...", its FMHA
// commit message and Summary) states for prefix-hit prefill; speculative verify
// (SGLang PR #36330, "... MTP unified attention on gfx950", Motivation) is the
// same rule with 2..4 query tokens; the per-tensor descales are the scalar
// descales of that PR's kernel notes; the selected-token variant is vLLM PR
// #62590 ("Tune sparse GQA prefill profile on gfx942 and gfx950", Overview and
// Earlier results), where each query row attends only to its own selected
// tokens.  Page addressing through a block table with a runtime row stride is
// from ROCm/ATOM PR #2830 (summary paragraph).
//
// Readings where the pages are silent (each also listed in the design notes):
//   * Lk_b counts the query tokens themselves, so the last query token of a
//     sequence sees all Lk_b keys.
//   * FP8 is OCP E4M3FN; real value = code * descale.
//   * Sparse entries outside [0, Lk_b) are padding and are skipped; every other
//     entry is attended as listed (a duplicate counts twice).
//   * No visible key: out = 0 and lse = -inf.
//   * One index list per query row, shared by all heads of that row.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include <omp.h>

namespace {

constexpr int kHeadDim = 256;
constexpr int kBF16 = 1;
constexpr int kFP8 = 2;

// bf16 is the upper half of an IEEE binary32; the widening is exact.
double decode_bf16(uint16_t bits) {
  uint32_t w = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return static_cast<double>(f);
}

// OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
// infinities, S.1111.111 is NaN, largest finite magnitude 448.
double decode_e4m3fn(uint8_t code) {
  const int sign = code >> 7;
  const int e = (code >> 3) & 0xF;
  const int m = code & 0x7;
  if (e == 0xF && m == 0x7) return std::numeric_limits<double>::quiet_NaN();
  double mag = (e == 0) ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

struct E4M3Table {
  double v[256];
  E4M3Table() {
    for (int c = 0; c < 256; ++c) v[c] = decode_e4m3fn(static_cast<uint8_t>(c));
  }
};
const E4M3Table& e4m3_table() {
  static const E4M3Table t;
  return t;
}

// Decode `n` consecutive codes of the given encoding starting at element `off`.
void decode_row(const void* base, int dtype, int64_t off, int n, double* dst) {
  if (dtype == kBF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    for (int i = 0; i < n; ++i) dst[i] = decode_bf16(p[i]);
  } else {
    const uint8_t* p = static_cast<const uint8_t*>(base) + off;
    const E4M3Table& t = e4m3_table();
    for (int i = 0; i < n; ++i) dst[i] = t.v[p[i]];
  }
}

}  // namespace

extern "C" {

// The oracle's own description of the paged KV cache (element strides).
typedef struct {
  const void* k_cache;
  const void* v_cache;
  int32_t dtype;  // 1 = bf16, 2 = FP8 E4M3FN
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_pages;
  int32_t pad_;
  int64_t k_stride_page, k_stride_token, k_stride_head;
  int64_t v_stride_page, v_stride_token, v_stride_head;
  const int32_t* block_table;
  int64_t block_table_stride;
  double k_descale;
  double v_descale;
} oracle_kv;

int oracle_abi_version(void) { return 1; }
double oracle_decode_bf16(uint16_t bits) { return decode_bf16(bits); }
double oracle_decode_e4m3fn(uint8_t code) { return decode_e4m3fn(code); }

}  // extern "C"

namespace {

struct Call {
  const void* q;
  int q_dtype;
  double q_descale;
  int hq;
  int num_seqs;
  const int32_t* cu_q;
  const int32_t* lens_k;
  const oracle_kv* kv;
  double scale;
  // sparse only
  const int32_t* indices;
  int64_t index_stride;
  int32_t num_selected;
};

// Logical key j of sequence b, kv head g: element offset inside the pool, or -1
// when the page id is outside the pool (never expected for valid inputs).
int64_t key_offset(const oracle_kv& kv, int b, int64_t j, int g, bool is_v) {
  const int64_t page = kv.block_table[static_cast<int64_t>(b) * kv.block_table_stride + j / kv.page_size];
  if (page < 0 || page >= kv.num_pages) return -1;
  const int64_t slot = j % kv.page_size;
  if (is_v) return page * kv.v_stride_page + slot * kv.v_stride_token + g * kv.v_stride_head;
  return page * kv.k_stride_page + slot * kv.k_stride_token + g * kv.k_stride_head;
}

// One (query token, kv group): all heads of the group attend the same key list.
// `keys` holds the logical positions to attend, in order.
void attend_group(const Call& c, int b, int64_t tok, int g, const std::vector<int64_t>& keys,
                  double* out, double* lse) {
  const oracle_kv& kv = *c.kv;
  const int r = c.hq / kv.num_kv_heads;
  const int64_t n = static_cast<int64_t>(keys.size());
  const double NEG_INF = -std::numeric_limits<double>::infinity();

  std::vector<double> qrow(static_cast<size_t>(r) * kHeadDim);
  for (int i = 0; i < r; ++i) {
    const int h = g * r + i;
    decode_row(c.q, c.q_dtype, (tok * c.hq + h) * kHeadDim, kHeadDim, &qrow[static_cast<size_t>(i) * kHeadDim]);
  }
  if (n == 0) {
    for (int i = 0; i < r; ++i) {
      const int h = g * r + i;
      for (int d = 0; d < kHeadDim; ++d) out[(tok * c.hq + h) * kHeadDim + d] = 0.0;
      lse[tok * c.hq + h] = NEG_INF;
    }
    return;
  }

  // Pass 1: scores s[i][j] for every head of the group.
  const double cscale = c.scale * c.q_descale * kv.k_descale;
  std::vector<double> s(static_cast<size_t>(r) * n);
  std::vector<double> row(kHeadDim);
  for (int64_t jj = 0; jj < n; ++jj) {
    const int64_t off = key_offset(kv, b, keys[jj], g, false);
    if (off < 0) {
      for (int d = 0; d < kHeadDim; ++d) row[d] = std::numeric_limits<double>::quiet_NaN();
    } else {
      decode_row(kv.k_cache, kv.dtype, off, kHeadDim, row.data());
    }
    for (int i = 0; i < r; ++i) {
      const double* qi = &qrow[static_cast<size_t>(i) * kHeadDim];
      double dot = 0.0;
      for (int d = 0; d < kHeadDim; ++d) dot += qi[d] * row[d];
      s[static_cast<size_t>(i) * n + jj] = cscale * dot;
    }
  }
  // Max, exponentials and their sum, per head.
  std::vector<double> m(r), l(r);
  for (int i = 0; i < r; ++i) {
    double* si = &s[static_cast<size_t>(i) * n];
    double mx = NEG_INF;
    for (int64_t jj = 0; jj < n; ++jj) mx = (si[jj] > mx || std::isnan(si[jj])) ? si[jj] : mx;
    double sum = 0.0;
    for (int64_t jj = 0; jj < n; ++jj) {
      si[jj] = std::exp(si[jj] - mx);  // s now holds p
      sum += si[jj];
    }
    m[i] = mx;
    l[i] = sum;
  }
  // Pass 2: weighted sum of V rows.
  std::vector<double> acc(static_cast<size_t>(r) * kHeadDim, 0.0);
  for (int64_t jj = 0; jj < n; ++jj) {
    const int64_t off = key_offset(kv, b, keys[jj], g, true);
    if (off < 0) {
      for (int d = 0; d < kHeadDim; ++d) row[d] = std::numeric_limits<double>::quiet_NaN();
    } else {
      decode_row(kv.v_cache, kv.dtype, off, kHeadDim, row.data());
    }
    for (int i = 0; i < r; ++i) {
      const double p = s[static_cast<size_t>(i) * n + jj];
      double* ai = &acc[static_cast<size_t>(i) * kHeadDim];
      for (int d = 0; d < kHeadDim; ++d) ai[d] += p * row[d];
    }
  }
  for (int i = 0; i < r; ++i) {
    const int h = g * r + i;
    for (int d = 0; d < kHeadDim; ++d)
      out[(tok * c.hq + h) * kHeadDim + d] = kv.v_descale * acc[static_cast<size_t>(i) * kHeadDim + d] / l[i];
    lse[tok * c.hq + h] = m[i] + std::log(l[i]);
  }
}

int check_common(const Call& c) {
  if (!c.q || !c.cu_q || !c.lens_k || !c.kv) return 1;
  const oracle_kv& kv = *c.kv;
  if (!kv.k_cache || !kv.v_cache || !kv.block_table) return 1;
  if (kv.head_dim != kHeadDim) return 2;
  if (kv.num_kv_heads <= 0 || c.hq <= 0 || c.hq % kv.num_kv_heads != 0) return 2;
  if (kv.page_size <= 0 || c.num_seqs < 0) return 2;
  if (c.q_dtype != kBF16 && c.q_dtype != kFP8) return 3;
  if (kv.dtype != kBF16 && kv.dtype != kFP8) return 3;
  return 0;
}

// Sequence of a global query token (cu_q is non-decreasing).
int seq_of_token(const Call& c, int64_t tok) {
  int lo = 0, hi = c.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (c.cu_q[mid] <= tok) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <class KeysFn>
int run(const Call& c, const int64_t* rows, int64_t num_rows, double* out, double* lse, int threads,
        KeysFn keys_of) {
  const int64_t T = c.num_seqs > 0 ? c.cu_q[c.num_seqs] : 0;
  std::vector<int64_t> toks;
  if (rows) {
    toks.assign(rows, rows + num_rows);
    for (int64_t t : toks)
      if (t < 0 || t >= T) return 2;
  } else {
    toks.resize(T);
    for (int64_t t = 0; t < T; ++t) toks[t] = t;
  }
  const int hkv = c.kv->num_kv_heads;
  const int64_t items = static_cast<int64_t>(toks.size()) * hkv;
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads)
  for (int64_t it = 0; it < items; ++it) {
    const int64_t tok = toks[it / hkv];
    const int g = static_cast<int>(it % hkv);
    const int b = seq_of_token(c, tok);
    std::vector<int64_t> keys;
    keys_of(b, tok, keys);
    attend_group(c, b, tok, g, keys, out, lse);
  }
  return 0;
}

}  // namespace

extern "C" {

// Bottom-right causal attention (speculative verify and prefix-hit prefill).
// q: [T, Hq, 256] codes of q_dtype, row-major.  out: [T, Hq, 256] fp64,
// lse: [T, Hq] fp64.  rows: optional list of global query-token indices to
// compute (the others are left untouched); NULL computes all tokens.
// Returns 0 on success, nonzero on invalid arguments.
int oracle_causal_attention(const void* q, int32_t q_dtype, double q_descale, int32_t num_q_heads,
                            int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                            const oracle_kv* kv, double softmax_scale, const int64_t* rows, int64_t num_rows,
                            double* out, double* lse, int32_t num_threads) {
  Call c{q, q_dtype, q_descale, num_q_heads, num_seqs, cu_seqlens_q, seq_lens_k, kv, softmax_scale,
         nullptr, 0, 0};
  if (int e = check_common(c)) return e;
  if (!out || !lse) return 1;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    if (lq < 0 || seq_lens_k[b] < lq) return 2;
  }
  return run(c, rows, num_rows, out, lse, num_threads, [&](int b, int64_t tok, std::vector<int64_t>& keys) {
    const int64_t lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    const int64_t t = tok - cu_seqlens_q[b];
    const int64_t last = static_cast<int64_t>(seq_lens_k[b]) - lq + t;  // inclusive
    keys.resize(static_cast<size_t>(last + 1));
    for (int64_t j = 0; j <= last; ++j) keys[static_cast<size_t>(j)] = j;
  });
}

// Selected-token attention.  indices: [T, index_stride] int32 logical key
// positions; the first num_selected entries of each row are read, and entries
// outside [0, Lk_b) are skipped.  No causal rule is applied beyond the list.
int oracle_sparse_attention(const void* q, int32_t q_dtype, double q_descale, int32_t num_q_heads,
                            int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                            const int32_t* indices, int64_t index_stride, int32_t num_selected,
                            const oracle_kv* kv, double softmax_scale, const int64_t* rows, int64_t num_rows,
                            double* out, double* lse, int32_t num_threads) {
  Call c{q, q_dtype, q_descale, num_q_heads, num_seqs, cu_seqlens_q, seq_lens_k, kv, softmax_scale,
         indices, index_stride, num_selected};
  if (int e = check_common(c)) return e;
  if (!out || !lse || !indices) return 1;
  if (num_selected < 0 || index_stride < num_selected) return 2;
  return run(c, rows, num_rows, out, lse, num_threads, [&](int b, int64_t tok, std::vector<int64_t>& keys) {
    keys.clear();
    const int32_t* row = indices + tok * index_stride;
    for (int32_t i = 0; i < num_selected; ++i)
      if (row[i] >= 0 && row[i] < seq_lens_k[b]) keys.push_back(row[i]);
  });
}

// Normalised attention weights of one (query token, head) over logical keys
// 0 .. Lk_b - 1 of its sequence (0 for keys it does not see), from the same
// definition as oracle_causal_attention.  probs: [Lk_b] fp64.
int oracle_causal_probs(const void* q, int32_t q_dtype, double q_descale, int32_t num_q_heads,
                        int32_t num_seqs, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                        const oracle_kv* kv, double softmax_scale, int64_t token, int32_t head, double* probs) {
  Call c{q, q_dtype, q_descale, num_q_heads, num_seqs, cu_seqlens_q, seq_lens_k, kv, softmax_scale,
         nullptr, 0, 0};
  if (int e = check_common(c)) return e;
  if (!probs || head < 0 || head >= num_q_heads || num_seqs <= 0) return 1;
  if (token < 0 || token >= cu_seqlens_q[num_seqs]) return 2;
  const int b = seq_of_token(c, token);
  const int64_t lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
  const int64_t lk = seq_lens_k[b];
  const int64_t last = lk - lq + (token - cu_seqlens_q[b]);
  const int r = num_q_heads / kv->num_kv_heads;
  const int g = head / r;
  std::vector<double> qrow(kHeadDim), row(kHeadDim);
  decode_row(q, q_dtype, (token * num_q_heads + head) * kHeadDim, kHeadDim, qrow.data());
  const double cscale = softmax_scale * q_descale * kv->k_descale;
  std::vector<double> s(static_cast<size_t>(last + 1));
  double mx = -std::numeric_limits<double>::infinity();
  for (int64_t j = 0; j <= last; ++j) {
    const int64_t off = key_offset(*kv, b, j, g, false);
    if (off < 0) return 4;
    decode_row(kv->k_cache, kv->dtype, off, kHeadDim, row.data());
    double dot = 0.0;
    for (int d = 0; d < kHeadDim; ++d) dot += qrow[d] * row[d];
    s[static_cast<size_t>(j)] = cscale * dot;
    if (s[static_cast<size_t>(j)] > mx) mx = s[static_cast<size_t>(j)];
  }
  double sum = 0.0;
  for (int64_t j = 0; j <= last; ++j) sum += (s[static_cast<size_t>(j)] = std::exp(s[static_cast<size_t>(j)] - mx));
  for (int64_t j = 0; j < lk; ++j) probs[j] = (j <= last) ? s[static_cast<size_t>(j)] / sum : 0.0;
  return 0;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Per-tensor FP8 quantisation of the prefill inputs: the casts of Q and of the
// new keys and values to FP8 that ROCm/ATOM PR #2534 counts inside its prefill
// timings (FMHA commit message; Results, per-layer trace).  The page fixes no
// scale rule, so the oracle takes the plainest one, in the precision the
// kernels use (fp32):
//   amax    = max |x| over the non-NaN elements (exact: x is bf16)
//   descale = fp32(amax / 448), or 1 when amax is 0 (dynamic scale, Q)
//   y       = fp32(x / descale)
//   code    = the E4M3FN value nearest to y, ties to the even code, with
//             finite y beyond +-448 saturated to +-448 and NaN kept NaN.
// New keys and values use the pool's own per-tensor descales (static scales:
// the pool already holds the cached prefix under them) and land at logical
// position Lk_b - Lq_b + t of their sequence, through the block table.

namespace {

// Codes 0x00 .. 0x7E are the finite non-negative E4M3FN values in increasing
// order; a binary search over their decoded values finds the neighbours of |y|.
uint8_t encode_e4m3fn(float y) {
  if (std::isnan(y)) return std::signbit(y) ? 0xFF : 0x7F;
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  const double a = std::fabs(static_cast<double>(y));
  const E4M3Table& t = e4m3_table();
  int lo = 0, hi = 0x7E;  // largest code c with value(c) <= a
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (t.v[mid] <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  if (c < 0x7E) {
    const double below = a - t.v[c], above = t.v[c + 1] - a;  // exact in fp64
    if (above < below || (above == below && (c & 1))) c += 1;
  }
  return static_cast<uint8_t>(sign | c);
}

float bf16_to_float(uint16_t bits) {
  uint32_t w = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return f;
}

uint8_t quantize_one(uint16_t bits, float descale) {
  const float y = bf16_to_float(bits) / descale;  // one IEEE fp32 division
  return encode_e4m3fn(y);
}

}  // namespace

extern "C" {

uint8_t oracle_encode_e4m3fn(float y) { return encode_e4m3fn(y); }

// x: n bf16 patterns.  descale_in: NULL for the dynamic scale, else the fp32
// descale to use.  codes: n bytes out.  descale_out: the descale used.
int oracle_quantize_fp8(const uint16_t* x, int64_t n, const float* descale_in, uint8_t* codes,
                        float* descale_out) {
  if ((!x && n > 0) || (!codes && n > 0) || !descale_out || n < 0) return 1;
  float descale;
  if (descale_in) {
    descale = *descale_in;
  } else {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
      const float a = std::fabs(bf16_to_float(x[i]));
      if (!std::isnan(a) && a > amax) amax = a;
    }
    descale = amax > 0.0f ? amax / 448.0f : 1.0f;
  }
  for (int64_t i = 0; i < n; ++i) codes[i] = quantize_one(x[i], descale);
  *descale_out = descale;
  return 0;
}

// Quantise the new tokens' keys and values ([T, Hkv, 256] bf16 each, token
// order of cu_seqlens_q) with the given descales and write them into the FP8
// pool of `kv` (its caches are written through) at logical positions
// Lk_b - Lq_b + t, Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b].  A position
// before the sequence start or on a page id outside the pool is not written.
int oracle_write_new_kv(const uint16_t* k_new, const uint16_t* v_new, int32_t num_seqs,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const oracle_kv* kv,
                        float k_descale, float v_descale) {
  if (!k_new || !v_new || !cu_seqlens_q || !cu_seqlens_k || !kv || kv->dtype != kFP8) return 1;
  uint8_t* kp = static_cast<uint8_t*>(const_cast<void*>(kv->k_cache));
  uint8_t* vp = static_cast<uint8_t*>(const_cast<void*>(kv->v_cache));
  const int hkv = kv->num_kv_heads;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t lq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    const int64_t lk = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
    for (int64_t t = 0; t < lq; ++t) {
      const int64_t pos = lk - lq + t;
      if (pos < 0) continue;
      const int64_t tok = cu_seqlens_q[b] + t;
      for (int g = 0; g < hkv; ++g) {
        const int64_t ko = key_offset(*kv, b, pos, g, false);
        const int64_t vo = key_offset(*kv, b, pos, g, true);
        const int64_t src = (tok * hkv + g) * kHeadDim;
        for (int d = 0; d < kHeadDim; ++d) {
          if (ko >= 0) kp[ko + d] = quantize_one(k_new[src + d], k_descale);
          if (vo >= 0) vp[vo + d] = quantize_one(v_new[src + d], v_descale);
        }
      }
    }
  }
  return 0;
}

}  // extern "C"

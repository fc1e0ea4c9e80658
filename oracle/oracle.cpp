// CPU oracle for the gated DSA forward: learned indexer, hard top-k, sparse latent attention,
// per-head V up-projection and sigmoid output gate.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file; only
// the tests, the package smoke check and the benchmark's CPU-baseline leg use it. It shares no
// code, header, table or constant with the GPU library: even the bf16 helpers are written here
// again.
//
// Sources (the pages are cited by title and section):
//  [KC] NeMo AutoModel, "Kimi-K3.1-Pro" model-coverage page.
//       - summary paragraph: every one of the 24 gated MLA layers has a learned indexer that keeps
//         at most 2,048 causal keys for each query.
//       - Implementation Limits, 1st bullet: the indexer produces top-k coordinates and the sparse
//         kernels attend directly to the selected latent KV; eager/sdpa are dense-mask references.
//       - Implementation Limits, 2nd bullet: indexer projections are BF16 with FP32 score
//         accumulation; the indexer scans every causal key; sparse MLA never expands per-head K/V.
//       - Implementation Limits, 3rd bullet: selection is hard top-k.
//       - Implementation Limits, 4th bullet: a sequence of at most 2,048 valid tokens keeps every
//         causal key.
//       - paragraph after the bullets on the output gate and kv_b_proj: the gate is kept; the V
//         projection is taken through its effective weight; packed documents are contiguous.
//  [AD] archdiff.com "Kimi K3.1 Pro" blueprint: LayerNorm on the indexer key; output gate
//       sigma(x W_g) * o; no positional encoding (tagline).
//  [API] NeMo AutoModel kimi_k3 API index, KimiK3TextConfig: 96 heads, kv_lora_rank 512,
//       qk_rope_head_dim 64 (left unrotated: mla_use_nope), v_head_dim 128.
//  The scoring form  S(t,s) = sum_h w[t,h] * ReLU(q_I[t,h] . LN(k_I[s]))  and the tie rule (equal
//  scores go to the lower key index) are not on the pages; they are the problem statement's
//  reading and are used here verbatim.
//
// Readings where the pages are silent (each is listed in the design notes):
//  - LayerNorm: biased variance, eps given by the caller (1e-5), optional affine; computed in
//    double and rounded once to bf16 (round-to-nearest-even) because the indexer contraction
//    consumes bf16 operands.
//  - Causal keys of token t are the tokens of its own document up to and including t.
//  - Scores: FP32 products and FP32 sequential accumulation, first over the d_I dims of each
//    indexer head, then over heads in head order. ReLU returns +0 for non-positive dots.
//  - Attention: softmax scale given by the caller (1/sqrt(192)); no sink; the first 512 latent
//    dims are V, all 576 are K; no rotation of the last 64 dims.
//  - Gate: one logit per (token, head), applied after the up-projection.
//  - Attention arithmetic is in double; the gated output is rounded once to bf16 (RNE).
//
// Build: g++ -O2 -std=c++17 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math, so every
// FP32 sum below is evaluated in the order written).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

constexpr int kDL = 576;  // latent row: kv_lora_rank 512 + 64 unrotated dims  [API]
constexpr int kDV = 512;  // V part of a latent row                            [API]
constexpr int kDO = 128;  // v_head_dim                                        [API]

float bf16_bits_to_float(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Value of one input element: bf16 bits, or a double (the double-input form used to pin the
// backward by finite differences).
inline double in_val(uint16_t b) { return bf16_bits_to_float(b); }
inline double in_val(double x) { return x; }

// Round a finite double to the nearest bf16 (ties to even), in one step.
uint16_t double_to_bf16_rne(double x) {
  if (x == 0.0) return std::signbit(x) ? 0x8000 : 0x0000;
  int e = 0;
  double m = std::frexp(x, &e);            // |m| in [0.5, 1)
  double r = std::nearbyint(std::ldexp(m, 8));  // 8 significant bits, ties to even
  float f = static_cast<float>(std::ldexp(r, e - 8));  // exact: at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}

// First token of the document holding token t. cu has n_docs+1 entries, strictly increasing,
// cu[0] = 0, cu[n_docs] = T. NULL cu means one document [0, T).
int64_t doc_begin(const int32_t* cu, int32_t n_docs, int64_t t) {
  if (cu == nullptr) return 0;
  for (int32_t d = 0; d < n_docs; ++d)
    if (t < cu[d + 1]) return cu[d];
  return -1;
}

// ---- FP8 E4M3 (the OCP 8-bit floating-point format "E4M3": 1 sign bit, 4 exponent bits with
// bias 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no infinities; S.1111.111
// is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448). Written from that definition.

// Value of an E4M3 code.
double e4m3_decode(uint8_t c) {
  const int sgn = c >> 7, E = (c >> 3) & 15, m = c & 7;
  if (E == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  const double mag = E == 0 ? std::ldexp(static_cast<double>(m), -9) : std::ldexp(1.0 + m / 8.0, E - 7);
  return sgn ? -mag : mag;
}

// Nearest E4M3 code to v (ties to the even code), for |v| <= 448.
uint8_t e4m3_encode(double v) {
  const uint8_t sgn = std::signbit(v) ? 0x80 : 0x00;
  const double a = std::fabs(v);
  if (a == 0.0) return sgn;
  if (a < std::ldexp(1.0, -6)) {  // subnormal range: multiples of 2^-9
    const double q = std::nearbyint(std::ldexp(a, 9));  // default rounding mode: ties to even
    return static_cast<uint8_t>(sgn | static_cast<int>(q));  // q == 8 is the smallest normal, code 0x08
  }
  int ex = 0;
  const double m = std::frexp(a, &ex);  // a = m * 2^ex, m in [0.5, 1)
  int E = ex - 1;                       // a = (2m) * 2^E, 2m in [1, 2)
  double q = std::nearbyint((2.0 * m - 1.0) * 8.0);
  if (q == 8.0) {
    q = 0.0;
    ++E;
  }
  return static_cast<uint8_t>(sgn | ((E + 7) << 3) | static_cast<int>(q));
}

// Exponent of a row's power-of-two scale: the smallest integer e with amax * 2^-e <= 448 (0 for an
// all-zero row).
int fp8_scale_exponent(double amax) {
  if (amax == 0.0) return 0;
  int e = std::ilogb(amax) - 8;
  while (std::ldexp(amax, -e) > 448.0) ++e;
  while (std::ldexp(amax, -(e - 1)) <= 448.0) --e;
  return e;
}

}  // namespace

extern "C" {

int oracle_abi_version() { return 1; }

// Threads the OpenMP loops below run with.
int oracle_num_threads() {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int64_t oracle_doc_begin(const int32_t* cu, int32_t n_docs, int64_t t) { return doc_begin(cu, n_docs, t); }

// Step: LayerNorm on the indexer key ([AD] "LayerNorm on the indexer key").
// LNk[s,i] = bf16( (x_i - mean) / sqrt(var + eps) * gamma_i + beta_i ), var biased, in double.
// pre (optional, [T,d_I]) receives the double value before rounding.
void oracle_key_layernorm(const uint16_t* k_I, int64_t T, int32_t d_I, const float* gamma, const float* beta,
                          double eps, uint16_t* LNk, double* pre) {
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < T; ++s) {
    const uint16_t* x = k_I + s * d_I;
    double mean = 0.0;
    for (int32_t i = 0; i < d_I; ++i) mean += bf16_bits_to_float(x[i]);
    mean /= d_I;
    double var = 0.0;
    for (int32_t i = 0; i < d_I; ++i) {
      double c = bf16_bits_to_float(x[i]) - mean;
      var += c * c;
    }
    var /= d_I;
    double inv = 1.0 / std::sqrt(var + eps);
    for (int32_t i = 0; i < d_I; ++i) {
      double y = (bf16_bits_to_float(x[i]) - mean) * inv;
      if (gamma) y *= gamma[i];
      if (beta) y += beta[i];
      if (pre) pre[s * d_I + i] = y;
      LNk[s * d_I + i] = double_to_bf16_rne(y);
    }
  }
}

// Step: indexer scores of one query over keys s0..s1 inclusive ([KC] Implementation Limits,
// 2nd bullet: BF16 operands, FP32 accumulation).
// S[s-s0] = sum_h w[h] * ReLU( sum_i qI[h,i] * LNk[s,i] ), all in FP32, in the order written.
void oracle_index_scores(const uint16_t* qI_row, const uint16_t* w_row, int32_t H_I, int32_t d_I,
                         const uint16_t* LNk, int64_t s0, int64_t s1, float* S) {
  for (int64_t s = s0; s <= s1; ++s) {
    const uint16_t* k = LNk + s * d_I;
    float score = 0.0f;
    for (int32_t h = 0; h < H_I; ++h) {
      const uint16_t* q = qI_row + static_cast<int64_t>(h) * d_I;
      float dot = 0.0f;
      for (int32_t i = 0; i < d_I; ++i) dot += bf16_bits_to_float(q[i]) * bf16_bits_to_float(k[i]);
      float r = dot > 0.0f ? dot : 0.0f;  // +0 for every non-positive dot
      score += bf16_bits_to_float(w_row[h]) * r;
    }
    S[s - s0] = score;
  }
}

// Error scale of one score: sum_h |w[h]| * sum_i |qI[h,i] * LNk[s,i]| in double. Any FP32
// evaluation of a score (any summation order) lies within (d_I + H_I) * 2^-24 / (1 - ...) times
// this value of the exact score.
void oracle_index_score_scale(const uint16_t* qI_row, const uint16_t* w_row, int32_t H_I, int32_t d_I,
                              const uint16_t* LNk, int64_t s0, int64_t s1, double* out) {
  for (int64_t s = s0; s <= s1; ++s) {
    const uint16_t* k = LNk + s * d_I;
    double acc = 0.0;
    for (int32_t h = 0; h < H_I; ++h) {
      const uint16_t* q = qI_row + static_cast<int64_t>(h) * d_I;
      double dot = 0.0;
      for (int32_t i = 0; i < d_I; ++i)
        dot += std::fabs(static_cast<double>(bf16_bits_to_float(q[i])) * bf16_bits_to_float(k[i]));
      acc += std::fabs(static_cast<double>(bf16_bits_to_float(w_row[h]))) * dot;
    }
    out[s - s0] = acc;
  }
}

// Step: hard top-k ([KC] summary; Implementation Limits 3rd and 4th bullets).
// For each listed query row t (global index rows[r]) with causal keys b(t)..t (n_t of them):
//  - n_t <= k: every causal key is kept (the short-sequence rule);
//  - otherwise the k keys that come first when the causal keys, listed in ascending index order,
//    are stably sorted by score, highest first (so equal scores keep the lower index).
// idx_out[r, :] holds the kept global indices in ascending order, then -1 up to k.
// theta_out[r] = score of the k-th kept key (NaN when n_t <= k); keff_out[r] = min(k, n_t).
}  // extern "C"

// Selection of one row (t in the document starting at b), given a function that fills the scores of
// keys b..t: every causal key when n_t <= k, else the first k of the causal keys listed in ascending
// index order and stably sorted by score, highest first.
template <typename ScoreFn>
static void select_row(int64_t b, int64_t t, int32_t k, ScoreFn scores, int32_t* out, float* theta_out,
                       int32_t* keff_out) {
  const int64_t n_t = t - b + 1;
  std::vector<int64_t> kept;
  float theta = std::numeric_limits<float>::quiet_NaN();
  if (n_t <= k) {
    for (int64_t s = b; s <= t; ++s) kept.push_back(s);
  } else {
    std::vector<float> S(static_cast<size_t>(n_t));
    scores(S.data());
    std::vector<int64_t> order(static_cast<size_t>(n_t));
    std::iota(order.begin(), order.end(), b);  // ascending key index
    std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) { return S[x - b] > S[y - b]; });
    kept.assign(order.begin(), order.begin() + k);
    theta = S[kept.back() - b];
    std::sort(kept.begin(), kept.end());
  }
  for (int32_t j = 0; j < k; ++j) out[j] = j < static_cast<int32_t>(kept.size()) ? static_cast<int32_t>(kept[j]) : -1;
  *theta_out = theta;
  *keff_out = static_cast<int32_t>(kept.size());
}

extern "C" {

void oracle_topk(int64_t n_rows, const int64_t* rows, const uint16_t* qI_rows, const uint16_t* w_rows,
                 int32_t H_I, int32_t d_I, const uint16_t* LNk, const int32_t* cu, int32_t n_docs, int32_t k,
                 int32_t* idx_out, float* theta_out, int32_t* keff_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = rows[r];
    const int64_t b = doc_begin(cu, n_docs, t);
    select_row(b, t, k, [&](float* S) {
      oracle_index_scores(qI_rows + r * static_cast<int64_t>(H_I) * d_I, w_rows + r * H_I, H_I, d_I, LNk, b, t, S);
    }, idx_out + r * k, theta_out + r, keff_out + r);
  }
}

// ---- FP8 indexer ([KC] Implementation Limits, 2nd bullet: the BF16 indexer "is not the FP8 indexer"
// of some serving kernels). The pages give no recipe; the one used here: each 128-wide row (a key's
// LN output, one head of a query's q_I) is scaled by a power of two 2^-e, e the smallest integer
// that brings its largest magnitude to at most 448, and rounded to E4M3 (nearest, ties to even).
// The products of two E4M3 values are exact in FP32 and are summed in FP32; ReLU, the head weight
// times the query row's head scale 2^e_q, the head sum in FP32, then the key's scale 2^e_k.

// Quantise n rows of d bf16 values: q8 [n,d] E4M3 codes, e [n] scale exponents.
void oracle_quantize_fp8_rows(const uint16_t* x, int64_t n, int32_t d, uint8_t* q8, int32_t* e) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    const uint16_t* xr = x + r * d;
    double amax = 0.0;
    for (int32_t i = 0; i < d; ++i) amax = std::max(amax, std::fabs(static_cast<double>(bf16_bits_to_float(xr[i]))));
    const int ex = fp8_scale_exponent(amax);
    e[r] = ex;
    for (int32_t i = 0; i < d; ++i) q8[r * d + i] = e4m3_encode(std::ldexp(static_cast<double>(bf16_bits_to_float(xr[i])), -ex));
  }
}

double oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t oracle_e4m3_encode(double v) { return e4m3_encode(v); }
int32_t oracle_fp8_scale_exponent(double amax) { return fp8_scale_exponent(amax); }

// FP8 scores of one query (q8_row [H_I,d_I] codes, eq [H_I], w_row [H_I] bf16) over keys s0..s1 of
// (k8 [*,d_I] codes, ek [*]):  S = 2^ek[s] * sum_h (w_h * 2^eq_h) * ReLU( sum_i q8[h,i] * k8[s,i] ).
void oracle_index_scores_fp8(const uint8_t* q8_row, const int32_t* eq, const uint16_t* w_row, int32_t H_I,
                             int32_t d_I, const uint8_t* k8, const int32_t* ek, int64_t s0, int64_t s1, float* S) {
  // the value of every code, from e4m3_decode (finite codes are exact in float)
  static const std::vector<float> dec = [] {
    std::vector<float> v(256);
    for (int c = 0; c < 256; ++c) v[c] = static_cast<float>(e4m3_decode(static_cast<uint8_t>(c)));
    return v;
  }();
  std::vector<float> qv(static_cast<size_t>(H_I) * d_I), wq(H_I);
  for (int64_t i = 0; i < static_cast<int64_t>(qv.size()); ++i) qv[i] = dec[q8_row[i]];
  for (int32_t h = 0; h < H_I; ++h) wq[h] = std::ldexp(bf16_bits_to_float(w_row[h]), eq[h]);  // exact
  for (int64_t s = s0; s <= s1; ++s) {
    float score = 0.0f;
    for (int32_t h = 0; h < H_I; ++h) {
      float dot = 0.0f;
      for (int32_t i = 0; i < d_I; ++i) dot += qv[h * d_I + i] * dec[k8[s * d_I + i]];
      const float rl = dot > 0.0f ? dot : 0.0f;
      score += wq[h] * rl;
    }
    S[s - s0] = std::ldexp(score, ek[s]);
  }
}

// Hard top-k on the FP8 scores; same outputs as oracle_topk.
void oracle_topk_fp8(int64_t n_rows, const int64_t* rows, const uint8_t* q8_rows, const int32_t* eq_rows,
                     const uint16_t* w_rows, int32_t H_I, int32_t d_I, const uint8_t* k8, const int32_t* ek,
                     const int32_t* cu, int32_t n_docs, int32_t k, int32_t* idx_out, float* theta_out,
                     int32_t* keff_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = rows[r];
    const int64_t b = doc_begin(cu, n_docs, t);
    select_row(b, t, k, [&](float* S) {
      oracle_index_scores_fp8(q8_rows + r * static_cast<int64_t>(H_I) * d_I, eq_rows + r * H_I, w_rows + r * H_I,
                              H_I, d_I, k8, ek, b, t, S);
    }, idx_out + r * k, theta_out + r, keff_out + r);
  }
}

// Step: sparse latent attention over the given key indices, then the per-head V up-projection
// and the sigmoid output gate ([KC] Implementation Limits 1st/2nd bullets and the paragraph on
// the output gate and kv_b_proj; [AD] output gate; [API] shapes).
// For row r (global token rows[r]) and head h, over the valid entries s_j of idx[r, :] (entries
// outside [0, T) are skipped):
//   l_j  = scale * sum_{i<576} q[r,h,i] * kv[s_j,i]
//   p_j  = exp(l_j - max l) / sum_j exp(l_j - max l)
//   ol_c = sum_j p_j * kv[s_j, c]                    (c < 512)
//   o_d  = sum_c ol_c * W_UV[h, c, d]                 (d < 128)
//   out  = o_d * 1 / (1 + exp(-gate[r, h]))
}  // extern "C"

// Accumulation type R: double on parity runs; float for the timed CPU baseline only (the same
// steps in the same order, in single precision). Outputs (each optional): o_pre [n,H,128] before
// the gate, out_f64 [n,H,128], out_bf16 (RNE of out_f64), lse [n,H] = log(sum_j exp(l_j) [+ exp(sink)]),
// psum [n,H] = sum_j p_j.
// Variants ([AD] blueprint entry "Output gate + sink": sigma(x W_g) * o and a learnable sink):
//  - gate_per_dim = 0: gate_rows [n,H], one logit per (row, head), broadcast over the 128 outputs;
//    gate_per_dim = 1: gate_rows [n,H,128], one logit per output element.
//  - sink [H] or NULL: head h's softmax gains one more term exp(sink[h]) in its denominator, a
//    logit whose value row is zero (it takes weight from the keys and adds nothing to o_lat).
template <typename R, typename In>
void sparse_mla_impl(int64_t n_rows, const In* q_rows, const In* kv, int64_t T, const int32_t* idx,
                     int32_t k, const In* W_UV, const In* gate_rows, int32_t H, double scale,
                     int32_t gate_per_dim, const double* sink, double* o_pre, double* out_f64, uint16_t* out_bf16,
                     double* lse, double* psum) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    std::vector<int64_t> sel;
    for (int32_t j = 0; j < k; ++j) {
      int64_t s = idx[r * k + j];
      if (s >= 0 && s < T) sel.push_back(s);
    }
    const size_t n = sel.size();
    std::vector<R> l(n), ol(kDV);
    for (int32_t h = 0; h < H; ++h) {
      const In* qh = q_rows + (r * H + h) * static_cast<int64_t>(kDL);
      for (size_t j = 0; j < n; ++j) {
        const In* kr = kv + sel[j] * kDL;
        R dot = 0;
        for (int i = 0; i < kDL; ++i)
          dot += static_cast<R>(in_val(qh[i])) * static_cast<R>(in_val(kr[i]));
        l[j] = static_cast<R>(scale) * dot;
      }
      R m = -std::numeric_limits<R>::infinity();
      for (size_t j = 0; j < n; ++j) m = std::max(m, l[j]);
      if (sink) m = std::max(m, static_cast<R>(sink[h]));
      R z = 0;
      for (size_t j = 0; j < n; ++j) z += std::exp(l[j] - m);
      if (sink) z += std::exp(static_cast<R>(sink[h]) - m);
      std::fill(ol.begin(), ol.end(), R(0));
      R ps = 0;
      for (size_t j = 0; j < n; ++j) {
        R p = std::exp(l[j] - m) / z;
        ps += p;
        const In* vr = kv + sel[j] * kDL;
        for (int c = 0; c < kDV; ++c) ol[c] += p * static_cast<R>(in_val(vr[c]));
      }
      const In* Wh = W_UV + static_cast<int64_t>(h) * kDV * kDO;
      for (int d = 0; d < kDO; ++d) {
        R o = 0;
        for (int c = 0; c < kDV; ++c) o += ol[c] * static_cast<R>(in_val(Wh[c * kDO + d]));
        const int64_t at = (r * H + h) * static_cast<int64_t>(kDO) + d;
        if (o_pre) o_pre[at] = o;
        const R g = static_cast<R>(in_val(gate_per_dim ? gate_rows[at] : gate_rows[r * H + h]));
        const R sig = R(1) / (R(1) + std::exp(-g));
        const R y = o * sig;
        if (out_f64) out_f64[at] = y;
        if (out_bf16) out_bf16[at] = double_to_bf16_rne(static_cast<double>(y));
      }
      if (lse) lse[r * H + h] = m + std::log(z);
      if (psum) psum[r * H + h] = ps;
    }
  }
}

extern "C" {

// All in double (the parity reference).
void oracle_sparse_mla(int64_t n_rows, const int64_t* rows, const uint16_t* q_rows, const uint16_t* kv, int64_t T,
                       const int32_t* idx, int32_t k, const uint16_t* W_UV, const uint16_t* gate_rows, int32_t H,
                       double scale, double* o_pre, double* out_f64, uint16_t* out_bf16, double* lse, double* psum) {
  (void)rows;
  sparse_mla_impl<double, uint16_t>(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, 0, nullptr, o_pre,
                                    out_f64, out_bf16, lse, psum);
}

// The gate and sink variants ([AD] "Output gate + sink"), in double: gate_per_dim selects a gate
// [n,H,128] instead of [n,H]; sink [H] (or NULL) adds exp(sink[h]) to head h's softmax denominator.
void oracle_sparse_mla_variant(int64_t n_rows, const int64_t* rows, const uint16_t* q_rows, const uint16_t* kv,
                               int64_t T, const int32_t* idx, int32_t k, const uint16_t* W_UV,
                               const uint16_t* gate_rows, int32_t H, double scale, int32_t gate_per_dim,
                               const double* sink, double* o_pre, double* out_f64, uint16_t* out_bf16, double* lse,
                               double* psum) {
  (void)rows;
  sparse_mla_impl<double, uint16_t>(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, gate_per_dim, sink,
                                    o_pre, out_f64, out_bf16, lse, psum);
}

// The same definition accumulated in float: used only to time the oracle as a CPU baseline.
void oracle_sparse_mla_f32(int64_t n_rows, const int64_t* rows, const uint16_t* q_rows, const uint16_t* kv,
                           int64_t T, const int32_t* idx, int32_t k, const uint16_t* W_UV, const uint16_t* gate_rows,
                           int32_t H, double scale, double* out_f64) {
  (void)rows;
  sparse_mla_impl<float, uint16_t>(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, 0, nullptr, nullptr,
                                   out_f64, nullptr, nullptr, nullptr);
}

// The step before the attention: the per-head W_UK absorption that gives the latent query ([KC]
// Implementation Limits, 2nd bullet: sparse MLA never expands the per-head K; [API]
// KimiK3TextConfig: qk_nope_head_dim 128, kv_lora_rank 512, qk_rope_head_dim 64, mla_use_nope).
// W_UK [H,512,128] is the key half of the kv_b_proj effective weight: head h's expanded key of a
// token would be k_nope[d] = sum_c c_KV[c] * W_UK[h,c,d]. So q_nope . k_nope = q_lat . c_KV with
//   q[t,h,c]       = sum_d q_nope[t,h,d] * W_UK[h,c,d]     c < 512, in double, one bf16 rounding
//   q[t,h,512 + j] = q_pe[t,h,j]                           j < 64, unrotated (no positional encoding)
// q_lat_f64 (optional) receives the unrounded latent part.
void oracle_q_absorb(int64_t n_rows, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* W_UK, int32_t H,
                     uint16_t* q_out, double* q_lat_f64) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t* qn = q_nope + (r * H + h) * 128;
      const uint16_t* Wh = W_UK + static_cast<int64_t>(h) * kDV * 128;
      uint16_t* dst = q_out + (r * H + h) * static_cast<int64_t>(kDL);
      for (int c = 0; c < kDV; ++c) {
        double acc = 0.0;
        for (int d = 0; d < 128; ++d)
          acc += static_cast<double>(bf16_bits_to_float(qn[d])) * bf16_bits_to_float(Wh[c * 128 + d]);
        if (q_lat_f64) q_lat_f64[(r * H + h) * kDV + c] = acc;
        dst[c] = double_to_bf16_rne(acc);
      }
      for (int j = 0; j < kDL - kDV; ++j) dst[kDV + j] = q_pe[(r * H + h) * (kDL - kDV) + j];
    }
  }
}

// The step after the gate: the attention output projection o_proj ([KC] paragraph on the output
// gate and kv_b_proj; [API] KimiK3TextConfig hidden_size 7168, v_head_dim 128, 96 heads). The
// gated head outputs of a row, heads in order, form x [K = H * 128]; W_o [N, K] is in the
// [out_features, in_features] layout:
//   y[t,n] = bf16( sum_k x[t,k] * W_o[n,k] )     in double, one rounding
// y_f64 (optional) receives the unrounded values.
void oracle_o_proj(int64_t n_rows, const uint16_t* x, const uint16_t* W_o, int32_t K, int32_t N, uint16_t* y,
                   double* y_f64) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    std::vector<double> xr(static_cast<size_t>(K));
    for (int32_t k = 0; k < K; ++k) xr[k] = bf16_bits_to_float(x[r * K + k]);
    for (int32_t n = 0; n < N; ++n) {
      const uint16_t* wn = W_o + static_cast<int64_t>(n) * K;
      double acc = 0.0;
      for (int32_t k = 0; k < K; ++k) acc += xr[k] * bf16_bits_to_float(wn[k]);
      if (y_f64) y_f64[r * N + n] = acc;
      y[r * N + n] = double_to_bf16_rne(acc);
    }
  }
}

// The same forward with double inputs (q [n,H,576], kv [T,576], W_UV [H,512,128], gate [n,H]): the
// point at which the backward below is checked by finite differences.
void oracle_sparse_mla_f64in(int64_t n_rows, const double* q_rows, const double* kv, int64_t T, const int32_t* idx,
                             int32_t k, const double* W_UV, const double* gate_rows, int32_t H, double scale,
                             double* out_f64, double* lse) {
  sparse_mla_impl<double, double>(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, 0, nullptr, nullptr,
                                  out_f64, nullptr, lse, nullptr);
}

// The gate and sink variants of the same forward with double inputs (gate [n,H] or [n,H,128]).
void oracle_sparse_mla_f64in_variant(int64_t n_rows, const double* q_rows, const double* kv, int64_t T,
                                     const int32_t* idx, int32_t k, const double* W_UV, const double* gate_rows,
                                     int32_t H, double scale, int32_t gate_per_dim, const double* sink,
                                     double* out_f64, double* lse) {
  sparse_mla_impl<double, double>(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, gate_per_dim, sink,
                                  nullptr, out_f64, nullptr, lse, nullptr);
}

// Backward of sparse latent attention, the per-head V up-projection and the per-head sigmoid gate
// ([KC] paragraph after the Implementation Limits bullets: the backward runs the native 96 heads;
// 3rd bullet: hard top-k carries no gradient, so the indices are constants). For the loss
// L = sum dout * out, with the forward's definitions and p_j = exp(l_j - lse), written out by the
// chain rule in double (inputs as double arrays):
//   sg = sigma(g); o = o_lat W_UV[h]; dgate = sg (1 - sg) sum_d dout[d] o[d]; do = sg dout
//   dW_UV[h,c,d] += o_lat[c] do[d]; do_lat[c] = sum_d W_UV[h,c,d] do[d]
//   dp_j = do_lat . kv_j[:512];  D = sum_j p_j dp_j;  dl_j = p_j (dp_j - D)
//   dq = scale sum_j dl_j kv_j (576 dims);  dkv_j += scale dl_j q (576) + p_j do_lat (512)
// Outputs: dq [n,H,576] and dgate [n,H] (written), dkv [T,576] and dW [H,512,128] (added to).
//
// The gate and sink variants ([AD] blueprint entry "Output gate + sink"), as in the forward:
//  - gate_per_dim = 1: gate [n,H,128], sg_d = sigma(g_d) per output element, so
//    dgate[d] = sg_d (1 - sg_d) dout[d] o[d] (dgate [n,H,128]) and do[d] = sg_d dout[d];
//  - sink [H]: the softmax over the keys and the sink logit s (value row zero):
//    p_j = exp(l_j - m) / z, p_s = exp(s - m) / z, z = sum_j exp(l_j - m) + exp(s - m). o_lat and
//    D = sum_j p_j dp_j take the keys only (the sink's dp is 0), dl_j = p_j (dp_j - D) as before,
//    and the sink logit's own gradient is p_s (0 - D): dsink[h] += -p_s D over the rows.
void oracle_sparse_mla_bwd_variant(int64_t n_rows, const double* q_rows, const double* kv, int64_t T,
                                   const int32_t* idx, int32_t k, const double* W_UV, const double* gate_rows,
                                   int32_t H, double scale, int32_t gate_per_dim, const double* sink,
                                   const double* dout, double* dq, double* dkv, double* dW, double* dgate,
                                   double* dsink) {
  for (int64_t r = 0; r < n_rows; ++r) {
    std::vector<int64_t> sel;
    for (int32_t j = 0; j < k; ++j) {
      const int64_t s = idx[r * k + j];
      if (s >= 0 && s < T) sel.push_back(s);
    }
    const size_t n = sel.size();
    // per head: the contributions to the selected rows of dkv, summed over heads afterwards
    std::vector<double> dkv_h(static_cast<size_t>(H) * n * kDL, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t h = 0; h < H; ++h) {
      const double* qh = q_rows + (r * H + h) * static_cast<int64_t>(kDL);
      const double* Wh = W_UV + static_cast<int64_t>(h) * kDV * kDO;
      std::vector<double> l(n), p(n), ol(kDV, 0.0), o(kDO, 0.0), dov(kDO), dol(kDV, 0.0), dp(n);
      for (size_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int i = 0; i < kDL; ++i) dot += qh[i] * kv[sel[j] * kDL + i];
        l[j] = scale * dot;
      }
      double m = -std::numeric_limits<double>::infinity();
      for (size_t j = 0; j < n; ++j) m = std::max(m, l[j]);
      if (sink) m = std::max(m, sink[h]);
      double z = 0.0;
      for (size_t j = 0; j < n; ++j) z += std::exp(l[j] - m);
      if (sink) z += std::exp(sink[h] - m);
      for (size_t j = 0; j < n; ++j) p[j] = std::exp(l[j] - m) / z;
      const double ps = sink ? std::exp(sink[h] - m) / z : 0.0;
      for (size_t j = 0; j < n; ++j)
        for (int c = 0; c < kDV; ++c) ol[c] += p[j] * kv[sel[j] * kDL + c];
      for (int d = 0; d < kDO; ++d)
        for (int c = 0; c < kDV; ++c) o[d] += ol[c] * Wh[c * kDO + d];
      const double* dorow = dout + (r * H + h) * static_cast<int64_t>(kDO);
      if (gate_per_dim) {
        for (int d = 0; d < kDO; ++d) {
          const int64_t at = (r * H + h) * static_cast<int64_t>(kDO) + d;
          const double sg = 1.0 / (1.0 + std::exp(-gate_rows[at]));
          dgate[at] = sg * (1.0 - sg) * dorow[d] * o[d];
          dov[d] = sg * dorow[d];
        }
      } else {
        const double sg = 1.0 / (1.0 + std::exp(-gate_rows[r * H + h]));
        double dgo = 0.0;
        for (int d = 0; d < kDO; ++d) dgo += dorow[d] * o[d];
        dgate[r * H + h] = sg * (1.0 - sg) * dgo;
        for (int d = 0; d < kDO; ++d) dov[d] = sg * dorow[d];
      }
      double* dWh = dW + static_cast<int64_t>(h) * kDV * kDO;
      for (int c = 0; c < kDV; ++c)
        for (int d = 0; d < kDO; ++d) {
          dWh[c * kDO + d] += ol[c] * dov[d];
          dol[c] += Wh[c * kDO + d] * dov[d];
        }
      double D = 0.0;
      for (size_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int c = 0; c < kDV; ++c) acc += dol[c] * kv[sel[j] * kDL + c];
        dp[j] = acc;
        D += p[j] * acc;
      }
      if (sink) dsink[h] += -ps * D;  // one iteration per head: no other thread writes dsink[h]
      double* dqh = dq + (r * H + h) * static_cast<int64_t>(kDL);
      for (int i = 0; i < kDL; ++i) dqh[i] = 0.0;
      for (size_t j = 0; j < n; ++j) {
        const double dl = p[j] * (dp[j] - D);
        double* dk = dkv_h.data() + (static_cast<size_t>(h) * n + j) * kDL;
        for (int i = 0; i < kDL; ++i) {
          dqh[i] += scale * dl * kv[sel[j] * kDL + i];
          dk[i] += scale * dl * qh[i];
        }
        for (int c = 0; c < kDV; ++c) dk[c] += p[j] * dol[c];
      }
    }
    for (int32_t h = 0; h < H; ++h)
      for (size_t j = 0; j < n; ++j)
        for (int i = 0; i < kDL; ++i) dkv[sel[j] * kDL + i] += dkv_h[(static_cast<size_t>(h) * n + j) * kDL + i];
  }
}

// The per-head gate without a sink (the backward the GPU path computes by default).
void oracle_sparse_mla_bwd(int64_t n_rows, const double* q_rows, const double* kv, int64_t T, const int32_t* idx,
                           int32_t k, const double* W_UV, const double* gate_rows, int32_t H, double scale,
                           const double* dout, double* dq, double* dkv, double* dW, double* dgate) {
  oracle_sparse_mla_bwd_variant(n_rows, q_rows, kv, T, idx, k, W_UV, gate_rows, H, scale, 0, nullptr, dout, dq, dkv,
                                dW, dgate, nullptr);
}

// Dense-mask reference ([KC] Implementation Limits 1st bullet: the eager/sdpa paths are
// dense-mask references). Written independently of oracle_sparse_mla: for each listed row the
// logits of all T keys are formed and keys outside the causal window of the row's own document
// are masked to -inf before a full-length softmax. Same gate and up-projection definition.
void oracle_dense_causal(int64_t n_rows, const int64_t* rows, const uint16_t* q_rows, const uint16_t* kv, int64_t T,
                         const int32_t* cu, int32_t n_docs, const uint16_t* W_UV, const uint16_t* gate_rows, int32_t H,
                         double scale, double* out_f64) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = rows[r];
    const int64_t b = doc_begin(cu, n_docs, t);
    std::vector<double> logits(static_cast<size_t>(T)), attn(kDV);
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t* qh = q_rows + (r * H + h) * static_cast<int64_t>(kDL);
      for (int64_t s = 0; s < T; ++s) {
        if (s < b || s > t) {
          logits[s] = -std::numeric_limits<double>::infinity();
          continue;
        }
        double dot = 0.0;
        for (int i = 0; i < kDL; ++i) dot += static_cast<double>(bf16_bits_to_float(qh[i])) * bf16_bits_to_float(kv[s * kDL + i]);
        logits[s] = dot * scale;
      }
      const double mx = *std::max_element(logits.begin(), logits.end());
      double den = 0.0;
      for (int64_t s = 0; s < T; ++s) den += std::exp(logits[s] - mx);
      for (int c = 0; c < kDV; ++c) {
        double acc = 0.0;
        for (int64_t s = b; s <= t; ++s) acc += std::exp(logits[s] - mx) / den * bf16_bits_to_float(kv[s * kDL + c]);
        attn[c] = acc;
      }
      const double gl = bf16_bits_to_float(gate_rows[r * H + h]);
      for (int d = 0; d < kDO; ++d) {
        double o = 0.0;
        for (int c = 0; c < kDV; ++c) o += attn[c] * bf16_bits_to_float(W_UV[(static_cast<int64_t>(h) * kDV + c) * kDO + d]);
        out_f64[(r * H + h) * static_cast<int64_t>(kDO) + d] = o / (1.0 + std::exp(-gl));
      }
    }
  }
}

}  // extern "C"

// Host side of the C ABI declared in include/dsa.h: argument checks (pure host code, no HIP
// call), workspace layout and the launch sequence of each entry point.
#include "dsa.h"

#include <algorithm>
#include <mutex>
#include <vector>

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "dsa_kernels.h"

namespace {

constexpr int kMaxTopk = dsa::kIdxMaxTopk;  // summary of the model-coverage page: at most 2,048 keys
constexpr int64_t kMlaChunkRows = 2048;  // rows per attention/up-projection pass: one chunk's o_lat (201 MB at 96 heads) stays in the Infinity Cache for the up-projection
constexpr int64_t kIdxPairedBelow = 4096;  // rows with a selection under which indexer blocks pair long and short rows
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t rows_of(const dsa_shape* s) { return (s->q_end == 0 ? s->T : s->q_end) - s->q_begin; }

// Workspace regions, each from a 256-byte-aligned offset:
//   LNk    [T + kIdxKeyPad, d_I] bf16   key LayerNorm output (the padding rows are staged, never scored)
//   flags  [kIdxSlots] int32           candidate-slot claims of the indexer's workgroups
//   cand   [kIdxSlots, slot words]     candidate lists (score keys, token indices) of the rows in flight
//   LNk8   [T + kIdxKeyPad, d_I] u8    FP8 indexer: E4M3 codes of LNk, and sk [T + kIdxKeyPad] f32
//   q8     [rows, H_I, d_I] u8         FP8 indexer: E4M3 codes of q_I, and sq [rows, H_I] f32
//   o_lat  [chunk rows, H, 512] bf16   latent attention output of one row chunk
struct Layout {
  size_t lnk_off, lnk_bytes, flags_off, cand_off, cand_bytes, lnk8_off, sk_off, q8_off, sq_off, olat_off, olat_bytes,
      total;
  int64_t chunk_rows;
};

Layout layout_of(const dsa_shape* s) {
  Layout L{};
  L.lnk_off = 0;
  L.lnk_bytes = align_up(static_cast<size_t>(s->T + dsa::kIdxKeyPad) * s->d_I * 2);
  L.flags_off = L.lnk_off + L.lnk_bytes;
  L.cand_off = L.flags_off + align_up(static_cast<size_t>(dsa::kIdxSlots) * 4);
  L.cand_bytes = align_up(static_cast<size_t>(dsa::kIdxSlots) * dsa::kIdxSlotWords * 4);
  const int64_t rows = rows_of(s);
  const size_t keys_pad = static_cast<size_t>(s->T + dsa::kIdxKeyPad);
  L.lnk8_off = L.cand_off + L.cand_bytes;
  L.sk_off = L.lnk8_off + align_up(keys_pad * s->d_I);
  L.q8_off = L.sk_off + align_up(keys_pad * 4);
  L.sq_off = L.q8_off + align_up(static_cast<size_t>(rows) * s->H_I * s->d_I);
  L.chunk_rows = rows < kMlaChunkRows ? rows : kMlaChunkRows;
  L.olat_off = L.sq_off + align_up(static_cast<size_t>(rows) * s->H_I * 4);
  L.olat_bytes = align_up(static_cast<size_t>(L.chunk_rows) * s->H * 512 * 2);
  L.total = L.olat_off + L.olat_bytes;
  return L;
}

dsa_status check_ws(const dsa_shape* s, const void* ws, size_t ws_bytes) {
  if (ws == nullptr || ws_bytes < layout_of(s).total) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status st) {
  switch (st) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    case DSA_ERR_TOO_LARGE:
      return "shape exceeds the fixed scratch of the allocation-free entry point (T <= 131072, at most 64 documents)";
  }
  return "unknown status";
}

dsa_status dsa_check_shape(const dsa_shape* s) {
  if (s == nullptr) return DSA_ERR_INVALID_ARG;
  if (s->T < 1 || s->n_docs < 1 || s->n_docs > s->T) return DSA_ERR_INVALID_ARG;
  if (s->n_docs > 1 && (s->cu_seqlens_host == nullptr || s->cu_seqlens_dev == nullptr)) return DSA_ERR_INVALID_ARG;
  if (s->cu_seqlens_host != nullptr) {
    const int32_t* cu = s->cu_seqlens_host;
    if (cu[0] != 0 || cu[s->n_docs] != s->T) return DSA_ERR_INVALID_ARG;
    for (int32_t d = 0; d < s->n_docs; ++d)
      if (cu[d + 1] <= cu[d]) return DSA_ERR_INVALID_ARG;
  }
  const int32_t q_end = s->q_end == 0 ? s->T : s->q_end;
  if (s->q_begin < 0 || q_end > s->T || s->q_begin >= q_end) return DSA_ERR_INVALID_ARG;
  if (s->topk < 1) return DSA_ERR_INVALID_ARG;
  if (!(s->ln_eps > 0.0f) || !std::isfinite(s->ln_eps)) return DSA_ERR_INVALID_ARG;
  if (!(s->softmax_scale > 0.0f) || !std::isfinite(s->softmax_scale)) return DSA_ERR_INVALID_ARG;
  if (s->topk > kMaxTopk) return DSA_ERR_UNSUPPORTED;
  const bool idx_ok = (s->H_I == 64 && s->d_I == 128) || (s->H_I == 4 && s->d_I == 64);
  if (!idx_ok) return DSA_ERR_UNSUPPORTED;
  if (s->H != 96 && s->H != 16) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

size_t dsa_workspace_size(const dsa_shape* s) {
  if (dsa_check_shape(s) != DSA_OK) return 0;
  return layout_of(s).total;
}

// One document's rows that need a selection: local rows [r0, r0 + m), document start token b.
struct Seg {
  int r0, m, b, order;
};

// Steps 1-3 into topk_idx. ws holds the LNk, flag and candidate regions of layout_of(s); segs is
// caller storage for at least s->n_docs entries (no allocation happens here).
static dsa_status run_index(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I, const float* gamma,
                            const float* beta, const uint16_t* w, int32_t* topk_idx, void* ws, Seg* segs,
                            hipStream_t st, bool fp8 = false, bool fused_ln = false) {
  const auto L = layout_of(s);
  uint16_t* lnk = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + L.lnk_off);
  dsa::IndexArgs a{};
  a.q_I = q_I;
  a.w = w;
  a.LNk = lnk;
  a.topk_idx = topk_idx;
  a.cu = s->n_docs > 1 ? s->cu_seqlens_dev : nullptr;
  a.n_docs = s->n_docs;
  a.T = s->T;
  a.row0 = s->q_begin;
  a.nrows = rows_of(s);
  a.k = s->topk;
  // Candidate lists live in kIdxSlots slots, one per workgroup in flight; every launch
  // frees the slots it claimed, and the prologue marks them all free first.
  a.slot_flags = reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + L.flags_off);
  a.cand = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + L.cand_off);
  a.n_slots = dsa::kIdxSlots;
  a.k_raw = k_I;
  a.ln_gamma = gamma;
  a.ln_beta = beta;
  a.ln_eps = static_cast<double>(s->ln_eps);
  if (dsa::launch_index_prologue(k_I, gamma, beta, static_cast<double>(s->ln_eps), s->d_I, lnk, a, st, !fused_ln) !=
      hipSuccess)
    return DSA_ERR_LAUNCH;
  if (fp8) {
    // E4M3 codes and scales of LNk (the T key rows) and of q_I (every head row of the query rows)
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint8_t* lnk8 = base + L.lnk8_off;
    float* sk = reinterpret_cast<float*>(base + L.sk_off);
    uint8_t* q8 = base + L.q8_off;
    float* sq = reinterpret_cast<float*>(base + L.sq_off);
    a.LNk8 = lnk8;
    a.sk = sk;
    a.q8 = q8;
    a.sq = sq;
    if (dsa::launch_quantize_fp8(lnk, s->T, lnk8, sk, q_I, static_cast<int64_t>(a.nrows) * s->H_I, q8, sq, st) !=
        hipSuccess)
      return DSA_ERR_LAUNCH;
  }
  // Rows with more than k causal keys, one segment per document. With few such rows per CU,
  // blocks pair long and short rows of a document so that every block carries about the same
  // work; otherwise blocks take consecutive rows, longest first.
  int nseg = 0;
  int64_t nsel = 0;
  for (int d = 0; d < s->n_docs; ++d) {
    const int64_t b0 = s->cu_seqlens_host ? s->cu_seqlens_host[d] : 0;
    const int64_t b1 = s->cu_seqlens_host ? s->cu_seqlens_host[d + 1] : s->T;
    const int64_t lo = std::max<int64_t>(b0 + s->topk, s->q_begin) - s->q_begin;
    const int64_t hi = std::min<int64_t>(b1, s->q_begin + a.nrows) - s->q_begin;
    if (hi > lo) {
      segs[nseg] = {static_cast<int>(lo), static_cast<int>(hi - lo), static_cast<int>(b0), nseg};
      ++nseg;
      nsel += hi - lo;
    }
  }
  a.paired = nsel < kIdxPairedBelow ? 1 : 0;
  // longest rows first (the longest row of a segment is its last), then document order
  std::sort(segs, segs + nseg, [](const Seg& x, const Seg& y) {
    const int lx = x.r0 + x.m - x.b, ly = y.r0 + y.m - y.b;
    return lx != ly ? lx > ly : x.order < y.order;
  });
  for (int i = 0; i < nseg;) {
    // one launch per kIdxMaxSeg documents
    a.nseg = 0;
    a.seg_blk0[0] = 0;
    for (; i < nseg && a.nseg < dsa::kIdxMaxSeg; ++i, ++a.nseg) {
      a.seg_r0[a.nseg] = segs[i].r0;
      a.seg_m[a.nseg] = segs[i].m;
      a.seg_b[a.nseg] = segs[i].b;
      a.seg_blk0[a.nseg + 1] = a.seg_blk0[a.nseg] + dsa::index_blocks(segs[i].m, a.paired);
    }
    const hipError_t e = dsa::launch_index_topk(a, s->H_I, s->d_I, fp8, st, fused_ln);
    if (e == hipErrorInvalidConfiguration) return DSA_ERR_UNSUPPORTED;  // more resident workgroups than slots
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

static dsa_status launch_attention(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q, const uint16_t* kv,
                                   const int32_t* idx, uint16_t* olat, float* lse, int64_t c0, int64_t n, hipStream_t st) {
  dsa::MlaArgs m{};
  m.q = q;
  m.kv = kv;
  m.idx = idx;
  m.o_lat = olat;
  m.lse = lse;
  m.sink = v ? v->sink : nullptr;
  m.cu = s->n_docs > 1 ? s->cu_seqlens_dev : nullptr;
  m.n_docs = s->n_docs;
  m.T = s->T;
  m.row0 = s->q_begin;
  m.chunk_r0 = static_cast<int>(c0);
  m.chunk_rows = static_cast<int>(n);
  m.k = s->topk;
  m.H = s->H;
  m.scale_log2 = s->softmax_scale * 1.4426950408889634f;
  return dsa::launch_sparse_mla(m, st) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

static dsa_status launch_up(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* olat, const uint16_t* W_UV,
                            const uint16_t* gate, uint16_t* out, int64_t c0, int64_t n, hipStream_t st) {
  dsa::UpArgs u{};
  u.gate_per_dim = v && v->gate_per_dim ? 1 : 0;
  u.o_lat = olat;
  u.W_UV = W_UV;
  u.gate = gate;
  u.out = out;
  u.chunk_r0 = static_cast<int>(c0);
  u.chunk_rows = static_cast<int>(n);
  u.H = s->H;
  return dsa::launch_up_gate(u, st) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

static dsa_status run_mla(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q, const uint16_t* kv,
                          const int32_t* idx, const uint16_t* W_UV, const uint16_t* gate, uint16_t* out, float* lse,
                          void* ws, hipStream_t st) {
  const auto L = layout_of(s);
  uint16_t* olat = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(ws) + L.olat_off);
  const int64_t rows = rows_of(s);
  for (int64_t c0 = 0; c0 < rows; c0 += L.chunk_rows) {
    const int64_t n = (rows - c0) < L.chunk_rows ? (rows - c0) : L.chunk_rows;
    dsa_status r = launch_attention(s, v, q, kv, idx, olat, lse, c0, n, st);
    if (r != DSA_OK) return r;
    if ((r = launch_up(s, v, olat, W_UV, gate, out, c0, n, st)) != DSA_OK) return r;
  }
  return DSA_OK;
}

dsa_status dsa_index_topk(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I, const float* ln_gamma,
                          const float* ln_beta, const uint16_t* w, int32_t* topk_idx, void* ws, size_t ws_bytes,
                          void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q_I || !k_I || !w || !topk_idx) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_I, 16) || !aligned(k_I, 2) || !aligned(w, 2) || !aligned(topk_idx, 16) || !aligned(ln_gamma, 4) ||
      !aligned(ln_beta, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != DSA_OK) return st;
  std::vector<Seg> segs(static_cast<size_t>(s->n_docs));
  return run_index(s, q_I, k_I, ln_gamma, ln_beta, w, topk_idx, ws, segs.data(), static_cast<hipStream_t>(stream));
}

// Checks of the attention variant: an elementwise gate is read with 16-byte copies; the sink is
// float32.
static dsa_status check_variant(const dsa_mla_variant* v, const uint16_t* gate) {
  if (v == nullptr) return DSA_OK;
  if (v->gate_per_dim != 0 && v->gate_per_dim != 1) return DSA_ERR_INVALID_ARG;
  if (v->gate_per_dim && !aligned(gate, 16)) return DSA_ERR_INVALID_ARG;
  if (!aligned(v->sink, 4)) return DSA_ERR_INVALID_ARG;
  return DSA_OK;
}

dsa_status dsa_index_topk_fp8(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I, const float* ln_gamma,
                              const float* ln_beta, const uint16_t* w, int32_t* topk_idx, void* ws, size_t ws_bytes,
                              void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!(s->H_I == 64 && s->d_I == 128)) return DSA_ERR_UNSUPPORTED;
  if (!q_I || !k_I || !w || !topk_idx) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_I, 16) || !aligned(k_I, 2) || !aligned(w, 2) || !aligned(topk_idx, 16) || !aligned(ln_gamma, 4) ||
      !aligned(ln_beta, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != DSA_OK) return st;
  std::vector<Seg> segs(static_cast<size_t>(s->n_docs));
  return run_index(s, q_I, k_I, ln_gamma, ln_beta, w, topk_idx, ws, segs.data(), static_cast<hipStream_t>(stream),
                   true);
}

dsa_status dsa_index_topk_fused_ln(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I, const float* ln_gamma,
                                   const float* ln_beta, const uint16_t* w, int32_t* topk_idx, void* ws, size_t ws_bytes,
                                   void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!(s->H_I == 64 && s->d_I == 128)) return DSA_ERR_UNSUPPORTED;
  if (!q_I || !k_I || !w || !topk_idx) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_I, 16) || !aligned(k_I, 16) || !aligned(w, 2) || !aligned(topk_idx, 16) || !aligned(ln_gamma, 4) ||
      !aligned(ln_beta, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes)) != DSA_OK) return st;
  std::vector<Seg> segs(static_cast<size_t>(s->n_docs));
  return run_index(s, q_I, k_I, ln_gamma, ln_beta, w, topk_idx, ws, segs.data(), static_cast<hipStream_t>(stream),
                   false, true);
}

dsa_status dsa_q_absorb(const dsa_shape* s, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* W_UK,
                        uint16_t* q, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q_nope || !q_pe || !W_UK || !q) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(W_UK, 16) || !aligned(q, 16)) return DSA_ERR_INVALID_ARG;
  dsa::AbsorbArgs a{q_nope, q_pe, W_UK, q, rows_of(s), s->H, 576};
  return dsa::launch_q_absorb(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

dsa_status dsa_o_proj(const dsa_shape* s, const uint16_t* x, const uint16_t* W_o, int32_t d_model, uint16_t* y,
                      void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!x || !W_o || !y) return DSA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(W_o, 16) || !aligned(y, 16)) return DSA_ERR_INVALID_ARG;
  if (d_model < 256 || d_model % 256 != 0) return DSA_ERR_UNSUPPORTED;
  dsa::GemmArgs g{x, W_o, y, rows_of(s), d_model, s->H * 128};
  return dsa::launch_gemm_nt(g, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

// Backward workspace: the forward's regions (o_lat is recomputed into its region), then per row chunk
// of at most kBwdChunkRows rows
//   do      [chunk rows, H, 128] bf16        sigma(g) dout
//   do_lat  [chunk rows, H, 512] bf16        do W_UV[h]^T
//   delta   [chunk rows, H] f32              sum dout * out
//   g       [chunk rows, g_stride, 2H] bf16  dS' and P of every selected key, for the dkv contraction
//   contrib [3][chunk rows * k][192] bf16     each (row, selected key)'s dkv contribution, by 192-dim group
//   count [T] and start [T + 1] int32, list [chunk rows * k] int32: the pairs grouped by key
//   bsum    [ceil(T / 4096)] int32          the key scan's tile sums
//   sterm   [chunk rows, H] f32             with a sink: each (row, head)'s term of the sink's gradient
constexpr int64_t kBwdChunkRows = 2048;  // bounds contrib (4.8 GB at k = 2048)

struct BwdLayout {
  size_t do_off, dolat_off, delta_off, g_off, contrib_off, count_off, start_off, list_off, bsum_off,
      sterm_off, total;
  int g_stride;
  int64_t chunk_rows;
};

static BwdLayout bwd_layout_of(const dsa_shape* s) {
  const Layout L = layout_of(s);
  BwdLayout B{};
  const int64_t rows = rows_of(s);
  B.chunk_rows = rows < kBwdChunkRows ? rows : kBwdChunkRows;
  const size_t crows = static_cast<size_t>(B.chunk_rows);
  const size_t cr = crows * s->H;
  B.g_stride = (s->topk + 31) / 32 * 32;
  B.do_off = L.total;
  B.dolat_off = B.do_off + align_up(cr * 128 * 2);
  B.delta_off = B.dolat_off + align_up(cr * 512 * 2);
  B.g_off = B.delta_off + align_up(cr * 4);
  B.contrib_off = B.g_off + align_up(crows * B.g_stride * 2 * s->H * 2);
  B.count_off = B.contrib_off + align_up(crows * s->topk * 576 * 2);
  B.start_off = B.count_off + align_up(static_cast<size_t>(s->T) * 4);
  B.list_off = B.start_off + align_up((static_cast<size_t>(s->T) + 1) * 4);
  B.bsum_off = B.list_off + align_up(crows * s->topk * 4);
  B.sterm_off = B.bsum_off + align_up((static_cast<size_t>(s->T) + dsa::kPairScanTile - 1) / dsa::kPairScanTile * 4);
  B.total = B.sterm_off + align_up(cr * 4);
  return B;
}

size_t dsa_bwd_workspace_size(const dsa_shape* s) {
  if (dsa_check_shape(s) != DSA_OK) return 0;
  return bwd_layout_of(s).total;
}

static dsa_status run_bwd(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q, const uint16_t* kv,
                          const int32_t* topk_idx, const uint16_t* W_UV, const uint16_t* gate, const uint16_t* out,
                          const float* lse, const uint16_t* olat_saved, const uint16_t* dout, float* dq, float* dkv,
                          float* dW_UV, float* dgate, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (s->H != 96) return DSA_ERR_UNSUPPORTED;
  if (!q || !kv || !topk_idx || !W_UV || !gate || !out || !lse || !dout || !dq || !dkv || !dW_UV || !dgate)
    return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(topk_idx, 4) || !aligned(W_UV, 16) || !aligned(gate, 2) ||
      !aligned(out, 16) || !aligned(lse, 4) || !aligned(dout, 16) || !aligned(dq, 4) || !aligned(dkv, 4) ||
      !aligned(dW_UV, 4) || !aligned(dgate, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_variant(v, gate)) != DSA_OK) return st;
  const bool per_dim = v && v->gate_per_dim;
  const float* sink = v ? v->sink : nullptr;
  if (per_dim && !aligned(dgate, 16)) return DSA_ERR_INVALID_ARG;
  if ((sink != nullptr) != (dsink != nullptr) || (dsink && !aligned(dsink, 4))) return DSA_ERR_INVALID_ARG;
  if (!aligned(olat_saved, 16)) return DSA_ERR_INVALID_ARG;
  const BwdLayout B = bwd_layout_of(s);
  if (ws == nullptr || ws_bytes < B.total) return DSA_ERR_WORKSPACE;
  if (!aligned(ws, kWsAlign)) return DSA_ERR_INVALID_ARG;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const Layout L = layout_of(s);
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint16_t* olat = reinterpret_cast<uint16_t*>(base + L.olat_off);
  uint16_t* d_o = reinterpret_cast<uint16_t*>(base + B.do_off);
  uint16_t* dolat = reinterpret_cast<uint16_t*>(base + B.dolat_off);
  float* delta = reinterpret_cast<float*>(base + B.delta_off);
  uint16_t* g = reinterpret_cast<uint16_t*>(base + B.g_off);
  uint16_t* contrib = reinterpret_cast<uint16_t*>(base + B.contrib_off);
  int* count = reinterpret_cast<int*>(base + B.count_off);
  int* start = reinterpret_cast<int*>(base + B.start_off);
  int* list = reinterpret_cast<int*>(base + B.list_off);
  int* bsum = reinterpret_cast<int*>(base + B.bsum_off);
  float* sterm = reinterpret_cast<float*>(base + B.sterm_off);
  if (dsa::launch_fill_zero(dkv, static_cast<int64_t>(s->T) * 576, hs) != hipSuccess ||
      dsa::launch_fill_zero(dW_UV, static_cast<int64_t>(s->H) * 512 * 128, hs) != hipSuccess ||
      (dsink && dsa::launch_fill_zero(dsink, s->H, hs) != hipSuccess))
    return DSA_ERR_LAUNCH;
  const int64_t rows = rows_of(s);
  for (int64_t c0 = 0; c0 < rows; c0 += B.chunk_rows) {
    const int n = static_cast<int>(std::min<int64_t>(B.chunk_rows, rows - c0));
    dsa::BwdPrepArgs p{dout, out, gate, d_o, delta, dgate, n, s->H, static_cast<int>(c0), per_dim ? 1 : 0, sink, lse,
                       sterm};
    if (dsa::launch_bwd_prep(p, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    if (sink) {
      dsa::SinkSumArgs ss{sterm, dsink, n, s->H};
      if (dsa::launch_sink_sum(ss, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    }
    dsa::AbsorbArgs ab{d_o, nullptr, W_UV, dolat, n, s->H, 512};  // do_lat = do W_UV[h]^T
    if (dsa::launch_q_absorb(ab, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    dsa::BwdArgs b{};
    b.q = q;
    b.kv = kv;
    b.idx = topk_idx;
    b.lse = lse;
    b.delta = delta;
    b.do_lat = dolat;
    b.dq = dq;
    b.g = g;
    b.g_stride = B.g_stride;
    b.cu = s->n_docs > 1 ? s->cu_seqlens_dev : nullptr;
    b.n_docs = s->n_docs;
    b.T = s->T;
    b.row0 = s->q_begin;
    b.chunk_r0 = static_cast<int>(c0);
    b.chunk_rows = n;
    b.k = s->topk;
    b.H = s->H;
    b.scale = s->softmax_scale;
    if (dsa::launch_sparse_mla_bwd(b, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    // the chunk's pairs sorted by key first, so that k_dkv stores each key's contributions together
    dsa::DkvListArgs dl{topk_idx, b.cu, s->n_docs, s->T, s->q_begin, static_cast<int>(c0), n, s->topk,
                        count, start, bsum, list, contrib, dkv};
    if (dsa::launch_pairs_sort(dl, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    dsa::DkvArgs dk{g, q, dolat, list, contrib, b.cu, s->n_docs, s->T, s->q_begin, static_cast<int>(c0), n,
                    s->topk, B.g_stride};
    if (dsa::launch_dkv(dk, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    if (dsa::launch_dkv_sum(dl, hs) != hipSuccess) return DSA_ERR_LAUNCH;
    // o_lat of the chunk for dW_UV: the caller's saved rows, or the forward's attention kernel again
    // (with the sink if any)
    const uint16_t* olat_c = olat;
    if (olat_saved != nullptr) olat_c = olat_saved + c0 * s->H * 512;
    else if ((st = launch_attention(s, v, q, kv, topk_idx, olat, nullptr, c0, n, hs)) != DSA_OK) return st;
    dsa::DwArgs dw{olat_c, d_o, dW_UV, n, s->H};
    if (dsa::launch_dwuv(dw, hs) != hipSuccess) return DSA_ERR_LAUNCH;
  }
  return DSA_OK;
}

dsa_status dsa_sparse_mla_bwd(const dsa_shape* s, const uint16_t* q, const uint16_t* kv, const int32_t* topk_idx,
                              const uint16_t* W_UV, const uint16_t* gate, const uint16_t* out, const float* lse,
                              const uint16_t* dout, float* dq, float* dkv, float* dW_UV, float* dgate, void* ws,
                              size_t ws_bytes, void* stream) {
  return run_bwd(s, nullptr, q, kv, topk_idx, W_UV, gate, out, lse, nullptr, dout, dq, dkv, dW_UV, dgate, nullptr, ws,
                 ws_bytes, stream);
}

dsa_status dsa_sparse_mla_bwd_ex(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q, const uint16_t* kv,
                                 const int32_t* topk_idx, const uint16_t* W_UV, const uint16_t* gate,
                                 const uint16_t* out, const float* lse, const uint16_t* dout, float* dq, float* dkv,
                                 float* dW_UV, float* dgate, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  return run_bwd(s, v, q, kv, topk_idx, W_UV, gate, out, lse, nullptr, dout, dq, dkv, dW_UV, dgate, dsink, ws, ws_bytes,
                 stream);
}

dsa_status dsa_sparse_mla_bwd_saved(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q,
                                    const uint16_t* kv, const int32_t* topk_idx, const uint16_t* W_UV,
                                    const uint16_t* gate, const uint16_t* out, const float* lse, const uint16_t* o_lat,
                                    const uint16_t* dout, float* dq, float* dkv, float* dW_UV, float* dgate,
                                    float* dsink, void* ws, size_t ws_bytes, void* stream) {
  if (o_lat == nullptr) return DSA_ERR_INVALID_ARG;
  return run_bwd(s, v, q, kv, topk_idx, W_UV, gate, out, lse, o_lat, dout, dq, dkv, dW_UV, dgate, dsink, ws, ws_bytes,
                 stream);
}

dsa_status dsa_quantize_fp8(int64_t n_rows, const uint16_t* x, uint8_t* q8, float* scale, void* stream) {
  if (n_rows < 0 || (n_rows > 0 && (!x || !q8 || !scale))) return DSA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(q8, 16) || !aligned(scale, 4)) return DSA_ERR_INVALID_ARG;
  return dsa::launch_quantize_fp8(x, n_rows, q8, scale, nullptr, 0, nullptr, nullptr, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? DSA_OK
             : DSA_ERR_LAUNCH;
}

dsa_status dsa_sparse_mla_fwd_ex(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q, const uint16_t* kv,
                                 const int32_t* topk_idx, const uint16_t* W_UV, const uint16_t* gate, uint16_t* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q || !kv || !topk_idx || !W_UV || !gate || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(W_UV, 16) || !aligned(topk_idx, 4) || !aligned(gate, 2) ||
      !aligned(out, 16) || !aligned(lse, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_variant(v, gate)) != DSA_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != DSA_OK) return st;
  return run_mla(s, v, q, kv, topk_idx, W_UV, gate, out, lse, ws, static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_mla_fwd(const dsa_shape* s, const uint16_t* q, const uint16_t* kv, const int32_t* topk_idx,
                              const uint16_t* W_UV, const uint16_t* gate, uint16_t* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  return dsa_sparse_mla_fwd_ex(s, nullptr, q, kv, topk_idx, W_UV, gate, out, lse, ws, ws_bytes, stream);
}

dsa_status dsa_sparse_attention_latent_ex(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q,
                                          const uint16_t* kv, const int32_t* topk_idx, uint16_t* o_lat, float* lse,
                                          void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q || !kv || !topk_idx || !o_lat) return DSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(topk_idx, 4) || !aligned(o_lat, 16) || !aligned(lse, 4))
    return DSA_ERR_INVALID_ARG;
  if (v && ((v->gate_per_dim != 0 && v->gate_per_dim != 1) || !aligned(v->sink, 4))) return DSA_ERR_INVALID_ARG;
  return launch_attention(s, v, q, kv, topk_idx, o_lat, lse, 0, rows_of(s), static_cast<hipStream_t>(stream));
}

dsa_status dsa_sparse_attention_latent(const dsa_shape* s, const uint16_t* q, const uint16_t* kv,
                                       const int32_t* topk_idx, uint16_t* o_lat, float* lse, void* stream) {
  return dsa_sparse_attention_latent_ex(s, nullptr, q, kv, topk_idx, o_lat, lse, stream);
}

dsa_status dsa_up_gate(const dsa_shape* s, const uint16_t* o_lat, const uint16_t* W_UV, const uint16_t* gate,
                       uint16_t* out, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!o_lat || !W_UV || !gate || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(o_lat, 16) || !aligned(W_UV, 16) || !aligned(gate, 2) || !aligned(out, 16)) return DSA_ERR_INVALID_ARG;
  return launch_up(s, nullptr, o_lat, W_UV, gate, out, 0, rows_of(s), static_cast<hipStream_t>(stream));
}

dsa_status dsa_fused_fwd_ex(const dsa_shape* s, const dsa_mla_variant* v, const uint16_t* q_I, const uint16_t* k_I,
                            const float* ln_gamma, const float* ln_beta, const uint16_t* w, const uint16_t* q,
                            const uint16_t* kv, const uint16_t* W_UV, const uint16_t* gate, int32_t* topk_idx,
                            uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q_I || !k_I || !w || !q || !kv || !W_UV || !gate || !topk_idx || !out) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_I, 16) || !aligned(k_I, 2) || !aligned(w, 2) || !aligned(ln_gamma, 4) || !aligned(ln_beta, 4) ||
      !aligned(q, 16) || !aligned(kv, 16) || !aligned(W_UV, 16) || !aligned(topk_idx, 16) || !aligned(gate, 2) ||
      !aligned(out, 16) || !aligned(lse, 4))
    return DSA_ERR_INVALID_ARG;
  if ((st = check_variant(v, gate)) != DSA_OK) return st;
  if ((st = check_ws(s, ws, ws_bytes)) != DSA_OK) return st;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  std::vector<Seg> segs(static_cast<size_t>(s->n_docs));
  if ((st = run_index(s, q_I, k_I, ln_gamma, ln_beta, w, topk_idx, ws, segs.data(), hs)) != DSA_OK) return st;
  return run_mla(s, v, q, kv, topk_idx, W_UV, gate, out, lse, ws, hs);
}

dsa_status dsa_fused_fwd(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I, const float* ln_gamma,
                         const float* ln_beta, const uint16_t* w, const uint16_t* q, const uint16_t* kv,
                         const uint16_t* W_UV, const uint16_t* gate, int32_t* topk_idx, uint16_t* out, float* lse,
                         void* ws, size_t ws_bytes, void* stream) {
  return dsa_fused_fwd_ex(s, nullptr, q_I, k_I, ln_gamma, ln_beta, w, q, kv, W_UV, gate, topk_idx, out, lse, ws,
                          ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Allocation-free indexer entry point, for callers that cannot allocate device memory. Its scratch
// (LNk, candidate-slot flags, candidate slots: the first three workspace regions of the largest
// shape it accepts) is a file-scope device array that each GPU holds from the library's first use
// on it until the process ends. Host code never passes the array's name to a kernel: that is a
// host-side stand-in. The device address comes from hipGetSymbolAddress, once per device.
namespace {

constexpr int32_t kNoAllocMaxT = 131072;
constexpr int32_t kNoAllocMaxDocs = dsa::kIdxMaxSeg;
constexpr size_t align_c(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }
constexpr size_t kNoAllocBytes = align_c(static_cast<size_t>(kNoAllocMaxT + dsa::kIdxKeyPad) * 128 * 2) +
                                 align_c(static_cast<size_t>(dsa::kIdxSlots) * 4) +
                                 align_c(static_cast<size_t>(dsa::kIdxSlots) * dsa::kIdxSlotWords * 4);
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

// Device address of this GPU's copy of scratch (the current device), looked up on the first call
// on each device. Returns nullptr on failure.
static void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

extern "C" dsa_status dsa_index_topk_noalloc(const dsa_shape* s, const uint16_t* q_I, const uint16_t* k_I,
                                             const float* ln_gamma, const float* ln_beta, const uint16_t* w,
                                             int32_t* topk_idx, void* stream) {
  dsa_status st = dsa_check_shape(s);
  if (st != DSA_OK) return st;
  if (!q_I || !k_I || !w || !topk_idx) return DSA_ERR_INVALID_ARG;
  if (!aligned(q_I, 16) || !aligned(k_I, 2) || !aligned(w, 2) || !aligned(topk_idx, 16) || !aligned(ln_gamma, 4) ||
      !aligned(ln_beta, 4))
    return DSA_ERR_INVALID_ARG;
  if (s->T > kNoAllocMaxT || s->n_docs > kNoAllocMaxDocs) return DSA_ERR_TOO_LARGE;
  const Layout L = layout_of(s);
  if (L.cand_off + L.cand_bytes > kNoAllocBytes) return DSA_ERR_TOO_LARGE;
  void* ws = scratch_address();
  if (ws == nullptr) return DSA_ERR_LAUNCH;
  Seg segs[kNoAllocMaxDocs];
  return run_index(s, q_I, k_I, ln_gamma, ln_beta, w, topk_idx, ws, segs, static_cast<hipStream_t>(stream));
}

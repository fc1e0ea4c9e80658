// Key LayerNorm prologue and the indexer + streaming top-k kernel (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, summary and Implementation Limits
// bullets 2-4; archdiff "Kimi K3.1 Pro" blueprint, LayerNorm on the indexer key):
//   LNk[s]   = bf16(LayerNorm(k_I[s]))
//   S(t,s)   = sum_h w[t,h] * ReLU(q_I[t,h,:] . LNk[s,:])    bf16 operands, FP32 accumulation,
//              for every causal key s of t; the T x T score matrix is never stored
//   topk(t)  = the min(k, n_t) causal keys largest by (score desc, index asc); a token with at
//              most k causal keys keeps all of them.
//
// Kernel design (one wave per query row, eight rows per workgroup, two waves per SIMD):
//  - The host describes the rows that need a selection as per-document segments; a workgroup
//    takes eight consecutive rows of a segment (longest first) or, when such rows are few, four of
//    the longest and four of the shortest rows left, so that workgroups carry similar work. Rows
//    with at most k causal keys are never scored: the prologue kernel writes them.
//  - The LNk keys of the workgroup's causal range stream through LDS in chunks of 128 keys
//    (asynchronous 16-byte global->LDS copies, double buffered, one barrier per chunk). A staged
//    chunk is laid out by MFMA operand: each 1 KB block is the B operand of one K step of one
//    key tile, so operand reads take constant offsets and are bank-conflict free. All eight rows
//    share every staged chunk; the candidate lists live in global memory, which leaves the LDS
//    for the 128-key chunks.
//  - Scores: v_mfma_f32_16x16x32_bf16 with the indexer heads as M (four 16-row tiles, q_I of the
//    row in registers), 16 keys as N and d_I as K; each M tile's four K steps run as one
//    same-accumulator chain, which the matrix core issues faster than alternating chains. Each
//    lane then owns one key column for four heads per M tile: ReLU, the head weight and the sum
//    over its heads happen in registers, and three lane swaps (permlane32, permlane16) join the
//    four head groups of four 16-key tiles, leaving one full score per lane for 64 consecutive
//    keys. The loop is software pipelined by one tile: the MFMAs of one tile run interleaved with
//    the VALU epilogue of the tile before it, and the next chunk's copies and the appends sit
//    between MFMAs too. (The FP8 form runs 32-key tiles on the 32x32x64 scaled MFMA.)
//  - Top-k: scores become order-preserving uint32 keys. A key is appended to the row's candidate
//    list (keys and token indices in the workspace, 4,608 per row) when it reaches the running
//    threshold (ballot + mbcnt compaction, so the list stays in ascending token order; branch-free,
//    lanes that drop their key write past the list). When a list nears capacity, the whole
//    workgroup runs a radix select over its varying bits (LDS histograms, DPP scans) and a stable
//    compaction keeps the k best (ties to the lower index), which raises the threshold. At the
//    end each wave finishes its own row's exact selection.
#include "dsa_device.h"
#include "dsa_kernels.h"

#include <mutex>
#include <type_traits>

namespace dsa {

// ---------------------------------------------------------------------------------------------
// Key LayerNorm: one wave per key row, double precision, one rounding to bf16.
template <int D_I>
__device__ __forceinline__ void key_layernorm_block(const uint16_t* __restrict__ k_I, const float* __restrict__ gamma,
                                                    const float* __restrict__ beta, double eps, int T,
                                                    uint16_t* __restrict__ LNk, int blk) {
#pragma clang fp contract(off)  // every product and sum rounds on its own, as the definition states
  constexpr int PER = D_I / kWave;
  const int row = blk * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= T) return;
  const uint16_t* x = k_I + static_cast<int64_t>(row) * D_I;
  double v[PER];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    v[i] = bf16_to_f32(x[lane * PER + i]);
    s += v[i];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  const double mean = s / D_I;
  double q = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    double c = v[i] - mean;
    q += c * c;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o);
  const double inv = 1.0 / sqrt(q / D_I + eps);
  uint16_t* y = LNk + static_cast<int64_t>(row) * D_I;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = lane * PER + i;
    double r = (v[i] - mean) * inv;
    if (gamma) r *= static_cast<double>(gamma[c]);
    if (beta) r += static_cast<double>(beta[c]);
    y[c] = f64_to_bf16(r);
  }
}

// ---------------------------------------------------------------------------------------------
constexpr int kHalf = 64;         // keys per score vector (one per lane)
constexpr int kChunk = 128;       // keys per staged LDS chunk: four 32-key MFMA tiles, one barrier
constexpr int kCap = kIdxCap;     // candidate capacity of a row's list
constexpr int kCandStride = kCap + 64;  // per-row words of the keys and of the token indices; the last 64 take the lanes an append drops
constexpr int kSelSlack = 64;     // extra entries a selection before the end of the row may keep
constexpr int kIdxRows = 8;       // query rows per workgroup, one wave each (two per SIMD)
static_assert(kCap >= kIdxMaxTopk + kSelSlack + kChunk, "a list takes a chunk after a selection that kept k + slack");
static_assert(kCap % (kIdxRows * kWave) == 0, "whole wave slices in the workgroup selection");
static_assert(kIdxSlotWords == kIdxRows * 2 * kCandStride, "slot size");

// Running head sums per lane in the FP8 epilogue (element j of a K step goes to sum j % kF8Parts),
// and their combination: the drain of a row's last tile uses the same order.
constexpr int kF8Parts = 1;
__device__ __forceinline__ float sum_parts(const float (&p)[kF8Parts]) {
  if constexpr (kF8Parts == 1) return p[0];
  else if constexpr (kF8Parts == 2) return p[0] + p[1];
  else return (p[0] + p[1]) + (p[2] + p[3]);
}

// max(x, +0) as an integer max on the bit pattern: negative values and -0 (sign bit set) give +0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ uint32_t hi_mask(int lo) { return lo >= 32 ? 0u : ~((1u << lo) - 1u); }

// Wave-wide scans on DPP lane moves (VALU only, no LDS traffic). A moved-in value from a lane
// outside the row, or into a row that row_mask leaves out, is the identity `id`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t id, uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(id), static_cast<int>(x), CTRL, ROW_MASK, 0xf, false));
}
// Inclusive scan of op over lanes 0..i: row_shr 1, 2, 4, 8 within each row of 16 lanes, then
// row_bcast15 and row_bcast31 carry the totals of earlier rows.
template <typename Op>
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_move<0x111, 0xf>(id, x));
  x = op(x, dpp_move<0x112, 0xf>(id, x));
  x = op(x, dpp_move<0x114, 0xf>(id, x));
  x = op(x, dpp_move<0x118, 0xf>(id, x));
  x = op(x, dpp_move<0x142, 0xa>(id, x));
  x = op(x, dpp_move<0x143, 0xc>(id, x));
  return x;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x = wave_inclusive_scan(x, 0u, [](uint32_t p, uint32_t q) { return p | q; });
  return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
  x = wave_inclusive_scan(x, 0xffffffffu, [](uint32_t p, uint32_t q) { return p & q; });
  return __builtin_amdgcn_readlane(x, 63);
}
// Lane i gets the sum over lanes i..63.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t x) {
  const uint32_t inc = wave_inclusive_scan(x, 0u, [](uint32_t p, uint32_t q) { return p + q; });
  return __builtin_amdgcn_readlane(inc, 63) - inc + x;
}

// Keep the k best of a row's cnt candidates (keys desc, then list order = ascending token index).
// Every wave of the workgroup takes part (NW waves, each on a slice of the list). Returns the new
// threshold: a future candidate must have key >= the returned value to possibly enter the top k.
// With slack > 0 the selection may stop early, at the first radix level whose bin holding the
// k-th key leaves at most `slack` extra entries: then every entry at or above that bin's lower
// bound is kept (at least k) and the bound becomes the threshold, which is still at or below the
// k-th key, so no key of the final top k is dropped. *kept_out receives the number kept.
// keys and their token indices live in global memory (the workspace); the list is compacted in
// place and stays in ascending token order.
// hist: 3 * 256 words, scratch: 4*NW words of LDS. Must be called by every thread of the
// workgroup. The compacted list is not waited for: a later reader from another wave waits for
// this workgroup's stores (s_waitcnt vmcnt(0)) and a barrier first.
template <int NW>
__device__ __forceinline__ uint32_t wg_select_topk(uint32_t* __restrict__ keys, int32_t* __restrict__ idxs, DSA_LDS uint32_t* hist,
                                                   DSA_LDS uint32_t* scratch, int cnt, int k, int slack, int* kept_out) {
  constexpr int kSelU = (kCap + NW * kWave - 1) / (NW * kWave);  // list entries per lane of a wave slice
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  // This wave's slice of the list: [s0, s0 + kSelU*64), entries s0 + 64*u + lane. Slots past the
  // list are skipped with uniform branches.
  const int s0 = wave * kWave * kSelU;
  uint32_t v[kSelU];
  int32_t x[kSelU];
  bool in[kSelU];
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const int i = s0 + kWave * u + lane;
    in[u] = i < cnt;
    v[u] = 0u;
    x[u] = 0;
    if (s0 + kWave * u < cnt && in[u]) {
      v[u] = keys[i];
      x[u] = idxs[i];  // needed only by the compaction
    }
  }
  uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    o |= v[u];
    a &= in[u] ? v[u] : 0xffffffffu;
  }
  o = wave_or(o);
  a = wave_and(a);
  if (lane == 0) {
    scratch[wave] = o;
    scratch[NW + wave] = a;
  }
  // Radix level L counts into histogram L % 3 and clears histogram (L + 1) % 3, last read two
  // levels earlier: one barrier per level.
  for (int i = threadIdx.x; i < 256; i += NW * kWave) hist[i] = 0u;
  barrier_lds();
  o = 0u;
  a = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    o |= scratch[w];
    a &= scratch[NW + w];
  }
  const uint32_t varying = o ^ a;
  int lo;           // bits >= lo of the k-th key are known: cur
  uint32_t cur;
  int need = k;     // how many of the entries matching cur (in list order) are kept
  if (varying == 0u) {
    lo = 0;
    cur = a;
  } else {
    lo = 32 - __clz(static_cast<int>(varying));
    cur = a & hi_mask(lo);
    int hb = 0;  // histogram of this level
    while (true) {
      const int sh = lo > 8 ? lo - 8 : 0;
      const int nb = lo - sh;
      const uint32_t dmask = (1u << nb) - 1u;
      const uint32_t hm = hi_mask(lo);
      DSA_LDS uint32_t* h_cur = hist + 256 * hb;
      const int hn = hb == 2 ? 0 : hb + 1;
#pragma unroll
      for (int u = 0; u < kSelU; ++u)
        if (s0 + kWave * u < cnt && in[u] && (v[u] & hm) == cur)
          __hip_atomic_fetch_add(h_cur + ((v[u] >> sh) & dmask), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      for (int i = threadIdx.x; i < 256; i += NW * kWave) hist[256 * hn + i] = 0u;
      barrier_lds();
      // lane owns bins 4*lane .. 4*lane+3; find the bin holding the need-th largest entry (every
      // wave computes the same answer)
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = h_cur[4 * lane + j];
      const uint32_t mine = h[0] + h[1] + h[2] + h[3];
      uint32_t above = wave_suffix_sum(mine) - mine;
      int found = -1;
      uint32_t f_above = 0, f_cnt = 0;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (found < 0 && above < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= above + h[j]) {
          found = 4 * lane + j;
          f_above = above;
          f_cnt = h[j];
        }
        above += h[j];
      }
      const uint64_t fm = ballot(found >= 0);
      const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(fm)) - 1);
      const int d = __builtin_amdgcn_readlane(found, src);
      const uint32_t dab = __builtin_amdgcn_readlane(f_above, src);
      const uint32_t dcnt = __builtin_amdgcn_readlane(f_cnt, src);
      need -= static_cast<int>(dab);
      cur |= static_cast<uint32_t>(d) << sh;
      lo = sh;
      hb = hn;
      if (dcnt == static_cast<uint32_t>(need) || sh == 0) break;
      if (static_cast<int>(dcnt) - need <= slack) {  // early stop: keep the whole bin
        need = static_cast<int>(dcnt);
        break;
      }
    }
  }
  // Stable compaction: keep (key_hi > cur) and the first `need` entries with key_hi == cur.
  // Phase 1: per-wave counts; phase 2: each wave writes its kept entries after the kept entries
  // of the waves before it. Every wave holds its entries in registers before any wave writes.
  const uint32_t hm = hi_mask(lo);
  int gt_w = 0, eq_w = 0;
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const uint32_t vh = v[u] & hm;
    gt_w += __popcll(ballot(in[u] && vh > cur));
    eq_w += __popcll(ballot(in[u] && vh == cur));
  }
  if (lane == 0) {
    scratch[2 * NW + wave] = static_cast<uint32_t>(gt_w);
    scratch[3 * NW + wave] = static_cast<uint32_t>(eq_w);
  }
  wait_vmem();    // this wave's list loads are complete before another wave overwrites them
  // Consume every index load here, on every path: the stores below then need no wait each, and the
  // compiler's wait insertion does not treat the loads as possibly outstanding at the caller's loop
  // head (it would drain every memory operation, the next chunk's copies included, there).
#pragma unroll
  for (int u = 0; u < kSelU; ++u) asm volatile("" ::"v"(x[u]));
  barrier_lds();
  // kept: entries kept by the waves before this one; eq_seen: their equal entries
  int kept = 0, eq_seen = 0, total = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int g = static_cast<int>(scratch[2 * NW + w]), e = static_cast<int>(scratch[3 * NW + w]);
    const int keq = min(e, max(need - eq_before, 0));  // equal entries wave w keeps
    if (w < wave) {
      kept += g + keq;
      eq_seen += e;
    }
    total += g + keq;
    eq_before += e;
  }
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const uint32_t vh = v[u] & hm;
    const bool gt = in[u] && vh > cur;
    const bool eq = in[u] && vh == cur;
    const uint64_t me = ballot(eq);
    const int r_eq = eq_seen + lanes_below(me);
    const bool keep = gt || (eq && r_eq < need);
    const uint64_t mk = ballot(keep);
    const int pos = kept + lanes_below(mk);
    if (keep) {
      keys[pos] = v[u];
      idxs[pos] = x[u];
    }
    kept += __popcll(mk);
    eq_seen += __popcll(me);
  }
  *kept_out = total;
  return lo == 0 ? cur + 1u : cur;
}

// Exact top k of one row's cnt candidates (k < cnt <= kCap) by one wave, without workgroup
// barriers, so that every wave can finish its own row at the same time. Keys and token indices in
// global memory (the row's list in the workspace), both in ascending token order; the k kept
// indices go to out[0 .. k) in that order (keys desc, ties to the lower index). hist (256 words)
// and obuf (k words) are LDS that only this wave uses.
//
// The eight waves of a block finish their rows together, so the selection keeps its memory
// instructions few and its waits few: every key and every token index of the list is loaded into
// registers at the start, group by group (the index loads land while the radix levels run), and
// the kept indices are compacted into obuf and leave from there in 16-byte stores.
__device__ __forceinline__ void wave_select_out(const uint32_t* __restrict__ keys, const int32_t* __restrict__ idxs,
                                                DSA_LDS uint32_t* hist, DSA_LDS uint32_t* obuf, int cnt, int k,
                                                int32_t* __restrict__ out) {
  constexpr int U = kCap / kWave;  // entries per lane: entry 64*u + lane
  constexpr int G = 8;             // slots per group
  static_assert(kCap % kWave == 0 && U % G == 0 && G * kWave * (U / G) <= kCandStride, "whole list rows and groups");
  const int lane = lane_id();
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  // Slots go in groups of G; the groups past the list are skipped by uniform branches, and within
  // a group nothing branches. The pad entries of the last group (past cnt) hold key 0: they take
  // part in a level only if key 0 matches its prefix, and each histogram then takes them back out
  // of bin 0. Their token-index slots lie inside the row's list area and are never kept.
  const int ng = (cnt + G * kWave - 1) / (G * kWave);
  const uint32_t pad = static_cast<uint32_t>(G * kWave * ng - cnt);
  uint32_t v[U];
  int32_t x[U];
#pragma unroll
  for (int g = 0; g < U / G; ++g) {
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < G; ++i) v[G * g + i] = keys[min(kWave * (G * g + i) + lane, cnt - 1)];
    }
  }
#pragma unroll
  for (int g = 0; g < U / G; ++g) {
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < G; ++i) x[G * g + i] = idxs[kWave * (G * g + i) + lane];
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i) x[G * g + i] = 0;
    }
  }
  uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
  for (int g = 0; g < U / G; ++g) {
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int u = G * g + i;
        const bool in = kWave * u + lane < cnt;
        v[u] = in ? v[u] : 0u;
        o |= v[u];
        a &= in ? v[u] : 0xffffffffu;
      }
    } else {
#pragma unroll
      for (int i = 0; i < G; ++i) v[G * g + i] = 0u;
    }
  }
  o = wave_or(o);
  a = wave_and(a);
  const uint32_t varying = o ^ a;
  int lo;  // bits >= lo of the k-th key are known: cur
  uint32_t cur;
  int need = k;  // how many of the entries matching cur (in list order) are kept
  bool whole_bin = false;  // every entry matching cur is kept: the kept entries are those >= cur
  if (varying == 0u) {
    lo = 0;
    cur = a;
  } else {
    lo = 32 - __clz(static_cast<int>(varying));
    cur = a & hi_mask(lo);
    while (true) {
      // digit: bits [sh, sh + 8) of the key; where lo < 8 the bits [lo, 8) are cur's in every
      // matching entry, so the digits still order the matching entries
      const int sh = lo > 8 ? lo - 8 : 0;
      const uint32_t hm = hi_mask(lo);
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0u;
#pragma unroll
      for (int g = 0; g < U / G; ++g) {
        if (g < ng) {
#pragma unroll
          for (int i = 0; i < G; ++i) {
            const uint32_t e = v[G * g + i];
            if ((e & hm) == cur) __hip_atomic_fetch_add(hist + __builtin_amdgcn_ubfe(e, sh, 8), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
          }
        }
      }
      const uint32_t pad0 = cur == 0u ? pad : 0u;  // the pad entries (digit 0) matched
      wave_lds_sync();
      // lane owns bins 4*lane .. 4*lane+3; find the bin holding the need-th largest entry
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = hist[4 * lane + j];
      if (lane == 0) h[0] -= pad0;
      const uint32_t mine = h[0] + h[1] + h[2] + h[3];
      uint32_t above = wave_suffix_sum(mine) - mine;
      int found = -1;
      uint32_t f_above = 0, f_cnt = 0;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (found < 0 && above < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= above + h[j]) {
          found = 4 * lane + j;
          f_above = above;
          f_cnt = h[j];
        }
        above += h[j];
      }
      const uint64_t fm = ballot(found >= 0);
      const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(fm)) - 1);
      const int d = __builtin_amdgcn_readlane(found, src);
      const uint32_t dab = __builtin_amdgcn_readlane(f_above, src);
      const uint32_t dcnt = __builtin_amdgcn_readlane(f_cnt, src);
      need -= static_cast<int>(dab);
      cur |= static_cast<uint32_t>(d) << sh;
      lo = sh;
      if (dcnt == static_cast<uint32_t>(need)) {
        whole_bin = true;
        break;
      }
      if (sh == 0) break;
    }
  }
  // Stable compaction into obuf (the indices are in registers; obuf's k words take exactly the kept ones).
  int kept = 0;
  if (whole_bin && cur != 0u) {
    // keep exactly the entries >= cur (the bits of cur below lo are zero, so (v & hi_mask(lo)) >=
    // cur exactly when v >= cur); the pad keys (0) are below cur
#pragma unroll
    for (int g = 0; g < U / G; ++g) {
      if (g < ng) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const bool keep = v[G * g + i] >= cur;
          const uint64_t mk = ballot(keep);
          if (keep) obuf[kept + lanes_below(mk)] = static_cast<uint32_t>(x[G * g + i]);
          kept += __popcll(mk);
        }
      }
    }
  } else {
    // keep (key_hi > cur) and the first `need` entries with key_hi == cur (ties: lower index)
    const uint32_t hm = hi_mask(lo);
    int eq_seen = 0;
#pragma unroll
    for (int g = 0; g < U / G; ++g) {
      if (g < ng) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int u = G * g + i;
          const bool in = kWave * u + lane < cnt;
          const uint32_t vh = v[u] & hm;
          const bool eq = in && vh == cur;
          const uint64_t me = ballot(eq);
          const bool keep = (in && vh > cur) || (eq && eq_seen + lanes_below(me) < need);
          const uint64_t mk = ballot(keep);
          if (keep) obuf[kept + lanes_below(mk)] = static_cast<uint32_t>(x[u]);
          kept += __popcll(mk);
          eq_seen += __popcll(me);
        }
      }
    }
  }
  wave_lds_sync();
  if ((k & 3) == 0) {  // rows of out are 16-byte aligned
    for (int e = 4 * lane; e < k; e += 4 * kWave)
      *reinterpret_cast<u32x4*>(out + e) = *reinterpret_cast<const DSA_LDS u32x4*>(obuf + e);
  } else {
    for (int e = lane; e < k; e += kWave) out[e] = static_cast<int32_t>(obuf[e]);
  }
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// F8: the FP8 indexer (E4M3 operands with power-of-two row scales, v_mfma_scale_f32_32x32x64_f8f6f4
// on 32-key tiles); otherwise BF16 operands on v_mfma_f32_16x16x32_bf16 with 16-key tiles.
// Everything after the scores is shared.
template <int H_I, int D_I, bool F8, bool LNF = false>
__global__ __launch_bounds__(kIdxRows * kWave, 1) void k_index_topk(IndexArgs a) {
  constexpr int TK = F8 ? 32 : 16;               // keys per MFMA N tile
  constexpr int NT = kChunk / TK;                // tiles per chunk
  constexpr int NTH = NT / 2;                    // tiles per 64-key half (one score per lane)
  constexpr int MT = F8 ? (H_I + 31) / 32 : (H_I + 15) / 16;  // M tiles of indexer heads
  constexpr int KS = F8 ? D_I / 64 : D_I / 32;   // MFMA K steps
  constexpr int NMF = MT * KS;                   // MFMAs per tile
  constexpr int EL = F8 ? 16 : 4;                // accumulator elements per lane of one M tile
  constexpr int GPR = F8 ? D_I / 16 : D_I / 8;   // 16-byte granules per key row
  constexpr int CHUNK_GRAN = kChunk * GPR;
  constexpr int CPW = CHUNK_GRAN / (kIdxRows * kWave);  // wave copies (1 KB operand blocks) per chunk and wave
  constexpr int TILE_BYTES = (F8 ? 2 : 1) * KS * 1024;  // one tile's operand blocks
  constexpr int STAGE_BYTES = NT * TILE_BYTES;           // one staged chunk
  // The ring holds two staged chunks; after the last chunk it holds each wave's k output indices.
  constexpr int RING_BYTES = 2 * STAGE_BYTES > kIdxRows * kIdxMaxTopk * 4 ? 2 * STAGE_BYTES : kIdxRows * kIdxMaxTopk * 4;
  // a tile's K step is one 1 KB block (BF16: 16 bytes per lane) or two (FP8: 32 bytes per lane)
  static_assert(CHUNK_GRAN % (kIdxRows * kWave) == 0 && STAGE_BYTES == 16 * CHUNK_GRAN, "chunk copy split");
  static_assert(CPW <= (F8 ? KS : NMF), "a chunk's copies fit beside the MFMAs of one tile");
  static_assert(NTH == 2 || NTH == 4, "a half chunk is joined from two or four tiles");
  // LNF: the wave's CPW blocks of a chunk are the KS K steps of 16-key tile `wave`, i.e. all d_I dims
  // of 16 keys, four lanes per key: the layout the fused key LayerNorm relies on.
  static_assert(!LNF || (!F8 && D_I == 128 && CPW == KS && NT == kIdxRows), "fused LN: BF16, d_I = 128, one tile per wave");
  using QOp = typename std::conditional<F8, i32x8, bf16x8>::type;
  using Acc = typename std::conditional<F8, f32x16, f32x4>::type;

  __shared__ __attribute__((aligned(256))) uint8_t s_ring[RING_BYTES];
  __shared__ uint32_t s_hist[kIdxRows * 256];  // the workgroup selection's three histograms; at the end one per wave
  // Candidate count of a row whose list must be compacted, else 0. Step c reads buffer c % 2 after
  // its barrier while appends of that step write buffer (c + 1) % 2, so no wave can see a flag
  // that another wave of the same step has not seen.
  __shared__ __attribute__((aligned(16))) int s_need[2][kIdxRows];
  __shared__ uint32_t s_sel[4 * kIdxRows];        // selection scratch
  constexpr int WROW = ((H_I + 31) / 32) * 32;
  __shared__ __attribute__((aligned(16))) float s_w[kIdxRows][WROW];  // head weights of each row (0 past H_I)
  __shared__ __attribute__((aligned(16))) float s_gb[LNF ? 2 * D_I : 4];  // fused LN: affine weight, then bias

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // = the row slot of this wave
  const int lane = threadIdx.x % kWave;
  const int k = a.k;

  // This block's segment and its rows. Every row here has more than k causal keys, all in the
  // segment's document, so the block's key range is [doc start, longest row + 1).
  int sg = 0;
  while (sg + 1 < a.nseg && static_cast<int>(blockIdx.x) >= a.seg_blk0[sg + 1]) ++sg;
  const int blk = blockIdx.x - a.seg_blk0[sg];
  const int m = a.seg_m[sg], A = a.seg_r0[sg];
  int i_row, i_top;  // position of this wave's row and of the block's longest row in the segment
  bool has_row;
  if (a.paired) {
    // waves w and w + 4 share a SIMD: one of the longest rows left and one of the shortest
    const int h = (m + 1) >> 1;
    const int p = 4 * blk + (wave & 3);
    has_row = wave < 4 ? p < h : p < m - h;
    i_row = wave < 4 ? m - 1 - p : p;
    i_top = m - 1 - 4 * blk;
  } else {
    i_row = m - kIdxRows * (blk + 1) + wave;
    has_row = i_row >= 0;
    i_top = m - 1 - kIdxRows * blk;
  }
  const int r = A + i_row;
  const int t = a.row0 + r;
  const int b = a.seg_b[sg];
  const bool select = has_row;
  int32_t* out = a.topk_idx + static_cast<int64_t>(r) * k;
  if (lane == 0) {
    s_need[0][wave] = 0;
    s_need[1][wave] = 0;
  }
  // Claim a candidate slot for the workgroup's lists. At most n_slots workgroups are resident at
  // once (the host checks this before the launch) and each frees its slot before it ends, so a
  // free slot always exists; the search is still bounded, and a workgroup that finds none writes
  // -1 rows instead of touching memory it does not own.
  __shared__ int s_slot;
  if (threadIdx.x == 0) {
    int got = -1;
    for (int i = 0; i < 4 * a.n_slots && got < 0; ++i) {
      const int sl = (static_cast<int>(blockIdx.x) + i) % a.n_slots;
      if (atomicCAS(a.slot_flags + sl, 0, 1) == 0) got = sl;
    }
    __threadfence();
    s_slot = got;
  }
  __syncthreads();
  const int slot = __builtin_amdgcn_readfirstlane(s_slot);
  if (slot < 0) {
    if (select)
      for (int j = lane; j < k; j += kWave) out[j] = -1;
    return;  // uniform over the workgroup
  }
  const int kb = b, ke = a.row0 + A + i_top + 1;

  // Query operand (A): rows = heads (zero beyond H_I), K = indexer dims; kept in registers, which
  // the MFMAs read directly. Head weights go to LDS, read back into registers for the epilogue.
  // BF16: M tile mt holds heads 16*mt + lane%16, K values 32*s + 8*(lane/16) .. +8.
  // FP8: 32 bytes per lane and K step, K values 64*s + 32*(lane/32) .. +32 of head 32*mt + lane%32
  // (the key operand takes the same K values, so the pairing does not depend on the instruction's
  // K order); the head's scale goes into its weight.
  QOp qa[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = F8 ? 32 * mt + (lane & 31) : 16 * mt + (lane & 15);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (select && head < H_I) {
        if constexpr (F8) {
          const uint8_t* src = a.q8 + (static_cast<int64_t>(r) * H_I + head) * D_I + 64 * s + 32 * (lane >> 5);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(src), hi = *reinterpret_cast<const i32x4*>(src + 16);
          qa[mt][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          qa[mt][s] = *reinterpret_cast<const bf16x8*>(a.q_I + (static_cast<int64_t>(r) * H_I + head) * D_I + 32 * s + 8 * (lane >> 4));
        }
      } else {
        qa[mt][s] = QOp{};
      }
    }
  }
  if (lane < 32) {
#pragma unroll
    for (int g = 0; g < WROW / 32; ++g) {
      const int head = 32 * g + lane;
      float wv = 0.0f;
      if (select && head < H_I) {
        wv = bf16_to_f32(a.w[static_cast<int64_t>(r) * H_I + head]);
        if constexpr (F8) wv *= a.sq[static_cast<int64_t>(r) * H_I + head];  // a power of two: exact
      }
      s_w[wave][head] = wv;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(qa[mt][s]));

  // LDS-typed pointers, so that every access is a ds_ instruction
  DSA_LDS uint32_t* hist = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_hist[0])));
  DSA_LDS uint32_t* sel_scratch = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_sel[0])));
  // Row rw's list in the claimed slot: kCandStride score keys, then kCandStride token indices.
  auto list_keys = [&](int rw) -> uint32_t* {
    return reinterpret_cast<uint32_t*>(a.cand) + (static_cast<int64_t>(slot) * kIdxRows + rw) * 2 * kCandStride;
  };
  uint32_t* ckeys = list_keys(wave);
  int32_t* cidx = reinterpret_cast<int32_t*>(ckeys + kCandStride);
  int cnt = 0;
  uint32_t thr = 0u;

  // Every wave selects for the rows that asked (rare): all waves of the workgroup share the work.
  auto run_selections = [&](int slack, int nbuf) {
    for (int rw = 0; rw < kIdxRows; ++rw) {
      const int c_rw = s_need[nbuf][rw];
      if (c_rw == 0) continue;  // uniform: every wave reads the same flag
      uint32_t* kr = list_keys(rw);
      int kept = 0;
      const uint32_t th = wg_select_topk<kIdxRows>(kr, reinterpret_cast<int32_t*>(kr + kCandStride), hist, sel_scratch,
                                                   c_rw, k, slack, &kept);
      if (rw == wave) {
        cnt = __builtin_amdgcn_readfirstlane(kept);  // wave-uniform: the list count stays in an SGPR
        thr = th;
      }
    }
    barrier_lds();  // every wave has read the flags
    if (lane == 0) s_need[nbuf][wave] = 0;
  };

  const int nchunks = (ke - kb + kChunk - 1) / kChunk;
  const uint16_t* __restrict__ LNk = a.LNk;

  // A staged chunk is laid out by MFMA operand, one 1 KB block per copy, each copy with a per-lane
  // source offset fixed for the kernel and the chunk's first key row as a scalar base. Operand
  // reads are then whole 1 KB blocks at constant offsets (bank-conflict free).
  // BF16: block n*KS + s holds, at lane i's 16 bytes, dims 32s + 8(i/16) .. +8 of key 16n + i%16:
  // the B operand of K step s of 16-key tile n.
  // FP8: block (n, s, h) = 4n + 2s + h holds, at lane i's 16 bytes, half h of lane i's 32-byte
  // operand of K step s of 32-key tile n: key 32n + i%32, K bytes 64s + 32(i/32) + 16h .. +16.
  // Copy j of this wave fills block CPW*wave + j.
  uint32_t cp_off[CPW];
  constexpr uint32_t kCopyBias = 1024 * (CPW - 1);
  static_assert(CPW <= 4, "copy offsets within the immediate range");
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int blk_j = CPW * wave + j;
    if constexpr (F8) {
      const int n = blk_j / (2 * KS), st = (blk_j % (2 * KS)) >> 1, hf = blk_j & 1;
      cp_off[j] = static_cast<uint32_t>((32 * n + (lane & 31)) * D_I + 64 * st + 32 * (lane >> 5) + 16 * hf);
    } else {
      const int n = blk_j / KS, st = blk_j % KS;
      cp_off[j] = static_cast<uint32_t>(((16 * n + (lane & 15)) * D_I + 32 * st + 8 * (lane >> 4)) * 2);
    }
    // Copy j takes 1024 j as its immediate offset, which moves its LDS address (so that one base per
    // slot serves all the wave's copies) and its global address (taken back here, against a scalar
    // base lowered by kCopyBias so that every per-lane offset stays non-negative).
    cp_off[j] += kCopyBias - 1024 * j;
  }
  const uint32_t ring = lds_addr_of(&s_ring[0]);
  uint32_t cbase = 0;  // this lane's LDS address in the slot of the chunk being scored, set per chunk
  // The last chunk may reach up to 127 rows past the last key row (see kIdxKeyPad): those rows of
  // the padded LNk are staged but never scored. A copy for the chunk after the last one refills the
  // free slot with the last chunk instead, which nothing reads.
  u32x4 raw[LNF ? CPW : 1];  // fused LN: this lane's raw k_I granules of the next chunk
  auto copy_j = [&](const void* chunk_base, int j, uint32_t lds_base) {
    const void* sb = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(chunk_base) - kCopyBias);
    switch (j) {
      case 0: copy16_to_lds_imm<0>(sb, cp_off[0], lds_base); break;
      case 1: if constexpr (CPW > 1) copy16_to_lds_imm<1024>(sb, cp_off[1], lds_base); break;
      case 2: if constexpr (CPW > 2) copy16_to_lds_imm<2048>(sb, cp_off[2], lds_base); break;
      default: if constexpr (CPW > 3) copy16_to_lds_imm<3072>(sb, cp_off[3], lds_base); break;
    }
  };
  auto issue_copy = [&](int c, int j) {
    const int K0 = kb + min(c, nchunks - 1) * kChunk;
    const uint32_t lds = ring + (c & 1) * STAGE_BYTES + 1024 * CPW * wave;  // + 1024 j, the immediate
    if constexpr (LNF) {
      // key 16*wave + lane%16 of the chunk (rows past the last key read the last key: never scored),
      // dims 32j + 8(lane/16) .. +8: the lane's granule of block CPW*wave + j
      const int key = min(K0 + 16 * wave + (lane & 15), a.T - 1);
      raw[j] = *reinterpret_cast<const u32x4*>(a.k_raw + static_cast<int64_t>(key) * D_I + 32 * j + 8 * (lane >> 4));
    } else if constexpr (F8) {
      copy_j(a.LNk8 + static_cast<int64_t>(K0) * D_I, j, lds);
    } else {
      copy_j(LNk + static_cast<int64_t>(K0) * D_I, j, lds);
    }
  };
  // Fused LN: normalise the raw granules of chunk c (loaded by issue_copy) and write them to the
  // chunk's staging slot as the B operand blocks. The four lanes lane%16 + 16m hold one key's 128
  // values; mean and biased variance in double (every sum here is exact for bf16 inputs, so the order
  // of the lane sums does not matter), then one rounding to bf16, as in the prologue.
  auto ln_stage = [&](int c) {
    if constexpr (LNF) {
#pragma clang fp contract(off)
      auto val = [&](int j, int e) -> double {  // value e of granule j, re-read from the raw registers
        return static_cast<double>(bf16_to_f32(static_cast<uint16_t>(raw[j][e >> 1] >> (16 * (e & 1)))));
      };
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += val(j, e);
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      const double mean = sum / D_I;
      // each pass converts the values again rather than keeping 32 doubles alive across the passes
#pragma unroll
      for (int j = 0; j < CPW; ++j) asm volatile("" : "+v"(raw[j]));
      double sq = 0.0;
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = val(j, e) - mean;
          sq += d * d;
        }
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
#pragma unroll
      for (int j = 0; j < CPW; ++j) asm volatile("" : "+v"(raw[j]));
      const double inv = 1.0 / sqrt(sq / D_I + a.ln_eps);
      const bool has_b = a.ln_beta != nullptr;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        u32x4 o;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t w2 = 0u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int e = 2 * e2 + h, dim = 32 * j + 8 * (lane >> 4) + e;
            // the weight defaults to 1 (an exact product); the bias is selected, not added as 0, so
            // that a -0 stays -0 as in the prologue
            double r = (val(j, e) - mean) * inv;
            r *= static_cast<double>(s_gb[dim]);
            const double rb = r + static_cast<double>(s_gb[D_I + dim]);
            r = has_b ? rb : r;
            w2 |= static_cast<uint32_t>(f64_to_bf16(r)) << (16 * h);
          }
          o[e2] = w2;
        }
        *reinterpret_cast<DSA_LDS u32x4*>(lds_ptr(ring + (c & 1) * STAGE_BYTES + 1024 * (CPW * wave + j) + 16 * lane)) = o;
        __builtin_amdgcn_sched_barrier(0);  // one granule at a time: bounds the live double temporaries
      }
    }
  };
  // Scores of a chunk come from NT tiles of TK keys (K = d_I), into accA and accB in turn. The loop
  // is software pipelined by one tile: the MFMAs of one tile run interleaved with the VALU
  // epilogue of the tile before it (ReLU, head weight, partial head sums), so the matrix core and
  // the vector ALU work at the same time.
  Acc accA[MT], accB[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) accB[mt] = Acc{};  // the epilogue of "chunk -1" adds nothing
  // Head weights in registers, in accumulator order: element 4*g + e of M tile mt holds head
  // 32*mt + 8*g + 4*(lane/32) + e (FP8, 32x32 tiles) or 16*mt + 4*(lane/16) + e (BF16, 16x16).
  f32x4 w4[MT][EL / 4];
  {
    const DSA_LDS float* wrow = reinterpret_cast<const DSA_LDS float*>(lds_ptr(lds_addr_of(&s_w[wave][0])));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < EL / 4; ++g)
        w4[mt][g] = *reinterpret_cast<const DSA_LDS f32x4*>(
            wrow + (F8 ? 32 * mt + 8 * g + 4 * (lane >> 5) : 16 * mt + 4 * (lane >> 4)));
  }
  auto epi = [&](const Acc (&prev)[MT], int el, float p) -> float {
    const int mt = el / EL, i = el % EL;
    return __builtin_fmaf(w4[mt][i / 4][i % 4], relu(prev[mt][i]), p);
  };
  // BF16: one 16-key tile n of chunk c. The K steps of each M tile run as one same-accumulator
  // chain, each MFMA beside its share of the epilogue of `prev`. The tile's key operands were read
  // by the tile before it (tile 0 reads its own after the chunk's barrier); this tile reads the
  // next tile's while its MFMAs run. Returns this lane's partial head sum of the previous tile.
  bf16x8 bkr[2][KS];
  auto tile16 = [&](int c, auto nn, Acc (&acc)[MT], const Acc (&prev)[MT], auto&& side) -> float {
    constexpr int n = decltype(nn)::value;
    constexpr int EPM = MT * EL / NMF;  // epilogue elements per MFMA
    static_assert(EPM * NMF == MT * EL && EPM >= 1, "epilogue split");
    constexpr int PF_M = MT >= 2 ? MT - 2 : 0;  // the M tile beside whose MFMAs the next tile's operands are read
    bf16x8 (&bk)[KS] = bkr[n & 1];
    bf16x8 (&bn)[KS] = bkr[(n + 1) & 1];
    const uint32_t a0 = cbase + n * TILE_BYTES;  // the tile's offsets fold into the reads' immediates
    if constexpr (n == 0) {
#pragma unroll
      for (int s = 0; s < KS; ++s) bk[s] = lds_read16(lds_ptr(a0 + 1024 * s));
    }
    // one running sum when each MFMA has one epilogue element beside it, else two
    float part[2] = {0.0f, 0.0f};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int j = mt * KS + s;
        if constexpr (!F8) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], bk[s], s == 0 ? Acc{} : acc[mt], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < EPM; ++e) part[e & 1] = epi(prev, j * EPM + e, part[e & 1]);
        if constexpr (EPM == 1) asm volatile("" : "+v"(part[0]));
        else asm volatile("" : "+v"(part[0]), "+v"(part[1]));
        const bool rd = n + 1 < NT && mt == PF_M;
        if (rd) bn[s] = lds_read16(lds_ptr(a0 + TILE_BYTES + 1024 * s));
        side(j);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2 * EPM, 0);
        if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (j < CPW) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (EPM == 1) return part[0];
    else return part[0] + part[1];
  };
  // FP8: one 32-key tile n of chunk c; its two K steps read as four 1 KB blocks at once, each K
  // step one 32x32x64 MFMA per M tile beside its half of the epilogue (kept in four partial sums).
  auto tile_step8 = [&](int c, auto nn, Acc (&acc)[MT], const Acc (&prev)[MT], auto&& side) -> float {
    constexpr int n = decltype(nn)::value;
    constexpr int kEps = MT * EL / KS;  // epilogue elements per K step
    const uint32_t a0 = cbase + n * TILE_BYTES;
    i32x8 bk[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x4 lo = __builtin_bit_cast(i32x4, lds_read16(lds_ptr(a0 + 2048 * s)));
      const i32x4 hi = __builtin_bit_cast(i32x4, lds_read16(lds_ptr(a0 + 2048 * s + 1024)));
      bk[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    constexpr int NP = kF8Parts;
    float part[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) part[j] = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (F8) acc[mt] = mfma32_fp8(qa[mt][s], bk[s], s == 0 ? Acc{} : acc[mt]);
      }
#pragma unroll
      for (int j = 0; j < kEps; ++j) part[j % NP] = epi(prev, s * kEps + j, part[j % NP]);
#pragma unroll
      for (int j = 0; j < NP; ++j) asm volatile("" : "+v"(part[j]));
      side(s);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MT - 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps + 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return sum_parts(part);
  };
  // The epilogue of `prev` alone (a row's last chunk, or a wave whose row has ended), summed in
  // exactly the order of the tile functions above, so that equal keys get bit-identical scores
  // wherever they fall.
  auto tile_drain = [&](const Acc (&prev)[MT]) -> float {
    if constexpr (F8) {
      constexpr int kEps = MT * EL / KS;
      float part[kF8Parts];
#pragma unroll
      for (int j = 0; j < kF8Parts; ++j) part[j] = 0.0f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int j = 0; j < kEps; ++j) part[j % kF8Parts] = epi(prev, s * kEps + j, part[j % kF8Parts]);
      return sum_parts(part);
    } else {
      constexpr int EPM = MT * EL / NMF;
      float part[2] = {0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NMF; ++j)
#pragma unroll
        for (int e = 0; e < EPM; ++e) part[e & 1] = epi(prev, j * EPM + e, part[e & 1]);
      if constexpr (EPM == 1) return part[0];
      else return part[0] + part[1];
    }
  };
  // One score per lane for the 64 keys of a half chunk, from the partial head sums of its tiles.
  // FP8 (two 32-key tiles): lanes < 32 hold key lane of tile 0 in p[0] and of tile 1 in p[1]
  // (heads with lane/32 = 0), lanes >= 32 the other heads; one permlane32 swap leaves lane l with
  // the full score of key l. BF16 (four 16-key tiles): lane l holds key l%16 of each tile for
  // head group l/16; two permlane32 swaps add groups g and g + 2, one permlane16 swap adds the
  // rest, again leaving lane l with key l.
  auto join = [](const float (&p)[NTH]) -> float {
    auto sum_swap32 = [](float x, float y) -> float {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
      return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    if constexpr (NTH == 2) {
      return sum_swap32(p[0], p[1]);
    } else {
      const float x = sum_swap32(p[0], p[2]), y = sum_swap32(p[1], p[3]);
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
      return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
  };
  // Append the keys of half chunk u (keys kb + 64u ..) that reach the threshold: keys and token
  // indices to the row's list, in ascending token order. Branch-free, so that it can sit between
  // MFMAs: lanes that do not take their key write it to a slot past the list. A list that may not
  // take another chunk while the row still has keys after half u raises its flag for the next step.
  auto append = [&](int u, float score, int nbuf) {
    const int s_key = kb + u * kHalf + lane;
    // score_key's order, in fewer instructions: adding +0 turns a -0 score into +0 (one key for both
    // zeros), then negative scores are complemented and the others get the sign bit
    const uint32_t su = __float_as_uint(score + 0.0f);
    const uint32_t key = su ^ (static_cast<uint32_t>(static_cast<int32_t>(su) >> 31) | 0x80000000u);
    // every key of the block is at or after the document start kb, and half u = -1 (before the first
    // chunk) takes nothing. The ballots of the two comparisons are their compare masks as they stand;
    // the wave-uniform condition selects the whole mask.
    const bool on = select & (u >= 0);
    const bool in_row = s_key <= t, above = key >= thr;
    const uint64_t msk = __builtin_amdgcn_ballot_w64(in_row) & __builtin_amdgcn_ballot_w64(above) & (0ull - static_cast<uint64_t>(on));
    const bool take = on & in_row & above;
    // 32-bit byte offsets from the lists' wave-uniform bases: every lane's rank among the taken ones
    // (one shift-and-add), then one select by the mask (no exec-masked region)
    uint32_t off_take = (static_cast<uint32_t>(lanes_below(msk)) << 2) + static_cast<uint32_t>(cnt) * 4u;
    asm volatile("" : "+v"(off_take));
    const uint32_t off = take ? off_take : static_cast<uint32_t>(kCap + lane) * 4u;
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ckeys) + off) = key;
    *reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(cidx) + off) = s_key;
    cnt += __popcll(msk);
    const bool more = kb + (u + 1) * kHalf <= t;
    s_need[nbuf][wave] = cnt > kCap - kChunk && more ? cnt : 0;  // every lane writes the same value
  };

  auto tile = [&](int c, auto nn, Acc (&acc)[MT], const Acc (&prev)[MT], auto&& side) -> float {
    if constexpr (F8) return tile_step8(c, nn, acc, prev, side);
    else return tile16(c, nn, acc, prev, side);
  };
  float ph_prev[NTH];  // partial sums of the previous chunk's second-half tiles (the last one unused)
#pragma unroll
  for (int i = 0; i < NTH; ++i) ph_prev[i] = 0.0f;
  // FP8: the key scales of the previous chunk's second half (lane l: key 64 + l), loaded a step
  // before they are used
  float sk_prev = 1.0f;
  if constexpr (LNF) {
    for (int i = threadIdx.x; i < D_I; i += kIdxRows * kWave) {
      s_gb[i] = a.ln_gamma != nullptr ? a.ln_gamma[i] : 1.0f;
      s_gb[D_I + i] = a.ln_beta != nullptr ? a.ln_beta[i] : 0.0f;
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < CPW; ++j) issue_copy(0, j);
  ln_stage(0);
  // Step c: tile 0 of chunk c (the next chunk's copies issued between its MFMAs); the selections
  // that the lists filled by step c-1 asked for; the other tiles, with the append of the second
  // half of chunk c-1 beside tile 1 and that of the first half of chunk c beside tile NTH + 1.
  // Step nchunks runs no MFMAs: it only finishes the last chunk.
  for (int c = 0; c <= nchunks; ++c) {
    wait_vmem();    // this wave's copies of chunk c and its list stores are complete
    barrier_lds();  // chunk c has landed; the slot of chunk c-1 is free
    // flags of the lists that step c-1 filled: read now, used after tile 0
    const i32x4 f0 = *reinterpret_cast<const DSA_LDS i32x4*>(lds_ptr(lds_addr_of(&s_need[c & 1][0])));
    const i32x4 f1 = *reinterpret_cast<const DSA_LDS i32x4*>(lds_ptr(lds_addr_of(&s_need[c & 1][4])));
    cbase = ring + (c & 1) * STAGE_BYTES + 16 * lane;
    asm volatile("" : "+v"(cbase));  // one VGPR for the whole chunk
    const bool act = select && c < nchunks && kb + c * kChunk <= t;                 // row has keys in chunk c
    const bool act_prev = select && c > 0 && kb + (c - 1) * kChunk + kHalf <= t;  // and in the second half of chunk c-1
    float sk_lo = 1.0f, sk_hi = 1.0f;
    if constexpr (F8) {
      if (c < nchunks) {  // within the padded key rows
        sk_lo = a.sk[kb + c * kChunk + lane];
        sk_hi = a.sk[kb + c * kChunk + kHalf + lane];
      }
    }
    float score_hi = 0.0f;  // scores of the second half of chunk c-1
    if (act) {
      // a wave whose row ends before this chunk leaves its SIMD to the other wave there
      auto copies = [&](int st) {
        if (!LNF && st < CPW) issue_copy(c + 1, st);
      };
      ph_prev[NTH - 1] = tile(c, std::integral_constant<int, 0>{}, accA, accB, copies);
      score_hi = join(ph_prev);
      if constexpr (F8) score_hi *= sk_prev;  // a power of two: exact
    } else if (c + 1 < nchunks) {
#pragma unroll
      for (int j = 0; j < CPW; ++j) issue_copy(c + 1, j);
      ln_stage(c + 1);
    }
    if ((f0[0] | f0[1] | f0[2] | f0[3] | f1[0] | f1[1] | f1[2] | f1[3]) != 0)
      run_selections(kSelSlack, c & 1);  // uniform, rare
    if (act) {
      float pc[NT];  // pc[i]: partial sums of tile i of chunk c
      float score_lo = 0.0f;
      static_for<1, NT>([&](auto nn) {
        constexpr int n = decltype(nn)::value;
        auto side = [&](int st) {
          // early in the tile, so that the list stores land before the next step's wait
          if constexpr (n == 1) {
            if (st == 0) append(2 * c - 1, score_hi, (c + 1) & 1);
          } else if constexpr (n == NTH + 1) {
            if (st == 0) append(2 * c, score_lo, (c + 1) & 1);
          } else if constexpr (LNF && n == NT - 1) {
            // fused LN: the next chunk's raw keys, loaded beside the last tile (their registers are
            // live only from here to the staging after it)
            if (st < CPW && c + 1 < nchunks) issue_copy(c + 1, st);
          }
        };
        if constexpr (n % 2 == 0) pc[n - 1] = tile(c, nn, accA, accB, side);
        else pc[n - 1] = tile(c, nn, accB, accA, side);
        if constexpr (n == NTH) {
          float lo[NTH];
#pragma unroll
          for (int i = 0; i < NTH; ++i) lo[i] = pc[i];
          score_lo = join(lo);
          if constexpr (F8) score_lo *= sk_lo;
        }
      });
#pragma unroll
      for (int i = 0; i + 1 < NTH; ++i) ph_prev[i] = pc[NTH + i];
      if (c + 1 < nchunks) ln_stage(c + 1);  // fused LN only; its LDS writes land before the next barrier
    } else if (act_prev) {
      ph_prev[NTH - 1] = tile_drain(accB);  // the last tile of chunk c-1 (odd: accB)
      float sc = join(ph_prev);
      if constexpr (F8) sc *= sk_prev;
      append(2 * c - 1, sc, (c + 1) & 1);
    }
    sk_prev = sk_hi;
  }

  // Final exact selection: each wave finishes its own row, with its histogram in s_hist and its
  // output indices in the staging ring, which no wave uses any more.
  wait_vmem();    // this wave's list stores are complete
  barrier_lds();  // every wave is done with the staging ring
  if (select) {
    if (cnt > k) {
      DSA_LDS uint32_t* obuf = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(ring + wave * kIdxMaxTopk * 4));
      wave_select_out(ckeys, cidx, hist + 256 * wave, obuf, cnt, k, out);
    } else {  // exactly k candidates
      for (int j = lane; j < k; j += kWave) out[j] = cidx[j];
    }
  }
  // Free the slot once every wave's reads of its list have completed.
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicExch(a.slot_flags + slot, 0);
  }
}

// ---------------------------------------------------------------------------------------------
int index_blocks(int m, int paired) { return paired ? ((m + 1) / 2 + 3) / 4 : (m + kIdxRows - 1) / kIdxRows; }

// Workgroups of the indexer kernel that the current device can hold at once (CUs x occupancy),
// computed once per device.
static const void* index_kernel(int v) {
  switch (v) {
    case 0: return reinterpret_cast<const void*>(k_index_topk<64, 128, false>);
    case 1: return reinterpret_cast<const void*>(k_index_topk<4, 64, false>);
    case 2: return reinterpret_cast<const void*>(k_index_topk<64, 128, true>);
    default: return reinterpret_cast<const void*>(k_index_topk<64, 128, false, true>);
  }
}

static int index_resident_blocks(int v) {
  static std::mutex mu;
  static int cached[4][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[v][dev] == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, index_kernel(v), kIdxRows * kWave, 0) != hipSuccess) return -1;
    cached[v][dev] = cus * occ;
  }
  return cached[v][dev];
}

hipError_t launch_index_topk(const IndexArgs& a, int H_I, int d_I, bool fp8, hipStream_t st, bool fused_ln) {
  if (a.nseg < 1 || a.nseg > kIdxMaxSeg || a.n_slots < 1) return hipErrorInvalidValue;
  const bool big = H_I == 64 && d_I == 128;
  if ((fp8 || fused_ln) && !big) return hipErrorInvalidValue;
  if (fp8 && fused_ln) return hipErrorInvalidValue;
  const int v = fused_ln ? 3 : fp8 ? 2 : (big ? 0 : 1);
  const int resident = index_resident_blocks(v);
  if (resident < 1 || resident > a.n_slots) return hipErrorInvalidConfiguration;  // slots could run out
  dim3 grid(a.seg_blk0[a.nseg]), block(kIdxRows * kWave);
  switch (v) {
    case 0: hipLaunchKernelGGL((k_index_topk<64, 128, false>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((k_index_topk<4, 64, false>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_index_topk<64, 128, true>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_index_topk<64, 128, false, true>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// FP8 operands: each 128-value bf16 row becomes E4M3 codes and one power-of-two scale 2^e, e the
// smallest integer with amax * 2^-e <= 448. Half a wave per row, four values per lane; the scaling
// is exact and v_cvt_pk_fp8_f32 rounds to the nearest code (ties to even).
__device__ __forceinline__ void quantize_row128(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                float* __restrict__ scale, int sub) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(x + 4 * sub);
  const float f0 = bf16_to_f32(static_cast<uint16_t>(v[0])), f1 = bf16_to_f32(static_cast<uint16_t>(v[0] >> 16));
  const float f2 = bf16_to_f32(static_cast<uint16_t>(v[1])), f3 = bf16_to_f32(static_cast<uint16_t>(v[1] >> 16));
  float m = fmaxf(fmaxf(fabsf(f0), fabsf(f1)), fmaxf(fabsf(f2), fabsf(f3)));
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
  int E = 0;
  const float mant = frexpf(m, &E);  // m = mant * 2^E, mant in [0.5, 1); 448 = 0.875 * 2^9
  const int e = m == 0.0f ? 0 : E - 9 + (mant > 0.875f ? 1 : 0);
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f0, -e), ldexpf(f1, -e), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f2, -e), ldexpf(f3, -e), w, true);
  *reinterpret_cast<uint32_t*>(q + 4 * sub) = w;
  if (sub == 0) *scale = ldexpf(1.0f, e);
}

__global__ __launch_bounds__(256) void k_quantize_fp8(const uint16_t* __restrict__ x1, int64_t n1, uint8_t* __restrict__ q1,
                                                      float* __restrict__ s1, const uint16_t* __restrict__ x2, int64_t n2,
                                                      uint8_t* __restrict__ q2, float* __restrict__ s2) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + threadIdx.x / 32;
  const int sub = threadIdx.x % 32;
  if (row < n1) quantize_row128(x1 + row * 128, q1 + row * 128, s1 + row, sub);
  else if (row - n1 < n2) quantize_row128(x2 + (row - n1) * 128, q2 + (row - n1) * 128, s2 + (row - n1), sub);
}

hipError_t launch_quantize_fp8(const uint16_t* x1, int64_t n1, uint8_t* q1, float* s1, const uint16_t* x2, int64_t n2,
                               uint8_t* q2, float* s2, hipStream_t st) {
  const int64_t blocks = (n1 + n2 + 7) / 8;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize_fp8, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, x1, n1, q1, s1, x2, n2, q2, s2);
  return hipGetLastError();
}

// Rows with at most k causal keys keep all of them in token order, then -1. One block per row
// at a time (block blk of nblk); rows with more keys are left to k_index_topk.
__device__ __forceinline__ void short_rows_block(const IndexArgs& a, int blk, int nblk) {
  for (int r = blk; r < a.nrows; r += nblk) {
    const int t = a.row0 + r;
    const int b = doc_begin(a.cu, a.n_docs, t);
    const int n = t - b + 1;
    if (n > a.k) continue;  // uniform
    int32_t* out = a.topk_idx + static_cast<int64_t>(r) * a.k;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < n ? b + j : -1;
  }
}

// The two independent parts before the scoring kernel, in one launch: blocks [0, nln) normalise
// four keys each, the others write the rows with at most k causal keys.
template <int D_I>
__global__ __launch_bounds__(256) void k_index_prologue(const uint16_t* __restrict__ k_I, const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, double eps,
                                                        uint16_t* __restrict__ LNk, IndexArgs a, int nln) {
  const int blk = blockIdx.x;
  if (blk == 0)  // every candidate slot starts free
    for (int i = threadIdx.x; i < a.n_slots; i += blockDim.x) a.slot_flags[i] = 0;
  if (blk < nln) key_layernorm_block<D_I>(k_I, gamma, beta, eps, a.T, LNk, blk);
  else short_rows_block(a, blk - nln, gridDim.x - nln);
}

hipError_t launch_index_prologue(const uint16_t* k_I, const float* gamma, const float* beta, double eps, int d_I,
                                 uint16_t* LNk, const IndexArgs& a, hipStream_t st, bool do_ln) {
  const int nln = do_ln ? (a.T + 3) / 4 : 0;
  const int nfill = a.nrows < 2048 ? a.nrows : 2048;
  dim3 grid(nln + nfill), block(256);
  if (d_I == 128) hipLaunchKernelGGL((k_index_prologue<128>), grid, block, 0, st, k_I, gamma, beta, eps, LNk, a, nln);
  else hipLaunchKernelGGL((k_index_prologue<64>), grid, block, 0, st, k_I, gamma, beta, eps, LNk, a, nln);
  return hipGetLastError();
}

}  // namespace dsa

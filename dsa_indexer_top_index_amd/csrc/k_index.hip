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
//  - The LNk keys of the workgroup's causal range stream through LDS in chunks of 64 keys
//    (asynchronous 16-byte global->LDS copies, double buffered, one barrier per chunk). A staged
//    chunk is laid out by MFMA operand: each 1 KB block is the B operand of one K step of one
//    32-key tile, so operand reads take constant offsets and are bank-conflict free. All eight
//    rows share every staged chunk.
//  - Scores: v_mfma_f32_32x32x16_bf16 with the indexer heads as M (q_I of the row in
//    registers), 32 keys as N and d_I as K. Each lane then owns one key column: ReLU, the head
//    weight and the sum over heads happen in registers, and one permlane32 swap joins the two
//    half-waves, leaving one full score per lane for 64 consecutive keys. The loop is software
//    pipelined by half a chunk: the MFMAs of one 32-key tile run interleaved with the VALU epilogue
//    of the tile before it, and the next chunk's copies and the previous chunk's append sit
//    between MFMAs too.
//  - Top-k: scores become order-preserving uint32 keys. A key is appended to the row's candidate
//    list (keys in LDS, token indices in the workspace) when it reaches the running threshold
//    (ballot + mbcnt compaction, so the list stays in ascending token order; branch-free, lanes
//    that drop their key write past the list). When a list nears capacity, the whole workgroup
//    runs a radix select over its varying bits (LDS histograms, DPP scans) and a stable
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
constexpr int kChunk = 64;        // keys per LDS chunk (two 32-key MFMA tiles)
constexpr int kCap = 3840;        // candidate capacity of a row's list (>= k + kSelSlack + 2 * kChunk for k <= 2048)
constexpr int kListSlots = kCap + 64;   // LDS slots per list: the last 64 take the lanes an append drops
// Waves w and w + 4 share a SIMD and their lists sit side by side. When a block pairs long and
// short rows, a long row that would overflow kCap may take kCapLong slots of the pair's space if
// its partner row fits in the rest (kCapShort), so that it needs no selection before its end.
constexpr int kCapLong = 4096;
constexpr int kCapShort = 2 * kListSlots - (kCapLong + 64) - 64;
constexpr int kCandStride = kCapLong + 64;  // per-row stride of the candidate token indices (global)
static_assert(kCapShort >= 2048 + 64 + 2 * 64, "a short list still holds k + slack + two chunks");
static_assert(kCap % 256 == 0 && kCapLong % 256 == 0 && kCapShort % 256 == 0, "the final selection copies 256 indices at a time");
constexpr int kSelSlack = 64;    // extra entries a selection before the end of the row may keep
constexpr int kIdxRows = 8;       // query rows per workgroup, one wave each (two per SIMD)


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
// keys live in LDS, their token indices in global memory (idxs); the list is compacted in place
// and stays in ascending token order.
// hist: 3 * 256 words, scratch: 4*NW words of LDS. Must be called by every thread of the
// workgroup. The compacted indices are not waited for: a later reader of idxs from another wave
// waits for this workgroup's stores (s_waitcnt vmcnt(0)) and a barrier first.
template <int NW>
__device__ __forceinline__ uint32_t wg_select_topk(DSA_LDS uint32_t* keys, int32_t* __restrict__ idxs, DSA_LDS uint32_t* hist,
                                                   DSA_LDS uint32_t* scratch, int cnt, int k, int slack, int* kept_out) {
  constexpr int kSelU = (kCapLong + NW * kWave - 1) / (NW * kWave);  // list entries per lane of a wave slice
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
      x[u] = idxs[i];  // global loads, needed only by the compaction
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
  wait_vmem();    // this wave's index loads are complete before another wave overwrites them
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

// Exact top k of one row's cnt candidates (k < cnt <= kCapLong) by one wave, without workgroup
// barriers, so that every wave can finish its own row at the same time. Keys in LDS (list, cap
// words rounded up to 256) and token indices in global memory (idxs), both in ascending token
// order; the k kept indices go to out[0 .. k) in that order (keys desc, ties to the lower index).
// hist: 256 words of LDS that only this wave uses.
//
// The eight waves of a block finish their rows together, so the selection keeps its memory
// instructions few and its LDS reads batched: once the keys are in registers, the token indices
// are copied into the list's own LDS slots (1 KB per copy), compacted there in place, and the k
// kept ones leave in 16-byte stores.
__device__ __forceinline__ void wave_select_out(DSA_LDS uint32_t* list, const int32_t* __restrict__ idxs,
                                                DSA_LDS uint32_t* hist, int cnt, int k, int32_t* __restrict__ out) {
  constexpr int U = kCapLong / kWave;  // entries per lane: entry 64*u + lane
  constexpr int G = 8;                 // slots per group
  static_assert(kCapLong % kWave == 0 && U % G == 0, "whole list rows and groups");
  const int lane = lane_id();
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  // Slots go in groups of G; the groups past the list are skipped by uniform branches, and within
  // a group nothing branches, so that the LDS reads of a group issue back to back and wait once.
  // The pad entries of the last group (past cnt) hold key 0: they take part in a level only if
  // key 0 matches its prefix, and each histogram then takes them back out of bin 0.
  const int ng = (cnt + G * kWave - 1) / (G * kWave);
  const uint32_t pad = static_cast<uint32_t>(G * kWave * ng - cnt);
  uint32_t v[U];
  uint32_t o = 0u, a = 0xffffffffu;
#pragma unroll
  for (int g = 0; g < U / G; ++g) {
    if (g < ng) {
#pragma unroll
      for (int i = 0; i < G; ++i) v[G * g + i] = list[min(kWave * (G * g + i) + lane, cnt - 1)];
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
  wave_lds_sync();  // every key is in registers before the copies below overwrite the list
  // entries [256j, 256j + 256) of idxs to list + 256j; they land while the radix levels run
  for (int j = 0; 256 * j < cnt; ++j) copy16_to_lds(idxs + 256 * j + 4 * lane, list + 256 * j);
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
  // Stable compaction in place, a group at a time: the group's indices are read before any of its
  // kept entries is written, and a kept entry moves to a slot at or below its own, so no entry is
  // overwritten before it is read.
  wait_vmem();
  int kept = 0;
  if (whole_bin && cur != 0u) {
    // keep exactly the entries >= cur (the bits of cur below lo are zero, so (v & hi_mask(lo)) >=
    // cur exactly when v >= cur); the pad keys (0) are below cur
#pragma unroll
    for (int g = 0; g < U / G; ++g) {
      if (g < ng) {
        uint32_t x[G];
#pragma unroll
        for (int i = 0; i < G; ++i) x[i] = list[kWave * (G * g + i) + lane];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const bool keep = v[G * g + i] >= cur;
          const uint64_t mk = ballot(keep);
          if (keep) list[kept + lanes_below(mk)] = x[i];
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
        uint32_t x[G];
#pragma unroll
        for (int i = 0; i < G; ++i) x[i] = list[kWave * (G * g + i) + lane];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          const int u = G * g + i;
          const bool in = kWave * u + lane < cnt;
          const uint32_t vh = v[u] & hm;
          const bool eq = in && vh == cur;
          const uint64_t me = ballot(eq);
          const bool keep = (in && vh > cur) || (eq && eq_seen + lanes_below(me) < need);
          const uint64_t mk = ballot(keep);
          if (keep) list[kept + lanes_below(mk)] = x[i];
          kept += __popcll(mk);
          eq_seen += __popcll(me);
        }
      }
    }
  }
  wave_lds_sync();
  if ((k & 3) == 0) {  // rows of out are 16-byte aligned
    for (int e = 4 * lane; e < k; e += 4 * kWave)
      *reinterpret_cast<u32x4*>(out + e) = *reinterpret_cast<const DSA_LDS u32x4*>(list + e);
  } else {
    for (int e = lane; e < k; e += kWave) out[e] = static_cast<int32_t>(list[e]);
  }
}

// F8: the FP8 indexer (E4M3 operands with power-of-two row scales, v_mfma_scale_f32_32x32x64_f8f6f4);
// otherwise BF16 operands on v_mfma_f32_32x32x16_bf16. Everything after the scores is shared.
template <int H_I, int D_I, bool F8>
__global__ __launch_bounds__(kIdxRows * kWave, 1) void k_index_topk(IndexArgs a) {
  constexpr int MT = (H_I + 31) / 32;   // 32-row M tiles of indexer heads
  constexpr int KS = F8 ? D_I / 64 : D_I / 16;  // MFMA K steps
  constexpr int GPR = F8 ? D_I / 16 : D_I / 8;  // 16-byte granules per key row
  constexpr int CHUNK_GRAN = kChunk * GPR;
  constexpr int CPW = CHUNK_GRAN / (kIdxRows * kWave);  // wave copies (1 KB operand blocks) per chunk and wave
  // a 32-key tile's K step is one 1 KB block (BF16: 16 bytes per lane) or two (FP8: 32 bytes per lane)
  static_assert(CHUNK_GRAN % (kIdxRows * kWave) == 0 && (F8 ? 4 : 2) * KS * kWave == CHUNK_GRAN, "chunk copy split");
  using QOp = typename std::conditional<F8, i32x8, bf16x8>::type;

  __shared__ __attribute__((aligned(256))) uint16_t stage[2][kChunk * D_I];
  __shared__ __attribute__((aligned(16))) uint32_t s_keys[kIdxRows * kListSlots];  // candidate score keys (token indices: global)
  __shared__ uint32_t s_hist[3 * 256];
  // Candidate count of a row whose list must be compacted, else 0. Step c reads buffer c % 2 after
  // its barrier while appends of that step write buffer (c + 1) % 2, so no wave can see a flag
  // that another wave of the same step has not seen.
  __shared__ __attribute__((aligned(16))) int s_need[2][kIdxRows];
  __shared__ int s_lbase[kIdxRows];               // first LDS slot of each wave's list
  __shared__ uint32_t s_sel[4 * kIdxRows];        // selection scratch
  __shared__ __attribute__((aligned(16))) float s_w[kIdxRows][MT * 32];  // head weights of each row (0 past H_I)

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
  // The lists of waves w and w + 4 share 2 * kListSlots slots; kCap each, unless a paired long row
  // has more keys than that and its short partner fits in kCapShort.
  const int pair_base = 2 * (wave & 3) * kListSlots;
  int lbase = pair_base + (wave >> 2) * kListSlots, cap = kCap;
  if (a.paired) {
    const int h = (m + 1) >> 1, p = 4 * blk + (wave & 3);
    const int n_long = p < h ? a.row0 + A + (m - 1 - p) - b + 1 : 0;
    const int n_short = p < m - h ? a.row0 + A + p - b + 1 : 0;
    if (n_long > kCap && n_short <= kCapShort) {
      lbase = wave < 4 ? pair_base : pair_base + kCapLong + 64;
      cap = wave < 4 ? kCapLong : kCapShort;
    }
  }
  if (lane == 0) {
    s_need[0][wave] = 0;
    s_need[1][wave] = 0;
    s_lbase[wave] = lbase;
  }
  // Claim a candidate slot for the workgroup's lists of token indices. At most n_slots workgroups
  // are resident at once (the host checks this before the launch) and each frees its slot before
  // it ends, so a free slot always exists; the search is still bounded, and a workgroup that finds
  // none writes -1 rows instead of touching memory it does not own.
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
  const int slot = s_slot;
  if (slot < 0) {
    if (select)
      for (int j = lane; j < k; j += kWave) out[j] = -1;
    return;  // uniform over the workgroup
  }
  const int kb = b, ke = a.row0 + A + i_top + 1;

  // Query operand (A): rows = heads (zero beyond H_I), K = indexer dims; kept in AGPRs, which
  // the MFMAs read directly. Head weights go to LDS, read back by the score epilogue.
  // FP8: 32 bytes per lane and K step, K values 64*s + 32*(lane/32) .. +32 of its head (the key
  // operand takes the same K values, so the pairing does not depend on the instruction's K order);
  // the head's scale goes into its weight.
  QOp qa[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = 32 * mt + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (select && head < H_I) {
        if constexpr (F8) {
          const uint8_t* src = a.q8 + (static_cast<int64_t>(r) * H_I + head) * D_I + 64 * s + 32 * (lane >> 5);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(src), hi = *reinterpret_cast<const i32x4*>(src + 16);
          qa[mt][s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          qa[mt][s] = *reinterpret_cast<const bf16x8*>(a.q_I + (static_cast<int64_t>(r) * H_I + head) * D_I + 16 * s + 8 * (lane >> 5));
        }
      } else {
        qa[mt][s] = QOp{};
      }
    }
    if (lane < 32) {
      float wv = 0.0f;
      if (select && head < H_I) {
        wv = bf16_to_f32(a.w[static_cast<int64_t>(r) * H_I + head]);
        if constexpr (F8) wv *= a.sq[static_cast<int64_t>(r) * H_I + head];  // a power of two: exact
      }
      s_w[wave][32 * mt + lane] = wv;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(qa[mt][s]));

  // LDS-typed pointers, so that every access is a ds_ instruction; candidate indices in global memory
  DSA_LDS uint32_t* keys = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_keys[lbase])));
  DSA_LDS uint32_t* hist = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_hist[0])));
  DSA_LDS uint32_t* sel_scratch = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_sel[0])));
  int32_t* cand = a.cand + (static_cast<int64_t>(slot) * kIdxRows + wave) * kCandStride;
  int cnt = 0;
  uint32_t thr = 0u;

  // Every wave selects for the rows that asked (rare): all waves of the workgroup share the work.
  auto run_selections = [&](int slack, int nbuf) {
    for (int rw = 0; rw < kIdxRows; ++rw) {
      const int c_rw = s_need[nbuf][rw];
      if (c_rw == 0) continue;  // uniform: every wave reads the same flag
      DSA_LDS uint32_t* kr = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_keys[s_lbase[rw]])));
      int32_t* cr = a.cand + (static_cast<int64_t>(slot) * kIdxRows + rw) * kCandStride;
      int kept = 0;
      const uint32_t th = wg_select_topk<kIdxRows>(kr, cr, hist, sel_scratch, c_rw, k, slack, &kept);
      if (rw == wave) {
        cnt = kept;
        thr = th;
      }
    }
    barrier_lds();  // every wave has read the flags
    if (lane == 0) s_need[nbuf][wave] = 0;
  };

  const int nchunks = (ke - kb + kChunk - 1) / kChunk;
  const uint16_t* __restrict__ LNk = a.LNk;

  // A staged chunk is laid out by MFMA operand: block n*KS + s (1 KB) holds, at lane i's 16 bytes,
  // granule 2s + i/32 of key 32n + i%32, i.e. the B operand of K step s of 32-key tile n. Operand
  // reads are then whole 1 KB blocks at constant offsets (bank-conflict free) and every copy fills
  // one block. Copy j of this wave fills block CPW*wave + j; its per-lane source offset within a
  // chunk is fixed, the chunk's first key row a scalar base.
  // FP8: block (n, s, h) = 4 * ... holds, at lane i's 16 bytes, half h of lane i's 32-byte operand of
  // K step s of tile n: key 32n + i%32, K bytes 64s + 32(i/32) + 16h .. +16.
  uint32_t cp_off[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int blk_j = CPW * wave + j;
    if constexpr (F8) {
      const int n = blk_j / (2 * KS), st = (blk_j % (2 * KS)) >> 1, hf = blk_j & 1;
      cp_off[j] = static_cast<uint32_t>((32 * n + (lane & 31)) * D_I + 64 * st + 32 * (lane >> 5) + 16 * hf);
    } else {
      const int n = blk_j / KS, st = blk_j % KS;
      cp_off[j] = static_cast<uint32_t>(((32 * n + (lane & 31)) * D_I + 8 * (2 * st + (lane >> 5))) * 2);
    }
  }
  // A chunk may reach past the last key row (up to two chunks past it, see kIdxKeyPad): those rows
  // of the padded LNk are staged but never scored.
  auto issue_copy = [&](int c, int j) {
    const int K0 = kb + c * kChunk;
    const uint32_t lds = lds_addr_of(stage[c & 1]) + 1024 * (CPW * wave + j);
    if constexpr (F8) copy16_to_lds_imm<0>(a.LNk8 + static_cast<int64_t>(K0) * D_I, cp_off[j], lds);
    else copy16_to_lds_imm<0>(LNk + static_cast<int64_t>(K0) * D_I, cp_off[j], lds);
  };
  auto issue_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) issue_copy(c, j);
  };
  // Scores of a chunk come from two 32-key N tiles (K = d_I): tile 0 into accA, tile 1 into accB.
  // The loop is software pipelined by half a chunk: the MFMAs of one tile run interleaved with
  // the VALU epilogue of the tile before it (ReLU, head weight, partial head sums), so the matrix
  // core and the vector ALU work at the same time. Step c runs tile 0 of chunk c beside the
  // epilogue of tile 1 of chunk c-1, then tile 1 of chunk c beside the epilogue of tile 0 of
  // chunk c and the append of chunk c-1.
  f32x16 accA[MT], accB[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) accB[mt] = f32x16{};  // the epilogue of "chunk -1" adds nothing
  // Head weights in registers: element 4*g + e of an accumulator tile mt holds head
  // 32*mt + 8*g + 4*(lane/32) + e.
  f32x4 w4[MT][4];
  {
    const DSA_LDS float* wrow = reinterpret_cast<const DSA_LDS float*>(lds_ptr(lds_addr_of(&s_w[wave][0])));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g) w4[mt][g] = *reinterpret_cast<const DSA_LDS f32x4*>(wrow + 32 * mt + 8 * g + 4 * (lane >> 5));
  }
  constexpr int kEl = MT * 16;        // accumulator elements per lane of one N tile
  constexpr int kEps = kEl / KS;      // epilogue elements per K step
  static_assert(kEl % KS == 0 && kEps >= 1 && kEps <= (F8 ? 16 : 8), "epilogue split");
  constexpr int kPf = KS < 2 ? KS : 2;  // key operands are read kPf K steps ahead of their MFMAs
  // One N tile of chunk c into acc, interleaved with the epilogue of `prev`; returns this lane's
  // partial sum over its heads of the previous tile (one key column per lane).
  auto tile_step = [&](int c, int n, f32x16 (&acc)[MT], const f32x16 (&prev)[MT], auto&& side) -> float {
    // the operand of K step s of tile n: block n*KS + s of the staged chunk, 16 bytes per lane
    uint32_t a0 = lds_addr_of(stage[c & 1]) + n * (KS * 1024) + 16 * lane;
    asm volatile("" : "+v"(a0));
    bf16x8 bk[kPf];
#pragma unroll
    for (int s = 0; s < kPf; ++s) bk[s] = lds_read16(lds_ptr(a0 + 1024 * s));
    float part[kEps];
#pragma unroll
    for (int j = 0; j < kEps; ++j) part[j] = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if constexpr (!F8) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][s], bk[s % kPf], s == 0 ? f32x16{} : acc[mt], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < kEps; ++j) {
        const int el = s * kEps + j, mt = el / 16, i = el % 16;
        part[j] = __builtin_fmaf(w4[mt][i / 4][i % 4], relu(prev[mt][i]), part[j]);
      }
      // keep this step's share of the epilogue in this step (IR passes would sink it below the MFMAs)
#pragma unroll
      for (int j = 0; j < kEps; ++j) asm volatile("" : "+v"(part[j]));
      if (s + kPf < KS) bk[s % kPf] = lds_read16(lds_ptr(a0 + 1024 * (s + kPf)));
      side(s);  // branch-free work of the caller, scheduled beside this step's MFMAs
      // one MFMA, then half of the epilogue, the other MFMA(s), the other half, the next read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MT - 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps + 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    float p = part[0];
#pragma unroll
    for (int j = 1; j < kEps; ++j) p += part[j];
    return p;
  };
  // The FP8 form of tile_step: the tile's two K steps read as four 1 KB blocks at once, each K step
  // one 32x32x64 MFMA per M tile beside its half of the epilogue (kept in four partial sums).
  auto tile_step8 = [&](int c, int n, f32x16 (&acc)[MT], const f32x16 (&prev)[MT], auto&& side) -> float {
    uint32_t a0 = lds_addr_of(stage[c & 1]) + n * (2 * KS * 1024) + 16 * lane;
    asm volatile("" : "+v"(a0));
    i32x8 bk[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const i32x4 lo = __builtin_bit_cast(i32x4, lds_read16(lds_ptr(a0 + 2048 * s)));
      const i32x4 hi = __builtin_bit_cast(i32x4, lds_read16(lds_ptr(a0 + 2048 * s + 1024)));
      bk[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    constexpr int NP = 4;
    float part[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) part[j] = 0.0f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (F8) acc[mt] = mfma32_fp8(qa[mt][s], bk[s], s == 0 ? f32x16{} : acc[mt]);
      }
#pragma unroll
      for (int j = 0; j < kEps; ++j) {
        const int el = s * kEps + j, mt = el / 16, i = el % 16;
        part[j % NP] = __builtin_fmaf(w4[mt][i / 4][i % 4], relu(prev[mt][i]), part[j % NP]);
      }
#pragma unroll
      for (int j = 0; j < NP; ++j) asm volatile("" : "+v"(part[j]));
      side(s);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MT - 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kEps + 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return (part[0] + part[1]) + (part[2] + part[3]);
  };
  // The epilogue of `prev` alone (a row's last chunk, or a wave whose row has ended).
  auto tile_drain = [&](const f32x16 (&prev)[MT]) -> float {
    float part[kEps];
#pragma unroll
    for (int j = 0; j < kEps; ++j) part[j] = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int j = 0; j < kEps; ++j) {
        const int el = s * kEps + j, mt = el / 16, i = el % 16;
        part[j] = __builtin_fmaf(w4[mt][i / 4][i % 4], relu(prev[mt][i]), part[j]);
      }
    float p = part[0];
#pragma unroll
    for (int j = 1; j < kEps; ++j) p += part[j];
    return p;
  };
  // lanes < 32 hold key lane of tile 0 in p0 and of tile 1 in p1 (heads with lane/32 = 0), lanes
  // >= 32 the other heads: one swap leaves lane l with the full score of key l of the chunk
  auto join = [](float p0, float p1) -> float {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  };
  // Append the keys of chunk c that reach the threshold: keys to LDS, token indices to global, in
  // ascending token order. Branch-free, so that it can sit between MFMAs: lanes that do not take
  // their key write it to a slot past the list. A list that may not take another chunk while the
  // row still has keys in chunk c + 1 raises its flag for the next step.
  auto append = [&](int c, float score, int nbuf) {
    const int s_key = kb + c * kChunk + lane;
    const uint32_t key = score_key(score);
    const bool take = select && s_key >= b && s_key <= t && key >= thr;
    const uint64_t msk = ballot(take);
    const int pos = take ? cnt + lanes_below(msk) : cap + lane;
    keys[pos] = key;
    cand[pos] = s_key;
    cnt += __popcll(msk);
    const bool more = kb + (c + 1) * kChunk <= t;
    s_need[nbuf][wave] = cnt > cap - kChunk && more ? cnt : 0;  // every lane writes the same value
  };

  auto tile = [&](int c, int n, f32x16 (&acc)[MT], const f32x16 (&prev)[MT], auto&& side) -> float {
    if constexpr (F8) return tile_step8(c, n, acc, prev, side);
    else return tile_step(c, n, acc, prev, side);
  };
  float p0_prev = 0.0f;  // tile-0 partial sums of the previous chunk
  // FP8: the key scales of the previous chunk (lane l: key l), loaded a step before they are used
  float sk_prev = 1.0f;
  issue_chunk(0);
  // Step c: tile 0 of chunk c (the next chunk's copies issued between its MFMAs), then the
  // selections that the lists filled by step c-1 asked for, then tile 1 of chunk c with the append
  // of chunk c-1 between its MFMAs. Step nchunks runs no MFMAs: it only finishes the last chunk.
  for (int c = 0; c <= nchunks; ++c) {
    wait_vmem();    // this wave's copies of chunk c and its index stores are complete
    barrier_lds();  // chunk c has landed; the slot of chunk c-1 is free
    // flags of the lists that step c-1 filled: read now, used after tile 0
    const i32x4 f0 = *reinterpret_cast<const DSA_LDS i32x4*>(lds_ptr(lds_addr_of(&s_need[c & 1][0])));
    const i32x4 f1 = *reinterpret_cast<const DSA_LDS i32x4*>(lds_ptr(lds_addr_of(&s_need[c & 1][4])));
    const bool act = select && c < nchunks && kb + c * kChunk <= t;      // row still has keys in chunk c
    const bool act_prev = select && c > 0 && kb + (c - 1) * kChunk <= t;  // chunk c-1 still to finish
    // copies of chunk c+1 (at c+1 == nchunks they fill a free slot with clamped rows, unused)
    auto copies = [&](int st) {
      if (st < CPW) issue_copy(c + 1, st);
    };
    float sk_cur = 1.0f;
    if constexpr (F8) {
      if (c < nchunks) sk_cur = a.sk[kb + c * kChunk + lane];  // within the padded key rows
    }
    float score_prev = 0.0f;
    if (act) {
      // a wave whose row ends before this chunk leaves its SIMD to the other wave there
      score_prev = join(p0_prev, tile(c, 0, accA, accB, copies));
      if constexpr (F8) score_prev *= sk_prev;  // a power of two: exact
    } else if (c + 1 < nchunks) {
#pragma unroll
      for (int j = 0; j < CPW; ++j) issue_copy(c + 1, j);
    }
    if ((f0[0] | f0[1] | f0[2] | f0[3] | f1[0] | f1[1] | f1[2] | f1[3]) != 0)
      run_selections(kSelSlack, c & 1);  // uniform, rare
    if (act) {
      auto app = [&](int st) {
        if (st == 0) append(c - 1, score_prev, (c + 1) & 1);  // early, so its index stores land before the next step's wait
      };
      p0_prev = tile(c, 1, accB, accA, app);
    } else if (act_prev) {
      float sc = join(p0_prev, tile_drain(accB));
      if constexpr (F8) sc *= sk_prev;
      append(c - 1, sc, (c + 1) & 1);
    }
    sk_prev = sk_cur;
  }

  // Final exact selection: each wave finishes its own row, with a histogram in the staging ring,
  // which no wave uses any more.
  wait_vmem();    // this wave's candidate index stores are complete
  barrier_lds();  // every wave is done with the staging ring
  if (select) {
    if (cnt > k) {
      DSA_LDS uint32_t* whist = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(stage[0]) + 1024 * wave));
      wave_select_out(keys, cand, whist, cnt, k, out);
    } else {  // exactly k candidates
      for (int j = lane; j < k; j += kWave) out[j] = cand[j];
    }
  }
  // Free the slot once every wave's reads of its token indices have completed.
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicExch(a.slot_flags + slot, 0);
  }
}

// ---------------------------------------------------------------------------------------------
static_assert(kIdxSlotWords == kIdxRows * kCandStride, "slot size");

int index_blocks(int m, int paired) { return paired ? ((m + 1) / 2 + 3) / 4 : (m + kIdxRows - 1) / kIdxRows; }

// Workgroups of the indexer kernel that the current device can hold at once (CUs x occupancy),
// computed once per device.
static const void* index_kernel(int v) {
  switch (v) {
    case 0: return reinterpret_cast<const void*>(k_index_topk<64, 128, false>);
    case 1: return reinterpret_cast<const void*>(k_index_topk<4, 64, false>);
    default: return reinterpret_cast<const void*>(k_index_topk<64, 128, true>);
  }
}

static int index_resident_blocks(int v) {
  static std::mutex mu;
  static int cached[3][64] = {};
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

hipError_t launch_index_topk(const IndexArgs& a, int H_I, int d_I, bool fp8, hipStream_t st) {
  if (a.nseg < 1 || a.nseg > kIdxMaxSeg || a.n_slots < 1) return hipErrorInvalidValue;
  const bool big = H_I == 64 && d_I == 128;
  if (fp8 && !big) return hipErrorInvalidValue;
  const int v = fp8 ? 2 : (big ? 0 : 1);
  const int resident = index_resident_blocks(v);
  if (resident < 1 || resident > a.n_slots) return hipErrorInvalidConfiguration;  // slots could run out
  dim3 grid(a.seg_blk0[a.nseg]), block(kIdxRows * kWave);
  if (v == 2) hipLaunchKernelGGL((k_index_topk<64, 128, true>), grid, block, 0, st, a);
  else if (v == 0) hipLaunchKernelGGL((k_index_topk<64, 128, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_index_topk<4, 64, false>), grid, block, 0, st, a);
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
                                 uint16_t* LNk, const IndexArgs& a, hipStream_t st) {
  const int nln = (a.T + 3) / 4;
  const int nfill = a.nrows < 2048 ? a.nrows : 2048;
  dim3 grid(nln + nfill), block(256);
  if (d_I == 128) hipLaunchKernelGGL((k_index_prologue<128>), grid, block, 0, st, k_I, gamma, beta, eps, LNk, a, nln);
  else hipLaunchKernelGGL((k_index_prologue<64>), grid, block, 0, st, k_I, gamma, beta, eps, LNk, a, nln);
  return hipGetLastError();
}

}  // namespace dsa

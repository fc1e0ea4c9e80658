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
// Kernel design (one wave per query row, four rows per workgroup, rows taken longest first):
//  - The LNk keys of the workgroup's causal range stream through LDS in chunks of 64 keys
//    (asynchronous 16-byte global->LDS copies, double buffered, XOR-swizzled granules so the
//    MFMA operand reads are bank-conflict free).
//  - Scores: v_mfma_f32_32x32x16_bf16 with the indexer heads as M (q_I of the row held in
//    registers), 32 keys as N and d_I as K. Each lane then owns one key column: ReLU, the head
//    weight and the sum over heads happen in registers, and one permlane32 swap joins the two
//    half-waves, leaving one full score per lane for 64 consecutive keys.
//  - Top-k: scores become order-preserving uint32 keys. A key is appended to the row's LDS
//    candidate list when it reaches the running threshold (ballot + mbcnt compaction, so the list
//    stays in ascending token order). When the list nears capacity, a radix select over the
//    candidates' varying bits (LDS histograms, wave prefix sums) finds the k-th key and a stable
//    ballot compaction keeps exactly k (ties to the lower index), which also raises the threshold.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

// ---------------------------------------------------------------------------------------------
// Key LayerNorm: one wave per key row, double precision, one rounding to bf16.
template <int D_I>
__global__ __launch_bounds__(256) void k_key_layernorm(const uint16_t* __restrict__ k_I, const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, double eps, int T,
                                                       uint16_t* __restrict__ LNk) {
  constexpr int PER = D_I / kWave;
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
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
constexpr int kIdxRows = 4;       // query rows per workgroup (two waves each)
constexpr int kChunk = 64;        // keys per LDS chunk (two 32-key MFMA tiles)
constexpr int kIdxRing = 3;       // staged chunks (copies run two chunks ahead)
constexpr int kCap = 3328;        // candidate capacity per row (>= k + 2 * kChunk for k <= 2048)
constexpr int kSelSlack = 256;    // extra entries a selection before the end of the row may keep

// Granule (16 bytes) position inside a staged key chunk: rows of GPR granules, XOR-swizzled.
template <int GPR>
__device__ __forceinline__ int stage_granule(int key, int g) {
  const int f = (GPR == 16) ? (key & 15) : ((key >> 1) & 7);
  return key * GPR + (g ^ f);
}

// max(x, +0) as an integer max on the bit pattern: negative values and -0 (sign bit set) give +0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ uint32_t hi_mask(int lo) { return lo >= 32 ? 0u : ~((1u << lo) - 1u); }

// Wave-wide inclusive suffix sum (lane i gets the sum over lanes i..63).
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t y = __shfl_down(x, off);
    if (lane + off < kWave) x += y;
  }
  return x;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x &= __shfl_xor(x, o);
  return x;
}

// Keep the k best of a row's cnt candidates (keys desc, then list order = ascending token index).
// Every wave of the workgroup takes part (NW waves, each on a slice of the list); the list is
// compacted in place and stays in ascending token order. Returns the new threshold: a future
// candidate must have key >= the returned value to possibly enter the top k.
// With slack > 0 the selection may stop early, at the first radix level whose bin holding the
// k-th key leaves at most `slack` extra entries: then every entry at or above that bin's lower
// bound is kept (at least k) and the bound becomes the threshold, which is still at or below the
// k-th key, so no key of the final top k is dropped. *kept_out receives the number kept.
// scratch: 4*NW words of LDS. Must be called by every thread of the workgroup.
constexpr int kSelU = 8;  // list entries per lane and wave slice (a slice holds kSelU * 64 entries)
template <int NW>
__device__ __forceinline__ uint32_t wg_select_topk(DSA_LDS uint32_t* keys, DSA_LDS int32_t* idxs, DSA_LDS uint32_t* hist,
                                                   DSA_LDS uint32_t* scratch, int cnt, int k, int slack, int* kept_out) {
  static_assert(NW * kWave * kSelU >= kCap, "the wave slices cover the candidate list");
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // This wave's slice of the list: [s0, s0 + kSelU*64), entries s0 + 64*u + lane.
  const int s0 = wave * kWave * kSelU;
  uint32_t v[kSelU];
  bool in[kSelU];
#pragma unroll
  for (int u = 0; u < kSelU; ++u) {
    const int i = s0 + kWave * u + lane;
    in[u] = i < cnt;
    v[u] = in[u] ? keys[i] : 0u;
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
    while (true) {
      const int sh = lo > 8 ? lo - 8 : 0;
      const int nb = lo - sh;
      const uint32_t dmask = (1u << nb) - 1u;
      const uint32_t hm = hi_mask(lo);
      for (int i = threadIdx.x; i < 256; i += NW * kWave) hist[i] = 0u;
      barrier_lds();
#pragma unroll
      for (int u = 0; u < kSelU; ++u)
        if (in[u] && (v[u] & hm) == cur)
          __hip_atomic_fetch_add(hist + ((v[u] >> sh) & dmask), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      barrier_lds();
      // lane owns bins 4*lane .. 4*lane+3; find the bin holding the need-th largest entry (every
      // wave computes the same answer)
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = hist[4 * lane + j];
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
      const int src = __ffsll(static_cast<unsigned long long>(fm)) - 1;
      const int d = __shfl(found, src);
      const uint32_t dab = __shfl(f_above, src);
      const uint32_t dcnt = __shfl(f_cnt, src);
      barrier_lds();  // every wave has read the histogram before it is cleared again
      need -= static_cast<int>(dab);
      cur |= static_cast<uint32_t>(d) << sh;
      lo = sh;
      if (dcnt == static_cast<uint32_t>(need) || sh == 0) break;
      if (static_cast<int>(dcnt) - need <= slack) {  // early stop: keep the whole bin
        need = static_cast<int>(dcnt);
        break;
      }
    }
  }
  // Stable compaction: keep (key_hi > cur) and the first `need` entries with key_hi == cur.
  // Phase 1: per-wave counts; phase 2: each wave writes its kept entries after the kept entries
  // of the waves before it. All entries were read into registers first, so writes cannot
  // overwrite an entry another wave has yet to read.
  const uint32_t hm = hi_mask(lo);
  int32_t x[kSelU];
#pragma unroll
  for (int u = 0; u < kSelU; ++u) x[u] = in[u] ? idxs[s0 + kWave * u + lane] : 0;
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
  barrier_lds();  // the compacted list and the scratch words are free for the next use
  *kept_out = total;
  return lo == 0 ? cur + 1u : cur;
}

template <int H_I, int D_I>
__global__ __launch_bounds__(2 * kIdxRows * kWave, 1) void k_index_topk(IndexArgs a) {
  constexpr int MT = (H_I + 31) / 32;   // 32-row M tiles of indexer heads
  constexpr int KS = D_I / 16;          // MFMA K steps
  constexpr int GPR = D_I / 8;          // 16-byte granules per key row
  constexpr int CHUNK_GRAN = kChunk * GPR;
  constexpr int CPW = CHUNK_GRAN / (kIdxRows * kWave);  // wave copies per chunk and second-half wave
  static_assert(CHUNK_GRAN % (kIdxRows * kWave) == 0, "chunk copy split");

  __shared__ __attribute__((aligned(16))) uint16_t stage[kIdxRing][kChunk * D_I];
  __shared__ uint32_t s_keys[kIdxRows][kCap];
  __shared__ int32_t s_idx[kIdxRows][kCap];
  __shared__ uint32_t s_hist[kIdxRows][256];
  __shared__ float s_xch[kIdxRows][2][32];  // second-half scores of a chunk, handed to the row's first wave
  __shared__ int s_range[2][kIdxRows];
  __shared__ int s_need[kIdxRows];          // candidate count of a row whose list must be compacted, else 0
  __shared__ uint32_t s_sel[4 * 2 * kIdxRows];  // selection scratch

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int slot = wave % kIdxRows;   // the row of this wave
  const int half = wave / kIdxRows;   // 0: keys 0..31 of every chunk and the row's top-k; 1: keys 32..63
  const int k = a.k;

  // Rows are taken from the end (longest causal ranges first).
  const int r = a.nrows - kIdxRows * (blockIdx.x + 1) + slot;
  const bool has_row = r >= 0;
  const int t = a.row0 + r;
  const int b = has_row ? doc_begin(a.cu, a.n_docs, t) : 0;
  const int n = t - b + 1;
  const bool select = has_row && n > k;
  int32_t* out = a.topk_idx + static_cast<int64_t>(r) * k;

  if (half == 0 && has_row && !select) {  // short row: every causal key, then -1
    for (int j = lane; j < k; j += kWave) out[j] = j < n ? b + j : -1;
  }
  if (half == 0 && lane == 0) {
    s_range[0][slot] = select ? b : 0x7fffffff;
    s_range[1][slot] = select ? t + 1 : -1;
    s_need[slot] = 0;
  }
  __syncthreads();
  int kb = 0x7fffffff, ke = -1;
#pragma unroll
  for (int w = 0; w < kIdxRows; ++w) {
    kb = min(kb, s_range[0][w]);
    ke = max(ke, s_range[1][w]);
  }
  if (ke < 0) return;  // uniform: no row of this block needs a selection

  // Query operand (A): rows = heads (zero beyond H_I), K = indexer dims; kept in AGPRs, which
  // the MFMAs read directly. wr: head weight of each accumulator row this lane holds.
  bf16x8 qa[MT][KS];
  float wr[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = 32 * mt + (lane & 31);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (select && head < H_I) {
        qa[mt][s] = *reinterpret_cast<const bf16x8*>(a.q_I + (static_cast<int64_t>(r) * H_I + head) * D_I + 16 * s + 8 * (lane >> 5));
      } else {
        qa[mt][s] = bf16x8{};
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int hr = 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      wr[mt][i] = (select && hr < H_I) ? bf16_to_f32(a.w[static_cast<int64_t>(r) * H_I + hr]) : 0.0f;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+a"(qa[mt][s]));

  // LDS-typed pointers, so that every access is a ds_ instruction
  DSA_LDS uint32_t* keys = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_keys[slot][0])));
  DSA_LDS int32_t* idxs = reinterpret_cast<DSA_LDS int32_t*>(lds_ptr(lds_addr_of(&s_idx[slot][0])));
  DSA_LDS float* xch = reinterpret_cast<DSA_LDS float*>(lds_ptr(lds_addr_of(&s_xch[slot][0][0])));
  DSA_LDS uint32_t* sel_scratch = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_sel[0])));
  int cnt = 0;
  uint32_t thr = 0u;
  // Every wave selects for the rows that asked (rare): all waves of the workgroup share the work.
  auto run_selections = [&](int slack) {
    for (int rw = 0; rw < kIdxRows; ++rw) {
      const int c_rw = s_need[rw];
      if (c_rw == 0) continue;  // uniform: every wave reads the same flag
      DSA_LDS uint32_t* kr = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_keys[rw][0])));
      DSA_LDS int32_t* ir = reinterpret_cast<DSA_LDS int32_t*>(lds_ptr(lds_addr_of(&s_idx[rw][0])));
      DSA_LDS uint32_t* hr = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_hist[rw][0])));
      int kept = 0;
      const uint32_t th = wg_select_topk<2 * kIdxRows>(kr, ir, hr, sel_scratch, c_rw, k, slack, &kept);
      if (rw == slot && half == 0) {
        cnt = kept;
        thr = th;
      }
    }
    barrier_lds();  // every wave has read the flags
    if (half == 0 && lane == 0) s_need[slot] = 0;
  };

  const int nchunks = (ke - kb + kChunk - 1) / kChunk;
  const uint16_t* __restrict__ LNk = a.LNk;
  const int T = a.T;

  // The second-half waves copy the chunks (the first-half waves also keep the row's top-k).
  // Copy j of this wave's share of chunk c: 64 granules, LDS slot P holds granule g = gl ^ f(key)
  // of key P / GPR (the swizzle of stage_granule).
  auto issue_chunk = [&](int c) {
    const int K0 = kb + c * kChunk;
    DSA_LDS uint8_t* base = (DSA_LDS uint8_t*)(stage[c % kIdxRing]);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int P0 = (slot * (CHUNK_GRAN / kIdxRows)) + j * kWave;  // first granule of this wave copy
      const int P = P0 + lane;
      const int key = P / GPR;
      const int gl = P % GPR;
      const int f = (GPR == 16) ? (key & 15) : ((key >> 1) & 7);
      const int g = gl ^ f;
      const int row = min(K0 + key, T - 1);
      copy16_to_lds(LNk + static_cast<int64_t>(row) * D_I + g * 8, base + P0 * 16);
    }
  };
  // Waits for this wave's copies of chunk c; the copies of chunk c+1 may stay in flight.
  auto wait_chunk = [&](int c) {
    if (c + 1 < nchunks) wait_vmem_le<CPW>();
    else wait_vmem_le<0>();
  };
  // Scores of this wave's 32 keys of chunk c (keys 32*half ..): lanes l and l+32 both end with
  // the full score of key 32*half + l%32.
  auto chunk_scores = [&](int c) -> float {
    const DSA_LDS uint8_t* sb = (const DSA_LDS uint8_t*)(stage[c % kIdxRing]);
    const int key = 32 * half + (lane & 31);
    f32x16 acc[MT];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kf = lds_read16(sb + stage_granule<GPR>(key, 2 * s + (lane >> 5)) * 16);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][s], kf, s == 0 ? f32x16{} : acc[mt], 0, 0, 0);
    }
    float p = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) p = __builtin_fmaf(wr[mt][i], relu(acc[mt][i]), p);
    // the two half-waves hold the two halves of the head sum
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  };
  // Append the keys of chunk c that reach the threshold: lanes < 32 hold keys 0..31 (own scores),
  // lanes >= 32 keys 32..63 (the second wave's, read from LDS beforehand).
  auto append = [&](int c, float own, float other) {
    const float score = lane < 32 ? own : other;
    const int s_key = kb + c * kChunk + lane;
    const uint32_t key = score_key(score);
    const bool take = select && s_key >= b && s_key <= t && key >= thr;
    const uint64_t msk = ballot(take);
    if (take) {
      const int pos = cnt + lanes_below(msk);
      keys[pos] = key;
      idxs[pos] = s_key;
    }
    cnt += __popcll(msk);
    // a full list is compacted at the start of the next step, before the next append
    if (cnt > kCap - kChunk && lane == 0) s_need[slot] = cnt;
  };

  if (half == 1) {
    issue_chunk(0);
    if (nchunks > 1) issue_chunk(1);
  }
  float prev = 0.0f;
  for (int c = 0; c <= nchunks; ++c) {
    if (half == 1 && c < nchunks) wait_chunk(c);
    barrier_lds();  // chunk c has landed; the slot of chunk c-1 is free; chunk c-1's hand-over is visible
    if (s_need[0] | s_need[1] | s_need[2] | s_need[3]) run_selections(kSelSlack);  // uniform, rare
    if (half == 1 && c + 2 < nchunks) issue_chunk(c + 2);
    // the hand-over is read before this chunk's MFMAs, so its latency is hidden under them
    const float other = (half == 0 && c > 0) ? xch[((c - 1) & 1) * 32 + (lane & 31)] : 0.0f;
    float cur = 0.0f;
    if (c < nchunks) cur = chunk_scores(c);
    if (half == 1) {
      if (c < nchunks && lane < 32) xch[(c & 1) * 32 + lane] = cur;
    } else if (c > 0) {
      append(c - 1, prev, other);
    }
    prev = cur;
  }

  // Final exact selections (every wave takes part), then each row's first wave writes the row.
  if (half == 0 && lane == 0) s_need[slot] = (select && cnt > k) ? cnt : 0;
  barrier_lds();
  run_selections(0);
  if (half == 0 && select) {
    for (int j = lane; j < k; j += kWave) out[j] = idxs[j];
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_key_layernorm(const uint16_t* k_I, const float* gamma, const float* beta, double eps, int T, int d_I,
                                uint16_t* LNk, hipStream_t st) {
  dim3 grid((T + 3) / 4), block(256);
  if (d_I == 128) hipLaunchKernelGGL((k_key_layernorm<128>), grid, block, 0, st, k_I, gamma, beta, eps, T, LNk);
  else hipLaunchKernelGGL((k_key_layernorm<64>), grid, block, 0, st, k_I, gamma, beta, eps, T, LNk);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexArgs& a, int H_I, int d_I, hipStream_t st) {
  dim3 grid((a.nrows + kIdxRows - 1) / kIdxRows), block(2 * kIdxRows * kWave);
  if (H_I == 64 && d_I == 128) hipLaunchKernelGGL((k_index_topk<64, 128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_index_topk<4, 64>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

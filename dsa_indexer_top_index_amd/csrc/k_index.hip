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

#include <type_traits>
#include <utility>

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
constexpr int kIdxWaves = 4;      // query rows per workgroup
constexpr int kChunk = 64;        // keys per LDS chunk (two 32-key MFMA tiles)
constexpr int kIdxRing = 3;       // staged chunks (copies run two chunks ahead)
constexpr int kCap = 3328;        // candidate capacity per row (>= k + 2 * kChunk for k <= 2048)

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

// Keep the k best of the cnt candidates (keys desc, then list order = ascending token index).
// The list is compacted in place and stays in ascending token order. Returns the new threshold:
// every future candidate must have key >= the returned value to possibly enter the top k.
// Every pass reads kSelU entries per lane before using them, so a pass over the list costs a few
// LDS latencies rather than one per 64 entries.
constexpr int kSelU = 8;
__device__ __forceinline__ uint32_t wave_select_topk(DSA_LDS uint32_t* keys, DSA_LDS int32_t* idxs, DSA_LDS uint32_t* hist,
                                                     int cnt, int k) {
  const int lane = lane_id();
  uint32_t o = 0u, a = 0xffffffffu;
  for (int base = 0; base < cnt; base += kWave * kSelU) {
    uint32_t v[kSelU];
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const int i = base + kWave * u + lane;
      v[u] = i < cnt ? keys[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const bool in = base + kWave * u + lane < cnt;
      o |= v[u];
      a &= in ? v[u] : 0xffffffffu;
    }
  }
  o = wave_or(o);
  a = wave_and(a);
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
      for (int i = lane; i < 256; i += kWave) hist[i] = 0u;
      wave_lds_sync();
      for (int base = 0; base < cnt; base += kWave * kSelU) {
        uint32_t v[kSelU];
#pragma unroll
        for (int u = 0; u < kSelU; ++u) {
          const int i = base + kWave * u + lane;
          v[u] = i < cnt ? keys[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kSelU; ++u) {
          const bool in = base + kWave * u + lane < cnt;
          if (in && (v[u] & hm) == cur) __hip_atomic_fetch_add(hist + ((v[u] >> sh) & dmask), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        }
      }
      wave_lds_sync();
      // lane owns bins 4*lane .. 4*lane+3; find the bin holding the need-th largest entry
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
      need -= static_cast<int>(dab);
      cur |= static_cast<uint32_t>(d) << sh;
      lo = sh;
      if (dcnt == static_cast<uint32_t>(need) || sh == 0) break;
    }
  }
  // Stable compaction: keep (key_hi > cur) and the first `need` entries with key_hi == cur.
  // Entries are written at or below their own position, so reading ahead is safe.
  const uint32_t hm = hi_mask(lo);
  int kept = 0, eq_seen = 0;
  for (int base = 0; base < cnt; base += kWave * kSelU) {
    uint32_t v[kSelU];
    int32_t x[kSelU];
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const int i = base + kWave * u + lane;
      v[u] = i < cnt ? keys[i] : 0u;
      x[u] = i < cnt ? idxs[i] : 0;
    }
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < kSelU; ++u) {
      const bool in = base + kWave * u + lane < cnt;
      const uint32_t vh = v[u] & hm;
      const bool gt = in && vh > cur;
      const bool eq = in && vh == cur;
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
    wave_lds_sync();
  }
  return lo == 0 ? cur + 1u : cur;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void idx_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void idx_static_for(F&& f) {
  idx_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int H_I, int D_I>
__global__ __launch_bounds__(256, 1) void k_index_topk(IndexArgs a) {
  constexpr int MT = (H_I + 31) / 32;   // 32-row M tiles of indexer heads
  constexpr int KS = D_I / 16;          // MFMA K steps
  constexpr int GPR = D_I / 8;          // 16-byte granules per key row
  constexpr int CHUNK_GRAN = kChunk * GPR;
  constexpr int CPW = CHUNK_GRAN / (kIdxWaves * kWave);  // wave copies per chunk and wave
  constexpr int NMF = MT * 2 * KS;      // MFMAs per chunk
  constexpr int NEL = MT * 2 * 16;      // score elements per lane per chunk
  constexpr int NMICRO = NEL / 2 + 2;   // epilogue micro-steps per chunk
  static_assert(CHUNK_GRAN % (kIdxWaves * kWave) == 0, "chunk copy split");

  __shared__ __attribute__((aligned(16))) uint16_t stage[kIdxRing][kChunk * D_I];
  __shared__ uint32_t s_keys[kIdxWaves][kCap];
  __shared__ int32_t s_idx[kIdxWaves][kCap];
  __shared__ uint32_t s_hist[kIdxWaves][256];
  __shared__ int s_range[2][kIdxWaves];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int k = a.k;

  // Rows are taken from the end (longest causal ranges first).
  const int r = a.nrows - kIdxWaves * (blockIdx.x + 1) + wave;
  const bool has_row = r >= 0;
  const int t = a.row0 + r;
  const int b = has_row ? doc_begin(a.cu, a.n_docs, t) : 0;
  const int n = t - b + 1;
  const bool select = has_row && n > k;
  int32_t* out = a.topk_idx + static_cast<int64_t>(r) * k;

  if (has_row && !select) {  // short row: every causal key, then -1
    for (int j = lane; j < k; j += kWave) out[j] = j < n ? b + j : -1;
  }
  if (lane == 0) {
    s_range[0][wave] = select ? b : 0x7fffffff;
    s_range[1][wave] = select ? t + 1 : -1;
  }
  __syncthreads();
  int kb = 0x7fffffff, ke = -1;
#pragma unroll
  for (int w = 0; w < kIdxWaves; ++w) {
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
  DSA_LDS uint32_t* keys = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_keys[wave][0])));
  DSA_LDS int32_t* idxs = reinterpret_cast<DSA_LDS int32_t*>(lds_ptr(lds_addr_of(&s_idx[wave][0])));
  DSA_LDS uint32_t* hist = reinterpret_cast<DSA_LDS uint32_t*>(lds_ptr(lds_addr_of(&s_hist[wave][0])));
  int cnt = 0;
  uint32_t thr = 0u;

  const int nchunks = (ke - kb + kChunk - 1) / kChunk;
  const uint16_t* __restrict__ LNk = a.LNk;
  const int T = a.T;

  // Copy j of this wave's share of chunk c: 64 granules, LDS slot P holds granule g = gl ^ f(key)
  // of key P / GPR (the swizzle of stage_granule).
  auto issue_copy = [&](int c, int j) {
    const int K0 = kb + c * kChunk;
    DSA_LDS uint8_t* base = (DSA_LDS uint8_t*)(stage[c % kIdxRing]);
    const int P0 = (wave * (CHUNK_GRAN / kIdxWaves)) + j * kWave;  // first granule of this wave copy
    const int P = P0 + lane;
    const int key = P / GPR;
    const int gl = P % GPR;
    const int f = (GPR == 16) ? (key & 15) : ((key >> 1) & 7);
    const int g = gl ^ f;
    const int row = min(K0 + key, T - 1);
    copy16_to_lds(LNk + static_cast<int64_t>(row) * D_I + g * 8, base + P0 * 16);
  };
  auto issue_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) issue_copy(c, j);
  };
  // Waits for this wave's copies of chunk c; the copies of chunk c+1 may stay in flight.
  auto wait_chunk = [&](int c) {
    if (c + 1 < nchunks) wait_vmem_le<CPW>();
    else wait_vmem_le<0>();
  };

  // Chunk c's scores: two 32-key N tiles, K = d_I. acc[mt][nb]: heads 32*mt.., keys 32*nb..
  auto mfma_step = [&](int c, int i, f32x16 (&acc)[MT][2], bf16x8 (&kb0)[KS], bf16x8 (&kb1)[KS]) {
    const int s = i / (2 * MT), rem = i % (2 * MT), nb = rem / MT, mt = rem % MT;
    const bf16x8& bb = nb == 0 ? kb0[s] : kb1[s];
    acc[mt][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][s], bb, s == 0 ? f32x16{} : acc[mt][nb], 0, 0, 0);
  };
  auto load_b = [&](int c, int s, bf16x8 (&kb0)[KS], bf16x8 (&kb1)[KS]) {
    const DSA_LDS uint8_t* sb = (const DSA_LDS uint8_t*)(stage[c % kIdxRing]);
    const int g = 2 * s + (lane >> 5);
    kb0[s] = lds_read16(sb + stage_granule<GPR>(lane & 31, g) * 16);
    kb1[s] = lds_read16(sb + stage_granule<GPR>(32 + (lane & 31), g) * 16);
  };
  // Epilogue of a chunk in micro-steps: ReLU, head weight and head sum (two elements a step),
  // then the join of the half-waves and the append of the keys that reach the threshold.
  float p0 = 0.0f, p1 = 0.0f;
  auto micro = [&](int m, int c, const f32x16 (&acc)[MT][2]) {
    if (m < NEL / 2) {
      const int e = 2 * m;  // elements e, e+1: same (mt, nb), rows i, i+1
      const int mt = e / 32, nb = (e / 16) % 2, i = e % 16;
      float& pp = nb == 0 ? p0 : p1;
      pp = __builtin_fmaf(wr[mt][i], relu(acc[mt][nb][i]), pp);
      pp = __builtin_fmaf(wr[mt][i + 1], relu(acc[mt][nb][i + 1]), pp);
    } else if (m == NEL / 2) {
      // Lanes < 32 end with key K0+lane of tile 0, lanes >= 32 with key K0+lane of tile 1.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
      p0 = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    } else {
      const int s_key = kb + c * kChunk + lane;
      const uint32_t key = score_key(p0);
      const bool take = select && s_key >= b && s_key <= t && key >= thr;
      const uint64_t msk = ballot(take);
      if (take) {
        const int pos = cnt + lanes_below(msk);
        keys[pos] = key;
        idxs[pos] = s_key;
      }
      cnt += __popcll(msk);
      p0 = 0.0f;
      p1 = 0.0f;
    }
  };
  auto maybe_select = [&]() {
    if (cnt > kCap - kChunk) {  // rare after the first few thousand keys
      wave_lds_sync();
      thr = wave_select_topk(keys, idxs, hist, cnt, k);
      cnt = k;
    }
  };
  // One chunk: the MFMAs of chunk c (if any) interleaved with the epilogue of chunk c-1 (if any).
  auto chunk_step = [&](int c, f32x16 (&cur)[MT][2], const f32x16 (&prev)[MT][2]) {
    if (c < nchunks) wait_chunk(c);
    barrier_lds();  // chunk c has landed; the slot of chunk c-1 is free
    // Copies issued between the MFMAs stall the matrix pipe for longer than they take here.
    if (c + 2 < nchunks) issue_chunk(c + 2);
    if (c < nchunks && c > 0) {
      // Order: first B fragments, the first epilogue steps of chunk c-1 (they cover the LDS
      // latency), then the MFMAs of chunk c with the remaining steps spread between them.
      constexpr int kLead = 3;
      bf16x8 kb0[KS], kb1[KS];
      load_b(c, 0, kb0, kb1);
      load_b(c, 1, kb0, kb1);
      idx_static_for<NMICRO>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m * NMF / NMICRO - kLead < 0) micro(m, c - 1, prev);
      });
      __builtin_amdgcn_sched_barrier(0);
      idx_static_for<NMF>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (i % (2 * MT) == 0 && i / (2 * MT) + 2 < KS) load_b(c, i / (2 * MT) + 2, kb0, kb1);
        mfma_step(c, i, cur, kb0, kb1);
        __builtin_amdgcn_sched_barrier(0);
        idx_static_for<NMICRO>([&](auto m_c) {
          constexpr int m = decltype(m_c)::value;
          if constexpr (m * NMF / NMICRO - kLead == i) micro(m, c - 1, prev);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      idx_static_for<NMICRO>([&](auto m_c) {
        constexpr int m = decltype(m_c)::value;
        if constexpr (m * NMF / NMICRO - kLead >= NMF) micro(m, c - 1, prev);
      });
      maybe_select();
    } else if (c < nchunks) {
      bf16x8 kb0[KS], kb1[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) load_b(c, s, kb0, kb1);
#pragma unroll
      for (int i = 0; i < NMF; ++i) mfma_step(c, i, cur, kb0, kb1);
    } else {
#pragma unroll
      for (int m = 0; m < NMICRO; ++m) micro(m, c - 1, prev);
      maybe_select();
    }
  };

  issue_chunk(0);
  if (nchunks > 1) issue_chunk(1);
  f32x16 accA[MT][2], accB[MT][2];
  int c = 0;
  for (; c + 1 <= nchunks; c += 2) {
    chunk_step(c, accA, accB);
    chunk_step(c + 1, accB, accA);
  }
  if (c <= nchunks) chunk_step(c, accA, accB);

  if (select) {
    wave_lds_sync();
    if (cnt > k) thr = wave_select_topk(keys, idxs, hist, cnt, k);
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
  dim3 grid((a.nrows + kIdxWaves - 1) / kIdxWaves), block(kIdxWaves * kWave);
  if (H_I == 64 && d_I == 128) hipLaunchKernelGGL((k_index_topk<64, 128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_index_topk<4, 64>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

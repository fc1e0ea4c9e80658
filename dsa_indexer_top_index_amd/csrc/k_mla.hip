// Sparse latent attention over the selected KV rows (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, Implementation Limits bullets 1-2:
// the sparse kernels attend directly to the selected latent KV rows and never expand per-head
// K/V; kimi_k3 API index, KimiK3TextConfig: kv_lora_rank 512 + 64 unrotated dims, 96 heads;
// archdiff blueprint tagline: no positional encoding):
//   for query t, head h and selected rows s_j:
//     l_j = scale * q[t,h,:] . kv[s_j,:]          (576 dims)
//     o_lat[t,h,:] = softmax_j(l) . kv[s_j, 0:512]
//   with an optional learnable sink per head (archdiff blueprint, "Output gate + sink"): the
//   softmax denominator gains exp(sink[h]), a logit whose value row is zero.
//
// Kernel design: persistent workgroups, one per CU, each running query rows one after another
// (longest rows first, dealt out zig-zag). Three kinds of waves meet in LDS; with 96 heads there
// are eight, two per SIMD, so every SIMD runs matrix instructions:
//  - Score waves (three for 96 heads, 32 heads each; one for 16 heads): q fragments stay in
//    registers; S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (16 keys as M, 16-head tiles as N,
//    K = 576); softmax numerators in FP32 (base 2) against a per-head reference maximum set by the
//    first usable tile; P (bf16) goes to a two-slot LDS ring already in the value waves' operand
//    layout.
//  - Value waves (four for 96 heads, 128 latent dims each; two for 16 heads): each owns the
//    output accumulators of all heads for its latent dims and computes O^T += V^T P^T on
//    v_mfma_f32_32x32x16_bf16: latent dims as M, 32-head tiles as N, 16 keys as K. V is read
//    straight from the natural row layout with ds_read_b64_tr_b16 and P from LDS. They run two
//    tiles behind the score waves.
//  - One copy wave issues every asynchronous 16-byte global->LDS copy of the gathered rows into a
//    ring of seven 16-row tiles (copies run four tiles ahead) and does nothing else. A CU accepts
//    about one 64-lane copy per 64 cycles, so a wave that issues copies stalls; with the copies on
//    a wave of their own, no MFMA wave does.
//  One barrier per tile hands both rings over. Each gathered row is read from memory once per
//  query. The tile layout is column-major in 16-byte granules with a row XOR, so the QK operand
//  reads and the transposed V reads are bank-conflict free and every address is affine in the
//  loop index. Accumulators are never rescaled: if a logit exceeds its head's reference by more
//  than 2^64 (impossible for bounded inputs, but possible in principle), the row is redone, first
//  a QK-only pass for each head's exact maximum, then the full pass against it, so no numerator
//  can overflow.
//  Epilogue: divide by the softmax sum, stage o_lat (bf16) in the ring and store it for the
//  up-projection kernel, and write the natural-log normaliser lse if requested. While the value
//  waves store a row, the score waves already load the next row's indices and q fragments.
#include "dsa_device.h"
#include "dsa_kernels.h"

#include <type_traits>
#include <utility>

namespace dsa {

constexpr int kTileKeys = 16;
constexpr int kRowGran = kLatent * 2 / 16;            // 72 granules (16 B) per latent row
constexpr int kTileBytes = kTileKeys * kRowGran * 16;  // 18432: 18 wave copies of 1 KB
constexpr int kRing = 7;                               // tiles in the shared LDS ring
constexpr int kAhead = kRing - 3;                      // tiles whose copies run ahead of the scores
constexpr int kPre = 4;                                // K fragments read ahead in the score loop
constexpr int kRun = 3;                                // K steps per head tile before switching tiles
constexpr float kRestartGap = 64.0f;                   // log2 headroom of a head's reference maximum
constexpr int kMaxIdx = 2048;

// Tile layout in LDS: granule (row r, column c) lives at slot c*16 + (r ^ 4*(c%4)). One wave
// copy fills four columns of all 16 rows; the QK operand reads (16 rows, one column) and the
// transposed V reads (4 rows x 4 columns per 16 lanes) both hit 16 distinct bank quads.

// Roles: NS score waves of HS heads (NTS 16-head tiles each); NV value waves, each holding MT
// 32-head M tiles (rows of heads beyond H stay zero) for 512/NV latent dims, NA of its
// accumulator tiles in AGPRs; one copy wave. Waves go to SIMDs round-robin, so with 96 heads
// (eight waves, two per SIMD) three SIMDs run a score wave beside a value wave and the fourth a
// value wave beside the copy wave.
template <int H> struct MlaRoles;
template <> struct MlaRoles<96> { static constexpr int NS = 3, HS = 32, NTS = 2, MT = 3, NV = 4, NA = 8; };
template <> struct MlaRoles<16> { static constexpr int NS = 1, HS = 16, NTS = 1, MT = 1, NV = 2, NA = 8; };
template <int H> constexpr int mla_waves() { return MlaRoles<H>::NS + MlaRoles<H>::NV + 1; }

// O^T += V^T P^T with the accumulator pinned to AGPRs. The compiler does not see this instruction's
// hazards: the operands must not be written by VALU within 4 wait states before it (here they
// come straight from LDS reads), and VALU access to acc must wait for mfma_agpr_drain().
__device__ __forceinline__ void mfma32_a(f32x16& acc, const u32x4& x, const u32x4& y) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int H>
__global__ __launch_bounds__(64 * mla_waves<H>(), 1) void k_sparse_mla(MlaArgs a) {
  using R = MlaRoles<H>;
  constexpr int NS = R::NS, HS = R::HS, NTS = R::NTS, MT = R::MT;
  constexpr int NV = R::NV, NA = R::NA;
  constexpr int NW = mla_waves<H>();  // score, value and copy waves
  constexpr int CT = kVDim / 32 / NV;   // 32-wide latent tiles per value wave
  constexpr int kCopies = kTileBytes / 1024;  // 1 KB wave copies per tile, all by the copy wave
  static_assert(kCopies * (kAhead - 1) <= 63, "vmcnt range");
  static_assert(kCopies * 64 <= 4095 && kVDim % (32 * NV) == 0 && NA <= MT * CT, "role shapes");
  static_assert(18 % kRun == 0, "whole runs of K steps");

  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kRing][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[2][MT][64 * 16];  // P in MFMA A layout
  __shared__ int32_t s_idx[kMaxIdx + kTileKeys];
  __shared__ float s_inv[MT * 32];
  __shared__ int s_flag;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // the block has exactly NW waves
  const int lane = threadIdx.x % kWave;
  const int T = a.T;
  const int g16 = lane >> 4, i16 = lane & 15;
  const uint32_t ring = lds_addr_of(&s_ring[0][0]);
  const uint32_t pbase = lds_addr_of(&s_p[0][0][0]);
  constexpr uint32_t kPSlot = MT * 1024;
  __shared__ int s_bad[2];  // by row parity: some full tile of the row holds unusable indices

  // Persistent blocks: in round j, block b runs dispatch row G*j + b (j even) or G*j + G-1-b
  // (j odd), G blocks in all; dispatch row i is local row chunk_r0 + chunk_rows-1-i, so rows go
  // longest first and the zig-zag evens out the blocks' work. Consecutive dispatch rows run on
  // different XCDs, so every XCD receives the same mix of long and short rows.
  const int G = gridDim.x, bid = blockIdx.x;
  auto dispatch_row = [&](int j) -> int { return G * j + ((j & 1) ? G - 1 - bid : bid); };
  struct Row {
    int rr, r, keff, ntiles;
  };
  auto row_of = [&](int i) -> Row {
    Row w;
    w.rr = a.chunk_rows - 1 - i;
    w.r = a.chunk_r0 + w.rr;
    const int t_row = a.row0 + w.r;
    w.keff = min(a.k, t_row - doc_begin(a.cu, a.n_docs, t_row) + 1);
    w.ntiles = (w.keff + kTileKeys - 1) / kTileKeys;
    return w;
  };
  // Threads [0, NT) load a row's indices into s_idx, checked once: entries outside [0, T) become
  // -1 (masked), and one before the last tile flags the row in s_bad[par]. All loads are issued
  // before the first store, so the list arrives in one latency. P starts at zero.
  auto load_row = [&](const Row& w, auto nt_c, int par) {
    constexpr int NT = decltype(nt_c)::value;
    constexpr int kPer = (kMaxIdx + NT - 1) / NT;
    const int32_t* __restrict__ ix = a.idx + static_cast<int64_t>(w.r) * a.k;
    int iv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = threadIdx.x + NT * i;
      iv[i] = j < w.keff ? ix[j] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = threadIdx.x + NT * i;
      const bool ok = iv[i] >= 0 && iv[i] < T;
      if (j < w.ntiles * kTileKeys) s_idx[j] = ok ? iv[i] : -1;
      bad |= !ok && j < (w.ntiles - 1) * kTileKeys;
    }
    for (int j = threadIdx.x; j < 2 * MT * 256; j += NT) reinterpret_cast<uint32_t*>(&s_p[0][0][0])[j] = 0u;
    if (bad) s_bad[par] = 1;
  };

  if (threadIdx.x < 2) s_bad[threadIdx.x] = 0;
  if (threadIdx.x == 0) s_flag = 0;
  __syncthreads();
  Row w = row_of(dispatch_row(0));  // the launch has at least G rows
  load_row(w, std::integral_constant<int, 64 * NW>{}, 0);

  if (wave < NS) {
    // ================================ score wave ================================
    const int sw = wave;
    bf16x8 qf[NTS][18];
    auto load_q = [&](int row) {
      // q fragments, B operand of S^T = K Q^T. lane: head sw*HS + 16*nt + i16, dims 32*st + 8*g16.
      // a wave-uniform row base and a 32-bit per-lane offset, so no per-lane 64-bit pointers are kept
      const uint8_t* qbase = reinterpret_cast<const uint8_t*>(a.q + static_cast<int64_t>(row) * a.H * kLatent);
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) {
        const uint32_t off = static_cast<uint32_t>(((sw * HS + 16 * nt + i16) * kLatent + 8 * g16) * 2);
#pragma unroll
        for (int st = 0; st < 18; ++st) qf[nt][st] = *reinterpret_cast<const bf16x8*>(qbase + off + 64 * st);
      }
      // the fragments live in AGPRs, which the MFMAs read directly; the VGPRs hold K fragments
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt)
#pragma unroll
        for (int st = 0; st < 18; ++st) asm volatile("" : "+a"(qf[nt][st]));
      mfma_agpr_settle();
    };
    load_q(w.r);
    // sink logit of this lane's head in log2 units, or nothing
    float sink_l2[NTS];
#pragma unroll
    for (int nt = 0; nt < NTS; ++nt) sink_l2[nt] = a.sink ? a.sink[sw * HS + 16 * nt + i16] * 1.4426950408889634f : 0.0f;
    const uint32_t qk_base = ring + (g16 * 16 + (i16 ^ (4 * g16))) * 16;  // row i16, column 4*st + g16
    // This lane's numerators (head gh, keys 4*g16 .. +3) in the B operand of the value waves:
    // M tile gh/32, lane 32*(g16/2) + gh%32, bytes 8*(g16&1) of that lane's 16.
    uint32_t p_off[NTS];
#pragma unroll
    for (int nt = 0; nt < NTS; ++nt) {
      const int gh = sw * HS + 16 * nt + i16;
      p_off[nt] = pbase + ((gh >> 5) * 64 + 32 * (g16 >> 1) + (gh & 31)) * 16 + 8 * (g16 & 1);
    }
    for (int j = 0;; ++j) {
      barrier_lds();  // (A) the row's indices, zeroed P and q fragments are ready
      const bool any_bad = s_bad[j & 1] != 0;
      const int r = w.r, ntiles = w.ntiles;
      float m_ref[NTS], l_part[NTS];
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) m_ref[nt] = -INFINITY;

      // K fragments of tile t (row i16, dims 32*st + 8*g16), all requested at once
      auto load_k = [&](int t, bf16x8 (&kf)[18]) {
        const DSA_LDS uint8_t* tq = lds_ptr(qk_base + (t % kRing) * kTileBytes);
#pragma unroll
        for (int st = 0; st < 18; ++st) kf[st] = lds_read16(tq + 1024 * st);
      };
      // S^T of one tile: rows = 16 keys, cols = heads, K = 576 in 18 steps
      auto qk = [&](const bf16x8 (&kf)[18], f32x4 (&sc)[NTS]) {
#pragma unroll
        for (int st = 0; st < 18; ++st)
#pragma unroll
          for (int nt = 0; nt < NTS; ++nt) sc[nt] = mfma16(kf[st], qf[nt][st], st == 0 ? f32x4{} : sc[nt]);
      };
      // Key-validity bits of a tile (bit j: key j has a usable index), from the index lanes 0..15 hold.
      auto valid_bits = [&](int idx_val) -> uint32_t {
        return static_cast<uint32_t>(ballot(idx_val >= 0) & 0xffffull);
      };
      // Masked scores -> per-head maxima in log2 units (lanes i16 + 16*g hold the same head).
      auto mask_max = [&](f32x4 (&sc)[NTS], uint32_t vm, float (&tmax)[NTS]) {
        const uint32_t bits = vm >> (4 * g16);
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[nt][j] = ((bits >> j) & 1u) ? sc[nt][j] : -INFINITY;
          float m = fmaxf(fmaxf(sc[nt][0], sc[nt][1]), fmaxf(sc[nt][2], sc[nt][3]));
          const auto m16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          m = fmaxf(__uint_as_float(m16[0]), __uint_as_float(m16[1]));
          const auto m32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
          tmax[nt] = fmaxf(__uint_as_float(m32[0]), __uint_as_float(m32[1])) * a.scale_log2;
        }
      };
      // Softmax numerators: x = scale*s - m_ref (log2 units), p = 2^x; masked keys get x = -inf
      // and p = 0. gx keeps the largest x of the pass: while the references are the first tile's
      // maxima, a value above kRestartGap means that the row has to be redone with exact maxima.
      float msub[NTS], gx = -INFINITY;
      struct Soft {
        float x[4], p[4];
      };
      // Micro-step k of a tile's softmax (12 per 16-head tile, a few VALU instructions each), so
      // that the steps fit between the MFMAs of the next tile. ok[j]: key 4*g16 + j is usable.
      auto micro = [&](int k, const f32x4 (&sc)[NTS], const bool (&ok)[4], uint32_t slot, Soft (&sf)[NTS],
                       auto masked_c) {
        const int nt = k / 12, s = k % 12;
        Soft& f = sf[nt];
        if (s < 4) {
          f.x[s] = __builtin_fmaf(sc[nt][s], a.scale_log2, -msub[nt]);
          if constexpr (decltype(masked_c)::value) f.x[s] = ok[s] ? f.x[s] : -INFINITY;
        } else if (s < 8) {
          f.p[s - 4] = fast_exp2(f.x[s - 4]);  // -inf gives 0
        } else if (s == 8) {
          gx = fmaxf(gx, fmaxf(fmaxf(f.x[0], f.x[1]), fmaxf(f.x[2], f.x[3])));
        } else if (s == 9) {
          l_part[nt] += f.p[0] + f.p[1];
        } else if (s == 10) {
          l_part[nt] += f.p[2] + f.p[3];
        } else {
          const u32x2 pk = {pack_bf16x2(f.p[0], f.p[1]), pack_bf16x2(f.p[2], f.p[3])};
          *reinterpret_cast<DSA_LDS u32x2*>(lds_ptr(p_off[nt] + slot)) = pk;
        }
      };
      auto key_ok = [&](uint32_t vm, bool (&ok)[4]) {
        const uint32_t bits = vm >> (4 * g16);
#pragma unroll
        for (int j = 0; j < 4; ++j) ok[j] = (bits >> j) & 1u;
      };
      // One pass writing numerators; ntiles+2 barriers. CHECK: the first tile's maxima become the
      // references and gx records growth beyond them; otherwise m_ref holds exact maxima. MASKED:
      // some full tile holds unusable indices (the last tile is always masked). The MFMAs of tile t
      // are interleaved with the micro-steps of tile t-1, so the VALU work runs while the matrix
      // core is busy; the value waves consume that P one tile later.
      auto numerator_pass = [&](auto check_c, auto masked_c) {
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt) l_part[nt] = 0.0f;
        f32x4 sprev[NTS];
        uint32_t vprev;
        // The first kPre K fragments of the next tile, read during the last K steps of the current
        // one (the copy wave waits for tile t+1 before barrier t), so that a tile's MFMAs start
        // right after its barrier instead of after an LDS read.
        bf16x8 kn[kPre];
        {
          barrier_lds();  // tiles 0 and 1 have landed
          bf16x8 kf[18];
          load_k(0, kf);
          const int iv0 = s_idx[lane & 15];
          qk(kf, sprev);
          {
            const DSA_LDS uint8_t* tqn = lds_ptr(qk_base + (1 % kRing) * kTileBytes);
#pragma unroll
            for (int st = 0; st < kPre; ++st) kn[st] = lds_read16(tqn + 1024 * st);
          }
          vprev = valid_bits(iv0);
          if constexpr (decltype(check_c)::value) {
            float tmax[NTS];
            mask_max(sprev, vprev, tmax);
#pragma unroll
            for (int nt = 0; nt < NTS; ++nt) m_ref[nt] = tmax[nt];
          }
#pragma unroll
          for (int nt = 0; nt < NTS; ++nt) msub[nt] = fmaxf(m_ref[nt], -3.0e38f);  // finite without usable keys
        }
        for (int t = 1; t < ntiles; ++t) {
          barrier_lds();  // tiles t and t+1 have landed; P slot (t-1)%2 has been consumed
          // K fragments are read kPre steps ahead of their MFMAs rather than all at once: right
          // after the barrier every wave of the CU reads LDS, and a burst would delay them all.
          // The last kPre steps read the next tile's first fragments (past the row's last tile
          // they read a ring slot that is not used).
          const DSA_LDS uint8_t* tq = lds_ptr(qk_base + (t % kRing) * kTileBytes);
          const DSA_LDS uint8_t* tqn = lds_ptr(qk_base + ((t + 1) % kRing) * kTileBytes);
          bf16x8 kf[18];
#pragma unroll
          for (int st = 0; st < kPre; ++st) kf[st] = kn[st];
          const int ivt = s_idx[t * kTileKeys + (lane & 15)];
          const uint32_t slot = ((t - 1) & 1) * kPSlot;
          bool ok[4];
          key_ok(vprev, ok);
          Soft sf[NTS];
          f32x4 sc[NTS];
#pragma unroll
          for (int i = 0; i < 18 * NTS; ++i) {
            // runs of kRun K steps per head tile: a 16x16x32 MFMA that follows one with the same
            // accumulator issues faster than one that switches accumulators
            const int blk = i / (kRun * NTS), r = i % (kRun * NTS);
            const int nt = r / kRun, st = kRun * blk + r % kRun;
            if (nt == 0 && st + kPre < 18) kf[st + kPre] = lds_read16(tq + 1024 * (st + kPre));
            if (nt == 0 && st + kPre >= 18) kn[st + kPre - 18] = lds_read16(tqn + 1024 * (st + kPre - 18));
            sc[nt] = mfma16(kf[st], qf[nt][st], st == 0 ? f32x4{} : sc[nt]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 12 * NTS; ++k)
              if (k * 3 / 2 == i) micro(k, sprev, ok, slot, sf, masked_c);
            __builtin_amdgcn_sched_barrier(0);
          }
          vprev = valid_bits(ivt);
#pragma unroll
          for (int nt = 0; nt < NTS; ++nt) sprev[nt] = sc[nt];
        }
        barrier_lds();  // B_ntiles
        {
          bool ok[4];
          key_ok(vprev, ok);
          Soft sf[NTS];
#pragma unroll
          for (int k = 0; k < 12 * NTS; ++k) micro(k, sprev, ok, ((ntiles - 1) & 1) * kPSlot, sf, std::true_type{});
        }
        barrier_lds();  // B_ntiles+1
      };
      // Exact per-head maxima (QK only); ntiles+2 barriers.
      auto max_pass = [&]() {
        for (int t = 0;; ++t) {
          barrier_lds();
          if (t == ntiles + 1) break;
          if (t == ntiles) continue;
          bf16x8 kf[18];
          load_k(t, kf);
          const int ivt = s_idx[t * kTileKeys + (lane & 15)];
          f32x4 sc[NTS];
          qk(kf, sc);
          float tmax[NTS];
          mask_max(sc, valid_bits(ivt), tmax);
#pragma unroll
          for (int nt = 0; nt < NTS; ++nt) m_ref[nt] = fmaxf(m_ref[nt], tmax[nt]);
        }
      };
      if (any_bad) numerator_pass(std::true_type{}, std::true_type{});
      else numerator_pass(std::true_type{}, std::false_type{});
      if (ballot(gx > kRestartGap) != 0ull && lane == 0) s_flag = 1;  // rare: the row is redone
      barrier_lds();  // (1) s_flag is final
      if (s_flag) {
#pragma unroll
        for (int nt = 0; nt < NTS; ++nt) m_ref[nt] = -INFINITY;
        max_pass();
        numerator_pass(std::false_type{}, std::true_type{});
      }
      // 1/sum for the value waves, and lse. The numerators are 2^(x - m_ref); a sink s adds
      // 2^(s - m_ref) to the sum (a logit with a zero value row). When the sink exceeds m_ref by
      // more than 2^64 the sum is scaled by 2^-(s - m_ref) instead, so nothing overflows (a head
      // with no usable key has m_ref = -inf and takes that branch: weight 0, lse = s).
#pragma unroll
      for (int nt = 0; nt < NTS; ++nt) {
        float l = l_part[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const int gh = sw * HS + 16 * nt + i16;
        float inv, lse2;
        if (a.sink == nullptr) {
          inv = l > 0.0f ? 1.0f / l : 0.0f;
          lse2 = l > 0.0f ? m_ref[nt] + log2f(l) : -INFINITY;
        } else {
          const float d = sink_l2[nt] - m_ref[nt];
          if (d <= kRestartGap) {
            const float lt = l + fast_exp2(d);
            inv = 1.0f / lt;
            lse2 = m_ref[nt] + log2f(lt);
          } else {
            const float e = fast_exp2(-d);
            const float lt = __builtin_fmaf(l, e, 1.0f);
            inv = e / lt;
            lse2 = sink_l2[nt] + log2f(lt);
          }
        }
        if (lane < 16) {
          s_inv[gh] = inv;
          if (a.lse) a.lse[static_cast<int64_t>(r) * a.H + gh] = lse2 * 0.69314718055994531f;
        }
      }
      if (MT * 32 > H && lane < MT * 32 - H) s_inv[H + lane] = 0.0f;
      barrier_lds();  // (2) s_inv is ready
      // While the value waves finish the row, load the next one.
      if (threadIdx.x == 0) s_bad[j & 1] = 0;  // every wave read it after (A)
      const int in = dispatch_row(j + 1);
      if (in >= a.chunk_rows) break;
      w = row_of(in);
      if (threadIdx.x == 0) s_flag = 0;  // the value waves read it between (1) and (2)
      load_row(w, std::integral_constant<int, 64 * NS>{}, (j + 1) & 1);
      load_q(w.r);
    }
  } else if (wave < NS + NV) {
    // ================================ value wave ================================
    const int vw = wave - NS;
    int ntiles = w.ntiles;
    // V operand (transposed reads): keys 8*hh + s4 (+4), latent granule 4*(CT*vw + ct) + vc
    const int hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;
    const int vc = 2 * chh + (q4 >> 1);
    const uint32_t v_off1 = (vc * 16 + ((8 * hh + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1) + 1024 * CT * vw;
    const uint32_t v_off2 = (vc * 16 + ((8 * hh + 4 + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1) + 1024 * CT * vw;
    const uint32_t p_rd = pbase + lane * 16;

    // Accumulator tile (mt, ct) lives in AGPRs when mt*CT + ct < NA, else in VGPRs.
    f32x16 O[MT][CT];
    // Ties the accumulators to this program point, so that no access to them moves across the
    // wait-state padding placed next to it.
    auto pin_acc = [&]() {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          if (mt * CT + ct < NA) asm volatile("" : "+a"(O[mt][ct]));
          else asm volatile("" : "+v"(O[mt][ct]));
        }
    };
    // One pass over the row; ntiles+2 barriers. mode 1 only keeps step (the scores redo their
    // maxima); modes 0 and 2 accumulate P V, two tiles behind the scores. The copy wave has waited
    // for tile t's copies before barrier t.
    auto value_pass = [&](int mode) {
      // a zero the compiler cannot see as a constant, so the accumulators' initial value is made
      // here in every row instead of being kept live across the row loop
      float z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) O[mt][ct] = f32x16{} + z;
      pin_acc();
      mfma_agpr_settle();
      for (int t = 0;; ++t) {
        barrier_lds();  // tile t has landed; P of tile t-2 is complete
        if (t > 1 && mode != 1) {
          const int tv = t - 2;
          const uint32_t tb = ring + (tv % kRing) * kTileBytes;
          const uint32_t pp = p_rd + (tv & 1) * kPSlot;
          u32x4 pa[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) pa[mt] = *reinterpret_cast<const DSA_LDS u32x4*>(lds_ptr(pp + mt * 1024));
          // V fragments two steps ahead of their MFMAs (see the K reads of the score waves)
          u32x2 v1[CT], v2[CT];
#pragma unroll
          for (int ct = 0; ct < 2 && ct < CT; ++ct) {
            v1[ct] = lds_read_tr16(lds_ptr(tb + v_off1 + 1024 * ct));
            v2[ct] = lds_read_tr16(lds_ptr(tb + v_off2 + 1024 * ct));
          }
          static_for<CT>([&](auto ct_c) {
            constexpr int ct = decltype(ct_c)::value;
            if constexpr (ct + 2 < CT) {
              v1[ct + 2] = lds_read_tr16(lds_ptr(tb + v_off1 + 1024 * (ct + 2)));
              v2[ct + 2] = lds_read_tr16(lds_ptr(tb + v_off2 + 1024 * (ct + 2)));
            }
            const u32x4 vb = {v1[ct][0], v1[ct][1], v2[ct][0], v2[ct][1]};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              // A = V^T (lane: latent dim, 8 keys), B = P^T (lane: head, 8 keys), D = O^T
              if (mt * CT + ct < NA) mfma32_a(O[mt][ct], vb, pa[mt]);
              else
                O[mt][ct] = mfma32(__builtin_bit_cast(bf16x8, vb), __builtin_bit_cast(bf16x8, pa[mt]), O[mt][ct]);
            }
            __builtin_amdgcn_sched_barrier(0);
          });
        }
        if (t == ntiles + 1) break;
      }
    };
    for (int j = 0;; ++j) {
      barrier_lds();  // (A)
      ntiles = w.ntiles;
      value_pass(0);
      barrier_lds();  // (1)
      if (s_flag) {
        value_pass(1);
        value_pass(2);
      }
      mfma_agpr_drain();  // the accumulators are read by VALU below
      pin_acc();
      barrier_lds();      // (2) s_inv is ready; the score waves are done with the ring
      // Normalise and stage [heads][512 dims] as bf16 in the ring (rows padded by 16 bytes against
      // bank conflicts), then 16-byte stores. O^T tile (mt, ct), lane: head 32*mt + lane%32,
      // element e: latent dim 32*(CT*vw + ct) + 8*(e/4) + 4*hh + e%4.
      constexpr uint32_t kStageRow = kVDim * 2 + 16;
      static_assert(MT * 32 * kStageRow <= kRing * kTileBytes, "staging fits in the ring");
      const uint32_t stage = ring + (lane & 31) * kStageRow + 2 * (32 * CT * vw + 4 * hh);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float inv = s_inv[32 * mt + (lane & 31)];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const f32x16 ov = O[mt][ct] * inv;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const u32x2 pk = {pack_bf16x2(ov[4 * e4], ov[4 * e4 + 1]), pack_bf16x2(ov[4 * e4 + 2], ov[4 * e4 + 3])};
            *reinterpret_cast<DSA_LDS u32x2*>(lds_ptr(stage + mt * 32 * kStageRow + 2 * (32 * ct + 8 * e4))) = pk;
          }
        }
      }
      wave_lds_sync();
      // this wave's dims of each head row: kLph lanes of 16 bytes per row, kHpi rows at a time
      constexpr int kDimsV = kVDim / NV, kLph = kDimsV / 8, kHpi = kWave / kLph;
      uint16_t* dst = a.o_lat + static_cast<int64_t>(w.rr) * H * kVDim;
      const int c0 = kDimsV * vw + 8 * (lane % kLph);
      for (int h = lane / kLph; h < H; h += kHpi) {
        const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(lds_ptr(ring + h * kStageRow + 2 * c0));
        *reinterpret_cast<u32x4*>(dst + h * kVDim + c0) = v;
      }
      const int in = dispatch_row(j + 1);
      if (in >= a.chunk_rows) break;
      w = row_of(in);
    }
  } else {
    // ================================ copy wave ================================
    // Issues every global->LDS copy of the gathered rows and nothing else, so that no MFMA wave
    // stalls on the vector-memory unit (a CU takes one 64-lane copy about every 64 cycles).
    // Copy c (of a tile's 18) fills tile column 4*c + g16 with this lane's 16 bytes of row
    // my_row. The per-lane global offset of a tile is computed once; the immediate offset 64*c
    // moves both the global and the LDS address, so M0 carries the rest of the LDS displacement,
    // 1024*c - 64*c.
    int ntiles = w.ntiles;
    const int my_row = i16 ^ (4 * g16);
    auto issue_tile = [&](int t) {
      const uint32_t voff = static_cast<uint32_t>(max(s_idx[t * kTileKeys + my_row], 0)) * (kLatent * 2) + 16 * g16;
      const uint32_t base = ring + (t % kRing) * kTileBytes;
      static_for<kCopies>([&](auto c_const) {
        constexpr int c = decltype(c_const)::value;
        copy16_to_lds_imm<64 * c>(a.kv, voff, base + (1024 - 64) * c);
      });
    };
    // Before barrier t: waits until the copies of tile u have landed; the tiles after u issued so
    // far (up to tile t + kAhead - 1) stay in flight.
    auto wait_tile = [&](int u, int t) {
      const int later = min(t + kAhead - 1, ntiles - 1) - u;
      if (later >= 3) wait_vmem_le<3 * kCopies>();
      else if (later == 2) wait_vmem_le<2 * kCopies>();
      else if (later == 1) wait_vmem_le<kCopies>();
      else wait_vmem_le<0>();
    };
    // One pass over the row's tiles; ntiles+2 barriers. Tile t+kAhead goes into the slot of tile
    // t-3, which every wave is done with after barrier t.
    auto copy_pass = [&]() {
#pragma unroll
      for (int p = 0; p < kAhead; ++p)
        if (p < ntiles) issue_tile(p);
      for (int t = 0;; ++t) {
        // tiles t and t+1 land before barrier t: the score waves read tile t+1's first fragments
        // during step t
        if (t + 1 < ntiles) wait_tile(t + 1, t);
        else if (t < ntiles) wait_tile(t, t);
        barrier_lds();
        if (t + kAhead < ntiles) issue_tile(t + kAhead);
        if (t == ntiles + 1) break;
      }
    };
    for (int j = 0;; ++j) {
      barrier_lds();  // (A)
      ntiles = w.ntiles;
      copy_pass();
      barrier_lds();  // (1)
      if (s_flag) {   // the row is redone: once for the maxima, once for the numerators
        copy_pass();
        copy_pass();
      }
      barrier_lds();  // (2)
      const int in = dispatch_row(j + 1);
      if (in >= a.chunk_rows) break;
      w = row_of(in);
    }
  }
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  if (a.k > kMaxIdx || a.chunk_rows < 1) return hipErrorInvalidValue;
  // one persistent workgroup per CU (its LDS use allows no second one), at most one per row
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return hipErrorInvalidValue;
  const dim3 grid(a.chunk_rows < cus ? a.chunk_rows : cus);
  if (a.H == 96) hipLaunchKernelGGL((k_sparse_mla<96>), grid, dim3(64 * mla_waves<96>()), 0, st, a);
  else if (a.H == 16) hipLaunchKernelGGL((k_sparse_mla<16>), grid, dim3(64 * mla_waves<16>()), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa

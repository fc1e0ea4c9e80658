// Backward of sparse latent attention, the per-head V up-projection and the per-head gate (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page: the backward runs the native 96 heads,
// paragraph after the Implementation Limits bullets; hard top-k carries no gradient, 3rd bullet, so
// the indices are constants). For L = sum dout * out, with p_j = exp(l_j - lse) from the forward's
// saved lse:
//   D[t,h]    = sum_d dout * out  (= do . o)        dgate = (1 - sigma(g)) D
//   do        = sigma(g) dout                        do_lat = do W_UV[h]^T       (the absorption kernel)
//   dp_j      = do_lat . kv_j[:512]                  dl_j = p_j (dp_j - D)
//   dq        = scale sum_j dl_j kv_j                dkv_j += scale dl_j q + p_j do_lat
//   dW_UV[h] += o_lat^T do                           (o_lat recomputed by the forward kernel)
//
// k_bwd_prep: D, dgate and do, half a wave per (row, head).
// k_sparse_mla_bwd_row: one workgroup per row and all 96 heads, eight waves. Per 16-key tile of the
//   row's selected keys (gathered into LDS with the forward's tile layout, two tiles ahead):
//   - six compute waves of 16 heads recompute S^T (K = 576) and dP^T = V do_lat^T (K = 512) on the
//     same K fragments, with q and do_lat fragments in registers, then form P = 2^(scale log2e S -
//     log2e lse) and dS' = scale P (dP - D) in bf16 in LDS and store them to the workspace (g) for
//     k_dkv;
//   - two copy waves issue the gathers;
//   - every wave adds dq^T += K^T dS'^T for its share of the 32x32 tiles, one tile behind (K^T read
//     transposed from the gathered tile, accumulators kept across the row).
// k_dkv: the dkv contribution of every (row, selected key) pair, dS' Q + P do_lat contracted over all
//   96 heads at once, rounded to bf16 and stored per pair (one workgroup per row and 192 latent dims,
//   Q and do_lat of its dims as MFMA B operands in LDS, dS' and P streamed from g in 32-key tiles).
//   A counting sort of the chunk's pairs by key (k_pairs_count, two scan passes, k_pairs_place)
//   runs first and gives each pair its position in key order; k_dkv stores each contribution there,
//   and k_dkv_sum adds each key's contiguous contributions to dkv, one wave per key: no float atomics,
//   which run at a fixed rate per lane (about 330 G lane operations per second on MI355X).
// k_dwuv: dW_UV[h] += o_lat^T do over a chunk of rows, 16 rows per K step staged in LDS in the
//   forward's tile layout so that both operands are read transposed; partial sums added with atomics.
#include "dsa_device.h"
#include "dsa_kernels.h"

#include <algorithm>

namespace dsa {

constexpr int kBwKeys = 16;    // keys per gathered tile
constexpr int kBwGran = kLatent * 2 / 16;             // 72 granules per latent row
constexpr int kBwTileBytes = kBwKeys * kBwGran * 16;  // 18 KB
constexpr int kBwMaxIdx = 2048;
constexpr int kGCols = 2 * 96;  // g: dS' of the 96 heads, then P
constexpr float kLog2e = 1.4426950408889634f;

// Copies C, C + 2, .. < 18 of a gathered 16-key tile: lane i of copy c reads 16 bytes at
// kv + voff + 64c and writes them to the tile at 1024c + 16i.
template <int C>
__device__ __forceinline__ void bw_gather_copies(const uint16_t* kv, uint32_t voff, uint32_t base) {
  if constexpr (C < 18) {
    copy16_to_lds_imm<64 * C>(kv, voff, base + (1024 - 64) * C);
    bw_gather_copies<C + 2>(kv, voff, base);
  }
}

// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_prep(BwdPrepArgs a) {
  const int64_t rh = static_cast<int64_t>(blockIdx.x) * 8 + threadIdx.x / 32;  // (row, head) within the chunk
  const int sub = threadIdx.x % 32;
  if (rh >= static_cast<int64_t>(a.rows) * a.H) return;  // whole half-waves
  const int64_t grh = static_cast<int64_t>(a.row_off) * a.H + rh;  // in the caller's row numbering
  const u32x2 dv = *reinterpret_cast<const u32x2*>(a.dout + grh * kODim + 4 * sub);
  const u32x2 ov = *reinterpret_cast<const u32x2*>(a.out + grh * kODim + 4 * sub);
  float d4[4], o4[4];
  d4[0] = bf16_to_f32(static_cast<uint16_t>(dv[0])), d4[1] = bf16_to_f32(static_cast<uint16_t>(dv[0] >> 16));
  d4[2] = bf16_to_f32(static_cast<uint16_t>(dv[1])), d4[3] = bf16_to_f32(static_cast<uint16_t>(dv[1] >> 16));
  o4[0] = bf16_to_f32(static_cast<uint16_t>(ov[0])), o4[1] = bf16_to_f32(static_cast<uint16_t>(ov[0] >> 16));
  o4[2] = bf16_to_f32(static_cast<uint16_t>(ov[1])), o4[3] = bf16_to_f32(static_cast<uint16_t>(ov[1] >> 16));
  float D = (d4[0] * o4[0] + d4[1] * o4[1]) + (d4[2] * o4[2] + d4[3] * o4[3]);
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) D += __shfl_xor(D, o, 32);
  float sg[4];
  if (a.gate_per_dim) {
    // one gate logit per output element: dgate = (1 - sigma) dout out, element by element
    const u32x2 gv = *reinterpret_cast<const u32x2*>(a.gate + grh * kODim + 4 * sub);
    const float g4[4] = {bf16_to_f32(static_cast<uint16_t>(gv[0])), bf16_to_f32(static_cast<uint16_t>(gv[0] >> 16)),
                         bf16_to_f32(static_cast<uint16_t>(gv[1])), bf16_to_f32(static_cast<uint16_t>(gv[1] >> 16))};
#pragma unroll
    for (int i = 0; i < 4; ++i) sg[i] = 1.0f / (1.0f + __expf(-g4[i]));
    *reinterpret_cast<f32x4*>(a.dgate + grh * kODim + 4 * sub) =
        f32x4{(1.0f - sg[0]) * d4[0] * o4[0], (1.0f - sg[1]) * d4[1] * o4[1], (1.0f - sg[2]) * d4[2] * o4[2],
              (1.0f - sg[3]) * d4[3] * o4[3]};
  } else {
    const float s1 = 1.0f / (1.0f + __expf(-bf16_to_f32(a.gate[grh])));
#pragma unroll
    for (int i = 0; i < 4; ++i) sg[i] = s1;
    if (sub == 0) a.dgate[grh] = (1.0f - s1) * D;
  }
  const u32x2 dov = {pack_bf16x2(sg[0] * d4[0], sg[1] * d4[1]), pack_bf16x2(sg[2] * d4[2], sg[3] * d4[3])};
  *reinterpret_cast<u32x2*>(a.d_o + rh * kODim + 4 * sub) = dov;
  if (sub == 0) {
    a.delta[rh] = D;
    // the sink logit's share of the softmax, exp(sink - lse), times its gradient 0 - D
    if (a.sink) a.sterm[rh] = -__expf(a.sink[rh % a.H] - a.lse[grh]) * D;
  }
}

// dsink[h] += the chunk's sterm[:, h], summed in a fixed order (one workgroup per head).
__global__ __launch_bounds__(256) void k_sink_sum(SinkSumArgs a) {
  __shared__ float s_part[4];
  const int h = blockIdx.x;
  float sum = 0.0f;
  for (int r = threadIdx.x; r < a.rows; r += 256) sum += a.sterm[static_cast<int64_t>(r) * a.H + h];
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (threadIdx.x % kWave == 0) s_part[threadIdx.x / kWave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) a.dsink[h] += (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------------------------------------
// k_sparse_mla_bwd_row: the backward of one row with all 96 heads in one workgroup, so that each
// selected kv row is gathered once per row (a workgroup per group of 32 heads would gather it three
// times, and the gather's copies per CU set the pace). Eight waves, two barriers per 16-key tile:
//  - waves 0..5 (compute): 16 heads each, their q and do_lat fragments in registers. Per tile S^T and
//    dP^T on 16x16x32 MFMAs over the same K fragments of the tile, then P and dS' of their heads, in
//    bf16 to LDS: s_g in g's [key][dS' of 96 heads | P of 96 heads] layout, s_dsT as [head][key];
//  - waves 6 and 7 (copy): the tile gathers, two tiles ahead through a four-slot ring;
//  - dq^T += K^T dS'^T over the 54 (32 dims x 32 heads) tiles, one tile behind the products (s_dsT is
//    double buffered and the ring keeps the previous tile): the compute waves take four each, spread
//    through the next tile's S^T and dP^T chain, the copy waves fifteen each beside it. After the
//    second barrier the compute waves store s_g to g, 1 KB each.
constexpr int kBrHeads = 96;
constexpr int kBrWaves = 8;
constexpr int kBrCompute = 6;
constexpr int kBrRing = 4;
constexpr int kBrDqC = 4;   // dq tiles of a compute wave
constexpr int kBrDqX = 15;  // of a copy wave
static_assert(kBrCompute * kBrDqC + (kBrWaves - kBrCompute) * kBrDqX == 18 * 3, "every dq tile has an owner");
static_assert(kBwKeys * kGCols * 2 == kBrCompute * 1024, "one 1 KB store of the tile's g rows per compute wave");

__global__ __launch_bounds__(kBrWaves * kWave, 1) void k_sparse_mla_bwd_row(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kBrRing][kBwTileBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_g[kBwKeys * kGCols];
  __shared__ __attribute__((aligned(16))) uint16_t s_dsT[2][kBrHeads * kBwKeys];  // tile t in buffer t % 2
  __shared__ int32_t s_idx[kBwMaxIdx + kBwKeys];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int crow = blockIdx.x;
  const int r = a.chunk_r0 + crow;
  const int t_row = a.row0 + r;
  const int keff = min(a.k, t_row - doc_begin(a.cu, a.n_docs, t_row) + 1);
  const int ntiles = (keff + kBwKeys - 1) / kBwKeys;
  const int32_t* __restrict__ ix = a.idx + static_cast<int64_t>(r) * a.k;
  for (int j = threadIdx.x; j < ntiles * kBwKeys; j += kBrWaves * kWave) {
    const int v = j < keff ? ix[j] : -1;
    s_idx[j] = (v >= 0 && v < a.T) ? v : -1;
  }
  const uint32_t ring = lds_addr_of(&s_ring[0][0]);
  // transposed reads of the tile (A = K^T: lane = latent dim, 8 keys), and the S^T / dP^T operand reads
  const int hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;
  const int vc = 2 * chh + (q4 >> 1);
  const uint32_t v_off1 = (vc * 16 + ((8 * hh + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const uint32_t v_off2 = (vc * 16 + ((8 * hh + 4 + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const uint32_t qk_off = (g16 * 16 + (i16 ^ (4 * g16))) * 16;  // key i16, dims 32*st + 8*g16
  const uint32_t dsT = lds_addr_of(&s_dsT[0][0]) + (lane & 31) * 32 + 16 * hh;  // + 32 * 32 * ht: head 32ht + lane%32
  constexpr uint32_t kDsTBytes = kBrHeads * kBwKeys * 2;
  // dS'^T fragment of head tile ht of tile t (B operand of the dq products)
  auto ds_frag = [&](int ht, int t) -> bf16x8 {
    return *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(dsT + (t & 1) * kDsTBytes + 32 * 32 * ht));
  };
  // dq^T += K^T dS'^T of tile t for dq tile (dt, ht) = (i % 18, i / 18), given head tile ht's dS'^T
  // fragment b
  auto dq_step_b = [&](f32x16& acc, int i, int t, const bf16x8& b) {
    const int dt = i % 18;
    const uint32_t tb = ring + (t % kBrRing) * kBwTileBytes;
    const u32x2 v1 = lds_read_tr16(lds_ptr(tb + v_off1 + 1024 * dt));
    const u32x2 v2 = lds_read_tr16(lds_ptr(tb + v_off2 + 1024 * dt));
    const u32x4 kt = {v1[0], v1[1], v2[0], v2[1]};
    acc = mfma32(__builtin_bit_cast(bf16x8, kt), b, acc);
  };
  // lane: head 32ht + lane%32, dims 32dt + 8(e/4) + 4(lane/32) + e%4
  auto dq_store = [&](const f32x16& acc, int i) {
    const int dt = i % 18, ht = i / 18;
    float* __restrict__ dst = a.dq + (static_cast<int64_t>(r) * kBrHeads + 32 * ht + (lane & 31)) * kLatent + 32 * dt;
#pragma unroll
    for (int e = 0; e < 16; ++e) dst[8 * (e >> 2) + 4 * hh + (e & 3)] = acc[e];
  };

  if (wave < kBrCompute) {
    // ================================ compute wave ================================
    const int h = 16 * wave + i16;  // this lane's head (column of S^T and dP^T)
    bf16x8 qf[18], df[16];
    const uint16_t* __restrict__ qh = a.q + (static_cast<int64_t>(r) * kBrHeads + h) * kLatent + 8 * g16;
    const uint16_t* __restrict__ dh = a.do_lat + (static_cast<int64_t>(crow) * kBrHeads + h) * kVDim + 8 * g16;
#pragma unroll
    for (int st = 0; st < 18; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qh + 32 * st);
#pragma unroll
    for (int st = 0; st < 16; ++st) df[st] = *reinterpret_cast<const bf16x8*>(dh + 32 * st);
    const float lse2 = a.lse[static_cast<int64_t>(r) * kBrHeads + h] * kLog2e;
    const float Dh = a.delta[static_cast<int64_t>(crow) * kBrHeads + h];
    const float sl2 = a.scale * kLog2e;
    f32x16 dq[kBrDqC];
#pragma unroll
    for (int i = 0; i < kBrDqC; ++i) dq[i] = f32x16{};
    uint16_t* __restrict__ gdst = a.g + static_cast<int64_t>(crow) * a.g_stride * kGCols + 512 * wave + 8 * lane;
    // dq tiles of compute wave w: (dims 3w + j, head tile 0) for j < 3 and (dims w, head tile 1) for
    // j = 3, so that the dS'^T fragment read for j = 0 serves j = 1 and 2 as well (the copy waves own
    // tiles 24 .. 53)
    static_assert(kBrDqC == 4 && kBrCompute == 6, "compute waves' dq tiles: all of head tile 0, dims 0..5 of 1");
    auto ci = [&](int j) { return j < 3 ? 3 * wave + j : 18 + wave; };
    bf16x8 bq;
    auto dq_step_c = [&](int j, int t) {
      if (j == 0 || j == 3) bq = ds_frag(j == 0 ? 0 : 1, t);
      dq_step_b(dq[j], ci(j), t, bq);
    };
    __syncthreads();  // indices (the copy waves issue tiles 0 and 1 meanwhile)
    for (int t = 0; t < ntiles; ++t) {
      barrier_lds();  // (A) tile t has landed; every wave is done with tile t - 1's s_g
      const uint32_t tb = ring + (t % kBrRing) * kBwTileBytes;
      // this tile's S^T and dP^T, with tile t - 1's four dq steps between them: independent MFMAs for
      // the matrix core while the chain waits for its next K fragment
      f32x4 sacc = f32x4{}, pacc = f32x4{};
#pragma unroll
      for (int st = 0; st < 18; ++st) {
        const bf16x8 kf = lds_read16(lds_ptr(tb + qk_off + 1024 * st));
        if (st % 4 == 1 && st / 4 < kBrDqC && t > 0) dq_step_c(st / 4, t - 1);
        sacc = mfma16(kf, qf[st], sacc);
        if (st < 16) pacc = mfma16(kf, df[st], pacc);  // V = the first 512 dims
      }
      // lane: head h, keys 4*g16 + e. s_g's 16-byte chunks are swizzled by key (chunk c of key row k at
      // c ^ 2((k / 4) % 4)), so that the four key rows one write instruction touches fall on
      // different banks; dS'^T takes the lane's four keys in one 8-byte write.
      uint16_t dsb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 4 * g16 + e;
        const bool ok = s_idx[t * kBwKeys + key] >= 0;
        const float p = ok ? fast_exp2(__builtin_fmaf(sacc[e], sl2, -lse2)) : 0.0f;
        const float ds = a.scale * p * (pacc[e] - Dh);
        dsb[e] = f32_to_bf16(ds);
        const int sw = 16 * g16;  // 2((key / 4) % 4) chunks of 8 values
        s_g[key * kGCols + (h ^ sw)] = dsb[e];
        s_g[key * kGCols + ((kBrHeads + h) ^ sw)] = f32_to_bf16(p);
      }
      *reinterpret_cast<DSA_LDS u32x2*>(lds_ptr(lds_addr_of(&s_dsT[t & 1][0]) + (h * kBwKeys + 4 * g16) * 2)) =
          u32x2{static_cast<uint32_t>(dsb[0]) | (static_cast<uint32_t>(dsb[1]) << 16),
                static_cast<uint32_t>(dsb[2]) | (static_cast<uint32_t>(dsb[3]) << 16)};
      barrier_lds();  // (B) the tile's P and dS' are in LDS
      {
        // chunk q = 64 * wave + lane of the tile's 384 (key q / 24, chunk q % 24), stored in place
        const int q = kWave * wave + lane, key = q / 24, c = q % 24;
        const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(
            lds_ptr(lds_addr_of(&s_g[0]) + key * kGCols * 2 + 16 * (c ^ (2 * ((key >> 2) & 3)))));
        *reinterpret_cast<u32x4*>(gdst + static_cast<int64_t>(t * kBwKeys) * kGCols) = v;
      }
    }
    if (ntiles > 0) {
#pragma unroll
      for (int j = 0; j < kBrDqC; ++j) dq_step_c(j, ntiles - 1);
    }
#pragma unroll
    for (int j = 0; j < kBrDqC; ++j) dq_store(dq[j], ci(j));
  } else {
    // ================================ copy wave ================================
    // Specialised per copy wave, so that its dq tiles (and their head tiles) are known at compile
    // time: each tile's dS'^T fragment of a head tile is then read once for all of the wave's dq
    // tiles in it (the wave's fifteen tiles span at most two head tiles).
    auto copy_wave = [&](auto cw_c) {
      constexpr int cw = decltype(cw_c)::value;  // copies cw, cw + 2, ... of each tile: tile column granules 4c + g16
      constexpr int i0 = kBrCompute * kBrDqC + kBrDqX * cw;
      const int my_row = i16 ^ (4 * g16);
      auto issue_tile = [&](int t) {
        // one 32-bit byte offset per tile (row s_key of kv, granule g16); copy c's 64-byte step is
        // the immediate offset, which moves the LDS address too
        const uint32_t voff = static_cast<uint32_t>(max(s_idx[t * kBwKeys + my_row], 0)) * (kLatent * 2) + 16 * g16;
        bw_gather_copies<cw>(a.kv, voff, ring + (t % kBrRing) * kBwTileBytes);
      };
      f32x16 dq[kBrDqX];
#pragma unroll
      for (int i = 0; i < kBrDqX; ++i) dq[i] = f32x16{};
      auto dq_steps = [&](int t) {
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < kBrDqX; ++i) {  // unrolled: the head-tile test folds to a constant
          if (i == 0 || (i0 + i) / 18 != (i0 + i - 1) / 18) b = ds_frag((i0 + i) / 18, t);
          dq_step_b(dq[i], i0 + i, t, b);
        }
      };
      __syncthreads();  // indices
      if (ntiles > 0) issue_tile(0);
      if (ntiles > 1) issue_tile(1);
      for (int t = 0; t < ntiles; ++t) {
        // tile t's copies are complete; tile t + 1's (nine per wave) may still be in flight
        if (t + 1 < ntiles) wait_vmem_le<9>();
        else wait_vmem();
        barrier_lds();  // (A)
        if (t + 2 < ntiles) issue_tile(t + 2);  // into the slot of tile t - 2, which every wave is done with
        // tile t - 1's dq, beside the compute waves' S^T and dP^T of tile t
        if (t > 0) dq_steps(t - 1);
        barrier_lds();  // (B)
      }
      if (ntiles > 0) dq_steps(ntiles - 1);
#pragma unroll
      for (int i = 0; i < kBrDqX; ++i) dq_store(dq[i], i0 + i);
    };
    if (wave == kBrCompute) copy_wave(std::integral_constant<int, 0>{});
    else copy_wave(std::integral_constant<int, 1>{});
  }
}

// ---------------------------------------------------------------------------------------------
// k_dkv: the dkv contribution of each (row, selected key) pair over all 96 heads,
//   contrib(r, j) = dS'[r, j, :] q[r] + P[r, j, :] do_lat[r]   (576 values),
// rounded to bf16 once after the FP32 sum over the heads. One workgroup of eight waves per (row,
// group of 192 latent dims); the three groups of a row are dealt to one XCD, so that the row's g
// comes from HBM once. The group's B operands (q and do_lat of its dims, 96 heads each; do_lat is
// zero past dim 512) are built once in LDS in MFMA operand order. Each wave takes 32-key tiles: the
// tile's dS' and P rows of g are the A operands (the next tile's loaded ahead, and loaded once for
// all 192 dims), over six 32-dim N tiles. N tile nt holds dims 6c + nt (c = lane % 32), so a lane
// ends with six adjacent dims of each of its keys and stores them as 12 bytes.
// contrib is [3][chunk rows * k][192] bf16: group, the pair's position in key order (from the pair
// sort), dim within the group.
constexpr int kDkGroups = 3;
constexpr int kDkGDims = kLatent / kDkGroups;  // 192
constexpr int kDkNT = kDkGDims / 32;           // 6 N tiles of 32 dims
constexpr int kDkWaves = 8;
constexpr int kDkHeads = 96;
constexpr int kDkKS = kDkHeads / 16;           // 6 K steps of 16 heads
typedef __attribute__((ext_vector_type(3))) unsigned int u32x3;

__global__ __launch_bounds__(kDkWaves * kWave, 1) void k_dkv(DkvArgs a) {
  // fragment (p, ks, nt): 64 lanes x 16 bytes, lane l holding heads 16ks + 8(l/32) .. +8 of dim
  // 6(l%32) + nt of part p (0: q, 1: do_lat)
  __shared__ __attribute__((aligned(16))) uint8_t s_b[2 * kDkKS * kDkNT * 1024];
  __shared__ __attribute__((aligned(16))) uint16_t s_nat[kDkHeads * kDkGDims];  // one part, [head][dim]
  __shared__ __attribute__((aligned(16))) int32_t s_pos[kBwMaxIdx + 32];  // the row's pairs' positions in key order
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int b = blockIdx.x, xcd = b % 8, loc = b / 8;
  const int crow = (loc / kDkGroups) * 8 + xcd, grp = loc % kDkGroups;
  if (crow >= a.chunk_rows) return;  // uniform over the workgroup
  const int r = a.chunk_r0 + crow;
  const int t_row = a.row0 + r;
  const int keff = min(a.k, t_row - doc_begin(a.cu, a.n_docs, t_row) + 1);
  const int ntiles = (keff + 31) / 32;
  const int d0 = kDkGDims * grp;
  const int32_t* __restrict__ pr = a.pos + static_cast<int64_t>(crow) * a.k;
  for (int j = threadIdx.x; j < ntiles * 32; j += kDkWaves * kWave) s_pos[j] = j < keff ? pr[j] : -1;
  for (int p = 0; p < 2; ++p) {
    // the part's 96 x 192 values in natural order, 24 granules of 8 dims per head
    for (int gi = threadIdx.x; gi < kDkHeads * (kDkGDims / 8); gi += kDkWaves * kWave) {
      const int h = gi / (kDkGDims / 8), gg = gi % (kDkGDims / 8), d = d0 + 8 * gg;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (p == 0)
        v = *reinterpret_cast<const u32x4*>(a.q + (static_cast<int64_t>(r) * kDkHeads + h) * kLatent + d);
      else if (d < kVDim)
        v = *reinterpret_cast<const u32x4*>(a.do_lat + (static_cast<int64_t>(crow) * kDkHeads + h) * kVDim + d);
      *reinterpret_cast<u32x4*>(&s_nat[h * kDkGDims + 8 * gg]) = v;
    }
    __syncthreads();
    for (int fi = threadIdx.x; fi < kDkKS * kDkNT * kWave; fi += kDkWaves * kWave) {
      const int ks = fi / (kDkNT * kWave), nt = (fi / kWave) % kDkNT, l = fi % kWave;
      const int h0 = 16 * ks + 8 * (l >> 5), d = 6 * (l & 31) + nt;
      u32x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = static_cast<uint32_t>(s_nat[(h0 + 2 * i) * kDkGDims + d]) |
               (static_cast<uint32_t>(s_nat[(h0 + 2 * i + 1) * kDkGDims + d]) << 16);
      *reinterpret_cast<u32x4*>(&s_b[((p * kDkKS + ks) * kDkNT + nt) * 1024 + 16 * l]) = v;
    }
    __syncthreads();  // the fragments are complete, and s_nat may be refilled
  }
  const int hh = lane >> 5, col = lane & 31;
  const uint32_t sb = lds_addr_of(&s_b[0]) + 16 * lane;
  const uint16_t* __restrict__ grow = a.g + static_cast<int64_t>(crow) * a.g_stride * kGCols;
  const int64_t npairs = static_cast<int64_t>(a.chunk_rows) * a.k;
  uint16_t* __restrict__ out = a.contrib + grp * npairs * kDkGDims + 6 * col;
  // A operands: key 32t + lane%32, heads 16ks + 8(lane/32) .. +8 of dS' (p = 0) and P (p = 1); two
  // waves per SIMD hide each other's loads
  const uint16_t* __restrict__ ga0 = grow + static_cast<int64_t>(col) * kGCols + 8 * hh;
  for (int t = wave; t < ntiles; t += kDkWaves) {
    bf16x8 af[2][kDkKS];
    const uint16_t* ga = ga0 + static_cast<int64_t>(32 * t) * kGCols;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ks = 0; ks < kDkKS; ++ks) af[p][ks] = *reinterpret_cast<const bf16x8*>(ga + 96 * p + 16 * ks);
    f32x16 acc[kDkNT];
#pragma unroll
    for (int nt = 0; nt < kDkNT; ++nt) acc[nt] = f32x16{};
    // one K step at a time: its six B fragments from LDS, then its six MFMAs (the fragments of all
    // twelve steps would not fit in registers beside the accumulators)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int ks = 0; ks < kDkKS; ++ks) {
        bf16x8 bv[kDkNT];
#pragma unroll
        for (int nt = 0; nt < kDkNT; ++nt) bv[nt] = lds_read16(lds_ptr(sb + ((p * kDkKS + ks) * kDkNT + nt) * 1024));
#pragma unroll
        for (int nt = 0; nt < kDkNT; ++nt) acc[nt] = mfma32(af[p][ks], bv[nt], acc[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    // element 4g + e: key 32t + 8g + 4(lane/32) + e, dims 6(lane%32) .. +6 of the group, stored at
    // the pair's position in key order; pairs without a usable index have none and are not stored
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const i32x4 kk = *reinterpret_cast<const DSA_LDS i32x4*>(lds_ptr(lds_addr_of(&s_pos[32 * t + 8 * g + 4 * hh])));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * g + e;
        if (kk[e] >= 0)
          *reinterpret_cast<u32x3*>(out + static_cast<int64_t>(kk[e]) * kDkGDims) =
              u32x3{pack_bf16x2(acc[0][i], acc[1][i]), pack_bf16x2(acc[2][i], acc[3][i]), pack_bf16x2(acc[4][i], acc[5][i])};
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Summing the contributions per key without atomics on dkv: a counting sort of the chunk's usable
// (row, j) pairs by key index (count, exclusive scan, and each pair's position in key order), then
// k_dkv stores each pair's contribution at its position and one wave per key adds its contiguous
// 576-float rows to dkv, which no other wave of the pass touches. A pair's rank among its key's pairs
// is the value its count's integer atomic returns (one per pair, not one per element), so the order of
// a key's pairs, and the last bits of its sum, may differ from run to run.
__device__ __forceinline__ int pair_key(const DkvListArgs& a, int crow, int j) {
  const int t_row = a.row0 + a.chunk_r0 + crow;
  const int keff = min(a.k, t_row - doc_begin(a.cu, a.n_docs, t_row) + 1);
  if (j >= keff) return -1;
  const int v = a.idx[static_cast<int64_t>(a.chunk_r0 + crow) * a.k + j];
  return (v >= 0 && v < a.T) ? v : -1;
}

// count[key] += 1 per pair; list takes the pair's rank among its key's pairs (-1 without a usable key).
__global__ __launch_bounds__(256) void k_pairs_count(DkvListArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x, crow = blockIdx.y;
  if (j >= a.k) return;
  const int key = pair_key(a, crow, j);
  a.list[static_cast<int64_t>(crow) * a.k + j] = key >= 0 ? atomicAdd(a.count + key, 1) : -1;
}

// Exclusive scan of count[0 .. T) into start (start[T] = total), in two passes over
// tiles of kPairScanTile keys: the tiles' sums, then each tile adds the sums of the tiles before it to
// a workgroup scan of its own keys. 256 threads, 16 consecutive keys each.
constexpr int kScanPer = kPairScanTile / 256;
static_assert(kScanPer == 16, "four 16-byte loads per thread");

__device__ __forceinline__ void load_counts(const DkvListArgs& a, int i0, int (&c)[kScanPer]) {
  if (i0 + kScanPer <= a.T) {
#pragma unroll
    for (int v = 0; v < kScanPer / 4; ++v) {
      const i32x4 x = *reinterpret_cast<const i32x4*>(a.count + i0 + 4 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) c[4 * v + e] = x[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kScanPer; ++e) c[e] = i0 + e < a.T ? a.count[i0 + e] : 0;
  }
}

// Sum over the workgroup of x (256 threads); every thread gets it.
__device__ __forceinline__ int block_sum(int x, int* s_part) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if (threadIdx.x % kWave == 0) s_part[threadIdx.x / kWave] = x;
  __syncthreads();
  return s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

__global__ __launch_bounds__(256) void k_pairs_tile_sums(DkvListArgs a) {
  __shared__ int s_part[4];
  int c[kScanPer];
  load_counts(a, blockIdx.x * kPairScanTile + kScanPer * threadIdx.x, c);
  int sum = 0;
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) sum += c[e];
  sum = block_sum(sum, s_part);
  if (threadIdx.x == 0) a.bsum[blockIdx.x] = sum;
}

__global__ __launch_bounds__(256) void k_pairs_scan(DkvListArgs a) {
  __shared__ int s_part[4];
  __shared__ int s_wave[4];
  const int b = blockIdx.x, lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int before = 0;  // the sums of the tiles before this one
  for (int t = threadIdx.x; t < b; t += 256) before += a.bsum[t];
  before = block_sum(before, s_part);
  const int i0 = b * kPairScanTile + kScanPer * threadIdx.x;
  int c[kScanPer];
  load_counts(a, i0, c);
  int sum = 0;
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) sum += c[e];
  // inclusive scan of the threads' sums: within the wave, then over the four wave totals
  int x = sum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int run = before + x - sum;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) {
    if (i0 + e < a.T) a.start[i0 + e] = run;
    run += c[e];
  }
  if (b == gridDim.x - 1 && threadIdx.x == 255) a.start[a.T] = run;  // the total
}

// Each pair's position in key order, start[key] + its rank (-1 stays for a pair without a usable
// key): k_dkv stores the pair's contribution there, so that each key's contributions are contiguous
// for k_dkv_sum.
__global__ __launch_bounds__(256) void k_pairs_place(DkvListArgs a) {
  const int j = blockIdx.x * 256 + threadIdx.x, crow = blockIdx.y;
  if (j >= a.k) return;
  int* slot = a.list + static_cast<int64_t>(crow) * a.k + j;
  const int rank = *slot;
  if (rank >= 0) *slot = a.start[pair_key(a, crow, j)] + rank;
}

// One wave per key: the sum of its pairs' contributions, contiguous in contrib at positions
// start[key] .. start[key + 1] - 1, added to dkv[key]. The two half-waves take alternate pairs (lane
// 32h + l, l < 24, takes pairs start + h, start + h + 2, .. and dims 8l .. 8l + 7 of each group, in
// 16-byte loads, four pairs in flight), and the halves' sums are added before the store.
__global__ __launch_bounds__(256) void k_dkv_sum(DkvListArgs a) {
  const int key = blockIdx.x * 4 + threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (key >= a.T) return;
  const int p0 = a.start[key], p1 = a.start[key + 1];
  if (p0 == p1) return;  // uniform over the wave
  const int h = lane >> 5, l = lane & 31;
  const bool active = l < kDkGDims / 8;
  const int64_t gstride = static_cast<int64_t>(a.chunk_rows) * a.k * kDkGDims;  // bf16 per group
  const uint16_t* __restrict__ base = a.contrib + 8 * (active ? l : 0);
  float acc[kDkGroups][8];
#pragma unroll
  for (int q = 0; q < kDkGroups; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[q][i] = 0.0f;
  auto add = [&](const u32x4& w, int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[q][2 * i] += __uint_as_float(w[i] << 16);
      acc[q][2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
    }
  };
  if (active) {
    int p = p0 + h;
    for (; p + 6 < p1; p += 8) {
      u32x4 v[4][kDkGroups];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t* src = base + static_cast<int64_t>(p + 2 * u) * kDkGDims;
#pragma unroll
        for (int q = 0; q < kDkGroups; ++q) v[u][q] = *reinterpret_cast<const u32x4*>(src + gstride * q);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < kDkGroups; ++q) add(v[u][q], q);
    }
    for (; p < p1; p += 2) {
      const uint16_t* src = base + static_cast<int64_t>(p) * kDkGDims;
#pragma unroll
      for (int q = 0; q < kDkGroups; ++q) add(*reinterpret_cast<const u32x4*>(src + gstride * q), q);
    }
  }
  // the upper half's sums onto the lower half (every lane takes part in the exchange)
#pragma unroll
  for (int q = 0; q < kDkGroups; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[q][i] += __shfl_xor(acc[q][i], 32);
  if (h == 0 && active) {
    float* dst = a.dkv + static_cast<int64_t>(key) * kLatent + 8 * l;
#pragma unroll
    for (int q = 0; q < kDkGroups; ++q)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x4* d = reinterpret_cast<f32x4*>(dst + kDkGDims * q + 4 * c);
        const f32x4 o = *d;
        *d = f32x4{o[0] + acc[q][4 * c], o[1] + acc[q][4 * c + 1], o[2] + acc[q][4 * c + 2], o[3] + acc[q][4 * c + 3]};
      }
  }
}

// ---------------------------------------------------------------------------------------------
// dW_UV[h] += o_lat[rows, h]^T do[rows, h]: a workgroup per (head, kDwRows rows), eight waves of 64
// latent dims x 128 outputs; K = rows in steps of 16 staged in LDS (o_lat 16 x 512, do 16 x 128) in
// the forward's tile layout and read transposed for both operands. The copies run kDwDepth steps
// ahead through a ring of kDwDepth + 1 buffers, and each workgroup adds its 512 x 128 partial sums
// with atomics once, so the rows per workgroup set the number of atomics.
constexpr int kDwRows = 1024;
constexpr int kDwWaves = 8;
constexpr int kDwDepth = 4;
constexpr int kDwRing = kDwDepth + 1;

__global__ __launch_bounds__(kDwWaves * kWave, 1) void k_dwuv(DwArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_o[kDwRing][16 * kVDim * 2];  // 16 KB each
  __shared__ __attribute__((aligned(16))) uint8_t s_d[kDwRing][16 * kODim * 2];  // 4 KB each
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kDwRows;
  const int nsteps = (min(kDwRows, a.rows - r0) + 15) / 16;
  const int H = a.H;
  const int my_row = i16 ^ (4 * g16);
  // copies of step s into ring slot b: o_lat columns 4c + g16 (c < 16) and do columns 4c + g16
  // (c < 4): 20 copies, waves take copies wave, wave + 8, wave + 16 (three for waves 0-3, two for 4-7)
  auto issue = [&](int s, int b) {
    const int row = min(r0 + 16 * s + my_row, a.rows - 1);
    const int64_t rh = static_cast<int64_t>(row) * H + h;
    for (int c = wave; c < 20; c += kDwWaves) {
      if (c < 16) copy16_to_lds(a.o_lat + rh * kVDim + 8 * (4 * c + g16), lds_ptr(lds_addr_of(&s_o[b][0]) + 1024 * c));
      else copy16_to_lds(a.d_o + rh * kODim + 8 * (4 * (c - 16) + g16), lds_ptr(lds_addr_of(&s_d[b][0]) + 1024 * (c - 16)));
    }
  };
  const int hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;
  const int vc = 2 * chh + (q4 >> 1);
  const uint32_t v_off1 = (vc * 16 + ((8 * hh + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const uint32_t v_off2 = (vc * 16 + ((8 * hh + 4 + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  // rows past the chunk are staged as the last row again; their contribution is removed by a zero
  // factor: the do operand of such rows is zeroed in registers
  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};
  for (int s = 0; s < kDwDepth && s < nsteps; ++s) issue(s, s);
  int slot = 0;  // ring slot of step s
  for (int s = 0; s < nsteps; ++s) {
    // step s's copies of this wave have landed once at most the later steps' copies are outstanding
    if (s + kDwDepth - 1 < nsteps) {
      if (wave < 4) wait_vmem_le<3 * (kDwDepth - 1)>();
      else wait_vmem_le<2 * (kDwDepth - 1)>();
    } else {
      wait_vmem();
    }
    barrier_lds();  // every wave's copies of step s have landed; step s - 1's slot is free
    if (s + kDwDepth < nsteps) issue(s + kDwDepth, slot == 0 ? kDwRing - 1 : slot - 1);
    const uint32_t ob = lds_addr_of(&s_o[slot][0]), db = lds_addr_of(&s_d[slot][0]);
    slot = slot == kDwRing - 1 ? 0 : slot + 1;
    // this lane's 8 K values are rows 16*s + 8*hh + (0..3) and + 4 .. 7
    const int valid_lo = min(max(a.rows - (r0 + 16 * s + 8 * hh), 0), 8);
    u32x4 bv[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const u32x2 v1 = lds_read_tr16(lds_ptr(db + v_off1 + 1024 * nt));
      const u32x2 v2 = lds_read_tr16(lds_ptr(db + v_off2 + 1024 * nt));
      bv[nt] = u32x4{v1[0], v1[1], v2[0], v2[1]};
      if (valid_lo < 8) {
        // zero the K values of rows past the end (element e of 8 is row 8*hh + e)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= valid_lo) bv[nt][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int ct = 2 * wave + mt;  // latent tile of 32 dims
      const u32x2 v1 = lds_read_tr16(lds_ptr(ob + v_off1 + 1024 * ct));
      const u32x2 v2 = lds_read_tr16(lds_ptr(ob + v_off2 + 1024 * ct));
      const u32x4 av = {v1[0], v1[1], v2[0], v2[1]};
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = mfma32(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv[nt]), acc[mt][nt]);
    }
  }
  // element e of tile (mt, nt): latent dim 32*(2*wave + mt) + 8*(e/4) + 4*hh + e%4, output 32*nt + lane%32
  float* __restrict__ dW = a.dW + static_cast<int64_t>(h) * kVDim * kODim;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int c = 32 * (2 * wave + mt) + 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) atomicAdd(dW + c * kODim + 32 * nt + (lane & 31), acc[mt][nt][e]);
    }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_sink_sum(const SinkSumArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.H <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sink_sum, dim3(static_cast<unsigned>(a.H)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(const BwdPrepArgs& a, hipStream_t st) {
  const int64_t n = static_cast<int64_t>(a.rows) * a.H;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bwd_prep, dim3(static_cast<unsigned>((n + 7) / 8)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(k_fill_zero, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_pairs_sort(const DkvListArgs& a, hipStream_t st) {
  if (a.chunk_rows <= 0) return hipSuccess;
  if (launch_fill_zero(reinterpret_cast<float*>(a.count), a.T, st) != hipSuccess) return hipGetLastError();  // int 0 == float +0 bits
  const dim3 pairs((a.k + 255) / 256, a.chunk_rows);
  hipLaunchKernelGGL(k_pairs_count, pairs, dim3(256), 0, st, a);
  const dim3 tiles((a.T + kPairScanTile - 1) / kPairScanTile);
  hipLaunchKernelGGL(k_pairs_tile_sums, tiles, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_pairs_scan, tiles, dim3(256), 0, st, a);
  hipLaunchKernelGGL(k_pairs_place, pairs, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dkv_sum(const DkvListArgs& a, hipStream_t st) {
  if (a.chunk_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_dkv_sum, dim3((a.T + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dkv(const DkvArgs& a, hipStream_t st) {
  if (a.chunk_rows <= 0) return hipSuccess;
  const int blocks = (a.chunk_rows + 7) / 8 * 8 * kDkGroups;
  hipLaunchKernelGGL(k_dkv, dim3(blocks), dim3(kDkWaves * kWave), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.H != kBrHeads || a.k > kBwMaxIdx || a.chunk_rows < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sparse_mla_bwd_row, dim3(static_cast<unsigned>(a.chunk_rows)), dim3(kBrWaves * kWave), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dwuv(const DwArgs& a, hipStream_t st) {
  if (a.rows < 1) return hipSuccess;
  hipLaunchKernelGGL(k_dwuv, dim3(static_cast<unsigned>((a.rows + kDwRows - 1) / kDwRows), a.H), dim3(kDwWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

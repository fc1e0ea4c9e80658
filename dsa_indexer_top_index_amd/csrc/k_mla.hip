// Sparse latent attention over the selected KV rows (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, Implementation Limits bullets 1-2:
// the sparse kernels attend directly to the selected latent KV rows and never expand per-head
// K/V; kimi_k3 API index, KimiK3TextConfig: kv_lora_rank 512 + 64 unrotated dims, 96 heads;
// archdiff blueprint tagline: no positional encoding):
//   for query t, head h and selected rows s_j:
//     l_j = scale * q[t,h,:] . kv[s_j,:]          (576 dims)
//     o_lat[t,h,:] = softmax_j(l) . kv[s_j, 0:512]
//
// Kernel design: one wave per (query row, group of 32 heads), four independent waves per
// workgroup, rows taken longest first, and the three head groups of a row placed on one XCD so
// its gathered rows are shared through that XCD's L2.
//  - Gather: the 16 selected rows of a tile (16 x 1152 bytes) are copied global -> LDS with
//    asynchronous 16-byte copies (18 wave instructions, each filling four 16-byte columns of all
//    16 rows), double buffered so the next tile's gather overlaps this tile's math. The layout
//    is column-major in 16-byte granules with a row XOR, so the QK operand reads and the
//    transposed V reads are bank-conflict free and every address is affine in the loop index.
//  - QK^T: v_mfma_f32_16x16x32_bf16 computes S^T[16 keys x 16 heads] (two head tiles), K = 576,
//    with the head group's q fragments resident in registers.
//  - Softmax in FP32 (base 2) against a per-head reference maximum taken from the first tile;
//    the accumulators are never rescaled inside the loop. If a later logit exceeds the
//    reference by more than 2^64 (never for bounded inputs, but possible in principle), the row
//    restarts with the larger reference, so no value can overflow.
//  - PV: P (bf16) becomes the A operand of v_mfma_f32_32x32x16_bf16 with the 32 heads as M
//    through one permlane16 swap per register; V is read straight from the natural row layout
//    with ds_read_b64_tr_b16, N = 512 latent dims, K = 16 keys.
//  - Epilogue: divide by the softmax sum, write o_lat (bf16) for the up-projection kernel, and
//    the natural-log normaliser lse if requested.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kMlaWaves = 4;
constexpr int kTileKeys = 16;
constexpr int kRowGran = kLatent * 2 / 16;            // 72 granules (16 B) per latent row
constexpr int kTileBytes = kTileKeys * kRowGran * 16;  // 18432: 18 wave copies of 1 KB
constexpr float kRestartGap = 64.0f;                   // log2 headroom of the running maximum
constexpr int kMaxRestarts = 8;

// Tile layout in LDS: granule (row r, column c) lives at slot c*16 + (r ^ 4*(c%4)). One wave
// copy fills four columns of all 16 rows; the QK operand reads (16 rows, one column) and the
// transposed V reads (4 rows x 4 columns per 16 lanes) both hit 16 distinct bank quads, and
// every read address is affine in the loop counter.
__device__ __forceinline__ int mla_slot(int r, int c) { return c * 16 + (r ^ (4 * (c & 3))); }

// One wave handles 32 heads; a layer with fewer heads per group zero-fills the rest.
__global__ __launch_bounds__(256, 1) void k_sparse_mla(MlaArgs a) {
  constexpr int NT = 2;        // 16-head tiles per wave
  constexpr int HG = 16 * NT;  // heads per wave
  __shared__ __attribute__((aligned(16))) uint8_t s_tiles[kMlaWaves][2][kTileBytes];
  __shared__ float s_vec[kMlaWaves][32];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int n_hg = (a.H + HG - 1) / HG;
  const int items = a.chunk_rows * n_hg;
  const int item = kMlaWaves * xcd_local_block(blockIdx.x, gridDim.x) + wave;
  if (item >= items) return;  // waves are independent: no workgroup barrier in this kernel

  const int rr = a.chunk_rows - 1 - item / n_hg;  // longest rows first
  const int hg = item % n_hg;
  const int r = a.chunk_r0 + rr;                  // local row
  const int t = a.row0 + r;
  const int b = doc_begin(a.cu, a.n_docs, t);
  const int keff = min(a.k, t - b + 1);
  const int ntiles = (keff + kTileKeys - 1) / kTileKeys;
  const int32_t* __restrict__ ix = a.idx + static_cast<int64_t>(r) * a.k;
  const int T = a.T;
  const int g16 = lane >> 4, i16 = lane & 15;

  // q fragments: B operand of S^T = K Q^T. lane: head 16*nt + i16, dims 32*st + 8*g16 .. +8.
  bf16x8 qf[NT][18];
  const int hv = min(HG, a.H - hg * HG);  // valid heads in this group (32, or 16 for a 16-head layer)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool live = 16 * nt + i16 < hv;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(r) * a.H + hg * HG + (live ? 16 * nt + i16 : 0)) * kLatent + 8 * g16;
#pragma unroll
    for (int st = 0; st < 18; ++st) qf[nt][st] = live ? *reinterpret_cast<const bf16x8*>(qrow + 32 * st) : bf16x8{};
  }

  DSA_LDS uint8_t* tiles = (DSA_LDS uint8_t*)(&s_tiles[wave][0][0]);
  // gather: this lane always fills row slot i16 of column 4*i + g16
  const int my_row = i16 ^ (4 * g16);
  const uint8_t* kv_col = reinterpret_cast<const uint8_t*>(a.kv) + 16 * g16;
  // QK operand: row i16, column 4*st + g16
  const int qk_off = (g16 * 16 + (i16 ^ (4 * g16))) * 16;
  // V operand (transposed reads): rows 8*hh + s4 (+4), column 4*ct + 2*chh + q4/2
  const int hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;
  const int vc = 2 * chh + (q4 >> 1);
  const int v_off1 = (vc * 16 + ((8 * hh + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const int v_off2 = (vc * 16 + ((8 * hh + 4 + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);

  auto fetch_idx = [&](int tile) -> int {
    const int j = tile * kTileKeys + lane;
    return (lane < kTileKeys && tile < ntiles && j < keff) ? ix[j] : -1;
  };
  auto issue_tile = [&](int my_idx, int buf) {
    const int src = (my_idx >= 0 && my_idx < T) ? my_idx : 0;
    const uint8_t* g = kv_col + static_cast<int64_t>(__shfl(src, my_row)) * (kLatent * 2);
    DSA_LDS uint8_t* dst = tiles + buf * kTileBytes;
#pragma unroll
    for (int i = 0; i < kRowGran / 4; ++i) copy16_to_lds(g + 64 * i, dst + 1024 * i);
  };
  auto valid_mask = [&](int my_idx) -> uint32_t {
    return static_cast<uint32_t>(ballot(my_idx >= 0 && my_idx < T) & 0xffffull);
  };

  f32x16 O[16];
  float m_ref[NT], l_part[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) m_ref[nt] = -INFINITY;

  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) O[ct] = f32x16{};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_part[nt] = 0.0f;
    int idx_cur = fetch_idx(0);
    uint32_t vmask = valid_mask(idx_cur);
    issue_tile(idx_cur, 0);
    int idx_next = fetch_idx(1);
    bool restart = false;

    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile & 1;
      wait_vmem();  // this tile is in LDS and idx_next has arrived
      const uint32_t vmask_next = valid_mask(idx_next);
      if (tile + 1 < ntiles) issue_tile(idx_next, buf ^ 1);
      const int idx_after = fetch_idx(tile + 2);
      const DSA_LDS uint8_t* tb = tiles + buf * kTileBytes;

      // ---- S^T = K Q^T : rows = 16 keys, cols = heads, K = 576 in 18 steps
      f32x4 sacc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt] = f32x4{};
#pragma unroll
      for (int st = 0; st < 18; ++st) {
        const bf16x8 kf = lds_read16(tb + qk_off + 1024 * st);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[nt] = mfma16(kf, qf[nt][st], sacc[nt]);
      }

      // ---- softmax numerators (base 2). lane: head 16*nt + i16, keys 4*g16 + j.
      float x[NT][4], tmax[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        tmax[nt] = -INFINITY;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool valid = (vmask >> (4 * g16 + j)) & 1u;
          x[nt][j] = valid ? sacc[nt][j] * a.scale_log2 : -INFINITY;
          tmax[nt] = fmaxf(tmax[nt], x[nt][j]);
        }
        tmax[nt] = fmaxf(tmax[nt], __shfl_xor(tmax[nt], 16));
        tmax[nt] = fmaxf(tmax[nt], __shfl_xor(tmax[nt], 32));
      }
      // The reference maximum is fixed once set; a logit more than 2^64 above it restarts the
      // row with the larger reference (the accumulators are never rescaled in the loop).
      bool risk = false, used = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        risk |= tmax[nt] > m_ref[nt] + kRestartGap;
        used |= l_part[nt] > 0.0f;
      }
      if (ballot(risk) != 0ull) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) m_ref[nt] = fmaxf(m_ref[nt], tmax[nt]);
        if (ballot(used) != 0ull && pass < kMaxRestarts) {
          restart = true;
          break;
        }
      }
      uint32_t pk[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = (x[nt][j] == -INFINITY) ? 0.0f : exp2f(x[nt][j] - m_ref[nt]);
          l_part[nt] += p[j];
        }
        pk[nt][0] = pack_bf16x2(p[0], p[1]);
        pk[nt][1] = pack_bf16x2(p[2], p[3]);
      }
      // ---- P as the A operand (rows = 32 heads, K = 16 keys): even 16-lane rows take head
      // block 0, odd rows block 1; the swap gathers keys 0..7 / 8..15 into one lane.
      const uint32_t y0 = NT == 2 ? pk[NT - 1][0] : 0u;
      const uint32_t y1 = NT == 2 ? pk[NT - 1][1] : 0u;
      const auto sw0 = __builtin_amdgcn_permlane16_swap(pk[0][0], y0, false, false);
      const auto sw1 = __builtin_amdgcn_permlane16_swap(pk[0][1], y1, false, false);
      const u32x4 pa_u = {sw0[0], sw1[0], sw0[1], sw1[1]};
      const bf16x8 pa = __builtin_bit_cast(bf16x8, pa_u);

      // ---- O += P V : N = 512 latent dims in 16 tiles of 32, V read transposed from LDS.
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) {
        const u32x2 v1 = lds_read_tr16(tb + v_off1 + 1024 * ct);
        const u32x2 v2 = lds_read_tr16(tb + v_off2 + 1024 * ct);
        const u32x4 vb_u = {v1[0], v1[1], v2[0], v2[1]};
        O[ct] = mfma32(pa, __builtin_bit_cast(bf16x8, vb_u), O[ct]);
      }
      vmask = vmask_next;
      idx_next = idx_after;
    }
    if (!restart) break;
    wait_vmem();  // no copy may still target the tile buffers
  }

  // ---- epilogue: 1/sum, lse, o_lat (bf16) through LDS for 16-byte stores
  float* sv = s_vec[wave];
  float l_tot[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_part[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_tot[nt] = l;
  }
  wave_lds_sync();
  if (lane < 16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sv[16 * nt + lane] = l_tot[nt] > 0.0f ? 1.0f / l_tot[nt] : 0.0f;
      if (a.lse && 16 * nt + lane < hv) {
        const float lse = l_tot[nt] > 0.0f ? (m_ref[nt] + log2f(l_tot[nt])) * 0.69314718055994531f : -INFINITY;
        a.lse[static_cast<int64_t>(r) * a.H + hg * HG + 16 * nt + lane] = lse;
      }
    }
  }
  wave_lds_sync();
  f32x16 inv;
#pragma unroll
  for (int e = 0; e < 16; ++e) inv[e] = sv[8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)];
  // stage [HG heads][512] bf16 in this wave's tile buffers (no copy is in flight now)
  uint16_t* so = reinterpret_cast<uint16_t*>(&s_tiles[wave][0][0]);
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) {
    const f32x16 ov = O[ct] * inv;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int head = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      so[head * kVDim + 32 * ct + (lane & 31)] = f32_to_bf16(ov[e]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wave_lds_sync();
  uint16_t* dst = a.o_lat + (static_cast<int64_t>(rr) * a.H + hg * HG) * kVDim;
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    if (h < hv) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(so + h * kVDim + 8 * lane);
      *reinterpret_cast<u32x4*>(dst + h * kVDim + 8 * lane) = v;
    }
  }
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  const int items = a.chunk_rows * ((a.H + 31) / 32);
  dim3 grid((items + kMlaWaves - 1) / kMlaWaves), block(kMlaWaves * kWave);
  hipLaunchKernelGGL(k_sparse_mla, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

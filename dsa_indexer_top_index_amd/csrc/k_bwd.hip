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
// k_sparse_mla_bwd: one workgroup per (row, group of 32 heads), four waves. Per 16-key tile of the
//   row's selected keys (gathered into LDS with the forward's tile layout, one tile ahead):
//   - waves 0 and 1 recompute S^T (16 keys x 16 heads each, K = 576) with their q fragments in
//     registers; waves 2 and 3 compute dP^T = V do_lat^T (K = 512) with do_lat fragments in registers
//     and pass it through LDS;
//   - waves 0 and 1 form P = 2^(scale log2e S - log2e lse) and dS' = scale P (dP - D) and write both
//     in bf16 in the layouts of the next products;
//   - all waves: dq^T += K^T dS'^T on 32x32x16 MFMAs (K^T read transposed from the gathered tile,
//     the latent dims split over the waves, accumulators kept across the row), and the tile's dkv
//     rows dS' Q + P do_lat on 16x16x32 MFMAs (Q and do_lat held transposed in LDS) added to dkv
//     with FP32 atomics (16 consecutive dims of 4 keys per instruction).
// k_dwuv: dW_UV[h] += o_lat^T do over a chunk of rows, 16 rows per K step staged in LDS in the
//   forward's tile layout so that both operands are read transposed; partial sums added with atomics.
#include "dsa_device.h"
#include "dsa_kernels.h"

#include <algorithm>

namespace dsa {

constexpr int kBwHeads = 32;   // heads per workgroup
constexpr int kBwWaves = 4;
constexpr int kBwKeys = 16;    // keys per gathered tile
constexpr int kBwGran = kLatent * 2 / 16;             // 72 granules per latent row
constexpr int kBwTileBytes = kBwKeys * kBwGran * 16;  // 18 KB
constexpr int kBwMaxIdx = 2048;
constexpr int kBwAtomics = kLatent / 16 / kBwWaves * 4;  // dkv atomics per wave and tile
static_assert(kLatent / 16 % kBwWaves == 0 && kBwAtomics <= 63, "a whole number of dkv column tiles per wave; vmcnt range");
constexpr float kLog2e = 1.4426950408889634f;

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
  const float sg = 1.0f / (1.0f + __expf(-bf16_to_f32(a.gate[grh])));
  const u32x2 dov = {pack_bf16x2(sg * d4[0], sg * d4[1]), pack_bf16x2(sg * d4[2], sg * d4[3])};
  *reinterpret_cast<u32x2*>(a.d_o + rh * kODim + 4 * sub) = dov;
  if (sub == 0) {
    a.delta[rh] = D;
    a.dgate[grh] = (1.0f - sg) * D;
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBwWaves * kWave, 1) void k_sparse_mla_bwd(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[2][kBwTileBytes];       // 36 KB
  __shared__ __attribute__((aligned(16))) uint16_t s_qT[kLatent * kBwHeads];       // Q^T [dim][head], 36 KB
  __shared__ __attribute__((aligned(16))) uint16_t s_dT[kVDim * kBwHeads];         // do_lat^T [dim][head], 32 KB
  __shared__ __attribute__((aligned(16))) float s_dp[2][kBwKeys * 16];             // dP [key][head] per head tile
  __shared__ __attribute__((aligned(16))) uint16_t s_ds[kBwKeys * kBwHeads];       // dS' [key][head]
  __shared__ __attribute__((aligned(16))) uint16_t s_p[kBwKeys * kBwHeads];        // P [key][head]
  __shared__ __attribute__((aligned(16))) uint16_t s_dsT[kBwHeads * kBwKeys];      // dS'^T [head][key]
  __shared__ int32_t s_idx[kBwMaxIdx + kBwKeys];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int ng = a.H / kBwHeads;
  const int crow = blockIdx.x / ng, hg = blockIdx.x % ng;  // chunk-local row, head group
  const int r = a.chunk_r0 + crow;                        // local row
  const int t_row = a.row0 + r;
  const int H = a.H, T = a.T;
  const int keff = min(a.k, t_row - doc_begin(a.cu, a.n_docs, t_row) + 1);
  const int ntiles = (keff + kBwKeys - 1) / kBwKeys;
  const int h0 = hg * kBwHeads;

  // the row's indices (-1: no usable key), and Q^T and do_lat^T of the head group in LDS
  const int32_t* __restrict__ ix = a.idx + static_cast<int64_t>(r) * a.k;
  for (int j = threadIdx.x; j < ntiles * kBwKeys; j += kBwWaves * kWave) {
    const int v = j < keff ? ix[j] : -1;
    s_idx[j] = (v >= 0 && v < T) ? v : -1;
  }
  const uint16_t* __restrict__ qrow = a.q + (static_cast<int64_t>(r) * H + h0) * kLatent;
  const uint16_t* __restrict__ drow = a.do_lat + (static_cast<int64_t>(crow) * H + h0) * kVDim;
  for (int gi = threadIdx.x; gi < kBwHeads * kBwGran; gi += kBwWaves * kWave) {
    const int h = gi / kBwGran, g = gi % kBwGran;
    const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + h * kLatent + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_qT[(8 * g + e) * kBwHeads + h] = static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
  }
  for (int gi = threadIdx.x; gi < kBwHeads * (kVDim / 8); gi += kBwWaves * kWave) {
    const int h = gi / (kVDim / 8), g = gi % (kVDim / 8);
    const u32x4 v = *reinterpret_cast<const u32x4*>(drow + h * kVDim + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; ++e) s_dT[(8 * g + e) * kBwHeads + h] = static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1)));
  }
  // Waves 0 and 1: q fragments (B of S^T = K Q^T: head 16*wave + i16, dims 32*st + 8*g16); their
  // heads' lse (log2 units) and D. Waves 2 and 3: do_lat fragments of heads 16*(wave-2) + i16.
  const int my_h = 16 * (wave & 1) + i16;  // head within the group of this lane's score column
  bf16x8 fr[18];
  if (wave < 2) {
#pragma unroll
    for (int st = 0; st < 18; ++st) fr[st] = *reinterpret_cast<const bf16x8*>(qrow + my_h * kLatent + 32 * st + 8 * g16);
  } else {
#pragma unroll
    for (int st = 0; st < 16; ++st) fr[st] = *reinterpret_cast<const bf16x8*>(drow + my_h * kVDim + 32 * st + 8 * g16);
#pragma unroll
    for (int st = 16; st < 18; ++st) fr[st] = bf16x8{};
  }
  const float lse2 = wave < 2 ? a.lse[static_cast<int64_t>(r) * H + h0 + my_h] * kLog2e : 0.0f;
  const float Dh = wave < 2 ? a.delta[static_cast<int64_t>(crow) * H + h0 + my_h] : 0.0f;
  const float sl2 = a.scale * kLog2e;

  // dq^T accumulators: latent tiles dt = wave + 4*i (i < 5, dt < 18), 32 dims x 32 heads each
  f32x16 dq[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) dq[i] = f32x16{};

  // gather copies: tile column granule 4*c + g16 of row (i16 ^ 4*g16), c = 0..17 over the 4 waves
  const uint32_t ring = lds_addr_of(&s_ring[0][0]);
  const int my_row = i16 ^ (4 * g16);
  auto issue_tile = [&](int t) {
    const int s_key = s_idx[t * kBwKeys + my_row];
    const uint16_t* src = a.kv + static_cast<int64_t>(max(s_key, 0)) * kLatent + 8 * g16;
    const uint32_t base = ring + (t & 1) * kBwTileBytes;
    for (int c = wave; c < 18; c += kBwWaves) copy16_to_lds(src + 32 * c, lds_ptr(base + 1024 * c));
  };
  __syncthreads();  // indices, Q^T, do_lat^T
  if (ntiles > 0) issue_tile(0);

  // transposed reads of the tile (A = K^T: lane = latent dim, 8 keys), as in the forward's value waves
  const int hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;
  const int vc = 2 * chh + (q4 >> 1);
  const uint32_t v_off1 = (vc * 16 + ((8 * hh + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const uint32_t v_off2 = (vc * 16 + ((8 * hh + 4 + s4) ^ (4 * vc))) * 16 + 8 * (q4 & 1);
  const uint32_t qk_off = (g16 * 16 + (i16 ^ (4 * g16))) * 16;  // A of S^T / dP^T: key i16, dims 32*st + 8*g16

  for (int t = 0; t < ntiles; ++t) {
    // Tile t has landed and every wave is done with tile t - 1 and its P / dS'. The wait leaves
    // out this wave's dkv atomics of tile t - 1, the last kBwAtomics vector-memory operations it
    // issued (vector-memory operations complete in issue order): they drain while this tile runs.
    if (t == 0) wait_vmem();
    else wait_vmem_le<kBwAtomics>();
    barrier_lds();
    if (t + 1 < ntiles) issue_tile(t + 1);
    const uint32_t tb = ring + (t & 1) * kBwTileBytes;
    // ---- S^T (waves 0, 1) or dP^T (waves 2, 3): 16 keys x 16 heads
    // 18 K steps in both products (the dP waves' last two fragments are zero), so that the chain
    // unrolls with constant register indices
    f32x4 acc = f32x4{};
#pragma unroll
    for (int st = 0; st < 18; ++st) acc = mfma16(lds_read16(lds_ptr(tb + qk_off + 1024 * st)), fr[st], acc);
    // lane: head column i16, keys 4*g16 + e
    if (wave >= 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s_dp[wave - 2][(4 * g16 + e) * 16 + i16] = acc[e];
    }
    barrier_lds();
    if (wave < 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 4 * g16 + e;
        const bool ok = s_idx[t * kBwKeys + key] >= 0;
        const float p = ok ? fast_exp2(__builtin_fmaf(acc[e], sl2, -lse2)) : 0.0f;
        const float ds = a.scale * p * (s_dp[wave][key * 16 + i16] - Dh);
        const uint16_t pb = f32_to_bf16(p), db = f32_to_bf16(ds);
        s_p[key * kBwHeads + my_h] = pb;
        s_ds[key * kBwHeads + my_h] = db;
        s_dsT[my_h * kBwKeys + key] = db;
      }
    }
    barrier_lds();
    // ---- dq^T += K^T dS'^T: M = 32 latent dims, N = 32 heads, K = 16 keys
    const bf16x8 bds = *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(lds_addr_of(s_dsT) + (lane & 31) * 32 + 16 * hh));
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int dt = wave + 4 * i;
      if (dt < 18) {
        const u32x2 v1 = lds_read_tr16(lds_ptr(tb + v_off1 + 1024 * dt));
        const u32x2 v2 = lds_read_tr16(lds_ptr(tb + v_off2 + 1024 * dt));
        const u32x4 kt = {v1[0], v1[1], v2[0], v2[1]};
        dq[i] = mfma32(__builtin_bit_cast(bf16x8, kt), bds, dq[i]);
      }
    }
    // ---- dkv rows of the tile: dS' Q (576 dims) + P do_lat (512 dims): M = 16 keys, N = 16 dims,
    // K = 32 heads; lane of the result: dim i16 of the tile, keys 4*g16 + e
    const bf16x8 a_ds = *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(lds_addr_of(s_ds) + i16 * 64 + 16 * g16));
    const bf16x8 a_p = *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(lds_addr_of(s_p) + i16 * 64 + 16 * g16));
    int keyrow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) keyrow[e] = s_idx[t * kBwKeys + 4 * g16 + e];
    // Every wave issues exactly kBwAtomics atomics per tile: a padding entry adds +0 to row 0.
    float* dkv_row[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) dkv_row[e] = a.dkv + static_cast<int64_t>(max(keyrow[e], 0)) * kLatent;
#pragma unroll
    for (int i = 0; i < kLatent / 16 / kBwWaves; ++i) {
      const int n = wave + kBwWaves * i;
      const int dim = 16 * n + i16;
      f32x4 d = mfma16(a_ds, *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(lds_addr_of(s_qT) + dim * 64 + 16 * g16)), f32x4{});
      if (n < kVDim / 16)
        d = mfma16(a_p, *reinterpret_cast<const DSA_LDS bf16x8*>(lds_ptr(lds_addr_of(s_dT) + dim * 64 + 16 * g16)), d);
#pragma unroll
      for (int e = 0; e < 4; ++e) atomicAdd(dkv_row[e] + dim, keyrow[e] >= 0 ? d[e] : 0.0f);
    }
  }
  // dq of the row: lane holds head (lane % 32), dims 32*dt + 8*(e/4) + 4*hh + e%4
  float* __restrict__ dqrow = a.dq + (static_cast<int64_t>(r) * H + h0 + (lane & 31)) * kLatent;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int dt = wave + 4 * i;
    if (dt < 18) {
#pragma unroll
      for (int e = 0; e < 16; ++e) dqrow[32 * dt + 8 * (e >> 2) + 4 * hh + (e & 3)] = dq[i][e];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dW_UV[h] += o_lat[rows, h]^T do[rows, h]: a workgroup per (head, 256 rows), eight waves of 64
// latent dims x 128 outputs; K = rows in steps of 16 staged in LDS (o_lat 16 x 512, do 16 x 128) in
// the forward's tile layout and read transposed for both operands.
constexpr int kDwRows = 256;
constexpr int kDwWaves = 8;

__global__ __launch_bounds__(kDwWaves * kWave, 1) void k_dwuv(DwArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_o[2][16 * kVDim * 2];  // 2 x 16 KB
  __shared__ __attribute__((aligned(16))) uint8_t s_d[2][16 * kODim * 2];  // 2 x 4 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kDwRows;
  const int nsteps = (min(kDwRows, a.rows - r0) + 15) / 16;
  const int H = a.H;
  const int my_row = i16 ^ (4 * g16);
  // copies of step s: o_lat columns 4c + g16 (c < 16) and do columns 4c + g16 (c < 4): 20 copies, waves
  // take copies wave, wave + 8, wave + 16
  auto issue = [&](int s) {
    const int row = min(r0 + 16 * s + my_row, a.rows - 1);
    const int64_t rh = static_cast<int64_t>(row) * H + h;
    for (int c = wave; c < 20; c += kDwWaves) {
      if (c < 16) copy16_to_lds(a.o_lat + rh * kVDim + 8 * (4 * c + g16), lds_ptr(lds_addr_of(&s_o[s & 1][0]) + 1024 * c));
      else copy16_to_lds(a.d_o + rh * kODim + 8 * (4 * (c - 16) + g16), lds_ptr(lds_addr_of(&s_d[s & 1][0]) + 1024 * (c - 16)));
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
  issue(0);
  for (int s = 0; s < nsteps; ++s) {
    wait_vmem();
    __syncthreads();
    if (s + 1 < nsteps) issue(s + 1);
    const uint32_t ob = lds_addr_of(&s_o[s & 1][0]), db = lds_addr_of(&s_d[s & 1][0]);
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

hipError_t launch_sparse_mla_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.H % kBwHeads != 0 || a.k > kBwMaxIdx || a.chunk_rows < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sparse_mla_bwd, dim3(static_cast<unsigned>(a.chunk_rows) * (a.H / kBwHeads)), dim3(kBwWaves * kWave), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_dwuv(const DwArgs& a, hipStream_t st) {
  if (a.rows < 1) return hipSuccess;
  hipLaunchKernelGGL(k_dwuv, dim3(static_cast<unsigned>((a.rows + kDwRows - 1) / kDwRows), a.H), dim3(kDwWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

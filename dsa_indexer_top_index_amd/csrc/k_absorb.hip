// W_UK absorption: the latent query of sparse MLA from the per-head query without position (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, Implementation Limits, 2nd bullet:
// sparse MLA never expands the per-head keys; kimi_k3 API index, KimiK3TextConfig:
// qk_nope_head_dim 128, kv_lora_rank 512, qk_rope_head_dim 64, mla_use_nope). W_UK [H, 512, 128]
// is the key half of the kv_b_proj effective weight, so q_nope . (c_KV W_UK[h]) = q_lat . c_KV with
//   q[t,h,c]       = bf16( sum_d q_nope[t,h,d] * W_UK[h,c,d] )   c < 512, d < 128, FP32 accumulation
//   q[t,h,512 + j] = q_pe[t,h,j]                                 j < 64 (no rotation)
//
// Kernel design: a workgroup owns one head and 256 rows (four waves of 64 rows, two 32-row M tiles
// each) and all 512 latent outputs, in four passes of 128. Each lane's query fragments (K = d) are
// loaded once and stay in registers; each pass stages its 128 x 128 slice of W_UK[h] in LDS (one row
// c per 256 bytes, its 16-byte granules XOR-swizzled by c, so that 16 lanes reading one granule of
// 16 consecutive rows hit distinct banks; a weight row holds the K values of one output
// contiguously, so no transposed copy is needed) and runs v_mfma_f32_32x32x16_bf16 with rows as M,
// c as N (four 32-wide tiles) and d as K (eight steps). The next pass's weight copies are issued
// before this pass's outputs leave (through a per-wave LDS tile, in 16-byte stores), so they are in
// flight meanwhile. Workgroups of one head run one after another on one XCD, so the head's weights
// (128 KB) stay in that XCD's L2 and q_nope is read from memory once. q_pe is copied into dims
// 512..575. HBM-bound: 1.5 KB per (row, head) against 131 K flop.
// The same product with a 512-wide output and no pass-through dims gives the backward's
// do_lat = do W_UV[h]^T (W_UV has the same [H, 512, 128] layout).
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kAbWaves = 4;
constexpr int kAbRowsW = 64;                  // rows per wave: two 32-row M tiles
constexpr int kAbRows = kAbWaves * kAbRowsW;  // rows per workgroup
constexpr int kAbN = 128;                     // latent outputs per workgroup
constexpr int kNope = 128;                    // qk_nope_head_dim
constexpr int kPe = kLatent - kVDim;          // 64 unrotated dims

// LDS slot of granule g (8 values of d) of weight row c.
__device__ __forceinline__ int ab_slot(int c, int g) { return 16 * c + (g ^ (c & 15)); }

__global__ __launch_bounds__(kAbWaves * kWave, 2) void k_q_absorb(AbsorbArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_w[kAbN * kNope * 2];            // 32 KB
  __shared__ __attribute__((aligned(16))) uint16_t s_st[kAbWaves][32 * kAbN];        // 8 KB per wave
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int H = a.H, rows = a.rows;
  // consecutive logical blocks (the row blocks of one head, in order) run on one XCD
  const int nrb = (rows + kAbRows - 1) / kAbRows;
  const int lb = xcd_local_block(static_cast<int>(blockIdx.x), H * nrb);
  const int h = lb / nrb;
  const int row0 = (lb % nrb) * kAbRows + kAbRowsW * wave;
  // a workgroup whose rows all exist issues exactly kStores stores per lane and pass (below)
  const bool full = (lb % nrb + 1) * kAbRows <= rows;

  // The weight slice W_UK[h][c0 .. c0 + 128][0 .. 128] of pass c0 / 128: 2,048 granules; wave w
  // copies rows 32w .. 32w + 31 in eight copies. Copy j fills slots 512w + 64j + lane, i.e. lane i
  // brings granule g = (i % 16) ^ (c % 16) of row c = 32w + 4j + i / 16, at byte 256c + 16g of the
  // slice. The row part 1024j is the copy's immediate offset (which also moves the LDS address) and
  // the rest depends on j % 4 only: four lane offsets serve all eight copies.
  const uint32_t sw_wave = lds_addr_of(s_w) + 8192 * wave;
  uint32_t wo[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    wo[jj] = static_cast<uint32_t>(256 * (lane >> 4) + 16 * ((lane & 15) ^ (4 * jj + (lane >> 4))));
  auto copy_w = [&](int c0) {
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(a.W_UK + (static_cast<int64_t>(h) * kVDim + c0) * kNope) + 8192 * wave;
    copy16_to_lds_imm<0>(sb, wo[0], sw_wave);
    copy16_to_lds_imm<1024>(sb, wo[1], sw_wave);
    copy16_to_lds_imm<2048>(sb, wo[2], sw_wave);
    copy16_to_lds_imm<3072>(sb, wo[3], sw_wave);
    copy16_to_lds_imm<0>(sb + 4096, wo[0], sw_wave + 4096);
    copy16_to_lds_imm<1024>(sb + 4096, wo[1], sw_wave + 4096);
    copy16_to_lds_imm<2048>(sb + 4096, wo[2], sw_wave + 4096);
    copy16_to_lds_imm<3072>(sb + 4096, wo[3], sw_wave + 4096);
  };
  copy_w(0);
  // query fragments: row 32*mt + lane%32 of the wave, d = 16*s + 8*(lane/32) .. +8
  bf16x8 af[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int arow = min(row0 + 32 * mt + (lane & 31), rows - 1);
    const uint16_t* p = a.q_nope + (static_cast<int64_t>(arow) * H + h) * kNope + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) af[mt][s] = *reinterpret_cast<const bf16x8*>(p + 16 * s);
  }
  const DSA_LDS uint8_t* wl = reinterpret_cast<const DSA_LDS uint8_t*>(lds_ptr(lds_addr_of(s_w)));
  DSA_LDS uint16_t* st = reinterpret_cast<DSA_LDS uint16_t*>(lds_ptr(lds_addr_of(&s_st[wave][0])));
  constexpr int kStores = 16;  // global stores of one pass per lane
  for (int pass = 0; pass < kVDim / kAbN; ++pass) {
    const int c0 = pass * kAbN;
    // this pass's weight copies (and, in the first pass, the query loads) have landed; the previous
    // pass's kStores stores, issued after them, may still be in flight (a workgroup with rows past
    // the last skips some stores, so it waits for everything)
    if (pass > 0 && full) wait_vmem_le<kStores>();
    else wait_vmem();
    __syncthreads();
    f32x16 acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};
    // one K step's four weight fragments at a time (the query fragments and accumulators already
    // hold 192 registers)
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 b[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt] = lds_read16(wl + 16 * ab_slot(32 * nt + (lane & 31), 2 * s + (lane >> 5)));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma32(af[mt][s], b[nt], acc[mt][nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // every wave has read this pass's weights
    if (c0 + kAbN < kVDim) copy_w(c0 + kAbN);

    // accumulator element e of tile (mt, nt): row 32*mt + 8*(e/4) + 4*(lane/32) + e%4 of the wave,
    // latent output c0 + 32*nt + lane%32
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rw = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) st[rw * kAbN + 32 * nt + (lane & 31)] = f32_to_bf16(acc[mt][nt][e]);
      }
      wave_lds_sync();
      // a wave-uniform base (row 32*mt of the wave, this pass's outputs) and 32-bit lane offsets
      uint8_t* const qb = reinterpret_cast<uint8_t*>(a.q + (static_cast<int64_t>(row0 + 32 * mt) * H + h) * a.out_stride + c0);
      const uint32_t rstride = static_cast<uint32_t>(H * a.out_stride * 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rw = 4 * i + (lane >> 4);  // 16 lanes per row, 16 bytes each
        const int row = row0 + 32 * mt + rw;
        const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(st + rw * kAbN + 8 * (lane & 15));
        if (row < rows) *reinterpret_cast<u32x4*>(qb + static_cast<uint32_t>(rw) * rstride + 16 * (lane & 15)) = v;
      }
      wave_lds_sync();  // the staged rows are read before the next M tile overwrites them
    }
  }
  if (a.q_pe != nullptr) {
    // q_pe: 64 rows x 8 granules of this wave
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = 64 * i + lane, rw = idx >> 3, g = idx & 7;
      const int row = row0 + rw;
      if (row < rows) {
        const int64_t rh = static_cast<int64_t>(row) * H + h;
        *reinterpret_cast<u32x4*>(a.q + rh * kLatent + kVDim + 8 * g) = *reinterpret_cast<const u32x4*>(a.q_pe + rh * kPe + 8 * g);
      }
    }
  }
}

hipError_t launch_q_absorb(const AbsorbArgs& a, hipStream_t st) {
  if (a.rows < 1 || a.H < 1) return hipErrorInvalidValue;
  const int64_t nb = (static_cast<int64_t>(a.rows) + kAbRows - 1) / kAbRows * a.H;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_q_absorb, dim3(static_cast<unsigned>(nb)), dim3(kAbWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

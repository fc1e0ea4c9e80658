// W_UK absorption: the latent query of sparse MLA from the per-head query without position (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, Implementation Limits, 2nd bullet:
// sparse MLA never expands the per-head keys; kimi_k3 API index, KimiK3TextConfig:
// qk_nope_head_dim 128, kv_lora_rank 512, qk_rope_head_dim 64, mla_use_nope). W_UK [H, 512, 128]
// is the key half of the kv_b_proj effective weight, so q_nope . (c_KV W_UK[h]) = q_lat . c_KV with
//   q[t,h,c]       = bf16( sum_d q_nope[t,h,d] * W_UK[h,c,d] )   c < 512, d < 128, FP32 accumulation
//   q[t,h,512 + j] = q_pe[t,h,j]                                 j < 64 (no rotation)
//
// Kernel design: a workgroup owns one quarter of the latent outputs (128), one head and 256 rows
// (four waves of 64 rows, two 32-row M tiles each). The quarter's 128 x 128 slice of W_UK[h] is
// staged in LDS once (one row c per 256 bytes, its 16-byte granules XOR-swizzled by c, so that 16
// lanes reading one granule of 16 consecutive rows hit distinct banks). A weight row holds the K
// values of one output contiguously, so no transposed copy is needed. Each lane's query fragments
// (K = d) stay in registers; v_mfma_f32_32x32x16_bf16 takes rows as M, c as N (four 32-wide tiles)
// and d as K (eight steps). Outputs leave through a per-wave LDS tile in 16-byte stores; the first
// quarter also copies q_pe into dims 512..575. HBM-bound: 1.5 KB per (row, head) against 131 K flop.
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
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int quarter = blockIdx.x, h = blockIdx.y;
  const int row0 = blockIdx.z * kAbRows + kAbRowsW * wave;
  const int H = a.H, rows = a.rows, c0 = quarter * kAbN;

  // the weight slice W_UK[h][c0 .. c0 + 128][0 .. 128]: 2,048 granules, eight wave copies each
  const uint16_t* __restrict__ W = a.W_UK + (static_cast<int64_t>(h) * kVDim + c0) * kNope;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int P0 = 512 * wave + 64 * j, P = P0 + lane;  // slot filled by this lane
    const int c = P >> 4, g = (P & 15) ^ (c & 15);
    copy16_to_lds(W + c * kNope + 8 * g, reinterpret_cast<DSA_LDS uint8_t*>(lds_ptr(lds_addr_of(s_w))) + 16 * P0);
  }
  // query fragments: row 32*mt + lane%32 of the wave, d = 16*s + 8*(lane/32) .. +8
  bf16x8 af[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int arow = min(row0 + 32 * mt + (lane & 31), rows - 1);
    const uint16_t* p = a.q_nope + (static_cast<int64_t>(arow) * H + h) * kNope + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) af[mt][s] = *reinterpret_cast<const bf16x8*>(p + 16 * s);
  }
  wait_vmem();
  __syncthreads();

  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};
  const DSA_LDS uint8_t* wl = reinterpret_cast<const DSA_LDS uint8_t*>(lds_ptr(lds_addr_of(s_w)));
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int c = 32 * nt + (lane & 31);
      const bf16x8 b = lds_read16(wl + 16 * ab_slot(c, 2 * s + (lane >> 5)));
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma32(af[mt][s], b, acc[mt][nt]);
    }
  }

  // accumulator element e of tile (mt, nt): row 32*mt + 8*(e/4) + 4*(lane/32) + e%4 of the wave,
  // latent output c0 + 32*nt + lane%32
  DSA_LDS uint16_t* st = reinterpret_cast<DSA_LDS uint16_t*>(lds_ptr(lds_addr_of(&s_st[wave][0])));
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rw = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) st[rw * kAbN + 32 * nt + (lane & 31)] = f32_to_bf16(acc[mt][nt][e]);
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rw = 4 * i + (lane >> 4);  // 16 lanes per row, 16 bytes each
      const int row = row0 + 32 * mt + rw;
      const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(st + rw * kAbN + 8 * (lane & 15));
      if (row < rows) *reinterpret_cast<u32x4*>(a.q + (static_cast<int64_t>(row) * H + h) * a.out_stride + c0 + 8 * (lane & 15)) = v;
    }
    wave_lds_sync();  // the staged rows are read before the next M tile overwrites them
  }
  if (quarter == 0 && a.q_pe != nullptr) {
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
  const int64_t zb = (static_cast<int64_t>(a.rows) + kAbRows - 1) / kAbRows;
  if (zb > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_q_absorb, dim3(kVDim / kAbN, a.H, static_cast<unsigned>(zb)), dim3(kAbWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

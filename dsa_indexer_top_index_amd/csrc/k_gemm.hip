// The step after the gate: o_proj, y = x W_o^T with bf16 operands and FP32 accumulation (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, paragraph on the output gate and
// kv_b_proj; kimi_k3 API index, KimiK3TextConfig: hidden_size 7168, 96 heads, v_head_dim 128):
//   y[t,n] = bf16( sum_k x[t,k] * W_o[n,k] )    x: the gated head outputs of a row [H * 128],
//                                               W_o [N, K] in the [out_features, in_features] layout
//
// Kernel design (both operands K-contiguous): a workgroup computes a 256 x 256 output tile with
// eight waves of 128 x 64 (four 32-row M tiles x two 32-column N tiles, 128 FP32 accumulators per
// lane) on v_mfma_f32_32x32x16_bf16. K advances in steps of 64: the 256 x 64 tiles of x and W_o
// are staged in LDS by asynchronous 16-byte global->LDS copies (eight per wave and step, from a
// scalar base with 32-bit lane offsets), double buffered with one barrier per step, so the next
// step's copies run under this step's MFMAs. A tile row is 128 bytes; its 16-byte granules are
// XOR-swizzled by (row / 2) % 8, so that the 16 lanes of each operand read hit 16 distinct bank
// groups. Blocks are renumbered so that each XCD runs patches of four row bands by a few column
// bands at a time, whose operand bands its L2 shares. The epilogue stages bf16 outputs in the then
// idle LDS and stores 16 bytes per lane.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kGM = 256, kGN = 256, kGK = 64;
constexpr int kGWaves = 8;
constexpr int kGTileBytes = kGM * kGK * 2;  // 32 KB per operand tile

// Byte offset of granule g (8 values of K) of tile row r.
__device__ __forceinline__ uint32_t g_off(int r, int g) { return 128u * r + 16u * (g ^ ((r >> 1) & 7)); }

__global__ __launch_bounds__(kGWaves * kWave, 1) void k_gemm_nt(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_t[2][2][kGTileBytes];  // [buffer][x, W_o]: 128 KB
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int nbn = a.N / kGN, nbm = (a.M + kGM - 1) / kGM;
  // Consecutive logical blocks run on one XCD; they walk groups of kGroupM row bands column by
  // column, so that the XCD's resident workgroups share a few x bands and a few W_o bands in L2
  // (a 4 x 8 patch of tiles reads 12 operand bands where a 1 x 28 row reads 29).
  constexpr int kGroupM = 4;
  const int lb = xcd_local_block(blockIdx.x, gridDim.x);
  const int grp = lb / (kGroupM * nbn), first_bm = grp * kGroupM;
  const int gsz = min(kGroupM, nbm - first_bm);
  const int in_grp = lb - grp * kGroupM * nbn;
  const int bm = first_bm + in_grp % gsz, bn = in_grp / gsz;
  const int m0 = bm * kGM, n0 = bn * kGN;
  const int wm = wave >> 2, wn = wave & 3;  // this wave: rows wm*128 .. +128, columns wn*64 .. +64
  const int K = a.K, nk = K / kGK;

  // Copy j of this wave (0..7) fills rows 8*part .. +8 of tile `tile` (0: x, 1: W_o), part =
  // (8*wave + j) % 32: lane i brings granule (i % 8) ^ ((row / 2) % 8) of row 8*part + i/8.
  // The copies of a wave read one operand (waves 0-3: x, 4-7: W_o) from a scalar base, the first row
  // of the workgroup's band, with 32-bit per-lane byte offsets (under 256 rows x K x 2 bytes).
  const int tile = wave >> 2;
  const uint16_t* sbase = tile == 0 ? a.A + static_cast<int64_t>(m0) * K : a.B + static_cast<int64_t>(n0) * K;
  uint32_t voff[8], dst[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int part = (8 * wave + j) & 31;
    const int row = 8 * part + (lane >> 3);
    const int g = (lane & 7) ^ ((row >> 1) & 7);
    const int brow = tile == 0 ? min(m0 + row, a.M - 1) - m0 : row;
    voff[j] = static_cast<uint32_t>(brow * K + 8 * g) * 2u;
    dst[j] = static_cast<uint32_t>(tile * kGTileBytes + 1024 * part);
  }
  const uint32_t lds0 = lds_addr_of(&s_t[0][0][0]);
  auto issue = [&](int kt) {
    const uint32_t b = lds0 + (kt & 1) * 2 * kGTileBytes;
    const uint16_t* sb = sbase + kt * kGK;
#pragma unroll
    for (int j = 0; j < 8; ++j) copy16_to_lds_imm<0>(sb, voff[j], __builtin_amdgcn_readfirstlane(b + dst[j]));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};

  issue(0);
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmem();    // this wave's copies of step kt have landed
    barrier_lds();  // everyone's have; every wave is done with the buffer of step kt - 1
    if (kt + 1 < nk) issue(kt + 1);
    const uint32_t ta = lds0 + (kt & 1) * 2 * kGTileBytes, tb = ta + kGTileBytes;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const int g = 2 * ks + (lane >> 5);
      bf16x8 af[4], bf[2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) af[mt] = lds_read16(lds_ptr(ta + g_off(wm * 128 + 32 * mt + (lane & 31), g)));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bf[nt] = lds_read16(lds_ptr(tb + g_off(wn * 64 + 32 * nt + (lane & 31), g)));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma32(af[mt], bf[nt], acc[mt][nt]);
    }
  }
  __syncthreads();  // every wave is past its last operand read: the LDS is free for staging

  // Accumulator element e of tile (mt, nt): row 32*mt + 8*(e/4) + 4*(lane/32) + e%4 of the wave's
  // 128, column 32*nt + lane%32 of its 64. Staged as bf16 [128][64], then 16 bytes per lane.
  DSA_LDS uint16_t* st = reinterpret_cast<DSA_LDS uint16_t*>(lds_ptr(lds0 + wave * (128 * 64 * 2)));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 32 * mt + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) st[r * 64 + 32 * nt + (lane & 31)] = f32_to_bf16(acc[mt][nt][e]);
    }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * i + (lane >> 3), g = lane & 7;
    const int row = m0 + wm * 128 + r;
    const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(st + r * 64 + 8 * g);
    if (row < a.M) *reinterpret_cast<u32x4*>(a.C + static_cast<int64_t>(row) * a.N + n0 + wn * 64 + 8 * g) = v;
  }
}

hipError_t launch_gemm_nt(const GemmArgs& a, hipStream_t st) {
  if (a.M < 1 || a.N < kGN || a.N % kGN != 0 || a.K < kGK || a.K % kGK != 0) return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>((a.M + kGM - 1) / kGM) * (a.N / kGN);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm_nt, dim3(static_cast<unsigned>(blocks)), dim3(kGWaves * kWave), 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

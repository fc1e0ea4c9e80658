// Per-head V up-projection and sigmoid output gate (gfx950).
//
// Method (NeMo AutoModel "Kimi-K3.1-Pro" model-coverage page, paragraph on the output gate and
// kv_b_proj: the gate is kept and the V projection is applied through its effective weight;
// archdiff "Kimi K3.1 Pro" blueprint, output gate sigma(x W_g) * o; kimi_k3 API index,
// v_head_dim 128):
//   o[t,h,d]   = sum_c o_lat[t,h,c] * W_UV[h,c,d]      (c < 512, d < 128)
//   out[t,h,d] = bf16( o[t,h,d] / (1 + exp(-gate[t,h])) )
// or, with the elementwise gate of the blueprint's "Output gate + sink" entry (gate_per_dim),
//   out[t,h,d] = bf16( o[t,h,d] / (1 + exp(-gate[t,h,d])) ).
//
// Kernel design: a workgroup owns one head and 256 query rows (four waves of 64 rows, two 32-row
// M tiles each), so the head's 128 KB weight is read once per 256 rows. The batched product runs
// on v_mfma_f32_32x32x16_bf16 with rows as M, the 128 outputs as N (four tiles) and c as K.
// W_UV[h] streams through LDS in 64-row chunks (asynchronous 16-byte copies, double buffered)
// and is read transposed with ds_read_b64_tr_b16, so no transposed copy of the weight exists;
// each weight fragment read from LDS serves both M tiles. The kernel is bound by the number of
// vector-memory instructions a CU can issue (about one 64-lane load or store per 64 cycles), so
// every access is 16 bytes per lane except the gate: one 2-byte load per wave (lane l: the gate of
// the wave's row l), spread to the lanes that need it by lane shuffles. The gate is applied in
// FP32 in the epilogue, which stages each wave's 32 x 128 outputs of one M tile at a time in the
// then idle weight buffer so that every row leaves in 16-byte stores. An elementwise gate tile is
// copied into that staging area first (16-byte copies) and overwritten in place by the gated outputs.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kUpRowsW = 64;                     // rows per wave: two 32-row M tiles
constexpr int kUpWaves = 4;
constexpr int kUpRows = kUpRowsW * kUpWaves;     // rows per workgroup
constexpr int kUpChunk = 64;                     // c rows of W_UV per LDS chunk
constexpr int kUpChunkBytes = kUpChunk * kODim * 2;  // 16 KB
constexpr int kUpWavesPerSimd = 2;               // waves per SIMD the register use must allow

// Chunk layout: granule g (16 B, 8 outputs) of weight row c lives at slot 16*c + (g ^ 4*(c%4)).
__device__ __forceinline__ int up_slot(int c, int g) { return 16 * c + (g ^ (4 * (c & 3))); }

__global__ __launch_bounds__(kUpWaves * kWave, kUpWavesPerSimd) void k_up_gate(UpArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][kUpChunkBytes];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kUpRows + kUpRowsW * wave;  // first chunk-local row of this wave
  const int H = a.H;
  const uint16_t* __restrict__ W = a.W_UV + static_cast<int64_t>(h) * kVDim * kODim;

  auto issue_chunk = [&](int cc, int buf) {
    DSA_LDS uint8_t* dst = (DSA_LDS uint8_t*)(&s_w[buf][0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int P0 = 256 * wave + 64 * j;
      const int P = P0 + lane;
      const int c = P >> 4;
      const int g = (P & 15) ^ (4 * (c & 3));
      copy16_to_lds(W + static_cast<int64_t>(kUpChunk * cc + c) * kODim + 8 * g, dst + 16 * P0);
    }
  };

  // A operand of M tile mt: row 32*mt + lane%32 of the wave, c = 16*step + 8*(lane/32) .. +8
  const uint16_t* arow_p[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int arow = min(row0 + 32 * mt + (lane & 31), a.chunk_rows - 1);
    arow_p[mt] = a.o_lat + (static_cast<int64_t>(arow) * H + h) * kVDim + 8 * (lane >> 5);
  }
  // B operand (transposed reads): rows c0 + 8*hh + s4 (+4), outputs 32*nt + 16*chh + 4*q4
  const int g16 = lane >> 4, i16 = lane & 15, hh = lane >> 5, chh = g16 & 1, s4 = i16 >> 2, q4 = i16 & 3;

  f32x16 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x16{};

  issue_chunk(0, 0);
  bf16x8 af[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) af[mt][s] = *reinterpret_cast<const bf16x8*>(arow_p[mt] + 16 * s);
  // the gate of the wave's row `lane`, as the sigmoid in FP32 (per-head gates only)
  const float gate_v = a.gate_per_dim ? 0.0f : bf16_to_f32(a.gate[(static_cast<int64_t>(a.chunk_r0) + min(row0 + lane, a.chunk_rows - 1)) * H + h]);
  wait_vmem();
  // af is complete (see the end of the chunk loop)
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(af[mt][s]));
  __syncthreads();
  const float sig_row = 1.0f / (1.0f + __expf(-gate_v));
  constexpr int nchunks = kVDim / kUpChunk;
  for (int cc = 0; cc < nchunks; ++cc) {
    const int buf = cc & 1;
    bf16x8 an[2][4];
    if (cc + 1 < nchunks) {
      issue_chunk(cc + 1, buf ^ 1);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) an[mt][s] = *reinterpret_cast<const bf16x8*>(arow_p[mt] + kUpChunk * (cc + 1) + 16 * s);
    }
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads go out before this chunk's products
    const DSA_LDS uint8_t* wb = (const DSA_LDS uint8_t*)(&s_w[buf][0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c1 = 16 * s + 8 * hh + s4, c2 = c1 + 4;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int g = 4 * nt + 2 * chh + (q4 >> 1);
        const u32x2 v1 = lds_read_tr16(wb + up_slot(c1, g) * 16 + 8 * (q4 & 1));
        const u32x2 v2 = lds_read_tr16(wb + up_slot(c2, g) * 16 + 8 * (q4 & 1));
        const u32x4 vb = {v1[0], v1[1], v2[0], v2[1]};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt][nt] = mfma32(af[mt][s], __builtin_bit_cast(bf16x8, vb), acc[mt][nt]);
      }
    }
    if (cc + 1 < nchunks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) af[mt][s] = an[mt][s];
    }
    wait_vmem();
    // The compiler does not count the weight copies (inline assembly) among the loads in flight, so
    // it would otherwise wait for them before the next chunk's first products to be sure of af;
    // passing af through an empty asm statement here, after the wait, makes af complete for it.
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(af[mt][s]));
    __syncthreads();
  }

  // Epilogue, one M tile at a time: accumulator element e of tile (mt, nt) is row
  // 32*mt + 8*(e/4) + 4*hh + e%4 of the wave's 64, output column 32*nt + lane%32. The gated bf16
  // values go to this wave's 8 KB of the weight buffer as [32 rows][128 outputs] (every wave is
  // past the last read of it), then each row's 256 bytes leave as sixteen 16-byte stores.
  static_assert(kUpWaves * 32 * kODim * 2 <= 2 * kUpChunkBytes, "staging fits the weight buffer");
  DSA_LDS uint16_t* st = reinterpret_cast<DSA_LDS uint16_t*>(lds_ptr(lds_addr_of(&s_w[0][0]))) + wave * 32 * kODim;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    if (a.gate_per_dim) {
      // The tile's gate logits [32 rows][128] land in the staging area first (16-byte copies, four
      // rows per copy); each element is then replaced in place by its gated output.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = min(row0 + 32 * mt + 4 * j + (lane >> 4), a.chunk_rows - 1);
        copy16_to_lds(a.gate + ((static_cast<int64_t>(a.chunk_r0) + row) * H + h) * kODim + 8 * (lane & 15),
                      st + 4 * j * kODim);
      }
      wait_vmem();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rw = 8 * (e >> 2) + 4 * hh + (e & 3);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int at = rw * kODim + 32 * nt + (lane & 31);
          const float sig = 1.0f / (1.0f + __expf(-bf16_to_f32(st[at])));
          st[at] = f32_to_bf16(acc[mt][nt][e] * sig);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rw = 8 * (e >> 2) + 4 * hh + (e & 3);
        const float sig = __shfl(sig_row, 32 * mt + rw);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) st[rw * kODim + 32 * nt + (lane & 31)] = f32_to_bf16(acc[mt][nt][e] * sig);
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rw = 4 * i + (lane >> 4);  // 16 lanes per row, 16 bytes each
      const int row = row0 + 32 * mt + rw;
      const u32x4 v = *reinterpret_cast<const DSA_LDS u32x4*>(st + rw * kODim + 8 * (lane & 15));
      if (row < a.chunk_rows)
        *reinterpret_cast<u32x4*>(a.out + ((static_cast<int64_t>(a.chunk_r0) + row) * H + h) * kODim + 8 * (lane & 15)) = v;
    }
    wave_lds_sync();  // the staged rows are read before the next M tile overwrites them
  }
}

hipError_t launch_up_gate(const UpArgs& a, hipStream_t st) {
  dim3 grid((a.chunk_rows + kUpRows - 1) / kUpRows, a.H), block(kUpWaves * kWave);
  hipLaunchKernelGGL(k_up_gate, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace dsa

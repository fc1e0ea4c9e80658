// Device-side helpers shared by the gfx950 kernels of libdsa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

#define DSA_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;
constexpr int kLatent = 576;  // kv_lora_rank 512 + 64 unrotated dims
constexpr int kVDim = 512;    // V part of a latent row
constexpr int kODim = 128;    // v_head_dim

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the hardware exponential unit (no range reduction; results below the normal range flush to 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// double -> bf16 bits in one rounding step (nearest, ties to even), for |x| in the normal float range or 0.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint64_t drop = 45;  // 52 - 7 mantissa bits
  u += ((1ull << (drop - 1)) - 1) + ((u >> drop) & 1ull);
  u &= ~((1ull << drop) - 1);
  float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));  // exact
  return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// Total order on FP32 scores as unsigned keys: larger score -> larger key; -0.0 and +0.0 equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Orders this wave's LDS accesses: later LDS reads see earlier LDS writes of any lane of the wave.
__device__ __forceinline__ void wave_lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void wait_vmem() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte asynchronous copy global -> LDS. Lane i of the wave writes lds_wave_base + 16*i.
// Issued as inline assembly on purpose: the compiler then does not treat the copy as an LDS write
// and does not drain every outstanding copy before the next LDS read of another buffer. Callers
// order the copies themselves with wait_vmem_le<N>() and a barrier.
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, DSA_LDS void* lds_wave_base) {
  // the LDS base is wave-uniform by contract; readfirstlane puts it in an SGPR for M0
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_wave_base)));
  // one wait state between the M0 write and the LDS DMA that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_addr) : "memory", "m0");
}

// The same copy with a scalar base address: lane i reads sbase + voff + OFF and writes
// lds + OFF + 16*i. The immediate offset moves both addresses; lds must be wave-uniform.
template <int OFF>
__device__ __forceinline__ void copy16_to_lds_imm(const void* sbase, uint32_t voff, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(voff), "s"(sbase), "s"(lds),
               "n"(OFF)
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are outstanding (they complete in order).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release/acquire fences of __syncthreads(): it does not wait for
// this wave's outstanding global->LDS copies. LDS reads and writes issued before it are complete.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS byte address of a __shared__ object, and the LDS pointer of a byte address. Working on 32-bit
// offsets lets the compiler fold constant displacements into the ds_read immediate offset.
__device__ __forceinline__ uint32_t lds_addr_of(const void* shared_obj) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const DSA_LDS void*)shared_obj));
}
__device__ __forceinline__ DSA_LDS uint8_t* lds_ptr(uint32_t addr) {
  return reinterpret_cast<DSA_LDS uint8_t*>(static_cast<uintptr_t>(addr));
}

__device__ __forceinline__ bf16x8 lds_read16(const DSA_LDS void* p) {
  return *reinterpret_cast<const DSA_LDS bf16x8*>(p);
}

// Transposed 4x16 read of b16 data (gfx950): in each 16-lane group, lane 4s+q supplies the 4
// elements [4q, 4q+4) of row s; lane i receives column i of that 4x16 block (rows 0..3).
__device__ __forceinline__ u32x2 lds_read_tr16(const DSA_LDS void* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<DSA_LDS s16x4*>(const_cast<DSA_LDS void*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

// O += A * B on v_mfma_f32_32x32x16_bf16 with the accumulator pinned to AGPRs. Issued as inline
// assembly so that a kernel whose other MFMAs use the VGPR form keeps a large accumulator set in
// AGPRs. The compiler cannot see this instruction's hazards, so callers must (1) leave at least 4
// wait states between a VALU write of a or b and this instruction, and (2) leave 40 wait states
// after the last of these instructions before any VALU access to acc (mfma_agpr_drain()).
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr_settle() { asm volatile("s_nop 4" ::: "memory"); }
__device__ __forceinline__ void mfma_agpr_drain() { asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// O += A * B on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0) and unit block
// scales (E8M0 127 = 2^0): 32 one-byte K values per lane, the same K order in A and B.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// First token of the document that holds token t; cu == nullptr means a single document.
__device__ __forceinline__ int doc_begin(const int32_t* __restrict__ cu, int n_docs, int t) {
  if (cu == nullptr) return 0;
  int lo = 0, hi = n_docs;  // find d with cu[d] <= t < cu[d+1]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return cu[lo];
}

// Block id remapped so that consecutive logical blocks run on the same XCD (blocks are dealt to
// the 8 XCDs round-robin by hardware id).
__device__ __forceinline__ int xcd_local_block(int b, int nblocks) {
  const int nx = 8;
  int q = nblocks / nx, r = nblocks % nx;
  int x = b % nx, p = b / nx;
  return x * q + (x < r ? x : r) + p;
}

}  // namespace dsa

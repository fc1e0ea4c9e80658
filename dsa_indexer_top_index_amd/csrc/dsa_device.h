// Device-side helpers shared by the gfx950 kernels of libdsa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

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

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

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
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, DSA_LDS void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 16, 0, 0);
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

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

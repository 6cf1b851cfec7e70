// Device helpers shared by the gfx950 kernels: MFMA wrappers, bf16 packing, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace focus {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds row (A) / column (B) l%16 and the 8 consecutive k-slots 8*(l/16)..+7; the result
// lane l holds column l%16, rows 4*(l/16)+0..3.
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(16x16, f32) += A(16x4, f32) * B(4x16, f32); lane l holds row/column l%16, k-slot l/16.
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 (lo in bits 0..15), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ u32x4_t load16v(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// s_waitcnt immediate with vmcnt = 0 and the other counters at their maxima (GFX9 encoding):
// waits until every vector memory access of the wave, stores included, has completed
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt immediate with lgkmcnt = 0 and the other counters at their maxima: waits until the
// wave's LDS (and scalar memory) accesses have completed, not for its vector memory accesses
constexpr int kWaitLgkmcnt0 = 0xC07F;

// Global-memory views of device pointers: loads through them are global (never flat)
// instructions, which the compiler's wait counting can order with the other vector loads
// (a pending flat load makes every later wait a full drain).
typedef const __attribute__((address_space(1))) u32x2_t global_u32x2_t;
typedef const __attribute__((address_space(1))) u32x4_t global_u32x4_t;

// 8-byte load of data read exactly once (non-temporal: the caches do not keep it)
__device__ __forceinline__ u32x2_t load8_stream(const void* p) {
  return __builtin_nontemporal_load((global_u32x2_t*)p);
}


// 16-byte load of data read exactly once (non-temporal: the caches do not keep it)
__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load((global_u32x4_t*)p);
}

}  // namespace focus

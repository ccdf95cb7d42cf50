// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }
// silu(z) = z / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32; about 1 ulp each): for activations that
// are rounded to bf16 right after, well below the output's rounding.
// e^-z overflows to +inf for very negative z, and the reciprocal gives 0.
__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(z * -1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Pins a loaded value where it stands: the compiler may otherwise sink a
// load whose result is used under a condition into that branch and wait on
// it there alone. Loads issued back to back and then pinned stay in flight
// together (the waits come in issue order at the pins).
template <typename V>
__device__ __forceinline__ void pin(V& v) { asm volatile("" : "+v"(v)); }
// The same for a wave-uniform value held in a scalar register.
__device__ __forceinline__ void pin_s(int& v) { asm volatile("" : "+s"(v)); }

// Uniform loads of tables through the constant address space, so they are
// scalar loads and never enter the vector-memory counter.
template <class T>
__device__ __forceinline__ T ldc(const T* q, int i) {
  return ((const __attribute__((address_space(4))) T*)q)[i];
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

// ---------------------------------------------------------------------------
// Direct global->LDS staging pipelines (shared by the GEMMs and the router)
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] in bits 3:0,
// vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8): at most N vector
// loads (the newer stages' DMA) still in flight, and every LDS access of this
// wave complete, so that after the barrier no wave still reads a buffer the
// next DMA overwrites.
template <int N>
__device__ __forceinline__ void wait_stage() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier for the stage pipeline. __builtin_amdgcn_s_barrier has
// no memory semantics for the compiler, which may then hoist the next
// stage's LDS fragment reads (or the next DMA issue) above it; the empty asm
// statements with a memory clobber pin every memory access to its side of
// the barrier without emitting the wait-for-all-loads that __syncthreads'
// fences would add.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS stage layout: rows of BK bf16 (BK / 8 chunks of 16 bytes), no padding.
// Logical chunk c of row r lives at a physical chunk chosen so that the 8
// lanes LDS serves per cycle (rows r..r+7 of one MFMA fragment, same logical
// chunk) hit 8 distinct 16-byte bank groups: c ^ (r & 7) for 128-byte rows,
// c ^ ((r >> 1) & 3) for 64-byte rows.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (BK == 64) return row * 64 + ((chunk ^ (row & 7)) << 3);
  else return row * 32 + ((chunk ^ ((row >> 1) & 3)) << 3);
}
template <int BK>
__device__ __forceinline__ int swz_phys_to_logical(int row, int phys) {
  if constexpr (BK == 64) return phys ^ (row & 7);
  else return phys ^ ((row >> 1) & 3);
}

}  // namespace moe

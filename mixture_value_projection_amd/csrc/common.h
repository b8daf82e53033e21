// Device-side helpers shared by the MoVA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mova {

constexpr int kWave = 64;
constexpr int kMaxExperts = 64;  // one wave lane per expert in the router
constexpr int kMaxTopK = 8;

typedef __bf16 bf16_t;
typedef _Float16 f16_t;  // slot partials: w * SiLU(z) rounded once (nearest even)
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// 16 B of memory viewed either as raw words (for copies) or as 8 bf16 (for MFMA).
union Frag16 {
  u32x4 u;
  bf16x8 h;
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// The same load with the non-temporal hint, for data read once per call (the
// decode kernels' expert weights): it keeps the stream from displacing what
// the caches hold for reuse.  Measured on the decode step at T = 64 (weights
// rotated over 4 copies): weight stream 60.4 -> 53.5 us.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Cache-policy operand of a direct-to-LDS load (global_load_lds) with the
// non-temporal bit set.
constexpr int kLdsLoadNonTemporal = 2;

__device__ __forceinline__ void store16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// D = A(16x32) * B(32x16) + C on bf16 inputs with fp32 accumulation.  Lane l
// supplies A row (l % 16) and B column (l % 16), 8 consecutive k values each;
// lanes in group q = l / 16 cover k = 8q .. 8q + 7.  C/D: lane l holds rows
// 4q .. 4q + 3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sigmoidf_fast(float z) {
  return 1.0f / (1.0f + __expf(-z));
}

__device__ __forceinline__ float siluf(float z) { return z * sigmoidf_fast(z); }

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---- direct-to-LDS staging (global_load_lds rings) --------------------------

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate: at most n vector-memory operations of this wave still
// outstanding, and all of its LDS operations complete.
constexpr int vmcnt_lgkm0_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// waits for every outstanding direct-to-LDS load, which would drain a
// multi-stage ring.  The caller waits on the counters it needs first; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace mova

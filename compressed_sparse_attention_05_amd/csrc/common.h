// Shared device helpers of the CSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"

namespace csa {

// ------------------------------------------------------------------ vector types for MFMA

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ bf16 <-> f32

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats to bf16 (round to nearest even, as f2bf) in one v_cvt_pk_bf16_f32; a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<CSA_F32>(const void* p, int64_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_elem<CSA_BF16>(const void* p, int64_t i) {
  return bf2f(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v);
template <>
__device__ __forceinline__ void store_elem<CSA_F32>(void* p, int64_t i, float v) {
  static_cast<float*>(p)[i] = v;
}
template <>
__device__ __forceinline__ void store_elem<CSA_BF16>(void* p, int64_t i, float v) {
  static_cast<uint16_t*>(p)[i] = f2bf(v);
}

// max(v, 0) in one v_med3_f32 (fmaxf adds a NaN-quieting max in IEEE mode); inputs are finite.
__device__ __forceinline__ float relu(float v) { return __builtin_amdgcn_fmed3f(v, 0.f, 3.0e38f); }

// ------------------------------------------------------------------ wave helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Orders this wave's LDS traffic around the call (the wave executes in lockstep; the fence keeps
// the compiler from moving LDS accesses across it).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((uint32_t)v, src, 64);
  uint32_t hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w < v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// ------------------------------------------------------------------ direct global -> LDS loads

// Global -> LDS copy of 16 bytes per lane: lane p writes LDS bytes [lds + 16p, lds + 16p + 16).
// Issued as inline asm so that the compiler does not make later LDS reads wait for it; the
// caller waits on vmcnt before the barrier that publishes the tile. M0 (the LDS base of the
// load) is saved and restored around it.
__device__ __forceinline__ void copy_to_lds16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// The same copy from a wave-uniform base address plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void copy_to_lds16_sbase(const void* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// Four bytes per lane (global_load_lds_dword): LDS destination M0 + 4 * lane.
__device__ __forceinline__ void copy_to_lds4(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// The same copy from a wave-uniform base address plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void copy_to_lds4_sbase(const void* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 16]
__device__ __forceinline__ void wait_vmcnt_upto16(int n);

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left free (vmcnt bits 3:0 and 15:14 of the immediate)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_vmcnt_upto16(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    default: wait_vmcnt<16>(); break;
  }
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Position of sequence b from a device array of per-sequence positions; NULL means every sequence
// is at 0, and a negative value counts as 0.
__device__ __forceinline__ int64_t pos_at(const int64_t* pos, int64_t b) {
  if (!pos) return 0;
  const int64_t p = pos[b];
  return p > 0 ? p : 0;
}

// An offset position from a device array, taken as given (NULL: 0).
__device__ __forceinline__ int64_t raw_at(const int64_t* pos, int64_t b) { return pos ? pos[b] : 0; }

// n_vis(p) = min(floor((p+1)/m), n_cap): entries whose block is complete at position p.
__host__ __device__ __forceinline__ int64_t n_visible(int64_t p, int m, int64_t n_cap) {
  int64_t v = (p + 1) / m;
  if (v < 0) v = 0;
  return v < n_cap ? v : n_cap;
}

}  // namespace csa

// Device building blocks for the gfx950 attention kernels: MFMA fragments, LDS
// swizzles, wave-half exchanges, bf16 packing.  CDNA4 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------
// MFMA 32x32x16 bf16 -> fp32.  Fragment layout (checked on gfx950 with a probe):
//   A (32 x 16): lane l supplies row (l % 32), k-slots 8*(l/32) .. +7
//   B (16 x 32): lane l supplies column (l % 32), the same k-slots
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4), column l%32
// Only the pairing of A and B k-slots matters for the product, so any consistent
// assignment of the contraction index to (l/32, j) is valid.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even pack of two fp32 values into one dword of two bf16
// (lo = a, hi = b); lowers to v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo(w) + hi(w) for a dword of two bf16 (v_dot2c_f32_bf16 against (1, 1)): sums
// exactly the rounded values that feed the MFMA.
__device__ __forceinline__ float add_bf16x2(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// v_permlane32_swap: after the swap lane l < 32 holds (own x, x of lane l+32) and lane
// l >= 32 holds (x of lane l-32, own x), so both results together are the two halves.
__device__ __forceinline__ float half_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

// Byte-select helpers for the 4x4 bf16 register transpose (v_perm_b32).
__device__ __forceinline__ uint32_t lo16_pair(uint32_t a, uint32_t b) {  // (a.lo16, b.lo16)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) {  // (a.hi16, b.hi16)
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---------------------------------------------------------------------------------
// LDS access helpers (explicit LDS address space so the compiler emits ds_* ops).
// ---------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ u32x4 lds_read128(const unsigned char* base, uint32_t byte) {
  return *(const lds_u32x4*)((const __attribute__((address_space(3))) unsigned char*)base + byte);
}
__device__ __forceinline__ void lds_write64(unsigned char* base, uint32_t byte, u32x2 v) {
  *(lds_u32x2*)((__attribute__((address_space(3))) unsigned char*)base + byte) = v;
}
__device__ __forceinline__ void lds_write128(unsigned char* base, uint32_t byte, u32x4 v) {
  *(lds_u32x4*)((__attribute__((address_space(3))) unsigned char*)base + byte) = v;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// lds_wave_base + 16*l (M0-relative; checked on gfx950 with a probe).
__device__ __forceinline__ void g2lds16(const void* gptr, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void*)gptr,
                                   (__attribute__((address_space(3))) void*)(
                                       (__attribute__((address_space(3))) unsigned char*)lds_wave_base),
                                   16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace fa355

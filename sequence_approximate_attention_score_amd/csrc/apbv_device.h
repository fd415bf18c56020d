// Device-side helpers shared by the gfx950 kernels: vector types, bf16 packing and the
// 32x32x16 bf16 MFMA fragment conventions.
//
// MFMA v_mfma_f32_32x32x16_bf16 (CDNA4): D[32x32] += A[32x16] * B[16x32].
//   A: lane l holds row (l % 32), 8 consecutive k values starting at 8 * (l / 32).
//   B: lane l holds column (l % 32), the same 8 k values.
//   D: lane l holds column (l % 32) and 16 rows: register r -> row 8*(r/4) + 4*(l/32) + r%4.
// The k <-> (lane half, element) mapping is used identically for A and B, so any
// consistent assignment of reduction indices to (half, element) slots is valid.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apbv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 p = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value held by the lane 32 positions away (lane l ^ 32). v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; with both operands x,
// each lane ends up with its own value in one result and its partner's in the other, so
// the XOR of the two results and x is the partner's value (bit-exact, also for -inf/NaN).
__device__ __forceinline__ float swap_half(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0] ^ r[1] ^ u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup index remapped so that each XCD (workgroups are dispatched round-robin over
// the 8 XCDs) receives one contiguous range of logical indices.
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t wg, uint32_t total) {
  const uint32_t nx = 8;
  const uint32_t q = total / nx, r = total % nx;
  const uint32_t x = wg % nx, s = wg / nx;
  return x * q + (x < r ? x : r) + s;
}

}  // namespace apbv

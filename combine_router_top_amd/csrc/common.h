// Shared device helpers for the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Host-side view of moe_problem_t with derived sizes.
struct Prob {
  int T, d, E, k, f, lo, n;  // n = n_local
  int dtype;                 // 0 = f32, 1 = bf16
  uint32_t flags;
  int64_t rows_max;          // T * min(k, n); n * capacity for the padded layout
  int64_t seg_rows = 0;      // rows of every local segment when fixed (padded layout), else 0
  int64_t tk() const { return (int64_t)T * k; }
  int elem() const { return dtype == 1 ? 2 : 4; }
};

typedef uint16_t bf16_t;  // bf16 bit pattern in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN is outside the library's contract.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// SiLU(a) * b = a / (1 + e^-a) * b for the bf16 GEMM epilogues, with the
// hardware's base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32: each
// within about one fp32 ulp, e^-a as 2^(-a log2 e)); the result is rounded to
// bf16 right after, 2^16 times coarser.  For a -> -inf the exponential
// overflows to inf and the reciprocal gives 0; for a -> +inf it underflows to
// 0 and the product is a.  About 6 instructions against about 25 for the
// correctly rounded exp and division, which a 160-row tile repeats for 80
// values per lane in its epilogue while nothing else is in flight.
__device__ __forceinline__ float silu_mul(float a, float b) {
  const float e = __builtin_amdgcn_exp2f(a * -1.4426950408889634f);
  return a * __builtin_amdgcn_rcpf(1.0f + e) * b;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key);
// -0.0 is first folded to +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t f32_order_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Exclusive/inclusive wave-wide helpers on 64-lane wavefronts.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = __lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe

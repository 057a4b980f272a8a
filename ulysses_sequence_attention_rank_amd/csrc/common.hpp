// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uly {

typedef unsigned int u32;
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

// Division by a run-time invariant divisor via a multiply-high and a shift
// (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994): for 1 <= d < 2^31 and n < 2^31,
// n / d == (umulhi(n, magic) + n) >> shift.
struct FastDiv {
  u32 d, magic, shift;
};

inline FastDiv make_fastdiv(u32 d) {
  FastDiv f;
  f.d = d;
  u32 s = 0;
  while ((1ull << s) < d) ++s;  // s = ceil(log2 d)
  f.shift = s;
  f.magic = (u32)((((1ull << s) - d) << 32) / d + 1);
  if (d == 1) f.magic = 0;
  return f;
}

__device__ __forceinline__ u32 fdiv(u32 n, const FastDiv& f) {
  return (__umulhi(n, f.magic) + n) >> f.shift;
}

// bf16 round-to-nearest-even from fp32, two at a time (v_cvt_pk_bf16_f32).
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(u32, p);
}

// Saturate to the finite fp16 range before an fp16 conversion.
__device__ __forceinline__ float clamp_f16(float x) { return fminf(fmaxf(x, -65504.f), 65504.f); }

__device__ __forceinline__ float bf16_lo(u32 w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(u32 w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace uly

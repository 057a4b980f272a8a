// A measurement aid, not part of the computation: what the matrix cores
// sustain with nothing else to do, and what feeding them through LDS costs.
// Every wave keeps eight independent 32x32x16 bf16 accumulators.  Its
// operands are pseudo-random and change from product to product (constant
// operands draw less power and let the clock run higher than real tensors
// do).  Modes:
//   0  operands from registers (eight pairs per lane, cycled);
//   1  as 0, with 8 independent fp32 FMAs after each product;
//   2  the B operand of each product read from LDS (1 KiB per product);
//   3  both operands read from LDS (2 KiB per product);
//   4  as 0, with 8 independent exp2 (each with two adds) after each product;
//   5  as 4 with a multiply in place of each exp2 (what the exp2 costs
//      beyond an ordinary vector operation).
// The sums land in `out` (one value per thread) so that nothing is
// optimised away.
#include "launch.hpp"

namespace uly {

namespace {

typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));
typedef unsigned cu32x4 __attribute__((ext_vector_type(4)));

struct XorShift {
  unsigned x;
  __device__ unsigned next() {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  }
  __device__ __bf16 bf16() { return (__bf16)((float)(int)(next() & 0xffffu) * (1.f / 32768.f) - 1.f); }
};

template <int MODE>
__global__ __launch_bounds__(256, 2) void calib_mfma_kernel(float* out, int iters) {
  XorShift rng{2463534242u ^ ((unsigned)(blockIdx.x * 256 + threadIdx.x) * 2654435761u)};
  cbf16x8 av[8], bv[8];
  for (int k = 0; k < 8; ++k)
    for (int i = 0; i < 8; ++i) {
      av[k][i] = rng.bf16();
      bv[k][i] = rng.bf16();
    }
  __shared__ __attribute__((aligned(16))) cu32x4 lds[MODE >= 2 ? 2048 : 1];  // 32 KiB of bf16 in [1, 2)
  if constexpr (MODE >= 2) {
    for (int i = threadIdx.x; i < 2048; i += 256) {
      cu32x4 v;
      for (int c = 0; c < 4; ++c) v[c] = (rng.next() & 0x3fff3fffu) | 0x3c003c00u;
      lds[i] = v;
    }
    __syncthreads();
  }
  cf32x16 acc[8];
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  float v0 = threadIdx.x * 1e-7f, v1 = v0 + 1e-7f, v2 = v1 + 1e-7f, v3 = v2 + 1e-7f;
  float xs[8], ss[8];
  for (int j = 0; j < 8; ++j) {
    xs[j] = -1.f + 0.1f * j + 1e-6f * threadIdx.x;
    ss[j] = 0.f;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (MODE <= 1 || MODE >= 4) {
    for (int it = 0; it < iters; it += 8)
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], bv[(k + u) & 7], acc[k], 0, 0, 0);
          if constexpr (MODE >= 4) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              xs[j] += 1e-7f;
              ss[j] += MODE == 4 ? __builtin_amdgcn_exp2f(xs[j]) : xs[j] * 1.0001f;
            }
          }
          if constexpr (MODE == 1) {
            v0 = __builtin_fmaf(v0, 0.999f, 1e-9f);
            v1 = __builtin_fmaf(v1, 0.999f, 1e-9f);
            v2 = __builtin_fmaf(v2, 0.999f, 1e-9f);
            v3 = __builtin_fmaf(v3, 0.999f, 1e-9f);
            v0 = __builtin_fmaf(v0, 0.999f, 1e-9f);
            v1 = __builtin_fmaf(v1, 0.999f, 1e-9f);
            v2 = __builtin_fmaf(v2, 0.999f, 1e-9f);
            v3 = __builtin_fmaf(v3, 0.999f, 1e-9f);
          }
        }
  } else {
    // each product reads 16 bytes a lane at a slot that moves with the
    // iteration (a wave's 64 lanes read 1 KiB of consecutive slots)
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int slot = ((it * 8 + k) * 64 + lane + wave * 512) & 2047;
        const cbf16x8 b = __builtin_bit_cast(cbf16x8, lds[slot]);
        const cbf16x8 a = MODE == 3 ? __builtin_bit_cast(cbf16x8, lds[(slot + 1024) & 2047]) : av[k];
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
      }
  }
  float s = v0 + v1 + v2 + v3;
  for (int j = 0; j < 8; ++j) s += ss[j];
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t calib_mfma_launch(float* out, int iters, int mode, hipStream_t st) {
  ProfScope prof("calib_mfma", st);
  const dim3 grid(kCalibBlocks), block(256);
  switch (mode) {
    case 0: hipLaunchKernelGGL((calib_mfma_kernel<0>), grid, block, 0, st, out, iters); break;
    case 1: hipLaunchKernelGGL((calib_mfma_kernel<1>), grid, block, 0, st, out, iters); break;
    case 2: hipLaunchKernelGGL((calib_mfma_kernel<2>), grid, block, 0, st, out, iters); break;
    case 3: hipLaunchKernelGGL((calib_mfma_kernel<3>), grid, block, 0, st, out, iters); break;
    case 4: hipLaunchKernelGGL((calib_mfma_kernel<4>), grid, block, 0, st, out, iters); break;
    default: hipLaunchKernelGGL((calib_mfma_kernel<5>), grid, block, 0, st, out, iters); break;
  }
  return hipGetLastError();
}

}  // namespace uly

// A measurement aid, not part of the computation: what the matrix cores
// sustain with nothing else to do.  Every wave keeps eight independent
// 32x32x16 bf16 accumulators and feeds them operands from registers (eight
// pseudo-random operand pairs per lane, cycled so that the products see
// changing data, as with real tensors: constant operands draw less power
// and let the clock run higher).  VALU_PER independent fp32 FMAs may
// follow each product, to see what vector work beside the products costs.
// The sums land in `out` (one value per lane) so that nothing is optimised
// away.
#include "launch.hpp"

namespace uly {

namespace {

typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x16 __attribute__((ext_vector_type(16)));

template <int VALU_PER>
__global__ __launch_bounds__(256, 2) void calib_mfma_kernel(float* out, int iters) {
  cbf16x8 av[8], bv[8];
  unsigned x = 2463534242u ^ ((unsigned)(blockIdx.x * 256 + threadIdx.x) * 2654435761u);
  auto next = [&x]() {  // xorshift32, mapped to [-1, 1)
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return (__bf16)((float)(int)(x & 0xffffu) * (1.f / 32768.f) - 1.f);
  };
  for (int k = 0; k < 8; ++k)
    for (int i = 0; i < 8; ++i) {
      av[k][i] = next();
      bv[k][i] = next();
    }
  cf32x16 acc[8];
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  float v0 = threadIdx.x * 1e-7f, v1 = v0 + 1e-7f, v2 = v1 + 1e-7f, v3 = v2 + 1e-7f;
  for (int it = 0; it < iters; it += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[k], bv[(k + u) & 7], acc[k], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < VALU_PER; j += 4) {
          v0 = __builtin_fmaf(v0, 0.999f, 1e-9f);
          v1 = __builtin_fmaf(v1, 0.999f, 1e-9f);
          v2 = __builtin_fmaf(v2, 0.999f, 1e-9f);
          v3 = __builtin_fmaf(v3, 0.999f, 1e-9f);
        }
      }
  float s = v0 + v1 + v2 + v3;
  for (int k = 0; k < 8; ++k)
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t calib_mfma_launch(float* out, int iters, int valu_per, hipStream_t st) {
  ProfScope prof("calib_mfma", st);
  const dim3 grid(kCalibBlocks), block(256);
  if (valu_per == 0) hipLaunchKernelGGL((calib_mfma_kernel<0>), grid, block, 0, st, out, iters);
  else if (valu_per == 4) hipLaunchKernelGGL((calib_mfma_kernel<4>), grid, block, 0, st, out, iters);
  else hipLaunchKernelGGL((calib_mfma_kernel<8>), grid, block, 0, st, out, iters);
  return hipGetLastError();
}

}  // namespace uly

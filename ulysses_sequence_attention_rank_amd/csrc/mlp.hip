// The sequence-tiled gated MLP of one rank (the TiledMLP feature of the
// DeepSpeed pull request that ports Ulysses to HF models): y = (silu(x Wg^T)
// * (x Wu^T)) Wd^T over the rank's tokens in tiles, the backward recomputing
// each tile's activations and adding its weight gradients to fp32 sums.
//
// Every product is one MFMA GEMM kernel, C[m][n] = sum_k A(m,k) B(n,k), with
// each operand stored either k-contiguous ("natural": A [M][lda], B [N][ldb])
// or k-major ("transposed": A [K][lda] holding A(m,k) at k*lda + m, B
// likewise).  Block tile 128 (m) x 128 (n) x 64 (k), four waves of 64 x 64.
// Operand tiles arrive by buffer-resource direct-to-LDS loads into the
// swizzled LDS tiles of the attention kernels (rows past the matrix end read
// as zero, so the token dimension may be ragged) and are read back in the two
// forms those tiles serve: natural 16-byte reads, or transposing reads for
// k-major storage.  The transposing reads deliver k in the slot order of
// attn_common.hpp (4 hf + e, then 8 + 4 hf + e); a natural operand paired
// with a transposed one is read in that same order (two 8-byte reads), so
// both operands of every product contract the same k.  The kernel computes
// C^T tiles (the B operand as the MFMA's A), which leaves each lane four
// consecutive n of one row m: one 8- or 16-byte store per four outputs.
#include "attn_common.hpp"
#include "launch.hpp"

namespace uly {

namespace mlp {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int TILE = BM * BK * 2;  // bytes of an A or B stage (both 128 x 64)

enum Epi {
  kStoreBf16 = 0,  // C bf16 [M][ldc]
  kSwiglu = 1,     // dual B (gate rows, up rows): C = silu(G) * U, bf16
  kStoreGU = 2,    // dual B: C = G, C1 = U, bf16
  kGatedGrad = 3,  // C = dH, with G, U read back: C = h = silu(G) U, C1 [M][2 ldc]: dG | dU, bf16
  kAccF32 = 4,     // C fp32 [M][ldc] += acc; rows m >= msplit go to c_hi (row m - msplit)
};

struct GemmArgs {
  const __bf16* a;
  const __bf16* b0;
  const __bf16* b1;  // dual: up-projection rows; transposed B: rows k >= ksplit
  int64_t lda, ldb;
  int M, N, K, ksplit;
  void* c;
  void* c1;
  float* c_hi;
  int64_t ldc;
  int msplit;
  const __bf16* g_in;  // kGatedGrad: G and U, [M][ldc] bf16
  const __bf16* u_in;
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }

// Natural operand read in the transposing reads' k order: lane l of half hf
// gets row r0 + l%32, k = 16 s + 4 hf .. +3 and 16 s + 8 + 4 hf .. +3.
template <int D>
__device__ __forceinline__ bf16x8 nat_perm(const char* lds, int r0, int s, int lane) {
  const int r = r0 + (lane & 31), hf = lane >> 5;
  typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
  const u32x2v lo = *reinterpret_cast<const u32x2v*>(lds + Swz<D>::off(r, 2 * s) + 8 * hf);
  const u32x2v hi = *reinterpret_cast<const u32x2v*>(lds + Swz<D>::off(r, 2 * s + 1) + 8 * hf);
  u32x4 x = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, x);
}

// Operand fragment of rows/columns [r0, r0 + 32) and k-step s of a stage:
// natural stages are 128 rows x 64 k (Swz<64>), transposed stages 64 k rows x
// 128 columns (Swz<128>).
template <bool T, bool PERM>
__device__ __forceinline__ bf16x8 frag(const char* st, int r0, int s, int lane) {
  if constexpr (T) return swz_tr<128>(st, 16 * s, r0, lane);
  else if constexpr (PERM) return nat_perm<64>(st, r0, s, lane);
  else return swz_nat<64>(st, r0, s, lane);
}

}  // namespace mlp

// The A and B stages of k tile KT into (SA, SB).
#define MLP_LOAD_STAGE(SA, SB, KT)                                                                   \
  do {                                                                                               \
    const int k0_ = (KT) * BK;                                                                       \
    if constexpr (TA) la.load((SA), g.a + (int64_t)k0_ * g.lda + m0, g.K - k0_, wave);             \
    else la.load((SA), g.a + (int64_t)m0 * g.lda + k0_, g.M - m0, wave);                           \
    if constexpr (DUAL) {                                                                            \
      lb_half.load((SB), g.b0 + (int64_t)n0 * g.ldb + k0_, 64, wave);                               \
      lb_half.load((SB) + TILE / 2, g.b1 + (int64_t)n0 * g.ldb + k0_, 64, wave);                    \
    } else if constexpr (TB) {                                                                       \
      const __bf16* src_ = k0_ < g.ksplit ? g.b0 + (int64_t)k0_ * g.ldb                             \
                                          : g.b1 + (int64_t)(k0_ - g.ksplit) * g.ldb;               \
      lb.load((SB), src_ + n0, (k0_ < g.ksplit ? g.ksplit : g.K) - k0_, wave);                       \
    } else {                                                                                         \
      lb.load((SB), g.b0 + (int64_t)n0 * g.ldb + k0_, g.N - n0, wave);                              \
    }                                                                                                \
  } while (0)

template <bool TA, bool TB, int EPI>
__global__ __launch_bounds__(256, 2) void mlp_gemm_kernel(mlp::GemmArgs g) {
  using namespace mlp;
  constexpr bool DUAL = EPI == kSwiglu || EPI == kStoreGU;
  constexpr bool PERM = TA != TB;  // the natural operand follows the transposed one's k order
  __shared__ __attribute__((aligned(1024))) char sa0[TILE];
  __shared__ __attribute__((aligned(1024))) char sa1[TILE];
  __shared__ __attribute__((aligned(1024))) char sb0[TILE];
  __shared__ __attribute__((aligned(1024))) char sb1[TILE];

  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // n tiles: 128 columns, or 64 of each matrix for a dual B
  const int n_tiles = DUAL ? g.N / 64 : g.N / BN;
  const int tn = blockIdx.x % n_tiles, tm = blockIdx.x / n_tiles;
  const int m0 = tm * BM, n0 = tn * (DUAL ? 64 : BN);
  const int kt_n = (g.K + BK - 1) / BK;

  // A stage: rows m0.. (natural, row stride lda) or k rows (transposed)
  constexpr int AD = TA ? 128 : 64, AR = TA ? 64 : 128, BD = TB ? 128 : 64, BR = TB ? 64 : 128;
  const BufTileLoader<AD, AR, 4> la(g.lda, wave, lane);
  const BufTileLoader<BD, BR, 4> lb(g.ldb, wave, lane);
  const BufTileLoader<64, 64, 4> lb_half(g.ldb, wave, lane);  // dual: 64 rows of each matrix

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // B rows of this wave's two n blocks within the B stage
  const int rb0 = DUAL ? wn * 32 : wn * 64, rb1 = DUAL ? 64 + wn * 32 : wn * 64 + 32;

  // one k tile: stage (SA, SB) holds tile KT, tile KT+1 goes to (NA, NB)
#define MLP_STEP(KT, SA, SB, NA, NB)                                                                 \
  do {                                                                                               \
    __builtin_amdgcn_s_waitcnt(0); /* this wave's loads of stage KT have landed */                   \
    __syncthreads();               /* everyone's have; stage KT-1 is no longer read */              \
    if ((KT) + 1 < kt_n) MLP_LOAD_STAGE(NA, NB, (KT) + 1);                                          \
    _Pragma("unroll") for (int s = 0; s < BK / 16; ++s) {                                            \
      const bf16x8 fa0 = frag<TA, PERM>((SA), wm * 64, s, lane);                                    \
      const bf16x8 fa1 = frag<TA, PERM>((SA), wm * 64 + 32, s, lane);                               \
      const bf16x8 fb0 = frag<TB, PERM>((SB), rb0, s, lane);                                        \
      const bf16x8 fb1 = frag<TB, PERM>((SB), rb1, s, lane);                                        \
      acc[0][0] = mfma32(fb0, fa0, acc[0][0]);                                                       \
      acc[0][1] = mfma32(fb0, fa1, acc[0][1]);                                                       \
      acc[1][0] = mfma32(fb1, fa0, acc[1][0]);                                                       \
      acc[1][1] = mfma32(fb1, fa1, acc[1][1]);                                                       \
    }                                                                                                \
  } while (0)
  MLP_LOAD_STAGE(sa0, sb0, 0);
  for (int kt = 0; kt < kt_n; kt += 2) {
    MLP_STEP(kt, sa0, sb0, sa1, sb1);
    if (kt + 1 < kt_n) MLP_STEP(kt + 1, sa1, sb1, sa0, sb0);
  }
#undef MLP_STEP

  // lane l: m = m0 + 64 wm + 32 mb + l%32; block nb's n = nbase + 8 i + 4 hf + j
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + (lane & 31);
    if (m >= g.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (EPI == kSwiglu || EPI == kStoreGU) {
        const int n = n0 + wn * 32 + 8 * i + 4 * hf;
        const f32x16& G = acc[0][mb];
        const f32x16& U = acc[1][mb];
        u32x2 w, w1;
        if constexpr (EPI == kSwiglu) {
          w[0] = pack_bf16x2(silu_f(G[4 * i + 0]) * U[4 * i + 0], silu_f(G[4 * i + 1]) * U[4 * i + 1]);
          w[1] = pack_bf16x2(silu_f(G[4 * i + 2]) * U[4 * i + 2], silu_f(G[4 * i + 3]) * U[4 * i + 3]);
        } else {
          w[0] = pack_bf16x2(G[4 * i + 0], G[4 * i + 1]);
          w[1] = pack_bf16x2(G[4 * i + 2], G[4 * i + 3]);
          w1[0] = pack_bf16x2(U[4 * i + 0], U[4 * i + 1]);
          w1[1] = pack_bf16x2(U[4 * i + 2], U[4 * i + 3]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(g.c1) + (int64_t)m * g.ldc + n) = w1;
        }
        *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(g.c) + (int64_t)m * g.ldc + n) = w;
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = n0 + wn * 64 + nb * 32 + 8 * i + 4 * hf;
          const f32x16& C = acc[nb][mb];
          if constexpr (EPI == kStoreBf16) {
            u32x2 w;
            w[0] = pack_bf16x2(C[4 * i + 0], C[4 * i + 1]);
            w[1] = pack_bf16x2(C[4 * i + 2], C[4 * i + 3]);
            *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(g.c) + (int64_t)m * g.ldc + n) = w;
          } else if constexpr (EPI == kGatedGrad) {
            // dH = C; h = silu(G) U; dG = dH U silu'(G); dU = dH silu(G)
            const int64_t o = (int64_t)m * g.ldc + n;
            const u32x2 gw = *reinterpret_cast<const u32x2*>(g.g_in + o);
            const u32x2 uw = *reinterpret_cast<const u32x2*>(g.u_in + o);
            float h[4], dg[4], du[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const unsigned gb = (gw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
              const unsigned ub = (uw[j >> 1] >> (16 * (j & 1))) & 0xffffu;
              const float gv = __uint_as_float(gb << 16), uv = __uint_as_float(ub << 16);
              const float sg = 1.f / (1.f + __expf(-gv));
              const float sl = gv * sg;
              h[j] = sl * uv;
              dg[j] = C[4 * i + j] * uv * (sg * (1.f + gv * (1.f - sg)));
              du[j] = C[4 * i + j] * sl;
            }
            u32x2 wh, wg2, wu2;
            wh[0] = pack_bf16x2(h[0], h[1]);
            wh[1] = pack_bf16x2(h[2], h[3]);
            wg2[0] = pack_bf16x2(dg[0], dg[1]);
            wg2[1] = pack_bf16x2(dg[2], dg[3]);
            wu2[0] = pack_bf16x2(du[0], du[1]);
            wu2[1] = pack_bf16x2(du[2], du[3]);
            __bf16* c1 = reinterpret_cast<__bf16*>(g.c1) + (int64_t)m * 2 * g.ldc;
            *reinterpret_cast<u32x2*>(reinterpret_cast<__bf16*>(g.c) + o) = wh;
            *reinterpret_cast<u32x2*>(c1 + n) = wg2;
            *reinterpret_cast<u32x2*>(c1 + g.ldc + n) = wu2;
          } else {  // kAccF32
            float* row = m < g.msplit ? reinterpret_cast<float*>(g.c) + (int64_t)m * g.ldc
                                      : g.c_hi + (int64_t)(m - g.msplit) * g.ldc;
            f32x4 v = *reinterpret_cast<const f32x4*>(row + n);
            v[0] += C[4 * i + 0];
            v[1] += C[4 * i + 1];
            v[2] += C[4 * i + 2];
            v[3] += C[4 * i + 3];
            *reinterpret_cast<f32x4*>(row + n) = v;
          }
        }
      }
    }
  }
}

#undef MLP_LOAD_STAGE

// Every variant the launches below use, instantiated explicitly: without
// this the host pass emitted the launch stub of only the first one.
template __global__ void mlp_gemm_kernel<false, false, mlp::kStoreBf16>(mlp::GemmArgs);
template __global__ void mlp_gemm_kernel<false, false, mlp::kSwiglu>(mlp::GemmArgs);
template __global__ void mlp_gemm_kernel<false, false, mlp::kStoreGU>(mlp::GemmArgs);
template __global__ void mlp_gemm_kernel<false, true, mlp::kStoreBf16>(mlp::GemmArgs);
template __global__ void mlp_gemm_kernel<false, true, mlp::kGatedGrad>(mlp::GemmArgs);
template __global__ void mlp_gemm_kernel<true, true, mlp::kAccF32>(mlp::GemmArgs);

__global__ __launch_bounds__(256) void mlp_zero_kernel(float* p, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i < n) *reinterpret_cast<f32x4*>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <bool TA, bool TB, int EPI>
static hipError_t gemm(const mlp::GemmArgs& g, const char* name, hipStream_t st) {
  constexpr bool DUAL = EPI == mlp::kSwiglu || EPI == mlp::kStoreGU;
  const int n_tiles = DUAL ? g.N / 64 : g.N / mlp::BN;
  const int blocks = n_tiles * ((g.M + mlp::BM - 1) / mlp::BM);
  if (blocks == 0) return hipSuccess;
  ProfScope prof(name, st);
  hipLaunchKernelGGL((mlp_gemm_kernel<TA, TB, EPI>), dim3(blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t mlp_fwd_launch(const MlpArgs& p, hipStream_t st) {
  using namespace mlp;
  __bf16* h = (__bf16*)p.ws;  // [tile][I]
  for (int t0 = 0; t0 < p.T; t0 += p.tile) {
    const int rows = min(p.tile, p.T - t0);
    GemmArgs g = {};
    // h = silu(x Wg^T) * (x Wu^T)
    g.a = p.x + (int64_t)t0 * p.H;
    g.lda = p.H;
    g.b0 = p.wg;
    g.b1 = p.wu;
    g.ldb = p.H;
    g.M = rows, g.N = p.I, g.K = p.H;
    g.c = h;
    g.ldc = p.I;
    hipError_t e = gemm<false, false, kSwiglu>(g, "mlp_gate_up", st);
    if (e != hipSuccess) return e;
    // y = h Wd^T
    g = GemmArgs{};
    g.a = h;
    g.lda = p.I;
    g.b0 = p.wd;
    g.ldb = p.I;
    g.M = rows, g.N = p.H, g.K = p.I;
    g.c = p.y + (int64_t)t0 * p.H;
    g.ldc = p.H;
    if ((e = gemm<false, false, kStoreBf16>(g, "mlp_down", st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t mlp_bwd_launch(const MlpArgs& p, hipStream_t st) {
  using namespace mlp;
  const int64_t ti = (int64_t)p.tile * p.I;
  __bf16* G = (__bf16*)p.ws;  // [tile][I] each
  __bf16* U = G + ti;
  __bf16* h = U + ti;
  __bf16* dgu = h + ti;       // [tile][2I]: dG | dU
  {
    ProfScope prof("mlp_zero", st);
    const int64_t ng = (int64_t)p.I * p.H, nd = (int64_t)p.H * p.I;
    hipLaunchKernelGGL(mlp_zero_kernel, dim3((ng / 4 + 255) / 256), dim3(256), 0, st, p.dwg, ng);
    hipLaunchKernelGGL(mlp_zero_kernel, dim3((ng / 4 + 255) / 256), dim3(256), 0, st, p.dwu, ng);
    hipLaunchKernelGGL(mlp_zero_kernel, dim3((nd / 4 + 255) / 256), dim3(256), 0, st, p.dwd, nd);
  }
  for (int t0 = 0; t0 < p.T; t0 += p.tile) {
    const int rows = min(p.tile, p.T - t0);
    const __bf16* xt = p.x + (int64_t)t0 * p.H;
    const __bf16* dyt = p.dy + (int64_t)t0 * p.H;
    hipError_t e;
    // recompute G = x Wg^T, U = x Wu^T
    GemmArgs g = {};
    g.a = xt, g.lda = p.H, g.b0 = p.wg, g.b1 = p.wu, g.ldb = p.H;
    g.M = rows, g.N = p.I, g.K = p.H;
    g.c = G, g.c1 = U, g.ldc = p.I;
    if ((e = gemm<false, false, kStoreGU>(g, "mlp_bwd_gate_up", st)) != hipSuccess) return e;
    // dH = dy Wd (Wd [H][I] is k-major for this product); h, dG, dU
    g = GemmArgs{};
    g.a = dyt, g.lda = p.H, g.b0 = p.wd, g.b1 = p.wd, g.ldb = p.I, g.ksplit = p.H;
    g.M = rows, g.N = p.I, g.K = p.H;
    g.c = h, g.c1 = dgu, g.ldc = p.I, g.g_in = G, g.u_in = U;
    if ((e = gemm<false, true, kGatedGrad>(g, "mlp_bwd_gated", st)) != hipSuccess) return e;
    // dx = dG Wg + dU Wu: K = 2I over [Wg; Wu], both k-major here
    g = GemmArgs{};
    g.a = dgu, g.lda = 2 * (int64_t)p.I, g.b0 = p.wg, g.b1 = p.wu, g.ldb = p.H, g.ksplit = p.I;
    g.M = rows, g.N = p.H, g.K = 2 * p.I;
    g.c = p.dx + (int64_t)t0 * p.H, g.ldc = p.H;
    if ((e = gemm<false, true, kStoreBf16>(g, "mlp_bwd_dx", st)) != hipSuccess) return e;
    // [dWg; dWu] += [dG | dU]^T x  (M = 2I rows, K = the tile's tokens)
    g = GemmArgs{};
    g.a = dgu, g.lda = 2 * (int64_t)p.I, g.b0 = xt, g.b1 = xt, g.ldb = p.H, g.ksplit = rows;
    g.M = 2 * p.I, g.N = p.H, g.K = rows;
    g.c = p.dwg, g.c_hi = p.dwu, g.msplit = p.I, g.ldc = p.H;
    if ((e = gemm<true, true, kAccF32>(g, "mlp_bwd_dw_gate_up", st)) != hipSuccess) return e;
    // dWd += dy^T h  (M = H, N = I)
    g = GemmArgs{};
    g.a = dyt, g.lda = p.H, g.b0 = h, g.b1 = h, g.ldb = p.I, g.ksplit = rows;
    g.M = p.H, g.N = p.I, g.K = rows;
    g.c = p.dwd, g.c_hi = p.dwd, g.msplit = p.H, g.ldc = p.I;
    if ((e = gemm<true, true, kAccF32>(g, "mlp_bwd_dw_down", st)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace uly

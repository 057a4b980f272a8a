// Attention backward of one Ulysses rank.
//
//   delta_i = sum_d dO_i,d O_i,d                         (attn_bwd_pre)
//   P_ij = exp(s_ij - LSE_i), dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - delta_i)
//   dK_j = scale sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i  (attn_bwd_dkdv: one
//          work-group owns 32*NW keys of one KV head and walks every query of
//          every head of its group, accumulating in registers)
//   dQ_i = scale sum_j dS_ij k_j                         (attn_bwd_dq: one
//          work-group owns 32*NW queries of one head and walks the keys)
//   dsink_h = -sum_i exp(sink_h - LSE_i) D_i             (dsink_partial/final)
//          with D_i = sum_j P_ij dP_ij accumulated by attn_bwd_dq: equal to
//          dO_i . O_i for the exact O, not the bf16-rounded O delta_i uses
// Both main kernels recompute P from LSE; neither uses atomics, so the
// gradients are deterministic.
#include "attn_common.hpp"
#include "launch.hpp"

namespace uly {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------- delta, dsink

// One 16-byte chunk of dO and O per thread, D/8 threads per (row, head).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(AttnArgs a) {
  constexpr int TPR = D / 8;  // threads per row
  const int row = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;  // row = t * hq + h
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  const bool valid = row < a.T * a.hq;
  if (valid) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.dout + (int64_t)row * D + 8 * c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.o + (int64_t)row * D + 8 * c);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += bf16_lo(x[w]) * bf16_lo(y[w]) + bf16_hi(x[w]) * bf16_hi(y[w]);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (valid && c == 0) {
    const int t = row / a.hq, h = row - t * a.hq;
    const int idx = lse_index(a, t, h);
    a.delta[idx] = acc;
    const float l = a.lse[idx];
    a.lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;  // rows with no key: P = 0
  }
}

// Per head, n_part partial sums of -exp(sink - LSE_i) delta_i over the rows.
__global__ __launch_bounds__(256) void dsink_partial_kernel(AttnArgs a) {
  __shared__ float red[256];
  const int h = blockIdx.y, part = blockIdx.x;
  const float s = a.sink[h];
  float acc = 0.f;
  for (int t = part * 256 + threadIdx.x; t < a.T; t += a.n_part * 256) {
    const int idx = lse_index(a, t, h);
    const float l = a.lse[idx];
    if (l != -INFINITY) acc -= __expf(s - l) * a.pdp[idx];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dsink_part[h * a.n_part + part] = red[0];
}

__global__ void dsink_final_kernel(AttnArgs a) {
  const int h = threadIdx.x;
  if (h < a.hq) {
    float acc = 0.f;
    for (int p = 0; p < a.n_part; ++p) acc += a.dsink_part[h * a.n_part + p];
    a.dsink[h] = acc;
  }
}

// ---------------------------------------------------------------------- dQ
//
// One work-group = NW waves x 32 query rows of one head (S^T form, as the
// forward: a lane owns one query).  K and V tiles of 64 keys arrive by
// global_load_lds into swizzled natural tiles; K also serves the K^T operand
// of dQ^T += K^T dS^T through the transposing reads.

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_kernel(AttnArgs a) {
  constexpr int BM = 32 * NW, NB = D / 32, KS = D / 16;
  constexpr int TILE = kBK * D * 2;
  constexpr int STAGE = 2 * TILE;  // K, then V
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  int qt, h;
  if (!decode_qtile(a, qt, h)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5;
  const int g = h / a.G;
  const int q0 = qt * BM;
  const int qrow = q0 + 32 * wave + (lane & 31);
  const bool qvalid = qrow < a.T;

  int klo = 0, khi = 0;
  if (qvalid) key_interval(a, qrow, klo, khi);
  const int q_last = min(q0 + BM, a.T) - 1;
  int wg_lo, wg_hi, full_lo, full_hi;
  key_interval(a, q0, wg_lo, full_hi);
  key_interval(a, q_last, full_lo, wg_hi);

  bf16x8 qf[KS], dof[KS];
  load_row_frags<D>(qf, a.q + ((int64_t)qrow * a.hq + h) * D, qvalid, lane);
  load_row_frags<D>(dof, a.dout + ((int64_t)qrow * a.hq + h) * D, qvalid, lane);
  float lse2 = INFINITY, dlt = 0.f;  // invalid rows: P = 0
  if (qvalid) {
    lse2 = a.lse2[lse_index(a, qrow, h)];
    dlt = a.delta[lse_index(a, qrow, h)];
  }

  f32x16 dqacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[nb][e] = 0.f;
  const bool want_pdp = a.sink != nullptr;
  float pdp = 0.f;
  const f32x16 zero = {};

  const __bf16* kbase = a.k + (int64_t)g * D;
  const __bf16* vbase = a.v + (int64_t)g * D;
  const int ld = a.hkv * D;
  const int n_iter = (wg_hi - wg_lo + kBK - 1) / kBK;
  if (n_iter > 0) {
    tile_load_lds<D, kBK, NW>(smem, kbase, ld, wg_lo, a.T, wave, lane);
    tile_load_lds<D, kBK, NW>(smem + TILE, vbase, ld, wg_lo, a.T, wave, lane);
  }

  for (int it = 0; it < n_iter; ++it) {
    const int cur = it & 1;
    const int k0 = wg_lo + it * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_iter) {
      char* nxt = smem + (cur ^ 1) * STAGE;
      tile_load_lds<D, kBK, NW>(nxt, kbase, ld, k0 + kBK, a.T, wave, lane);
      tile_load_lds<D, kBK, NW>(nxt + TILE, vbase, ld, k0 + kBK, a.T, wave, lane);
    }
    const char* kt = smem + cur * STAGE;
    const char* vt = kt + TILE;

    const bool full = k0 >= full_lo && k0 + kBK <= full_hi;
    // one 32-key block at a time keeps two accumulators live, not four
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = mfma32(swz_nat<D>(kt, 32 * mb, s, lane), qf[s], s == 0 ? zero : sacc);
        dpacc = mfma32(swz_nat<D>(vt, 32 * mb, s, lane), dof[s], s == 0 ? zero : dpacc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.scale_log2, -lse2));
        if (!full) {
          const int key = k0 + 32 * mb + 8 * (e >> 2) + 4 * hf + (e & 3);
          if (key < klo || key >= khi) p = 0.f;
        }
        if (want_pdp) pdp = __builtin_fmaf(p, dpacc[e], pdp);
        sacc[e] = p * (dpacc[e] - dlt);  // dS^T
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const bf16x8 df = acc_frag(sacc, ii);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          dqacc[nb] = mfma32(swz_tr<D>(kt, 32 * mb + 16 * ii, 32 * nb, lane), df, dqacc[nb]);
      }
    }
  }

  pdp = halves_sum(pdp);
  if (qvalid && want_pdp && hf == 0) a.pdp[lse_index(a, qrow, h)] = pdp;
  if (qvalid) {
    __bf16* row = a.out + ((int64_t)qrow * a.hq + h) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(dqacc[nb][4 * i + 0] * a.scale, dqacc[nb][4 * i + 1] * a.scale);
        w[1] = pack_bf16x2(dqacc[nb][4 * i + 2] * a.scale, dqacc[nb][4 * i + 3] * a.scale);
        *reinterpret_cast<u32x2*>(row + 32 * nb + 8 * i + 4 * hf) = w;
      }
  }
}

// ------------------------------------------------------------------ dK, dV
//
// One work-group = NW waves x 32 keys of one KV head; K and V rows stay in
// registers as B operands.  The work-group walks every query tile (64 rows)
// of every query head of the group: Q and dO tiles plus their LSE*log2(e)
// and delta rows arrive by global_load_lds, and each tile serves both the
// natural operand (S = Q K^T, dP = dO V^T) and, through the transposing
// reads, the operand of dV += P^T dO and dK += dS^T Q.

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bwd_dkdv_kernel(AttnArgs a) {
  static_assert(NW >= 2, "two waves stage the per-row statistics");
  constexpr int BN = 32 * NW, NB = D / 32, KS = D / 16;
  constexpr int TILE = kBK * D * 2;
  constexpr int STAGE = 2 * TILE + 2 * kBK * 4;  // Q, dO, LSE*log2e, delta
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int L = blockIdx.x;
  if (L >= a.n_tiles * a.hkv) return;
  const int kt = L / a.hkv, g = L % a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5;
  const int k0 = kt * BN;
  const int krow = k0 + 32 * wave + (lane & 31);
  const bool kvalid = krow < a.T;

  int qlo = 0, qhi = 0;
  if (kvalid) query_interval(a, krow, qlo, qhi);
  const int k_last = min(k0 + BN, a.T) - 1;
  int wg_lo, wg_hi, full_lo, full_hi;
  query_interval(a, k0, wg_lo, full_hi);
  query_interval(a, k_last, full_lo, wg_hi);

  bf16x8 kf[KS], vf[KS];
  load_row_frags<D>(kf, a.k + ((int64_t)krow * a.hkv + g) * D, kvalid, lane);
  load_row_frags<D>(vf, a.v + ((int64_t)krow * a.hkv + g) * D, kvalid, lane);

  f32x16 dkacc[NB], dvacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkacc[nb][e] = 0.f;
      dvacc[nb][e] = 0.f;
    }
  const f32x16 zero = {};

  const int ld = a.hq * D;
  const int nq = (wg_hi - wg_lo + kBK - 1) / kBK;  // query tiles per head
  const int n_iter = nq * a.G;

  auto issue = [&](int it, char* buf) {
    const int hh = it / nq, qa = wg_lo + (it - hh * nq) * kBK;
    const int h = g * a.G + hh;
    tile_load_lds<D, kBK, NW>(buf, a.q + (int64_t)h * D, ld, qa, a.T, wave, lane);
    tile_load_lds<D, kBK, NW>(buf + TILE, a.dout + (int64_t)h * D, ld, qa, a.T, wave, lane);
    if (wave < 2) {
      const int idx = lse_index(a, min(qa + lane, a.T - 1), h);
      const float* src = wave == 0 ? a.lse2 + idx : a.delta + idx;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + 2 * TILE + wave * kBK * 4), 4, 0, 0);
    }
  };

  if (n_iter > 0) issue(0, smem);

  for (int it = 0; it < n_iter; ++it) {
    const int cur = it & 1;
    const int hh = it / nq, qa = wg_lo + (it - hh * nq) * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_iter) issue(it + 1, smem + (cur ^ 1) * STAGE);
    const char* qs = smem + cur * STAGE;
    const char* dos = qs + TILE;
    const float* lsd = reinterpret_cast<const float*>(qs + 2 * TILE);
    const bool full = qa >= full_lo && qa + kBK <= full_hi;

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q K^T and dP = dO V^T: column = this lane's key, rows = 32 queries
      f32x16 sacc, dpacc;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = mfma32(swz_nat<D>(qs, 32 * qb, s, lane), kf[s], s == 0 ? zero : sacc);
        dpacc = mfma32(swz_nat<D>(dos, 32 * qb, s, lane), vf[s], s == 0 ? zero : dpacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 32 * qb + 8 * i + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsd + r0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(lsd + kBK + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * i + j], a.scale_log2, -l4[j]));
          if (!full) {
            const int qi = qa + r0 + j;
            if (qi < qlo || qi >= qhi) p = 0.f;
          }
          sacc[4 * i + j] = p;
          dpacc[4 * i + j] = p * (dpacc[4 * i + j] - d4[j]);
        }
      }
      // dV += P^T dO, dK += dS^T Q (contraction over the 32 queries)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const bf16x8 pf = acc_frag(sacc, ii);
        const bf16x8 df = acc_frag(dpacc, ii);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          dvacc[nb] = mfma32(pf, swz_tr<D>(dos, 32 * qb + 16 * ii, 32 * nb, lane), dvacc[nb]);
          dkacc[nb] = mfma32(df, swz_tr<D>(qs, 32 * qb + 16 * ii, 32 * nb, lane), dkacc[nb]);
        }
      }
    }
  }

  // dK, dV: lane holds column d = 32 nb + l % 32 of key rows 8 i + 4 hf + j
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = k0 + 32 * wave + 8 * (e >> 2) + 4 * hf + (e & 3);
      if (key < a.T) {
        const int64_t off = ((int64_t)key * a.hkv + g) * D + 32 * nb + (lane & 31);
        a.dk[off] = (__bf16)(dkacc[nb][e] * a.scale);
        a.dv[off] = (__bf16)dvacc[nb][e];
      }
    }
}

// ------------------------------------------------------------------ launches

template <int D, int NW>
static hipError_t launch_bwd_t(const AttnArgs& args, hipStream_t st) {
  AttnArgs a = args;
  {
    const int rows = a.T * a.hq, rpb = 256 / (D / 8);
    ProfScope prof("attn_bwd_pre", st);
    hipLaunchKernelGGL(attn_bwd_pre_kernel<D>, dim3((rows + rpb - 1) / rpb), dim3(256), 0, st, a);
  }
  {
    AttnArgs b = a;
    b.n_tiles = (a.T + 32 * NW - 1) / (32 * NW);
    ProfScope prof("attn_bwd_dkdv", st);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, NW>), dim3(b.n_tiles * a.hkv), dim3(NW * 64), 0, st, b);
  }
  {
    AttnArgs b = a;
    b.n_tiles = (a.T + 32 * NW - 1) / (32 * NW);
    const int groups = b.n_tiles * a.hkv;
    const int blocks = ((groups + kXcds - 1) / kXcds) * kXcds * a.G;
    ProfScope prof("attn_bwd_dq", st);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NW>), dim3(blocks), dim3(NW * 64), 0, st, b);
  }
  if (a.sink != nullptr) {
    ProfScope prof("attn_bwd_dsink", st);
    hipLaunchKernelGGL(dsink_partial_kernel, dim3(a.n_part, a.hq), dim3(256), 0, st, a);
    hipLaunchKernelGGL(dsink_final_kernel, dim3(1), dim3(((a.hq + 63) / 64) * 64), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t attn_bwd_launch(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128) return launch_bwd_t<128, 4>(a, st);
  return launch_bwd_t<64, 4>(a, st);
}

}  // namespace uly

// Attention forward of one Ulysses rank: O = softmax(scale Q K^T + mask, sink) V
// and the per-row log-sum-exp.
//
// One work-group = NW waves = 32*NW consecutive query rows of one query head.
// Each wave keeps its 32 query rows in registers as the B operand of
// S^T = K Q^T; K tiles (natural layout) and V tiles (transposed layout) of
// 64 keys are staged through double-buffered LDS, the next tile's global
// loads in flight while the current tile is multiplied.  The online softmax
// is per lane (one query per lane, see attn_common.hpp): running max in the
// log2 domain, running sum, and a rescale of the output accumulator only
// when the max grows by more than 2^8 (the final O / l is exact for any
// reference max; the bound keeps every exponent <= 2^8).
#include "attn_common.hpp"
#include "launch.hpp"

namespace uly {

constexpr float kRescaleLog2 = 8.0f;

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(AttnArgs a) {
  constexpr int NT = NW * 64, BM = 32 * NW, NB = D / 32, KS = D / 16;
  typedef Tile<D> TL;
  constexpr int BUF = TL::kNatElems + TL::kTrElems;  // K natural, then V transposed
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * BUF];

  int qt, h;
  if (!decode_qtile(a, qt, h)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5;
  const int g = h / a.G;
  const int q0 = qt * BM;
  const int qrow = q0 + 32 * wave + (lane & 31);
  const bool qvalid = qrow < a.T;

  // key interval of this lane's query, and of the work-group
  int klo = 0, khi = 0;
  if (qvalid) key_interval(a, qrow, klo, khi);
  const int q_last = min(q0 + BM, a.T) - 1;
  int wg_lo, wg_hi, full_lo, full_hi;
  key_interval(a, q0, wg_lo, full_hi);     // full_hi: smallest khi over the rows
  key_interval(a, q_last, full_lo, wg_hi); // full_lo: largest klo over the rows

  bf16x8 qf[KS];
  load_row_frags<D>(qf, a.q + ((int64_t)qrow * a.hq + h) * D, qvalid, lane);

  f32x16 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[nb][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const __bf16* kbase = a.k + (int64_t)g * D;
  const __bf16* vbase = a.v + (int64_t)g * D;
  const int ld = a.hkv * D;
  TileLoader<D, NT> ldk, ldv;

  const int n_iter = (wg_hi - wg_lo + kBK - 1) / kBK;
  if (n_iter > 0) {
    ldk.load_nat(kbase, ld, wg_lo, a.T, tid);
    ldv.load_tr(vbase, ld, wg_lo, a.T, tid);
    ldk.store_nat(smem, tid);
    ldv.store_tr(smem + TL::kNatElems, tid);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int cur = it & 1;
    const int k0 = wg_lo + it * kBK;
    if (it + 1 < n_iter) {
      ldk.load_nat(kbase, ld, k0 + kBK, a.T, tid);
      ldv.load_tr(vbase, ld, k0 + kBK, a.T, tid);
    }
    const __bf16* ks = smem + cur * BUF;
    const __bf16* vs = ks + TL::kNatElems;

    // S^T = K Q^T for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[mb][e] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) sacc[mb] = mfma32(nat_frag<D>(ks, 32 * mb, s, lane), qf[s], sacc[mb]);
    }

    // mask (only tiles that are not fully visible to every row)
    const bool full = k0 >= full_lo && k0 + kBK <= full_hi;
    if (!full) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * mb + 8 * (e >> 2) + 4 * hf + (e & 3);
          if (key < klo || key >= khi) sacc[mb][e] = -INFINITY;
        }
    }

    // online softmax, log2 domain
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mb][e]);
    mx = halves_max(mx) * a.scale_log2;
    const bool grow = mx > m_run + kRescaleLog2;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[nb][e] *= alpha;
    }
    const float msub = m_run == -INFINITY ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][e], a.scale_log2, -msub));
        sacc[mb][e] = p;
        lsum += p;
      }
    l_run += lsum;

    // O^T += V^T P^T
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const bf16x8 pf = acc_frag(sacc[mb], ii);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          oacc[nb] = mfma32(tr_frag<D>(vs, 32 * mb + 16 * ii, 32 * nb, lane), pf, oacc[nb]);
      }

    if (it + 1 < n_iter) {
      ldk.store_nat(smem + (cur ^ 1) * BUF, tid);
      ldv.store_tr(smem + (cur ^ 1) * BUF + TL::kNatElems, tid);
    }
    __syncthreads();
  }

  // finish: both halves hold partial sums of the same row; fold in the sink
  float l_tot = halves_sum(l_run);
  float m_fin = m_run;
  if (a.sink != nullptr) {
    const float s2 = a.sink[h] * 1.4426950408889634f;
    m_fin = fmaxf(m_run, s2);
    l_tot = (m_run == -INFINITY ? 0.f : l_tot * exp2f(m_run - m_fin)) + exp2f(s2 - m_fin);
  }
  const float oscale = (m_fin == -INFINITY || l_tot == 0.f) ? 0.f
                       : (m_run == -INFINITY ? 0.f : exp2f(m_run - m_fin) / l_tot);
  if (qvalid) {
    __bf16* orow = a.out + ((int64_t)qrow * a.hq + h) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[nb][4 * i + 0] * oscale, oacc[nb][4 * i + 1] * oscale);
        w[1] = pack_bf16x2(oacc[nb][4 * i + 2] * oscale, oacc[nb][4 * i + 3] * oscale);
        *reinterpret_cast<u32x2*>(orow + 32 * nb + 8 * i + 4 * hf) = w;
      }
    if (hf == 0) {
      const float lse = (m_fin == -INFINITY || l_tot == 0.f) ? -INFINITY
                        : (m_fin + __log2f(l_tot)) * 0.6931471805599453f;
      a.lse[lse_index(a, qrow, h)] = lse;
    }
  }
}

template <int D, int NW>
static hipError_t launch_fwd_t(const AttnArgs& args, hipStream_t st) {
  AttnArgs a = args;
  a.n_tiles = (a.T + 32 * NW - 1) / (32 * NW);
  const int groups = a.n_tiles * a.hkv;
  const int blocks = ((groups + kXcds - 1) / kXcds) * kXcds * a.G;
  ProfScope prof("attn_fwd", st);
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW>), dim3(blocks), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

hipError_t attn_fwd_launch(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128) return launch_fwd_t<128, 4>(a, st);
  return launch_fwd_t<64, 4>(a, st);
}

}  // namespace uly

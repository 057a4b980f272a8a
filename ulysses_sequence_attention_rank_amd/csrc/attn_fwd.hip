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

// K and V tiles of the 64 keys from row0 into dst (V one tile after K):
// uniformly strided rows through buffer loads (rows past kt_hi read as zero
// and are masked), general layouts through per-row address maps with the
// rows clamped to [kt_lo, kt_hi)
template <int D, int NW, bool KV_UNIFORM>
__device__ __forceinline__ void load_kv(char* dst, const AttnArgs& a, const BufTileLoader<D, kBK, NW>& kvl,
                                        const __bf16* kbase, const __bf16* vbase, int row0, int wave,
                                        int lane) {
  constexpr int TILE = kBK * D * 2;
  if constexpr (KV_UNIFORM) {
    const int64_t o = (int64_t)(row0 - a.mk.s0) * a.mk.token;
    kvl.load(dst, kbase + o, a.kt_hi - row0, wave);
    kvl.load(dst + TILE, vbase + o, a.kt_hi - row0, wave);
  } else {
    tile_load_lds_map<D, kBK, NW, false>(dst, kbase, a.mk, row0, a.kt_lo, a.kt_hi, wave, lane);
    tile_load_lds_map<D, kBK, NW, false>(dst + TILE, vbase, a.mk, row0, a.kt_lo, a.kt_hi, wave, lane);
  }
}

// S^T = K Q^T for one 64-key tile `kt`: each K operand read feeds QB products.
template <int D, int QB>
__device__ __forceinline__ void tile_scores(f32x16 (&sacc)[QB][2], const SwzOffsets<D>& so, const char* kt,
                                            const bf16x8 (&qf)[QB][D / 16]) {
  const f32x16 zero = {};
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 kf = so.nat_at(kt, 32 * mb, s);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][mb] = mfma32(kf, qf[qb][s], s == 0 ? zero : sacc[qb][mb]);
    }
  if constexpr (QB == 1) {
    // keep 8 operand reads in flight ahead of the products (the default
    // schedule issues each read just before its product and waits out the
    // LDS latency every time)
    constexpr int PF = 8, N = 2 * (D / 16);
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < N - PF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  }
}

// First half of the online softmax of one query block over one tile: the
// mask (unless the tile is wholly visible; vis_lo / vis_hi are the lane's
// visible keys relative to its first key slot, slot e of block mb holding
// key offset 32 mb + 8 (e / 4) + e % 4), the tile's row max in the log2
// domain, and the lazy rescale of the running state when that max exceeds
// the reference max by more than 2^8.  Returns the max to subtract.
template <int NB>
__device__ __forceinline__ float softmax_max(f32x16 (&sacc)[2], bool full, int vis_lo, int vis_hi,
                                             float scale_log2, float& m_run, float& l_run,
                                             f32x16 (&oacc)[NB]) {
  if (!full) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = 32 * mb + 8 * (e >> 2) + (e & 3);
        if (c < vis_lo || c >= vis_hi) sacc[mb][e] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mb][e]);
  mx = halves_max(mx) * scale_log2;
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
  return m_run == -INFINITY ? 0.f : m_run;
}

// Second half: the probabilities 2^(s scale_log2 - msub), their fp32 row sum
// (the LSE it yields also sets dsink's sink probabilities) and their bf16 B
// operands of O^T += V^T P^T.
__device__ __forceinline__ void softmax_exp(f32x16 (&sacc)[2], float msub, float scale_log2, float& l_run,
                                            bf16x8 (&pf)[4]) {
  float lsum = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][e], scale_log2, -msub));
      sacc[mb][e] = p;
      lsum += p;
    }
  l_run += lsum;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) pf[2 * mb + ii] = acc_frag(sacc[mb], ii);
}

// O^T += V^T P^T for one tile `vt`: each V operand read feeds QB products.
template <int D, int QB>
__device__ __forceinline__ void tile_pv(f32x16 (&oacc)[QB][D / 32], const SwzOffsets<D>& so, const char* vt,
                                        const bf16x8 (&pf)[QB][4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      const bf16x8 vf = so.tr_at(vt, 16 * ks, nb);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[qb][nb] = mfma32(vf, pf[qb][ks], oacc[qb][nb]);
    }
}

template <int D, int NW, int QB, bool KV_UNIFORM>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int BM = 32 * QB * NW, NB = D / 32, KS = D / 16;
  constexpr int TILE = kBK * D * 2;  // bytes of one K or V tile
  constexpr int STAGE = 2 * TILE;
  // Two LDS stages as distinct objects: each access below names one of them
  // statically, which lets the compiler see that the next tile's
  // direct-to-LDS loads cannot alias the current tile's reads, so it does not
  // make those reads wait for the loads.
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];

  int qt, h;
  if (!decode_qtile(a, qt, h)) return;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = h / a.G;
  const int q0 = qt * BM;

  // this lane's QB queries (one per 32-row block of the wave) and their key intervals
  int qrow[QB], klo[QB], khi[QB];
  bool qvalid[QB];
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = q0 + 32 * (wave * QB + qb) + (lane & 31);
    qvalid[qb] = qrow[qb] < a.T;
    klo[qb] = khi[qb] = 0;
    if (qvalid[qb]) key_interval(a, qrow[qb], klo[qb], khi[qb]);
    load_row_frags<D>(qf[qb], a.q + (qvalid[qb] ? row_of(a.mq, qrow[qb]) : 0) + (int64_t)h * a.mq.head,
                      qvalid[qb], lane);
  }
  const int q_last = min(q0 + BM, a.T) - 1;
  int wg_lo, wg_hi, full_lo, full_hi;
  key_interval(a, q0, wg_lo, full_hi);      // full_hi: smallest khi over the rows
  key_interval(a, q_last, full_lo, wg_hi);  // full_lo: largest klo over the rows

  f32x16 oacc[QB][NB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[qb][nb][e] = 0.f;
  }

  const __bf16* kbase = a.k + (int64_t)g * a.mk.head;
  const __bf16* vbase = a.v + (int64_t)g * a.mk.head;
  // this split's share of the key tiles
  int it_lo, it_hi;
  split_range((wg_hi - wg_lo + kBK - 1) / kBK, blockIdx.y, a.nsplit, it_lo, it_hi);
  const BufTileLoader<D, kBK, NW> kvl(a.mk.token, wave, lane);
  SwzOffsets<D> so(lane);
  // one key tile: `cur` holds tile `it` (K, then V), tile it+1 goes to `nxt`
  auto step = [&](int it, const char* cur, char* nxt) __attribute__((always_inline)) {
    const int k0 = wg_lo + it * kBK;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `it` have landed
    __syncthreads();                // everyone's have, and tile it-1 is no longer read
    if (it + 1 < it_hi) load_kv<D, NW, KV_UNIFORM>(nxt, a, kvl, kbase, vbase, k0 + kBK, wave, lane);
    so.refresh();  // one set of read offsets serves both stages
    f32x16 sacc[QB][2];
    tile_scores<D, QB>(sacc, so, cur, qf);
    const bool full = k0 >= full_lo && k0 + kBK <= full_hi;
    bf16x8 pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float msub = softmax_max<NB>(sacc[qb], full, klo[qb] - (k0 + 4 * hf), khi[qb] - (k0 + 4 * hf),
                                         a.scale_log2, m_run[qb], l_run[qb], oacc[qb]);
      softmax_exp(sacc[qb], msub, a.scale_log2, l_run[qb], pf[qb]);
    }
    tile_pv<D, QB>(oacc, so, cur + TILE, pf);
  };
  if (it_lo < it_hi) load_kv<D, NW, KV_UNIFORM>(stage0, a, kvl, kbase, vbase, wg_lo + it_lo * kBK, wave, lane);
  if constexpr (QB == 1) {
    for (int it = it_lo; it < it_hi; it += 2) {
      step(it, stage0, stage1);
      if (it + 1 < it_hi) step(it + 1, stage1, stage0);
    }
  } else {  // two query blocks: one copy of the body keeps them in registers
    for (int it = it_lo; it < it_hi; ++it) {
      const bool odd = (it - it_lo) & 1;
      step(it, odd ? stage1 : stage0, odd ? stage0 : stage1);
    }
  }

  if (a.nsplit > 1) {
    // this split's unnormalised output, running max (log2 domain) and sum,
    // merged by attn_fwd_merge_kernel
    const int64_t rows = (int64_t)a.T * a.hq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = halves_sum(l_run[qb]);
      if (!qvalid[qb]) continue;
      float* orow = a.part + ((int64_t)blockIdx.y * rows + (int64_t)qrow[qb] * a.hq + h) * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 w = {oacc[qb][nb][4 * i + 0], oacc[qb][nb][4 * i + 1], oacc[qb][nb][4 * i + 2],
                           oacc[qb][nb][4 * i + 3]};
          *reinterpret_cast<f32x4*>(orow + 32 * nb + 8 * i + 4 * hf) = w;
        }
      if (hf == 0) {
        const int idx = lse_index(a, qrow[qb], h);
        a.part_pdp[(int64_t)blockIdx.y * rows + idx] = m_run[qb];
        a.part_pdp[(int64_t)(a.nsplit + blockIdx.y) * rows + idx] = l_tot;
      }
    }
    return;
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    // both halves hold partial sums of the same row; fold in the sink
    float l_tot = halves_sum(l_run[qb]);
    const float mr = m_run[qb];
    float m_fin = mr;
    if (a.sink != nullptr) {
      const float s2 = a.sink[h] * 1.4426950408889634f;
      m_fin = fmaxf(mr, s2);
      l_tot = (mr == -INFINITY ? 0.f : l_tot * exp2f(mr - m_fin)) + exp2f(s2 - m_fin);
    }
    const float oscale = (m_fin == -INFINITY || l_tot == 0.f || mr == -INFINITY)
                             ? 0.f : exp2f(mr - m_fin) / l_tot;
    if (qvalid[qb]) {
      if (a.o_f32) {
        float* orow = reinterpret_cast<float*>(a.out) + ((int64_t)qrow[qb] * a.hq + h) * D;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 w = {oacc[qb][nb][4 * i + 0] * oscale, oacc[qb][nb][4 * i + 1] * oscale,
                             oacc[qb][nb][4 * i + 2] * oscale, oacc[qb][nb][4 * i + 3] * oscale};
            *reinterpret_cast<f32x4*>(orow + 32 * nb + 8 * i + 4 * hf) = w;
          }
      } else {
        __bf16* orow = a.out + row_of(a.mq, qrow[qb]) + (int64_t)h * a.mq.head;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[qb][nb][4 * i + 0] * oscale, oacc[qb][nb][4 * i + 1] * oscale);
            w[1] = pack_bf16x2(oacc[qb][nb][4 * i + 2] * oscale, oacc[qb][nb][4 * i + 3] * oscale);
            *reinterpret_cast<u32x2*>(orow + 32 * nb + 8 * i + 4 * hf) = w;
          }
      }
      if (hf == 0) {
        const float lse = (m_fin == -INFINITY || l_tot == 0.f) ? -INFINITY
                          : (m_fin + __log2f(l_tot)) * 0.6931471805599453f;
        a.lse[lse_index(a, qrow[qb], h)] = lse;
      }
    }
  }
}

// Merge of the split partials of one (row, head): with M = max(m_s, sink),
// Z = sum_s l_s 2^(m_s - M) + 2^(sink - M), O = sum_s O_s 2^(m_s - M) / Z and
// LSE = (M + log2 Z) ln 2.  One thread per 4 output columns.
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(AttnArgs a) {
  const int64_t rows = (int64_t)a.T * a.hq;
  const int64_t idx4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = idx4 / (D / 4);  // flattened (token, head) row
  const int c = (int)(idx4 % (D / 4)) * 4;
  if (r >= rows) return;
  const int t = (int)(r / a.hq), h = (int)(r % a.hq);
  const int li = lse_index(a, t, h);
  float m = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) m = fmaxf(m, a.part_pdp[s * rows + li]);
  const float s2 = a.sink != nullptr ? a.sink[h] * 1.4426950408889634f : -INFINITY;
  const float mf = fmaxf(m, s2);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (mf != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.part_pdp[s * rows + li];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - mf);
      z += a.part_pdp[(a.nsplit + s) * rows + li] * w;
      o += *reinterpret_cast<const f32x4*>(a.part + (s * rows + r) * D + c) * w;
    }
    if (a.sink != nullptr) z += exp2f(s2 - mf);
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  if (a.o_f32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + r * D + c) = o * inv;
  } else {
    u32x2 w;
    w[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
    w[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
    *reinterpret_cast<u32x2*>(a.out + row_of(a.mq, t) + (int64_t)h * a.mq.head + c) = w;
  }
  if (c == 0) a.lse[li] = z > 0.f ? (mf + __log2f(z)) * 0.6931471805599453f : -INFINITY;
}

template <int D, int NW, int QB>
static hipError_t launch_fwd_t(const AttnArgs& args, hipStream_t st) {
  AttnArgs a = args;
  a.n_tiles = (a.T + 32 * QB * NW - 1) / (32 * QB * NW);
  const int groups = a.n_tiles * a.hkv;
  const int blocks = ((groups + kXcds - 1) / kXcds) * kXcds * a.G;
  {
    ProfScope prof("attn_fwd", st);
    if (a.mk.uniform)
      hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, true>), dim3(blocks, a.nsplit), dim3(NW * 64), 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_kernel<D, NW, QB, false>), dim3(blocks, a.nsplit), dim3(NW * 64), 0, st, a);
  }
  if (a.nsplit > 1) {
    ProfScope prof("attn_fwd_merge", st);
    const int64_t items = (int64_t)a.T * a.hq * (D / 4);
    hipLaunchKernelGGL(attn_fwd_merge_kernel<D>, dim3((items + 255) / 256), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

// D=64: two query blocks per wave (halves the LDS operand traffic per
// product) still fit two waves per SIMD; D=128 takes one block per wave.
// ---------------------------------------------------------- chunk merge
//
// Exact combination of attention over two disjoint KV chunks (the ring inner
// step): with L = log(e^La + e^Lb), O = e^(La - L) Oa + e^(Lb - L) Ob.  In
// place on the accumulator (acc_o fp32 [T][hq][D], acc_lse [B][hq][S]).  One
// thread per 4 columns; a (row, head) never spans two blocks, and its new LSE
// is written after the block has read the old one.
struct MergeArgs {
  float* acc_o;
  float* acc_lse;
  const float* o;
  const float* lse;
  const float* sink;
  __bf16* out;
  float* lse_out;
  int T, S, hq, D;
};

__device__ __forceinline__ int merge_lse_index(const MergeArgs& m, int t, int h) {
  const int b = t / m.S;
  return (b * m.hq + h) * m.S + (t - b * m.S);
}

__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs m) {
  const int64_t rows = (int64_t)m.T * m.hq;
  const int64_t idx4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q4 = m.D / 4;
  const int64_t r = idx4 / q4;  // flattened (token, head) row
  const int c = (int)(idx4 - r * q4) * 4;
  float la = -INFINITY, lb = -INFINITY, l = -INFINITY;
  int li = 0;
  if (r < rows) {
    const int t = (int)(r / m.hq), h = (int)(r - (int64_t)t * m.hq);
    li = merge_lse_index(m, t, h);
    la = m.acc_lse[li];
    lb = m.lse[li];
    const float mx = fmaxf(la, lb);
    if (mx != -INFINITY) l = mx + log1pf(__expf(-fabsf(la - lb)));
    const float wa = la == -INFINITY ? 0.f : __expf(la - l);
    const float wb = lb == -INFINITY ? 0.f : __expf(lb - l);
    f32x4* pa = reinterpret_cast<f32x4*>(m.acc_o + r * m.D + c);
    const f32x4 ob = *reinterpret_cast<const f32x4*>(m.o + r * m.D + c);
    *pa = *pa * wa + ob * wb;
  }
  __syncthreads();
  if (r < rows && c == 0) m.acc_lse[li] = l;
}

// The accumulator's final form: the sink joins the denominator (L' =
// log(e^L + e^sink), O' = e^(L - L') O), O rounded to bf16 [T][hq][D].
__global__ __launch_bounds__(256) void attn_merge_finish_kernel(MergeArgs m) {
  const int64_t rows = (int64_t)m.T * m.hq;
  const int64_t idx4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q4 = m.D / 4;
  const int64_t r = idx4 / q4;
  const int c = (int)(idx4 - r * q4) * 4;
  if (r >= rows) return;
  const int t = (int)(r / m.hq), h = (int)(r - (int64_t)t * m.hq);
  const int li = merge_lse_index(m, t, h);
  const float l = m.acc_lse[li];
  float lf = l, w = l == -INFINITY ? 0.f : 1.f;
  if (m.sink != nullptr) {
    const float s = m.sink[h];
    const float mx = fmaxf(l, s);
    lf = mx + log1pf(__expf(-fabsf(l - s)));
    w = l == -INFINITY ? 0.f : __expf(l - lf);
  }
  const f32x4 o = *reinterpret_cast<const f32x4*>(m.acc_o + r * m.D + c) * w;
  u32x2 pk;
  pk[0] = pack_bf16x2(o[0], o[1]);
  pk[1] = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<u32x2*>(m.out + r * m.D + c) = pk;
  if (c == 0) m.lse_out[li] = lf;
}

hipError_t attn_merge_launch(float* acc_o, float* acc_lse, const float* o, const float* lse, int B,
                             int S, int hq, int D, hipStream_t st) {
  MergeArgs m = {acc_o, acc_lse, o, lse, nullptr, nullptr, nullptr, B * S, S, hq, D};
  const int64_t items = (int64_t)B * S * hq * (D / 4);
  if (items == 0) return hipSuccess;
  ProfScope prof("attn_merge", st);
  hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t attn_merge_finish_launch(const float* acc_o, const float* acc_lse, const float* sink,
                                    void* out, float* lse, int B, int S, int hq, int D,
                                    hipStream_t st) {
  MergeArgs m = {const_cast<float*>(acc_o), const_cast<float*>(acc_lse), nullptr, nullptr, sink,
                 (__bf16*)out, lse, B * S, S, hq, D};
  const int64_t items = (int64_t)B * S * hq * (D / 4);
  if (items == 0) return hipSuccess;
  ProfScope prof("attn_merge_finish", st);
  hipLaunchKernelGGL(attn_merge_finish_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st,
                     m);
  return hipGetLastError();
}

hipError_t attn_fwd_launch(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128) return launch_fwd_t<128, 4, 1>(a, st);
  // a window narrower than 256 keys: 128-row work-groups (each walks the
  // union of its rows' windows, so 256 rows would multiply masked products;
  // the split partials do not depend on the rows per work-group)
  return fwd_block_rows(a.B, a.S, a.hq, D) == 256 && !narrow_window(a.causal, a.wl, a.wr)
             ? launch_fwd_t<64, 4, 2>(a, st)
             : launch_fwd_t<64, 4, 1>(a, st);
}

}  // namespace uly

// Attention backward of one Ulysses rank.
//
//   delta_i = sum_d dO_i,d O_i,d                         (attn_bwd_stats, stored negated)
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
// gradients are deterministic.  Their products run in fp16 on fp16 copies of
// q, k, v and dout * 2^e (made here, in the workspace; the power-of-two scale
// below keeps dout and dS inside fp16's range whatever the gradients'
// magnitude): P and dS are rounded to fp16's 11 significant bits instead of
// bf16's 8 before the dV, dK and dQ products, which keeps the gradients within
// the bf16-output tolerance even where attention is concentrated on few keys.
#include <climits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace uly {

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------- statistics, the copies' scales
//
// The products run in fp16, whose finite range is 2^-24 .. 65504: bf16
// gradients far below 1 (a loss averaged over many tokens) would fall into
// fp16's subnormals or flush to zero, and values beyond 65504 would
// saturate.  So each copy is an exact power-of-two scaling of its tensor:
// dout * 2^e, v * 2^c, q * 2^a, k * 2^b, with the integer exponents chosen on
// the device such that every scaled value that becomes an fp16 operand stays
// below 2^15 in magnitude:
//   |q| 2^a, |k| 2^b, |dout| 2^e, |v| 2^c     (the copies themselves), and
//   |dS_ij| 2^(e+c) = P_ij |dP_ij - delta_i| 2^(e+c)
//              <= (max_i |dout_i| max_j |v_j| + max_i |delta_i|) 2^(e+c)
// (Euclidean norms over the head dimension, Cauchy-Schwarz; 0 <= P <= 1).
// a and b take the largest such value; e and c share the headroom the dS
// bound leaves, each giving up half of what is missing.  All are clamped to
// |x| <= kScaleExpMax.  Then S_ij comes out 2^(a+b) times larger (the softmax
// scale absorbs it, so P is the very same), dP and dS 2^(e+c), dV 2^e, dK
// 2^(e+c+a), dQ 2^(e+c+b), until the epilogues remove the factors with
// v_ldexp_f32 (exact).  Each copy is checked element by element; elements
// that saturated or are inexact are counted.

constexpr float kF16Max = 65504.f;

// The fp16 copy of two values (saturating at +-65504), counting those that
// saturated (or are NaN) and those whose copy is not the value itself.
__device__ __forceinline__ u32 f16_copy2(float x0, float x1, int& sat, int& inexact) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const u32 h = pack_f16x2(clamp_f16(x0), clamp_f16(x1));
  const f16x2 hv = __builtin_bit_cast(f16x2, h);
  const bool s0 = !(fabsf(x0) <= kF16Max), s1 = !(fabsf(x1) <= kF16Max);
  sat += (int)s0 + (int)s1;
  inexact += (int)(!s0 && (float)hv[0] != x0) + (int)(!s1 && (float)hv[1] != x1);
  return h;
}

// Adds the wave's counts to the status words (only when one is nonzero).
__device__ __forceinline__ void add_counts(const AttnArgs& a, int sat, int inexact) {
  if (!__any(sat | inexact)) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sat += __shfl_xor(sat, off, 64);
    inexact += __shfl_xor(inexact, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    if (sat) atomicAdd(a.bwd_status + kCntSat, sat);
    if (inexact) atomicAdd(a.bwd_status + kCntInexact, inexact);
  }
}

constexpr int kStats = kStatFloats;  // per-block maxima (7 used)
enum { kMaxDoutNorm2, kMaxDout, kMaxDelta, kMaxVNorm2, kMaxV, kMaxQ, kMaxK };

// Per (row, head): delta = dO . O (bf16 O, fp32 sums; stored negated) and
// LSE * log2(e).  Per block, over its share of the rows, the maxima listed
// above: stat_part[block][kStats].  D/8 threads per row, one 16-byte chunk
// each; blocks stride over the rows.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_stats_kernel(AttnArgs a) {
  constexpr int TPR = D / 8, RPB = 256 / TPR;
  __shared__ float red[4][kStats];
  const int c = threadIdx.x % TPR;
  float m[kStats] = {};
  const int rows = a.T * a.hq;
  for (int r0 = blockIdx.x * RPB; r0 < rows; r0 += gridDim.x * RPB) {
    const int row = r0 + threadIdx.x / TPR;  // row = t * hq + h
    const bool valid = row < rows;
    const int t = row / a.hq, hh = row - t * a.hq;
    float acc = 0.f, n2 = 0.f;
    if (valid) {
      const int64_t src = row_of(a.mq, t) + (int64_t)hh * a.mq.head + 8 * c;
      const u32x4 x = *reinterpret_cast<const u32x4*>(a.dout + src);
      const u32x4 y = *reinterpret_cast<const u32x4*>(a.o + src);
      const u32x4 z = *reinterpret_cast<const u32x4*>(a.q + src);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
        acc += x0 * bf16_lo(y[w]) + x1 * bf16_hi(y[w]);
        n2 = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, n2));
        m[kMaxDout] = fmaxf(m[kMaxDout], fmaxf(fabsf(x0), fabsf(x1)));
        m[kMaxQ] = fmaxf(m[kMaxQ], fmaxf(fabsf(bf16_lo(z[w])), fabsf(bf16_hi(z[w]))));
      }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) {
      acc += __shfl_xor(acc, off, TPR);
      n2 += __shfl_xor(n2, off, TPR);
    }
    if (valid && c == 0) {
      const int idx = lse_index(a, t, hh);
      a.ndelta[idx] = -acc;
      const float l = a.lse[idx];
      a.lse2[idx] = l == -INFINITY ? INFINITY : l * kLog2e;  // rows with no key: P = 0
      m[kMaxDelta] = fmaxf(m[kMaxDelta], fabsf(acc));
      m[kMaxDoutNorm2] = fmaxf(m[kMaxDoutNorm2], n2);
    }
  }
  const int vrows = a.T * a.hkv;
  for (int r0 = blockIdx.x * RPB; r0 < vrows; r0 += gridDim.x * RPB) {
    const int row = r0 + threadIdx.x / TPR;  // row = t * hkv + g
    const bool valid = row < vrows;
    float n2 = 0.f;
    if (valid) {
      const int t = row / a.hkv, g = row - t * a.hkv;
      const int64_t src = row_of(a.mk, t) + (int64_t)g * a.mk.head + 8 * c;
      const u32x4 x = *reinterpret_cast<const u32x4*>(a.v + src);
      const u32x4 z = *reinterpret_cast<const u32x4*>(a.k + src);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
        n2 = __builtin_fmaf(x0, x0, __builtin_fmaf(x1, x1, n2));
        m[kMaxV] = fmaxf(m[kMaxV], fmaxf(fabsf(x0), fabsf(x1)));
        m[kMaxK] = fmaxf(m[kMaxK], fmaxf(fabsf(bf16_lo(z[w])), fabsf(bf16_hi(z[w]))));
      }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) n2 += __shfl_xor(n2, off, TPR);
    if (valid && c == 0) m[kMaxVNorm2] = fmaxf(m[kMaxVNorm2], n2);
  }
#pragma unroll
  for (int k = 0; k < kStats; ++k)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m[k] = fmaxf(m[k], __shfl_xor(m[k], off, 64));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < kStats; ++k) red[wave][k] = m[k];
  __syncthreads();
  if (threadIdx.x < kStats) {
    const int k = threadIdx.x;
    a.stat_part[kStats * blockIdx.x + k] = fmaxf(fmaxf(red[0][k], red[1][k]), fmaxf(red[2][k], red[3][k]));
  }
}

// The largest e with 2^e x < 2^15 for x = m 2^p (frexp, 0.5 <= m < 1):
// e = 15 - p.  x = 0 leaves the scale free (0 here); inf or NaN: the lowest.
__device__ __forceinline__ int exp_below_2p15(float x) {
  if (!(x <= 3.0e38f)) return -kScaleExpMax;
  if (x == 0.f) return 0;
  int p;
  frexpf(x, &p);
  return 15 - p;
}

__device__ __forceinline__ int clamp_exp(int e) { return min(max(e, -kScaleExpMax), kScaleExpMax); }

// One block: the maxima over the stats blocks, the four exponents, and zero
// counts.
__global__ __launch_bounds__(256) void attn_bwd_scale_kernel(AttnArgs a, int nparts) {
  __shared__ float red[4][kStats];
  float m[kStats] = {};
  for (int i = threadIdx.x; i < nparts; i += 256)
#pragma unroll
    for (int k = 0; k < kStats; ++k) m[k] = fmaxf(m[k], a.stat_part[kStats * i + k]);
#pragma unroll
  for (int k = 0; k < kStats; ++k)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m[k] = fmaxf(m[k], __shfl_xor(m[k], off, 64));
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < kStats; ++k) red[threadIdx.x >> 6][k] = m[k];
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < kStats; ++k) m[k] = fmaxf(fmaxf(red[0][k], red[1][k]), fmaxf(red[2][k], red[3][k]));
    // >= |dP - delta| for every pair
    const float bound = sqrtf(m[kMaxDoutNorm2]) * sqrtf(m[kMaxVNorm2]) + m[kMaxDelta];
    int e = exp_below_2p15(m[kMaxDout]), c = exp_below_2p15(m[kMaxV]);
    if (bound != 0.f) {
      const int room = exp_below_2p15(bound);  // e + c may not exceed it
      const int over = e + c - room;
      if (over > 0) {
        e -= (over + 1) / 2;
        c -= over / 2;
      }
    }
    e = clamp_exp(e);
    c = clamp_exp(c);
    a.bwd_status[kExpDout] = e;
    a.bwd_status[kExpV] = c;
    a.bwd_status[kExpQ] = clamp_exp(exp_below_2p15(m[kMaxQ]));
    a.bwd_status[kExpK] = clamp_exp(exp_below_2p15(m[kMaxK]));
    a.bwd_status[kCntSat] = 0;
    a.bwd_status[kCntInexact] = 0;
  }
}

// The fp16 copy of dout * 2^e for one 16-byte chunk per thread (D/8 threads
// per (row, head)), and delta scaled by 2^(e+c); `block` plays the role of
// the block index.  Rows T .. T + kPad - 1 of the copy are zero.
template <int D>
__device__ __forceinline__ void dout_block(const AttnArgs& a, int block, int e) {
  constexpr int TPR = D / 8;  // threads per row
  const int row = block * (256 / TPR) + threadIdx.x / TPR;  // row = t * hq + h
  const int c = threadIdx.x % TPR;
  const bool valid = row < a.T * a.hq;
  int sat = 0, inexact = 0;
  if (!valid && row < (a.T + kPad) * a.hq) {  // the zero rows after the last token
    const u32x4 z = {0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(a.do16 + (int64_t)row * D + 8 * c) = z;
  }
  if (valid) {
    const int t = row / a.hq, hh = row - t * a.hq;
    const int64_t src = row_of(a.mq, t) + (int64_t)hh * a.mq.head + 8 * c;
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.dout + src);
    u32x4 h;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      h[w] = f16_copy2(ldexpf(bf16_lo(x[w]), e), ldexpf(bf16_hi(x[w]), e), sat, inexact);
    *reinterpret_cast<u32x4*>(a.do16 + (int64_t)row * D + 8 * c) = h;
    if (c == 0) {  // delta joins dP = dO V, which carries 2^(e+c)
      const int idx = lse_index(a, t, hh);
      a.ndelta[idx] = ldexpf(a.ndelta[idx], e + a.bwd_status[kExpV]);
    }
  }
  add_counts(a, sat, inexact);
}

// The fp16 copy times 2^ex, in the head layout [T][H][D], of a bf16 tensor
// laid out as `m` says: exact for every scaled value with 2^-17 <= |x| <=
// 65504 (fp16 keeps 11 significant bits, bf16 8); larger magnitudes saturate,
// smaller ones round to a multiple of 2^-24 (both counted).  One 16-byte
// chunk per thread; hd8 = H*D/8.  Elements n .. n_pad - 1 (the kPad rows
// after the last token) are zero.
__device__ __forceinline__ void f16_block(const AttnArgs& a, const __bf16* src, const RowMap& m,
                                          FastDiv hd8, FastDiv d8, _Float16* dst, int64_t n,
                                          int64_t n_pad, int block, int ex) {
  const int64_t i = ((int64_t)block * 256 + threadIdx.x) * 8;
  int sat = 0, inexact = 0;
  if (i >= n && i < n_pad) {
    const u32x4 z = {0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(dst + i) = z;
  }
  if (i < n) {
    const u32 chunk = (u32)(i >> 3);
    const u32 t = fdiv(chunk, hd8), rest = chunk - t * hd8.d;
    const u32 hh = fdiv(rest, d8), c = rest - hh * d8.d;
    const u32x4 x = *reinterpret_cast<const u32x4*>(src + row_of(m, (int)t) + (int64_t)hh * m.head + 8 * c);
    u32x4 h;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      h[w] = f16_copy2(ldexpf(bf16_lo(x[w]), ex), ldexpf(bf16_hi(x[w]), ex), sat, inexact);
    *reinterpret_cast<u32x4*>(dst + i) = h;
  }
  add_counts(a, sat, inexact);
}

// The backward's copies in one launch: blocks [0, nb_pre) make the fp16
// dout * 2^e and scale delta (dout_block); the next ones make the fp16
// copies of q * 2^a, then k * 2^b, then v * 2^c (f16_block).
struct PrepArgs {
  int nb_pre, nb_q, nb_kv;
  FastDiv d8, q8, k8;
  int64_t nq, pq, nkv, pkv;
};

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(AttnArgs a, PrepArgs p) {
  int b = blockIdx.x;
  if (b < p.nb_pre) {
    dout_block<D>(a, b, a.bwd_status[kExpDout]);
    return;
  }
  b -= p.nb_pre;
  if (b < p.nb_q) {
    f16_block(a, a.q, a.mq, p.q8, p.d8, a.q16, p.nq, p.pq, b, a.bwd_status[kExpQ]);
    return;
  }
  b -= p.nb_q;
  if (b < p.nb_kv) {
    f16_block(a, a.k, a.mk, p.k8, p.d8, a.k16, p.nkv, p.pkv, b, a.bwd_status[kExpK]);
    return;
  }
  f16_block(a, a.v, a.mk, p.k8, p.d8, a.v16, p.nkv, p.pkv, b - p.nb_kv, a.bwd_status[kExpV]);
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

// SINK: the rows' sum of P dP is accumulated too (it feeds dsink).
// a compile-time flag carried by a generic lambda's argument type
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int D, int NW, int SINK>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_kernel(AttnArgs a) {
  // S from the copies q 2^a and k 2^b: the scale absorbs 2^-(a+b), exactly
  a.scale_log2 = ldexpf(a.scale_log2, -(a.bwd_status[kExpQ] + a.bwd_status[kExpK]));
  constexpr int BM = 32 * NW, NB = D / 32, KS = D / 16;
  constexpr int TILE = kBK * D * 2;
  constexpr int STAGE = 2 * TILE;  // K, then V
  // distinct LDS objects per stage, each access naming one statically: the
  // next tile's direct-to-LDS loads then provably miss the current tile's
  // reads, and those reads do not wait for them
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];

  int qt, h;
  if (!decode_qtile(a, qt, h)) return;
  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  load_row_frags<D>(qf, a.q16 + ((int64_t)qrow * a.hq + h) * D, qvalid, lane);
  load_row_frags<D>(dof, a.do16 + ((int64_t)qrow * a.hq + h) * D, qvalid, lane);
  float lse2 = INFINITY, dlt = 0.f;  // invalid rows: P = 0
  if (qvalid) {
    lse2 = a.lse2[lse_index(a, qrow, h)];
    dlt = -a.ndelta[lse_index(a, qrow, h)];
  }

  f32x16 dqacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[nb][e] = 0.f;
  constexpr bool want_pdp = SINK != 0;
  float pdp = 0.f;
  const f32x16 zero = {};

  const _Float16* kbase = a.k16 + (int64_t)g * D;
  const _Float16* vbase = a.v16 + (int64_t)g * D;
  const int ld = a.hkv * D;
  // K and V tiles share row stride and swizzle: one set of per-lane offsets;
  // rows up to wg_hi + 63 < T + kPad exist (zero past the last token)
  const BufTileLoader<D, kBK, NW> offs(ld, wave, lane);
  SwzOffsets<D> so(lane);
  // this split's share of the key tiles
  int it_lo, it_hi;
  split_range((wg_hi - wg_lo + kBK - 1) / kBK, blockIdx.y, a.nsplit, it_lo, it_hi);
  if (it_lo < it_hi) {
    const int64_t r0 = (int64_t)(wg_lo + it_lo * kBK) * ld;
    offs.load(stage0, kbase + r0, kBK, wave);
    offs.load(stage0 + TILE, vbase + r0, kBK, wave);
  }

  // the products and softmax of one staged key tile (FULL: every key of
  // the tile is visible to every row of the work-group, no mask)
  auto body = [&](auto full_c, int k0, const char* kt, const char* vt) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_c)::value;
    // this lane's visible keys relative to its first key slot of the tile
    // (slot e of block mb holds key offset 32 mb + 8 (e / 4) + e % 4)
    const int vis_lo = klo - (k0 + 4 * hf), vis_hi = khi - (k0 + 4 * hf);
    // one 32-key block at a time keeps two accumulators live, not four
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        sacc = mfma32h(so.nat_at(kt, 32 * mb, s), qf[s], s == 0 ? zero : sacc);
        dpacc = mfma32h(so.nat_at(vt, 32 * mb, s), dof[s], s == 0 ? zero : dpacc);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.scale_log2, -lse2));
        if constexpr (!FULL) {
          const int c = 32 * mb + 8 * (e >> 2) + (e & 3);
          p = (c >= vis_lo && c < vis_hi) ? p : 0.f;
        }
        if (want_pdp) pdp = __builtin_fmaf(p, dpacc[e], pdp);
        sacc[e] = p * (dpacc[e] - dlt);  // dS^T
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const bf16x8 df = acc_frag_h(sacc, ii);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          dqacc[nb] = mfma32h(so.tr_at(kt, 32 * mb + 16 * ii, nb), df, dqacc[nb]);
      }
    }
    // keep 4 operand reads in flight ahead of the products (the default
    // schedule issues each read just before its product and waits out the
    // LDS latency every time): per 32-key block, S and dP (2 KS products,
    // one read each), then dQ (2 NB products, two reads each)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      constexpr int PF = 4;
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < 2 * KS - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < 2 * NB - PF / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, PF / 2, 0);
    }
  };
  // one key tile: `cur` holds tile `it`, tile it+1 goes to `nxt`
  auto step = [&](int it, const char* cur, char* nxt) __attribute__((always_inline)) {
    const int k0 = wg_lo + it * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < it_hi) {
      const int64_t r0 = (int64_t)(k0 + kBK) * ld;
      offs.load(nxt, kbase + r0, kBK, wave);
      offs.load(nxt + TILE, vbase + r0, kBK, wave);
    }
    const char* kt = cur;
    const char* vt = cur + TILE;
    // one set of read offsets for both stages (two hoisted sets would not
    // fit the register budget next to the accumulators)
    so.refresh();
    // a fully visible tile (wave-uniform) takes a copy of the body without
    // the per-element mask; each copy is one scheduling region
    if (__builtin_amdgcn_readfirstlane((int)(k0 >= full_lo && k0 + kBK <= full_hi)))
      body(BoolC<true>{}, k0, kt, vt);
    else
      body(BoolC<false>{}, k0, kt, vt);
  };
  for (int it = it_lo; it < it_hi; it += 2) {
    step(it, stage0, stage1);
    if (it + 1 < it_hi) step(it + 1, stage1, stage0);
  }

  // P dP carries 2^(e+c), dQ 2^(e+c+b) (removed here, exactly)
  const int edp = a.bwd_status[kExpDout] + a.bwd_status[kExpV], es = edp + a.bwd_status[kExpK];
  pdp = ldexpf(halves_sum(pdp), -edp);
  if (a.nsplit > 1) {  // fp32 partials (still scaled by 2^e), summed by dq_reduce_kernel
    if (qvalid && want_pdp && hf == 0)
      a.part_pdp[(int64_t)blockIdx.y * a.T * a.hq + lse_index(a, qrow, h)] = pdp;
    if (qvalid) {
      float* row = a.part + ((int64_t)blockIdx.y * a.T * a.hq + (int64_t)qrow * a.hq + h) * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 w = {dqacc[nb][4 * i + 0], dqacc[nb][4 * i + 1], dqacc[nb][4 * i + 2],
                           dqacc[nb][4 * i + 3]};
          *reinterpret_cast<f32x4*>(row + 32 * nb + 8 * i + 4 * hf) = w;
        }
    }
    return;
  }
  if (qvalid && want_pdp && hf == 0) a.pdp[lse_index(a, qrow, h)] = pdp;
  if (qvalid) {
    __bf16* row = a.out + row_of(a.mq, qrow) + (int64_t)h * a.mq.head;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(ldexpf(dqacc[nb][4 * i + 0] * a.scale, -es),
                           ldexpf(dqacc[nb][4 * i + 1] * a.scale, -es));
        w[1] = pack_bf16x2(ldexpf(dqacc[nb][4 * i + 2] * a.scale, -es),
                           ldexpf(dqacc[nb][4 * i + 3] * a.scale, -es));
        *reinterpret_cast<u32x2*>(row + 32 * nb + 8 * i + 4 * hf) = w;
      }
  }
}

// Explicit instantiations: with the two launches of the launcher's if/else,
// hipcc emitted the host stub of only one of them.
template __global__ void attn_bwd_dq_kernel<128, 4, 0>(AttnArgs);
template __global__ void attn_bwd_dq_kernel<128, 4, 1>(AttnArgs);
template __global__ void attn_bwd_dq_kernel<64, 4, 0>(AttnArgs);
template __global__ void attn_bwd_dq_kernel<64, 4, 1>(AttnArgs);

// dQ = scale * 2^-(e+c+b) * the sum of the split partials (fixed order), to
// bf16; the same sum for the rows' P dP (its parts already unscaled).
template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(AttnArgs a, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i < n) {
    const int es = a.bwd_status[kExpDout] + a.bwd_status[kExpV] + a.bwd_status[kExpK];
    f32x4 q = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < a.nsplit; ++s) q += *reinterpret_cast<const f32x4*>(a.part + s * n + i);
    u32x2 w;
    w[0] = pack_bf16x2(ldexpf(q[0] * a.scale, -es), ldexpf(q[1] * a.scale, -es));
    w[1] = pack_bf16x2(ldexpf(q[2] * a.scale, -es), ldexpf(q[3] * a.scale, -es));
    const int rr = (int)(i / D), t = rr / a.hq, h = rr - t * a.hq;  // row rr = t * hq + h
    *reinterpret_cast<u32x2*>(a.out + row_of(a.mq, t) + (int64_t)h * a.mq.head + (i - (int64_t)rr * D)) = w;
  }
  const int64_t rows = (int64_t)a.T * a.hq;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (a.sink != nullptr && r < rows) {
    float p = 0.f;
    for (int s = 0; s < a.nsplit; ++s) p += a.part_pdp[s * rows + r];
    a.pdp[r] = p;
  }
}

// ------------------------------------------------------------------ launches

template <int D, int NW>
static hipError_t launch_bwd_t(const AttnArgs& args, hipStream_t st) {
  AttnArgs a = args;
  {
    ProfScope prof("attn_bwd_stats", st);
    constexpr int rpb = 256 / (D / 8);
    const long need = ((long)a.T * (a.hq > a.hkv ? a.hq : a.hkv) + rpb - 1) / rpb;
    const int nb = (int)(need < kStatBlocks ? (need > 0 ? need : 1) : kStatBlocks);
    hipLaunchKernelGGL(attn_bwd_stats_kernel<D>, dim3(nb), dim3(256), 0, st, a);
    hipLaunchKernelGGL(attn_bwd_scale_kernel, dim3(1), dim3(256), 0, st, a, nb);
  }
  {
    ProfScope prof("attn_bwd_prep", st);
    PrepArgs p;
    const int rows = (a.T + kPad) * a.hq, rpb = 256 / (D / 8);
    p.nq = (int64_t)a.T * a.hq * D;
    p.nkv = (int64_t)a.T * a.hkv * D;
    p.pq = p.nq + (int64_t)kPad * a.hq * D;
    p.pkv = p.nkv + (int64_t)kPad * a.hkv * D;
    p.d8 = make_fastdiv(D / 8);
    p.q8 = make_fastdiv(a.hq * D / 8);
    p.k8 = make_fastdiv(a.hkv * D / 8);
    p.nb_pre = (rows + rpb - 1) / rpb;
    p.nb_q = (int)((p.pq / 8 + 255) / 256);
    p.nb_kv = (int)((p.pkv / 8 + 255) / 256);
    hipLaunchKernelGGL(attn_bwd_prep_kernel<D>, dim3(p.nb_pre + p.nb_q + 2 * p.nb_kv), dim3(256), 0, st,
                       a, p);
  }
  dkdv_launch(a, D, st);
  {
    AttnArgs b = a;
    b.n_tiles = (a.T + 32 * NW - 1) / (32 * NW);
    const int groups = b.n_tiles * a.hkv;
    const int blocks = ((groups + kXcds - 1) / kXcds) * kXcds * a.G;
    b.nsplit = qtile_splits(a.B, a.S, a.hq, D, uneven_layer(a.causal, a.wl, a.wr));
    {
      ProfScope prof("attn_bwd_dq", st);
      if (a.sink != nullptr)
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NW, 1>), dim3(blocks, b.nsplit), dim3(NW * 64), 0, st, b);
      else
        hipLaunchKernelGGL((attn_bwd_dq_kernel<D, NW, 0>), dim3(blocks, b.nsplit), dim3(NW * 64), 0, st, b);
    }
    if (b.nsplit > 1) {
      ProfScope prof("attn_bwd_dq_reduce", st);
      const int64_t n = (int64_t)a.T * a.hq * D;
      const int64_t items = n / 4 > (int64_t)a.T * a.hq ? n / 4 : (int64_t)a.T * a.hq;
      hipLaunchKernelGGL(dq_reduce_kernel<D>, dim3((items + 255) / 256), dim3(256), 0, st, b, n);
    }
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

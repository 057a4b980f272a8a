// Attention backward of one Ulysses rank: the key-stationary dK/dV kernel.
// (The delta pre-pass, the dQ kernel and dsink are in attn_bwd.hip.)
#include <climits>

#include "attn_common.hpp"
#include "launch.hpp"

namespace uly {

// ------------------------------------------------------------------ dK, dV
//
// Products in fp16 on the fp16 copies the pre-pass makes (see attn_bwd.hip).
// One work-group = KG key groups of 32 keys of one KV head, two waves per
// group (2 KG waves, two per SIMD).  The work-group's K and V rows are staged
// once in LDS (swizzled natural tiles) and read as B operands when needed.
// The work-group walks every query tile (64 rows) of every query head of the
// group: Q and dO tiles plus their LSE*log2(e) and -delta rows arrive by
// global_load_lds, double-buffered in two distinct LDS arrays (the loop is
// unrolled by two, so reads of one stage are provably disjoint from the loads
// into the other).  Of each tile, the two waves of a key group take one
// 32-query block each (S = Q K^T, dP = dO V^T from the natural operands, then
// dV += P^T dO and dK += dS^T Q through the transposing reads), so a SIMD
// runs two independent waves whose products and softmax overlap.  Each wave
// accumulates its block's share of its keys' dK and dV; the two shares are
// added once, through LDS, after the last tile.  At D = 64 each wave also
// keeps its keys' K and V operands in registers (32 VGPRs, read from LDS once
// per item), which the D = 128 kernel's register budget does not allow.

// K and V operands in registers (else read from LDS for every tile)
template <int D>
constexpr bool kKvInRegs = D <= 64;

template <int D, int KG>
struct DkdvSmem {
  static constexpr int kTile = kBK * D * 2;
  static constexpr int kStage = 2 * kTile + 2 * kBK * 4;  // Q, dO, LSE*log2e, delta
  static constexpr int kKV = 32 * KG * D * 2;              // K or V rows of the work-group
  // the second block's dK (in the K/V area) and dV (half the key groups in
  // each stage) for the final sum
  static constexpr int kRed = (D / 32) * 16 * 64 * 4;      // one wave's dK or dV, fp32
  static_assert(KG * kRed <= 2 * kKV && (KG / 2) * kRed <= kStage, "final sum fits the LDS arrays");
};

// One 32-query block of a staged tile for this wave's 32 keys.  `so` holds
// the per-lane read offsets of the wave's block rows in a stage tile, `kvo`
// those of its key rows in the K/V area.
template <int D, int KG>
__device__ __forceinline__ void dkdv_tile(const AttnArgs& a, const char* buf, const char* kvs,
                                          SwzOffsets<D>& so, int (&kvo)[D / 16],
                                          const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                          f32x16 (&dkacc)[D / 32], f32x16 (&dvacc)[D / 32],
                                          int qa, int qb, int full_lo, int full_hi, int qlo, int qhi,
                                          int lane) {
  typedef DkdvSmem<D, KG> SM;
  constexpr int NB = D / 32, KS = D / 16;
  const int hf = lane >> 5;
  const char* qs = buf;
  const char* dos = buf + SM::kTile;
  const float* lsw = reinterpret_cast<const float*>(buf + 2 * SM::kTile) + 32 * qb + 4 * hf;
  const char* ks = kvs;
  const char* vs = kvs + SM::kKV;
  const f32x16 zero = {};

  // visible queries of this lane's key, as offsets from the first row this
  // lane holds (row 8 i + 4 hf + j of the block holds value 4 i + j), so each
  // test compares with a constant; a fully visible tile opens them
  const bool full = qa >= full_lo && qa + kBK <= full_hi;
  const int rel = qa + 32 * qb + 4 * hf;
  const int mlo = full ? -(1 << 30) : qlo - rel, mhi = full ? (1 << 30) : qhi - rel;

  // per-lane read offsets, opaque here so that each read forms its address
  // from them (plus an immediate) instead of the compiler keeping one
  // register per distinct address across the loop
  so.refresh();
  if constexpr (!kKvInRegs<D>) {
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(kvo[s]));
  }
  auto k_at = [&](int s) {
    if constexpr (kKvInRegs<D>) return kf[s];
    else return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks + kvo[s]));
  };
  auto v_at = [&](int s) {
    if constexpr (kKvInRegs<D>) return vf[s];
    else return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vs + kvo[s]));
  };

  // dP - delta: the sums start from the rows' -delta (value 4 i + j of a lane
  // belongs to row 8 i + j of its first row)
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(lsw + kBK + 8 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) dinit[4 * i + j] = d4[j];
  }
  f32x16 sacc, dpacc;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    sacc = mfma32h(so.nat_at(qs, 0, s), k_at(s), s == 0 ? zero : sacc);
    dpacc = mfma32h(so.nat_at(dos, 0, s), v_at(s), s == 0 ? dinit : dpacc);
  }
  // a fully visible tile (wave-uniform) skips the per-element mask
  if (__builtin_amdgcn_readfirstlane((int)full)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsw + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * i + j], a.scale_log2, -l4[j]));
        sacc[4 * i + j] = p;
        dpacc[4 * i + j] *= p;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsw + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * i + j], a.scale_log2, -l4[j]));
        const int rc = 8 * i + j;
        p = (rc >= mlo && rc < mhi) ? p : 0.f;
        sacc[4 * i + j] = p;
        dpacc[4 * i + j] *= p;
      }
    }
  }
  bf16x8 pf[2], df[2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii) {
    pf[ii] = acc_frag_h(sacc, ii);
    df[ii] = acc_frag_h(dpacc, ii);
  }
  // dV += P^T dO, dK += dS^T Q (contraction over the block's 32 queries)
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      dvacc[nb] = mfma32h(pf[ii], so.tr_at(dos, 16 * ii, nb), dvacc[nb]);
      dkacc[nb] = mfma32h(df[ii], so.tr_at(qs, 16 * ii, nb), dkacc[nb]);
    }
}

// (query tile, head) iterations a key tile of BN keys visits (at least one
// unit: see the balanced schedule in attn_common.hpp)
template <int BN>
__device__ __forceinline__ int dkdv_tile_units(const AttnArgs& a, int kt) {
  const int k0 = kt * BN, kl = min(k0 + BN, a.T) - 1;
  int lo, hi, x, y;
  query_interval(a, k0, lo, x);
  query_interval(a, kl, y, hi);
  return max(a.G * ((hi - lo + kBK - 1) / kBK), 1);
}

// BAL: the balanced schedule of small grids (a 1-D grid of bal_W
// work-groups, each walking its share of the (key tile, KV head) items);
// otherwise one item per work-group, its iterations split over blockIdx.y.
template <int D, int KG, bool BAL>
__global__ __launch_bounds__(KG * 128) void attn_bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NW = 2 * KG, BN = 32 * KG, NB = D / 32;
  // S from the copies q 2^a and k 2^b: the scale absorbs 2^-(a+b), exactly
  a.scale_log2 = ldexpf(a.scale_log2, -(a.bwd_status[kExpQ] + a.bwd_status[kExpK]));
  static_assert(NW >= 2, "two waves stage the per-row statistics");
  typedef DkdvSmem<D, KG> SM;
  __shared__ __attribute__((aligned(1024))) char kvs[2 * SM::kKV];
  __shared__ __attribute__((aligned(1024))) char st0[SM::kStage];
  __shared__ __attribute__((aligned(1024))) char st1[SM::kStage];

  const int lane = threadIdx.x & 63, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave % KG, qb = wave / KG;  // key group, query block
  const int ld = a.hq * D;
  // Q and dO tiles share row stride and swizzle: one set of per-lane offsets
  const TileOffsets<D, kBK, NW> offs(ld, wave, lane);
  // LDS read offsets: this wave's key rows in the K/V area, and its block's
  // swizzled rows of a stage tile (the swizzle repeats every 16 rows)
  SwzOffsets<D> so(lane);
  int kvo[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kvo[s] = 32 * kg * 2 * D + so.nat[s];
    so.nat[s] += 32 * qb * 2 * D;
  }
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) {
    so.tr[nb][0] += 32 * qb * 2 * D;
    so.tr[nb][1] += 32 * qb * 2 * D;
  }

  // Key tile kt of KV head g, iterations [seg_lo, seg_hi) of its walk (BAL),
  // into part slot `slot` (BAL, slot >= 0) or finished.
  auto item = [&](int kt, int g, int seg_lo, int seg_hi, int slot) __attribute__((always_inline)) {
  const int k0 = kt * BN;
  const int krow = k0 + 32 * kg + (lane & 31);
  const bool kvalid = krow < a.T;

  int qlo = 0, qhi = 0;
  if (kvalid) query_interval(a, krow, qlo, qhi);
  const int k_last = min(k0 + BN, a.T) - 1;
  int wg_lo, wg_hi, full_lo, full_hi;
  query_interval(a, k0, wg_lo, full_hi);
  query_interval(a, k_last, full_lo, wg_hi);

  // the work-group's K and V rows, once
  tile_load_lds<D, BN, NW>(kvs, a.k16 + (int64_t)g * D, a.hkv * D, k0, a.T, wave, lane);
  tile_load_lds<D, BN, NW>(kvs + SM::kKV, a.v16 + (int64_t)g * D, a.hkv * D, k0, a.T, wave, lane);

  f32x16 dkacc[NB], dvacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkacc[nb][e] = 0.f;
      dvacc[nb][e] = 0.f;
    }

  const int nq = (wg_hi - wg_lo + kBK - 1) / kBK;  // query tiles per head
  const int n_iter = nq * a.G;
  // Tiles are walked last first, the group's heads inner: every work-group of
  // a KV head starts on the same (last) query tile, so the work-groups that
  // share an XCD (neighbouring key tiles) stream the same Q/dO tiles at about
  // the same time and share them through its L2.  (Starting each at its own
  // first visible tile, the S=131072 causal kernel fetched 115 GB a launch
  // from beyond L2.)
  int nh = 0, nt = 0;  // (head in the group, tile counted from the last) of the next tile to issue
  auto issue = [&](char* buf) {
    const int qa = wg_lo + (nq - 1 - nt) * kBK, h = g * a.G + nh;
    const int64_t row0 = (int64_t)qa * a.hq + h;  // rows up to wg_hi + 63 < T + kPad exist
    offs.load(buf, a.q16 + row0 * D, wave);
    offs.load(buf + SM::kTile, a.do16 + row0 * D, wave);
    if (wave < 2) {
      const int idx = lse_index(a, min(qa + lane, a.T - 1), h);
      const float* src = wave == 0 ? a.lse2 + idx : a.ndelta + idx;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + 2 * SM::kTile + wave * kBK * 4), 4, 0, 0);
    }
    if (++nh == a.G) {
      nh = 0;
      ++nt;
    }
    return qa;
  };
  // K/V operands in registers: read once the work-group's K/V rows have
  // landed (after the loop's first barrier)
  bf16x8 kf[D / 16], vf[D / 16];
  auto read_kv = [&]() {
    if constexpr (kKvInRegs<D>) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        kf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kvs + kvo[s]));
        vf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kvs + SM::kKV + kvo[s]));
      }
    }
  };
  auto compute = [&](const char* buf, int qa) {
    dkdv_tile<D, KG>(a, buf, kvs, so, kvo, kf, vf, dkacc, dvacc, qa, qb, full_lo, full_hi, qlo, qhi,
                     lane);
  };

  // this split's (or segment's) share of the (query tile, head) iterations
  int it_lo, it_hi;
  if constexpr (BAL) {
    it_lo = seg_lo;
    it_hi = min(seg_hi, n_iter);
  } else {
    split_range(n_iter, blockIdx.y, a.nsplit, it_lo, it_hi);
  }
  if (it_lo < it_hi) {
    nt = it_lo / a.G;
    nh = it_lo - nt * a.G;
  }
  int qa0 = it_lo < it_hi ? issue(st0) : 0, qa1 = 0;
  for (int it = it_lo; it < it_hi; it += 2) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile `it` have landed
    __syncthreads();                // everyone's have, and stage 1 is free
    if (it + 1 < it_hi) qa1 = issue(st1);
    if (it == it_lo) read_kv();
    compute(st0, qa0);
    if (it + 1 < it_hi) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (it + 2 < it_hi) qa0 = issue(st0);
      compute(st1, qa1);
    }
  }

  // the second block's shares join the first's: one lane-major fp32 slot per
  // (key group, column block, value); dK in the K/V area, dV in the stages
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is past its last tile's reads
  float* red_k = reinterpret_cast<float*>(kvs) + kg * (SM::kRed / 4);
  float* red_v = reinterpret_cast<float*>(kg < KG / 2 ? st0 : st1) + (kg % (KG / 2)) * (SM::kRed / 4);
  if (qb == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red_k[(nb * 16 + e) * 64 + lane] = dkacc[nb][e];
        red_v[(nb * 16 + e) * 64 + lane] = dvacc[nb][e];
      }
  }
  __syncthreads();
  if (qb == 1) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dkacc[nb][e] += red_k[(nb * 16 + e) * 64 + lane];
      dvacc[nb][e] += red_v[(nb * 16 + e) * 64 + lane];
    }

  // dK, dV: lane holds column d = 32 nb + l % 32 of key rows 8 i + 4 hf + j
  if (BAL && slot >= 0) {  // this part, as accumulated: slot [2][BN][D] (dK, then dV)
    float* sk = a.part + (int64_t)slot * 2 * BN * D;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int kr = 32 * kg + 8 * (e >> 2) + 4 * hf + (e & 3);
      const int64_t off = (int64_t)kr * D + (lane & 31);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sk[off + 32 * nb] = dkacc[nb][e];
        sk[BN * D + off + 32 * nb] = dvacc[nb][e];
      }
    }
    return;
  }
  // dV carries 2^e, dK 2^(e+c+a) (removed here, exactly)
  const int ev = a.bwd_status[kExpDout], es = ev + a.bwd_status[kExpV] + a.bwd_status[kExpQ];
  const int64_t plane = (int64_t)a.T * a.hkv * D;
  float* pk = a.part + blockIdx.y * plane;
  float* pv = a.part + (a.nsplit + blockIdx.y) * plane;
  // one row offset per key, shared by the NB column blocks
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int key = k0 + 32 * kg + 8 * (e >> 2) + 4 * hf + (e & 3);
    if (key >= a.T) continue;
    const int col = lane & 31;
    if (!BAL && a.nsplit > 1) {
      const int64_t off = ((int64_t)key * a.hkv + g) * D + col;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        pk[off + 32 * nb] = dkacc[nb][e];
        pv[off + 32 * nb] = dvacc[nb][e];
      }
      continue;
    }
    const int64_t off = row_of(a.mk, key) + (int64_t)g * a.mk.head + col;
    if (a.dkv_f32) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        reinterpret_cast<float*>(a.dk)[off + 32 * nb] = ldexpf(dkacc[nb][e] * a.scale, -es);
        reinterpret_cast<float*>(a.dv)[off + 32 * nb] = ldexpf(dvacc[nb][e], -ev);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        a.dk[off + 32 * nb] = (__bf16)ldexpf(dkacc[nb][e] * a.scale, -es);
        a.dv[off + 32 * nb] = (__bf16)ldexpf(dvacc[nb][e], -ev);
      }
    }
  }
  };

  if constexpr (BAL) {
    __shared__ int pre[kBalMaxTiles + 1];
    bal_prefix(pre, a.n_tiles, [&](int t) { return dkdv_tile_units<BN>(a, t); });
    if (blockIdx.x == 0)
      for (int t = threadIdx.x; t <= a.n_tiles; t += blockDim.x) a.bal_prefix[t] = pre[t];
    bal_walk(pre, a.n_tiles, a.hkv, a.bal_W, item);
  } else {
    // Unsplit (large) grids: key tiles of one KV head in bands per XCD, so
    // neighbouring key tiles, which read mostly the same Q/dO tiles at about
    // the same time, share an L2 (measured 4 % on a 131072-token causal head;
    // on small split grids the plain order is faster).
    int L = (int)blockIdx.x, g, kt;
    if (a.nsplit == 1) {
      L = xcd_band_item(L, a.n_tiles * a.hkv, 32);
      if (L < 0) return;
      g = L / a.n_tiles;
      kt = L - g * a.n_tiles;
    } else {
      if (L >= a.n_tiles * a.hkv) return;
      kt = L / a.hkv;
      g = L - kt * a.hkv;
    }
    item(kt, g, 0, 0, -1);
  }
}

// dK = scale * 2^-(e+c+a) * k and dV = 2^-e * v (the sums of an item's
// parts, which carry those factors from the copies' scales), four
// consecutive columns at element offset `off`, to bf16 (or fp32).
__device__ __forceinline__ void store_dkdv4(const AttnArgs& a, int64_t off, f32x4 k, f32x4 v) {
  const int ev = a.bwd_status[kExpDout], es = ev + a.bwd_status[kExpV] + a.bwd_status[kExpQ];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    k[c] = ldexpf(k[c] * a.scale, -es);
    v[c] = ldexpf(v[c], -ev);
  }
  if (a.dkv_f32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dk) + off) = k;
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dv) + off) = v;
    return;
  }
  u32x2 wk, wv;
  wk[0] = pack_bf16x2(k[0], k[1]);
  wk[1] = pack_bf16x2(k[2], k[3]);
  wv[0] = pack_bf16x2(v[0], v[1]);
  wv[1] = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<u32x2*>(a.dk + off) = wk;
  *reinterpret_cast<u32x2*>(a.dv + off) = wv;
}

// dK = scale * sum of the split partials, dV = sum (fixed order), to bf16
// (or fp32).
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(AttnArgs a, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 k = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.nsplit; ++s) {
    k += *reinterpret_cast<const f32x4*>(a.part + s * n + i);
    v += *reinterpret_cast<const f32x4*>(a.part + (a.nsplit + s) * n + i);
  }
  const int rr = (int)(i / D), t = rr / a.hkv, g = rr - t * a.hkv;  // row rr = t * hkv + g
  const int64_t off = row_of(a.mk, t) + (int64_t)g * a.mk.head + (i - (int64_t)rr * D);
  store_dkdv4(a, off, k, v);
}

// dK = scale * the sum of the parts of a balanced schedule's items, dV = the
// sum, in work-group order (rows of items finished in place are skipped).
template <int D, int BN>
__global__ __launch_bounds__(256) void dkdv_reduce_bal_kernel(AttnArgs a, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const int rr = (int)(i / D), t = rr / a.hkv, g = rr - t * a.hkv;  // row rr = t * hkv + g
  const int c = (int)(i - (int64_t)rr * D);
  const int kt = t / BN, lr = t - kt * BN;
  const BalItem it(a.bal_prefix, a.n_tiles, kt, g, a.hkv, a.bal_W);
  if (it.la == it.lb) return;
  f32x4 k = {0.f, 0.f, 0.f, 0.f}, v = {0.f, 0.f, 0.f, 0.f};
  for (int lam = it.la; lam <= it.lb; ++lam) {
    if (!it.holds(lam)) continue;
    const float* p = a.part + (int64_t)it.slot(lam) * 2 * BN * D + (int64_t)lr * D + c;
    k += *reinterpret_cast<const f32x4*>(p);
    v += *reinterpret_cast<const f32x4*>(p + BN * D);
  }
  const int64_t off = row_of(a.mk, t) + (int64_t)g * a.mk.head + c;
  store_dkdv4(a, off, k, v);
}

// Explicit instantiations: with two launches of one kernel template in an
// if/else, hipcc has emitted the host stub of only one of them.
template __global__ void attn_bwd_dkdv_kernel<128, 4, true>(AttnArgs);
template __global__ void attn_bwd_dkdv_kernel<128, 4, false>(AttnArgs);
template __global__ void attn_bwd_dkdv_kernel<64, 4, true>(AttnArgs);
template __global__ void attn_bwd_dkdv_kernel<64, 4, false>(AttnArgs);

static_assert(kBalMaxTiles == kBalMaxTilesHost, "host and device agree on the balanced tile cap");

template <int D, int KG>
static void launch_dkdv_t(const AttnArgs& args, hipStream_t st) {
  AttnArgs b = args;
  b.n_tiles = (b.T + 32 * KG - 1) / (32 * KG);
  // under a window narrower than 256 keys every key tile walks about the same
  // few query tiles: the grid needs neither the balanced schedule nor splits
  // (so no reduce launch)
  const bool narrow = narrow_window(b.causal, b.wl, b.wr);
  if (narrow) b.bal_W = 0;
  if (b.bal_W > 0) {  // balanced schedule: parts in 2 bal_W slots, then their sum
    {
      ProfScope prof("attn_bwd_dkdv", st);
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, KG, true>), dim3(b.bal_W), dim3(KG * 128), 0, st, b);
    }
    ProfScope prof("attn_bwd_dkdv_reduce", st);
    const int64_t n = (int64_t)b.T * b.hkv * D;
    hipLaunchKernelGGL((dkdv_reduce_bal_kernel<D, 32 * KG>), dim3((n / 4 + 255) / 256), dim3(256), 0, st, b, n);
    return;
  }
  b.nsplit = dkdv_splits(b.B, b.S, b.hkv, D, uneven_layer(b.causal, b.wl, b.wr) && !narrow);
  {
    ProfScope prof("attn_bwd_dkdv", st);
    const int items = b.n_tiles * b.hkv;
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, KG, false>), dim3((items + kXcds - 1) / kXcds * kXcds, b.nsplit),
                       dim3(KG * 128),
                       0, st, b);
  }
  if (b.nsplit > 1) {
    ProfScope prof("attn_bwd_dkdv_reduce", st);
    const int64_t n = (int64_t)b.T * b.hkv * D;
    hipLaunchKernelGGL(dkdv_reduce_kernel<D>, dim3((n / 4 + 255) / 256), dim3(256), 0, st, b, n);
  }
}

void dkdv_launch(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128) launch_dkdv_t<128, 4>(a, st);
  else launch_dkdv_t<64, 4>(a, st);
}

}  // namespace uly

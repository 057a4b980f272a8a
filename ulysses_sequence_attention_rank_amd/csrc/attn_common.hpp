// Device helpers shared by the attention kernels (gfx950, wave64, bf16 MFMA).
//
// Matrix-core conventions (v_mfma_f32_32x32x16_bf16, lane l, half hf = l / 32):
//   A operand (32 x 16, M x K): lane holds A[l % 32][8 hf .. 8 hf + 7]
//   B operand (16 x 32, K x N): lane holds B[8 hf .. 8 hf + 7][l % 32]
//   C (32 x 32 fp32, 16 values): value 4 i + j is C[8 i + 4 hf + j][l % 32]
// so after a product the lane owns one COLUMN.  Attention keeps the query in
// that column (S^T = K Q^T): a lane then owns one query row's scores, its
// running max/sum are per-lane scalars, and the only cross-lane step is one
// swap between the two 32-lane halves.  The 16 scores a lane owns in a
// 32-key block serve directly as the B operand of the next product that
// contracts over keys, if the A operand reads its keys in the same order:
// operand slot e of half hf  <->  key 4 hf + e (e < 4), 8 + 4 hf + (e - 4) (e >= 4)
// within each 16-key step.  The "transposed" LDS tiles below store rows in
// groups of four so that this A operand is two 8-byte reads.
#pragma once

#include "common.hpp"

namespace uly {

constexpr int kBK = 64;   // keys (or queries) per LDS tile
constexpr int kPad = 64;  // zero rows after the backward's fp16 copies

// Where the D contiguous elements of (token t of the flattened B*S, head h)
// of a bf16 tensor start: with t = b*S + s and s = r*Sl + sl (sequence shard
// r of Sl tokens), at b*batch + r*shard + sl*token + h*head elements.  The
// head layout [B][S][H][D] and, for B = 1, the rank's heads of the
// sequence-sharded [P][B][S/P][H][D] are `uniform`: t*token.
// A KV chunk (positions [s0, s0 + s_len) of every batch row, the inner step
// of a ring over KV chunks) is addressed by its position s - s0, clamped
// into the chunk (rows outside it are never visible; the clamp keeps their
// loads inside the tensor).  Whole tensors: s0 = 0, s_len = S.
struct RowMap {
  int64_t batch, shard, token, head;
  FastDiv S, Sl;
  int uniform;  // row(t) = (t - s0) * token (the caller keeps t inside the chunk)
  int s0, s_len;
};

__device__ __forceinline__ int64_t row_of(const RowMap& m, int t) {
  if (m.uniform) return (int64_t)(t - m.s0) * m.token;
  const u32 b = fdiv((u32)t, m.S);
  const int sc = min(max((int)((u32)t - b * m.S.d) - m.s0, 0), m.s_len - 1);
  const u32 r = fdiv((u32)sc, m.Sl), sl = (u32)sc - r * m.Sl.d;
  return (int64_t)b * m.batch + (int64_t)r * m.shard + (int64_t)sl * m.token;
}

struct AttnArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  __bf16* out;   // fwd: O; bwd dq kernel: dQ
  __bf16* dk;    // fp32 (float*) when dkv_f32
  __bf16* dv;
  int dkv_f32;   // dK, dV written unrounded in fp32
  float* lse;    // fwd output / bwd input, [B][hq][S]
  float* ndelta;  // bwd: -rowsum(dO * O) with the bf16 O, [B][hq][S] (negated: dK/dV starts its dP sums from it)
  float* pdp;    // bwd: sum_j P_ij dP_ij = dO_i . O_i with the exact O, [B][hq][S]
  float* lse2;   // bwd: LSE * log2(e) (+inf for rows without keys), [B][hq][S]
  // bwd: exact fp16 copies of q, k, v, dout (the backward's products run in
  // fp16, whose 11-bit significand rounds P and dS 8x finer than bf16), each
  // followed by kPad zero rows so that tiles starting anywhere below T can
  // be loaded without clamping
  _Float16* q16;
  _Float16* k16;
  _Float16* v16;
  _Float16* do16;
  // bwd: [0] the exponent e of the power-of-two scale 2^e of the fp16 dout
  // copy (every gradient is 2^e times the true one until its epilogue),
  // [1] and [2] the counts of q, k, v, dout*2^e elements whose fp16 copy
  // saturated or is inexact; stat_part: per-block maxima behind the choice of
  // e ([kStatBlocks][4])
  int* bwd_status;
  float* stat_part;
  const float* sink;
  float* dsink_part;  // [hq][n_part]
  float* dsink;
  const int32_t* cu;
  const int32_t* n_seqs;
  RowMap mq;  // q, out, dout, dq
  RowMap mk;  // k, v, dk, dv
  // keys restricted to positions [k_lo_s, k_hi_s) of each batch row (one KV
  // chunk; 0 and S otherwise); K/V tile rows are clamped to [kt_lo, kt_hi)
  int k_lo_s, k_hi_s, kt_lo, kt_hi;
  int o_f32;  // forward: O written normalised in fp32, [T][hq][D] (chunk results)
  int B, S, T, hq, hkv, G;
  float scale;       // softmax scale
  float scale_log2;  // softmax scale * log2(e)
  int causal, wl, wr;
  int n_tiles;       // query tiles (fwd, dq) or key tiles (dkdv)
  int n_part;
  // Split of the reduction dimension over blockIdx.y when the natural grid is
  // too small for the GPU: partial sums in fp32, summed by a fixed-order
  // reduce kernel (so results stay deterministic).
  int nsplit;
  float* part;       // dq: [nsplit][T][hq][D]; dkdv: dK then dV, [nsplit][T][hkv][D]
  float* part_pdp;   // dq: [nsplit][B][hq][S]; fwd: running max then sum, [2][nsplit][B][hq][S]
  // dK/dV balanced schedule (bal_W > 0 work-groups, see the balanced
  // schedule below): `part` then holds 2 bal_W slots of [2][BN][D] fp32
  // parts, and bal_prefix receives the unit prefix over the key tiles.
  int bal_W;
  int* bal_prefix;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product on fp16 operands.  Operand fragments travel as 16-bit
// bit patterns (bf16x8); the backward kernels fill them with fp16 data.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32h(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Values of the partner lane (l ^ 32) combined with this lane's: both
// halves of v_permlane32_swap(v, v) together hold {v[l], v[l ^ 32]}.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Document [start, end) of flattened token t.
__device__ __forceinline__ void doc_bounds(const AttnArgs& a, int t, int& start, int& end) {
  if (a.cu == nullptr) {
    start = (t / a.S) * a.S;
    end = start + a.S;
    return;
  }
  int lo = 0, hi = max(*a.n_seqs, 1);  // largest d in [0, n) with cu[d] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.cu[mid] <= t) lo = mid; else hi = mid;
  }
  start = a.cu[lo];
  end = a.cu[lo + 1];
}

// Keys visible to query i form the interval [klo, khi).
__device__ __forceinline__ void key_interval(const AttnArgs& a, int i, int& klo, int& khi) {
  int ds, de;
  doc_bounds(a, i, ds, de);
  const int b0 = (i / a.S) * a.S;  // the chunk's keys in query i's batch row
  klo = max(ds, b0 + a.k_lo_s);
  khi = min(de, b0 + a.k_hi_s);
  if (a.causal) khi = min(khi, i + 1);
  if (a.wl >= 0) klo = max(klo, i - a.wl);
  if (a.wr >= 0) khi = min(khi, i + a.wr + 1);
  if (khi < klo) khi = klo;
}

// Queries that see key j form the interval [qlo, qhi).
__device__ __forceinline__ void query_interval(const AttnArgs& a, int j, int& qlo, int& qhi) {
  int ds, de;
  doc_bounds(a, j, ds, de);
  qlo = ds;
  qhi = de;
  if (a.causal) qlo = max(qlo, j);
  if (a.wl >= 0) qhi = min(qhi, j + a.wl + 1);
  if (a.wr >= 0) qlo = max(qlo, j - a.wr);
  if (qhi < qlo) qhi = qlo;
}

__device__ __forceinline__ int lse_index(const AttnArgs& a, int t, int h) {
  const int b = t / a.S;
  return (b * a.hq + h) * a.S + (t - b * a.S);
}

// XCD-aware deal of n work items over a grid of 8 * ceil(n / 8) blocks:
// blocks go round-robin to the 8 XCDs, and the j-th block of an XCD takes
// the j-th item of that XCD's share, the shares interleaved in bands of W
// consecutive items.  The W work-groups resident on an XCD at once then
// work on neighbouring items and share what they stream through its L2.
// The XCD order reverses every other band (a snake), so work that grows or
// shrinks linearly along the items evens out over the XCDs (which cannot
// take over each other's blocks).  Returns -1 for padding blocks.
__device__ __forceinline__ int xcd_band_item(int b, int n, int W) {
  const int n8 = (n + kXcds - 1) / kXcds;  // blocks per XCD
  const int xcd = b % kXcds, j = b / kXcds;
  const int band = j / W, within = j - band * W;
  const int w = min(W, n8 - band * W);     // the last band may be narrower
  const int slot = (band & 1) ? kXcds - 1 - xcd : xcd;
  const int item = band * kXcds * W + slot * w + within;
  return item < n ? item : -1;
}

// Work decode shared by the query-tile kernels.  Query tiles are ordered last
// first (causal tiles near the end see the most keys); the G query heads of a
// KV head that work on the same tile are put on one XCD (L2 shares their K/V).
__device__ __forceinline__ bool decode_qtile(const AttnArgs& a, int& qt, int& h) {
  const int L = blockIdx.x;
  const int xcd = L % kXcds, slot = L / kXcds;
  const int grp = (slot / a.G) * kXcds + xcd, member = slot % a.G;
  if (grp >= a.n_tiles * a.hkv) return false;
  qt = a.n_tiles - 1 - grp / a.hkv;
  h = (grp % a.hkv) * a.G + member;
  return true;
}

// ------------------------------------------------ swizzled tiles (gfx950)
//
// A tile of R rows x D bf16 sits in LDS row-major, 2*D bytes a row, its
// 16-byte slots XOR-swizzled per row: logical slot c of row r lives at
// physical slot c ^ swz(r).  The LDS has 64 four-byte banks (256 bytes a
// pass).  A 16-byte operand read serves 16 lanes a pass: 16 consecutive rows,
// one slot each, so swz is a bijection on 16 rows.  A transposing read serves
// 32 lanes a pass: four consecutive rows, 64 bytes each, so swz also sends
// those four rows' 64-byte groups to the four distinct 64-byte bank groups
// (bits 2-3 of the slot for D=128; the row parity and bit 2 for D=64).
// Measured with SQ_LDS_BANK_CONFLICT: zero conflicts for both read forms.  Tiles arrive by global_load_lds
// (16 bytes a lane, lane l at byte 16*l of the instruction's 1 KiB): no
// registers, no VALU beyond the address.  One tile serves both operand
// forms:
//   natural  (A or B): lane l gets row r0 + l%32, columns 16s + 8hf .. + 7
//   transposed (A or B): lane l gets column d0 + l%32 of the rows in the
//     k-slot order of attn_common.hpp, via two ds_read_b64_tr_b16: within a
//     16-lane group, lane j receives element j%4 of the 8-byte chunks that
//     lanes j/4, j/4+4, j/4+8, j/4+12 address, so lane s addresses row
//     kb + s/4, columns c0 + 4(s%4) .. + 3 and gets rows kb..kb+3 of column
//     c0 + (its own index in the group).

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Swz {
  static constexpr int kSlots = D / 8;  // 16-byte slots per row
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // byte offset of logical 16-byte slot c of row r
  __device__ static __forceinline__ int off(int r, int c) { return r * (2 * D) + ((c ^ f(r)) << 4); }
};

// Issue the direct-to-LDS loads of a R x D tile: rows row0 .. row0+R-1 of a
// global matrix with row stride ld elements (rows at or past row_end are
// clamped to row_end - 1: finite data that the masks then ignore).
template <int D, int R, int NW, typename E>
__device__ __forceinline__ void tile_load_lds(char* lds, const E* g, int ld, int row0,
                                              int row_end, int wave, int lane) {
  static_assert(sizeof(E) == 2, "16-bit elements");
  constexpr int kInstr = R * D * 2 / 1024;  // 1 KiB per wave instruction
  static_assert(kInstr % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int k = 0; k < kInstr / NW; ++k) {
    const int i = wave + k * NW;
    const int pos = i * 64 + lane;               // 16-byte slot index in the tile
    const int r = pos / Swz<D>::kSlots;
    const int c = (pos % Swz<D>::kSlots) ^ Swz<D>::f(r);
    const int row = min(row0 + r, row_end - 1);
    const char* src = reinterpret_cast<const char*>(g) + ((int64_t)row * ld + c * 8) * 2;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds + i * 1024), 16, 0, 0);
  }
}

// The same for a bf16 tensor addressed through a RowMap (`base` already
// offset to the head): rows row0 .. row0+R-1, clamped to row_end - 1.
template <int D, int R, int NW, bool UNIFORM>
__device__ __forceinline__ void tile_load_lds_map(char* lds, const __bf16* base, const RowMap& m,
                                                  int row0, int row_lo, int row_end, int wave,
                                                  int lane) {
  constexpr int kInstr = R * D * 2 / 1024;
  static_assert(kInstr % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int k = 0; k < kInstr / NW; ++k) {
    const int i = wave + k * NW;
    const int pos = i * 64 + lane;
    const int r = pos / Swz<D>::kSlots;
    const int c = (pos % Swz<D>::kSlots) ^ Swz<D>::f(r);
    const int row = max(min(row0 + r, row_end - 1), row_lo);
    const __bf16* src = base + (UNIFORM ? (int64_t)(row - m.s0) * m.token : row_of(m, row)) + c * 8;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds + i * 1024), 16, 0, 0);
  }
}

// Direct-to-LDS loads of R x D tiles whose rows lie `ld` elements apart,
// through a buffer resource: the tile's first row is a wave-uniform base in
// scalar registers and each lane's byte offset inside the tile is computed
// once, so a load costs no vector instruction.  Rows at or beyond the
// resource's bound read as zero, so a tile that runs past the matrix's last
// row needs no clamping (callers mask those rows).  Needs 64 * ld < 2^24.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
template <int D, int R, int NW>
struct BufTileLoader {
  static constexpr int kN = R * D * 2 / 1024 / NW;  // loads per wave
  unsigned off[kN];
  int row_bytes;
  __device__ __forceinline__ BufTileLoader(int64_t ld, int wave, int lane) : row_bytes((int)ld * 2) {
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int pos = (wave + k * NW) * 64 + lane;
      const int r = pos / Swz<D>::kSlots;
      off[k] = (unsigned)(r * row_bytes + (((pos % Swz<D>::kSlots) ^ Swz<D>::f(r)) << 4));
    }
  }
  // rows [0, rows) of the tile at `tile0` exist (rows >= 1); `wave` uniform
  __device__ __forceinline__ void load(char* lds, const void* tile0, int rows, int wave) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(tile0), (short)0, min(rows, R) * row_bytes, kRsrcWord3);
#pragma unroll
    for (int k = 0; k < kN; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (wave + k * NW) * 1024), 16, off[k],
                                               0, 0, 0);
  }
};

// Per-lane byte offsets of a wave's direct-to-LDS loads of an R x D tile of
// a matrix with row stride `ld` elements, relative to the tile's first row:
// the same for every tile, so a loop computes them once and issues each load
// as a uniform base plus this offset (the rows must exist: callers pad).
template <int D, int R, int NW>
struct TileOffsets {
  static constexpr int kN = R * D * 2 / 1024 / NW;  // loads per wave
  int off[kN];
  __device__ __forceinline__ TileOffsets(int ld, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < kN; ++k) {
      const int pos = (wave + k * NW) * 64 + lane;
      const int r = pos / Swz<D>::kSlots;
      off[k] = (r * ld + (((pos % Swz<D>::kSlots) ^ Swz<D>::f(r)) << 3)) * 2;
    }
  }
  __device__ __forceinline__ void load(char* lds, const void* tile0, int wave) const {
#pragma unroll
    for (int k = 0; k < kN; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(tile0) + off[k]),
                                       (lds_void*)(lds + (wave + k * NW) * 1024), 16, 0, 0);
  }
};

// natural operand: rows r0 + l%32, columns 16 s + 8 hf .. + 7
template <int D>
__device__ __forceinline__ bf16x8 swz_nat(const char* lds, int r0, int s, int lane) {
  const int r = r0 + (lane & 31);
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + Swz<D>::off(r, 2 * s + (lane >> 5))));
}

// transposed operand for the 16-row step at r0: column d0 + l%32
template <int D>
__device__ __forceinline__ bf16x8 swz_tr(const char* lds, int r0, int d0, int lane) {
  const int j = lane & 15, grp = lane >> 4;
  const int col = d0 + 16 * (grp & 1) + 4 * (j & 3);
  const int kb = r0 + 4 * (grp >> 1) + (j >> 2);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + Swz<D>::off(kb, col >> 3) + (col & 7) * 2));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + Swz<D>::off(kb + 8, col >> 3) + (col & 7) * 2));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// Per-lane byte offsets of the swz_nat / swz_tr reads, computed once: the
// swizzle repeats every 16 rows, so for r0 a multiple of 16 the natural
// operand of step s at rows r0 + l%32 lies at r0 * 2D + nat[s] and the
// transposed operand of columns 32 nb at rows r0 .. r0+15 at r0 * 2D +
// tr[nb][0] (rows +0..7) and r0 * 2D + tr[nb][1] (rows +8..15).  Kernels
// with two LDS stages share one set between the stages, the stage base
// folding into each read's immediate offset.
template <int D>
struct SwzOffsets {
  int nat[D / 16];
  int tr[D / 32][2];
  __device__ __forceinline__ explicit SwzOffsets(int lane) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) nat[s] = Swz<D>::off(lane & 31, 2 * s + (lane >> 5));
    const int j = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) {
      const int col = 32 * nb + 16 * (grp & 1) + 4 * (j & 3);
      const int kb = 4 * (grp >> 1) + (j >> 2);
      tr[nb][0] = Swz<D>::off(kb, col >> 3) + (col & 7) * 2;
      tr[nb][1] = Swz<D>::off(kb + 8, col >> 3) + (col & 7) * 2;
    }
  }
  // Makes the offsets opaque to the optimiser at this point, so that
  // addresses derived from them are formed where they are used instead of
  // being hoisted, one register each, out of an enclosing loop.
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) asm volatile("" : "+v"(nat[s]));
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) asm volatile("" : "+v"(tr[nb][0]), "+v"(tr[nb][1]));
  }
  __device__ __forceinline__ bf16x8 nat_at(const char* lds, int r0, int s) const {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + r0 * 2 * D + nat[s]));
  }
  __device__ __forceinline__ bf16x8 tr_at(const char* lds, int r0, int nb) const {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + r0 * 2 * D + tr[nb][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + r0 * 2 * D + tr[nb][1]));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, x);
  }
};

// ------------------------------------------------ balanced schedule
//
// For grids too small to fill the GPU with one work-group per item.  An item
// is (tile t, head h), numbered i = h * n_tiles + t; it is a run of c[t] >= 1
// units (the tiles it visits; an item with none still takes one, to write its
// empty result).  With the runs concatenated, U units in all, work-group lam
// takes units [start(lam), start(lam + 1)), start(lam) = floor(lam U / W):
// equal shares whatever the mask makes of the runs.  An item whose run lies
// inside one share is finished by that work-group.  Otherwise each
// work-group writes its part of the item to a slot: 2 lam for an item begun
// by an earlier work-group, 2 lam + 1 for one continued by a later one; a
// reduce kernel adds an item's parts in work-group order (deterministic).
constexpr int kBalMaxTiles = 2048;

__device__ __forceinline__ int64_t bal_start(int64_t lam, int64_t U, int W) { return lam * U / W; }
// the work-group whose share holds unit u (the largest lam with start <= u)
__device__ __forceinline__ int bal_owner(int64_t u, int64_t U, int W) { return (int)(((u + 1) * W - 1) / U); }

// Exclusive prefix P[0..n] of count(t), t < n (n <= kBalMaxTiles), in LDS;
// every thread of the work-group calls it.
template <typename F>
__device__ __forceinline__ void bal_prefix(int* P, int n, F count) {
  for (int t = threadIdx.x; t < n; t += blockDim.x) P[t + 1] = count(t);
  __syncthreads();
  if (threadIdx.x < 64) {  // one wave scans: lane l owns tiles [l C, (l + 1) C)
    const int lane = threadIdx.x, C = (n + 63) / 64;
    const int lo = min(lane * C, n), hi = min(lo + C, n);
    int s = 0;
    for (int t = lo; t < hi; ++t) s += P[t + 1];
    int x = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    int run = x - s;
    for (int t = lo; t < hi; ++t) {
      run += P[t + 1];
      P[t + 1] = run;
    }
    if (lane == 0) P[0] = 0;
  }
  __syncthreads();
}

// The tile t holding unit r of a head's run (P[t] <= r < P[t + 1]).
__device__ __forceinline__ int bal_tile(const int* P, int n, int r) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// This work-group's share, item by item: f(t, h, seg_lo, seg_hi, slot) runs
// units [seg_lo, seg_hi) of item (t, h) (offsets in its run) and writes the
// finished result (slot < 0) or part slot `slot`.  Work-groups are dealt to
// the XCDs round-robin; consecutive shares go to one XCD (W % kXcds == 0).
template <typename F>
__device__ __forceinline__ void bal_walk(const int* P, int n, int nh, int W, F f) {
  const int tot = P[n];
  const int64_t U = (int64_t)nh * tot;
  const int lam = (int)(blockIdx.x % kXcds) * (W / kXcds) + (int)(blockIdx.x / kXcds);
  const int64_t s0 = bal_start(lam, U, W), s1 = bal_start(lam + 1, U, W);
  int64_t u = s0;
  bool first = true;
  while (u < s1) {
    const int h = (int)(u / tot), r = (int)(u - (int64_t)h * tot);
    const int t = bal_tile(P, n, r);
    const int64_t p0 = (int64_t)h * tot + P[t], p1 = p0 + (P[t + 1] - P[t]);
    const int64_t e = min(s1, p1);
    const int slot = (u == p0 && e == p1) ? -1 : (p0 < s0 ? 2 * lam : 2 * lam + 1);
    if (!first) __syncthreads();  // the previous item's LDS is no longer read
    first = false;
    f(t, h, (int)(u - p0), (int)(e - p0), slot);
    u = e;
  }
}

// For the reduce of item (t, h) of n tiles and nh heads: the work-groups
// la .. lb that hold its parts (la == lb: finished in place), whether
// work-group lam of them holds one (shares can be empty when U < W), and
// its slot (2 lam + 1 for la, which begins the item; 2 lam after).
struct BalItem {
  int la, lb, W;
  int64_t U;
  __device__ __forceinline__ BalItem(const int* P, int n, int t, int h, int nh, int W_) : W(W_) {
    const int tot = P[n];
    U = (int64_t)nh * tot;
    const int64_t p0 = (int64_t)h * tot + P[t], p1 = p0 + (P[t + 1] - P[t]);
    la = bal_owner(p0, U, W);
    lb = bal_owner(p1 - 1, U, W);
  }
  __device__ __forceinline__ bool holds(int lam) const {
    return lam == la || bal_start(lam + 1, U, W) > bal_start(lam, U, W);
  }
  __device__ __forceinline__ int slot(int lam) const { return lam == la ? 2 * lam + 1 : 2 * lam; }
};

// Contiguous share [lo, hi) of n iterations for split s of ns.
__device__ __forceinline__ void split_range(int n, int s, int ns, int& lo, int& hi) {
  lo = (int)(((int64_t)n * s) / ns);
  hi = (int)(((int64_t)n * (s + 1)) / ns);
}

// B operand held in registers: row `row` (or zeros), columns 16 s + 8 hf ..
template <int D, typename E>
__device__ __forceinline__ void load_row_frags(bf16x8 (&f)[D / 16], const E* rowp, bool valid, int lane) {
  static_assert(sizeof(E) == 2, "16-bit elements");
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 x = {0, 0, 0, 0};
    if (valid) x = *reinterpret_cast<const u32x4*>(rowp + 16 * s + 8 * (lane >> 5));
    f[s] = __builtin_bit_cast(bf16x8, x);
  }
}

// fp16 round-to-nearest-even from fp32, two at a time (v_cvt_pk_f16_f32).
__device__ __forceinline__ u32 pack_f16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(u32, __builtin_convertvector(x, f16x2));
}

// Eight accumulator values as an fp16 operand (slot order as acc_frag).
__device__ __forceinline__ bf16x8 acc_frag_h(const f32x16& c, int ii) {
  u32x4 x;
  x[0] = pack_f16x2(c[8 * ii + 0], c[8 * ii + 1]);
  x[1] = pack_f16x2(c[8 * ii + 2], c[8 * ii + 3]);
  x[2] = pack_f16x2(c[8 * ii + 4], c[8 * ii + 5]);
  x[3] = pack_f16x2(c[8 * ii + 6], c[8 * ii + 7]);
  return __builtin_bit_cast(bf16x8, x);
}

// Eight accumulator values (C rows 8(2ii) + 4hf + j and 8(2ii+1) + 4hf + j)
// as the bf16 operand of the next product: exactly slots e = 0..7 above.
__device__ __forceinline__ bf16x8 acc_frag(const f32x16& c, int ii) {
  u32x4 x;
  x[0] = pack_bf16x2(c[8 * ii + 0], c[8 * ii + 1]);
  x[1] = pack_bf16x2(c[8 * ii + 2], c[8 * ii + 3]);
  x[2] = pack_bf16x2(c[8 * ii + 4], c[8 * ii + 5]);
  x[3] = pack_bf16x2(c[8 * ii + 6], c[8 * ii + 7]);
  return __builtin_bit_cast(bf16x8, x);
}

}  // namespace uly

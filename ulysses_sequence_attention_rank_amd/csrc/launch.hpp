// Internal launch functions behind the C ABI (host side), and the optional
// per-kernel event recorder used by ulysses_profile_*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uly {

struct AttnArgs;

hipError_t permute_launch(bool pack, int n, const void* const* src, void* const* dst, const int* H,
                          int P, int B, int S, int D, int elem_bytes, hipStream_t st);
hipError_t reduce_replicated_launch(const void* head, bool head_f32, void* seq, int P, int B, int S,
                                    int H, int D, hipStream_t st);
hipError_t segments_launch(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
                           int64_t cu_capacity, int32_t* n_seqs, int32_t* max_len, hipStream_t st);
// int32 slots the many-work-group scan needs after cu_seqlens[B*S]
int64_t segments_scratch_slots(int B, int S);
hipError_t attn_fwd_launch(const AttnArgs& a, int D, hipStream_t st);
hipError_t attn_merge_launch(float* acc_o, float* acc_lse, const float* o, const float* lse, int B,
                             int S, int hq, int D, hipStream_t st);
hipError_t attn_merge_finish_launch(const float* acc_o, const float* acc_lse, const float* sink,
                                    void* out, float* lse, int B, int S, int hq, int D,
                                    hipStream_t st);
hipError_t attn_bwd_launch(const AttnArgs& a, int D, hipStream_t st);
void dkdv_launch(const AttnArgs& a, int D, hipStream_t st);  // part of attn_bwd_launch

// The sequence-tiled gated MLP (mlp.hip): x, dy, y, dx [T][H]; gate and up
// weights [I][H], down weight [H][I] (bf16); weight gradients fp32; ws holds
// one tile's activations (mlp_workspace_bytes).
struct MlpArgs {
  const __bf16 *x, *wg, *wu, *wd, *dy;
  __bf16 *y, *dx;
  float *dwg, *dwu, *dwd;
  void* ws;
  int T, H, I, tile;
};
hipError_t mlp_fwd_launch(const MlpArgs& p, hipStream_t st);
hipError_t mlp_bwd_launch(const MlpArgs& p, hipStream_t st);

// The matrix-core calibration (calib.hip, a measurement aid): kCalibBlocks
// work-groups of 256 threads, two per CU, each wave `iters` (a multiple of 8)
// 32x32x16 bf16 products on each of its eight accumulators, in `mode` 0-5
// (see calib.hip); one float per thread into out.
constexpr int kCalibBlocks = 512;
hipError_t calib_mfma_launch(float* out, int iters, int mode, hipStream_t st);

// Number of splits of a reduction dimension for a kernel whose natural grid
// has `wgs` work-groups of which `per_round` are resident at once on MI355X
// (256 CUs times the work-groups a CU holds): the split count (at most 4, at
// most one per 64-row tile) that minimises the rounds of resident work-groups
// per unit of work, ceil(wgs * ns / per_round) / ns.  On an `uneven` layer
// (causal or windowed), when the unsplit grid fills at most two rounds, a
// split that only ties with it is still taken: halving the work-groups evens
// out causal and variable-length work, which the count of rounds does not
// see (measured, dK/dV with 2 splits instead of 1: S=32768 packed 1.20 ->
// 1.01 ms, S=65536 window 8.8 -> 5.8 ms; on S=131072, four rounds, it lost
// 4 %).  On a full layer the work-groups are even (packed documents aside,
// which the host does not see) and a tie only adds the partials and their
// reduce (dK/dV on the full S=4096 layer: 182 us with 2 splits, 160 with
// none).  Among splits, ties go to fewer.  Each split writes fp32 partials of `split_bytes` that a reduce reads
// back: two splits may write up to 256 MiB of them, more splits up to 64 MiB
// (S=4096: dK/dV with 4 splits, 100 MB of partials, took 147 us with its
// reduce, with 2 splits 142 us).  A function of the sizes only, so the
// workspace query and the launch agree.
constexpr double kSplitBytesCap2 = 256.0 * 1024 * 1024, kSplitBytesCapN = 64.0 * 1024 * 1024;
inline int choose_splits(long wgs, long tiles, long per_round, double split_bytes, bool uneven) {
  if (wgs <= 0) return 1;
  int best = 1;
  const double t1 = (double)((wgs + per_round - 1) / per_round);
  double best_t = t1;
  for (long ns = 2; ns <= 4 && ns <= tiles; ++ns) {
    if (ns * split_bytes > (ns == 2 ? kSplitBytesCap2 : kSplitBytesCapN)) break;
    const double t = (double)((wgs * ns + per_round - 1) / per_round) / (double)ns;
    if (t < best_t - 1e-9 || (uneven && best == 1 && t1 <= 2.0 && t <= best_t + 1e-9)) {
      best_t = t;
      best = (int)ns;
    }
  }
  return best;
}
// dK/dV: 128-key work-groups, one per CU (its LDS footprint); partials dK, dV
inline int dkdv_splits(int B, int S, int hkv, int D, bool uneven) {
  const long T = (long)B * S;
  return choose_splits(((T + 127) / 128) * hkv, (T + 63) / 64, 256, 8.0 * T * hkv * D, uneven);
}
// dQ: 128-query work-groups, two per CU; partials dQ and sum P dP
inline int qtile_splits(int B, int S, int hq, int D, bool uneven) {
  const long T = (long)B * S;
  return choose_splits(((T + 127) / 128) * hq, (T + 63) / 64, 512, 4.0 * T * hq * (D + 1), uneven);
}

// Forward: query tiles of `bm` rows, two work-groups per CU; partials O and
// the running max and sum
inline int fwd_splits(int B, int S, int hq, int bm, int D, bool uneven) {
  const long T = (long)B * S;
  return choose_splits(((T + bm - 1) / bm) * hq, (T + 63) / 64, 512, 4.0 * T * hq * (D + 2), uneven);
}
// dK/dV balanced schedule (attn_common.hpp): one round of 256 work-groups
// takes equal shares of the (query tile, head) iterations of all (key tile,
// KV head) items of 128 keys.  Used when the items fill at most two rounds of
// one-per-CU work-groups and there are at least 256 key tiles: long causal
// or packed sequences, whose key tiles carry very uneven work (measured,
// dK/dV per launch: packed S=32768, GQA 4, 825 -> 643 us; the same over 16
// ranks with replicated KV, 295 -> 193 us; S=65536 window + causal,
// unchanged).  On short sequences (S=4096, 32 key tiles) it lost: every
// item is split, the parts must be summed, and work-groups that continue an
// item walk other query tiles than their XCD neighbours, which loses the
// shared L2 streaming (full layer 132 -> 132 + 14 us, causal 84 -> 107 us).
// Returns the work-group count, 0 for none.
constexpr int kBalMaxTilesHost = 2048;
constexpr int kDkdvBalWorkgroups = 256;
inline int dkdv_bal_workgroups(int B, int S, int hkv) {
  const long tiles = ((long)B * S + 127) / 128;
  if (tiles < 256 || tiles > kBalMaxTilesHost || tiles * hkv > 2 * 256) return 0;
  return kDkdvBalWorkgroups;
}
// A layer's work-groups are uneven when it is causal or windowed.  Split
// counts never fall when `uneven` is set, so workspaces sized with it serve
// every layer.
inline bool uneven_layer(int causal, int wl, int wr) { return causal || wl >= 0 || wr >= 0; }
// A sliding window whose span (keys a row sees, queries a key is seen by) is
// under 256: bounded on the left and, unless causal, on the right.
inline bool narrow_window(int causal, int wl, int wr) {
  return wl >= 0 && (causal || wr >= 0) && wl + (causal ? 0 : wr) < 256;
}
// Rows of a forward query tile for head dim D (the launcher's variant choice).
inline int fwd_block_rows(int B, int S, int hq, int D) {
  if (D == 128) return 128;
  return (long)(((long)B * S + 255) / 256) * hq >= 512 ? 256 : 128;
}

// The backward's power-of-two scales of its fp16 copies (attn_bwd.hip):
// kStatFloats per-block maxima from kStatBlocks blocks at most; exponents
// clamped to [-kScaleExpMax, kScaleExpMax].  The status words: the exponents
// of dout, v, q, k, then the counts of saturated and of inexact copies.
constexpr int kStatBlocks = 1024;
constexpr int kStatFloats = 8;
constexpr int kScaleExpMax = 100;
enum { kExpDout = 0, kExpV = 1, kExpQ = 2, kExpK = 3, kCntSat = 4, kCntInexact = 5 };

// When profiling is on, prof_mark(name, st) records a HIP event on `st`
// before a kernel launch and prof_mark(nullptr, st) after it.
void prof_mark(const char* name, hipStream_t st);

struct ProfScope {
  hipStream_t st;
  ProfScope(const char* name, hipStream_t s) : st(s) { prof_mark(name, s); }
  ~ProfScope() { prof_mark(nullptr, st); }
};

}  // namespace uly

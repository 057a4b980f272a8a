// cu_seqlens / n_seqs / max_len from the P position_ids shards, in one
// work-group with no host synchronisation.
//
// The gathered sequence is the concatenation of the shards in rank order;
// a document starts at every flattened token t = b*S + i with i == 0 or
// pos == 0.  Each thread owns a contiguous chunk of tokens: it counts its
// starts, an exclusive scan over the work-group gives each chunk its first
// output slot, and the chunk writes its starts.  The length of a chunk's last
// document needs the first start of a later chunk, found with a suffix
// minimum; max_len is a work-group maximum.  A thread reads its chunk kBatch
// tokens at a time (the loads of a batch are in flight together); the scans
// run within each wave by lane shuffles, then over the waves' totals.
#include "common.hpp"
#include "launch.hpp"

namespace uly {

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / 64;
constexpr int kBatch = 8;

struct SegArgs {
  const void* pos;
  int32_t* cu;
  int32_t* n_out;
  int32_t* max_len;
  u32 T;      // B * S
  u32 chunk;  // tokens per thread
  FastDiv S, Sl;
  u32 B;
};

template <typename PosT>
__device__ __forceinline__ bool is_start(const SegArgs& a, u32 t) {
  const u32 b = fdiv(t, a.S), i = t - b * a.S.d;
  if (i == 0) return true;
  const u32 r = fdiv(i, a.Sl), s = i - r * a.Sl.d;
  const PosT* p = reinterpret_cast<const PosT*>(a.pos);
  return p[((uint64_t)r * a.B + b) * a.Sl.d + s] == 0;
}

// f(t) for every start t of [lo, hi), in order
template <typename PosT, typename F>
__device__ __forceinline__ void for_starts(const SegArgs& a, u32 lo, u32 hi, F f) {
  for (u32 t0 = lo; t0 < hi; t0 += kBatch) {
    bool st[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) st[k] = t0 + k < hi && is_start<PosT>(a, t0 + k);
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (st[k]) f(t0 + k);
  }
}

template <typename PosT>
__global__ __launch_bounds__(kSegThreads) void segments_kernel(SegArgs a) {
  __shared__ int32_t s_sum[kSegWaves], s_min[kSegWaves], s_max[kSegWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const u32 lo = min(a.T, (u32)tid * a.chunk), hi = min(a.T, lo + a.chunk);
  constexpr int32_t kNone = 0x7fffffff;

  // pass 1: count starts, remember the first and last one and the longest
  // document that ends inside the chunk
  int32_t cnt = 0, first = kNone, last = -1, best = 0;
  for_starts<PosT>(a, lo, hi, [&](u32 t) {
    if (last >= 0) best = max(best, (int32_t)t - last);
    if (first == kNone) first = (int32_t)t;
    last = (int32_t)t;
    ++cnt;
  });

  // inclusive prefix sum of the counts and suffix minimum of the first
  // starts, within the wave
  int32_t x = cnt, f = first;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    const int32_t z = __shfl_down(f, off, 64);
    if (lane >= off) x += y;
    if (lane + off < 64) f = min(f, z);
  }
  if (lane == 63) s_sum[w] = x;
  if (lane == 0) s_min[w] = f;
  __syncthreads();
  int32_t before = 0, after = kNone;  // counts of earlier waves, first start of later ones
  for (int i = 0; i < kSegWaves; ++i) {
    if (i < w) before += s_sum[i];
    if (i > w) after = min(after, s_min[i]);
  }
  const int32_t incl = x + before;
  int32_t next = __shfl_down(f, 1, 64);  // first start after this chunk
  if (lane == 63) next = kNone;
  next = min(next, after);
  if (last >= 0) best = max(best, (next == kNone ? (int32_t)a.T : next) - last);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off, 64));
  if (lane == 0) s_max[w] = best;

  // pass 2: write the starts of this chunk
  int32_t slot = incl - cnt;
  for_starts<PosT>(a, lo, hi, [&](u32 t) { a.cu[slot++] = (int32_t)t; });
  __syncthreads();
  if (tid == kSegThreads - 1) {
    a.cu[incl] = (int32_t)a.T;
    *a.n_out = incl;
  }
  if (tid == 0) {
    int32_t m = 0;
    for (int i = 0; i < kSegWaves; ++i) m = max(m, s_max[i]);
    *a.max_len = m;
  }
}

hipError_t segments_launch(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
                           int32_t* n_seqs, int32_t* max_len, hipStream_t st) {
  SegArgs a;
  a.pos = pos;
  a.cu = cu;
  a.n_out = n_seqs;
  a.max_len = max_len;
  a.T = (u32)B * (u32)S;
  a.chunk = (a.T + kSegThreads - 1) / kSegThreads;
  a.S = make_fastdiv(S);
  a.Sl = make_fastdiv(S / P);
  a.B = B;
  ProfScope prof("cu_seqlens", st);
  if (pos_bytes == 8)
    hipLaunchKernelGGL(segments_kernel<int64_t>, dim3(1), dim3(kSegThreads), 0, st, a);
  else
    hipLaunchKernelGGL(segments_kernel<int32_t>, dim3(1), dim3(kSegThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace uly

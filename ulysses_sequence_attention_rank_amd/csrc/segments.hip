// cu_seqlens / n_seqs / max_len from the P position_ids shards, in one
// work-group with no host synchronisation.
//
// The gathered sequence is the concatenation of the shards in rank order;
// a document starts at every flattened token t = b*S + i with i == 0 or
// pos == 0.  Each thread owns a contiguous chunk of tokens: it counts its
// starts, an exclusive scan over the work-group gives each chunk its first
// output slot, and the chunk writes its starts.  The length of a chunk's last
// document needs the first start of a later chunk, found with a suffix
// minimum; max_len is a work-group maximum.
#include "common.hpp"
#include "launch.hpp"

namespace uly {

constexpr int kSegThreads = 1024;

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

template <typename PosT>
__global__ __launch_bounds__(kSegThreads) void segments_kernel(SegArgs a) {
  __shared__ int32_t s_cnt[kSegThreads];
  __shared__ int32_t s_first[kSegThreads];
  __shared__ int32_t s_max[kSegThreads];
  const int tid = threadIdx.x;
  const u32 lo = min(a.T, (u32)tid * a.chunk), hi = min(a.T, lo + a.chunk);

  // pass 1: count starts, remember the first and last one
  int32_t cnt = 0, first = 0x7fffffff, last = -1, best = 0;
  for (u32 t = lo; t < hi; ++t) {
    if (is_start<PosT>(a, t)) {
      if (last >= 0) best = max(best, (int32_t)t - last);
      if (first == 0x7fffffff) first = (int32_t)t;
      last = (int32_t)t;
      ++cnt;
    }
  }
  s_cnt[tid] = cnt;
  s_first[tid] = first;
  __syncthreads();
  // exclusive scan of the counts and suffix minimum of the first starts
  // (Hillis-Steele over the work-group, log2(1024) rounds)
  for (int off = 1; off < kSegThreads; off <<= 1) {
    const int32_t c = tid >= off ? s_cnt[tid - off] : 0;
    const int32_t f = tid + off < kSegThreads ? s_first[tid + off] : 0x7fffffff;
    __syncthreads();
    s_cnt[tid] += c;
    s_first[tid] = min(s_first[tid], f);
    __syncthreads();
  }
  const int32_t incl = s_cnt[tid];
  const int32_t next = tid + 1 < kSegThreads ? s_first[tid + 1] : 0x7fffffff;
  const int32_t next_start = next == 0x7fffffff ? (int32_t)a.T : next;
  if (last >= 0) best = max(best, next_start - last);
  s_max[tid] = best;

  // pass 2: write the starts of this chunk
  int32_t slot = incl - cnt;
  for (u32 t = lo; t < hi; ++t)
    if (is_start<PosT>(a, t)) a.cu[slot++] = (int32_t)t;
  __syncthreads();
  for (int off = kSegThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_max[tid] = max(s_max[tid], s_max[tid + off]);
    __syncthreads();
  }
  if (tid == kSegThreads - 1) {
    a.cu[incl] = (int32_t)a.T;
    *a.n_out = incl;
  }
  if (tid == 0) *a.max_len = s_max[0];
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

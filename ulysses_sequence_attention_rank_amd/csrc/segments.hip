// cu_seqlens / n_seqs / max_len from the P position_ids shards, with no host
// synchronisation: on many work-groups when the cu_seqlens buffer has room
// for their scratch (the wide scan below), else in one work-group.
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
constexpr int kSegWideBlocks = 1024;

hipError_t segments_launch_one(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
                               int32_t* n_seqs, int32_t* max_len, hipStream_t st);
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

// ----------------------------------------------------------------- wide scan
//
// The same result from many work-groups, when the caller's cu_seqlens buffer
// has room for scratch after slot B*S (4 int32 per chunk).  Each work-group
// owns a contiguous chunk of C tokens (C a multiple of kSegRound, at most
// kSegWideBlocks chunks), taken kSegRound at a time: 2 tiles of 256 tokens,
// thread j reading token tile*256 + j, so a wave reads 64 consecutive
// positions per load (coalesced, both loads in flight together).  The start
// flags of a round are wave ballots kept in LDS in token order; a start's
// rank among the chunk's starts is then a sum of popcounts.
//   pass 1 (segments_part_kernel): per chunk, the number of starts, the first
//     and the last start, and the longest document that begins and ends
//     inside the chunk -> part[4 chunk .. 4 chunk + 3];
//   pass 2 (segments_write_kernel): each chunk adds up the counts of the
//     chunks before it (its first output slot) and writes its starts; chunk
//     0 also writes n, max_len (adding the documents that span chunks and the
//     last one) and cu[n] = B*S.
// Pass 2 writes only slots 0..n <= B*S, never the scratch it reads.

constexpr int kSegRound = 512;  // tokens per round: 2 tiles of 256 threads
constexpr int kSegTiles = kSegRound / 256;
constexpr int32_t kNoStart = -1;

struct WideArgs {
  const void* pos;
  int32_t* cu;
  int32_t* part;  // cu + B*S + 1: 4 int32 per chunk
  int32_t* n_out;
  int32_t* max_len;
  u32 T, C, nb;
  FastDiv S, Sl;
  u32 B;
};

template <typename PosT>
__device__ __forceinline__ bool wide_is_start(const WideArgs& a, u32 t) {
  if (t >= a.T) return false;
  const u32 b = fdiv(t, a.S), i = t - b * a.S.d;
  if (i == 0) return true;
  const u32 r = fdiv(i, a.Sl), s = i - r * a.Sl.d;
  return reinterpret_cast<const PosT*>(a.pos)[((uint64_t)r * a.B + b) * a.Sl.d + s] == 0;
}

// The start flags of tokens [base, base + kSegRound) as 4 kSegTiles masks in token
// order (mask 4 k + w holds tile k, wave w); returns this thread's flags.
template <typename PosT>
__device__ __forceinline__ unsigned round_masks(const WideArgs& a, u32 base, unsigned long long* masks) {
  bool f[kSegTiles];
#pragma unroll
  for (int k = 0; k < kSegTiles; ++k) f[k] = wide_is_start<PosT>(a, base + k * 256 + threadIdx.x);
  unsigned bits = 0;
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < kSegTiles; ++k) {
    const unsigned long long m = __ballot(f[k]);
    if ((threadIdx.x & 63) == 0) masks[4 * k + w] = m;
    bits |= (unsigned)f[k] << k;
  }
  return bits;
}

// Token of the highest set bit of mask index j (token order), or of the
// highest set bit below `lane` in mask j when lane < 64.
__device__ __forceinline__ int32_t mask_token(u32 base, int j, unsigned long long m) {
  return (int32_t)(base + (j >> 2) * 256 + (j & 3) * 64 + (63 - __clzll(m)));
}

// Last start at or before mask index j (inclusive), from the round's masks;
// kNoStart if none.
__device__ __forceinline__ int32_t last_start_upto(const unsigned long long* masks, u32 base, int j) {
  for (; j >= 0; --j)
    if (masks[j]) return mask_token(base, j, masks[j]);
  return kNoStart;
}

__device__ __forceinline__ int32_t block_reduce(int32_t x, int32_t* red, int op) {  // 0 sum, 1 max, 2 min
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int32_t y = __shfl_xor(x, off, 64);
    x = op == 0 ? x + y : (op == 1 ? max(x, y) : min(x, y));
  }
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  x = red[0];
  for (int i = 1; i < 4; ++i) x = op == 0 ? x + red[i] : (op == 1 ? max(x, red[i]) : min(x, red[i]));
  return x;
}

// The chunk's count (sum), first start (min), last start and longest inner
// document (max) over the work-group, in one pass.
__device__ __forceinline__ void block_reduce_part(int32_t& cnt, int32_t& first, int32_t& last,
                                                  int32_t& gap, int32_t* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    cnt += __shfl_xor(cnt, off, 64);
    first = min(first, __shfl_xor(first, off, 64));
    last = max(last, __shfl_xor(last, off, 64));
    gap = max(gap, __shfl_xor(gap, off, 64));
  }
  if (lane == 0) {
    red[4 * w] = cnt;
    red[4 * w + 1] = first;
    red[4 * w + 2] = last;
    red[4 * w + 3] = gap;
  }
  __syncthreads();
  cnt = red[0];
  first = red[1];
  last = red[2];
  gap = red[3];
  for (int i = 1; i < 4; ++i) {
    cnt += red[4 * i];
    first = min(first, red[4 * i + 1]);
    last = max(last, red[4 * i + 2]);
    gap = max(gap, red[4 * i + 3]);
  }
}

template <typename PosT>
__global__ __launch_bounds__(256) void segments_part_kernel(WideArgs a) {
  __shared__ unsigned long long masks[4 * kSegTiles];
  __shared__ int32_t red[16];
  const u32 c0 = blockIdx.x * a.C, c1 = min(a.T, c0 + a.C);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t cnt = 0, first = 0x7fffffff, last = kNoStart, gap = 0;
  int32_t carry = kNoStart;  // last start of the earlier rounds of this chunk
  for (u32 base = c0; base < c1; base += kSegRound) {
    __syncthreads();  // the previous round's masks are no longer read
    const unsigned bits = round_masks<PosT>(a, base, masks);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSegTiles; ++k) {
      if (!((bits >> k) & 1)) continue;
      const int32_t t = (int32_t)(base + k * 256 + threadIdx.x);
      const int j = 4 * k + w;
      const unsigned long long below = masks[j] & ((1ull << lane) - 1);
      int32_t prev = below ? mask_token(base, j, below) : last_start_upto(masks, base, j - 1);
      if (prev == kNoStart) prev = carry;
      if (prev != kNoStart) gap = max(gap, t - prev);
      ++cnt;
      first = min(first, t);
      last = max(last, t);
    }
    const int32_t l = last_start_upto(masks, base, 4 * kSegTiles - 1);
    if (l != kNoStart) carry = l;
  }
  block_reduce_part(cnt, first, last, gap, red);
  if (threadIdx.x == 0) {
    int32_t* p = a.part + 4 * blockIdx.x;
    p[0] = cnt;
    p[1] = cnt ? first : kNoStart;
    p[2] = last;
    p[3] = gap;
  }
}

template <typename PosT>
__global__ __launch_bounds__(256) void segments_write_kernel(WideArgs a) {
  __shared__ unsigned long long masks[4 * kSegTiles];
  __shared__ int32_t red[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // first output slot: the starts of the chunks before this one
  int32_t off = 0;
  for (u32 i = threadIdx.x; i < blockIdx.x; i += 256) off += a.part[4 * i];
  off = block_reduce(off, red, 0);
  if (blockIdx.x == 0) {
    // n, and max_len: the longest document inside a chunk, one that runs from
    // a chunk's first start back to the last start of an earlier chunk, and
    // the last document (to B*S).  Thread i owns chunks [i K, (i + 1) K).
    const u32 K = (a.nb + 255) / 256, i0 = min(a.nb, threadIdx.x * K), i1 = min(a.nb, i0 + K);
    int32_t n = 0, mine = kNoStart;
    for (u32 i = i0; i < i1; ++i) {
      n += a.part[4 * i];
      mine = max(mine, a.part[4 * i + 2]);
    }
    // exclusive prefix max of the chunks' last starts over the threads
    int32_t x = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x = max(x, y);
    }
    __shared__ int32_t wmax[4];
    __syncthreads();
    if (lane == 63) wmax[w] = x;
    __syncthreads();
    int32_t before = __shfl_up(x, 1, 64);
    if (lane == 0) before = kNoStart;
    for (int i = 0; i < w; ++i) before = max(before, wmax[i]);
    int32_t best = 0;
    for (u32 i = i0; i < i1; ++i) {
      const int32_t f = a.part[4 * i + 1], l = a.part[4 * i + 2];
      best = max(best, a.part[4 * i + 3]);
      if (f != kNoStart && before != kNoStart) best = max(best, f - before);
      if (l != kNoStart) before = l;
    }
    n = block_reduce(n, red, 0);
    best = block_reduce(best, red, 1);
    int32_t lastall = block_reduce(mine, red, 1);
    if (threadIdx.x == 0) {
      if (lastall != kNoStart) best = max(best, (int32_t)a.T - lastall);
      *a.n_out = n;
      *a.max_len = best;
      a.cu[n] = (int32_t)a.T;
    }
  }
  const u32 c0 = blockIdx.x * a.C, c1 = min(a.T, c0 + a.C);
  for (u32 base = c0; base < c1; base += kSegRound) {
    __syncthreads();
    const unsigned bits = round_masks<PosT>(a, base, masks);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSegTiles; ++k) {
      if (!((bits >> k) & 1)) continue;
      const int j = 4 * k + w;
      int32_t r = __popcll(masks[j] & ((1ull << lane) - 1));
      for (int i = 0; i < j; ++i) r += __popcll(masks[i]);
      a.cu[off + r] = (int32_t)(base + k * 256 + threadIdx.x);
    }
    int32_t tot = 0;
    for (int i = 0; i < 4 * kSegTiles; ++i) tot += __popcll(masks[i]);
    off += tot;
  }
}

// Tokens per chunk of the wide scan for T tokens, and the chunk count.
inline u32 seg_wide_chunk(u32 T) {
  const u32 rounds = (T + kSegRound - 1) / kSegRound;
  return kSegRound * ((rounds + kSegWideBlocks - 1) / kSegWideBlocks);
}

int64_t segments_scratch_slots(int B, int S) {
  const u32 T = (u32)B * (u32)S, C = seg_wide_chunk(T);
  return 4 * (int64_t)((T + C - 1) / C);
}

hipError_t segments_launch(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
                           int64_t cu_capacity, int32_t* n_seqs, int32_t* max_len, hipStream_t st) {
  const int64_t T = (int64_t)B * S;
  if (cu_capacity >= T + 1 + segments_scratch_slots(B, S)) {
    WideArgs a;
    a.pos = pos;
    a.cu = cu;
    a.part = cu + T + 1;
    a.n_out = n_seqs;
    a.max_len = max_len;
    a.T = (u32)T;
    a.C = seg_wide_chunk(a.T);
    a.nb = (a.T + a.C - 1) / a.C;
    a.S = make_fastdiv(S);
    a.Sl = make_fastdiv(S / P);
    a.B = B;
    ProfScope prof("cu_seqlens", st);
    if (pos_bytes == 8) {
      hipLaunchKernelGGL(segments_part_kernel<int64_t>, dim3(a.nb), dim3(256), 0, st, a);
      hipLaunchKernelGGL(segments_write_kernel<int64_t>, dim3(a.nb), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL(segments_part_kernel<int32_t>, dim3(a.nb), dim3(256), 0, st, a);
      hipLaunchKernelGGL(segments_write_kernel<int32_t>, dim3(a.nb), dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  return segments_launch_one(pos, pos_bytes, P, B, S, cu, n_seqs, max_len, st);
}

// One work-group (no scratch needed): the kernel above.
hipError_t segments_launch_one(const void* pos, int pos_bytes, int P, int B, int S, int32_t* cu,
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

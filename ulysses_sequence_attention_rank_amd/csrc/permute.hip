// Layout permutation of the Ulysses all-to-all, all P simulated ranks at once.
//
// pack:   seq [P][B][S/P][H][D] -> head [P][B][S][H/P][D]
// unpack: head -> seq
// For a fixed (rank c, batch b, gathered token t) the H/P*D elements of the
// head layout are one contiguous run, and so are the source elements (heads
// c*H/P .. of token t's row in its sequence shard).  The copy therefore moves
// runs of H/P*D elements with coalesced vector loads and stores on both
// sides.  It is bound by HBM bandwidth: every byte is read once and written
// once.
#include "common.hpp"
#include "launch.hpp"

namespace uly {

struct PermArgs {
  const char* src;
  char* dst;
  u32 n_chunks;     // total vector chunks
  u32 run_bytes;    // H/P * D * elem_bytes
  FastDiv cpr;      // chunks per run
  FastDiv S, B, Sl, P;
};

template <int VW>
struct VecT;
template <> struct VecT<16> { typedef u32x4 T; };
template <> struct VecT<8> { typedef u32x2 T; };
template <> struct VecT<4> { typedef u32 T; };
template <> struct VecT<2> { typedef unsigned short T; };
template <> struct VecT<1> { typedef unsigned char T; };

constexpr int kPermThreads = 256;
constexpr int kPermUnroll = 4;

// Source run of destination run `run` (pack direction):
//   dst run (c, b, t) -> src run (r = t / Sl, b, s = t % Sl, c)
__device__ __forceinline__ u32 pack_src_run(u32 run, const PermArgs& a) {
  const u32 cb = fdiv(run, a.S), t = run - cb * a.S.d;
  const u32 c = fdiv(cb, a.B), b = cb - c * a.B.d;
  const u32 r = fdiv(t, a.Sl), s = t - r * a.Sl.d;
  return ((r * a.B.d + b) * a.Sl.d + s) * a.P.d + c;
}

// Source run of destination run `run` (unpack direction):
//   dst run (r, b, s, c) -> src run (c, b, t = r * Sl + s)
__device__ __forceinline__ u32 unpack_src_run(u32 run, const PermArgs& a) {
  const u32 x = fdiv(run, a.P), c = run - x * a.P.d;
  const u32 y = fdiv(x, a.Sl), s = x - y * a.Sl.d;
  const u32 r = fdiv(y, a.B), b = y - r * a.B.d;
  return (c * a.B.d + b) * a.S.d + r * a.Sl.d + s;
}

template <int VW, bool PACK>
__global__ __launch_bounds__(kPermThreads) void permute_kernel(PermArgs a) {
  typedef typename VecT<VW>::T V;
  V val[kPermUnroll];
  uint64_t dst_off[kPermUnroll];
  const u32 base = blockIdx.x * (kPermThreads * kPermUnroll) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const u32 i = base + u * kPermThreads;
    dst_off[u] = ~0ull;
    if (i < a.n_chunks) {
      const u32 run = fdiv(i, a.cpr), off = (i - run * a.cpr.d) * VW;
      const u32 srun = PACK ? pack_src_run(run, a) : unpack_src_run(run, a);
      val[u] = *reinterpret_cast<const V*>(a.src + (uint64_t)srun * a.run_bytes + off);
      dst_off[u] = (uint64_t)run * a.run_bytes + off;
    }
  }
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u)
    if (dst_off[u] != ~0ull) __builtin_nontemporal_store(val[u], reinterpret_cast<V*>(a.dst + dst_off[u]));
}

template <bool PACK>
static hipError_t launch_perm(int vw, const PermArgs& a, hipStream_t st) {
  const u32 per_block = kPermThreads * kPermUnroll;
  const dim3 grid((a.n_chunks + per_block - 1) / per_block), block(kPermThreads);
  ProfScope prof(PACK ? "a2a_pack" : "a2a_unpack", st);
  switch (vw) {
    case 16: hipLaunchKernelGGL((permute_kernel<16, PACK>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((permute_kernel<8, PACK>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((permute_kernel<4, PACK>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((permute_kernel<2, PACK>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((permute_kernel<1, PACK>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t permute_launch(bool pack, const void* src, void* dst, int P, int B, int S, int H, int D,
                          int eb, hipStream_t st) {
  const uint64_t run_bytes = (uint64_t)(H / P) * D * eb;
  int vw = 16;
  while (vw > 1 && (run_bytes % vw || ((uintptr_t)src % vw) || ((uintptr_t)dst % vw))) vw >>= 1;
  PermArgs a;
  a.src = (const char*)src;
  a.dst = (char*)dst;
  const uint64_t total = (uint64_t)P * B * S * run_bytes;
  a.n_chunks = (u32)(total / vw);
  a.run_bytes = (u32)run_bytes;
  a.cpr = make_fastdiv((u32)(run_bytes / vw));
  a.S = make_fastdiv(S);
  a.B = make_fastdiv(B);
  a.Sl = make_fastdiv(S / P);
  a.P = make_fastdiv(P);
  if (a.n_chunks == 0) return hipSuccess;
  return pack ? launch_perm<true>(vw, a, st) : launch_perm<false>(vw, a, st);
}

}  // namespace uly

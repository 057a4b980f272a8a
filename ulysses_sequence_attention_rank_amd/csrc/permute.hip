// Layout permutation of the Ulysses all-to-all, all P simulated ranks at once
// (and up to four tensors of one exchange, e.g. Q, K, V, in one launch).
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

constexpr int kMaxTensors = 4;

// Up to kMaxTensors tensors of equal P, B, S, D (each its own H) in one
// launch: tensor i owns blocks [blk0[i], blk0[i+1]) of the grid.
struct PermArgs {
  int n;
  const char* src[kMaxTensors];
  char* dst[kMaxTensors];
  u32 n_chunks[kMaxTensors];   // vector chunks of the tensor
  u32 run_bytes[kMaxTensors];  // H/P * D * elem_bytes
  FastDiv cpr[kMaxTensors];    // chunks per run
  u32 src_runs[kMaxTensors];   // runs per token row of the sequence shards (P, or H replicated)
  FastDiv rep[kMaxTensors];    // ranks sharing a run (1, or P / H replicated)
  u32 blk0[kMaxTensors + 1];
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
constexpr int kPermUnroll = 1;  // one 16-byte chunk a thread: more waves in flight measured best

// Source run of destination run `run` (pack direction):
//   dst run (c, b, t) -> src run (r = t / Sl, b, s = t % Sl, c / rep)
// (a run is H/P heads; with fewer heads than ranks it is one head, which
// the rep = P/H ranks of its query group all receive)
__device__ __forceinline__ u32 pack_src_run(u32 run, const PermArgs& a, int ti) {
  const u32 cb = fdiv(run, a.S), t = run - cb * a.S.d;
  const u32 c = fdiv(cb, a.B), b = cb - c * a.B.d;
  const u32 r = fdiv(t, a.Sl), s = t - r * a.Sl.d;
  return ((r * a.B.d + b) * a.Sl.d + s) * a.src_runs[ti] + fdiv(c, a.rep[ti]);
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
  // this block's tensor (uniform)
  int ti = 0;
#pragma unroll
  for (int i = 1; i < kMaxTensors; ++i)
    if (i < a.n && blockIdx.x >= a.blk0[i]) ti = i;
  const char* src = a.src[ti];
  char* dst = a.dst[ti];
  const u32 n_chunks = a.n_chunks[ti], run_bytes = a.run_bytes[ti];
  const FastDiv cpr = a.cpr[ti];
  V val[kPermUnroll];
  uint64_t dst_off[kPermUnroll];
  const u32 base = (blockIdx.x - a.blk0[ti]) * (kPermThreads * kPermUnroll) + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u) {
    const u32 i = base + u * kPermThreads;
    dst_off[u] = ~0ull;
    if (i < n_chunks) {
      const u32 run = fdiv(i, cpr), off = (i - run * cpr.d) * VW;
      const u32 srun = PACK ? pack_src_run(run, a, ti) : unpack_src_run(run, a);
      val[u] = *reinterpret_cast<const V*>(src + (uint64_t)srun * run_bytes + off);
      dst_off[u] = (uint64_t)run * run_bytes + off;
    }
  }
#pragma unroll
  for (int u = 0; u < kPermUnroll; ++u)
    if (dst_off[u] != ~0ull) __builtin_nontemporal_store(val[u], reinterpret_cast<V*>(dst + dst_off[u]));
}

template <bool PACK>
static hipError_t launch_perm(int vw, const PermArgs& a, hipStream_t st) {
  const dim3 grid(a.blk0[a.n]), block(kPermThreads);
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

hipError_t permute_launch(bool pack, int n, const void* const* src, void* const* dst, const int* H,
                          int P, int B, int S, int D, int eb, hipStream_t st) {
  // heads per run: H/P, or one (replicated) when there are fewer heads than ranks
  auto run_heads = [&](int i) { return H[i] >= P ? H[i] / P : 1; };
  // the widest vector every tensor's runs and pointers allow
  int vw = 16;
  for (int i = 0; i < n; ++i) {
    const uint64_t run_bytes = (uint64_t)run_heads(i) * D * eb;
    while (vw > 1 && (run_bytes % vw || ((uintptr_t)src[i] % vw) || ((uintptr_t)dst[i] % vw))) vw >>= 1;
  }
  PermArgs a = {};
  a.n = n;
  a.S = make_fastdiv(S);
  a.B = make_fastdiv(B);
  a.Sl = make_fastdiv(S / P);
  a.P = make_fastdiv(P);
  const u32 per_block = kPermThreads * kPermUnroll;
  a.blk0[0] = 0;
  for (int i = 0; i < n; ++i) {
    const uint64_t run_bytes = (uint64_t)run_heads(i) * D * eb;
    a.src_runs[i] = H[i] >= P ? P : H[i];
    a.rep[i] = make_fastdiv(H[i] >= P ? 1 : P / H[i]);
    a.src[i] = (const char*)src[i];
    a.dst[i] = (char*)dst[i];
    a.n_chunks[i] = (u32)((uint64_t)P * B * S * run_bytes / vw);
    a.run_bytes[i] = (u32)run_bytes;
    a.cpr[i] = make_fastdiv((u32)(run_bytes / vw));
    a.blk0[i + 1] = a.blk0[i] + (a.n_chunks[i] + per_block - 1) / per_block;
  }
  if (a.blk0[n] == 0) return hipSuccess;
  return pack ? launch_perm<true>(vw, a, st) : launch_perm<false>(vw, a, st);
}

// Gradient of the replicated pack: head [P][B][S][1][D] (bf16, or fp32 when
// the backward kept the replicas' dK/dV unrounded) -> seq [P][B][S/P][H][D]
// bf16, each head the fp32 sum of its rep = P/H replicas in rank order,
// rounded once to bf16.  One thread per 8 elements (D % 8 == 0).
struct RepArgs {
  const void* head;
  __bf16* seq;
  u32 n8;  // 8-element chunks of seq
  FastDiv d8, H, Sl, B;
  int rep, S, D;
};

template <bool F32>
__global__ __launch_bounds__(256) void reduce_replicated_kernel(RepArgs a) {
  const u32 i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n8) return;
  // seq chunk i = (((r * B + b) * Sl + s) * H + h) * D/8 + dc
  const u32 x = fdiv(i, a.d8), dc = i - x * a.d8.d;
  const u32 y = fdiv(x, a.H), h = x - y * a.H.d;
  const u32 z = fdiv(y, a.Sl), s = y - z * a.Sl.d;
  const u32 r = fdiv(z, a.B), b = z - r * a.B.d;
  const u32 t = r * a.Sl.d + s;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < a.rep; ++j) {
    const u32 c = h * a.rep + j;
    const uint64_t e = ((uint64_t)(c * a.B.d + b) * a.S + t) * a.D + 8 * dc;
    if (F32) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.head) + e);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.head) + e + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] += w0[k];
        acc[4 + k] += w1[k];
      }
    } else {
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const __bf16*>(a.head) + e);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += bf16_lo(w[k]);
        acc[2 * k + 1] += bf16_hi(w[k]);
      }
    }
  }
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
  *reinterpret_cast<u32x4*>(a.seq + (uint64_t)i * 8) = o;
}

hipError_t reduce_replicated_launch(const void* head, bool head_f32, void* seq, int P, int B, int S,
                                    int H, int D, hipStream_t st) {
  RepArgs a;
  a.head = head;
  a.seq = (__bf16*)seq;
  a.n8 = (u32)((uint64_t)B * S * H * D / 8);
  a.d8 = make_fastdiv(D / 8);
  a.H = make_fastdiv(H);
  a.Sl = make_fastdiv(S / P);
  a.B = make_fastdiv(B);
  a.rep = P / H;
  a.S = S;
  a.D = D;
  if (a.n8 == 0) return hipSuccess;
  ProfScope prof("a2a_reduce_replicated", st);
  if (head_f32)
    hipLaunchKernelGGL(reduce_replicated_kernel<true>, dim3((a.n8 + 255) / 256), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(reduce_replicated_kernel<false>, dim3((a.n8 + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace uly

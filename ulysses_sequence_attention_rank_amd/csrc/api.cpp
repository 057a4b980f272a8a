// C ABI of the per-rank Ulysses hot path: argument checks, workspace layout
// and kernel dispatch.  Declared (with the meaning of every argument) in
// include/ulysses.h.
#include <algorithm>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ulysses.h"
#include "attn_common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return ULY_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ULY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxI32 = 2147483647;

int check_permute(const void* src, const void* dst, int P, int B, int S, int H, int D, int eb) {
  if (!src || !dst) return fail(ULY_ERR_NULL, "NULL tensor pointer");
  if (P <= 0 || B <= 0 || S <= 0 || H <= 0 || D <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (P=%d B=%d S=%d H=%d D=%d)", P, B, S, H, D);
  if (S % P) return fail(ULY_ERR_SHAPE, "S=%d is not divisible by P=%d", S, P);
  if (H % P) return fail(ULY_ERR_HEADS, "H=%d heads are not divisible by P=%d ranks", H, P);
  if (eb != 1 && eb != 2 && eb != 4 && eb != 8)
    return fail(ULY_ERR_UNSUPPORTED, "elem_bytes=%d not in {1,2,4,8}", eb);
  const int64_t elems = (int64_t)B * S * H * D;
  if (elems >= kMaxI32 || (int64_t)P * B * S >= kMaxI32)
    return fail(ULY_ERR_SHAPE, "tensor of %lld elements exceeds 2^31 - 1", (long long)elems);
  if (!aligned(src, eb) || !aligned(dst, eb))
    return fail(ULY_ERR_ALIGN, "pointers must be aligned to elem_bytes=%d", eb);
  const uintptr_t a0 = (uintptr_t)src, a1 = a0 + elems * eb, b0 = (uintptr_t)dst, b1 = b0 + elems * eb;
  if (a0 < b1 && b0 < a1) return fail(ULY_ERR_UNSUPPORTED, "source and destination overlap");
  return ok();
}

int check_attn(const void* q, const void* k, const void* v, const int32_t* cu, const int32_t* n_seqs,
               int B, int S, int hq, int hkv, int D, float scale, int wl, int wr) {
  if (!q || !k || !v) return fail(ULY_ERR_NULL, "NULL q/k/v");
  if (cu && !n_seqs) return fail(ULY_ERR_NULL, "cu_seqlens given without n_seqs");
  if (B <= 0 || S <= 0 || hq <= 0 || hkv <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (B=%d S=%d hq=%d hkv=%d)", B, S, hq, hkv);
  if (hq % hkv) return fail(ULY_ERR_HEADS, "hq=%d query heads not divisible by hkv=%d", hq, hkv);
  if (D != 64 && D != 128) return fail(ULY_ERR_UNSUPPORTED, "head_dim D=%d not in {64,128}", D);
  if (wl < -1 || wr < -1)
    return fail(ULY_ERR_UNSUPPORTED, "window (%d,%d): values below -1 are not a window", wl, wr);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(ULY_ERR_UNSUPPORTED, "softmax_scale must be finite and > 0");
  if ((int64_t)B * S * hq * D >= kMaxI32 * 8ll || (int64_t)B * S * hq >= kMaxI32)
    return fail(ULY_ERR_SHAPE, "problem too large for 32-bit row indices");
  return ok();
}

// RowMap of the contiguous head layout [B][S][H][D].
// RowMap of a uly_layout for a tensor of H heads (checked: shards divide S,
// non-negative strides, 16-byte rows, every element addressable).
int make_map(const uly_layout* L, int B, int S, int H, int D, const char* name, uly::RowMap& m) {
  if (!L) return fail(ULY_ERR_NULL, "NULL %s layout", name);
  if (L->shards < 1 || S % L->shards)
    return fail(ULY_ERR_SHAPE, "%s layout: %d shards do not divide S=%d", name, L->shards, S);
  if (L->batch < 0 || L->shard < 0 || L->token <= 0 || L->head < 0)
    return fail(ULY_ERR_SHAPE, "%s layout: strides must be >= 0 (token > 0)", name);
  if (L->batch % 8 || L->shard % 8 || L->token % 8 || L->head % 8)
    return fail(ULY_ERR_ALIGN, "%s layout: strides must be multiples of 8 elements (16-byte rows)", name);
  const int Sl = S / L->shards;
  const double span = (double)(B - 1) * L->batch + (double)(L->shards - 1) * L->shard +
                      (double)(Sl - 1) * L->token + (double)(H - 1) * L->head + D;
  if (span >= 9.0e18) return fail(ULY_ERR_SHAPE, "%s layout: offsets exceed 64 bits", name);
  m = uly::RowMap{};
  m.batch = L->batch;
  m.shard = L->shard;
  m.token = L->token;
  m.head = L->head;
  m.S = uly::make_fastdiv(S);
  m.Sl = uly::make_fastdiv(Sl);
  // one stride per token (and 64-row tiles addressable with 32-bit offsets)
  m.uniform = (B == 1 || L->batch == (int64_t)S * L->token) &&
              (L->shards == 1 || L->shard == (int64_t)Sl * L->token) && L->token < (1 << 24);
  m.s0 = 0;
  m.s_len = S;
  return ok();
}

uly_layout head_layout(int S, int H, int D) {
  uly_layout L;
  L.shards = 1;
  L.batch = (int64_t)S * H * D;
  L.shard = 0;
  L.token = (int64_t)H * D;
  L.head = D;
  return L;
}

uly::AttnArgs make_args(const void* q, const void* k, const void* v, const float* sink,
                        const int32_t* cu, const int32_t* n_seqs, int B, int S, int hq, int hkv,
                        float scale, int causal, int wl, int wr) {
  uly::AttnArgs a = {};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.sink = sink;
  a.cu = cu;
  a.n_seqs = cu ? n_seqs : nullptr;
  a.B = B;
  a.S = S;
  a.T = B * S;
  a.hq = hq;
  a.hkv = hkv;
  a.G = hq / hkv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.causal = causal ? 1 : 0;
  a.wl = wl;
  a.wr = wr;
  a.nsplit = 1;
  a.k_lo_s = 0;
  a.k_hi_s = S;
  a.kt_lo = 0;
  a.kt_hi = B * S;
  a.o_f32 = 0;
  return a;
}

constexpr int kDsinkParts = 64;

size_t align256(size_t x);

// fp32 partial sums of the split backward kernels (they run one after the
// other, so one buffer serves both): max(dQ partials, dK+dV partials) plus
// the split sums of P dP.
// The dK/dV balanced schedule's part slots (2 W of dK and dV for 128 keys)
// share that buffer; its key-tile prefix follows it.
size_t bal_slot_bytes(int B, int S, int hkv, int D) {
  const int W = uly::dkdv_bal_workgroups(B, S, hkv);
  return W > 0 ? (size_t)2 * W * 2 * 128 * D * 4 : 0;
}
size_t split_main_bytes(int B, int S, int hq, int hkv, int D) {
  const size_t T = (size_t)B * S;
  const int nq = uly::qtile_splits(B, S, hq, D, true), nk = uly::dkdv_splits(B, S, hkv, D, true);
  size_t part = bal_slot_bytes(B, S, hkv, D);
  if (nq > 1 && (size_t)nq * T * hq * D * 4 > part) part = (size_t)nq * T * hq * D * 4;
  if (nk > 1 && (size_t)nk * 2 * T * hkv * D * 4 > part) part = (size_t)nk * 2 * T * hkv * D * 4;
  return align256(part) + align256((size_t)(uly::kBalMaxTilesHost + 1) * 4);
}
size_t split_part_bytes(int B, int S, int hq, int hkv, int D) {
  const size_t T = (size_t)B * S;
  const int nq = uly::qtile_splits(B, S, hq, D, true);
  const size_t pdp = nq > 1 ? (size_t)nq * T * hq * 4 : 0;
  return split_main_bytes(B, S, hq, hkv, D) + align256(pdp);
}

// ---- optional per-kernel timing: a HIP event before and after each launch
struct Prof {
  bool on = false;
  bool open = false;  // a start event is recorded, its stop is not
  size_t n = 0;       // events recorded
  std::vector<hipEvent_t> ev;
  std::vector<const char*> name;  // one per launch
};
Prof g_prof;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace uly {
void prof_mark(const char* name, hipStream_t st) {
  Prof& p = g_prof;
  if (!p.on) return;
  if (name != nullptr) {
    if (p.n + 2 > p.ev.size()) return;  // full: later launches are not recorded
    p.name[p.n / 2] = name;
    p.open = hipEventRecord(p.ev[p.n], st) == hipSuccess;
  } else if (p.open) {
    if (hipEventRecord(p.ev[p.n + 1], st) == hipSuccess) p.n += 2;
    p.open = false;
  }
}
}  // namespace uly

extern "C" {

int ulysses_profile_start(int max_launches) {
  if (max_launches <= 0) return fail(ULY_ERR_SHAPE, "max_launches must be positive");
  Prof& p = g_prof;
  const size_t need = 2 * (size_t)max_launches;
  while (p.ev.size() < need) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return hip_status(err, "hipEventCreate");
    p.ev.push_back(e);
  }
  p.name.assign(p.ev.size() / 2, nullptr);
  p.n = 0;
  p.open = false;
  p.on = true;
  return ok();
}

int ulysses_calibrate_mfma(float* out, size_t out_bytes, int iters, int mode, void* stream) {
  if (!out) return fail(ULY_ERR_NULL, "NULL out");
  const size_t need = (size_t)uly::kCalibBlocks * 256 * sizeof(float);
  if (out_bytes < need) return fail(ULY_ERR_CAPACITY, "out of %zu bytes < %zu needed", out_bytes, need);
  if (iters <= 0 || iters % 8)
    return fail(ULY_ERR_SHAPE, "iters=%d: a positive multiple of 8", iters);
  if (mode < 0 || mode > 5) return fail(ULY_ERR_UNSUPPORTED, "mode=%d: 0 to 5", mode);
  if (!aligned(out, 4)) return fail(ULY_ERR_ALIGN, "out needs 4-byte alignment");
  return hip_status(uly::calib_mfma_launch(out, iters, mode, (hipStream_t)stream),
                    "ulysses_calibrate_mfma launch");
}

size_t ulysses_calibrate_mfma_flops(int iters) {
  // 4 waves a work-group, 8 accumulators a wave, 2*32*32*16 FLOPs a product
  return iters > 0 ? (size_t)uly::kCalibBlocks * 4 * (size_t)iters * 8 * 32768 : 0;
}

int ulysses_profile_stop(void) {
  g_prof.on = false;
  return ok();
}

int ulysses_profile_report(char* buf, size_t buf_bytes) {
  Prof& p = g_prof;
  if (!buf || buf_bytes == 0) return fail(ULY_ERR_NULL, "NULL report buffer");
  struct Agg {
    std::string name;
    int count;
    double total_ms, min_ms, max_ms;
  };
  std::vector<Agg> agg;
  for (size_t i = 0; i + 1 < p.n; i += 2) {
    hipError_t err = hipEventSynchronize(p.ev[i + 1]);
    if (err != hipSuccess) return hip_status(err, "hipEventSynchronize");
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, p.ev[i], p.ev[i + 1]);
    if (err != hipSuccess) return hip_status(err, "hipEventElapsedTime");
    const char* nm = p.name[i / 2];
    Agg* a = nullptr;
    for (auto& x : agg)
      if (x.name == nm) a = &x;
    if (!a) {
      agg.push_back({nm, 0, 0.0, 1e30, 0.0});
      a = &agg.back();
    }
    a->count++;
    a->total_ms += ms;
    a->min_ms = ms < a->min_ms ? ms : a->min_ms;
    a->max_ms = ms > a->max_ms ? ms : a->max_ms;
  }
  std::string out;
  char line[256];
  for (auto& x : agg) {
    snprintf(line, sizeof(line), "%s %d %.6f %.6f %.6f\n", x.name.c_str(), x.count, x.total_ms,
             x.min_ms, x.max_ms);
    out += line;
  }
  if (out.size() + 1 > buf_bytes) return fail(ULY_ERR_CAPACITY, "report needs %zu bytes", out.size() + 1);
  memcpy(buf, out.c_str(), out.size() + 1);
  ok();
  return (int)(p.n / 2);
}

int ulysses_a2a_pack(const void* seq_shards, void* head_shards, int P, int B, int S, int H, int D,
                     int elem_bytes, void* stream) {
  int rc = check_permute(seq_shards, head_shards, P, B, S, H, D, elem_bytes);
  if (rc) return rc;
  void* dst = head_shards;
  return hip_status(uly::permute_launch(true, 1, &seq_shards, &dst, &H, P, B, S, D, elem_bytes,
                                        (hipStream_t)stream),
                    "ulysses_a2a_pack launch");
}

int ulysses_a2a_unpack(const void* head_shards, void* seq_shards, int P, int B, int S, int H,
                       int D, int elem_bytes, void* stream) {
  int rc = check_permute(head_shards, seq_shards, P, B, S, H, D, elem_bytes);
  if (rc) return rc;
  void* dst = seq_shards;
  return hip_status(uly::permute_launch(false, 1, &head_shards, &dst, &H, P, B, S, D, elem_bytes,
                                        (hipStream_t)stream),
                    "ulysses_a2a_unpack launch");
}

// ---- sequence-tiled MLP
size_t ulysses_tiled_mlp_workspace_bytes(int T, int H, int I, int tile) {
  if (T <= 0 || H <= 0 || I <= 0 || tile <= 0) return 0;
  const size_t rows = (size_t)std::min(T, tile);
  // one tile's G, U, h (each [rows][I]) and dG | dU ([rows][2I]), bf16
  return align256(rows * I * 2 * 5);
}

static int check_mlp(const void* x, const void* wg, const void* wu, const void* wd, int T, int H,
                     int I, int tile, void* ws, size_t ws_bytes) {
  if (!x || !wg || !wu || !wd) return fail(ULY_ERR_NULL, "NULL x or weight");
  if (T <= 0 || H <= 0 || I <= 0 || tile <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (T=%d H=%d I=%d tile=%d)", T, H, I, tile);
  if (H % 128 || I % 128)
    return fail(ULY_ERR_UNSUPPORTED, "H=%d and I=%d must be multiples of 128", H, I);
  // a 256-row operand tile of the widest operand (4 I bytes a row) must span
  // fewer than 2^31 bytes
  if ((int64_t)T * H >= kMaxI32 * 8ll || (int64_t)I * H >= kMaxI32 * 8ll || H > (1 << 20) ||
      I > (1 << 20))
    return fail(ULY_ERR_SHAPE, "problem too large (H=%d, I=%d: at most 2^20 each)", H, I);
  const size_t need = ulysses_tiled_mlp_workspace_bytes(T, H, I, tile);
  if (!ws) return fail(ULY_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(ULY_ERR_CAPACITY, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned(x, 16) || !aligned(wg, 16) || !aligned(wu, 16) || !aligned(wd, 16) || !aligned(ws, 256))
    return fail(ULY_ERR_ALIGN, "tensors need 16-byte alignment, workspace 256-byte");
  return ok();
}

int ulysses_tiled_mlp_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          void* y, int T, int H, int I, int tile, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int rc = check_mlp(x, w_gate, w_up, w_down, T, H, I, tile, workspace, workspace_bytes);
  if (rc) return rc;
  if (!y) return fail(ULY_ERR_NULL, "NULL y");
  if (!aligned(y, 16)) return fail(ULY_ERR_ALIGN, "y needs 16-byte alignment");
  uly::MlpArgs p = {};
  p.x = (const __bf16*)x, p.wg = (const __bf16*)w_gate, p.wu = (const __bf16*)w_up;
  p.wd = (const __bf16*)w_down, p.y = (__bf16*)y, p.ws = workspace;
  p.T = T, p.H = H, p.I = I, p.tile = std::min(T, tile);
  return hip_status(uly::mlp_fwd_launch(p, (hipStream_t)stream), "ulysses_tiled_mlp_fwd launch");
}

int ulysses_tiled_mlp_bwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          const void* dy, void* dx, float* dw_gate, float* dw_up, float* dw_down,
                          int T, int H, int I, int tile, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = check_mlp(x, w_gate, w_up, w_down, T, H, I, tile, workspace, workspace_bytes);
  if (rc) return rc;
  if (!dy || !dx || !dw_gate || !dw_up || !dw_down) return fail(ULY_ERR_NULL, "NULL dy, dx or dw");
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(dw_gate, 16) || !aligned(dw_up, 16) ||
      !aligned(dw_down, 16))
    return fail(ULY_ERR_ALIGN, "tensors need 16-byte alignment");
  uly::MlpArgs p = {};
  p.x = (const __bf16*)x, p.wg = (const __bf16*)w_gate, p.wu = (const __bf16*)w_up;
  p.wd = (const __bf16*)w_down, p.dy = (const __bf16*)dy, p.dx = (__bf16*)dx;
  p.dwg = dw_gate, p.dwu = dw_up, p.dwd = dw_down, p.ws = workspace;
  p.T = T, p.H = H, p.I = I, p.tile = std::min(T, tile);
  return hip_status(uly::mlp_bwd_launch(p, (hipStream_t)stream), "ulysses_tiled_mlp_bwd launch");
}

int check_replicated(const void* a, const void* b, int P, int B, int S, int H, int D, int eb) {
  if (!a || !b) return fail(ULY_ERR_NULL, "NULL tensor pointer");
  if (P <= 0 || B <= 0 || S <= 0 || H <= 0 || D <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (P=%d B=%d S=%d H=%d D=%d)", P, B, S, H, D);
  if (S % P) return fail(ULY_ERR_SHAPE, "S=%d is not divisible by P=%d", S, P);
  if (H > P || P % H)
    return fail(ULY_ERR_HEADS, "replication needs H=%d heads dividing P=%d ranks", H, P);
  if (eb != 1 && eb != 2 && eb != 4 && eb != 8)
    return fail(ULY_ERR_UNSUPPORTED, "elem_bytes=%d not in {1,2,4,8}", eb);
  const int64_t elems = (int64_t)P * B * S * D;  // the replicated side, the larger
  if (elems >= kMaxI32) return fail(ULY_ERR_SHAPE, "tensor of %lld elements exceeds 2^31 - 1",
                                    (long long)elems);
  if (!aligned(a, eb) || !aligned(b, eb))
    return fail(ULY_ERR_ALIGN, "pointers must be aligned to elem_bytes=%d", eb);
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  const uintptr_t na = (uintptr_t)elems * eb, nb = (uintptr_t)B * S * H * D * eb;
  if (a0 < b0 + nb && b0 < a0 + na) return fail(ULY_ERR_UNSUPPORTED, "the two buffers overlap");
  return ok();
}

int ulysses_a2a_pack_replicated(const void* seq_shards, void* head_shards, int P, int B, int S,
                                int H, int D, int elem_bytes, void* stream) {
  int rc = check_replicated(head_shards, seq_shards, P, B, S, H, D, elem_bytes);
  if (rc) return rc;
  void* dst = head_shards;
  return hip_status(uly::permute_launch(true, 1, &seq_shards, &dst, &H, P, B, S, D, elem_bytes,
                                        (hipStream_t)stream),
                    "ulysses_a2a_pack_replicated launch");
}

int ulysses_a2a_reduce_replicated(const void* head_shards, int in_elem_bytes, void* seq_shards,
                                  int P, int B, int S, int H, int D, void* stream) {
  if (in_elem_bytes != 2 && in_elem_bytes != 4)
    return fail(ULY_ERR_UNSUPPORTED, "in_elem_bytes=%d not 2 (bf16) or 4 (fp32)", in_elem_bytes);
  int rc = check_replicated(head_shards, seq_shards, P, B, S, H, D, 2);
  if (rc) return rc;
  if (D % 8) return fail(ULY_ERR_UNSUPPORTED, "D=%d is not a multiple of 8", D);
  if (!aligned(head_shards, 16) || !aligned(seq_shards, 16))
    return fail(ULY_ERR_ALIGN, "the gradient buffers need 16-byte alignment");
  const uintptr_t a0 = (uintptr_t)head_shards, b0 = (uintptr_t)seq_shards;
  const uintptr_t na = (uintptr_t)P * B * S * D * in_elem_bytes, nb = (uintptr_t)B * S * H * D * 2;
  if (a0 < b0 + nb && b0 < a0 + na) return fail(ULY_ERR_UNSUPPORTED, "the two buffers overlap");
  return hip_status(uly::reduce_replicated_launch(head_shards, in_elem_bytes == 4, seq_shards, P,
                                                  B, S, H, D, (hipStream_t)stream),
                    "ulysses_a2a_reduce_replicated launch");
}

static int permute_multi(bool pack, int n, const void* const* src, void* const* dst, const int* H,
                         int P, int B, int S, int D, int elem_bytes, void* stream, const char* what) {
  if (!src || !dst || !H) return fail(ULY_ERR_NULL, "NULL src/dst/H array");
  if (n < 1 || n > 4) return fail(ULY_ERR_UNSUPPORTED, "n=%d tensors not in 1..4", n);
  for (int i = 0; i < n; ++i) {
    int rc = check_permute(src[i], dst[i], P, B, S, H[i], D, elem_bytes);
    if (rc) return rc;
  }
  // no destination may overlap any source or another destination
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      const uintptr_t ei = (uintptr_t)B * S * H[i] * D * elem_bytes, ej = (uintptr_t)B * S * H[j] * D * elem_bytes;
      const uintptr_t d0 = (uintptr_t)dst[i], s0 = (uintptr_t)src[j], d1 = (uintptr_t)dst[j];
      if (d0 < s0 + ej && s0 < d0 + ei)
        return fail(ULY_ERR_UNSUPPORTED, "destination %d overlaps source %d", i, j);
      if (i != j && d0 < d1 + ej && d1 < d0 + ei)
        return fail(ULY_ERR_UNSUPPORTED, "destinations %d and %d overlap", i, j);
    }
  return hip_status(uly::permute_launch(pack, n, src, dst, H, P, B, S, D, elem_bytes,
                                        (hipStream_t)stream),
                    what);
}

int ulysses_a2a_pack_multi(int n, const void* const* seq_shards, void* const* head_shards,
                           const int* H, int P, int B, int S, int D, int elem_bytes, void* stream) {
  return permute_multi(true, n, seq_shards, head_shards, H, P, B, S, D, elem_bytes, stream,
                       "ulysses_a2a_pack_multi launch");
}

int ulysses_a2a_unpack_multi(int n, const void* const* head_shards, void* const* seq_shards,
                             const int* H, int P, int B, int S, int D, int elem_bytes, void* stream) {
  return permute_multi(false, n, head_shards, seq_shards, H, P, B, S, D, elem_bytes, stream,
                       "ulysses_a2a_unpack_multi launch");
}

int ulysses_cu_seqlens_capacity(int B, int S) {
  if (B <= 0 || S <= 0 || (int64_t)B * S >= kMaxI32) return 0;
  const int64_t c = (int64_t)B * S + 1 + uly::segments_scratch_slots(B, S);
  return c <= kMaxI32 ? (int)c : 0;
}

int ulysses_cu_seqlens_from_positions(const void* pos_shards, int pos_bytes, int P, int B, int S,
                                      int32_t* cu_seqlens, int cu_capacity, int32_t* n_seqs,
                                      int32_t* max_len, void* stream) {
  if (!pos_shards || !cu_seqlens || !n_seqs || !max_len) return fail(ULY_ERR_NULL, "NULL pointer");
  if (P <= 0 || B <= 0 || S <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (P=%d B=%d S=%d)", P, B, S);
  if (S % P) return fail(ULY_ERR_SHAPE, "S=%d is not divisible by P=%d", S, P);
  if ((int64_t)B * S >= kMaxI32) return fail(ULY_ERR_SHAPE, "B*S exceeds 2^31 - 2");
  if (pos_bytes != 4 && pos_bytes != 8)
    return fail(ULY_ERR_UNSUPPORTED, "pos_bytes=%d not in {4,8}", pos_bytes);
  if ((int64_t)cu_capacity < (int64_t)B * S + 1)
    return fail(ULY_ERR_CAPACITY, "cu_capacity=%d < B*S+1=%lld", cu_capacity,
                (long long)((int64_t)B * S + 1));
  if (!aligned(pos_shards, pos_bytes) || !aligned(cu_seqlens, 4) || !aligned(n_seqs, 4) ||
      !aligned(max_len, 4))
    return fail(ULY_ERR_ALIGN, "misaligned pointer");
  return hip_status(uly::segments_launch(pos_shards, pos_bytes, P, B, S, cu_seqlens, cu_capacity,
                                         n_seqs, max_len, (hipStream_t)stream),
                    "ulysses_cu_seqlens_from_positions launch");
}

// Forward workspace: the split partials, O_s fp32 [nsplit][T][hq][D], then the
// running max and sum of each split, fp32 [2][nsplit][B][hq][S].
size_t ulysses_attn_fwd_workspace_bytes(int B, int S, int hq, int hkv, int D) {
  if (B <= 0 || S <= 0 || hq <= 0 || hkv <= 0 || (D != 64 && D != 128)) return 0;
  const int ns = uly::fwd_splits(B, S, hq, uly::fwd_block_rows(B, S, hq, D), D, true);
  if (ns == 1) return 0;
  const size_t rows = (size_t)B * S * hq;
  return align256((size_t)ns * rows * D * 4) + align256(2 * (size_t)ns * rows * 4);
}

int ulysses_attn_fwd_layout(const void* q, const void* k, const void* v, void* out, float* lse,
                            const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                            void* workspace, size_t workspace_bytes, const uly_layout* q_layout,
                            const uly_layout* kv_layout, int B, int S, int hq, int hkv, int D,
                            float softmax_scale, int causal, int window_left, int window_right,
                            void* stream) {
  int rc = check_attn(q, k, v, cu_seqlens, n_seqs, B, S, hq, hkv, D, softmax_scale, window_left,
                      window_right);
  if (rc) return rc;
  if (!out || !lse) return fail(ULY_ERR_NULL, "NULL out/lse");
  const size_t need = ulysses_attn_fwd_workspace_bytes(B, S, hq, hkv, D);
  if (need > 0 && !workspace) return fail(ULY_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(ULY_ERR_CAPACITY, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(sink, 4) || !aligned(cu_seqlens, 4) || !aligned(n_seqs, 4) ||
      !aligned(workspace, 256))
    return fail(ULY_ERR_ALIGN, "q/k/v/out need 16-byte alignment, lse/sink/cu 4-byte, workspace 256-byte");
  uly::AttnArgs a = make_args(q, k, v, sink, cu_seqlens, n_seqs, B, S, hq, hkv, softmax_scale,
                              causal, window_left, window_right);
  if ((rc = make_map(q_layout, B, S, hq, D, "q", a.mq)) || (rc = make_map(kv_layout, B, S, hkv, D, "kv", a.mk)))
    return rc;
  a.out = (__bf16*)out;
  a.lse = lse;
  if (need > 0) {
    a.nsplit = uly::fwd_splits(B, S, hq, uly::fwd_block_rows(B, S, hq, D), D,
                                uly::uneven_layer(a.causal, a.wl, a.wr));
    a.part = (float*)workspace;
    a.part_pdp = (float*)((char*)workspace + align256((size_t)a.nsplit * B * S * hq * D * 4));
  }
  return hip_status(uly::attn_fwd_launch(a, D, (hipStream_t)stream), "ulysses_attn_fwd launch");
}

int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                     void* workspace, size_t workspace_bytes, int B, int S, int hq, int hkv, int D,
                     float softmax_scale, int causal, int window_left, int window_right,
                     void* stream) {
  const uly_layout lq = head_layout(S, hq, D), lk = head_layout(S, hkv, D);
  return ulysses_attn_fwd_layout(q, k, v, out, lse, sink, cu_seqlens, n_seqs, workspace,
                                 workspace_bytes, &lq, &lk, B, S, hq, hkv, D, softmax_scale, causal,
                                 window_left, window_right, stream);
}

// ---- allocation-free forward: the split partials in a file-scope array
//
// One array per GPU, held until the process ends.  In host code `scratch` is
// a stand-in for the device symbol, not an address: every use goes through
// the pointer hipGetSymbolAddress returns for the current device, looked up
// on the first call on that device and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

static int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(ULY_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

size_t ulysses_attn_fwd_noalloc_max_workspace(void) { return kNoAllocScratchBytes; }

int ulysses_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                             int B, int S, int hq, int hkv, int D, float softmax_scale, int causal,
                             int window_left, int window_right, void* stream) {
  const size_t need = ulysses_attn_fwd_workspace_bytes(B, S, hq, hkv, D);
  if (need > kNoAllocScratchBytes)
    return fail(ULY_ERR_CAPACITY,
                "this problem's forward needs %zu bytes of split partials, above the %zu-byte "
                "static scratch of the allocation-free entry point (use ulysses_attn_fwd)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int rc = scratch_for_current_device(&ws);
    if (rc) return rc;
  }
  return ulysses_attn_fwd(q, k, v, out, lse, sink, cu_seqlens, n_seqs, ws, need > 0 ? kNoAllocScratchBytes : 0,
                          B, S, hq, hkv, D, softmax_scale, causal, window_left, window_right, stream);
}

int ulysses_attn_fwd_chunk(const void* q, const void* k_chunk, const void* v_chunk, float* out,
                           float* lse, const int32_t* cu_seqlens, const int32_t* n_seqs,
                           void* workspace, size_t workspace_bytes, const uly_layout* q_layout,
                           const uly_layout* kv_layout, int B, int S, int k_start, int Sk, int hq,
                           int hkv, int D, float softmax_scale, int causal, int window_left,
                           int window_right, void* stream) {
  int rc = check_attn(q, k_chunk, v_chunk, cu_seqlens, n_seqs, B, S, hq, hkv, D, softmax_scale,
                      window_left, window_right);
  if (rc) return rc;
  if (!out || !lse) return fail(ULY_ERR_NULL, "NULL out/lse");
  if (k_start < 0 || Sk <= 0 || (int64_t)k_start + Sk > S)
    return fail(ULY_ERR_SHAPE, "chunk [%d, %d) is not inside [0, S=%d)", k_start, k_start + Sk, S);
  const size_t need = ulysses_attn_fwd_workspace_bytes(B, S, hq, hkv, D);
  if (need > 0 && !workspace) return fail(ULY_ERR_NULL, "NULL workspace (%zu bytes needed)", need);
  if (workspace_bytes < need)
    return fail(ULY_ERR_CAPACITY, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (!aligned(q, 16) || !aligned(k_chunk, 16) || !aligned(v_chunk, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(cu_seqlens, 4) || !aligned(n_seqs, 4) || !aligned(workspace, 256))
    return fail(ULY_ERR_ALIGN, "q/k/v/out need 16-byte alignment, lse/cu 4-byte, workspace 256-byte");
  uly::AttnArgs a = make_args(q, k_chunk, v_chunk, nullptr, cu_seqlens, n_seqs, B, S, hq, hkv,
                              softmax_scale, causal, window_left, window_right);
  if ((rc = make_map(q_layout, B, S, hq, D, "q", a.mq)) || (rc = make_map(kv_layout, B, Sk, hkv, D, "kv", a.mk)))
    return rc;
  // the chunk tensors hold positions [k_start, k_start + Sk) of each batch row
  a.mk.S = uly::make_fastdiv(S);
  a.mk.s0 = k_start;
  a.mk.s_len = Sk;
  if (B > 1) a.mk.uniform = 0;
  a.k_lo_s = k_start;
  a.k_hi_s = k_start + Sk;
  if (a.mk.uniform) {  // B == 1: keep every tile row inside the chunk
    a.kt_lo = k_start;
    a.kt_hi = k_start + Sk;
  }
  a.out = (__bf16*)out;
  a.lse = lse;
  a.o_f32 = 1;
  if (need > 0) {
    a.nsplit = uly::fwd_splits(B, S, hq, uly::fwd_block_rows(B, S, hq, D), D,
                                uly::uneven_layer(a.causal, a.wl, a.wr));
    a.part = (float*)workspace;
    a.part_pdp = (float*)((char*)workspace + align256((size_t)a.nsplit * B * S * hq * D * 4));
  }
  return hip_status(uly::attn_fwd_launch(a, D, (hipStream_t)stream), "ulysses_attn_fwd_chunk launch");
}

static int check_merge(const void* a, const void* b, int B, int S, int hq, int D) {
  if (!a || !b) return fail(ULY_ERR_NULL, "NULL pointer");
  if (B <= 0 || S <= 0 || hq <= 0 || D <= 0)
    return fail(ULY_ERR_SHAPE, "sizes must be positive (B=%d S=%d hq=%d D=%d)", B, S, hq, D);
  if (D % 4 || 256 % (D / 4))
    return fail(ULY_ERR_UNSUPPORTED, "D=%d: a multiple of 4 with D/4 dividing 256", D);
  if ((int64_t)B * S * hq * D >= kMaxI32 * 8ll) return fail(ULY_ERR_SHAPE, "problem too large");
  return ok();
}

int ulysses_attn_merge(float* acc_out, float* acc_lse, const float* out, const float* lse, int B,
                       int S, int hq, int D, void* stream) {
  int rc = check_merge(acc_out, out, B, S, hq, D);
  if (rc) return rc;
  if (!acc_lse || !lse) return fail(ULY_ERR_NULL, "NULL lse");
  if (!aligned(acc_out, 16) || !aligned(out, 16) || !aligned(acc_lse, 4) || !aligned(lse, 4))
    return fail(ULY_ERR_ALIGN, "outputs need 16-byte alignment, LSE 4-byte");
  return hip_status(uly::attn_merge_launch(acc_out, acc_lse, out, lse, B, S, hq, D,
                                           (hipStream_t)stream),
                    "ulysses_attn_merge launch");
}

int ulysses_attn_merge_finish(const float* acc_out, const float* acc_lse, const float* sink,
                              void* out, float* lse, int B, int S, int hq, int D, void* stream) {
  int rc = check_merge(acc_out, out, B, S, hq, D);
  if (rc) return rc;
  if (!acc_lse || !lse) return fail(ULY_ERR_NULL, "NULL lse");
  if (lse == acc_lse) return fail(ULY_ERR_UNSUPPORTED, "lse must not alias acc_lse");
  if (!aligned(acc_out, 16) || !aligned(out, 8) || !aligned(acc_lse, 4) || !aligned(lse, 4) ||
      !aligned(sink, 4))
    return fail(ULY_ERR_ALIGN, "acc_out needs 16-byte alignment, out 8-byte, LSE/sink 4-byte");
  return hip_status(uly::attn_merge_finish_launch(acc_out, acc_lse, sink, out, lse, B, S, hq, D,
                                                  (hipStream_t)stream),
                    "ulysses_attn_merge_finish launch");
}

// Backward workspace: delta, sum_j P dP, LSE*log2(e) (each [B][hq][S] fp32),
// dsink partials [hq][parts], the status words (scale exponent, counts) and
// the stats blocks' maxima, fp16 copies of q, dout ([B*S + kPad][hq][D]) and
// k, v ([B*S + kPad][hkv][D]), then the split partials.
constexpr size_t kStatusBytes = 256;
static size_t bwd_status_offset(int B, int S, int hq) {
  return 3 * align256((size_t)B * S * hq * sizeof(float)) +
         align256((size_t)hq * kDsinkParts * sizeof(float));
}
static size_t bwd_copies_offset(int B, int S, int hq) {
  return bwd_status_offset(B, S, hq) + kStatusBytes + align256((size_t)uly::kStatBlocks * uly::kStatFloats * sizeof(float));
}

size_t ulysses_attn_bwd_workspace_bytes(int B, int S, int hq, int hkv, int D) {
  if (B <= 0 || S <= 0 || hq <= 0 || hkv <= 0 || D <= 0) return 0;
  const size_t qsz = align256(((size_t)B * S + uly::kPad) * hq * D * 2),
               kvsz = align256(((size_t)B * S + uly::kPad) * hkv * D * 2);
  return bwd_copies_offset(B, S, hq) + 2 * qsz + 2 * kvsz + split_part_bytes(B, S, hq, hkv, D);
}

size_t ulysses_attn_bwd_status_offset(int B, int S, int hq, int hkv, int D) {
  if (B <= 0 || S <= 0 || hq <= 0 || hkv <= 0 || D <= 0) return 0;
  return bwd_status_offset(B, S, hq);
}

static int attn_bwd_impl(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, const float* sink,
                         const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq, void* dk,
                         void* dv, float* dsink, void* workspace, size_t workspace_bytes,
                         const uly_layout* q_layout, const uly_layout* kv_layout, int B, int S,
                         int hq, int hkv, int D, float softmax_scale, int causal, int window_left,
                         int window_right, void* stream, int dkv_f32) {
  int rc = check_attn(q, k, v, cu_seqlens, n_seqs, B, S, hq, hkv, D, softmax_scale, window_left,
                      window_right);
  if (rc) return rc;
  if (!out || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(ULY_ERR_NULL, "NULL out/dout/lse/dq/dk/dv/workspace");
  if ((sink == nullptr) != (dsink == nullptr))
    return fail(ULY_ERR_NULL, "sink and dsink must both be NULL or both be set");
  const size_t need = ulysses_attn_bwd_workspace_bytes(B, S, hq, hkv, D);
  if (workspace_bytes < need)
    return fail(ULY_ERR_CAPACITY, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(sink, 4) || !aligned(dsink, 4) || !aligned(workspace, 256) ||
      !aligned(cu_seqlens, 4) || !aligned(n_seqs, 4))
    return fail(ULY_ERR_ALIGN, "bf16 tensors need 16-byte alignment, workspace 256-byte");
  uly::AttnArgs a = make_args(q, k, v, sink, cu_seqlens, n_seqs, B, S, hq, hkv, softmax_scale,
                              causal, window_left, window_right);
  if ((rc = make_map(q_layout, B, S, hq, D, "q", a.mq)) || (rc = make_map(kv_layout, B, S, hkv, D, "kv", a.mk)))
    return rc;
  a.o = (const __bf16*)out;
  a.dout = (const __bf16*)dout;
  a.lse = const_cast<float*>(lse);
  a.out = (__bf16*)dq;
  a.dk = (__bf16*)dk;
  a.dv = (__bf16*)dv;
  a.dkv_f32 = dkv_f32;
  a.dsink = dsink;
  char* ws = (char*)workspace;
  const size_t rows = align256((size_t)B * S * hq * sizeof(float));
  a.ndelta = (float*)ws;
  a.pdp = (float*)(ws + rows);
  a.lse2 = (float*)(ws + 2 * rows);
  a.dsink_part = (float*)(ws + 3 * rows);
  a.bwd_status = (int*)(ws + bwd_status_offset(B, S, hq));
  a.stat_part = (float*)(ws + bwd_status_offset(B, S, hq) + kStatusBytes);
  char* h16 = ws + bwd_copies_offset(B, S, hq);
  const size_t qsz = align256(((size_t)B * S + uly::kPad) * hq * D * 2),
               kvsz = align256(((size_t)B * S + uly::kPad) * hkv * D * 2);
  a.q16 = (_Float16*)h16;
  a.do16 = (_Float16*)(h16 + qsz);
  a.k16 = (_Float16*)(h16 + 2 * qsz);
  a.v16 = (_Float16*)(h16 + 2 * qsz + kvsz);
  {
    char* base = h16 + 2 * qsz + 2 * kvsz;
    const size_t main = split_main_bytes(B, S, hq, hkv, D);
    a.part = (float*)base;
    a.bal_prefix = (int*)(base + main - align256((size_t)(uly::kBalMaxTilesHost + 1) * 4));
    a.part_pdp = (float*)(base + main);
    a.bal_W = uly::dkdv_bal_workgroups(B, S, hkv);
  }
  a.n_part = kDsinkParts;
  return hip_status(uly::attn_bwd_launch(a, D, (hipStream_t)stream), "ulysses_attn_bwd launch");
}

int ulysses_attn_bwd_layout(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, const float* sink,
                            const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq, void* dk,
                            void* dv, float* dsink, void* workspace, size_t workspace_bytes,
                            const uly_layout* q_layout, const uly_layout* kv_layout, int B, int S,
                            int hq, int hkv, int D, float softmax_scale, int causal, int window_left,
                            int window_right, void* stream) {
  return attn_bwd_impl(q, k, v, out, dout, lse, sink, cu_seqlens, n_seqs, dq, dk, dv, dsink,
                       workspace, workspace_bytes, q_layout, kv_layout, B, S, hq, hkv, D,
                       softmax_scale, causal, window_left, window_right, stream, 0);
}

int ulysses_attn_bwd_layout_f32kv(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, const float* sink,
                                  const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq,
                                  float* dk, float* dv, float* dsink, void* workspace,
                                  size_t workspace_bytes, const uly_layout* q_layout,
                                  const uly_layout* kv_layout, int B, int S, int hq, int hkv, int D,
                                  float softmax_scale, int causal, int window_left,
                                  int window_right, void* stream) {
  return attn_bwd_impl(q, k, v, out, dout, lse, sink, cu_seqlens, n_seqs, dq, dk, dv, dsink,
                       workspace, workspace_bytes, q_layout, kv_layout, B, S, hq, hkv, D,
                       softmax_scale, causal, window_left, window_right, stream, 1);
}

int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                     const void* dout, const float* lse, const float* sink,
                     const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq, void* dk,
                     void* dv, float* dsink, void* workspace, size_t workspace_bytes, int B, int S,
                     int hq, int hkv, int D, float softmax_scale, int causal, int window_left,
                     int window_right, void* stream) {
  const uly_layout lq = head_layout(S, hq, D), lk = head_layout(S, hkv, D);
  return ulysses_attn_bwd_layout(q, k, v, out, dout, lse, sink, cu_seqlens, n_seqs, dq, dk, dv,
                                 dsink, workspace, workspace_bytes, &lq, &lk, B, S, hq, hkv, D,
                                 softmax_scale, causal, window_left, window_right, stream);
}

const char* ulysses_last_error(void) { return g_err; }

}  // extern "C"

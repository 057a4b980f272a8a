/*
 * ulysses.h -- C ABI of the per-rank Ulysses sequence-parallel hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * After the sequence-to-head all-to-all, each of P ranks holds the whole
 * gathered sequence for H/P of the heads and runs exact softmax attention on
 * them; the inverse all-to-all then returns sequence shards.  This library
 * provides, for one GPU on which the P ranks are simulated in memory:
 *
 *   ulysses_a2a_pack / ulysses_a2a_unpack    the layout permutation of the
 *                                            all-to-all (all P ranks at once)
 *   ulysses_cu_seqlens_from_positions        cu_seqlens / max_len rebuilt from
 *                                            the gathered position_ids
 *   ulysses_attn_fwd / ulysses_attn_bwd      one rank's attention, fwd and bwd
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library keeps no pointer after a call returns and allocates nothing.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and never synchronises the host.
 *   - Arguments are checked on the host before any launch.  A call returns 0
 *     (ULY_OK) or a negative uly_status and then launches nothing;
 *     ulysses_last_error() gives a readable reason (thread-local).
 *   - bf16 tensors are raw IEEE bfloat16 bits; fp32 is IEEE binary32.
 *
 * Citations name the web pages this path is defined by:
 *   [accelerate#4209]  accelerate PR "Add an FSDP2-native Ulysses sequence
 *                      parallelism backend"
 *   [lca#135]          long-context-attention issue "usage with pytorch FSDP"
 *   [arctic#45]        ArcticTraining PR "Add Sequence Parallelism via Ulysses"
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ULY_OK = 0,
  ULY_ERR_NULL = -1,        /* a required pointer is NULL                          */
  ULY_ERR_SHAPE = -2,       /* a size is <= 0, S % P != 0, or a size overflows     */
  ULY_ERR_HEADS = -3,       /* H % P, Hkv % P or Hq % Hkv is not 0                 */
  ULY_ERR_UNSUPPORTED = -4, /* head_dim, element size or mask not supported        */
  ULY_ERR_CAPACITY = -5,    /* an output or workspace buffer is too small          */
  ULY_ERR_ALIGN = -6,       /* a pointer is not aligned as documented              */
  ULY_ERR_HIP = -7          /* a HIP launch failed                                 */
} uly_status;

/* ------------------------------------------------------------------------
 * Layout permutation of the sequence-to-head all-to-all ([accelerate#4209]
 * PR body; the layouts are stated in its reply on the four all-to-all call
 * sites, where the backward of the differentiable all-to-all runs the same
 * exchange with the two directions exchanged, so the same two calls serve dO
 * and dQ/dK/dV).
 *
 * ulysses_a2a_pack: seq_shards [P][B][S/P][H][D] -> head_shards [P][B][S][H/P][D]
 *   head[c][b][r*S/P + s][h'][d] = seq[r][b][s][c*H/P + h'][d]
 *   Rank r holds tokens [r*S/P, (r+1)*S/P) (shards are numbered by where they
 *   sit in the sequence, [accelerate#4209] _prepare_sp_model comment); rank c
 *   receives heads [c*H/P, (c+1)*H/P).
 * ulysses_a2a_unpack: the inverse, head_shards -> seq_shards.
 *
 *   elem_bytes in {1, 2, 4, 8}; the copy is bit-exact for any dtype.
 *   The two buffers must not overlap.  Pointers need elem_bytes alignment;
 *   16-byte aligned buffers whose runs of H/P*D elements are a multiple of
 *   16 bytes take the vectorised path.
 *   Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (a size <= 0, S % P), ULY_ERR_HEADS
 *   (H % P), ULY_ERR_UNSUPPORTED (elem_bytes), ULY_ERR_ALIGN.
 * ---------------------------------------------------------------------- */
int ulysses_a2a_pack(const void* seq_shards, void* head_shards, int P, int B, int S, int H,
                     int D, int elem_bytes, void* stream);
int ulysses_a2a_unpack(const void* head_shards, void* seq_shards, int P, int B, int S, int H,
                       int D, int elem_bytes, void* stream);

/* KV heads fewer than ranks (the follow-up [accelerate#4209] leaves open: it
 * requires the KV heads to be divisible by sp_size): with H < P and P % H == 0,
 * each head goes to the R = P / H ranks
 * whose query heads use it under contiguous GQA groups, rank c getting head
 * c / R.
 * ulysses_a2a_pack_replicated: seq_shards [P][B][S/P][H][D] -> head_shards
 *   [P][B][S][1][D], head[c][b][r*S/P + s][0][d] = seq[r][b][s][c/R][d];
 *   bit-exact, elem_bytes in {1, 2, 4, 8}.
 * ulysses_a2a_reduce_replicated: its gradient: head_shards [P][B][S][1][D]
 *   (in_elem_bytes 4: fp32, as ulysses_attn_bwd_layout_f32kv leaves the
 *   replicas' dK/dV; or 2: bf16) -> seq_shards [P][B][S/P][H][D] bf16, each
 *   element the fp32 sum of its R replicas in rank order, rounded once to
 *   bf16 (D % 8 == 0, 16-byte aligned buffers).
 * Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (sizes, S % P), ULY_ERR_HEADS (H > P or
 *   P % H), ULY_ERR_UNSUPPORTED (elem_bytes, D % 8, overlap), ULY_ERR_ALIGN. */
int ulysses_a2a_pack_replicated(const void* seq_shards, void* head_shards, int P, int B, int S,
                                int H, int D, int elem_bytes, void* stream);
int ulysses_a2a_reduce_replicated(const void* head_shards, int in_elem_bytes, void* seq_shards,
                                  int P, int B, int S, int H, int D, void* stream);

/* The same permutation for n (1..4) tensors of one exchange in one launch
 * (the forward's all-to-all carries Q, K and V together, the backward's dQ, dK
 * and dV: [accelerate#4209] reply on the four all-to-all call sites).
 * seq_shards, head_shards and H are HOST arrays of n entries: device
 * pointers, and the head count of each tensor (K and V have Hkv heads under
 * GQA); P, B, S, D and elem_bytes are shared.  Each tensor is checked as in
 * ulysses_a2a_pack; no destination may overlap a source or another
 * destination.  Errors: as above, ULY_ERR_UNSUPPORTED for n outside 1..4 or
 * overlapping buffers, ULY_ERR_NULL for a NULL array. */
int ulysses_a2a_pack_multi(int n, const void* const* seq_shards, void* const* head_shards,
                           const int* H, int P, int B, int S, int D, int elem_bytes, void* stream);
int ulysses_a2a_unpack_multi(int n, const void* const* head_shards, void* const* seq_shards,
                             const int* H, int P, int B, int S, int D, int elem_bytes, void* stream);

/* ------------------------------------------------------------------------
 * cu_seqlens / max_len from the gathered position_ids ([accelerate#4209],
 * comment on the flash-attention kwargs: a padding-free collator's
 * cu_seq_lens/max_length describe the local shard, so they are dropped and
 * rebuilt from the position_ids gathered over the whole sequence; the gather
 * happens once per forward, comment on the per-layer all-gather).
 *
 *   pos_shards  [P][B][S/P] integers (pos_bytes = 4: int32, 8: int64), the P
 *               rank shards in rank order; their concatenation along the
 *               sequence is the gathered position_ids [B][S].
 *   A document starts at every flattened token t = b*S + i with i == 0 or
 *   pos[b][i] == 0.  Outputs (device, int32):
 *     cu_seqlens[0..n]  document starts in increasing order, then B*S
 *     *n_seqs           n, the number of documents
 *     *max_len          the longest document
 *   cu_capacity is the number of int32 slots in cu_seqlens; it must be at
 *   least B*S + 1 (the worst case, one token per document), so the host never
 *   needs n.  Slots n+1 .. B*S are left untouched; with cu_capacity >=
 *   ulysses_cu_seqlens_capacity(B, S) the slots after B*S serve as scratch.
 *   Errors: ULY_ERR_NULL, ULY_ERR_SHAPE, ULY_ERR_UNSUPPORTED (pos_bytes),
 *   ULY_ERR_CAPACITY (cu_capacity < B*S + 1), ULY_ERR_ALIGN (pos_shards not
 *   pos_bytes-aligned, outputs not 4-byte aligned).
 * ---------------------------------------------------------------------- */
int ulysses_cu_seqlens_from_positions(const void* pos_shards, int pos_bytes, int P, int B, int S,
                                      int32_t* cu_seqlens, int cu_capacity, int32_t* n_seqs,
                                      int32_t* max_len, void* stream);

/* The cu_capacity at which ulysses_cu_seqlens_from_positions runs its scan on
 * many work-groups, in two passes: B*S + 1 plus 4 int32 per chunk of at least
 * 512 tokens (at most 1024 chunks).  Those slots past B*S are its scratch:
 * their contents on return are unspecified.  With a smaller (still valid)
 * capacity the scan runs in one work-group.  Both give the same result.
 * 0 for sizes the scan rejects. */
int ulysses_cu_seqlens_capacity(int B, int S);

/* ------------------------------------------------------------------------
 * One rank's attention over the whole gathered sequence ([accelerate#4209]
 * PR body: the model's own attention runs between the two all-to-alls, with
 * flash attention, packing and sliding windows; [lca#135] test script for the
 * flash_attn_func arguments causal and window_size=(left, right), -1 meaning
 * unbounded).
 *
 * Layouts (bf16, contiguous, 16-byte aligned):
 *   q, out, dout, dq      [B][S][hq][D]
 *   k, v, dk, dv          [B][S][hkv][D]
 *   lse                   fp32 [B][hq][S], natural-log log-sum-exp per row
 * GQA: query head h uses KV head h / (hq/hkv) (contiguous groups; the rank
 * holds hq = Hq/P query heads and hkv = Hkv/P KV heads, [arctic#45] feature
 * list, on attention variants beyond plain multi-head).
 * Documents: cu_seqlens (int32, n+1 entries over the B*S flattened tokens,
 * as produced by ulysses_cu_seqlens_from_positions) with *n_seqs on the
 * device; both NULL means one document per batch row.  Documents must not
 * cross batch rows.
 * Mask: key j is visible to query i iff both lie in the same document, and
 *   (!causal || j <= i), (window_left < 0 || i - j <= window_left),
 *   (window_right < 0 || j - i <= window_right).
 * Sink ([accelerate#4209] findings: one logit per head, sliced to the heads
 * the rank holds): fp32 [hq] (pass sink + r*hq for rank r; 4-byte
 * alignment) or NULL.  It is an extra logit in every row's softmax
 * denominator, not multiplied by softmax_scale, with no value vector.
 *   O_i = sum_j softmax_j(scale * q_i . k_j) v_j,  LSE_i = ln(sum_j e^{s_ij} + e^{sink})
 * Rows that see no key and have no sink get O = 0 and LSE = -inf.
 * workspace: device memory of at least ulysses_attn_fwd_workspace_bytes()
 *   bytes, 256-byte aligned, owned by the caller (may be NULL when that is
 *   zero); its contents on entry do not matter and on return are unspecified.
 * Supported: D in {64, 128}; window_left, window_right >= -1.
 * Errors: ULY_ERR_NULL, ULY_ERR_SHAPE, ULY_ERR_HEADS (hq % hkv),
 *   ULY_ERR_UNSUPPORTED (D, window < -1, cu_seqlens given without n_seqs),
 *   ULY_ERR_CAPACITY (workspace too small), ULY_ERR_ALIGN.
 * ---------------------------------------------------------------------- */
int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                     void* workspace, size_t workspace_bytes, int B, int S, int hq, int hkv, int D,
                     float softmax_scale, int causal, int window_left, int window_right,
                     void* stream);

/* ------------------------------------------------------------------------
 * ulysses_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It computes exactly what ulysses_attn_fwd
 * computes, with the same kernels.  Its split partials (small problems only,
 * as ulysses_attn_fwd_workspace_bytes gives them) live in a file-scope device
 * array of ulysses_attn_fwd_noalloc_max_workspace() bytes (32 MiB), one per
 * GPU, held until the process ends; the call allocates nothing.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race.  Nothing in the array needs to be zero
 * on entry.
 * Errors: as ulysses_attn_fwd, plus ULY_ERR_CAPACITY when the problem needs
 *   more split-partial bytes than the array holds, ULY_ERR_HIP if the array's
 *   device address cannot be obtained.
 * ---------------------------------------------------------------------- */
int ulysses_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                             int B, int S, int hq, int hkv, int D, float softmax_scale, int causal,
                             int window_left, int window_right, void* stream);
size_t ulysses_attn_fwd_noalloc_max_workspace(void);

/* ------------------------------------------------------------------------
 * The same two calls on tensors in other layouts, read and written in place:
 * attention takes the rank's heads straight from the sequence shards and
 * writes its outputs back into them, with no pack or unpack (the all-to-all's
 * permutation folded into the kernels' addressing; [accelerate#4209] reply
 * on the four all-to-all call sites for the [B, S/P, H, D] and the wrapper's
 * [B, H, S/P, D] forms).
 *
 * A layout says where the D contiguous elements of (batch row b, token s,
 * head h) start, counting elements (not bytes) from the tensor pointer:
 *   s = r * (S / shards) + sl  ->  b*batch + r*shard + sl*token + h*head
 * All query-side tensors (q, out, dout, dq) follow q_layout, all KV-side ones
 * (k, v, dk, dv) kv_layout.  Strides are multiples of 8 elements (16-byte
 * rows), token > 0, the others >= 0; shards divides S.  Examples, for the
 * rank r of P holding heads [r*h, (r+1)*h) of H (h = hq or hkv):
 *   head layout [B][S][h][D]:           shards=1, batch=S*h*D, token=h*D, head=D
 *   sequence shards [P][B][S/P][H][D]:  pointer + r*h*D; shards=P,
 *       shard=B*(S/P)*H*D, batch=(S/P)*H*D, token=H*D, head=D
 *   wrapper form, P x [B][H][S/P][D]:   pointer + r*h*(S/P)*D; shards=P,
 *       shard=B*H*(S/P)*D, batch=H*(S/P)*D, token=D, head=(S/P)*D
 * LSE, dsink, workspace and everything else as in ulysses_attn_fwd/_bwd.
 * Errors: as those calls, plus ULY_ERR_NULL (NULL layout), ULY_ERR_SHAPE
 * (shards, negative strides), ULY_ERR_ALIGN (strides not multiples of 8).
 * ---------------------------------------------------------------------- */
typedef struct uly_layout {
  int shards;
  int64_t batch, shard, token, head;
} uly_layout;

int ulysses_attn_fwd_layout(const void* q, const void* k, const void* v, void* out, float* lse,
                            const float* sink, const int32_t* cu_seqlens, const int32_t* n_seqs,
                            void* workspace, size_t workspace_bytes, const uly_layout* q_layout,
                            const uly_layout* kv_layout, int B, int S, int hq, int hkv, int D,
                            float softmax_scale, int causal, int window_left, int window_right,
                            void* stream);
int ulysses_attn_bwd_layout(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, const float* sink,
                            const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq, void* dk,
                            void* dv, float* dsink, void* workspace, size_t workspace_bytes,
                            const uly_layout* q_layout, const uly_layout* kv_layout, int B, int S,
                            int hq, int hkv, int D, float softmax_scale, int causal, int window_left,
                            int window_right, void* stream);

/* As ulysses_attn_bwd_layout, except that dk and dv are fp32 (same layout,
 * strides in elements) and not rounded: for KV gradients that are summed
 * further, as the replicas of a KV head shared by several ranks are
 * (ulysses_a2a_reduce_replicated), so that the sum is rounded only once. */
int ulysses_attn_bwd_layout_f32kv(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, const float* sink,
                                  const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq,
                                  float* dk, float* dv, float* dsink, void* workspace,
                                  size_t workspace_bytes, const uly_layout* q_layout,
                                  const uly_layout* kv_layout, int B, int S, int hq, int hkv, int D,
                                  float softmax_scale, int causal, int window_left,
                                  int window_right, void* stream);

/* ------------------------------------------------------------------------
 * The inner step of a ring over KV chunks, combined with Ulysses (the
 * long-context-attention "unified sequence parallel" scheme: Ulysses heads
 * inside, a ring over sequence chunks outside; the accelerate PR leaves ring
 * attention to context parallelism).  The rank's queries, all S positions,
 * meet one chunk of the keys at a time; exact per-chunk results are merged.
 *
 * ulysses_attn_fwd_chunk: attention of q ([B][S][hq][D] as q_layout says)
 *   against keys at positions [k_start, k_start + Sk) of every batch row.
 *   k_chunk, v_chunk hold only those Sk positions (kv_layout describes the
 *   chunk tensors, e.g. [B][Sk][hkv][D]: shards=1, batch=Sk*hkv*D,
 *   token=hkv*D, head=D).  Masks (documents, causal, windows) use the keys'
 *   positions in the whole sequence.  out: fp32 [B][S][hq][D], normalised
 *   over the chunk's keys; lse: fp32 [B][hq][S] over the chunk's keys.  Rows
 *   that see no key of the chunk get O = 0, LSE = -inf.  No sink (it joins
 *   once, in ulysses_attn_merge_finish).  Workspace as ulysses_attn_fwd.
 * ulysses_attn_merge: acc := merge(acc, chunk), in place:
 *   L = log(e^acc_lse + e^lse), acc_out = e^(acc_lse - L) acc_out + e^(lse - L) out,
 *   acc_lse = L.  Start from the first chunk's result (or acc_lse = -inf).
 * ulysses_attn_merge_finish: out (bf16 [B][S][hq][D]) and lse (fp32
 *   [B][hq][S], not aliasing acc_lse) from the accumulator, the sink (fp32
 *   [hq] or NULL) joining the denominator: L' = log(e^L + e^sink),
 *   out = e^(L - L') acc_out.
 * Buffers 16-byte aligned (out 8); D a multiple of 4 with D/4 dividing 256.
 * Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (sizes, chunk outside [0, S)),
 *   ULY_ERR_UNSUPPORTED (D, aliasing), ULY_ERR_ALIGN, ULY_ERR_CAPACITY, and as
 *   ulysses_attn_fwd_layout.
 * ---------------------------------------------------------------------- */
int ulysses_attn_fwd_chunk(const void* q, const void* k_chunk, const void* v_chunk, float* out,
                           float* lse, const int32_t* cu_seqlens, const int32_t* n_seqs,
                           void* workspace, size_t workspace_bytes, const uly_layout* q_layout,
                           const uly_layout* kv_layout, int B, int S, int k_start, int Sk, int hq,
                           int hkv, int D, float softmax_scale, int causal, int window_left,
                           int window_right, void* stream);
int ulysses_attn_merge(float* acc_out, float* acc_lse, const float* out, const float* lse, int B,
                       int S, int hq, int D, void* stream);
int ulysses_attn_merge_finish(const float* acc_out, const float* acc_lse, const float* sink,
                              void* out, float* lse, int B, int S, int hq, int D, void* stream);

/* ------------------------------------------------------------------------
 * The sequence-tiled MLP of one rank (the TiledMLP / SequenceTiledCompute
 * features of the DeepSpeed pull request that ports Ulysses to HF models:
 * the layer's MLP computed over the rank's tokens in tiles along the
 * sequence, so that only one tile's activations exist at a time, and the
 * weight gradients added once after the tiles).  The gated MLP of the
 * Llama-family models:  y = (silu(x Wg^T) * (x Wu^T)) Wd^T.
 *
 * x, y, dy, dx: bf16 [T][H] (row-major, token-major); w_gate, w_up: bf16
 * [I][H]; w_down: bf16 [H][I]; dw_gate, dw_up: fp32 [I][H]; dw_down: fp32
 * [H][I].  `tile` tokens per tile (the last tile may be shorter).  H and I
 * must be multiples of 128 and at most 2^20; T >= 1, tile >= 1.  The forward rounds the gated
 * activation to bf16 before the down projection; the backward recomputes
 * each tile's projections from x, rounds them and the gated derivatives to
 * bf16, accumulates the weight gradients in fp32 over the tiles and
 * overwrites dw_* with the sums.  The caller owns all buffers (16-byte
 * aligned), including `workspace` (ulysses_tiled_mlp_workspace_bytes; one
 * tile's activations).  Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (sizes, H or I
 * above 2^20), ULY_ERR_UNSUPPORTED (H or I not a multiple of 128),
 * ULY_ERR_ALIGN, ULY_ERR_CAPACITY (workspace), ULY_ERR_HIP.
 * ---------------------------------------------------------------------- */
size_t ulysses_tiled_mlp_workspace_bytes(int T, int H, int I, int tile);
int ulysses_tiled_mlp_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          void* y, int T, int H, int I, int tile, void* workspace,
                          size_t workspace_bytes, void* stream);
int ulysses_tiled_mlp_bwd(const void* x, const void* w_gate, const void* w_up, const void* w_down,
                          const void* dy, void* dx, float* dw_gate, float* dw_up, float* dw_down,
                          int T, int H, int I, int tile, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of device workspace ulysses_attn_fwd needs for these sizes: zero when
 * one pass of query tiles fills the GPU, else room for fp32 partial outputs of
 * the key-range splits that small problems are cut into (merged, with the
 * sink, by a second kernel).  Zero also for sizes ulysses_attn_fwd rejects. */
size_t ulysses_attn_fwd_workspace_bytes(int B, int S, int hq, int hkv, int D);

/* Bytes of device workspace ulysses_attn_bwd needs for these sizes. */
size_t ulysses_attn_bwd_workspace_bytes(int B, int S, int hq, int hkv, int D);

/* Byte offset, inside the workspace of a ulysses_attn_bwd* call with these
 * sizes, of six int32 values the call leaves there (valid once the call's
 * work on its stream has completed, until the workspace is reused):
 *   [0..3] the exponents e, c, a, b of the power-of-two scales of the fp16
 *       copies dout * 2^e, v * 2^c, q * 2^a, k * 2^b (see "Precision" below);
 *   [4] the number of copied elements that saturated at +-65504 (scaled
 *       magnitude above 65504, or NaN): the gradients may then be wrong;
 *   [5] the number of other copied elements that are inexact (scaled
 *       magnitude below 2^-17 with bits below 2^-24; error <= 2^-25 each,
 *       before the scale is removed).
 * A function of the sizes only (0 for sizes the backward rejects). */
size_t ulysses_attn_bwd_status_offset(int B, int S, int hq, int hkv, int D);

/* Backward of ulysses_attn_fwd for the loss sum(out * dout) ([accelerate#4209]:
 * gradients compared against an unsharded run; [lca#135]: backward of the
 * sharded attention).  Inputs as in the forward, plus out and lse from it.
 *   dq [B][S][hq][D], dk/dv [B][S][hkv][D] (bf16, overwritten; dk/dv summed
 *   over the query heads of each group), dsink fp32 [hq] (overwritten; must be
 *   non-NULL exactly when sink is non-NULL):
 *     dsink_h = -sum_i exp(sink_h - LSE_i) * sum_d dout_i,d out_i,d
 *   workspace: device memory of at least ulysses_attn_bwd_workspace_bytes()
 *   bytes, 256-byte aligned, owned by the caller; its contents on entry do
 *   not matter and on return are unspecified (it holds per-row statistics,
 *   fp16 copies of q, k, v, dout and, on small problems, fp32 partial sums).
 * Precision: the products run in fp16 (fp32 accumulation) on fp16 copies of
 *   q, k, v and dout that the call makes in the workspace, each an exact
 *   power-of-two scaling of its bf16 tensor: q * 2^a, k * 2^b, v * 2^c,
 *   dout * 2^e, with integer exponents (|x| <= 100) chosen on the device so
 *   that every copied value, and every scaled dS_ij = P_ij (dP_ij - delta_i)
 *   2^(e+c), stays below 2^15 in magnitude (bound for dS: max_i |dout_i|
 *   max_j |v_j| + max_i |delta_i|, norms over the head dimension; a and b
 *   are the largest such exponents, e and c share what the dS bound leaves).
 *   The softmax scale absorbs 2^-(a+b) exactly and the gradients are
 *   multiplied back by exact powers of two before they are stored, so inputs
 *   and gradients of any magnitude keep fp16's 11 significant bits in P and
 *   dS (a loss averaged over many tokens gives dout far below 1, which
 *   unscaled fp16 would flush to zero).  A copied value is exact when its
 *   scaled magnitude is at least 2^-17 (for q and k: magnitudes down to about
 *   2^-32 of the tensor's largest); smaller ones round to a multiple of 2^-24
 *   of the scaled value.  The call does not fail on inputs it cannot copy
 *   exactly; it counts them on the device (ulysses_attn_bwd_status_offset).
 * Errors: as ulysses_attn_fwd, plus ULY_ERR_CAPACITY (workspace too small)
 *   and ULY_ERR_NULL (sink and dsink not both NULL or both set).
 */
int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                     const void* dout, const float* lse, const float* sink,
                     const int32_t* cu_seqlens, const int32_t* n_seqs, void* dq, void* dk,
                     void* dv, float* dsink, void* workspace, size_t workspace_bytes, int B, int S,
                     int hq, int hkv, int D, float softmax_scale, int causal, int window_left,
                     int window_right, void* stream);

/* ------------------------------------------------------------------------
 * Per-kernel timing (a measurement aid, not part of the computation).
 * ulysses_profile_start(max_launches): from now on every kernel the library
 *   launches is bracketed by two HIP events recorded on the caller's stream,
 *   for up to max_launches launches (later ones are not recorded).  Creates
 *   the HIP events it needs (the only allocation in the library); resets
 *   earlier records.
 * ulysses_profile_stop(): stop recording.
 * ulysses_profile_report(buf, buf_bytes): waits for the recorded events and
 *   writes one line per kernel name, "name count total_ms min_ms max_ms",
 *   into buf (NUL-terminated); returns the number of recorded launches, or a
 *   negative uly_status (ULY_ERR_CAPACITY if buf is too small).
 * Not thread-safe: profile from one host thread.
 * ---------------------------------------------------------------------- */
int ulysses_profile_start(int max_launches);
int ulysses_profile_stop(void);
int ulysses_profile_report(char* buf, size_t buf_bytes);

/* ------------------------------------------------------------------------
 * Matrix-core calibration (a measurement aid, not part of the computation):
 * what the GPU's MFMA units sustain with nothing else to do, as context for
 * the attention kernels' rates against the published dense peak.
 * ulysses_calibrate_mfma(out, out_bytes, iters, mode, stream): one launch of
 *   512 work-groups of 256 threads (two per CU); every wave runs iters
 *   32x32x16 bf16 products (bf16 in, fp32 accumulate) on each of eight
 *   independent accumulators, their operands pseudo-random and changing
 *   from product to product (the power real tensors draw).  mode 0: operands
 *   from registers, nothing else in the loop; 1: as 0 with 8 independent
 *   fp32 FMAs after each product; 2: each product's B operand read from LDS
 *   (1 KiB a product); 3: both operands from LDS (2 KiB a product); 4: as 0
 *   with 8 independent fp32 exp2 (each with two adds) after each product;
 *   5: as 4 with a multiply in place of each exp2.  No
 *   global memory traffic in the loop.  out: device, at least 512*256
 *   floats (one checksum a thread, caller-owned scratch).  iters: a positive
 *   multiple of 8.  Asynchronous on `stream`.  Errors: ULY_ERR_NULL,
 *   ULY_ERR_CAPACITY (out_bytes), ULY_ERR_SHAPE (iters), ULY_ERR_UNSUPPORTED
 *   (mode), ULY_ERR_ALIGN, ULY_ERR_HIP.
 * ulysses_calibrate_mfma_flops(iters): the FLOPs one such launch executes
 *   (0 for iters <= 0).
 * ---------------------------------------------------------------------- */
int ulysses_calibrate_mfma(float* out, size_t out_bytes, int iters, int mode, void* stream);
size_t ulysses_calibrate_mfma_flops(int iters);

/* Reason for the last non-zero status returned on this thread ("" if none). */
const char* ulysses_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */

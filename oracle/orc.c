/*
 * CPU oracle for the work of one Ulysses rank -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  The GPU product path never calls it, links it or shares a
 * header, helper or constant with it.
 *
 * Everything here is the plain definition, written out with naive loops in
 * fp64 (inputs arrive already widened to double, which is exact for bf16):
 *
 *  - orc_pack / orc_unpack: the sequence-to-head all-to-all and its inverse
 *    as a brute-force index formula per element.  Layouts from the accelerate
 *    PR "Add an FSDP2-native Ulysses sequence parallelism backend" (reply on
 *    the four all-to-all call sites: queries/keys/values arrive sequence
 *    sharded, the output leaves as [batch, seq, heads / sp_size, head_dim]);
 *    shards are numbered by where they sit in the sequence (same PR, the
 *    _prepare_sp_model comment); rank c receives the c-th contiguous chunk of
 *    heads (the sequence-to-head all-to-all of the PR body).
 *  - orc_pack_replicated / orc_reduce_replicated: KV heads fewer than ranks,
 *    each sent to the ranks whose query heads use it, and the sum of the
 *    replicas' gradients (see the functions).
 *  - orc_gather_positions / orc_segments: concatenate the P position_ids
 *    shards in rank order, then a new document starts wherever the gathered
 *    position is 0 and at every batch-row start; cu_seqlens lists the starts
 *    plus the total, max_len the longest document.  The PR's comment on the
 *    flash-attention kwargs: cu_seq_lens/max_length are dropped and rebuilt
 *    from the gathered position_ids, never taken from the local shard.
 *  - orc_fwd / orc_bwd: exact softmax attention of the rank's heads over the
 *    whole gathered sequence (or over one chunk of key positions, the inner
 *    step of a ring over KV chunks: the long-context-attention "unified
 *    sequence parallel" combination of Ulysses with ring attention), with an
 *    explicit per-pair mask (same document,
 *    causal, window (left, right) with -1 meaning unbounded, as in the
 *    flash_attn_func argument list of the long-context-attention issue
 *    "usage with pytorch FSDP"), GQA with contiguous head groups, and an
 *    optional per-head sink logit (the PR's findings: one logit per head,
 *    sliced to the heads the rank holds).  The sink joins every row's softmax
 *    denominator as an extra logit that is not multiplied by the softmax
 *    scale and carries no value vector.
 *
 * Backward (the gradients the PR compares against an unsharded run):
 *   D_i = sum_d dO[i,d] O[i,d];  P_ij = exp(s_ij - LSE_i);  dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - D_i);  dQ_i = scale sum_j dS_ij k_j
 *   dK_j = scale sum_{h in group} sum_i dS_ij q_i;  dV_j = sum_{h in group} sum_i P_ij dO_i
 *   dsink_h = - sum_i exp(sink_h - LSE_i) D_i
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ layout */

/* seq: [P][B][S/P][H][D]  ->  head: [P][B][S][H/P][D]   (eb bytes per element) */
int orc_pack(const void* seq, void* head, int64_t P, int64_t B, int64_t S, int64_t H,
             int64_t D, int64_t eb) {
  if (P <= 0 || S % P || H % P) return -1;
  const int64_t Sl = S / P, hp = H / P;
  const char* src = (const char*)seq;
  char* dst = (char*)head;
  for (int64_t c = 0; c < P; ++c)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < S; ++t)
        for (int64_t hh = 0; hh < hp; ++hh)
          for (int64_t d = 0; d < D; ++d) {
            const int64_t r = t / Sl, s = t % Sl, h = c * hp + hh;
            const int64_t si = (((r * B + b) * Sl + s) * H + h) * D + d;
            const int64_t di = (((c * B + b) * S + t) * hp + hh) * D + d;
            memcpy(dst + di * eb, src + si * eb, (size_t)eb);
          }
  return 0;
}

/* head: [P][B][S][H/P][D]  ->  seq: [P][B][S/P][H][D] */
int orc_unpack(const void* head, void* seq, int64_t P, int64_t B, int64_t S, int64_t H,
               int64_t D, int64_t eb) {
  if (P <= 0 || S % P || H % P) return -1;
  const int64_t Sl = S / P, hp = H / P;
  const char* src = (const char*)head;
  char* dst = (char*)seq;
  for (int64_t c = 0; c < P; ++c)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < S; ++t)
        for (int64_t hh = 0; hh < hp; ++hh)
          for (int64_t d = 0; d < D; ++d) {
            const int64_t r = t / Sl, s = t % Sl, h = c * hp + hh;
            const int64_t si = (((c * B + b) * S + t) * hp + hh) * D + d;
            const int64_t di = (((r * B + b) * Sl + s) * H + h) * D + d;
            memcpy(dst + di * eb, src + si * eb, (size_t)eb);
          }
  return 0;
}

/* KV heads when there are fewer of them than ranks (H < P, P % H == 0): the
 * follow-up the accelerate PR leaves open (it requires H % sp_size == 0).
 * Every head goes to the R = P / H ranks whose query heads use it under
 * contiguous GQA groups: rank c holds query heads [c*Hq/P, (c+1)*Hq/P), which
 * belong to KV head (c*Hq/P) / (Hq/H) = c / R.
 * seq: [P][B][S/P][H][D]  ->  head: [P][B][S][1][D] */
int orc_pack_replicated(const void* seq, void* head, int64_t P, int64_t B, int64_t S, int64_t H,
                        int64_t D, int64_t eb) {
  if (P <= 0 || H <= 0 || S % P || P % H) return -1;
  const int64_t Sl = S / P, R = P / H;
  const char* src = (const char*)seq;
  char* dst = (char*)head;
  for (int64_t c = 0; c < P; ++c)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < S; ++t)
        for (int64_t d = 0; d < D; ++d) {
          const int64_t r = t / Sl, s = t % Sl, h = c / R;
          const int64_t si = (((r * B + b) * Sl + s) * H + h) * D + d;
          const int64_t di = ((c * B + b) * S + t) * D + d;
          memcpy(dst + di * eb, src + si * eb, (size_t)eb);
        }
  return 0;
}

/* bf16 bit pattern <-> float.  bf16 is the upper half of an IEEE binary32;
 * rounding to it keeps the upper 16 bits, rounded to nearest, ties to even. */
static float bf16_to_f32(uint16_t x) {
  uint32_t u = (uint32_t)x << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* The gradient of that replication: head j of the sequence shards receives
 * the sum of its R replicas' gradients, accumulated in fp32 in rank order and
 * rounded once to bf16.  head: [P][B][S][1][D] bf16  ->  seq: [P][B][S/P][H][D] */
int orc_reduce_replicated(const uint16_t* head, uint16_t* seq, int64_t P, int64_t B, int64_t S,
                          int64_t H, int64_t D) {
  if (P <= 0 || H <= 0 || S % P || P % H) return -1;
  const int64_t Sl = S / P, R = P / H;
  for (int64_t r = 0; r < P; ++r)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t s = 0; s < Sl; ++s)
        for (int64_t h = 0; h < H; ++h)
          for (int64_t d = 0; d < D; ++d) {
            float acc = 0.f;
            for (int64_t j = 0; j < R; ++j) {
              const int64_t c = h * R + j, t = r * Sl + s;
              acc += bf16_to_f32(head[((c * B + b) * S + t) * D + d]);
            }
            seq[(((r * B + b) * Sl + s) * H + h) * D + d] = f32_to_bf16(acc);
          }
  return 0;
}

/* The same sum from fp32 replica gradients (kept unrounded by the backward):
 * fp32 accumulation in rank order, one rounding to bf16.
 * head: [P][B][S][1][D] fp32  ->  seq: [P][B][S/P][H][D] bf16 */
int orc_reduce_replicated_f32(const float* head, uint16_t* seq, int64_t P, int64_t B, int64_t S,
                              int64_t H, int64_t D) {
  if (P <= 0 || H <= 0 || S % P || P % H) return -1;
  const int64_t Sl = S / P, R = P / H;
  for (int64_t r = 0; r < P; ++r)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t s = 0; s < Sl; ++s)
        for (int64_t h = 0; h < H; ++h)
          for (int64_t d = 0; d < D; ++d) {
            float acc = 0.f;
            for (int64_t j = 0; j < R; ++j) acc += head[(((h * R + j) * B + b) * S + r * Sl + s) * D + d];
            seq[(((r * B + b) * Sl + s) * H + h) * D + d] = f32_to_bf16(acc);
          }
  return 0;
}

/* --------------------------------------------------------------- segments */

/* shards: [P][B][S/P] int64  ->  gathered: [B][S] int64 (concatenation in rank order) */
int orc_gather_positions(const int64_t* shards, int64_t* gathered, int64_t P, int64_t B,
                         int64_t S) {
  if (P <= 0 || S % P) return -1;
  const int64_t Sl = S / P;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < S; ++t) gathered[b * S + t] = shards[((t / Sl) * B + b) * Sl + t % Sl];
  return 0;
}

/* gathered positions [B][S] -> cu (starts + total), n documents, longest document */
int orc_segments(const int64_t* pos, int64_t B, int64_t S, int32_t* cu, int64_t cap,
                 int32_t* n_out, int32_t* max_len_out) {
  int64_t n = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < S; ++i) {
      const int64_t t = b * S + i;
      if (i == 0 || pos[t] == 0) {
        if (n + 1 >= cap) return -5;
        cu[n++] = (int32_t)t;
      }
    }
  cu[n] = (int32_t)(B * S);
  int32_t mx = 0;
  for (int64_t k = 0; k < n; ++k)
    if (cu[k + 1] - cu[k] > mx) mx = cu[k + 1] - cu[k];
  *n_out = (int32_t)n;
  *max_len_out = mx;
  return 0;
}

/* -------------------------------------------------------------- attention */

typedef struct {
  const double* q;    /* [T][hq][D], T = B*S flattened tokens */
  const double* k;    /* [T][hkv][D] */
  const double* v;    /* [T][hkv][D] */
  const double* sink; /* [hq] or NULL */
  const int32_t* cu;  /* [n+1] document starts + total, or NULL: one document per batch row */
  int64_t n;
  int64_t B, S;
  int64_t hq, hkv, D;
  double scale;
  int64_t causal, wl, wr;
  /* keys restricted to positions [k_lo, k_hi) of each batch row (a KV chunk
     of the ring inner step; 0 and S: every key) */
  int64_t k_lo, k_hi;
} orc_prob;

/* Document index of every flattened token, and each document's first and
   one-past-last token. */
typedef struct {
  int64_t* doc;
  int64_t* first;
  int64_t* end;
} orc_docs;

static orc_docs doc_ids(const orc_prob* p) {
  const int64_t T = p->B * p->S;
  const size_t nb = sizeof(int64_t) * (size_t)(T > 0 ? T : 1);
  orc_docs dd = {(int64_t*)malloc(nb), (int64_t*)malloc(nb), (int64_t*)malloc(nb)};
  if (!p->cu) {
    for (int64_t t = 0; t < T; ++t) dd.doc[t] = t / p->S;
  } else {
    for (int64_t t = 0; t < T; ++t) dd.doc[t] = -1;
    for (int64_t d = 0; d < p->n; ++d)
      for (int64_t t = p->cu[d]; t < p->cu[d + 1]; ++t) dd.doc[t] = d;
  }
  for (int64_t t = 0; t < T; ++t)
    dd.first[t] = (t > 0 && dd.doc[t - 1] == dd.doc[t]) ? dd.first[t - 1] : t;
  for (int64_t t = T - 1; t >= 0; --t)
    dd.end[t] = (t + 1 < T && dd.doc[t + 1] == dd.doc[t]) ? dd.end[t + 1] : t + 1;
  return dd;
}

static void free_docs(orc_docs* dd) {
  free(dd->doc);
  free(dd->first);
  free(dd->end);
}

/* The mask: key j is visible to query i. */
static int allowed(const orc_prob* p, const orc_docs* dd, int64_t i, int64_t j) {
  if (dd->doc[i] != dd->doc[j] || dd->doc[i] < 0) return 0;
  if (j % p->S < p->k_lo || j % p->S >= p->k_hi) return 0;
  if (p->causal && j > i) return 0;
  if (p->wl >= 0 && i - j > p->wl) return 0;
  if (p->wr >= 0 && j - i > p->wr) return 0;
  return 1;
}

static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* Keys outside [lo, hi) are never visible to query i (other document,
   causal, window); the mask is still evaluated for every key in the range. */
static void key_range(const orc_prob* p, const orc_docs* dd, int64_t i, int64_t* lo,
                      int64_t* hi) {
  int64_t a = dd->first[i], b = dd->end[i];
  if (p->causal) b = min64(b, i + 1);
  if (p->wl >= 0) a = max64(a, i - p->wl);
  if (p->wr >= 0) b = min64(b, i + p->wr + 1);
  *lo = a;
  *hi = b > a ? b : a;
}

/* Queries outside [lo, hi) never see key j. */
static void query_range(const orc_prob* p, const orc_docs* dd, int64_t j, int64_t* lo,
                        int64_t* hi) {
  int64_t a = dd->first[j], b = dd->end[j];
  if (p->causal) a = max64(a, j);
  if (p->wl >= 0) b = min64(b, j + p->wl + 1);
  if (p->wr >= 0) a = max64(a, j - p->wr);
  *lo = a;
  *hi = b > a ? b : a;
}

static double dot(const double* x, const double* y, int64_t D) {
  double s = 0.0;
  for (int64_t d = 0; d < D; ++d) s += x[d] * y[d];
  return s;
}

/* Row i, query head h: logits, softmax, output row and log-sum-exp.
   s is scratch of length T. */
static void row_forward(const orc_prob* p, const orc_docs* doc, int64_t i, int64_t h,
                        double* s, double* o, double* lse) {
  const int64_t D = p->D, g = h / (p->hq / p->hkv);
  const double* qi = p->q + (i * p->hq + h) * D;
  int64_t lo, hi;
  key_range(p, doc, i, &lo, &hi);
  double m = -INFINITY;
  for (int64_t j = lo; j < hi; ++j) {
    if (!allowed(p, doc, i, j)) continue;
    s[j] = p->scale * dot(qi, p->k + (j * p->hkv + g) * D, D);
    if (s[j] > m) m = s[j];
  }
  if (p->sink && p->sink[h] > m) m = p->sink[h];
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  if (m == -INFINITY) { /* no visible key and no sink */
    *lse = -INFINITY;
    return;
  }
  double Z = 0.0;
  for (int64_t j = lo; j < hi; ++j) {
    if (!allowed(p, doc, i, j)) continue;
    const double e = exp(s[j] - m);
    Z += e;
    const double* vj = p->v + (j * p->hkv + g) * D;
    for (int64_t d = 0; d < D; ++d) o[d] += e * vj[d];
  }
  if (p->sink) Z += exp(p->sink[h] - m);
  for (int64_t d = 0; d < D; ++d) o[d] /= Z;
  *lse = m + log(Z);
}

/* Forward of the selected flattened rows (rows == NULL: every row).
   out: [nrows][hq][D], lse: [nrows][hq] (natural log). */
int orc_fwd(const orc_prob* p, const int64_t* rows, int64_t nrows, double* out, double* lse) {
  const int64_t T = p->B * p->S;
  if (p->hkv <= 0 || p->hq % p->hkv) return -3;
  if (!rows) nrows = T;
  orc_docs docs = doc_ids(p);
  const orc_docs* doc = &docs;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < nrows * p->hq; ++x) {
      const int64_t r = x / p->hq, h = x % p->hq;
      const int64_t i = rows ? rows[r] : r;
      row_forward(p, doc, i, h, s, out + (r * p->hq + h) * p->D, lse + r * p->hq + h);
    }
    free(s);
  }
  free_docs(&docs);
  return 0;
}

/* Backward.  dout: [T][hq][D].
   dQ of the selected rows (qrows == NULL: all; nq ignored then) -> dq [nq][hq][D];
   dK, dV of the selected keys (krows == NULL: all) -> dk, dv [nk][hkv][D];
   dsink [hq] when non-NULL (needs every row's statistics).
   Any output pointer may be NULL to skip it. */
int orc_bwd(const orc_prob* p, const double* dout, const int64_t* qrows, int64_t nq,
            double* dq, const int64_t* krows, int64_t nk, double* dk, double* dv,
            double* dsink) {
  const int64_t T = p->B * p->S, hq = p->hq, hkv = p->hkv, D = p->D;
  if (hkv <= 0 || hq % hkv) return -3;
  const int64_t G = hq / hkv;
  if (!qrows) nq = T;
  if (!krows) nk = T;
  orc_docs docs = doc_ids(p);
  const orc_docs* doc = &docs;

  /* 1. which rows need their softmax statistics (LSE_i and D_i) */
  char* need = (char*)calloc((size_t)(T > 0 ? T : 1), 1);
  if (dq)
    for (int64_t r = 0; r < nq; ++r) need[qrows ? qrows[r] : r] = 1;
  if (dk || dv)
    for (int64_t r = 0; r < nk; ++r) {
      const int64_t j = krows ? krows[r] : r;
      int64_t lo, hi;
      query_range(p, doc, j, &lo, &hi);
      for (int64_t i = lo; i < hi; ++i)
        if (allowed(p, doc, i, j)) need[i] = 1;
    }
  if (dsink)
    for (int64_t i = 0; i < T; ++i) need[i] = 1;

  /* 2. LSE_i and D_i = dO_i . O_i for those rows (NaN for the others: a
        result that read them would come out NaN, not silently wrong) */
  double* lse = (double*)malloc(sizeof(double) * (size_t)(T * hq > 0 ? T * hq : 1));
  double* Di = (double*)malloc(sizeof(double) * (size_t)(T * hq > 0 ? T * hq : 1));
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t x = 0; x < T * hq; ++x) {
      const int64_t i = x / hq, h = x % hq;
      if (!need[i]) {
        lse[x] = NAN;
        Di[x] = NAN;
        continue;
      }
      row_forward(p, doc, i, h, s, o, &lse[x]);
      Di[x] = dot(dout + x * D, o, D);
    }
    free(o);
    free(s);
  }

  /* 3. dQ_i = scale * sum_j P_ij (dP_ij - D_i) k_j */
  if (dq) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < nq * hq; ++x) {
      const int64_t r = x / hq, h = x % hq, i = qrows ? qrows[r] : r, g = h / G;
      const double* qi = p->q + (i * hq + h) * D;
      const double* doi = dout + (i * hq + h) * D;
      double* out = dq + (r * hq + h) * D;
      for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
      if (lse[i * hq + h] == -INFINITY) continue;
      int64_t lo, hi;
      key_range(p, doc, i, &lo, &hi);
      for (int64_t j = lo; j < hi; ++j) {
        if (!allowed(p, doc, i, j)) continue;
        const double* kj = p->k + (j * hkv + g) * D;
        const double* vj = p->v + (j * hkv + g) * D;
        const double P = exp(p->scale * dot(qi, kj, D) - lse[i * hq + h]);
        const double dS = P * (dot(doi, vj, D) - Di[i * hq + h]);
        for (int64_t d = 0; d < D; ++d) out[d] += p->scale * dS * kj[d];
      }
    }
  }

  /* 4. dK_j, dV_j summed over the query heads of KV head g and the rows that see j */
  if (dk || dv) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < nk * hkv; ++x) {
      const int64_t r = x / hkv, g = x % hkv, j = krows ? krows[r] : r;
      const double* kj = p->k + (j * hkv + g) * D;
      const double* vj = p->v + (j * hkv + g) * D;
      double* ok = dk ? dk + (r * hkv + g) * D : NULL;
      double* ov = dv ? dv + (r * hkv + g) * D : NULL;
      for (int64_t d = 0; d < D; ++d) {
        if (ok) ok[d] = 0.0;
        if (ov) ov[d] = 0.0;
      }
      int64_t lo, hi;
      query_range(p, doc, j, &lo, &hi);
      for (int64_t h = g * G; h < (g + 1) * G; ++h)
        for (int64_t i = lo; i < hi; ++i) {
          if (!allowed(p, doc, i, j)) continue;
          const double* qi = p->q + (i * hq + h) * D;
          const double* doi = dout + (i * hq + h) * D;
          const double P = exp(p->scale * dot(qi, kj, D) - lse[i * hq + h]);
          const double dS = P * (dot(doi, vj, D) - Di[i * hq + h]);
          for (int64_t d = 0; d < D; ++d) {
            if (ok) ok[d] += p->scale * dS * qi[d];
            if (ov) ov[d] += P * doi[d];
          }
        }
    }
  }

  /* 5. dsink_h = - sum_i exp(sink_h - LSE_i) D_i */
  if (dsink) {
    for (int64_t h = 0; h < hq; ++h) {
      double acc = 0.0;
      if (p->sink)
        for (int64_t i = 0; i < T; ++i)
          if (lse[i * hq + h] != -INFINITY) acc -= exp(p->sink[h] - lse[i * hq + h]) * Di[i * hq + h];
      dsink[h] = acc;
    }
  }
  free(Di);
  free(lse);
  free(need);
  free_docs(&docs);
  return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

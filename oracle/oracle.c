/*
 * oracle.c -- plain, slow FP64 reference for the Gated DeltaNet recurrent-state
 * path.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the GPU library never links, calls or
 * includes anything from here, and this file includes nothing of the GPU
 * library's (the two share no headers, helpers or constants).
 *
 * Everything is computed token by token in double precision, by the literal
 * definitions below, with no chunking, blocking or algebraic rearrangement.
 *
 * Sources (web pages, by title and section):
 *  [GDN]   "Gated DeltaNet" glossary entry (InferenceX), Technical definition:
 *          each step decays the state by a gate, applies a rank-one delta-rule
 *          correction, then projects the state by the query.
 *  [GDN2]  "Seven Architectures Replacing KV Cache With Bounded Mutable State",
 *          section Gated DeltaNet-2: the erase/write form
 *          S_t = Diag(alpha_t)(I - b_t k_t k_t^T) S_{t-1} + w_t k_t v_t^T, which
 *          is Gated DeltaNet when alpha, b and w are tied to scalars (b = w = beta).
 *          S here is d_k x d_v (rows indexed by the key dimension).
 *  [ONNX]  same article, section ONNX LinearAttention / FlashInfer: the four
 *          update rules (linear = plain additive, gated = exponential decay,
 *          delta = delta rule without decay, gated_delta = the full form,
 *          the default), past/present state of shape (B, H_kv, d_k, d_v), and
 *          grouped heads sharing a state across a group of query heads.
 *  [RS]    "Recurrent state" glossary entry (InferenceX), Why it matters: the
 *          state is stored in BF16 while computing in FP32, and prefix caching
 *          needs separate read (checkpoint) and write (live) slots.
 *  [GDN-E] "Gated DeltaNet" glossary entry, Engineering details / Why it
 *          matters: Conv1D is part of the layer, and checkpoint read slots
 *          differ from live write slots.
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes):
 *  - State orientation: M is d_k x d_v, row i = key index, contiguous along
 *    d_v, matching the (B, H_kv, d_k, d_v) state shape; output o = scale*M^T q.
 *  - The gate is passed as its logarithm g <= 0, a = exp(g); beta is the
 *    write strength.  One g and one beta per (token, state head).
 *  - linear:      M <- M + k v^T
 *    gated:       M <- a M + k v^T
 *    delta:       M <- (I - beta k k^T) M + beta k v^T
 *    gated_delta: M <- a (I - beta k k^T) M + beta k v^T
 *  - Grouped heads: state head h uses q/k head floor(h * H_qk / H_v).
 *  - Slots: past = pool[read_slot[r]], present = pool[write_slot[r]];
 *    read index -1 = zero initial state, write index -1 = no store, a NULL
 *    index array means slot r for request r.  An index outside [-1, n_slots)
 *    skips the request (nothing written for it) and sets bit 0 of the result.
 *  - BF16 state storage: wherever the state is stored, it is rounded from
 *    FP64 to the nearest BF16 value, ties to even (round_state != 0).
 *  - Front-end: per-channel causal conv of width conv_k (tap j multiplies
 *    x[t-(conv_k-1)+j], never across a sequence boundary; before the
 *    sequence's first token x is the stored window the sequence resumes, the
 *    raw inputs of the conv_k-1 tokens before it, else zero), then SiLU; q and k are then L2-normalised per
 *    (token, head) as y / sqrt(sum y^2 + eps); g = -softplus(a_raw) and
 *    beta = sigmoid(b_raw).
 *  - Channel-wise decay (Kimi Delta Attention, "Seven Architectures ...",
 *    Kimi Linear section): one log-decay per key channel, alpha_i = exp(g_i);
 *    the state is decayed row by row first, and the delta correction then
 *    reads the decayed state: S~ = Diag(alpha) S, S' = S~ + beta k (v - S~^T
 *    k)^T (without erase: S~ + k v^T).  The same page's GDN-2 section puts
 *    the decay after the erase and says that recovers KDA, which holds only
 *    for a scalar decay; the Kimi Linear section's own formula is followed.
 *  - Decode-side conv: the window a decode token sees is the conv_k-1 raw
 *    inputs before it, kept per request in a conv-state slot ([conv_k-1,
 *    channels], oldest first, channels in q|k|v order); read index -1 = no
 *    history (zeros, a fresh request), write index -1 = not stored, the same
 *    slot contract as the recurrent state.  The stored window holds raw
 *    inputs, so it is exact in the input precision.
 *  - 8-bit state storage ("Seven Architectures ...", ONNX LinearAttention /
 *    FlashInfer section and Limitations: DAMP keeps the high-risk key
 *    channels in higher precision and the rest in INT8, about 9.9 bits per
 *    value).  A key channel is a row of the d_k x d_v tile.  The first n_hi
 *    rows are stored in BF16; every other row in INT8 with its own scale:
 *    s = rowmax / 127, code = round-to-nearest-even(x * (127 / rowmax))
 *    clamped to [-127, 127], stored value code * s (a zero row: codes 0,
 *    s = 0).  The pages fix neither the scale granularity nor the rounding;
 *    this per-row absmax form is the plainest.  The code is an integer that
 *    floating point decides, so the decision is taken in binary32, the
 *    precision of the stored scale: x, rowmax, 127 / rowmax, the product and
 *    code * s are binary32 values.  Which channels are high-risk is a
 *    calibration result the pages leave to DAMP; here they are the first
 *    n_hi (a model orders its key channels so).  A stored tile is the BF16
 *    rows, the codes and the scales, zero-padded to a multiple of 256 bytes
 *    (the packing is in oracle/__init__.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 6

int oracle_version(void) { return ORACLE_VERSION; }

/* Nearest BF16 value (8 significant bits, binary32 exponent range) to x,
 * ties to even, returned as a double.  Written from the definition of the
 * format: scale x so one BF16 unit in the last place is 1, round to the
 * nearest integer with ties to even (nearbyint under the default rounding
 * mode), scale back.  NaN stays NaN, +-0 and +-inf are kept, values that
 * round past the largest finite BF16 become infinite. */
double oracle_round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  double ax = fabs(x);
  int e;
  frexp(ax, &e);          /* ax = m * 2^e, 0.5 <= m < 1 */
  int q = e - 8;          /* exponent of one unit in the 8th significant bit */
  if (q < -133) q = -133; /* below 2^-126 the spacing stays 2^-133 (subnormals) */
  double y = ldexp(nearbyint(ldexp(ax, -q)), q);
  if (y > 0x1.FEp127) y = INFINITY; /* largest finite BF16 is 255 * 2^120 */
  return copysign(y, x);
}

void oracle_round_bf16_array(const double *in, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* one token of the recurrence on one head's state, literal form             */

enum { R_LINEAR = 0, R_GATED = 1, R_DELTA = 2, R_GATED_DELTA = 3 };

/* M: d_k x d_v, updated in place; tmp: d_v scratch; o: d_v output. */
static void token_step(double *M, int dk, int dv, int rule, double scale,
                       const double *q, const double *k, const double *v,
                       double g, double beta, double *tmp, double *o) {
  int erase = (rule == R_DELTA || rule == R_GATED_DELTA);
  int decay = (rule == R_GATED || rule == R_GATED_DELTA);
  double a = decay ? exp(g) : 1.0;
  double w = erase ? beta : 1.0; /* write strength */
  if (erase) {
    /* (I - beta k k^T) M : tmp = k^T M, then M -= beta k tmp^T */
    for (int j = 0; j < dv; ++j) tmp[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) tmp[j] += k[i] * M[(int64_t)i * dv + j];
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) M[(int64_t)i * dv + j] -= beta * k[i] * tmp[j];
  }
  if (decay)
    for (int64_t e = 0; e < (int64_t)dk * dv; ++e) M[e] *= a;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) M[(int64_t)i * dv + j] += w * k[i] * v[j];
  /* read-out by the query: o = scale * M^T q */
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += M[(int64_t)i * dv + j] * q[i];
    o[j] = scale * s;
  }
}

/* ------------------------------------------------------------------------ */
/* a tiny thread pool: units [0, n_units) handed out round-robin              */

typedef void (*unit_fn)(void *ctx, int64_t unit, double *work);

typedef struct {
  unit_fn fn;
  void *ctx;
  int64_t n_units;
  int n_threads, tid;
  size_t work_len;
  int fail;
} pool_job;

static void *pool_worker(void *p) {
  pool_job *j = (pool_job *)p;
  double *work = (double *)malloc(j->work_len * sizeof(double));
  if (!work) { j->fail = 1; return NULL; }
  for (int64_t u = j->tid; u < j->n_units; u += j->n_threads) j->fn(j->ctx, u, work);
  free(work);
  return NULL;
}

static int run_units(unit_fn fn, void *ctx, int64_t n_units, size_t work_len, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if ((int64_t)n_threads > n_units) n_threads = (int)(n_units > 0 ? n_units : 1);
  pool_job jobs[256];
  pthread_t th[256];
  int created[256];
  int fail = 0;
  for (int t = 0; t < n_threads; ++t) {
    jobs[t].fn = fn; jobs[t].ctx = ctx; jobs[t].n_units = n_units;
    jobs[t].n_threads = n_threads; jobs[t].tid = t; jobs[t].work_len = work_len;
    jobs[t].fail = 0;
  }
  if (n_threads == 1) {
    pool_worker(&jobs[0]);
    return jobs[0].fail;
  }
  for (int t = 0; t < n_threads; ++t)
    created[t] = pthread_create(&th[t], NULL, pool_worker, &jobs[t]) == 0;
  for (int t = 0; t < n_threads; ++t) {
    if (created[t]) pthread_join(th[t], NULL);
    else fail = 1;
    fail |= jobs[t].fail;
  }
  return fail;
}

/* resolve a request's slots; returns 0 if the request must be skipped */
static int resolve_slots(const int32_t *read_slot, const int32_t *write_slot, int64_t r,
                         int64_t n_slots, int64_t *rs, int64_t *ws) {
  *rs = read_slot ? (int64_t)read_slot[r] : r;
  *ws = write_slot ? (int64_t)write_slot[r] : r;
  if (*rs < -1 || *rs >= n_slots) return 0;
  if (*ws < -1 || *ws >= n_slots) return 0;
  return 1;
}

/* ------------------------------------------------------------------------ */
/* decode: one token per request                                             */

typedef struct {
  int B, Hqk, Hv, dk, dv, rule, round_state;
  int64_t n_slots;
  double scale;
  const double *q, *k, *v, *g, *beta;
  double *pool;
  const int32_t *read_slot, *write_slot;
  double *o;
  volatile int *bad;
} decode_ctx;

static void decode_unit(void *p, int64_t unit, double *work) {
  decode_ctx *c = (decode_ctx *)p;
  int64_t r = unit / c->Hv;
  int h = (int)(unit % c->Hv);
  int hq = (int)((int64_t)h * c->Hqk / c->Hv);
  int64_t rs, ws;
  if (!resolve_slots(c->read_slot, c->write_slot, r, c->n_slots, &rs, &ws)) {
    *c->bad = 1;
    return;
  }
  int64_t tile = (int64_t)c->dk * c->dv;
  double *M = work, *tmp = work + tile;
  if (rs >= 0) memcpy(M, c->pool + (rs * c->Hv + h) * tile, tile * sizeof(double));
  else memset(M, 0, tile * sizeof(double));
  token_step(M, c->dk, c->dv, c->rule, c->scale,
             c->q + (r * c->Hqk + hq) * c->dk, c->k + (r * c->Hqk + hq) * c->dk,
             c->v + (r * c->Hv + h) * c->dv, c->g[r * c->Hv + h], c->beta[r * c->Hv + h],
             tmp, c->o + (r * c->Hv + h) * c->dv);
  if (ws >= 0) {
    double *dst = c->pool + (ws * c->Hv + h) * tile;
    for (int64_t e = 0; e < tile; ++e) dst[e] = c->round_state ? oracle_round_bf16(M[e]) : M[e];
  }
}

/* One decode token for B requests (Gated DeltaNet glossary, Technical
 * definition; update rules and state shape from the ONNX LinearAttention
 * section; slots from the Recurrent state glossary, Why it matters).
 * q, k: [B, Hqk, dk]; v: [B, Hv, dv]; g, beta: [B, Hv]; pool: [n_slots, Hv,
 * dk, dv] updated in place; o: [B, Hv, dv].  Returns 0, or 1 if any request
 * was skipped for an out-of-range slot, or -1 on bad arguments. */
int oracle_decode(int B, int Hqk, int Hv, int dk, int dv, int64_t n_slots, int rule,
                  double scale, int round_state, const double *q, const double *k,
                  const double *v, const double *g, const double *beta, double *pool,
                  const int32_t *read_slot, const int32_t *write_slot, double *o,
                  int n_threads) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0) return -1;
  volatile int bad = 0;
  decode_ctx c = {B, Hqk, Hv, dk, dv, rule, round_state, n_slots, scale, q, k, v, g, beta,
                  pool, read_slot, write_slot, o, &bad};
  if (run_units(decode_unit, &c, (int64_t)B * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* sequences: tokens of each sequence in order (the prefill recurrence)      */

typedef struct {
  int n_seq, Hqk, Hv, dk, dv, rule, round_state;
  int64_t n_slots;
  double scale;
  const int32_t *cu;
  const double *q, *k, *v, *g, *beta;
  double *pool;
  const int32_t *read_slot, *write_slot;
  double *o;
  volatile int *bad;
} seq_ctx;

static void seq_unit(void *p, int64_t unit, double *work) {
  seq_ctx *c = (seq_ctx *)p;
  int64_t s = unit / c->Hv;
  int h = (int)(unit % c->Hv);
  int hq = (int)((int64_t)h * c->Hqk / c->Hv);
  int64_t rs, ws;
  if (!resolve_slots(c->read_slot, c->write_slot, s, c->n_slots, &rs, &ws)) {
    *c->bad = 1;
    return;
  }
  int64_t tile = (int64_t)c->dk * c->dv;
  double *M = work, *tmp = work + tile;
  if (rs >= 0) memcpy(M, c->pool + (rs * c->Hv + h) * tile, tile * sizeof(double));
  else memset(M, 0, tile * sizeof(double));
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t)
    token_step(M, c->dk, c->dv, c->rule, c->scale,
               c->q + (t * c->Hqk + hq) * c->dk, c->k + (t * c->Hqk + hq) * c->dk,
               c->v + (t * c->Hv + h) * c->dv, c->g[t * c->Hv + h], c->beta[t * c->Hv + h],
               tmp, c->o + (t * c->Hv + h) * c->dv);
  if (ws >= 0) {
    double *dst = c->pool + (ws * c->Hv + h) * tile;
    for (int64_t e = 0; e < tile; ++e) dst[e] = c->round_state ? oracle_round_bf16(M[e]) : M[e];
  }
}

/* Sequential recurrence over n_seq variable-length sequences (cu: [n_seq+1]
 * token offsets).  q, k: [N, Hqk, dk]; v: [N, Hv, dv]; g, beta: [N, Hv];
 * o: [N, Hv, dv].  The initial state comes from read_slot[s], the final state
 * goes to write_slot[s]; only the final state is rounded when round_state is
 * set, because that is the only point where it is stored.  Return codes as
 * for oracle_decode. */
int oracle_sequences(int n_seq, const int32_t *cu, int Hqk, int Hv, int dk, int dv,
                     int64_t n_slots, int rule, double scale, int round_state, const double *q,
                     const double *k, const double *v, const double *g, const double *beta,
                     double *pool, const int32_t *read_slot, const int32_t *write_slot,
                     double *o, int n_threads) {
  if (n_seq < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0) return -1;
  for (int s = 0; s < n_seq; ++s)
    if (cu[s + 1] < cu[s]) return -1;
  volatile int bad = 0;
  seq_ctx c = {n_seq, Hqk, Hv, dk, dv, rule, round_state, n_slots, scale, cu, q, k, v, g, beta,
               pool, read_slot, write_slot, o, &bad};
  if (run_units(seq_unit, &c, (int64_t)n_seq * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* front-end: causal depthwise conv + SiLU, L2 norm of q and k, gates        */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* causal conv + SiLU of one channel column over one sequence.  Inputs
 * before the sequence's first token come from `init` (the K-1 raw tokens
 * that precede it, oldest first, row length C, this channel at column cw of
 * a row), or are 0 when init is NULL: the conv window a resumed sequence
 * continues from. */
static void conv_silu(const double *x, int64_t ld, int64_t c, int64_t t0, int64_t t1,
                      const double *w, int K, const double *init, int64_t C, int64_t cw,
                      double *y) {
  for (int64_t t = t0; t < t1; ++t) {
    double s = 0.0;
    for (int j = 0; j < K; ++j) {
      int64_t src = t - (K - 1) + j;
      if (src >= t0) s += w[j] * x[src * ld + c];
      else if (init) s += w[j] * init[(src - t0 + K - 1) * C + cw];
    }
    y[t * ld + c] = s * sigmoid(s);
  }
}

/* Front-end of one layer for n_seq sequences (conv fused with the layer per
 * the Gated DeltaNet glossary, Engineering details).  q_raw, k_raw:
 * [N, Hqk*dk]; v_raw: [N, Hv*dv]; wq, wk: [Hqk*dk, K]; wv: [Hv*dv, K];
 * a_raw, b_raw: [N, Hv].  init: NULL (every sequence starts from an empty
 * window) or [n_seq, K-1, C] with C = 2*Hqk*dk + Hv*dv, the raw q|k|v
 * inputs of the K-1 tokens before each sequence (oldest first): a sequence
 * resumed from a stored window, as a checkpoint is resumed (Recurrent state
 * glossary, Why it matters).  Outputs have the input shapes; g_out,
 * beta_out: [N, Hv]. */
int oracle_frontend(int n_seq, const int32_t *cu, int Hqk, int Hv, int dk, int dv, int K,
                    double eps, const double *q_raw, const double *k_raw, const double *v_raw,
                    const double *wq, const double *wk, const double *wv, const double *a_raw,
                    const double *b_raw, const double *init, double *q_out, double *k_out,
                    double *v_out, double *g_out, double *beta_out) {
  if (n_seq < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || K <= 0) return -1;
  int64_t cq = (int64_t)Hqk * dk, cv = (int64_t)Hv * dv, C = 2 * cq + cv;
  for (int s = 0; s < n_seq; ++s) {
    int64_t t0 = cu[s], t1 = cu[s + 1];
    if (t1 < t0) return -1;
    const double *win = init ? init + (int64_t)s * (K - 1) * C : NULL;
    for (int64_t c = 0; c < cq; ++c) {
      conv_silu(q_raw, cq, c, t0, t1, wq + c * K, K, win, C, c, q_out);
      conv_silu(k_raw, cq, c, t0, t1, wk + c * K, K, win, C, cq + c, k_out);
    }
    for (int64_t c = 0; c < cv; ++c)
      conv_silu(v_raw, cv, c, t0, t1, wv + c * K, K, win, C, 2 * cq + c, v_out);
    for (int64_t t = t0; t < t1; ++t) {
      for (int h = 0; h < Hqk; ++h) {
        double *yq = q_out + t * cq + (int64_t)h * dk, *yk = k_out + t * cq + (int64_t)h * dk;
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) { sq += yq[i] * yq[i]; sk += yk[i] * yk[i]; }
        double nq = sqrt(sq + eps), nk = sqrt(sk + eps);
        for (int i = 0; i < dk; ++i) { yq[i] /= nq; yk[i] /= nk; }
      }
      for (int h = 0; h < Hv; ++h) {
        g_out[t * Hv + h] = -softplus(a_raw[t * Hv + h]);
        beta_out[t * Hv + h] = sigmoid(b_raw[t * Hv + h]);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* decode-side front-end: one token per request, conv window from a slot     */

/* One decode token of the front-end for B requests.  The conv is part of the
 * layer (Gated DeltaNet glossary, Engineering details), so a decode token's
 * window continues the raw inputs of the tokens before it; those conv_k-1
 * inputs live in a conv-state slot, read and written like the recurrent
 * state's slots (Recurrent state glossary, Why it matters).
 * q_raw, k_raw: [B, Hqk*dk]; v_raw: [B, Hv*dv]; w*: [channels, K];
 * a_raw, b_raw: [B, Hv]; pool: [n_slots, K-1, C], C = 2*Hqk*dk + Hv*dv in
 * q|k|v channel order, entry 0 the oldest token, updated in place.  Outputs
 * as oracle_frontend's for one token per request.  A request with a slot
 * index outside [-1, n_slots) is skipped (nothing written) and the result
 * is 1; otherwise 0; -1 on bad arguments. */
int oracle_conv_decode(int B, int Hqk, int Hv, int dk, int dv, int K, double eps,
                       int64_t n_slots, const double *q_raw, const double *k_raw,
                       const double *v_raw, const double *wq, const double *wk,
                       const double *wv, const double *a_raw, const double *b_raw,
                       double *pool, const int32_t *read_slot, const int32_t *write_slot,
                       double *q_out, double *k_out, double *v_out, double *g_out,
                       double *beta_out) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || K < 1 || n_slots < 0) return -1;
  const int64_t cq = (int64_t)Hqk * dk, cv = (int64_t)Hv * dv, C = 2 * cq + cv;
  const int64_t slot_len = (int64_t)(K - 1) * C;
  double *win = (double *)malloc(sizeof(double) * (size_t)(K * C > 0 ? K * C : 1));
  if (!win) return -1;
  int bad = 0;
  for (int64_t r = 0; r < B; ++r) {
    int64_t rs, ws;
    if (!resolve_slots(read_slot, write_slot, r, n_slots, &rs, &ws)) { bad = 1; continue; }
    /* the window: K-1 tokens of history (zeros without a read slot), then this token */
    for (int j = 0; j < K - 1; ++j)
      for (int64_t c = 0; c < C; ++c)
        win[j * C + c] = rs >= 0 ? pool[rs * slot_len + j * C + c] : 0.0;
    for (int64_t c = 0; c < C; ++c) {
      double x;
      if (c < cq) x = q_raw[r * cq + c];
      else if (c < 2 * cq) x = k_raw[r * cq + (c - cq)];
      else x = v_raw[r * cv + (c - 2 * cq)];
      win[(int64_t)(K - 1) * C + c] = x;
    }
    /* conv over the window + SiLU, channel by channel */
    for (int64_t c = 0; c < C; ++c) {
      const double *w;
      double *y;
      if (c < cq) { w = wq + c * K; y = q_out + r * cq + c; }
      else if (c < 2 * cq) { w = wk + (c - cq) * K; y = k_out + r * cq + (c - cq); }
      else { w = wv + (c - 2 * cq) * K; y = v_out + r * cv + (c - 2 * cq); }
      double s = 0.0;
      for (int j = 0; j < K; ++j) s += w[j] * win[(int64_t)j * C + c];
      *y = s * sigmoid(s);
    }
    /* q and k to unit L2 norm per head; the gates */
    for (int h = 0; h < Hqk; ++h) {
      double *yq = q_out + r * cq + (int64_t)h * dk, *yk = k_out + r * cq + (int64_t)h * dk;
      double sq = 0.0, sk = 0.0;
      for (int i = 0; i < dk; ++i) { sq += yq[i] * yq[i]; sk += yk[i] * yk[i]; }
      double nq = sqrt(sq + eps), nk = sqrt(sk + eps);
      for (int i = 0; i < dk; ++i) { yq[i] /= nq; yk[i] /= nk; }
    }
    for (int h = 0; h < Hv; ++h) {
      g_out[r * Hv + h] = -softplus(a_raw[r * Hv + h]);
      beta_out[r * Hv + h] = sigmoid(b_raw[r * Hv + h]);
    }
    /* the window slides by one token into the write slot */
    if (ws >= 0)
      for (int j = 0; j < K - 1; ++j)
        for (int64_t c = 0; c < C; ++c) pool[ws * slot_len + j * C + c] = win[(int64_t)(j + 1) * C + c];
  }
  free(win);
  return bad;
}

/* ------------------------------------------------------------------------ */
/* decode with channel-wise decay: one log-decay per key channel             */

typedef struct {
  int B, Hqk, Hv, dk, dv, rule, round_state;
  int64_t n_slots;
  double scale;
  const double *q, *k, *v, *g, *beta;
  double *pool;
  const int32_t *read_slot, *write_slot;
  double *o;
  volatile int *bad;
  int n_hi; /* >= 0: the state is stored in the 8-bit format with n_hi BF16 rows */
} decode_cw_ctx;

static void q8_store(double *M, int dk, int dv, int n_hi, int8_t *codes, float *scales);

/* One token of the channel-wise decay recurrence on one head's state S
 * (d_k x d_v, updated in place): row i decays by alpha_i = exp(g[i]), then
 * the write beta k (v - S~^T k)^T reads the decayed state S~ (without erase:
 * k v^T), then o = scale S^T q.  rd: d_v scratch. */
static void cw_step(double *S, int dk, int dv, int rule, double scale, const double *q,
                    const double *k, const double *v, const double *g, double beta, double *rd,
                    double *o) {
  const int decay = rule == 1 || rule == 3, erase = rule >= 2;
  /* decay row i (key channel i) by its own alpha_i */
  if (decay)
    for (int i = 0; i < dk; ++i) {
      const double a = exp(g[i]);
      for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] *= a;
    }
  /* the write: beta k (v - S~^T k)^T with erase, k v^T without */
  for (int j = 0; j < dv; ++j) {
    double read = 0.0;
    if (erase)
      for (int i = 0; i < dk; ++i) read += S[(int64_t)i * dv + j] * k[i];
    rd[j] = erase ? beta * (v[j] - read) : v[j];
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(int64_t)i * dv + j] += k[i] * rd[j];
  /* read-out from the new state */
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * q[i];
    o[j] = scale * acc;
  }
}

static void decode_cw_unit(void *p, int64_t unit, double *work) {
  decode_cw_ctx *c = (decode_cw_ctx *)p;
  int64_t r = unit / c->Hv;
  int h = (int)(unit % c->Hv);
  int hq = (int)((int64_t)h * c->Hqk / c->Hv);
  int64_t rs, ws;
  if (!resolve_slots(c->read_slot, c->write_slot, r, c->n_slots, &rs, &ws)) {
    *c->bad = 1;
    return;
  }
  const int dk = c->dk, dv = c->dv;
  int64_t tile = (int64_t)dk * dv;
  double *S = work, *rd = work + tile;
  if (rs >= 0) memcpy(S, c->pool + (rs * c->Hv + h) * tile, tile * sizeof(double));
  else memset(S, 0, tile * sizeof(double));
  cw_step(S, dk, dv, c->rule, c->scale, c->q + (r * c->Hqk + hq) * dk,
          c->k + (r * c->Hqk + hq) * dk, c->v + (r * c->Hv + h) * dv,
          c->g + (r * c->Hv + h) * dk, c->beta ? c->beta[r * c->Hv + h] : 1.0, rd,
          c->o + (r * c->Hv + h) * dv);
  if (ws >= 0) {
    double *dst = c->pool + (ws * c->Hv + h) * tile;
    if (c->n_hi >= 0) {
      q8_store(S, dk, dv, c->n_hi, NULL, NULL);
      memcpy(dst, S, tile * sizeof(double));
    } else {
      for (int64_t e = 0; e < tile; ++e) dst[e] = c->round_state ? oracle_round_bf16(S[e]) : S[e];
    }
  }
}

/* One decode token for B requests with a per-key-channel decay (Kimi Delta
 * Attention, Kimi Linear section).  As oracle_decode, except g is
 * [B, Hv, dk]: the log-decay of each key channel of each state head. */
int oracle_decode_cw(int B, int Hqk, int Hv, int dk, int dv, int64_t n_slots, int rule,
                     double scale, int round_state, const double *q, const double *k,
                     const double *v, const double *g, const double *beta, double *pool,
                     const int32_t *read_slot, const int32_t *write_slot, double *o,
                     int n_threads) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0) return -1;
  volatile int bad = 0;
  decode_cw_ctx c = {B, Hqk, Hv, dk, dv, rule, round_state, n_slots, scale, q, k, v, g, beta,
                     pool, read_slot, write_slot, o, &bad, -1};
  if (run_units(decode_cw_unit, &c, (int64_t)B * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

/* The same with the state stored in the 8-bit format (n_hi BF16 rows, the
 * rest INT8 per row; pool holds the values the stored tiles represent). */
int oracle_decode_cw_q8(int B, int Hqk, int Hv, int dk, int dv, int64_t n_slots, int rule,
                        double scale, int n_hi, const double *q, const double *k,
                        const double *v, const double *g, const double *beta, double *pool,
                        const int32_t *read_slot, const int32_t *write_slot, double *o,
                        int n_threads) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0 || n_hi < 0 || n_hi > dk) return -1;
  volatile int bad = 0;
  decode_cw_ctx c = {B, Hqk, Hv, dk, dv, rule, 0, n_slots, scale, q, k, v, g, beta,
                     pool, read_slot, write_slot, o, &bad, n_hi};
  if (run_units(decode_cw_unit, &c, (int64_t)B * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* 8-bit state storage with a BF16 head of key channels                      */

/* Store one d_k x d_v tile in the 8-bit format and replace its values by the
 * ones the stored tile represents.  codes [(dk - n_hi) * dv] and scales
 * [dk - n_hi] receive the stored INT8 rows when non-NULL. */
static void q8_store(double *M, int dk, int dv, int n_hi, int8_t *codes, float *scales) {
  for (int i = 0; i < dk; ++i) {
    double *row = M + (int64_t)i * dv;
    if (i < n_hi) {
      for (int j = 0; j < dv; ++j) row[j] = oracle_round_bf16(row[j]);
      continue;
    }
    float m = 0.0f;
    for (int j = 0; j < dv; ++j) {
      float ax = fabsf((float)row[j]);
      if (ax > m) m = ax;
    }
    const float inv = m > 0.0f ? 127.0f / m : 0.0f;
    const float sc = m / 127.0f;
    for (int j = 0; j < dv; ++j) {
      float y = (float)row[j] * inv;
      if (y > 127.0f) y = 127.0f;
      if (y < -127.0f) y = -127.0f;
      const float c = nearbyintf(y);
      row[j] = (double)(c * sc);
      if (codes) codes[(int64_t)(i - n_hi) * dv + j] = (int8_t)c;
    }
    if (scales) scales[i - n_hi] = sc;
  }
}

/* Encode n_tiles tiles of values [n_tiles, dk, dv] in the 8-bit format: the
 * BF16 rows are returned as their (exact) values in bf16_rows [n_tiles, n_hi,
 * dv]; codes [n_tiles, dk - n_hi, dv]; scales [n_tiles, dk - n_hi].  values
 * is left unchanged.  Returns 0, or -1 on bad arguments. */
int oracle_q8_encode(int64_t n_tiles, int dk, int dv, int n_hi, const double *values,
                     double *bf16_rows, int8_t *codes, float *scales) {
  if (n_tiles < 0 || dk <= 0 || dv <= 0 || n_hi < 0 || n_hi > dk) return -1;
  const int64_t tile = (int64_t)dk * dv;
  double *M = (double *)malloc(sizeof(double) * (size_t)tile);
  if (!M) return -1;
  for (int64_t t = 0; t < n_tiles; ++t) {
    memcpy(M, values + t * tile, sizeof(double) * (size_t)tile);
    q8_store(M, dk, dv, n_hi, codes + t * (int64_t)(dk - n_hi) * dv, scales + t * (dk - n_hi));
    memcpy(bf16_rows + t * (int64_t)n_hi * dv, M, sizeof(double) * (size_t)n_hi * dv);
  }
  free(M);
  return 0;
}

typedef struct {
  int B, Hqk, Hv, dk, dv, rule, n_hi;
  int64_t n_slots;
  double scale;
  const double *q, *k, *v, *g, *beta;
  double *pool;
  const int32_t *read_slot, *write_slot;
  double *o;
  volatile int *bad;
} decode_q8_ctx;

static void decode_q8_unit(void *p, int64_t unit, double *work) {
  decode_q8_ctx *c = (decode_q8_ctx *)p;
  int64_t r = unit / c->Hv;
  int h = (int)(unit % c->Hv);
  int hq = (int)((int64_t)h * c->Hqk / c->Hv);
  int64_t rs, ws;
  if (!resolve_slots(c->read_slot, c->write_slot, r, c->n_slots, &rs, &ws)) {
    *c->bad = 1;
    return;
  }
  int64_t tile = (int64_t)c->dk * c->dv;
  double *M = work, *tmp = work + tile;
  if (rs >= 0) memcpy(M, c->pool + (rs * c->Hv + h) * tile, tile * sizeof(double));
  else memset(M, 0, tile * sizeof(double));
  token_step(M, c->dk, c->dv, c->rule, c->scale,
             c->q + (r * c->Hqk + hq) * c->dk, c->k + (r * c->Hqk + hq) * c->dk,
             c->v + (r * c->Hv + h) * c->dv, c->g[r * c->Hv + h], c->beta[r * c->Hv + h],
             tmp, c->o + (r * c->Hv + h) * c->dv);
  if (ws >= 0) {
    q8_store(M, c->dk, c->dv, c->n_hi, NULL, NULL);
    memcpy(c->pool + (ws * c->Hv + h) * tile, M, tile * sizeof(double));
  }
}

/* One decode token for B requests on a state pool kept in the 8-bit format.
 * As oracle_decode, except that pool holds the values the stored tiles
 * represent and the new state is stored in the 8-bit format (n_hi BF16
 * rows, the rest INT8 per row) at the write slot. */
int oracle_decode_q8(int B, int Hqk, int Hv, int dk, int dv, int64_t n_slots, int rule,
                     double scale, int n_hi, const double *q, const double *k, const double *v,
                     const double *g, const double *beta, double *pool,
                     const int32_t *read_slot, const int32_t *write_slot, double *o,
                     int n_threads) {
  if (B < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0 || n_hi < 0 || n_hi > dk) return -1;
  volatile int bad = 0;
  decode_q8_ctx c = {B, Hqk, Hv, dk, dv, rule, n_hi, n_slots, scale, q, k, v, g, beta,
                     pool, read_slot, write_slot, o, &bad};
  if (run_units(decode_q8_unit, &c, (int64_t)B * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

/* ------------------------------------------------------------------------ */
/* sequences with a channel-wise decay (the prefill recurrence of KDA)       */

static void seq_cw_unit(void *p, int64_t unit, double *work) {
  seq_ctx *c = (seq_ctx *)p;
  int64_t s = unit / c->Hv;
  int h = (int)(unit % c->Hv);
  int hq = (int)((int64_t)h * c->Hqk / c->Hv);
  int64_t rs, ws;
  if (!resolve_slots(c->read_slot, c->write_slot, s, c->n_slots, &rs, &ws)) {
    *c->bad = 1;
    return;
  }
  const int dk = c->dk, dv = c->dv;
  int64_t tile = (int64_t)dk * dv;
  double *S = work, *rd = work + tile;
  if (rs >= 0) memcpy(S, c->pool + (rs * c->Hv + h) * tile, tile * sizeof(double));
  else memset(S, 0, tile * sizeof(double));
  for (int64_t t = c->cu[s]; t < c->cu[s + 1]; ++t)
    cw_step(S, dk, dv, c->rule, c->scale, c->q + (t * c->Hqk + hq) * dk,
            c->k + (t * c->Hqk + hq) * dk, c->v + (t * c->Hv + h) * dv,
            c->g + (t * c->Hv + h) * dk, c->beta ? c->beta[t * c->Hv + h] : 1.0, rd,
            c->o + (t * c->Hv + h) * dv);
  if (ws >= 0) {
    double *dst = c->pool + (ws * c->Hv + h) * tile;
    for (int64_t e = 0; e < tile; ++e) dst[e] = c->round_state ? oracle_round_bf16(S[e]) : S[e];
  }
}

/* The channel-wise decay recurrence (Kimi Delta Attention, Kimi Linear
 * section) over n_seq variable-length sequences: as oracle_sequences, except
 * g is [N, Hv, dk], one log-decay per key channel of each state head. */
int oracle_sequences_cw(int n_seq, const int32_t *cu, int Hqk, int Hv, int dk, int dv,
                        int64_t n_slots, int rule, double scale, int round_state,
                        const double *q, const double *k, const double *v, const double *g,
                        const double *beta, double *pool, const int32_t *read_slot,
                        const int32_t *write_slot, double *o, int n_threads) {
  if (n_seq < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || rule < 0 || rule > 3) return -1;
  if (Hv % Hqk != 0) return -1;
  for (int s = 0; s < n_seq; ++s)
    if (cu[s + 1] < cu[s]) return -1;
  volatile int bad = 0;
  seq_ctx c = {n_seq, Hqk, Hv, dk, dv, rule, round_state, n_slots, scale, cu, q, k, v, g, beta,
               pool, read_slot, write_slot, o, &bad};
  if (run_units(seq_cw_unit, &c, (int64_t)n_seq * Hv, (size_t)dk * dv + dv, n_threads)) return -1;
  return bad ? 1 : 0;
}

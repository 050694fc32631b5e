/*
 * gdn.h -- C ABI of an MI355X (gfx950) library for the Gated DeltaNet
 * recurrent-state hot path: one-token decode over a batch of slot-indexed
 * states, a fused causal-conv/SiLU/L2-norm/gate front-end, a chunked prefill
 * over variable-length sequences, and a single launch that mixes the two.
 *
 * The operation (web pages, by title and section):
 *  - "Gated DeltaNet" glossary entry, Technical definition: at each step the
 *    per-head state is decayed by a gate, corrected by a rank-one delta-rule
 *    term, and read out by the query.
 *  - "Seven Architectures Replacing KV Cache With Bounded Mutable State",
 *    Gated DeltaNet-2 section: S_t = a_t (I - beta_t k_t k_t^T) S_{t-1}
 *    + beta_t k_t v_t^T once the gates are tied to scalars, with S of size
 *    d_k x d_v; Kimi Linear section: the same update in residual form
 *    S_t = a S + beta k (v - a S^T k)^T.
 *  - Same article, ONNX LinearAttention / FlashInfer section: update_rule in
 *    {linear, gated, delta, gated_delta} (default gated_delta), optional
 *    past_state / present_state of shape (B, H_kv, d_k, d_v), grouped heads.
 *  - "Recurrent state" glossary entry, Engineering details / Why it matters:
 *    slots for the state, BF16 storage with FP32 compute, and separate read
 *    (checkpoint) and write (live) slots for prefix caching.
 *  - "Gated DeltaNet" glossary entry, Engineering details: Conv1D fused with
 *    the layer.
 *
 * Conventions shared by every call:
 *  - Every tensor argument is a DEVICE pointer to contiguous row-major memory
 *    that the caller owns, aligned to its element size; q, k, v, o, the
 *    state pool, the front-end's raw inputs, conv weights and outputs, and
 *    the workspace are read and written as 16-byte vectors and must be
 *    16-byte aligned (GDN_ERR_ALIGN otherwise); the library never allocates, frees or
 *    synchronises, keeps no global mutable state other than one cached device
 *    address per GPU for gdn_prefill_noalloc, and reads argument structs
 *    only during the call.  All work is enqueued on `stream` (a hipStream_t;
 *    NULL = the null stream).
 *  - State tensors hold M = S with rows indexed by the key dimension:
 *    pool[n_slots][H_v][d_k][d_v]; the output is o = scale * M_t^T q_t, read
 *    after the token's update.  State head h uses q/k head
 *    h / (H_v / H_qk) (contiguous groups); H_v must be a multiple of H_qk.
 *  - Gates: g is the log of the decay (a = exp(g), g <= 0 normally) and beta
 *    the write strength, one FP32 value per (token, state head).
 *      linear:      M <- M + k v^T                    (g, beta ignored)
 *      gated:       M <- a M + k v^T                  (beta ignored)
 *      delta:       M <- (I - beta k k^T) M + beta k v^T  (g ignored)
 *      gated_delta: M <- a (I - beta k k^T) M + beta k v^T
 *  - Slots: past = pool[read_slot[r]], present = pool[write_slot[r]].  A read
 *    index of -1 means a zero initial state, a write index of -1 means the
 *    new state is not stored; a NULL index array means slot r for request r
 *    (then n_slots must cover the batch).  An index outside [-1, n_slots)
 *    makes the kernel skip that request (neither o nor the state is written
 *    for it) and set GDN_DEVICE_BAD_SLOT in *status when status is non-NULL.
 *  - Caller contract: write indices >= 0 are unique within a call, and no
 *    request's write index equals another request's read index (a request
 *    may read and write the same slot).  gdn_validate_slots checks this on
 *    host copies.  Violations give undefined results, never out-of-bounds
 *    accesses.
 *  - Synchronous errors (bad pointer, shape, dtype, rule, workspace) return
 *    a non-zero gdn_status and launch nothing; a failed launch returns
 *    GDN_ERR_LAUNCH.
 *  - Supported sizes: d_k, d_v in {16, 32, 64, 128}; chunk = 64; conv_k = 4.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 10

typedef enum gdn_rule {
  GDN_RULE_LINEAR = 0,
  GDN_RULE_GATED = 1,
  GDN_RULE_DELTA = 2,
  GDN_RULE_GATED_DELTA = 3
} gdn_rule;

/* Element types.  GDN_Q8 is a state storage format only (gdn_decode's
 * state_dtype): DAMP's mixed precision ("Seven Architectures ...", ONNX
 * LinearAttention / FlashInfer section and Limitations: high-risk key
 * channels kept in higher precision, the rest in INT8, ~9.9 bits per value).
 * Each (slot, head) tile stores its first state_bf16_rows key channels (rows)
 * in BF16 and every other row in INT8 with one binary32 scale per row:
 *   [state_bf16_rows, d_v] BF16 | [d_k - state_bf16_rows, d_v] int8 codes |
 *   [d_k - state_bf16_rows] binary32 scales | zero padding to a multiple of
 *   256 bytes (gdn_state_q8_bytes per head; tiles start on 256-byte lines).  An INT8 row represents code * scale; when
 * stored it is requantised against its own largest magnitude rowmax:
 * code = round-to-nearest-even(x * (127 / rowmax)) within [-127, 127] and
 * scale = rowmax / 127, in binary32 (an all-zero row: codes and scale 0).
 * INT8 rows hold finite values only.  The BF16 rows are the model's
 * high-risk key channels: a calibration that picks other channels orders the
 * key dimension of its q/k projections so they come first (the conv, norm
 * and recurrence treat key channels alike). */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_Q8 = 2 } gdn_dtype;

/* How the decay of the gated rules is given.  HEAD: one per (token, state
 * head), Gated DeltaNet's scalar forget gate.  CHANNEL: one per key channel
 * of each state head, the channel-wise gate of Kimi Delta Attention ("Seven
 * Architectures ...", Kimi Linear section): row i of the state decays by
 * exp(g_i) before the delta correction reads the state, i.e.
 * M' = D M + beta k (v - (D M)^T k)^T with D = Diag(exp(g)). */
typedef enum gdn_decay_mode { GDN_DECAY_HEAD = 0, GDN_DECAY_CHANNEL = 1 } gdn_decay_mode;

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or inconsistent */
  GDN_ERR_DTYPE = 3,       /* unknown dtype code */
  GDN_ERR_RULE = 4,        /* unknown update rule */
  GDN_ERR_UNSUPPORTED = 5, /* a valid but unsupported size (d, chunk, conv width, head ratio) */
  GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than gdn_prefill_workspace_size */
  GDN_ERR_LAUNCH = 7,      /* the HIP runtime refused a launch */
  GDN_ERR_SLOTS = 8,       /* gdn_validate_slots found a range error or a hazard */
  GDN_ERR_ALIGN = 9,       /* a tensor pointer that is read as 16-byte vectors is not 16-byte aligned */
  GDN_ERR_SCRATCH = 10     /* gdn_prefill_noalloc: the call needs more workspace than the
                              library's fixed device workspace holds */
} gdn_status;

/* bits set in the optional device status word: a request (decode) or
 * sequence (prefill) was skipped because of a slot index outside
 * [-1, n_slots), or a prefill sequence whose offsets lie outside
 * [0, n_tokens] or decrease */
#define GDN_DEVICE_BAD_SLOT 1u
#define GDN_DEVICE_BAD_SEQ 2u

/* Decode: one token for each of B requests (the per-token recurrence of the
 * "Gated DeltaNet" glossary entry, Technical definition; the residual /
 * rearranged read-out of its Engineering details). */
typedef struct gdn_decode_args {
  int32_t B;           /* requests (>= 0; 0 launches nothing) */
  int32_t H_qk;        /* q/k heads */
  int32_t H_v;         /* state heads (the H_kv of the state shape), multiple of H_qk */
  int32_t d_k, d_v;    /* state tile is d_k x d_v */
  int32_t rule;        /* gdn_rule */
  int32_t state_dtype; /* gdn_dtype of state_pool: BF16 storage with FP32 compute, FP32, or
                          GDN_Q8 (then state_pool is [n_slots, H_v, gdn_state_q8_bytes(1, ...)]
                          bytes; gdn_decode only) */
  int32_t act_dtype;   /* gdn_dtype of q, k, v and o */
  int64_t n_slots;     /* pool capacity in slots */
  float scale;         /* read-out scale (1.0 for none) */
  int32_t decay_mode;  /* gdn_decay_mode: the shape of g (gdn_mixed: the prefill half's
                          decay_mode when both halves are present) */
  const void *q;       /* [B, H_qk, d_k] act_dtype; normalised by the caller */
  const void *k;       /* [B, H_qk, d_k] act_dtype */
  const void *v;       /* [B, H_v, d_v] act_dtype */
  const float *g;      /* log-decay, [B, H_v] (GDN_DECAY_HEAD) or [B, H_v, d_k]
                          (GDN_DECAY_CHANNEL, 16-byte aligned); unused by linear and delta
                          (may be NULL then) */
  const float *beta;   /* [B, H_v] write strength (unused by linear and gated; may be NULL then) */
  void *state_pool;    /* [n_slots, H_v, d_k, d_v] state_dtype, read and written in place */
  const int32_t *read_slot;  /* [B] or NULL */
  const int32_t *write_slot; /* [B] or NULL */
  void *o;             /* [B, H_v, d_v] act_dtype */
  uint32_t *status;    /* optional device word; bits are OR-ed in, never cleared */
  int32_t state_bf16_rows; /* state_dtype GDN_Q8: key channels per tile kept in BF16, a
                              multiple of gdn_state_q8_row_quantum(d_k, d_v) in [0, d_k]
                              (32 at d_k = d_v = 128); must be 0 otherwise */
  int32_t reserved0;   /* must be 0 */
} gdn_decode_args;

/* Prefill: the same recurrence over n_seq variable-length sequences packed
 * along the token axis, evaluated chunk by chunk (chunk = 64 tokens).  With
 * use_frontend = 1 the inputs are raw projections: each channel goes through
 * a causal depthwise conv of width conv_k (tap j multiplies x[t-conv_k+1+j],
 * zero before a sequence's first token) and SiLU; q and k are then scaled to
 * unit L2 norm per (token, head) as y / sqrt(sum y^2 + eps); g =
 * -softplus(a_raw), beta = sigmoid(b_raw).  With use_frontend = 0, q/k/v and
 * g/beta are used as given. */
typedef struct gdn_prefill_args {
  int32_t n_seq;       /* sequences (>= 0) */
  int32_t H_qk, H_v, d_k, d_v;
  int32_t rule, state_dtype, act_dtype;
  int32_t use_frontend; /* 0 or 1 */
  int32_t conv_k;      /* conv width; 4 (ignored when use_frontend = 0) */
  int32_t chunk;       /* 64 */
  int32_t ckpt_interval; /* 0, or tokens between intermediate checkpoints: a positive multiple
                            of chunk (see ckpt_slot) */
  int64_t n_tokens;    /* total tokens = cu_seqlens[n_seq] */
  int64_t n_slots;
  float scale;         /* read-out scale */
  float eps;           /* L2-norm epsilon (front-end only), e.g. 1e-6 */
  const int32_t *cu_seqlens; /* [n_seq + 1] device, non-decreasing, cu[0] = 0, cu[n_seq] = n_tokens;
                                a sequence s with cu[s] < 0, cu[s+1] < cu[s] or cu[s+1] > n_tokens is
                                skipped (no o, no state) and sets GDN_DEVICE_BAD_SEQ */
  const void *q;       /* [n_tokens, H_qk * d_k] act_dtype (raw or final) */
  const void *k;       /* [n_tokens, H_qk * d_k] act_dtype */
  const void *v;       /* [n_tokens, H_v * d_v] act_dtype */
  const float *g;      /* [n_tokens, H_v] log-decay when use_frontend = 0 ([n_tokens, H_v, d_k]
                          with GDN_DECAY_CHANNEL) */
  const float *beta;   /* [n_tokens, H_v] write strength when use_frontend = 0 */
  const float *a_raw;  /* [n_tokens, H_v] when use_frontend = 1: g = -softplus(a_raw) */
  const float *b_raw;  /* [n_tokens, H_v] when use_frontend = 1: beta = sigmoid(b_raw) */
  const float *conv_wq;  /* [H_qk * d_k, conv_k] when use_frontend = 1 */
  const float *conv_wk;  /* [H_qk * d_k, conv_k] */
  const float *conv_wv;  /* [H_v * d_v, conv_k] */
  void *state_pool;    /* [n_slots, H_v, d_k, d_v] state_dtype */
  const int32_t *read_slot;  /* [n_seq] or NULL: initial state (-1 = zero, a fresh request) */
  const int32_t *write_slot; /* [n_seq] or NULL: final state (-1 = not stored) */
  void *o;             /* [n_tokens, H_v, d_v] act_dtype */
  void *workspace;     /* device scratch of gdn_prefill_workspace_size() bytes (may be NULL if 0) */
  size_t workspace_bytes;
  uint32_t *status;    /* optional device word */
  /* Intermediate checkpoints at block boundaries ("Gated DeltaNet" glossary
   * entry, Why it matters: hybrid prefix caching keeps GDN checkpoints in
   * their own slots, aligned to KV block boundaries).  With ckpt_interval > 0,
   * ckpt_slot[s * ckpt_per_seq + j] receives sequence s's state after its
   * first (j + 1) * ckpt_interval tokens, if it has that many (j <
   * ckpt_per_seq): FP32 across chunks, rounded once when stored as BF16, the
   * value a prefill of just those tokens would store in its write slot.  -1
   * stores nothing; an index outside [-1, n_slots) stores nothing and sets
   * GDN_DEVICE_BAD_SLOT.  Checkpoint slots follow the write-slot contract
   * (unique, no other request's read slot).  Ignored when ckpt_interval = 0. */
  const int32_t *ckpt_slot; /* [n_seq, ckpt_per_seq] device */
  int32_t ckpt_per_seq;
  int32_t decay_mode;  /* gdn_decay_mode.  GDN_DECAY_CHANNEL: g is [n_tokens, H_v, d_k], one
                          log-decay per key channel (Kimi Delta Attention), with use_frontend = 0
                          (q, k, v, g, beta given); FP32 state or activations then need
                          d_k <= 64 */
  /* The front-end's conv window across calls (use_frontend = 1; with
   * use_frontend = 0 the three slot arrays must be NULL).  conv_pool is the
   * conv-state pool of gdn_conv_args: [conv_n_slots, conv_k - 1, C]
   * act_dtype, C = 2 * H_qk * d_k + H_v * d_v raw channels in q|k|v order,
   * oldest token first.  A sequence that resumes a stored state resumes its
   * conv window too (the conv is part of the layer, "Gated DeltaNet"
   * glossary entry, Engineering details; checkpoints are resumed, "Recurrent
   * state" glossary entry, Why it matters):
   *  - conv_read_slot[s]: the window before sequence s's first token (its
   *    conv_k - 1 previous raw inputs); -1 or a NULL array = an empty window
   *    (zeros), as a fresh request starts.
   *  - conv_write_slot[s]: receives the window sequence s leaves (its last
   *    conv_k - 1 raw inputs; when it has fewer tokens, the older rows come
   *    from the window it resumed), what gdn_conv_decode continues from.
   *  - conv_ckpt_slot[s * ckpt_per_seq + j]: the window at intermediate
   *    checkpoint j (the raw inputs of the conv_k - 1 tokens before token
   *    (j + 1) * ckpt_interval of the sequence), stored beside ckpt_slot's
   *    state under the same conditions.
   * -1 stores nothing; an index outside [-1, conv_n_slots) is read as an
   * empty window or stores nothing, and sets GDN_DEVICE_BAD_SLOT.  Conv slots
   * follow the write-slot contract among themselves (a sequence may write
   * the slot it reads).  The windows are raw inputs: copied bit for bit. */
  void *conv_pool;
  int64_t conv_n_slots;
  const int32_t *conv_read_slot;  /* [n_seq] device or NULL */
  const int32_t *conv_write_slot; /* [n_seq] device or NULL */
  const int32_t *conv_ckpt_slot;  /* [n_seq, ckpt_per_seq] device or NULL */
} gdn_prefill_args;

/* The front-end's conv window across calls.  The short conv is part of the
 * layer ("Gated DeltaNet" glossary entry, Engineering details), so a decode
 * token's conv window holds the raw inputs of the conv_k - 1 tokens before
 * it.  They live per request in a conv-state slot of conv_pool, laid out
 * [n_slots, conv_k - 1, C] in act_dtype with C = 2 * H_qk * d_k + H_v * d_v
 * channels in q|k|v order, the oldest token first; slots follow the
 * recurrent state's read/write rules ("Recurrent state" glossary entry, Why
 * it matters).  gdn_conv_decode runs the front-end for one token per request
 * and slides the window; gdn_conv_store fills slots from prefilled
 * sequences.  A prefill reads and stores windows through gdn_prefill_args'
 * conv fields. */
typedef struct gdn_conv_args {
  int32_t B;           /* requests (gdn_conv_decode) or sequences (gdn_conv_store), >= 0 */
  int32_t H_qk, H_v, d_k, d_v;
  int32_t act_dtype;   /* gdn_dtype of the raw inputs, q_out/k_out/v_out and conv_pool */
  int32_t conv_k;      /* conv width; 4 */
  int32_t reserved0;   /* must be 0 */
  int64_t n_slots;     /* conv_pool capacity in slots */
  int64_t n_tokens;    /* gdn_conv_store: rows of q/k/v (= cu_seqlens[B]); ignored by decode */
  float eps;           /* L2-norm epsilon (decode), e.g. 1e-6 */
  int32_t reserved1;   /* must be 0 */
  const void *q;       /* raw [B or n_tokens, H_qk * d_k] act_dtype */
  const void *k;       /* raw [B or n_tokens, H_qk * d_k] act_dtype */
  const void *v;       /* raw [B or n_tokens, H_v * d_v] act_dtype */
  const float *a_raw;  /* decode: [B, H_v], g = -softplus(a_raw) */
  const float *b_raw;  /* decode: [B, H_v], beta = sigmoid(b_raw) */
  const float *conv_wq;  /* decode: [H_qk * d_k, conv_k] taps (tap j multiplies x[t-conv_k+1+j]) */
  const float *conv_wk;  /* decode: [H_qk * d_k, conv_k] */
  const float *conv_wv;  /* decode: [H_v * d_v, conv_k] */
  void *conv_pool;     /* [n_slots, conv_k - 1, C] act_dtype, read and written in place */
  const int32_t *read_slot;  /* [B] or NULL (-1 = empty window, a fresh request): decode, the
                                window before this token; store, the window each sequence
                                resumed (the older rows of a sequence shorter than
                                conv_k - 1 tokens) */
  const int32_t *write_slot; /* [B] or NULL (-1 = not stored) */
  const int32_t *cu_seqlens; /* store: [B + 1] device offsets into q/k/v; a sequence with
                                cu[s] < 0, cu[s+1] < cu[s] or cu[s+1] > n_tokens is skipped
                                and sets GDN_DEVICE_BAD_SEQ */
  void *q_out;         /* decode: [B, H_qk, d_k] act_dtype, unit L2 norm per head */
  void *k_out;         /* decode: [B, H_qk, d_k] act_dtype */
  void *v_out;         /* decode: [B, H_v, d_v] act_dtype */
  float *g_out;        /* decode: [B, H_v] */
  float *beta_out;     /* decode: [B, H_v] */
  uint32_t *status;    /* optional device word; slot indices outside [-1, n_slots) skip the
                          request and set GDN_DEVICE_BAD_SLOT */
} gdn_conv_args;

/* State tiles copied from one pool to another whose storage format may
 * differ: FP32, BF16, or the 8-bit format (GDN_Q8, the DAMP-like mixed
 * precision of "Seven Architectures ...", ONNX LinearAttention / FlashInfer
 * section).  A prefill stores BF16 or FP32 states, so a prefilled state
 * enters an 8-bit decode pool through this call, and an 8-bit checkpoint is
 * read back through it before a prefill resumes ("Recurrent state" glossary
 * entry, Why it matters: checkpoint slots).  For each pair i and head h:
 * dst_pool[dst_slot[i], h] = the tile src_pool[src_slot[i], h] represents,
 * stored in dst_dtype: BF16 rounds to nearest even; an 8-bit tile keeps its
 * first dst_bf16_rows rows in BF16 and stores every other row as INT8 codes
 * rne(x * (127 / rowmax)) clamped to +-127 with scale rowmax / 127, each step
 * in binary32 (the rule gdn_decode stores with); an 8-bit row is read as
 * code * scale in binary32. */
typedef struct gdn_convert_args {
  int32_t n;                       /* slot pairs, >= 0 */
  int32_t H_v, d_k, d_v;           /* heads per slot and tile shape (16, 32, 64 or 128) */
  int32_t src_dtype, dst_dtype;    /* GDN_F32, GDN_BF16 or GDN_Q8 */
  int32_t src_bf16_rows;           /* src GDN_Q8: BF16 rows per tile (gdn_state_q8_bytes rules), else 0 */
  int32_t dst_bf16_rows;           /* dst GDN_Q8: the same for the destination, else 0 */
  int64_t src_n_slots, dst_n_slots;
  const void *src_pool;            /* [src_n_slots, H_v, tile], 16-byte aligned */
  void *dst_pool;                  /* [dst_n_slots, H_v, tile], 16-byte aligned */
  const int32_t *src_slot;         /* [n] device or NULL (pair i reads slot i); -1 = a zero state */
  const int32_t *dst_slot;         /* [n] device or NULL (pair i writes slot i); -1 = not stored */
  uint32_t *status;                /* optional device word: an index outside [-1, n_slots)
                                      skips the pair and sets GDN_DEVICE_BAD_SLOT */
} gdn_convert_args;

/* Bytes of one slot (all H_v heads of one request, one layer).  The ONNX
 * LinearAttention section of "Seven Architectures ..." sizes 64 heads of
 * 128 x 128 at 16 bits as 2 MB per request. */
size_t gdn_state_bytes(int32_t H_v, int32_t d_k, int32_t d_v, int32_t state_dtype);

/* The step of valid BF16-row counts of the 8-bit format at these head sizes
 * (the rows one wavefront of the decode kernel holds, at least 8, at most
 * d_k: 32 at d_k = d_v = 128), so that each wavefront's rows are of one
 * kind; 0 for unsupported sizes.  Host-only. */
int32_t gdn_state_q8_row_quantum(int32_t d_k, int32_t d_v);

/* Bytes of one slot in the 8-bit format (GDN_Q8): per head
 * bf16_rows * d_v * 2 + (d_k - bf16_rows) * (d_v + 4) rounded up to a
 * multiple of 256; 0 for invalid sizes (bf16_rows must be a multiple of
 * gdn_state_q8_row_quantum in [0, d_k]).  At d_k = d_v = 128 with 32 BF16
 * rows: 20,992 bytes per head (10.25 bits per value, 0.64 of BF16); with
 * none, 16,896 (8.25 bits). */
size_t gdn_state_q8_bytes(int32_t H_v, int32_t d_k, int32_t d_v, int32_t bf16_rows);

/* Workspace that gdn_prefill / gdn_mixed need for these arguments (host-only
 * arithmetic on the sizes; no pointer is read). */
size_t gdn_prefill_workspace_size(const gdn_prefill_args *args);

/* "linear" | "gated" | "delta" | "gated_delta"; NULL or "" gives the default
 * gated_delta (ONNX LinearAttention section).  Host-only. */
gdn_status gdn_parse_rule(const char *name, int32_t *out_rule);

/* One decode token for B requests: gather each request's state from its read
 * slot, decay, apply the rank-one delta update in FP32, read out
 * o = scale * M_t^T q_t, store the state (rounded to nearest-even BF16 when
 * state_dtype is BF16) into its write slot. */
gdn_status gdn_decode(const gdn_decode_args *args, void *stream);

/* The front-end alone, for checking it in isolation (use_frontend must be 1):
 * q_out, k_out [n_tokens, H_qk, d_k] and v_out [n_tokens, H_v, d_v] in
 * act_dtype; g_out, beta_out [n_tokens, H_v] FP32.  No recurrence is run. */
gdn_status gdn_frontend(const gdn_prefill_args *args, void *q_out, void *k_out, void *v_out,
                        float *g_out, float *beta_out, void *stream);

/* The front-end for one decode token per request (the same conv + SiLU,
 * L2 norm and gates as gdn_frontend, bitwise equal for the same window):
 * the window is the read slot's conv_k - 1 raw tokens and this token; the
 * window slid by one token (the last conv_k - 1 raw inputs) is stored into
 * the write slot.  The outputs feed gdn_decode. */
gdn_status gdn_conv_decode(const gdn_conv_args *args, void *stream);

/* One decode token with the layer's short conv fused into the state update,
 * one kernel for both ("Gated DeltaNet" glossary entry, Engineering details:
 * Conv1D and GDN fused for decode).  It computes what gdn_conv_decode
 * followed by gdn_decode computes, bit for bit, without writing q, k, v, g
 * and beta to memory:
 *  - decode: gdn_decode's arguments, except that q, k, v, g and beta must be
 *    NULL (they come from the conv step) and decay_mode must be
 *    GDN_DECAY_HEAD (the front-end makes one decay per head); state_dtype
 *    BF16 or F32 (not the 8-bit format);
 *  - conv: gdn_conv_decode's arguments (raw q, k, v, a_raw, b_raw, taps,
 *    conv_pool with its read and write slots), except that q_out, k_out,
 *    v_out, g_out and beta_out must be NULL; B, H_qk, H_v, d_k, d_v and
 *    act_dtype equal to decode's.
 * A request whose state or conv slot index is outside [-1, n_slots) is
 * skipped entirely (no o, state or window is written) and sets
 * GDN_DEVICE_BAD_SLOT in decode->status.  H_v / H_qk is at most 8, else
 * GDN_ERR_UNSUPPORTED.  The state and conv slot contracts are gdn_decode's
 * and gdn_conv_decode's. */
gdn_status gdn_decode_conv(const gdn_decode_args *decode, const gdn_conv_args *conv,
                           void *stream);

/* gdn_convert_args' copy.  A pair may read and write the same slot of one
 * pool; pairs follow the write-slot contract among themselves (no slot
 * written by two pairs or read by one pair and written by another).  Host
 * validation only: GDN_ERR_DTYPE, _SHAPE (an 8-bit BF16-row count that
 * gdn_state_q8_bytes refuses, NULL slot arrays with fewer slots than pairs),
 * _NULL, _ALIGN. */
gdn_status gdn_state_convert(const gdn_convert_args *args, void *stream);

/* After a prefill of B sequences packed by cu_seqlens: store each sequence's
 * last conv_k - 1 raw inputs into conv_pool[write_slot[s]], so that decode
 * continues its conv window.  Rows before a sequence's first token come from
 * conv_pool[read_slot[s]] (zeros for -1 or a NULL array); a sequence may
 * write the slot it read.  gdn_prefill stores the same windows itself when
 * given conv_write_slot. */
gdn_status gdn_conv_store(const gdn_conv_args *args, void *stream);

/* Bytes of one conv-state slot. */
size_t gdn_conv_slot_bytes(int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t conv_k,
                           int32_t act_dtype);

/* Chunked prefill: initial state from read_slot[s], outputs for every token,
 * final state (FP32 across chunks, rounded once when stored as BF16) into
 * write_slot[s]. */
gdn_status gdn_prefill(const gdn_prefill_args *args, void *stream);

/* gdn_prefill for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same kernels and results as gdn_prefill, but the front-end's workspace
 * is a fixed device array inside the library (gdn_noalloc_workspace_bytes()
 * bytes, 128 MiB: 8,065 tokens with the fused front-end at H_qk = 16,
 * H_v = 32, d = 128 in BF16, any number without it; gdn_prefill_workspace_size()
 * tells what a call needs), so args->workspace
 * and args->workspace_bytes are ignored.  The caller still owns and passes
 * every input and output.  Nothing is allocated or freed: each GPU the
 * library runs on holds its own copy of the array from the first use until
 * the process ends, and the first call on a device looks up its address
 * (hipGetSymbolAddress).  A call that would need more workspace returns
 * GDN_ERR_SCRATCH and launches nothing; other errors as for gdn_prefill.
 * Calls on one GPU share its array, whatever their stream: calls that
 * overlap in time on one GPU race (serialise them, e.g. on one stream).  No
 * part of the array needs clearing: each call writes every byte it reads. */
gdn_status gdn_prefill_noalloc(const gdn_prefill_args *args, void *stream);

/* Bytes of gdn_prefill_noalloc's fixed workspace (host-only). */
size_t gdn_noalloc_workspace_bytes(void);

/* A decode batch and a prefill batch in ONE kernel launch (each half has its
 * own rule and slot arrays; they may share a pool).  The halves' results are
 * those of gdn_decode and gdn_prefill called separately; either half may be
 * empty (B = 0 or n_seq = 0).  The caller contract on slots applies across
 * both halves.  Both halves describe one layer: the same heads, d_k, d_v,
 * state and activation dtypes and decay_mode, else GDN_ERR_UNSUPPORTED; the
 * 8-bit state format (GDN_Q8) is not taken (GDN_ERR_UNSUPPORTED). */
gdn_status gdn_mixed(const gdn_decode_args *decode, const gdn_prefill_args *prefill,
                     void *stream);

/* Host-side check of the slot contract on host copies of the index arrays
 * (NULL = identity): every index in [-1, n_slots), write indices >= 0
 * unique, no write index equal to another request's read index.  Returns
 * GDN_OK or GDN_ERR_SLOTS. */
gdn_status gdn_validate_slots(const int32_t *host_read, const int32_t *host_write, int32_t n,
                              int64_t n_slots);

const char *gdn_status_string(int32_t status);
int32_t gdn_abi_version(void);
/* sizeof of the argument structs as compiled into the library, so that a
 * binding can check its own layout */
size_t gdn_sizeof_decode_args(void);
size_t gdn_sizeof_prefill_args(void);
size_t gdn_sizeof_conv_args(void);
size_t gdn_sizeof_convert_args(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */

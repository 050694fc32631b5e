// api.hip -- the extern "C" entry points declared in include/gdn.h:
// argument validation (host only, before any HIP call) and dispatch.
#include <string.h>

#include <mutex>
#include <new>

#include "decode.cuh"
#include "internal.h"

// The workspace of gdn_prefill_noalloc: a fixed device array of this file, one
// copy on every GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never device memory: host code
// uses only the per-device address that hipGetSymbolAddress returns.
static constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

bool supported_d(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_dtype(int32_t t) { return t == GDN_F32 || t == GDN_BF16; }
bool valid_rule(int32_t r) { return r >= GDN_RULE_LINEAR && r <= GDN_RULE_GATED_DELTA; }
// pointers the kernels access as 16-byte vectors (NULL passes: absence is checked separately)
bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdn_status check_heads(int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v) {
  if (H_qk <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
  if (H_v % H_qk != 0) return GDN_ERR_UNSUPPORTED;  // q/k heads must group evenly
  if (!supported_d(d_k) || !supported_d(d_v)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn_status check_decode(const gdn_decode_args *a) {
  if (!a) return GDN_ERR_NULL;
  if (a->B < 0 || a->n_slots < 0) return GDN_ERR_SHAPE;
  if (!valid_rule(a->rule)) return GDN_ERR_RULE;
  const bool q8 = a->state_dtype == GDN_Q8;
  if ((!valid_dtype(a->state_dtype) && !q8) || !valid_dtype(a->act_dtype)) return GDN_ERR_DTYPE;
  if (a->reserved0 != 0) return GDN_ERR_UNSUPPORTED;
  if (!q8 && a->state_bf16_rows != 0) return GDN_ERR_SHAPE;
  if (a->decay_mode != GDN_DECAY_HEAD && a->decay_mode != GDN_DECAY_CHANNEL)
    return GDN_ERR_UNSUPPORTED;
  gdn_status st = check_heads(a->H_qk, a->H_v, a->d_k, a->d_v);
  if (st != GDN_OK) return st;
  if (q8 && gdn_state_q8_bytes(1, a->d_k, a->d_v, a->state_bf16_rows) == 0) return GDN_ERR_SHAPE;
  if ((int64_t)a->B * a->H_v > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;  // grid size
  if (a->B == 0) return GDN_OK;
  if (!a->q || !a->k || !a->v || !a->state_pool || !a->o) return GDN_ERR_NULL;
  if ((a->rule & gdn::kRuleDecay) && !a->g) return GDN_ERR_NULL;
  if ((a->rule & gdn::kRuleErase) && !a->beta) return GDN_ERR_NULL;
  if ((!a->read_slot || !a->write_slot) && a->n_slots < a->B) return GDN_ERR_SHAPE;
  if (!al16(a->q) || !al16(a->k) || !al16(a->v) || !al16(a->o) || !al16(a->state_pool))
    return GDN_ERR_ALIGN;
  // channel-wise log-decays are read as 16-byte runs
  if (a->decay_mode == GDN_DECAY_CHANNEL && !al16(a->g)) return GDN_ERR_ALIGN;
  return GDN_OK;
}

// need_state: the recurrence runs (pool, outputs, slots, workspace are used);
// false for the stand-alone front-end, which reads only the inputs.
gdn_status check_prefill(const gdn_prefill_args *a, bool need_state) {
  if (!a) return GDN_ERR_NULL;
  if (a->n_seq < 0 || a->n_tokens < 0 || a->n_slots < 0) return GDN_ERR_SHAPE;
  if (!valid_rule(a->rule)) return GDN_ERR_RULE;
  if (a->state_dtype == GDN_Q8) return GDN_ERR_UNSUPPORTED;  // the 8-bit format is decode-only
  if (!valid_dtype(a->state_dtype) || !valid_dtype(a->act_dtype)) return GDN_ERR_DTYPE;
  if (a->decay_mode != GDN_DECAY_HEAD && a->decay_mode != GDN_DECAY_CHANNEL)
    return GDN_ERR_UNSUPPORTED;
  if (a->use_frontend != 0 && a->use_frontend != 1) return GDN_ERR_UNSUPPORTED;
  // the front-end produces one decay per (token, head): the channel-wise
  // decay takes q, k, v, g and beta as given
  if (a->decay_mode == GDN_DECAY_CHANNEL && a->use_frontend) return GDN_ERR_UNSUPPORTED;
  // channel-wise decays are read four channels (16 bytes) at a time
  if (a->decay_mode == GDN_DECAY_CHANNEL && !al16(a->g)) return GDN_ERR_ALIGN;
  gdn_status st = check_heads(a->H_qk, a->H_v, a->d_k, a->d_v);
  if (st != GDN_OK) return st;
  if (a->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (a->use_frontend && a->conv_k != 4) return GDN_ERR_UNSUPPORTED;
  if (a->use_frontend && !(a->eps >= 0.0f)) return GDN_ERR_SHAPE;
  // conv windows across calls belong to the front-end
  const bool conv = a->conv_read_slot || a->conv_write_slot || a->conv_ckpt_slot;
  if (conv && !a->use_frontend) return GDN_ERR_UNSUPPORTED;
  if (conv && !a->conv_pool) return GDN_ERR_NULL;
  if (a->conv_n_slots < 0) return GDN_ERR_SHAPE;
  if (!al16(a->conv_pool)) return GDN_ERR_ALIGN;
  if ((int64_t)a->n_seq * a->H_v > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
  if (a->n_tokens > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;  // token index fits int32
  if (a->n_seq == 0) return a->n_tokens == 0 ? GDN_OK : GDN_ERR_SHAPE;
  if (!a->cu_seqlens) return GDN_ERR_NULL;
  if (need_state && !a->state_pool) return GDN_ERR_NULL;
  if (a->n_tokens > 0 && (!a->q || !a->k || !a->v)) return GDN_ERR_NULL;
  if (need_state && a->n_tokens > 0 && !a->o) return GDN_ERR_NULL;
  if (a->n_tokens > 0) {
    if (a->use_frontend) {
      if (!a->conv_wq || !a->conv_wk || !a->conv_wv) return GDN_ERR_NULL;
      if ((a->rule & gdn::kRuleDecay) && !a->a_raw) return GDN_ERR_NULL;
      if ((a->rule & gdn::kRuleErase) && !a->b_raw) return GDN_ERR_NULL;
    } else {
      if ((a->rule & gdn::kRuleDecay) && !a->g) return GDN_ERR_NULL;
      if ((a->rule & gdn::kRuleErase) && !a->beta) return GDN_ERR_NULL;
    }
  }
  if (!al16(a->q) || !al16(a->k) || !al16(a->v)) return GDN_ERR_ALIGN;
  if (a->use_frontend && (!al16(a->conv_wq) || !al16(a->conv_wk) || !al16(a->conv_wv)))
    return GDN_ERR_ALIGN;
  if (!need_state) return GDN_OK;
  if (!al16(a->o) || !al16(a->state_pool) || !al16(a->workspace)) return GDN_ERR_ALIGN;
  // FP32 activations keep FP32 MFMA operands in LDS, which fits d_k, d_v <= 64
  if (a->act_dtype == GDN_F32 && (a->d_k > 64 || a->d_v > 64)) return GDN_ERR_UNSUPPORTED;
  if ((!a->read_slot || !a->write_slot) && a->n_slots < a->n_seq) return GDN_ERR_SHAPE;
  // intermediate checkpoints: a whole number of chunks apart, and somewhere to put them
  if (a->ckpt_interval < 0 || a->ckpt_interval % a->chunk != 0) return GDN_ERR_SHAPE;
  if (a->ckpt_interval > 0) {
    if (a->ckpt_per_seq <= 0) return GDN_ERR_SHAPE;
    if (!a->ckpt_slot) return GDN_ERR_NULL;
  }
  const size_t need = gdn::prefill_workspace_bytes(*a);
  if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return GDN_ERR_WORKSPACE;
  return GDN_OK;
}

// decode: the conv step for B requests; otherwise the store after a prefill
gdn_status check_conv(const gdn_conv_args *a, bool decode) {
  if (!a) return GDN_ERR_NULL;
  if (a->B < 0 || a->n_slots < 0 || a->n_tokens < 0) return GDN_ERR_SHAPE;
  if (!valid_dtype(a->act_dtype)) return GDN_ERR_DTYPE;
  if (a->reserved0 != 0 || a->reserved1 != 0) return GDN_ERR_UNSUPPORTED;
  if (a->H_qk <= 0 || a->H_v <= 0 || a->d_k <= 0 || a->d_v <= 0) return GDN_ERR_SHAPE;
  if (!supported_d(a->d_k) || !supported_d(a->d_v)) return GDN_ERR_UNSUPPORTED;
  if (a->conv_k != 4) return GDN_ERR_UNSUPPORTED;
  if (decode && !(a->eps >= 0.0f)) return GDN_ERR_SHAPE;
  if (gdn::conv_grid_rows(*a) > 65535) return GDN_ERR_UNSUPPORTED;  // grid size
  if (!decode && a->n_tokens > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
  if (a->B == 0) return !decode && a->n_tokens != 0 ? GDN_ERR_SHAPE : GDN_OK;
  if (!a->write_slot && a->n_slots < a->B) return GDN_ERR_SHAPE;
  if (decode && !a->read_slot && a->n_slots < a->B) return GDN_ERR_SHAPE;
  if (!a->conv_pool) return GDN_ERR_NULL;
  if (!al16(a->conv_pool)) return GDN_ERR_ALIGN;
  if (decode) {
    if (!a->q || !a->k || !a->v || !a->a_raw || !a->b_raw) return GDN_ERR_NULL;
    if (!a->conv_wq || !a->conv_wk || !a->conv_wv) return GDN_ERR_NULL;
    if (!a->q_out || !a->k_out || !a->v_out || !a->g_out || !a->beta_out) return GDN_ERR_NULL;
    if (!al16(a->conv_wq) || !al16(a->conv_wk) || !al16(a->conv_wv) || !al16(a->q_out) ||
        !al16(a->k_out) || !al16(a->v_out))
      return GDN_ERR_ALIGN;
  } else {
    if (!a->cu_seqlens) return GDN_ERR_NULL;
    if (a->n_tokens > 0 && (!a->q || !a->k || !a->v)) return GDN_ERR_NULL;
  }
  if (!al16(a->q) || !al16(a->k) || !al16(a->v)) return GDN_ERR_ALIGN;
  return GDN_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

gdn_status scratch_address(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_state_bytes(int32_t H_v, int32_t d_k, int32_t d_v, int32_t state_dtype) {
  if (H_v <= 0 || d_k <= 0 || d_v <= 0 || !valid_dtype(state_dtype)) return 0;
  return (size_t)H_v * (size_t)d_k * (size_t)d_v * (state_dtype == GDN_BF16 ? 2u : 4u);
}

int32_t gdn_state_q8_row_quantum(int32_t d_k, int32_t d_v) {
  if (!supported_d(d_k) || !supported_d(d_v)) return 0;
  return gdn::q8_row_quantum(d_k, d_v);
}

size_t gdn_state_q8_bytes(int32_t H_v, int32_t d_k, int32_t d_v, int32_t bf16_rows) {
  const int32_t quantum = gdn_state_q8_row_quantum(d_k, d_v);
  if (H_v <= 0 || quantum == 0 || bf16_rows < 0 || bf16_rows > d_k || bf16_rows % quantum)
    return 0;
  const size_t lo = (size_t)(d_k - bf16_rows);
  const size_t tile = (size_t)bf16_rows * d_v * 2 + lo * d_v + lo * 4;
  return (size_t)H_v * ((tile + 255) / 256 * 256);  // tiles start on 256-byte boundaries
}

size_t gdn_prefill_workspace_size(const gdn_prefill_args *args) {
  return args ? gdn::prefill_workspace_bytes(*args) : 0;
}

gdn_status gdn_parse_rule(const char *name, int32_t *out_rule) {
  if (!out_rule) return GDN_ERR_NULL;
  if (!name || !*name || !strcmp(name, "gated_delta")) { *out_rule = GDN_RULE_GATED_DELTA; return GDN_OK; }
  if (!strcmp(name, "linear")) { *out_rule = GDN_RULE_LINEAR; return GDN_OK; }
  if (!strcmp(name, "gated")) { *out_rule = GDN_RULE_GATED; return GDN_OK; }
  if (!strcmp(name, "delta")) { *out_rule = GDN_RULE_DELTA; return GDN_OK; }
  return GDN_ERR_RULE;
}

gdn_status gdn_decode(const gdn_decode_args *args, void *stream) {
  gdn_status st = check_decode(args);
  if (st != GDN_OK || args->B == 0) return st;
  return gdn::launch_decode(*args, static_cast<hipStream_t>(stream));
}

gdn_status gdn_frontend(const gdn_prefill_args *args, void *q_out, void *k_out, void *v_out,
                        float *g_out, float *beta_out, void *stream) {
  gdn_status st = check_prefill(args, false);
  if (st != GDN_OK) return st;
  if (!args->use_frontend) return GDN_ERR_UNSUPPORTED;
  if (args->n_seq == 0 || args->n_tokens == 0) return GDN_OK;
  if (!q_out || !k_out || !v_out || !g_out || !beta_out) return GDN_ERR_NULL;
  if (!al16(q_out) || !al16(k_out) || !al16(v_out)) return GDN_ERR_ALIGN;
  if (!args->a_raw || !args->b_raw) return GDN_ERR_NULL;
  return gdn::launch_frontend(*args, q_out, k_out, v_out, g_out, beta_out,
                              static_cast<hipStream_t>(stream));
}

gdn_status gdn_conv_decode(const gdn_conv_args *args, void *stream) {
  gdn_status st = check_conv(args, true);
  if (st != GDN_OK || args->B == 0) return st;
  return gdn::launch_conv_decode(*args, static_cast<hipStream_t>(stream));
}

gdn_status gdn_decode_conv(const gdn_decode_args *decode, const gdn_conv_args *conv,
                           void *stream) {
  if (!decode || !conv) return GDN_ERR_NULL;
  // the token's inputs come from the conv step: none may be passed
  if (decode->q || decode->k || decode->v || decode->g || decode->beta) return GDN_ERR_UNSUPPORTED;
  if (conv->q_out || conv->k_out || conv->v_out || conv->g_out || conv->beta_out)
    return GDN_ERR_UNSUPPORTED;
  // every other check of the two calls, with the raw inputs standing in for
  // the pointers the fused kernel does not take
  gdn_decode_args d = *decode;
  d.q = d.k = d.v = conv->q;
  d.g = d.beta = conv->a_raw;
  gdn_conv_args c = *conv;
  c.q_out = c.k_out = c.v_out = const_cast<void *>(conv->q);
  c.g_out = c.beta_out = const_cast<float *>(conv->a_raw);
  gdn_status st = check_decode(&d);
  if (st != GDN_OK) return st;
  st = check_conv(&c, true);
  if (st != GDN_OK) return st;
  if (conv->B != decode->B || conv->H_qk != decode->H_qk || conv->H_v != decode->H_v ||
      conv->d_k != decode->d_k || conv->d_v != decode->d_v)
    return GDN_ERR_SHAPE;
  if (conv->act_dtype != decode->act_dtype) return GDN_ERR_DTYPE;
  if (decode->state_dtype == GDN_Q8 || decode->decay_mode != GDN_DECAY_HEAD)
    return GDN_ERR_UNSUPPORTED;
  const int group = decode->H_v / decode->H_qk;
  if (group > gdn::decode_conv_max_group() ||
      gdn::decode_conv_stage_threads(decode->d_k, decode->d_v, group,
                                     decode->act_dtype == GDN_BF16) >
          gdn::decode_conv_block_threads(decode->d_k, decode->d_v,
                                         decode->state_dtype == GDN_BF16))
    return GDN_ERR_UNSUPPORTED;
  if ((int64_t)decode->B * decode->H_qk > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
  if (decode->B == 0) return GDN_OK;
  return gdn::launch_decode_conv(*decode, *conv, static_cast<hipStream_t>(stream));
}

gdn_status gdn_state_convert(const gdn_convert_args *a, void *stream) {
  if (!a) return GDN_ERR_NULL;
  if (a->n < 0 || a->src_n_slots < 0 || a->dst_n_slots < 0) return GDN_ERR_SHAPE;
  auto kind_ok = [](int32_t k) { return k == GDN_F32 || k == GDN_BF16 || k == GDN_Q8; };
  if (!kind_ok(a->src_dtype) || !kind_ok(a->dst_dtype)) return GDN_ERR_DTYPE;
  if (a->H_v <= 0 || a->d_k <= 0 || a->d_v <= 0) return GDN_ERR_SHAPE;
  if (!supported_d(a->d_k) || !supported_d(a->d_v)) return GDN_ERR_UNSUPPORTED;
  // BF16 rows: a valid count for an 8-bit side, none otherwise
  auto rows_ok = [&](int32_t kind, int32_t rows) {
    return kind == GDN_Q8 ? gdn_state_q8_bytes(1, a->d_k, a->d_v, rows) != 0 : rows == 0;
  };
  if (!rows_ok(a->src_dtype, a->src_bf16_rows) || !rows_ok(a->dst_dtype, a->dst_bf16_rows))
    return GDN_ERR_SHAPE;
  if ((int64_t)a->n * a->H_v > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;  // grid size
  if (a->n == 0) return GDN_OK;
  if ((!a->src_slot && a->src_n_slots < a->n) || (!a->dst_slot && a->dst_n_slots < a->n))
    return GDN_ERR_SHAPE;
  if (!a->src_pool || !a->dst_pool) return GDN_ERR_NULL;
  if (!al16(a->src_pool) || !al16(a->dst_pool)) return GDN_ERR_ALIGN;
  return gdn::launch_state_convert(*a, static_cast<hipStream_t>(stream));
}

gdn_status gdn_conv_store(const gdn_conv_args *args, void *stream) {
  gdn_status st = check_conv(args, false);
  if (st != GDN_OK || args->B == 0) return st;
  return gdn::launch_conv_store(*args, static_cast<hipStream_t>(stream));
}

size_t gdn_conv_slot_bytes(int32_t H_qk, int32_t H_v, int32_t d_k, int32_t d_v, int32_t conv_k,
                           int32_t act_dtype) {
  if (H_qk <= 0 || H_v <= 0 || d_k <= 0 || d_v <= 0 || conv_k < 1 || !valid_dtype(act_dtype))
    return 0;
  const size_t C = 2 * (size_t)H_qk * (size_t)d_k + (size_t)H_v * (size_t)d_v;
  return (size_t)(conv_k - 1) * C * (act_dtype == GDN_BF16 ? 2u : 4u);
}

gdn_status gdn_prefill(const gdn_prefill_args *args, void *stream) {
  gdn_status st = check_prefill(args, true);
  if (st != GDN_OK || args->n_seq == 0) return st;
  return gdn::launch_prefill(*args, static_cast<hipStream_t>(stream));
}

gdn_status gdn_prefill_noalloc(const gdn_prefill_args *args, void *stream) {
  if (!args) return GDN_ERR_NULL;
  gdn_prefill_args a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  // every other check first; the only one left to fail is the workspace's
  gdn_status st = check_prefill(&a, true);
  if (st != GDN_OK && st != GDN_ERR_WORKSPACE) return st;
  if (a.n_seq == 0) return GDN_OK;
  const size_t need = gdn::prefill_workspace_bytes(a);
  if (need > kScratchBytes) return GDN_ERR_SCRATCH;
  if (need > 0) {
    st = scratch_address(&a.workspace);
    if (st != GDN_OK) return st;
    a.workspace_bytes = kScratchBytes;
  }
  return gdn::launch_prefill(a, static_cast<hipStream_t>(stream));
}

size_t gdn_noalloc_workspace_bytes(void) { return kScratchBytes; }

gdn_status gdn_mixed(const gdn_decode_args *decode, const gdn_prefill_args *prefill,
                     void *stream) {
  gdn_status st = check_decode(decode);
  if (st != GDN_OK) return st;
  // decode tiles on a BF16 or FP32 state (not the 8-bit format)
  if (decode->state_dtype == GDN_Q8) return GDN_ERR_UNSUPPORTED;
  st = check_prefill(prefill, true);
  if (st != GDN_OK) return st;
  if (decode->B == 0 && prefill->n_seq == 0) return GDN_OK;
  return gdn::launch_mixed(*decode, *prefill, static_cast<hipStream_t>(stream));
}

gdn_status gdn_validate_slots(const int32_t *host_read, const int32_t *host_write, int32_t n,
                              int64_t n_slots) {
  if (n < 0 || n_slots < 0) return GDN_ERR_SHAPE;
  if ((!host_read || !host_write) && n_slots < n) return GDN_ERR_SLOTS;
  // per slot: which request writes it (-1 none), and a count of its readers
  int32_t *writer = new (std::nothrow) int32_t[n_slots > 0 ? n_slots : 1];
  if (!writer) return GDN_ERR_SHAPE;
  for (int64_t s = 0; s < n_slots; ++s) writer[s] = -1;
  gdn_status st = GDN_OK;
  for (int32_t r = 0; r < n && st == GDN_OK; ++r) {
    const int64_t rs = host_read ? host_read[r] : r, ws = host_write ? host_write[r] : r;
    if (rs < -1 || rs >= n_slots || ws < -1 || ws >= n_slots) st = GDN_ERR_SLOTS;
    else if (ws >= 0) {
      if (writer[ws] != -1) st = GDN_ERR_SLOTS;  // two requests write one slot
      else writer[ws] = r;
    }
  }
  for (int32_t r = 0; r < n && st == GDN_OK; ++r) {
    const int64_t rs = host_read ? host_read[r] : r;
    if (rs >= 0 && writer[rs] != -1 && writer[rs] != r) st = GDN_ERR_SLOTS;  // read-after-write hazard
  }
  delete[] writer;
  return st;
}

const char *gdn_status_string(int32_t status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid or inconsistent sizes";
    case GDN_ERR_DTYPE: return "unknown dtype";
    case GDN_ERR_RULE: return "unknown update rule";
    case GDN_ERR_UNSUPPORTED: return "unsupported size or option";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_SLOTS: return "slot index out of range or slot hazard";
    case GDN_ERR_ALIGN: return "a vector-accessed tensor is not 16-byte aligned";
    case GDN_ERR_SCRATCH: return "the call needs more than the fixed no-allocation workspace";
  }
  return "unknown status";
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }
size_t gdn_sizeof_decode_args(void) { return sizeof(gdn_decode_args); }
size_t gdn_sizeof_prefill_args(void) { return sizeof(gdn_prefill_args); }
size_t gdn_sizeof_conv_args(void) { return sizeof(gdn_conv_args); }
size_t gdn_sizeof_convert_args(void) { return sizeof(gdn_convert_args); }

}  // extern "C"

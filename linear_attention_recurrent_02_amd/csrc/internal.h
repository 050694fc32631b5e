// internal.h -- launchers behind the C ABI.  Arguments have been validated by
// the API layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn.h"

namespace gdn {

// rule bits: bit 0 = the state decays by a = exp(g), bit 1 = delta-rule erase
// with write strength beta (linear = 0, gated = 1, delta = 2, gated_delta = 3)
constexpr int kRuleDecay = 1;
constexpr int kRuleErase = 2;

gdn_status launch_decode(const gdn_decode_args &a, hipStream_t stream);
gdn_status launch_frontend(const gdn_prefill_args &a, void *q_out, void *k_out, void *v_out,
                           float *g_out, float *beta_out, hipStream_t stream);
gdn_status launch_prefill(const gdn_prefill_args &a, hipStream_t stream);
gdn_status launch_mixed(const gdn_decode_args &d, const gdn_prefill_args &p, hipStream_t stream);
size_t prefill_workspace_bytes(const gdn_prefill_args &a);
gdn_status launch_conv_decode(const gdn_conv_args &a, hipStream_t stream);
gdn_status launch_conv_store(const gdn_conv_args &a, hipStream_t stream);
gdn_status launch_decode_conv(const gdn_decode_args &d, const gdn_conv_args &c, hipStream_t stream);
int decode_conv_stage_threads(int d_k, int d_v, int group, bool act_bf16);
int decode_conv_max_group();
int decode_conv_block_threads(int d_k, int d_v, bool state_bf16);
gdn_status launch_state_convert(const gdn_convert_args &a, hipStream_t stream);
gdn_status launch_prefill_conv_store(const gdn_prefill_args &a, hipStream_t stream);
int64_t conv_grid_rows(const gdn_conv_args &a);  // blockIdx.y extent of the conv kernels

struct PrefillParams;
// Kernel parameters of a prefill call; runs the front-end kernel into the
// workspace first when the inputs are raw.
gdn_status prepare_prefill(const gdn_prefill_args &a, hipStream_t stream, PrefillParams *out);

}  // namespace gdn

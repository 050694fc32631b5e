// stubs.hip -- placeholders for the entry points whose kernels are not built yet.
#include "internal.h"

namespace gdn {
gdn_status launch_frontend(const gdn_prefill_args &, void *, void *, void *, float *, float *,
                           hipStream_t) { return GDN_ERR_UNSUPPORTED; }
gdn_status launch_prefill(const gdn_prefill_args &, hipStream_t) { return GDN_ERR_UNSUPPORTED; }
gdn_status launch_mixed(const gdn_decode_args &, const gdn_prefill_args &, hipStream_t) {
  return GDN_ERR_UNSUPPORTED;
}
size_t prefill_workspace_bytes(const gdn_prefill_args &) { return 0; }
}  // namespace gdn

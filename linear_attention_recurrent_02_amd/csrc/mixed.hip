// mixed.hip -- placeholder until the single-launch mixed batch is built.
#include "internal.h"

namespace gdn {
gdn_status launch_mixed(const gdn_decode_args &, const gdn_prefill_args &, hipStream_t) {
  return GDN_ERR_UNSUPPORTED;
}
}  // namespace gdn

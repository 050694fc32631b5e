"""MI355X (gfx950) Gated DeltaNet recurrent-state hot path.

The compute lives in the HIP library ``libgdn.so`` (C ABI: include/gdn.h);
``gdn`` is its thin ctypes binding and ``synthetic`` makes seeded inputs.
Importing the package loads nothing; the first binding call loads the
library and raises if it has not been built.
"""
from .gdn import (DECAY_CHANNEL, DECAY_HEAD, ConvArgs, DecodeArgs, GdnError,  # noqa: F401
                  PrefillArgs, gdn_abi_version, gdn_conv_decode, gdn_conv_slot_bytes, gdn_conv_store, gdn_decode,
                  gdn_decode_conv, make_decode_conv_args, ConvertArgs, gdn_state_convert,
                  gdn_frontend, gdn_mixed, gdn_noalloc_workspace_bytes, gdn_parse_rule,
                  gdn_prefill, gdn_prefill_noalloc, gdn_state_bytes, gdn_state_q8_bytes,
                  gdn_status_string, gdn_validate_slots, load_library, make_conv_args,
                  make_decode_args, make_prefill_args)

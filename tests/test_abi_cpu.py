"""The C ABI without a GPU: the library loads, exports every function the
header declares, struct layouts agree, host-only calls work, and invalid
arguments are refused synchronously (nothing is launched)."""
import ctypes
import json
import os

import pytest

import linear_attention_recurrent_02_amd as gdn
from linear_attention_recurrent_02_amd import gdn as B

HERE = os.path.dirname(os.path.abspath(__file__))
OK, NULL, SHAPE, DTYPE, RULE, UNSUP, WORKSPACE, LAUNCH, SLOTS, ALIGN, SCRATCH = range(11)
FAKE = 0x10000  # never dereferenced: these calls fail validation before any device work


def test_exports_every_declared_symbol():
    lib = gdn.load_library()
    names = B.header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches():
    lib = gdn.load_library()
    assert lib.gdn_sizeof_decode_args() == ctypes.sizeof(B.DecodeArgs)
    assert lib.gdn_sizeof_prefill_args() == ctypes.sizeof(B.PrefillArgs)
    assert lib.gdn_sizeof_conv_args() == ctypes.sizeof(B.ConvArgs)
    assert gdn.gdn_abi_version() == 10
    assert lib.gdn_sizeof_convert_args() == ctypes.sizeof(B.ConvertArgs)


def test_state_bytes_against_the_pages():
    gold = json.load(open(os.path.join(HERE, "golden", "state_sizes.json")))
    for c in gold["cases"]:
        code = B.BF16 if c["dtype"] == "bf16" else B.F32
        got = gdn.gdn_state_bytes(c["H_v"], c["d_k"], c["d_v"], code)
        assert got == c["bytes"], c["what"]
        if "layers" in c:
            assert got * c["layers"] == c["bytes_all_layers"]
    assert gdn.gdn_state_bytes(32, 128, 128, B.F32) == 2 * gdn.gdn_state_bytes(32, 128, 128, B.BF16)
    assert gdn.gdn_state_bytes(0, 128, 128, B.BF16) == 0
    assert gdn.gdn_state_bytes(1, 16, 16, 9) == 0


def test_parse_rule():
    assert gdn.gdn_parse_rule(None) == 3 and gdn.gdn_parse_rule("") == 3
    for i, n in enumerate(["linear", "gated", "delta", "gated_delta"]):
        assert gdn.gdn_parse_rule(n) == i
    with pytest.raises(gdn.GdnError):
        gdn.gdn_parse_rule("mamba")


def test_status_strings():
    for c in range(11):
        assert gdn.gdn_status_string(c) != "unknown status"
    assert gdn.gdn_status_string(99) == "unknown status"


def _decode_args(**over):
    a = B.DecodeArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = 4, 2, 4, 128, 128
    a.rule, a.state_dtype, a.act_dtype = 3, 1, 1
    a.n_slots, a.scale, a.decay_mode = 8, 1.0, 0
    for f in ("q", "k", "v", "g", "beta", "state_pool", "o"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _call_decode(a):
    return gdn.load_library().gdn_decode(ctypes.byref(a), None)


@pytest.mark.parametrize("over,code", [
    (dict(rule=4), RULE), (dict(rule=-1), RULE),
    (dict(state_dtype=3), DTYPE), (dict(act_dtype=-1), DTYPE), (dict(act_dtype=2), DTYPE),
    # the 8-bit state format: a multiple of 8 BF16 rows within d_k, none for other formats
    (dict(decay_mode=1, g=FAKE + 4), ALIGN),  # channel-wise decays are read 16 bytes at a time
    (dict(state_dtype=2, state_bf16_rows=12), SHAPE), (dict(state_dtype=2, state_bf16_rows=136), SHAPE),
    (dict(state_dtype=2, state_bf16_rows=24), SHAPE),
    (dict(state_dtype=2, state_bf16_rows=-8), SHAPE), (dict(state_bf16_rows=8), SHAPE),
    (dict(reserved0=1), UNSUP),
    (dict(B=-1), SHAPE), (dict(n_slots=-1), SHAPE), (dict(H_qk=0), SHAPE), (dict(d_k=0), SHAPE),
    (dict(H_qk=3), UNSUP), (dict(d_k=48), UNSUP), (dict(d_v=256), UNSUP), (dict(decay_mode=2), UNSUP), (dict(decay_mode=-1), UNSUP),
    (dict(q=None), NULL), (dict(state_pool=None), NULL), (dict(o=None), NULL),
    (dict(g=None), NULL), (dict(beta=None), NULL),
    (dict(n_slots=3), SHAPE),  # identity slots need n_slots >= B
    (dict(q=FAKE + 2), ALIGN), (dict(v=FAKE + 8), ALIGN), (dict(o=FAKE + 4), ALIGN),
    (dict(state_pool=FAKE + 2), ALIGN),
])
def test_decode_validation(over, code):
    assert _call_decode(_decode_args(**over)) == code


def test_state_q8_bytes_and_q8_elsewhere():
    """Slot bytes of the 8-bit format (the oracle's layout: BF16 head rows,
    int8 codes, binary32 scales), and the calls that refuse it."""
    import oracle
    lib = gdn.load_library()
    for dk, dv, n_hi in ((128, 128, 32), (128, 128, 0), (128, 128, 128), (64, 32, 16),
                         (16, 16, 16), (16, 128, 8)):
        assert gdn.gdn_state_q8_bytes(32, dk, dv, n_hi) == 32 * oracle.q8_tile_bytes(dk, dv, n_hi)
    # the BF16 head comes in steps of the rows one decode wavefront holds
    lib = gdn.load_library()
    quanta = {(128, 128): 32, (128, 64): 32, (128, 16): 32, (64, 128): 16, (64, 64): 16,
              (64, 32): 16, (32, 64): 8, (32, 32): 16, (16, 128): 8, (16, 16): 16}
    for (dk, dv), q in quanta.items():
        assert lib.gdn_state_q8_row_quantum(dk, dv) == q, (dk, dv)
    assert lib.gdn_state_q8_row_quantum(48, 128) == 0
    for bad in (8, 12, 24, 136):
        assert gdn.gdn_state_q8_bytes(32, 128, 128, bad) == 0, bad
    # 32 BF16 rows at d = 128: 10.25 bits per value, 0.64 of the BF16 slot
    assert gdn.gdn_state_q8_bytes(32, 128, 128, 32) == 32 * 20992
    # an 8-bit pool passes the decode's checks (stops at B = 0); mixed and prefill refuse it
    assert _call_decode(_decode_args(B=0, state_dtype=2, state_bf16_rows=32)) == OK
    assert _call_decode(_decode_args(B=0, state_dtype=2, state_bf16_rows=24)) == SHAPE
    a = _decode_args(state_dtype=2, state_bf16_rows=32)
    p = _prefill_args(state_dtype=2)
    assert lib.gdn_mixed(ctypes.byref(a), ctypes.byref(_prefill_args()), None) == UNSUP
    assert lib.gdn_prefill(ctypes.byref(p), None) == UNSUP


def test_decode_rule_specific_pointers_and_empty_batch():
    # linear ignores g and beta, so they may be NULL (then validation passes; we stop at B=0)
    assert _call_decode(_decode_args(B=0, rule=0, g=None, beta=None)) == OK
    assert _call_decode(_decode_args(B=0)) == OK
    assert _call_decode(_decode_args(B=0, q=None)) == OK  # nothing to read
    assert _call_decode(_decode_args(rule=1, beta=None, g=None)) == NULL  # gated needs g
    assert _call_decode(_decode_args(rule=2, g=None, beta=None)) == NULL  # delta needs beta
    assert gdn.load_library().gdn_decode(None, None) == NULL


def _prefill_args(**over):
    a = B.PrefillArgs()
    a.n_seq, a.H_qk, a.H_v, a.d_k, a.d_v = 2, 2, 4, 128, 128
    a.rule, a.state_dtype, a.act_dtype = 3, 1, 1
    a.use_frontend, a.conv_k, a.chunk, a.ckpt_interval = 1, 4, 64, 0
    a.n_tokens, a.n_slots, a.scale, a.eps = 100, 8, 1.0, 1e-6
    for f in ("cu_seqlens", "q", "k", "v", "a_raw", "b_raw", "conv_wq", "conv_wk", "conv_wv",
              "state_pool", "o", "g", "beta"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(chunk=32), UNSUP), (dict(conv_k=3), UNSUP), (dict(use_frontend=2), UNSUP),
    (dict(rule=9), RULE), (dict(act_dtype=3), DTYPE), (dict(n_seq=-1), SHAPE),
    (dict(n_seq=0), SHAPE), (dict(eps=-1.0), SHAPE), (dict(cu_seqlens=None), NULL),
    (dict(conv_wk=None), NULL), (dict(a_raw=None), NULL), (dict(state_pool=None), NULL),
    (dict(H_v=5), UNSUP), (dict(d_v=96), UNSUP), (dict(n_slots=1), SHAPE),
    (dict(), WORKSPACE),  # the fused front-end needs gdn_prefill_workspace_size() bytes
    (dict(q=FAKE + 2), ALIGN), (dict(v=FAKE + 8), ALIGN), (dict(conv_wv=FAKE + 4), ALIGN),
    (dict(o=FAKE + 2), ALIGN), (dict(state_pool=FAKE + 8), ALIGN),
    (dict(workspace=FAKE + 8, workspace_bytes=1 << 40), ALIGN),
    # intermediate checkpoints: a positive multiple of the chunk, a slot matrix; decay modes
    (dict(ckpt_interval=32), SHAPE), (dict(ckpt_interval=-64), SHAPE),
    (dict(ckpt_interval=64), SHAPE), (dict(ckpt_interval=64, ckpt_per_seq=2), NULL),
    (dict(decay_mode=2), UNSUP), (dict(decay_mode=-1), UNSUP),
    (dict(decay_mode=1), UNSUP),  # the channel-wise decay takes final q/k/v/g (no front-end)
    # the channel-wise checks pass (an empty batch launches nothing)
    (dict(decay_mode=1, use_frontend=0, n_seq=0, n_tokens=0), OK),
    (dict(ckpt_interval=128, ckpt_per_seq=2, ckpt_slot=FAKE), WORKSPACE),  # the checks pass
])
def test_prefill_validation(over, code):
    lib = gdn.load_library()
    a = _prefill_args(**over)
    assert lib.gdn_prefill(ctypes.byref(a), None) == code


NOALLOC_SAME = [
    (dict(chunk=32), UNSUP), (dict(rule=9), RULE), (dict(act_dtype=3), DTYPE),
    (dict(n_seq=-1), SHAPE), (dict(cu_seqlens=None), NULL), (dict(conv_wk=None), NULL),
    (dict(H_v=5), UNSUP), (dict(n_slots=1), SHAPE), (dict(q=FAKE + 2), ALIGN),
    (dict(ckpt_interval=32), SHAPE), (dict(decay_mode=3), UNSUP),
]


@pytest.mark.parametrize("over,code", NOALLOC_SAME)
def test_prefill_noalloc_validation(over, code):
    """The no-allocation prefill refuses what gdn_prefill refuses, before any
    device work (its workspace fields are ignored, so they cannot fail)."""
    lib = gdn.load_library()
    a = _prefill_args(**over)
    assert lib.gdn_prefill_noalloc(ctypes.byref(a), None) == code
    assert lib.gdn_prefill(ctypes.byref(a), None) == code


def test_prefill_noalloc_too_large_and_empty():
    lib = gdn.load_library()
    cap = lib.gdn_noalloc_workspace_bytes()
    assert cap == 128 << 20
    # the workload's heads: 16,640 workspace bytes per token (q, k, v in BF16,
    # g and beta in FP32), so 8,065 tokens fit and 8,066 do not
    a = _prefill_args(H_qk=16, H_v=32, n_tokens=8065)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(a)) <= cap
    a = _prefill_args(H_qk=16, H_v=32, n_tokens=8066)
    assert lib.gdn_prefill_workspace_size(ctypes.byref(a)) > cap
    assert lib.gdn_prefill_noalloc(ctypes.byref(a), None) == SCRATCH
    # an empty batch is a no-op, as for gdn_prefill
    assert lib.gdn_prefill_noalloc(ctypes.byref(_prefill_args(n_seq=0, n_tokens=0)), None) == OK
    assert lib.gdn_prefill_noalloc(None, None) == NULL


def test_prefill_workspace_size():
    lib = gdn.load_library()
    a = _prefill_args()
    need = lib.gdn_prefill_workspace_size(ctypes.byref(a))
    # q, k, v of 100 tokens in BF16 plus g, beta in FP32, 256-byte aligned segments
    assert need >= 100 * (2 * 2 * 128 + 4 * 128) * 2 + 2 * 100 * 4 * 4
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert lib.gdn_prefill(ctypes.byref(a), None) == WORKSPACE
    a.use_frontend = 0
    assert lib.gdn_prefill_workspace_size(ctypes.byref(a)) == 0


def test_prefill_fp32_needs_small_heads():
    lib = gdn.load_library()
    # FP32 activations keep FP32 MFMA operands in LDS: d_k, d_v <= 64 only
    a = _prefill_args(act_dtype=0, use_frontend=0)
    assert lib.gdn_prefill(ctypes.byref(a), None) == UNSUP
    a = _prefill_args(act_dtype=0, use_frontend=0, d_k=64, d_v=128)
    assert lib.gdn_prefill(ctypes.byref(a), None) == UNSUP


def test_prefill_conv_width_ignored_without_frontend_and_empty_batch():
    lib = gdn.load_library()
    a = _prefill_args(n_seq=0, n_tokens=0, use_frontend=0, conv_k=0)
    assert lib.gdn_prefill(ctypes.byref(a), None) == OK
    d = _decode_args(B=0)
    assert lib.gdn_mixed(ctypes.byref(d), ctypes.byref(a), None) == OK
    bad = _decode_args(rule=11)
    assert lib.gdn_mixed(ctypes.byref(bad), ctypes.byref(a), None) == RULE


@pytest.mark.parametrize("over,code", [
    # conv windows belong to the front-end
    (dict(use_frontend=0, conv_pool=FAKE, conv_n_slots=4, conv_read_slot=FAKE), UNSUP),
    (dict(use_frontend=0, conv_pool=FAKE, conv_n_slots=4, conv_write_slot=FAKE), UNSUP),
    (dict(conv_write_slot=FAKE, conv_n_slots=4), NULL),      # slots without a pool
    (dict(conv_ckpt_slot=FAKE, conv_n_slots=4), NULL),
    (dict(conv_pool=FAKE, conv_n_slots=-1, conv_read_slot=FAKE), SHAPE),
    (dict(conv_pool=FAKE + 8, conv_n_slots=4, conv_read_slot=FAKE), ALIGN),
    (dict(conv_pool=FAKE, conv_n_slots=4, conv_read_slot=FAKE, conv_write_slot=FAKE),
     WORKSPACE),  # valid conv fields: the call reaches the workspace check
])
def test_prefill_conv_window_fields(over, code):
    lib = gdn.load_library()
    a = _prefill_args(**over)
    assert lib.gdn_prefill(ctypes.byref(a), None) == code


def test_mixed_halves_must_share_the_decay_mode():
    """One layer per launch: a per-head decode half with a channel-wise
    prefill half (or the reverse) is refused before any launch."""
    lib = gdn.load_library()
    p = _prefill_args(use_frontend=0, decay_mode=1)
    d = _decode_args(decay_mode=0)
    assert lib.gdn_mixed(ctypes.byref(d), ctypes.byref(p), None) == UNSUP
    p = _prefill_args(use_frontend=0, decay_mode=0)
    d = _decode_args(decay_mode=1)
    assert lib.gdn_mixed(ctypes.byref(d), ctypes.byref(p), None) == UNSUP
    # the channel-wise prefill takes no fused front-end, in gdn_mixed as in gdn_prefill
    p = _prefill_args(decay_mode=1)
    assert lib.gdn_mixed(ctypes.byref(d), ctypes.byref(p), None) == UNSUP


def test_validate_slots():
    v = gdn.gdn_validate_slots
    assert v([0, 1, 2], [3, 4, 5], 3, 8) == OK
    assert v([0, 1, 2], [0, 1, 2], 3, 8) == OK            # in place
    assert v([-1, -1], [-1, -1], 2, 8) == OK              # fresh requests, nothing stored
    assert v([0, 1], [2, 2], 2, 8) == SLOTS               # duplicate write slot
    assert v([0, 2], [2, 3], 2, 8) == SLOTS               # request 1 reads what request 0 writes
    assert v([0, 8], [1, 2], 2, 8) == SLOTS               # out of range
    assert v([0, -2], [1, 2], 2, 8) == SLOTS
    assert v(None, None, 4, 4) == OK
    assert v(None, None, 5, 4) == SLOTS


def test_conv_slot_bytes():
    # three raw tokens of 2*16*128 + 32*128 = 8192 BF16 channels: 48 KiB per request
    assert gdn.gdn_conv_slot_bytes(16, 32, 128, 128, 4, B.BF16) == 3 * 8192 * 2 == 48 * 1024
    assert gdn.gdn_conv_slot_bytes(16, 32, 128, 128, 4, B.F32) == 96 * 1024
    assert gdn.gdn_conv_slot_bytes(0, 32, 128, 128, 4, B.BF16) == 0
    assert gdn.gdn_conv_slot_bytes(1, 1, 16, 16, 4, 7) == 0


def _conv_args(**over):
    a = B.ConvArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = 4, 2, 4, 64, 64
    a.act_dtype, a.conv_k, a.n_slots, a.n_tokens, a.eps = B.BF16, 4, 8, 0, 1e-6
    for f in ("q", "k", "v", "a_raw", "b_raw", "conv_wq", "conv_wk", "conv_wv", "conv_pool",
              "q_out", "k_out", "v_out", "g_out", "beta_out"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


CONV_BAD = [
    (dict(B=-1), SHAPE), (dict(n_slots=-1), SHAPE), (dict(act_dtype=5), DTYPE),
    (dict(reserved0=1), UNSUP), (dict(reserved1=1), UNSUP), (dict(H_qk=0), SHAPE),
    (dict(d_k=48), UNSUP), (dict(d_v=256), UNSUP), (dict(conv_k=3), UNSUP),
    (dict(eps=-1.0), SHAPE), (dict(n_slots=3), SHAPE), (dict(conv_pool=None), NULL),
    (dict(q=None), NULL), (dict(a_raw=None), NULL), (dict(conv_wv=None), NULL),
    (dict(beta_out=None), NULL), (dict(conv_pool=FAKE + 8), ALIGN), (dict(q_out=FAKE + 4), ALIGN),
    (dict(conv_wk=FAKE + 4), ALIGN), (dict(H_v=2000000, d_v=128), UNSUP),
]


@pytest.mark.parametrize("over,code", CONV_BAD)
def test_conv_decode_validation(over, code):
    a = _conv_args(**over)
    assert gdn.load_library().gdn_conv_decode(ctypes.byref(a), None) == code


def test_conv_store_validation_and_empty():
    lib = gdn.load_library()
    a = _conv_args(n_tokens=10, cu_seqlens=None)
    assert lib.gdn_conv_store(ctypes.byref(a), None) == NULL
    a = _conv_args(n_tokens=10, cu_seqlens=FAKE, v=None)
    assert lib.gdn_conv_store(ctypes.byref(a), None) == NULL
    a = _conv_args(n_tokens=-1, cu_seqlens=FAKE)
    assert lib.gdn_conv_store(ctypes.byref(a), None) == SHAPE
    a = _conv_args(n_tokens=1 << 31, cu_seqlens=FAKE)
    assert lib.gdn_conv_store(ctypes.byref(a), None) == UNSUP
    # the store needs no decode inputs or outputs
    a = _conv_args(n_tokens=10, cu_seqlens=FAKE, a_raw=None, conv_wq=None, q_out=None,
                   n_slots=2, write_slot=None)
    assert lib.gdn_conv_store(ctypes.byref(a), None) == SHAPE   # NULL write_slot needs B slots
    # empty batches launch nothing
    assert lib.gdn_conv_decode(ctypes.byref(_conv_args(B=0, q=None, conv_pool=None)), None) == OK
    assert lib.gdn_conv_store(ctypes.byref(_conv_args(B=0, cu_seqlens=None)), None) == OK
    assert lib.gdn_conv_store(ctypes.byref(_conv_args(B=0, n_tokens=5)), None) == SHAPE


def _fused_args(dover=None, cover=None):
    """gdn_decode_conv's pair: the decode's token inputs and the conv step's
    outputs NULL, everything else as for the separate calls."""
    d = _decode_args(**{"q": None, "k": None, "v": None, "g": None, "beta": None,
                        "d_k": 64, "d_v": 64, **(dover or {})})
    c = _conv_args(**{"q_out": None, "k_out": None, "v_out": None, "g_out": None,
                      "beta_out": None, **(cover or {})})
    return d, c


@pytest.mark.parametrize("dover,cover,code", [
    # the fused call takes no token inputs and writes no conv outputs
    (dict(q=FAKE), None, UNSUP), (dict(beta=FAKE), None, UNSUP),
    (None, dict(v_out=FAKE), UNSUP), (None, dict(g_out=FAKE), UNSUP),
    # the halves must describe one layer
    (dict(B=5), None, SHAPE), (None, dict(H_v=8), SHAPE), (None, dict(d_v=32), SHAPE),
    (None, dict(act_dtype=0), DTYPE),
    # per-head decay only (the front-end makes one decay per head); no 8-bit state
    (dict(decay_mode=1), None, UNSUP), (dict(state_dtype=2, state_bf16_rows=32), None, UNSUP),
    # every check of each separate call still applies
    (dict(rule=7), None, RULE), (dict(state_pool=None), None, NULL), (dict(o=FAKE + 4), None, ALIGN),
    (None, dict(conv_pool=None), NULL), (None, dict(a_raw=None), NULL),
    (None, dict(conv_wq=FAKE + 4), ALIGN), (None, dict(eps=-1.0), SHAPE),
    # more than 8 state heads per q/k head
    (dict(H_qk=1, H_v=16), dict(H_qk=1, H_v=16), UNSUP),
])
def test_decode_conv_validation(dover, cover, code):
    lib = gdn.load_library()
    d, c = _fused_args(dover, cover)
    assert lib.gdn_decode_conv(ctypes.byref(d), ctypes.byref(c), None) == code


def test_decode_conv_null_and_empty():
    lib = gdn.load_library()
    d, c = _fused_args()
    assert lib.gdn_decode_conv(None, ctypes.byref(c), None) == NULL
    assert lib.gdn_decode_conv(ctypes.byref(d), None, None) == NULL
    d, c = _fused_args(dict(B=0, state_pool=None, o=None), dict(B=0, q=None, conv_pool=None))
    assert lib.gdn_decode_conv(ctypes.byref(d), ctypes.byref(c), None) == OK


def _convert_args(**over):
    a = B.ConvertArgs()
    a.n, a.H_v, a.d_k, a.d_v = 4, 2, 128, 128
    a.src_dtype, a.dst_dtype, a.src_bf16_rows, a.dst_bf16_rows = B.BF16, B.Q8, 0, 32
    a.src_n_slots = a.dst_n_slots = 8
    a.src_pool = a.dst_pool = FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,code", [
    (dict(n=-1), SHAPE), (dict(src_n_slots=-1), SHAPE), (dict(src_dtype=3), DTYPE),
    (dict(dst_dtype=-1), DTYPE), (dict(H_v=0), SHAPE), (dict(d_k=48), UNSUP),
    (dict(d_v=256), UNSUP),
    # BF16-row counts: valid for an 8-bit side (multiples of the decode's row quantum), none else
    (dict(dst_bf16_rows=12), SHAPE), (dict(dst_bf16_rows=136), SHAPE),
    (dict(src_bf16_rows=32), SHAPE), (dict(src_dtype=B.Q8, src_bf16_rows=24), SHAPE),
    (dict(n=9, src_slot=None), SHAPE),       # identity slots need n <= n_slots
    (dict(src_pool=None), NULL), (dict(dst_pool=None), NULL),
    (dict(src_pool=FAKE + 8), ALIGN), (dict(dst_pool=FAKE + 4), ALIGN),
    (dict(n=1 << 30, H_v=4), UNSUP),         # grid size
])
def test_state_convert_validation(over, code):
    a = _convert_args(**over)
    assert gdn.load_library().gdn_state_convert(ctypes.byref(a), None) == code


def test_state_convert_null_and_empty():
    lib = gdn.load_library()
    assert lib.gdn_state_convert(None, None) == NULL
    a = _convert_args(n=0, src_pool=None, dst_pool=None)
    assert lib.gdn_state_convert(ctypes.byref(a), None) == OK

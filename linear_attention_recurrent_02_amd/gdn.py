"""Thin ctypes binding of ``libgdn.so`` (the C ABI in include/gdn.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
dtypes, ``torch.cuda.current_stream()`` supplies the stream, and every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the library is missing or refuses a call, these functions raise.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "gdn.h")

RULES = {"linear": 0, "gated": 1, "delta": 2, "gated_delta": 3}
F32, BF16, Q8 = 0, 1, 2
DECAY_HEAD, DECAY_CHANNEL = 0, 1
DEVICE_BAD_SLOT = 1
DEVICE_BAD_SEQ = 2

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class DecodeArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("H_qk", _I32), ("H_v", _I32), ("d_k", _I32), ("d_v", _I32),
                ("rule", _I32), ("state_dtype", _I32), ("act_dtype", _I32),
                ("n_slots", _I64), ("scale", ctypes.c_float), ("decay_mode", _I32),
                ("q", _P), ("k", _P), ("v", _P), ("g", _P), ("beta", _P),
                ("state_pool", _P), ("read_slot", _P), ("write_slot", _P), ("o", _P),
                ("status", _P), ("state_bf16_rows", _I32), ("reserved0", _I32)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("n_seq", _I32), ("H_qk", _I32), ("H_v", _I32), ("d_k", _I32), ("d_v", _I32),
                ("rule", _I32), ("state_dtype", _I32), ("act_dtype", _I32),
                ("use_frontend", _I32), ("conv_k", _I32), ("chunk", _I32),
                ("ckpt_interval", _I32),
                ("n_tokens", _I64), ("n_slots", _I64), ("scale", ctypes.c_float),
                ("eps", ctypes.c_float), ("cu_seqlens", _P), ("q", _P), ("k", _P), ("v", _P),
                ("g", _P), ("beta", _P), ("a_raw", _P), ("b_raw", _P), ("conv_wq", _P),
                ("conv_wk", _P), ("conv_wv", _P), ("state_pool", _P), ("read_slot", _P),
                ("write_slot", _P), ("o", _P), ("workspace", _P),
                ("workspace_bytes", ctypes.c_size_t), ("status", _P), ("ckpt_slot", _P),
                ("ckpt_per_seq", _I32), ("decay_mode", _I32), ("conv_pool", _P),
                ("conv_n_slots", _I64), ("conv_read_slot", _P), ("conv_write_slot", _P),
                ("conv_ckpt_slot", _P)]


class ConvArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("H_qk", _I32), ("H_v", _I32), ("d_k", _I32), ("d_v", _I32),
                ("act_dtype", _I32), ("conv_k", _I32), ("reserved0", _I32),
                ("n_slots", _I64), ("n_tokens", _I64), ("eps", ctypes.c_float),
                ("reserved1", _I32), ("q", _P), ("k", _P), ("v", _P), ("a_raw", _P),
                ("b_raw", _P), ("conv_wq", _P), ("conv_wk", _P), ("conv_wv", _P),
                ("conv_pool", _P), ("read_slot", _P), ("write_slot", _P), ("cu_seqlens", _P),
                ("q_out", _P), ("k_out", _P), ("v_out", _P), ("g_out", _P), ("beta_out", _P),
                ("status", _P)]


class ConvertArgs(ctypes.Structure):
    _fields_ = [("n", _I32), ("H_v", _I32), ("d_k", _I32), ("d_v", _I32),
                ("src_dtype", _I32), ("dst_dtype", _I32), ("src_bf16_rows", _I32),
                ("dst_bf16_rows", _I32), ("src_n_slots", _I64), ("dst_n_slots", _I64),
                ("src_pool", _P), ("dst_pool", _P), ("src_slot", _P), ("dst_slot", _P),
                ("status", _P)]


class GdnError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: status {code} ({gdn_status_string(code)})")


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libgdn.so (built by ``build.build()``); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_state_bytes.restype = ctypes.c_size_t
    lib.gdn_state_bytes.argtypes = [_I32, _I32, _I32, _I32]
    lib.gdn_state_q8_bytes.restype = ctypes.c_size_t
    lib.gdn_state_q8_bytes.argtypes = [_I32, _I32, _I32, _I32]
    lib.gdn_state_q8_row_quantum.restype = _I32
    lib.gdn_state_q8_row_quantum.argtypes = [_I32, _I32]
    lib.gdn_prefill_workspace_size.restype = ctypes.c_size_t
    lib.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillArgs)]
    lib.gdn_parse_rule.restype = _I32
    lib.gdn_parse_rule.argtypes = [ctypes.c_char_p, ctypes.POINTER(_I32)]
    lib.gdn_decode.restype = _I32
    lib.gdn_decode.argtypes = [ctypes.POINTER(DecodeArgs), _P]
    lib.gdn_frontend.restype = _I32
    lib.gdn_frontend.argtypes = [ctypes.POINTER(PrefillArgs), _P, _P, _P, _P, _P, _P]
    lib.gdn_prefill.restype = _I32
    lib.gdn_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _P]
    lib.gdn_prefill_noalloc.restype = _I32
    lib.gdn_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillArgs), _P]
    lib.gdn_noalloc_workspace_bytes.restype = ctypes.c_size_t
    lib.gdn_noalloc_workspace_bytes.argtypes = []
    lib.gdn_mixed.restype = _I32
    lib.gdn_mixed.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(PrefillArgs), _P]
    lib.gdn_conv_decode.restype = _I32
    lib.gdn_conv_decode.argtypes = [ctypes.POINTER(ConvArgs), _P]
    lib.gdn_conv_store.restype = _I32
    lib.gdn_conv_store.argtypes = [ctypes.POINTER(ConvArgs), _P]
    lib.gdn_state_convert.restype = _I32
    lib.gdn_state_convert.argtypes = [ctypes.POINTER(ConvertArgs), _P]
    lib.gdn_sizeof_convert_args.restype = ctypes.c_size_t
    lib.gdn_sizeof_convert_args.argtypes = []
    lib.gdn_decode_conv.restype = _I32
    lib.gdn_decode_conv.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ConvArgs), _P]
    lib.gdn_conv_slot_bytes.restype = ctypes.c_size_t
    lib.gdn_conv_slot_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32]
    lib.gdn_validate_slots.restype = _I32
    lib.gdn_validate_slots.argtypes = [_P, _P, _I32, _I64]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [_I32]
    lib.gdn_abi_version.restype = _I32
    lib.gdn_abi_version.argtypes = []
    lib.gdn_sizeof_decode_args.restype = ctypes.c_size_t
    lib.gdn_sizeof_prefill_args.restype = ctypes.c_size_t
    lib.gdn_sizeof_conv_args.restype = ctypes.c_size_t
    if lib.gdn_sizeof_decode_args() != ctypes.sizeof(DecodeArgs) or \
            lib.gdn_sizeof_prefill_args() != ctypes.sizeof(PrefillArgs) or \
            lib.gdn_sizeof_conv_args() != ctypes.sizeof(ConvArgs) or \
            lib.gdn_sizeof_convert_args() != ctypes.sizeof(ConvertArgs):
        raise RuntimeError("libgdn.so argument-struct layout differs from this binding")
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions that include/gdn.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, flags=re.M)))


# ----------------------------------------------------------------------------
# marshalling helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_ACT = (torch.bfloat16, torch.float32)


def _need(t, name, *, dtype=None, dtypes=None, shape=None):
    """Check a tensor's dtype and exact shape (None passes: absence is the
    library's to judge).  Runs before any device check, so a wrong dtype or
    shape is reported as such on any device."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, "
                         f"got {tuple(t.shape)}")
    return t


def _row_dim(t, name, rows, heads):
    """Per-head size of a [rows, heads * d] or [rows, heads, d] tensor."""
    if t.dim() == 3:
        if t.shape[0] != rows or t.shape[1] != heads:
            raise ValueError(f"{name} must be [{rows}, {heads}, d], got {tuple(t.shape)}")
        return int(t.shape[2])
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] % heads != 0 or t.shape[1] == 0:
        raise ValueError(f"{name} must be [{rows}, {heads} * d], got {tuple(t.shape)}")
    return int(t.shape[1]) // heads


def _status(t):
    return _need(t, "status", dtypes=(torch.int32,), shape=(1,)) if t is not None else None


def _rule(rule) -> int:
    if isinstance(rule, str):
        out = _I32()
        code = load_library().gdn_parse_rule(rule.encode(), ctypes.byref(out))
        if code:
            raise GdnError("gdn_parse_rule", code)
        return out.value
    return int(rule)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)

def gdn_state_bytes(H_v: int, d_k: int, d_v: int, state_dtype: int = BF16) -> int:
    return int(load_library().gdn_state_bytes(H_v, d_k, d_v, state_dtype))


def gdn_state_q8_bytes(H_v: int, d_k: int, d_v: int, bf16_rows: int) -> int:
    """Bytes of one slot in the 8-bit state format (0 for invalid sizes)."""
    return int(load_library().gdn_state_q8_bytes(H_v, d_k, d_v, bf16_rows))


def gdn_parse_rule(name: str | None) -> int:
    out = _I32()
    code = load_library().gdn_parse_rule(None if name is None else name.encode(), ctypes.byref(out))
    if code:
        raise GdnError("gdn_parse_rule", code)
    return out.value


def gdn_status_string(code: int) -> str:
    return load_library().gdn_status_string(int(code)).decode()


def gdn_abi_version() -> int:
    return int(load_library().gdn_abi_version())


def gdn_validate_slots(read_slot, write_slot, n: int, n_slots: int) -> int:
    """Host-side slot-contract check; returns the status code (0 = OK)."""
    def host(a):
        if a is None:
            return None, None
        t = torch.as_tensor(a, dtype=torch.int32).contiguous().cpu()
        return t, ctypes.c_void_p(t.data_ptr())
    rt, rp = host(read_slot)
    wt, wp = host(write_slot)
    return int(load_library().gdn_validate_slots(rp, wp, int(n), int(n_slots)))


def make_decode_args(q, k, v, g, beta, state_pool, read_slot=None, write_slot=None, o=None, *,
                     rule="gated_delta", scale=1.0, status=None, state_bf16_rows=None):
    """Build a DecodeArgs struct.  q, k: [B, H_qk, d_k]; v: [B, H_v, d_v];
    g: [B, H_v] float32, or [B, H_v, d_k] for a per-key-channel decay; beta:
    [B, H_v] float32; state_pool: [n_slots, H_v, d_k, d_v] bfloat16 or
    float32, or the 8-bit format as uint8 [n_slots, H_v, tile bytes] with
    state_bf16_rows BF16 key channels per tile; read_slot / write_slot: [B]
    int32 or None.  Returns (args, o, keepalive)."""
    _need(q, "q", dtypes=_ACT)
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H_qk, d_k], got {tuple(q.shape)}")
    B, H_qk, d_k = q.shape
    _need(k, "k", dtype=q.dtype, shape=q.shape)
    _need(v, "v", dtype=q.dtype)
    if v.dim() != 3 or v.shape[0] != B:
        raise ValueError(f"v must be [B={B}, H_v, d_v], got {tuple(v.shape)}")
    H_v, d_v = v.shape[1], v.shape[2]
    if g is not None and g.dim() == 3:
        _need(g, "g", dtype=torch.float32, shape=(B, H_v, d_k))
    else:
        _need(g, "g", dtype=torch.float32, shape=(B, H_v))
    _need(beta, "beta", dtype=torch.float32, shape=(B, H_v))
    q8 = isinstance(state_pool, torch.Tensor) and state_pool.dtype == torch.uint8
    if q8:
        if state_bf16_rows is None:
            raise ValueError("an 8-bit state pool (uint8) needs state_bf16_rows")
        tb = gdn_state_q8_bytes(1, d_k, d_v, int(state_bf16_rows))
        if tb == 0:
            step = int(load_library().gdn_state_q8_row_quantum(d_k, d_v))
            raise ValueError(f"state_bf16_rows must be a multiple of {step} in [0, {d_k}]")
        if state_pool.dim() != 3 or tuple(state_pool.shape[1:]) != (H_v, tb):
            raise ValueError(f"state_pool must be [n_slots, {H_v}, {tb}] bytes, "
                             f"got {tuple(state_pool.shape)}")
    else:
        if state_bf16_rows:
            raise ValueError("state_bf16_rows applies to an 8-bit (uint8) state pool only")
        _need(state_pool, "state_pool", dtypes=_ACT)
        if state_pool.dim() != 4 or tuple(state_pool.shape[1:]) != (H_v, d_k, d_v):
            raise ValueError(f"state_pool must be [n_slots, {H_v}, {d_k}, {d_v}], "
                             f"got {tuple(state_pool.shape)}")
    _need(read_slot, "read_slot", dtype=torch.int32, shape=(B,))
    _need(write_slot, "write_slot", dtype=torch.int32, shape=(B,))
    _need(o, "o", dtype=q.dtype, shape=(B, H_v, d_v))
    _status(status)
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                    ("state_pool", state_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("o", o), ("status", status)):
        _dev(t, name)
    if o is None:
        o = torch.empty((B, H_v, d_v), dtype=q.dtype, device=q.device)
    a = DecodeArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = B, H_qk, H_v, d_k, d_v
    a.rule = _rule(rule)
    a.state_dtype = Q8 if q8 else _dtype_code(state_pool)
    a.state_bf16_rows = int(state_bf16_rows) if q8 else 0
    a.reserved0 = 0
    a.act_dtype = _dtype_code(q)
    a.n_slots = state_pool.shape[0]
    a.scale = float(scale)
    # g [B, H_v]: one decay per state head; [B, H_v, d_k]: one per key channel
    a.decay_mode = DECAY_CHANNEL if g is not None and g.dim() == 3 else DECAY_HEAD
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.state_pool, a.read_slot, a.write_slot = _ptr(state_pool), _ptr(read_slot), _ptr(write_slot)
    a.o, a.status = _ptr(o), _ptr(status)
    return a, o, (q, k, v, g, beta, state_pool, read_slot, write_slot, o, status)


def gdn_decode(q, k, v, g, beta, state_pool, read_slot=None, write_slot=None, o=None, *,
               rule="gated_delta", scale=1.0, status=None, stream=None, state_bf16_rows=None):
    """One decode token for B requests; updates ``state_pool`` in place and
    returns o [B, H_v, d_v] (dtype of q)."""
    a, o, keep = make_decode_args(q, k, v, g, beta, state_pool, read_slot, write_slot, o,
                                  rule=rule, scale=scale, status=status,
                                  state_bf16_rows=state_bf16_rows)
    code = load_library().gdn_decode(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_decode", code)
    return o


def make_prefill_args(cu_seqlens, q, k, v, state_pool, read_slot=None, write_slot=None, o=None, *,
                      H_qk, H_v, g=None, beta=None, a_raw=None, b_raw=None, conv_wq=None,
                      conv_wk=None, conv_wv=None, rule="gated_delta", scale=1.0, eps=1e-6,
                      chunk=64, workspace=None, status=None, ckpt_interval=0, ckpt_slot=None,
                      conv_pool=None, conv_read_slot=None, conv_write_slot=None,
                      conv_ckpt_slot=None, alloc_workspace=True):
    """Build a PrefillArgs struct.  q, k: [N, H_qk*d_k] (or [N, H_qk, d_k]);
    v: [N, H_v*d_v]; with conv weights given the front-end runs (a_raw,
    b_raw are the gate logits), otherwise g, beta are used as given.  With
    ckpt_interval > 0 (a multiple of chunk), ckpt_slot [n_seq, per_seq] int32
    names the slots of the intermediate checkpoints.  With the front-end,
    conv_pool [n, conv_k-1, 2*H_qk*d_k + H_v*d_v] holds conv windows:
    conv_read_slot / conv_write_slot [n_seq] and conv_ckpt_slot (shaped as
    ckpt_slot) name the windows each sequence resumes and leaves.
    Returns (args, o, keepalive); allocates the workspace when needed unless
    alloc_workspace is False."""
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be [n_seq + 1]")
    n_seq = cu_seqlens.shape[0] - 1
    _need(q, "q", dtypes=_ACT)
    _need(state_pool, "state_pool", dtypes=_ACT)
    if state_pool.dim() != 4:
        raise ValueError(f"state_pool must be [n_slots, H_v, d_k, d_v], got {tuple(state_pool.shape)}")
    N = q.shape[0]
    d_k = _row_dim(q, "q", N, H_qk) if N else state_pool.shape[2]
    _need(k, "k", dtype=q.dtype, shape=q.shape)
    _need(v, "v", dtype=q.dtype)
    d_v = _row_dim(v, "v", N, H_v) if N else state_pool.shape[3]
    if tuple(state_pool.shape[1:]) != (H_v, d_k, d_v):
        raise ValueError(f"state_pool must be [n_slots, {H_v}, {d_k}, {d_v}], "
                         f"got {tuple(state_pool.shape)}")
    _need(read_slot, "read_slot", dtype=torch.int32, shape=(n_seq,))
    _need(write_slot, "write_slot", dtype=torch.int32, shape=(n_seq,))
    _need(o, "o", dtype=q.dtype, shape=(N, H_v, d_v))
    channel = g is not None and g.dim() == 3  # one log-decay per key channel
    if channel:
        _need(g, "g", dtype=torch.float32, shape=(N, H_v, d_k))
    for name, t in ((("g", g),) if not channel else ()) + (("beta", beta), ("a_raw", a_raw),
                                                           ("b_raw", b_raw)):
        _need(t, name, dtype=torch.float32, shape=(N, H_v))
    use_fe = conv_wq is not None
    K = conv_wq.shape[-1] if use_fe and conv_wq.dim() == 2 else 4
    _need(conv_wq, "conv_wq", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wk, "conv_wk", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wv, "conv_wv", dtype=torch.float32, shape=(H_v * d_v, K))
    if ckpt_slot is not None:
        _need(ckpt_slot, "ckpt_slot", dtype=torch.int32)
        if ckpt_slot.dim() != 2 or ckpt_slot.shape[0] != n_seq:
            raise ValueError(f"ckpt_slot must be [{n_seq}, per_seq], got {tuple(ckpt_slot.shape)}")
    _conv_slots(conv_pool, conv_read_slot, conv_write_slot, conv_ckpt_slot, ckpt_slot, q, n_seq,
                H_qk, H_v, d_k, d_v, K, use_fe)
    _need(workspace, "workspace", dtype=torch.uint8)
    _status(status)
    for name, t in (("cu_seqlens", cu_seqlens), ("q", q), ("k", k), ("v", v),
                    ("state_pool", state_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("o", o), ("g", g), ("beta", beta),
                    ("a_raw", a_raw), ("b_raw", b_raw), ("conv_wq", conv_wq),
                    ("conv_wk", conv_wk), ("conv_wv", conv_wv), ("status", status),
                    ("ckpt_slot", ckpt_slot), ("workspace", workspace), ("conv_pool", conv_pool),
                    ("conv_read_slot", conv_read_slot), ("conv_write_slot", conv_write_slot),
                    ("conv_ckpt_slot", conv_ckpt_slot)):
        _dev(t, name)
    if o is None:
        o = torch.empty((N, H_v, d_v), dtype=q.dtype, device=q.device)
    a = PrefillArgs()
    a.n_seq = n_seq
    a.H_qk, a.H_v, a.d_k, a.d_v = H_qk, H_v, d_k, d_v
    a.rule = _rule(rule)
    a.state_dtype = _dtype_code(state_pool)
    a.act_dtype = _dtype_code(q)
    a.use_frontend = 1 if use_fe else 0
    a.conv_k = K
    a.chunk = chunk
    a.ckpt_interval = int(ckpt_interval)
    a.n_tokens = N
    a.n_slots = state_pool.shape[0]
    a.scale, a.eps = float(scale), float(eps)
    a.cu_seqlens, a.q, a.k, a.v = _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v)
    a.g, a.beta, a.a_raw, a.b_raw = _ptr(g), _ptr(beta), _ptr(a_raw), _ptr(b_raw)
    a.conv_wq, a.conv_wk, a.conv_wv = _ptr(conv_wq), _ptr(conv_wk), _ptr(conv_wv)
    a.state_pool, a.read_slot, a.write_slot = _ptr(state_pool), _ptr(read_slot), _ptr(write_slot)
    a.o, a.status = _ptr(o), _ptr(status)
    a.ckpt_slot = _ptr(ckpt_slot)
    a.ckpt_per_seq = 0 if ckpt_slot is None else int(ckpt_slot.shape[-1])
    # g [N, H_v]: one decay per state head; [N, H_v, d_k]: one per key channel
    a.decay_mode = DECAY_CHANNEL if channel else DECAY_HEAD
    a.conv_pool = _ptr(conv_pool)
    a.conv_n_slots = 0 if conv_pool is None else conv_pool.shape[0]
    a.conv_read_slot, a.conv_write_slot = _ptr(conv_read_slot), _ptr(conv_write_slot)
    a.conv_ckpt_slot = _ptr(conv_ckpt_slot)
    need = int(load_library().gdn_prefill_workspace_size(ctypes.byref(a)))
    if need and workspace is None and alloc_workspace:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    keep = (cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o, g, beta, a_raw, b_raw,
            conv_wq, conv_wk, conv_wv, workspace, status, ckpt_slot, conv_pool, conv_read_slot,
            conv_write_slot, conv_ckpt_slot)
    return a, o, keep


def _conv_slots(conv_pool, read_slot, write_slot, ckpt_slot, state_ckpt_slot, q, n_seq, H_qk,
                H_v, d_k, d_v, K, use_fe):
    """Checks of a prefill's conv-window arguments (see gdn_prefill_args)."""
    given = [t is not None for t in (read_slot, write_slot, ckpt_slot)]
    if any(given) and not use_fe:
        raise ValueError("conv slots need the front-end (conv weights)")
    if any(given) and conv_pool is None:
        raise ValueError("conv slots need conv_pool")
    if conv_pool is not None:
        C = 2 * H_qk * d_k + H_v * d_v
        _need(conv_pool, "conv_pool", dtype=q.dtype)
        if conv_pool.dim() != 3 or tuple(conv_pool.shape[1:]) != (K - 1, C):
            raise ValueError(f"conv_pool must be [n_slots, {K - 1}, {C}], "
                             f"got {tuple(conv_pool.shape)}")
    _need(read_slot, "conv_read_slot", dtype=torch.int32, shape=(n_seq,))
    _need(write_slot, "conv_write_slot", dtype=torch.int32, shape=(n_seq,))
    if ckpt_slot is not None:
        if state_ckpt_slot is None:
            raise ValueError("conv_ckpt_slot goes with ckpt_slot")
        _need(ckpt_slot, "conv_ckpt_slot", dtype=torch.int32, shape=tuple(state_ckpt_slot.shape))


def gdn_prefill(cu_seqlens, q, k, v, state_pool, read_slot=None, write_slot=None, o=None, *,
                stream=None, **kw):
    """Chunked prefill over packed sequences; returns o [N, H_v, d_v]."""
    a, o, keep = make_prefill_args(cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o, **kw)
    code = load_library().gdn_prefill(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_prefill", code)
    return o


def gdn_prefill_noalloc(cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o, *,
                        stream=None, **kw):
    """gdn_prefill without any allocation: the library's fixed device
    workspace replaces the caller's, and the caller passes o [N, H_v, d_v]
    (nothing is allocated here either).  Returns o."""
    if o is None:
        raise ValueError("gdn_prefill_noalloc needs the output tensor o")
    if kw.get("workspace") is not None:
        raise ValueError("gdn_prefill_noalloc uses the library's workspace, not the caller's")
    a, o, keep = make_prefill_args(cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o,
                                   alloc_workspace=False, **kw)
    code = load_library().gdn_prefill_noalloc(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_prefill_noalloc", code)
    return o


def gdn_noalloc_workspace_bytes() -> int:
    return int(load_library().gdn_noalloc_workspace_bytes())


def gdn_frontend(cu_seqlens, q_raw, k_raw, v_raw, *, H_qk, H_v, conv_wq, conv_wk, conv_wv,
                 a_raw, b_raw, eps=1e-6, conv_pool=None, conv_read_slot=None, stream=None):
    """The front-end alone: returns (q [N,H_qk,d_k], k, v [N,H_v,d_v], g, beta).
    conv_pool / conv_read_slot: the windows the sequences resume, as for
    make_prefill_args."""
    _need(cu_seqlens, "cu_seqlens", dtype=torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
        raise ValueError("cu_seqlens must be [n_seq + 1]")
    _need(q_raw, "q_raw", dtypes=_ACT)
    N = q_raw.shape[0]
    if N == 0:
        raise ValueError("gdn_frontend needs at least one token")
    d_k = _row_dim(q_raw, "q_raw", N, H_qk)
    d_v = _row_dim(v_raw, "v_raw", N, H_v)
    _need(k_raw, "k_raw", dtype=q_raw.dtype, shape=q_raw.shape)
    _need(v_raw, "v_raw", dtype=q_raw.dtype)
    K = conv_wq.shape[-1] if conv_wq.dim() == 2 else 4
    _need(conv_wq, "conv_wq", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wk, "conv_wk", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wv, "conv_wv", dtype=torch.float32, shape=(H_v * d_v, K))
    _need(a_raw, "a_raw", dtype=torch.float32, shape=(N, H_v))
    _need(b_raw, "b_raw", dtype=torch.float32, shape=(N, H_v))
    _conv_slots(conv_pool, conv_read_slot, None, None, None, q_raw, cu_seqlens.shape[0] - 1,
                H_qk, H_v, d_k, d_v, K, True)
    for name, t in (("cu_seqlens", cu_seqlens), ("q_raw", q_raw), ("k_raw", k_raw),
                    ("v_raw", v_raw), ("conv_wq", conv_wq), ("conv_wk", conv_wk),
                    ("conv_wv", conv_wv), ("a_raw", a_raw), ("b_raw", b_raw),
                    ("conv_pool", conv_pool), ("conv_read_slot", conv_read_slot)):
        _dev(t, name)
    a = PrefillArgs()
    a.n_seq = cu_seqlens.shape[0] - 1
    a.H_qk, a.H_v, a.d_k, a.d_v = H_qk, H_v, d_k, d_v
    a.rule = RULES["gated_delta"]
    a.state_dtype = F32
    a.act_dtype = _dtype_code(q_raw)
    a.use_frontend, a.conv_k, a.chunk, a.ckpt_interval = 1, K, 64, 0
    a.decay_mode = DECAY_HEAD
    a.n_tokens, a.n_slots = N, 0
    a.scale, a.eps = 1.0, float(eps)
    a.cu_seqlens, a.q, a.k, a.v = _ptr(cu_seqlens), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw)
    a.a_raw, a.b_raw = _ptr(a_raw), _ptr(b_raw)
    a.conv_wq, a.conv_wk, a.conv_wv = _ptr(conv_wq), _ptr(conv_wk), _ptr(conv_wv)
    a.conv_pool = _ptr(conv_pool)
    a.conv_n_slots = 0 if conv_pool is None else conv_pool.shape[0]
    a.conv_read_slot = _ptr(conv_read_slot)
    q = torch.empty((N, H_qk, d_k), dtype=q_raw.dtype, device=q_raw.device)
    k = torch.empty_like(q)
    v = torch.empty((N, H_v, d_v), dtype=v_raw.dtype, device=q_raw.device)
    g = torch.empty((N, H_v), dtype=torch.float32, device=q_raw.device)
    beta = torch.empty_like(g)
    code = load_library().gdn_frontend(ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _stream(stream))
    if code:
        raise GdnError("gdn_frontend", code)
    return q, k, v, g, beta


def gdn_mixed(decode_args: DecodeArgs, prefill_args: PrefillArgs, stream=None):
    """One launch for a decode batch and a prefill batch built with
    make_decode_args / make_prefill_args (keep their keepalive tuples)."""
    code = load_library().gdn_mixed(ctypes.byref(decode_args), ctypes.byref(prefill_args),
                                    _stream(stream))
    if code:
        raise GdnError("gdn_mixed", code)


def gdn_conv_slot_bytes(H_qk: int, H_v: int, d_k: int, d_v: int, conv_k: int = 4,
                        act_dtype: int = BF16) -> int:
    return int(load_library().gdn_conv_slot_bytes(H_qk, H_v, d_k, d_v, conv_k, act_dtype))


def make_conv_args(q_raw, k_raw, v_raw, conv_pool, *, H_qk, H_v, read_slot=None, write_slot=None,
                   cu_seqlens=None, a_raw=None, b_raw=None, conv_wq=None, conv_wk=None,
                   conv_wv=None, outputs=None, eps=1e-6, status=None):
    """Build a ConvArgs struct.  Decode (cu_seqlens None): q_raw, k_raw [B,
    H_qk*d_k], v_raw [B, H_v*d_v]; store: the same over n_tokens rows with
    cu_seqlens [B+1].  conv_pool: [n_slots, conv_k-1, 2*H_qk*d_k + H_v*d_v].
    outputs: (q, k, v, g, beta) tensors or None.  Returns (args, keepalive)."""
    _need(q_raw, "q_raw", dtypes=_ACT)
    rows = q_raw.shape[0]
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32)
        if cu_seqlens.dim() != 1 or cu_seqlens.shape[0] < 1:
            raise ValueError("cu_seqlens must be [n_seq + 1]")
    B = rows if cu_seqlens is None else cu_seqlens.shape[0] - 1
    _need(conv_pool, "conv_pool", dtype=q_raw.dtype)
    if conv_pool.dim() != 3:
        raise ValueError(f"conv_pool must be [n_slots, conv_k - 1, C], got {tuple(conv_pool.shape)}")
    if rows:
        d_k = _row_dim(q_raw, "q_raw", rows, H_qk)
        d_v = _row_dim(v_raw, "v_raw", rows, H_v)
    else:  # an empty store: the head sizes come from the pool's channel count
        d_k = q_raw.shape[-1] // H_qk if q_raw.dim() == 2 else q_raw.shape[-1]
        d_v = v_raw.shape[-1] // H_v if v_raw.dim() == 2 else v_raw.shape[-1]
    _need(k_raw, "k_raw", dtype=q_raw.dtype, shape=q_raw.shape)
    _need(v_raw, "v_raw", dtype=q_raw.dtype)
    C = 2 * H_qk * d_k + H_v * d_v
    if conv_pool.shape[2] != C:
        raise ValueError(f"conv_pool must have {C} channels (2*H_qk*d_k + H_v*d_v), "
                         f"got {tuple(conv_pool.shape)}")
    K = conv_pool.shape[1] + 1
    _need(read_slot, "read_slot", dtype=torch.int32, shape=(B,))
    _need(write_slot, "write_slot", dtype=torch.int32, shape=(B,))
    _need(a_raw, "a_raw", dtype=torch.float32, shape=(B, H_v))
    _need(b_raw, "b_raw", dtype=torch.float32, shape=(B, H_v))
    _need(conv_wq, "conv_wq", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wk, "conv_wk", dtype=torch.float32, shape=(H_qk * d_k, K))
    _need(conv_wv, "conv_wv", dtype=torch.float32, shape=(H_v * d_v, K))
    if outputs is not None:
        qo, ko, vo, go, bo = outputs
        _need(qo, "q_out", dtype=q_raw.dtype, shape=(B, H_qk, d_k))
        _need(ko, "k_out", dtype=q_raw.dtype, shape=(B, H_qk, d_k))
        _need(vo, "v_out", dtype=q_raw.dtype, shape=(B, H_v, d_v))
        _need(go, "g_out", dtype=torch.float32, shape=(B, H_v))
        _need(bo, "beta_out", dtype=torch.float32, shape=(B, H_v))
    _status(status)
    for name, t in (("q_raw", q_raw), ("k_raw", k_raw), ("v_raw", v_raw),
                    ("conv_pool", conv_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("cu_seqlens", cu_seqlens), ("a_raw", a_raw),
                    ("b_raw", b_raw), ("conv_wq", conv_wq), ("conv_wk", conv_wk),
                    ("conv_wv", conv_wv), ("status", status)):
        _dev(t, name)
    a = ConvArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = B, H_qk, H_v, d_k, d_v
    a.act_dtype = _dtype_code(q_raw)
    a.conv_k = K
    a.reserved0 = a.reserved1 = 0
    a.n_slots = conv_pool.shape[0]
    a.n_tokens = 0 if cu_seqlens is None else rows
    a.eps = float(eps)
    a.q, a.k, a.v = _ptr(q_raw), _ptr(k_raw), _ptr(v_raw)
    a.a_raw, a.b_raw = _ptr(a_raw), _ptr(b_raw)
    a.conv_wq, a.conv_wk, a.conv_wv = _ptr(conv_wq), _ptr(conv_wk), _ptr(conv_wv)
    a.conv_pool, a.read_slot, a.write_slot = _ptr(conv_pool), _ptr(read_slot), _ptr(write_slot)
    a.cu_seqlens, a.status = _ptr(cu_seqlens), _ptr(status)
    if outputs is not None:
        for name, t in zip(("q_out", "k_out", "v_out", "g_out", "beta_out"), outputs):
            setattr(a, name, _ptr(_dev(t, name)))
    keep = (q_raw, k_raw, v_raw, conv_pool, read_slot, write_slot, cu_seqlens, a_raw, b_raw,
            conv_wq, conv_wk, conv_wv, outputs, status)
    return a, keep


def gdn_conv_decode(q_raw, k_raw, v_raw, conv_pool, read_slot=None, write_slot=None, *, H_qk,
                    H_v, conv_wq, conv_wk, conv_wv, a_raw, b_raw, eps=1e-6, status=None,
                    stream=None):
    """The front-end for one decode token per request, conv window from
    conv_pool (updated in place).  Returns (q [B,H_qk,d_k], k, v [B,H_v,d_v],
    g, beta)."""
    B = q_raw.shape[0]
    d_k = q_raw.shape[-1] // H_qk if q_raw.dim() == 2 else q_raw.shape[-1]
    d_v = v_raw.shape[-1] // H_v if v_raw.dim() == 2 else v_raw.shape[-1]
    dev = q_raw.device
    q = torch.empty((B, H_qk, d_k), dtype=q_raw.dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((B, H_v, d_v), dtype=v_raw.dtype, device=dev)
    g = torch.empty((B, H_v), dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)
    a, keep = make_conv_args(q_raw, k_raw, v_raw, conv_pool, H_qk=H_qk, H_v=H_v,
                             read_slot=read_slot, write_slot=write_slot, a_raw=a_raw,
                             b_raw=b_raw, conv_wq=conv_wq, conv_wk=conv_wk, conv_wv=conv_wv,
                             outputs=(q, k, v, g, beta), eps=eps, status=status)
    code = load_library().gdn_conv_decode(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_conv_decode", code)
    return q, k, v, g, beta


def make_decode_conv_args(q_raw, k_raw, v_raw, conv_pool, state_pool, *, H_qk, H_v, conv_wq,
                          conv_wk, conv_wv, a_raw, b_raw, read_slot=None, write_slot=None,
                          conv_read_slot=None, conv_write_slot=None, o=None,
                          rule="gated_delta", scale=1.0, eps=1e-6, status=None):
    """Build the (DecodeArgs, ConvArgs) pair of gdn_decode_conv: the decode's
    token inputs are NULL (the conv step makes them) and so are the conv
    step's outputs.  Returns (decode_args, conv_args, o, keepalive)."""
    _need(q_raw, "q_raw", dtypes=_ACT)
    B = q_raw.shape[0]
    d_k = _row_dim(q_raw, "q_raw", B, H_qk)
    d_v = _row_dim(v_raw, "v_raw", B, H_v)
    _need(k_raw, "k_raw", dtype=q_raw.dtype, shape=q_raw.shape)
    _need(v_raw, "v_raw", dtype=q_raw.dtype)
    # the decode's checks, with views of the raw inputs and the raw gates standing in
    d, o, keep_d = make_decode_args(q_raw.reshape(B, H_qk, d_k), k_raw.reshape(B, H_qk, d_k),
                                    v_raw.reshape(B, H_v, d_v), a_raw, b_raw, state_pool,
                                    read_slot, write_slot, o, rule=rule, scale=scale,
                                    status=status)
    d.q = d.k = d.v = d.g = d.beta = None
    c, keep_c = make_conv_args(q_raw, k_raw, v_raw, conv_pool, H_qk=H_qk, H_v=H_v,
                               read_slot=conv_read_slot, write_slot=conv_write_slot, a_raw=a_raw,
                               b_raw=b_raw, conv_wq=conv_wq, conv_wk=conv_wk, conv_wv=conv_wv,
                               eps=eps)
    return d, c, o, (keep_d, keep_c)


def gdn_decode_conv(q_raw, k_raw, v_raw, conv_pool, state_pool, *, H_qk, H_v, conv_wq, conv_wk,
                    conv_wv, a_raw, b_raw, read_slot=None, write_slot=None, conv_read_slot=None,
                    conv_write_slot=None, o=None, rule="gated_delta", scale=1.0, eps=1e-6,
                    status=None, stream=None):
    """One decode token with the conv step fused in: raw q, k [B, H_qk*d_k]
    and v [B, H_v*d_v], the conv window from conv_pool and the state from
    state_pool (both updated through their slots).  Returns o [B, H_v, d_v];
    bitwise gdn_conv_decode followed by gdn_decode."""
    d, c, o, keep = make_decode_conv_args(
        q_raw, k_raw, v_raw, conv_pool, state_pool, H_qk=H_qk, H_v=H_v, conv_wq=conv_wq,
        conv_wk=conv_wk, conv_wv=conv_wv, a_raw=a_raw, b_raw=b_raw, read_slot=read_slot,
        write_slot=write_slot, conv_read_slot=conv_read_slot, conv_write_slot=conv_write_slot,
        o=o, rule=rule, scale=scale, eps=eps, status=status)
    code = load_library().gdn_decode_conv(ctypes.byref(d), ctypes.byref(c), _stream(stream))
    if code:
        raise GdnError("gdn_decode_conv", code)
    return o


def _pool_kind(pool, name, bf16_rows):
    """Storage format of a state pool tensor: BF16, FP32, or the 8-bit format
    (uint8 [n_slots, H_v, tile bytes], which needs its BF16-row count)."""
    if pool.dtype == torch.uint8:
        if bf16_rows is None:
            raise ValueError(f"an 8-bit {name} (uint8) needs its bf16_rows")
        if pool.dim() != 3:
            raise ValueError(f"{name} must be [n_slots, H_v, tile bytes], got {tuple(pool.shape)}")
        return Q8, int(bf16_rows)
    _need(pool, name, dtypes=_ACT)
    if pool.dim() != 4:
        raise ValueError(f"{name} must be [n_slots, H_v, d_k, d_v], got {tuple(pool.shape)}")
    if bf16_rows:
        raise ValueError(f"bf16_rows applies to an 8-bit (uint8) {name} only")
    return _dtype_code(pool), 0


def gdn_state_convert(src_pool, dst_pool, src_slot=None, dst_slot=None, *, d_k=None, d_v=None,
                      src_bf16_rows=None, dst_bf16_rows=None, status=None, stream=None):
    """dst_pool[dst_slot[i]] = the states src_pool[src_slot[i]] represents, in
    dst_pool's format (torch.bfloat16 / torch.float32 [n, H_v, d_k, d_v], or
    the 8-bit format as uint8 [n, H_v, tile bytes] with its bf16_rows)."""
    sk, sh = _pool_kind(src_pool, "src_pool", src_bf16_rows)
    dk_, dh = _pool_kind(dst_pool, "dst_pool", dst_bf16_rows)
    for pool in (src_pool, dst_pool):
        if pool.dim() == 4:
            d_k = pool.shape[2] if d_k is None else d_k
            d_v = pool.shape[3] if d_v is None else d_v
    if d_k is None or d_v is None:
        raise ValueError("two 8-bit pools need d_k and d_v")
    H_v = src_pool.shape[1]
    for pool, kind, rows, name in ((src_pool, sk, sh, "src_pool"), (dst_pool, dk_, dh, "dst_pool")):
        want = (H_v, gdn_state_q8_bytes(1, d_k, d_v, rows)) if kind == Q8 else (H_v, d_k, d_v)
        if tuple(pool.shape[1:]) != tuple(want):
            raise ValueError(f"{name} must be [n_slots, {', '.join(map(str, want))}], "
                             f"got {tuple(pool.shape)}")
    n = None
    for t, name in ((src_slot, "src_slot"), (dst_slot, "dst_slot")):
        if t is not None:
            _need(t, name, dtype=torch.int32)
            if t.dim() != 1 or (n is not None and t.shape[0] != n):
                raise ValueError("src_slot and dst_slot must be [n] int32 of one length")
            n = t.shape[0]
    if n is None:
        n = min(src_pool.shape[0], dst_pool.shape[0])
    _status(status)
    for name, t in (("src_pool", src_pool), ("dst_pool", dst_pool), ("src_slot", src_slot),
                    ("dst_slot", dst_slot), ("status", status)):
        _dev(t, name)
    a = ConvertArgs()
    a.n, a.H_v, a.d_k, a.d_v = n, H_v, d_k, d_v
    a.src_dtype, a.dst_dtype, a.src_bf16_rows, a.dst_bf16_rows = sk, dk_, sh, dh
    a.src_n_slots, a.dst_n_slots = src_pool.shape[0], dst_pool.shape[0]
    a.src_pool, a.dst_pool = _ptr(src_pool), _ptr(dst_pool)
    a.src_slot, a.dst_slot, a.status = _ptr(src_slot), _ptr(dst_slot), _ptr(status)
    code = load_library().gdn_state_convert(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_state_convert", code)
    return dst_pool


def gdn_conv_store(cu_seqlens, q_raw, k_raw, v_raw, conv_pool, write_slot=None, *, H_qk, H_v,
                   read_slot=None, status=None, stream=None):
    """Store each prefilled sequence's last conv_k-1 raw inputs into
    conv_pool[write_slot[s]]; rows before a sequence's first token come from
    conv_pool[read_slot[s]] (zeros for -1 or None)."""
    a, keep = make_conv_args(q_raw, k_raw, v_raw, conv_pool, H_qk=H_qk, H_v=H_v,
                             read_slot=read_slot, write_slot=write_slot, cu_seqlens=cu_seqlens,
                             status=status)
    code = load_library().gdn_conv_store(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_conv_store", code)

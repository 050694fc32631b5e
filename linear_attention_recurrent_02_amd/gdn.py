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
F32, BF16 = 0, 1
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
                ("status", _P)]


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
                ("ckpt_per_seq", _I32), ("reserved1", _I32)]


class ConvArgs(ctypes.Structure):
    _fields_ = [("B", _I32), ("H_qk", _I32), ("H_v", _I32), ("d_k", _I32), ("d_v", _I32),
                ("act_dtype", _I32), ("conv_k", _I32), ("reserved0", _I32),
                ("n_slots", _I64), ("n_tokens", _I64), ("eps", ctypes.c_float),
                ("reserved1", _I32), ("q", _P), ("k", _P), ("v", _P), ("a_raw", _P),
                ("b_raw", _P), ("conv_wq", _P), ("conv_wk", _P), ("conv_wv", _P),
                ("conv_pool", _P), ("read_slot", _P), ("write_slot", _P), ("cu_seqlens", _P),
                ("q_out", _P), ("k_out", _P), ("v_out", _P), ("g_out", _P), ("beta_out", _P),
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
    lib.gdn_mixed.restype = _I32
    lib.gdn_mixed.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(PrefillArgs), _P]
    lib.gdn_conv_decode.restype = _I32
    lib.gdn_conv_decode.argtypes = [ctypes.POINTER(ConvArgs), _P]
    lib.gdn_conv_store.restype = _I32
    lib.gdn_conv_store.argtypes = [ctypes.POINTER(ConvArgs), _P]
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
            lib.gdn_sizeof_conv_args() != ctypes.sizeof(ConvArgs):
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
                     rule="gated_delta", scale=1.0, status=None):
    """Build a DecodeArgs struct.  q, k: [B, H_qk, d_k]; v: [B, H_v, d_v];
    g: [B, H_v] float32, or [B, H_v, d_k] for a per-key-channel decay; beta:
    [B, H_v] float32; state_pool: [n_slots, H_v, d_k, d_v];
    read_slot / write_slot: [B] int32 or None.  Returns (args, o, keepalive)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
                    ("state_pool", state_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("o", o), ("status", status)):
        _dev(t, name)
    B, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if o is None:
        o = torch.empty((B, H_v, d_v), dtype=q.dtype, device=q.device)
    a = DecodeArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = B, H_qk, H_v, d_k, d_v
    a.rule = _rule(rule)
    a.state_dtype = _dtype_code(state_pool)
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
               rule="gated_delta", scale=1.0, status=None, stream=None):
    """One decode token for B requests; updates ``state_pool`` in place and
    returns o [B, H_v, d_v] (dtype of q)."""
    a, o, keep = make_decode_args(q, k, v, g, beta, state_pool, read_slot, write_slot, o,
                                  rule=rule, scale=scale, status=status)
    code = load_library().gdn_decode(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_decode", code)
    return o


def make_prefill_args(cu_seqlens, q, k, v, state_pool, read_slot=None, write_slot=None, o=None, *,
                      H_qk, H_v, g=None, beta=None, a_raw=None, b_raw=None, conv_wq=None,
                      conv_wk=None, conv_wv=None, rule="gated_delta", scale=1.0, eps=1e-6,
                      chunk=64, workspace=None, status=None, ckpt_interval=0, ckpt_slot=None):
    """Build a PrefillArgs struct.  q, k: [N, H_qk*d_k] (or [N, H_qk, d_k]);
    v: [N, H_v*d_v]; with conv weights given the front-end runs (a_raw,
    b_raw are the gate logits), otherwise g, beta are used as given.  With
    ckpt_interval > 0 (a multiple of chunk), ckpt_slot [n_seq, per_seq] int32
    names the slots of the intermediate checkpoints.
    Returns (args, o, keepalive); allocates the workspace when needed."""
    for name, t in (("cu_seqlens", cu_seqlens), ("q", q), ("k", k), ("v", v),
                    ("state_pool", state_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("o", o), ("g", g), ("beta", beta),
                    ("a_raw", a_raw), ("b_raw", b_raw), ("conv_wq", conv_wq),
                    ("conv_wk", conv_wk), ("conv_wv", conv_wv), ("status", status),
                    ("ckpt_slot", ckpt_slot)):
        _dev(t, name)
    N = q.shape[0]
    d_k = q.numel() // max(1, N * H_qk) if N else state_pool.shape[2]
    d_v = v.numel() // max(1, N * H_v) if N else state_pool.shape[3]
    use_fe = conv_wq is not None
    if o is None:
        o = torch.empty((N, H_v, d_v), dtype=q.dtype, device=q.device)
    a = PrefillArgs()
    a.n_seq = cu_seqlens.shape[0] - 1
    a.H_qk, a.H_v, a.d_k, a.d_v = H_qk, H_v, d_k, d_v
    a.rule = _rule(rule)
    a.state_dtype = _dtype_code(state_pool)
    a.act_dtype = _dtype_code(q)
    a.use_frontend = 1 if use_fe else 0
    a.conv_k = conv_wq.shape[1] if use_fe else 4
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
    a.reserved1 = 0
    need = int(load_library().gdn_prefill_workspace_size(ctypes.byref(a)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    keep = (cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o, g, beta, a_raw, b_raw,
            conv_wq, conv_wk, conv_wv, workspace, status, ckpt_slot)
    return a, o, keep


def gdn_prefill(cu_seqlens, q, k, v, state_pool, read_slot=None, write_slot=None, o=None, *,
                stream=None, **kw):
    """Chunked prefill over packed sequences; returns o [N, H_v, d_v]."""
    a, o, keep = make_prefill_args(cu_seqlens, q, k, v, state_pool, read_slot, write_slot, o, **kw)
    code = load_library().gdn_prefill(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_prefill", code)
    return o


def gdn_frontend(cu_seqlens, q_raw, k_raw, v_raw, *, H_qk, H_v, conv_wq, conv_wk, conv_wv,
                 a_raw, b_raw, eps=1e-6, stream=None):
    """The front-end alone: returns (q [N,H_qk,d_k], k, v [N,H_v,d_v], g, beta)."""
    for name, t in (("cu_seqlens", cu_seqlens), ("q_raw", q_raw), ("k_raw", k_raw),
                    ("v_raw", v_raw), ("conv_wq", conv_wq), ("conv_wk", conv_wk),
                    ("conv_wv", conv_wv), ("a_raw", a_raw), ("b_raw", b_raw)):
        _dev(t, name)
    N = q_raw.shape[0]
    d_k = q_raw.numel() // max(1, N * H_qk)
    d_v = v_raw.numel() // max(1, N * H_v)
    a = PrefillArgs()
    a.n_seq = cu_seqlens.shape[0] - 1
    a.H_qk, a.H_v, a.d_k, a.d_v = H_qk, H_v, d_k, d_v
    a.rule = RULES["gated_delta"]
    a.state_dtype = F32
    a.act_dtype = _dtype_code(q_raw)
    a.use_frontend, a.conv_k, a.chunk, a.ckpt_interval = 1, conv_wq.shape[1], 64, 0
    a.n_tokens, a.n_slots = N, 0
    a.scale, a.eps = 1.0, float(eps)
    a.cu_seqlens, a.q, a.k, a.v = _ptr(cu_seqlens), _ptr(q_raw), _ptr(k_raw), _ptr(v_raw)
    a.a_raw, a.b_raw = _ptr(a_raw), _ptr(b_raw)
    a.conv_wq, a.conv_wk, a.conv_wv = _ptr(conv_wq), _ptr(conv_wk), _ptr(conv_wv)
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
    for name, t in (("q_raw", q_raw), ("k_raw", k_raw), ("v_raw", v_raw),
                    ("conv_pool", conv_pool), ("read_slot", read_slot),
                    ("write_slot", write_slot), ("cu_seqlens", cu_seqlens), ("a_raw", a_raw),
                    ("b_raw", b_raw), ("conv_wq", conv_wq), ("conv_wk", conv_wk),
                    ("conv_wv", conv_wv), ("status", status)):
        _dev(t, name)
    rows = q_raw.shape[0]
    B = rows if cu_seqlens is None else cu_seqlens.shape[0] - 1
    d_k = q_raw.shape[-1] // H_qk if q_raw.dim() == 2 else q_raw.shape[-1]
    d_v = v_raw.shape[-1] // H_v if v_raw.dim() == 2 else v_raw.shape[-1]
    a = ConvArgs()
    a.B, a.H_qk, a.H_v, a.d_k, a.d_v = B, H_qk, H_v, d_k, d_v
    a.act_dtype = _dtype_code(q_raw)
    a.conv_k = conv_pool.shape[1] + 1
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


def gdn_conv_store(cu_seqlens, q_raw, k_raw, v_raw, conv_pool, write_slot=None, *, H_qk, H_v,
                   status=None, stream=None):
    """Store each prefilled sequence's last conv_k-1 raw inputs into
    conv_pool[write_slot[s]]."""
    a, keep = make_conv_args(q_raw, k_raw, v_raw, conv_pool, H_qk=H_qk, H_v=H_v,
                             write_slot=write_slot, cu_seqlens=cu_seqlens, status=status)
    code = load_library().gdn_conv_store(ctypes.byref(a), _stream(stream))
    if code:
        raise GdnError("gdn_conv_store", code)

"""FP64 CPU oracle for the Gated DeltaNet recurrent-state path.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers; the GPU library and its
Python binding never import this package.  The arithmetic lives in
``oracle.c`` (plain C, double precision, token by token); this module only
marshals NumPy arrays into it.  See the header of ``oracle.c`` for the pages
and readings each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

RULES = {"linear": 0, "gated": 1, "delta": 2, "gated_delta": 3}


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_round_bf16.restype = f64
        lib.oracle_round_bf16.argtypes = [f64]
        lib.oracle_round_bf16_array.restype = None
        lib.oracle_round_bf16_array.argtypes = [P, P, i64]
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [i32, i32, i32, i32, i32, i64, i32, f64, i32,
                                      P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_sequences.restype = i32
        lib.oracle_sequences.argtypes = [i32, P, i32, i32, i32, i32, i64, i32, f64, i32,
                                         P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_frontend.restype = i32
        lib.oracle_frontend.argtypes = [i32, P, i32, i32, i32, i32, i32, f64,
                                        P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_decode_cw.restype = i32
        lib.oracle_decode_cw.argtypes = [i32, i32, i32, i32, i32, i64, i32, f64, i32,
                                         P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_conv_decode.restype = i32
        lib.oracle_conv_decode.argtypes = [i32, i32, i32, i32, i32, i32, f64, i64,
                                           P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_q8_encode.restype = i32
        lib.oracle_q8_encode.argtypes = [i64, i32, i32, i32, P, P, P, P]
        lib.oracle_decode_q8.restype = i32
        lib.oracle_decode_q8.argtypes = [i32, i32, i32, i32, i32, i64, i32, f64, i32,
                                         P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_decode_cw_q8.restype = i32
        lib.oracle_decode_cw_q8.argtypes = [i32, i32, i32, i32, i32, i64, i32, f64, i32,
                                            P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_sequences_cw.restype = i32
        lib.oracle_sequences_cw.argtypes = [i32, P, i32, i32, i32, i32, i64, i32, f64, i32,
                                            P, P, P, P, P, P, P, P, P, i32]
        lib.oracle_version.restype = i32
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rule(rule):
    return RULES[rule] if isinstance(rule, str) else int(rule)


def default_threads() -> int:
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def round_bf16(x):
    """Nearest BF16 value of each element (ties to even), as float64."""
    x = _f64(x)
    out = np.empty_like(x)
    _load().oracle_round_bf16_array(_p(x), _p(out), x.size)
    return out


def decode(q, k, v, g, beta, pool, read_slot=None, write_slot=None, *, rule="gated_delta",
           scale=1.0, round_state=False, n_threads=None):
    """One decode token for B requests.

    q, k: [B, Hqk, dk]; v: [B, Hv, dv]; g, beta: [B, Hv]; pool: [n_slots, Hv,
    dk, dv] (a float64 copy is updated and returned).  Returns
    ``(o [B, Hv, dv], pool_after, code)``; code 1 means a request was skipped
    because one of its slots was out of range.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((B, Hv, dv), np.float64)
    code = _load().oracle_decode(B, Hqk, Hv, dk, dv, pool.shape[0], _rule(rule), float(scale),
                                 int(bool(round_state)), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                 _p(pool), _p(rs), _p(ws), _p(o),
                                 n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o, pool, code


def decode_cw(q, k, v, g, beta, pool, read_slot=None, write_slot=None, *, rule="gated_delta",
              scale=1.0, round_state=False, n_threads=None):
    """One decode token for B requests with a per-key-channel decay.

    As ``decode`` except g is [B, Hv, dk] (the log-decay of each key channel;
    the Kimi Linear section's channel-wise gate).  Returns ``(o, pool_after,
    code)``.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if g.shape != (B, Hv, dk):
        raise ValueError("g must be [B, Hv, dk]")
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((B, Hv, dv), np.float64)
    code = _load().oracle_decode_cw(B, Hqk, Hv, dk, dv, pool.shape[0], _rule(rule), float(scale),
                                    int(bool(round_state)), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                    _p(pool), _p(rs), _p(ws), _p(o),
                                    n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_decode_cw rejected its arguments")
    return o, pool, code


def sequences(cu_seqlens, q, k, v, g, beta, pool, read_slot=None, write_slot=None, *,
              rule="gated_delta", scale=1.0, round_state=False, n_threads=None):
    """Token-by-token recurrence over variable-length sequences.

    cu_seqlens: [n_seq+1]; q, k: [N, Hqk, dk]; v: [N, Hv, dv]; g, beta:
    [N, Hv]; pool: [n_slots, Hv, dk, dv].  Returns ``(o, pool_after, code)``.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    cu = _i32(cu_seqlens)
    n_seq = cu.shape[0] - 1
    N, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((N, Hv, dv), np.float64)
    code = _load().oracle_sequences(n_seq, _p(cu), Hqk, Hv, dk, dv, pool.shape[0], _rule(rule),
                                    float(scale), int(bool(round_state)), _p(q), _p(k), _p(v),
                                    _p(g), _p(beta), _p(pool), _p(rs), _p(ws), _p(o),
                                    n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_sequences rejected its arguments")
    return o, pool, code


def sequences_cw(cu_seqlens, q, k, v, g, beta, pool, read_slot=None, write_slot=None, *,
                 rule="gated_delta", scale=1.0, round_state=False, n_threads=None):
    """``sequences`` with a per-key-channel decay: g is [N, Hv, dk] (Kimi Delta
    Attention's gate, the Kimi Linear section).  Returns ``(o, pool_after,
    code)``."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    cu = _i32(cu_seqlens)
    n_seq = cu.shape[0] - 1
    N, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if g.shape != (N, Hv, dk):
        raise ValueError("g must be [N, Hv, dk]")
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((N, Hv, dv), np.float64)
    code = _load().oracle_sequences_cw(n_seq, _p(cu), Hqk, Hv, dk, dv, pool.shape[0],
                                       _rule(rule), float(scale), int(bool(round_state)), _p(q),
                                       _p(k), _p(v), _p(g), _p(beta), _p(pool), _p(rs), _p(ws),
                                       _p(o), n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_sequences_cw rejected its arguments")
    return o, pool, code


def frontend(cu_seqlens, q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw, *, Hqk, Hv, eps=1e-6,
             conv_init=None):
    """Causal depthwise conv + SiLU, L2 norm of q/k per head, gates.

    q_raw, k_raw: [N, Hqk*dk]; v_raw: [N, Hv*dv]; w*: [channels, K];
    a_raw, b_raw: [N, Hv]; conv_init: None (empty windows) or
    [n_seq, K-1, 2*Hqk*dk + Hv*dv], the raw inputs of the K-1 tokens before
    each sequence (oldest first).  Returns (q, k, v, g, beta) with q, k as
    [N, Hqk, dk], v as [N, Hv, dv], g and beta as [N, Hv].
    """
    q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw = map(
        _f64, (q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw))
    cu = _i32(cu_seqlens)
    N = q_raw.shape[0]
    dk = q_raw.shape[1] // Hqk
    dv = v_raw.shape[1] // Hv
    K = wq.shape[1]
    C = 2 * Hqk * dk + Hv * dv
    init = None
    if conv_init is not None:
        init = _f64(conv_init)
        if init.shape != (cu.shape[0] - 1, K - 1, C):
            raise ValueError("conv_init must be [n_seq, K-1, 2*Hqk*dk + Hv*dv]")
    qo, ko, vo = np.zeros_like(q_raw), np.zeros_like(k_raw), np.zeros_like(v_raw)
    g = np.zeros((N, Hv), np.float64)
    beta = np.zeros((N, Hv), np.float64)
    code = _load().oracle_frontend(cu.shape[0] - 1, _p(cu), Hqk, Hv, dk, dv, K, float(eps),
                                   _p(q_raw), _p(k_raw), _p(v_raw), _p(wq), _p(wk), _p(wv),
                                   _p(a_raw), _p(b_raw), _p(init), _p(qo), _p(ko), _p(vo), _p(g),
                                   _p(beta))
    if code != 0:
        raise ValueError("oracle_frontend rejected its arguments")
    return qo.reshape(N, Hqk, dk), ko.reshape(N, Hqk, dk), vo.reshape(N, Hv, dv), g, beta


def conv_decode(q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw, conv_pool, read_slot=None,
                write_slot=None, *, Hqk, Hv, eps=1e-6):
    """One decode token of the front-end for B requests, conv window from slots.

    q_raw, k_raw: [B, Hqk*dk]; v_raw: [B, Hv*dv]; w*: [channels, K]; a_raw,
    b_raw: [B, Hv]; conv_pool: [n_slots, K-1, 2*Hqk*dk + Hv*dv] (a float64
    copy is updated and returned).  Returns ``(q, k, v, g, beta, pool_after,
    code)`` with q, k as [B, Hqk, dk] and v as [B, Hv, dv]; code 1 means a
    request was skipped for an out-of-range slot (its outputs stay 0).
    """
    q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw = map(
        _f64, (q_raw, k_raw, v_raw, wq, wk, wv, a_raw, b_raw))
    pool = _f64(conv_pool).copy()
    B = q_raw.shape[0]
    dk = q_raw.shape[1] // Hqk
    dv = v_raw.shape[1] // Hv
    K = wq.shape[1]
    if pool.ndim != 3 or pool.shape[1] != K - 1 or pool.shape[2] != 2 * Hqk * dk + Hv * dv:
        raise ValueError("conv_pool must be [n_slots, K-1, 2*Hqk*dk + Hv*dv]")
    rs, ws = _i32(read_slot), _i32(write_slot)
    qo, ko, vo = np.zeros_like(q_raw), np.zeros_like(k_raw), np.zeros_like(v_raw)
    g = np.zeros((B, Hv), np.float64)
    beta = np.zeros((B, Hv), np.float64)
    code = _load().oracle_conv_decode(B, Hqk, Hv, dk, dv, K, float(eps), pool.shape[0],
                                      _p(q_raw), _p(k_raw), _p(v_raw), _p(wq), _p(wk), _p(wv),
                                      _p(a_raw), _p(b_raw), _p(pool), _p(rs), _p(ws), _p(qo),
                                      _p(ko), _p(vo), _p(g), _p(beta))
    if code < 0:
        raise ValueError("oracle_conv_decode rejected its arguments")
    return (qo.reshape(B, Hqk, dk), ko.reshape(B, Hqk, dk), vo.reshape(B, Hv, dv), g, beta,
            pool, code)


def conv_tail(cu_seqlens, q_raw, k_raw, v_raw, K=4, conv_init=None):
    """The conv window each sequence leaves behind: its last K-1 raw inputs.

    Returns [n_seq, K-1, 2*Hqk*dk + Hv*dv] (q|k|v channels, oldest token
    first): the history a decode step or a resumed prefill of that sequence
    continues from.  Where a sequence has fewer than K-1 tokens the older
    rows are those of the window it started from (conv_init, as for
    ``frontend``), or zero without one.
    """
    q_raw, k_raw, v_raw = map(_f64, (q_raw, k_raw, v_raw))
    cu = _i32(cu_seqlens)
    rows = np.concatenate([q_raw, k_raw, v_raw], axis=1)
    out = np.zeros((cu.shape[0] - 1, K - 1, rows.shape[1]), np.float64)
    init = None if conv_init is None else _f64(conv_init)
    for s in range(cu.shape[0] - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        for j in range(K - 1):
            t = t1 - (K - 1) + j
            if t >= t0:
                out[s, j] = rows[t]
            elif init is not None:
                out[s, j] = init[s, t - t0 + K - 1]
    return out


# ----------------------------------------------------------------------------
# 8-bit state storage: the first n_hi key channels (rows) of every tile in
# BF16, the other rows INT8 with one binary32 scale each (oracle.c states the
# quantisation).  A stored tile is laid out as
#   [n_hi, dv] BF16 bits | [dk - n_hi, dv] int8 codes | [dk - n_hi] binary32 scales
# (little endian) followed by zero padding up to a multiple of 256 bytes, one
# tile per (slot, head).

Q8_TILE_ALIGN = 256


def q8_tile_bytes(dk: int, dv: int, n_hi: int) -> int:
    raw = n_hi * dv * 2 + (dk - n_hi) * dv + 4 * (dk - n_hi)
    return (raw + Q8_TILE_ALIGN - 1) // Q8_TILE_ALIGN * Q8_TILE_ALIGN


def q8_encode(values, n_hi: int):
    """Encode tiles [..., dk, dv] (float64 values).  Returns (bf16 rows as
    float64 [..., n_hi, dv], codes int8 [..., dk-n_hi, dv], scales float32
    [..., dk-n_hi])."""
    v = _f64(values)
    lead, (dk, dv) = v.shape[:-2], v.shape[-2:]
    n = int(np.prod(lead)) if lead else 1
    hi = np.zeros((n, n_hi, dv), np.float64)
    codes = np.zeros((n, dk - n_hi, dv), np.int8)
    scales = np.zeros((n, dk - n_hi), np.float32)
    code = _load().oracle_q8_encode(n, dk, dv, n_hi, _p(v), _p(hi), _p(codes), _p(scales))
    if code != 0:
        raise ValueError("oracle_q8_encode rejected its arguments")
    return (hi.reshape(*lead, n_hi, dv), codes.reshape(*lead, dk - n_hi, dv),
            scales.reshape(*lead, dk - n_hi))


def q8_pack(values, n_hi: int) -> np.ndarray:
    """Tiles [..., dk, dv] of float64 values -> their stored bytes [...,
    q8_tile_bytes] (uint8)."""
    v = _f64(values)
    dk, dv = v.shape[-2:]
    hi, codes, scales = q8_encode(v, n_hi)
    lead = v.shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    bits = (hi.reshape(n, -1).astype(np.float32).view(np.uint32) >> 16).astype("<u2")
    body = [bits.view(np.uint8).reshape(n, -1), codes.reshape(n, -1).view(np.uint8),
            scales.reshape(n, -1).astype("<f4").view(np.uint8).reshape(n, -1)]
    used = sum(b.shape[1] for b in body)
    pad = np.zeros((n, q8_tile_bytes(dk, dv, n_hi) - used), np.uint8)
    out = np.concatenate(body + [pad], axis=1)
    return out.reshape(*lead, out.shape[1])


def q8_unpack(raw, dk: int, dv: int, n_hi: int) -> np.ndarray:
    """Stored bytes [..., q8_tile_bytes] -> the float64 values they represent
    [..., dk, dv]: a BF16 row widened, an INT8 row as code * scale in
    binary32."""
    raw = np.ascontiguousarray(np.asarray(raw, np.uint8))
    tb = q8_tile_bytes(dk, dv, n_hi)
    lead = raw.shape[:-1]
    assert raw.shape[-1] == tb, (raw.shape, tb)
    n = int(np.prod(lead)) if lead else 1
    r = raw.reshape(n, tb)
    a, b = n_hi * dv * 2, n_hi * dv * 2 + (dk - n_hi) * dv
    c = b + 4 * (dk - n_hi)
    hi = (r[:, :a].copy().view("<u2").astype(np.uint32) << 16).view(np.float32)
    codes = r[:, a:b].copy().view(np.int8).astype(np.float32).reshape(n, dk - n_hi, dv)
    scales = r[:, b:c].copy().view("<f4").reshape(n, dk - n_hi, 1)
    lo = (codes * scales).astype(np.float32)
    out = np.concatenate([hi.reshape(n, n_hi, dv), lo], axis=1).astype(np.float64)
    return out.reshape(*lead, dk, dv)


def decode_q8(q, k, v, g, beta, pool, read_slot=None, write_slot=None, *, n_hi,
              rule="gated_delta", scale=1.0, n_threads=None):
    """One decode token for B requests on a pool kept in the 8-bit format.

    pool: [n_slots, Hv, dk, dv] of the values the stored tiles represent (e.g.
    q8_unpack of the stored bytes); a copy is updated with the new states as
    stored (quantised) and returned.  Returns ``(o, pool_after, code)``.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((B, Hv, dv), np.float64)
    code = _load().oracle_decode_q8(B, Hqk, Hv, dk, dv, pool.shape[0], _rule(rule),
                                    float(scale), int(n_hi), _p(q), _p(k), _p(v), _p(g),
                                    _p(beta), _p(pool), _p(rs), _p(ws), _p(o),
                                    n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_decode_q8 rejected its arguments")
    return o, pool, code


def decode_cw_q8(q, k, v, g, beta, pool, read_slot=None, write_slot=None, *, n_hi,
                 rule="gated_delta", scale=1.0, n_threads=None):
    """``decode_cw`` (g of shape [B, Hv, dk]) with the state stored in the
    8-bit format; pool as for ``decode_q8``.  Returns ``(o, pool_after, code)``."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    pool = _f64(pool).copy()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if g.shape != (B, Hv, dk):
        raise ValueError("g must be [B, Hv, dk]")
    rs, ws = _i32(read_slot), _i32(write_slot)
    o = np.zeros((B, Hv, dv), np.float64)
    code = _load().oracle_decode_cw_q8(B, Hqk, Hv, dk, dv, pool.shape[0], _rule(rule),
                                       float(scale), int(n_hi), _p(q), _p(k), _p(v), _p(g),
                                       _p(beta), _p(pool), _p(rs), _p(ws), _p(o),
                                       n_threads or default_threads())
    if code < 0:
        raise ValueError("oracle_decode_cw_q8 rejected its arguments")
    return o, pool, code

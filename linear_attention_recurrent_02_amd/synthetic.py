"""Seeded synthetic inputs for the Gated DeltaNet decode / prefill workloads.

This module only draws random numbers and shapes their distributions; it
holds none of the recurrence's arithmetic.  Both the GPU path and the CPU
oracle consume the tensors made here: values are drawn in float64 with
``numpy.random.default_rng([workload, layer, stream])`` and cast once to the
dtype the GPU receives, and that cast tensor is the shared input (the oracle
widens it back to float64).  Large state pools can instead be drawn directly
on the device with a seeded torch generator (``state_on_device=True``); the
oracle then reads back the same device tensor.

Distributions (the workload descriptions of the task):
  q, k   ~ N(0, 1), then scaled to unit L2 norm per (token, head) in float64
  v      ~ N(0, 1)
  beta   = sigmoid(N(0, 1))          (write strength)
  g      = -softplus(N(0, 1))        (log of the decay a = exp(g))
  channel-wise g = -softplus(N(0, 1) + b), b ~ U(-5, 1) fixed per (head,
           key channel): one head's channels forget at different rates
  state  ~ N(0, 0.02^2)  (0.02 is the standard deviation)
  raw q/k/v for the front-end ~ N(0, 1); conv weights ~ N(0, 0.5^2);
  a_raw, b_raw ~ N(0, 1)
"""
from __future__ import annotations

import numpy as np
import torch

# stream ids keep independent draws independent
(_S_Q, _S_K, _S_V, _S_G, _S_B, _S_STATE, _S_SLOTS, _S_LEN, _S_W, _S_RAW, _S_CONV, _S_GC,
 _S_GCB) = range(13)

WORKLOADS = {
    # tiny FP32 recurrence: B=1, H=2, d=16, T=32, zero initial state
    "tiny_fp32": dict(index=0, B=1, H_qk=2, H_v=2, d_k=16, d_v=16, T=32),
    # one decode step, BF16 state, 64 live slots of a 256-slot pool
    "decode_b64": dict(index=1, B=64, H_qk=16, H_v=32, d_k=128, d_v=128, n_slots=256),
    # decode at batch 512, 48 layers back to back, one 512-slot pool per layer
    "decode_b512_x48": dict(index=2, B=512, H_qk=16, H_v=32, d_k=128, d_v=128, n_slots=512,
                            layers=48),
    # chunked prefill with the conv front-end, 8 ragged sequences of 1024..8192
    "prefill_varlen": dict(index=3, n_seq=8, H_qk=16, H_v=32, d_k=128, d_v=128, n_slots=64,
                           min_len=1024, max_len=8192, conv_k=4, chunk=64),
    # mixed: 448 decode requests + 4 prefills of 8192 tokens, 1024-slot pool
    "mixed": dict(index=4, n_decode=448, n_prefill=4, prefill_len=8192, H_qk=16, H_v=32,
                  d_k=128, d_v=128, n_slots=1024, conv_k=4),
}


def rng(workload: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(workload), int(layer), int(stream)])


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _neg_softplus(x):
    return -(np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))))


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)


def _device_gen(wl: int, layer: int, stream: int) -> torch.Generator:
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1_000_003 * (int(wl) + 1) + 7919 * int(layer) + 101 * int(stream) + 17)
    return gen


def token_inputs(wl: int, layer: int, n_tok: int, H_qk: int, H_v: int, d_k: int, d_v: int,
                 act_dtype: torch.dtype = torch.bfloat16, on_device: bool = False):
    """Per-token q, k (unit norm), v, g, beta for ``n_tok`` tokens (CPU tensors).

    q, k: [n_tok, H_qk, d_k] act_dtype; v: [n_tok, H_v, d_v] act_dtype;
    g, beta: [n_tok, H_v] float32.  ``on_device`` draws the same
    distributions on the current CUDA device in float32 with seeded torch
    generators (for benchmark-sized batches; other values than the host draw).
    """
    if on_device:
        def normal(stream, shape):
            return torch.randn(shape, generator=_device_gen(wl, layer, stream), device="cuda")
        q = normal(_S_Q, (n_tok, H_qk, d_k))
        k = normal(_S_K, (n_tok, H_qk, d_k))
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
        v = normal(_S_V, (n_tok, H_v, d_v))
        g = -torch.nn.functional.softplus(normal(_S_G, (n_tok, H_v)))
        beta = torch.sigmoid(normal(_S_B, (n_tok, H_v)))
        return q.to(act_dtype), k.to(act_dtype), v.to(act_dtype), g, beta
    q = _unit_rows(rng(wl, layer, _S_Q).standard_normal((n_tok, H_qk, d_k)))
    k = _unit_rows(rng(wl, layer, _S_K).standard_normal((n_tok, H_qk, d_k)))
    v = rng(wl, layer, _S_V).standard_normal((n_tok, H_v, d_v))
    g = _neg_softplus(rng(wl, layer, _S_G).standard_normal((n_tok, H_v)))
    beta = _sigmoid(rng(wl, layer, _S_B).standard_normal((n_tok, H_v)))
    return (_cast(q, act_dtype), _cast(k, act_dtype), _cast(v, act_dtype),
            _cast(g, torch.float32), _cast(beta, torch.float32))


def channel_gates(wl: int, layer: int, n_tok: int, H_v: int, d_k: int, lo: float = -5.0,
                  hi: float = 1.0, on_device: bool = False) -> torch.Tensor:
    """Per-key-channel log-decays g [n_tok, H_v, d_k] float32 (Kimi Delta
    Attention's channel-wise gate): -softplus(x + b) with x ~ N(0, 1) per
    (token, head, channel) and a bias b ~ U(lo, hi) fixed per (head, channel),
    so the mean decay per token ranges from about e^-0.01 to e^-1.3 across
    one head's channels.  ``on_device``: drawn on the current CUDA device."""
    if on_device:
        b = torch.rand((1, H_v, d_k), generator=_device_gen(wl, layer, _S_GCB),
                       device="cuda") * (hi - lo) + lo
        x = torch.randn((n_tok, H_v, d_k), generator=_device_gen(wl, layer, _S_GC), device="cuda")
        return -torch.nn.functional.softplus(x + b)
    b = rng(wl, layer, _S_GCB).uniform(lo, hi, size=(1, H_v, d_k))
    x = rng(wl, layer, _S_GC).standard_normal((n_tok, H_v, d_k))
    return _cast(_neg_softplus(x + b), torch.float32)


def state_pool(wl: int, layer: int, n_slots: int, H_v: int, d_k: int, d_v: int,
               state_dtype: torch.dtype = torch.bfloat16, std: float = 0.02,
               on_device: bool = False) -> torch.Tensor:
    """Pool [n_slots, H_v, d_k, d_v] ~ N(0, std^2).

    With ``on_device`` the draw is made on the current CUDA device with a
    torch generator seeded from (workload, layer) -- for multi-GiB pools where
    a float64 host draw would be too slow; otherwise a float64 NumPy draw.
    """
    shape = (n_slots, H_v, d_k, d_v)
    if std == 0.0:
        t = torch.zeros(shape, dtype=state_dtype)
        return t.cuda() if on_device else t
    if on_device:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1_000_003 * (int(wl) + 1) + 7919 * int(layer) + 17)
        out = torch.empty(shape, dtype=state_dtype, device="cuda")
        flat = out.view(-1)
        step = 1 << 26  # float32 temporary of at most 256 MiB
        for s in range(0, flat.numel(), step):
            e = min(flat.numel(), s + step)
            flat[s:e] = (torch.randn(e - s, generator=gen, device="cuda", dtype=torch.float32)
                         * std).to(state_dtype)
        return out
    a = rng(wl, layer, _S_STATE).standard_normal(shape) * std
    return _cast(a, state_dtype)


def state_pool_q8_bytes(wl: int, layer: int, n_slots: int, H_v: int, d_k: int, d_v: int,
                        n_hi: int, std: float = 0.02) -> torch.Tensor:
    """A stored pool in the 8-bit state layout, drawn on the current CUDA device
    (uint8 [n_slots, H_v, tile bytes], tile = [n_hi, d_v] BF16 | [d_k - n_hi,
    d_v] int8 | [d_k - n_hi] float32 | zero padding to 256 bytes): BF16 rows ~ N(0, std^2), codes drawn as
    integers spread over [-127, 127] (N(0, 36^2) rounded and clipped) and every
    scale 3.5 std / 127, i.e. random states of the scale of ``state_pool``.
    Benchmark-sized pools; tests encode their pools with the oracle instead."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3_000_017 * (int(wl) + 1) + 7901 * int(layer) + 41)
    lo = d_k - n_hi
    used = n_hi * d_v * 2 + lo * d_v + 4 * lo
    tile = (used + 255) // 256 * 256  # tiles are padded to 256-byte lines
    out = torch.zeros((n_slots, H_v, tile), dtype=torch.uint8, device="cuda")
    step = max(1, (1 << 22) // max(1, H_v * d_k * d_v))  # slots per chunk of the draw
    for s in range(0, n_slots, step):
        e = min(n_slots, s + step)
        n = (e - s) * H_v
        hi = (torch.randn((n, n_hi * d_v), generator=gen, device="cuda") * std).to(torch.bfloat16)
        codes = torch.randn((n, lo * d_v), generator=gen, device="cuda").mul_(36.0).round_()
        codes = codes.clamp_(-127, 127).to(torch.int8)
        scales = torch.full((n, lo), 3.5 * std / 127.0, dtype=torch.float32, device="cuda")
        out[s:e, :, :used] = torch.cat([hi.view(torch.uint8), codes.view(torch.uint8),
                                        scales.view(torch.uint8)], dim=1).view(e - s, H_v, used)
    return out


def distinct_slots(wl: int, layer: int, n_slots: int, B: int, in_place: bool):
    """Read / write slot indices (int32).

    in_place: read = write = the first B entries of a seeded permutation.
    Otherwise read = perm[:B] and write = perm[B:2B] (distinct, no overlap).
    """
    perm = rng(wl, layer, _S_SLOTS).permutation(n_slots).astype(np.int32)
    if in_place:
        r = perm[:B].copy()
        return torch.from_numpy(r), torch.from_numpy(r.copy())
    if 2 * B > n_slots:
        raise ValueError("need 2*B <= n_slots for distinct read and write slots")
    return torch.from_numpy(perm[:B].copy()), torch.from_numpy(perm[B:2 * B].copy())


def seq_lengths(wl: int, layer: int, n_seq: int, lo: int, hi: int) -> np.ndarray:
    """Ragged lengths drawn uniformly from [lo, hi] (inclusive)."""
    return rng(wl, layer, _S_LEN).integers(lo, hi + 1, size=n_seq).astype(np.int64)


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    return torch.from_numpy(cu.astype(np.int32))


def frontend_inputs(wl: int, layer: int, n_tok: int, H_qk: int, H_v: int, d_k: int, d_v: int,
                    conv_k: int = 4, act_dtype: torch.dtype = torch.bfloat16):
    """Raw q, k [n_tok, H_qk*d_k], v [n_tok, H_v*d_v] (act_dtype); conv weights
    [channels, conv_k] float32 ~ N(0, 0.25); a_raw, b_raw [n_tok, H_v] float32."""
    r = rng(wl, layer, _S_RAW)
    q = r.standard_normal((n_tok, H_qk * d_k))
    k = r.standard_normal((n_tok, H_qk * d_k))
    v = r.standard_normal((n_tok, H_v * d_v))
    w = rng(wl, layer, _S_W)
    wq = w.standard_normal((H_qk * d_k, conv_k)) * 0.5
    wk = w.standard_normal((H_qk * d_k, conv_k)) * 0.5
    wv = w.standard_normal((H_v * d_v, conv_k)) * 0.5
    a_raw = rng(wl, layer, _S_G).standard_normal((n_tok, H_v))
    b_raw = rng(wl, layer, _S_B).standard_normal((n_tok, H_v))
    f32 = torch.float32
    return dict(q_raw=_cast(q, act_dtype), k_raw=_cast(k, act_dtype), v_raw=_cast(v, act_dtype),
                conv_wq=_cast(wq, f32), conv_wk=_cast(wk, f32), conv_wv=_cast(wv, f32),
                a_raw=_cast(a_raw, f32), b_raw=_cast(b_raw, f32))


def conv_pool(wl: int, layer: int, n_slots: int, channels: int, conv_k: int = 4,
              act_dtype: torch.dtype = torch.bfloat16, on_device: bool = False) -> torch.Tensor:
    """A conv-state pool [n_slots, conv_k-1, channels] of raw inputs ~ N(0, 1)
    in act_dtype: earlier tokens' raw q|k|v rows, as a decode step finds them.
    ``on_device`` draws on the current CUDA device with a seeded torch
    generator (for benchmark-sized pools); otherwise a float64 NumPy draw."""
    shape = (n_slots, conv_k - 1, channels)
    if on_device:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(2_000_029 * (int(wl) + 1) + 7907 * int(layer) + 29)
        return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(act_dtype)
    a = rng(wl, layer, _S_CONV).standard_normal(shape)
    return _cast(a, act_dtype)


def mixed_slots(wl: int, n_decode: int, n_prefill: int, n_slots: int, frac: float = 0.25):
    """Slots for a mixed batch sharing one pool: every request writes a distinct
    slot; a seeded `frac` of all requests read a prefix-cache checkpoint slot
    (distinct from every write slot); the other decode requests update in
    place and the other prefills start fresh (read -1).  Returns int32 tensors
    (dec_read, dec_write, pre_read, pre_write)."""
    n = n_decode + n_prefill
    r = rng(wl, 0, _S_SLOTS)
    perm = r.permutation(n_slots).astype(np.int32)
    n_ckpt = int(round(frac * n))
    if n + n_ckpt > n_slots:
        raise ValueError("pool too small for distinct write and checkpoint slots")
    write = perm[:n].copy()
    ckpt_req = np.sort(r.choice(n, size=n_ckpt, replace=False))
    read = np.concatenate([write[:n_decode], np.full(n_prefill, -1, np.int32)])
    read[ckpt_req] = perm[n:n + n_ckpt]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    return t(read[:n_decode]), t(write[:n_decode]), t(read[n_decode:]), t(write[n_decode:])

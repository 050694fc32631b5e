"""Decode on a state pool in the 8-bit format (a BF16 head of key channels,
INT8 rows with one scale each; DAMP's mixed precision, "Seven Architectures
Replacing KV Cache With Bounded Mutable State", ONNX LinearAttention /
FlashInfer section): the HIP kernel through the C ABI against the oracle's
decode on the same stored pool.

Tolerance: the oracle stores its FP64 state in the same format, taking the
code decision in binary32 as the kernel does; the kernel's FP32 state can sit
on the other side of a rounding point, so a code may differ by one step,
rowmax / 127 < 7.9e-3 of the row's (and so the tile's) largest magnitude.
With FP32 arithmetic on top that is inside the BF16-storage bar, 2e-2 scaled
per (slot, head) tile, which is the bar used here for states and outputs."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import gdn_decode, gdn_state_q8_bytes, synthetic as syn
from gpu_util import f64, say, scaled_err, tol

pytestmark = pytest.mark.gpu
RULES = ["linear", "gated", "delta", "gated_delta"]
DEV = "cuda"
BAR = 2e-2


def q8_pool(seed, n_slots, Hv, dk, dv, n_hi, std=0.02):
    """A stored pool (uint8 [n_slots, Hv, tile bytes]) and the values it holds."""
    vals = np.random.default_rng(seed).standard_normal((n_slots, Hv, dk, dv)) * std
    raw = oracle.q8_pack(vals, n_hi)
    return torch.from_numpy(raw), oracle.q8_unpack(raw, dk, dv, n_hi)


def run(wl, B, Hqk, Hv, dk, dv, n_slots, n_hi, adt, rule="gated_delta", in_place=False,
        std=0.02, rs=None, ws=None, scale=1.0, gcw=None):
    q, k, v, g, beta = syn.token_inputs(wl, 0, B, Hqk, Hv, dk, dv, adt)
    raw, vals = q8_pool(wl, n_slots, Hv, dk, dv, n_hi, std)
    if rs is None:
        rs, ws = syn.distinct_slots(wl, 0, n_slots, B, in_place)
    gg = g if gcw is None else gcw
    dpool = raw.to(DEV)
    o = gdn_decode(q.to(DEV), k.to(DEV), v.to(DEV), gg.to(DEV), beta.to(DEV), dpool, rs.to(DEV),
                   ws.to(DEV), rule=rule, scale=scale, state_bf16_rows=n_hi)
    torch.cuda.synchronize()
    fn = oracle.decode_q8 if gcw is None else oracle.decode_cw_q8
    ro, rvals, code = fn(f64(q), f64(k), f64(v), f64(gg), f64(beta), vals, rs.numpy(), ws.numpy(),
                         n_hi=n_hi, rule=rule, scale=scale)
    return dict(o=o, ro=ro, raw=raw, dpool=dpool.cpu(), rvals=rvals, rs=rs, ws=ws, code=code)


def got_vals(r, dk, dv, n_hi):
    return oracle.q8_unpack(r["dpool"].numpy(), dk, dv, n_hi)


@pytest.mark.parametrize("rule", RULES)
def test_q8_decode_b64(rule):
    """B = 64, H_qk = 16, H_v = 32, d = 128, 32 BF16 rows of 128 (10.25 bits per
    value), 64 live slots of a 256-slot pool, distinct read and write slots."""
    say("q8 decode b64", rule)
    r = run(61, 64, 16, 32, 128, 128, 256, 32, torch.bfloat16, rule=rule)
    assert r["code"] == 0
    w = r["ws"].numpy()
    assert scaled_err(f64(r["o"]), r["ro"], 2) < BAR
    assert scaled_err(got_vals(r, 128, 128, 32)[w], r["rvals"][w], 2) < BAR
    others = np.setdiff1d(np.arange(256), w)
    assert torch.equal(r["dpool"][others], r["raw"][others])  # bytes of unwritten slots


# BF16 heads in steps of gdn_state_q8_row_quantum: 16 at (16, 16), 8 at
# (32, 64) and (16, 128), 16 at (64, 32) and (64, 64), 32 at d_k = 128
@pytest.mark.parametrize("dk,dv,n_hi", [(16, 16, 16), (16, 16, 0), (32, 64, 8), (64, 32, 16),
                                        (128, 16, 32), (16, 128, 8), (64, 64, 48),
                                        (128, 128, 0), (128, 64, 96)])
@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float32])
def test_q8_decode_shapes(dk, dv, n_hi, adt):
    say("q8 decode shapes", dk, dv, n_hi, adt)
    r = run(62, 5, 2, 4, dk, dv, 12, n_hi, adt, std=0.3, scale=0.5)
    w = r["ws"].numpy()
    assert scaled_err(f64(r["o"]), r["ro"], 2) < max(tol(adt), BAR)
    assert scaled_err(got_vals(r, dk, dv, n_hi)[w], r["rvals"][w], 2) < BAR


def test_q8_slot_rules_and_bad_slot():
    """Read -1 = zero state, write -1 = nothing stored, an out-of-range slot
    skips its request (status bit) and leaves every byte of the pool alone."""
    say("q8 decode slot rules")
    B, Hqk, Hv, d, n_hi = 5, 1, 2, 64, 16
    rs = torch.tensor([-1, 2, 3, 9, 0], dtype=torch.int32)
    ws = torch.tensor([4, -1, 5, 6, 7], dtype=torch.int32)
    r = run(63, B, Hqk, Hv, d, d, 8, n_hi, torch.bfloat16, rs=rs, ws=ws, std=0.3)
    # request 3 reads slot 9 of 8: skipped
    assert r["code"] == 1
    keep = [0, 1, 2, 4]
    assert scaled_err(f64(r["o"])[keep], r["ro"][keep], 2) < BAR
    for s in (4, 5, 7):
        assert scaled_err(got_vals(r, d, d, n_hi)[s:s + 1], r["rvals"][s:s + 1], 2) < BAR
    for s in (0, 1, 2, 3, 6):  # read-only, skipped-write and untouched slots
        assert torch.equal(r["dpool"][s], r["raw"][s])


def test_q8_in_place_equals_out_of_place_and_frozen_state():
    say("q8 decode in place / frozen")
    B, Hqk, Hv, d, n_hi = 16, 2, 4, 128, 32
    q, k, v, g, beta = syn.token_inputs(64, 0, B, Hqk, Hv, d, d)
    raw, vals = q8_pool(64, 40, Hv, d, d, n_hi)
    rs, ws = syn.distinct_slots(64, 0, 40, B, in_place=False)
    args = [t.to(DEV) for t in (q, k, v, g, beta)]
    p1, p2 = raw.to(DEV), raw.to(DEV)
    o1 = gdn_decode(*args, p1, rs.to(DEV), ws.to(DEV), state_bf16_rows=n_hi)
    o2 = gdn_decode(*args, p2, rs.to(DEV), rs.to(DEV), state_bf16_rows=n_hi)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(p1.cpu()[ws.long()], p2.cpu()[rs.long()])
    # a = 1, beta = 0: the stored tile is the read tile requantised: the same
    # BF16 rows and codes, each scale within one binary32 step of the old one
    g0, b0 = torch.zeros_like(g).to(DEV), torch.zeros_like(beta).to(DEV)
    p3 = raw.to(DEV)
    gdn_decode(args[0], args[1], args[2], g0, b0, p3, rs.to(DEV), ws.to(DEV),
               state_bf16_rows=n_hi)
    torch.cuda.synchronize()
    got, want = p3.cpu()[ws.long()].numpy(), raw[rs.long()].numpy()
    sb = n_hi * d * 2 + (d - n_hi) * d  # bytes before the scales
    assert np.array_equal(got[..., :sb], want[..., :sb])
    s_got = got[..., sb:].copy().view("<f4")
    s_want = want[..., sb:].copy().view("<f4")
    assert np.all(np.abs(s_got.view(np.int32) - s_want.view(np.int32)) <= 1)


def test_q8_steps_accumulate():
    """Eight decode tokens in place on one 8-bit pool (each stores and reloads
    the quantised state) against the oracle stepping the same way."""
    say("q8 decode 8 steps")
    B, Hqk, Hv, d, n_hi, T = 16, 2, 4, 128, 32, 8
    raw, vals = q8_pool(65, B, Hv, d, d, n_hi, std=0.05)
    own = torch.arange(B, dtype=torch.int32)
    dpool = raw.to(DEV)
    outs = []
    for t in range(T):
        q, k, v, g, beta = syn.token_inputs(65, t, B, Hqk, Hv, d, d)
        outs.append(gdn_decode(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), beta.to(DEV), dpool,
                               own.to(DEV), own.to(DEV), state_bf16_rows=n_hi))
        ro, vals, _ = oracle.decode_q8(f64(q), f64(k), f64(v), f64(g), f64(beta), vals,
                                       own.numpy(), own.numpy(), n_hi=n_hi)
        torch.cuda.synchronize()
        assert scaled_err(f64(outs[-1]), ro, 2) < BAR, t
    got = oracle.q8_unpack(dpool.cpu().numpy(), d, d, n_hi)
    assert scaled_err(got, vals, 2) < BAR


def test_q8_channel_decay():
    """The per-key-channel decay (g [B, H_v, d_k]) on an 8-bit pool."""
    say("q8 decode channel decay")
    B, Hqk, Hv, d, n_hi = 8, 2, 4, 128, 32
    gen = torch.Generator().manual_seed(66)
    gcw = -torch.nn.functional.softplus(torch.randn((B, Hv, d), generator=gen))
    for rule in ("gated", "gated_delta"):
        r = run(66, B, Hqk, Hv, d, d, 20, n_hi, torch.bfloat16, rule=rule, gcw=gcw)
        w = r["ws"].numpy()
        assert scaled_err(f64(r["o"]), r["ro"], 2) < BAR, rule
        assert scaled_err(got_vals(r, d, d, n_hi)[w], r["rvals"][w], 2) < BAR, rule


def test_q8_decode_b512_full_size():
    """Batch 512 at the benchmark's shapes with 32 BF16 rows per 128 (one layer:
    a 512-slot 8-bit pool, in place), every request against the oracle."""
    say("q8 decode b512")
    B, Hqk, Hv, d, n, n_hi = 512, 16, 32, 128, 512, 32
    assert gdn_state_q8_bytes(Hv, d, d, n_hi) == Hv * oracle.q8_tile_bytes(d, d, n_hi)
    r = run(67, B, Hqk, Hv, d, d, n, n_hi, torch.bfloat16, in_place=True)
    w = r["ws"].numpy()
    assert scaled_err(f64(r["o"]), r["ro"], 2) < BAR
    assert scaled_err(got_vals(r, d, d, n_hi)[w], r["rvals"][w], 2) < BAR

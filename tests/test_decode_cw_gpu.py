"""Decode with a per-key-channel decay (Kimi Delta Attention, the Kimi Linear
section of "Seven Architectures Replacing KV Cache With Bounded Mutable
State"): the HIP decode kernel's channel-wise instance (g of shape [B, H_v,
d_k]) against the FP64 oracle on the same seeded inputs.  Outputs are
compared per (request, head) slice and states per (slot, head) tile, as for
the scalar decay."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import gdn_decode, synthetic as syn
from gpu_util import f64, say, scaled_err, tol

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cw_gates(wl, B, Hv, dk):
    """Per-channel log-decays: -softplus(N(0,1)) per (request, head, key channel)."""
    r = np.random.default_rng([wl, 77])
    a = r.standard_normal((B, Hv, dk))
    return torch.from_numpy(-(np.maximum(a, 0) + np.log1p(np.exp(-np.abs(a)))).astype(np.float32))


def run_cw(wl, B, Hqk, Hv, dk, dv, n_slots, sdt, adt, rule, fresh_every=0, in_place=False):
    q, k, v, _, beta = syn.token_inputs(wl, 0, B, Hqk, Hv, dk, dv, adt)
    g = cw_gates(wl, B, Hv, dk)
    pool = syn.state_pool(wl, 0, n_slots, Hv, dk, dv, sdt)
    rs, ws = syn.distinct_slots(wl, 0, n_slots, B, in_place)
    if fresh_every:
        rs[::fresh_every] = -1
    dpool = pool.to(DEV)
    o = gdn_decode(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), beta.to(DEV), dpool, rs.to(DEV),
                   ws.to(DEV), rule=rule, scale=0.5)
    torch.cuda.synchronize()
    ro, rpool, code = oracle.decode_cw(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(pool),
                                       rs.numpy(), ws.numpy(), rule=rule, scale=0.5,
                                       round_state=(sdt == torch.bfloat16))
    assert code == 0
    t = tol(sdt, adt)
    assert scaled_err(f64(o), ro, 2) < t
    w = ws.numpy()
    assert scaled_err(f64(dpool.cpu())[w], rpool[w], 2) < t
    others = np.setdiff1d(np.arange(n_slots), w)
    assert torch.equal(dpool.cpu()[others], pool[others])


@pytest.mark.parametrize("rule", ["gated", "gated_delta", "delta"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 16), (16, 64), (32, 32)])
def test_decode_cw_bf16(rule, dk, dv):
    say("decode cw bf16", rule, dk, dv)
    run_cw(501, 37, 2, 4, dk, dv, 80, torch.bfloat16, torch.bfloat16, rule, fresh_every=5)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (16, 128)])
def test_decode_cw_fp32(dk, dv):
    say("decode cw fp32", dk, dv)
    run_cw(502, 19, 1, 2, dk, dv, 40, torch.float32, torch.float32, "gated_delta")


def test_decode_cw_in_place_full_size():
    """B = 512, H_qk = 16, H_v = 32, d = 128, BF16 state updated in place: the
    decode workload's shape with a per-channel decay."""
    say("decode cw full size B=512")
    run_cw(503, 512, 16, 32, 128, 128, 512, torch.bfloat16, torch.bfloat16, "gated_delta",
           in_place=True)


def test_mixed_decode_half_with_channel_decay_equals_gdn_decode():
    """gdn_mixed with a channel-wise decode half and an empty prefill half
    runs gdn_decode's channel-wise tiles: the same outputs and state, bit
    for bit."""
    from linear_attention_recurrent_02_amd import gdn as B
    q, k, v, _, beta = syn.token_inputs(504, 0, 2, 1, 1, 16, 16, torch.bfloat16)
    g = cw_gates(504, 2, 1, 16)
    pool0 = syn.state_pool(504, 0, 4, 1, 16, 16, torch.bfloat16, std=0.3)
    p1, p2 = pool0.to(DEV), pool0.to(DEV)
    args = [t.to(DEV) for t in (q, k, v, g, beta)]
    da, o1, dkeep = B.make_decode_args(*args, p1)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    e = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    pa, _, pkeep = B.make_prefill_args(cu, e, e, e, p1, H_qk=1, H_v=1,
                                       g=torch.zeros((0, 1), device=DEV),
                                       beta=torch.zeros((0, 1), device=DEV))
    assert da.decay_mode == B.DECAY_CHANNEL
    B.gdn_mixed(da, pa)
    o2 = gdn_decode(*args, p2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1.view(torch.int16), p2.view(torch.int16))

"""Decode parity: the HIP decode kernel (through the C ABI) against the FP64
oracle on the same seeded inputs, plus slot bit-exactness and edge cases."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import gdn_decode, synthetic as syn
from gpu_util import f64, say, scaled_err, state_tol, tol

pytestmark = pytest.mark.gpu
RULES = ["linear", "gated", "delta", "gated_delta"]
DEV = "cuda"


def make_case(wl, B, Hqk, Hv, dk, dv, n_slots, sdt, adt, std=0.02, in_place=False, layer=0):
    q, k, v, g, beta = syn.token_inputs(wl, layer, B, Hqk, Hv, dk, dv, adt)
    pool = syn.state_pool(wl, layer, n_slots, Hv, dk, dv, sdt, std=std)
    rs, ws = syn.distinct_slots(wl, layer, n_slots, B, in_place)
    return q, k, v, g, beta, pool, rs, ws


def run_both(case, rule, scale=1.0, status=None):
    q, k, v, g, beta, pool, rs, ws = case
    sdt = pool.dtype
    dq, dk_, dv_, dg, db = (t.to(DEV) for t in (q, k, v, g, beta))
    dpool = pool.to(DEV)
    drs = None if rs is None else rs.to(DEV)
    dws = None if ws is None else ws.to(DEV)
    o = gdn_decode(dq, dk_, dv_, dg, db, dpool, drs, dws, rule=rule, scale=scale, status=status)
    torch.cuda.synchronize()
    ro, rpool, code = oracle.decode(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(pool),
                                    None if rs is None else rs.numpy(),
                                    None if ws is None else ws.numpy(), rule=rule, scale=scale,
                                    round_state=(sdt == torch.bfloat16))
    return o, dpool, ro, rpool, code


@pytest.mark.parametrize("rule", RULES)
def test_decode_b64_bf16_state(rule):
    """B=64, H_qk=16, H_v=32, d=128, BF16 state in a 256-slot pool, distinct read and
    write slots; BF16 q/k/v/o, FP32 gates."""
    say("decode_b64", rule)
    case = make_case(1, 64, 16, 32, 128, 128, 256, torch.bfloat16, torch.bfloat16)
    o, dpool, ro, rpool, code = run_both(case, rule)
    assert code == 0
    pool0 = case[5]
    ws = case[7].numpy()
    assert scaled_err(f64(o), ro, 2) < tol(torch.bfloat16)
    gp = f64(dpool.cpu())
    assert scaled_err(gp[ws], rpool[ws], 2) < tol(torch.bfloat16)
    # slots not written are bitwise unchanged
    others = np.setdiff1d(np.arange(256), ws)
    assert torch.equal(dpool.cpu()[others].view(torch.int16), pool0[others].view(torch.int16))


def test_tiny_fp32_as_decode_steps():
    """B=1, H=2, d=16, T=32 tokens, all FP32, zero initial state, run as 32 decode
    steps in place; outputs and final state within 1e-4 of the oracle."""
    say("tiny_fp32 decode steps")
    T, H, d = 32, 2, 16
    q, k, v, g, beta = syn.token_inputs(0, 0, T, H, H, d, d, torch.float32)
    pool = torch.zeros((1, H, d, d), dtype=torch.float32, device=DEV)
    slot = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = []
    for t in range(T):
        outs.append(gdn_decode(q[t:t + 1].to(DEV), k[t:t + 1].to(DEV), v[t:t + 1].to(DEV),
                               g[t:t + 1].to(DEV), beta[t:t + 1].to(DEV), pool, slot, slot))
    torch.cuda.synchronize()
    o = torch.cat(outs).cpu()
    ro, rpool, _ = oracle.sequences(np.array([0, T], np.int32), f64(q), f64(k), f64(v), f64(g),
                                    f64(beta), np.zeros((1, H, d, d)), [0], [0])
    assert scaled_err(f64(o), ro, 2) < 1e-4
    assert scaled_err(f64(pool), rpool, 2) < 1e-4


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (64, 64),
                                   (128, 128)])
@pytest.mark.parametrize("sdt,adt", [(torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32),
                                     (torch.float32, torch.bfloat16)])
def test_decode_shapes_and_dtypes(dk, dv, sdt, adt):
    say("decode shapes", dk, dv, sdt, adt)
    case = make_case(101, 5, 2, 4, dk, dv, 12, sdt, adt, std=0.3)
    o, dpool, ro, rpool, code = run_both(case, "gated_delta", scale=0.5)
    ws = case[7].numpy()
    assert scaled_err(f64(o), ro, 2) < tol(adt)
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < state_tol(sdt)


@pytest.mark.parametrize("group", [1, 4])
@pytest.mark.parametrize("rule", RULES)
def test_decode_head_groups(group, rule):
    say("decode groups", group, rule)
    case = make_case(102, 3, 2, 2 * group, 64, 64, 6, torch.float32, torch.float32, std=0.3)
    o, dpool, ro, rpool, code = run_both(case, rule)
    ws = case[7].numpy()
    assert scaled_err(f64(o), ro, 2) < 1e-4
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < 1e-4


def test_identity_slots_and_zero_and_skip_indices():
    """NULL index arrays = slot r; read -1 = zero state; write -1 = nothing stored."""
    say("decode identity / -1 slots")
    B, Hqk, Hv, d = 4, 1, 2, 32
    q, k, v, g, beta, pool, _, _ = make_case(103, B, Hqk, Hv, d, d, 8, torch.bfloat16,
                                             torch.bfloat16, std=0.3)
    o, dpool, ro, rpool, _ = run_both((q, k, v, g, beta, pool, None, None), "gated_delta")
    assert scaled_err(f64(o), ro, 2) < 2e-2
    assert scaled_err(f64(dpool)[:B], rpool[:B], 2) < 2e-2
    assert torch.equal(dpool.cpu()[B:].view(torch.int16), pool[B:].view(torch.int16))
    rs = torch.tensor([-1, 2, -1, 5], dtype=torch.int32)
    ws = torch.tensor([0, -1, 3, 4], dtype=torch.int32)
    o, dpool, ro, rpool, code = run_both((q, k, v, g, beta, pool, rs, ws), "gated_delta")
    assert code == 0
    assert scaled_err(f64(o), ro, 2) < 2e-2
    for s in (0, 3, 4):
        assert scaled_err(f64(dpool)[s:s + 1], rpool[s:s + 1], 2) < 2e-2
    for s in (1, 2, 5):
        assert torch.equal(dpool.cpu()[s].view(torch.int16), pool[s].view(torch.int16))


def test_frozen_state_is_a_bitwise_copy():
    """a = 1 (g = 0) and beta = 0 under gated_delta: the write slot receives the read
    slot's bits exactly (+0 and -0 compare equal); o = M0^T q."""
    say("decode frozen copy")
    B, Hqk, Hv, d = 8, 2, 4, 128
    q, k, v, g, beta, pool, rs, ws = make_case(104, B, Hqk, Hv, d, d, 20, torch.bfloat16,
                                               torch.bfloat16)
    g.zero_()
    beta.zero_()
    o, dpool, ro, rpool, _ = run_both((q, k, v, g, beta, pool, rs, ws), "gated_delta")
    got = dpool.cpu()[ws.long()].to(torch.float32)
    want = pool[rs.long()].to(torch.float32)
    assert torch.equal(got, want)  # float compare: +0 == -0, every other value bitwise
    assert scaled_err(f64(o), ro, 2) < 2e-2


def test_in_place_equals_out_of_place():
    say("decode in place vs out of place")
    B, Hqk, Hv, d = 16, 2, 4, 128
    q, k, v, g, beta, pool, rs, ws = make_case(105, B, Hqk, Hv, d, d, 40, torch.bfloat16,
                                               torch.bfloat16)
    o1, p1, _, _, _ = run_both((q, k, v, g, beta, pool, rs, ws), "gated_delta")
    o2, p2, _, _, _ = run_both((q, k, v, g, beta, pool, rs, rs), "gated_delta")
    assert torch.equal(o1.cpu(), o2.cpu())
    assert torch.equal(p1.cpu()[ws.long()].view(torch.int16), p2.cpu()[rs.long()].view(torch.int16))


def test_bad_slot_sets_status_and_skips_only_that_request():
    say("decode bad slot")
    B, Hqk, Hv, d = 6, 1, 2, 64
    q, k, v, g, beta, pool, rs, ws = make_case(106, B, Hqk, Hv, d, d, 16, torch.bfloat16,
                                               torch.bfloat16, std=0.3)
    rs = rs.clone()
    rs[2] = 16  # == n_slots: out of range
    ws = ws.clone()
    ws[4] = -7  # below -1: out of range
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    sentinel = torch.full((B, Hv, d), 7.0, dtype=torch.bfloat16, device=DEV)
    dq, dk_, dv_, dg, db = (t.to(DEV) for t in (q, k, v, g, beta))
    dpool = pool.to(DEV)
    gdn_decode(dq, dk_, dv_, dg, db, dpool, rs.to(DEV), ws.to(DEV), sentinel,
               status=status.view(torch.int32))
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    ro, rpool, code = oracle.decode(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(pool),
                                    rs.numpy(), ws.numpy(), round_state=True)
    assert code == 1
    for r in range(B):
        if r in (2, 4):
            assert torch.all(sentinel[r].cpu() == 7.0)  # o not written
        else:
            assert scaled_err(f64(sentinel[r:r + 1]), ro[r:r + 1], 2) < 2e-2
    assert torch.equal(dpool.cpu()[ws[2]].view(torch.int16), pool[ws[2]].view(torch.int16))
    good = [int(ws[r]) for r in range(B) if r not in (2, 4)]
    assert scaled_err(f64(dpool)[good], rpool[good], 2) < 2e-2


def test_nan_in_one_request_stays_there():
    say("decode nan isolation")
    B, Hqk, Hv, d = 4, 1, 2, 64
    q, k, v, g, beta, pool, rs, ws = make_case(107, B, Hqk, Hv, d, d, 8, torch.float32,
                                               torch.float32, std=0.3)
    v = v.clone()
    v[1, 0, 3] = float("nan")
    o, dpool, ro, rpool, _ = run_both((q, k, v, g, beta, pool, rs, ws), "gated_delta")
    oc = o.cpu()
    assert torch.isnan(oc[1, 0]).any()
    keep = [0, 2, 3]
    assert not torch.isnan(oc[keep]).any() and not torch.isnan(oc[1, 1]).any()
    assert scaled_err(f64(oc[keep]), ro[keep], 2) < 1e-4
    w = ws.long()
    assert not torch.isnan(dpool.cpu()[w[keep]]).any()


def test_empty_batch_is_a_no_op():
    say("decode B=0")
    z = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    zv = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    zg = torch.empty((0, 4), dtype=torch.float32, device=DEV)
    pool = torch.randn((3, 4, 64, 64), device=DEV).to(torch.bfloat16)
    before = pool.clone()
    o = gdn_decode(z, z, zv, zg, zg, pool)
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 64) and torch.equal(pool, before)


def test_decode_b512_full_size():
    """Batch 512 at the benchmark's shapes (one layer: a 512-slot, 512 MiB BF16 pool,
    in place, slots a seeded permutation), every (request, head) tile's o and
    written state against the oracle."""
    say("decode_b512 one layer, every request")
    B, Hqk, Hv, d, n = 512, 16, 32, 128, 512
    q, k, v, g, beta = syn.token_inputs(2, 0, B, Hqk, Hv, d, d, torch.bfloat16)
    pool = syn.state_pool(2, 0, n, Hv, d, d, torch.bfloat16, on_device=True)
    rs, ws = syn.distinct_slots(2, 0, n, B, in_place=True)
    before = pool.cpu()
    dq, dk_, dv_, dg, db = (t.to(DEV) for t in (q, k, v, g, beta))
    o = gdn_decode(dq, dk_, dv_, dg, db, pool, rs.to(DEV), ws.to(DEV))
    torch.cuda.synchronize()
    ro, rpool, code = oracle.decode(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(before),
                                    rs.numpy(), ws.numpy(), round_state=True)
    assert code == 0
    assert scaled_err(f64(o.cpu()), ro, 2) < 2e-2
    w = ws.numpy()
    assert scaled_err(f64(pool.cpu())[w], rpool[w], 2) < 2e-2


@pytest.mark.parametrize("B,n_slots", [(4200, 8400), (64, 40000)])
def test_decode_request_order_fallback(B, n_slots):
    """Batches larger than the slot-order table (B > 4096) or pools larger than
    its bitmap (n_slots > 32768) are walked in request order; results are the
    same as ever (small heads keep the oracle quick)."""
    say("decode order fallback", B, n_slots)
    case = make_case(9, B, 1, 2, 16, 16, n_slots, torch.bfloat16, torch.float32)
    o, dpool, ro, rpool, code = run_both(case, "gated_delta")
    assert code == 0
    ws = case[7].numpy()
    assert scaled_err(f64(o), ro, 2) < tol(torch.bfloat16)
    assert scaled_err(f64(dpool.cpu())[ws], rpool[ws], 2) < tol(torch.bfloat16)

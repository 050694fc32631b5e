"""Decode-side conv step and conv-state store: the HIP kernels (through the C
ABI) against the FP64 oracle on the same seeded inputs, and against the
prefill front-end (bitwise: the two share their per-channel arithmetic).

Outputs q, k, v are compared per (request, head) slice at the front-end's
tolerance; the conv pool holds raw inputs copied bit for bit, so it is
compared exactly."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import (gdn_conv_decode, gdn_conv_store, gdn_frontend,
                                               synthetic as syn)
from gpu_util import f64, say, scaled_err, tol

pytestmark = pytest.mark.gpu
DEV = "cuda"
K = 4


def dev(t):
    return None if t is None else t.to(DEV)


def channels(Hqk, Hv, dk, dv):
    return 2 * Hqk * dk + Hv * dv


def run_decode(x, pool, rs, ws, Hqk, Hv, status=None):
    return gdn_conv_decode(dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]), pool, dev(rs),
                           dev(ws), H_qk=Hqk, H_v=Hv, conv_wq=dev(x["conv_wq"]),
                           conv_wk=dev(x["conv_wk"]), conv_wv=dev(x["conv_wv"]),
                           a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]), status=status)


def run_oracle(x, pool_host, rs, ws, Hqk, Hv):
    return oracle.conv_decode(f64(x["q_raw"]), f64(x["k_raw"]), f64(x["v_raw"]),
                              f64(x["conv_wq"]), f64(x["conv_wk"]), f64(x["conv_wv"]),
                              f64(x["a_raw"]), f64(x["b_raw"]), pool_host,
                              None if rs is None else rs.numpy(),
                              None if ws is None else ws.numpy(), Hqk=Hqk, Hv=Hv)


def check(out, ref, adt, rows=None):
    rows = slice(None) if rows is None else rows
    t = tol(adt)
    for got, want in zip(out[:3], ref[:3]):
        assert scaled_err(f64(got)[rows], want[rows], 2) < t
    np.testing.assert_allclose(f64(out[3])[rows], ref[3][rows], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(f64(out[4])[rows], ref[4][rows], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 64), (64, 16), (32, 32)])
def test_conv_decode_parity(adt, dk, dv):
    say("conv decode", adt, dk, dv)
    Hqk, Hv, B, n_slots = 2, 4, 37, 80
    x = syn.frontend_inputs(401, 0, B, Hqk, Hv, dk, dv, K, adt)
    pool0 = syn.conv_pool(401, 0, n_slots, channels(Hqk, Hv, dk, dv), K, adt)
    rs, ws = syn.distinct_slots(401, 0, n_slots, B, in_place=False)
    rs[::5] = -1   # fresh requests: empty window
    pool = dev(pool0.clone())
    out = run_decode(x, pool, rs, ws, Hqk, Hv)
    torch.cuda.synchronize()
    ref = run_oracle(x, f64(pool0), rs, ws, Hqk, Hv)
    assert ref[6] == 0
    check(out, ref, adt)
    np.testing.assert_array_equal(f64(pool), ref[5])


def test_conv_decode_in_place_identity_and_bad_slot():
    say("conv decode in place + bad slot")
    Hqk, Hv, dk, dv, B = 16, 32, 128, 128, 24
    adt = torch.bfloat16
    x = syn.frontend_inputs(402, 0, B, Hqk, Hv, dk, dv, K, adt)
    pool0 = syn.conv_pool(402, 0, B, channels(Hqk, Hv, dk, dv), K, adt)
    # NULL slot arrays: request r reads and writes slot r in place
    pool = dev(pool0.clone())
    out = run_decode(x, pool, None, None, Hqk, Hv)
    torch.cuda.synchronize()
    ref = run_oracle(x, f64(pool0), None, None, Hqk, Hv)
    check(out, ref, adt)
    np.testing.assert_array_equal(f64(pool), ref[5])
    # request 5 names a slot past the pool: skipped, status bit set, its slot untouched
    rs = torch.arange(B, dtype=torch.int32)
    ws = rs.clone()
    rs[5] = B
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool = dev(pool0.clone())
    out = run_decode(x, pool, rs, ws, Hqk, Hv, status=status)
    torch.cuda.synchronize()
    ref = run_oracle(x, f64(pool0), rs, ws, Hqk, Hv)
    assert ref[6] == 1 and int(status.item()) == 1
    keep = np.arange(B) != 5
    check(out, ref, adt, rows=keep)
    np.testing.assert_array_equal(f64(pool), ref[5])
    np.testing.assert_array_equal(f64(pool)[5], f64(pool0)[5])


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float32])
def test_conv_store_parity(adt):
    say("conv store", adt)
    Hqk, Hv, dk, dv = 2, 4, 64, 32
    lengths = [0, 1, 2, 3, 5, 70, 4]
    N = int(sum(lengths))
    cu = syn.cu_from_lengths(lengths)
    x = syn.frontend_inputs(403, 0, N, Hqk, Hv, dk, dv, K, adt)
    n_slots = 10
    pool0 = syn.conv_pool(403, 0, n_slots, channels(Hqk, Hv, dk, dv), K, adt)
    ws = torch.tensor([9, 0, 3, -1, 7, 2, 5], dtype=torch.int32)
    pool = dev(pool0.clone())
    gdn_conv_store(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]), pool, dev(ws),
                   H_qk=Hqk, H_v=Hv)
    torch.cuda.synchronize()
    tail = oracle.conv_tail(cu.numpy(), f64(x["q_raw"]), f64(x["k_raw"]), f64(x["v_raw"]), K)
    want = f64(pool0)
    for s, w in enumerate(ws.tolist()):
        if w >= 0:
            want[w] = tail[s]
    np.testing.assert_array_equal(f64(pool), want)


def test_conv_store_bad_offsets_and_slots():
    say("conv store bad offsets / slots")
    Hqk, Hv, dk, dv = 1, 2, 16, 16
    adt = torch.bfloat16
    x = syn.frontend_inputs(404, 0, 12, Hqk, Hv, dk, dv, K, adt)
    pool0 = syn.conv_pool(404, 0, 4, channels(Hqk, Hv, dk, dv), K, adt)
    cu = torch.tensor([0, 5, 3, 12], dtype=torch.int32)   # sequence 1 runs backwards
    ws = torch.tensor([0, 1, 6], dtype=torch.int32)       # sequence 2 names a slot past the pool
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    pool = dev(pool0.clone())
    gdn_conv_store(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]), pool, dev(ws),
                   H_qk=Hqk, H_v=Hv, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 3   # bad slot | bad sequence
    want = f64(pool0)
    want[0] = oracle.conv_tail(np.array([0, 5]), f64(x["q_raw"]), f64(x["k_raw"]),
                               f64(x["v_raw"]), K)[0]
    np.testing.assert_array_equal(f64(pool), want)


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float32])
def test_store_then_decode_equals_frontend_bitwise(adt):
    """Front-end over whole sequences == store after the first L tokens, then
    two decode steps (the second in place), token for token, bit for bit."""
    say("conv store + decode == frontend", adt)
    Hqk, Hv, dk, dv = 2, 4, 64, 64
    L = [0, 1, 2, 5, 64, 130]          # prefilled lengths; each sequence then decodes 2 tokens
    full = [l + 2 for l in L]
    N = int(sum(full))
    x = syn.frontend_inputs(405, 0, N, Hqk, Hv, dk, dv, K, adt)
    cu_full = syn.cu_from_lengths(full)
    fq, fk, fv, fg, fb = gdn_frontend(dev(cu_full), dev(x["q_raw"]), dev(x["k_raw"]),
                                      dev(x["v_raw"]), H_qk=Hqk, H_v=Hv,
                                      conv_wq=dev(x["conv_wq"]), conv_wk=dev(x["conv_wk"]),
                                      conv_wv=dev(x["conv_wv"]), a_raw=dev(x["a_raw"]),
                                      b_raw=dev(x["b_raw"]))
    starts = cu_full[:-1].long()
    pre = torch.cat([torch.arange(int(s), int(s) + l) for s, l in zip(starts, L)]).long() \
        if sum(L) else torch.zeros(0, dtype=torch.long)
    pick = lambda key, rows: x[key][rows].contiguous()
    n_seq = len(L)
    pool = torch.zeros((n_seq, K - 1, channels(Hqk, Hv, dk, dv)), dtype=adt, device=DEV)
    slots = torch.arange(n_seq, dtype=torch.int32)
    gdn_conv_store(dev(syn.cu_from_lengths(L)), dev(pick("q_raw", pre)), dev(pick("k_raw", pre)),
                   dev(pick("v_raw", pre)), pool, dev(slots), H_qk=Hqk, H_v=Hv)
    for step in range(2):
        rows = starts + torch.tensor(L) + step
        xd = {kk: pick(kk, rows) for kk in ("q_raw", "k_raw", "v_raw", "a_raw", "b_raw")}
        xd.update({kk: x[kk] for kk in ("conv_wq", "conv_wk", "conv_wv")})
        q, k, v, g, b = run_decode(xd, pool, slots, slots, Hqk, Hv)
        torch.cuda.synchronize()
        r = rows.to(DEV)
        assert torch.equal(q, fq[r]) and torch.equal(k, fk[r]) and torch.equal(v, fv[r])
        assert torch.equal(g, fg[r]) and torch.equal(b, fb[r])


def test_conv_decode_full_size():
    """B = 512 requests of H_qk = 16, H_v = 32, d = 128 BF16 (the decode
    workload's shape), distinct read/write slots in a 1024-slot pool."""
    say("conv decode full size B=512")
    Hqk, Hv, d, B, n_slots = 16, 32, 128, 512, 1024
    adt = torch.bfloat16
    x = syn.frontend_inputs(406, 0, B, Hqk, Hv, d, d, K, adt)
    pool0 = syn.conv_pool(406, 0, n_slots, channels(Hqk, Hv, d, d), K, adt)
    rs, ws = syn.distinct_slots(406, 0, n_slots, B, in_place=False)
    pool = dev(pool0.clone())
    out = run_decode(x, pool, rs, ws, Hqk, Hv)
    torch.cuda.synchronize()
    ref = run_oracle(x, f64(pool0), rs, ws, Hqk, Hv)
    check(out, ref, adt)
    np.testing.assert_array_equal(f64(pool), ref[5])


def test_prefill_store_then_conv_decode_steps_match_the_oracle():
    """A whole layer across calls: gdn_prefill (fused front-end) over L tokens of
    each sequence, gdn_conv_store, then two decode steps of conv then
    gdn_decode (in-place slots) == the oracle's front-end and token recurrence
    over all L + 2 tokens."""
    say("prefill + conv store + 2 x (conv decode + decode) vs oracle")
    from linear_attention_recurrent_02_amd import gdn_decode, gdn_prefill
    Hqk, Hv, d = 2, 4, 64
    adt = torch.bfloat16
    L = [1, 3, 70, 129]
    full = [l + 2 for l in L]
    N = int(sum(full))
    x = syn.frontend_inputs(407, 0, N, Hqk, Hv, d, d, K, adt)
    cu_full = syn.cu_from_lengths(full)
    starts = cu_full[:-1].long()
    pre = torch.cat([torch.arange(int(s), int(s) + l) for s, l in zip(starts, L)]).long()
    pick = lambda key, rows: x[key][rows].contiguous()
    n = len(L)
    slots = torch.arange(n, dtype=torch.int32, device=DEV)
    pool = torch.zeros((n, Hv, d, d), dtype=torch.float32, device=DEV)
    cpool = torch.zeros((n, K - 1, channels(Hqk, Hv, d, d)), dtype=adt, device=DEV)
    cu_pre = dev(syn.cu_from_lengths(L))
    o_pre = gdn_prefill(cu_pre, dev(pick("q_raw", pre)), dev(pick("k_raw", pre)),
                        dev(pick("v_raw", pre)), pool, torch.full((n,), -1, dtype=torch.int32,
                                                                  device=DEV), slots,
                        H_qk=Hqk, H_v=Hv, a_raw=dev(pick("a_raw", pre)),
                        b_raw=dev(pick("b_raw", pre)), conv_wq=dev(x["conv_wq"]),
                        conv_wk=dev(x["conv_wk"]), conv_wv=dev(x["conv_wv"]))
    gdn_conv_store(cu_pre, dev(pick("q_raw", pre)), dev(pick("k_raw", pre)),
                   dev(pick("v_raw", pre)), cpool, slots, H_qk=Hqk, H_v=Hv)
    outs = []
    for step in range(2):
        rows = starts + torch.tensor(L) + step
        xd = {kk: pick(kk, rows) for kk in ("q_raw", "k_raw", "v_raw", "a_raw", "b_raw")}
        xd.update({kk: x[kk] for kk in ("conv_wq", "conv_wk", "conv_wv")})
        q, k, v, g, b = run_decode(xd, cpool, slots, slots, Hqk, Hv)
        outs.append(gdn_decode(q, k, v, g, b, pool, slots, slots))
    torch.cuda.synchronize()
    # oracle: front-end over whole sequences (its q, k, v rounded to the activation dtype
    # where the GPU path stores them), then the token recurrence from a zero state
    rq, rk, rv, rg, rb = oracle.frontend(cu_full.numpy(), f64(x["q_raw"]), f64(x["k_raw"]),
                                         f64(x["v_raw"]), f64(x["conv_wq"]), f64(x["conv_wk"]),
                                         f64(x["conv_wv"]), f64(x["a_raw"]), f64(x["b_raw"]),
                                         Hqk=Hqk, Hv=Hv)
    rq, rk, rv = (oracle.round_bf16(t) for t in (rq, rk, rv))
    ro, rpool, code = oracle.sequences(cu_full.numpy(), rq, rk, rv, rg, rb,
                                       np.zeros((n, Hv, d, d)), [-1] * n, list(range(n)))
    assert code == 0
    t = tol(adt)
    last = [int(s) + l for s, l in zip(starts, L)]
    for step in range(2):
        want = ro[[r + step for r in last]]
        assert scaled_err(f64(outs[step]), want, 2) < t
    assert scaled_err(f64(pool), rpool, 2) < t
    got_pre = f64(o_pre)
    assert scaled_err(got_pre, ro[pre.numpy()], 2) < t

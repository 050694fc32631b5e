"""Front-end and chunked-prefill parity: the HIP kernels (through the C ABI)
against the FP64 oracle on the same seeded inputs.

Prefill outputs are compared per (sequence, head) slice -- the (request, head)
slice of a prefill call -- and final states per (slot, head) tile.  When the
activations are BF16, the fused path stores the front-end's q, k, v in BF16
before the recurrence reads them, so the oracle rounds its own front-end
outputs to BF16 at that point (as it rounds a BF16-stored state)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import (gdn_decode, gdn_frontend, gdn_prefill,
                                               synthetic as syn)
from gpu_util import f64, say, scaled_err, seq_err, state_tol, tol

pytestmark = pytest.mark.gpu
RULES = ["linear", "gated", "delta", "gated_delta"]
DEV = "cuda"


def dev(t):
    return None if t is None else t.to(DEV)


def prefill_case(wl, lengths, Hqk, Hv, dk, dv, n_slots, sdt, adt, std=0.02, fresh=()):
    """Final (post front-end) inputs for sequences of the given lengths, a pool,
    read slots (indices in `fresh` start from zero) and distinct write slots."""
    lengths = list(lengths)
    N = int(sum(lengths))
    cu = syn.cu_from_lengths(lengths)
    q, k, v, g, beta = syn.token_inputs(wl, 0, N, Hqk, Hv, dk, dv, adt)
    pool = syn.state_pool(wl, 0, n_slots, Hv, dk, dv, sdt, std=std)
    rs, ws = syn.distinct_slots(wl, 0, n_slots, len(lengths), in_place=False)
    rs = rs.clone()
    for i in fresh:
        rs[i] = -1
    return cu, q, k, v, g, beta, pool, rs, ws


def run_prefill_both(case, rule, scale=1.0):
    cu, q, k, v, g, beta, pool, rs, ws = case
    N, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dpool = dev(pool)
    o = gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), H_qk=Hqk, H_v=Hv,
                    g=dev(g), beta=dev(beta), rule=rule, scale=scale)
    torch.cuda.synchronize()
    ro, rpool, code = oracle.sequences(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                       f64(pool), None if rs is None else rs.numpy(),
                                       None if ws is None else ws.numpy(), rule=rule, scale=scale,
                                       round_state=(pool.dtype == torch.bfloat16))
    assert code == 0
    return o, dpool, ro, rpool


def test_tiny_fp32_prefill():
    """B=1, H=2, d=16, T=32 tokens, all FP32, zero initial state, one prefill call
    (a single ragged chunk); outputs and final state within 1e-4."""
    say("tiny_fp32 prefill")
    case = prefill_case(0, [32], 2, 2, 16, 16, 2, torch.float32, torch.float32, std=0.0)
    cu, q, k, v, g, beta, pool, _, _ = case
    slot = torch.zeros(1, dtype=torch.int32)
    o, dpool, ro, rpool = run_prefill_both((cu, q, k, v, g, beta, pool, slot, slot), "gated_delta")
    assert seq_err(f64(o), ro, cu) < 1e-4
    assert scaled_err(f64(dpool), rpool, 2) < 1e-4


@pytest.mark.parametrize("rule", RULES)
def test_prefill_bf16_ragged(rule):
    """BF16 q/k/v/o and state, d=128, H_qk=2, H_v=4; sequences of 1, 63, 64, 200
    tokens (ragged tails, several chunks); one fresh request, the others start
    from a checkpoint slot."""
    say("prefill bf16 ragged", rule)
    case = prefill_case(201, [1, 63, 64, 200], 2, 4, 128, 128, 12, torch.bfloat16,
                        torch.bfloat16, fresh=(1,))
    o, dpool, ro, rpool = run_prefill_both(case, rule)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 2e-2
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < 2e-2
    others = np.setdiff1d(np.arange(12), ws)
    assert torch.equal(dpool.cpu()[others].view(torch.int16), case[6][others].view(torch.int16))


def checkpoint_case(wl, lengths, d, sdt, adt, per_seq, skip=()):
    """A prefill case plus a checkpoint slot matrix [n_seq, per_seq] drawn from
    the slots that are neither read nor written (entries in `skip` are -1)."""
    n_seq = len(lengths)
    n_slots = 2 * n_seq + n_seq * per_seq + 4
    case = prefill_case(wl, lengths, 1, 2, d, d, n_slots, sdt, adt, std=0.1, fresh=(0,))
    used = set(case[7].tolist()) | set(case[8].tolist())
    free = [s for s in np.random.default_rng(wl).permutation(n_slots) if s not in used]
    ck = np.array(free[:n_seq * per_seq], np.int32).reshape(n_seq, per_seq)
    for s_, j in skip:
        ck[s_, j] = -1
    return case, ck


@pytest.mark.parametrize("d,dt,tol,interval", [(128, torch.bfloat16, 2e-2, 64),
                                               (128, torch.bfloat16, 2e-2, 128),
                                               (32, torch.float32, 1e-4, 64)])
def test_prefill_checkpoints(d, dt, tol, interval):
    """Intermediate checkpoints at block boundaries: slot [s, j] holds sequence
    s's state after its first (j + 1) * interval tokens, i.e. the state that a
    prefill of just those tokens stores (checked against the oracle run on each
    prefix); slots past a sequence's end and -1 entries are left alone, and the
    outputs and final states are those of a prefill without checkpoints.  d = 128
    runs the pipelined chain, d = 32 in FP32 the plain one."""
    say("prefill checkpoints", d, interval)
    lengths = [300, 128, 64, 65, 0, 1, 256]
    case, ck = checkpoint_case(212, lengths, d, dt, dt, per_seq=4, skip=((0, 1),))
    cu, q, k, v, g, beta, pool, rs, ws = case
    dpool = dev(pool)
    o = gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), H_qk=1, H_v=2,
                    g=dev(g), beta=dev(beta), ckpt_interval=interval,
                    ckpt_slot=dev(torch.from_numpy(ck)))
    torch.cuda.synchronize()
    rnd = dt == torch.bfloat16
    ro, rpool, code = oracle.sequences(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                       f64(pool), rs.numpy(), ws.numpy(), round_state=rnd)
    assert code == 0
    assert seq_err(f64(o), ro, cu) < tol
    assert scaled_err(f64(dpool)[ws.numpy()], rpool[ws.numpy()], 2) < tol
    got = f64(dpool.cpu())
    written = set()
    for s_, L in enumerate(lengths):
        for j in range(ck.shape[1]):
            n = (j + 1) * interval
            slot = int(ck[s_, j])
            if slot < 0 or n > L:
                continue
            a, b = int(cu[s_]), int(cu[s_]) + n
            _, ppool, c2 = oracle.sequences(np.array([0, n], np.int32), f64(q[a:b]), f64(k[a:b]),
                                            f64(v[a:b]), f64(g[a:b]), f64(beta[a:b]), f64(pool),
                                            rs.numpy()[s_:s_ + 1], np.array([slot], np.int32),
                                            round_state=rnd)
            assert c2 == 0
            assert scaled_err(got[slot], ppool[slot], 2) < tol, (s_, j)
            written.add(slot)
    expect = sum(1 for s_, L in enumerate(lengths) for j in range(ck.shape[1])
                 if (j + 1) * interval <= L and ck[s_, j] >= 0)
    assert len(written) == expect > 0
    untouched = np.setdiff1d(np.arange(pool.shape[0]),
                             np.concatenate([ws.numpy(), np.array(sorted(written), np.int64)]))
    assert torch.equal(dpool.cpu()[untouched], pool[untouched])


def test_prefill_checkpoint_bad_slot():
    """An out-of-range checkpoint slot stores nothing and sets the status bit;
    everything else is computed as usual."""
    say("prefill checkpoint bad slot")
    case, ck = checkpoint_case(213, [130, 64], 128, torch.bfloat16, torch.bfloat16, per_seq=2)
    cu, q, k, v, g, beta, pool, rs, ws = case
    ck[0, 1] = pool.shape[0] + 3
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dpool = dev(pool)
    gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), H_qk=1, H_v=2,
                g=dev(g), beta=dev(beta), ckpt_interval=64, ckpt_slot=dev(torch.from_numpy(ck)),
                status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    ro, rpool, code = oracle.sequences(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                       f64(pool), rs.numpy(), ws.numpy(), round_state=True)
    assert scaled_err(f64(dpool)[ws.numpy()], rpool[ws.numpy()], 2) < 2e-2
    # the valid checkpoints (sequence 0 at 64, sequence 1 at 64) were stored
    for s_, j in ((0, 0), (1, 0)):
        assert not torch.equal(dpool.cpu()[int(ck[s_, j])], pool[int(ck[s_, j])])


@pytest.mark.parametrize("rule", RULES)
def test_prefill_bf16_fp32_state(rule):
    """BF16 q/k/v/o with an FP32 state pool at d = 128: the chain computes in
    FP32 (FP32 MFMA operands, the BF16 inputs widened exactly), so the FP32
    state meets the FP32 bar, 1e-4, against the oracle on the same BF16
    inputs; o is stored in BF16 and meets the BF16 bar.  Ragged sequences over
    several chunks, one fresh request."""
    say("prefill bf16 act, fp32 state", rule)
    case = prefill_case(211, [5, 64, 130, 300], 2, 4, 128, 128, 10, torch.float32,
                        torch.bfloat16, std=0.05, fresh=(0,))
    o, dpool, ro, rpool = run_prefill_both(case, rule)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < tol(torch.bfloat16)
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < state_tol(torch.float32)


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128), (32, 32), (16, 128)])
def test_prefill_bf16_fp32_state_shapes(dk, dv):
    """The FP32 chain for FP32 states with BF16 activations at other head sizes."""
    say("prefill bf16 act, fp32 state, shapes", dk, dv)
    case = prefill_case(214, [70, 129], 2, 4, dk, dv, 6, torch.float32, torch.bfloat16, std=0.1)
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < tol(torch.bfloat16)
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < state_tol(torch.float32)


def test_prefill_bf16_fp32_state_long():
    """One 2,000-token sequence (32 chunks) from a checkpoint, FP32 state with
    BF16 activations at d = 128: the FP32 chain's error does not grow past the
    FP32 bar over a long chain."""
    say("prefill bf16 act, fp32 state, long")
    case = prefill_case(215, [2000], 1, 2, 128, 128, 2, torch.float32, torch.bfloat16, std=0.05)
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < tol(torch.bfloat16)
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < state_tol(torch.float32)


@pytest.mark.parametrize("rule", RULES)
def test_prefill_fp32_rules(rule):
    say("prefill fp32", rule)
    case = prefill_case(202, [150, 17], 1, 2, 64, 64, 4, torch.float32, torch.float32, std=0.3)
    o, dpool, ro, rpool = run_prefill_both(case, rule, scale=0.5)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 1e-4
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < 1e-4


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128),
                                   (128, 64), (64, 64), (64, 128), (32, 128)])
def test_prefill_shapes_bf16(dk, dv):
    say("prefill shapes", dk, dv)
    case = prefill_case(203, [70, 130], 2, 4, dk, dv, 6, torch.bfloat16, torch.bfloat16, std=0.1)
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 2e-2
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < 2e-2


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (16, 64), (64, 16)])
def test_prefill_shapes_fp32(dk, dv):
    say("prefill shapes fp32", dk, dv)
    case = prefill_case(204, [97], 1, 1, dk, dv, 2, torch.float32, torch.float32, std=0.3)
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 1e-4
    assert scaled_err(f64(dpool)[ws], rpool[ws], 2) < 1e-4


def test_prefill_empty_sequences_and_identity_slots():
    """Zero-length sequences store their initial state unchanged (rounded); NULL
    slot arrays mean slot s for sequence s."""
    say("prefill empty sequences")
    case = prefill_case(205, [0, 10, 0, 65], 2, 2, 64, 64, 8, torch.float32, torch.float32,
                        std=0.3)
    cu, q, k, v, g, beta, pool, _, _ = case
    o, dpool, ro, rpool = run_prefill_both((cu, q, k, v, g, beta, pool, None, None), "gated_delta")
    assert seq_err(f64(o), ro, cu) < 1e-4
    assert scaled_err(f64(dpool), rpool, 2) < 1e-4
    assert torch.equal(dpool.cpu()[0], pool[0]) and torch.equal(dpool.cpu()[2], pool[2])


def test_prefill_then_decode_equals_longer_prefill():
    """prefill(T1) into a checkpoint slot, then T2 decode steps from it, equals the
    oracle's run over T1 + T2 tokens (FP32 throughout)."""
    say("prefill then decode")
    T1, T2, Hqk, Hv, d = 130, 5, 1, 2, 64
    q, k, v, g, beta = syn.token_inputs(206, 0, T1 + T2, Hqk, Hv, d, d, torch.float32)
    pool = torch.zeros((2, Hv, d, d), dtype=torch.float32, device=DEV)
    s0 = torch.tensor([-1], dtype=torch.int32, device=DEV)
    s1 = torch.tensor([1], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, T1], dtype=torch.int32, device=DEV)
    o1 = gdn_prefill(cu, dev(q[:T1]), dev(k[:T1]), dev(v[:T1]), pool, s0, s1, H_qk=Hqk, H_v=Hv,
                     g=dev(g[:T1]), beta=dev(beta[:T1]))
    outs = [o1]
    for t in range(T1, T1 + T2):
        outs.append(gdn_decode(dev(q[t:t + 1]), dev(k[t:t + 1]), dev(v[t:t + 1]), dev(g[t:t + 1]),
                               dev(beta[t:t + 1]), pool, s1, s1))
    torch.cuda.synchronize()
    ro, rpool, _ = oracle.sequences(np.array([0, T1 + T2], np.int32), f64(q), f64(k), f64(v),
                                    f64(g), f64(beta), np.zeros((1, Hv, d, d)), [0], [0])
    assert seq_err(f64(torch.cat(outs)), ro, [0, T1 + T2]) < 1e-4
    assert scaled_err(f64(pool)[1:2], rpool, 2) < 1e-4


# (d, dtype, tolerance): a plain-chain shape and the pipelined chain's shape
CHAIN_KINDS = [(32, torch.float32, 1e-4), (128, torch.bfloat16, 2e-2)]


def test_prefill_many_short_sequences_d128():
    """The pipelined chain's shape (d = 128, BF16): 60 sequences of 0..150
    tokens (empty, one-chunk and ragged ones; the producers' prefetch runs
    past the end of most of them), gated_delta, half from checkpoint slots."""
    say("prefill many short sequences d128")
    lengths = np.random.default_rng(12).integers(0, 151, size=60)
    lengths[::7] = 0
    case = prefill_case(210, lengths, 1, 2, 128, 128, 120, torch.bfloat16, torch.bfloat16,
                        fresh=range(0, 60, 2))
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    cu, ws = case[0], case[8].numpy()
    assert seq_err(f64(o), ro, cu) < 2e-2
    assert scaled_err(f64(dpool.cpu())[ws], rpool[ws], 2) < 2e-2


@pytest.mark.parametrize("d,dt,tol", CHAIN_KINDS)
def test_prefill_bad_slot_status(d, dt, tol):
    say("prefill bad slot", d)
    case = prefill_case(207, [40, 40], 1, 2, d, d, 4, dt, dt, std=0.3)
    cu, q, k, v, g, beta, pool, rs, ws = case
    rs = rs.clone()
    rs[1] = 9
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dpool = dev(pool)
    o = torch.full((80, 2, d), 5.0, dtype=dt, device=DEV)
    gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), o, H_qk=1, H_v=2,
                g=dev(g), beta=dev(beta), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    assert torch.all(o[40:].cpu() == 5.0)
    ro, rpool, code = oracle.sequences(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                       f64(pool), rs.numpy(), ws.numpy())
    assert code == 1
    assert seq_err(f64(o[:40]), ro[:40], [0, 40]) < tol


def test_prefill_many_short_sequences():
    """300 sequences of 0..150 tokens (chain count not a multiple of the
    16-chain block groups, many one-chunk and empty sequences), gated_delta,
    BF16 state in a 600-slot pool."""
    say("prefill many short sequences")
    lengths = np.random.default_rng(11).integers(0, 151, size=300)
    lengths[::37] = 0
    case = prefill_case(209, lengths, 1, 2, 32, 32, 600, torch.bfloat16, torch.bfloat16,
                        fresh=range(0, 300, 5))
    o, dpool, ro, rpool = run_prefill_both(case, "gated_delta")
    cu, ws = case[0], case[8].numpy()
    assert seq_err(f64(o), ro, cu) < 2e-2
    assert scaled_err(f64(dpool.cpu())[ws], rpool[ws], 2) < 2e-2


@pytest.mark.parametrize("d,dt,tol", CHAIN_KINDS)
@pytest.mark.parametrize("bad_cu", [[0, 40, 120], [0, 60, 40]])
def test_prefill_bad_offsets_status(bad_cu, d, dt, tol):
    """A sequence whose offsets break the cu_seqlens contract (ending past
    n_tokens, or decreasing) is skipped and flags GDN_DEVICE_BAD_SEQ; the other
    sequence is computed as usual.  The kernel's own offset check keeps every
    access inside the token arrays."""
    say("prefill bad offsets", bad_cu, d)
    case = prefill_case(208, [40, 40], 1, 2, d, d, 4, dt, dt, std=0.3)
    cu, q, k, v, g, beta, pool, rs, ws = case
    bad = torch.tensor(bad_cu, dtype=torch.int32)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dpool = dev(pool)
    o = torch.full((80, 2, d), 5.0, dtype=dt, device=DEV)
    gdn_prefill(dev(bad), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), o, H_qk=1, H_v=2,
                g=dev(g), beta=dev(beta), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    first = bad_cu[1] if bad_cu[1] <= 80 else 80
    ro, rpool, code = oracle.sequences(np.array([0, first]), f64(q[:first]), f64(k[:first]),
                                       f64(v[:first]), f64(g[:first]), f64(beta[:first]),
                                       f64(pool), rs[:1].numpy(), ws[:1].numpy())
    assert code == 0
    assert seq_err(f64(o[:first]), ro, [0, first]) < tol
    assert torch.all(o[first:].cpu() == 5.0)  # the skipped sequence wrote nothing
    assert scaled_err(f64(dpool)[ws[1]], f64(pool)[ws[1]], 2) == 0  # nor its state


# --------------------------------------------------------------------------
# front-end


def frontend_case(wl, lengths, Hqk, Hv, dk, dv, adt):
    N = int(sum(lengths))
    cu = syn.cu_from_lengths(lengths)
    x = syn.frontend_inputs(wl, 0, N, Hqk, Hv, dk, dv, 4, adt)
    return cu, x


def oracle_frontend(cu, x, Hqk, Hv):
    return oracle.frontend(cu.numpy(), f64(x["q_raw"]), f64(x["k_raw"]), f64(x["v_raw"]),
                           f64(x["conv_wq"]), f64(x["conv_wk"]), f64(x["conv_wv"]),
                           f64(x["a_raw"]), f64(x["b_raw"]), Hqk=Hqk, Hv=Hv)


@pytest.mark.parametrize("adt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 64), (64, 16)])
def test_frontend(adt, dk, dv):
    say("frontend", adt, dk, dv)
    lengths = [1, 2, 0, 5, 70, 0, 131]  # starts inside 64-token runs, empty sequences, ragged end
    Hqk, Hv = 2, 4
    cu, x = frontend_case(301, lengths, Hqk, Hv, dk, dv, adt)
    q, k, v, g, beta = gdn_frontend(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]),
                                    H_qk=Hqk, H_v=Hv, conv_wq=dev(x["conv_wq"]),
                                    conv_wk=dev(x["conv_wk"]), conv_wv=dev(x["conv_wv"]),
                                    a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]))
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb = oracle_frontend(cu, x, Hqk, Hv)
    t = tol(adt)
    assert scaled_err(f64(q), rq, 2) < t
    assert scaled_err(f64(k), rk, 2) < t
    assert scaled_err(f64(v), rv, 2) < t
    np.testing.assert_allclose(f64(g), rg, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(f64(beta), rb, rtol=1e-5, atol=1e-6)


def test_frontend_full_heads_long_ranges():
    """H_qk=16, H_v=32, d=128 BF16 over 17,000 tokens: each workgroup then walks
    several 64-token runs, and sequence starts fall on run boundaries (64, 8384),
    next to empty sequences and one-token ones."""
    say("frontend long ranges")
    lengths = [64, 0, 8192, 128, 63, 1, 8552]
    Hqk, Hv, d = 16, 32, 128
    cu, x = frontend_case(304, lengths, Hqk, Hv, d, d, torch.bfloat16)
    q, k, v, g, beta = gdn_frontend(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]),
                                    H_qk=Hqk, H_v=Hv, conv_wq=dev(x["conv_wq"]),
                                    conv_wk=dev(x["conv_wk"]), conv_wv=dev(x["conv_wv"]),
                                    a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]))
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb = oracle_frontend(cu, x, Hqk, Hv)
    t = tol(torch.bfloat16)
    assert scaled_err(f64(q), rq, 2) < t
    assert scaled_err(f64(k), rk, 2) < t
    assert scaled_err(f64(v), rv, 2) < t
    np.testing.assert_allclose(f64(g), rg, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(f64(beta), rb, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("rule", ["gated_delta", "delta"])
def test_prefill_with_frontend(rule):
    """Raw projections through the fused front-end then the chunked recurrence,
    against the oracle's front-end followed by its token recurrence."""
    say("prefill with frontend", rule)
    lengths = [3, 64, 190]
    Hqk, Hv, d = 2, 4, 128
    cu, x = frontend_case(302, lengths, Hqk, Hv, d, d, torch.bfloat16)
    pool = syn.state_pool(302, 0, 6, Hv, d, d, torch.bfloat16)
    rs = torch.tensor([-1, 0, 1], dtype=torch.int32)
    ws = torch.tensor([3, 4, 5], dtype=torch.int32)
    dpool = dev(pool)
    o = gdn_prefill(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]), dpool, dev(rs),
                    dev(ws), H_qk=Hqk, H_v=Hv, a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]),
                    conv_wq=dev(x["conv_wq"]), conv_wk=dev(x["conv_wk"]),
                    conv_wv=dev(x["conv_wv"]), rule=rule)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb = oracle_frontend(cu, x, Hqk, Hv)
    rq, rk, rv = (oracle.round_bf16(t) for t in (rq, rk, rv))  # stored in BF16 before use
    ro, rpool, _ = oracle.sequences(cu.numpy(), rq, rk, rv, rg, rb, f64(pool), rs.numpy(),
                                    ws.numpy(), rule=rule, round_state=True)
    assert seq_err(f64(o), ro, cu) < 2e-2
    assert scaled_err(f64(dpool)[3:6], rpool[3:6], 2) < 2e-2


def test_prefill_varlen_full_size():
    """The chunked-prefill workload at full size (8 sequences of 1024..8192 tokens,
    H_qk=16, H_v=32, d=128, BF16, fused front-end, fresh requests, final states to
    8 checkpoint slots of a 64-slot pool), every state head of every sequence
    against the oracle's front-end and token recurrence."""
    say("prefill_varlen full size, every head")
    wl = syn.WORKLOADS["prefill_varlen"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lengths = syn.seq_lengths(wl["index"], 0, wl["n_seq"], wl["min_len"], wl["max_len"])
    cu = syn.cu_from_lengths(lengths)
    N = int(cu[-1])
    x = syn.frontend_inputs(wl["index"], 0, N, Hqk, Hv, d, d, 4, torch.bfloat16)
    pool = torch.zeros((wl["n_slots"], Hv, d, d), dtype=torch.bfloat16, device=DEV)
    rs = torch.full((len(lengths),), -1, dtype=torch.int32)
    ws = torch.from_numpy(np.random.default_rng(3).permutation(wl["n_slots"])[:len(lengths)]
                          .astype(np.int32))
    o = gdn_prefill(dev(cu), dev(x["q_raw"]), dev(x["k_raw"]), dev(x["v_raw"]), pool, dev(rs),
                    dev(ws), H_qk=Hqk, H_v=Hv, a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]),
                    conv_wq=dev(x["conv_wq"]), conv_wk=dev(x["conv_wk"]),
                    conv_wv=dev(x["conv_wv"]))
    torch.cuda.synchronize()
    oc = o.cpu()
    pc = pool.cpu()
    rq, rk, rv, rg, rb = oracle_frontend(cu, x, Hqk, Hv)
    rq, rk, rv = (oracle.round_bf16(t) for t in (rq, rk, rv))  # stored in BF16 before use
    ro, rpool, _ = oracle.sequences(cu.numpy(), rq, rk, rv, rg, rb,
                                    np.zeros((wl["n_slots"], Hv, d, d)), rs.numpy(), ws.numpy(),
                                    round_state=True)
    assert seq_err(f64(oc), ro, cu) < 2e-2
    w = ws.numpy()
    assert scaled_err(f64(pc[w]), rpool[w], 2) < 2e-2

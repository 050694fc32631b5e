"""Chunked prefill with one decay per key channel (Kimi Delta Attention's
channel-wise gate, "Seven Architectures Replacing KV Cache With Bounded
Mutable State", Kimi Linear and Gated DeltaNet-2 sections): the HIP chain
through the C ABI against the oracle's token recurrence with the same gate.

Tolerances are the scalar prefill's: 2e-2 (scaled per slice) when the state
or the outputs are stored in BF16, 1e-4 when every stored value is FP32.  The
channel-wise chain takes FP32 operands whenever the state or the activations
are FP32; that needs d_k <= 64 (LDS), and d_k = 128 is refused."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import GdnError, gdn_decode, gdn_prefill, synthetic as syn
from gpu_util import f64, say, scaled_err, seq_err, state_tol

pytestmark = pytest.mark.gpu
RULES = ["linear", "gated", "delta", "gated_delta"]
DEV = "cuda"


def dev(t):
    return None if t is None else t.to(DEV)


def cw_case(wl, lengths, Hqk, Hv, dk, dv, n_slots, sdt, adt, std=0.02, fresh=(), gates=None):
    """Inputs for sequences of the given lengths with channel-wise gates g
    [N, H_v, d_k], a pool, read slots (indices in `fresh` start from zero) and
    distinct write slots."""
    lengths = list(lengths)
    N = int(sum(lengths))
    cu = syn.cu_from_lengths(lengths)
    q, k, v, _, beta = syn.token_inputs(wl, 0, N, Hqk, Hv, dk, dv, adt)
    g = syn.channel_gates(wl, 0, N, Hv, dk) if gates is None else gates
    pool = syn.state_pool(wl, 0, n_slots, Hv, dk, dv, sdt, std=std)
    rs, ws = syn.distinct_slots(wl, 0, n_slots, len(lengths), in_place=False)
    rs = rs.clone()
    for i in fresh:
        rs[i] = -1
    return cu, q, k, v, g, beta, pool, rs, ws


def run_both(case, rule, scale=1.0, **kw):
    cu, q, k, v, g, beta, pool, rs, ws = case
    N, Hqk, dk = q.shape
    Hv = v.shape[1]
    dpool = dev(pool)
    o = gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), H_qk=Hqk, H_v=Hv,
                    g=dev(g), beta=dev(beta), rule=rule, scale=scale, **kw)
    torch.cuda.synchronize()
    ro, rpool, code = oracle.sequences_cw(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                          f64(pool), None if rs is None else rs.numpy(),
                                          None if ws is None else ws.numpy(), rule=rule,
                                          scale=scale,
                                          round_state=(pool.dtype == torch.bfloat16))
    assert code == 0
    return o, dpool.cpu(), ro, rpool


@pytest.mark.parametrize("rule", RULES)
def test_cw_prefill_bf16_ragged(rule):
    """BF16 activations and state, d = 128, H_qk = 2, H_v = 4; sequences of 1,
    63, 64, 200 tokens (ragged tails, several chunks); one fresh request, the
    others start from a checkpoint slot."""
    say("cw prefill bf16 ragged", rule)
    case = cw_case(301, [1, 63, 64, 200], 2, 4, 128, 128, 12, torch.bfloat16, torch.bfloat16,
                   fresh=(1,))
    o, pool, ro, rpool = run_both(case, rule, scale=128 ** -0.5)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 2e-2
    assert scaled_err(f64(pool)[ws], rpool[ws], 2) < 2e-2


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("dk,dv", [(64, 64), (32, 32), (16, 16)])
def test_cw_prefill_fp32(rule, dk, dv):
    """FP32 activations and state: FP32 MFMA operands throughout, 1e-4."""
    say("cw prefill fp32", rule, dk, dv)
    case = cw_case(302, [130, 1, 64, 77], 2, 4, dk, dv, 12, torch.float32, torch.float32,
                   std=0.3, fresh=(2,))
    o, pool, ro, rpool = run_both(case, rule)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 1e-4
    assert scaled_err(f64(pool)[ws], rpool[ws], 2) < 1e-4


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (32, 64), (16, 32)])
def test_cw_prefill_bf16_fp32_state(dk, dv):
    """BF16 activations on an FP32 state (exact inputs to both sides): FP32
    operands, state within 1e-4, BF16 outputs within 2e-2."""
    say("cw prefill bf16 act fp32 state", dk, dv)
    case = cw_case(303, [200, 33], 2, 4, dk, dv, 6, torch.float32, torch.bfloat16, std=0.1)
    o, pool, ro, rpool = run_both(case, "gated_delta")
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 2e-2
    assert scaled_err(f64(pool)[ws], rpool[ws], 2) < state_tol(torch.float32)


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 32), (64, 128),
                                   (128, 16), (128, 64)])
def test_cw_prefill_shapes_bf16(dk, dv):
    say("cw prefill shapes bf16", dk, dv)
    case = cw_case(304, [70, 129], 1, 2, dk, dv, 6, torch.bfloat16, torch.bfloat16, std=0.1)
    o, pool, ro, rpool = run_both(case, "gated_delta", scale=0.5)
    ws = case[8].numpy()
    assert seq_err(f64(o), ro, case[0]) < 2e-2
    assert scaled_err(f64(pool)[ws], rpool[ws], 2) < 2e-2


def test_cw_prefill_fp32_d128_refused():
    """FP32 operands at d_k = 128 do not fit the chain's LDS: the call is
    refused before any launch and the pool is left alone."""
    say("cw prefill fp32 d128 refused")
    case = cw_case(305, [10], 1, 1, 128, 128, 2, torch.float32, torch.float32)
    cu, q, k, v, g, beta, pool, rs, ws = case
    dpool = dev(pool)
    with pytest.raises(GdnError):
        gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), H_qk=1, H_v=1,
                    g=dev(g), beta=dev(beta))
    torch.cuda.synchronize()
    assert torch.equal(dpool.cpu(), pool)


def extreme_gates(N, Hv, dk, seed):
    """Channel gates with hard cases side by side in every head: channels
    that never decay (g = 0), channels that forget almost everything each
    token (g = -40: the cumulative decay over a chunk underflows FP32),
    channels that switch between the two, and ordinary ones."""
    r = np.random.default_rng(seed)
    g = -np.logaddexp(0.0, r.standard_normal((N, Hv, dk)))
    g[:, :, 0::4] = 0.0
    g[:, :, 1::4] = -40.0
    flip = r.random((N, Hv, dk // 4)) < 0.5
    g[:, :, 2::4] = np.where(flip, 0.0, -40.0)
    return torch.from_numpy(g).float()


@pytest.mark.parametrize("d,sdt,adt,bar", [(128, torch.bfloat16, torch.bfloat16, 2e-2),
                                           (64, torch.float32, torch.float32, 1e-4)])
def test_cw_prefill_extreme_gates(d, sdt, adt, bar):
    say("cw prefill extreme gates", d)
    lengths = [150, 64, 3]
    gates = extreme_gates(sum(lengths), 2, d, 306)
    case = cw_case(306, lengths, 1, 2, d, d, 8, sdt, adt, std=0.3, gates=gates)
    for rule in ("gated", "gated_delta"):
        o, pool, ro, rpool = run_both(case, rule)
        ws = case[8].numpy()
        assert np.all(np.isfinite(f64(o))) and np.all(np.isfinite(f64(pool)))
        assert seq_err(f64(o), ro, case[0]) < bar, rule
        assert scaled_err(f64(pool)[ws], rpool[ws], 2) < bar, rule


@pytest.mark.parametrize("d,sdt,bar", [(128, torch.bfloat16, 2e-2), (32, torch.float32, 1e-4)])
def test_cw_prefill_equal_channels_is_the_scalar_gate(d, sdt, bar):
    """Channel gates that are equal across a head's channels are Gated
    DeltaNet's scalar gate: the channel-wise chain matches the oracle's scalar
    recurrence."""
    say("cw prefill equal channels", d)
    lengths = [100, 64]
    N = sum(lengths)
    q, k, v, g, beta = syn.token_inputs(307, 0, N, 1, 2, d, d, sdt)
    gates = g[:, :, None].expand(N, 2, d).contiguous()
    case = cw_case(307, lengths, 1, 2, d, d, 6, sdt, sdt, gates=gates)
    cu, _, _, _, _, _, pool, rs, ws = case
    case = (cu, q, k, v, gates, beta, pool, rs, ws)
    o, dpool, _, _ = run_both(case, "gated_delta")
    ro, rpool, _ = oracle.sequences(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                    f64(pool), rs.numpy(), ws.numpy(),
                                    round_state=(sdt == torch.bfloat16))
    w = ws.numpy()
    assert seq_err(f64(o), ro, cu) < bar
    assert scaled_err(f64(dpool)[w], rpool[w], 2) < bar


@pytest.mark.parametrize("d,dt,bar,interval", [(128, torch.bfloat16, 2e-2, 64),
                                               (128, torch.bfloat16, 2e-2, 128),
                                               (32, torch.float32, 1e-4, 64)])
def test_cw_prefill_checkpoints(d, dt, bar, interval):
    """Intermediate checkpoints: slot [s, j] holds sequence s's state after
    its first (j + 1) * interval tokens (the oracle run on that prefix);
    slots past a sequence's end and -1 entries are left alone."""
    say("cw prefill checkpoints", d, interval)
    lengths = [300, 128, 64, 65, 0, 1, 256]
    per_seq = 4
    n_seq = len(lengths)
    n_slots = 2 * n_seq + n_seq * per_seq + 4
    case = cw_case(308, lengths, 1, 2, d, d, n_slots, dt, dt, std=0.1, fresh=(0,))
    cu, q, k, v, g, beta, pool, rs, ws = case
    used = set(rs.tolist()) | set(ws.tolist())
    free = [s for s in np.random.default_rng(308).permutation(n_slots) if s not in used]
    ck = np.array(free[:n_seq * per_seq], np.int32).reshape(n_seq, per_seq)
    ck[0, 1] = -1
    o, dpool, ro, rpool = run_both(case, "gated_delta", ckpt_interval=interval,
                                   ckpt_slot=dev(torch.from_numpy(ck)))
    rnd = dt == torch.bfloat16
    assert seq_err(f64(o), ro, cu) < bar
    assert scaled_err(f64(dpool)[ws.numpy()], rpool[ws.numpy()], 2) < bar
    got = f64(dpool)
    written = []
    for s_, L in enumerate(lengths):
        for j in range(per_seq):
            n, slot = (j + 1) * interval, int(ck[s_, j])
            if slot < 0 or n > L:
                continue
            a, b = int(cu[s_]), int(cu[s_]) + n
            _, ppool, c2 = oracle.sequences_cw(np.array([0, n], np.int32), f64(q[a:b]),
                                               f64(k[a:b]), f64(v[a:b]), f64(g[a:b]),
                                               f64(beta[a:b]), f64(pool), rs.numpy()[s_:s_ + 1],
                                               np.array([slot], np.int32), round_state=rnd)
            assert c2 == 0
            assert scaled_err(got[slot], ppool[slot], 2) < bar, (s_, j)
            written.append(slot)
    assert len(written) > 0
    untouched = np.setdiff1d(np.arange(n_slots), np.concatenate([ws.numpy(), written]))
    assert torch.equal(dpool[untouched], pool[untouched])


def test_cw_prefill_bad_slot_and_empty_sequences():
    """An out-of-range slot skips its sequence (status bit set, its outputs and
    write slot left alone); an empty sequence stores its read state; the other
    sequences are unaffected."""
    say("cw prefill bad slot / empty")
    case = cw_case(309, [40, 0, 70, 5], 1, 2, 64, 64, 10, torch.bfloat16, torch.bfloat16,
                   std=0.3)
    cu, q, k, v, g, beta, pool, rs, ws = case
    rs = rs.clone()
    rs[3] = 10  # one past the pool
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    dpool = dev(pool)
    o = torch.full((115, 2, 64), 5.0, dtype=torch.bfloat16, device=DEV)
    gdn_prefill(dev(cu), dev(q), dev(k), dev(v), dpool, dev(rs), dev(ws), o, H_qk=1, H_v=2,
                g=dev(g), beta=dev(beta), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) & 1
    assert torch.all(o[110:].cpu() == 5.0)
    ro, rpool, code = oracle.sequences_cw(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                          f64(pool), rs.numpy(), ws.numpy(), round_state=True)
    assert code == 1
    assert seq_err(f64(o[:110]), ro[:110], cu[:4]) < 2e-2
    got = f64(dpool)
    w = ws.numpy()
    assert scaled_err(got[w[:3]], rpool[w[:3]], 2) < 2e-2
    assert torch.equal(dpool.cpu()[int(w[3])], pool[int(w[3])])  # skipped: nothing stored
    assert np.array_equal(got[int(w[1])], f64(pool)[int(rs[1])])  # empty: the read state


def test_cw_prefill_then_decode_equals_longer_prefill():
    """prefill(T1) with channel gates into a slot, then T2 channel-gated decode
    steps from it, equals the oracle's run over T1 + T2 tokens (FP32)."""
    say("cw prefill then decode")
    T1, T2, Hqk, Hv, d = 130, 5, 1, 2, 64
    q, k, v, _, beta = syn.token_inputs(310, 0, T1 + T2, Hqk, Hv, d, d, torch.float32)
    g = syn.channel_gates(310, 0, T1 + T2, Hv, d)
    pool = torch.zeros((2, Hv, d, d), dtype=torch.float32, device=DEV)
    s0 = torch.tensor([-1], dtype=torch.int32, device=DEV)
    s1 = torch.tensor([1], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, T1], dtype=torch.int32, device=DEV)
    outs = [gdn_prefill(cu, dev(q[:T1]), dev(k[:T1]), dev(v[:T1]), pool, s0, s1, H_qk=Hqk,
                        H_v=Hv, g=dev(g[:T1]), beta=dev(beta[:T1]))]
    for t in range(T1, T1 + T2):
        outs.append(gdn_decode(dev(q[t:t + 1]), dev(k[t:t + 1]), dev(v[t:t + 1]),
                               dev(g[t:t + 1]), dev(beta[t:t + 1]), pool, s1, s1))
    torch.cuda.synchronize()
    ro, rpool, _ = oracle.sequences_cw(np.array([0, T1 + T2], np.int32), f64(q), f64(k), f64(v),
                                       f64(g), f64(beta), np.zeros((1, Hv, d, d)), [0], [0])
    assert seq_err(f64(torch.cat(outs)), ro, [0, T1 + T2]) < 1e-4
    assert scaled_err(f64(pool)[1:2], rpool, 2) < 1e-4


def test_cw_prefill_varlen_full_size():
    """The chunked-prefill workload's shapes (8 sequences of 1024..8192
    tokens, H_qk = 16, H_v = 32, d = 128, BF16, fresh requests into 8 slots of
    a 64-slot pool) with channel gates in place of the front-end's scalar
    gate, every state head of every sequence against the oracle."""
    say("cw prefill_varlen full size")
    wl = syn.WORKLOADS["prefill_varlen"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lengths = syn.seq_lengths(wl["index"], 0, wl["n_seq"], wl["min_len"], wl["max_len"])
    cu = syn.cu_from_lengths(lengths)
    N = int(cu[-1])
    q, k, v, _, beta = syn.token_inputs(wl["index"], 0, N, Hqk, Hv, d, d, torch.bfloat16)
    g = syn.channel_gates(wl["index"], 0, N, Hv, d)
    pool = torch.zeros((wl["n_slots"], Hv, d, d), dtype=torch.bfloat16, device=DEV)
    rs = torch.full((len(lengths),), -1, dtype=torch.int32)
    ws = torch.from_numpy(np.random.default_rng(3).permutation(wl["n_slots"])[:len(lengths)]
                          .astype(np.int32))
    o = gdn_prefill(dev(cu), dev(q), dev(k), dev(v), pool, dev(rs), dev(ws), H_qk=Hqk, H_v=Hv,
                    g=dev(g), beta=dev(beta), scale=d ** -0.5)
    torch.cuda.synchronize()
    ro, rpool, _ = oracle.sequences_cw(cu.numpy(), f64(q), f64(k), f64(v), f64(g), f64(beta),
                                       np.zeros((wl["n_slots"], Hv, d, d)), rs.numpy(),
                                       ws.numpy(), scale=d ** -0.5, round_state=True)
    assert seq_err(f64(o), ro, cu) < 2e-2
    w = ws.numpy()
    assert scaled_err(f64(pool.cpu()[w]), rpool[w], 2) < 2e-2


@pytest.mark.parametrize("d,sdt,bar", [(128, torch.bfloat16, 2e-2), (64, torch.float32, 1e-4)])
@pytest.mark.parametrize("g_fast", [-4.5, -4.7])
def test_cw_prefill_diagonal_span_at_the_limit(d, sdt, bar, g_fast):
    """Diagonal tiles whose decay span sits just inside (g = -4.5 per token:
    15 * 4.5 * log2(e) = 97.4 < 100, column factors up to 2^97 in the scaled
    product) or just outside (g = -4.7: 101.7, the entry-by-entry form) the
    limit of the scaled MFMA product, beside channels that do not decay."""
    say("cw prefill diagonal span", d, g_fast)
    lengths = [130, 64]
    N = sum(lengths)
    g = np.zeros((N, 2, d))
    g[:, :, 0::3] = g_fast
    g[:, :, 1::3] = -np.logaddexp(0.0, np.random.default_rng(311).standard_normal((N, 2, d))[:, :, 1::3])
    case = cw_case(311, lengths, 1, 2, d, d, 6, sdt, sdt, std=0.3,
                   gates=torch.from_numpy(g).float())
    o, pool, ro, rpool = run_both(case, "gated_delta")
    ws = case[8].numpy()
    assert np.all(np.isfinite(f64(o)))
    assert seq_err(f64(o), ro, case[0]) < bar
    assert scaled_err(f64(pool)[ws], rpool[ws], 2) < bar

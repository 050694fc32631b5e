"""Mixed decode + prefill batches in one launch: results equal the separate
gdn_decode and gdn_prefill calls bit for bit (the same device code runs), and
match the FP64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_recurrent_02_amd import (gdn_decode, gdn_mixed, gdn_prefill,
                                               make_decode_args, make_prefill_args,
                                               synthetic as syn)
from gpu_util import f64, say, scaled_err, seq_err

pytestmark = pytest.mark.gpu
RULES = ["linear", "gated", "delta", "gated_delta"]
DEV = "cuda"


def dev(t):
    return None if t is None else t.to(DEV)


def build(wl, n_dec, lengths, Hqk, Hv, d, n_slots, frontend, std=0.02, sdt=torch.bfloat16):
    q, k, v, g, beta = (dev(t) for t in syn.token_inputs(wl, 1, n_dec, Hqk, Hv, d, d))
    pool = syn.state_pool(wl, 0, n_slots, Hv, d, d, sdt, std=std)
    drs, dws, prs, pws = syn.mixed_slots(wl, n_dec, len(lengths), n_slots)
    cu = syn.cu_from_lengths(lengths)
    N = int(cu[-1])
    if frontend:
        x = syn.frontend_inputs(wl, 2, N, Hqk, Hv, d, d, 4, torch.bfloat16)
        pin = dict(q=x["q_raw"], k=x["k_raw"], v=x["v_raw"],
                   kw=dict(a_raw=dev(x["a_raw"]), b_raw=dev(x["b_raw"]), conv_wq=dev(x["conv_wq"]),
                           conv_wk=dev(x["conv_wk"]), conv_wv=dev(x["conv_wv"])), raw=x)
    else:
        pq, pk, pv, pg, pb = syn.token_inputs(wl, 2, N, Hqk, Hv, d, d)
        pin = dict(q=pq, k=pk, v=pv, kw=dict(g=dev(pg), beta=dev(pb)), final=(pq, pk, pv, pg, pb))
    return dict(dec=(q, k, v, g, beta), pool=pool, drs=drs, dws=dws, prs=prs, pws=pws, cu=cu,
                pin=pin, Hqk=Hqk, Hv=Hv)


def run_mixed(c, rule):
    pool = dev(c["pool"])
    q, k, v, g, beta = c["dec"]
    da, do, dkeep = make_decode_args(q, k, v, g, beta, pool, dev(c["drs"]), dev(c["dws"]), rule=rule)
    pa, po, pkeep = make_prefill_args(dev(c["cu"]), dev(c["pin"]["q"]), dev(c["pin"]["k"]),
                                      dev(c["pin"]["v"]), pool, dev(c["prs"]), dev(c["pws"]),
                                      H_qk=c["Hqk"], H_v=c["Hv"], **c["pin"]["kw"])
    gdn_mixed(da, pa)
    torch.cuda.synchronize()
    return do, po, pool


def run_separate(c, rule):
    pool = dev(c["pool"])
    q, k, v, g, beta = c["dec"]
    do = gdn_decode(q, k, v, g, beta, pool, dev(c["drs"]), dev(c["dws"]), rule=rule)
    po = gdn_prefill(dev(c["cu"]), dev(c["pin"]["q"]), dev(c["pin"]["k"]), dev(c["pin"]["v"]),
                     pool, dev(c["prs"]), dev(c["pws"]), H_qk=c["Hqk"], H_v=c["Hv"],
                     **c["pin"]["kw"])
    torch.cuda.synchronize()
    return do, po, pool


@pytest.mark.parametrize("rule", RULES)
def test_mixed_equals_separate_and_oracle(rule):
    say("mixed small", rule)
    c = build(401, 9, [70, 130, 1], 2, 4, 128, 48, frontend=False, std=0.05)
    do, po, pool = run_mixed(c, rule)
    so, spo, spool = run_separate(c, rule)
    assert torch.equal(do, so) and torch.equal(po, spo)
    assert torch.equal(pool.view(torch.int16), spool.view(torch.int16))
    # oracle: decode half with `rule`, prefill half gated_delta, on the shared pool
    q, k, v, g, beta = c["dec"]
    ro, rpool, _ = oracle.decode(f64(q), f64(k), f64(v), f64(g), f64(beta), f64(c["pool"]),
                                 c["drs"].numpy(), c["dws"].numpy(), rule=rule, round_state=True)
    pq, pk, pv, pg, pb = c["pin"]["final"]
    rpo, rpool, _ = oracle.sequences(c["cu"].numpy(), f64(pq), f64(pk), f64(pv), f64(pg), f64(pb),
                                     rpool, c["prs"].numpy(), c["pws"].numpy(), round_state=True)
    assert scaled_err(f64(do), ro, 2) < 2e-2
    assert seq_err(f64(po), rpo, c["cu"]) < 2e-2
    w = np.concatenate([c["dws"].numpy(), c["pws"].numpy()])
    assert scaled_err(f64(pool)[w], rpool[w], 2) < 2e-2
    untouched = np.setdiff1d(np.arange(48), w)
    assert torch.equal(pool.cpu()[untouched].view(torch.int16),
                       c["pool"][untouched].view(torch.int16))


def test_mixed_fp32_state_equals_separate():
    """FP32 state pool with BF16 activations at d = 128: the mixed launch runs
    4-wave blocks (plain chains) while gdn_prefill runs the pipelined chain;
    the two chains compute the same products in the same order, so the
    results still equal the separate calls bit for bit."""
    say("mixed fp32 state")
    c = build(404, 7, [70, 130, 1], 2, 4, 128, 48, frontend=False, std=0.05, sdt=torch.float32)
    do, po, pool = run_mixed(c, "gated_delta")
    so, spo, spool = run_separate(c, "gated_delta")
    assert torch.equal(do, so) and torch.equal(po, spo)
    assert torch.equal(pool, spool)


def test_mixed_checkpoints_equal_separate():
    """Intermediate prefill checkpoints (every 64 tokens) through the mixed
    launch land exactly where gdn_prefill puts them."""
    say("mixed checkpoints")
    c = build(405, 9, [70, 130, 1], 2, 4, 128, 64, frontend=False, std=0.05)
    used = set(c["drs"].tolist()) | set(c["dws"].tolist()) | set(c["prs"].tolist()) | set(c["pws"].tolist())
    free = [x for x in range(64) if x not in used]
    ck = torch.tensor(free[:6], dtype=torch.int32).reshape(3, 2)
    c["pin"]["kw"] = dict(c["pin"]["kw"], ckpt_interval=64, ckpt_slot=dev(ck))
    do, po, pool = run_mixed(c, "gated_delta")
    so, spo, spool = run_separate(c, "gated_delta")
    assert torch.equal(do, so) and torch.equal(po, spo)
    assert torch.equal(pool.view(torch.int16), spool.view(torch.int16))
    # sequence 1 (130 tokens) reached checkpoints at 64 and 128, sequence 0 at 64
    for slot in (int(ck[0, 0]), int(ck[1, 0]), int(ck[1, 1])):
        assert not torch.equal(pool[slot].cpu(), c["pool"][slot])


def test_mixed_one_half_empty():
    say("mixed empty halves")
    c = build(402, 6, [90], 1, 2, 64, 16, frontend=False, std=0.05)
    pool = dev(c["pool"])
    q, k, v, g, beta = c["dec"]
    z = lambda t: t[:0]
    da, do, _ = make_decode_args(z(q), z(k), z(v), z(g), z(beta), pool)
    pa, po, pk = make_prefill_args(dev(c["cu"]), dev(c["pin"]["q"]), dev(c["pin"]["k"]),
                                   dev(c["pin"]["v"]), pool, dev(c["prs"]), dev(c["pws"]),
                                   H_qk=1, H_v=2, **c["pin"]["kw"])
    gdn_mixed(da, pa)
    spool = dev(c["pool"])
    spo = gdn_prefill(dev(c["cu"]), dev(c["pin"]["q"]), dev(c["pin"]["k"]), dev(c["pin"]["v"]),
                      spool, dev(c["prs"]), dev(c["pws"]), H_qk=1, H_v=2, **c["pin"]["kw"])
    torch.cuda.synchronize()
    assert torch.equal(po, spo) and torch.equal(pool, spool)
    da, do, _ = make_decode_args(q, k, v, g, beta, pool, dev(c["drs"]), dev(c["dws"]))
    empty_cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    e = torch.empty((0, 1, 64), dtype=torch.bfloat16, device=DEV)
    pa, _, _ = make_prefill_args(empty_cu, e, e, torch.empty((0, 2, 64), dtype=torch.bfloat16,
                                                             device=DEV), pool, H_qk=1, H_v=2)
    gdn_mixed(da, pa)
    so = gdn_decode(q, k, v, g, beta, spool, dev(c["drs"]), dev(c["dws"]))
    torch.cuda.synchronize()
    assert torch.equal(do, so) and torch.equal(pool, spool)


def test_mixed_uneven_workers():
    """Decode workers of one block with different tile counts: 200 short
    prefills (one state head each) leave the decode half its minimum of a
    quarter of the CUs, and 131 decode tiles over those workers give the first
    few two tiles and the rest one, so one worker of a block ends while its
    partner still reduces.  Mixed = separate bit for bit."""
    say("mixed uneven decode workers")
    lengths = np.random.default_rng(11).integers(1, 81, size=200)
    c = build(403, 131, lengths, 1, 1, 128, 512, frontend=False, std=0.05)
    for rule in ("gated_delta", "linear"):
        do, po, pool = run_mixed(c, rule)
        so, spo, spool = run_separate(c, rule)
        assert torch.equal(do, so) and torch.equal(po, spo), rule
        assert torch.equal(pool.view(torch.int16), spool.view(torch.int16)), rule


def test_mixed_full_size_sampled():
    """448 decode requests (each update rule on a quarter of them would need four
    calls; here all four rules run back to back on the same pool state) plus 4
    prefills of 8192 tokens through the fused front-end, one 1024-slot BF16 pool,
    25% of the requests reading a checkpoint slot.  Mixed = separate bit for bit;
    the oracle checks 16 sampled decode requests and two heads of every prefill."""
    wl = syn.WORKLOADS["mixed"]
    Hqk, Hv, d = wl["H_qk"], wl["H_v"], wl["d_k"]
    lengths = [wl["prefill_len"]] * wl["n_prefill"]
    c = build(wl["index"], wl["n_decode"], lengths, Hqk, Hv, d, wl["n_slots"], frontend=True)
    for rule in RULES:
        say("mixed full size", rule)
        do, po, pool = run_mixed(c, rule)
        so, spo, spool = run_separate(c, rule)
        assert torch.equal(do, so) and torch.equal(po, spo), rule
        assert torch.equal(pool.view(torch.int16), spool.view(torch.int16)), rule
        sample = np.random.default_rng(7).choice(wl["n_decode"], 16, replace=False)
        q, k, v, g, beta = (t[sample].cpu() for t in c["dec"])
        rs = c["drs"].numpy()[sample]
        ro, _, _ = oracle.decode(f64(q), f64(k), f64(v), f64(g), f64(beta),
                                 f64(c["pool"][torch.from_numpy(np.maximum(rs, 0)).long()]),
                                 np.where(rs >= 0, np.arange(16), -1).astype(np.int32),
                                 np.full(16, -1, np.int32), rule=rule, round_state=True)
        assert scaled_err(f64(do.cpu()[sample]), ro, 2) < 2e-2, rule
    # prefill half (gated_delta) on two heads, initial states from the pool
    x = c["pin"]["raw"]
    cu = c["cu"]
    pc = po.cpu()
    pool_after = pool.cpu()
    for j in (0, 9):
        hs = [2 * j, 2 * j + 1]
        qs, vs = slice(j * d, (j + 1) * d), slice(2 * j * d, (2 * j + 2) * d)
        rq, rk, rv, rg, rb = oracle.frontend(cu.numpy(), f64(x["q_raw"][:, qs]),
                                             f64(x["k_raw"][:, qs]), f64(x["v_raw"][:, vs]),
                                             f64(x["conv_wq"][qs]), f64(x["conv_wk"][qs]),
                                             f64(x["conv_wv"][vs]), f64(x["a_raw"][:, hs]),
                                             f64(x["b_raw"][:, hs]), Hqk=1, Hv=2)
        rq, rk, rv = (oracle.round_bf16(t) for t in (rq, rk, rv))
        sub_pool = f64(c["pool"][:, hs])
        rpo, rpool, _ = oracle.sequences(cu.numpy(), rq, rk, rv, rg, rb, sub_pool,
                                         c["prs"].numpy(), c["pws"].numpy(), round_state=True)
        assert seq_err(f64(pc[:, hs]), rpo, cu) < 2e-2, j
        w = c["pws"].numpy()
        assert scaled_err(f64(pool_after[w][:, hs]), rpool[w], 2) < 2e-2, j

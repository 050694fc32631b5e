"""The Python binding's own checks, on CPU tensors: a wrong dtype or shape is
rejected with ValueError before anything reaches the library (a float32 tap
read as BF16, or an int64 slot read as int32, would otherwise read past the
tensor), and a well-formed call on host tensors is refused for its placement."""
import pytest
import torch

from linear_attention_recurrent_02_amd import gdn

B, HQK, HV, D = 3, 2, 4, 16


def decode_tensors(**over):
    t = dict(q=torch.zeros(B, HQK, D, dtype=torch.bfloat16),
             k=torch.zeros(B, HQK, D, dtype=torch.bfloat16),
             v=torch.zeros(B, HV, D, dtype=torch.bfloat16),
             g=torch.zeros(B, HV), beta=torch.zeros(B, HV),
             state_pool=torch.zeros(5, HV, D, D, dtype=torch.bfloat16),
             read_slot=torch.zeros(B, dtype=torch.int32),
             write_slot=torch.zeros(B, dtype=torch.int32))
    t.update(over)
    return t


def call_decode(t):
    return gdn.make_decode_args(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state_pool"],
                                t["read_slot"], t["write_slot"], t.get("o"),
                                status=t.get("status"))


@pytest.mark.parametrize("over,what", [
    (dict(g=torch.zeros(B, HV, dtype=torch.bfloat16)), "g must be torch.float32"),
    (dict(beta=torch.zeros(B, HV, dtype=torch.float64)), "beta must be torch.float32"),
    (dict(read_slot=torch.zeros(B, dtype=torch.int64)), "read_slot must be torch.int32"),
    (dict(write_slot=torch.zeros(B + 1, dtype=torch.int32)), "write_slot must have shape"),
    (dict(g=torch.zeros(B, HV, 1)), "g must have shape"),
    (dict(g=torch.zeros(B, HV, D + 1)), "g must have shape"),
    (dict(state_pool=torch.zeros(5, HV, D, D + 16, dtype=torch.bfloat16)), "state_pool must be"),
    (dict(state_pool=torch.zeros(5, HV, D, D, dtype=torch.float16)), "state_pool must be one of"),
    (dict(k=torch.zeros(B, HQK, D)), "k must be torch.bfloat16"),
    (dict(v=torch.zeros(B + 1, HV, D, dtype=torch.bfloat16)), "v must be"),
    (dict(o=torch.zeros(B, HV, D)), "o must be torch.bfloat16"),
    (dict(o=torch.zeros(B, HV, D + 1, dtype=torch.bfloat16)), "o must have shape"),
    (dict(status=torch.zeros(2, dtype=torch.int32)), "status must have shape"),
])
def test_decode_rejects(over, what):
    with pytest.raises(ValueError, match=what):
        call_decode(decode_tensors(**over))


def test_decode_well_formed_host_tensors_refused_for_placement():
    with pytest.raises(ValueError, match="device tensor"):
        call_decode(decode_tensors())
    # a per-key-channel decay of the right shape passes the shape checks
    with pytest.raises(ValueError, match="device tensor"):
        call_decode(decode_tensors(g=torch.zeros(B, HV, D)))


N = 10


def prefill_tensors(**over):
    t = dict(cu=torch.tensor([0, 4, N], dtype=torch.int32),
             q=torch.zeros(N, HQK * D, dtype=torch.bfloat16),
             k=torch.zeros(N, HQK * D, dtype=torch.bfloat16),
             v=torch.zeros(N, HV * D, dtype=torch.bfloat16),
             state_pool=torch.zeros(4, HV, D, D, dtype=torch.bfloat16),
             read_slot=torch.zeros(2, dtype=torch.int32),
             write_slot=torch.ones(2, dtype=torch.int32),
             a_raw=torch.zeros(N, HV), b_raw=torch.zeros(N, HV),
             conv_wq=torch.zeros(HQK * D, 4), conv_wk=torch.zeros(HQK * D, 4),
             conv_wv=torch.zeros(HV * D, 4))
    t.update(over)
    return t


def call_prefill(t):
    keys = ("a_raw", "b_raw", "conv_wq", "conv_wk", "conv_wv", "g", "beta", "ckpt_slot",
            "status")
    kw = {k: t[k] for k in keys if k in t}
    return gdn.make_prefill_args(t["cu"], t["q"], t["k"], t["v"], t["state_pool"],
                                 t["read_slot"], t["write_slot"], t.get("o"), H_qk=HQK, H_v=HV,
                                 **kw)


@pytest.mark.parametrize("over,what", [
    (dict(cu=torch.tensor([0, 4, N], dtype=torch.int64)), "cu_seqlens must be torch.int32"),
    (dict(conv_wq=torch.zeros(HQK * D, 4, dtype=torch.bfloat16)), "conv_wq must be torch.float32"),
    (dict(conv_wv=torch.zeros(HV * D + 8, 4)), "conv_wv must have shape"),
    (dict(conv_wk=torch.zeros(HQK * D, 3)), "conv_wk must have shape"),
    (dict(a_raw=torch.zeros(N, HV, dtype=torch.bfloat16)), "a_raw must be torch.float32"),
    (dict(b_raw=torch.zeros(N, HV + 1)), "b_raw must have shape"),
    (dict(read_slot=torch.zeros(2, dtype=torch.int64)), "read_slot must be torch.int32"),
    (dict(write_slot=torch.zeros(3, dtype=torch.int32)), "write_slot must have shape"),
    (dict(q=torch.zeros(N, HQK * D + 1, dtype=torch.bfloat16)), "q must be"),
    (dict(v=torch.zeros(N, HV * D)), "v must be torch.bfloat16"),
    (dict(state_pool=torch.zeros(4, HV, D, 2 * D, dtype=torch.bfloat16)), "state_pool must be"),
    (dict(g=torch.zeros(N, HV, dtype=torch.float16)), "g must be torch.float32"),
    (dict(ckpt_slot=torch.zeros(3, 2, dtype=torch.int32)), "ckpt_slot must be"),
    (dict(ckpt_slot=torch.zeros(2, 2, dtype=torch.int64)), "ckpt_slot must be torch.int32"),
    (dict(o=torch.zeros(N, HV, D + 1, dtype=torch.bfloat16)), "o must have shape"),
])
def test_prefill_rejects(over, what):
    with pytest.raises(ValueError, match=what):
        call_prefill(prefill_tensors(**over))


def test_prefill_well_formed_host_tensors_refused_for_placement():
    with pytest.raises(ValueError, match="device tensor"):
        call_prefill(prefill_tensors())
    # [N, H, d] activations are accepted as well as [N, H * d]
    with pytest.raises(ValueError, match="device tensor"):
        call_prefill(prefill_tensors(q=torch.zeros(N, HQK, D, dtype=torch.bfloat16),
                                     k=torch.zeros(N, HQK, D, dtype=torch.bfloat16)))


C = 2 * HQK * D + HV * D


def conv_tensors(**over):
    t = dict(q_raw=torch.zeros(B, HQK * D, dtype=torch.bfloat16),
             k_raw=torch.zeros(B, HQK * D, dtype=torch.bfloat16),
             v_raw=torch.zeros(B, HV * D, dtype=torch.bfloat16),
             conv_pool=torch.zeros(6, 3, C, dtype=torch.bfloat16),
             read_slot=torch.zeros(B, dtype=torch.int32),
             write_slot=torch.ones(B, dtype=torch.int32),
             a_raw=torch.zeros(B, HV), b_raw=torch.zeros(B, HV),
             conv_wq=torch.zeros(HQK * D, 4), conv_wk=torch.zeros(HQK * D, 4),
             conv_wv=torch.zeros(HV * D, 4))
    t.update(over)
    return t


def call_conv(t):
    return gdn.gdn_conv_decode(t["q_raw"], t["k_raw"], t["v_raw"], t["conv_pool"], t["read_slot"],
                               t["write_slot"], H_qk=HQK, H_v=HV, conv_wq=t["conv_wq"],
                               conv_wk=t["conv_wk"], conv_wv=t["conv_wv"], a_raw=t["a_raw"],
                               b_raw=t["b_raw"])


@pytest.mark.parametrize("over,what", [
    (dict(conv_pool=torch.zeros(6, 3, C + 8, dtype=torch.bfloat16)), "conv_pool must have"),
    (dict(conv_pool=torch.zeros(6, 3, C)), "conv_pool must be torch.bfloat16"),
    (dict(conv_pool=torch.zeros(6, C, dtype=torch.bfloat16)), "conv_pool must be"),
    (dict(conv_wv=torch.zeros(HV * D, 4, dtype=torch.bfloat16)), "conv_wv must be torch.float32"),
    (dict(conv_wq=torch.zeros(HQK * D, 3)), "conv_wq must have shape"),
    (dict(read_slot=torch.zeros(B, dtype=torch.int64)), "read_slot must be torch.int32"),
    (dict(a_raw=torch.zeros(B, HV, dtype=torch.float64)), "a_raw must be torch.float32"),
    (dict(b_raw=torch.zeros(B + 2, HV)), "b_raw must have shape"),
])
def test_conv_rejects(over, what):
    with pytest.raises(ValueError, match=what):
        call_conv(conv_tensors(**over))


def test_conv_store_rejects_int64_offsets():
    t = conv_tensors()
    with pytest.raises(ValueError, match="cu_seqlens must be torch.int32"):
        gdn.gdn_conv_store(torch.tensor([0, 1, 3], dtype=torch.int64), t["q_raw"], t["k_raw"],
                           t["v_raw"], t["conv_pool"], torch.zeros(2, dtype=torch.int32),
                           H_qk=HQK, H_v=HV)


def test_conv_well_formed_host_tensors_refused_for_placement():
    with pytest.raises(ValueError, match="device tensor"):
        call_conv(conv_tensors())

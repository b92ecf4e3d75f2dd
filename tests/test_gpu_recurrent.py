"""Parity of the HIP recurrent / decode kernel with oracle R (GPU)."""
import numpy as np
import pytest

from kda_workloads import make_config, make_inputs
from tests.conftest import rel_err
from tests.gpu_util import TOL, pick, run_oracle, run_recurrent, say, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
def test_tiny_f32_recurrent(mode):
    """Single head, T=64, d=16, fp32: max|do|/rms(o) <= 1e-4."""
    w = make_config("tiny_f32", mode=mode, gate_law="softplus" if mode != "none" else "zero")
    say("tiny_f32 recurrent", mode)
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    assert rel_err(o, o_r) <= 1e-4 and rel_err(hT, h_r) <= 1e-4, (rel_err(o, o_r), rel_err(hT, h_r))


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
def test_decode_full_size(mode):
    """Decode step at batch 256, H=32, d=128 (bf16 q/k/v, fp32 state in place),
    every (b, h) compared."""
    over = {} if mode == "channel" else dict(mode=mode, gate_law="softplus" if mode == "scalar" else "zero")
    w = make_config("decode_b256_h32", **over)
    say("decode_b256_h32", mode)
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    eo, eh = rel_err(o, o_r), rel_err(hT, h_r)
    print(f"[parity] decode_b256_h32 {mode} o {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (eo, eh)


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (16, 128), (32, 64), (64, 32), (128, 16), (128, 128)])
def test_shapes_f32(Dk, Dv):
    w = make_inputs(2, 9, 3, Dk, Dv, dtype="f32", seed=Dk * 1000 + Dv, h0_std=0.2)
    say("recurrent f32 shape", Dk, Dv)
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    assert rel_err(o, o_r) <= 1e-4 and rel_err(hT, h_r) <= 1e-4


@pytest.mark.parametrize("T", [2, 3, 4, 5, 7, 300])
def test_multi_token_lengths_f32(T):
    """Multi-token sequences of every length modulo the three input slots
    the kernel rotates (and one of 300 tokens): each token's inputs are
    requested three token steps ahead, the last token's again past the end."""
    w = make_inputs(2, T, 2, 64, 64, dtype="f32", seed=300 + T, h0_std=0.2)
    say("recurrent f32 multi-token T", T)
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    eo, eh = rel_err(o, o_r), rel_err(hT, h_r)
    print(f"[parity] recurrent multi-token T{T} o {eo:.3e} state {eh:.3e}", flush=True)
    assert eo <= 1e-4 and eh <= 1e-4, (eo, eh)


def test_multi_token_bf16():
    w = make_inputs(2, 37, 3, 128, 128, dtype="bf16", seed=11, gate_shift=-2.0, h0_std=0.05)
    say("recurrent bf16 T=37")
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    assert rel_err(o, o_r) <= TOL["bf16"] and rel_err(hT, h_r) <= TOL["bf16"]


def test_unnormalised_keys_and_hard_forget_f32():
    w = make_inputs(1, 20, 2, 64, 64, dtype="f32", seed=12, normalise_k=False, h0_std=0.3)
    w.g[:, 5:8] = -30.0           # hard forget on three tokens
    w.g[:, 12, :, ::3] = 0.0      # exact keep on some channels
    say("recurrent unnormalised keys + hard forget")
    o, hT = run_recurrent(w)
    o_r, h_r = run_oracle(w)
    assert rel_err(o, o_r) <= 1e-4 and rel_err(hT, h_r) <= 1e-4


def test_state_handoff_and_determinism():
    """T1 + T2 tokens in two calls equal one call (the same kernel per token:
    bit-identical), and two identical calls give identical bits."""
    import torch
    import gated_delta_rule_17_amd as K
    w = make_inputs(2, 12, 4, 128, 128, dtype="bf16", seed=13, h0_std=0.05)
    d = to_device(w)
    say("recurrent handoff")
    s1 = d["h0"].clone()
    o1 = K.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s1, scale=w.scale)
    s2 = d["h0"].clone()
    oa = K.kda_recurrent_step(d["q"][:, :5].contiguous(), d["k"][:, :5].contiguous(),
                              d["v"][:, :5].contiguous(), d["g"][:, :5].contiguous(),
                              d["beta"][:, :5].contiguous(), s2, scale=w.scale)
    ob = K.kda_recurrent_step(d["q"][:, 5:].contiguous(), d["k"][:, 5:].contiguous(),
                              d["v"][:, 5:].contiguous(), d["g"][:, 5:].contiguous(),
                              d["beta"][:, 5:].contiguous(), s2, scale=w.scale)
    s3 = d["h0"].clone()
    o3 = K.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s3, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], 1), o1) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)


def test_mode_reduction_on_device():
    """Equal per-channel gates reproduce the scalar-gate mode, and a zero
    scalar gate reproduces the ungated mode, on the GPU kernels."""
    import torch
    import gated_delta_rule_17_amd as K
    w = make_inputs(2, 6, 3, 64, 64, mode="scalar", dtype="f32", seed=14, h0_std=0.1)
    d = to_device(w)
    gc = d["g"][..., None].expand(-1, -1, -1, 64).contiguous()
    say("recurrent mode reduction")
    outs = []
    for g, m in ((gc, "channel"), (d["g"], "scalar"), (torch.zeros_like(d["g"]), "scalar"), (None, "none")):
        st = d["h0"].clone()
        o = K.kda_recurrent_step(d["q"], d["k"], d["v"], g, d["beta"], st, mode=m)
        outs.append((o, st))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[2][0], outs[3][0]) and torch.equal(outs[2][1], outs[3][1])

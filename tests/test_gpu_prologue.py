"""Parity of the fused prologue with the prologue oracle (GPU).

Inputs are pre-activations (q, k unnormalised, beta and g raw); the oracle
applies the transforms in float64 and then runs oracle R.
"""
import numpy as np
import pytest

import gated_delta_rule_17_amd as K
import oracle
from kda_workloads import make_inputs, make_lengths, make_varlen
from tests.conftest import rel_err
from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu


def _oracle(w, flags, q=None, k=None):
    q = w.q if q is None else q
    k = w.k if k is None else k
    qq, kk, g, b = oracle.apply_prologue(q, k, w.g, w.beta, flags)
    return oracle.recurrent_grouped(qq, kk, w.v, g, b, w.h0, scale=w.scale, mode=w.mode)


def _dev(w, q=None, k=None):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda x, d=torch.float32: None if x is None else \
        torch.from_numpy(np.ascontiguousarray(x)).cuda().to(d)
    return (t(w.q if q is None else q, dt), t(w.k if k is None else k, dt), t(w.v, dt), t(w.g),
            t(w.beta), t(w.h0))


def _run(w, flags, form, chunk=32, q=None, k=None):
    import torch
    dq, dk, dv, dg, db, dh0 = _dev(w, q, k)
    if form == "chunk":
        o, hT = K.kda_chunk_fwd(dq, dk, dv, dg, db, initial_state=dh0, chunk=chunk, scale=w.scale,
                                mode=w.mode, out_dtype=torch.float32, prologue=flags)
    else:
        hT = dh0.clone()
        o = K.kda_recurrent_step(dq, dk, dv, dg, db, hT, scale=w.scale, mode=w.mode,
                                 out_dtype=torch.float32, prologue=flags)
    torch.cuda.synchronize()
    return o.cpu().numpy(), hT.cpu().numpy()


def _check(name, o, hT, ref, tol):
    eo, eh = rel_err(o, ref[0]), rel_err(hT, ref[1])
    print(f"[parity] prologue {name} o {eo:.3e} state {eh:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(hT).all()
    assert eo <= tol and eh <= tol, (name, eo, eh)


def _mixed_inputs(flags, **kw):
    """Pre-activations for the transformed inputs only; the others as the
    kernels take them without a prologue (unit keys, beta in (0, 1), g <= 0)."""
    import dataclasses
    pre = make_inputs(preact=True, gate_shift=2.0, **kw)
    std = make_inputs(**kw)
    return dataclasses.replace(
        std,
        q=pre.q if flags & 1 else std.q, k=pre.k if flags & 1 else std.k,
        beta=pre.beta if flags & 2 else std.beta, g=pre.g if flags & 4 else std.g)


@pytest.mark.parametrize("flags", [1, 2, 4, 7])
@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("form", ["chunk", "recurrent"])
def test_prologue_flags_f32(flags, mode, form):
    w = _mixed_inputs(flags, B=2, T=2 * 32 + 9, H=2, Dk=64, Dv=64, mode=mode, dtype="f32",
                      seed=flags * 7, h0_std=0.1)
    say("prologue f32", flags, mode, form)
    o, hT = _run(w, flags, form)
    _check(f"f32 flags{flags} {mode} {form}", o, hT, _oracle(w, flags), TOL["f32"])


def test_prologue_prefill_full_size_bf16():
    """B1 H16 T4096 d128 chunk 64, pre-activations, all three transforms."""
    w = make_inputs(1, 4096, 16, 128, 128, dtype="bf16", seed=11, gate_shift=3.0, h0_std=0.01,
                    preact=True)
    say("prologue prefill full size")
    o, hT = _run(w, 7, "chunk", chunk=64)
    _check("prefill full size bf16", o, hT, _oracle(w, 7), TOL["bf16"])


def test_prologue_decode_full_size_bf16():
    """B256 H32 d128, one token, all three transforms."""
    w = make_inputs(256, 1, 32, 128, 128, dtype="bf16", seed=12, gate_shift=3.0, h0_std=0.05,
                    preact=True)
    say("prologue decode full size")
    o, hT = _run(w, 7, "recurrent")
    _check("decode full size bf16", o, hT, _oracle(w, 7), TOL["bf16"])


def test_prologue_packed_grouped():
    import torch
    lengths = make_lengths(7, max_len=130, seed=3, edge=(0, 1, 64, 65))
    vw = make_varlen(lengths, 4, 64, 64, dtype="f32", seed=3, h0_std=0.1, gate_shift=2.0,
                     preact=True)
    w = vw.w
    q = np.ascontiguousarray(w.q[0][:, ::2])
    k = np.ascontiguousarray(w.k[0][:, ::2])
    qq, kk, g, b = oracle.apply_prologue(q, k, w.g[0], w.beta[0], 7)
    ref = oracle.recurrent_varlen(qq, kk, w.v[0], g, b, vw.cu, vw.h0, scale=w.scale)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    cu = t(vw.cu)
    say("prologue packed grouped", list(lengths))
    o_c, h_c = K.kda_chunk_fwd_varlen(t(q), t(k), t(w.v[0]), t(w.g[0]), t(w.beta[0]), cu,
                                      initial_state=t(vw.h0), chunk=16, scale=w.scale,
                                      prologue=7)
    st = t(vw.h0).clone()
    o_r = K.kda_recurrent_varlen(t(q), t(k), t(w.v[0]), t(w.g[0]), t(w.beta[0]), st, cu,
                                 scale=w.scale, prologue=7)
    torch.cuda.synchronize()
    _check("packed grouped chunk", o_c.cpu().numpy(), h_c.cpu().numpy(), ref, TOL["f32"])
    _check("packed grouped recurrent", o_r.cpu().numpy(), st.cpu().numpy(), ref, TOL["f32"])

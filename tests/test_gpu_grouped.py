"""Parity of grouped value heads and d_k != d_v with the oracle (GPU).

q and k have Hqk heads, v, g, beta, o and the state have H = G * Hqk value
heads; value head h reads query/key head h // G.  d_k is any of {16, 32, 64,
128} and d_v any of {16, 32, 64, 128, 256}.
"""
import numpy as np
import pytest

import gated_delta_rule_17_amd as K
import oracle
from kda_workloads import make_inputs, make_lengths, make_varlen
from tests.conftest import rel_err
from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu


def _inputs(B, T, Hqk, G, Dk, Dv, mode="channel", dtype="f32", seed=0, h0_std=0.1):
    w = make_inputs(B, T, Hqk * G, Dk, Dv, mode=mode, dtype=dtype, seed=seed, h0_std=h0_std,
                    gate_law="softplus" if mode != "none" else "zero")
    q = np.ascontiguousarray(w.q[:, :, ::G])
    k = np.ascontiguousarray(w.k[:, :, ::G])
    return w, q, k


def _dev(w, q, k):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda x, d=torch.float32: None if x is None else \
        torch.from_numpy(np.ascontiguousarray(x)).cuda().to(d)
    return t(q, dt), t(k, dt), t(w.v, dt), t(w.g), t(w.beta), t(w.h0)


def _run(w, q, k, form, chunk=64):
    import torch
    dq, dk, dv, dg, db, dh0 = _dev(w, q, k)
    if form == "chunk":
        o, hT = K.kda_chunk_fwd(dq, dk, dv, dg, db, initial_state=dh0, chunk=chunk,
                                scale=w.scale, mode=w.mode, out_dtype=torch.float32)
    else:
        hT = dh0.clone()
        o = K.kda_recurrent_step(dq, dk, dv, dg, db, hT, scale=w.scale, mode=w.mode,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o.cpu().numpy(), hT.cpu().numpy()


def _check(name, w, q, k, o, hT, tol):
    o_r, h_r = oracle.recurrent_grouped(q, k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=w.mode)
    eo, eh = rel_err(o, o_r), rel_err(hT, h_r)
    print(f"[parity] {name} o {eo:.3e} state {eh:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(hT).all()
    assert eo <= tol and eh <= tol, (name, eo, eh)


@pytest.mark.parametrize("form", ["chunk", "recurrent"])
@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("Hqk,G", [(2, 4), (1, 3)])
def test_grouped_heads_f32(form, mode, Hqk, G):
    w, q, k = _inputs(2, 2 * 32 + 9, Hqk, G, 64, 64, mode=mode, seed=Hqk * 10 + G)
    say("grouped f32", form, mode, Hqk, G)
    o, hT = _run(w, q, k, form, chunk=32)
    _check(f"grouped {form} {mode} Hqk{Hqk} G{G}", w, q, k, o, hT, TOL["f32"])


@pytest.mark.parametrize("Dk,Dv", [(64, 128), (128, 64), (16, 128), (128, 16), (32, 64)])
@pytest.mark.parametrize("chunk", [16, 64])
def test_mixed_dims_f32(Dk, Dv, chunk):
    w, q, k = _inputs(2, 2 * chunk + 7, 2, 1, Dk, Dv, seed=Dk + Dv + chunk, h0_std=0.2)
    say("mixed dims f32", Dk, Dv, chunk)
    for form in ("chunk", "recurrent"):
        o, hT = _run(w, q, k, form, chunk=chunk)
        _check(f"mixed {form} Dk{Dk} Dv{Dv} C{chunk}", w, q, k, o, hT, TOL["f32"])


@pytest.mark.parametrize("Dk,Dv,Hqk,G", [(64, 128, 2, 2), (128, 32, 1, 4), (128, 128, 4, 4)])
def test_grouped_mixed_bf16(Dk, Dv, Hqk, G):
    w, q, k = _inputs(1, 300, Hqk, G, Dk, Dv, dtype="bf16", seed=Dv, h0_std=0.05)
    say("grouped mixed bf16", Dk, Dv, Hqk, G)
    o, hT = _run(w, q, k, "chunk")
    _check(f"grouped mixed bf16 Dk{Dk} Dv{Dv} Hqk{Hqk} G{G}", w, q, k, o, hT, TOL["bf16"])


def test_packed_grouped_mixed():
    """Packed batch with grouped heads and d_k != d_v, both forms."""
    import torch
    lengths = make_lengths(9, max_len=150, seed=6, edge=(0, 1, 64, 65))
    vw = make_varlen(lengths, 4, 64, 128, dtype="bf16", seed=6, h0_std=0.05)
    w = vw.w
    q = np.ascontiguousarray(w.q[0][:, ::2])      # Hqk = 2, G = 2
    k = np.ascontiguousarray(w.k[0][:, ::2])
    t = lambda x, d=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(d)
    dq, dk, dv = t(q, torch.bfloat16), t(k, torch.bfloat16), t(w.v[0], torch.bfloat16)
    dg, db, dh0, cu = t(w.g[0]), t(w.beta[0]), t(vw.h0), torch.from_numpy(vw.cu).cuda()
    say("packed grouped mixed", list(lengths))
    o_c, h_c = K.kda_chunk_fwd_varlen(dq, dk, dv, dg, db, cu, initial_state=dh0, chunk=64,
                                      scale=w.scale, out_dtype=torch.float32)
    st = dh0.clone()
    o_r = K.kda_recurrent_varlen(dq, dk, dv, dg, db, st, cu, scale=w.scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_varlen(q, k, w.v[0], w.g[0], w.beta[0], vw.cu, vw.h0,
                                           scale=w.scale)
    for tag, o, h in (("chunk", o_c, h_c), ("recurrent", o_r, st)):
        eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(h.cpu().numpy(), h_ref)
        print(f"[parity] packed grouped mixed {tag} o {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


@pytest.mark.parametrize("Dk,Dv,Hqk", [(128, 128, 4), (64, 128, 16)])
def test_full_size_prefill_grouped_or_mixed(Dk, Dv, Hqk):
    """B1 T4096, 16 value heads, bf16, chunk 64: grouped heads (Hqk 4) and
    mixed dims (d_k 64, d_v 128); every head compared."""
    w, q, k = _inputs(1, 4096, Hqk, 16 // Hqk, Dk, Dv, dtype="bf16", seed=Dk + Hqk, h0_std=0.01)
    say("full size", Dk, Dv, Hqk)
    o, hT = _run(w, q, k, "chunk")
    _check(f"full size Dk{Dk} Dv{Dv} Hqk{Hqk}", w, q, k, o, hT, TOL["bf16"])


@pytest.mark.parametrize("Dk,chunk", [(128, 32), (64, 64), (16, 16)])
def test_value_dim_256_f32(Dk, chunk):
    """d_v = 256 with float32 operands, both forms (the recurrent form as
    two 128-column workgroups per head), ragged tail."""
    w, q, k = _inputs(2, 2 * chunk + 7, 2, 1, Dk, 256, seed=Dk + chunk, h0_std=0.2)
    say("d_v 256 f32", Dk, chunk)
    for form in ("chunk", "recurrent"):
        o, hT = _run(w, q, k, form, chunk=chunk)
        _check(f"d_v 256 {form} Dk{Dk} C{chunk}", w, q, k, o, hT, TOL["f32"])


def test_value_dim_256_f32_chunk64_dk128_not_supported():
    """float32 operands with chunk 64, d_k 128 and d_v 256 are refused by the
    chunk forward before anything is enqueued (chunk 32 serves the shape)."""
    import torch
    assert K.kda_chunk_fwd_workspace_size(1, 64, 1, 128, 256, 64, K.GATE_CHANNEL, K.F32) == 0
    w, q, k = _inputs(1, 64, 1, 1, 128, 256, seed=3)
    dq, dk, dv, dg, db, dh0 = _dev(w, q, k)
    with pytest.raises(RuntimeError, match="NOT_SUPPORTED"):
        K.kda_chunk_fwd(dq, dk, dv, dg, db, initial_state=dh0, chunk=64, scale=w.scale)
    torch.cuda.synchronize()


@pytest.mark.parametrize("form", ["chunk", "recurrent"])
def test_value_dim_256_grouped_bf16(form):
    w, q, k = _inputs(1, 300, 2, 2, 128, 256, dtype="bf16", seed=256, h0_std=0.05)
    say("d_v 256 grouped bf16", form)
    o, hT = _run(w, q, k, form)
    _check(f"d_v 256 grouped bf16 {form}", w, q, k, o, hT, TOL["bf16"])


def test_value_dim_256_decode_step():
    """The decode step (one token per sequence) with d_v = 256, bf16."""
    w, q, k = _inputs(8, 1, 4, 1, 128, 256, dtype="bf16", seed=11, h0_std=0.05)
    say("d_v 256 decode")
    o, hT = _run(w, q, k, "recurrent")
    _check("d_v 256 decode bf16", w, q, k, o, hT, TOL["bf16"])


def test_value_dim_256_packed():
    """Packed batch with d_v = 256, both forms, bf16."""
    import torch
    lengths = make_lengths(7, max_len=150, seed=8, edge=(0, 1, 64, 65))
    vw = make_varlen(lengths, 2, 128, 256, dtype="bf16", seed=8, h0_std=0.05)
    w = vw.w
    t = lambda x, d=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(d)
    dq, dk, dv = t(w.q[0], torch.bfloat16), t(w.k[0], torch.bfloat16), t(w.v[0], torch.bfloat16)
    dg, db, dh0, cu = t(w.g[0]), t(w.beta[0]), t(vw.h0), torch.from_numpy(vw.cu).cuda()
    say("d_v 256 packed", list(lengths))
    o_c, h_c = K.kda_chunk_fwd_varlen(dq, dk, dv, dg, db, cu, initial_state=dh0, chunk=64,
                                      scale=w.scale, out_dtype=torch.float32)
    st = dh0.clone()
    o_r = K.kda_recurrent_varlen(dq, dk, dv, dg, db, st, cu, scale=w.scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_varlen(w.q[0], w.k[0], w.v[0], w.g[0], w.beta[0], vw.cu,
                                           vw.h0, scale=w.scale)
    for tag, o, h in (("chunk", o_c, h_c), ("recurrent", o_r, st)):
        eo, eh = rel_err(o.cpu().numpy(), o_ref), rel_err(h.cpu().numpy(), h_ref)
        print(f"[parity] d_v 256 packed {tag} o {eo:.3e} state {eh:.3e}", flush=True)
        assert eo <= TOL["bf16"] and eh <= TOL["bf16"]

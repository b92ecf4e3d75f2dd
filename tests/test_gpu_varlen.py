"""Parity of the packed variable-length HIP paths with the packed oracle (GPU).

Both entry points take a packed [T, H, D] batch and device offsets
cu_seqlens [N+1]; every sequence runs its own recurrence from its own state.
"""
import numpy as np
import pytest

import gated_delta_rule_17_amd as K
import oracle
from kda_workloads import make_lengths, make_varlen
from tests.conftest import rel_err
from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu

EDGE = (0, 1, 2, 15, 16, 17, 63, 64, 65, 0, 130)


def _dev(vw):
    import torch
    w = vw.w
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda x, d=torch.float32: None if x is None else \
        torch.from_numpy(np.ascontiguousarray(x)).cuda().to(d)
    return dict(q=t(w.q[0], dt), k=t(w.k[0], dt), v=t(w.v[0], dt),
                g=None if w.g is None else t(w.g[0]), beta=t(w.beta[0]), h0=t(vw.h0),
                cu=torch.from_numpy(vw.cu).cuda())


def _oracle(vw):
    w = vw.w
    g = None if w.g is None else w.g[0]
    return oracle.recurrent_varlen(w.q[0], w.k[0], w.v[0], g, w.beta[0], vw.cu, vw.h0,
                                   scale=w.scale, mode=w.mode)


def _run_rec(vw, d=None):
    import torch
    d = d or _dev(vw)
    w = vw.w
    st = d["h0"].clone() if d["h0"] is not None else torch.zeros(
        (vw.N, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    o = K.kda_recurrent_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu"],
                               scale=w.scale, mode=w.mode, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o.cpu().numpy(), st.cpu().numpy()


def _run_chunk(vw, chunk, d=None):
    import torch
    d = d or _dev(vw)
    w = vw.w
    o, hT = K.kda_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                   initial_state=d["h0"], chunk=chunk, scale=w.scale, mode=w.mode,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    return o.cpu().numpy(), hT.cpu().numpy()


def _check(name, vw, o, hT, tol):
    o_r, h_r = _oracle(vw)
    eo, eh = rel_err(o, o_r), rel_err(hT, h_r)
    print(f"[parity] varlen {name} o {eo:.3e} state {eh:.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(hT).all()
    assert eo <= tol and eh <= tol, (name, eo, eh)


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_varlen_ragged(mode, dtype):
    lengths = make_lengths(14, max_len=90, seed=3, edge=EDGE)
    vw = make_varlen(lengths, 3, 64, 64, mode=mode, dtype=dtype, seed=21, h0_std=0.1,
                     gate_law="softplus" if mode != "none" else "zero")
    say("recurrent varlen", mode, dtype, list(lengths))
    o, hT = _run_rec(vw)
    _check(f"recurrent {mode} {dtype}", vw, o, hT, TOL[dtype])


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_chunk_varlen_ragged_f32(mode, chunk):
    lengths = make_lengths(14, max_len=200, seed=chunk, edge=EDGE)
    vw = make_varlen(lengths, 2, 32, 32, mode=mode, dtype="f32", seed=7 + chunk, h0_std=0.2,
                     gate_law="softplus" if mode != "none" else "zero")
    say("chunk varlen f32", mode, chunk, list(lengths))
    o, hT = _run_chunk(vw, chunk)
    _check(f"chunk f32 {mode} C{chunk}", vw, o, hT, TOL["f32"])


@pytest.mark.parametrize("D,chunk", [(16, 32), (64, 32), (128, 64)])
def test_chunk_varlen_ragged_bf16(D, chunk):
    lengths = make_lengths(12, max_len=300, seed=D, edge=EDGE)
    vw = make_varlen(lengths, 3, D, D, dtype="bf16", seed=D, h0_std=0.05)
    say("chunk varlen bf16", D, chunk, list(lengths))
    o, hT = _run_chunk(vw, chunk)
    _check(f"chunk bf16 D{D} C{chunk}", vw, o, hT, TOL["bf16"])


def test_equal_lengths_match_dense_path_bitwise():
    """With equal lengths the packed batch is the dense [N, L] batch, cut into
    the same chunks: both paths must give identical bits."""
    import torch
    N, L, H, D = 3, 150, 2, 128
    vw = make_varlen([L] * N, H, D, D, dtype="bf16", seed=5, h0_std=0.05)
    d = _dev(vw)
    say("varlen vs dense, equal lengths")
    o_v, h_v = _run_chunk(vw, 64, d)
    rs = lambda x: None if x is None else x.reshape((N, L) + tuple(x.shape[1:])).contiguous()
    o_d, h_d = K.kda_chunk_fwd(rs(d["q"]), rs(d["k"]), rs(d["v"]), rs(d["g"]), rs(d["beta"]),
                               initial_state=d["h0"], chunk=64, scale=vw.w.scale,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(o_v, o_d.cpu().numpy().reshape(o_v.shape))
    assert np.array_equal(h_v, h_d.cpu().numpy())
    st = d["h0"].clone()
    o_r = K.kda_recurrent_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], st, d["cu"],
                                 scale=vw.w.scale, out_dtype=torch.float32)
    st_d = d["h0"].clone()
    o_rd = K.kda_recurrent_step(rs(d["q"]), rs(d["k"]), rs(d["v"]), rs(d["g"]), rs(d["beta"]),
                                st_d, scale=vw.w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_r, o_rd.reshape(o_r.shape)) and torch.equal(st, st_d)


def test_chunk_varlen_in_place_state_and_empty_batch():
    import torch
    lengths = [40, 0, 70]
    vw = make_varlen(lengths, 2, 64, 64, dtype="f32", seed=8, h0_std=0.3)
    d = _dev(vw)
    say("chunk varlen in place")
    st = d["h0"].clone()
    o, _ = K.kda_chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                  initial_state=st, final_state=st, chunk=32, scale=vw.w.scale,
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check("in place", vw, o.cpu().numpy(), st.cpu().numpy(), TOL["f32"])
    # every sequence empty: the final states are the initial ones
    e = make_varlen([0, 0, 0], 2, 64, 64, dtype="f32", seed=9, h0_std=0.3)
    de = _dev(e)
    say("chunk varlen all empty")
    q0 = torch.zeros((0, 2, 64), device="cuda")
    _, hT = K.kda_chunk_fwd_varlen(q0, q0, q0, torch.zeros((0, 2, 64), device="cuda"),
                                   torch.zeros((0, 2), device="cuda"), de["cu"],
                                   initial_state=de["h0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(hT, de["h0"])


def test_serving_mix_full_size_every_sequence():
    """64 sequences of log-uniform lengths up to 2048 (H16, d128, bf16), the
    chunk form and the recurrent form; every sequence (all heads) against the
    oracle, the worst printed."""
    lengths = make_lengths(64, max_len=2048, seed=17, edge=(1, 64, 2048))
    vw = make_varlen(lengths, 16, 128, 128, dtype="bf16", seed=17, h0_std=0.02)
    d = _dev(vw)
    say("serving mix", int(vw.cu[-1]), "tokens")
    o_c, h_c = _run_chunk(vw, 64, d)
    o_r, h_r = _run_rec(vw, d)
    w = vw.w
    worst = {"chunk": (0.0, -1), "recurrent": (0.0, -1)}
    for n in range(vw.N):
        a, b = int(vw.cu[n]), int(vw.cu[n + 1])
        sl = lambda x: None if x is None else x[0, a:b][None]
        on, hn = oracle.recurrent(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta),
                                  vw.h0[n:n + 1], scale=w.scale, mode=w.mode)
        for tag, o, h in (("chunk", o_c, h_c), ("recurrent", o_r, h_r)):
            eo, eh = rel_err(o[a:b], on[0]), rel_err(h[n], hn[0])
            if b > a:
                worst[tag] = max(worst[tag], (max(eo, eh), n))
            assert eo <= TOL["bf16"] and eh <= TOL["bf16"], (tag, n, eo, eh)
    print(f"[parity] varlen serving, all {vw.N} sequences: worst chunk {worst['chunk'][0]:.3e} "
          f"(seq {worst['chunk'][1]}), recurrent {worst['recurrent'][0]:.3e} "
          f"(seq {worst['recurrent'][1]})", flush=True)

"""Helpers for the GPU parity tests: move a seeded workload to the device,
run the HIP path through the C ABI, and run the oracle on the same values."""
from __future__ import annotations

import sys

import numpy as np

import gated_delta_rule_17_amd as K
import oracle
from kda_workloads import slice_heads

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, file=sys.stderr, flush=True)


def to_device(w, device="cuda"):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def t(x, d=torch.float32):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device).to(d)

    return dict(q=t(w.q, dt), k=t(w.k, dt), v=t(w.v, dt), g=t(w.g), beta=t(w.beta), h0=t(w.h0))


def run_chunk(w, chunk=None, d=None, out="f32"):
    """Run the chunk path; parity is measured on a float32 output (a bf16
    output is that float32 result rounded, see test_bf16_output_is_rounded)."""
    import torch
    d = d or to_device(w)
    od = torch.float32 if out == "f32" else torch.bfloat16
    o, hT = K.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                            chunk=chunk or w.chunk, scale=w.scale, mode=w.mode, out_dtype=od)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), hT.cpu().numpy()


def run_recurrent(w, d=None, out="f32"):
    import torch
    d = d or to_device(w)
    st = d["h0"].clone() if d["h0"] is not None else torch.zeros(
        (w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    od = torch.float32 if out == "f32" else torch.bfloat16
    o = K.kda_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, scale=w.scale,
                             mode=w.mode, out_dtype=od)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), st.cpu().numpy()


def run_oracle(w, pairs=None):
    """Oracle R over the whole workload, or over sampled (b, h) pairs.
    Returns (o, hT) with the shapes of the full tensors restricted to the
    sampled pairs: o [n, T, Dv], hT [n, Dk, Dv] when pairs is given."""
    if pairs is None:
        return oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=w.mode)
    sl = slice_heads(w, pairs)
    cat = lambda i: None if sl[0][i] is None else np.concatenate([x[i] for x in sl], axis=0)
    q, k, v, g, beta, h0 = (cat(i) for i in range(6))
    o, hT = oracle.recurrent(q, k, v, g, beta, h0, scale=w.scale, mode=w.mode)
    return o[:, :, 0], hT[:, 0]


def pick(o_full, hT_full, pairs):
    return (np.stack([o_full[b, :, h] for b, h in pairs]),
            np.stack([hT_full[b, h] for b, h in pairs]))


def per_head_errors(w, o, hT, batches=None):
    """Oracle R one batch entry at a time (host memory stays bounded at the
    largest workloads), compared with the kernels' o [B,T,H,Dv] and
    hT [B,H,Dk,Dv] on every head of those entries.

    Returns (whole, worst, table): ``whole`` = (o, state) errors over all
    compared heads together (the max|d|/rms measure over the whole run);
    ``worst`` = the largest per-head (o, state) errors, each with its (b, h);
    ``table`` = {(b, h): (o error, state error)}, each against that head's
    own rms."""
    from tests.conftest import rel_err
    batches = range(w.B) if batches is None else batches
    table = {}
    num_o = num_h = 0.0
    ss_o = ss_h = 0.0
    n_o = n_h = 0
    for b in batches:
        sl = lambda x: None if x is None else np.ascontiguousarray(x[b:b + 1])
        o_r, h_r = oracle.recurrent(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), sl(w.h0),
                                    scale=w.scale, mode=w.mode)
        for h in range(w.H):
            og, orf = o[b, :, h], o_r[0, :, h]
            hg, hrf = hT[b, h], h_r[0, h]
            table[(b, h)] = (rel_err(og, orf), rel_err(hg, hrf))
            num_o = max(num_o, float(np.abs(og.astype(np.float64) - orf).max()) if og.size else 0.0)
            num_h = max(num_h, float(np.abs(hg.astype(np.float64) - hrf).max()))
            ss_o += float(np.sum(orf * orf))
            ss_h += float(np.sum(hrf * hrf))
            n_o += orf.size
            n_h += hrf.size
        del o_r, h_r
    rms_o = np.sqrt(ss_o / max(n_o, 1))
    rms_h = np.sqrt(ss_h / max(n_h, 1))
    whole = (num_o / rms_o if rms_o > 0 else num_o, num_h / rms_h if rms_h > 0 else num_h)
    wo = max(table.items(), key=lambda kv: kv[1][0])
    wh = max(table.items(), key=lambda kv: kv[1][1])
    worst = ((wo[1][0], wo[0]), (wh[1][1], wh[0]))
    return whole, worst, table

#!/usr/bin/env python3
"""Benchmark of the KDA forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * chunked prefill  B=1, H=16, T=4096, d_k=d_v=128, chunk 64, bf16 q/k/v,
    fp32 gates/beta/state, bf16 output            (kda_chunk_fwd)
  * decode step      B=256, H=32, d_k=d_v=128, one token, fp32 state
    (512 MiB) updated in place, bf16 q/k/v/o       (kda_recurrent_step)

Prints ONE JSON line.  ``value`` is prefill tokens/s; the decode step's state
GB/s is reported next to it (the metric names both).  Timing uses HIP events
on the stream the kernels are launched on (torch's current stream), W untimed
warm-up steps, then exactly K timed steps between device synchronisations:
the K prefill calls back to back, then the K decode steps.  The prefill time
is the event interval from the end of the first timed prefill call to the end
of the last, over K - 1 calls (the first call covers the host's launch lead);
the decode time is the interval over the K decode steps that follow.  An event
pair around every call would add the events' own GPU time (~5 us a pair) to
each measured call.  Prefill inputs rotate over three resident copies so that
they do not sit in the 256 MB last-level cache between calls.

``roofline`` is the decode kernel (the step's dominant kernel by time, HBM
bound); ``roofline_prefill`` is the prefill call (two kernels).  Achieved
figures use algorithmic bytes: decode 132 612 B per (b, h); prefill 1540 B per
token-head plus 2 * d_k * d_v * 4 B of initial/final state per (b, h).
``traffic`` comes from rocprofv3 FETCH_SIZE/WRITE_SIZE counter runs stored in
profiles/traffic.json and is null when the kernel source changed since.
``cpu_baseline`` times the fp64 CPU oracle (test infrastructure) on the host.
``varlen`` (outside the timed steps) times the packed variable-length entry
points (both forward forms and the gradient) on a serving mix: 64 sequences of log-uniform lengths 1..2048, H=16,
d=128, bf16, in both forms.  ``grouped_heads`` (4 query/key heads for the 16
value heads), ``mixed_dims`` (d_k 64, d_v 128) and ``value_dim_256`` (d_k
128, d_v 256) time kda_chunk_fwd on the prefill shape B1 T4096 H16, likewise
outside the timed steps.  ``backward`` (also outside them) times
kda_chunk_bwd, the gradients of the prefill call, on the prefill workload
with seeded output gradients, against the float32 matrix-core peak (its
products are computed to float32 accuracy).  The large workloads -- the
training shape B8 H32 T8192 and T = 65536 at H8 in the three gate modes --
are timed last, each as a whole kda_chunk_fwd call (outside the timed steps),
with the oracle's rate on a bounded sample of each beside them; then
``backward_train_b8_h32_t8192`` times kda_chunk_bwd at the training shape
(its workspace holds one group of batch entries).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix, published

PREFILL = dict(B=1, H=16, T=4096, D=128, chunk=64)
DECODE = dict(B=256, H=32, D=128)


def decode_bytes(B, H, D):
    # state read + write (fp32), q, k, v (bf16), g (fp32 per channel), beta, o (bf16)
    return B * H * (2 * D * D * 4 + 3 * D * 2 + D * 4 + 4 + D * 2)


def prefill_bytes(B, H, T, D):
    per_token_head = 4 * D * 2 + D * 4 + 4          # q, k, v, o bf16; g fp32; beta
    return B * H * T * per_token_head + B * H * 2 * D * D * 4


def prefill_flops(B, H, T, D, C):
    # triangle-exploiting count per token-head: 6 d^2 + (C-1) d + (C+1)(2d + 2d) + C^2/3
    per = 6 * D * D + (C - 1) * D + (C + 1) * (4 * D) + C * C / 3.0
    return B * H * T * per


def backward_flops(B, H, T, Dk, Dv, C):
    """Matrix products of the chunkwise gradient per chunk, 2 m n k each and
    half that for a triangular factor: 16 C Dk Dv (Qg^T dO, the two state
    carries at two products each, the three products with the state and its
    gradient) + 7 C^2 Dk (both couplings, W, and the four decayed sums of the
    key/query gradients) + 5 C^2 Dv (U, Aqk^T dO, T^T dE and the two C x C
    products with E)."""
    nc = B * H * ((T + C - 1) // C)
    return nc * (16 * C * Dk * Dv + 7 * C * C * Dk + 5 * C * C * Dv)


def backward_bytes(B, H, T, Dk, Dv):
    # in: q, k, v, dO bf16, g fp32, beta; out: dq, dk, dv bf16, dg fp32, dbeta;
    # initial state, final-state gradient and initial-state gradient fp32
    per = (2 * Dk + 2 * Dv) * 2 + Dk * 4 + 4 + (2 * Dk + Dv) * 2 + Dk * 4 + 4
    return B * H * T * per + 3 * B * H * Dk * Dv * 4


def source_hash(*names):
    """Hash of the kernel code: `//` comments, trailing blanks and empty lines
    are left out, so an edit of comments alone does not mark the stored
    counter figures as stale."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_17_amd", "csrc", n), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic():
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return {}
    with open(p) as f:
        return json.load(f)


def cpu_baseline():
    """The oracle as it stands, on the host cores: the full prefill workload
    (all 16 heads x 4096 tokens) and one full decode step."""
    import oracle
    from kda_workloads import make_config
    w = make_config("prefill_h16_t4096")
    t0 = time.perf_counter()
    oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=w.mode)
    tp = time.perf_counter() - t0
    d = make_config("decode_b256_h32")
    t0 = time.perf_counter()
    oracle.recurrent(d.q, d.k, d.v, d.g, d.beta, d.h0, scale=d.scale, mode=d.mode)
    td = time.perf_counter() - t0
    state_bytes = d.B * d.H * d.Dk * d.Dv * 4 * 2
    from kda_workloads import make_lengths, make_varlen
    vw = make_varlen(make_lengths(64, max_len=2048, seed=17, edge=(1, 64, 2048)), 16, 128, 128,
                     dtype="bf16", seed=17, h0_std=0.02)
    vq = vw.w
    t0 = time.perf_counter()
    oracle.recurrent_varlen(vq.q[0], vq.k[0], vq.v[0], vq.g[0], vq.beta[0], vw.cu, vw.h0,
                            scale=vq.scale, mode=vq.mode)
    tv = time.perf_counter() - t0
    from kda_workloads import make_inputs
    rows = {}
    for name, Hqk, Dk, Dv in (("grouped_heads", 4, 128, 128), ("mixed_dims", 16, 64, 128),
                              ("value_dim_256", 16, 128, 256)):
        x = make_inputs(1, 4096, 16, Dk, Dv, dtype="bf16", seed=5, gate_shift=2.0, h0_std=0.01)
        G = 16 // Hqk
        t0 = time.perf_counter()
        oracle.recurrent_grouped(x.q[:, :, ::G], x.k[:, :, ::G], x.v, x.g, x.beta, x.h0,
                                 scale=x.scale, mode=x.mode)
        rows[name + "_tokens_per_s"] = 4096 / (time.perf_counter() - t0)
    from kda_workloads import make_cotangents
    cot = make_cotangents(w, seed=0, dhT_std=0.01)
    t0 = time.perf_counter()
    oracle.recurrent_bwd(w.q, w.k, w.v, w.g, w.beta, w.h0, cot.do, cot.dhT, scale=w.scale,
                         mode=w.mode)
    rows["backward_tokens_per_s"] = w.B * w.T / (time.perf_counter() - t0)
    return {"value": w.B * w.T / tp, "unit": "tokens/s", "cores": oracle.oracle_threads(),
            "kind": "oracle",
            "sample": "fp64 oracle R over the whole prefill workload (B1 H16 T4096 d128, "
                      f"{tp:.2f} s) and one whole decode step (B256 H32 d128, {td:.2f} s)",
            "decode_state_GBps": state_bytes / td / 1e9,
            "varlen_tokens_per_s": int(vw.cu[-1]) / tv,
            **rows,
            "host_cpus": len(os.sched_getaffinity(0))}


def bench_varlen(K, torch, dev, warmup, reps):
    """Packed serving mix through kda_chunk_fwd_varlen and kda_recurrent_varlen
    (each timed on its own, HIP events on the launch stream)."""
    from kda_workloads import make_lengths, make_varlen
    lengths = make_lengths(64, max_len=2048, seed=17, edge=(1, 64, 2048))
    vw = make_varlen(lengths, 16, 128, 128, dtype="bf16", seed=17, h0_std=0.02)
    w = vw.w
    t = lambda x, d=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(d)
    q, k, v = t(w.q[0], torch.bfloat16), t(w.k[0], torch.bfloat16), t(w.v[0], torch.bfloat16)
    g, beta, h0 = t(w.g[0]), t(w.beta[0]), t(vw.h0)
    cu = torch.from_numpy(vw.cu).to(dev)
    N, T, H, D = vw.N, int(vw.cu[-1]), w.H, w.Dk
    ws = torch.empty(K.kda_chunk_fwd_varlen_workspace_size(N, T, H, D, D, 64, 0, K.BF16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(h0)
    st = h0.clone()

    def chunk():
        K.kda_chunk_fwd_varlen(q, k, v, g, beta, cu, initial_state=h0, final_state=hT, o=o,
                               chunk=64, workspace=ws)

    def rec():
        K.kda_recurrent_varlen(q, k, v, g, beta, st, cu, o=o)

    do = t(np.random.default_rng(np.random.SeedSequence([17, 0xD0])).standard_normal(
        (T, H, D), dtype=np.float32), torch.bfloat16)
    wsb = torch.empty(K.kda_chunk_bwd_varlen_workspace_size(N, T, H, H, D, D, 64, 0, K.BF16),
                      dtype=torch.uint8, device=dev)
    grads = K.kda_chunk_bwd_varlen(q, k, v, g, beta, do, cu, initial_state=h0, chunk=64,
                                   workspace=wsb)

    def bwd():
        K.kda_chunk_bwd_varlen(q, k, v, g, beta, do, cu, initial_state=h0, chunk=64,
                               workspace=wsb, out=grads)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    tc, tr, tb = timed(chunk), timed(rec), timed(bwd)
    nbytes = T * H * (4 * D * 2 + D * 4 + 4) + N * H * 2 * D * D * 4
    return {"workload": f"{N} sequences, log-uniform lengths 1..2048 (seed 17), {T} tokens, "
                        "H16 d128 bf16, fp32 states",
            "tokens": T, "sequences": N, "longest": int(lengths.max()),
            "chunk_ms": tc * 1e3, "chunk_tokens_per_s": T / tc,
            "chunk_hbm_frac": nbytes / tc / 1e9 / HBM_PEAK_GBPS,
            "recurrent_ms": tr * 1e3, "recurrent_tokens_per_s": T / tr,
            "backward_ms": tb * 1e3, "backward_tokens_per_s": T / tb,
            "algorithmic_bytes": nbytes}


def bench_prefill_shape(K, torch, dev, warmup, reps, *, Hqk, Dk, Dv, H=16, T=4096):
    """kda_chunk_fwd on B1 T4096 with H value heads, Hqk query/key heads and
    (Dk, Dv); HIP events on the launch stream."""
    from kda_workloads import make_inputs
    w = make_inputs(1, T, H, Dk, Dv, dtype="bf16", seed=5, gate_shift=2.0, h0_std=0.01)
    G = H // Hqk
    t = lambda x, d=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(d)
    q = t(w.q[:, :, ::G], torch.bfloat16)
    k = t(w.k[:, :, ::G], torch.bfloat16)
    v, g, beta, h0 = t(w.v, torch.bfloat16), t(w.g), t(w.beta), t(w.h0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(1, T, H, Dk, Dv, 64, 0, K.BF16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((1, T, H, Dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(h0)

    def run():
        K.kda_chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o, chunk=64,
                        workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / reps / 1e3
    # q, k per query/key head; v, o bf16, g fp32, beta per value head; states
    nbytes = T * (Hqk * 2 * Dk * 2 + H * (2 * Dv * 2 + Dk * 4 + 4)) + H * 2 * Dk * Dv * 4
    return {"workload": f"B1 T{T} H{H} value heads, {Hqk} query/key heads, d_k {Dk}, d_v {Dv}, "
                        "chunk 64, bf16",
            "ms": sec * 1e3, "tokens_per_s": T / sec, "algorithmic_bytes": nbytes,
            "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBPS}


def config_bytes(w):
    """Algorithmic HBM bytes of one kda_chunk_fwd call on workload w with a
    bf16 output: q, k, v, o (bf16), the gates (float32: Dk per token-head in
    channel mode, one in scalar mode, none in the ungated mode), beta, the
    initial state when there is one and the final state."""
    gate = {"channel": 4 * w.Dk, "scalar": 4, "none": 0}[w.mode]
    per = (2 * w.Dk + w.Dv) * 2 + w.Dv * 2 + gate + 4
    states = (2 if w.h0 is not None else 1) * w.Dk * w.Dv * 4
    return w.B * w.H * (w.T * per + states)


def bench_config(K, torch, dev, name, warmup, reps):
    """kda_chunk_fwd on one named workload at full size (bf16 in and out,
    float32 gates, beta and states), HIP events on the launch stream; the
    whole call is timed (both kernels)."""
    from kda_workloads import make_config
    w = make_config(name)
    t = lambda x, d=torch.float32: None if x is None else \
        torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(d)
    bf = torch.bfloat16
    q, k, v, g, beta, h0 = t(w.q, bf), t(w.k, bf), t(w.v, bf), t(w.g), t(w.beta), t(w.h0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(w.B, w.T, w.H, w.Dk, w.Dv, 64, w.mode, K.BF16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=bf, device=dev)
    hT = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)

    def run():
        K.kda_chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o, chunk=64,
                        mode=w.mode, workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / reps / 1e3
    nbytes = config_bytes(w)
    flops = prefill_flops(w.B, w.H, w.T, w.Dk, 64)
    res = {"workload": f"{name}: B{w.B} H{w.H} T{w.T} d_k {w.Dk} d_v {w.Dv}, chunk 64, "
                       f"{w.mode} gates, bf16 q/k/v/o, fp32 gates/beta/states",
           "ms": sec * 1e3, "tokens_per_s": w.B * w.T / sec,
           "token_heads_per_s": w.B * w.T * w.H / sec,
           "algorithmic_bytes": nbytes, "hbm_GBps": nbytes / sec / 1e9,
           "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBPS,
           "mfma_frac_algorithmic": flops / sec / 1e12 / BF16_MFMA_PEAK_TFLOPS,
           "serial_chunk_steps": (w.T + 63) // 64}
    del q, k, v, g, beta, h0, ws, o, hT
    torch.cuda.empty_cache()
    return res


LARGE_LEGS = ("train_b8_h32_t8192", "long_t65536_channel", "long_t65536_scalar",
              "long_t65536_none")
# gradient legs at full size (the workspace holds one group of batch entries)
LARGE_BWD_LEGS = ("train_b8_h32_t8192",)


def cpu_large_sample():
    """The oracle's rate on bounded samples of the large workloads: batch
    entry 0 of the training shape (32 heads x 8192 tokens), and head 0 of
    each T = 65536 mode."""
    import oracle
    from kda_workloads import make_config
    rows = {}
    for name in LARGE_LEGS:
        w = make_config(name)
        if name.startswith("train"):
            sl = lambda x: None if x is None else np.ascontiguousarray(x[:1])
            what = "batch entry 0 (32 heads x 8192 tokens)"
        else:
            sl = lambda x: None if x is None else np.ascontiguousarray(x[:, :, :1])
            what = "head 0 (65536 tokens)"
        q, k, v, g, beta = sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta)
        t0 = time.perf_counter()
        oracle.recurrent(q, k, v, g, beta, None, scale=w.scale, mode=w.mode)
        dt = time.perf_counter() - t0
        th = q.shape[0] * q.shape[1] * q.shape[2]
        rows[name] = {"token_heads_per_s": th / dt, "sample": what, "seconds": dt}
        del w, q, k, v, g, beta
    return rows


def bench_backward(K, torch, dev, warmup, reps, name="prefill_h16_t4096"):
    """kda_chunk_bwd on a named workload (by default the prefill workload, B1
    H16 T4096 d128; chunk 64, bf16 q/k/v and output gradient, bf16 input
    gradients), HIP events on the launch stream."""
    from kda_workloads import make_config, make_cotangents
    w = make_config(name)
    cot = make_cotangents(w, seed=0, dhT_std=0.01)
    t = lambda x, d=torch.float32: None if x is None else \
        torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(d)
    bf = torch.bfloat16
    q, k, v, do = t(w.q, bf), t(w.k, bf), t(w.v, bf), t(cot.do, bf)
    g, beta, h0, dhT = t(w.g), t(w.beta), t(w.h0), t(cot.dhT)
    B, T, H, Dk, Dv, C = w.B, w.T, w.H, w.Dk, w.Dv, 64
    ws = torch.empty(K.kda_chunk_bwd_workspace_size(B, T, H, H, Dk, Dv, C, w.mode, K.BF16),
                     dtype=torch.uint8, device=dev)
    out = K.kda_chunk_bwd(q, k, v, g, beta, do, initial_state=h0, d_final_state=dhT, chunk=C,
                          mode=w.mode, workspace=ws)

    def run():
        K.kda_chunk_bwd(q, k, v, g, beta, do, initial_state=h0, d_final_state=dhT, chunk=C,
                        mode=w.mode, workspace=ws, out=out)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / reps / 1e3
    flops = backward_flops(B, H, T, Dk, Dv, C)
    nbytes = backward_bytes(B, H, T, Dk, Dv)
    what = ("the prefill call: B1 H16 T4096 d128" if name == "prefill_h16_t4096" else
            f"{name}: B{B} H{H} T{T} d_k {Dk} d_v {Dv}, {w.mode} gates")
    res = {"workload": f"gradients of {what}, chunk 64, bf16 "
                        "q/k/v/dO and input gradients, fp32 gates/beta/states",
            "ms": sec * 1e3, "tokens_per_s": B * T / sec,
            "roofline": {"kernel": "kda_chunk_bwd (bwd_prep + bwd_states + bwd_grad)",
                         "bound": "mfma", "achieved": flops / sec / 1e12,
                         "peak": F32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops / sec / 1e12 / F32_MFMA_PEAK_TFLOPS,
                         "algorithmic_flops_per_launch": flops},
            "algorithmic_bytes": nbytes, "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBPS,
            "workspace_bytes": int(ws.numel())}
    del q, k, v, do, g, beta, h0, dhT, ws, out
    torch.cuda.empty_cache()
    return res


def bench_prologue(K, torch, dev, warmup, reps):
    """The prefill and decode shapes with all three prologue transforms fused
    (q, k L2-normalised; beta = sigmoid; g = log sigmoid of pre-activations)."""
    from kda_workloads import make_inputs
    t = lambda x, d=torch.float32: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(d)
    flags = K.NORMALIZE_QK | K.BETA_SIGMOID | K.GATE_LOGSIGMOID
    w = make_inputs(1, 4096, 16, 128, 128, dtype="bf16", seed=11, gate_shift=3.0, h0_std=0.01,
                    preact=True)
    q, k, v = t(w.q, torch.bfloat16), t(w.k, torch.bfloat16), t(w.v, torch.bfloat16)
    g, beta, h0 = t(w.g), t(w.beta), t(w.h0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(1, 4096, 16, 128, 128, 64, 0, K.BF16),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((1, 4096, 16, 128), dtype=torch.bfloat16, device=dev)
    hT = torch.empty_like(h0)
    d = make_inputs(256, 1, 32, 128, 128, dtype="bf16", seed=12, gate_shift=3.0, h0_std=0.05,
                    preact=True)
    dq, dk, dv = t(d.q, torch.bfloat16), t(d.k, torch.bfloat16), t(d.v, torch.bfloat16)
    dg, db, st = t(d.g), t(d.beta), t(d.h0)
    od = torch.empty((256, 1, 32, 128), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    tp = timed(lambda: K.kda_chunk_fwd(q, k, v, g, beta, initial_state=h0, final_state=hT, o=o,
                                       chunk=64, workspace=ws, prologue=flags))
    td = timed(lambda: K.kda_recurrent_step(dq, dk, dv, dg, db, st, o=od, prologue=flags))
    return {"workload": "prefill B1 H16 T4096 d128 and decode B256 H32 d128, bf16, "
                        "pre-activations with all three transforms fused",
            "prefill_ms": tp, "prefill_tokens_per_s": 4096 / (tp / 1e3),
            "decode_ms": td, "decode_state_GBps": 256 * 32 * 128 * 128 * 8 / (td / 1e3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="skip the untimed legs after the steps (packed batches, grouped heads, "
                         "mixed dims): profiling runs, whose launches would share kernel names "
                         "with the prefill")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a float32 copy of exactly 256 MiB (reads 256 MiB, writes "
                         "256 MiB) three times, as the reference for HBM byte counters")
    ap.add_argument("--only", choices=LARGE_LEGS,
                    help="run only kda_chunk_fwd on this named workload (5 timed calls after 2 "
                         "warm-ups) and print its JSON object: profiling runs of one workload")
    ap.add_argument("--backward-only", action="store_true",
                    help="run only the gradient leg (kda_chunk_bwd on the prefill workload, or "
                         "on --backward-workload) and print its JSON object: profiling runs of "
                         "the gradient kernels")
    ap.add_argument("--backward-workload", choices=("prefill_h16_t4096",) + LARGE_BWD_LEGS,
                    default="prefill_h16_t4096")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_17_amd as K
    from kda_workloads import make_config
    dev = torch.device("cuda:0")
    if args.calibrate_copy and (args.only or args.backward_only):
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only:
        print(json.dumps({args.only: bench_config(K, torch, dev, args.only, 2, 5)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": bench_backward(K, torch, dev, args.warmup, args.steps,
                                                     args.backward_workload)}), flush=True)
        return

    def dev_inputs(w):
        dt = torch.bfloat16
        t = lambda x, d=torch.float32: None if x is None else torch.from_numpy(x).to(dev).to(d)
        return dict(q=t(w.q, dt), k=t(w.k, dt), v=t(w.v, dt), g=t(w.g), beta=t(w.beta), h0=t(w.h0))

    # prefill: three resident input sets (different seeds), shared workspace
    P = PREFILL
    sets = [dev_inputs(make_config("prefill_h16_t4096", seed=s)) for s in range(3)]
    ws_bytes = K.kda_chunk_fwd_workspace_size(P["B"], P["T"], P["H"], P["D"], P["D"], P["chunk"], 0, K.BF16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o_pre = torch.empty((P["B"], P["T"], P["H"], P["D"]), dtype=torch.bfloat16, device=dev)
    h_fin = torch.empty((P["B"], P["H"], P["D"], P["D"]), dtype=torch.float32, device=dev)
    # decode
    Dc = DECODE
    dw = make_config("decode_b256_h32")
    dd = dev_inputs(dw)
    state = dd["h0"]
    o_dec = torch.empty((Dc["B"], 1, Dc["H"], Dc["D"]), dtype=torch.bfloat16, device=dev)

    def prefill(i):
        s = sets[i % 3]
        K.kda_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], initial_state=s["h0"],
                        final_state=h_fin, o=o_pre, chunk=P["chunk"], workspace=ws)

    def decode():
        K.kda_recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state, o=o_dec)

    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        prefill(i)
        decode()
    torch.cuda.synchronize()

    if args.steps < 2:
        raise SystemExit("bench.py needs --steps >= 2 (the prefill time spans calls 2 .. K)")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    prefill(0)
    ev[0].record()
    for i in range(1, args.steps):
        prefill(i)
    ev[1].record()
    for i in range(args.steps):
        decode()
    ev[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = wall * 1e3 / args.steps

    pre_s = ev[0].elapsed_time(ev[1]) / (args.steps - 1) / 1e3
    dec_s = ev[1].elapsed_time(ev[2]) / args.steps / 1e3
    tokens = P["B"] * P["T"]
    pbytes = prefill_bytes(P["B"], P["H"], P["T"], P["D"])
    pflops = prefill_flops(P["B"], P["H"], P["T"], P["D"], P["chunk"])
    dbytes = decode_bytes(Dc["B"], Dc["H"], Dc["D"])
    state_bytes = Dc["B"] * Dc["H"] * Dc["D"] * Dc["D"] * 4 * 2

    traffic = load_traffic()
    rec_hash = source_hash("kda_recurrent.hip", "kda_device.hpp")
    chk_hash = source_hash("kda_chunk.hpp", "kda_device.hpp")
    t_dec = traffic.get("decode")
    t_dec_bytes = t_dec["bytes_per_launch"] if t_dec and t_dec.get("source_hash") == rec_hash else None
    t_pre = traffic.get("prefill")
    t_pre_bytes = t_pre["bytes_per_launch"] if t_pre and t_pre.get("source_hash") == chk_hash else None
    mfma = traffic.get("prefill_mfma")
    mfma_util = mfma.get("mfma_util") if mfma and mfma.get("source_hash") == chk_hash else None

    out = {
        "metric": "KDA chunked prefill tokens/s (H=16,d=128,T=4096) + decode-step state GB/s",
        "value": tokens / pre_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA prefill B1 H16 T4096 d128 chunk64 bf16 (value) + "
                               "decode step B256 H32 d128 fp32 state (decode_state_GBps)",
                   "global_batch": P["B"], "seq_len": P["T"], "heads": P["H"],
                   "d_k": P["D"], "d_v": P["D"], "chunk": P["chunk"],
                   "decode_batch": Dc["B"], "decode_heads": Dc["H"],
                   "parallelism": "single GPU"},
        "prefill_ms": float(pre_s * 1e3),
        "prefill_token_heads_per_s": tokens * P["H"] / pre_s,
        "decode_ms": float(dec_s * 1e3),
        "decode_state_GBps": state_bytes / dec_s / 1e9,
        "decode_total_GBps": dbytes / dec_s / 1e9,
        "roofline": {
            "kernel": "recurrent_kernel<128,128,bf16,bf16> (decode step)",
            "bound": "hbm", "achieved": dbytes / dec_s / 1e9, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": dbytes / dec_s / 1e9 / HBM_PEAK_GBPS,
            "traffic": t_dec_bytes,
            "algorithmic_bytes_per_launch": dbytes,
        },
        "roofline_prefill": {
            "kernel": "kda_chunk_fwd (chunk_prepare + chunk_state)",
            "bound": "hbm", "achieved": pbytes / pre_s / 1e9, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": pbytes / pre_s / 1e9 / HBM_PEAK_GBPS,
            "traffic": t_pre_bytes,
            "algorithmic_bytes_per_launch": pbytes,
            "mfma_tflops_algorithmic": pflops / pre_s / 1e12,
            "mfma_frac_algorithmic": pflops / pre_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "mfma_util_counters": mfma_util,
        },
    }
    if not args.no_extra_legs:
        reps = max(args.steps // 2, 3)
        out["varlen"] = bench_varlen(K, torch, dev, args.warmup, reps)
        out["grouped_heads"] = bench_prefill_shape(K, torch, dev, args.warmup, reps, Hqk=4, Dk=128, Dv=128)
        out["mixed_dims"] = bench_prefill_shape(K, torch, dev, args.warmup, reps, Hqk=16, Dk=64, Dv=128)
        out["value_dim_256"] = bench_prefill_shape(K, torch, dev, args.warmup, reps, Hqk=16, Dk=128,
                                                   Dv=256)
        out["prologue"] = bench_prologue(K, torch, dev, args.warmup, reps)
        out["backward"] = bench_backward(K, torch, dev, args.warmup, reps)
        for name in LARGE_LEGS:
            out[name] = bench_config(K, torch, dev, name, 2, 5)
        for name in LARGE_BWD_LEGS:
            out["backward_" + name] = bench_backward(K, torch, dev, 2, 5, name)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
        if not args.no_extra_legs:
            out["cpu_baseline"]["large_workloads"] = cpu_large_sample()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""The entry points under HIP graph capture (GPU).

A launch sequence that a caller captures must replay correctly: the library
enqueues only kernels (no memset nodes, no host synchronisation), and the
packed form builds its chunk table on the device.  Each graph is replayed
several times, with eager work and synchronisations between the replays, and
every replay is compared bit for bit with the eager result.
"""
import numpy as np
import pytest

import gated_delta_rule_17_amd as K
from kda_workloads import make_inputs, make_lengths, make_varlen
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _t(x, d=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if d is None else t.to(d)


def _replays(name, capture_fn, reset_fn, outputs, eager):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset_fn()
        capture_fn()            # warm-up outside the graph (first-call setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture_fn()
    for rep in range(4):
        reset_fn()
        junk = torch.randn(1 << 20, device="cuda") * 3.0        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs(), eager):
            assert torch.equal(o, e), (name, rep)
        del junk
    say(name, "4 replays equal")


def test_chunk_and_decode_replay():
    import torch
    w = make_inputs(2, 300, 4, 128, 128, dtype="bf16", seed=3, h0_std=0.05)
    q, k, v = (_t(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    g_, beta, h0 = _t(w.g), _t(w.beta), _t(w.h0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(2, 300, 4, 128, 128, 64, 0, K.BF16),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((2, 300, 4, 128), dtype=torch.float32, device="cuda")
    hT = torch.empty_like(h0)
    st = torch.empty_like(h0)
    od = torch.empty((2, 1, 4, 128), dtype=torch.float32, device="cuda")
    q1, k1, v1, g1, b1 = q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous(), \
        g_[:, :1].contiguous(), beta[:, :1].contiguous()

    def run():
        K.kda_chunk_fwd(q, k, v, g_, beta, initial_state=h0, final_state=hT, o=o, chunk=64,
                        workspace=ws)
        st.copy_(hT)
        K.kda_recurrent_step(q1, k1, v1, g1, b1, st, o=od)

    def reset():
        for x in (o, hT, st, od):
            x.fill_(float("nan"))
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone(), hT.clone(), st.clone(), od.clone()]
    _replays("chunk + decode", run, reset, lambda: [o, hT, st, od], eager)


def test_segmented_replay():
    """A long sequence over few heads takes the segmented state pass (phase 1,
    the combine of the segment states, phase 3), all inside the captured
    call; the segment states in the workspace are written before they are
    read in every call, so replays repeat the eager bits."""
    import torch
    T = 256 * 32 + 5
    w = make_inputs(1, T, 2, 32, 32, dtype="bf16", seed=12, h0_std=0.05)
    q, k, v = (_t(x, torch.bfloat16) for x in (w.q, w.k, w.v))
    g_, beta, h0 = _t(w.g), _t(w.beta), _t(w.h0)
    ws = torch.empty(K.kda_chunk_fwd_workspace_size(1, T, 2, 32, 32, 32, 0, K.BF16),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((1, T, 2, 32), dtype=torch.float32, device="cuda")
    hT = torch.empty_like(h0)

    def run():
        K.kda_chunk_fwd(q, k, v, g_, beta, initial_state=h0, final_state=hT, o=o, chunk=32,
                        workspace=ws)

    def reset():
        for x in (o, hT):
            x.fill_(float("nan"))
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone(), hT.clone()]
    _replays("segmented", run, reset, lambda: [o, hT], eager)


def test_packed_replay():
    import torch
    lengths = make_lengths(9, max_len=200, seed=8, edge=(0, 1, 64, 65))
    vw = make_varlen(lengths, 4, 64, 128, dtype="bf16", seed=8, h0_std=0.05)
    w = vw.w
    q, k, v = (_t(x[0], torch.bfloat16) for x in (w.q, w.k, w.v))
    g_, beta, h0, cu = _t(w.g[0]), _t(w.beta[0]), _t(vw.h0), _t(vw.cu)
    N, T = vw.N, int(vw.cu[-1])
    ws = torch.empty(K.kda_chunk_fwd_varlen_workspace_size(N, T, 4, 64, 128, 32, 0, K.BF16),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((T, 4, 128), dtype=torch.float32, device="cuda")
    hT = torch.empty_like(h0)
    o2 = torch.empty_like(o)
    st = torch.empty_like(h0)

    def run():
        K.kda_chunk_fwd_varlen(q, k, v, g_, beta, cu, initial_state=h0, final_state=hT, o=o,
                               chunk=32, workspace=ws)
        st.copy_(h0)
        K.kda_recurrent_varlen(q, k, v, g_, beta, st, cu, o=o2)

    def reset():
        for x in (o, hT, o2, st):
            x.fill_(float("nan"))
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone(), hT.clone(), o2.clone(), st.clone()]
    _replays("packed", run, reset, lambda: [o, hT, o2, st], eager)

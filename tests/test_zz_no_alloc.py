"""kda_chunk_fwd_noalloc (the allocation-free entry point) against
kda_chunk_fwd, through the C ABI (GPU).

Both run the same kernels, so their outputs must agree bit for bit.  Two
calls in a row on one stream, the second with a smaller input, check that
the shared scratch array carries nothing from one call into the next; a
call sized beyond the scratch is rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import gated_delta_rule_17_amd as K
from kda_workloads import make_config, make_inputs
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def _both(w, chunk=64, mode=None):
    import torch
    d = to_device(w)
    mode = mode or w.mode
    shape = (w.B, w.T, w.H, w.Dv)
    o_ref, h_ref = K.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                   initial_state=d["h0"], chunk=chunk, scale=w.scale, mode=mode,
                                   out_dtype=torch.float32)
    o = torch.empty(shape, dtype=torch.float32, device="cuda")
    hT = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device="cuda")
    st = K.lib().kda_chunk_fwd_noalloc(
        ctypes.c_void_p(d["q"].data_ptr()), ctypes.c_void_p(d["k"].data_ptr()),
        ctypes.c_void_p(d["v"].data_ptr()),
        None if d["g"] is None else ctypes.c_void_p(d["g"].data_ptr()),
        ctypes.c_void_p(d["beta"].data_ptr()),
        None if d["h0"] is None else ctypes.c_void_p(d["h0"].data_ptr()),
        ctypes.c_void_p(hT.data_ptr()), ctypes.c_void_p(o.data_ptr()),
        w.B, w.T, w.H, w.H, w.Dk, w.Dv, chunk, ctypes.c_float(w.scale),
        {"channel": 0, "scalar": 1, "none": 2}[mode], K.BF16 if w.dtype == "bf16" else K.F32,
        K.F32, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, K.STATUS.get(st, st)
    torch.cuda.synchronize()
    return (o.cpu().numpy(), hT.cpu().numpy()), (o_ref.cpu().numpy(), h_ref.cpu().numpy())


def test_noalloc_matches_kda_chunk_fwd_twice_then_smaller():
    big = make_config("prefill_h16_t4096")          # 112.5 MiB of records
    small = make_inputs(2, 150, 3, 128, 128, dtype="bf16", seed=41, h0_std=0.1)
    for name, w in (("prefill B1 H16 T4096", big), ("prefill B1 H16 T4096 again", big),
                    ("smaller B2 H3 T150", small)):
        say("noalloc", name)
        (o, h), (o_r, h_r) = _both(w)
        assert np.array_equal(o, o_r), name
        assert np.array_equal(h, h_r), name


def test_noalloc_modes_and_the_python_binding():
    import torch
    for mode in ("scalar", "none"):
        w = make_inputs(1, 200, 2, 64, 64, mode=mode, dtype="f32", seed=42, h0_std=0.1,
                        gate_law="softplus" if mode != "none" else "zero")
        say("noalloc mode", mode)
        (o, h), (o_r, h_r) = _both(w, chunk=32)
        assert np.array_equal(o, o_r) and np.array_equal(h, h_r)
    w = make_inputs(1, 100, 2, 128, 128, dtype="bf16", seed=43, h0_std=0.1)
    d = to_device(w)
    o = torch.empty((1, 100, 2, 128), dtype=torch.bfloat16, device="cuda")
    o2, _ = K.kda_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, o)
    r, _ = K.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"])
    torch.cuda.synchronize()
    assert o2 is o and torch.equal(o, r)


def test_noalloc_rejects_calls_beyond_the_scratch():
    import torch
    T = 8192                                           # B1 H16 T8192: 225 MiB of records
    need = K.kda_chunk_fwd_workspace_size(1, T, 16, 128, 128, 64, 0, K.BF16)
    assert need > K.NOALLOC_SCRATCH_BYTES
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda")
    q, k, v, o = z(1, T, 16, 128), z(1, T, 16, 128), z(1, T, 16, 128), z(1, T, 16, 128)
    g, beta = z(1, T, 16, 128, dt=torch.float32), z(1, T, 16, dt=torch.float32)
    o.fill_(7.0)
    say("noalloc too large")
    with pytest.raises(K.KDAError) as e:
        K.kda_chunk_fwd_noalloc(q, k, v, g, beta, None, None, o)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())                      # nothing was enqueued

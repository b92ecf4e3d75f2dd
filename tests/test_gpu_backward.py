"""Parity of the chunkwise gradient (kda_chunk_bwd) with the gradient oracle
(GPU).

The reference is oracle R-bwd, reverse mode through the token recurrence in
double precision, pinned to finite differences of the forward oracle
(tests/test_oracle_backward.py).  Every gradient (dq, dk, dv, dg, dbeta and
the initial-state gradient) is compared element by element with the
max|delta| / rms measure of the forward tests, at the forward tolerances:
1e-4 for float32 inputs, 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest

import gated_delta_rule_17_amd as K
import oracle
from kda_workloads import make_config, make_cotangents, make_inputs
from tests.conftest import rel_err
from tests.gpu_util import TOL, say

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _t(x, dt=None):
    import torch
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt or torch.float32)


def _run(w, cot, chunk, q=None, k=None, grad="f32"):
    """Run the gradient path; parity is measured on float32 gradients (a
    bf16 gradient is that float32 result rounded, see
    test_bf16_gradients_are_the_rounded_float32_ones)."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gd = torch.bfloat16 if grad == "bf16" else torch.float32
    q = w.q if q is None else q
    k = w.k if k is None else k
    out = K.kda_chunk_bwd(_t(q, dt), _t(k, dt), _t(w.v, dt), _t(w.g), _t(w.beta), _t(cot.do, dt),
                          initial_state=_t(w.h0), d_final_state=_t(cot.dhT), chunk=chunk,
                          scale=w.scale, mode=w.mode, grad_dtype=gd)
    torch.cuda.synchronize()
    res = {}
    for name, key in zip(NAMES, ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")):
        x = out[key]
        res[name] = None if x is None else x.float().cpu().numpy()
    return res


def _compare(label, got, ref, tol):
    errs = {}
    for name in NAMES:
        if ref[name] is None:
            assert got[name] is None, name
            continue
        assert np.isfinite(got[name]).all(), (label, name)
        errs[name] = rel_err(got[name], ref[name])
    print(f"[parity] bwd {label} " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()),
          flush=True)
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, (label, bad)


def _oracle(w, cot, q=None, k=None):
    q = w.q if q is None else q
    k = w.k if k is None else k
    if q.shape[2] != w.H:
        return oracle.recurrent_grouped_bwd(q, k, w.v, w.g, w.beta, w.h0, cot.do, cot.dhT,
                                            scale=w.scale, mode=w.mode)
    return oracle.recurrent_bwd(q, k, w.v, w.g, w.beta, w.h0, cot.do, cot.dhT, scale=w.scale,
                                mode=w.mode)


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("chunk,T", [(16, 64), (32, 100), (64, 200), (64, 64)])
def test_bwd_f32_small(mode, chunk, T):
    w = make_inputs(2, T, 2, 32, 32, mode=mode, dtype="f32", seed=T + chunk, h0_std=0.2,
                    gate_law="softplus" if mode != "none" else "zero")
    cot = make_cotangents(w, seed=1, dhT_std=0.3)
    say("bwd f32", mode, chunk, T)
    _compare(f"f32 {mode} C{chunk} T{T}", _run(w, cot, chunk), _oracle(w, cot), TOL["f32"])


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (16, 128), (128, 16), (64, 32), (128, 128)])
def test_bwd_f32_dims(Dk, Dv):
    w = make_inputs(1, 150, 2, Dk, Dv, mode="channel", dtype="f32", seed=Dk + 3 * Dv,
                    h0_std=0.2)
    cot = make_cotangents(w, seed=2, dhT_std=0.3)
    say("bwd f32 dims", Dk, Dv)
    _compare(f"f32 Dk{Dk} Dv{Dv}", _run(w, cot, 64), _oracle(w, cot), TOL["f32"])


def test_bwd_without_initial_state_or_final_gradient():
    w = make_inputs(1, 90, 3, 64, 64, mode="channel", dtype="f32", seed=9, h0_std=0.0)
    cot = make_cotangents(w, seed=3)
    assert w.h0 is None and cot.dhT is None
    say("bwd zero state")
    _compare("f32 zero state", _run(w, cot, 32), _oracle(w, cot), TOL["f32"])


@pytest.mark.parametrize("Hqk,G", [(2, 2), (1, 4)])
def test_bwd_grouped_heads(Hqk, G):
    w = make_inputs(1, 130, Hqk * G, 64, 32, mode="channel", dtype="f32", seed=40 + G,
                    h0_std=0.1)
    q = np.ascontiguousarray(w.q[:, :, ::G])
    k = np.ascontiguousarray(w.k[:, :, ::G])
    cot = make_cotangents(w, seed=4, dhT_std=0.2)
    say("bwd grouped", Hqk, G)
    _compare(f"grouped Hqk{Hqk} G{G}", _run(w, cot, 64, q, k), _oracle(w, cot, q, k), TOL["f32"])


def test_bwd_zero_length_copies_the_final_state_gradient():
    import torch
    w = make_inputs(1, 0, 2, 32, 32, dtype="f32", seed=5)
    cot = make_cotangents(w, seed=5, dhT_std=1.0)
    say("bwd T=0")
    got = _run(w, cot, 64)
    np.testing.assert_array_equal(got["dh0"], cot.dhT)
    assert got["dq"].size == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
def test_bwd_bf16_mid(mode):
    w = make_inputs(1, 512, 2, 128, 128, mode=mode, dtype="bf16", seed=77, h0_std=0.01,
                    gate_law="softplus" if mode != "none" else "zero", gate_shift=2.0)
    cot = make_cotangents(w, seed=6, dhT_std=0.1)
    say("bwd bf16", mode)
    _compare(f"bf16 {mode} T512", _run(w, cot, 64), _oracle(w, cot), TOL["bf16"])


@pytest.mark.parametrize("chunk,Dk,Dv", [(32, 128, 128), (32, 64, 64), (64, 128, 64),
                                          (64, 64, 128), (16, 128, 128), (32, 32, 32)])
def test_bwd_bf16_chunks_and_dims(chunk, Dk, Dv):
    """bf16 inputs over chunk lengths and head dims, ragged tail.  With bf16
    inputs the preparation's products with T, Aqk and scale Q e^G run on bf16
    matrix cores over three-part splits where the chunk is a multiple of 32
    and each thread holds whole 8-row groups (the first four cases), the
    float32 path elsewhere.  Both keep float32-level accuracy, so the bound
    here is 2e-3, a tenth of the bf16 bar: a split that lost a part (about
    2^-16 of each operand) would fail it."""
    w = make_inputs(1, 200, 2, Dk, Dv, mode="channel", dtype="bf16", seed=40 + chunk + Dk + Dv,
                    h0_std=0.05)
    cot = make_cotangents(w, seed=3, dhT_std=0.1)
    say("bwd bf16 chunk", chunk, "dims", Dk, Dv)
    _compare(f"bf16 C{chunk} Dk{Dk} Dv{Dv}", _run(w, cot, chunk), _oracle(w, cot), 2e-3)


@pytest.mark.parametrize("dtype,chunk,Dk", [("f32", 64, 128), ("f32", 32, 64), ("bf16", 64, 128),
                                            ("bf16", 32, 16)])
def test_bwd_value_dim_256(dtype, chunk, Dk):
    """d_v = 256 (eight 32-column slices in the gradient kernel, sixteen
    value tiles per head in the carries), ragged tail."""
    w = make_inputs(1, 150, 2, Dk, 256, mode="channel", dtype=dtype, seed=256 + Dk + chunk,
                    h0_std=0.05)
    cot = make_cotangents(w, seed=4, dhT_std=0.1)
    say("bwd d_v 256", dtype, chunk, Dk)
    tol = TOL["f32"] if dtype == "f32" else 2e-3
    _compare(f"{dtype} d_v 256 C{chunk} Dk{Dk}", _run(w, cot, chunk), _oracle(w, cot), tol)


@pytest.mark.parametrize("Hqk,G", [(4, 1), (2, 2)])
def test_bf16_gradients_are_the_rounded_float32_ones(Hqk, G):
    from kda_workloads import bf16_round
    w = make_inputs(1, 200, Hqk * G, 64, 64, mode="channel", dtype="bf16", seed=8, h0_std=0.01)
    q = np.ascontiguousarray(w.q[:, :, ::G])
    k = np.ascontiguousarray(w.k[:, :, ::G])
    cot = make_cotangents(w, seed=8, dhT_std=0.1)
    say("bwd bf16 gradient storage", Hqk, G)
    g32 = _run(w, cot, 64, q, k, grad="f32")
    g16 = _run(w, cot, 64, q, k, grad="bf16")
    for name in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(g16[name], bf16_round(g32[name].astype(np.float32)))
    for name in ("dg", "dbeta", "dh0"):
        np.testing.assert_array_equal(g16[name], g32[name])


def test_bwd_strong_gates_within_range():
    # per-token log gates down to -4.5 on half the channels: 16-token decays
    # reach e^-70, inside the range the kernels support
    w = make_inputs(1, 192, 2, 64, 64, mode="channel", dtype="f32", seed=12, h0_std=0.1)
    g = w.g.copy()
    g[..., ::2] = -4.5 * np.random.default_rng(0).uniform(0.5, 1.0, g[..., ::2].shape)
    w.g = g.astype(np.float32)
    cot = make_cotangents(w, seed=7, dhT_std=0.2)
    say("bwd strong gates")
    _compare("f32 strong gates", _run(w, cot, 64), _oracle(w, cot), TOL["f32"])


def _extreme_gates(mode, dtype, seed=21, T=150, D=64):
    """The forward's gate-boundary cases: three hard-forget tokens (g = -30)
    inside one 16-token block, a single channel at g = -40 for four tokens
    followed by exact keeps (g = 0), one token at g = -95 (beyond the float32
    exponent range on its own), and a run of g = 0."""
    w = make_inputs(1, T, 2, D, D, mode=mode, dtype=dtype, seed=seed, h0_std=0.2)
    w.g[:, 3:6] = -30.0
    if mode == "channel":
        w.g[0, 40:44, 0, 5] = -40.0
        w.g[0, 44:60, 0, 5] = 0.0
        w.g[0, 70, 1, :] = -95.0
    else:
        w.g[0, 70, 1] = -95.0
    w.g[0, 100:128] = 0.0
    return w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["channel", "scalar"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_bwd_hard_forget_and_extreme_gates(dtype, mode, chunk):
    """Gradients at the gate boundaries the forward supports ([GN] "Gated
    DeltaNet: forget the whole state first"): key channels whose decay
    across a 16-token block leaves the factored range take their in-block
    terms exactly in both gradient kernels.  Everything stays finite and
    matches R-bwd at the forward tolerances."""
    w = _extreme_gates(mode, dtype)
    cot = make_cotangents(w, seed=9, dhT_std=0.2)
    say("bwd extreme gates", mode, dtype, chunk)
    got = _run(w, cot, chunk)
    _compare(f"extreme gates {mode} {dtype} C{chunk}", got, _oracle(w, cot), TOL[dtype])


def test_bwd_extreme_gates_every_block_deterministic():
    """Every 16-token block holds three hard-forget tokens (all channels of
    all blocks on the exact path at once, d 128); the gradients match R-bwd
    and a second call gives the same bits."""
    w = make_inputs(1, 192, 2, 128, 128, mode="channel", dtype="bf16", seed=33, h0_std=0.1)
    for b0 in range(0, 192, 16):
        w.g[0, b0 + 5:b0 + 8] = -30.0
    cot = make_cotangents(w, seed=10, dhT_std=0.1)
    say("bwd extreme gates every block")
    got = _run(w, cot, 64)
    _compare("extreme gates every block", got, _oracle(w, cot), TOL["bf16"])
    again = _run(w, cot, 64)
    for n in NAMES:
        if got[n] is not None:
            np.testing.assert_array_equal(got[n], again[n], err_msg=n)


def test_bwd_training_shape_every_sequence():
    """The training shape at full size (B8 H32 T8192 d128, chunk 64, bf16, mixed
    fast and slow channels): 32768 chunk records, a workspace whose float
    offsets pass 2^31, run in batch groups.  The gradient oracle runs on every
    one of the 256 sequences, one batch entry at a time (bounded host memory);
    each entry's measure and the worst single sequence are held to the bound."""
    w = make_config("train_b8_h32_t8192")
    cot = make_cotangents(w, seed=0, dhT_std=0.01)
    say("bwd train_b8_h32_t8192")
    got = _run(w, cot, 64)
    worst = {}
    for b in range(w.B):
        sl = lambda x: None if x is None else np.ascontiguousarray(x[b:b + 1])
        ref = oracle.recurrent_bwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta), sl(w.h0),
                                   sl(cot.do), sl(cot.dhT), scale=w.scale, mode=w.mode)
        sub = {n: None if got[n] is None else sl(got[n]) for n in NAMES}
        _compare(f"training shape, b {b}, all 32 heads", sub, ref, TOL["bf16"])
        for n in NAMES:
            if ref[n] is None:
                continue
            for h in range(w.H):
                x, y = (sub[n][0, h], ref[n][0, h]) if n == "dh0" else \
                    (sub[n][0, :, h], ref[n][0, :, h])
                e = rel_err(x, y)
                if e > worst.get(n, (0.0, None))[0]:
                    worst[n] = (e, (b, h))
        del ref, sub
    print("[parity] bwd training shape worst sequence: " +
          " ".join(f"{n} {e:.2e}@{bh}" for n, (e, bh) in worst.items()), flush=True)
    assert all(e <= TOL["bf16"] for e, _ in worst.values()), worst


def test_bwd_batch_groups_with_grouped_heads():
    """Records over 4 GiB run in groups of whole batch entries: B3 H32 T8192
    d128 (2 GiB of records per entry) runs as entries {0, 1} and then {2},
    here with two value heads per query/key head, so the second group's
    float partials of dq and dk and their sum land at that entry's offsets.
    The grouped-head gradient oracle runs on every entry, one at a time."""
    w = make_inputs(3, 8192, 32, 128, 128, mode="channel", dtype="bf16", seed=21, h0_std=0.02)
    q = np.ascontiguousarray(w.q[:, :, ::2])
    k = np.ascontiguousarray(w.k[:, :, ::2])
    cot = make_cotangents(w, seed=21, dhT_std=0.05)
    assert K.kda_chunk_bwd_workspace_size(3, 8192, 32, 16, 128, 128, 64, w.mode, K.BF16) == \
        K.kda_chunk_bwd_workspace_size(2, 8192, 32, 16, 128, 128, 64, w.mode, K.BF16)
    say("bwd batch groups, grouped heads, B3 H32 T8192")
    got = _run(w, cot, 64, q, k)
    for b in range(w.B):
        sl = lambda x: None if x is None else np.ascontiguousarray(x[b:b + 1])
        ref = oracle.recurrent_grouped_bwd(sl(q), sl(k), sl(w.v), sl(w.g), sl(w.beta), sl(w.h0),
                                           sl(cot.do), sl(cot.dhT), scale=w.scale, mode=w.mode)
        sub = {n: None if got[n] is None else sl(got[n]) for n in NAMES}
        _compare(f"batch groups, grouped heads, entry {b}", sub, ref, TOL["bf16"])


def test_bwd_full_size_prefill_every_head():
    """The prefill workload at full size (B1 H16 T4096 d128, bf16), in the
    launch configuration the benchmark times; the oracle runs on all sixteen
    heads."""
    w = make_config("prefill_h16_t4096")
    cot = make_cotangents(w, seed=0, dhT_std=0.01)
    say("bwd full size prefill")
    got = _run(w, cot, 64)
    _compare("full size prefill, every head", got, _oracle(w, cot), TOL["bf16"])


# ---- packed variable-length batches ----------------------------------------
from kda_workloads import make_lengths, make_varlen  # noqa: E402

EDGE = (0, 1, 2, 15, 16, 17, 63, 64, 65, 130)


def _varlen_cot(vw, seed, dhT_std):
    import numpy as _np
    w = vw.w
    cot = make_cotangents(w, seed=seed)
    do = cot.do[0]
    dhT = None
    if dhT_std > 0:
        r = _np.random.default_rng(_np.random.SeedSequence([seed, 0xD1]))
        dhT = (dhT_std * r.standard_normal((vw.N, w.H, w.Dk, w.Dv))).astype(_np.float32)
    return do, dhT


def _run_varlen(vw, do, dhT, chunk, q=None, k=None):
    import torch
    w = vw.w
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = w.q[0] if q is None else q
    k = w.k[0] if k is None else k
    g = None if w.g is None else w.g[0]
    cu = torch.from_numpy(vw.cu).cuda()
    out = K.kda_chunk_bwd_varlen(_t(q, dt), _t(k, dt), _t(w.v[0], dt), _t(g), _t(w.beta[0]),
                                 _t(do, dt), cu, initial_state=_t(vw.h0), d_final_state=_t(dhT),
                                 chunk=chunk, scale=w.scale, mode=w.mode,
                                 grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return {n: None if out[key] is None else out[key].float().cpu().numpy()
            for n, key in zip(NAMES, ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state"))}


def _oracle_varlen(vw, do, dhT, q=None, k=None):
    w = vw.w
    q = w.q[0] if q is None else q
    k = w.k[0] if k is None else k
    return oracle.recurrent_varlen_bwd(q, k, w.v[0], None if w.g is None else w.g[0], w.beta[0],
                                       vw.cu, vw.h0, do, dhT, scale=w.scale, mode=w.mode)


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_bwd_varlen_ragged_f32(mode, chunk):
    lengths = make_lengths(14, max_len=200, seed=chunk, edge=EDGE)
    vw = make_varlen(lengths, 2, 32, 32, mode=mode, dtype="f32", seed=7 + chunk, h0_std=0.2,
                     gate_law="softplus" if mode != "none" else "zero")
    do, dhT = _varlen_cot(vw, 3, 0.3)
    say("bwd varlen f32", mode, chunk, list(lengths))
    _compare(f"varlen f32 {mode} C{chunk}", _run_varlen(vw, do, dhT, chunk),
             _oracle_varlen(vw, do, dhT), TOL["f32"])


def test_bwd_varlen_grouped_heads_bf16():
    lengths = make_lengths(10, max_len=300, seed=4, edge=(0, 1, 64, 65))
    vw = make_varlen(lengths, 4, 64, 32, dtype="bf16", seed=12, h0_std=0.05)
    q = np.ascontiguousarray(vw.w.q[0][:, ::2])
    k = np.ascontiguousarray(vw.w.k[0][:, ::2])
    do, dhT = _varlen_cot(vw, 5, 0.1)
    say("bwd varlen grouped bf16", list(lengths))
    _compare("varlen grouped bf16", _run_varlen(vw, do, dhT, 64, q, k),
             _oracle_varlen(vw, do, dhT, q, k), TOL["bf16"])


def test_bwd_varlen_equal_lengths_match_dense_bitwise():
    import torch
    N, L, H, D = 3, 150, 2, 64
    vw = make_varlen([L] * N, H, D, D, dtype="bf16", seed=5, h0_std=0.05)
    do, dhT = _varlen_cot(vw, 6, 0.1)
    say("bwd varlen = dense")
    got = _run_varlen(vw, do, dhT, 64)
    w = vw.w
    r = lambda x: None if x is None else np.ascontiguousarray(x[0].reshape((N, L) + x.shape[2:]))
    bf = torch.bfloat16
    dense = K.kda_chunk_bwd(_t(r(w.q), bf), _t(r(w.k), bf), _t(r(w.v), bf), _t(r(w.g)),
                            _t(r(w.beta)), _t(np.ascontiguousarray(do.reshape(N, L, H, D)), bf),
                            initial_state=_t(vw.h0), d_final_state=_t(dhT), chunk=64,
                            scale=w.scale, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for name, key in zip(NAMES, ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")):
        x = dense[key].cpu().numpy()
        np.testing.assert_array_equal(got[name], x.reshape(got[name].shape), err_msg=name)


def test_bwd_varlen_empty_sequences_pass_the_state_gradient():
    vw = make_varlen([0, 5, 0], 2, 32, 32, dtype="f32", seed=9, h0_std=0.3)
    do, dhT = _varlen_cot(vw, 7, 1.0)
    say("bwd varlen empty")
    got = _run_varlen(vw, do, dhT, 64)
    np.testing.assert_array_equal(got["dh0"][0], dhT[0])
    np.testing.assert_array_equal(got["dh0"][2], dhT[2])
    _compare("varlen empty", got, _oracle_varlen(vw, do, dhT), TOL["f32"])


def test_bwd_varlen_empty_sequences_matrix_core_carries():
    """bf16 inputs at d = 64, chunk 64 take the matrix-core carries
    (bwd_states_mc): an empty sequence there passes its final-state gradient
    through unchanged, and the others match the oracle."""
    vw = make_varlen([0, 70, 0, 130], 2, 64, 64, dtype="bf16", seed=10, h0_std=0.05)
    do, dhT = _varlen_cot(vw, 11, 0.1)
    say("bwd varlen empty, matrix-core carries")
    got = _run_varlen(vw, do, dhT, 64)
    np.testing.assert_array_equal(got["dh0"][0], dhT[0])
    np.testing.assert_array_equal(got["dh0"][2], dhT[2])
    _compare("varlen empty bf16 d64", got, _oracle_varlen(vw, do, dhT), TOL["bf16"])


def test_bwd_varlen_serving_mix_every_sequence():
    """The serving mix (64 sequences, lengths log-uniform in [1, 2048], H16
    d128 bf16) through one call; every sequence against the oracle, each
    against its own scale."""
    lengths = make_lengths(64, max_len=2048, seed=17, edge=(1, 64, 2048))
    vw = make_varlen(lengths, 16, 128, 128, dtype="bf16", seed=17, h0_std=0.02)
    do, dhT = _varlen_cot(vw, 8, 0.02)
    say("bwd varlen serving mix")
    got = _run_varlen(vw, do, dhT, 64)
    w = vw.w
    for n in range(vw.N):
        s, e = int(vw.cu[n]), int(vw.cu[n + 1])
        sl = lambda x: None if x is None else np.ascontiguousarray(x[0][s:e])[None]
        ref = oracle.recurrent_bwd(sl(w.q), sl(w.k), sl(w.v), sl(w.g), sl(w.beta),
                                   vw.h0[n:n + 1], np.ascontiguousarray(do[s:e])[None],
                                   dhT[n:n + 1], scale=w.scale, mode=w.mode)
        sub = {name: (got[name][n:n + 1] if name == "dh0" else got[name][s:e][None])
               for name in NAMES}
        _compare(f"varlen serving seq {n} len {e - s}", sub, ref, TOL["bf16"])

"""Pins of the gradient oracles (CPU only).

Oracle R-bwd (reverse mode through the token recurrence) is pinned to
central finite differences of oracle R: for the scalar loss
L = sum(dO * o) + sum(dHT * H_T) the derivative along every single input
element must match (L(x + h) - L(x - h)) / 2h.  That check is independent of
how the gradient is derived, so a dropped term, a wrong sign or a
transposed operand anywhere in R-bwd fails it; the planted mistakes below
show that it does.  The chunkwise gradient (oracle C-bwd) and the grouped
gradient are then pinned to R-bwd, and the grouped one to finite
differences of the grouped forward as well; the packed-batch gradient to
finite differences of the packed forward and to the dense batch.
"""
import functools

import numpy as np
import pytest

import oracle

MODES = ("channel", "scalar", "none")


def _case(seed, B=1, T=7, H=2, Dk=3, Dv=4, mode="channel", h0=True, dhT=True, Hqk=None):
    r = np.random.default_rng(seed)
    Hq = H if Hqk is None else Hqk
    q = r.standard_normal((B, T, Hq, Dk))
    k = r.standard_normal((B, T, Hq, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.1, 1.0, (B, T, H))
    if mode == "channel":
        g = -r.uniform(0.0, 1.0, (B, T, H, Dk))
    elif mode == "scalar":
        g = -r.uniform(0.0, 1.0, (B, T, H))
    else:
        g = None
    s0 = 0.5 * r.standard_normal((B, H, Dk, Dv)) if h0 else None
    do = r.standard_normal((B, T, H, Dv))
    dh = r.standard_normal((B, H, Dk, Dv)) if dhT else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=s0), do, dh


def _loss(fwd, inputs, do, dhT, mode, scale):
    o, hT = fwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"], inputs["beta"],
                inputs["h0"], scale=scale, mode=mode)
    val = float(np.sum(do * o))
    if dhT is not None:
        val += float(np.sum(dhT * hT))
    return val


def _finite_differences(fwd, inputs, do, dhT, mode, scale, step=1e-5):
    grads = {}
    names = ["q", "k", "v", "beta", "h0"] + (["g"] if mode != "none" else [])
    for name in names:
        x = inputs[name]
        if x is None:
            continue
        gx = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = x[idx]
            x[idx] = keep + step
            lp = _loss(fwd, inputs, do, dhT, mode, scale)
            x[idx] = keep - step
            lm = _loss(fwd, inputs, do, dhT, mode, scale)
            x[idx] = keep
            gx[idx] = (lp - lm) / (2 * step)
        grads["d" + name] = gx
    return grads


def _check_fd(bwd, fwd=oracle.recurrent, seed=0, mode="channel", tol=2e-7, **kw):
    inputs, do, dhT = _case(seed, mode=mode, **kw)
    scale = 0.7
    got = bwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"], inputs["beta"],
              inputs["h0"], do, dhT, scale=scale, mode=mode)
    if inputs["h0"] is None:
        # the gradient of a zero initial state is checked as a zero array
        Dk, Dv = inputs["q"].shape[-1], inputs["v"].shape[-1]
        B, H = inputs["v"].shape[0], inputs["v"].shape[2]
        inputs["h0"] = np.zeros((B, H, Dk, Dv))
    fd = _finite_differences(fwd, inputs, do, dhT, mode, scale)
    for name, ref in fd.items():
        err = np.max(np.abs(got[name] - ref)) / max(1.0, np.max(np.abs(ref)))
        assert err < tol, f"{name}: finite-difference mismatch {err:.3e} ({mode})"
    if mode == "none":
        assert got["dg"] is None


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("h0,dhT", [(True, True), (False, True), (True, False)])
def test_recurrent_bwd_matches_finite_differences(mode, h0, dhT):
    _check_fd(oracle.recurrent_bwd, seed=11, mode=mode, h0=h0, dhT=dhT)


def test_recurrent_bwd_finite_differences_two_batches_long():
    # T > 64 crosses a checkpoint segment of the oracle's reverse sweep
    _check_fd(oracle.recurrent_bwd, seed=5, mode="channel", B=2, T=70, H=1, Dk=2, Dv=2)


def test_recurrent_bwd_empty_sequence():
    inputs, do, dhT = _case(2, T=0)
    got = oracle.recurrent_bwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"],
                               inputs["beta"], inputs["h0"], do, dhT)
    np.testing.assert_array_equal(got["dh0"], dhT)
    assert got["dq"].size == 0


BWD_MUTANTS = {
    101: "query gradient from the state before the write",
    102: "sign of the prediction path flipped",
    103: "key gradient of the prediction dropped",
    104: "gate chain factor alpha dropped",
    105: "adjoint state not decayed",
}


@pytest.mark.parametrize("mutant", sorted(BWD_MUTANTS),
                         ids=lambda m: BWD_MUTANTS[m].replace(" ", "_"))
def test_finite_differences_catch_planted_gradient_mistakes(mutant):
    bwd = functools.partial(oracle.recurrent_bwd, mutant=mutant)
    caught = False
    for mode in ("channel", "scalar"):
        try:
            _check_fd(bwd, seed=3, mode=mode)
        except AssertionError:
            caught = True
    assert caught, f"finite differences missed mutant {mutant}: {BWD_MUTANTS[mutant]}"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("chunk,T", [(1, 5), (3, 10), (4, 16), (16, 37), (64, 64)])
def test_chunkwise_bwd_equals_recurrent_bwd(mode, chunk, T):
    inputs, do, dhT = _case(21 + chunk, B=2, T=T, H=2, Dk=5, Dv=3, mode=mode)
    args = (inputs["q"], inputs["k"], inputs["v"], inputs["g"], inputs["beta"],
            inputs["h0"], do, dhT)
    ref = oracle.recurrent_bwd(*args, scale=0.4, mode=mode)
    got = oracle.chunkwise_bwd(*args, chunk=chunk, scale=0.4, mode=mode)
    for name in ("dq", "dk", "dv", "dbeta", "dh0") + (("dg",) if mode != "none" else ()):
        err = np.max(np.abs(got[name] - ref[name])) / max(1e-30, np.max(np.abs(ref[name])))
        assert err < 1e-11, f"{name} chunk={chunk} {mode}: {err:.3e}"


def test_chunkwise_bwd_strong_decay():
    # log gates down to -4 per token: chunk-internal decays reach e^-250,
    # far outside single-precision range; the differences keep fp64 exact
    inputs, do, dhT = _case(8, T=64, H=1, Dk=4, Dv=4)
    inputs["g"] = -4.0 * np.random.default_rng(1).uniform(0, 1, inputs["g"].shape)
    args = (inputs["q"], inputs["k"], inputs["v"], inputs["g"], inputs["beta"],
            inputs["h0"], do, dhT)
    ref = oracle.recurrent_bwd(*args)
    got = oracle.chunkwise_bwd(*args, chunk=64)
    for name in ("dq", "dk", "dv", "dbeta", "dh0", "dg"):
        err = np.max(np.abs(got[name] - ref[name])) / max(1e-30, np.max(np.abs(ref[name])))
        assert err < 1e-10, f"{name}: {err:.3e}"


@pytest.mark.parametrize("mode", ("channel", "scalar"))
def test_grouped_bwd_matches_finite_differences(mode):
    _check_fd(oracle.recurrent_grouped_bwd, fwd=oracle.recurrent_grouped, seed=4,
              mode=mode, H=4, Hqk=2, T=5, Dk=3, Dv=2)


def test_grouped_bwd_sums_over_the_group():
    inputs, do, dhT = _case(9, T=9, H=6, Hqk=2, Dk=4, Dv=3)
    got = oracle.recurrent_grouped_bwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"],
                                       inputs["beta"], inputs["h0"], do, dhT)
    idx = np.arange(6) // 3
    ref = oracle.recurrent_bwd(inputs["q"][:, :, idx], inputs["k"][:, :, idx], inputs["v"],
                               inputs["g"], inputs["beta"], inputs["h0"], do, dhT)
    for name in ("dq", "dk"):
        summed = ref[name].reshape(1, 9, 2, 3, 4).sum(axis=3)
        np.testing.assert_allclose(got[name], summed, rtol=1e-12, atol=1e-12)
    for name in ("dv", "dbeta", "dg", "dh0"):
        np.testing.assert_array_equal(got[name], ref[name])


def _packed_case(seed, lengths, H=2, Hq=2, Dk=3, Dv=2, mode="channel"):
    r = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, N = int(cu[-1]), len(lengths)
    q = r.standard_normal((T, Hq, Dk))
    k = r.standard_normal((T, Hq, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, Dv))
    beta = r.uniform(0.1, 1.0, (T, H))
    g = -r.uniform(0, 1, (T, H, Dk)) if mode == "channel" else \
        (-r.uniform(0, 1, (T, H)) if mode == "scalar" else None)
    h0 = 0.5 * r.standard_normal((N, H, Dk, Dv))
    do = r.standard_normal((T, H, Dv))
    dhT = r.standard_normal((N, H, Dk, Dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), do, dhT, cu


@pytest.mark.parametrize("mode", MODES)
def test_varlen_bwd_matches_finite_differences(mode):
    inputs, do, dhT, cu = _packed_case(31, [3, 0, 4, 1], H=2, Hq=1, mode=mode)
    fwd = lambda q, k, v, g, beta, h0, scale, mode: oracle.recurrent_varlen(
        q, k, v, g, beta, cu, h0, scale=scale, mode=mode)
    got = oracle.recurrent_varlen_bwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"],
                                      inputs["beta"], cu, inputs["h0"], do, dhT, scale=0.6,
                                      mode=mode)
    fd = _finite_differences(fwd, inputs, do, dhT, mode, 0.6)
    for name, ref in fd.items():
        err = np.max(np.abs(got[name] - ref)) / max(1.0, np.max(np.abs(ref)))
        assert err < 2e-7, (name, err)
    # the empty sequence passes its final-state gradient through
    np.testing.assert_array_equal(got["dh0"][1], dhT[1])


def test_varlen_bwd_equal_lengths_equal_the_dense_batch():
    inputs, do, dhT, cu = _packed_case(32, [5, 5, 5], H=2, Hq=2, Dk=4, Dv=3)
    got = oracle.recurrent_varlen_bwd(inputs["q"], inputs["k"], inputs["v"], inputs["g"],
                                      inputs["beta"], cu, inputs["h0"], do, dhT)
    r = lambda x: x.reshape((3, 5) + x.shape[1:])
    ref = oracle.recurrent_bwd(r(inputs["q"]), r(inputs["k"]), r(inputs["v"]), r(inputs["g"]),
                               r(inputs["beta"]), inputs["h0"], r(do), dhT)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        np.testing.assert_array_equal(got[name], ref[name].reshape(got[name].shape))
    np.testing.assert_array_equal(got["dh0"], ref["dh0"])

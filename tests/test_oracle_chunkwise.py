"""Oracle C (chunkwise, NumPy) against oracle R (recurrence, C), CPU only.

Pin P8: the chunkwise form must give exactly the same states and outputs as
the token loop (GeekNews #31925, section "Chunkwise KDA: recasting the
recurrence as matrix products"; the F29 outline's "KDA recurrent and
chunkwise with equality tests").  Chunk length 1 degenerates to the
recurrence, so this also pins the reconstructed steps 5-7 of the chunk form.
"""
import numpy as np
import pytest

import oracle
from kda_workloads import make_inputs, make_config
from tests.conftest import rel_err


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("T", [1, 7, 64])
@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64])
def test_chunk_equals_recurrence(mode, T, chunk):
    w = make_inputs(2, T, 2, 8, 6, mode=mode, dtype="f32", seed=T * 100 + chunk,
                    gate_law="softplus", h0_std=0.3)
    o_r, h_r = oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=mode)
    for solve in ("substitution", "ut"):
        o_c, h_c = oracle.chunkwise(w.q, w.k, w.v, w.g, w.beta, w.h0, chunk=chunk,
                                    scale=w.scale, mode=mode, solve=solve)
        assert rel_err(o_c, o_r) < 1e-12, (solve, rel_err(o_c, o_r))
        assert rel_err(h_c, h_r) < 1e-12, (solve, rel_err(h_c, h_r))


def test_chunk_equals_recurrence_tiny_config():
    """The single-head fp32 workload (T=64, d=16) at chunk 16."""
    w = make_config("tiny_f32")
    o_r, h_r = oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=w.mode)
    o_c, h_c = oracle.chunkwise(w.q, w.k, w.v, w.g, w.beta, w.h0, chunk=16,
                                scale=w.scale, mode=w.mode)
    assert rel_err(o_c, o_r) < 1e-12 and rel_err(h_c, h_r) < 1e-12


def test_chunk_strong_decay_no_overflow():
    """Cumulative log-decay far below -88 inside a chunk (fp32 exp range) is
    handled because the chunk form only exponentiates differences G_i - G_j
    with j <= i (the "log-space decay ratios" of the F29 outline)."""
    w = make_inputs(1, 64, 1, 8, 8, mode="channel", dtype="f32", seed=5,
                    gate_law="softplus", gate_shift=3.0, h0_std=0.1)
    assert np.cumsum(w.g[0, :, 0], axis=0).min() < -150
    o_r, h_r = oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale)
    o_c, h_c = oracle.chunkwise(w.q, w.k, w.v, w.g, w.beta, w.h0, chunk=64, scale=w.scale)
    assert np.isfinite(o_c).all()
    assert rel_err(o_c, o_r) < 1e-12 and rel_err(h_c, h_r) < 1e-12


def test_unnormalised_keys():
    """The chunk form is the general formula: it matches the recurrence with
    keys that are not unit length (the F29 exercise that breaks the delta
    memory with unnormalised keys)."""
    w = make_inputs(1, 33, 2, 8, 8, mode="channel", dtype="f32", seed=6,
                    normalise_k=False, h0_std=0.2)
    o_r, h_r = oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale)
    o_c, h_c = oracle.chunkwise(w.q, w.k, w.v, w.g, w.beta, w.h0, chunk=16, scale=w.scale)
    assert rel_err(o_c, o_r) < 1e-11 and rel_err(h_c, h_r) < 1e-11

"""Pins of the packed variable-length oracle (CPU only).

The packed form is defined as N separate recurrences (GeekNews #31925,
section "Fused recurrent kernel for decode": sequences run independently).
The pins check the wrapper against things other than itself:
- equal lengths: the packed batch is the dense [N, L] batch of oracle R
  (catches offset and reshape mistakes);
- independence: changing one sequence leaves every other one bitwise
  unchanged (catches a state or token leaking across a boundary);
- the chunkwise oracle C, run per sequence, agrees (a second implementation);
- an empty sequence keeps its initial state.
"""
import numpy as np
import pytest

import oracle
from kda_workloads import make_lengths, make_varlen
from tests.conftest import rel_err


def _packed(vw):
    w = vw.w
    g = None if w.g is None else w.g[0]
    return w.q[0], w.k[0], w.v[0], g, w.beta[0]


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
def test_equal_lengths_equal_dense_batch(mode):
    N, L = 4, 9
    vw = make_varlen([L] * N, 2, 8, 6, mode=mode, dtype="f32", seed=11, h0_std=0.3)
    q, k, v, g, beta = _packed(vw)
    o, hT = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, vw.h0, scale=vw.w.scale, mode=mode)
    rs = lambda x: None if x is None else x.reshape((N, L) + x.shape[1:])
    o_d, h_d = oracle.recurrent(rs(q), rs(k), rs(v), rs(g), rs(beta), vw.h0,
                                scale=vw.w.scale, mode=mode)
    assert np.array_equal(o.reshape(o_d.shape), o_d)
    assert np.array_equal(hT, h_d)


def test_sequences_are_independent():
    lengths = [5, 0, 17, 1, 33]
    vw = make_varlen(lengths, 2, 8, 8, dtype="f32", seed=5, h0_std=0.2)
    q, k, v, g, beta = _packed(vw)
    o, hT = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, vw.h0, scale=vw.w.scale)
    # perturb every input of sequence 2 and its initial state
    s, e = vw.cu[2], vw.cu[3]
    q2, k2, v2, g2, b2 = (x.copy() for x in (q, k, v, g, beta))
    for x in (q2, k2, v2):
        x[s:e] += 0.5
    g2[s:e] *= 2.0
    b2[s:e] = 1.0 - b2[s:e]
    h02 = vw.h0.copy()
    h02[2] += 1.0
    o2, hT2 = oracle.recurrent_varlen(q2, k2, v2, g2, b2, vw.cu, h02, scale=vw.w.scale)
    for n in range(len(lengths)):
        a, b = vw.cu[n], vw.cu[n + 1]
        same = n != 2
        assert np.array_equal(o[a:b], o2[a:b]) == same or b == a
        assert np.array_equal(hT[n], hT2[n]) == same


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
def test_chunkwise_per_sequence_agrees(mode):
    lengths = make_lengths(6, max_len=40, seed=2, edge=(0, 1, 16, 17))
    vw = make_varlen(lengths, 2, 8, 8, mode=mode, dtype="f32", seed=9, h0_std=0.2)
    q, k, v, g, beta = _packed(vw)
    o, hT = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, vw.h0, scale=vw.w.scale, mode=mode)
    for n in range(vw.N):
        a, b = int(vw.cu[n]), int(vw.cu[n + 1])
        if a == b:
            continue
        sl = lambda x: None if x is None else x[a:b][None]
        o_c, h_c = oracle.chunkwise(sl(q), sl(k), sl(v), sl(g), sl(beta), vw.h0[n:n + 1],
                                    chunk=16, scale=vw.w.scale, mode=mode)
        assert rel_err(o[a:b], o_c[0]) < 1e-12
        assert rel_err(hT[n], h_c[0]) < 1e-12


def test_empty_sequence_keeps_state():
    vw = make_varlen([3, 0, 4], 1, 8, 8, dtype="f32", seed=1, h0_std=0.5)
    q, k, v, g, beta = _packed(vw)
    _, hT = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, vw.h0, scale=vw.w.scale)
    assert np.array_equal(hT[1], vw.h0[1])
    _, hT0 = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, None, scale=vw.w.scale)
    assert not hT0[1].any()


@pytest.mark.parametrize("mutant", [1, 2])
def test_planted_mistakes_fail_a_pin(mutant):
    """Each planted mistake in the wrapper breaks the dense-batch pin."""
    N, L = 3, 7
    vw = make_varlen([L] * N, 2, 8, 6, dtype="f32", seed=4, h0_std=0.3)
    q, k, v, g, beta = _packed(vw)
    o, hT = oracle.recurrent_varlen(q, k, v, g, beta, vw.cu, vw.h0, scale=vw.w.scale,
                                    mutant=mutant)
    rs = lambda x: x.reshape((N, L) + x.shape[1:])
    o_d, h_d = oracle.recurrent(rs(q), rs(k), rs(v), rs(g), rs(beta), vw.h0, scale=vw.w.scale)
    assert not (np.array_equal(o.reshape(o_d.shape), o_d) and np.array_equal(hT, h_d))

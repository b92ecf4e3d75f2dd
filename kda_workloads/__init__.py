"""Seeded synthetic inputs for the KDA forward pass.

This module is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark.  It only draws random numbers and shapes them into the
workloads described below; it holds none of the arithmetic of the delta rule
itself (no decay, no prediction, no write, no read).

Layout of every token tensor is ``[B, T, H, D]`` (contiguous); the state is
kept transposed per (batch, head) as ``[B, H, Dk, Dv]`` (row = key channel,
column = value channel), the orientation used by the reference
implementation that "You could have come up with Kimi Delta Attention"
(GeekNews summary, section "Kimi Delta Attention: per-channel decay") points
to.  Gates are passed in log space, ``g = log(alpha) <= 0``, as that summary
notes implementations usually store them.

Random draws follow one ``numpy.random.SeedSequence(seed).spawn`` child per
tensor, in the fixed order q, k, v, beta, g, h0, each drawn as float32 from
PCG64.  Where a workload is bf16, q/k/v are rounded to bf16 by
round-to-nearest-even and both sides (oracle and kernels) consume exactly the
rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CHANNEL, SCALAR, NONE = "channel", "scalar", "none"
GATE_MODES = (CHANNEL, SCALAR, NONE)


# --------------------------------------------------------------------------
# bf16 helpers (pure bit manipulation, no model arithmetic)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Expand bf16 bits (uint16) to float32 values exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


# --------------------------------------------------------------------------
# distributions used by the workloads
# --------------------------------------------------------------------------
def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2_normalise_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


@dataclasses.dataclass
class Workload:
    """One seeded input set.

    q, k, v: float32 arrays [B,T,H,D] holding exactly the values the kernels
    see (already bf16-rounded when ``dtype == 'bf16'``).
    g: float32 log-gates, [B,T,H,Dk] (channel), [B,T,H] (scalar) or None.
    beta: float32 [B,T,H].  h0: float32 [B,H,Dk,Dv] or None (zero state).
    """
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    mode: str
    dtype: str            # "f32" or "bf16": storage type of q, k, v, o
    chunk: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: Optional[np.ndarray]
    beta: np.ndarray
    h0: Optional[np.ndarray]
    scale: float

    def qkv_bits(self):
        """bf16 bit patterns of q, k, v (only meaningful for dtype bf16)."""
        return bf16_bits(self.q), bf16_bits(self.k), bf16_bits(self.v)


def _children(seed: int, n: int = 6):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape, std=1.0, mean=0.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make_inputs(B, T, H, Dk, Dv, *, mode=CHANNEL, dtype="bf16", chunk=64,
                seed=0, gate_law="softplus", gate_shift=0.0, beta_law="sigmoid",
                h0_std=0.0, normalise_k=True, scale=None, name="custom",
                scalar_gate_per_head=True, preact=False):
    """Draw one workload.

    gate_law:
      "softplus"   log a = -softplus(z + gate_shift), z ~ N(0,1)
      "mixed"      log a = -softplus(z + mu_c), mu_c = +0.847 on even key
                   channels (a ~ 0.3 at z = 0) and -6.907 on odd ones
                   (a ~ 0.999 at z = 0)
      "expnormal"  log a = -exp(z), z ~ N(-6, 1)   (gates close to 1)
      "zero"       log a = 0
    beta_law: "sigmoid" (sigmoid(N(0,1))) or "uniform" (U[0.1, 1]).
    In scalar mode one gate value is drawn per (b, t, h).
    preact: draw pre-activations for the fused prologue instead: q, k ~ N(0,1)
    unnormalised, beta ~ N(0,1), g ~ N(gate_shift, 1) (gate_law ignored).
    """
    if mode not in GATE_MODES:
        raise ValueError(mode)
    rq, rk, rv, rb, rg, rh = _children(seed)
    q = _normal(rq, (B, T, H, Dk))
    k = _normal(rk, (B, T, H, Dk))
    if normalise_k and not preact:
        k = _l2_normalise_last(k)
    v = _normal(rv, (B, T, H, Dv))
    if preact:
        beta = _normal(rb, (B, T, H))
    elif beta_law == "sigmoid":
        beta = _sigmoid(_normal(rb, (B, T, H)))
    elif beta_law == "uniform":
        beta = rb.uniform(0.1, 1.0, size=(B, T, H)).astype(np.float32)
    else:
        raise ValueError(beta_law)

    if mode == NONE:
        g = None
    elif preact:
        gshape = (B, T, H, Dk) if mode == CHANNEL else (B, T, H)
        g = _normal(rg, gshape, mean=float(gate_shift))
    else:
        gshape = (B, T, H, Dk) if mode == CHANNEL else (B, T, H)
        if gate_law == "softplus":
            g = -_softplus(_normal(rg, gshape) + np.float32(gate_shift))
        elif gate_law == "mixed":
            z = _normal(rg, gshape)
            if mode == CHANNEL:
                mu = np.where(np.arange(Dk) % 2 == 0, 0.847, -6.907).astype(np.float32)
                z = z + mu
            g = -_softplus(z)
        elif gate_law == "expnormal":
            g = -np.exp(_normal(rg, gshape, mean=-6.0)).astype(np.float32)
        elif gate_law == "zero":
            g = np.zeros(gshape, np.float32)
        else:
            raise ValueError(gate_law)
        g = np.ascontiguousarray(g, dtype=np.float32)

    h0 = None
    if h0_std > 0.0:
        h0 = _normal(rh, (B, H, Dk, Dv), std=h0_std)

    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    return Workload(name=name, B=B, T=T, H=H, Dk=Dk, Dv=Dv, mode=mode, dtype=dtype,
                    chunk=chunk, q=q, k=k, v=v, g=g, beta=beta, h0=h0, scale=float(scale))


# --------------------------------------------------------------------------
# gradients of a loss with respect to the forward outputs (backward inputs)
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Cotangents:
    """Seeded gradients dL/do [B,T,H,Dv] (bf16-rounded for a bf16 workload,
    like o) and dL/dH_T [B,H,Dk,Dv] float32 or None (zero)."""
    do: np.ndarray
    dhT: Optional[np.ndarray]


def make_cotangents(w: Workload, *, seed: int = 0, do_std: float = 1.0,
                    dhT_std: float = 0.0) -> Cotangents:
    """Draw dL/do ~ N(0, do_std^2) and dL/dH_T ~ N(0, dhT_std^2) (None when
    dhT_std is 0) from their own seed sequence, independent of the inputs."""
    rd, rh = [np.random.Generator(np.random.PCG64(s))
              for s in np.random.SeedSequence([seed, 0xD0]).spawn(2)]
    do = _normal(rd, (w.B, w.T, w.H, w.Dv), std=do_std)
    if w.dtype == "bf16":
        do = bf16_round(do)
    dhT = _normal(rh, (w.B, w.H, w.Dk, w.Dv), std=dhT_std) if dhT_std > 0.0 else None
    return Cotangents(do=np.ascontiguousarray(do), dhT=dhT)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
CONFIGS = {
    # 1: single head, fp32, recurrent and chunk=16 paths
    "tiny_f32": dict(B=1, T=64, H=1, Dk=16, Dv=16, mode=CHANNEL, dtype="f32", chunk=16,
                     gate_law="softplus", gate_shift=0.0, beta_law="sigmoid", h0_std=0.0),
    # 2: chunked prefill B1 H16 T4096 d128 C64, literal gate law -softplus(z+2)
    "prefill_h16_t4096": dict(B=1, T=4096, H=16, Dk=128, Dv=128, mode=CHANNEL, dtype="bf16",
                              chunk=64, gate_law="softplus", gate_shift=2.0,
                              beta_law="sigmoid", h0_std=0.01),
    # 2b: parity-only variant with gates near 0.9 (-softplus(z-2))
    "prefill_h16_t4096_slow": dict(B=1, T=4096, H=16, Dk=128, Dv=128, mode=CHANNEL,
                                   dtype="bf16", chunk=64, gate_law="softplus",
                                   gate_shift=-2.0, beta_law="sigmoid", h0_std=0.01),
    # 3: decode step, batch 256, H32, d128, one token, state N(0, 0.05)
    "decode_b256_h32": dict(B=256, T=1, H=32, Dk=128, Dv=128, mode=CHANNEL, dtype="bf16",
                            chunk=64, gate_law="softplus", gate_shift=2.0,
                            beta_law="sigmoid", h0_std=0.05),
    # 4: training shape with mixed fast / slow channels
    "train_b8_h32_t8192": dict(B=8, T=8192, H=32, Dk=128, Dv=128, mode=CHANNEL, dtype="bf16",
                               chunk=64, gate_law="mixed", beta_law="sigmoid", h0_std=0.0),
    # 5: long prefill stress, three gate modes
    "long_t65536_channel": dict(B=1, T=65536, H=8, Dk=128, Dv=128, mode=CHANNEL, dtype="bf16",
                                chunk=64, gate_law="expnormal", beta_law="uniform", h0_std=0.0),
    "long_t65536_scalar": dict(B=1, T=65536, H=8, Dk=128, Dv=128, mode=SCALAR, dtype="bf16",
                               chunk=64, gate_law="expnormal", beta_law="uniform", h0_std=0.0),
    "long_t65536_none": dict(B=1, T=65536, H=8, Dk=128, Dv=128, mode=NONE, dtype="bf16",
                             chunk=64, gate_law="zero", beta_law="uniform", h0_std=0.0),
}


def make_config(name: str, seed: int = 0, **overrides) -> Workload:
    """Build one of the named workloads (optionally with shape overrides)."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    B, T, H, Dk, Dv = (spec.pop(x) for x in ("B", "T", "H", "Dk", "Dv"))
    return make_inputs(B, T, H, Dk, Dv, seed=seed, name=name, **spec)


def slice_heads(w: Workload, pairs):
    """Return (q, k, v, g, beta, h0) restricted to a list of (b, h) pairs,
    each as a separate batch entry with H = 1 (for sampled oracle runs)."""
    out = []
    for b, h in pairs:
        q = np.ascontiguousarray(w.q[b:b + 1, :, h:h + 1])
        k = np.ascontiguousarray(w.k[b:b + 1, :, h:h + 1])
        v = np.ascontiguousarray(w.v[b:b + 1, :, h:h + 1])
        g = None if w.g is None else np.ascontiguousarray(w.g[b:b + 1, :, h:h + 1])
        beta = np.ascontiguousarray(w.beta[b:b + 1, :, h:h + 1])
        h0 = None if w.h0 is None else np.ascontiguousarray(w.h0[b:b + 1, h:h + 1])
        out.append((q, k, v, g, beta, h0))
    return out


# --------------------------------------------------------------------------
# packed variable-length batches
# --------------------------------------------------------------------------
def make_lengths(N: int, *, max_len: int, seed: int = 0, edge=()) -> np.ndarray:
    """N sequence lengths: the given edge lengths first, the rest drawn
    log-uniformly from [1, max_len] (many short sequences, a few long ones)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x7a11]))
    n_draw = max(N - len(edge), 0)
    drawn = np.exp(rng.uniform(0.0, math.log(max_len + 1), size=n_draw)).astype(np.int64)
    drawn = np.clip(drawn, 1, max_len)
    return np.concatenate([np.asarray(edge, np.int64)[:N], drawn]).astype(np.int64)


@dataclasses.dataclass
class VarlenWorkload:
    """A packed batch: ``w`` holds the tokens of all sequences as one B = 1
    workload of T = sum(lengths) tokens; ``cu`` [N+1] int32 are the sequence
    offsets and ``h0`` [N,H,Dk,Dv] float32 (or None) the initial states."""
    w: Workload
    cu: np.ndarray
    h0: Optional[np.ndarray]

    @property
    def N(self) -> int:
        return len(self.cu) - 1


def make_varlen(lengths, H, Dk, Dv, *, seed=0, h0_std=0.0, **kw) -> VarlenWorkload:
    """Draw a packed batch with the given sequence lengths (same laws as
    :func:`make_inputs`; keyword arguments are passed on to it)."""
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    w = make_inputs(1, T, H, Dk, Dv, seed=seed, h0_std=0.0, name="varlen", **kw)
    h0 = None
    if h0_std > 0.0:
        rh = np.random.default_rng(np.random.SeedSequence([seed, 0x40]))
        h0 = _normal(rh, (len(lengths), H, Dk, Dv), std=h0_std)
    return VarlenWorkload(w=w, cu=cu.astype(np.int32), h0=h0)

"""ctypes wrapper of oracle R (``kda_recurrence.c``) and of its gradient
(``kda_backward.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The C source is compiled with the host C compiler (``gcc -O2 -fopenmp``, no
fast-math) into ``oracle/_build/libkda_oracle.so``.  ``build_oracle_library``
is also what the package build step calls: compiling the oracle is not running
it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_recurrence.c")
_SRC_BWD = os.path.join(_HERE, "kda_backward.c")
_BUILD = os.path.join(_HERE, "_build")
_MODES = {"channel": 0, "scalar": 1, "none": 2}

_libs = {}


def build_oracle_library(out_path: Optional[str] = None, mutant: int = 0,
                         force: bool = True) -> str:
    """Compile ``kda_recurrence.c`` and return the path of the shared library.

    ``mutant`` > 0 builds a deliberately wrong variant (tests only).
    """
    if out_path is None:
        name = "libkda_oracle.so" if mutant == 0 else f"libkda_oracle_m{mutant}.so"
        out_path = os.path.join(_BUILD, name)
    if not force and os.path.exists(out_path) and \
            os.path.getmtime(out_path) >= max(os.path.getmtime(_SRC),
                                              os.path.getmtime(_SRC_BWD)):
        return out_path
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    tmp = out_path + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           f"-DKDA_MUTANT={int(mutant)}", _SRC, _SRC_BWD, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def _load(mutant: int = 0):
    lib = _libs.get(mutant)
    if lib is not None:
        return lib
    # KDA_ORACLE_LIBRARY: an already built oracle library to load instead
    # (the sanitizer test builds one with host ASan/UBSan)
    override = os.environ.get("KDA_ORACLE_LIBRARY")
    if override and mutant == 0:
        path = override
    else:
        path = build_oracle_library(mutant=mutant, force=False)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_recurrent.argtypes = [dp] * 8 + [ctypes.c_long] * 5 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_recurrent.restype = ctypes.c_int
    lib.kda_oracle_recurrent_bwd.argtypes = [dp] * 14 + [ctypes.c_long] * 5 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_recurrent_bwd.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    _libs[mutant] = lib
    return lib


def oracle_threads() -> int:
    """Threads the OpenMP runtime of the oracle would use by default."""
    return int(_load().kda_oracle_max_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, g, beta, h0=None, *, scale: Optional[float] = None,
              mode: str = "channel", threads: int = 0, mutant: int = 0):
    """Run oracle R.

    q, k: [B,T,H,Dk]; v: [B,T,H,Dv]; g: [B,T,H,Dk] (channel), [B,T,H]
    (scalar) or None (none); beta: [B,T,H]; h0: [B,H,Dk,Dv] or None.
    scale defaults to Dk**-0.5.  Returns (o [B,T,H,Dv], hT [B,H,Dk,Dv]) in
    float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    g, h0 = _f64(g), _f64(h0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    assert beta.shape == (B, T, H)
    if mode == "channel":
        assert g is not None and g.shape == (B, T, H, Dk)
    elif mode == "scalar":
        assert g is not None and g.shape == (B, T, H)
    elif mode == "none":
        g = None
    else:
        raise ValueError(mode)
    if h0 is not None:
        assert h0.shape == (B, H, Dk, Dv)
    if scale is None:
        scale = Dk ** -0.5
    o = np.zeros((B, T, H, Dv), np.float64)
    hT = np.zeros((B, H, Dk, Dv), np.float64)
    rc = _load(mutant).kda_oracle_recurrent(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
        B, T, H, Dk, Dv, float(scale), _MODES[mode], int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle R failed with code {rc}")
    return o, hT


def recurrent_bwd(q, k, v, g, beta, h0, do, dhT=None, *, scale: Optional[float] = None,
                  mode: str = "channel", threads: int = 0, mutant: int = 0):
    """Gradients of oracle R (``kda_backward.c``).

    Inputs as for :func:`recurrent`, plus ``do`` = dL/do [B,T,H,Dv] and
    ``dhT`` = dL/dH_T [B,H,Dk,Dv] or None (zero).  Returns a dict of float64
    arrays: dq, dk [B,T,H,Dk]; dv [B,T,H,Dv]; dg (shape of g, None in the
    ungated mode); dbeta [B,T,H]; dh0 [B,H,Dk,Dv] (the gradient of the
    initial state, also when ``h0`` is None, i.e. zero).
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    g, h0, do, dhT = _f64(g), _f64(h0), _f64(do), _f64(dhT)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    assert do.shape == (B, T, H, Dv) and beta.shape == (B, T, H)
    if mode == "channel":
        assert g is not None and g.shape == (B, T, H, Dk)
    elif mode == "scalar":
        assert g is not None and g.shape == (B, T, H)
    elif mode == "none":
        g = None
    else:
        raise ValueError(mode)
    for x in (h0, dhT):
        if x is not None:
            assert x.shape == (B, H, Dk, Dv)
    if scale is None:
        scale = Dk ** -0.5
    out = {
        "dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)),
        "dv": np.zeros((B, T, H, Dv)), "dbeta": np.zeros((B, T, H)),
        "dg": None if g is None else np.zeros(g.shape),
        "dh0": np.zeros((B, H, Dk, Dv)),
    }
    rc = _load(mutant).kda_oracle_recurrent_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dhT),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
        _ptr(out["dbeta"]), _ptr(out["dh0"]),
        B, T, H, Dk, Dv, float(scale), _MODES[mode], int(threads))
    if rc != 0:
        raise RuntimeError(f"oracle R-bwd failed with code {rc}")
    return out

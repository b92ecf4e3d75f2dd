"""MI355X-native Kimi Delta Attention (KDA) forward: Python binding.

A thin ctypes layer over the C ABI of ``libkda.so`` (declared in
``include/kda.h``).  It only marshals arguments: tensors are passed as device
pointers, the stream is torch's current HIP stream, and every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing, importing works but every call raises.

Entry points (same names as the C ABI):
  kda_recurrent_step(q, k, v, g, beta, state, o=None, scale=None, mode=None)
  kda_chunk_fwd(q, k, v, g, beta, initial_state=None, final_state=None,
                o=None, chunk=64, scale=None, mode=None, workspace=None)
  kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, mode, dtype)
  kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, final_state, o,
                        chunk=64, scale=None, mode=None)
  kda_recurrent_varlen(q, k, v, g, beta, state, cu_seqlens, o=None, scale=None, mode=None)
  kda_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None,
                       final_state=None, o=None, chunk=64, scale=None, mode=None,
                       workspace=None)
  kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, mode, dtype)
  kda_chunk_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                chunk=64, scale=None, mode=None, workspace=None, out=None)
  kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, mode, dtype)
  kda_chunk_bwd_varlen(q, k, v, g, beta, d_o, cu_seqlens, initial_state=None,
                       d_final_state=None, chunk=64, scale=None, mode=None, workspace=None)
  kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, mode, dtype)

Every compute call takes ``prologue``, a bitwise OR of NORMALIZE_QK,
BETA_SIGMOID and GATE_LOGSIGMOID (0: inputs used as given).
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY: load another build of the same library (e.g. one whose host
# code carries sanitizers); by default the in-tree libkda.so
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(HERE, "libkda.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kda.h")

GATE_CHANNEL, GATE_SCALAR, GATE_NONE = 0, 1, 2
# fused prologue flags (kda_prologue)
NORMALIZE_QK, BETA_SIGMOID, GATE_LOGSIGMOID = 1, 2, 4
F32, BF16 = 0, 1
_MODE_NAMES = {"channel": GATE_CHANNEL, "scalar": GATE_SCALAR, "none": GATE_NONE}
STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERROR_INVALID_VALUE", 2: "KDA_ERROR_NOT_SUPPORTED",
          3: "KDA_ERROR_MISALIGNED", 4: "KDA_ERROR_WORKSPACE", 5: "KDA_ERROR_HIP",
          6: "KDA_ERROR_SCRATCH"}
# bytes of the fixed device scratch array behind kda_chunk_fwd_noalloc
# (KDA_NOALLOC_SCRATCH_BYTES in kda.h)
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class KDAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib():
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m gated_delta_rule_17_amd.build`")
    # The HIP runtime (torch's, which the library binds to) is brought up
    # before the library registers its code objects: code objects registered
    # while the runtime is still down fail every launch (hipErrorNoDevice)
    # once it comes up.  Without a GPU nothing is initialised.
    try:
        import torch
        if torch.cuda.is_available():
            torch.cuda.init()
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.kda_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, i, f, i, i, i, i, vp]
    L.kda_recurrent_step.restype = i
    L.kda_chunk_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    L.kda_chunk_fwd_workspace_size.restype = sz
    L.kda_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, i, i, i, i, i, i, i, f, i, i, i, i,
                                vp, sz, vp]
    L.kda_chunk_fwd.restype = i
    L.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, i, i, i, i, i, i, i, f, i,
                                        i, i, i, vp]
    L.kda_chunk_fwd_noalloc.restype = i
    L.kda_recurrent_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, vp, i, i, i, i, i, i, f, i, i, i,
                                       i, vp]
    L.kda_recurrent_varlen.restype = i
    L.kda_chunk_fwd_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    L.kda_chunk_fwd_varlen_workspace_size.restype = sz
    L.kda_chunk_fwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp, vp, i, i, i, i, i, i, i, f, i,
                                       i, i, i, vp, sz, vp]
    L.kda_chunk_fwd_varlen.restype = i
    L.kda_chunk_bwd_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i]
    L.kda_chunk_bwd_workspace_size.restype = sz
    L.kda_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp,
                                i, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    L.kda_chunk_bwd.restype = i
    L.kda_chunk_bwd_varlen_workspace_size.argtypes = [i, i, i, i, i, i, i, i, i]
    L.kda_chunk_bwd_varlen_workspace_size.restype = sz
    L.kda_chunk_bwd_varlen.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, vp, vp, vp, fp, fp, fp, vp,
                                       i, i, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    L.kda_chunk_bwd_varlen.restype = i
    L.kda_status_string.argtypes = [i]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_version.restype = i
    _lib = L
    return L


def header_functions():
    """Names of the functions ``include/kda.h`` declares."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_meta(name, t, dtype=None, shape=None):
    """dtype and shape of an argument (no device access)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_dev(name, t, dtype=None, shape=None, device=None):
    if t is None:
        return
    _check_meta(name, t, dtype, shape)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gate_shape(m, lead, H, Dk):
    """The shape the kernels index g with: lead + (H, Dk) per channel,
    lead + (H,) per token and head, no tensor in the ungated mode."""
    if m == GATE_CHANNEL:
        return tuple(lead) + (H, Dk)
    if m == GATE_SCALAR:
        return tuple(lead) + (H,)
    if m == GATE_NONE:
        return None
    raise ValueError(f"unknown gate mode {m}")


def _check_gate(g, m, lead, H, Dk):
    """g must match its mode: the kernels index it as [.., H, Dk] (channel)
    or [.., H] (scalar), so any other shape would be read out of bounds."""
    shape = _gate_shape(m, lead, H, Dk)
    if shape is None:
        if g is not None:
            raise ValueError("g must be None in the ungated mode")
        return
    if g is None:
        raise ValueError("g is required in the channel and scalar gate modes")
    _check_meta("g", g, None, shape)


def _check_workspace(ws, need, device):
    """A caller-supplied workspace: a contiguous uint8 tensor on the device
    of the other arguments, with at least `need` bytes (its numel() is the
    byte count passed on)."""
    torch = _torch()
    _check_meta("workspace", ws, torch.uint8)
    if ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} are needed")
    _check_dev("workspace", ws, torch.uint8, None, device)


def _mode_of(g, mode):
    if mode is None:
        if g is None:
            return GATE_NONE
        return GATE_CHANNEL if g.dim() == 4 else GATE_SCALAR
    if isinstance(mode, str):
        return _MODE_NAMES[mode]
    return int(mode)


def _common(q, k, v, g, beta, mode, packed, extra=()):
    """Metadata checks shared by every compute entry (before any device
    access): q, k [*lead, Hqk, Dk], v [*lead, H, Dv] of one dtype, g matching
    the gate mode, beta [*lead, H] float32, where lead is (B, T) for a dense
    batch and (T,) for a packed one.  `extra` are further (name, tensor)
    pairs of the dtype of q with v's shape.  Returns (lead, Hqk, Dk, H, Dv,
    mode code)."""
    torch = _torch()
    nd = 3 if packed else 4
    if q.dim() != nd:
        raise ValueError(f"q must have {nd} dimensions, got shape {tuple(q.shape)}")
    lead, Hqk, Dk = tuple(q.shape[:-2]), q.shape[-2], q.shape[-1]
    _dtype_code(q)
    _check_meta("k", k, q.dtype, q.shape)
    _check_meta("v", v, q.dtype)
    if v.dim() != nd or tuple(v.shape[:-2]) != lead:
        raise ValueError(f"v has shape {tuple(v.shape)}, inconsistent with q {tuple(q.shape)}")
    H, Dv = v.shape[-2], v.shape[-1]
    for name, t in extra:
        _check_meta(name, t, q.dtype, v.shape)
    m = _mode_of_packed(g, mode) if packed else _mode_of(g, mode)
    _check_meta("g", g, torch.float32)
    _check_gate(g, m, lead, H, Dk)
    _check_meta("beta", beta, torch.float32, lead + (H,))
    return lead, Hqk, Dk, H, Dv, m


def _on_device(dev, *named):
    """Device, placement and contiguity of every (name, tensor) pair."""
    for name, t in named:
        _check_dev(name, t, None, None, dev)


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def kda_recurrent_step(q, k, v, g, beta, state, o=None, scale: Optional[float] = None,
                       mode=None, out_dtype=None, prologue: int = 0):
    """Recurrent form over T >= 1 tokens; updates ``state`` in place.

    q, k [B,T,Hqk,Dk] and v [B,T,H,Dv] (float32 or bfloat16; H a multiple of
    Hqk: grouped value heads), g float32 log-gates ([B,T,H,Dk] channel /
    [B,T,H] scalar / None), beta float32 [B,T,H], state float32 [B,H,Dk,Dv].
    Returns o [B,T,H,Dv] (``out_dtype``, default the dtype of q; ignored when
    ``o`` is given).
    """
    torch = _torch()
    (B, T), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=False)
    _check_meta("state", state, torch.float32, (B, H, Dk, Dv))
    if state is None:
        raise ValueError("state is required")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype or q.dtype, device=q.device)
    _check_meta("o", o, None, (B, T, H, Dv))
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("state", state), ("o", o))
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                  _ptr(o), B, T, H, Hqk, Dk, Dv, float(scale), m, _dtype_code(q),
                                  _dtype_code(o), int(prologue), _stream())
    if st != 0:
        raise KDAError(st, "kda_recurrent_step")
    return o


def kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, mode, dtype) -> int:
    if isinstance(mode, str):
        mode = _MODE_NAMES[mode]
    return int(lib().kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, int(mode), int(dtype)))


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                  chunk: int = 64, scale: Optional[float] = None, mode=None, workspace=None,
                  output_final_state: bool = True, out_dtype=None, prologue: int = 0):
    """Chunkwise form.  Returns (o, final_state).

    ``final_state`` may be passed (it may be ``initial_state`` itself); if it
    is None and ``output_final_state`` is true a new float32 tensor is made.
    ``workspace`` (a uint8 device tensor) is allocated when not given.
    Shapes as for :func:`kda_recurrent_step`.
    """
    torch = _torch()
    (B, T), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=False)
    _check_meta("initial_state", initial_state, torch.float32, (B, H, Dk, Dv))
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_meta("final_state", final_state, torch.float32, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=out_dtype or q.dtype, device=q.device)
    _check_meta("o", o, None, (B, T, H, Dv))
    dt = _dtype_code(q)
    need = kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, m, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("initial_state", initial_state), ("final_state", final_state), ("o", o))
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                             _ptr(final_state), _ptr(o), B, T, H, Hqk, Dk, Dv, int(chunk), float(scale),
                             m, dt, _dtype_code(o), int(prologue), _ptr(workspace), workspace.numel(),
                             _stream())
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd")
    return o, final_state


def kda_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, final_state, o, chunk: int = 64,
                          scale: Optional[float] = None, mode=None, prologue: int = 0):
    """:func:`kda_chunk_fwd` without a workspace: the library's fixed device
    scratch array (NOALLOC_SCRATCH_BYTES) holds the chunk records, and the
    C entry point allocates nothing.  The caller passes every output
    (``o``; ``final_state`` or None), so this wrapper allocates nothing
    either.  Calls that overlap in time on one device race on the scratch.
    Returns (o, final_state)."""
    torch = _torch()
    (B, T), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=False)
    _check_meta("initial_state", initial_state, torch.float32, (B, H, Dk, Dv))
    _check_meta("final_state", final_state, torch.float32, (B, H, Dk, Dv))
    if o is None:
        raise ValueError("o is required (the allocation-free entry allocates no output)")
    _check_meta("o", o, None, (B, T, H, Dv))
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("initial_state", initial_state), ("final_state", final_state), ("o", o))
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(initial_state), _ptr(final_state), _ptr(o), B, T, H, Hqk,
                                     Dk, Dv, int(chunk), float(scale), m, _dtype_code(q),
                                     _dtype_code(o), int(prologue), _stream())
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_noalloc")
    return o, final_state


# ---------------------------------------------------------------------------
# packed variable-length batches
def _mode_of_packed(g, mode):
    if mode is None:
        if g is None:
            return GATE_NONE
        return GATE_CHANNEL if g.dim() == 3 else GATE_SCALAR
    if isinstance(mode, str):
        return _MODE_NAMES[mode]
    return int(mode)


def _check_cu(cu_seqlens):
    torch = _torch()
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required")
    _check_meta("cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of N + 1 offsets")
    return cu_seqlens.numel() - 1


def kda_recurrent_varlen(q, k, v, g, beta, state, cu_seqlens, o=None,
                         scale: Optional[float] = None, mode=None, out_dtype=None,
                         prologue: int = 0):
    """Recurrent form over a packed batch; updates ``state`` in place.

    q, k [T,Hqk,Dk], v [T,H,Dv] (float32 or bfloat16), g [T,H,Dk] / [T,H] /
    None, beta [T,H] float32, state [N,H,Dk,Dv] float32, cu_seqlens int32
    [N+1] on the device.  Returns o [T,H,Dv].
    """
    torch = _torch()
    (T,), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=True)
    N = _check_cu(cu_seqlens)
    _check_meta("state", state, torch.float32, (N, H, Dk, Dv))
    if state is None:
        raise ValueError("state is required")
    if o is None:
        o = torch.empty((T, H, Dv), dtype=out_dtype or q.dtype, device=q.device)
    _check_meta("o", o, None, (T, H, Dv))
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("state", state), ("o", o), ("cu_seqlens", cu_seqlens))
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_recurrent_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                    _ptr(o), _ptr(cu_seqlens), N, T, H, Hqk, Dk, Dv, float(scale), m,
                                    _dtype_code(q), _dtype_code(o), int(prologue), _stream())
    if st != 0:
        raise KDAError(st, "kda_recurrent_varlen")
    return o


def kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, mode, dtype) -> int:
    if isinstance(mode, str):
        mode = _MODE_NAMES[mode]
    return int(lib().kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, int(mode),
                                                         int(dtype)))


def kda_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None, final_state=None,
                         o=None, chunk: int = 64, scale: Optional[float] = None, mode=None,
                         workspace=None, output_final_state: bool = True, out_dtype=None,
                         prologue: int = 0):
    """Chunkwise form over a packed batch.  Returns (o, final_state).

    Shapes as for :func:`kda_recurrent_varlen`; initial_state / final_state
    are [N,H,Dk,Dv] float32 (final_state may be initial_state itself).
    """
    torch = _torch()
    (T,), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=True)
    N = _check_cu(cu_seqlens)
    _check_meta("initial_state", initial_state, torch.float32, (N, H, Dk, Dv))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _check_meta("final_state", final_state, torch.float32, (N, H, Dk, Dv))
    if o is None:
        o = torch.empty((T, H, Dv), dtype=out_dtype or q.dtype, device=q.device)
    _check_meta("o", o, None, (T, H, Dv))
    dt = _dtype_code(q)
    need = kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, m, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta),
               ("initial_state", initial_state), ("final_state", final_state), ("o", o),
               ("cu_seqlens", cu_seqlens))
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(initial_state), _ptr(final_state), _ptr(o),
                                    _ptr(cu_seqlens), N, T, H, Hqk, Dk, Dv, int(chunk), float(scale),
                                    m, dt, _dtype_code(o), int(prologue), _ptr(workspace),
                                    workspace.numel(), _stream())
    if st != 0:
        raise KDAError(st, "kda_chunk_fwd_varlen")
    return o, final_state


# ---------------------------------------------------------------------------
# gradients of the chunkwise form
_GRAD_KEYS = ("dq", "dk", "dv", "dg", "dbeta", "d_initial_state")


def _grad_outputs(out, q, k, v, g, beta, m, grad_dtype, want_d_initial_state, state_shape):
    """The gradient outputs: those given in `out` are checked (their dtype
    sets the storage type of dq, dk, dv), the others allocated.  dg takes the
    shape of g, which the gate check has already tied to the gate mode."""
    torch = _torch()
    out = dict(out or {})
    dev = q.device
    if out.get("dq") is not None:
        grad_dtype = out["dq"].dtype
    gdt = grad_dtype or q.dtype
    if gdt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"gradients must be float32 or bfloat16, got {gdt}")
    for name, ref in (("dq", q), ("dk", k), ("dv", v)):
        if out.get(name) is None:
            out[name] = torch.empty(ref.shape, dtype=gdt, device=dev)
    if m == GATE_NONE:
        out["dg"] = None
    elif out.get("dg") is None:
        out["dg"] = torch.empty(g.shape, dtype=torch.float32, device=dev)
    if out.get("dbeta") is None:
        out["dbeta"] = torch.empty(beta.shape, dtype=torch.float32, device=dev)
    if not want_d_initial_state:
        out["d_initial_state"] = None
    elif out.get("d_initial_state") is None:
        out["d_initial_state"] = torch.empty(state_shape, dtype=torch.float32, device=dev)
    _check_meta("dq", out["dq"], gdt, q.shape)
    _check_meta("dk", out["dk"], gdt, k.shape)
    _check_meta("dv", out["dv"], gdt, v.shape)
    _check_meta("dg", out["dg"], torch.float32, None if g is None else g.shape)
    _check_meta("dbeta", out["dbeta"], torch.float32, beta.shape)
    _check_meta("d_initial_state", out["d_initial_state"], torch.float32, state_shape)
    return out


def kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, mode, dtype) -> int:
    if isinstance(mode, str):
        mode = _MODE_NAMES[mode]
    return int(lib().kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, int(mode),
                                                  int(dtype)))


def kda_chunk_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                  chunk: int = 64, scale: Optional[float] = None, mode=None, workspace=None,
                  out=None, want_d_initial_state: bool = True, grad_dtype=None):
    """Gradients of :func:`kda_chunk_fwd` for the same inputs.

    ``d_o`` [B,T,H,Dv] has the dtype of q; ``d_final_state`` float32
    [B,H,Dk,Dv] or None (zero).  Returns a dict with dq, dk (shape of q),
    dv (shape of v), all of ``grad_dtype`` (default the dtype of q), dg
    (shape of g, None in the ungated mode), dbeta [B,T,H] and
    d_initial_state [B,H,Dk,Dv] (None when ``want_d_initial_state`` is
    false).  ``out`` may hold preallocated tensors under those keys (their
    dtype then sets the gradient storage type).
    """
    torch = _torch()
    (B, T), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=False,
                                         extra=(("d_o", d_o),))
    _check_meta("initial_state", initial_state, torch.float32, (B, H, Dk, Dv))
    _check_meta("d_final_state", d_final_state, torch.float32, (B, H, Dk, Dv))
    out = _grad_outputs(out, q, k, v, g, beta, m, grad_dtype, want_d_initial_state,
                        (B, H, Dk, Dv))
    dt = _dtype_code(q)
    need = kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, m, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("d_o", d_o),
               ("initial_state", initial_state), ("d_final_state", d_final_state),
               *[(n, out[n]) for n in _GRAD_KEYS])
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                             _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
                             _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                             _ptr(out["d_initial_state"]), B, T, H, Hqk, Dk, Dv, int(chunk),
                             float(scale), m, dt, _dtype_code(out["dq"]), _ptr(workspace),
                             workspace.numel(), _stream())
    if st != 0:
        raise KDAError(st, "kda_chunk_bwd")
    return out


def kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, mode, dtype) -> int:
    if isinstance(mode, str):
        mode = _MODE_NAMES[mode]
    return int(lib().kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, int(mode),
                                                         int(dtype)))


def kda_chunk_bwd_varlen(q, k, v, g, beta, d_o, cu_seqlens, initial_state=None,
                         d_final_state=None, chunk: int = 64, scale: Optional[float] = None,
                         mode=None, workspace=None, out=None, want_d_initial_state: bool = True,
                         grad_dtype=None):
    """Gradients of :func:`kda_chunk_fwd_varlen` for the same packed inputs.

    Token tensors are packed [T, heads, D] as for the packed forward;
    ``cu_seqlens`` is an int32 device tensor [N + 1]; ``initial_state`` and
    ``d_final_state`` are float32 [N, H, Dk, Dv] or None.  Returns the dict of
    :func:`kda_chunk_bwd` (d_initial_state [N, H, Dk, Dv]).
    """
    torch = _torch()
    (T,), Hqk, Dk, H, Dv, m = _common(q, k, v, g, beta, mode, packed=True,
                                      extra=(("d_o", d_o),))
    N = _check_cu(cu_seqlens)
    _check_meta("initial_state", initial_state, torch.float32, (N, H, Dk, Dv))
    _check_meta("d_final_state", d_final_state, torch.float32, (N, H, Dk, Dv))
    out = _grad_outputs(out, q, k, v, g, beta, m, grad_dtype, want_d_initial_state,
                        (N, H, Dk, Dv))
    dt = _dtype_code(q)
    need = kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, m, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    _on_device(q.device, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("d_o", d_o),
               ("initial_state", initial_state), ("d_final_state", d_final_state),
               ("cu_seqlens", cu_seqlens), *[(n, out[n]) for n in _GRAD_KEYS])
    if scale is None:
        scale = Dk ** -0.5
    st = lib().kda_chunk_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(d_o),
        _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
        _ptr(out["dbeta"]), _ptr(out["d_initial_state"]), _ptr(cu_seqlens), N, T, H, Hqk, Dk, Dv,
        int(chunk), float(scale), m, dt, _dtype_code(out["dq"]), _ptr(workspace),
        workspace.numel(), _stream())
    if st != 0:
        raise KDAError(st, "kda_chunk_bwd_varlen")
    return out

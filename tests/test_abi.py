"""The C-ABI library loads, exports what include/kda.h declares, and rejects
bad arguments on the host before any HIP call (CPU only: every call here
fails validation, so nothing is ever enqueued)."""
import ctypes

import pytest

import gated_delta_rule_17_amd as K

A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004        # misaligned


@pytest.fixture(scope="module")
def L():
    return K.lib()


def test_exports_every_declared_symbol(L):
    names = K.header_functions()
    assert set(names) >= {"kda_recurrent_step", "kda_chunk_fwd", "kda_chunk_fwd_workspace_size",
                          "kda_recurrent_varlen", "kda_chunk_fwd_varlen",
                          "kda_chunk_fwd_varlen_workspace_size", "kda_status_string",
                          "kda_version", "kda_chunk_bwd", "kda_chunk_bwd_workspace_size",
                          "kda_chunk_bwd_varlen", "kda_chunk_bwd_varlen_workspace_size"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in K.STATUS.items():
        assert L.kda_status_string(code).decode() == name
    assert L.kda_status_string(99).decode() == "KDA_ERROR_UNKNOWN"
    assert L.kda_version() >= 10000


def _rec(L, q=A, k=A, v=A, g=A, beta=A, state=A, o=A, B=1, T=1, H=1, Hqk=None, Dk=128, Dv=128,
         scale=1.0, mode=0, dtype=1, o_dtype=0, pro=0):
    Hqk = H if Hqk is None else Hqk
    return L.kda_recurrent_step(q, k, v, g, beta, state, o, B, T, H, Hqk, Dk, Dv, scale, mode,
                                dtype, o_dtype, pro, None)


def _chunk(L, q=A, k=A, v=A, g=A, beta=A, h0=None, hT=None, o=A, B=1, T=64, H=1, Hqk=None,
           Dk=128, Dv=128, chunk=64, scale=1.0, mode=0, dtype=1, o_dtype=0, ws=A, wsb=None,
           pro=0):
    Hqk = H if Hqk is None else Hqk
    if wsb is None:
        wsb = L.kda_chunk_fwd_workspace_size(B, T, H, Dk, Dv, chunk, mode, dtype)
    return L.kda_chunk_fwd(q, k, v, g, beta, h0, hT, o, B, T, H, Hqk, Dk, Dv, chunk, scale, mode,
                           dtype, o_dtype, pro, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(beta=None), 1),
    (dict(o=None), 1), (dict(state=None), 1), (dict(g=None, mode=0), 1),
    (dict(g=None, mode=1), 1), (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1),
    (dict(mode=3), 1), (dict(dtype=2), 1), (dict(o_dtype=-1), 1), (dict(Dk=48), 2), (dict(Dv=512), 2), (dict(Dk=256), 2),
    (dict(H=4, Hqk=3), 1), (dict(H=2, Hqk=4), 1), (dict(Hqk=0), 1), (dict(pro=8), 1),
    (dict(pro=-1), 1),
    (dict(Dk=8), 2), (dict(q=MIS), 3), (dict(state=MIS), 3), (dict(g=MIS), 3),
    (dict(o=MIS), 3),
])
def test_recurrent_validation(L, kw, code):
    assert _rec(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(g=None, mode=0), 1), (dict(B=0), 1), (dict(mode=7), 1),
    (dict(o_dtype=5), 1),
    (dict(chunk=48), 2), (dict(chunk=128), 2), (dict(Dk=256, Dv=256), 2), (dict(Dv=512), 2),
    (dict(Dv=256, dtype=0), 2),   # float32, chunk 64, d_k 128, d_v 256: staging exceeds the LDS
    (dict(H=6, Hqk=4), 1), (dict(pro=16), 1),
    (dict(q=MIS), 3), (dict(h0=MIS), 3), (dict(hT=MIS), 3), (dict(ws=None), 4),
    (dict(wsb=16), 4), (dict(ws=A + 16), 3),
])
def test_chunk_validation(L, kw, code):
    assert _chunk(L, **kw) == code


def test_value_dim_256_passes_validation(L):
    # d_v = 256 with bf16 operands, and with float32 operands at chunk 32:
    # only the workspace check remains to fail
    assert _chunk(L, Dv=256, ws=None) == 4
    assert _chunk(L, Dv=256, dtype=0, chunk=32, ws=None) == 4
    assert _chunk(L, Dk=64, Dv=256, dtype=0, ws=None) == 4
    assert _bwd(L, Dv=256, ws=None) == 4
    assert _bwd(L, Dv=256, dtype=0, ws=None) == 4


def test_none_mode_accepts_null_gate(L):
    # only the workspace check remains to fail, proving g=NULL passed validation
    assert _chunk(L, g=None, mode=2, ws=None) == 4


def test_zero_length_recurrent_is_a_no_op(L):
    # T = 0: nothing to do, nothing enqueued, even with NULL tensors
    assert _rec(L, q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0


def test_workspace_size(L):
    f = L.kda_chunk_fwd_workspace_size
    assert f(1, 0, 1, 128, 128, 64, 0, 1) == 0
    assert f(1, 64, 1, 128, 128, 48, 0, 1) == 0
    a = f(1, 64, 1, 128, 128, 64, 0, 1)
    b = f(1, 65, 1, 128, 128, 64, 0, 1)         # a ragged tail costs a whole chunk record
    assert 0 < a < b == 2 * a
    assert f(2, 64, 3, 128, 128, 64, 0, 1) == 6 * a
    assert f(1, 64, 1, 128, 128, 64, 0, 0) >= a  # float32 records are no smaller
    # d_k != d_v is supported; the U record grows with d_v
    assert 0 < f(1, 64, 1, 64, 128, 64, 0, 1) and f(1, 64, 1, 128, 64, 64, 0, 1) > 0
    assert f(1, 64, 1, 64, 128, 64, 0, 1) > f(1, 64, 1, 64, 64, 64, 0, 1)
    # d_v = 256; not built for float32 operands at chunk 64 with d_k 128
    assert f(1, 64, 1, 128, 256, 64, 0, 1) > f(1, 64, 1, 128, 128, 64, 0, 1)
    assert f(1, 64, 1, 128, 256, 64, 0, 0) == 0
    assert f(1, 64, 1, 128, 256, 32, 0, 0) > 0
    assert f(1, 64, 1, 128, 512, 64, 0, 1) == 0


def test_workspace_size_of_the_segmented_state_pass(L):
    """A sequence of 256 or more chunks over few heads runs its state pass in
    segments; the workspace then holds three sets of per-segment states
    (entering states, final states from zero, transition matrices) after the
    chunk records: 8 segments at B1 H2 d128, none below 256 chunks."""
    f = L.kda_chunk_fwd_workspace_size
    a = f(1, 64, 1, 128, 128, 64, 0, 1)          # one chunk record
    assert f(1, 255 * 64, 2, 128, 128, 64, 0, 1) == 2 * 255 * a
    rec = 2 * 256 * a
    seg = 3 * 8 * 2 * 128 * 128 * 4
    assert f(1, 256 * 64, 2, 128, 128, 64, 0, 1) == (rec + 255) // 256 * 256 + seg
    # d_k != d_v: never segmented
    assert f(1, 256 * 64, 2, 64, 128, 64, 0, 1) == 2 * 256 * f(1, 64, 1, 64, 128, 64, 0, 1)


# ---- packed variable-length batches (host validation only)
CU = 0x20000          # a 4-byte aligned fake device address of the offsets


def _rec_v(L, q=A, k=A, v=A, g=A, beta=A, state=A, o=A, cu=CU, N=2, T=10, H=1, Hqk=None,
           Dk=128, Dv=128, scale=1.0, mode=0, dtype=1, o_dtype=0, pro=0):
    Hqk = H if Hqk is None else Hqk
    return L.kda_recurrent_varlen(q, k, v, g, beta, state, o, cu, N, T, H, Hqk, Dk, Dv, scale,
                                  mode, dtype, o_dtype, pro, None)


def _chunk_v(L, q=A, k=A, v=A, g=A, beta=A, h0=None, hT=None, o=A, cu=CU, N=2, T=64, H=1,
             Hqk=None, Dk=128, Dv=128, chunk=64, scale=1.0, mode=0, dtype=1, o_dtype=0, ws=A,
             wsb=None, pro=0):
    Hqk = H if Hqk is None else Hqk
    if wsb is None:
        wsb = L.kda_chunk_fwd_varlen_workspace_size(N, T, H, Dk, Dv, chunk, mode, dtype)
    return L.kda_chunk_fwd_varlen(q, k, v, g, beta, h0, hT, o, cu, N, T, H, Hqk, Dk, Dv, chunk,
                                  scale, mode, dtype, o_dtype, pro, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(state=None), 1), (dict(cu=None), 1), (dict(N=-1), 1),
    (dict(H=4, Hqk=8), 1), (dict(pro=9), 1),
    (dict(T=-1), 1), (dict(H=0), 1), (dict(g=None, mode=1), 1), (dict(Dk=48), 2),
    (dict(cu=CU + 2), 3), (dict(state=MIS), 3), (dict(o=MIS), 3),
])
def test_recurrent_varlen_validation(L, kw, code):
    assert _rec_v(L, **kw) == code


def test_recurrent_varlen_nothing_to_do(L):
    # no sequences, or no tokens: states unchanged, nothing enqueued
    assert _rec_v(L, N=0, cu=None, state=None) == 0
    assert _rec_v(L, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(N=-1), 1), (dict(mode=9), 1),
    (dict(H=3, Hqk=2), 1), (dict(pro=32), 1), (dict(chunk=8), 2), (dict(Dv=512), 2), (dict(cu=CU + 1), 3), (dict(h0=MIS), 3),
    (dict(hT=MIS), 3), (dict(ws=None), 4), (dict(wsb=64), 4), (dict(ws=A + 16), 3),
])
def test_chunk_varlen_validation(L, kw, code):
    assert _chunk_v(L, **kw) == code


def test_chunk_varlen_workspace_size(L):
    f = L.kda_chunk_fwd_varlen_workspace_size
    assert f(0, 64, 1, 128, 128, 64, 0, 1) == 0
    assert f(1, 64, 1, 128, 128, 48, 0, 1) == 0
    dense = L.kda_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 64, 0, 1)
    # room for ceil(T / chunk) + N chunk records plus the tables
    one = f(1, 64, 1, 128, 128, 64, 0, 1)
    assert one >= 2 * dense
    assert f(3, 64, 1, 128, 128, 64, 0, 1) >= 4 * dense
    # T = 0 still needs the tables (the final states are copied)
    assert f(2, 0, 1, 128, 128, 64, 0, 1) > 0


# ---- gradients of the chunk path (host validation only)
def _bwd(L, q=A, k=A, v=A, g=A, beta=A, h0=None, do=A, dhT=None, dq=A, dk=A, dv=A, dg=A,
         dbeta=A, dh0=None, B=1, T=64, H=1, Hqk=None, Dk=128, Dv=128, chunk=64, scale=1.0,
         mode=0, dtype=1, gdtype=0, ws=A, wsb=None):
    Hqk = H if Hqk is None else Hqk
    if wsb is None:
        wsb = L.kda_chunk_bwd_workspace_size(B, T, H, Hqk, Dk, Dv, chunk, mode, dtype)
    return L.kda_chunk_bwd(q, k, v, g, beta, h0, do, dhT, dq, dk, dv, dg, dbeta, dh0, B, T, H,
                           Hqk, Dk, Dv, chunk, scale, mode, dtype, gdtype, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(beta=None), 1),
    (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1), (dict(dv=None), 1),
    (dict(dbeta=None), 1), (dict(dg=None), 1), (dict(dg=None, mode=1), 1),
    (dict(g=None, mode=0), 1), (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1),
    (dict(mode=3), 1), (dict(dtype=2), 1), (dict(gdtype=2), 1), (dict(H=6, Hqk=4), 1),
    (dict(Hqk=0), 1),
    (dict(chunk=48), 2), (dict(chunk=128), 2), (dict(Dk=256), 2), (dict(Dv=8), 2),
    (dict(q=MIS), 3), (dict(do=MIS), 3), (dict(dq=MIS), 3), (dict(dk=MIS), 3), (dict(dv=MIS), 3),
    (dict(dg=MIS), 3), (dict(dbeta=MIS), 3), (dict(h0=MIS), 3), (dict(dhT=MIS), 3),
    (dict(dh0=MIS), 3), (dict(ws=None), 4), (dict(wsb=64), 4), (dict(ws=A + 16), 3),
])
def test_chunk_bwd_validation(L, kw, code):
    assert _bwd(L, **kw) == code


def test_chunk_bwd_none_mode_accepts_null_gates(L):
    # only the workspace check remains to fail: g = dg = NULL passed validation
    assert _bwd(L, g=None, dg=None, mode=2, ws=None) == 4


def test_chunk_bwd_zero_length_without_state_gradient_is_a_no_op(L):
    assert _bwd(L, T=0, q=None, k=None, v=None, g=None, beta=None, do=None, dq=None, dk=None,
                dv=None, dg=None, dbeta=None, ws=None) == 0


def test_chunk_bwd_workspace_size(L):
    f = L.kda_chunk_bwd_workspace_size
    assert f(1, 0, 1, 1, 128, 128, 64, 0, 1) == 0
    assert f(1, 64, 1, 1, 128, 128, 48, 0, 1) == 0
    assert f(1, 64, 4, 3, 128, 128, 64, 0, 1) == 0
    one = f(1, 64, 1, 1, 128, 128, 64, 0, 1)
    # per chunk: 2 Dk Dv + 4 C Dk + 3 C Dv + 3 C^2 floats (each record 256-byte aligned)
    assert one >= 4 * (2 * 128 * 128 + 7 * 64 * 128 + 3 * 64 * 64)
    assert f(1, 65, 1, 1, 128, 128, 64, 0, 1) >= 2 * one - 16 * 256
    # grouped heads add float partials of dq and dk per value head
    assert f(1, 64, 4, 2, 128, 128, 64, 0, 1) >= 4 * one + 2 * 4 * 64 * 4 * 128 - 16 * 256
    # large batches run in groups of whole batch entries whose records fit in
    # 4 GiB: the workspace is one group's
    assert f(2, 4096, 16, 16, 128, 128, 64, 0, 1) == 2 * f(1, 4096, 16, 16, 128, 128, 64, 0, 1)
    train = f(8, 8192, 32, 32, 128, 128, 64, 0, 1)
    assert train == 2 * f(1, 8192, 32, 32, 128, 128, 64, 0, 1) <= 4 * 2 ** 30 + 2 ** 20


def _bwd_v(L, q=A, k=A, v=A, g=A, beta=A, h0=None, do=A, dhT=None, dq=A, dk=A, dv=A, dg=A,
           dbeta=A, dh0=None, cu=CU, N=2, T=64, H=1, Hqk=None, Dk=128, Dv=128, chunk=64,
           scale=1.0, mode=0, dtype=1, gdtype=0, ws=A, wsb=None):
    Hqk = H if Hqk is None else Hqk
    if wsb is None:
        wsb = L.kda_chunk_bwd_varlen_workspace_size(N, T, H, Hqk, Dk, Dv, chunk, mode, dtype)
    return L.kda_chunk_bwd_varlen(q, k, v, g, beta, h0, do, dhT, dq, dk, dv, dg, dbeta, dh0, cu,
                                  N, T, H, Hqk, Dk, Dv, chunk, scale, mode, dtype, gdtype, ws, wsb,
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(do=None), 1), (dict(cu=None), 1), (dict(N=-1), 1),
    (dict(dq=None), 1), (dict(dg=None), 1), (dict(mode=5), 1), (dict(gdtype=3), 1),
    (dict(H=4, Hqk=3), 1), (dict(chunk=24), 2), (dict(Dk=8), 2), (dict(cu=CU + 2), 3),
    (dict(dq=MIS), 3), (dict(h0=MIS), 3), (dict(dh0=MIS), 3), (dict(ws=None), 4),
    (dict(wsb=100), 4), (dict(ws=A + 64), 3),
])
def test_chunk_bwd_varlen_validation(L, kw, code):
    assert _bwd_v(L, **kw) == code


def test_chunk_bwd_varlen_nothing_to_do(L):
    assert _bwd_v(L, N=0, cu=None) == 0
    assert _bwd_v(L, T=0, q=None, k=None, v=None, g=None, beta=None, do=None, dq=None, dk=None,
                  dv=None, dg=None, dbeta=None) == 0


def test_chunk_bwd_varlen_workspace_size(L):
    f = L.kda_chunk_bwd_varlen_workspace_size
    assert f(0, 64, 1, 1, 128, 128, 64, 0, 1) == 0
    dense = L.kda_chunk_bwd_workspace_size(1, 64, 1, 1, 128, 128, 64, 0, 1)
    # room for ceil(T / chunk) + N chunk records plus the tables
    assert f(1, 64, 1, 1, 128, 128, 64, 0, 1) >= 2 * dense
    assert f(3, 64, 1, 1, 128, 128, 64, 0, 1) >= 4 * dense
    assert f(2, 0, 1, 1, 128, 128, 64, 0, 1) > 0


def test_noalloc_scratch_size_matches_header():
    import re
    text = open(K.HEADER).read()
    m = re.search(r"#define\s+KDA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*\*\s*(\d+)u\s*\*\s*(\d+)u\)", text)
    assert m, "KDA_NOALLOC_SCRATCH_BYTES not found"
    assert int(m.group(1)) * int(m.group(2)) * int(m.group(3)) == K.NOALLOC_SCRATCH_BYTES


def test_noalloc_validation_before_any_hip_call(L):
    def call(B=1, T=64, H=1, Dk=128, Dv=128, chunk=64, mode=0, dtype=1, o_dtype=0, q=A):
        return L.kda_chunk_fwd_noalloc(q, A, A, A, A, None, None, A, B, T, H, H, Dk, Dv, chunk,
                                       1.0, mode, dtype, o_dtype, 0, None)
    # beyond the fixed scratch: B1 H16 T8192 d128 needs 225 MiB of records
    assert call(T=8192, H=16) == 6
    assert call(mode=3) == 1 and call(dtype=2) == 1 and call(o_dtype=-1) == 1
    assert call(q=None) == 1 and call(q=MIS) == 3 and call(Dk=48) == 2

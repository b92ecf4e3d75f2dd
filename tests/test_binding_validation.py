"""The Python binding's argument checks (CPU only: every case below is
rejected from tensor metadata alone, before any device access).

The kernels index the gates as [.., H, Dk] in the channel mode and [.., H]
in the scalar mode, and write dg with that shape; a gate of any other shape
would be read (and its gradient written) out of bounds.  A caller-supplied
workspace's numel() is passed on as its byte count, so it must be a uint8
tensor of at least the required size.
"""
import pytest

torch = pytest.importorskip("torch")

import gated_delta_rule_17_amd as K  # noqa: E402

B, T, H, HQK, D = 2, 8, 4, 2, 16


def _dense(h=H, hq=H, gate="channel", dtype=torch.float32):
    q = torch.zeros(B, T, hq, D, dtype=dtype)
    k = torch.zeros(B, T, hq, D, dtype=dtype)
    v = torch.zeros(B, T, h, D, dtype=dtype)
    g = {"channel": torch.zeros(B, T, h, D), "scalar": torch.zeros(B, T, h), "none": None}[gate]
    beta = torch.zeros(B, T, h)
    return q, k, v, g, beta


def _packed(gate="channel"):
    q = torch.zeros(T, H, D)
    k = torch.zeros(T, H, D)
    v = torch.zeros(T, H, D)
    g = {"channel": torch.zeros(T, H, D), "scalar": torch.zeros(T, H), "none": None}[gate]
    beta = torch.zeros(T, H)
    cu = torch.tensor([0, 3, T], dtype=torch.int32)
    return q, k, v, g, beta, cu


def test_valid_metadata_reaches_the_device_check():
    q, k, v, g, beta = _dense()
    state = torch.zeros(B, H, D, D)
    with pytest.raises(ValueError, match="device tensor"):
        K.kda_recurrent_step(q, k, v, g, beta, state)
    with pytest.raises(ValueError, match="device tensor"):
        K.kda_chunk_fwd(q, k, v, g, beta)
    with pytest.raises(ValueError, match="device tensor"):
        K.kda_chunk_bwd(q, k, v, g, beta, torch.zeros_like(v))
    pq, pk, pv, pg, pb, cu = _packed()
    with pytest.raises(ValueError, match="device tensor"):
        K.kda_chunk_fwd_varlen(pq, pk, pv, pg, pb, cu)


@pytest.mark.parametrize("entry", ["recurrent", "chunk", "bwd"])
def test_channel_mode_needs_a_per_channel_gate(entry):
    q, k, v, _, beta = _dense()
    g = torch.zeros(B, T, H)                      # scalar-shaped gate, channel mode
    with pytest.raises(ValueError, match="g has shape"):
        if entry == "recurrent":
            K.kda_recurrent_step(q, k, v, g, beta, torch.zeros(B, H, D, D), mode="channel")
        elif entry == "chunk":
            K.kda_chunk_fwd(q, k, v, g, beta, mode="channel")
        else:
            K.kda_chunk_bwd(q, k, v, g, beta, torch.zeros_like(v), mode="channel")


def test_scalar_mode_rejects_a_per_channel_gate():
    q, k, v, g, beta = _dense()                   # 4-D gate
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_chunk_fwd(q, k, v, g, beta, mode="scalar")


def test_grouped_heads_gate_is_per_value_head():
    q, k, v, _, beta = _dense(h=H, hq=HQK)
    g = torch.zeros(B, T, HQK, D)                 # per query/key head: too small
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_chunk_fwd(q, k, v, g, beta)
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_chunk_bwd(q, k, v, g, beta, torch.zeros_like(v))


def test_gate_presence_matches_the_mode():
    q, k, v, g, beta = _dense()
    with pytest.raises(ValueError, match="None in the ungated mode"):
        K.kda_chunk_fwd(q, k, v, g, beta, mode="none")
    with pytest.raises(ValueError, match="required"):
        K.kda_chunk_fwd(q, k, v, None, beta, mode="scalar")


def test_packed_gate_shape():
    q, k, v, _, beta, cu = _packed()
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_chunk_fwd_varlen(q, k, v, torch.zeros(T, H), beta, cu, mode="channel")
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_recurrent_varlen(q, k, v, torch.zeros(T, H, D), beta, torch.zeros(2, H, D, D), cu,
                               mode="scalar")
    with pytest.raises(ValueError, match="g has shape"):
        K.kda_chunk_bwd_varlen(q, k, v, torch.zeros(T, HQK, D), beta, torch.zeros_like(v), cu)


def test_gradient_outputs_are_checked():
    q, k, v, g, beta = _dense()
    do = torch.zeros_like(v)
    with pytest.raises(ValueError, match="dg has shape"):
        K.kda_chunk_bwd(q, k, v, g, beta, do, out={"dg": torch.zeros(B, T, H)})
    with pytest.raises(ValueError, match="dbeta has shape"):
        K.kda_chunk_bwd(q, k, v, g, beta, do, out={"dbeta": torch.zeros(B, T, HQK)})
    with pytest.raises(TypeError):
        K.kda_chunk_bwd(q, k, v, g, beta, do, grad_dtype=torch.float16)


def test_caller_workspace_is_checked():
    q, k, v, g, beta = _dense()
    need = K.kda_chunk_fwd_workspace_size(B, T, H, D, D, 64, "channel", K.F32)
    assert need > 0
    with pytest.raises(TypeError, match="workspace"):
        K.kda_chunk_fwd(q, k, v, g, beta, workspace=torch.zeros(need, dtype=torch.float32))
    with pytest.raises(ValueError, match="bytes"):
        K.kda_chunk_fwd(q, k, v, g, beta, workspace=torch.zeros(need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="1-D"):
        K.kda_chunk_fwd(q, k, v, g, beta, workspace=torch.zeros(2, need, dtype=torch.uint8))


def test_shapes_of_the_token_tensors():
    q, k, v, g, beta = _dense()
    with pytest.raises(ValueError, match="beta has shape"):
        K.kda_chunk_fwd(q, k, v, g, beta[:, :, :2])
    with pytest.raises(ValueError, match="v has shape"):
        K.kda_chunk_fwd(q, k, v[:, :4], g, beta)
    with pytest.raises(TypeError):
        K.kda_chunk_fwd(q, k.to(torch.bfloat16), v, g, beta)
    with pytest.raises(ValueError, match="dimensions"):
        K.kda_chunk_fwd(q[0], k, v, g, beta)
    with pytest.raises(ValueError, match="d_o has shape"):
        K.kda_chunk_bwd(q, k, v, g, beta, torch.zeros(B, T, H, D + 16))

"""Host-side argument checks of the Python binding (no GPU).  The C ABI sees
only pointers and strides, so the binding checks every tensor's extent, the
decay vector and the device before it calls the library; each call below is
rejected before anything is enqueued."""
import pytest
import torch

from gated_linear_attention_gla_amd import _binding as gb

B, H, T, DK, DV = 1, 2, 32, 96, 192


def bf(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def qkv():
    return bf(B, H, T, DK), bf(B, H, T, DK), bf(B, H, T, DV)


def lam():
    return torch.full((H,), 0.9, dtype=torch.float32)


@pytest.fixture(autouse=True)
def _lib():
    gb.load_library()


def test_chunk_fwd_extents():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="k must have shape"):
        gb.chunk_fwd(q, bf(B, H, T - 1, DK), v, lam())
    with pytest.raises(ValueError, match="v must have shape"):
        gb.chunk_fwd(q, k, bf(B, H + 1, T, DV), lam())
    with pytest.raises(ValueError, match="lam must have shape"):
        gb.chunk_fwd(q, k, v, torch.full((H - 1,), 0.9))
    with pytest.raises(ValueError, match="lam must be torch.float32"):
        gb.chunk_fwd(q, k, v, torch.full((H,), 0.9, dtype=torch.float64))
    with pytest.raises(ValueError, match="o must have shape"):
        gb.chunk_fwd(q, k, v, lam(), o=bf(B, H, T, DK))
    with pytest.raises(ValueError, match="S0 must have shape"):
        gb.chunk_fwd(q, k, v, lam(), S0=torch.zeros(B, H, DV, DK))


def test_chunk_fwd_requires_gpu_tensors():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="same GPU device"):
        gb.chunk_fwd(q, k, v, lam())


def test_chunk_bwd_extents():
    q, k, v = qkv()
    dO = bf(B, H, T, DV)
    with pytest.raises(ValueError, match="dO must have shape"):
        gb.chunk_bwd(q, k, v, lam(), bf(B, H, T, DK))
    with pytest.raises(ValueError, match="dv must have shape"):
        gb.chunk_bwd(q, k, v, lam(), dO, dv=bf(B, H, T, DK))
    with pytest.raises(ValueError, match="dS_T must have shape"):
        gb.chunk_bwd(q, k, v, lam(), dO, dS_T=torch.zeros(B, H, DK, DK))
    with pytest.raises(ValueError, match="same GPU device"):
        gb.chunk_bwd(q, k, v, lam(), dO)


def test_decode_extents():
    N = 3
    q, k, v = bf(N, H, DK), bf(N, H, DK), bf(N, H, DV)
    S = torch.zeros(N, H, DK, DV)
    with pytest.raises(ValueError, match="v must have shape"):
        gb.decode_step_(q, k, bf(N - 1, H, DV), lam(), S)
    with pytest.raises(ValueError, match="o must have shape"):
        gb.decode_step_(q, k, v, lam(), S, o=bf(N, H, DK))
    with pytest.raises(ValueError, match="same GPU device"):
        gb.decode_step_(q, k, v, lam(), S)


def test_fused_and_varlen_extents():
    q, k, v = qkv()
    aug, gam = torch.zeros(H, DK), torch.ones(H, DV)
    with pytest.raises(ValueError, match="g must have shape"):
        gb.chunk_fwd_fused(q, k, v, lam(), bf(B, H, T, DK), aug, gam)
    Tt = 40
    pq, pk, pv = bf(Tt, H, DK), bf(Tt, H, DK), bf(Tt, H, DV)
    cu = torch.tensor([0, 10, 40], dtype=torch.int32)
    pool = torch.zeros(4, H, DK, DV)
    with pytest.raises(ValueError, match="k must have shape"):
        gb.chunk_fwd_varlen(pq, bf(Tt - 1, H, DK), pv, lam(), cu, pool)
    with pytest.raises(ValueError, match="same GPU device"):
        gb.chunk_fwd_varlen(pq, pk, pv, lam(), cu, pool)


def test_conv_extents():
    x = bf(2, 16, 64)
    w = torch.zeros(64, 4)
    with pytest.raises(ValueError, match="y must have shape"):
        gb.conv1d_fwd(x, w, y=bf(2, 15, 64))
    with pytest.raises(ValueError, match="same GPU device"):
        gb.conv1d_fwd(x, w)
    with pytest.raises(ValueError, match="y must have shape"):
        gb.conv1d_step_(bf(4, 64), w, None, torch.zeros(4, 3, 64), y=bf(4, 32))

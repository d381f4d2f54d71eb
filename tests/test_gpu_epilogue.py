"""GPU parity of the chunked forward with the fused output epilogue
(gla_chunk_fwd_fused) against the fp64 oracle: oracle.fwd followed by
oracle.epilogue (page "Beyond the KV cache ...", section "GLA mixer":
self-augmentation gate, Head RMSNorm per decay tier, SiLU(g) output gate).
Tolerances as for the forward: 1e-5 (fp32 inputs), 2e-3 (bf16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import inputs
from gpu_util import TOL, dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu
EPS = 1e-6


def run_fused(gla, x, e, dtype, chunk, g_dev=None):
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    g = g_dev if g_dev is not None else dev(e["g"], dtype)
    y, S = gla.chunk_fwd_fused(q, k, v, dev_f32(x["lam"]), g, dev_f32(e["aug"]), dev_f32(e["gamma"]), EPS,
                               dev_f32(x["S0"]), chunk=chunk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return host(y), host(S)


def reference(x, e, sl=slice(None)):
    ro, rS = oracle.fwd(x["q"][sl], x["k"][sl], x["v"][sl], x["lam"], None if x["S0"] is None else x["S0"][sl])
    ry = oracle.epilogue(x["q"][sl], x["k"][sl], x["v"][sl], ro, e["aug"], e["gamma"], EPS, e["g"][sl])
    return ry, rS


def check(gla, x, e, dtype, chunk):
    y, S = run_fused(gla, x, e, dtype, chunk)
    ry, rS = reference(x, e)
    ey, eS = oracle.rel_err(y, ry), oracle.rel_err(S, rS)
    flush(f"  fused chunk={chunk} {dtype} err y={ey:.3e} S_T={eS:.3e}")
    assert ey <= TOL[dtype] and eS <= TOL[dtype]


@pytest.mark.parametrize("T", [1, 17, 200])
@pytest.mark.parametrize("chunk", [16, 64])
def test_fused_small_fp32(gla, T, chunk):
    flush(f"test_fused_small_fp32 T={T} chunk={chunk}")
    x = inputs.random_chunk_inputs(700 + T, 2, 3, T, 16, 32, dtype="f32", scale=0.5)
    e = inputs.epilogue_inputs(700 + T, 2, 3, T, 16, 32, "f32")
    check(gla, x, e, "f32", chunk)


def test_fused_zero_balance_fp32(gla):
    """aug = 0 (the initial aug_balance): a half-strength skip of v."""
    flush("test_fused_zero_balance_fp32")
    x = inputs.random_chunk_inputs(710, 1, 2, 90, 16, 32, dtype="f32", scale=0.5)
    e = inputs.epilogue_inputs(710, 1, 2, 90, 16, 32, "f32", aug_scale=0.0)
    check(gla, x, e, "f32", 32)


@pytest.mark.parametrize("chunk", [16, 32])
def test_fused_full_dims_fp32(gla, chunk):
    flush(f"test_fused_full_dims_fp32 chunk={chunk}")
    x = inputs.random_chunk_inputs(720, 1, 2, 150, 96, 192, dtype="f32")
    e = inputs.epilogue_inputs(720, 1, 2, 150, 96, 192, "f32", aug_scale=0.1)
    check(gla, x, e, "f32", chunk)


@pytest.mark.parametrize("chunk", [32, 64])
def test_fused_laplace_bf16(gla, chunk):
    flush(f"test_fused_laplace_bf16 chunk={chunk}")
    x = inputs.make_chunk_inputs("laplace", T=700)
    e = inputs.epilogue_inputs(730, 1, 16, 700, 96, 192, "bf16", aug_scale=0.1)
    check(gla, x, e, "bf16", chunk)


def test_fused_token_major_gate_stream(gla):
    """g in the model's [B, T, H*dv] layout, viewed as (B, H, T, dv)."""
    flush("test_fused_token_major_gate_stream")
    B, H, T = 2, 4, 130
    x = inputs.random_chunk_inputs(740, B, H, T, 96, 192, dtype="bf16", scale=0.3)
    e = inputs.epilogue_inputs(740, B, H, T, 96, 192, "bf16", aug_scale=0.1)
    gtm = dev(np.ascontiguousarray(e["g"].transpose(0, 2, 1, 3)).reshape(B, T, H * 192), "bf16")
    g_view = gtm.view(B, T, H, 192).transpose(1, 2)
    y, S = run_fused(gla, x, e, "bf16", 64, g_dev=g_view)
    ry, rS = reference(x, e)
    assert oracle.rel_err(y, ry) <= TOL["bf16"] and oracle.rel_err(S, rS) <= TOL["bf16"]


def test_fused_training_shape_sampled(gla):
    """The benched shape (B=8, H=16, T=2,048, chunk 64); the oracle rechecks
    the (b, h) units of b in {0, 7}."""
    flush("test_fused_training_shape_sampled")
    x = inputs.make_chunk_inputs("training")
    e = inputs.epilogue_inputs(750, 8, 16, 2048, 96, 192, "bf16", aug_scale=0.1)
    y, S = run_fused(gla, x, e, "bf16", 64)
    for b in (0, 7):
        sl = slice(b, b + 1)
        ry, rS = reference(x, e, sl)
        ey, eS = oracle.rel_err(y[sl], ry), oracle.rel_err(S[sl], rS)
        flush(f"  b={b} err y={ey:.3e} S_T={eS:.3e}")
        assert ey <= TOL["bf16"] and eS <= TOL["bf16"]


@pytest.mark.parametrize("dims", [(16, 32, "f32"), (96, 192, "bf16"), (96, 192, "f32")])
def test_fused_decode_steps(gla, dims):
    """The decode step with the epilogue against oracle.decode_step followed
    by oracle.epilogue, over several steps (state updated in place)."""
    dk, dv, dtype = dims
    flush(f"test_fused_decode_steps dk={dk} dv={dv} {dtype}")
    N, H, steps = 29, 3, 4
    x = inputs.random_chunk_inputs(760 + dk, N, H, steps, dk, dv, dtype=dtype, scale=1.0)
    e = inputs.epilogue_inputs(760 + dk, N, H, steps, dk, dv, dtype, aug_scale=0.2)
    S_host = inputs.normal(760 + dk, inputs.TID["S"], (N, H, dk, dv), 0.01, "f32")
    S, lam, Sref = dev_f32(S_host), dev_f32(x["lam"]), S_host.copy()
    aug, gam = dev_f32(e["aug"]), dev_f32(e["gamma"])
    for t in range(steps):
        q, k, v, g = (dev(np.ascontiguousarray(arr[:, :, t]), dtype)
                      for arr in (x["q"], x["k"], x["v"], e["g"]))
        y = gla.decode_step_fused_(q, k, v, lam, S, g, aug, gam, EPS, out_dtype=torch.float32)
        ro, Sref = oracle.decode_step(x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t], x["lam"], Sref)
        sl = lambda a: a[:, :, t:t + 1]
        ry = oracle.epilogue(sl(x["q"]), sl(x["k"]), sl(x["v"]), ro[:, :, None], e["aug"], e["gamma"], EPS,
                             sl(e["g"]))[:, :, 0]
        torch.cuda.synchronize()
        assert oracle.rel_err(host(y), ry) <= 1e-5
    assert oracle.rel_err(host(S), Sref) <= 1e-5

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


@pytest.mark.parametrize("chunk", [32, 64, 128])
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


@pytest.mark.parametrize("use_ws", [True, False])
@pytest.mark.parametrize("dims", [(16, 32, "f32"), (96, 192, "bf16"), (96, 192, "f32")])
def test_fused_decode_steps(gla, dims, use_ws):
    """The decode step with the epilogue against oracle.decode_step followed
    by oracle.epilogue, over several steps (state updated in place), with the
    workspace (column slices + normalisation kernel at (96, 192)) and
    without (one workgroup per state)."""
    dk, dv, dtype = dims
    flush(f"test_fused_decode_steps dk={dk} dv={dv} {dtype} workspace={use_ws}")
    N, H, steps = 29, 3, 4
    x = inputs.random_chunk_inputs(760 + dk, N, H, steps, dk, dv, dtype=dtype, scale=1.0)
    e = inputs.epilogue_inputs(760 + dk, N, H, steps, dk, dv, dtype, aug_scale=0.2)
    S_host = inputs.normal(760 + dk, inputs.TID["S"], (N, H, dk, dv), 0.01, "f32")
    S, lam, Sref = dev_f32(S_host), dev_f32(x["lam"]), S_host.copy()
    aug, gam = dev_f32(e["aug"]), dev_f32(e["gamma"])
    for t in range(steps):
        q, k, v, g = (dev(np.ascontiguousarray(arr[:, :, t]), dtype)
                      for arr in (x["q"], x["k"], x["v"], e["g"]))
        y = gla.decode_step_fused_(q, k, v, lam, S, g, aug, gam, EPS, out_dtype=torch.float32,
                                   use_workspace=use_ws)
        ro, Sref = oracle.decode_step(x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t], x["lam"], Sref)
        sl = lambda a: a[:, :, t:t + 1]
        ry = oracle.epilogue(sl(x["q"]), sl(x["k"]), sl(x["v"]), ro[:, :, None], e["aug"], e["gamma"], EPS,
                             sl(e["g"]))[:, :, 0]
        torch.cuda.synchronize()
        assert oracle.rel_err(host(y), ry) <= 1e-5
    assert oracle.rel_err(host(S), Sref) <= 1e-5


def test_fused_decode_full_slab_sampled(gla):
    """The fused decode step in the launch configuration the benchmark times:
    one 1,280 x 16 slab of fp32 96 x 192 states, q/k/v as strided views of one
    packed bf16 block per step, a bf16 gate stream, bf16 output.  Two steps.
    Each call is repeated with fp32 output on a copy of the slab and with the
    plain decode step on another copy: the three state updates must agree bit
    for bit, the bf16 output must be the fp32 output rounded to nearest
    (within one bf16 ulp), and for 12 sampled (sequence, head) pairs the fp32
    output and the state must match oracle.decode_step + oracle.epilogue to
    1e-5.  The step runs with its workspace, as benchmarked; the same step
    without a workspace (one workgroup per state) on a third copy must give
    the same state and an fp32 output within 1e-5 of it."""
    flush("test_fused_decode_full_slab_sampled N=1280 H=16")
    N, H, dk, dv, steps = 1280, 16, 96, 192, 2
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_303)
    S = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    S.normal_(0.0, 0.01, generator=g)
    qkv = torch.randn((steps, N, H, dk + dk + dv), generator=g, device="cuda").to(torch.bfloat16)
    gz = torch.randn((steps, N, H, dv), generator=g, device="cuda").to(torch.bfloat16)
    aug = (0.2 * torch.randn((H, dk), generator=g, device="cuda")).contiguous()
    gam = (1.0 + 0.1 * torch.randn((H, dv), generator=g, device="cuda")).contiguous()
    lam_h = np.asarray(inputs.lambda_log_spaced(H, 0.95, 0.9999), dtype=np.float32)
    lam = dev_f32(lam_h)
    aug_h, gam_h = host(aug), host(gam)
    rng = np.random.default_rng(11)
    pairs = [(int(n), int(h)) for n, h in zip(rng.integers(0, N, 12), rng.integers(0, H, 12))]
    ref_S = {(n, h): host(S[n, h]) for n, h in pairs}
    y16 = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    for st in range(steps):
        blk, gs = qkv[st], gz[st]
        qv, kv, vv = blk[..., :dk], blk[..., dk:2 * dk], blk[..., 2 * dk:]
        S32, Spl, Snw = S.clone(), S.clone(), S.clone()
        gla.decode_step_fused_(qv, kv, vv, lam, S, gs, aug, gam, EPS, y=y16)
        y32 = gla.decode_step_fused_(qv, kv, vv, lam, S32, gs, aug, gam, EPS, out_dtype=torch.float32)
        gla.decode_step_(qv, kv, vv, lam, Spl, out_dtype=torch.float32)
        ynw = gla.decode_step_fused_(qv, kv, vv, lam, Snw, gs, aug, gam, EPS, out_dtype=torch.float32,
                                     use_workspace=False)
        torch.cuda.synchronize()
        assert torch.equal(S, S32) and torch.equal(S, Spl) and torch.equal(S, Snw), st
        assert oracle.rel_err(host(ynw), host(y32)) <= 1e-5, st
        del S32, Spl, Snw, ynw
        a = y16.view(torch.int16).cpu().numpy().astype(np.int32)
        b = y32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
        assert np.max(np.abs(a - b)) <= 1, st
        got, bh, gh = host(y32), host(blk), host(gs)
        for n, h in pairs:
            q1 = bh[n, h, :dk][None, None, None]
            k1 = bh[n, h, dk:2 * dk][None, None, None]
            v1 = bh[n, h, 2 * dk:][None, None, None]
            ro, rS = oracle.decode_step(q1[:, :, 0], k1[:, :, 0], v1[:, :, 0], lam_h[h:h + 1],
                                        ref_S[(n, h)][None, None])
            ref_S[(n, h)] = rS[0, 0]
            ry = oracle.epilogue(q1, k1, v1, ro[:, :, None], aug_h[h:h + 1], gam_h[h:h + 1], EPS,
                                 gh[n, h][None, None, None])
            assert oracle.rel_err(got[n, h], ry[0, 0, 0]) <= 1e-5, (st, n, h)
    for n, h in pairs:
        assert oracle.rel_err(host(S[n, h]), ref_S[(n, h)]) <= 1e-5, (n, h)


def test_fused_decode_single_state_bf16_out(gla):
    """One sequence and one head (N * H = 1) with bf16 inputs and output: the
    workspace path (column slices + normalisation kernel) against the oracle,
    with the bf16 output equal to the fp32 output rounded to nearest (within
    one bf16 ulp), and the same state as the path without a workspace."""
    flush("test_fused_decode_single_state_bf16_out")
    dk, dv = 96, 192
    x = inputs.random_chunk_inputs(790, 1, 1, 1, dk, dv, dtype="bf16", scale=1.0)
    e = inputs.epilogue_inputs(790, 1, 1, 1, dk, dv, "bf16", aug_scale=0.2)
    S_host = inputs.normal(790, inputs.TID["S"], (1, 1, dk, dv), 0.01, "f32")
    q, k, v, g = (dev(np.ascontiguousarray(arr[:, :, 0]), "bf16") for arr in (x["q"], x["k"], x["v"], e["g"]))
    lam, aug, gam = dev_f32(x["lam"]), dev_f32(e["aug"]), dev_f32(e["gamma"])
    S16, S32, Snw = dev_f32(S_host), dev_f32(S_host), dev_f32(S_host)
    y16 = gla.decode_step_fused_(q, k, v, lam, S16, g, aug, gam, EPS, out_dtype=torch.bfloat16)
    y32 = gla.decode_step_fused_(q, k, v, lam, S32, g, aug, gam, EPS, out_dtype=torch.float32)
    gla.decode_step_fused_(q, k, v, lam, Snw, g, aug, gam, EPS, out_dtype=torch.float32, use_workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(S16, S32) and torch.equal(S16, Snw)
    a = y16.view(torch.int16).cpu().numpy().astype(np.int32)
    b = y32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
    assert np.max(np.abs(a - b)) <= 1
    ro, rS = oracle.decode_step(x["q"][:, :, 0], x["k"][:, :, 0], x["v"][:, :, 0], x["lam"], S_host)
    ry = oracle.epilogue(x["q"], x["k"], x["v"], ro[:, :, None], e["aug"], e["gamma"], EPS, e["g"])[:, :, 0]
    assert oracle.rel_err(host(y32), ry) <= 1e-5
    assert oracle.rel_err(host(S32), rS) <= 1e-5


"""Every (head dims, chunk, input dtype) combination the library accepts,
run once against the fp64 oracle: the chunked forward, the backward and the
forward with the fused output epilogue, on a small ragged input (B=1, H=2,
T=77, with S0 and dS_T).  A combination the C ABI rejects as unsupported is
skipped (the rejection itself is covered by the CPU ABI tests); the
supported set is the one include/gla.h documents."""
import itertools

import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import _binding as gb
from gated_linear_attention_gla_amd import inputs
from gpu_util import TOL, dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu
UNSUPPORTED = 5
DIMS = [(96, 192), (16, 32)]
CHUNKS = [16, 32, 64, 128]
DTYPES = ["bf16", "f32"]
CASES = list(itertools.product(DIMS, CHUNKS, DTYPES))


def _inputs(dims, dtype, seed):
    dk, dv = dims
    return inputs.random_chunk_inputs(seed, 1, 2, 77, dk, dv, dtype=dtype, dS_T=True,
                                      scale=0.5 if dtype == "bf16" else None)


def _call_or_skip(fn):
    try:
        return fn()
    except gb.GlaError as err:
        if err.status == UNSUPPORTED:
            pytest.skip("combination not supported by the ABI")
        raise


@pytest.mark.parametrize("dims,chunk,dtype", CASES)
def test_fwd_bwd_every_supported_combination(gla, dims, chunk, dtype):
    flush(f"test_fwd_bwd_every_supported_combination dims={dims} chunk={chunk} {dtype}")
    x = _inputs(dims, dtype, 900 + dims[0] + chunk)
    q, k, v, dO = (dev(x[n], dtype) for n in ("q", "k", "v", "dO"))
    lam, S0, dST = dev_f32(x["lam"]), dev_f32(x["S0"]), dev_f32(x["dS_T"])
    o, S = _call_or_skip(lambda: gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32))
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    assert oracle.rel_err(host(o), ro) <= TOL[dtype] and oracle.rel_err(host(S), rS) <= TOL[dtype]
    g = _call_or_skip(lambda: gla.chunk_bwd(q, k, v, lam, dO, S0, dST, chunk=chunk, grad_dtype=torch.float32))
    torch.cuda.synchronize()
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"], x["dS_T"])
    errs = [oracle.rel_err(host(a), b) for a, b in zip(g, r)]
    flush("  err o/S_T " + f"{oracle.rel_err(host(o), ro):.2e} {oracle.rel_err(host(S), rS):.2e}"
          + "  dq/dk/dv/dS0 " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= TOL[dtype]


@pytest.mark.parametrize("dims,chunk,dtype", CASES)
def test_fused_every_supported_combination(gla, dims, chunk, dtype):
    flush(f"test_fused_every_supported_combination dims={dims} chunk={chunk} {dtype}")
    dk, dv = dims
    x = _inputs(dims, dtype, 950 + dk + chunk)
    e = inputs.epilogue_inputs(950 + dk + chunk, 1, 2, 77, dk, dv, dtype, aug_scale=0.5)
    q, k, v, g = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype), dev(e["g"], dtype)
    y, S = _call_or_skip(lambda: gla.chunk_fwd_fused(q, k, v, dev_f32(x["lam"]), g, dev_f32(e["aug"]),
                                                     dev_f32(e["gamma"]), 1e-6, dev_f32(x["S0"]), chunk=chunk,
                                                     out_dtype=torch.float32))
    torch.cuda.synchronize()
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    ry = oracle.epilogue(x["q"], x["k"], x["v"], ro, e["aug"], e["gamma"], 1e-6, e["g"])
    ey, eS = oracle.rel_err(host(y), ry), oracle.rel_err(host(S), rS)
    flush(f"  err y {ey:.2e} S_T {eS:.2e}")
    assert ey <= TOL[dtype] and eS <= TOL[dtype]

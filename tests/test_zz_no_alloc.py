"""gla_chunk_fwd_noalloc (the forward whose segment states live in the
library's static device scratch) against gla_chunk_fwd (caller workspace):
two calls in a row on workloads that use the segment split, the second
smaller and ragged, so it runs over what the first left in the scratch.
Both must give the workspace entry point's results bit for bit (same kernels,
same segments), and those are within the bf16 gate of the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import inputs
from gpu_util import TOL, dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu

# (seed, B, H, T, chunk): the Laplace layer shape (128 segment states, 9.4 MB
# of scratch), then 4 heads over 700 tokens (44 states, a ragged last chunk)
CASES = [(601, 1, 16, 2048, 64), (602, 1, 4, 700, 32)]


def test_noalloc_matches_workspace_entry_point(gla):
    lib = gla.load_library()
    for seed, B, H, T, chunk in CASES:
        flush(f"test_noalloc_matches_workspace_entry_point B={B} H={H} T={T} chunk={chunk}")
        x = inputs.random_chunk_inputs(seed, B, H, T, 96, 192, dtype="bf16")
        d = gla.GlaDims(B, H, T, 96, 192, chunk)
        need = lib.gla_chunk_fwd_workspace(ctypes.byref(d))
        assert 0 < need <= 16 << 20, need  # the case exercises the scratch
        q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
        lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
        o = torch.empty((B, H, T, 192), dtype=torch.float32, device="cuda")
        S_T = torch.empty((B, H, 96, 192), dtype=torch.float32, device="cuda")
        gla.chunk_fwd_noalloc(q, k, v, lam, S0, o, S_T, chunk=chunk)
        o_ref, S_ref = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)
        ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
        eo, eS = oracle.rel_err(host(o), ro), oracle.rel_err(host(S_T), rS)
        flush(f"  equal to gla_chunk_fwd; oracle err o={eo:.3e} S_T={eS:.3e}")
        assert eo <= TOL["bf16"] and eS <= TOL["bf16"]


def test_noalloc_without_segment_split_and_empty(gla):
    """Dims that need no segment states (the training batch size, and an
    empty sequence) take no scratch at all: results equal gla_chunk_fwd's;
    T = 0 passes S0 through as S_T."""
    lib = gla.load_library()
    for seed, B, H, T, chunk in ((603, 8, 16, 256, 64), (604, 1, 2, 0, 64)):
        flush(f"test_noalloc_without_segment_split_and_empty B={B} H={H} T={T}")
        x = inputs.random_chunk_inputs(seed, B, H, T, 96, 192, dtype="bf16")
        d = gla.GlaDims(B, H, T, 96, 192, chunk)
        assert lib.gla_chunk_fwd_workspace(ctypes.byref(d)) == 0
        q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
        lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
        o = torch.empty((B, H, T, 192), dtype=torch.bfloat16, device="cuda")
        S_T = torch.empty((B, H, 96, 192), dtype=torch.float32, device="cuda")
        gla.chunk_fwd_noalloc(q, k, v, lam, S0, o, S_T, chunk=chunk)
        o_ref, S_ref = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)
        if T == 0:
            assert torch.equal(S_T, S0)


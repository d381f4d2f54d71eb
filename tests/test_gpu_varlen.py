"""GPU parity of the packed variable-length prefill into the decode state pool
(gla_chunk_fwd_varlen) against the fp64 oracle, sequence by sequence (page
"Beyond the KV cache ...", sections "GLA mixer" and "Inference optimization
on Trainium2": one fixed-size state page per sequence, filled by prefill and
then read and written by every decode step).

Each sequence must match oracle.fwd run on it alone, starting from its
page's state (or zero), within the benchmark spec's tolerance; pages of other
slots and other layers must be left bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import inputs
from gpu_util import TOL, dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu


def run_varlen(gla, x, dtype, chunk, layer=0, slots=True, has=True):
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    lam = dev_f32(x["lam"])
    pool_all = dev_f32(x["pool"])
    pool = pool_all[:, layer]
    cu = torch.tensor(x["cu"], dtype=torch.int32, device="cuda")
    sl = torch.tensor(x["slots"], dtype=torch.int32, device="cuda") if slots else None
    hs = torch.tensor(x["has_state"], dtype=torch.int32, device="cuda") if has else None
    o = gla.chunk_fwd_varlen(q, k, v, lam, cu, pool, sl, hs, chunk=chunk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return host(o), host(pool_all)


def check_varlen(gla, x, dtype, chunk, layer=0):
    o, pool = run_varlen(gla, x, dtype, chunk, layer)
    tol = TOL[dtype]
    expect_pool = x["pool"].copy()
    worst = 0.0
    for n, (c0, c1) in enumerate(zip(x["cu"][:-1], x["cu"][1:])):
        sl = x["slots"][n]
        s0 = x["pool"][sl, layer][None] if x["has_state"][n] else None
        q, k, v = (x[t][c0:c1].transpose(1, 0, 2)[None] for t in ("q", "k", "v"))
        ro, rS = oracle.fwd(q, k, v, x["lam"], s0)
        if c1 > c0:
            e = oracle.rel_err(o[c0:c1].transpose(1, 0, 2)[None], ro)
            worst = max(worst, e)
            assert e <= tol, (n, e)
        assert oracle.rel_err(pool[sl, layer][None], rS) <= tol, n
        expect_pool[sl, layer] = pool[sl, layer]
    flush(f"  varlen worst o err {worst:.3e}")
    # nothing outside the sequences' pages changed
    assert np.array_equal(pool, expect_pool)


@pytest.mark.parametrize("chunk", [16, 64])
def test_varlen_small_fp32(gla, chunk):
    flush(f"test_varlen_small_fp32 chunk={chunk}")
    lengths = [0, 1, 15, 64, 65, 200, 3, 130]
    x = inputs.varlen_inputs(600, lengths, 3, 16, 32, num_slots=12, dtype="f32", pages=2)
    x["lam"] = inputs.round_f32(np.array([0.5, 0.9, 0.999]))
    check_varlen(gla, x, "f32", chunk, layer=1)


@pytest.mark.parametrize("chunk", [64, 128])
def test_varlen_page_shape_bf16(gla, chunk):
    flush(f"test_varlen_page_shape_bf16 chunk={chunk}")
    lengths = [300, 1, 0, 777, 64, 129, 1500, 17]
    x = inputs.varlen_inputs(610, lengths, 16, 96, 192, num_slots=20, dtype="bf16", pages=3)
    x["lam"] = inputs.lambda_log_spaced(16, 0.9, 0.999)
    check_varlen(gla, x, "bf16", chunk, layer=2)


def test_varlen_serving_mix(gla):
    """The benched length mix (64 prompts, 16..4,096 tokens), sampled: the
    oracle rechecks every fourth sequence."""
    flush("test_varlen_serving_mix")
    c = inputs.CONFIGS["varlen"]
    lengths = inputs.varlen_lengths(c["cid"], c["N"], c["min_len"], c["max_len"])
    x = inputs.varlen_inputs(c["cid"], lengths, c["H"], c["dk"], c["dv"], num_slots=c["slots"])
    x["lam"] = inputs.lambda_log_spaced(c["H"], 0.95, 0.9999)
    o, pool = run_varlen(gla, x, "bf16", 64)
    for n in range(0, c["N"], 4):
        c0, c1, sl = x["cu"][n], x["cu"][n + 1], x["slots"][n]
        s0 = x["pool"][sl, 0][None] if x["has_state"][n] else None
        q, k, v = (x[t][c0:c1].transpose(1, 0, 2)[None] for t in ("q", "k", "v"))
        ro, rS = oracle.fwd(q, k, v, x["lam"], s0)
        assert oracle.rel_err(o[c0:c1].transpose(1, 0, 2)[None], ro) <= TOL["bf16"]
        assert oracle.rel_err(pool[sl, 0][None], rS) <= TOL["bf16"]


@pytest.mark.parametrize("n,chunk", [(300, 16), (600, 32)])
def test_varlen_many_sequences_with_ties(gla, n, chunk):
    """Many short sequences with heavily repeated lengths (ties in the
    longest-first order are broken by index), below and above the 512
    sequences up to which the workgroups rank the lengths (natural order
    beyond): every sequence must be served exactly once."""
    flush(f"test_varlen_many_sequences_with_ties n={n} chunk={chunk}")
    rng = np.random.default_rng(650 + n)
    lengths = rng.choice([0, 1, 5, 16, 17, 33], size=n)
    x = inputs.varlen_inputs(650 + n, lengths, 2, 16, 32, num_slots=n + 7, dtype="f32")
    x["lam"] = inputs.round_f32(np.array([0.7, 0.99]))
    check_varlen(gla, x, "f32", chunk)


def test_varlen_identity_slots_all_continue(gla):
    """slots = NULL (sequence n uses page n) and has_state = NULL (all continue)."""
    flush("test_varlen_identity_slots_all_continue")
    lengths = [40, 0, 100, 7]
    x = inputs.varlen_inputs(620, lengths, 2, 16, 32, num_slots=4, dtype="f32", slots=False,
                             has_state=False)
    x["lam"] = inputs.round_f32(np.array([0.8, 0.95]))
    q, k, v = dev(x["q"], "f32"), dev(x["k"], "f32"), dev(x["v"], "f32")
    pool = dev_f32(x["pool"])[:, 0]
    cu = torch.tensor(x["cu"], dtype=torch.int32, device="cuda")
    o = gla.chunk_fwd_varlen(q, k, v, dev_f32(x["lam"]), cu, pool, None, None, chunk=32,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    for n in range(4):
        c0, c1 = x["cu"][n], x["cu"][n + 1]
        q_, k_, v_ = (x[t][c0:c1].transpose(1, 0, 2)[None] for t in ("q", "k", "v"))
        ro, rS = oracle.fwd(q_, k_, v_, x["lam"], x["pool"][n, 0][None])
        if c1 > c0:
            assert oracle.rel_err(host(o)[c0:c1].transpose(1, 0, 2)[None], ro) <= TOL["f32"]
        assert oracle.rel_err(host(pool[n])[None], rS) <= TOL["f32"]


def test_varlen_skips_out_of_range_slots_and_clamps_offsets(gla):
    """Slots outside [0, num_slots) skip their sequence; offsets beyond the
    packed tokens are clamped on the device (no access outside the tensors)."""
    flush("test_varlen_skips_out_of_range_slots_and_clamps_offsets")
    lengths = [20, 30, 10]
    x = inputs.varlen_inputs(630, lengths, 2, 16, 32, num_slots=6, dtype="f32", has_state=False)
    x["lam"] = inputs.round_f32(np.array([0.7, 0.9]))
    x["slots"] = np.array([-1, 2, 6])
    q, k, v = dev(x["q"], "f32"), dev(x["k"], "f32"), dev(x["v"], "f32")
    pool_all = dev_f32(x["pool"])
    pool = pool_all[:, 0]
    # the last sequence's end offset points far past the packed tokens
    cu = torch.tensor([0, 20, 50, 100000], dtype=torch.int32, device="cuda")
    o = torch.full((60, 2, 32), 7.0, dtype=torch.float32, device="cuda")
    gla.chunk_fwd_varlen(q, k, v, dev_f32(x["lam"]), cu, pool,
                         torch.tensor(x["slots"], dtype=torch.int32, device="cuda"), None, chunk=16, o=o)
    torch.cuda.synchronize()
    pool_h = host(pool_all)
    # sequence 1 (slot 2) is computed, 0 and 2 are skipped
    q_, k_, v_ = (x[t][20:50].transpose(1, 0, 2)[None] for t in ("q", "k", "v"))
    ro, rS = oracle.fwd(q_, k_, v_, x["lam"], x["pool"][2, 0][None])
    assert oracle.rel_err(host(o)[20:50].transpose(1, 0, 2)[None], ro) <= TOL["f32"]
    assert oracle.rel_err(pool_h[2, 0][None], rS) <= TOL["f32"]
    expect = x["pool"].copy()
    expect[2, 0] = pool_h[2, 0]
    assert np.array_equal(pool_h, expect)
    assert torch.all(o[:20] == 7.0) and torch.all(o[50:] == 7.0)


def test_varlen_prefill_then_decode(gla):
    """Serving hand-off: prefill into the pool, then decode steps on the same
    pages, equal the oracle run over prompt + generated tokens."""
    flush("test_varlen_prefill_then_decode")
    H, dk, dv, steps = 16, 96, 192, 4
    prompts = [50, 200, 1, 130]
    total = [p + steps for p in prompts]
    x = inputs.varlen_inputs(640, total, H, dk, dv, num_slots=8, dtype="bf16", has_state=False)
    x["lam"] = inputs.lambda_log_spaced(H, 0.9, 0.999)
    N = len(prompts)
    # packed prompt tokens only
    idx = np.concatenate([np.arange(x["cu"][n], x["cu"][n] + prompts[n]) for n in range(N)])
    cu_p = np.concatenate([[0], np.cumsum(prompts)])
    q, k, v = (dev(np.ascontiguousarray(x[t][idx]), "bf16") for t in ("q", "k", "v"))
    lam = dev_f32(x["lam"])
    pool = torch.zeros((8, H, dk, dv), dtype=torch.float32, device="cuda")
    sl = torch.tensor(x["slots"], dtype=torch.int32, device="cuda")
    zero = torch.zeros(N, dtype=torch.int32, device="cuda")
    gla.chunk_fwd_varlen(q, k, v, lam, torch.tensor(cu_p, dtype=torch.int32, device="cuda"), pool, sl,
                         zero, chunk=64)
    # decode: the pages of the N sequences, gathered as a strided view is not
    # possible for arbitrary slots, so step a dense copy and scatter back
    S = pool[sl.long()].contiguous()
    outs = []
    for t in range(steps):
        rows = [x["cu"][n] + prompts[n] + t for n in range(N)]
        qt, kt, vt = (dev(np.ascontiguousarray(x[nm][rows]), "bf16") for nm in ("q", "k", "v"))
        outs.append(host(gla.decode_step_(qt, kt, vt, lam, S, out_dtype=torch.float32)))
    torch.cuda.synchronize()
    for n in range(N):
        c0, c1 = x["cu"][n], x["cu"][n + 1]
        q_, k_, v_ = (x[t][c0:c1].transpose(1, 0, 2)[None] for t in ("q", "k", "v"))
        ro, rS = oracle.fwd(q_, k_, v_, x["lam"])
        got = np.stack([outs[t][n] for t in range(steps)], axis=1)[None]  # (1, H, steps, dv)
        assert oracle.rel_err(got, ro[:, :, prompts[n]:]) <= TOL["bf16"]
        assert oracle.rel_err(host(S[n])[None], rS) <= TOL["bf16"]

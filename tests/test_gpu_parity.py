"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Gate (per output tensor, max|err| / max|ref| in fp64): 2e-3 for bf16 inputs,
1e-5 for fp32 inputs, measured on fp32-stored outputs.  bf16-stored outputs
must equal the round-to-nearest-even of the fp32-stored run (within one bf16
ulp, for the accumulation order may differ between the two launches).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import inputs
from gpu_util import TOL, dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu


def run_fwd(gla, x, dtype, chunk, out_dtype=torch.float32):
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
    o, S = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(o), host(S)


def check_fwd(gla, x, dtype, chunk, tol=None):
    tol = tol or TOL[dtype]
    o, S = run_fwd(gla, x, dtype, chunk)
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    eo, eS = oracle.rel_err(o, ro), oracle.rel_err(S, rS)
    flush(f"  fwd chunk={chunk} dtype={dtype} err o={eo:.3e} S_T={eS:.3e}")
    assert eo <= tol and eS <= tol
    return eo, eS


# ------------------------------------------------------------------ forward
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fwd_tiny_fp32(gla, chunk):
    flush(f"test_fwd_tiny_fp32 chunk={chunk}")
    x = inputs.make_chunk_inputs("tiny")
    check_fwd(gla, x, "f32", chunk)


@pytest.mark.parametrize("T", [1, 15, 17, 63, 65, 129, 200])
@pytest.mark.parametrize("chunk", [16, 64])
def test_fwd_ragged_fp32(gla, T, chunk):
    flush(f"test_fwd_ragged_fp32 T={T} chunk={chunk}")
    x = inputs.random_chunk_inputs(100 + T, 2, 3, T, 16, 32, dtype="f32")
    check_fwd(gla, x, "f32", chunk)


def test_fwd_empty_sequence(gla):
    flush("test_fwd_empty_sequence")
    x = inputs.random_chunk_inputs(99, 1, 2, 0, 16, 32, dtype="f32")
    o, S = run_fwd(gla, x, "f32", 32)
    assert o.shape == (1, 2, 0, 32)
    assert np.array_equal(S, x["S0"])


@pytest.mark.parametrize("lam", [0.0, 1.0, 0.5])
def test_fwd_lambda_edges_fp32(gla, lam):
    flush(f"test_fwd_lambda_edges_fp32 lam={lam}")
    x = inputs.random_chunk_inputs(120, 1, 2, 100, 16, 32, dtype="f32", lam=np.full(2, lam))
    check_fwd(gla, x, "f32", 32)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_fwd_fp32_full_head_dims(gla, chunk):
    flush(f"test_fwd_fp32_full_head_dims chunk={chunk}")
    x = inputs.random_chunk_inputs(130, 1, 2, 200, 96, 192, dtype="f32")
    check_fwd(gla, x, "f32", chunk)


@pytest.mark.parametrize("chunk", [16, 32])
def test_bwd_fp32_full_head_dims(gla, chunk):
    """fp32 backward at dk=96, dv=192 (the transposed passes' three-plane
    kernels), ragged T with dS_T; the small batch also takes the segment
    split."""
    flush(f"test_bwd_fp32_full_head_dims chunk={chunk}")
    x = inputs.random_chunk_inputs(135, 1, 2, 150, 96, 192, dtype="f32", dS_T=True)
    assert segments_of(gla, 1, 2, 150, 96, 192, chunk, bwd=True) >= 2
    check_bwd(gla, x, "f32", chunk)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_fwd_bf16_chunk_invariance(gla, chunk):
    """Same bf16 inputs (Laplace recipe, 4 heads, ragged T) at every chunk."""
    flush(f"test_fwd_bf16_chunk_invariance chunk={chunk}")
    x = inputs.make_chunk_inputs("laplace", T=700)
    for key in ("q", "k", "v", "S0"):
        x[key] = x[key][:, :4]
    x["lam"] = x["lam"][:4]
    check_fwd(gla, x, "bf16", chunk)


@pytest.mark.parametrize("chunk", [64, 128])
def test_fwd_laplace_full(gla, chunk):
    """Laplace layer shape (B=1, H=16, T=2048, dk=96, dv=192, bf16)."""
    flush(f"test_fwd_laplace_full chunk={chunk}")
    x = inputs.make_chunk_inputs("laplace")
    check_fwd(gla, x, "bf16", chunk)
    # bf16-stored o = RNE(fp32-stored o) within one bf16 ulp
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
    o32, _ = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
    o16, _ = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = o16.view(torch.int16).cpu().numpy().astype(np.int32)
    b = o32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
    assert np.max(np.abs(a - b)) <= 1



def test_fwd_long_context_full(gla):
    """Long-context prefill at its full size (B=1, H=16, T=65,536, bf16,
    lambda in [0.95, 0.9999]) in the launch configurations the benchmark times
    (64-token chunks: all 192 columns per workgroup, 16 segments per head;
    128-token chunks: two column blocks, 8 segments): the whole fp32-stored
    output and the final state against the oracle, and the bf16-stored output
    equal to the fp32-stored one rounded to nearest, within one bf16 ulp."""
    flush("test_fwd_long_context_full T=65536")
    x = inputs.make_chunk_inputs("long")
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
    for chunk in (64, 128):
        assert segments_of(gla, 1, 16, 65536, 96, 192, chunk) == (16 if chunk == 64 else 8)
        o32, S32 = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
        o16, _ = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        eo, eS = oracle.rel_err(host(o32), ro), oracle.rel_err(host(S32), rS)
        flush(f"  chunk={chunk} err o={eo:.3e} S_T={eS:.3e}")
        assert eo <= TOL["bf16"] and eS <= TOL["bf16"]
        a = o16.view(torch.int16).cpu().numpy().astype(np.int32)
        b = o32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
        assert np.max(np.abs(a - b)) <= 1
        del o32, o16, S32


def test_fwd_token_major_layout(gla):
    """q, k, v, o as (B, T, H, d) storage viewed as (B, H, T, d)."""
    flush("test_fwd_token_major_layout")
    x = inputs.random_chunk_inputs(140, 2, 4, 300, 96, 192, dtype="bf16", scale=0.3)
    ref_o, ref_S = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    tm = lambda a: dev(np.ascontiguousarray(np.swapaxes(a, 1, 2)), "bf16").transpose(1, 2)
    q, k, v = tm(x["q"]), tm(x["k"]), tm(x["v"])
    o = torch.empty((2, 300, 4, 192), dtype=torch.float32, device="cuda").transpose(1, 2)
    gla.chunk_fwd(q, k, v, dev_f32(x["lam"]), dev_f32(x["S0"]), chunk=128, o=o)
    S = gla.chunk_fwd(q, k, v, dev_f32(x["lam"]), dev_f32(x["S0"]), chunk=128,
                      out_dtype=torch.float32)[1]
    torch.cuda.synchronize()
    assert oracle.rel_err(host(o), ref_o) <= TOL["bf16"]
    assert oracle.rel_err(host(S), ref_S) <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 128])
def test_deterministic(gla, chunk):
    """Two runs of the same forward and backward give identical bits."""
    flush(f"test_deterministic chunk={chunk}")
    x = inputs.make_chunk_inputs("laplace", T=1000)
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
    dO = dev(inputs.normal(2, inputs.TID["dO"], x["v"].shape, 1.0, "bf16"), "bf16")
    a = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
    b = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
    ga = gla.chunk_bwd(q, k, v, lam, dO, S0, None, chunk=chunk, grad_dtype=torch.float32)
    gb = gla.chunk_bwd(q, k, v, lam, dO, S0, None, chunk=chunk, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert all(torch.equal(t, u) for t, u in zip(ga, gb))


# ------------------------------------------------------------------ backward
def run_bwd(gla, x, dtype, chunk):
    q, k, v = dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype)
    dO = dev(x["dO"], dtype)
    lam, S0, dST = dev_f32(x["lam"]), dev_f32(x["S0"]), dev_f32(x["dS_T"])
    g = gla.chunk_bwd(q, k, v, lam, dO, S0, dST, chunk=chunk, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return [host(t) for t in g]


def check_bwd(gla, x, dtype, chunk):
    g = run_bwd(gla, x, dtype, chunk)
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"], x["dS_T"])
    errs = [oracle.rel_err(a, b) for a, b in zip(g, r)]
    flush(f"  bwd chunk={chunk} dtype={dtype} err dq/dk/dv/dS0 = " + " ".join(f"{e:.3e}" for e in errs))
    assert max(errs) <= TOL[dtype]
    return errs


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("T", [1, 40, 97, 256])
def test_bwd_tiny_fp32(gla, chunk, T):
    flush(f"test_bwd_tiny_fp32 chunk={chunk} T={T}")
    x = inputs.random_chunk_inputs(200 + T, 1, 2, T, 16, 32, dtype="f32", dS_T=True)
    check_bwd(gla, x, "f32", chunk)


def test_bwd_tiny_fp32_no_state_grads(gla):
    flush("test_bwd_tiny_fp32_no_state_grads")
    x = inputs.random_chunk_inputs(210, 2, 2, 70, 16, 32, dtype="f32", s0=False, dS_T=False)
    check_bwd(gla, x, "f32", 16)


def test_bwd_training_slice(gla):
    """B=1, T=256 slice of the training recipe (bf16, dk=96, dv=192, chunk 128)."""
    flush("test_bwd_training_slice")
    x = inputs.make_chunk_inputs("training", B=1, T=256, with_grad=True)
    check_bwd(gla, x, "bf16", 128)


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_bwd_bf16_ragged(gla, chunk):
    flush(f"test_bwd_bf16_ragged chunk={chunk}")
    x = inputs.random_chunk_inputs(220, 1, 3, 333, 96, 192, dtype="bf16", dS_T=True, scale=0.5)
    check_bwd(gla, x, "bf16", chunk)


@pytest.mark.parametrize("chunk", [64, 128])
def test_training_full_shape(gla, chunk):
    """The whole training workload (B=8, H=16, T=2048, bf16, dk=96, dv=192) in
    the launches the benchmark times, forward and backward, compared element
    by element with the fp64 oracle over every (b, h) unit: o, S_T, dq, dk,
    dv and dS0 each within the bf16-input gate.  The forward's bf16-stored
    output must be its fp32-stored output rounded to nearest, within one bf16
    ulp, over the whole batch."""
    flush(f"test_training_full_shape chunk={chunk}")
    x = inputs.make_chunk_inputs("training", with_grad=True)
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    lam, S0 = dev_f32(x["lam"]), dev_f32(x["S0"])
    o32, S32 = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
    o16, _ = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = o16.view(torch.int16).cpu().numpy().astype(np.int32)
    bb = o32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
    assert np.max(np.abs(a - bb)) <= 1
    del a, bb, o16
    o, S = host(o32), host(S32)
    del q, k, v, o32, S32
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    _check_per_sequence(["o", "S_T"], [o, S], [ro, rS])
    del o, S, ro, rS
    g = run_bwd(gla, x, "bf16", chunk)
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"])
    _check_per_sequence(["dq", "dk", "dv", "dS0"], g, r)


def _check_per_sequence(names, got, ref):
    """Whole-tensor gate per output, plus the worst sequence printed so a
    failure names the unit range it comes from."""
    for name, a, rr in zip(names, got, ref):
        e = oracle.rel_err(a, rr)
        den = np.max(np.abs(rr))
        worst = max(range(a.shape[0]), key=lambda b: np.max(np.abs(a[b] - rr[b])))
        flush(f"  {name}: err {e:.3e} (worst sequence b={worst})")
        assert e <= TOL["bf16"], (name, worst, e, den)


# ------------------------------------------------------- page decay schedule
# Half-lives geometrically spaced from 1 to 2,048 tokens (the page's section
# "Decay schedule"): head 0 decays by 1/2 per token, so a 128-token chunk
# forms lambda^128 = 2^-128, below the smallest normal fp32.
def test_fwd_page_schedule_full_sequence(gla):
    flush("test_fwd_page_schedule_full_sequence")
    x = inputs.make_chunk_inputs("schedule", B=1)
    assert x["lam"][0] == 0.5
    check_fwd(gla, x, "bf16", 128)


def test_bwd_page_schedule_full_sequence(gla):
    flush("test_bwd_page_schedule_full_sequence")
    x = inputs.make_chunk_inputs("schedule", B=1, with_grad=True)
    x["dS_T"] = inputs.normal(6, inputs.TID["dS_T"], (1, 16, 96, 192), 0.5, "f32")
    check_bwd(gla, x, "bf16", 128)


@pytest.mark.parametrize("chunk", [64, 128])
def test_page_schedule_training_shape(gla, chunk):
    """The whole B=8 schedule workload in the benched launch, every (b, h)
    unit compared with the oracle."""
    flush(f"test_page_schedule_training_shape chunk={chunk}")
    x = inputs.make_chunk_inputs("schedule", with_grad=True)
    o, S = run_fwd(gla, x, "bf16", chunk)
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    _check_per_sequence(["o", "S_T"], [o, S], [ro, rS])
    del o, S, ro, rS
    g = run_bwd(gla, x, "bf16", chunk)
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"])
    _check_per_sequence(["dq", "dk", "dv", "dS0"], g, r)


@pytest.mark.parametrize("chunk", [16, 64])
def test_fwd_bwd_half_decay_fp32(gla, chunk):
    """lambda = 1/2 and the schedule's next heads at fp32 (tolerance 1e-5)."""
    flush(f"test_fwd_bwd_half_decay_fp32 chunk={chunk}")
    lam = inputs.lambda_half_life_schedule(16, 1.0, 2048.0)[:3]
    x = inputs.random_chunk_inputs(440 + chunk, 1, 3, 300, 16, 32, dtype="f32", dS_T=True, lam=lam)
    check_fwd(gla, x, "f32", chunk)
    check_bwd(gla, x, "f32", chunk)


# ------------------------------------------------------------ segment split
# With few (b, h) units the library splits each sequence into segments of
# whole chunks (a state pass, then a full pass whose entry state folds the
# earlier segments' end states).  These cases pick T so that the last segment
# is ragged, segments are dropped by the rounding of the segment length, and
# the reverse-time passes of the backward carry dS0 across segments.
def segments_of(gla, B, H, T, dk, dv, chunk, bwd=False):
    """Segments per (b, h) implied by the workspace query (fp32 end states
    and dv / 16 8-byte flags per state)."""
    lib, d = gla.load_library(), ctypes.byref(gla.GlaDims(B, H, T, dk, dv, chunk))
    nws = lib.gla_chunk_bwd_workspace(d) if bwd else lib.gla_chunk_fwd_workspace(d)
    per = dk * dv * 4 + -(-dv // 16) * 8
    if not bwd:  # the backward's region also holds a second pass's flags
        assert nws % (B * H * per) == 0
    return nws // (B * H * per)


@pytest.mark.parametrize("T,chunk", [(1000, 32), (1000, 128), (9 * 64 - 5, 64), (4 * 16, 16)])
def test_fwd_segments_bf16(gla, T, chunk):
    flush(f"test_fwd_segments_bf16 T={T} chunk={chunk}")
    x = inputs.random_chunk_inputs(400 + T, 1, 2, T, 96, 192, dtype="bf16", scale=0.3)
    assert segments_of(gla, 1, 2, T, 96, 192, chunk) >= 2
    check_fwd(gla, x, "bf16", chunk)


@pytest.mark.parametrize("lam", [0.0, 1.0, 0.999])
def test_fwd_segments_lambda_edges_fp32(gla, lam):
    flush(f"test_fwd_segments_lambda_edges_fp32 lam={lam}")
    x = inputs.random_chunk_inputs(410, 1, 1, 1500, 16, 32, dtype="f32", lam=np.full(1, lam))
    assert segments_of(gla, 1, 1, 1500, 16, 32, 16) == 47
    check_fwd(gla, x, "f32", 16)


def test_fwd_segments_long_decay(gla):
    """T=16,384 at B=1, slowest heads of the long-context decay profile: 64
    segments whose entry states are sums over up to 63 earlier ones."""
    flush("test_fwd_segments_long_decay")
    x = inputs.make_chunk_inputs("long", T=16384)
    for key in ("q", "k", "v"):
        x[key] = x[key][:, -2:]
    x["lam"] = x["lam"][-2:]
    x["S0"] = inputs.normal(411, inputs.TID["S"], (1, 2, 96, 192), 0.01, "f32")
    assert segments_of(gla, 1, 2, 16384, 96, 192, 128) == 64
    check_fwd(gla, x, "bf16", 128)


@pytest.mark.parametrize("shape", [(1, 2, 1000, 96, 192, "bf16", 64), (1, 1, 1500, 16, 32, "f32", 16)])
def test_fwd_segments_without_waiting(gla, shape):
    """The forward publishes each segment's end state within its one launch;
    with no wait at all, a workgroup forms every earlier state it finds
    unpublished itself.  The arithmetic is the same either way, so the
    outputs equal those of the default wait bit for bit (and pass the gate)."""
    B, H, T, dk, dv, dtype, chunk = shape
    flush(f"test_fwd_segments_without_waiting {shape}")
    x = inputs.random_chunk_inputs(450 + T, B, H, T, dk, dv, dtype=dtype, scale=0.3)
    assert segments_of(gla, B, H, T, dk, dv, chunk) >= 2
    base = run_fwd(gla, x, dtype, chunk)
    try:
        gla.set_segment_wait(0)
        forced = run_fwd(gla, x, dtype, chunk)
        forced2 = run_fwd(gla, x, dtype, chunk)
    finally:
        gla.set_segment_wait(-1)
    for got in (forced, forced2):
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
    assert oracle.rel_err(base[0], ro) <= TOL[dtype] and oracle.rel_err(base[1], rS) <= TOL[dtype]


@pytest.mark.parametrize("B,H,T", [(4, 25, 640 - 3), (1, 127, 300)])
def test_fwd_segments_more_workgroups_than_cus(gla, B, H, T):
    """Two segments per (b, h) with 100 and 127 heads: 400 and 508 workgroups
    of the one-launch forward, more than one per compute unit, so some wait
    on earlier segments that are resident while others are still queued."""
    flush(f"test_fwd_segments_more_workgroups_than_cus B={B} H={H} T={T}")
    x = inputs.random_chunk_inputs(480 + H, B, H, T, 96, 192, dtype="bf16", scale=0.3)
    assert segments_of(gla, B, H, T, 96, 192, 64) == 2
    check_fwd(gla, x, "bf16", 64)


def test_fwd_segments_token_major_no_s0(gla):
    """The one-launch segment split on token-major views (q, k, v, o stored
    (B, T, H, d)) with no initial state and a ragged last chunk."""
    flush("test_fwd_segments_token_major_no_s0")
    B, H, T = 1, 4, 2000
    x = inputs.random_chunk_inputs(510, B, H, T, 96, 192, dtype="bf16", s0=False, scale=0.3)
    assert segments_of(gla, B, H, T, 96, 192, 64) >= 8
    ref_o, ref_S = oracle.fwd(x["q"], x["k"], x["v"], x["lam"], None)
    tm = lambda a: dev(np.ascontiguousarray(np.swapaxes(a, 1, 2)), "bf16").transpose(1, 2)
    q, k, v = tm(x["q"]), tm(x["k"]), tm(x["v"])
    o = torch.empty((B, T, H, 192), dtype=torch.float32, device="cuda").transpose(1, 2)
    _, S = gla.chunk_fwd(q, k, v, dev_f32(x["lam"]), None, chunk=64, o=o)
    torch.cuda.synchronize()
    assert oracle.rel_err(host(o), ref_o) <= TOL["bf16"]
    assert oracle.rel_err(host(S), ref_S) <= TOL["bf16"]


def test_fwd_segments_graph_replays(gla):
    """A captured segmented forward replays with the tag of its capture: each
    replay, with new inputs copied in and eager calls in between, must equal
    the eager result bit for bit (no replay may take a flag left by the one
    before it)."""
    flush("test_fwd_segments_graph_replays")
    B, H, T, chunk = 1, 2, 777, 64
    assert segments_of(gla, B, H, T, 96, 192, chunk) >= 2
    sets = [inputs.random_chunk_inputs(460 + i, B, H, T, 96, 192, dtype="bf16", scale=0.3) for i in range(3)]
    q, k, v = (dev(sets[0][n], "bf16") for n in ("q", "k", "v"))
    lam, S0 = dev_f32(sets[0]["lam"]), dev_f32(sets[0]["S0"])
    o = torch.empty((B, H, T, 192), dtype=torch.float32, device="cuda")
    S = torch.empty((B, H, 96, 192), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, o=o, S_T=S)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, o=o, S_T=S)
    torch.cuda.synchronize()
    for i in range(6):
        x = sets[i % 3]
        for name, t in (("q", q), ("k", k), ("v", v)):
            t.copy_(dev(x[name], "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_S = host(o), host(S)
        eo, eS = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(got_o, host(eo)) and np.array_equal(got_S, host(eS)), f"replay {i}"
    # the decay and entry state stay those of the first set
    ro, rS = oracle.fwd(x["q"], x["k"], x["v"], sets[0]["lam"], sets[0]["S0"])
    assert oracle.rel_err(got_o, ro) <= TOL["bf16"] and oracle.rel_err(got_S, rS) <= TOL["bf16"]


def test_segments_on_two_streams(gla):
    """Segmented forwards and backwards of the Laplace-layer shape enqueued on
    two streams at once (each call with its own workspace): the one-launch
    kernels then share the compute units, so a workgroup may find an earlier
    segment's producer not yet resident and form that state itself.  Every
    result must equal the same call run alone, bit for bit."""
    flush("test_segments_on_two_streams")
    B, H, T, chunk = 1, 16, 2048, 64
    assert segments_of(gla, B, H, T, 96, 192, chunk) >= 2
    sets = [inputs.random_chunk_inputs(530 + i, B, H, T, 96, 192, dtype="bf16", dS_T=True, scale=0.3)
            for i in range(2)]
    args = []
    for x in sets:
        q, k, v, dO = (dev(x[n], "bf16") for n in ("q", "k", "v", "dO"))
        args.append((q, k, v, dev_f32(x["lam"]), dO, dev_f32(x["S0"]), dev_f32(x["dS_T"])))

    def run(a):
        q, k, v, lam, dO, S0, dST = a
        o, S = gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, out_dtype=torch.float32)
        g = gla.chunk_bwd(q, k, v, lam, dO, S0, dST, chunk=chunk, grad_dtype=torch.float32)
        return (o, S) + tuple(g)

    alone = []
    for a in args:
        alone.append([host(t) for t in run(a)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        outs = [None, None]
        for i, s_ in enumerate(streams):
            with torch.cuda.stream(s_):
                outs[i] = run(args[i])
        torch.cuda.synchronize()
        for i in range(2):
            for j, t in enumerate(outs[i]):
                assert np.array_equal(host(t), alone[i][j]), f"rep {rep} stream {i} output {j}"
    ro, rS = oracle.fwd(sets[1]["q"], sets[1]["k"], sets[1]["v"], sets[1]["lam"], sets[1]["S0"])
    assert oracle.rel_err(alone[1][0], ro) <= TOL["bf16"] and oracle.rel_err(alone[1][1], rS) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,chunk,T", [("bf16", 16, 8192 + 37), ("f32", 32, 16384 + 5), ("bf16", 64, 32768 - 11)])
def test_wide_tiles_fwd_bwd(gla, dtype, chunk, T):
    """Few (b, h) units with at least 8 chunks per segment: the (96, 192)
    passes run all 192 columns of a head in one 12-wave workgroup (the
    forward, and the backward's dv pass).  Ragged T, up to 64 segments,
    fp32 up to its 32-token limit for that tiling."""
    flush(f"test_wide_tiles_fwd_bwd {dtype} chunk={chunk} T={T}")
    x = inputs.random_chunk_inputs(470 + chunk, 1, 2, T, 96, 192, dtype=dtype, dS_T=True, scale=0.3)
    n, nchunks = segments_of(gla, 1, 2, T, 96, 192, chunk), -(-T // chunk)
    assert 2 <= n <= 64 and nchunks >= 8 * n
    check_fwd(gla, x, dtype, chunk)
    check_bwd(gla, x, dtype, chunk)


@pytest.mark.parametrize("shape", [(1, 2, 1000, 96, 192, "bf16", 64), (1, 1, 1001, 16, 32, "f32", 16)])
def test_bwd_segments_without_waiting(gla, shape):
    """The backward's segmented passes (the paired dq/dk launch and dv) also
    run in one launch each; with no wait at all every workgroup forms the
    earlier end states itself: the same bits as the default wait."""
    B, H, T, dk, dv, dtype, chunk = shape
    flush(f"test_bwd_segments_without_waiting {shape}")
    x = inputs.random_chunk_inputs(490 + T, B, H, T, dk, dv, dtype=dtype, dS_T=True, scale=0.3)
    assert segments_of(gla, B, H, T, dk, dv, chunk, bwd=True) >= 2
    base = run_bwd(gla, x, dtype, chunk)
    try:
        gla.set_segment_wait(0)
        forced = run_bwd(gla, x, dtype, chunk)
    finally:
        gla.set_segment_wait(-1)
    for a, b in zip(base, forced):
        assert np.array_equal(a, b)
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"], x["dS_T"])
    assert max(oracle.rel_err(a, b) for a, b in zip(base, r)) <= TOL[dtype]


def test_bwd_segments_token_major(gla):
    """The segmented backward with every (B, H, T, d) operand and gradient a
    token-major view ((B, T, H, d) storage) and a ragged last chunk."""
    flush("test_bwd_segments_token_major")
    B, H, T = 1, 4, 2000
    x = inputs.random_chunk_inputs(520, B, H, T, 96, 192, dtype="bf16", dS_T=True, scale=0.3)
    assert segments_of(gla, B, H, T, 96, 192, 64, bwd=True) >= 8
    r = oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"], x["dS_T"])
    tm = lambda a: dev(np.ascontiguousarray(np.swapaxes(a, 1, 2)), "bf16").transpose(1, 2)
    out = lambda d: torch.empty((B, T, H, d), dtype=torch.float32, device="cuda").transpose(1, 2)
    dq, dk, dv = out(96), out(96), out(192)
    g = gla.chunk_bwd(tm(x["q"]), tm(x["k"]), tm(x["v"]), dev_f32(x["lam"]), tm(x["dO"]),
                      dev_f32(x["S0"]), dev_f32(x["dS_T"]), chunk=64, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    errs = [oracle.rel_err(host(a), b) for a, b in zip(g, r)]
    flush("  err dq/dk/dv/dS0 = " + " ".join(f"{e:.3e}" for e in errs))
    assert max(errs) <= TOL["bf16"]


def test_bwd_segments_graph_replays(gla):
    """A captured segmented backward (paired dq/dk launch and dv, one launch
    each) replays with the tags of its capture: each replay, with new inputs
    copied in and eager calls in between, equals the eager result bit for
    bit."""
    flush("test_bwd_segments_graph_replays")
    B, H, T, chunk = 1, 2, 900, 64
    assert segments_of(gla, B, H, T, 96, 192, chunk, bwd=True) >= 2
    sets = [inputs.random_chunk_inputs(500 + i, B, H, T, 96, 192, dtype="bf16", dS_T=True, scale=0.3)
            for i in range(3)]
    q, k, v, dO = (dev(sets[0][n], "bf16") for n in ("q", "k", "v", "dO"))
    lam, S0, dST = dev_f32(sets[0]["lam"]), dev_f32(sets[0]["S0"]), dev_f32(sets[0]["dS_T"])
    outs = [torch.empty((B, H, T, 96), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, T, 96), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, T, 192), dtype=torch.float32, device="cuda"),
            torch.empty((B, H, 96, 192), dtype=torch.float32, device="cuda")]
    call = lambda: gla.chunk_bwd(q, k, v, lam, dO, S0, dST, chunk=chunk, dq=outs[0], dk=outs[1], dv=outs[2],
                                 dS0=outs[3])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(6):
        x = sets[i % 3]
        for name, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
            t.copy_(dev(x[name], "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in outs]
        eager = gla.chunk_bwd(q, k, v, lam, dO, S0, dST, chunk=chunk, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        for a, b in zip(got, eager):
            assert np.array_equal(a, host(b)), f"replay {i}"
    # the decay, S0 and dS_T stay those of the first set
    r = oracle.bwd(x["q"], x["k"], x["v"], sets[0]["lam"], x["dO"], sets[0]["S0"], sets[0]["dS_T"])
    assert max(oracle.rel_err(a, b) for a, b in zip(got, r)) <= TOL["bf16"]


@pytest.mark.parametrize("T,chunk", [(777, 64), (1000, 128), (300, 32)])
def test_bwd_segments_bf16(gla, T, chunk):
    flush(f"test_bwd_segments_bf16 T={T} chunk={chunk}")
    x = inputs.random_chunk_inputs(420 + T, 1, 2, T, 96, 192, dtype="bf16", dS_T=True, scale=0.5)
    assert segments_of(gla, 1, 2, T, 96, 192, chunk, bwd=True) >= 2
    check_bwd(gla, x, "bf16", chunk)


def test_bwd_segments_fp32(gla):
    flush("test_bwd_segments_fp32")
    x = inputs.random_chunk_inputs(430, 1, 1, 1001, 16, 32, dtype="f32", dS_T=True)
    assert segments_of(gla, 1, 1, 1001, 16, 32, 16, bwd=True) >= 21
    check_bwd(gla, x, "f32", 16)


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dims", [(16, 32, "f32"), (96, 192, "bf16"), (96, 192, "f32")])
def test_decode_steps_vs_oracle(gla, dims):
    dk, dv, dtype = dims
    flush(f"test_decode_steps_vs_oracle dk={dk} dv={dv} {dtype}")
    N, H, steps = 37, 3, 5
    x = inputs.random_chunk_inputs(300 + dk, N, H, steps, dk, dv, dtype=dtype, scale=1.0)
    S_host = inputs.normal(300 + dk, inputs.TID["S"], (N, H, dk, dv), 0.01, "f32")
    S = dev_f32(S_host)
    lam = dev_f32(x["lam"])
    Sref = S_host.copy()
    for t in range(steps):
        q, k, v = (dev(np.ascontiguousarray(x[n][:, :, t]), dtype) for n in ("q", "k", "v"))
        o = gla.decode_step_(q, k, v, lam, S, out_dtype=torch.float32)
        ro, Sref = oracle.decode_step(x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t], x["lam"], Sref)
        torch.cuda.synchronize()
        assert oracle.rel_err(host(o), ro) <= 1e-5
    assert oracle.rel_err(host(S), Sref) <= 1e-5


def test_decode_page_schedule(gla):
    """Decode steps of all 16 heads of the page's decay schedule (lambda_0 = 1/2)."""
    flush("test_decode_page_schedule")
    N, H, dk, dv, steps = 21, 16, 96, 192, 6
    lam_h = inputs.lambda_half_life_schedule(H, 1.0, 2048.0)
    x = inputs.random_chunk_inputs(450, N, H, steps, dk, dv, dtype="bf16", scale=1.0, lam=lam_h)
    S_host = inputs.normal(450, inputs.TID["S"], (N, H, dk, dv), 0.01, "f32")
    S, lam, Sref = dev_f32(S_host), dev_f32(x["lam"]), S_host.copy()
    for t in range(steps):
        q, k, v = (dev(np.ascontiguousarray(x[n][:, :, t]), "bf16") for n in ("q", "k", "v"))
        o = gla.decode_step_(q, k, v, lam, S, out_dtype=torch.float32)
        ro, Sref = oracle.decode_step(x["q"][:, :, t], x["k"][:, :, t], x["v"][:, :, t], x["lam"], Sref)
        torch.cuda.synchronize()
        assert oracle.rel_err(host(o), ro) <= 1e-5
    assert oracle.rel_err(host(S), Sref) <= 1e-5


def test_decode_strided_page_pool(gla):
    """States inside a per-sequence page holding several layers (S_stride_n >
    H*dk*dv); only the addressed layer changes."""
    flush("test_decode_strided_page_pool")
    N, Lyr, H, dk, dv = 9, 3, 2, 96, 192
    pool_host = inputs.normal(310, inputs.TID["S"], (N, Lyr, H, dk, dv), 0.01, "f32")
    pool = dev_f32(pool_host)
    x = inputs.random_chunk_inputs(311, N, H, 1, dk, dv, dtype="bf16", scale=1.0)
    q, k, v = (dev(np.ascontiguousarray(x[n][:, :, 0]), "bf16") for n in ("q", "k", "v"))
    layer = 1
    o = gla.decode_step_(q, k, v, dev_f32(x["lam"]), pool[:, layer], out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, Sref = oracle.decode_step(x["q"][:, :, 0], x["k"][:, :, 0], x["v"][:, :, 0], x["lam"],
                                  pool_host[:, layer])
    got = host(pool)
    assert oracle.rel_err(host(o), ro) <= 1e-5
    assert oracle.rel_err(got[:, layer], Sref) <= 1e-5
    assert np.array_equal(got[:, 0], pool_host[:, 0]) and np.array_equal(got[:, 2], pool_host[:, 2])


def test_decode_equals_chunked_long_context(gla):
    """Long-context recipe (H=16, bf16, lambda in [0.95, 0.9999]): the final
    state of gla_chunk_fwd equals T gla_decode_step calls and the oracle.
    T is 8192 here; the full 65,536 runs in the bench-shaped test below."""
    flush("test_decode_equals_chunked_long_context")
    x = inputs.make_chunk_inputs("long", T=8192)
    _check_decode_equivalence(gla, x)


def _check_decode_equivalence(gla, x):
    T = x["q"].shape[2]
    q, k, v = dev(x["q"], "bf16"), dev(x["k"], "bf16"), dev(x["v"], "bf16")
    lam = dev_f32(x["lam"])
    _, S_chunk = gla.chunk_fwd(q, k, v, lam, None, chunk=128, out_dtype=torch.float32)
    H, dk, dv = q.shape[1], q.shape[3], v.shape[3]
    S = torch.zeros((1, H, dk, dv), dtype=torch.float32, device="cuda")
    o = torch.empty((1, H, dv), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        gla.decode_step_(q[:, :, t], k[:, :, t], v[:, :, t], lam, S, o=o)
    torch.cuda.synchronize()
    _, rS = oracle.fwd(x["q"], x["k"], x["v"], x["lam"])
    e_chunk, e_dec = oracle.rel_err(host(S_chunk), rS), oracle.rel_err(host(S), rS)
    flush(f"  T={T} err chunked={e_chunk:.3e} decode={e_dec:.3e}")
    assert e_chunk <= TOL["bf16"] and e_dec <= TOL["bf16"]
    assert oracle.rel_err(host(S_chunk), host(S)) <= TOL["bf16"]


def test_decode_equals_chunked_long_context_full(gla):
    flush("test_decode_equals_chunked_long_context_full T=65536")
    x = inputs.make_chunk_inputs("long")
    _check_decode_equivalence(gla, x)


def test_decode_full_workload_subset(gla):
    """The batched-decode workload as the benchmark runs it: a (24, 1280, 16,
    96, 192) fp32 state pool (36 GB), 64 steps, each step one call per layer
    slab in layer order, q/k/v strided views of one packed bf16 block per
    (step, layer).  Layers 0 and 23 store o in fp32; for sequences {0, 1,
    639, 1279} x all 16 heads, every step's o and both layers' final states
    are compared with the fp64 oracle run over the same 64 steps (sequences
    are independent, so the subset is exact).  On the first and the last step
    layer 0 is also run on a copy of its slab with bf16 output: the states
    must agree bit for bit and the bf16 output must be the fp32 output
    rounded to nearest (within one bf16 ulp).  A layer outside the subset is
    checked to have been updated."""
    flush("test_decode_full_workload_subset N=1280 layers=24 H=16 steps=64")
    Lyr, N, H, dk, dv, steps = 24, 1280, 16, 96, 192, 64
    seqs = [0, 1, 639, 1279]
    layers = (0, Lyr - 1)
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_101)
    S = torch.empty((Lyr, N, H, dk, dv), dtype=torch.float32, device="cuda")
    S.normal_(0.0, 0.01, generator=g)
    lam_h = np.asarray(inputs.lambda_log_spaced(H, 0.95, 0.9999), dtype=np.float32)
    lam = dev_f32(lam_h)
    sel = torch.tensor(seqs, device="cuda")
    ref_S = {ly: host(S[ly].index_select(0, sel)) for ly in layers}
    mid_before = host(S[Lyr // 2, :2])
    o16 = torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((N, H, dv), dtype=torch.float32, device="cuda")
    err_o = {ly: 0.0 for ly in layers}
    for st in range(steps):
        for ly in range(Lyr):
            blk = torch.randn((N, H, dk + dk + dv), generator=g, device="cuda").to(torch.bfloat16)
            qv, kv, vv = blk[..., :dk], blk[..., dk:2 * dk], blk[..., 2 * dk:]
            if ly not in layers:
                gla.decode_step_(qv, kv, vv, lam, S[ly], o=o16)
                continue
            S_copy = S[ly].clone() if (ly == 0 and st in (0, steps - 1)) else None
            gla.decode_step_(qv, kv, vv, lam, S[ly], o=o32)
            if S_copy is not None:
                gla.decode_step_(qv, kv, vv, lam, S_copy, o=o16)
                torch.cuda.synchronize()
                assert torch.equal(S[ly], S_copy), (st, ly)
                a = o16.view(torch.int16).cpu().numpy().astype(np.int32)
                b = o32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
                assert np.max(np.abs(a - b)) <= 1, (st, ly)
                del S_copy
            bh = host(blk.index_select(0, sel))
            ro, ref_S[ly] = oracle.decode_step(bh[..., :dk], bh[..., dk:2 * dk], bh[..., 2 * dk:], lam_h, ref_S[ly])
            err_o[ly] = max(err_o[ly], oracle.rel_err(host(o32.index_select(0, sel)), ro))
        if st % 16 == 15:
            flush(f"  step {st + 1}: max o err layer0={err_o[0]:.2e} layer23={err_o[Lyr - 1]:.2e}")
    for ly in layers:
        e = oracle.rel_err(host(S[ly].index_select(0, sel)), ref_S[ly])
        flush(f"  layer {ly}: o err {err_o[ly]:.3e}, final state err {e:.3e}")
        assert err_o[ly] <= 1e-5 and e <= 1e-5, (ly, err_o[ly], e)
    assert not np.array_equal(host(S[Lyr // 2, :2]), mid_before)


def test_fwd_bwd_max_units(gla):
    """The largest launch the ABI accepts: B*H = 2^21 (b, h) units, here
    B = 131,072 sequences of T = 2 tokens (bf16, dk=96, dv=192, chunk 64, no
    state tensors).  The forward launches 2^22 workgroups and the backward's
    paired launch 2^22 as well (1.6e9 work-items each); sampled heads,
    including the last one, match the oracle."""
    flush("test_fwd_bwd_max_units B=131072 H=16 T=2")
    B, H, T, dk, dv = 1 << 17, 16, 2, 96, 192
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_202)
    q = torch.randn((B, H, T, dk), generator=g, device="cuda").to(torch.bfloat16)
    k = (torch.randn((B, H, T, dk), generator=g, device="cuda") / dk ** 0.5).to(torch.bfloat16)
    v = torch.randn((B, H, T, dv), generator=g, device="cuda").to(torch.bfloat16)
    dO = torch.randn((B, H, T, dv), generator=g, device="cuda").to(torch.bfloat16)
    lam_h = np.asarray(inputs.lambda_log_spaced(H, 0.9, 0.999), dtype=np.float32)
    lam = dev_f32(lam_h)
    o, _ = gla.chunk_fwd(q, k, v, lam, None, chunk=64, out_dtype=torch.float32, return_state=False)
    dq, dk_, dv_, _ = gla.chunk_bwd(q, k, v, lam, dO, None, None, chunk=64, grad_dtype=torch.float32,
                                    need_dS0=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    samples = [(B - 1, H - 1), (0, 0)] + [(int(b), int(h)) for b, h in
                                           zip(rng.integers(0, B, 6), rng.integers(0, H, 6))]
    for b, h in samples:
        sl = lambda t: host(t[b:b + 1, h:h + 1])
        qs, ks, vs, dOs = sl(q), sl(k), sl(v), sl(dO)
        lh = lam_h[h:h + 1]
        ro, _ = oracle.fwd(qs, ks, vs, lh)
        rdq, rdk, rdv, _ = oracle.bwd(qs, ks, vs, lh, dOs)
        assert oracle.rel_err(sl(o), ro) <= TOL["bf16"], (b, h)
        for got, ref in ((dq, rdq), (dk_, rdk), (dv_, rdv)):
            assert oracle.rel_err(sl(got), ref) <= TOL["bf16"], (b, h)

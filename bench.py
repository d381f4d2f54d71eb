"""Benchmark of the Simple GLA hot path on one MI355X.

A step is one chunked forward + backward (gla_chunk_fwd + gla_chunk_bwd) on
the training-shape workload: B=8, H=16, T=2048, dk=96, dv=192, bf16
q/k/v/dO, fp32 states, seeded synthetic inputs resident in HBM, 64-token
chunks (the same step at the pages' 128-token chunk is reported under
"extra").  The JSON line's value is whole-step tokens/s (B*T per step).  The
same run also measures the batched decode workload (1,280 sequences x 24
layers x 16 heads of fp32 96x192 states, 64 steps) and reports it under
"decode", and times the fp64 CPU oracle on a bounded sample under
"cpu_baseline" (and beside the decode, convolution, packed-prefill and
fused-epilogue rows under their "cpu_oracle" keys).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-decode] [--no-cpu]
                    [--decode-steps N] [--calibrate-copy]
"""
import argparse
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

METRIC = "GLA fwd+bwd tokens/s (H=16,dk=96,dv=192) + decode tok/s, % roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA

# Chunk length of every timed call.  The output does not depend on it beyond
# rounding (the tests check 16, 32, 64 and 128 against the oracle); the pages'
# 128-token chunk matched Trainium's 128 SBUF partitions, while on gfx950 the
# 64-token chunk runs faster (fewer causal-tile flops per token; at 128 the
# library tiles the backward's transposed passes at 64 tokens anyway).  The
# 128-token chunk is timed as well and reported under "extra".
C = 64
C_PAGE = 128
DK, DV = 96, 192
FWD_BYTES = 2 * (DK + DK + DV + DV)  # q, k, v in; o out (bf16)
BWD_BYTES = 2 * (DK + DK + DV + DV) + 2 * (DK + DK + DV)  # q, k, v, dO in; dq, dk, dv out
STATE_BYTES = DK * DV * 4
# algorithmic work per token-head (one token of one head) at chunk c
def FWD_FLOPS(c):
    return 2 * c * (DK + DV) + 4 * DK * DV


def BWD_FLOPS(c):
    return 2 * c * (3 * DK + 2 * DV) + 8 * DK * DV


DEC_BYTES = 2 * STATE_BYTES + 2 * (DK + DK + DV) + 2 * DV + 4  # state r+w, q k v, o, lambda


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def event_time_ms(fn, n, stream):
    """Average milliseconds of fn() over n calls, timed with HIP events on
    the stream the library launches on."""
    import torch

    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(n):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / n


def call_stats(fn, stream, n=20):
    """Per-call figures after warm-up: the median and minimum of n calls
    timed one by one with HIP events while the calls run back to back, and
    the median host wall time of an isolated call (launch, run, synchronize)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in ev:
        s.record(stream)
        fn()
        e.record(stream)
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in ev)
    lat = []
    for _ in range(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t0) * 1e3)
    lat.sort()
    return dict(ms_median=per[n // 2], ms_min=per[0], ms_single_call_median=lat[n // 2])


def warm_up(fn, min_seconds=0.05):
    """Run fn until min_seconds of wall time have passed.  After the host has
    generated a workload's inputs the GPU has been idle, and its clock takes
    about 30 ms of sustained load to return to speed (measured: the training
    forward runs 112-129 us for its first ~100 calls after a pause, then 99
    us), so timing right away reads low."""
    import torch

    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= min_seconds:
            return


def bench_train(gla, inputs, steps, warmup, chunk=C):
    import numpy as np
    import torch

    x = inputs.make_chunk_inputs("training", with_grad=True)
    cfg = x["cfg"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v, dO = (d(x[n]).to(torch.bfloat16) for n in ("q", "k", "v", "dO"))
    lam, S0 = d(x["lam"]), d(x["S0"])
    o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv, dS0 = torch.empty_like(v), torch.empty_like(S0)
    stream = torch.cuda.current_stream()

    def fwd():
        gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, o=o, S_T=S_T)

    def bwd():
        gla.chunk_bwd(q, k, v, lam, dO, S0, None, chunk=chunk, dq=dq, dk=dk, dv=dv, dS0=dS0)

    def step():
        fwd()
        bwd()

    # the GPU clock first has to come back to speed after input generation
    # (warm_up), then the requested number of untimed steps
    warm_up(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    # per-launch durations with events (the forward is one kernel launch; the
    # backward one call of three passes), averaged over many calls
    n = max(10, steps)
    ms_fwd = event_time_ms(fwd, n, stream)
    ms_bwd = event_time_ms(bwd, n, stream)
    units = B * H * T
    res = dict(
        B=B, H=H, T=T, ms_step=ms_step, ms_fwd=ms_fwd, ms_bwd=ms_bwd,
        tokens_per_s=B * T / (ms_step / 1e3),
        fwd_bytes=units * FWD_BYTES + 2 * B * H * STATE_BYTES,
        bwd_bytes=units * BWD_BYTES + 2 * B * H * STATE_BYTES,
        fwd_flops=units * FWD_FLOPS(chunk), bwd_flops=units * BWD_FLOPS(chunk), chunk=chunk,
        lam=[float(t) for t in x["lam"]],
    )
    return res


def bench_fwd_bwd_events(gla, inputs, name, reps, chunk=C):
    """Event-timed forward and backward calls of a chunked workload (the
    page's decay-schedule variant of the training step, the step at the
    pages' 128-token chunk, and the Laplace layer's segmented passes)."""
    import numpy as np
    import torch

    x = inputs.make_chunk_inputs(name, with_grad=True)
    cfg = x["cfg"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v, dO = (d(x[n]).to(torch.bfloat16) for n in ("q", "k", "v", "dO"))
    lam, S0 = d(x["lam"]), d(x["S0"])
    o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")
    dq, dk, dv, dS0 = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(S0)
    fwd = lambda: gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, o=o, S_T=S_T)
    bwd = lambda: gla.chunk_bwd(q, k, v, lam, dO, S0, None, chunk=chunk, dq=dq, dk=dk, dv=dv, dS0=dS0)
    warm_up(lambda: (fwd(), bwd()))
    stream = torch.cuda.current_stream()
    ms_fwd = event_time_ms(fwd, reps, stream)
    ms_bwd = event_time_ms(bwd, reps, stream)
    units = B * H * T
    return dict(workload=name, B=B, H=H, T=T, chunk=chunk, ms_fwd=ms_fwd, ms_bwd=ms_bwd,
                tokens_per_s=B * T / ((ms_fwd + ms_bwd) / 1e3),
                fwd_bytes=units * FWD_BYTES + 2 * B * H * STATE_BYTES,
                bwd_bytes=units * BWD_BYTES + 2 * B * H * STATE_BYTES,
                fwd_flops=units * FWD_FLOPS(chunk), bwd_flops=units * BWD_FLOPS(chunk),
                lam=[float(t) for t in x["lam"]])


def bench_fwd_only(gla, inputs, name, reps, chunk=C):
    import numpy as np
    import torch

    x = inputs.make_chunk_inputs(name)
    cfg = x["cfg"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v = (d(x[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    lam = d(x["lam"])
    S0 = d(x["S0"]) if x["S0"] is not None else None
    o = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")
    fn = lambda: gla.chunk_fwd(q, k, v, lam, S0, chunk=chunk, o=o, S_T=S_T)
    warm_up(fn)
    ms = event_time_ms(fn, reps, torch.cuda.current_stream())
    units = B * H * T
    nbytes = units * FWD_BYTES + (2 if S0 is not None else 1) * B * H * STATE_BYTES
    return dict(workload=name, B=B, H=H, T=T, chunk=chunk, ms=ms, tokens_per_s=B * T / (ms / 1e3),
                gbs=nbytes / (ms / 1e3) / 1e9, hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                per_call=call_stats(fn, torch.cuda.current_stream()))


def bench_decode(gla, inputs, steps_override=None):
    """1,280 sequences x 24 layers x 16 heads, fp32 states, 64 steps; each
    step runs the 24 layer slabs in order.  Inputs for every (step, layer)
    are drawn on the device from a seeded generator before timing."""
    import torch

    c = inputs.CONFIGS["decode"]
    N, Lyr, H, steps = c["N"], c["L"], c["H"], steps_override or c["steps"]
    lam = torch.tensor(inputs.lambda_log_spaced(H, 0.95, 0.9999), dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(5_000_001)
    S = torch.empty((Lyr, N, H, DK, DV), dtype=torch.float32, device="cuda")
    S.normal_(0.0, 0.01, generator=g)
    qkv = torch.empty((steps, Lyr, N, H, DK + DK + DV), dtype=torch.bfloat16, device="cuda")
    for st in range(steps):
        qkv[st].copy_(torch.randn((Lyr, N, H, DK + DK + DV), generator=g, device="cuda"))
    o = torch.empty((N, H, DV), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def run(nsteps):
        for st in range(nsteps):
            for layer in range(Lyr):
                blk = qkv[st, layer]
                gla.decode_step_(blk[..., :DK], blk[..., DK:2 * DK], blk[..., 2 * DK:], lam, S[layer], o=o)

    # warm up on a scratch copy of one slab so the timed steps start from the seeded states
    tmp = S[0].clone()
    blk = qkv[0, 0]
    warm_up(lambda: gla.decode_step_(blk[..., :DK], blk[..., DK:2 * DK], blk[..., 2 * DK:], lam, tmp, o=o))
    del tmp
    stream = torch.cuda.current_stream()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    run(steps)
    e.record(stream)
    e.synchronize()
    ms = s.elapsed_time(e)
    calls = steps * Lyr
    nbytes = calls * N * H * DEC_BYTES
    per_call_ms = ms / calls
    # the same layer call with the output epilogue fused (gate stream g bf16)
    gz = torch.randn((N, H, DV), generator=g, device="cuda").to(torch.bfloat16)
    aug = torch.zeros((H, DK), dtype=torch.float32, device="cuda")
    gam = torch.ones((H, DV), dtype=torch.float32, device="cuda")
    blk = qkv[0, 0]
    lib = gla.load_library()
    ws = torch.empty(lib.gla_decode_step_fused_workspace(N, H, DK, DV), dtype=torch.uint8, device="cuda")
    fused = lambda: gla.decode_step_fused_(blk[..., :DK], blk[..., DK:2 * DK], blk[..., 2 * DK:], lam, S[0], gz,
                                           aug, gam, 1e-6, y=o, ws=ws)
    warm_up(fused)
    fused_ms = event_time_ms(fused, 20, stream)
    # the same without a workspace (one workgroup per state, row normalised in the kernel)
    fused1 = lambda: gla.decode_step_fused_(blk[..., :DK], blk[..., DK:2 * DK], blk[..., 2 * DK:], lam, S[0], gz,
                                            aug, gam, 1e-6, y=o, use_workspace=False)
    warm_up(fused1)
    fused1_ms = event_time_ms(fused1, 20, stream)
    # per-call samples: one step's 24 layer calls, each timed with its own events
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(Lyr)]
    for layer, (s1, e1) in enumerate(ev):
        blk = qkv[0, layer]
        s1.record(stream)
        gla.decode_step_(blk[..., :DK], blk[..., DK:2 * DK], blk[..., 2 * DK:], lam, S[layer], o=o)
        e1.record(stream)
    torch.cuda.synchronize()
    per = sorted(s1.elapsed_time(e1) for s1, e1 in ev)
    # device stream ceiling for the same state traffic: an in-place scale of
    # one layer's states (read and write every state once, as a decode call does)
    scale = lambda: S[0].mul_(0.9999)
    warm_up(scale)
    ms_scale = event_time_ms(scale, 20, stream)
    scale_gbs = S[0].numel() * 8 / (ms_scale / 1e3) / 1e9
    return dict(
        workload="decode: 1280 seqs x 24 layers x H=16, fp32 96x192 states, 64 steps, bf16 q/k/v",
        N=N, layers=Lyr, H=H, steps=steps, ms_total=ms, ms_per_layer_call=per_call_ms,
        tokens_per_s=N * steps / (ms / 1e3), gbs=nbytes / (ms / 1e3) / 1e9,
        hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        state_gb=S.numel() * 4 / 1e9,
        ms_per_layer_call_fused_epilogue=fused_ms,
        ms_per_layer_call_fused_epilogue_no_workspace=fused1_ms,
        per_call=dict(ms_median=per[Lyr // 2], ms_min=per[0], calls=Lyr),
        stream_ceiling=dict(kernel="in-place scale of one layer's states (torch mul_)", gbs=scale_gbs,
                            decode_frac_of_it=(nbytes / (ms / 1e3) / 1e9) / scale_gbs),
    )


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of nbytes (read nbytes, write nbytes):
    the reference dispatch that scales the HBM byte counters of a
    rocprofv3 --pmc run (FETCH_SIZE, WRITE_SIZE) to bytes."""
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return dict(bytes=nbytes, reps=reps)


# the sources that decide the chunked kernels and their launches, and those
# of the decode step
CHUNK_SOURCES = ("gla_api.cpp", "gla_chunk.hip", "gla_common.hpp", "gla_internal.h")
DECODE_SOURCES = ("gla_api.cpp", "gla_decode.hip", "gla_common.hpp", "gla_internal.h")


def kernel_source_digest(names=CHUNK_SOURCES):
    """sha256 over kernel sources; counted figures are only valid for the
    sources they were counted on."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(REPO, "gated_linear_attention_gla_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


TRAFFIC_FILE = os.path.join(REPO, "profiles", "chunk_kernel_bwd_training_traffic.json")


def counted_traffic():
    """HBM bytes per backward call from the committed counter summary, or
    None when it is missing or was counted on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return t.get("bwd_call_bytes")


DECODE_TRAFFIC_FILE = os.path.join(REPO, "profiles", "decode_and_conv_kernels_traffic.json")


def counted_decode_traffic():
    """HBM bytes per decode layer call (1,280 x 16 states) from the committed
    counter summary, or None when it is missing or was counted on other
    decode sources."""
    try:
        with open(DECODE_TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest(DECODE_SOURCES):
        return None
    return t.get("decode_call_bytes")


MFMA_FILE = os.path.join(REPO, "profiles", "chunk_kernels_training_mfma_lds.json")


def counted_mfma():
    """MFMA utilisation of the training kernels from the committed counter
    summary (busy MFMA cycles over active cycles of all 1,024 SIMDs, i.e. the
    executed bf16 MFMA flops over the dense peak), or None when it is missing
    or was counted on other kernel sources."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return {k: t[k] for k in ("fwd_mfma_util", "bwd_mfma_util", "fwd_executed_over_algorithmic_flops",
                              "bwd_executed_over_algorithmic_flops")}


def bench_conv(gla, inputs, reps=50):
    """Depthwise causal conv + SiLU in front of the mixer: the training batch
    (B=8, T=2,048, D=3,072, bf16 in and out) and one decode step of 1,280
    sequences (window state fp32, updated in place)."""
    import numpy as np
    import torch

    c = inputs.make_conv_inputs()
    B, T, D = c["cfg"]["B"], c["cfg"]["T"], c["cfg"]["D"]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    x = d(c["x"]).to(torch.bfloat16)
    w, bias = d(c["w"]), d(c["bias"])
    y = torch.empty_like(x)
    st = torch.empty((B, 3, D), dtype=torch.float32, device="cuda")
    fwd = lambda: gla.conv1d_fwd(x, w, bias, None, y=y, state_out=st)
    warm_up(fwd)
    stream = torch.cuda.current_stream()
    ms = event_time_ms(fwd, reps, stream)
    nbytes = B * T * D * (2 + 2) + B * 3 * D * 4 + D * 5 * 4
    N = inputs.CONFIGS["decode"]["N"]
    xs = torch.randn((N, D), device="cuda").to(torch.bfloat16)
    win = torch.randn((N, 3, D), device="cuda")
    ys = torch.empty_like(xs)
    step = lambda: gla.conv1d_step_(xs, w, bias, win, y=ys)
    warm_up(step)
    ms_s = event_time_ms(step, reps, stream)
    sbytes = N * D * (2 + 2 + 2 * 3 * 4) + D * 5 * 4
    return dict(
        prefill=dict(workload=f"conv1d width 4 + SiLU, B={B} T={T} D={D}, bf16", ms=ms,
                     tokens_per_s=B * T / (ms / 1e3), gbs=nbytes / (ms / 1e3) / 1e9,
                     hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS),
        decode_step=dict(workload=f"conv1d decode step, N={N} D={D}, bf16, fp32 window", ms=ms_s,
                         gbs=sbytes / (ms_s / 1e3) / 1e9,
                         hbm_frac=sbytes / (ms_s / 1e3) / 1e9 / HBM_PEAK_GBS),
    )


def bench_fused(gla, inputs, reps=20):
    """Training-shape forward with the output epilogue fused into the store
    (self-augmentation, Head RMSNorm, SiLU gate over a bf16 gate stream)."""
    import numpy as np
    import torch

    x = inputs.make_chunk_inputs("training")
    cfg = x["cfg"]
    B, H, T = cfg["B"], cfg["H"], cfg["T"]
    e = inputs.epilogue_inputs(750, B, H, T, DK, DV, "bf16", aug_scale=0.1)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v, g = (d(t).to(torch.bfloat16) for t in (x["q"], x["k"], x["v"], e["g"]))
    lam, S0, aug, gamma = d(x["lam"]), d(x["S0"]), d(e["aug"]), d(e["gamma"])
    y = torch.empty((B, H, T, DV), dtype=torch.bfloat16, device="cuda")
    S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device="cuda")
    fn = lambda: gla.chunk_fwd_fused(q, k, v, lam, g, aug, gamma, 1e-6, S0, chunk=C, y=y, S_T=S_T)
    warm_up(fn)
    ms = event_time_ms(fn, reps, torch.cuda.current_stream())
    nbytes = B * H * T * (FWD_BYTES + 2 * DV) + 2 * B * H * STATE_BYTES
    return dict(workload=f"fwd + fused output epilogue, B={B} H={H} T={T} chunk={C}, bf16 q/k/v/g/y",
                ms=ms, tokens_per_s=B * T / (ms / 1e3), gbs=nbytes / (ms / 1e3) / 1e9,
                hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS)


def bench_varlen(gla, inputs, reps=20):
    """Packed prefill of 64 prompts (lengths log-uniform in 16..4,096 tokens)
    straight into their pages of a 1,280-sequence state pool."""
    import numpy as np
    import torch

    c = inputs.CONFIGS["varlen"]
    lengths = inputs.varlen_lengths(c["cid"], c["N"], c["min_len"], c["max_len"])
    x = inputs.varlen_inputs(c["cid"], lengths, c["H"], c["dk"], c["dv"], num_slots=c["slots"])
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    q, k, v = (d(x[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    lam = torch.tensor(inputs.lambda_log_spaced(c["H"], 0.95, 0.9999), dtype=torch.float32, device="cuda")
    pool = d(x["pool"])[:, 0]
    cu = torch.tensor(x["cu"], dtype=torch.int32, device="cuda")
    slots = torch.tensor(x["slots"], dtype=torch.int32, device="cuda")
    has = torch.tensor(x["has_state"], dtype=torch.int32, device="cuda")
    total = int(lengths.sum())
    o = torch.empty((total, c["H"], c["dv"]), dtype=torch.bfloat16, device="cuda")
    fn = lambda: gla.chunk_fwd_varlen(q, k, v, lam, cu, pool, slots, has, chunk=C, o=o)
    warm_up(fn)
    ms = event_time_ms(fn, reps, torch.cuda.current_stream())
    units = total * c["H"]
    nbytes = units * FWD_BYTES + 2 * c["N"] * c["H"] * STATE_BYTES
    return dict(workload=f"varlen prefill into the decode pool: {c['N']} prompts, {total} tokens "
                         f"(16..4096 log-uniform), H={c['H']}, chunk={C}",
                ms=ms, tokens_per_s=total / (ms / 1e3), gbs=nbytes / (ms / 1e3) / 1e9,
                hbm_frac=nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS)


def cpu_baseline(inputs, min_seconds=5.0):
    """The fp64 oracle (token recurrence forward + two-sweep backward) on the
    training workload itself (B=8, 16 heads, 2,048 tokens; same recipe and
    seeds as the GPU step), repeated until min_seconds of wall time have
    passed, timed on the host cores with OpenMP over the (b, h) units."""
    import oracle

    x = inputs.make_chunk_inputs("training", with_grad=True)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd(x["q"], x["k"], x["v"], x["lam"], x["S0"])
        oracle.bwd(x["q"], x["k"], x["v"], x["lam"], x["dO"], x["S0"])
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    B, T = x["cfg"]["B"], x["cfg"]["T"]
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=reps * B * T / dt, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model,
                sample=f"{reps} fwd+bwd pass(es) of the full training workload (B=8, H=16, "
                       f"T=2048, fp64 oracle), {dt:.2f} s wall")


def _timed(fn, min_seconds):
    """Calls fn until min_seconds of wall time have passed; (calls, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return reps, dt


def oracle_rows(inputs, min_seconds=0.5):
    """The fp64 oracle timed beside the other rows, each on a bounded sample
    of the row's own workload (same recipes), scaled to that row's unit."""
    import numpy as np

    import oracle

    out = {}
    # decode: one step of 64 of the 1,280 sequences (16 heads), per layer call
    N, H = 64, 16
    x = inputs.random_chunk_inputs(5_000_011, N, H, 1, DK, DV, dtype="bf16", scale=1.0)
    S = inputs.normal(5_000_011, inputs.TID["S"], (N, H, DK, DV), 0.01, "f32")
    q, k, v = (np.ascontiguousarray(x[n][:, :, 0]) for n in ("q", "k", "v"))
    reps, dt = _timed(lambda: oracle.decode_step(q, k, v, x["lam"], S), min_seconds)
    out["decode"] = dict(ms_per_layer_call=dt / reps * 1e3 * 1280 / N,
                         sample=f"{reps} steps of {N} sequences x {H} heads, scaled to 1,280 sequences")
    # convolution prefill: one of the 8 sequences (2,048 tokens x 3,072 channels)
    c = inputs.conv_inputs(5_000_012, 1, 2048, 3072, "bf16", state=False)
    reps, dt = _timed(lambda: oracle.conv1d(c["x"], c["w"], c["bias"]), min_seconds)
    out["conv1d_prefill"] = dict(ms=dt / reps * 1e3 * 8, sample=f"{reps} calls on 1 of 8 sequences, scaled to 8")
    # packed prefill: the forward recurrence of the first 4 prompts of the benched mix
    cv = inputs.CONFIGS["varlen"]
    lengths = inputs.varlen_lengths(cv["cid"], cv["N"], cv["min_len"], cv["max_len"])
    sub = [int(t) for t in lengths[:4]]
    xs = [inputs.random_chunk_inputs(5_000_013 + i, 1, cv["H"], t, DK, DV, dtype="bf16") for i, t in enumerate(sub)]
    reps, dt = _timed(lambda: [oracle.fwd(a["q"], a["k"], a["v"], a["lam"], a["S0"]) for a in xs], min_seconds)
    out["varlen_prefill"] = dict(tokens_per_s=reps * sum(sub) / dt,
                                 sample=f"{reps} passes over 4 prompts ({sum(sub)} tokens, 16 heads)")
    # fused epilogue: forward + epilogue on a 256-token slice of one training sequence
    xe = inputs.random_chunk_inputs(5_000_014, 1, 16, 256, DK, DV, dtype="bf16")
    e = inputs.epilogue_inputs(5_000_014, 1, 16, 256, DK, DV, "bf16", aug_scale=0.1)

    def fused():
        o, _ = oracle.fwd(xe["q"], xe["k"], xe["v"], xe["lam"], xe["S0"])
        oracle.epilogue(xe["q"], xe["k"], xe["v"], o, e["aug"], e["gamma"], 1e-6, e["g"])

    reps, dt = _timed(fused, min_seconds)
    out["fused_epilogue_fwd"] = dict(tokens_per_s=reps * 256 / dt, sample=f"{reps} passes over 256 tokens, 16 heads")
    for row in out.values():
        row.update(kind="oracle", cores=oracle.num_threads())
    return out


def rooflines(tr, ms_step):
    """Roofline of the dominant launch (the longer of the forward launch and
    the backward call: algorithmic bytes per launch over its event-timed
    duration) and the whole step's HBM, MFMA and attainable fractions."""
    fwd_gbs = tr["fwd_bytes"] / (tr["ms_fwd"] / 1e3) / 1e9
    bwd_gbs = tr["bwd_bytes"] / (tr["ms_bwd"] / 1e3) / 1e9
    if tr["ms_bwd"] >= tr["ms_fwd"]:
        kernel, achieved, nbytes, ms = "gla_chunk_bwd", bwd_gbs, tr["bwd_bytes"], tr["ms_bwd"]
    else:
        kernel, achieved, nbytes, ms = "gla_chunk_fwd", fwd_gbs, tr["fwd_bytes"], tr["ms_fwd"]
    rf = {"bound": "hbm", "kernel": f"{kernel} (chunk {tr['chunk']})", "achieved": achieved,
          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
          "bytes_per_launch": nbytes, "ms_per_launch": ms}
    step_bytes = tr["fwd_bytes"] + tr["bwd_bytes"]
    step_flops = tr["fwd_flops"] + tr["bwd_flops"]
    srf = {
        "algorithmic_bytes": step_bytes,
        "algorithmic_flops": step_flops,
        "hbm_frac": step_bytes / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "mfma_frac": step_flops / (ms_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
        "attainable_frac": max(step_bytes / (HBM_PEAK_GBS * 1e9),
                               step_flops / (BF16_PEAK_TFLOPS * 1e12)) / (ms_step / 1e3),
        "fwd_gbs": fwd_gbs, "bwd_gbs": bwd_gbs, "ms_fwd": tr["ms_fwd"], "ms_bwd": tr["ms_bwd"],
    }
    return rf, srf


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 100 steps (~40 ms) also bring the GPU clock to speed (see warm_up)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (reference dispatch for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (every call works on "
              "one device; the hot path would shard over (b, h) units and sequences with no "
              "communication between devices)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_linear_attention_gla_amd import _binding as gla, inputs

    gla.load_library()
    torch.cuda.set_device(0)
    log("bench: training-shape fwd+bwd")
    tr = bench_train(gla, inputs, args.steps, args.warmup)
    log(f"  step {tr['ms_step']:.3f} ms  fwd {tr['ms_fwd']:.3f} ms  bwd {tr['ms_bwd']:.3f} ms")
    extra = {}
    for name, reps in (("laplace", 50), ("long", 20)):
        log(f"bench: {name} fwd")
        extra[name + "_fwd"] = bench_fwd_only(gla, inputs, name, reps)
        log(f"  {extra[name + '_fwd']['ms']:.3f} ms")
        # the same workload at the pages' 128-token chunk (results agree up to rounding)
        extra[name + f"_fwd_chunk{C_PAGE}"] = bench_fwd_only(gla, inputs, name, reps, chunk=C_PAGE)
        log(f"  chunk {C_PAGE}: {extra[name + f'_fwd_chunk{C_PAGE}']['ms']:.3f} ms")
    log("bench: laplace fwd+bwd (segment split in both directions)")
    extra["laplace_fwd_bwd"] = bench_fwd_bwd_events(gla, inputs, "laplace", 50)
    log(f"  fwd {extra['laplace_fwd_bwd']['ms_fwd']:.3f} ms  bwd {extra['laplace_fwd_bwd']['ms_bwd']:.3f} ms")
    log(f"bench: training shape fwd+bwd at the pages' {C_PAGE}-token chunk")
    extra["training_chunk128"] = bench_fwd_bwd_events(gla, inputs, "training", 20, chunk=C_PAGE)
    # tile length of each pass at this chunk (the backward's 192 x 96 passes
    # tile at 64 tokens: 128-token tiles fit them on no more than three waves
    # per compute unit; results are equal up to rounding at any tile length)
    extra["training_chunk128"]["tiles"] = {"forward": C_PAGE, "bwd_dq_dk": 64, "bwd_dv": C_PAGE}
    log(f"  fwd {extra['training_chunk128']['ms_fwd']:.3f} ms  bwd {extra['training_chunk128']['ms_bwd']:.3f} ms")
    log("bench: page decay schedule, training shape fwd+bwd")
    extra["schedule_fwd_bwd"] = bench_fwd_bwd_events(gla, inputs, "schedule", 20)
    log(f"  fwd {extra['schedule_fwd_bwd']['ms_fwd']:.3f} ms  bwd {extra['schedule_fwd_bwd']['ms_bwd']:.3f} ms")
    log("bench: fwd with the fused output epilogue")
    extra["fused_epilogue_fwd"] = bench_fused(gla, inputs)
    log(f"  {extra['fused_epilogue_fwd']['ms']:.3f} ms")
    log("bench: varlen prefill into the decode pool")
    extra["varlen_prefill"] = bench_varlen(gla, inputs)
    log(f"  {extra['varlen_prefill']['ms']:.3f} ms  {extra['varlen_prefill']['tokens_per_s'] / 1e6:.2f} Mtok/s")
    log("bench: conv1d (prefill batch and decode step)")
    extra["conv1d"] = bench_conv(gla, inputs)
    log(f"  prefill {extra['conv1d']['prefill']['ms'] * 1e3:.1f} us  {extra['conv1d']['prefill']['gbs']:.0f} GB/s;"
        f"  step {extra['conv1d']['decode_step']['ms'] * 1e3:.1f} us  {extra['conv1d']['decode_step']['gbs']:.0f} GB/s")
    dec = None
    if not args.no_decode:
        log("bench: decode")
        dec = bench_decode(gla, inputs, args.decode_steps)
        log(f"  {dec['ms_total']:.1f} ms  {dec['gbs']:.0f} GB/s")
    if args.calibrate_copy:
        log("bench: 1 GiB copy (counter calibration)")
        copy_calibration()
    cpu = None
    if not args.no_cpu:
        log("bench: cpu oracle baseline")
        cpu = cpu_baseline(inputs)
        log(f"  {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")
        log("bench: cpu oracle beside the other rows")
        rows = oracle_rows(inputs)
        for key, target in (("decode", dec), ("conv1d_prefill", extra["conv1d"]["prefill"]),
                            ("varlen_prefill", extra["varlen_prefill"]),
                            ("fused_epilogue_fwd", extra["fused_epilogue_fwd"])):
            if target is not None:
                target["cpu_oracle"] = rows[key]

    rf, srf = rooflines(tr, tr["ms_step"])
    rf["traffic"] = counted_traffic() if rf["kernel"].startswith("gla_chunk_bwd") else None
    srf["mfma_counted"] = counted_mfma()
    # the same step at the pages' 128-token chunk (config as the pages run it):
    # its per-launch rooflines, with the step taken as forward + backward
    t128 = extra["training_chunk128"]
    rf128, srf128 = rooflines(t128, t128["ms_fwd"] + t128["ms_bwd"])
    t128["roofline"] = rf128
    t128["step_roofline"] = srf128
    out = {
        "metric": METRIC,
        "value": tr["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": tr["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"training-shape chunked GLA fwd+bwd, B=8 H=16 T=2048 dk=96 dv=192 "
                        f"chunk={C}, bf16 q/k/v/dO, fp32 state",
            "chunk_note": f"chunk {C}: results are chunk-invariant up to rounding (tested at 16/32/64/128); "
                          f"the pages' {C_PAGE}-token chunk is timed under extra.training_chunk128 (its "
                          f"backward's dq and dk passes tile at 64 tokens)",
            "global_batch": tr["B"], "seq_len": tr["T"], "heads": tr["H"], "dk": DK, "dv": DV,
            "chunk": C, "parallelism": "single GPU",
        },
        "roofline": rf,
        "step_roofline": srf,
        "cpu_baseline": cpu,
        "decode": dec,
        "extra": extra,
        "lambda": tr["lam"],
    }
    if dec is not None:
        out["decode_roofline"] = {"bound": "hbm", "achieved": dec["gbs"], "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": dec["hbm_frac"], "traffic": counted_decode_traffic(),
                                  "bytes_per_launch": DEC_BYTES * 1280 * 16,
                                  "ms_per_launch": dec["ms_per_layer_call"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

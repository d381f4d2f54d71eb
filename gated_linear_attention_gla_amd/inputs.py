"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no part of the GLA arithmetic: it only draws numbers and
rounds them to the storage dtype.  Every tensor comes from
numpy default_rng(SeedSequence([config_id, tensor_id])), drawn in float64,
scaled, then rounded to fp32 and, where the storage is bf16, to bf16 with
round-to-nearest-even.  Arrays are returned as float64 holding exactly the
stored values, plus the storage dtype name, so the oracle (fp64) and the
device see bit-identical inputs.

Workload shapes follow the page "Beyond the KV cache: Training and serving
i14's Laplace 3B linear attention model on AWS Trainium2 with native PyTorch"
(16 heads, dk = 96 half-width queries/keys, dv = 192 full-width values,
sequence 2,048 in 16 chunks of 128, serving at 1,280 concurrent sequences with
24 layers).  The pages give no value distributions; the Gaussian recipes below
are the synthetic stand-ins.
"""
import math

import numpy as np

# tensor ids inside a config's seed sequence
TID = {"q": 1, "k": 2, "v": 3, "S0": 4, "dO": 5, "dS_T": 6, "S": 7}


def rng(config_id, tensor_id):
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(tensor_id)]))


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x):
    """float -> bf16 bit pattern (uint16), round-to-nearest-even via fp32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b):
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_bf16(x):
    return bf16_bits_to_f64(bf16_bits(x))


def round_to(x, dtype):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)


def normal(config_id, tensor_id, shape, scale=1.0, dtype="f32"):
    x = rng(config_id, tensor_id).standard_normal(size=shape) * scale
    return round_to(x, dtype)


def lambda_log_spaced(H, lo, hi):
    """Per-head decays whose log-decay rates -ln(lambda) are geometrically
    spaced between -ln(lo) and -ln(hi) (both endpoints exact in fp64, then
    rounded to fp32)."""
    g0, g1 = -math.log(lo), -math.log(hi)
    if H == 1:
        gam = np.array([g0])
    else:
        gam = g0 * (g1 / g0) ** (np.arange(H) / (H - 1))
    return round_f32(np.exp(-gam))


def lambda_half_life_schedule(H, t_min, t_max):
    """Decay schedule with half-lives geometrically spaced from t_min to t_max
    tokens: lambda_h = 2^(-1/T_h), T_h = t_min (t_max/t_min)^(h/(H-1)).
    (Reading of the page's section "Decay schedule", whose formula image is
    lost; it reproduces the printed endpoints lambda_0 = 0.5, lambda_15 ~ 0.9997.)"""
    h = np.arange(H)
    th = t_min * (t_max / t_min) ** (h / (H - 1))
    return round_f32(2.0 ** (-1.0 / th))


def lambda_tiny(H):
    return round_f32(1.0 - 2.0 ** (-(4.0 + np.arange(H))))


# ---------------------------------------------------------------------------
# workload configurations
CONFIGS = {
    "tiny": dict(cid=1, B=1, H=2, T=256, dk=16, dv=32, chunk=64, dtype="f32"),
    "laplace": dict(cid=2, B=1, H=16, T=2048, dk=96, dv=192, chunk=128, dtype="bf16"),
    "training": dict(cid=3, B=8, H=16, T=2048, dk=96, dv=192, chunk=128, dtype="bf16"),
    "long": dict(cid=4, B=1, H=16, T=65536, dk=96, dv=192, chunk=128, dtype="bf16"),
    "decode": dict(cid=5, N=1280, L=24, H=16, dk=96, dv=192, steps=64, dtype="bf16"),
    # the training recipe under the page's own decay schedule (half-lives 1 to
    # 2,048 tokens): head 0 has lambda = 1/2, so lambda^128 = 2^-128 is below
    # the smallest normal fp32
    "schedule": dict(cid=6, B=8, H=16, T=2048, dk=96, dv=192, chunk=128, dtype="bf16"),
    # the convolution in front of the mixer: the training batch over the
    # page's D = 3,072 residual channels
    "conv": dict(cid=7, B=8, T=2048, D=3072, dtype="bf16"),
}

CONV_TID = {"x": 1, "w": 2, "bias": 3, "state": 4}

# packed prefill of a batch of prompts into the decode state pool: prompt
# lengths log-uniform in [16, 4,096] tokens, pages for 1,280 sequences
CONFIGS["varlen"] = dict(cid=8, N=64, H=16, dk=96, dv=192, min_len=16, max_len=4096, slots=1280,
                         dtype="bf16")
VARLEN_TID = {"len": 1, "q": 2, "k": 3, "v": 4, "slots": 5, "has": 6, "pool": 7}


def varlen_lengths(seed, N, lo, hi):
    """Seeded prompt lengths, log-uniform in [lo, hi] tokens."""
    u = rng(seed, VARLEN_TID["len"]).uniform(math.log(lo), math.log(hi), size=N)
    return np.floor(np.exp(u)).astype(np.int64)


def varlen_inputs(seed, lengths, H, dk, dv, num_slots, dtype="bf16", pages=1, has_state=True,
                  slots=True):
    """Packed q, k, v [total_T, H, d] (~ N(0, 1/dk)), cu_seqlens, distinct
    pool slots (a seeded choice among num_slots, or 0..N-1), per-sequence
    has_state flags (seeded half/half, or all 1) and an initial pool
    (num_slots, pages, H, dk, dv) ~ N(0, 0.01^2) fp32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    N, total = len(lengths), int(lengths.sum())
    sc = 1.0 / math.sqrt(dk)
    cu = np.zeros(N + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    out = dict(
        lengths=lengths, cu=cu,
        q=normal(seed, VARLEN_TID["q"], (total, H, dk), sc, dtype),
        k=normal(seed, VARLEN_TID["k"], (total, H, dk), sc, dtype),
        v=normal(seed, VARLEN_TID["v"], (total, H, dv), sc, dtype),
        slots=(rng(seed, VARLEN_TID["slots"]).choice(num_slots, size=N, replace=False) if slots
               else np.arange(N)).astype(np.int64),
        has_state=(rng(seed, VARLEN_TID["has"]).integers(0, 2, size=N) if has_state
                   else np.ones(N, dtype=np.int64)),
        pool=normal(seed, VARLEN_TID["pool"], (num_slots, pages, H, dk, dv), 0.01, "f32"),
    )
    return out


def conv_inputs(seed, B, T, D, dtype="bf16", state=True, bias=True):
    """Seeded convolution inputs: x ~ N(0, 1) (storage dtype), taps
    w ~ N(0, 1/4) and bias ~ N(0, 1/100) in fp32, carried window
    state ~ N(0, 1) fp32 (the inputs before token 0) or None."""
    return dict(
        x=normal(seed, CONV_TID["x"], (B, T, D), 1.0, dtype),
        w=normal(seed, CONV_TID["w"], (D, 4), 0.5, "f32"),
        bias=normal(seed, CONV_TID["bias"], (D,), 0.1, "f32") if bias else None,
        state=normal(seed, CONV_TID["state"], (B, 3, D), 1.0, "f32") if state else None,
    )


def make_conv_inputs(B=None, T=None):
    c = dict(CONFIGS["conv"])
    if B is not None:
        c["B"] = B
    if T is not None:
        c["T"] = T
    out = conv_inputs(c["cid"], c["B"], c["T"], c["D"], c["dtype"], state=False)
    out["cfg"] = c
    return out


def make_chunk_inputs(name, B=None, T=None, with_grad=False, s0=None):
    """Inputs of a chunked config (optionally a B/T slice of the same recipe:
    a slice draws its own numbers, it is not a view of the full tensors)."""
    c = dict(CONFIGS[name])
    if B is not None:
        c["B"] = B
    if T is not None:
        c["T"] = T
    cid, B, H, T, dk, dv, dt = c["cid"], c["B"], c["H"], c["T"], c["dk"], c["dv"], c["dtype"]
    out = dict(cfg=c)
    if name == "tiny":
        sc = 1.0 / math.sqrt(dk)
        out["q"] = normal(cid, TID["q"], (B, H, T, dk), sc, dt)
        out["k"] = normal(cid, TID["k"], (B, H, T, dk), sc, dt)
        out["v"] = normal(cid, TID["v"], (B, H, T, dv), sc, dt)
        out["lam"] = lambda_tiny(H)
        out["S0"] = None
    elif name in ("laplace", "training", "schedule"):
        out["q"] = normal(cid, TID["q"], (B, H, T, dk), 1.0, dt)
        out["k"] = normal(cid, TID["k"], (B, H, T, dk), 1.0 / math.sqrt(dk), dt)
        out["v"] = normal(cid, TID["v"], (B, H, T, dv), 1.0, dt)
        if name == "schedule":
            out["lam"] = lambda_half_life_schedule(H, 1.0, 2048.0)
        else:
            out["lam"] = lambda_log_spaced(H, 0.9, 0.999)
        out["S0"] = normal(cid, TID["S0"], (B, H, dk, dv), 0.01, "f32")
    elif name == "long":
        sc = 1.0 / math.sqrt(dk)
        out["q"] = normal(cid, TID["q"], (B, H, T, dk), sc, dt)
        out["k"] = normal(cid, TID["k"], (B, H, T, dk), sc, dt)
        out["v"] = normal(cid, TID["v"], (B, H, T, dv), sc, dt)
        out["lam"] = lambda_log_spaced(H, 0.95, 0.9999)
        out["S0"] = None
    else:
        raise ValueError(name)
    if s0 == "zero":
        out["S0"] = None
    elif s0 == "random":
        out["S0"] = normal(cid, TID["S0"], (B, H, dk, dv), 0.01 if dt == "bf16" else 0.5, "f32")
    if with_grad:
        out["dO"] = normal(cid, TID["dO"], (B, H, T, dv), 1.0, dt)
        out["dS_T"] = None
    return out


def random_chunk_inputs(seed, B, H, T, dk, dv, dtype="f32", s0=True, dS_T=False, lam=None,
                        scale=None):
    """Generic seeded inputs for edge-case tests (seed plays the config id)."""
    sc = scale if scale is not None else 1.0 / math.sqrt(dk)
    out = dict(
        q=normal(seed, TID["q"], (B, H, T, dk), sc, dtype),
        k=normal(seed, TID["k"], (B, H, T, dk), sc, dtype),
        v=normal(seed, TID["v"], (B, H, T, dv), sc, dtype),
        dO=normal(seed, TID["dO"], (B, H, T, dv), 1.0, dtype),
        lam=round_f32(lam) if lam is not None else round_f32(
            rng(seed, 99).uniform(0.5, 1.0, size=H)),
        S0=normal(seed, TID["S0"], (B, H, dk, dv), 0.5, "f32") if s0 else None,
        dS_T=normal(seed, TID["dS_T"], (B, H, dk, dv), 0.5, "f32") if dS_T else None,
    )
    return out


EPI_TID = {"g": 11, "aug": 12, "gamma": 13}


def epilogue_inputs(seed, B, H, T, dk, dv, dtype="bf16", aug_scale=0.5):
    """Gate stream g ~ N(0, 1) (storage dtype, (B, H, T, dv)), per-channel
    balance aug ~ N(0, aug_scale^2) (aug_scale 0: the initial a = 0) and
    RMSNorm weights gamma ~ 1 + N(0, 0.1^2), fp32."""
    return dict(
        g=normal(seed, EPI_TID["g"], (B, H, T, dv), 1.0, dtype),
        aug=(normal(seed, EPI_TID["aug"], (H, dk), aug_scale, "f32") if aug_scale
             else np.zeros((H, dk))),
        gamma=round_f32(1.0 + rng(seed, EPI_TID["gamma"]).standard_normal((H, dv)) * 0.1),
    )

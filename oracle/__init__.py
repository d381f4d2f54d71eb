"""fp64 CPU oracle of the Simple GLA mixer -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check (__graft_entry__.smoke) and the bench's
cpu_baseline leg may import this package.  The product path (libgla.so and
its binding) never does.  The arithmetic lives in gla_oracle.c (plain C,
double precision, OpenMP over independent (b, h) units); this module builds
it with gcc and calls it through its own small C ABI.  It shares no code with
the HIP library.

Functions take numpy arrays (any float dtype, widened exactly to float64) in
dense (B, H, T, d) / (B, H, dk, dv) layout and return float64 arrays.  See
gla_oracle.c for the definitions and the page passages they follow.
"""
import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "gla_oracle.c")
_SRCS = [_SRC, os.path.join(_DIR, "gla_conv_oracle.c"), os.path.join(_DIR, "gla_epilogue_oracle.c")]
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
_LIB = None


def build():
    """Compile liboracle.so with gcc (always rebuilds)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", *_SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(map(os.path.getmtime, _SRCS)):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64 = ctypes.c_int64
        dp = ctypes.c_void_p
        lib.gla_oracle_fwd.argtypes = [i64] * 5 + [dp] * 7
        lib.gla_oracle_fwd_bruteforce.argtypes = [i64] * 5 + [dp] * 6
        lib.gla_oracle_state_closed_form.argtypes = [i64] * 5 + [dp] * 5
        lib.gla_oracle_fwd_chunked.argtypes = [i64] * 6 + [dp] * 7
        lib.gla_oracle_bwd.argtypes = [i64] * 5 + [dp] * 11
        lib.gla_oracle_bwd_bruteforce.argtypes = [i64] * 5 + [dp] * 11
        lib.gla_oracle_decode_step.argtypes = [i64] * 4 + [dp] * 6
        lib.gla_oracle_num_threads.restype = ctypes.c_int
        lib.gla_oracle_conv1d.argtypes = [i64] * 4 + [dp] * 6
        lib.gla_oracle_epilogue.argtypes = [i64] * 5 + [dp] * 6 + [ctypes.c_double] + [dp] * 2
        lib.gla_oracle_conv1d_step.argtypes = [i64] * 3 + [dp] * 5
        _LIB = lib
    return _LIB


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    return None if x is None else ctypes.c_void_p(x.ctypes.data)


def num_threads():
    return _lib().gla_oracle_num_threads()


def _dims(q, v):
    B, H, T, dk = q.shape
    return B, H, T, dk, v.shape[-1]


def fwd(q, k, v, lam, S0=None):
    """Token recurrence: returns (o, S_T)."""
    q, k, v, lam, S0 = map(_f64, (q, k, v, lam, S0))
    B, H, T, dk, dv = _dims(q, v)
    o = np.zeros((B, H, T, dv))
    S_T = np.zeros((B, H, dk, dv))
    _lib().gla_oracle_fwd(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(lam), _p(S0), _p(o), _p(S_T))
    return o, S_T


def fwd_bruteforce(q, k, v, lam, S0=None):
    q, k, v, lam, S0 = map(_f64, (q, k, v, lam, S0))
    B, H, T, dk, dv = _dims(q, v)
    o = np.zeros((B, H, T, dv))
    _lib().gla_oracle_fwd_bruteforce(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(lam), _p(S0), _p(o))
    return o


def state_closed_form(k, v, lam, S0=None):
    k, v, lam, S0 = map(_f64, (k, v, lam, S0))
    B, H, T, dk, dv = _dims(k, v)
    S_T = np.zeros((B, H, dk, dv))
    _lib().gla_oracle_state_closed_form(B, H, T, dk, dv, _p(k), _p(v), _p(lam), _p(S0), _p(S_T))
    return S_T


def fwd_chunked(q, k, v, lam, S0=None, chunk=64):
    q, k, v, lam, S0 = map(_f64, (q, k, v, lam, S0))
    B, H, T, dk, dv = _dims(q, v)
    o = np.zeros((B, H, T, dv))
    S_T = np.zeros((B, H, dk, dv))
    _lib().gla_oracle_fwd_chunked(B, H, T, dk, dv, int(chunk), _p(q), _p(k), _p(v), _p(lam),
                                  _p(S0), _p(o), _p(S_T))
    return o, S_T


def bwd(q, k, v, lam, dO, S0=None, dS_T=None):
    """Returns (dq, dk, dv, dS0) of sum <dO, o> + <dS_T, S_T>."""
    q, k, v, lam, dO, S0, dS_T = map(_f64, (q, k, v, lam, dO, S0, dS_T))
    B, H, T, dk, dv = _dims(q, v)
    dq, dkk = np.zeros((B, H, T, dk)), np.zeros((B, H, T, dk))
    dvv, dS0 = np.zeros((B, H, T, dv)), np.zeros((B, H, dk, dv))
    _lib().gla_oracle_bwd(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(lam), _p(S0), _p(dO),
                          _p(dS_T), _p(dq), _p(dkk), _p(dvv), _p(dS0))
    return dq, dkk, dvv, dS0


def bwd_bruteforce(q, k, v, lam, dO, S0=None, dS_T=None):
    q, k, v, lam, dO, S0, dS_T = map(_f64, (q, k, v, lam, dO, S0, dS_T))
    B, H, T, dk, dv = _dims(q, v)
    dq, dkk = np.zeros((B, H, T, dk)), np.zeros((B, H, T, dk))
    dvv, dS0 = np.zeros((B, H, T, dv)), np.zeros((B, H, dk, dv))
    _lib().gla_oracle_bwd_bruteforce(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(lam), _p(S0),
                                     _p(dO), _p(dS_T), _p(dq), _p(dkk), _p(dvv), _p(dS0))
    return dq, dkk, dvv, dS0


def decode_step(q, k, v, lam, S):
    """One step for (N, H, d) inputs; returns (o, S_new) (S is not modified)."""
    q, k, v, lam = map(_f64, (q, k, v, lam))
    S = np.array(S, dtype=np.float64, copy=True, order="C")
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    _lib().gla_oracle_decode_step(N, H, dk, dv, _p(q), _p(k), _p(v), _p(lam), _p(S), _p(o))
    return o, S


def rel_err(got, ref):
    """max|got - ref| / max|ref| over the whole tensor, in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


CONV_WIDTH = 4  # the page's convolution width


def conv1d(x, w, bias=None, state_in=None):
    """Depthwise causal conv + SiLU over x (B, T, D) with weights w (D, W):
    returns (y, state_out) where state_out (B, W-1, D) holds the last W-1
    inputs (see gla_conv_oracle.c)."""
    x, w, bias, state_in = map(_f64, (x, w, bias, state_in))
    B, T, D = x.shape
    W = w.shape[1]
    y = np.zeros((B, T, D))
    st = np.zeros((B, W - 1, D))
    _lib().gla_oracle_conv1d(B, T, D, W, _p(x), _p(w), _p(bias), _p(state_in), _p(y), _p(st))
    return y, st


def conv1d_step(x, w, bias, state):
    """One decode token: x (N, D), state (N, W-1, D); returns (y, new_state)."""
    x, w, bias = map(_f64, (x, w, bias))
    st = np.array(state, dtype=np.float64, copy=True)
    N, D = x.shape
    W = w.shape[1]
    y = np.zeros((N, D))
    _lib().gla_oracle_conv1d_step(N, D, W, _p(x), _p(w), _p(bias), _p(st), _p(y))
    return y, st


def epilogue(q, k, v, o, a, gamma, eps, g):
    """Mixer output epilogue (self-augmentation, Head RMSNorm, SiLU gate):
    q, k (B, H, T, dk); v, o, g (B, H, T, dv); a (H, dk); gamma (H, dv).
    Returns y (B, H, T, dv); see gla_epilogue_oracle.c."""
    q, k, v, o, a, gamma, g = map(_f64, (q, k, v, o, a, gamma, g))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    y = np.zeros((B, H, T, dv))
    _lib().gla_oracle_epilogue(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(o), _p(a), _p(gamma),
                               float(eps), _p(g), _p(y))
    return y

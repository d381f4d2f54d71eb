"""ctypes binding of libgla.so (argument marshalling only).

Every entry point here forwards device pointers, strides and the current HIP
stream to the C ABI declared in include/gla.h; all arithmetic runs in the HIP
kernels.  PyTorch is used for device memory and streams.  If libgla.so is
missing the calls raise: there is no fallback path.
"""
import ctypes
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgla.so")

GLA_F32 = 0
GLA_BF16 = 1

STATUS_NAMES = {
    0: "GLA_OK",
    1: "GLA_ERR_NULL",
    2: "GLA_ERR_SHAPE",
    3: "GLA_ERR_STRIDE",
    4: "GLA_ERR_DTYPE",
    5: "GLA_ERR_UNSUPPORTED",
    6: "GLA_ERR_ALIAS",
    7: "GLA_ERR_WORKSPACE",
    8: "GLA_ERR_HIP",
}


class GlaTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


class GlaDims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("dk", ctypes.c_int64),
        ("dv", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
    ]


class GlaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_LIB = None


def load_library(path=LIB_PATH):
    """Load libgla.so and declare its signatures.  Raises if it is missing."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m gated_linear_attention_gla_amd.build)"
        )
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.gla_abi_version.restype = ctypes.c_int
    lib.gla_abi_version.argtypes = []
    lib.gla_status_string.restype = ctypes.c_char_p
    lib.gla_status_string.argtypes = [ctypes.c_int]
    lib.gla_chunk_fwd_workspace.restype = ctypes.c_size_t
    lib.gla_chunk_fwd_workspace.argtypes = [P(GlaDims)]
    lib.gla_chunk_bwd_workspace.restype = ctypes.c_size_t
    lib.gla_chunk_bwd_workspace.argtypes = [P(GlaDims)]
    lib.gla_set_segment_wait.restype = None
    lib.gla_set_segment_wait.argtypes = [ctypes.c_int32]
    lib.gla_chunk_fwd.restype = ctypes.c_int
    lib.gla_chunk_fwd.argtypes = [
        P(GlaDims), P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp,
        P(GlaTensor), vp, vp, ctypes.c_size_t, vp,
    ]
    lib.gla_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gla_chunk_fwd_noalloc.argtypes = [
        P(GlaDims), P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp, P(GlaTensor), vp, vp,
    ]
    lib.gla_chunk_bwd.restype = ctypes.c_int
    lib.gla_chunk_bwd.argtypes = [
        P(GlaDims), P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp,
        P(GlaTensor), vp, P(GlaTensor), P(GlaTensor), P(GlaTensor), vp,
        vp, ctypes.c_size_t, vp,
    ]
    lib.gla_decode_step.restype = ctypes.c_int
    lib.gla_decode_step.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp, ctypes.c_int64,
        P(GlaTensor), vp,
    ]
    lib.gla_decode_workgroups_per_state.restype = ctypes.c_int
    lib.gla_decode_workgroups_per_state.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    lib.gla_decode_step_fused_workspace.restype = ctypes.c_size_t
    lib.gla_decode_step_fused_workspace.argtypes = [ctypes.c_int64] * 4
    lib.gla_decode_step_fused.restype = ctypes.c_int
    lib.gla_decode_step_fused.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp, ctypes.c_int64,
        P(GlaTensor), vp, vp, ctypes.c_float, P(GlaTensor), vp, ctypes.c_size_t, vp,
    ]
    lib.gla_chunk_fwd_fused_workspace.restype = ctypes.c_size_t
    lib.gla_chunk_fwd_fused_workspace.argtypes = [P(GlaDims)]
    lib.gla_chunk_fwd_fused.restype = ctypes.c_int
    lib.gla_chunk_fwd_fused.argtypes = [
        P(GlaDims), P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp, P(GlaTensor), vp, vp,
        ctypes.c_float, P(GlaTensor), vp, vp, ctypes.c_size_t, vp,
    ]
    lib.gla_chunk_fwd_varlen.restype = ctypes.c_int
    lib.gla_chunk_fwd_varlen.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        P(GlaTensor), P(GlaTensor), P(GlaTensor), vp, vp, vp, ctypes.c_int64, ctypes.c_int64, vp, vp,
        P(GlaTensor), vp,
    ]
    lib.gla_conv1d_fwd.restype = ctypes.c_int
    lib.gla_conv1d_fwd.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P(GlaTensor), vp, vp, vp,
        P(GlaTensor), vp, vp,
    ]
    lib.gla_conv1d_step.restype = ctypes.c_int
    lib.gla_conv1d_step.argtypes = [
        ctypes.c_int64, ctypes.c_int64, P(GlaTensor), vp, vp, vp, ctypes.c_int64,
        P(GlaTensor), vp,
    ]
    if path == LIB_PATH:
        _LIB = lib
    return lib


def _dtype_code(t):
    if t == torch.float32:
        return GLA_F32
    if t == torch.bfloat16:
        return GLA_BF16
    raise TypeError(f"unsupported dtype {t}: use torch.bfloat16 or torch.float32")


def _view4(x):
    """(b, h, t, d) tensor -> GlaTensor (last dim must be contiguous)."""
    if x.dim() != 4:
        raise ValueError("expected a 4-D (b, h, t, d) tensor")
    if x.numel() == 0:
        return GlaTensor(None, _dtype_code(x.dtype), 0, 0, 0)
    if x.shape[-1] > 1 and x.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    sb, sh, st, _ = x.stride()
    return GlaTensor(x.data_ptr(), _dtype_code(x.dtype), sb, sh, st)


def _view3(x):
    """(n, h, d) tensor -> GlaTensor with stride_t unused."""
    if x.dim() != 3:
        raise ValueError("expected a 3-D (n, h, d) tensor")
    if x.shape[-1] > 1 and x.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    sn, sh, _ = x.stride()
    return GlaTensor(x.data_ptr(), _dtype_code(x.dtype), sn, sh, 0)


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(lib, status):
    if status != 0:
        raise GlaError(status, lib.gla_status_string(status).decode())


def _expect(t, shape, name, dtype=None, contiguous=False):
    """Shape (and optionally dtype / contiguity) of an argument: the C ABI sees
    only pointers and strides, so extents are checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*tensors):
    """Every tensor must live on one GPU: the kernels dereference the pointers."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise ValueError(f"every tensor must be on the same GPU device (got {t.device} and {dev})")


def _state_ok(S, B, H, dk, dv, name):
    _expect(S, (B, H, dk, dv), name, torch.float32, contiguous=True)


def set_segment_wait(microseconds):
    """Bound on how long a workgroup of the one-launch segment split waits for
    an earlier segment's end state before forming it itself (negative: the
    default; 0: form every unpublished state at once).  Speed only."""
    load_library().gla_set_segment_wait(int(microseconds))


def chunk_fwd(q, k, v, lam, S0=None, chunk=64, out_dtype=None, o=None, S_T=None,
              return_state=True):
    """o, S_T = chunk_fwd(q, k, v, lam, S0): chunked Simple GLA forward.

    q, k: (B, H, T, dk); v: (B, H, T, dv) device views (bf16 or fp32, last dim
    contiguous); lam: float32 (H,); S0: float32 (B, H, dk, dv) or None.
    """
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _expect(k, (B, H, T, dk), "k")
    _expect(v, (B, H, T, dv), "v")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(o, (B, H, T, dv), "o")
    _state_ok(S0, B, H, dk, dv, "S0")
    _state_ok(S_T, B, H, dk, dv, "S_T")
    _same_device(q, k, v, lam, o, S0, S_T)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=out_dtype or q.dtype, device=q.device)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    dims = GlaDims(B, H, T, dk, dv, chunk)
    nws = lib.gla_chunk_fwd_workspace(ctypes.byref(dims))
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    tq, tk, tv, to = _view4(q), _view4(k), _view4(v), _view4(o)
    st = lib.gla_chunk_fwd(
        ctypes.byref(dims), ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
        _ptr(lam), _ptr(S0), ctypes.byref(to), _ptr(S_T), _ptr(ws), nws, _stream(),
    )
    _check(lib, st)
    return o, S_T


def chunk_fwd_noalloc(q, k, v, lam, S0, o, S_T=None, chunk=64):
    """chunk_fwd into caller-provided o (and S_T) through gla_chunk_fwd_noalloc:
    the library call allocates nothing (segment states go to the library's
    static device scratch); returns (o, S_T)."""
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _expect(k, (B, H, T, dk), "k")
    _expect(v, (B, H, T, dv), "v")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(o, (B, H, T, dv), "o")
    _state_ok(S0, B, H, dk, dv, "S0")
    _state_ok(S_T, B, H, dk, dv, "S_T")
    _same_device(q, k, v, lam, o, S0, S_T)
    dims = GlaDims(B, H, T, dk, dv, chunk)
    tq, tk, tv, to = _view4(q), _view4(k), _view4(v), _view4(o)
    st = lib.gla_chunk_fwd_noalloc(
        ctypes.byref(dims), ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
        _ptr(lam), _ptr(S0), ctypes.byref(to), _ptr(S_T), _stream(),
    )
    _check(lib, st)
    return o, S_T


def chunk_bwd(q, k, v, lam, dO, S0=None, dS_T=None, chunk=64, grad_dtype=None,
              need_dS0=True, dq=None, dk=None, dv=None, dS0=None):
    """dq, dk, dv, dS0 = chunk_bwd(...): gradients of sum <dO, o> + <dS_T, S_T>."""
    lib = load_library()
    B, H, T, DK = q.shape
    DV = v.shape[-1]
    _expect(k, (B, H, T, DK), "k")
    _expect(v, (B, H, T, DV), "v")
    _expect(dO, (B, H, T, DV), "dO")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    for name, t, d in (("dq", dq, DK), ("dk", dk, DK), ("dv", dv, DV)):
        _expect(t, (B, H, T, d), name)
    _state_ok(S0, B, H, DK, DV, "S0")
    _state_ok(dS_T, B, H, DK, DV, "dS_T")
    _state_ok(dS0, B, H, DK, DV, "dS0")
    _same_device(q, k, v, dO, lam, dq, dk, dv, S0, dS_T, dS0)
    gd = grad_dtype or q.dtype
    if dq is None:
        dq = torch.empty((B, H, T, DK), dtype=gd, device=q.device)
    if dk is None:
        dk = torch.empty((B, H, T, DK), dtype=gd, device=q.device)
    if dv is None:
        dv = torch.empty((B, H, T, DV), dtype=gd, device=q.device)
    if dS0 is None and need_dS0:
        dS0 = torch.empty((B, H, DK, DV), dtype=torch.float32, device=q.device)
    dims = GlaDims(B, H, T, DK, DV, chunk)
    nws = lib.gla_chunk_bwd_workspace(ctypes.byref(dims))
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    views = [_view4(x) for x in (q, k, v, dO, dq, dk, dv)]
    st = lib.gla_chunk_bwd(
        ctypes.byref(dims), *(ctypes.byref(x) for x in views[:3]), _ptr(lam), _ptr(S0),
        ctypes.byref(views[3]), _ptr(dS_T), *(ctypes.byref(x) for x in views[4:]),
        _ptr(dS0), _ptr(ws), nws, _stream(),
    )
    _check(lib, st)
    return dq, dk, dv, dS0


def decode_step_(q, k, v, lam, S, o=None, out_dtype=None):
    """o = decode_step_(q, k, v, lam, S): one recurrent step, S updated in place.

    q, k: (N, H, dk); v: (N, H, dv); S: float32 (N, H, dk, dv) view whose heads
    are dense (stride (S_stride_n, dk*dv, dv, 1)); returns o (N, H, dv).
    """
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    _expect(k, (N, H, dk), "k")
    _expect(v, (N, H, dv), "v")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(o, (N, H, dv), "o")
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("S must be float32 of shape (N, H, dk, dv)")
    if S.stride()[1:] != (dk * dv, dv, 1):
        raise ValueError("each sequence's heads must be dense in S")
    _same_device(q, k, v, lam, S, o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    tq, tk, tv, to = _view3(q), _view3(k), _view3(v), _view3(o)
    st = lib.gla_decode_step(
        N, H, dk, dv, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(lam),
        _ptr(S), S.stride(0), ctypes.byref(to), _stream(),
    )
    _check(lib, st)
    return o


def chunk_fwd_fused(q, k, v, lam, g, aug, gamma, eps=1e-6, S0=None, chunk=64, out_dtype=None, y=None,
                    S_T=None, return_state=True):
    """y, S_T = chunk_fwd_fused(q, k, v, lam, g, aug, gamma, eps, S0): chunked
    forward with the output epilogue (self-augmentation, Head RMSNorm, SiLU
    gate) fused into the store.  g: (B, H, T, dv) view of the gate stream;
    aug float32 (H, dk); gamma float32 (H, dv)."""
    lib = load_library()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _expect(k, (B, H, T, dk), "k")
    _expect(v, (B, H, T, dv), "v")
    _expect(g, (B, H, T, dv), "g")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(y, (B, H, T, dv), "y")
    _state_ok(S0, B, H, dk, dv, "S0")
    _state_ok(S_T, B, H, dk, dv, "S_T")
    for name, t, shp in (("aug", aug, (H, dk)), ("gamma", gamma, (H, dv))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shp}")
    _same_device(q, k, v, g, lam, y, S0, S_T, aug, gamma)
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype or q.dtype, device=q.device)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    dims = GlaDims(B, H, T, dk, dv, chunk)
    nws = lib.gla_chunk_fwd_fused_workspace(ctypes.byref(dims))
    ws = torch.empty(nws, dtype=torch.uint8, device=q.device) if nws else None
    tq, tk, tv, tg, ty = _view4(q), _view4(k), _view4(v), _view4(g), _view4(y)
    st = lib.gla_chunk_fwd_fused(
        ctypes.byref(dims), ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(lam), _ptr(S0),
        ctypes.byref(tg), _ptr(aug), _ptr(gamma), ctypes.c_float(eps), ctypes.byref(ty), _ptr(S_T),
        _ptr(ws), nws, _stream(),
    )
    _check(lib, st)
    return y, S_T


def decode_step_fused_(q, k, v, lam, S, g, aug, gamma, eps=1e-6, y=None, out_dtype=None, ws=None,
                       use_workspace=True):
    """y = decode_step_fused_(q, k, v, lam, S, g, aug, gamma, eps): one
    recurrent step (S in place) with the output epilogue; g (N, H, dv).
    ws: a uint8 device tensor of at least gla_decode_step_fused_workspace()
    bytes, or None to allocate one (use_workspace=False runs the step
    without a workspace)."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError("S must be float32 of shape (N, H, dk, dv)")
    if S.stride()[1:] != (dk * dv, dv, 1):
        raise ValueError("each sequence's heads must be dense in S")
    for name, t, shp in (("aug", aug, (H, dk)), ("gamma", gamma, (H, dv))):
        if t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of shape {shp}")
    _expect(k, (N, H, dk), "k")
    _expect(v, (N, H, dv), "v")
    _expect(g, (N, H, dv), "g")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(y, (N, H, dv), "y")
    _same_device(q, k, v, g, lam, S, y, aug, gamma)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    nws = lib.gla_decode_step_fused_workspace(N, H, dk, dv) if use_workspace else 0
    if nws and ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=q.device)
    if not nws:
        ws = None
    elif ws.dtype != torch.uint8 or ws.numel() < nws or not ws.is_contiguous():
        raise ValueError(f"ws must be a contiguous uint8 tensor of at least {nws} bytes")
    else:
        _same_device(q, ws)
    tq, tk, tv, tg, ty = _view3(q), _view3(k), _view3(v), _view3(g), _view3(y)
    st = lib.gla_decode_step_fused(
        N, H, dk, dv, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), _ptr(lam), _ptr(S), S.stride(0),
        ctypes.byref(tg), _ptr(aug), _ptr(gamma), ctypes.c_float(eps), ctypes.byref(ty), _ptr(ws),
        nws, _stream(),
    )
    _check(lib, st)
    return y


def _packed(x):
    """(t, h, d) packed tensor -> GlaTensor (stride_b unused)."""
    if x.dim() != 3:
        raise ValueError("expected a 3-D (t, h, d) tensor")
    if x.numel() == 0:
        return GlaTensor(None, _dtype_code(x.dtype), 0, 0, 0)
    if x.shape[-1] > 1 and x.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    st, sh, _ = x.stride()
    return GlaTensor(x.data_ptr(), _dtype_code(x.dtype), 0, sh, st)


def chunk_fwd_varlen(q, k, v, lam, cu_seqlens, pool, slots=None, has_state=None, chunk=64,
                     out_dtype=None, o=None):
    """o = chunk_fwd_varlen(q, k, v, lam, cu_seqlens, pool): packed prefill of
    N sequences (cu_seqlens int32 (N+1,) on the device) whose final states go
    to their pages in pool (float32 (num_slots, H, dk, dv) view, heads dense),
    in place.  slots / has_state: int32 (N,) or None."""
    lib = load_library()
    total_T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    N = cu_seqlens.shape[0] - 1
    if pool.dtype != torch.float32 or pool.dim() != 4 or tuple(pool.shape[1:]) != (H, dk, dv):
        raise ValueError(f"pool must be float32 of shape (num_slots, {H}, {dk}, {dv})")
    if pool.stride()[1:] != (dk * dv, dv, 1):
        raise ValueError("each page's heads must be dense in pool")
    for name, t in (("slots", slots), ("has_state", has_state)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (N,)):
            raise ValueError(f"{name} must be int32 of shape ({N},)")
    _expect(k, (total_T, H, dk), "k")
    _expect(v, (total_T, H, dv), "v")
    _expect(lam, (H,), "lam", torch.float32, contiguous=True)
    _expect(o, (total_T, H, dv), "o")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    _same_device(q, k, v, lam, cu_seqlens, pool, slots, has_state, o)
    if o is None:
        o = torch.empty((total_T, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    tq, tk, tv, to = _packed(q), _packed(k), _packed(v), _packed(o)
    st = lib.gla_chunk_fwd_varlen(
        N, H, total_T, dk, dv, chunk, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
        _ptr(cu_seqlens), _ptr(lam), _ptr(pool), pool.shape[0], pool.stride(0), _ptr(slots),
        _ptr(has_state), ctypes.byref(to), _stream(),
    )
    _check(lib, st)
    return o


CONV_WIDTH = 4


def _act3(x):
    """(b, t, d) activation tensor -> GlaTensor (stride_h unused)."""
    if x.dim() != 3:
        raise ValueError("expected a 3-D (b, t, d) tensor")
    if x.numel() == 0:
        return GlaTensor(None, _dtype_code(x.dtype), 0, 0, 0)
    if x.shape[-1] > 1 and x.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    sb, st, _ = x.stride()
    return GlaTensor(x.data_ptr(), _dtype_code(x.dtype), sb, 0, st)


def _conv_w_ok(w, bias, D):
    if w.dtype != torch.float32 or tuple(w.shape) != (D, CONV_WIDTH) or not w.is_contiguous():
        raise ValueError(f"w must be a contiguous float32 tensor of shape {(D, CONV_WIDTH)}")
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (D,)
                             or not bias.is_contiguous()):
        raise ValueError(f"bias must be a contiguous float32 tensor of shape {(D,)}")


def conv1d_fwd(x, w, bias=None, state_in=None, out_dtype=None, y=None, state_out=None,
               return_state=True):
    """y, state_out = conv1d_fwd(x, w, bias, state_in): depthwise causal conv
    (width 4) + SiLU over x (B, T, D); state_in/state_out float32 (B, 3, D)."""
    lib = load_library()
    B, T, D = x.shape
    _conv_w_ok(w, bias, D)
    _expect(y, (B, T, D), "y")
    for name, st_ in (("state_in", state_in), ("state_out", state_out)):
        if st_ is not None and (st_.dtype != torch.float32 or tuple(st_.shape) != (B, CONV_WIDTH - 1, D)
                                or not st_.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 of shape {(B, CONV_WIDTH - 1, D)}")
    _same_device(x, w, bias, state_in, state_out, y)
    if y is None:
        y = torch.empty((B, T, D), dtype=out_dtype or x.dtype, device=x.device)
    if state_out is None and return_state:
        state_out = torch.empty((B, CONV_WIDTH - 1, D), dtype=torch.float32, device=x.device)
    tx, ty = _act3(x), _act3(y)
    st = lib.gla_conv1d_fwd(B, T, D, ctypes.byref(tx), _ptr(w), _ptr(bias), _ptr(state_in),
                            ctypes.byref(ty), _ptr(state_out), _stream())
    _check(lib, st)
    return y, state_out


def conv1d_step_(x, w, bias, state, y=None, out_dtype=None):
    """y = conv1d_step_(x, w, bias, state): one decode token per sequence;
    x (N, D); state float32 (N, 3, D) view (windows dense per sequence), updated
    in place; returns y (N, D)."""
    lib = load_library()
    N, D = x.shape
    _conv_w_ok(w, bias, D)
    if state.dtype != torch.float32 or tuple(state.shape) != (N, CONV_WIDTH - 1, D):
        raise ValueError(f"state must be float32 of shape {(N, CONV_WIDTH - 1, D)}")
    if state.stride()[1:] != (D, 1):
        raise ValueError("each sequence's window must be dense in state")
    _expect(y, (N, D), "y")
    _same_device(x, w, bias, state, y)
    if y is None:
        y = torch.empty((N, D), dtype=out_dtype or x.dtype, device=x.device)
    if x.stride(-1) != 1 or y.stride(-1) != 1:
        raise ValueError("the last dimension must be contiguous")
    tx = GlaTensor(x.data_ptr(), _dtype_code(x.dtype), x.stride(0), 0, 0)
    ty = GlaTensor(y.data_ptr(), _dtype_code(y.dtype), y.stride(0), 0, 0)
    st = lib.gla_conv1d_step(N, D, ctypes.byref(tx), _ptr(w), _ptr(bias), _ptr(state), state.stride(0),
                             ctypes.byref(ty), _stream())
    _check(lib, st)
    return y

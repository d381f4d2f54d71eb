"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/gla.h declares, and rejects bad arguments before anything is
enqueued.  Every call below fails validation, so no kernel is ever launched;
the fake device pointers are never dereferenced."""
import ctypes
import os
import re

import pytest

from gated_linear_attention_gla_amd import _binding as gb

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(REPO, "include", "gla.h")

OK, NULL, SHAPE, STRIDE, DTYPE, UNSUP, ALIAS, WS, HIP = range(9)


@pytest.fixture(scope="module")
def lib():
    return gb.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("gla_chunk_fwd", "gla_chunk_bwd", "gla_decode_step"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gla_abi_version() == 2
    for s in range(9):
        assert lib.gla_status_string(s)
    assert lib.gla_status_string(42) == b"unknown status"


def T(ptr, dtype=gb.GLA_BF16, sb=0, sh=0, st=0):
    return gb.GlaTensor(ptr, dtype, sb, sh, st)


def dims(B=1, H=2, Tn=64, dk=96, dv=192, chunk=64):
    return gb.GlaDims(B, H, Tn, dk, dv, chunk)


def fwd(lib, d, q, k, v, o, lam=0x9000, S0=None, ST=None, ws=None, nws=0):
    ref = lambda x: None if x is None else ctypes.byref(x)
    return lib.gla_chunk_fwd(ref(d), ref(q), ref(k), ref(v), lam, S0, ref(o), ST, ws, nws, None)


def views(H=2, Tn=64, dk=96, dv=192):
    # dense (1, H, T, d) bf16 views at distinct fake, aligned addresses
    q = T(0x100000, sb=H * Tn * dk, sh=Tn * dk, st=dk)
    k = T(0x200000, sb=H * Tn * dk, sh=Tn * dk, st=dk)
    v = T(0x300000, sb=H * Tn * dv, sh=Tn * dv, st=dv)
    o = T(0x400000, sb=H * Tn * dv, sh=Tn * dv, st=dv)
    return q, k, v, o


def test_fwd_null_and_shape(lib):
    q, k, v, o = views()
    assert fwd(lib, None, q, k, v, o) == NULL
    assert fwd(lib, dims(), None, k, v, o) == NULL
    assert fwd(lib, dims(), q, k, v, o, lam=None) == NULL
    assert fwd(lib, dims(B=0), q, k, v, o) == SHAPE
    assert fwd(lib, dims(H=0), q, k, v, o) == SHAPE
    assert fwd(lib, dims(Tn=-1), q, k, v, o) == SHAPE


def test_fwd_dtype(lib):
    q, k, v, o = views()
    k.dtype = gb.GLA_F32
    assert fwd(lib, dims(), q, k, v, o) == DTYPE
    q2, k2, v2, o2 = views()
    o2.dtype = 7
    assert fwd(lib, dims(), q2, k2, v2, o2) == DTYPE


@pytest.mark.parametrize("dk,dv,chunk", [(64, 128, 64), (96, 96, 64), (96, 192, 48), (96, 192, 256),
                                         (16, 32, 8)])
def test_fwd_unsupported(lib, dk, dv, chunk):
    q, k, v, o = views(dk=dk, dv=dv)
    assert fwd(lib, dims(dk=dk, dv=dv, chunk=chunk), q, k, v, o) == UNSUP


def test_fwd_fp32_large_chunk_unsupported(lib):
    q, k, v, o = views()
    for x in (q, k, v):
        x.dtype = gb.GLA_F32
    assert fwd(lib, dims(chunk=128), q, k, v, o) == UNSUP


def test_fwd_stride_checks(lib):
    q, k, v, o = views()
    q.data = 0x100008  # not 16-byte aligned
    assert fwd(lib, dims(), q, k, v, o) == STRIDE
    q, k, v, o = views()
    q.stride_t = 100  # 200-byte rows: row starts not 16-byte aligned
    assert fwd(lib, dims(), q, k, v, o) == STRIDE
    q, k, v, o = views()
    v.stride_h = -192
    assert fwd(lib, dims(), q, k, v, o) == STRIDE
    q, k, v, o = views()
    assert fwd(lib, dims(), q, k, v, o, S0=0x500004) == STRIDE


def test_fwd_alias(lib):
    q, k, v, o = views()
    o.data = q.data
    assert fwd(lib, dims(), q, k, v, o) == ALIAS
    q, k, v, o = views()
    assert fwd(lib, dims(), q, k, v, o, S0=0x500000, ST=0x500000) == ALIAS
    q, k, v, o = views()
    assert fwd(lib, dims(), q, k, v, o, ST=v.data) == ALIAS


def test_workspace_queries(lib):
    d = dims()
    assert lib.gla_chunk_fwd_workspace(ctypes.byref(d)) >= 0
    assert lib.gla_chunk_bwd_workspace(ctypes.byref(d)) >= 0
    assert lib.gla_chunk_fwd_workspace(None) == 0
    assert lib.gla_chunk_fwd_workspace(ctypes.byref(dims(B=0))) == 0


def test_workspace_segment_rule(lib):
    """The workspace holds one fp32 dk x dv end state and dv / 16 8-byte flags
    per (b, h, segment).  No split when the (b, h, column block) units
    already fill the GPU or the sequence has fewer than 4 chunks; otherwise
    2 to 64 segments of at least 2 whole chunks, and the segment length never
    leaves an empty segment."""
    per = lambda B, H: B * H * (96 * 192 * 4 + 192 // 16 * 8)
    q = lambda **kw: lib.gla_chunk_fwd_workspace(ctypes.byref(dims(dk=96, dv=192, **kw)))
    assert q(B=8, H=16, Tn=2048, chunk=128) == 0           # 256 units: no split
    assert q(B=1, H=16, Tn=3 * 128, chunk=128) == 0        # 3 chunks: no split
    assert q(B=1, H=16, Tn=0, chunk=128) == 0
    assert q(B=1, H=16, Tn=2048, chunk=128) == per(1, 16) * 8
    assert q(B=1, H=16, Tn=65536, chunk=128) == per(1, 16) * 8
    assert q(B=1, H=2, Tn=16384, chunk=128) == per(1, 2) * 64
    for T in range(1, 3000, 37):
        for chunk in (16, 64, 128):
            n = q(B=1, H=2, Tn=T, chunk=chunk) // per(1, 2)
            nchunks = -(-T // chunk)
            if n == 0:
                assert nchunks < 4
                continue
            assert 2 <= n <= min(64, nchunks // 2)
            seg = -(-nchunks // n)                   # whole chunks per segment
            assert (n - 1) * seg < nchunks <= n * seg   # the last segment is non-empty
    d = dims(B=1, H=2, Tn=1000, dk=96, dv=192, chunk=64)
    assert lib.gla_chunk_bwd_workspace(ctypes.byref(d)) >= lib.gla_chunk_fwd_workspace(ctypes.byref(d))


def test_bwd_workspace_follows_transposed_tiles(lib):
    """At chunk 128 the backward's dq and dk passes (192 x 96 state) tile at
    64 tokens, so their segment split follows 64-token chunks.  B=1, H=16,
    T=512: 32 (b, h) units of the paired passes, 8 chunks of 64 tokens, so 4
    segments each (two chunks per segment), not the 2 that four 128-token
    chunks would allow; their two regions outweigh the dv pass's."""
    per_t = 192 * 96 * 4 + 96 // 16 * 8  # one transposed state + its flags
    d128 = dims(B=1, H=16, Tn=512, chunk=128)
    d64 = dims(B=1, H=16, Tn=512, chunk=64)
    assert lib.gla_chunk_bwd_workspace(ctypes.byref(d128)) == 2 * 16 * 4 * per_t
    assert lib.gla_chunk_bwd_workspace(ctypes.byref(d64)) == 2 * 16 * 4 * per_t


def test_fused_workspace_follows_its_tile(lib):
    """The fused forward tiles 128-token chunks at 64 tokens (bf16), so its
    segment split at chunk 128 is the one of chunk 64: B=1, H=16, T=2048
    gives 16 (b, h) units, 32 chunks of 64 tokens and 16 segments."""
    q = lambda c: lib.gla_chunk_fwd_fused_workspace(ctypes.byref(dims(B=1, H=16, Tn=2048, chunk=c)))
    assert q(128) == q(64) == 16 * 16 * 96 * 192 * 4


def test_fwd_workspace_checks(lib):
    d = dims(Tn=1000, chunk=64)
    need = lib.gla_chunk_fwd_workspace(ctypes.byref(d))
    assert need > 0
    q, k, v, o = views(Tn=1000)
    assert fwd(lib, d, q, k, v, o) == WS                                  # missing
    assert fwd(lib, d, q, k, v, o, ws=0x800000, nws=need - 4) == WS      # too small
    assert fwd(lib, d, q, k, v, o, ws=0x800008, nws=need) == WS          # misaligned


def fwd_noalloc(lib, d, q, k, v, o, lam=0x9000, S0=None, ST=None):
    ref = lambda x: None if x is None else ctypes.byref(x)
    return lib.gla_chunk_fwd_noalloc(ref(d), ref(q), ref(k), ref(v), lam, S0, ref(o), ST, None)


def test_fwd_noalloc_validation(lib):
    """The allocation-free forward validates like gla_chunk_fwd, and rejects
    dims whose segment states exceed its 16 MiB static scratch before any HIP
    call: B*H = 120 at (96, 192) over 4 chunks needs 240 states of 73,728 B
    (and 96 B of flags each)."""
    assert lib.gla_chunk_fwd_noalloc.restype is ctypes.c_int
    q, k, v, o = views(H=120, Tn=256)
    d = dims(H=120, Tn=256, chunk=64)
    need = lib.gla_chunk_fwd_workspace(ctypes.byref(d))
    assert need == 120 * 2 * (96 * 192 * 4 + 96) > 16 << 20
    assert fwd_noalloc(lib, d, q, k, v, o) == WS
    # the largest B*H that still fits: 113 heads, 226 states
    q2, k2, v2, o2 = views(H=113, Tn=256)
    d2 = dims(H=113, Tn=256, chunk=64)
    assert lib.gla_chunk_fwd_workspace(ctypes.byref(d2)) == 226 * (96 * 192 * 4 + 96) <= 16 << 20
    # ordinary validation comes first and is the same as gla_chunk_fwd's
    assert fwd_noalloc(lib, None, q, k, v, o) == NULL
    assert fwd_noalloc(lib, d, q, k, v, o, lam=None) == NULL
    assert fwd_noalloc(lib, dims(B=0), q, k, v, o) == SHAPE
    assert fwd_noalloc(lib, dims(H=120, Tn=256, chunk=48), q, k, v, o) == UNSUP
    o.data = q.data
    assert fwd_noalloc(lib, d, q, k, v, o) == ALIAS


def bwd(lib, d, q, k, v, dO, dq, dk, dv, lam=0x9000, S0=None, dST=None, dS0=None):
    ref = lambda x: None if x is None else ctypes.byref(x)
    return lib.gla_chunk_bwd(ref(d), ref(q), ref(k), ref(v), lam, S0, ref(dO), dST,
                             ref(dq), ref(dk), ref(dv), dS0, None, 0, None)


def bwd_views():
    q, k, v, o = views()
    dq = T(0x600000, sb=q.stride_b, sh=q.stride_h, st=q.stride_t)
    dk = T(0x700000, sb=q.stride_b, sh=q.stride_h, st=q.stride_t)
    dv = T(0x800000, sb=v.stride_b, sh=v.stride_h, st=v.stride_t)
    return q, k, v, o, dq, dk, dv


def test_bwd_validation(lib):
    q, k, v, dO, dq, dk, dv = bwd_views()
    assert bwd(lib, dims(), q, k, v, None, dq, dk, dv) == NULL
    assert bwd(lib, dims(B=0), q, k, v, dO, dq, dk, dv) == SHAPE
    dO.dtype = gb.GLA_F32
    assert bwd(lib, dims(), q, k, v, dO, dq, dk, dv) == DTYPE
    q, k, v, dO, dq, dk, dv = bwd_views()
    assert bwd(lib, dims(dk=64, dv=128), q, k, v, dO, dq, dk, dv) == UNSUP
    q, k, v, dO, dq, dk, dv = bwd_views()
    dk.data = dq.data
    assert bwd(lib, dims(), q, k, v, dO, dq, dk, dv) == ALIAS
    q, k, v, dO, dq, dk, dv = bwd_views()
    assert bwd(lib, dims(), q, k, v, dO, dq, dk, dv, S0=0x500000, dS0=0x500000) == ALIAS
    q, k, v, dO, dq, dk, dv = bwd_views()
    dv.data = dO.data
    assert bwd(lib, dims(), q, k, v, dO, dq, dk, dv) == ALIAS
    q, k, v, dO, dq, dk, dv = bwd_views()
    for x in (q, k, v, dO):
        x.dtype = gb.GLA_F32
    assert bwd(lib, dims(chunk=64), q, k, v, dO, dq, dk, dv) == UNSUP


def dec(lib, N, H, dk, dv, q, k, v, S=0xA00000, stride=None, o=None, lam=0x9000):
    ref = lambda x: None if x is None else ctypes.byref(x)
    stride = H * dk * dv if stride is None else stride
    return lib.gla_decode_step(N, H, dk, dv, ref(q), ref(k), ref(v), lam, S, stride, ref(o), None)


def dec_views(N=4, H=2, dk=96, dv=192):
    q = T(0x100000, sb=H * dk, sh=dk)
    k = T(0x200000, sb=H * dk, sh=dk)
    v = T(0x300000, sb=H * dv, sh=dv)
    o = T(0x400000, sb=H * dv, sh=dv)
    return q, k, v, o


def test_decode_validation(lib):
    q, k, v, o = dec_views()
    assert dec(lib, 4, 2, 96, 192, q, k, v, S=None, o=o) == NULL
    assert dec(lib, 0, 2, 96, 192, q, k, v, o=o) == SHAPE
    assert dec(lib, 4, 2, 64, 192, q, k, v, o=o) == UNSUP
    assert dec(lib, 4, 2, 96, 192, q, k, v, o=o, stride=100) == SHAPE
    assert dec(lib, 4, 2, 96, 192, q, k, v, S=0xA00004, o=o) == STRIDE
    v.dtype = gb.GLA_F32
    assert dec(lib, 4, 2, 96, 192, q, k, v, o=o) == DTYPE
    q, k, v, o = dec_views()
    o.data = q.data
    assert dec(lib, 4, 2, 96, 192, q, k, v, o=o) == ALIAS
    q, k, v, o = dec_views()
    assert dec(lib, 4, 2, 96, 192, q, k, v, S=k.data, o=o) == ALIAS


def test_decode_launch_shape_boundary(lib):
    """The decode step's per-state workgroup count: three 384-thread column
    slices while N * H * 1152 work-items fit one launch (2^32 - 1), else one
    workgroup per state; the fused step the same with its workspace and one
    without; 0 for rejected sizes."""
    f = lib.gla_decode_workgroups_per_state
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int]
    assert f(1280, 16, 96, 192, 0) == 3
    assert 3_728_270 * 3 * 384 <= 0xFFFFFFFF < 3_728_271 * 3 * 384
    assert f(3_728_270, 1, 96, 192, 0) == 3
    assert f(3_728_271, 1, 96, 192, 0) == 1
    assert f(1 << 20, 4, 96, 192, 0) == 1  # 2^22 states: the old guard's bound, now one workgroup each
    assert f(1 << 24, 1, 96, 192, 0) == 1  # the largest N * H gla_decode_step accepts
    assert f((1 << 24) + 1, 1, 96, 192, 0) == 0
    assert f(1280, 16, 96, 192, 1) == 3  # fused step with its workspace: the same slices
    assert f(3_728_271, 1, 96, 192, 1) == 1
    assert f(1280, 16, 96, 192, 2) == 1  # fused step without a workspace
    assert f(1280, 16, 96, 192, 3) == 0
    assert f(4, 2, 16, 32, 0) == 1
    assert f(4, 2, 16, 32, 1) == 1
    assert f(4, 2, 64, 192, 0) == 0
    assert f(0, 2, 96, 192, 0) == 0


# ------------------------------------------------------------ convolution
def conv_fwd(lib, B, T, D, x, y, w=0xA000, bias=None, sin=None, sout=None):
    ref = lambda t: None if t is None else ctypes.byref(t)
    return lib.gla_conv1d_fwd(B, T, D, ref(x), w, bias, sin, ref(y), sout, None)


def act(ptr, T=16, D=64, dtype=gb.GLA_BF16):
    return T_(ptr, dtype, T * D, D)


def T_(ptr, dtype, sb, st):
    return gb.GlaTensor(ptr, dtype, sb, 0, st)


def test_conv_fwd_rejects_bad_arguments(lib):
    x, y = act(0x100000), act(0x200000)
    assert conv_fwd(lib, 2, 16, 64, None, y) == NULL
    assert conv_fwd(lib, 2, 16, 64, x, y, w=None) == NULL
    assert conv_fwd(lib, 0, 16, 64, x, y) == SHAPE
    assert conv_fwd(lib, 2, -1, 64, x, y) == SHAPE
    assert conv_fwd(lib, 2, 16, 60, x, y) == SHAPE           # D not a multiple of 8
    assert conv_fwd(lib, 2, 16, 0, x, y) == SHAPE
    assert conv_fwd(lib, 2, 16, 64, act(0x100008), y) == STRIDE   # misaligned base
    assert conv_fwd(lib, 2, 16, 64, T_(0x100000, gb.GLA_BF16, 16 * 64, 32), y) == STRIDE  # stride_t < D
    assert conv_fwd(lib, 2, 16, 64, x, y, w=0xA004) == STRIDE
    assert conv_fwd(lib, 2, 16, 64, x, y, sin=0xB008) == STRIDE
    assert conv_fwd(lib, 2, 16, 64, act(0x100000, dtype=7), y) == DTYPE
    assert conv_fwd(lib, 2, 16, 64, x, act(0x100000)) == ALIAS       # y aliases x
    assert conv_fwd(lib, 2, 16, 64, x, y, sin=0xB000, sout=0xB000) == ALIAS
    assert conv_fwd(lib, 2, 16, 64, x, y, sout=0xA000) == ALIAS      # state_out aliases w


def test_conv_step_rejects_bad_arguments(lib):
    ref = ctypes.byref
    x, y = T_(0x100000, gb.GLA_BF16, 64, 0), T_(0x200000, gb.GLA_BF16, 64, 0)
    step = lambda N, D, xx, yy, state=0xC000, stride=192, w=0xA000: lib.gla_conv1d_step(
        N, D, ref(xx), w, None, state, stride, ref(yy), None)
    assert lib.gla_conv1d_step(4, 64, None, 0xA000, None, 0xC000, 192, ref(y), None) == NULL
    assert step(4, 64, x, y, state=None) == NULL
    assert step(0, 64, x, y) == SHAPE
    assert step(4, 64, x, y, stride=191) == SHAPE            # window stride < 3 D
    assert step(4, 64, x, y, stride=194) == STRIDE           # window rows misaligned
    assert step(4, 64, x, y, state=0xC004) == STRIDE
    assert step(4, 64, x, x) == ALIAS
    assert step(4, 64, x, y, state=0x200000) == ALIAS


# ------------------------------------------------------------ varlen prefill
def test_varlen_rejects_bad_arguments(lib):
    ref = ctypes.byref

    def call(N=4, H=2, Tt=100, dk=96, dv=192, chunk=64, q=0x100000, o=0x400000, cu=0x700000, lam=0x9000,
             pool=0x800000, slots_n=8, pstride=2 * 96 * 192, dtype=gb.GLA_BF16):
        tq = gb.GlaTensor(q, dtype, 0, dk, H * dk)
        tk = gb.GlaTensor(0x200000, dtype, 0, dk, H * dk)
        tv = gb.GlaTensor(0x300000, dtype, 0, dv, H * dv)
        to = gb.GlaTensor(o, dtype, 0, dv, H * dv)
        return lib.gla_chunk_fwd_varlen(N, H, Tt, dk, dv, chunk, ref(tq), ref(tk), ref(tv), cu, lam, pool,
                                        slots_n, pstride, None, None, ref(to), None)

    assert call(cu=None) == NULL
    assert call(pool=None) == NULL
    assert call(N=0) == SHAPE
    assert call(Tt=-1) == SHAPE
    assert call(slots_n=0) == SHAPE
    assert call(pstride=2 * 96 * 192 - 1) == SHAPE
    assert call(dk=64) == UNSUP
    assert call(chunk=48) == UNSUP
    assert call(pool=0x800008) == STRIDE
    assert call(pstride=2 * 96 * 192 + 2) == STRIDE
    assert call(o=0x100000) == ALIAS
    assert call(pool=0x400000) == ALIAS
    assert call(dtype=9) == DTYPE


def test_fused_entry_points_reject_bad_arguments(lib):
    ref = ctypes.byref
    q, k, v, o = views()
    g = T(0x500000, sb=2 * 64 * 192, sh=64 * 192, st=192)
    d = dims()
    call = lambda dd=d, gg=g, aug=0xA000, gam=0xB000, eps=1e-6, y=o: lib.gla_chunk_fwd_fused(
        ref(dd), ref(q), ref(k), ref(v), 0x9000, None, ref(gg) if gg else None, aug, gam, ctypes.c_float(eps),
        ref(y), None, None, 0, None)
    assert call(gg=None) == NULL
    assert call(aug=None) == NULL
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(dd=dims(chunk=256)) == UNSUP
    # fp32 inputs at (96, 192) fuse only 16- and 32-token tiles
    q32, k32, v32, _ = views()
    g32 = T(0x500000, gb.GLA_F32, sb=2 * 64 * 192, sh=64 * 192, st=192)
    for x in (q32, k32, v32):
        x.dtype = gb.GLA_F32
    for c in (64, 128):
        assert lib.gla_chunk_fwd_fused(ref(dims(chunk=c)), ref(q32), ref(k32), ref(v32), 0x9000, None, ref(g32),
                                       0xA000, 0xB000, ctypes.c_float(1e-6), ref(o), None, None, 0, None) == UNSUP
    assert call(aug=0xA004) == STRIDE
    assert call(y=T(0x500000, sb=2 * 64 * 192, sh=64 * 192, st=192)) == ALIAS
    # decode with the epilogue
    dq = T(0x100000, sb=2 * 96, sh=96)
    dk_ = T(0x200000, sb=2 * 96, sh=96)
    dv_ = T(0x300000, sb=2 * 192, sh=192)
    dout = T(0x400000, sb=2 * 192, sh=192)
    dg = T(0x500000, sb=2 * 192, sh=192)
    dec = lambda gg=dg, aug=0xA000, y=dout, ws=None, nws=0: lib.gla_decode_step_fused(
        4, 2, 96, 192, ref(dq), ref(dk_), ref(dv_), 0x9000, 0xC00000, 2 * 96 * 192, ref(gg) if gg else None,
        aug, 0xB000, ctypes.c_float(1e-6), ref(y), ws, nws, None)
    assert dec(gg=None) == NULL
    assert dec(aug=None) == NULL
    assert dec(y=T(0x500000, sb=2 * 192, sh=192)) == ALIAS
    # the optional workspace: o' and the slices' sums of squares
    need = lib.gla_decode_step_fused_workspace(4, 2, 96, 192)
    assert need == 4 * 2 * (192 + 4) * 4
    assert lib.gla_decode_step_fused_workspace(4, 2, 16, 32) == 0  # one workgroup per state
    assert lib.gla_decode_step_fused_workspace(0, 2, 96, 192) == 0
    assert dec(ws=0xE00000, nws=need - 4) == WS
    assert dec(ws=0xE00008, nws=need) == WS
    assert dec(ws=0x500000, nws=need) == ALIAS  # the gate stream


# ------------------------------------------------------------ launch-size limits
def test_launch_size_limits(lib):
    """Every launch stays below 2^32 work-items: B*H (and N*H for the packed
    prefill) at most 2^21, N*H at most 2^24 for decode, and the convolution's
    work-item count is checked; the calls are rejected before any launch."""
    ref = ctypes.byref
    q, k, v, o = views()
    # chunked forward: B*H = 2^21 + 2^10 is rejected (H = 2^10, B = 2^11 + 1)
    assert fwd(lib, dims(B=(1 << 11) + 1, H=1 << 10), q, k, v, o) == SHAPE
    # decode: N*H = 2^24 + 16
    dq_, dk_, dv_, do_ = dec_views()
    assert dec(lib, (1 << 20) + 1, 16, 96, 192, dq_, dk_, dv_, o=do_) == SHAPE
    # packed prefill: N*H = 2^21 + 2^10
    tq = gb.GlaTensor(0x100000, gb.GLA_BF16, 0, 96, 1024 * 96)
    tk = gb.GlaTensor(0x200000, gb.GLA_BF16, 0, 96, 1024 * 96)
    tv = gb.GlaTensor(0x300000, gb.GLA_BF16, 0, 192, 1024 * 192)
    to = gb.GlaTensor(0x400000, gb.GLA_BF16, 0, 192, 1024 * 192)
    assert lib.gla_chunk_fwd_varlen((1 << 11) + 1, 1024, 100, 96, 192, 64, ref(tq), ref(tk), ref(tv), 0x700000,
                                    0x9000, 0x800000, 8, 1024 * 96 * 192, None, None, ref(to), None) == SHAPE
    # convolution: 2^16 sequences of 2^16 tokens, 64 channels: 2^26
    # workgroups of 4 waves (fewer than 2^32) but 2^34 work-items
    x, y = act(0x100000), act(0x200000)
    assert conv_fwd(lib, 1 << 16, 1 << 16, 64, x, y) == SHAPE
    # conv decode step: 2^24 sequences of 2^15 channels: 2^30 workgroups
    xs, ys = T_(0x100000, gb.GLA_BF16, 1 << 15, 0), T_(0x200000, gb.GLA_BF16, 1 << 15, 0)
    assert lib.gla_conv1d_step(1 << 24, 1 << 15, ref(xs), 0xA000, None, 0xC000, 3 << 15, ref(ys), None) == SHAPE


def test_c_consumer_compiles():
    """The plain-C consumer of include/gla.h builds with gcc against libgla.so
    (it runs on the GPU in test_gpu_c_abi)."""
    import importlib.util

    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(REPO, "tests", "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert os.path.exists(mod.build())

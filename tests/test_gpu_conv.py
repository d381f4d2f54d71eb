"""GPU parity of the convolution kernels (through the C ABI) against the
fp64 oracle: depthwise causal Conv1d of width 4 + SiLU in front of the mixer
(page "Beyond the KV cache ...", section "i14 and Laplace 3B architecture",
paragraph "Normalization and convolution").

The kernels compute in fp32 from exact stored inputs, so every output (fp32
storage) must match the oracle to max|err|/max|ref| <= 1e-5, and carried
windows (copies of inputs) must match exactly.  bf16-stored outputs must be
the round-to-nearest-even of the fp32-stored run within one bf16 ulp.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_linear_attention_gla_amd import inputs
from gpu_util import dev, dev_f32, flush, host

pytestmark = pytest.mark.gpu
TOL = 1e-5


def run_conv(gla, c, dtype, out_dtype=torch.float32, with_state=True):
    x = dev(c["x"], dtype)
    w, b = dev_f32(c["w"]), dev_f32(c["bias"])
    sin = dev_f32(c["state"]) if with_state else None
    y, st = gla.conv1d_fwd(x, w, b, sin, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(y), host(st)


def check_conv(gla, c, dtype, with_state=True):
    y, st = run_conv(gla, c, dtype, with_state=with_state)
    ry, rst = oracle.conv1d(c["x"], c["w"], c["bias"], c["state"] if with_state else None)
    e = oracle.rel_err(y, ry) if ry.size else 0.0
    flush(f"  conv err y={e:.3e}")
    assert e <= TOL
    assert np.array_equal(st, rst)


@pytest.mark.parametrize("T", [0, 1, 2, 3, 5, 63, 64, 65, 200])
def test_conv_ragged_fp32(gla, T):
    flush(f"test_conv_ragged_fp32 T={T}")
    c = inputs.conv_inputs(500 + T, 2, T, 24, "f32")
    check_conv(gla, c, "f32")


@pytest.mark.parametrize("bias,state", [(False, False), (True, False), (False, True)])
def test_conv_optional_operands(gla, bias, state):
    flush(f"test_conv_optional_operands bias={bias} state={state}")
    c = inputs.conv_inputs(520, 3, 77, 40, "bf16", state=state, bias=bias)
    check_conv(gla, c, "bf16", with_state=state)


@pytest.mark.parametrize("D,dtype", [(520, "bf16"), (1048, "f32"), (1048, "bf16")])
def test_conv_partial_channel_block(gla, D, dtype):
    """Widths that end in a partly filled workgroup after full ones (a
    workgroup covers 512 channels): its taps are staged by every thread,
    also those past the last channel, which then leave without output."""
    flush(f"test_conv_partial_channel_block D={D} {dtype}")
    c = inputs.conv_inputs(590 + D, 3, 37, D, dtype)
    check_conv(gla, c, dtype)


@pytest.mark.parametrize("D", [520, 1048])
def test_conv_step_partial_channel_block(gla, D):
    """The decode step at the same widths, three steps, windows in place."""
    flush(f"test_conv_step_partial_channel_block D={D}")
    N, steps = 9, 3
    c = inputs.conv_inputs(600 + D, N, steps, D, "bf16")
    w, b = dev_f32(c["w"]), dev_f32(c["bias"])
    state = dev_f32(c["state"])
    ref = c["state"].copy()
    for t in range(steps):
        x = dev(np.ascontiguousarray(c["x"][:, t]), "bf16")
        y = gla.conv1d_step_(x, w, b, state, out_dtype=torch.float32)
        ry, ref = oracle.conv1d_step(c["x"][:, t], c["w"], c["bias"], ref)
        torch.cuda.synchronize()
        assert oracle.rel_err(host(y), ry) <= TOL
    assert np.array_equal(host(state), ref)


def test_conv_page_width_bf16(gla):
    """The page's D = 3,072 channels, bf16 activations, fp32 and bf16 outputs."""
    flush("test_conv_page_width_bf16")
    c = inputs.conv_inputs(530, 2, 300, 3072, "bf16")
    check_conv(gla, c, "bf16")
    x = dev(c["x"], "bf16")
    w, b, sin = dev_f32(c["w"]), dev_f32(c["bias"]), dev_f32(c["state"])
    y32, _ = gla.conv1d_fwd(x, w, b, sin, out_dtype=torch.float32)
    y16, _ = gla.conv1d_fwd(x, w, b, sin, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a = y16.view(torch.int16).cpu().numpy().astype(np.int32)
    r = y32.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
    assert np.max(np.abs(a - r)) <= 1


def test_conv_training_batch_full(gla):
    """The full benched shape (B=8, T=2,048, D=3,072, bf16), whole output."""
    flush("test_conv_training_batch_full")
    c = inputs.make_conv_inputs()
    check_conv(gla, c, "bf16", with_state=False)


def test_conv_strided_rows(gla):
    """x and y as column slices of wider rows (stride_t > D)."""
    flush("test_conv_strided_rows")
    c = inputs.conv_inputs(540, 2, 90, 64, "bf16")
    xw = torch.zeros((2, 90, 96), dtype=torch.bfloat16, device="cuda")
    xw[..., 16:80] = dev(c["x"], "bf16")
    x = xw[..., 16:80]
    yw = torch.zeros((2, 90, 128), dtype=torch.float32, device="cuda")
    y = yw[..., 32:96]
    gla.conv1d_fwd(x, dev_f32(c["w"]), dev_f32(c["bias"]), dev_f32(c["state"]), y=y)
    torch.cuda.synchronize()
    ry, _ = oracle.conv1d(c["x"], c["w"], c["bias"], c["state"])
    assert oracle.rel_err(host(y), ry) <= TOL
    assert torch.count_nonzero(yw[..., :32]) == 0 and torch.count_nonzero(yw[..., 96:]) == 0


@pytest.mark.parametrize("split", [1, 3, 64, 100])
def test_conv_chained_calls(gla, split):
    """Two calls carrying the window equal one call."""
    flush(f"test_conv_chained_calls split={split}")
    c = inputs.conv_inputs(550, 2, 150, 32, "f32")
    x = dev(c["x"], "f32")
    w, b, sin = dev_f32(c["w"]), dev_f32(c["bias"]), dev_f32(c["state"])
    ya, sa = gla.conv1d_fwd(x[:, :split], w, b, sin, out_dtype=torch.float32)
    yb, sb = gla.conv1d_fwd(x[:, split:], w, b, sa, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ry, rst = oracle.conv1d(c["x"], c["w"], c["bias"], c["state"])
    assert oracle.rel_err(np.concatenate([host(ya), host(yb)], axis=1), ry) <= TOL
    assert np.array_equal(host(sb), rst)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_decode_steps(gla, dtype):
    """Decode steps against the oracle's steps; windows updated in place."""
    flush(f"test_conv_decode_steps {dtype}")
    N, D, steps = 33, 3072, 5
    c = inputs.conv_inputs(560, N, steps, D, dtype)
    w, b = dev_f32(c["w"]), dev_f32(c["bias"])
    state = dev_f32(c["state"])
    ref = c["state"].copy()
    for t in range(steps):
        x = dev(np.ascontiguousarray(c["x"][:, t]), dtype)
        y = gla.conv1d_step_(x, w, b, state, out_dtype=torch.float32)
        ry, ref = oracle.conv1d_step(c["x"][:, t], c["w"], c["bias"], ref)
        torch.cuda.synchronize()
        assert oracle.rel_err(host(y), ry) <= TOL
    assert np.array_equal(host(state), ref)



def test_conv_decode_step_full_batch(gla):
    """The decode step in the launch configuration the benchmark times:
    1,280 sequences x D = 3,072, bf16 input, fp32 windows, bias, two steps.
    The fp32-stored output and the windows against the oracle; the
    bf16-stored output of the same step (on a copy of the windows) equal to
    the fp32-stored one rounded to nearest, within one bf16 ulp."""
    flush("test_conv_decode_step_full_batch N=1280 D=3072")
    N, D, steps = 1280, 3072, 2
    c = inputs.conv_inputs(575, N, steps, D, "bf16")
    w, b = dev_f32(c["w"]), dev_f32(c["bias"])
    state = dev_f32(c["state"])
    ref = c["state"].copy()
    y16 = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        x = dev(np.ascontiguousarray(c["x"][:, t]), "bf16")
        st16 = state.clone()
        gla.conv1d_step_(x, w, b, st16, y=y16)
        y = gla.conv1d_step_(x, w, b, state, out_dtype=torch.float32)
        ry, ref = oracle.conv1d_step(c["x"][:, t], c["w"], c["bias"], ref)
        torch.cuda.synchronize()
        assert oracle.rel_err(host(y), ry) <= TOL, t
        assert torch.equal(st16, state), t
        a = y16.view(torch.int16).cpu().numpy().astype(np.int32)
        bb = y.to(torch.bfloat16).view(torch.int16).cpu().numpy().astype(np.int32)
        assert np.max(np.abs(a - bb)) <= 1, t
    assert np.array_equal(host(state), ref)

def test_conv_decode_page_pool(gla):
    """Windows inside a per-sequence page holding several layers: only the
    addressed layer's window changes."""
    flush("test_conv_decode_page_pool")
    N, Lyr, D = 7, 3, 64
    c = inputs.conv_inputs(570, N, 1, D, "bf16")
    pool = torch.randn((N, Lyr, 3, D), dtype=torch.float32, device="cuda")
    before = pool.clone()
    win = pool[:, 1]
    ref = host(win)
    y = gla.conv1d_step_(dev(np.ascontiguousarray(c["x"][:, 0]), "bf16"), dev_f32(c["w"]),
                         dev_f32(c["bias"]), win, out_dtype=torch.float32)
    ry, rst = oracle.conv1d_step(c["x"][:, 0], c["w"], c["bias"], ref)
    torch.cuda.synchronize()
    assert oracle.rel_err(host(y), ry) <= TOL
    assert np.array_equal(host(pool[:, 1]), rst)
    assert torch.equal(pool[:, 0], before[:, 0]) and torch.equal(pool[:, 2], before[:, 2])


def test_conv_prefill_then_decode(gla):
    """Prefill hands its window to decode: prefill(T) + steps == prefill(T + steps)."""
    flush("test_conv_prefill_then_decode")
    B, T, steps, D = 4, 70, 6, 128
    c = inputs.conv_inputs(580, B, T + steps, D, "bf16")
    x = dev(c["x"], "bf16")
    w, b = dev_f32(c["w"]), dev_f32(c["bias"])
    _, st = gla.conv1d_fwd(x[:, :T], w, b, None, out_dtype=torch.float32)
    ys = [gla.conv1d_step_(x[:, T + i].contiguous(), w, b, st, out_dtype=torch.float32) for i in range(steps)]
    torch.cuda.synchronize()
    ry, rst = oracle.conv1d(c["x"], c["w"], c["bias"])
    assert oracle.rel_err(np.stack([host(t) for t in ys], axis=1), ry[:, T:]) <= TOL
    assert np.array_equal(host(st), rst)

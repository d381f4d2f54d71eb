"""Simple GLA mixer on AMD MI355X (gfx950): chunked forward/backward and the
recurrent decode step as hand-written HIP kernels behind a C ABI (libgla.so),
plus the fused output epilogue, packed prefill into a decode state pool and
the depthwise causal convolution in front of the mixer.

    from gated_linear_attention_gla_amd import chunk_fwd, chunk_bwd, decode_step_

The Python layer only marshals device pointers and the current stream; the
library must be built in-tree first (python -m gated_linear_attention_gla_amd.build).
"""
__all__ = [
    "chunk_fwd", "chunk_bwd", "decode_step_",
    "chunk_fwd_fused", "decode_step_fused_", "chunk_fwd_varlen",
    "conv1d_fwd", "conv1d_step_", "set_segment_wait",
    "load_library", "GlaError",
]


def __getattr__(name):
    # the binding imports torch; load it only when an entry point is used
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)

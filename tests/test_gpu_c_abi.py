"""The C ABI used from plain C (no Python, no torch): tests/c_abi/gla_abi_demo
allocates with hipMalloc, calls gla_chunk_fwd and gla_decode_step on fp32
inputs and compares both with the fp64 oracle to 1e-5, checks that
gla_chunk_fwd_noalloc gives gla_chunk_fwd's results bit for bit and that
gla_decode_step_fused with its workspace matches the oracle's decode step and
epilogue to 1e-5; it also checks that a NULL argument is rejected."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "gla_abi_demo")


@pytest.mark.gpu
def test_c_program_uses_the_abi():
    assert os.path.exists(EXE), "tests/c_abi/gla_abi_demo is missing: run __graft_entry__.build()"
    print("test_c_program_uses_the_abi", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr

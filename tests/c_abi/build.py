"""Build the plain-C consumer of the C ABI (test infrastructure).

gla_abi_demo links libgla.so (the product library) and liboracle.so (the
fp64 oracle, for the comparison only) with rpaths relative to the executable,
so the tree can move.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "gla_abi_demo")


def build():
    pkg = os.path.join(REPO, "gated_linear_attention_gla_amd")
    orc = os.path.join(REPO, "oracle")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(REPO, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "gla_abi_demo.c"), "-o", EXE + ".tmp",
           "-L", pkg, "-lgla", "-L", orc, "-loracle", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../gated_linear_attention_gla_amd:$ORIGIN/../../oracle:" + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())

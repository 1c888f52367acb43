"""Compile libmoe.so (HIP, gfx950) in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_abi.hip", "moe_kernels.hip", "moe_layer.hip", "moe_batch.hip"]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(force: bool = False, extra=None) -> str:
    if not force and os.path.exists(SO):
        return SO
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *(extra or []), *srcs, "-o", SO + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(SO + ".tmp", SO)
    return SO

"""Compile libmoe.so (HIP, gfx950) in-tree: every translation unit in
parallel, then one link."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libmoe.so")
OBJ_DIR = os.path.join(HERE, "_obj")
# (source, extra defines, object name)
UNITS = [
    ("moe_abi.hip", [], "moe_abi.o"),
    ("moe_kernels.hip", [], "moe_kernels.o"),
    ("moe_gemv.hip", [], "moe_gemv.o"),
    # MFMA results in VGPRs (the AGPR form costs a copy per result register)
    ("moe_batch.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"], "moe_batch.o"),
    ("moe_stack.hip", ["-DMOE_STACK_BITS=4"], "moe_stack4.o"),
    ("moe_stack.hip", ["-DMOE_STACK_BITS=2"], "moe_stack2.o"),
]

HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(force: bool = False, extra=None, jobs: int = 8) -> str:
    if not force and os.path.exists(SO):
        return SO
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]

    def compile_unit(unit):
        src, defs, obj = unit
        out = os.path.join(OBJ_DIR, obj)
        subprocess.check_call(["hipcc", *HIPCC_FLAGS, *inc, *defs, *(extra or []), "-c",
                               os.path.join(HERE, "csrc", src), "-o", out])
        return out

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_unit, UNITS))
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", SO + ".tmp"])
    os.replace(SO + ".tmp", SO)
    return SO

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


def build(force: bool = False, extra=None, jobs: int = 8, out: str = SO) -> str:
    """Compile every unit and link `out` (default: the library itself;
    another path with extra defines gives a variant, such as the timeline
    build)."""
    if not force and os.path.exists(out):
        return out
    obj_dir = OBJ_DIR if out == SO else os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(out))[0])
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]

    def compile_unit(unit):
        src, defs, obj = unit
        o = os.path.join(obj_dir, obj)
        subprocess.check_call(["hipcc", *HIPCC_FLAGS, *inc, *defs, *(extra or []), "-c",
                               os.path.join(HERE, "csrc", src), "-o", o])
        return o

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_unit, UNITS))
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    return out

"""Microbenchmarks (standalone programs, not part of libmoe):

- the exchange latency of the persistent stack kernel's tagged all-gathers
  (csrc/xbench.hip): per case, the time from the last block's store to each
  polling wave seeing every word (median, p90, max), the spread of the
  blocks' store times and the period of one exchange, in microseconds;
- with --read, the HBM read rate of a plain streaming read over the bytes of
  one all-experts GEMV launch (csrc/readbw.hip), the ceiling the dequant
  GEMV is compared with.

    python -m expert_weight_streaming_amd.xbench [--read]   # build and run
    python -m expert_weight_streaming_amd.xbench --build-only

Each prints a markdown table.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

from . import _build

SRC = os.path.join(_build.HERE, "csrc", "xbench.hip")
EXE = os.path.join(_build.OBJ_DIR, "xbench")
READ_SRC = os.path.join(_build.HERE, "csrc", "readbw.hip")
READ_EXE = os.path.join(_build.OBJ_DIR, "readbw")


def build(force: bool = False) -> str:
    """Compile both programs (when missing, or always with force); returns
    the exchange benchmark's path."""
    os.makedirs(_build.OBJ_DIR, exist_ok=True)
    for src, exe in ((SRC, EXE), (READ_SRC, READ_EXE)):
        if force or not os.path.exists(exe):
            subprocess.check_call(["hipcc", *_build.HIPCC_FLAGS, src, "-o", exe])
    return EXE


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--read", action="store_true", help="the HBM read-rate benchmark instead")
    args = ap.parse_args()
    build(force=args.build_only)
    if args.build_only:
        print(EXE)
        print(READ_EXE)
        return
    sys.exit(subprocess.call([READ_EXE if args.read else EXE]))


if __name__ == "__main__":
    main()

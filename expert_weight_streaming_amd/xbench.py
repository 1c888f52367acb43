"""Exchange-latency microbenchmark of the persistent stack kernel's tagged
all-gathers (csrc/xbench.hip, a standalone program).

    python -m expert_weight_streaming_amd.xbench            # build and run
    python -m expert_weight_streaming_amd.xbench --build-only

Prints a markdown table: per case, the time from the last block's store to
each polling wave seeing every word (median, p90, max), the spread of the
blocks' store times and the period of one exchange, in microseconds.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

from . import _build

SRC = os.path.join(_build.HERE, "csrc", "xbench.hip")
EXE = os.path.join(_build.OBJ_DIR, "xbench")


def build(force: bool = False) -> str:
    if force or not os.path.exists(EXE):
        os.makedirs(_build.OBJ_DIR, exist_ok=True)
        subprocess.check_call(["hipcc", *_build.HIPCC_FLAGS, SRC, "-o", EXE])
    return EXE


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--build-only", action="store_true")
    args = ap.parse_args()
    exe = build(force=args.build_only)
    if args.build_only:
        print(exe)
        return
    sys.exit(subprocess.call([exe]))


if __name__ == "__main__":
    main()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


@pytest.fixture(scope="session", autouse=True)
def _host_libs():
    """Build the host-only libraries (oracle, generator) if they are absent."""
    import oracle
    import seedgen
    oracle.build()
    seedgen_so = os.path.join(ROOT, "seedgen", "libseedgen.so")
    if not os.path.exists(seedgen_so):
        import subprocess
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                               os.path.join(ROOT, "seedgen", "seedgen.c"), "-o", seedgen_so, "-lm"])
    yield

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmsk.so")


def _ensure_cpu_libs():
    # The CPU-side libraries (oracle, host filler) are built here if absent;
    # the HIP libraries must be built beforehand (moe_decode_megakernel_amd/build.py).
    if not os.path.exists(os.path.join(ROOT, "oracle", "libmsk_oracle.so")):
        subprocess.run([sys.executable, os.path.join(ROOT, "oracle", "build.py")], check=True)
    if not os.path.exists(os.path.join(ROOT, "moe_decode_megakernel_amd", "libmsk_synth.so")):
        from moe_decode_megakernel_amd import build
        build.build_synth_host()


_ensure_cpu_libs()


def read_golden(name):
    path = os.path.join(ROOT, "tests", "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows

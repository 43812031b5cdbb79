"""Build the native libraries of the package in place (gfx950).

libmsk.so          the verify-step layer kernel and its C ABI (include/msk.h)
libmsk_synth.so    host filler of the seeded synthetic inputs
libmsk_synth_gpu.so device filler of the same inputs

Every call compiles again, whether or not a built library is present.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled for every HIP source. -O2: built with
# -O3 (same register counts) the layer kernel ran the 62-layer step 0.6 %
# slower, and with the scheduler strategies max-ilp, max-memory-clause or
# iterative-minreg 1.8-2.8 % slower.
HIP_FLAGS = ["-O2", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_msk(extra_flags=()):
    csrc = os.path.join(HERE, "csrc")
    out = os.path.join(HERE, "libmsk.so")
    tmp = out + ".tmp"
    _run([HIPCC, *HIP_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"),
          os.path.join(csrc, "msk_layer.hip"), os.path.join(csrc, "msk_api.cpp"), "-o", tmp])
    os.replace(tmp, out)
    return out


def build_synth_host():
    sdir = os.path.join(HERE, "synth")
    out = os.path.join(HERE, "libmsk_synth.so")
    _run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
          os.path.join(sdir, "synth.c"), "-o", out + ".tmp", "-lm"])
    os.replace(out + ".tmp", out)
    return out


def build_synth():
    sdir = os.path.join(HERE, "synth")
    out = build_synth_host()
    gout = os.path.join(HERE, "libmsk_synth_gpu.so")
    _run([HIPCC, *HIP_FLAGS, "-ffp-contract=off", os.path.join(sdir, "synth_gpu.hip"), "-o", gout + ".tmp"])
    os.replace(gout + ".tmp", gout)
    return out, gout


def build_all():
    build_synth()
    build_msk()


if __name__ == "__main__":
    build_all()
    sys.exit(0)

"""Host-side checks of the native library (no GPU needed):
- libmsk.so loads and exports every function include/msk.h declares, and the
  Python binding names the same set;
- the gfx950 code of the layer kernel contains no packed-fp32 arithmetic, no
  scalar-cache stores or atomics, and no register spills to scratch.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msk.h")
LIB = os.path.join(ROOT, "moe_decode_megakernel_amd", "libmsk.so")
KERNEL = os.path.join(ROOT, "moe_decode_megakernel_amd", "csrc", "msk_layer.hip")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = set(re.findall(r"\b(msk_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("msk_workspace_bytes", "msk_create", "msk_load_layer", "msk_verify_layer", "msk_verify_step",
              "msk_destroy", "msk_down_scale_bytes", "msk_pack_down_scale", "msk_last_error"):
        assert n in names, n


def test_library_exports_every_declared_function():
    if not os.path.exists(LIB):
        pytest.skip("libmsk.so not built")
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared in include/msk.h but not exported: {missing}"


def test_binding_names_match_the_header():
    from moe_decode_megakernel_amd import msk
    assert sorted(msk.EXPORTS) == declared_functions()


def test_error_paths_without_a_device():
    """Configuration checks run on the host before any device call."""
    if not os.path.exists(LIB):
        pytest.skip("libmsk.so not built")
    from moe_decode_megakernel_amd import msk, synth
    w = synth.WORKLOADS["tiny_swa"]
    assert msk.msk_workspace_bytes(msk.make_config(w)) > 0
    bad = msk.make_config(w)
    bad.hidden = 300  # not a power of two
    assert msk.msk_workspace_bytes(bad) == 0
    bad = msk.make_config(w, max_tokens=32)
    assert msk.msk_workspace_bytes(bad) == 0
    # flags: the NVFP4-activation and KV-prefetch flags are accepted, unknown bits are not
    assert msk.msk_workspace_bytes(msk.make_config(w, flags=msk.MSK_FLAG_ACT_FP4)) > 0
    assert msk.msk_workspace_bytes(msk.make_config(w, flags=msk.MSK_FLAG_NO_NORM | msk.MSK_FLAG_ACT_FP4)) > 0
    assert msk.msk_workspace_bytes(msk.make_config(w, flags=msk.MSK_FLAG_KV_PREFETCH)) > 0
    assert msk.msk_workspace_bytes(msk.make_config(w, flags=0x8)) == 0
    assert msk.lib().msk_destroy(None) == msk.MSK_E_INVALID


def test_down_scale_packing_checks_without_a_device():
    """Size rule of the tiled down-projection scales, and the argument checks
    msk_pack_down_scale makes before it launches anything."""
    if not os.path.exists(LIB):
        pytest.skip("libmsk.so not built")
    from moe_decode_megakernel_amd import msk
    # [E][P/16][ceil(I/128)][16][8] bytes
    assert msk.msk_down_scale_bytes(256, 2048, 1024) == 256 * 2048 * 1024 // 16
    assert msk.msk_down_scale_bytes(16, 128, 64) == 16 * 8 * 1 * 128
    assert msk.msk_down_scale_bytes(4, 32, 160) == 4 * 2 * 2 * 128
    for bad in ((0, 128, 64), (16, 100, 64), (16, 128, 48), (16, 128, 0)):
        assert msk.msk_down_scale_bytes(*bad) == 0, bad
    assert msk.msk_pack_down_scale(0, 4096, 16, 128, 64, 0) == msk.MSK_E_INVALID
    assert "required" in msk.msk_last_error(None)
    assert msk.msk_pack_down_scale(4104, 4096, 16, 128, 64, 0) == msk.MSK_E_ALIGN
    assert msk.msk_pack_down_scale(4096, 8192, 16, 100, 64, 0) == msk.MSK_E_SHAPE


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from moe_decode_megakernel_amd import build
    out = tmp_path_factory.mktemp("asm") / "msk_layer.s"
    flags = [f for f in build.HIP_FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([hipcc, *flags, "-S", "--cuda-device-only", "-I", os.path.join(ROOT, "include"),
                    KERNEL, "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def _instructions(asm):
    for line in asm.splitlines():
        s = line.strip()
        if not s or s.startswith((".", ";", "//")) or s.endswith(":"):
            continue
        yield s.split()[0]


def test_no_packed_fp32_instructions(kernel_asm):
    bad = sorted({op for op in _instructions(kernel_asm) if re.fullmatch(r"v_pk_(add|mul|fma|mov)_f32", op)})
    assert not bad, bad


def test_no_scalar_cache_writes(kernel_asm):
    bad = sorted({op for op in _instructions(kernel_asm)
                  if op.startswith(("s_store", "s_buffer_store", "s_atomic", "s_buffer_atomic", "s_dcache_wb",
                                    "s_scratch_store"))})
    assert not bad, bad


# Scalar registers the compiler parks in vector-register lanes (v_writelane /
# v_readlane; no memory involved). Each phase of the layer kernel reads the
# kernel arguments it needs afresh, so few argument fields stay live across
# phases; the bound sits above today's level (at most ~55 per instantiation)
# so that a change that brings the launch-long argument registers back is
# noticed.
MAX_SGPR_SPILLS = 80


def test_no_scratch_spills(kernel_asm):
    """No kernel spills registers to scratch, and the production and
    self-timing variants of the layer kernel use no private memory at all.
    The stage-dump variant (template argument 1) may keep a private copy of
    its argument block (<= 1 KiB): it runs in parity tests only. Scalar
    spills into vector lanes are bounded and printed."""
    names = re.findall(r"^\s+\.name:\s+(\S+)", kernel_asm, re.M)
    priv = [int(m) for m in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", kernel_asm)]
    vspill = [int(m) for m in re.findall(r"\.vgpr_spill_count:\s+(\d+)", kernel_asm)]
    sspill = [int(m) for m in re.findall(r"\.sgpr_spill_count:\s+(\d+)", kernel_asm)]
    vgprs = [int(m) for m in re.findall(r"\.vgpr_count:\s+(\d+)", kernel_asm)]
    assert names and len(names) == len(priv) == len(vspill) == len(sspill), (len(names), len(priv), len(vspill))
    for n, pv, vs, ss, vg in zip(names, priv, vspill, sspill, vgprs):
        if "layer_kernel" in n:
            print(f"{n}: {vg} VGPRs, {ss} SGPR spills to lanes, {pv} B private")
        assert vs == 0, (n, "vgpr spills", vs)
        assert ss <= MAX_SGPR_SPILLS, (n, "sgpr spills", ss)
        limit = 1024 if re.search(r"layer_kernelILj\d+ELi1EE", n) else 0
        assert pv <= limit, (n, "private segment", pv)

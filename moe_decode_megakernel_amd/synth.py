"""Seeded synthetic workloads for the verify-step layer (host and device fillers).

The generator is the only code both the oracle and the HIP path consume: it
defines input bytes (weights, KV caches, activations, router bias) as pure
functions of (seed, stream, index) -- see synth/synth_core.h. It holds no
step of the layer's arithmetic.

Workloads (shapes of the pages' model, orcarouter.ai model paragraph and
newruntime.com "What happened": 62 layers, 46 sliding-window (2,048) + 16
global, 8 of 256 experts, NVFP4 experts, bf16 dense layers, pooler/unpooler,
16 verified tokens):
  tiny_swa      one small sliding-window layer (oracle in seconds)
  swa_layer     one working-size sliding-window layer, 8192-token cache
  global_layer  the same layer with global attention over 32768 tokens
  step62        62 layers, global at 3, 7, ..., 59 and 61, 16384-token caches
  batch4_step62 4 requests x 16 tokens through the 62-layer stack, 65536-token caches
"""
import ctypes
import math
import os
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# stream tensor ids (synth_core.h, enum msk_syn_tensor)
W_QKV, W_O, W_ROUTER, W_POOL, W_UNPOOL = 1, 2, 3, 4, 5
E_GATE_UP, E_DOWN, K_CACHE, V_CACHE, H_IN, ROUTER_PERM, H_NOISE = 6, 7, 8, 9, 10, 11, 12

WEIGHT_STD = 0.02
BF16_ONE = 0x3F80


def stream_id(layer: int, tensor: int, sub: int = 0) -> int:
    return ((layer << 40) ^ (tensor << 32) ^ sub) & 0xFFFFFFFFFFFFFFFF


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    nq: int
    nkv: int
    d: int
    E: int
    k: int
    P: int
    I: int
    n_layers: int
    windows: tuple          # per layer; 0 = global
    ctx: int                # prior context per request
    T: int = 16
    R: int = 1
    zipf_s: Optional[float] = None   # router bias -s*ln(rank); None = no bias
    step_rho: Optional[float] = None  # AR(1) correlation of consecutive steps' inputs
    eps: float = 1e-6
    seed: int = 0

    @property
    def NT(self):
        return self.R * self.T

    @property
    def Dq(self):
        return self.nq * self.d

    @property
    def Dkv(self):
        return self.nkv * self.d

    @property
    def cap(self):
        return self.ctx + self.T

    @property
    def gu_scale(self):
        return np.float32(WEIGHT_STD / 64.0)

    @property
    def dn_scale(self):
        return np.float32(WEIGHT_STD / 96.0)


def _step_windows(n=62, window=2048, global_idx=None):
    if global_idx is None:
        global_idx = set(range(3, 60, 4)) | {61}
    return tuple(0 if i in global_idx else window for i in range(n))


WORKLOADS: Dict[str, Workload] = {
    "tiny_swa": Workload("tiny_swa", H=256, nq=4, nkv=1, d=64, E=16, k=2, P=128, I=64,
                         n_layers=1, windows=(32,), ctx=64),
    "swa_layer": Workload("swa_layer", H=4096, nq=32, nkv=4, d=128, E=256, k=8, P=2048, I=1024,
                          n_layers=1, windows=(2048,), ctx=8192, zipf_s=1.1),
    "global_layer": Workload("global_layer", H=4096, nq=32, nkv=4, d=128, E=256, k=8, P=2048, I=1024,
                             n_layers=1, windows=(0,), ctx=32768, zipf_s=1.1),
    "step62": Workload("step62", H=4096, nq=32, nkv=4, d=128, E=256, k=8, P=2048, I=1024,
                       n_layers=62, windows=_step_windows(), ctx=16384, zipf_s=1.1, step_rho=0.9),
    "batch4_step62": Workload("batch4_step62", H=4096, nq=32, nkv=4, d=128, E=256, k=8, P=2048, I=1024,
                              n_layers=62, windows=_step_windows(), ctx=65536, R=4),
}


def small_stack(n_layers=4, base="tiny_swa"):
    """A few layers at tiny shapes (window 32 and global alternating) for
    step-level parity at oracle-friendly sizes."""
    w = WORKLOADS[base]
    wins = tuple(0 if i % 2 else w.windows[0] for i in range(n_layers))
    return replace(w, name=f"{base}_x{n_layers}", n_layers=n_layers, windows=wins)


# ---------------------------------------------------------------------------
# ctypes bindings of the host and device fillers
# ---------------------------------------------------------------------------
_lib = None
_glib = None


def _host():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "libmsk_synth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run moe_decode_megakernel_amd/build.py")
        lib = ctypes.CDLL(path)
        u64, i64, f32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float
        vp = ctypes.c_void_p
        lib.msk_synth_fill_f32.argtypes = [vp, i64, u64, u64, f32, i64]
        lib.msk_synth_fill_bf16.argtypes = [vp, i64, u64, u64, f32, i64]
        lib.msk_synth_fill_nvfp4.argtypes = [vp, vp, i64, i64, u64, u64, f32, f32]
        lib.msk_synth_zipf_bias.argtypes = [vp, ctypes.c_int32, u64, u64, f32]
        lib.msk_synth_ar1.argtypes = [vp, vp, i64, u64, u64, f32, f32]
        lib.msk_synth_normal_const.argtypes = [f32]
        lib.msk_synth_normal_const.restype = f32
        _lib = lib
    return _lib


def _dev():
    global _glib
    if _glib is None:
        path = os.path.join(HERE, "libmsk_synth_gpu.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run moe_decode_megakernel_amd/build.py")
        lib = ctypes.CDLL(path)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        lib.msk_synth_gpu_fill_f32.argtypes = [vp, i64, u64, u64, f32, i64, vp]
        lib.msk_synth_gpu_fill_bf16.argtypes = [vp, i64, u64, u64, f32, i64, vp]
        lib.msk_synth_gpu_fill_nvfp4.argtypes = [vp, vp, i64, i64, u64, u64, f32, f32, vp]
        for f in (lib.msk_synth_gpu_fill_f32, lib.msk_synth_gpu_fill_bf16, lib.msk_synth_gpu_fill_nvfp4):
            f.restype = ctypes.c_int
        _glib = lib
    return _glib


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def normal_f32(n, seed, stream, std=1.0, idx0=0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host().msk_synth_fill_f32(_ptr(out), n, seed, stream, std, idx0)
    return out


def normal_bf16(n, seed, stream, std=1.0, idx0=0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    _host().msk_synth_fill_bf16(_ptr(out), n, seed, stream, std, idx0)
    return out


def nvfp4(rows, cols, seed, stream, std, s_tensor):
    codes = np.empty((rows, cols // 2), dtype=np.uint8)
    scales = np.empty((rows, cols // 16), dtype=np.uint8)
    _host().msk_synth_fill_nvfp4(_ptr(codes), _ptr(scales), rows, cols, seed, stream, std, s_tensor)
    return codes, scales


def zipf_bias(n, seed, stream, s) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _host().msk_synth_zipf_bias(_ptr(out), n, seed, stream, s)
    return out


# ---------------------------------------------------------------------------
# Layers, caches and inputs (host arrays)
# ---------------------------------------------------------------------------
def layer_weights(w: Workload, layer: int, experts: Optional[List[int]] = None) -> dict:
    """All weights of one layer as numpy arrays in the library's layouts.
    experts: restrict the expert tensors to these experts (others zero-filled
    bytes are not generated; used by the oracle to regenerate on demand)."""
    s = w.seed
    Nqkv = w.Dq + 2 * w.Dkv
    out = {
        "window": int(w.windows[layer]),
        "w_qkv": normal_bf16(Nqkv * w.H, s, stream_id(layer, W_QKV), WEIGHT_STD).reshape(Nqkv, w.H),
        "w_o": normal_bf16(w.H * w.Dq, s, stream_id(layer, W_O), WEIGHT_STD).reshape(w.H, w.Dq),
        "w_router": normal_f32(w.E * w.H, s, stream_id(layer, W_ROUTER), WEIGHT_STD).reshape(w.E, w.H),
        "b_router": (zipf_bias(w.E, s, stream_id(layer, ROUTER_PERM), w.zipf_s) if w.zipf_s else None),
        "w_pool": normal_bf16(w.P * w.H, s, stream_id(layer, W_POOL), WEIGHT_STD).reshape(w.P, w.H),
        "w_unpool": normal_bf16(w.H * w.P, s, stream_id(layer, W_UNPOOL), WEIGHT_STD).reshape(w.H, w.P),
        "g_attn": np.full(w.H, BF16_ONE, dtype=np.uint16),
        "g_moe": np.full(w.H, BF16_ONE, dtype=np.uint16),
    }
    E, I, P = w.E, w.I, w.P
    gu = np.zeros((E, 2 * I, P // 2), np.uint8)
    gus = np.zeros((E, 2 * I, P // 16), np.uint8)
    dn = np.zeros((E, P, I // 2), np.uint8)
    dns = np.zeros((E, P, I // 16), np.uint8)
    for e in (range(E) if experts is None else experts):
        gu[e], gus[e] = nvfp4(2 * I, P, s, stream_id(layer, E_GATE_UP, e), WEIGHT_STD, w.gu_scale)
        dn[e], dns[e] = nvfp4(P, I, s, stream_id(layer, E_DOWN, e), WEIGHT_STD, w.dn_scale)
    out.update(e_gate_up=gu, e_gate_up_scale=gus, e_down=dn, e_down_scale=dns,
               e_tensor_scale=np.tile(np.array([w.gu_scale, w.dn_scale], np.float32), (E, 1)))
    return out


def kv_cache(w: Workload, layer: int):
    """bf16 K and V caches [R][nkv][cap][d] of one layer (N(0,1) history)."""
    n = w.nkv * w.cap * w.d
    k = np.empty((w.R, w.nkv, w.cap, w.d), np.uint16)
    v = np.empty_like(k)
    for r in range(w.R):
        k[r] = normal_bf16(n, w.seed, stream_id(layer, K_CACHE, r)).reshape(w.nkv, w.cap, w.d)
        v[r] = normal_bf16(n, w.seed, stream_id(layer, V_CACHE, r)).reshape(w.nkv, w.cap, w.d)
    return k, v


def h_input(w: Workload, step: int = 0) -> np.ndarray:
    """Residual input fp32 [NT][H] of a verify step. Steps of a workload with
    step_rho are AR(1)-correlated: h_s = rho*h_{s-1} + sqrt(1-rho^2)*noise_s."""
    n = w.NT * w.H
    h = normal_f32(n, w.seed, stream_id(0, H_IN, 0))
    if w.step_rho is not None and step > 0:
        a = np.float32(w.step_rho)
        b = np.float32(math.sqrt(1.0 - w.step_rho ** 2))
        for s in range(1, step + 1):
            nxt = np.empty_like(h)
            _host().msk_synth_ar1(_ptr(nxt), _ptr(h), n, w.seed, stream_id(0, H_NOISE, s), a, b)
            h = nxt
    return h.reshape(w.NT, w.H)


# ---------------------------------------------------------------------------
# Device fillers (torch tensors on the GPU), same bytes as the host fillers
# ---------------------------------------------------------------------------
def _check(rc):
    if rc != 0:
        raise RuntimeError(f"device filler failed with HIP error {rc}")


def dev_normal_bf16(t, seed, stream, std=1.0, stream_ptr=None):
    _check(_dev().msk_synth_gpu_fill_bf16(t.data_ptr(), t.numel(), seed, stream, std, 0, stream_ptr))


def dev_normal_f32(t, seed, stream, std=1.0, stream_ptr=None):
    _check(_dev().msk_synth_gpu_fill_f32(t.data_ptr(), t.numel(), seed, stream, std, 0, stream_ptr))


def dev_nvfp4(codes, scales, rows, cols, seed, stream, std, s_tensor, stream_ptr=None):
    _check(_dev().msk_synth_gpu_fill_nvfp4(codes.data_ptr(), scales.data_ptr(), rows, cols, seed, stream,
                                           std, float(s_tensor), stream_ptr))


# ---------------------------------------------------------------------------
# Upload of host arrays (torch tensors in device memory)
# ---------------------------------------------------------------------------
def to_device(arrays: dict, device="cuda") -> dict:
    """numpy arrays -> torch tensors on `device` (same dtypes; uint16 as int16 bits)."""
    import torch
    out = {}
    for name, a in arrays.items():
        if a is None or not isinstance(a, np.ndarray):
            out[name] = a
            continue
        if a.dtype == np.uint16:
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out[name] = t.to(device)
    return out


def device_layer(w: Workload, layer: int, device="cuda", with_cache=True, stream_ptr=None) -> dict:
    """One layer's weights (and KV caches) filled directly in device memory by
    the device filler: the same bytes layer_weights()/kv_cache() produce."""
    import torch
    s = w.seed
    Nqkv = w.Dq + 2 * w.Dkv
    i16 = dict(dtype=torch.int16, device=device)
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    t = {
        "w_qkv": torch.empty((Nqkv, w.H), **i16),
        "w_o": torch.empty((w.H, w.Dq), **i16),
        "w_router": torch.empty((w.E, w.H), **f32),
        "w_pool": torch.empty((w.P, w.H), **i16),
        "w_unpool": torch.empty((w.H, w.P), **i16),
        "g_attn": torch.full((w.H,), BF16_ONE, **i16),
        "g_moe": torch.full((w.H,), BF16_ONE, **i16),
        "e_gate_up": torch.empty((w.E, 2 * w.I, w.P // 2), **u8),
        "e_gate_up_scale": torch.empty((w.E, 2 * w.I, w.P // 16), **u8),
        "e_down": torch.empty((w.E, w.P, w.I // 2), **u8),
        "e_down_scale": torch.empty((w.E, w.P, w.I // 16), **u8),
    }
    dev_normal_bf16(t["w_qkv"], s, stream_id(layer, W_QKV), WEIGHT_STD, stream_ptr)
    dev_normal_bf16(t["w_o"], s, stream_id(layer, W_O), WEIGHT_STD, stream_ptr)
    dev_normal_f32(t["w_router"], s, stream_id(layer, W_ROUTER), WEIGHT_STD, stream_ptr)
    dev_normal_bf16(t["w_pool"], s, stream_id(layer, W_POOL), WEIGHT_STD, stream_ptr)
    dev_normal_bf16(t["w_unpool"], s, stream_id(layer, W_UNPOOL), WEIGHT_STD, stream_ptr)
    for e in range(w.E):
        dev_nvfp4(t["e_gate_up"][e], t["e_gate_up_scale"][e], 2 * w.I, w.P, s,
                  stream_id(layer, E_GATE_UP, e), WEIGHT_STD, w.gu_scale, stream_ptr)
        dev_nvfp4(t["e_down"][e], t["e_down_scale"][e], w.P, w.I, s,
                  stream_id(layer, E_DOWN, e), WEIGHT_STD, w.dn_scale, stream_ptr)
    t["e_tensor_scale"] = torch.from_numpy(
        np.tile(np.array([w.gu_scale, w.dn_scale], np.float32), (w.E, 1))).to(device)
    t["b_router"] = (torch.from_numpy(zipf_bias(w.E, s, stream_id(layer, ROUTER_PERM), w.zipf_s)).to(device)
                     if w.zipf_s else None)
    if with_cache:
        k = torch.empty((w.R, w.nkv, w.cap, w.d), **i16)
        v = torch.empty((w.R, w.nkv, w.cap, w.d), **i16)
        for r in range(w.R):
            dev_normal_bf16(k[r], s, stream_id(layer, K_CACHE, r), 1.0, stream_ptr)
            dev_normal_bf16(v[r], s, stream_id(layer, V_CACHE, r), 1.0, stream_ptr)
        t["k_cache"], t["v_cache"] = k, v
    return t


def algorithmic_bytes_per_layer(w: Workload, layer: int, n_sel: int) -> int:
    """Bytes the layer must move (each once): dense weights, the selected
    experts' codes and scales, the KV rows in the union of the verify tokens'
    windows, and the KV write. Unselected experts and out-of-window rows are
    not counted."""
    Nqkv = w.Dq + 2 * w.Dkv
    dense = 2 * (Nqkv * w.H + w.H * w.Dq + w.P * w.H + w.H * w.P) + 4 * w.E * w.H + 2 * 2 * w.H
    expert = (2 * w.I * w.P) // 2 + (2 * w.I * w.P) // 16 + (w.P * w.I) // 2 + (w.P * w.I) // 16 + 8
    win = w.windows[layer]
    rows = (w.ctx + w.T) if win <= 0 else min(w.ctx + w.T, win + w.T - 1)
    kv_read = w.R * rows * w.nkv * w.d * 2 * 2
    kv_write = w.R * w.T * w.nkv * w.d * 2 * 2
    return dense + n_sel * expert + kv_read + kv_write


def verify_tree(T, seed):
    """Seeded tree of T verify tokens: the parent of token t is drawn uniformly
    from -1 (a root on the prior context) and 0 .. t-1. Returns the ancestor
    bitmask of every token (self included), uint16 [T]."""
    rng = np.random.default_rng(seed)
    anc = []
    for t in range(T):
        par = int(rng.integers(-1, t)) if t > 0 else -1
        anc.append((1 << t) | (anc[par] if par >= 0 else 0))
    return np.array(anc, np.uint16)

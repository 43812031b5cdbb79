"""Python wrapper of the oracle (libmsk_oracle.so): TEST INFRASTRUCTURE.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
use this module. It shares no code with the HIP path: it reads the same
seeded input arrays (numpy) and runs the plain C definition of the layer
(msk_oracle.c) on the CPU. Functions without a pin against the pages or the
mathematics are listed in the repository's design notes as "parity unpinned";
every function here is pinned by a test under tests/ (test_oracle_*.py).
"""
import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

c_i32, c_f32, c_f64, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_void_p


class OrcLayer(ctypes.Structure):
    _fields_ = [
        ("hidden", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
        ("n_experts", c_i32), ("top_k", c_i32), ("pool_dim", c_i32), ("expert_inter", c_i32),
        ("window", c_i32), ("kv_capacity", c_i32), ("rms_eps", c_f32), ("use_norm", c_i32),
        ("act_fp4", c_i32),
        ("w_qkv", vp), ("w_o", vp), ("w_router", vp), ("b_router", vp), ("w_pool", vp),
        ("w_unpool", vp), ("g_attn", vp), ("g_moe", vp), ("e_gate_up", vp),
        ("e_gate_up_scale", vp), ("e_down", vp), ("e_down_scale", vp), ("e_tensor_scale", vp),
    ]


class OrcStages(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("q", "k_new", "v_new", "attn", "h1", "n2_f32", "logits", "ids",
                                  "gates", "p", "acc")]


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "libmsk_oracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run oracle/build.py")
        L = ctypes.CDLL(path)
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = c_f64
        L.orc_bf16_rne.argtypes = [c_f64]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_value.restype = c_f64
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = c_f64
        L.orc_nvfp4_dequant.argtypes = [vp, vp, c_f64, ctypes.c_int64, ctypes.c_int64, vp]
        L.orc_dot_canon_f32.argtypes = [vp, vp, c_i32]
        L.orc_dot_canon_f32.restype = c_f32
        L.orc_topk.argtypes = [vp, c_i32, c_i32, vp]
        L.orc_gates.argtypes = [vp, vp, c_i32, vp]
        L.orc_prefetch_list.argtypes = [vp, c_i32, c_i32, c_i32, vp]
        L.orc_rmsnorm.argtypes = [vp, vp, c_i32, c_f64, vp]
        L.orc_silu.argtypes = [c_f64]
        L.orc_silu.restype = c_f64
        L.orc_attention.argtypes = [vp, vp, vp, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, vp, vp]
        L.orc_layer_forward.argtypes = [ctypes.POINTER(OrcLayer), c_i32, c_i32, vp, vp, vp, vp, vp, vp,
                                        ctypes.POINTER(OrcStages)]
        L.orc_e4m3_rne_sat.argtypes = [c_f32]
        L.orc_e4m3_rne_sat.restype = ctypes.c_uint8
        L.orc_e2m1_rne_sat.argtypes = [c_f32]
        L.orc_e2m1_rne_sat.restype = ctypes.c_uint8
        L.orc_nvfp4_quant16.argtypes = [vp, vp, vp, vp]
        L.orc_tree_valid.argtypes = [vp, c_i32]
        L.orc_tree_valid.restype = c_i32
        L.orc_layer_forward.restype = c_i32
        L.orc_dense_swiglu.argtypes = [vp, c_i32, vp, vp, c_i32, c_i32, vp]
        L.orc_threads.restype = c_i32
        L.orc_set_threads.argtypes = [c_i32]
        L.orc_set_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous, "arrays must be C-contiguous numpy"
    return a.ctypes.data_as(vp)


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (timing only)."""
    lib().orc_set_threads(int(n))


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def bf16_rne(x: float) -> int:
    return lib().orc_bf16_rne(x)


def e2m1_value(n: int) -> float:
    return lib().orc_e2m1_value(n)


def e4m3_value(c: int) -> float:
    return lib().orc_e4m3_value(c)


def nvfp4_dequant(codes, scales, s_tensor, rows, cols):
    out = np.empty((rows, cols), np.float64)
    lib().orc_nvfp4_dequant(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)),
                            float(s_tensor), rows, cols, _p(out))
    return out


def dot_canon_f32(x, w) -> np.float32:
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w, np.float32)
    return np.float32(lib().orc_dot_canon_f32(_p(x), _p(w), x.size))


def topk(logits, k):
    lg = np.ascontiguousarray(logits, np.float32)
    ids = np.empty(k, np.int32)
    lib().orc_topk(_p(lg), lg.size, k, _p(ids))
    return ids


def gates(logits, ids):
    lg = np.ascontiguousarray(logits, np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    g = np.empty(ids.size, np.float64)
    lib().orc_gates(_p(lg), _p(ids), ids.size, _p(g))
    return g


def prefetch_list(ids, n_experts, p):
    """Top-p experts by selection count in ids (count desc, index asc)."""
    ids = np.ascontiguousarray(ids, np.int32).ravel()
    out = np.empty(p, np.int32)
    lib().orc_prefetch_list(_p(ids), ids.size, n_experts, p, _p(out))
    return out


def rmsnorm(x, g_bf16, eps):
    x = np.ascontiguousarray(x, np.float64)
    g = np.ascontiguousarray(g_bf16, np.uint16)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(y))
    return y


def silu(x: float) -> float:
    return lib().orc_silu(x)


def _tree_arg(tree, n):
    if tree is None:
        return None
    a = np.ascontiguousarray(np.asarray(tree, np.uint16).reshape(-1))
    if a.size != n:
        raise ValueError(f"tree mask needs {n} entries")
    return a


def e4m3_rne_sat(x: float) -> int:
    return int(lib().orc_e4m3_rne_sat(float(x)))


def e2m1_rne_sat(y: float) -> int:
    return int(lib().orc_e2m1_rne_sat(float(y)))


def nvfp4_quant16(x):
    """16 fp32 values -> (codes uint8 [16], E4M3 scale code, dequantized fp32 [16])."""
    x = np.ascontiguousarray(np.asarray(x, np.float32).reshape(16))
    codes = np.empty(16, np.uint8)
    sc = np.empty(1, np.uint8)
    deq = np.empty(16, np.float32)
    lib().orc_nvfp4_quant16(_p(x), _p(codes), _p(sc), _p(deq))
    return codes, int(sc[0]), deq


def nvfp4_quant_rows(x):
    """[rows][n] fp32 (n a multiple of 16) -> dequantized fp32, block by block."""
    x = np.asarray(x, np.float32)
    out = np.empty_like(x)
    for r in range(x.shape[0]):
        for b in range(0, x.shape[1], 16):
            out[r, b:b + 16] = nvfp4_quant16(x[r, b:b + 16])[2]
    return out


def tree_valid(tree, T) -> bool:
    """orc_tree_valid: self bit set, no later bit, closed under ancestry."""
    a = _tree_arg(tree, T)
    return bool(lib().orc_tree_valid(_p(a), T))


def attention(q, k_cache, v_cache, nq, nkv, d, cap, T, ctx, window, tree=None):
    """q: [T][nq*d] fp64; caches: [nkv][cap][d] bf16 of one request; tree: [T]
    ancestor bitmasks of the verified tokens, or None for the chain."""
    q = np.ascontiguousarray(q, np.float64)
    out = np.empty((T, nq * d), np.float64)
    tr = _tree_arg(tree, T)
    lib().orc_attention(_p(q), _p(np.ascontiguousarray(k_cache)), _p(np.ascontiguousarray(v_cache)),
                        nq, nkv, d, cap, T, ctx, window, _p(tr), _p(out))
    return out


def dense_swiglu(x, wgu, wd):
    x = np.ascontiguousarray(x, np.float64)
    wgu = np.ascontiguousarray(wgu, np.float64)
    wd = np.ascontiguousarray(wd, np.float64)
    nt, P = x.shape
    I = wgu.shape[0] // 2
    y = np.empty((nt, wd.shape[0]), np.float64)
    lib().orc_dense_swiglu(_p(x), nt, _p(wgu), _p(wd), P, I, _p(y))
    return y


def layer_forward(shape, w: dict, R: int, T: int, ctx, h_in, k_cache, v_cache, cap: int,
                  eps: float = 1e-6, use_norm: bool = True, stages: bool = True, tree=None,
                  act_fp4: bool = False):
    """One layer on the CPU. shape: object with H, nq, nkv, d, E, k, P, I.
    k_cache / v_cache ([R][nkv][cap][d] uint16) are updated in place (KV write).
    Returns (h_out fp64 [R*T][H], stages dict or None)."""
    s = shape
    NT = R * T
    L = OrcLayer(hidden=s.H, n_q_heads=s.nq, n_kv_heads=s.nkv, head_dim=s.d, n_experts=s.E,
                 top_k=s.k, pool_dim=s.P, expert_inter=s.I, window=int(w["window"]),
                 kv_capacity=cap, rms_eps=eps, use_norm=1 if use_norm else 0, act_fp4=1 if act_fp4 else 0)
    keep = {}
    for name in ("w_qkv", "w_o", "w_router", "b_router", "w_pool", "w_unpool", "g_attn", "g_moe",
                 "e_gate_up", "e_gate_up_scale", "e_down", "e_down_scale", "e_tensor_scale"):
        a = w.get(name)
        if a is not None:
            a = np.ascontiguousarray(a)
            keep[name] = a
        setattr(L, name, _p(a))
    ctx_a = np.ascontiguousarray(np.asarray(ctx, np.int32))
    h = np.ascontiguousarray(h_in, np.float64)
    out = np.empty((NT, s.H), np.float64)
    st = None
    stp = None
    if stages:
        st = {
            "q": np.empty((NT, s.nq * s.d)), "k_new": np.empty((NT, s.nkv * s.d)),
            "v_new": np.empty((NT, s.nkv * s.d)), "attn": np.empty((NT, s.nq * s.d)),
            "h1": np.empty((NT, s.H)), "n2_f32": np.empty((NT, s.H), np.float32),
            "logits": np.empty((NT, s.E), np.float32), "ids": np.empty((NT, s.k), np.int32),
            "gates": np.empty((NT, s.k)), "p": np.empty((NT, s.P)), "acc": np.empty((NT, s.P)),
        }
        stp = OrcStages(**{k: _p(v) for k, v in st.items()})
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    tr = _tree_arg(tree, R * T)
    rc = lib().orc_layer_forward(ctypes.byref(L), R, T, _p(ctx_a), _p(tr), _p(h), _p(k_cache), _p(v_cache),
                                 _p(out), ctypes.byref(stp) if stp is not None else None)
    if rc != 0:
        raise ValueError("orc_layer_forward rejected its arguments")
    return out, st

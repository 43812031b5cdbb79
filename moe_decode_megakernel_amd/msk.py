"""Thin ctypes binding of libmsk.so (include/msk.h): the same entry points
under the same names, plus helpers that marshal torch tensors into the ABI
structs. All compute runs in the library's HIP kernels; there is no fallback.
"""
import ctypes
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmsk.so")

i32, u32, f32, vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p

MSK_OK, MSK_E_INVALID, MSK_E_SHAPE, MSK_E_ALIGN, MSK_E_STATE, MSK_E_CAPACITY, MSK_E_HIP, MSK_E_TIMEOUT = range(8)
STATUS_NAMES = ["MSK_OK", "MSK_E_INVALID", "MSK_E_SHAPE", "MSK_E_ALIGN", "MSK_E_STATE",
                "MSK_E_CAPACITY", "MSK_E_HIP", "MSK_E_TIMEOUT"]
MSK_FLAG_NO_NORM = 0x1
MSK_FLAG_ACT_FP4 = 0x2
MSK_FLAG_KV_PREFETCH = 0x4

EXPORTS = ("msk_workspace_bytes", "msk_create", "msk_create_static", "msk_load_layer", "msk_verify_layer",
           "msk_verify_step", "msk_synchronize", "msk_destroy", "msk_down_scale_bytes",
           "msk_pack_down_scale", "msk_last_error")


class msk_config(ctypes.Structure):
    _fields_ = [("hidden", i32), ("n_q_heads", i32), ("n_kv_heads", i32), ("head_dim", i32),
                ("n_experts", i32), ("top_k", i32), ("pool_dim", i32), ("expert_inter", i32),
                ("n_layers", i32), ("max_tokens", i32), ("max_requests", i32), ("kv_capacity", i32),
                ("rms_eps", f32), ("flags", u32), ("expert_prefetch", i32)]


LAYER_PTRS = ("w_qkv", "w_o", "w_router", "b_router", "w_pool", "w_unpool", "g_attn", "g_moe",
              "e_gate_up", "e_gate_up_scale", "e_down", "e_down_scale", "e_tensor_scale",
              "k_cache", "v_cache")


class msk_layer_desc(ctypes.Structure):
    _fields_ = [("window", i32)] + [(n, vp) for n in LAYER_PTRS]


DEBUG_PTRS = ("q", "k_new", "v_new", "attn", "h1", "n2", "logits", "p", "acc")


class msk_debug(ctypes.Structure):
    _fields_ = [(n, vp) for n in DEBUG_PTRS] + [("dq_expert", i32), ("dq_gate_up", vp), ("dq_down", vp),
                                                ("act", vp), ("act_codes", vp), ("act_scales", vp),
                                                ("act_codes_all", vp), ("act_scales_all", vp)]


class msk_io(ctypes.Structure):
    _fields_ = [("n_requests", i32), ("n_tokens", i32), ("ctx_len", vp),
                ("h_in", vp), ("h_out", vp), ("expert_ids", vp), ("gates", vp),
                ("debug", ctypes.POINTER(msk_debug)), ("prefetch_ids", vp), ("trace", vp),
                ("tree_mask", vp), ("layer_out", vp)]


TRACE_SLOTS = ["start", "qkv_own", "qkv_own_bar", "attn_q", "attn_kv", "attn", "attn_bar", "merge", "merge_bar", "oproj_fill",
               "oproj", "oproj_bar", "pool_fill", "router_pool", "router_pool_bar", "routing", "gemm1",
               "gemm1_bar", "gemm2", "gemm2_bar", "unpool_fill", "unpool", "unpool_bar", "qkv_fill", "qkv_next"]
MAX_GRID = 256
# tokens of one MFMA row tile: a call's requests run in passes of
# max(1, MAX_TOKENS_PER_PASS // tokens) whole requests
MAX_TOKENS_PER_PASS = 16


_lib = None


def lib():
    """Load libmsk.so; raises if the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with moe_decode_megakernel_amd/build.py "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        L.msk_workspace_bytes.argtypes = [ctypes.POINTER(msk_config)]
        L.msk_workspace_bytes.restype = ctypes.c_size_t
        L.msk_create.argtypes = [ctypes.POINTER(msk_config), vp, ctypes.c_size_t, ctypes.POINTER(vp)]
        L.msk_create.restype = i32
        L.msk_create_static.argtypes = [ctypes.POINTER(msk_config), ctypes.POINTER(vp)]
        L.msk_create_static.restype = i32
        L.msk_load_layer.argtypes = [vp, i32, ctypes.POINTER(msk_layer_desc)]
        L.msk_load_layer.restype = i32
        L.msk_verify_layer.argtypes = [vp, i32, ctypes.POINTER(msk_io), vp]
        L.msk_verify_layer.restype = i32
        L.msk_verify_step.argtypes = [vp, ctypes.POINTER(msk_io), vp]
        L.msk_verify_step.restype = i32
        L.msk_synchronize.argtypes = [vp]
        L.msk_synchronize.restype = i32
        L.msk_destroy.argtypes = [vp]
        L.msk_destroy.restype = i32
        L.msk_down_scale_bytes.argtypes = [i32, i32, i32]
        L.msk_down_scale_bytes.restype = ctypes.c_size_t
        L.msk_pack_down_scale.argtypes = [vp, vp, i32, i32, i32, vp]
        L.msk_pack_down_scale.restype = i32
        L.msk_last_error.argtypes = [vp]
        L.msk_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


class MskError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < 8 else status}: {msg}")
        self.status = status


# --- the C entry points under their own names -------------------------------
def msk_workspace_bytes(cfg: msk_config) -> int:
    return lib().msk_workspace_bytes(ctypes.byref(cfg))


def msk_create(cfg: msk_config, workspace_ptr: int, nbytes: int):
    h = vp()
    st = lib().msk_create(ctypes.byref(cfg), vp(workspace_ptr), nbytes, ctypes.byref(h))
    if st != MSK_OK:
        raise MskError(st, msk_last_error(None))
    return h


def msk_create_static(cfg: msk_config):
    h = vp()
    st = lib().msk_create_static(ctypes.byref(cfg), ctypes.byref(h))
    if st != MSK_OK:
        raise MskError(st, msk_last_error(None))
    return h


MSK_STATIC_WORKSPACE_BYTES = 32 << 20


def msk_load_layer(h, layer: int, desc: msk_layer_desc) -> int:
    return lib().msk_load_layer(h, layer, ctypes.byref(desc))


def msk_verify_layer(h, layer: int, io: msk_io, stream: int) -> int:
    return lib().msk_verify_layer(h, layer, ctypes.byref(io), vp(stream))


def msk_verify_step(h, io: msk_io, stream: int) -> int:
    return lib().msk_verify_step(h, ctypes.byref(io), vp(stream))


def msk_synchronize(h) -> int:
    return lib().msk_synchronize(h)


def msk_destroy(h) -> int:
    return lib().msk_destroy(h)


def msk_down_scale_bytes(n_experts: int, pool_dim: int, expert_inter: int) -> int:
    return lib().msk_down_scale_bytes(n_experts, pool_dim, expert_inter)


def msk_pack_down_scale(src_ptr: int, dst_ptr: int, n_experts: int, pool_dim: int, expert_inter: int,
                        stream: int) -> int:
    return lib().msk_pack_down_scale(vp(src_ptr), vp(dst_ptr), n_experts, pool_dim, expert_inter, vp(stream))


def msk_last_error(h) -> str:
    s = lib().msk_last_error(h)
    return s.decode() if s else ""


# --- marshalling helpers (torch tensors -> ABI structs) ----------------------
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# Experts prefetched per layer when the caller does not say. On MI355X at the
# 62-layer shape, 6 to 10 give the same, shortest step; 14 (the count the
# pages name) is 0.06 ms slower, as the workgroups that read them finish
# their share of the merge later.
DEFAULT_EXPERT_PREFETCH = 8


def make_config(w, n_layers=None, max_tokens=None, max_requests=None, flags=0, expert_prefetch=None) -> msk_config:
    if expert_prefetch is None:
        expert_prefetch = min(DEFAULT_EXPERT_PREFETCH, w.E)
    return msk_config(hidden=w.H, n_q_heads=w.nq, n_kv_heads=w.nkv, head_dim=w.d, n_experts=w.E,
                      top_k=w.k, pool_dim=w.P, expert_inter=w.I,
                      n_layers=w.n_layers if n_layers is None else n_layers,
                      max_tokens=w.T if max_tokens is None else max_tokens,
                      max_requests=w.R if max_requests is None else max_requests,
                      kv_capacity=w.cap, rms_eps=w.eps, flags=flags, expert_prefetch=expert_prefetch)


def make_layer_desc(t: Dict, window: int) -> msk_layer_desc:
    d = msk_layer_desc(window=window)
    for n in LAYER_PTRS:
        setattr(d, n, _ptr(t.get(n)))
    return d


def make_io(n_requests, n_tokens, ctx, h_in, h_out, expert_ids=None, gates=None,
            debug: Optional[msk_debug] = None, trace=None, prefetch_ids=None, tree_mask=None, layer_out=None):
    """ctx: device int32 tensor [n_requests], or a host sequence (copied to a
    device tensor on h_in's device, kept alive by the returned struct).
    tree_mask: device uint16/int16 tensor [n_requests][n_tokens], a host
    array-like of ancestor bitmasks (copied likewise), or None (the chain)."""
    import torch
    dev = h_in.device
    if not torch.is_tensor(ctx):
        ctx = torch.tensor([int(c) for c in ctx], dtype=torch.int32, device=dev)
    if tree_mask is not None and not torch.is_tensor(tree_mask):
        flat = [int(x) for row in tree_mask for x in (row if hasattr(row, "__len__") else [row])]
        if len(flat) != n_requests * n_tokens:
            raise ValueError("tree_mask needs n_requests * n_tokens entries")
        tree_mask = torch.tensor([x - 65536 if x >= 32768 else x for x in flat], dtype=torch.int16, device=dev)
    io = msk_io(n_requests=n_requests, n_tokens=n_tokens, ctx_len=_ptr(ctx),
                h_in=_ptr(h_in), h_out=_ptr(h_out), expert_ids=_ptr(expert_ids), gates=_ptr(gates),
                debug=ctypes.pointer(debug) if debug is not None else None, prefetch_ids=_ptr(prefetch_ids),
                trace=_ptr(trace), tree_mask=_ptr(tree_mask), layer_out=_ptr(layer_out))
    io._keep = (ctx, debug, tree_mask)
    return io


def make_debug(t: Dict, dq_expert: int = -1) -> msk_debug:
    d = msk_debug(dq_expert=dq_expert, dq_gate_up=_ptr(t.get("dq_gate_up")), dq_down=_ptr(t.get("dq_down")),
                  act=_ptr(t.get("act")), act_codes=_ptr(t.get("act_codes")), act_scales=_ptr(t.get("act_scales")),
                  act_codes_all=_ptr(t.get("act_codes_all")), act_scales_all=_ptr(t.get("act_scales_all")))
    for n in DEBUG_PTRS:
        setattr(d, n, _ptr(t.get(n)))
    return d


class Handle:
    """Owns a workspace tensor and a library handle (convenience wrapper)."""

    def __init__(self, cfg: msk_config, device="cuda", static=False):
        """static: use the library's own static workspace (msk_create_static)
        instead of a workspace tensor."""
        import torch
        self.cfg = cfg
        self.layers = {}
        self.workspace = None
        if static:
            self.h = msk_create_static(cfg)
            return
        n = msk_workspace_bytes(cfg)
        if n == 0:
            raise MskError(MSK_E_SHAPE, "configuration rejected by msk_workspace_bytes")
        self.workspace = torch.empty(n + 256, dtype=torch.uint8, device=device)
        base = self.workspace.data_ptr()
        self.ws_ptr = (base + 255) // 256 * 256
        self.h = msk_create(cfg, self.ws_ptr, n)

    def check(self, st):
        if st != MSK_OK:
            raise MskError(st, msk_last_error(self.h))

    def pack_down_scale(self, scale, stream=None):
        """Tiled copy of a row-major [E][P][I/16] down-projection scale tensor
        (the order msk_load_layer takes), written by msk_pack_down_scale on
        the current stream."""
        import torch
        c = self.cfg
        n = msk_down_scale_bytes(c.n_experts, c.pool_dim, c.expert_inter)
        if n == 0:
            raise MskError(MSK_E_SHAPE, "msk_down_scale_bytes rejected the shape")
        out = torch.empty(n, dtype=torch.uint8, device=scale.device)
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        st = msk_pack_down_scale(scale.data_ptr(), out.data_ptr(), c.n_experts, c.pool_dim, c.expert_inter, s)
        if st != MSK_OK:
            raise MskError(st, msk_last_error(None))
        return out

    def load_layer(self, layer, tensors: Dict, window: int):
        """Register a layer whose tensors use the row-major layouts (the
        down-projection scales are packed here into a tensor the handle
        keeps)."""
        t = dict(tensors)
        t["e_down_scale"] = self.pack_down_scale(tensors["e_down_scale"])
        self.layers[layer] = t
        self.check(msk_load_layer(self.h, layer, make_layer_desc(t, window)))

    def verify_layer(self, layer, io, stream=None):
        import torch
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        self.check(msk_verify_layer(self.h, layer, io, s))

    def verify_step(self, io, stream=None):
        import torch
        s = torch.cuda.current_stream().cuda_stream if stream is None else stream
        self.check(msk_verify_step(self.h, io, s))

    def synchronize(self):
        """Wait for the last call and raise MskError if the device reported one."""
        self.check(msk_synchronize(self.h))

    def close(self):
        if self.h:
            msk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

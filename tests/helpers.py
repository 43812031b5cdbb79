"""Shared helpers of the GPU parity tests: upload a seeded layer, run it
through the C ABI with stage dumps, and run the oracle on the same inputs."""
import sys

import numpy as np

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    """max |got - ref| / RMS(ref)."""
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / rms) if rms > 0 else float(np.max(np.abs(got - ref)))


def bf16_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


class GpuLayerRun:
    """One standalone layer on the GPU with every stage dumped."""

    def __init__(self, w, lw, k, v, h, flags=0, dq_expert=-1, ctx=None):
        import torch
        self.torch = torch
        dev = "cuda"
        self.w = w
        self.handle = msk.Handle(msk.make_config(w, n_layers=1, flags=flags))
        self.t = synth.to_device(lw, dev)
        self.t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
        self.t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
        self.handle.load_layer(0, self.t, int(lw["window"]))
        NT = w.NT
        f32 = dict(dtype=torch.float32, device=dev)
        self.h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
        self.h_out = torch.zeros((NT, w.H), **f32)
        self.ids = torch.zeros((NT, w.k), dtype=torch.int32, device=dev)
        self.gates = torch.zeros((NT, w.k), **f32)
        self.dbg = {
            "q": torch.zeros((NT, w.Dq), **f32), "k_new": torch.zeros((NT, w.Dkv), **f32),
            "v_new": torch.zeros((NT, w.Dkv), **f32), "attn": torch.zeros((NT, w.Dq), **f32),
            "h1": torch.zeros((NT, w.H), **f32), "n2": torch.zeros((NT, w.H), **f32),
            "logits": torch.zeros((NT, w.E), **f32), "p": torch.zeros((NT, w.P), **f32),
            "acc": torch.zeros((NT, w.P), **f32),
            "dq_gate_up": torch.zeros((2 * w.I, w.P), dtype=torch.int16, device=dev),
            "dq_down": torch.zeros((w.P, w.I), dtype=torch.int16, device=dev),
            "act": torch.zeros((NT, w.I), **f32),
            "act_codes": torch.zeros((NT, w.I // 2), dtype=torch.uint8, device=dev),
            "act_scales": torch.zeros((NT, w.I // 16), dtype=torch.uint8, device=dev),
            "act_codes_all": torch.zeros((w.E, NT, w.I // 2), dtype=torch.uint8, device=dev),
            "act_scales_all": torch.zeros((w.E, NT, w.I // 16), dtype=torch.uint8, device=dev),
        }
        self.ctx = [w.ctx] * w.R if ctx is None else list(ctx)
        self.dq_expert = dq_expert

    def run(self, debug=True, tree=None, trace=None):
        """One msk_verify_layer call; debug=False runs the production kernel
        (the benchmark's variant) with no stage dumps. Device-side errors are
        raised (msk_synchronize)."""
        torch = self.torch
        d = msk.make_debug(self.dbg, self.dq_expert) if debug else None
        io = msk.make_io(self.w.R, self.w.T, self.ctx, self.h_in, self.h_out, self.ids, self.gates, d,
                         tree_mask=tree, trace=trace)
        self.handle.verify_layer(0, io)
        self.handle.synchronize()
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in self.dbg.items()}
        out["h_out"] = self.h_out.cpu().numpy()
        out["ids"] = self.ids.cpu().numpy()
        out["gates"] = self.gates.cpu().numpy()
        out["k_cache"] = self.t["k_cache"].cpu().numpy().view(np.uint16)
        out["v_cache"] = self.t["v_cache"].cpu().numpy().view(np.uint16)
        return out

    def close(self):
        self.handle.close()


def oracle_layer(w, lw, k, v, h, use_norm=True, ctx=None, tree=None, act_fp4=False):
    ctx = [w.ctx] * w.R if ctx is None else list(ctx)
    kk, vv = k.copy(), v.copy()
    out, st = orc.layer_forward(w, lw, w.R, w.T, ctx, np.asarray(h, np.float64), kk, vv, w.cap,
                                eps=w.eps, use_norm=use_norm, tree=tree, act_fp4=act_fp4)
    st["h_out"] = out
    st["k_cache"] = kk
    st["v_cache"] = vv
    return st


def routing_margins(logits, k):
    """Per token: gap between the k-th and (k+1)-th largest logit."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=1)
    return s[:, k - 1] - s[:, k]


def routing_mismatches(gpu_ids, logits, k, thr):
    """Tokens whose GPU selection disagrees with the oracle's logits beyond
    near-ties: the selected set must equal the oracle's top-k wherever the
    k-th/(k+1)-th margin exceeds thr, and consecutive GPU ranks must not
    invert two logits that differ by more than thr (the ranking is by value,
    ties to the lower index; values closer than thr may legitimately swap)."""
    bad = []
    lg_all = np.asarray(logits, np.float64)
    for t in range(lg_all.shape[0]):
        lg = lg_all[t]
        ref = np.lexsort((np.arange(lg.size), -lg))[:k]
        s = -np.sort(-lg)
        margin = s[k - 1] - s[k]
        ids = np.asarray(gpu_ids[t])
        if margin > thr and set(ids.tolist()) != set(ref.tolist()):
            bad.append(t)
            continue
        if any(lg[ids[r + 1]] - lg[ids[r]] > thr for r in range(k - 1)):
            bad.append(t)
    return bad


def random_tree(T, seed):
    """Seeded tree of T verify tokens (ancestor bitmasks, self included)."""
    return synth.verify_tree(T, seed)


def teacher_forced_layer(w, layer, h_prev, gpu_out, gpu_ids, label, tol=2e-2, route_thr=2e-3, ctx=None):
    """The oracle's layer `layer` fed the GPU's own input residual h_prev
    (teacher forcing), against the GPU's output residual of that layer.

    Routing: the GPU's expert set of a token must equal the oracle's wherever
    the oracle's k-th/(k+1)-th logit margin exceeds route_thr, and ranks
    closer than route_thr may swap (R20). The output residual is gated at
    max|err| <= tol * RMS(oracle output) over the tokens whose expert sets
    agree (a near-tie selection legitimately changes a token's output); at
    most max(2, NT/16) tokens may be near-ties. Only the experts either side selects
    are generated. Returns (max error / RMS, error on the layer delta / RMS
    of the delta, number of near-tie tokens, the oracle's K and V caches
    after its KV write)."""
    ctx = [w.ctx] * w.R if ctx is None else list(ctx)
    need = set(np.unique(gpu_ids).tolist())
    h64 = np.asarray(h_prev, np.float64)
    for _ in range(3):
        lw = synth.layer_weights(w, layer, experts=sorted(need))
        k, v = synth.kv_cache(w, layer)
        out, st = orc.layer_forward(w, lw, w.R, w.T, ctx, h64, k, v, w.cap, eps=w.eps)
        extra = set(np.unique(st["ids"]).tolist()) - need
        if not extra:
            break
        need |= extra
    else:
        raise AssertionError(f"{label}: expert sets did not settle")
    K = w.k
    bad = routing_mismatches(gpu_ids, st["logits"], K, route_thr)
    assert not bad, f"{label}: routing differs beyond near-ties for tokens {bad}"
    same = np.array([set(gpu_ids[t].tolist()) == set(st["ids"][t].tolist()) for t in range(w.NT)])
    n_tie = int((~same).sum())
    assert n_tie <= max(2, w.NT // 16), f"{label}: {n_tie} near-tie tokens"
    ref = np.asarray(out, np.float64)
    got = np.asarray(gpu_out, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got[same] - ref[same]))) / rms
    d_ref = ref - h64
    d_rms = float(np.sqrt(np.mean(d_ref * d_ref)))
    derr = float(np.max(np.abs((got - h64)[same] - d_ref[same]))) / d_rms
    say(f"[{label}] layer {layer} (window {w.windows[layer]}): h_out max|err|/RMS {err:.2e}, "
        f"on the layer delta {derr:.2e}, near-tie tokens {n_tie}, distinct experts {len(np.unique(gpu_ids))}")
    assert err <= tol, f"{label}: layer {layer} output error {err:.3e} > {tol}"
    return err, derr, n_tie, k, v

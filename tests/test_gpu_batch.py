"""Several requests in one verify call: 4 requests x 16 tokens (64 tokens, the
larger-batch configuration) and 4 x 8 tokens with different context lengths.
The library runs a call's requests in passes of at most 16 tokens. Each
request uses its own cache slice and positions; every token's MoE output
depends only on that token. The oracle runs all requests jointly (attention
per request, MoE over all tokens at once), so agreement also checks that
requests stay independent."""
from dataclasses import replace

import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc
from tests.helpers import bf16_to_f64, rel_err, routing_mismatches, say, teacher_forced_layer

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _run_stack(w, ctx, h, dev="cuda"):
    import torch
    handle = msk.Handle(msk.make_config(w))
    layers = [synth.layer_weights(w, l) for l in range(w.n_layers)]
    caches = [synth.kv_cache(w, l) for l in range(w.n_layers)]
    tens = []
    for l in range(w.n_layers):
        t = synth.to_device(layers[l], dev)
        t["k_cache"] = torch.from_numpy(caches[l][0].view(np.int16)).to(dev)
        t["v_cache"] = torch.from_numpy(caches[l][1].view(np.int16)).to(dev)
        handle.load_layer(l, t, int(layers[l]["window"]))
        tens.append(t)
    h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
    h_out = torch.zeros_like(h_in)
    ids = torch.zeros((w.n_layers, w.NT, w.k), dtype=torch.int32, device=dev)
    io = msk.make_io(w.R, w.T, ctx, h_in, h_out, ids)
    handle.verify_step(io)
    handle.synchronize()
    torch.cuda.synchronize()
    out = h_out.cpu().numpy()
    gids = ids.cpu().numpy()
    kv = [(t["k_cache"].cpu().numpy().view(np.uint16), t["v_cache"].cpu().numpy().view(np.uint16)) for t in tens]
    handle.close()
    return out, gids, kv, layers, caches


@pytest.mark.parametrize("R,T,ctx", [(4, 16, [64, 64, 64, 64]), (4, 8, [64, 40, 10, 57])])
def test_tiny_requests_match_joint_oracle(R, T, ctx):
    base = synth.small_stack(2)
    w = replace(base, name=f"tiny_r{R}_t{T}", R=R, T=T)
    h = synth.h_input(w)
    say(f"[batch] tiny stack, {R} requests x {T} tokens, ctx {ctx}")
    out, gids, kv, layers, caches = _run_stack(w, ctx, h)
    hh = h.astype(np.float64)
    for l in range(w.n_layers):
        k, v = caches[l][0].copy(), caches[l][1].copy()
        hh, st = orc.layer_forward(w, layers[l], w.R, w.T, ctx, hh, k, v, w.cap, eps=w.eps)
        assert not routing_mismatches(gids[l], st["logits"], w.k, 1e-3), f"layer {l} routing"
        for r in range(R):
            rows = slice(ctx[r], ctx[r] + T)
            assert rel_err(bf16_to_f64(kv[l][0][r, :, rows]), bf16_to_f64(k[r, :, rows])) < TOL
            # rows other than the request's verify slots are untouched
            keep = np.ones(w.cap, bool)
            keep[rows] = False
            assert np.array_equal(kv[l][0][r][:, keep], caches[l][0][r][:, keep]), (l, r)
    e = rel_err(out, hh)
    say(f"[batch] h_out rel err {e:.2e}")
    assert e < TOL


def test_batch4_step62_full_size():
    """4 requests x 16 tokens through the 62-layer stack at working size,
    65536-token caches per request, uniform routing. Each layer's output
    residual is returned (msk_io.layer_out); the oracle runs layers 0
    (sliding window, first launch), 3 (global, middle launch) and 61 (global,
    last launch) teacher-forced on the GPU's input residual of that layer, all
    four requests jointly (attention per request, MoE over the 64 tokens), and
    each output is gated at max|err| <= 2e-2 * RMS. A repeated step gives
    identical bytes."""
    import torch
    w = synth.WORKLOADS["batch4_step62"]
    dev = "cuda"
    say("[batch4] filling 62 layers (weights + 4 x 65552-row caches) on the device")
    handle = msk.Handle(msk.make_config(w))
    layers = []
    for l in range(w.n_layers):
        t = synth.device_layer(w, l, dev)
        handle.load_layer(l, t, int(w.windows[l]))
        layers.append(t)
    h = synth.h_input(w, 0)
    h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
    L, NT, K = w.n_layers, w.NT, w.k
    outs, ids_runs, lo_out = [], [], None
    for run in range(2):
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((L, NT, K), dtype=torch.int32, device=dev)
        lo = torch.zeros((L, NT, w.H), dtype=torch.float32, device=dev) if run == 0 else None
        io = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_out, ids, layer_out=lo)
        say(f"[batch4] gpu step, run {run}")
        handle.verify_step(io)
        handle.synchronize()
        torch.cuda.synchronize()
        outs.append(h_out.cpu().numpy())
        ids_runs.append(ids.cpu().numpy())
        if lo is not None:
            lo_out = lo.cpu().numpy()
    handle.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(ids_runs[0], ids_runs[1])
    assert np.array_equal(lo_out[L - 1], outs[0])
    assert np.all(np.isfinite(lo_out))
    n_sel = [len(np.unique(ids_runs[0][l])) for l in range(L)]
    say(f"[batch4] distinct experts per layer: mean {np.mean(n_sel):.1f}, min {min(n_sel)}, max {max(n_sel)}")
    del layers
    torch.cuda.empty_cache()
    errs = {}
    for l in (0, 3, 61):
        h_prev = h if l == 0 else lo_out[l - 1]
        errs[l] = teacher_forced_layer(w, l, h_prev, lo_out[l], ids_runs[0][l], "batch4", tol=TOL)[:3]
    say("[batch4] per-layer h_out error / RMS: " + " ".join(f"{l}:{e[0]:.2e}" for l, e in errs.items()))

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
from tests.helpers import bf16_to_f64, rel_err, routing_mismatches, say

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
    65536-token caches per request, uniform routing: the oracle's joint chain
    over the first two layers, and run-to-run identity of the whole step."""
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
    outs, ids_runs = [], []
    rows = slice(w.ctx, w.ctx + w.T)
    kv0 = None
    for run in range(2):
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((L, NT, K), dtype=torch.int32, device=dev)
        io = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_out, ids)
        say(f"[batch4] gpu step, run {run}")
        handle.verify_step(io)
        torch.cuda.synchronize()
        outs.append(h_out.cpu().numpy())
        ids_runs.append(ids.cpu().numpy())
        if kv0 is None:
            kv0 = [(layers[l]["k_cache"][:, :, rows].cpu().numpy().view(np.uint16),
                    layers[l]["v_cache"][:, :, rows].cpu().numpy().view(np.uint16)) for l in range(2)]
    handle.close()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(ids_runs[0], ids_runs[1])
    assert np.all(np.isfinite(outs[0]))
    n_sel = [len(np.unique(ids_runs[0][l])) for l in range(L)]
    say(f"[batch4] distinct experts per layer: mean {np.mean(n_sel):.1f}, min {min(n_sel)}, max {max(n_sel)}")
    del layers
    torch.cuda.empty_cache()
    hh = h.astype(np.float64)
    for l in range(2):
        say(f"[batch4] oracle layer {l}")
        lw = synth.layer_weights(w, l)
        k, v = synth.kv_cache(w, l)
        hh, st = orc.layer_forward(w, lw, w.R, w.T, [w.ctx] * w.R, hh, k, v, w.cap, eps=w.eps)
        bad = routing_mismatches(ids_runs[0][l], st["logits"], K, 1e-3 if l == 0 else 4e-3)
        say(f"[batch4] layer {l}: routing mismatches {bad}")
        assert not bad
        for name, got, ref in (("K", kv0[l][0], k[:, :, rows]), ("V", kv0[l][1], v[:, :, rows])):
            g64, r64 = bf16_to_f64(got), bf16_to_f64(ref)
            rms = float(np.sqrt(np.mean(r64 * r64)))
            bound = TOL * rms + np.ldexp(1.0, -7) * np.abs(r64)
            assert float(np.max(np.abs(g64 - r64) - bound)) <= 0.0, f"layer {l}: {name} write"
        del lw, k, v

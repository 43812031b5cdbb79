"""GPU parity of the whole verify step (msk_verify_step: one launch per layer
boundary) against the oracle's layer-by-layer chain."""
import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc
from tests.helpers import bf16_to_f64, rel_err, routing_margins, routing_mismatches, say

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _run_step(w, layers, caches, h, n_runs=1):
    import torch
    dev = "cuda"
    handle = msk.Handle(msk.make_config(w))
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
    gates = torch.zeros((w.n_layers, w.NT, w.k), dtype=torch.float32, device=dev)
    io = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_out, ids, gates)
    outs = []
    for _ in range(n_runs):
        handle.verify_step(io)
        torch.cuda.synchronize()
        outs.append(h_out.cpu().numpy().copy())
    res = {"h_out": outs, "ids": ids.cpu().numpy(), "gates": gates.cpu().numpy(),
           "k": [t["k_cache"].cpu().numpy().view(np.uint16) for t in tens],
           "v": [t["v_cache"].cpu().numpy().view(np.uint16) for t in tens]}
    handle.close()
    return res


def test_small_stack_step_matches_oracle_chain():
    w = synth.small_stack(4)
    layers = [synth.layer_weights(w, l) for l in range(w.n_layers)]
    caches = [synth.kv_cache(w, l) for l in range(w.n_layers)]
    h = synth.h_input(w)
    say("[stack4] gpu step")
    g = _run_step(w, layers, [(k.copy(), v.copy()) for k, v in caches], h, n_runs=2)
    assert np.array_equal(g["h_out"][0], g["h_out"][1]), "two identical steps differ"
    say("[stack4] oracle chain")
    hh = h.astype(np.float64)
    for l in range(w.n_layers):
        k, v = caches[l]
        hh, st = orc.layer_forward(w, layers[l], w.R, w.T, [w.ctx], hh, k, v, w.cap, eps=w.eps)
        m = routing_margins(st["logits"], w.k)
        say(f"[stack4] layer {l}: min routing margin {m.min():.2e}")
        assert not routing_mismatches(g["ids"][l], st["logits"], w.k, 1e-3), f"layer {l} routing differs"
        rows = slice(w.ctx, w.ctx + w.T)
        assert rel_err(bf16_to_f64(g["k"][l][:, :, rows]), bf16_to_f64(k[:, :, rows])) < TOL
        assert np.array_equal(g["k"][l][:, :, :w.ctx], caches[l][0][:, :, :w.ctx])
    e = rel_err(g["h_out"][0], hh)
    say(f"[stack4] h_out rel err {e:.2e}")
    assert e < TOL

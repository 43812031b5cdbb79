"""Full-size parity of the 62-layer verify step (16 tokens, hidden 4096, 46
sliding-window layers of window 2048 + 16 global layers, 16384-token caches,
top-8 of 256 NVFP4 experts, Zipf-skewed routing), run exactly as the benchmark
runs it: one msk_verify_step over 62 resident layer launches, production
kernel variants (first, middle and last launch).

Each layer's output residual is returned (msk_io.layer_out). The oracle runs
a set of layers teacher-forced on the GPU's own input residual of that layer
(layer 0 on the step's input): sliding-window layers 0, 1, 30, 60 and global
layers 3, 31, 59, 61, covering the first launch (its own QKV projection), the
middle launches (QKV projected at the previous launch's tail) and the last
launch. Each is gated at max|err| <= 2e-2 * RMS, with routing checked per R20.
The whole step is also checked by properties at any size: repeated calls and
the self-timing variant give identical bytes, cache rows outside the verify
slots are unchanged, and the K/V rows each checked layer writes agree with
the oracle's.
"""
import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from tests.helpers import bf16_to_f64, say, teacher_forced_layer

pytestmark = pytest.mark.gpu

TOL = 2e-2
CHECK_LAYERS = (0, 1, 3, 30, 31, 59, 60, 61)


def test_step62_full_size_teacher_forced():
    import torch
    w = synth.WORKLOADS["step62"]
    dev = "cuda"
    say("[step62] filling 62 layers on the device")
    handle = msk.Handle(msk.make_config(w))
    layers = []
    for l in range(w.n_layers):
        t = synth.device_layer(w, l, dev)
        handle.load_layer(l, t, int(w.windows[l]))
        layers.append(t)
    h = synth.h_input(w, 0)
    h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
    L, NT, K = w.n_layers, w.NT, w.k
    rows = slice(w.ctx, w.ctx + w.T)
    probe = torch.tensor([0, 1, w.ctx // 2, w.ctx - 2, w.ctx - 1], device=dev)
    before = [(t["k_cache"][:, :, probe].cpu().numpy(), t["v_cache"][:, :, probe].cpu().numpy()) for t in layers]

    runs = []
    for run, mode in enumerate(("layer_out", "plain", "trace")):
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((L, NT, K), dtype=torch.int32, device=dev)
        lo = torch.zeros((L, NT, w.H), dtype=torch.float32, device=dev) if mode == "layer_out" else None
        tr = torch.zeros((L, msk.MAX_GRID, len(msk.TRACE_SLOTS)), dtype=torch.int64, device=dev) if mode == "trace" else None
        io = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_out, ids, trace=tr, layer_out=lo)
        say(f"[step62] gpu step, run {run} ({mode})")
        handle.verify_step(io)
        handle.synchronize()
        torch.cuda.synchronize()
        r = {"h_out": h_out.cpu().numpy(), "ids": ids.cpu().numpy()}
        if lo is not None:
            r["layer_out"] = lo.cpu().numpy()
            r["kv"] = {l: (layers[l]["k_cache"][:, :, rows].cpu().numpy().view(np.uint16),
                           layers[l]["v_cache"][:, :, rows].cpu().numpy().view(np.uint16)) for l in CHECK_LAYERS}
        if tr is not None:
            st = tr.cpu().numpy()
            assert np.all(st[:, :, 0] != 0), "every workgroup of every launch stamps its start"
        runs.append(r)
    handle.close()

    a = runs[0]
    for r, name in ((runs[1], "repeat"), (runs[2], "self-timing variant")):
        assert np.array_equal(a["h_out"], r["h_out"]), f"{name}: h_out differs"
        assert np.array_equal(a["ids"], r["ids"]), f"{name}: expert ids differ"
    assert np.array_equal(a["layer_out"][L - 1], a["h_out"])
    assert np.all(np.isfinite(a["layer_out"]))
    for l, t in enumerate(layers):
        kb, vb = before[l]
        assert np.array_equal(t["k_cache"][:, :, probe].cpu().numpy(), kb), f"layer {l}: K rows outside the verify slots changed"
        assert np.array_equal(t["v_cache"][:, :, probe].cpu().numpy(), vb), f"layer {l}: V rows outside the verify slots changed"
    del layers
    torch.cuda.empty_cache()

    errs = {}
    for l in CHECK_LAYERS:
        h_prev = h if l == 0 else a["layer_out"][l - 1]
        errs[l] = teacher_forced_layer(w, l, h_prev, a["layer_out"][l], a["ids"][l], "step62", tol=TOL)
        # the K/V rows the step wrote for layer l against the oracle's own
        # projection of the same input (float tolerance plus one bf16 ulp, R19)
        k, v = errs[l][3], errs[l][4]
        for name, got, ref in (("K", a["kv"][l][0], k[:, :, rows]), ("V", a["kv"][l][1], v[:, :, rows])):
            g64, r64 = bf16_to_f64(got), bf16_to_f64(ref)
            rms = float(np.sqrt(np.mean(r64 * r64)))
            bound = TOL * rms + np.ldexp(1.0, -7) * np.abs(r64)
            assert float(np.max(np.abs(g64 - r64) - bound)) <= 0.0, f"layer {l}: {name} write"
        errs[l] = errs[l][:3]
    say("[step62] per-layer h_out error / RMS: " + " ".join(f"{l}:{e[0]:.2e}" for l, e in errs.items()))

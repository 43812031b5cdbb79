"""A verify step captured in a HIP graph (torch.cuda.CUDAGraph) replays to the
same bytes as the eager call: several replays, with eager steps and host
synchronisations between them, each compared with the eager result."""
import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from tests.helpers import say

pytestmark = pytest.mark.gpu


def test_captured_step_replays_match_eager():
    import torch
    dev = "cuda"
    w = synth.small_stack(4)
    handle = msk.Handle(msk.make_config(w))
    keep = []
    for l in range(w.n_layers):
        lw = synth.layer_weights(w, l)
        k, v = synth.kv_cache(w, l)
        t = synth.to_device(lw, dev)
        t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
        t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
        handle.load_layer(l, t, int(lw["window"]))
        keep.append(t)
    h_in = torch.from_numpy(np.ascontiguousarray(synth.h_input(w), np.float32)).to(dev)
    L = w.n_layers
    h_eager = torch.zeros_like(h_in)
    ids_eager = torch.zeros((L, w.NT, w.k), dtype=torch.int32, device=dev)
    io_eager = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_eager, ids_eager)
    handle.verify_step(io_eager)
    handle.synchronize()
    torch.cuda.synchronize()
    ref = h_eager.cpu().numpy().copy()
    ref_ids = ids_eager.cpu().numpy().copy()

    h_g = torch.zeros_like(h_in)
    ids_g = torch.zeros_like(ids_eager)
    io_g = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_g, ids_g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        handle.verify_step(io_g, stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("[graph] capturing one step")
    with torch.cuda.graph(g):
        handle.verify_step(io_g)
    for rep in range(3):
        h_g.zero_()
        ids_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(h_g.cpu().numpy(), ref), f"replay {rep}: h_out differs from eager"
        assert np.array_equal(ids_g.cpu().numpy(), ref_ids), f"replay {rep}: expert ids differ from eager"
        handle.verify_step(io_eager)  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(h_eager.cpu().numpy(), ref)
    say("[graph] 3 replays match the eager step")
    handle.close()


def test_captured_step_follows_device_ctx():
    """ctx_len is read by the kernels at run time: one captured step, replayed
    with two different context lengths written into the same device tensor,
    equals the eager step at each length (outputs, routing and the cache rows
    the step writes)."""
    import torch
    dev = "cuda"
    w = synth.small_stack(2)
    handle = msk.Handle(msk.make_config(w))
    keep = []
    for l in range(w.n_layers):
        lw = synth.layer_weights(w, l)
        k, v = synth.kv_cache(w, l)
        t = synth.to_device(lw, dev)
        t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
        t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
        handle.load_layer(l, t, int(lw["window"]))
        keep.append(t)
    h_in = torch.from_numpy(np.ascontiguousarray(synth.h_input(w), np.float32)).to(dev)
    pristine = [(t["k_cache"].clone(), t["v_cache"].clone()) for t in keep]

    def restore():  # each run starts from the same cache bytes
        for t, (k0, v0) in zip(keep, pristine):
            t["k_cache"].copy_(k0)
            t["v_cache"].copy_(v0)

    ctx_values = (w.ctx, w.ctx - 23)
    eager = {}
    for c in ctx_values:
        restore()
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((w.n_layers, w.NT, w.k), dtype=torch.int32, device=dev)
        handle.verify_step(msk.make_io(w.R, w.T, [c], h_in, h_out, ids))
        handle.synchronize()
        eager[c] = (h_out.cpu().numpy(), ids.cpu().numpy(), [t["k_cache"].cpu().numpy() for t in keep])
    assert not np.array_equal(eager[ctx_values[0]][0], eager[ctx_values[1]][0])
    restore()
    ctx_dev = torch.tensor([ctx_values[0]], dtype=torch.int32, device=dev)
    h_g = torch.zeros_like(h_in)
    ids_g = torch.zeros((w.n_layers, w.NT, w.k), dtype=torch.int32, device=dev)
    io = msk.make_io(w.R, w.T, ctx_dev, h_in, h_g, ids_g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        handle.verify_step(io, stream=s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        handle.verify_step(io)
    for rep in range(4):
        c = ctx_values[rep % 2]
        ctx_dev.fill_(c)
        restore()
        h_g.zero_()
        ids_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = eager[c]
        assert np.array_equal(h_g.cpu().numpy(), ref[0]), f"replay {rep} (ctx {c}): h_out differs from eager"
        assert np.array_equal(ids_g.cpu().numpy(), ref[1]), f"replay {rep} (ctx {c}): ids differ from eager"
        for l, t in enumerate(keep):
            assert np.array_equal(t["k_cache"].cpu().numpy(), ref[2][l]), (rep, l)
    handle.synchronize()
    say("[graph] one capture, replays at two context lengths match eager")
    handle.close()

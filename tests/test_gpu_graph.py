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

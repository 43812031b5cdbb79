"""GPU checks of the speculative expert prefetch (routing history -> prefetch
list): the list a call uses is the oracle's ranking of the previous call's
selections of that layer (bit-exact), and prefetching changes no output."""
import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc
from tests.helpers import say

pytestmark = pytest.mark.gpu

NPF = 14


def _step_handle(w, expert_prefetch, dev="cuda"):
    import torch
    handle = msk.Handle(msk.make_config(w, expert_prefetch=expert_prefetch))
    keep = []
    for l in range(w.n_layers):
        lw = synth.layer_weights(w, l)
        k, v = synth.kv_cache(w, l)
        t = synth.to_device(lw, dev)
        t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
        t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
        handle.load_layer(l, t, int(lw["window"]))
        keep.append(t)
    return handle, keep


def _run(handle, w, h, npf, dev="cuda"):
    import torch
    h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
    h_out = torch.zeros_like(h_in)
    L = w.n_layers
    ids = torch.zeros((L, w.NT, w.k), dtype=torch.int32, device=dev)
    pl = torch.full((L, max(npf, 1)), -1, dtype=torch.int32, device=dev)
    io = msk.make_io(w.R, w.T, [w.ctx] * w.R, h_in, h_out, ids, None, prefetch_ids=pl if npf else None)
    if L == 1:
        handle.verify_layer(0, io)
    else:
        handle.verify_step(io)
    torch.cuda.synchronize()
    return h_out.cpu().numpy(), ids.cpu().numpy(), pl.cpu().numpy()


def test_prefetch_list_is_ranking_of_previous_step_small_stack():
    w = synth.small_stack(4)
    h = synth.h_input(w)
    say("[prefetch] small stack, two steps")
    handle, keep = _step_handle(w, NPF)
    out1, ids1, pl1 = _run(handle, w, h, NPF)
    out2, ids2, pl2 = _run(handle, w, -h, NPF)
    handle.close()
    zero_rank = orc.prefetch_list(np.zeros(0, np.int32), w.E, NPF)
    for l in range(w.n_layers):
        assert np.array_equal(pl1[l], zero_rank), f"layer {l}: first call's list"
        assert np.array_equal(pl2[l], orc.prefetch_list(ids1[l], w.E, NPF)), f"layer {l}: second call's list"
    # prefetching has no effect on results
    handle0, keep0 = _step_handle(w, 0)
    ref1, rids1, _ = _run(handle0, w, h, 0)
    ref2, rids2, _ = _run(handle0, w, -h, 0)
    handle0.close()
    assert np.array_equal(out1, ref1) and np.array_equal(out2, ref2)
    assert np.array_equal(ids1, rids1) and np.array_equal(ids2, rids2)


def test_prefetch_list_working_size_layer():
    import torch
    w = synth.WORKLOADS["swa_layer"]
    say("[prefetch] working-size layer, two calls")
    handle = msk.Handle(msk.make_config(w, expert_prefetch=NPF))
    t = synth.device_layer(w, 0, "cuda")
    handle.load_layer(0, t, int(w.windows[0]))
    h = synth.h_input(w)
    out1, ids1, pl1 = _run(handle, w, h, NPF)
    out2, ids2, pl2 = _run(handle, w, -h, NPF)
    assert np.array_equal(pl1[0], orc.prefetch_list(np.zeros(0, np.int32), w.E, NPF))
    ref = orc.prefetch_list(ids1[0], w.E, NPF)
    say(f"[prefetch] list {pl2[0].tolist()}")
    assert np.array_equal(pl2[0], ref)
    assert len(np.unique(ids1[0])) > NPF
    handle.close()
    del t
    torch.cuda.empty_cache()


def test_kv_tail_prefetch_changes_no_output():
    """MSK_FLAG_KV_PREFETCH only reads the next layer's KV window: a step with
    the flag gives the same bytes as one without (several requests with
    different contexts, so every request's window is walked)."""
    import torch
    from dataclasses import replace
    dev = "cuda"
    w = replace(synth.small_stack(3), R=4, T=4)
    h = synth.h_input(w)
    outs = []
    for flags in (0, msk.MSK_FLAG_KV_PREFETCH):
        handle = msk.Handle(msk.make_config(w, flags=flags))
        keep = []
        for l in range(w.n_layers):
            lw = synth.layer_weights(w, l)
            k, v = synth.kv_cache(w, l)
            t = synth.to_device(lw, dev)
            t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
            t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
            handle.load_layer(l, t, int(lw["window"]))
            keep.append(t)
        h_in = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((w.n_layers, w.NT, w.k), dtype=torch.int32, device=dev)
        handle.verify_step(msk.make_io(w.R, w.T, [64, 50, 20, 3], h_in, h_out, ids))
        handle.synchronize()
        outs.append((h_out.cpu().numpy(), ids.cpu().numpy(), [t["k_cache"].cpu().numpy() for t in keep]))
        handle.close()
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    for a, b in zip(outs[0][2], outs[1][2]):
        assert np.array_equal(a, b)

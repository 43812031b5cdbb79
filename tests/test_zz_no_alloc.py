"""msk_create_static: a handle whose workspace is the library's own static
device array (for callers that cannot allocate device memory). Its calls
must give the same bytes as a handle on a caller workspace, on two calls in a
row where the second is smaller (fewer tokens, then fewer requests), for the
standalone layer and for a several-layer step; configurations that need more
than the static array are refused."""
from dataclasses import replace

import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from tests.helpers import say

pytestmark = pytest.mark.gpu


def _load(handle, w, dev):
    import torch
    keep = []
    for l in range(w.n_layers):
        lw = synth.layer_weights(w, l)
        k, v = synth.kv_cache(w, l)
        t = synth.to_device(lw, dev)
        t["k_cache"] = torch.from_numpy(k.view(np.int16)).to(dev)
        t["v_cache"] = torch.from_numpy(v.view(np.int16)).to(dev)
        handle.load_layer(l, t, int(lw["window"]))
        keep.append(t)
    return keep


def _calls(handle, w, keep, dev):
    """Two calls in a row: all requests x T tokens, then fewer tokens and
    fewer requests. Returns the outputs, ids and written cache rows."""
    import torch
    out = []
    h_all = torch.from_numpy(np.ascontiguousarray(synth.h_input(w), np.float32)).to(dev)
    for R, T in ((w.R, w.T), (max(1, w.R // 2), w.T // 2)):
        h_in = h_all.view(w.R, w.T, w.H)[:R, :T].contiguous().view(R * T, w.H)
        h_out = torch.zeros_like(h_in)
        ids = torch.zeros((w.n_layers, R * T, w.k), dtype=torch.int32, device=dev)
        io = msk.make_io(R, T, [w.ctx - 3 * r for r in range(R)], h_in, h_out, ids)
        if w.n_layers == 1:
            handle.verify_layer(0, io)
        else:
            handle.verify_step(io)
        handle.synchronize()
        out.append((h_out.cpu().numpy(), ids.cpu().numpy(), [t["k_cache"].cpu().numpy() for t in keep]))
    return out


@pytest.mark.parametrize("name,layers", [("tiny_swa", 1), ("tiny_stack", 3), ("swa_layer", 1)])
def test_static_workspace_matches_caller_workspace(name, layers):
    dev = "cuda"
    if name == "tiny_stack":
        w = replace(synth.small_stack(layers), R=2)
    else:
        w = replace(synth.WORKLOADS[name], R=2)
    results = []
    for static in (False, True):
        say(f"[no-alloc {name}] {'static' if static else 'caller'} workspace")
        handle = msk.Handle(msk.make_config(w), device=dev, static=static)
        keep = _load(handle, w, dev)
        results.append(_calls(handle, w, keep, dev))
        handle.close()
        del keep
    for c in range(2):
        a, b = results[0][c], results[1][c]
        assert np.array_equal(a[0], b[0]), (name, c, "h_out")
        assert np.array_equal(a[1], b[1]), (name, c, "ids")
        for l in range(len(a[2])):
            assert np.array_equal(a[2][l], b[2][l]), (name, c, "cache", l)
    say(f"[no-alloc {name}] both calls bit-identical to the caller-workspace handle")


def test_static_workspace_refuses_oversized_configs():
    w = synth.WORKLOADS["tiny_swa"]
    cfg = msk.make_config(w)
    assert msk.msk_workspace_bytes(cfg) <= msk.MSK_STATIC_WORKSPACE_BYTES
    big = msk.make_config(replace(synth.WORKLOADS["swa_layer"], n_layers=20000))
    need = msk.msk_workspace_bytes(big)
    assert need > msk.MSK_STATIC_WORKSPACE_BYTES
    with pytest.raises(msk.MskError) as ei:
        msk.msk_create_static(big)
    assert ei.value.status == msk.MSK_E_CAPACITY
    assert "static workspace" in str(ei.value)

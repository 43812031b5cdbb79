"""GPU checks that must hold bit for bit: the KV write on inputs whose
projection is exact, and the attention window read through a probe whose
averages are exact ratios of integers."""
from dataclasses import replace

import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc
from tests.helpers import GpuLayerRun, oracle_layer, say

pytestmark = pytest.mark.gpu

ONE = synth.BF16_ONE


def test_kv_write_bit_exact_on_exact_projection():
    """No norm, QKV rows that each select one input column, inputs k/8 with
    |k| <= 64: every projected value is exact on both sides, so the caches
    after the KV write must match byte for byte (new rows and untouched rows)."""
    w = synth.WORKLOADS["tiny_swa"]
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    Nqkv = w.Dq + 2 * w.Dkv
    sel = np.zeros((Nqkv, w.H), np.uint16)
    for n in range(Nqkv):
        sel[n, (7 * n + 3) % w.H] = ONE
    lw["w_qkv"] = sel
    rng = np.random.default_rng(0)
    h = (rng.integers(-64, 65, size=(w.NT, w.H)) / 8.0).astype(np.float32)
    say("[kv-exact] gpu run")
    run = GpuLayerRun(w, lw, k, v, h, flags=msk.MSK_FLAG_NO_NORM)
    g = run.run()
    run.close()
    o = oracle_layer(w, lw, k, v, h, use_norm=False)
    assert np.array_equal(g["k_new"], o["k_new"]) and np.array_equal(g["v_new"], o["v_new"])
    assert np.array_equal(g["k_cache"], o["k_cache"])
    assert np.array_equal(g["v_cache"], o["v_cache"])


def _probe(w, ctx):
    """Q = 0 (zero query rows) so every visible key weighs the same; value
    rows hold bits of their position. The attention output is then the
    fraction of visible positions with each bit set: exact ratios the oracle
    computes in fp64 and the kernel in fp32 from exact integer sums."""
    lw = synth.layer_weights(w, 0, experts=[])
    lw["w_qkv"][:w.Dq] = 0
    k, v = synth.kv_cache(w, 0)
    pos = np.arange(w.cap)
    bits = ((pos[:, None] >> np.arange(min(w.d, 16))[None, :]) & 1).astype(np.uint16) * ONE
    v[:, :, :, :] = 0
    v[:, :, :, :bits.shape[1]] = bits[None, None]
    h = synth.h_input(w)
    return lw, k, v, h


@pytest.mark.parametrize("name,ctx", [("tiny_swa", 64), ("tiny_swa", 10), ("swa_layer", 8192),
                                      ("global_layer", 32768)])
def test_window_mask_probe(name, ctx):
    w = synth.WORKLOADS[name]
    w = replace(w, ctx=ctx) if ctx != w.ctx else w
    lw, k, v, h = _probe(w, ctx)
    say(f"[probe {name} ctx={ctx}] gpu run")
    run = GpuLayerRun(w, lw, k, v, h)
    g = run.run()
    run.close()
    say(f"[probe {name} ctx={ctx}] oracle run")
    o = oracle_layer(w, lw, k, v, h)
    assert np.all(g["q"] == 0.0)
    # the new rows' value vectors come from the projection; compare only the bit columns of
    # old positions through the exact expectation on both sides
    diff = np.max(np.abs(g["attn"].astype(np.float64) - o["attn"]))
    # one position more or less in a window of n changes a column by about 1/(2n)
    n_vis = (w.windows[0] if w.windows[0] > 0 else ctx + w.T)
    say(f"[probe {name} ctx={ctx}] max diff {diff:.3e} (one-key change ~{0.5 / n_vis:.1e})")
    assert diff < 0.05 / n_vis

"""Tree verification on the GPU: the verify tokens of a request form a tree
of candidates (orcarouter.ai, "Muse Spark Open: 1.109 token al secondo ...",
section "Anche il modello draft e' diventato piu' veloce ..."); each token
attends to the prior context and to its ancestors, with the window placed at
its position on its own path. The oracle with the same ancestor masks is the
reference."""
from dataclasses import replace

import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth
from oracle import oracle as orc
from tests.helpers import GpuLayerRun, oracle_layer, random_tree, rel_err, routing_mismatches, say
from tests.test_gpu_exact import _probe

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _stages(g, o, label):
    errs = {k: rel_err(g[k], o[ko]) for k, ko in (("q", "q"), ("k_new", "k_new"), ("v_new", "v_new"),
                                                  ("attn", "attn"), ("h1", "h1"), ("n2", "n2_f32"),
                                                  ("logits", "logits"), ("p", "p"), ("acc", "acc"),
                                                  ("h_out", "h_out"))}
    say(f"[{label}] rel errs " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, e in errs.items():
        assert e <= TOL, (label, k, e)


@pytest.mark.parametrize("seed", [1, 2])
def test_tiny_tree_layer_matches_oracle(seed):
    w = synth.WORKLOADS["tiny_swa"]
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w)
    tree = random_tree(w.T, seed)
    assert orc.tree_valid(tree, w.T)
    say(f"[tree tiny seed={seed}] masks {[hex(int(a)) for a in tree]}")
    run = GpuLayerRun(w, lw, k, v, h)
    g = run.run(tree=[tree])
    chain = run.run()
    run.close()
    o = oracle_layer(w, lw, k, v, h, tree=[tree])
    _stages(g, o, f"tree tiny seed={seed}")
    assert not routing_mismatches(g["ids"], o["logits"], w.k, 1e-3)
    # the tree changes attention relative to the chain
    assert rel_err(g["attn"], chain["attn"]) > 10 * TOL * 1e-2


@pytest.mark.parametrize("name,ctx", [("tiny_swa", 64), ("tiny_swa", 10), ("swa_layer", 8192)])
def test_tree_window_probe(name, ctx):
    """Q = 0 and value rows that encode their position: each token's output is
    the per-bit fraction of its visible rows, so a wrong visible set (a missing
    ancestor, a sibling seen, a window misplaced on the path) shows as a
    difference of about 1/(2n) or more."""
    w = synth.WORKLOADS[name]
    w = replace(w, ctx=ctx) if ctx != w.ctx else w
    lw, k, v, h = _probe(w, ctx)
    tree = random_tree(w.T, 7)
    run = GpuLayerRun(w, lw, k, v, h)
    g = run.run(tree=[tree])
    run.close()
    o = oracle_layer(w, lw, k, v, h, tree=[tree])
    diff = np.max(np.abs(g["attn"].astype(np.float64) - o["attn"]))
    n_vis = w.windows[0] if w.windows[0] > 0 else ctx + w.T
    say(f"[tree probe {name} ctx={ctx}] max diff {diff:.3e} (one-key change ~{0.5 / n_vis:.1e})")
    assert diff < 0.05 / n_vis


def test_tree_requests_match_joint_oracle():
    """Four requests of 8 tokens (two 16-token passes), each with its own tree
    and context length."""
    base = synth.small_stack(1)
    w = replace(base, name="tiny_tree_r4_t8", R=4, T=8)
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w)
    ctx = [64, 40, 10, 57]
    trees = [random_tree(w.T, 11 + r) for r in range(w.R)]
    run = GpuLayerRun(w, lw, k, v, h, ctx=ctx)
    g = run.run(debug=False, tree=trees)
    run.close()
    o = oracle_layer(w, lw, k, v, h, ctx=ctx, tree=trees)
    e = rel_err(g["h_out"], o["h_out"])
    say(f"[tree r4] h_out rel err {e:.2e}")
    assert e < TOL
    assert not routing_mismatches(g["ids"], o["logits"], w.k, 1e-3)


def test_explicit_chain_mask_is_the_default_bit_for_bit():
    w = synth.WORKLOADS["tiny_swa"]
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w)
    chain = [[(2 << t) - 1 for t in range(w.T)]]
    run = GpuLayerRun(w, lw, k, v, h)
    a = run.run(debug=False)
    b = run.run(debug=False, tree=chain)
    run.close()
    assert np.array_equal(a["h_out"], b["h_out"]) and np.array_equal(a["ids"], b["ids"])


def test_invalid_tree_masks_are_rejected():
    import torch
    w = synth.WORKLOADS["tiny_swa"]
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w)
    run = GpuLayerRun(w, lw, k, v, h)
    chain = [(2 << t) - 1 for t in range(w.T)]
    bad = []
    m = list(chain); m[3] = 0b0111; bad.append(m)            # no self bit
    m = list(chain); m[2] = 0b1111; bad.append(m)            # a later token
    m = list(chain); m[5] = (1 << 5) | (1 << 4); bad.append(m)  # ancestor 4 without 4's ancestors
    for m in bad:
        with pytest.raises(msk.MskError) as ei:
            run.run(debug=False, tree=[m])
        assert ei.value.status == msk.MSK_E_INVALID
    torch.cuda.synchronize()
    run.close()

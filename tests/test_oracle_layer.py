"""Pins of the oracle's whole layer: special cases that reduce it to closed
forms, exact permutations, or a dense network (no GPU)."""
from dataclasses import replace

import numpy as np
import pytest

from moe_decode_megakernel_amd import synth
from oracle import oracle as orc

W = synth.WORKLOADS["tiny_swa"]
ONE = synth.BF16_ONE


def _layer(w=W):
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w).astype(np.float64)
    return lw, k, v, h


def _run(lw, k, v, h, w=W, use_norm=True, R=1, ctx=None):
    ctx = [w.ctx] * R if ctx is None else ctx
    return orc.layer_forward(w, lw, R, w.T, ctx, h, k, v, w.cap, eps=w.eps, use_norm=use_norm)


def _perm_matrix_bf16(n, seed):
    pi = np.random.default_rng(seed).permutation(n)
    m = np.zeros((n, n), np.uint16)
    m[np.arange(n), pi] = ONE
    return m, pi


def test_qkv_row_order_and_kv_write_placement():
    lw, k, v, h = _layer()
    Nqkv = W.Dq + 2 * W.Dkv
    sel = np.zeros((Nqkv, W.H), np.uint16)
    src = np.empty(Nqkv, np.int64)
    for n in range(Nqkv):
        src[n] = (n if n < W.Dq else (3 * n + 1)) % W.H
        sel[n, src[n]] = ONE
    lw["w_qkv"] = sel
    k0, v0 = k.copy(), v.copy()
    _, st = _run(lw, k, v, h, use_norm=False)
    assert np.array_equal(st["q"], h[:, src[:W.Dq]])
    assert np.array_equal(st["k_new"], h[:, src[W.Dq:W.Dq + W.Dkv]])
    assert np.array_equal(st["v_new"], h[:, src[W.Dq + W.Dkv:]])
    rows = slice(W.ctx, W.ctx + W.T)
    for g in range(W.nkv):
        ref_k = np.array([[orc.bf16_rne(x) for x in st["k_new"][t, g * W.d:(g + 1) * W.d]] for t in range(W.T)], np.uint16)
        ref_v = np.array([[orc.bf16_rne(x) for x in st["v_new"][t, g * W.d:(g + 1) * W.d]] for t in range(W.T)], np.uint16)
        assert np.array_equal(k[0, g, rows], ref_k)
        assert np.array_equal(v[0, g, rows], ref_v)
    mask = np.ones(W.cap, bool)
    mask[rows] = False
    assert np.array_equal(k[:, :, mask], k0[:, :, mask]) and np.array_equal(v[:, :, mask], v0[:, :, mask])


def test_zero_output_projection_keeps_residual():
    lw, k, v, h = _layer()
    lw["w_o"] = np.zeros_like(lw["w_o"])
    _, st = _run(lw, k, v, h)
    assert np.array_equal(st["h1"], h)


def test_zero_experts_keep_residual():
    lw, k, v, h = _layer()
    lw["e_gate_up"][:] = 0
    lw["e_down"][:] = 0
    out, st = _run(lw, k, v, h)
    assert np.all(st["acc"] == 0.0)
    assert np.array_equal(out, st["h1"])


def test_permutation_output_projection_with_zero_query():
    # Wq = 0 => every visible key equally weighted; Wo = permutation => h1 = h + attn[:, pi]
    lw, k, v, h = _layer()
    assert W.Dq == W.H
    lw["w_qkv"][:W.Dq] = 0
    lw["w_o"], pi = _perm_matrix_bf16(W.H, 11)
    _, st = _run(lw, k, v, h)
    assert np.array_equal(st["h1"], h + st["attn"][:, pi])
    assert np.all(st["q"] == 0.0)


def test_permutation_pooler_and_unpooler():
    w = replace(W, P=W.H, I=64)
    lw, k, v, h = _layer(w)
    lw["w_pool"], pi = _perm_matrix_bf16(w.H, 12)
    lw["w_unpool"], sigma = _perm_matrix_bf16(w.H, 13)
    out, st = _run(lw, k, v, h, w=w)
    n2 = np.stack([orc.rmsnorm(st["h1"][t], lw["g_moe"], float(np.float32(w.eps))) for t in range(w.NT)])
    assert np.array_equal(st["p"], n2[:, pi])
    assert np.array_equal(out, st["h1"] + st["acc"][:, sigma])


def test_router_stage_wiring():
    lw, k, v, h = _layer()
    lw["b_router"] = synth.zipf_bias(W.E, 0, 99, 1.1)
    _, st = _run(lw, k, v, h)
    n2 = np.stack([orc.rmsnorm(st["h1"][t], lw["g_moe"], float(np.float32(W.eps))) for t in range(W.NT)])
    assert np.array_equal(st["n2_f32"], n2.astype(np.float32))
    for t in range(W.NT):
        for e in range(W.E):
            want = np.float32(orc.dot_canon_f32(st["n2_f32"][t], lw["w_router"][e]) + lw["b_router"][e])
            assert st["logits"][t, e] == want
        order = sorted(range(W.E), key=lambda e: (-float(st["logits"][t, e]), e))[:W.k]
        assert list(st["ids"][t]) == order
        assert abs(st["gates"][t].sum() - 1.0) < 1e-15


def _dense_expert(lw, e):
    I, P = W.I, W.P
    wgu = orc.nvfp4_dequant(lw["e_gate_up"][e], lw["e_gate_up_scale"][e], lw["e_tensor_scale"][e, 0], 2 * I, P)
    wd = orc.nvfp4_dequant(lw["e_down"][e], lw["e_down_scale"][e], lw["e_tensor_scale"][e, 1], P, I)
    return wgu, wd


def test_identical_experts_equal_one_dense_ffn():
    lw, k, v, h = _layer()
    for name in ("e_gate_up", "e_gate_up_scale", "e_down", "e_down_scale", "e_tensor_scale"):
        lw[name][:] = lw[name][0]
    _, st = _run(lw, k, v, h)
    wgu, wd = _dense_expert(lw, 0)
    y = orc.dense_swiglu(st["p"], wgu, wd)
    assert np.allclose(st["acc"], y, rtol=1e-12, atol=1e-14)


def test_dense_swiglu_matches_library_composition():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 32))
    wgu = rng.standard_normal((2 * 16, 32)) * 0.3
    wd = rng.standard_normal((32, 16)) * 0.3
    gu = x @ wgu.T
    gate, up = gu[:, :16], gu[:, 16:]
    silu = np.vectorize(orc.silu)(gate)
    assert np.allclose(orc.dense_swiglu(x, wgu, wd), (silu * up) @ wd.T, rtol=1e-13, atol=1e-14)
    # gate first: a large positive gate pre-activation passes `up` through ~linearly
    wgu2 = np.zeros((32, 32))
    wgu2[:16, 0] = 40.0     # gate rows read x0
    wgu2[16:, 1] = 1.0      # up rows read x1
    x2 = np.zeros((1, 32))
    x2[0, 0], x2[0, 1] = 1.0, 0.5
    eye = np.eye(32, 16)
    y = orc.dense_swiglu(x2, wgu2, eye)
    assert np.allclose(y[0, :16], 40.0 * 0.5, rtol=1e-15)


def test_expert_ids_address_the_right_experts():
    # shared codes, down tensor scale of expert e = (e + 1) * s: acc = sum_j g_j (id_j + 1) y_base
    lw, k, v, h = _layer()
    for name in ("e_gate_up", "e_gate_up_scale", "e_down", "e_down_scale"):
        lw[name][:] = lw[name][0]
    s = np.float32(lw["e_tensor_scale"][0, 1])
    lw["e_tensor_scale"][:, 0] = lw["e_tensor_scale"][0, 0]
    lw["e_tensor_scale"][:, 1] = s * (np.arange(W.E, dtype=np.float32) + 1)
    _, st = _run(lw, k, v, h)
    wgu, wd = _dense_expert(lw, 0)
    y = orc.dense_swiglu(st["p"], wgu, wd)
    ratio = lw["e_tensor_scale"][:, 1].astype(np.float64) / float(s)  # fl32((e+1)*s)/s ~ e+1
    assert np.allclose(ratio, np.arange(W.E) + 1, rtol=1e-6)
    f = (st["gates"] * ratio[st["ids"]]).sum(axis=1)
    assert np.allclose(st["acc"], f[:, None] * y, rtol=1e-12, atol=1e-14)


def test_stage_compositions_match_library_matmuls():
    lw, k, v, h = _layer()
    k0, v0 = k.copy(), v.copy()
    out, st = _run(lw, k, v, h)
    dec = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    n1 = np.stack([orc.rmsnorm(h[t], lw["g_attn"], float(np.float32(W.eps))) for t in range(W.NT)])
    qkv = n1 @ dec(lw["w_qkv"]).T
    assert np.allclose(st["q"], qkv[:, :W.Dq], rtol=1e-12, atol=1e-12)
    attn = orc.attention(st["q"], k[0], v[0], W.nq, W.nkv, W.d, W.cap, W.T, W.ctx, W.windows[0])
    assert np.array_equal(st["attn"], attn)
    assert np.allclose(st["h1"], h + attn @ dec(lw["w_o"]).T, rtol=1e-12, atol=1e-12)
    assert np.allclose(out, st["h1"] + st["acc"] @ dec(lw["w_unpool"]).T, rtol=1e-12, atol=1e-12)


def test_requests_are_independent():
    lw, k, v, h = _layer()
    out1, st1 = _run(lw, k.copy(), v.copy(), h)
    w2 = replace(W, R=2)
    k2 = np.concatenate([k, k])
    v2 = np.concatenate([v, v])
    h2 = np.concatenate([h, h])
    out2, st2 = orc.layer_forward(w2, lw, 2, W.T, [W.ctx, W.ctx], h2, k2, v2, W.cap, eps=W.eps)
    assert np.array_equal(out2[:W.T], out1) and np.array_equal(out2[W.T:], out1)
    assert np.array_equal(k2[0], k2[1])


def test_act_fp4_expert_path_matches_library_composition():
    """NVFP4 activations: recompute the experts from the pooled stage with
    library matmuls and the pinned block quantizer."""
    lw, k, v, h = _layer()
    _, st = orc.layer_forward(W, lw, 1, W.T, [W.ctx], h, k.copy(), v.copy(), W.cap, eps=W.eps,
                              act_fp4=True)
    _, st0 = _run(lw, k.copy(), v.copy(), h)
    acc = np.zeros((W.NT, W.P))
    for t in range(W.NT):
        for j in range(W.k):
            e = int(st["ids"][t, j])
            wgu, wd = _dense_expert(lw, e)
            gu = st["p"][t] @ wgu.T
            a = np.vectorize(orc.silu)(gu[:W.I]) * gu[W.I:]
            aq = orc.nvfp4_quant_rows(a.astype(np.float32)[None, :])[0].astype(np.float64)
            acc[t] += st["gates"][t, j] * (aq @ wd.T)
    assert np.allclose(st["acc"], acc, rtol=1e-9, atol=1e-12)
    # the quantization changes the result (fp4 keeps 8 magnitudes per block,
    # so the change is of the order of the data itself, not of rounding)
    d = np.abs(st["acc"] - st0["acc"]).max() / np.abs(st0["acc"]).max()
    assert 1e-3 < d < 1.0, d


def test_layer_result_does_not_depend_on_the_thread_count():
    """The oracle parallelises over independent outputs only, so one host
    thread and all of them give the same bits (the bench times both)."""
    w = synth.WORKLOADS["tiny_swa"]
    lw = synth.layer_weights(w, 0)
    k, v = synth.kv_cache(w, 0)
    h = synth.h_input(w, 0).astype(np.float64)
    n = orc.threads()
    outs = []
    try:
        for t in (1, max(2, n)):
            orc.set_threads(t)
            kk, vv = k.copy(), v.copy()
            out, st = orc.layer_forward(w, lw, w.R, w.T, [w.ctx] * w.R, h, kk, vv, w.cap, eps=w.eps)
            outs.append((out, st["ids"].copy(), kk, vv))
    finally:
        orc.set_threads(n)
    (o1, i1, k1, v1), (o2, i2, k2, v2) = outs
    assert np.array_equal(o1, o2)
    assert np.array_equal(i1, i2)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)

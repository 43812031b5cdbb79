"""Pins of the oracle's attention against special cases with closed forms
(no GPU). Caches are [nkv][cap][d] bf16 of one request."""
import math

import numpy as np
import pytest

from oracle import oracle as orc
from tests.conftest import read_golden


def _bf16(x):
    return np.array([orc.bf16_rne(float(v)) for v in np.ravel(x)], np.uint16).reshape(np.shape(x))


def _bf16_fast(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _dec(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(nq=4, nkv=2, d=16, cap=48, seed=0):
    rng = np.random.default_rng(seed)
    k = _bf16_fast(rng.standard_normal((nkv, cap, d)))
    v = _bf16_fast(rng.standard_normal((nkv, cap, d)))
    return rng, k, v


def test_single_visible_key_returns_its_value_row():
    rng, k, v = _setup()
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 48, 5, 20
    q = rng.standard_normal((T, nq * d))
    out = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, 1)
    for t in range(T):
        for h in range(nq):
            g = h // (nq // nkv)
            assert np.array_equal(out[t, h * d:(h + 1) * d], _dec(v[g, ctx + t]))


def test_window_covering_context_equals_global_bit_for_bit():
    rng, k, v = _setup()
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 48, 6, 30
    q = rng.standard_normal((T, nq * d))
    g = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, 0)
    for w in (ctx + T, ctx + T + 1, 10 ** 6):
        assert np.array_equal(orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, w), g)
    # a window one short of the context differs for the last token
    assert not np.array_equal(orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, ctx + T - 1)[T - 1], g[T - 1])


def test_constant_value_rows_are_returned_weights_sum_to_one():
    rng, k, _ = _setup()
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 48, 4, 40
    c = _bf16_fast(rng.standard_normal(d))
    v = np.broadcast_to(c, (nkv, cap, d)).copy()
    q = rng.standard_normal((T, nq * d)) * 3
    for w in (0, 7):
        out = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, w)
        for h in range(nq):
            assert np.allclose(out[:, h * d:(h + 1) * d], _dec(c)[None, :], rtol=0, atol=1e-14)


def test_zero_query_is_mean_of_the_visible_window_rows():
    """Q = 0 makes every visible key equally weighted; the visible set comes
    from the hand-derived window table of the tiny layer (ctx 64, window 32)."""
    rng = np.random.default_rng(1)
    nq, nkv, d, T, ctx, W = 4, 1, 64, 16, 64, 32
    cap = ctx + T
    k = _bf16_fast(rng.standard_normal((nkv, cap, d)))
    v = _bf16_fast(rng.standard_normal((nkv, cap, d)))
    q = np.zeros((T, nq * d))
    out = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, W)
    for t, lo, hi in read_golden("window_tiny_swa.txt"):
        t, lo, hi = int(t), int(lo), int(hi)
        expect = _dec(v[0, lo:hi + 1]).mean(axis=0)
        for h in range(nq):
            assert np.allclose(out[t, h * d:(h + 1) * d], expect, rtol=0, atol=1e-13)


def test_two_keys_logistic_weights_and_head_dim_scale():
    # window 2 leaves keys pos-1 and pos; q = a*e0, K rows e0 * (b0, b1):
    # weights are logistic in a*(b1 - b0)/sqrt(d).
    nq, nkv, d, T, ctx = 1, 1, 64, 1, 10
    cap = ctx + T
    k = np.zeros((nkv, cap, d), np.uint16)
    v = np.zeros((nkv, cap, d), np.uint16)
    k[0, ctx - 1, 0] = orc.bf16_rne(0.5)
    k[0, ctx, 0] = orc.bf16_rne(2.0)
    v[0, ctx - 1, 1] = orc.bf16_rne(1.0)
    v[0, ctx, 2] = orc.bf16_rne(1.0)
    a = 3.0
    q = np.zeros((T, d))
    q[0, 0] = a
    out = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, 2)
    z = a * (2.0 - 0.5) / math.sqrt(d)
    w_new = 1.0 / (1.0 + math.exp(-z))
    assert abs(out[0, 2] - w_new) < 1e-15 and abs(out[0, 1] - (1 - w_new)) < 1e-15


def test_gqa_consecutive_grouping():
    nq, nkv, d, T, ctx = 8, 2, 16, 3, 12
    cap = ctx + T
    rng = np.random.default_rng(2)
    k = _bf16_fast(rng.standard_normal((nkv, cap, d)))
    v = np.zeros((nkv, cap, d), np.uint16)
    v[0] = orc.bf16_rne(-1.0)
    v[1] = orc.bf16_rne(1.0)
    out = orc.attention(rng.standard_normal((T, nq * d)), k, v, nq, nkv, d, cap, T, ctx, 0)
    for h in range(nq):
        assert np.all(out[:, h * d:(h + 1) * d] == (-1.0 if h < 4 else 1.0))


def test_causal_among_verify_tokens():
    # Q = 0, V row j = one-hot(j): token t's output is uniform over 0..ctx+t exactly.
    nq, nkv, T, ctx = 1, 1, 6, 10
    d = 16
    cap = ctx + T
    k = np.zeros((nkv, cap, d), np.uint16)
    v = np.zeros((nkv, cap, d), np.uint16)
    for j in range(cap):
        v[0, j, j] = orc.bf16_rne(1.0)
    out = orc.attention(np.zeros((T, d)), k, v, nq, nkv, d, cap, T, ctx, 0)
    for t in range(T):
        n = ctx + t + 1
        assert np.allclose(out[t, :n], 1.0 / n, rtol=0, atol=1e-16)
        assert np.all(out[t, n:] == 0.0)

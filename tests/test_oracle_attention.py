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


# --- verify-token trees --------------------------------------------------------
# The 16 verified tokens form a tree of candidates rather than a chain
# (orcarouter.ai, "Muse Spark Open: 1.109 token al secondo ...", section "Anche
# il modello draft e' diventato piu' veloce ..."). A token attends to the prior
# context and to its own ancestors; its sequence is prior context + the path
# from the root to itself.

def _random_tree(T, rng):
    """Parent pointers (parent < child, -1 = root) and the ancestor bitmasks."""
    parent = [-1] + [int(rng.integers(-1, t)) for t in range(1, T)]
    anc = []
    for t in range(T):
        a = 1 << t
        if parent[t] >= 0:
            a |= anc[parent[t]]
        anc.append(a)
    return parent, np.array(anc, np.uint16)


def _sequence_rows(parent, t, ctx, window):
    """Cache rows of token t's own sequence, last `window` of them (0 = all):
    the prior context 0..ctx-1, then the path root .. t (new row of token u is
    ctx + u). Built by walking parents, not from the bitmasks."""
    path = []
    u = t
    while u >= 0:
        path.append(ctx + u)
        u = parent[u]
    seq = list(range(ctx)) + path[::-1]
    return sorted(seq[-window:] if window > 0 else seq)


def test_tree_chain_mask_equals_default_bit_for_bit():
    rng, k, v = _setup(cap=64)
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 64, 12, 30
    q = rng.standard_normal((T, nq * d))
    chain = np.array([(2 << t) - 1 for t in range(T)], np.uint16)
    for w in (0, 1, 5, 17, 40):
        assert np.array_equal(orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, w, tree=chain),
                              orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, w))


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("window", [0, 1, 4, 9, 33])
def test_tree_zero_query_is_mean_of_the_sequence_window(seed, window):
    """Q = 0 weighs every visible key equally, so each output is the mean of the
    V rows of the token's own sequence window."""
    rng, k, v = _setup(cap=64, seed=seed)
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 64, 16, 24
    parent, anc = _random_tree(T, rng)
    out = orc.attention(np.zeros((T, nq * d)), k, v, nq, nkv, d, cap, T, ctx, window, tree=anc)
    for t in range(T):
        rows = _sequence_rows(parent, t, ctx, window)
        for h in range(nq):
            g = h // (nq // nkv)
            want = np.mean(_dec(v[g, rows]), axis=0)
            assert np.max(np.abs(out[t, h * d:(h + 1) * d] - want)) < 1e-12, (t, h, rows)


def test_tree_window_of_one_returns_own_value_row():
    rng, k, v = _setup(cap=64, seed=4)
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 64, 10, 20
    _, anc = _random_tree(T, rng)
    q = rng.standard_normal((T, nq * d))
    out = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, 1, tree=anc)
    for t in range(T):
        for h in range(nq):
            assert np.array_equal(out[t, h * d:(h + 1) * d], _dec(v[h // (nq // nkv), ctx + t]))


def test_tree_siblings_do_not_see_each_other():
    """All tokens are roots: changing one token's new K/V rows leaves every
    other token's output unchanged, bit for bit."""
    rng, k, v = _setup(cap=64, seed=5)
    nq, nkv, d, cap, T, ctx = 4, 2, 16, 64, 8, 30
    roots = np.array([1 << t for t in range(T)], np.uint16)
    q = rng.standard_normal((T, nq * d))
    a = orc.attention(q, k, v, nq, nkv, d, cap, T, ctx, 0, tree=roots)
    k2, v2 = k.copy(), v.copy()
    k2[:, ctx + 3] = _bf16_fast(rng.standard_normal((nkv, d)))
    v2[:, ctx + 3] = _bf16_fast(rng.standard_normal((nkv, d)))
    b = orc.attention(q, k2, v2, nq, nkv, d, cap, T, ctx, 0, tree=roots)
    for t in range(T):
        if t != 3:
            assert np.array_equal(a[t], b[t])
    assert not np.array_equal(a[3], b[3])


def test_tree_validation():
    chain = [(2 << t) - 1 for t in range(6)]
    assert orc.tree_valid(None, 6) and orc.tree_valid(chain, 6)
    assert orc.tree_valid([1, 2, 5, 9, 18, 37], 6)  # parents: root, root, 0, 0, 1, 2
    assert not orc.tree_valid([1, 2, 5, 9, 26, 49], 6)  # token 4 lists 3 but not 3's ancestor 0
    bad_self = list(chain); bad_self[2] = 0b011
    bad_later = list(chain); bad_later[1] = 0b111
    bad_closure = [1, 3, 0b101, 0b1100]            # token 3's ancestor 2 has ancestor 0, missing
    for b, T in ((bad_self, 6), (bad_later, 6), (bad_closure, 4)):
        assert not orc.tree_valid(b, T), b

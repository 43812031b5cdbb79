"""Pins of the oracle's number formats and small operators against the
mathematics and library routines (no GPU)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from tests.conftest import read_golden


def test_e2m1_table_matches_ocp_spec():
    for code, value in read_golden("e2m1_table.txt"):
        v = orc.e2m1_value(int(code))
        assert v == float(value)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(value))


def test_e4m3_all_codes_match_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = orc.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c], (c, v, ref[c])
    # the format's extremes: 448 and the smallest subnormal 2^-9
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x01) == 2.0 ** -9


def test_bf16_decode_exhaustive_matches_torch():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for c in range(0, 65536, 1):
        v = orc.bf16_value(c)
        r = ref[c]
        if np.isnan(r):
            assert np.isnan(v)
        else:
            assert v == r


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_rne(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_rne_ties_and_specials():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert orc.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert orc.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a tie rounds up
    assert orc.bf16_rne(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert orc.bf16_rne(-0.0) == 0x8000
    assert orc.bf16_rne(float("nan")) == 0x7FC0
    assert orc.bf16_rne(1e39) == 0x7F80


def test_nvfp4_dequant_is_table_times_scales():
    rng = np.random.default_rng(2)
    rows, cols = 8, 64
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(rows, cols // 16), dtype=np.uint8)  # no NaN code
    s_t = np.float32(3.0517578e-05)
    table = {int(c): float(v) for c, v in read_golden("e2m1_table.txt")}
    e4 = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.nvfp4_dequant(codes, scales, s_t, rows, cols)
    for r in range(rows):
        for c in range(cols):
            byte = int(codes[r, c // 2])
            nib = (byte >> 4) if (c & 1) else (byte & 15)
            expect = Fraction(table[nib]) * Fraction(e4[r, c // 16]) * Fraction(float(s_t))
            assert Fraction(got[r, c]) == expect, (r, c)


def test_router_order_hand_cases():
    cases, cur = [], None
    for r in read_golden("router_order_case.txt"):
        if r[0] == "case":
            cur = {"name": r[1], "w": np.zeros(int(r[2]), np.float32)}
            cases.append(cur)
        elif r[0] == "k":
            cur["w"][int(r[1])] = np.float32(float(r[2]))
        elif r[0] == "expect":
            cur["expect"] = float(r[1])
        elif r[0] == "other":
            cur["other"] = float(r[1])
    assert [c["name"] for c in cases] == ["chain", "tree", "cancel"]
    for c in cases:
        x = np.ones(c["w"].size, np.float32)
        got = float(orc.dot_canon_f32(x, c["w"]))
        assert got == c["expect"], c["name"]
        assert got != c["other"], c["name"]


def test_router_dot_exact_on_small_integers():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=4096).astype(np.float32)
    w = rng.integers(-8, 9, size=4096).astype(np.float32)
    assert float(orc.dot_canon_f32(x, w)) == float(np.dot(x.astype(np.int64), w.astype(np.int64)))


def test_router_dot_within_fp32_error_bound():
    rng = np.random.default_rng(4)
    for n in (64, 256, 4096):
        x = rng.standard_normal(n).astype(np.float32)
        w = (rng.standard_normal(n) * 0.02).astype(np.float32)
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w))
        got = Fraction(float(orc.dot_canon_f32(x, w)))
        # depth of the order: 8 fma steps + log2(n/8) pairwise adds
        depth = 8 + int(np.log2(n // 8))
        u = 2.0 ** -24
        bound = depth * u / (1 - depth * u) * float(np.sum(np.abs(x.astype(np.float64) * w)))
        assert abs(float(got - exact)) <= bound


def test_topk_matches_bruteforce_sort_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.choice([16, 64, 256]))
        k = int(rng.integers(1, 9))
        # few distinct values force ties
        vals = rng.integers(-3, 4, size=n).astype(np.float32) if trial % 2 else rng.standard_normal(n).astype(np.float32)
        expect = sorted(range(n), key=lambda i: (-float(vals[i]), i))[:k]
        assert list(orc.topk(vals, k)) == expect


def test_gates_softmax_properties():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal(32).astype(np.float32)
    ids = orc.topk(lg, 8)
    g = orc.gates(lg, ids)
    assert abs(g.sum() - 1.0) < 1e-15
    assert np.all(np.diff(g) <= 0)  # sorted by logit => non-increasing gates
    for i in range(8):
        for j in range(8):
            assert abs(math.log(g[i] / g[j]) - (float(lg[ids[i]]) - float(lg[ids[j]]))) < 1e-12
    assert orc.gates(lg, ids[:1])[0] == 1.0
    eq = np.zeros(8, np.float32)
    assert np.allclose(orc.gates(eq, np.arange(4, dtype=np.int32)), 0.25, rtol=0, atol=0)


def test_rmsnorm_invariants():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4096) * 3.0
    ones = np.full(4096, 0x3F80, np.uint16)
    eps = 1e-6
    y = orc.rmsnorm(x, ones, eps)
    ms = np.mean(x * x)
    assert abs(np.mean(y * y) - ms / (ms + eps)) < 1e-12
    # scale invariance without eps; gain multiplies
    y0 = orc.rmsnorm(x, ones, 0.0)
    y1 = orc.rmsnorm(x * 7.5, ones, 0.0)
    assert np.allclose(y0, y1, rtol=1e-14, atol=0)
    twos = np.full(4096, 0x4000, np.uint16)  # bf16 2.0
    assert np.array_equal(orc.rmsnorm(x, twos, eps), 2.0 * y)


def test_silu_closed_forms():
    assert orc.silu(0.0) == 0.0
    for x in (0.3, 1.0, 2.5, 7.0):
        # x*sigma(x) - (-x)*sigma(-x) = x
        assert abs(orc.silu(x) - orc.silu(-x) - x) < 1e-15
    assert abs(orc.silu(40.0) - 40.0) < 1e-12
    assert abs(orc.silu(-40.0)) < 1e-15
    # silu(ln 3) = ln 3 * 3/4 (sigma(ln 3) = 3/4)
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15


def test_prefetch_list_matches_bruteforce_sort():
    """Top-p by (count desc, index asc) against numpy's stable lexsort of the
    bincount (a library routine), on random selections and on constructed ties."""
    rng = np.random.default_rng(5)
    for E, p, n in [(256, 14, 128), (16, 14, 32), (64, 8, 40), (256, 14, 0)]:
        ids = rng.integers(0, E, size=n).astype(np.int32)
        cnt = np.bincount(ids, minlength=E)
        ref = np.lexsort((np.arange(E), -cnt))[:p]
        assert np.array_equal(orc.prefetch_list(ids, E, p), ref)
    # hand case: counts 3,3,1 at experts 7,2,5 -> [2, 7, 5, then unused 0, 1, ...]
    ids = np.array([7, 2, 7, 2, 5, 7, 2], np.int32)
    assert orc.prefetch_list(ids, 10, 6).tolist() == [2, 7, 5, 0, 1, 3]


# --- NVFP4 activation quantizer (SwiGLU output before the down projection) ----

def _e4m3_positive_values():
    return [orc.e4m3_value(c) for c in range(1, 0x7F)]


def test_e4m3_rne_matches_torch_float8_on_values_midpoints_and_neighbours():
    import torch
    vals = _e4m3_positive_values()
    xs = list(vals)
    for a, b in zip(vals, vals[1:]):
        m = (a + b) / 2.0                      # exact in fp32 (<= 5 significant bits)
        xs += [m, np.nextafter(np.float32(m), np.float32(0)), np.nextafter(np.float32(m), np.float32(1e9))]
    xs += [np.float32(2.0 ** -10), np.float32(2.0 ** -11), np.float32(3 * 2.0 ** -11)]
    x = np.array(xs, np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_rne_sat(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, ref), x[got != ref][:8]
    for big in (448.0, 460.0, 464.0, 1e4):
        assert orc.e4m3_rne_sat(big) == 0x7E
    assert orc.e4m3_rne_sat(0.0) == 0


def _e2m1_bruteforce(y):
    vals = [orc.e2m1_value(c) for c in range(8)]
    a = abs(y)
    if a > 6.0:
        c = 7
    else:
        d = [abs(a - v) for v in vals]
        best = min(d)
        cand = [c for c in range(8) if d[c] == best]
        c = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
    return c | (8 if np.signbit(y) else 0)


def test_e2m1_rne_matches_nearest_even_bruteforce():
    vals = [orc.e2m1_value(c) for c in range(8)]
    ys = []
    for a, b in zip(vals, vals[1:]):
        m = (a + b) / 2.0
        ys += [m, float(np.nextafter(np.float32(m), np.float32(0))), float(np.nextafter(np.float32(m), np.float32(9)))]
    ys += vals + [6.5, 7.0, 100.0, 1e-30, 0.0]
    rng = np.random.default_rng(3)
    ys += list(rng.uniform(0, 7, 400))
    for y in ys + [-y for y in ys]:
        y32 = float(np.float32(y))
        assert orc.e2m1_rne_sat(y32) == _e2m1_bruteforce(y32), y32


def test_nvfp4_quant16_closed_forms():
    vals = np.array([orc.e2m1_value(c) for c in range(8)])
    rng = np.random.default_rng(4)
    for sc in (0x08, 0x30, 0x38, 0x41, 0x66):           # block scales 2^-6 .. 104
        s = orc.e4m3_value(sc)
        q = rng.integers(0, 16, 16)
        x = np.where(q >= 8, -1.0, 1.0) * vals[q % 8] * s
        x[int(rng.integers(0, 16))] = 6.0 * s           # amax = 6 s: the block scale is s itself
        codes, scale, deq = orc.nvfp4_quant16(x.astype(np.float32))
        assert scale == sc
        assert np.array_equal(deq.astype(np.float64), x)
    codes, scale, deq = orc.nvfp4_quant16(np.zeros(16, np.float32))
    assert scale == 0 and not np.any(codes) and not np.any(deq)
    # random blocks: every output is an E2M1 value times the block scale, the
    # one the brute-force nearest-even rule picks for fl32(x / s)
    for _ in range(50):
        x = (rng.standard_normal(16) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        codes, scale, deq = orc.nvfp4_quant16(x)
        s = np.float32(orc.e4m3_value(scale))
        assert s == np.float32(orc.e4m3_value(orc.e4m3_rne_sat(float(np.max(np.abs(x)) / np.float32(6.0)))))
        if s == 0:  # the block scale underflows E4M3: the whole block is 0
            assert not np.any(codes) and not np.any(deq)
            continue
        for i in range(16):
            c = _e2m1_bruteforce(float(x[i] / s))
            assert codes[i] == c
            assert deq[i] == np.float32(orc.e2m1_value(c & 7) * (-1 if c & 8 else 1) * float(s))

"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle step to a closed form, a brute-force enumeration, a
library routine for a special case, a hand-worked value, an invariant, or a
figure the pages print (tests/golden/pages_figures.json).  The cases are
chosen so a plausible slip (dropped term, wrong sign or index, transposed
operand, swapped W1/W3, missing scale) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import moe_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _route_inputs(T, H, E, seed, scale=0.3):
    r = _rng(seed)
    return r.standard_normal((T, H)), r.standard_normal((E, H)) * scale


# ----------------------------------------------------------------- router
def test_softmax_matches_library():
    x, wg = _route_inputs(50, 16, 12, 1)
    l = oracle.gate_logits(x, wg)
    np.testing.assert_allclose(oracle.softmax_rows(l), scipy.special.softmax(l, axis=1), rtol=0, atol=1e-15)


def test_gate_is_x_times_wg_transposed():
    # one-hot gate rows: logits[t, e] = x[t, e] exactly, so the routing is known
    T, E, H = 9, 5, 7
    x = _rng(2).standard_normal((T, H))
    wg = np.zeros((E, H))
    wg[np.arange(E), np.arange(E)] = 1.0
    l = oracle.gate_logits(x, wg)
    np.testing.assert_array_equal(l, x[:, :E])
    r = oracle.route(x, wg, 2)
    expect = np.argsort(-x[:, :E], axis=1)[:, :2]
    np.testing.assert_array_equal(r["ids"], expect)


def test_bias_enters_with_plus_sign():
    E, H, k = 6, 4, 3
    bias = np.array([0.1, 2.0, -1.0, 1.5, 0.0, 3.0])
    r = oracle.route(np.zeros((2, H)), _rng(3).standard_normal((E, H)), k, bias)
    np.testing.assert_array_equal(r["ids"], [[5, 1, 3]] * 2)
    sel = bias[[5, 1, 3]]
    np.testing.assert_allclose(r["w"][0], np.exp(sel) / np.exp(sel).sum(), atol=1e-15)


def test_selected_weights_sum_to_one():
    x, wg = _route_inputs(200, 32, 16, 4)
    for k in (1, 2, 5, 16):
        r = oracle.route(x, wg, k)
        np.testing.assert_allclose(r["w"].sum(axis=1), 1.0, atol=1e-12)


def test_k2_weight_is_sigmoid_of_logit_gap():
    x, wg = _route_inputs(100, 24, 8, 5)
    r = oracle.route(x, wg, 2)
    l = np.take_along_axis(r["logits"], r["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(r["w"][:, 0], 1.0 / (1.0 + np.exp(l[:, 1] - l[:, 0])), atol=1e-14)


def test_weights_are_softmax_of_selected_logits():
    x, wg = _route_inputs(64, 24, 32, 6)
    r = oracle.route(x, wg, 6)
    l = np.take_along_axis(r["logits"], r["ids"].astype(np.int64), axis=1)
    np.testing.assert_allclose(r["w"], scipy.special.softmax(l, axis=1), atol=1e-14)
    # p_sel is the full softmax at the selected experts, descending
    assert np.all(np.diff(r["p_sel"], axis=1) <= 0)


def test_topk_brute_force_with_ties():
    T, H, E, k = 24, 6, 6, 3
    x, wg = _route_inputs(T, H, E, 7, scale=1.0)
    x[3] = 0.0                 # exact ties across all experts
    x[10] = 0.0
    wg[4] = wg[2]              # experts 2 and 4 always tie
    r = oracle.route(x, wg, k)
    p = r["p"]
    for t in range(T):
        best, best_key = None, None
        for sub in itertools.combinations(range(E), k):
            key = (-sum(p[t, list(sub)]), sub)       # max total p, then lexicographic
            if best_key is None or key < best_key:
                best, best_key = sub, key
        got = list(r["ids"][t])
        assert sorted(got) == list(best), (t, got, best)
        pv = p[t, got]
        assert np.all(np.diff(pv) <= 0)
        for a in range(k - 1):                          # equal p -> lower id first
            if pv[a] == pv[a + 1]:
                assert got[a] < got[a + 1]


def test_zero_row_routes_to_first_k_experts():
    for E, k in ((8, 2), (256, 8), (64, 6)):
        r = oracle.route(np.zeros((3, 16)), _rng(8).standard_normal((E, 16)), k)
        np.testing.assert_array_equal(r["ids"], np.tile(np.arange(k), (3, 1)))
        np.testing.assert_allclose(r["w"], 1.0 / k, atol=1e-15)


# ----------------------------------------------------------------- quantisation
def test_quant_rounding_half_even_and_scale():
    x = np.array([[2.5, 1.5, 0.5, -0.5, -63.5, 127.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0, 0.0],
                  [-254.0, 1.0, 3.0, 0.0, 0.0, 2.0]], dtype=np.float32)
    q, s = oracle.quant_per_token_int8(x)
    np.testing.assert_array_equal(q[0], [2, 2, 0, 0, -64, 127])
    np.testing.assert_array_equal(q[1], 0)
    assert s[0] == np.float32(1.0) and s[1] == np.float32(1.0) and s[2] == np.float32(2.0)
    np.testing.assert_array_equal(q[2], [-127, 0, 2, 0, 0, 1])      # 0.5 -> 0, 1.5 -> 2, 1.0 -> 1
    assert q.dtype == np.int8 and s.dtype == np.float32


def test_quant_error_bound_and_range():
    x = (_rng(9).standard_normal((300, 257)) * _rng(10).uniform(0.01, 30, (300, 1))).astype(np.float32)
    q, s = oracle.quant_per_token_int8(x)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    np.testing.assert_array_equal(np.abs(q.astype(np.int32)).max(axis=1), 127)
    assert q.min() >= -127


# ----------------------------------------------------------------- align
def _align_brute(ids, E, C):
    """The definition, slot by slot: rank = earlier slots on the same expert."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    n = len(flat)
    rank = [sum(1 for s2 in range(s) if flat[s2] == flat[s]) for s in range(n)]
    counts = [flat.count(e) for e in range(E)]
    kept = [c if C is None else min(c, C) for c in counts]
    pos, sorted_slot = [], [-1] * n
    for s in range(n):
        if C is not None and rank[s] >= C:
            pos.append(-1)
        else:
            p = sum(kept[:flat[s]]) + rank[s]
            pos.append(p)
            sorted_slot[p] = s
    return counts, kept, pos, sorted_slot, n - sum(kept)


@pytest.mark.parametrize("T,E,k,C", [(30, 5, 2, None), (30, 5, 2, 7), (40, 9, 3, 4), (17, 4, 4, 3), (1, 3, 1, None)])
def test_align_brute_force(T, E, k, C):
    r = _rng(T * 100 + E)
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    a = oracle.align(ids, E, C)
    counts, kept, pos, sorted_slot, nd = _align_brute(ids, E, C)
    np.testing.assert_array_equal(a["counts"], counts)
    np.testing.assert_array_equal(a["kept"], kept)
    np.testing.assert_array_equal(a["pos"].reshape(-1), pos)
    np.testing.assert_array_equal(a["sorted_slot"], sorted_slot)
    assert a["num_dropped"] == nd
    assert a["counts"].sum() == T * k
    assert a["kept"].sum() == T * k - a["num_dropped"]
    np.testing.assert_array_equal(a["offsets"], np.concatenate([[0], np.cumsum(kept)]))


def test_drop_rule_first_come_first_served():
    # every token routes to experts {0, 1}: exactly the first C tokens are kept
    T, E, k, C = 50, 4, 2, 13
    ids = np.tile([0, 1], (T, 1))
    a = oracle.align(ids, E, C)
    kept = a["pos"] >= 0
    np.testing.assert_array_equal(kept[:, 0], np.arange(T) < C)
    np.testing.assert_array_equal(kept[:, 1], np.arange(T) < C)
    np.testing.assert_array_equal(a["pos"][:C, 0], np.arange(C))
    np.testing.assert_array_equal(a["pos"][:C, 1], C + np.arange(C))
    assert a["num_dropped"] == 2 * (T - C)


def test_kept_counts_invariant_under_token_permutation():
    T, E, k = 300, 16, 4
    r = _rng(11)
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    C = oracle.capacity(T, k, E, 0.8)
    a = oracle.align(ids, E, C)
    b = oracle.align(ids[r.permutation(T)], E, C)
    np.testing.assert_array_equal(a["kept"], b["kept"])
    assert a["num_dropped"] == b["num_dropped"] > 0


def test_capacity_closed_forms():
    assert oracle.capacity(4096, 8, 256, 1.25) == 160
    assert oracle.capacity(16384, 6, 64, 1.25) == 1920
    assert oracle.capacity(10, 3, 4, 1.25) == 10          # 9.375 rounds up
    assert oracle.capacity(64, 2, 8, 0.0) is None
    # factors written in decimal: the decimal value decides, not its binary float
    # (the double nearest 1.1 lies above it, so a float product would round to 12)
    assert oracle.capacity(80, 2, 16, 1.1) == 11
    assert oracle.capacity(100, 1, 10, 1.1) == 11
    assert oracle.capacity(7, 1, 3, 1.1) == 3           # ceil(2.566...)


def test_capacity_is_the_decimal_ceiling():
    """C = ceil(f * T * k / E) with f the decimal the caller wrote, computed in
    exact rationals from the decimal string (not from the oracle's float)."""
    from fractions import Fraction
    factors = ["0.1", "0.3", "0.7", "1.0", "1.05", "1.1", "1.15", "1.2", "1.25", "1.3", "1.35", "1.5", "1.7",
               "1.9", "2.2", "2.5", "3.3", "1.333", "0.001"]
    loads = [(80, 2, 16), (100, 1, 10), (4096, 8, 256), (16384, 6, 64), (7, 1, 3), (1000, 3, 7), (30, 1, 9),
             (65536, 8, 256), (12, 5, 11)]
    for f in factors:
        for T, k, E in loads:
            want = math.ceil(Fraction(f) * Fraction(T * k, E))
            assert oracle.capacity(T, k, E, float(f)) == want, (f, T, k, E)


def test_tiles_cover_rows():
    offsets = np.array([0, 0, 5, 5, 300, 301])
    t = oracle.tiles(offsets, 128)
    assert t == [(1, 0, 5), (3, 5, 128), (3, 133, 128), (3, 261, 39), (4, 300, 1)]


# ----------------------------------------------------------------- FFN / combine
def test_swiglu_hand_worked():
    a = np.array([[1.0, 2.0]])
    out = oracle.swiglu_ffn(a, np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]]), np.array([[1.0], [-1.0]]))
    h = 2.0 / (1.0 + math.exp(-1.0))          # silu(1) * 2
    np.testing.assert_allclose(out, [[h, -h]], atol=1e-15)


def test_swiglu_gate_and_up_roles():
    r = _rng(12)
    a = np.abs(r.standard_normal((4, 8))) + 0.1
    w3 = r.standard_normal((5, 8))
    w2 = r.standard_normal((8, 5))
    w1_neg = -np.ones((5, 8)) * 10.0       # gate far negative: silu ~ 0
    assert np.abs(oracle.swiglu_ffn(a, w1_neg, w3, w2)).max() < 1e-6
    w1_pos = np.ones((5, 8)) * 10.0        # gate far positive: silu(g) ~ g
    ref = ((a @ w1_pos.T) * (a @ w3.T)) @ w2.T
    np.testing.assert_allclose(oracle.swiglu_ffn(a, w1_pos, w3, w2), ref, rtol=1e-9)
    z = np.linspace(-5, 5, 11)
    np.testing.assert_allclose(oracle.silu(-z), oracle.silu(z) - z, atol=1e-14)


def _small_inputs(T, H, E, k, I, w_dtype="f32", cap=0.0, seed=77, x_dtype="f32", wg_dtype="f32"):
    spec = moe_synth.Spec("t", T, H, E, k, I, x_dtype=x_dtype, wg_dtype=wg_dtype, w_dtype=w_dtype,
                          out_dtype="f32", capacity_factor=cap)
    return moe_synth.make_inputs(spec, seed, threads=2)


def _layer(inp, **kw):
    s = inp.spec
    args = dict(x=inp.x, x_dtype=s.x_dtype, wg=inp.wg, wg_dtype=s.wg_dtype, bias=inp.bias, w13=inp.w13,
                w2=inp.w2, w_dtype=s.w_dtype, k=s.k, capacity_factor=s.capacity_factor, s13=inp.s13, s2=inp.s2)
    args.update(kw)
    return args


def test_single_expert_is_dense_ffn():
    inp = _small_inputs(20, 16, 1, 1, 24)
    out = oracle.layer(**_layer(inp))["out"]
    x = inp.x.astype(np.float64)
    w1, w3 = inp.w13[0, :24].astype(np.float64), inp.w13[0, 24:].astype(np.float64)
    g = np.einsum("th,ih->ti", x, w1)
    u = np.einsum("th,ih->ti", x, w3)
    ref = np.einsum("ti,hi->th", g * scipy.special.expit(g) * u, inp.w2[0].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_identical_experts_reduce_to_one_ffn():
    inp = _small_inputs(40, 16, 6, 3, 8)
    inp.w13[:] = inp.w13[0]
    inp.w2[:] = inp.w2[0]
    out = oracle.layer(**_layer(inp))["out"]
    ref = oracle.swiglu_ffn(inp.x.astype(np.float64), inp.w13[0, :8].astype(np.float64),
                            inp.w13[0, 8:].astype(np.float64), inp.w2[0].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-14)


def test_k_equals_e_is_dense_soft_mixture():
    T, H, E, I = 12, 8, 4, 6
    inp = _small_inputs(T, H, E, E, I)
    out = oracle.layer(**_layer(inp))["out"]
    x = inp.x.astype(np.float64)
    p = scipy.special.softmax(x @ inp.wg.astype(np.float64).T, axis=1)
    ref = np.zeros((T, H))
    for e in range(E):
        w13 = inp.w13[e].astype(np.float64)
        ref += p[:, e:e + 1] * oracle.swiglu_ffn(x, w13[:I], w13[I:], inp.w2[e].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("w_dtype,cap", [("f32", 0.0), ("f32", 0.6), ("i8", 0.0), ("i8", 0.7), ("bf16", 1.0),
                                         ("i4", 0.0), ("i4", 0.6), ("i4a8", 0.6)])
def test_expert_major_equals_token_major(w_dtype, cap):
    inp = _small_inputs(48, 32, 8, 3, 16, w_dtype=w_dtype, cap=cap,
                        x_dtype="bf16" if w_dtype != "f32" else "f32")
    res = oracle.layer(**_layer(inp))
    if cap > 0:
        assert res["align"]["num_dropped"] > 0 or cap >= 1.0
    ref = oracle.layer_token_major(**_layer(inp))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-13)


def test_fully_dropped_token_gives_zero_and_no_renormalisation():
    T, H, E, k, I = 30, 8, 4, 2, 4
    inp = _small_inputs(T, H, E, k, I)
    inp.wg[:] = 0.0
    inp.wg[0, 0] = inp.wg[1, 1] = 1.0
    inp.x[:, 0] = 5.0 + np.arange(T)          # expert 0 first, expert 1 second for every token
    inp.x[:, 1] = 4.0 + np.arange(T)
    inp.x[:, 2:] = 0.0
    res = oracle.layer(**_layer(inp, capacity_factor=0.5))          # C = ceil(0.5*60/4) = 8
    assert res["capacity"] == 8
    np.testing.assert_array_equal(res["out"][8:], 0.0)
    y0 = oracle.swiglu_ffn(inp.x[:8].astype(np.float64), inp.w13[0, :I].astype(np.float64),
                           inp.w13[0, I:].astype(np.float64), inp.w2[0].astype(np.float64))
    y1 = oracle.swiglu_ffn(inp.x[:8].astype(np.float64), inp.w13[1, :I].astype(np.float64),
                           inp.w13[1, I:].astype(np.float64), inp.w2[1].astype(np.float64))
    w = res["route"]["w"][:8]
    np.testing.assert_allclose(res["out"][:8], w[:, :1] * y0 + w[:, 1:] * y1, rtol=1e-12)


def test_output_permutation_equivariant_without_drops():
    inp = _small_inputs(32, 16, 8, 2, 8)
    perm = _rng(13).permutation(32)
    a = oracle.layer(**_layer(inp))["out"]
    b = oracle.layer(**_layer(inp, x=inp.x[perm]))["out"]
    np.testing.assert_allclose(b, a[perm], rtol=1e-13, atol=1e-15)


# ----------------------------------------------------------------- W8A8
def test_w8a8_integer_products_exact():
    r = _rng(14)
    a = r.integers(-128, 128, (64, 2048)).astype(np.int8)
    b = r.integers(-127, 128, (96, 2048)).astype(np.int8)
    exact = a.astype(np.int64) @ b.astype(np.int64).T
    np.testing.assert_array_equal((a.astype(np.float64) @ b.astype(np.float64).T).astype(np.int64), exact)


def test_w8a8_close_to_dequantised_fp64_layer():
    T, H, E, k, I = 64, 64, 4, 2, 32
    inp = _small_inputs(T, H, E, k, I, w_dtype="i8", x_dtype="bf16")
    q = oracle.layer(**_layer(inp))["out"]
    w13 = (inp.w13.astype(np.float64) * inp.s13[:, :, None]).astype(np.float32)
    w2 = (inp.w2.astype(np.float64) * inp.s2[:, :, None]).astype(np.float32)
    ref = oracle.layer(**_layer(inp, w13=w13, w2=w2, w_dtype="f32", s13=None, s2=None))["out"]
    rel = np.linalg.norm(q - ref) / np.linalg.norm(ref)
    assert 1e-4 < rel < 2e-2, rel


def _w8a8_hand_case():
    """One token, H = 4, I = 2, one expert, k = 1 (weight 1).

    x = (127, -3, 2.5, 0.5): absmax 127, so the per-token scale is exactly 1
    and the codes are the half-even roundings (127, -3, 2, 0).
    W1 codes (0,0,16,0), (0,0,2,0) with scales 1, 1:        g = (32, 4)
    W3 codes (2,-1,0,0), (0,0,-8,0) with scales 1/32, 1:    u = (257/32, -16)
    h = silu(g) * u = (257 / (1 + e^-32), -64 / (1 + e^-4))
      in fp32: (257, -62.849...);  in bf16: (256, -62.75)
      (257 is the tie between 256 and 258: even mantissa 256; bf16 steps by
      1/4 between 32 and 64, and -62.849 is nearest -62.75)
    row scale s_h = 256 / 127 (fp32 division), codes round(h / s_h) =
      (127, round(-31.13)) = (127, -31)
    W2 codes (1,0), (0,1), (2,-3), (-1,1) with scales (1, 1/2, 1/4, 1):
      acc2 = (127, -31, 347, -158), y = acc2 * s_h * s2."""
    x = np.array([[127.0, -3.0, 2.5, 0.5]], dtype=np.float32)
    wg = np.zeros((1, 4), dtype=np.float32)
    w13 = np.array([[[0, 0, 16, 0], [0, 0, 2, 0], [2, -1, 0, 0], [0, 0, -8, 0]]], dtype=np.int8)
    s13 = np.array([[1.0, 1.0, 1.0 / 32.0, 1.0]], dtype=np.float32)
    w2 = np.array([[[1, 0], [0, 1], [2, -3], [-1, 1]]], dtype=np.int8)
    s2 = np.array([[1.0, 0.5, 0.25, 1.0]], dtype=np.float32)
    return x, wg, w13, s13, w2, s2


def test_w8a8_hand_worked():
    """The W8A8 FFN step by step ([LightOP] section 4.1: per-token int8
    quantisation of each GEMM's input, integer accumulation, dequantisation
    by the row scale times the channel scale; h held in bf16 between the
    GEMMs, reading R7).  A variant that skips the re-quantisation of h,
    quantises h per column, or leaves out its bf16 rounding lands off the
    hand-worked output by far more than the 1e-12 used here."""
    x, wg, w13, s13, w2, s2 = _w8a8_hand_case()
    res = oracle.layer(x, "f32", wg, "f32", None, w13, w2, "i8", 1, 0.0, s13, s2)
    np.testing.assert_array_equal(res["xq"], [[127, -3, 2, 0]])
    assert res["xs"][0] == np.float32(1.0)
    # h: the fp32 values, then the bf16 ones, by hand (see _w8a8_hand_case)
    g = np.array([32.0, 4.0])
    u = np.array([257.0 / 32.0, -16.0])
    h32 = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    assert h32[0] == np.float32(257.0) and -62.86 < h32[1] < -62.84
    hb = np.array([256.0, -62.75])
    s_h = float(np.float32(256.0) / np.float32(127.0))
    hq = np.array([127.0, -31.0])
    assert abs(hb[1] / s_h - (-31.13)) < 1e-3
    acc2 = np.array([[1, 0], [0, 1], [2, -3], [-1, 1]], dtype=np.float64) @ hq
    np.testing.assert_array_equal(acc2, [127.0, -31.0, 347.0, -158.0])
    want = acc2 * s_h * s2[0].astype(np.float64)
    np.testing.assert_allclose(res["out"][0], want, rtol=1e-12, atol=0)

    # the slips this pin must catch: each lands far outside 1e-12
    w2f = np.array([[1, 0], [0, 1], [2, -3], [-1, 1]], dtype=np.float64) * s2[0].astype(np.float64)[:, None]
    no_requant = w2f @ hb                                    # h straight into the second GEMM
    per_column = w2f @ hb                                    # one scale per column: codes +-127 give back h
    s_h32 = float(np.float32(257.0) / np.float32(127.0))     # h left in fp32
    no_bf16 = w2f @ (np.rint(h32.astype(np.float64) / s_h32) * s_h32)
    for slip in (no_requant, per_column, no_bf16):
        assert np.max(np.abs(slip - want) / np.abs(want)) > 1e-3


# ----------------------------------------------------------------- the pages' figures
def test_pages_figures():
    g = json.load(open(GOLDEN))
    d = g["dispatch_volume"]
    ids = np.stack([np.arange(d["top_k"]) + (t % 32) * 8 for t in range(d["tokens"])])
    a = oracle.align(ids, d["num_experts"], None)
    n_rows = int(a["offsets"][-1])
    assert n_rows == d["expert_accesses"] == d["tokens"] * d["top_k"]
    assert d["hidden"] * 2 == d["bytes_per_row"]
    assert n_rows * d["bytes_per_row"] == d["total_bytes_approx"]
    r = g["router_params"]
    assert abs(r["hidden"] * r["num_experts"] - r["params_approx"]) / r["params_approx"] < 0.05
    h = g["unfused_hbm_passes"]
    assert sum(v[0] for k, v in h.items() if isinstance(v, list)) == h["total_reads"]
    assert sum(v[1] for k, v in h.items() if isinstance(v, list)) == h["total_writes"]
    assert oracle.capacity(4096, 8, 256, g["capacity_factor"]["factor"]) == 160


# ---------------------------------------------------------- combine_shared
def test_combine_shared_closed_forms():
    """R8: the shared-expert term and the bias are added to the routed sum.
    Pins: every slot dropped leaves exactly factor*S + b; the difference from
    the plain combine is factor*S + b whatever the routing; factor 0 and no
    bias give the plain combine; a lone kept slot with weight 1 and a zero
    shared term reproduces the expert row plus b."""
    rng = np.random.default_rng(11)
    T, k, H, N = 9, 3, 16, 20
    y = rng.standard_normal((N, H))
    pos = rng.integers(-1, N, size=(T, k))
    w = rng.random((T, k))
    S = rng.standard_normal((T, H))
    b = rng.standard_normal(H)
    f = -0.75
    dropped = np.full((T, k), -1)
    np.testing.assert_array_equal(oracle.combine_shared(y, dropped, w, S, f, b), f * S + b[None, :])
    diff = oracle.combine_shared(y, pos, w, S, f, b) - oracle.combine(y, pos, w)
    np.testing.assert_allclose(diff, f * S + b[None, :], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(oracle.combine_shared(y, pos, w, S, 0.0, None), oracle.combine(y, pos, w))
    np.testing.assert_array_equal(oracle.combine_shared(y, pos, w, None, f, None), oracle.combine(y, pos, w))
    one = np.full((1, k), -1)
    one[0, 1] = 7
    got = oracle.combine_shared(y, one, np.ones((1, k)), np.zeros((1, H)), 3.0, b)
    np.testing.assert_array_equal(got[0], y[7] + b)


# ----------------------------------------------------------- route_grouped
def _identity_gate(logits):
    """x = the logits, Wg = identity: the router sees exactly these logits."""
    logits = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    return logits, np.eye(logits.shape[1])


def test_route_grouped_hand_worked():
    """E=8 in 4 groups of 2, 2 groups kept, top-2.  Probabilities
    (.26 .01 | .20 .15 | .19 .17 | .01 .01): group scores .27 .35 .36 .02, so
    groups 2 and 1 are kept and the global favourite, expert 0, is excluded;
    the top-2 among experts 2..5 is (2, 4) with weights .20/.39 and .19/.39.
    The plain router would pick (0, 2)."""
    p = np.array([0.26, 0.01, 0.20, 0.15, 0.19, 0.17, 0.01, 0.01])
    x, wg = _identity_gate(np.log(p))
    r = oracle.route_grouped(x, wg, 2, 4, 2)
    np.testing.assert_allclose(r["group_scores"][0], [0.27, 0.35, 0.36, 0.02], rtol=1e-12)
    np.testing.assert_array_equal(r["groups"][0], [1, 2])
    np.testing.assert_array_equal(r["ids"][0], [2, 4])
    np.testing.assert_allclose(r["w"][0], [0.20 / 0.39, 0.19 / 0.39], rtol=1e-12)
    np.testing.assert_allclose(r["p_sel"][0], [0.20, 0.19], rtol=1e-12)
    np.testing.assert_array_equal(oracle.route(x, wg, 2)["ids"][0], [0, 2])


def test_route_grouped_reduces_to_plain_route():
    """Keeping every group, or groups of one expert with k <= topk_group,
    leaves the plain top-k."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((50, 24))
    wg = rng.standard_normal((16, 24))
    b = rng.standard_normal(16)
    plain = oracle.route(x, wg, 3, b)
    for G in (1, 2, 4, 8, 16):
        r = oracle.route_grouped(x, wg, 3, G, G, b)
        np.testing.assert_array_equal(r["ids"], plain["ids"])
        np.testing.assert_array_equal(r["w"], plain["w"])
    for TG in (3, 5, 16):
        r = oracle.route_grouped(x, wg, 3, 16, TG, b)
        np.testing.assert_array_equal(r["ids"], plain["ids"])


@pytest.mark.parametrize("E,G,TG,k", [(12, 4, 2, 3), (8, 4, 1, 2), (12, 3, 2, 5), (6, 2, 1, 3)])
def test_route_grouped_brute_force(E, G, TG, k):
    """Every subset of TG groups and every k-subset of their experts, scored
    from the definition: a group's score is its best pair sum, the kept groups
    maximise the summed score, the kept experts maximise the summed
    probability among the kept groups' experts."""
    rng = np.random.default_rng(E * 100 + G * 10 + TG)
    x = rng.standard_normal((40, 8))
    wg = rng.standard_normal((E, 8))
    r = oracle.route_grouped(x, wg, k, G, TG)
    p = oracle.softmax_rows(x @ wg.T)
    gsz = E // G
    for t in range(x.shape[0]):
        score = []
        for g in range(G):
            members = range(g * gsz, (g + 1) * gsz)
            if gsz == 1:
                score.append(p[t, g])
            else:
                score.append(max(p[t, i] + p[t, j] for i, j in itertools.combinations(members, 2)))
        best_groups = max(itertools.combinations(range(G), TG), key=lambda c: sum(score[g] for g in c))
        cand = [e for g in best_groups for e in range(g * gsz, (g + 1) * gsz)]
        best = max(itertools.combinations(cand, k), key=lambda c: sum(p[t, e] for e in c))
        assert set(r["ids"][t]) == set(best), t
        assert tuple(r["groups"][t]) == tuple(sorted(best_groups)), t
        assert np.all(np.diff(p[t, r["ids"][t]]) <= 0)


def test_route_grouped_ties_and_invariants():
    # groups 0 and 1 score the same: the lower group wins, then the lower ids
    x, wg = _identity_gate([0.0, 0.0, 0.0, 0.0, -5.0, -5.0, -5.0, -5.0])
    r = oracle.route_grouped(x, wg, 2, 4, 1)
    np.testing.assert_array_equal(r["groups"][0], [0])
    np.testing.assert_array_equal(r["ids"][0], [0, 1])
    np.testing.assert_allclose(r["w"][0], [0.5, 0.5], rtol=0, atol=0)
    # random rows: ids lie in at most TG groups, weights sum to 1, and every
    # selected probability beats every other candidate of the kept groups
    rng = np.random.default_rng(3)
    E, G, TG, k = 64, 8, 3, 6
    x = rng.standard_normal((200, 32))
    wg = rng.standard_normal((E, 32))
    r = oracle.route_grouped(x, wg, k, G, TG)
    gsz = E // G
    for t in range(200):
        gs = set(int(i) // gsz for i in r["ids"][t])
        assert gs <= set(r["groups"][t].tolist()) and len(r["groups"][t]) == TG
        cand = [e for g in r["groups"][t] for e in range(g * gsz, (g + 1) * gsz) if e not in r["ids"][t]]
        assert r["p"][t, r["ids"][t]].min() >= r["p"][t, cand].max()
    np.testing.assert_allclose(r["w"].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.route_grouped(x, wg, k, 7, 3)          # E not a multiple of n_group
    with pytest.raises(ValueError):
        oracle.route_grouped(x, wg, 9, 8, 1)          # k beyond one group's 8 experts


# ------------------------------------------------------------------- W4A16
def test_w4a16_hand_worked():
    """One token, H=2, I=1.  x = (1, 2); W1 codes (1, -1) at scale 1/2 give
    g = -1/2; W3 codes (2, 1) at scale 1/4 give u = 1; W2 codes (3, -8) at
    scales (1, 1/2) give y = (3, -4) * silu(-1/2)."""
    spec = moe_synth.Spec("w4", 1, 2, 1, 1, 1, x_dtype="f32", wg_dtype="f32", w_dtype="i4", out_dtype="f32")
    x = np.array([[1.0, 2.0]], dtype=np.float32)
    wg = np.zeros((1, 2), dtype=np.float32)
    w13 = np.array([[[1, -1], [2, 1]]], dtype=np.int8)
    s13 = np.array([[0.5, 0.25]], dtype=np.float32)
    w2 = np.array([[[3], [-8]]], dtype=np.int8)
    s2 = np.array([[1.0, 0.5]], dtype=np.float32)
    res = oracle.layer(x, "f32", wg, "f32", None, w13, w2, "i4", 1, 0.0, s13, s2)
    h = -0.5 / (1.0 + math.exp(0.5))
    np.testing.assert_allclose(res["out"][0], [3.0 * h, -4.0 * h], rtol=1e-15)
    assert spec.w_dtype == "i4"


def test_w4a16_scales_are_per_output_row():
    """Unit scales give the layer of float weights equal to the codes; a
    scale on W2 rows or on W3 rows scales those outputs linearly, a scale on
    W1 rows does not (it passes through silu); a transposed scale (per input
    column) would break the first check of each pair."""
    inp = _small_inputs(24, 32, 4, 2, 16, w_dtype="i4", x_dtype="bf16")
    I = 16
    ones13 = np.ones_like(inp.s13)
    ones2 = np.ones_like(inp.s2)
    base = _layer(inp, s13=ones13, s2=ones2)
    out1 = oracle.layer(**base)["out"]
    as_f32 = dict(base, w13=inp.w13.astype(np.float32), w2=inp.w2.astype(np.float32), w_dtype="f32")
    np.testing.assert_allclose(out1, oracle.layer(**as_f32)["out"], rtol=1e-13, atol=1e-13)
    # W2 row h scaled by 3: output column h scaled by 3, others unchanged
    s2 = ones2.copy()
    s2[:, 5] = 3.0
    out2 = oracle.layer(**dict(base, s2=s2))["out"]
    np.testing.assert_allclose(out2[:, 5], 3.0 * out1[:, 5], rtol=1e-12)
    np.testing.assert_array_equal(np.delete(out2, 5, axis=1), np.delete(out1, 5, axis=1))
    # every W3 row scaled by 2: the whole output doubles
    s13 = ones13.copy()
    s13[:, I:] = 2.0
    np.testing.assert_allclose(oracle.layer(**dict(base, s13=s13))["out"], 2.0 * out1, rtol=1e-12, atol=1e-14)
    # every W1 row scaled by 2: not linear
    s13 = ones13.copy()
    s13[:, :I] = 2.0
    assert not np.allclose(oracle.layer(**dict(base, s13=s13))["out"], 2.0 * out1, rtol=1e-3)
    # dequant_rows is codes times the row's scale
    q = np.array([[-8, 7], [1, -1]], dtype=np.int8)
    np.testing.assert_array_equal(oracle.dequant_rows(q, np.array([0.5, 4.0])), [[-4.0, 3.5], [4.0, -4.0]])


def test_int4_codes_in_range():
    inp = moe_synth.make_inputs(moe_synth.Spec("w4", 8, 128, 4, 2, 64, w_dtype="i4"), 3)
    for q in (inp.w13, inp.w2):
        assert q.dtype == np.int8 and q.min() >= -8 and q.max() <= 7
        assert q.min() == -8 and q.max() == 7      # both ends occur
    assert inp.s13.shape == (4, 128) and inp.s2.shape == (4, 128)


# -------------------------------------------------------------------- W4A8
def test_w4a8_is_w8a8_on_int4_codes():
    """W4A8 (R11) is the W8A8 pipeline (R7) run on int4 codes: the same
    numbers when the same codes are given as int8 weights; and it differs
    from W4A16 only by the activation and h quantisation (small)."""
    inp = _small_inputs(40, 64, 8, 2, 32, w_dtype="i4a8", x_dtype="bf16", cap=0.8)
    a = oracle.layer(**_layer(inp))["out"]
    b = oracle.layer(**_layer(inp, w_dtype="i8"))["out"]
    np.testing.assert_array_equal(a, b)
    c = oracle.layer(**_layer(inp, w_dtype="i4"))["out"]
    rel = np.linalg.norm(a - c) / np.linalg.norm(c)
    assert 0 < rel < 5e-2, rel
    assert inp.w13.min() >= -8 and inp.w13.max() <= 7


def test_layer_options_compose_the_pinned_steps():
    """The layer with group-limited routing and a shared expert is the plain
    composition of the pinned steps: route_grouped's ids and weights through
    the same FFN, merged by combine_shared; with every group kept, no shared
    term and no bias it is the plain layer."""
    inp = _small_inputs(40, 32, 16, 3, 16, cap=0.9)
    base = oracle.layer(**_layer(inp))
    same = oracle.layer(**_layer(inp, n_group=4, topk_group=4))
    np.testing.assert_array_equal(same["out"], base["out"])
    rng = np.random.default_rng(4)
    S = rng.standard_normal((40, 32))
    b = rng.standard_normal(32)
    res = oracle.layer(**_layer(inp, n_group=4, topk_group=2, shared=S, shared_factor=0.5, out_bias=b))
    r = oracle.route_grouped(inp.x.astype(np.float64), inp.wg.astype(np.float64), 3, 4, 2)
    np.testing.assert_array_equal(res["route"]["ids"], r["ids"])
    plain = oracle.layer(**_layer(inp, n_group=4, topk_group=2))
    np.testing.assert_allclose(res["out"], plain["out"] + 0.5 * S + b[None, :], rtol=1e-12, atol=1e-12)


def test_round_bf16_is_nearest_with_ties_to_even():
    """round_bf16 (R7's h storage) against brute force: of the two bf16
    values around x (x truncated to 16 bits, and the next one up in
    magnitude), the nearer, and the one with an even last bit on a tie."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 4000),
                        np.float32([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 0.0, -0.0])])
    got = oracle.round_bf16(x)
    for xi, gi in zip(x.tolist(), got.tolist()):
        b = np.float32(xi).view(np.uint32)
        lo = np.uint32(b & 0xFFFF0000)
        hi = np.uint32(lo + 0x10000)
        flo, fhi = float(lo.view(np.float32)), float(hi.view(np.float32))
        dlo, dhi = abs(xi - flo), abs(fhi - xi)
        want = flo if (dlo < dhi or (dlo == dhi and ((int(lo) >> 16) & 1) == 0)) else fhi
        assert gi == want, (xi, gi, want)
    assert oracle.round_bf16(np.float32([1 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.float32([1 + 3 * 2.0 ** -8]))[0] == np.float32(1 + 2.0 ** -6)

"""Pins of the fp64 CPU oracle against things other than itself.

* router selection: brute force over every group subset and every expert subset
  (exact rational sums) on tiny seeded inputs, including constructed exact ties;
* special cases that reduce to a library routine (one group: a stable argsort;
  zero bias: top-k of the logits);
* closed-form weights (tests/golden/router_hand_example.json) and the invariant
  sum(w) = routed_scaling_factor;
* fp16 / bf16 decoders against numpy over every bit pattern; dequantisation
  against the closed form q * s computed with numpy;
* the expert FFN and the routed + shared composition against numpy float64
  matmuls on independently dequantised matrices; zero input gives exactly zero;
  a single routed expert gets weight rsf exactly.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from gen import inputs as gen
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cfg_of(E, G, Gk, k, rsf=2.5, norm=1, H=8, I=32):
    return gen.LayerConfig(hidden=H, n_experts=E, n_group=G, topk_group=Gk, top_k=k, moe_inter=I,
                           shared_inter=I, routed_scaling_factor=rsf, norm_topk_prob=norm)


# ------------------------------------------------------------------ decoders

def test_f16_decoder_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    mine = np.array([O.f16_to_f64(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all((ref == mine) | both_nan)
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(mine[~both_nan]))


def test_bf16_decoder_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    mine = np.array([O.bf16_to_f64(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.all((ref == mine) | both_nan)


def numpy_dequant(q, s, gsz=32):
    """Independent closed form: offset-binary nibbles (low nibble = even element) times fp16 scales."""
    lo = (q & 0x0F).astype(np.int64) - 8
    hi = (q >> 4).astype(np.int64) - 8
    vals = np.empty((q.shape[0], q.shape[1] * 2), np.float64)
    vals[:, 0::2] = lo
    vals[:, 1::2] = hi
    sc = np.repeat(s.view(np.float16).astype(np.float64), gsz, axis=1)
    return vals * sc


def test_dequant_closed_form():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (7, 48), dtype=np.uint8)
    s = gen.encode_f16(np.abs(rng.normal(0, 0.02, (7, 3))))
    s[0, 0] = 0x0001  # smallest subnormal
    s[1, 1] = 0x7BFF  # largest normal
    got = O.dequant(q, s)
    assert np.array_equal(got, numpy_dequant(q, s))
    # q * s is exact in fp32 as well (4-bit integer times 11-bit significand)
    assert np.array_equal(got.astype(np.float32).astype(np.float64), got)


def test_nibble_order_and_offset_binary():
    # byte 0x8F: low nibble 15 -> +7 at element 0, high nibble 8 -> 0 at element 1
    q = np.array([[0x8F, 0x07]], np.uint8)
    s = gen.encode_f16(np.ones((1, 1)))
    q32 = np.zeros((1, 16), np.uint8)
    q32[0, :2] = q[0]
    got = O.dequant(q32, s)[0, :4]
    assert list(got) == [7.0, 0.0, -1.0, -8.0]


# ------------------------------------------------------------- router: brute force

def brute_force_select(E, G, Gk, k, s, bias, rsf=2.5, norm=1):
    """Every subset, exact rational sums: the kept groups are the Gk-subset of
    maximal total score (ties: lexicographically smallest), the experts the
    k-subset of maximal total key among the kept ones (ties likewise); rank by
    key desc then index asc."""
    per = E // G
    key = [np.float32(np.float64(s[e]) + np.float64(bias[e])) for e in range(E)]
    kf = [Fraction(float(v)) for v in key]
    gscore = []
    for j in range(G):
        mem = list(range(j * per, (j + 1) * per))
        if per == 1:
            best = kf[mem[0]]
        else:
            best = max(kf[a] + kf[b] for a, b in itertools.combinations(mem, 2))
        gscore.append(Fraction(float(np.float32(float(best)))))
    best_groups, best_val = None, None
    for sub in itertools.combinations(range(G), Gk):  # lexicographic order
        v = sum(gscore[j] for j in sub)
        if best_val is None or v > best_val:
            best_groups, best_val = sub, v
    cand = [e for e in range(E) if e // per in best_groups]
    best_set, best_val = None, None
    for sub in itertools.combinations(cand, k):
        v = sum(kf[e] for e in sub)
        if best_val is None or v > best_val:
            best_set, best_val = sub, v
    order = sorted(best_set, key=lambda e: (-kf[e], e))
    ssum = sum(s[e] for e in order)
    w = [s[e] / ssum * rsf if norm else s[e] * rsf for e in order]
    return order, w


SHAPES = [(16, 4, 2, 2), (16, 4, 2, 3), (16, 4, 4, 5), (32, 8, 3, 4), (12, 3, 1, 2), (8, 8, 3, 2), (6, 2, 2, 6)]


@pytest.mark.parametrize("E,G,Gk,k", SHAPES)
def test_router_selection_brute_force_random(E, G, Gk, k):
    rng = np.random.default_rng(1000 + E * 7 + G * 3 + k)
    cfg = cfg_of(E, G, Gk, k)
    n_subsets = math.comb(Gk * (E // G), k)
    n = 1500 if n_subsets < 1000 else 120
    for _ in range(n):
        logits = rng.normal(0, 1, E)
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
        idx, w, s, dg = O.select(cfg, logits, bias)
        ref_idx, ref_w = brute_force_select(E, G, Gk, k, s, bias)
        assert list(idx) == ref_idx
        np.testing.assert_allclose(w, ref_w, rtol=1e-15)


@pytest.mark.parametrize("E,G,Gk,k", SHAPES)
def test_router_selection_brute_force_ties(E, G, Gk, k):
    """Exact key ties: zero logits (s = 1/2) and biases drawn from a small set."""
    rng = np.random.default_rng(77 + E + k)
    cfg = cfg_of(E, G, Gk, k)
    n_trials = 400 if math.comb(Gk * (E // G), k) < 1000 else 60
    for trial in range(n_trials):
        choices = np.float32([0.0, 0.125, 0.25, -0.125]) if trial % 2 else np.float32([0.0, 0.25])
        bias = rng.choice(choices, E).astype(np.float32)
        logits = np.zeros(E) if trial % 3 else rng.choice([0.0, 1.0], E)
        idx, w, s, dg = O.select(cfg, logits, bias)
        ref_idx, ref_w = brute_force_select(E, G, Gk, k, s, bias)
        assert list(idx) == ref_idx
        np.testing.assert_allclose(w, ref_w, rtol=1e-15)


def test_single_group_is_stable_argsort():
    rng = np.random.default_rng(3)
    E, k = 24, 5
    cfg = cfg_of(E, 1, 1, k)
    for trial in range(500):
        logits = rng.normal(0, 1, E) if trial % 2 else np.zeros(E)
        bias = rng.choice(np.float32([0, 0.25, 0.5]), E).astype(np.float32)
        idx, w, s, _ = O.select(cfg, logits, bias)
        key = (s + bias.astype(np.float64)).astype(np.float32)
        assert list(idx) == list(np.argsort(-key, kind="stable")[:k])


def test_zero_bias_is_topk_of_logits():
    rng = np.random.default_rng(4)
    E, k = 64, 8
    cfg = cfg_of(E, 1, 1, k)
    for _ in range(200):
        logits = rng.normal(0, 3, E)
        idx, _, _, _ = O.select(cfg, logits, np.zeros(E, np.float32))
        assert set(idx) == set(np.argsort(-logits)[:k])


def test_hand_examples_golden():
    d = json.load(open(os.path.join(GOLDEN, "router_hand_example.json")))
    vals = {"ln3": math.log(3), "-ln3": -math.log(3), "0": 0.0, "ln4": math.log(4)}
    cfg = cfg_of(4, 1, 1, 2)
    for case in d["cases"]:
        logits = np.array([vals[v] for v in case["logits"]])
        idx, w, s, _ = O.select(cfg, logits, np.array(case["bias"], np.float32))
        assert list(idx) == case["idx"], case["note"]
        want = [a / b for a, b in case["w_fraction"]]
        np.testing.assert_allclose(w, want, rtol=1e-15)


def test_weights_sum_to_rsf_and_no_norm():
    rng = np.random.default_rng(6)
    cfg = cfg_of(256, 8, 4, 8)
    cfg_nonorm = cfg_of(256, 8, 4, 8, norm=0)
    for _ in range(200):
        logits = rng.normal(0, 1, 256)
        bias = rng.uniform(-0.1, 0.1, 256).astype(np.float32)
        idx, w, s, _ = O.select(cfg, logits, bias)
        assert abs(w.sum() - 2.5) <= 4e-15
        assert len(set(idx)) == 8
        idx2, w2, _, _ = O.select(cfg_nonorm, logits, bias)
        assert list(idx2) == list(idx)
        np.testing.assert_allclose(w2, 2.5 / (1 + np.exp(-logits[idx])), rtol=1e-15)


def test_group_limit_excludes_strong_expert_outside_kept_groups():
    # expert 0 has the single best key but its group's second key is poor;
    # groups 1 and 2 have two strong experts each and win the group stage.
    E, G, Gk, k = 12, 3, 2, 2
    bias = np.zeros(E, np.float32)
    bias[0] = 0.5
    bias[[4, 5, 8, 9]] = 0.3
    idx, _, _, _ = O.select(cfg_of(E, G, Gk, k), np.zeros(E), bias)
    assert 0 not in idx and list(idx) == [4, 5]


def test_rejects_bad_config():
    with pytest.raises(ValueError):
        O.select(cfg_of(16, 5, 2, 2), np.zeros(16), np.zeros(16, np.float32))
    with pytest.raises(ValueError):
        O.select(cfg_of(16, 4, 1, 5), np.zeros(16), np.zeros(16, np.float32))


# --------------------------------------------------------------- router logits

def test_route_logits_match_numpy_fp64():
    w = gen.WORKLOADS["tiny"].with_(tokens=9)
    x = gen.tokens(w)
    W = gen.router_weights(w)
    b = gen.router_bias(w)
    idx, wt, logits, flags, _ = O.route(w.cfg, x, W, b)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(logits, ref, rtol=0, atol=1e-13)
    for t in range(9):
        i2, w2, _, _ = O.select(w.cfg, logits[t], b)
        assert list(i2) == list(idx[t])
    assert not flags.any()


def test_route_bf16_input_decoding():
    w = gen.WORKLOADS["tiny"].with_(tokens=3, x_dtype="bf16")
    xb = gen.tokens(w)
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    W = gen.router_weights(w)
    b = gen.router_bias(w)
    i1, w1, l1, _, _ = O.route(w.cfg, xb, W, b, x_is_bf16=True)
    i2, w2, l2, _, _ = O.route(w.cfg, np.ascontiguousarray(xf), W, b)
    assert np.array_equal(i1, i2) and np.array_equal(l1, l2)


def test_zero_input_router():
    w = gen.WORKLOADS["tiny"].with_(tokens=2)
    c = w.cfg
    x = np.zeros((2, c.hidden), np.float32)
    b = gen.router_bias(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), b)
    assert np.all(wt == c.routed_scaling_factor / c.top_k)  # 1.25, exactly representable
    ref_idx, _ = brute_force_select(c.n_experts, c.n_group, c.topk_group, c.top_k, np.full(c.n_experts, 0.5), b)
    assert list(idx[0]) == ref_idx and list(idx[1]) == ref_idx


# ------------------------------------------------------------------- expert FFN

def numpy_expert(ex, x):
    Wg = numpy_dequant(ex.qg, ex.sg)
    Wu = numpy_dequant(ex.qu, ex.su)
    Wd = numpy_dequant(ex.qd, ex.sd)
    g = Wg @ x
    u = Wu @ x
    h = g / (1.0 + np.exp(-g)) * u
    return Wd @ h, h


def test_expert_ffn_matches_numpy():
    w = gen.WORKLOADS["tiny"]
    c = w.cfg
    ex = gen.expert_weights(w, 0, 3)
    x = gen.tokens(w)[0].astype(np.float64)
    y, h = O.expert_ffn(ex, x, c.hidden, return_h=True)
    ry, rh = numpy_expert(ex, x)
    np.testing.assert_allclose(h, rh, rtol=1e-12, atol=1e-14 * np.abs(rh).max())
    np.testing.assert_allclose(y, ry, rtol=1e-12, atol=1e-13 * np.abs(ry).max())
    assert np.abs(ry).max() > 0.1


def test_layer_composition_matches_numpy():
    w = gen.WORKLOADS["tiny"].with_(tokens=5)
    c = w.cfg
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist()) | {c.n_experts}}
    y = O.moe_ffn(c, x, idx, wt, experts)
    for t in range(5):
        xt = x[t].astype(np.float64)
        ref = sum(wt[t, j] * numpy_expert(experts[idx[t, j]], xt)[0] for j in range(c.top_k))
        ref = ref + numpy_expert(experts[c.n_experts], xt)[0]
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_zero_input_gives_zero_output():
    w = gen.WORKLOADS["tiny"].with_(tokens=2)
    c = w.cfg
    x = np.zeros((2, c.hidden), np.float32)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist()) | {c.n_experts}}
    y = O.moe_ffn(c, x, idx, wt, experts)
    assert np.all(y == 0.0)


def test_single_expert_weight_is_rsf():
    base = gen.WORKLOADS["tiny"]
    c = gen.LayerConfig(**{**base.cfg.__dict__, "top_k": 1})
    w = base.with_(cfg=c, tokens=3)
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    assert np.all(wt == 2.5)
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist()) | {c.n_experts}}
    y = O.moe_ffn(c, x, idx, wt, experts)
    for t in range(3):
        xt = x[t].astype(np.float64)
        ref = 2.5 * numpy_expert(experts[idx[t, 0]], xt)[0] + numpy_expert(experts[c.n_experts], xt)[0]
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_no_shared_expert():
    base = gen.WORKLOADS["tiny"]
    c = gen.LayerConfig(**{**base.cfg.__dict__, "shared_inter": 0})
    w = base.with_(cfg=c, tokens=2)
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist())}
    y = O.moe_ffn(c, x, idx, wt, experts)
    ref = sum(wt[0, j] * numpy_expert(experts[idx[0, j]], x[0].astype(np.float64))[0] for j in range(c.top_k))
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_missing_expert_is_an_error():
    w = gen.WORKLOADS["tiny"]
    c = w.cfg
    x = gen.tokens(w)
    idx = np.array([[0, 1]], np.int32)
    with pytest.raises(ValueError):
        O.moe_ffn(c, x, idx, np.ones((1, 2)), {0: gen.expert_weights(w, 0, 0)})


# ------------------------------------------------------ row-scaled weight formats
# Format 1 is Colibri's production int4 container (one fp32 scale per row,
# "G3 implementation status"), format 2 the MTP layer's signed int8 experts
# ("G4"); "G2 implementation status" states that repeating a row's scale over
# 32-element groups leaves every dequantised value unchanged.

def fmt_cfg(fmt, **kw):
    return gen.LayerConfig(**{**gen.TINY.__dict__, "weight_format": fmt, **kw})


def as_group_scaled(ex):
    """A format-1 expert whose scales are fp16-representable, as format 0 with the
    row scale repeated over every 32-element group."""
    parts = []
    for q, s in ((ex.qg, ex.sg), (ex.qu, ex.su), (ex.qd, ex.sd)):
        h = gen.encode_f16(s.astype(np.float64))
        assert np.array_equal(h.view(np.float16).astype(np.float32), s)  # representable
        parts += [q, np.repeat(h[:, None], q.shape[1] * 2 // 32, axis=1)]
    return gen.ExpertWeights(ex.inter, *parts)


def row_expert_fp16_scales(seed, fmt=1):
    c = fmt_cfg(fmt)
    ex = gen.expert_weights(gen.WORKLOADS["tiny"].with_(cfg=c, seed=seed), 0, 2)
    for s in (ex.sg, ex.su, ex.sd):  # round the scales to fp16 values, kept in fp32
        s[:] = gen.encode_f16(s.astype(np.float64)).view(np.float16).astype(np.float32)
    return c, ex


def test_row_scale_is_repeated_group_scale():
    c, ex = row_expert_fp16_scales(11)
    g = as_group_scaled(ex)
    for (q, s), (q0, s0) in zip(((ex.qg, ex.sg), (ex.qu, ex.su), (ex.qd, ex.sd)),
                                ((g.qg, g.sg), (g.qu, g.su), (g.qd, g.sd))):
        assert np.array_equal(O.dequant_fmt(1, q, s), O.dequant(q0, s0))
    x = gen.tokens(gen.WORKLOADS["tiny"])[0].astype(np.float64)
    y1, h1 = O.expert_ffn(ex, x, c.hidden, return_h=True)
    y0, h0 = O.expert_ffn(g, x, c.hidden, return_h=True)
    assert np.array_equal(h1, h0) and np.array_equal(y1, y0)


def test_row_scale_layer_equals_group_scale_layer():
    w = gen.WORKLOADS["tiny"].with_(tokens=3)
    c1 = fmt_cfg(1)
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c1, x, gen.router_weights(w), gen.router_bias(w))
    ex1, ex0 = {}, {}
    for e in set(idx.ravel().tolist()) | {c1.n_experts}:
        _, ex = row_expert_fp16_scales(100 + e)
        ex1[e], ex0[e] = ex, as_group_scaled(ex)
    assert np.array_equal(O.moe_ffn(c1, x, idx, wt, ex1), O.moe_ffn(w.cfg, x, idx, wt, ex0))


def test_int8_every_byte_and_row_scale():
    q = np.arange(256, dtype=np.uint8).reshape(1, 256).repeat(3, axis=0).view(np.int8)
    s = np.array([1.0, 0.5, 3.0], np.float32)
    got = O.dequant_fmt(2, q, s)
    two = np.array([b if b < 128 else b - 256 for b in range(256)], np.float64)  # two's complement
    assert np.array_equal(got, np.stack([two, two * 0.5, two * 3.0]))


def test_int8_small_values_equal_int4_row_format():
    rng = np.random.default_rng(9)
    v = rng.integers(-8, 8, (6, 64))
    q8 = v.astype(np.int8)
    q4 = ((v[:, 0::2] + 8) | ((v[:, 1::2] + 8) << 4)).astype(np.uint8)  # offset-binary nibbles
    s = np.abs(rng.normal(0, 0.02, 6)).astype(np.float32)
    assert np.array_equal(O.dequant_fmt(2, q8, s), O.dequant_fmt(1, q4, s))


def test_int8_expert_one_hot_closed_form():
    """One nonzero weight per row: every output is a closed form of a few scalars."""
    c = fmt_cfg(2)
    H, I = c.hidden, c.moe_inter
    rng = np.random.default_rng(13)
    ex = gen.empty_expert(c, I)
    for q in (ex.qg, ex.qu, ex.qd):
        q[:] = 0
    cg, cu, cd = rng.integers(0, H, I), rng.integers(0, H, I), rng.integers(0, I, H)
    ag, au, ad = rng.integers(-128, 128, I), rng.integers(-128, 128, I), rng.integers(-128, 128, H)
    ex.qg[np.arange(I), cg] = ag
    ex.qu[np.arange(I), cu] = au
    ex.qd[np.arange(H), cd] = ad
    for s in (ex.sg, ex.su, ex.sd):
        s[:] = np.abs(rng.normal(0, 0.01, s.size)).astype(np.float32)
    x = rng.normal(0, 1, H)
    y, h = O.expert_ffn(ex, x, H, return_h=True)
    for r in range(I):
        g = float(ag[r]) * float(ex.sg[r]) * x[cg[r]]
        u = float(au[r]) * float(ex.su[r]) * x[cu[r]]
        assert h[r] == pytest.approx(g / (1.0 + math.exp(-g)) * u, rel=1e-14, abs=1e-300)
    for j in range(H):
        assert y[j] == pytest.approx(float(ad[j]) * float(ex.sd[j]) * h[cd[j]], rel=1e-14, abs=1e-300)


@pytest.mark.parametrize("fmt", [1, 2])
def test_row_scale_power_of_two_is_exact(fmt):
    """Doubling every down-row scale doubles y exactly; doubling one gate row's
    scale changes only that row's h."""
    c = fmt_cfg(fmt)
    ex = gen.expert_weights(gen.WORKLOADS["tiny"].with_(cfg=c), 0, 4)
    x = gen.tokens(gen.WORKLOADS["tiny"])[0].astype(np.float64)
    y, h = O.expert_ffn(ex, x, c.hidden, return_h=True)
    ex2 = gen.ExpertWeights(ex.inter, ex.qg, ex.sg.copy(), ex.qu, ex.su, ex.qd, ex.sd * 2, fmt)
    ex2.sg[5] *= 2
    y2, h2 = O.expert_ffn(ex2, x, c.hidden, return_h=True)
    changed = np.nonzero(h2 != h)[0]
    assert list(changed) == [5]
    ex3 = gen.ExpertWeights(ex.inter, ex.qg, ex.sg, ex.qu, ex.su, ex.qd, ex.sd * 2, fmt)
    assert np.array_equal(O.expert_ffn(ex3, x, c.hidden), 2 * y)


# ------------------------------------------------------ int8 activations (IDOT)
# [PORT] "G2 implementation status": with Colibri's IDOT=1 setting, every activation
# row becomes int8 ahead of its dot products with the int4 weights, at a cost the
# page puts near 0.3 % RMS per matmul; the oracle's reading: d = amax / 127,
# q = rint(v / d), both in fp32.

def test_quant_row_grid_values_are_exact():
    k = np.arange(-127, 128)
    v = (k * 2.0 ** -3).astype(np.float32)
    q, d, out = O.quant_row(v)
    assert d == np.float32(2.0 ** -3)
    assert np.array_equal(q, k.astype(np.int8)) and np.array_equal(out, v.astype(np.float64))


def test_quant_row_ties_to_even_and_whole_row_scale():
    v = np.array([127.0, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, 0.4, -126.6], np.float32)
    q, d, out = O.quant_row(v)
    assert d == np.float32(1.0)
    assert q.tolist() == [127, 2, 4, -2, 0, 0, 2, 0, -127]
    # the scale is the whole row's: the same small values in a row of small values keep their resolution
    q2, d2, _ = O.quant_row(np.array([2.5, 0.4, -1.27], np.float32))
    assert d2 == np.float32(np.float32(2.5) / np.float32(127)) and q2[0] == 127 and q2[1] != 0


def test_quant_row_zero_row():
    q, d, out = O.quant_row(np.zeros(64, np.float32))
    assert d == 0.0 and not q.any() and not out.any()


def test_int8act_grid_input_gives_the_exact_gate_up():
    """With x on the quantisation grid the gate/up products (h before its own
    quantisation) equal the exact path's bitwise."""
    c = gen.TINY
    ex = gen.expert_weights(gen.WORKLOADS["tiny"], 0, 3)
    rng = np.random.default_rng(4)
    k = rng.integers(-127, 128, c.hidden)
    k[0] = 127
    x = (k * 2.0 ** -5).astype(np.float32)
    _, h_q = O.expert_ffn_int8act(ex, x, c.hidden, return_h=True)
    _, h_e = O.expert_ffn(ex, x.astype(np.float64), c.hidden, return_h=True)
    assert np.array_equal(h_q, h_e)


def test_int8act_down_uses_the_quantised_hidden_row():
    """One-hot int8 weights: y_j = ad_j * sd_j * hhat[cd_j], where hhat is h (closed
    form) rounded to fp32 and quantised with the whole row's scale."""
    c = gen.LayerConfig(**{**gen.TINY.__dict__, "weight_format": 2})
    H, I = c.hidden, c.moe_inter
    rng = np.random.default_rng(17)
    ex = gen.empty_expert(c, I)
    for q in (ex.qg, ex.qu, ex.qd):
        q[:] = 0
    cg, cu, cd = rng.integers(0, H, I), rng.integers(0, H, I), rng.integers(0, I, H)
    ag, au, ad = rng.integers(-128, 128, I), rng.integers(-128, 128, I), rng.integers(-128, 128, H)
    ex.qg[np.arange(I), cg] = ag
    ex.qu[np.arange(I), cu] = au
    ex.qd[np.arange(H), cd] = ad
    for s in (ex.sg, ex.su, ex.sd):
        s[:] = np.abs(rng.normal(0, 0.01, s.size)).astype(np.float32)
    kx = rng.integers(-127, 128, H)
    kx[5] = -127
    x = (kx * 2.0 ** -6).astype(np.float32)  # on the grid: x is its own quantisation
    y, h = O.expert_ffn_int8act(ex, x, H, return_h=True)
    for r in range(I):
        g = float(ag[r]) * float(ex.sg[r]) * float(x[cg[r]])
        u = float(au[r]) * float(ex.su[r]) * float(x[cu[r]])
        assert h[r] == pytest.approx(g / (1.0 + math.exp(-g)) * u, rel=1e-14, abs=1e-300)
    h32 = h.astype(np.float32)
    amax = float(np.abs(h32).max())
    d = float(np.float32(np.float32(amax) / np.float32(127.0)))
    hhat = np.array([float(np.rint(np.float32(v) / np.float32(d))) * d for v in h32])
    for j in range(H):
        assert y[j] == pytest.approx(float(ad[j]) * float(ex.sd[j]) * hhat[cd[j]], rel=1e-14, abs=1e-300)
    assert not np.allclose(hhat, h)  # the quantisation really changes h


def test_int8act_error_is_the_pages_order():
    """Extra RMS error of one expert in int8-activation mode, relative to the exact
    output: the pages quote about 0.3 % per matmul; a per-row int8 grid on Gaussian
    activations gives a few tenths of a percent to about one percent."""
    w = gen.WORKLOADS["tiny"].with_(cfg=gen.LayerConfig(**{**gen.TINY.__dict__, "hidden": 2048, "moe_inter": 512}))
    ex = gen.expert_weights(w, 0, 1)
    errs = []
    for t in range(4):
        x = gen.tokens(w, step=t)[0]
        y_e = O.expert_ffn(ex, x.astype(np.float64), w.cfg.hidden)
        y_q = O.expert_ffn_int8act(ex, x, w.cfg.hidden)
        errs.append(np.sqrt(np.mean((y_q - y_e) ** 2)) / np.sqrt(np.mean(y_e ** 2)))
    assert 1e-3 < np.mean(errs) < 2e-2, errs


def test_int8act_layer_is_the_weighted_sum_of_int8act_experts():
    w = gen.WORKLOADS["tiny"].with_(tokens=3)
    c = w.cfg
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist()) | {c.n_experts}}
    y = O.moe_ffn(c, x, idx, wt, experts, act_int8=True)
    for t in range(3):
        ref = np.zeros(c.hidden)
        for j in range(c.top_k):
            ref += wt[t, j] * O.expert_ffn_int8act(experts[idx[t, j]], x[t], c.hidden)
        ref += O.expert_ffn_int8act(experts[c.n_experts], x[t], c.hidden)
        assert np.array_equal(y[t], ref)
    assert not np.array_equal(y, O.moe_ffn(c, x, idx, wt, experts))


# ------------------------------------------------------------------ bf16 operands (R8)

def test_bf16_round_matches_torch():
    """R8's rounding against torch's float32 -> bfloat16 conversion (round to
    nearest, ties to even) on random values over the whole exponent range and on
    constructed ties (both parities), half-way points just above and below,
    subnormals, the largest finite values and the infinities."""
    import torch
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32)
    ties = np.array([(m << 16) | 0x8000 for m in range(0, 2**16, 97)], np.uint32)
    near = np.concatenate([ties + 1, ties - 1])
    special = np.array([0x00000001, 0x00008000, 0x00018000, 0x007FFFFF, 0x7F7FFFFF, 0x7F7F8000, 0xFF7FFFFF,
                        0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000], np.uint32)
    vals = np.concatenate([bits, ties, near, special]).view(np.float32)
    vals = vals[np.isfinite(vals) | np.isinf(vals)]
    vals = vals[~np.isnan(vals)]
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    mine = np.array([O.bf16_round(float(v)) for v in vals], np.float32)
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))


def one_hot_expert(c, inter, q, s_bits):
    """An expert whose gate, up and down matrices each hold one weight: row 0,
    column 0, value q[part] (int4) with fp16 scale bits s_bits[part]; every other
    weight is 0 (nibble 8) with the same scale."""
    ex = gen.empty_expert(c, inter)
    for j, (qa, sa) in enumerate(((ex.qg, ex.sg), (ex.qu, ex.su), (ex.qd, ex.sd))):
        qa[:] = 0x88
        qa[0, 0] = 0x80 | ((q[j] + 8) & 0xF)
        sa[:] = s_bits[j]
    return ex


def test_bf16_operands_worked_example():
    """Values computed by hand.  x0 = 1 + 2^-10 (bf16: 1); gate and down weights
    1 * (1 + 2^-10) (bf16: 1), up weight 3 * (1 + 2^-10) (bf16: 3).  Exact:
    g = (1 + 2^-10)^2, u = 3 g, y0 = (1 + 2^-10) silu(g) u.  bf16 operands:
    g = 1, u = 3, h = silu(1) * 3 = 2.19317... -> bf16 2.1875 (steps of 2^-6
    between 2 and 4), y0 = 2.1875.  Each rounding changes the result (without the
    input's: g = 1 + 2^-10; without the weights': g = (1 + 2^-10)^2; without h's:
    y0 = 2.19317...), and only marked experts round: routed and shared apart."""
    c = gen.LayerConfig(hidden=32, n_experts=2, n_group=1, topk_group=1, top_k=1, moe_inter=32, shared_inter=32)
    one_p = 0x3C01  # fp16 1 + 2^-10
    ex = one_hot_expert(c, 32, (1, 3, 1), (one_p, one_p, one_p))
    experts = {0: ex, 1: ex, 2: ex}  # routed 0 and 1, shared (id 2) the same weights
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1 + 2.0**-10
    idx = np.array([[0]], np.int32)
    w = np.array([[1.0]])
    a = 1 + 2.0**-10
    g = a * a
    exact0 = a * (g / (1 + math.exp(-g))) * (3 * g)
    bf0 = 2.1875
    assert O.bf16_round(3 / (1 + math.exp(-1.0))) == bf0
    for mark, want in (((), 2 * exact0), ((0,), bf0 + exact0), ((2,), exact0 + bf0), ((0, 2), 2 * bf0),
                       ((1,), 2 * exact0)):
        y = O.moe_ffn(c, x, idx, w, experts, bf16_experts=mark)
        assert y[0, 0] == pytest.approx(want, rel=1e-15), mark
        assert np.all(y[0, 1:] == 0.0)
    assert O.moe_ffn(c, x, idx, w, experts, bf16_experts=(0, 2))[0, 0] == 2 * bf0


def test_bf16_operands_unmarked_is_exact_and_int8_is_refused():
    w = gen.WORKLOADS["tiny"].with_(tokens=3)
    c = w.cfg
    x = gen.tokens(w)
    idx, wt, _, _, _ = O.route(c, x, gen.router_weights(w), gen.router_bias(w))
    experts = {e: gen.expert_weights(w, 0, e) for e in set(idx.ravel().tolist()) | {c.n_experts}}
    exact = O.moe_ffn(c, x, idx, wt, experts)
    assert np.array_equal(O.moe_ffn(c, x, idx, wt, experts, bf16_experts=()), exact)
    unused = sorted(set(range(c.n_experts)) - set(idx.ravel().tolist()))
    if unused:
        assert np.array_equal(O.moe_ffn(c, x, idx, wt, experts, bf16_experts=unused[:1]), exact)
    marked = O.moe_ffn(c, x, idx, wt, experts, bf16_experts=range(c.n_experts + 1))
    rel = np.abs(marked - exact).max() / np.abs(exact).max()
    assert 1e-5 < rel < 5e-2
    with pytest.raises(ValueError):
        O.moe_ffn(c, x, idx, wt, experts, act_int8=True, bf16_experts=(c.n_experts,))

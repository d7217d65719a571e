"""Pins of the oracle's decision diagnostics (the per-token margins and the
near-midpoint flag) against hand-built cases.

The selection key of expert e is fp32(sigmoid(l_e) + bias_e) with the sigmoid
and the sum in fp64.  A GPU that accumulates the logit in a different order
reaches the same fp64 value only up to ~2^-46 relative, so its fp32 key can
differ from the oracle's only when the fp64 value sits within about that
distance of an fp32 rounding midpoint.  The oracle therefore flags a token
(flags = 1) when a decision whose outcome depends on the order of two keys (two
adjacent ranks, the cut-off between the k-th pick and the best excluded
candidate, or the last kept group against a dropped one) compares values at
most one fp32 ulp apart (two for group scores) and one of the fp64 values
behind them is within 2^-40 relative of an fp32 midpoint.  The cases here put
such values in place on purpose: with bias 0 the key is sigmoid(l), so a logit
l = ln(s / (1 - s)) places the fp64 key at s to within a few fp64 ulps.

The margins (fp32 keys and group scores, differences taken in fp64) are
checked against values worked out by hand with dyadic keys (exact in fp32).
"""
import math

import numpy as np

from gen import inputs as gen
from oracle import oracle as O


def cfg_of(E, G, Gk, k):
    return gen.LayerConfig(hidden=8, n_experts=E, n_group=G, topk_group=Gk, top_k=k, moe_inter=32, shared_inter=32)


def logit(s: float) -> float:
    return math.log(s) - math.log1p(-s)


F = np.float32(0.6)                    # an fp32 value in [0.5, 1): ulp 2^-24
G_UP = np.nextafter(F, np.float32(1))  # the next fp32 value
MID = (float(F) + float(G_UP)) / 2     # the rounding midpoint between them


def select(E, G, Gk, k, s, bias=None):
    """The oracle's selection for sigmoid scores s (bias 0 unless given)."""
    l = np.array([logit(v) for v in s])
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    return O.select(cfg_of(E, G, Gk, k), l, b)


def test_placed_key_sits_on_the_midpoint():
    """The construction itself: sigmoid(logit(MID)) is within 2^-50 of MID."""
    l = logit(MID)
    s = 1.0 / (1.0 + math.exp(-l))
    assert abs(s - MID) <= MID * 2.0 ** -50
    assert float(F) < MID < float(G_UP)


def test_flag_adjacent_ranks_near_midpoint():
    # experts 0 and 1 are the two picks, one fp32 ulp apart at most; expert 0's
    # fp64 key is on the midpoint, so their order hinges on its rounding
    idx, _, _, dg = select(4, 1, 1, 2, [MID, float(F), 0.3, 0.2])
    assert sorted(idx) == [0, 1]
    assert dg.flags == 1


def test_flag_cut_off_near_midpoint():
    # one pick: expert 0 (key exactly G_UP) against expert 1, whose fp64 key is the midpoint
    idx, _, _, dg = select(4, 1, 1, 1, [float(G_UP), MID, 0.3, 0.2])
    assert list(idx) == [0]
    assert dg.flags == 1
    # the excluded candidate on the midpoint below the pick: same decision, same flag
    idx, _, _, dg = select(4, 1, 1, 1, [0.2, MID, float(F), 0.3])
    assert dg.flags == 1


def test_flag_group_scores_near_midpoint():
    # two groups of two; group 0 = {MID, 0.25}, group 1 = {F, 0.25}: scores
    # fp32(key + 0.25) are at most one ulp apart and group 0's top key is on the
    # midpoint, so which group is kept hinges on it.  Inside the kept group the
    # pick (0.6 vs 0.25) is clear, so only the group decision can raise the flag.
    idx, _, _, dg = select(4, 2, 1, 1, [MID, 0.25, float(F), 0.25])
    assert dg.group_margin <= 2 * 2.0 ** -24
    assert dg.flags == 1


def test_no_flag_when_midpoint_key_has_no_close_competitor():
    idx, _, _, dg = select(4, 1, 1, 1, [MID, 0.3, 0.2, 0.1])
    assert list(idx) == [0]
    assert dg.flags == 0
    idx, _, _, dg = select(4, 1, 1, 2, [MID, 0.3, 0.2, 0.1])
    assert dg.flags == 0


def test_no_flag_for_exact_ties_off_the_midpoint():
    # equal keys (both exactly F): the tie rule decides, no rounding is involved
    idx, _, _, dg = select(4, 1, 1, 1, [float(F), float(F), 0.2, 0.1])
    assert list(idx) == [0]
    assert dg.flags == 0
    assert dg.expert_margin == 0.0
    # equal group scores off the midpoint
    idx, _, _, dg = select(4, 2, 1, 1, [float(F), 0.25, float(F), 0.25])
    assert list(idx) == [0]
    assert dg.flags == 0
    assert dg.group_margin == 0.0


def test_flag_threshold_is_two_to_the_minus_40():
    # a key 2^-36 (relative) above the midpoint rounds up for sure: no flag;
    # 2^-44 above it is within the oracle's 2^-40 window: flagged
    far = MID * (1.0 + 2.0 ** -36)
    near = MID * (1.0 + 2.0 ** -44)
    _, _, _, dg = select(4, 1, 1, 1, [float(F), far, 0.2, 0.1])
    assert dg.flags == 0
    _, _, _, dg = select(4, 1, 1, 1, [float(F), near, 0.2, 0.1])
    assert dg.flags == 1


def test_margins_hand_values():
    # groups of four, keep one, pick two; dyadic keys are exact in fp32
    s = [0.75, 0.5, 0.3125, 0.125, 0.625, 0.5625, 0.0625, 0.03125]
    idx, _, _, dg = select(8, 2, 1, 2, s)
    # group scores 0.75 + 0.5 = 1.25 and 0.625 + 0.5625 = 1.1875: group 0 kept
    assert list(idx) == [0, 1]
    assert dg.group_margin == 1.25 - 1.1875
    # second pick 0.5 against the best excluded candidate 0.3125
    assert dg.expert_margin == 0.5 - 0.3125
    assert dg.n_candidates == 4
    assert dg.flags == 0
    # a bias of +0.25 on expert 2 (key 0.5625) changes the second pick and the group score
    bias = np.zeros(8, np.float32)
    bias[2] = 0.25
    idx, _, _, dg = select(8, 2, 1, 2, s, bias)
    assert list(idx) == [0, 2]
    assert dg.expert_margin == 0.5625 - 0.5
    assert dg.group_margin == (0.75 + 0.5625) - 1.1875
    # keep both groups: no group is dropped, the group margin is infinite
    idx, _, _, dg = select(8, 2, 2, 2, s)
    assert list(idx) == [0, 4]
    assert math.isinf(dg.group_margin)
    assert dg.expert_margin == 0.625 - 0.5625
    # every candidate picked: no excluded candidate, the expert margin is infinite
    idx, _, _, dg = select(4, 2, 1, 2, [0.75, 0.5, 0.25, 0.125])
    assert list(idx) == [0, 1]
    assert math.isinf(dg.expert_margin)
    assert dg.group_margin == 1.25 - 0.375


def split_f32(v: float):
    """v as hi + lo with hi, lo fp32 (exact to about 2^-48 relative)."""
    hi = np.float32(v)
    lo = np.float32(v - float(hi))
    return hi, lo


def test_route_reports_flags_per_token():
    """oracle_route hands each token's diagnostics back.  Expert e's logit is
    x[2e] + x[2e+1] (router row e has ones there), so a token can place an fp64
    logit to about 2^-48: token 1 puts expert 0 exactly on G_UP and expert 1 on
    the midpoint below it (flagged); tokens 0 and 2 are clear."""
    c = gen.LayerConfig(hidden=8, n_experts=4, n_group=1, topk_group=1, top_k=1, moe_inter=32, shared_inter=32)
    W = np.zeros((4, 8), np.float32)
    for e in range(4):
        W[e, 2 * e] = W[e, 2 * e + 1] = 1.0
    x = np.zeros((3, 8), np.float32)
    x[0, 0::2] = [0.5, 0.1, -0.2, -0.3]
    x[1, 0:2] = split_f32(logit(float(G_UP)))
    x[1, 2:4] = split_f32(logit(MID))
    x[1, 4::2] = [-1.0, -1.0]
    x[2, 0::2] = [1.0, -1.0, -1.0, 2.0]
    idx, _, logits, flags, margins = O.route(c, x, W, np.zeros(4, np.float32))
    assert list(idx[:, 0]) == [0, 0, 3]
    assert list(flags) == [0, 1, 0]
    assert margins[1, 0] <= 2.0 ** -24

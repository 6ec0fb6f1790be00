"""Pins of the CPU oracle against things other than itself: published numbers,
closed forms, brute force, invariants and special cases that reduce to library
routines (numpy / torch float64). Each test names what a plausible mistake in
the oracle would break."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests import _ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_inputs(w, seed_shift=0):
    ws = recipes.Workload(**{**w.__dict__, "seed_base": w.seed_base + seed_shift})
    x = synth.hidden(ws)
    Wr = synth.router_weight(ws)
    b = synth.bias(ws)
    return ws, x, Wr, b


# --- published numbers -------------------------------------------------------------------

def test_golden_shape_facts():
    """Constants of the workloads against the numbers printed on the pages."""
    g = json.load(open(os.path.join(GOLDEN, "beam_shape_facts.json")))
    w = recipes.WORKLOADS[2]
    assert w.d == g["hidden_size"]["value"]
    assert w.I == g["moe_intermediate_size"]["value"]
    assert w.E == g["num_experts"]["value"]
    assert w.top_k == g["num_experts_per_tok"]["value"]
    assert w.n_group == g["n_group"]["value"]
    assert w.topk_group == g["topk_group"]["value"]
    assert w.E // w.n_group == g["experts_per_group"]["value"]
    assert w.scale == g["routed_scaling_factor"]["value"]
    assert w.eps == g["rms_norm_eps"]["value"]
    per_expert = 3 * w.d * w.I                        # gate, up, down; no biases
    assert per_expert == 39_321_600
    assert round(per_expert / 1e6) == g["params_per_expert_approx_millions"]["value"]
    share = g["moe_layers"]["value"] * w.E * per_expert / (g["total_params_billions"]["value"] * 1e9)
    assert round(100 * share, 1) == g["expert_weight_share_percent"]["value"]
    emb = 2 * g["vocab_size"]["value"] * w.d          # untied embedding + head
    assert round(emb / 1e9, 3) == g["embedding_plus_head_billions"]["value"]
    assert w.E // w.top_k == g["experts_over_top_k"]["value"]
    assert w.I / w.d == g["expert_dim_over_d_model"]["value"]
    ratio = g["active_params_billions"]["value"] / g["total_params_billions"]["value"]
    assert round(ratio, 7) == g["active_over_total"]["value"]


# --- bf16 rounding -------------------------------------------------------------------------

def test_bf16_round_cases_and_random():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2 ** -8: 0x3F80,             # halfway, ties to even (down)
        one + 3 * 2 ** -8: 0x3F82,         # halfway, ties to even (up)
        one + 2 ** -8 + 2 ** -30: 0x3F81,  # just above halfway
        -2.0: 0xC000,
        0.0: 0x0000,
        2.0 ** -133: 0x0001,               # smallest subnormal
        3.0e38: 0x7F62,
    }
    got = oracle.bf16_round(np.array(list(cases.keys())))
    assert [int(v) for v in got] == list(cases.values())
    rng = np.random.default_rng(0)
    v = rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))
    assert np.array_equal(oracle.bf16_round(v), _ref.f64_to_bf16_bits_rne(v))


# --- router -------------------------------------------------------------------------------

def test_logits_onehot_and_matmul():
    w = recipes.WORKLOADS[0]
    _, x, Wr, _ = _tiny_inputs(w)
    onehot = np.zeros((w.d, w.d), dtype=np.uint16)
    onehot[np.arange(w.d), np.arange(w.d)] = 0x3F80   # bf16 1.0
    z = oracle.logits(onehot, Wr)
    assert np.array_equal(z, Wr.astype(np.float64))  # one-hot x picks a row of Wr exactly
    z = oracle.logits(x, Wr)
    ref = _ref.bf16_bits_to_f64(x) @ Wr.astype(np.float64)
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed_shift", [0, 1, 2])
def test_route_matches_brute_force_tiny(seed_shift):
    """Exhaustive enumeration of group pairs, group subsets and expert subsets."""
    w = recipes.WORKLOADS[0]
    ws, x, Wr, b = _tiny_inputs(w, seed_shift)
    idx, wt, gap, z = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale, want_logits=True)
    zr = _ref.bf16_bits_to_f64(x) @ Wr.astype(np.float64)
    checked = 0
    for t in range(w.T):
        if gap[t] < 1e-9:
            continue
        sel, wref = _ref.brute_route_token(zr[t], b, w.n_group, w.topk_group, w.top_k, w.scale)
        assert sorted(idx[t].tolist()) == sel, t
        for j in range(w.top_k):
            assert abs(wt[t, j] - wref[int(idx[t, j])]) < 1e-12
        checked += 1
    assert checked >= w.T - 2


def test_route_random_small_shapes_brute_force():
    rng = np.random.default_rng(1)
    for (E, G, KG, K) in [(8, 2, 1, 2), (12, 3, 2, 3), (16, 4, 3, 5), (16, 8, 3, 4), (20, 5, 5, 6)]:
        d = 64
        x = _ref.f64_to_bf16_bits_rne(rng.standard_normal((40, d)))
        Wr = (rng.standard_normal((d, E)) / 8).astype(np.float32)
        bias = rng.uniform(-0.3, 0.3, E).astype(np.float32)
        idx, wt, gap = oracle.route(x, Wr, bias, G, KG, K, 2.5)
        zr = _ref.bf16_bits_to_f64(x) @ Wr.astype(np.float64)
        for t in range(40):
            if gap[t] < 1e-9:
                continue
            sel, _ = _ref.brute_route_token(zr[t], bias, G, KG, K, 2.5)
            assert sorted(idx[t].tolist()) == sel


def test_route_full_shape_group_stage_and_certificate():
    """Beam shape: group scores by all 496 pairs per group, kept groups by all 70
    subsets, chosen experts certified by min(chosen b) > max(other candidate b)."""
    w = recipes.WORKLOADS[2].with_T(48)
    x = synth.hidden(w)
    Wr = synth.router_weight(w)
    b = synth.bias(w)
    idx, wt, gap, z = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale, want_logits=True)
    s = _ref.sigmoid(z)
    bb = s + b.astype(np.float64)
    gsz = w.E // w.n_group
    for t in range(w.T):
        gs = [max(bb[t, i] + bb[t, j] for i, j in itertools.combinations(range(g * gsz, (g + 1) * gsz), 2))
              for g in range(w.n_group)]
        kept = max(itertools.combinations(range(w.n_group), w.topk_group), key=lambda c: sum(gs[g] for g in c))
        groups = {int(e) // gsz for e in idx[t]}
        assert groups <= set(kept)
        cand = [e for g in kept for e in range(g * gsz, (g + 1) * gsz)]
        others = [e for e in cand if e not in set(idx[t].tolist())]
        assert bb[t, idx[t]].min() > bb[t, others].max()
        assert np.all(np.diff(bb[t, idx[t]]) < 0)          # descending biased score
        assert abs(wt[t].sum() - w.scale) < 1e-12
        np.testing.assert_allclose(wt[t] / wt[t].sum(), s[t, idx[t]] / s[t, idx[t]].sum(), rtol=1e-13)


def test_route_invariants():
    w = recipes.WORKLOADS[0]
    _, x, Wr, b = _tiny_inputs(w)
    G, KG, K, S = w.n_group, w.topk_group, w.top_k, w.scale
    idx, wt, gap, z = oracle.route(x, Wr, b, G, KG, K, S, want_logits=True)
    ok = gap > 1e-9
    # weights sum to the routed scaling factor; at most KG groups per token
    np.testing.assert_allclose(wt.sum(1), S, rtol=0, atol=1e-12)
    assert max(len({e // (w.E // G) for e in row}) for row in idx) <= KG
    # a constant bias shift selects the same experts with the same weights (bias only selects)
    idx2, wt2, _ = oracle.route(x, Wr, b + np.float32(0.25), G, KG, K, S)
    assert np.array_equal(idx[ok], idx2[ok])
    assert np.array_equal(wt[ok], wt2[ok])
    # weights are proportional to the unbiased sigmoid scores of the chosen experts
    s = _ref.sigmoid(z)
    for t in np.nonzero(ok)[0]:
        np.testing.assert_allclose(wt[t], S * s[t, idx[t]] / s[t, idx[t]].sum(), rtol=1e-13)
    # norm_topk_prob off: w = S * s
    idx3, wt3, _ = oracle.route(x, Wr, b, G, KG, K, S, norm_topk_prob=False)
    assert np.array_equal(idx3, idx)
    np.testing.assert_allclose(wt3, S * np.take_along_axis(s, idx, 1), rtol=1e-14)
    # keeping every group reduces to a plain top-K of the biased scores
    idx4, _, gap4 = oracle.route(x, Wr, b, G, G, K, S)
    bb = s + b.astype(np.float64)
    order = np.argsort(-bb, axis=1, kind="stable")[:, :K]
    m = gap4 > 1e-9
    assert np.array_equal(idx4[m], order[m])
    # with no bias and every group kept, the top-K of b is the top-K of the logits (sigmoid is monotone)
    idx5, _, gap5 = oracle.route(x, Wr, np.zeros_like(b), G, G, K, S)
    order = np.argsort(-z, axis=1, kind="stable")[:, :K]
    m = gap5 > 1e-9
    assert np.array_equal(idx5[m], order[m])
    # weights_for on the oracle's own selection reproduces its weights
    np.testing.assert_allclose(oracle.weights_for(z, idx, S), wt, rtol=1e-15)


def _brute_margins(z_row, bias, G, KG, K):
    """Both selection margins by exhaustive enumeration, written from their meaning: how much
    the best admissible choice beats the runner-up. Group stage: every pair of a group gives
    the group score; the best KG-subset of groups by total score minus the best other
    KG-subset. Expert stage (inside the best groups): the best K-subset of candidates by
    total biased score minus the best other K-subset. inf where there is no runner-up."""
    E = len(z_row)
    gsz = E // G
    b = _ref.sigmoid(np.asarray(z_row, np.float64)) + np.asarray(bias, np.float64)
    gs = [max(b[i] + b[j] for i, j in itertools.combinations(range(g * gsz, (g + 1) * gsz), 2)) for g in range(G)]
    subsets = sorted((sum(gs[g] for g in c), c) for c in itertools.combinations(range(G), KG))
    m_group = subsets[-1][0] - subsets[-2][0] if len(subsets) > 1 else math.inf
    kept = subsets[-1][1]
    cand = [e for g in kept for e in range(g * gsz, (g + 1) * gsz)]
    sums = sorted(sum(b[e] for e in c) for c in itertools.combinations(cand, K))
    m_expert = sums[-1] - sums[-2] if len(sums) > 1 else math.inf
    return m_group, m_expert


def test_route_gap_equals_brute_force_margins():
    """The oracle's gap (the smaller of the two selection margins, which decides which tokens
    the GPU parity rule may excuse) against both margins found by enumerating every group
    subset and every expert subset, on the tiny shape and on random small shapes. A slip in
    which ranked score the gap subtracts (KG-2 for KG-1, K for K-1, the candidate list before
    or after the kept-group filter) changes it on most tokens."""
    cases = []
    w = recipes.WORKLOADS[0]
    for shift in (0, 1):
        _, x, Wr, b = _tiny_inputs(w, shift)
        cases.append((x, Wr, b, w.n_group, w.topk_group, w.top_k))
    rng = np.random.default_rng(7)
    for (E, G, KG, K) in [(8, 2, 1, 2), (12, 3, 2, 3), (16, 4, 3, 5), (16, 8, 3, 4), (20, 5, 4, 6), (16, 4, 4, 3),
                          (12, 4, 2, 6)]:
        x = _ref.f64_to_bf16_bits_rne(rng.standard_normal((30, 64)))
        Wr = (rng.standard_normal((64, E)) / 8).astype(np.float32)
        bias = rng.uniform(-0.3, 0.3, E).astype(np.float32)
        cases.append((x, Wr, bias, G, KG, K))
    n = 0
    for x, Wr, bias, G, KG, K in cases:
        _, _, gap = oracle.route(x, Wr, bias, G, KG, K, 2.5)
        zr = _ref.bf16_bits_to_f64(x) @ Wr.astype(np.float64)
        for t in range(x.shape[0]):
            mg, me = _brute_margins(zr[t], bias, G, KG, K)
            want = min(mg, me)
            if math.isinf(want):
                assert math.isinf(gap[t]), (G, KG, K, t)
            else:
                assert abs(gap[t] - want) <= 1e-12, (G, KG, K, t, gap[t], mg, me)
            n += 1
    assert n == 2 * 128 + 7 * 30


def test_route_ties_go_to_lower_index():
    E, G, KG, K, d = 16, 4, 2, 4, 64
    x = np.zeros((1, d), dtype=np.uint16)          # all logits 0, all scores 0.5
    Wr = np.zeros((d, E), dtype=np.float32)
    bias = np.zeros(E, dtype=np.float32)
    idx, wt, gap = oracle.route(x, Wr, bias, G, KG, K, 2.5)
    assert idx[0].tolist() == [0, 1, 2, 3]           # groups 0,1 kept; lowest ids first
    np.testing.assert_allclose(wt[0], 2.5 / 4)
    assert gap[0] == 0.0


# --- dispatch -----------------------------------------------------------------------------

def test_dispatch_matches_stable_argsort():
    rng = np.random.default_rng(3)
    for T, K, E in [(1, 1, 4), (7, 3, 16), (300, 8, 256), (1000, 4, 16)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        off, sp, pr = oracle.dispatch(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(sp, np.argsort(flat, kind="stable"))
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(pr[sp], np.arange(T * K))
        for e in range(E):
            seg = sp[off[e]:off[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# --- experts ------------------------------------------------------------------------------

def _expert_torch(x_bits, wg, wu, wd):
    """SwiGLU expert from torch float64 library ops, h rounded to bf16 by the test's own RNE."""
    x = torch.from_numpy(_ref.bf16_bits_to_f64(x_bits))
    g = torch.nn.functional.linear(x, torch.from_numpy(_ref.bf16_bits_to_f64(wg)))
    u = torch.nn.functional.linear(x, torch.from_numpy(_ref.bf16_bits_to_f64(wu)))
    a = (torch.nn.functional.silu(g) * u).numpy()
    h = _ref.bf16_bits_to_f64(_ref.f64_to_bf16_bits_rne(a))
    return torch.nn.functional.linear(torch.from_numpy(h), torch.from_numpy(_ref.bf16_bits_to_f64(wd))).numpy(), a


def test_expert_matches_torch_float64():
    w = recipes.WORKLOADS[0]
    x = synth.hidden(w)[:24]
    wg, wu, wd = synth.expert_weights(w, 5)
    o = oracle.expert(x, wg, wu, wd)
    ref, a = _expert_torch(x, wg, wu, wd)
    # identical up to summation order, unless a lies within rounding noise of a bf16 midpoint
    rel = np.abs(o - ref).max() / np.sqrt((ref ** 2).mean())
    assert rel < 1e-12


def test_expert_full_shape_one_token():
    w = recipes.WORKLOADS[2]
    x = synth.hidden(w, rows=[17])
    wg, wu, wd = synth.expert_weights(w, 200)
    o = oracle.expert(x, wg, wu, wd)
    ref, _ = _expert_torch(x, wg, wu, wd)
    assert np.abs(o - ref).max() / np.sqrt((ref ** 2).mean()) < 1e-9


def test_expert_exact_small_integers():
    """Inputs that are small integers times powers of two: every sum is exact, so the
    oracle must match a hand-derivable result bit for bit."""
    d, I = 8, 4
    x = _ref.f64_to_bf16_bits_rne(np.array([[1, 2, 0, -1, 0, 0, 3, 0]], dtype=np.float64))
    wg = np.zeros((I, d)); wu = np.zeros((I, d)); wd = np.zeros((d, I))
    wg[0, 0] = 1.0; wu[0, 1] = 0.5        # g0 = 1, u0 = 1
    wg[1, 3] = 2.0; wu[1, 6] = 1.0        # g1 = -2, u1 = 3
    wg[2, 6] = 0.0; wu[2, 0] = 4.0        # g2 = 0 -> silu 0
    wg[3, 1] = 0.25; wu[3, 3] = -1.0      # g3 = 0.5, u3 = (-1)(-1) = 1
    wd[0, 0] = 1.0; wd[1, 1] = 1.0; wd[2, 2] = 1.0; wd[3, 3] = 1.0; wd[4, :] = 1.0
    to = _ref.f64_to_bf16_bits_rne
    o = oracle.expert(x, to(wg), to(wu), to(wd))[0]
    silu = lambda v: v / (1.0 + math.exp(-v))
    h = [silu(1.0) * 1.0, silu(-2.0) * 3.0, 0.0, silu(0.5) * 1.0]
    hb = _ref.bf16_bits_to_f64(to(np.array(h)))
    exp = np.zeros(d)
    exp[0:4] = hb
    exp[4] = hb.sum()
    assert np.array_equal(o, exp)


def test_layer_invariants_tiny():
    w = recipes.WORKLOADS[0]
    x = synth.hidden(w)
    Wr = synth.router_weight(w)
    b = synth.bias(w)
    wg0, wu0, wd0 = synth.expert_weights(w, 0)
    E = w.E
    # identical experts: y = S * expert(x) whatever the routing (weights sum to S)
    Wg = np.stack([wg0] * E); Wu = np.stack([wu0] * E); Wd = np.stack([wd0] * E)
    y, idx, wt, gap = oracle.forward(x, Wr, b, Wg, Wu, Wd, w.n_group, w.topk_group, w.top_k, w.scale)
    one = oracle.expert(x, wg0, wu0, wd0)
    np.testing.assert_allclose(y, w.scale * one, rtol=0, atol=1e-12 * np.abs(one).max())
    # gate weights zero: silu(0) = 0, so y = 0 exactly
    y0, *_ = oracle.forward(x, Wr, b, np.zeros_like(Wg), Wu, Wd, w.n_group, w.topk_group, w.top_k, w.scale)
    assert np.all(y0 == 0.0)
    # different experts: doubling every down projection doubles y exactly
    mats = [synth.expert_weights(w, e) for e in range(E)]
    Wg = np.stack([m[0] for m in mats]); Wu = np.stack([m[1] for m in mats]); Wd = np.stack([m[2] for m in mats])
    y1, *_ = oracle.forward(x, Wr, b, Wg, Wu, Wd, w.n_group, w.topk_group, w.top_k, w.scale)
    Wd2 = _ref.f64_to_bf16_bits_rne(2.0 * _ref.bf16_bits_to_f64(Wd))
    y2, *_ = oracle.forward(x, Wr, b, Wg, Wu, Wd2, w.n_group, w.topk_group, w.top_k, w.scale)
    assert np.array_equal(y2, 2.0 * y1)
    # the layer is the routed sum of single experts (checked per token against the expert routine)
    for t in (0, 77):
        acc = np.zeros(w.d)
        for j in range(w.top_k):
            e = idx[t, j]
            acc += wt[t, j] * oracle.expert(x[t:t + 1], Wg[e], Wu[e], Wd[e])[0]
        np.testing.assert_allclose(y1[t], acc, rtol=0, atol=1e-13 * np.abs(acc).max())



def test_expert_share_partitions_the_layer():
    """Expert-parallel shares ("Use HF Transformers" cookbook, Parallelism): over any partition
    of the experts into contiguous blocks the shares add up to the layer; the whole range is the
    layer itself; a one-expert share is that expert's weighted output on the rows that chose it
    and exactly 0 elsewhere; checked per token against torch float64 experts."""
    w = recipes.WORKLOADS[0]
    x = synth.hidden(w)
    Wr = synth.router_weight(w)
    b = synth.bias(w)
    idx, wt, _ = oracle.route(x, Wr, b, w.n_group, w.topk_group, w.top_k, w.scale)
    experts = {e: synth.expert_weights(w, e) for e in range(w.E)}
    y = oracle.moe_rows(x, idx, wt, experts, w.E)
    assert np.array_equal(oracle.moe_share_rows(x, idx, wt, experts, 0, w.E), y)
    gs = w.E // w.n_group
    for blocks in ([(g * gs, gs) for g in range(w.n_group)], [(0, 5), (5, 1), (6, w.E - 6)]):
        tot = sum(oracle.moe_share_rows(x, idx, wt, experts, e0, n) for e0, n in blocks)
        np.testing.assert_allclose(tot, y, rtol=0, atol=1e-13 * np.abs(y).max())
    e1 = int(idx[3, 2])
    one = oracle.moe_share_rows(x, idx, wt, experts, e1, 1)
    for t in range(w.T):
        hit = np.nonzero(idx[t] == e1)[0]
        if len(hit) == 0:
            assert np.all(one[t] == 0.0)
        else:
            exp = wt[t, hit[0]] * oracle.expert(x[t:t + 1], *experts[e1])[0]
            assert np.array_equal(one[t], exp)
    g0 = oracle.moe_share_rows(x, idx, wt, experts, 0, gs)
    for t in (0, 3, 77):
        ref = np.zeros(w.d)
        for j in range(w.top_k):
            if idx[t, j] < gs:
                ref += wt[t, j] * _expert_torch(x[t:t + 1], *experts[int(idx[t, j])])[0][0]
        np.testing.assert_allclose(g0[t], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))

# --- RMSNorm ------------------------------------------------------------------------------

def test_rmsnorm_matches_torch_float64():
    w = recipes.WORKLOADS[4].with_T(16)
    h = synth.hidden(w)
    nw = synth.norm_weight(w)
    x = oracle.rmsnorm(h, nw, w.eps)
    ht = torch.from_numpy(_ref.bf16_bits_to_f64(h))
    r = torch.rsqrt(ht.pow(2).mean(-1, keepdim=True) + w.eps)
    ref = _ref.f64_to_bf16_bits_rne(((ht * r) * torch.from_numpy(_ref.bf16_bits_to_f64(nw))).numpy())
    diff = np.count_nonzero(x != ref)
    assert diff <= 2   # rsqrt vs 1/sqrt may differ in the last double bit; a flip needs a midpoint
    # a constant row normalises to (1/sqrt(1+eps)) * w
    c = np.full((1, w.d), 0x3F80, dtype=np.uint16)
    xc = _ref.bf16_bits_to_f64(oracle.rmsnorm(c, nw, w.eps))[0]
    exp = _ref.bf16_bits_to_f64(_ref.f64_to_bf16_bits_rne(_ref.bf16_bits_to_f64(nw) / math.sqrt(1 + w.eps)))
    assert np.array_equal(xc, exp)


# --- post-MLP norm and depth-scaled residual ------------------------------------------------

def test_dense_layer_shape_facts():
    """The dense MLP workloads use the pages' intermediate size, and the dense + MoE layer
    counts add up to the model's depth."""
    g = json.load(open(os.path.join(GOLDEN, "beam_shape_facts.json")))
    for w in recipes.DENSE_WORKLOADS.values():
        if w.d == 5120:
            assert w.I == g["intermediate_size"]["value"]
    assert g["dense_layers"]["value"] + g["moe_layers"]["value"] == g["num_hidden_layers"]["value"]
    # a dense MLP holds 3*d*I parameters: 8x the intermediate width of one routed expert
    assert g["intermediate_size"]["value"] == 8 * g["moe_intermediate_size"]["value"]


def test_dense_mlp_is_the_single_expert_case():
    """The dense MLP is the layer's expert arithmetic with one expert and weight 1: moe_rows
    with K = 1, w = 1 equals expert() on the same rows, bit for bit."""
    w = recipes.DENSE_WORKLOADS[12].with_T(5)
    x = synth.dense_hidden(w)
    wg, wu, wd = synth.dense_weights(w)
    o = oracle.expert(x, wg, wu, wd)
    y = oracle.moe_rows(x, np.zeros((w.T, 1), np.int32), np.ones((w.T, 1)), {0: (wg, wu, wd)}, 1)
    assert np.array_equal(o, y)


def test_residual_step_telescopes_to_sum_over_sqrt_k():
    """After contributions c_1..c_m the stream is their sum over sqrt(m), the property the
    Beam page states for the depth-scaled residual. A wrong k offset, a swapped keep/add
    factor or a missing square root breaks it."""
    rng = np.random.default_rng(7)
    m, n = 12, 257
    cs = rng.standard_normal((m, n))
    r = rng.standard_normal(n) * 1e3            # k = 1 keeps nothing of what came before
    for k in range(1, m + 1):
        r = oracle.residual_step(r, cs[k - 1], k)
        np.testing.assert_allclose(r, cs[:k].sum(0) / math.sqrt(k), rtol=1e-13, atol=1e-13)


def test_residual_schedule_over_the_whole_model():
    """Embedding first, then attention and MLP of each layer: the contribution indices run
    2, 3, ..., 105 without a gap, there are as many additions as the pages print, and at the
    end every contribution weighs the same (sum of squared weights 1)."""
    g = json.load(open(os.path.join(GOLDEN, "beam_shape_facts.json")))
    L = g["num_hidden_layers"]["value"]
    ks = []
    for i in range(L):
        ks += [oracle.contribution_index(i, False), oracle.contribution_index(i, True)]
    assert ks == list(range(2, 2 * L + 2))
    assert len(ks) == g["residual_additions"]["value"]
    n = len(ks) + 1
    eye = np.eye(n)
    r = oracle.residual_step(np.zeros(n), eye[0], 1)      # the embedding
    for j, k in enumerate(ks):
        r = oracle.residual_step(r, eye[j + 1], k)
    np.testing.assert_allclose(r, np.full(n, 1 / math.sqrt(n)), rtol=1e-13)
    assert abs((r ** 2).sum() - 1.0) < 1e-13
    # the MoE layers are MLP sublayers: layer i enters as contribution 2(i+1)+1
    assert [oracle.contribution_index(i, True) for i in (0, 3, 51)] == [3, 9, 105]


def test_post_norm_closed_forms_and_torch():
    """RMSNorm of the FP32 layer output: constant and one-hot rows in closed form, exact
    power-of-two scale invariance at eps = 0, and torch float64 on random rows. A sum in
    place of the mean, eps outside the root or a dropped weight fails one of them."""
    w = recipes.WORKLOADS[1]
    nw = synth.norm_weight(w)
    wv = _ref.bf16_bits_to_f64(nw)
    d, eps = w.d, w.eps
    c = np.full((1, d), 0.37)
    np.testing.assert_allclose(oracle.post_norm(c, nw, eps)[0], 0.37 / math.sqrt(0.37 ** 2 + eps) * wv, rtol=1e-15)
    oh = np.zeros((1, d)); oh[0, 11] = -3.0
    n = oracle.post_norm(oh, nw, eps)[0]
    assert np.count_nonzero(n) == 1
    assert abs(n[11] - (-3.0 / math.sqrt(9.0 / d + eps)) * wv[11]) <= 1e-15 * abs(n[11])
    rng = np.random.default_rng(3)
    y = rng.standard_normal((9, d)) * 0.05
    base = oracle.post_norm(y, nw, 0.0)
    for s in (8.0, 0.25):
        assert np.array_equal(oracle.post_norm(y * s, nw, 0.0), base)
    ones = np.full(d, 0x3F80, dtype=np.uint16)
    n1 = oracle.post_norm(y, ones, eps)
    ms = (y ** 2).mean(1)
    np.testing.assert_allclose((n1 ** 2).mean(1), ms / (ms + eps), rtol=1e-13)
    yt = torch.from_numpy(y)
    ref = yt * torch.rsqrt(yt.pow(2).mean(-1, keepdim=True) + eps) * torch.from_numpy(wv)
    np.testing.assert_allclose(oracle.post_norm(y, nw, eps), ref.numpy(), rtol=1e-14, atol=0)


# --- FP8 (OCP E4M3 elements, MX block scales) ------------------------------------------------

def test_e4m3_decode_matches_torch_and_ocp_anchors():
    """Every one of the 256 codes decodes like torch's float8_e4m3fn (NaN where it has NaN),
    and the defining values of the OCP E4M3 format sit where the standard puts them."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    anchors = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x07: 0.875 * 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0, 0xFE: -448.0}
    for c, v in anchors.items():
        assert oracle.e4m3_value(c) == v
    assert np.isnan(oracle.e4m3_value(0x7F)) and np.isnan(oracle.e4m3_value(0xFF))


def test_e4m3_round_matches_torch_on_every_bf16_in_range():
    """Round-to-nearest-even against torch's float8_e4m3fn conversion for every finite bf16
    value below the first value torch turns into NaN (464); above 448 the oracle saturates."""
    bits = np.arange(65536, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) < 464.0)
    vals = vals[keep]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_round(float(v)) for v in vals], dtype=np.uint8)
    diff = got != ref
    assert not diff.any(), vals[diff][:8]
    for v in (448.0, 463.9, 1e4, 1e30):
        assert oracle.e4m3_round(v) == 0x7E and oracle.e4m3_round(-v) == 0xFE


def _grid_matrix(rng, rows, K):
    """Values exactly on the E4M3 x 2^s grid with one e-field-15 element per block."""
    nb = K // 32
    finite = np.array([c for c in range(0x7F) if not np.isnan(oracle.e4m3_value(c))], dtype=np.uint8)
    q = rng.choice(finite, size=(rows, K)).astype(np.uint8)
    q |= (rng.integers(0, 2, size=(rows, K)) << 7).astype(np.uint8)
    top = rng.integers(0x78, 0x7F, size=(rows, nb)).astype(np.uint8)      # exponent field 15
    pos = rng.integers(0, 32, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            q[r, 32 * b + pos[r, b]] = top[r, b] | (q[r, 32 * b + pos[r, b]] & 0x80)
    s = rng.integers(127 - 20, 127 - 8, size=(rows, nb)).astype(np.uint8)
    return q, s


def test_fp8_quantize_round_trips_grid_values():
    """A matrix already on the grid (with the block maximum in the top binade) comes back
    with the same codes and scales: pins the shared-exponent rule and the element rounding."""
    rng = np.random.default_rng(11)
    q, s = _grid_matrix(rng, 6, 128)
    w = oracle.fp8_dequantize(q, s)
    q2, s2 = oracle.fp8_quantize(w)
    assert np.array_equal(s2, s)
    # +0 and -0 are the same value; compare values
    assert np.array_equal(oracle.fp8_dequantize(q2, s2), w)


def test_fp8_quantize_nearest_and_bounds():
    """On random bf16 weights: each code is the nearest grid value (brute force over all
    finite codes, ties to the even code), the block maximum lands in [256, 448] * 2^s, and
    a block of zeros gets scale 2^0."""
    rng = np.random.default_rng(5)
    vals = (rng.standard_normal((4, 96)) * 0.02).astype(np.float32)
    vals[1, 32:64] = 0.0
    w = _ref.f64_to_bf16_bits_rne(vals.astype(np.float64))
    q, s = oracle.fp8_quantize(w)
    wv = _ref.bf16_bits_to_f64(w)
    grid = np.array([oracle.e4m3_value(c) for c in range(256)])
    fin = np.nonzero(~np.isnan(grid))[0]
    for r in range(4):
        for k in range(96):
            sc = 2.0 ** (int(s[r, k // 32]) - 127)
            x = wv[r, k] / sc
            d = np.abs(grid[fin] - x)
            best = fin[d == d.min()]
            best_vals = set(grid[best].tolist())
            assert grid[q[r, k]] in best_vals or (x == 0 and grid[q[r, k]] == 0)
            if len(best_vals) > 1:                     # an exact tie: the even mantissa wins
                assert q[r, k] % 2 == 0
    assert s[1, 1] == 127 and not (q[1, 32:64] & 0x7F).any()
    for r in range(4):
        for b in range(3):
            if r == 1 and b == 1:
                continue
            top = max(abs(grid[c]) for c in q[r, 32 * b: 32 * b + 32])
            assert 256 <= top <= 448

"""Pins for the oracle's gating: closed forms, a library sigmoid, brute-force
enumeration of group subsets and expert subsets, invariants and tie cases."""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import synth
from oracle import route


def test_sigmoid_closed_forms_and_library():
    l = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 1e-8], dtype=np.float32)
    s = route.sigmoid_scores(l)
    assert s[0] == np.float32(0.5)
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 3
    assert np.array_equal(route.sigmoid_scores(r), expit(r.astype(np.float64)).astype(np.float32))
    # 1 - s(x) = s(-x)
    assert np.allclose(1.0 - route.sigmoid_scores(r).astype(np.float64), route.sigmoid_scores(-r), atol=1e-7)


def test_router_logits_against_float_loop():
    x = synth.bf16_bits_to_f32(synth.gen_x(synth.TINY, tokens=3))
    w = synth.bf16_bits_to_f32(synth.gen_router_w(synth.TINY))
    lg = route.router_logits(x, w)
    for t in range(3):
        for e in range(0, 16, 5):
            acc = sum(float(a) * float(b) for a, b in zip(x[t], w[e]))   # bf16*bf16 products are exact in fp64
            assert abs(float(lg[t, e]) - acc) <= abs(acc) * 2.0 ** -23 + 1e-30


def _brute_select(b, s, n_group, topk_group, top_k, group_rule="top2_sum"):
    """Independent formulation: the kept groups are the g_k-subset with the largest
    total group score (scores distinct), the experts the k-subset of the kept ones
    with the largest total b; slots ordered by descending b."""
    e = b.shape[0]
    gsz = e // n_group
    gs = []
    for g in range(n_group):
        vals = sorted((float(v) for v in b[g * gsz:(g + 1) * gsz]), reverse=True)
        gs.append(float(np.float32(vals[0]) + np.float32(vals[1])) if group_rule == "top2_sum" and gsz > 1 else vals[0])
    best_groups = max(itertools.combinations(range(n_group), topk_group), key=lambda c: sum(gs[g] for g in c))
    cands = [x for g in best_groups for x in range(g * gsz, (g + 1) * gsz)]
    best = max(itertools.combinations(cands, top_k), key=lambda c: sum(float(b[x]) for x in c))
    slots = sorted(best, key=lambda x: -float(b[x]))
    w = np.array([s[x] for x in slots], dtype=np.float32)
    tot = np.float32(0)
    for v in w:
        tot = np.float32(tot + v)
    return slots, (w / tot).astype(np.float32)


@pytest.mark.parametrize("bias_scale", [0.0, 0.3])
def test_tiny_shape_matches_brute_force(bias_scale):
    sc = synth.gen_scores(64, 16, cfg_id=0)
    bias = synth.gen_bias(16, scale=bias_scale) if bias_scale else None
    idx, w = route.select(sc, bias, 4, 2, 2)
    b = route.biased(sc, bias)
    for t in range(64):
        slots, wb = _brute_select(b[t], sc[t], 4, 2, 2)
        assert idx[t].tolist() == slots
        assert np.array_equal(w[t], wb)


def test_all_groups_kept_is_plain_topk():
    sc = synth.gen_scores(200, 64, cfg_id=1)
    idx, _ = route.select(sc, None, 8, 8, 6)
    want = np.argsort(-sc, axis=1, kind="stable")[:, :6]
    assert np.array_equal(idx, want)


def test_v3_shape_invariants():
    sc = synth.gen_scores(256, 256, cfg_id=2)
    bias = synth.gen_bias(256, scale=0.2)
    idx, w = route.select(sc, bias, 8, 4, 8)
    b = route.biased(sc, bias)
    gs = route.group_scores(b, 8)
    for t in range(256):
        chosen = idx[t]
        assert len(set(chosen.tolist())) == 8                                    # exactly k distinct
        groups = set((chosen // 32).tolist())
        assert len(groups) <= 4                                                  # <= topk_group groups
        kept = route.kept_groups(gs[t:t + 1], 4)[0]
        assert groups <= set(kept.tolist())
        dropped = [g for g in range(8) if g not in kept]
        assert min(gs[t, kept]) >= max(gs[t, dropped])                           # kept groups score highest
        pool = [x for g in kept for x in range(32 * g, 32 * g + 32)]
        others = [x for x in pool if x not in chosen]
        assert b[t, chosen].min() >= b[t, others].max()                          # chosen b dominate
        assert np.all(np.diff(b[t, chosen]) <= 0)                                # slots descend
        assert abs(float(w[t].astype(np.float64).sum()) - 1.0) <= 8 * 2.0 ** -23  # normalised


def test_bias_changes_selection_only():
    sc = synth.gen_scores(128, 64, cfg_id=3)
    bias = np.zeros(64, np.float32)
    bias[5] = 10.0                                     # force expert 5 everywhere
    idx, w = route.select(sc, bias, 4, 2, 4)
    assert np.all(idx[:, 0] == 5)
    for t in range(128):
        s = sc[t, idx[t]]
        tot = np.float32(0)
        for v in s:
            tot = np.float32(tot + v)
        assert np.array_equal(w[t], (s / tot).astype(np.float32))        # unbiased scores weight the output


def test_tie_rules():
    # every score equal: lowest groups, then lowest expert ids, in index order
    sc = np.full((1, 16), 0.5, np.float32)
    idx, w = route.select(sc, None, 4, 2, 3)
    assert idx[0].tolist() == [0, 1, 2]
    assert np.all(w == np.float32(1 / 3))
    # equal group scores: the lower group index wins
    sc = np.array([[0.1, 0.2, 0.9, 0.9, 0.2, 0.1, 0.3, 0.3]], np.float32)   # groups of 2: 0.3, 1.8, 0.3, 0.6
    idx, _ = route.select(sc, None, 4, 2, 2)
    assert idx[0].tolist() == [2, 3]
    idx, _ = route.select(sc, None, 4, 3, 3)                    # groups 1, 3 and (tie 0 vs 2) 0
    assert sorted(idx[0].tolist()) == [2, 3, 6]
    sc2 = np.array([[0.3, 0.0, 0.9, 0.9, 0.2, 0.1, 0.25, 0.25]], np.float32)  # groups 0.3, 1.8, 0.3, 0.5
    idx, _ = route.select(sc2, None, 4, 3, 4)
    assert idx[0].tolist() == [2, 3, 0, 6]                     # group 0 (tie with 2) kept; slot order by b, then index
    # -0 and +0 compare equal: the lower index comes first
    b = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)
    with np.errstate(invalid="ignore"):                        # zero scores: weights 0/0 (outside sigmoid's range)
        idx, _ = route.select(b, None, 1, 1, 2)
    assert idx[0].tolist() == [0, 1]


def test_ties_match_brute_force_lexicographic():
    """With many ties: the chosen set maximises sum(b); among those, the
    lexicographically smallest sorted index tuple (lower index wins)."""
    sc = synth.gen_scores(300, 16, cfg_id=4, ties=True)
    idx, _ = route.select(sc, None, 4, 4, 3)
    for t in range(300):
        sets = list(itertools.combinations(range(16), 3))
        best = max(sum(float(sc[t, x]) for x in c) for c in sets)
        lex = min(c for c in sets if sum(float(sc[t, x]) for x in c) == best)
        assert sorted(idx[t].tolist()) == list(lex)


def test_group_score_max_rule_and_singletons():
    sc = synth.gen_scores(50, 32, cfg_id=5)
    gs = route.group_scores(sc, 4, "max")
    assert np.array_equal(gs, sc.reshape(50, 4, 8).max(-1))
    gs1 = route.group_scores(sc, 32)                           # one expert per group: its own score
    assert np.array_equal(gs1, sc)


def test_weights_scale():
    sc = synth.gen_scores(10, 16, cfg_id=6)
    _, w1 = route.select(sc, None, 4, 2, 4)
    _, w2 = route.select(sc, None, 4, 2, 4, routed_scale=2.5)
    assert np.array_equal(w2, (w1 * np.float32(2.5)).astype(np.float32))


@pytest.mark.parametrize("case", [(256, 8, 8, 4, 0.0), (256, 8, 8, 4, 0.05), (64, 6, 8, 3, 0.1), (16, 2, 4, 2, 0.2)])
def test_group_rule_matches_transformers_deepseek_v3_router(case):
    """The top-2-sum group score, the kept-group mask and the normalised weights against an
    independent implementation of the same gating: transformers' DeepSeek-V3 router module
    (library code, not part of the oracle).  Its router is a linear layer followed by the sigmoid;
    with the hidden size equal to E and an identity weight the linear layer returns its input, so
    both sides route the same fp32 scores.  Random continuous scores have no ties, so the
    chosen sets are unique; the weights agree to fp32 rounding of the sum's order."""
    import torch
    from transformers.models.deepseek_v3.configuration_deepseek_v3 import DeepseekV3Config
    from transformers.models.deepseek_v3.modeling_deepseek_v3 import DeepseekV3TopkRouter
    E, k, G, gk, bscale = case
    cfg = DeepseekV3Config(hidden_size=E, n_routed_experts=E, num_experts_per_tok=k, n_group=G, topk_group=gk,
                           norm_topk_prob=True, routed_scaling_factor=1.0)
    router = DeepseekV3TopkRouter(cfg)
    logits = (np.random.default_rng(E + k + G).standard_normal((500, E)) * 1.7).astype(np.float32)
    bias = synth.gen_bias(E, cfg_id=E + k, scale=bscale) if bscale else np.zeros(E, np.float32)
    with torch.no_grad():
        router.weight.copy_(torch.eye(E))
        router.e_score_correction_bias.copy_(torch.from_numpy(bias))
        lg, w_lib, idx_lib = router(torch.from_numpy(logits))
        assert torch.equal(lg, torch.from_numpy(logits))
        scores = torch.sigmoid(torch.from_numpy(logits)).numpy()
    idx, w = route.select(scores, bias if bscale else None, G, gk, k)
    idx_lib = idx_lib.numpy()
    assert np.array_equal(np.sort(idx, 1), np.sort(idx_lib, 1))
    # weights per expert id: the library returns its slots in its own order
    order, order_lib = np.argsort(idx, 1), np.argsort(idx_lib, 1)
    w_by_id = np.take_along_axis(w, order, 1)
    w_lib_by_id = np.take_along_axis(w_lib.numpy(), order_lib, 1)
    assert np.allclose(w_by_id, w_lib_by_id, rtol=4 * k * 2.0 ** -24, atol=0)

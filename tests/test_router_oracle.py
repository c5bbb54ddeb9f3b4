"""Pins of the router oracle (oracle/moe_router.py) against things other than
itself: a counting-rank formulation of top-k on tiny inputs, scipy's softmax
and expit, the alternative evaluation order of the renormalised softmax,
shift invariance, hand-built cases whose picks follow from the definitions,
and planted mistakes that must make a pin fail.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from oracle import moe_router as R


def rank_pick(score, k, allowed=None):
    """Top-k by counting ranks: expert e's rank is the number of experts that
    beat it (larger score, or equal score and lower index)."""
    T, E = score.shape
    out = np.zeros((T, k), np.int64)
    for t in range(T):
        cand = [e for e in range(E) if allowed is None or allowed[t, e]]
        for e in cand:
            r = sum(1 for f in cand if score[t, f] > score[t, e] or (score[t, f] == score[t, e] and f < e))
            if r < k:
                out[t, r] = e
    return out


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (6, 6)])
def test_renormalize_ids_match_rank_count(seed, E, k):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((7, E)).astype(np.float32)
    l[0, :] = 0.5                      # all tied: ascending ids
    l[1, 1] = l[1, 3] = l[1].max() + 1  # tie at the top
    ids, _ = R.route_renormalize(l, k)
    assert np.array_equal(ids, rank_pick(l.astype(np.float64), k))


@pytest.mark.parametrize("seed", range(4))
def test_renormalize_weights_are_softmax_over_picks(seed):
    rng = np.random.default_rng(seed)
    l = (3 * rng.standard_normal((9, 12))).astype(np.float32)
    ids, w = R.route_renormalize(l, 4)
    # the other evaluation order: softmax over the picked logits only
    picked = np.take_along_axis(l.astype(np.float64), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, softmax(picked, axis=1), rtol=1e-13)
    # full softmax, pick, renormalise (scipy)
    p = np.take_along_axis(softmax(l.astype(np.float64), axis=1), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, p / p.sum(axis=1, keepdims=True), rtol=1e-12)


def test_renormalize_all_experts_is_softmax():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((5, 8)).astype(np.float32)
    ids, w = R.route_renormalize(l, 8)
    full = np.zeros_like(w)
    np.put_along_axis(full, ids.astype(np.int64), w, axis=1)
    np.testing.assert_allclose(full, softmax(l.astype(np.float64), axis=1), rtol=1e-13)
    assert np.all(np.diff(np.take_along_axis(l, ids.astype(np.int64), axis=1), axis=1) <= 0)


def test_renormalize_shift_invariance():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((6, 16)).astype(np.float32)
    ids, w = R.route_renormalize(l, 3)
    ids2, w2 = R.route_renormalize(l + np.float32(4.0), 3)  # exact in float32 for |l| < 4
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=1e-6)


def test_nonfinite_logits():
    l = np.array([[np.nan, -np.inf, 1.0, np.inf]], np.float32)
    ids, w = R.route_renormalize(l, 2)
    assert ids.tolist() == [[3, 2]]
    assert w.tolist() == [[1.0, 0.0]]
    ids, _ = R.route_renormalize(l, 4)
    assert ids.tolist() == [[3, 2, 0, 1]]  # NaN and -inf both clamp to -FLT_MAX: lower id first


def test_deepseek_without_groups_or_bias_is_sigmoid_topk():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((8, 16)).astype(np.float32)
    ids, w = R.route_deepseek_v3(l, 4)
    ids_r, _ = R.route_renormalize(l, 4)  # sigmoid is increasing: same picks
    assert np.array_equal(ids, ids_r)
    s = expit(np.take_along_axis(l.astype(np.float64), ids.astype(np.int64), axis=1))
    np.testing.assert_allclose(w, s / s.sum(axis=1, keepdims=True), rtol=1e-6)
    ids1, w1 = R.route_deepseek_v3(l, 4, n_group=1, topk_group=1, routed_scaling_factor=2.5)
    assert np.array_equal(ids1, ids)
    np.testing.assert_allclose(w1, 2.5 * w, rtol=1e-15)


def test_deepseek_bias_selects_but_does_not_weight():
    l = np.array([[2.0, 1.0, 0.0]], np.float32)
    ids, w = R.route_deepseek_v3(l, 1, bias=np.array([0, 0, 5], np.float32))
    assert ids.tolist() == [[2]] and w.tolist() == [[1.0]]
    ids, w = R.route_deepseek_v3(l, 2, bias=np.array([0, 0, 5], np.float32))
    assert ids.tolist() == [[2, 0]]
    s = expit(np.array([0.0, 2.0]))
    np.testing.assert_allclose(w[0], s / s.sum(), rtol=1e-6)


def test_deepseek_group_limit_hand_case():
    # sigmoid scores s; groups of 2: {0,1} {2,3} {4,5} {6,7}
    s = np.array([0.95, 0.05, 0.80, 0.75, 0.60, 0.55, 0.10, 0.20])
    l = np.log(s / (1 - s)).astype(np.float32)[None, :]
    # one group kept: {2,3} (0.80 + 0.75) beats {0,1} (0.95 + 0.05) though expert 0 is best
    ids, _ = R.route_deepseek_v3(l, 2, n_group=4, topk_group=1)
    assert ids.tolist() == [[2, 3]]
    # two groups kept: {2,3} and {4,5}; the best three of their experts
    ids, _ = R.route_deepseek_v3(l, 3, n_group=4, topk_group=2)
    assert ids.tolist() == [[2, 3, 4]]
    # all four groups kept: plain top-k
    ids, _ = R.route_deepseek_v3(l, 3, n_group=4, topk_group=4)
    assert ids.tolist() == [[0, 2, 3]]


@pytest.mark.parametrize("seed", range(3))
def test_deepseek_group_limit_matches_brute_force(seed):
    """Group scores and kept groups by explicit enumeration of group subsets."""
    rng = np.random.default_rng(seed)
    T, E, ng, tg, k = 5, 12, 4, 2, 3
    l = rng.standard_normal((T, E)).astype(np.float32)
    b = (0.1 * rng.standard_normal(E)).astype(np.float32)
    ids, _ = R.route_deepseek_v3(l, k, bias=b, n_group=ng, topk_group=tg)
    sb = ((1 / (1 + np.exp(-l.astype(np.float64)))).astype(np.float32) + b).astype(np.float32)
    G = E // ng
    for t in range(T):
        gs = [np.float32(sorted(sb[t, g * G:(g + 1) * G])[-1]) + np.float32(sorted(sb[t, g * G:(g + 1) * G])[-2])
              for g in range(ng)]
        # the kept set is the subset of tg groups with the best sorted scores, ties to lower ids
        best = max(itertools.combinations(range(ng), tg),
                   key=lambda c: (sorted((gs[g] for g in c), reverse=True), [-g for g in c]))
        allowed = np.zeros((1, E), bool)
        for g in best:
            allowed[0, g * G:(g + 1) * G] = True
        assert ids[t].tolist() == rank_pick(sb[t:t + 1].astype(np.float64), k, allowed)[0].tolist()


def test_deepseek_zero_scores_give_zero_weights():
    l = np.full((1, 4), -np.inf, np.float32)
    _, w = R.route_deepseek_v3(l, 2)
    assert w.tolist() == [[0.0, 0.0]]


# ------------------------------------------------------------------ planted mistakes
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_router_mistakes_are_caught(monkeypatch):
    orig_topk = R.topk_order
    # 1. ties to the higher index
    def bad_ties(score, k, allowed=None):
        s = np.asarray(score, np.float64)
        if allowed is not None:
            s = np.where(allowed, s, -np.inf)
        return (s.shape[-1] - 1 - np.argsort(-s[..., ::-1], axis=-1, kind="stable"))[..., :k]
    with monkeypatch.context() as m:
        m.setattr(R, "topk_order", bad_ties)
        assert _fails(lambda: test_renormalize_ids_match_rank_count(0, 5, 2))
    # 2. picks in ascending score order
    with monkeypatch.context() as m:
        m.setattr(R, "topk_order", lambda s, k, a=None: orig_topk(s, k, a)[..., ::-1])
        assert _fails(test_renormalize_all_experts_is_softmax)
    # 3. weights not renormalised over the picks
    orig_rn = R.route_renormalize
    def no_renorm(l, k):
        ids, _ = orig_rn(l, k)
        p = softmax(R.clamp_logits(l), axis=1)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)
    with monkeypatch.context() as m:
        m.setattr(R, "route_renormalize", no_renorm)
        assert _fails(lambda: test_renormalize_weights_are_softmax_over_picks(0))
    # 4. DeepSeekV3 weights from the biased scores
    orig_ds = R.route_deepseek_v3
    def biased_weights(l, k, bias=None, **kw):
        ids, w = orig_ds(l, k, bias=bias, **kw)
        if bias is None:
            return ids, w
        s = expit(R.clamp_logits(l)) + np.asarray(bias, np.float64)[None, :]
        sk = np.take_along_axis(s, ids.astype(np.int64), axis=1)
        return ids, sk / sk.sum(axis=1, keepdims=True)
    with monkeypatch.context() as m:
        m.setattr(R, "route_deepseek_v3", biased_weights)
        assert _fails(test_deepseek_bias_selects_but_does_not_weight)
    # 5. group score from the top-1 instead of the top-2 sum
    def top1_groups(l, k, bias=None, n_group=0, topk_group=0, routed_scaling_factor=1.0):
        lc = R.clamp_logits(l)
        T, E = lc.shape
        sb = R._sigmoid_f32(lc) + (0 if bias is None else np.asarray(bias, np.float32))
        G = E // n_group
        g1 = sb.reshape(T, n_group, G).max(axis=2)
        keep = orig_topk(g1, topk_group)
        gm = np.zeros((T, n_group), bool)
        np.put_along_axis(gm, keep, True, axis=1)
        ids = orig_topk(sb, k, np.repeat(gm, G, axis=1))
        return ids.astype(np.int32), np.ones(ids.shape)
    with monkeypatch.context() as m:
        m.setattr(R, "route_deepseek_v3", top1_groups)
        assert _fails(test_deepseek_group_limit_hand_case)


def test_deepseek_on_fine_grained_logits_is_well_formed():
    import synth
    wl = synth.workload("fine_grained_prefill")
    l = synth.make_logits(wl, T=512)
    ids, w = R.route_deepseek_v3(l, 8, bias=synth.make_router_bias(wl), n_group=8, topk_group=4,
                                 routed_scaling_factor=2.5)
    G = wl.E // 8
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == 8
        assert len({int(e) // G for e in ids[t]}) <= 4
    np.testing.assert_allclose(w.sum(axis=1), 2.5, rtol=1e-12)

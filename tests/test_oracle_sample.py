"""Pins for the sampling oracle (oracle/sample.py): a hand-worked example,
scipy's softmax, a brute-force min-p filter on probabilities, the inversion
of the cumulative distribution on a grid of draws, and limit cases."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle.sample import kept_probs, penalize, penalty_window, sample_ref, sample_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sample_example.json")


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    par, dt, hist = ex["parent"], ex["draft_tok"], ex["hist"]
    R = len(ex["logits"])
    for r in range(R):
        win = penalty_window(hist, par, dt, r, ex["window"])
        assert win == ex["windows"][r]
        z = penalize(ex["logits"][r], win, ex["penalty"])
        np.testing.assert_allclose(z, ex["penalised"][r], rtol=0, atol=1e-12)
        q, _, _ = kept_probs(z, 1.0, ex["min_p"])
        np.testing.assert_allclose(q, ex["probs"][r], rtol=0, atol=2e-6)
    g, _ = sample_ref(ex["logits"], hist, par, dt, window=ex["window"], penalty=ex["penalty"],
                      temperature=0.0, min_p=ex["min_p"], u=[0.5] * R)
    assert g.tolist() == ex["greedy"]
    for d in ex["draws"]:
        t, _ = sample_ref(ex["logits"], hist, par, dt, window=ex["window"], penalty=ex["penalty"],
                          temperature=1.0, min_p=ex["min_p"], u=d["u"])
        assert t.tolist() == d["tok"], d


@pytest.mark.parametrize("tau", [0.5, 1.0, 1.7])
def test_no_filter_no_penalty_is_softmax(tau):
    """min-p 0 and no window: the kept distribution is scipy's softmax of x / tau."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(50) * 3
    q, keep, _ = kept_probs(penalize(x, [], 1.2), tau, 0.0)
    assert keep.all()
    np.testing.assert_allclose(q, softmax(x / tau), rtol=1e-12, atol=0)


@pytest.mark.parametrize("min_p", [0.01, 0.1, 0.5, 0.9])
def test_min_p_filter_on_probabilities(min_p):
    """The log-domain filter keeps exactly the tokens whose softmax probability
    is at least min_p times the largest (brute force on probabilities)."""
    rng = np.random.default_rng(2)
    for _ in range(20):
        x = rng.standard_normal(200) * 2
        tau = float(rng.uniform(0.3, 2.0))
        q, keep, _ = kept_probs(x, tau, min_p)
        p = softmax(x / tau)
        brute = p >= min_p * p.max()
        margin = np.abs(p - min_p * p.max()) > 1e-12
        assert np.array_equal(keep[margin], brute[margin])
        pk = np.where(brute, p, 0)
        np.testing.assert_allclose(q, pk / pk.sum(), rtol=1e-10, atol=1e-15)


def test_cdf_inversion_frequencies():
    """Draws on a fine grid of u land on each token in proportion to its kept
    probability (the inversion of the cumulative distribution)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(9) * 1.5
    x[4] = -np.inf
    N = 20000
    q, _, _ = kept_probs(x, 1.3, 0.05)
    counts = np.zeros(9)
    for k in range(N):
        t, _ = sample_row(x, [], 1.2, 1.3, 0.05, (k + 0.5) / N)
        counts[t] += 1
    np.testing.assert_allclose(counts / N, q, rtol=0, atol=1.5 / N)
    assert counts[4] == 0


def test_first_kept_token_at_u_zero_and_last_near_one():
    x = np.array([-5.0, 1.0, -9.0, 0.9, 1.0, -7.0])
    t0, _ = sample_row(x, [], 1.0, 1.0, 0.5, 0.0)
    t1, _ = sample_row(x, [], 1.0, 1.0, 0.5, np.nextafter(1.0, 0.0))
    assert (t0, t1) == (1, 4)


def test_penalty_sign_once_and_theta_one():
    x = np.array([2.0, -2.0, 0.0, 1.5, -0.5])
    z = penalize(x, [0, 1, 2, 0, 0, 1, 99, -3], 2.0)       # repeats count once; out-of-range ids ignored
    np.testing.assert_array_equal(z, [1.0, -4.0, 0.0, 1.5, -0.5])
    np.testing.assert_array_equal(penalize(x, [0, 1, 2, 3, 4], 1.0), x)
    for v in (3.0, -3.0):                                   # either sign loses probability
        zz = penalize(np.array([v, 0.0]), [0], 1.2)
        assert softmax(zz)[0] < softmax(np.array([v, 0.0]))[0]


def test_windows():
    parent = [-1, 0, 1, 2, 3, 4, 5, 6, 7, 8]               # a chain of 10 drafts
    draft = [10 + i for i in range(10)]
    hist = [1, 2, 3]
    assert penalty_window(hist, parent, draft, 0, 2) == [2, 3]
    assert penalty_window(hist, parent, draft, 1, 2) == [3, 10]
    assert penalty_window(hist, parent, draft, 10, 4) == [16, 17, 18, 19]
    assert penalty_window(hist, parent, draft, 3, 100) == [1, 2, 3, 10, 11, 12]
    assert penalty_window(hist, parent, draft, 5, 0) == []
    assert penalty_window([], parent, draft, 0, 8) == []
    # parents outside [-1, t) count as roots, as in the attention mask
    assert penalty_window([7], [-1, 5, -9], [4, 5, 6], 3, 8) == [7, 6]


def test_greedy_ties_and_small_temperature():
    x = np.array([0.5, 3.0, -1.0, 3.0, 2.9])
    assert sample_row(x, [], 1.2, 0.0, 0.1, 0.99)[0] == 1           # ties: lower id
    assert sample_row(x, [1], 1.2, 0.0, 0.1, 0.99)[0] == 3          # 1 is penalised
    for u in (1e-9, 0.3, 0.999):                                    # tau -> 0: the argmax
        assert sample_row(x, [1, 3], 1.2, 1e-3, 0.0, u)[0] == 4


def test_min_p_one_keeps_only_the_maximum():
    x = np.array([1.0, 4.0, 2.0, 4.0])
    assert sample_row(x, [], 1.0, 1.0, 1.0, 0.49)[0] == 1
    assert sample_row(x, [], 1.0, 1.0, 1.0, 0.51)[0] == 3


def test_rows_follow_the_forest():
    """Row t+1's window holds draft t's root path: on a forest whose drafts are
    all token 0, row t+1 penalises token 0 and row 0 (empty history) does not."""
    parent = [-1, 0, -1, 2]
    draft = [0, 0, 0, 0]
    x = np.tile(np.array([1.0, 0.95]), (5, 1))
    g, _ = sample_ref(x, [], parent, draft, window=4, penalty=1.2, temperature=0.0, min_p=0.1, u=[0.5] * 5)
    assert g.tolist() == [0, 1, 1, 1, 1]


# ---------------------------------------------------------------------------
# top-p (nucleus) filter
# ---------------------------------------------------------------------------
TOPP_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "top_p_example.json")


def test_top_p_hand_worked_example():
    """Kept sets, renormalised probabilities and draws worked by hand (tests/golden/top_p_example.json)."""
    ex = json.load(open(TOPP_GOLDEN))
    x = np.array(ex["logits"])
    for c in ex["cases"]:
        q, keep, _ = kept_probs(x, c["temperature"], c["min_p"], c["top_p"])
        assert np.nonzero(keep)[0].tolist() == c["kept"], c
        np.testing.assert_allclose(q, c["probs"], rtol=0, atol=1e-12)
        for u, tok in c["draws"]:
            t, _ = sample_row(x, [], 1.2, c["temperature"], c["min_p"], u, c["top_p"])
            assert t == tok, (c, u)


def _brute_keep(p, top_p):
    """Token i is kept iff the exact sum of the strictly larger probabilities is below top_p."""
    import math
    return np.array([math.fsum(pj for pj in p if pj > pi) < top_p for pi in p])


@pytest.mark.parametrize("seed", range(6))
def test_top_p_brute_force_with_ties(seed):
    """Against an O(V^2) exact sum over strictly more probable tokens, on
    logits with many exact ties."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 60))
    x = np.round(rng.standard_normal(V) * 2, 1)          # one decimal: ties are common
    tau = float(rng.choice([0.4, 0.8, 1.0, 1.2]))
    for top_p in (0.05, 0.3, 0.5, 0.77, 0.9, 0.99):
        _, keep, y = kept_probs(x, tau, 0.0, top_p)
        p = softmax(y)
        above = np.array([sum(pj for pj in p if pj > pi) for pi in p])
        clear = np.abs(above - top_p) > 1e-9
        assert np.array_equal(keep[clear], _brute_keep(p, top_p)[clear]), (seed, top_p)
        # ties are kept or dropped together
        for v in np.unique(p):
            assert len(set(keep[p == v])) == 1


def test_top_p_is_the_sorted_cumulative_rule_on_distinct_values():
    """With distinct probabilities the rule is the textbook one: sort
    descending and keep while the cumulative mass before a token is below
    top_p (the smallest prefix whose mass reaches top_p)."""
    rng = np.random.default_rng(9)
    for _ in range(30):
        x = rng.standard_normal(300) * 2.5
        top_p = float(rng.uniform(0.05, 0.99))
        _, keep, y = kept_probs(x, 1.0, 0.0, top_p)
        p = softmax(y)
        order = np.argsort(-p)
        before = np.cumsum(p[order]) - p[order]
        ref = np.zeros(len(p), bool)
        ref[order[before < top_p]] = True
        assert np.array_equal(keep, ref)
        assert p[keep].sum() >= top_p - 1e-12 and p[keep].sum() - p[keep].min() < top_p


def test_top_p_limits_and_monotone():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(500)
    x[[3, 77]] = x.max() + 1.0                          # two tokens tie at the maximum
    x[5] = -np.inf
    _, keep1, _ = kept_probs(x, 1.0, 0.0, 1.0)
    assert keep1.sum() == 499 and not keep1[5]          # top_p = 1: every token of non-zero probability
    _, keep0, _ = kept_probs(x, 1.0, 0.0, 1e-9)
    assert np.nonzero(keep0)[0].tolist() == [3, 77]     # tiny top_p: the tied maxima only
    prev = keep0
    for top_p in np.linspace(0.01, 0.999, 40):
        _, k, _ = kept_probs(x, 1.0, 0.0, float(top_p))
        assert (k | prev).sum() == k.sum()              # growing top_p only adds tokens
        prev = k


def test_top_p_and_min_p_intersect_like_the_sequential_filters():
    """Kept = passes min-p and passes top-p on the same distribution; the same
    as top-p first, then min-p on the renormalised remainder."""
    rng = np.random.default_rng(11)
    for _ in range(30):
        x = rng.standard_normal(200) * 2
        tau, min_p, top_p = float(rng.uniform(0.4, 1.5)), float(rng.uniform(0.01, 0.5)), float(rng.uniform(0.1, 0.99))
        _, keep, y = kept_probs(x, tau, min_p, top_p)
        p = softmax(y)
        k1 = _brute_keep(p, top_p)
        r = np.where(k1, p, 0.0)
        r = r / r.sum()
        seq = k1 & (r >= min_p * r.max())
        both = k1 & (p >= min_p * p.max())
        assert np.array_equal(seq, both)
        clear = (np.abs(p - min_p * p.max()) > 1e-12)
        assert np.array_equal(keep[clear], both[clear])


def test_top_p_diagnostics_flag_the_nearest_boundary():
    """The near-boundary set flips exactly the value whose mass-above is nearest top_p."""
    ex = json.load(open(TOPP_GOLDEN))
    x = np.array(ex["logits"])
    _, d = sample_row(x, [], 1.2, 1.0, 0.0, 0.5, 0.66)
    assert abs(d["topp_margin"] - 0.01) < 1e-12                 # id 2 has 0.65 above it
    assert np.nonzero(d["keep"])[0].tolist() == [1, 2, 4]
    assert np.nonzero(d["keep_alt"])[0].tolist() == [1, 4]

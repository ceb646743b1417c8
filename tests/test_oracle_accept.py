"""Pins for the acceptance / KV-commit oracle (CPU only)."""
import json
import os

import numpy as np
import pytest

from long_context_kv_ts_amd import inputs
from oracle import accept_ref, commit_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_example.json")


def test_hand_worked_example():
    """tests/golden/accept_example.json: every answer derived by hand."""
    ex = json.load(open(GOLDEN))
    for case in ex["cases"]:
        tgt = list(ex["target_tok"])
        if "target0" in case:
            tgt[0] = case["target0"]
        n, path, bonus = accept_ref(ex["parent"], ex["draft_tok"], tgt, case["rand"])
        assert (n, path, bonus) == (case["n"], case["path"], case["bonus"]), case


def _valid_dp(parent, draft, target):
    """Validity and depth by one pass in node order (parent[t] < t): an
    algorithm independent of the oracle's path enumeration."""
    T = len(parent)
    valid = np.zeros(T, bool)
    depth = np.zeros(T, int)
    for t in range(T):
        p = int(parent[t])
        p = p if -1 <= p < t else -1
        if p < 0:
            valid[t] = draft[t] == target[0]
        else:
            valid[t] = valid[p] and draft[t] == target[p + 1]
            depth[t] = depth[p] + 1
    return valid, depth


@pytest.mark.parametrize("seed", range(30))
def test_random_forests_against_dynamic_programming(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 60))
    parent = np.array([int(rng.integers(-1, t)) if t else -1 for t in range(T)])
    vocab = int(rng.integers(2, 5))                 # small vocabulary: many matches and ties
    draft = rng.integers(0, vocab, T)
    target = rng.integers(0, vocab, T + 1)
    rand = int(rng.integers(0, 2**32))
    n, path, bonus = accept_ref(parent, draft, target, rand)
    valid, depth = _valid_dp(parent, draft, target)
    if not valid.any():
        assert (n, path, bonus) == (0, [], int(target[0]))
        return
    best = depth[valid].max()
    cands = [t for t in range(T) if valid[t] and depth[t] == best]
    last = cands[rand % len(cands)]
    assert n == best + 1 and path[-1] == last and bonus == int(target[last + 1])
    assert all(valid[a] for a in path)
    assert all(int(parent[path[i]]) == path[i - 1] for i in range(1, n)) and int(parent[path[0]]) < 0


def test_planted_path_is_the_unique_answer():
    """The verify workload's forest; targets planted so that exactly one
    root-to-leaf path of the [1,3,3,3] tree matches."""
    c = inputs.make_verify("acc", dtype="f32", Hq=1, Hkv=1, D=64, L=0, seed=7, with_chains=True)
    parent = c.parent
    T = len(parent)
    draft = np.arange(T) + 1000                      # all tokens distinct
    target = np.full(T + 1, -5)
    leaf = max(t for t in range(T) if t < 40 and all(parent[u] != t for u in range(T)))
    path = []
    a = leaf
    while a >= 0:
        path.append(a)
        a = int(parent[a])
    path = path[::-1]
    target[0] = draft[path[0]]
    for i in range(1, len(path)):
        target[path[i - 1] + 1] = draft[path[i]]
    target[leaf + 1] = 77
    assert accept_ref(parent, draft, target, 12345) == (len(path), path, 77)


def test_everything_valid_picks_among_the_deepest():
    """A single chain of T tokens all matching: n = T for any random number."""
    T = 9
    parent = np.arange(-1, T - 1)
    draft = np.arange(T) * 3
    target = np.concatenate([draft, [42]])           # target[t+1] = draft[t+1]
    for r in (0, 1, 7, 2**32 - 1):
        assert accept_ref(parent, draft, target, r) == (T, list(range(T)), 42)


def test_commit_copies_exactly_the_path_rows():
    rng = np.random.default_rng(3)
    Hkv, S, T, D, L = 2, 20, 6, 8, 11
    kc = rng.integers(0, 65535, (Hkv, S, D)).astype(np.uint16)
    vc = rng.integers(0, 65535, (Hkv, S, D)).astype(np.uint16)
    kd = rng.integers(0, 65535, (Hkv, T, D)).astype(np.uint16)
    vd = rng.integers(0, 65535, (Hkv, T, D)).astype(np.uint16)
    path = [4, 1, 5]
    k2, v2 = commit_ref(kc, vc, L, kd, vd, path)
    for i, a in enumerate(path):
        assert np.array_equal(k2[:, L + i], kd[:, a]) and np.array_equal(v2[:, L + i], vd[:, a])
    rest = [j for j in range(S) if not L <= j < L + len(path)]
    assert np.array_equal(k2[:, rest], kc[:, rest]) and np.array_equal(v2[:, rest], vc[:, rest])

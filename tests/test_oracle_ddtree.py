"""Pins of the draft-tree builder oracle (oracle/ddtree.py): hand-worked cases, brute-force
enumeration of every path of small drafts, and the invariants the pages name (ancestor
closure, budget cap, confidence pruning against q* - tau, chain pre-seed, chain mode)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import ddtree as od

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ddtree_E1_three_positions.json")


def _draft(rng, L, K, quantum=None):
    x = rng.normal(0.0, 2.0, size=(L, max(K, 8)))
    lp = x - np.log(np.exp(x).sum(axis=1, keepdims=True))
    lp = -np.sort(-lp, axis=1)[:, :K]
    if quantum:  # coarse values make exact score ties common
        lp = np.minimum(-np.round(-lp / quantum) * quantum, 0.0)
        lp = -np.sort(-lp, axis=1)
    return lp.astype(np.float32)


def test_hand_worked_cases():
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        tau = math.inf if case["tau"] is None else case["tau"]
        t = od.build(g["logp"], case["budget"], tau, case["chain_seed"])
        for key in ("parent", "depth", "rank"):
            assert t[key].tolist() == case[key], (case["derivation"], key, t[key])


@pytest.mark.parametrize("seed", range(40))
def test_best_first_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, K = int(rng.integers(0, 6)), int(rng.integers(1, 5))
    lp = _draft(rng, L, K, quantum=0.5 if seed % 3 == 0 else None)
    budget = int(rng.integers(1, 30))
    tau = [0.0, 0.5, 2.0, 6.0, math.inf][seed % 5]
    for chain in (True, False):
        a = od.build(lp, budget, tau, chain)
        b = od.enumerate_tree(lp, budget, tau, chain)
        for key in ("parent", "depth", "rank", "score"):
            assert np.array_equal(a[key], b[key]), (seed, chain, key)


@pytest.mark.parametrize("seed", range(20))
def test_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    L, K = int(rng.integers(1, 12)), int(rng.integers(1, 9))
    lp = _draft(rng, L, K, quantum=0.25 if seed % 4 == 0 else None)
    budget, tau = int(rng.integers(1, 40)), [0.0, 1.0, 6.0, math.inf][seed % 4]
    t = od.build(lp, budget, tau, chain_seed=True)
    n = len(t["parent"])
    assert 1 <= n <= budget
    q = od.greedy_scores(lp)
    for i in range(1, n):
        p, d = t["parent"][i], t["depth"][i]
        assert 0 <= p < i and t["depth"][p] == d - 1  # ancestor closure, topological ids
        assert t["score"][i] == np.float32(t["score"][p] + lp[d - 1, t["rank"][i]])
        if math.isfinite(tau):
            assert not (t["score"][i] < np.float32(q[d] - np.float32(tau)))  # tau pruning
    chain_len = min(L, budget - 1)
    assert t["rank"][1:chain_len + 1].tolist() == [0] * chain_len  # pre-seeded chain first
    # siblings are distinct candidates
    seen = set(zip(t["parent"][1:].tolist(), t["rank"][1:].tolist()))
    assert len(seen) == n - 1
    # a smaller budget gives a prefix of the same insertion order
    t2 = od.build(lp, max(1, budget - 3), tau, chain_seed=True)
    m = len(t2["parent"])
    assert np.array_equal(t2["parent"], t["parent"][:m])


def test_chain_mode_is_a_tree_without_branching():
    """Luce DFlash README, How it works: chain mode is DDTree with budget = n_spec + 1 and no
    branching (top-1)."""
    rng = np.random.default_rng(7)
    lp = _draft(rng, 15, 1)
    t = od.build(lp, 16, math.inf, chain_seed=True)
    assert t["parent"].tolist() == list(range(-1, 15))
    t = od.build(lp, 16, math.inf, chain_seed=False)
    assert t["parent"].tolist() == list(range(-1, 15))


def test_zero_tau_keeps_only_best_scores():
    rng = np.random.default_rng(8)
    lp = _draft(rng, 6, 4)
    t = od.build(lp, 22, 0.0, chain_seed=False)
    assert t["rank"][1:].tolist() == [0] * 6  # untied random draft: the greedy chain alone


def test_no_pruning_fills_the_budget_when_paths_suffice():
    rng = np.random.default_rng(9)
    lp = _draft(rng, 10, 4)
    t = od.build(lp, 22, math.inf)
    assert len(t["parent"]) == 22


def test_tokens_follow_depth_and_rank():
    lp = np.array([[-0.1, -1.0], [-0.2, -0.5]], dtype=np.float32)
    tok = np.array([[11, 12], [21, 22]], dtype=np.int32)
    t = od.build(lp, 4, math.inf, chain_seed=False)
    assert od.tokens_of(t, tok, 99).tolist() == [99, 11, 21, 22]


def test_rejects_bad_drafts():
    with pytest.raises(ValueError):
        od.build([[0.5, -1.0]], 4)  # positive log-probability
    with pytest.raises(ValueError):
        od.build([[-1.0, -0.5]], 4)  # not sorted
    with pytest.raises(ValueError):
        od.build([[-0.1]], 0)  # empty budget
    with pytest.raises(ValueError):
        od.build([[-0.1]], 4, tau=-1.0)
    with pytest.raises(ValueError):
        od.build(np.zeros((17, 2), dtype=np.float32) - 1, 4)  # too many positions

"""Host draft-tree builder of the library (gdn_ddtree_build) against the oracle
(oracle/ddtree.py): bit-exact trees and fp32 scores on random drafts, including exact score
ties, every pruning margin, both seeds; batched calls; error codes.  No GPU needed."""
import math

import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth
from oracle import ddtree as od


def _draft(rng, L, K, quantum=None):
    x = rng.normal(0.0, 2.0, size=(L, max(K, 8)))
    lp = x - np.log(np.exp(x).sum(axis=1, keepdims=True))
    lp = -np.sort(-lp, axis=1)[:, :K]
    if quantum:
        lp = np.minimum(-np.round(-lp / quantum) * quantum, 0.0)
        lp = -np.sort(-lp, axis=1)
    return lp.astype(np.float32)


@pytest.mark.parametrize("seed", range(60))
def test_matches_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    L, K = int(rng.integers(0, 17)), int(rng.integers(1, 9))
    lp = _draft(rng, L, K, quantum=[None, 0.5, 0.125][seed % 3])
    budget = int(rng.integers(1, 64))
    tau = [0.0, 0.7, 3.0, 6.0, math.inf][seed % 5]
    for chain in (True, False):
        want = od.build(lp, budget, tau, chain)
        got = binding.ddtree_build(lp, budget=budget, tau=tau, chain_seed=chain)
        for key in ("parent", "depth", "rank", "score"):
            assert np.array_equal(got[key], want[key]), (seed, chain, key)


def test_batch_and_tokens():
    rng = np.random.default_rng(5)
    B, L, K = 32, 15, 4
    lp = np.stack([_draft(rng, L, K) for _ in range(B)])
    tok = rng.integers(0, 50000, size=(B, L, K)).astype(np.int32)
    roots = rng.integers(0, 50000, size=B).astype(np.int32)
    trees = binding.ddtree_build(lp, tok, roots, budget=22, tau=6.0)
    for b in range(B):
        want = od.build(lp[b], 22, 6.0, True)
        assert np.array_equal(trees[b]["parent"], want["parent"])
        assert np.array_equal(trees[b]["token"], od.tokens_of(want, tok[b], roots[b]))
    # the trees feed the schedule directly
    image = binding.hld_schedule([t["parent"] for t in trees])
    assert int(image[2]) == sum(len(t["parent"]) for t in trees)


def test_chain_mode():
    lp = _draft(np.random.default_rng(3), 15, 1)
    t = binding.ddtree_build(lp, budget=16, tau=math.inf)
    assert t["parent"].tolist() == list(range(-1, 15))


def test_errors():
    L = binding.lib()
    good = np.full((1, 2, 2), -1.0, dtype=np.float32)
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(good, budget=0)
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(good, tau=-1.0)
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(np.array([[[0.5, -1.0]]], dtype=np.float32))
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(np.array([[[-1.0, -0.5]]], dtype=np.float32))
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(np.full((1, 17, 2), -1.0, dtype=np.float32))
    with pytest.raises(binding.GdnError):
        binding.ddtree_build(np.full((1, 2, 17), -1.0, dtype=np.float32))
    with pytest.raises(binding.GdnError) as e:
        binding.ddtree_build(np.array([[[np.nan, -1.0]]], dtype=np.float32))
    assert e.value.status == -1
    assert L is not None

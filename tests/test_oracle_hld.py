"""Pins of the heavy-light schedule oracle: hand-worked examples, structural properties and
agreement of two independent formulations over every small tree and many random ones."""
import glob
import itertools
import json
import os

import numpy as np
import pytest

from gated_deltanet_tree_amd import synth
from oracle import hld

KEYS = ["seq_offsets", "wave_offsets", "chain_offsets", "chain_nodes", "chain_seq",
        "chain_src", "node_store", "node_parent", "node_depth"]
COUNTS = ["n_chains", "n_waves", "n_boundaries", "max_chain_len"]


def _golden(golden_dir):
    return sorted(glob.glob(os.path.join(golden_dir, "hld_*.json")))


def _same(a, b):
    for key in KEYS:
        assert np.array_equal(a[key], b[key]), key
    for key in COUNTS + ["n_seqs", "n_nodes"]:
        assert a[key] == b[key], key


def test_golden_examples(golden_dir):
    files = _golden(golden_dir)
    assert len(files) >= 5
    for f in files:
        case = json.load(open(f))
        for fn in (hld.schedule, hld.schedule_recursive):
            s = fn([np.array(p) for p in case["parents"]])
            for key, val in case["expected"].items():
                got = s[key]
                if isinstance(val, list):
                    assert np.array_equal(got, np.array(val)), (f, key, got)
                else:
                    assert got == val, (f, key, got)


def check_properties(parents, s):
    """Structural invariants of a heavy-light schedule."""
    offsets = s["seq_offsets"]
    total = int(offsets[-1])
    nodes = s["chain_nodes"]
    assert sorted(nodes.tolist()) == list(range(total))  # chains partition the nodes
    par = s["node_parent"]
    size = np.ones(total, dtype=int)
    for n in range(total - 1, -1, -1):
        if par[n] >= 0:
            size[par[n]] += size[n]
    heavy = {}
    for n in range(total):
        kids = [c for c in range(total) if par[c] == n]
        if kids:
            best = max(size[c] for c in kids)
            heavy[n] = min(c for c in kids if size[c] == best)
    wave_of_node = {}
    for w in range(s["n_waves"]):
        for c in range(s["wave_offsets"][w], s["wave_offsets"][w + 1]):
            ch = nodes[s["chain_offsets"][c]:s["chain_offsets"][c + 1]]
            head = ch[0]
            b = s["chain_seq"][c]
            assert offsets[b] <= head < offsets[b + 1]
            for a, bnode in zip(ch, ch[1:]):
                assert par[bnode] == a and heavy[a] == bnode  # heavy edges inside chains
            assert ch[-1] not in heavy  # chains end at leaves
            if par[head] < 0:
                assert w == 0 and s["chain_src"][c] == -1
            else:
                assert heavy[par[head]] != head  # light head
                assert w == wave_of_node[par[head]] + 1
                assert s["chain_src"][c] == s["node_store"][par[head]] >= 0
            for n in ch:
                wave_of_node[n] = w
    n_leaves = sum(1 for n in range(total) if n not in heavy)
    assert s["n_chains"] == n_leaves
    assert s["n_boundaries"] <= s["n_chains"] - len(parents)
    n_max = max(len(p) for p in parents)
    assert s["n_waves"] <= int(np.floor(np.log2(n_max))) + 1  # a light edge halves the subtree
    slots = s["node_store"][s["node_store"] >= 0]
    assert np.array_equal(slots, np.arange(s["n_boundaries"]))  # ascending global id order


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7])
def test_all_small_trees_two_formulations(N):
    count = 0
    for choice in itertools.product(*[range(i) for i in range(1, N)]):
        parent = np.array((-1,) + choice)
        a = hld.schedule([parent])
        b = hld.schedule_recursive([parent])
        _same(a, b)
        check_properties([parent], a)
        count += 1
    assert count == [1, 1, 2, 6, 24, 120, 720][N - 1]


def test_random_batches_two_formulations():
    rng = np.random.default_rng(99)
    for trial in range(300):
        n_seqs = int(rng.integers(1, 5))
        parents = []
        for _ in range(n_seqs):
            N = int(rng.integers(1, 65))
            K = int(rng.integers(1, 9))
            D = int(rng.integers(1, 17))
            try:
                parents.append(synth.make_tree(rng, N, K, D))
            except ValueError:
                parents.append(np.arange(-1, N - 1))
        a = hld.schedule(parents)
        b = hld.schedule_recursive(parents)
        _same(a, b)
        check_properties(parents, a)

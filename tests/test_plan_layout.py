"""Properties of the tree-masked verify plan's layout (tests/plan_layout.py): every record
block is the node's root path upward, nodes are ordered by (depth, id), levels are contiguous
and blocks are laid out back to back in level order."""
import numpy as np

from gated_deltanet_tree_amd import synth

import plan_layout


def test_ut_plan_records_are_root_paths_by_level():
    rng = np.random.default_rng(77)
    trees = [np.array([-1, 0, 0, 1, 1, 2, 3]), np.arange(-1, 7), np.array([-1]),
             synth.make_tree(rng, 22, 4, 12), synth.make_tree(rng, 40, 8, 16)]
    plan = plan_layout.ut_plan(trees)
    for b, parent in enumerate(trees):
        n = len(parent)
        depth = synth.node_depths(parent)
        r0, r1 = plan["rec_base"][b], plan["rec_base"][b + 1]
        recs = plan["rec_anc"][r0:r1]
        assert r1 - r0 == int(np.sum(depth + 1))
        off = sum(len(t) for t in trees[:b])
        poff = plan["node_rec"][off:off + n]
        for t in range(n):  # block = t, then its root path upward
            block = recs[poff[t]:poff[t] + depth[t] + 1]
            assert block.tolist() == list(reversed(synth.root_path(parent, t)))
        order = plan["lvnode"][off:off + n]
        assert sorted(order.tolist()) == list(range(n))
        keys = [(depth[t], t) for t in order]
        assert keys == sorted(keys)
        lvn = plan["lvn"][plan["lv_base"][b]:plan["lv_base"][b + 1]]
        assert len(lvn) == depth.max() + 2 and lvn[0] == 0 and lvn[-1] == n
        for d in range(depth.max() + 1):  # level d = positions lvn[d] .. lvn[d+1]
            assert all(depth[t] == d for t in order[lvn[d]:lvn[d + 1]])
        # blocks laid out in level order, back to back
        assert [poff[t] for t in order] == np.concatenate(
            [[0], np.cumsum([depth[t] + 1 for t in order])[:-1]]).tolist()

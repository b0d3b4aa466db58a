"""Layout checker of the tree-masked verify plan in the schedule image (test infrastructure).

The plan is device bookkeeping, not part of the method: it lists, per tree, the nodes by depth
level and each node's block of records (the node, then its ancestors nearest first), which the
UT and fused verify kernels walk.  `ut_plan` builds the same arrays by plain construction so
that tests can check the library's image against it bit for bit.
"""
from __future__ import annotations

import numpy as np


def ut_plan(parents):
    """Tree structure the tree-masked (UT) verify kernels read from the schedule image, for a
    batch of trees (each node's output sums over its ancestors, and a node's residual needs
    all its ancestors' first).  Plain construction, per tree:
      * nodes ordered by (depth, local id): `lvnode`, with `lvn[d]` the first position of
        depth level d (dmax + 2 entries);
      * one block of depth + 1 records per node, blocks in that order: the node itself, then
        its ancestors nearest first (`rec_anc`, local ids); `node_rec[t]` = first record of
        node t's block, relative to the tree's first record;
      * `rec_base[b]` (global first record of tree b) and `lv_base[b]` (first entry of tree b
        in the concatenated `lvn`).
    Returns a dict of int32 arrays, concatenated over the batch."""
    rec_base, node_rec, lv_base, lvn, lvnode, rec_anc = [0], [], [0], [], [], []
    for parent in parents:
        parent = np.asarray(parent, dtype=np.int64)
        assert parent[0] == -1 and all(0 <= parent[i] < i for i in range(1, len(parent)))
        n = len(parent)
        depth = [0] * n
        for t in range(1, n):
            depth[t] = depth[parent[t]] + 1
        order = sorted(range(n), key=lambda t: (depth[t], t))
        dmax = max(depth)
        first = [0] * (dmax + 2)
        for t in order:
            first[depth[t] + 1] += 1
        for d in range(dmax + 1):
            first[d + 1] += first[d]
        poff = [0] * n
        recs = []
        for t in order:
            poff[t] = len(recs)
            a = t
            while a >= 0:  # t itself, then its ancestors nearest first
                recs.append(a)
                a = int(parent[a])
        node_rec += poff
        lvnode += order
        lvn += first
        rec_anc += recs
        rec_base.append(rec_base[-1] + len(recs))
        lv_base.append(lv_base[-1] + len(first))
    as32 = lambda x: np.asarray(x, dtype=np.int32)  # noqa: E731
    return dict(rec_base=as32(rec_base), node_rec=as32(node_rec), lv_base=as32(lv_base),
                lvn=as32(lvn), lvnode=as32(lvnode), rec_anc=as32(rec_anc))

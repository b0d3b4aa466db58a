"""Heavy-light chain schedule of a batch of candidate trees (integer, deterministic).

SpecLA guide, mechanism 2 (chain decomposition and dependency waves): a speculative tree
cannot stay resident as a whole, so it is cut into chains by heavy-light decomposition. The
child with the largest subtree is a node's heavy continuation and stays in the node's chain;
every other (light) child starts a new chain.  Only states at chain boundaries are
materialised.  Chains are grouped into waves by dependency and all chains of one wave run
in parallel.  The scheduler is a deterministic, testable host function whose compact output
is fed to the device kernels.

Readings fixed here (the pages leave them open):
  * heavy child: largest subtree, ties to the smallest node index;
  * chain = heavy path from the root or from a light child, nodes root-to-leaf;
  * wave(root chain) = 0; wave(c) = wave(chain holding parent(head c)) + 1;
  * boundary node = a node with at least one light child; its state is stored once and
    every light chain hanging off it starts from it; slots are numbered by ascending global
    node id (global id = seq_offsets[b] + local id);
  * chains ordered by (wave, seq, global head id); waves merged across the batch;
  * chain_src = -1 for root chains (start from the committed state), else the slot of the
    head's parent; node_store = slot of the node or -1; node_depth with root = 0.

Output: dict of int32 arrays seq_offsets, wave_offsets, chain_offsets, chain_nodes,
chain_seq, chain_src, node_store, node_parent, node_depth (global ids), plus counts.
"""
from __future__ import annotations

import sys

import numpy as np

from .gdn import check_tree


def _subtree_sizes(parent):
    size = np.ones(len(parent), dtype=np.int64)
    for i in range(len(parent) - 1, 0, -1):
        size[parent[i]] += size[i]
    return size


def _heavy(parent, size):
    heavy = np.full(len(parent), -1, dtype=np.int64)
    for i in range(1, len(parent)):  # increasing index: a strictly larger size wins
        p = parent[i]
        if heavy[p] < 0 or size[i] > size[heavy[p]]:
            heavy[p] = i
    return heavy


def _assemble(chains, n_nodes_per_seq, parents):
    """chains: list of (wave, seq, head_global, [global nodes]) -> schedule dict."""
    seq_offsets = np.concatenate([[0], np.cumsum(n_nodes_per_seq)]).astype(np.int32)
    total = int(seq_offsets[-1])
    node_parent = np.full(total, -1, dtype=np.int32)
    node_depth = np.zeros(total, dtype=np.int32)
    for b, par in enumerate(parents):
        off = seq_offsets[b]
        for i in range(1, len(par)):
            node_parent[off + i] = off + par[i]
            node_depth[off + i] = node_depth[off + par[i]] + 1
    chains = sorted(chains, key=lambda c: (c[0], c[1], c[2]))
    light_parents = sorted({int(node_parent[c[2]]) for c in chains if node_parent[c[2]] >= 0})
    slot = {n: s for s, n in enumerate(light_parents)}
    node_store = np.full(total, -1, dtype=np.int32)
    for n, s in slot.items():
        node_store[n] = s
    n_waves = (max(c[0] for c in chains) + 1) if chains else 0
    wave_offsets = np.zeros(n_waves + 1, dtype=np.int32)
    for c in chains:
        wave_offsets[c[0] + 1] += 1
    wave_offsets = np.cumsum(wave_offsets).astype(np.int32)
    chain_offsets = np.concatenate([[0], np.cumsum([len(c[3]) for c in chains])]).astype(np.int32)
    chain_nodes = np.array([n for c in chains for n in c[3]], dtype=np.int32)
    chain_seq = np.array([c[1] for c in chains], dtype=np.int32)
    chain_src = np.array([-1 if node_parent[c[2]] < 0 else slot[int(node_parent[c[2]])]
                          for c in chains], dtype=np.int32)
    return dict(
        n_seqs=len(parents), n_nodes=total, n_chains=len(chains), n_waves=n_waves,
        n_boundaries=len(light_parents),
        max_chain_len=max((len(c[3]) for c in chains), default=0),
        seq_offsets=seq_offsets, wave_offsets=wave_offsets, chain_offsets=chain_offsets,
        chain_nodes=chain_nodes, chain_seq=chain_seq, chain_src=chain_src,
        node_store=node_store, node_parent=node_parent, node_depth=node_depth,
    )


def schedule(parents):
    """Iterative formulation. `parents`: list of parent arrays, one tree per sequence."""
    parents = [check_tree(p) for p in parents]
    chains = []
    offset = 0
    for b, par in enumerate(parents):
        size = _subtree_sizes(par)
        heavy = _heavy(par, size)
        chain_of = np.full(len(par), -1, dtype=np.int64)
        wave_of_chain = {}
        for head in range(len(par)):
            if head > 0 and heavy[par[head]] == head:
                continue  # continues its parent's chain
            wave = 0 if head == 0 else wave_of_chain[chain_of[par[head]]] + 1
            wave_of_chain[head] = wave
            nodes, n = [], head
            while n >= 0:
                chain_of[n] = head
                nodes.append(offset + n)
                n = heavy[n]
            chains.append((wave, b, offset + head, nodes))
        offset += len(par)
    return _assemble(chains, [len(p) for p in parents], parents)


def schedule_recursive(parents):
    """Second formulation: recursive sizes and a recursive descent that peels heavy paths."""
    parents = [check_tree(p) for p in parents]
    sys.setrecursionlimit(max(10000, sys.getrecursionlimit()))
    chains = []
    offset = 0
    for b, par in enumerate(parents):
        children = [[] for _ in par]
        for i in range(1, len(par)):
            children[par[i]].append(i)

        def size_of(n):
            return 1 + sum(size_of(c) for c in children[n])

        sizes = {n: size_of(n) for n in range(len(par))}

        def heavy_of(n):
            if not children[n]:
                return None
            best = max(sizes[c] for c in children[n])
            return min(c for c in children[n] if sizes[c] == best)

        def descend(head, wave):
            path, n = [], head
            while n is not None:
                path.append(n)
                n = heavy_of(n)
            chains.append((wave, b, offset + head, [offset + m for m in path]))
            for m in path:
                for c in children[m]:
                    if c != heavy_of(m):
                        descend(c, wave + 1)

        descend(0, 0)
        offset += len(par)
    return _assemble(chains, [len(p) for p in parents], parents)

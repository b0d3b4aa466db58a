"""Seeded synthetic workloads for draft-tree verification through Gated DeltaNet layers.

This module only draws numbers: candidate trees, per-node inputs, committed states, conv
windows and weights, and accepted paths. It contains none of the recurrence, the conv, the
schedule or the commit arithmetic, so both the HIP path and the CPU oracle can take their
inputs from here without sharing any of the method.

Workload shape (stand-in for the draft trees described on the "Luce DFlash server README",
section "How it works", DDTree tree verify; and the defaults of budget 22 / top-k 4 in the
"Lucebox SpecLA and Gated DeltaNet state-resident verification guide", section on enabling
SpecLA): best-first trees of up to 22 nodes with at most K children per node, grown from a
main chain (the chain pre-seed), labelled so that every parent index is lower than its child's.

Every stream is a PCG64 generator seeded by
``SeedSequence([20261202, seed, step, layer, seq, stream])``, where ``seed`` is the workload
preset's number (or a test's own number).
bf16 values are produced by round-to-nearest-even from the float32 draws and are kept as
raw ``uint16`` bit patterns; ``bf16_to_f32`` widens them exactly.
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 20261202
STREAMS = {
    "tree": 0, "q": 1, "k": 2, "v": 3, "beta": 4, "gate": 5, "state": 6,
    "x": 7, "weight": 8, "conv_state": 9, "path": 10, "draft": 11,
}

# Workload presets, by name.  d = head dim (d_k = d_v), H = heads, N = nodes per tree, K = top-k,
# D = max edge depth, Bs = sequences, Ly = GDN layers, Kc = conv width, Cch = conv channels;
# seed = the preset's number in every seed sequence below.
WORKLOADS = {
    "tiny": dict(seed=0, H=1, d=16, N=None, K=None, D=None, Bs=1, Ly=1, Kc=4, Cch=16,
                 dtype="f32"),
    "one-layer": dict(seed=1, H=48, d=128, N=22, K=4, D=12, Bs=1, Ly=1, Kc=4,
                      Cch=3 * 48 * 128, dtype="bf16", accept_len=6),
    "48-layer": dict(seed=2, H=48, d=128, N=22, K=4, D=12, Bs=1, Ly=48, Kc=4,
                     Cch=3 * 48 * 128, dtype="bf16", steps=10, accept_len=6),
    "batched": dict(seed=3, H=48, d=128, N=22, K=4, D=12, Bs=32, Ly=48, Kc=4,
                    Cch=3 * 48 * 128, dtype="bf16", accept_max=9),
    "wide-deep": dict(seed=4, H=48, d=128, N=64, K=8, D=16, Bs=8, Ly=48, Kc=4,
                      Cch=3 * 48 * 128, dtype="bf16"),
    "chain16": dict(seed=5, H=48, d=128, N=16, K=1, D=15, Bs=8, Ly=48, Kc=4,
                    Cch=3 * 48 * 128, dtype="bf16"),
}

TINY_TREE = np.array([-1, 0, 0, 1, 1, 2, 3], dtype=np.int32)
TINY_CHAIN = np.arange(-1, 7, dtype=np.int32)


def rng_for(seed: int, step: int, layer: int, seq: int, stream: str) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, seed, step, layer, seq, STREAMS[stream]])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------------
# trees and paths
# ----------------------------------------------------------------------------------------

def make_tree(rng: np.random.Generator, n_nodes: int, top_k: int, max_depth: int) -> np.ndarray:
    """Random candidate tree as a parent array.

    A main chain of min(N, D+1) nodes is laid down first; every further node hangs off a
    uniformly chosen existing node that is shallower than D and has fewer than K children.
    The result is relabelled in DFS preorder, children visited in creation order, so every
    parent index is lower than its child's and the main chain is 0, 1, 2, ...
    """
    main = min(n_nodes, max_depth + 1)
    parent = [-1] + list(range(main - 1))
    depth = list(range(main))
    children: list[list[int]] = [[] for _ in range(n_nodes)]
    for i in range(1, main):
        children[i - 1].append(i)
    for i in range(main, n_nodes):
        cands = [j for j in range(i) if depth[j] < max_depth and len(children[j]) < top_k]
        if not cands:
            raise ValueError("tree parameters admit no further node")
        p = cands[int(rng.integers(len(cands)))]
        parent.append(p)
        depth.append(depth[p] + 1)
        children[p].append(i)
    order, stack = [], [0]
    while stack:
        n = stack.pop()
        order.append(n)
        stack.extend(reversed(children[n]))
    new_id = {old: i for i, old in enumerate(order)}
    out = np.full(n_nodes, -1, dtype=np.int32)
    for old in order[1:]:
        out[new_id[old]] = new_id[parent[old]]
    return out


def node_depths(parent: np.ndarray) -> np.ndarray:
    depth = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    return depth


def root_path(parent: np.ndarray, node: int) -> np.ndarray:
    path = []
    while node >= 0:
        path.append(node)
        node = int(parent[node])
    return np.array(path[::-1], dtype=np.int32)


def deepest_leaf_path(parent: np.ndarray) -> np.ndarray:
    depth = node_depths(parent)
    return root_path(parent, int(np.argmax(depth)))  # argmax: smallest index among ties


def random_path(rng: np.random.Generator, parent: np.ndarray, length: int) -> np.ndarray:
    """Uniformly chosen root path of `length` nodes (root included); length 0 = empty."""
    if length == 0:
        return np.zeros(0, dtype=np.int32)
    depth = node_depths(parent)
    cands = np.flatnonzero(depth == length - 1)
    if len(cands) == 0:
        raise ValueError("no node at depth %d" % (length - 1))
    return root_path(parent, int(cands[int(rng.integers(len(cands)))]))


def workload_tree(name: str, seq: int) -> np.ndarray:
    """Candidate tree of sequence `seq` of a preset (the 48-layer stack reuses the one-layer
    workload's tree)."""
    c = WORKLOADS[name]
    if name == "tiny":
        return TINY_TREE.copy() if seq == 0 else TINY_CHAIN.copy()
    tree_seed = WORKLOADS["one-layer"]["seed"] if name == "48-layer" else c["seed"]
    return make_tree(rng_for(tree_seed, 0, 0, seq, "tree"), c["N"], c["K"], c["D"])


def workload_path(name: str, step: int, seq: int, parent: np.ndarray) -> np.ndarray:
    """Accepted root path for (preset, step, seq): the deepest leaf for the tiny cases, a fixed
    length for the one-layer and 48-layer presets, a uniform length otherwise."""
    c = WORKLOADS[name]
    if name == "tiny":
        return deepest_leaf_path(parent)
    rng = rng_for(c["seed"], step, 0, seq, "path")
    if "accept_len" in c:
        length = c["accept_len"]
    elif "accept_max" in c:
        length = int(rng.integers(1, c["accept_max"] + 1))
    else:
        length = int(rng.integers(1, int(node_depths(parent).max()) + 2))
    return random_path(rng, parent, length)


def draft_scores(seed: int, step: int, seq: int, positions: int, top_k: int,
                 vocab: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic draft of one sequence: for each of `positions` tokens after the root, the
    top-k candidates (ids, fp32 log-probabilities sorted descending) of a softmax over `vocab`
    logits ~ N(0, s^2), with s falling from 4 to 1.5 along the block (later positions are less
    certain).  Returns (logp [positions][top_k], tokens [positions][top_k])."""
    rng = rng_for(seed, step, 0, seq, "draft")
    scale = np.linspace(4.0, 1.5, max(positions, 1))[:positions, None]
    logits = rng.normal(size=(positions, vocab)) * scale
    logp = logits - np.log(np.exp(logits - logits.max(axis=1, keepdims=True)).sum(
        axis=1, keepdims=True)) - logits.max(axis=1, keepdims=True)
    order = np.argsort(-logp, axis=1, kind="stable")[:, :top_k]
    lp = np.take_along_axis(logp, order, axis=1).astype(np.float32)
    return np.minimum(lp, np.float32(0.0)), order.astype(np.int32)


# ----------------------------------------------------------------------------------------
# per-(layer, seq) values
# ----------------------------------------------------------------------------------------

def _normal(rng, shape, scale=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _unit_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _exp_neg_softplus(x):
    return np.exp(-np.logaddexp(0.0, x.astype(np.float64))).astype(np.float32)


def _cast(x, dtype):
    return f32_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def node_inputs(seed: int, step: int, layer: int, seq: int, n_nodes: int, heads: int,
                d: int, dtype: str) -> dict:
    """q, k, v [N,H,d]; beta, gate [N,H] in `dtype` (uint16 bits for bf16).

    q and k are unit-norm per (node, head) before rounding; beta = sigmoid(z);
    gate = exp(-softplus(z)), so gate lies in (0, 1).
    """
    sh = (n_nodes, heads, d)
    out = {
        "q": _unit_rows(_normal(rng_for(seed, step, layer, seq, "q"), sh)),
        "k": _unit_rows(_normal(rng_for(seed, step, layer, seq, "k"), sh)),
        "v": _normal(rng_for(seed, step, layer, seq, "v"), sh),
        "beta": _sigmoid(_normal(rng_for(seed, step, layer, seq, "beta"), sh[:2])),
        "gate": _exp_neg_softplus(_normal(rng_for(seed, step, layer, seq, "gate"), sh[:2])),
    }
    return {key: _cast(val, dtype) for key, val in out.items()}


def initial_state(seed: int, layer: int, seq: int, heads: int, d: int) -> np.ndarray:
    """Committed recurrent state [H, d_v, d_k], float32, N(0, 0.02^2)."""
    return _normal(rng_for(seed, 0, layer, seq, "state"), (heads, d, d), 0.02)


def conv_inputs(seed: int, step: int, layer: int, seq: int, n_nodes: int, channels: int,
                dtype: str) -> np.ndarray:
    """Raw (pre-conv) per-node channel inputs [N, Cch] in `dtype`."""
    return _cast(_normal(rng_for(seed, step, layer, seq, "x"), (n_nodes, channels)), dtype)


def conv_weight(seed: int, layer: int, channels: int, width: int, dtype: str) -> np.ndarray:
    """Depthwise conv weight [Cch, Kc]; column Kc-1 multiplies the current token."""
    return _cast(_normal(rng_for(seed, 0, layer, 0, "weight"), (channels, width), 0.5), dtype)


def initial_conv_state(seed: int, layer: int, seq: int, channels: int, width: int) -> np.ndarray:
    """Committed conv window [Cch, Kc-1], float32, oldest input first."""
    return _normal(rng_for(seed, 0, layer, seq, "conv_state"), (channels, width - 1))

"""Best-first draft-tree builder with a budget cap, confidence pruning and a chain pre-seed.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline use it.

Pages:
  * "Luce DFlash server README", How it works: DDTree verifies a best-first tree of up to 22
    nodes that spans the top-K branches at each draft position, one target forward for the
    whole tree through parent pointers; chain pre-seed (chain_seed) matters.
  * "Lucebox SpecLA and Gated DeltaNet state-resident verification" guide, "enable with one
    flag": budget 22, tau 6, top-k 4; tau is a confidence margin, nodes scoring below
    q* - tau are pruned; "how correctness is guaranteed": CPU tests cover cumulative-score
    pruning, ancestor closure and the budget cap.

Readings fixed here (the pages leave them open):
  * the draft gives, for each of L positions after the root, K candidates sorted by
    log-probability, logp[i][0] >= logp[i][1] >= ... (candidate 0 is the greedy token), all
    <= 0; a node at depth d takes candidate k of position d (0-based: row d - 1); its
    children are the K candidates of the next position;
  * score(root) = 0, score(node) = score(parent) + logp, summed in fp32 along the path;
  * q*(d) = the best score at depth d, which is the greedy chain's (every term of it is the
    largest of its position, and fp32 addition is monotone); a node scoring below
    q*(d) - tau (in fp32) is pruned together with its subtree; tau = inf prunes nothing;
  * the budget counts the root;
  * with the chain pre-seed the greedy chain is placed first, depths 1 .. min(L, budget - 1);
  * the other slots go best-first: highest score first, ties to the shallower node, then to
    the lexicographically smaller sequence of candidate ranks along the path;
  * node ids are insertion order, so parent[i] < i.

Two implementations that share nothing: `build` follows the construction as the pages
describe it (a frontier of candidate children, best one taken each time), `enumerate_tree`
scores every path of a small draft and sorts them.  They must agree exactly.
"""
from __future__ import annotations

import heapq
import itertools
import math

import numpy as np

MAX_POSITIONS = 16  # depth limit of the tie-break key (4 bits of rank per position)
MAX_TOP_K = 16


def check_draft(logp, budget, tau):
    logp = np.asarray(logp, dtype=np.float32)
    if logp.ndim != 2:
        raise ValueError("logp must be [L][K]")
    L, K = logp.shape
    if L > MAX_POSITIONS or K < 1 or K > MAX_TOP_K or budget < 1:
        raise ValueError("unsupported draft shape or budget")
    if not np.all(np.isfinite(logp)) or np.any(logp > 0):
        raise ValueError("log-probabilities must be finite and <= 0")
    if np.any(np.diff(logp, axis=1) > 0):
        raise ValueError("candidates of a position must be sorted by log-probability")
    if not (tau >= 0):
        raise ValueError("tau must be >= 0 (inf: no pruning)")
    return logp


def _f32(x):
    return np.float32(x)


def greedy_scores(logp):
    """q*(d) for d = 0..L: fp32 running sum of the greedy candidates."""
    q = [_f32(0.0)]
    for i in range(logp.shape[0]):
        q.append(_f32(q[-1] + logp[i, 0]))
    return q


def _threshold(q, tau):
    return [_f32(x - _f32(tau)) if math.isfinite(tau) else -np.inf for x in q]


def build(logp, budget, tau=math.inf, chain_seed=True):
    """Best-first construction.  Returns dict of parent, depth, rank (candidate index), score
    (fp32) per node, in insertion order; the root has parent -1, rank -1."""
    logp = check_draft(logp, budget, tau)
    L, K = logp.shape
    q = greedy_scores(logp)
    thr = _threshold(q, tau)
    parent, depth, rank, score, ranks = [-1], [0], [-1], [_f32(0.0)], [()]
    if chain_seed:
        for d in range(1, min(L, budget - 1) + 1):
            parent.append(len(parent) - 1)
            depth.append(d)
            rank.append(0)
            score.append(q[d])
            ranks.append(ranks[-1] + (0,))
    in_tree = set(ranks)
    frontier = []  # (-score, depth, rank sequence, parent id)

    def push_children(node):
        d = depth[node]
        if d >= L:
            return
        for k in range(K):
            child = ranks[node] + (k,)
            if child in in_tree:
                continue
            s = _f32(score[node] + logp[d, k])
            heapq.heappush(frontier, (-float(s), d + 1, child, node))

    for node in range(len(parent)):
        push_children(node)
    while len(parent) < budget and frontier:
        neg_s, d, child, par = heapq.heappop(frontier)
        s = _f32(-neg_s)
        if s < thr[d]:
            continue  # pruned: its children are never generated
        parent.append(par)
        depth.append(d)
        rank.append(child[-1])
        score.append(s)
        ranks.append(child)
        in_tree.add(child)
        push_children(len(parent) - 1)
    return dict(parent=np.array(parent, dtype=np.int32), depth=np.array(depth, dtype=np.int32),
                rank=np.array(rank, dtype=np.int32), score=np.array(score, dtype=np.float32))


def enumerate_tree(logp, budget, tau=math.inf, chain_seed=True):
    """Brute force for small drafts: score every path, keep the paths none of whose prefixes
    is pruned, take the greedy chain first (with the pre-seed) and then the best of the rest
    by the tie-break order.  Same output format as `build`."""
    logp = check_draft(logp, budget, tau)
    L, K = logp.shape
    q = greedy_scores(logp)
    thr = _threshold(q, tau)
    ok = {(): True}
    sc = {(): _f32(0.0)}
    paths = []
    for d in range(1, L + 1):
        for path in itertools.product(range(K), repeat=d):
            s = _f32(sc[path[:-1]] + logp[d - 1, path[-1]])
            sc[path] = s
            ok[path] = ok[path[:-1]] and not (s < thr[d])
            if ok[path]:
                paths.append(path)
    chain = [tuple([0] * d) for d in range(1, min(L, budget - 1) + 1)] if chain_seed else []
    rest = sorted((p for p in paths if p not in set(chain)),
                  key=lambda p: (-float(sc[p]), len(p), p))
    chosen = [()] + chain + rest[:max(0, budget - 1 - len(chain))]
    index = {p: i for i, p in enumerate(chosen)}
    return dict(parent=np.array([-1] + [index[p[:-1]] for p in chosen[1:]], dtype=np.int32),
                depth=np.array([len(p) for p in chosen], dtype=np.int32),
                rank=np.array([-1] + [p[-1] for p in chosen[1:]], dtype=np.int32),
                score=np.array([sc[p] for p in chosen], dtype=np.float32))


def tokens_of(tree, tok, root_token):
    """Token id of every node: the root's own, else candidate rank of position depth - 1."""
    tok = np.asarray(tok)
    out = np.empty(len(tree["parent"]), dtype=np.int32)
    out[0] = root_token
    for i in range(1, len(out)):
        out[i] = tok[tree["depth"][i] - 1, tree["rank"][i]]
    return out

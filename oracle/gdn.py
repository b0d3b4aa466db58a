"""Gated delta rule over a parent-indexed candidate tree, float64, by plain definition.

What is computed (SpecLA guide, "Why speculative decoding is harder for linear-attention
models"): a GDN layer keeps a recurrent state matrix S per head that every token advances
with the delta rule, one token after another. Verifying a tree of candidates means that
every node sees the state advanced along its own root-to-node path, starting from the
committed state; siblings see different histories, and a rejected candidate must leave the
committed state exactly as it was. The per-token update is the gated delta rule

    S  <-  g * S (I - beta k k^T) + beta v k^T ,        o = S q

with S of shape [d_v, d_k] (o = S q reads the state with the query). The DFlash README
("How it works", DDTree tree verify) gives the tree as parent pointers with node 0 the root;
chain mode is the same tree with no branching.

Conventions of the arrays (one layer, one sequence):
    parent [N] int, parent[0] == -1, 0 <= parent[i] < i
    S0     [H, d_v, d_k]            committed state
    q, k   [N, H, d_k];  v [N, H, d_v];  beta, gate [N, H]  (gate = g in [0, 1], linear)
All arithmetic is float64; callers pass the exact values the device reads (bf16 widened).
"""
from __future__ import annotations

import numpy as np


def check_tree(parent) -> np.ndarray:
    """Validate a parent array: root first, every parent index below its child's."""
    parent = np.asarray(parent, dtype=np.int64)
    if parent.ndim != 1 or len(parent) == 0 or parent[0] != -1:
        raise ValueError("parent[0] must be -1")
    for i in range(1, len(parent)):
        if not 0 <= parent[i] < i:
            raise ValueError("parent[%d] = %d is not a lower index" % (i, parent[i]))
    return parent


def root_path(parent, node: int) -> list[int]:
    """Nodes from the root down to `node`, inclusive."""
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parent[node])
    return path[::-1]


def gdn_step(S, k, v, beta, gate):
    """One token of the gated delta rule for all heads.

    S [H, dv, dk]; k [H, dk]; v [H, dv]; beta, gate [H].
    S (I - beta k k^T) is evaluated as S - beta (S k) k^T.
    """
    Sk = np.einsum("hij,hj->hi", S, k)
    b = beta[:, None, None]
    return gate[:, None, None] * (S - b * Sk[:, :, None] * k[:, None, :]) \
        + b * v[:, :, None] * k[:, None, :]


def gdn_step_matrix(S, k, v, beta, gate):
    """The same token update with the literal d x d product S @ (I - beta k k^T)."""
    H, dv, dk = S.shape
    out = np.empty_like(S)
    for h in range(H):
        proj = np.eye(dk) - beta[h] * np.outer(k[h], k[h])
        out[h] = gate[h] * (S[h] @ proj) + beta[h] * np.outer(v[h], k[h])
    return out


def _as64(*arrays):
    return [np.asarray(a, dtype=np.float64) for a in arrays]


def verify(parent, S0, q, k, v, beta, gate, step=gdn_step, keep_states=True):
    """Per-node outputs o [N,H,dv] and post-states [N,H,dv,dk].

    Each node's state is obtained by replaying the update over its own root path from S0
    (literal, deliberately naive: the cost is the sum of path lengths).
    """
    parent = check_tree(parent)
    S0, q, k, v, beta, gate = _as64(S0, q, k, v, beta, gate)
    N, H, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv))
    states = np.zeros((N, H, dv, dk)) if keep_states else None
    for n in range(N):
        S = S0.copy()
        for m in root_path(parent, n):
            S = step(S, k[m], v[m], beta[m], gate[m])
        o[n] = np.einsum("hij,hj->hi", S, q[n])
        if keep_states:
            states[n] = S
    return o, states


def verify_dfs(parent, S0, q, k, v, beta, gate):
    """Second formulation: depth-first walk carrying the parent's state on an explicit stack."""
    parent = check_tree(parent)
    S0, q, k, v, beta, gate = _as64(S0, q, k, v, beta, gate)
    N = len(parent)
    children = [[] for _ in range(N)]
    for i in range(1, N):
        children[parent[i]].append(i)
    o = np.zeros((N,) + v.shape[1:])
    states = np.zeros((N,) + S0.shape)
    stack = [(0, S0)]
    while stack:
        node, S_par = stack.pop()
        S = gdn_step(S_par, k[node], v[node], beta[node], gate[node])
        states[node] = S
        o[node] = np.einsum("hij,hj->hi", S, q[node])
        for c in children[node]:
            stack.append((c, S))
    return o, states


def verify_ut(parent, S0, q, k, v, beta, gate):
    """Third formulation: the tree-masked UT closed form (no per-node state is formed).

    With lambda_n = sum of ln g over the root path of n and E[n,j] = exp(lambda_n - lambda_j)
    for ancestors-or-self j of n, unrolling S_n = g_n S_parent + u_n k_n^T gives
        S_n = e^{lambda_n} S0 + sum_j E[n,j] u_j k_j^T
        (I + A) U = diag(beta) (V - diag(e^lambda) K S0^T),  A[n,j] = beta_n E[n,j] k_n.k_j
                                                              for strict ancestors j
        O = diag(e^lambda) Q S0^T + (M * E * Q K^T) U,        M[n,j] = 1 iff j on n's path
    The "topology-mask (UT decomposition)" verify named in the SpecLA guide (mechanism 1) is
    this form; it is derived here from the recurrence.
    Returns (o [N,H,dv], u [N,H,dv]).
    """
    parent = check_tree(parent)
    S0, q, k, v, beta, gate = _as64(S0, q, k, v, beta, gate)
    N, H, _ = k.shape
    lam = np.zeros((N, H))
    mask = np.zeros((N, N))
    for n in range(N):
        path = root_path(parent, n)
        mask[n, path] = 1.0
        lam[n] = np.sum(np.log(gate[path]), axis=0)
    o = np.zeros((N, H, v.shape[2]))
    u = np.zeros_like(o)
    for h in range(H):
        E = np.exp(lam[:, None, h] - lam[None, :, h]) * mask
        strict = mask - np.eye(N)
        A = beta[:, None, h] * E * strict * (k[:, h] @ k[:, h].T)
        rhs = beta[:, None, h] * (v[:, h] - np.exp(lam[:, None, h]) * (k[:, h] @ S0[h].T))
        u[:, h] = np.linalg.solve(np.eye(N) + A, rhs)
        o[:, h] = np.exp(lam[:, None, h]) * (q[:, h] @ S0[h].T) \
            + (E * (q[:, h] @ k[:, h].T)) @ u[:, h]
    return o, u


def factors(parent, S0, k, v, beta, gate, states=None):
    """Accepted-factor rows per node (SpecLA guide, mechanism 3: normalised key, delta-rule
    residual update vector, log decay gate).

    Returns k [N,H,dk], u [N,H,dv] with u_n = beta_n (v_n - g_n S_parent k_n) so that
    S_n = g_n S_parent + u_n k_n^T, and lg [N,H] = ln g_n.  S_parent of the root is S0.
    """
    parent = check_tree(parent)
    S0, k, v, beta, gate = _as64(S0, k, v, beta, gate)
    if states is None:
        dummy_q = np.zeros_like(k)
        _, states = verify(parent, S0, dummy_q, k, v, beta, gate)
    u = np.zeros_like(v)
    for n in range(len(parent)):
        S_par = S0 if parent[n] < 0 else states[parent[n]]
        Sk = np.einsum("hij,hj->hi", S_par, k[n])
        u[n] = beta[n][:, None] * (v[n] - gate[n][:, None] * Sk)
    return k.copy(), u, np.log(gate)


def replay(S0, k, v, beta, gate, path):
    """Committed state after accepting `path`: the update replayed token by token from S0
    (DFlash README, "How it works": after accept the state is that of the committed prefix)."""
    S0, k, v, beta, gate = _as64(S0, k, v, beta, gate)
    S = S0.copy()
    for m in path:
        S = gdn_step(S, k[m], v[m], beta[m], gate[m])
    return S


def prefill(S0, q, k, v, beta, gate, step=gdn_step):
    """Sequential prefill of a token sequence (SpecLA guide, the flush section: after a flush
    the runtime continues without speculation; the GDN layer then runs over plain token
    sequences): for t = 0..T-1, S <- g S (I - beta k k^T) + beta v k^T and o_t = S q_t.
    Returns (o [T,H,dv], S_T).  This is the definition the chunked kernel must reach."""
    S0, q, k, v, beta, gate = _as64(S0, q, k, v, beta, gate)
    S = S0.copy()
    out = np.empty((len(k),) + S.shape[:2])
    for t in range(len(k)):
        S = step(S, k[t], v[t], beta[t], gate[t])
        out[t] = np.einsum("hij,hj->hi", S, q[t])
    return out, S


def fold(S0, kf, uf, lgf):
    """Apply accepted factors in path order: S <- exp(lg) S + u k^T (SpecLA guide, mechanisms
    3 and 4).  kf [L,H,dk], uf [L,H,dv], lgf [L,H].  Used only to pin `factors`."""
    S = np.asarray(S0, dtype=np.float64).copy()
    for i in range(len(lgf)):
        S = np.exp(lgf[i])[:, None, None] * S + uf[i][:, :, None] * kf[i][:, None, :]
    return S

"""Tree-aware short causal depthwise conv, float64, by plain definition.

DFlash README ("How it works", the tree-aware conv state gather kernel): in tree verify each
node's Kc-1 input window is gathered along its parent chain, not along DFS order, so a
sibling never sees a DFS neighbour's input.  SpecLA guide (mechanism 1): the depthwise conv
window uses the same state-resident treatment; (mechanism 3): the conv raw inputs are among
the accepted factors, so the committed window is replayed from them.

Readings taken where the pages are silent: width Kc, depthwise over the channels, no bias,
no activation; W[c, Kc-1] multiplies the current token and W[c, 0] the oldest one; the
committed window X0 [Cch, Kc-1] holds the last Kc-1 committed raw inputs, oldest first, and
continues every root path.

    x  [N, Cch] raw node inputs;  W [Cch, Kc];  X0 [Cch, Kc-1]
"""
from __future__ import annotations

import numpy as np

from .gdn import check_tree, root_path


def tree_conv(parent, X0, x, W):
    """y [N, Cch]: y[n, c] = sum_j W[c, j] * window_n[j, c], window = last Kc entries of
    (X0 columns, then x along the root path of n)."""
    parent = check_tree(parent)
    X0 = np.asarray(X0, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Kc = W.shape[1]
    y = np.zeros(x.shape)
    for n in range(len(parent)):
        history = np.concatenate([X0.T, x[root_path(parent, n)]], axis=0)  # [Kc-1+len, Cch]
        window = history[-Kc:]
        y[n] = np.sum(W.T * window, axis=0)
    return y


def commit_window(X0, x, path):
    """Committed window after accepting `path`: last Kc-1 of (X0 columns, x[path])."""
    X0 = np.asarray(X0, dtype=np.float64)
    history = np.concatenate([X0.T, np.asarray(x, dtype=np.float64)[list(path)]], axis=0)
    return history[history.shape[0] - X0.shape[1]:].T.copy()

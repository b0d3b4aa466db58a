"""Conv -> activation -> normalisation prologue that turns the conv raw inputs into q, k, v,
and the tree verify fed by it, float64, by plain definition.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline use it.

Pages: the SpecLA guide, mechanism 1 and mechanism 3, names the conv raw input as a recurrent
factor next to the normalised key, and the DFlash README ("How it works") rolls the conv
window back together with the recurrent state: the conv output feeds the delta rule's q, k
and v.  The pages do not give the wiring between the two; the reading taken here is the
plainest one those sentences support, the one the Qwen3.5/3.6 hybrid layer uses:

  * the conv runs over 3 H d channels laid out [q heads | k heads | v heads], head-major
    inside each block: channel (blk, h, i) = blk H d + h d + i;
  * every conv output goes through SiLU, silu(y) = y sigmoid(y);
  * q and k of each (node, head) are scaled to unit Euclidean length, the length floored at
    NORM_FLOOR so a zero vector stays zero; v is used as it comes out of the SiLU;
  * beta and g come from their own projections and are inputs, as in the unfused verify.

Arrays (one layer, one sequence): parent [N]; X0 [3Hd, 3] committed conv window; x [N, 3Hd]
raw conv inputs; W [3Hd, 4]; S0 [H, d, d]; beta, gate [N, H].
"""
from __future__ import annotations

import numpy as np

from . import conv, gdn

NORM_FLOOR = 1e-6


def silu(y):
    """y * sigmoid(y), written as y / (1 + exp(-y))."""
    y = np.asarray(y, dtype=np.float64)
    return y / (1.0 + np.exp(-y))


def unit_rows(a, floor=NORM_FLOOR):
    """Each row of a [..., d] divided by max(its Euclidean length, floor)."""
    a = np.asarray(a, dtype=np.float64)
    n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True))
    return a / np.maximum(n, floor)


def split_heads(a, H, d):
    """[N, 3Hd] -> three [N, H, d] blocks (q, k, v)."""
    a = np.asarray(a)
    N = a.shape[0]
    if a.shape[1] != 3 * H * d:
        raise ValueError("expected 3 H d channels")
    return tuple(a[:, b * H * d:(b + 1) * H * d].reshape(N, H, d) for b in range(3))


def qkv_from_conv(parent, X0, x, W, H, d):
    """q, k, v [N, H, d] of every tree node: tree conv along root paths, SiLU, unit q and k."""
    y = conv.tree_conv(parent, X0, x, W)
    q, k, v = split_heads(silu(y), H, d)
    return unit_rows(q), unit_rows(k), v


def conv_verify(parent, S0, X0, x, W, beta, gate, H, d):
    """The fused step on one layer and sequence: q, k, v from the prologue, then the tree
    verify (gdn.verify).  Returns (o [N, H, d], q, k, v)."""
    q, k, v = qkv_from_conv(parent, X0, x, W, H, d)
    o, _ = gdn.verify(parent, S0, q, k, v, beta, gate, keep_states=False)
    return o, q, k, v

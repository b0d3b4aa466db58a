"""Pins of the conv -> SiLU -> unit-norm prologue oracle and of the verify it feeds: closed
forms of SiLU, invariants of the normalisation, the channel layout by construction, library
routines (numpy correlation, scipy's logistic function, numpy's norm) on a chain, and per-path
brute force on trees."""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import conv, gdn, prologue

RNG = np.random.default_rng(4242)
TINY = np.array([-1, 0, 0, 1, 1, 2, 3])
MIXED = np.array([-1, 0, 1, 1, 0, 4, 5, 2, 2, 4])


def test_silu_closed_forms():
    assert prologue.silu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert math.isclose(prologue.silu(math.log(3.0)), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert math.isclose(prologue.silu(-math.log(3.0)), -0.25 * math.log(3.0), rel_tol=1e-15)
    x = RNG.standard_normal(50) * 4
    # y sigmoid(y) - (-y) sigmoid(-y) = y (sigmoid(y) + sigmoid(-y)) = y
    np.testing.assert_allclose(prologue.silu(x) - prologue.silu(-x), x, rtol=1e-14, atol=1e-15)
    assert math.isclose(prologue.silu(40.0), 40.0, rel_tol=1e-15)
    assert abs(prologue.silu(-40.0)) < 1e-15


def test_silu_matches_library_logistic():
    y = RNG.standard_normal(200) * 6
    np.testing.assert_allclose(prologue.silu(y), y * expit(y), rtol=1e-14, atol=1e-300)


def test_unit_rows_invariants():
    a = RNG.standard_normal((7, 3, 16))
    u = prologue.unit_rows(a)
    np.testing.assert_allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(prologue.unit_rows(3.5 * a), u, rtol=1e-14)  # scale invariant
    cos = np.sum(u * a, axis=-1) / np.linalg.norm(a, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-14)  # same direction
    z = np.zeros((2, 8))
    assert np.array_equal(prologue.unit_rows(z), z)  # a zero vector stays zero
    tiny = np.full(4, 1e-9)  # length 2e-9 < floor: divided by the floor
    np.testing.assert_allclose(prologue.unit_rows(tiny), tiny / prologue.NORM_FLOOR, rtol=1e-15)


def test_channel_layout_by_construction():
    H, d, N = 3, 4, 2
    ch = np.tile(np.arange(3 * H * d, dtype=np.float64), (N, 1))
    q, k, v = prologue.split_heads(ch, H, d)
    for h in range(H):
        for i in range(d):
            assert q[1, h, i] == h * d + i
            assert k[1, h, i] == H * d + h * d + i
            assert v[1, h, i] == 2 * H * d + h * d + i
    with pytest.raises(ValueError):
        prologue.split_heads(ch[:, :-1], H, d)


def _layer(N, H, d):
    C = 3 * H * d
    X0 = RNG.standard_normal((C, 3))
    x = RNG.standard_normal((N, C))
    W = RNG.standard_normal((C, 4)) * 0.5
    S0 = RNG.standard_normal((H, d, d)) * 0.02
    beta = expit(RNG.standard_normal((N, H)))
    gate = np.exp(-np.logaddexp(0.0, RNG.standard_normal((N, H))))
    return X0, x, W, S0, beta, gate


def _chain_by_library(X0, x, W, S0, beta, gate, H, d):
    """Chain of tokens: numpy correlation per channel, y expit(y), numpy norms, then the
    sequential recurrence token by token."""
    N, C = x.shape
    y = np.empty((N, C))
    for c in range(C):
        y[:, c] = np.correlate(np.concatenate([X0[c], x[:, c]]), W[c], mode="valid")
    a = y * expit(y)
    q = a[:, :H * d].reshape(N, H, d)
    k = a[:, H * d:2 * H * d].reshape(N, H, d)
    v = a[:, 2 * H * d:].reshape(N, H, d)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    S = S0.copy()
    o = np.empty((N, H, d))
    for t in range(N):
        for h in range(H):
            S[h] = gate[t, h] * (S[h] - beta[t, h] * np.outer(S[h] @ k[t, h], k[t, h])) \
                + beta[t, h] * np.outer(v[t, h], k[t, h])
            o[t, h] = S[h] @ q[t, h]
    return o, q, k, v


def test_chain_equals_library_pipeline():
    H, d, N = 2, 8, 9
    X0, x, W, S0, beta, gate = _layer(N, H, d)
    o, q, k, v = prologue.conv_verify(np.arange(-1, N - 1), S0, X0, x, W, beta, gate, H, d)
    o_ref, q_ref, k_ref, v_ref = _chain_by_library(X0, x, W, S0, beta, gate, H, d)
    for a, b in ((q, q_ref), (k, k_ref), (v, v_ref), (o, o_ref)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("parent", [TINY, MIXED])
def test_every_node_equals_its_root_path_as_a_chain(parent):
    """Brute force: node n's q, k, v and output are those of the last token of the chain made
    of n's root path."""
    H, d, N = 2, 4, len(parent)
    X0, x, W, S0, beta, gate = _layer(N, H, d)
    o, q, k, v = prologue.conv_verify(parent, S0, X0, x, W, beta, gate, H, d)
    for n in range(N):
        p = gdn.root_path(parent, n)
        oc, qc, kc, vc = _chain_by_library(X0, x[p], W, S0, beta[p], gate[p], H, d)
        for a, b in ((q[n], qc[-1]), (k[n], kc[-1]), (v[n], vc[-1]), (o[n], oc[-1])):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_sibling_isolation_through_the_prologue():
    H, d, N = 1, 4, len(MIXED)
    X0, x, W, S0, beta, gate = _layer(N, H, d)
    o, *_ = prologue.conv_verify(MIXED, S0, X0, x, W, beta, gate, H, d)
    m = 4
    x2 = x.copy()
    x2[m] += 0.5
    o2, *_ = prologue.conv_verify(MIXED, S0, X0, x2, W, beta, gate, H, d)
    for n in range(N):
        changed = not np.array_equal(o2[n], o[n])
        assert changed == (m in gdn.root_path(MIXED, n)), n


def test_committed_window_continues_the_stream():
    """Committing a chain prefix (window from the committed inputs, state by replay of the
    prologue's k, v) and verifying the rest equals verifying the whole chain."""
    H, d, N = 2, 4, 8
    X0, x, W, S0, beta, gate = _layer(N, H, d)
    full, q, k, v = prologue.conv_verify(np.arange(-1, N - 1), S0, X0, x, W, beta, gate, H, d)
    acc = [0, 1, 2]
    X1 = conv.commit_window(X0, x, acc)
    S1 = gdn.replay(S0, k, v, beta, gate, acc)
    tail, *_ = prologue.conv_verify(np.arange(-1, N - 4), S1, X1, x[3:], W, beta[3:], gate[3:],
                                    H, d)
    np.testing.assert_allclose(tail, full[3:], rtol=1e-12, atol=1e-14)

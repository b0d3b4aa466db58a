"""Pins of the tree-aware depthwise conv oracle (closed forms, a library routine, a hand-worked
window table and invariants)."""
import numpy as np
import pytest

from oracle import conv, gdn

RNG = np.random.default_rng(777)
TINY = np.array([-1, 0, 0, 1, 1, 2, 3])
MIXED = np.array([-1, 0, 1, 1, 0, 4, 5, 2, 2, 4])


def _data(N, C=5, Kc=4):
    return RNG.standard_normal((C, Kc - 1)), RNG.standard_normal((N, C)), RNG.standard_normal((C, Kc))


def _unit_weight(C, j, Kc=4):
    W = np.zeros((C, Kc))
    W[:, j] = 1.0
    return W


@pytest.mark.parametrize("parent", [TINY, MIXED, np.arange(-1, 9)])
def test_c1_current_tap_is_identity(parent):
    X0, x, _ = _data(len(parent))
    y = conv.tree_conv(parent, X0, x, _unit_weight(x.shape[1], 3))
    assert np.array_equal(y, x)


@pytest.mark.parametrize("parent", [TINY, MIXED, np.arange(-1, 9)])
def test_c2_oldest_tap_reads_three_steps_up(parent):
    """W = e_0: y_n is the input three steps up n's root path, or the matching committed
    window entry when the path is shorter than that."""
    X0, x, _ = _data(len(parent))
    y = conv.tree_conv(parent, X0, x, _unit_weight(x.shape[1], 0))
    for n in range(len(parent)):
        a = n
        for _ in range(3):
            a = int(parent[a]) if a >= 0 else a - 1  # below the root: -1, -2, -3 = X0 taps 2, 1, 0
        if a >= 0:
            assert np.array_equal(y[n], x[a])
        else:
            assert np.array_equal(y[n], X0[:, 3 + a])


def test_c3_chain_equals_library_correlation():
    """Pure chain: each channel is numpy's 'valid' correlation of (X0 ++ x) with W[c]."""
    N, C = 9, 6
    X0, x, W = _data(N, C)
    y = conv.tree_conv(np.arange(-1, N - 1), X0, x, W)
    for c in range(C):
        series = np.concatenate([X0[c], x[:, c]])
        np.testing.assert_allclose(y[:, c], np.correlate(series, W[c], mode="valid"),
                                   rtol=0, atol=1e-13)


def test_tiny_tree_windows_hand_worked():
    """Windows of the 7-node tree [-1,0,0,1,1,2,3], worked out by hand from the parent chains
    (oldest first), checked one tap at a time."""
    X0, x, _ = _data(7, 3)
    c = [X0[:, 0], X0[:, 1], X0[:, 2]]
    expect = {
        0: [c[0], c[1], c[2], x[0]],
        1: [c[1], c[2], x[0], x[1]],
        2: [c[1], c[2], x[0], x[2]],
        3: [c[2], x[0], x[1], x[3]],
        4: [c[2], x[0], x[1], x[4]],
        5: [c[2], x[0], x[2], x[5]],
        6: [x[0], x[1], x[3], x[6]],
    }
    for j in range(4):
        y = conv.tree_conv(TINY, X0, x, _unit_weight(3, j))
        for n, win in expect.items():
            assert np.array_equal(y[n], win[j]), (n, j)


@pytest.mark.parametrize("parent", [TINY, MIXED])
def test_c4_sibling_isolation(parent):
    N = len(parent)
    X0, x, W = _data(N)
    y = conv.tree_conv(parent, X0, x, W)
    for m in range(1, N):
        x2 = x.copy()
        x2[m] += 1.0
        y2 = conv.tree_conv(parent, X0, x2, W)
        for n in range(N):
            if m in gdn.root_path(parent, n):
                assert not np.array_equal(y2[n], y[n])
            else:
                assert np.array_equal(y2[n], y[n])


def test_c5_commit_window():
    X0, x, _ = _data(7, 3)
    assert np.array_equal(conv.commit_window(X0, x, [0, 1, 3, 6]), np.stack([x[1], x[3], x[6]], 1))
    assert np.array_equal(conv.commit_window(X0, x, [0]), np.stack([X0[:, 1], X0[:, 2], x[0]], 1))
    assert np.array_equal(conv.commit_window(X0, x, []), X0)


def test_commit_then_conv_continues_the_stream():
    """After committing a path, a chain's conv over the new window equals the conv of the
    longer chain that includes the committed tokens."""
    X0, x, W = _data(10, 4)
    path = [0, 1, 2, 3]
    X1 = conv.commit_window(X0, x, path)
    y_tail = conv.tree_conv(np.arange(-1, 5), X1, x[4:10], W)
    y_full = conv.tree_conv(np.arange(-1, 9), X0, x, W)
    np.testing.assert_allclose(y_tail, y_full[4:], atol=1e-14)

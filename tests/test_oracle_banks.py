"""Pins of the factor-bank bookkeeping oracle (integer semantics, brute force)."""
import numpy as np

from gated_deltanet_tree_amd import synth
from oracle import banks, gdn


def test_compaction_is_row_gather():
    rng = np.random.default_rng(5)
    src = rng.standard_normal((22, 3, 7))
    for L in range(0, 10):
        path = rng.choice(22, size=L, replace=False)
        dst = banks.compact(src, path)
        for i in range(L):
            assert np.array_equal(dst[i], src[path[i]])


def test_in_order_paths():
    assert banks.is_in_order([]) and banks.is_in_order([0]) and banks.is_in_order([0, 1, 2])
    assert not banks.is_in_order([0, 2]) and not banks.is_in_order([1])


def test_path_validation_against_enumeration():
    parent = np.array([-1, 0, 0, 1, 1, 2, 3])
    valid = {tuple(gdn.root_path(parent, n)) for n in range(7)} | {()}
    rng = np.random.default_rng(3)
    for _ in range(2000):
        L = int(rng.integers(0, 6))
        path = tuple(int(x) for x in rng.integers(-1, 8, size=L))
        assert banks.check_path(parent, path) == (path in valid)
    for p in valid:
        assert banks.check_path(parent, p)


def test_bookkeeping():
    assert banks.commit_bookkeeping(0, [0, 1, 2]) == (1, 3, False)
    assert banks.commit_bookkeeping(1, [0, 1, 3, 6]) == (1, 4, True)
    assert banks.commit_bookkeeping(1, []) == (1, 0, False)
    assert banks.commit_bookkeeping(0, [0]) == (1, 1, False)


def test_rotation_and_compaction_hold_the_same_rows():
    """For an in-order path, compacting the written bank yields exactly the rows a role swap
    exposes; either way the pending rows are the path's rows."""
    rng = np.random.default_rng(11)
    parent = synth.make_tree(rng, 22, 4, 12)
    written = rng.standard_normal((22, 5))
    for L in range(1, 13):
        path = np.arange(L)
        assert banks.check_path(parent, path)
        assert np.array_equal(banks.compact(written, path), written[:L])


def test_row_map_commit_reads_the_compacted_rows():
    """The no-copy commit: for every root path of a tree, the written rows read through the row
    map are the rows compaction would produce, the written bank becomes pending whenever
    something was accepted, and an empty path changes nothing."""
    rng = np.random.default_rng(13)
    parent = synth.make_tree(rng, 22, 4, 12)
    written = rng.standard_normal((22, 5))
    for node in range(22):
        path = gdn.root_path(parent, node)
        role, L, rows = banks.commit_row_map(1, path)
        assert (role, L) == (0, len(path))
        assert np.array_equal(written[rows], banks.compact(written, path))
        old_role, _, compacted = banks.commit_bookkeeping(1, path)
        # the guide's commit: the rows sit at 0..L-1 of the pending bank either way
        assert banks.pending_rows_after_compaction(path) == list(range(L))
        assert old_role == (0 if banks.is_in_order(path) else 1) and compacted != \
            banks.is_in_order(path)
    assert banks.commit_row_map(0, []) == (0, 0, [])
    assert banks.commit_row_map(1, [0]) == (0, 1, [0])

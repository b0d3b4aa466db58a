"""Accepted-factor banks: compaction and role bookkeeping (integer and copy semantics).

SpecLA guide, mechanism 3: the accepted path's raw factors live in two FP32 double-buffered
banks that alternate between "pending, to be consumed" and "being written".  When the
accepted path is already in order the banks simply swap roles with no device copy; for a
branched acceptance a compaction moves the rows at arbitrary tree indices back into path
order.

Readings: "already in order" means path == [0, 1, ..., L-1]; compaction writes into the
consumed pending bank and leaves the roles unchanged; pending length becomes L either way.

A second commit form (not on the pages, a design of this library) never copies: the written
bank always becomes pending, and a row map records where each pending factor sits, i.e. the
accepted path itself.  Reading the written rows through that map gives exactly the rows the
compaction would have produced, so the fold that follows is the same.
"""
from __future__ import annotations

import numpy as np


def is_in_order(path) -> bool:
    path = np.asarray(path)
    return bool(np.array_equal(path, np.arange(len(path))))


def compact(src_rows, path):
    """dst[i] = src[path[i]] for i < L."""
    return np.asarray(src_rows)[np.asarray(path, dtype=np.int64)].copy()


def check_path(parent, path) -> bool:
    """A committable path starts at the root and follows parent pointers (empty allowed)."""
    path = [int(p) for p in path]
    if not path:
        return True
    if path[0] != 0:
        return False
    for a, b in zip(path, path[1:]):
        if not 0 <= b < len(parent) or parent[b] != a:
            return False
    return all(0 <= p < len(parent) for p in path)


def commit_bookkeeping(role: int, path) -> tuple[int, int, bool]:
    """(new role, new pending length, compaction needed) after accepting `path`.

    role = index of the pending bank; the other bank is the one the verify wrote."""
    L = len(path)
    if L == 0:
        return role, 0, False
    if is_in_order(path):
        return role ^ 1, L, False
    return role, L, True


def commit_row_map(role: int, path) -> tuple[int, int, list[int]]:
    """(new role, new pending length, row map) of the no-copy commit: pending factor i is row
    path[i] of the bank the verify wrote, which becomes the pending bank."""
    L = len(path)
    if L == 0:
        return role, 0, []
    return role ^ 1, L, [int(p) for p in path]


def pending_rows_after_compaction(path) -> list[int]:
    """Row map after the guide's commit: compacted (or already in-order) rows sit at 0..L-1."""
    return list(range(len(path)))

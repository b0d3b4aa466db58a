"""Host side of the HIP library, no GPU needed: the C ABI loads and exports every declared
symbol, the heavy-light schedule is bit-exact against the oracle, and malformed input is
rejected with the documented status codes."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth
from oracle import hld

import plan_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# tests that need the device entry points of the full library (not in the sanitized host build)
full_library = pytest.mark.skipif(binding.host_only(),
                                  reason="device entry points are not in the host-only build")
KEYS = ["seq_offsets", "wave_offsets", "chain_offsets", "chain_nodes", "chain_seq",
        "chain_src", "node_store", "node_parent", "node_depth"]


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn_tree.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


@full_library
def test_library_exports_every_declared_symbol():
    L = binding.lib()
    declared = _declared_functions()
    assert set(declared) == set(binding.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def _check_same(image, ref):
    v = binding.schedule_view(image)
    for key in ("n_seqs", "n_nodes", "n_chains", "n_waves", "n_boundaries", "max_chain_len"):
        assert v[key] == ref[key], key
    for key in KEYS:
        assert np.array_equal(v[key], ref[key]), key


def test_golden_examples(golden_dir):
    import glob
    import json
    for f in sorted(glob.glob(os.path.join(golden_dir, "hld_*.json"))):
        case = json.load(open(f))
        v = binding.schedule_view(binding.hld_schedule(case["parents"]))
        for key, val in case["expected"].items():
            if isinstance(val, list):
                assert np.array_equal(v[key], np.array(val)), (f, key)
            else:
                assert v[key] == val, (f, key)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7])
def test_all_small_trees_bit_exact(N):
    for choice in itertools.product(*[range(i) for i in range(1, N)]):
        parent = np.array((-1,) + choice, dtype=np.int32)
        _check_same(binding.hld_schedule([parent]), hld.schedule([parent]))


def test_random_batches_bit_exact():
    rng = np.random.default_rng(2024)
    for trial in range(10000 // 20):
        parents = []
        for _ in range(int(rng.integers(1, 40))):
            N, K, D = int(rng.integers(1, 65)), int(rng.integers(1, 9)), int(rng.integers(1, 17))
            try:
                parents.append(synth.make_tree(rng, N, K, D))
            except ValueError:
                parents.append(np.arange(-1, N - 1, dtype=np.int32))
        _check_same(binding.hld_schedule(parents), hld.schedule(parents))


@pytest.mark.parametrize("name", ["one-layer", "batched", "wide-deep", "chain16"])
def test_workload_trees_bit_exact(name):
    parents = [synth.workload_tree(name, b) for b in range(synth.WORKLOADS[name]["Bs"])]
    _check_same(binding.hld_schedule(parents), hld.schedule(parents))


def test_empty_batch():
    image = binding.hld_schedule([])
    v = binding.schedule_view(image)
    assert v["n_seqs"] == 0 and v["n_chains"] == 0 and v["n_waves"] == 0


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 2], [-1, -1], [-1, 0, 0, 5], [3, -1]])
def test_malformed_trees_rejected(bad):
    with pytest.raises(binding.GdnError) as e:
        binding.hld_schedule([np.array(bad)])
    assert e.value.status == -2


def test_capacity_and_null_errors():
    L = binding.lib()
    parent = np.array([-1, 0, 0], dtype=np.int32)
    offs = np.array([0, 3], dtype=np.int32)
    need = binding.schedule_words(1, 3)
    small = np.zeros(need - 1, dtype=np.int32)
    sentinel = small.copy()
    rc = L.gdn_hld_schedule(binding._ptr(parent), binding._ptr(offs), 1, binding._ptr(small),
                            small.size)
    assert rc == -4 and np.array_equal(small, sentinel)  # nothing written on error
    assert L.gdn_hld_schedule(None, binding._ptr(offs), 1, binding._ptr(small), small.size) == -1
    assert b"null" in L.gdn_last_error()
    too_big = np.full(1025, 0, dtype=np.int32)
    too_big[0] = -1
    with pytest.raises(binding.GdnError) as e:
        binding.hld_schedule([too_big])
    assert e.value.status == -1


@pytest.mark.parametrize("offs,status", [
    ([1, 3], -1),                      # seq_offsets[0] != 0
    ([0, 3, 3], -2),                   # an empty tree
    ([0, 3, 1], -2),                   # decreasing offsets
    ([0, 3, 3 + 1025], -1),            # a tree above 1024 nodes
    ([0, 3, -(2 ** 31)], -2),          # an offset whose difference overflows 32 bits
    ([0, 2 ** 31 - 1], -1),            # a huge tree, refused before any parent is read
])
def test_malformed_seq_offsets_rejected(offs, status):
    """Offsets are validated before any parent is read, in 64-bit arithmetic; nothing is
    written on error."""
    L = binding.lib()
    parent = np.array([-1, 0, 0, -1, 0], dtype=np.int32)
    offs = np.array(offs, dtype=np.int64).astype(np.int32)
    image = np.full(binding.schedule_words(2, 5), 7, dtype=np.int32)
    rc = L.gdn_hld_schedule(binding._ptr(parent), binding._ptr(offs), len(offs) - 1,
                            binding._ptr(image), image.size)
    assert rc == status, L.gdn_last_error()
    assert np.all(image == 7)
    assert L.gdn_hld_schedule(binding._ptr(parent), binding._ptr(offs), -1,
                              binding._ptr(image), image.size) == -1


@full_library
def test_device_calls_validate_before_launch():
    """Argument errors are reported before any device work (no GPU is touched here)."""
    L = binding.lib()
    image = binding.hld_schedule([np.array([-1, 0, 0, 1])])
    args = binding.VerifyArgs()
    args.n_seqs, args.n_nodes, args.n_heads, args.head_dim = 1, 4, 1, 64  # bad head_dim
    args.max_nodes, args.n_layers, args.in_dtype = 4, 1, 0
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(image), 1, None) == -1
    assert b"head_dim" in L.gdn_last_error()
    args.head_dim = 16
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(image), 1, None) == -1  # nulls
    for name in ("state", "role", "pending_len", "q", "k", "v", "beta", "gate", "out", "workspace"):
        setattr(args, name, 16)
    for i in range(2):
        args.bank_k[i] = args.bank_u[i] = args.bank_lg[i] = 16
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(image), 1, None) == -1
    assert b"pending_rows" in L.gdn_last_error()  # the row map is required
    args.pending_rows = 16
    args.max_nodes = 3  # smaller than the tree
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(image), 1, None) == -4
    args.max_nodes, args.n_nodes = 4, 5  # disagrees with the schedule
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(image), 1, None) == -1
    args.n_nodes = 4
    assert L.gdn_tree_verify_wave(ctypes.byref(args), binding._ptr(image), 1, 7, None) == -1
    bad_image = image.copy()
    bad_image[0] = 0
    assert L.gdn_tree_verify(ctypes.byref(args), binding._ptr(bad_image), 1, None) == -1
    cargs = binding.ConvArgs()
    cargs.width = 3
    assert L.gdn_tree_conv(ctypes.byref(cargs), binding._ptr(image), 1, None) == -1


@full_library
def test_commit_rejects_bad_paths_before_launch():
    """Non-root paths, broken parent links and out-of-range ids give GDN_EPATH and leave the
    host mirrors untouched."""
    L = binding.lib()
    parent = np.array([-1, 0, 0, 1, 1, 2, 3], dtype=np.int32)
    image = binding.hld_schedule([parent])
    args = binding.VerifyArgs()
    args.n_seqs, args.n_nodes, args.n_heads, args.head_dim = 1, 7, 1, 16
    args.max_nodes, args.n_layers = 7, 1
    for name in ("state", "role", "pending_len", "pending_rows"):
        setattr(args, name, 16)
    for i in range(2):
        args.bank_k[i] = args.bank_u[i] = args.bank_lg[i] = 16
    role, pend = np.array([0], dtype=np.int32), np.array([3], dtype=np.int32)

    def commit(path, mode=binding.COMMIT_ROW_MAP, dev_paths=16):
        flat, offs = binding.pack_paths([path])
        return L.gdn_commit_path(binding._ptr(image), binding._ptr(flat), binding._ptr(offs),
                                 dev_paths, 16, ctypes.byref(args), None, binding._ptr(role),
                                 binding._ptr(pend), mode, None)

    for mode in (binding.COMMIT_COMPACT, binding.COMMIT_ROW_MAP):
        for bad in ([1], [0, 2, 3], [0, 1, 5], [0, 7], [0, 1, 3, 6, 6], [0, -1]):
            assert commit(bad, mode) == -3, (bad, mode)
            assert role[0] == 0 and pend[0] == 3
    assert commit([0, 1, 3], mode=2) == -1  # unknown mode
    assert b"mode" in L.gdn_last_error()
    assert commit([0, 1, 3], dev_paths=None) == -1  # a non-empty path needs its device copy
    assert b"dev_paths" in L.gdn_last_error()
    args.pending_rows = None
    assert commit([0, 1, 3]) == -1
    assert role[0] == 0 and pend[0] == 3


def test_ut_plan_matches_layout_checker_bit_exact():
    """The tree-masked verify plan in the image equals the layout checker's construction."""
    rng = np.random.default_rng(31)
    batches = [[np.array([-1, 0, 0, 1, 1, 2, 3])],
               [synth.make_tree(rng, 22, 4, 12) for _ in range(32)],
               [synth.make_tree(rng, 64, 8, 16) for _ in range(8)] + [np.array([-1])],
               [np.arange(-1, 15) for _ in range(4)]]
    for trees in batches:
        image = binding.hld_schedule(trees)
        got = binding.schedule_view(image)["ut_plan"]
        want = plan_layout.ut_plan(trees)
        for key in ("rec_base", "node_rec", "lv_base", "lvn", "lvnode", "rec_anc"):
            assert np.array_equal(got[key], want[key]), key
        assert got["records"] == int(want["rec_base"][-1])
        assert got["max_records"] == int(np.max(np.diff(want["rec_base"])))
        assert got["max_levels"] == int(np.max(np.diff(want["lv_base"])))


def test_ut_plan_absent_when_too_deep():
    """A 1024-node chain needs 1024*1025/2 records, above the 32-per-node budget."""
    image = binding.hld_schedule([np.arange(-1, 1023)])
    assert int(image[8]) == -1 and binding.schedule_view(image)["ut_plan"] is None

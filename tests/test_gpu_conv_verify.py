"""GPU parity of the fused conv -> SiLU -> unit-length -> tree-masked verify
(gdn_tree_conv_verify) against the float64 oracle (oracle.prologue + oracle.gdn), through the
C ABI, on seeded bf16 inputs: per-node outputs, banked keys, residual vectors, log gates and conv
inputs, the folded conv window and the committed state, over several verify + commit steps and
a flush.  Cases: ragged small trees (a 7-node tree, an 8-node chain, single nodes), a 16-node
chain whose pending path outgrows one LDS fold chunk, a 40-node tree (two passes of S0
products), a 48-node top-8 tree of depth 16, a 64-node top-8 tree next to a 16-node chain
(the wide/deep workload's shapes), a 24-node chain (the level-by-level inverse), a 66-node
tree (two-chunk lists, a record walk over two waves), trees of depth 12 and 13 (the boundary
between the kernel's two builds), 1056 (sequence, head) workgroups of ragged trees (more than
the device holds at once), and the batched workload (32 sequences x 22-node trees x 48 heads)
on sampled sequences; one launch over several layers is bit-identical to one per layer.

Tolerances: o per (node, head) vector <= 1e-3 normwise max relative error; committed state <= 1e-5
relative Frobenius per (layer, seq, head) tile; banked u <= 1e-5 relative 2-norm per row; ln g
within 4 fp32 ulp; conv inputs and folded windows bit-exact (copies of bf16 / fp32 values).
The banked key is the kernel's fp32 unit key: conv (4 fused multiply-adds of exact products),
SiLU (exp and a division) and the normalisation (a sum of squares, a square root and a
reciprocal) round a handful of times in fp32, about 1e-6 of the vector's norm; the bar is 1e-5
relative 2-norm per row."""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload
from oracle import conv as oconv
from oracle import gdn as ogdn
from oracle import prologue

import gpu_harness as gh

pytestmark = pytest.mark.gpu

D = 128
K_TOL = gh.K_TOL


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def fused_inputs(trees, step, n_layers, H, cfg_id):
    """Seeded bf16 conv inputs x [Ly][T][3Hd] and beta, gate [Ly][T][H] of one step."""
    C = 3 * H * D
    sizes = [len(t) for t in trees]
    T = sum(sizes)
    x = np.empty((n_layers, T, C), np.uint16)
    beta = np.empty((n_layers, T, H), np.uint16)
    gate = np.empty((n_layers, T, H), np.uint16)
    for layer in range(n_layers):
        off = 0
        for b, n in enumerate(sizes):
            vals = synth.node_inputs(cfg_id, step, layer, b, n, H, D, "bf16")
            beta[layer, off:off + n] = vals["beta"]
            gate[layer, off:off + n] = vals["gate"]
            x[layer, off:off + n] = synth.conv_inputs(cfg_id, step, layer, b, n, C, "bf16")
            off += n
    return x, beta, gate


class FusedRun:
    """A batch of trees on the device, driven through gdn_tree_conv_verify, with the oracle's
    committed states and windows carried alongside."""

    def __init__(self, torch_cuda, trees, H, n_layers, cfg_id, max_nodes=None,
                 commit_mode="row-map"):
        self.torch = torch_cuda
        self.H, self.Ly, self.cfg = H, n_layers, cfg_id
        self.C = 3 * H * D
        self.b = gh.Batch(trees, n_layers, H, D, self.C, max_nodes=max_nodes, mode="fused",
                          commit_mode=commit_mode, conv_dtype="bf16")
        b = self.b
        S0 = np.stack([np.stack([synth.initial_state(cfg_id, l, s, H, D) for s in range(b.S)])
                       for l in range(n_layers)])
        X0 = np.stack([np.stack([synth.initial_conv_state(cfg_id, l, s, self.C, 4)
                                 for s in range(b.S)]) for l in range(n_layers)])
        self.W = np.stack([synth.conv_weight(cfg_id, l, self.C, 4, "bf16") for l in range(n_layers)])
        b.set_state(S0, X0)
        self.Wd = workload._to_torch(self.W, "bf16", "cuda")
        self.W64 = workload.widen(self.W, "bf16")
        self.committed = S0.astype(np.float64)
        self.window = X0.astype(np.float64)

    def verify(self, step, layers=None):
        b = self.b
        x, beta, gate = fused_inputs(b.trees, step, self.Ly, self.H, self.cfg)
        xd, bd, gd = (workload._to_torch(a, "bf16", "cuda") for a in (x, beta, gate))
        self.role_before = b.layers.role_host.copy()
        for layer in range(self.Ly) if layers is None else layers:
            va = binding.verify_args(b.image, b.layers, None, None, None, bd, gd, b.out, None,
                                     layer_begin=layer, n_layers=1)
            ca = binding.conv_args(b.image, b.layers, xd, self.Wd, None, layer_begin=layer,
                                   n_layers=1)
            binding.tree_conv_verify(va, ca, b.image, b.dev_image)
        self.torch.cuda.synchronize()
        self.h64 = {"x": workload.widen(x, "bf16"), "beta": workload.widen(beta, "bf16"),
                    "gate": workload.widen(gate, "bf16")}

    def check_fold(self, what):
        gh.assert_state(gh.to_np(self.b.layers.state), self.committed, what=what, mode="fused")
        cs = gh.to_np(self.b.layers.conv_state)
        assert np.array_equal(cs, self.window.astype(np.float32)), f"conv window after {what}"

    def oracle(self, layer, s):
        b = self.b
        sl = slice(b.offs[s], b.offs[s + 1])
        x, beta, gate = (self.h64[k][layer, sl] for k in ("x", "beta", "gate"))
        o, q, k, v = prologue.conv_verify(b.trees[s], self.committed[layer, s],
                                          self.window[layer, s], x, self.W64[layer], beta, gate,
                                          self.H, D)
        with np.errstate(divide="ignore"):  # a zero gate banks ln g = -inf
            kf, uf, lg = ogdn.factors(b.trees[s], self.committed[layer, s], k, v, beta, gate)
        return dict(o=o, k=kf, u=uf, lg=lg, v=v, beta=beta, gate=gate, x=x)

    def check_outputs(self, seqs=None, layers=None):
        """Outputs and written banks of the last verify; returns the oracle records."""
        b = self.b
        refs = {}
        for layer in range(self.Ly) if layers is None else layers:
            o_gpu = gh.to_np(b.out[layer])
            for s in range(b.S) if seqs is None else seqs:
                r = self.oracle(layer, s)
                sl = slice(b.offs[s], b.offs[s + 1])
                n = len(b.trees[s])
                gh.assert_outputs(o_gpu[sl], r["o"], what=f"o layer {layer} seq {s}",
                                  mode="fused")
                wb = 1 - int(self.role_before[s])
                gh.assert_bank_rows(b, layer, s, wb, range(n), r["k"], r["u"], r["lg"])
                xb = gh.to_np(b.layers.bank_x[wb][layer, s][:n])
                assert np.array_equal(xb, r["x"]), "banked conv inputs not exact"
                refs[(layer, s)] = r
        return refs

    def commit(self, paths, refs):
        """Accept one path per sequence on the device; advance the oracle's committed state and
        window by replaying the path."""
        b = self.b
        b.commit(None, paths)
        self.torch.cuda.synchronize()
        exp_role, exp_pend, exp_rows = gh.role_pending_expect(self.role_before, paths,
                                                              b.commit_mode)
        assert np.array_equal(b.layers.role_host, exp_role)
        assert np.array_equal(b.layers.pending_host, exp_pend)
        row_map = b.layers.pending_rows.cpu().numpy()
        for s, rows in enumerate(exp_rows):
            assert list(row_map[s, :len(rows)]) == rows, f"row map seq {s}"
        for (layer, s), r in refs.items():
            p = [int(i) for i in paths[s]]
            self.committed[layer, s] = ogdn.replay(self.committed[layer, s], r["k"], r["v"],
                                                   r["beta"], r["gate"], p)
            self.window[layer, s] = oconv.commit_window(self.window[layer, s], r["x"], p)

    def flush(self):
        self.b.flush()
        self.torch.cuda.synchronize()


def _steps(torch_cuda, trees, H, n_layers, steps_paths, cfg_id, max_nodes=None,
           commit_mode="row-map", commit_modes=None):
    """Verify + check + commit per step, then flush; commit_modes switches the commit form
    step by step."""
    run = FusedRun(torch_cuda, trees, H, n_layers, cfg_id, max_nodes, commit_mode)
    for step, paths in enumerate(steps_paths):
        if commit_modes is not None:
            run.b.commit_mode = commit_modes[step]
        run.verify(step)
        run.check_fold(f"fold before step {step}")
        refs = run.check_outputs()
        run.commit(paths, refs)
    run.flush()
    run.check_fold("flush")
    return run


@pytest.mark.parametrize("commit_mode", ["row-map", "compact"])
def test_small_trees_steps_and_flush(torch_cuda, commit_mode):
    """7-node tree, 8-node chain and a single node; branched, in-order, single-node and empty
    paths over three steps, then a flush; both commit forms."""
    tiny, chain, single = synth.TINY_TREE, synth.TINY_CHAIN, np.array([-1])
    trees = [tiny, chain, single]
    steps = [
        [[0, 1, 3, 6], list(range(8)), [0]],      # branched (compaction), in order (swap), root
        [[0, 2, 5], [0, 1, 2], []],               # branched, short prefix, nothing committed
        [[0, 1, 4], list(range(5)), [0]],
    ]
    _steps(torch_cuda, trees, H=2, n_layers=2, steps_paths=steps, cfg_id=11,
           commit_mode=commit_mode)


@pytest.mark.parametrize("commit_mode", ["row-map", "compact"])
def test_pending_path_longer_than_one_fold_chunk(torch_cuda, commit_mode):
    """A 16-node chain next to a 10-node tree: at 16 nodes and 16 bank rows the LDS room after
    the v plane holds 6 fold rows (7 would need 8448 bytes of its 8192), so a pending path of
    16 rows folds in three chunks (6, 6, 4) and one of 9 in two; both commit forms."""
    chain = np.arange(-1, 15)
    tree = np.array([-1, 0, 0, 1, 2, 3, 4, 5, 6, 7])
    steps = [[list(range(16)), [0, 1, 3, 5, 7, 9]],
             [list(range(9)), [0, 2, 4, 6, 8]],
             [list(range(16)), [0]]]
    _steps(torch_cuda, [chain, tree], H=1, n_layers=1, steps_paths=steps, cfg_id=12,
           commit_mode=commit_mode)


def test_commit_modes_alternate(torch_cuda):
    """A caller may switch commit forms between steps: row map, compaction, row map,
    compaction over four steps of the tiny tree, the 8-node chain and a single node (branched,
    in-order, root-only and empty paths), then flush; every fused fold reads the rows the last
    commit recorded."""
    trees = [synth.TINY_TREE, synth.TINY_CHAIN, np.array([-1])]
    steps = [[[0, 1, 3, 6], list(range(8)), [0]],
             [[0, 2, 5], [0, 1, 2], []],
             [[0, 1, 4], [], [0]],
             [[0, 2], list(range(6)), [0]]]
    _steps(torch_cuda, trees, H=2, n_layers=1, steps_paths=steps, cfg_id=19,
           commit_modes=["row-map", "compact", "row-map", "compact"])


def test_forty_node_tree(torch_cuda):
    """More than 32 nodes: the S0 products take two passes and W gets its own LDS region."""
    rng = synth.rng_for(13, 0, 0, 0, "tree")
    tree = synth.make_tree(rng, 40, 4, 14)
    path = synth.deepest_leaf_path(tree)
    steps = [[path, [0, 1, 3, 6]], [path[:5], [0, 2]]]
    _steps(torch_cuda, [tree, synth.TINY_TREE], H=1, n_layers=1, steps_paths=steps, cfg_id=13)


def test_deep_chain_level_inverse(torch_cuda):
    """A 24-node chain (depth 23: past the per-lane register form of the tree inverse, which
    stops at depth 16, so the level-by-level form runs) next to a branched tree."""
    rng = synth.rng_for(16, 0, 0, 0, "tree")
    tree = synth.make_tree(rng, 30, 4, 10)
    chain = np.arange(-1, 23, dtype=np.int32)
    steps = [[list(range(20)), synth.deepest_leaf_path(tree)],
             [list(range(24)), [0]]]
    _steps(torch_cuda, [chain, tree], H=1, n_layers=1, steps_paths=steps, cfg_id=16)


@pytest.mark.parametrize("depth", [12, 13])
def test_inverse_build_boundary(torch_cuda, depth):
    """The deepest tree of the batch picks the kernel's build: depth 12 runs the 80-VGPR build
    (per-lane inverse up to depth 12), depth 13 the 128-VGPR one (per-lane inverse up to 16).
    A chain of that depth with one branch off its middle, next to the tiny tree."""
    tree = np.array(list(range(-1, depth)) + [depth // 2], dtype=np.int32)
    assert synth.node_depths(tree).max() == depth
    steps = [[list(range(depth + 1)), [0, 1, 3]],
             [list(range(depth // 2 + 1)) + [depth + 1], [0, 2]]]
    _steps(torch_cuda, [tree, synth.TINY_TREE], H=1, n_layers=1, steps_paths=steps,
           cfg_id=30 + depth)


def test_more_items_than_one_round(torch_cuda):
    """22 sequences x 48 heads = 1056 (sequence, head) workgroups: more than the device holds at
    once (three on each of 256 CUs), so later ones start on CUs as earlier ones retire, with
    ragged trees (single nodes, a 3-node fan, the tiny tree and chain, 12-node top-4 trees)
    side by side; every (sequence, head) of two steps against the oracle, then a flush."""
    rng = synth.rng_for(20, 0, 0, 0, "tree")
    kinds = [np.array([-1]), np.array([-1, 0, 0]), synth.TINY_TREE, synth.TINY_CHAIN]
    trees = [kinds[i % 5] if i % 5 < 4 else synth.make_tree(rng, 12, 4, 6) for i in range(22)]

    def path_to(t, v):  # root .. v
        p = []
        while v >= 0:
            p.append(int(v))
            v = t[v]
        return p[::-1]

    steps = [[synth.deepest_leaf_path(t) for t in trees],
             [path_to(t, len(t) // 2) for t in trees]]
    _steps(torch_cuda, trees, H=48, n_layers=1, steps_paths=steps, cfg_id=20)


def test_48_node_tree(torch_cuda):
    """A 48-node top-8 tree of depth <= 16 (two passes of S0 products, the depth-16 per-lane
    inverse), next to a 7-node tree."""
    rng = synth.rng_for(17, 0, 0, 0, "tree")
    tree = synth.make_tree(rng, 48, 8, 16)
    steps = [[synth.random_path(rng, tree, 11), [0, 1, 3]],
             [synth.deepest_leaf_path(tree), [0, 2, 5]]]
    _steps(torch_cuda, [tree, synth.TINY_TREE], H=1, n_layers=1, steps_paths=steps, cfg_id=17)


def test_tree_past_64_nodes(torch_cuda):
    """A 66-node top-4 tree of depth <= 10 (about 149 KB of LDS, one workgroup per CU): every
    per-node list takes two 64-entry chunks, the record walk spans two waves and the S0
    products take three passes; next to the tiny tree."""
    rng = synth.rng_for(21, 0, 0, 0, "tree")
    tree = synth.make_tree(rng, 66, 4, 10)
    assert len(tree) == 66
    steps = [[synth.deepest_leaf_path(tree), [0, 1, 3]],
             [synth.random_path(rng, tree, 9), [0, 2, 5]]]
    _steps(torch_cuda, [tree, synth.TINY_TREE], H=1, n_layers=1, steps_paths=steps, cfg_id=21)


def test_wide_deep_64_node_tree_and_chain(torch_cuda):
    """The wide/deep workload's shapes: a 64-node top-8 tree of depth <= 16 (two passes of S0
    products, each handing its nodes' k and q rows to w and G r) next to a 16-node chain."""
    rng = synth.rng_for(18, 0, 0, 0, "tree")
    tree, chain = synth.make_tree(rng, 64, 8, 16), np.arange(-1, 15, dtype=np.int32)
    steps = [[synth.random_path(rng, tree, 9), list(range(12))],
             [synth.deepest_leaf_path(tree), list(range(16))]]
    _steps(torch_cuda, [tree, chain], H=2, n_layers=1, steps_paths=steps, cfg_id=18)


def test_batched_workload_sampled(torch_cuda):
    """The batched workload's trees (32 sequences, 22 nodes, top-4, depth <= 12) at 48 heads,
    one layer, two steps (the second folds the first's accepted paths); every head of sampled
    sequences against the oracle."""
    trees = workload.workload_trees("batched")
    run = FusedRun(torch_cuda, trees, 48, 1, cfg_id=synth.WORKLOADS["batched"]["seed"])
    seqs = [0, 7, 31]
    run.verify(0)
    refs = run.check_outputs(seqs=seqs)
    paths = [synth.workload_path("batched", 0, s, t) for s, t in enumerate(trees)]
    run.commit(paths, refs)
    run.verify(1)
    S = gh.to_np(run.b.layers.state[0][seqs])
    gh.assert_state(S, run.committed[0][seqs], what="batched fold")
    cs = gh.to_np(run.b.layers.conv_state[0][seqs])
    assert np.array_equal(cs, run.window[0][seqs].astype(np.float32))
    run.check_outputs(seqs=seqs)


def _fused_snapshots(torch, trees, one_call):
    """Two steps (verify, then a commit) of 3 layers x 2 heads through the fused entry point,
    either one call over all layers or one call per layer; device buffers after each verify."""
    run = FusedRun(torch, trees, 2, 3, cfg_id=22)
    b = run.b
    snaps = []
    for step in range(2):
        x, beta, gate = fused_inputs(b.trees, step, run.Ly, run.H, run.cfg)
        xd, bd, gd = (workload._to_torch(a, "bf16", "cuda") for a in (x, beta, gate))
        spans = [(0, run.Ly)] if one_call else [(layer, 1) for layer in range(run.Ly)]
        for l0, nl in spans:
            va = binding.verify_args(b.image, b.layers, None, None, None, bd, gd, b.out, None,
                                     layer_begin=l0, n_layers=nl)
            ca = binding.conv_args(b.image, b.layers, xd, run.Wd, None, layer_begin=l0,
                                   n_layers=nl)
            binding.tree_conv_verify(va, ca, b.image, b.dev_image)
        torch.cuda.synchronize()
        lay = b.layers
        snaps.append({name: gh.to_np(t).copy() for name, t in [
            ("out", b.out), ("state", lay.state), ("conv_state", lay.conv_state),
            *[(f"{n}{r}", getattr(lay, n)[r]) for n in ("bank_k", "bank_u", "bank_lg", "bank_x")
              for r in range(2)]]})
        b.commit(None, [synth.deepest_leaf_path(t) if step == 0 else [0] for t in trees])
        torch.cuda.synchronize()
    return snaps


def test_one_call_over_layers_equals_one_call_per_layer(torch_cuda):
    """One fused launch over three layers (workgroup b takes layer b / (S H)) gives bit-identical
    outputs, banks, windows and committed states to one launch per layer, over two steps (the
    second folds the first's accepted paths in every layer)."""
    rng = np.random.default_rng(22)
    trees = [synth.TINY_TREE, synth.TINY_CHAIN, synth.make_tree(rng, 20, 3, 8)]
    a = _fused_snapshots(torch_cuda, trees, one_call=False)
    b = _fused_snapshots(torch_cuda, trees, one_call=True)
    for step, (sa, sb) in enumerate(zip(a, b)):
        for name in sa:
            assert np.array_equal(sa[name], sb[name], equal_nan=True), f"{name} @ step {step}"


def test_run_to_run_deterministic(torch_cuda):
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    outs = []
    for _ in range(2):
        run = FusedRun(torch_cuda, trees, 2, 1, cfg_id=14)
        run.verify(0)
        outs.append((gh.to_np(run.b.out), gh.to_np(run.b.layers.bank_u[1])))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


def test_rejects_bad_arguments(torch_cuda):
    """Validation runs before any launch; nothing is written on error."""
    run = FusedRun(torch_cuda, [synth.TINY_TREE], 2, 1, cfg_id=15)
    b = run.b
    x, beta, gate = fused_inputs(b.trees, 0, 1, 2, 15)
    xd, bd, gd = (workload._to_torch(a, "bf16", "cuda") for a in (x, beta, gate))
    before = gh.to_np(b.out).copy()

    def args():
        va = binding.verify_args(b.image, b.layers, None, None, None, bd, gd, b.out, None)
        ca = binding.conv_args(b.image, b.layers, xd, run.Wd, None)
        return va, ca

    va, ca = args()
    ca.channels = 3 * 2 * 128 - 1
    with pytest.raises(binding.GdnError):
        binding.tree_conv_verify(va, ca, b.image, b.dev_image)
    va, ca = args()
    ca.pending_len = 0
    with pytest.raises(binding.GdnError):
        binding.tree_conv_verify(va, ca, b.image, b.dev_image)
    va, ca = args()
    ca.pending_rows = 0
    with pytest.raises(binding.GdnError):
        binding.tree_conv_verify(va, ca, b.image, b.dev_image)
    va, ca = args()
    va.in_dtype = binding.GDN_F32
    with pytest.raises(binding.GdnError):
        binding.tree_conv_verify(va, ca, b.image, b.dev_image)
    big = binding.hld_schedule([synth.make_tree(synth.rng_for(15, 0, 0, 0, "tree"), 64, 8, 16)])
    va, ca = args()
    with pytest.raises(binding.GdnError):  # n_nodes disagree with the 64-node schedule
        binding.tree_conv_verify(va, ca, big, b.dev_image)
    torch_cuda.cuda.synchronize()
    assert np.array_equal(gh.to_np(b.out), before)
    # a 96-node top-8 tree needs more LDS than one workgroup has: refused, nothing launched
    wide = FusedRun(torch_cuda, [synth.make_tree(synth.rng_for(15, 0, 0, 1, "tree"), 96, 8, 16)],
                    1, 1, cfg_id=15)
    with pytest.raises(binding.GdnError, match="LDS"):
        wide.verify(0)

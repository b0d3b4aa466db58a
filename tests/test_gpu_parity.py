"""GPU parity: the HIP path through the C ABI against the float64 oracle, element by element,
on seeded inputs (tiny fp32 trees, every tree with N <= 6, one bf16 layer of 48 heads x 128,
and a 48-layer stack over 10 verify + commit steps with a final flush)."""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload
from oracle import conv as oconv
from oracle import gdn as ogdn

import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def _check_step(b: gh.Batch, h64, S0s, X0s, W, layer=0, write_bank=None, conv=True, host_layer=None):
    """Compare one layer's outputs, conv outputs and written banks with the oracle.
    S0s/X0s: per sequence committed state/window used by this verify; `host_layer` indexes
    the host input arrays (defaults to `layer`).  Returns the oracle record of each sequence
    (its "kv" are the k and v a commit replays)."""
    hl = layer if host_layer is None else host_layer
    o_gpu = gh.to_np(b.out[layer])
    y_gpu = gh.to_np(b.y[layer]) if conv and b.mode != "fused" else None
    refs = []
    for s in range(b.S):
        sl = slice(b.offs[s], b.offs[s + 1])
        seq = {k: v[hl, sl] for k, v in h64.items()}
        r = gh.oracle_pair(b.trees[s], S0s[s], X0s[s] if conv else None, W, seq, b.mode, b.H,
                           b.d)
        gh.assert_outputs(o_gpu[sl], r["o"], what=f"o seq {s}", mode=b.mode)
        if y_gpu is not None:
            gh.assert_outputs(y_gpu[sl], r["y"], what=f"conv y seq {s}", mode=b.mode,
                              quantity="conv y")
        if conv:
            wb = write_bank[s]
            xb = gh.to_np(b.layers.bank_x[wb][layer, s][:len(b.trees[s]), :b.C])
            assert np.array_equal(xb, seq["x"]), "banked conv input not exact"
        gh.assert_bank_rows(b, layer, s, write_bank[s], range(len(b.trees[s])),
                            r["k"], r["u"], r["lg"])
        refs.append(r)
    return refs


MODES = ["chain", "ut"]
COMMITS = ["row-map", "compact"]


def _tiny_setup(torch_cuda, trees, H=1, d=16, C=16, dtype="f32", cfg_id=0, mode="chain",
                commit_mode="row-map"):
    b = gh.Batch(trees, 1, H, d, C, mode=mode, commit_mode=commit_mode, conv_dtype=dtype)
    S0 = np.stack([synth.initial_state(cfg_id, 0, s, H, d) for s in range(b.S)])[None]
    X0 = np.stack([synth.initial_conv_state(cfg_id, 0, s, C, 4) for s in range(b.S)])[None]
    W = synth.conv_weight(cfg_id, 0, C, 4, dtype)[None]
    b.set_state(S0, X0)
    Wd = workload._to_torch(W, dtype, "cuda")
    return b, S0[0].astype(np.float64), X0[0].astype(np.float64), workload.widen(W[0], dtype), Wd


def _run_steps(torch_cuda, b, S0, X0, W64, Wd, steps_paths, dtype, cfg_id, H, d, C,
               commit_modes=None, x_offset=0):
    """Several verify+commit steps then a flush, each checked against the oracle carrying the
    exact committed state (replay of the accepted paths).  x_offset > 0 hands the conv its
    inputs that many elements past an aligned address."""
    committed, window = [s.copy() for s in S0], [x.copy() for x in X0]
    for step, paths in enumerate(steps_paths):
        h = gh.tiny_inputs(b.trees, step, H, d, C, dtype, cfg_id)
        h64 = gh.widen_inputs(h, dtype)
        inp = gh.to_device(h, dtype)
        if x_offset:
            buf = torch_cuda.empty(inp.x.numel() + x_offset, dtype=inp.x.dtype, device="cuda")
            moved = buf[x_offset:].view(inp.x.shape)
            moved.copy_(inp.x)
            inp.x = moved
        role_before = b.layers.role_host.copy()
        b.step(inp, Wd)
        torch_cuda.cuda.synchronize()
        # the fold of the previous step's path happened inside this verify
        gh.assert_state(gh.to_np(b.layers.state[0]), np.stack(committed), what=f"fold @ {step}",
                        mode=b.mode)
        cs = gh.to_np(b.layers.conv_state[0])
        assert np.array_equal(cs, np.stack(window).astype(np.float32)), "conv window fold"
        _check_step(b, h64, committed, window, W64, 0, write_bank=1 - role_before)
        written = {name: [t.clone() for t in getattr(b.layers, name)]
                   for name in ("bank_k", "bank_u", "bank_lg", "bank_x")}
        if commit_modes is not None:
            b.commit_mode = commit_modes[step]
        b.commit(inp, paths, Wd)
        torch_cuda.cuda.synchronize()
        exp_role, exp_pend, exp_rows = gh.role_pending_expect(role_before, paths, b.commit_mode)
        assert np.array_equal(b.layers.role_host, exp_role)
        assert np.array_equal(b.layers.pending_host, exp_pend)
        assert np.array_equal(b.layers.role.cpu().numpy(), exp_role)
        assert np.array_equal(b.layers.pending.cpu().numpy(), exp_pend)
        row_map = b.layers.pending_rows.cpu().numpy()
        for s, path in enumerate(paths):
            wb, pb = 1 - role_before[s], exp_role[s]
            rows = list(row_map[s, :len(path)])
            assert rows == exp_rows[s], f"row map seq {s}"
            for name in ("bank_k", "bank_u", "bank_lg", "bank_x"):
                src = written[name][wb][0, s]
                dst = getattr(b.layers, name)[pb][0, s]
                # pending factor i, read where the fold reads it: row rows[i] of the pending bank
                if name == "bank_x":
                    got, ref = dst[rows], src[list(path)]
                else:
                    got, ref = dst[:, rows], src[:, list(path)]
                assert torch_cuda.equal(got, ref), f"pending {name} rows seq {s}"
            sl = slice(b.offs[s], b.offs[s + 1])
            seq = {k: h64[k][0, sl] for k in h64}
            committed[s] = ogdn.replay(committed[s], seq["k"], seq["v"], seq["beta"],
                                       seq["gate"], path)
            window[s] = oconv.commit_window(window[s], seq["x"], path)
    b.flush()
    torch_cuda.cuda.synchronize()
    gh.assert_state(gh.to_np(b.layers.state[0]), np.stack(committed), what="flush", mode=b.mode)
    assert np.array_equal(gh.to_np(b.layers.conv_state[0]), np.stack(window).astype(np.float32))
    assert np.all(b.layers.pending.cpu().numpy() == 0) and np.all(b.layers.pending_host == 0)
    before = b.layers.state.clone(), b.layers.conv_state.clone()
    b.flush()  # nothing pending: bit-identical
    torch_cuda.cuda.synchronize()
    assert torch_cuda.equal(before[0], b.layers.state)
    assert torch_cuda.equal(before[1], b.layers.conv_state)


@pytest.mark.parametrize("commit_mode", COMMITS)
@pytest.mark.parametrize("mode", MODES)
def test_tiny_tree_and_chain(torch_cuda, mode, commit_mode):
    """The tiny workload: the 7-node tree [-1,0,0,1,1,2,3] and an 8-node chain, batched, fp32,
    d = 16.  Step 0 accepts the deepest leaves ([0,1,3,6] is branched -> compaction or a row map;
    the chain is in order -> role swap); step 1 accepts [0,2,5] and [0,1,2]; then flush."""
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, mode=mode, commit_mode=commit_mode)
    paths0 = [synth.deepest_leaf_path(t) for t in trees]
    assert list(paths0[0]) == [0, 1, 3, 6] and list(paths0[1]) == list(range(8))
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, [paths0, [[0, 2, 5], [0, 1, 2]], [[0], []]],
               "f32", 0, 1, 16, 16)


@pytest.mark.parametrize("mode", MODES)
def test_commit_modes_alternate(torch_cuda, mode):
    """A caller may switch commit forms between steps: row map, compaction, row map, compaction
    over four steps of the tiny tree and chain (branched, in-order and empty paths), then flush;
    every fold reads the rows the last commit recorded."""
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, mode=mode)
    steps = [[[0, 1, 3, 6], list(range(8))], [[0, 2, 5], [0, 1, 2]], [[0, 1, 4], []],
             [[0, 2], list(range(6))]]
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, steps, "f32", 0, 1, 16, 16,
               commit_modes=["row-map", "compact", "row-map", "compact"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_odd_channel_count_conv(torch_cuda, dtype):
    """An odd conv channel count (15) takes the one-channel-per-thread conv kernel; the tiny
    tree and chain over two steps and a flush, conv outputs, banked inputs and windows against
    the oracle."""
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, C=15, dtype=dtype, cfg_id=91)
    paths0 = [synth.deepest_leaf_path(t) for t in trees]
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, [paths0, [[0, 2, 5], [0, 1, 2]]], dtype, 91, 1,
               16, 15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_trees_cross_table_blocks(torch_cuda, dtype):
    """Trees past 64 nodes (a 150-node chain, a 130-node top-3 tree): the conv tables a tree's
    nodes 64 at a time, so the first nodes of a block find ancestors in the previous block
    through the schedule image; the whole chain is accepted at step 0 (a 150-row fold at step
    1).  Two steps and a flush, conv outputs, banks and windows against the oracle."""
    rng = np.random.default_rng(11)
    trees = [np.array([-1] + list(range(149)), np.int32), synth.make_tree(rng, 130, 3, 40)]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, C=16, dtype=dtype, cfg_id=93)
    paths0 = [synth.deepest_leaf_path(t) for t in trees]
    paths1 = [synth.random_path(rng, t, 5) for t in trees]
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, [paths0, paths1], dtype, 93, 1, 16, 16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_unaligned_input_rows(torch_cuda, dtype):
    """x handed over one element past an aligned address: the conv's two-channel loads need 4-
    (bf16) or 8-byte (fp32) alignment, so it takes one channel per thread; the tiny tree and
    chain over two steps and a flush against the oracle."""
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, C=16, dtype=dtype, cfg_id=94)
    paths0 = [synth.deepest_leaf_path(t) for t in trees]
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, [paths0, [[0, 2, 5], [0, 1, 2]]], dtype, 94, 1,
               16, 16, x_offset=1)


def _all_trees(N):
    import itertools
    for choice in itertools.product(*[range(i) for i in range(1, N)]):
        yield np.array((-1,) + choice, dtype=np.int32)


@pytest.mark.parametrize("commit_mode", COMMITS)
@pytest.mark.parametrize("mode", MODES)
def test_every_small_tree_batched(torch_cuda, mode, commit_mode):
    """All 154 labelled trees with N <= 6 in one batch (d = 16, 2 heads, fp32): three steps of
    verify + commit with seeded random paths of every length (0 included), then flush."""
    trees = [t for N in range(1, 7) for t in _all_trees(N)]
    assert len(trees) == 154
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, H=2, C=8, cfg_id=90, mode=mode,
                                     commit_mode=commit_mode)
    rng = np.random.default_rng(4)
    steps = []
    for _ in range(3):
        paths = []
        for t in trees:
            L = int(rng.integers(0, synth.node_depths(t).max() + 2))
            paths.append(synth.random_path(rng, t, L))
        steps.append(paths)
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, steps, "f32", 90, 2, 16, 8)


@pytest.mark.parametrize("mode", MODES)
def test_bf16_inputs_small(torch_cuda, mode):
    """bf16 inputs at d = 16 over a branched batch (exercises the bf16 staging path)."""
    rng = np.random.default_rng(8)
    trees = [synth.make_tree(rng, 12, 3, 5) for _ in range(5)]
    b, S0, X0, W64, Wd = _tiny_setup(torch_cuda, trees, H=3, C=24, dtype="bf16", cfg_id=91,
                                     mode=mode)
    steps = [[synth.random_path(rng, t, int(rng.integers(1, 4))) for t in trees] for _ in range(2)]
    _run_steps(torch_cuda, b, S0, X0, W64, Wd, steps, "bf16", 91, 3, 16, 24)


def _layer_case(torch_cuda, name, n_layers, trees, steps, sample_layers, check_outputs_at,
                mode="chain", commit_mode="row-map"):
    c = synth.WORKLOADS[name]
    H, d, C, dtype = c["H"], c["d"], c["Cch"], c["dtype"]
    b = gh.Batch(trees, n_layers, H, d, C, mode=mode, commit_mode=commit_mode, conv_dtype=dtype)
    layers = range(n_layers)
    S0, X0 = workload.host_initial_state(name, layers, b.S)
    W = workload.host_weights(name, layers)
    b.set_state(S0, X0)
    Wd = workload._to_torch(W, dtype, "cuda")
    committed = {l: [S0[l, s].astype(np.float64) for s in range(b.S)] for l in sample_layers}
    window = {l: [X0[l, s].astype(np.float64) for s in range(b.S)] for l in sample_layers}
    W64 = {l: workload.widen(W[l], dtype) for l in sample_layers}
    for step in range(steps):
        h = workload.host_step_inputs(name, step, trees, layers)
        inp = workload.StepInputs(**{k: workload._to_torch(v, dtype, "cuda") for k, v in h.items()})
        role_before = b.layers.role_host.copy()
        b.step(inp, Wd)
        torch_cuda.cuda.synchronize()
        h64 = {k: workload.widen(v[list(sample_layers)], dtype) for k, v in h.items()}
        kv = {}
        for li, l in enumerate(sample_layers):
            gh.assert_state(gh.to_np(b.layers.state[l]), np.stack(committed[l]), mode=mode,
                            what=f"committed layer {l} step {step}")
            if step in check_outputs_at or mode == "fused":
                # the fused form's k and v come from the conv: the oracle computes them here
                refs = _check_step(b, h64, committed[l], window[l], W64[l], l,
                                   write_bank=1 - role_before, host_layer=li)
                kv[l] = [r["kv"] for r in refs]
        paths = [synth.workload_path(name, step, s, trees[s]) for s in range(b.S)]
        b.commit(inp, paths, Wd)
        for li, l in enumerate(sample_layers):
            for s, path in enumerate(paths):
                sl = slice(b.offs[s], b.offs[s + 1])
                k, v = kv[l][s] if l in kv else (h64["k"][li, sl], h64["v"][li, sl])
                committed[l][s] = ogdn.replay(committed[l][s], k, v, h64["beta"][li, sl],
                                              h64["gate"][li, sl], path)
                window[l][s] = oconv.commit_window(window[l][s], h64["x"][li, sl], path)
    b.flush()
    torch_cuda.cuda.synchronize()
    for l in sample_layers:
        gh.assert_state(gh.to_np(b.layers.state[l]), np.stack(committed[l]), what=f"flush {l}",
                        mode=mode)
        assert np.array_equal(gh.to_np(b.layers.conv_state[l]),
                              np.stack(window[l]).astype(np.float32))


@pytest.mark.parametrize("mode", MODES + ["fused"])
def test_one_layer_bf16_48_heads(torch_cuda, mode):
    """The one-layer workload: 48 heads x 128, bf16 inputs, the seeded 22-node top-4 tree; verify,
    conv and banks for every node and head, then commit of a length-6 path and flush."""
    trees = workload.workload_trees("one-layer")
    _layer_case(torch_cuda, "one-layer", 1, trees, steps=2, sample_layers=[0], check_outputs_at={0, 1},
                mode=mode)


@pytest.mark.parametrize("mode,commit_mode", [("chain", "compact"), ("ut", "row-map"),
                                              ("fused", "row-map"), ("fused", "compact")])
def test_48_layers_ten_steps(torch_cuda, mode, commit_mode):
    """The 48-layer workload: 48 independent layers, 10 verify steps each folding the previous
    step's accepted length-6 path, then flush; oracle on three sampled layers (states every step,
    outputs and banks at steps 0, 4 and 9; every step in the fused form, whose replayed k and v
    are the conv's).  Each verify form runs with one commit form, the fused form with both."""
    trees = workload.workload_trees("48-layer")
    _layer_case(torch_cuda, "48-layer", 48, trees, steps=10, sample_layers=[0, 23, 47],
                check_outputs_at={0, 4, 9}, mode=mode, commit_mode=commit_mode)

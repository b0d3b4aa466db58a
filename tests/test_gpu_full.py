"""GPU parity at full workload sizes, in the launch configuration bench.py times (one GDN
layer per call), checked on seeded samples of (sequence, layer) pairs the oracle can compute;
plus GPU invariants that hold at any size (sibling isolation, power-of-two scaling,
run-to-run determinism, all bit-exact) and edge cases (single-node trees, an empty batch,
a 1024-node tree, a 128-node chain, oversized bank rows, empty commits)."""
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


MODES = ["chain", "ut", "fused"]


def _full_case(torch, name, steps, n_samples, seed, mode="chain"):
    """Run `steps` verify+commit steps of a full-size preset, then flush; check sampled pairs.
    In the fused form q, k and v come from the conv of the preset's x (3 H d channels), and
    the oracle is the prologue followed by the tree verify."""
    c = synth.WORKLOADS[name]
    H, d, C, dtype, Ly = c["H"], c["d"], c["Cch"], c["dtype"], c["Ly"]
    trees = workload.workload_trees(name)
    b = gh.Batch(trees, Ly, H, d, C, mode=mode, conv_dtype=dtype)
    S0, X0 = workload.host_initial_state(name, range(Ly), b.S)
    W = workload.host_weights(name, range(Ly))
    b.set_state(S0, X0)
    Wd = workload._to_torch(W, dtype, "cuda")
    rng = np.random.default_rng(seed)
    pairs = sorted({(int(rng.integers(Ly)), int(rng.integers(b.S))) for _ in range(n_samples)})
    committed = {p: S0[p[0], p[1]].astype(np.float64) for p in pairs}
    window = {p: X0[p[0], p[1]].astype(np.float64) for p in pairs}
    for step in range(steps):
        h = workload.host_step_inputs(name, step, trees, range(Ly))
        inp = workload.StepInputs(**{k: workload._to_torch(v, dtype, "cuda") for k, v in h.items()})
        role_before = b.layers.role_host.copy()
        b.step(inp, Wd)
        torch.cuda.synchronize()
        refs = {}
        for (l, s) in pairs:
            sl = slice(b.offs[s], b.offs[s + 1])
            h64 = {k: workload.widen(v[l, sl], dtype) for k, v in h.items()}
            gh.assert_state(gh.to_np(b.layers.state[l, s]), committed[(l, s)], mode=mode,
                            what=f"committed layer {l} seq {s} step {step}")
            assert np.array_equal(gh.to_np(b.layers.conv_state[l, s]),
                                  window[(l, s)].astype(np.float32))
            r = gh.oracle_pair(trees[s], committed[(l, s)], window[(l, s)],
                               workload.widen(W[l], dtype), h64, mode, H, d)
            gh.assert_outputs(gh.to_np(b.out[l, sl]), r["o"], mode=mode,
                              what=f"o layer {l} seq {s}")
            if r["y"] is not None:
                gh.assert_outputs(gh.to_np(b.y[l, sl]), r["y"], mode=mode, quantity="conv y",
                                  what=f"y layer {l} seq {s}")
            gh.assert_bank_rows(b, l, s, 1 - role_before[s], range(len(trees[s])), r["k"],
                                r["u"], r["lg"])
            xb = gh.to_np(b.layers.bank_x[1 - role_before[s]][l, s][:len(trees[s])])
            assert np.array_equal(xb, h64["x"]), f"banked conv inputs layer {l} seq {s}"
            refs[(l, s)] = (r, h64)
        paths = [synth.workload_path(name, step, s, trees[s]) for s in range(b.S)]
        b.commit(inp, paths, Wd)
        for (l, s) in pairs:
            r, h64 = refs[(l, s)]
            k, v = r["kv"]
            committed[(l, s)] = ogdn.replay(committed[(l, s)], k, v, h64["beta"], h64["gate"],
                                            paths[s])
            window[(l, s)] = oconv.commit_window(window[(l, s)], h64["x"], paths[s])
    b.flush()
    torch.cuda.synchronize()
    for (l, s) in pairs:
        gh.assert_state(gh.to_np(b.layers.state[l, s]), committed[(l, s)], mode=mode,
                        what=f"flush {l} {s}")
        assert np.array_equal(gh.to_np(b.layers.conv_state[l, s]), window[(l, s)].astype(np.float32))


@pytest.mark.parametrize("mode", MODES)
def test_batched_32x48_full_size(torch_cuda, mode):
    """The benchmarked workload: 32 sequences x 48 layers x 48 heads x 128, 22-node top-4
    trees, two verify+commit steps (the second folds the first's accepted paths), flush."""
    _full_case(torch_cuda, "batched", steps=2, n_samples=6, seed=31, mode=mode)


@pytest.mark.parametrize("mode", MODES)
def test_wide_deep_64_node_trees_full_size(torch_cuda, mode):
    """64-node top-8 trees of depth up to 16, batch 8, 48 layers: long heavy chains and
    many sibling boundaries."""
    _full_case(torch_cuda, "wide-deep", steps=2, n_samples=4, seed=41, mode=mode)


@pytest.mark.parametrize("mode", MODES)
def test_pure_16_node_chains_full_size(torch_cuda, mode):
    """Batch 8 of 16-node pure chains (block-diffusion draft blocks), 48 layers: every
    acceptance is in order, so commits only swap bank roles."""
    _full_case(torch_cuda, "chain16", steps=2, n_samples=4, seed=51, mode=mode)


# ---------------------------------------------------------------------------------------
# invariants at the one-layer 48-head shape
# ---------------------------------------------------------------------------------------

def _one_layer(torch, h, S0, trees, dtype="bf16", mode="chain", X0=None, W=None):
    """One verify of the one-layer workload.  The q/k/v forms read h's q, k, v; the fused form
    reads its conv inputs x (3 H d channels) with the window X0 and weights W."""
    fused = mode == "fused"
    C = 3 * 48 * 128 if fused else 0
    b = gh.Batch(trees, 1, 48, 128, C, mode=mode, conv_dtype=dtype)
    b.set_state(S0[None], X0[None] if fused else None)
    keep = ("beta", "gate", "x") if fused else ("q", "k", "v", "beta", "gate")
    dev = {k: workload._to_torch(v, dtype, "cuda") for k, v in h.items() if k in keep}
    inp = workload.StepInputs(**{k: dev.get(k) for k in ("q", "k", "v", "beta", "gate", "x")})
    b.step(inp, workload._to_torch(W[None], dtype, "cuda") if fused else None)
    torch.cuda.synchronize()
    return b


def _one_layer_inputs():
    """Trees, step-0 inputs (q, k, v, beta, gate, x), S0, X0 and W of the one-layer workload."""
    c = synth.WORKLOADS["one-layer"]
    trees = workload.workload_trees("one-layer")
    h = workload.host_step_inputs("one-layer", 0, trees, range(1))
    S0 = synth.initial_state(c["seed"], 0, 0, 48, 128)
    X0 = synth.initial_conv_state(c["seed"], 0, 0, c["Cch"], 4)
    W = synth.conv_weight(c["seed"], 0, c["Cch"], 4, c["dtype"])
    return trees, h, S0, X0, W


@pytest.mark.parametrize("mode", MODES)
def test_sibling_isolation_bit_identical(torch_cuda, mode):
    """Changing every input of one node changes its subtree's outputs and leaves every other
    node's output bit-identical (same schedule, same inputs elsewhere).  The q/k/v forms get a
    new q, k, v and beta at the node; the fused form a new raw conv input row x (all 3 H d
    channels) and beta, which reaches the node's subtree through both the conv window and the
    state."""
    trees, h, S0, X0, W = _one_layer_inputs()
    parent = trees[0]
    run = lambda hh: gh.to_np(_one_layer(torch_cuda, hh, S0, trees, mode=mode, X0=X0,
                                         W=W).out[0])
    base = run(h)
    for m in (3, 13, 17):
        h2 = {k: v.copy() for k, v in h.items()}
        for k in ("x",) if mode == "fused" else ("q", "k", "v"):
            h2[k][0, m] = synth.f32_to_bf16(-synth.bf16_to_f32(h2[k][0, m]))
        h2["beta"][0, m] = synth.f32_to_bf16(0.5 * synth.bf16_to_f32(h2["beta"][0, m]))
        out = run(h2)
        sub = {n for n in range(len(parent)) if m in ogdn.root_path(parent, n)}
        for n in range(len(parent)):
            if n in sub:
                assert not np.array_equal(out[n], base[n]), (m, n)
            else:
                assert np.array_equal(out[n], base[n]), (m, n)


# forms that take q, k, v as inputs (the fused form's v = SiLU(conv) is not linear in x, and
# it needs d = 128 and bf16)
QKV_MODES = ["chain", "ut"]


@pytest.mark.parametrize("mode", QKV_MODES)
def test_power_of_two_scaling_bit_exact(torch_cuda, mode):
    """Scaling the committed state and every v by 2 scales outputs, residual vectors and
    boundary-derived states by exactly 2 (no rounding difference anywhere)."""
    trees, h, S0, _, _ = _one_layer_inputs()
    b1 = _one_layer(torch_cuda, h, S0, trees, mode=mode)
    h2 = {k: v.copy() for k, v in h.items()}
    h2["v"] = synth.f32_to_bf16(2 * synth.bf16_to_f32(h2["v"]))
    b2 = _one_layer(torch_cuda, h2, 2 * S0, trees, mode=mode)
    assert torch_cuda.equal(b2.out, 2 * b1.out)
    assert torch_cuda.equal(b2.layers.bank_u[1], 2 * b1.layers.bank_u[1])
    assert torch_cuda.equal(b2.layers.bank_k[1], b1.layers.bank_k[1])


@pytest.mark.parametrize("mode", MODES)
def test_run_to_run_deterministic(torch_cuda, mode):
    trees, h, S0, X0, W = _one_layer_inputs()
    b1 = _one_layer(torch_cuda, h, S0, trees, mode=mode, X0=X0, W=W)
    b2 = _one_layer(torch_cuda, h, S0, trees, mode=mode, X0=X0, W=W)
    assert torch_cuda.equal(b1.out, b2.out)
    for name in ("bank_k", "bank_u", "bank_lg"):
        assert torch_cuda.equal(getattr(b1.layers, name)[1], getattr(b2.layers, name)[1])


# ---------------------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------------------

def _edge_run(torch, trees, H, d, C, steps_paths, cfg_id, max_nodes=None, dtype="f32",
              mode="chain"):
    b = gh.Batch(trees, 1, H, d, C, max_nodes=max_nodes, mode=mode, conv_dtype=dtype)
    S0 = np.stack([synth.initial_state(cfg_id, 0, s, H, d) for s in range(b.S)])
    X0 = np.stack([synth.initial_conv_state(cfg_id, 0, s, C, 4) for s in range(b.S)])
    W = synth.conv_weight(cfg_id, 0, C, 4, dtype)
    b.set_state(S0[None], X0[None])
    Wd = workload._to_torch(W[None], dtype, "cuda")
    committed = [S0[s].astype(np.float64) for s in range(b.S)]
    window = [X0[s].astype(np.float64) for s in range(b.S)]
    for step, paths in enumerate(steps_paths):
        hh = gh.tiny_inputs(trees, step, H, d, C, dtype, cfg_id)
        h64 = gh.widen_inputs(hh, dtype)
        inp = gh.to_device(hh, dtype)
        b.step(inp, Wd)
        torch.cuda.synchronize()
        o_gpu, y_gpu = gh.to_np(b.out[0]), gh.to_np(b.y[0])
        for s in range(b.S):
            sl = slice(b.offs[s], b.offs[s + 1])
            o, _ = ogdn.verify(trees[s], committed[s], h64["q"][0, sl], h64["k"][0, sl],
                               h64["v"][0, sl], h64["beta"][0, sl], h64["gate"][0, sl],
                               keep_states=False)
            gh.assert_outputs(o_gpu[sl], o, what=f"o seq {s}")
            y = oconv.tree_conv(trees[s], window[s], h64["x"][0, sl], workload.widen(W, dtype))
            gh.assert_outputs(y_gpu[sl], y, what=f"y seq {s}")
            committed[s] = ogdn.replay(committed[s], h64["k"][0, sl], h64["v"][0, sl],
                                       h64["beta"][0, sl], h64["gate"][0, sl], paths[s])
            window[s] = oconv.commit_window(window[s], h64["x"][0, sl], paths[s])
        b.commit(inp, paths, Wd)
    b.flush()
    torch.cuda.synchronize()
    gh.assert_state(gh.to_np(b.layers.state[0]), np.stack(committed), what="flush")
    assert np.array_equal(gh.to_np(b.layers.conv_state[0]), np.stack(window).astype(np.float32))


@pytest.mark.parametrize("mode", QKV_MODES)
def test_single_node_trees(torch_cuda, mode):
    """Trees of one node (the root only), with accept-nothing and accept-root steps."""
    trees = [np.array([-1], dtype=np.int32)] * 5
    steps = [[[0], [], [0], [], [0]], [[], [0], [0], [], []], [[0]] * 5]
    _edge_run(torch_cuda, trees, 2, 16, 8, steps, 92, mode=mode)


def test_largest_tree_1024_nodes(torch_cuda):
    """A 1024-node tree (the largest accepted), deep and bushy, d = 16."""
    rng = np.random.default_rng(9)
    tree = synth.make_tree(rng, 1024, 6, 40)
    steps = [[synth.random_path(rng, tree, 30)], [synth.random_path(rng, tree, 7)]]
    _edge_run(torch_cuda, [tree], 1, 16, 8, steps, 93)


def test_long_chain_d128_and_padded_banks(torch_cuda):
    """A 128-node chain at d = 128 (many staging blocks in one workgroup), next to a branched
    tree, with bank rows padded beyond the largest tree."""
    rng = np.random.default_rng(10)
    trees = [np.arange(-1, 127, dtype=np.int32), synth.make_tree(rng, 40, 4, 12)]
    steps = [[np.arange(100), synth.random_path(rng, trees[1], 5)],
             [np.arange(3), synth.random_path(rng, trees[1], 9)]]
    _edge_run(torch_cuda, trees, 3, 128, 16, steps, 94, max_nodes=160, dtype="bf16")


def _ut_refused(torch, trees, seed):
    b = gh.Batch(trees, 1, 2, 128, 0, mode="ut")
    h = gh.tiny_inputs(trees, 0, 2, 128, 4, "bf16", seed)
    h.pop("x")
    inp = workload.StepInputs(**{k: workload._to_torch(v, "bf16", "cuda") for k, v in h.items()},
                              x=None)
    before = b.out.clone()
    with pytest.raises(binding.GdnError) as e:
        binding.tree_verify_ut(b.vargs(inp, 0), b.image, b.dev_image)
    torch.cuda.synchronize()
    assert torch.equal(before, b.out)  # refused before any launch
    return e.value


def test_ut_rejects_trees_beyond_its_budgets(torch_cuda):
    """The UT path keeps a whole tree in one workgroup's LDS and reads its record plan from
    the schedule: a 128-node chain needs 8256 records, above the plan's 32 per node; a wide
    150-node tree has a plan but needs more than 160 KiB of LDS.  Both are refused before
    any launch."""
    e = _ut_refused(torch_cuda, [np.arange(-1, 127, dtype=np.int32)], 95)
    assert e.status == -1 and "plan" in str(e)
    rng = np.random.default_rng(95)
    e = _ut_refused(torch_cuda, [synth.make_tree(rng, 150, 8, 12)], 96)
    assert e.status == -1 and "LDS" in str(e)


def test_ut_largest_fitting_tree_64_nodes_d128(torch_cuda):
    """64-node top-8 trees of depth <= 16 at d = 128, bf16 (close to the UT path's LDS
    budget), next to a 16-node chain."""
    rng = np.random.default_rng(12)
    trees = [synth.make_tree(rng, 64, 8, 16), np.arange(-1, 15, dtype=np.int32)]
    steps = [[synth.random_path(rng, trees[0], 12), np.arange(10)],
             [synth.random_path(rng, trees[0], 3), np.arange(16)]]
    _edge_run(torch_cuda, trees, 2, 128, 16, steps, 96, dtype="bf16", mode="ut")


def test_ut_deep_chain_level_inverse(torch_cuda):
    """A 24-node chain (depth 23: past the per-lane register form of the tree inverse, which
    stops at depth 16, so the level-by-level form runs) next to a branched tree, d = 128,
    bf16."""
    rng = np.random.default_rng(13)
    trees = [np.arange(-1, 23, dtype=np.int32), synth.make_tree(rng, 30, 4, 10)]
    steps = [[np.arange(20), synth.random_path(rng, trees[1], 6)],
             [np.arange(24), synth.random_path(rng, trees[1], 3)]]
    _edge_run(torch_cuda, trees, 2, 128, 16, steps, 97, dtype="bf16", mode="ut")


def test_empty_batch_is_a_no_op(torch_cuda):
    import ctypes
    image = binding.hld_schedule([])
    L = binding.lib()
    va, ca = binding.VerifyArgs(), binding.ConvArgs()
    va.n_heads, va.head_dim, va.max_nodes, va.n_layers, va.in_dtype = 1, 16, 1, 1, 0
    ca.channels, ca.width, ca.max_nodes, ca.n_layers = 4, 4, 1, 1
    stream = torch_cuda.cuda.current_stream().cuda_stream
    dev = torch_cuda.zeros(32, dtype=torch_cuda.int32, device="cuda")
    assert L.gdn_tree_verify(ctypes.byref(va), binding._ptr(image), dev.data_ptr(), stream) == 0
    assert L.gdn_tree_conv(ctypes.byref(ca), binding._ptr(image), dev.data_ptr(), stream) == 0
    pend = np.zeros(1, dtype=np.int32)
    assert L.gdn_flush(ctypes.byref(va), ctypes.byref(ca), binding._ptr(pend), stream) == 0
    torch_cuda.cuda.synchronize()

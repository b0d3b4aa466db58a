"""GPU parity with zero and tiny gates on the accepted paths, through every verify form (chain,
tree-masked UT, fused conv -> verify), against the float64 oracle.

A gate g = 0 (a bf16 gate can underflow to zero) erases the state before its token; its banked
log gate is -inf, and the next verify's deferred fold must still reach the oracle's finite
state (SpecLA guide, mechanisms 3 and 4: the log decay gate is banked and folded).  A gate of
1e-30 keeps a trace of 1e-30 of the past.  Both sit on the paths accepted at step 0, so step 1
folds them; step 1's own paths carry a zero gate at a root, and the final flush folds those.
"""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload
from oracle import conv as oconv
from oracle import gdn as ogdn

import gpu_harness as gh

pytestmark = pytest.mark.gpu

H, D = 2, 128
C = 3 * H * D


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def _set_gate(h, node, head, value):
    """gate[0, node, head] = value, as the bf16 (or fp32) the device reads."""
    h["gate"][0, node, head] = synth.f32_to_bf16(np.array([value], np.float32))[0]


@pytest.mark.parametrize("mode", ["chain", "ut", "fused"])
def test_zero_and_tiny_gates_on_accepted_paths(torch_cuda, mode):
    trees = [synth.TINY_TREE, synth.TINY_CHAIN]
    cfg = 70
    b = gh.Batch(trees, 1, H, D, C, mode=mode, conv_dtype="bf16")
    S0 = np.stack([synth.initial_state(cfg, 0, s, H, D) for s in range(b.S)])
    X0 = np.stack([synth.initial_conv_state(cfg, 0, s, C, 4) for s in range(b.S)])
    W = synth.conv_weight(cfg, 0, C, 4, "bf16")
    b.set_state(S0[None], X0[None])
    Wd = workload._to_torch(W[None], "bf16", "cuda")
    W64 = workload.widen(W, "bf16")
    committed = [S0[s].astype(np.float64) for s in range(b.S)]
    window = [X0[s].astype(np.float64) for s in range(b.S)]
    offs = b.offs
    steps = [
        # tiny tree: deepest leaf [0,1,3,6] with g = 0 at node 1 (both heads) and 1e-30 at
        # node 3 (head 0); chain: all 8 nodes with 1e-30 at node 2 and g = 0 at node 5
        ([[0, 1, 3, 6], list(range(8))],
         [(0, 1, 0, 0.0), (0, 1, 1, 0.0), (0, 3, 0, 1e-30), (1, 2, 0, 1e-30), (1, 2, 1, 1e-30),
          (1, 5, 0, 0.0), (1, 5, 1, 0.0)]),
        # step 1: zero gates at both roots (head 1) and 1e-30 at node 2 of the tiny tree
        ([[0, 2, 5], [0, 1, 2]],
         [(0, 0, 1, 0.0), (1, 0, 1, 0.0), (0, 2, 0, 1e-30)]),
    ]
    for step, (paths, gates) in enumerate(steps):
        h = gh.tiny_inputs(trees, step, H, D, C, "bf16", cfg)
        for s, node, head, g in gates:
            _set_gate(h, offs[s] + node, head, g)
        h64 = gh.widen_inputs(h, "bf16")
        assert np.count_nonzero(h64["gate"] == 0.0) >= 2
        inp = gh.to_device(h, "bf16")
        role_before = b.layers.role_host.copy()
        b.step(inp, Wd)
        torch_cuda.cuda.synchronize()
        S_gpu = gh.to_np(b.layers.state[0])
        assert np.all(np.isfinite(S_gpu)), "committed state not finite after the fold"
        gh.assert_state(S_gpu, np.stack(committed), what=f"fold @ {step}", mode=mode)
        assert np.array_equal(gh.to_np(b.layers.conv_state[0]),
                              np.stack(window).astype(np.float32))
        o_gpu = gh.to_np(b.out[0])
        assert np.all(np.isfinite(o_gpu))
        for s in range(b.S):
            sl = slice(offs[s], offs[s + 1])
            seq = {k: v[0, sl] for k, v in h64.items()}
            r = gh.oracle_pair(trees[s], committed[s], window[s], W64, seq, mode, H, D)
            gh.assert_outputs(o_gpu[sl], r["o"], what=f"o step {step} seq {s}", mode=mode)
            gh.assert_bank_rows(b, 0, s, 1 - role_before[s], range(len(trees[s])), r["k"],
                                r["u"], r["lg"])
            k, v = r["kv"]
            committed[s] = ogdn.replay(committed[s], k, v, seq["beta"], seq["gate"], paths[s])
            window[s] = oconv.commit_window(window[s], seq["x"], paths[s])
        b.commit(inp, paths, Wd)
    b.flush()
    torch_cuda.cuda.synchronize()
    S_gpu = gh.to_np(b.layers.state[0])
    assert np.all(np.isfinite(S_gpu))
    gh.assert_state(S_gpu, np.stack(committed), what="flush", mode=mode)
    assert np.array_equal(gh.to_np(b.layers.conv_state[0]), np.stack(window).astype(np.float32))

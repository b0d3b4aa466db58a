"""One launch over several layers is the same computation as one launch per layer: the conv
(grid over layers, two channels per thread or one) and the chain and tree-masked verifies give
bit-identical outputs, conv outputs, banks, windows and committed states either way, over two
steps with a commit between them (so the second step folds pending rows in every layer)."""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload

import gpu_harness as gh

pytestmark = pytest.mark.gpu

LY, H, D = 3, 2, 16


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def _inputs(trees, step, C, cfg):
    per = [gh.tiny_inputs(trees, step, H, D, C, "f32", cfg + layer) for layer in range(LY)]
    return {name: np.concatenate([p[name] for p in per]) for name in per[0]}


def _run(torch, trees, mode, C, one_call):
    cfg = 95
    b = gh.Batch(trees, LY, H, D, C, mode=mode)
    S0 = np.stack([np.stack([synth.initial_state(cfg, l, s, H, D) for s in range(b.S)])
                   for l in range(LY)])
    X0 = np.stack([np.stack([synth.initial_conv_state(cfg, l, s, C, 4) for s in range(b.S)])
                   for l in range(LY)])
    W = np.stack([synth.conv_weight(cfg, l, C, 4, "f32") for l in range(LY)])
    b.set_state(S0, X0)
    Wd = workload._to_torch(W, "f32", "cuda")
    ws = torch.zeros(max(binding.verify_workspace_bytes(b.image, H, D, LY) // 4, 1),
                     device="cuda")
    rng = np.random.default_rng(3)
    snaps = []
    for step in range(2):
        inp = gh.to_device(_inputs(trees, step, C, cfg), "f32")
        if one_call:
            ca = binding.conv_args(b.image, b.layers, inp.x, Wd, b.y, layer_begin=0, n_layers=LY)
            binding.tree_conv(ca, b.image, b.dev_image)
            va = binding.verify_args(b.image, b.layers, inp.q, inp.k, inp.v, inp.beta, inp.gate,
                                     b.out, ws, layer_begin=0, n_layers=LY)
            if mode == "ut":
                binding.tree_verify_ut(va, b.image, b.dev_image)
            else:
                binding.tree_verify(va, b.image, b.dev_image)
        else:
            b.step(inp, Wd)
        torch.cuda.synchronize()
        lay = b.layers
        snaps.append({name: gh.to_np(t).copy() for name, t in [
            ("out", b.out), ("y", b.y), ("state", lay.state), ("conv_state", lay.conv_state),
            *[(f"{n}{r}", getattr(lay, n)[r]) for n in ("bank_k", "bank_u", "bank_lg", "bank_x")
              for r in range(2)]]})
        paths = [synth.random_path(rng, t, int(rng.integers(1, synth.node_depths(t).max() + 2)))
                 for t in trees]
        b.commit(inp, paths, Wd)
        torch.cuda.synchronize()
    return snaps


@pytest.mark.parametrize("C", [16, 15])
@pytest.mark.parametrize("mode", ["chain", "ut"])
def test_one_call_over_layers_equals_one_call_per_layer(torch_cuda, mode, C):
    rng = np.random.default_rng(9)
    trees = [synth.TINY_TREE, synth.TINY_CHAIN, synth.make_tree(rng, 20, 3, 8)]
    a = _run(torch_cuda, trees, mode, C, one_call=False)
    b = _run(torch_cuda, trees, mode, C, one_call=True)
    for step, (sa, sb) in enumerate(zip(a, b)):
        for name in sa:
            assert np.array_equal(sa[name], sb[name], equal_nan=True), f"{name} @ step {step}"

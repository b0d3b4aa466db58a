"""gdn_tree_verify_noalloc (the chain verify with its boundary states in the library's fixed
device scratch, for callers that cannot allocate) against gdn_tree_verify (boundary states in a
caller workspace), through the C ABI: two calls in a row on one GPU, the second with a smaller
batch, each compared with the workspace entry point (bit-identical: the same kernels) and with
the float64 oracle (outputs within 1e-3 normwise, committed states within 1e-5 Frobenius);
then a batch whose boundary states exceed the scratch is refused before any launch."""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload

import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def _pair(trees, H, d, dtype, cfg, step, max_nodes=None):
    """Two identical batches (workspace / no-alloc) with the same seeded state and inputs."""
    out = []
    for _ in range(2):
        b = gh.Batch(trees, 1, H, d, 0, max_nodes=max_nodes, mode="chain")
        S0 = np.stack([synth.initial_state(cfg, 0, s, H, d) for s in range(b.S)])
        b.set_state(S0[None])
        out.append(b)
    h = gh.tiny_inputs(trees, step, H, d, 4, dtype, cfg)
    h.pop("x")
    return out, h, S0


def _check(torch, trees, H, d, dtype, cfg):
    (bw, bn), h, S0 = _pair(trees, H, d, dtype, cfg, 0)
    inp = workload.StepInputs(**{k: workload._to_torch(v, dtype, "cuda") for k, v in h.items()},
                              x=None)
    assert int(bw.view["n_boundaries"]) > 0
    binding.tree_verify(bw.vargs(inp, 0), bw.image, bw.dev_image)
    va = bn.vargs(inp, 0)
    va.workspace = None  # the no-alloc call uses no caller workspace
    binding.tree_verify_noalloc(va, bn.image, bn.dev_image)
    torch.cuda.synchronize()
    assert torch.equal(bw.out, bn.out)
    for name in ("bank_k", "bank_u", "bank_lg"):
        assert torch.equal(getattr(bw.layers, name)[1], getattr(bn.layers, name)[1]), name
    h64 = gh.widen_inputs(h, dtype)
    o = gh.to_np(bn.out[0])
    for s in range(bn.S):
        r = gh.oracle_pair(trees[s], S0[s].astype(np.float64), None, None,
                           {k: v[0, bn.offs[s]:bn.offs[s + 1]] for k, v in h64.items()},
                           "chain", H, d)
        gh.assert_outputs(o[bn.offs[s]:bn.offs[s + 1]], r["o"], mode="noalloc",
                          what=f"o seq {s}")
    # commit the same paths in both, then a second verify that folds them
    paths = [synth.deepest_leaf_path(t) for t in trees]
    for b in (bw, bn):
        b.commit(inp, paths)
    h2 = gh.tiny_inputs(trees, 1, H, d, 4, dtype, cfg)
    h2.pop("x")
    inp2 = workload.StepInputs(**{k: workload._to_torch(v, dtype, "cuda") for k, v in h2.items()},
                               x=None)
    binding.tree_verify(bw.vargs(inp2, 0), bw.image, bw.dev_image)
    va = bn.vargs(inp2, 0)
    va.workspace = None
    binding.tree_verify_noalloc(va, bn.image, bn.dev_image)
    torch.cuda.synchronize()
    assert torch.equal(bw.out, bn.out)
    assert torch.equal(bw.layers.state, bn.layers.state)
    for s in range(bn.S):
        sl = slice(bn.offs[s], bn.offs[s + 1])
        seq = {k: v[0, sl] for k, v in h64.items()}  # step 0's inputs: the folded path's
        ref = gh.ogdn.replay(S0[s].astype(np.float64), seq["k"], seq["v"], seq["beta"],
                             seq["gate"], paths[s])
        gh.assert_state(gh.to_np(bn.layers.state[0, s]), ref, mode="noalloc",
                        what=f"folded state seq {s}")


def test_noalloc_matches_workspace_verify_twice_then_smaller(torch_cuda):
    """Call 1: the one-layer workload's 22-node top-4 tree at 48 heads x 128, bf16 (its
    boundary states fill part of the scratch).  Call 2, right after on the same GPU: the tiny
    7-node tree and the 8-node chain at 2 heads x 128 (fewer boundary states: the second call
    reads only what it wrote)."""
    _check(torch_cuda, workload.workload_trees("one-layer"), 48, 128, "bf16", 81)
    _check(torch_cuda, [synth.TINY_TREE, synth.TINY_CHAIN], 2, 128, "bf16", 82)


def test_noalloc_refuses_batches_beyond_its_scratch(torch_cuda):
    """The batched workload's 32 trees at 48 heads need ~190 boundary tiles x 48 heads of
    64 KiB, far beyond the 32 MiB scratch: GDN_ECAPACITY, nothing launched or written."""
    trees = workload.workload_trees("batched")
    b = gh.Batch(trees, 1, 48, 128, 0, mode="chain")
    need = binding.verify_workspace_bytes(b.image, 48, 128, 1)
    assert need > 32 << 20
    h = gh.tiny_inputs(trees, 0, 48, 128, 4, "bf16", 83)
    h.pop("x")
    inp = workload.StepInputs(**{k: workload._to_torch(v, "bf16", "cuda") for k, v in h.items()},
                              x=None)
    before = b.out.clone()
    va = b.vargs(inp, 0)
    va.workspace = None
    with pytest.raises(binding.GdnError) as e:
        binding.tree_verify_noalloc(va, b.image, b.dev_image)
    torch_cuda.cuda.synchronize()
    assert e.value.status == -4 and "scratch" in str(e.value)
    assert torch_cuda.equal(before, b.out)

"""GPU parity of the chunked prefill (gdn_prefill) against the oracle's sequential prefill.

Ragged batches cover an empty sequence, single tokens, chunk boundaries (16, 32), ragged tails
and a few hundred tokens; a full-width case runs 48 heads over 1024-token sequences and checks
sampled heads; zero and 1e-30 gates sit at chunk starts, ends and inside chunks.  Bars: per-token output vectors max-relative 1e-3, final states relative
Frobenius 1e-5 (the same bars as the tree verify).
"""
import numpy as np
import pytest

from gated_deltanet_tree_amd import binding, synth, workload
from oracle import gdn as ogdn
import gpu_harness as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    return torch


def _run(torch, lengths, H, seed, n_layers=1, check_heads=None, layer_begin=0, gate_edit=None):
    d = 128
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S, T = len(lengths), int(offs[-1])
    Ly = layer_begin + n_layers
    host = {k: [] for k in ("q", "k", "v", "beta", "gate")}
    for layer in range(Ly):
        per = [synth.node_inputs(90 + seed, 0, layer, b, max(n, 1), H, d, "bf16")
               for b, n in enumerate(lengths)]
        for key in host:
            host[key].append(np.concatenate([p[key][:n] for p, n in zip(per, lengths)])
                             if T else np.zeros((0,) + per[0][key].shape[1:], per[0][key].dtype))
    host = {k: np.stack(v) for k, v in host.items()}
    if gate_edit is not None:  # [(layer, token, head, value)] written as bf16 gates
        for layer, t, h, value in gate_edit(offs):
            host["gate"][layer, t, h] = synth.f32_to_bf16(np.array([value], np.float32))[0]
    S0 = np.stack([np.stack([synth.initial_state(90 + seed, layer, b, H, d) for b in range(S)])
                   for layer in range(Ly)]).astype(np.float32)
    dev = {k: workload._to_torch(v, "bf16", "cuda") for k, v in host.items()}
    state = torch.from_numpy(S0.copy()).cuda()
    out = torch.full((Ly, max(T, 1), H, d), float("nan"), device="cuda")
    dev_offs = torch.from_numpy(offs).cuda()
    a = binding.prefill_args(offs, dev_offs, dev["q"], dev["k"], dev["v"], dev["beta"],
                             dev["gate"], state, out, layer_begin=layer_begin,
                             n_layers=n_layers)
    binding.prefill(a)
    torch.cuda.synchronize()
    o_gpu, S_gpu = gh.to_np(out), gh.to_np(state)
    heads = range(H) if check_heads is None else check_heads
    for layer in range(layer_begin, Ly):
        for b, n in enumerate(lengths):
            sl = slice(offs[b], offs[b + 1])
            w = {k: workload.widen(v[layer, sl], "bf16") for k, v in host.items()}
            hs = list(heads)
            o_ref, S_ref = ogdn.prefill(S0[layer, b][hs].astype(np.float64), w["q"][:, hs],
                                        w["k"][:, hs], w["v"][:, hs], w["beta"][:, hs],
                                        w["gate"][:, hs])
            if n:
                gh.assert_outputs(o_gpu[layer, sl][:, hs], o_ref, what=f"o seq {b} (n={n})")
            gh.assert_state(S_gpu[layer, b][hs], S_ref, what=f"state seq {b} (n={n})")
    for layer in range(0, layer_begin):  # layers outside the call are untouched
        assert np.array_equal(S_gpu[layer], S0[layer])
    return o_gpu, S_gpu


def test_ragged_lengths_and_chunk_boundaries(torch_cuda):
    _run(torch_cuda, [0, 1, 5, 16, 17, 32, 33, 100, 255], H=3, seed=0)


def test_two_layers_second_only(torch_cuda):
    _run(torch_cuda, [40, 7], H=2, seed=1, n_layers=1, layer_begin=1)


def test_two_layers_in_one_call(torch_cuda):
    _run(torch_cuda, [64, 19, 0], H=2, seed=2, n_layers=2)


def test_full_width_long_sequences_sampled_heads(torch_cuda):
    """48 heads x 4 sequences of 1024 tokens (one layer), heads 0, 17 and 47 checked."""
    _run(torch_cuda, [1024, 1000, 1024, 513], H=48, seed=3, check_heads=[0, 17, 47])


def test_zero_and_tiny_gates(torch_cuda):
    """Gates of 0 and 1e-30 (a bf16 gate can underflow to zero) at the first token, inside a
    chunk, at a chunk's first and last token, in a run, at the last token; a sequence whose
    gates are all 0 (head 0) or all 1 (head 1).  The chunk's gate products are exact products,
    so a zero gate erases the state before its token exactly as the oracle's recurrence does."""
    lengths = [40, 33, 16, 1]

    def edit(offs):
        s0, s1, s2, s3 = (int(o) for o in offs[:4])
        ed = [(0, s0 + 0, 0, 0.0), (0, s0 + 5, 0, 1e-30), (0, s0 + 5, 1, 1e-30),
              (0, s0 + 16, 1, 0.0), (0, s0 + 31, 0, 1e-30), (0, s0 + 39, 1, 0.0)]
        ed += [(0, s0 + t, 0, 0.0) for t in (17, 18, 19)]
        ed += [(0, s1 + 15, 0, 1e-30), (0, s1 + 15, 1, 0.0), (0, s1 + 32, 0, 0.0)]
        ed += [(0, s2 + t, 0, 0.0) for t in range(16)] + [(0, s2 + t, 1, 1.0) for t in range(16)]
        ed += [(0, s3, 0, 0.0), (0, s3, 1, 1e-30)]
        return ed

    o, S = _run(torch_cuda, lengths, H=2, seed=6, gate_edit=edit)
    assert np.isfinite(o[0, :sum(lengths)]).all() and np.isfinite(S).all()


def test_run_to_run_deterministic(torch_cuda):
    o1, s1 = _run(torch_cuda, [50, 31], H=2, seed=4)
    o2, s2 = _run(torch_cuda, [50, 31], H=2, seed=4)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_rejects_bad_arguments(torch_cuda):
    torch = torch_cuda
    offs = np.array([0, 4], dtype=np.int32)
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((1, 4, 1), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((1, 1, 1, 128, 128), device="cuda")
    out = torch.zeros((1, 4, 1, 128), device="cuda")
    a = binding.prefill_args(offs, torch.from_numpy(offs).cuda(), q, q, q, g, g, st, out)
    a.host_offsets = np.array([0, 5], dtype=np.int32)  # does not end at n_tokens
    with pytest.raises(binding.GdnError):
        binding.prefill(a)
    a.host_offsets = offs
    a.in_dtype = binding.GDN_F32
    with pytest.raises(binding.GdnError):
        binding.prefill(a)
    a.in_dtype = binding.GDN_BF16
    a.head_dim = 64
    with pytest.raises(binding.GdnError):
        binding.prefill(a)

"""Device tensors for the synthetic workloads (plumbing: numpy draws -> torch on ROCm).

Nothing here computes any part of the method; it lays the seeded draws of `synth` out in the
layouts that include/gdn_tree.h documents:
    q, k, v [Ly][T][H][d], beta, gate [Ly][T][H], x [Ly][T][Cch], weight [Ly][Cch][4],
    state [Ly][S][H][d][d], conv_state [Ly][S][Cch][3]
where T is the batch's total node count and node ids are global (seq_offsets[b] + local).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import synth


@dataclass
class StepInputs:
    q: object
    k: object
    v: object
    beta: object
    gate: object
    x: object


def workload_trees(name: str) -> list:
    """The candidate trees of a preset's sequences."""
    return [synth.workload_tree(name, b) for b in range(synth.WORKLOADS[name]["Bs"])]


def _to_torch(a: np.ndarray, dtype: str, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_step_inputs(name: str, step: int, trees: list, layers: range, cfg=None,
                     threads: int = 8) -> dict:
    """numpy arrays of one step's node inputs for the given layers (all sequences) of a
    preset (`cfg` overrides its fields)."""
    c = dict(synth.WORKLOADS[name], **(cfg or {}))
    seed = c["seed"]
    H, d, C, dtype = c["H"], c["d"], c["Cch"], c["dtype"]
    sizes = [len(t) for t in trees]
    T = int(sum(sizes))
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    el = np.uint16 if dtype == "bf16" else np.float32
    Ly = len(layers)
    out = {name: np.empty((Ly, T, H, d), dtype=el) for name in ("q", "k", "v")}
    out.update({name: np.empty((Ly, T, H), dtype=el) for name in ("beta", "gate")})
    out["x"] = np.empty((Ly, T, C), dtype=el)

    def fill(job):
        li, layer, b = job
        n = sizes[b]
        sl = slice(offs[b], offs[b] + n)
        vals = synth.node_inputs(seed, step, layer, b, n, H, d, dtype)
        for name, arr in vals.items():
            out[name][li, sl] = arr
        out["x"][li, sl] = synth.conv_inputs(seed, step, layer, b, n, C, dtype)

    jobs = [(li, layer, b) for li, layer in enumerate(layers) for b in range(len(trees))]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, jobs))
    return out


def device_step_inputs(name: str, step: int, trees: list, layers: range, device="cuda",
                       cfg=None) -> StepInputs:
    c = dict(synth.WORKLOADS[name], **(cfg or {}))
    h = host_step_inputs(name, step, trees, layers, cfg)
    return StepInputs(**{k: _to_torch(v, c["dtype"], device) for k, v in h.items()})


def host_initial_state(name: str, layers: range, n_seqs: int, cfg=None, threads: int = 8):
    c = dict(synth.WORKLOADS[name], **(cfg or {}))
    H, d, C, seed = c["H"], c["d"], c["Cch"], c["seed"]
    state = np.empty((len(layers), n_seqs, H, d, d), dtype=np.float32)
    conv = np.empty((len(layers), n_seqs, C, 3), dtype=np.float32)

    def fill(job):
        li, layer, b = job
        state[li, b] = synth.initial_state(seed, layer, b, H, d)
        conv[li, b] = synth.initial_conv_state(seed, layer, b, C, 4)

    jobs = [(li, layer, b) for li, layer in enumerate(layers) for b in range(n_seqs)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, jobs))
    return state, conv


def host_weights(name: str, layers: range, cfg=None) -> np.ndarray:
    c = dict(synth.WORKLOADS[name], **(cfg or {}))
    return np.stack([synth.conv_weight(c["seed"], layer, c["Cch"], 4, c["dtype"]) for layer in layers])


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (bf16 bits or float32)."""
    return (synth.bf16_to_f32(a) if dtype == "bf16" else a).astype(np.float64)

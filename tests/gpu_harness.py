"""Shared pieces of the GPU parity tests: run verify/conv/commit through the C ABI and compare
with the float64 oracle under the stated tolerances.

Tolerances (fp32 state and accumulation, bf16 or fp32 inputs):
  outputs o and conv y, per vector r:  max|x - r| / max|r|          <= 1e-3
  committed state, per (layer, seq, head) tile:  ||S - R||_F / ||R||_F <= 1e-5
  banked k and conv inputs: bit-exact (widened copies of the inputs); in the fused form the
    key is the kernel's fp32 unit key: <= 1e-5 relative 2-norm per row
  banked u, per row:  ||x - r||_2 / ||r||_2 <= 1e-5
  banked ln g: within 4 ulp (fp32) of ln g (-inf exactly for a zero gate)
Every check records the largest error it saw (`record`); the session's maxima are printed at
the end of the run, per quantity and verify form.
"""
from __future__ import annotations

import numpy as np

from gated_deltanet_tree_amd import binding, synth, workload
from oracle import banks as obanks
from oracle import conv as oconv
from oracle import gdn as ogdn
from oracle import prologue

OUT_TOL = 1e-3
STATE_TOL = 1e-5
U_TOL = 1e-5
K_TOL = 1e-5  # fused form only: the banked key is computed (conv, SiLU, unit length) in fp32

# largest error seen per (quantity, verify form) over the session
MAX_ERR: dict = {}


def record(what: str, mode: str, err: float) -> float:
    key = (what, mode)
    MAX_ERR[key] = max(MAX_ERR.get(key, 0.0), float(err))
    return float(err)


def vec_rel(x, r, axis=-1):
    """Normwise max relative error per vector along `axis`."""
    num = np.max(np.abs(x - r), axis=axis)
    den = np.max(np.abs(r), axis=axis)
    return num / np.maximum(den, 1e-300)


def frob_rel(x, r):
    return np.sqrt(np.sum((x - r) ** 2, axis=(-2, -1))) / np.sqrt(np.sum(r ** 2, axis=(-2, -1)))


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, np.finfo(np.float32).tiny)))
    return 2.0 ** (e - 23)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


class Batch:
    """One batch of trees on the device with its schedule and layer buffers."""

    def __init__(self, trees, n_layers, H, d, C, max_nodes=None, device="cuda", mode="chain",
                 commit_mode="row-map", conv_dtype="f32"):
        """mode: "chain" = heavy-light chains in dependency waves (gdn_tree_verify),
        "ut" = tree-masked UT form in one launch (gdn_tree_verify_ut), "fused" = conv ->
        SiLU -> unit q/k -> tree-masked verify in one launch (gdn_tree_conv_verify; d = 128,
        bf16, C = 3 H d; q, k, v come from the conv of x, and no conv output is written).
        commit_mode: "row-map" (no copy) or "compact" (the guide's compaction)."""
        if mode == "fused":
            assert d == 128 and C == 3 * H * d and conv_dtype == "bf16", "fused form shape"
        import torch
        self.mode = mode
        self.commit_mode = commit_mode
        self.trees = [np.asarray(t, dtype=np.int32) for t in trees]
        self.image = binding.hld_schedule(self.trees)
        self.view = binding.schedule_view(self.image)
        self.dev_image = torch.from_numpy(self.image).to(device)
        self.S, self.T = len(trees), int(self.view["n_nodes"])
        self.offs = self.view["seq_offsets"].astype(int)
        self.Ly, self.H, self.d, self.C = n_layers, H, d, C
        self.max_nodes = max_nodes or max(len(t) for t in trees)
        self.layers = binding.alloc_layers(n_layers, self.S, H, d, self.max_nodes, C, device,
                                           conv_dtype=conv_dtype)
        ws = binding.verify_workspace_bytes(self.image, H, d, 1)
        self.workspace = torch.zeros(max(ws // 4, 1), device=device, dtype=torch.float32)
        self.out = torch.zeros((n_layers, self.T, H, d), device=device, dtype=torch.float32)
        self.y = torch.zeros((n_layers, self.T, max(C, 1)), device=device, dtype=torch.float32)
        self.device = device

    def set_state(self, state: np.ndarray, conv_state: np.ndarray | None = None):
        import torch
        self.layers.state.copy_(torch.from_numpy(np.ascontiguousarray(state, dtype=np.float32)))
        if conv_state is not None:
            self.layers.conv_state.copy_(torch.from_numpy(np.ascontiguousarray(conv_state,
                                                                               dtype=np.float32)))

    def vargs(self, inp, layer):
        return binding.verify_args(self.image, self.layers, inp.q, inp.k, inp.v, inp.beta,
                                   inp.gate, self.out, self.workspace, layer_begin=layer,
                                   n_layers=1)

    def cargs(self, inp, layer, weight):
        return binding.conv_args(self.image, self.layers, inp.x, weight, self.y,
                                 layer_begin=layer, n_layers=1)

    def fused_args(self, inp, layer, weight):
        va = binding.verify_args(self.image, self.layers, None, None, None, inp.beta, inp.gate,
                                 self.out, None, layer_begin=layer, n_layers=1)
        ca = binding.conv_args(self.image, self.layers, inp.x, weight, None, layer_begin=layer,
                               n_layers=1)
        return va, ca

    def step(self, inp, weight=None):
        """conv + verify for every layer, one layer per call (the model's dependency)."""
        for layer in range(self.Ly):
            if self.mode == "fused":
                va, ca = self.fused_args(inp, layer, weight)
                binding.tree_conv_verify(va, ca, self.image, self.dev_image)
                continue
            if self.C:
                binding.tree_conv(self.cargs(inp, layer, weight), self.image, self.dev_image)
            if self.mode == "ut":
                binding.tree_verify_ut(self.vargs(inp, layer), self.image, self.dev_image)
            else:
                binding.tree_verify(self.vargs(inp, layer), self.image, self.dev_image)

    def commit(self, inp, paths, weight=None):
        va = binding.verify_args(self.image, self.layers, None, None, None, None, None, None,
                                 None, 0, self.Ly)
        ca = binding.conv_args(self.image, self.layers, None, None, None, 0, self.Ly) \
            if self.C else None
        binding.commit_path(self.image, paths, self.layers, va, ca, mode=COMMIT_MODES[self.commit_mode])

    def flush(self):
        va = binding.verify_args(self.image, self.layers, None, None, None, None, None, None,
                                 None, 0, self.Ly)
        ca = binding.conv_args(self.image, self.layers, None, None, None, 0, self.Ly) \
            if self.C else None
        binding.flush(va, ca, self.layers)


def oracle_pair(parent, S0, X0, W64, seq: dict, mode: str, H: int, d: int) -> dict:
    """Oracle of one (layer, sequence) in verify form `mode`, from the widened inputs of the
    sequence (`seq`: q, k, v, beta, gate, x as [N, ...] float64).  Returns o, y (None in the
    fused form, which writes no conv output), the factors k, u, lg, and the k and v that a
    commit replays (the conv's in the fused form)."""
    beta, gate = seq["beta"], seq["gate"]
    if mode == "fused":
        o, q, k, v = prologue.conv_verify(parent, S0, X0, seq["x"], W64, beta, gate, H, d)
        y = None
    else:
        q, k, v = seq["q"], seq["k"], seq["v"]
        o, _ = ogdn.verify(parent, S0, q, k, v, beta, gate, keep_states=False)
        y = oconv.tree_conv(parent, X0, seq["x"], W64) if X0 is not None else None
    with np.errstate(divide="ignore"):
        kf, uf, lg = ogdn.factors(parent, S0, k, v, beta, gate)
    return dict(o=o, y=y, k=kf, u=uf, lg=lg, kv=(k, v))


def oracle_seq(parent, S0, X0, W, h, layer, b, offs, with_states=True):
    """Oracle verify + conv of sequence b at one layer from host input dict `h` (widened)."""
    sl = slice(offs[b], offs[b + 1])
    q, k, v = h["q"][layer, sl], h["k"][layer, sl], h["v"][layer, sl]
    beta, gate = h["beta"][layer, sl], h["gate"][layer, sl]
    o, states = ogdn.verify(parent, S0, q, k, v, beta, gate, keep_states=with_states)
    kf, uf, lg = ogdn.factors(parent, S0, k, v, beta, gate, states) if with_states else (None,) * 3
    y = oconv.tree_conv(parent, X0, h["x"][layer, sl], W) if X0 is not None else None
    return dict(o=o, states=states, k=kf, u=uf, lg=lg, y=y)


def widen_inputs(h: dict, dtype: str) -> dict:
    return {name: workload.widen(a, dtype) for name, a in h.items()}


def assert_outputs(o_gpu, o_ref, tol=OUT_TOL, what="o", mode="?", quantity="o"):
    err = float(np.max(vec_rel(o_gpu, o_ref)))
    record(quantity, mode, err)
    assert err <= tol, f"{what}: max normwise rel error {err:.3e} > {tol}"
    return err


def assert_state(S_gpu, S_ref, tol=STATE_TOL, what="state", mode="?"):
    err = float(np.max(frob_rel(S_gpu, S_ref)))
    record("state", mode, err)
    assert err <= tol, f"{what}: max Frobenius rel error {err:.3e} > {tol}"
    return err


def row_rel(x, r):
    """Relative 2-norm error per row (last axis); a zero reference row must match exactly."""
    num = np.linalg.norm(x - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    return np.where(den > 0, num / np.maximum(den, 1e-300), np.where(num > 0, np.inf, 0.0))


def assert_lg(lgg, ref_lg):
    """Banked ln g within 4 fp32 ulp of ln g; a zero gate's -inf exactly."""
    ninf = np.isneginf(ref_lg)
    assert np.array_equal(np.isneginf(lgg), ninf), "banked ln g: -inf where the gate is not 0"
    fin = ~ninf
    assert np.all(np.abs(lgg[fin] - ref_lg[fin]) <= 4 * ulp32(ref_lg[fin])), \
        "banked ln g beyond 4 ulp"


def assert_bank_rows(b: Batch, layer: int, seq: int, bank: int, rows, ref_k, ref_u, ref_lg):
    """Rows of one bank for (layer, seq), all heads, against oracle factors [n,H,...]."""
    rows = list(rows)
    kg = to_np(b.layers.bank_k[bank][layer, seq][:, rows]).transpose(1, 0, 2)
    ug = to_np(b.layers.bank_u[bank][layer, seq][:, rows]).transpose(1, 0, 2)
    lgg = to_np(b.layers.bank_lg[bank][layer, seq][:, rows]).T
    if b.mode == "fused":
        kerr = float(np.max(row_rel(kg, ref_k)))
        record("banked k", b.mode, kerr)
        assert kerr <= K_TOL, f"banked k: rel error {kerr:.3e}"
    else:
        assert np.array_equal(kg, ref_k), "banked k differs from the widened input"
    uerr = float(np.max(row_rel(ug, ref_u)))
    record("banked u", b.mode, uerr)
    assert uerr <= U_TOL, f"banked u: rel error {uerr:.3e}"
    assert_lg(lgg, ref_lg)


COMMIT_MODES = {"row-map": binding.COMMIT_ROW_MAP, "compact": binding.COMMIT_COMPACT}


def role_pending_expect(role, paths, commit_mode="row-map"):
    """Oracle bookkeeping of a commit: new roles, pending lengths and row maps."""
    if commit_mode == "row-map":
        new = [obanks.commit_row_map(int(r), p) for r, p in zip(role, paths)]
        rows = [n[2] for n in new]
    else:
        new = [obanks.commit_bookkeeping(int(r), p) for r, p in zip(role, paths)]
        rows = [obanks.pending_rows_after_compaction(p) for p in paths]
    return np.array([n[0] for n in new]), np.array([n[1] for n in new]), rows


def tiny_inputs(trees, step, H=1, d=16, C=16, dtype="f32", cfg_id=0):
    """Per-step inputs for a batch of small trees (seeded per (step, seq))."""
    sizes = [len(t) for t in trees]
    T = sum(sizes)
    el = np.uint16 if dtype == "bf16" else np.float32
    h = {name: np.empty((1, T, H, d), dtype=el) for name in ("q", "k", "v")}
    h.update({name: np.empty((1, T, H), dtype=el) for name in ("beta", "gate")})
    h["x"] = np.empty((1, T, C), dtype=el)
    off = 0
    for b, n in enumerate(sizes):
        vals = synth.node_inputs(cfg_id, step, 0, b, n, H, d, dtype)
        for name, a in vals.items():
            h[name][0, off:off + n] = a
        h["x"][0, off:off + n] = synth.conv_inputs(cfg_id, step, 0, b, n, C, dtype)
        off += n
    return h


def to_device(h: dict, dtype: str, device="cuda"):
    return workload.StepInputs(**{k: workload._to_torch(v, dtype, device) for k, v in h.items()})

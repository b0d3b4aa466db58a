"""ctypes binding of libgdn_tree.so -- argument marshalling only.

Every computation runs in the HIP library; this module converts numpy arrays and torch
tensors (device memory on ROCm) into the pointers and sizes that include/gdn_tree.h
declares, and raises GdnError on a non-zero status.  torch is imported before the library is
loaded so that both share one HIP runtime.  There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn_tree.so")

GDN_F32, GDN_BF16 = 0, 1
STATUS = {0: "GDN_OK", -1: "GDN_EINVAL", -2: "GDN_ETREE", -3: "GDN_EPATH",
          -4: "GDN_ECAPACITY", -5: "GDN_EDEVICE"}
EXPORTS = [
    "gdn_last_error", "gdn_schedule_words", "gdn_hld_schedule", "gdn_ddtree_build",
    "gdn_verify_workspace_bytes",
    "gdn_tree_verify", "gdn_tree_verify_noalloc", "gdn_tree_verify_wave",
    "gdn_tree_verify_wave_timed",
    "gdn_tree_verify_ut", "gdn_tree_verify_ut_timed", "gdn_tree_conv",
    "gdn_tree_conv_verify", "gdn_tree_conv_verify_timed",
    "gdn_commit_path", "gdn_prefill", "gdn_prefill_timed",
    "gdn_compact_factors", "gdn_flush",
]
IMAGE_HEADER = 16
IMAGE_MAGIC = 0x53444E47


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}: {text}")
        self.status = status


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I32P = ctypes.POINTER(ctypes.c_int32)
_FP = ctypes.POINTER(ctypes.c_float)


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("n_seqs", _I32), ("n_heads", _I32), ("head_dim", _I32), ("n_nodes", _I32),
        ("max_nodes", _I32), ("layer_begin", _I32), ("n_layers", _I32), ("in_dtype", _I32),
        ("q", _P), ("k", _P), ("v", _P), ("beta", _P), ("gate", _P), ("state", _P),
        ("bank_k", _P * 2), ("bank_u", _P * 2), ("bank_lg", _P * 2),
        ("role", _P), ("pending_len", _P), ("pending_rows", _P), ("workspace", _P), ("out", _P),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("n_seqs", _I32), ("n_heads", _I32), ("head_dim", _I32), ("n_tokens", _I32),
        ("layer_begin", _I32), ("n_layers", _I32), ("in_dtype", _I32), ("reserved", _I32),
        ("q", _P), ("k", _P), ("v", _P), ("beta", _P), ("gate", _P), ("seq_offsets", _P),
        ("state", _P), ("out", _P),
    ]


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("n_seqs", _I32), ("channels", _I32), ("width", _I32), ("n_nodes", _I32),
        ("max_nodes", _I32), ("layer_begin", _I32), ("n_layers", _I32), ("in_dtype", _I32),
        ("x", _P), ("weight", _P), ("conv_state", _P), ("bank_x", _P * 2),
        ("role", _P), ("pending_len", _P), ("pending_rows", _P), ("out", _P),
    ]


_lib = None


# A host-only build of the library's plain C++ parts (schedule, draft-tree builder, commit
# bookkeeping) with AddressSanitizer and UndefinedBehaviorSanitizer (build_host_san.py): when
# this variable names it, lib() loads it instead, for host-side tests; device entry points are
# then absent and torch is not imported.
HOST_LIB_ENV = "GDN_TREE_HOST_LIB"


def host_only() -> bool:
    return bool(os.environ.get(HOST_LIB_ENV))


def _prototypes():
    VA, CA, PA = ctypes.POINTER(VerifyArgs), ctypes.POINTER(ConvArgs), ctypes.POINTER(PrefillArgs)
    return {
        "gdn_last_error": (ctypes.c_char_p, []),
        "gdn_schedule_words": (ctypes.c_size_t, [_I32, _I32]),
        "gdn_hld_schedule": (_I32, [_I32P, _I32P, _I32, _I32P, ctypes.c_size_t]),
        "gdn_ddtree_build": (_I32, [_FP, _I32P, _I32P, _I32, _I32, _I32, _I32, ctypes.c_float,
                                    _I32, _I32P, _I32P, _I32P, _I32P, _FP, _I32P]),
        "gdn_verify_workspace_bytes": (ctypes.c_size_t, [_I32P, _I32, _I32, _I32]),
        "gdn_tree_verify": (_I32, [VA, _I32P, _P, _P]),
        "gdn_tree_verify_noalloc": (_I32, [VA, _I32P, _P, _P]),
        "gdn_tree_verify_wave": (_I32, [VA, _I32P, _P, _I32, _P]),
        "gdn_tree_verify_wave_timed": (_I32, [VA, _I32P, _P, _I32, _P, _P, _P]),
        "gdn_tree_verify_ut": (_I32, [VA, _I32P, _P, _P]),
        "gdn_tree_verify_ut_timed": (_I32, [VA, _I32P, _P, _P, _P, _P]),
        "gdn_prefill": (_I32, [PA, _I32P, _P]),
        "gdn_prefill_timed": (_I32, [PA, _I32P, _P, _P, _P]),
        "gdn_tree_conv_verify": (_I32, [VA, CA, _I32P, _P, _P]),
        "gdn_tree_conv_verify_timed": (_I32, [VA, CA, _I32P, _P, _P, _P, _P]),
        "gdn_tree_conv": (_I32, [CA, _I32P, _P, _P]),
        "gdn_commit_path": (_I32, [_I32P, _I32P, _I32P, _P, _P, VA, CA, _I32P, _I32P, _I32, _P]),
        "gdn_compact_factors": (_I32, [_P, _P, ctypes.c_int64, _P, _P, _I32, _P]),
        "gdn_flush": (_I32, [VA, CA, _I32P, _P]),
    }


def lib() -> ctypes.CDLL:
    """Load the HIP library (after torch, so the HIP runtime is shared), or the sanitized
    host-only build named by GDN_TREE_HOST_LIB."""
    global _lib
    if _lib is not None:
        return _lib
    host = os.environ.get(HOST_LIB_ENV)
    if host:
        L = ctypes.CDLL(host)
    else:
        import torch  # noqa: F401  -- must precede the library: one HIP runtime per process
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_deltanet_tree_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _prototypes().items():
        if host and not hasattr(L, name):
            continue  # device entry points are not in the host-only build
        fn = getattr(L, name)
        fn.restype = res
        if args:
            fn.argtypes = args
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise GdnError(status, where, lib().gdn_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _dev(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


# ------------------------------------------------------------------------------------
# schedule (host)
# ------------------------------------------------------------------------------------

def schedule_words(n_seqs: int, n_nodes: int) -> int:
    return int(lib().gdn_schedule_words(n_seqs, n_nodes))


def hld_schedule(parents) -> np.ndarray:
    """Schedule image (int32) of a batch of trees given as a list of local parent arrays."""
    parents = [_i32(p) for p in parents]
    seq_offsets = _i32(np.concatenate([[0], np.cumsum([len(p) for p in parents])]))
    flat = _i32(np.concatenate(parents)) if parents else np.zeros(1, dtype=np.int32)
    n_words = schedule_words(len(parents), int(seq_offsets[-1]))
    image = np.zeros(max(n_words, IMAGE_HEADER + 3), dtype=np.int32)
    _check(lib().gdn_hld_schedule(_ptr(flat), _ptr(seq_offsets), len(parents), _ptr(image),
                                  image.size), "gdn_hld_schedule")
    return image


def schedule_view(image: np.ndarray) -> dict:
    """Named views of a schedule image, following the layout in gdn_tree.h."""
    S, T = int(image[1]), int(image[2])
    n_chains, n_waves = int(image[3]), int(image[4])
    o = IMAGE_HEADER
    seq = image[o:o + S + 1]
    o += S + 1
    wave = image[o:o + n_waves + 1]
    o += T + 1
    chain = image[o:o + n_chains + 1]
    o += T + 1
    fields = {}
    for name in ("chain_nodes", "chain_seq", "chain_src", "node_store", "node_parent",
                 "node_depth"):
        fields[name] = image[o:o + T]
        o += T
    fields["chain_seq"] = fields["chain_seq"][:n_chains]
    fields["chain_src"] = fields["chain_src"][:n_chains]
    ut = None
    if int(image[8]) >= 0:  # tree-masked verify plan
        rec_base = image[o:o + S + 1]
        o += S + 1
        node_rec = image[o:o + T]
        o += T
        lv_base = image[o:o + S + 1]
        o += S + 1
        lvn = image[o:o + int(lv_base[-1])]
        o += T + S
        lvnode = image[o:o + T]
        o += T
        rec_anc = image[o:o + int(rec_base[-1])]
        ut = dict(records=int(image[8]), max_records=int(image[9]), max_levels=int(image[10]),
                  rec_base=rec_base, node_rec=node_rec, lv_base=lv_base, lvn=lvn,
                  lvnode=lvnode, rec_anc=rec_anc)
    return dict(n_seqs=S, n_nodes=T, n_chains=n_chains, n_waves=n_waves,
                n_boundaries=int(image[5]), max_chain_len=int(image[6]), max_tree=int(image[7]),
                seq_offsets=seq, wave_offsets=wave, chain_offsets=chain, ut_plan=ut, **fields)


def ddtree_build(logp, tokens=None, root_tokens=None, budget=22, tau=6.0, chain_seed=True):
    """Best-first draft trees of a batch: logp [B][L][K] (or [L][K]) fp32 log-probabilities,
    tokens of the same shape (optional).  Returns a list of dicts parent/depth/rank/score
    (and token) per tree, each cut to its node count."""
    lp = np.ascontiguousarray(logp, dtype=np.float32)
    single = lp.ndim == 2
    if single:
        lp = lp[None]
    B, L, K = lp.shape
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, L, K)
    rt = None if root_tokens is None else _i32(np.reshape(root_tokens, (B,)))
    out = {name: np.full((B, budget), -1, dtype=np.int32) for name in ("parent", "depth", "rank",
                                                                        "token")}
    sc = np.zeros((B, budget), dtype=np.float32)
    n = np.zeros(B, dtype=np.int32)
    fp = lambda a: a.ctypes.data_as(_FP)  # noqa: E731
    _check(lib().gdn_ddtree_build(fp(lp), None if tk is None else _ptr(tk),
                                  None if rt is None else _ptr(rt), B, L, K, budget,
                                  ctypes.c_float(tau), int(bool(chain_seed)), _ptr(out["parent"]),
                                  _ptr(out["depth"]), _ptr(out["rank"]),
                                  None if tk is None else _ptr(out["token"]), fp(sc), _ptr(n)),
           "gdn_ddtree_build")
    trees = []
    for b in range(B):
        m = int(n[b])
        t = {k: v[b, :m].copy() for k, v in out.items() if k != "token" or tk is not None}
        t["score"] = sc[b, :m].copy()
        trees.append(t)
    return trees[0] if single else trees


def verify_workspace_bytes(image: np.ndarray, n_heads: int, head_dim: int, n_layers: int) -> int:
    """Workspace bytes of the chain verify (boundary states) for this schedule."""
    return int(lib().gdn_verify_workspace_bytes(_ptr(image), n_heads, head_dim, n_layers))





# ------------------------------------------------------------------------------------
# device calls
# ------------------------------------------------------------------------------------

@dataclass
class Layers:
    """Device buffers of a stack of GDN layers for one batch of sequences (torch tensors).

    Shapes: state [Ly,S,H,d,d]; bank_k/bank_u [2][Ly,S,H,max_nodes,d]; bank_lg
    [2][Ly,S,H,max_nodes]; conv_state [Ly,S,Cch,3]; bank_x [2][Ly,S,max_nodes,Cch];
    bank_x holds the raw conv inputs in their own dtype (bf16 or fp32);
    role, pending [S] int32 (device) with host mirrors role_host, pending_host;
    pending_rows [S,max_nodes] int32 (device): the bank row of each pending factor.
    """
    state: object
    bank_k: list
    bank_u: list
    bank_lg: list
    role: object
    pending: object
    role_host: np.ndarray
    pending_host: np.ndarray
    pending_rows: object = None
    conv_state: object = None
    bank_x: list = None


def _need(t, n, what):
    """Reject a tensor that is smaller than the call will address (or not contiguous)."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements, the call addresses {n}")


def verify_args(image, layers: Layers, q, k, v, beta, gate, out, workspace,
                layer_begin=0, n_layers=1, max_nodes=None) -> VerifyArgs:
    import torch
    S, T = int(image[1]), int(image[2])
    Ly_end = layer_begin + n_layers
    H, d = int(layers.state.shape[2]), int(layers.state.shape[3])
    Nm = int(layers.bank_lg[0].shape[-1]) if max_nodes is None else max_nodes
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need(t, Ly_end * T * H * d, name)
    _need(beta, Ly_end * T * H, "beta")
    _need(gate, Ly_end * T * H, "gate")
    _need(layers.state, Ly_end * S * H * d * d, "state")
    for i in range(2):
        _need(layers.bank_k[i], Ly_end * S * H * Nm * d, "bank_k")
        _need(layers.bank_u[i], Ly_end * S * H * Nm * d, "bank_u")
        _need(layers.bank_lg[i], Ly_end * S * H * Nm, "bank_lg")
    _need(layers.role, S, "role")
    _need(layers.pending, S, "pending")
    _need(layers.pending_rows, S * Nm, "pending_rows")
    _need(workspace, 0, "workspace")
    a = VerifyArgs()
    # kept for the size check of the chain entry points
    a.ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.sizes = (H, d, n_layers)
    a.n_seqs, a.n_nodes = int(image[1]), int(image[2])
    a.n_heads, a.head_dim = int(layers.state.shape[2]), int(layers.state.shape[3])
    a.max_nodes = int(layers.bank_lg[0].shape[-1]) if max_nodes is None else max_nodes
    a.layer_begin, a.n_layers = layer_begin, n_layers
    ref = q if q is not None else beta  # the fused conv -> verify call passes no q/k/v
    a.in_dtype = GDN_BF16 if (ref is not None and ref.dtype == torch.bfloat16) else GDN_F32
    a.q, a.k, a.v, a.beta, a.gate = (_dev(t) for t in (q, k, v, beta, gate))
    a.state = _dev(layers.state)
    for i in range(2):
        a.bank_k[i] = _dev(layers.bank_k[i])
        a.bank_u[i] = _dev(layers.bank_u[i])
        a.bank_lg[i] = _dev(layers.bank_lg[i])
    a.role, a.pending_len = _dev(layers.role), _dev(layers.pending)
    a.pending_rows = _dev(layers.pending_rows)
    a.workspace, a.out = _dev(workspace), _dev(out)
    return a


def conv_args(image, layers: Layers, x, weight, out, layer_begin=0, n_layers=1,
              max_nodes=None) -> ConvArgs:
    import torch
    S, T = int(image[1]), int(image[2])
    Ly_end = layer_begin + n_layers
    C = int(layers.conv_state.shape[2])
    Nm = int(layers.bank_x[0].shape[2]) if max_nodes is None else max_nodes
    _need(x, Ly_end * T * C, "x")
    _need(out, Ly_end * T * C, "conv out")
    _need(weight, Ly_end * C * 4, "weight")
    _need(layers.conv_state, Ly_end * S * C * 3, "conv_state")
    for i in range(2):
        _need(layers.bank_x[i], Ly_end * S * Nm * C, "bank_x")
    a = ConvArgs()
    a.n_seqs, a.n_nodes = int(image[1]), int(image[2])
    a.channels, a.width = int(layers.conv_state.shape[2]), 4
    a.max_nodes = int(layers.bank_x[0].shape[2]) if max_nodes is None else max_nodes
    a.layer_begin, a.n_layers = layer_begin, n_layers
    # the conv bank keeps the raw inputs in their own dtype: x (when given) must match it
    bank_bf16 = layers.bank_x[0].dtype == torch.bfloat16
    if x is not None and (x.dtype == torch.bfloat16) != bank_bf16:
        raise ValueError(f"x is {x.dtype} but the conv bank holds {layers.bank_x[0].dtype}: "
                         "allocate the layers with conv_dtype matching the conv inputs")
    a.in_dtype = GDN_BF16 if bank_bf16 else GDN_F32
    a.x, a.weight, a.out = _dev(x), _dev(weight), _dev(out)
    a.conv_state = _dev(layers.conv_state)
    a.bank_x[0], a.bank_x[1] = _dev(layers.bank_x[0]), _dev(layers.bank_x[1])
    _need(layers.pending_rows, S * Nm, "pending_rows")
    a.role, a.pending_len = _dev(layers.role), _dev(layers.pending)
    a.pending_rows = _dev(layers.pending_rows)
    return a


def _need_ws(args: VerifyArgs, image: np.ndarray):
    """The chain verify writes boundary states into the workspace: check its size."""
    if args.q is None:
        return
    H, d, n_layers = args.sizes
    need = verify_workspace_bytes(image, H, d, n_layers)
    if need and args.ws_bytes < need:
        raise ValueError(f"workspace holds {args.ws_bytes} bytes, the call needs {need}")


def tree_verify(args: VerifyArgs, image: np.ndarray, dev_image, stream=None):
    _need_ws(args, image)
    _check(lib().gdn_tree_verify(ctypes.byref(args), _ptr(image), _dev(dev_image),
                                 _stream(stream)), "gdn_tree_verify")


def tree_verify_noalloc(args: VerifyArgs, image: np.ndarray, dev_image, stream=None):
    """gdn_tree_verify with the boundary states in the library's fixed device scratch
    (args.workspace is ignored); allocates nothing."""
    _check(lib().gdn_tree_verify_noalloc(ctypes.byref(args), _ptr(image), _dev(dev_image),
                                         _stream(stream)), "gdn_tree_verify_noalloc")


def tree_verify_wave(args: VerifyArgs, image: np.ndarray, dev_image, wave: int, stream=None):
    _need_ws(args, image)
    _check(lib().gdn_tree_verify_wave(ctypes.byref(args), _ptr(image), _dev(dev_image), wave,
                                      _stream(stream)), "gdn_tree_verify_wave")


def tree_verify_wave_timed(args: VerifyArgs, image: np.ndarray, dev_image, wave: int,
                           start: "HipEvent", stop: "HipEvent", stream=None):
    _need_ws(args, image)
    _check(lib().gdn_tree_verify_wave_timed(ctypes.byref(args), _ptr(image), _dev(dev_image), wave,
                                            start.handle, stop.handle, _stream(stream)),
           "gdn_tree_verify_wave_timed")


def tree_verify_ut(args: VerifyArgs, image: np.ndarray, dev_image, stream=None):
    _check(lib().gdn_tree_verify_ut(ctypes.byref(args), _ptr(image), _dev(dev_image),
                                    _stream(stream)), "gdn_tree_verify_ut")


def tree_verify_ut_timed(args: VerifyArgs, image: np.ndarray, dev_image, start: "HipEvent",
                         stop: "HipEvent", stream=None):
    _check(lib().gdn_tree_verify_ut_timed(ctypes.byref(args), _ptr(image), _dev(dev_image),
                                          start.handle, stop.handle, _stream(stream)),
           "gdn_tree_verify_ut_timed")


def tree_conv_verify(vargs: VerifyArgs, cargs: ConvArgs, image: np.ndarray, dev_image,
                     stream=None):
    """Fused conv -> SiLU -> unit-length q/k -> tree-masked verify (gdn_tree_conv_verify);
    vargs carries no q/k/v, cargs no conv output."""
    _check(lib().gdn_tree_conv_verify(ctypes.byref(vargs), ctypes.byref(cargs), _ptr(image),
                                      _dev(dev_image), _stream(stream)), "gdn_tree_conv_verify")


def tree_conv_verify_timed(vargs: VerifyArgs, cargs: ConvArgs, image: np.ndarray, dev_image,
                           start: "HipEvent", stop: "HipEvent", stream=None):
    _check(lib().gdn_tree_conv_verify_timed(ctypes.byref(vargs), ctypes.byref(cargs),
                                            _ptr(image), _dev(dev_image), start.handle,
                                            stop.handle, _stream(stream)),
           "gdn_tree_conv_verify_timed")


def prefill_args(host_offsets, dev_offsets, q, k, v, beta, gate, state, out, layer_begin=0,
                 n_layers=1):
    """Arguments of gdn_prefill; q/k/v [Ly][T][H][d], beta/gate [Ly][T][H], state
    [Ly][S][H][d][d], out [Ly][T][H][d] (torch tensors), offsets [S+1] (numpy + device)."""
    import torch
    host_offsets = _i32(host_offsets)
    S, T = len(host_offsets) - 1, int(host_offsets[-1])
    H, d = int(state.shape[2]), int(state.shape[3])
    Ly_end = layer_begin + n_layers
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _need(t, Ly_end * T * H * d, name)
    _need(beta, Ly_end * T * H, "beta")
    _need(gate, Ly_end * T * H, "gate")
    _need(state, Ly_end * S * H * d * d, "state")
    _need(dev_offsets, S + 1, "seq_offsets")
    a = PrefillArgs()
    a.n_seqs, a.n_heads, a.head_dim, a.n_tokens = S, H, d, T
    a.layer_begin, a.n_layers = layer_begin, n_layers
    a.in_dtype = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    a.q, a.k, a.v, a.beta, a.gate = (_dev(t) for t in (q, k, v, beta, gate))
    a.seq_offsets, a.state, a.out = _dev(dev_offsets), _dev(state), _dev(out)
    a.host_offsets = host_offsets
    return a


def prefill(args: PrefillArgs, stream=None):
    _check(lib().gdn_prefill(ctypes.byref(args), _ptr(args.host_offsets), _stream(stream)),
           "gdn_prefill")


def prefill_timed(args: PrefillArgs, start: "HipEvent", stop: "HipEvent", stream=None):
    _check(lib().gdn_prefill_timed(ctypes.byref(args), _ptr(args.host_offsets), start.handle,
                                   stop.handle, _stream(stream)), "gdn_prefill_timed")


class HipEvent:
    """A timing-enabled hipEvent_t from the process's HIP runtime (the one torch loaded)."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            lib()
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = self._runtime().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")

    def elapsed_ms(self, stop: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle, stop.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.handle:
            self._hip.hipEventDestroy(self.handle)


def tree_conv(args: ConvArgs, image: np.ndarray, dev_image, stream=None):
    _check(lib().gdn_tree_conv(ctypes.byref(args), _ptr(image), _dev(dev_image),
                               _stream(stream)), "gdn_tree_conv")


def pack_paths(paths):
    flat = _i32(np.concatenate([np.asarray(p, dtype=np.int32) for p in paths])) \
        if any(len(p) for p in paths) else np.zeros(1, dtype=np.int32)
    offsets = _i32(np.concatenate([[0], np.cumsum([len(p) for p in paths])]))
    return flat, offsets


COMMIT_COMPACT, COMMIT_ROW_MAP = 0, 1


def commit_path(image, paths, layers: Layers, vargs: VerifyArgs, cargs: ConvArgs | None,
                dev_paths=None, dev_offsets=None, stream=None, mode=COMMIT_ROW_MAP):
    """Accept one root path per sequence (local ids); updates layers.role/pending/pending_rows
    (device on the stream, host mirrors now).  dev_paths/dev_offsets default to fresh
    uploads.  mode: COMMIT_ROW_MAP (no copy) or COMMIT_COMPACT (branched paths gathered into
    path order)."""
    import torch
    flat, offsets = pack_paths(paths)
    if dev_paths is None:
        dev_paths = torch.from_numpy(flat).to(layers.role.device)
        dev_offsets = torch.from_numpy(offsets).to(layers.role.device)
    _check(lib().gdn_commit_path(
        _ptr(image), _ptr(flat), _ptr(offsets), _dev(dev_paths), _dev(dev_offsets),
        ctypes.byref(vargs), ctypes.byref(cargs) if cargs is not None else None,
        _ptr(layers.role_host), _ptr(layers.pending_host), int(mode), _stream(stream)),
        "gdn_commit_path")
    return dev_paths, dev_offsets


def compact_factors(src, dst, row_elems: int, src_rows, dst_rows, stream=None):
    _check(lib().gdn_compact_factors(_dev(src), _dev(dst), row_elems, _dev(src_rows),
                                     _dev(dst_rows), int(src_rows.numel()), _stream(stream)),
           "gdn_compact_factors")


def flush(vargs: VerifyArgs, cargs: ConvArgs | None, layers: Layers, stream=None):
    _check(lib().gdn_flush(ctypes.byref(vargs), ctypes.byref(cargs) if cargs is not None else None,
                           _ptr(layers.pending_host), _stream(stream)), "gdn_flush")


def alloc_layers(n_layers, n_seqs, n_heads, head_dim, max_nodes, channels=0, device="cuda",
                 conv_dtype="f32"):
    """Zero-initialised device buffers for `n_layers` layers (torch.empty/zeros on device);
    conv_dtype ("f32" or "bf16") is the dtype of the conv inputs, which the conv bank keeps."""
    import torch
    f = dict(device=device, dtype=torch.float32)
    Ly, S, H, d, Nm = n_layers, n_seqs, n_heads, head_dim, max_nodes
    lay = Layers(
        state=torch.zeros((Ly, S, H, d, d), **f),
        bank_k=[torch.zeros((Ly, S, H, Nm, d), **f) for _ in range(2)],
        bank_u=[torch.zeros((Ly, S, H, Nm, d), **f) for _ in range(2)],
        bank_lg=[torch.zeros((Ly, S, H, Nm), **f) for _ in range(2)],
        role=torch.zeros(S, device=device, dtype=torch.int32),
        pending=torch.zeros(S, device=device, dtype=torch.int32),
        role_host=np.zeros(S, dtype=np.int32),
        pending_host=np.zeros(S, dtype=np.int32),
        pending_rows=torch.zeros((S, Nm), device=device, dtype=torch.int32),
    )
    if channels:
        lay.conv_state = torch.zeros((Ly, S, channels, 3), **f)
        xdt = torch.bfloat16 if conv_dtype == "bf16" else torch.float32
        lay.bank_x = [torch.zeros((Ly, S, Nm, channels), device=device, dtype=xdt)
                      for _ in range(2)]
    return lay

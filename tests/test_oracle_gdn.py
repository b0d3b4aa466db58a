"""Pins of the float64 GDN tree oracle against closed forms, invariants and brute force.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, a
parent/child index mix-up, a transposed state) fails at least one of them.
"""
import itertools

import numpy as np
import pytest

from oracle import gdn

RNG = np.random.default_rng(12345)


def _inputs(N, H, d, rng, unit_keys=True):
    q = rng.standard_normal((N, H, d))
    k = rng.standard_normal((N, H, d))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, d))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, H))))
    gate = np.exp(-np.logaddexp(0.0, rng.standard_normal((N, H))))
    S0 = 0.3 * rng.standard_normal((H, d, d))  # deliberately non-symmetric
    return S0, q, k, v, beta, gate


TREES = {
    "tiny": np.array([-1, 0, 0, 1, 1, 2, 3]),
    "chain": np.arange(-1, 7),
    "star": np.array([-1, 0, 0, 0, 0]),
    "mixed": np.array([-1, 0, 1, 1, 0, 4, 5, 2, 2, 4]),
}


def _gamma(parent, gate):
    out = np.zeros(gate.shape)
    for n in range(len(parent)):
        out[n] = np.prod(gate[gdn.root_path(parent, n)], axis=0)
    return out


@pytest.mark.parametrize("name", sorted(TREES))
def test_v1_identity_update(name):
    """beta = 0 and g = 1: no token changes the state, o_n = S0 q_n."""
    parent = TREES[name]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 16, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, 0 * beta, np.ones_like(gate))
    assert np.array_equal(S, np.broadcast_to(S0, S.shape))
    np.testing.assert_allclose(o, np.einsum("hij,nhj->nhi", S0, q), rtol=0, atol=1e-14)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v2_pure_decay(name):
    """beta = 0: S_n = (product of g over n's root path) * S0."""
    parent = TREES[name]
    S0, q, k, v, beta, gate = _inputs(len(parent), 3, 8, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, 0 * beta, gate)
    gam = _gamma(parent, gate)
    np.testing.assert_allclose(S, gam[:, :, None, None] * S0[None], rtol=1e-13, atol=0)
    np.testing.assert_allclose(o, gam[:, :, None] * np.einsum("hij,nhj->nhi", S0, q),
                               rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v3_delta_write_identity(name):
    """S_n k_n = g(1 - beta|k|^2) S_parent k_n + beta |k|^2 v_n; with beta = 1, |k| = 1 the
    state reads back exactly the value just written."""
    parent = TREES[name]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 16, RNG, unit_keys=False)
    _, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    for n in range(len(parent)):
        Sp = S0 if parent[n] < 0 else S[parent[n]]
        kk = np.sum(k[n] ** 2, axis=-1)
        lhs = np.einsum("hij,hj->hi", S[n], k[n])
        rhs = (gate[n] * (1 - beta[n] * kk))[:, None] * np.einsum("hij,hj->hi", Sp, k[n]) \
            + (beta[n] * kk)[:, None] * v[n]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    _, S = gdn.verify(parent, S0, q, kn, v, np.ones_like(beta), gate)
    for n in range(len(parent)):
        np.testing.assert_allclose(np.einsum("hij,hj->hi", S[n], kn[n]), v[n], atol=1e-12)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v4_orthonormal_keys_closed_form(name):
    """Mutually orthonormal keys: S_n k_j = G_n (1-b_j) S0 k_j + (G_n/G_j) b_j v_j for each j
    on n's path, and S_n w = G_n S0 w for w orthogonal to all keys."""
    parent = TREES[name]
    N, H, d = len(parent), 2, 16
    S0, q, _, v, beta, gate = _inputs(N, H, d, RNG)
    basis = np.stack([np.linalg.qr(RNG.standard_normal((d, d)))[0] for _ in range(H)])
    k = np.transpose(basis[:, :, :N], (2, 0, 1)).copy()  # node n -> column n, per head
    w = np.transpose(basis[:, :, N:], (0, 2, 1))  # [H, d-N, d] orthogonal complement
    _, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    gam = _gamma(parent, gate)
    for n in range(N):
        for j in gdn.root_path(parent, n):
            lhs = np.einsum("hij,hj->hi", S[n], k[j])
            rhs = (gam[n] * (1 - beta[j]))[:, None] * np.einsum("hij,hj->hi", S0, k[j]) \
                + (gam[n] / gam[j] * beta[j])[:, None] * v[j]
            np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)
        lhs = np.einsum("hij,hmj->hmi", S[n], w)
        rhs = gam[n][:, None, None] * np.einsum("hij,hmj->hmi", S0, w)
        np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)


def test_v5_chain_equals_explicit_projector_products():
    """Pure chain: per-path replay equals the token loop written with the literal d x d
    projector S @ (I - beta k k^T), and node n's output is that loop's n-th output."""
    parent = TREES["chain"]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 16, RNG, unit_keys=False)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    St = S0.copy()
    for n in range(len(parent)):
        St = gdn.gdn_step_matrix(St, k[n], v[n], beta[n], gate[n])
        np.testing.assert_allclose(S[n], St, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(o[n], np.einsum("hij,hj->hi", St, q[n]), atol=1e-12)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v6_sibling_isolation(name):
    """Changing every input of node m leaves all nodes outside m's subtree bit-identical."""
    parent = TREES[name]
    N = len(parent)
    S0, q, k, v, beta, gate = _inputs(N, 2, 8, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    for m in range(1, N):
        sub = {n for n in range(N) if m in gdn.root_path(parent, n)}
        q2, k2, v2, b2, g2 = (a.copy() for a in (q, k, v, beta, gate))
        q2[m] += 1.0
        k2[m] = -k2[m]
        v2[m] *= 3.0
        b2[m] = 1 - b2[m]
        g2[m] = g2[m] ** 2
        o2, S2 = gdn.verify(parent, S0, q2, k2, v2, b2, g2)
        for n in range(N):
            if n in sub:
                assert not np.array_equal(o2[n], o[n])
            else:
                assert np.array_equal(o2[n], o[n]) and np.array_equal(S2[n], S[n])


def _all_trees(N):
    for choice in itertools.product(*[range(i) for i in range(1, N)]):
        yield np.array((-1,) + choice)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6])
def test_v7_exhaustive_small_trees(N):
    """Every labelled tree with parent[i] < i and N <= 6 nodes: per-path replay equals the
    depth-first state-stack walk and the tree-masked UT closed form."""
    trees = list(_all_trees(N))
    assert len(trees) == [1, 1, 2, 6, 24, 120][N - 1]
    rng = np.random.default_rng(N)
    for parent in trees:
        S0, q, k, v, beta, gate = _inputs(N, 1, 6, rng)
        o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
        o2, S2 = gdn.verify_dfs(parent, S0, q, k, v, beta, gate)
        o3, _ = gdn.verify_ut(parent, S0, q, k, v, beta, gate)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(S2, S, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o3, o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("e", [-3, 1, 5])
def test_v8_power_of_two_scaling(e):
    """Scaling S0 and every v by 2^e scales o, u and every state by exactly 2^e."""
    parent = TREES["mixed"]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 8, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    _, u, _ = gdn.factors(parent, S0, k, v, beta, gate, S)
    s = 2.0 ** e
    o2, S2 = gdn.verify(parent, s * S0, q, k, s * v, beta, gate)
    _, u2, _ = gdn.factors(parent, s * S0, k, s * v, beta, gate, S2)
    assert np.array_equal(o2, s * o) and np.array_equal(S2, s * S) and np.array_equal(u2, s * u)


def test_v9_joint_linearity():
    """o and the states are jointly linear in (S0, V) for fixed keys, queries and gates."""
    parent = TREES["mixed"]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 8, RNG)
    S0b = RNG.standard_normal(S0.shape)
    vb = RNG.standard_normal(v.shape)
    oa, Sa = gdn.verify(parent, S0, q, k, v, beta, gate)
    ob, Sb = gdn.verify(parent, S0b, q, k, vb, beta, gate)
    oc, Sc = gdn.verify(parent, S0 + S0b, q, k, v + vb, beta, gate)
    np.testing.assert_allclose(oc, oa + ob, atol=1e-12)
    np.testing.assert_allclose(Sc, Sa + Sb, atol=1e-12)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v10_ut_closed_form(name):
    """The tree-masked UT closed form gives the same outputs and residual vectors."""
    parent = TREES[name]
    S0, q, k, v, beta, gate = _inputs(len(parent), 3, 16, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    o3, u3 = gdn.verify_ut(parent, S0, q, k, v, beta, gate)
    _, u, _ = gdn.factors(parent, S0, k, v, beta, gate, S)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(u3, u, atol=1e-12)


def test_matrix_form_agrees_on_tree():
    """Replay with the literal projector product agrees on a branched tree."""
    parent = TREES["tiny"]
    S0, q, k, v, beta, gate = _inputs(len(parent), 1, 16, RNG, unit_keys=False)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    o2, S2 = gdn.verify(parent, S0, q, k, v, beta, gate, step=gdn.gdn_step_matrix)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(S2, S, atol=1e-12)


@pytest.mark.parametrize("name", sorted(TREES))
def test_v11_fold_of_factors_equals_replay(name):
    """Folding a path's factors (exp(lg) S + u k^T, in order) equals replaying the path token
    by token, and equals the verify's own state at the path's last node."""
    parent = TREES[name]
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 16, RNG)
    o, S = gdn.verify(parent, S0, q, k, v, beta, gate)
    kf, uf, lg = gdn.factors(parent, S0, k, v, beta, gate, S)
    for leaf in range(len(parent)):
        path = gdn.root_path(parent, leaf)
        R = gdn.replay(S0, k, v, beta, gate, path)
        F = gdn.fold(S0, kf[path], uf[path], lg[path])
        np.testing.assert_allclose(R, S[leaf], rtol=0, atol=1e-13)
        np.testing.assert_allclose(F, R, rtol=0, atol=1e-13)


def test_v11_zero_and_tiny_gates_fold_closed_form():
    """A zero gate erases everything before its token: after it, the state is u k^T of that
    token (u = beta v, since g S k vanishes) and the later tokens' updates, whatever S0 was.
    Its banked ln g is -inf, and the fold (exp(-inf) = 0) gives the same finite state as the
    replay.  A 1e-30 gate keeps a 1e-30 trace of the past, which the fold keeps too."""
    parent = TREES["chain"]
    rng = np.random.default_rng(11)
    S0, q, k, v, beta, gate = _inputs(len(parent), 2, 16, rng)
    gate = gate.copy()
    gate[3] = 0.0
    gate[5, 0] = 1e-30
    path = list(range(len(parent)))
    with np.errstate(divide="ignore"):
        kf, uf, lg = gdn.factors(parent, S0, k, v, beta, gate)
    assert np.all(np.isneginf(lg[3]))
    R = gdn.replay(S0, k, v, beta, gate, path)
    F = gdn.fold(S0, kf, uf, lg)
    assert np.all(np.isfinite(F))
    np.testing.assert_allclose(F, R, rtol=0, atol=1e-13)
    # independent of S0 once the zero gate has passed
    R2 = gdn.replay(5.0 * S0 + 1.0, k, v, beta, gate, path)
    np.testing.assert_allclose(R2, R, rtol=0, atol=1e-13)
    # from the zero gate on: the replay from a zero state with g = 1 at that token
    g1 = gate.copy()
    g1[3] = 1.0
    R3 = gdn.replay(np.zeros_like(S0), k, v, beta, g1, path[3:])
    np.testing.assert_allclose(R3, R, rtol=0, atol=1e-13)
    np.testing.assert_allclose(uf[3], beta[3][:, None] * v[3], rtol=0, atol=1e-15)


def test_v12_multi_step_commit_is_sequential_replay():
    """Carrying the committed state over several verify+accept steps equals one sequential
    replay of all accepted tokens (accepted paths may branch off the main chain)."""
    parent = TREES["mixed"]
    rng = np.random.default_rng(7)
    S0 = 0.3 * rng.standard_normal((2, 8, 8))
    committed, seq_k, seq_v, seq_b, seq_g = S0.copy(), [], [], [], []
    for step in range(4):
        _, q, k, v, beta, gate = _inputs(len(parent), 2, 8, rng)
        o, S = gdn.verify(parent, committed, q, k, v, beta, gate)
        leaf = int(rng.integers(len(parent)))
        path = gdn.root_path(parent, leaf)
        committed = S[leaf]
        seq_k += [k[m] for m in path]
        seq_v += [v[m] for m in path]
        seq_b += [beta[m] for m in path]
        seq_g += [gate[m] for m in path]
    chain = np.arange(-1, len(seq_k) - 1)
    _, Sc = gdn.verify(chain, S0, np.zeros(np.shape(seq_k)), np.array(seq_k), np.array(seq_v),
                       np.array(seq_b), np.array(seq_g))
    np.testing.assert_allclose(committed, Sc[-1], rtol=0, atol=1e-13)


def test_rejects_bad_trees():
    for bad in ([0, 0], [-1, 1], [-1, 0, 2], [-1, -1]):
        with pytest.raises(ValueError):
            gdn.check_tree(bad)


# ---------------------------------------------------------------------------------------
# sequential prefill (the plain sequence path after a flush)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 7, 16, 33])
def test_prefill_equals_chain_verify_and_replay(T):
    """A token sequence is a tree without branching: prefill outputs equal the per-path
    verify of the chain tree, and its final state equals the replay of the whole path."""
    rng = np.random.default_rng(400 + T)
    S0, q, k, v, beta, gate = _inputs(T, 2, 16, rng)
    o, S = gdn.prefill(S0, q, k, v, beta, gate)
    chain = np.arange(-1, T - 1)
    o_ref, _ = gdn.verify(chain, S0, q, k, v, beta, gate, keep_states=False)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, gdn.replay(S0, k, v, beta, gate, np.arange(T)), rtol=1e-12,
                               atol=1e-13)


def test_prefill_matrix_form_and_split_sequences():
    """The literal d x d projector form gives the same prefill, and prefilling A then B from
    A's final state equals prefilling A+B."""
    rng = np.random.default_rng(450)
    S0, q, k, v, beta, gate = _inputs(20, 3, 8, rng)
    o, S = gdn.prefill(S0, q, k, v, beta, gate)
    o2, S2 = gdn.prefill(S0, q, k, v, beta, gate, step=gdn.gdn_step_matrix)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-13)
    oa, Sa = gdn.prefill(S0, q[:9], k[:9], v[:9], beta[:9], gate[:9])
    ob, Sb = gdn.prefill(Sa, q[9:], k[9:], v[9:], beta[9:], gate[9:])
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-13)


def test_prefill_empty_and_zero_gate():
    rng = np.random.default_rng(460)
    S0, q, k, v, beta, gate = _inputs(3, 1, 8, rng)
    o, S = gdn.prefill(S0, q[:0], k[:0], v[:0], beta[:0], gate[:0])
    assert o.shape == (0, 1, 8) and np.array_equal(S, S0)
    gate = gate.copy()
    gate[1] = 0.0  # a zero gate erases the history: S_1 = beta v k^T
    _, S = gdn.prefill(S0, q[:2], k[:2], v[:2], beta[:2], gate[:2])
    want = gdn.prefill(np.zeros_like(S0), q[1:2], k[1:2], v[1:2], beta[1:2],
                       np.ones_like(gate[1:2]))[1]
    np.testing.assert_allclose(S, want, rtol=1e-12, atol=1e-13)

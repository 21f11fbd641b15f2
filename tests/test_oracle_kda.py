"""Pins of the oracle's per-channel decay (Kimi Delta Attention).

SEED appendix B.1 eq. (6) writes every layer type as S_t = Phi_t S_{t-1} + b k v^T with
Phi_t = (I - theta b k k^T) Lambda_t; Kimi Delta Attention has theta = 1 and a diagonal
Lambda_t, one decay per key channel.  The oracle applies Lambda literally to every stored u and
pad key each step.  Pins:
  * eps = 0: the factored path equals the dense recurrence at every step (both rules);
  * the dense step equals eq. (6) evaluated with explicit matrices;
  * Lambda = g I reproduces the scalar-decay (Gated DeltaNet) path of the oracle, truncation and
    all, as SEED states for theta = 1, Lambda = g I;
  * recall: with b = 1 and |k| = 1, S_t^T k = v;
  * eps > 0: the open-loop bound of SEED Prop. 3 with lambda_t = max entry of Lambda_t;
  * a compaction leaves the frozen part with unit vectors, sorted by the renormalized sigma.
"""
import numpy as np
import pytest

from oracle import OraclePool, schedule_due
from oracle.oracle import OracleState


def _orth(rng, d, m):
    q, _ = np.linalg.qr(rng.standard_normal((d, m)))
    return q[:, :m]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _inputs(rng, N, d_k, d_v, Pk, Pv, lam_lo=0.8):
    k = rng.standard_normal((N, Pk.shape[1])) @ Pk.T + 0.1 * rng.standard_normal((N, d_k))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.standard_normal((N, Pk.shape[1])) @ Pk.T + 0.1 * rng.standard_normal((N, d_k))
    v = rng.standard_normal((N, Pv.shape[1])) @ Pv.T + 0.1 * rng.standard_normal((N, d_v))
    lam = rng.uniform(lam_lo, 1.0, (N, d_k))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal(N)))
    return q, k, v, lam, b


def _pair(N, d_k, d_v, K, r, rule, eps=0.0, L=-1, promote=False):
    Pf = OraclePool(N, d_k, d_v, K, r, L, promote, diag_decay=True)
    Pd = OraclePool(N, d_k, d_v, K, r, L, promote, diag_decay=True)
    for s in range(N):
        Pf.set_state(s, OracleState(rule=rule, eps=eps))
        Pd.set_state(s, OracleState(S=np.zeros((d_k, d_v)), rule=rule, eps=eps))
    return Pf, Pd


@pytest.mark.parametrize("rule,shape,offsets", [(1, (16, 32), (0,)), (0, (16, 32), (0,)),
                                                (1, (24, 20), tuple(range(8)))])
def test_eps0_factored_equals_dense(rule, shape, offsets):
    d_k, d_v = shape
    rng = np.random.default_rng(40 + rule)
    N, K = 8, 8
    Pf, Pd = _pair(N, d_k, d_v, K, 8, rule)
    groups = np.arange(N, dtype=np.int32) % len(offsets)
    Pk, Pv = _orth(rng, d_k, 4), _orth(rng, d_v, 4)
    worst_o = worst_s = 0.0
    for t in range(1, 97):
        q, k, v, lam, b = _inputs(rng, N, d_k, d_v, Pk, Pv)
        of = Pf.decode(q, k, v, lam, b)
        od = Pd.decode(q, k, v, lam, b)
        due = schedule_due(t, K, list(offsets))
        if due:
            Pf.compact(np.nonzero(np.isin(groups, due))[0])
        worst_o = max(worst_o, _rel(of, od))
        for s in range(N):
            worst_s = max(worst_s, _rel(Pf.reconstruct(s), Pd.reconstruct(s)))
    assert worst_o <= 1e-12 and worst_s <= 1e-12, (worst_o, worst_s)
    assert sum(Pf.compactions(s) for s in range(N)) >= N * 11


def test_eps0_promotion_keeps_state():
    """Promotion into the dense form after a compaction is exact under per-channel decay too."""
    rng = np.random.default_rng(44)
    N, d_k, d_v, K = 6, 16, 32, 8
    Pf, Pd = _pair(N, d_k, d_v, K, 8, 1, promote=True)
    Pk, Pv = _orth(rng, d_k, 4), _orth(rng, d_v, 4)
    for t in range(1, 65):
        q, k, v, lam, b = _inputs(rng, N, d_k, d_v, Pk, Pv)
        of, od = Pf.decode(q, k, v, lam, b), Pd.decode(q, k, v, lam, b)
        if t % K == 0:
            Pf.compact()
        assert _rel(of, od) <= 1e-12
    assert all(Pf.get_state(s).dense for s in range(N))
    for s in range(N):
        assert _rel(Pf.reconstruct(s), Pd.reconstruct(s)) <= 1e-12


@pytest.mark.parametrize("rule", [0, 1])
def test_dense_step_is_eq6(rule):
    """S_t = (I - theta b k k^T) Lambda S_{t-1} + b' k v^T with explicit matrices (theta = rule;
    the scalar rule writes k v^T, i.e. b' = 1), and o = S_t^T q."""
    rng = np.random.default_rng(45 + rule)
    d_k, d_v = 9, 7
    S = rng.standard_normal((d_k, d_v))
    P = OraclePool(1, d_k, d_v, 8, 8, -1, False, diag_decay=True)
    P.set_state(0, OracleState(S=S, rule=rule))
    for _ in range(4):
        k = rng.standard_normal(d_k)
        k /= np.linalg.norm(k)
        v, q = rng.standard_normal(d_v), rng.standard_normal(d_k)
        lam = rng.uniform(0.5, 1.0, d_k)
        b = 0.37
        o = P.decode(q[None], k[None], v[None], lam[None], np.array([b]))[0]
        if rule == 1:
            S = (np.eye(d_k) - b * np.outer(k, k)) @ np.diag(lam) @ S + b * np.outer(k, v)
        else:
            S = np.diag(lam) @ S + np.outer(k, v)
        assert np.allclose(P.reconstruct(0), S, atol=1e-13)
        assert np.allclose(o, S.T @ q, atol=1e-12)


@pytest.mark.parametrize("rule", [0, 1])
def test_uniform_channels_equal_scalar_decay(rule):
    """Lambda = g I: the per-channel path gives the scalar-decay path's outputs, states, ranks and
    singular values (eps > 0, so truncation decisions are compared too)."""
    rng = np.random.default_rng(47 + rule)
    N, d_k, d_v, K = 12, 16, 24, 8
    Pd_ = OraclePool(N, d_k, d_v, K, 4, -1, True, diag_decay=True)
    Ps = OraclePool(N, d_k, d_v, K, 4, -1, True)
    for s in range(N):
        R = 1 + s % 5
        U, V = _orth(rng, d_k, R), _orth(rng, d_v, R)
        sig = np.geomspace(1.0, 0.05, R)
        for P in (Pd_, Ps):
            P.set_state(s, OracleState(U.T, V.T, sig, rule=rule, eps=0.01))
    Pk, Pv = _orth(rng, d_k, 3), _orth(rng, d_v, 3)
    dropped = 0
    for t in range(1, 65):
        q, k, v, _, b = _inputs(rng, N, d_k, d_v, Pk, Pv)
        g = rng.uniform(0.85, 1.0, N)
        o1 = Pd_.decode(q, k, v, np.repeat(g[:, None], d_k, axis=1), b)
        o2 = Ps.decode(q, k, v, g, b)
        assert _rel(o1, o2) <= 1e-12
        if t % K == 0:
            Pd_.compact()
            Ps.compact()
            for s in range(N):
                a, c = Pd_.get_state(s), Ps.get_state(s)
                assert a.dense == c.dense
                if not a.dense:
                    assert len(a.sigma) == len(c.sigma)
                    assert np.allclose(a.sigma, c.sigma, rtol=1e-11, atol=0)
                assert _rel(Pd_.reconstruct(s), Ps.reconstruct(s)) <= 1e-11
                dropped += Pd_.bound(s) > 0
    assert dropped > 0


def test_recall_with_channel_decay():
    """b = 1, |k| = 1: (I - k k^T) kills the decayed state along k, so S_t^T k = v, factored
    (eps = 0) and dense alike."""
    rng = np.random.default_rng(49)
    d_k, d_v = 12, 9
    U, V = _orth(rng, d_k, 5), _orth(rng, d_v, 5)
    sig = np.geomspace(2.0, 0.1, 5)
    for dense in (False, True):
        P = OraclePool(1, d_k, d_v, 8, 8, -1, False, diag_decay=True)
        P.set_state(0, OracleState(S=U @ np.diag(sig) @ V.T, rule=1) if dense
                    else OracleState(U.T, V.T, sig, rule=1, eps=0.0))
        for _ in range(3):
            k = rng.standard_normal(d_k)
            k /= np.linalg.norm(k)
            v = rng.standard_normal(d_v)
            P.decode(k[None], k[None], v[None], rng.uniform(0.3, 1.0, (1, d_k)), np.array([1.0]))
            assert np.allclose(P.reconstruct(0).T @ k, v, atol=1e-13)


@pytest.mark.parametrize("rule", [0, 1])
def test_truncation_error_bound(rule):
    """SEED Prop. 3 with |Phi_t| <= lambda_t (largest entry of Lambda_t), every step."""
    rng = np.random.default_rng(50 + rule)
    N, d_k, d_v, K = 16, 16, 24, 8
    Pf, Pd = _pair(N, d_k, d_v, K, 4, rule, eps=0.05, L=99)
    Pk, Pv = _orth(rng, d_k, 3), _orth(rng, d_v, 3)
    dropped_any = False
    for t in range(1, 97):
        q, k, v, lam, b = _inputs(rng, N, d_k, d_v, Pk, Pv, lam_lo=0.7)
        Pf.decode(q, k, v, lam, b)
        Pd.decode(q, k, v, lam, b)
        if t % K == 0:
            Pf.compact()
        for s in range(N):
            err = np.linalg.norm(Pf.reconstruct(s) - Pd.reconstruct(s))
            bnd = Pf.bound(s)
            dropped_any |= bnd > 0
            assert err <= bnd + 1e-12 * max(1.0, np.linalg.norm(Pd.reconstruct(s))), (t, s, err, bnd)
    assert dropped_any


def test_compaction_renormalizes_and_sorts_frozen():
    """Frozen components decayed along different channels: after a compaction every stored u has
    unit norm, the frozen list is sorted by sigma |Lambda u| (descending), and, at eps = 0, the
    state is unchanged."""
    d = 8
    e = np.eye(d)
    P = OraclePool(1, d, d, 2, 1, 99, False, diag_decay=True)
    # active e0 (sigma 4); frozen e1 (sigma 2.0), e2 (sigma 1.5) -- the channel decay swaps their order
    P.set_state(0, OracleState(np.stack([e[0], e[1], e[2]]), np.stack([e[0], e[1], e[2]]),
                               np.array([4.0, 2.0, 1.5]), rule=0, eps=0.0))
    lam = np.ones(d)
    lam[1] = 0.5
    k = e[5]
    P.decode(np.zeros((1, d)), k[None], e[5][None], lam[None])
    P.decode(np.zeros((1, d)), k[None], e[5][None], lam[None])
    S_before = P.reconstruct(0)
    P.compact([0])
    st = P.get_state(0)
    assert np.allclose(np.linalg.norm(st.U, axis=1), 1.0, atol=1e-14)
    assert np.allclose(P.reconstruct(0), S_before, atol=1e-13)
    # local: 4 (e0) and 2 (two pad writes of e5 e5^T); frozen: 1.5 (e2) now above 2 * 0.25 = 0.5 (e1)
    assert np.allclose(st.sigma, [4.0, 2.0, 1.5, 0.5], atol=1e-13)
    assert np.allclose(np.abs(st.U[2]), e[2]) and np.allclose(np.abs(st.U[3]), e[1])

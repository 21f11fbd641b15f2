"""Pins for the fp64 CPU oracle (CPU only).

Each test ties the oracle to something other than itself: a value the pages
print, a closed form, an invariant, a library routine on a special case, or a
brute-force dense computation.  Plausible mistakes (a dropped term, a wrong
sign, index or transpose, a missing decay) fail at least one of them.
"""
import json
import os

import numpy as np
import pytest

from oracle import OraclePool, brand_update, householder_qr, jacobi_svd, schedule_due
from oracle.oracle import rsvd_init
from oracle.oracle import OracleState

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _orth(rng, d, m):
    q, r = np.linalg.qr(rng.standard_normal((d, m)))
    return q * np.sign(np.diag(r))


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# --------------------------------------------------------------------------
# building blocks against textbook / library facts
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape,rank", [((16, 9), 9), ((128, 16), 16), ((20, 12), 5), ((6, 10), 6), ((32, 16), 0)])
def test_householder_qr(shape, rank):
    rng = np.random.default_rng(1)
    d, m = shape
    A = rng.standard_normal((d, rank)) @ rng.standard_normal((rank, m)) if rank else np.zeros((d, m))
    Q, R = householder_qr(A)
    p = min(d, m)
    assert Q.shape == (d, p) and R.shape == (p, m)
    assert np.allclose(Q.T @ Q, np.eye(p), atol=1e-13)
    assert np.allclose(np.tril(R, -1), 0.0)
    assert np.linalg.norm(Q @ R - A) <= 1e-13 * max(1.0, np.linalg.norm(A))
    # |diag R| agrees with LAPACK's QR (unique up to signs for full column rank)
    if rank == min(d, m) == m:
        R2 = np.linalg.qr(A, mode="r")
        assert np.allclose(np.abs(np.diag(R)), np.abs(np.diag(R2)), rtol=1e-10)


@pytest.mark.parametrize("shape,rank", [((16, 16), 16), ((16, 16), 5), ((10, 16), 10), ((24, 7), 7), ((3, 3), 0)])
def test_jacobi_svd_matches_lapack(shape, rank):
    rng = np.random.default_rng(2)
    r_, c_ = shape
    A = rng.standard_normal((r_, rank)) @ rng.standard_normal((rank, c_)) if rank else np.zeros(shape)
    U, s, V = jacobi_svd(A)
    ref = np.linalg.svd(A, compute_uv=False)
    k = min(shape)
    assert np.all(np.diff(s) <= 0)
    assert np.allclose(s[:k], ref, atol=1e-12 * max(1.0, ref[0] if ref.size else 1.0))
    assert np.allclose(s[k:], 0.0, atol=1e-12 * max(1.0, s[0]))
    assert np.allclose(V.T @ V, np.eye(c_), atol=1e-13)
    assert np.linalg.norm(U @ np.diag(s) @ V.T - A) <= 1e-12 * max(1.0, np.linalg.norm(A))
    nz = s > 1e-12 * max(1.0, s[0])
    assert np.allclose(U[:, nz].T @ U[:, nz], np.eye(nz.sum()), atol=1e-12)


def test_jacobi_svd_of_diagonal_is_sorted_abs():
    # special case with a closed form: the SVD of a diagonal matrix is its |entries|, sorted
    d = np.array([0.3, -2.0, 0.0, 1.5, -0.7])
    U, s, V = jacobi_svd(np.diag(d))
    assert np.allclose(s, np.sort(np.abs(d))[::-1], atol=0)


def _projector_clusters_match(U1, s1, U2, s2, gap=1e-6, tol=1e-10):
    """Compare subspaces by projectors of singular-value clusters split at relative gaps."""
    smax = max(s1[0], 1e-300)
    cuts = [0]
    for i in range(1, len(s1)):
        if (s1[i - 1] - s1[i]) / smax > gap:
            cuts.append(i)
    cuts.append(len(s1))
    for a, b in zip(cuts[:-1], cuts[1:]):
        if s1[a] <= 1e-9 * smax:
            break
        P1 = U1[:, a:b] @ U1[:, a:b].T
        P2 = U2[:, a:b] @ U2[:, a:b].T
        assert np.linalg.norm(P1 - P2) <= tol, (a, b)


@pytest.mark.parametrize("case", ["random", "k_in_span", "duplicate_k", "zero_pad", "partial_pad", "m_gt_dk"])
def test_brand_equals_full_svd(case):
    """One Brand update equals the SVD of the concatenated factors (SinkState 4.2 (ii): U_C Sigma_C V_C^T = Q_L C Q_R^T)."""
    rng = np.random.default_rng({"random": 3, "k_in_span": 4, "duplicate_k": 5, "zero_pad": 6, "partial_pad": 7,
                                 "m_gt_dk": 8}[case])
    d_k, d_v, ra, n = 24, 20, 8, 8
    if case == "m_gt_dk":
        d_k, d_v = 12, 20
    if case == "partial_pad":
        n = 3
    Ua = _orth(rng, d_k, min(ra, d_k))
    Va = _orth(rng, d_v, ra)[:, :Ua.shape[1]]
    ra = Ua.shape[1]
    sa = np.sort(rng.uniform(0.1, 3.0, ra))[::-1]
    Kp = rng.standard_normal((d_k, n))
    W = rng.standard_normal((d_v, n))
    c = rng.uniform(0.2, 1.0, n)
    if case == "k_in_span":
        Kp[:, :4] = Ua @ rng.standard_normal((ra, 4))
    if case == "duplicate_k":
        Kp[:, 1] = Kp[:, 0]
        Kp[:, 2] = 2.0 * Kp[:, 0]
    if case == "zero_pad":
        Kp[:] = 0.0
        W[:] = 0.0
    UC = np.hstack([Ua, Kp])
    VC = np.hstack([Va, W])
    sc = np.concatenate([sa, c])
    U, s, V = brand_update(UC, VC, sc)
    M = UC @ np.diag(sc) @ VC.T
    Ur, sr, Vrt = np.linalg.svd(M)
    k = min(len(s), len(sr))
    assert np.allclose(s[:k], sr[:k], atol=1e-12 * sr[0])
    assert np.allclose(s[k:], 0.0, atol=1e-12 * sr[0])
    assert np.linalg.norm(U @ np.diag(s) @ V.T - M) <= 1e-12 * np.linalg.norm(M)
    _projector_clusters_match(U, s, Ur, sr)
    _projector_clusters_match(V, s, Vrt.T, sr)


# --------------------------------------------------------------------------
# the recurrence: eps = 0 reproduces the dense recurrence exactly
# --------------------------------------------------------------------------
def _drive(Pf, Pd, N, d_k, d_v, steps, rule, K, rng, check_every=1, eps=0.0, offsets=(0,), groups=None):
    """Run a factored pool and a dense pool on the same inputs; yield per-step errors."""
    groups = np.zeros(N, np.int32) if groups is None else groups
    Pk = _orth(rng, d_k, 4)
    Pv = _orth(rng, d_v, 4)
    worst_o, worst_s = 0.0, 0.0
    for t in range(1, steps + 1):
        k = rng.standard_normal((N, 4)) @ Pk.T + 0.05 * rng.standard_normal((N, d_k))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q = rng.standard_normal((N, 4)) @ Pk.T + 0.05 * rng.standard_normal((N, d_k))
        v = rng.standard_normal((N, 4)) @ Pv.T + 0.05 * rng.standard_normal((N, d_v))
        a = rng.uniform(0.9, 1.0, N)
        b = 1.0 / (1.0 + np.exp(-rng.standard_normal(N)))
        of = Pf.decode(q, k, v, a, b)
        od = Pd.decode(q, k, v, a, b)
        due = schedule_due(t, K, list(offsets))
        if due:
            Pf.compact(np.nonzero(np.isin(groups, due))[0])
        if t % check_every == 0:
            worst_o = max(worst_o, _rel(of, od))
            for s in range(N):
                worst_s = max(worst_s, _rel(Pf.reconstruct(s), Pd.reconstruct(s)))
    return worst_o, worst_s


def _pair(N, d_k, d_v, K, r, rule, promote=False):
    Pf = OraclePool(N, d_k, d_v, K, r, -1, promote)
    Pd = OraclePool(N, d_k, d_v, K, r, -1, promote)
    for s in range(N):
        Pf.set_state(s, OracleState(rule=rule, eps=0.0))
        Pd.set_state(s, OracleState(S=np.zeros((d_k, d_v)), rule=rule, eps=0.0))
    return Pf, Pd


def test_eps0_factored_equals_dense_scalar():
    """eps = 0, no promotion: the factored path equals the dense recurrence (16x32, 256 steps)."""
    rng = np.random.default_rng(10)
    Pf, Pd = _pair(64, 16, 32, 8, 8, 0)
    wo, ws = _drive(Pf, Pd, 64, 16, 32, 256, 0, 8, rng, check_every=8)
    assert wo <= 1e-12 and ws <= 1e-12, (wo, ws)
    assert Pf.compactions(0) == 32


def test_eps0_factored_equals_dense_delta():
    """Same for the delta rule at 128x128, staggered groups (offsets 0..7)."""
    rng = np.random.default_rng(11)
    N = 8
    Pf, Pd = _pair(N, 128, 128, 8, 8, 1)
    wo, ws = _drive(Pf, Pd, N, 128, 128, 48, 1, 8, rng, check_every=4, offsets=tuple(range(8)),
                    groups=np.arange(N, dtype=np.int32))
    assert wo <= 1e-12 and ws <= 1e-12, (wo, ws)


def test_eps0_promotion_keeps_state():
    """With promotion on, the dense conversion is exact (16x32: L = 10)."""
    rng = np.random.default_rng(12)
    Pf, Pd = _pair(16, 16, 32, 8, 8, 0, promote=True)
    wo, ws = _drive(Pf, Pd, 16, 16, 32, 64, 0, 8, rng, check_every=8)
    assert wo <= 1e-12 and ws <= 1e-12
    assert all(Pf.get_state(s).dense for s in range(16))


# --------------------------------------------------------------------------
# worked example printed by the paper (Figure 6)
# --------------------------------------------------------------------------
def test_fig6_decay_and_buffer_weights():
    g = json.load(open(os.path.join(GOLD, "sinkstate_fig6_worked_example.json")))
    rng = np.random.default_rng(13)
    U, V = _orth(rng, 4, 3), _orth(rng, 4, 3)
    P = OraclePool(1, 4, 4, g["K"], g["r"], 99, False)
    P.set_state(0, OracleState(U.T, V.T, np.array(g["sigma0"]), eps=g["eps"]))
    ks = [np.array([0.74, 0.52, 1.48, 1.04]), np.array([1.68, 0.64, -0.64, -0.72])]
    vs = [np.array([0.52, 1.04, 0.74, 1.48]), np.array([0.48, -0.04, 0.76, -0.48])]
    q = np.zeros((1, 4))
    P.decode(q, ks[0][None], vs[0][None], np.array([g["alpha"][0]]))
    st = P.get_state(0)
    assert np.allclose(st.sigma, g["after_step1_sigma_printed"], atol=0.006)
    assert np.allclose(st.pc, g["after_step1_pad_weights"], atol=0)
    P.decode(q, ks[1][None], vs[1][None], np.array([g["alpha"][1]]))
    st = P.get_state(0)
    assert np.allclose(st.sigma, g["after_step2_exact_sigma"], atol=1e-14)
    assert np.allclose(st.pc, g["after_step2_exact_pad_weights"], atol=1e-15)
    assert np.allclose(np.concatenate([st.sigma, st.pc]), g["after_step2_printed"], atol=0.006)


def test_fig6_merge_and_threshold():
    """Active part + pad whose local SVD is [8.99, 2.08, 0.04], frozen [1.41, 0.79], eps = 0.1
    keeps [8.99, 2.08, 1.41]; the top r = 1 stays active."""
    g = json.load(open(os.path.join(GOLD, "sinkstate_fig6_worked_example.json")))
    e = np.eye(6)
    loc = g["local_svd_sigma_printed"]
    fr = g["frozen_sigma_printed"]
    P = OraclePool(1, 6, 6, 2, g["r"], 99, False)
    # components: active (8.99 on e0), frozen (1.41 on e3, 0.79 on e4); pad: e1 (2.08), e2 (0.04)
    P.set_state(0, OracleState(np.stack([e[0], e[3], e[4]]), np.stack([e[0], e[3], e[4]]),
                               np.array([loc[0], fr[0], fr[1]]), np.stack([e[1], e[2]]), np.stack([e[1], e[2]]),
                               np.array([loc[1], loc[2]]), eps=g["eps"]))
    S_before = P.reconstruct(0)
    P.compact([0])
    st = P.get_state(0)
    assert np.allclose(st.sigma, g["kept_printed"], atol=1e-14)
    assert len(st.pc) == 0
    # what was dropped is exactly 0.79 e4 e4^T + 0.04 e2 e2^T, and its norm is the error bound
    S_after = P.reconstruct(0)
    dropped = S_before - S_after
    assert np.allclose(dropped, 0.79 * np.outer(e[4], e[4]) + 0.04 * np.outer(e[2], e[2]), atol=1e-14)
    assert abs(P.bound(0) - np.linalg.norm(dropped)) <= 1e-14
    assert abs(g["threshold_printed"] - g["eps"] * g["kept_printed"][0]) < 1e-12


# --------------------------------------------------------------------------
# exact reconstruction, idempotence, empty states
# --------------------------------------------------------------------------
def test_rank_r_state_reconstructs_exactly():
    rng = np.random.default_rng(14)
    U, V = _orth(rng, 128, 8), _orth(rng, 80, 8)
    sig = 0.5 ** np.arange(8)
    P = OraclePool(1, 128, 80, 8, 8, -1, True)
    P.set_state(0, OracleState(U.T, V.T, sig, eps=3e-3))
    M = U @ np.diag(sig) @ V.T
    assert _rel(P.reconstruct(0), M) <= 1e-15
    q = rng.standard_normal((1, 128))
    assert _rel(P.readout(q)[0], M.T @ q[0]) <= 1e-14
    # empty pad: compaction is a no-op
    before = P.get_state(0)
    P.compact([0])
    after = P.get_state(0)
    assert np.array_equal(before.sigma, after.sigma) and np.array_equal(before.U, after.U)


def test_zero_weight_pad_compaction_is_idempotent():
    rng = np.random.default_rng(15)
    U, V = _orth(rng, 32, 10), _orth(rng, 24, 10)
    sig = np.geomspace(1.0, 0.01, 10)
    P = OraclePool(1, 32, 24, 8, 8, -1, False)
    P.set_state(0, OracleState(U.T, V.T, sig, rng.standard_normal((3, 32)), rng.standard_normal((3, 24)),
                               np.zeros(3), eps=1e-3))
    P.compact([0])
    st = P.get_state(0)
    assert np.allclose(st.sigma, sig, rtol=1e-13)
    assert np.linalg.norm(st.U @ st.U.T - np.eye(10)) < 1e-12
    assert _rel(P.reconstruct(0), U @ np.diag(sig) @ V.T) <= 1e-13


def test_empty_state_reads_zero_and_all_zero_becomes_empty():
    P = OraclePool(1, 8, 8, 4, 2, -1, True)
    P.set_state(0, OracleState(eps=1e-3))
    assert np.all(P.readout(np.ones((1, 8))) == 0.0)
    # a pad of zero vectors compacts to an empty state (sigma_max = 0)
    P.decode(np.ones((1, 8)), np.zeros((1, 8)), np.zeros((1, 8)), np.array([0.9]))
    P.compact([0])
    st = P.get_state(0)
    assert len(st.sigma) == 0 and len(st.pc) == 0


def test_tie_order_local_first():
    """Equal singular values: the local result precedes the frozen component."""
    e = np.eye(5)
    P = OraclePool(1, 5, 5, 2, 1, 99, False)
    P.set_state(0, OracleState(np.stack([e[0], e[3]]), np.stack([e[0], e[3]]), np.array([2.0, 1.0]),
                               np.stack([e[1]]), np.stack([e[1]]), np.array([1.0]), eps=0.0))
    P.compact([0])
    st = P.get_state(0)
    assert np.allclose(st.sigma, [2.0, 1.0, 1.0])
    assert abs(st.U[1] @ e[1]) == 1.0 and abs(st.U[2] @ e[3]) == 1.0


# --------------------------------------------------------------------------
# delta rule identities
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dense", [False, True])
def test_delta_rule_recall(dense):
    """alpha = beta = 1, |k| = 1: S_t^T k = v (the delta rule writes v at key k exactly)."""
    rng = np.random.default_rng(16)
    d_k, d_v = 12, 9
    U, V = _orth(rng, d_k, 5), _orth(rng, d_v, 5)
    sig = np.geomspace(2.0, 0.1, 5)
    P = OraclePool(1, d_k, d_v, 8, 8, -1, False)
    if dense:
        P.set_state(0, OracleState(S=U @ np.diag(sig) @ V.T, rule=1))
    else:
        P.set_state(0, OracleState(U.T, V.T, sig, rule=1, eps=0.0))
    for _ in range(3):
        k = rng.standard_normal(d_k)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(d_v)
        P.decode(k[None], k[None], v[None], np.array([1.0]), np.array([1.0]))
        assert np.allclose(P.reconstruct(0).T @ k, v, atol=1e-13)


def test_delta_rule_beta0_is_pure_decay():
    rng = np.random.default_rng(17)
    U, V = _orth(rng, 10, 4), _orth(rng, 6, 4)
    P = OraclePool(1, 10, 6, 8, 8, -1, False)
    P.set_state(0, OracleState(U.T, V.T, np.ones(4), rule=1))
    S0 = P.reconstruct(0)
    k = rng.standard_normal(10)
    k /= np.linalg.norm(k)
    P.decode(rng.standard_normal((1, 10)), k[None], rng.standard_normal((1, 6)), np.array([0.7]), np.array([0.0]))
    assert np.allclose(P.reconstruct(0), 0.7 * S0, atol=1e-14)


def test_delta_rule_equals_projector_form():
    """S_t = a (I - b k k^T) S_{t-1} + b k v^T (Gated DeltaNet) computed by brute force."""
    rng = np.random.default_rng(18)
    d_k, d_v = 7, 5
    S = rng.standard_normal((d_k, d_v))
    P = OraclePool(1, d_k, d_v, 8, 8, -1, False)
    P.set_state(0, OracleState(S=S, rule=1))
    k = rng.standard_normal(d_k)
    k /= np.linalg.norm(k)
    v, q = rng.standard_normal(d_v), rng.standard_normal(d_k)
    a, b = 0.93, 0.4
    o = P.decode(q[None], k[None], v[None], np.array([a]), np.array([b]))[0]
    S1 = a * (np.eye(d_k) - b * np.outer(k, k)) @ S + b * np.outer(k, v)
    assert np.allclose(P.reconstruct(0), S1, atol=1e-14)
    assert np.allclose(o, S1.T @ q, atol=1e-13)


# --------------------------------------------------------------------------
# eps > 0: open-loop error bound (SEED Prop. 3) holds every step
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rule", [0, 1])
def test_truncation_error_bound(rule):
    rng = np.random.default_rng(19 + rule)
    N, d_k, d_v, K = 16, 16, 24, 8
    Pf = OraclePool(N, d_k, d_v, K, 4, 99, False)
    Pd = OraclePool(N, d_k, d_v, K, 4, 99, False)
    for s in range(N):
        Pf.set_state(s, OracleState(rule=rule, eps=0.05))
        Pd.set_state(s, OracleState(S=np.zeros((d_k, d_v)), rule=rule))
    Pk = _orth(rng, d_k, 3)
    dropped_any = False
    for t in range(1, 97):
        k = rng.standard_normal((N, 3)) @ Pk.T + 0.2 * rng.standard_normal((N, d_k))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q = rng.standard_normal((N, d_k))
        v = rng.standard_normal((N, d_v))
        a = rng.uniform(0.85, 1.0, N)
        b = rng.uniform(0.1, 0.9, N)
        Pf.decode(q, k, v, a, b)
        Pd.decode(q, k, v, a, b)
        if t % K == 0:
            Pf.compact()
        for s in range(N):
            err = np.linalg.norm(Pf.reconstruct(s) - Pd.reconstruct(s))
            bnd = Pf.bound(s)
            dropped_any |= bnd > 0
            assert err <= bnd + 1e-12 * max(1.0, np.linalg.norm(Pd.reconstruct(s))), (t, s, err, bnd)
    assert dropped_any


def test_truncation_is_best_approximation_for_orthogonal_state():
    """When frozen and local components are mutually orthogonal, compaction equals the
    truncated SVD of the whole state (SinkState 2.2: truncation is Frobenius-optimal)."""
    rng = np.random.default_rng(21)
    d = 20
    B = _orth(rng, d, d)
    C = _orth(rng, d, d)
    P = OraclePool(1, d, d, 4, 3, 99, False)
    sig_a = np.array([5.0, 3.0, 1.0])
    sig_f = np.array([0.8, 0.02, 0.01])
    pad_w = np.array([2.0, 0.6, 0.005, 0.3])
    P.set_state(0, OracleState(np.vstack([B[:, :3].T, B[:, 3:6].T]), np.vstack([C[:, :3].T, C[:, 3:6].T]),
                               np.concatenate([sig_a, sig_f]), B[:, 6:10].T, C[:, 6:10].T, pad_w, eps=0.01))
    M = P.reconstruct(0)
    P.compact([0])
    U, s, Vt = np.linalg.svd(M)
    keep = s >= 0.01 * s[0]
    best = U[:, keep] @ np.diag(s[keep]) @ Vt[keep]
    assert _rel(P.reconstruct(0), best) <= 1e-13
    assert np.allclose(P.get_state(0).sigma, s[keep], rtol=1e-13)


# --------------------------------------------------------------------------
# dense fallback threshold, stagger and arithmetic printed by the pages
# --------------------------------------------------------------------------
def test_dense_threshold_and_init_fallback():
    g = json.load(open(os.path.join(GOLD, "memory_arithmetic.json")))
    for (dk, dv), L in [((128, 80), 49), ((128, 128), g["threshold_128x128"]), ((16, 32), 10)]:
        P = OraclePool(2, dk, dv, 8, 8, -1, True)
        assert P.L == L
        rng = np.random.default_rng(dk + dv)
        for s, R in enumerate([L, L + 1]):
            U = rng.standard_normal((R, dk))
            V = rng.standard_normal((R, dv))
            sig = np.sort(rng.uniform(0.1, 1, R))[::-1]
            P.set_state(s, OracleState(U, V, sig))
            assert P.get_state(s).dense == (R > L)
            assert _rel(P.reconstruct(s), U.T @ np.diag(sig) @ V) <= 1e-14
        # the memory reason: (d_k + d_v) r values exceed d_k d_v exactly when r > L
        assert (dk + dv) * L <= dk * dv < (dk + dv) * (L + 1)


def test_memory_arithmetic():
    g = json.load(open(os.path.join(GOLD, "memory_arithmetic.json")))
    a, b, r = g["d_small"], g["d_large"], g["rank"]
    assert a * b == g["dense_values"] and 4 * a * b == g["dense_bytes"]
    assert r * (a + b + 1) == g["factor_values_rank8"] == g["pad_values_full"]
    assert 4 * 2 * r * (a + b + 1) == g["total_bytes"]
    assert g["n_layers"] * g["n_heads"] * g["n_requests"] == g["n_states"]
    assert abs(g["n_states"] * g["dense_bytes"] / 1e9 - g["dense_total_gb_printed"]) < 0.05


def test_stagger_three_layers_per_step():
    g = json.load(open(os.path.join(GOLD, "memory_arithmetic.json")))
    L, K = g["stagger_layers"], g["stagger_K"]
    offsets = [l % K for l in range(L)]
    per_layer_count = np.zeros(L, int)
    for t in range(1, 4 * K + 1):
        due = schedule_due(t, K, offsets)
        assert len(due) == g["stagger_per_step"]
        per_layer_count[due] += 1
    assert np.all(per_layer_count == 4)     # each layer once every K steps


def test_pad_overflow_is_reported():
    P = OraclePool(1, 4, 4, 2, 1, -1, False)
    P.set_state(0, OracleState(eps=0.0))
    x = np.ones((1, 4))
    P.decode(x, x, x, np.array([0.9]))
    P.decode(x, x, x, np.array([0.9]))
    with pytest.raises(RuntimeError):
        P.decode(x, x, x, np.array([0.9]))


# --------------------------------------------------------------------------
# randomized block SVD initialization after prefill
# --------------------------------------------------------------------------
def test_rsvd_fig6a_blocks_and_stop():
    """Figure 6(a): blocks of 2 on a 4x4 state with singular values [8.0, 1.95, 1.10, 0.06] and
    eps = 0.1: the first block finds [8.0, 1.95], the second [1.10, 0.06]; 0.06 < 0.8 is dropped
    and no third block is taken."""
    g = json.load(open(os.path.join(GOLD, "sinkstate_fig6a_rsvd_init.json")))
    rng = np.random.default_rng(61)
    U, V = _orth(rng, 4, 4), _orth(rng, 4, 4)
    S = (U * np.array(g["state_sigma"])) @ V.T
    om = rng.standard_normal((3, 4, g["block"]))
    Uo, Vo, so = rsvd_init(S, om, g["eps"], iters=40)
    assert np.allclose(so, g["kept_printed"], atol=1e-9)
    assert abs(g["threshold_printed"] - g["eps"] * g["block1_printed"][0]) < 1e-12
    # what is left out is the 0.06 component: the reconstruction error is exactly it
    err = np.linalg.norm(S - Uo.T @ np.diag(so) @ Vo, 2)
    assert abs(err - g["block2_printed"][1]) < 1e-9
    # the threshold is eps times the first block's sigma_0, not the current block's largest:
    # a second-block 0.5 is below 0.8 although it is above 0.1 * 1.10
    S2 = (U * np.array([8.0, 1.95, 1.10, 0.5])) @ V.T
    _, _, so2 = rsvd_init(S2, om, g["eps"], iters=40)
    assert np.allclose(so2, [8.0, 1.95, 1.10], atol=1e-9)


@pytest.mark.parametrize("shape,rank,b", [((16, 12), 5, 8), ((32, 20), 8, 8), ((24, 24), 3, 4)])
def test_rsvd_exact_when_rank_fits_one_block(shape, rank, b):
    """A state whose rank fits in one block: the range finder spans it exactly, so the first
    block is the exact SVD (numpy's, to 1e-10) and the second finds nothing (stop)."""
    rng = np.random.default_rng(7 + rank)
    d_k, d_v = shape
    U, V = _orth(rng, d_k, rank), _orth(rng, d_v, rank)
    sig = np.sort(rng.uniform(0.1, 3.0, rank))[::-1]
    S = (U * sig) @ V.T
    om = rng.standard_normal((3, d_k, b))
    Uo, Vo, so = rsvd_init(S, om, 1e-8, iters=1)
    assert len(so) == rank
    assert np.allclose(so, np.linalg.svd(S, compute_uv=False)[:rank], rtol=1e-10, atol=0)
    assert np.linalg.norm(S - Uo.T @ np.diag(so) @ Vo) <= 1e-12 * np.linalg.norm(S)
    assert np.allclose(Uo @ Uo.T, np.eye(rank), atol=1e-10)
    assert np.allclose(Vo @ Vo.T, np.eye(rank), atol=1e-10)


def test_rsvd_full_block_is_exact_svd():
    """With one block as wide as the state, orth(S^T Omega) spans everything and the block SVD is
    the SVD of the state (numpy's singular values to 1e-10); eps drops the tail exactly as the
    threshold says."""
    rng = np.random.default_rng(5)
    d_k, d_v = 12, 8
    S = rng.standard_normal((d_k, d_v)) * np.logspace(0, -3, d_v)
    ref = np.linalg.svd(S, compute_uv=False)
    om = rng.standard_normal((1, d_k, d_v))
    eps = 0.02
    Uo, Vo, so = rsvd_init(S, om, eps, iters=1)
    keep = ref[ref >= eps * ref[0]]
    assert np.allclose(so, keep, rtol=1e-10, atol=0)
    assert np.allclose(np.linalg.norm(S - Uo.T @ np.diag(so) @ Vo, 2), ref[len(keep)], rtol=1e-8)


def test_rsvd_blocks_cover_the_state_and_zero_state_is_empty():
    """Blocks after the first are taken from the residual: on a full-rank state with eps = 0
    they keep going until max_rank, and the factors then reconstruct the state exactly.
    A zero state has no component."""
    rng = np.random.default_rng(9)
    S = rng.standard_normal((10, 6))
    om = rng.standard_normal((3, 10, 2))
    Uo, Vo, so = rsvd_init(S, om, 0.0, iters=2)
    assert len(so) == 6
    assert np.linalg.norm(S - Uo.T @ np.diag(so) @ Vo) <= 1e-12 * np.linalg.norm(S)
    Uz, Vz, sz = rsvd_init(np.zeros((10, 6)), om, 0.1, iters=2)
    assert len(sz) == 0


# --------------------------------------------------------------------------
# the bound's per-step decay is exact: after a compaction drops a known E, decode steps that
# write nothing (k = 0, v = 0) only decay the state, so the factored state stays exactly
# (prod alpha) E away from the untruncated one, and SEED Prop. 3's bound is attained
# --------------------------------------------------------------------------
@pytest.mark.parametrize("promote", [False, True])
@pytest.mark.parametrize("rule,dense_ref", [(0, False), (1, False), (0, True), (1, True)])
def test_bound_decays_exactly_and_is_attained(rule, dense_ref, promote):
    """With promote, the compaction leaves 3 > L = 2 components and the state goes dense: its
    bound must keep decaying on the dense path."""
    g = json.load(open(os.path.join(GOLD, "sinkstate_fig6_worked_example.json")))
    e = np.eye(6)
    loc, fr = g["local_svd_sigma_printed"], g["frozen_sigma_printed"]
    comps = dict(U=np.stack([e[0], e[3], e[4]]), V=np.stack([e[0], e[3], e[4]]),
                 sigma=np.array([loc[0], fr[0], fr[1]]), PK=np.stack([e[1], e[2]]), PW=np.stack([e[1], e[2]]),
                 pc=np.array([loc[1], loc[2]]))
    P = OraclePool(1, 6, 6, 2, g["r"], 2 if promote else 99, promote)
    P.set_state(0, OracleState(**comps, rule=rule, eps=g["eps"]), as_init=False)   # no fallback test at load
    S0 = P.reconstruct(0)
    R = OraclePool(1, 6, 6, 2, g["r"], 99, False)   # the same state, never truncated
    R.set_state(0, OracleState(S=S0, rule=rule) if dense_ref else OracleState(**comps, rule=rule, eps=0.0),
                as_init=False)
    if not dense_ref:
        R.compact([0])   # eps = 0: exact up to rounding, and R's pad is free again
    P.compact([0])
    E = 0.79 * np.outer(e[4], e[4]) + 0.04 * np.outer(e[2], e[2])   # what the Figure 6 example drops
    assert abs(P.bound(0) - np.linalg.norm(E)) <= 1e-14
    assert P.get_state(0).dense == promote
    alphas = [0.9, 0.8, 0.95, 0.7, 0.99]   # fewer than K = 2 steps between compactions of R
    prod = 1.0
    z = np.zeros((1, 6))
    for t, a in enumerate(alphas[:1]):
        P.decode(z, z, z, np.array([a]), np.array([0.5]))
        R.decode(z, z, z, np.array([a]), np.array([0.5]))
        prod *= a
        assert abs(P.bound(0) - prod * np.linalg.norm(E)) <= 1e-14, (t, P.bound(0))
        err = np.linalg.norm(P.reconstruct(0) - R.reconstruct(0))
        assert abs(err - P.bound(0)) <= 1e-14, (t, err, P.bound(0))
    # a second compaction of the zero-weight pad drops nothing more; the bound keeps decaying
    P.compact([0])
    for a in alphas[1:]:
        if not dense_ref:
            R.compact([0])   # eps = 0: exact, keeps R's pad from filling
        P.decode(z, z, z, np.array([a]), np.array([0.5]))
        R.decode(z, z, z, np.array([a]), np.array([0.5]))
        P.compact([0])
        prod *= a
        assert abs(P.bound(0) - prod * np.linalg.norm(E)) <= 1e-14, (a, P.bound(0))
        err = np.linalg.norm(P.reconstruct(0) - R.reconstruct(0))
        assert abs(err - P.bound(0)) <= 1e-14, (a, err, P.bound(0))


@pytest.mark.parametrize("promote", [False, True])
def test_bound_decays_with_the_largest_channel_decay(promote):
    """Per-channel decay: the contraction factor is the largest channel decay; with every channel
    decaying alike the bound is attained exactly."""
    rng = np.random.default_rng(31)
    d = 8
    U, V = _orth(rng, d, 3), _orth(rng, d, 3)
    P = OraclePool(1, d, d, 8, 2, 1 if promote else 99, promote, diag_decay=True)
    # two components and one pad slot orthogonal to them, whose weight 0.01 falls below 0.05 * 4
    P.set_state(0, OracleState(U[:, :2].T, V[:, :2].T, np.array([4.0, 1.0]), U[:, 2:].T, V[:, 2:].T,
                               np.array([0.01]), eps=0.05), as_init=False)
    S0 = P.reconstruct(0)   # before the truncation
    P.compact([0])
    assert P.get_state(0).dense == promote
    assert abs(P.bound(0) - 0.01) <= 1e-15
    prod = 1.0
    z = np.zeros((1, d))
    for lam in [0.9, 0.97, 0.8]:
        P.decode(z, z, z, np.full((1, d), lam), np.array([0.3]))
        prod *= lam
        assert abs(P.bound(0) - 0.01 * prod) <= 1e-15
        err = np.linalg.norm(P.reconstruct(0) - prod * S0)
        assert abs(err - P.bound(0)) <= 1e-14
    # unequal channel decays: the bound follows the largest one and still holds
    lam = np.linspace(0.5, 0.9, d)[None]
    P.decode(z, z, z, lam, np.array([0.3]))
    assert abs(P.bound(0) - 0.01 * prod * 0.9) <= 1e-15
    Sref = (lam[0][:, None] * prod) * S0
    assert np.linalg.norm(P.reconstruct(0) - Sref) <= P.bound(0) + 1e-14

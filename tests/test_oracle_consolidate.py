"""Pins for the oracle's consolidation of the frozen part (CPU only).

SinkState 4.3 "Asynchronous CPU Consolidation", Figure 7(a): the frozen
components are replaced by the exact SVD of their sum, truncated below
eps * sigma_0, with the active part and the pad left as they are.  The pins
tie it to LAPACK's SVD of the dense frozen matrix, to closed forms for two
components, to Eckart-Young for the dropped part, to the dense recurrence at
eps = 0, and to the decision printed in Figure 7(a).
"""
import json
import os

import numpy as np
import pytest

from oracle import OraclePool
from oracle.oracle import OracleState

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x):
    return x / np.linalg.norm(x)


def _orth(rng, d, m):
    q, r = np.linalg.qr(rng.standard_normal((d, m)))
    return q * np.sign(np.diag(r))


def _redundant_state(rng, d_k, d_v, r, n_dirs, per_dir, noise, eps, n_pad=3):
    """r orthonormal active components with large sigma, then n_dirs clusters of per_dir
    near-duplicate frozen components (directions perturbed by `noise`), then a pad."""
    Ua, Va = _orth(rng, d_k, r).T, _orth(rng, d_v, r).T
    sa = np.linspace(10.0, 7.0, r)
    Uf, Vf, sf = [], [], []
    for _ in range(n_dirs):
        u0, v0 = rng.standard_normal(d_k), rng.standard_normal(d_v)
        for _ in range(per_dir):
            Uf.append(_unit(u0 + noise * rng.standard_normal(d_k)))
            Vf.append(_unit(v0 + noise * rng.standard_normal(d_v)))
            sf.append(rng.uniform(0.3, 3.0))
    sf = np.array(sf)
    U = np.vstack([Ua, np.array(Uf)])
    V = np.vstack([Va, np.array(Vf)])
    sig = np.concatenate([sa, sf])
    PK = rng.standard_normal((n_pad, d_k))
    PW = rng.standard_normal((n_pad, d_v))
    pc = rng.uniform(0.5, 1.0, n_pad)
    return OracleState(U, V, sig, PK, PW, pc, rule=0, eps=eps)


def _pool(st, d_k, d_v, r, K=8):
    P = OraclePool(1, d_k, d_v, K=K, r=r, promote=False)
    P.set_state(0, st, as_init=False)
    return P


@pytest.mark.parametrize("d_k,d_v,r,n_dirs,per_dir,noise,eps", [
    (16, 32, 4, 3, 4, 0.05, 1e-2), (128, 128, 8, 6, 7, 0.02, 1e-2), (80, 128, 8, 5, 6, 0.1, 3e-3),
    (32, 16, 2, 4, 5, 0.0, 1e-3)])
def test_consolidate_equals_lapack_svd_of_frozen_part(d_k, d_v, r, n_dirs, per_dir, noise, eps):
    rng = np.random.default_rng(d_k + 3 * d_v + n_dirs)
    st = _redundant_state(rng, d_k, d_v, r, n_dirs, per_dir, noise, eps)
    P = _pool(st, d_k, d_v, r)
    before = P.get_state(0)
    P.consolidate()
    after = P.get_state(0)
    # active part and pad untouched, bit for bit
    assert np.array_equal(after.U[:r], before.U[:r]) and np.array_equal(after.V[:r], before.V[:r])
    assert np.array_equal(after.sigma[:r], before.sigma[:r])
    assert np.array_equal(after.PK, before.PK) and np.array_equal(after.PW, before.PW)
    assert np.array_equal(after.pc, before.pc)
    # the frozen part is the truncated SVD of the dense frozen matrix
    Mf = (before.U[r:].T * before.sigma[r:]) @ before.V[r:]
    Ul, sl, Vlt = np.linalg.svd(Mf)
    s0 = max(before.sigma[0], before.sigma[r])
    keep = sl >= eps * s0
    k = int(keep.sum())
    sf = after.sigma[r:]
    assert len(sf) == k and k < len(before.sigma) - r  # redundancy removed
    assert np.allclose(sf, sl[:k], rtol=1e-11, atol=0)
    assert np.all(np.diff(sf) <= 0)
    Mk = (Ul[:, :k] * sl[:k]) @ Vlt[:k]
    Mo = (after.U[r:].T * sf) @ after.V[r:]
    assert np.linalg.norm(Mo - Mk) <= 1e-11 * np.linalg.norm(Mk)
    assert np.allclose(after.U[r:] @ after.U[r:].T, np.eye(k), atol=1e-12)
    assert np.allclose(after.V[r:] @ after.V[r:].T, np.eye(k), atol=1e-12)
    P.close()


def test_consolidate_error_is_the_dropped_part():
    """Eckart-Young: the state moves by exactly the dropped singular values, and the
    open-loop bound grows by that Frobenius norm."""
    rng = np.random.default_rng(5)
    d_k, d_v, r, eps = 24, 40, 3, 0.08
    st = _redundant_state(rng, d_k, d_v, r, 4, 4, 0.3, eps)
    P = _pool(st, d_k, d_v, r)
    S0 = P.reconstruct(0)
    b0 = P.bound(0)
    before = P.get_state(0)
    P.consolidate()
    S1 = P.reconstruct(0)
    Mf = (before.U[r:].T * before.sigma[r:]) @ before.V[r:]
    sl = np.linalg.svd(Mf, compute_uv=False)
    thr = eps * max(before.sigma[0], before.sigma[r])
    dropped = sl[sl < thr]
    assert len(dropped) > 0 and np.any(dropped > 1e-6)
    err = np.linalg.norm(S1 - S0)
    assert abs(err - np.sqrt(np.sum(dropped ** 2))) <= 1e-11 * np.linalg.norm(S0)
    assert abs((P.bound(0) - b0) - np.sqrt(np.sum(dropped ** 2))) <= 1e-11 * np.linalg.norm(S0)
    P.close()


def _two_frozen(cu, cv, s1, s2, s0, eps, d=4, sign=1.0, seed=9):
    """One active component (s0) and two frozen unit components with the given cosines."""
    rng = np.random.default_rng(seed)
    Q = _orth(rng, d, 3)
    W = _orth(rng, d, 3)
    u0, v0 = Q[:, 0], W[:, 0]
    u1, v1 = Q[:, 1], W[:, 1]
    u2 = cu * Q[:, 1] + np.sqrt(1 - cu * cu) * Q[:, 2]
    v2 = sign * (cv * W[:, 1] + np.sqrt(1 - cv * cv) * W[:, 2])
    U = np.vstack([u0, u1, u2])
    V = np.vstack([v0, v1, v2])
    return OracleState(U, V, np.array([s0, s1, s2]), rule=0, eps=eps)


def test_fig7a_two_frozen_components():
    g = json.load(open(os.path.join(GOLD, "sinkstate_fig7a_consolidation.json")))
    s1, s2 = g["frozen_sigma"]
    cu, cv = g["cos_u"], g["cos_v"]
    st = _two_frozen(cu, cv, s1, s2, g["sigma0"], g["eps"])
    P = _pool(st, 4, 4, g["r"])
    P.consolidate()
    after = P.get_state(0)
    # the printed decision: rank 3 -> 2, the active value stays, one frozen value is kept
    assert len(after.sigma) == g["rank_after"]
    assert after.sigma[0] == g["sigma0"]
    assert abs(after.sigma[1] - g["sigma_after_printed"][1]) <= 0.01 * g["sigma_after_printed"][1]
    # closed forms for the sum of two unit rank-one terms
    su, sv = np.sqrt(1 - cu * cu), np.sqrt(1 - cv * cv)
    F2 = s1 * s1 + s2 * s2 + 2 * s1 * s2 * cu * cv
    det = s1 * s2 * su * sv
    big = np.sqrt((F2 + np.sqrt(F2 * F2 - 4 * det * det)) / 2)  # roots of x^2 - F2 x + det^2
    small = det / big
    assert abs(after.sigma[1] - big) <= 1e-12 * big
    assert small < g["threshold_printed"] <= g["eps"] * g["sigma0"] + 1e-12
    assert abs(P.bound(0) - small) <= 1e-12
    P.close()


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_duplicate_and_opposite_directions_merge(sign):
    """Two frozen copies of one direction merge into sigma1 + sigma2; with the v of the second
    reversed they cancel to |sigma1 - sigma2|.  The remainder is at rounding level (1e-32 here),
    so any eps above rounding drops it."""
    st = _two_frozen(1.0, 1.0, 2.5, 1.5, 9.0, 1e-9, d=6, sign=sign)
    P = _pool(st, 6, 6, 1)
    P.consolidate()
    after = P.get_state(0)
    want = 4.0 if sign > 0 else 1.0
    assert len(after.sigma) == 2
    assert abs(after.sigma[1] - want) <= 1e-12 * want
    P.close()


def test_sigma0_is_the_largest_stored_value_before_consolidation():
    """sigma_0 = max(first active, first frozen) of the stored values before the SVD.  A frozen
    part that merges into a value above the active one raises the threshold only for the next
    consolidation."""
    rng = np.random.default_rng(3)
    d, eps = 8, 0.05
    Q, W = _orth(rng, d, 3), _orth(rng, d, 3)
    U = np.vstack([Q[:, 0], Q[:, 1], Q[:, 1], Q[:, 2]])
    V = np.vstack([W[:, 0], W[:, 1], W[:, 1], W[:, 2]])
    sig = np.array([5.0, 4.0, 4.0, 0.3])
    P = _pool(OracleState(U, V, sig, rule=0, eps=eps), d, d, 1)
    P.consolidate()
    a = P.get_state(0)
    # threshold 0.05 * 5 = 0.25: the merged 8 and the 0.3 are both kept
    assert len(a.sigma) == 3 and abs(a.sigma[1] - 8.0) < 1e-12 and abs(a.sigma[2] - 0.3) < 1e-12
    assert a.sigma[0] == 5.0
    P.consolidate()
    b = P.get_state(0)
    # now sigma_0 = 8 and the threshold 0.4 drops the 0.3
    assert len(b.sigma) == 2 and abs(b.sigma[1] - 8.0) < 1e-12
    P.close()


def test_noop_cases_and_idempotence():
    rng = np.random.default_rng(4)
    d_k, d_v, r = 16, 24, 4
    P = OraclePool(4, d_k, d_v, K=8, r=r, promote=False)
    S = rng.standard_normal((d_k, d_v))
    P.set_state(0, OracleState(S=S, rule=0, eps=1e-2))
    U, V = _orth(rng, d_k, 3).T, _orth(rng, d_v, 3).T
    P.set_state(1, OracleState(U, V, np.array([3.0, 2.0, 1.0]), rule=0, eps=1e-2), as_init=False)
    P.set_state(2, OracleState(rule=0, eps=1e-2))
    P.set_state(3, _redundant_state(rng, d_k, d_v, r, 3, 3, 0.2, 1e-2), as_init=False)
    before = [P.get_state(s) for s in range(4)]
    P.consolidate()
    a = [P.get_state(s) for s in range(4)]
    assert np.array_equal(a[0].S, S)                      # dense: unchanged
    assert np.array_equal(a[1].U, before[1].U) and np.array_equal(a[1].sigma, before[1].sigma)  # no frozen part
    assert len(a[2].sigma) == 0                            # empty state
    P.consolidate([3])
    b = P.get_state(3)
    assert len(b.sigma) == len(a[3].sigma)
    assert np.allclose(b.sigma, a[3].sigma, rtol=1e-12, atol=0)
    Sa = (a[3].U.T * a[3].sigma) @ a[3].V
    Sb = (b.U.T * b.sigma) @ b.V
    assert np.linalg.norm(Sa - Sb) <= 1e-12 * np.linalg.norm(Sa)
    P.close()


@pytest.mark.parametrize("rule", [0, 1])
def test_eps0_run_with_consolidation_equals_dense(rule):
    """At eps = 0 a run of decode steps, compactions and consolidations stays equal to the
    dense recurrence (consolidation then drops only exact zeros)."""
    rng = np.random.default_rng(20 + rule)
    N, d_k, d_v, K, r = 8, 16, 24, 4, 3
    Pf = OraclePool(N, d_k, d_v, K=K, r=r, promote=False)
    Pd = OraclePool(N, d_k, d_v, K=K, r=r, promote=False)
    for s in range(N):
        Pf.set_state(s, OracleState(rule=rule, eps=0.0))
        Pd.set_state(s, OracleState(S=np.zeros((d_k, d_v)), rule=rule, eps=0.0))
    worst = 0.0
    for t in range(1, 97):
        q = rng.standard_normal((N, d_k))
        k = rng.standard_normal((N, d_k))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        v = rng.standard_normal((N, d_v))
        a = rng.uniform(0.9, 1.0, N)
        b = 1 / (1 + np.exp(-rng.standard_normal(N))) if rule else None
        of = Pf.decode(q, k, v, a, b)
        od = Pd.decode(q, k, v, a, b)
        worst = max(worst, np.max(np.abs(of - od)) / max(np.max(np.abs(od)), 1e-30))
        if t % K == 0:
            Pf.compact()
            if t % (2 * K) == 0:
                Pf.consolidate()
    for s in range(N):
        Sf, Sd = Pf.reconstruct(s), Pd.reconstruct(s)
        worst = max(worst, np.linalg.norm(Sf - Sd) / np.linalg.norm(Sd))
    assert worst <= 1e-11, worst
    assert max(len(Pf.get_state(s).sigma) for s in range(N)) > r  # frozen parts existed
    Pf.close()
    Pd.close()


def test_mid_run_reload_keeps_the_active_frozen_split():
    """After a consolidation the frozen list may start above the last active value; a state
    reloaded as a mid-run state keeps its split, so both copies compact identically."""
    rng = np.random.default_rng(8)
    d, eps = 8, 0.01
    Q, W = _orth(rng, d, 4), _orth(rng, d, 4)
    U = np.vstack([Q[:, 0], Q[:, 1], Q[:, 2], Q[:, 2]])
    V = np.vstack([W[:, 0], W[:, 1], W[:, 2], W[:, 2]])
    P = _pool(OracleState(U, V, np.array([6.0, 5.0, 4.0, 3.5]), rule=0, eps=eps), d, d, 2)
    P.consolidate()
    a = P.get_state(0)
    assert len(a.sigma) == 3 and abs(a.sigma[2] - 7.5) < 1e-12 and a.sigma[2] > a.sigma[1]
    a.PK = rng.standard_normal((2, d))
    a.PW = rng.standard_normal((2, d))
    a.pc = np.array([1.0, 0.5])
    P2 = _pool(a, d, d, 2)
    b = P2.get_state(0)
    assert np.array_equal(b.sigma, a.sigma) and np.array_equal(b.U, a.U)
    P3 = _pool(OracleState(a.U, a.V, a.sigma, a.PK, a.PW, a.pc, rule=0, eps=eps), d, d, 2)
    P2.compact()
    P3.compact()
    assert np.array_equal(P2.reconstruct(0), P3.reconstruct(0))
    # the compaction merges the frozen 7.5 into the active part: the first two values are the top two
    c = P2.get_state(0)
    assert c.sigma[0] >= c.sigma[1] >= c.sigma[2]
    P.close()
    P2.close()
    P3.close()

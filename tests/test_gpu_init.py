"""GPU parity of the randomized block SVD initialization (ss_rsvd_init) against the fp64 oracle.

Both sides get the same fp32 states and the same Gaussian blocks (drawn on the host from a
seeded generator).  Compared per state: the number of components (equal, except when a
singular value lies within 1e-5 sigma_0 of the threshold: then the values that differ must all lie
there, the shared ones are still compared, and the reconstructions may differ by those values only),
each singular value to 1e-4 sigma_0 (the normwise form used for compaction) and, at or above
1e-2 sigma_0, to 1e-4 of itself, and the reconstruction to 1e-4 in relative Frobenius norm.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
from oracle.oracle import rsvd_init as oracle_rsvd


def _states(rng, n, d_k, d_v, kind):
    """Prefill-like states: a decaying spectrum plus a little noise ('lowrank'), or noise only
    ('flat', full rank), or an exact low rank that fits one block ('exact')."""
    S = np.zeros((n, d_k, d_v))
    for i in range(n):
        if kind == "flat":
            S[i] = rng.standard_normal((d_k, d_v)) / np.sqrt(d_v)
            continue
        r = int(rng.integers(1, min(d_k, d_v, 24) + 1)) if kind == "lowrank" else int(rng.integers(1, 5))
        U = np.linalg.qr(rng.standard_normal((d_k, r)))[0]
        V = np.linalg.qr(rng.standard_normal((d_v, r)))[0]
        sig = 0.6 ** np.arange(r) * rng.uniform(0.5, 2.0)
        S[i] = (U * sig) @ V.T
        if kind == "lowrank":
            S[i] += 1e-4 * rng.standard_normal((d_k, d_v)) / np.sqrt(d_v)
    return S.astype(np.float32)


def _check(d_k, d_v, b, nb, iters, eps, kind, n=24, seed=0):
    rng = np.random.default_rng(seed)
    S = _states(rng, n, d_k, d_v, kind)
    om = rng.standard_normal((n, nb, d_k, b)).astype(np.float32)
    max_rank = min(d_k, d_v, nb * b)
    u, v, sg, rk = ss.rsvd_init(torch.from_numpy(S).cuda(), torch.from_numpy(om).cuda(), eps, iters=iters,
                                max_rank=max_rank)
    torch.cuda.synchronize()
    u, v, sg, rk = u.cpu().numpy(), v.cpu().numpy(), sg.cpu().numpy(), rk.cpu().numpy()
    worst = {"sigma": 0.0, "sigma_rel": 0.0, "S": 0.0}
    guard = 0
    for i in range(n):
        Uo, Vo, so = oracle_rsvd(S[i].astype(np.float64), om[i].astype(np.float64), eps, iters=iters,
                                 max_rank=max_rank)
        R = int(rk[i])
        s0 = so[0] if len(so) else 1.0
        Rc = min(R, len(so))
        extra = 0.0
        if R != len(so):
            # a decision at the threshold may differ only inside the guard band: every value one
            # side keeps and the other drops lies within 1e-5 sigma_0 of eps sigma_0
            xo, xg = so[Rc:], sg[i, Rc:R].astype(np.float64)
            assert np.all(np.abs(xo - eps * s0) <= 1e-5 * s0) and np.all(np.abs(xg - eps * s0) <= 1e-5 * s0), \
                (i, R, len(so), so, sg[i, :R])
            guard += 1
            extra = float(np.sqrt(np.sum(xo ** 2) + np.sum(xg ** 2)))
        if Rc == 0:
            continue
        d = np.abs(sg[i, :Rc].astype(np.float64) - so[:Rc])
        worst["sigma"] = max(worst["sigma"], float(np.max(d) / s0))
        # per value, where an fp32 factorization can resolve it (Weyl: |d sigma| <= ||d S||, about
        # 1e-7 sigma_0 here): relative error of every value at or above 1e-2 sigma_0
        big = so[:Rc] >= 1e-2 * s0
        if big.any():
            worst["sigma_rel"] = max(worst["sigma_rel"], float(np.max(d[big] / so[:Rc][big])))
        Sg = (u[i, :R].T.astype(np.float64) * sg[i, :R]) @ v[i, :R].astype(np.float64)
        So = (Uo.T * so) @ Vo
        nS = max(np.linalg.norm(So), 1e-30)
        worst["S"] = max(worst["S"], max(0.0, np.linalg.norm(Sg - So) - extra) / nS)
    print(kind, (d_k, d_v, b, nb, iters), worst, "guard", guard)
    for k, x in worst.items():
        assert x <= TOL, f"{k}: {x:.3e} > {TOL} ({worst})"
    return rk


@pytest.mark.parametrize("d_k,d_v,b", [(16, 32, 4), (128, 80, 8), (128, 128, 8), (44, 64, 8), (12, 20, 3),
                                       (256, 64, 16), (64, 256, 16)])
def test_rsvd_lowrank(d_k, d_v, b):
    nb = -(-min(d_k, d_v) // b)
    _check(d_k, d_v, b, nb, 2, 3e-3, "lowrank", seed=d_k + d_v)


def test_rsvd_exact_rank_one_block():
    rk = _check(128, 80, 8, 3, 1, 1e-3, "exact", seed=3)
    assert rk.max() <= 4


def test_rsvd_flat_states_reach_max_rank():
    """Noise-only states keep every block up to max_rank (they are the ones the dense fallback
    takes), and the blocks are taken from the residual."""
    rk = _check(32, 24, 8, 3, 2, 1e-3, "flat", seed=4)
    assert (rk == 24).all()


def test_rsvd_rejects_bad_shapes():
    S = torch.zeros(1, 16, 16, device="cuda")
    om = torch.zeros(1, 2, 16, 17, device="cuda")
    with pytest.raises(ss.SinkStateError):
        ss.rsvd_init(S, om, 1e-3)


def test_pool_from_dense_states():
    """Prefill-like 128x80 states through state_pool_from_dense: low-rank ones become factored
    with the oracle's components, full-rank ones (rank > L = 49) are kept dense and exactly as
    given; the pool then decodes in lock-step with the oracle."""
    from parity_util import oracle_from_export, rel_out_err, reconstruct
    rng = np.random.default_rng(11)
    n, d_k, d_v, b = 48, 128, 80, 8
    S = np.concatenate([_states(rng, 40, d_k, d_v, "lowrank"), _states(rng, 8, d_k, d_v, "flat")])
    nb = 7
    om = rng.standard_normal((n, nb, d_k, b)).astype(np.float32)
    eps = 3e-3
    pool = ss.state_pool_from_dense(S, om, eps, group_of_state=np.arange(n) % 4, group_offset=[0, 2, 4, 6])
    st = ss.pool_stats(pool)
    assert st["n_dense"] == 8
    ex = ss.state_export(pool, np.arange(n))
    worst = 0.0
    for i, x in enumerate(ex):
        if i >= 40:
            assert x["dense"] and np.array_equal(x["S"], S[i]), i
            continue
        assert not x["dense"]
        Uo, Vo, so = oracle_rsvd(S[i].astype(np.float64), om[i].astype(np.float64), eps, iters=2,
                                 max_rank=min(d_k, d_v, nb * b))
        So = (Uo.T * so) @ Vo
        worst = max(worst, np.linalg.norm(reconstruct(x) - So) / np.linalg.norm(So))
        assert len(x["sigma"]) == len(so)
    assert worst <= TOL, worst
    # a few decode steps in lock-step with the oracle
    import rank_recurrent_state_amd.workloads as W
    eps_a = np.full(n, eps)
    for t in range(1, 4):
        q = torch.randn(n, d_k, device="cuda")
        k = torch.nn.functional.normalize(torch.randn(n, d_k, device="cuda"), dim=1)
        v = torch.randn(n, d_v, device="cuda")
        al = torch.rand(n, device="cuda") * 0.05 + 0.95
        before = ss.state_export(pool, np.arange(n))
        P = oracle_from_export(before, eps_a, d_k, d_v, 8, 8)
        o = torch.empty(n, d_v, device="cuda")
        ss.decode_step(pool, q, k, v, al, None, o)
        torch.cuda.synchronize()
        f64 = lambda x: x.cpu().numpy().astype(np.float64)  # noqa: E731
        oo = P.decode(f64(q), f64(k), f64(v), f64(al), None)
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(n)])
        e = rel_out_err(o.cpu().numpy(), oo, Sn, np.linalg.norm(f64(q), axis=1))
        assert e.max() <= TOL, (t, e.max())
    pool.close()


@pytest.mark.parametrize("d_k,d_v,b", [(4, 8, 1), (8, 4, 4), (20, 12, 2)])
def test_rsvd_small_edge_shapes(d_k, d_v, b):
    nb = -(-min(d_k, d_v) // b)
    _check(d_k, d_v, b, nb, 3, 1e-3, "lowrank", n=16, seed=d_k * 7 + d_v)


def test_pool_from_dense_all_dense_and_none_dense():
    """Every state given dense (full rank) or none (low rank): both create paths."""
    rng = np.random.default_rng(21)
    n, d_k, d_v, b = 16, 16, 32, 4
    S = _states(rng, n, d_k, d_v, "flat")
    om = rng.standard_normal((n, 4, d_k, b)).astype(np.float32)
    pool = ss.state_pool_from_dense(S, om, 1e-3)
    ex = ss.state_export(pool, np.arange(n))
    assert all(x["dense"] and np.array_equal(x["S"], S[i]) for i, x in enumerate(ex))
    pool.close()
    S2 = _states(rng, n, d_k, d_v, "exact")
    pool = ss.state_pool_from_dense(S2, om, 1e-3)
    ex = ss.state_export(pool, np.arange(n))
    from parity_util import reconstruct
    for i, x in enumerate(ex):
        assert not x["dense"]
        assert np.linalg.norm(reconstruct(x) - S2[i]) <= 1e-4 * np.linalg.norm(S2[i])
    pool.close()

"""GPU parity of the frozen-capacity limit.

A pool is created with room for at most r + max_frozen components per state.  When a compaction
keeps more (all above eps * sigma_max), the library keeps the largest r + max_frozen of the merged,
descending list and counts the excess in `cap_truncations`.  The pages set no such limit, so the
oracle compacts without it; the expected state is the oracle's merged list cut the same way, to its
r + max_frozen largest singular values.  Lock-step protocol and tolerances as in test_gpu_parity,
on both compaction variants (scalar decay and per-channel decay).
"""
import numpy as np
import pytest
import torch

from parity_util import GUARD, TOL, oracle_from_export, reconstruct, rel_out_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss


@pytest.mark.parametrize("diag", [False, True])
def test_frozen_capacity_keeps_the_largest(diag):
    rng = np.random.default_rng(21 + int(diag))
    dk, dv, K, r, fcap, N = 64, 44, 8, 4, 3, 9
    R = rng.integers(4, 8, N)
    off = np.concatenate([[0], np.cumsum(R)]).astype(np.int64)
    T = int(off[-1])
    u = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    sig = np.concatenate([np.sort(rng.uniform(0.2, 2, x))[::-1] for x in R]).astype(np.float32)
    rule = (np.arange(N) % 2).astype(np.uint8)
    eps = np.full(N, 1e-4, np.float32)
    pool = ss.state_pool_create(N, dk, dv, K, r, rule=rule, eps=eps, comp_off=off, u=u, v=v, sigma=sig,
                                group_offset=[0], promote_on_compact=False, max_frozen=fcap, diag_decay=diag)
    o = torch.empty(N, dv, device="cuda")
    ids = np.arange(N)
    cap = r + fcap
    worst, cut = 0.0, 0
    for t in range(1, 3 * K + 1):
        before = ss.state_export(pool, ids)
        q = torch.randn(N, dk, device="cuda")
        k = torch.nn.functional.normalize(torch.randn(N, dk, device="cuda"), dim=1)
        vv = torch.randn(N, dv, device="cuda")
        a = (0.9 + 0.1 * torch.rand((N, dk) if diag else (N,), device="cuda")).contiguous()
        b = torch.rand(N, device="cuda")
        P = oracle_from_export(before, eps, dk, dv, K, r, promote=False, diag_decay=diag)
        ss.decode_step(pool, q, k, vv, a, b, o)
        due = ss.schedule_due(pool, t)
        if due:
            ss.compact(pool, 0)
        torch.cuda.synchronize()
        oo = P.decode(q.cpu().numpy(), k.cpu().numpy(), vv.cpu().numpy(), a.cpu().numpy(), b.cpu().numpy())
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(N)])
        worst = max(worst, float(rel_out_err(o.cpu().numpy(), oo, Sn, np.linalg.norm(q.cpu().numpy(), axis=1)).max()))
        if not due:
            continue
        P.compact()
        after = ss.state_export(pool, ids)
        for j, st in enumerate(after):
            ost = P.get_state(j)
            so = np.asarray(ost.sigma, np.float64)
            order = np.argsort(-so, kind="stable")
            keep = order[:cap]
            sg = np.sort(st["sigma"].astype(np.float64))[::-1]
            assert len(sg) == min(cap, len(so)), (t, j, len(sg), len(so))
            if len(so) > cap:
                cut += 1
                if so[order[cap - 1]] - so[order[cap]] <= GUARD * so[order[0]]:
                    continue  # a tie at the cut: either component is a valid choice
            St = (ost.U[keep].T * so[keep]) @ ost.V[keep]
            err = np.linalg.norm(reconstruct(st) - St) / max(np.linalg.norm(St), 1e-30)
            assert err <= TOL, (t, j, err)
            assert np.max(np.abs(sg - so[keep]) / so[keep]) <= TOL, (t, j)
    st = ss.pool_stats(pool)
    pool.close()
    assert cut > 0 and st["cap_truncations"] > 0, (cut, st["cap_truncations"])
    assert st["jacobi_limit_hits"] == 0
    assert worst <= TOL, worst

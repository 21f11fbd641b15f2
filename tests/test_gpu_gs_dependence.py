"""GPU parity of the compaction when the pad's keys and values lie nearly, or exactly, in the span
of the active factors (SinkState 4.2 "(ii) Top-subspace SVD": the thin QRs of [U_a | K] and
[V_a | W]).

Each state gets keys k = U_a c + delta n (and, for the scalar rule, values v = V_a d + delta m),
with one residual scale delta per state, from well conditioned (1) through the range where the
GPU's Gram-Schmidt takes its second pass (a first pass that keeps less than a tenth of the squared
norm: delta around 0.3 and below) down to columns it must find dependent (delta <= 1e-5 and 0),
and states that repeat one key at every step.  Two compaction cycles run on each of the two
compaction kernels (two sides per wavefront, and the per-channel-decay one); the second cycle's
keys follow the active factors the first compaction left.  Lock-step protocol and tolerances as
in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare_compacted, oracle_from_export, rel_out_err, states_of

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss

DELTAS = [1.0, 0.5, 0.3, 0.2, 0.1, 3e-2, 1e-2, 1e-3, 1e-4, 1e-5, 1e-6, 1e-7, 0.0, -1.0, -1.0, 0.3]
# -1: the state repeats one random key (and value) at every step of a cycle


def _orth(rng, d, m):
    q, _ = np.linalg.qr(rng.standard_normal((d, m)))
    return q


@pytest.mark.parametrize("diag", [False, True])
def test_pads_near_the_active_span(diag):
    rng = np.random.default_rng(11 + int(diag))
    dk, dv, K, r = 128, 80, 8, 8
    N = len(DELTAS)
    R = np.full(N, r)
    off = np.concatenate([[0], np.cumsum(R)]).astype(np.int64)
    u = np.concatenate([_orth(rng, dk, r).T for _ in range(N)]).astype(np.float32)
    v = np.concatenate([_orth(rng, dv, r).T for _ in range(N)]).astype(np.float32)
    sig = np.tile(np.logspace(0.0, np.log10(0.05), r), N).astype(np.float32)
    rule = (np.arange(N) % 2).astype(np.uint8)
    eps = np.full(N, 1e-3, np.float32)
    pool = ss.state_pool_create(N, dk, dv, K, r, rule=rule, eps=eps, comp_off=off, u=u, v=v, sigma=sig,
                                group_offset=[0], promote_on_compact=False, max_frozen=64, diag_decay=diag)
    o = torch.empty(N, dv, device="cuda")
    ids = np.arange(N)
    worst = 0.0
    compactions = 0
    rep_k = rep_v = None
    for t in range(1, 2 * K + 1):
        before = ss.state_export(pool, ids)
        if (t - 1) % K == 0:  # a new cycle: keys follow the active factors the state has now
            Ua = [st["U"][:min(r, len(st["sigma"]))].T.astype(np.float64) for st in before]
            Va = [st["V"][:min(r, len(st["sigma"]))].T.astype(np.float64) for st in before]
            rep_k = rng.standard_normal((N, dk))
            rep_v = rng.standard_normal((N, dv))
        k = np.empty((N, dk))
        vv = np.empty((N, dv))
        for j, dl in enumerate(DELTAS):
            if dl < 0:
                k[j], vv[j] = rep_k[j], rep_v[j]
            else:
                k[j] = Ua[j] @ rng.standard_normal(Ua[j].shape[1]) + dl * rng.standard_normal(dk)
                vv[j] = Va[j] @ rng.standard_normal(Va[j].shape[1]) + dl * rng.standard_normal(dv)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        kt = torch.from_numpy(k.astype(np.float32)).cuda()
        vt = torch.from_numpy(vv.astype(np.float32)).cuda()
        q = torch.randn(N, dk, device="cuda")
        a = (0.9 + 0.1 * torch.rand((N, dk) if diag else (N,), device="cuda")).contiguous()
        b = torch.rand(N, device="cuda")
        P = oracle_from_export(before, eps, dk, dv, K, r, promote=False, diag_decay=diag)
        ss.decode_step(pool, q, kt, vt, a, b, o)
        due = ss.schedule_due(pool, t)
        if due:
            ss.compact(pool, 0)
        torch.cuda.synchronize()
        oo = P.decode(q.cpu().numpy(), kt.cpu().numpy(), vt.cpu().numpy(), a.cpu().numpy(), b.cpu().numpy())
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(N)])
        e = rel_out_err(o.cpu().numpy(), oo, Sn, np.linalg.norm(q.cpu().numpy(), axis=1))
        worst = max(worst, float(e.max()))
        if due:
            pre = states_of(P, N)
            P.compact()
            after = ss.state_export(pool, ids)
            ws, wsig, gd, bad = compare_compacted(after, P, eps, before=pre)
            assert not bad and ws <= TOL and wsig <= TOL, (t, ws, wsig, bad)
            if compactions == 0:
                # The first compaction's components all come from one SVD (no frozen part before
                # it).  U = Q_L U_hat is orthonormal to working precision whatever the pad held;
                # a missing second Gram-Schmidt pass would leave Q_L's nearly dependent columns
                # off by about u sqrt(n0 / nu), 1e-4 and more at delta <= 1e-4.  V is recovered
                # as C^T u_j / s_j, whose rounding error grows as u sigma_max / s_j, so V_i . V_j
                # is bounded after scaling by min(s_i, s_j) / sigma_max (the error of each
                # component s_j u_j v_j^T then stays at rounding level of the state).
                for j, st in enumerate(after):
                    if not st["dense"] and len(st["sigma"]):
                        sg = st["sigma"].astype(np.float64)
                        U, V = st["U"].astype(np.float64), st["V"].astype(np.float64)
                        off_u = np.abs(U @ U.T - np.eye(len(U))).max()
                        off_v = (np.abs(V @ V.T - np.eye(len(V))) * np.minimum.outer(sg, sg) / sg.max()).max()
                        assert off_u <= 1e-5 and off_v <= 1e-5, (DELTAS[j], off_u, off_v)
            compactions += 1
    pool.close()
    assert compactions == 2
    assert worst <= TOL, worst

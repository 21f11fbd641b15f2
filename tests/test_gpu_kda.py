"""GPU parity of per-channel decay (Kimi Delta Attention, SEED appendix B.1 eq. (6)) against the
oracle, which applies each step's diag(lambda) literally to every factor and pad key.

The GPU keeps the decays accumulated per key channel since the last compaction (pad keys stored
divided by them, queries scaled by them) and folds them into the factors at the compaction; an
export hands the oracle the effective state.  Lock-step protocol and tolerances as in
test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare_compacted, states_of, oracle_from_export, reconstruct, rel_out_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W
    from test_gpu_parity import _assert_worst, _lockstep, _pool_from_init


def _kda_pool(w, init, **kw):
    return _pool_from_init(w, init, diag_decay=True, **kw)


def test_kda_lockstep_one_request():
    """640 KDA states 128x128 (one request), random initial ranks 2..16, staggered groups."""
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _kda_pool(w, init)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 5), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24, check_readout=True)
    st = ss.pool_stats(pool)
    pool.close()
    print("kda", worst, "guard", guard, "n_dense", st["n_dense"], "max_rank", st["max_rank"])
    _assert_worst(worst)


def test_kda_dense_region_and_promotion():
    """L = 12: states above it start dense (buffered dense region with per-slot decays), and
    compactions promote more; decode, fold, readout and promotion against the oracle."""
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _kda_pool(w, init, dense_rank_limit=12)
    st0 = ss.pool_stats(pool)
    assert st0["n_dense"] == int(np.sum(np.diff(init["comp_off"]) > 12)) > 0
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 7), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24, check_readout=True, L=12)
    st = ss.pool_stats(pool)
    pool.close()
    print("kda dense", worst, "guard", guard, "n_dense", st0["n_dense"], "->", st["n_dense"])
    assert st["n_dense"] > st0["n_dense"]
    _assert_worst(worst)


def test_kda_fp16_factors():
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _kda_pool(w, init, factor_fp16=True)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 9), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 20, fp16=True)
    pool.close()
    print("kda fp16", worst, "guard", guard)
    _assert_worst(worst)


def test_kda_dense_baseline():
    """force_dense pool: the plain dense recurrence with per-channel decay, against the oracle's
    dense recurrence."""
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _kda_pool(w, init, force_dense=True)
    ids = np.arange(0, w.n_states, 11)
    worst, _ = _lockstep(w, init, pool, ids, 6, check_readout=True)
    pool.close()
    _assert_worst(worst)


@pytest.mark.parametrize("rule,fp16", [(0, False), (1, False), (0, True), (1, True)])
def test_kda_edge_shapes(rule, fp16):
    """Ragged counts, small and odd shapes, K = 1 and 3, both rules, decays down to 0.5; with fp16
    factors both fp16 decode kernels (eight elements per lane when d_k, d_v are multiples of 8).
    d = 256 takes the compaction's two float4 blocks per lane."""
    rng = np.random.default_rng(7 + rule)
    for (dk, dv, K, r, N) in [(4, 8, 1, 1, 37), (12, 20, 3, 2, 37), (64, 44, 8, 8, 9), (16, 32, 2, 3, 21),
                              (256, 16, 8, 8, 13), (40, 256, 2, 3, 9)]:
        R = rng.integers(0, 6, N)
        R[0] = 0
        off = np.concatenate([[0], np.cumsum(R)]).astype(np.int64)
        T = int(off[-1])
        u = rng.standard_normal((T, dk)).astype(np.float32)
        v = rng.standard_normal((T, dv)).astype(np.float32)
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        sig = np.concatenate([np.sort(rng.uniform(0.1, 2, x))[::-1] for x in R]).astype(np.float32)
        rl = np.full(N, rule, np.uint8)
        eps = np.full(N, 1e-3, np.float32)
        pool = ss.state_pool_create(N, dk, dv, K, r, rule=rl, eps=eps, comp_off=off, u=u, v=v, sigma=sig,
                                    group_offset=[0], promote_on_compact=False, max_frozen=64, diag_decay=True,
                                    factor_fp16=fp16)
        o = torch.empty(N, dv, device="cuda")
        ids = np.arange(N)
        worst = 0.0
        for t in range(1, 3 * K + 2):
            q = torch.randn(N, dk, device="cuda")
            k = torch.nn.functional.normalize(torch.randn(N, dk, device="cuda"), dim=1)
            vv = torch.randn(N, dv, device="cuda")
            a = 0.5 + 0.5 * torch.rand(N, dk, device="cuda")
            b = torch.rand(N, device="cuda")
            before = ss.state_export(pool, ids)
            P = oracle_from_export(before, eps, dk, dv, K, r, promote=False, diag_decay=True, factor_fp16=fp16)
            ss.decode_step(pool, q, k, vv, a, b, o)
            due = ss.schedule_due(pool, t)
            if due:
                ss.compact(pool, 0)
            torch.cuda.synchronize()
            oo = P.decode(q.cpu().numpy(), k.cpu().numpy(), vv.cpu().numpy(), a.cpu().numpy(), b.cpu().numpy())
            Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(N)])
            e = rel_out_err(o.cpu().numpy(), oo, Sn, np.linalg.norm(q.cpu().numpy(), axis=1))
            worst = max(worst, float(e.max()))
            if due:
                pre = states_of(P, len(ids))
                P.compact()
                after = ss.state_export(pool, ids)
                ws, wsig, gd, bad = compare_compacted(after, P, eps, fp16=fp16, before=pre)
                assert not bad and ws <= TOL and wsig <= TOL, (dk, dv, K, r, ws, wsig, bad)
                for st in after:  # the compaction folded the decays in: unit factors again
                    if not st["dense"] and len(st["sigma"]):
                        assert np.allclose(np.linalg.norm(st["U"], axis=1), 1.0, atol=2e-3 if fp16 else 1e-5)
        pool.close()
        assert worst <= TOL, (dk, dv, K, r, worst)


def test_kda_consolidation_is_rejected():
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _kda_pool(w, init)
    with pytest.raises(RuntimeError):
        ss.consolidate(pool)
    pool.close()


def test_kda_uniform_channels_match_scalar_pool():
    """lambda = alpha 1 on every channel: the per-channel pool follows the scalar-decay pool (same
    inputs, fp32 on both sides) to rounding, ranks included."""
    w = W.get("kda_delta", n_requests=1)
    init = W.initial_state(w)
    pd = _kda_pool(w, init)
    ps = _pool_from_init(w, init)
    gen = W.StepInputs(w, device="cuda")
    o1 = torch.empty(w.n_states, w.d_v, device="cuda")
    o2 = torch.empty_like(o1)
    worst = 0.0
    for t in range(1, 25):
        x = gen.generate(t)
        a = x["alpha"][:, 0].contiguous()
        ss.decode_step(pd, x["q"], x["k"], x["v"], a[:, None].expand(-1, w.d_k).contiguous(), x["beta"], o1)
        ss.decode_step(ps, x["q"], x["k"], x["v"], a, x["beta"], o2)
        for g in ss.schedule_due(pd, t):
            ss.compact(pd, g)
            ss.compact(ps, g)
        torch.cuda.synchronize()
        worst = max(worst, float(((o1 - o2).norm(dim=1) / o2.norm(dim=1).clamp_min(1e-30)).max()))
    s1, s2 = ss.pool_stats(pd), ss.pool_stats(ps)
    pd.close()
    ps.close()
    print("uniform channels vs scalar", worst, s1["active_components"] + s1["frozen_components"],
          s2["active_components"] + s2["frozen_components"])
    assert worst <= 1e-5

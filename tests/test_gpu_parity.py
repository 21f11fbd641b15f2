"""GPU parity: the HIP path (through the C-ABI) against the fp64 oracle.

Lock-step protocol: before each call the sampled states are exported from the
GPU (canonical form, fp32 upcast to fp64) and loaded into the oracle; both
sides then run the same call on bit-identical inputs and the results are
compared with the tolerances in parity_util.
"""
import numpy as np
import pytest
import torch

from parity_util import (TOL, active_projector_err, compare_compacted, oracle_from_export, reconstruct,
                         rel_out_err)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


def _pool_from_init(w, init, **kw):
    return ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"], **kw)


def _lockstep(w, init, pool, ids, steps, promote=True, check_readout=False, fp16=False, L=-1, t0=0):
    """Run `steps` decode(+compaction) steps in lock-step on the states `ids`.  fp16: the pool
    stores fp16 factors; the oracle rounds the factors it writes the same way, and every exported
    factor must be exactly representable in fp16."""
    gen = W.StepInputs(w, device="cuda")
    eps = init["eps"][ids]
    grp = init["group_of_state"][ids]
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    worst = {"o": 0.0, "S": 0.0, "S_c": 0.0, "sigma": 0.0, "proj": 0.0, "ro": 0.0}
    guard = 0
    for t in range(t0 + 1, t0 + steps + 1):
        x = gen.generate(t)
        before = ss.state_export(pool, ids)
        if fp16:
            _assert_fp16_factors(before, w.diag_decay)
        P = oracle_from_export(before, eps, w.d_k, w.d_v, w.K, w.r, L=L, promote=promote, factor_fp16=fp16,
                               diag_decay=w.diag_decay)
        sub = {k: v.cpu().numpy()[ids].astype(np.float64) for k, v in x.items()}
        if check_readout:
            ss.readout(pool, x["q"], o)
            torch.cuda.synchronize()
            oro = P.readout(sub["q"])
            Sn = np.array([np.linalg.norm(reconstruct(s)) for s in before])
            e = rel_out_err(o.cpu().numpy()[ids], oro, Sn, np.linalg.norm(sub["q"], axis=1))
            worst["ro"] = max(worst["ro"], float(e.max()))
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        torch.cuda.synchronize()
        oo = P.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
        after = ss.state_export(pool, ids)
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(len(ids))])
        e = rel_out_err(o.cpu().numpy()[ids], oo, Sn, np.linalg.norm(sub["q"], axis=1))
        worst["o"] = max(worst["o"], float(e.max()))
        for j, st in enumerate(after):
            So = P.reconstruct(j)
            worst["S"] = max(worst["S"], np.linalg.norm(reconstruct(st) - So) / max(np.linalg.norm(So), 1e-30))
        due = ss.schedule_due(pool, t)
        if due:
            for g in due:
                ss.compact(pool, g)
            P2 = oracle_from_export(after, eps, w.d_k, w.d_v, w.K, w.r, L=L, promote=promote, factor_fp16=fp16,
                                    diag_decay=w.diag_decay)
            sel = np.nonzero(np.isin(grp, due))[0]
            P2.compact(sel)
            comp = ss.state_export(pool, ids)
            ws, wsig, gd, bad = compare_compacted(comp, P2, eps, fp16=fp16, before=after)
            assert not bad, f"step {t}: rank/dense mismatches outside the guard band: {bad[:5]}"
            guard += gd
            worst["S_c"] = max(worst["S_c"], ws)
            worst["sigma"] = max(worst["sigma"], wsig)
            for j in sel:
                worst["proj"] = max(worst["proj"], active_projector_err(comp[j], P2.get_state(j), w.r, fp16=fp16))
    return worst, guard


def _assert_fp16_factors(states, diag=False):
    """Stored factors are fp16 values.  With per-channel decay the exported u is the stored u times
    the decays accumulated since the last compaction, so it is checked only when the pad is empty."""
    for st in states:
        if not st["dense"]:
            for key in (("V",) if diag and len(st["c"]) else ("U", "V")):
                x = st[key]
                assert np.array_equal(x.astype(np.float16).astype(np.float32), x), key


def _assert_worst(worst):
    for k, v in worst.items():
        assert v <= TOL, f"{k}: {v:.3e} > {TOL}  (all: {worst})"


@pytest.mark.parametrize("promote", [True, False])
def test_tiny_lockstep(promote):
    """64 states 16x32, empty start, compaction every 8 steps; with promotion the
    states move to the dense region, without it the frozen part keeps growing."""
    w = W.get("tiny")
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, promote_on_compact=promote, max_frozen=200)
    worst, guard = _lockstep(w, init, pool, np.arange(w.n_states), 40, promote=promote, check_readout=True)
    st = ss.pool_stats(pool)
    pool.close()
    print("tiny", promote, worst, "guard", guard, "dense", st["n_dense"], "max_rank", st["max_rank"])
    _assert_worst(worst)
    if promote:
        assert st["n_dense"] > 0
    else:
        assert st["n_dense"] == 0 and st["max_rank"] > 10


def test_mamba2_lockstep_one_request():
    """2,016 Mamba-2 states (one request of the 258k workload), 4 stagger groups, ragged sample."""
    w = W.get("mamba2_258k", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 17), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24, check_readout=True)
    pool.close()
    print("mamba2", worst, "guard", guard)
    _assert_worst(worst)


def test_gdn_delta_lockstep_one_request():
    """1,536 delta-rule states 128x128 (one request), random initial ranks 2..16."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 13), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24)
    pool.close()
    print("gdn", worst, "guard", guard)
    _assert_worst(worst)


def test_mixed_dense_lockstep():
    """Mixed scalar/delta states with ranks 2..64 + frozen extras; above 49 the state starts dense."""
    w = W.get("mixed_dense", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init)
    st0 = ss.pool_stats(pool)
    ranks = np.diff(init["comp_off"])
    assert st0["n_dense"] == int(np.sum(ranks > 49))
    ids = np.arange(w.n_states)
    worst, guard = _lockstep(w, init, pool, ids, 16, check_readout=True)
    pool.close()
    print("mixed", worst, "guard", guard)
    _assert_worst(worst)


def test_dense_baseline_matches_dense_recurrence():
    """force_dense pool (the dense HIP baseline) against the oracle's dense recurrence."""
    w = W.get("mamba2_258k", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, force_dense=True)
    ids = np.arange(0, w.n_states, 31)
    worst, _ = _lockstep(w, init, pool, ids, 6)
    st = ss.pool_stats(pool)
    pool.close()
    assert st["n_dense"] == w.n_states
    _assert_worst(worst)


def test_decode_bytes_accounting():
    """In-kernel algorithmic byte counter equals the host formula over the live ranks and pad fills,
    across the steps where dense states fold their pad into H and the compactions between them."""
    w = W.get("mixed_dense", n_requests=1)
    init = W.initial_state(w)
    for force_dense in (False, True):
        pool = _pool_from_init(w, init, force_dense=force_dense)
        gen = W.StepInputs(w, device="cuda")
        o = torch.empty(w.n_states, w.d_v, device="cuda")
        folds = 0
        for t in range(1, 2 * w.K + 2):
            states = ss.state_export(pool, np.arange(w.n_states))
            expect = 0
            for s in states:
                if not s["dense"]:
                    kind, nc, npad = ss.DECODE_FACTORED, len(s["sigma"]), len(s["c"])
                elif force_dense:
                    kind, nc, npad = ss.DECODE_DENSE_PLAIN, 0, 0
                else:
                    kind, nc, npad = ss.DECODE_DENSE_BUFFERED, 0, s["dense_pad"]
                    folds += npad + 1 == w.K
                expect += ss.decode_bytes_per_state(w.d_k, w.d_v, w.K, nc, npad, s["rule"], kind)
            b0 = ss.pool_stats(pool)["decode_bytes"]
            x = gen.generate(t)
            ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
            b1 = ss.pool_stats(pool)["decode_bytes"]
            assert b1 - b0 == expect, (force_dense, t)
            for g in ss.schedule_due(pool, t):
                ss.compact(pool, g)
        pool.close()
        if not force_dense:
            assert folds > 0


@pytest.mark.parametrize("fp16", [False, True])
def test_edge_shapes_and_ragged(fp16):
    """d = 4 (one lane per vector), 37 states (ragged workgroups), K = 1 (compaction every
    step), r = 1, empty states, delta rule, against the oracle in lock-step.  With fp16 factors
    the shapes cover both decode kernels: eight elements per lane (d_k, d_v multiples of 8) and
    four (the rest)."""
    rng = np.random.default_rng(5)
    for (dk, dv, K, r, N) in [(4, 8, 1, 1, 37), (12, 20, 3, 2, 37), (64, 44, 8, 8, 9), (8, 256, 2, 3, 37),
                              (256, 16, 8, 8, 13)]:
        R = rng.integers(0, 6, N)
        R[0] = 0
        off = np.concatenate([[0], np.cumsum(R)]).astype(np.int64)
        T = int(off[-1])
        u = rng.standard_normal((T, dk)).astype(np.float32)
        v = rng.standard_normal((T, dv)).astype(np.float32)
        sig = np.concatenate([np.sort(rng.uniform(0.1, 2, x))[::-1] for x in R]).astype(np.float32)
        rule = (np.arange(N) % 2).astype(np.uint8)
        eps = np.full(N, 1e-3, np.float32)
        pool = ss.state_pool_create(N, dk, dv, K, r, rule=rule, eps=eps, comp_off=off, u=u, v=v, sigma=sig,
                                    group_offset=[0], promote_on_compact=False, max_frozen=64, factor_fp16=fp16)
        o = torch.empty(N, dv, device="cuda")
        ids = np.arange(N)
        worst = 0.0
        for t in range(1, 3 * K + 2):
            q = torch.randn(N, dk, device="cuda")
            k = torch.nn.functional.normalize(torch.randn(N, dk, device="cuda"), dim=1)
            vv = torch.randn(N, dv, device="cuda")
            a = 0.9 + 0.1 * torch.rand(N, device="cuda")
            b = torch.rand(N, device="cuda")
            before = ss.state_export(pool, ids)
            if fp16:
                _assert_fp16_factors(before)
            P = oracle_from_export(before, eps, dk, dv, K, r, promote=False, factor_fp16=fp16)
            ss.decode_step(pool, q, k, vv, a, b, o)
            if ss.schedule_due(pool, t):
                ss.compact(pool, 0)
            torch.cuda.synchronize()
            oo = P.decode(q.cpu().numpy(), k.cpu().numpy(), vv.cpu().numpy(), a.cpu().numpy(), b.cpu().numpy())
            Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(N)])
            e = rel_out_err(o.cpu().numpy(), oo, Sn, np.linalg.norm(q.cpu().numpy(), axis=1))
            worst = max(worst, float(e.max()))
            if ss.schedule_due(pool, t):
                P.compact()
                ws, wsig, gd, bad = compare_compacted(ss.state_export(pool, ids), P, eps, fp16=fp16)
                assert not bad and ws <= TOL and wsig <= TOL, (dk, dv, K, r, ws, wsig, bad)
        pool.close()
        assert worst <= TOL, (dk, dv, K, r, worst)


def test_pad_overflow_poisons_pool():
    """A skipped compaction is caught by the kernel's own check and reported on a later call."""
    w = W.get("tiny")
    init = W.initial_state(w)
    pool = _pool_from_init(w, init)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for t in range(1, w.K + 1):
        x = gen.generate(t)
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
    x = gen.generate(w.K + 1)
    ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)  # pad full: flagged, state untouched
    torch.cuda.synchronize()
    with pytest.raises(ss.SinkStateError) as ei:
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
    assert ei.value.status == ss.SS_ERR_STATE
    pool.close()


def test_dense_capacity_exhaustion_is_reported():
    w = W.get("tiny")
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, dense_capacity=2)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    with pytest.raises(ss.SinkStateError) as ei:
        for t in range(1, 65):
            x = gen.generate(t)
            ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
            for g in ss.schedule_due(pool, t):
                ss.compact(pool, g)
            torch.cuda.synchronize()
    assert ei.value.status == ss.SS_ERR_CAPACITY
    pool.close()


@pytest.mark.parametrize("buffered", [False, True])
@pytest.mark.parametrize("dk,dv", [(4, 8), (12, 20), (44, 64), (128, 80), (80, 128), (256, 256), (256, 4)])
def test_dense_path_shapes(dk, dv, buffered):
    """Dense region (stored transposed) on edge shapes: one lane per row (d_k = 4), lane groups with
    idle lanes (12, 44), a full wavefront per row (256), both rules, ragged state count, readout and
    decode against the oracle's dense recurrence.  Plain: a force_dense pool (the dense baseline).
    Buffered: states start dense (rank L + 1) in a factored pool with K = 3; the steps cross full
    pads (folded inside decode) and an explicit compaction folds a partial pad."""
    rng = np.random.default_rng(dk * 1000 + dv)
    N, K = 37, 3
    L = ss.dense_rank_limit(dk, dv)
    R = np.full(N, L + 1 if buffered else 3)
    off = np.concatenate([[0], np.cumsum(R)]).astype(np.int64)
    u = rng.standard_normal((int(off[-1]), dk)).astype(np.float32)
    v = rng.standard_normal((int(off[-1]), dv)).astype(np.float32)
    sig = np.concatenate([np.geomspace(2.0, 0.5, r) for r in R]).astype(np.float32)
    rule = (np.arange(N) % 2).astype(np.uint8)
    eps = np.full(N, 1e-3, np.float32)
    pool = ss.state_pool_create(N, dk, dv, K, 2, rule=rule, eps=eps, comp_off=off, u=u, v=v, sigma=sig,
                                force_dense=not buffered)
    ids = np.arange(N)
    o = torch.empty(N, dv, device="cuda")
    worst, folds = 0.0, 0
    for t in range(1, 9):
        q = torch.randn(N, dk, device="cuda")
        k = torch.nn.functional.normalize(torch.randn(N, dk, device="cuda"), dim=1)
        vv = torch.randn(N, dv, device="cuda")
        a = 0.9 + 0.1 * torch.rand(N, device="cuda")
        b = torch.rand(N, device="cuda")
        before = ss.state_export(pool, ids)
        assert all(st["dense"] for st in before)
        folds += sum(st["dense_pad"] + 1 == K for st in before)
        P = oracle_from_export(before, eps, dk, dv, K, 2)
        Sn = np.array([np.linalg.norm(reconstruct(st)) for st in before])
        qn = np.linalg.norm(q.cpu().numpy(), axis=1)
        ss.readout(pool, q, o)
        torch.cuda.synchronize()
        worst = max(worst, float(rel_out_err(o.cpu().numpy(), P.readout(q.cpu().numpy()), Sn, qn).max()))
        ss.decode_step(pool, q, k, vv, a, b, o)
        torch.cuda.synchronize()
        oo = P.decode(q.cpu().numpy(), k.cpu().numpy(), vv.cpu().numpy(), a.cpu().numpy(), b.cpu().numpy())
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(N)])
        worst = max(worst, float(rel_out_err(o.cpu().numpy(), oo, Sn, qn).max()))
        if t == 4:
            mid = ss.state_export(pool, ids)
            assert buffered == any(st["dense_pad"] > 0 for st in mid)
            ss.compact(pool, 0)  # folds the partial pads of the dense states
            assert all(st["dense_pad"] == 0 for st in ss.state_export(pool, ids))
        for j, st in enumerate(ss.state_export(pool, ids)):
            So = P.reconstruct(j)
            worst = max(worst, float(np.linalg.norm(reconstruct(st) - So) / np.linalg.norm(So)))
    pool.close()
    assert worst <= TOL, (dk, dv, buffered, worst)
    assert folds > 0 or not buffered


@pytest.mark.parametrize("name,promote,order", [("tiny", False, "schedule"), ("mamba2_258k", True, "schedule"),
                                                ("gdn_delta", True, "random")])
def test_ring_growth_wrap_and_repack(name, promote, order):
    """Component rings created at exactly the initial size (arena_components=1): the first
    compaction must grow them, later ones wrap around the ring end (once the ranks settle), and
    with groups compacted in random order (out of their schedule) the segments leave gaps that
    force defragmenting re-packs.  Sampled states are checked in lock-step against the oracle."""
    w = W.get(name, n_requests=1 if name != "tiny" else None)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, promote_on_compact=promote, max_frozen=0 if promote else 200, arena_components=1)
    st0 = ss.pool_stats(pool)
    ranks = np.diff(init["comp_off"])
    fact = ranks <= ss.dense_rank_limit(w.d_k, w.d_v)
    assert st0["ring_capacity"][0] == max(1, int(np.minimum(ranks[fact], w.r).sum()))
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, max(1, w.n_states // 96)), [w.n_states - 1]]))
    if order == "schedule":
        worst, guard = _lockstep(w, init, pool, ids, 40 if name == "tiny" else 24, promote=promote)
    else:
        rng = np.random.default_rng(5)
        gen = W.StepInputs(w, device="cuda")
        eps = init["eps"][ids]
        o = torch.empty(w.n_states, w.d_v, device="cuda")
        worst = {"o": 0.0, "S_c": 0.0, "sigma": 0.0}
        grp = init["group_of_state"][ids]
        for t in range(1, 25):
            x = gen.generate(t)
            before = ss.state_export(pool, ids)
            P = oracle_from_export(before, eps, w.d_k, w.d_v, w.K, w.r)
            sub = {k: v.cpu().numpy()[ids].astype(np.float64) for k, v in x.items()}
            ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
            torch.cuda.synchronize()
            oo = P.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
            Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(len(ids))])
            e = rel_out_err(o.cpu().numpy()[ids], oo, Sn, np.linalg.norm(sub["q"], axis=1))
            worst["o"] = max(worst["o"], float(e.max()))
            # a random group each step (pads never overflow: every group is compacted at least
            # once in K steps below), plus the scheduled ones
            due = sorted(set(ss.schedule_due(pool, t)) | {int(rng.integers(len(init["group_offset"])))})
            after = ss.state_export(pool, ids)
            for g in due:
                ss.compact(pool, g)
            P2 = oracle_from_export(after, eps, w.d_k, w.d_v, w.K, w.r)
            sel = np.nonzero(np.isin(grp, due))[0]
            P2.compact(sel)
            ws, wsig, gd, bad = compare_compacted(ss.state_export(pool, ids), P2, eps)
            assert not bad, f"step {t}: rank/dense mismatches outside the guard band: {bad[:5]}"
            worst["S_c"] = max(worst["S_c"], ws)
            worst["sigma"] = max(worst["sigma"], wsig)
    st = ss.pool_stats(pool)
    pool.close()
    print(name, order, worst, {k: st[k] for k in ("ring_capacity", "ring_used", "ring_head", "ring_repacks",
                                                  "ring_syncs", "n_dense")})
    _assert_worst(worst)
    assert st["ring_repacks"] >= 1
    if name == "tiny":  # ranks settle here, so the rings stop growing and the heads pass the ring end
        assert max(h - c for h, c in zip(st["ring_head"], st["ring_capacity"])) > 0, "no ring wrapped"
    for R in range(2):
        assert st["ring_used"][R] <= st["ring_capacity"][R]


# ---------------------------------------------------------------------------------------------
# fp16 factor storage (SEED 6 "Lower precision composes"): factors rounded when written, pad fp32
# ---------------------------------------------------------------------------------------------

def test_fp16_create_rounds_initial_factors_exactly():
    """The stored initial factors are the round-to-nearest-even fp16 values of the given ones
    (bit-exact against numpy's float16 conversion); sigma and the layout are unchanged, and the
    factor part of the live bytes halves."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    p16 = _pool_from_init(w, init, factor_fp16=True)
    p32 = _pool_from_init(w, init)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 37), [w.n_states - 1]]))
    off = init["comp_off"]
    for s, a, b in zip(ids, ss.state_export(p16, ids), ss.state_export(p32, ids)):
        U0 = init["u"][off[s]:off[s + 1]]
        V0 = init["v"][off[s]:off[s + 1]]
        assert np.array_equal(a["U"], U0.astype(np.float16).astype(np.float32))
        assert np.array_equal(a["V"], V0.astype(np.float16).astype(np.float32))
        assert np.array_equal(a["sigma"], b["sigma"]) and a["n_active"] == b["n_active"]
    s16, s32 = ss.pool_stats(p16), ss.pool_stats(p32)
    ncomp = s32["active_components"] + s32["frozen_components"]
    assert s32["live_bytes"] - s16["live_bytes"] == ncomp * 2 * (w.d_k + w.d_v)
    p16.close()
    p32.close()


@pytest.mark.parametrize("promote", [True, False])
def test_fp16_tiny_lockstep(promote):
    w = W.get("tiny")
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, promote_on_compact=promote, max_frozen=200, factor_fp16=True)
    worst, guard = _lockstep(w, init, pool, np.arange(w.n_states), 40, promote=promote, check_readout=True,
                             fp16=True)
    pool.close()
    print("fp16 tiny", promote, worst, "guard", guard)
    _assert_worst(worst)


def test_fp16_mamba2_lockstep_one_request():
    w = W.get("mamba2_258k", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, factor_fp16=True)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 17), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24, check_readout=True, fp16=True)
    pool.close()
    print("fp16 mamba2", worst, "guard", guard)
    _assert_worst(worst)


def test_fp16_gdn_delta_lockstep_one_request():
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, factor_fp16=True)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 13), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 24, fp16=True)
    pool.close()
    print("fp16 gdn", worst, "guard", guard)
    _assert_worst(worst)


def test_fp16_mixed_dense_lockstep():
    """Mixed rules, ranks 2..64 (dense above 49), promotion of fp16-stored factors into the dense region."""
    w = W.get("mixed_dense", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, factor_fp16=True)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 11), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 16, fp16=True)
    pool.close()
    print("fp16 mixed", worst, "guard", guard)
    _assert_worst(worst)


@pytest.mark.parametrize("name", ["tiny", "gdn_delta"])
def test_fp16_ring_growth_and_repack(name):
    """fp16 rings created at the initial size: growth re-packs copy fp16 components unchanged."""
    w = W.get(name, n_requests=1 if name != "tiny" else None)
    init = W.initial_state(w)
    promote = name != "tiny"
    pool = _pool_from_init(w, init, promote_on_compact=promote, max_frozen=0 if promote else 200,
                           arena_components=1, factor_fp16=True)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, max(1, w.n_states // 96)), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 40 if name == "tiny" else 24, promote=promote, fp16=True)
    st = ss.pool_stats(pool)
    pool.close()
    print("fp16 ring", name, worst, "guard", guard, st["ring_repacks"])
    _assert_worst(worst)
    assert st["ring_repacks"] >= 1


def test_fp16_decode_bytes_accounting():
    """The in-kernel byte counter of an fp16 pool follows the FACTORED_FP16 formula."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init, factor_fp16=True)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for t in range(1, w.K + 3):
        expect = 0
        for s in ss.state_export(pool, np.arange(w.n_states)):
            if s["dense"]:
                kind, nc, npad = ss.DECODE_DENSE_BUFFERED, 0, s["dense_pad"]
            else:
                kind, nc, npad = ss.DECODE_FACTORED_FP16, len(s["sigma"]), len(s["c"])
            expect += ss.decode_bytes_per_state(w.d_k, w.d_v, w.K, nc, npad, s["rule"], kind)
        b0 = ss.pool_stats(pool)["decode_bytes"]
        x = gen.generate(t)
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        assert ss.pool_stats(pool)["decode_bytes"] - b0 == expect, t
        for g in ss.schedule_due(pool, t):
            ss.compact(pool, g)
    pool.close()


@pytest.mark.parametrize("name", ["gdn_delta", "mixed_dense"])
def test_compact_ids_lockstep(name):
    """ss_compact_ids on a ragged subset across groups (dense states included for mixed_dense), with
    pads partly filled: the listed states match the oracle's compaction of the same states; every
    other state is exported bit for bit as before; decoding and the schedule then continue in
    lock-step with the oracle."""
    w = W.get(name, n_requests=1)
    init = W.initial_state(w)
    pool = _pool_from_init(w, init)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for t in range(1, 12):
        x = gen.generate(t)
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        for g in ss.schedule_due(pool, t):
            ss.compact(pool, g)
    rng = np.random.default_rng(3)
    sel = np.unique(rng.choice(w.n_states, size=w.n_states // 7, replace=False))
    ids = np.arange(w.n_states)
    before = ss.state_export(pool, ids)
    ss.compact_ids(pool, sel)
    torch.cuda.synchronize()
    after = ss.state_export(pool, ids)
    mask = np.zeros(w.n_states, bool)
    mask[sel] = True
    for j in np.nonzero(~mask)[0]:
        b, a = before[j], after[j]
        assert b["dense"] == a["dense"]
        for key in (("S",) if b["dense"] else ("U", "V", "sigma", "c", "K", "W")):
            assert np.array_equal(a[key], b[key]), (j, key)
    eps = init["eps"][sel]
    P = oracle_from_export([before[j] for j in sel], eps, w.d_k, w.d_v, w.K, w.r)
    P.compact()
    ws, wsig, gd, bad = compare_compacted([after[j] for j in sel], P, eps)
    assert not bad and ws <= TOL and wsig <= TOL, (ws, wsig, bad[:5])
    assert any(len(before[j].get("c", [])) for j in sel if not before[j]["dense"])  # pads were non-empty
    worst, guard = _lockstep(w, init, pool, np.unique(np.concatenate([sel[::5], [0]])), 10, t0=11)
    pool.close()
    print(name, "compact_ids", ws, wsig, "then", worst)
    _assert_worst(worst)

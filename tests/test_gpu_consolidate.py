"""GPU parity of the frozen-part consolidation (SinkState 4.3, Figure 7(a)) against the oracle.

Each test runs decode steps and compactions on the GPU until frozen parts have
built up, exports the states, loads them into the oracle, consolidates on both
sides and compares: active parts and pads unchanged bit for bit, states and
singular values within the parity tolerance, ranks equal outside the guard
band, and the new frozen factors orthonormal.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare_compacted, oracle_from_export, reconstruct

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


def _pool(w, init, **kw):
    return ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"], **kw)


def _run(w, pool, t0, t1):
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for t in range(t0, t1 + 1):
        x = gen.generate(t)
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        for g in ss.schedule_due(pool, t):
            ss.compact(pool, g)
    torch.cuda.synchronize()


def _host_consolidate_all(pool, G, threads=0):
    """Every group through the host-core pipeline, one at a time, each result installed."""
    for g in range(G):
        assert ss.consolidate_host(pool, g, threads=threads) == g
        assert ss.consolidate_poll(pool, wait=True) == ss.CONS_INSTALLED


def _consolidate_and_compare(w, init, pool, ids, group=-1, fp16=False, host=False):
    eps = init["eps"][ids]
    before = ss.state_export(pool, ids)
    P = oracle_from_export(before, eps, w.d_k, w.d_v, w.K, w.r, factor_fp16=fp16)
    # fp16 factors: each stored element is within 2^-11 (relative) of its exact value, so the
    # Gram matrix of unit vectors deviates from I by at most about 2 * 2^-11
    otol = 1.0e-3 + 1e-5 if fp16 else 1e-4
    st0 = ss.pool_stats(pool)
    if host:
        G = len(init["group_offset"])
        if group < 0:
            _host_consolidate_all(pool, G)
        else:
            assert ss.consolidate_host(pool, group) == group
            assert ss.consolidate_poll(pool, wait=True) == ss.CONS_INSTALLED
    else:
        ss.consolidate(pool, group)
    torch.cuda.synchronize()
    after = ss.state_export(pool, ids)
    sel = np.arange(len(ids)) if group < 0 else np.nonzero(init["group_of_state"][ids] == group)[0]
    P.consolidate(sel)
    in_sel = np.zeros(len(ids), bool)
    in_sel[sel] = True
    for b, a, mine in zip(before, after, in_sel):
        assert a["dense"] == b["dense"]
        if b["dense"]:
            assert np.array_equal(a["S"], b["S"])
            continue
        ra = b["n_active"]
        assert a["n_active"] == ra
        for key in ("U", "V", "sigma"):
            assert np.array_equal(a[key][:ra], b[key][:ra]), key
        for key in ("c", "K", "W"):
            assert np.array_equal(a[key], b[key]), key
        rf = len(a["sigma"]) - ra
        assert rf <= len(b["sigma"]) - ra
        if rf and mine:  # states of other groups keep their frozen parts as they were
            Uf = a["U"][ra:].astype(np.float64)
            Vf = a["V"][ra:].astype(np.float64)
            assert np.abs(Uf @ Uf.T - np.eye(rf)).max() <= otol
            assert np.abs(Vf @ Vf.T - np.eye(rf)).max() <= otol
            if fp16:
                for x in (a["U"], a["V"]):
                    assert np.array_equal(x.astype(np.float16).astype(np.float32), x)
            assert np.all(np.diff(a["sigma"][ra:]) <= 0)
    ws, wsig, guard, bad = compare_compacted(after, P, eps, fp16=fp16)
    assert not bad, bad[:5]
    assert ws <= TOL and wsig <= TOL, (ws, wsig)
    st1 = ss.pool_stats(pool)
    removed = st1["consolidate_removed"] - st0["consolidate_removed"]
    assert st0["frozen_components"] - st1["frozen_components"] == removed
    return removed, guard


def test_consolidate_tiny():
    w = W.get("tiny")
    init = W.initial_state(w)
    pool = _pool(w, init)
    _run(w, pool, 1, 64)
    removed, _ = _consolidate_and_compare(w, init, pool, np.arange(w.n_states))
    print("tiny removed", removed)
    pool.close()


@pytest.mark.parametrize("name,steps", [("gdn_delta", 48), ("mamba2_258k", 48)])
def test_consolidate_one_request(name, steps):
    w = W.get(name, n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    _run(w, pool, 1, steps)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 7), [w.n_states - 1]]))
    removed, guard = _consolidate_and_compare(w, init, pool, ids)
    st = ss.pool_stats(pool)
    print(name, "removed", st["consolidate_removed"], "states", st["consolidate_states"], "guard", guard)
    if name == "gdn_delta":
        assert st["consolidate_removed"] > 0
    pool.close()


def test_consolidate_mixed_initial_tails_and_dense_states():
    """Initial frozen tails and dense states (mixed workload), one group at a time."""
    w = W.get("mixed_dense", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    ids = np.arange(w.n_states)
    for g in range(len(init["group_offset"])):
        _consolidate_and_compare(w, init, pool, ids, group=g)
    _run(w, pool, 1, 16)
    _consolidate_and_compare(w, init, pool, ids)
    pool.close()


def test_decode_and_compaction_continue_after_consolidation():
    """Lock-step decode and compaction after a consolidation (frozen lists may now start above
    the last active value)."""
    from test_gpu_parity import _assert_worst, _lockstep
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    _run(w, pool, 1, 40)
    ss.consolidate(pool)
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, 11), [w.n_states - 1]]))
    worst, guard = _lockstep(w, init, pool, ids, 16)
    print("after consolidation", worst, "guard", guard)
    _assert_worst(worst)
    pool.close()


def test_consolidate_twice_changes_nothing():
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    _run(w, pool, 1, 32)
    ss.consolidate(pool)
    ids = np.arange(0, w.n_states, 5)
    a = ss.state_export(pool, ids)
    st0 = ss.pool_stats(pool)
    ss.consolidate(pool)
    b = ss.state_export(pool, ids)
    st1 = ss.pool_stats(pool)
    assert st1["consolidate_removed"] == st0["consolidate_removed"]
    for x, y in zip(a, b):
        if x["dense"]:
            continue
        assert len(x["sigma"]) == len(y["sigma"])
        Sx, Sy = reconstruct(x), reconstruct(y)
        assert np.linalg.norm(Sx - Sy) <= 1e-5 * np.linalg.norm(Sx)
    pool.close()


def test_consolidate_next_queue_order():
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    G = len(init["group_offset"])
    assert G >= 3
    assert ss.consolidate_next(pool, 4) == []
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    x = gen.generate(1)
    ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
    ss.compact(pool, 2)
    ss.compact(pool, 0)
    assert ss.consolidate_next(pool, 1) == [0]       # never consolidated: lowest id first
    assert ss.consolidate_next(pool, 5) == [2]
    assert ss.consolidate_next(pool, 5) == []
    x = gen.generate(2)
    ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
    ss.compact(pool, 2)
    ss.compact(pool, 0)
    ss.compact(pool, 1)
    assert ss.consolidate_next(pool, 2) == [1, 0]    # 1 never; then 0 (consolidated before 2)
    assert ss.consolidate_next(pool, 2) == [2]
    torch.cuda.synchronize()
    st = ss.pool_stats(pool)
    assert st["consolidate_calls"] == 5
    pool.close()


def test_consolidate_rejects_frozen_parts_beyond_lds():
    """Without promotion a 256x256 pool allows 255 frozen components: more than the kernel's LDS."""
    pool = ss.state_pool_create(4, 256, 256, 8, 8, promote_on_compact=False, max_frozen=255)
    with pytest.raises(RuntimeError):
        ss.consolidate(pool)
    pool.close()
    pool = ss.state_pool_create(4, 256, 256, 8, 8, promote_on_compact=False, max_frozen=64)
    ss.consolidate(pool)
    pool.close()


@pytest.mark.parametrize("name", ["tiny", "gdn_delta"])
def test_consolidate_fp16_factors(name):
    """fp16 factor storage: the consolidated frozen factors are rounded to fp16 on both sides; Q is
    kept in fp32 while the kernel runs, so only the final factors carry the rounding."""
    w = W.get(name, n_requests=1 if name != "tiny" else None)
    init = W.initial_state(w)
    pool = _pool(w, init, factor_fp16=True)
    _run(w, pool, 1, 48 if name != "tiny" else 64)
    ids = np.arange(w.n_states) if name == "tiny" else \
        np.unique(np.concatenate([np.arange(0, w.n_states, 7), [w.n_states - 1]]))
    removed, guard = _consolidate_and_compare(w, init, pool, ids, fp16=True)
    print("fp16", name, "removed", removed, "guard", guard)
    pool.close()


# ---------------------------------------------------------------------------------------------
# asynchronous consolidation on a second stream (SinkState 4.3): staged, installed, or dropped
# ---------------------------------------------------------------------------------------------
def _run_steps(w, pool, t0, t1, o, gen):
    for t in range(t0, t1 + 1):
        x = gen.generate(t)
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        for g in ss.schedule_due(pool, t):
            ss.compact(pool, g)


def _not_due(pool, t0, t1, G):
    due = set()
    for t in range(t0, t1 + 1):
        due |= set(ss.schedule_due(pool, t))
    return [g for g in range(G) if g not in due]


@pytest.mark.parametrize("name,fp16", [("gdn_delta", False), ("gdn_delta", True), ("mamba2_258k", False)])
def test_consolidate_async_equals_sync(name, fp16):
    """Launch on a side stream, keep decoding on the pool's stream (the group is not compacted
    meanwhile), install: the group's frozen parts equal those of a twin pool consolidated
    synchronously at the launch point; every other part of the state stays the pool's own."""
    w = W.get(name, n_requests=1)
    init = W.initial_state(w)
    kw = {"factor_fp16": True} if fp16 else {}
    pa, pb = _pool(w, init, **kw), _pool(w, init, **kw)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for p in (pa, pb):
        _run_steps(w, p, 1, 40, o, gen)
    G = len(init["group_offset"])
    g = _not_due(pa, 41, 43, G)[0]
    side = torch.cuda.Stream()
    assert ss.consolidate_async(pa, side, group=g) == g
    with pytest.raises(RuntimeError):  # one in flight per pool
        ss.consolidate_async(pa, side, group=g)
    ss.consolidate(pb, g)
    for p in (pa, pb):
        _run_steps(w, p, 41, 43, o, gen)
    assert ss.consolidate_poll(pa, wait=True) == ss.CONS_INSTALLED
    assert ss.consolidate_poll(pa) == ss.CONS_IDLE
    torch.cuda.synchronize()
    ids = np.nonzero(init["group_of_state"] == g)[0]
    a, b = ss.state_export(pa, ids), ss.state_export(pb, ids)
    removed = 0
    for x, y in zip(a, b):
        assert x["dense"] == y["dense"]
        if x["dense"]:
            continue
        ra = x["n_active"]
        assert ra == y["n_active"] and len(x["sigma"]) == len(y["sigma"])
        for key in ("U", "V", "sigma"):
            assert np.array_equal(x[key][ra:], y[key][ra:]), key  # the same kernel arithmetic
            assert np.array_equal(x[key][:ra], y[key][:ra]), key
    sa, sb = ss.pool_stats(pa), ss.pool_stats(pb)
    assert sa["consolidate_removed"] == sb["consolidate_removed"]
    print(name, fp16, "group", g, "removed", sa["consolidate_removed"])
    pa.close()
    pb.close()


def test_consolidate_async_stale_is_dropped():
    """The group compacts before the poll: the result is dropped and the pool equals a twin that
    never consolidated."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pa, pb = _pool(w, init), _pool(w, init)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for p in (pa, pb):
        _run_steps(w, p, 1, 40, o, gen)
    due = ss.schedule_due(pa, 41)
    g = due[0]
    side = torch.cuda.Stream()
    assert ss.consolidate_async(pa, side, group=g) == g
    for p in (pa, pb):
        _run_steps(w, p, 41, 41, o, gen)  # compacts g
    assert ss.consolidate_poll(pa, wait=True) == ss.CONS_DISCARDED
    torch.cuda.synchronize()
    ids = np.arange(w.n_states)
    for x, y in zip(ss.state_export(pa, ids), ss.state_export(pb, ids)):
        assert x["dense"] == y["dense"]
        key = "S" if x["dense"] else "sigma"
        assert np.array_equal(x[key], y[key])
    pa.close()
    pb.close()


def test_consolidate_async_across_ring_repacks():
    """Rings created at the initial size: compactions of other groups re-pack them while the
    consolidation reads them (the re-pack waits for it); the install then lands at the moved
    positions, equal to a synchronous twin."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pa = _pool(w, init, arena_components=1)
    pb = _pool(w, init, arena_components=1)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for p in (pa, pb):
        _run_steps(w, p, 1, 12, o, gen)
    G = len(init["group_offset"])
    g = _not_due(pa, 13, 16, G)[0]
    side = torch.cuda.Stream()
    r0 = ss.pool_stats(pa)["ring_repacks"]
    assert ss.consolidate_async(pa, side, group=g) == g
    ss.consolidate(pb, g)
    for p in (pa, pb):
        _run_steps(w, p, 13, 16, o, gen)
    st = ss.consolidate_poll(pa, wait=True)
    r1 = ss.pool_stats(pa)["ring_repacks"]
    print("repacks during the consolidation", r1 - r0)
    assert st == ss.CONS_INSTALLED
    torch.cuda.synchronize()
    ids = np.nonzero(init["group_of_state"] == g)[0]
    for x, y in zip(ss.state_export(pa, ids), ss.state_export(pb, ids)):
        if not x["dense"]:
            for key in ("U", "V", "sigma"):
                assert np.array_equal(x[key], y[key]), key
    pa.close()
    pb.close()


def test_consolidate_async_queue_head_and_rejections():
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    side = torch.cuda.Stream()
    assert ss.consolidate_async(pool, side) == -1  # nothing compacted yet: no group waits
    assert ss.consolidate_poll(pool) == ss.CONS_IDLE
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    x = gen.generate(1)
    ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
    ss.compact(pool, 3)
    ss.compact(pool, 1)
    assert ss.consolidate_async(pool, side) == 1   # compacted most recently first
    assert ss.consolidate_poll(pool, wait=True) == ss.CONS_INSTALLED
    assert ss.consolidate_async(pool, side) == 3
    assert ss.consolidate_poll(pool, wait=True) == ss.CONS_INSTALLED
    assert ss.consolidate_async(pool, side) == -1
    pool.close()
    kda = W.get("kda_delta", n_requests=1)
    ki = W.initial_state(kda)
    kp = ss.state_pool_create(kda.n_states, kda.d_k, kda.d_v, kda.K, kda.r, group_of_state=ki["group_of_state"],
                              group_offset=ki["group_offset"], rule=ki["rule"], eps=ki["eps"], comp_off=ki["comp_off"],
                              u=ki["u"], v=ki["v"], sigma=ki["sigma"], diag_decay=True)
    with pytest.raises(RuntimeError):
        ss.consolidate_async(kp, side, group=0)
    kp.close()


# --------------------------------------------------------------------------------------------
# host-core pipeline (SinkState 4.3, Figure 7(b)): download, exact fp64 SVD on host threads,
# upload, install unless stale
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,steps,fp16", [("tiny", 64, False), ("gdn_delta", 48, False), ("gdn_delta", 48, True),
                                             ("mamba2_258k", 48, False)])
def test_consolidate_host_matches_oracle(name, steps, fp16):
    """Every group consolidated on host cores: states, values and ranks as the oracle's exact
    consolidation, active parts and pads untouched, new frozen factors orthonormal."""
    w = W.get(name, n_requests=None if name == "tiny" else 1)
    init = W.initial_state(w)
    pool = _pool(w, init, **({"factor_fp16": True} if fp16 else {}))
    _run(w, pool, 1, steps)
    ids = np.arange(w.n_states) if name == "tiny" else \
        np.unique(np.concatenate([np.arange(0, w.n_states, 7), [w.n_states - 1]]))
    removed, guard = _consolidate_and_compare(w, init, pool, ids, fp16=fp16, host=True)
    print(name, fp16, "removed", removed, "guard", guard)
    if name == "gdn_delta":
        assert removed > 0
    pool.close()


def test_consolidate_host_stale_is_dropped_and_retried_first():
    """The group compacts while its host result is being computed: the result is dropped, the pool
    equals a twin that never consolidated, and the next launch from the queue takes that group
    before a group that was never consolidated (dropped first, then least recently consolidated)."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pa, pb = _pool(w, init), _pool(w, init)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for p in (pa, pb):
        _run_steps(w, p, 1, 40, o, gen)
    g = ss.schedule_due(pa, 41)[0]
    assert ss.consolidate_host(pa, g) == g
    with pytest.raises(RuntimeError):  # one in flight per pool
        ss.consolidate_host(pa, g)
    for p in (pa, pb):
        _run_steps(w, p, 41, 41, o, gen)  # compacts g
    assert ss.consolidate_poll(pa, wait=True) == ss.CONS_DISCARDED
    torch.cuda.synchronize()
    ids = np.arange(w.n_states)
    for x, y in zip(ss.state_export(pa, ids), ss.state_export(pb, ids)):
        assert x["dense"] == y["dense"]
        key = "S" if x["dense"] else "sigma"
        assert np.array_equal(x[key], y[key])
    # every other group waits too and was never consolidated; g goes first all the same
    assert ss.consolidate_host(pa) == g
    assert ss.consolidate_poll(pa, wait=True) == ss.CONS_INSTALLED
    h = ss.consolidate_host(pa)
    assert h != g and h >= 0
    assert ss.consolidate_poll(pa, wait=True) == ss.CONS_INSTALLED
    pa.close()
    pb.close()


def test_consolidate_async_retries_dropped_group_first():
    """The GPU asynchronous form follows the same queue rule."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pool = _pool(w, init)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    _run_steps(w, pool, 1, 40, o, gen)
    g = ss.schedule_due(pool, 41)[0]
    side = torch.cuda.Stream()
    assert ss.consolidate_async(pool, side, group=g) == g
    _run_steps(w, pool, 41, 41, o, gen)
    assert ss.consolidate_poll(pool, wait=True) == ss.CONS_DISCARDED
    assert ss.consolidate_async(pool, side) == g
    assert ss.consolidate_poll(pool, wait=True) == ss.CONS_INSTALLED
    pool.close()


def test_consolidate_host_across_ring_repacks():
    """Rings created at the initial size: compactions of other groups re-pack them while the host
    computes (the re-pack waits only for the gather); the install then lands at the moved
    positions and agrees with a twin consolidated synchronously on the GPU, to the parity
    tolerance (the host works in fp64)."""
    w = W.get("gdn_delta", n_requests=1)
    init = W.initial_state(w)
    pa = _pool(w, init, arena_components=1)
    pb = _pool(w, init, arena_components=1)
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    for p in (pa, pb):
        _run_steps(w, p, 1, 12, o, gen)
    G = len(init["group_offset"])
    g = _not_due(pa, 13, 16, G)[0]
    r0 = ss.pool_stats(pa)["ring_repacks"]
    assert ss.consolidate_host(pa, g) == g
    ss.consolidate(pb, g)
    for p in (pa, pb):
        _run_steps(w, p, 13, 16, o, gen)
    st = ss.consolidate_poll(pa, wait=True)
    print("repacks during the consolidation", ss.pool_stats(pa)["ring_repacks"] - r0)
    assert st == ss.CONS_INSTALLED
    torch.cuda.synchronize()
    ids = np.nonzero(init["group_of_state"] == g)[0]
    for x, y in zip(ss.state_export(pa, ids), ss.state_export(pb, ids)):
        assert x["dense"] == y["dense"]
        if x["dense"]:
            continue
        ra = x["n_active"]
        assert ra == y["n_active"] and len(x["sigma"]) == len(y["sigma"])
        for key in ("U", "V", "sigma"):  # the active parts were never touched
            assert np.array_equal(x[key][:ra], y[key][:ra]), key
        # the frozen parts (the pads differ: delta-rule steps read the state before the install)
        fx = (x["U"][ra:].T.astype(np.float64) * x["sigma"][ra:]) @ x["V"][ra:].astype(np.float64)
        fy = (y["U"][ra:].T.astype(np.float64) * y["sigma"][ra:]) @ y["V"][ra:].astype(np.float64)
        full = (y["U"].T.astype(np.float64) * y["sigma"]) @ y["V"].astype(np.float64)
        assert np.linalg.norm(fx - fy) <= TOL * np.linalg.norm(full)
        if len(y["sigma"]) > ra:
            assert np.max(np.abs(x["sigma"][ra:] - y["sigma"][ra:]) / y["sigma"][ra:]) <= TOL
    pa.close()
    pb.close()

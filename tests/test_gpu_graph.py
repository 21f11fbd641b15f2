"""Whole steps replayed as HIP graphs (ss_step_graph_*), through the C-ABI.

Two pools start from the same state.  One runs eagerly (ss_decode_step, then ss_compact for the
groups due), the other replays the captured step graphs on fixed input buffers.  The kernels and
their inputs are the same, so every output and every exported state must be bit-identical after
every replay (ring and dense-slot placement may differ: they come from atomics).  Eager work and
synchronizations run between the replays, a re-pack forces a new capture, and the graph pool is
also checked against the fp64 oracle in lock-step.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare_compacted, states_of, oracle_from_export, reconstruct, rel_out_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


def _pool(w, init, **kw):
    return ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"], **kw)


def _same_states(a, b, t):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x["dense"] == y["dense"], f"step {t} state {x['id']}"
        keys = ("S",) if x["dense"] else ("sigma", "U", "V", "c", "K", "W")
        for key in keys:
            assert np.array_equal(x[key], y[key]), f"step {t} state {x['id']} field {key}"


def _twin_run(name, steps, requests=1, arena=0, eager_extra=False, oracle_steps=(), fp16=False):
    w = W.get(name, n_requests=requests if name != "tiny" else None)
    init = W.initial_state(w)
    diag = w.diag_decay
    A = _pool(w, init, arena_components=arena, factor_fp16=fp16, diag_decay=diag)
    B = _pool(w, init, arena_components=arena, factor_fp16=fp16, diag_decay=diag)
    N, dk, dv = w.n_states, w.d_k, w.d_v
    delta = bool(np.any(init["rule"] == 1))
    buf = {"q": torch.zeros(N, dk, device="cuda"), "k": torch.zeros(N, dk, device="cuda"),
           "v": torch.zeros(N, dv, device="cuda"),
           "alpha": torch.zeros((N, dk) if diag else (N,), device="cuda"),
           "beta": torch.zeros(N, device="cuda") if delta else None}
    oA = torch.empty(N, dv, device="cuda")
    oB = torch.empty(N, dv, device="cuda")
    graph = ss.StepGraph(B, buf["q"], buf["k"], buf["v"], buf["alpha"], buf["beta"], oB)
    gen = W.StepInputs(w, device="cuda")
    ids = np.unique(np.concatenate([np.arange(0, N, max(1, N // 64)), [N - 1]]))
    eps = init["eps"][ids]
    grp = init["group_of_state"][ids]
    worst = {"o": 0.0, "S_c": 0.0, "sigma": 0.0}
    for t in range(1, steps + 1):
        x = gen.generate(t)
        for key, b in buf.items():
            if b is not None:
                b.copy_(x[key])
        check = t in oracle_steps
        if check:
            before = ss.state_export(B, ids)
            P = oracle_from_export(before, eps, dk, dv, w.K, w.r, factor_fp16=fp16, diag_decay=diag)
            sub = {k: v.cpu().numpy()[ids].astype(np.float64) for k, v in x.items()}
        graph.launch(t)
        ss.decode_step(A, x["q"], x["k"], x["v"], x["alpha"], x["beta"] if delta else None, oA)
        due = ss.schedule_due(A, t)
        for g in due:
            ss.compact(A, g)
        torch.cuda.synchronize()
        assert torch.equal(oA, oB), f"{name} step {t}: outputs differ"
        if check:
            oo = P.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
            Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(len(ids))])
            e = rel_out_err(oB.cpu().numpy()[ids], oo, Sn, np.linalg.norm(sub["q"], axis=1))
            worst["o"] = max(worst["o"], float(e.max()))
            if due:
                pre = states_of(P, len(ids))
                P.compact(np.nonzero(np.isin(grp, due))[0])
                ws, wsig, gd, bad = compare_compacted(ss.state_export(B, ids), P, eps, fp16=fp16, before=pre)
                assert not bad, f"step {t}: rank/dense mismatches outside the guard band: {bad[:5]}"
                worst["S_c"] = max(worst["S_c"], ws)
                worst["sigma"] = max(worst["sigma"], wsig)
        if t % 4 == 0 or t == steps:
            _same_states(ss.state_export(A, ids), ss.state_export(B, ids), t)
        if eager_extra and t % 5 == 0:
            # eager work between replays: a read-only readout on both, and a compaction of a group
            # that is not due, on both pools
            g = (t // 5) % len(init["group_offset"])
            for pool, out in ((A, oA), (B, oB)):
                ss.readout(pool, x["q"], out)
                ss.compact(pool, g)
            torch.cuda.synchronize()
            assert torch.equal(oA, oB), f"{name} step {t}: readouts differ"
    sa, sb = ss.pool_stats(A), ss.pool_stats(B)
    graph.close()
    A.close()
    B.close()
    for key in ("n_dense", "active_components", "frozen_components", "pad_entries", "promotions", "decode_calls"):
        assert sa[key] == sb[key], (key, sa[key], sb[key])
    for k, v in worst.items():
        assert v <= TOL, f"{k}: {v:.3e} > {TOL} (all: {worst})"
    print(name, "repacks", sb["ring_repacks"], "dense", sb["n_dense"], worst)
    return sb


def test_graph_tiny_matches_eager_and_oracle():
    """64 states 16x32: the states go dense during the run (the captured dense grid must cover
    promotions), and the graph pool is checked against the oracle at every step."""
    st = _twin_run("tiny", 40, oracle_steps=set(range(1, 41)))
    assert st["n_dense"] > 0


def test_graph_mamba2_recapture_after_repack():
    """2,016 Mamba-2 states with rings created at their initial size: re-packs move the rings and
    the graphs are captured again before the next replay."""
    st = _twin_run("mamba2_258k", 24, arena=1, oracle_steps={1, 2, 8, 9})
    assert st["ring_repacks"] >= 1


def test_graph_gdn_delta_with_eager_work_between_replays():
    """1,536 delta-rule states 128x128, with eager readouts and out-of-schedule compactions
    between the replays."""
    _twin_run("gdn_delta", 20, eager_extra=True, oracle_steps={3, 8})


def test_graph_kda_per_channel_decay():
    """640 Kimi-Delta-Attention states 128x128 with per-channel decay: the decay accumulated in the
    pads (gamma) and its reset at compaction are captured like every other kernel argument."""
    _twin_run("kda_delta", 20, eager_extra=True, oracle_steps={3, 8})


@pytest.mark.parametrize("name", ["gdn_delta", "kda_delta"])
def test_graph_fp16_factors(name):
    """Factors stored in binary16: the graph pool stays bit-identical to the eager one and within
    the fp16 rounding bound of the oracle."""
    _twin_run(name, 20, arena=1, oracle_steps={3, 8}, fp16=True)


def test_graph_on_dense_baseline_pool():
    """A force_dense pool has no compaction: its graphs hold the plain dense decode only and must
    match eager decode steps bit for bit."""
    w = W.get("tiny")
    init = W.initial_state(w)
    A = _pool(w, init, force_dense=True)
    B = _pool(w, init, force_dense=True)
    N, dk, dv = w.n_states, w.d_k, w.d_v
    buf = {"q": torch.zeros(N, dk, device="cuda"), "k": torch.zeros(N, dk, device="cuda"),
           "v": torch.zeros(N, dv, device="cuda"), "alpha": torch.zeros(N, device="cuda")}
    oA = torch.empty(N, dv, device="cuda")
    oB = torch.empty(N, dv, device="cuda")
    graph = ss.StepGraph(B, buf["q"], buf["k"], buf["v"], buf["alpha"], None, oB)
    gen = W.StepInputs(w, device="cuda")
    for t in range(1, 13):
        x = gen.generate(t)
        for key, b in buf.items():
            b.copy_(x[key])
        graph.launch(t)
        ss.decode_step(A, x["q"], x["k"], x["v"], x["alpha"], None, oA)
        torch.cuda.synchronize()
        assert torch.equal(oA, oB), t
    _same_states(ss.state_export(A, np.arange(N)), ss.state_export(B, np.arange(N)), 12)
    graph.close()
    A.close()
    B.close()

"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

Every state of the pool is decoded and compacted on the GPU; a stratified sample of states (every
compaction group, both rules, the first and last states, ragged ids) is checked in lock-step
against the fp64 oracle with the tolerances of parity_util: before each call the sampled states
are exported and loaded into the oracle, both sides run the same call on bit-identical inputs,
and the outputs, the states after decode and the compacted states are compared.
"""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare_compacted, states_of, oracle_from_export, reconstruct, rel_out_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


def _sample(w, init, n, seed):
    rng = np.random.default_rng(seed)
    grp = init["group_of_state"]
    ids = [0, w.n_states - 1]
    for g in range(len(init["group_offset"])):
        members = np.nonzero(grp == g)[0]
        ids += list(rng.choice(members, size=min(len(members), max(1, n // len(init["group_offset"]))),
                               replace=False))
    return np.unique(np.array(ids, dtype=np.int64))


def _fullsize(name, steps, n_sample, requests=None, fp16=False):
    w = W.get(name, n_requests=requests)
    init = W.initial_state(w)
    pool = ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"],
                                diag_decay=w.diag_decay, factor_fp16=fp16)
    ids = _sample(w, init, n_sample, seed=w.seed_id)
    idx = torch.as_tensor(ids, device="cuda")
    eps = init["eps"][ids]
    grp = init["group_of_state"][ids]
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    worst = {"o": 0.0, "S": 0.0, "S_c": 0.0, "sigma": 0.0}
    guard = 0
    for t in range(1, steps + 1):
        x = gen.generate(t)
        before = ss.state_export(pool, ids)
        P = oracle_from_export(before, eps, w.d_k, w.d_v, w.K, w.r, factor_fp16=fp16, diag_decay=w.diag_decay)
        sub = {k: v[idx].cpu().numpy().astype(np.float64) for k, v in x.items()}
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        due = ss.schedule_due(pool, t)
        for g in due:
            ss.compact(pool, g)
        torch.cuda.synchronize()
        oo = P.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
        Sn = np.array([np.linalg.norm(P.reconstruct(j)) for j in range(len(ids))])
        e = rel_out_err(o[idx].cpu().numpy(), oo, Sn, np.linalg.norm(sub["q"], axis=1))
        worst["o"] = max(worst["o"], float(e.max()))
        after = ss.state_export(pool, ids)
        if due:
            sel = np.nonzero(np.isin(grp, due))[0]
            pre = states_of(P, len(ids))
            P.compact(sel)
            ws, wsig, gd, bad = compare_compacted(after, P, eps, fp16=fp16, before=pre)
            assert not bad, f"{name} step {t}: rank/dense mismatches outside the guard band: {bad[:5]}"
            guard += gd
            worst["S_c"] = max(worst["S_c"], ws)
            worst["sigma"] = max(worst["sigma"], wsig)
        else:
            for j, st in enumerate(after):
                So = P.reconstruct(j)
                worst["S"] = max(worst["S"], np.linalg.norm(reconstruct(st) - So) / max(np.linalg.norm(So), 1e-30))
    stats = ss.pool_stats(pool)
    pool.close()
    print(name, w.n_states, "states", len(ids), "sampled", worst, "guard", guard, "dense", stats["n_dense"])
    for k, v in worst.items():
        assert v <= TOL, f"{name} {k}: {v:.3e} > {TOL} (all: {worst})"
    return stats


def test_fullsize_mamba2_258k():
    """258,048 Mamba-2 states (128 requests x 21 layers x 96 heads), 12 steps: every stagger group
    compacts at least once (partial pads) and two groups twice."""
    _fullsize("mamba2_258k", steps=12, n_sample=256)


def test_fullsize_gdn_delta():
    """98,304 Gated-DeltaNet states 128x128 with 8 stagger groups, 10 steps."""
    _fullsize("gdn_delta", steps=10, n_sample=256)


def test_fullsize_mixed_dense():
    """32,768 mixed-rule states with a dense fallback at rank > 49, 10 steps."""
    st = _fullsize("mixed_dense", steps=10, n_sample=256)
    assert st["n_dense"] > 0


def test_fullsize_mamba2_1m():
    """1,032,192 Mamba-2 states (512 requests), 4 steps with the compaction of the first due group."""
    _fullsize("mamba2_1m", steps=4, n_sample=128)


def test_fullsize_kda_delta():
    """40,960 Kimi Delta Attention states 128x128 (per-channel decay), 10 steps."""
    _fullsize("kda_delta", steps=10, n_sample=256)


def test_fullsize_gdn_delta_fp16():
    """98,304 Gated-DeltaNet states with fp16 factors, 10 steps."""
    _fullsize("gdn_delta", steps=10, n_sample=256, fp16=True)

"""Free-running parity: the fp64 oracle runs its own trajectory from the same initial states on the
same (bit-identical) inputs as the GPU pool, with no re-loading between steps.

Checked every step: the outputs agree within 1e-4 (relative, as in parity_util), and after every
compaction the states agree within 1e-4 with equal ranks.  A keep/drop or active/frozen decision
that falls in the guard band (parity_util.GUARD) may go differently on the two sides; the oracle
state is then re-synchronized from the GPU export and the event is counted.  Both trajectories
also keep within the open-loop bound of SEED Prop. 3 against the dense recurrence: the oracle by
its own bound, the GPU by the same bound plus the 1e-4 parity tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import OraclePool
from oracle.oracle import OracleState
from parity_util import GUARD, TOL, reconstruct, rel_out_err, to_oracle_state

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


def _freerun(name, steps, stride, requests=None, need_promotions=False):
    w = W.get(name, n_requests=requests)
    L = ss.dense_rank_limit(w.d_k, w.d_v)
    init = W.initial_state(w)
    pool = ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"])
    ids = np.unique(np.concatenate([np.arange(0, w.n_states, stride), [w.n_states - 1]]))
    n = len(ids)
    off = init["comp_off"]
    Pf = OraclePool(n, w.d_k, w.d_v, w.K, w.r, -1, True)
    Pd = OraclePool(n, w.d_k, w.d_v, w.K, w.r, -1, False)  # the dense recurrence
    for j, s in enumerate(ids):
        U = init["u"][off[s]:off[s + 1]].astype(np.float64)
        V = init["v"][off[s]:off[s + 1]].astype(np.float64)
        sig = init["sigma"][off[s]:off[s + 1]].astype(np.float64)
        rule, eps = int(init["rule"][s]), float(init["eps"][s])
        Pf.set_state(j, OracleState(U, V, sig, rule=rule, eps=eps))
        Pd.set_state(j, OracleState(S=(U.T * sig) @ V if len(sig) else np.zeros((w.d_k, w.d_v)), rule=rule, eps=0.0),
                     as_init=False)
    grp = init["group_of_state"][ids]
    eps = init["eps"][ids]
    gen = W.StepInputs(w, device="cuda")
    o = torch.empty(w.n_states, w.d_v, device="cuda")
    idx = torch.as_tensor(ids, device="cuda")
    worst = {"o": 0.0, "S": 0.0, "bound_or": 0.0, "bound_gpu": 0.0}
    resync = 0
    resynced = set()  # states re-loaded after a guard-band decision: the oracle's bound no longer covers them
    for t in range(1, steps + 1):
        x = gen.generate(t)
        sub = {k: v[idx].cpu().numpy().astype(np.float64) for k, v in x.items()}
        ss.decode_step(pool, x["q"], x["k"], x["v"], x["alpha"], x["beta"], o)
        due = ss.schedule_due(pool, t)
        for g in due:
            ss.compact(pool, g)
        torch.cuda.synchronize()
        oo = Pf.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
        od = Pd.decode(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"])
        Sn = np.array([np.linalg.norm(Pd.reconstruct(j)) for j in range(n)])
        e = rel_out_err(o[idx].cpu().numpy(), oo, Sn, np.linalg.norm(sub["q"], axis=1))
        worst["o"] = max(worst["o"], float(e.max()))
        sel = np.nonzero(np.isin(grp, due))[0]
        if len(sel):
            Pf.compact(sel)
        gpu = ss.state_export(pool, ids)
        for j in range(n):
            Sg, So, Sd = reconstruct(gpu[j]), Pf.reconstruct(j), Pd.reconstruct(j)
            nd = max(np.linalg.norm(Sd), 1e-30)
            ost = Pf.get_state(j)
            if gpu[j]["dense"] != ost.dense:
                # one side promoted: accepted only when the factored side holds exactly L components
                # and the states differ by no more than one component at the threshold, i.e. the
                # other side kept an (L+1)-th component that fell in the guard band
                fac = ost if not ost.dense else None
                rk = len(fac.sigma) if fac is not None else len(gpu[j]["sigma"])
                smax = float(fac.sigma[0]) if fac is not None else float(np.max(gpu[j]["sigma"]))
                diff = np.linalg.norm(Sg - So)
                assert rk == L and diff <= (eps[j] + GUARD) * smax + TOL * np.linalg.norm(So), \
                    (name, t, j, rk, diff, smax)
                Pf.set_state(j, to_oracle_state(gpu[j], eps[j]), as_init=False)
                resync += 1
                resynced.add(j)
                continue
            ranks_differ = not ost.dense and len(gpu[j]["sigma"]) != len(ost.sigma)
            if ranks_differ:
                # accepted only for a guard-band decision: the components the two sides keep
                # differently lie within GUARD sigma_max of the threshold
                sg = np.sort(np.asarray(gpu[j].get("sigma", []), np.float64))[::-1]
                so = np.sort(np.asarray(ost.sigma if ost.sigma is not None else [], np.float64))[::-1]
                smax = max(sg[0] if len(sg) else 0.0, so[0] if len(so) else 0.0)
                longer = sg if len(sg) > len(so) else so
                extra = longer[min(len(sg), len(so)):]
                assert not gpu[j]["dense"] and not ost.dense and np.all(np.abs(extra - eps[j] * smax) <= GUARD * smax), \
                    (name, t, j, len(sg), len(so))
                Pf.set_state(j, to_oracle_state(gpu[j], eps[j]), as_init=False)
                resync += 1
                resynced.add(j)
                continue
            worst["S"] = max(worst["S"], np.linalg.norm(Sg - So) / max(np.linalg.norm(So), 1e-30))
            if j in resynced:
                continue
            b = Pf.bound(j)
            worst["bound_or"] = max(worst["bound_or"], (np.linalg.norm(So - Sd) - b) / nd)
            worst["bound_gpu"] = max(worst["bound_gpu"], (np.linalg.norm(Sg - Sd) - b) / nd)
    n_dense_or = sum(Pf.get_state(j).dense for j in range(n))
    n_dense_gpu = sum(st["dense"] for st in ss.state_export(pool, ids))
    promotions = ss.pool_stats(pool)["promotions"]
    pool.close()
    print(name, n, "states", steps, "steps", worst, "resyncs", resync, "dense in the sample: oracle", n_dense_or,
          "gpu", n_dense_gpu, "gpu promotions", promotions)
    if need_promotions:
        assert n_dense_or > 0 and n_dense_gpu > 0 and promotions > 0, (n_dense_or, n_dense_gpu, promotions)
    assert worst["o"] <= TOL and worst["S"] <= TOL, worst
    assert worst["bound_or"] <= 1e-12, worst
    assert worst["bound_gpu"] <= TOL, worst


def test_freerun_tiny():
    """All 64 states 16x32 from an empty start over the workload's whole 256 steps (32 compactions,
    promotions to dense), outputs checked every step."""
    _freerun("tiny", steps=256, stride=1, need_promotions=True)


def test_freerun_mamba2_one_request():
    """One request (2,016 states, every 41st sampled) over the workload's whole 1,024 steps: ranks
    cross L = 49 near step 44 and the whole sample is dense by step 64; the remaining steps run the
    dense region's buffered steps and pad folds."""
    _freerun("mamba2_258k", steps=1024, stride=41, requests=1, need_promotions=True)


def test_freerun_gdn_one_request():
    """One request (1,536 delta-rule states, every 31st sampled) over the workload's whole 512
    steps, past the sample's first promotions (near step 75)."""
    _freerun("gdn_delta", steps=512, stride=31, requests=1, need_promotions=True)


def test_freerun_mixed_one_request():
    """One request of the mixed pool (1,024 states, half scalar-decay, half delta-rule, some dense
    from the start, every 19th sampled) over the workload's whole 256 steps."""
    _freerun("mixed_dense", steps=256, stride=19, requests=1, need_promotions=True)

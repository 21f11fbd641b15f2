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


def _freerun(name, steps, stride, requests=None):
    w = W.get(name, n_requests=requests)
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
            ranks_differ = gpu[j]["dense"] != ost.dense or (
                not ost.dense and len(gpu[j]["sigma"]) != len(ost.sigma))
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
    pool.close()
    print(name, n, "states", steps, "steps", worst, "resyncs", resync)
    assert worst["o"] <= TOL and worst["S"] <= TOL, worst
    assert worst["bound_or"] <= 1e-12, worst
    assert worst["bound_gpu"] <= TOL, worst


def test_freerun_tiny():
    """All 64 states 16x32 from an empty start, 64 steps (8 compactions, promotions to dense)."""
    _freerun("tiny", steps=64, stride=1)


def test_freerun_mamba2_one_request():
    _freerun("mamba2_258k", steps=32, stride=41, requests=1)


def test_freerun_gdn_one_request():
    _freerun("gdn_delta", steps=32, stride=31, requests=1)

"""Helpers shared by the GPU parity tests: convert exported GPU states to oracle
states and compare results with the tolerances of the parity protocol.

Tolerances (fp32 GPU against the fp64 oracle):
  outputs o         ||o_gpu - o_or|| <= 1e-4 * max(||o_or||, ||S||_F ||q||)
  states            ||S_gpu - S_or||_F <= 1e-4 ||S_or||_F
  singular values   |sigma_gpu - sigma_or| <= 1e-4 sigma_or for every kept component
  subspaces         projectors of clusters split at relative gaps > 1e-2
  ranks             equal, except keep/drop decisions within 1e-5 sigma_max of
                    eps * sigma_max and active/frozen splits within 1e-5
                    sigma_max ("guard band"), which are counted and accepted

fp16 factor storage: each side rounds the factors it writes to binary16.  Where
singular values cluster, the two sides' exact results are different bases of
the same subspace, and their roundings differ.  Rounding moves an element by at
most 2^-11 of itself (normal range) or 2^-25 (subnormal range), so a stored unit
vector moves by at most delta = 2^-11 + sqrt(d) 2^-25 and a component
sigma u v^T by at most sigma (delta_u + delta_v + delta_u delta_v).  A compacted
state is therefore compared as ||S_gpu - S_or||_F <= 1e-4 ||S_or||_F + 2 rho,
rho = sum_i sigma_i (delta_u + delta_v + delta_u delta_v) over the oracle's
components (both sides round).  The projector of an active block of r rounded
unit vectors moves by at most 2 sqrt(r) delta + r delta^2 (Frobenius), so the
active projectors are compared within 1e-4 plus twice that.
"""
import numpy as np

from oracle import OraclePool
from oracle.oracle import OracleState

TOL = 1e-4
GUARD = 1e-5
U16 = 2.0 ** -11   # binary16 unit roundoff (round to nearest)
SUB16 = 2.0 ** -25  # binary16 half spacing of the subnormals


def fp16_rounding_bound(sigma, d_k, d_v):
    """rho: the Frobenius-norm bound on how far rounding unit factors to binary16 moves sum sigma_i u_i v_i^T."""
    du = U16 + np.sqrt(d_k) * SUB16
    dv = U16 + np.sqrt(d_v) * SUB16
    return float(np.sum(np.abs(sigma)) * (du + dv + du * dv))


def to_oracle_state(st, eps):
    if st["dense"]:
        return OracleState(S=st["S"].astype(np.float64), rule=st["rule"], eps=float(eps))
    return OracleState(st["U"].astype(np.float64), st["V"].astype(np.float64), st["sigma"].astype(np.float64),
                       st["K"].astype(np.float64), st["W"].astype(np.float64), st["c"].astype(np.float64),
                       rule=st["rule"], eps=float(eps))


def reconstruct(st):
    if st["dense"]:
        return st["S"].astype(np.float64)
    S = (st["U"].T.astype(np.float64) * st["sigma"].astype(np.float64)) @ st["V"].astype(np.float64)
    if len(st["c"]):
        S += (st["K"].T.astype(np.float64) * st["c"].astype(np.float64)) @ st["W"].astype(np.float64)
    return S


def oracle_from_export(states, eps, d_k, d_v, K, r, L=-1, promote=True, factor_fp16=False, diag_decay=False):
    P = OraclePool(len(states), d_k, d_v, K, r, L, promote, factor_fp16=factor_fp16, diag_decay=diag_decay)
    for j, st in enumerate(states):
        P.set_state(j, to_oracle_state(st, eps[j]), as_init=False)
    return P


def rel_out_err(o_gpu, o_or, S_norm, q_norm):
    den = np.maximum(np.linalg.norm(o_or, axis=1), S_norm * q_norm)
    den = np.maximum(den, 1e-30)
    return np.linalg.norm(o_gpu - o_or, axis=1) / den


def nuclear_bound(st):
    """An upper bound on the sum of the singular values a compaction of the exported factored state
    `st` can keep: the local part sum_a sigma_a u_a v_a^T + sum_j c_j k_j w_j^T has nuclear norm at
    most sum_a sigma_a + sum_j |c_j| |k_j| |w_j|, and the frozen values are kept or dropped as they
    are."""
    if isinstance(st, dict):  # a GPU export
        if st["dense"]:
            return 0.0
        sig, c, Kp, Wp = st["sigma"], st["c"], st["K"], st["W"]
    else:  # an oracle state
        if st.dense:
            return 0.0
        sig, c, Kp, Wp = st.sigma, st.pc, st.PK, st.PW
    sig, c = np.asarray(sig, np.float64), np.asarray(c, np.float64)
    pad = np.sum(np.abs(c) * np.linalg.norm(np.asarray(Kp, np.float64), axis=1)
                 * np.linalg.norm(np.asarray(Wp, np.float64), axis=1)) if len(c) else 0.0
    return float(np.sum(np.abs(sig)) + pad)


def states_of(P, n):
    """The oracle pool's states 0..n-1 (e.g. just before a compaction, for compare_compacted's `before`)."""
    return [P.get_state(j) for j in range(n)]


def compare_compacted(gpu_states, P, eps, K=None, fp16=False, before=None):
    """Compare GPU states after a compaction with the oracle's.  Returns
    (max state rel err, max sigma rel err, guard-band count, rank mismatches outside the guard band).
    fp16: the state error is reported as TOL * err / (TOL ||S|| + 2 rho), so that TOL stays the bar.
    A state the compaction promoted (factored in `before`, the exports the compaction started from,
    dense after it) is built on each side from the factors that side rounded to fp16 at this
    compaction, so it gets the same allowance, with rho taken from nuclear_bound(before[j])."""
    worst_s, worst_sig, guard, bad = 0.0, 0.0, 0, []
    for j, st in enumerate(gpu_states):
        ost = P.get_state(j)
        Sg = reconstruct(st)
        So = P.reconstruct(j)
        nrm = np.linalg.norm(So)
        err = np.linalg.norm(Sg - So)
        promoted = before is not None and ost.dense and st["dense"] and nuclear_bound(before[j]) > 0.0
        if fp16 and (not ost.dense or promoted):
            d_k, d_v = So.shape
            rho = fp16_rounding_bound(ost.sigma, d_k, d_v) if not ost.dense else \
                fp16_rounding_bound([nuclear_bound(before[j])], d_k, d_v)
            allowed = TOL * nrm + 2.0 * rho
            worst_s = max(worst_s, TOL * err / max(allowed, 1e-30))
        else:
            worst_s = max(worst_s, err / max(nrm, 1e-30))
        if st["dense"] != ost.dense:
            bad.append((j, "dense flag"))
            continue
        if st["dense"]:
            continue
        sg = np.sort(st["sigma"].astype(np.float64))[::-1]
        so = np.sort(ost.sigma)[::-1]
        smax = max(sg[0] if len(sg) else 0.0, so[0] if len(so) else 0.0)
        if len(sg) != len(so):
            thr = eps[j] * smax
            longer = sg if len(sg) > len(so) else so
            extra = longer[min(len(sg), len(so)):]
            if np.all(np.abs(extra - thr) <= GUARD * smax):
                guard += 1
            else:
                bad.append((j, f"rank {len(sg)} vs {len(so)}"))
            continue
        if len(sg):
            worst_sig = max(worst_sig, float(np.max(np.abs(sg - so) / so)))
    return worst_s, worst_sig, guard, bad


def active_projector_err(gpu_state, ost, r, fp16=False):
    """Projector distance of the active block when it is separated from the rest by a gap > 1e-2 sigma_max.
    fp16: reported as TOL * err / (TOL + 2 (2 sqrt(r) delta + r delta^2)), so that TOL stays the bar."""
    if gpu_state["dense"] or ost.dense:
        return 0.0
    sg = gpu_state["sigma"]
    if len(sg) <= r:
        return 0.0
    smax = float(sg[0])
    if (sg[r - 1] - sg[r]) / smax <= 1e-2:
        return 0.0
    Ug = gpu_state["U"][:r].T.astype(np.float64)
    Uo = ost.U[:r].T
    Vg = gpu_state["V"][:r].T.astype(np.float64)
    Vo = ost.V[:r].T
    eu, ev = np.linalg.norm(Ug @ Ug.T - Uo @ Uo.T), np.linalg.norm(Vg @ Vg.T - Vo @ Vo.T)
    if not fp16:
        return max(eu, ev)
    out = 0.0
    for e, d in ((eu, Ug.shape[0]), (ev, Vg.shape[0])):
        delta = U16 + np.sqrt(d) * SUB16
        out = max(out, TOL * e / (TOL + 2.0 * (2.0 * np.sqrt(r) * delta + r * delta * delta)))
    return out

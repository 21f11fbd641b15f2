"""Python side of the fp64 CPU oracle (test infrastructure only).

Thin ctypes wrapper over ``sinkstate_oracle.c``.  Only tests/,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it; the HIP library never does.  Arrays cross the boundary as contiguous
float64 numpy arrays.

The arithmetic lives in the C file, whose header cites the passages each
function follows (SinkState arXiv 2611.14246: 2.1 recurrence, 3.2 Design 1,
4.2 buffering / top-subspace SVD / staggering, 4.4 memory layout; SEED
arXiv 2611.06084: section 2 eq. (2) delta rule, Prop. 3 error bound).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sinkstate_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build_oracle(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build_oracle(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_create.restype = ctypes.c_void_p
    lib.orc_create.argtypes = [ctypes.c_int64] + [ctypes.c_int] * 6
    lib.orc_destroy.argtypes = [ctypes.c_void_p]
    lib.orc_dense_limit.argtypes = [ctypes.c_void_p]
    lib.orc_set_state.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                  _dp, _dp, _dp, ctypes.c_int, _dp, _dp, _dp, ctypes.c_int, _dp, ctypes.c_int]
    lib.orc_get_sizes.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [ctypes.POINTER(ctypes.c_int)] * 4 + [_dp]
    lib.orc_get_state.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [_dp] * 7
    lib.orc_get_bound.restype = ctypes.c_double
    lib.orc_get_bound.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.orc_get_compactions.restype = ctypes.c_int64
    lib.orc_get_compactions.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.orc_reconstruct.argtypes = [ctypes.c_void_p, ctypes.c_int64, _dp]
    lib.orc_decode.restype = ctypes.c_int64
    lib.orc_decode.argtypes = [ctypes.c_void_p] + [_dp] * 6 + [ctypes.c_int]
    lib.orc_readout.argtypes = [ctypes.c_void_p, _dp, _dp, ctypes.c_int]
    lib.orc_compact.restype = ctypes.c_int64
    lib.orc_compact.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, ctypes.c_int]
    lib.orc_round_fp16.restype = ctypes.c_double
    lib.orc_round_fp16.argtypes = [ctypes.c_double]
    lib.orc_set_factor_fp16.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.orc_set_diag_decay.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.orc_consolidate.restype = ctypes.c_int64
    lib.orc_consolidate.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64, ctypes.c_int]
    lib.orc_householder_qr.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
    lib.orc_jacobi_svd.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp]
    lib.orc_brand.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.orc_schedule_due.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.orc_rsvd_init.argtypes = [ctypes.c_int, ctypes.c_int, _dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp,
                                  ctypes.c_double, ctypes.c_int, _dp, _dp, _dp]
    lib.orc_rsvd_init.restype = ctypes.c_int
    lib.orc_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_dp)


def max_threads() -> int:
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------
# building blocks, exposed so that tests can pin them on their own
# --------------------------------------------------------------------------
def householder_qr(A):
    """A (d x m) -> Q (d x p), R (p x m), p = min(d, m): Householder thin QR."""
    A = np.asarray(A, dtype=np.float64)
    d, m = A.shape
    p = min(d, m)
    Acm = _f64(A.T)  # column-major == transpose in row-major
    Q = np.zeros((p, d))
    R = np.zeros((m, p))
    _load().orc_householder_qr(d, m, _ptr(Acm), _ptr(Q), _ptr(R))
    return Q.T.copy(), R.T.copy()


def jacobi_svd(A):
    """A (rows x cols) -> U (rows x cols), s (cols, descending), V (cols x cols)."""
    A = np.asarray(A, dtype=np.float64)
    rows, cols = A.shape
    Acm = _f64(A.T)
    U = np.zeros((cols, rows))
    s = np.zeros(cols)
    V = np.zeros((cols, cols))
    _load().orc_jacobi_svd(rows, cols, _ptr(Acm), _ptr(U), _ptr(s), _ptr(V))
    return U.T.copy(), s, V.T.copy()


def brand_update(UC, VC, sc):
    """SVD of UC diag(sc) VC^T via Brand's core (UC: d_k x m, VC: d_v x m)."""
    UC = np.asarray(UC, dtype=np.float64)
    VC = np.asarray(VC, dtype=np.float64)
    d_k, m = UC.shape
    d_v = VC.shape[0]
    pr = min(d_v, m)
    Uo = np.zeros((pr, d_k))
    Vo = np.zeros((pr, d_v))
    so = np.zeros(pr)
    rc = _load().orc_brand(d_k, d_v, m, _ptr(_f64(UC.T)), _ptr(_f64(VC.T)), _ptr(_f64(sc)), _ptr(Uo), _ptr(Vo),
                           _ptr(so))
    if rc < 0:
        raise MemoryError("oracle brand update failed")
    return Uo.T.copy(), so, Vo.T.copy()


def rsvd_init(S, omega, eps, iters=2, max_rank=None):
    """Randomized block SVD of a dense state S (d_k x d_v): omega is (nb, d_k, b), one Gaussian
    block per entry.  Returns U (R x d_k), V (R x d_v), sigma (R) with S ~ U^T diag(sigma) V."""
    S = np.asarray(S, dtype=np.float64)
    d_k, d_v = S.shape
    omega = np.asarray(omega, dtype=np.float64)
    nb, dk2, b = omega.shape
    assert dk2 == d_k
    max_rank = min(d_k, d_v) if max_rank is None else int(max_rank)
    om = _f64(np.transpose(omega, (0, 2, 1)))  # per block column-major (d_k x b)
    U = np.zeros((max(1, max_rank), d_k))
    V = np.zeros((max(1, max_rank), d_v))
    sig = np.zeros(max(1, max_rank))
    R = _load().orc_rsvd_init(d_k, d_v, _ptr(_f64(S)), b, nb, int(iters), _ptr(om), float(eps), max_rank, _ptr(U),
                              _ptr(V), _ptr(sig))
    if R < 0:
        raise MemoryError("oracle randomized SVD failed")
    return U[:R].copy(), V[:R].copy(), sig[:R].copy()


def round_fp16(x: float) -> float:
    """binary16 rounding (nearest, ties to even) of one value, as the oracle stores fp16 factors."""
    return float(_load().orc_round_fp16(float(x)))


def schedule_due(step: int, K: int, offsets) -> list:
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    out = np.zeros(max(1, len(offs)), dtype=np.int32)
    c = _load().orc_schedule_due(int(step), int(K), len(offs), offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    return [int(x) for x in out[:c]]


class OracleState:
    """Canonical fp64 state: components (sigma descending), pad, or dense S."""

    def __init__(self, U=None, V=None, sigma=None, PK=None, PW=None, pc=None, S=None, rule=0, eps=0.0):
        self.U = U
        self.V = V
        self.sigma = sigma
        self.PK = PK
        self.PW = PW
        self.pc = pc
        self.S = S
        self.rule = rule
        self.eps = eps

    @property
    def dense(self):
        return self.S is not None


class OraclePool:
    """A pool of N states held by the C oracle."""

    def __init__(self, n_states, d_k, d_v, K=8, r=8, L=-1, promote=True, factor_fp16=False, diag_decay=False):
        lib = _load()
        self._lib = lib
        self.N, self.d_k, self.d_v, self.K, self.r = int(n_states), int(d_k), int(d_v), int(K), int(r)
        self._p = lib.orc_create(self.N, self.d_k, self.d_v, self.K, self.r, int(L), int(bool(promote)))
        if not self._p:
            raise MemoryError("orc_create failed")
        lib.orc_set_factor_fp16(self._p, int(bool(factor_fp16)))
        lib.orc_set_diag_decay(self._p, int(bool(diag_decay)))
        self.diag_decay = bool(diag_decay)
        self.L = int(lib.orc_dense_limit(self._p))

    def close(self):
        if self._p:
            self._lib.orc_destroy(self._p)
            self._p = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- state access ------------------------------------------------------
    def set_state(self, s, st: OracleState, as_init: bool = True):
        """Load a state.  as_init=True applies the create-time dense fallback (R > L);
        as_init=False loads a mid-run state as given: its first min(r, R) components are the
        active part and the rest the frozen part, each sorted on its own."""
        dk, dv = self.d_k, self.d_v
        if st.S is not None:
            S = _f64(st.S).reshape(dk, dv)
            rc = self._lib.orc_set_state(self._p, int(s), int(st.rule), float(st.eps), 0, None, None, None, 0, None,
                                         None, None, 1, _ptr(S), int(as_init))
        else:
            sig = _f64(st.sigma if st.sigma is not None else np.zeros(0))
            R = sig.shape[0]
            U = _f64(st.U if R else np.zeros((0, dk))).reshape(R, dk)
            V = _f64(st.V if R else np.zeros((0, dv))).reshape(R, dv)
            pc = _f64(st.pc if st.pc is not None else np.zeros(0))
            n = pc.shape[0]
            PK = _f64(st.PK if n else np.zeros((0, dk))).reshape(n, dk)
            PW = _f64(st.PW if n else np.zeros((0, dv))).reshape(n, dv)
            rc = self._lib.orc_set_state(self._p, int(s), int(st.rule), float(st.eps), R, _ptr(U), _ptr(V), _ptr(sig),
                                         n, _ptr(PK), _ptr(PW), _ptr(pc), 0, None, int(as_init))
        if rc != 0:
            raise ValueError(f"orc_set_state failed for state {s}")

    def get_state(self, s) -> OracleState:
        R, n, dense, rule = (ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int())
        eps = ctypes.c_double()
        self._lib.orc_get_sizes(self._p, int(s), ctypes.byref(R), ctypes.byref(n), ctypes.byref(dense),
                                ctypes.byref(rule), ctypes.byref(eps))
        dk, dv = self.d_k, self.d_v
        if dense.value:
            S = np.zeros((dk, dv))
            self._lib.orc_get_state(self._p, int(s), None, None, None, None, None, None, _ptr(S))
            return OracleState(S=S, rule=rule.value, eps=eps.value)
        U = np.zeros((R.value, dk))
        V = np.zeros((R.value, dv))
        sig = np.zeros(R.value)
        PK = np.zeros((n.value, dk))
        PW = np.zeros((n.value, dv))
        pc = np.zeros(n.value)
        self._lib.orc_get_state(self._p, int(s), _ptr(U), _ptr(V), _ptr(sig), _ptr(PK), _ptr(PW), _ptr(pc), None)
        return OracleState(U, V, sig, PK, PW, pc, None, rule.value, eps.value)

    def reconstruct(self, s):
        out = np.zeros((self.d_k, self.d_v))
        self._lib.orc_reconstruct(self._p, int(s), _ptr(out))
        return out

    def bound(self, s) -> float:
        return float(self._lib.orc_get_bound(self._p, int(s)))

    def compactions(self, s) -> int:
        return int(self._lib.orc_get_compactions(self._p, int(s)))

    # -- the recurrence ----------------------------------------------------
    def decode(self, q, k, v, alpha, beta=None, nthreads=0):
        N, dk, dv = self.N, self.d_k, self.d_v
        q = _f64(q).reshape(N, dk)
        k = _f64(k).reshape(N, dk)
        v = _f64(v).reshape(N, dv)
        alpha = _f64(alpha).reshape((N, dk) if self.diag_decay else N)  # per-channel decay: [N][d_k]
        b = None if beta is None else _f64(beta).reshape(N)
        o = np.zeros((N, dv))
        bad = self._lib.orc_decode(self._p, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(o), int(nthreads))
        if bad:
            raise RuntimeError(f"oracle decode: {bad} states had a full pad (schedule missed a compaction)")
        return o

    def readout(self, q, nthreads=0):
        q = _f64(q).reshape(self.N, self.d_k)
        o = np.zeros((self.N, self.d_v))
        self._lib.orc_readout(self._p, _ptr(q), _ptr(o), int(nthreads))
        return o

    def compact(self, ids=None, nthreads=0):
        if ids is None:
            bad = self._lib.orc_compact(self._p, None, 0, int(nthreads))
        else:
            ids = np.ascontiguousarray(ids, dtype=np.int64)
            bad = self._lib.orc_compact(self._p, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ids.shape[0],
                                        int(nthreads))
        if bad:
            raise RuntimeError(f"oracle compact failed for {bad} states")

    def consolidate(self, ids=None, nthreads=0):
        """Exact SVD of each listed state's frozen part, dropping singular values below
        eps * sigma_0 (SinkState 4.3, Figure 7(a)); the active part and the pad stay."""
        if ids is None:
            bad = self._lib.orc_consolidate(self._p, None, 0, int(nthreads))
        else:
            ids = np.ascontiguousarray(ids, dtype=np.int64)
            bad = self._lib.orc_consolidate(self._p, ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                            ids.shape[0], int(nthreads))
        if bad:
            raise RuntimeError(f"oracle consolidate failed for {bad} states")

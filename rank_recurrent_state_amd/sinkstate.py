"""ctypes binding of libsinkstate.so (argument marshalling only).

Every function keeps the name of the C entry point it wraps, without the
``ss_`` prefix.  Tensors are torch fp32 tensors on the GPU; only their data
pointers and the current HIP stream cross the boundary.  There is no CPU
fallback: if the library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
import weakref

import numpy as np
import torch  # loaded first so that the library binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkstate.so")

SS_OK, SS_ERR_ARG, SS_ERR_SHAPE, SS_ERR_OOM, SS_ERR_CAPACITY, SS_ERR_HIP, SS_ERR_STATE = range(7)
RULE_SCALAR, RULE_DELTA = 0, 1

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_f32p = ctypes.POINTER(ctypes.c_float)


class PoolDesc(ctypes.Structure):
    _fields_ = [
        ("n_states", ctypes.c_int64),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("pad_slots", ctypes.c_int32), ("r_active", ctypes.c_int32),
        ("dense_rank_limit", ctypes.c_int32), ("promote_on_compact", ctypes.c_int32),
        ("max_frozen", ctypes.c_int32), ("force_dense", ctypes.c_int32),
        ("n_groups", ctypes.c_int32),
        ("group_of_state", _c_i32p), ("group_offset", _c_i32p),
        ("rule", _c_u8p), ("eps", _c_f32p), ("eps_default", ctypes.c_float),
        ("dense_capacity", ctypes.c_int64), ("arena_components", ctypes.c_int64),
        ("factor_fp16", ctypes.c_int32), ("diag_decay", ctypes.c_int32),
    ]


class Init(ctypes.Structure):
    _fields_ = [("comp_off", _c_i64p), ("u", _c_f32p), ("v", _c_f32p), ("sigma", _c_f32p),
                ("dense_mask", _c_u8p), ("dense", _c_f32p)]


class Stats(ctypes.Structure):
    _fields_ = [
        ("n_states", ctypes.c_int64), ("n_dense", ctypes.c_int64), ("n_factored", ctypes.c_int64),
        ("active_components", ctypes.c_int64), ("frozen_components", ctypes.c_int64),
        ("pad_entries", ctypes.c_int64), ("live_bytes", ctypes.c_int64), ("reserved_bytes", ctypes.c_int64),
        ("max_rank", ctypes.c_int64), ("rank_hist", ctypes.c_int64 * 65),
        ("decode_calls", ctypes.c_int64), ("compact_calls", ctypes.c_int64), ("readout_calls", ctypes.c_int64),
        ("decode_bytes", ctypes.c_uint64), ("decode_bytes_factored", ctypes.c_uint64),
        ("decode_bytes_dense", ctypes.c_uint64), ("compact_states", ctypes.c_uint64),
        ("compact_flops", ctypes.c_uint64), ("promotions", ctypes.c_int64), ("cap_truncations", ctypes.c_int64),
        ("ring_capacity", ctypes.c_int64 * 2), ("ring_used", ctypes.c_int64 * 2),
        ("ring_head", ctypes.c_int64 * 2),
        ("ring_repacks", ctypes.c_int64), ("ring_syncs", ctypes.c_int64),
        ("kernel_ms", ctypes.c_double * 8), ("kernel_launches", ctypes.c_int64 * 8),
        ("consolidate_calls", ctypes.c_int64), ("consolidate_states", ctypes.c_uint64),
        ("consolidate_flops", ctypes.c_uint64), ("consolidate_removed", ctypes.c_uint64),
        ("jacobi_limit_hits", ctypes.c_int64),
    ]


KERNELS = ("decode_factored", "decode_dense", "readout_factored", "readout_dense", "compact", "materialize",
           "dense_fold", "consolidate")


_lib = None


def load_library():
    """Load libsinkstate.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with rank_recurrent_state_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.ss_state_pool_create.argtypes = [ctypes.POINTER(PoolDesc), ctypes.POINTER(Init), vp, ctypes.POINTER(vp)]
    lib.ss_state_pool_destroy.argtypes = [vp]
    lib.ss_decode_step.argtypes = [vp] + [vp] * 6 + [vp]
    lib.ss_readout.argtypes = [vp, vp, vp, vp]
    lib.ss_compact.argtypes = [vp, ctypes.c_int32, vp]
    lib.ss_compact_ids.argtypes = [vp, _c_i32p, ctypes.c_int64, vp]
    lib.ss_consolidate.argtypes = [vp, ctypes.c_int32, vp]
    lib.ss_consolidate_next.argtypes = [vp, ctypes.c_int32, _c_i32p, _c_i32p, vp]
    lib.ss_consolidate_async.argtypes = [vp, ctypes.c_int32, vp, vp, _c_i32p]
    lib.ss_consolidate_poll.argtypes = [vp, ctypes.c_int32, vp, _c_i32p]
    lib.ss_consolidate_host.argtypes = [vp, ctypes.c_int32, vp, ctypes.c_int32, _c_i32p]
    lib.ss_host_consolidate_frozen.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _c_f32p, _c_f32p,
                                               _c_f32p, ctypes.c_float, ctypes.c_float, _c_i32p]
    lib.ss_schedule_due.argtypes = [vp, ctypes.c_int64, _c_i32p, ctypes.c_int32, _c_i32p]
    lib.ss_state_export.argtypes = [vp, _c_i64p, ctypes.c_int64, vp, ctypes.c_size_t,
                                    ctypes.POINTER(ctypes.c_size_t), vp]
    lib.ss_pool_stats.argtypes = [vp, ctypes.POINTER(Stats), vp]
    lib.ss_pool_timing.argtypes = [vp, ctypes.c_int32]
    lib.ss_dense_rank_limit.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.ss_dense_rank_limit.restype = ctypes.c_int32
    lib.ss_decode_bytes_per_state.argtypes = [ctypes.c_int32] * 7
    lib.ss_decode_bytes_per_state.restype = ctypes.c_uint64
    lib.ss_step_graph_create.argtypes = [vp] + [vp] * 6 + [ctypes.POINTER(vp)]
    lib.ss_step_graph_launch.argtypes = [vp, ctypes.c_int64, vp]
    lib.ss_step_graph_destroy.argtypes = [vp]
    lib.ss_rsvd_init.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp]
    lib.ss_rsvd_init.restype = ctypes.c_int
    lib.ss_rsvd_init_noalloc.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp, vp, vp, vp]
    lib.ss_rsvd_init_noalloc.restype = ctypes.c_int
    lib.ss_state_pool_create_from_dense.argtypes = [ctypes.POINTER(PoolDesc)] + [vp] * 5 + [ctypes.c_int32, vp,
                                                                                         ctypes.POINTER(vp)]
    lib.ss_state_pool_create_from_dense.restype = ctypes.c_int
    lib.ss_status_string.argtypes = [ctypes.c_int]
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_last_error.restype = ctypes.c_char_p
    for name in ("ss_state_pool_create", "ss_state_pool_destroy", "ss_decode_step", "ss_readout", "ss_compact",
                 "ss_schedule_due", "ss_state_export", "ss_pool_stats", "ss_pool_timing", "ss_step_graph_create",
                 "ss_step_graph_launch", "ss_step_graph_destroy"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


class SinkStateError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def _check(st):
    if st != SS_OK:
        lib = load_library()
        raise SinkStateError(st, f"{lib.ss_status_string(st).decode()}: {lib.ss_last_error().decode()}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, n_expected, name):
    if t is None:
        return None
    if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    if t.numel() != n_expected:
        raise ValueError(f"{name} has {t.numel()} elements, expected {n_expected}")
    return ctypes.c_void_p(t.data_ptr())


def _arr(a, dtype, ctype):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctype)


def dense_rank_limit(d_k: int, d_v: int) -> int:
    return int(load_library().ss_dense_rank_limit(d_k, d_v))


DECODE_FACTORED, DECODE_DENSE_BUFFERED, DECODE_DENSE_PLAIN, DECODE_FACTORED_FP16 = 0, 1, 2, 3


def decode_bytes_per_state(d_k, d_v, pad_slots, n_comp, n_pad, rule, kind) -> int:
    return int(load_library().ss_decode_bytes_per_state(d_k, d_v, pad_slots, n_comp, n_pad, rule, int(kind)))


class StatePool:
    """Owner of one ss_pool handle."""

    def __init__(self, handle, n_states, d_k, d_v, K, r, n_groups, any_delta, diag_decay=False):
        self.handle = handle
        self.N, self.d_k, self.d_v, self.K, self.r, self.n_groups = n_states, d_k, d_v, K, r, n_groups
        self.any_delta = any_delta
        self.diag_decay = diag_decay
        self.n_alpha = n_states * d_k if diag_decay else n_states  # per-channel decay: alpha is [N][d_k]
        self._graphs = weakref.WeakSet()  # step graphs over this pool: destroyed before it

    def close(self):
        if self.handle:
            for g in list(self._graphs):
                g.close()
            load_library().ss_state_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _desc(n_states, d_k, d_v, pad_slots, r_active, dense_rank_limit, promote_on_compact, max_frozen, force_dense,
          group_of_state, group_offset, rule, eps, eps_default, dense_capacity, arena_components, factor_fp16,
          diag_decay):
    """ss_pool_desc and the host arrays it points to (kept alive by the caller)."""
    n_groups = 1 if group_offset is None else len(group_offset)
    g_a, g_p = _arr(group_of_state, np.int32, _c_i32p)
    o_a, o_p = _arr(group_offset, np.int32, _c_i32p)
    r_a, r_p = _arr(rule, np.uint8, _c_u8p)
    e_a, e_p = _arr(eps, np.float32, _c_f32p)
    desc = PoolDesc(int(n_states), int(d_k), int(d_v), int(pad_slots), int(r_active), int(dense_rank_limit),
                    int(bool(promote_on_compact)), int(max_frozen), int(bool(force_dense)), int(n_groups),
                    g_p, o_p, r_p, e_p, float(eps_default), int(dense_capacity),
                    int(arena_components), int(factor_fp16), int(bool(diag_decay)))
    return desc, [g_a, o_a, r_a, e_a], n_groups


def state_pool_create(n_states, d_k, d_v, pad_slots=8, r_active=8, dense_rank_limit=-1, promote_on_compact=True,
                      max_frozen=0, force_dense=False, group_of_state=None, group_offset=None, rule=None, eps=None,
                      eps_default=0.0, dense_capacity=0, comp_off=None, u=None, v=None, sigma=None,
                      arena_components=0, dense_mask=None, dense=None, factor_fp16=False, diag_decay=False,
                      stream=None) -> StatePool:
    lib = load_library()
    desc, keep, n_groups = _desc(n_states, d_k, d_v, pad_slots, r_active, dense_rank_limit, promote_on_compact,
                                 max_frozen, force_dense, group_of_state, group_offset, rule, eps, eps_default,
                                 dense_capacity, arena_components, factor_fp16, diag_decay)
    init = None
    if comp_off is not None or dense_mask is not None:
        c_a, c_p = _arr(comp_off, np.int64, _c_i64p)
        u_a, u_p = _arr(u, np.float32, _c_f32p)
        v_a, v_p = _arr(v, np.float32, _c_f32p)
        s_a, s_p = _arr(sigma, np.float32, _c_f32p)
        m_a, m_p = _arr(dense_mask, np.uint8, _c_u8p)
        d_a, d_p = _arr(dense, np.float32, _c_f32p)
        keep += [c_a, u_a, v_a, s_a, m_a, d_a]
        init = Init(c_p, u_p, v_p, s_p, m_p, d_p)
    handle = ctypes.c_void_p()
    st = lib.ss_state_pool_create(ctypes.byref(desc), ctypes.byref(init) if init is not None else None,
                                  _stream(stream) if torch.cuda.is_available() else None, ctypes.byref(handle))
    _check(st)
    any_delta = rule is not None and bool(np.any(np.asarray(rule) == 1))
    return StatePool(handle, int(n_states), int(d_k), int(d_v), int(pad_slots), int(r_active), n_groups, any_delta,
                     bool(diag_decay))


def decode_step(pool: StatePool, q, k, v, alpha, beta, o, stream=None):
    N, dk, dv = pool.N, pool.d_k, pool.d_v
    args = [_ptr(q, N * dk, "q"), _ptr(k, N * dk, "k"), _ptr(v, N * dv, "v"), _ptr(alpha, pool.n_alpha, "alpha"),
            _ptr(beta, N, "beta") if beta is not None else None, _ptr(o, N * dv, "o")]
    _check(load_library().ss_decode_step(pool.handle, *args, _stream(stream)))


class StepGraph:
    """Owner of one ss_step_graph: whole steps (decode + due compactions) replayed as HIP graphs
    on fixed input/output tensors."""

    def __init__(self, pool: StatePool, q, k, v, alpha, beta, o):
        N, dk, dv = pool.N, pool.d_k, pool.d_v
        self.pool = pool
        self.buffers = (q, k, v, alpha, beta, o)  # kept alive while the graphs may read them
        args = [_ptr(q, N * dk, "q"), _ptr(k, N * dk, "k"), _ptr(v, N * dv, "v"), _ptr(alpha, pool.n_alpha, "alpha"),
                _ptr(beta, N, "beta") if beta is not None else None, _ptr(o, N * dv, "o")]
        h = ctypes.c_void_p()
        self.handle = None
        _check(load_library().ss_step_graph_create(pool.handle, *args, ctypes.byref(h)))
        self.handle = h
        pool._graphs.add(self)

    def launch(self, step: int, stream=None):
        if not self.handle:
            raise SinkStateError(SS_ERR_STATE, "the step graph is closed (or its pool was)")
        _check(load_library().ss_step_graph_launch(self.handle, int(step), _stream(stream)))

    def close(self):
        if self.handle:
            load_library().ss_step_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rsvd_init(S, omega, eps, iters=2, max_rank=None, stream=None):
    """Randomized block SVD of dense states on the GPU.  S: (n, d_k, d_v) float32 CUDA tensor;
    omega: (n, n_blocks, d_k, block) Gaussian; eps: (n,).  Returns u (n, max_rank, d_k),
    v (n, max_rank, d_v), sigma (n, max_rank) and rank (n,) as CUDA tensors (entries beyond a
    state's rank are unspecified)."""
    n, dk, dv = S.shape
    n2, nb, dk2, b = omega.shape
    if n2 != n or dk2 != dk:
        raise ValueError("omega must be (n, n_blocks, d_k, block)")
    max_rank = min(dk, dv, nb * b) if max_rank is None else int(max_rank)
    dev = S.device
    work = torch.empty_like(S)
    u = torch.empty(n, max_rank, dk, device=dev)
    v = torch.empty(n, max_rank, dv, device=dev)
    sigma = torch.empty(n, max_rank, device=dev)
    rank = torch.empty(n, dtype=torch.int32, device=dev)
    eps_t = torch.as_tensor(eps, dtype=torch.float32, device=dev).expand(n).contiguous()
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    for t, name in ((S, "S"), (omega, "omega")):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 CUDA tensor")
    _check(load_library().ss_rsvd_init(p(S), n, dk, dv, b, nb, int(iters), p(omega), p(eps_t), max_rank, p(work),
                                       p(u), p(v), p(sigma), p(rank), _stream(stream)))
    return u, v, sigma, rank


def rsvd_init_noalloc(S, omega, eps, u, v, sigma, rank, iters=2, stream=None):
    """ss_rsvd_init_noalloc: the randomized block SVD with the library's fixed workspace.  The caller
    passes the outputs, allocated beforehand: u (n, max_rank, d_k), v (n, max_rank, d_v),
    sigma (n, max_rank) float32 and rank (n,) int32 CUDA tensors; eps is an (n,) float32 CUDA tensor."""
    n, dk, dv = S.shape
    n2, nb, dk2, b = omega.shape
    if n2 != n or dk2 != dk:
        raise ValueError("omega must be (n, n_blocks, d_k, block)")
    max_rank = u.shape[1]
    if u.shape != (n, max_rank, dk) or v.shape != (n, max_rank, dv) or sigma.shape != (n, max_rank) \
            or rank.shape != (n,) or eps.shape != (n,):
        raise ValueError("outputs must be u (n, max_rank, d_k), v (n, max_rank, d_v), sigma (n, max_rank), "
                         "rank (n,); eps (n,)")
    for t, name, dt in ((S, "S", torch.float32), (omega, "omega", torch.float32), (eps, "eps", torch.float32),
                        (u, "u", torch.float32), (v, "v", torch.float32), (sigma, "sigma", torch.float32),
                        (rank, "rank", torch.int32)):
        if not (t.is_cuda and t.dtype == dt and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dt} CUDA tensor")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    _check(load_library().ss_rsvd_init_noalloc(p(S), n, dk, dv, b, nb, int(iters), p(omega), p(eps), max_rank,
                                               p(u), p(v), p(sigma), p(rank), _stream(stream)))


def state_pool_from_dense(S, omega, eps, d_k=None, d_v=None, pad_slots=8, r_active=8, iters=2, rule=None,
                          dense_rank_limit=-1, promote_on_compact=True, max_frozen=0, group_of_state=None,
                          group_offset=None, dense_capacity=0, arena_components=0, factor_fp16=False,
                          diag_decay=False, stream=None) -> StatePool:
    """A pool initialized from dense states after prefill: rsvd_init on the GPU, then
    ss_state_pool_create_from_dense, where the library applies the dense fallback and orders each
    state's components.  S: (N, d_k, d_v) float32 (host array or CUDA tensor); omega: (N, n_blocks,
    d_k, block) Gaussian; eps: scalar or (N,)."""
    St = torch.as_tensor(S, dtype=torch.float32).cuda().contiguous()
    Om = torch.as_tensor(omega, dtype=torch.float32).cuda().contiguous()
    N, dk, dv = St.shape
    nb, b = Om.shape[1], Om.shape[3]
    max_rank = min(dk, dv, nb * b)
    eps_a = np.broadcast_to(np.asarray(eps, dtype=np.float32), (N,)).copy()
    u, v, sg, rk = rsvd_init(St, Om, torch.from_numpy(eps_a).cuda(), iters=iters, max_rank=max_rank, stream=stream)
    desc, keep, n_groups = _desc(N, dk, dv, pad_slots, r_active, dense_rank_limit, promote_on_compact, max_frozen,
                                 False, group_of_state, group_offset, rule, eps_a, 0.0, dense_capacity,
                                 arena_components, factor_fp16, diag_decay)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    handle = ctypes.c_void_p()
    _check(load_library().ss_state_pool_create_from_dense(ctypes.byref(desc), p(St), p(u), p(v), p(sg), p(rk),
                                                          max_rank, _stream(stream), ctypes.byref(handle)))
    any_delta = rule is not None and bool(np.any(np.asarray(rule) == 1))
    return StatePool(handle, int(N), int(dk), int(dv), int(pad_slots), int(r_active), n_groups, any_delta,
                     bool(diag_decay))


def readout(pool: StatePool, q, o, stream=None):
    N, dk, dv = pool.N, pool.d_k, pool.d_v
    _check(load_library().ss_readout(pool.handle, _ptr(q, N * dk, "q"), _ptr(o, N * dv, "o"), _stream(stream)))


def compact(pool: StatePool, group: int = -1, stream=None):
    _check(load_library().ss_compact(pool.handle, int(group), _stream(stream)))


def consolidate(pool: StatePool, group: int = -1, stream=None):
    """Consolidate the frozen parts of group `group` (all groups when < 0) on the device."""
    _check(load_library().ss_consolidate(pool.handle, int(group), _stream(stream)))


def consolidate_next(pool: StatePool, max_groups: int, stream=None) -> list:
    """Consolidate up to max_groups groups from the wait queue; returns their ids."""
    out = (ctypes.c_int32 * max(1, int(max_groups)))()
    n = ctypes.c_int32()
    _check(load_library().ss_consolidate_next(pool.handle, int(max_groups), out, ctypes.byref(n), _stream(stream)))
    return [int(out[i]) for i in range(n.value)]


CONS_IDLE, CONS_RUNNING, CONS_INSTALLED, CONS_DISCARDED = 0, 1, 2, 3


def consolidate_async(pool: StatePool, side, group: int = -1, stream=None) -> int:
    """Start the consolidation of one group on the stream `side` (group < 0: the head of the wait
    queue); returns the group launched, or -1 when none waits."""
    g = ctypes.c_int32()
    _check(load_library().ss_consolidate_async(pool.handle, int(group), _stream(stream), _stream(side), ctypes.byref(g)))
    return int(g.value)


def host_consolidate_frozen(u, v, sigma, sigma0, eps):
    """ss_host_consolidate_frozen on host arrays u (f, d_k), v (f, d_v), sigma (f,): returns the kept
    (u, v, sigma) as new float32 arrays."""
    u = np.ascontiguousarray(u, np.float32).copy()
    v = np.ascontiguousarray(v, np.float32).copy()
    sg = np.ascontiguousarray(sigma, np.float32).copy()
    f, dk = u.shape
    dv = v.shape[1]
    kept = ctypes.c_int32(0)
    _check(load_library().ss_host_consolidate_frozen(dk, dv, f, u.ctypes.data_as(_c_f32p), v.ctypes.data_as(_c_f32p),
                                                     sg.ctypes.data_as(_c_f32p), float(sigma0), float(eps),
                                                     ctypes.byref(kept)))
    k = kept.value
    return u[:k], v[:k], sg[:k]


def consolidate_host(pool: StatePool, group: int = -1, threads: int = 0, stream=None) -> int:
    """ss_consolidate_host: the group launched (-1: none waits)."""
    out = ctypes.c_int32(-1)
    _check(load_library().ss_consolidate_host(pool.handle, int(group), _stream(stream), int(threads), ctypes.byref(out)))
    return out.value


def consolidate_poll(pool: StatePool, wait: bool = False, stream=None) -> int:
    """CONS_IDLE, CONS_RUNNING, CONS_INSTALLED (install enqueued on `stream`) or CONS_DISCARDED."""
    st = ctypes.c_int32()
    _check(load_library().ss_consolidate_poll(pool.handle, int(bool(wait)), _stream(stream), ctypes.byref(st)))
    return int(st.value)


def compact_ids(pool: StatePool, ids, stream=None):
    """Compact the listed states only (the rest of their groups moves unchanged)."""
    a = np.ascontiguousarray(ids, dtype=np.int32)
    _check(load_library().ss_compact_ids(pool.handle, a.ctypes.data_as(_c_i32p), int(a.shape[0]), _stream(stream)))


def schedule_due(pool: StatePool, step: int) -> list:
    out = (ctypes.c_int32 * max(1, pool.n_groups))()
    n = ctypes.c_int32()
    _check(load_library().ss_schedule_due(pool.handle, int(step), out, max(1, pool.n_groups), ctypes.byref(n)))
    return [int(out[i]) for i in range(n.value)]


def pool_stats(pool: StatePool, stream=None) -> dict:
    s = Stats()
    _check(load_library().ss_pool_stats(pool.handle, ctypes.byref(s), _stream(stream)))
    d = {name: getattr(s, name) for name, _ in Stats._fields_ if name not in ("rank_hist", "kernel_ms",
                                                                              "kernel_launches", "ring_capacity",
                                                                              "ring_used", "ring_head")}
    for name in ("ring_capacity", "ring_used", "ring_head"):
        d[name] = list(getattr(s, name))
    d["rank_hist"] = list(s.rank_hist)
    d["kernel_ms"] = {k: s.kernel_ms[i] for i, k in enumerate(KERNELS)}
    d["kernel_launches"] = {k: s.kernel_launches[i] for i, k in enumerate(KERNELS)}
    return d


def pool_timing(pool: StatePool, enable: bool = True):
    _check(load_library().ss_pool_timing(pool.handle, int(bool(enable))))


def state_export(pool: StatePool, ids, stream=None) -> list:
    """Canonical states (effective weights) as a list of dicts of float32 arrays."""
    lib = load_library()
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    need = ctypes.c_size_t()
    st = lib.ss_state_export(pool.handle, ids.ctypes.data_as(_c_i64p), ids.shape[0], None, 0, ctypes.byref(need),
                             _stream(stream))
    if st not in (SS_OK, SS_ERR_CAPACITY):
        _check(st)
    buf = np.zeros(max(1, need.value), dtype=np.uint8)
    _check(lib.ss_state_export(pool.handle, ids.ctypes.data_as(_c_i64p), ids.shape[0],
                               buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes, ctypes.byref(need), _stream(stream)))
    dk, dv = pool.d_k, pool.d_v
    out, pos = [], 0
    for _ in range(ids.shape[0]):
        hdr = buf[pos:pos + 32].view(np.int32)
        pos += 32
        sid, dense, R, ra, n, rule, dpad = (int(x) for x in hdr[:7])
        if dense:
            S = buf[pos:pos + 4 * dk * dv].view(np.float32).reshape(dk, dv).copy()
            pos += 4 * dk * dv
            out.append({"id": sid, "dense": True, "S": S, "rule": rule, "dense_pad": dpad})
            continue
        f = buf[pos:pos + 4 * (R * (1 + dk + dv) + n * (1 + dk + dv))].view(np.float32)
        pos += f.nbytes
        o = 0
        sig = f[o:o + R].copy(); o += R
        U = f[o:o + R * dk].reshape(R, dk).copy(); o += R * dk
        V = f[o:o + R * dv].reshape(R, dv).copy(); o += R * dv
        c = f[o:o + n].copy(); o += n
        Kp = f[o:o + n * dk].reshape(n, dk).copy(); o += n * dk
        W = f[o:o + n * dv].reshape(n, dv).copy(); o += n * dv
        out.append({"id": sid, "dense": False, "sigma": sig, "U": U, "V": V, "n_active": ra, "c": c, "K": Kp,
                    "W": W, "rule": rule})
    return out

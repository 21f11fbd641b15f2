"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before any HIP call, and its host-side
arithmetic matches what the pages print."""
import ctypes
import json
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkstate.h")
GOLD = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    from rank_recurrent_state_amd import sinkstate
    if not os.path.exists(sinkstate.LIB_PATH):
        from rank_recurrent_state_amd.build import build
        build()
    return sinkstate.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from rank_recurrent_state_amd import sinkstate
    names = _declared()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", sinkstate.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if " T " in line)
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_library_links_only_expected_runtimes():
    from rank_recurrent_state_amd import sinkstate
    out = subprocess.run(["readelf", "-d", sinkstate.LIB_PATH], capture_output=True, text=True, check=True).stdout
    needed = re.findall(r"NEEDED.*\[(.*)\]", out)
    assert any("amdhip64" in n for n in needed)
    assert not any("torch" in n or "python" in n or "oracle" in n for n in needed), needed


def test_status_strings(lib):
    for st in range(7):
        assert lib.ss_status_string(st)
    assert lib.ss_last_error() is not None


def test_create_rejects_bad_arguments_without_touching_the_gpu(lib):
    from rank_recurrent_state_amd import sinkstate as ss
    out = ctypes.c_void_p()
    assert lib.ss_state_pool_create(None, None, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert lib.ss_state_pool_create(None, None, None, None) == ss.SS_ERR_ARG
    base = dict(n_states=4, d_k=16, d_v=32, pad_slots=8, r_active=8, dense_rank_limit=-1, promote_on_compact=1,
                max_frozen=0, force_dense=0, n_groups=1, group_of_state=None, group_offset=None, rule=None,
                eps=None, eps_default=1e-3, dense_capacity=0, arena_components=0, factor_fp16=0, diag_decay=0)
    cases = [({"n_states": 0}, ss.SS_ERR_ARG), ({"d_k": 18}, ss.SS_ERR_SHAPE), ({"d_v": 260}, ss.SS_ERR_SHAPE),
             ({"pad_slots": 9}, ss.SS_ERR_SHAPE), ({"r_active": 0}, ss.SS_ERR_SHAPE),
             ({"n_groups": 0}, ss.SS_ERR_ARG), ({"max_frozen": 300}, ss.SS_ERR_ARG),
             ({"eps_default": -1.0}, ss.SS_ERR_ARG), ({"dense_capacity": 5}, ss.SS_ERR_ARG),
             ({"d_k": 260, "d_v": 128}, ss.SS_ERR_SHAPE), ({"arena_components": -1}, ss.SS_ERR_ARG),
             ({"arena_components": 1 << 31}, ss.SS_ERR_ARG), ({"factor_fp16": 2}, ss.SS_ERR_ARG),
             ({"factor_fp16": -1}, ss.SS_ERR_ARG), ({"diag_decay": 2}, ss.SS_ERR_ARG)]
    for over, expect in cases:
        d = dict(base, **over)
        desc = ss.PoolDesc(*[d[f] for f, _ in ss.PoolDesc._fields_])
        st = lib.ss_state_pool_create(ctypes.byref(desc), None, None, ctypes.byref(out))
        assert st == expect, (over, st, lib.ss_last_error())
        assert not out.value
    # unsorted sigma and a bad CSR are rejected on the host too
    import numpy as np
    d = dict(base)
    desc = ss.PoolDesc(*[d[f] for f, _ in ss.PoolDesc._fields_])
    off = np.array([0, 2, 2, 2, 2], np.int64)
    u = np.zeros((2, 16), np.float32)
    v = np.zeros((2, 32), np.float32)
    for sig, expect in [(np.array([0.1, 0.5], np.float32), ss.SS_ERR_ARG), (np.array([1, np.nan], np.float32),
                                                                             ss.SS_ERR_ARG)]:
        init = ss.Init(off.ctypes.data_as(ss._c_i64p), u.ctypes.data_as(ss._c_f32p), v.ctypes.data_as(ss._c_f32p),
                       sig.ctypes.data_as(ss._c_f32p))
        assert lib.ss_state_pool_create(ctypes.byref(desc), ctypes.byref(init), None, ctypes.byref(out)) == expect


def test_calls_on_null_pool_are_rejected(lib):
    from rank_recurrent_state_amd import sinkstate as ss
    assert lib.ss_decode_step(None, None, None, None, None, None, None, None) == ss.SS_ERR_ARG
    assert lib.ss_readout(None, None, None, None) == ss.SS_ERR_ARG
    assert lib.ss_compact(None, 0, None) == ss.SS_ERR_ARG
    assert lib.ss_pool_stats(None, None, None) == ss.SS_ERR_ARG
    n = ctypes.c_size_t()
    assert lib.ss_state_export(None, None, 0, None, 0, ctypes.byref(n), None) == ss.SS_ERR_ARG
    assert lib.ss_state_pool_destroy(None) == ss.SS_OK
    out = ctypes.c_void_p()
    assert lib.ss_step_graph_create(None, None, None, None, None, None, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert lib.ss_step_graph_create(None, None, None, None, None, None, None, None) == ss.SS_ERR_ARG
    assert lib.ss_step_graph_launch(None, 0, None) == ss.SS_ERR_ARG
    assert lib.ss_step_graph_destroy(None) == ss.SS_OK
    assert lib.ss_consolidate(None, 0, None) == ss.SS_ERR_ARG
    assert lib.ss_compact_ids(None, None, 0, None) == ss.SS_ERR_ARG
    g = ctypes.c_int32()
    assert lib.ss_consolidate_async(None, 0, None, None, ctypes.byref(g)) == ss.SS_ERR_ARG
    assert lib.ss_consolidate_poll(None, 0, None, ctypes.byref(g)) == ss.SS_ERR_ARG
    n32 = ctypes.c_int32(7)
    assert lib.ss_consolidate_next(None, 1, None, ctypes.byref(n32), None) == ss.SS_ERR_ARG
    assert n32.value == 7
    assert lib.ss_consolidate_next(None, 1, None, None, None) == ss.SS_ERR_ARG


def test_dense_rank_limit_pins(lib):
    g = json.load(open(os.path.join(GOLD, "memory_arithmetic.json")))
    assert lib.ss_dense_rank_limit(128, 128) == g["threshold_128x128"]
    assert lib.ss_dense_rank_limit(128, 80) == lib.ss_dense_rank_limit(80, 128) == 49
    assert lib.ss_dense_rank_limit(16, 32) == 10


def test_decode_byte_formula(lib):
    """Algorithmic bytes: rank 8 with a half-full pad on 128x80 is the 12,126 B of the plan
    (which counts Gamma as two 4-byte accesses) with the 16-byte record read and written instead."""
    f = lib.ss_decode_bytes_per_state
    FAC, BUF, PLAIN = 0, 1, 2
    avg = (f(128, 80, 8, 8, 3, 0, FAC) + f(128, 80, 8, 8, 4, 0, FAC)) / 2
    assert avg == 12126 - 8 + 32
    # a factored rank-r state with n slots reads (r + n) components of d_k + d_v + 1 floats
    assert f(128, 80, 8, 9, 0, 0, FAC) - f(128, 80, 8, 8, 0, 0, FAC) == 4 * (128 + 80 + 1)
    assert f(128, 80, 8, 8, 0, 1, FAC) - f(128, 80, 8, 8, 0, 0, FAC) == 4        # beta
    # plain dense (the baseline): the state read and written
    inputs = 4 * (2 * 128 + 80 + 1)
    assert f(128, 80, 8, 0, 0, 0, PLAIN) == 16 + 2 * 4 * 128 * 80 + inputs + 4 * 80
    # buffered dense: H read, the pad read, one slot written; the step that fills the pad writes H
    comp = 4 * (128 + 80 + 1)
    assert f(128, 80, 8, 0, 3, 0, BUF) == 32 + 4 * 128 * 80 + 3 * comp + inputs + 4 * 80 + comp
    assert f(128, 80, 8, 0, 7, 0, BUF) == 32 + 4 * 128 * 80 + 7 * comp + inputs + 4 * 80 + 4 * 128 * 80
    # fp16 factors: a stored component is 2 (d_k + d_v) + 4 bytes, a pad slot stays 4 (d_k + d_v + 1)
    H16 = 3
    assert f(128, 80, 8, 9, 0, 0, H16) - f(128, 80, 8, 8, 0, 0, H16) == 2 * (128 + 80) + 4
    assert f(128, 80, 8, 8, 4, 0, H16) - f(128, 80, 8, 8, 3, 0, H16) == comp
    assert f(128, 80, 8, 8, 3, 0, FAC) - f(128, 80, 8, 8, 3, 0, H16) == 8 * 2 * (128 + 80)
    assert f(128, 80, 8, 0, 0, 0, 4) == 0 and f(128, 80, 8, 0, 0, 0, -1) == 0
    # page-printed footprint: rank-8 factors + a full pad of one 80x128 state = 13,376 B
    g = json.load(open(os.path.join(GOLD, "memory_arithmetic.json")))
    assert 2 * 8 * 4 * (128 + 80 + 1) == g["total_bytes"]


def test_rsvd_init_rejects_bad_arguments_without_touching_the_gpu(lib):
    from rank_recurrent_state_amd import sinkstate as ss
    vp = ctypes.c_void_p(1)  # never dereferenced: every case fails the host-side checks first
    base = dict(n=4, d_k=16, d_v=16, block=4, n_blocks=2, iters=2, max_rank=8)
    cases = [({"n": -1}, ss.SS_ERR_ARG), ({"d_k": 18}, ss.SS_ERR_SHAPE), ({"d_v": 260}, ss.SS_ERR_SHAPE),
             ({"block": 0}, ss.SS_ERR_SHAPE), ({"block": 17}, ss.SS_ERR_SHAPE),
             ({"block": 8, "d_k": 4}, ss.SS_ERR_SHAPE), ({"n_blocks": 0}, ss.SS_ERR_ARG),
             ({"iters": 0}, ss.SS_ERR_ARG), ({"iters": 65}, ss.SS_ERR_ARG), ({"max_rank": 0}, ss.SS_ERR_ARG),
             ({"max_rank": 9}, ss.SS_ERR_ARG), ({"max_rank": 17, "n_blocks": 8}, ss.SS_ERR_ARG)]
    for over, expect in cases:
        d = dict(base, **over)
        st = lib.ss_rsvd_init(vp, d["n"], d["d_k"], d["d_v"], d["block"], d["n_blocks"], d["iters"], vp, vp,
                              d["max_rank"], vp, vp, vp, vp, vp, None)
        assert st == expect, (over, st, lib.ss_last_error())
    d = base
    assert lib.ss_rsvd_init(None, 4, 16, 16, 4, 2, 2, None, None, 8, None, None, None, None, None, None) == ss.SS_ERR_ARG
    assert lib.ss_rsvd_init(None, 0, 16, 16, 4, 2, 2, None, None, 8, None, None, None, None, None, None) == ss.SS_OK


def test_rsvd_init_noalloc_checks_without_touching_the_gpu(lib):
    """The allocation-free initialization checks its arguments like ss_rsvd_init and rejects a batch
    larger than its fixed 32 MiB workspace before any HIP call; states whose residual fits the LDS
    need no workspace, so their batch size is not limited by it."""
    from rank_recurrent_state_amd import sinkstate as ss
    vp = ctypes.c_void_p(1)  # never dereferenced: every case fails the host-side checks first
    f = lib.ss_rsvd_init_noalloc
    assert f(vp, -1, 16, 16, 4, 2, 2, vp, vp, 8, vp, vp, vp, vp, None) == ss.SS_ERR_ARG
    assert f(vp, 4, 18, 16, 4, 2, 2, vp, vp, 8, vp, vp, vp, vp, None) == ss.SS_ERR_SHAPE
    assert f(vp, 4, 16, 16, 4, 2, 2, vp, vp, 9, vp, vp, vp, vp, None) == ss.SS_ERR_ARG
    assert f(None, 4, 16, 16, 4, 2, 2, None, None, 8, None, None, None, None, None) == ss.SS_ERR_ARG
    assert f(None, 0, 16, 16, 4, 2, 2, None, None, 8, None, None, None, None, None) == ss.SS_OK
    # 256 x 128 needs the workspace: 257 states are 8,421,376 floats, one more than fits
    assert f(vp, 257, 256, 128, 8, 2, 2, vp, vp, 16, vp, vp, vp, vp, None) == ss.SS_ERR_CAPACITY
    assert b"32 MiB" in lib.ss_last_error()
    # 128 x 80 fits the LDS: a large batch passes the capacity check and stops at the null pointer
    assert f(None, 10**6, 128, 80, 8, 2, 2, vp, vp, 16, vp, vp, vp, vp, None) == ss.SS_ERR_ARG


def test_create_from_dense_rejects_bad_arguments_without_touching_the_gpu(lib):
    from rank_recurrent_state_amd import sinkstate as ss
    vp = ctypes.c_void_p(1)  # never dereferenced: every case fails the host-side checks first
    out = ctypes.c_void_p()
    desc, keep, _ = ss._desc(16, 16, 32, 8, 8, -1, True, 0, False, None, None, None, None, 1e-3, 0, 0, False, False)
    f = lib.ss_state_pool_create_from_dense
    assert f(None, vp, vp, vp, vp, vp, 8, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert f(ctypes.byref(desc), vp, vp, vp, vp, vp, 8, None, None) == ss.SS_ERR_ARG
    assert f(ctypes.byref(desc), vp, vp, vp, vp, vp, 0, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert f(ctypes.byref(desc), vp, vp, vp, vp, vp, 17, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert f(ctypes.byref(desc), vp, None, vp, vp, vp, 8, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    bad, keep2, _ = ss._desc(16, 18, 32, 8, 8, -1, True, 0, False, None, None, None, None, 1e-3, 0, 0, False, False)
    assert f(ctypes.byref(bad), vp, vp, vp, vp, vp, 8, None, ctypes.byref(out)) == ss.SS_ERR_SHAPE
    fd, keep3, _ = ss._desc(16, 16, 32, 8, 8, -1, True, 0, True, None, None, None, None, 1e-3, 0, 0, False, False)
    assert f(ctypes.byref(fd), vp, vp, vp, vp, vp, 8, None, ctypes.byref(out)) == ss.SS_ERR_ARG
    assert not out.value


def test_create_rejects_bad_dense_given_states(lib):
    import numpy as np
    from rank_recurrent_state_amd import sinkstate as ss
    out = ctypes.c_void_p()
    desc = ss.PoolDesc(4, 16, 16, 8, 8, -1, 1, 0, 0, 1, None, None, None, None, 1e-3, 0, 0)
    off = np.array([0, 2, 2, 2, 2], np.int64)
    u = np.zeros((2, 16), np.float32)
    sig = np.array([1.0, 0.5], np.float32)
    mask = np.array([1, 0, 0, 0], np.uint8)  # state 0 has components: rejected
    S = np.zeros((4, 16, 16), np.float32)
    init = ss.Init(off.ctypes.data_as(ss._c_i64p), u.ctypes.data_as(ss._c_f32p), u.ctypes.data_as(ss._c_f32p),
                   sig.ctypes.data_as(ss._c_f32p), mask.ctypes.data_as(ss._c_u8p), S.ctypes.data_as(ss._c_f32p))
    assert lib.ss_state_pool_create(ctypes.byref(desc), ctypes.byref(init), None, ctypes.byref(out)) == ss.SS_ERR_ARG
    mask2 = np.array([0, 1, 0, 0], np.uint8)  # a masked state without `dense`: rejected
    init2 = ss.Init(off.ctypes.data_as(ss._c_i64p), u.ctypes.data_as(ss._c_f32p), u.ctypes.data_as(ss._c_f32p),
                    sig.ctypes.data_as(ss._c_f32p), mask2.ctypes.data_as(ss._c_u8p), None)
    assert lib.ss_state_pool_create(ctypes.byref(desc), ctypes.byref(init2), None, ctypes.byref(out)) == ss.SS_ERR_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every entry point raises: there is no CPU path to fall back on."""
    from rank_recurrent_state_amd import sinkstate
    monkeypatch.setattr(sinkstate, "LIB_PATH", str(tmp_path / "libsinkstate.so"))
    monkeypatch.setattr(sinkstate, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        sinkstate.load_library()
    with pytest.raises(RuntimeError, match="missing"):
        sinkstate.state_pool_create(4, 16, 32, 8, 2)


def test_product_path_does_not_reach_the_oracle():
    """The package and the binding import nothing from the oracle, and bench.py touches it only in
    its CPU-baseline leg."""
    pkg = os.path.join(ROOT, "rank_recurrent_state_amd")
    pat = re.compile(r"^\s*(import|from)\s+\S*oracle", re.M)
    for name in sorted(os.listdir(pkg)):
        if name.endswith(".py"):
            assert not pat.search(open(os.path.join(pkg, name)).read()), name
    for src in ("ss_pool.cpp", "ss_decode.hip", "ss_compact.hip", "ss_consolidate.hip", "ss_init.hip"):
        text = open(os.path.join(pkg, "csrc", src)).read()
        assert "orc_" not in text and "oracle" not in text.lower(), src
    bench = open(os.path.join(ROOT, "bench.py")).read()
    uses = [m.start() for m in re.finditer(r"\boracle\b", bench)]
    fn = re.search(r"def cpu_baseline\b.*?(?=\ndef |\Z)", bench, re.S)
    assert fn is not None
    for u in uses:
        line = bench[bench.rfind("\n", 0, u) + 1:bench.find("\n", u)]
        if line.lstrip().startswith("#") or "\"" in line or "'" in line:
            continue  # comments and strings
        assert fn.start() <= u < fn.end(), line


def test_pool_close_destroys_its_step_graphs_first(monkeypatch):
    """A step graph must be destroyed before its pool: closing the pool closes its live graphs
    first, and a closed graph refuses to launch instead of handing the library a dangling handle
    (a stand-in library records the calls; no GPU involved)."""
    import types
    from rank_recurrent_state_amd import sinkstate as ss
    calls = []

    class Lib:
        def ss_step_graph_create(self, pool, *args):
            args[-1]._obj.value = 0x20
            calls.append(("create", pool))
            return 0

        def ss_step_graph_launch(self, h, step, stream):
            calls.append(("launch", h.value, step))
            return 0

        def ss_step_graph_destroy(self, h):
            calls.append(("graph_destroy", h.value))
            return 0

        def ss_state_pool_destroy(self, h):
            calls.append(("pool_destroy", h))
            return 0

    monkeypatch.setattr(ss, "_lib", Lib())
    stream = types.SimpleNamespace(cuda_stream=0)
    pool = ss.StatePool(0x10, 4, 16, 32, 8, 2, 1, False)
    g = ss.StepGraph(pool, None, None, None, None, None, None)
    g.launch(3, stream=stream)
    pool.close()
    assert calls == [("create", 0x10), ("launch", 0x20, 3), ("graph_destroy", 0x20), ("pool_destroy", 0x10)]
    with pytest.raises(ss.SinkStateError):
        g.launch(4, stream=stream)
    g.close()
    pool.close()
    assert len(calls) == 4

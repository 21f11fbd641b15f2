"""Pins for the oracle's fp16 factor storage (CPU only).

Shallow Encoding Emits Deep Memories, section 6: factors stored in fp16 and
quantized when a compression writes them, with the newest (buffered) columns
kept in fp32.  The oracle rounds every factor vector it writes (initial
factors, compaction results, consolidation results) to binary16, nearest with
ties to even; sigma and the pad stay in full precision.  Pinned against
numpy's float16 conversion and against the error such a rounding can make.
"""
import numpy as np
import pytest

from oracle import OraclePool
from oracle.oracle import OracleState, round_fp16


def test_round_fp16_matches_numpy_float16():
    rng = np.random.default_rng(0)
    scales = rng.choice([1e-8, 1e-6, 1e-4, 1e-2, 1.0, 10.0, 1000.0], 5000)
    xs = np.concatenate([rng.standard_normal(5000) * scales,
                         [0.0, 65504.0, 65519.99, 1e-9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
                          1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2049.0, 2051.0, -0.1, 0.1]])
    for x in xs:
        assert round_fp16(x) == float(np.float16(x)), x
    assert np.isinf(round_fp16(65520.0)) and np.isinf(round_fp16(-1e6))
    # ties go to even: 1 + 2^-11 lies halfway between 1 and 1 + 2^-10
    assert round_fp16(1 + 2.0 ** -11) == 1.0 and round_fp16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9


def _drive(P, rng, N, d_k, d_v, K, steps, rule):
    outs = []
    for t in range(1, steps + 1):
        q = rng.standard_normal((N, d_k))
        k = rng.standard_normal((N, d_k))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        v = rng.standard_normal((N, d_v))
        a = rng.uniform(0.9, 1.0, N)
        b = 1 / (1 + np.exp(-rng.standard_normal(N))) if rule else None
        outs.append(P.decode(q, k, v, a, b))
        if t % K == 0:
            P.compact()
    return outs


@pytest.mark.parametrize("rule", [0, 1])
def test_fp16_factors_are_representable_and_sigma_is_not_rounded(rule):
    rng = np.random.default_rng(3 + rule)
    N, d_k, d_v, K, r = 6, 16, 24, 4, 3
    P = OraclePool(N, d_k, d_v, K=K, r=r, promote=False, factor_fp16=True)
    for s in range(N):
        P.set_state(s, OracleState(rule=rule, eps=1e-3))
    _drive(P, rng, N, d_k, d_v, K, 24, rule)
    P.consolidate()
    n_sig_unrounded = 0
    for s in range(N):
        st = P.get_state(s)
        assert len(st.sigma) > r
        for A in (st.U, st.V):
            assert all(x == round_fp16(x) for x in A.ravel())
        n_sig_unrounded += sum(x != round_fp16(x) for x in st.sigma)
    assert n_sig_unrounded > 0


@pytest.mark.parametrize("rule", [0, 1])
def test_fp16_run_stays_within_the_rounding_bound_of_the_fp32_run(rule):
    """Same inputs into an fp32-factor and an fp16-factor oracle pool, compacting together.  Each
    factor entry moves by at most 2^-11 of itself when it is written, so one compaction moves
    a state by at most about 2^-10 sum(sigma); the gap between the two runs must stay at that
    scale over 32 steps (8 compactions), and must not be zero."""
    N, d_k, d_v, K, r = 6, 16, 24, 4, 3
    P32 = OraclePool(N, d_k, d_v, K=K, r=r, promote=False)
    P16 = OraclePool(N, d_k, d_v, K=K, r=r, promote=False, factor_fp16=True)
    for P in (P32, P16):
        for s in range(N):
            P.set_state(s, OracleState(rule=rule, eps=1e-3))
    o32 = _drive(P32, np.random.default_rng(7), N, d_k, d_v, K, 32, rule)
    o16 = _drive(P16, np.random.default_rng(7), N, d_k, d_v, K, 32, rule)
    worst = 0.0
    for s in range(N):
        S32, S16 = P32.reconstruct(s), P16.reconstruct(s)
        ssum = P32.get_state(s).sigma.sum()
        worst = max(worst, np.linalg.norm(S16 - S32) / (2.0 ** -10 * ssum))
    assert 0.0 < worst <= 8.0, worst  # at most 8 compactions' worth of rounding
    d = max(np.max(np.abs(a - b)) / np.max(np.abs(a)) for a, b in zip(o32, o16))
    assert 0.0 < d < 1e-2


def test_fp16_initial_factors_are_rounded_and_fp32_pools_are_not():
    rng = np.random.default_rng(5)
    U = rng.standard_normal((3, 8))
    V = rng.standard_normal((3, 12))
    st = OracleState(U, V, np.array([3.0, 2.0, 1.0]), rule=0, eps=0.0)
    P16 = OraclePool(1, 8, 12, K=4, r=2, promote=False, factor_fp16=True)
    P32 = OraclePool(1, 8, 12, K=4, r=2, promote=False)
    P16.set_state(0, st)
    P32.set_state(0, st)
    assert np.array_equal(P16.get_state(0).U, np.float16(U).astype(np.float64))
    assert np.array_equal(P32.get_state(0).U, U)


def test_fp16_with_channel_decay_rounds_at_compaction_only():
    """Per-channel decay with fp16 factors: between compactions the stored u carry the decays
    applied since the last one (not fp16 values); right after a compaction every factor is an
    fp16 value again, and the run stays within the rounding bound of the fp32 run."""
    N, d_k, d_v, K, r = 5, 16, 12, 4, 3
    P32 = OraclePool(N, d_k, d_v, K=K, r=r, promote=False, diag_decay=True)
    P16 = OraclePool(N, d_k, d_v, K=K, r=r, promote=False, factor_fp16=True, diag_decay=True)
    for P in (P32, P16):
        for s in range(N):
            P.set_state(s, OracleState(rule=1, eps=1e-3))
    rng = np.random.default_rng(11)
    mid_rounded = True
    for t in range(1, 25):
        q = rng.standard_normal((N, d_k))
        k = rng.standard_normal((N, d_k))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        v = rng.standard_normal((N, d_v))
        lam = rng.uniform(0.7, 1.0, (N, d_k))
        b = 1 / (1 + np.exp(-rng.standard_normal(N)))
        for P in (P32, P16):
            P.decode(q, k, v, lam, b)
        if t % K == 0:
            for P in (P32, P16):
                P.compact()
            for s in range(N):
                st = P16.get_state(s)
                for A in (st.U, st.V):
                    assert all(x == round_fp16(x) for x in A.ravel())
        elif t > K:
            st = P16.get_state(0)
            mid_rounded = mid_rounded and all(x == round_fp16(x) for x in st.U.ravel())
    assert not mid_rounded  # decayed u are not fp16 values until the next compaction
    worst = 0.0
    for s in range(N):
        S32, S16 = P32.reconstruct(s), P16.reconstruct(s)
        worst = max(worst, np.linalg.norm(S16 - S32) / (2.0 ** -10 * P32.get_state(s).sigma.sum()))
    assert 0.0 < worst <= 8.0, worst


def test_mid_run_load_keeps_values_as_given():
    """A mid-run state (as_init=False) is loaded as given; only initial factors are rounded."""
    rng = np.random.default_rng(12)
    U = rng.standard_normal((2, 8)) * np.array([[0.3], [0.7]])
    V = rng.standard_normal((2, 6))
    st = OracleState(U, V, np.array([2.0, 1.0]), rule=0, eps=0.0)
    P = OraclePool(1, 8, 6, K=4, r=2, promote=False, factor_fp16=True)
    P.set_state(0, st, as_init=False)
    assert np.array_equal(P.get_state(0).U, U)
    P.set_state(0, st)
    assert np.array_equal(P.get_state(0).U, np.float16(U).astype(np.float64))

"""The host arithmetic of the host-core consolidation (SinkState 4.3, Figure 7(a)), on the CPU:
the exact SVD of a frozen part, truncated at eps * sigma_0, against LAPACK's SVD of the dense
frozen matrix (numpy), on frozen parts with clusters of near-duplicate directions."""
import numpy as np
import pytest

from rank_recurrent_state_amd import sinkstate as ss


def _unit(rng, d, n):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


@pytest.mark.parametrize("dk,dv,f,seed", [(128, 80, 40, 1), (128, 128, 44, 2), (16, 32, 20, 3), (80, 128, 12, 4),
                                          (8, 4, 10, 5)])
def test_host_consolidation_is_the_truncated_svd(dk, dv, f, seed):
    rng = np.random.default_rng(seed)
    # clusters of near-duplicate directions, as frozen tails pile up
    base_u, base_v = _unit(rng, dk, max(1, f // 4)), _unit(rng, dv, max(1, f // 4))
    pick = rng.integers(0, len(base_u), f)
    u = base_u[pick] + 0.05 * rng.standard_normal((f, dk))
    v = base_v[pick] + 0.05 * rng.standard_normal((f, dv))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    sig = np.sort(np.exp(rng.uniform(np.log(1e-3), 0.0, f)))[::-1]
    u32, v32, s32 = u.astype(np.float32), v.astype(np.float32), sig.astype(np.float32)
    F = (u32.T.astype(np.float64) * s32) @ v32.astype(np.float64)
    s0, eps = 2.0, 1e-2
    U2, V2, S2 = ss.host_consolidate_frozen(u32, v32, s32, s0, eps)
    ref = np.linalg.svd(F, compute_uv=False)
    keep = ref[(ref >= eps * s0) & (ref > 0)]
    assert len(S2) == len(keep)
    assert np.all(np.diff(S2) <= 0)
    assert np.allclose(S2, keep, rtol=1e-5, atol=1e-7 * ref[0])
    assert np.abs(U2.astype(np.float64) @ U2.T - np.eye(len(S2))).max() <= 1e-5
    assert np.abs(V2.astype(np.float64) @ V2.T - np.eye(len(S2))).max() <= 1e-5
    # the state moves by exactly the dropped values (Eckart-Young), up to fp32 storage
    F2 = (U2.T.astype(np.float64) * S2) @ V2.astype(np.float64)
    dropped = np.sqrt(np.sum(ref[len(keep):] ** 2))
    assert abs(np.linalg.norm(F - F2) - dropped) <= 1e-5 * np.linalg.norm(F) + 1e-6


def test_host_consolidation_edge_cases():
    rng = np.random.default_rng(9)
    # a duplicated direction merges into one component of the summed value
    u = _unit(rng, 12, 1)
    v = _unit(rng, 9, 1)
    U2, V2, S2 = ss.host_consolidate_frozen(np.vstack([u, u]), np.vstack([v, v]), [0.7, 0.2], 1.0, 1e-3)
    assert len(S2) == 1 and abs(S2[0] - 0.9) <= 1e-6
    # and a reversed one into the difference
    U2, V2, S2 = ss.host_consolidate_frozen(np.vstack([u, u]), np.vstack([v, -v]), [0.7, 0.2], 1.0, 1e-3)
    assert len(S2) == 1 and abs(S2[0] - 0.5) <= 1e-6
    # everything below the threshold: nothing is kept
    U2, V2, S2 = ss.host_consolidate_frozen(_unit(rng, 12, 3), _unit(rng, 9, 3), [1e-3, 5e-4, 1e-4], 1.0, 1e-2)
    assert len(S2) == 0
    # no component at all
    U2, V2, S2 = ss.host_consolidate_frozen(np.zeros((0, 12)), np.zeros((0, 9)), np.zeros(0), 1.0, 1e-2)
    assert len(S2) == 0

"""ss_rsvd_init_noalloc (the initialization entry point that allocates nothing) against
ss_rsvd_init with a caller's workspace: the same kernel on the same inputs must give the same
ranks, singular values and factors, bit for bit, on two calls in a row (the second smaller, so
that it runs over what the first left in the library's fixed workspace), for a shape whose
residual needs the workspace (256 x 128) and one that fits the kernel's LDS (128 x 80)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss


def _states(rng, n, dk, dv, rank):
    U = np.linalg.qr(rng.standard_normal((n, dk, rank)))[0]
    V = np.linalg.qr(rng.standard_normal((n, dv, rank)))[0]
    sig = np.logspace(0, -3, rank)
    S = np.einsum("nir,r,njr->nij", U, sig, V) + 1e-4 * rng.standard_normal((n, dk, dv))
    return torch.tensor(S, dtype=torch.float32, device="cuda")


def _both(S, omega, eps, iters, max_rank):
    n, dk, dv = S.shape
    u_ref, v_ref, s_ref, r_ref = ss.rsvd_init(S, omega, eps, iters=iters, max_rank=max_rank)
    u = torch.full((n, max_rank, dk), float("nan"), device="cuda")
    v = torch.full((n, max_rank, dv), float("nan"), device="cuda")
    sg = torch.full((n, max_rank), float("nan"), device="cuda")
    rk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    ss.rsvd_init_noalloc(S, omega, eps, u, v, sg, rk, iters=iters)
    torch.cuda.synchronize()
    r_ref, rk = r_ref.cpu().numpy(), rk.cpu().numpy()
    assert np.array_equal(rk, r_ref)
    assert rk.min() >= 1
    for t, (a, b) in enumerate(((u, u_ref), (v, v_ref), (sg, s_ref))):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        for i in range(n):  # entries past a state's rank are unspecified
            assert np.array_equal(a[i, :rk[i]], b[i, :rk[i]]), (t, i)
    return rk


@pytest.mark.parametrize("dk,dv", [(256, 128), (128, 80)])
def test_noalloc_matches_workspace_entry_point(dk, dv):
    rng = np.random.default_rng(7 + dk)
    block, nb, iters, max_rank = 8, 3, 2, 24
    for n, rank in ((40, 20), (13, 11)):  # second call smaller, over the first call's workspace contents
        S = _states(rng, n, dk, dv, rank)
        omega = torch.tensor(rng.standard_normal((n, nb, dk, block)), dtype=torch.float32, device="cuda")
        eps = torch.full((n,), 1e-2, dtype=torch.float32, device="cuda")
        rk = _both(S, omega, eps, iters, max_rank)
        print(dk, dv, n, "ranks", rk.min(), rk.max())


def test_noalloc_rejects_sizes_beyond_its_workspace():
    n, dk, dv = 300, 256, 128  # 9.8 M floats > 8,388,608
    S = torch.zeros(1, device="cuda")
    with pytest.raises(ss.SinkStateError) as e:
        lib = ss.load_library()
        import ctypes
        p = ctypes.c_void_p(S.data_ptr())
        ss._check(lib.ss_rsvd_init_noalloc(p, n, dk, dv, 8, 2, 2, p, p, 16, p, p, p, p, None))
    assert e.value.status == ss.SS_ERR_CAPACITY

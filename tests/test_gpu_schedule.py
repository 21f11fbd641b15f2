"""The GPU pool's compaction schedule against the oracle's (SinkState 4.2 "Staggered compaction":
a group with offset o compacts after step t when (t + o) mod K == 0).

The free-running and lock-step parity tests hand the library's schedule to the oracle, so a wrong
schedule there would be mirrored rather than caught; here the two are computed independently
from each workload's own group offsets and compared over 4,096 steps."""
import numpy as np
import pytest
import torch

from oracle import schedule_due as orc_schedule_due

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from rank_recurrent_state_amd import sinkstate as ss
    from rank_recurrent_state_amd import workloads as W


@pytest.mark.parametrize("name", ["tiny", "mamba2_258k", "gdn_delta", "mixed_dense", "mamba2_1m", "kda_delta"])
def test_schedule_matches_oracle(name):
    w = W.get(name, n_requests=1)
    init = W.initial_state(w)
    g, offs = W.groups(w)
    assert np.array_equal(g, init["group_of_state"]) and np.array_equal(offs, init["group_offset"])
    pool = ss.state_pool_create(w.n_states, w.d_k, w.d_v, w.K, w.r, group_of_state=init["group_of_state"],
                                group_offset=init["group_offset"], rule=init["rule"], eps=init["eps"],
                                comp_off=init["comp_off"], u=init["u"], v=init["v"], sigma=init["sigma"],
                                diag_decay=w.diag_decay)
    try:
        per_step = []
        for t in range(0, 4097):
            got = sorted(ss.schedule_due(pool, t))
            want = sorted(int(x) for x in orc_schedule_due(t, w.K, offs))
            assert got == want, (name, t, got, want)
            per_step.append(len(got))
        # every group falls due exactly once per K steps
        assert sum(per_step[1:w.K + 1]) == len(offs)
    finally:
        pool.close()

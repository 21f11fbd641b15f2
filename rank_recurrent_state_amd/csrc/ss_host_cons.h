// ss_host_cons.h -- host-core consolidation of frozen parts (ss_host_cons.cpp).
#pragma once
#include <stdint.h>

namespace ss {

// Exact fp64 SVD of the frozen part of one state, f fp32 components u [f][d_k], v [f][d_v],
// s [f], truncated at eps * s0; the kept components (descending) overwrite the first rows.
// Returns the kept count (<= f).
int host_consolidate_one(int dk, int dv, int f, float *u, float *v, float *s, float s0, float eps);

// host_consolidate_one over n states laid out [n][fmax] rows, cnt[i] components each (0: skipped),
// on `threads` host threads; cnt receives the kept counts.
void host_consolidate_batch(int n, int dk, int dv, int fmax, float *u, float *v, float *s, int32_t *cnt,
                            const float *s0, const float *eps, int threads);

}  // namespace ss

/*
 * sinkstate.h -- C-ABI of libsinkstate.so: a pool of linear-attention
 * recurrent states held in factored (low-rank) form on one AMD Instinct
 * MI355X (gfx950), with buffered decode, factored readout, Brand-style
 * compaction and a dense fallback.
 *
 * The operations follow "SinkState: On-the-Fly SVD of Recurrent States for
 * Efficient Hybrid LLM Serving" (arXiv 2611.14246), cited below as [SS], and
 * the gated delta rule as written in "Shallow Encoding Emits Deep Memories"
 * (arXiv 2611.06084) section 2, eq. (2), cited as [SEED].
 *
 * Orientation.  A state is S (d_k x d_v) with o = S^T q.  [SS] 2.1 writes the
 * transpose H = S^T (d_v x d_k); the two are the same object.  Factored form:
 *   S = Gamma * ( sum_i sigma_i u_i v_i^T  +  sum_j c_j k_j w_j^T )
 * where (u_i in R^{d_k}, v_i in R^{d_v}, sigma_i) are the components ([SS]
 * 3.2 Design 1: the first min(r, R) by sigma are "active", the rest
 * "frozen"), (k_j, w_j, c_j) are the pad slots ([SS] 4.2 "(i) Buffering"),
 * and Gamma is the decay accumulated since the last compaction ([SS] 4.4:
 * the decode kernel scales by the decay accumulated since the last compaction).
 *
 * Conventions for every entry point:
 *  - Every call returns ss_status.  Argument and shape checks run on the host
 *    before any HIP call; a failing check changes nothing.
 *  - Device pointers (q, k, v, alpha, beta, o) are caller-owned fp32 device
 *    memory, contiguous, row-major [n_states][d]; they must stay valid until
 *    the enqueued work completes.  Host pointers are only read during the call.
 *  - All device work is enqueued on the given stream (NULL = the null stream);
 *    calls return without waiting unless stated.  A pool is used by one stream
 *    at a time and is not reentrant.
 *  - A failure detected by a kernel (capacity exhausted, pad overflow) is
 *    sticky: the pool records it and every later call returns it.
 *  - ss_last_error() returns a thread-local message for the last failure.
 *  - No C++ exception crosses the ABI.
 */
#ifndef SINKSTATE_H_
#define SINKSTATE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SS_OK = 0,
  SS_ERR_ARG = 1,      /* NULL pointer, bad enum, negative size */
  SS_ERR_SHAPE = 2,    /* unsupported d_k / d_v / K / r combination */
  SS_ERR_OOM = 3,      /* device or host allocation failed */
  SS_ERR_CAPACITY = 4, /* a region of the pool is full */
  SS_ERR_HIP = 5,      /* a HIP runtime call failed */
  SS_ERR_STATE = 6     /* the pool is poisoned by an earlier kernel-side failure */
} ss_status;

/* Update rule of a state ([SS] 4.2, "the same procedure also applies to GDN").
 *  SCALAR (Mamba-2):       S_t = alpha S_{t-1} + k v^T                ([SS] 2.1)
 *  DELTA  (Gated DeltaNet): S_t = alpha (I - beta k k^T) S_{t-1} + beta k v^T
 *                          = alpha S_{t-1} + k w^T,  w = beta (v - alpha S_{t-1}^T k)
 *                          ([SEED] eq. (2) with g = alpha), S_{t-1}^T k read
 *                          from the factors. */
typedef enum { SS_RULE_SCALAR = 0, SS_RULE_DELTA = 1 } ss_rule;

typedef struct ss_pool ss_pool; /* opaque; owns all of its device memory */

typedef struct {
  int64_t n_states;           /* N >= 1 */
  int32_t d_k, d_v;           /* each a multiple of 4, 4..256 */
  int32_t pad_slots;          /* K, 1..8 ([SS] 5.1 uses 8) */
  int32_t r_active;           /* r, 1..8 ([SS] 5.1 uses 8); r + K <= 16 */
  int32_t dense_rank_limit;   /* L; < 0 selects floor(d_k d_v / (d_k + d_v)) ([SS] 4.4) */
  int32_t promote_on_compact; /* 1: re-apply the dense test after every compaction */
  int32_t max_frozen;         /* frozen components per state when promotion is off, 1..255; 0 = 255 */
  int32_t force_dense;        /* 1: every state is held dense (the dense baseline) */
  int32_t n_groups;           /* compaction groups (stagger groups), >= 1 */
  const int32_t *group_of_state; /* host [N] in [0, n_groups), or NULL: all in group 0 */
  const int32_t *group_offset;   /* host [n_groups] step offsets in [0, K), or NULL: all 0 */
  const uint8_t *rule;        /* host [N] ss_rule, or NULL: all SS_RULE_SCALAR */
  const float *eps;           /* host [N] truncation threshold eps >= 0, or NULL: eps_default */
  float eps_default;
  int64_t dense_capacity;     /* dense slots; 0 = N */
  int64_t arena_components;   /* initial capacity (components) of each component ring, at least
                                 what the initial data needs; 0 = automatic: the most the pool
                                 can ever need when that fits in a quarter of the free device
                                 memory, else a smaller start.  The rings grow on their own (see
                                 ss_compact); a growth is a device allocation. */
  int32_t factor_fp16;        /* 1: the component vectors u, v are stored in IEEE binary16
                                 ([SEED] 6 "Lower precision composes": fp16 factors, rounded
                                 when a compression writes them, while the newest columns, the
                                 pad, stay in fp32).  Rounding (to nearest, ties to even) happens
                                 when create stores the initial factors and whenever a
                                 compaction or a consolidation writes factors; sigma, the pad,
                                 the dense region and all arithmetic stay fp32, and the dense
                                 test keeps the same L.  A stored component then takes
                                 2 (d_k + d_v) + 4 bytes instead of 4 (d_k + d_v + 1).
                                 0: fp32 factors.  Other values: SS_ERR_ARG. */
  int32_t diag_decay;         /* 1: per-channel decay (Kimi Delta Attention; [SEED] appendix B.1
                                 eq. (6): Lambda_t = diag(lambda_1 .. lambda_{d_k}), one decay
                                 per key channel): ss_decode_step's alpha is [n_states][d_k]
                                 and a step is S_t = Lambda_t S_{t-1} + k w^T with
                                 w = beta (v - S_{t-1}^T Lambda_t k) (delta rule) or w = v.
                                 The pool keeps the decays accumulated since the last
                                 compaction per state and key channel (d_k floats per state,
                                 and per dense slot); a compaction folds them into the
                                 factors.  Consolidation is not available on such a pool
                                 (SS_ERR_ARG).  0: scalar decay, alpha is [n_states]. */
} ss_pool_desc;

/* Initial states, host memory, copied during create.  Components of state s
 * are rows comp_off[s] .. comp_off[s+1]-1 of u / v / sigma and must be sorted
 * by sigma, descending.  A state with more than L components is stored dense
 * ([SS] 4.4: the dense test is made once the initial factors exist).  The pad starts
 * empty and Gamma = 1.  A NULL ss_init (or NULL comp_off) creates empty
 * states (S = 0). */
typedef struct {
  const int64_t *comp_off; /* [N+1], comp_off[0] = 0 */
  const float *u;          /* [comp_off[N]][d_k] */
  const float *v;          /* [comp_off[N]][d_v] */
  const float *sigma;      /* [comp_off[N]] */
  const uint8_t *dense_mask; /* [N] or NULL: 1 = the state is given dense, in `dense`
                                (it must have no components in the CSR) */
  const float *dense;      /* [N][d_k][d_v] row-major S, read for the masked states only */
} ss_init;

/* kernels timed by ss_pool_timing */
enum {
  SS_KERNEL_DECODE_FACTORED = 0,
  SS_KERNEL_DECODE_DENSE = 1,
  SS_KERNEL_READOUT_FACTORED = 2,
  SS_KERNEL_READOUT_DENSE = 3,
  SS_KERNEL_COMPACT = 4,
  SS_KERNEL_MATERIALIZE = 5,
  SS_KERNEL_DENSE_FOLD = 6,
  SS_KERNEL_CONSOLIDATE = 7,
  SS_KERNEL_COUNT = 8
};

typedef struct {
  int64_t n_states, n_dense, n_factored;
  int64_t active_components, frozen_components, pad_entries;
  int64_t live_bytes;       /* bytes of live factors, pads, dense states and metadata */
  int64_t reserved_bytes;   /* device bytes held by the pool */
  int64_t max_rank;         /* largest components count of a factored state */
  int64_t rank_hist[65];    /* factored states by total components; [64] = 64 or more */
  int64_t decode_calls, compact_calls, readout_calls;
  uint64_t decode_bytes;    /* algorithmic bytes moved by all decode_step calls so far */
  uint64_t decode_bytes_factored; /* ... by the factored-state kernel */
  uint64_t decode_bytes_dense;    /* ... by the dense-region kernel */
  uint64_t compact_states;  /* states compacted (non-empty pad) so far */
  uint64_t compact_flops;   /* algorithmic flops of all compactions so far */
  int64_t promotions;       /* factored -> dense conversions after create */
  int64_t cap_truncations;  /* frozen components dropped because max_frozen was reached */
  int64_t ring_capacity[2]; /* component capacity of the active [0] and frozen [1] rings */
  int64_t ring_used[2];     /* ring span from the oldest live segment to the head */
  int64_t ring_head[2];     /* components allocated since the last re-pack (> capacity: wrapped) */
  int64_t ring_repacks;     /* re-packs (growth or defragmentation) so far */
  int64_t ring_syncs;       /* compactions that had to wait for the device to check ring room */
  double kernel_ms[SS_KERNEL_COUNT];       /* summed HIP-event durations while timing is on */
  int64_t kernel_launches[SS_KERNEL_COUNT];
  int64_t consolidate_calls;     /* group consolidations launched so far */
  uint64_t consolidate_states;   /* states whose frozen part was consolidated */
  uint64_t consolidate_flops;    /* algorithmic flops of those consolidations */
  uint64_t consolidate_removed;  /* frozen components they removed */
  int64_t jacobi_limit_hits;     /* compactions whose small SVD still rotated in its last allowed sweep */
} ss_stats;

/* Create a pool ([SS] 4.4 "Memory layout"): per state a 16-byte metadata
 * record; an active region and a separate frozen region of components, each
 * a ring in which every compaction group holds one exactly packed segment
 * (groups laid out in the order they fall due); a pad of K slots per state
 * kept apart from the factors; and a dense region.  Initial data is uploaded on `stream`, and
 * the call waits for it.  Errors: SS_ERR_ARG, SS_ERR_SHAPE, SS_ERR_OOM,
 * SS_ERR_HIP.  On success *out owns the pool; release it with
 * ss_state_pool_destroy. */
ss_status ss_state_pool_create(const ss_pool_desc *desc, const ss_init *init, hipStream_t stream, ss_pool **out);

/* Create a pool from dense states and their randomized block SVD ([SS] 4.2
 * "Randomized SVD initialization after prefill"; 4.4 "Memory layout": the
 * dense fallback is decided once a state has been factored).  S, u, v, sigma
 * and rank are device memory as ss_rsvd_init (or ss_rsvd_init_noalloc) with
 * the same max_rank reads and writes them: S [n_states][d_k][d_v], u
 * [n_states][max_rank][d_k], v [n_states][max_rank][d_v], sigma
 * [n_states][max_rank], rank [n_states].  The library reads the factors and
 * ranks back (the call synchronizes `stream`), keeps a state whose rank
 * exceeds L (desc->dense_rank_limit, or floor(d_k d_v / (d_k + d_v))) dense
 * as its exact S, read in place on the device, and gives every other state
 * its rank[s] components in descending sigma (the blocks are each
 * descending, not across blocks; equal values keep block order), first r
 * active, the rest frozen.  Then as ss_state_pool_create, whose desc fields
 * apply (force_dense is refused).  The caller keeps ownership of every
 * pointer; S may be freed once the call returns.  Errors: SS_ERR_ARG (also
 * for a rank outside [0, max_rank]), SS_ERR_SHAPE, SS_ERR_OOM, SS_ERR_CAPACITY,
 * SS_ERR_HIP. */
ss_status ss_state_pool_create_from_dense(const ss_pool_desc *desc, const float *S, const float *u, const float *v,
                                          const float *sigma, const int32_t *rank, int32_t max_rank,
                                          hipStream_t stream, ss_pool **out);

/* Waits for the pool's streams and frees all of its memory.  NULL is a no-op. */
ss_status ss_state_pool_destroy(ss_pool *pool);

/* One decode step of every state ([SS] 4.2 "(i) Buffering", 4.4 fused decode
 * kernel): Gamma <- alpha Gamma; w = v (scalar) or beta (v - alpha S_{t-1}^T k)
 * (delta); append (k, w, 1/Gamma) to the pad; o = S_t^T q, read after the
 * update.  States of the dense region are buffered the same way: the
 * region holds H = S^T and a pad, a step appends to the pad, and the step
 * that fills the pad folds it into H (exact algebra, no truncation).  In a
 * force_dense pool (the dense baseline) every step runs S <- alpha S + k w^T.
 * q, k: [N][d_k]; v, o: [N][d_v]; alpha: [N] in (0, 1] ([N][d_k] in a diag_decay pool); beta: [N], may be
 * NULL when no state uses the delta rule.  A factored state whose pad is
 * already full poisons the pool (SS_ERR_STATE on the next call): compact its
 * group first. */
ss_status ss_decode_step(ss_pool *pool, const float *q, const float *k, const float *v, const float *alpha,
                         const float *beta, float *o, hipStream_t stream);

/* Read-only readout o = S^T q of every state from factors, pad and dense
 * region, without changing the pool ([SS] 4.2 "(i) Buffering": the output is
 * computed from the extended factors; 4.4: no dense state is formed). */
ss_status ss_readout(ss_pool *pool, const float *q, float *o, hipStream_t stream);

/* Compact every state of compaction group `group` (or of all groups when
 * group < 0) whose pad is not empty ([SS] 4.2 "(ii) Top-subspace SVD" and
 * 3.2 Design 1): U_C = [U_active | pad keys], V_C = [V_active | pad w],
 * Sigma_C = Gamma diag(sigma_active, c); thin QR of both; SVD of the core
 * C = R_L Sigma_C R_R^T; rotate back; merge with the frozen components (whose
 * sigma are scaled by Gamma); drop sigma < eps * sigma_max; the first r of
 * the merged list become active, the rest frozen; the pad empties and Gamma
 * resets to 1.  The group's new components are allocated as one segment at
 * the head of each ring and its old segment is released.  Before that, the
 * host checks that the segment fits: it bounds each ring's usage without
 * waiting for the device and, only when the bound is too close to the
 * capacity, synchronizes `stream`, and re-packs the rings (growing them, a
 * device allocation, when the live components need it).  With
 * promote_on_compact, a state left with more than L components moves to the
 * dense region ([SS] 4.4).  Dense states of the group get a non-empty pad
 * folded into H.  A ring found full on the device (not expected: the host
 * check is conservative) leaves the pool in error (SS_ERR_CAPACITY). */
ss_status ss_compact(ss_pool *pool, int32_t group, hipStream_t stream);

/* Compaction of the listed states only (ids: host [n], each in [0, n_states), repeats allowed):
 * the same Brand update, merge, truncation, re-split and promotion as ss_compact for each listed
 * state, legal with any pad fill.  The other members of the groups the ids belong to are moved
 * unchanged (components, pad and Gamma kept), because a compaction writes each touched group as
 * one new ring segment.  It therefore costs a copy of the touched groups; the schedule of
 * ss_compact is not affected.  Bad ids: SS_ERR_ARG before any device work.  It waits for
 * `stream` before uploading the selection (not for use inside a captured graph). */
ss_status ss_compact_ids(ss_pool *pool, const int32_t *ids, int64_t n, hipStream_t stream);

/* Consolidation of the frozen part ([SS] 4.3 "Asynchronous CPU
 * Consolidation", Figure 7(a)), run on the device: for every factored state
 * of group `group` (of all groups when group < 0), the frozen components are
 * replaced by the exact SVD of their sum, keeping the singular values
 * >= eps * sigma_0, where sigma_0 is the state's largest stored singular
 * value before the call (the larger of the first active and the first frozen
 * one).  The active part, the pad and Gamma are left as they are; the new
 * frozen list is sorted descending on its own.  The components are rewritten
 * in place (there are never more of them), so the group's ring segment keeps
 * its size until its next compaction.  The work is ordered on `stream` with
 * decode steps and compactions: it sees the frozen part the last compaction
 * left and is done before the next one reads it, so a result is never stale.
 * Errors: SS_ERR_ARG (bad group), SS_ERR_SHAPE (the pool's largest frozen part,
 * f = min(max_frozen, L - r_active) with promotion and max_frozen without,
 * needs more than 160 KB of LDS: 4 (f' d_k + f d_v + f'^2 + 3 f' + 4) bytes,
 * f' = f rounded up to even), SS_ERR_HIP.  A force_dense pool is a no-op. */
ss_status ss_consolidate(ss_pool *pool, int32_t group, hipStream_t stream);

/* Consolidation scheduling ([SS] 4.3, Figure 7(b)) on one stream: each
 * compaction puts its group in a wait queue; this call consolidates up to
 * max_groups waiting groups, the least recently consolidated first (groups
 * never consolidated before all others, then by id), removes them from the
 * queue, writes their ids to out (NULL: not reported; otherwise room for
 * max_groups) and their count to *n_done.  The pages' drop of stale results
 * and retry-first rule have nothing to act on here: stream order makes every
 * result current.  Errors as ss_consolidate. */
ss_status ss_consolidate_next(ss_pool *pool, int32_t max_groups, int32_t *out, int32_t *n_done, hipStream_t stream);

/* Asynchronous consolidation ([SS] 4.3 "Asynchronous CPU Consolidation": the consolidation runs
 * beside the decode, a result that has gone stale is dropped, and a fresh one replaces the frozen
 * part).  Here the exact SVD runs on the GPU, on a second stream `side` given by the caller, while
 * the pool's stream goes on decoding.
 *  ss_consolidate_async: group >= 0 selects that group; group < 0 takes, among the groups waiting
 *    (compacted since their last consolidation), those whose last asynchronous result was dropped
 *    as stale first, then the least recently consolidated (never consolidated first), then the
 *    lowest id ([SS] Figure 7(b); *launched = -1 when no group waits).  On
 *    `stream` it copies the group's 16-byte records aside; `side` waits for that copy and runs the
 *    kernel, which reads the frozen parts and writes its results to staging only (the rings and
 *    records are not touched).  One consolidation may be in flight per pool (SS_ERR_STATE for a
 *    second); the staging (largest group x frozen cap x (d_k + d_v + 1) floats) is allocated at the
 *    first call.  Not available with diag_decay (SS_ERR_ARG); a frozen part too large for the
 *    kernel's LDS gives SS_ERR_SHAPE.
 *  ss_consolidate_poll: *state = SS_CONS_IDLE (nothing in flight), SS_CONS_RUNNING (the kernel has
 *    not finished; wait = 0 returns at once, wait != 0 blocks until it has), SS_CONS_INSTALLED (an
 *    install is enqueued on `stream`: each state whose record still shows the active and frozen
 *    counts of the copy gets the result in place of its frozen part), or SS_CONS_DISCARDED (the
 *    group was compacted, or consolidated synchronously, after the launch: the result is dropped).
 * The caller keeps `side` alive until the poll has returned INSTALLED or DISCARDED; a ring re-pack
 * waits for the kernel before it frees the rings the kernel reads.  Streams of default priority. */
enum { SS_CONS_IDLE = 0, SS_CONS_RUNNING = 1, SS_CONS_INSTALLED = 2, SS_CONS_DISCARDED = 3 };
ss_status ss_consolidate_async(ss_pool *pool, int32_t group, hipStream_t stream, hipStream_t side, int32_t *launched);
ss_status ss_consolidate_poll(ss_pool *pool, int32_t wait, hipStream_t stream, int32_t *state);

/* Asynchronous consolidation on host cores, the pipeline of [SS] 4.3 "Asynchronous CPU
 * Consolidation" and Figure 7(b): download the frozen parts, exact SVD on the host, upload, and
 * install unless the group has compacted meanwhile.  Group selection, the snapshot of the records
 * on `stream`, the one-in-flight rule, SS_CONS_* states and the install with its staleness check
 * are those of ss_consolidate_async, and ss_consolidate_poll completes it; the frozen part a
 * result replaces is the one the snapshot names.  The library's own second stream (created at the
 * first call, default priority) gathers the group's frozen components into device staging (the
 * group's segment of the frozen ring, packed per member as [group][f][d_k], [.][f][d_v], [.][f])
 * and copies them, with each state's sigma_0, into pinned host memory.  A host thread then waits
 * for the download and runs, on `threads` host threads (0: one per hardware thread), an exact
 * fp64 SVD of every frozen part (thin QR of V_F, B = U_F Sigma_F R^T, thin QR of B, one-sided
 * Jacobi on its R to 1e-15), drops values below eps * sigma_0, and enqueues the upload of the
 * results on the same stream.  ss_consolidate_poll returns SS_CONS_RUNNING until that upload is
 * enqueued (wait != 0 blocks), then installs on `stream` after it, or drops a stale result.  A
 * ring re-pack waits only for the gather.  Pinned host memory of the staging's size is allocated
 * at the first call.  Not available with diag_decay (SS_ERR_ARG).  Errors: SS_ERR_ARG,
 * SS_ERR_STATE (one in flight), SS_ERR_OOM, SS_ERR_HIP. */
ss_status ss_consolidate_host(ss_pool *pool, int32_t group, hipStream_t stream, int32_t threads, int32_t *launched);

/* The host arithmetic of ss_consolidate_host for one state, on host memory (a test and
 * measurement hook; touches no GPU): the f components u [f][d_k], v [f][d_v], sigma [f] (fp32,
 * caller-owned) are replaced by the exact SVD of sum_k sigma_k u_k v_k^T with the values below
 * eps * sigma0 dropped, in descending order; *kept receives their count (<= f) and rows past it
 * are left as they were.  Errors: SS_ERR_ARG (null pointer, f < 0), SS_ERR_SHAPE (d_k, d_v < 1). */
ss_status ss_host_consolidate_frozen(int32_t d_k, int32_t d_v, int32_t f, float *u, float *v, float *sigma,
                                     float sigma0, float eps, int32_t *kept);

/* Staggered schedule ([SS] 4.2 "Staggered compaction across layers"): the
 * groups due after decode step `step` (counted from 1) are those with
 * (step + group_offset[g]) mod K == 0.  Writes up to `cap` group ids to out
 * and returns their count in *n_due.  Host only. */
ss_status ss_schedule_due(const ss_pool *pool, int64_t step, int32_t *out, int32_t cap, int32_t *n_due);

/* Randomized block SVD initialization of dense states after prefill
 * ([SS] 4.1; 4.2 "Randomized SVD initialization after prefill", Figure
 * 6(a)).  For each of the n states S [d_k][d_v] (the pages' H = S^T), block
 * by block, from the caller's Gaussian Omega_k [d_k][block]:
 *   `iters` times:  Y = S^T Omega,  Q = orth(Y),  Omega = S Q;
 *   block SVD Omega = X diag(sigma) W^T;  components u = X, v = Q W, sigma;
 * sigma_0 is the first block's largest sigma; components with
 * sigma >= eps sigma_0 and sigma > 0 are kept, in descending order within a
 * block; if one is below, no further block is taken; otherwise the block is
 * subtracted from the residual and the next block starts.  At most n_blocks
 * blocks and max_rank components.  (The dense-fallback decision, rank > L,
 * is taken when a pool is built from these results:
 * ss_state_pool_create_from_dense.)
 * All pointers are device memory, row-major, caller-owned:
 *   S [n][d_k][d_v] (read), omega [n][n_blocks][d_k][block] (read),
 *   eps [n] (read), work [n][d_k][d_v] (scratch, overwritten),
 *   u [n][max_rank][d_k], v [n][max_rank][d_v], sigma [n][max_rank] (written
 *   up to rank[s] per state), rank [n] (written).
 * Enqueued on `stream`, no synchronization.  Shapes: d_k, d_v multiples of 4
 * in [4, 256]; 1 <= block <= min(16, d_k, d_v); 1 <= iters <= 64;
 * 1 <= max_rank <= min(d_k, d_v, n_blocks block).  Errors: SS_ERR_ARG,
 * SS_ERR_SHAPE (checked on the host), SS_ERR_HIP. */
ss_status ss_rsvd_init(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                       int32_t iters, const float *omega, const float *eps, int32_t max_rank, float *work, float *u,
                       float *v, float *sigma, int32_t *rank, hipStream_t stream);

/* ss_rsvd_init without the caller's workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing: a state whose
 * d_k x d_v residual does not fit the kernel's LDS (d_k (d_v + 1) floats
 * above 120 KB, e.g. 256 x 128) keeps it in a fixed 32 MiB device array that
 * the library holds on each GPU it runs on until the process ends; smaller
 * states use no workspace at all.  Arguments, layouts, results and errors are
 * those of ss_rsvd_init (the same kernel runs), without `work`.  Limit: when
 * the workspace is used, n * d_k * d_v must not exceed 8,388,608 floats, else
 * SS_ERR_CAPACITY (checked on the host before any HIP call); split larger
 * batches over several calls.  Every call on a GPU shares that GPU's array
 * (its contents are overwritten, none needs to start at zero), so calls that
 * overlap on one GPU, on different streams or threads, race; calls on one
 * stream do not. */
ss_status ss_rsvd_init_noalloc(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                               int32_t iters, const float *omega, const float *eps, int32_t max_rank, float *u,
                               float *v, float *sigma, int32_t *rank, hipStream_t stream);

/* Whole decode steps as HIP graphs ([SS] 4.4 "Kernel fusion, load balancing,
 * and support for CUDA graphs": the pages replay steps as graphs; here one
 * graph is captured per phase of the schedule, step mod K).  Replaying
 * phase p runs ss_decode_step on the fixed buffers given at creation,
 * followed by ss_compact of every group due at a step in that phase and the
 * pruning of the factored-state list, with no launch from the host but the
 * graph's.  The caller writes each step's inputs into q, k, v, alpha, beta
 * (device, [N][d_k], [N][d_k], [N][d_v], [N], [N]; beta may be NULL when the
 * pool has no delta-rule state) before launching, in stream order; o [N][d_v]
 * receives the output.  The buffers stay owned by the caller and must
 * outlive the graph object, which must be destroyed before its pool.
 *
 * ss_step_graph_launch(g, step, stream) is equivalent, result for result,
 * to ss_decode_step followed by ss_compact for each group returned by
 * ss_schedule_due(step), and may be mixed freely with those calls.  Before
 * the launch it runs the host-side ring check of ss_compact (which may
 * synchronize `stream` and re-pack); a re-pack moves the rings, and the
 * graphs are then captured again before the launch.  Kernel timing
 * (ss_pool_timing) does not cover graph launches.  Errors: SS_ERR_ARG,
 * SS_ERR_OOM, SS_ERR_HIP, and the pool's sticky errors. */
typedef struct ss_step_graph ss_step_graph;
ss_status ss_step_graph_create(ss_pool *pool, const float *q, const float *k, const float *v, const float *alpha,
                               const float *beta, float *o, ss_step_graph **out);
ss_status ss_step_graph_launch(ss_step_graph *graph, int64_t step, hipStream_t stream);
ss_status ss_step_graph_destroy(ss_step_graph *graph);

/* Test hook: copy states `ids` (host array) to host memory in the canonical
 * form, effective weights (Gamma folded in).  Waits on `stream`.  Layout per
 * state, packed in id order:
 *   int32 header[8] = {id_lo, dense, n_components, n_active, n_pad, rule, dense_pad, 0}
 *   then, if dense: float S[d_k][d_v] (dense_pad buffered slots folded in, on the host, in double);
 *   else: float sigma[n_components], u[n_components][d_k], v[n_components][d_v],
 *         c[n_pad], k[n_pad][d_k], w[n_pad][d_v]
 * Components are in stored order: the n_active active ones first, then the
 * frozen ones.  *needed receives the byte size; if cap is too small nothing
 * is written and SS_ERR_CAPACITY is returned. */
ss_status ss_state_export(ss_pool *pool, const int64_t *ids, int64_t n, void *host_buf, size_t cap, size_t *needed,
                          hipStream_t stream);

/* Pool statistics; waits on `stream`.  Reading the statistics also collects
 * the kernel durations recorded since the previous call. */
ss_status ss_pool_stats(ss_pool *pool, ss_stats *out, hipStream_t stream);

/* Measurement hook: with enable = 1 every later kernel launch of the pool is
 * bracketed by a pair of HIP events recorded on the launch stream, and
 * ss_pool_stats adds their elapsed times to kernel_ms / kernel_launches.
 * enable = 0 stops recording.  Costs two event records per launch. */
ss_status ss_pool_timing(ss_pool *pool, int32_t enable);

/* L = floor(d_k d_v / (d_k + d_v)): above this many components the factored
 * form (d_k + d_v + 1 values each) is larger than the dense d_k d_v ([SS] 4.4). */
int32_t ss_dense_rank_limit(int32_t d_k, int32_t d_v);

/* How a state is decoded, for ss_decode_bytes_per_state. */
enum {
  SS_DECODE_FACTORED = 0,       /* factors + pad */
  SS_DECODE_DENSE_BUFFERED = 1, /* dense region of a factored pool: H + pad */
  SS_DECODE_DENSE_PLAIN = 2,    /* force_dense pool (the dense baseline) */
  SS_DECODE_FACTORED_FP16 = 3   /* factors + pad in a pool with factor_fp16 = 1 */
};

/* Algorithmic bytes one decode_step moves for one state with n_comp
 * components and n_pad filled slots before the step (K = pad_slots).
 * FACTORED: reads the 16-byte record, all components and slots
 * (4 (d_k + d_v + 1) bytes each), q, k, v, alpha (and beta for the delta
 * rule); writes the record, one slot and o.  DENSE_BUFFERED: reads the
 * 16-byte slot record, H (4 d_k d_v bytes), the slots and the inputs;
 * writes the record, o, and one slot, or H when the step fills the pad
 * (n_pad + 1 >= K).  DENSE_PLAIN: reads the slot record and reads and
 * writes H every step.  FACTORED_FP16: as FACTORED with 2 (d_k + d_v) + 4
 * bytes per stored component (pad slots stay 4 (d_k + d_v + 1)).  Returns 0
 * for an unknown kind. */
uint64_t ss_decode_bytes_per_state(int32_t d_k, int32_t d_v, int32_t pad_slots, int32_t n_comp, int32_t n_pad,
                                   int32_t rule, int32_t kind);

const char *ss_status_string(ss_status status);
const char *ss_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SINKSTATE_H_ */

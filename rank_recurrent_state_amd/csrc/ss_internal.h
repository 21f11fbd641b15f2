// ss_internal.h -- device-side layout and kernel launchers shared by the
// HIP sources of libsinkstate.so (not part of the public ABI).
//
// Layout in HBM (SinkState, 4.4 "Memory layout": buffer apart from the
// factors, active and frozen parts in separate contiguous regions, offsets
// per state, a separate dense region):
//   meta   [N]                16-byte record per state (offsets, Gamma, counts)
//   active arena              components: u [cap][d_k], v [cap][d_v], sigma [cap]
//   frozen arena              same shape, separate allocation
//   pad    [N][K]             k [N][K][d_k], w [N][K][d_v], c [N][K] (c = 1/Gamma at insertion)
//   dense  [cap_d][d_v][d_k]  states of the dense region stored transposed (H = S^T)
//   dslot  [cap_d]            16-byte record per dense slot (state id, pad fill, flags, Gamma)
//   dense pads [cap_d][K]     k [.][K][d_k], w [.][K][d_v], c [.][K], indexed by slot
// Everything a dense-region step reads, except q, k, v, is addressed by the slot alone.
//
// The active and frozen arenas are rings of `cap` components.  Positions are
// virtual (64-bit, only growing); component c lives at c mod cap, and a
// state's components are consecutive in that sense, so the record holds the
// physical start and a reader wraps once (wrap()).  A compaction places the
// new components of its group from the ring head: each member gets a slot of
// the largest counts its record allows (at most r active, at most its pad size
// more than before), at a prefix sum taken before the compaction, so the
// kernel allocates nothing and a group's components form one segment whose
// slack is bounded by the pads; the group's previous segment is released
// when the compaction completes, and the ring tail is the oldest segment
// still live.  A re-pack lays the segments out exactly again.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr uint32_t FLAG_DELTA = 1u;
constexpr uint32_t FLAG_DENSE = 2u;
constexpr int kMaxM = 16;      // r + K
constexpr int kAcctSlots = 256;
// accounting arrays, kAcctSlots entries each
enum Acct : int {
  A_DECODE_FACTORED = 0, A_DECODE_DENSE = 1, A_COMPACT_FLOPS = 2, A_COMPACT_STATES = 3,
  A_CONS_FLOPS = 4, A_CONS_STATES = 5, A_CONS_REMOVED = 6, A_N = 7
};

// 16-byte per-state record.  packed: ra | rf << 8 | n << 16 | flags << 24.
struct __attribute__((aligned(16))) Meta {
  int32_t off_a;   // factored: first active component; dense: dense slot
  int32_t off_f;   // first frozen component
  float gamma;     // decay accumulated since the last compaction
  uint32_t packed;
};

__host__ __device__ inline uint32_t meta_ra(uint32_t p) { return p & 0xffu; }
__host__ __device__ inline uint32_t meta_rf(uint32_t p) { return (p >> 8) & 0xffu; }
__host__ __device__ inline uint32_t meta_n(uint32_t p) { return (p >> 16) & 0xffu; }
__host__ __device__ inline uint32_t meta_flags(uint32_t p) { return p >> 24; }
__host__ __device__ inline uint32_t meta_pack(uint32_t ra, uint32_t rf, uint32_t n, uint32_t flags) {
  return (ra & 0xffu) | ((rf & 0xffu) << 8) | ((n & 0xffu) << 16) | (flags << 24);
}

// Device-side counters (uint32 unless noted).
enum Counter : int {
  C_DENSE_COUNT = 0,   // dense slots in use
  C_PROMOTE_COUNT = 1, // states queued for promotion by the running compaction
  C_ERR_PAD = 2,       // decode found a full pad (also raised on a host-mapped flag)
  C_ERR_DENSE_CAP = 3, // promotion found the dense region full (also host-mapped)
  C_CAP_TRUNC = 4,     // frozen components dropped because max_frozen was reached
  C_PROMOTIONS = 5,    // total promotions
  C_FACT0 = 6,         // length of the factored-state list
  C_FACT1 = 7,         // length of its scratch copy while it is pruned
  C_MAT_BASE = 8,      // first dense slot of the states a materialization places
  C_JACOBI_LIMIT = 9,  // compactions whose Jacobi SVD still rotated in its last allowed sweep
  C_N = 10
};

// 16-byte record of a dense slot.  packed: n << 16 | flags << 24, as Meta.
struct __attribute__((aligned(16))) DenseSlot {
  int32_t s;       // state id
  uint32_t packed;
  float gamma;     // decay accumulated since the pad was last folded
  uint32_t spare;
};

// A ring of components.  The factor vectors u, v are stored in fp32 or, in a
// pool created with fp16 factors (SEED 6 "Lower precision composes": factors
// rounded to fp16 when a compaction writes them, the pad kept in fp32), in
// fp16; sigma is always fp32.  Kernels take the element type F as a template
// parameter and reach the vectors through U<F>() / V<F>().
struct Arena {
  void *u, *v;
  float *s;
  int64_t cap;  // components (a ring)
  int half;     // 1: u, v hold _Float16
  template <typename F> __host__ __device__ F *U() const { return static_cast<F *>(u); }
  template <typename F> __host__ __device__ F *V() const { return static_cast<F *>(v); }
};
// bytes of one factor element
__host__ __device__ inline int fac_bytes(const Arena &a) { return a.half ? 2 : 4; }

// physical slot of ring position (start + i), start < cap, i < cap
__host__ __device__ inline int64_t wrap(int64_t c, int64_t cap) { return c >= cap ? c - cap : c; }

// allocation state of one ring (device memory)
struct Ring {
  unsigned long long head;   // next free virtual position
  unsigned long long limit;  // allocations must end at or before this (tail + cap), set per compaction
  unsigned long long begin;  // head when the running compaction started
  unsigned long long overflow;  // allocations refused (the ring was full)
};

struct DecodeArgs {
  int64_t N;
  int dk, dv, K;
  const int32_t *fact_ids;     // ids of the factored states (dense ones are served by the dense kernel)
  const uint32_t *fact_count;  // its length (device)
  int64_t n_states;            // states in the pool: a list of that length holds every state once
  Meta *meta;
  Arena act, frz;
  float *pk, *pw, *pc;
  const float *q, *k, *v, *alpha, *beta;
  float *o;
  uint32_t *counters;
  unsigned long long *acct;   // [kAcctSlots] algorithmic bytes
  uint32_t *hflag;            // host-mapped flag raised when a pad is found full
  float *gam;                 // per-channel decay pools: [N][d_k] decay accumulated since the last
                              // compaction (alpha is then [N][d_k]); nullptr: scalar decay
};

struct DenseArgs {
  int dk, dv, K;
  uint32_t cap_d;
  Meta *meta;
  float *dense;
  DenseSlot *dslot;
  float *pk, *pw, *pc;         // slot-indexed pads of the buffered dense region (nullptr: plain baseline)
  const int32_t *members;      // fold mode: state ids of a compaction group
  int32_t n_members;
  const float *q, *k, *v, *alpha, *beta;
  float *o;
  uint32_t *counters;
  unsigned long long *acct;
  int diag;                    // per-channel decay: alpha is [N][d_k]
  float *dgam;                 // buffered region with per-channel decay: [cap_d][d_k] per slot
  const uint8_t *sel;          // fold mode: [N] states to fold, or nullptr: all members
};

struct CompactArgs {
  int dk, dv, K, r, L, promote, fcap;
  int32_t n_members;
  const int32_t *members;      // state ids of the group, in member order
  const float *eps;
  Meta *meta;
  Arena act, frz;
  Ring *ring_a, *ring_f;       // the new components go to [begin, head) of these
  const unsigned long long *slot_in, *slot_blk;  // member slots (launch_ring_begin)
  uint32_t *hflag;             // host-mapped flag raised when a ring is full
  float *pk, *pw, *pc;
  int32_t *promote_list;
  uint32_t *counters;
  unsigned long long *acct_flops;
  unsigned long long *acct_states;
  float *gam;                  // per-channel decay pools: [N][d_k] (reset to 1 by a compaction); nullptr otherwise
  const uint8_t *sel;          // [N] states to compact, or nullptr: all members.  An unselected member
                               // of the group is moved to the new segment unchanged (pad, Gamma kept).
};

struct MaterializeArgs {
  int dk, dv, cap_d;
  const int32_t *list;         // state ids
  const uint32_t *count;       // number of entries in list (device)
  int32_t fixed_count;         // used when count == nullptr
  Meta *meta;
  const Meta *src_meta;        // where the components are (meta after compaction), or nullptr
  const int64_t *csr_off;      // alternative source: CSR offsets per state (init)
  const float *csr_u, *csr_v, *csr_s;
  const int64_t *dsrc_idx;     // init: per state, index of its given dense S in dsrc, or -1
  const float *dsrc;           // [.][d_k][d_v] row-major
  Arena act, frz;
  float *dense;
  DenseSlot *dslot;
  uint32_t *counters;
  uint32_t *hflag;             // host-mapped flag raised when the dense region is full
  float *dgam;                 // per-channel decay pools: the new slot's [d_k] decay, set to 1; or nullptr
};

struct ScatterArgs {
  int64_t N;
  int dk, dv, r, L, fcap, force_dense;
  const int64_t *csr_off;
  const float *csr_u, *csr_v, *csr_s;
  const int64_t *dst_a, *dst_f;   // per state: first ring position of its active / frozen components
  const uint8_t *rule;
  const uint8_t *dense_mask;     // states given dense (or nullptr)
  Meta *meta;
  Arena act, frz;
  int32_t *dense_list;           // states to materialize
  uint32_t *counters;            // uses C_PROMOTE_COUNT as the list length
};

// launchers (return hipError_t of the launch)
hipError_t launch_decode_factored(const DecodeArgs &a, bool readonly, bool any_delta, hipStream_t st);
// dense region: buffered (pads present) or plain (the dense baseline)
hipError_t launch_decode_dense(const DenseArgs &a, int64_t n_upper, bool readonly, bool any_delta, hipStream_t st);
// fold the pads of the dense states among a.members into their H (compaction of the dense region)
hipError_t launch_dense_fold(const DenseArgs &a, hipStream_t st);
hipError_t launch_compact(const CompactArgs &a, hipStream_t st);
hipError_t launch_materialize(const MaterializeArgs &a, int64_t grid_upper, hipStream_t st);
hipError_t launch_scatter(const ScatterArgs &a, hipStream_t st);
hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t st);
hipError_t launch_fill_f32(float *p, int64_t n, float x, hipStream_t st);
// Before a compaction of a group: each member's slots in the new segments (slot_in, per member
// relative to the block of kSlotBlock members it falls in; slot_blk, per block; both packed as
// active | frozen << 32), and per ring limit = (oldest live segment start) + cap, begin = head,
// head = begin + the slots; the promotion list and the pruning scratch emptied.  After it: the
// group's segment becomes [begin, head).
constexpr int kSlotBlock = 1024;
struct RingBeginArgs {
  Ring *ring_a, *ring_f;
  const unsigned long long *seg_a, *seg_f;
  int n_groups;
  int64_t cap_a, cap_f;
  uint32_t *counters;
  const int32_t *members;             // the group's members
  int n_members;
  const Meta *meta;
  int r, fcap;
  unsigned long long *slot_in;        // [n_members]
  unsigned long long *slot_blk;       // [ceil(n_members / kSlotBlock)]
  uint32_t *hflag;                    // host-mapped flag raised when a ring is full
};
hipError_t launch_ring_begin(const RingBeginArgs &b, hipStream_t st);
hipError_t launch_ring_end(Ring *ra, Ring *rf, unsigned long long *seg_a, unsigned long long *seg_f, int g,
                           hipStream_t st);
// copy every factored state's components into new rings at the given positions (arena growth)
struct RepackArgs {
  int64_t N;
  int dk, dv;
  Meta *meta;
  Arena src_a, src_f, dst_a, dst_f;
  const int64_t *new_a, *new_f;  // per state: new first position (physical) or -1 for dense states
};
hipError_t launch_repack(const RepackArgs &a, hipStream_t st);
// Exact ring layout of every factored state on the device: groups in the order `ord` (device
// [G]: group id; gstart/gsize: device [G] of the groups' member ranges in `members`), each
// group's members in member order, counts from the records; writes new_a/new_f per state (-1 for
// dense states), seg [2][2G] and the rings' head = begin = total.  scratch: see layout_scratch_bytes.
struct LayoutArgs {
  int64_t N;
  int G;
  const int32_t *members, *ord;
  const int64_t *gstart, *gsize, *lstart;  // lstart [G + 1]: layout index where ord slot k starts
  const Meta *meta;
  int64_t *cnt_a, *cnt_f, *off_a, *off_f;  // [N] each
  int64_t *new_a, *new_f;                  // [N]
  unsigned long long *seg;
  Ring *ring;
  void *scan_tmp;
  size_t scan_bytes;
};
size_t layout_scan_bytes(int64_t N);
hipError_t launch_ring_layout(const LayoutArgs &a, hipStream_t st);
// drop the states that have become dense from the factored-state list: list -> tmp, then back into
// list, so the decode always reads the same list; the new length goes to *count and a host-visible word.
// *tmp_count must be 0 (a compaction's launch_ring_begin clears it).
hipError_t launch_prune_factored(int32_t *list, uint32_t *count, int32_t *tmp, uint32_t *tmp_count, int64_t n_upper,
                                 const Meta *meta, uint32_t *host_count, hipStream_t st);

// randomized block SVD initialization of n dense states (one workgroup each)
struct RsvdArgs {
  int64_t n;
  int dk, dv, b, nb, iters, max_rank;
  const float *S;      // [n][d_k][d_v]
  const float *omega;  // [n][nb][d_k][b]
  const float *eps;    // [n]
  float *work;         // [n][d_k][d_v] residual
  float *u, *v, *sigma;  // [n][max_rank][d_k], [n][max_rank][d_v], [n][max_rank]
  int32_t *rank;       // [n]
};
hipError_t launch_rsvd_init(const RsvdArgs &a, hipStream_t st);
// whether a d_k x d_v residual fits the initialization kernel's LDS (else it needs a workspace)
bool rsvd_residual_in_lds(int dk, int dv);
// the fixed device workspace of ss_rsvd_init_noalloc: kRsvdScratchFloats floats (32 MiB) per GPU;
// its address on the current device (looked up once per device)
constexpr size_t kRsvdScratchFloats = size_t(8) << 20;
hipError_t rsvd_scratch(float **out);

// consolidation of the frozen parts of a group's factored states (one workgroup each, in place)
struct ConsolidateArgs {
  int dk, dv, fmax;            // fmax: largest frozen count a state can hold (sizes the LDS)
  int32_t n_members;
  const int32_t *members;
  const float *eps;
  Meta *meta;
  Arena act, frz;
  unsigned long long *acct_flops, *acct_states, *acct_removed;
  // asynchronous form (all nullptr: in place).  The kernel reads the group's records from `snap`
  // (taken at launch) and writes its results to staging instead of the rings:
  const Meta *snap;            // [n_members]
  float *st_u, *st_v, *st_s;   // [n_members][fmax][d_k], [n_members][fmax][d_v], [n_members][fmax]
  int32_t *st_cnt;             // [n_members] kept frozen components
};
constexpr size_t kConsolidateLdsMax = 160 * 1024;  // LDS per workgroup on gfx950
size_t consolidate_lds_bytes(int dk, int dv, int fmax, bool q_in_lds);
hipError_t launch_consolidate(const ConsolidateArgs &a, hipStream_t st);
// asynchronous consolidation: the group's records copied aside at launch (on the pool's stream),
// and the install of the staged results, state by state, where a state's record still shows the
// frozen part the result was computed from (same active and frozen counts, not dense)
hipError_t launch_cons_snapshot(const Meta *meta, const int32_t *members, int32_t n, Meta *snap, hipStream_t st);
struct InstallArgs {
  int dk, dv, fmax;
  int32_t n_members;
  const int32_t *members;
  const Meta *snap;
  Meta *meta;
  Arena frz;
  const float *st_u, *st_v, *st_s;
  const int32_t *st_cnt;
  unsigned long long *acct_removed;
  uint32_t *installed;         // states installed (device counter)
};
hipError_t launch_cons_install(const InstallArgs &a, hipStream_t st);
// host-core consolidation: the frozen parts the snapshot names, copied into staging for download
struct GatherArgs {
  int dk, dv, fmax;
  int32_t n_members;
  const Meta *snap;
  Arena act, frz;
  float *st_u, *st_v, *st_s;   // [n_members][fmax][d_k], [.][fmax][d_v], [.][fmax]
  int32_t *st_cnt;             // [n_members] frozen count copied (0: left alone)
  float *st_s0;                // [n_members] sigma_0 of the state
};
hipError_t launch_cons_gather(const GatherArgs &a, hipStream_t st);

// how a state is decoded
enum DecodeKind : int { KIND_FACTORED = 0, KIND_DENSE_BUFFERED = 1, KIND_DENSE_PLAIN = 2 };

// algorithmic bytes of one decode step of one state (kept identical to the
// in-kernel accounting).  n_pad is the pad fill before the step; a buffered
// dense state whose pad fills in this step rewrites H instead of a pad slot.
// fsz: bytes of a stored factor element (4, or 2 with fp16 factors); pad slots are fp32.
// diag: per-channel decay (alpha has d_k entries; the buffered forms also read and write the
// d_k accumulated decays).
__host__ __device__ inline unsigned long long decode_bytes(int dk, int dv, int K, int ncomp, int npad, bool delta,
                                                           int kind, int fsz = 4, bool diag = false) {
  const unsigned long long in = 4ull * (2ull * dk + dv + (diag ? dk : 1) + (delta ? 1 : 0)) +
                                (diag && kind != KIND_DENSE_PLAIN ? 8ull * dk : 0ull);
  const unsigned long long comp = 4ull * (unsigned long long)(dk + dv + 1);
  const unsigned long long fcomp = (unsigned long long)fsz * (unsigned long long)(dk + dv) + 4ull;
  const unsigned long long st = 4ull * (unsigned long long)dk * dv;
  if (kind == KIND_DENSE_PLAIN)  // slot record read, state read and written, inputs, output
    return 16ull + 2ull * st + in + 4ull * dv;
  if (kind == KIND_DENSE_BUFFERED)  // slot record read+write, H and the pad read, inputs, output, slot or H written
    return 32ull + st + comp * (unsigned long long)npad + in + 4ull * dv + (npad + 1 >= K ? st : comp);
  // record read+write, components and pad slots read, inputs, one slot written, output
  return 32ull + fcomp * (unsigned long long)ncomp + comp * (unsigned long long)npad + in + comp + 4ull * dv;
}

}  // namespace ss

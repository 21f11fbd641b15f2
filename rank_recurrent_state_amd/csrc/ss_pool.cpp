// ss_pool.cpp -- host side of libsinkstate.so: argument checks, pool layout
// and device allocation, launch orchestration, export and statistics.
//
// Pool layout (SinkState 4.4 "Memory layout": active and frozen factors in
// their own contiguous regions, offsets per state).  Each region is a ring of
// components; the states are listed by compaction group, and each group's
// components form one segment of the ring (exactly packed when laid out or
// re-packed; after a compaction each member's slot may hold up to its pad
// size of slack).  A compaction of group g places the group's new segment at
// the ring head (never writing what may still be read) and releases the old
// one, so with the groups laid out in the order in which they fall due the
// ring holds the live components plus one group's growth.  The host bounds the ring usage without waiting
// for the device (see ensure_ring_space) and re-packs, growing the ring,
// only when the bound says the next compaction might not fit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <deque>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <thread>
#include <vector>

#include "../../include/sinkstate.h"
#include "ss_host_cons.h"
#include "ss_internal.h"

namespace {

thread_local std::string g_last_error;

ss_status fail(ss_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

// host-mapped words: error flags raised by kernels, and the length of the factored-state list
enum HostFlag { HF_PAD = 0, HF_DENSE_CAP = 1, HF_FACT = 2, HF_RING = 3, HF_N = 4 };
constexpr int64_t kPruneEvery = 8;

}  // namespace

struct ss_pool {
  int64_t N = 0;
  int dk = 0, dv = 0, K = 0, r = 0, L = 0, promote = 0, force_dense = 0, fcap = 0, G = 0;
  int half = 0;  // factor vectors stored in fp16
  int diag = 0;  // per-channel decay (alpha is [N][d_k])
  bool any_delta = false;
  std::vector<int32_t> group_offset;
  std::vector<int64_t> group_start, group_size;
  std::vector<int32_t> members_host;  // state ids grouped by compaction group
  std::vector<float> eps_host;        // per state epsilon (host copy)
  int64_t cap_d = 0;
  int64_t dense_upper = 0;
  // device memory
  ss::Meta *meta = nullptr;
  int32_t *members = nullptr;
  float *eps = nullptr;
  ss::Arena act{nullptr, nullptr, nullptr, 0, 0}, frz{nullptr, nullptr, nullptr, 0, 0};
  // rings of components (0: active, 1: frozen): device allocation state and per-group segments,
  // and the host's bounds on them (see ensure_ring_space)
  void *ring_blk[2] = {nullptr, nullptr};
  size_t ring_bytes[2] = {0, 0};
  ss::Ring *ring = nullptr;            // [2]
  unsigned long long *seg = nullptr;   // [2][2 G]: virtual start, end of each group's segment
  unsigned long long *slot_in = nullptr, *slot_blk = nullptr;  // a compaction's member slots (largest group)
  // Segments of each ring in allocation order (group -1: a released gap), each with an upper
  // bound of its size; the latest record of a group is its live segment.
  struct RingRec { int64_t seq; int g; int64_t n; };
  std::deque<RingRec> recs[2];
  std::vector<int64_t> last_seq[2];    // per group: seq of its live segment, -1 if none
  std::vector<int64_t> seg_bound[2];   // per group: upper bound of its live segment size
  int64_t seq = 0;
  int64_t repacks = 0, ring_syncs = 0;
  int64_t layout_version = 0;          // bumped whenever device addresses captured in graphs change
  // device scratch of a re-pack's layout (allocated at the first re-pack)
  int64_t *lay_cnt = nullptr;          // [6][N]: counts, offsets, new positions (active, frozen)
  int64_t *lay_g = nullptr;            // [3G + 1]: group starts, sizes, layout starts
  int32_t *lay_ord = nullptr;          // [G]
  unsigned char *lay_scan = nullptr;
  size_t lay_scan_bytes = 0;
  float *pk = nullptr, *pw = nullptr, *pc = nullptr;
  float *gam = nullptr, *dgam = nullptr;  // per-channel decay: accumulated decays per state [N][d_k], per dense slot
  uint8_t *sel = nullptr;                 // [N] selection mask of ss_compact_ids (allocated at its first call)
  float *dense = nullptr;
  ss::DenseSlot *dslot = nullptr;
  float *dpk = nullptr, *dpw = nullptr, *dpc = nullptr;  // slot-indexed pads of the dense region
  int32_t *promote_list = nullptr;
  int32_t *fact_ids[2] = {nullptr, nullptr};  // factored-state list and its scratch copy, lengths in counters
  int64_t fact_upper = 0;                     // host upper bound of the current list's length
  uint32_t *counters = nullptr;
  unsigned long long *acct = nullptr;  // [A_N][kAcctSlots] accounting (see ss::Acct)
  uint32_t *hflags = nullptr;          // host-mapped words (HostFlag)
  uint32_t fact_count_host = 0;        // staging for the initial list length
  uint32_t *hflags_dev = nullptr;
  std::vector<void *> dev_allocs;
  int64_t reserved = 0;
  int64_t decode_calls = 0, compact_calls = 0, readout_calls = 0;
  // The factored-state list may hold states that have gone dense (the decode skips them), so the
  // eager path prunes it on every kPruneEvery-th compaction call only; the list then shrinks a
  // little later, for two launches fewer on the other calls.
  int64_t prune_due = 0;
  // consolidation queue: groups compacted since their last consolidation, and when each group
  // was last consolidated (-1: never)
  std::vector<char> cons_wait;
  std::vector<int64_t> cons_last;
  int64_t cons_seq = 0, consolidate_calls = 0;
  // asynchronous consolidation: one group at a time on a caller's second stream, results staged and
  // installed by ss_consolidate_poll on the pool's stream; stale once the group compacts meanwhile
  std::vector<char> cons_dropped;  // per group: its last asynchronous result was dropped as stale
  struct ConsAsync {
    bool inflight = false, stale = false;
    int group = -1;
    hipEvent_t snap_ev = nullptr, done_ev = nullptr;
    // the host-core form: the library's own stream for the gather, the download and the upload;
    // read_ev: the rings have been read (a re-pack waits for it); dl_ev: the download is done;
    // the host worker runs the SVDs, enqueues the upload and records done_ev
    bool host = false;
    hipStream_t own_side = nullptr;
    hipEvent_t read_ev = nullptr, dl_ev = nullptr;
    float *st_s0 = nullptr;
    float *h_u = nullptr, *h_v = nullptr, *h_s = nullptr, *h_s0 = nullptr, *h_eps = nullptr;
    int32_t *h_cnt = nullptr;
    int64_t h_members = 0;
    std::thread worker;
    std::atomic<int> hstate{0};  // 0 idle, 1 running, 2 done, 3 failed
    std::string herr;
    double host_ms = 0.0;        // wall time of the host SVDs of the last job
    ss::Meta *snap = nullptr;
    float *st_u = nullptr, *st_v = nullptr, *st_s = nullptr;
    int32_t *st_cnt = nullptr;
    uint32_t *installed = nullptr;
    int64_t cap_members = 0;
    int fmax = 0;
    int64_t launched = 0, installs = 0, discarded = 0;
    std::vector<int64_t> last_compact;  // per group: sequence number of its latest compaction (-1: none)
    int64_t compact_seq = 0;
  } ca;
  ss_status sticky = SS_OK;
  std::string sticky_msg;
  // measurement hook: event pairs around kernel launches
  struct EvPair {
    hipEvent_t a, b;
    int kernel;
  };
  bool timing = false;
  std::vector<EvPair> pending;
  std::vector<hipEvent_t> spare;
  double kernel_ms[SS_KERNEL_COUNT] = {0};
  int64_t kernel_launches[SS_KERNEL_COUNT] = {0};

  ss::Arena &arena(int R) { return R == 0 ? act : frz; }
  int64_t per_state_cap(int R) const { return R == 0 ? r : fcap; }
};

namespace {

template <typename T>
hipError_t dalloc(ss_pool *p, T **ptr, size_t count) {
  *ptr = nullptr;
  if (count == 0) return hipSuccess;
  void *q = nullptr;
  hipError_t e = hipMalloc(&q, count * sizeof(T));
  if (e != hipSuccess) return e;
  p->dev_allocs.push_back(q);
  p->reserved += (int64_t)(count * sizeof(T));
  *ptr = static_cast<T *>(q);
  return hipSuccess;
}

void free_all(ss_pool *p) {
  for (auto &e : p->pending) {
    (void)hipEventDestroy(e.a);
    (void)hipEventDestroy(e.b);
  }
  p->pending.clear();
  for (hipEvent_t e : p->spare) (void)hipEventDestroy(e);
  p->spare.clear();
  for (void *q : p->dev_allocs) (void)hipFree(q);
  p->dev_allocs.clear();
  for (int R = 0; R < 2; ++R) {
    if (p->ring_blk[R]) (void)hipFree(p->ring_blk[R]);
    p->ring_blk[R] = nullptr;
  }
  if (p->hflags) (void)hipHostFree(p->hflags);
  p->hflags = nullptr;
}

hipError_t take_event(ss_pool *p, hipEvent_t *e) {
  if (!p->spare.empty()) {
    *e = p->spare.back();
    p->spare.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(e);
}

// launch through `fn`, bracketed by events on `st` while timing is on
template <typename F>
hipError_t timed(ss_pool *p, int kernel, hipStream_t st, F fn) {
  if (!p->timing) return fn();
  ss_pool::EvPair ev{nullptr, nullptr, kernel};
  hipError_t e = take_event(p, &ev.a);
  if (e == hipSuccess) e = take_event(p, &ev.b);
  if (e == hipSuccess) e = hipEventRecord(ev.a, st);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = hipEventRecord(ev.b, st);
  if (e == hipSuccess) p->pending.push_back(ev);
  return e;
}

// IEEE 754 binary16 -> binary32 (exact): sign, 5-bit exponent (bias 15), 10-bit fraction;
// exponent 0 holds zero and the subnormals (fraction * 2^-24), exponent 31 infinities and NaNs
float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31, ex = (h >> 10) & 0x1fu, fr = h & 0x3ffu;
  float mag;
  if (ex == 0) mag = std::ldexp((float)fr, -24);
  else if (ex == 31) mag = fr ? std::numeric_limits<float>::quiet_NaN() : std::numeric_limits<float>::infinity();
  else mag = std::ldexp((float)(fr | 0x400u), (int)ex - 25);
  uint32_t bits;
  std::memcpy(&bits, &mag, 4);
  bits |= sign;
  std::memcpy(&mag, &bits, 4);
  return mag;
}

ss_status hip_fail(hipError_t e, const char *what) {
  return fail(SS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// bytes of one stored component: u and v (fp32 or fp16) and sigma (fp32)
int64_t comp_bytes(const ss_pool *p) { return (int64_t)(p->half ? 2 : 4) * (p->dk + p->dv) + 4; }

// one ring: u [cap][d_k], v [cap][d_v] (fp32 or fp16), sigma [cap] in a single allocation
hipError_t ring_alloc(ss_pool *p, int64_t cap, void **blk, size_t *bytes, ss::Arena *out) {
  const size_t fsz = p->half ? 2 : 4;
  *bytes = (size_t)cap * (size_t)comp_bytes(p);
  hipError_t e = hipMalloc(blk, *bytes);
  if (e != hipSuccess) return e;
  char *b = static_cast<char *>(*blk);  // d_k, d_v are multiples of 4: every part stays 8-byte aligned
  out->u = b;
  out->v = b + (size_t)cap * p->dk * fsz;
  out->s = reinterpret_cast<float *>(b + (size_t)cap * (p->dk + p->dv) * fsz);
  out->cap = cap;
  out->half = p->half;
  return hipSuccess;
}

// Group order in which the rings are laid out: by the next step at which each group is
// due, counted from a step at which group `first` is due (first < 0: from step 0, before
// any compaction), so that the group compacted next holds the oldest segment.
std::vector<int> ring_order(const ss_pool *p, int first) {
  std::vector<int> ord(p->G);
  std::vector<int64_t> key(p->G);
  for (int g = 0; g < p->G; ++g) {
    ord[g] = g;
    if (first >= 0) {
      key[g] = (((int64_t)p->group_offset[first] - p->group_offset[g]) % p->K + p->K) % p->K;
    } else {
      const int64_t k = ((-(int64_t)p->group_offset[g]) % p->K + p->K) % p->K;
      key[g] = k == 0 ? p->K : k;
    }
  }
  std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return key[x] < key[y]; });
  return ord;
}

// Lay the factored states' components out group by group in `ord`, from ring position 0.
// cnt[R][s]: active (R = 0) / frozen (R = 1) components of state s, -1 for dense states.
void ring_layout(const ss_pool *p, const std::vector<int> &ord, const std::vector<int32_t> (&cnt)[2],
                 std::vector<int64_t> (&pos)[2], std::vector<unsigned long long> &seg, int64_t (&tot)[2]) {
  for (int R = 0; R < 2; ++R) {
    pos[R].assign(p->N, -1);
    tot[R] = 0;
  }
  seg.assign(4 * (size_t)p->G, 0ull);
  for (int g : ord) {
    for (int R = 0; R < 2; ++R) seg[(size_t)R * 2 * p->G + 2 * g] = (unsigned long long)tot[R];
    for (int64_t i = p->group_start[g]; i < p->group_start[g] + p->group_size[g]; ++i) {
      const int32_t s = p->members_host[i];
      if (cnt[0][s] < 0) continue;
      for (int R = 0; R < 2; ++R) {
        pos[R][s] = tot[R];
        tot[R] += cnt[R][s];
      }
    }
    for (int R = 0; R < 2; ++R) seg[(size_t)R * 2 * p->G + 2 * g + 1] = (unsigned long long)tot[R];
  }
}

ss_status hip_fail(hipError_t e, const char *what);

// Reset a ring's records from exact segments ([2 G] virtual start, end) and head.
void ring_records(ss_pool *p, int R, const unsigned long long *seg, unsigned long long head) {
  std::vector<int> live;
  for (int g = 0; g < p->G; ++g) {
    p->last_seq[R][g] = -1;
    p->seg_bound[R][g] = (int64_t)(seg[2 * g + 1] - seg[2 * g]);
    if (seg[2 * g + 1] > seg[2 * g]) live.push_back(g);
  }
  std::sort(live.begin(), live.end(), [&](int x, int y) { return seg[2 * x] < seg[2 * y]; });
  p->recs[R].clear();
  unsigned long long at = live.empty() ? head : seg[2 * live[0]];
  for (int g : live) {
    if (seg[2 * g] > at) p->recs[R].push_back({p->seq++, -1, (int64_t)(seg[2 * g] - at)});
    p->last_seq[R][g] = p->seq;
    p->recs[R].push_back({p->seq++, g, (int64_t)(seg[2 * g + 1] - seg[2 * g])});
    at = seg[2 * g + 1];
  }
  if (head > at) p->recs[R].push_back({p->seq++, -1, (int64_t)(head - at)});
}

// Upper bound of head - tail of ring R: the records from the oldest live segment on.
int64_t ring_usage_bound(ss_pool *p, int R) {
  int64_t oldest = INT64_MAX;
  for (int g = 0; g < p->G; ++g)
    if (p->last_seq[R][g] >= 0 && p->seg_bound[R][g] > 0) oldest = std::min(oldest, p->last_seq[R][g]);
  while (!p->recs[R].empty() && p->recs[R].front().seq < oldest) p->recs[R].pop_front();
  int64_t u = 0;
  for (const auto &x : p->recs[R]) u += x.n;
  return u;
}

// Re-pack every factored state's components, exactly, into rings of capacity newcap (after a
// synchronization), with group `first` at the tail.
ss_status ring_repack(ss_pool *p, int first, const int64_t (&newcap)[2], hipStream_t stream) {
  hipError_t e = hipSuccess;
  const int64_t N = p->N;
  const int G = p->G;
  if (!p->lay_cnt) {  // device scratch of the layout, kept for later re-packs
    auto chk = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    chk(dalloc(p, &p->lay_cnt, 6 * (size_t)N));
    chk(dalloc(p, &p->lay_g, 3 * (size_t)G + 1));
    chk(dalloc(p, &p->lay_ord, (size_t)G));
    p->lay_scan_bytes = ss::layout_scan_bytes(N);
    chk(dalloc(p, &p->lay_scan, p->lay_scan_bytes + 1));
    std::vector<int64_t> gs(2 * (size_t)G);
    for (int g = 0; g < G; ++g) {
      gs[g] = p->group_start[g];
      gs[G + g] = p->group_size[g];
    }
    if (e == hipSuccess) e = hipMemcpy(p->lay_g, gs.data(), sizeof(int64_t) * gs.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? fail(SS_ERR_OOM, "ring re-pack scratch") : hip_fail(e, "ring re-pack");
  }
  const std::vector<int> ord = ring_order(p, first);
  std::vector<int64_t> lstart(G + 1, 0);
  for (int k = 0; k < G; ++k) lstart[k + 1] = lstart[k] + p->group_size[ord[k]];
  e = hipMemcpyAsync(p->lay_ord, ord.data(), sizeof(int32_t) * G, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(p->lay_g + 2 * G, lstart.data(), sizeof(int64_t) * (G + 1), hipMemcpyHostToDevice, stream);
  void *blk[2] = {nullptr, nullptr};
  size_t bytes[2] = {0, 0};
  ss::Arena na[2];
  for (int R = 0; R < 2 && e == hipSuccess; ++R) e = ring_alloc(p, newcap[R], &blk[R], &bytes[R], &na[R]);
  ss::LayoutArgs la{};
  la.N = N; la.G = G; la.members = p->members; la.ord = p->lay_ord;
  la.gstart = p->lay_g; la.gsize = p->lay_g + G; la.lstart = p->lay_g + 2 * G; la.meta = p->meta;
  la.cnt_a = p->lay_cnt; la.cnt_f = p->lay_cnt + N; la.off_a = p->lay_cnt + 2 * N; la.off_f = p->lay_cnt + 3 * N;
  la.new_a = p->lay_cnt + 4 * N; la.new_f = p->lay_cnt + 5 * N;
  la.seg = p->seg; la.ring = p->ring; la.scan_tmp = p->lay_scan; la.scan_bytes = p->lay_scan_bytes;
  if (e == hipSuccess) e = ss::launch_ring_layout(la, stream);
  if (e == hipSuccess) {
    ss::RepackArgs ra{};
    ra.N = N; ra.dk = p->dk; ra.dv = p->dv; ra.meta = p->meta;
    ra.src_a = p->act; ra.src_f = p->frz; ra.dst_a = na[0]; ra.dst_f = na[1]; ra.new_a = la.new_a; ra.new_f = la.new_f;
    e = ss::launch_repack(ra, stream);
  }
  std::vector<unsigned long long> seg(4 * (size_t)G);
  ss::Ring ring[2];
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(seg.data(), p->seg, sizeof(unsigned long long) * seg.size(), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(ring, p->ring, sizeof(ring), hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    for (int R = 0; R < 2; ++R)
      if (blk[R]) (void)hipFree(blk[R]);
    return e == hipErrorOutOfMemory ? fail(SS_ERR_OOM, "ring growth: device allocation failed")
                                    : hip_fail(e, "ring repack");
  }
  if (p->ca.inflight) {  // an asynchronous consolidation may still read the old rings
    e = hipEventSynchronize(p->ca.host ? p->ca.read_ev : p->ca.done_ev);
    if (e != hipSuccess) {
      for (int R = 0; R < 2; ++R) (void)hipFree(blk[R]);
      return hip_fail(e, "ring repack: waiting for the consolidation");
    }
  }
  for (int R = 0; R < 2; ++R) {
    (void)hipFree(p->ring_blk[R]);
    p->ring_blk[R] = blk[R];
    p->ring_bytes[R] = bytes[R];
    p->arena(R) = na[R];
    ring_records(p, R, seg.data() + (size_t)R * 2 * G, ring[R].head);
  }
  p->repacks++;
  p->layout_version++;
  return SS_OK;
}

// Before the compactions of groups gs[0..ng) (in that order, with nothing else allocating in
// between): make sure each ring can take their new segments.  A state's new active (frozen) count
// exceeds its old one by at most its pad fill, and is at most r (the frozen capacity), so a
// group's segment bound ab[i][R] is its old bound plus K per member, capped.  The host bounds
// head - tail by the records from the oldest live segment on and synchronizes only when that
// bound plus the new segments could exceed the capacity; it then takes the exact figures from the
// device, and re-packs (growing the ring if the live components need it) only if those leave
// too little room.
ss_status ensure_ring_space(ss_pool *p, const int *gs, int ng, hipStream_t stream, int64_t (*ab)[2]) {
  auto bounds = [&](int64_t (&need)[2]) {
    need[0] = need[1] = 0;
    for (int i = 0; i < ng; ++i) {
      const int64_t n = p->group_size[gs[i]];
      for (int R = 0; R < 2; ++R) {
        ab[i][R] = std::min<int64_t>(n * p->per_state_cap(R), p->seg_bound[R][gs[i]] + (int64_t)p->K * n);
        need[R] += ab[i][R];
      }
    }
  };
  int64_t need[2];
  bounds(need);
  bool sync = false;
  for (int R = 0; R < 2; ++R) sync = sync || ring_usage_bound(p, R) + need[R] > p->arena(R).cap;
  if (!sync) return SS_OK;
  hipError_t e = hipStreamSynchronize(stream);
  ss::Ring ring[2];
  std::vector<unsigned long long> seg(4 * (size_t)p->G);
  if (e == hipSuccess) e = hipMemcpy(ring, p->ring, sizeof(ring), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(seg.data(), p->seg, sizeof(unsigned long long) * seg.size(), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "ring sync");
  p->ring_syncs++;
  int64_t live[2] = {0, 0};
  for (int R = 0; R < 2; ++R) {
    ring_records(p, R, seg.data() + (size_t)R * 2 * p->G, ring[R].head);
    for (int g = 0; g < p->G; ++g) live[R] += p->seg_bound[R][g];
  }
  bounds(need);
  bool repack = false;
  for (int R = 0; R < 2; ++R) repack = repack || ring_usage_bound(p, R) + need[R] > p->arena(R).cap;
  if (!repack) return SS_OK;
  int64_t newcap[2];
  for (int R = 0; R < 2; ++R) {
    // grow to twice what the live components and this step need, when they pass half the ring
    const int64_t want = live[R] + need[R], cap = p->arena(R).cap;
    newcap[R] = 2 * want > cap ? std::max<int64_t>(cap, 2 * want) : cap;
    if (newcap[R] >= (int64_t)INT32_MAX) return fail(SS_ERR_CAPACITY, "a component ring would exceed 2^31 slots");
  }
  const ss_status st = ring_repack(p, gs[0], newcap, stream);
  if (st != SS_OK) return st;
  bounds(need);
  return SS_OK;
}

// check the host-visible error flags that kernels raise
ss_status poll(ss_pool *p) {
  if (p->sticky != SS_OK) return fail(p->sticky, p->sticky_msg);
  if (p->hflags) {
    const volatile uint32_t *f = p->hflags;
    if (f[HF_PAD]) {
      p->sticky = SS_ERR_STATE;
      p->sticky_msg = "decode_step found a full pad: a compaction of the state's group was skipped";
    } else if (f[HF_DENSE_CAP]) {
      p->sticky = SS_ERR_CAPACITY;
      p->sticky_msg = "the dense region is full; raise dense_capacity";
    } else if (f[HF_RING]) {
      p->sticky = SS_ERR_CAPACITY;
      p->sticky_msg = "a component ring was full during a compaction";
    }
  }
  if (p->sticky != SS_OK) return fail(p->sticky, p->sticky_msg);
  return SS_OK;
}

}  // namespace

extern "C" {

int32_t ss_dense_rank_limit(int32_t d_k, int32_t d_v) {
  if (d_k <= 0 || d_v <= 0) return 0;
  return (int32_t)(((int64_t)d_k * d_v) / ((int64_t)d_k + d_v));
}

uint64_t ss_decode_bytes_per_state(int32_t d_k, int32_t d_v, int32_t pad_slots, int32_t n_comp, int32_t n_pad,
                                   int32_t rule, int32_t kind) {
  if (kind < SS_DECODE_FACTORED || kind > SS_DECODE_FACTORED_FP16) return 0;
  if (kind == SS_DECODE_FACTORED_FP16)
    return ss::decode_bytes(d_k, d_v, pad_slots, n_comp, n_pad, rule == SS_RULE_DELTA, ss::KIND_FACTORED, 2);
  return ss::decode_bytes(d_k, d_v, pad_slots, n_comp, n_pad, rule == SS_RULE_DELTA, kind);
}

const char *ss_status_string(ss_status st) {
  switch (st) {
    case SS_OK: return "ok";
    case SS_ERR_ARG: return "invalid argument";
    case SS_ERR_SHAPE: return "unsupported shape";
    case SS_ERR_OOM: return "out of memory";
    case SS_ERR_CAPACITY: return "capacity exhausted";
    case SS_ERR_HIP: return "HIP runtime error";
    case SS_ERR_STATE: return "pool poisoned by an earlier failure";
  }
  return "unknown status";
}

const char *ss_last_error(void) { return g_last_error.c_str(); }

// dense_dev: device [N][d_k][d_v] holding the S of the states init->dense_mask marks (instead of
// the host array init->dense); read in place, never copied to the host
static ss_status pool_create(const ss_pool_desc *d, const ss_init *init, const float *dense_dev, hipStream_t stream,
                             ss_pool **out) {
  if (!out) return fail(SS_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(SS_ERR_ARG, "desc is NULL");
  const int64_t N = d->n_states;
  if (N < 1) return fail(SS_ERR_ARG, "n_states must be >= 1");
  if (d->d_k < 4 || d->d_v < 4 || d->d_k > 256 || d->d_v > 256 || (d->d_k & 3) || (d->d_v & 3))
    return fail(SS_ERR_SHAPE, "d_k and d_v must be multiples of 4 in [4, 256]");
  if (d->pad_slots < 1 || d->pad_slots > 8) return fail(SS_ERR_SHAPE, "pad_slots must be in [1, 8]");
  if (d->r_active < 1 || d->r_active > 8) return fail(SS_ERR_SHAPE, "r_active must be in [1, 8]");
  if (d->r_active + d->pad_slots > ss::kMaxM) return fail(SS_ERR_SHAPE, "r_active + pad_slots must be <= 16");
  if (d->n_groups < 1) return fail(SS_ERR_ARG, "n_groups must be >= 1");
  if (d->max_frozen < 0 || d->max_frozen > 255) return fail(SS_ERR_ARG, "max_frozen must be in [0, 255]");
  if (d->dense_capacity < 0 || d->dense_capacity > N) return fail(SS_ERR_ARG, "dense_capacity must be in [0, N]");
  const int dk = d->d_k, dv = d->d_v, K = d->pad_slots, r = d->r_active, G = d->n_groups;
  const int L = d->dense_rank_limit < 0 ? ss_dense_rank_limit(dk, dv) : d->dense_rank_limit;
  if (L > 255 + r) return fail(SS_ERR_ARG, "dense_rank_limit too large (frozen part is limited to 255)");
  const int promote = d->promote_on_compact ? 1 : 0;
  int fcap = promote ? std::max(1, std::min(255, L + K - r)) : (d->max_frozen ? d->max_frozen : 255);
  if (d->group_offset)
    for (int g = 0; g < G; ++g)
      if (d->group_offset[g] < 0 || d->group_offset[g] >= K) return fail(SS_ERR_ARG, "group_offset out of [0, K)");
  std::vector<int32_t> grp(N, 0);
  if (d->group_of_state) {
    for (int64_t s = 0; s < N; ++s) {
      if (d->group_of_state[s] < 0 || d->group_of_state[s] >= G) return fail(SS_ERR_ARG, "group_of_state out of range");
      grp[s] = d->group_of_state[s];
    }
  }
  bool any_delta = false;
  if (d->rule)
    for (int64_t s = 0; s < N; ++s) {
      if (d->rule[s] > 1) return fail(SS_ERR_ARG, "rule must be 0 (scalar) or 1 (delta)");
      any_delta |= d->rule[s] == 1;
    }
  if (d->eps) {
    for (int64_t s = 0; s < N; ++s)
      if (!(d->eps[s] >= 0.f) || !std::isfinite(d->eps[s])) return fail(SS_ERR_ARG, "eps must be finite and >= 0");
  } else if (!(d->eps_default >= 0.f) || !std::isfinite(d->eps_default)) {
    return fail(SS_ERR_ARG, "eps_default must be finite and >= 0");
  }
  // initial components
  const int64_t *off = (init && init->comp_off) ? init->comp_off : nullptr;
  int64_t total = 0, n_dense0 = 0;
  if (off) {
    if (off[0] != 0) return fail(SS_ERR_ARG, "comp_off[0] must be 0");
    for (int64_t s = 0; s < N; ++s) {
      const int64_t R = off[s + 1] - off[s];
      if (R < 0) return fail(SS_ERR_ARG, "comp_off must be non-decreasing");
      if (!d->force_dense && R <= L && R - std::min<int64_t>(R, r) > fcap)
        return fail(SS_ERR_CAPACITY, "initial frozen part exceeds max_frozen");
      if (d->force_dense || R > L) ++n_dense0;
    }
    total = off[N];
    if (total > 0 && (!init->u || !init->v || !init->sigma)) return fail(SS_ERR_ARG, "u, v and sigma are required");
    for (int64_t s = 0; s < N; ++s)
      for (int64_t c = off[s] + 1; c < off[s + 1]; ++c)
        if (!(init->sigma[c] <= init->sigma[c - 1])) return fail(SS_ERR_ARG, "sigma must be sorted descending per state");
    for (int64_t c = 0; c < total; ++c)
      if (!std::isfinite(init->sigma[c]) || init->sigma[c] < 0.f) return fail(SS_ERR_ARG, "sigma must be finite, >= 0");
  } else if (d->force_dense) {
    n_dense0 = N;
  }
  // states given dense
  const uint8_t *dmask = (init && init->dense_mask) ? init->dense_mask : nullptr;
  int64_t n_given = 0;
  if (dmask) {
    for (int64_t s = 0; s < N; ++s) {
      if (!dmask[s]) continue;
      if (off && off[s + 1] != off[s]) return fail(SS_ERR_ARG, "a state given dense must have no components");
      ++n_given;
      if (!d->force_dense) ++n_dense0;  // (force_dense already counts every state)
    }
    if (n_given > 0 && !init->dense && !dense_dev) return fail(SS_ERR_ARG, "dense is required when dense_mask marks states");
    if (!off && !d->force_dense) n_dense0 = n_given;
  }
  auto given = [&](int64_t s) { return dmask && dmask[s]; };
  const int64_t cap_d = d->force_dense ? N : (d->dense_capacity ? d->dense_capacity : N);
  if (n_dense0 > cap_d) return fail(SS_ERR_CAPACITY, "more initial dense states than dense_capacity");
  const bool factored = !d->force_dense;
  if (d->arena_components < 0 || d->arena_components >= (int64_t)INT32_MAX)
    return fail(SS_ERR_ARG, "arena_components must be in [0, 2^31)");
  if (d->factor_fp16 != 0 && d->factor_fp16 != 1) return fail(SS_ERR_ARG, "factor_fp16 must be 0 or 1");
  if (d->diag_decay != 0 && d->diag_decay != 1) return fail(SS_ERR_ARG, "diag_decay must be 0 or 1");

  ss_pool *p = new (std::nothrow) ss_pool();
  if (!p) return fail(SS_ERR_OOM, "host allocation failed");
  p->N = N; p->dk = dk; p->dv = dv; p->K = K; p->r = r; p->L = L; p->promote = promote;
  p->force_dense = d->force_dense ? 1 : 0; p->half = d->factor_fp16; p->diag = d->diag_decay; p->fcap = fcap; p->G = G; p->any_delta = any_delta; p->cap_d = cap_d;
  p->group_offset.assign(G, 0);
  if (d->group_offset) for (int g = 0; g < G; ++g) p->group_offset[g] = d->group_offset[g];
  p->group_size.assign(G, 0);
  p->group_start.assign(G, 0);
  for (int64_t s = 0; s < N; ++s) p->group_size[grp[s]]++;
  for (int g = 1; g < G; ++g) p->group_start[g] = p->group_start[g - 1] + p->group_size[g - 1];
  std::vector<int32_t> &members = p->members_host;
  members.assign(N, 0);
  {
    std::vector<int64_t> fill(p->group_start);
    for (int64_t s = 0; s < N; ++s) members[fill[grp[s]]++] = (int32_t)s;
  }
  std::vector<int64_t> zero_off;
  if (!off) zero_off.assign(N + 1, 0);
  const int64_t *offp = off ? off : zero_off.data();
  // ring layout: the factored states' components, group by group in the order the groups fall due
  std::vector<int64_t> pos[2];
  std::vector<unsigned long long> seg;
  int64_t tot[2] = {0, 0}, cap_ring[2] = {0, 0};
  if (factored) {
    std::vector<int32_t> cnt[2] = {std::vector<int32_t>(N, -1), std::vector<int32_t>(N, -1)};
    for (int64_t s = 0; s < N; ++s) {
      const int64_t R = offp[s + 1] - offp[s];
      if (R > L || given(s)) continue;
      cnt[0][s] = (int32_t)std::min<int64_t>(R, r);
      cnt[1][s] = (int32_t)(R - cnt[0][s]);
    }
    ring_layout(p, ring_order(p, -1), cnt, pos, seg, tot);
    // Automatic capacity.  No ring ever needs more than (factored states + one group) times the
    // per-state cap (r active; L + K - r, or max_frozen, frozen).  Growing a ring later costs a
    // device allocation, and large ones are slow (tens of ms per GB here), so when that maximum
    // fits in a quarter of the free device memory it is reserved at once; otherwise the active
    // ring starts at its maximum and the frozen ring at twice its contents plus one group's
    // growth, and they grow when needed.  Either way a state's slot never exceeds its cap.
    int64_t nf = 0, ngmax = 0;
    for (int g = 0; g < G; ++g) ngmax = std::max(ngmax, p->group_size[g]);
    for (int64_t s = 0; s < N; ++s) nf += cnt[0][s] >= 0 ? 1 : 0;
    const int64_t cbytes = (int64_t)(d->factor_fp16 ? 2 : 4) * (dk + dv) + 4;
    int64_t maxcap[2];
    for (int R = 0; R < 2; ++R) maxcap[R] = (nf + ngmax) * (R == 0 ? (int64_t)r : (int64_t)fcap);
    size_t free_b = 0, total_b = 0;
    const bool roomy = hipMemGetInfo(&free_b, &total_b) == hipSuccess &&
                       (maxcap[0] + maxcap[1]) * cbytes <= (int64_t)(free_b / 4) &&
                       maxcap[1] < (int64_t)INT32_MAX;
    for (int R = 0; R < 2; ++R) {
      const int64_t autocap = R == 0 || roomy ? maxcap[R] : 2 * (tot[1] + (int64_t)K * ngmax);
      cap_ring[R] = std::max<int64_t>({1, tot[R], d->arena_components ? d->arena_components : autocap});
      if (cap_ring[R] >= (int64_t)INT32_MAX) return fail(SS_ERR_CAPACITY, "too many components for 32-bit offsets");
    }
    // a compaction sums its members' slots in 32 bits per ring
    if (ngmax * (int64_t)std::max(r, fcap) >= (int64_t)INT32_MAX)
      return fail(SS_ERR_CAPACITY, "a compaction group holds too many components for 32-bit slot sums");
  }
  std::vector<float> &epsv = p->eps_host;
  epsv.assign(N, 0.f);
  for (int64_t s = 0; s < N; ++s) epsv[s] = d->eps ? d->eps[s] : d->eps_default;
  std::vector<uint8_t> rulev(N, 0);
  if (d->rule) std::memcpy(rulev.data(), d->rule, N);

  // device allocations
  hipError_t e = hipSuccess;
  auto chk = [&](hipError_t x) { if (e == hipSuccess) e = x; };
  chk(dalloc(p, &p->meta, N));
  chk(dalloc(p, &p->members, N));
  chk(dalloc(p, &p->eps, N));
  if (factored) {
    for (int R = 0; R < 2; ++R) chk(ring_alloc(p, cap_ring[R], &p->ring_blk[R], &p->ring_bytes[R], &p->arena(R)));
    chk(dalloc(p, &p->ring, 2));
    chk(dalloc(p, &p->seg, 4 * (size_t)G));
    int64_t gmax = 0;
    for (int g = 0; g < G; ++g) gmax = std::max(gmax, p->group_size[g]);
    chk(dalloc(p, &p->slot_in, (size_t)gmax + 1));
    chk(dalloc(p, &p->slot_blk, (size_t)(gmax + ss::kSlotBlock - 1) / ss::kSlotBlock + 1));
    chk(dalloc(p, &p->pk, (size_t)N * K * dk));
    chk(dalloc(p, &p->pw, (size_t)N * K * dv));
    chk(dalloc(p, &p->pc, (size_t)N * K));
    chk(dalloc(p, &p->promote_list, N));
    chk(dalloc(p, &p->fact_ids[0], N));
    chk(dalloc(p, &p->fact_ids[1], N));
  }
  chk(dalloc(p, &p->dense, (size_t)cap_d * dk * dv));
  chk(dalloc(p, &p->dslot, cap_d));
  if (factored) {
    chk(dalloc(p, &p->dpk, (size_t)cap_d * K * dk));
    chk(dalloc(p, &p->dpw, (size_t)cap_d * K * dv));
    chk(dalloc(p, &p->dpc, (size_t)cap_d * K));
    if (p->diag) {
      chk(dalloc(p, &p->gam, (size_t)N * dk));
      chk(dalloc(p, &p->dgam, (size_t)cap_d * dk));
    }
  }
  chk(dalloc(p, &p->counters, ss::C_N));
  chk(dalloc(p, &p->acct, ss::A_N * ss::kAcctSlots));
  if (e == hipSuccess) {
    void *h = nullptr;
    e = hipHostMalloc(&h, HF_N * sizeof(uint32_t), hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) {
      p->hflags = static_cast<uint32_t *>(h);
      std::memset(p->hflags, 0, HF_N * sizeof(uint32_t));
      void *dp = nullptr;
      e = hipHostGetDevicePointer(&dp, h, 0);
      p->hflags_dev = static_cast<uint32_t *>(dp);
    }
  }
  if (e != hipSuccess) {
    const bool oom = e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation;
    free_all(p);
    delete p;
    return oom ? fail(SS_ERR_OOM, "device allocation failed") : hip_fail(e, "allocation");
  }
  // temporaries for the initial upload
  int64_t *d_off = nullptr;
  float *d_u = nullptr, *d_v = nullptr, *d_s = nullptr;
  int32_t *d_dlist = nullptr;
  int64_t *d_pos[2] = {nullptr, nullptr};
  uint8_t *d_rule = nullptr;
  std::vector<void *> tmp;
  auto talloc = [&](void **q, size_t bytes) {
    if (e != hipSuccess || bytes == 0) return;
    e = hipMalloc(q, bytes);
    if (e == hipSuccess) tmp.push_back(*q);
  };
  talloc((void **)&d_off, (N + 1) * sizeof(int64_t));
  talloc((void **)&d_u, total * dk * sizeof(float));
  talloc((void **)&d_v, total * dv * sizeof(float));
  talloc((void **)&d_s, total * sizeof(float));
  talloc((void **)&d_dlist, N * sizeof(int32_t));
  uint8_t *d_mask = nullptr;
  int64_t *d_didx = nullptr;
  float *d_dsrc = nullptr;
  std::vector<int64_t> didx;
  std::vector<float> dense_pack;
  if (n_given > 0) {
    talloc((void **)&d_mask, N);
    talloc((void **)&d_didx, N * sizeof(int64_t));
    didx.assign(N, -1);
    if (dense_dev) {  // read where it is: state s at row s
      d_dsrc = const_cast<float *>(dense_dev);
      for (int64_t s = 0; s < N; ++s)
        if (dmask[s]) didx[s] = s;
    } else {
      talloc((void **)&d_dsrc, (size_t)n_given * dk * dv * sizeof(float));
      int64_t k = 0;
      for (int64_t s = 0; s < N; ++s)
        if (dmask[s]) didx[s] = k++;
    }
  }
  if (factored)
    for (int R = 0; R < 2; ++R) talloc((void **)&d_pos[R], N * sizeof(int64_t));
  talloc((void **)&d_rule, N);
  auto up = [&](void *dst, const void *src, size_t bytes) {
    if (e == hipSuccess && bytes) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, stream);
  };
  up(d_off, offp, (N + 1) * sizeof(int64_t));
  if (total) {
    up(d_u, init->u, total * dk * sizeof(float));
    up(d_v, init->v, total * dv * sizeof(float));
    up(d_s, init->sigma, total * sizeof(float));
  }
  ss::Ring ring0[2] = {};
  if (factored) {
    for (int R = 0; R < 2; ++R) {
      up(d_pos[R], pos[R].data(), N * sizeof(int64_t));
      ring0[R].head = ring0[R].begin = (unsigned long long)tot[R];
    }
    up(p->ring, ring0, sizeof(ring0));
    up(p->seg, seg.data(), seg.size() * sizeof(unsigned long long));
  }
  up(d_rule, rulev.data(), N);
  if (n_given > 0) {
    up(d_mask, dmask, N);
    up(d_didx, didx.data(), N * sizeof(int64_t));
    const size_t per = (size_t)dk * dv;
    if (dense_dev) {
      // nothing to upload
    } else if (n_given == N) {
      up(d_dsrc, init->dense, sizeof(float) * per * N);
    } else {  // the given states' S, packed in state order (the upload is synchronized below)
      dense_pack.resize(per * n_given);
      for (int64_t s = 0; s < N; ++s)
        if (dmask[s]) std::memcpy(dense_pack.data() + (size_t)didx[s] * per, init->dense + (size_t)s * per, sizeof(float) * per);
      up(d_dsrc, dense_pack.data(), sizeof(float) * dense_pack.size());
    }
  }
  up(p->members, members.data(), N * sizeof(int32_t));
  up(p->eps, epsv.data(), N * sizeof(float));
  if (e == hipSuccess) e = hipMemsetAsync(p->counters, 0, ss::C_N * sizeof(uint32_t), stream);
  if (e == hipSuccess) e = hipMemsetAsync(p->acct, 0, ss::A_N * ss::kAcctSlots * sizeof(unsigned long long), stream);
  std::vector<int32_t> fact;
  if (factored) {
    fact.reserve(N);
    for (int64_t s2 = 0; s2 < N; ++s2)
      if (offp[s2 + 1] - offp[s2] <= L && !given(s2)) fact.push_back((int32_t)s2);
    p->fact_count_host = (uint32_t)fact.size();
    up(p->fact_ids[0], fact.data(), fact.size() * sizeof(int32_t));
    up(p->counters + ss::C_FACT0, &p->fact_count_host, sizeof(uint32_t));
  }
  if (e == hipSuccess) {
    ss::ScatterArgs sa{};
    sa.N = N; sa.dk = dk; sa.dv = dv; sa.r = r; sa.L = L; sa.fcap = fcap; sa.force_dense = p->force_dense;
    sa.csr_off = d_off; sa.csr_u = d_u; sa.csr_v = d_v; sa.csr_s = d_s;
    sa.dst_a = d_pos[0]; sa.dst_f = d_pos[1]; sa.rule = d_rule; sa.dense_mask = d_mask;
    sa.meta = p->meta; sa.act = p->act; sa.frz = p->frz; sa.dense_list = d_dlist; sa.counters = p->counters;
    e = ss::launch_scatter(sa, stream);
  }
  if (e == hipSuccess && n_dense0 > 0) {
    ss::MaterializeArgs ma{};
    ma.dk = dk; ma.dv = dv; ma.cap_d = (int)cap_d; ma.list = d_dlist; ma.count = p->counters + ss::C_PROMOTE_COUNT;
    ma.meta = p->meta; ma.csr_off = d_off; ma.csr_u = d_u; ma.csr_v = d_v; ma.csr_s = d_s;
    ma.dsrc_idx = d_didx; ma.dsrc = d_dsrc;
    ma.act = p->act; ma.frz = p->frz; ma.dense = p->dense; ma.dslot = p->dslot; ma.counters = p->counters;
    ma.hflag = p->hflags_dev + HF_DENSE_CAP; ma.dgam = p->dgam;
    e = ss::launch_materialize(ma, n_dense0, stream);
  }
  if (e == hipSuccess && p->gam) e = ss::launch_fill_f32(p->gam, N * (int64_t)dk, 1.0f, stream);
  if (e == hipSuccess) e = ss::launch_zero_u32(p->counters + ss::C_PROMOTE_COUNT, 1, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  for (void *q : tmp) (void)hipFree(q);
  if (e != hipSuccess) {
    free_all(p);
    delete p;
    return hip_fail(e, "pool upload");
  }
  p->dense_upper = n_dense0;
  p->fact_upper = factored ? (int64_t)fact.size() : 0;
  for (int R = 0; R < 2; ++R) {
    p->last_seq[R].assign(G, -1);
    p->seg_bound[R].assign(G, 0);
    if (factored) ring_records(p, R, seg.data() + (size_t)R * 2 * G, (unsigned long long)tot[R]);
  }
  p->cons_wait.assign(G, 0);
  p->cons_last.assign(G, -1);
  if (p->hflags) p->hflags[HF_FACT] = (uint32_t)p->fact_upper;
  *out = p;
  return SS_OK;
}

ss_status ss_state_pool_create(const ss_pool_desc *d, const ss_init *init, hipStream_t stream, ss_pool **out) {
  return pool_create(d, init, nullptr, stream, out);
}

ss_status ss_state_pool_create_from_dense(const ss_pool_desc *d, const float *S, const float *u, const float *v,
                                          const float *sigma, const int32_t *rank, int32_t max_rank,
                                          hipStream_t stream, ss_pool **out) {
  if (!out) return fail(SS_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!d) return fail(SS_ERR_ARG, "desc is NULL");
  const int64_t N = d->n_states;
  if (N < 1) return fail(SS_ERR_ARG, "n_states must be >= 1");
  if (d->d_k < 4 || d->d_v < 4 || d->d_k > 256 || d->d_v > 256 || (d->d_k & 3) || (d->d_v & 3))
    return fail(SS_ERR_SHAPE, "d_k and d_v must be multiples of 4 in [4, 256]");
  const int dk = d->d_k, dv = d->d_v;
  if (max_rank < 1 || max_rank > std::min(dk, dv)) return fail(SS_ERR_ARG, "max_rank must be in [1, min(d_k, d_v)]");
  if (!S || !u || !v || !sigma || !rank) return fail(SS_ERR_ARG, "null pointer");
  if (d->force_dense) return fail(SS_ERR_ARG, "a pool built from factors cannot be force_dense");
  const int L = d->dense_rank_limit < 0 ? ss_dense_rank_limit(dk, dv) : d->dense_rank_limit;
  const size_t M = (size_t)max_rank;
  std::vector<int32_t> rk(N);
  std::vector<float> hs((size_t)N * M), hu, hv;
  try {
    hu.resize((size_t)N * M * dk);
    hv.resize((size_t)N * M * dv);
  } catch (const std::bad_alloc &) {
    return fail(SS_ERR_OOM, "host allocation failed");
  }
  hipError_t e = hipMemcpyAsync(rk.data(), rank, N * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(hs.data(), sigma, hs.size() * sizeof(float), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(hu.data(), u, hu.size() * sizeof(float), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(hv.data(), v, hv.size() * sizeof(float), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading the initialization results");
  // the dense fallback ([SS] 4.4 "Memory layout": decided once the state is factored): rank > L
  // keeps the state's exact S; the others keep their components in descending sigma (the blocks
  // are each descending, not across blocks; ties keep block order)
  std::vector<int64_t> off(N + 1, 0);
  std::vector<uint8_t> dmask(N, 0);
  int64_t n_dense = 0;
  for (int64_t s = 0; s < N; ++s) {
    if (rk[s] < 0 || rk[s] > max_rank) return fail(SS_ERR_ARG, "rank out of [0, max_rank]");
    const bool dn = rk[s] > L;
    dmask[s] = dn ? 1 : 0;
    n_dense += dn ? 1 : 0;
    off[s + 1] = off[s] + (dn ? 0 : rk[s]);
  }
  std::vector<float> cu((size_t)off[N] * dk), cv((size_t)off[N] * dv), cs((size_t)off[N]);
  std::vector<int> ord;
  for (int64_t s = 0; s < N; ++s) {
    if (dmask[s]) continue;
    const int R = rk[s];
    const float *sg = hs.data() + (size_t)s * M;
    ord.resize(R);
    for (int i = 0; i < R; ++i) ord[i] = i;
    std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return sg[a] > sg[b]; });
    for (int i = 0; i < R; ++i) {
      const size_t src = (size_t)s * M + ord[i], dst = (size_t)off[s] + i;
      std::memcpy(cu.data() + dst * dk, hu.data() + src * dk, dk * sizeof(float));
      std::memcpy(cv.data() + dst * dv, hv.data() + src * dv, dv * sizeof(float));
      cs[dst] = sg[ord[i]];
    }
  }
  ss_init in{};
  in.comp_off = off.data();
  in.u = cu.data();
  in.v = cv.data();
  in.sigma = cs.data();
  in.dense_mask = n_dense ? dmask.data() : nullptr;
  in.dense = nullptr;
  return pool_create(d, &in, S, stream, out);
}

ss_status ss_state_pool_destroy(ss_pool *p) {
  if (!p) return SS_OK;
  if (p->ca.worker.joinable()) p->ca.worker.join();
  (void)hipDeviceSynchronize();
  if (p->ca.snap_ev) (void)hipEventDestroy(p->ca.snap_ev);
  if (p->ca.done_ev) (void)hipEventDestroy(p->ca.done_ev);
  if (p->ca.read_ev) (void)hipEventDestroy(p->ca.read_ev);
  if (p->ca.dl_ev) (void)hipEventDestroy(p->ca.dl_ev);
  if (p->ca.own_side) (void)hipStreamDestroy(p->ca.own_side);
  for (void *h : {(void *)p->ca.h_u, (void *)p->ca.h_v, (void *)p->ca.h_s, (void *)p->ca.h_s0, (void *)p->ca.h_eps,
                  (void *)p->ca.h_cnt})
    if (h) (void)hipHostFree(h);
  free_all(p);
  delete p;
  return SS_OK;
}

// Enqueue the decode (or read-only readout) of every state.  fact_grid / dense_grid bound the
// factored-state list and the dense slots in use (the kernels read the exact counts on the device).
static hipError_t enqueue_decode(ss_pool *p, const float *q, const float *k, const float *v, const float *alpha,
                                 const float *beta, float *o, bool readonly, int64_t fact_grid, int64_t dense_grid,
                                 bool timing, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (!p->force_dense && fact_grid > 0) {
    ss::DecodeArgs a{};
    a.N = fact_grid; a.dk = p->dk; a.dv = p->dv; a.K = p->K; a.meta = p->meta; a.act = p->act; a.frz = p->frz;
    a.fact_ids = p->fact_ids[0]; a.fact_count = p->counters + ss::C_FACT0; a.n_states = p->N;
    a.pk = p->pk; a.pw = p->pw; a.pc = p->pc; a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.o = o;
    a.counters = p->counters; a.acct = p->acct + ss::A_DECODE_FACTORED * ss::kAcctSlots;
    a.hflag = p->hflags_dev + HF_PAD; a.gam = p->gam;
    auto fn = [&] { return ss::launch_decode_factored(a, readonly, p->any_delta, stream); };
    e = timing ? timed(p, readonly ? SS_KERNEL_READOUT_FACTORED : SS_KERNEL_DECODE_FACTORED, stream, fn) : fn();
    if (e != hipSuccess) return e;
  }
  if (dense_grid > 0) {
    ss::DenseArgs a{};
    a.dk = p->dk; a.dv = p->dv; a.K = p->K; a.cap_d = (uint32_t)p->cap_d; a.meta = p->meta; a.dense = p->dense;
    a.dslot = p->dslot; a.pk = p->dpk; a.pw = p->dpw; a.pc = p->dpc;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.o = o;
    a.counters = p->counters; a.acct = p->acct + ss::A_DECODE_DENSE * ss::kAcctSlots;
    a.diag = p->diag; a.dgam = p->dgam;
    auto fn = [&] { return ss::launch_decode_dense(a, dense_grid, readonly, p->any_delta, stream); };
    e = timing ? timed(p, readonly ? SS_KERNEL_READOUT_DENSE : SS_KERNEL_DECODE_DENSE, stream, fn) : fn();
  }
  return e;
}

// Enqueue the compaction of group g (the ring space must have been checked): fold the pads of its
// dense members, compact its factored members into a new ring segment, promote.  with_dense:
// whether dense members may exist.

// Largest frozen count a factored state of the pool can hold: with promotion a state keeps at
// most L components, r of them active; without, the per-state frozen capacity.
static int frozen_max(const ss_pool *p) {
  return p->promote ? std::max(0, std::min(p->fcap, p->L - p->r)) : p->fcap;
}

// with_factored: whether factored members may exist; without them only the dense fold runs (the
// pool's factored states are all gone dense, and states never return to factored form).
static hipError_t enqueue_compact_group(ss_pool *p, int g, bool with_dense, bool with_factored, bool timing,
                                        hipStream_t stream, const uint8_t *sel = nullptr) {
  if (!with_factored) {
    if (!with_dense) return hipSuccess;
    ss::DenseArgs da{};
    da.dk = p->dk; da.dv = p->dv; da.K = p->K; da.cap_d = (uint32_t)p->cap_d; da.meta = p->meta;
    da.dense = p->dense; da.dslot = p->dslot; da.pk = p->dpk; da.pw = p->dpw; da.pc = p->dpc;
    da.members = p->members + p->group_start[g]; da.n_members = (int32_t)p->group_size[g];
    da.counters = p->counters; da.acct = p->acct; da.diag = p->diag; da.dgam = p->dgam; da.sel = sel;
    auto fn = [&] { return ss::launch_dense_fold(da, stream); };
    return timing ? timed(p, SS_KERNEL_DENSE_FOLD, stream, fn) : fn();
  }
  ss::RingBeginArgs rb{};
  rb.ring_a = p->ring; rb.ring_f = p->ring + 1; rb.seg_a = p->seg; rb.seg_f = p->seg + 2 * p->G; rb.n_groups = p->G;
  rb.cap_a = p->act.cap; rb.cap_f = p->frz.cap; rb.counters = p->counters;
  rb.members = p->members + p->group_start[g]; rb.n_members = (int)p->group_size[g]; rb.meta = p->meta;
  rb.r = p->r; rb.fcap = p->fcap; rb.slot_in = p->slot_in; rb.slot_blk = p->slot_blk;
  rb.hflag = p->hflags_dev + HF_RING;
  hipError_t e = ss::launch_ring_begin(rb, stream);
  if (e != hipSuccess) return e;
  if (with_dense) {
    ss::DenseArgs da{};
    da.dk = p->dk; da.dv = p->dv; da.K = p->K; da.cap_d = (uint32_t)p->cap_d; da.meta = p->meta;
    da.dense = p->dense; da.dslot = p->dslot; da.pk = p->dpk; da.pw = p->dpw; da.pc = p->dpc;
    da.members = p->members + p->group_start[g]; da.n_members = (int32_t)p->group_size[g];
    da.counters = p->counters; da.acct = p->acct; da.diag = p->diag; da.dgam = p->dgam; da.sel = sel;
    auto fn = [&] { return ss::launch_dense_fold(da, stream); };
    e = timing ? timed(p, SS_KERNEL_DENSE_FOLD, stream, fn) : fn();
    if (e != hipSuccess) return e;
  }
  ss::CompactArgs a{};
  a.dk = p->dk; a.dv = p->dv; a.K = p->K; a.r = p->r; a.L = p->L; a.promote = p->promote; a.fcap = p->fcap;
  a.n_members = (int32_t)p->group_size[g];
  a.members = p->members + p->group_start[g];
  a.eps = p->eps; a.meta = p->meta; a.act = p->act; a.frz = p->frz;
  a.ring_a = p->ring; a.ring_f = p->ring + 1; a.hflag = p->hflags_dev + HF_RING;
  a.slot_in = p->slot_in; a.slot_blk = p->slot_blk;
  a.pk = p->pk; a.pw = p->pw; a.pc = p->pc; a.promote_list = p->promote_list; a.counters = p->counters;
  a.acct_flops = p->acct + ss::A_COMPACT_FLOPS * ss::kAcctSlots;
  a.acct_states = p->acct + ss::A_COMPACT_STATES * ss::kAcctSlots;
  a.gam = p->gam; a.sel = sel;
  auto fc = [&] { return ss::launch_compact(a, stream); };
  e = timing ? timed(p, SS_KERNEL_COMPACT, stream, fc) : fc();
  if (e == hipSuccess) e = ss::launch_ring_end(p->ring, p->ring + 1, p->seg, p->seg + 2 * p->G, g, stream);
  if (e != hipSuccess || !p->promote) return e;
  ss::MaterializeArgs ma{};
  ma.dk = p->dk; ma.dv = p->dv; ma.cap_d = (int)p->cap_d; ma.list = p->promote_list;
  ma.count = p->counters + ss::C_PROMOTE_COUNT; ma.meta = p->meta; ma.act = p->act; ma.frz = p->frz;
  ma.dense = p->dense; ma.dslot = p->dslot; ma.counters = p->counters;
  ma.hflag = p->hflags_dev + HF_DENSE_CAP; ma.dgam = p->dgam;
  const int64_t gsz = p->group_size[g];
  auto fm = [&] { return ss::launch_materialize(ma, gsz, stream); };
  return timing ? timed(p, SS_KERNEL_MATERIALIZE, stream, fm) : fm();
}

// promoted states leave the factored-state list
static hipError_t enqueue_prune(ss_pool *p, int64_t fact_grid, hipStream_t stream) {
  return ss::launch_prune_factored(p->fact_ids[0], p->counters + ss::C_FACT0, p->fact_ids[1],
                                   p->counters + ss::C_FACT1, fact_grid, p->meta, p->hflags_dev + HF_FACT, stream);
}

// host bookkeeping after the compaction of group g was enqueued with segment bounds ab (ab == nullptr:
// only the dense fold ran, the rings and the factored states are untouched)
static void after_compact_group(ss_pool *p, int g, const int64_t (*ab)[2]) {
  p->cons_wait[g] = 1;
  if (p->ca.inflight && p->ca.group == g) p->ca.stale = true;  // its snapshot no longer describes the group
  if ((int)p->ca.last_compact.size() < p->G) p->ca.last_compact.assign(p->G, -1);
  p->ca.last_compact[g] = p->ca.compact_seq++;
  if (!ab) return;
  for (int R = 0; R < 2; ++R) {  // the group's new segment, by its bound
    p->last_seq[R][g] = p->seq;
    p->seg_bound[R][g] = (*ab)[R];
    p->recs[R].push_back({p->seq++, g, (*ab)[R]});
  }
  if (p->promote) p->dense_upper = std::min<int64_t>(p->cap_d, p->dense_upper + p->group_size[g]);
}

static void refresh_fact_upper(ss_pool *p) {
  if (p->hflags) {  // a stale value is still an upper bound: the list only shrinks
    const uint32_t seen = ((const volatile uint32_t *)p->hflags)[HF_FACT];
    p->fact_upper = std::min<int64_t>(p->fact_upper, seen);
  }
}

static ss_status run_decode(ss_pool *p, const float *q, const float *k, const float *v, const float *alpha,
                            const float *beta, float *o, bool readonly, hipStream_t stream) {
  if (!p) return fail(SS_ERR_ARG, "pool is NULL");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (!q || !o) return fail(SS_ERR_ARG, "q and o are required");
  if (!readonly && (!k || !v || !alpha)) return fail(SS_ERR_ARG, "k, v and alpha are required");
  if (!readonly && p->any_delta && !beta) return fail(SS_ERR_ARG, "beta is required: the pool has delta-rule states");
  refresh_fact_upper(p);
  const hipError_t e = enqueue_decode(p, q, k, v, alpha, beta, o, readonly, p->fact_upper, p->dense_upper, true, stream);
  return e == hipSuccess ? SS_OK : hip_fail(e, "decode launch");
}

ss_status ss_decode_step(ss_pool *p, const float *q, const float *k, const float *v, const float *alpha,
                         const float *beta, float *o, hipStream_t stream) {
  ss_status st = run_decode(p, q, k, v, alpha, beta, o, false, stream);
  if (st == SS_OK) p->decode_calls++;
  return st;
}

ss_status ss_readout(ss_pool *p, const float *q, float *o, hipStream_t stream) {
  ss_status st = run_decode(p, q, nullptr, nullptr, nullptr, nullptr, o, true, stream);
  if (st == SS_OK) p->readout_calls++;
  return st;
}

ss_status ss_compact(ss_pool *p, int32_t group, hipStream_t stream) {
  if (!p) return fail(SS_ERR_ARG, "pool is NULL");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (group >= p->G) return fail(SS_ERR_ARG, "group out of range");
  if (p->force_dense) return SS_OK;  // dense states have no pad to compact
  const int g0 = group < 0 ? 0 : group, g1 = group < 0 ? p->G : group + 1;
  bool any = false;
  refresh_fact_upper(p);
  const bool fact = p->fact_upper > 0;  // otherwise every state is dense: only the folds run
  for (int g = g0; g < g1; ++g) {
    if (p->group_size[g] == 0) continue;
    any = true;
    int64_t ab[1][2];
    if (fact) {
      st = ensure_ring_space(p, &g, 1, stream, ab);
      if (st != SS_OK) return st;
    }
    const hipError_t e = enqueue_compact_group(p, g, p->dense_upper > 0, fact, true, stream);
    if (e != hipSuccess) return hip_fail(e, "compact launch");
    after_compact_group(p, g, fact ? ab : nullptr);
  }
  refresh_fact_upper(p);
  if (any && p->promote && p->fact_upper > 0 && p->prune_due++ % kPruneEvery == 0) {
    const hipError_t e = enqueue_prune(p, p->fact_upper, stream);
    if (e != hipSuccess) return hip_fail(e, "factored-list launch");
  }
  p->compact_calls++;
  return SS_OK;
}

ss_status ss_compact_ids(ss_pool *p, const int32_t *ids, int64_t n, hipStream_t stream) {
  if (!p || n < 0 || (n > 0 && !ids)) return fail(SS_ERR_ARG, "bad arguments");
  for (int64_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= p->N) return fail(SS_ERR_ARG, "state id out of range");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (p->force_dense || n == 0) return SS_OK;
  std::vector<uint8_t> mask(p->N, 0);
  std::vector<char> touched(p->G, 0);
  std::vector<int32_t> grp(p->N);
  for (int g = 0; g < p->G; ++g)
    for (int64_t i = 0; i < p->group_size[g]; ++i) grp[p->members_host[p->group_start[g] + i]] = g;
  for (int64_t i = 0; i < n; ++i) {
    mask[ids[i]] = 1;
    touched[grp[ids[i]]] = 1;
  }
  hipError_t e = hipSuccess;
  if (!p->sel) {
    e = dalloc(p, &p->sel, (size_t)p->N);
    if (e != hipSuccess) return e == hipErrorOutOfMemory ? fail(SS_ERR_OOM, "selection mask") : hip_fail(e, "selection mask");
  }
  e = hipStreamSynchronize(stream);  // the previous mask may still be read by enqueued work
  if (e == hipSuccess) e = hipMemcpy(p->sel, mask.data(), (size_t)p->N, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "selection mask upload");
  bool any = false;
  for (int g = 0; g < p->G; ++g) {
    if (!touched[g] || p->group_size[g] == 0) continue;
    any = true;
    int64_t ab[1][2];
    st = ensure_ring_space(p, &g, 1, stream, ab);
    if (st != SS_OK) return st;
    e = enqueue_compact_group(p, g, p->dense_upper > 0, true, true, stream, p->sel);
    if (e != hipSuccess) return hip_fail(e, "compact launch");
    after_compact_group(p, g, &ab[0]);
  }
  refresh_fact_upper(p);
  if (any && p->promote && p->fact_upper > 0 && p->prune_due++ % kPruneEvery == 0) {
    e = enqueue_prune(p, p->fact_upper, stream);
    if (e != hipSuccess) return hip_fail(e, "factored-list launch");
  }
  p->compact_calls++;
  return SS_OK;
}

// host-side checks shared by both initialization entry points (before any HIP call)
static ss_status rsvd_check(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                            int32_t iters, const float *omega, const float *eps, int32_t max_rank, const void *u,
                            const void *v, const void *sigma, const void *rank) {
  if (n < 0) return fail(SS_ERR_ARG, "n must be >= 0");
  if (d_k < 4 || d_v < 4 || d_k > 256 || d_v > 256 || (d_k & 3) || (d_v & 3))
    return fail(SS_ERR_SHAPE, "d_k and d_v must be multiples of 4 in [4, 256]");
  if (block < 1 || block > ss::kMaxM || block > d_k || block > d_v)
    return fail(SS_ERR_SHAPE, "block must be in [1, min(16, d_k, d_v)]");
  if (n_blocks < 1 || iters < 1 || iters > 64) return fail(SS_ERR_ARG, "n_blocks >= 1 and iters in [1, 64] required");
  if (max_rank < 1 || max_rank > std::min(d_k, d_v) || (int64_t)max_rank > (int64_t)n_blocks * block)
    return fail(SS_ERR_ARG, "max_rank must be in [1, min(d_k, d_v, n_blocks * block)]");
  if (n == 0) return SS_OK;
  if (!S || !omega || !eps || !u || !v || !sigma || !rank) return fail(SS_ERR_ARG, "null pointer");
  if (n > (int64_t)INT32_MAX) return fail(SS_ERR_ARG, "too many states for one launch");
  return SS_OK;
}

static ss_status rsvd_launch(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                             int32_t iters, const float *omega, const float *eps, int32_t max_rank, float *work,
                             float *u, float *v, float *sigma, int32_t *rank, hipStream_t stream) {
  ss::RsvdArgs a{};
  a.n = n; a.dk = d_k; a.dv = d_v; a.b = block; a.nb = n_blocks; a.iters = iters; a.max_rank = max_rank;
  a.S = S; a.omega = omega; a.eps = eps; a.work = work; a.u = u; a.v = v; a.sigma = sigma; a.rank = rank;
  const hipError_t e = ss::launch_rsvd_init(a, stream);
  return e == hipSuccess ? SS_OK : hip_fail(e, "randomized SVD launch");
}

ss_status ss_rsvd_init(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                       int32_t iters, const float *omega, const float *eps, int32_t max_rank, float *work, float *u,
                       float *v, float *sigma, int32_t *rank, hipStream_t stream) {
  ss_status st = rsvd_check(S, n, d_k, d_v, block, n_blocks, iters, omega, eps, max_rank, u, v, sigma, rank);
  if (st != SS_OK || n == 0) return st;
  if (!work) return fail(SS_ERR_ARG, "null pointer");
  return rsvd_launch(S, n, d_k, d_v, block, n_blocks, iters, omega, eps, max_rank, work, u, v, sigma, rank, stream);
}

ss_status ss_rsvd_init_noalloc(const float *S, int64_t n, int32_t d_k, int32_t d_v, int32_t block, int32_t n_blocks,
                               int32_t iters, const float *omega, const float *eps, int32_t max_rank, float *u,
                               float *v, float *sigma, int32_t *rank, hipStream_t stream) {
  ss_status st = rsvd_check(S, n, d_k, d_v, block, n_blocks, iters, omega, eps, max_rank, u, v, sigma, rank);
  if (st != SS_OK || n == 0) return st;
  const bool need_ws = !ss::rsvd_residual_in_lds(d_k, d_v);
  if (need_ws && n * (int64_t)d_k * d_v > (int64_t)ss::kRsvdScratchFloats)
    return fail(SS_ERR_CAPACITY, "n * d_k * d_v exceeds the 8,388,608-float (32 MiB) fixed workspace of "
                                 "ss_rsvd_init_noalloc; split the states over several calls");
  float *ws = nullptr;
  if (need_ws) {
    const hipError_t e = ss::rsvd_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "workspace address");
  }
  // states whose residual fits the LDS read no workspace
  return rsvd_launch(S, n, d_k, d_v, block, n_blocks, iters, omega, eps, max_rank, ws, u, v, sigma, rank, stream);
}


static hipError_t enqueue_consolidate_group(ss_pool *p, int g, hipStream_t stream) {
  ss::ConsolidateArgs a{};
  a.dk = p->dk; a.dv = p->dv; a.fmax = frozen_max(p);
  a.n_members = (int32_t)p->group_size[g];
  a.members = p->members + p->group_start[g];
  a.eps = p->eps; a.meta = p->meta; a.act = p->act; a.frz = p->frz;
  a.acct_flops = p->acct + ss::A_CONS_FLOPS * ss::kAcctSlots;
  a.acct_states = p->acct + ss::A_CONS_STATES * ss::kAcctSlots;
  a.acct_removed = p->acct + ss::A_CONS_REMOVED * ss::kAcctSlots;
  auto fn = [&] { return ss::launch_consolidate(a, stream); };
  return timed(p, SS_KERNEL_CONSOLIDATE, stream, fn);
}

static ss_status consolidate_checked(ss_pool *p, int g, hipStream_t stream) {
  if (p->ca.inflight && p->ca.group == g) p->ca.stale = true;
  p->cons_wait[g] = 0;
  p->cons_last[g] = p->cons_seq++;
  if (p->group_size[g] == 0 || frozen_max(p) == 0) return SS_OK;
  const hipError_t e = enqueue_consolidate_group(p, g, stream);
  if (e != hipSuccess) return hip_fail(e, "consolidate launch");
  p->consolidate_calls++;
  return SS_OK;
}

static ss_status consolidate_precheck(ss_pool *p) {
  if (!p) return fail(SS_ERR_ARG, "pool is NULL");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (ss::consolidate_lds_bytes(p->dk, p->dv, frozen_max(p), p->half != 0) > ss::kConsolidateLdsMax)
    return fail(SS_ERR_SHAPE, "the pool's largest frozen part does not fit the consolidation kernel's LDS");
  if (p->diag) return fail(SS_ERR_ARG, "consolidation is not available with per-channel decay");
  return SS_OK;
}

ss_status ss_consolidate(ss_pool *p, int32_t group, hipStream_t stream) {
  ss_status st = consolidate_precheck(p);
  if (st != SS_OK) return st;
  if (group >= p->G) return fail(SS_ERR_ARG, "group out of range");
  if (p->force_dense) return SS_OK;
  const int g0 = group < 0 ? 0 : group, g1 = group < 0 ? p->G : group + 1;
  for (int g = g0; g < g1; ++g) {
    st = consolidate_checked(p, g, stream);
    if (st != SS_OK) return st;
  }
  return SS_OK;
}

ss_status ss_consolidate_next(ss_pool *p, int32_t max_groups, int32_t *out, int32_t *n_done, hipStream_t stream) {
  if (!p || !n_done || max_groups < 0) return fail(SS_ERR_ARG, "bad arguments");
  *n_done = 0;
  ss_status st = consolidate_precheck(p);
  if (st != SS_OK) return st;
  if (p->force_dense) return SS_OK;
  std::vector<int> wait;
  for (int g = 0; g < p->G; ++g)
    if (p->cons_wait[g]) wait.push_back(g);
  // least recently consolidated first (never consolidated: -1), then by group id
  std::stable_sort(wait.begin(), wait.end(), [&](int x, int y) { return p->cons_last[x] < p->cons_last[y]; });
  const int take = std::min<int>(max_groups, (int)wait.size());
  for (int i = 0; i < take; ++i) {
    st = consolidate_checked(p, wait[i], stream);
    if (st != SS_OK) return st;
    if (out) out[i] = wait[i];
    *n_done = i + 1;
  }
  return SS_OK;
}

// Queue head of the asynchronous forms ([SS] 4.3, Figure 7(b)): among the groups waiting (compacted
// since their last consolidation), those whose last result was dropped as stale first, then the
// least recently consolidated (never consolidated first), then the lowest id.  group >= 0 selects it.
static int async_pick(ss_pool *p, int group) {
  if ((int)p->cons_dropped.size() < p->G) p->cons_dropped.assign(p->G, 0);
  if (group >= 0) return group;
  int g = -1;
  for (int h = 0; h < p->G; ++h) {
    if (!p->cons_wait[h]) continue;
    if (g < 0 || p->cons_dropped[h] > p->cons_dropped[g] ||
        (p->cons_dropped[h] == p->cons_dropped[g] && p->cons_last[h] < p->cons_last[g]))
      g = h;
  }
  return g;
}

// Staging of the asynchronous forms, for the largest group (allocated at the first call; the host
// form adds pinned host buffers of the same shape, sigma_0 and epsilon per member, and its own
// stream and events)
static hipError_t async_staging(ss_pool *p, int fmax, bool host) {
  hipError_t e = hipSuccess;
  int64_t gmax = 0;
  for (int h = 0; h < p->G; ++h) gmax = std::max<int64_t>(gmax, p->group_size[h]);
  if (p->ca.cap_members < gmax || p->ca.fmax < fmax) {
    if (p->ca.cap_members) return hipErrorInvalidValue;
    e = dalloc(p, &p->ca.snap, (size_t)gmax);
    if (e == hipSuccess) e = dalloc(p, &p->ca.st_u, (size_t)gmax * fmax * p->dk);
    if (e == hipSuccess) e = dalloc(p, &p->ca.st_v, (size_t)gmax * fmax * p->dv);
    if (e == hipSuccess) e = dalloc(p, &p->ca.st_s, (size_t)gmax * fmax);
    if (e == hipSuccess) e = dalloc(p, &p->ca.st_cnt, (size_t)gmax);
    if (e == hipSuccess) e = dalloc(p, &p->ca.installed, 1);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ca.snap_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ca.done_ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    p->ca.cap_members = gmax;
    p->ca.fmax = fmax;
  }
  if (host && !p->ca.own_side) {
    const size_t rows = (size_t)gmax * fmax;
    auto pin = [&](void **q, size_t bytes) {
      if (e == hipSuccess) e = hipHostMalloc(q, bytes, hipHostMallocDefault);
    };
    e = dalloc(p, &p->ca.st_s0, (size_t)gmax);
    pin((void **)&p->ca.h_u, rows * p->dk * sizeof(float));
    pin((void **)&p->ca.h_v, rows * p->dv * sizeof(float));
    pin((void **)&p->ca.h_s, rows * sizeof(float));
    pin((void **)&p->ca.h_cnt, (size_t)gmax * sizeof(int32_t));
    pin((void **)&p->ca.h_s0, (size_t)gmax * sizeof(float));
    pin((void **)&p->ca.h_eps, (size_t)gmax * sizeof(float));
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ca.read_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->ca.dl_ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->ca.own_side, hipStreamNonBlocking);
  }
  return e;
}

ss_status ss_consolidate_async(ss_pool *p, int32_t group, hipStream_t stream, hipStream_t side, int32_t *launched) {
  if (!p || !launched) return fail(SS_ERR_ARG, "bad arguments");
  *launched = -1;
  ss_status st = consolidate_precheck(p);
  if (st != SS_OK) return st;
  if (group >= p->G) return fail(SS_ERR_ARG, "group out of range");
  if (p->ca.inflight) return fail(SS_ERR_STATE, "an asynchronous consolidation is already in flight");
  if (p->force_dense) return SS_OK;
  const int fmax = frozen_max(p);
  if (ss::consolidate_lds_bytes(p->dk, p->dv, fmax, false) > ss::kConsolidateLdsMax)
    return fail(SS_ERR_SHAPE, "the pool's largest frozen part does not fit the consolidation kernel's LDS");
  const int g = async_pick(p, group);
  if (g < 0) return SS_OK;
  p->cons_wait[g] = 0;
  p->cons_last[g] = p->cons_seq++;
  if (p->group_size[g] == 0 || fmax == 0) return SS_OK;
  hipError_t e = async_staging(p, fmax, false);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? fail(SS_ERR_OOM, "consolidation staging") : hip_fail(e, "consolidation staging");
  const int32_t n = (int32_t)p->group_size[g];
  const int32_t *members = p->members + p->group_start[g];
  e = ss::launch_cons_snapshot(p->meta, members, n, p->ca.snap, stream);
  if (e == hipSuccess) e = hipEventRecord(p->ca.snap_ev, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, p->ca.snap_ev, 0);
  if (e == hipSuccess) {
    ss::ConsolidateArgs a{};
    a.dk = p->dk; a.dv = p->dv; a.fmax = fmax; a.n_members = n; a.members = members;
    a.eps = p->eps; a.meta = p->meta; a.act = p->act; a.frz = p->frz;
    a.acct_flops = p->acct + ss::A_CONS_FLOPS * ss::kAcctSlots;
    a.acct_states = p->acct + ss::A_CONS_STATES * ss::kAcctSlots;
    a.acct_removed = p->acct + ss::A_CONS_REMOVED * ss::kAcctSlots;
    a.snap = p->ca.snap; a.st_u = p->ca.st_u; a.st_v = p->ca.st_v; a.st_s = p->ca.st_s; a.st_cnt = p->ca.st_cnt;
    e = ss::launch_consolidate(a, side);
  }
  if (e == hipSuccess) e = hipEventRecord(p->ca.done_ev, side);
  if (e != hipSuccess) return hip_fail(e, "asynchronous consolidation launch");
  p->ca.inflight = true;
  p->ca.host = false;
  p->ca.stale = false;
  p->ca.group = g;
  p->ca.launched++;
  *launched = g;
  return SS_OK;
}

ss_status ss_host_consolidate_frozen(int32_t d_k, int32_t d_v, int32_t f, float *u, float *v, float *sigma,
                                     float sigma0, float eps, int32_t *kept) {
  if (!kept || f < 0) return fail(SS_ERR_ARG, "bad arguments");
  if (d_k < 1 || d_v < 1) return fail(SS_ERR_SHAPE, "d_k and d_v must be >= 1");
  if (f > 0 && (!u || !v || !sigma)) return fail(SS_ERR_ARG, "null pointer");
  *kept = ss::host_consolidate_one(d_k, d_v, f, u, v, sigma, sigma0, eps);
  return SS_OK;
}

ss_status ss_consolidate_host(ss_pool *p, int32_t group, hipStream_t stream, int32_t threads, int32_t *launched) {
  if (!p || !launched) return fail(SS_ERR_ARG, "bad arguments");
  *launched = -1;
  if (threads < 0) return fail(SS_ERR_ARG, "threads must be >= 0");
  if (p->diag) return fail(SS_ERR_ARG, "consolidation is not available with per-channel decay");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (group >= p->G) return fail(SS_ERR_ARG, "group out of range");
  if (p->ca.inflight) return fail(SS_ERR_STATE, "an asynchronous consolidation is already in flight");
  if (p->force_dense) return SS_OK;
  const int fmax = frozen_max(p);
  const int g = async_pick(p, group);
  if (g < 0) return SS_OK;
  p->cons_wait[g] = 0;
  p->cons_last[g] = p->cons_seq++;
  if (p->group_size[g] == 0 || fmax == 0) return SS_OK;
  hipError_t e = async_staging(p, fmax, true);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? fail(SS_ERR_OOM, "consolidation staging") : hip_fail(e, "consolidation staging");
  const int32_t n = (int32_t)p->group_size[g];
  const int32_t *members = p->members + p->group_start[g];
  hipStream_t side = p->ca.own_side;
  // snapshot of the records on the pool's stream; the side stream copies the frozen parts they
  // name into staging and downloads them with the states' sigma_0 and epsilon
  e = ss::launch_cons_snapshot(p->meta, members, n, p->ca.snap, stream);
  if (e == hipSuccess) e = hipEventRecord(p->ca.snap_ev, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(side, p->ca.snap_ev, 0);
  if (e == hipSuccess) {
    ss::GatherArgs ga{};
    ga.dk = p->dk; ga.dv = p->dv; ga.fmax = fmax; ga.n_members = n; ga.snap = p->ca.snap;
    ga.act = p->act; ga.frz = p->frz; ga.st_u = p->ca.st_u; ga.st_v = p->ca.st_v; ga.st_s = p->ca.st_s;
    ga.st_cnt = p->ca.st_cnt; ga.st_s0 = p->ca.st_s0;
    e = ss::launch_cons_gather(ga, side);
  }
  if (e == hipSuccess) e = hipEventRecord(p->ca.read_ev, side);
  const size_t rows = (size_t)n * fmax;
  auto d2h = [&](void *dst, const void *src, size_t bytes) {
    if (e == hipSuccess) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, side);
  };
  d2h(p->ca.h_u, p->ca.st_u, rows * p->dk * sizeof(float));
  d2h(p->ca.h_v, p->ca.st_v, rows * p->dv * sizeof(float));
  d2h(p->ca.h_s, p->ca.st_s, rows * sizeof(float));
  d2h(p->ca.h_cnt, p->ca.st_cnt, (size_t)n * sizeof(int32_t));
  d2h(p->ca.h_s0, p->ca.st_s0, (size_t)n * sizeof(float));
  if (e == hipSuccess) e = hipEventRecord(p->ca.dl_ev, side);
  if (e != hipSuccess) return hip_fail(e, "host consolidation download");
  for (int32_t i = 0; i < n; ++i) p->ca.h_eps[i] = p->eps_host[p->members_host[p->group_start[g] + i]];
  // the host worker: wait for the download, run the SVDs, enqueue the upload and its event
  const int nt = threads > 0 ? threads : std::max(1, (int)std::thread::hardware_concurrency());
  p->ca.hstate.store(1);
  p->ca.herr.clear();
  const int dk = p->dk, dv = p->dv;
  p->ca.worker = std::thread([p, n, fmax, nt, dk, dv, side]() {
    auto &c = p->ca;
    hipError_t we = hipEventSynchronize(c.dl_ev);
    if (we == hipSuccess) {
      const auto t0 = std::chrono::steady_clock::now();
      ss::host_consolidate_batch(n, dk, dv, fmax, c.h_u, c.h_v, c.h_s, c.h_cnt, c.h_s0, c.h_eps, nt);
      c.host_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
      const size_t rows = (size_t)n * fmax;
      auto h2d = [&](void *dst, const void *src, size_t bytes) {
        if (we == hipSuccess) we = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, side);
      };
      h2d(c.st_u, c.h_u, rows * dk * sizeof(float));
      h2d(c.st_v, c.h_v, rows * dv * sizeof(float));
      h2d(c.st_s, c.h_s, rows * sizeof(float));
      h2d(c.st_cnt, c.h_cnt, (size_t)n * sizeof(int32_t));
      if (we == hipSuccess) we = hipEventRecord(c.done_ev, side);
    }
    if (we != hipSuccess) c.herr = hipGetErrorString(we);
    c.hstate.store(we == hipSuccess ? 2 : 3);
  });
  p->ca.inflight = true;
  p->ca.host = true;
  p->ca.stale = false;
  p->ca.group = g;
  p->ca.launched++;
  *launched = g;
  return SS_OK;
}

ss_status ss_consolidate_poll(ss_pool *p, int32_t wait, hipStream_t stream, int32_t *state) {
  if (!p || !state) return fail(SS_ERR_ARG, "bad arguments");
  *state = SS_CONS_IDLE;
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  if (!p->ca.inflight) return SS_OK;
  if (p->ca.host) {  // the host worker enqueues the upload and records done_ev when it is through
    if (!wait && p->ca.hstate.load() == 1) {
      *state = SS_CONS_RUNNING;
      return SS_OK;
    }
    if (p->ca.worker.joinable()) p->ca.worker.join();
    if (p->ca.hstate.load() == 3) {
      p->ca.inflight = false;
      return fail(SS_ERR_HIP, "host consolidation: " + p->ca.herr);
    }
  }
  hipError_t e = wait ? hipEventSynchronize(p->ca.done_ev) : hipEventQuery(p->ca.done_ev);
  if (e == hipErrorNotReady) {
    *state = SS_CONS_RUNNING;
    return SS_OK;
  }
  if (e != hipSuccess) return hip_fail(e, "asynchronous consolidation");
  p->ca.inflight = false;
  if (p->ca.stale) {
    p->ca.discarded++;
    p->cons_dropped[p->ca.group] = 1;  // retried first ([SS] Figure 7(b))
    p->cons_wait[p->ca.group] = 1;
    *state = SS_CONS_DISCARDED;
    return SS_OK;
  }
  p->cons_dropped[p->ca.group] = 0;
  ss::InstallArgs ia{};
  const int g = p->ca.group;
  ia.dk = p->dk; ia.dv = p->dv; ia.fmax = p->ca.fmax; ia.n_members = (int32_t)p->group_size[g];
  ia.members = p->members + p->group_start[g]; ia.snap = p->ca.snap; ia.meta = p->meta; ia.frz = p->frz;
  ia.st_u = p->ca.st_u; ia.st_v = p->ca.st_v; ia.st_s = p->ca.st_s; ia.st_cnt = p->ca.st_cnt;
  ia.acct_removed = p->acct + ss::A_CONS_REMOVED * ss::kAcctSlots; ia.installed = p->ca.installed;
  e = hipStreamWaitEvent(stream, p->ca.done_ev, 0);
  if (e == hipSuccess) e = ss::launch_cons_install(ia, stream);
  if (e != hipSuccess) return hip_fail(e, "consolidation install");
  p->ca.installs++;
  p->consolidate_calls++;
  *state = SS_CONS_INSTALLED;
  return SS_OK;
}

ss_status ss_schedule_due(const ss_pool *p, int64_t step, int32_t *out, int32_t cap, int32_t *n_due) {
  if (!p || !n_due || (cap > 0 && !out) || cap < 0) return fail(SS_ERR_ARG, "bad arguments");
  int32_t c = 0;
  for (int g = 0; g < p->G; ++g) {
    int64_t x = (step + p->group_offset[g]) % p->K;
    if (x < 0) x += p->K;
    if (x == 0) {
      if (c < cap) out[c] = g;
      ++c;
    }
  }
  *n_due = c;
  return c > cap ? fail(SS_ERR_CAPACITY, "out is too small") : SS_OK;
}

ss_status ss_state_export(ss_pool *p, const int64_t *ids, int64_t n, void *host_buf, size_t cap, size_t *needed,
                          hipStream_t stream) {
  if (!p || (n > 0 && !ids) || n < 0 || !needed) return fail(SS_ERR_ARG, "bad arguments");
  for (int64_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= p->N) return fail(SS_ERR_ARG, "state id out of range");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "export sync");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  const int dk = p->dk, dv = p->dv, K = p->K;
  std::vector<ss::Meta> metas(n);
  for (int64_t i = 0; i < n; ++i) {
    e = hipMemcpy(&metas[i], p->meta + ids[i], sizeof(ss::Meta), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "export meta");
  }
  size_t need = 0;
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t pk = metas[i].packed;
    need += 8 * sizeof(int32_t);
    if (ss::meta_flags(pk) & ss::FLAG_DENSE) {
      need += sizeof(float) * (size_t)dk * dv;
    } else {
      const size_t R = ss::meta_ra(pk) + ss::meta_rf(pk), nn = ss::meta_n(pk);
      need += sizeof(float) * (R * (1 + dk + dv) + nn * (1 + dk + dv));
    }
  }
  *needed = need;
  if (!host_buf || cap < need) return fail(SS_ERR_CAPACITY, "export buffer too small");
  char *w = static_cast<char *>(host_buf);
  for (int64_t i = 0; i < n; ++i) {
    const ss::Meta m = metas[i];
    const uint32_t pkd = m.packed;
    const bool dense = ss::meta_flags(pkd) & ss::FLAG_DENSE;
    const int ra = dense ? 0 : ss::meta_ra(pkd), rf = dense ? 0 : ss::meta_rf(pkd), nn = dense ? 0 : ss::meta_n(pkd);
    ss::DenseSlot rec{};
    if (dense) {  // a dense state's pad fill and Gamma live in its slot record
      e = hipMemcpy(&rec, p->dslot + m.off_a, sizeof(rec), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(e, "export slot");
    }
    const int dpad = (dense && !p->force_dense) ? (int)ss::meta_n(rec.packed) : 0;
    int32_t hdr[8] = {(int32_t)ids[i], dense ? 1 : 0, ra + rf, ra, nn,
                      (ss::meta_flags(pkd) & ss::FLAG_DELTA) ? 1 : 0, dpad, 0};
    std::memcpy(w, hdr, sizeof(hdr));
    w += sizeof(hdr);
    auto dl = [&](void *dst, const void *src, size_t bytes) {
      if (e == hipSuccess && bytes) e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
    };
    if (dense) {  // the region holds H = S^T [d_v][d_k] and a pad; the export format is S [d_k][d_v]
      const int np = dpad;
      std::vector<float> H((size_t)dk * dv), PK((size_t)np * dk), PW((size_t)np * dv), PC(np);
      dl(H.data(), p->dense + (size_t)m.off_a * dk * dv, sizeof(float) * H.size());
      dl(PK.data(), p->dpk + (size_t)m.off_a * K * dk, sizeof(float) * PK.size());
      dl(PW.data(), p->dpw + (size_t)m.off_a * K * dv, sizeof(float) * PW.size());
      dl(PC.data(), p->dpc + (size_t)m.off_a * K, sizeof(float) * PC.size());
      std::vector<float> G(dk, 1.0f);  // per-channel decay: the slot's accumulated decays scale row i2 of S
      if (p->dgam) dl(G.data(), p->dgam + (size_t)m.off_a * dk, sizeof(float) * dk);
      if (e != hipSuccess) return hip_fail(e, "export copy");
      const double g = p->force_dense ? 1.0 : (double)rec.gamma;
      float *S = reinterpret_cast<float *>(w);
      for (int i2 = 0; i2 < dk; ++i2)
        for (int j = 0; j < dv; ++j) {
          double x = H[(size_t)j * dk + i2];
          for (int t = 0; t < np; ++t) x += (double)PC[t] * PK[(size_t)t * dk + i2] * PW[(size_t)t * dv + j];
          S[(size_t)i2 * dv + j] = (float)(g * (double)G[i2] * x);
        }
      w += sizeof(float) * (size_t)dk * dv;
      continue;
    }
    const int R = ra + rf;
    float *sig = reinterpret_cast<float *>(w);
    float *u = sig + R;
    float *v = u + (size_t)R * dk;
    float *c = v + (size_t)R * dv;
    float *kk = c + nn;
    float *ww = kk + (size_t)nn * dk;
    // `cnt` components of a ring from physical slot c0, wrapping once at the ring's end
    // (elements of `esz` bytes; fp16 elements are staged and widened to fp32)
    std::vector<uint16_t> hbuf;
    auto dl_ring = [&](float *dst, const void *base, int64_t cap, int64_t c0, int64_t cnt, int row, int esz) {
      const int64_t first = std::min(cnt, cap - c0);
      char *d8 = reinterpret_cast<char *>(dst);
      if (esz == 2) {
        hbuf.resize((size_t)cnt * row);
        d8 = reinterpret_cast<char *>(hbuf.data());
      }
      const char *b8 = static_cast<const char *>(base);
      dl(d8, b8 + (size_t)c0 * row * esz, (size_t)esz * first * row);
      dl(d8 + (size_t)first * row * esz, b8, (size_t)esz * (cnt - first) * row);
      if (esz == 2 && e == hipSuccess)
        for (size_t x = 0; x < hbuf.size(); ++x) dst[x] = half_to_float(hbuf[x]);
    };
    const int fz = p->half ? 2 : 4;
    dl_ring(sig, p->act.s, p->act.cap, m.off_a, ra, 1, 4);
    dl_ring(sig + ra, p->frz.s, p->frz.cap, m.off_f, rf, 1, 4);
    dl_ring(u, p->act.u, p->act.cap, m.off_a, ra, dk, fz);
    dl_ring(u + (size_t)ra * dk, p->frz.u, p->frz.cap, m.off_f, rf, dk, fz);
    dl_ring(v, p->act.v, p->act.cap, m.off_a, ra, dv, fz);
    dl_ring(v + (size_t)ra * dv, p->frz.v, p->frz.cap, m.off_f, rf, dv, fz);
    dl(c, p->pc + (size_t)ids[i] * K, sizeof(float) * nn);
    dl(kk, p->pk + (size_t)ids[i] * K * dk, sizeof(float) * (size_t)nn * dk);
    dl(ww, p->pw + (size_t)ids[i] * K * dv, sizeof(float) * (size_t)nn * dv);
    std::vector<float> G;
    if (p->gam) {  // per-channel decay: the effective u and pad keys carry the accumulated decays
      G.resize(dk);
      dl(G.data(), p->gam + (size_t)ids[i] * dk, sizeof(float) * dk);
    }
    if (e != hipSuccess) return hip_fail(e, "export copy");
    for (int j = 0; j < R; ++j) sig[j] *= m.gamma;
    for (int j = 0; j < nn; ++j) c[j] *= m.gamma;
    if (p->gam) {
      for (int j = 0; j < R; ++j)
        for (int x = 0; x < dk; ++x) u[(size_t)j * dk + x] *= G[x];
      for (int j = 0; j < nn; ++j)
        for (int x = 0; x < dk; ++x) kk[(size_t)j * dk + x] *= G[x];
    }
    w = reinterpret_cast<char *>(ww + (size_t)nn * dv);
  }
  if (e != hipSuccess) return hip_fail(e, "export copy");
  return SS_OK;
}

ss_status ss_pool_stats(ss_pool *p, ss_stats *out, hipStream_t stream) {
  if (!p || !out) return fail(SS_ERR_ARG, "bad arguments");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "stats sync");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  std::vector<ss::Meta> meta(p->N);
  e = hipMemcpy(meta.data(), p->meta, sizeof(ss::Meta) * p->N, hipMemcpyDeviceToHost);
  uint32_t ctr[ss::C_N];
  if (e == hipSuccess) e = hipMemcpy(ctr, p->counters, sizeof(ctr), hipMemcpyDeviceToHost);
  std::vector<unsigned long long> acct(ss::A_N * ss::kAcctSlots);
  if (e == hipSuccess) e = hipMemcpy(acct.data(), p->acct, acct.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
  const int64_t nd = std::min<int64_t>(p->cap_d, ctr[ss::C_DENSE_COUNT]);
  std::vector<ss::DenseSlot> dslot(nd);
  if (e == hipSuccess && nd) e = hipMemcpy(dslot.data(), p->dslot, sizeof(ss::DenseSlot) * nd, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "stats copy");
  std::memset(out, 0, sizeof(*out));
  out->n_states = p->N;
  const int64_t comp = 4ll * (p->dk + p->dv + 1), fcomp = comp_bytes(p);  // a pad slot, a stored component
  int64_t live = 16ll * p->N + 16ll * nd;
  for (int64_t s = 0; s < p->N; ++s) {
    const uint32_t pk = meta[s].packed;
    if (ss::meta_flags(pk) & ss::FLAG_DENSE) {
      const int64_t slot = meta[s].off_a;
      const int64_t nn = (p->force_dense || slot < 0 || slot >= nd) ? 0 : ss::meta_n(dslot[slot].packed);
      out->n_dense++;
      out->pad_entries += nn;
      live += 4ll * p->dk * p->dv + comp * nn;
      continue;
    }
    out->n_factored++;
    const int64_t ra = ss::meta_ra(pk), rf = ss::meta_rf(pk), nn = ss::meta_n(pk);
    out->active_components += ra;
    out->frozen_components += rf;
    out->pad_entries += nn;
    live += fcomp * (ra + rf) + comp * nn;
    out->max_rank = std::max<int64_t>(out->max_rank, ra + rf);
    out->rank_hist[std::min<int64_t>(64, ra + rf)]++;
  }
  out->live_bytes = live;
  out->reserved_bytes = p->reserved + (int64_t)(p->ring_bytes[0] + p->ring_bytes[1]);
  out->decode_calls = p->decode_calls;
  out->compact_calls = p->compact_calls;
  out->readout_calls = p->readout_calls;
  for (int i = 0; i < ss::kAcctSlots; ++i) {
    out->decode_bytes_factored += acct[ss::A_DECODE_FACTORED * ss::kAcctSlots + i];
    out->decode_bytes_dense += acct[ss::A_DECODE_DENSE * ss::kAcctSlots + i];
    out->compact_flops += acct[ss::A_COMPACT_FLOPS * ss::kAcctSlots + i];
    out->compact_states += acct[ss::A_COMPACT_STATES * ss::kAcctSlots + i];
    out->consolidate_flops += acct[ss::A_CONS_FLOPS * ss::kAcctSlots + i];
    out->consolidate_states += acct[ss::A_CONS_STATES * ss::kAcctSlots + i];
    out->consolidate_removed += acct[ss::A_CONS_REMOVED * ss::kAcctSlots + i];
  }
  out->consolidate_calls = p->consolidate_calls;
  out->decode_bytes = out->decode_bytes_factored + out->decode_bytes_dense;
  out->promotions = ctr[ss::C_PROMOTIONS];
  out->cap_truncations = ctr[ss::C_CAP_TRUNC];
  out->jacobi_limit_hits = ctr[ss::C_JACOBI_LIMIT];
  if (!p->force_dense) {  // exact ring figures (the stream is idle here)
    ss::Ring ring[2];
    std::vector<unsigned long long> seg(4 * (size_t)p->G);
    e = hipMemcpy(ring, p->ring, sizeof(ring), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(seg.data(), p->seg, sizeof(unsigned long long) * seg.size(), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "stats copy");
    for (int R = 0; R < 2; ++R) {
      unsigned long long tail = ring[R].head;
      for (int g = 0; g < p->G; ++g) {
        const unsigned long long *sg = seg.data() + (size_t)R * 2 * p->G + 2 * g;
        if (sg[1] > sg[0]) tail = std::min(tail, sg[0]);
      }
      out->ring_capacity[R] = p->arena(R).cap;
      out->ring_used[R] = (int64_t)(ring[R].head - tail);
      out->ring_head[R] = (int64_t)ring[R].head;
    }
  }
  out->ring_repacks = p->repacks;
  out->ring_syncs = p->ring_syncs;
  for (auto &ev : p->pending) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev.a, ev.b) == hipSuccess) {
      p->kernel_ms[ev.kernel] += ms;
      p->kernel_launches[ev.kernel] += 1;
    }
    p->spare.push_back(ev.a);
    p->spare.push_back(ev.b);
  }
  p->pending.clear();
  for (int k = 0; k < SS_KERNEL_COUNT; ++k) {
    out->kernel_ms[k] = p->kernel_ms[k];
    out->kernel_launches[k] = p->kernel_launches[k];
  }
  p->dense_upper = std::min<int64_t>(p->cap_d, ctr[ss::C_DENSE_COUNT]);
  return SS_OK;
}

ss_status ss_pool_timing(ss_pool *p, int32_t enable) {
  if (!p) return fail(SS_ERR_ARG, "pool is NULL");
  p->timing = enable != 0;
  return SS_OK;
}

// ---- graph replay of whole steps ---------------------------------------------------------------
}  // extern "C"

struct ss_step_graph {
  ss_pool *pool = nullptr;
  const float *q = nullptr, *k = nullptr, *v = nullptr, *alpha = nullptr, *beta = nullptr;
  float *o = nullptr;
  hipStream_t cs = nullptr;                // capture stream (graphs are launched on the caller's stream)
  std::vector<hipGraphExec_t> exec;        // one per phase of the schedule (step mod K)
  std::vector<std::vector<int>> due;       // groups compacted in each phase
  int64_t version = -1;                    // pool layout the graphs were captured against
  int64_t fact_grid = 0, dense_grid = 0;   // grid bounds captured
};

namespace {

void drop_execs(ss_step_graph *sg) {
  for (auto &x : sg->exec)
    if (x) (void)hipGraphExecDestroy(x);
  for (auto &x : sg->exec) x = nullptr;
}

// Capture one graph per phase: the decode of every state, then the compactions due in that
// phase, then the pruning of the factored-state list.  Grid sizes are bounds that stay valid for
// the pool's life: the factored list only shrinks, and the dense slots in use never exceed the
// dense states at capture plus every factored one.
ss_status capture_all(ss_step_graph *sg) {
  ss_pool *p = sg->pool;
  drop_execs(sg);
  refresh_fact_upper(p);
  sg->fact_grid = p->force_dense ? 0 : p->fact_upper;
  sg->dense_grid = std::min<int64_t>(p->cap_d, p->dense_upper + (p->promote ? sg->fact_grid : 0));
  for (int ph = 0; ph < p->K; ++ph) {
    hipError_t e = hipStreamBeginCapture(sg->cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "graph capture");
    e = enqueue_decode(p, sg->q, sg->k, sg->v, sg->alpha, sg->beta, sg->o, false, sg->fact_grid, sg->dense_grid,
                       false, sg->cs);
    for (size_t i = 0; e == hipSuccess && i < sg->due[ph].size(); ++i)
      e = enqueue_compact_group(p, sg->due[ph][i], sg->dense_grid > 0, sg->fact_grid > 0, false, sg->cs);
    if (e == hipSuccess && !sg->due[ph].empty() && p->promote && sg->fact_grid > 0)
      e = enqueue_prune(p, sg->fact_grid, sg->cs);
    hipGraph_t graph = nullptr;
    const hipError_t e2 = hipStreamEndCapture(sg->cs, &graph);
    if (e == hipSuccess) e = e2;
    if (e == hipSuccess) e = hipGraphInstantiate(&sg->exec[ph], graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    if (e != hipSuccess) {
      drop_execs(sg);
      return hip_fail(e, "graph capture");
    }
  }
  sg->version = p->layout_version;
  return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_step_graph_create(ss_pool *p, const float *q, const float *k, const float *v, const float *alpha,
                               const float *beta, float *o, ss_step_graph **out) {
  if (!out) return fail(SS_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!p) return fail(SS_ERR_ARG, "pool is NULL");
  if (!q || !k || !v || !alpha || !o) return fail(SS_ERR_ARG, "q, k, v, alpha and o are required");
  if (p->any_delta && !beta) return fail(SS_ERR_ARG, "beta is required: the pool has delta-rule states");
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  ss_step_graph *sg = new (std::nothrow) ss_step_graph();
  if (!sg) return fail(SS_ERR_OOM, "host allocation failed");
  sg->pool = p; sg->q = q; sg->k = k; sg->v = v; sg->alpha = alpha; sg->beta = beta; sg->o = o;
  sg->exec.assign(p->K, nullptr);
  sg->due.assign(p->K, {});
  for (int ph = 0; ph < p->K; ++ph)
    for (int g = 0; g < p->G; ++g)
      if (!p->force_dense && p->group_size[g] > 0 && (ph + p->group_offset[g]) % p->K == 0) sg->due[ph].push_back(g);
  hipError_t e = hipStreamCreateWithFlags(&sg->cs, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete sg;
    return hip_fail(e, "capture stream");
  }
  st = capture_all(sg);
  if (st != SS_OK) {
    (void)hipStreamDestroy(sg->cs);
    delete sg;
    return st;
  }
  *out = sg;
  return SS_OK;
}

ss_status ss_step_graph_launch(ss_step_graph *sg, int64_t step, hipStream_t stream) {
  if (!sg) return fail(SS_ERR_ARG, "graph is NULL");
  ss_pool *p = sg->pool;
  ss_status st = poll(p);
  if (st != SS_OK) return st;
  const int ph = (int)(((step % p->K) + p->K) % p->K);
  const std::vector<int> &due = sg->due[ph];
  std::vector<int64_t> ab(2 * due.size() + 2, 0);
  auto abp = reinterpret_cast<int64_t(*)[2]>(ab.data());
  // whether the graph launched below places components in the rings: it does while factored states
  // remain (fact_upper <= the captured grid, and a pool left with none is captured again below)
  refresh_fact_upper(p);
  const bool fact = !p->force_dense && p->fact_upper > 0;
  if (!due.empty() && fact) {
    st = ensure_ring_space(p, due.data(), (int)due.size(), stream, abp);
    if (st != SS_OK) return st;
  }
  refresh_fact_upper(p);
  // capture again when a re-pack moved the rings, or when the factored list has shrunk to half the
  // captured grid (the graphs then stop launching work for states that have gone dense)
  if (sg->version != p->layout_version || 2 * p->fact_upper < sg->fact_grid) {
    st = capture_all(sg);
    if (st != SS_OK) return st;
  }
  const hipError_t e = hipGraphLaunch(sg->exec[ph], stream);
  if (e != hipSuccess) return hip_fail(e, "graph launch");
  for (size_t i = 0; i < due.size(); ++i) after_compact_group(p, due[i], fact ? &abp[i] : nullptr);
  p->decode_calls++;
  if (!due.empty()) p->compact_calls++;
  return SS_OK;
}

ss_status ss_step_graph_destroy(ss_step_graph *sg) {
  if (!sg) return SS_OK;
  (void)hipStreamSynchronize(sg->cs);
  drop_execs(sg);
  (void)hipStreamDestroy(sg->cs);
  delete sg;
  return SS_OK;
}

}  // extern "C"

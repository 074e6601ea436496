// Host side of the jagged attention library: argument checks, the jagged tile scheduler, the
// workspace layout and the C ABI entry points declared in include/jfa.h.
//
// Scheduler. Removing padding leaves compute units idle when short sequences finish early, and the
// bottleneck moves to tile scheduling and load balance (aihot.vn GEM page, "Jagged Sequence Flash
// Attention"; vibekk.com GEM page, section on moving from padding to jagged kernels). Every tile of
// useful work becomes one work item; an item whose cost (visible tiles on its inner loop) exceeds a
// fair share ceil(total / slots) is split into R = ceil(cost / share) equal ranges whose partial
// results are merged in a fixed order; the list is sorted longest first, ties by (b, h, tile,
// range start), so that greedy in-order dispatch of workgroups is longest-processing-time
// scheduling and the list is unique.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <tuple>
#include <new>
#include <string>
#include <vector>

#include "jfa.h"
#include "jfa_internal.h"

using namespace jfa;

namespace {

thread_local std::string g_last_error;

jfa_status fail(jfa_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

jfa_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return JFA_ERR_HIP;
}

enum ListId { kFwd = 0, kDq = 1, kKv = 2 };

struct List {
  std::vector<int32_t> items;   // 6 ints per item: b, h, tile, lo, hi, slot
  std::vector<int32_t> groups;  // 5 ints per group: b, h, tile, slot0, R
  std::vector<char> first;      // per item: the first piece of its tile (unsplit items included)
  std::vector<int> order;       // dispatch order: device item p is items[order[p]]
  int nslots = 0;
  int slots = 0;                // concurrency the split rule balanced for
  int32_t* d_items = nullptr;
  int32_t* d_groups = nullptr;
  size_t n_items() const { return items.size() / 6; }
  size_t n_groups() const { return groups.size() / 5; }
};

struct Raw {
  int b, h, t, lo, hi;
};

void finish(const std::vector<Raw>& raw, int slots, bool split, List& out) {
  int64_t total = 0;
  int max_cost = 0;
  for (const Raw& r : raw) {
    total += r.hi - r.lo;
    max_cost = std::max(max_cost, r.hi - r.lo);
  }
  const int64_t s = std::max(1, slots);
  const int64_t target = std::max<int64_t>(1, (total + s - 1) / s);
  // With less than one tile of work per slot nothing is split: merging the pieces would cost a
  // launch of its own, more than the tiles it saves.
  const bool do_split = split && total > s;
  // Pieces in generation order, which is ascending (b, h, tile, range start).
  struct Item {
    int b, h, t, lo, hi, slot;
    bool first;
  };
  std::vector<Item> items;
  items.reserve(raw.size());
  int next = 0;
  for (const Raw& r : raw) {
    const int64_t cost = r.hi - r.lo;
    if (do_split && cost > target) {
      const int64_t R = (cost + target - 1) / target;
      out.groups.insert(out.groups.end(), {r.b, r.h, r.t, next, (int32_t)R});
      for (int64_t k = 0; k < R; ++k)
        items.push_back({r.b, r.h, r.t, (int)(r.lo + (k * cost) / R), (int)(r.lo + ((k + 1) * cost) / R), next + (int)k,
                         k == 0});
      next += (int)R;
    } else {
      items.push_back({r.b, r.h, r.t, r.lo, r.hi, -1, true});
    }
  }
  // Longest first, ties in generation order: a stable counting sort by cost (descending) gives the
  // order of the key (cost desc, b, h, tile, range start) in linear time.
  std::vector<int> start(max_cost + 2, 0);
  for (const Item& i : items) ++start[max_cost - (i.hi - i.lo) + 1];
  for (int c = 0; c <= max_cost; ++c) start[c + 1] += start[c];
  out.items.assign(items.size() * 6, 0);
  out.first.assign(items.size(), 0);
  for (const Item& i : items) {
    const size_t p = (size_t)start[max_cost - (i.hi - i.lo)]++;
    int32_t* o = &out.items[p * 6];
    o[0] = i.b, o[1] = i.h, o[2] = i.t, o[3] = i.lo, o[4] = i.hi, o[5] = i.slot;
    out.first[p] = i.first;
  }
  out.nslots = next;
  out.slots = slots;
}



// Dispatch order. The GPU hands workgroup p of a launch to XCD p % kXcds, and each of MI355X's eight
// XCDs has its own L2. Items of one (b, h) group read the same K/V (query-tile lists) or Q/dO
// (key-tile lists), so the order keeps a group on one XCD and its items together:
//   groups (b, h) with cost = total item cost, sorted by cost descending, then (b, h) ascending;
//   each group goes to the XCD with the least cost so far (lowest index on ties);
//   XCD x's queue holds its items by group rank, then in list order;
//   position p takes the next item of queue p % kXcds, or, once that queue is empty, of the queue
//   with the most items left (lowest index on ties).
// Longest groups first keeps the longest-first dispatch of the list within each XCD.
constexpr int kXcds = 8;

std::vector<int> dispatch_order(const List& L, int B, int H) {
  // Dense per-group arrays (group id b * H + h, ascending in (b, h)) and counting sorts keep this
  // linear in the items apart from one sort of the groups.
  const size_t n = L.n_items();
  const size_t G = (size_t)B * H;
  std::vector<int64_t> cost(G, 0);
  std::vector<int> count(G, 0);
  for (size_t i = 0; i < n; ++i) {
    const size_t g = (size_t)L.items[i * 6] * H + L.items[i * 6 + 1];
    cost[g] += L.items[i * 6 + 4] - L.items[i * 6 + 3];
    ++count[g];
  }
  std::vector<int> gs;  // groups with at least one item, longest first, then (b, h) ascending
  for (size_t g = 0; g < G; ++g)
    if (count[g]) gs.push_back((int)g);
  std::stable_sort(gs.begin(), gs.end(), [&](int x, int y) { return cost[x] > cost[y]; });
  std::vector<int> xcd_of(G, 0);
  std::vector<int64_t> load(kXcds, 0);
  for (int g : gs) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    xcd_of[g] = x;
    load[x] += cost[g];
  }
  // items of each group in list order (counting sort by group)
  std::vector<int> start(G + 1, 0);
  for (size_t g = 0; g < G; ++g) start[g + 1] = start[g] + count[g];
  std::vector<int> by_group(n), fill(start.begin(), start.end() - 1);
  for (size_t i = 0; i < n; ++i) by_group[fill[(size_t)L.items[i * 6] * H + L.items[i * 6 + 1]]++] = (int)i;
  // XCD x's queue: its groups in rank order, each group's items in list order
  std::vector<std::vector<int>> q(kXcds);
  for (int g : gs) q[xcd_of[g]].insert(q[xcd_of[g]].end(), by_group.begin() + start[g], by_group.begin() + start[g + 1]);
  std::vector<size_t> head(kXcds, 0);
  std::vector<int> order;
  order.reserve(n);
  for (size_t p = 0; p < n; ++p) {
    int x = (int)(p % kXcds);
    if (head[x] == q[x].size()) {
      int best = -1;
      for (int y = 0; y < kXcds; ++y)
        if (head[y] < q[y].size() && (best < 0 || q[y].size() - head[y] > q[best].size() - head[best])) best = y;
      x = best;
    }
    order.push_back(q[x][head[x]++]);
  }
  return order;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Optional window / block limits on visibility (0 = off). With either on, an item covers only the
// tiles that hold a visible pair: the keys seen by a run of rows, and the rows that see a run of
// keys, form one interval because every bound is non-decreasing in the position.
struct Limits {
  bool causal;
  int window, block;
  bool band() const { return window > 0 || block > 0; }
};

// Key tiles [lo, hi) holding a visible pair for query tile t (band limits on).
void band_key_tiles(int t, int Lq, int Lkv, const Limits& m, int BM, int BN, int& lo, int& hi) {
  const int64_t r0 = (int64_t)t * BM, r1 = std::min<int64_t>((int64_t)(t + 1) * BM, Lq) - 1;
  int64_t first = 0, last = (int64_t)Lkv - 1;
  if (m.window) {
    first = std::max<int64_t>(first, r0 - m.window + 1);
    if (!m.causal) last = std::min<int64_t>(last, r1 + m.window - 1);
  }
  if (m.causal) last = std::min(last, r1);
  if (m.block) {
    first = std::max<int64_t>(first, (r0 / m.block) * m.block);
    last = std::min<int64_t>(last, (r1 / m.block) * m.block + m.block - 1);
  }
  if (last < first) {
    lo = hi = 0;
    return;
  }
  lo = (int)(first / BN);
  hi = (int)(last / BN) + 1;
}

// Query tiles [lo, hi) holding a visible pair for key tile kt (band limits on); empty: [lo, lo).
void band_query_tiles(int kt, int Lq, int Lkv, const Limits& m, int BMq, int BNk, int& lo, int& hi) {
  const int64_t c0 = (int64_t)kt * BNk, c1 = std::min<int64_t>((int64_t)(kt + 1) * BNk, Lkv) - 1;
  int64_t first = 0, last = (int64_t)Lq - 1;
  if (m.causal) first = c0;
  if (m.window) {
    last = std::min<int64_t>(last, c1 + m.window - 1);
    if (!m.causal) first = std::max<int64_t>(first, c0 - m.window + 1);
  }
  if (m.block) {
    first = std::max<int64_t>(first, (c0 / m.block) * m.block);
    last = std::min<int64_t>(last, (c1 / m.block) * m.block + m.block - 1);
  }
  lo = (int)(first / BMq);
  hi = last < first ? lo : (int)(last / BMq) + 1;
}

// Query-tile list: item (b, h, t) covers key tiles [0, cost) (band limits: the tiles holding a
// visible pair).
void query_tile_list(const std::vector<int>& lq, const std::vector<int>& lkv, int H, const Limits& m, int BM, int BN,
                     int slots, bool split, List& out) {
  std::vector<Raw> raw;
  for (size_t b = 0; b < lq.size(); ++b) {
    const int n_kv = ceil_div(lkv[b], BN);
    const int n_t = ceil_div(lq[b], BM);
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < n_t; ++t) {
        int lo = 0, hi = 0;
        if (m.band())
          band_key_tiles(t, lq[b], lkv[b], m, BM, BN, lo, hi);
        else
          hi = m.causal ? std::min(ceil_div((t + 1) * BM, BN), n_kv) : n_kv;
        raw.push_back({(int)b, h, t, lo, hi});
      }
  }
  finish(raw, slots, split, out);
}

// Key-tile list: item (b, h, kt) covers query tiles [first, first + cost) (band limits: the tiles
// holding a visible pair).
void key_tile_list(const std::vector<int>& lq, const std::vector<int>& lkv, int H, const Limits& m, int BMq, int BNk,
                   int slots, bool split, List& out) {
  std::vector<Raw> raw;
  for (size_t b = 0; b < lq.size(); ++b) {
    const int n_q = ceil_div(lq[b], BMq);
    const int n_kt = ceil_div(lkv[b], BNk);
    for (int h = 0; h < H; ++h)
      for (int kt = 0; kt < n_kt; ++kt) {
        int lo = 0, hi = 0;
        if (m.band()) {
          band_query_tiles(kt, lq[b], lkv[b], m, BMq, BNk, lo, hi);
        } else {
          lo = m.causal ? (int)(((int64_t)kt * BNk) / BMq) : 0;
          hi = lo + std::max(0, n_q - lo);
        }
        raw.push_back({(int)b, h, kt, lo, hi});
      }
  }
  finish(raw, slots, split, out);
}

// Shared queries: the gradient of a query row is the sum over every sequence that uses it, so each
// dQ piece writes an fp32 partial and one group per (head, query tile) sums the pieces of all
// sequences in a fixed order (sequence, then range start). Group records name sequence 0, whose
// offsets (row 0, Ls rows) address the shared dQ.
void share_query_slots(List& L) {
  const size_t n = L.n_items();
  std::vector<int> idx(n);
  for (size_t i = 0; i < n; ++i) idx[i] = (int)i;
  auto key = [&](int i) { return std::make_tuple(L.items[i * 6 + 1], L.items[i * 6 + 2], L.items[i * 6], L.items[i * 6 + 3]); };
  std::sort(idx.begin(), idx.end(), [&](int x, int y) { return key(x) < key(y); });
  L.groups.clear();
  int slot = 0;
  for (size_t k = 0; k < n; ++k) {
    const int i = idx[k];
    const int h = L.items[i * 6 + 1], t = L.items[i * 6 + 2];
    if (k == 0 || h != L.items[idx[k - 1] * 6 + 1] || t != L.items[idx[k - 1] * 6 + 2])
      L.groups.insert(L.groups.end(), {0, h, t, slot, 0});
    L.groups.back() += 1;  // R
    L.items[i * 6 + 5] = slot++;
  }
  L.nslots = slot;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- buffer cache
// Work lists change with every batch of offsets, so planning sits on the training step's critical
// path (vibekk.com GEM page, section on moving from padding to jagged kernels: once padding is gone,
// time moves to tile scheduling). A plan therefore never synchronises: its records are written into
// pinned host memory and uploaded with an asynchronous copy, and both buffers come from a small
// process-wide cache. A cached buffer carries the events after which the device no longer uses it
// (the upload, and the last forward / backward call on every stream that used the plan); it is
// handed out again only once all of them have completed, so no wait is ever needed.
struct CachedBuf {
  void* ptr = nullptr;
  size_t bytes = 0;
  int device = -1;
  bool pinned = false;
  std::vector<hipEvent_t> pending;  // owned; the buffer is free once every one has completed
};

struct BufCache {
  std::mutex mu;
  std::vector<CachedBuf> free_bufs;
  std::vector<hipEvent_t> free_events;
};

BufCache& buf_cache() {
  static BufCache* c = new BufCache();  // never destroyed: plans may outlive static destructors
  return *c;
}

hipEvent_t cache_event() {
  BufCache& c = buf_cache();
  {
    std::lock_guard<std::mutex> lk(c.mu);
    if (!c.free_events.empty()) {
      hipEvent_t e = c.free_events.back();
      c.free_events.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
  return e;
}

// A buffer of at least `bytes` (pinned host memory or device memory of `device`); rounded up to a
// power of two from 64 KiB so that plans of similar size reuse each other's buffers.
hipError_t cache_acquire(size_t bytes, bool pinned, int device, CachedBuf& out) {
  size_t want = 65536;
  while (want < bytes) want <<= 1;
  BufCache& c = buf_cache();
  {
    std::lock_guard<std::mutex> lk(c.mu);
    for (size_t i = 0; i < c.free_bufs.size(); ++i) {
      CachedBuf& b = c.free_bufs[i];
      if (b.pinned != pinned || b.device != device || b.bytes != want) continue;
      bool done = true;
      for (hipEvent_t e : b.pending)
        if (hipEventQuery(e) != hipSuccess) done = false;
      if (!done) continue;
      for (hipEvent_t e : b.pending) c.free_events.push_back(e);
      b.pending.clear();
      out = b;
      c.free_bufs.erase(c.free_bufs.begin() + (long)i);
      return hipSuccess;
    }
  }
  out = CachedBuf{};
  out.bytes = want;
  out.device = device;
  out.pinned = pinned;
  return pinned ? hipHostMalloc(&out.ptr, want, hipHostMallocDefault) : hipMalloc(&out.ptr, want);
}

void cache_release(CachedBuf& b) {
  if (!b.ptr) return;
  BufCache& c = buf_cache();
  std::lock_guard<std::mutex> lk(c.mu);
  c.free_bufs.push_back(b);
  b = CachedBuf{};
}

// Device properties and kernel occupancies, queried once per device and kernel shape.
struct DeviceInfo {
  int cus = 0;
  int occ[2][2][3] = {};  // [D == 128][kv_short][forward, dQ, dK/dV]; 0 = not yet queried
};

hipError_t device_info(int dev, const Modes& m, int& cus, int occ[3]) {
  static std::mutex mu;
  static std::vector<DeviceInfo> infos;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)infos.size() <= dev) infos.resize(dev + 1);
  DeviceInfo& d = infos[dev];
  if (d.cus == 0) {
    hipError_t e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
      d.cus = 0;
      return e;
    }
  }
  int* o = d.occ[m.D == 128][m.kv_short];
  if (o[0] == 0) {
    o[0] = occupancy_forward(m);
    o[1] = occupancy_dq(m);
    o[2] = occupancy_dkdv(m);
  }
  cus = d.cus;
  std::copy_n(o, 3, occ);
  return hipSuccess;
}

}  // namespace

struct jfa_plan_s {
  int B = 0, H = 0, D = 0, Tq = 0, Tkv = 0;
  int kv_bn = kKvBN;  // keys per dK/dV item
  Modes modes{};
  Band band{};
  float scale = 0.0f;
  int out_f32 = 0, grad_f32 = 0;
  int q_shared = 0;  // JFA_PLAN_SHARED_Q
  // Backward as one fused pass over the dQ items (every sequence has at most kKvBM queries, D = 128,
  // no band limits, and every sequence with keys has queries, so that the dQ items cover every key)
  int fused_bwd = 0;
  int mx = 0;        // JFA_PLAN_MXFP8
  int n_vtiles = 0;  // MXFP8: 64-key tiles over all sequences (transposed quantised V)
  std::vector<int32_t> vtiles;  // [n_vtiles][2]: first key row, keys in the tile
  std::vector<int32_t> vtile0;  // per sequence: its first tile
  size_t off_qq = 0, off_qs = 0, off_kq = 0, off_ks = 0, off_vq = 0, off_vs = 0;
  int32_t* d_vtiles = nullptr;
  uint32_t flags = 0;
  std::vector<int32_t> q_off, kv_off;
  List lists[3];
  CachedBuf dev;        // device copy of all work lists (from the buffer cache)
  int device = -1;
  // Last use of the device lists on each stream (the upload's stream included): the buffer goes back
  // to the cache with these events and is not handed out again before they have all completed.
  std::mutex use_mu;
  std::vector<std::pair<hipStream_t, hipEvent_t>> uses;
  // workspace layout
  size_t ws_fwd = 0, off_part_lse = 0;
  size_t ws_bwd = 0, off_delta = 0, off_part_dq = 0, off_part_dk = 0, off_part_dv = 0, off_dbias = 0;
  size_t off_queue = 0;  // dK/dV work-queue counters (D = 128)
  int kv_resident = 1;   // dK/dV workgroups the GPU holds at once (grid of the persistent kernel)
  // timing
  bool timing = false;
  struct Rec {
    int kernel;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t pool_used = 0;
};

namespace {

jfa_status check_problem(const jfa_problem* p, std::vector<int>& lq, std::vector<int>& lkv) {
  if (!p) return fail(JFA_ERR_NULL_ARG, "problem is NULL");
  if (!p->q_offsets_host || !p->kv_offsets_host) return fail(JFA_ERR_NULL_ARG, "host offsets are NULL");
  if (p->num_seqs < 1) return fail(JFA_ERR_BAD_SHAPE, "num_seqs must be >= 1");
  if (p->num_heads < 1) return fail(JFA_ERR_BAD_SHAPE, "num_heads must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128) return fail(JFA_ERR_BAD_SHAPE, "head_dim must be 64 or 128");
  if (p->mask < 0 || p->mask > 1) return fail(JFA_ERR_UNSUPPORTED, "unknown mask mode");
  if (p->act < 0 || p->act > 2) return fail(JFA_ERR_UNSUPPORTED, "unknown activation");
  if (p->bias < 0 || p->bias > 2) return fail(JFA_ERR_UNSUPPORTED, "unknown bias kind");
  if (p->out_dtype < 0 || p->out_dtype > 1 || p->grad_dtype < 0 || p->grad_dtype > 1)
    return fail(JFA_ERR_UNSUPPORTED, "unknown dtype");
  if (p->num_slots < 0) return fail(JFA_ERR_BAD_SHAPE, "num_slots must be >= 0");
  // A negative scale would flip the order of the scores that the masks rely on (-inf stays the
  // smallest score only for a non-negative multiplier).
  if (!std::isfinite(p->scale) || p->scale < 0.0f) return fail(JFA_ERR_UNSUPPORTED, "scale must be finite and >= 0");
  if ((p->flags & ~(JFA_PLAN_HOST_ONLY | JFA_PLAN_NO_SPLIT | JFA_PLAN_SHARED_Q | JFA_PLAN_MXFP8)) != 0)
    return fail(JFA_ERR_UNSUPPORTED, "unknown flags");
  if (p->flags & JFA_PLAN_MXFP8) {
    if (p->head_dim != 128) return fail(JFA_ERR_BAD_SHAPE, "MXFP8 needs head_dim 128");
    if (p->act != JFA_ACT_SOFTMAX) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 supports the softmax activation only");
    if (p->flags & JFA_PLAN_SHARED_Q) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 does not take shared queries");
  }
  if (p->window < 0 || p->block < 0) return fail(JFA_ERR_BAD_SHAPE, "window and block must be >= 0");
  const int B = p->num_seqs;
  if (p->q_offsets_host[0] != 0 || p->kv_offsets_host[0] != 0) return fail(JFA_ERR_BAD_OFFSETS, "offsets[0] must be 0");
  lq.resize(B);
  lkv.resize(B);
  for (int b = 0; b < B; ++b) {
    const int64_t a = (int64_t)p->q_offsets_host[b + 1] - p->q_offsets_host[b];
    const int64_t c = (int64_t)p->kv_offsets_host[b + 1] - p->kv_offsets_host[b];
    if (a < 0 || c < 0) return fail(JFA_ERR_BAD_OFFSETS, "offsets must be non-decreasing (sequence " + std::to_string(b) + ")");
    lq[b] = (int)a;
    lkv[b] = (int)c;
    // Causal: j <= i. With more queries than keys, the rows past the keys are target rows that see
    // every key (the fused self + target pass); fewer queries than keys has no such reading.
    if (p->mask == JFA_MASK_CAUSAL && a < c)
      return fail(JFA_ERR_BAD_SHAPE, "causal mask needs Lq >= Lkv (sequence " + std::to_string(b) + ")");
    if ((p->flags & JFA_PLAN_SHARED_Q) && a != lq[0])
      return fail(JFA_ERR_BAD_SHAPE, "shared queries need the same Lq for every sequence (sequence " + std::to_string(b) + ")");
  }
  const int64_t tq = p->q_offsets_host[B], tkv = p->kv_offsets_host[B];
  if (tq * p->num_heads * (int64_t)p->head_dim >= ((int64_t)1 << 40) || tkv * p->num_heads * (int64_t)p->head_dim >= ((int64_t)1 << 40))
    return fail(JFA_ERR_BAD_SHAPE, "tensor too large");
  // The kernels address a (sequence, head) slice with signed 32-bit byte offsets from its first row,
  // up to one tile (at most 128 rows) past its end where ragged tails read zeros: (L + 128) rows of
  // H * D elements must stay within 2^30 elements (2^31 bytes).
  for (int b = 0; b < B; ++b) {
    const int64_t L = std::max(lq[b], lkv[b]);
    if (L > 0 && (L + 128) * p->num_heads * (int64_t)p->head_dim > kMaxSliceElems)
      return fail(JFA_ERR_BAD_SHAPE, "sequence " + std::to_string(b) + " spans more than 2^30 elements of a [T, H, D] "
                                     "tensor (its length times H times D); split it or shard the heads");
  }
  return JFA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Timing events only measure: recording one skips the system-scope memory fence (cache write-back
// and invalidation) that a default event performs, which would otherwise slow the launches it
// brackets.
hipEvent_t take_event(jfa_plan_s* P) {
  if (P->pool_used == P->pool.size()) {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    P->pool.push_back(e);
  }
  return P->pool[P->pool_used++];
}

// Launch `fn` on stream s, bracketed by timing events when timing is on.
template <class F>
jfa_status timed(jfa_plan_s* P, int kernel, hipStream_t s, F fn, const char* what) {
  hipEvent_t a = nullptr, b = nullptr;
  if (P->timing) {
    a = take_event(P);
    b = take_event(P);
    if (!a || !b) return fail(JFA_ERR_HIP, "hipEventCreate failed");
    const hipError_t e = hipEventRecord(a, s);
    if (e != hipSuccess) return hip_fail(e, "timing event record");
  }
  hipError_t e = fn();
  if (e != hipSuccess) return hip_fail(e, what);
  if (P->timing) {
    e = hipEventRecord(b, s);
    if (e != hipSuccess) return hip_fail(e, "timing event record");
    P->recs.push_back({kernel, a, b});
  }
  return JFA_OK;
}

// With JFA_DEBUG=1 in the environment, device offsets passed to a pass are copied back (a
// synchronising check) and compared with the offsets the plan was built from.
jfa_status debug_check_offsets(jfa_plan_s* P, const int32_t* dq, const int32_t* dkv, hipStream_t s) {
  const char* env = std::getenv("JFA_DEBUG");
  if (!env || env[0] != '1' || (!dq && !dkv)) return JFA_OK;
  std::vector<int32_t> a(P->B + 1), b(P->B + 1);
  if (hipStreamSynchronize(s) != hipSuccess) return fail(JFA_ERR_HIP, "JFA_DEBUG sync failed");
  if ((dq && hipMemcpy(a.data(), dq, a.size() * 4, hipMemcpyDeviceToHost) != hipSuccess) ||
      (dkv && hipMemcpy(b.data(), dkv, b.size() * 4, hipMemcpyDeviceToHost) != hipSuccess))
    return fail(JFA_ERR_HIP, "JFA_DEBUG offset copy failed");
  if ((dq && a != P->q_off) || (dkv && b != P->kv_off))
    return fail(JFA_ERR_BAD_OFFSETS, "device offsets differ from the planned host offsets");
  return JFA_OK;
}

// ---------------------------------------------------------------- forward / backward
// Argument checks of one pass (everything but the workspace), before any launch.
jfa_status check_forward(jfa_plan_s* P, const void* q, const void* k, const void* v, const float* bias,
                         const void* out, const float* lse) {
  if (!P) return fail(JFA_ERR_NULL_ARG, "plan is NULL");
  if (P->flags & JFA_PLAN_HOST_ONLY) return fail(JFA_ERR_HOST_ONLY, "plan was built host-only");
  const bool softmax = P->modes.act == kSoftmax;
  if (!q || !k || !v || !out) return fail(JFA_ERR_NULL_ARG, "a tensor pointer is NULL");
  if (P->modes.bias != kBiasNone && !bias) return fail(JFA_ERR_NULL_ARG, "bias is NULL");
  if (softmax && !lse) return fail(JFA_ERR_NULL_ARG, "lse is NULL (required for softmax)");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && !aligned16(lse)) ||
      (bias && !aligned16(bias)))
    return fail(JFA_ERR_MISALIGNED, "tensor pointers must be 16-byte aligned");
  return JFA_OK;
}

jfa_status check_backward(jfa_plan_s* P, const void* q, const void* k, const void* v, const float* bias,
                          const void* out, const float* lse, const void* dout, const void* dq, const void* dk,
                          const void* dv, const float* dbias) {
  if (!P) return fail(JFA_ERR_NULL_ARG, "plan is NULL");
  if (P->flags & JFA_PLAN_HOST_ONLY) return fail(JFA_ERR_HOST_ONLY, "plan was built host-only");
  const bool softmax = P->modes.act == kSoftmax;
  if (dbias && P->modes.bias == kBiasNone) return fail(JFA_ERR_UNSUPPORTED, "dbias requested without a bias");
  if (P->mx) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 plans are forward only");
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return fail(JFA_ERR_NULL_ARG, "a tensor pointer is NULL");
  if (P->modes.bias != kBiasNone && !bias) return fail(JFA_ERR_NULL_ARG, "bias is NULL");
  if (softmax && (!out || !lse)) return fail(JFA_ERR_NULL_ARG, "out and lse are required for softmax");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || (out && !aligned16(out)) || (lse && !aligned16(lse)) || (bias && !aligned16(bias)) ||
      (dbias && !aligned16(dbias)))
    return fail(JFA_ERR_MISALIGNED, "tensor pointers must be 16-byte aligned");
  return JFA_OK;
}

// Launches of one pass on stream s with a checked workspace of the plan's size.
jfa_status run_forward(jfa_plan_s* P, const void* q, const void* k, const void* v, const float* bias, void* out,
                       float* lse, void* workspace, hipStream_t s) {
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bias = bias;
  a.out = out;
  a.lse = lse;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + P->off_part_lse) : nullptr;
  a.items = P->lists[kFwd].d_items;
  a.groups = P->lists[kFwd].d_groups;
  a.H = P->H;
  a.Tq = P->Tq;
  a.scale = P->scale;
  a.out_f32 = P->out_f32;
  a.band = P->band;
  a.q_shared = P->q_shared;
  const List& L = P->lists[kFwd];
  jfa_status st = JFA_OK;
  if (P->mx) {
    char* ws = static_cast<char*>(workspace);
    MxArgs x{};
    x.f = a;
    x.qq = reinterpret_cast<uint8_t*>(ws + P->off_qq);
    x.qs = reinterpret_cast<uint8_t*>(ws + P->off_qs);
    x.kq = reinterpret_cast<uint8_t*>(ws + P->off_kq);
    x.ks = reinterpret_cast<uint8_t*>(ws + P->off_ks);
    x.vq = reinterpret_cast<uint8_t*>(ws + P->off_vq);
    x.vs = reinterpret_cast<uint8_t*>(ws + P->off_vs);
    x.vtiles = P->d_vtiles;
    st = timed(P, 7, s, [&] { return launch_mx_quantize(x, P->Tq, P->Tkv, P->n_vtiles, s); }, "MXFP8 quantise launch");
    if (st != JFA_OK) return st;
    st = timed(P, 0, s, [&] { return launch_forward_mx(x, P->modes, (int)L.n_items(), s); }, "MXFP8 forward launch");
  } else {
    st = timed(P, 0, s, [&] { return launch_forward(a, P->modes, (int)L.n_items(), s); }, "forward launch");
  }
  if (st != JFA_OK) return st;
  if (L.n_groups() > 0)
    st = timed(P, 1, s, [&] { return launch_forward_combine(a, P->modes, (int)L.n_groups(), s); }, "combine launch");
  return st;
}

jfa_status run_backward(jfa_plan_s* P, const void* q, const void* k, const void* v, const float* bias,
                        const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* dbias, void* workspace, hipStream_t s, bool allow_timing = true) {
  // Timing records events it may have to create; callers that cannot allocate switch it off.
  const bool timing = P->timing;
  P->timing = timing && allow_timing;
  struct Restore {
    jfa_plan_s* p;
    bool t;
    ~Restore() { p->timing = t; }
  } restore{P, timing};
  char* ws = static_cast<char*>(workspace);
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.bias = bias;
  a.out = out;
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = ws ? reinterpret_cast<float*>(ws + P->off_delta) : nullptr;
  a.part_dq = ws ? reinterpret_cast<float*>(ws + P->off_part_dq) : nullptr;
  a.part_dk = ws ? reinterpret_cast<float*>(ws + P->off_part_dk) : nullptr;
  a.part_dv = ws ? reinterpret_cast<float*>(ws + P->off_part_dv) : nullptr;
  a.dbias_acc = (ws && dbias) ? reinterpret_cast<unsigned long long*>(ws + P->off_dbias) : nullptr;
  a.dbias = dbias;
  a.dq_items = P->lists[kDq].d_items;
  a.dq_groups = P->lists[kDq].d_groups;
  a.kv_items = P->lists[kKv].d_items;
  a.kv_groups = P->lists[kKv].d_groups;
  a.H = P->H;
  a.Tq = P->Tq;
  a.Tkv = P->Tkv;
  a.scale = P->scale;
  a.out_f32 = P->out_f32;
  a.band = P->band;
  a.grad_f32 = P->grad_f32;
  a.kv_bn = P->kv_bn;
  a.kv_queue = (ws && P->D == 128) ? reinterpret_cast<int*>(ws + P->off_queue) : nullptr;
  a.kv_n = (int)P->lists[kKv].n_items();
  a.q_shared = P->q_shared;
  Modes m = P->modes;
  m.dbias = dbias ? 1 : 0;
  jfa_status st = JFA_OK;
  if (P->fused_bwd) {
    // one pass over the dQ items: dQ (or its partial sums) and the dK / dV of every key
    if (dbias) {
      st = timed(P, 6, s, [&] { return launch_bwd_dbias_clear(a, m, s); }, "bias-gradient clear launch");
      if (st != JFA_OK) return st;
    }
    st = timed(P, 8, s, [&] { return launch_bwd_fused(a, m, (int)P->lists[kDq].n_items(), s); }, "fused backward launch");
    if (st != JFA_OK) return st;
    if (P->lists[kDq].n_groups() > 0) {
      // shared queries: one piece per sequence in every group, summed by many workgroups per group
      const int ng = (int)P->lists[kDq].n_groups();
      st = timed(P, 5, s, [&] { return P->q_shared ? launch_bwd_reduce_dq_wide(a, m, ng, s) : launch_bwd_reduce_dq(a, m, ng, s); },
                 "dQ reduce launch");
      if (st != JFA_OK) return st;
    }
    if (dbias) st = timed(P, 6, s, [&] { return launch_bwd_dbias_finish(a, m, s); }, "bias-gradient finish launch");
    return st;
  }
  // The queue counters are zeroed by the dQ kernel, or here when there is no dQ item.
  if (dbias || (a.kv_queue && P->lists[kDq].n_items() == 0 && a.kv_n > 0)) {
    st = timed(P, 6, s, [&] { return launch_bwd_dbias_clear(a, m, s); }, "bias-gradient clear launch");
    if (st != JFA_OK) return st;
  }
  // dQ first: it also computes Delta = rowsum(dO * O) (softmax) for the dK/dV kernel.
  st = timed(P, 4, s, [&] { return launch_bwd_dq(a, m, (int)P->lists[kDq].n_items(), s); }, "dQ launch");
  if (st != JFA_OK) return st;
  // The persistent dK/dV kernel (D = 128, full-width items) takes the dQ partial sums once its items
  // are exhausted; otherwise a reduce kernel does.
  const int dq_groups = (int)P->lists[kDq].n_groups();
  const bool dq_in_kv = P->D == 128 && !P->modes.kv_short && a.kv_n > 0 && dq_groups > 0;
  a.dq_reduce_n = dq_in_kv ? dq_groups : 0;
  if (dq_groups > 0 && !dq_in_kv) {
    st = timed(P, 5, s, [&] { return launch_bwd_reduce_dq(a, m, dq_groups, s); }, "dQ reduce launch");
    if (st != JFA_OK) return st;
  }
  st = timed(P, 3, s, [&] { return launch_bwd_dkdv(a, m, a.kv_n, P->kv_resident, s); }, "dK/dV launch");
  if (st != JFA_OK) return st;
  if (P->lists[kKv].n_groups() > 0) {
    st = timed(P, 5, s, [&] { return launch_bwd_reduce_dkdv(a, m, (int)P->lists[kKv].n_groups(), s); }, "dK/dV reduce launch");
    if (st != JFA_OK) return st;
  }
  if (dbias) st = timed(P, 6, s, [&] { return launch_bwd_dbias_finish(a, m, s); }, "bias-gradient finish launch");
  return st;
}

// Record that the plan's device lists are read by work enqueued on stream s (up to this point).
jfa_status note_use(jfa_plan_s* P, hipStream_t s) {
  std::lock_guard<std::mutex> lk(P->use_mu);
  for (auto& u : P->uses)
    if (u.first == s) {
      const hipError_t e = hipEventRecord(u.second, s);
      return e == hipSuccess ? JFA_OK : hip_fail(e, "event record");
    }
  hipEvent_t ev = cache_event();
  if (!ev) return fail(JFA_ERR_HIP, "event creation failed");
  const hipError_t e = hipEventRecord(ev, s);
  P->uses.push_back({s, ev});  // kept even on failure, so that the event is recycled with the plan
  return e == hipSuccess ? JFA_OK : hip_fail(e, "event record");
}

}  // namespace

namespace jfa {

// jfa_backward with a workspace the library provides itself (the allocation-free entry point):
// the same checks and launches, no timing events, no use-tracking event.
jfa_status backward_into(jfa_plan_s* P, const void* q, const void* k, const void* v, const int32_t* q_offsets,
                         const int32_t* kv_offsets, const float* bias, const void* out, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* dbias, void* (*workspace)(size_t, jfa_status*),
                         hipStream_t s) {
  jfa_status st = check_backward(P, q, k, v, bias, out, lse, dout, dq, dk, dv, dbias);
  if (st != JFA_OK) return st;
  void* ws = workspace(P->ws_bwd, &st);
  if (st != JFA_OK) return st;
  st = debug_check_offsets(P, q_offsets, kv_offsets, s);
  if (st != JFA_OK) return st;
  return run_backward(P, q, k, v, bias, out, lse, dout, dq, dk, dv, dbias, ws, s, false);
}

jfa_status set_error(jfa_status s, const char* msg) { return fail(s, msg); }

}  // namespace jfa

extern "C" {

jfa_status jfa_plan(const jfa_problem* problem, jfa_stream_t stream, jfa_plan_t* plan_out) {
  if (!plan_out) return fail(JFA_ERR_NULL_ARG, "plan_out is NULL");
  *plan_out = nullptr;
  std::vector<int> lq, lkv;
  jfa_status st = check_problem(problem, lq, lkv);
  if (st != JFA_OK) return st;
  const jfa_problem& p = *problem;
  jfa_plan_s* P = new (std::nothrow) jfa_plan_s();
  if (!P) return fail(JFA_ERR_UNSUPPORTED, "out of host memory");
  P->B = p.num_seqs;
  P->H = p.num_heads;
  P->D = p.head_dim;
  P->q_off.assign(p.q_offsets_host, p.q_offsets_host + P->B + 1);
  P->kv_off.assign(p.kv_offsets_host, p.kv_offsets_host + P->B + 1);
  P->Tq = P->q_off[P->B];
  P->Tkv = P->kv_off[P->B];
  P->modes = Modes{p.head_dim, p.act, p.bias, p.mask == JFA_MASK_CAUSAL ? 1 : 0};
  P->band = Band{p.window, p.block, p.mask == JFA_MASK_CAUSAL ? 1 : 0};
  P->modes.band = (p.window > 0 || p.block > 0) ? 1 : 0;
  {
    int max_lq = 0;
    for (int x : lq) max_lq = std::max(max_lq, x);
    // softmax only: the GDPA hand-off (P and act'/Lkv) needs too much LDS for two workgroups per CU
    P->modes.kv_short = (p.head_dim == 128 && p.act == kSoftmax && max_lq <= kKvBM) ? 1 : 0;
  }
  P->kv_bn = P->modes.kv_short ? kKvBNShort : kKvBN;
  P->scale = p.scale != 0.0f ? p.scale : 1.0f / std::sqrt((float)p.head_dim);
  P->out_f32 = p.out_dtype == JFA_F32;
  P->grad_f32 = p.grad_dtype == JFA_F32;
  P->flags = p.flags;
  const bool host_only = (p.flags & JFA_PLAN_HOST_ONLY) != 0;
  const bool split = (p.flags & JFA_PLAN_NO_SPLIT) == 0;

  int slots[3] = {p.num_slots, p.num_slots, p.num_slots};
  if (!host_only) {
    int cus = 0, occ[3] = {1, 1, 1};
    hipError_t e = hipGetDevice(&P->device);
    if (e == hipSuccess) e = device_info(P->device, P->modes, cus, occ);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "device query");
    }
    if (p.num_slots == 0)
      for (int l = 0; l < 3; ++l) slots[l] = cus * occ[l];
    P->kv_resident = std::max(1, cus * occ[kKv]);
  } else if (p.num_slots == 0) {
    slots[0] = slots[1] = slots[2] = 512;
  }
  const Limits lim{P->modes.causal != 0, p.window, p.block};
  query_tile_list(lq, lkv, P->H, lim, kFwdBM, kFwdBN, slots[kFwd], split, P->lists[kFwd]);
  query_tile_list(lq, lkv, P->H, lim, kDqBM, kDqBN, slots[kDq], split, P->lists[kDq]);
  key_tile_list(lq, lkv, P->H, lim, kKvBM, P->kv_bn, slots[kKv], split, P->lists[kKv]);
  P->mx = (p.flags & JFA_PLAN_MXFP8) ? 1 : 0;
  if (P->mx) {
    P->vtile0.assign(P->B + 1, 0);
    for (int b = 0; b < P->B; ++b) {
      const int n = ceil_div(lkv[b], kFwdBN);
      for (int t = 0; t < n; ++t)
        P->vtiles.insert(P->vtiles.end(), {P->kv_off[b] + t * kFwdBN, std::min(kFwdBN, lkv[b] - t * kFwdBN)});
      P->vtile0[b + 1] = P->vtile0[b] + n;
    }
    P->n_vtiles = P->vtile0[P->B];
    // the kernels address quantised V tiles with 32-bit byte offsets
    if ((int64_t)P->n_vtiles * P->H * kFwdBN * 128 >= ((int64_t)1 << 32)) {
      delete P;
      return fail(JFA_ERR_BAD_SHAPE, "MXFP8: quantised V beyond 4 GiB");
    }
  }
  P->q_shared = (p.flags & JFA_PLAN_SHARED_Q) ? 1 : 0;
  if (P->q_shared) share_query_slots(P->lists[kDq]);
  if (P->D == 128 && !P->modes.band) {
    bool fits = true;
    for (int b = 0; b < P->B; ++b) fits = fits && lq[b] <= kKvBM && (lq[b] > 0 || lkv[b] == 0);
    P->fused_bwd = fits ? 1 : 0;
  }
  for (auto& L : P->lists) L.order = dispatch_order(L, P->B, P->H);

  // workspace layout
  const size_t D = P->D;
  P->ws_fwd = align256((size_t)P->lists[kFwd].nslots * kFwdBM * D * 4);
  P->off_part_lse = P->ws_fwd;
  P->ws_fwd += align256((size_t)P->lists[kFwd].nslots * kFwdBM * 4);
  if (P->mx) {  // quantised copies of Q, K, V and their block scales
    const size_t H = P->H;
    P->off_qq = P->ws_fwd;
    P->off_qs = P->off_qq + align256((size_t)P->Tq * H * D);
    P->off_kq = P->off_qs + align256((size_t)P->Tq * H * (D / 32));
    P->off_ks = P->off_kq + align256((size_t)P->Tkv * H * D);
    P->off_vq = P->off_ks + align256((size_t)P->Tkv * H * (D / 32));
    P->off_vs = P->off_vq + align256((size_t)P->n_vtiles * H * D * kFwdBN);
    P->ws_fwd = P->off_vs + align256((size_t)P->n_vtiles * H * 2 * D);
  }
  size_t o = 0;
  P->off_delta = o;
  if (P->modes.act == kSoftmax) o += align256((size_t)P->H * P->Tq * 4);
  P->off_part_dq = o;
  o += align256((size_t)P->lists[kDq].nslots * kDqBM * D * 4);
  P->off_part_dk = o;
  o += align256((size_t)P->lists[kKv].nslots * P->kv_bn * D * 4);
  P->off_part_dv = o;
  o += align256((size_t)P->lists[kKv].nslots * P->kv_bn * D * 4);
  P->off_dbias = o;  // fixed-point bias-gradient totals, used when the caller asks for dbias
  if (P->modes.bias != kBiasNone) o += align256((size_t)P->H * (P->modes.bias == kBiasBucket ? kBuckets : 1) * 8);
  P->off_queue = o;
  if (P->D == 128) o += align256(kQueueCounters * 4);
  P->ws_bwd = o;
  if (P->lists[kFwd].nslots == 0 && !P->mx) P->ws_fwd = 0;

  if (!host_only) {
    // Device records (kItemInts / kGroupInts int32 each): the list fields followed by the sequence's
    // offsets and lengths, so that a workgroup needs no second, dependent load. They are written
    // straight into pinned staging memory and uploaded asynchronously; nothing waits for the copy.
    size_t total = 0;
    for (auto& L : P->lists) total += L.n_items() * kItemInts + L.n_groups() * kGroupInts;
    total += P->vtiles.size();
    total = std::max<size_t>(total, kItemInts);
    CachedBuf stage;
    hipError_t e = cache_acquire(total * 4, true, P->device, stage);
    if (e == hipSuccess) e = cache_acquire(total * 4, false, P->device, P->dev);
    if (e != hipSuccess) {
      cache_release(stage);
      cache_release(P->dev);
      delete P;
      return hip_fail(e, "plan buffer allocation");
    }
    int32_t* host = static_cast<int32_t*>(stage.ptr);
    auto put_seq = [&](int32_t* r, int b) {
      r[0] = P->q_off[b];
      r[1] = P->q_off[b + 1] - P->q_off[b];
      r[2] = P->kv_off[b];
      r[3] = P->kv_off[b + 1] - P->kv_off[b];
    };
    size_t pos = 0;
    size_t offs[3][2];
    for (int l = 0; l < 3; ++l) {
      List& L = P->lists[l];
      offs[l][0] = pos;
      for (size_t i = 0; i < L.n_items(); ++i, pos += kItemInts) {
        const int32_t* it = &L.items[(size_t)L.order[i] * 6];
        int32_t* r = host + pos;
        std::copy_n(it, 6, r);
        put_seq(r + 6, it[0]);
        r[10] = L.first[(size_t)L.order[i]] ? 1 : 0;
        std::fill(r + 11, r + kItemInts, 0);
        if (P->mx) r[11] = P->vtile0[it[0]];  // MXFP8: the sequence's first quantised V tile
      }
      offs[l][1] = pos;
      for (size_t g = 0; g < L.n_groups(); ++g, pos += kGroupInts) {
        const int32_t* gr = &L.groups[g * 5];
        int32_t* r = host + pos;
        std::copy_n(gr, 5, r);
        put_seq(r + 5, gr[0]);
        std::fill(r + 9, r + kGroupInts, 0);
      }
    }
    const size_t off_vt = pos;
    std::copy(P->vtiles.begin(), P->vtiles.end(), host + pos);
    pos += P->vtiles.size();
    if (pos == 0) std::fill(host, host + kItemInts, 0);
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t copied = cache_event(), used = cache_event();
    e = (copied && used) ? hipMemcpyAsync(P->dev.ptr, host, total * 4, hipMemcpyHostToDevice, s) : hipErrorOutOfMemory;
    if (e == hipSuccess) e = hipEventRecord(copied, s);
    if (e == hipSuccess) e = hipEventRecord(used, s);
    if (e != hipSuccess) {
      // the copy may be in flight: wait for the stream before the buffers can be reused
      (void)hipStreamSynchronize(s);
      for (hipEvent_t x : {copied, used})
        if (x) (void)hipEventDestroy(x);
      cache_release(stage);
      cache_release(P->dev);
      delete P;
      return hip_fail(e, "plan upload");
    }
    stage.pending.push_back(copied);  // the staging memory is reusable once the copy has run
    cache_release(stage);
    P->uses.push_back({s, used});
    for (int l = 0; l < 3; ++l) {
      P->lists[l].d_items = static_cast<int32_t*>(P->dev.ptr) + offs[l][0];
      P->lists[l].d_groups = static_cast<int32_t*>(P->dev.ptr) + offs[l][1];
    }
    P->d_vtiles = static_cast<int32_t*>(P->dev.ptr) + off_vt;
  }
  *plan_out = P;
  return JFA_OK;
}

jfa_status jfa_workspace_bytes(jfa_plan_t P, size_t* fwd_bytes, size_t* bwd_bytes) {
  if (!P) return fail(JFA_ERR_NULL_ARG, "plan is NULL");
  if (fwd_bytes) *fwd_bytes = P->ws_fwd;
  if (bwd_bytes) *bwd_bytes = P->ws_bwd;
  return JFA_OK;
}

jfa_status jfa_forward(jfa_plan_t P, const void* q, const void* k, const void* v, const int32_t* q_offsets,
                       const int32_t* kv_offsets, const float* bias, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, jfa_stream_t stream) {
  jfa_status st = check_forward(P, q, k, v, bias, out, lse);
  if (st != JFA_OK) return st;
  if (!aligned16(workspace)) return fail(JFA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (workspace_bytes < P->ws_fwd || (P->ws_fwd > 0 && !workspace))
    return fail(JFA_ERR_WORKSPACE, "forward workspace needs " + std::to_string(P->ws_fwd) + " bytes");
  hipStream_t s = (hipStream_t)stream;
  st = debug_check_offsets(P, q_offsets, kv_offsets, s);
  if (st != JFA_OK) return st;
  st = run_forward(P, q, k, v, bias, out, lse, workspace, s);
  const jfa_status su = note_use(P, s);
  return st != JFA_OK ? st : su;
}

jfa_status jfa_backward(jfa_plan_t P, const void* q, const void* k, const void* v, const int32_t* q_offsets,
                        const int32_t* kv_offsets, const float* bias, const void* out, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* dbias, void* workspace,
                        size_t workspace_bytes, jfa_stream_t stream) {
  jfa_status st = check_backward(P, q, k, v, bias, out, lse, dout, dq, dk, dv, dbias);
  if (st != JFA_OK) return st;
  if (!aligned16(workspace)) return fail(JFA_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (workspace_bytes < P->ws_bwd || (P->ws_bwd > 0 && !workspace))
    return fail(JFA_ERR_WORKSPACE, "backward workspace needs " + std::to_string(P->ws_bwd) + " bytes");
  hipStream_t s = (hipStream_t)stream;
  st = debug_check_offsets(P, q_offsets, kv_offsets, s);
  if (st != JFA_OK) return st;
  st = run_backward(P, q, k, v, bias, out, lse, dout, dq, dk, dv, dbias, workspace, s);
  const jfa_status su = note_use(P, s);
  return st != JFA_OK ? st : su;
}

jfa_status jfa_plan_schedule(jfa_plan_t P, int32_t which, int32_t* out, size_t cap, size_t* count) {
  if (!P || !count) return fail(JFA_ERR_NULL_ARG, "plan or count is NULL");
  if (which < 0 || which > 8) return fail(JFA_ERR_UNSUPPORTED, "which must be 0..8");
  if (which >= 6) {  // items in dispatch order
    const List& D = P->lists[which - 6];
    *count = D.n_items();
    for (size_t i = 0; i < std::min(*count, cap) && out; ++i) std::copy_n(&D.items[(size_t)D.order[i] * 6], 6, out + i * 6);
    return JFA_OK;
  }
  const List& L = P->lists[which / 2];
  const bool groups = (which & 1) != 0;
  const std::vector<int32_t>& v = groups ? L.groups : L.items;
  const size_t per = groups ? 5 : 6;
  *count = v.size() / per;
  if (out) std::copy_n(v.data(), std::min(*count, cap) * per, out);
  return JFA_OK;
}

jfa_status jfa_plan_info(jfa_plan_t P, int32_t* info, size_t n) {
  if (!P || !info) return fail(JFA_ERR_NULL_ARG, "plan or info is NULL");
  const int32_t v[10] = {kFwdBM, kFwdBN, kDqBM, kDqBN, kKvBM, P->kv_bn, P->lists[kFwd].slots, P->lists[kDq].slots,
                         P->lists[kKv].slots, P->fused_bwd};
  std::copy_n(v, std::min<size_t>(n, 10), info);
  return JFA_OK;
}

jfa_status jfa_timing_enable(jfa_plan_t P, int32_t enable) {
  if (!P) return fail(JFA_ERR_NULL_ARG, "plan is NULL");
  P->timing = enable != 0;
  P->recs.clear();
  P->pool_used = 0;
  return JFA_OK;
}

jfa_status jfa_timing_read(jfa_plan_t P, int32_t kernel, float* total_ms, int32_t* launches) {
  if (!P || !total_ms || !launches) return fail(JFA_ERR_NULL_ARG, "NULL argument");
  float sum = 0.0f;
  int n = 0;
  for (const auto& r : P->recs) {
    if (r.kernel != kernel) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "timing read");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return JFA_OK;
}

void jfa_plan_destroy(jfa_plan_t P) {
  if (!P) return;
  if (P->dev.ptr) {
    // The lists go back to the cache with the last use on every stream; no wait here.
    for (auto& u : P->uses) P->dev.pending.push_back(u.second);
    P->uses.clear();
    cache_release(P->dev);
  }
  for (hipEvent_t e : P->pool) (void)hipEventDestroy(e);
  delete P;
}

const char* jfa_status_string(jfa_status s) {
  switch (s) {
    case JFA_OK: return "JFA_OK";
    case JFA_ERR_NULL_ARG: return "JFA_ERR_NULL_ARG";
    case JFA_ERR_BAD_OFFSETS: return "JFA_ERR_BAD_OFFSETS";
    case JFA_ERR_BAD_SHAPE: return "JFA_ERR_BAD_SHAPE";
    case JFA_ERR_UNSUPPORTED: return "JFA_ERR_UNSUPPORTED";
    case JFA_ERR_MISALIGNED: return "JFA_ERR_MISALIGNED";
    case JFA_ERR_WORKSPACE: return "JFA_ERR_WORKSPACE";
    case JFA_ERR_HIP: return "JFA_ERR_HIP";
    case JFA_ERR_HOST_ONLY: return "JFA_ERR_HOST_ONLY";
  }
  return "JFA_ERR_UNKNOWN";
}

const char* jfa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

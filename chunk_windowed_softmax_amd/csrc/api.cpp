// C ABI of the chunk-windowed softmax attention library: plan cache, argument checks,
// device resources and launches.  Declarations and contracts: include/wa.h.
//
// Plans are cached by geometry, at most four (lqnn.cn article on VDN-Minimax-H3 window
// attention, §三: the decomposed form's plan is cached per geometry shape, four plans).
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "wa.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

struct DeviceResources {
  wa::Item* items = nullptr;
  float* part = nullptr;     // partial O then partial (m, l) of the global leg
  void* staging = nullptr;   // bf16 copies of fp32 q, k, v (allocated on first fp32 call)
  int64_t staging_bytes = 0;
  int n_cus = 0;             // compute units of the device: one persistent block each
  // Ordering of calls that share this plan's tables, queue counters and workspace: the
  // event is recorded on the stream of the last call, and a call on another stream first
  // makes its stream wait for it.
  hipEvent_t done = nullptr;
  hipStream_t last_stream = nullptr;
  bool launched = false;
};

}  // namespace

struct wa_plan {
  wa::HostPlan host;
  // Image of the plan's device tables as int32: the work items, the launch order,
  // kXcdCount + 1 zeroed work-queue counters, then the tile lists of a block-sparse plan
  // (uploaded as one block).
  std::vector<int32_t> table;
  std::atomic<int> refs{1};
  std::atomic<bool> cached{true};
  std::mutex dev_mu;     // creation of device resources, staging growth
  std::mutex launch_mu;  // stream ordering + launches of one call (see DeviceResources::done)
  std::map<int, DeviceResources> dev;

  ~wa_plan() {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    for (auto& kv : dev) {
      if (hipSetDevice(kv.first) != hipSuccess) continue;
      if (kv.second.items) (void)hipFree(kv.second.items);
      if (kv.second.part) (void)hipFree(kv.second.part);
      if (kv.second.staging) (void)hipFree(kv.second.staging);
      if (kv.second.done) (void)hipEventDestroy(kv.second.done);
    }
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

namespace {

constexpr size_t kCacheCapacity = 4;
std::mutex g_cache_mu;
// Front = most recently created or fetched.  Cached plans live until the process ends: the
// list is never destroyed (no plan is freed during static destruction, when the HIP
// runtime may already be gone), so the plans it holds stay reachable to the end.
std::list<wa_plan*>& g_cache = *new std::list<wa_plan*>;

void unref(wa_plan* p) {
  if (p->refs.fetch_sub(1) == 1) delete p;
}

// Device tables and workspace of `p` on the current device (created on first use).
int device_resources(wa_plan* p, DeviceResources** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(p->dev_mu);
  auto found = p->dev.find(dev);
  if (found != p->dev.end()) {
    *out = &found->second;
    return WA_OK;
  }
  DeviceResources r;
  e = hipDeviceGetAttribute(&r.n_cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || r.n_cus < 1) return fail(WA_ERR_HIP, "hipDeviceGetAttribute(multiprocessor count) failed");
  // items, then the launch order (int32), then the work-queue counters, in one allocation
  // filled by one blocking copy (the counters must read zero before the first launch, on
  // whatever stream it comes)
  const size_t table_bytes = p->table.size() * sizeof(int32_t);
  e = hipMalloc(&r.items, table_bytes);
  if (e != hipSuccess) return fail(WA_ERR_ALLOC, std::string("hipMalloc(items): ") + hipGetErrorString(e));
  e = hipMemcpy(r.items, p->table.data(), table_bytes, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(r.items);
    return fail(WA_ERR_HIP, std::string("hipMemcpy(items): ") + hipGetErrorString(e));
  }
  e = hipEventCreateWithFlags(&r.done, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipFree(r.items);
    return fail(WA_ERR_HIP, std::string("hipEventCreate: ") + hipGetErrorString(e));
  }
  if (p->host.partial_bytes > 0) {
    e = hipMalloc(&r.part, (size_t)p->host.partial_bytes);
    if (e != hipSuccess) {
      (void)hipFree(r.items);
      (void)hipEventDestroy(r.done);
      return fail(WA_ERR_ALLOC, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
    }
  }
  *out = &(p->dev[dev] = r);
  return WA_OK;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

bool overlaps(const void* a, const void* b, size_t n) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

// Enqueue one call's work that uses the plan's device tables, queue counters and workspace:
// under the plan's launch lock, when the plan's previous call went to another stream, make
// `stream` wait for it first; then run `enqueue` and record the plan's event on `stream`.
// Calls that share a plan (equal geometries share one) so never overlap on the device.
template <class F>
int ordered_launch(wa_plan* p, DeviceResources* r, hipStream_t stream, const char* who, F&& enqueue) {
  std::lock_guard<std::mutex> lk(p->launch_mu);
  if (r->launched && r->last_stream != stream) {
    const hipError_t e = hipStreamWaitEvent(stream, r->done, 0);
    if (e != hipSuccess) return fail(WA_ERR_HIP, std::string(who) + ": hipStreamWaitEvent: " + hipGetErrorString(e));
  }
  const int st = enqueue();
  if (st != WA_OK) return st;
  const hipError_t e = hipEventRecord(r->done, stream);
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string(who) + ": hipEventRecord: " + hipGetErrorString(e));
  r->launched = true;
  r->last_stream = stream;
  return WA_OK;
}

// One-line summary of a newly built plan on stderr when the environment sets WA_LOG=1.
void log_plan(const wa::HostPlan& h, double build_us) {
  const char* env = std::getenv("WA_LOG");
  if (!env || std::strcmp(env, "1") != 0) return;
  std::fprintf(stderr,
               "wa: plan %s T=%d S=%d G=%d K=%d radius=%d H=%d d=%d: L=%d chunks=%d groups=%zu items=%zu "
               "(window %d) splits=%d queue=%dx%d kept_pairs/head=%lld workspace=%lld B, built in %.0f us\n",
               h.geo.causal ? "causal" : "window", h.geo.T, h.geo.S, h.geo.G, h.geo.K, h.geo.radius, h.geo.H,
               h.geo.d, h.L, h.n_chunks, h.groups.size(), h.items.size(), h.n_window_items, h.n_splits, wa::kXcdCount,
               h.work_per_xcd, (long long)h.kept_pairs_per_head, (long long)h.partial_bytes, build_us);
}

}  // namespace

extern "C" {

// Fetch the cached plan of `geo` or build and cache it (shared by both plan constructors).
static int create_cached(const wa::Geometry& geo, wa_plan** out, const char* who) {
  if (!out) return fail(WA_ERR_INVALID, std::string(who) + ": out is NULL");
  *out = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (auto it = g_cache.begin(); it != g_cache.end(); ++it) {
      if ((*it)->host.geo == geo) {
        wa_plan* p = *it;
        g_cache.erase(it);
        g_cache.push_front(p);
        p->refs.fetch_add(1);
        *out = p;
        return WA_OK;
      }
    }
  }
  wa::HostPlan hp;
  std::string err;
  const auto t0 = std::chrono::steady_clock::now();
  const int st = geo.causal        ? wa::build_causal_plan(geo.S, geo.H, geo.d, &hp, &err)
                 : geo.block_q > 0 ? wa::build_blocksparse_plan(geo, &hp, &err)
                                   : wa::build_plan(geo, &hp, &err);
  if (st != 0) return fail(st, std::string(who) + ": " + err);
  log_plan(hp, std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count());
  wa_plan* p = nullptr;
  try {
    p = new wa_plan();
  } catch (...) {
    return fail(WA_ERR_ALLOC, std::string(who) + ": out of host memory");
  }
  p->host = std::move(hp);
  {
    const wa::HostPlan& h = p->host;
    const size_t item_words = h.items.size() * (sizeof(wa::Item) / sizeof(int32_t));
    const size_t tiles_at = item_words + h.work.size() + (wa::kXcdCount + 1);
    p->table.assign(tiles_at + h.tiles.size(), 0);
    std::memcpy(p->table.data(), h.items.data(), item_words * sizeof(int32_t));
    std::memcpy(p->table.data() + item_words, h.work.data(), h.work.size() * sizeof(int32_t));
    if (!h.tiles.empty()) std::memcpy(p->table.data() + tiles_at, h.tiles.data(), h.tiles.size() * sizeof(int32_t));
  }
  p->refs.store(2);  // the caller's handle + the cache's
  wa_plan* evicted = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (wa_plan* other : g_cache) {
      if (other->host.geo == geo) {  // another thread built the same plan meanwhile
        other->refs.fetch_add(1);
        delete p;
        *out = other;
        return WA_OK;
      }
    }
    g_cache.push_front(p);
    if (g_cache.size() > kCacheCapacity) {
      evicted = g_cache.back();
      g_cache.pop_back();
      evicted->cached.store(false);
    }
  }
  if (evicted) unref(evicted);
  *out = p;
  return WA_OK;
}

int wa_plan_create(int T, int S, int G, int K, int radius, int H, int d, wa_plan** out) {
  return create_cached(wa::Geometry{T, S, G, K, radius, H, d, 0}, out, "wa_plan_create");
}

int wa_blocksparse_plan_create(int T, int S, int G, int K, int radius, int H, int d, int block_q, int block_kv,
                               wa_plan** out) {
  if (block_q <= 0 || block_kv <= 0)
    return fail(WA_ERR_INVALID, "wa_blocksparse_plan_create: block sizes must be positive");
  wa::Geometry geo{T, S, G, K, radius, H, d, 0};
  geo.block_q = block_q;
  geo.block_kv = block_kv;
  return create_cached(geo, out, "wa_blocksparse_plan_create");
}

int wa_causal_plan_create(int n, int H, int d, wa_plan** out) {
  return create_cached(wa::Geometry{1, n, 0, 1, 0, H, d, 1}, out, "wa_causal_plan_create");
}

int wa_plan_release(wa_plan* plan) {
  if (!plan) return fail(WA_ERR_INVALID, "wa_plan_release: plan is NULL");
  unref(plan);
  return WA_OK;
}

int wa_plan_info(const wa_plan* plan, wa_plan_info_t* info) {
  if (!plan || !info) return fail(WA_ERR_INVALID, "wa_plan_info: NULL argument");
  const wa::HostPlan& h = plan->host;
  std::memset(info, 0, sizeof(*info));
  info->T = h.geo.T;
  info->S = h.geo.S;
  info->G = h.geo.G;
  info->K = h.geo.K;
  info->radius = h.geo.radius;
  info->H = h.geo.H;
  info->d = h.geo.d;
  info->L = h.L;
  info->n_chunks = h.n_chunks;
  info->n_groups = (int32_t)h.groups.size();
  info->kept_pairs_per_head = h.kept_pairs_per_head;
  info->block_m = h.block_m;
  info->block_n = h.block_n;
  info->n_splits = h.n_splits;
  info->n_items = (int32_t)h.items.size();
  info->causal = h.geo.causal;
  info->launch_xcds = wa::kXcdCount;
  info->launch_per_xcd = h.work_per_xcd;
  info->workspace_bytes = h.partial_bytes;
  info->block_q = h.geo.block_q;
  info->block_kv = h.geo.block_kv;
  info->n_qblocks = h.n_qblocks;
  info->n_kvblocks = h.n_kvblocks;
  info->n_tiles = (int32_t)h.tiles.size();
  info->computed_pairs_per_head = h.computed_pairs_per_head;
  return WA_OK;
}

int wa_plan_block_mask(const wa_plan* plan, int32_t* kv_num_blocks, int32_t* kv_indices, int32_t* full_kv_num_blocks,
                       int32_t* full_kv_indices, size_t n) {
  if (!plan || !kv_num_blocks || !kv_indices || !full_kv_num_blocks || !full_kv_indices)
    return fail(WA_ERR_INVALID, "wa_plan_block_mask: NULL argument");
  const wa::HostPlan& h = plan->host;
  if (h.geo.block_q <= 0) return fail(WA_ERR_INVALID, "wa_plan_block_mask: not a block-sparse plan");
  const size_t nq = size_t(h.n_qblocks), nk = size_t(h.n_kvblocks);
  if (n < nq * nk) return fail(WA_ERR_INVALID, "wa_plan_block_mask: destination too small");
  std::memcpy(kv_num_blocks, h.kv_num.data(), nq * sizeof(int32_t));
  std::memcpy(full_kv_num_blocks, h.full_num.data(), nq * sizeof(int32_t));
  std::memcpy(kv_indices, h.kv_idx.data(), nq * nk * sizeof(int32_t));
  std::memcpy(full_kv_indices, h.full_idx.data(), nq * nk * sizeof(int32_t));
  return WA_OK;
}

int wa_plan_tiles(const wa_plan* plan, int32_t* dst, size_t n) {
  if (!plan || !dst) return fail(WA_ERR_INVALID, "wa_plan_tiles: NULL argument");
  const auto& tiles = plan->host.tiles;
  if (n < tiles.size()) return fail(WA_ERR_INVALID, "wa_plan_tiles: destination too small");
  if (!tiles.empty()) std::memcpy(dst, tiles.data(), tiles.size() * sizeof(int32_t));
  return WA_OK;
}

int wa_plan_groups(const wa_plan* plan, int32_t* dst, size_t n) {
  if (!plan || !dst) return fail(WA_ERR_INVALID, "wa_plan_groups: NULL argument");
  const auto& g = plan->host.groups;
  if (n < g.size() * 6) return fail(WA_ERR_INVALID, "wa_plan_groups: destination too small");
  for (size_t i = 0; i < g.size(); ++i) {
    dst[6 * i + 0] = g[i].q_begin;
    dst[6 * i + 1] = g[i].q_end;
    dst[6 * i + 2] = g[i].kv_begin;
    dst[6 * i + 3] = g[i].kv_end;
    dst[6 * i + 4] = g[i].chunk_lo;
    dst[6 * i + 5] = g[i].chunk_hi;
  }
  return WA_OK;
}

int wa_plan_kv_indices(const wa_plan* plan, int g, int32_t* dst, size_t n) {
  if (!plan || !dst) return fail(WA_ERR_INVALID, "wa_plan_kv_indices: NULL argument");
  const wa::HostPlan& h = plan->host;
  if (g < 0 || g >= (int)h.groups.size()) return fail(WA_ERR_INVALID, "wa_plan_kv_indices: bad group index");
  const wa::Group& gr = h.groups[g];
  const size_t need = size_t(gr.kv_end - gr.kv_begin) + size_t(h.geo.G);
  if (n < need) return fail(WA_ERR_INVALID, "wa_plan_kv_indices: destination too small");
  size_t o = 0;
  for (int32_t j = gr.kv_begin; j < gr.kv_end; ++j) dst[o++] = j;
  for (int32_t j = h.n_frame_rows; j < h.L; ++j) dst[o++] = j;
  return WA_OK;
}

int wa_plan_items(const wa_plan* plan, int32_t* dst, size_t n) {
  if (!plan || !dst) return fail(WA_ERR_INVALID, "wa_plan_items: NULL argument");
  const auto& items = plan->host.items;
  if (n < items.size() * WA_ITEM_COLS) return fail(WA_ERR_INVALID, "wa_plan_items: destination too small");
  std::memcpy(dst, items.data(), items.size() * sizeof(wa::Item));
  return WA_OK;
}

int wa_plan_launch_order(const wa_plan* plan, int32_t* dst, size_t n) {
  if (!plan || !dst) return fail(WA_ERR_INVALID, "wa_plan_launch_order: NULL argument");
  const auto& work = plan->host.work;
  if (n < work.size()) return fail(WA_ERR_INVALID, "wa_plan_launch_order: destination too small");
  std::memcpy(dst, work.data(), work.size() * sizeof(int32_t));
  return WA_OK;
}

// Argument checks shared by wa_forward and wa_forward_noalloc.
static int check_forward(const char* who, const wa_plan* plan, const void* q, const void* k, const void* v,
                         const void* out, int dtype) {
  if (!plan) return fail(WA_ERR_INVALID, std::string(who) + ": plan is NULL");
  if (!q || !k || !v || !out) return fail(WA_ERR_INVALID, std::string(who) + ": NULL tensor pointer");
  if (dtype != WA_BF16 && dtype != WA_F32)
    return fail(WA_ERR_INVALID, std::string(who) + ": dtype must be WA_BF16 or WA_F32");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(WA_ERR_INVALID, std::string(who) + ": tensors must be 16-byte aligned");
  const wa::HostPlan& h = plan->host;
  const size_t bytes = size_t(int64_t(h.L) * h.geo.H * h.geo.d) * (dtype == WA_F32 ? 4 : 2);
  if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
    return fail(WA_ERR_INVALID, std::string(who) + ": out overlaps an input");
  return WA_OK;
}

// Launch arguments of `h` with its device tables at `table` (the int32 image of
// wa_plan::table) and the global leg's partials at `part` (may be NULL without splits).
static wa::ForwardArgs forward_args(const wa::HostPlan& h, int32_t* table, float* part, int n_cus, void* out,
                                    int dtype) {
  wa::ForwardArgs a;
  a.q = a.k = a.v = nullptr;
  a.out = out;
  a.out_f32 = dtype == WA_F32;
  a.d = h.geo.d;
  a.H = h.geo.H;
  a.L = h.L;
  a.G = h.geo.G;
  a.frame_rows = h.n_frame_rows;
  a.block_m = h.block_m;
  a.items = reinterpret_cast<const wa::Item*>(table);
  a.n_items = (int)h.items.size();
  a.work = table + h.items.size() * (sizeof(wa::Item) / sizeof(int32_t));
  a.work_per_xcd = h.work_per_xcd;
  a.counters = const_cast<int32_t*>(a.work) + h.work.size();
  // Persistent blocks pay a few memory round trips per unit for the queues; they pay off only
  // when each CU runs several units.  Otherwise one block per unit.
  const int64_t units = int64_t(h.items.size()) * h.geo.H;
  a.persistent = units > 2 * int64_t(n_cus) ? 1 : 0;
  a.grid = a.persistent ? n_cus : wa::kXcdCount * h.work_per_xcd;
  a.n_splits = h.n_splits;
  a.part_o = part;
  a.part_ml = part ? part + int64_t(h.n_splits) * h.geo.G * h.geo.H * h.geo.d : nullptr;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(h.geo.d)));
  a.tile_list = h.geo.block_q > 0;
  a.tiles = a.counters + (wa::kXcdCount + 1);
  a.T = h.geo.T;
  a.S = h.geo.S;
  a.K = h.geo.K;
  a.radius = h.geo.radius;
  a.n_chunks = h.n_chunks;
  return a;
}

// Enqueue one call: for fp32 inputs their bf16 copies into `staging` (3 * elems * 2 bytes),
// then the attention and the merge.
static int enqueue_forward(const char* who, wa::ForwardArgs a, const void* q, const void* k, const void* v, int dtype,
                           char* staging, int64_t elems, hipStream_t stream) {
  a.q = q;
  a.k = k;
  a.v = v;
  if (dtype == WA_F32) {
    const void* src[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
      hipError_t e = wa::launch_f32_to_bf16(static_cast<const float*>(src[i]), staging + i * elems * 2, elems, stream);
      if (e != hipSuccess) return fail(WA_ERR_HIP, std::string(who) + ": f32_to_bf16 launch: " + hipGetErrorString(e));
    }
    a.q = staging;
    a.k = staging + elems * 2;
    a.v = staging + 2 * elems * 2;
  }
  hipError_t e = wa::launch_forward(a, stream);
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string(who) + ": launch: " + hipGetErrorString(e));
  return WA_OK;
}

int wa_forward(const wa_plan* cplan, const void* q, const void* k, const void* v, void* out, int dtype,
               void* stream_v) {
  int st = check_forward("wa_forward", cplan, q, k, v, out, dtype);
  if (st != WA_OK) return st;
  wa_plan* plan = const_cast<wa_plan*>(cplan);
  const wa::HostPlan& h = plan->host;
  const int64_t elems = int64_t(h.L) * h.geo.H * h.geo.d;
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  DeviceResources* r = nullptr;
  st = device_resources(plan, &r);
  if (st != WA_OK) return st;
  const wa::ForwardArgs a = forward_args(h, reinterpret_cast<int32_t*>(r->items), r->part, r->n_cus, out, dtype);

  return ordered_launch(plan, r, stream, "wa_forward", [&]() -> int {
    if (dtype == WA_F32) {
      const int64_t need = 3 * elems * 2;
      std::lock_guard<std::mutex> lk(plan->dev_mu);
      if (r->staging_bytes < need) {
        if (r->staging) (void)hipFree(r->staging);
        r->staging = nullptr;
        r->staging_bytes = 0;
        hipError_t e = hipMalloc(&r->staging, (size_t)need);
        if (e != hipSuccess) return fail(WA_ERR_ALLOC, std::string("hipMalloc(staging): ") + hipGetErrorString(e));
        r->staging_bytes = need;
      }
    }
    return enqueue_forward("wa_forward", a, q, k, v, dtype, static_cast<char*>(r->staging), elems, stream);
  });
}

int wa_forward_noalloc(const wa_plan* cplan, const void* q, const void* k, const void* v, void* out, int dtype,
                       void* stream_v) {
  int st = check_forward("wa_forward_noalloc", cplan, q, k, v, out, dtype);
  if (st != WA_OK) return st;
  const wa_plan* plan = cplan;
  const wa::HostPlan& h = plan->host;
  const int64_t elems = int64_t(h.L) * h.geo.H * h.geo.d;
  // workspace layout: table | partials | staging, each part at a 256-byte boundary
  auto up256 = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t table_bytes = plan->table.size() * sizeof(int32_t);
  const size_t part_off = up256(table_bytes);
  const size_t staging_off = part_off + up256(size_t(h.partial_bytes));
  const size_t need = staging_off + (dtype == WA_F32 ? size_t(3 * elems * 2) : 0);
  if (need > wa::kStaticWorkspaceBytes)
    return fail(WA_ERR_UNSUPPORTED, "wa_forward_noalloc: this plan needs " + std::to_string(need) +
                                        " bytes of workspace (tables, global-leg partials" +
                                        (dtype == WA_F32 ? ", bf16 staging" : "") + "), above the static " +
                                        std::to_string(wa::kStaticWorkspaceBytes) + " bytes");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string("wa_forward_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  void* ws = nullptr;
  e = wa::static_workspace(dev, &ws);
  if (e != hipSuccess)
    return fail(WA_ERR_HIP, std::string("wa_forward_noalloc: static workspace address: ") + hipGetErrorString(e));
  int n_cus = 0;
  e = hipDeviceGetAttribute(&n_cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || n_cus < 1) return fail(WA_ERR_HIP, "wa_forward_noalloc: hipDeviceGetAttribute failed");
  char* base = static_cast<char*>(ws);
  hipStream_t stream = static_cast<hipStream_t>(stream_v);
  // The plan's tables, zeroed queue counters included, go into the workspace ahead of the
  // kernels on the same stream (the workspace holds whatever the previous call left).
  e = hipMemcpyAsync(base, plan->table.data(), table_bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string("wa_forward_noalloc: table upload: ") + hipGetErrorString(e));
  float* part = h.partial_bytes > 0 ? reinterpret_cast<float*>(base + part_off) : nullptr;
  const wa::ForwardArgs a = forward_args(h, reinterpret_cast<int32_t*>(base), part, n_cus, out, dtype);
  return enqueue_forward("wa_forward_noalloc", a, q, k, v, dtype, base + staging_off, elems, stream);
}

int wa_forward_fp8(const wa_plan* cplan, const void* q, const void* k, const void* v, float scale_q, float scale_k,
                   float scale_v, void* out, void* stream_v) {
  if (!cplan) return fail(WA_ERR_INVALID, "wa_forward_fp8: plan is NULL");
  if (!q || !k || !v || !out) return fail(WA_ERR_INVALID, "wa_forward_fp8: NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(WA_ERR_INVALID, "wa_forward_fp8: tensors must be 16-byte aligned");
  const float sc[3] = {scale_q, scale_k, scale_v};
  for (float s : sc)
    if (!(s > 0.f) || s > 1e30f) return fail(WA_ERR_INVALID, "wa_forward_fp8: scales must be finite and > 0");
  wa_plan* plan = const_cast<wa_plan*>(cplan);
  const wa::HostPlan& h = plan->host;
  if (h.geo.d != 128) return fail(WA_ERR_UNSUPPORTED, "wa_forward_fp8: head size must be 128");
  if (h.geo.block_q > 0) return fail(WA_ERR_UNSUPPORTED, "wa_forward_fp8: block-sparse plans run through wa_forward");
  const int64_t elems = int64_t(h.L) * h.geo.H * h.geo.d;
  // out holds 2 bytes per element, the inputs 1
  auto hits = [&](const void* in) {
    const uintptr_t o = reinterpret_cast<uintptr_t>(out), i = reinterpret_cast<uintptr_t>(in);
    return o < i + size_t(elems) && i < o + size_t(elems) * 2;
  };
  if (hits(q) || hits(k) || hits(v)) return fail(WA_ERR_INVALID, "wa_forward_fp8: out overlaps an input");
  DeviceResources* r = nullptr;
  int st = device_resources(plan, &r);
  if (st != WA_OK) return st;
  wa::ForwardArgs a = forward_args(h, reinterpret_cast<int32_t*>(r->items), r->part, r->n_cus, out, WA_BF16);
  a.q = q;
  a.k = k;
  a.v = v;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(h.geo.d)) * double(scale_q) * double(scale_k));
  const hipStream_t stream = static_cast<hipStream_t>(stream_v);
  return ordered_launch(plan, r, stream, "wa_forward_fp8", [&]() -> int {
    hipError_t e = wa::launch_forward_fp8(a, scale_v, stream);
    if (e != hipSuccess) return fail(WA_ERR_HIP, std::string("wa_forward_fp8 launch: ") + hipGetErrorString(e));
    return WA_OK;
  });
}

int wa_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, const float* cos, const float* sin,
                    const float* wq, const float* wk, int L, int H, int d, float eps, int flags, int dtype,
                    void* stream_v) {
  if (dtype != WA_BF16 && dtype != WA_F32) return fail(WA_ERR_INVALID, "wa_qk_norm_rope: dtype must be WA_BF16 or WA_F32");
  if (flags & ~WA_ROPE_INTERLEAVED) return fail(WA_ERR_INVALID, "wa_qk_norm_rope: unknown flags");
  if (L < 0 || H < 1) return fail(WA_ERR_INVALID, "wa_qk_norm_rope: need L >= 0 and H >= 1");
  if (!(eps >= 0.f) || eps > 1e30f) return fail(WA_ERR_INVALID, "wa_qk_norm_rope: eps must be finite and >= 0");
  if (d != 64 && d != 128) return fail(WA_ERR_UNSUPPORTED, "wa_qk_norm_rope: d must be 64 or 128");
  if (int64_t(L) * H * d >= (int64_t(1) << 31))
    return fail(WA_ERR_UNSUPPORTED, "wa_qk_norm_rope: L*H*d must be below 2^31");
  if (L == 0) return WA_OK;  // nothing to touch: the pointers may be anything, NULL included
  if (!q || !k || !q_out || !k_out || !cos || !sin)
    return fail(WA_ERR_INVALID, "wa_qk_norm_rope: NULL tensor pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(cos) ||
      !aligned16(sin) || (wq && !aligned16(wq)) || (wk && !aligned16(wk)))
    return fail(WA_ERR_INVALID, "wa_qk_norm_rope: pointers must be 16-byte aligned");
  {
    const size_t bytes = size_t(L) * H * d * (dtype == WA_F32 ? 4 : 2);
    // each output may be its own input (in place) but must not touch any other tensor
    const void* ins[2] = {q, k};
    const void* outs[2] = {q_out, k_out};
    for (int o = 0; o < 2; ++o)
      for (int i = 0; i < 2; ++i)
        if (o != i && overlaps(outs[o], ins[i], bytes))
          return fail(WA_ERR_INVALID, "wa_qk_norm_rope: an output overlaps the other input");
    if (overlaps(q_out, k_out, bytes)) return fail(WA_ERR_INVALID, "wa_qk_norm_rope: q_out overlaps k_out");
    for (int o = 0; o < 2; ++o)
      if (outs[o] != ins[o] && overlaps(outs[o], ins[o], bytes))
        return fail(WA_ERR_INVALID, "wa_qk_norm_rope: an output partly overlaps its input");
  }
  wa::PrologueArgs a;
  a.q = q;
  a.k = k;
  a.q_out = q_out;
  a.k_out = k_out;
  a.cos = cos;
  a.sin = sin;
  a.wq = wq;
  a.wk = wk;
  a.L = L;
  a.H = H;
  a.d = d;
  a.eps = eps;
  a.f32 = dtype == WA_F32;
  a.interleaved = (flags & WA_ROPE_INTERLEAVED) != 0;
  hipError_t e = wa::launch_qk_norm_rope(a, static_cast<hipStream_t>(stream_v));
  if (e != hipSuccess) return fail(WA_ERR_HIP, std::string("wa_qk_norm_rope launch: ") + hipGetErrorString(e));
  return WA_OK;
}

const char* wa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

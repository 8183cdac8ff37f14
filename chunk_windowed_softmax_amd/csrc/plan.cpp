// Host-side plan builder: window groups, work items and global-leg splits.
#include "plan.h"

#include <algorithm>

namespace wa {

void build_launch_order(HostPlan* p);

namespace {

// Rows [begin, end) of the whole chunks lo..hi; the last chunk may be partial.
inline void span_rows(const Geometry& g, int lo, int hi, int32_t* begin, int32_t* end) {
  *begin = lo * g.K * g.S;
  *end = std::min(g.T, (hi + 1) * g.K) * g.S;
}

}  // namespace

int build_plan(const Geometry& g, HostPlan* out, std::string* err) {
  if (g.T < 1 || g.S < 1 || g.K < 1 || g.H < 1 || g.G < 0 || g.radius < 0) {
    *err = "invalid geometry: need T, S, K, H >= 1, G >= 0, radius >= 0";
    return 1;
  }
  if (g.d != 64 && g.d != 128) {
    *err = "unsupported head size d=" + std::to_string(g.d) + " (supported: 64, 128)";
    return 2;
  }
  const int64_t L64 = int64_t(g.T) * g.S + g.G;
  if (L64 * g.H * g.d >= (int64_t(1) << 31)) {
    *err = "unsupported size: L*H*d must be below 2^31 elements";
    return 2;
  }
  HostPlan p;
  p.geo = g;
  p.L = int32_t(L64);
  p.n_frame_rows = g.T * g.S;
  p.n_chunks = (g.T + g.K - 1) / g.K;
  p.block_m = kBlockM;
  p.block_n = kBlockN;

  // Window groups: maximal runs of consecutive chunks with an identical window.
  for (int c = 0; c < p.n_chunks;) {
    int lo, hi;
    chunk_window(c, p.n_chunks, g.radius, &lo, &hi);
    int c_end = c;
    for (;;) {
      if (c_end + 1 >= p.n_chunks) break;
      int lo2, hi2;
      chunk_window(c_end + 1, p.n_chunks, g.radius, &lo2, &hi2);
      if (lo2 != lo || hi2 != hi) break;
      ++c_end;
    }
    Group gr;
    span_rows(g, c, c_end, &gr.q_begin, &gr.q_end);
    span_rows(g, lo, hi, &gr.kv_begin, &gr.kv_end);
    gr.chunk_lo = lo;
    gr.chunk_hi = hi;
    p.groups.push_back(gr);
    c = c_end + 1;
  }

  // Kept pairs of one head: window rows see their span plus the globals; globals see all.
  int64_t kept = 0, max_window_kv = 0;
  for (const Group& gr : p.groups) {
    const int64_t kv = int64_t(gr.kv_end - gr.kv_begin) + g.G;
    kept += int64_t(gr.q_end - gr.q_begin) * kv;
    max_window_kv = std::max(max_window_kv, kv);
  }
  kept += int64_t(g.G) * p.L;
  p.kept_pairs_per_head = kept;

  // First leg: block_m-row tiles of each group, keys = span then the global rows.
  for (const Group& gr : p.groups) {
    for (int32_t q = gr.q_begin; q < gr.q_end; q += p.block_m) {
      Item it;
      it.q_begin = q;
      it.q_end = std::min(gr.q_end, q + p.block_m);
      it.kv0_begin = gr.kv_begin;
      it.kv0_end = gr.kv_end;
      it.kv1_begin = p.n_frame_rows;
      it.kv1_end = p.L;
      it.split = -1;
      it.flags = 0;
      p.items.push_back(it);
    }
  }
  p.n_window_items = int32_t(p.items.size());

  // Second leg: the G global rows over all L keys, split into whole key tiles (split length
  // as set out next to kGlobalSplitDiv).
  p.n_splits = 0;
  if (g.G > 0) {
    const bool fine = int64_t(p.n_window_items) * g.H >= int64_t(kFineSplitRounds) * kComputeUnits;
    const int64_t split_len = std::max<int64_t>(p.block_n, max_window_kv / (fine ? kGlobalSplitDiv : 1));
    int64_t n_splits = std::max<int64_t>(1, (p.L + split_len - 1) / split_len);
    int64_t chunk = (p.L + n_splits - 1) / n_splits;
    chunk = (chunk + p.block_n - 1) / p.block_n * p.block_n;
    n_splits = (p.L + chunk - 1) / chunk;
    p.n_splits = int32_t(n_splits);
    for (int s = 0; s < p.n_splits; ++s) {
      for (int32_t q = p.n_frame_rows; q < p.L; q += p.block_m) {
        Item it;
        it.q_begin = q;
        it.q_end = std::min(p.L, q + p.block_m);
        it.kv0_begin = int32_t(s * chunk);
        it.kv0_end = int32_t(std::min<int64_t>(p.L, (s + 1) * chunk));
        it.kv1_begin = it.kv1_end = 0;
        it.split = p.n_splits > 1 ? s : -1;
        it.flags = 0;
        p.items.push_back(it);
      }
    }
    if (p.n_splits > 1)
      p.partial_bytes = int64_t(p.n_splits) * g.G * g.H * (g.d + 2) * int64_t(sizeof(float));
  }

  build_launch_order(&p);
  *out = std::move(p);
  return 0;
}

int build_causal_plan(int n, int H, int d, HostPlan* out, std::string* err) {
  if (n < 1 || H < 1) {
    *err = "invalid causal geometry: need n, H >= 1";
    return 1;
  }
  if (d != 64 && d != 128) {
    *err = "unsupported head size d=" + std::to_string(d) + " (supported: 64, 128)";
    return 2;
  }
  if (int64_t(n) * H * d >= (int64_t(1) << 31)) {
    *err = "unsupported size: n*H*d must be below 2^31 elements";
    return 2;
  }
  HostPlan p;
  p.geo = Geometry{1, n, 0, 1, 0, H, d, 1};
  p.L = n;
  p.n_frame_rows = n;
  p.n_chunks = 1;
  p.block_m = kBlockM;
  p.block_n = kBlockN;
  p.kept_pairs_per_head = int64_t(n) * (n + 1) / 2;
  for (int32_t q = 0; q < n; q += p.block_m) {
    Item it;
    it.q_begin = q;
    it.q_end = std::min(n, q + p.block_m);
    it.kv0_begin = 0;
    it.kv0_end = it.q_end;
    it.kv1_begin = it.kv1_end = 0;
    it.split = -1;
    it.flags = kItemCausal;
    p.items.push_back(it);
  }
  p.n_window_items = int32_t(p.items.size());
  build_launch_order(&p);
  *out = std::move(p);
  return 0;
}

// Launch order (see HostPlan::work).
void build_launch_order(HostPlan* pp) {
  HostPlan& p = *pp;
  const Geometry& g = p.geo;
  const int32_t n_items = int32_t(p.items.size());
  std::vector<int32_t> win, glob;
  for (int32_t h = 0; h < g.H; ++h)
    for (int32_t i = 0; i < n_items; ++i) (i < p.n_window_items ? win : glob).push_back(h * n_items + i);
  const int32_t pw = int32_t((win.size() + kXcdCount - 1) / kXcdCount);
  const int32_t pg = int32_t((glob.size() + kXcdCount - 1) / kXcdCount);
  p.work_per_xcd = pw + pg;
  p.work.assign(size_t(kXcdCount) * p.work_per_xcd, -1);
  for (int x = 0; x < kXcdCount; ++x) {
    int32_t* dst = p.work.data() + size_t(x) * p.work_per_xcd;
    int32_t n = 0;  // units are packed at the front of the row; -1 padding only at its end
    for (int32_t j = 0; j < pw && size_t(x) * pw + j < win.size(); ++j) dst[n++] = win[size_t(x) * pw + j];
    for (int32_t j = 0; j < pg && size_t(x) * pg + j < glob.size(); ++j) dst[n++] = glob[size_t(x) * pg + j];
  }
}

}  // namespace wa

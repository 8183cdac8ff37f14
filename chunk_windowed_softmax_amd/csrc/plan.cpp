// Host-side plan builder: window groups, work items and global-leg splits.
#include "plan.h"

#include <algorithm>

namespace wa {

void build_launch_order(HostPlan* p);
void add_global_leg(HostPlan* p, int64_t max_item_keys, int64_t window_items, bool tile_list);

namespace {

// Rows [begin, end) of the whole chunks lo..hi; the last chunk may be partial.
inline void span_rows(const Geometry& g, int lo, int hi, int32_t* begin, int32_t* end) {
  *begin = lo * g.K * g.S;
  *end = std::min(g.T, (hi + 1) * g.K) * g.S;
}

}  // namespace

// Second leg: the G global rows over all L keys, split into whole key tiles (split length
// as set out next to kGlobalSplitDiv; max_item_keys is the longest window item's key count and
// window_items the number of window items per head).
// With tile_list, each item's keys are appended to p->tiles as 64-key tile entries (the
// last tile of a split that ends inside it flagged for masking) instead of one segment.
void add_global_leg(HostPlan* pp, int64_t max_item_keys, int64_t window_items, bool tile_list) {
  HostPlan& p = *pp;
  const Geometry& g = p.geo;
  p.n_splits = 0;
  if (g.G <= 0) return;
  const bool fine = window_items * g.H >= int64_t(kFineSplitRounds) * kComputeUnits;
  const int64_t split_len = std::max<int64_t>(p.block_n, max_item_keys / (fine ? kGlobalSplitDiv : 1));
  int64_t n_splits = std::max<int64_t>(1, (p.L + split_len - 1) / split_len);
  int64_t chunk = (p.L + n_splits - 1) / n_splits;
  chunk = (chunk + p.block_n - 1) / p.block_n * p.block_n;
  n_splits = (p.L + chunk - 1) / chunk;
  p.n_splits = int32_t(n_splits);
  for (int s = 0; s < p.n_splits; ++s) {
    const int32_t k0 = int32_t(s * chunk), k1 = int32_t(std::min<int64_t>(p.L, (s + 1) * chunk));
    for (int32_t q = p.n_frame_rows; q < p.L; q += p.block_m) {
      Item it;
      it.q_begin = q;
      it.q_end = std::min(p.L, q + p.block_m);
      it.kv1_begin = it.kv1_end = 0;
      it.split = p.n_splits > 1 ? s : -1;
      if (tile_list) {
        it.kv0_begin = int32_t(p.tiles.size());
        for (int32_t t0 = k0; t0 < k1; t0 += p.block_n)
          p.tiles.push_back((t0 << 1) | (t0 + p.block_n > k1 ? 1 : 0));
        it.kv0_end = int32_t(p.tiles.size()) - it.kv0_begin;
        it.flags = kItemTileList;
      } else {
        it.kv0_begin = k0;
        it.kv0_end = k1;
        it.flags = 0;
      }
      p.computed_pairs_per_head += int64_t(it.q_end - it.q_begin) * ((k1 - k0 + p.block_n - 1) / p.block_n) * p.block_n;
      p.items.push_back(it);
    }
  }
  if (p.n_splits > 1)
    p.partial_bytes = int64_t(p.n_splits) * g.G * g.H * (g.d + 2) * int64_t(sizeof(float));
}

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
      const int64_t tiles = (gr.kv_end - gr.kv_begin + p.block_n - 1) / p.block_n + (g.G + p.block_n - 1) / p.block_n;
      p.computed_pairs_per_head += int64_t(it.q_end - it.q_begin) * tiles * p.block_n;
      p.items.push_back(it);
    }
  }
  p.n_window_items = int32_t(p.items.size());

  add_global_leg(&p, max_window_kv, p.n_window_items, false);
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
    p.computed_pairs_per_head += int64_t(it.q_end - it.q_begin) * ((it.q_end + p.block_n - 1) / p.block_n) * p.block_n;
    p.items.push_back(it);
  }
  p.n_window_items = int32_t(p.items.size());
  build_launch_order(&p);
  *out = std::move(p);
  return 0;
}

int build_blocksparse_plan(const Geometry& g, HostPlan* out, std::string* err) {
  if ((g.block_q != 128 && g.block_q != 256) || (g.block_kv != 64 && g.block_kv != 128)) {
    *err = "unsupported block sizes (" + std::to_string(g.block_q) + ", " + std::to_string(g.block_kv) +
           "): block_q must be 128 or 256 and block_kv 64 or 128";
    return 2;
  }
  Geometry base = g;
  base.block_q = base.block_kv = 0;
  HostPlan ref;  // validation, row counts, kept pairs and the global-leg sizing of the decomposed plan
  const int st = build_plan(base, &ref, err);
  if (st != 0) return st;

  HostPlan p;
  p.geo = g;
  p.L = ref.L;
  p.n_frame_rows = ref.n_frame_rows;
  p.n_chunks = ref.n_chunks;
  p.block_m = kBlockM;
  p.block_n = kBlockN;
  p.kept_pairs_per_head = ref.kept_pairs_per_head;
  const int32_t TS = p.n_frame_rows, L = p.L, bq = g.block_q, bk = g.block_kv;
  p.n_qblocks = (TS + bq - 1) / bq;
  p.n_kvblocks = (L + bk - 1) / bk;
  const size_t nq = size_t(p.n_qblocks), nk = size_t(p.n_kvblocks);
  p.kv_num.assign(nq, 0);
  p.full_num.assign(nq, 0);
  p.kv_idx.assign(nq * nk, -1);
  p.full_idx.assign(nq * nk, -1);

  // Block status: count the kept pairs of query block i and key block j frame by frame (the
  // rows of one frame share a window); full when every pair of a whole key block is kept.
  std::vector<int64_t> kept(nk);
  for (size_t i = 0; i < nq; ++i) {
    const int32_t r0 = int32_t(i) * bq, r1 = std::min(TS, r0 + bq);
    std::fill(kept.begin(), kept.end(), 0);
    for (int32_t r = r0; r < r1;) {
      const int t = r / g.S;
      const int32_t r_end = std::min(r1, (t + 1) * g.S);  // rows of frame t in the block
      int lo, hi;
      chunk_window(t / g.K, p.n_chunks, g.radius, &lo, &hi);
      int32_t a, b;
      span_rows(g, lo, hi, &a, &b);
      for (size_t j = 0; j < nk; ++j) {
        const int32_t k0 = int32_t(j) * bk, k1 = std::min(L, k0 + bk);
        const int64_t in_span = std::max(0, std::min(b, k1) - std::max(a, k0));
        const int64_t in_glob = std::max(0, std::min(L, k1) - std::max(TS, k0));
        kept[j] += int64_t(r_end - r) * (in_span + in_glob);
      }
      r = r_end;
    }
    for (size_t j = 0; j < nk; ++j) {
      if (kept[j] == 0) continue;
      const int32_t k0 = int32_t(j) * bk, k1 = std::min(L, k0 + bk);
      const bool full = k1 - k0 == bk && kept[j] == int64_t(r1 - r0) * bk;
      if (full) p.full_idx[i * nk + size_t(p.full_num[i]++)] = int32_t(j);
      else p.kv_idx[i * nk + size_t(p.kv_num[i]++)] = int32_t(j);
    }
  }

  // Frame items: 256 query rows = one query block of 256 or two of 128.  Keys: the union of
  // the blocks' key blocks, ascending, as 64-key tiles; a block's tiles are masked element by
  // element unless the block is full for every query block of the item.
  const int qpi = kBlockM / bq;  // query blocks per item
  std::vector<int> state(nk);    // per key block: bit 0 present, bit 1 needs mask
  for (size_t i0 = 0; i0 < nq; i0 += size_t(qpi)) {
    std::fill(state.begin(), state.end(), 0);
    const size_t i1 = std::min(nq, i0 + size_t(qpi));
    for (size_t i = i0; i < i1; ++i) {
      std::vector<int> here(nk, 0);  // 1 partial, 2 full
      for (int32_t e = 0; e < p.kv_num[i]; ++e) here[size_t(p.kv_idx[i * nk + size_t(e)])] = 1;
      for (int32_t e = 0; e < p.full_num[i]; ++e) here[size_t(p.full_idx[i * nk + size_t(e)])] = 2;
      for (size_t j = 0; j < nk; ++j) {
        if (here[j]) state[j] |= 1;
        if (here[j] != 2) state[j] |= 2;  // partial here, or absent here but kept in a sibling block
      }
    }
    Item it;
    it.q_begin = int32_t(i0) * bq;
    it.q_end = std::min(TS, int32_t(i1) * bq);
    it.kv0_begin = int32_t(p.tiles.size());
    for (size_t j = 0; j < nk; ++j) {
      if (!(state[j] & 1)) continue;
      const int32_t k0 = int32_t(j) * bk, k1 = std::min(L, k0 + bk);
      for (int32_t t0 = k0; t0 < k1; t0 += kBlockN)
        p.tiles.push_back((t0 << 1) | ((state[j] & 2) || t0 + kBlockN > k1 ? 1 : 0));
    }
    it.kv0_end = int32_t(p.tiles.size()) - it.kv0_begin;
    if (it.kv0_end > kMaxListTiles) {
      *err = "unsupported: a block-sparse work item would list " + std::to_string(it.kv0_end) +
             " key tiles (at most " + std::to_string(kMaxListTiles) + ")";
      return 2;
    }
    it.kv1_begin = it.kv1_end = 0;
    it.split = -1;
    it.flags = kItemTileList;
    p.computed_pairs_per_head += int64_t(it.q_end - it.q_begin) * it.kv0_end * kBlockN;
    p.items.push_back(it);
  }
  p.n_window_items = int32_t(p.items.size());
  // the global leg split exactly as in the decomposed plan (sized by its longest window
  // item), so that the two plans differ in the window leg only
  int64_t max_window_kv = 0;
  for (const Group& gr : ref.groups) max_window_kv = std::max<int64_t>(max_window_kv, gr.kv_end - gr.kv_begin + g.G);
  add_global_leg(&p, max_window_kv, ref.n_window_items, true);
  for (const Item& it : p.items)
    if (it.kv0_end > kMaxListTiles) {
      *err = "unsupported: a block-sparse global-leg item would list " + std::to_string(it.kv0_end) + " key tiles";
      return 2;
    }
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

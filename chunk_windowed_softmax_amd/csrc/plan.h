// Host-side plan of the decomposed chunk-windowed attention (no HIP dependency).
//
// The decomposition follows the lqnn.cn article on VDN-Minimax-H3 window attention:
// §一 gives the window rule (chunks of K latent frames, whole chunks within +-radius of
// the frame's chunk, global tokens fully connected); §三 groups query rows with identical
// kept-KV sets into plain dense attentions, runs the window groups and the global rows as
// two legs with disjoint row sets, and caches the plan by geometry.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace wa {

struct Geometry {
  int T, S, G, K, radius, H, d;
  int causal = 0;  // 1: causal dense attention over S rows (T = 1, G = 0); see build_causal_plan
  // > 0: block-sparse plan with query blocks of block_q rows and key blocks of block_kv
  // keys (see build_blocksparse_plan)
  int block_q = 0, block_kv = 0;
  bool operator==(const Geometry& o) const {
    return T == o.T && S == o.S && G == o.G && K == o.K && radius == o.radius && H == o.H && d == o.d &&
           causal == o.causal && block_q == o.block_q && block_kv == o.block_kv;
  }
};

struct Group {  // a maximal run of chunks sharing one window
  int32_t q_begin, q_end, kv_begin, kv_end, chunk_lo, chunk_hi;
};

struct Item {  // one block_m-row query tile over up to two key segments (all heads alike)
  int32_t q_begin, q_end;
  int32_t kv0_begin, kv0_end;
  int32_t kv1_begin, kv1_end;
  int32_t split;     // -1: final rows; s >= 0: partial result of key split s (global leg)
  int32_t flags;     // kItemCausal: query row r sees keys <= r only
};
constexpr int32_t kItemCausal = 1;
// The item's keys are a list of 64-key tiles (block-sparse plans): kv0_begin is the offset
// of its first entry in HostPlan::tiles, kv0_end the number of entries.
constexpr int32_t kItemTileList = 2;
static_assert(sizeof(Item) == 32, "Item is uploaded as 8 int32");

struct HostPlan {
  Geometry geo{};
  int32_t L = 0, n_frame_rows = 0, n_chunks = 0;
  int64_t kept_pairs_per_head = 0;
  int32_t block_m = 0, block_n = 0, n_splits = 0;
  int32_t n_window_items = 0;
  std::vector<Group> groups;
  std::vector<Item> items;  // window items (group-major), then global-leg items (split-major)
  int64_t partial_bytes = 0;  // device workspace of the global leg's partial results
  // Launch order: one work queue per XCD; row x holds units work[x * work_per_xcd + i], unit =
  // head * items.size() + item, packed at the front, then -1 padding.  Each XCD's queue is a
  // contiguous run of window units (same group's query tiles side by side, sharing its L2)
  // and then a run of the shorter global-leg units, so the last units to start are the short
  // ones; blocks that empty their own queue take units from the other XCDs' queues.
  std::vector<int32_t> work;
  int32_t work_per_xcd = 0;
  // Block-sparse plans only.  The block mask of the frame (window) rows in the layout of
  // FlexAttention's BlockMask: for query block i (rows [i*block_q, min(T*S, (i+1)*block_q)))
  // the key blocks with some but not all pairs kept (kv_num[i] entries of kv_idx row i) and
  // those with every pair kept (full_num[i] entries of full_idx row i), ascending; rows are
  // n_kvblocks long, unused entries -1.  Key block j covers keys [j*block_kv, (j+1)*block_kv)
  // cut at L.
  int32_t n_qblocks = 0, n_kvblocks = 0;
  std::vector<int32_t> kv_num, kv_idx, full_num, full_idx;
  // Tile lists of the items (kItemTileList): entry = (first key row << 1) | needs_mask.
  std::vector<int32_t> tiles;
  int64_t computed_pairs_per_head = 0;  // (query, key) pairs the work items compute, one head
};

constexpr int kBlockM = 256;  // query rows per work item: 4 waves x 64 rows
constexpr int kBlockN = 64;   // keys per staged K/V tile
constexpr int kXcdCount = 8;  // MI355X: workgroups are dispatched round-robin over 8 XCDs
// When the window leg alone fills the chip for several rounds, a global-leg key split is
// about 1/kGlobalSplitDiv of the longest window item: the short units finish each XCD's
// queue and even out the tail of the launch.  Otherwise one split is about as long as the
// longest window item (fewer partial results to merge).
constexpr int kGlobalSplitDiv = 2;
constexpr int kComputeUnits = 256;   // MI355X
// Longest tile list of one item: the kernel keeps it in the 32 KB output staging area of the
// LDS (four 8 KB wave areas) past a 64-byte slot.
constexpr int kMaxListTiles = (4 * 8192 - 64) / 4;
constexpr int kFineSplitRounds = 4;  // window units >= this many rounds of all compute units

// Status codes mirror the C ABI (0 ok, 1 invalid, 2 unsupported).
int build_plan(const Geometry& g, HostPlan* out, std::string* err);

// Causal dense attention over n rows (the audio VAE's attention): no groups, one leg of
// block_m-row items, item rows [q0, q1) over keys [0, q1) with kItemCausal set.
int build_causal_plan(int n, int H, int d, HostPlan* out, std::string* err);

// Block-sparse (FlexAttention-style) plan of the same attention: the frame rows' block
// mask at (block_q, block_kv) granularity and work items that run 256 query rows (one
// query block of 256, or two of 128 over the union of their key blocks) over their key
// blocks as 64-key tiles, masking the tiles of partially kept blocks element by element;
// the global rows run the same split-KV leg as build_plan's, as tile lists.
// block_q in {128, 256}, block_kv in {64, 128}.
int build_blocksparse_plan(const Geometry& g, HostPlan* out, std::string* err);

// Chunk window [lo, hi] of chunk c (clipped to existing chunks).
inline void chunk_window(int c, int n_chunks, int radius, int* lo, int* hi) {
  *lo = c - radius < 0 ? 0 : c - radius;
  *hi = c + radius > n_chunks - 1 ? n_chunks - 1 : c + radius;
}

}  // namespace wa

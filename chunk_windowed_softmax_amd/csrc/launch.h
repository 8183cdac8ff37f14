// Internal interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace wa {

struct ForwardArgs {
  const void* q;          // bf16 [L, H, d]
  const void* k;          // bf16 [L, H, d]
  const void* v;          // bf16 [L, H, d]
  void* out;              // [L, H, d], bf16 or fp32 (out_f32)
  bool out_f32;
  int d, H, L, G, frame_rows;
  int block_m;            // query rows per work item: 256 (4 waves x 64 rows)
  const Item* items;      // device copy of the plan's items
  int n_items;
  const int32_t* work;    // device copy of the launch order (kXcdCount * work_per_xcd units)
  int work_per_xcd;
  int32_t* counters;      // kXcdCount + 1 device counters, zero between launches
  int persistent;         // 1: `grid` blocks (one per compute unit) run the queues
  int grid;               // blocks to launch
  int n_splits;           // > 1: global-leg items write partials, then a combine pass
  float* part_o;          // [n_splits, G, H, d] fp32
  float* part_ml;         // [n_splits, G, H, 2] fp32: running max (log2 units), row sum
  float scale_log2;       // log2(e) / sqrt(d)
  // Block-sparse plans: every item is a list of 64-key tiles (kItemTileList) in `tiles`,
  // entry = (first key row << 1) | needs_mask; masked tiles apply the window rule of the
  // geometry below element by element.
  bool tile_list;
  const int32_t* tiles;
  int T, S, K, radius, n_chunks;
};

// Enqueue the attention pass (both legs) and, when the global leg is split, the combine
// pass on `stream`.
hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream);

// Size of the static device workspace that wa_forward_noalloc uses (one per GPU).
constexpr size_t kStaticWorkspaceBytes = size_t(128) << 20;

// Device address of the static workspace on `device`, which must be the current device;
// looked up once per device, then cached.
hipError_t static_workspace(int device, void** ptr);

// Enqueue an fp32 -> bf16 (round to nearest even) conversion of n elements (n % 4 == 0).
hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t stream);

struct PrologueArgs {
  const void* q;          // [L, H, d] bf16 or fp32 (f32)
  const void* k;
  void* q_out;            // same shape and type; may be q itself
  void* k_out;
  const float* cos;       // [L, d/2] fp32
  const float* sin;
  const float* wq;        // [d] fp32 or nullptr (affine-free)
  const float* wk;
  int L, H, d;
  float eps;
  bool f32, interleaved;
};

// Enqueue the QK-RMSNorm + rotary-embedding pass (q and k in one launch).
hipError_t launch_qk_norm_rope(const PrologueArgs& a, hipStream_t stream);

// Enqueue the FP8 attention pass and, when the global leg is split, its merge.  `a` is set
// up as for launch_forward (bf16 output, no tile lists, d = 128) with q, k, v pointing at
// e4m3 codes and scale_log2 = log2(e) / sqrt(d) * scale_q * scale_k; the output is
// multiplied by scale_v.
hipError_t launch_forward_fp8(const ForwardArgs& a, float scale_v, hipStream_t stream);

}  // namespace wa

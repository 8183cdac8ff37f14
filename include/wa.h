/*
 * wa.h -- C ABI of the chunk-windowed softmax attention library (gfx950 / MI355X).
 *
 * What it computes.  The softmax window branch of VDN-H3's HybridAttention, as
 * described in the lqnn.cn article on VDN-Minimax-H3 window attention:
 *   - §一: the input is one packed sequence of T latent frames x S spatial tokens,
 *     followed by G global (text / audio) tokens.  Every K latent frames form a chunk;
 *     frame t (chunk c = t / K) attends to all tokens of the whole chunks whose index
 *     lies in [c - radius, c + radius] (clipped to the chunks that exist) and to every
 *     global token; global tokens attend to the whole sequence.
 *   - §三: the "decomposed" form.  Query rows with an identical kept-KV set form one
 *     group and each group is one plain mask-free dense attention; the window groups
 *     and the global rows are two legs whose row sets are disjoint and together cover
 *     the sequence, and their results are scattered into one contiguous output.  The
 *     plan (groups, index construction) is cached by geometry, at most four plans.
 * Softmax scale is 1/sqrt(d) (inputs are not pre-scaled).  Attention is non-causal.
 *
 * Layout.  q, k, v and out are dense row-major [L, H, d] tensors, L = T*S + G, rows in
 * the packed order (frame-major frame rows t*S + s, then the G global rows), row
 * stride H*d elements -- the [B, L, H, d] layout of the H3 attention modules in sglang
 * PR #34949 with B = 1.  A caller with a batch calls once per sequence.
 *
 * Status codes.  Every function returns WA_OK (0) or one of the WA_ERR_* codes; no
 * exception or abort crosses this boundary.  After a non-zero status, wa_last_error()
 * returns a message for the calling thread.  Device faults inside a kernel surface at
 * the caller's next synchronisation, not as a status of wa_forward.
 */
#ifndef WA_H_
#define WA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  WA_OK = 0,
  WA_ERR_INVALID = 1,     /* invalid argument (geometry, pointer, alignment, size) */
  WA_ERR_UNSUPPORTED = 2, /* valid but not supported (head size, dtype, index range) */
  WA_ERR_ALLOC = 3,       /* host or device allocation failed */
  WA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
};

/* Element types of q, k, v and out (all four share one type). */
enum {
  WA_BF16 = 0, /* bfloat16: computed with bf16 MFMA products, fp32 softmax/accumulators */
  WA_F32 = 1   /* float32 in and out: rounded to bf16 (nearest-even) for the products */
};

/* Opaque, reference-counted plan for one geometry. */
typedef struct wa_plan wa_plan;

/* Summary of a plan (filled by wa_plan_info). */
typedef struct wa_plan_info_t {
  int32_t T, S, G, K, radius, H, d; /* the geometry the plan was built for */
  int32_t L;                        /* T*S + G rows */
  int32_t n_chunks;                 /* ceil(T / K) */
  int32_t n_groups;                 /* window groups (first leg) */
  int64_t kept_pairs_per_head;      /* kept (query, key) pairs of one head */
  int32_t block_m;                  /* query rows per work item */
  int32_t block_n;                  /* keys per staged K/V tile */
  int32_t n_splits;                 /* key splits of the global leg (1 = no split) */
  int32_t n_items;                  /* work items per head (both legs) */
  int64_t workspace_bytes;          /* device workspace of the global leg's partials */
  int32_t launch_xcds;              /* launch order: number of XCD queues ... */
  int32_t launch_per_xcd;           /* ... and entries per queue (see wa_plan_launch_order) */
  int32_t causal;                   /* 1 for a wa_causal_plan_create plan */
  int32_t block_q, block_kv;        /* block sizes of a block-sparse plan (0 otherwise) */
  int32_t n_qblocks, n_kvblocks;    /* its block mask: query blocks x key blocks */
  int32_t n_tiles;                  /* entries of wa_plan_tiles (0 without tile lists) */
  int64_t computed_pairs_per_head;  /* (query, key) pairs the work items compute, one head:
                                       rows x 64-key tiles, so at least kept_pairs_per_head */
} wa_plan_info_t;

/* Item flag bits (column WA_ITEM_FLAGS). */
#define WA_ITEM_CAUSAL 1
#define WA_ITEM_TILE_LIST 2 /* keys: a list of 64-key tiles (block-sparse plans, see below) */

/* Columns of one row of wa_plan_items(). */
enum {
  WA_ITEM_Q_BEGIN = 0, /* first query row of the item */
  WA_ITEM_Q_END,       /* one past the last query row (at most block_m rows) */
  WA_ITEM_KV0_BEGIN,   /* first key segment [begin, end); with WA_ITEM_TILE_LIST: first entry
                          of the item's tiles in wa_plan_tiles, then the number of entries */
  WA_ITEM_KV0_END,
  WA_ITEM_KV1_BEGIN,   /* second key segment [begin, end); empty when begin == end */
  WA_ITEM_KV1_END,
  WA_ITEM_SPLIT,       /* -1: writes normalised output rows; s >= 0: split s of the global leg */
  WA_ITEM_FLAGS,       /* bit 0 (WA_ITEM_CAUSAL): query row r sees keys <= r only */
  WA_ITEM_COLS
};

/*
 * wa_plan_create -- build (or fetch from the cache) the plan of one geometry.
 *
 * The plan holds the window groups of §三 (maximal runs of consecutive chunks whose
 * windows are identical), each group's kept-KV list (its chunk span followed by the
 * global rows), the global leg (rows [T*S, L) over keys [0, L), split into n_splits
 * key ranges), and the work items the kernels run.  Plans are cached by the seven
 * arguments; at most four are cached, least recently created-or-fetched evicted first.
 *
 * Arguments: T, S, K, H >= 1; G >= 0; radius >= 0; d in {64, 128}; L*H*d < 2^31.
 * On success *out receives a handle that the caller owns one reference of; release it
 * with wa_plan_release.  Building a plan touches no device: device tables and the
 * workspace are created on the first wa_forward on each device.  With the environment
 * variable WA_LOG=1, building a plan (a cache miss) prints a one-line summary of it
 * (groups, items, splits, launch queues, kept pairs, workspace bytes, build time) to stderr.
 * Errors: WA_ERR_INVALID (bad geometry or out == NULL), WA_ERR_UNSUPPORTED (d, index
 * range), WA_ERR_ALLOC.
 */
int wa_plan_create(int T, int S, int G, int K, int radius, int H, int d, wa_plan** out);

/*
 * wa_causal_plan_create -- plan for causal dense attention over n rows: query row i of
 * every head attends to key rows 0..i, scale 1/sqrt(d).  This is the audio VAE's
 * attention in the prhub digest of sglang PR #34949 ("H3 VAE attention via the native USP
 * backend", item 3 and its CausalAttention listing): causal SDPA over q, k, v laid out as
 * (B, N, heads, head_dim), run once per batch element here (B = 1, so [n, H, d]); with
 * WA_F32 tensors wa_forward keeps that module's FP32 contract (fp32 in and out, the
 * attention itself in bf16 with fp32 accumulation, as for its fused backends).
 * Same cache, handle and error rules as wa_plan_create (n, H >= 1; d in {64, 128};
 * n*H*d < 2^31).  wa_forward with this plan takes [n, H, d] tensors; the plan has no
 * window groups (wa_plan_info reports n_groups = 0, causal = 1).
 */
int wa_causal_plan_create(int n, int H, int d, wa_plan** out);

/*
 * wa_blocksparse_plan_create -- plan of the same window attention computed the
 * block-sparse way, as the FlexAttention path of the lqnn.cn article on VDN-Minimax-H3 window
 * attention does (§二: a block-level mask built from the window rule, computed at block
 * granularity, so window edges are rounded up to whole blocks; §四 compares that path with
 * the decomposed one).  The frame rows' block mask at (block_q, block_kv) granularity lists,
 * for every query block, the key blocks with some kept pair; blocks kept in part are
 * computed with the window rule applied element by element, blocks kept in full without
 * it.  Work items are 256 query rows (one query block of 256, or two of 128 over the union of
 * their key blocks) over their key blocks as 64-key tiles, read through an index list.  The
 * global rows run the same split-KV leg as the wa_plan_create plan, so the two plans differ
 * in the window leg only.  wa_forward with this plan returns the same attention (to rounding).
 * block_q in {128, 256}, block_kv in {64, 128}; other arguments, cache and errors as
 * wa_plan_create (the block sizes are part of the cache key).  wa_forward_fp8 rejects it.
 */
int wa_blocksparse_plan_create(int T, int S, int G, int K, int radius, int H, int d, int block_q,
                               int block_kv, wa_plan** out);

/*
 * wa_plan_block_mask -- copy a block-sparse plan's block mask of the frame rows to host
 * memory, in the layout of FlexAttention's BlockMask: query block i covers rows
 * [i*block_q, min(T*S, (i+1)*block_q)), key block j keys [j*block_kv, min(L, (j+1)*block_kv)).
 * kv_num_blocks[i] / kv_indices row i: the key blocks with some but not every pair kept;
 * full_kv_num_blocks[i] / full_kv_indices row i: those with every pair kept (only whole
 * blocks).  Indices ascending; each index row has n_kvblocks entries, unused ones -1.
 * kv_num_blocks and full_kv_num_blocks hold n_qblocks entries; `n` is the capacity of each
 * index array (at least n_qblocks * n_kvblocks).  WA_ERR_INVALID for other plans or a small n.
 */
int wa_plan_block_mask(const wa_plan* plan, int32_t* kv_num_blocks, int32_t* kv_indices,
                       int32_t* full_kv_num_blocks, int32_t* full_kv_indices, size_t n);

/*
 * wa_plan_tiles -- copy the tile lists of a block-sparse plan's items to host memory (n_tiles
 * int32; an item with WA_ITEM_TILE_LIST owns entries [KV0_BEGIN, KV0_BEGIN + KV0_END)): entry
 * = (first key row << 1) | m, m = 1 when the tile's keys are masked element by element.
 * WA_ERR_INVALID if n is too small.
 */
int wa_plan_tiles(const wa_plan* plan, int32_t* dst, size_t n);

/*
 * wa_plan_release -- drop one reference.  The plan (and its device memory) is freed
 * once no handle refers to it and the cache no longer holds it.  Releasing a handle more
 * often than it was obtained is undefined.  WA_ERR_INVALID for NULL.
 */
int wa_plan_release(wa_plan* plan);

/*
 * wa_forward -- run the decomposed window attention of §三 for one packed sequence.
 *
 * q, k, v: device pointers to [L, H, d] tensors of element type `dtype` (WA_BF16 or
 * WA_F32), 16-byte aligned, caller-owned, read only.  out: device pointer to an [L, H, d]
 * tensor of the same type, 16-byte aligned, caller-owned, written in full (every row and
 * head exactly once); it must not overlap q, k or v.  stream: a hipStream_t (NULL = the
 * default stream); all work is enqueued on it and the call returns without
 * synchronising.  The first call on a device allocates the plan's device tables and
 * workspace (and, for WA_F32, a bf16 staging copy of q, k, v); later calls allocate
 * nothing.  Equal geometries share one cached plan, and with it one set of device tables,
 * work-queue counters and workspace: the library orders calls that use one plan, so a
 * call on a stream other than that of the plan's previous call (from any handle, through
 * wa_forward or wa_forward_fp8) first makes its stream wait for that call to finish.
 * Calls that use one plan on different streams therefore do not overlap on the device.
 * Every element of q, k and v must be finite: key tiles are
 * read whole, so rows next to a row's kept keys are read and masked to zero weight, and a
 * NaN or infinity there would still reach the output (finite values never do).
 * Errors: WA_ERR_INVALID (NULL / misaligned / overlapping pointers, bad dtype),
 * WA_ERR_ALLOC, WA_ERR_HIP (launch failure).
 */
int wa_forward(const wa_plan* plan, const void* q, const void* k, const void* v, void* out,
               int dtype, void* stream);

/* Bytes of the static device workspace of wa_forward_noalloc (one per GPU). */
#define WA_STATIC_WORKSPACE_BYTES (128u << 20)

/*
 * wa_forward_noalloc -- wa_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, result and errors as wa_forward, computed by the same kernels; but no
 * call allocates anything, on the host or the device.  Instead of the plan's own device
 * tables and workspace, every call uses one static workspace per GPU of
 * WA_STATIC_WORKSPACE_BYTES (a device array that each GPU the library runs on holds until
 * the process ends): the call enqueues, on `stream`, a copy of the plan's tables (work
 * items, launch order, zeroed work-queue counters) from host memory that the plan owns
 * into that workspace, then the kernels, which keep the global leg's partial results (and,
 * for WA_F32, the bf16 copies of q, k, v) there too.  A plan whose tables, partials and
 * staging need more than WA_STATIC_WORKSPACE_BYTES is rejected with WA_ERR_UNSUPPORTED
 * (e.g. 56 heads of the H3-scale geometry; its 7-head share fits).
 * Every call on one GPU shares that GPU's workspace, which keeps the last call's contents:
 * calls that overlap on one GPU (on different streams, or from different threads without
 * ordering) race and give wrong results; order them.  When the call is captured into a
 * graph, the plan must outlive the graph (its tables are read at each launch).
 */
int wa_forward_noalloc(const wa_plan* plan, const void* q, const void* k, const void* v, void* out,
                       int dtype, void* stream);

/* wa_plan_info -- fill *info.  WA_ERR_INVALID for NULL arguments. */
int wa_plan_info(const wa_plan* plan, wa_plan_info_t* info);

/*
 * wa_plan_groups -- copy the window groups of the decomposed form (§三: query rows whose
 * kept-KV sets are identical form one group, one dense attention each; for frame rows that
 * is a maximal run of consecutive chunks sharing one window of §一) to host memory:
 * n_groups rows of six int32
 * {q_begin, q_end, kv_begin, kv_end, chunk_lo, chunk_hi}; rows [q_begin, q_end) attend
 * to keys [kv_begin, kv_end) (the span of chunks chunk_lo..chunk_hi) plus the global
 * rows.  `n` is the capacity of dst in int32 elements; WA_ERR_INVALID if it is too small.
 */
int wa_plan_groups(const wa_plan* plan, int32_t* dst, size_t n);

/*
 * wa_plan_kv_indices -- copy group g's explicit ascending kept-KV index list (chunk
 * span, then the global rows) to host memory: (kv_end - kv_begin + G) int32.  These are
 * the gather indices of the decomposed form (§三: each group's kept keys, its window's
 * chunk span of §一 plus the global rows, which §五 notes the reference gathers per group);
 * the kernels never materialise them (they read the span and the global rows in place).  WA_ERR_INVALID for a bad g or small n.
 */
int wa_plan_kv_indices(const wa_plan* plan, int g, int32_t* dst, size_t n);

/*
 * wa_plan_items -- copy the per-head work items to host memory: n_items rows of
 * WA_ITEM_COLS int32 (columns named by WA_ITEM_*).  Every head runs the same items.
 * WA_ERR_INVALID if n is too small.
 */
int wa_plan_items(const wa_plan* plan, int32_t* dst, size_t n);

/*
 * wa_plan_launch_order -- copy the launch order to host memory: launch_xcds * launch_per_xcd
 * int32 entries; entry j of queue x is the work unit that block (x + launch_xcds * j) runs,
 * unit = head * n_items + item, or -1 for a block with no work.  Each unit appears exactly
 * once.  (The attention launch takes blocks round-robin over the XCDs; each queue holds a
 * contiguous run of window units and then the shorter global-leg units.)
 * WA_ERR_INVALID if n is too small.
 */
int wa_plan_launch_order(const wa_plan* plan, int32_t* dst, size_t n);

/*
 * wa_forward_fp8 -- the decomposed window attention of `plan` (any plan of wa_plan_create
 * or wa_causal_plan_create with d = 128) on FP8 inputs.  (The lqnn.cn article on
 * VDN-Minimax-H3 window attention quotes its fastest H3 configurations in FP8, §四; which
 * operands of the attention run in FP8 is not stated there: here both matrix products do.)
 * q, k, v: device pointers to [L, H, 128] OCP e4m3 (e4m3fn) codes, one byte each, 16-byte
 * aligned, caller-owned; the value of a code is its e4m3 value times scale_q, scale_k or
 * scale_v (finite, > 0).  out: device pointer to [L, H, 128] bf16, 16-byte aligned,
 * overlapping no input.
 * Computes out = softmax(scale_q scale_k q k^T / sqrt(d)) (scale_v v) over each row's kept
 * keys, like wa_forward: scores and the softmax in fp32, the softmax weights rounded to e4m3
 * for the second product (the one approximation beyond the inputs), each row divided by the
 * sum of exactly those rounded weights (so the weights applied to v sum to one), output
 * rounded to bf16.
 * stream: a hipStream_t (NULL = default).  Enqueues the kernels and returns without
 * synchronising; shares the plan's workspace with wa_forward and is ordered with the
 * plan's other calls in the same way (see wa_forward).
 * Errors: WA_ERR_INVALID (NULL plan or tensor, misalignment, overlap, bad scale),
 * WA_ERR_UNSUPPORTED (d != 128, or a plan of wa_blocksparse_plan_create), WA_ERR_ALLOC,
 * WA_ERR_HIP.
 */
int wa_forward_fp8(const wa_plan* plan, const void* q, const void* k, const void* v, float scale_q,
                   float scale_k, float scale_v, void* out, void* stream);

/* Flags of wa_qk_norm_rope. */
#define WA_ROPE_INTERLEAVED 1 /* rotate channel pairs (2j, 2j+1) instead of (j, j + d/2) */

/*
 * wa_qk_norm_rope -- the step before the attention, fused and out of place: RMSNorm of q
 * and k followed by the rotary position embedding, written as the attention's input.
 * (The ViT attention of the prhub digest of sglang PR #34949 applies qk_norm and the
 * rotary embedding to q and k before attending, with an affine-free RMSNorm among the
 * forms its contract tests cover; sglang PR #43164, Modifications item 2, fuses the norm
 * and RoPE into one out-of-place kernel that writes the attention's input.)
 * For every row t < L, head h < H and tensor x in {q, k} with weight w = wq or wk:
 *   y = x[t,h,:] / sqrt(mean_c x[t,h,c]^2 + eps) * w      (w = 1 when the pointer is NULL)
 *   out[t,h,j]     = y[j] cos[t,j] - y[j+d/2] sin[t,j]    for j < d/2
 *   out[t,h,j+d/2] = y[j+d/2] cos[t,j] + y[j] sin[t,j]
 * or, with WA_ROPE_INTERLEAVED, the same rotation of pair (2j, 2j+1) by angle j.
 * q, k, q_out, k_out: device pointers to [L, H, d] tensors (the wa_forward layout) of
 * element type `dtype` (WA_BF16 or WA_F32), 16-byte aligned, caller-owned; q_out may be q
 * and k_out may be k (in place), other overlaps are rejected.  cos, sin: device pointers
 * to [L, d/2] fp32 angle tables (row t's cosines and sines), 16-byte aligned.  wq, wk:
 * device pointers to d fp32 weights, 16-byte aligned, or NULL.  eps >= 0.  d is 64 or 128.
 * Computed in fp32; outputs rounded to `dtype` (nearest even).  v is not involved.
 * stream: a hipStream_t (NULL = default); the call enqueues one kernel and returns
 * without synchronising; it allocates nothing.  L = 0 enqueues nothing and reads no pointer
 * (NULL is accepted then: an empty tensor may have no storage).
 * Errors: WA_ERR_INVALID (NULL / misaligned / overlapping pointers, bad dtype, flags,
 * L, H or eps), WA_ERR_UNSUPPORTED (d, or L*H*d >= 2^31), WA_ERR_HIP (launch failure).
 */
int wa_qk_norm_rope(const void* q, const void* k, void* q_out, void* k_out, const float* cos,
                    const float* sin, const float* wq, const float* wk, int L, int H, int d,
                    float eps, int flags, int dtype, void* stream);

/* wa_last_error -- message of the calling thread's last non-zero status ("" if none). */
const char* wa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WA_H_ */

// HIP kernels of the decomposed chunk-windowed softmax attention, written for gfx950.
//
// Method: lqnn.cn article on VDN-Minimax-H3 window attention.  §一 defines the window
// (whole chunks within +-radius, global tokens fully connected); §三 replaces the masked
// attention by plain dense attentions over row groups with identical kept-KV sets, plus
// the global rows, scattered into one contiguous output.
//
// Kernels
//   attn_kernel     one work item = (block of up to 256 query rows, head, <= 2 key
//                   segments).  Both legs run in the same launch: window items read their
//                   chunk span and then the global rows in place (no gathered copy);
//                   global-leg items read one key split and write fp32 partials.
//   combine_kernel  log-sum-exp merge of the global leg's key splits into the output.
//   f32_to_bf16     staging of fp32 inputs into bf16 for the matrix products.
//
// Attention mainloop (4 waves per block, one per SIMD; per wave 64 query rows as two
// 32-row blocks; all of q/k/v/out are [L, H, d]):
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K tile rows (keys) from LDS, B = the
//   wave's Q rows held in registers.  In the accumulator layout each lane then holds 16
//   keys of ONE query per 32-key block, so the row max / row sum are in-lane reductions
//   plus a single exchange with the lane 32 apart (v_permlane32_swap).
//   O^T += V^T P^T on the same instruction: B = P^T straight from the S^T accumulators
//   (rounded to bf16), A = V^T read from the row-major V tile with ds_read_tr16_b64
//   (LDS transpose read), so V needs no transposed copy anywhere.  Each K and V fragment
//   read from LDS feeds the matrix ops of both 32-row blocks.
//   Softmax runs in the log2 domain (exp2 with log2(e)/sqrt(d) folded into one FMA),
//   online over 64-key tiles with fp32 running max / sum / accumulators.
//   The matrix ops of one tile come in four groups (S of block 0, PV of block 1 for the
//   previous tile, S of block 1, PV of block 0; 16 each at d = 128); the exponentials, bf16
//   packing and row sums of the other block, and the LDS reads of the next fragments, are
//   interleaved one matrix op at a time, so the vector ALU and LDS work hides under the
//   matrix pipe.  At d = 64, where the vector ALU is the bound, the row sums are four more
//   matrix ops per PV group against an all-ones operand instead.
//   A wave whose rows lie past the end of an item runs a loop of its own that only takes
//   its share of the tile loads and the barriers.  An item of at most 64 rows (d = 128; at
//   H3 the last rows of every group) is instead split over all four waves: 32 rows and one
//   32-key half of every tile each, the halves merged by log-sum-exp through the LDS.
//   K/V tiles stream through a 4-deep LDS ring filled by direct global->LDS 16-byte loads
//   (no registers, no LDS write instructions), issued three tiles ahead and spread over
//   the matrix ops; one barrier per tile.  The loads go through range-checked buffer
//   resources, so a tile costs one scalar row offset and one add per slice, with no
//   per-lane clamping at segment or tensor ends.  LDS rows hold d bf16; 16-byte chunks are
//   XOR-swizzled per row (applied on the global side of the DMA) so the K reads and the
//   transpose reads are free of bank conflicts.
//   The running max is raised lazily: exponentials are taken against the running max as it
//   stands, and only when some weight of a tile may exceed 2^8 (its row sums exceed 2^8)
//   does a wave-uniform slow path find the tile max and raise each row's max to it
//   (rescaling its accumulators); the same path masks keys past a segment end.  Whether a
//   tile needs it for reasons other than its data (first tile, masked keys) is known before
//   the tile: one scalar compare.
//   The launch is persistent: one block per CU takes work units from its XCD's queue in the
//   plan's launch order (blocks are dispatched round-robin over the XCDs), a contiguous run
//   of window units, so the query tiles of one group run side by side and share that XCD's
//   L2, followed by its share of the shorter global-leg units.  A block whose queue is empty
//   takes units from the other XCDs' queues, which evens out the end of the launch.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace wa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;         // waves per block, one per SIMD
constexpr int kWaveRows = 64;  // query rows per wave (two 32-row blocks)
constexpr int kBN = kBlockN;   // keys per tile
static_assert(kBN == 64, "the fragment code below assumes 64-key tiles");

constexpr int kXcds = kXcdCount;  // blocks are dispatched round-robin over the XCDs
constexpr int kListOffset = 64;   // byte offset of a tile list in the output staging area

// 16-byte chunk swizzle of an LDS row.  The LDS has 64 banks (256 bytes per pass); a
// ds_read_b128 pass serves 16 lanes and a ds_read_tr16_b64 pass 32 lanes.
//   d = 128 (256-byte rows, 16 chunks): a bijection on row % 16, so 16 consecutive rows at
//     one logical chunk hit 16 distinct bank groups, and the 4 rows of a transpose read
//     land their 4-chunk groups in distinct quarters.
//   d = 64 (128-byte rows, two rows per bank line): a bijection on (row / 2) % 8 within
//     each row parity; rows 2 apart differ in bit 2 so a transpose read's 4-chunk groups
//     do not collide.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (1.0, 1.0) in bf16: v_dot2 against it adds the two bf16 halves of a word in fp32.
#define kOnes2 (__builtin_bit_cast(bf16x2, 0x3f803f80u))

// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 cvt_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_convertvector(x, bf16x2);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) { return __builtin_bit_cast(uint32_t, cvt_bf16x2(a, b)); }

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

struct AttnParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  void* __restrict__ out;
  const Item* __restrict__ items;
  const int32_t* __restrict__ work;
  int32_t* __restrict__ counters;  // kXcds queue counters, then the count of finished blocks
  int persistent;                   // 0: block b runs unit work[(b % 8) * per_xcd + b / 8] only
  float* __restrict__ part_o;
  float* __restrict__ part_ml;
  int H, G, frame_rows, n_items, total, per_xcd;
  uint32_t tensor_bytes;  // bytes of one of q/k/v: L * H * D * 2
  float scale_log2;
};

// Parameters of the tile-list instantiation (block-sparse plans): entries (first key row
// << 1) | needs_mask, and the geometry whose window rule masks the flagged tiles.
struct AttnParamsTL : AttnParams {
  const int32_t* __restrict__ tiles;
  int T, S, K, radius, n_chunks;
};

// One block = 4 waves (one per SIMD); one wave = 64 query rows as two 32-row blocks
// (qb = 0, 1).  Every K and V fragment read from LDS feeds both blocks' matrix ops.
//
// Per 64-key tile the wave runs four slots of matrix ops (S of block 0, PV of block 1 for
// the previous tile, S of block 1, PV of block 0), each paired with vector work of the
// other block that does not depend on them, so the matrix pipe stays busy (the software
// pipeline is laid out before the tile loop).  The exponentials of a tile are taken
// against the running max before the tile's own max is known; a wave-uniform slow path
// redoes a block's tile when some weight exceeds 2^8, and for a unit's first tile and
// tiles with masked keys (segment end, causal diagonal).
//
// TL (block-sparse plans): every item's keys are a list of 64-key tiles read through an
// index list (copied into the idle output staging area of the LDS at the start of the unit);
// flagged tiles take the slow path, which keeps each row's kept keys by the window rule of
// the geometry (the row's chunk span and the global rows) instead of a segment end.
template <int D, bool OUT_F32, bool TL>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_kernel(std::conditional_t<TL, AttnParamsTL, AttnParams> p) {
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int ROWB = D * 2;                   // bytes per LDS row
  constexpr int TILEB = kBN * ROWB;             // bytes per K or V tile
  constexpr int NJ = TILEB / 1024;              // 1 KB DMA slices (one wave instruction) per tile
  constexpr int JPW = NJ / kNW;                 // slices per wave per tensor per tile
  constexpr int KS = D / 16;                    // MFMA k-steps over d
  constexpr int DB = D / 32;                    // 32-wide output column blocks
  static_assert(NJ % kNW == 0, "tile slices must divide evenly over the waves");
  constexpr float kRowSumLimit = 256.f;         // fast path only while every P of the tile <= 2^8
  // d = 64: the row sums of P come from matrix ops against an all-ones operand (four per
  // block and tile, at the end of the PV slot) instead of vector adds.  At d = 64 a tile has
  // half the matrix work of d = 128 and the same vector work, so the vector ALU is the
  // bound and the trade pays; at d = 128 the matrix pipe is the busier one and it would not.
  constexpr bool ONES = D == 64;
  // Items of at most 64 rows run split over the four waves by key half (d = 128, window
  // and global-leg items without tile lists; see the split-item loop below).
  constexpr bool kSplitItems = !ONES && !TL;

  constexpr int NBUF = 4;                       // LDS ring of (K, V) tile pairs
  constexpr int RINGB = NBUF * 2 * TILEB;       // bytes of the ring
  constexpr int STAGEB = 8192;                  // per-wave output staging area after the ring
  static_assert(kListOffset + 4 * kMaxListTiles <= kNW * STAGEB, "a tile list fits the staging areas");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[RINGB + kNW * STAGEB];  // K0 V0 K1 V1 ... stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;     // half of the wave: k sub-block of the MFMA operands
  const int l32 = lane & 31;

  // Persistent blocks, one per CU: each runs work units (fetch_unit) until all queues are
  // empty.  Blocks are dispatched round-robin over the XCDs.
  const int xcd = blockIdx.x % kXcds;
  // ONES: bf16 1.0 in every element, the A operand of the row-sum matrix ops, kept in AGPRs
  // (the empty asm stops the compiler from rebuilding it before every use)
  bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  if constexpr (ONES) asm volatile("" : "+a"(ones));
  // The next unit, broadcast by wave 0; it shares wave 0's staging area, which is idle from
  // the end of one unit's epilogue to the next unit's epilogue.
  int& s_unit = *reinterpret_cast<int*>(smem + RINGB);
  auto run_item = [&](const int unit) __attribute__((always_inline)) {
  const int h = unit / p.n_items;
  const Item it = p.items[unit - h * p.n_items];
  const int H = p.H;
  const uint32_t row_bytes = uint32_t(H) * D * 2;  // bytes between consecutive rows of q/k/v

  // ---- Q fragments (B operand of S^T = K Q^T): lane = query row, 8 d each
  const int row0 = it.q_begin + wave * kWaveRows;
  const bool wave_active = row0 < it.q_end;
  const bool causal = (it.flags & kItemCausal) != 0;  // row r sees keys <= r only
  bf16x8 qf[2][KS];  // loaded in the prologue below, together with the first K/V tile

  // ---- DMA source offsets: LDS slice j holds tile rows [j*1024/ROWB, ...); lane writes LDS
  // chunk (j*64 + lane), i.e. row m/CH, physical chunk m%CH, which holds the logical chunk
  // (physical ^ swz(row)) of that key row.
  // Slice i of a lane lies RPI rows below slice 0 and has the same swizzle (the swizzle
  // depends on row % 16 and RPI is a multiple of 16).  The loads go through buffer
  // resources based at this head's first element: each lane's offset is its slice offset
  // plus the tile's row offset, range checked against the end of the tensor (rows past it
  // read as zero; they only ever land in masked key rows).
  constexpr int RPI = kNW * 64 / CH;  // tile rows between consecutive slices of one wave
  static_assert(RPI % 16 == 0, "slices of one lane must share the row swizzle");
  const uint32_t dma_row0 = uint32_t((wave * 64 + lane) / CH);
  uint32_t dma_off[JPW];  // byte offset of the lane's 16 bytes of slice i within a tile
#pragma unroll
  for (int i = 0; i < JPW; ++i)
    dma_off[i] = (dma_row0 + uint32_t(i * RPI)) * row_bytes +
                 uint32_t((((wave * 64 + lane) % CH) ^ swz<D>(dma_row0)) * 16);
  auto make_rsrc = [&](const uint16_t* t) __attribute__((always_inline)) -> i32x4 {
    const uint64_t a = reinterpret_cast<uint64_t>(t) + uint64_t(h) * (D * 2);
    // readfirstlane: the descriptor is uniform, and the buffer loads need it in SGPRs even
    // where the compiler cannot prove that through the unit loop's control flow
    return i32x4{__builtin_amdgcn_readfirstlane(int32_t(uint32_t(a))),
                 __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(int32_t(p.tensor_bytes - uint32_t(h) * (D * 2))), kBufferWord3};
  };
  i32x4 rsrc_k = make_rsrc(p.k), rsrc_v = make_rsrc(p.v);
  // A buffer load may read an SGPR that a vector instruction wrote (the readfirstlane above)
  // only 5 wait states later.  The loads are inline asm, which the compiler's hazard checks
  // do not see, so the wait is explicit, once per unit; from here on the descriptors are
  // this asm's results, so nothing but scalar moves lies between them and the loads.
  asm volatile("s_nop 4" : "+s"(rsrc_k), "+s"(rsrc_v));

  // ---- LDS read offsets (bytes within a tile)
  uint32_t koff[KS];  // K fragment (key row l32 of a 32-key block, chunk 2s+hh)
#pragma unroll
  for (int s = 0; s < KS; ++s) koff[s] = uint32_t(l32 * ROWB + (((2 * s + hh) ^ swz<D>(l32)) << 4));
  uint32_t voff[DB][2];  // V^T fragment via transpose reads: 4 key rows x 16 dv per 16 lanes
  {
    const int pl = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 8 * rr + 4 * hh + (pl >> 2);  // + 32*b + 16*tt (multiples of 16)
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (pl & 3);
        voff[db][rr] = uint32_t(row * ROWB + (((col >> 3) ^ swz<D>(row)) << 4) + (((col >> 2) & 1) << 3));
      }
  }

  // ---- tile schedule: segment 0 then segment 1, 64 keys per tile (TL: the item's list)
  const int nt0 = (it.kv0_end - it.kv0_begin + kBN - 1) / kBN;
  const int nt1 = (it.kv1_end - it.kv1_begin + kBN - 1) / kBN;
  const int nt = TL ? it.kv0_end : nt0 + nt1;
  // TL: the item's entries in LDS, past the unit slot of wave 0's staging area (the staging
  // areas are idle until the output epilogue, and the loop reads its last entries before its
  // last barrier, so no wave still reads them when another starts its epilogue)
  int32_t* const list = reinterpret_cast<int32_t*>(smem + RINGB + kListOffset);
  if constexpr (TL) {
    for (int i = tid; i < nt; i += kNW * 64) list[i] = p.tiles[it.kv0_begin + i];
    __syncthreads();
  }
  // entry of tile u (clamped to the last tile), a uniform LDS read
  auto entry = [&](int u) __attribute__((always_inline)) -> int { return list[u < nt ? u : nt - 1]; };
  auto tile_range = [&](int t, int& n0, int& nend) __attribute__((always_inline)) {
    if (t < nt0) {
      n0 = it.kv0_begin + t * kBN;
      nend = it.kv0_end;
    } else {
      n0 = it.kv1_begin + (t - nt0) * kBN;
      nend = it.kv1_end;
    }
  };

  // Row offset (bytes) of the first key row of tile u.  Tiles past the last one re-load the
  // last tile (into a slot nobody reads), so every tile issues the same number of loads.
  // Rows past a segment end are the next rows of the tensor (finite data, masked out of the
  // softmax) or, past the tensor, zeros.
  auto tile_off = [&](int u) __attribute__((always_inline)) -> uint32_t {
    if constexpr (TL) {
      return uint32_t(entry(u) >> 1) * row_bytes;
    } else {
      int n0, nend;
      tile_range(u < nt ? u : nt - 1, n0, nend);
      return uint32_t(n0) * row_bytes;
    }
  };
  // DMA load `idx` (slice idx / 2, K for even idx and V for odd) of the tile at row offset
  // `toff` into ring slot u % NBUF.
  // Row offset of tile u from that of tile u - 1 (u >= 1, without tile lists): the next 64
  // rows, the start of segment 1 at its first tile, and past the last tile the last tile again.
  const uint32_t tile_step = kBN * row_bytes, seg1_off = uint32_t(it.kv1_begin) * row_bytes;
  auto next_off = [&](int u, uint32_t prev) __attribute__((always_inline)) -> uint32_t {
    return u >= nt ? prev : u == nt0 ? seg1_off : prev + tile_step;
  };
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));
  auto dma_load = [&](int u, int idx, uint32_t toff) __attribute__((always_inline)) {
    const int i = idx >> 1;
    const uint32_t l = lds_base + uint32_t((2 * (u % NBUF) + (idx & 1)) * TILEB + (i * kNW + wave) * 1024);
    const uint32_t off = dma_off[i] + toff;
    // Issued as asm: the compiler would otherwise make the next LDS read of any buffer wait
    // for every DMA in flight (it cannot tell the ring slots apart).  Completion is ordered
    // by the explicit vmcnt waits before each barrier.  M0 holds the LDS destination (set
    // by the compiler through the operand; the nop covers the M0-write-to-DMA hazard).
    if (idx & 1)
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(rsrc_v), "{m0}"(l) : "memory");
    else
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(rsrc_k), "{m0}"(l) : "memory");
  };
  constexpr int NLD = 2 * JPW;  // DMA loads per tile per wave

  const float c2 = p.scale_log2;
  // Initial running max: finite (so a rescale factor is never exp2 of inf - inf) and below
  // every finite score; the first tile of a unit always takes the slow path, which raises it
  // before any weight is used.
  constexpr float kMaxInit = -0x1p100f;

  float m_run[2], mc[2], l_run[2];  // running max of raw scores (this lane's queries), * c2, sum
  f32x16 oacc[2][DB];
  f32x16 lacc[2];  // ONES: row sums (every element of a lane holds its query's sum)
  float pm[2];     // ONES: max weight of the block's current tile
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m_run[qb] = kMaxInit;
    mc[qb] = kMaxInit * c2;
    l_run[qb] = 0.f;
    if constexpr (ONES) {
      lacc[qb] = f32x16{};
      pm[qb] = 0.f;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
  }

  bf16x8 kf[KS][2];        // K fragments of the current tile: [k-step][32-key block]
  i16x4 vr[4 * DB][2];     // V^T fragments as transpose-read halves: [(b*2+tt)*DB+db][half]
  bf16x2 pw[2][16];        // P^T as bf16 pairs: [qb][pair]; pair n = b*8 + tt*4 + k holds
                           // S elements (b, 8*tt + 2*k + {0, 1}) of this lane
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int n = 0; n < 16; ++n) pw[qb][n] = cvt_bf16x2(0.f, 0.f);

  // koff / voff hold the byte offset of the ring slot being read (K: the tile after the
  // current one; V: the current tile) plus the lane's part; they advance once per tile.
  auto read_k = [&](int idx) __attribute__((always_inline)) {
    const int s = idx >> 1, b = idx & 1;
    kf[s][b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + koff[s] + b * 32 * ROWB));
  };
  auto read_v = [&](int idx) __attribute__((always_inline)) {
    const int f = idx >> 1, rr = idx & 1;
    const int b = f / (2 * DB), tt = (f / DB) & 1, db = f % DB;
    vr[f][rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + voff[db][rr] + (32 * b + 16 * tt) * ROWB));
  };
  // byte offset of ring slot r's K (V: + TILEB)
  auto ring = [](int r) __attribute__((always_inline)) -> uint32_t { return uint32_t(r % NBUF) * 2 * TILEB; };
  auto vfrag = [&](int b, int tt, int db) __attribute__((always_inline)) -> bf16x8 {
    const int f = (b * 2 + tt) * DB + db;
    const u32x4 vw = {__builtin_bit_cast(u32x2, vr[f][0])[0], __builtin_bit_cast(u32x2, vr[f][0])[1],
                      __builtin_bit_cast(u32x2, vr[f][1])[0], __builtin_bit_cast(u32x2, vr[f][1])[1]};
    return __builtin_bit_cast(bf16x8, vw);
  };
  auto pfrag = [&](int qb, int b, int tt) __attribute__((always_inline)) -> bf16x8 {
    const int n = b * 8 + tt * 4;
    return __builtin_shufflevector(__builtin_shufflevector(pw[qb][n], pw[qb][n + 1], 0, 1, 2, 3),
                                   __builtin_shufflevector(pw[qb][n + 2], pw[qb][n + 3], 0, 1, 2, 3), 0, 1, 2, 3,
                                   4, 5, 6, 7);
  };
  // Row sums of exactly the rounded P that multiplies V, so the weights applied to V sum to
  // one (with one dominant key the output is then that key's value row, whatever its
  // rounding); two fp32 accumulation chains per block over this lane's keys.  A pair is
  // added either by one v_dot2 against (1, 1) or by widening its two bf16 halves (a shift
  // and a mask) and two fp32 adds.  Measured per slot: beside the S matrix ops (operands in
  // AGPRs) a dot op stalls the matrix pipe for about 13 cycles while the four plain ops
  // issue for free; beside the PV matrix ops the single dot op is the cheaper one.
  float rs[2][2];
  auto add_pair = [&](int qb, bf16x2 w) __attribute__((always_inline)) {
    const uint32_t u = __builtin_bit_cast(uint32_t, w);
    rs[qb][0] += __builtin_bit_cast(float, u << 16);
    rs[qb][1] += __builtin_bit_cast(float, u & 0xFFFF0000u);
  };
  auto dot_pair = [&](int qb, int k, bf16x2 w) __attribute__((always_inline)) {
    rs[qb][k & 1] = __builtin_amdgcn_fdot2_f32_bf16(w, kOnes2, rs[qb][k & 1], false);
  };
  // One pair of P against the given max, and its row sums.
  auto p_pair = [&](int qb, const f32x16 (&sa)[2], int n, float mcq) __attribute__((always_inline)) {
    const int b = n >> 3, e = 2 * (n & 7);
    const float x0 = sa[b][e], x1 = sa[b][e + 1];
    pw[qb][n] = cvt_bf16x2(fast_exp2(__builtin_fmaf(x0, c2, -mcq)), fast_exp2(__builtin_fmaf(x1, c2, -mcq)));
    if constexpr (!ONES) add_pair(qb, pw[qb][n]);
  };
  // Value of the lane 32 apart (the other half of the same query's keys), in both orders.
  auto other_half = [](float x) __attribute__((always_inline)) -> f32x2 {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return f32x2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
  };
  // max over both halves of the wave: {own, other} in some order per lane
  auto pair_max = [&](float x) __attribute__((always_inline)) -> float {
    const f32x2 r = other_half(x);
    return __builtin_fmaxf(r[0], r[1]);
  };
  // ---- Software pipeline over 64-key tiles, one "slot" = one group of matrix ops with a
  // share of the vector work that is independent of them:
  //   slot 0: S0(t) = K(t) Q0^T          | P1(t-1) pairs 8..15, 2nd half of the DMA of t+2;
  //                                        then the slow path of block 1 (tile t-1) if due
  //   slot 1: O1 += V(t-1)^T P1(t-1)^T   | P0(t) pairs 0..7, row sums of P1(t-1), V(t)
  //                                        transpose reads (each fragment right after its
  //                                        last use by this slot)
  //   slot 2: S1(t) = K(t) Q1^T          | P0(t) pairs 8..15; then the slow path of block 0
  //                                        (tile t) if due
  //   barrier: tile t+1 has landed for every wave
  //   slot 3: O0 += V(t)^T P0(t)^T       | P1(t) pairs 0..7, K(t+1) reads, row sums of P0(t),
  //                                        1st half of the DMA of t+3
  // The LDS ring has 4 slots: the DMA of t+3 overwrites tile t-1, whose reads every wave
  // finished before the barrier of tile t.  Before the first tile, block 1's "previous tile"
  // is empty (scores -inf, V zero), so every iteration runs the same code; block 1's last
  // PV runs after the loop.
  // P pairs are staged: pair k's FMAs issue at step fs(k), its exponentials one step later,
  // its bf16 packing and its row sums in the next steps (see stage_at); beside the S
  // matrix ops the packing waits two steps, since an op that reads a fresh exp2 result one
  // matrix op later stalls there.
  // Each stage's result is pinned at its step (an empty asm that reads it): without the
  // pins the compiler sinks pure arithmetic next to its first use, which puts dependent
  // vector ops back to back.
  // Slow path.  The exponentials are taken against the running max as it stands; a block's
  // tile goes to the slow path (wave-uniform), which finds the tile max and raises the
  // running max of every row whose tile max exceeds it, when
  //   - it is the unit's first tile or has masked keys (segment end, causal diagonal): known
  //     before the tile, one scalar compare per tile;
  //   - some row sum of the tile exceeds 2^8 (any P above 2^8 makes it so; ONES: some P
  //     exceeds 2^8, from one max per pair).
  constexpr int NS = 2 * KS;                // matrix ops of an S slot
  constexpr int NPV = 4 * DB;               // PV matrix ops of a PV slot
  constexpr int NP = NPV + (ONES ? 4 : 0);  // all matrix ops of a PV slot (ONES: + the row sums)
  static_assert(NS % 4 == 0 && NPV % 4 == 0 && (2 * KS) % NPV == 0 && 16 % NPV == 0 && NLD % 2 == 0,
                "slot work must divide evenly over the steps");
  // Slow path of block qb on tile t (TL: first key row n0 and whether the tile is masked).
  auto slow_block = [&](int qb, f32x16 (&sa)[2], int t, int n0, bool masked) __attribute__((always_inline)) {
    if constexpr (TL) {
      if (masked) {
        // the window rule for this lane's query row: frame rows keep their window's chunk
        // span and the global rows, global rows keep every key; keys past L are none
        const int qrow = row0 + 32 * qb + l32;
        int klo = 0, khi = p.frame_rows;
        if (qrow < p.frame_rows) {
          const int c = qrow / p.S / p.K;
          const int lo = c - p.radius > 0 ? c - p.radius : 0;
          const int hi = c + p.radius < p.n_chunks - 1 ? c + p.radius : p.n_chunks - 1;
          const int fend = (hi + 1) * p.K < p.T ? (hi + 1) * p.K : p.T;
          klo = lo * p.K * p.S;
          khi = fend * p.S;
        }
        const int L = p.frame_rows + p.G;
        // key (n0 + b*32 + (i/4)*8 + 4*hh + i%4) kept iff in [klo, khi) or in [frame_rows, L)
        const int base = n0 + 4 * hh;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = base + b * 32 + (i >> 2) * 8 + (i & 3);
            const bool keep = (j >= klo && j < khi) || (j >= p.frame_rows && j < L);
            sa[b][i] = keep ? sa[b][i] : -__builtin_inff();
          }
      }
    } else {
      int k0, kend;
      tile_range(t, k0, kend);
      const int valid = kend - k0;
      if (valid < kBN || causal) {
        // tile keys at or past `lim` are masked: the segment end, and for causal items also
        // every key after this lane's own query row
        int lim = valid;
        if (causal) lim = __builtin_elementwise_min(lim, row0 + 32 * qb + l32 - k0 + 1);
        lim -= 4 * hh;  // key (b*32 + (i/4)*8 + 4*hh + i%4) >= valid
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sa[b][i] = (b * 32 + (i >> 2) * 8 + (i & 3)) >= lim ? -__builtin_inff() : sa[b][i];
      }
    }
    float mt = sa[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, sa[b][i]);
    mt = pair_max(mt);
    // Every row whose tile max exceeds its running max raises it to that max (the branch is
    // wave-uniform, the choice per row): the other rows keep their max and rescale by
    // exactly 1, so a row's arithmetic never depends on the scores of the other rows in the
    // wave.  Raising to the exact max, not only past a 2^8 growth, matters for the row-sum
    // test: a row whose weights sit between 2^3 and 2^8 on many keys trips it, and left at
    // its old max it would trip it again on every following tile.
    const bool grow = mt > m_run[qb];
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_run[qb];
      const float alpha = fast_exp2((m_run[qb] - m_new) * c2);
      m_run[qb] = m_new;
      mc[qb] = m_new * c2;
      if constexpr (ONES) lacc[qb] *= alpha;
      else l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[qb][db][i] *= alpha;
    }
    rs[qb][0] = rs[qb][1] = 0.f;
#pragma unroll
    for (int n = 0; n < 16; ++n) p_pair(qb, sa, n, mc[qb]);
  };

  f32x16 s0[2], s1[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) s1[b][i] = -__builtin_inff();
#pragma unroll
  for (int f = 0; f < 4 * DB; ++f) vr[f][0] = vr[f][1] = i16x4{0, 0, 0, 0};
  rs[1][0] = rs[1][1] = 0.f;
  const f32x16 zero = {};
  float fa[8], fb[8];  // staged pair values

  // stage work of pairs [lo, lo + 8) of block qb at step i of an N-step slot.  Pairs 0..7
  // run beside PV matrix ops (packing at fs + 2, one v_dot2 at fs + 3), pairs 8..15 beside
  // S matrix ops (packing at fs + 3, shift/mask/add row sums at fs + 4).
  auto stage_at = [&](int qb, const f32x16 (&sa)[2], int lo, int N, int i) __attribute__((always_inline)) {
    const bool pv = lo == 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int fs = k * N / 8;
      const int n = lo + k, b = n >> 3, e = 2 * (n & 7);
      const int f_pack = pv ? fs + 2 : fs + 3, f_sum = f_pack + 1;
      if constexpr (!ONES) {
        if (f_sum == i) {
          if (pv) {
            dot_pair(qb, k, pw[qb][n]);
          } else {
            add_pair(qb, pw[qb][n]);
            asm volatile("" ::"v"(rs[qb][0]), "v"(rs[qb][1]));
          }
        }
      }
      if (f_pack == i) {
        pw[qb][n] = cvt_bf16x2(fa[k], fb[k]);
        if constexpr (ONES) {
          pm[qb] = __builtin_fmaxf(__builtin_fmaxf(pm[qb], fa[k]), fb[k]);
          asm volatile("" ::"v"(pw[qb][n]), "v"(pm[qb]));
        } else {
          asm volatile("" ::"v"(pw[qb][n]));
        }
      }
      if (fs + 1 == i) {
        fa[k] = fast_exp2(fa[k]);
        fb[k] = fast_exp2(fb[k]);
        asm volatile("" ::"v"(fa[k]), "v"(fb[k]));
      }
      if (fs == i) {
        if constexpr (ONES) {
          if (pv && k == 0) pm[qb] = 0.f;  // the block's first pair of the tile
        }
        const float x0 = sa[b][e], x1 = sa[b][e + 1];
        fa[k] = __builtin_fmaf(x0, c2, -mc[qb]);
        fb[k] = __builtin_fmaf(x1, c2, -mc[qb]);
        asm volatile("" ::"v"(fa[k]), "v"(fb[k]));
      }
    }
  };
  // Keeps the fast-path P computed ahead of the slow-path branch (and so inside the slot
  // whose matrix ops hide it): an empty asm that reads it.
  auto pin_p = [&](int qb) __attribute__((always_inline)) {
    asm volatile("" ::"v"(pw[qb][0]), "v"(pw[qb][1]), "v"(pw[qb][2]), "v"(pw[qb][3]), "v"(pw[qb][4]),
                 "v"(pw[qb][5]), "v"(pw[qb][6]), "v"(pw[qb][7]), "v"(pw[qb][8]), "v"(pw[qb][9]), "v"(pw[qb][10]),
                 "v"(pw[qb][11]), "v"(pw[qb][12]), "v"(pw[qb][13]), "v"(pw[qb][14]), "v"(pw[qb][15]));
  };
  // block qb's verdict on tile t (its scores in sa; TL: n0, masked from the tile's entry)
  auto check_block = [&](int qb, f32x16 (&sa)[2], int t, int n0, bool dirty, bool masked)
                         __attribute__((always_inline)) {
    pin_p(qb);
    if constexpr (ONES) {
      asm volatile("" ::"v"(pm[qb]));
      if (dirty || __builtin_amdgcn_ballot_w64(pm[qb] > kRowSumLimit) != 0) slow_block(qb, sa, t, n0, masked);
    } else {
      asm volatile("" ::"v"(rs[qb][0]), "v"(rs[qb][1]));
      if (dirty || __builtin_amdgcn_ballot_w64(rs[qb][0] + rs[qb][1] > kRowSumLimit) != 0)
        slow_block(qb, sa, t, n0, masked);
      l_run[qb] += rs[qb][0] + rs[qb][1];
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Tiles that take the slow path whatever their data (see above), as "the next such tile
  // after u": the first tile, the last tile of a segment that ends inside it, and for causal
  // items every tile from the first one with a key after some row of the wave (all tiles when
  // forced).  Block 1 checks each tile one iteration after block 0 and reuses its verdict
  // (block 0's causal rows come first, so this is conservative for block 1).
  const int t_rag0 = (it.kv0_end - it.kv0_begin) % kBN != 0 ? nt0 - 1 : -1;
  const int t_rag1 = nt1 > 0 && (it.kv1_end - it.kv1_begin) % kBN != 0 ? nt - 1 : -1;
  const int t_all = !causal ? nt : [&] {
    const int x = row0 - (kBN - 1) - it.kv0_begin;  // tile t is masked for row0 iff t * kBN > x
    return x < 0 ? 0 : x / kBN + 1;
  }();
  auto next_dirty = [&](int u) __attribute__((always_inline)) -> int {
    int n = u + 1 > t_all ? u + 1 : t_all;
    if (t_rag0 > u && t_rag0 < n) n = t_rag0;
    if (t_rag1 > u && t_rag1 < n) n = t_rag1;
    return n;
  };
  // PV slot of block qb: N matrix ops (when `mma`), then the tail steps for the staged pairs.
  // Steps after the last matrix op of a slot in which the staged pairs finish: the last pair
  // starts at step 7 * N / 8 and ends at most 4 steps later (N = NS = NP).
  static_assert(NS == NPV, "S and PV slots have the same number of value steps");
  constexpr int kTail = 7 * NS / 8 + 5 - NS;
  constexpr int kTailP = 7 * NP / 8 + 5 - NP;
  auto pv_slot = [&](int qb, bool mma, auto&& extra) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NP + kTailP; ++i) {
      if (mma && i < NPV) {
        const int b = i / (2 * DB), tt = (i / DB) & 1, db = i % DB;
        oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(b, tt, db), pfrag(qb, b, tt), oacc[qb][db], 0, 0, 0);
      } else if (ONES && mma && i < NP) {
        const int j = i - NPV;  // 16-key piece j of the tile: l += 1 P^T
        lacc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pfrag(qb, j >> 1, j & 1), lacc[qb], 0, 0, 0);
      }
      extra(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto s_slot = [&](int qb, f32x16 (&sa)[2], bool mma, auto&& extra) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NS + kTail; ++i) {
      if (mma && i < NS) {
        const int st = i >> 1, b = i & 1;
        sa[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st][b], qf[qb][st], st == 0 ? zero : sa[b], 0, 0, 0);
      }
      extra(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // s_waitcnt with vmcnt = n (n < 16) and the other counters at their maximum
#define WA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

  // ---- Output of the 32-row block qb (rows r0 ..): a lane holds 4-column pieces of its row
  // spread over the row, so direct stores would write 32 rows per instruction in 8- or
  // 16-byte pieces.  The block goes through this wave's LDS staging area instead (16-byte
  // chunks XOR-swizzled by row) and leaves as whole rows: 16 lanes x 16 bytes per 256 bytes
  // of a row.  Global-leg items write the fp32 partial result (O, max, sum) instead.
  auto output_block = [&](int qb, int r0) __attribute__((always_inline)) {
    unsigned char* const stage = smem + RINGB + wave * STAGEB;
    const bool partial = it.split >= 0;
    // Lane indices redefined here (empty asm) so that the staging addresses, which depend
    // only on them, are computed here and not hoisted out of the unit loop into the tile
    // loop's register budget.
    int orow_l = l32, olane = lane;
    asm volatile("" : "+v"(orow_l), "+v"(olane));
    constexpr int EB = OUT_F32 ? 4 : 2;  // bytes per element of the final output
    const float l_tot = ONES ? lacc[qb][0] : [&] {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, l_run[qb]),
                                                      __builtin_bit_cast(uint32_t, l_run[qb]), false, false);
      return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
    }();
    const int rows_here = it.q_end - r0;  // valid rows of this block (may be <= 0)
    if (rows_here <= 0) return;

    auto emit = [&](auto eb_c, auto row_dst) __attribute__((always_inline)) {
      constexpr int E = decltype(eb_c)::value;       // bytes per element
      constexpr int RB = D * E;                      // bytes per output row
      constexpr int CR = (RB < 256 ? RB : 256) / 16;  // 16-byte chunks per row per round
      constexpr int ROUNDS = RB / (CR * 16);
      static_assert(32 * CR * 16 <= STAGEB, "one round of 32 rows fits the staging area");
      const float mul = 1.f / l_tot;
#pragma unroll
      for (int rd = 0; rd < ROUNDS; ++rd) {
        // write: the lane's 4-element pieces of row l32 that fall in this round
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int off = (32 * db + 8 * g4) * E + (E == 2 ? 8 : 16) * hh - rd * CR * 16;  // byte offset in the round
            if (off < 0 || off >= CR * 16) continue;
            const int c = off >> 4, within = off & 15;
            unsigned char* dst = stage + orow_l * (CR * 16) + ((c ^ (orow_l & (CR - 1))) << 4) + within;
            const float v0 = oacc[qb][db][4 * g4] * mul, v1 = oacc[qb][db][4 * g4 + 1] * mul;
            const float v2 = oacc[qb][db][4 * g4 + 2] * mul, v3 = oacc[qb][db][4 * g4 + 3] * mul;
            if constexpr (E == 2) {
              *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            } else {
              *reinterpret_cast<f32x4*>(dst) = f32x4{v0, v1, v2, v3};
            }
          }
        // read back whole chunks in row order and store them
#pragma unroll
        for (int k = 0; k < 32 * CR / 64; ++k) {
          const int j = k * 64 + olane, r = j / CR, c = j % CR;
          const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * (CR * 16) + ((c ^ (r & (CR - 1))) << 4));
          if (r < rows_here) *reinterpret_cast<u32x4*>(row_dst(r0 + r) + rd * CR * 16 + c * 16) = x;
        }
      }
    };
    if (!partial) {
      emit(std::integral_constant<int, EB>{}, [&](int qrow) __attribute__((always_inline)) {
        return reinterpret_cast<unsigned char*>(p.out) + ((int64_t)qrow * H + h) * D * EB;
      });
    } else {
      const int qrow = r0 + l32;
      if (qrow < it.q_end) {
        const int64_t slot = ((int64_t)it.split * p.G + (qrow - p.frame_rows)) * H + h;
        float* po = p.part_o + slot * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int dv = 32 * db + 8 * g4 + 4 * hh;
            const f32x4 o = {oacc[qb][db][4 * g4], oacc[qb][db][4 * g4 + 1], oacc[qb][db][4 * g4 + 2],
                             oacc[qb][db][4 * g4 + 3]};
            *reinterpret_cast<f32x4*>(po + dv) = o;
          }
        if (hh == 0) {
          const float2 ml = make_float2(m_run[qb] * c2, l_tot);
          *reinterpret_cast<float2*>(p.part_ml + slot * 2) = ml;
        }
      }
    }
  };

  // ---- Items of at most one wave's rows (at H3 the last 64 rows of every 2880-row group):
  // run as above, one wave would work while three SIMDs idle.  Here every wave takes one
  // 32-row block (qs = wave & 1) and one 32-key half (kh = wave >> 1) of every tile, with the
  // same ring, loads and barriers; the two key halves of a block merge by log-sum-exp through
  // the LDS at the end.  Per tile two slots of KS matrix ops:
  //   slot A: S(t) = K(t) Q^T (this key half)  | P(t-1) pairs 4..7, second half of the DMA
  //                                             of t+2; then the slow path of tile t-1 if
  //                                             due (as above, over this wave's 16 keys per row)
  //   barrier: tile t+1 has landed for every wave
  //   slot B: O += V(t-1)^T P(t-1)^T          | P(t) pairs 0..3, V(t) reads (each right
  //                                             after its fragment's last use), K(t+1)
  //                                             reads, first half of the DMA of t+3
  // S, P and the row sums of a tile alternate between two register sets (tile t's are
  // written while tile t-1's are still read), so the tile loop is unrolled twice.
  if constexpr (kSplitItems) {
    if (!causal && it.q_end - it.q_begin <= kWaveRows) {
      const int qs = wave & 1, kh = wave >> 1;
      const int r0q = it.q_begin + 32 * qs;
      constexpr int NQ = KS;  // matrix ops of either slot (= 2 * DB)
      static_assert(NQ == 2 * DB && NQ % (NLD / 2) == 0 && NQ % 8 == 0, "split-item slots");
      f32x16(&sq)[2] = s0;
#pragma unroll
      for (int s = 0; s < KS; ++s) koff[s] += uint32_t(kh * 32 * ROWB);
#pragma unroll
      for (int db = 0; db < DB; ++db) voff[db][0] += uint32_t(kh * 32 * ROWB), voff[db][1] += uint32_t(kh * 32 * ROWB);
      {
        const uint32_t toff0 = tile_off(0);
#pragma unroll
        for (int idx = 0; idx < NLD; ++idx) dma_load(0, idx, toff0);
      }
      {
        const int qrow = r0q + l32;
        const bool ok = qrow < it.q_end;
        const uint16_t* src = p.q + ((int64_t)qrow * H + h) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (ok) x = *reinterpret_cast<const u32x4*>(src + 16 * s);
          qf[0][s] = __builtin_bit_cast(bf16x8, x);
        }
      }
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      uint32_t toff_q = tile_off(1);
#pragma unroll
      for (int idx = 0; idx < NLD; ++idx) dma_load(1, idx, toff_q);
      toff_q = tile_off(2);
#pragma unroll
      for (int idx = 0; idx < NLD / 2; ++idx) dma_load(2, idx, toff_q);
      barrier();
#pragma unroll
      for (int s = 0; s < KS; ++s) read_k(2 * s);
#pragma unroll
      for (int st = 0; st < KS; ++st) koff[st] += ring(1);
#pragma unroll
      for (int db = 0; db < DB; ++db) voff[db][0] += TILEB, voff[db][1] += TILEB;

      // pairs lo .. lo+3 of P into register set `buf` at step i of a slot: pair k's FMA at
      // step (k - lo) * NQ / 4, exp2 one step later, packing the step after, row sum (v_dot2)
      // the step after that
      constexpr int kTailQ = 3 * NQ / 4 + 4 - NQ;
      auto stage_q = [&](int buf, int lo, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int k = lo; k < lo + 4; ++k) {
          const int fs = (k - lo) * NQ / 4;
          if (fs + 3 == i) dot_pair(buf, k, pw[buf][k]);
          if (fs + 2 == i) {
            pw[buf][k] = cvt_bf16x2(fa[k], fb[k]);
            asm volatile("" ::"v"(pw[buf][k]));
          }
          if (fs + 1 == i) {
            fa[k] = fast_exp2(fa[k]);
            fb[k] = fast_exp2(fb[k]);
            asm volatile("" ::"v"(fa[k]), "v"(fb[k]));
          }
          if (fs == i) {
            fa[k] = __builtin_fmaf(sq[buf][2 * k], c2, -mc[0]);
            fb[k] = __builtin_fmaf(sq[buf][2 * k + 1], c2, -mc[0]);
            asm volatile("" ::"v"(fa[k]), "v"(fb[k]));
          }
        }
      };
      // slow path of tile t: mask keys past the segment end, raise the max of every row whose
      // tile max exceeds it, recompute P(t) into `buf`
      auto slow_q = [&](int buf, int t) __attribute__((always_inline)) {
        int k0, kend;
        tile_range(t, k0, kend);
        const int valid = kend - k0;
        if (valid < kBN) {
          const int lim = valid - 32 * kh - 4 * hh;  // key (32*kh + (i/4)*8 + 4*hh + i%4) >= valid
#pragma unroll
          for (int i = 0; i < 16; ++i) sq[buf][i] = ((i >> 2) * 8 + (i & 3)) >= lim ? -__builtin_inff() : sq[buf][i];
        }
        float mt = sq[buf][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = __builtin_fmaxf(mt, sq[buf][i]);
        mt = pair_max(mt);
        const bool grow = mt > m_run[0];
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mt : m_run[0];
          const float alpha = fast_exp2((m_run[0] - m_new) * c2);
          m_run[0] = m_new;
          mc[0] = m_new * c2;
          l_run[0] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[0][db][i] *= alpha;
        }
        rs[buf][0] = rs[buf][1] = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pw[buf][k] = cvt_bf16x2(fast_exp2(__builtin_fmaf(sq[buf][2 * k], c2, -mc[0])),
                                  fast_exp2(__builtin_fmaf(sq[buf][2 * k + 1], c2, -mc[0])));
          add_pair(buf, pw[buf][k]);
        }
      };
      // slot B's matrix op i: O += V^T P^T for (16-key piece tt, 32 columns db) of the tile
      auto pv_q = [&](int buf, int i) __attribute__((always_inline)) {
        const int tt = i / DB, db = i % DB;
        oacc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfrag(0, tt, db), pfrag(buf, 0, tt), oacc[0][db], 0, 0, 0);
      };
      // tile t's verdict once all its pairs are done (register set `buf`); then its row sums
      // join the running sum
      auto check_q = [&](int buf, int t, bool dirty) __attribute__((always_inline)) {
        asm volatile("" ::"v"(pw[buf][0]), "v"(pw[buf][1]), "v"(pw[buf][2]), "v"(pw[buf][3]), "v"(pw[buf][4]),
                     "v"(pw[buf][5]), "v"(pw[buf][6]), "v"(pw[buf][7]), "v"(rs[buf][0]), "v"(rs[buf][1]));
        if (dirty || __builtin_amdgcn_ballot_w64(rs[buf][0] + rs[buf][1] > kRowSumLimit) != 0) slow_q(buf, t);
        l_run[0] += rs[buf][0] + rs[buf][1];
        __builtin_amdgcn_sched_barrier(0);
      };
      int nd = 0;               // next tile that takes the slow path
      bool dirty_prev = false;  // verdict input of tile t-1 (tile -1: none)
      // tile -1 (register set 1): scores -inf, so its weights, row sums and PV are zero
#pragma unroll
      for (int i = 0; i < 16; ++i) sq[1][i] = -__builtin_inff();
      rs[1][0] = rs[1][1] = 0.f;
      auto tile_q = [&](int t, auto cur_c) __attribute__((always_inline)) {
        constexpr int cur = decltype(cur_c)::value, prv = cur ^ 1;  // register sets of tiles t, t-1
        const uint32_t step_k = ring(t + 2) - ring(t + 1);
        const uint32_t step_v = ring(t + 1) - ring(t);
        const bool dirty = t == nd;
        if (__builtin_expect(dirty, 0)) nd = next_dirty(t);
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
        __builtin_amdgcn_sched_barrier(0);
        // slot A
#pragma unroll
        for (int i = 0; i < NQ + kTailQ; ++i) {
          if (i < NQ) {
            sq[cur] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i][0], qf[0][i], i == 0 ? zero : sq[cur], 0, 0, 0);
            if (i % (NQ / (NLD / 2)) == 0) dma_load(t + 2, NLD / 2 + i / (NQ / (NLD / 2)), toff_q);
          }
          stage_q(prv, 4, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        check_q(prv, t - 1, dirty_prev);
        WA_WAIT_VMCNT(NLD);  // tile t+1 has landed (tile t+2 may still be in flight) ...
        barrier();           // ... for every wave
        toff_q = next_off(t + 3, toff_q);
        // slot B
        rs[cur][0] = rs[cur][1] = 0.f;
#pragma unroll
        for (int i = 0; i < NQ + kTailQ; ++i) {
          if (i < NQ) {
            pv_q(prv, i);
            read_v(2 * i);
            read_v(2 * i + 1);
            read_k(2 * i);
            if (i % (NQ / (NLD / 2)) == 0) dma_load(t + 3, i / (NQ / (NLD / 2)), toff_q);
          }
          stage_q(cur, 0, i);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) voff[db][0] += step_v, voff[db][1] += step_v;
#pragma unroll
        for (int st = 0; st < KS; ++st) koff[st] += step_k;
        dirty_prev = dirty;
      };
      for (int t = 0; t < nt; t += 2) {
        tile_q(t, std::integral_constant<int, 0>{});
        if (t + 1 < nt) tile_q(t + 1, std::integral_constant<int, 1>{});
      }
      // the last tile: its pairs 4..7, its verdict, its PV
      auto last_q = [&](auto buf_c) __attribute__((always_inline)) {
        constexpr int buf = decltype(buf_c)::value;
#pragma unroll
        for (int i = 0; i < NQ + kTailQ; ++i) {
          stage_q(buf, 4, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        check_q(buf, nt - 1, dirty_prev);
#pragma unroll
        for (int i = 0; i < NQ; ++i) pv_q(buf, i);
      };
      if ((nt - 1) & 1) last_q(std::integral_constant<int, 1>{});
      else last_q(std::integral_constant<int, 0>{});
      // merge the key halves: the kh = 1 wave of each block leaves O (64 floats per lane, in
      // lane order, conflict free) and its (max, sum) in the idle ring; the kh = 0 wave, whose
      // lanes own the same rows and columns, merges them and writes the block
      __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the ring's last loads have landed ...
      barrier();                            // ... and no wave reads it any more
      unsigned char* const mb = smem + qs * (DB * 4 * 1024 + 512);
      if (kh == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f32x4*>(mb + (db * 4 + g4) * 1024 + lane * 16) =
                f32x4{oacc[0][db][4 * g4], oacc[0][db][4 * g4 + 1], oacc[0][db][4 * g4 + 2], oacc[0][db][4 * g4 + 3]};
        *reinterpret_cast<f32x2*>(mb + DB * 4 * 1024 + lane * 8) = f32x2{m_run[0], l_run[0]};
      }
      barrier();
      if (kh == 0) {
        const f32x2 ml = *reinterpret_cast<const f32x2*>(mb + DB * 4 * 1024 + lane * 8);
        const float m_new = __builtin_fmaxf(m_run[0], ml[0]);
        const float a0 = fast_exp2((m_run[0] - m_new) * c2), a1 = fast_exp2((ml[0] - m_new) * c2);
        m_run[0] = m_new;
        l_run[0] = l_run[0] * a0 + ml[1] * a1;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(mb + (db * 4 + g4) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[0][db][4 * g4 + j] = oacc[0][db][4 * g4 + j] * a0 + x[j] * a1;
          }
        output_block(0, r0q);
      }
      return;
    }
  }

  // prologue: tile 0 and the Q fragments land together (the explicit wait also tells the
  // compiler that Q is complete, so it adds no wait inside the loop); then tiles 1 and the
  // first half of 2 go in flight.
  {
    const uint32_t toff0 = tile_off(0);
#pragma unroll
    for (int idx = 0; idx < NLD; ++idx) dma_load(0, idx, toff0);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = row0 + 32 * qb + l32;
    const bool ok = qrow < it.q_end;
    const uint16_t* src = p.q + ((int64_t)qrow * H + h) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *reinterpret_cast<const u32x4*>(src + 16 * s);
      qf[qb][s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  uint32_t toff_a = tile_off(1);  // the tile whose DMA is in flight in two halves
#pragma unroll
  for (int idx = 0; idx < NLD; ++idx) dma_load(1, idx, toff_a);
  toff_a = tile_off(2);
#pragma unroll
  for (int idx = 0; idx < NLD / 2; ++idx) dma_load(2, idx, toff_a);
  barrier();
  if (wave_active) {
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) read_k(i);
  }
#pragma unroll
  for (int st = 0; st < KS; ++st) koff[st] += ring(1);  // from here on: the tile after the current
#pragma unroll
  for (int db = 0; db < DB; ++db) voff[db][0] += TILEB, voff[db][1] += TILEB;

  if (!wave_active) {
    // a wave without rows in this item takes only its share of the loads and the barriers
    // (TL: reading each load's entry before the barrier, like the active waves)
    for (int t = 0; t < nt; ++t) {
      int e_dma = 0;
      if constexpr (TL) e_dma = entry(t + 3);
#pragma unroll
      for (int idx = NLD / 2; idx < NLD; ++idx) dma_load(t + 2, idx, toff_a);
      WA_WAIT_VMCNT(NLD);
      barrier();
      if constexpr (TL) toff_a = uint32_t(e_dma >> 1) * row_bytes;
      else toff_a = next_off(t + 3, toff_a);
#pragma unroll
      for (int idx = 0; idx < NLD / 2; ++idx) dma_load(t + 3, idx, toff_a);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // no DMA may still write this block's LDS at exit
    return;
  }
  int n0_prev = 0;
  int nd = 0;                // next tile that takes the slow path
  bool dirty_prev = false;   // block 0's verdict on the previous tile (tile -1: none)
  bool masked_prev = false;
  for (int t = 0; t < nt; ++t) {
    const uint32_t step_k = ring(t + 2) - ring(t + 1);  // slot advance after this tile's reads
    const uint32_t step_v = ring(t + 1) - ring(t);
    int n0 = 0;                // TL: first key row of tile t (set after slot 2)
    bool dirty, masked;
    int e_cur = 0, e_dma = 0;  // TL: entries of tile t and of tile t + 3 (read before the barrier)
    if constexpr (TL) {
      e_cur = entry(t);
      e_dma = entry(t + 3);
      dirty = masked = false;
    } else {
      dirty = t == nd;
      if (__builtin_expect(dirty, 0)) nd = next_dirty(t);
      masked = false;  // (TL only: without tile lists the slow path masks by segment end)
    }

    // slot 0.  The K fragments it reads were loaded in slot 3 of the previous tile, long
    // done: one wait for all of them instead of one per matrix op.
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    s_slot(0, s0, true, [&](int i) __attribute__((always_inline)) {
      stage_at(1, s1, 8, NS, i);
      if (i < NS && i % (NS / (NLD / 2)) == 0) dma_load(t + 2, NLD / 2 + i / (NS / (NLD / 2)), toff_a);
    });
    check_block(1, s1, t - 1, n0_prev, dirty_prev, masked_prev);
    // slot 1
    rs[0][0] = rs[0][1] = 0.f;
    pv_slot(1, true, [&](int i) __attribute__((always_inline)) {
      if (i < NPV) {
        read_v(2 * i);
        read_v(2 * i + 1);
      }
      stage_at(0, s0, 0, NP, i);
    });
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[db][0] += step_v, voff[db][1] += step_v;
    // slot 2
    s_slot(1, s1, true, [&](int i) __attribute__((always_inline)) { stage_at(0, s0, 8, NS, i); });
    if constexpr (TL) {
      const int e = __builtin_amdgcn_readfirstlane(e_cur);
      n0 = e >> 1;
      masked = (e & 1) != 0;
      dirty = t == 0 || masked;
    }
    check_block(0, s0, t, n0, dirty, masked);

    WA_WAIT_VMCNT(NLD);  // tile t+1 has landed (tile t+2 may still be in flight) ...
    barrier();           // ... for every wave
    if constexpr (TL) toff_a = uint32_t(e_dma >> 1) * row_bytes;
    else toff_a = next_off(t + 3, toff_a);

    // slot 3 (after the last tile the K reads hit a buffer nobody uses)
    rs[1][0] = rs[1][1] = 0.f;
    pv_slot(0, true, [&](int i) __attribute__((always_inline)) {
      if (i < NPV) {
#pragma unroll
        for (int r = 0; r < 2 * KS / NPV; ++r) read_k(i * (2 * KS / NPV) + r);
        if (i % (NPV / (NLD / 2)) == 0) dma_load(t + 3, i / (NPV / (NLD / 2)), toff_a);
      }
      stage_at(1, s1, 0, NP, i);
    });
#pragma unroll
    for (int st = 0; st < KS; ++st) koff[st] += step_k;
    n0_prev = n0;
    dirty_prev = dirty;
    masked_prev = masked;
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // no DMA may still write this block's LDS at exit
  // block 1 of the last tile
  s_slot(0, s0, false, [&](int i) __attribute__((always_inline)) { stage_at(1, s1, 8, NS, i); });
  check_block(1, s1, nt - 1, n0_prev, dirty_prev, masked_prev);
  pv_slot(1, true, [&](int) __attribute__((always_inline)) {});
#undef WA_WAIT_VMCNT

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) output_block(qb, row0 + 32 * qb);
  };  // run_item

  for (int n = 0;; ++n) {
    // The barrier also orders this block's LDS use: every wave has finished the previous
    // unit (its DMA drained, its reads done) before the next unit's prologue refills the ring.
    // Without queues (few units) block b runs the one unit at its place in the launch order.
    if (wave == 0) {
      const int u = p.persistent ? fetch_unit(p.work, p.counters, p.per_xcd, xcd, lane)
                                 : (n == 0 ? p.work[xcd * p.per_xcd + int(blockIdx.x) / kXcds] : -1);
      if (lane == 0) s_unit = u;
    }
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(s_unit);
    if (unit < 0) break;
    run_item(unit);
  }
  if (p.persistent && tid == 0) finish_persistent(p.counters);  // the last block resets the queues
}

// Merge the global leg's key splits: for each (global row, head), with m_s in log2 units,
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.  A thread merges four
// columns of one (row, head) with 16-byte loads; the D / 4 threads of a (row, head) read
// each split's partial row as one contiguous piece, and the (row, head) slots of a block are
// adjacent in every split.
constexpr int kCombineThreads = 256;
template <int D, bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  void* __restrict__ out, int G, int H, int n_splits,
                                                                  int frame_rows) {
  constexpr int TPS = D / 4;                     // threads per (row, head)
  constexpr int SPB = kCombineThreads / TPS;     // (row, head) slots per block
  const int64_t slot = int64_t(blockIdx.x) * SPB + threadIdx.x / TPS;  // = global row * H + head
  const int64_t stride = int64_t(G) * H;         // slots per split
  if (slot >= stride) return;
  const int c4 = (threadIdx.x % TPS) * 4;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = __builtin_fmaxf(M, part_ml[(s * stride + slot) * 2]);
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < n_splits; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + (s * stride + slot) * 2);
    const float w = fast_exp2(ml.x - M);
    den += w * ml.y;
    const f32x4 o = *reinterpret_cast<const f32x4*>(part_o + (s * stride + slot) * D + c4);
    num += w * o;
  }
  const float inv = 1.f / den;
  const f32x4 r = num * inv;
  const int64_t orow = (int64_t(frame_rows) * H + slot) * D + c4;  // row frame_rows + slot / H, head slot % H
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow) = r;
  } else {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + orow) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                          int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const f32x4 x = reinterpret_cast<const f32x4*>(src)[i];
    const u32x2 y = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    reinterpret_cast<u32x2*>(dst)[i] = y;
  }
}

template <int D, bool OUT_F32, bool TL>
hipError_t launch_typed(const ForwardArgs& a, hipStream_t stream) {
  std::conditional_t<TL, AttnParamsTL, AttnParams> p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = a.out;
  p.items = a.items;
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.H = a.H;
  p.G = a.G;
  p.frame_rows = a.frame_rows;
  p.n_items = a.n_items;
  p.work = a.work;
  p.counters = a.counters;
  p.persistent = a.persistent;
  p.per_xcd = a.work_per_xcd;
  p.total = kXcds * a.work_per_xcd;
  p.scale_log2 = a.scale_log2;
  p.tensor_bytes = uint32_t(a.L) * uint32_t(a.H) * uint32_t(D * 2);
  if constexpr (TL) {
    p.tiles = a.tiles;
    p.T = a.T;
    p.S = a.S;
    p.K = a.K;
    p.radius = a.radius;
    p.n_chunks = a.n_chunks;
  }
  const int grid = a.grid;
  hipLaunchKernelGGL((attn_kernel<D, OUT_F32, TL>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_splits > 1) {
    constexpr int spb = kCombineThreads / (D / 4);
    hipLaunchKernelGGL((combine_kernel<D, OUT_F32>), dim3((a.G * a.H + spb - 1) / spb), dim3(kCombineThreads), 0,
                       stream, a.part_o, a.part_ml, a.out, a.G, a.H, a.n_splits, a.frame_rows);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
  if (a.block_m != kNW * kWaveRows) return hipErrorInvalidValue;
  if (a.tile_list) {
    if (a.d == 128)
      return a.out_f32 ? launch_typed<128, true, true>(a, stream) : launch_typed<128, false, true>(a, stream);
    if (a.d == 64) return a.out_f32 ? launch_typed<64, true, true>(a, stream) : launch_typed<64, false, true>(a, stream);
    return hipErrorInvalidValue;
  }
  if (a.d == 128)
    return a.out_f32 ? launch_typed<128, true, false>(a, stream) : launch_typed<128, false, false>(a, stream);
  if (a.d == 64) return a.out_f32 ? launch_typed<64, true, false>(a, stream) : launch_typed<64, false, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_f32_to_bf16(const float* src, void* dst, int64_t n, hipStream_t stream) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src,
                     static_cast<uint16_t*>(dst), n4);
  return hipGetLastError();
}

}  // namespace wa

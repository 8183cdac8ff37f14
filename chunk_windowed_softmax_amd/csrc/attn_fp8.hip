// FP8 (e4m3) variant of the decomposed window attention (gfx950).
//
// Same work items and output contract as attn_kernel (window items over their chunk span and
// the global rows; global-leg items write fp32 partials that a combine pass merges), with q,
// k and v given as OCP e4m3 codes plus one fp32 scale per tensor (value = code * scale).  The
// lqnn.cn article's fastest H3 configurations run in FP8 (§四); it does not say which
// operands of the attention do, so both products run on gfx950's fp8 matrix cores here:
//   S^T = K Q^T      v_mfma_f32_32x32x64_f8f6f4, A = K rows from LDS, B = the wave's Q rows
//                    held in registers; the head dimension (128) is two k-steps of 64;
//   O^T += V^T P^T   same instruction, once per 64-key half of a tile: B = P^T rounded to
//                    e4m3 straight from the S^T accumulators, A = V^T gathered from the
//                    row-major V tile with ds_read_b64_tr_b8 (LDS transpose read), in the
//                    key order of P.
// Both operands of one matrix op map lane half h, byte j to the same k index, so any
// consistent key (or channel) order is correct; the order used makes P's bytes the S^T
// accumulator elements in register order.
// Softmax: online over the tiles in the log2 domain with a lazily raised running max (the
// weights may reach 2^8 before it rises; see the loop); the row sum adds the fp32 weights.
// Output: O * scale_v / rowsum, rounded to bf16.
//
// Block = 4 waves of 32 query rows, half of one of the plan's 256-row items; two blocks per
// CU (two waves per SIMD from different blocks, whose phases drift apart: 2.4% faster than
// one 8-wave block per item).  Blocks follow the plan's XCD-aware launch order, the two
// halves of an item on one XCD.  K/V tiles of 128 keys (16 KB each) are double-buffered in
// LDS and filled by direct global->LDS loads issued at the start of the previous tile; one
// barrier per tile (128-key tiles: 11% faster than 64-key ones, whose barriers came twice as
// often).
// Rows are stored with their 16-byte chunks swizzled by row, so that the K fragment reads
// and the V transpose reads are free of bank conflicts.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace wa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;             // head size = bytes per fp8 row
constexpr int kBN = 2 * kBlockN;    // keys per tile
constexpr int kWaves = 4;           // waves per block (two blocks per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per block
constexpr int kHalves = kBlockM / kRows;  // blocks per plan item
static_assert(kHalves * kRows == kBlockM, "blocks split a plan item evenly");
static_assert(kBN == 128, "a tile is two 64-key P^T operands");
constexpr int kTileB = kBN * kD;  // bytes of one K (or V) tile
constexpr int kBufB = 2 * kTileB;  // K then V

// s_waitcnt with vmcnt = 0 and the other counters left at their maximum.
constexpr int kVmcnt0 = 0x0F70;
// Word 3 of a raw buffer resource on gfx9 parts: 32-bit data format, no swizzle, so each
// access of a lane is range checked against num_records (word 2) and reads 0 past it.
constexpr int32_t kBufferWord3 = 0x00020000;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 16-byte chunk c of key row r sits at physical chunk c ^ swz(r) (rows of 128 bytes, two
// per 256-byte bank line).
//   K: swz = (r / 2) % 8, so the 16 consecutive rows of one ds_read_b128 pass at one logical
//      chunk cover all 64 banks.
//   V: swz = 2 * ((r / 2) % 2 + 2 * ((r / 8) % 2)).  One ds_read_b64_tr_b8 pass (32 lanes)
//      reads 8 rows {B..B+3, B+8..B+11} (B a multiple of 4 with bits 1 and 3 clear) at the 4
//      eight-byte pieces of two adjacent logical chunks; per row parity the 4 rows get 4
//      distinct chunk pairs, so the pass covers all 64 banks.
__device__ __forceinline__ int k_off(int r, int col) { return r * kD + (((col >> 4) ^ ((r >> 1) & 7)) << 4) + (col & 15); }
__device__ __forceinline__ int v_off(int r, int col) {
  const int sw = 2 * (((r >> 1) & 1) | ((r >> 2) & 2));
  return r * kD + (((col >> 4) ^ sw) << 4) + (col & 15);
}

// Key of byte j (0..31) of a P^T / V^T operand in lane half h: the S^T accumulator element
// j % 16 of key block j / 16, i.e. key (j/16)*32 + ((j%16)/4)*8 + 4h + j%4.
__device__ __forceinline__ int key_of(int h, int j) { return (j >> 4) * 32 + ((j & 15) >> 2) * 8 + 4 * h + (j & 3); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

__global__ __launch_bounds__(kThreads, 2) void attn_fp8_kernel(Fp8Args p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  // the plan's launch order: blocks are dispatched round-robin over the XCDs, and each XCD's
  // queue runs one group's query tiles side by side (they share its L2)
  const int slot = int(blockIdx.x / kXcdCount);
  const int unit = p.work[int(blockIdx.x % kXcdCount) * p.per_xcd + slot / kHalves];
  const int part = slot % kHalves;  // this block's rows of the item
  if (unit < 0) return;
  const int head = unit / p.n_items;
  const Item it = p.items[unit - head * p.n_items];
  const int H = p.H;
  const int64_t row_stride = int64_t(H) * kD;  // bytes between consecutive rows of q/k/v
  const bool causal = (it.flags & kItemCausal) != 0;

  const int nt0 = (it.kv0_end - it.kv0_begin + kBN - 1) / kBN;
  const int nt1 = it.kv1_end > it.kv1_begin ? (it.kv1_end - it.kv1_begin + kBN - 1) / kBN : 0;
  const int nt = nt0 + nt1;
  auto tile_range = [&](int t, int& n0, int& nend) {
    if (t < nt0) {
      n0 = it.kv0_begin + t * kBN;
      nend = it.kv0_end;
    } else {
      n0 = it.kv1_begin + (t - nt0) * kBN;
      nend = it.kv1_end;
    }
  };

  // K/V tiles go straight from global memory into LDS (buffer loads with the LDS bit: no
  // registers, no LDS write instructions).  One load moves 64 lanes x 16 bytes into 1 KB of
  // LDS (8 rows); wave w fills slices w, w + 4, w + 8 and w + 12 of the K and of the V
  // tile.  Lane l of slice s writes LDS chunk 64 s + l, i.e. row 8 s + l / 8 at physical
  // chunk l % 8, which holds the row's logical chunk (l % 8) ^ swizzle(row): the swizzle is
  // applied on the global side.  The buffer resources are based at this head's first byte and range checked
  // against the end of the tensor (rows past it read as zero).
  auto make_rsrc = [&](const void* t) __attribute__((always_inline)) -> i32x4 {
    const uint64_t a = reinterpret_cast<uint64_t>(t) + uint64_t(head) * kD;
    return i32x4{__builtin_amdgcn_readfirstlane(int32_t(uint32_t(a))),
                 __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(int32_t(uint32_t(int64_t(p.L) * row_stride - int64_t(head) * kD))),
                 kBufferWord3};
  };
  i32x4 rsrc_k = make_rsrc(p.k), rsrc_v = make_rsrc(p.v);
  // a buffer load may read an SGPR written by a vector instruction (the readfirstlane) only
  // 5 wait states later; the loads are inline asm, unseen by the compiler's hazard checks
  asm volatile("s_nop 4" : "+s"(rsrc_k), "+s"(rsrc_v));
  constexpr int kSl = kTileB / 1024 / kWaves;  // 1 KB slices of a tile per wave
  uint32_t dk[kSl], dv[kSl];  // byte offsets of the lane's 16 bytes within a tile
#pragma unroll
  for (int x = 0; x < kSl; ++x) {
    const int row = 8 * (wave + kWaves * x) + (lane >> 3);
    dk[x] = uint32_t(row) * uint32_t(row_stride) + uint32_t(((lane & 7) ^ ((row >> 1) & 7)) << 4);
    dv[x] = uint32_t(row) * uint32_t(row_stride) +
            uint32_t(((lane & 7) ^ (2 * (((row >> 1) & 1) | ((row >> 2) & 2)))) << 4);
  }
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)smem));
  auto dma_tile = [&](int t, int buf) __attribute__((always_inline)) {
    int n0, nend;
    tile_range(t, n0, nend);
    const uint32_t toff = uint32_t(n0) * uint32_t(row_stride);
#pragma unroll
    for (int x = 0; x < kSl; ++x) {
      const uint32_t lk = lds_base + uint32_t(buf * kBufB + (wave + kWaves * x) * 1024);
      const uint32_t lv = lk + kTileB;
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(dk[x] + toff), "s"(rsrc_k), "{m0}"(lk)
                   : "memory");
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(dv[x] + toff), "s"(rsrc_v), "{m0}"(lv)
                   : "memory");
    }
  };

  dma_tile(0, 0);

  // Q fragments: lane = query row, bytes [64 s + 32 hh, +32) of the row for k-step s
  const int wrow0 = it.q_begin + part * kRows + wave * 32;  // the wave's first row
  const int qrow = wrow0 + l32;
  const bool q_ok = qrow < it.q_end;
  i32x8 qf[2];
  {
    const unsigned char* qg = static_cast<const unsigned char*>(p.q) + int64_t(qrow) * row_stride + int64_t(head) * kD;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (q_ok) {
        a = *reinterpret_cast<const u32x4*>(qg + 64 * s + 32 * hh);
        b = *reinterpret_cast<const u32x4*>(qg + 64 * s + 32 * hh + 16);
      }
      qf[s] = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // tile 0 (and Q) have landed ...
  __syncthreads();                       // ... for every wave

  // V^T gather: transpose read m of lane (group g = lane / 16, index i = lane % 16) names
  // key row key_of(hh, 8m + i/2) at column 16 (g & 1) + 8 (i & 1) of the d-block; the
  // instruction hands lane i byte i % 8 of the rows named by lanes 2j + i / 8, j = 0..7.
  const int gi = lane & 15, gsel = (lane >> 4) & 1;
  int vrow[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) vrow[m] = key_of(hh, 8 * m + (gi >> 1));
  const int vcol = 16 * gsel + 8 * (gi & 1);

  const float c = p.scale_log2;  // log2(e) / sqrt(d) * scale_q * scale_k
  float m_run = -__builtin_inff(), l_run = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) dma_tile(t + 1, buf ^ 1);
    const unsigned char* kb = smem + buf * kBufB;
    const unsigned char* vb = kb + kTileB;
    int n0, nend;
    tile_range(t, n0, nend);
    const int valid = nend - n0;

    // S^T for the four 32-key blocks of the tile
    f32x16 sa[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      sa[b] = f32x16{};
      const int r = 32 * b + l32;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kb + k_off(r, 64 * s + 32 * hh));
        const u32x4 a2 = *reinterpret_cast<const u32x4*>(kb + k_off(r, 64 * s + 32 * hh + 16));
        const i32x8 kf = {int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(a2[0]), int(a2[1]), int(a2[2]), int(a2[3])};
        sa[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[s], sa[b], 0, 0, 0, 0, 0, 0);
      }
    }
    // mask keys past the segment end (and, for causal items, after the lane's own row)
    const bool need_mask = valid < kBN || (causal && n0 + kBN - 1 > wrow0);
    if (need_mask) {
      int lim = valid;
      if (causal) lim = __builtin_elementwise_min(lim, qrow - n0 + 1);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * b + (i >> 2) * 8 + 4 * hh + (i & 3) >= lim) sa[b][i] = -__builtin_inff();
    }
    // P = 2^(S c - m) against the running max m as it stands (lazy max): the weights may
    // reach 2^8 (exact in e4m3, whose largest value is 448) before m must rise.  A tile
    // whose row sum exceeds 2^8 (so possibly some weight too), and the first tile, take the
    // wave-uniform slow path: tile max, raise m, rescale, recompute P.  Byte j of the P^T
    // operand is element j % 16 of key block j / 16.
    i32x8 pb[2];  // keys 0..63 and 64..127 of the tile
    float l_tile = 0.f;
    auto weights = [&](float mneg) __attribute__((always_inline)) {
      l_tile = 0.f;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int b = w >> 2, e = 4 * (w & 3);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][e], c, mneg));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][e + 1], c, mneg));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][e + 2], c, mneg));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][e + 3], c, mneg));
        l_tile += (p0 + p1) + (p2 + p3);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
        pb[w >> 3][w & 7] = x;
      }
    };
    bool slow = t == 0;
    if (!slow) {
      weights(-m_run);
      slow = __builtin_amdgcn_ballot_w64(l_tile > 256.f) != 0;
    }
    if (slow) {
      // tile max (log2 units); lanes l and l ^ 32 hold the two halves of one query's keys
      float mt = sa[0][0];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, sa[b][i]);
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mt), __builtin_bit_cast(uint32_t, mt),
                                                      false, false);
      mt = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
      // Per row: the max rises only where the tile's weights could exceed 2^8 against it
      // (and on the first tile), so a row's weights never depend on the other rows' scores.
      const float m_new = mt * c > m_run + 8.f ? mt * c : m_run;
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      m_run = m_new;
      weights(-m_run);
    }
    l_run += l_tile;
    // O^T += V^T P^T per 32-row d-block
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        i32x8 vf;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2*)(vb + v_off(vrow[m] + 64 * hf, 32 * db + vcol)));
          vf[2 * m] = x[0];
          vf[2 * m + 1] = x[1];
        }
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pb[hf], oacc[db], 0, 0, 0, 0, 0, 0);
      }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // tile t + 1 has landed ...
    __syncthreads();                       // ... for every wave
  }

  // ---- output: lane holds O^T[d][query] for d = 32 db + 8 (i / 4) + 4 hh + i % 4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_ok) return;
  if (it.split < 0) {
    const float mul = p.scale_v / l_tot;
    uint16_t* o = static_cast<uint16_t*>(p.out) + (int64_t(qrow) * H + head) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * db + 8 * r + 4 * hh;
        const u32x2 y = {pack_bf16x2(oacc[db][4 * r] * mul, oacc[db][4 * r + 1] * mul),
                         pack_bf16x2(oacc[db][4 * r + 2] * mul, oacc[db][4 * r + 3] * mul)};
        *reinterpret_cast<u32x2*>(o + d0) = y;
      }
  } else {
    const int64_t slot = (int64_t(it.split) * p.G + (qrow - p.frame_rows)) * H + head;
    float* po = p.part_o + slot * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = 32 * db + 8 * r + 4 * hh;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(oacc[db][4 * r] * p.scale_v, oacc[db][4 * r + 1] * p.scale_v,
                        oacc[db][4 * r + 2] * p.scale_v, oacc[db][4 * r + 3] * p.scale_v);
      }
    if (hh == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run, l_tot);
  }
}

// Merge of the global leg's key splits (as for the bf16 path): for each (global row, head),
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s, in bf16.  A thread
// merges four columns of one (row, head) with 16-byte loads; the 32 threads of a (row, head)
// read each split's partial row as one contiguous piece.
constexpr int kCombineThreads = 256;
constexpr int kCombineSlots = kCombineThreads / (kD / 4);  // (row, head) slots per block
__global__ __launch_bounds__(kCombineThreads) void combine_fp8_kernel(const float* __restrict__ part_o,
                                                                      const float* __restrict__ part_ml,
                                                                      uint16_t* __restrict__ out, int G, int H,
                                                                      int n_splits, int frame_rows) {
  const int64_t stride = int64_t(G) * H;  // slots per split
  const int64_t slot = int64_t(blockIdx.x) * kCombineSlots + threadIdx.x / (kD / 4);  // global row * H + head
  if (slot >= stride) return;
  const int c4 = (threadIdx.x % (kD / 4)) * 4;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = __builtin_fmaxf(M, part_ml[(s * stride + slot) * 2]);
  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
  for (int s = 0; s < n_splits; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + (s * stride + slot) * 2);
    const float w = __builtin_amdgcn_exp2f(ml.x - M);
    den += w * ml.y;
    const float4 o = *reinterpret_cast<const float4*>(part_o + (s * stride + slot) * kD + c4);
    num.x += w * o.x;
    num.y += w * o.y;
    num.z += w * o.z;
    num.w += w * o.w;
  }
  const float inv = 1.f / den;
  const int64_t orow = (int64_t(frame_rows) * H + slot) * kD + c4;  // row frame_rows + slot / H, head slot % H
  const __bf16 b0 = (__bf16)(num.x * inv), b1 = (__bf16)(num.y * inv), b2 = (__bf16)(num.z * inv),
               b3 = (__bf16)(num.w * inv);
  const uint32_t lo = uint32_t(__builtin_bit_cast(uint16_t, b0)) | (uint32_t(__builtin_bit_cast(uint16_t, b1)) << 16);
  const uint32_t hi = uint32_t(__builtin_bit_cast(uint16_t, b2)) | (uint32_t(__builtin_bit_cast(uint16_t, b3)) << 16);
  *reinterpret_cast<uint2*>(out + orow) = make_uint2(lo, hi);
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  const int grid = kXcdCount * a.per_xcd * kHalves;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3(grid), dim3(kThreads), 2 * kBufB, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits <= 1) return e;
  hipLaunchKernelGGL(combine_fp8_kernel, dim3((a.G * a.H + kCombineSlots - 1) / kCombineSlots), dim3(kCombineThreads),
                     0, stream, a.part_o, a.part_ml, static_cast<uint16_t*>(a.out), a.G, a.H, a.n_splits,
                     a.frame_rows);
  return hipGetLastError();
}

}  // namespace wa

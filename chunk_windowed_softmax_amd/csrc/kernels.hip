// HIP kernels of the decomposed chunk-windowed softmax attention, written for gfx950.
//
// Method: lqnn.cn article on VDN-Minimax-H3 window attention.  §一 defines the window
// (whole chunks within +-radius, global tokens fully connected); §三 replaces the masked
// attention by plain dense attentions over row groups with identical kept-KV sets, plus
// the global rows, scattered into one contiguous output.
//
// Kernels
//   attn_kernel     one work item = (block of up to 128 or 256 query rows, head, <= 2
//                   key segments).  Both legs run in the same launch: window items read
//                   their chunk span and then the global rows in place (no gathered
//                   copy); global-leg items read one key split and write fp32 partials.
//   combine_kernel  log-sum-exp merge of the global leg's key splits into the output.
//   f32_to_bf16     staging of fp32 inputs into bf16 for the matrix products.
//
// Attention mainloop (per wave: 32 query rows, all heads' rows are [L, H, d]):
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K tile rows (keys) from LDS, B = the
//   wave's Q rows held in registers.  In the accumulator layout each lane then holds 16
//   keys of ONE query per 32-key block, so the row max / row sum are in-lane reductions
//   plus a single exchange with the lane 32 apart.
//   O^T += V^T P^T on the same instruction: B = P^T straight from the S^T accumulators
//   (rounded to bf16), A = V^T read from the row-major V tile with ds_read_tr16_b64
//   (LDS transpose read), so V needs no transposed copy anywhere.
//   Softmax runs in the log2 domain (exp2 with log2(e)/sqrt(d) folded into one FMA),
//   online over 64-key tiles with fp32 running max / sum / accumulators.
//   K/V tiles are double-buffered in LDS and filled by direct global->LDS 16-byte loads
//   (no registers, no LDS write instructions): the next tile's loads are issued before
//   the current tile's math, one barrier per tile.  LDS rows hold d bf16; 16-byte chunks
//   are XOR-swizzled per row (applied on the global side of the DMA) so the K reads and
//   the transpose reads are free of bank conflicts.
//   The running max is raised lazily: the accumulators are rescaled only when some
//   row's max grows by more than 2^8 (wave-uniform branch), otherwise exponentials are
//   taken against the stale max (values up to 2^8, exact in the softmax ratio).
//   Blocks are remapped so that consecutive work items (same head, same group, adjacent
//   query tiles sharing all their keys) land on the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include <cstdint>

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

constexpr int kWaveRows = 32;  // query rows per wave
constexpr int kBN = kBlockN;   // keys per tile
static_assert(kBN == 64, "the fragment code below assumes 64-key tiles");

constexpr int kXcds = 8;  // MI355X: blocks are dispatched round-robin over 8 XCDs

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

// s_waitcnt with vmcnt = 0 and the other counters left at their maximum.
constexpr int kVmcnt0 = 0x0F70;

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
  float* __restrict__ part_o;
  float* __restrict__ part_ml;
  int H, G, frame_rows, n_items, total, per_xcd;
  float scale_log2;
};

template <int D, int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnParams p) {
  constexpr int NT = NW * 64;                   // threads per block
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int ROWB = D * 2;                   // bytes per LDS row
  constexpr int TILEB = kBN * ROWB;             // bytes per K or V tile
  constexpr int NJ = TILEB / 1024;              // 1 KB DMA slices (one wave instruction) per tile
  constexpr int JPW = NJ / NW;                  // slices per wave per tensor per tile
  constexpr int KS = D / 16;                    // MFMA k-steps over d
  constexpr int DB = D / 32;                    // 32-wide output column blocks
  static_assert(NJ % NW == 0, "tile slices must divide evenly over the waves");
  constexpr float kLazyLog2 = 8.f;              // rescale only when the max grows by > 2^8

  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * TILEB];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;     // half of the wave: k sub-block of the MFMA operands
  const int l32 = lane & 31;

  const int bid = blockIdx.x;
  const int logical = (bid % kXcds) * p.per_xcd + bid / kXcds;
  if (logical >= p.total) return;
  const int h = logical / p.n_items;
  const Item it = p.items[logical - h * p.n_items];
  const int H = p.H;
  const uint32_t row_bytes = uint32_t(H) * D * 2;  // bytes between consecutive rows of q/k/v

  // ---- Q fragments of this wave (B operand of S^T = K Q^T): lane = query row, 8 d each
  const int qrow = it.q_begin + wave * kWaveRows + l32;
  const bool wave_active = it.q_begin + wave * kWaveRows < it.q_end;
  bf16x8 qf[KS];
  {
    const bool ok = qrow < it.q_end;
    const uint16_t* src = p.q + ((int64_t)qrow * H + h) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *reinterpret_cast<const u32x4*>(src + 16 * s);
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- DMA source offsets: LDS slice j holds tile rows [j*1024/ROWB, ...); lane writes LDS
  // chunk (j*64 + lane), i.e. row m/CH, physical chunk m%CH, which holds the logical chunk
  // (physical ^ swz(row)) of that key row.
  uint32_t dma_off[JPW];
  int dma_row[JPW];
#pragma unroll
  for (int i = 0; i < JPW; ++i) {
    const int j = i * NW + wave;
    const int m = j * 64 + lane;
    const int row = m / CH, phys = m % CH;
    dma_row[i] = row;
    dma_off[i] = uint32_t(row) * row_bytes + uint32_t(h * D * 2) + uint32_t(((phys ^ swz<D>(row)) * 8) * 2);
  }

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

  // ---- tile schedule: segment 0 then segment 1, 64 keys per tile
  const int nt0 = (it.kv0_end - it.kv0_begin + kBN - 1) / kBN;
  const int nt1 = (it.kv1_end - it.kv1_begin + kBN - 1) / kBN;
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

  // Issue the DMA of tile t into buffer `buf`.  Rows past the segment end re-read the
  // segment's last row (finite data, masked out of the softmax), so no key outside the
  // item's kept set is ever read.
  auto issue_tile = [&](int t, int buf) {
    int n0, nend;
    tile_range(t, n0, nend);
    const unsigned char* kg = reinterpret_cast<const unsigned char*>(p.k) + (int64_t)n0 * row_bytes;
    const unsigned char* vg = reinterpret_cast<const unsigned char*>(p.v) + (int64_t)n0 * row_bytes;
    unsigned char* kl = smem + (2 * buf) * TILEB;
    unsigned char* vl = kl + TILEB;
    const int last = nend - 1 - n0;
#pragma unroll
    for (int i = 0; i < JPW; ++i) {
      const int j = i * NW + wave;
      uint32_t off = dma_off[i];
      if (last < kBN - 1 && dma_row[i] > last) off -= uint32_t(dma_row[i] - last) * row_bytes;
      __builtin_amdgcn_global_load_lds(kg + off, (lds_void*)(kl + j * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vg + off, (lds_void*)(vl + j * 1024), 16, 0, 0);
    }
  };

  float m_run = -__builtin_inff();  // running max of raw scores (this lane's query)
  float mc = 0.f;                   // m_run * c2
  float l_run0 = 0.f, l_run1 = 0.f;  // this lane's half of the running sum (two chains)
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const float c2 = p.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;

  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int cur = t & 1;
    if (t + 1 < nt) issue_tile(t + 1, cur ^ 1);

    if (wave_active) {
      const unsigned char* kb = smem + (2 * cur) * TILEB;
      const unsigned char* vb = kb + TILEB;

      // S^T[key][query] for the two 32-key blocks of the tile
      f32x16 sacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(kb + koff[s] + b * 32 * ROWB);
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), qf[s], sacc[b], 0, 0, 0);
        }

      // mask keys past the segment end (only the last tile of a segment)
      int n0, nend;
      tile_range(t, n0, nend);
      const int valid = nend - n0;
      if (valid < kBN) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = b * 32 + (i >> 2) * 8 + 4 * hh + (i & 3);
            if (key >= valid) sacc[b][i] = -__builtin_inff();
          }
      }

      // online softmax (log2 domain) with lazy rescaling
      float mt = sacc[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, sacc[b][i]);
      mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
      if (__builtin_amdgcn_ballot_w64(mt > m_run + lazy_raw) != 0) {
        const float m_new = __builtin_fmaxf(m_run, mt);
        const float alpha = fast_exp2((m_run - m_new) * c2);
        m_run = m_new;
        mc = m_new * c2;
        l_run0 *= alpha;
        l_run1 *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b][i] = fast_exp2(__builtin_fmaf(sacc[b][i], c2, -mc));

      // O^T += V^T P^T.  P is rounded to bf16 for the product, and the row sum adds up
      // exactly those rounded values (v_dot2 with (1, 1)), so the weights applied to V sum
      // to one and a row dominated by one key reproduces that key's value.
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const bf16x2 p0 = cvt_bf16x2(sacc[b][8 * tt + 0], sacc[b][8 * tt + 1]);
          const bf16x2 p1 = cvt_bf16x2(sacc[b][8 * tt + 2], sacc[b][8 * tt + 3]);
          const bf16x2 p2 = cvt_bf16x2(sacc[b][8 * tt + 4], sacc[b][8 * tt + 5]);
          const bf16x2 p3 = cvt_bf16x2(sacc[b][8 * tt + 6], sacc[b][8 * tt + 7]);
          l_run0 = __builtin_amdgcn_fdot2_f32_bf16(p0, kOnes2, l_run0, false);
          l_run1 = __builtin_amdgcn_fdot2_f32_bf16(p1, kOnes2, l_run1, false);
          l_run0 = __builtin_amdgcn_fdot2_f32_bf16(p2, kOnes2, l_run0, false);
          l_run1 = __builtin_amdgcn_fdot2_f32_bf16(p3, kOnes2, l_run1, false);
          const bf16x8 pf = __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                                    __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
          const unsigned char* vt = vb + (32 * b + 16 * tt) * ROWB;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db][0]));
            const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vt + voff[db][1]));
            const u32x4 vw = {__builtin_bit_cast(u32x2, r0)[0], __builtin_bit_cast(u32x2, r0)[1],
                              __builtin_bit_cast(u32x2, r1)[0], __builtin_bit_cast(u32x2, r1)[1]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf, oacc[db], 0, 0, 0);
          }
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the next tile's DMA has landed in LDS
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_run = l_run0 + l_run1;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow >= it.q_end) return;

  if (it.split < 0) {
    const float inv = 1.f / l_tot;
    if constexpr (OUT_F32) {
      float* orow = reinterpret_cast<float*>(p.out) + ((int64_t)qrow * H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dv = 32 * db + 8 * g4 + 4 * hh;
          const f32x4 o = {oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv, oacc[db][4 * g4 + 2] * inv,
                           oacc[db][4 * g4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + dv) = o;
        }
    } else {
      uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)qrow * H + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dv = 32 * db + 8 * g4 + 4 * hh;
          const u32x2 o = {pack_bf16x2(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv),
                           pack_bf16x2(oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + dv) = o;
        }
    }
  } else {
    const int64_t slot = ((int64_t)it.split * p.G + (qrow - p.frame_rows)) * H + h;
    float* po = p.part_o + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = 32 * db + 8 * g4 + 4 * hh;
        const f32x4 o = {oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]};
        *reinterpret_cast<f32x4*>(po + dv) = o;
      }
    if (hh == 0) {
      const float2 ml = make_float2(m_run * c2, l_tot);
      *reinterpret_cast<float2*>(p.part_ml + slot * 2) = ml;
    }
  }
}

// Merge the global leg's key splits: for each (global row, head), with m_s in log2 units,
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ part_o,
                                                     const float* __restrict__ part_ml, void* __restrict__ out,
                                                     int G, int H, int n_splits, int frame_rows) {
  const int gi = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t stride = (int64_t)G * H;  // slots per split
  const int64_t slot0 = (int64_t)gi * H + h;
  float M = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) M = __builtin_fmaxf(M, part_ml[(s * stride + slot0) * 2]);
  float den = 0.f;
  for (int s = 0; s < n_splits; ++s) {
    const float* ml = part_ml + (s * stride + slot0) * 2;
    den += fast_exp2(ml[0] - M) * ml[1];
  }
  const float inv = 1.f / den;
  const int64_t orow = ((int64_t)(frame_rows + gi) * H + h) * D;
  for (int dv = threadIdx.x; dv < D; dv += 64) {
    float num = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float w = fast_exp2(part_ml[(s * stride + slot0) * 2] - M);
      num += w * part_o[(s * stride + slot0) * D + dv];
    }
    const float o = num * inv;
    if constexpr (OUT_F32) {
      reinterpret_cast<float*>(out)[orow + dv] = o;
    } else {
      const __bf16 b = (__bf16)o;
      reinterpret_cast<uint16_t*>(out)[orow + dv] = __builtin_bit_cast(uint16_t, b);
    }
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

template <int D, int NW, bool OUT_F32>
hipError_t launch_typed(const ForwardArgs& a, hipStream_t stream) {
  AttnParams p;
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
  p.total = a.n_items * a.H;
  p.per_xcd = (p.total + kXcds - 1) / kXcds;
  p.scale_log2 = a.scale_log2;
  const int grid = p.per_xcd * kXcds;
  hipLaunchKernelGGL((attn_kernel<D, NW, OUT_F32>), dim3(grid), dim3(NW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_splits > 1) {
    hipLaunchKernelGGL((combine_kernel<D, OUT_F32>), dim3(a.G * a.H), dim3(64), 0, stream, a.part_o, a.part_ml,
                       a.out, a.G, a.H, a.n_splits, a.frame_rows);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool OUT_F32>
hipError_t launch_rows(const ForwardArgs& a, hipStream_t stream) {
  switch (a.block_m) {
    case 128: return launch_typed<D, 4, OUT_F32>(a, stream);
    case 256: return launch_typed<D, 8, OUT_F32>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.out_f32 ? launch_rows<128, true>(a, stream) : launch_rows<128, false>(a, stream);
  if (a.d == 64) return a.out_f32 ? launch_rows<64, true>(a, stream) : launch_rows<64, false>(a, stream);
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

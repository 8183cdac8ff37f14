// HIP kernels of the decomposed chunk-windowed softmax attention, written for gfx950.
//
// Method: lqnn.cn article on VDN-Minimax-H3 window attention.  §一 defines the window
// (whole chunks within +-radius, global tokens fully connected); §三 replaces the masked
// attention by plain dense attentions over row groups with identical kept-KV sets, plus
// the global rows, scattered into one contiguous output.
//
// Kernels
//   attn_kernel     one work item = (block of up to 128 query rows, head, <= 2 key
//                   segments).  Both legs run in the same launch: window items read
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
//   K/V tiles are double-buffered in LDS; the next tile's global loads are issued
//   before the current tile's math and stored to LDS after it (one barrier per tile).
//   LDS rows hold d bf16; 16-byte chunks are XOR-swizzled per row so that both the
//   128-bit K reads (8 consecutive rows) and the transpose reads (two 4-row groups)
//   hit distinct banks.
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

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaveRows = 32;  // query rows per wave
constexpr int kBN = kBlockN;   // keys per tile
static_assert(kBlockM == 4 * kWaveRows, "block_m must be 4 waves x 32 rows");
static_assert(kBN == 64, "the fragment code below assumes 64-key tiles");

constexpr int kXcds = 8;  // MI355X: blocks are dispatched round-robin over 8 XCDs

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
  constexpr int CH = D / 8;                     // 16-byte chunks per row
  constexpr int ROWB = D * 2;                   // bytes per LDS row
  constexpr int TILEB = kBN * ROWB;             // bytes per K or V tile
  constexpr int LPT = kBN * CH / kThreads;      // 16-byte loads per thread per tensor per tile
  constexpr int KS = D / 16;                    // MFMA k-steps over d
  constexpr int DB = D / 32;                    // 32-wide output column blocks
  static_assert(LPT * kThreads == kBN * CH, "tile must divide evenly over the block");

  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * TILEB];  // K0 V0 K1 V1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;     // which half of the wave (k sub-block of MFMA operands)
  const int l32 = lane & 31;

  const int bid = blockIdx.x;
  const int logical = (bid % kXcds) * p.per_xcd + bid / kXcds;
  if (logical >= p.total) return;
  const int h = logical / p.n_items;
  const Item it = p.items[logical - h * p.n_items];
  const int H = p.H;

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

  u32x4 kreg[LPT], vreg[LPT];
  auto gload = [&](int t) {
    int n0, nend;
    tile_range(t, n0, nend);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + kThreads * i;
      const int row = e / CH, c = e % CH;
      const int key = n0 + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < nend) {
        const int64_t off = ((int64_t)key * H + h) * D + c * 8;
        a = *reinterpret_cast<const u32x4*>(p.k + off);
        b = *reinterpret_cast<const u32x4*>(p.v + off);
      }
      kreg[i] = a;
      vreg[i] = b;
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* kb = smem + (2 * buf) * TILEB;
    unsigned char* vb = kb + TILEB;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + kThreads * i;
      const int row = e / CH, c = e % CH;
      const int off = row * ROWB + ((c ^ swz(row)) << 4);
      *reinterpret_cast<u32x4*>(kb + off) = kreg[i];
      *reinterpret_cast<u32x4*>(vb + off) = vreg[i];
    }
  };

  float m_run = -__builtin_inff();  // running max of raw scores (this lane's query)
  float l_run = 0.f;                // this lane's half of the running sum
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const float c2 = p.scale_log2;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int cur = t & 1;
    const bool has_next = t + 1 < nt;
    if (has_next) gload(t + 1);

    if (wave_active) {
      const unsigned char* kb = smem + (2 * cur) * TILEB;
      const unsigned char* vb = kb + TILEB;

      // S^T[key][query] for the two 32-key blocks of the tile
      f32x16 sacc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[b][i] = 0.f;
        const int row = b * 32 + l32;
        const unsigned char* rbase = kb + row * ROWB;
        const int sw = swz(row);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int c = 2 * s + hh;
          const u32x4 x = *reinterpret_cast<const u32x4*>(rbase + ((c ^ sw) << 4));
          sacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), qf[s], sacc[b], 0, 0, 0);
        }
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

      // online softmax (log2 domain)
      float mt = sacc[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, sacc[b][i]);
      mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = __builtin_fmaxf(m_run, mt);
      const float mc = m_new * c2;
      const float alpha = fast_exp2(m_run * c2 - mc);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fast_exp2(__builtin_fmaf(sacc[b][i], c2, -mc));
          sacc[b][i] = e;
          l_run += e;
        }

      // O^T += V^T P^T
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 pw;
          pw[0] = pack_bf16x2(sacc[b][8 * tt + 0], sacc[b][8 * tt + 1]);
          pw[1] = pack_bf16x2(sacc[b][8 * tt + 2], sacc[b][8 * tt + 3]);
          pw[2] = pack_bf16x2(sacc[b][8 * tt + 4], sacc[b][8 * tt + 5]);
          pw[3] = pack_bf16x2(sacc[b][8 * tt + 6], sacc[b][8 * tt + 7]);
          const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
          const int pl = lane & 15;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (pl & 3);
            const int cidx = col >> 3, half = (col >> 2) & 1;
            i16x4 r[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int row = b * 32 + 16 * tt + 8 * rr + 4 * hh + (pl >> 2);
              const unsigned char* a = vb + row * ROWB + ((cidx ^ swz(row)) << 4) + (half << 3);
              r[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
            }
            const u32x4 vw = {__builtin_bit_cast(u32x2, r[0])[0], __builtin_bit_cast(u32x2, r[0])[1],
                              __builtin_bit_cast(u32x2, r[1])[0], __builtin_bit_cast(u32x2, r[1])[1]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vw), pf, oacc[db], 0, 0, 0);
          }
        }
      }
    }

    if (has_next) lstore(cur ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;
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

template <int D, bool OUT_F32>
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
  hipLaunchKernelGGL((attn_kernel<D, OUT_F32>), dim3(grid), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_splits > 1) {
    hipLaunchKernelGGL((combine_kernel<D, OUT_F32>), dim3(a.G * a.H), dim3(64), 0, stream, a.part_o, a.part_ml,
                       a.out, a.G, a.H, a.n_splits, a.frame_rows);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.out_f32 ? launch_typed<128, true>(a, stream) : launch_typed<128, false>(a, stream);
  return a.out_f32 ? launch_typed<64, true>(a, stream) : launch_typed<64, false>(a, stream);
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

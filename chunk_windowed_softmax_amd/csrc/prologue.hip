// QK-RMSNorm + rotary embedding of q and k, out of place, in one pass (gfx950).
//
// The step before the attention: the ViT attention of the prhub digest of sglang PR
// #34949 passes q and k through qk_norm (an RMSNorm, with or without a weight) and the
// rotary position embedding before attending, and sglang PR #43164 (Modifications, item 2)
// fuses that norm and RoPE into one out-of-place kernel that writes the attention's input.
//
// For every row t, head h and tensor x in {q, k} (weight w = wq or wk, or 1):
//   y = x[t,h,:] / sqrt(mean(x[t,h,:]^2) + eps) * w
//   pair j (j < d/2) of y, (j, j + d/2) or, interleaved, (2j, 2j + 1), is rotated by the
//   row's angle: (a, b) -> (a cos[t,j] - b sin[t,j], b cos[t,j] + a sin[t,j]).
//
// Memory bound: each element is read and written once, the angle tables and weights once
// per thread.  A group of lanes owns one row: each lane owns EPL channel pairs (16 bytes of
// first members and 16 bytes of second members per vector), holds the row's cos / sin of
// those pairs and the weights in registers, and walks the row's 2H (tensor, head) vectors,
// loading several vectors ahead of their use.  Both members of every pair sit in the same lane, so the
// rotation needs no exchange and the mean square one reduction over the group.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace wa {
namespace {

// 16-byte load / store of EPL elements, widened to fp32.  Every element is touched once, so
// the accesses are non-temporal (streamed past the caches): measured 7% faster at the H3
// shape than cached ones.
template <bool F32>
struct Io;
template <>
struct Io<false> {
  static constexpr int EPL = 8;
  typedef __bf16 raw __attribute__((ext_vector_type(8)));
  typedef float f32v __attribute__((ext_vector_type(8)));
  static __device__ __forceinline__ raw load(const void* base, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw*>(static_cast<const __bf16*>(base) + i));
  }
  static __device__ __forceinline__ f32v widen(raw x) { return __builtin_convertvector(x, f32v); }
  static __device__ __forceinline__ void store(void* base, int64_t i, f32v v) {
    __builtin_nontemporal_store(__builtin_convertvector(v, raw), reinterpret_cast<raw*>(static_cast<__bf16*>(base) + i));
  }
};
template <>
struct Io<true> {
  static constexpr int EPL = 4;
  typedef float raw __attribute__((ext_vector_type(4)));
  typedef float f32v __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ raw load(const void* base, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw*>(static_cast<const float*>(base) + i));
  }
  static __device__ __forceinline__ f32v widen(raw x) { return x; }
  static __device__ __forceinline__ void store(void* base, int64_t i, f32v v) {
    __builtin_nontemporal_store(v, reinterpret_cast<raw*>(static_cast<float*>(base) + i));
  }
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kAhead = 4;  // vectors loaded before the first of them is used

template <int D, bool F32, bool INTERLEAVED>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                                void* q_out, void* k_out,
                                                                const float* __restrict__ cosv,
                                                                const float* __restrict__ sinv,
                                                                const float* __restrict__ wq,
                                                                const float* __restrict__ wk, int L, int H, float eps) {
  using IO = Io<F32>;
  using V = typename IO::f32v;
  constexpr int EPL = IO::EPL;           // pairs per lane
  constexpr int GL = D / 2 / EPL;        // lanes per row
  constexpr int RPB = kThreads / GL;     // rows per block
  const int g = threadIdx.x % GL;
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / GL;
  if (row >= L) return;  // whole lane groups leave together
  const int j0 = EPL * g;  // first pair of this lane
  // channel offsets of this lane's first members (a) and second members (b)
  const int ca = INTERLEAVED ? 2 * j0 : j0;
  const int cb = INTERLEAVED ? 2 * j0 + EPL : D / 2 + j0;  // interleaved: second 16-byte half
  V c, s;  // the row's angles of this lane's pairs (16-byte aligned: j0 is a multiple of 4)
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    const f32x4 c4 = *reinterpret_cast<const f32x4*>(cosv + row * (D / 2) + j0 + e);
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(sinv + row * (D / 2) + j0 + e);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      c[e + x] = c4[x];
      s[e + x] = s4[x];
    }
  }
  // weights of this lane's pairs, (first, second) member, for q and k; 1 when absent
  V w[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float* wt = t ? wk : wq;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int ea = INTERLEAVED ? 2 * (j0 + e) : j0 + e;
      const int eb = INTERLEAVED ? ea + 1 : D / 2 + j0 + e;
      w[t][0][e] = wt ? wt[ea] : 1.f;
      w[t][1][e] = wt ? wt[eb] : 1.f;
    }
  }
  const float inv_d = 1.f / float(D);
  const int nv = 2 * H;
  for (int v0 = 0; v0 < nv; v0 += kAhead) {
    typename IO::raw lo[kAhead], hi[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int v = v0 + u;
      if (v < nv) {
        const bool is_k = v >= H;
        const int64_t base = (row * H + (is_k ? v - H : v)) * D;
        const void* src = is_k ? k : q;
        lo[u] = IO::load(src, base + ca);
        hi[u] = IO::load(src, base + cb);
      }
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int v = v0 + u;
      if (v < nv) {
        const bool is_k = v >= H;
        const int64_t base = (row * H + (is_k ? v - H : v)) * D;
        const V x0 = IO::widen(lo[u]), x1 = IO::widen(hi[u]);
        V a, b;
        if constexpr (INTERLEAVED) {  // x0 holds pairs j0 .. j0+EPL/2-1, x1 the rest
#pragma unroll
          for (int e = 0; e < EPL / 2; ++e) {
            a[e] = x0[2 * e];
            b[e] = x0[2 * e + 1];
            a[EPL / 2 + e] = x1[2 * e];
            b[EPL / 2 + e] = x1[2 * e + 1];
          }
        } else {
          a = x0;
          b = x1;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) ss += a[e] * a[e] + b[e] * b[e];
#pragma unroll
        for (int m = 1; m < GL; m <<= 1) ss += __shfl_xor(ss, m, GL);
        const float r = __builtin_amdgcn_rsqf(ss * inv_d + eps);
        a *= w[is_k][0] * r;
        b *= w[is_k][1] * r;
        const V ra = a * c - b * s;
        const V rb = b * c + a * s;
        void* dst = is_k ? k_out : q_out;
        if constexpr (INTERLEAVED) {
          V y0, y1;
#pragma unroll
          for (int e = 0; e < EPL / 2; ++e) {
            y0[2 * e] = ra[e];
            y0[2 * e + 1] = rb[e];
            y1[2 * e] = ra[EPL / 2 + e];
            y1[2 * e + 1] = rb[EPL / 2 + e];
          }
          IO::store(dst, base + ca, y0);
          IO::store(dst, base + cb, y1);
        } else {
          IO::store(dst, base + ca, ra);
          IO::store(dst, base + cb, rb);
        }
      }
    }
  }
}

template <int D, bool F32, bool IL>
hipError_t launch_t(const PrologueArgs& a, hipStream_t stream) {
  constexpr int RPB = kThreads / (D / 2 / Io<F32>::EPL);
  const int64_t blocks = (int64_t(a.L) + RPB - 1) / RPB;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((qk_norm_rope_kernel<D, F32, IL>), dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a.q, a.k,
                     a.q_out, a.k_out, a.cos, a.sin, a.wq, a.wk, a.L, a.H, a.eps);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrologueArgs& a, hipStream_t stream) {
  if (a.f32) return a.interleaved ? launch_t<D, true, true>(a, stream) : launch_t<D, true, false>(a, stream);
  return a.interleaved ? launch_t<D, false, true>(a, stream) : launch_t<D, false, false>(a, stream);
}

}  // namespace

hipError_t launch_qk_norm_rope(const PrologueArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_d<128>(a, stream);
  if (a.d == 64) return launch_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace wa

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
// Memory bound: each element is read and written once, the angle tables once per row (the
// 2H vectors of a row hit them in cache).  A group of d/8 lanes owns one (row, tensor,
// head) vector, each lane four channel pairs (8 elements, both members of each pair in the
// lane), so the rotation needs no exchange and the mean square one reduction over the
// group.  Vectors are numbered row-major (row, tensor, head): a wave's 64 lanes cover
// 64 / (d/8) consecutive head vectors, contiguous in memory.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace wa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool F32>
struct Elems;  // load / store of 4 or 8 consecutive elements as fp32
template <>
struct Elems<false> {
  static __device__ __forceinline__ f32x4 load4(const void* base, int64_t i) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(static_cast<const __bf16*>(base) + i);
    return __builtin_convertvector(x, f32x4);
  }
  static __device__ __forceinline__ void store4(void* base, int64_t i, f32x4 v) {
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(base) + i) = __builtin_convertvector(v, bf16x4);
  }
};
template <>
struct Elems<true> {
  static __device__ __forceinline__ f32x4 load4(const void* base, int64_t i) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
  }
  static __device__ __forceinline__ void store4(void* base, int64_t i, f32x4 v) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + i) = v;
  }
};

template <int D, bool F32, bool INTERLEAVED>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                           void* q_out, void* k_out, const float* __restrict__ cosv,
                                                           const float* __restrict__ sinv,
                                                           const float* __restrict__ wq, const float* __restrict__ wk,
                                                           int L, int H, float eps) {
  constexpr int GL = D / 8;              // lanes per vector
  constexpr int VPB = 256 / GL;          // vectors per block per pass
  const int g = threadIdx.x % GL;        // lane within the vector's group: pairs 4g .. 4g+3
  const int64_t n_vec = int64_t(L) * 2 * H;
  const float inv_d = 1.f / float(D);
  for (int64_t vec = int64_t(blockIdx.x) * VPB + threadIdx.x / GL; vec < n_vec; vec += int64_t(gridDim.x) * VPB) {
    const int64_t row = vec / (2 * H);
    const int rem = int(vec - row * 2 * H);
    const bool is_k = rem >= H;
    const int h = is_k ? rem - H : rem;
    const void* src = is_k ? k : q;
    void* dst = is_k ? k_out : q_out;
    const float* w = is_k ? wk : wq;
    const int64_t base = (row * H + h) * D;
    // this lane's elements: a = first members of pairs 4g..4g+3, b = second members
    f32x4 a, b;
    int ia, ib;  // channel of a[0], b[0] (stride 1 within a and b when not interleaved)
    if constexpr (INTERLEAVED) {
      const f32x4 lo = Elems<F32>::load4(src, base + 8 * g), hi = Elems<F32>::load4(src, base + 8 * g + 4);
      a = f32x4{lo[0], lo[2], hi[0], hi[2]};
      b = f32x4{lo[1], lo[3], hi[1], hi[3]};
      ia = 8 * g;
      ib = 8 * g + 1;
    } else {
      a = Elems<F32>::load4(src, base + 4 * g);
      b = Elems<F32>::load4(src, base + D / 2 + 4 * g);
      ia = 4 * g;
      ib = D / 2 + 4 * g;
    }
    float ss = a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3] + b[0] * b[0] + b[1] * b[1] + b[2] * b[2] +
               b[3] * b[3];
#pragma unroll
    for (int m = 1; m < GL; m <<= 1) ss += __shfl_xor(ss, m, GL);
    const float r = __builtin_amdgcn_rsqf(ss * inv_d + eps);
    if (w) {
      if constexpr (INTERLEAVED) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + ia), w1 = *reinterpret_cast<const f32x4*>(w + ia + 4);
        a *= f32x4{w0[0], w0[2], w1[0], w1[2]};
        b *= f32x4{w0[1], w0[3], w1[1], w1[3]};
      } else {
        a *= *reinterpret_cast<const f32x4*>(w + ia);
        b *= *reinterpret_cast<const f32x4*>(w + ib);
      }
    }
    a *= r;
    b *= r;
    const f32x4 c = *reinterpret_cast<const f32x4*>(cosv + row * (D / 2) + 4 * g);
    const f32x4 s = *reinterpret_cast<const f32x4*>(sinv + row * (D / 2) + 4 * g);
    const f32x4 ra = a * c - b * s;
    const f32x4 rb = b * c + a * s;
    if constexpr (INTERLEAVED) {
      Elems<F32>::store4(dst, base + 8 * g, f32x4{ra[0], rb[0], ra[1], rb[1]});
      Elems<F32>::store4(dst, base + 8 * g + 4, f32x4{ra[2], rb[2], ra[3], rb[3]});
    } else {
      Elems<F32>::store4(dst, base + ia, ra);
      Elems<F32>::store4(dst, base + ib, rb);
    }
  }
}

template <int D, bool F32, bool IL>
hipError_t launch_t(const PrologueArgs& a, hipStream_t stream) {
  constexpr int VPB = 256 / (D / 8);
  const int64_t n_vec = int64_t(a.L) * 2 * a.H;
  int64_t blocks = (n_vec + VPB - 1) / VPB;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL((qk_norm_rope_kernel<D, F32, IL>), dim3(blocks), dim3(256), 0, stream, a.q, a.k, a.q_out,
                     a.k_out, a.cos, a.sin, a.wq, a.wk, a.L, a.H, a.eps);
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

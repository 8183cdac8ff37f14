// FP8 (e4m3) variant of the decomposed window attention (gfx950).
//
// Same work units, launch order and output contract as attn_kernel (window items over their
// chunk span and the global rows; global-leg items write fp32 partials that a combine pass
// merges), with q, k and v given as OCP e4m3 codes plus one fp32 scale per tensor (value =
// code * scale).  The lqnn.cn article's fastest H3 configurations run in FP8 (§四); it does
// not say which operands of the attention do, so both products run on gfx950's fp8 matrix
// cores:
//   S^T = K Q^T      v_mfma_f32_32x32x64_f8f6f4, A = K rows from LDS, B = the wave's Q rows
//                    held in registers; the head dimension (128) is two k-steps of 64;
//   O^T += V^T P^T   the same instruction, once per 32-row d-block over a whole 64-key tile:
//                    B = P^T rounded to e4m3 straight from the S^T accumulators, A = V^T
//                    gathered from the row-major V tile with ds_read_b64_tr_b8 (LDS
//                    transpose read), in the key order of P;
//   l += 1 P^T       the same instruction with an all-ones A: the row sums of exactly the
//                    rounded weights that multiply V, accumulated in fp32 by the matrix
//                    core, so the weights applied to V sum to one.
// Both operands of one matrix op map lane half h, byte j to the same k index, so any
// consistent key order is correct; the one used makes P's bytes the S^T accumulator elements
// in register order.
//
// The structure is attn_kernel's: persistent blocks of 4 waves (one per SIMD), 64 query rows
// per wave as two 32-row blocks (qb), 64-key tiles streamed through a 4-deep LDS ring by
// direct global->LDS loads issued three tiles ahead, and per tile four slots of matrix ops
// (S of block 0, PV of block 1 for the previous tile, S of block 1, PV of block 0), each
// interleaved one matrix op at a time with the softmax of the other block, the LDS reads of
// the next fragments and the loads.  A matrix op here takes 64 cycles and the vector work of
// four weights (FMA, exp2, e4m3 packing, max) slightly longer (v_exp_f32 issues in about 10
// cycles), so one group of four weights rides beside each matrix op and the kernel is bound
// by vector issue, not by the matrix pipe.  A wave whose rows lie past the end of an item runs
// a loop of its own that only takes its share of the tile loads and the barriers.  An item
// of at most 64 rows (at H3 the last rows of every group) is instead split over all four
// waves: 32 rows and one 32-key half of every tile each, the halves merged by log-sum-exp
// through the LDS.
// Softmax: online over the tiles in the log2 domain, weights against a lazily raised running
// max (they may reach 2^8, exact in e4m3, whose largest finite value is 448, before it
// rises).  A block's tile takes the wave-uniform slow path when some weight exceeds 2^8, and
// on a unit's first tile and tiles with masked keys: tile max, per-row raise of the running
// max, rescale, weights again.
// Output: O * scale_v / l, rounded to bf16, through an LDS staging area as whole rows.
// LDS rows hold the 128 bytes of a key; their 16-byte chunks are swizzled per row (on the
// global side of the loads) so that the K fragment reads and the V transpose reads are free
// of bank conflicts.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_common.h"
#include "launch.h"

namespace wa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;               // head size = bytes per e4m3 row
constexpr int kNW = 4;                // waves per block, one per SIMD
constexpr int kWaveRows = 64;         // query rows per wave (two 32-row blocks)
constexpr int kBN = kBlockN;          // keys per tile
static_assert(kBN == 64, "one P^T operand covers a 64-key tile");
constexpr int kTileB = kBN * kD;      // bytes of one K (or V) tile
constexpr int kJPW = kTileB / 1024 / kNW;  // 1 KB load slices per wave per tensor per tile
constexpr int kNLD = 2 * kJPW;        // loads per tile per wave (K and V)
constexpr int kNBUF = 4;              // LDS ring of (K, V) tile pairs
constexpr int kRingB = kNBUF * 2 * kTileB;
constexpr int kStageB = 32 * kD * 2;  // per-wave output staging: 32 bf16 rows
static_assert(kJPW == 2, "the slots below issue two loads per half tile");

// 16-byte chunk c of key row r sits at physical chunk c ^ swizzle(r) (rows of 128 bytes, two
// per 256-byte bank line).
//   K: (r / 2) % 8, so the 16 consecutive rows of one ds_read_b128 pass at one logical chunk
//      cover all 64 banks.
//   V: 2 ((r / 2) % 2 + 2 ((r / 8) % 2)).  One ds_read_b64_tr_b8 pass (32 lanes) reads 8
//      rows {B..B+3, B+8..B+11} (B a multiple of 4 with bits 1 and 3 clear) at the 4
//      eight-byte pieces of two adjacent logical chunks; per row parity the 4 rows get 4
//      distinct chunk pairs, so the pass covers all 64 banks.
// Both depend on r % 16 only.
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_v(int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

struct Fp8Params {
  const unsigned char* __restrict__ q;
  const unsigned char* __restrict__ k;
  const unsigned char* __restrict__ v;
  uint16_t* __restrict__ out;
  const Item* __restrict__ items;
  const int32_t* __restrict__ work;
  int32_t* __restrict__ counters;  // kXcdCount queue counters, then the count of finished blocks
  int persistent;                   // 0: block b runs unit work[(b % 8) * per_xcd + b / 8] only
  float* __restrict__ part_o;
  float* __restrict__ part_ml;
  int H, G, frame_rows, n_items, per_xcd;
  uint32_t tensor_bytes;  // bytes of one of q/k/v: L * H * 128
  float scale_log2;       // log2(e) / sqrt(d) * scale_q * scale_k
  float scale_v;
};

// Per 64-key tile a wave runs four slots of matrix ops (P^T words k = 0..7, four weights
// each; see step_work):
//   slot 0: S0(t) = K(t) Q0^T            | words 4..7 of block 1 (tile t-1), 2nd half of the
//                                          loads of t+2; then block 1's slow path if due
//   slot 1: O1 += V(t-1)^T P1^T, l1 += 1 P1^T | words 0..4 of block 0 (tile t), V(t)
//                                          transpose reads (each d-block right after its last
//                                          use by this slot)
//   slot 2: S1(t) = K(t) Q1^T            | words 4..7 of block 0; then its slow path if due
//   barrier: tile t+1 has landed for every wave
//   slot 3: O0 += V(t)^T P0^T, l0 += 1 P0^T | words 0..4 of block 1 (tile t), K(t+1) reads,
//                                          1st half of the loads of t+3
// The loads of t+3 overwrite tile t-1, whose reads every wave finished before the barrier of
// tile t.  Before the first tile, block 1's "previous tile" is empty (scores -inf, V and P
// zero), so every iteration runs the same code; block 1's last PV runs after the loop.
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fp8_kernel(Fp8Params p) {
  constexpr float kLazyLog2 = 8.f;    // the running max rises only when the max grows by > 2^8
  constexpr float kWeightLimit = 256.f;  // fast path only while every weight is <= 2^8
  constexpr int NS = 4;               // matrix ops of an S slot: 2 k-steps x 2 key blocks
  constexpr int NP = 5;               // of a PV slot: 4 d-blocks and the row sums
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kRingB + kNW * kStageB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;  // half of the wave: k sub-block of the matrix operands
  const int l32 = lane & 31;
  const int xcd = blockIdx.x % kXcdCount;
  // the next unit, broadcast by wave 0 through its staging area (idle between epilogues)
  int& s_unit = *reinterpret_cast<int*>(smem + kRingB);
  // e4m3 1.0 in every byte: the A operand of the row-sum matrix op, kept in registers (the
  // empty asm stops the compiler from rebuilding it before every use)
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
  asm volatile("" : "+a"(ones));

  auto run_item = [&](const int unit) __attribute__((always_inline)) {
  const int h = unit / p.n_items;
  const Item it = p.items[unit - h * p.n_items];
  const uint32_t row_bytes = uint32_t(p.H) * kD;  // bytes between consecutive rows of q/k/v
  const int row0 = it.q_begin + wave * kWaveRows;
  const bool wave_active = row0 < it.q_end;
  const bool causal = (it.flags & kItemCausal) != 0;

  // ---- loads: lane l of slice i writes LDS chunk 64 (i kNW + wave) + l, i.e. tile row
  // 8 wave + l / 8 + 32 i at physical chunk l % 8, which holds the row's logical chunk
  // (l % 8) ^ swizzle(row).  The resources are based at this head's first byte and range
  // checked against the end of the tensor (rows past it read as zero).
  const uint32_t dma_row0 = uint32_t(8 * wave + (lane >> 3));
  uint32_t dk[kJPW], dv[kJPW];
#pragma unroll
  for (int i = 0; i < kJPW; ++i) {
    const uint32_t r = dma_row0 + uint32_t(32 * i);
    dk[i] = r * row_bytes + uint32_t(((lane & 7) ^ swz_k(int(r))) << 4);
    dv[i] = r * row_bytes + uint32_t(((lane & 7) ^ swz_v(int(r))) << 4);
  }
  auto make_rsrc = [&](const unsigned char* t) __attribute__((always_inline)) -> i32x4 {
    const uint64_t a = reinterpret_cast<uint64_t>(t) + uint64_t(h) * kD;
    return i32x4{__builtin_amdgcn_readfirstlane(int32_t(uint32_t(a))),
                 __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(int32_t(p.tensor_bytes - uint32_t(h) * kD)), kBufferWord3};
  };
  i32x4 rsrc_k = make_rsrc(p.k), rsrc_v = make_rsrc(p.v);
  // a buffer load may read an SGPR that a vector instruction wrote (the readfirstlane) only
  // 5 wait states later; the loads are inline asm, unseen by the compiler's hazard checks
  asm volatile("s_nop 4" : "+s"(rsrc_k), "+s"(rsrc_v));

  // ---- LDS read offsets (bytes within a ring slot)
  // K fragment of k-step s, key block b: key row 32 b + l32, bytes [64 s + 32 hh, +32) as two
  // chunks (c = 0, 1); the block adds 4096 bytes (the swizzle repeats every 16 rows).
  uint32_t koff[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c = 0; c < 2; ++c) koff[s][c] = uint32_t(l32 * kD + (((4 * s + 2 * hh + c) ^ swz_k(l32)) << 4));
  // V^T fragment of d-block db from four transpose reads m = 0..3: lane (i = lane % 16,
  // g = lane / 16) names key row 16 m + r0 (r0 = 8 (i / 8) + 4 hh + (i / 2) % 4, which is the
  // key of P byte 8 m + i / 2 in lane half hh) at column 32 db + 16 (g % 2) + 8 (i % 2); the
  // instruction hands lane i byte i % 8 of the rows named by lanes 2 j + i / 8, j = 0..7.
  // Read m adds 16 rows (2048 bytes), which keeps the swizzle.
  uint32_t voff[4];
  {
    const int gi = lane & 15, gsel = (lane >> 4) & 1;
    const int r0 = 8 * (gi >> 3) + 4 * hh + ((gi >> 1) & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      voff[db] = uint32_t(kTileB + r0 * kD + (((2 * db + gsel) ^ swz_v(r0)) << 4) + 8 * (gi & 1));
  }

  // ---- tile schedule: segment 0 then segment 1, 64 keys per tile
  const int nt0 = (it.kv0_end - it.kv0_begin + kBN - 1) / kBN;
  const int nt1 = (it.kv1_end - it.kv1_begin + kBN - 1) / kBN;
  const int nt = nt0 + nt1;
  auto tile_range = [&](int t, int& n0, int& nend) __attribute__((always_inline)) {
    if (t < nt0) {
      n0 = it.kv0_begin + t * kBN;
      nend = it.kv0_end;
    } else {
      n0 = it.kv1_begin + (t - nt0) * kBN;
      nend = it.kv1_end;
    }
  };
  // Row offset (bytes) of the first key row of tile u; tiles past the last one re-load the
  // last tile into a slot nobody reads, so every tile issues the same number of loads.
  auto tile_off = [&](int u) __attribute__((always_inline)) -> uint32_t {
    int n0, nend;
    tile_range(u < nt ? u : nt - 1, n0, nend);
    return uint32_t(n0) * row_bytes;
  };
  // Row offset of tile u from that of tile u - 1 (u >= 1): the next 64 rows, the start of
  // segment 1 at its first tile, and past the last tile the last tile again.
  const uint32_t tile_step = 64 * row_bytes, seg1_off = uint32_t(it.kv1_begin) * row_bytes;
  auto next_off = [&](int u, uint32_t prev) __attribute__((always_inline)) -> uint32_t {
    return u >= nt ? prev : u == nt0 ? seg1_off : prev + tile_step;
  };
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)smem));
  // load `idx` (slice idx / 2; K for even idx, V for odd) of the tile at row offset `toff`
  // into ring slot u % kNBUF.  Issued as asm so that the compiler does not make every LDS read
  // wait for the loads in flight; completion is ordered by the vmcnt waits before the
  // barriers.  M0 holds the LDS destination (the nop covers the M0-write hazard).
  auto dma_load = [&](int u, int idx, uint32_t toff) __attribute__((always_inline)) {
    const int i = idx >> 1;
    const uint32_t l = lds_base + uint32_t((2 * (u % kNBUF) + (idx & 1)) * kTileB + (i * kNW + wave) * 1024);
    if (idx & 1)
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(dv[i] + toff), "s"(rsrc_v), "{m0}"(l)
                   : "memory");
    else
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(dk[i] + toff), "s"(rsrc_k), "{m0}"(l)
                   : "memory");
  };

  const float c2 = p.scale_log2;
  const float lazy_raw = kLazyLog2 / c2;
  // initial running max: finite, below every finite score by more than 2^8, so the first
  // tile (which takes the slow path) raises it; weights against it are then exactly zero
  constexpr float kMaxInit = -0x1p100f;
  float m_run[2], mc[2];  // running max of raw scores of this lane's query, and * c2
  f32x16 oacc[2][4], lacc[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    m_run[qb] = kMaxInit;
    mc[qb] = kMaxInit * c2;
    lacc[qb] = f32x16{};
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[qb][db] = f32x16{};
  }

  i32x8 qf[2][2];  // Q fragments [qb][k-step]: lane = query row, bytes [64 s + 32 hh, +32)
  i32x8 kf[2][2];  // K fragments of the current tile [k-step][key block]
  i32x8 vf[4];     // V^T fragments [d-block]
  i32x8 pb[2];     // P^T [qb]: word w = S elements 4 (w % 4) .. +3 of key block w / 4
  float pm[2];     // max weight of the block's current tile (fast path)
  f32x16 s0_split;  // scores of the split-item path
  pb[1] = i32x8{};
#pragma unroll
  for (int db = 0; db < 4; ++db) vf[db] = i32x8{};

  auto read_k = [&](int idx) __attribute__((always_inline)) {  // half idx % 2 of fragment idx / 2
    const int f = idx >> 1, s = f >> 1, b = f & 1, c = idx & 1;
    const u32x4 x = *reinterpret_cast<const u32x4*>(smem + koff[s][c] + b * 32 * kD);
#pragma unroll
    for (int j = 0; j < 4; ++j) kf[s][b][4 * c + j] = int(x[j]);
  };
  auto read_v = [&](int db, int m) __attribute__((always_inline)) {
    const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(smem + voff[db] + m * 16 * kD));
    vf[db][2 * m] = x[0];
    vf[db][2 * m + 1] = x[1];
  };
  auto ring = [](int r) __attribute__((always_inline)) -> uint32_t { return uint32_t(r % kNBUF) * 2 * kTileB; };
  auto other_half = [](float x) __attribute__((always_inline)) -> f32x2 {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return f32x2{__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
  };
  // the four weights of word w of block qb against the running max, packed to e4m3
  auto p_word = [&](int qb, const f32x16 (&sa)[2], int w) __attribute__((always_inline)) {
    const int b = w >> 2, e = 4 * (w & 3);
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][e + j], c2, -mc[qb]));
    const int y = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pb[qb][w], true);
    pb[qb][w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], y, false);
  };
  // Slow path of block qb's tile: mask keys past the segment end (and, for causal items,
  // after the lane's own row), tile max, per-row raise of the running max, weights again.
  auto slow_block = [&](int qb, f32x16 (&sa)[2], int t) __attribute__((always_inline)) {
    int n0, nend;
    tile_range(t, n0, nend);
    const int valid = nend - n0;
    if (valid < kBN || causal) {
      int lim = valid;
      if (causal) lim = __builtin_elementwise_min(lim, row0 + 32 * qb + l32 - n0 + 1);
      lim -= 4 * hh;  // key (b*32 + (i/4)*8 + 4*hh + i%4) >= limit
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sa[b][i] = (b * 32 + (i >> 2) * 8 + (i & 3)) >= lim ? -__builtin_inff() : sa[b][i];
    }
    float mt = sa[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = __builtin_fmaxf(mt, sa[b][i]);
    const f32x2 o = other_half(mt);
    mt = __builtin_fmaxf(o[0], o[1]);
    // Only rows whose own max grew by more than 2^8 raise it (the branch is wave-uniform,
    // the choice per row): a row's arithmetic never depends on the other rows' scores.
    const bool grow = mt > m_run[qb] + lazy_raw;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mt : m_run[qb];
      const float alpha = __builtin_amdgcn_exp2f((m_run[qb] - m_new) * c2);
      m_run[qb] = m_new;
      mc[qb] = m_new * c2;
      lacc[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[qb][db] *= alpha;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) p_word(qb, sa, w);
  };

  // Staged weights.  Word k (k = 0..7) of a block's P^T takes two steps: at step s its
  // FMAs and exponentials, at step s + 1 its e4m3 packing and the max.  The 8 words of block
  // 0 run over the 9 matrix-op steps of slots 1 and 2, those of block 1 over slot 3 and the
  // next tile's slot 0, so every step carries about one word of vector work (about as long
  // as its matrix op) and no step is without a matrix op.  fb holds the exponentials between
  // the two stages, by word parity.  Each stage's result is pinned at its step (an empty asm
  // that reads it): without the pins the compiler sinks pure arithmetic next to its first
  // use, which puts dependent vector ops back to back.
  float fb[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) fb[0][j] = fb[1][j] = 0.f;
  // one step's weight work for block qb: FMAs of word `fe_k`, packing of word `pk_k`, then the
  // exponentials of word `fe_k` (a word < 0 is none)
  auto step_work = [&](int qb, const f32x16 (&sa)[2], int pk_k, int fe_k) __attribute__((always_inline)) {
    if (fe_k >= 0) {
      const int b = fe_k >> 2, e = 4 * (fe_k & 3);
      float* f = fb[fe_k & 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = __builtin_fmaf(sa[b][e + j], c2, -mc[qb]);
      asm volatile("" ::"v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]));
      if (fe_k == 0) pm[qb] = 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
    // Packing of word pk_k to e4m3, in two halves around the exponentials of word fe_k: on
    // gfx950 an instruction that reads the result of a v_cvt_pk_fp8_f32 writing the high
    // half of its register needs a wait state, which the exponentials fill.  (Both halves
    // of the word are written: its old contents only save a move.)
    int y = 0;
    if (pk_k >= 0) {
      const float* f = fb[pk_k & 1];
      pm[qb] = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(pm[qb], f[0]), f[1]), f[2]), f[3]);
      asm volatile("" ::"v"(pm[qb]));
      y = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pb[qb][pk_k], true);
      asm volatile("" ::"v"(y));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (fe_k >= 0) {
      float* f = fb[fe_k & 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_exp2f(f[j]);
      asm volatile("" ::"v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (pk_k >= 0) {
      const float* f = fb[pk_k & 1];
      pb[qb][pk_k] = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], y, false);
      asm volatile("" ::"v"(pb[qb][pk_k]));
    }
  };
  auto pin_p = [&](int qb) __attribute__((always_inline)) {
    asm volatile("" ::"v"(pb[qb][0]), "v"(pb[qb][1]), "v"(pb[qb][2]), "v"(pb[qb][3]), "v"(pb[qb][4]),
                 "v"(pb[qb][5]), "v"(pb[qb][6]), "v"(pb[qb][7]));
  };
  // block qb's verdict on tile t (its scores in sa)
  auto check_block = [&](int qb, f32x16 (&sa)[2], int t, bool dirty) __attribute__((always_inline)) {
    pin_p(qb);
    asm volatile("" ::"v"(pm[qb]));
    if (dirty || __builtin_amdgcn_ballot_w64(pm[qb] > kWeightLimit) != 0) slow_block(qb, sa, t);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Tiles that take the slow path whatever their data, as "the next such tile after u": the
  // first tile, the last tile of a segment that ends inside it, and for causal items every
  // tile from the first one with a key after some row of the wave.  Block 1 checks each tile
  // one iteration after block 0 and reuses its verdict (block 0's causal rows come first, so
  // this is conservative for block 1).
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
  const f32x16 zero = {};
  // A matrix op leads its step (a scheduling barrier keeps the step's vector work after it),
  // except in the last step of a slot, where it follows the vector work: issued last, it
  // runs on through the slot boundary (the checks, the barrier, the loop's scalar work),
  // none of which depends on it.
  auto s_slot = [&](int qb, f32x16 (&sa)[2], bool mma, auto&& extra) __attribute__((always_inline)) {
    auto op = [&](int i) __attribute__((always_inline)) {
      const int s = i >> 1, b = i & 1;
      sa[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[s][b], qf[qb][s], s == 0 ? zero : sa[b], 0, 0, 0, 0,
                                                              0, 0);
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (mma && i < NS - 1) op(i);
      __builtin_amdgcn_sched_barrier(0);
      extra(i);
      __builtin_amdgcn_sched_barrier(0);
      if (mma && i == NS - 1) {
        op(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto pv_slot = [&](int qb, auto&& extra) __attribute__((always_inline)) {
    auto op = [&](int i) __attribute__((always_inline)) {
      if (i < 4) oacc[qb][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[i], pb[qb], oacc[qb][i], 0, 0, 0, 0,
                                                                              0, 0);
      else lacc[qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb[qb], lacc[qb], 0, 0, 0, 0, 0, 0);
    };
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i < NP - 1) op(i);
      __builtin_amdgcn_sched_barrier(0);
      extra(i);
      __builtin_amdgcn_sched_barrier(0);
      if (i == NP - 1) {
        op(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- Output of the 32-row block qb (rows r0 ..).  A lane holds 4-column pieces of its row
  // spread over the row; the block goes through this wave's LDS staging area (16-byte chunks
  // XOR-swizzled by row) and leaves as whole rows, 16 lanes x 16 bytes per row.  Global-leg
  // partials (fp32, already times scale_v) go straight out.
  auto output_block = [&](int qb, int r0) __attribute__((always_inline)) {
    unsigned char* const stage = smem + kRingB + wave * kStageB;
    // lane indices redefined here (empty asm) so that the staging addresses are computed
    // here and not hoisted out of the unit loop into the tile loop's register budget
    int orow_l = l32, olane = lane;
    asm volatile("" : "+v"(orow_l), "+v"(olane));
    const int rows_here = it.q_end - r0;
    if (rows_here <= 0) return;
    const float l_tot = lacc[qb][0];  // every element holds the row sum over both halves
    if (it.split < 0) {
      const float mul = p.scale_v / l_tot;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int off = (32 * db + 8 * g4) * 2 + 8 * hh;  // byte offset in the row
          unsigned char* dst = stage + orow_l * (kD * 2) + (((off >> 4) ^ (orow_l & 15)) << 4) + (off & 15);
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{pack_bf16x2(oacc[qb][db][4 * g4] * mul, oacc[qb][db][4 * g4 + 1] * mul),
                    pack_bf16x2(oacc[qb][db][4 * g4 + 2] * mul, oacc[qb][db][4 * g4 + 3] * mul)};
        }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = k * 64 + olane, r = j >> 4, c = j & 15;
        const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * (kD * 2) + ((c ^ (r & 15)) << 4));
        if (r < rows_here) *reinterpret_cast<u32x4*>(p.out + (int64_t(r0 + r) * p.H + h) * kD + c * 8) = x;
      }
    } else {
      const int qrow = r0 + l32;
      if (qrow < it.q_end) {
        const int64_t slot = (int64_t(it.split) * p.G + (qrow - p.frame_rows)) * p.H + h;
        float* po = p.part_o + slot * kD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<f32x4*>(po + 32 * db + 8 * g4 + 4 * hh) =
                f32x4{oacc[qb][db][4 * g4], oacc[qb][db][4 * g4 + 1], oacc[qb][db][4 * g4 + 2],
                      oacc[qb][db][4 * g4 + 3]} * p.scale_v;
        if (hh == 0) *reinterpret_cast<float2*>(p.part_ml + slot * 2) = make_float2(m_run[qb] * c2, l_tot);
      }
    }
  };

  // ---- Items of at most 64 rows (at H3 the last rows of every 2880-row group) run split
  // over the four waves: wave w takes the 32-row block qs = w & 1 and the 32-key half
  // kh = w >> 1 of every tile, through the same ring, loads and barriers.  In registers the
  // half is key block 0 (its K and V rows are read 32 rows further for kh = 1); P words 4..7
  // and the V fragments' second half stay zero, so each PV matrix op (64 keys) sees only
  // this half.  Per tile:
  //   slot A: S(t) = K(t) Q^T (2 ops)        | second half of the loads of t+2
  //   barrier: tile t+1 has landed for every wave
  //   slot B: O += V(t-1)^T P(t-1)^T, l += 1 P(t-1)^T (5 ops) | P(t) words 0..3, V(t) reads,
  //           K(t+1) reads, first half of the loads of t+3; then the slow path of t if due
  // P(t) is written while the PV ops read P(t-1): P alternates between pb[0] and pb[1] and
  // the tile loop is unrolled twice.  The key halves merge by log-sum-exp through the LDS.
  if (!causal && it.q_end - it.q_begin <= kWaveRows) {
    const int qs = wave & 1, kh = wave >> 1;
    const int r0q = it.q_begin + 32 * qs;
    f32x16& sq = s0_split;
#pragma unroll
    for (int s = 0; s < 2; ++s) koff[s][0] += uint32_t(kh * 32 * kD), koff[s][1] += uint32_t(kh * 32 * kD);
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] += uint32_t(kh * 32 * kD);
    pb[0] = pb[1] = i32x8{};
    {
      const uint32_t toff0 = tile_off(0);
#pragma unroll
      for (int idx = 0; idx < kNLD; ++idx) dma_load(0, idx, toff0);
    }
    {
      const int qrow = r0q + l32;
      const bool ok = qrow < it.q_end;
      const unsigned char* src = p.q + (int64_t(qrow) * p.H + h) * kD + 32 * hh;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (ok) {
          a = *reinterpret_cast<const u32x4*>(src + 64 * s);
          b = *reinterpret_cast<const u32x4*>(src + 64 * s + 16);
        }
        qf[0][s] = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
      }
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    uint32_t toff_q = tile_off(1);
#pragma unroll
    for (int idx = 0; idx < kNLD; ++idx) dma_load(1, idx, toff_q);
    toff_q = tile_off(2);
#pragma unroll
    for (int idx = 0; idx < kNLD / 2; ++idx) dma_load(2, idx, toff_q);
    barrier();
#pragma unroll
    for (int s = 0; s < 2; ++s) read_k(4 * s), read_k(4 * s + 1);  // key block 0 of both k-steps
#pragma unroll
    for (int s = 0; s < 2; ++s) koff[s][0] += ring(1), koff[s][1] += ring(1);

    // one step of slot B: FMAs and exponentials of word fe, packing (high half first, around
    // the exponentials) and the max of word pk, into register set buf
    auto step_q = [&](int buf, int pk, int fe) __attribute__((always_inline)) {
      if (fe >= 0) {
        float* f = fb[fe & 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __builtin_fmaf(sq[4 * fe + j], c2, -mc[0]);
        asm volatile("" ::"v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]));
        if (fe == 0) pm[0] = 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
      int y = 0;
      if (pk >= 0) {
        const float* f = fb[pk & 1];
        pm[0] = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(pm[0], f[0]), f[1]), f[2]), f[3]);
        asm volatile("" ::"v"(pm[0]));
        y = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], pb[buf][pk], true);
        asm volatile("" ::"v"(y));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (fe >= 0) {
        float* f = fb[fe & 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = __builtin_amdgcn_exp2f(f[j]);
        asm volatile("" ::"v"(f[0]), "v"(f[1]), "v"(f[2]), "v"(f[3]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (pk >= 0) {
        const float* f = fb[pk & 1];
        pb[buf][pk] = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], y, false);
        asm volatile("" ::"v"(pb[buf][pk]));
      }
    };
    // slow path of tile t: mask keys past the segment end, raise the max of rows whose max
    // grew by more than 2^8, words 0..3 of P(t) again
    auto slow_q = [&](int buf, int t) __attribute__((always_inline)) {
      int n0, nend;
      tile_range(t, n0, nend);
      const int valid = nend - n0;
      if (valid < kBN) {
        const int lim = valid - 32 * kh - 4 * hh;  // key (32 kh + (i/4)*8 + 4*hh + i%4) >= valid
#pragma unroll
        for (int i = 0; i < 16; ++i) sq[i] = ((i >> 2) * 8 + (i & 3)) >= lim ? -__builtin_inff() : sq[i];
      }
      float mt = sq[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = __builtin_fmaxf(mt, sq[i]);
      const f32x2 o = other_half(mt);
      mt = __builtin_fmaxf(o[0], o[1]);
      const bool grow = mt > m_run[0] + lazy_raw;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : m_run[0];
        const float alpha = __builtin_amdgcn_exp2f((m_run[0] - m_new) * c2);
        m_run[0] = m_new;
        mc[0] = m_new * c2;
        lacc[0] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[0][db] *= alpha;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sq[4 * w + j], c2, -mc[0]));
        const int y = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pb[buf][w], true);
        pb[buf][w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], y, false);
      }
    };
    // slot B's matrix op i: four d-blocks of O, then the row sums
    auto pv_q = [&](int buf, int i) __attribute__((always_inline)) {
      if (i < 4) oacc[0][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[i], pb[buf], oacc[0][i], 0, 0, 0, 0, 0, 0);
      else lacc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pb[buf], lacc[0], 0, 0, 0, 0, 0, 0);
    };
    int nd = 0;  // next tile that takes the slow path
    auto tile_q = [&](int t, auto cur_c) __attribute__((always_inline)) {
      constexpr int cur = decltype(cur_c)::value;  // register set of P(t); P(t-1) is in the other
      const uint32_t step_k = ring(t + 2) - ring(t + 1);
      const uint32_t step_v = ring(t + 1) - ring(t);
      const bool dirty = t == nd;
      if (__builtin_expect(dirty, 0)) nd = next_dirty(t);
      __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
      __builtin_amdgcn_sched_barrier(0);
      // slot A
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        sq = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[s][0], qf[0][s], s == 0 ? zero : sq, 0, 0, 0, 0, 0, 0);
        dma_load(t + 2, kNLD / 2 + s, toff_q);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70 | kNLD);  // tile t+1 has landed (t+2 may be in flight) ...
      barrier();                                   // ... for every wave
      toff_q = next_off(t + 3, toff_q);
      // slot B
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        pv_q(cur ^ 1, i);
        __builtin_amdgcn_sched_barrier(0);
        if (i < 4) {
          read_v(i, 0);
          read_v(i, 1);
        }
        if (i < 2) read_k(4 * i), read_k(4 * i + 1);
        if (i == 0 || i == 2) dma_load(t + 3, i / 2, toff_q);
        step_q(cur, i - 1, i < 4 ? i : -1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) voff[db] += step_v;
#pragma unroll
      for (int s = 0; s < 2; ++s) koff[s][0] += step_k, koff[s][1] += step_k;
      asm volatile("" ::"v"(pb[cur][0]), "v"(pb[cur][1]), "v"(pb[cur][2]), "v"(pb[cur][3]), "v"(pm[0]));
      if (dirty || __builtin_amdgcn_ballot_w64(pm[0] > kWeightLimit) != 0) slow_q(cur, t);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int t = 0; t < nt; t += 2) {
      tile_q(t, std::integral_constant<int, 0>{});
      if (t + 1 < nt) tile_q(t + 1, std::integral_constant<int, 1>{});
    }
    // PV of the last tile
    if ((nt - 1) & 1) {
#pragma unroll
      for (int i = 0; i < 5; ++i) pv_q(1, i);
    } else {
#pragma unroll
      for (int i = 0; i < 5; ++i) pv_q(0, i);
    }
    // merge the key halves: the kh = 1 wave of each block leaves O (64 floats per lane, in
    // lane order) and its (max, row sum) in the idle ring; the kh = 0 wave, whose lanes own
    // the same rows and columns, merges them and writes the block
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // the ring's last loads have landed ...
    barrier();                            // ... and no wave reads it any more
    unsigned char* const mb = smem + qs * (16 * 1024 + 512);
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<f32x4*>(mb + (db * 4 + g4) * 1024 + lane * 16) =
              f32x4{oacc[0][db][4 * g4], oacc[0][db][4 * g4 + 1], oacc[0][db][4 * g4 + 2], oacc[0][db][4 * g4 + 3]};
      *reinterpret_cast<f32x2*>(mb + 16 * 1024 + lane * 8) = f32x2{m_run[0], lacc[0][0]};
    }
    barrier();
    if (kh == 0) {
      const f32x2 ml = *reinterpret_cast<const f32x2*>(mb + 16 * 1024 + lane * 8);
      const float m_new = __builtin_fmaxf(m_run[0], ml[0]);
      const float a0 = __builtin_amdgcn_exp2f((m_run[0] - m_new) * c2), a1 = __builtin_amdgcn_exp2f((ml[0] - m_new) * c2);
      m_run[0] = m_new;
      lacc[0][0] = lacc[0][0] * a0 + ml[1] * a1;
#pragma unroll
      for (int db = 0; db < 4; ++db)
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

  // prologue: tile 0 and the Q fragments land together; then tile 1 and the first half of
  // tile 2 go in flight
  {
    const uint32_t toff0 = tile_off(0);
#pragma unroll
    for (int idx = 0; idx < kNLD; ++idx) dma_load(0, idx, toff0);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = row0 + 32 * qb + l32;
    const bool ok = qrow < it.q_end;
    const unsigned char* src = p.q + (int64_t(qrow) * p.H + h) * kD + 32 * hh;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (ok) {
        a = *reinterpret_cast<const u32x4*>(src + 64 * s);
        b = *reinterpret_cast<const u32x4*>(src + 64 * s + 16);
      }
      qf[qb][s] = i32x8{int(a[0]), int(a[1]), int(a[2]), int(a[3]), int(b[0]), int(b[1]), int(b[2]), int(b[3])};
    }
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  uint32_t toff_a = tile_off(1);  // the tile whose loads are in flight in two halves
#pragma unroll
  for (int idx = 0; idx < kNLD; ++idx) dma_load(1, idx, toff_a);
  toff_a = tile_off(2);
#pragma unroll
  for (int idx = 0; idx < kNLD / 2; ++idx) dma_load(2, idx, toff_a);
  barrier();
  if (wave_active) {
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) read_k(idx);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) koff[s][0] += ring(1), koff[s][1] += ring(1);  // from here on: the next tile

  f32x16 s0[2], s1[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) s1[b][i] = -__builtin_inff();
  pm[1] = 0.f;

  if (!wave_active) {
    // a wave without rows in this item takes only its share of the loads and the barriers
    for (int t = 0; t < nt; ++t) {
#pragma unroll
      for (int idx = kNLD / 2; idx < kNLD; ++idx) dma_load(t + 2, idx, toff_a);
      __builtin_amdgcn_s_waitcnt(0x0F70 | kNLD);
      barrier();
      toff_a = next_off(t + 3, toff_a);
#pragma unroll
      for (int idx = 0; idx < kNLD / 2; ++idx) dma_load(t + 3, idx, toff_a);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // no load may still write this block's LDS at exit
    return;
  }
  int nd = 0;               // next tile that takes the slow path
  bool dirty_prev = false;  // block 0's verdict on the previous tile (tile -1: none)
  for (int t = 0; t < nt; ++t) {
    const uint32_t step_k = ring(t + 2) - ring(t + 1);  // slot advance after this tile's reads
    const uint32_t step_v = ring(t + 1) - ring(t);
    const bool dirty = t == nd;
    if (__builtin_expect(dirty, 0)) nd = next_dirty(t);

    // slot 0 (its K fragments were read in slot 3 of the previous tile, long done)
    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    s_slot(0, s0, true, [&](int i) __attribute__((always_inline)) {
      if (i == 0 || i == 2) dma_load(t + 2, kNLD / 2 + i / 2, toff_a);
      step_work(1, s1, 4 + i, i < 3 ? 5 + i : -1);
    });
    check_block(1, s1, t - 1, dirty_prev);
    // slot 1
    pv_slot(1, [&](int i) __attribute__((always_inline)) {
      if (i < 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) read_v(i, m);
      }
      step_work(0, s0, i - 1, i);
    });
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] += step_v;
    // slot 2
    s_slot(1, s1, true, [&](int i) __attribute__((always_inline)) { step_work(0, s0, 4 + i, i < 3 ? 5 + i : -1); });
    check_block(0, s0, t, dirty);
    __builtin_amdgcn_s_waitcnt(0x0F70 | kNLD);  // tile t+1 has landed (t+2 may be in flight) ...
    barrier();                                   // ... for every wave
    toff_a = next_off(t + 3, toff_a);
    // slot 3 (after the last tile the K reads hit a slot nobody uses)
    pv_slot(0, [&](int i) __attribute__((always_inline)) {
      if (i < 4) {
        read_k(2 * i);
        read_k(2 * i + 1);
      }
      if (i == 0 || i == 2) dma_load(t + 3, i / 2, toff_a);
      step_work(1, s1, i - 1, i);
    });
#pragma unroll
    for (int s = 0; s < 2; ++s) koff[s][0] += step_k, koff[s][1] += step_k;
    dirty_prev = dirty;
  }
  __builtin_amdgcn_s_waitcnt(kVmcnt0);  // no load may still write this block's LDS at exit
  // block 1 of the last tile
  s_slot(0, s0, false, [&](int i) __attribute__((always_inline)) { step_work(1, s1, 4 + i, i < 3 ? 5 + i : -1); });
  check_block(1, s1, nt - 1, dirty_prev);
  pv_slot(1, [&](int) __attribute__((always_inline)) {});

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) output_block(qb, row0 + 32 * qb);
  };  // run_item

  for (int n = 0;; ++n) {
    // The barrier also orders this block's LDS use: every wave has finished the previous unit
    // before the next unit's prologue refills the ring.  Without queues (few units) block b
    // runs the one unit at its place in the launch order.
    if (wave == 0) {
      const int u = p.persistent ? fetch_unit(p.work, p.counters, p.per_xcd, xcd, lane)
                                 : (n == 0 ? p.work[xcd * p.per_xcd + int(blockIdx.x) / kXcdCount] : -1);
      if (lane == 0) s_unit = u;
    }
    __syncthreads();
    const int unit = __builtin_amdgcn_readfirstlane(s_unit);
    if (unit < 0) break;
    run_item(unit);
  }
  if (p.persistent && tid == 0) finish_persistent(p.counters);  // the last block resets the queues
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
  *reinterpret_cast<uint2*>(out + orow) =
      make_uint2(pack_bf16x2(num.x * inv, num.y * inv), pack_bf16x2(num.z * inv, num.w * inv));
}

}  // namespace

hipError_t launch_forward_fp8(const ForwardArgs& a, float scale_v, hipStream_t stream) {
  if (a.d != kD || a.block_m != kNW * kWaveRows || a.out_f32 || a.tile_list) return hipErrorInvalidValue;
  Fp8Params p;
  p.q = static_cast<const unsigned char*>(a.q);
  p.k = static_cast<const unsigned char*>(a.k);
  p.v = static_cast<const unsigned char*>(a.v);
  p.out = static_cast<uint16_t*>(a.out);
  p.items = a.items;
  p.work = a.work;
  p.counters = a.counters;
  p.persistent = a.persistent;
  p.part_o = a.part_o;
  p.part_ml = a.part_ml;
  p.H = a.H;
  p.G = a.G;
  p.frame_rows = a.frame_rows;
  p.n_items = a.n_items;
  p.per_xcd = a.work_per_xcd;
  p.tensor_bytes = uint32_t(a.L) * uint32_t(a.H) * uint32_t(kD);
  p.scale_log2 = a.scale_log2;
  p.scale_v = scale_v;
  if (a.grid < 1) return hipSuccess;
  hipLaunchKernelGGL(attn_fp8_kernel, dim3(a.grid), dim3(kNW * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits <= 1) return e;
  hipLaunchKernelGGL(combine_fp8_kernel, dim3((a.G * a.H + kCombineSlots - 1) / kCombineSlots), dim3(kCombineThreads),
                     0, stream, a.part_o, a.part_ml, p.out, a.G, a.H, a.n_splits, a.frame_rows);
  return hipGetLastError();
}

}  // namespace wa

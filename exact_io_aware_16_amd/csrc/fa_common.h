// Device-side building blocks shared by the attention kernels (gfx950).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one
// 64-lane wave, lane l, half g = l / 32, column c = l % 32):
//   A operand (32 x 16, row-major M x K): lane holds A[c][8g .. 8g+7]
//   B operand (16 x 32, K x N):           lane holds B[8g .. 8g+7][c]
//   C result  (32 x 32):                  register i holds C[8(i/4) + 4g + i%4][c]
// So every operand register group is 8 consecutive elements along the
// contraction axis, and a result column belongs to one lane.  The row order
// of the result can be chosen freely by choosing which source row each lane
// loads as A row c; the kernels use the bit permutation perm32 (swap bits 2
// and 3 of the row index) so that register i of half g lands on row
// 16(i/8) + 8g + i%8: runs of 8 consecutive rows per register octet, which
// is exactly the operand layout of the next product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

template <int V>
using ic = std::integral_constant<int, V>;

// Compile-time loop: f(ic<i>{}) for i = B .. E-1.  Group, phase and piece
// indices of the backward kernels go through this rather than through
// unrolled loops, so every register-array index is a constant from the start.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    static_for<B + 1, E>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_raw;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// swap bits 2 and 3 of a row index in 0..31 (an involution)
__device__ __forceinline__ constexpr int perm32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// result register i of half g of a perm32-loaded product -> row in 0..31
__device__ __forceinline__ constexpr int perm_row(int i, int g) {
  return 16 * (i / 8) + 8 * g + (i % 8);
}

// plain (unpermuted) result row of register i in half g
__device__ __forceinline__ constexpr int acc_row(int i, int g) {
  return 8 * (i / 4) + 4 * g + (i % 4);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Operand-register reuse and the matrix core.  An issued MFMA may wait for
// the matrix unit (behind the previous MFMA) before it reads its A/B
// registers, and nothing stops a later load from overwriting those registers
// in the meantime; the compiler does not guard that write-after-read.  The
// kernels therefore rotate operand registers through two sets and release a
// set only after the next group of MFMAs has been issued:
//   anchor_*(acc)  -- empty asm that takes (and formally rewrites) an MFMA
//                     result: the product is a pure value, so without it the
//                     instruction selector may place the MFMA after the fence
//                     that follows; with it the MFMA is emitted before the
//                     anchor.  anchor_v for results kept in VGPRs, anchor_a
//                     for results kept in AGPRs (the wrong class costs copies);
//   group_fence()  -- no instruction is scheduled across it, so every MFMA of
//                     the group before it (anchored) is issued before
//                     anything after it;
//   pin(v)         -- empty asm reading v: keeps v's registers live (and not
//                     reused) up to this point.  Emits no code.
// At the end of a phase, pin(v, x) with x computed from all of the phase's
// MFMA results keeps the operands live until those MFMAs have completed.
__device__ __forceinline__ void anchor_v(f32x16& acc) { asm volatile("" : "+v"(acc)); }
__device__ __forceinline__ void anchor_a(f32x16& acc) { asm volatile("" : "+a"(acc)); }
__device__ __forceinline__ void group_fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void pin(const bf16x8& v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void pin(const bf16x8& v, float after) { asm volatile("" ::"v"(v), "v"(after)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight float32 values rounded to bf16 (round to nearest even) and packed.
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)p[e];
  return r;
}

// Combine each lane with its partner in the other half of the wave (lane
// l and l ^ 32) using v_permlane32_swap, without a trip through LDS.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + sum of the eight bf16 values, exactly as stored (v_dot2 against 1.0).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const uint4 w = __builtin_bit_cast(uint4, v);
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), one, acc, false);
  return acc;
}

// Workgroup order: the hardware hands consecutive workgroup ids to the eight
// XCDs in turn, and each XCD has its own L2.  Mapping id -> (id % 8) * per +
// id / 8 gives XCD x the contiguous logical range [x*per, (x+1)*per), so the
// query blocks of one head -- which stream the same K and V -- share an L2.
// grid must be a multiple of 8; ids mapping past `total` do nothing.
__device__ __forceinline__ int xcd_logical_block(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// Packed variable-length sequences: Q, K, V (and O, L and the gradients) are
// [H, total, d] head-major, and sequence b occupies rows cu[b] .. cu[b+1]-1
// of every head.  cu == nullptr means the dense [B, H, N, d] layout.
struct Seqs {
  const int* cu;
  int H;      // heads
  int total;  // packed rows per head
};
// Rows [s0, s1) of sequence b, clamped into [0, total] and non-decreasing:
// offsets out of order cost correctness, never an access outside the tensors.
__device__ __forceinline__ void seq_range(const Seqs& sq, int b, int& s0, int& s1) {
  const int a = min(max(sq.cu[b], 0), sq.total);
  s0 = a;
  s1 = min(max(sq.cu[b + 1], a), sq.total);
}

// Causal work items come in ranks of different length (the key range of a
// query block, the query range of a key block), one item per head and rank,
// rank 0 the longest.  The hardware deals consecutive ids to the eight XCDs
// in turn, so XCD x runs ids x, x + 8, x + 16, ... in that order, each on
// the next free CU.  With BH a multiple of 8, heads h = x (mod 8) go to XCD
// x, which takes them in groups of G heads, rank-major inside a group
// (longest first).  The items running at once on an XCD then stream the
// K/V (or Q/dO) of at most G heads, which its L2 holds, and the lengths
// still pair up long with short.  Otherwise ids are taken rank-major over
// all heads, id = rank * BH + head, which is also what G >= BH / 8 gives.
// ids from BH * n_rank on do nothing.
//
// Measured on MI355X (B=2, H=16, N=4096): one or two heads per group brings
// the backward kernels' HBM bytes down to the algorithmic count, but costs
// 1-3% of their time against rank-major order over all heads -- their
// re-reads hit the L2 and the memory-side cache and never limit them -- so
// the d = 128 kernels pass kAllHeads.  The 128-row forward kernel, which
// runs two workgroups per CU over many heads, keeps two heads per group:
// same time, a third of the HBM bytes.
constexpr int kAllHeads = 1 << 30;
__device__ __forceinline__ void causal_order(int bid, int BH, int n_rank, int G, int& rank, int& head) {
  if ((BH & 7) == 0) {
    const int x = bid & 7, s = bid >> 3;
    const int hx = BH >> 3;  // heads per XCD
    const int gs = min(G, hx);
    const int gi = s / (gs * n_rank), w = s - gi * gs * n_rank;
    const int in_group = min(gs, hx - gi * gs);  // the last group may be smaller
    rank = w / in_group;
    head = x + 8 * (gi * gs + (w - rank * in_group));
  } else {
    rank = bid / BH;
    head = bid - rank * BH;
  }
}

}  // namespace fa

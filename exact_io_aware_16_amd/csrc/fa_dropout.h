// Attention dropout with a regenerated mask (gfx950).
//
// The backward keeps the generator's state, not the mask, and rebuilds the
// same mask tile by tile ("Backward can recreate tiles instead of retaining
// the square", Why FlashAttention Can Avoid a Square Attention Array Without
// Making Attention Linear).  The generator is Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).
//
// Mask of head bh (= b H + h), query row i, key j, seed s, offset o:
//   words = Philox4x32-10(counter (j/4, i/4, bh, o), key (s mod 2^32, s / 2^32))
//   byte  = byte (j mod 4) of words[i mod 4];  kept iff byte >= t
// with t = min(255, round(256 p)); kept weights are scaled by 256 / (256 - t).
// One call covers a 4 x 4 block of (row, key) pairs.  In every kernel's
// register layout an aligned group of 4 lanes holds exactly four such blocks
// per 32 x 32 product block, so each lane makes one call and the group
// exchanges words (quad_transpose).
#pragma once

#include "fa_common.h"

namespace fa {

struct Dropout {
  uint32_t k0, k1;  // Philox key: the seed's low and high words
  uint32_t offset;  // fourth counter word
  int t;            // keep iff byte >= t
  float r;          // 256 / (256 - t)
};

// Ten Philox rounds on (x0, x1, x2, x3): multiply words 0 and 2 by the two
// Philox multipliers, keep both halves of the products, mix the high halves
// with the other words and the key; the key advances by the Weyl constants
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)x[0] * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)x[2] * 0xCD9E8D57u;
    const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x[1] ^ k0;
    const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x[3] ^ k1;
    x[1] = (uint32_t)p1;
    x[3] = (uint32_t)p0;
    x[0] = y0;
    x[2] = y2;
  }
}

// Word exchange within each aligned group of 4 lanes (q = lane & 3): lane q
// returns out[x] = w[q] of lane x.  Four rotations: in rotation s, lane k
// sends w[(k - s) & 3] and lane q receives it from lane (q + s) & 3.
template <int S>
__device__ __forceinline__ uint32_t quad_rotate(uint32_t v) {
  constexpr int ctrl = ((0 + S) & 3) | (((1 + S) & 3) << 2) | (((2 + S) & 3) << 4) | (((3 + S) & 3) << 6);
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t pick4(const uint32_t (&w)[4], int i) {
  const uint32_t lo = (i & 1) ? w[1] : w[0];
  const uint32_t hi = (i & 1) ? w[3] : w[2];
  return (i & 2) ? hi : lo;
}
__device__ __forceinline__ void quad_transpose(const uint32_t (&w)[4], uint32_t (&out)[4], int q) {
  uint32_t recv[4];
  recv[0] = pick4(w, q);
  recv[1] = quad_rotate<1>(pick4(w, (q - 1) & 3));
  recv[2] = quad_rotate<2>(pick4(w, (q - 2) & 3));
  recv[3] = quad_rotate<3>(pick4(w, (q - 3) & 3));
  // recv[s] came from lane (q + s) & 3
#pragma unroll
  for (int x = 0; x < 4; ++x) out[x] = pick4(recv, (x - q) & 3);
}

// In-lane 4 x 4 byte transpose: out[c] byte r = w[r] byte c.
__device__ __forceinline__ void byte_transpose(const uint32_t (&w)[4], uint32_t (&out)[4]) {
  // v_perm_b32(hi, lo, sel): byte selector 0-3 picks lo's bytes, 4-7 hi's
  const uint32_t a = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
  const uint32_t b = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);  // w2.b0 w3.b0 w2.b1 w3.b1
  const uint32_t c = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
  const uint32_t d = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);  // w2.b2 w3.b2 w2.b3 w3.b3
  out[0] = __builtin_amdgcn_perm(b, a, 0x05040100u);  // a.b0 a.b1 b.b0 b.b1
  out[1] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.b2 a.b3 b.b2 b.b3
  out[2] = __builtin_amdgcn_perm(d, c, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(d, c, 0x07060302u);
}

// Keep flag of byte e (0..3) of a mask word.
__device__ __forceinline__ bool kept(uint32_t word, int e, int t) { return (int)((word >> (8 * e)) & 0xffu) >= t; }

// Zero the dropped bf16 weights of one 8-element operand: elements 0..3 take
// bytes 0..3 of m0, elements 4..7 those of m1.
__device__ __forceinline__ bf16x8 drop_bf16x8(bf16x8 p, uint32_t m0, uint32_t m1, int t) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v u = __builtin_bit_cast(u32x4v, p);
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const uint32_t m = pr < 2 ? m0 : m1;
    const int e = 2 * (pr & 1);
    const uint32_t keep = (kept(m, e, t) ? 0x0000ffffu : 0u) | (kept(m, e + 1, t) ? 0xffff0000u : 0u);
    u[pr] &= keep;
  }
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace fa

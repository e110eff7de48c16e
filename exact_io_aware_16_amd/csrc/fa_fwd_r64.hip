// Exact attention forward for head width 128 (d = dv = 128), bf16 inputs,
// float32 outputs: the wide-wave kernel.
//
// Same results contract as fwd_bf16_kernel (fa_fwd_bf16.hip): softmax(c S) V
// and the row log-sum-exp L, computed tile by tile with one division by the
// running sum after the last tile ("From softmax to attention: rescale the
// output too", FlashAttention: The Matrix You Never Have to Write Down).
//
// Reference of the exponentials.  The page's recurrence keeps sums against a
// running max and rescales them when a tile raises it; the FA4 paragraph
// under "What it doesn't solve" defers that rescale until the shift is large.
// Any common reference gives the same quotient (the identity both rest on);
// the max only keeps the exponentials in range.  This kernel takes the
// deferral to its end: a row's reference is the exact max of its first key
// sub-tile and never moves, so the loop has no per-tile max and no rescale of
// O.  Later weights may exceed 1; float32 holds them unless a weight, the sum
// or an O element overflows, and a check after the loop sees exactly that (a
// non-finite value).  Then the workgroup starts again with the exact row max
// over all of its keys as the reference (a separate pass over K), for which
// no weight exceeds 1 -- the page's own frame.  A weight that underflows
// against the fixed reference is below 2^-126 of the weight (1) of the
// reference's own key, which the sum always holds.
//
// Why a second kernel: on gfx950 the local data share serves about 128 bytes
// per clock per CU.  With 32 query rows per wave every 32x32x16 product reads
// its 1 KiB K or V^T operand from LDS, which at the full matrix rate is that
// whole bandwidth.  Here each wave owns 64 query rows (two 32-row halves h0,
// h1) and one wave runs per SIMD: every K and V^T operand read from LDS feeds
// two products (one per half), halving the LDS bytes per product.  With one
// wave per SIMD the softmax must overlap the wave's own matrix work, so the
// loop is software pipelined:
//   step u, phase 1:  S(u+1) = K(u+1) Q^T for both halves (16 products)
//                     beside the weights of sub-tile u, half 1;
//   step u, phase 2:  O^T += V(u)^T P(u)^T for both halves (16 products)
//                     beside the weights of sub-tile u+1, half 0.
// The weights go in pieces of two per lane, one piece per group of two
// products (phase 2's first group reads no S of the next sub-tile, so its
// second group takes two pieces); sched_group_barrier keeps each piece's
// vector instructions between the products in program order, so a lone wave
// issues them while its products run.  K runs one tile ahead of V in the LDS
// rings.
//
// Register plan per wave (one wave per SIMD, up to 512 registers): Q as the
// B operand of S^T (16 x 4 registers), O^T accumulators 2 x 4 blocks of
// 32 x 32 (128), two S tiles (S(u) half 1 and S(u+1) in flight), the bf16
// weights of two sub-tiles, K and V^T operand rings of three sets each.
//
// Operand registers follow the rule of fa_common.h (a register read by one
// product is overwritten only after the next product has been issued): each
// phase is cut into groups of products separated by group_fence(), and after
// every product an empty asm ties its result to the operands the previous
// product read.
#include <algorithm>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kD = 128, kDV = 128;
constexpr int kBC = 64;           // keys per LDS tile (one copy and one barrier each)
constexpr int kSub = 32;          // keys per pipeline step (a sub-tile)
constexpr int kNKK = kD / 16;     // 16-wide slices of the head dimension (S product)
constexpr int kNKG = kSub / 16;   // 16-key groups of a sub-tile (P V product)
constexpr int kNDB = kDV / 32;    // 32-row blocks of O^T
constexpr int kWaves = 4;         // one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kKSlots = 3;        // K ring: the tile in use, the next one, the one arriving

constexpr int kComputeUnits = 256;

// SPLIT = 1: 4 row groups of 64 rows share every key tile.  SPLIT = 2: 2 row
// groups, the key tiles cut into two ranges taken by waves {0,1} and {2,3},
// merged through LDS at the end (split-KV inside the workgroup, for grids
// with fewer workgroups than compute units).
template <int SPLIT>
struct Smem {
  bf16_raw k[SPLIT][kKSlots][kBC * kD];
  // V ring: three slots with one key range, two with two ranges (LDS holds
  // no more); the steady loop unrolls over a multiple of both ring sizes so
  // every slot is known at compile time
  static constexpr int kVSlots = SPLIT == 1 ? 3 : 2;
  bf16_raw v[SPLIT][kVSlots][kBC * kDV];
};

// LDS tile layout (16-byte slots, XOR swizzle, no padding):
//   K tile: row r holds key (r & ~31) + perm32(r & 31); chunk c of it sits in
//           slot c ^ (r & 15), so the 32 rows x 16 bytes of one operand read
//           spread over all 64 banks;
//   V tile: row r holds key r; chunk c sits in slot c ^ 4 (r & 3), which keeps
//           the transpose reads (4 rows x 4 slots per 16 lanes) conflict free.
__device__ __forceinline__ constexpr int kswz(int r) { return r & 15; }
__device__ __forceinline__ constexpr int vswz(int r) { return 4 * (r & 3); }

// Per-lane source offsets (bytes from the tile's first row) of the 16-byte
// chunks that copy-wave cw of W copies into one K and one V tile.  LDS-direct
// loads write 64 consecutive 16-byte slots per instruction, so the swizzle is
// applied on the source side; reads past the head's last key return zeros.
template <int W>
struct Copy {
  static constexpr int NI = kBC * (kD / 8) / (64 * W);  // instructions per tile and wave
  uint32_t k_off[NI], v_off[NI];
  __device__ __forceinline__ void init(int cw, int lane, uint32_t k_row, uint32_t v_row) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (i * W + cw) * 4 + lane / 16;
      const int slot = lane % 16;
      k_off[i] = (uint32_t)((r & ~31) + perm32(r & 31)) * k_row + (uint32_t)(16 * (slot ^ kswz(r)));
      v_off[i] = (uint32_t)r * v_row + (uint32_t)(16 * (slot ^ vswz(r)));
    }
  }
};

// One tile of BC rows from key0 of a head (K offsets when IS_K, else V).  The
// descriptor starts at the tile's first row and spans the rest of the head,
// so the lane offsets stay loop invariant and the hardware range check zeroes
// reads past the head's last key.
template <int W, bool IS_K>
__device__ __forceinline__ void issue_tile(bf16_raw* dst, const bf16_raw* base_ptr, int Nk, int key0, uint32_t row,
                                           const Copy<W>& cp, int cw_s) {
  key0 = __builtin_amdgcn_readfirstlane(key0);
  const uint32_t b0 = (uint32_t)key0 * row;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)base_ptr + b0), (short)0, (int)((uint32_t)Nk * row - b0), 0x00020000);
  const uint32_t base = lds_addr_of(dst);
#pragma unroll
  for (int i = 0; i < Copy<W>::NI; ++i)
    lds_copy(rs, IS_K ? cp.k_off[i] : cp.v_off[i], 0u, base + (uint32_t)(i * W + cw_s) * 1024u);
}

// sched_group_barrier masks
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;
template <int MASK, int N>
__device__ __forceinline__ void sg() { __builtin_amdgcn_sched_group_barrier(MASK, N, 0); }

// Running softmax state of one 32-row half (per lane: the row of its column).
struct Half {
  float m_ref;   // reference of the exponentials (log2 units, scaled); -inf: no visible key
  float m_use;   // m_ref, or 0 for a row that sees nothing
  float l;       // running sum of the float32 weights
};

// Per-wave state of the main loop.  s[p][h]: S^T of the sub-tile of parity p
// (sub-tile v lives in s[v & 1]) for half h, as the product returns it:
// register 8 hh + e of lane half g holds key 16 hh + 8 g + e of the sub-tile
// for the query in the lane's column.  Products accumulate in AGPRs; Q,
// read-only, sits in AGPRs too.
struct Wave {
  f32x16 s[2][2];
  f32x16 o[2][kNDB];          // O^T accumulators: d-row 32 db + acc_row(i, g), query = column
  bf16x8 qf[2][kNKK];         // Q^T operand slices, per half
  bf16x8 pb[2][2][kNKG];      // bf16 weights, [parity][half][16-key group]
  bf16x8 ak[3];               // K operand ring: slice kk in slot kk % 3
  bf16x8 av[3];               // V^T operand ring: group gi in slot gi % 3
  Half hs[2];
  float part[2][8];          // piece sums of the sub-tile in progress, per half
  float pf[2][2][8];         // float32 weights before packing, [half][16-key group]
  uint32_t kaddr[kNKK];       // LDS byte address of this lane's K operand row in slot 0 of the ring
  uint32_t vaddr[kNDB];       // same for the V^T transpose reads
  float c;                    // |scale| log2(e)
  int last_key[2];            // highest visible key per half row (causal: the row; always < Nk)

  // K operand of slice kk of a 32-key sub-tile (byte address of its first row)
  __device__ __forceinline__ void load_k(int kk, uint32_t ksub) { ak[kk % 3] = lds_row16(ksub + kaddr[kk]); }
  // a sub-tile base address the compiler cannot take apart (one add per read)
  __device__ __forceinline__ static uint32_t opaque(uint32_t a) {
    a = __builtin_amdgcn_readfirstlane(a);
    asm volatile("" : "+s"(a));
    return a;
  }
  // V^T operand of phase-2 group gi: row block gi % 4 of 16-key group gi / 4
  __device__ __forceinline__ void load_v(int gi, uint32_t vsub) {
    const int kg = gi / kNDB, db = gi % kNDB;
    av[gi % 3] = tr_pair(vsub + vaddr[db] + (16 * kg) * kDV * 2, vsub + vaddr[db] + (16 * kg + 4) * kDV * 2);
  }

  __device__ __forceinline__ void apply_mask(int p, int h, int key0) {
    const int g = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int lim = last_key[h] - (key0 + 16 * hh + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[p][h][8 * hh + e] = e > lim ? -INFINITY : s[p][h][8 * hh + e];
    }
  }
  // Weight piece q (0 .. 7) of half h of the sub-tile of parity p: two
  // weights against the current reference and their sum; pieces 3 and 7
  // pack their 16-key group to bf16.  The empty asm keeps the sum where it
  // is computed: nothing in the loop reads it before commit(), and the
  // compiler otherwise sinks every piece's add past the loop's tile branches
  // into one burst of vector work with no product beside it.
  // MASKED: keys past the row's last visible key get weight 0; lim is that
  // key minus (first key of the sub-tile + 8 g), so register 8 kg + e (key
  // 16 kg + 8 g + e of the sub-tile) is visible iff 16 kg + e <= lim.
  template <bool MASKED = false>
  __device__ __forceinline__ void piece(int p, int h, int q, int lim = 0) {
    const int kg = q >> 2, e0 = 2 * (q & 3);
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e) {
      float x = s[p][h][8 * kg + e];
      if constexpr (MASKED) x = 16 * kg + e > lim ? -INFINITY : x;
      pf[h][kg][e] = fast_exp2(fmaf(x, c, -hs[h].m_use));
    }
    part[h][q] = pf[h][kg][e0] + pf[h][kg][e0 + 1];
    asm volatile("" : "+v"(part[h][q]));
    if ((q & 3) == 3) pb[p][h][kg] = pack_bf16x8(pf[h][kg]);
  }
  // The sub-tile's weights join the running sum (pairs, then pairs of
  // pairs: four weights, eight, sixteen).
  __device__ __forceinline__ void commit(int h) {
    hs[h].l += ((part[h][0] + part[h][1]) + (part[h][2] + part[h][3])) +
               ((part[h][4] + part[h][5]) + (part[h][6] + part[h][7]));
    asm volatile("" : "+v"(hs[h].l));
  }
  // The reference of half h: the exact row max of the (masked) sub-tile of
  // parity p.
  __device__ __forceinline__ void set_ref(int p, int h) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[p][h][i]);
    mx = halves_max(mx) * c;
    hs[h].m_ref = mx;
    hs[h].m_use = mx == -INFINITY ? 0.f : mx;
  }
  // The weights of one half outside the pipelined phases.
  __device__ __forceinline__ void softmax(int p, int h) {
    static_for<0, 8>([&](auto Q) { piece(p, h, decltype(Q)::value); });
    commit(h);
  }

  // Operand registers and the matrix core.  After every product, an empty
  // asm takes the product's result and reads the K / V^T / weight registers
  // the previous product read: those stay allocated (nothing is written into
  // them) until the next product has been issued.  Q is never written.
  __device__ __forceinline__ static void after(f32x16& acc, const bf16x8& prev) {
    asm volatile("" : "+a"(acc) : "v"(prev));
  }
  __device__ __forceinline__ static void after(f32x16& acc, const bf16x8& prev0, const bf16x8& prev1) {
    asm volatile("" : "+a"(acc) : "v"(prev0), "v"(prev1));
  }
  __device__ __forceinline__ static void anchor(f32x16& acc) { asm volatile("" : "+a"(acc)); }

  // Phase 1: S^T of the next sub-tile into s[pn] (both halves; slices 0 and 1
  // of it already loaded) beside the softmax of (current sub-tile, half 1).
  // Group kk: the two products of slice kk (one per half) share one K
  // operand; slice kk + 2 loads between them, into the slot group kk - 1
  // read; weight piece kk follows.  LOAD_V: the first two V^T operands of phase 2 load in the last
  // groups.  The product before the phase read av[1] and pb[pn][1][1] (the
  // last product of phase 2).
  template <bool WITH_SOFT, bool LOAD_V, bool MASKED = false>
  __device__ __forceinline__ void phase1(int pc, int pn, uint32_t ksub, uint32_t vsub, int lim = 0) {
    static_for<0, kNKK>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      s[pn][0] = mfma32(ak[kk % 3], qf[0][kk], kk == 0 ? f32x16{} : s[pn][0]);
      if constexpr (kk == 0) after(s[pn][0], av[1], pb[pn][1][1]);
      else after(s[pn][0], ak[(kk - 1) % 3]);
      if constexpr (kk + 2 < kNKK) load_k(kk + 2, ksub);
      if constexpr (LOAD_V && kk >= kNKK - 2) load_v(kk - (kNKK - 2), vsub);
      s[pn][1] = mfma32(ak[kk % 3], qf[1][kk], kk == 0 ? f32x16{} : s[pn][1]);
      anchor(s[pn][1]);
      if constexpr (WITH_SOFT) piece<MASKED>(pc, 1, kk, lim);
      sg<kSgMfma, 1>(); sg<kSgDsRead, 2>(); sg<kSgValu, 4>(); sg<kSgMfma, 1>(); sg<kSgValu, 30>();
      group_fence();
    });
  }

  // Phase 2: O^T += V^T P^T of the current sub-tile (both halves; groups 0
  // and 1 already loaded) beside the softmax of (next sub-tile, half 0).
  // Group gi: row block gi % 4 of 16-key group gi / 4, two products (one per
  // half) sharing one V^T operand; group gi + 2 loads between them; weight
  // pieces 0 and 1 follow group 1, piece gi follows group gi >= 2 (S of the
  // next sub-tile is not read right after its last product).  NEXT_K:
  // slices 0 and 1 of the sub-tile after next load in the last groups.  The
  // product before the phase read ak[1] (and Q).
  template <bool WITH_SOFT, bool NEXT_K, bool MASKED = false>
  __device__ __forceinline__ void phase2(int pc, int pn, uint32_t vsub, uint32_t knext, int lim = 0) {
    static_for<0, 2 * kNDB>([&](auto GI) {
      constexpr int gi = decltype(GI)::value;
      constexpr int kg = gi / kNDB, db = gi % kNDB;
      o[0][db] = mfma32(av[gi % 3], pb[pc][0][kg], o[0][db]);
      if constexpr (gi == 0) after(o[0][db], ak[1]);
      else after(o[0][db], av[(gi - 1) % 3], pb[pc][1][(gi - 1) / kNDB]);
      if constexpr (gi + 2 < 2 * kNDB) load_v(gi + 2, vsub);
      if constexpr (NEXT_K && gi >= 2 * kNDB - 2) load_k(gi - (2 * kNDB - 2), knext);
      o[1][db] = mfma32(av[gi % 3], pb[pc][1][kg], o[1][db]);
      after(o[1][db], pb[pc][0][kg]);
      if constexpr (WITH_SOFT && gi == 1) {
        piece<MASKED>(pn, 0, 0, lim);
        piece<MASKED>(pn, 0, 1, lim);
      }
      if constexpr (WITH_SOFT && gi >= 2) piece<MASKED>(pn, 0, gi, lim);
      sg<kSgMfma, 1>(); sg<kSgDsRead, 2>(); sg<kSgValu, 4>(); sg<kSgMfma, 1>(); sg<kSgValu, 30>();
      group_fence();
    });
  }
};

template <bool CAUSAL, int SPLIT>
__global__ __launch_bounds__(kThreads, 1) void fwd_r64_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Nq, int Nk, int n_qblk, int total, float c_in,
    Seqs seqs, Strides lay) {
  constexpr int RG = kWaves / SPLIT;  // row groups
  constexpr int RW = 64 * RG;         // query rows per workgroup
  __shared__ __attribute__((aligned(16))) Smem<SPLIT> sm;

  int bh, qb;
  if (CAUSAL || seqs.cu) {
    if ((int)blockIdx.x >= total) return;
    causal_order(blockIdx.x, total / n_qblk, n_qblk, kAllHeads, qb, bh);
    if (CAUSAL) qb = n_qblk - 1 - qb;  // longest rows first
  } else {
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    if (blk >= total) return;
    bh = blk / n_qblk;
    qb = blk - bh * n_qblk;
  }
  size_t q_row0 = (size_t)bh * Nq;
  const bf16_raw *Qh, *Kh, *Vh;
  int q_stride, k_stride, v_stride;
  if (seqs.cu) {
    const int b = bh / seqs.H, h = bh - b * seqs.H;
    int s0, s1;
    seq_range(seqs, b, s0, s1);
    Nq = Nk = s1 - s0;
    q_row0 = (size_t)h * seqs.total + s0;
    if (qb * RW >= Nq) return;  // past the end of a shorter sequence
    Qh = Q + q_row0 * kD;
    Kh = K + q_row0 * kD;
    Vh = V + q_row0 * kDV;
    q_stride = k_stride = kD;
    v_stride = kDV;
  } else {
    const int b = bh / lay.H, h = bh - b * lay.H;
    Qh = Q + (size_t)(b * lay.qb + h * lay.qh);
    Kh = K + (size_t)(b * lay.kb + h * lay.kh);
    Vh = V + (size_t)(b * lay.vb + h * lay.vh);
    q_stride = lay.qr;
    k_stride = lay.kr;
    v_stride = lay.vr;
  }

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-level quantities in scalar registers, so every branch on them is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RG, kr = wave / RG;
  const int g = lane >> 5, col = lane & 31;

  const int q_start = qb * RW;
  const int r0 = q_start + 64 * rg;  // this wave's first row

  // LDS tiles of the workgroup (cut at the causal diagonal of its last row)
  // and of this wave's key range; sub-tiles (32 keys) this wave computes, and
  // how many of them need no mask (every key visible to every row of the wave)
  const int kv_end = CAUSAL ? min(Nk, q_start + RW) : Nk;
  const int n_tiles = (kv_end + kBC - 1) / kBC;
  const int n_iter = (n_tiles + SPLIT - 1) / SPLIT;
  const int ra = kr * n_iter;
  const int rb = min(n_tiles, ra + n_iter);
  const int key_a = ra * kBC;  // first key of the range
  int n_w = 0, n_clean = 0;
  if (r0 < Nq && ra < rb) {
    const int vis_end = min(CAUSAL ? min(Nk, r0 + 64) : Nk, rb * kBC);  // keys some row of the wave sees
    n_w = max((vis_end - key_a + kSub - 1) / kSub, 0);
    const int clean_end = min(CAUSAL ? min(Nk, r0 + 1) : Nk, rb * kBC);  // keys every row of the wave sees
    n_clean = min(max((clean_end - key_a) / kSub, 0), n_w);
  }

  Wave w;
  const uint32_t k_row = (uint32_t)k_stride * 2u, v_row = (uint32_t)v_stride * 2u;
  Copy<RG> cp;
  cp.init(rg, lane, k_row, v_row);
  // LDS byte addresses of this range's rings (vector and scalar copies)
  const uint32_t kring = lds_addr_of(sm.k[kr][0]), vring = lds_addr_of(sm.v[kr][0]);
  bf16_raw(*ks_s)[kBC * kD] = sm.k[kr];
  bf16_raw(*vs_s)[kBC * kDV] = sm.v[kr];
  constexpr uint32_t kTileBytes = kBC * kD * 2, vTileBytes = kBC * kDV * 2, kSubBytes = kSub * kD * 2;
  // K sub-tile t of the range sits in slot (t / 2) % 3, rows 32 (t % 2) ..
  // (byte offsets from the ring's first slot; the lane's operand addresses
  // carry the ring base)
  constexpr int kVSlots = Smem<SPLIT>::kVSlots;
  auto ksub_addr = [&](int t) {
    return Wave::opaque((uint32_t)((t >> 1) % kKSlots) * kTileBytes + (uint32_t)(t & 1) * kSubBytes);
  };
  auto vsub_addr = [&](int t) {
    return Wave::opaque((uint32_t)((t >> 1) % kVSlots) * vTileBytes + (uint32_t)(t & 1) * kSubBytes);
  };

  // prologue copies: K(0), V(0), K(1) of the range
  auto first_copies = [&]() {
    if (ra < rb) {
      issue_tile<RG, true>(ks_s[0], Kh, Nk, key_a, k_row, cp, rg);
      issue_tile<RG, false>(vs_s[0], Vh, Nk, key_a, v_row, cp, rg);
    }
    if (ra + 1 < rb) issue_tile<RG, true>(ks_s[1], Kh, Nk, key_a + kBC, k_row, cp, rg);
  };
  first_copies();

  // scale sign folded into Q (exact: a sign flip of bf16), c = |scale| log2 e
  w.c = fabsf(c_in);
  const uint32_t qsign = c_in < 0.f ? 0x80008000u : 0u;
  // All of the wave's Q loads are issued before any is moved: a move right
  // behind its load waits for it, and sixteen such waits in a row cost
  // sixteen memory round trips before the first product.
  uint4 xq[2][kNKK];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int qr = min(r0 + 32 * h + col, Nq - 1);
#pragma unroll
    for (int kk = 0; kk < kNKK; ++kk) xq[h][kk] = ld16(Qh + (size_t)qr * q_stride + 16 * kk + 8 * g);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int kk = 0; kk < kNKK; ++kk) {
      uint4 x = xq[h][kk];
      x.x ^= qsign; x.y ^= qsign; x.z ^= qsign; x.w ^= qsign;
      w.qf[h][kk] = as_bf16x8(x);
      // Q stays in AGPRs for the whole kernel (the matrix core reads its B
      // operand there), leaving the VGPRs to the softmax and operand rings
      asm volatile("" : "+a"(w.qf[h][kk]));
    }
    w.last_key[h] = CAUSAL ? min(r0 + 32 * h + col, Nk - 1) : Nk - 1;
    w.hs[h] = Half{-INFINITY, 0.f, 0.f};
  }
#pragma unroll
  for (int kk = 0; kk < kNKK; ++kk) w.kaddr[kk] = kring + (uint32_t)(col * kD * 2 + 16 * ((2 * kk + g) ^ kswz(col)));
  {
    const int grp = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int db = 0; db < kNDB; ++db) {
      const int krow = 8 * (grp >> 1) + (sl >> 2);
      const int d = 32 * db + 16 * (grp & 1) + 4 * (sl & 3);
      w.vaddr[db] = vring + (uint32_t)(krow * kDV * 2 + 16 * ((d >> 3) ^ vswz(krow)) + 2 * (d & 7));
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) w.ak[j] = w.av[j] = bf16x8{};
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kg = 0; kg < kNKG; ++kg) w.pb[p][h][kg] = bf16x8{};

  // The reference of each row is the exact max of its first sub-tile and
  // stays there: no per-tile max, no rescale of O.  Weights of later keys
  // may then exceed 1; in float32 that is harmless unless some weight or O
  // element overflows, which the check after the loop sees (a non-finite
  // sum).  Then the whole workgroup starts again with the exact row max over
  // every key of the range (a separate pass over K), for which no weight
  // exceeds 1.
  bool exact_ref = false;
#pragma clang loop unroll(disable)
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w.hs[h].l = 0.f;
#pragma unroll
      for (int db = 0; db < kNDB; ++db) w.o[h][db] = f32x16{};
    }
    wait_loads();
    __syncthreads();
    // prologue compute: S of sub-tile 0, the references, the softmax of
    // (0, h0), slices 0 and 1 of sub-tile 1
    if (n_w > 0) {
      w.load_k(0, ksub_addr(0));
      w.load_k(1, ksub_addr(0));
      w.template phase1<false, false>(0, 0, ksub_addr(0), 0u);
      if (n_clean == 0) {
        w.apply_mask(0, 0, key_a);
        w.apply_mask(0, 1, key_a);
      }
      if (!exact_ref) {
        w.set_ref(0, 0);
        w.set_ref(0, 1);
      }
      w.softmax(0, 0);
      // the products of S(0) have completed (their results are read) before
      // their K operand slots are refilled
      pin(w.ak[0], w.s[0][1][15] + w.s[0][0][15]);
      pin(w.ak[1], w.s[0][1][15] + w.s[0][0][15]);
      pin(w.ak[2], w.s[0][1][15] + w.s[0][0][15]);
      if (n_w > 1) {
        w.load_k(0, ksub_addr(1));
        w.load_k(1, ksub_addr(1));
      }
    }

    // LDS tile u: K(u+1) and V(u) resident; refill the slots of K(u-1) and V(u-1)
    auto top = [&](int u) {
      wait_loads();
      __syncthreads();
      if (ra + u + 2 < rb)
        issue_tile<RG, true>(ks_s[(u + 2) % kKSlots], Kh, Nk, key_a + (u + 2) * kBC, k_row, cp, rg);
      if (ra + u + 1 < rb)
        issue_tile<RG, false>(vs_s[(u + 1) % kVSlots], Vh, Nk, key_a + (u + 1) * kBC, v_row, cp, rg);
    };
    // Steady state, two sub-tiles (one LDS tile) per iteration: every
    // sub-tile involved is mask-free and the next one exists.  Slices 0, 1 of
    // sub-tile v + 2 are loaded ahead even when it does not exist (an in-range
    // LDS read whose value is never used).
    auto fast_step_at = [&](auto P, uint32_t k_next, uint32_t v_cur, uint32_t k_after) {
      constexpr int pc = decltype(P)::value, pn = 1 - pc;
      w.template phase1<true, true>(pc, pn, k_next, v_cur);
      w.commit(1);
      w.template phase2<true, true>(pc, pn, v_cur, k_after);
      w.commit(0);
    };
    auto fast_step = [&](auto P, int v) { fast_step_at(P, ksub_addr(v + 1), vsub_addr(v), ksub_addr(v + 2)); };
    int u = 0;
    {
      // TPI LDS tiles per iteration from u = 0, a multiple of both ring
      // sizes: tile u + i sits in slot i % 3 of the K ring and i % kVSlots of
      // the V ring, so every operand address is a lane register plus an
      // immediate offset (no address arithmetic in the loop).
      constexpr int TPI = kVSlots == kKSlots ? kKSlots : kKSlots * kVSlots;
      constexpr auto koff = [](int j) {
        return (uint32_t)(((j >> 1) % kKSlots) * (int)kTileBytes + (j & 1) * (int)kSubBytes);
      };
      constexpr auto voff = [](int j) {
        return (uint32_t)(((j >> 1) % kVSlots) * (int)vTileBytes + (j & 1) * (int)kSubBytes);
      };
      for (; 2 * u + 2 * TPI < n_clean; u += TPI) {
        static_for<0, TPI>([&](auto I) {
          constexpr int i = decltype(I)::value;
          top(u + i);
          fast_step_at(ic<0>{}, koff(2 * i + 1), voff(2 * i), koff(2 * i + 2));
          fast_step_at(ic<1>{}, koff(2 * i + 2), voff(2 * i + 1), koff(2 * i + 3));
        });
      }
    }
    for (; 2 * u + 2 < n_clean; ++u) {
      top(u);
      fast_step(ic<0>{}, 2 * u);
      fast_step(ic<1>{}, 2 * u + 1);
    }
    // The last sub-tiles of the wave (masks; possibly no next sub-tile) and
    // the iterations a wave only helps with copies.  Masks are selects in the
    // weight pieces, on the values as they leave the accumulators (a clean
    // sub-tile masks nothing); S of a missing next sub-tile is computed from a
    // resident tile and its weights are never committed.
    auto tail_step = [&](auto P, int v) {
      constexpr int pc = decltype(P)::value, pn = 1 - pc;
      const bool has_next = v + 1 < n_w;
      const int vn = has_next ? v + 1 : v;
      const int g8 = 8 * ((threadIdx.x >> 5) & 1);
      w.template phase1<true, true, true>(pc, pn, ksub_addr(vn), vsub_addr(v), w.last_key[1] - (key_a + v * kSub + g8));
      w.commit(1);
      w.template phase2<true, true, true>(pc, pn, vsub_addr(v), ksub_addr(has_next ? v + 2 : v),
                                          w.last_key[0] - (key_a + vn * kSub + g8));
      if (has_next) w.commit(0);
    };
    for (; u < n_iter; ++u) {
      top(u);
      if (2 * u < n_w) tail_step(ic<0>{}, 2 * u);
      if (2 * u + 1 < n_w) tail_step(ic<1>{}, 2 * u + 1);
    }
    if (exact_ref) break;

    // the check: a non-finite running sum or O element in any wave
    float chk[kNDB];
#pragma unroll
    for (int db = 0; db < kNDB; ++db) chk[db] = db == 0 ? w.hs[0].l + w.hs[1].l : 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) chk[db] += w.o[h][db][i];
    const float tot = (chk[0] + chk[1]) + (chk[2] + chk[3]);
    const bool bad = __any(!(fabsf(tot) <= 3.0e38f));
    // the flags go through the first K slot once every wave is done with it
    int* redo = reinterpret_cast<int*>(&sm.k[0][0][0]);
    __syncthreads();
    if (lane == 0) redo[wave] = bad ? 1 : 0;
    __syncthreads();
    const int any_bad = __builtin_amdgcn_readfirstlane(redo[0] | redo[1] | redo[2] | redo[3]);
    if (!any_bad) break;

    // The exact row max over the range, S recomputed from K in global memory
    // (rows of the operand in the order the LDS tiles hold them).
    float mx[2] = {-INFINITY, -INFINITY};
    for (int t = 0; t < n_w; ++t) {
      const int key0 = key_a + t * kSub;
      const int key = min(key0 + perm32(col), Nk - 1);
      const bf16_raw* kp = Kh + (size_t)key * k_stride + 8 * g;
      bf16x8 kf[kNKK];
#pragma unroll
      for (int kk = 0; kk < kNKK; ++kk) kf[kk] = as_bf16x8(ld16(kp + 16 * kk));
      f32x16 a0{}, a1{};
#pragma unroll
      for (int kk = 0; kk < kNKK; ++kk) {
        a0 = mfma32(kf[kk], w.qf[0][kk], a0);
        a1 = mfma32(kf[kk], w.qf[1][kk], a1);
      }
      w.s[0][0] = a0;
      w.s[0][1] = a1;
      w.apply_mask(0, 0, key0);
      w.apply_mask(0, 1, key0);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx[h] = fmaxf(mx[h], w.s[0][h][i]);
      // the products have completed before their operand registers are reused
      const float z = a0[15] + a1[15];
#pragma unroll
      for (int kk = 0; kk < kNKK; ++kk) pin(kf[kk], z);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float m = halves_max(mx[h]) * w.c;
      w.hs[h].m_ref = m;
      w.hs[h].m_use = m == -INFINITY ? 0.f : m;
    }
    exact_ref = true;
    __syncthreads();  // every wave has read the flags before the rings refill
    first_copies();
  }

  if constexpr (SPLIT == 2) {
    // merge the second key range into the first: with m = max(m0, m1),
    // O = 2^(m0-m) O0 + 2^(m1-m) O1, l = 2^(m0-m) l0 + 2^(m1-m) l1 (a range
    // that saw no key has m = -inf and weight 0)
    constexpr int NV = 2 * (kNDB * 16 + 2);  // floats per lane: O^T, m, l of both halves
    __syncthreads();  // every wave is done with the tiles
    float* xch = reinterpret_cast<float*>(&sm.k[0][0][0]) + (size_t)rg * NV * 64;
    if (kr == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float* x = xch + h * (NV / 2) * 64;
#pragma unroll
        for (int db = 0; db < kNDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) x[(db * 16 + i) * 64 + lane] = w.o[h][db][i];
        x[(kNDB * 16) * 64 + lane] = w.hs[h].m_ref;
        x[(kNDB * 16 + 1) * 64 + lane] = w.hs[h].l;
      }
    }
    __syncthreads();
    if (kr == 1) return;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* x = xch + h * (NV / 2) * 64;
      const float m1 = x[(kNDB * 16) * 64 + lane];
      const float m = fmaxf(w.hs[h].m_ref, m1);
      const float a0 = m == -INFINITY ? 0.f : fast_exp2(w.hs[h].m_ref - m);
      const float a1 = m == -INFINITY ? 0.f : fast_exp2(m1 - m);
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) w.o[h][db][i] = a0 * w.o[h][db][i] + a1 * x[(db * 16 + i) * 64 + lane];
      w.hs[h].l = a0 * w.hs[h].l + a1 * x[(kNDB * 16 + 1) * 64 + lane];
      w.hs[h].m_ref = m;
    }
  }

  // epilogue: combine the two half-row sums, normalise once, write O and L
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float l_tot = halves_sum(w.hs[h].l);
    const int my_q = r0 + 32 * h + col;
    if (my_q < Nq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* Orow = O + (q_row0 + my_q) * kDV;
#pragma unroll
      for (int db = 0; db < kNDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          float4 v;
          v.x = w.o[h][db][4 * i4 + 0] * inv;
          v.y = w.o[h][db][4 * i4 + 1] * inv;
          v.z = w.o[h][db][4 * i4 + 2] * inv;
          v.w = w.o[h][db][4 * i4 + 3] * inv;
          *reinterpret_cast<float4*>(Orow + 32 * db + 8 * i4 + 4 * g) = v;
        }
      if (g == 0) LSE[q_row0 + my_q] = l_tot > 0.f ? (w.hs[h].m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <bool CAUSAL, int SPLIT>
hipError_t launch_split(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq, int Nk,
                        float c, const Seqs& seqs, const Strides& lay, hipStream_t stream) {
  constexpr int RW = 64 * (kWaves / SPLIT);
  const int n_qblk = (Nq + RW - 1) / RW;
  const long long total = (long long)BH * n_qblk;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((fwd_r64_kernel<CAUSAL, SPLIT>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                     static_cast<const bf16_raw*>(v), o, lse, BH, Nq, Nk, n_qblk, (int)total, c, seqs, lay);
  return hipGetLastError();
}

}  // namespace

bool fwd_r64_applies(int d, int dv) { return d == kD && dv == kDV; }

hipError_t launch_fwd_r64(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq, int Nk,
                          int causal, float scale, const Seqs* seqs, const Strides& lay, hipStream_t stream) {
  const Seqs sq = seqs ? *seqs : Seqs{nullptr, 0, 0};
  const float c = scale * kLog2e;
  // fewer 256-row workgroups than compute units: two key ranges per workgroup
  const long long wgs = (long long)BH * ((Nq + 255) / 256);
  const bool split = wgs < kComputeUnits && Nk > 2 * kBC;
  if (causal)
    return split ? launch_split<true, 2>(q, k, v, o, lse, BH, Nq, Nk, c, sq, lay, stream)
                 : launch_split<true, 1>(q, k, v, o, lse, BH, Nq, Nk, c, sq, lay, stream);
  return split ? launch_split<false, 2>(q, k, v, o, lse, BH, Nq, Nk, c, sq, lay, stream)
               : launch_split<false, 1>(q, k, v, o, lse, BH, Nq, Nk, c, sq, lay, stream);
}

}  // namespace fa

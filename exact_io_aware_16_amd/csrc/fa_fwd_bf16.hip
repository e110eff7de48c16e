// Exact attention forward, bf16 inputs, float32 outputs, gfx950 matrix cores.
//
// The blocked computation of "From softmax to attention: rescale the output
// too" (FlashAttention: The Matrix You Never Have to Write Down): per query
// row a running sum l and unnormalised output O over the key tiles, both
// against a reference m, and one division of O by l after the last tile.
// Scores never leave the chip.
//
// Reference of the exponentials: any common reference per row gives the same
// O / l and L = m + log l (the identity the recurrence rests on); the max
// only keeps the terms in range.  The FA4 paragraph under "What it doesn't
// solve" on the same page defers the rescale until the max has moved far;
// this kernel defers it to the end.  Each row's reference is the exact max
// of the first key tile its wave computes and never moves: no per-tile max,
// no rescale.  Later weights may exceed 1; float32 holds them unless a
// weight, a sum or an O element overflows, and a check after the loop sees
// exactly that (a non-finite value).  Then the workgroup runs again with the
// exact row max over all of its keys as the reference (a pass over K in
// global memory), the page's own frame, in which no weight exceeds 1.  A
// row's visible keys are a prefix of the range (the causal mask and the end
// of the sequence only hide later keys), so a row that sees nothing in its
// wave's first tile sees nothing at all.
//
// Contract (the first page's flash_attention, "Build it"): Q [Nq, d],
// K [Nk, d], V [Nk, dv] per head; O [Nq, dv]; upper-left causal masking
// (key j visible to query i iff j <= i); no keys gives O = 0, L = -inf.
//
// Work split (one workgroup = 4 waves = 128 query rows of one head):
//  * each wave owns 32 query rows; its Q block stays in registers for the
//    whole kernel as the B operand of S^T = K Q^T (keys along M, queries
//    along N), so a query's scores sit in one lane pair (lanes c, c+32) and
//    the row max needs one cross-half exchange;
//  * K and V tiles (BC keys) are copied global -> LDS directly
//    (global_load_lds, 16 bytes per lane, no register staging), double
//    buffered, with a 16-byte-slot XOR swizzle instead of padding:
//      K: row r holds key perm32(r), slot (chunk ^ (r & 7))
//      V: row r holds key r,         slot (chunk ^ 2*(r & 3))
//    so operand reads are bank-conflict free;
//  * V stays row-major: the O^T += V^T P^T operand is read with
//    ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one
//    head-dimension column;
//  * P is rounded to bf16 in registers and used directly as the B operand
//    (the perm32 key order makes the S result layout equal to the operand
//    layout);
//  * two waves per SIMD hide each other's softmax behind matrix-core work:
//    two 4-wave workgroups per CU when the grid is large enough, otherwise
//    one 8-wave workgroup whose two halves take half of the key tiles each
//    (split-KV inside the workgroup, merged through LDS at the end);
//  * causal: query block qb visits key tiles up to its diagonal only, masks
//    are applied only on tiles that straddle the diagonal or the ragged end.
#include <algorithm>

#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;        // query rows per workgroup
constexpr int kComputeUnits = 256;      // MI355X

// keys per tile: 128 when both widths are 64, else 64 (two buffers of K and V
// per key range fit in 64 KiB either way)
template <int D, int DV>
struct FwdTile {
  static constexpr int BC = (D == 64 && DV == 64) ? 128 : 64;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// SPLIT key ranges per workgroup, each with its own double-buffered tiles
template <int D, int DV, int SPLIT>
struct FwdSmem {
  static constexpr int BC = FwdTile<D, DV>::BC;
  bf16_raw k[SPLIT][2][BC * D];
  bf16_raw v[SPLIT][2][BC * DV];
};

// LDS tile layout.  Each BC x D bf16 tile is stored densely, row by row,
// in 16-byte slots; a slot's position is XOR-swizzled so that the operand
// reads hit 64 distinct banks per 16-lane phase (rows of 256 B span the whole
// bank width for d = 128, rows of 128 B span half of it for d = 64):
//   K tile: row r holds key perm32(r) (within each 32-row group), chunk c of
//           the row sits in slot c ^ kswz(r)
//   V tile: row r holds key r, chunk c sits in slot c ^ vswz(r)
template <int D>
__device__ __forceinline__ constexpr int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int DV>
__device__ __forceinline__ constexpr int vswz(int r) {
  return DV == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Per-lane byte offsets of the 16-byte chunks one thread copies for a tile
// (relative to the tile's first key).  The copy is an LDS-direct buffer load:
// lane l of an instruction writes LDS bytes [m0 + 16 l, m0 + 16 l + 16), so
// the swizzle is applied on the source side, and offsets past the end of the
// head (the ragged last tile) read as zeros -- nothing outside the head is
// ever read.
template <int D, int DV>
struct TileCopy {
  static constexpr int BC = FwdTile<D, DV>::BC;
  static constexpr int KSLOTS = D / 8, VSLOTS = DV / 8;
  static constexpr int KINSTR = BC * KSLOTS / kThreads, VINSTR = BC * VSLOTS / kThreads;
  uint32_t k_off[KINSTR], v_off[VINSTR];
  uint32_t k_row, v_row;  // bytes between consecutive K / V rows in global memory

  __device__ __forceinline__ void init(int wave, int lane, int k_stride, int v_stride) {
    k_row = (uint32_t)k_stride * 2u;
    v_row = (uint32_t)v_stride * 2u;
#pragma unroll
    for (int i = 0; i < KINSTR; ++i) {
      const int r = (i * kWaves + wave) * (64 / KSLOTS) + lane / KSLOTS;
      const int slot = lane % KSLOTS;
      k_off[i] = (uint32_t)((r & ~31) + perm32(r & 31)) * k_row + (uint32_t)(16 * (slot ^ kswz<D>(r)));
    }
#pragma unroll
    for (int i = 0; i < VINSTR; ++i) {
      const int r = (i * kWaves + wave) * (64 / VSLOTS) + lane / VSLOTS;
      const int slot = lane % VSLOTS;
      v_off[i] = (uint32_t)r * v_row + (uint32_t)(16 * (slot ^ vswz<DV>(r)));
    }
  }
};

// One 16-byte-per-lane LDS-direct load.  Issued as inline assembly so that
// the compiler does not serialise every later LDS read behind it (it cannot
// tell which LDS bytes the copy writes); completion is awaited explicitly
// with wait_tile_loads() before the barrier that publishes the tile.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                           uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr)
               : "memory");
}
// vmcnt(0) as the compiler's own wait instruction (vmcnt 0, expcnt 7,
// lgkmcnt 15 in the gfx9 encoding), so its wait-count tracking knows that
// every earlier vector memory load has completed and adds no wait of its
// own for registers loaded before (an asm wait is opaque to it, and it then
// kept a vmcnt(0) in every iteration, which also waited for the copies just
// issued for the next tile); the empty asm keeps memory accesses in place.
__device__ __forceinline__ void wait_tile_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One K and one V tile (BC keys from key0) of a head.  The descriptors start
// at the tile's first row and span the rest of the head, so the lane offsets
// stay loop invariant and the hardware range check still zeroes reads past
// the head's last key; the scalar offset stays 0.
template <int D, int DV>
__device__ __forceinline__ void issue_tiles(bf16_raw* k_tile, bf16_raw* v_tile, const bf16_raw* Kh,
                                            const bf16_raw* Vh, int Nk, int key0, const TileCopy<D, DV>& tc,
                                            int wave) {
  key0 = __builtin_amdgcn_readfirstlane(key0);  // wave-uniform: scalar arithmetic
  const uint32_t kb0 = (uint32_t)key0 * tc.k_row, vb0 = (uint32_t)key0 * tc.v_row;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)Kh + kb0), (short)0, (int)((uint32_t)Nk * tc.k_row - kb0), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)Vh + vb0), (short)0, (int)((uint32_t)Nk * tc.v_row - vb0), 0x00020000);
  const uint32_t kbase = lds_addr_of(k_tile), vbase = lds_addr_of(v_tile);
#pragma unroll
  for (int i = 0; i < TileCopy<D, DV>::KINSTR; ++i)
    lds_copy16(krs, tc.k_off[i], 0u, kbase + (uint32_t)(i * kWaves + wave) * 1024u);
#pragma unroll
  for (int i = 0; i < TileCopy<D, DV>::VINSTR; ++i)
    lds_copy16(vrs, tc.v_off[i], 0u, vbase + (uint32_t)(i * kWaves + wave) * 1024u);
}

// S^T (BC keys x 32 queries) = K Q^T from one LDS K tile.  kaddr[kk] is the
// lane's byte offset of its 16-byte operand for head-dim slice kk in key
// block 0; key block kb adds the constant 32 * kb rows.  K operands rotate
// through the two sets of ak (see pin()), loaded one group ahead; the set
// used last stays live for the caller to release once the scores have been
// consumed.
template <int D, int BC>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[BC / 32], const char* ktile, const int (&kaddr)[D / 16],
                                            const bf16x8 (&qf)[D / 16], bf16x8 (&ak)[2][BC / 32]) {
  constexpr int NKB = BC / 32;
  constexpr int NKK = D / 16;
  // the next group's operands load while this group's products run
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) ak[0][kb] = as_bf16x8(ld16(ktile + kaddr[0] + kb * 32 * D * 2));
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(ak[kk & 1][kb], qf[kk], kk == 0 ? f32x16{} : s[kb]);
    // group kk is issued: the other set (group kk-1) may be overwritten from here on
    group_fence();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) pin(ak[(kk + 1) & 1][kb]);
    if (kk + 1 < NKK)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) ak[(kk + 1) & 1][kb] = as_bf16x8(ld16(ktile + kaddr[kk + 1] + kb * 32 * D * 2));
  }
}

// SPLIT = 1: 4 waves, all keys.  SPLIT = 2 (split-KV inside the workgroup,
// for grids too small to give every SIMD two waves): 8 waves, waves 4h .. 4h+3
// take the h-th half of the key tiles for the same 128 query rows, and the
// two partial (m, l, O) are merged through LDS at the end with the
// logsumexp identity of "The identity" (FlashAttention: The Matrix You Never
// Have to Write Down), the same merge Flash-Decoding applies across
// workgroups ("What it doesn't solve").
//
// Key ranges across workgroups (Flash-Decoding, "What it doesn't solve"):
// with n_ksplit > 1 the key tiles are cut into n_ksplit contiguous ranges of
// tiles_per_split tiles; workgroup (head, query block, range ks) writes the
// range's own normalised output and logsumexp to O + ks * BH*Nq*DV and
// LSE + ks * BH*Nq, and splitkv_merge_kernel combines the ranges.
template <int D, int DV, bool CAUSAL, int SPLIT, bool DROP>
__global__ __launch_bounds__(kThreads * SPLIT, SPLIT == 1 ? 2 : 1) void fwd_bf16_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Nq, int Nk, int n_qblk, int n_ksplit,
    int tiles_per_split, int total, float c, Dropout dp, Seqs seqs, Strides lay) {
  constexpr int BC = FwdTile<D, DV>::BC;
  constexpr int NKB = BC / 32;   // 32-key blocks per tile
  constexpr int NKK = D / 16;    // 16-wide slices of the head dimension
  constexpr int NDB = DV / 32;   // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) FwdSmem<D, DV, SPLIT> sm;

  const int per_head = n_qblk * n_ksplit;
  int bh, rem;
  if (CAUSAL || seqs.cu) {
    if ((int)blockIdx.x >= total) return;
    causal_order(blockIdx.x, total / per_head, per_head, 2, rem, bh);
  } else {
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    if (blk >= total) return;
    bh = blk / per_head;
    rem = blk - bh * per_head;
  }
  int qb = rem / n_ksplit;
  const int ks = rem - qb * n_ksplit;
  if (CAUSAL) qb = n_qblk - 1 - qb;  // longest rows first
  // first rows of this head in Q, in K / V and in O / L; for packed
  // sequences, of sequence b = bh / H in head h = bh % H (then Nq = Nk is
  // that sequence's length and n_qblk covers the longest one)
  size_t q_row0 = (size_t)bh * Nq, k_row0 = (size_t)bh * Nk, o_row0 = ((size_t)ks * BH + bh) * Nq;
  if (seqs.cu) {
    const int b = bh / seqs.H, h = bh - b * seqs.H;
    int s0, s1;
    seq_range(seqs, b, s0, s1);
    Nq = Nk = s1 - s0;
    q_row0 = k_row0 = o_row0 = (size_t)h * seqs.total + s0;
    if (qb * kBR >= Nq) return;  // past the end of a shorter sequence
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (tid >> 6) & (kWaves - 1);  // query wave: rows 32 wave .. + 31
  const int half = SPLIT == 1 ? 0 : (tid >> 8);  // key range of this wave
  const int g = lane >> 5, col = lane & 31;
  // this head's Q, K, V: packed sequences are dense rows of one head;
  // otherwise batch / head / row strides (dense tensors pass dense strides)
  const bf16_raw *Qh, *Kh, *Vh;
  int q_stride, k_stride, v_stride;
  if (seqs.cu) {
    Qh = Q + q_row0 * D;
    Kh = K + k_row0 * D;
    Vh = V + k_row0 * DV;
    q_stride = k_stride = D;
    v_stride = DV;
  } else {
    const int b = bh / lay.H, h = bh - b * lay.H;
    Qh = Q + (size_t)(b * lay.qb + h * lay.qh);
    Kh = K + (size_t)(b * lay.kb + h * lay.kh);
    Vh = V + (size_t)(b * lay.vb + h * lay.vh);
    q_stride = lay.qr;
    k_stride = lay.kr;
    v_stride = lay.vr;
  }

  const int q_start = qb * kBR;
  const int q0w = q_start + 32 * wave;
  const int my_q = q0w + col;

  // key tiles [ks_first, ks_end) of this workgroup: its key range, cut at
  // the causal diagonal of the query block
  const int kv_end = CAUSAL ? min(Nk, q_start + kBR) : Nk;
  const int ks_first = ks * tiles_per_split;
  const int ks_end = min((kv_end + BC - 1) / BC, ks_first + tiles_per_split);
  const int n_tiles = max(ks_end - ks_first, 0);
  // tiles [t_first, t_end) of this wave's half of it; every wave runs n_iter
  // iterations so that the workgroup barriers line up
  const int n_iter = (n_tiles + SPLIT - 1) / SPLIT;
  const int t_first = ks_first + half * n_iter;
  const int t_end = min(ks_first + n_tiles, t_first + n_iter);

  TileCopy<D, DV> tc;
  tc.init(wave, lane, k_stride, v_stride);
  // the wave index in a scalar register: the copies' LDS addresses (M0) are
  // then scalar arithmetic
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // prologue loads: first K and V tile of the range
  auto first_copies = [&]() {
    if (t_first < t_end) issue_tiles<D, DV>(sm.k[half][0], sm.v[half][0], Kh, Vh, Nk, t_first * BC, tc, wave_s);
  };
  first_copies();

  // loop-invariant lane parts of the LDS operand addresses (bytes)
  int kaddr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kaddr[kk] = col * D * 2 + 16 * ((2 * kk + g) ^ kswz<D>(col));
  const int grp = lane >> 4, sl = lane & 15;
  int vaddr[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int kr = 8 * (grp >> 1) + (sl >> 2);  // row within a 16-row slice (plus constants)
    const int d = 32 * db + 16 * (grp & 1) + 4 * (sl & 3);
    vaddr[db] = kr * DV * 2 + 16 * ((d >> 3) ^ vswz<DV>(kr)) + 2 * (d & 7);
  }

  // A negative scale is folded into Q (a bf16 sign flip is exact), so the
  // scores' row max times c = |scale| log2(e) is the max of the scaled row.
  bf16x8 qf[NKK];
  {
    const int qr = min(my_q, Nq - 1);
    const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 x = ld16(Qh + (size_t)qr * q_stride + 16 * kk + 8 * g);
      x.x ^= qsign;
      x.y ^= qsign;
      x.z ^= qsign;
      x.w ^= qsign;
      qf[kk] = as_bf16x8(x);
    }
    c = fabsf(c);
  }

  f32x16 oacc[NDB];
  float m_ref = -INFINITY, l_run = 0.f, l_rnd = 0.f;

  // operand register sets (see pin()): K operands of the score product and
  // V^T operands of the P V product, two sets each
  bf16x8 ak[2][NKB], av[2][NDB], pb[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) pb[kb][0] = pb[kb][1] = bf16x8{};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) ak[j][kb] = bf16x8{};
#pragma unroll
    for (int db = 0; db < NDB; ++db) av[j][db] = bf16x8{};
  }

  f32x16 s_cur[NKB];
  // One pass over the key tiles.  exact_ref: the reference is already set
  // (the exact max over the range); otherwise each wave's first tile sets it.
  auto run_pass = [&](bool exact_ref) {
    bool ref_set = exact_ref;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    l_run = 0.f;
    l_rnd = 0.f;
    for (int it = 0; it < n_iter; ++it) {
      const int t = t_first + it;
      const int key0 = t * BC;
      // K(t) and V(t) have landed (own loads) and are visible (barrier); every
      // wave is done with tile t-1, whose buffers refill now with tile t+1.
      wait_tile_loads();
      __syncthreads();
      if (t >= t_end) continue;  // the shorter key range idles through the barriers
      if (t + 1 < t_end)
        issue_tiles<D, DV>(sm.k[half][(it + 1) & 1], sm.v[half][(it + 1) & 1], Kh, Vh, Nk, key0 + BC, tc, wave_s);
      // a wave whose 32 rows all lie past the last query (few query rows, as in
      // decoding, or the ragged last block), or (causal) before the tile's
      // first key, only helps copy the tiles
      if (q0w >= Nq || (CAUSAL && key0 > q0w + 31)) continue;
      tile_scores<D, BC>(s_cur, reinterpret_cast<const char*>(sm.k[half][it & 1]), kaddr, qf, ak);

      const bool need_mask = (CAUSAL && key0 + BC - 1 > q0w) || key0 + BC > Nk;
      if (need_mask) {
        // register 8 h + e of half g holds key key0 + 32 kb + 16 h + 8 g + e;
        // keys above last_key (causal: the row; always: Nk - 1) are masked
        const int last_key = CAUSAL ? min(my_q, Nk - 1) : Nk - 1;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int lim = last_key - (key0 + 32 * kb + 16 * h + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) s_cur[kb][8 * h + e] = e > lim ? -INFINITY : s_cur[kb][8 * h + e];
          }
      }
      // the first tile this wave computes sets the reference: its exact row max
      // (both lane halves), in log2 units; -inf for a row that sees no key
      if (!ref_set) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
        m_ref = halves_max(mx) * c;
        ref_set = true;
      }
      // every score product of tile t has completed once mx exists (products
      // complete in order): so have all earlier products, and the K and V^T
      // operand sets of this and the previous tile may be reused
      float mx = s_cur[0][15];
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb) mx += s_cur[kb][15];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) pin(ak[j][kb], mx);
#pragma unroll
        for (int db = 0; db < NDB; ++db) pin(av[j][db], mx);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pin(pb[kb][0], mx);
        pin(pb[kb][1], mx);
      }
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;  // row with nothing visible yet

#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        // dropout mask words of this 32-key block: dm[x] is this row's word of
        // the 4 x 4 block holding keys 16 (x / 2) + 8 g + 4 (x % 2) .. + 3 (lane
        // x of the 4-lane group computes that block)
        uint32_t dm[4];
        if constexpr (DROP) {
          const int qd = col & 3;
          uint32_t w[4] = {(uint32_t)(key0 + 32 * kb + 16 * (qd >> 1) + 8 * g + 4 * (qd & 1)) >> 2,
                           (uint32_t)my_q >> 2, (uint32_t)bh, dp.offset};
          philox4x32_10(w, dp.k0, dp.k1);
          quad_transpose(w, dm, qd);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(s_cur[kb][8 * h + e], c, -m_use));
            l_run += p[e];
          }
          pb[kb][h] = pack_bf16x8(p);
          // l_rnd sums the bf16-rounded weights that actually multiply V, so O
          // is normalised by exactly the weights applied (a dominant weight's
          // rounding cancels in O / l_rnd); l_run (exact terms) gives L.  With
          // dropout both sums cover every weight; only the product with V
          // loses the dropped ones.
          l_rnd = sum_bf16x8(pb[kb][h], l_rnd);
          if constexpr (DROP) pb[kb][h] = drop_bf16x8(pb[kb][h], dm[2 * h], dm[2 * h + 1], dp.t);
        }
      }

      // O^T += V^T P^T, V^T operand via transpose reads of the row-major tile;
      // operand sets rotate per (key block, half) group
      const char* vtile = reinterpret_cast<const char*>(sm.v[half][it & 1]);
      // the other wave on this SIMD is usually in its softmax here: raised
      // issue priority keeps the matrix core fed through this product
      // (measured 2% on the forward workloads)
      __builtin_amdgcn_s_setprio(2);
      // V^T operands of group gi = (key block gi / 2, half gi % 2) into set gi % 2
      auto load_v = [&](int gi) {
        const int kb = gi >> 1, h = gi & 1;
        bf16x8(&a)[NDB] = av[gi & 1];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          v4i16 part[2];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr)
            part[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(vtile + vaddr[db] + (32 * kb + 16 * h + 4 * rr) * DV * 2));
          a[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      // the next group's operands load while this group's products run
      load_v(0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int grp_i = 2 * kb + h;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(av[grp_i & 1][db], pb[kb][h], oacc[db]);
          group_fence();
#pragma unroll
          for (int db = 0; db < NDB; ++db) pin(av[(grp_i + 1) & 1][db]);
          if (grp_i > 0) pin(pb[(grp_i - 1) >> 1][(grp_i - 1) & 1]);
          if (grp_i + 1 < 2 * NKB) load_v(grp_i + 1);
        }
      __builtin_amdgcn_s_setprio(0);
    }
  };
  run_pass(false);
  // The check: a non-finite running sum or O element in any wave of the
  // workgroup runs the pass again against the exact row max.
  do {
    float tot = l_run + l_rnd;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) tot += oacc[db][i];
    const bool bad = __any(!(fabsf(tot) <= 3.0e38f));
    // the flags go through the first K buffer once every wave is done with it
    int* redo = reinterpret_cast<int*>(&sm.k[0][0][0]);
    __syncthreads();
    if (lane == 0) redo[tid >> 6] = bad ? 1 : 0;
    __syncthreads();
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves * SPLIT; ++w) any_bad |= redo[w];
    if (!__builtin_amdgcn_readfirstlane(any_bad)) break;

    // The exact row max over the wave's tiles, S recomputed from K in global
    // memory (rows in the order the LDS tiles hold them, so the register
    // layout and the masks are those of the loop).
    float mx = -INFINITY;
    if (q0w < Nq) {
      const int last_key = CAUSAL ? min(my_q, Nk - 1) : Nk - 1;
      for (int t = t_first; t < t_end; ++t) {
        const int key0 = t * BC;
        if (CAUSAL && key0 > q0w + 31) break;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int key = min(key0 + 32 * kb + perm32(col), Nk - 1);
          const bf16_raw* kp = Kh + (size_t)key * k_stride + 8 * g;
          bf16x8 kf[NKK];
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) kf[kk] = as_bf16x8(ld16(kp + 16 * kk));
          f32x16 a{};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) a = mfma32(kf[kk], qf[kk], a);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int lim = last_key - (key0 + 32 * kb + 16 * h + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = e > lim ? mx : fmaxf(mx, a[8 * h + e]);
          }
          // the products have completed (their results are read) before the
          // next block's loads reuse the operand registers
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) pin(kf[kk], mx);
        }
      }
    }
    m_ref = halves_max(mx) * c;
    __syncthreads();  // every wave has read the flags before the tiles refill
    first_copies();
    run_pass(true);
  } while (false);

  if constexpr (SPLIT == 2) {
    // merge the second key range into the first: with m = max(m0, m1),
    // O = 2^(m0-m) O0 + 2^(m1-m) O1 and l = 2^(m0-m) l0 + 2^(m1-m) l1
    // (a range that saw no key has m = -inf and weight 0)
    constexpr int NV = NDB * 16 + 3;  // floats per lane: O^T, m, l_run, l_rnd
    float* xch = reinterpret_cast<float*>(&sm.k[0][0][0]) + (size_t)wave * NV * 64;
    __syncthreads();  // every wave is done with the tiles
    if (half == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(db * 16 + i) * 64 + lane] = oacc[db][i];
      xch[(NV - 3) * 64 + lane] = m_ref;
      xch[(NV - 2) * 64 + lane] = l_run;
      xch[(NV - 1) * 64 + lane] = l_rnd;
    }
    __syncthreads();
    if (half == 1) return;
    const float m1 = xch[(NV - 3) * 64 + lane];
    const float m = fmaxf(m_ref, m1);
    const float a0 = m == -INFINITY ? 0.f : fast_exp2(m_ref - m);
    const float a1 = m == -INFINITY ? 0.f : fast_exp2(m1 - m);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = a0 * oacc[db][i] + a1 * xch[(db * 16 + i) * 64 + lane];
    l_run = a0 * l_run + a1 * xch[(NV - 2) * 64 + lane];
    l_rnd = a0 * l_rnd + a1 * xch[(NV - 1) * 64 + lane];
    m_ref = m;
  }

  // epilogue: combine the two half-row sums, normalise once, write O and L
  // (of this workgroup's key range when the keys are split across workgroups)
  const float l_tot = halves_sum(l_run);
  const float l_nrm = halves_sum(l_rnd);
  if (my_q < Nq) {
    const float inv = l_nrm > 0.f ? (DROP ? dp.r : 1.f) / l_nrm : 0.f;
    float* Orow = O + (o_row0 + my_q) * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v;
        v.x = oacc[db][4 * i4 + 0] * inv;
        v.y = oacc[db][4 * i4 + 1] * inv;
        v.z = oacc[db][4 * i4 + 2] * inv;
        v.w = oacc[db][4 * i4 + 3] * inv;
        *reinterpret_cast<float4*>(Orow + 32 * db + 8 * i4 + 4 * g) = v;
      }
    if (g == 0) LSE[o_row0 + my_q] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merges n_split partial (O_s, L_s) of each query row (written by the
// forward with key ranges across workgroups) with the logsumexp identity:
// L = m + ln sum_s e^(L_s - m), O = sum_s e^(L_s - L) O_s; rows whose
// ranges all saw no key get O = 0, L = -inf.  One wave per row: lane s holds
// the weight of ranges s, s + 64, ...; the columns' sums over the ranges run
// with independent loads, so the merge costs a few memory round trips.
template <int DV>
__global__ __launch_bounds__(64) void splitkv_merge_kernel(const float* __restrict__ Opart,
                                                           const float* __restrict__ Lpart, float* __restrict__ O,
                                                           float* __restrict__ LSE, long long rows, int n_split) {
  constexpr int CPL = DV / 64;  // columns per lane
  const long long row = blockIdx.x;
  const int lane = threadIdx.x;
  float ls[4];  // n_split <= 256
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int sp = lane + 64 * r;
    ls[r] = sp < n_split ? Lpart[(size_t)sp * rows + row] : -INFINITY;
  }
  float m = fmaxf(fmaxf(ls[0], ls[1]), fmaxf(ls[2], ls[3]));
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
  float ws[4], den = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ws[r] = m == -INFINITY ? 0.f : __expf(ls[r] - m);
    den += ws[r];
  }
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) den += __shfl_xor(den, x);
  float acc[CPL];
#pragma unroll
  for (int cc = 0; cc < CPL; ++cc) acc[cc] = 0.f;
  constexpr int U = 8;
  for (int s0 = 0; s0 < n_split; s0 += U) {
    float part[U][CPL], w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, n_split - 1);
      w[u] = __shfl(ws[sp >> 6], sp & 63);
      if (s0 + u >= n_split) w[u] = 0.f;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) part[u][cc] = Opart[((size_t)sp * rows + row) * DV + lane + 64 * cc];
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) acc[cc] = fmaf(w[u], part[u][cc], acc[cc]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int cc = 0; cc < CPL; ++cc) O[(size_t)row * DV + lane + 64 * cc] = acc[cc] * inv;
  if (lane == 0) LSE[row] = den > 0.f ? m + __logf(den) : -INFINITY;
}

template <int D, int DV, bool CAUSAL, bool DROP>
hipError_t launch(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq, int Nk,
                  int n_ksplit, float* ws, float scale, const Dropout& dp, const Seqs& seqs, const Strides& lay,
                  bool dense, hipStream_t stream) {
  constexpr int BC = FwdTile<D, DV>::BC;
  const int n_qblk = (Nq + kBR - 1) / kBR;
  const int n_ktiles = (Nk + BC - 1) / BC;
  n_ksplit = max(1, min(n_ksplit, max(n_ktiles, 1)));
  const int tiles_per_split = n_ktiles == 0 ? 1 : (n_ktiles + n_ksplit - 1) / n_ksplit;
  n_ksplit = n_ktiles == 0 ? 1 : (n_ktiles + tiles_per_split - 1) / tiles_per_split;
  const long long total = (long long)BH * n_qblk * n_ksplit;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  float* o_dst = n_ksplit > 1 ? ws : o;
  float* l_dst = n_ksplit > 1 ? ws + (size_t)n_ksplit * BH * Nq * DV : lse;
  // Two 4-wave workgroups per CU keep two waves on every SIMD; a grid too
  // small for that (fewer than two workgroups per CU) splits each
  // workgroup's key tiles over 8 waves instead.
  const bool split = total < 2 * kComputeUnits && (n_ktiles + n_ksplit - 1) / n_ksplit > 1;
  // a few query rows against key ranges (decoding): the same ranges on the
  // vector ALUs, which stream K and V at close to HBM speed
  if (!DROP && dense && n_ksplit > 1 && !seqs.cu && decode_applies(Nq, D, DV)) {
    const hipError_t ed = launch_decode_bf16(q, k, v, o_dst, l_dst, BH, Nq, Nk, D, n_ksplit, tiles_per_split * BC,
                                             scale * kLog2e, CAUSAL ? 1 : 0, stream);
    if (ed != hipSuccess) return ed;
  } else if (split)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, CAUSAL, 2, DROP>), dim3(grid), dim3(2 * kThreads), 0, stream,
                       static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                       static_cast<const bf16_raw*>(v), o_dst, l_dst, BH, Nq, Nk, n_qblk, n_ksplit, tiles_per_split,
                       (int)total, scale * kLog2e, dp, seqs, lay);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, CAUSAL, 1, DROP>), dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                       static_cast<const bf16_raw*>(v), o_dst, l_dst, BH, Nq, Nk, n_qblk, n_ksplit, tiles_per_split,
                       (int)total, scale * kLog2e, dp, seqs, lay);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_ksplit == 1) return e;
  const long long rows = (long long)BH * Nq;
  if (rows > (1LL << 31) - 1 || n_ksplit > 256) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((splitkv_merge_kernel<DV>), dim3((unsigned)rows), dim3(64), 0, stream, o_dst, l_dst, o, lse,
                     rows, n_ksplit);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dv(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq, int Nk,
                     int dv, int n_ksplit, float* ws, float scale, const Dropout* drop, const Seqs& seqs,
                     const Strides& lay, bool dense, hipStream_t stream) {
  // dropout is offered for the square dense contract (dv = d) only
  if (drop) {
    if (dv != D || seqs.cu) return hipErrorInvalidValue;
    return launch<D, D, CAUSAL, true>(q, k, v, o, lse, BH, Nq, Nk, n_ksplit, ws, scale, *drop, seqs, lay, dense,
                                      stream);
  }
  const Dropout none{};
  return dv == 128 ? launch<D, 128, CAUSAL, false>(q, k, v, o, lse, BH, Nq, Nk, n_ksplit, ws, scale, none, seqs,
                                                   lay, dense, stream)
                   : launch<D, 64, CAUSAL, false>(q, k, v, o, lse, BH, Nq, Nk, n_ksplit, ws, scale, none, seqs, lay,
                                                  dense, stream);
}

}  // namespace

int fwd_splitkv_resolve(int BH, int Nq, int Nk, int d, int dv, int n_splits) {
  const int BC = (d == 64 && dv == 64) ? 128 : 64;
  const int n_ktiles = (Nk + BC - 1) / BC;
  if (n_ktiles <= 1) return 1;
  if (n_splits <= 0) {
    // enough workgroups for two per CU, and each range at least 4 tiles
    const long long base = (long long)BH * ((Nq + kBR - 1) / kBR);
    long long want = (2LL * kComputeUnits + base - 1) / base;
    want = std::min<long long>(want, std::max(1, n_ktiles / 4));
    n_splits = (int)std::max<long long>(1, std::min<long long>(want, 256));
  }
  n_splits = std::min(n_splits, n_ktiles);
  const int tps = (n_ktiles + n_splits - 1) / n_splits;
  return (n_ktiles + tps - 1) / tps;
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq,
                           int Nk, int d, int dv, int causal, int n_ksplit, float* ws, float scale,
                           const Dropout* drop, const Seqs* seqs, hipStream_t stream, const Strides* strides) {
  const Seqs sq = seqs ? *seqs : Seqs{nullptr, 0, 0};
  if (sq.cu && (n_ksplit != 1 || strides)) return hipErrorInvalidValue;
  // dense [BH, N, d] unless strides are given
  const Strides lay = strides ? *strides
                              : Strides{0, (long long)Nq * d, 0, (long long)Nk * d, 0, (long long)Nk * dv, d, d, dv, BH};
  const bool dense = strides == nullptr;
  if (!drop && n_ksplit == 1 && fwd_r64_applies(d, dv))
    return launch_fwd_r64(q, k, v, o, lse, BH, Nq, Nk, causal, scale, sq.cu ? &sq : nullptr, lay, stream);
  if (d == 128)
    return causal ? launch_dv<128, true>(q, k, v, o, lse, BH, Nq, Nk, dv, n_ksplit, ws, scale, drop, sq, lay, dense,
                                         stream)
                  : launch_dv<128, false>(q, k, v, o, lse, BH, Nq, Nk, dv, n_ksplit, ws, scale, drop, sq, lay, dense,
                                          stream);
  return causal ? launch_dv<64, true>(q, k, v, o, lse, BH, Nq, Nk, dv, n_ksplit, ws, scale, drop, sq, lay, dense,
                                      stream)
                : launch_dv<64, false>(q, k, v, o, lse, BH, Nq, Nk, dv, n_ksplit, ws, scale, drop, sq, lay, dense,
                                       stream);
}

}  // namespace fa

// dQ of the attention backward, query-stationary (bf16 inputs, float32 dQ).
//
// Recomputation as on the pages ("The forward pass is only half of it",
// FlashAttention: The Matrix You Never Have to Write Down; "Backward can
// recreate tiles instead of retaining the square", leviathansystems.co),
// with the chain rule written out in fa_bwd.hip:
//   dQ_i = sum_j dS'_ij K_j,   dS'_ij = P_ij (scale dP_ij - scale D_i),
//   P_ij = exp2(scale log2(e) S_ij - L_i log2(e)),   dP_ij = dO_i . V_j.
// Each query row's dQ is summed on chip over all its key tiles and written
// once, so no partial sums cross the memory fabric.
//
// Work split (one workgroup = 4 waves = 128 query rows of one head), the
// mirror image of the forward kernel:
//  * each wave owns 32 query rows; their Q and dO rows stay in AGPRs as the
//    B operands of S^T = K Q^T and dP^T = V dO^T (keys along M; the matrix
//    core reads AGPR operands directly), so a query's values sit in one lane
//    pair and its L and D are lane scalars;
//  * every product result (S^T, dP^T, dQ^T) lives in VGPRs, where the vector
//    ALUs read it without a copy: this file is built with the compiler's
//    VGPR form for matrix-core results (-amdgpu-mfma-vgpr-form), and only
//    the Q / dO operands are placed in AGPRs;
//  * K and V tiles of BC keys arrive by LDS-direct buffer loads, triple
//    buffered, rows in perm32 order with the backward's slot swizzle: the
//    S^T / dP^T results then hold 8 consecutive keys per register octet --
//    the B-operand layout of dQ^T += K^T dS'^T -- and the K^T operand is a
//    transpose read of the same K tile;
//  * causal: query block qb visits key tiles up to its diagonal only, masks
//    are applied only on tiles that straddle the diagonal or the ragged end.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup
// operand loads run kAhead MFMA groups ahead, through kSets register sets
constexpr int kAhead = 3;
constexpr int kSets = kAhead + 1;

template <int D> struct DqTile;
template <> struct DqTile<128> { static constexpr int BC = 64; };
template <> struct DqTile<64> { static constexpr int BC = 128; };

// three key tiles in flight: tile t's (dQ products), tile t+1's (S^T / dP^T
// products) and tile t+2's (arriving)
constexpr int kTiles = 3;

template <int D>
struct DqSmem {
  static constexpr int BC = DqTile<D>::BC;
  bf16_raw k[kTiles][BC * D];  // K tiles: row r holds key perm32(r) of its 32-row group
  bf16_raw v[kTiles][BC * D];  // V tiles, same layout
};

// 16-byte chunks a thread copies for one BC x D tile: LDS block (i*4 + wave)
// of 1 KiB, lane l -> row r, slot s; the source is key perm32(r) (within 32)
// and chunk s ^ swz(r).
template <int D>
struct KvCopy {
  static constexpr int BC = DqTile<D>::BC;
  static constexpr int SLOTS = D / 8;
  static constexpr int ROWS_PER_INSTR = 64 / SLOTS;
  static constexpr int INSTR = BC * SLOTS / kThreads;
  uint32_t off[INSTR];
  // row_bytes: distance of consecutive K (and V) rows in memory
  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int r = (i * kWaves + wave) * ROWS_PER_INSTR + lane / SLOTS;
      const int slot = lane % SLOTS;
      off[i] = (uint32_t)((r & ~31) + perm32(r & 31)) * row_bytes + (uint32_t)(16 * (slot ^ swz<D * 2>(r)));
    }
  }
};

// FUSED: the row statistics the backward needs (scale D = scale dO . O and
// L log2(e)) are computed here from O and L for this workgroup's rows and
// stored to L2 / Dsc for the dK/dV pass, which then runs after this one;
// otherwise they are read from L2 / Dsc (written by bwd_pre_kernel).
// STRIDED: Q, K, V are views (lay: element strides of batch, head and row;
// K and V share the row stride); otherwise dense, with the layout compiled in.
template <int D, bool CAUSAL, bool DROP, bool FUSED, bool STRIDED>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const bf16_raw* __restrict__ dO, float* __restrict__ L2, float* __restrict__ Dsc, const float* __restrict__ O,
    const float* __restrict__ LSE, float* __restrict__ dQ, int Nq, int Nk, int n_qblk, int total, float scale,
    float c, Dropout drop, Seqs seqs, Strides lay) {
  constexpr int BC = DqTile<D>::BC;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NKK = D / 16;   // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;   // 32-row blocks of dQ^T
  constexpr int RB = D * 2;     // bytes per row
  constexpr uint32_t kTileBytes = BC * D * 2;
  constexpr uint32_t kVMinusK = kTiles * kTileBytes;  // sm.v[b] - sm.k[b]
  __shared__ __attribute__((aligned(1024))) DqSmem<D> sm;

  int bh, qblk;
  if (CAUSAL || seqs.cu) {
    if ((int)blockIdx.x >= total) return;
    causal_order(blockIdx.x, total / n_qblk, n_qblk, kAllHeads, qblk, bh);
    if (CAUSAL) qblk = n_qblk - 1 - qblk;  // the last query block sees every key
  } else {
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    if (blk >= total) return;
    bh = blk / n_qblk;
    qblk = blk - bh * n_qblk;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  // first query row (Q, dO, O, statistics, dQ) and first key row (K, V) of
  // this head; for packed sequences, of sequence b = bh / H in head h = bh % H
  // (then Nq = Nk is that sequence's length and n_qblk covers the longest
  // one)
  size_t row0 = (size_t)bh * Nq, krow0 = (size_t)bh * Nk;
  if (seqs.cu) {
    const int b = bh / seqs.H, hh = bh - b * seqs.H;
    int s0, s1;
    seq_range(seqs, b, s0, s1);
    Nq = Nk = s1 - s0;
    row0 = krow0 = (size_t)hh * seqs.total + s0;
    if (qblk * kBR >= Nq) return;  // past the end of a shorter sequence
  }
  const size_t head = row0 * D;
  // Q, K, V bases and row strides (elements); dO, O, the statistics and dQ
  // are always dense
  const bf16_raw *Qh = Q + head, *Kh = K + krow0 * D, *Vh = V + krow0 * D;
  int q_stride = D, kv_stride = D;
  if constexpr (STRIDED) {
    const int b = bh / lay.H, hh = bh - b * lay.H;
    Qh = Q + (size_t)(b * lay.qb + hh * lay.qh);
    Kh = K + (size_t)(b * lay.kb + hh * lay.kh);
    Vh = V + (size_t)(b * lay.vb + hh * lay.vh);
    q_stride = lay.qr;
    kv_stride = lay.kr;
  }

  const int q_start = qblk * kBR;
  const int q0w = q_start + 32 * wave;
  const int my_q = q0w + col;
  // keys some row of the workgroup sees (upper-left causal mask): at least
  // key 0, since Nk >= 1 on every launch
  const int kv_end = CAUSAL ? min(Nk, q_start + kBR) : Nk;
  const int n_tiles = (kv_end + BC - 1) / BC;
  if (n_tiles == 0) {
    // no keys at all (Nk == 0): dQ = 0.  Workgroup-uniform, before any copy
    // or barrier; the statistics are not needed (no dK / dV rows exist).
    if (my_q < Nq) {
      float* row = dQ + head + (size_t)my_q * D;
#pragma unroll
      for (int d4 = 0; d4 < D / 8; ++d4)
        *reinterpret_cast<float4*>(row + 8 * d4 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return;
  }

  const uint32_t kv_row = (uint32_t)kv_stride * 2u;
  KvCopy<D> kc;
  kc.init(wave, lane, kv_row);
  // the wave index in a scalar register: the copies' LDS addresses (M0) are
  // scalar arithmetic
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // K and V of one key tile into buffer b.  The descriptors start at the
  // tile's first row and span the rest of the head, so the lane offsets stay
  // loop invariant and rows past the end of the head read as zeros.
  auto issue_tile = [&](uint32_t b, int key0) {
    key0 = __builtin_amdgcn_readfirstlane(key0);
    // the head's key rows from key0 on, up to the end of the last one
    const uint32_t rest = STRIDED ? (uint32_t)(Nk - 1 - key0) * kv_row + (uint32_t)(D * 2)
                                  : (uint32_t)(Nk * D * 2) - (uint32_t)key0 * D * 2;
    const __amdgpu_buffer_rsrc_t kt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kh + (size_t)key0 * kv_stride), (short)0, (int)rest, 0x00020000);
    const __amdgpu_buffer_rsrc_t vt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Vh + (size_t)key0 * kv_stride), (short)0, (int)rest, 0x00020000);
    const uint32_t kb = lds_addr_of(sm.k[b]), vb = lds_addr_of(sm.v[b]);
#pragma unroll
    for (int i = 0; i < KvCopy<D>::INSTR; ++i) {
      lds_copy(kt, kc.off[i], 0u, kb + (uint32_t)(i * kWaves + wave_s) * 1024u);
      lds_copy(vt, kc.off[i], 0u, vb + (uint32_t)(i * kWaves + wave_s) * 1024u);
    }
  };
  issue_tile(0u, 0);

  // this lane's query row: Q and dO slices (B operands), L log2(e), scale D
  bf16x8 qf[NKK], dof[NKK];
  float l2q, dq_sc;
  {
    const int qr = min(my_q, Nq - 1);
    const bf16_raw* Qrow = Qh + (size_t)qr * q_stride;
    const bf16_raw* Grow = dO + head + (size_t)qr * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = as_bf16x8(ld16(Qrow + 16 * kk + 8 * g));
      dof[kk] = as_bf16x8(ld16(Grow + 16 * kk + 8 * g));
    }
    // fused: this row's O (elements 16 kk + 8 g .. + 7) and L, in flight
    // with Q and dO
    float4 orow[FUSED ? 2 * NKK : 1];
    float lse_q = 0.f;
    if constexpr (FUSED) {
      lse_q = LSE[row0 + qr];
      const float* Orow = O + (row0 + qr) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        orow[2 * kk] = *reinterpret_cast<const float4*>(Orow + 16 * kk + 8 * g);
        orow[2 * kk + 1] = *reinterpret_cast<const float4*>(Orow + 16 * kk + 8 * g + 4);
      }
    }
    // in AGPRs for the whole kernel: they leave the VGPRs to the products
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      asm volatile("" : "+a"(qf[kk]));
      asm volatile("" : "+a"(dof[kk]));
    }
    if constexpr (FUSED) {
      // D = dO . O of this row, summed in the order of bwd_pre_kernel (so the
      // statistics, and every gradient, are bitwise those of the separate
      // preprocess): part p = 2 kk + g holds elements 8p .. 8p+7, each part a
      // chain of fused multiply-adds, the parts combined as p ^ 8, p ^ 4,
      // p ^ 2 (in this lane) and p ^ 1 (the lane of the other half).
      float part[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const float4 o0 = orow[2 * kk], o1 = orow[2 * kk + 1];
        const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)dof[kk][e], ov[e], acc);
        part[kk] = acc;
      }
#pragma unroll
      for (int sft = NKK / 2; sft > 0; sft >>= 1)
#pragma unroll
        for (int kk = 0; kk < sft; ++kk) part[kk] = part[kk] + part[kk + sft];
      dq_sc = scale * halves_sum(part[0]);
      l2q = lse_q * kLog2e;
      if (g == 0 && my_q < Nq) {
        Dsc[row0 + my_q] = dq_sc;
        L2[row0 + my_q] = l2q;
      }
    } else {
      l2q = L2[row0 + qr];
      dq_sc = Dsc[row0 + qr];
    }
  }

  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_acc[db][i] = 0.f;

  // ---- software pipeline over key tiles.  Tile t's work per 32-key block
  // kb is a score phase S(t, kb) (S^T and dP^T, NKK groups of two MFMAs), a
  // dQ phase Q(t, kb) (dQ^T += K^T dS'^T, NDB groups of two MFMAs) and the
  // softmax of the block (dS'^T) on the vector ALUs.  Iteration t runs the
  // pairs  S(t+1, kb) | Q(t, kb)  for kb = 0 .. NKB-1; beside pair 0 runs the
  // softmax of tile t's last block, beside pair kb > 0 that of tile t+1's
  // block kb-1, so every matrix-core phase has independent vector work.  The
  // prologue runs S(0, *) with the softmax of block kb-1 beside S(0, kb); the
  // last tile runs Q(*) with its last block's softmax beside the first phases.
  constexpr int GS = NKK;        // groups of a score phase
  constexpr int GQ = NDB;        // groups of a dQ phase: (half h, pair of head-dim blocks)
  constexpr int GP = GS + GQ;    // groups of a pair
  // Operand ring (see pin()): every group takes two operands -- K and V rows
  // in score phases, K^T transpose reads of two head-dim blocks in dQ phases.
  // Group g + kAhead loads into set (g + kAhead) % kSets while group g runs:
  // that set was last read by group g - 1, which has started once group g is
  // issued.  Group counts per run are multiples of kSets, so the sets a run
  // loads first were not read by the previous run's last group.
  static_assert((NKB * GS) % kSets == 0 && (NKB * GQ) % kSets == 0 && (NKB * GP) % kSets == 0,
                "operand ring must restart on a run boundary");
  bf16x8 op[kSets][2], dsb[NKB][2];
#pragma unroll
  for (int j = 0; j < kSets; ++j) op[j][0] = op[j][1] = bf16x8{};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) dsb[kb][0] = dsb[kb][1] = bf16x8{};
  f32x16 st[NKB], dpt[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) st[kb] = dpt[kb] = f32x16{};

  // per-lane LDS address constants (every tile base is a multiple of 1 KiB)
  // row reads: row 32 kb + col, chunk 2 kk + g -> lane constant ^ (32 kk)
  const int sw_r = swz<RB>(col);
  const uint32_t row_lane = (uint32_t)(col * RB + 16 * ((g ^ sw_r) & 1) + 32 * (sw_r >> 1));
  // transpose reads of the K tile: rows 32 kb + 16 h + tr_row (and + 8),
  // columns 32 db + 8 c0 + 4 (sl & 1) .. + 3
  const int tr_row = 4 * g + (sl >> 2);
  const int c0 = 2 * (grp & 1) + ((sl & 3) >> 1);
  const int sw_t = swz<RB>(tr_row);
  const uint32_t tk_lane = (uint32_t)(tr_row * RB + 64 * (sw_t >> 2) + 16 * (c0 ^ (sw_t & 3)) + 8 * (sl & 1));
  const uint32_t k_base0 = lds_addr_of(sm.k[0]);
  const int last_key = CAUSAL ? min(my_q, Nk - 1) : Nk - 1;  // keys above are masked

  // per-tile context: LDS addresses in the tile's buffer, first key
  struct Tile {
    uint32_t krow, tk, tk1;
    int key0;
  };
  auto tile_ctx = [&](int t) {
    const uint32_t kbase = k_base0 + (uint32_t)(t % kTiles) * kTileBytes;
    Tile x;
    x.krow = opaque(kbase + row_lane);
    x.tk = opaque(kbase + tk_lane);
    x.tk1 = opaque(x.tk ^ 32u);  // row + 8: swizzle ^ 2
    x.key0 = t * BC;
    return x;
  };
  // The same addresses for a loop whose buffers are known at compile time:
  // per-lane constants with the XOR of each k-slice / head-dim block folded
  // in (buffer 0), to which the buffer and row offsets add as immediates.
  // V rows get their own constants (their offset would not fit the field).
  uint32_t rlk[NKK], rlv[NKK], tkd[NDB], tk1d[NDB];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    rlk[kk] = opaque(k_base0 + (row_lane ^ (uint32_t)(32 * kk)));
    rlv[kk] = opaque(k_base0 + kVMinusK + (row_lane ^ (uint32_t)(32 * kk)));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tkd[db] = opaque(k_base0 + (tk_lane ^ (uint32_t)(64 * db)));
    tk1d[db] = opaque(k_base0 + ((tk_lane ^ 32u) ^ (uint32_t)(64 * db)));
  }

  // score group (key block kb, k-slice kk) and dQ group (kh = 2 kb + h,
  // head-dim blocks 2 pr, 2 pr + 1): operand loads and products
  auto load_s = [&](const Tile& x, int kb, int kk, bf16x8(&o)[2]) {
    const uint32_t ra = (x.krow ^ (uint32_t)(32 * kk)) + (uint32_t)(32 * kb * RB);
    o[0] = lds_row16(ra);
    o[1] = lds_row16(ra + kVMinusK);
  };
  auto load_q = [&](const Tile& x, int kh, int pr, bf16x8(&o)[2]) {
    const uint32_t rows = (uint32_t)(16 * kh * RB);
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int db = 2 * pr + y;
      o[y] = tr_pair((x.tk ^ (uint32_t)(64 * db)) + rows, (x.tk1 ^ (uint32_t)(64 * db)) + rows + 8 * RB);
    }
  };
  auto load_s_c = [&](auto buf, int kb, int kk, bf16x8(&o)[2]) {
    constexpr uint32_t b = decltype(buf)::value * kTileBytes;
    o[0] = lds_row16(rlk[kk] + b + (uint32_t)(32 * kb * RB));
    o[1] = lds_row16(rlv[kk] + b + (uint32_t)(32 * kb * RB));
  };
  auto load_q_c = [&](auto buf, int kh, int pr, bf16x8(&o)[2]) {
    constexpr uint32_t b = decltype(buf)::value * kTileBytes;
    const uint32_t rows = b + (uint32_t)(16 * kh * RB);
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int db = 2 * pr + y;
      o[y] = tr_pair(tkd[db] + rows, tk1d[db] + rows + 8 * RB);
    }
  };
  auto mfma_s = [&](int kb, int kk, const bf16x8(&o)[2]) {
    st[kb] = mfma32(o[0], qf[kk], kk == 0 ? f32x16{} : st[kb]);
    dpt[kb] = mfma32(o[1], dof[kk], kk == 0 ? f32x16{} : dpt[kb]);
    anchor_v(st[kb]);
    anchor_v(dpt[kb]);
  };
  auto mfma_q = [&](int kh, int pr, const bf16x8(&o)[2]) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      dq_acc[2 * pr + y] = mfma32(o[y], dsb[kh >> 1][kh & 1], dq_acc[2 * pr + y]);
      anchor_v(dq_acc[2 * pr + y]);
    }
  };
  // group i of a dQ phase: half h = i / (NDB / 2), pair pr = i % (NDB / 2)
  auto q_kh = [&](int kb, int i) { return 2 * kb + i / (NDB / 2); };
  auto q_pr = [&](int i) { return i % (NDB / 2); };

  // dS'^T = P^T (scale dP^T - scale D), P^T = exp2(S^T c - L log2 e), in
  // 8 pieces of 2 elements per lane; masked pairs get 0.  `masked` is a
  // compile-time flag: tiles below the diagonal and inside the sequence take
  // the code without masks.
  float dsv[8];
  uint32_t dm[4] = {0u, 0u, 0u, 0u};  // dropout mask words of the current block
  const float scale_r = DROP ? scale * drop.r : scale;
  auto softmax_piece = [&](const Tile& x, int kb, auto pc, auto masked) {
    constexpr int piece = decltype(pc)::value, h = piece >> 2, e0 = 2 * (piece & 3);
    if constexpr (DROP && piece == 0) {
      // dropout mask of this 32-key block: lane q of each 4-lane group
      // computes the 4 x 4 block of the group's rows and keys
      // 16 (q / 2) + 8 g + 4 (q % 2) .. + 3; after the word exchange dm[x]
      // holds this row's word of block x
      const int qd = col & 3;
      uint32_t w[4] = {(uint32_t)(x.key0 + 32 * kb + 16 * (qd >> 1) + 8 * g + 4 * (qd & 1)) >> 2,
                       (uint32_t)my_q >> 2, (uint32_t)bh, drop.offset};
      philox4x32_10(w, drop.k0, drop.k1);
      quad_transpose(w, dm, qd);
    }
    // register 8 h + e of half g holds key key0 + 32 kb + 16 h + 8 g + e
    int lim = 0;
    if constexpr (decltype(masked)::value) lim = last_key - (x.key0 + 32 * kb + 16 * h + 8 * g);
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e) {
      float pe = fast_exp2(fmaf(st[kb][8 * h + e], c, -l2q));
      if constexpr (decltype(masked)::value) pe = e > lim ? 0.f : pe;
      if constexpr (DROP)  // a dropped pair's dP term vanishes from dS'
        dsv[e] = pe * fmaf(dpt[kb][8 * h + e], kept(dm[2 * h + (e >> 2)], e & 3, drop.t) ? scale_r : 0.f, -dq_sc);
      else
        dsv[e] = pe * fmaf(dpt[kb][8 * h + e], scale, -dq_sc);
    }
    if constexpr ((piece & 3) == 3) dsb[kb][h] = pack_bf16x8(dsv);
  };
  // the softmax pieces of 8 that go beside group k of n
  auto pieces = [&](auto k, auto n, auto&& piece) {
    constexpr int K = decltype(k)::value, Nn = decltype(n)::value;
    static_for<(8 * K) / Nn, (8 * (K + 1)) / Nn>(piece);
  };
  // dQ products of tile t-1 read block kb's dS', which the softmax of tile t
  // rewrites: keep the old value alive past the first group of the next run
  auto release_ds = [&](int kb) {
    pin(dsb[kb][0]);
    pin(dsb[kb][1]);
  };

  // ---- one run of NG groups.  load(gi, o) loads group gi's operands into o,
  // mfma(gi, o) issues its products; between(gi) runs vector work after
  // group gi has issued.  At gi = 0 the ring pin keeps the set read by the
  // previous run's last group alive past the run's first product, so no
  // preamble load reuses its registers.
  auto run = [&](auto n_groups, auto load, auto mfma, auto between) {
    constexpr int NG = decltype(n_groups)::value;
    static_for<0, kAhead>([&](auto gi) { load(gi, op[decltype(gi)::value % kSets]); });
    static_for<0, NG>([&](auto gi) {
      constexpr int n = decltype(gi)::value, nxt = (n + kAhead) % kSets;
      mfma(gi, op[n % kSets]);
      group_fence();
      pin(op[nxt][0]);
      pin(op[nxt][1]);
      if constexpr (n + kAhead < NG) load(ic<n + kAhead>{}, op[nxt]);
      between(gi);
    });
  };
  const std::true_type with_masks;
  const std::false_type no_masks;

  // ---- prologue: S(0, *) with the softmax of block kb-1 beside S(0, kb)
  wait_loads();
  __syncthreads();  // tile 0 visible
  if (n_tiles > 1) issue_tile(1u, BC);
  {
    const Tile x0 = tile_ctx(0);
    run(ic<NKB * GS>{},
        [&](auto gi, bf16x8(&o)[2]) { load_s(x0, gi / GS, gi % GS, o); },
        [&](auto gi, const bf16x8(&o)[2]) { mfma_s(gi / GS, gi % GS, o); },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value;
          if constexpr (n >= GS)
            pieces(ic<n % GS>{}, ic<GS>{}, [&](auto pc) { softmax_piece(x0, n / GS - 1, pc, with_masks); });
        });
  }
  wait_loads();  // this wave's copies of tile 1 have landed

  // ---- steady state: S(t+1, kb) | Q(t, kb) for every block kb
  // BUFC: buffer of tile t when known at compile time (else -1); tile t+1
  // sits in the next one
  auto iterate = [&](const Tile& xc, const Tile& xn, auto masked, auto bufc) {
    constexpr int BUFC = decltype(bufc)::value;
    run(ic<NKB * GP>{},
        [&](auto gi, bf16x8(&o)[2]) {
          constexpr int n = decltype(gi)::value, kb = n / GP, i = n % GP;
          if constexpr (BUFC >= 0) {
            if constexpr (i < GS) load_s_c(ic<(BUFC + 1) % kTiles>{}, kb, i, o);
            else load_q_c(ic<BUFC>{}, q_kh(kb, i - GS), q_pr(i - GS), o);
          } else {
            if constexpr (i < GS) load_s(xn, kb, i, o);
            else load_q(xc, q_kh(kb, i - GS), q_pr(i - GS), o);
          }
        },
        [&](auto gi, const bf16x8(&o)[2]) {
          constexpr int n = decltype(gi)::value, kb = n / GP, i = n % GP;
          if constexpr (i < GS) mfma_s(kb, i, o);
          else mfma_q(q_kh(kb, i - GS), q_pr(i - GS), o);
        },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value, kb = n / GP, i = n % GP;
          if constexpr (i == 0) release_ds(kb == 0 ? NKB - 1 : kb - 1);
          if constexpr (kb == 0)
            pieces(ic<i>{}, ic<GP>{}, [&](auto pc) { softmax_piece(xc, NKB - 1, pc, masked); });
          else
            pieces(ic<i>{}, ic<GP>{}, [&](auto pc) { softmax_piece(xn, kb - 1, pc, masked); });
        });
  };
  auto step = [&](int t, auto masked) {
    __syncthreads();  // tile t+1 visible; every wave is done with tile t-1
    if (t + 2 < n_tiles) issue_tile((uint32_t)((t + 2) % kTiles), (t + 2) * BC);
    iterate(tile_ctx(t), tile_ctx(t + 1), masked, ic<-1>{});
    wait_loads();  // this wave's copies of tile t+2 have landed
  };
  // the same with tile t in buffer BUFC (t % 3 == BUFC)
  auto step_c = [&](int t, auto bufc) {
    __syncthreads();
    if (t + 2 < n_tiles) issue_tile((uint32_t)((decltype(bufc)::value + 2) % kTiles), (t + 2) * BC);
    Tile xc, xn;  // only key0 is read
    xc.key0 = t * BC;
    xn.key0 = (t + 1) * BC;
    iterate(xc, xn, no_masks, bufc);
    wait_loads();
  };
  // Tiles that need masks (for any row of the workgroup) form a suffix: the
  // ones that meet the diagonal and the one holding the end of the sequence.
  // Iteration t touches tiles t and t+1, so it needs masks iff t+1 >= t_mask.
  const int t_mask = min(CAUSAL ? (q_start + 1) / BC : n_tiles, Nk / BC);
  int t = 0;
  // mask-free tiles three at a time from t = 0: tile t + i in buffer i
  for (; t + 3 < n_tiles && t + 3 < t_mask; t += 3) {
    step_c(t, ic<0>{});
    step_c(t + 1, ic<1>{});
    step_c(t + 2, ic<2>{});
  }
  for (; t + 1 < n_tiles && t + 1 < t_mask; ++t) step(t, no_masks);
  for (; t + 1 < n_tiles; ++t) step(t, with_masks);

  // ---- last tile: Q(*), its last block's softmax beside the phases before
  // the last one
  {
    const Tile xc = tile_ctx(n_tiles - 1);
    constexpr int NSM = (NKB - 1) * GQ;  // groups that carry the softmax
    run(ic<NKB * GQ>{},
        [&](auto gi, bf16x8(&o)[2]) { load_q(xc, q_kh(gi / GQ, gi % GQ), q_pr(gi % GQ), o); },
        [&](auto gi, const bf16x8(&o)[2]) { mfma_q(q_kh(gi / GQ, gi % GQ), q_pr(gi % GQ), o); },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value;
          if constexpr (n == 0) {
            release_ds(NKB - 1);
            // with a single tile the prologue's last score product precedes
            // this run: its Q / dO operands stay unwritten until now
            pin(qf[NKK - 1]);
            pin(dof[NKK - 1]);
          }
          if constexpr (n < NSM)
            pieces(ic<n>{}, ic<NSM>{}, [&](auto pc) { softmax_piece(xc, NKB - 1, pc, with_masks); });
        });
  }

  // every MFMA has completed once fin exists: operand registers may be reused
  float fin = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) fin += dq_acc[db][0];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    pin(op[j][0], fin);
    pin(op[j][1], fin);
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    pin(dsb[kb][0], fin);
    pin(dsb[kb][1], fin);
  }
  group_fence();  // nothing after this point is scheduled above the pins

  if (my_q < Nq) {
    float* row = dQ + head + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(row + 32 * db + 8 * i4 + 4 * g) =
            make_float4(dq_acc[db][4 * i4], dq_acc[db][4 * i4 + 1], dq_acc[db][4 * i4 + 2], dq_acc[db][4 * i4 + 3]);
  }
}

// o, lse non-null: the fused launch (statistics computed here and stored to
// l2 / dsc); else l2 / dsc hold them already
template <int D, bool CAUSAL, bool DROP, bool STRIDED = false>
hipError_t launch(const void* q, const void* k, const void* v, const void* dout, float* l2, float* dsc,
                  const float* o, const float* lse, float* dq, int BH, int Nq, int Nk, float scale,
                  const Dropout& drop, const Seqs& sq, const Strides& lay, hipStream_t stream) {
  const int n_qblk = (Nq + kBR - 1) / kBR;
  const long long total = (long long)BH * n_qblk;
  if (total == 0) return hipSuccess;  // no query rows: no dQ
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  if (o)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, DROP, true, STRIDED>), dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                       static_cast<const bf16_raw*>(v), static_cast<const bf16_raw*>(dout), l2, dsc, o, lse, dq, Nq,
                       Nk, n_qblk, (int)total, scale, scale * kLog2e, drop, sq, lay);
  else if constexpr (!STRIDED)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, DROP, false, false>), dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                       static_cast<const bf16_raw*>(v), static_cast<const bf16_raw*>(dout), l2, dsc, o, lse, dq, Nq,
                       Nk, n_qblk, (int)total, scale, scale * kLog2e, drop, sq, lay);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_drop(const void* q, const void* k, const void* v, const void* dout, float* l2, float* dsc,
                       const float* o, const float* lse, float* dq, int BH, int Nq, int Nk, float scale,
                       const Dropout* drop, const Seqs& sq, const Strides* lay, hipStream_t stream) {
  if (lay) {
    // strided views: the fused launch only, without packing or dropout
    if (drop || sq.cu || !o) return hipErrorInvalidValue;
    return launch<D, CAUSAL, false, true>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, Dropout{}, sq, *lay,
                                          stream);
  }
  const Strides dense = dense_strides(Nq, Nk, D);
  if (drop) {
    if (sq.cu) return hipErrorInvalidValue;  // dropout is offered for the dense layout only
    return launch<D, CAUSAL, true>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, *drop, sq, dense, stream);
  }
  return launch<D, CAUSAL, false>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, Dropout{}, sq, dense,
                                  stream);
}

hipError_t launch_any(const void* q, const void* k, const void* v, const void* dout, float* l2, float* dsc,
                      const float* o, const float* lse, float* dq, int BH, int Nq, int Nk, int d, float scale,
                      int causal, const Dropout* drop, const Seqs* seqs, hipStream_t stream, const Strides* lay) {
  const Seqs sq = seqs ? *seqs : Seqs{nullptr, 0, 0};
  if (d == 128)
    return causal
               ? launch_drop<128, true>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, drop, sq, lay, stream)
               : launch_drop<128, false>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, drop, sq, lay, stream);
  return causal ? launch_drop<64, true>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, drop, sq, lay, stream)
                : launch_drop<64, false>(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, scale, drop, sq, lay, stream);
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout, const float* l2,
                              const float* dsc, float* dq, int BH, int Nq, int Nk, int d, float scale, int causal,
                              const Dropout* drop, const Seqs* seqs, hipStream_t stream, const Strides* lay) {
  // statistics only read on this launch
  return launch_any(q, k, v, dout, const_cast<float*>(l2), const_cast<float*>(dsc), nullptr, nullptr, dq, BH, Nq,
                    Nk, d, scale, causal, drop, seqs, stream, lay);
}

hipError_t launch_bwd_dq_fused(const void* q, const void* k, const void* v, const void* dout, const float* o,
                               const float* lse, float* l2, float* dsc, float* dq, int BH, int Nq, int Nk, int d,
                               float scale, int causal, const Dropout* drop, const Seqs* seqs, hipStream_t stream,
                               const Strides* lay) {
  return launch_any(q, k, v, dout, l2, dsc, o, lse, dq, BH, Nq, Nk, d, scale, causal, drop, seqs, stream, lay);
}

}  // namespace fa

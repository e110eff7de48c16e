// Exact attention backward by recomputation, bf16 inputs, float32 gradients.
//
// Per the pages, the forward saves only Q, K, V, O and the per-row
// logsumexp L, and the backward recomputes every score / probability tile it
// needs from them ("The forward pass is only half of it", FlashAttention:
// The Matrix You Never Have to Write Down; "Backward can recreate tiles
// instead of retaining the square", leviathansystems.co).  They give no gradient formulas; the
// kernels use the chain rule on softmax(scale Q K^T) V:
//   P = exp(scale S - L),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// The factor `scale` is folded into dS once: the kernels form
//   dS' = scale dS = P * (scale dP - scale D)
// (scale D comes from the preprocess), so dK = dS'^T Q and dQ = dS' K.
//
// Kernels (no atomics, every output written once; fa_bwd launches the dQ
// pass with the preprocess folded in, then dK/dV):
//  * bwd_pre_kernel: per query row scale * (dO_i . O_i) and L_i log2(e) into
//    the workspace (the separate preprocess phase).
//  * bwd_dkdv_kernel: one workgroup per (head, block of 128 keys).  Each of
//    its 4 waves owns 32 keys: their K and V rows stay in AGPRs for the whole
//    kernel (B operands of S = Q K^T and dP = dO V^T), and dK^T, dV^T
//    accumulate in registers.  The workgroup walks the query rows 64 at a
//    time (causal: from the block's diagonal on).  Per step:
//      A. S and dP for the 64 rows of the tile (Q and dO tiles arrive by
//         LDS-direct buffer loads, three buffers, rows in perm32 order so
//         that S and dP come out with 8 consecutive query rows per register
//         octet -- the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS');
//      B. P and dS' on the vector ALUs;
//      C. dV^T += dO^T P and dK^T += Q^T dS', the A operands read from the
//         row-major tiles with ds_read_b64_tr_b16.
//    One barrier per step publishes the tile and frees the buffer the step
//    refills.
//  * bwd_dq_kernel (fa_bwd_dq.hip): query-stationary, recomputes S and dP
//    per key tile and accumulates dQ in registers; in fa_bwd it also forms
//    the row statistics of its rows for the dK/dV pass.
// dQ is not accumulated across key blocks with atomics: on this part
// device-scope float atomics are performed at the memory side, and the
// partial sums of every key block would cross the fabric once each; the
// second recomputation of S and dP costs less.
//  One 16-byte-slot XOR swizzle per row width serves both the row reads and
//  the transpose reads of a tile without LDS bank conflicts; every per-lane
//  LDS address is a lane constant XOR a compile-time mask, plus an
//  immediate.
#include "fa_common.h"
#include "fa_dropout.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

// ----------------------------------------------------------------------------------- preprocess
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_raw* __restrict__ dO, const float* __restrict__ O,
                                                       const float* __restrict__ LSE, float* __restrict__ Dsc,
                                                       float* __restrict__ L2, long long rows, float scale) {
  constexpr int TPR = D / 8;  // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + 8 * part;
    const uint4 g = ld16(dO + off);
    const float4 o0 = *reinterpret_cast<const float4*>(O + off);
    const float4 o1 = *reinterpret_cast<const float4*>(O + off + 4);
    const uint32_t w[4] = {g.x, g.y, g.z, g.w};
    const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(w[e] << 16), ov[2 * e], acc);
      acc = fmaf(__uint_as_float(w[e] & 0xffff0000u), ov[2 * e + 1], acc);
    }
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (row < rows && part == 0) {
    Dsc[row] = scale * acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ----------------------------------------------------------------------------------- main kernel
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 32 * kWaves;  // keys per workgroup
constexpr int kBQ = 64;            // query rows per step
// operand loads run kAhead MFMA groups ahead, through kSets register sets
constexpr int kAhead = 3;
constexpr int kSets = kAhead + 1;

// three query tiles in flight: step st's (dV / dK products), step st+1's
// (S / dP products) and step st+2's (arriving)
constexpr int kTiles = 3;

template <int D>
struct DkdvSmem {
  bf16_raw q[kTiles][kBQ * D];     // Q tiles, rows in perm32 order
  bf16_raw dout[kTiles][kBQ * D];  // dO tiles, rows in perm32 order
  float l2[kTiles][kBQ];           // L log2(e) of the tile's rows
  float dsc[kTiles][kBQ];          // scale * D of the tile's rows
};

// 16-byte chunks a thread copies for one BQ x D query tile: LDS block
// (i*4 + wave) of 1 KiB, lane l -> row r, slot s; the source is row
// perm32(r) (within 32) and chunk s ^ swz(r), rows row_bytes apart in memory.
template <int D>
struct QCopy {
  static constexpr int SLOTS = D / 8;
  static constexpr int ROWS_PER_INSTR = 64 / SLOTS;
  static constexpr int INSTR = kBQ * SLOTS / kThreads;
  uint32_t off[INSTR];
  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int r = (i * kWaves + wave) * ROWS_PER_INSTR + lane / SLOTS;
      const int slot = lane % SLOTS;
      off[i] = (uint32_t)((r & ~31) + perm32(r & 31)) * row_bytes + (uint32_t)(16 * (slot ^ swz<D * 2>(r)));
    }
  }
};

// STRIDED: Q, K, V are views (lay: element strides of batch, head and row);
// otherwise dense, with the layout compiled in.
template <int D, bool CAUSAL, bool DROP, bool STRIDED>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const bf16_raw* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dsc,
    float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nk, int n_kvblk, int total, float scale, float c,
    Dropout drop, Seqs seqs, Strides lay) {
  constexpr int NKK = D / 16;  // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;  // 32-row blocks of dK^T / dV^T
  constexpr int RB = D * 2;    // bytes per Q / dO / K row
  constexpr uint32_t kTileBytes = kBQ * D * 2;
  constexpr uint32_t kDoutMinusQ = kTiles * kTileBytes;  // sm.dout[b] - sm.q[b]
  constexpr uint32_t kDscMinusL2 = kTiles * kBQ * 4;     // sm.dsc[b] - sm.l2[b]
  __shared__ __attribute__((aligned(1024))) DkdvSmem<D> sm;

  int bh, kvb;
  if (CAUSAL || seqs.cu) {
    if ((int)blockIdx.x >= total) return;
    causal_order(blockIdx.x, total / n_kvblk, n_kvblk, kAllHeads, kvb, bh);  // key block 0 sees every query row
  } else {
    const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
    if (blk >= total) return;
    bh = blk / n_kvblk;
    kvb = blk - bh * n_kvblk;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  // first query row (Q, dO, statistics) and first key row (K, V, dK, dV) of
  // this head; for packed sequences, of sequence b = bh / H in head h = bh % H
  // (then Nq = Nk is that sequence's length and n_kvblk covers the longest
  // one)
  size_t row0 = (size_t)bh * Nq, krow0 = (size_t)bh * Nk;
  if (seqs.cu) {
    const int b = bh / seqs.H, hh = bh - b * seqs.H;
    int s0, s1;
    seq_range(seqs, b, s0, s1);
    Nq = Nk = s1 - s0;
    row0 = krow0 = (size_t)hh * seqs.total + s0;
    if (kvb * kBKV >= Nk) return;  // past the end of a shorter sequence
  }
  const size_t head = row0 * D, khead = krow0 * D;
  // Q, K, V bases and row strides (elements); dO, the statistics and the
  // gradients are always dense
  const bf16_raw *Qh = Q + head, *Kh = K + khead, *Vh = V + khead;
  int q_stride = D, k_stride = D, v_stride = D;
  if constexpr (STRIDED) {
    const int b = bh / lay.H, hh = bh - b * lay.H;
    Qh = Q + (size_t)(b * lay.qb + hh * lay.qh);
    Kh = K + (size_t)(b * lay.kb + hh * lay.kh);
    Vh = V + (size_t)(b * lay.vb + hh * lay.vh);
    q_stride = lay.qr;
    k_stride = lay.kr;
    v_stride = lay.vr;
  }

  const int k0 = kvb * kBKV;
  const int my_key = k0 + 32 * wave + col;

  const int q_first = CAUSAL ? k0 : 0;  // k0 is a multiple of kBQ
  const int n_steps = (Nq - q_first + kBQ - 1) / kBQ;
  if (n_steps <= 0) {
    // no query row sees these keys (causal, Nq <= k0): zero gradients
    if (my_key < Nk) {
      float* dKrow = dK + khead + (size_t)my_key * D;
      float* dVrow = dV + khead + (size_t)my_key * D;
#pragma unroll
      for (int d4 = 0; d4 < D / 8; ++d4) {
        *reinterpret_cast<float4*>(dKrow + 8 * d4 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(dVrow + 8 * d4 + 4 * g) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;  // workgroup-uniform: every wave leaves before any barrier
  }

  // byte spans of a head's rows: up to the end of the last row, D elements
  const uint32_t q_row = (uint32_t)q_stride * 2u, k_row = (uint32_t)k_stride * 2u, v_row = (uint32_t)v_stride * 2u;
  const int head_bytes = Nq * D * 2;
  const int k_bytes = (int)((uint32_t)(Nk - 1) * k_row + (uint32_t)(D * 2));
  const int v_bytes = (int)((uint32_t)(Nk - 1) * v_row + (uint32_t)(D * 2));
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, k_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, v_bytes, 0x00020000);

  // copy offsets: Q rows q_row apart; dO rows dense (a set of their own only
  // when Q is strided)
  QCopy<D> qc, gc;
  qc.init(wave, lane, q_row);
  if constexpr (STRIDED) gc.init(wave, lane, (uint32_t)(D * 2));
  const QCopy<D>& gq = STRIDED ? gc : qc;
  // the wave index in a scalar register: the copies' LDS addresses (M0) are
  // scalar arithmetic
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // Q / dO / L2 / scale*D of one query tile into buffer b.  The descriptors
  // start at the tile's first row and span the rest of the head, so the lane
  // offsets stay loop invariant and rows past the end of the head read as
  // zeros.
  auto issue_qtile = [&](uint32_t b, int q0) {
    q0 = __builtin_amdgcn_readfirstlane(q0);
    const uint32_t toff = (uint32_t)q0 * D * 2, rest = (uint32_t)head_bytes - toff;
    const uint32_t qrest = STRIDED ? (uint32_t)(Nq - 1 - q0) * q_row + (uint32_t)(D * 2) : rest;
    const __amdgpu_buffer_rsrc_t qt = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Qh + (size_t)q0 * q_stride), (short)0, (int)qrest, 0x00020000);
    const __amdgpu_buffer_rsrc_t gt =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dO + head + (size_t)q0 * D), (short)0, (int)rest, 0x00020000);
    const uint32_t qb = lds_addr_of(sm.q[b]), gb = lds_addr_of(sm.dout[b]);
#pragma unroll
    for (int i = 0; i < QCopy<D>::INSTR; ++i) {
      lds_copy(qt, qc.off[i], 0u, qb + (uint32_t)(i * kWaves + wave_s) * 1024u);
      lds_copy(gt, gq.off[i], 0u, gb + (uint32_t)(i * kWaves + wave_s) * 1024u);
    }
    if (wave_s < 2) {
      const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((wave_s == 0 ? L2 : Dsc) + row0 + q0), (short)0, (Nq - q0) * 4, 0x00020000);
      lds_copy4(rt, (uint32_t)lane * 4u, 0u, lds_addr_of(wave_s == 0 ? sm.l2[b] : sm.dsc[b]));
    }
  };

  issue_qtile(0u, q_first);

  // K and V rows of this wave's keys, 8 head-dim elements per k-slice: the
  // B operands of S = Q K^T and dP = dO V^T for the whole kernel (rows past
  // Nk read as zero)
  bf16x8 kres[NKK], vres[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const uint32_t col_b = (uint32_t)(16 * kk + 8 * g) * 2u;
    kres[kk] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, (uint32_t)my_key * k_row + col_b, 0, 0));
    vres[kk] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vrs, (uint32_t)my_key * v_row + col_b, 0, 0));
  }
  // kept in AGPRs, which the matrix cores read directly.  The pins follow
  // all of the loads: a pin reads its register, so a pin right behind its
  // load would wait for it, one memory round trip per slice.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    asm volatile("" : "+a"(kres[kk]));
    asm volatile("" : "+a"(vres[kk]));
  }

  f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk_acc[db][i] = 0.f;
      dv_acc[db][i] = 0.f;
    }

  // ---- software pipeline over steps.  Step st's work is four MFMA phases
  // of G groups (two MFMAs each):
  //   A0 / A1: S and dP of query block 0 / 1 (32 rows) against the wave's keys
  //   C0 / C1: dV^T, dK^T from query block 0 / 1
  // and the softmax of each block (P, dS') on the vector ALUs.  Iteration st
  // runs   A0(st+1) | C0(st) | A1(st+1) | C1(st)
  // with softmax(st, block 1) spread over the groups of the first two phases
  // and softmax(st+1, block 0) over the last two, so every matrix-core phase
  // has independent vector work beside it.  The prologue runs A0(0), A1(0) and
  // softmax(0, block 0); the last step runs C0, C1 with softmax(block 1).
  constexpr int G = NKK;  // groups per phase (= 2 NDB)
  // Operand ring (see pin()): every group takes two operands -- Q and dO rows
  // in phases A, dO^T and Q^T transpose reads in phases C.  Group g + kAhead
  // loads into set (g + kAhead) % kSets while group g runs: that set was last
  // read by group g - 1, which has started once group g is issued.  Group
  // counts per run (4G, 2G) are multiples of kSets, so the sets a run loads
  // first were not read by the previous run's last group.
  static_assert((2 * G) % kSets == 0, "operand ring must restart on a phase boundary");
  bf16x8 op[kSets][2], pb[2][2], dsb[2][2];
#pragma unroll
  for (int j = 0; j < kSets; ++j) op[j][0] = op[j][1] = bf16x8{};
#pragma unroll
  for (int j = 0; j < 2; ++j) pb[j][0] = pb[j][1] = dsb[j][0] = dsb[j][1] = bf16x8{};
  f32x16 s[2], dp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) s[j] = dp[j] = f32x16{};

  // ---- per-lane LDS address constants.  Every tile base is a multiple of
  // 1 KiB, so XOR masks below bit 10 pass through the base.
  // S / dP row reads: row 32 qb + col, chunk 2 kk + g:
  // offset = lane constant ^ (32 kk), + 32 qb rows as an immediate.
  const int sw_r = swz<RB>(col);
  const uint32_t row_lane = (uint32_t)(col * RB + 16 * ((g ^ sw_r) & 1) + 32 * (sw_r >> 1));
  // transpose reads of the Q / dO tiles: rows 16 (2 qb + h) + tr_row (and
  // + 8), columns 32 db + 8 c0 + 4 (sl & 1) .. + 3
  const int tr_row = 4 * g + (sl >> 2);
  const int c0 = 2 * (grp & 1) + ((sl & 3) >> 1);
  const int sw_t = swz<RB>(tr_row);
  const uint32_t tq_lane = (uint32_t)(tr_row * RB + 64 * (sw_t >> 2) + 16 * (c0 ^ (sw_t & 3)) + 8 * (sl & 1));
  const uint32_t q_base0 = lds_addr_of(sm.q[0]);
  const uint32_t l2_base0 = lds_addr_of(sm.l2[0]);

  // per-step context: LDS addresses in the step's tile buffer, first query row
  struct Step {
    uint32_t qrow, tq, tq1, l2;
    int q0;
  };
  auto step_ctx = [&](int st) {
    const uint32_t b = (uint32_t)(st % kTiles);
    const uint32_t qbase = q_base0 + b * kTileBytes;
    Step x;
    x.qrow = opaque(qbase + row_lane);
    x.tq = opaque(qbase + tq_lane);
    x.tq1 = opaque(x.tq ^ 32u);  // row + 8: swizzle ^ 2
    x.l2 = l2_base0 + b * (kBQ * 4) + (uint32_t)(32 * g);
    x.q0 = q_first + st * kBQ;
    return x;
  };

  // The same addresses for steps whose buffer is known at compile time:
  // per-lane constants with the XOR of each k-slice / head-dim block folded
  // in (buffer 0), to which the buffer and row offsets add as immediates.
  // dO gets its own constants (its offset would not fit the field).
  uint32_t rq[NKK], rgo[NKK], tqd[NDB], tq1d[NDB], tgd[NDB], tg1d[NDB];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    rq[kk] = opaque(q_base0 + (row_lane ^ (uint32_t)(32 * kk)));
    rgo[kk] = opaque(q_base0 + kDoutMinusQ + (row_lane ^ (uint32_t)(32 * kk)));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tqd[db] = opaque(q_base0 + (tq_lane ^ (uint32_t)(64 * db)));
    tq1d[db] = opaque(q_base0 + ((tq_lane ^ 32u) ^ (uint32_t)(64 * db)));
    tgd[db] = opaque(q_base0 + kDoutMinusQ + (tq_lane ^ (uint32_t)(64 * db)));
    tg1d[db] = opaque(q_base0 + kDoutMinusQ + ((tq_lane ^ 32u) ^ (uint32_t)(64 * db)));
  }
  const uint32_t l2_lane = l2_base0 + (uint32_t)(32 * g);
  auto step_ctx_c = [&](int st, auto buf) {
    Step x;
    x.qrow = x.tq = x.tq1 = 0u;  // not read on this path
    x.l2 = l2_lane + (uint32_t)(decltype(buf)::value * kBQ * 4);
    x.q0 = q_first + st * kBQ;
    return x;
  };

  // phase A group (query block qb, k-slice kk) and phase C group (qh = 2 qb + h,
  // head-dim block db): operand loads and products
  auto load_a = [&](const Step& x, int qb, int kk, bf16x8(&o)[2]) {
    const uint32_t ra = (x.qrow ^ (uint32_t)(32 * kk)) + (uint32_t)(32 * qb * RB);
    o[0] = lds_row16(ra);
    o[1] = lds_row16(ra + kDoutMinusQ);
  };
  auto load_c = [&](const Step& x, int qh, int db, bf16x8(&o)[2]) {
    const uint32_t rows = (uint32_t)(16 * qh * RB);
    const uint32_t o0 = (x.tq ^ (uint32_t)(64 * db)) + rows;
    const uint32_t o1 = (x.tq1 ^ (uint32_t)(64 * db)) + rows + 8 * RB;
    o[0] = tr_pair(o0 + kDoutMinusQ, o1 + kDoutMinusQ);
    o[1] = tr_pair(o0, o1);
  };
  auto load_a_c = [&](auto buf, int qb, int kk, bf16x8(&o)[2]) {
    constexpr uint32_t b = decltype(buf)::value * kTileBytes;
    o[0] = lds_row16(rq[kk] + b + (uint32_t)(32 * qb * RB));
    o[1] = lds_row16(rgo[kk] + b + (uint32_t)(32 * qb * RB));
  };
  auto load_c_c = [&](auto buf, int qh, int db, bf16x8(&o)[2]) {
    constexpr uint32_t b = decltype(buf)::value * kTileBytes;
    const uint32_t rows = b + (uint32_t)(16 * qh * RB);
    o[0] = tr_pair(tgd[db] + rows, tg1d[db] + rows + 8 * RB);
    o[1] = tr_pair(tqd[db] + rows, tq1d[db] + rows + 8 * RB);
  };
  auto mfma_a = [&](int qb, int kk, const bf16x8(&o)[2]) {
    s[qb] = mfma32(o[0], kres[kk], kk == 0 ? f32x16{} : s[qb]);
    dp[qb] = mfma32(o[1], vres[kk], kk == 0 ? f32x16{} : dp[qb]);
    anchor_a(s[qb]);
    anchor_a(dp[qb]);
  };
  auto mfma_c = [&](int qh, int db, const bf16x8(&o)[2]) {
    dv_acc[db] = mfma32(o[0], pb[qh >> 1][qh & 1], dv_acc[db]);
    dk_acc[db] = mfma32(o[1], dsb[qh >> 1][qh & 1], dk_acc[db]);
    anchor_a(dv_acc[db]);
    anchor_a(dk_acc[db]);
  };

  // ---- softmax of query block qb of a step, in 8 pieces of 2 elements per
  // lane: P = exp2(S c - L log2 e), dS' = P (scale dP - scale D); masked
  // pairs get 0.  Chunk h = piece / 4 covers 8 consecutive query rows.  Its
  // L log2 e and scale D (lvd[h]) are read from LDS one chunk ahead, so the
  // reads never hold up the operand loads queued behind them.  `masked` is
  // a compile-time flag: steps off the diagonal and inside the sequence
  // take the code without masks.
  float lvd[2][16], pv[8], dv8[8];
  int dead = 0;
  uint32_t dm[4] = {0u, 0u, 0u, 0u};           // dropout mask words of the current block
  const float scale_r = DROP ? scale * drop.r : scale;
  // L log2 e and scale D of chunk h of block qb of step x into lvd[h]
  auto load_ld = [&](const Step& x, int qb, auto hc) {
    constexpr int h = decltype(hc)::value;
    const uint32_t a = x.l2 + 4u * (uint32_t)(32 * qb + 16 * h);
    const f32x4 l0 = *(lds_f4*)(uintptr_t)a;
    const f32x4 l1 = *(lds_f4*)(uintptr_t)(a + 16);
    const f32x4 d0 = *(lds_f4*)(uintptr_t)(a + kDscMinusL2);
    const f32x4 d1 = *(lds_f4*)(uintptr_t)(a + kDscMinusL2 + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lvd[h][e] = l0[e];
      lvd[h][4 + e] = l1[e];
      lvd[h][8 + e] = d0[e];
      lvd[h][12 + e] = d1[e];
    }
  };
  // piece pc of block (x, qb); (xn, qbn) is the block whose softmax follows
  // (none when !has_next)
  auto softmax_piece = [&](const Step& x, int qb, auto pc, auto masked, const Step& xn, int qbn, bool has_next) {
    constexpr int piece = decltype(pc)::value, h = piece >> 2, e0 = 2 * (piece & 3);
    constexpr bool M = decltype(masked)::value;
    if constexpr (DROP && piece == 0) {
      // dropout mask of this 32-row block: lane q of each 4-lane group
      // computes the 4 x 4 block of rows 16 (q / 2) + 8 g + 4 (q % 2) .. + 3
      // and the group's keys; after the byte and word exchange dm[x] holds
      // this key's column of block x, row r in byte r
      const int qd = col & 3;
      uint32_t w[4] = {(uint32_t)my_key >> 2,
                       (uint32_t)(x.q0 + 32 * qb + 16 * (qd >> 1) + 8 * g + 4 * (qd & 1)) >> 2, (uint32_t)bh,
                       drop.offset};
      philox4x32_10(w, drop.k0, drop.k1);
      uint32_t cols[4];
      byte_transpose(w, cols);
      quad_transpose(cols, dm, qd);
    }
    if constexpr ((piece & 3) == 0) {
      if constexpr (h == 0) load_ld(x, qb, ic<1>{});
      else if (has_next) load_ld(xn, qbn, ic<0>{});
      // masked pairs of this chunk: e < dead (row q0 + 32 qb + 16 h + 8 g + e
      // sees key my_key iff my_key <= that row, and only keys below Nk exist)
      if constexpr (M) {
        dead = CAUSAL ? my_key - (x.q0 + 32 * qb + 16 * h + 8 * g) : 0;
        dead = my_key >= Nk ? 8 : dead;
      }
    }
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e) {
      float pe = fast_exp2(fmaf(s[qb][8 * h + e], c, -lvd[h][e]));
      if constexpr (M) pe = e < dead ? 0.f : pe;
      if constexpr (DROP) {
        // a dropped pair adds nothing to dV and its dP term vanishes from dS'
        const bool keep = kept(dm[2 * h + (e >> 2)], e & 3, drop.t);
        pv[e] = keep ? pe : 0.f;
        dv8[e] = pe * fmaf(dp[qb][8 * h + e], keep ? scale_r : 0.f, -lvd[h][8 + e]);
      } else {
        pv[e] = pe;
        dv8[e] = pe * fmaf(dp[qb][8 * h + e], scale, -lvd[h][8 + e]);
      }
    }
    if constexpr ((piece & 3) == 3) {
      pb[qb][h] = pack_bf16x8(pv);
      dsb[qb][h] = pack_bf16x8(dv8);
    }
  };
  // the softmax pieces of 8 that go beside group k of n
  auto pieces = [&](auto k, auto n, auto&& piece) {
    constexpr int K = decltype(k)::value, Nn = decltype(n)::value;
    static_for<(8 * K) / Nn, (8 * (K + 1)) / Nn>(piece);
  };
  // the products of the previous run read block qb's P / dS', which the
  // softmax beside this run rewrites
  auto release_p = [&](int qb) {
    pin(pb[qb][0]);
    pin(pb[qb][1]);
    pin(dsb[qb][0]);
    pin(dsb[qb][1]);
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

  // ---- prologue: A0(0), A1(0) with softmax(0, block 0) beside A1
  wait_loads();
  __syncthreads();  // tile 0 visible
  if (n_steps > 1) issue_qtile(1u, q_first + kBQ);
  {
    const Step x0 = step_ctx(0);
    load_ld(x0, 0, ic<0>{});
    run(ic<2 * G>{},
        [&](auto gi, bf16x8(&o)[2]) { load_a(x0, gi / G, gi % G, o); },
        [&](auto gi, const bf16x8(&o)[2]) { mfma_a(gi / G, gi % G, o); },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value;
          if constexpr (n >= G)
            pieces(ic<n - G>{}, ic<G>{}, [&](auto pc) { softmax_piece(x0, 0, pc, with_masks, x0, 1, true); });
        });
  }
  wait_loads();  // this wave's copies of tile 1 have landed

  // ---- steady state: A0(st+1) | C0(st) | A1(st+1) | C1(st), softmax(st, 1)
  // beside the first two phases and softmax(st+1, 0) beside the last two
  // BUFC: buffer of step st's tile when known at compile time (else -1);
  // step st+1's tile sits in the next one
  auto iterate = [&](const Step& xc, const Step& xn, auto masked, auto bufc) {
    constexpr int BUFC = decltype(bufc)::value;
    run(ic<4 * G>{},
        [&](auto gi, bf16x8(&o)[2]) {
          constexpr int n = decltype(gi)::value, ph = n / G, i = n % G;
          if constexpr (BUFC >= 0) {
            if constexpr (ph == 0 || ph == 2) load_a_c(ic<(BUFC + 1) % kTiles>{}, ph >> 1, i, o);
            else load_c_c(ic<BUFC>{}, 2 * (ph >> 1) + i / NDB, i % NDB, o);
          } else {
            if constexpr (ph == 0 || ph == 2) load_a(xn, ph >> 1, i, o);   // A0, A1 of step st+1
            else load_c(xc, 2 * (ph >> 1) + i / NDB, i % NDB, o);          // C0, C1 of step st
          }
        },
        [&](auto gi, const bf16x8(&o)[2]) {
          constexpr int n = decltype(gi)::value, ph = n / G, i = n % G;
          if constexpr (ph == 0 || ph == 2) mfma_a(ph >> 1, i, o);
          else mfma_c(2 * (ph >> 1) + i / NDB, i % NDB, o);
        },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value;
          if constexpr (n == 0) release_p(1);      // read by C1(st-1)
          if constexpr (n == 2 * G) release_p(0);  // read by C0(st)
          if constexpr (n < 2 * G)
            pieces(ic<n>{}, ic<2 * G>{}, [&](auto pc) { softmax_piece(xc, 1, pc, masked, xn, 0, true); });
          else
            pieces(ic<n - 2 * G>{}, ic<2 * G>{}, [&](auto pc) { softmax_piece(xn, 0, pc, masked, xn, 1, true); });
        });
  };
  auto step = [&](int st, auto masked) {
    __syncthreads();  // tile st+1 visible; every wave is done with tile st-1
    if (st + 2 < n_steps) issue_qtile((uint32_t)((st + 2) % kTiles), q_first + (st + 2) * kBQ);
    iterate(step_ctx(st), step_ctx(st + 1), masked, ic<-1>{});
    wait_loads();  // this wave's copies of tile st+2 have landed
  };
  // the same with step st's tile in buffer BUF (st % 3 == BUF)
  auto step_c = [&](int st, auto buf) {
    constexpr int BUF = decltype(buf)::value;
    __syncthreads();
    if (st + 2 < n_steps) issue_qtile((uint32_t)((BUF + 2) % kTiles), q_first + (st + 2) * kBQ);
    iterate(step_ctx_c(st, buf), step_ctx_c(st + 1, ic<(BUF + 1) % kTiles>{}), no_masks, buf);
    wait_loads();
  };
  // Steps that need masks form a prefix: the ones that meet the diagonal, or
  // all of them in the block that holds the end of the sequence.  Iteration
  // st touches steps st and st+1, so it needs masks iff st < n_mask.  Two
  // loops rather than a branch per iteration keep one register assignment
  // per loop body.
  const int n_mask = k0 + kBKV > Nk ? n_steps : CAUSAL ? min(n_steps, (k0 + kBKV - q_first + kBQ - 1) / kBQ) : 0;
  int st = 0;
  for (; st + 1 < n_steps && st < n_mask; ++st) step(st, with_masks);
  // mask-free steps three at a time from a multiple of 3: tile st + i in buffer i
  for (; st + 1 < n_steps && st % kTiles != 0; ++st) step(st, no_masks);
  for (; st + 3 < n_steps; st += 3) {
    step_c(st, ic<0>{});
    step_c(st + 1, ic<1>{});
    step_c(st + 2, ic<2>{});
  }
  for (; st + 1 < n_steps; ++st) step(st, no_masks);

  // ---- last step: C0 with softmax(block 1) beside it, then C1
  {
    const Step xc = step_ctx(n_steps - 1);
    run(ic<2 * G>{},
        [&](auto gi, bf16x8(&o)[2]) { load_c(xc, 2 * (gi / G) + (gi % G) / NDB, (gi % G) % NDB, o); },
        [&](auto gi, const bf16x8(&o)[2]) { mfma_c(2 * (gi / G) + (gi % G) / NDB, (gi % G) % NDB, o); },
        [&](auto gi) {
          constexpr int n = decltype(gi)::value;
          if constexpr (n == 0) release_p(1);
          if constexpr (n < G)
            pieces(ic<n>{}, ic<G>{}, [&](auto pc) { softmax_piece(xc, 1, pc, with_masks, xc, 0, false); });
        });
  }

  // every MFMA has completed once fin exists: operand registers may be reused
  const float fin = dk_acc[NDB - 1][0] + dv_acc[NDB - 1][0];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
    pin(op[j][0], fin);
    pin(op[j][1], fin);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    pin(pb[j][0], fin);
    pin(pb[j][1], fin);
    pin(dsb[j][0], fin);
    pin(dsb[j][1], fin);
  }
  group_fence();  // nothing after this point is scheduled above the pins

  if (my_key < Nk) {
    float* dKrow = dK + khead + (size_t)my_key * D;
    float* dVrow = dV + khead + (size_t)my_key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * g;
        *reinterpret_cast<float4*>(dKrow + d) =
            make_float4(dk_acc[db][4 * i4], dk_acc[db][4 * i4 + 1], dk_acc[db][4 * i4 + 2], dk_acc[db][4 * i4 + 3]);
        const float rv = DROP ? drop.r : 1.f;  // kept weights carry the factor 256 / (256 - t)
        *reinterpret_cast<float4*>(dVrow + d) = make_float4(rv * dv_acc[db][4 * i4], rv * dv_acc[db][4 * i4 + 1],
                                                            rv * dv_acc[db][4 * i4 + 2], rv * dv_acc[db][4 * i4 + 3]);
      }
  }
}

template <int D>
hipError_t launch_prep(const void* dout, const float* o, const float* lse, float* ws, int BH, int N, float scale,
                       hipStream_t stream) {
  const long long rows = (long long)BH * N;
  constexpr int RPB = 256 / (D / 8);
  const long long pre_grid = (rows + RPB - 1) / RPB;
  if (pre_grid > (1LL << 31) - 1) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_grid), dim3(256), 0, stream,
                     static_cast<const bf16_raw*>(dout), o, lse, ws, ws + rows, rows, scale);
  return hipGetLastError();
}

// BH, Nq: heads and query rows; for packed sequences the B * H (sequence,
// head) units and the longest length, the workspace then holding H * total
// rows.
long long workspace_rows(int BH, int Nq, const Seqs& sq) {
  return sq.cu ? (long long)sq.H * sq.total : (long long)BH * Nq;
}

template <int D, bool CAUSAL, bool DROP, bool STRIDED = false>
hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* ws, float* dk,
                       float* dv, int BH, int Nq, int Nk, float scale, const Dropout& drop, const Seqs& sq,
                       const Strides& lay, hipStream_t stream) {
  const long long rows = workspace_rows(BH, Nq, sq);
  const int n_kvblk = (Nk + kBKV - 1) / kBKV;
  const long long total = (long long)BH * n_kvblk;
  if (total == 0) return hipSuccess;  // no keys: no dK, dV
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, DROP, STRIDED>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k), static_cast<const bf16_raw*>(v),
                     static_cast<const bf16_raw*>(dout), ws + rows, ws, dk, dv, Nq, Nk, n_kvblk, (int)total, scale,
                     scale * kLog2e, drop, sq, lay);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const void* dout, const float* o, const float* lse, float* ws, int BH, int N, int d,
                           float scale, hipStream_t stream) {
  return d == 128 ? launch_prep<128>(dout, o, lse, ws, BH, N, scale, stream)
                  : launch_prep<64>(dout, o, lse, ws, BH, N, scale, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv_drop(const void* q, const void* k, const void* v, const void* dout, const float* ws,
                            float* dk, float* dv, int BH, int Nq, int Nk, float scale, const Dropout* drop,
                            const Seqs& sq, const Strides* lay, hipStream_t stream) {
  if (lay) {
    // strided views: dense packing of sequences and dropout are not offered
    if (drop || sq.cu) return hipErrorInvalidValue;
    return launch_dkdv<D, CAUSAL, false, true>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, Dropout{}, sq, *lay,
                                               stream);
  }
  const Strides dense = dense_strides(Nq, Nk, D);
  if (drop) {
    if (sq.cu) return hipErrorInvalidValue;  // dropout is offered for the dense layout only
    return launch_dkdv<D, CAUSAL, true>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, *drop, sq, dense, stream);
  }
  return launch_dkdv<D, CAUSAL, false>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, Dropout{}, sq, dense, stream);
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* ws,
                           float* dk, float* dv, int BH, int Nq, int Nk, int d, float scale, int causal,
                           const Dropout* drop, const Seqs* seqs, hipStream_t stream, const Strides* lay) {
  const Seqs sq = seqs ? *seqs : Seqs{nullptr, 0, 0};
  if (d == 128)
    return causal ? launch_dkdv_drop<128, true>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, drop, sq, lay, stream)
                  : launch_dkdv_drop<128, false>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, drop, sq, lay, stream);
  return causal ? launch_dkdv_drop<64, true>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, drop, sq, lay, stream)
                : launch_dkdv_drop<64, false>(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, scale, drop, sq, lay, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* ws, int BH, int Nq, int Nk,
                           int d, float scale, int causal, const Dropout* drop, const Seqs* seqs,
                           hipStream_t stream, const Strides* lay) {
  const Seqs sq = seqs ? *seqs : Seqs{nullptr, 0, 0};
  const long long rows = workspace_rows(BH, Nq, sq);
  // The dQ pass computes the row statistics of its own rows (the
  // preprocess, fused: every row belongs to exactly one of its workgroups)
  // and stores them for the dK/dV pass, which runs after it on the stream.
  hipError_t e = launch_bwd_dq_fused(q, k, v, dout, o, lse, ws + rows, ws, dq, BH, Nq, Nk, d, scale, causal, drop,
                                     seqs, stream, lay);
  if (e != hipSuccess) return e;
  return launch_bwd_dkdv(q, k, v, dout, ws, dk, dv, BH, Nq, Nk, d, scale, causal, drop, seqs, stream, lay);
}

}  // namespace fa

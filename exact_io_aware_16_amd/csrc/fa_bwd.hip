// Exact attention backward by recomputation, bf16 inputs, float32 gradients.
//
// The pages keep Q, K, V, O and the per-row logsumexp L from the forward and
// rebuild the score and probability tiles when the gradients need them ("The
// forward pass is only half of it", FlashAttention: The Matrix You Never
// Have to Write Down; "Backward can recreate tiles instead of retaining the
// square", leviathansystems.co).  They give no gradient formulas; the
// kernels use the chain rule on softmax(scale Q K^T) V:
//   P = exp(scale S - L),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_j P_ij dP_ij = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// The factor `scale` is folded into dS once: the kernels form
//   dS' = scale dS = P * (scale dP - scale D)
// (scale D comes from the preprocess), so dK = dS'^T Q and dQ = dS' K.
//
// Kernels (three launches, no atomics, every output written once):
//  * bwd_pre_kernel: per query row scale * (dO_i . O_i) and L_i log2(e) into
//    the workspace.
//  * bwd_dkdv_kernel: one workgroup per (head, block of 128 keys).  Each of
//    its 4 waves owns 32 keys: their V rows stay in registers (B operands of
//    dP = dO V^T), their K rows come from the block's K tile in LDS (B
//    operands of S = Q K^T), and dK^T, dV^T accumulate in registers.  The
//    workgroup walks the query rows 64 at a time (causal: from the block's
//    diagonal on).  Per step:
//      A. S and dP for the 64 rows of the tile (Q and dO tiles arrive by
//         LDS-direct buffer loads, double buffered, rows in perm32 order so
//         that S and dP come out with 8 consecutive query rows per register
//         octet -- the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS');
//      B. P and dS' on the vector ALUs;
//      C. dV^T += dO^T P and dK^T += Q^T dS', the A operands read from the
//         row-major tiles with ds_read_b64_tr_b16.
//    One barrier per step publishes the tile and frees the buffer the step
//    refills.
//  * bwd_dq_kernel (fa_bwd_dq.hip): query-stationary, recomputes S and dP
//    per key tile and accumulates dQ in registers.
// dQ is not accumulated across key blocks with atomics: on this part
// device-scope float atomics are performed at the memory side, and the
// partial sums of every key block would cross the fabric once each; the
// second recomputation of S and dP costs less.
//  One 16-byte-slot XOR swizzle per row width serves both the row reads and
//  the transpose reads of a tile without LDS bank conflicts; every per-lane
//  LDS address is a lane constant XOR a compile-time mask, plus an
//  immediate.
#include "fa_common.h"
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

template <int D>
struct DkdvSmem {
  bf16_raw q[2][kBQ * D];        // Q tiles, rows in perm32 order
  bf16_raw dout[2][kBQ * D];     // dO tiles, rows in perm32 order
  float l2[2][kBQ];              // L log2(e) of the tile's rows
  float dsc[2][kBQ];             // scale * D of the tile's rows
};

// 16-byte chunks a thread copies for one BQ x D query tile: LDS block
// (i*4 + wave) of 1 KiB, lane l -> row r, slot s; the source is row
// perm32(r) (within 32) and chunk s ^ swz(r).
template <int D>
struct QCopy {
  static constexpr int SLOTS = D / 8;
  static constexpr int ROWS_PER_INSTR = 64 / SLOTS;
  static constexpr int INSTR = kBQ * SLOTS / kThreads;
  uint32_t off[INSTR];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int r = (i * kWaves + wave) * ROWS_PER_INSTR + lane / SLOTS;
      const int slot = lane % SLOTS;
      off[i] = (uint32_t)(((r & ~31) + perm32(r & 31)) * D * 2 + 16 * (slot ^ swz<D * 2>(r)));
    }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const bf16_raw* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dsc,
    float* __restrict__ dK, float* __restrict__ dV, int N, int n_kvblk, int total, float scale, float c) {
  constexpr int NKK = D / 16;  // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;  // 32-row blocks of dK^T / dV^T
  constexpr int RB = D * 2;    // bytes per Q / dO / K row
  constexpr uint32_t kTileBytes = kBQ * D * 2;
  constexpr uint32_t kDoutMinusQ = 2 * kTileBytes;  // sm.dout[b] - sm.q[b]
  constexpr uint32_t kDscMinusL2 = 2 * kBQ * 4;     // sm.dsc[b] - sm.l2[b]
  __shared__ __attribute__((aligned(1024))) DkdvSmem<D> sm;

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int bh = blk / n_kvblk;
  const int kvb = blk - bh * n_kvblk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  const size_t head = (size_t)bh * N * D;

  const int k0 = kvb * kBKV;
  const int my_key = k0 + 32 * wave + col;

  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Q + head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t grs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dO + head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t lrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(L2 + (size_t)bh * N), (short)0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(Dsc + (size_t)bh * N), (short)0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head), (short)0, head_bytes, 0x00020000);

  QCopy<D> qc;
  qc.init(wave, lane);
  // Q / dO / L2 / scale*D of one query tile into buffer b
  // (the tile offset goes into the range-checked per-lane offset, so rows
  // past the end of the head read as zeros)
  auto issue_qtile = [&](uint32_t b, int q0) {
    const uint32_t toff = (uint32_t)q0 * D * 2;
    const uint32_t qb = lds_addr_of(sm.q[b]), gb = lds_addr_of(sm.dout[b]);
#pragma unroll
    for (int i = 0; i < QCopy<D>::INSTR; ++i) {
      lds_copy(qrs, qc.off[i] + toff, 0u, qb + (uint32_t)(i * kWaves + wave) * 1024u);
      lds_copy(grs, qc.off[i] + toff, 0u, gb + (uint32_t)(i * kWaves + wave) * 1024u);
    }
    if (wave == 0) lds_copy4(lrs, (uint32_t)(q0 + lane) * 4u, 0u, lds_addr_of(sm.l2[b]));
    if (wave == 1) lds_copy4(drs, (uint32_t)(q0 + lane) * 4u, 0u, lds_addr_of(sm.dsc[b]));
  };

  const int q_first = CAUSAL ? k0 : 0;  // k0 is a multiple of kBQ
  const int n_steps = (N - q_first + kBQ - 1) / kBQ;

  issue_qtile(0u, q_first);

  // K and V rows of this wave's keys, 8 head-dim elements per k-slice: the
  // B operands of S = Q K^T and dP = dO V^T for the whole kernel (rows past
  // N read as zero)
  bf16x8 kres[NKK], vres[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const uint32_t off = (uint32_t)(my_key * D + 16 * kk + 8 * g) * 2u;
    kres[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0));
    vres[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0));
    // kept in AGPRs, which the matrix cores read directly
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

  // Operand register sets (see pin()).  Each MFMA phase keeps three sets and
  // loads group g + 2 while group g runs: the set it overwrites was last
  // read by group g - 1, which has started once group g is issued.
  //   ar: Q / dO rows of the S and dP products (one query block, k-slice)
  //   at: dO^T / Q^T transpose reads of the dV and dK products
  //   pb, dsb: P and dS' tiles (B operands)
  constexpr int NCG = 4 * NDB;  // (query block, half, head-dim block) groups of phase C
  constexpr int NAG = 2 * NKK;   // (k-slice, query block) groups of phase A
  bf16x8 ar[3][2], at[3][2], pb[2][2], dsb[2][2];
#pragma unroll
  for (int j = 0; j < 3; ++j) ar[j][0] = ar[j][1] = at[j][0] = at[j][1] = bf16x8{};
#pragma unroll
  for (int j = 0; j < 2; ++j) pb[j][0] = pb[j][1] = dsb[j][0] = dsb[j][1] = bf16x8{};

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

  wait_loads();
  for (int st = 0; st < n_steps; ++st) {
    const int q0 = q_first + st * kBQ;
    const uint32_t buf = (uint32_t)(st & 1);
    __syncthreads();  // tile st visible; every wave is done with tile st-1
    if (st + 1 < n_steps) issue_qtile(buf ^ 1u, q0 + kBQ);
    const uint32_t qbase = q_base0 + buf * kTileBytes;

    // The step runs as four MFMA phases; the softmax of one query block
    // runs on the vector ALUs between the MFMA groups of the next phase:
    //   A0: S, dP of query block 0      A1: S, dP of block 1  + softmax(0)
    //   C0: dV, dK from block 0 + softmax(1)      C1: dV, dK from block 1
    f32x16 s[2], dp[2];
    const uint32_t qrow = opaque(qbase + row_lane);
    // phase-A group ga = NKK qb + kk: Q and dO rows of block qb, k-slice kk
    auto load_a = [&](int ga) {
      const int qb = ga / NKK, kk = ga % NKK;
      const uint32_t ra = (qrow ^ (uint32_t)(32 * kk)) + (uint32_t)(32 * qb * RB);
      ar[ga % 3][0] = lds_row16(ra);
      ar[ga % 3][1] = lds_row16(ra + kDoutMinusQ);
    };
    const uint32_t tq = opaque(qbase + tq_lane);
    const uint32_t tq1 = opaque(tq ^ 32u);  // row + 8: swizzle ^ 2
    // phase-C group gi = NDB (2 qb + h) + db
    auto load_c = [&](int gi) {
      const int qh = gi / NDB, db = gi % NDB;  // qh = 2 qb + h
      bf16x8(&a)[2] = at[gi % 3];
      const uint32_t rows = (uint32_t)(16 * qh * RB);
      const uint32_t o0 = (tq ^ (uint32_t)(64 * db)) + rows;
      const uint32_t o1 = (tq1 ^ (uint32_t)(64 * db)) + rows + 8 * RB;
      a[0] = tr_pair(o0 + kDoutMinusQ, o1 + kDoutMinusQ);
      a[1] = tr_pair(o0, o1);
    };

    // ---- softmax of query block qb in 8 pieces of 2 elements per lane:
    // P = exp2(S c - L log2 e), dS' = P (scale dP - scale D); masked pairs get 0
    const bool need_mask = (CAUSAL && q0 < k0 + kBKV) || k0 + kBKV > N;
    const uint32_t l2_addr = l2_base0 + buf * (kBQ * 4) + (uint32_t)(32 * g);
    float lv[8], dd[8], pv[8], dv8[8];
    int dead = 0;
    auto softmax_piece = [&](int qb, int piece) {
      const int h = piece >> 2, e0 = 2 * (piece & 3);
      const uint32_t qr = (uint32_t)(32 * qb + 16 * h);  // + 8 g: 8 consecutive local query rows
      if ((piece & 3) == 0) {
        const f32x4 l0 = *(lds_f4*)(uintptr_t)(l2_addr + 4 * qr);
        const f32x4 l1 = *(lds_f4*)(uintptr_t)(l2_addr + 4 * qr + 16);
        const f32x4 d0 = *(lds_f4*)(uintptr_t)(l2_addr + kDscMinusL2 + 4 * qr);
        const f32x4 d1 = *(lds_f4*)(uintptr_t)(l2_addr + kDscMinusL2 + 4 * qr + 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lv[e] = l0[e];
          lv[4 + e] = l1[e];
          dd[e] = d0[e];
          dd[4 + e] = d1[e];
        }
        // masked pairs of this chunk: e < dead (row q0 + qr + 8 g + e sees
        // key my_key iff my_key <= that row, and only keys below N exist)
        if (need_mask) {
          dead = CAUSAL ? my_key - (q0 + (int)qr + 8 * g) : 0;
          dead = my_key >= N ? 8 : dead;
        }
      }
#pragma unroll
      for (int e = e0; e < e0 + 2; ++e) {
        float pe = fast_exp2(fmaf(s[qb][8 * h + e], c, -lv[e]));
        if (need_mask) pe = e < dead ? 0.f : pe;
        pv[e] = pe;
        dv8[e] = pe * fmaf(dp[qb][8 * h + e], scale, -dd[e]);
      }
      if ((piece & 3) == 3) {
        pb[qb][h] = pack_bf16x8(pv);
        dsb[qb][h] = pack_bf16x8(dv8);
      }
    };

    // ---- A0, A1: S = Q K^T and dP = dO V^T, 32 query rows x this wave's 32 keys each
    load_a(0);
    load_a(1);
#pragma unroll
    for (int ga = 0; ga < NAG; ++ga) {
      const int qb = ga / NKK, kk = ga % NKK;
      s[qb] = mfma32(ar[ga % 3][0], kres[kk], kk == 0 ? f32x16{} : s[qb]);
      dp[qb] = mfma32(ar[ga % 3][1], vres[kk], kk == 0 ? f32x16{} : dp[qb]);
      anchor_a(s[qb]);
      anchor_a(dp[qb]);
      group_fence();
      if (ga == 0) {  // operands of step st-1's dV / dK products are released
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          pin(at[j][0]);
          pin(at[j][1]);
        }
        pin(pb[1][1]);
        pin(dsb[1][1]);
      }
      pin(ar[(ga + 2) % 3][0]);
      pin(ar[(ga + 2) % 3][1]);
      if (ga + 2 < NAG) load_a(ga + 2);
      if (ga + 2 == NAG) load_c(0);
      if (ga + 1 == NAG) load_c(1);
      if (qb == 1) {  // softmax of block 0 while block 1's products run
#pragma unroll
        for (int pc = 0; pc < 8 / NKK; ++pc) softmax_piece(0, kk * (8 / NKK) + pc);
      }
    }

    // ---- C0, C1: dV^T += dO^T P and dK^T += Q^T dS', contraction over the
    // query rows; A operands by transpose reads
#pragma unroll
    for (int gi = 0; gi < NCG; ++gi) {
      const int qh = gi / NDB, db = gi % NDB;
      const int qb = qh >> 1, h = qh & 1;
      bf16x8(&a)[2] = at[gi % 3];
      dv_acc[db] = mfma32(a[0], pb[qb][h], dv_acc[db]);
      dk_acc[db] = mfma32(a[1], dsb[qb][h], dk_acc[db]);
      anchor_a(dv_acc[db]);
      anchor_a(dk_acc[db]);
      group_fence();
      if (gi == 0) {  // operands of the S / dP products are released
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          pin(ar[j][0]);
          pin(ar[j][1]);
        }
      }
      if (db == 0 && qh > 0) {  // first group of (qb, h): the previous P / dS' pair is released
        pin(pb[(qh - 1) >> 1][(qh - 1) & 1]);
        pin(dsb[(qh - 1) >> 1][(qh - 1) & 1]);
      }
      pin(at[(gi + 2) % 3][0]);
      pin(at[(gi + 2) % 3][1]);
      if (gi + 2 < NCG) load_c(gi + 2);
      if (qb == 0) {  // softmax of block 1 while block 0's products run
#pragma unroll
        for (int pc = 0; pc < 4 / NDB; ++pc) softmax_piece(1, gi * (4 / NDB) + pc);
      }
    }
    wait_loads();  // this wave's copies of tile st+1 have landed
  }

  // every MFMA has completed once fin exists: operand registers may be reused
  const float fin = dk_acc[NDB - 1][0] + dv_acc[NDB - 1][0];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    pin(at[j][0], fin);
    pin(at[j][1], fin);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    pin(pb[j][0], fin);
    pin(pb[j][1], fin);
    pin(dsb[j][0], fin);
    pin(dsb[j][1], fin);
  }
  group_fence();  // nothing after this point is scheduled above the pins

  if (my_key < N) {
    float* dKrow = dK + head + (size_t)my_key * D;
    float* dVrow = dV + head + (size_t)my_key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * g;
        *reinterpret_cast<float4*>(dKrow + d) =
            make_float4(dk_acc[db][4 * i4], dk_acc[db][4 * i4 + 1], dk_acc[db][4 * i4 + 2], dk_acc[db][4 * i4 + 3]);
        *reinterpret_cast<float4*>(dVrow + d) =
            make_float4(dv_acc[db][4 * i4], dv_acc[db][4 * i4 + 1], dv_acc[db][4 * i4 + 2], dv_acc[db][4 * i4 + 3]);
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

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* ws, float* dk,
                       float* dv, int BH, int N, float scale, hipStream_t stream) {
  const long long rows = (long long)BH * N;
  const int n_kvblk = (N + kBKV - 1) / kBKV;
  const long long total = (long long)BH * n_kvblk;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k), static_cast<const bf16_raw*>(v),
                     static_cast<const bf16_raw*>(dout), ws + rows, ws, dk, dv, N, n_kvblk, (int)total, scale,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep(const void* dout, const float* o, const float* lse, float* ws, int BH, int N, int d,
                           float scale, hipStream_t stream) {
  return d == 128 ? launch_prep<128>(dout, o, lse, ws, BH, N, scale, stream)
                  : launch_prep<64>(dout, o, lse, ws, BH, N, scale, stream);
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* ws,
                           float* dk, float* dv, int BH, int N, int d, float scale, int causal, hipStream_t stream) {
  if (d == 128) return causal ? launch_dkdv<128, true>(q, k, v, dout, ws, dk, dv, BH, N, scale, stream)
                              : launch_dkdv<128, false>(q, k, v, dout, ws, dk, dv, BH, N, scale, stream);
  return causal ? launch_dkdv<64, true>(q, k, v, dout, ws, dk, dv, BH, N, scale, stream)
                : launch_dkdv<64, false>(q, k, v, dout, ws, dk, dv, BH, N, scale, stream);
}

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* ws, int BH, int N, int d,
                           float scale, int causal, hipStream_t stream) {
  hipError_t e = launch_bwd_prep(dout, o, lse, ws, BH, N, d, scale, stream);
  if (e != hipSuccess) return e;
  e = launch_bwd_dkdv(q, k, v, dout, ws, dk, dv, BH, N, d, scale, causal, stream);
  if (e != hipSuccess) return e;
  const long long rows = (long long)BH * N;
  return launch_bwd_dq_bf16(q, k, v, dout, ws + rows, ws, dq, BH, N, d, scale, causal, stream);
}

}  // namespace fa

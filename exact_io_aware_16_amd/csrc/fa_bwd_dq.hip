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
//  * each wave owns 32 query rows; their Q and dO rows stay in registers as
//    the B operands of S^T = K Q^T and dP^T = V dO^T (keys along M), so a
//    query's values sit in one lane pair and its L and D are lane scalars;
//  * K and V tiles of BC keys arrive by LDS-direct buffer loads, double
//    buffered, rows in perm32 order with the backward's slot swizzle: the
//    S^T / dP^T results then hold 8 consecutive keys per register octet --
//    the B-operand layout of dQ^T += K^T dS'^T -- and the K^T operand is a
//    transpose read of the same K tile;
//  * causal: query block qb visits key tiles up to its diagonal only, masks
//    are applied only on tiles that straddle the diagonal or the ragged end.
#include "fa_common.h"
#include "fa_launch.h"
#include "fa_lds.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup

template <int D> struct DqTile;
template <> struct DqTile<128> { static constexpr int BC = 64; };
template <> struct DqTile<64> { static constexpr int BC = 128; };

template <int D>
struct DqSmem {
  static constexpr int BC = DqTile<D>::BC;
  bf16_raw k[2][BC * D];  // K tiles: row r holds key perm32(r) of its 32-row group
  bf16_raw v[2][BC * D];  // V tiles, same layout
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
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const bf16_raw* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dsc,
    float* __restrict__ dQ, int N, int n_qblk, int total, float scale, float c) {
  constexpr int BC = DqTile<D>::BC;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NKK = D / 16;   // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;   // 32-row blocks of dQ^T
  constexpr int RB = D * 2;     // bytes per row
  constexpr uint32_t kTileBytes = BC * D * 2;
  constexpr uint32_t kVMinusK = 2 * kTileBytes;  // sm.v[b] - sm.k[b]
  __shared__ __attribute__((aligned(1024))) DqSmem<D> sm;

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int bh = blk / n_qblk;
  int qblk = blk - bh * n_qblk;
  if (CAUSAL) qblk = n_qblk - 1 - qblk;  // longest rows first

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  const size_t head = (size_t)bh * N * D;

  const int q_start = qblk * kBR;
  const int q0w = q_start + 32 * wave;
  const int my_q = q0w + col;
  const int kv_end = CAUSAL ? min(N, q_start + kBR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(K + head), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(V + head), (short)0, head_bytes, 0x00020000);
  KvCopy<D> kc;
  kc.init(wave, lane);
  auto issue_tile = [&](uint32_t b, int key0) {
    const uint32_t toff = (uint32_t)key0 * D * 2;
    const uint32_t kb = lds_addr_of(sm.k[b]), vb = lds_addr_of(sm.v[b]);
#pragma unroll
    for (int i = 0; i < KvCopy<D>::INSTR; ++i) {
      lds_copy(krs, kc.off[i] + toff, 0u, kb + (uint32_t)(i * kWaves + wave) * 1024u);
      lds_copy(vrs, kc.off[i] + toff, 0u, vb + (uint32_t)(i * kWaves + wave) * 1024u);
    }
  };
  issue_tile(0u, 0);

  // this lane's query row: Q and dO slices (B operands), L log2(e), scale D
  bf16x8 qf[NKK], dof[NKK];
  float l2q, dq_sc;
  {
    const int qr = min(my_q, N - 1);
    const bf16_raw* Qrow = Q + head + (size_t)qr * D;
    const bf16_raw* Grow = dO + head + (size_t)qr * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = as_bf16x8(ld16(Qrow + 16 * kk + 8 * g));
      dof[kk] = as_bf16x8(ld16(Grow + 16 * kk + 8 * g));
    }
    l2q = L2[(size_t)bh * N + qr];
    dq_sc = Dsc[(size_t)bh * N + qr];
  }

  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq_acc[db][i] = 0.f;

  // Operand register sets (see pin()).  Each MFMA phase keeps three sets
  // and loads group g + 2 while group g runs: the set it overwrites was last
  // read by group g - 1, which has started once group g is issued.
  //   ar: K and V rows of the S^T and dP^T products (one key block, k-slice)
  //   at: K^T transpose reads of the dQ product (two head-dim blocks)
  //   dsb: dS'^T tiles (B operands)
  constexpr int NAG = NKB * NKK;      // (key block, k-slice) groups of the score phase
  constexpr int NDG = NKB * NDB;      // (key block, half, pair of head-dim blocks) groups of the dQ phase
  constexpr int PPA = 8 / NKK;        // softmax pieces per score group
  constexpr int PPD = 8 / (2 * (NDB / 2));  // softmax pieces per dQ group of key block 0
  bf16x8 ar[3][2], at[3][2], dsb[NKB][2];
#pragma unroll
  for (int j = 0; j < 3; ++j) ar[j][0] = ar[j][1] = at[j][0] = at[j][1] = bf16x8{};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) dsb[kb][0] = dsb[kb][1] = bf16x8{};

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
  const int last_key = CAUSAL ? min(my_q, N - 1) : N - 1;  // keys above are masked

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BC;
    const uint32_t buf = (uint32_t)(t & 1);
    // K(t), V(t) have landed (own copies) and are visible (barrier); every
    // wave is done with tile t-1, whose buffers refill now with tile t+1.
    wait_loads();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(buf ^ 1u, key0 + BC);
    const uint32_t kbase = k_base0 + buf * kTileBytes;

    // The tile runs as MFMA phases per 32-key block; the softmax of one
    // block runs on the vector ALUs between the MFMA groups of the next:
    //   S^T, dP^T of block 0 | of block 1 + softmax(0) | ... |
    //   dQ from block 0 + softmax(last) | dQ from the other blocks
    f32x16 st[NKB], dpt[NKB];
    const uint32_t krow = opaque(kbase + row_lane);
    auto load_a = [&](int ga) {
      const int kb = ga / NKK, kk = ga % NKK;
      const uint32_t ra = (krow ^ (uint32_t)(32 * kk)) + (uint32_t)(32 * kb * RB);
      ar[ga % 3][0] = lds_row16(ra);
      ar[ga % 3][1] = lds_row16(ra + kVMinusK);
    };
    const uint32_t tk = opaque(kbase + tk_lane);
    const uint32_t tk1 = opaque(tk ^ 32u);  // row + 8: swizzle ^ 2
    // dQ group gd = (2 kb + h) (NDB / 2) + pair: head-dim blocks 2 pair, 2 pair + 1
    auto load_d = [&](int gd) {
      const int kh = gd / (NDB / 2), pr = gd % (NDB / 2);
      const uint32_t rows = (uint32_t)(16 * kh * RB);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int db = 2 * pr + x;
        at[gd % 3][x] = tr_pair((tk ^ (uint32_t)(64 * db)) + rows, (tk1 ^ (uint32_t)(64 * db)) + rows + 8 * RB);
      }
    };

    // dS'^T = P^T (scale dP^T - scale D), P^T = exp2(S^T c - L log2 e), in
    // 8 pieces of 2 elements per lane; masked pairs get 0
    const bool need_mask = (CAUSAL && key0 + BC - 1 > q0w) || key0 + BC > N;
    float dsv[8];
    auto softmax_piece = [&](int kb, int piece) {
      const int h = piece >> 2, e0 = 2 * (piece & 3);
      // register 8 h + e of half g holds key key0 + 32 kb + 16 h + 8 g + e
      const int lim = last_key - (key0 + 32 * kb + 16 * h + 8 * g);
#pragma unroll
      for (int e = e0; e < e0 + 2; ++e) {
        float pe = fast_exp2(fmaf(st[kb][8 * h + e], c, -l2q));
        if (need_mask) pe = e > lim ? 0.f : pe;
        dsv[e] = pe * fmaf(dpt[kb][8 * h + e], scale, -dq_sc);
      }
      if ((piece & 3) == 3) dsb[kb][h] = pack_bf16x8(dsv);
    };

    // ---- S^T = K Q^T and dP^T = V dO^T, one 32-key block per phase
    load_a(0);
    load_a(1);
#pragma unroll
    for (int ga = 0; ga < NAG; ++ga) {
      const int kb = ga / NKK, kk = ga % NKK;
      st[kb] = mfma32(ar[ga % 3][0], qf[kk], kk == 0 ? f32x16{} : st[kb]);
      dpt[kb] = mfma32(ar[ga % 3][1], dof[kk], kk == 0 ? f32x16{} : dpt[kb]);
      anchor_a(st[kb]);
      anchor_a(dpt[kb]);
      group_fence();
      if (ga == 0) {  // operands of tile t-1's dQ product are released
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          pin(at[j][0]);
          pin(at[j][1]);
        }
        pin(dsb[NKB - 1][1]);
      }
      pin(ar[(ga + 2) % 3][0]);
      pin(ar[(ga + 2) % 3][1]);
      if (ga + 2 < NAG) load_a(ga + 2);
      if (ga + 2 == NAG) load_d(0);
      if (ga + 1 == NAG) load_d(1);
      if (kb > 0) {  // softmax of the previous block
#pragma unroll
        for (int pc = 0; pc < PPA; ++pc) softmax_piece(kb - 1, kk * PPA + pc);
      }
    }

    // ---- dQ^T += K^T dS'^T, K^T by transpose reads of the K tile
#pragma unroll
    for (int gd = 0; gd < NDG; ++gd) {
      const int kh = gd / (NDB / 2), pr = gd % (NDB / 2);
      const int kb = kh >> 1, h = kh & 1;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        dq_acc[2 * pr + x] = mfma32(at[gd % 3][x], dsb[kb][h], dq_acc[2 * pr + x]);
        anchor_a(dq_acc[2 * pr + x]);
      }
      group_fence();
      if (gd == 0) {  // operands of the score products are released
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          pin(ar[j][0]);
          pin(ar[j][1]);
        }
      }
      if (pr == 0 && kh > 0) pin(dsb[(kh - 1) >> 1][(kh - 1) & 1]);  // the previous dS' group is released
      pin(at[(gd + 2) % 3][0]);
      pin(at[(gd + 2) % 3][1]);
      if (gd + 2 < NDG) load_d(gd + 2);
      if (kb == 0) {  // softmax of the last block
#pragma unroll
        for (int pc = 0; pc < PPD; ++pc) softmax_piece(NKB - 1, gd * PPD + pc);
      }
    }
  }

  // every MFMA has completed once fin exists: operand registers may be reused
  float fin = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) fin += dq_acc[db][0];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    pin(at[j][0], fin);
    pin(at[j][1], fin);
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    pin(dsb[kb][0], fin);
    pin(dsb[kb][1], fin);
  }
  group_fence();  // nothing after this point is scheduled above the pins

  if (my_q < N) {
    float* row = dQ + head + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(row + 32 * db + 8 * i4 + 4 * g) =
            make_float4(dq_acc[db][4 * i4], dq_acc[db][4 * i4 + 1], dq_acc[db][4 * i4 + 2], dq_acc[db][4 * i4 + 3]);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* dout, const float* l2, const float* dsc,
                  float* dq, int BH, int N, float scale, hipStream_t stream) {
  const int n_qblk = (N + kBR - 1) / kBR;
  const long long total = (long long)BH * n_qblk;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k), static_cast<const bf16_raw*>(v),
                     static_cast<const bf16_raw*>(dout), l2, dsc, dq, N, n_qblk, (int)total, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout, const float* l2,
                              const float* dsc, float* dq, int BH, int N, int d, float scale, int causal,
                              hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, dout, l2, dsc, dq, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, dout, l2, dsc, dq, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, dout, l2, dsc, dq, BH, N, scale, stream)
                : launch<64, false>(q, k, v, dout, l2, dsc, dq, BH, N, scale, stream);
}

}  // namespace fa

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
//
// Kernels:
//  * bwd_pre_kernel: per query row D_i = dO_i . O_i and L_i log2(e) into the
//    workspace, and dQ := 0.
//  * bwd_main_kernel: one workgroup per (head, block of 128 keys).  Each of
//    its 4 waves owns 32 keys: their K and V rows stay in registers (B
//    operands of S = Q K^T and dP = dO V^T, keys along N), and dK^T, dV^T
//    accumulate in registers.  The workgroup walks the query rows 64 at a
//    time (causal: from the block's diagonal on).  Per query tile:
//      - Q and dO tiles arrive by LDS-direct buffer loads (double buffered);
//        their rows sit in perm32 order so that S and dP come out with 8
//        consecutive query rows per register octet -- the B-operand layout
//        of dV^T = dO^T P and dK^T = Q^T dS, whose A operands (dO^T, Q^T)
//        are read from the same row-major tiles with ds_read_b64_tr_b16;
//      - dS goes to LDS transposed (dS^T, one 16-byte store per octet) and
//        is read back, again with transpose reads, as the A operand of
//        dQ = dS K; K^T comes from the block's K tile in LDS the same way;
//      - dQ partial sums are added to global memory with float32 atomics.
//  One 16-byte-slot XOR swizzle per row width serves both the row reads and
//  the transpose reads of a tile without LDS bank conflicts.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ----------------------------------------------------------------------------------- preprocess
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_raw* __restrict__ dO, const float* __restrict__ O,
                                                       const float* __restrict__ LSE, float* __restrict__ Dvec,
                                                       float* __restrict__ L2, float* __restrict__ dQ,
                                                       long long rows) {
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
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dQ + off) = z;
    *reinterpret_cast<float4*>(dQ + off + 4) = z;
  }
#pragma unroll
  for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (row < rows && part == 0) {
    Dvec[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ----------------------------------------------------------------------------------- main kernel
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 32 * kWaves;  // keys per workgroup
constexpr int kBQ = 64;            // query rows per step

// Slot swizzle for tiles read both row-wise (16 consecutive rows, one 16-byte
// slot each) and by transpose reads (4 consecutive rows x 4 slots): the
// 16-byte slot of chunk c in row r is c ^ swz(r).
template <int ROW_BYTES>
__device__ __forceinline__ constexpr int swz(int r) {
  return ROW_BYTES == 256 ? (4 * (r & 3) | ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) | ((r >> 2) & 3));
}
template <int ROW_BYTES>
__device__ __forceinline__ constexpr int slot_off(int r, int chunk) {
  return r * ROW_BYTES + 16 * (chunk ^ swz<ROW_BYTES>(r));
}

template <int D>
struct BwdSmem {
  bf16_raw k[kBKV * D];        // K block, rows in key order
  bf16_raw v[kBKV * D];        // V block, rows in key order
  bf16_raw q[2][kBQ * D];      // Q tiles, rows in perm32 order
  bf16_raw dout[2][kBQ * D];   // dO tiles, rows in perm32 order
  bf16_raw dst[kBKV * kBQ];    // dS^T: row = key, columns = query rows
  float l2[2][kBQ];
  float dv[2][kBQ];
};

__device__ __forceinline__ void lds_copy(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

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

// A transpose read: four bf16 of one column, 4 consecutive rows; two of them
// make the 8-element operand.
__device__ __forceinline__ bf16x8 tr_pair(const char* base, int off0, int off1) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + off0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + off1));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const bf16_raw* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dvec,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int N, int n_kvblk, int total,
    float scale, float c) {
  constexpr int NKK = D / 16;           // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;           // 32-row blocks of dK^T / dV^T
  constexpr int NQT = 2 * NDB / kWaves; // dQ 32x32 tiles per wave (2 for d=128, 1 for d=64)
  constexpr int RB = D * 2;             // bytes per Q / dO / K row
  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int bh = blk / n_kvblk;
  const int kvb = blk - bh * n_kvblk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;
  const size_t head = (size_t)bh * N * D;
  const bf16_raw* Kh = K + head;
  const bf16_raw* Vh = V + head;

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
      __builtin_amdgcn_make_buffer_rsrc((void*)(Dvec + (size_t)bh * N), (short)0, N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, head_bytes, 0x00020000);

  QCopy<D> qc;
  qc.init(wave, lane);
  // Q / dO / L2 / D of one query tile into buffer b
  // (the tile offset goes into the range-checked per-lane offset, so rows
  // past the end of the head read as zeros)
  auto issue_qtile = [&](int b, int q0) {
    const uint32_t toff = (uint32_t)q0 * D * 2;
    const uint32_t qb = lds_addr_of(sm.q[b]), gb = lds_addr_of(sm.dout[b]);
#pragma unroll
    for (int i = 0; i < QCopy<D>::INSTR; ++i) {
      lds_copy(qrs, qc.off[i] + toff, 0u, qb + (uint32_t)(i * kWaves + wave) * 1024u);
      lds_copy(grs, qc.off[i] + toff, 0u, gb + (uint32_t)(i * kWaves + wave) * 1024u);
    }
    if (wave == 0) lds_copy4(lrs, (uint32_t)(q0 + lane) * 4u, 0u, lds_addr_of(sm.l2[b]));
    if (wave == 1) lds_copy4(drs, (uint32_t)(q0 + lane) * 4u, 0u, lds_addr_of(sm.dv[b]));
  };

  const int q_first = CAUSAL ? k0 : 0;  // k0 is a multiple of kBQ
  const int n_steps = (N - q_first + kBQ - 1) / kBQ;

  // K and V blocks into LDS (natural row order), first query tile
  {
    constexpr int KINSTR = kBKV * (D / 8) / kThreads;
    constexpr int SLOTS = D / 8, RPI = 64 / SLOTS;
#pragma unroll
    for (int i = 0; i < KINSTR; ++i) {
      const int r = (i * kWaves + wave) * RPI + lane / SLOTS;
      const int slot = lane % SLOTS;
      const uint32_t off = (uint32_t)((k0 + r) * D * 2 + 16 * (slot ^ swz<RB>(r)));
      lds_copy(krs, off, 0u, lds_addr_of(sm.k) + (uint32_t)(i * kWaves + wave) * 1024u);
      lds_copy(vrs, off, 0u, lds_addr_of(sm.v) + (uint32_t)(i * kWaves + wave) * 1024u);
    }
  }
  issue_qtile(0, q_first);

  f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk_acc[db][i] = 0.f;
      dv_acc[db][i] = 0.f;
    }

  // operand register sets (see pin()): row operands of S / dP, transposed
  // operands of dV / dK, operands of dQ; P and dS tiles (B operands)
  bf16x8 ar[2][6], at[2][2], aq[2][3], pb[2][2], dsb[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int x = 0; x < 6; ++x) ar[j][x] = bf16x8{};
#pragma unroll
    for (int x = 0; x < 2; ++x) at[j][x] = bf16x8{};
#pragma unroll
    for (int x = 0; x < 3; ++x) aq[j][x] = bf16x8{};
    pb[j][0] = pb[j][1] = dsb[j][0] = dsb[j][1] = bf16x8{};
  }

  // lane parts of the transpose-read offsets (bytes): rows 4g + (sl >> 2)
  // of a 16-row group, columns 16 (grp & 1) + 4 (sl & 3) of a 32-wide block
  const int tr_row = 4 * g + (sl >> 2);     // Q / dO tiles (perm32 row order)
  const int tk_row = 8 * g + (sl >> 2);     // K and dS^T tiles (natural order)
  const int tr_col = 16 * (grp & 1) + 4 * (sl & 3);

  for (int st = 0; st < n_steps; ++st) {
    const int q0 = q_first + st * kBQ;
    const int buf = st & 1;
    wait_loads();
    __syncthreads();  // tile st visible; every wave is done with step st-1
    if (st + 1 < n_steps) issue_qtile(buf ^ 1, q0 + kBQ);
    const char* qt = reinterpret_cast<const char*>(sm.q[buf]);
    const char* gt = reinterpret_cast<const char*>(sm.dout[buf]);
    const char* kt = reinterpret_cast<const char*>(sm.k);
    const char* vt = reinterpret_cast<const char*>(sm.v);

    // S = Q K^T and dP = dO V^T: 64 query rows (2 blocks) x this wave's 32 keys
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8(&a)[6] = ar[kk & 1];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        a[qb] = as_bf16x8(ld16(qt + slot_off<RB>(32 * qb + col, 2 * kk + g)));
        a[2 + qb] = as_bf16x8(ld16(gt + slot_off<RB>(32 * qb + col, 2 * kk + g)));
      }
      a[4] = as_bf16x8(ld16(kt + slot_off<RB>(32 * wave + col, 2 * kk + g)));  // K rows of this wave's keys
      a[5] = as_bf16x8(ld16(vt + slot_off<RB>(32 * wave + col, 2 * kk + g)));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = mfma32(a[qb], a[4], kk == 0 ? f32x16{} : s[qb]);
        dp[qb] = mfma32(a[2 + qb], a[5], kk == 0 ? f32x16{} : dp[qb]);
      }
      group_fence();
#pragma unroll
      for (int x = 0; x < 6; ++x) pin(ar[(kk + 1) & 1][x]);
    }

    // P = exp2(S c - L log2 e) and dS = P (dP - D); masked pairs get 0
    const bool need_mask = (CAUSAL && q0 < k0 + kBKV) || k0 + kBKV > N;
    const float* l2t = sm.l2[buf];
    const float* dvt = sm.dv[buf];
    float guard = 0.f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qr = 32 * qb + 16 * h + 8 * g;  // 8 consecutive local query rows
        const float4 l0 = *reinterpret_cast<const float4*>(&l2t[qr]);
        const float4 l1 = *reinterpret_cast<const float4*>(&l2t[qr + 4]);
        const float4 d0 = *reinterpret_cast<const float4*>(&dvt[qr]);
        const float4 d1 = *reinterpret_cast<const float4*>(&dvt[qr + 4]);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        float p[8], ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float pe = fast_exp2(fmaf(s[qb][8 * h + e], c, -lv[e]));
          if (need_mask) {
            const int q = q0 + qr + e;
            if (my_key >= N || (CAUSAL && my_key > q)) pe = 0.f;
          }
          p[e] = pe;
          ds[e] = pe * (dp[qb][8 * h + e] - dd[e]);
        }
        guard += ds[7];
        pb[qb][h] = pack_bf16x8(p);
        dsb[qb][h] = pack_bf16x8(ds);
        // dS^T row = this lane's key, 8 consecutive query rows
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(sm.dst) +
                                  slot_off<kBQ * 2>(32 * wave + col, qr >> 3)) = __builtin_bit_cast(uint4, dsb[qb][h]);
      }
    // S and dP are consumed: all MFMAs issued so far have run
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int x = 0; x < 6; ++x) pin(ar[j][x], guard);
#pragma unroll
      for (int x = 0; x < 2; ++x) pin(at[j][x], guard);
#pragma unroll
      for (int x = 0; x < 3; ++x) pin(aq[j][x], guard);
    }

    // dV^T += dO^T P and dK^T += Q^T dS, contraction over the 64 query rows;
    // A operands by transpose reads, one (query block, half) group at a time
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int gi = (2 * qb + h) * NDB + db;
          bf16x8(&a)[2] = at[gi & 1];
          const int r0 = 32 * qb + 16 * h + tr_row;  // rows r0, r0 + 8 hold queries 8g + 0..3, 8g + 4..7
          const int cc = 32 * db + tr_col;
          const int o0 = slot_off<RB>(r0, cc >> 3) + 2 * (cc & 7);
          const int o1 = slot_off<RB>(r0 + 8, cc >> 3) + 2 * (cc & 7);
          a[0] = tr_pair(gt, o0, o1);
          a[1] = tr_pair(qt, o0, o1);
          dv_acc[db] = mfma32(a[0], pb[qb][h], dv_acc[db]);
          dk_acc[db] = mfma32(a[1], dsb[qb][h], dk_acc[db]);
          group_fence();
          pin(at[(gi + 1) & 1][0]);
          pin(at[(gi + 1) & 1][1]);
          if (db == 0 && (qb | h)) {  // first group of (qb, h): the previous P / dS pair is released
            const int pg = 2 * qb + h - 1;
            pin(pb[pg >> 1][pg & 1]);
            pin(dsb[pg >> 1][pg & 1]);
          }
        }
    __syncthreads();  // dS^T complete

    // dQ[q][d] += scale sum_key dS[q][key] K[key][d] over the block's keys
    f32x16 dq[NQT];
    const char* dtt = reinterpret_cast<const char*>(sm.dst);
#pragma unroll
    for (int kk = 0; kk < kBKV / 16; ++kk) {
      bf16x8(&a)[3] = aq[kk & 1];
      const int kr0 = 16 * kk + tk_row;  // keys kr0 .. +3 and kr0 + 4 .. +7
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int tt = NQT == 2 ? t : (wave & 1);  // query block of this tile
        const int cq = 32 * tt + tr_col;
        a[t] = tr_pair(dtt, slot_off<kBQ * 2>(kr0, cq >> 3) + 2 * (cq & 7),
                       slot_off<kBQ * 2>(kr0 + 4, cq >> 3) + 2 * (cq & 7));
      }
      const int db = NQT == 2 ? wave : (wave >> 1);
      const int cd = 32 * db + tr_col;
      a[2] = tr_pair(kt, slot_off<RB>(kr0, cd >> 3) + 2 * (cd & 7), slot_off<RB>(kr0 + 4, cd >> 3) + 2 * (cd & 7));
#pragma unroll
      for (int t = 0; t < NQT; ++t) dq[t] = mfma32(a[t], a[2], kk == 0 ? f32x16{} : dq[t]);
      group_fence();
#pragma unroll
      for (int x = 0; x < 3; ++x) pin(aq[(kk + 1) & 1][x]);
    }
    float qsum = 0.f;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int tt = NQT == 2 ? t : (wave & 1);
      const int db = NQT == 2 ? wave : (wave >> 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 32 * tt + acc_row(i, g);
        const float v = scale * dq[t][i];
        qsum += v;
        if (q < N) unsafeAtomicAdd(dQ + head + (size_t)q * D + 32 * db + col, v);
      }
    }
    // dQ consumed: every MFMA of this step has run
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int x = 0; x < 3; ++x) pin(aq[j][x], qsum);
#pragma unroll
      for (int x = 0; x < 2; ++x) pin(at[j][x], qsum);
      pin(pb[j][0], qsum);
      pin(pb[j][1], qsum);
      pin(dsb[j][0], qsum);
      pin(dsb[j][1], qsum);
    }
  }

  if (my_key < N) {
    float* dKrow = dK + head + (size_t)my_key * D;
    float* dVrow = dV + head + (size_t)my_key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * g;
        *reinterpret_cast<float4*>(dKrow + d) =
            make_float4(scale * dk_acc[db][4 * i4], scale * dk_acc[db][4 * i4 + 1], scale * dk_acc[db][4 * i4 + 2],
                        scale * dk_acc[db][4 * i4 + 3]);
        *reinterpret_cast<float4*>(dVrow + d) =
            make_float4(dv_acc[db][4 * i4], dv_acc[db][4 * i4 + 1], dv_acc[db][4 * i4 + 2], dv_acc[db][4 * i4 + 3]);
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                  float* dq, float* dk, float* dv, float* ws, int BH, int N, float scale, hipStream_t stream) {
  const long long rows = (long long)BH * N;
  constexpr int RPB = 256 / (D / 8);
  const long long pre_grid = (rows + RPB - 1) / RPB;
  const int n_kvblk = (N + kBKV - 1) / kBKV;
  const long long total = (long long)BH * n_kvblk;
  if (pre_grid > (1LL << 31) - 1 || total > (1LL << 30)) return hipErrorInvalidConfiguration;
  float* dvec = ws;
  float* l2 = ws + rows;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_grid), dim3(256), 0, stream,
                     static_cast<const bf16_raw*>(dout), o, lse, dvec, l2, dq, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k), static_cast<const bf16_raw*>(v),
                     static_cast<const bf16_raw*>(dout), l2, dvec, dq, dk, dv, N, n_kvblk, (int)total, scale,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* ws, int BH, int N, int d,
                           float scale, int causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, BH, N, scale, stream);
}

}  // namespace fa

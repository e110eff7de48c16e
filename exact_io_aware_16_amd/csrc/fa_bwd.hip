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
//  * bwd_pre_kernel: D_i = dO_i . O_i per query row, and dQ := 0.
//  * bwd_main_kernel: one workgroup per (head, block of 128 keys); each of
//    its 4 waves keeps 32 keys of K and V in registers and accumulates dK^T
//    and dV^T for them in registers, while the workgroup walks the query
//    rows 64 at a time (causal: from the block's diagonal onwards).  Per
//    query tile: S = Q K^T and dP = dO V^T on matrix cores with keys along
//    N (so P and dS come out with one key per lane and 8 consecutive query
//    rows per register octet -- the B-operand layout of dV^T = dO^T P and
//    dK^T = Q^T dS), dS goes through LDS once to be re-read query-major for
//    dQ = dS K, and dQ partial sums are added to global memory with float32
//    atomics.  Q and dO tiles are held in LDS both row-major and transposed.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

// ----------------------------------------------------------------------------------- D and dQ := 0
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16_raw* __restrict__ dO, const float* __restrict__ O,
                                                       float* __restrict__ Dvec, float* __restrict__ dQ,
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
  if (row < rows && part == 0) Dvec[row] = acc;
}

// ----------------------------------------------------------------------------------- main kernel
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBKV = 32 * kWaves;  // keys per workgroup
constexpr int kBQ = 64;            // query rows per step

template <int D>
struct BwdSmem {
  static constexpr int RLD = D + 8;      // row-major Q / dO tile stride
  static constexpr int TLD = kBQ + 8;    // transposed Q^T / dO^T stride
  static constexpr int SLD = kBKV + 8;   // dS [q][key] and K^T [d][key] stride
  bf16_raw q[kBQ * RLD];
  bf16_raw dout[kBQ * RLD];
  bf16_raw qt[D * TLD];
  bf16_raw dot[D * TLD];
  bf16_raw ds[kBQ * SLD];
  bf16_raw kt[D * SLD];
  float lse2[kBQ];
  float dvec[kBQ];
};

template <int D>
struct QTileRegs {
  static constexpr int RPT = kBQ * D / 8 / kThreads;  // rows per thread block (4 for d=128, 2 for d=64)
  uint4 q[RPT];
  uint4 g[RPT];
  float lse2, dv;
};

template <int D>
__device__ __forceinline__ void load_qtile(QTileRegs<D>& r, const bf16_raw* __restrict__ Qh,
                                           const bf16_raw* __restrict__ dOh, const float* __restrict__ Lh,
                                           const float* __restrict__ Dh, int q0, int N, int tid) {
  constexpr int RPT = QTileRegs<D>::RPT;
  const int rb = tid % (kBQ / RPT), d8 = tid / (kBQ / RPT);
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int q = q0 + RPT * rb + j;
    const bool ok = q < N;
    r.q[j] = ok ? ld16(Qh + (size_t)q * D + 8 * d8) : make_uint4(0, 0, 0, 0);
    r.g[j] = ok ? ld16(dOh + (size_t)q * D + 8 * d8) : make_uint4(0, 0, 0, 0);
  }
  if (tid < kBQ) {
    const int q = q0 + tid;
    r.lse2 = q < N ? Lh[q] * kLog2e : INFINITY;  // rows past the end get P = 0
    r.dv = q < N ? Dh[q] : 0.f;
  }
}

// Writes the RPT x 8 block in both layouts: row-major (rows in perm32 order
// within each 32-row group) and transposed (natural row order).
template <int D>
__device__ __forceinline__ void store_block_both(const uint4* v, bf16_raw* rowmajor, bf16_raw* trans, int rb, int d8) {
  constexpr int RPT = QTileRegs<D>::RPT;
  constexpr int RLD = BwdSmem<D>::RLD, TLD = BwdSmem<D>::TLD;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = RPT * rb + j;
    const int lrow = (row & ~31) | perm32(row & 31);
    st16(&rowmajor[lrow * RLD + 8 * d8], v[j]);
  }
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if constexpr (RPT == 4) {
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
      uint2 lo, hi;
      lo.x = (w0[w] & 0xffffu) | (w1[w] << 16);
      lo.y = (w2[w] & 0xffffu) | (w3[w] << 16);
      hi.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
      hi.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
      *reinterpret_cast<uint2*>(&trans[(8 * d8 + 2 * w) * TLD + 4 * rb]) = lo;
      *reinterpret_cast<uint2*>(&trans[(8 * d8 + 2 * w + 1) * TLD + 4 * rb]) = hi;
    } else {
      const uint32_t lo = (w0[w] & 0xffffu) | (w1[w] << 16);
      const uint32_t hi = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&trans[(8 * d8 + 2 * w) * TLD + 2 * rb]) = lo;
      *reinterpret_cast<uint32_t*>(&trans[(8 * d8 + 2 * w + 1) * TLD + 2 * rb]) = hi;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_qtile(const QTileRegs<D>& r, BwdSmem<D>& sm, int tid) {
  constexpr int RPT = QTileRegs<D>::RPT;
  const int rb = tid % (kBQ / RPT), d8 = tid / (kBQ / RPT);
  store_block_both<D>(r.q, sm.q, sm.qt, rb, d8);
  store_block_both<D>(r.g, sm.dout, sm.dot, rb, d8);
  if (tid < kBQ) {
    sm.lse2[tid] = r.lse2;
    sm.dvec[tid] = r.dv;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    const float* __restrict__ LSE, const bf16_raw* __restrict__ dO, const float* __restrict__ Dvec,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int N, int n_kvblk, int total,
    float scale, float c) {
  constexpr int NKK = D / 16;  // 16-wide head-dim slices (contraction of S and dP)
  constexpr int NDB = D / 32;  // 32-row blocks of dK^T / dV^T
  constexpr int RLD = BwdSmem<D>::RLD, TLD = BwdSmem<D>::TLD, SLD = BwdSmem<D>::SLD;
  constexpr int NQT = 2 * NDB / kWaves;  // dQ 32x32 tiles per wave
  __shared__ __attribute__((aligned(16))) BwdSmem<D> sm;

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int bh = blk / n_kvblk;
  const int kvb = blk - bh * n_kvblk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const bf16_raw* Qh = Q + head;
  const bf16_raw* Kh = K + head;
  const bf16_raw* Vh = V + head;
  const bf16_raw* dOh = dO + head;
  const float* Lh = LSE + (size_t)bh * N;
  const float* Dh = Dvec + (size_t)bh * N;

  const int k0 = kvb * kBKV;
  const int my_key = k0 + 32 * wave + col;

  // this wave's 32 keys of K and V, as B operands along the head dimension
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const bool ok = my_key < N;
    kf[kk] = as_bf16x8(ok ? ld16(Kh + (size_t)my_key * D + 16 * kk + 8 * g) : make_uint4(0, 0, 0, 0));
    vf[kk] = as_bf16x8(ok ? ld16(Vh + (size_t)my_key * D + 16 * kk + 8 * g) : make_uint4(0, 0, 0, 0));
  }
  // the workgroup's K block transposed into LDS (B operand of dQ = dS K)
  {
    constexpr int BLKS = (kBKV / 4) * (D / 8);
#pragma unroll
    for (int b = tid; b < BLKS; b += kThreads) {
      const int kb4 = b % (kBKV / 4), d8 = b / (kBKV / 4);
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * kb4 + j;
        v[j] = key < N ? ld16(Kh + (size_t)key * D + 8 * d8) : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&v[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&v[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&v[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&v[3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint2 lo, hi;
        lo.x = (w0[w] & 0xffffu) | (w1[w] << 16);
        lo.y = (w2[w] & 0xffffu) | (w3[w] << 16);
        hi.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
        hi.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
        *reinterpret_cast<uint2*>(&sm.kt[(8 * d8 + 2 * w) * SLD + 4 * kb4]) = lo;
        *reinterpret_cast<uint2*>(&sm.kt[(8 * d8 + 2 * w + 1) * SLD + 4 * kb4]) = hi;
      }
    }
  }

  f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk_acc[db][i] = 0.f;
      dv_acc[db][i] = 0.f;
    }

  const int q_first = CAUSAL ? k0 : 0;  // k0 is a multiple of kBQ
  const int n_steps = (N - q_first + kBQ - 1) / kBQ;

  QTileRegs<D> tr;
  load_qtile<D>(tr, Qh, dOh, Lh, Dh, q_first, N, tid);
  store_qtile<D>(tr, sm, tid);
  __syncthreads();

  for (int st = 0; st < n_steps; ++st) {
    const int q0 = q_first + st * kBQ;
    const bool has_next = st + 1 < n_steps;
    if (has_next) load_qtile<D>(tr, Qh, dOh, Lh, Dh, q0 + kBQ, N, tid);

    // S = Q K^T and dP = dO V^T for 64 query rows x this wave's 32 keys
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[qb][i] = 0.f;
        dp[qb][i] = 0.f;
      }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bf16x8 aq = as_bf16x8(ld16(&sm.q[(32 * qb + col) * RLD + 16 * kk + 8 * g]));
        s[qb] = mfma32(aq, kf[kk], s[qb]);
        const bf16x8 ag = as_bf16x8(ld16(&sm.dout[(32 * qb + col) * RLD + 16 * kk + 8 * g]));
        dp[qb] = mfma32(ag, vf[kk], dp[qb]);
      }

    const bool need_mask = (CAUSAL && q0 < k0 + kBKV) || k0 + kBKV > N;
    bf16x8 pb[2][2], dsb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qr = 32 * qb + 16 * h + 8 * g;  // first of 8 consecutive local query rows
        const float4 l0 = *reinterpret_cast<const float4*>(&sm.lse2[qr]);
        const float4 l1 = *reinterpret_cast<const float4*>(&sm.lse2[qr + 4]);
        const float4 d0 = *reinterpret_cast<const float4*>(&sm.dvec[qr]);
        const float4 d1 = *reinterpret_cast<const float4*>(&sm.dvec[qr + 4]);
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
        pb[qb][h] = pack_bf16x8(p);
        dsb[qb][h] = pack_bf16x8(ds);
        // dS into LDS, query-major, for dQ = dS K (elements taken from the
        // packed words: per-element access of a bf16 vector is avoided)
        const uint4 packed = __builtin_bit_cast(uint4, dsb[qb][h]);
        const uint32_t pw[4] = {packed.x, packed.y, packed.z, packed.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sm.ds[(qr + e) * SLD + 32 * wave + col] = (bf16_raw)(e & 1 ? pw[e >> 1] >> 16 : pw[e >> 1] & 0xffffu);
      }

    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 64 query rows)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int qc = 32 * qb + 16 * h + 8 * g;
          const bf16x8 ag = as_bf16x8(ld16(&sm.dot[(32 * db + col) * TLD + qc]));
          dv_acc[db] = mfma32(ag, pb[qb][h], dv_acc[db]);
          const bf16x8 aq = as_bf16x8(ld16(&sm.qt[(32 * db + col) * TLD + qc]));
          dk_acc[db] = mfma32(aq, dsb[qb][h], dk_acc[db]);
        }
    __syncthreads();  // dS complete; Q/dO tiles no longer read

    if (has_next) store_qtile<D>(tr, sm, tid);

    // dQ[q][d] += scale * sum_key dS[q][key] K[key][d] over the block's 128 keys
    f32x16 dq[NQT];
#pragma unroll
    for (int t = 0; t < NQT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) dq[t][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < kBKV / 16; ++kk)
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int tt = wave + kWaves * t, qb = tt & 1, db = tt >> 1;
        const bf16x8 a = as_bf16x8(ld16(&sm.ds[(32 * qb + col) * SLD + 16 * kk + 8 * g]));
        const bf16x8 b = as_bf16x8(ld16(&sm.kt[(32 * db + col) * SLD + 16 * kk + 8 * g]));
        dq[t] = mfma32(a, b, dq[t]);
      }
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int tt = wave + kWaves * t, qb = tt & 1, db = tt >> 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + 32 * qb + acc_row(i, g);
        if (q < N) unsafeAtomicAdd(dQ + head + (size_t)q * D + 32 * db + col, scale * dq[t][i]);
      }
    }
    __syncthreads();  // next tile visible; dS reads done before it is rewritten
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
                  float* dq, float* dk, float* dv, float* dvec, int BH, int N, float scale, hipStream_t stream) {
  const long long rows = (long long)BH * N;
  constexpr int RPB = 256 / (D / 8);
  const long long pre_grid = (rows + RPB - 1) / RPB;
  const int n_kvblk = (N + kBKV - 1) / kBKV;
  const long long total = (long long)BH * n_kvblk;
  if (pre_grid > (1LL << 31) - 1 || total > (1LL << 30)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)pre_grid), dim3(256), 0, stream,
                     static_cast<const bf16_raw*>(dout), o, dvec, dq, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k), static_cast<const bf16_raw*>(v),
                     lse, static_cast<const bf16_raw*>(dout), dvec, dq, dk, dv, N, n_kvblk, (int)total, scale,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* dvec, int BH, int N, int d,
                           float scale, int causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, dout, dq, dk, dv, dvec, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, dout, dq, dk, dv, dvec, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, dout, dq, dk, dv, dvec, BH, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, dout, dq, dk, dv, dvec, BH, N, scale, stream);
}

}  // namespace fa

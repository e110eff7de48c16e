// Exact attention forward, bf16 inputs, float32 outputs, gfx950 matrix cores.
//
// Follows the blocked recurrence of "From softmax to attention: rescale the
// output too" (FlashAttention: The Matrix You Never Have to Write Down):
// per query row a running max m, running sum l and unnormalised output O;
// each key tile raises m to m_new, scales l and O by e^(m - m_new), adds the
// tile's terms, and O is divided by l once after the last tile.  The scores
// never leave the chip.
//
// Work split (one workgroup = 4 waves = 128 query rows of one head):
//  * each wave owns 32 query rows; its Q block stays in registers for the
//    whole kernel as the B operand of S^T = K Q^T (keys along M, queries
//    along N), so a query's scores sit in one lane pair (lanes c, c+32) and
//    the row max needs a single cross-half exchange;
//  * key/value tiles of BC rows are staged through LDS, double buffered:
//    K row-major (rows loaded in perm32 order, see fa_common.h), V
//    transposed (V^T[d][key]) so both products read 16-byte operand runs;
//  * P is rounded to bf16 in registers and used directly as the B operand of
//    O^T += V^T P^T -- the perm32 key order makes the S result layout equal
//    to the operand layout, so P never touches LDS;
//  * scores are scaled by scale*log2(e) and exponentiated with v_exp_f32
//    (base 2); L is converted back to natural log in the epilogue.
//  * causal: query block qb visits key tiles up to its diagonal only; waves
//    whose rows all precede a tile skip its arithmetic; element masks are
//    applied only on tiles that straddle the diagonal or the ragged end.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup

template <int D> struct FwdTile;
template <> struct FwdTile<128> { static constexpr int BC = 64; };
template <> struct FwdTile<64> { static constexpr int BC = 128; };

template <int D>
struct FwdSmem {
  static constexpr int BC = FwdTile<D>::BC;
  static constexpr int KLD = D + 8;   // K row stride (elements); 16-byte pad
  static constexpr int VLD = BC + 8;  // V^T row stride (elements)
  bf16_raw k[2][BC * KLD];
  bf16_raw vt[2][D * VLD];
};

// Per-thread staging of one K/V tile between the global load and the LDS store.
template <int D>
struct TileRegs {
  static constexpr int BC = FwdTile<D>::BC;
  static constexpr int KCH = BC * D / 8 / kThreads;  // 16-byte K chunks per thread (4)
  uint4 k[KCH];
  uint4 v[4];  // 4 consecutive key rows x 8 d of V
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const bf16_raw* __restrict__ Kh,
                                          const bf16_raw* __restrict__ Vh, int key0, int N, int tid) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int j = 0; j < TileRegs<D>::KCH; ++j) {
    const int ch = j * kThreads + tid;
    const int row = ch / CPR, col = (ch % CPR) * 8;
    const int key = key0 + row;
    r.k[j] = key < N ? ld16(Kh + (size_t)key * D + col) : make_uint4(0, 0, 0, 0);
  }
  const int kb4 = tid % (BC / 4), d8 = tid / (BC / 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int key = key0 + 4 * kb4 + j;
    r.v[j] = key < N ? ld16(Vh + (size_t)key * D + 8 * d8) : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, FwdSmem<D>& sm, int buf, int tid) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int CPR = D / 8;
  constexpr int KLD = FwdSmem<D>::KLD, VLD = FwdSmem<D>::VLD;
#pragma unroll
  for (int j = 0; j < TileRegs<D>::KCH; ++j) {
    const int ch = j * kThreads + tid;
    const int row = ch / CPR, col = (ch % CPR) * 8;
    const int lrow = (row & ~31) | perm32(row & 31);
    st16(&sm.k[buf][lrow * KLD + col], r.k[j]);
  }
  // transpose 4 keys x 8 d into 8 rows of V^T, 4 keys (8 bytes) each
  const int kb4 = tid % (BC / 4), d8 = tid / (BC / 4);
  const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&r.v[0]);
  const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&r.v[1]);
  const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&r.v[2]);
  const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&r.v[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint2 lo, hi;  // d = 8*d8 + 2w (low halves) and 2w+1 (high halves)
    lo.x = (v0[w] & 0xffffu) | (v1[w] << 16);
    lo.y = (v2[w] & 0xffffu) | (v3[w] << 16);
    hi.x = (v0[w] >> 16) | (v1[w] & 0xffff0000u);
    hi.y = (v2[w] >> 16) | (v3[w] & 0xffff0000u);
    *reinterpret_cast<uint2*>(&sm.vt[buf][(8 * d8 + 2 * w) * VLD + 4 * kb4]) = lo;
    *reinterpret_cast<uint2*>(&sm.vt[buf][(8 * d8 + 2 * w + 1) * VLD + 4 * kb4]) = hi;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16_raw* __restrict__ Q, const bf16_raw* __restrict__ K, const bf16_raw* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qblk, int total, float c) {
  constexpr int BC = FwdTile<D>::BC;
  constexpr int NKB = BC / 32;   // 32-key blocks per tile
  constexpr int NKK = D / 16;    // 16-wide slices of the head dimension
  constexpr int NDB = D / 32;    // 32-row blocks of O^T
  constexpr int KLD = FwdSmem<D>::KLD, VLD = FwdSmem<D>::VLD;
  __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;

  const int blk = xcd_logical_block(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int bh = blk / n_qblk;
  int qb = blk - bh * n_qblk;
  if (CAUSAL) qb = n_qblk - 1 - qb;  // longest rows first

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, col = lane & 31;
  const size_t head = (size_t)bh * N * D;
  const bf16_raw* Qh = Q + head;
  const bf16_raw* Kh = K + head;
  const bf16_raw* Vh = V + head;

  const int q_start = qb * kBR;
  const int q0w = q_start + 32 * wave;
  const int my_q = q0w + col;
  const bool wave_live = q0w < N;

  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    qf[kk] = as_bf16x8(my_q < N ? ld16(Qh + (size_t)my_q * D + 16 * kk + 8 * g) : make_uint4(0, 0, 0, 0));

  const int kv_end = CAUSAL ? min(N, q_start + kBR) : N;
  const int n_tiles = (kv_end + BC - 1) / BC;

  TileRegs<D> tr;
  load_tile<D>(tr, Kh, Vh, 0, N, tid);
  store_tile<D>(tr, sm, 0, tid);
  __syncthreads();

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int key0 = t * BC;
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile<D>(tr, Kh, Vh, key0 + BC, N, tid);

    const bool active = wave_live && (!CAUSAL || key0 <= q0w + 31);
    if (active) {
      // S^T = K Q^T for this tile: NKB blocks of 32 keys x 32 queries
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 a = as_bf16x8(ld16(&sm.k[buf][(32 * kb + col) * KLD + 16 * kk + 8 * g]));
          s[kb] = mfma32(a, qf[kk], s[kb]);
        }
      }
      const bool need_mask = (CAUSAL && key0 + BC - 1 > q0w) || key0 + BC > N;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb + perm_row(i, g);
            if (key >= N || (CAUSAL && key > my_q)) s[kb][i] = -INFINITY;
          }
      }
      // online softmax: running max over this tile (both lane halves)
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row with nothing visible yet
      const float alpha = fast_exp2(m_run - m_use);           // 0 on the first visible tile
      m_run = m_new;

      bf16x8 pb[NKB][2];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(s[kb][8 * h + e], c, -m_use));
            rs += p[e];
          }
          pb[kb][h] = pack_bf16x8(p);
        }
      l_run = l_run * alpha + rs;  // this lane's half of the row sum

      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 a = as_bf16x8(ld16(&sm.vt[buf][(32 * db + col) * VLD + 32 * kb + 16 * h + 8 * g]));
            oacc[db] = mfma32(a, pb[kb][h], oacc[db]);
          }
    }
    if (t + 1 < n_tiles) store_tile<D>(tr, sm, buf ^ 1, tid);
    __syncthreads();
  }

  // epilogue: combine the two half-row sums, normalise once, write O and L
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* Orow = O + head + (size_t)my_q * D;
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
    if (g == 0) LSE[(size_t)bh * N + my_q] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int N,
                  float scale, hipStream_t stream) {
  const int n_qblk = (N + kBR - 1) / kBR;
  const long long total = (long long)BH * n_qblk;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 7) / 8 * 8);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const bf16_raw*>(q), static_cast<const bf16_raw*>(k),
                     static_cast<const bf16_raw*>(v), o, lse, N, n_qblk, (int)total, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int N,
                           int d, float scale, int causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa

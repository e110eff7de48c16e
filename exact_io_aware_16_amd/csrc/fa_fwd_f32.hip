// Exact attention forward with float32 inputs, computed in float32 on the
// vector ALUs (no matrix cores).  For small exact checks, where the answer
// must stay within float32 rounding of the definition; not a throughput path.
//
// Same recurrence as the bf16 kernel ("From softmax to attention: rescale the
// output too", FlashAttention: The Matrix You Never Have to Write Down): per
// query row a running max, running sum and unnormalised output, rescaled by
// e^(m - m_new) when a key tile raises the max, divided by the sum once.
//
// One workgroup = 256 threads = 64 query rows x 4 threads per row; key tiles
// of 64 rows go through LDS.  Thread (row r, part p) scores keys p, p+4, ...
// of the tile, the four parts of a row combine max/sum with lane shuffles,
// and the thread accumulates output columns p, p+4, ... of its row.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = 64, kKeys = 64, kThreads = 256;

template <int D>
struct F32Smem {
  float q[kRows][D + 1];
  float k[kKeys][D + 1];
  float v[kKeys][D];
  float p[kRows][kKeys + 1];
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, float* __restrict__ O,
                                                          float* __restrict__ LSE, int N, int n_qblk, float c) {
  __shared__ F32Smem<D> sm;
  const int bh = blockIdx.x / n_qblk;
  const int q_start = (blockIdx.x - bh * n_qblk) * kRows;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const size_t head = (size_t)bh * N * D;
  const int my_q = q_start + r;

  for (int e = tid; e < kRows * D; e += kThreads) {
    const int row = e / D, cc = e % D;
    sm.q[row][cc] = q_start + row < N ? Q[head + (size_t)(q_start + row) * D + cc] : 0.f;
  }

  constexpr int NK = kKeys / 4, NC = D / 4;
  float o[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) o[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, q_start + kRows) : N;
  for (int key0 = 0; key0 < kv_end; key0 += kKeys) {
    __syncthreads();  // previous tile fully consumed (and Q stored, first time)
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int row = e / D, cc = e % D;
      const bool ok = key0 + row < N;
      sm.k[row][cc] = ok ? K[head + (size_t)(key0 + row) * D + cc] : 0.f;
      sm.v[row][cc] = ok ? V[head + (size_t)(key0 + row) * D + cc] : 0.f;
    }
    __syncthreads();

    float s[NK];
#pragma unroll
    for (int j = 0; j < NK; ++j) s[j] = 0.f;
    for (int cc = 0; cc < D; ++cc) {
      const float qv = sm.q[r][cc];
#pragma unroll
      for (int j = 0; j < NK; ++j) s[j] = fmaf(qv, sm.k[4 * j + p][cc], s[j]);
    }
    // scores in log2 units (scaled before the max, so any sign of the scale
    // works), masked ones -inf
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int key = key0 + 4 * j + p;
      s[j] = (key >= N || (CAUSAL && key > my_q)) ? -INFINITY : s[j] * c;
      mx = fmaxf(mx, s[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const float pv = exp2f(s[j] - m_use);
      rs += pv;
      sm.p[r][4 * j + p] = pv;
    }
    l_run = l_run * alpha + rs;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NC; ++j) o[j] *= alpha;
    for (int key = 0; key < kKeys; ++key) {
      const float pv = sm.p[r][key];
#pragma unroll
      for (int j = 0; j < NC; ++j) o[j] = fmaf(pv, sm.v[key][4 * j + p], o[j]);
    }
  }
  l_run += __shfl_xor(l_run, 1);
  l_run += __shfl_xor(l_run, 2);
  if (my_q < N) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) O[head + (size_t)my_q * D + 4 * j + p] = o[j] * inv;
    if (p == 0) LSE[(size_t)bh * N + my_q] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, float scale,
                  hipStream_t stream) {
  const int n_qblk = (N + kRows - 1) / kRows;
  const long long total = (long long)BH * n_qblk;
  if (total > (1LL << 30)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(kThreads), 0, stream, q, k, v, o, lse,
                     N, n_qblk, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N, int d,
                          float scale, int causal, hipStream_t stream) {
  if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                              : launch<128, false>(q, k, v, o, lse, BH, N, scale, stream);
  return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                : launch<64, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa

// Split-KV forward for few query rows (decoding), bf16 inputs, float32 partials.
//
// The key range of one head is cut into contiguous ranges, one workgroup
// each, as in Flash-Decoding ("What it doesn't solve", FlashAttention: The
// Matrix You Never Have to Write Down).  Every range produces the exact
// softmax of its own keys, normalised within the range, and its logsumexp;
// splitkv_merge_kernel then combines the ranges with the logsumexp identity
// ("The identity" on the same page).
//
// With one to four query rows there is no dense contraction to give the
// matrix cores: a key costs one dot product and one scaled row of V per
// query, and the launch is bound by reading K and V from HBM once.  So this
// kernel streams K and V rows straight into registers and does the
// arithmetic on the vector ALUs:
//  * a key row of D bf16 is D / 8 lanes x 16 bytes; a wave covers 64 / (D / 8)
//    keys per load, and each lane keeps CH keys of K and V in flight;
//  * a lane group (the D / 8 lanes of one key) forms its slices of the dot
//    products of CH keys and sums them across the group by a reduce-scatter,
//    so that each lane ends with one key's score; one exponential per lane,
//    and the weights go back to every lane of the group for the V update;
//  * each lane group keeps its own running max m, sum l and output slice O
//    over the keys it sees (the blocked recurrence of "From softmax to
//    attention: rescale the output too"), rescaling once per chunk of CH keys;
//  * the groups of a wave, then the waves, are merged with the same
//    identity, and the range's O / l and L = m + ln l are written once.
// Causal masking is upper-left (query i sees keys 0 .. i), so with at most
// four query rows only the first keys are ever visible; ranges past them
// report an empty range (O = 0, L = -inf).
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecCh = 8;   // keys per lane group in flight

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16 bytes that are read once: a nontemporal load
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ void unpack8(uint4 r, float (&f)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = bf16_lo(w[e]);
    f[2 * e + 1] = bf16_hi(w[e]);
  }
}

// Reduce-scatter of H values over the lane bits M, M / 2, ... (log2 H steps):
// at each step the lane keeps the upper half of its values if its bit M is
// set, else the lower half, and adds the partner's copy of the kept half.
// Afterwards v[0] holds value sum over the exchanged lanes of the index
// formed by the lane's bits M, M / 2, ... (most significant first).
template <int M, int H>
__device__ __forceinline__ void reduce_scatter(float (&v)[kDecCh], int sl) {
  if constexpr (H > 1) {
    const bool up = (sl & M) != 0;
#pragma unroll
    for (int t = 0; t < H / 2; ++t) {
      const float send = up ? v[t] : v[t + H / 2];
      const float keep = up ? v[t + H / 2] : v[t];
      v[t] = keep + __shfl_xor(send, M);
    }
    reduce_scatter<M / 2, H / 2>(v, sl);
  }
}

// (m, l, o) <- merge of two partial softmax states over disjoint key sets,
// each with sums taken against its own reference max; m = -inf marks a state
// that has seen no visible key (then l = 0, o = 0).
__device__ __forceinline__ void merge_state(float& m, float& l, float (&o)[8], float m2, float l2, const float (&o2)[8]) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a = fast_exp2(m - mm), b = fast_exp2(m2 - mm);
  l = a * l + b * l2;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = a * o[e] + b * o2[e];
  m = mm;
}

// Grid: one workgroup per (head bh, key range ks), blockIdx = bh * n_split + ks.
// Range ks covers keys [ks * keys_per_split, min(Nk, (ks + 1) * keys_per_split)).
// Opart / Lpart: [n_split][BH * Nq] rows of D floats / one float (natural log).
template <int D, int NQ, bool CAUSAL>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const bf16_raw* __restrict__ Q,
                                                            const bf16_raw* __restrict__ K,
                                                            const bf16_raw* __restrict__ V, float* __restrict__ Opart,
                                                            float* __restrict__ Lpart, int BH, int Nq, int Nk,
                                                            int n_split, int keys_per_split, float c) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPW = 64 / LPK;  // keys per wave and load
  constexpr int DUP = LPK / kDecCh;  // lanes holding each key after the reduce-scatter
  static_assert(DUP >= 1, "a lane group must hold at least as many lanes as keys in flight");
  __shared__ float red_m[kDecWaves][NQ], red_l[kDecWaves][NQ];
  __shared__ float red_o[kDecWaves][NQ][D];

  const int blk = blockIdx.x;
  const int bh = blk / n_split, ks = blk - bh * n_split;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPK, sl = lane % LPK;
  const int k_begin = ks * keys_per_split;
  int k_end = min(Nk, k_begin + keys_per_split);
  if (CAUSAL) k_end = min(k_end, Nq);  // no row of this launch sees key Nq or later

  const bf16_raw* Kh = K + (size_t)bh * Nk * D;
  const bf16_raw* Vh = V + (size_t)bh * Nk * D;
  const bf16_raw* Qh = Q + (size_t)bh * Nq * D;

  float qv[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i < Nq)
      unpack8(ld16(Qh + (size_t)i * D + 8 * sl), qv[i]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[i][e] = 0.f;
  }
  float m[NQ], l[NQ], o[NQ][8];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  // wave w takes chunks of KPW * kDecCh keys, every kDecWaves-th chunk;
  // key j of a chunk for this lane group is base + j * KPW + grp
  constexpr int kChunk = KPW * kDecCh;
  for (int base = k_begin + wave * kChunk; base < k_end; base += kDecWaves * kChunk) {
    uint4 kr[kDecCh], vr[kDecCh];
#pragma unroll
    for (int j = 0; j < kDecCh; ++j) {
      const int key = base + j * KPW + grp;
      if (key < k_end) {  // read once: streaming loads
        kr[j] = ld16_stream(Kh + (size_t)key * D + 8 * sl);
        vr[j] = ld16_stream(Vh + (size_t)key * D + 8 * sl);
      } else {
        kr[j] = vr[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i >= Nq) break;
      // this lane's slice of the dot products of the chunk's keys
      float v[kDecCh];
#pragma unroll
      for (int j = 0; j < kDecCh; ++j) {
        float kf[8];
        unpack8(kr[j], kf);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot = fmaf(qv[i][e], kf[e], dot);
        v[j] = dot;
      }
      // reduce-scatter across the group: at the exchange over lane bit M the
      // lane keeps the half of its keys selected by that bit and adds the
      // partner's slices of them; after log2(CH) exchanges lane sl holds key
      // sl / DUP summed over the lanes that differ in the bits exchanged, and
      // the remaining low bits are summed in full
      reduce_scatter<LPK / 2, kDecCh>(v, sl);
#pragma unroll
      for (int x = DUP / 2; x > 0; x >>= 1) v[0] += __shfl_xor(v[0], x);
      const int my_key = base + (sl / DUP) * KPW + grp;
      const bool vis = my_key < k_end && (!CAUSAL || my_key <= i);
      const float s_own = vis ? v[0] * c : -INFINITY;  // log2 units
      float mx = s_own;
#pragma unroll
      for (int x = LPK / 2; x > 0; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
      const float m_new = fmaxf(m[i], mx);
      if (m_new == -INFINITY) continue;  // nothing visible to this group yet
      const float alpha = fast_exp2(m[i] - m_new);  // 0 while nothing was accumulated
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
      const float p_own = fast_exp2(s_own - m_new);
      if (sl % DUP == 0) l[i] += p_own;  // one lane per key adds its weight
#pragma unroll
      for (int j = 0; j < kDecCh; ++j) {
        const float p = __shfl(p_own, grp * LPK + j * DUP);
        float vf[8];
        unpack8(vr[j], vf);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, vf[e], o[i][e]);
      }
      m[i] = m_new;
    }
  }

  // each lane's l covers its own keys: sum over the group
#pragma unroll
  for (int i = 0; i < NQ; ++i)
#pragma unroll
    for (int x = LPK / 2; x > 0; x >>= 1) l[i] += __shfl_xor(l[i], x);

  // merge the KPW lane groups of the wave (lane bits above the slice index)
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
      float o2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[i][e], x);
      const float m2 = __shfl_xor(m[i], x), l2 = __shfl_xor(l[i], x);
      merge_state(m[i], l[i], o[i], m2, l2, o2);
    }
    if (lane < LPK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][i][8 * sl + e] = o[i][e];
      if (lane == 0) {
        red_m[wave][i] = m[i];
        red_l[wave][i] = l[i];
      }
    }
  }
  __syncthreads();
  // then the waves, and write this range's partial result
  if (wave == 0 && lane < LPK) {
    const long long rows = (long long)BH * Nq;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i >= Nq) break;
      float mm = red_m[0][i], ll = red_l[0][i], oo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) oo[e] = red_o[0][i][8 * sl + e];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) {
        float o2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o2[e] = red_o[w][i][8 * sl + e];
        merge_state(mm, ll, oo, red_m[w][i], red_l[w][i], o2);
      }
      const size_t row = (size_t)ks * rows + (size_t)bh * Nq + i;
      const float inv = ll > 0.f ? 1.f / ll : 0.f;
      float* dst = Opart + row * D + 8 * sl;
      *reinterpret_cast<float4*>(dst) = make_float4(oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(oo[4] * inv, oo[5] * inv, oo[6] * inv, oo[7] * inv);
      if (lane == 0) Lpart[row] = ll > 0.f ? (mm + __log2f(ll)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, int NQ>
hipError_t launch_nq(const void* q, const void* k, const void* v, float* opart, float* lpart, int BH, int Nq, int Nk,
                     int n_split, int keys_per_split, float c, int causal, hipStream_t stream) {
  const long long total = (long long)BH * n_split;
  if (total > (1LL << 31) - 1) return hipErrorInvalidConfiguration;
  auto kq = static_cast<const bf16_raw*>(q);
  auto kk = static_cast<const bf16_raw*>(k);
  auto kv = static_cast<const bf16_raw*>(v);
  if (causal)
    hipLaunchKernelGGL((decode_kernel<D, NQ, true>), dim3((unsigned)total), dim3(kDecThreads), 0, stream, kq, kk, kv,
                       opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c);
  else
    hipLaunchKernelGGL((decode_kernel<D, NQ, false>), dim3((unsigned)total), dim3(kDecThreads), 0, stream, kq, kk, kv,
                       opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c);
  return hipGetLastError();
}

}  // namespace

bool decode_applies(int Nq, int d, int dv) { return Nq >= 1 && Nq <= kDecodeMaxRows && d == dv && (d == 64 || d == 128); }

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, float* opart, float* lpart, int BH, int Nq,
                              int Nk, int d, int n_split, int keys_per_split, float c, int causal,
                              hipStream_t stream) {
  if (n_split < 1 || keys_per_split < 1 || !decode_applies(Nq, d, d)) return hipErrorInvalidValue;
  if (d == 128)
    return Nq == 1 ? launch_nq<128, 1>(q, k, v, opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c, causal, stream)
                   : launch_nq<128, kDecodeMaxRows>(q, k, v, opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c,
                                                    causal, stream);
  return Nq == 1 ? launch_nq<64, 1>(q, k, v, opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c, causal, stream)
                 : launch_nq<64, kDecodeMaxRows>(q, k, v, opart, lpart, BH, Nq, Nk, n_split, keys_per_split, c, causal,
                                                 stream);
}

}  // namespace fa

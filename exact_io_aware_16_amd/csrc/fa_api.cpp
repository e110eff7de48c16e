// C ABI of libfa.so: host-side argument checks, then the kernel launches.
// Every check runs before anything touches the HIP runtime, so invalid
// arguments return an fa_status code without a device present.
#include "../../include/fa.h"

#include <cmath>
#include <cstdint>

#include "fa_dropout.h"
#include "fa_launch.h"

namespace {

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Validates shape arguments; sets *empty when there is nothing to compute.
int check_shape(int B, int H, int N, int d, int causal, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  *empty = (B == 0 || H == 0 || N == 0);
  // element offsets are computed in 64 bits; B*H must fit an int and the
  // total element count must stay well inside 2^62
  const long long bh = (long long)B * H;
  if (bh > INT32_MAX) return FA_ERR_SHAPE;
  if ((double)bh * N * d > 4.0e18) return FA_ERR_SHAPE;
  // one head of a float32 [N,d] tensor is addressed through a buffer
  // descriptor with 32-bit byte offsets
  if ((long long)N * d * 4 > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

// Shapes of the general forward: Q [B,H,Nq,d], K [B,H,Nk,d], V [B,H,Nk,dv].
int check_shape_ex(int B, int H, int Nq, int Nk, int d, int dv, int causal, bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d) || !head_dim_ok(dv)) return FA_ERR_HEADDIM;
  *empty = (B == 0 || H == 0 || Nq == 0);
  const long long bh = (long long)B * H;
  if (bh > INT32_MAX) return FA_ERR_SHAPE;
  if ((double)bh * Nq * dv > 4.0e18 || (double)bh * Nk * (d + dv) > 4.0e18) return FA_ERR_SHAPE;
  // per-head byte ranges of the buffer descriptors stay below 2^31
  if ((long long)Nq * dv * 4 > INT32_MAX || (long long)Nk * d * 2 > INT32_MAX ||
      (long long)Nk * dv * 2 > INT32_MAX)
    return FA_ERR_SHAPE;
  return FA_OK;
}

// Packed sequences: Q, K, V [H, total, d]; cu_seqlens has B + 1 entries.
int check_varlen(int B, int H, int total, int max_seqlen, int d, int causal, bool* empty) {
  if (B < 0 || H < 0 || total < 0 || max_seqlen < 0) return FA_ERR_SHAPE;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!head_dim_ok(d)) return FA_ERR_HEADDIM;
  *empty = (B == 0 || H == 0 || total == 0 || max_seqlen == 0);
  if ((long long)B * H > INT32_MAX) return FA_ERR_SHAPE;
  if ((double)H * total * d > 4.0e18) return FA_ERR_SHAPE;
  // a sequence is addressed through buffer descriptors with 32-bit byte
  // offsets, and none is longer than the packed axis
  if ((long long)total * d * 4 > INT32_MAX || max_seqlen > total) return FA_ERR_SHAPE;
  return FA_OK;
}

// Strided inputs: element strides (batch, head, row) >= 0, multiples of 8
// (16-byte rows), a row stride no smaller than the row, tensors 16-byte
// aligned, and one head's K / V rows byte-addressable in 31 bits.
int check_strides(const void* p, const int64_t* st, int n_rows, int width) {
  if (!st) return FA_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % 8 != 0) return FA_ERR_SHAPE;
  if (st[2] < width || st[2] > INT32_MAX) return FA_ERR_SHAPE;
  if ((double)n_rows * (double)st[2] * 2.0 > (double)INT32_MAX) return FA_ERR_SHAPE;
  if (p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Any finite scale is accepted: 0 gives uniform weights over the visible
// keys, a negative scale reverses the order of the scores.
int check_scale(float scale) { return std::isfinite(scale) ? FA_OK : FA_ERR_SCALE; }

// The forward kernels mark hidden keys with -inf scores before multiplying
// by the scale, which for scale 0 would give 0 * -inf.  Scale 0 therefore
// runs as 2^-100: every visible score then differs from the row reference by
// less than 2^-80 in log2 units, and its float32 weight 2^(that) rounds to 1,
// which is the uniform weighting scale 0 defines (L = ln of the visible
// count up to about 1e-28).  The backward masks after the exponential and
// takes the scale as given.
float forward_scale(float scale) { return scale == 0.f ? 0x1p-100f : scale; }

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout parameters for probability p: keep iff the generator byte >= t,
// t = min(255, round(256 p)); kept weights are scaled by 256 / (256 - t).
// Returns FA_ERR_DROPOUT unless 0 <= p < 1; *active is false when t = 0
// (nothing is dropped, the plain kernels run).
int make_dropout(float p, uint64_t seed, uint32_t offset, fa::Dropout* out, bool* active) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return FA_ERR_DROPOUT;
  int t = (int)std::floor(256.0 * (double)p + 0.5);
  if (t > 255) t = 255;
  out->k0 = (uint32_t)(seed & 0xffffffffu);
  out->k1 = (uint32_t)(seed >> 32);
  out->offset = offset;
  out->t = t;
  out->r = (float)(256.0 / (256 - t));
  *active = t > 0;
  return FA_OK;
}

}  // namespace

extern "C" {

float fa_dropout_applied_p(float p_drop) {
  fa::Dropout dp{};
  bool active = false;
  if (make_dropout(p_drop, 0, 0, &dp, &active) != FA_OK) return -1.f;
  return (float)dp.t / 256.f;
}

int fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  return hip_status(
      fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, N, d, d, causal, 1, nullptr, forward_scale(scale), nullptr,
                          nullptr, stream));
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream) {
  bool empty = false, active = false;
  fa::Dropout dp{};
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = make_dropout(p_drop, seed, offset, &dp, &active)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, N, d, d, causal, 1, nullptr,
                                        forward_scale(scale), active ? &dp : nullptr, nullptr, stream));
}

int fa_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int Nq, int Nk, int d,
              int dv, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape_ex(B, H, Nq, Nk, d, dv, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!o || !lse || (Nk > 0 && (!q || !k || !v))) return FA_ERR_NULL;
  return hip_status(
      fa::launch_fwd_bf16(q, k, v, o, lse, B * H, Nq, Nk, d, dv, causal, 1, nullptr, forward_scale(scale), nullptr,
                          nullptr, stream));
}

int fa_fwd_strided(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int Nq, int Nk,
                   int d, int dv, const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                   float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape_ex(B, H, Nq, Nk, d, dv, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_strides(q, q_strides, Nq, d)) != FA_OK) return st;
  if ((st = check_strides(k, k_strides, Nk, d)) != FA_OK) return st;
  if ((st = check_strides(v, v_strides, Nk, dv)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!o || !lse || (Nk > 0 && (!q || !k || !v))) return FA_ERR_NULL;
  const fa::Strides lay{q_strides[0], q_strides[1], k_strides[0], k_strides[1], v_strides[0], v_strides[1],
                        (int)q_strides[2],  (int)k_strides[2],  (int)v_strides[2],  H};
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, Nq, Nk, d, dv, causal, 1, nullptr,
                                        forward_scale(scale), nullptr, nullptr, stream, &lay));
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dv, int n_splits) {
  bool empty = false;
  if (check_shape_ex(B, H, Nq, Nk, d, dv, 0, &empty) != FA_OK || empty) return 0;
  if (n_splits < 0 || n_splits > 256) return 0;
  const int n = fa::fwd_splitkv_resolve(B * H, Nq, Nk, d, dv, n_splits);
  if (n <= 1) return 0;
  return (size_t)n * (size_t)B * (size_t)H * (size_t)Nq * (size_t)(dv + 1) * sizeof(float);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, void* workspace, int B, int H,
                   int Nq, int Nk, int d, int dv, float scale, int causal, int n_splits, hipStream_t stream) {
  bool empty = false;
  int st = check_shape_ex(B, H, Nq, Nk, d, dv, causal, &empty);
  if (st != FA_OK) return st;
  if (n_splits < 0 || n_splits > 256) return FA_ERR_SHAPE;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!o || !lse || (Nk > 0 && (!q || !k || !v))) return FA_ERR_NULL;
  const int n = fa::fwd_splitkv_resolve(B * H, Nq, Nk, d, dv, n_splits);
  if (n > 1 && !workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, Nq, Nk, d, dv, causal, n,
                                        static_cast<float*>(workspace), forward_scale(scale), nullptr, nullptr, stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  return hip_status(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, forward_scale(scale), causal, stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  bool empty = false;
  if (check_shape(B, H, N, d, 0, &empty) != FA_OK || empty) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
           float* dq, float* dk, float* dv, void* workspace, int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B * H,
                                        N, N, d, scale, causal, nullptr, nullptr, stream));
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
              float* dq, float* dk, float* dv, void* workspace, int B, int H, int Nq, int Nk, int d, float scale,
              int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape_ex(B, H, Nq, Nk, d, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  // nothing to write only when there are neither query rows nor keys; with
  // keys but no query rows dK = dV = 0, with rows but no keys dQ = 0
  if (B == 0 || H == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
  if (Nq > 0 && (!q || !o || !lse || !dout || !dq)) return FA_ERR_NULL;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  if (Nq > 0 && Nk > 0 && (!q || !k || !v)) return FA_ERR_NULL;
  if (Nq > 0 && Nk > 0 && !workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B * H,
                                        Nq, Nk, d, scale, causal, nullptr, nullptr, stream));
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                   float* dq, float* dk, float* dv, void* workspace, int B, int H, int N, int d,
                   const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides, float scale,
                   int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = check_strides(q, q_strides, N, d)) != FA_OK) return st;
  if ((st = check_strides(k, k_strides, N, d)) != FA_OK) return st;
  if ((st = check_strides(v, v_strides, N, d)) != FA_OK) return st;
  if (k_strides[2] != v_strides[2]) return FA_ERR_SHAPE;  // K and V rows share one stride
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  const fa::Strides lay{q_strides[0], q_strides[1], k_strides[0], k_strides[1], v_strides[0], v_strides[1],
                        (int)q_strides[2],  (int)k_strides[2],  (int)v_strides[2],  H};
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B * H,
                                        N, N, d, scale, causal, nullptr, nullptr, stream, &lay));
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                   float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                   hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (2 * (unsigned long long)B * (unsigned long long)H * (unsigned long long)N > fa::scratch_floats())
    return FA_ERR_SCRATCH;
  float* ws = nullptr;
  if (fa::scratch_on_current_device(&ws) != hipSuccess) return FA_ERR_HIP;
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, ws, B * H, N, N, d, scale, causal,
                                        nullptr, nullptr, stream));
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                   float* dq, float* dk, float* dv, void* workspace, int B, int H, int N, int d, float scale,
                   int causal, float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream) {
  bool empty = false, active = false;
  fa::Dropout dp{};
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if ((st = make_dropout(p_drop, seed, offset, &dp, &active)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B * H,
                                        N, N, d, scale, causal, active ? &dp : nullptr, nullptr, stream));
}

int fa_bwd_prep(const void* dout, const float* o, const float* lse, void* workspace, int B, int H, int N, int d,
                float scale, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, 0, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!dout || !o || !lse) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_bwd_prep(dout, o, lse, static_cast<float*>(workspace), B * H, N, d, scale, stream));
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const void* workspace, float* dk,
                float* dv, int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !dout || !dk || !dv) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  return hip_status(fa::launch_bwd_dkdv(q, k, v, dout, static_cast<const float*>(workspace), dk, dv, B * H, N, N, d,
                                        scale, causal, nullptr, nullptr, stream));
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const void* workspace, float* dq,
              int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_shape(B, H, N, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !dout || !dq) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  const float* ws = static_cast<const float*>(workspace);
  const size_t rows = (size_t)B * (size_t)H * (size_t)N;
  return hip_status(
      fa::launch_bwd_dq_bf16(q, k, v, dout, ws + rows, ws, dq, B * H, N, N, d, scale, causal, nullptr, nullptr,
                             stream));
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse, const int* cu_seqlens, int B,
                  int H, int total, int max_seqlen, int d, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_varlen(B, H, total, max_seqlen, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !cu_seqlens) return FA_ERR_NULL;
  const fa::Seqs sq{cu_seqlens, H, total};
  return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, max_seqlen, max_seqlen, d, d, causal, 1, nullptr,
                                        forward_scale(scale), nullptr, &sq, stream));
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                  float* dq, float* dk, float* dv, void* workspace, const int* cu_seqlens, int B, int H, int total,
                  int max_seqlen, int d, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  int st = check_varlen(B, H, total, max_seqlen, d, causal, &empty);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens) return FA_ERR_NULL;
  if (!workspace) return FA_ERR_WORKSPACE;
  const fa::Seqs sq{cu_seqlens, H, total};
  return hip_status(fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B * H,
                                        max_seqlen, max_seqlen, d, scale, causal, nullptr, &sq, stream));
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (negative B/H/N, causal not 0/1, or size overflow)";
    case FA_ERR_HEADDIM: return "unsupported head dimension (supported: 64, 128)";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_WORKSPACE: return "workspace is NULL";
    case FA_ERR_HIP: return "HIP runtime rejected a kernel launch";
    case FA_ERR_DROPOUT: return "dropout probability must be in [0, 1)";
    case FA_ERR_SCRATCH: return "problem too large for the built-in scratch (B*H*N above 2^21 query rows)";
    default: return "unknown fa_status";
  }
}

}  // extern "C"

// Host-only checks of the C ABI's argument handling under AddressSanitizer
// and UndefinedBehaviorSanitizer (built with launch_stubs.cpp, no GPU).  Each
// case calls an entry point with arguments its header declares invalid (or
// empty, or extreme) and compares the status code; a case whose arguments
// are valid must reach a launcher (the stubs answer FA_ERR_HIP), and no
// invalid or empty call may reach one.  Extreme sizes (INT_MAX dimensions)
// run the size arithmetic where a signed overflow would be reported.
// Test infrastructure only.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "fa.h"

extern int g_launches;

namespace {

int n_cases = 0, n_failed = 0;
alignas(16) char buf[256];
void* P = buf;
float* F = reinterpret_cast<float*>(buf);
const float nan_f = std::numeric_limits<float>::quiet_NaN();
const float inf_f = std::numeric_limits<float>::infinity();

// status must equal want; a launcher must have run iff want == FA_ERR_HIP
void expect(int line, int status, int want, int launches_before) {
  ++n_cases;
  const bool launched = g_launches != launches_before;
  if (status != want || launched != (want == FA_ERR_HIP)) {
    ++n_failed;
    std::printf("FAIL line %d: status %d (%s), expected %d; launcher %s\n", line, status, fa_status_string(status),
                want, launched ? "reached" : "not reached");
  }
}
#define EXPECT(call, want)               \
  do {                                   \
    const int before_ = g_launches;      \
    const int st_ = (call);              \
    expect(__LINE__, st_, want, before_); \
  } while (0)

void size_check(int line, size_t got, size_t want) {
  ++n_cases;
  if (got != want) {
    ++n_failed;
    std::printf("FAIL line %d: size %zu, expected %zu\n", line, got, want);
  }
}
#define EXPECT_SIZE(call, want) size_check(__LINE__, (call), (want))

int fwd(int B, int H, int N, int d, float scale, int causal, void* q = P, float* o = F) {
  return fa_fwd(q, P, P, o, F, B, H, N, d, scale, causal, nullptr);
}
int fwd_f32(int B, int H, int N, int d, float scale, int causal, const float* q = F) {
  return fa_fwd_f32(q, F, F, F, F, B, H, N, d, scale, causal, nullptr);
}
int fwd_ex(int B, int H, int Nq, int Nk, int d, int dv, float scale, int causal, float* o = F) {
  return fa_fwd_ex(P, P, P, o, F, B, H, Nq, Nk, d, dv, scale, causal, nullptr);
}
int bwd(int B, int H, int N, int d, float scale, int causal, void* ws = P, float* dv = F) {
  return fa_bwd(P, P, P, F, F, P, F, F, dv, ws, B, H, N, d, scale, causal, nullptr);
}
int bwd_ex(int B, int H, int Nq, int Nk, int d, float scale, int causal, void* ws = P, float* dk = F,
           const void* q = P) {
  return fa_bwd_ex(q, P, P, F, F, P, F, dk, F, ws, B, H, Nq, Nk, d, scale, causal, nullptr);
}
int noalloc(int B, int H, int N, int d, float scale, int causal, float* dq = F) {
  return fa_bwd_noalloc(P, P, P, F, F, P, dq, F, F, B, H, N, d, scale, causal, nullptr);
}
int fwd_drop(int B, int N, int d, float p, float scale = 0.125f, float* o = F) {
  return fa_fwd_dropout(P, P, P, o, F, B, 2, N, d, scale, 0, p, UINT64_MAX, UINT32_MAX, nullptr);
}
int bwd_drop(int B, int N, int d, float p, void* ws = P) {
  return fa_bwd_dropout(P, P, P, F, F, P, F, F, F, ws, B, 2, N, d, 0.125f, 1, p, 7, 0, nullptr);
}
int fwd_varlen(int B, int H, int total, int max_len, int d, const int* cu) {
  return fa_fwd_varlen(P, P, P, F, F, cu, B, H, total, max_len, d, 0.125f, 1, nullptr);
}
int bwd_varlen(int B, int H, int total, int max_len, int d, const int* cu, void* ws = P) {
  return fa_bwd_varlen(P, P, P, F, F, P, F, F, F, ws, cu, B, H, total, max_len, d, 0.125f, 0, nullptr);
}
int strided(const int64_t* qs, const int64_t* ks, const int64_t* vs, int Nq, int Nk, int d, int dv,
            void* q = P) {
  return fa_fwd_strided(q, P, P, F, F, 1, 2, Nq, Nk, d, dv, qs, ks, vs, 0.125f, 0, nullptr);
}

}  // namespace

int main() {
  const int cu[3] = {0, 4, 10};

  // ---- fa_fwd / fa_fwd_f32: shapes, head widths, scale, pointers, empty
  for (int f = 0; f < 2; ++f) {
    auto call = [&](int B, int H, int N, int d, float s, int c) {
      return f == 0 ? fwd(B, H, N, d, s, c) : fwd_f32(B, H, N, d, s, c);
    };
    EXPECT(call(1, 1, 8, 96, 0.125f, 0), FA_ERR_HEADDIM);
    EXPECT(call(1, 1, 8, 0, 0.125f, 0), FA_ERR_HEADDIM);
    EXPECT(call(1, 1, 8, INT_MIN, 0.125f, 0), FA_ERR_HEADDIM);
    EXPECT(call(1, 1, -1, 64, 0.125f, 0), FA_ERR_SHAPE);
    EXPECT(call(INT_MIN, 1, 8, 64, 0.125f, 0), FA_ERR_SHAPE);
    EXPECT(call(1, 1, 8, 64, 0.125f, 2), FA_ERR_SHAPE);
    EXPECT(call(1, 1, 8, 64, 0.125f, -1), FA_ERR_SHAPE);
    EXPECT(call(INT_MAX, INT_MAX, INT_MAX, 128, 0.125f, 1), FA_ERR_SHAPE);
    EXPECT(call(65536, 65536, 1, 64, 0.125f, 0), FA_ERR_SHAPE);   // B*H above 2^31 - 1
    EXPECT(call(1, 1, 1 << 23, 128, 0.125f, 0), FA_ERR_SHAPE);    // one head of O past 2^31 bytes
    EXPECT(call(1, 1, 8, 64, nan_f, 0), FA_ERR_SCALE);
    EXPECT(call(1, 1, 8, 64, -inf_f, 1), FA_ERR_SCALE);
    EXPECT(call(0, INT_MAX, 1000, 64, 0.125f, 0), FA_OK);         // empty: nothing runs
    EXPECT(call(0, 1, INT_MAX, 64, 0.125f, 0), FA_ERR_SHAPE);     // the per-head size limit still holds
    EXPECT(call(1, 1, 0, 64, 0.125f, 1), FA_OK);
    EXPECT(call(1, 1, 8, 64, 0.f, 0), FA_ERR_HIP);                 // scale 0 is valid
    EXPECT(call(3, 5, 1000, 128, -0.5f, 1), FA_ERR_HIP);          // so is a negative one
  }
  EXPECT(fwd(1, 1, 8, 64, 0.125f, 0, nullptr), FA_ERR_NULL);
  EXPECT(fwd(1, 1, 8, 64, 0.125f, 0, P, nullptr), FA_ERR_NULL);
  EXPECT(fwd_f32(1, 1, 8, 64, 0.125f, 0, nullptr), FA_ERR_NULL);

  // ---- fa_fwd_ex: independent lengths and widths
  EXPECT(fwd_ex(1, 2, 8, 8, 64, 96, 0.1f, 0), FA_ERR_HEADDIM);
  EXPECT(fwd_ex(1, 2, 8, 8, 32, 64, 0.1f, 0), FA_ERR_HEADDIM);
  EXPECT(fwd_ex(1, 2, -1, 8, 64, 64, 0.1f, 0), FA_ERR_SHAPE);
  EXPECT(fwd_ex(1, 2, 8, -1, 64, 64, 0.1f, 0), FA_ERR_SHAPE);
  EXPECT(fwd_ex(1, 2, 1 << 22, 8, 64, 128, 0.1f, 0), FA_ERR_SHAPE);
  EXPECT(fwd_ex(1, 2, 8, 1 << 23, 128, 64, 0.1f, 0), FA_ERR_SHAPE);
  EXPECT(fwd_ex(INT_MAX, 1, INT_MAX, INT_MAX, 128, 128, 0.1f, 1), FA_ERR_SHAPE);
  EXPECT(fwd_ex(1, 2, 8, 8, 64, 64, inf_f, 0), FA_ERR_SCALE);
  EXPECT(fwd_ex(1, 2, 8, 8, 64, 64, 0.1f, 0, nullptr), FA_ERR_NULL);
  EXPECT(fwd_ex(1, 2, 0, 8, 64, 64, 0.1f, 0, nullptr), FA_OK);
  EXPECT(fwd_ex(1, 2, 37, 300, 128, 64, 0.1f, 1), FA_ERR_HIP);
  EXPECT(fwd_ex(1, 2, 5, 0, 64, 128, 0.1f, 1), FA_ERR_HIP);     // no keys: still a launch (0, -inf)

  // ---- fa_fwd_strided
  {
    const int64_t ok[3] = {4096, 512, 128}, odd[3] = {4096, 512, 60}, narrow[3] = {4096, 512, 56},
                  neg[3] = {-8, 512, 128}, wide[3] = {0, 0, 2048}, huge[3] = {0, 0, INT64_MAX - 7};
    EXPECT(strided(nullptr, ok, ok, 8, 8, 64, 64), FA_ERR_NULL);
    EXPECT(strided(odd, ok, ok, 8, 8, 64, 64), FA_ERR_SHAPE);
    EXPECT(strided(ok, narrow, ok, 8, 8, 64, 64), FA_ERR_SHAPE);
    EXPECT(strided(ok, ok, neg, 8, 8, 64, 64), FA_ERR_SHAPE);
    EXPECT(strided(ok, wide, ok, 8, 1 << 20, 64, 64), FA_ERR_SHAPE);
    EXPECT(strided(ok, huge, ok, 8, 8, 64, 64), FA_ERR_SHAPE);
    EXPECT(strided(ok, ok, ok, 8, 8, 64, 64, buf + 8), FA_ERR_SHAPE);  // not 16-byte aligned
    EXPECT(strided(ok, ok, ok, 8, 8, 96, 64), FA_ERR_HEADDIM);
    EXPECT(strided(ok, ok, ok, 8, 8, 64, 64), FA_ERR_HIP);
  }

  // ---- split-KV: request range, workspace
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, P, 1, 1, 1, 8192, 128, 128, 0.1f, 0, 300, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, P, 1, 1, 1, 8192, 128, 128, 0.1f, 0, -1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, nullptr, 1, 1, 1, 8192, 128, 128, 0.1f, 0, 4, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, P, 1, 1, 1, 8192, 128, 32, 0.1f, 0, 4, nullptr), FA_ERR_HEADDIM);
  EXPECT(fa_fwd_splitkv(P, P, P, F, F, P, 1, 1, 1, 8192, 128, 128, 0.1f, 0, 4, nullptr), FA_ERR_HIP);
  EXPECT_SIZE(fa_fwd_splitkv_workspace_bytes(1, 1, 1, 8192, 128, 128, 4), 4 * 129 * 4);
  EXPECT_SIZE(fa_fwd_splitkv_workspace_bytes(1, 1, 1, 8192, 128, 128, 300), 0);
  EXPECT_SIZE(fa_fwd_splitkv_workspace_bytes(1, 1, 1, 8192, 96, 128, 4), 0);
  EXPECT_SIZE(fa_fwd_splitkv_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, 128, 256), 0);

  // ---- backward with a caller workspace
  EXPECT(bwd(1, 2, 8, 32, 0.125f, 0), FA_ERR_HEADDIM);
  EXPECT(bwd(1, 2, -5, 64, 0.125f, 0), FA_ERR_SHAPE);
  EXPECT(bwd(1, 2, 8, 64, nan_f, 0), FA_ERR_SCALE);
  EXPECT(bwd(1, 2, 8, 64, 0.125f, 0, nullptr), FA_ERR_WORKSPACE);
  EXPECT(bwd(1, 2, 8, 64, 0.125f, 0, P, nullptr), FA_ERR_NULL);
  EXPECT(bwd(0, 2, 8, 64, 0.125f, 0, nullptr, nullptr), FA_OK);
  EXPECT(bwd(INT_MAX, INT_MAX, INT_MAX, 64, 0.125f, 1), FA_ERR_SHAPE);
  EXPECT(bwd(2, 16, 4096, 128, 0.125f, 1), FA_ERR_HIP);
  EXPECT_SIZE(fa_bwd_workspace_bytes(2, 16, 4096, 128), 2 * 16 * 4096 * 8);
  EXPECT_SIZE(fa_bwd_workspace_bytes(0, 16, 4096, 128), 0);
  EXPECT_SIZE(fa_bwd_workspace_bytes(1, 1, 10, 48), 0);
  EXPECT_SIZE(fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128), 0);

  // ---- backward with differing query and key counts
  EXPECT(bwd_ex(1, 2, 8, 5, 96, 0.125f, 0), FA_ERR_HEADDIM);
  EXPECT(bwd_ex(1, 2, -1, 5, 64, 0.125f, 0), FA_ERR_SHAPE);
  EXPECT(bwd_ex(1, 2, 8, INT_MIN, 64, 0.125f, 0), FA_ERR_SHAPE);
  EXPECT(bwd_ex(1, 2, 8, 5, 64, 0.125f, 2), FA_ERR_SHAPE);
  EXPECT(bwd_ex(1, 2, 8, 5, 64, inf_f, 0), FA_ERR_SCALE);
  EXPECT(bwd_ex(1, 2, 8, 5, 64, 0.125f, 0, nullptr), FA_ERR_WORKSPACE);
  EXPECT(bwd_ex(1, 2, 8, 5, 64, 0.125f, 0, P, nullptr), FA_ERR_NULL);
  EXPECT(bwd_ex(1, 2, 8, 5, 64, 0.125f, 0, P, F, nullptr), FA_ERR_NULL);
  EXPECT(bwd_ex(1, 2, 0, 0, 64, 0.125f, 1, nullptr, nullptr, nullptr), FA_OK);
  EXPECT(bwd_ex(0, 2, 8, 5, 64, 0.125f, 1, nullptr, nullptr, nullptr), FA_OK);
  EXPECT(bwd_ex(1, 2, 0, 5, 64, 0.125f, 1, nullptr, F, nullptr), FA_ERR_HIP);   // no rows: dK = dV = 0 written
  EXPECT(bwd_ex(1, 2, 0, 5, 64, 0.125f, 1, nullptr, nullptr, nullptr), FA_ERR_NULL);
  EXPECT(bwd_ex(1, 2, 8, 0, 64, 0.125f, 0, nullptr, nullptr), FA_ERR_HIP);       // no keys: dQ = 0 written
  EXPECT(bwd_ex(1, 2, 1 << 23, 5, 64, 0.125f, 0), FA_ERR_SHAPE);
  EXPECT(bwd_ex(INT_MAX, INT_MAX, 8, 5, 128, 0.125f, 1), FA_ERR_SHAPE);
  EXPECT(bwd_ex(2, 16, 4096, 1000, 128, 0.125f, 1), FA_ERR_HIP);

  // ---- backward on strided inputs
  {
    const int64_t dense[3] = {2 * 8 * 64, 8 * 64, 64}, packed[3] = {8 * 3 * 2 * 64, 64, 3 * 2 * 64};
    const int64_t narrow[3] = {0, 0, 56}, odd[3] = {0, 0, 68}, wide[3] = {0, 0, 1 << 30};
    auto sb = [&](const int64_t* qs, const int64_t* ks, const int64_t* vs, int N = 8, void* ws = P) {
      return fa_bwd_strided(P, P, P, F, F, P, F, F, F, ws, 1, 2, N, 64, qs, ks, vs, 0.125f, 1, nullptr);
    };
    EXPECT(sb(packed, packed, packed), FA_ERR_HIP);
    EXPECT(sb(dense, packed, packed), FA_ERR_HIP);
    EXPECT(sb(packed, dense, packed), FA_ERR_SHAPE);  // K and V row strides differ
    EXPECT(sb(narrow, packed, packed), FA_ERR_SHAPE);
    EXPECT(sb(packed, odd, odd), FA_ERR_SHAPE);
    EXPECT(sb(packed, wide, wide), FA_ERR_SHAPE);     // one head past 2^31 bytes
    EXPECT(sb(nullptr, packed, packed), FA_ERR_NULL);
    EXPECT(sb(packed, packed, packed, 8, nullptr), FA_ERR_WORKSPACE);
    EXPECT(sb(packed, packed, packed, 0, nullptr), FA_OK);
  }

  // ---- the backward phases
  EXPECT(fa_bwd_prep(P, F, F, P, 1, 2, 8, 96, 0.1f, nullptr), FA_ERR_HEADDIM);
  EXPECT(fa_bwd_prep(P, F, F, nullptr, 1, 2, 8, 64, 0.1f, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_bwd_prep(P, nullptr, F, P, 1, 2, 8, 64, 0.1f, nullptr), FA_ERR_NULL);
  EXPECT(fa_bwd_prep(P, F, F, P, 1, 2, 8, 64, -inf_f, nullptr), FA_ERR_SCALE);
  EXPECT(fa_bwd_prep(P, F, F, P, 1, 2, 8, 64, 0.1f, nullptr), FA_ERR_HIP);
  EXPECT(fa_bwd_dkdv(P, P, P, P, P, F, nullptr, 1, 2, 8, 64, 0.1f, 0, nullptr), FA_ERR_NULL);
  EXPECT(fa_bwd_dkdv(P, P, P, P, nullptr, F, F, 1, 2, 8, 64, 0.1f, 0, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_bwd_dkdv(P, P, P, P, P, F, F, 1, 2, 8, 64, 0.1f, 3, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_bwd_dkdv(P, P, P, P, P, F, F, 1, 2, 8, 64, 0.1f, 1, nullptr), FA_ERR_HIP);
  EXPECT(fa_bwd_dq(P, P, nullptr, P, P, F, 1, 2, 8, 64, 0.1f, 0, nullptr), FA_ERR_NULL);
  EXPECT(fa_bwd_dq(P, P, P, P, P, F, 1, 2, -1, 64, 0.1f, 0, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_bwd_dq(P, P, P, P, nullptr, F, 0, 2, 8, 64, 0.1f, 0, nullptr), FA_OK);
  EXPECT(fa_bwd_dq(P, P, P, P, P, F, 1, 2, 8, 128, 0.1f, 1, nullptr), FA_ERR_HIP);

  // ---- the allocation-free backward: scratch of 2^21 query rows
  EXPECT(noalloc(1, 1, (1 << 21) + 1, 64, 0.125f, 0), FA_ERR_SCRATCH);
  EXPECT(noalloc(2, 16, 65537, 64, 0.125f, 1), FA_ERR_SCRATCH);
  EXPECT(noalloc(1, 1, 8, 64, 0.125f, 0, nullptr), FA_ERR_NULL);
  EXPECT(noalloc(1, 1, 8, 64, nan_f, 0), FA_ERR_SCALE);
  EXPECT(noalloc(0, 1, 8, 64, 0.125f, 0, nullptr), FA_OK);
  EXPECT(noalloc(1, 1, 1 << 21, 128, 0.125f, 0), FA_ERR_HIP);   // at the limit: reaches the device lookup

  // ---- dropout
  const float bad_p[5] = {-0.01f, 1.0f, 1.5f, nan_f, inf_f};
  for (float p : bad_p) {
    EXPECT(fwd_drop(1, 8, 64, p), FA_ERR_DROPOUT);
    EXPECT(bwd_drop(1, 8, 64, p), FA_ERR_DROPOUT);
  }
  EXPECT(fwd_drop(1, 8, 96, 0.1f), FA_ERR_HEADDIM);
  EXPECT(fwd_drop(1, -1, 64, 0.1f), FA_ERR_SHAPE);
  EXPECT(fwd_drop(1, 8, 64, 0.1f, nan_f), FA_ERR_SCALE);
  EXPECT(fwd_drop(1, 8, 64, 0.1f, 0.125f, nullptr), FA_ERR_NULL);
  EXPECT(bwd_drop(1, 8, 64, 0.1f, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fwd_drop(0, 8, 64, 0.1f), FA_OK);
  EXPECT(fwd_drop(1, 8, 64, 0.1f), FA_ERR_HIP);
  EXPECT(bwd_drop(1, 8, 64, 0.999f), FA_ERR_HIP);
  ++n_cases;
  if (fa_dropout_applied_p(0.1f) != 26.f / 256.f || fa_dropout_applied_p(0.999f) != 255.f / 256.f ||
      fa_dropout_applied_p(0.f) != 0.f || fa_dropout_applied_p(1.f) != -1.f || fa_dropout_applied_p(nan_f) != -1.f) {
    ++n_failed;
    std::printf("FAIL: fa_dropout_applied_p\n");
  }

  // ---- packed sequences
  for (int f = 0; f < 2; ++f) {
    auto call = [&](int B, int H, int total, int max_len, int d, const int* c) {
      return f == 0 ? fwd_varlen(B, H, total, max_len, d, c) : bwd_varlen(B, H, total, max_len, d, c);
    };
    EXPECT(call(2, 2, 10, 6, 96, cu), FA_ERR_HEADDIM);
    EXPECT(call(-1, 2, 10, 6, 64, cu), FA_ERR_SHAPE);
    EXPECT(call(2, -1, 10, 6, 64, cu), FA_ERR_SHAPE);
    EXPECT(call(2, 2, -1, 6, 64, cu), FA_ERR_SHAPE);
    EXPECT(call(2, 2, 10, -1, 64, cu), FA_ERR_SHAPE);
    EXPECT(call(2, 2, 10, 11, 64, cu), FA_ERR_SHAPE);               // longest above the packed axis
    EXPECT(call(2, 2, 1 << 22, 1, 128, cu), FA_ERR_SHAPE);          // 31-bit byte range of a sequence
    EXPECT(call(INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128, cu), FA_ERR_SHAPE);
    EXPECT(call(2, 2, 10, 6, 64, nullptr), FA_ERR_NULL);
    EXPECT(call(0, 2, 10, 6, 64, nullptr), FA_OK);
    EXPECT(call(2, 2, 0, 0, 64, nullptr), FA_OK);
    EXPECT(call(2, 2, 10, 6, 64, cu), FA_ERR_HIP);
  }
  EXPECT(bwd_varlen(2, 2, 10, 6, 64, cu, nullptr), FA_ERR_WORKSPACE);

  // ---- status strings: every code has its own text, unknown codes one too
  for (int s = -3; s < 12; ++s) {
    ++n_cases;
    const char* t = fa_status_string(s);
    if (!t || !t[0]) {
      ++n_failed;
      std::printf("FAIL: empty status string for %d\n", s);
    }
  }

  std::printf("%d cases, %d failed\n", n_cases, n_failed);
  return n_failed == 0 ? 0 : 1;
}

// Internal host-side launchers; called by the C ABI in fa_api.cpp after all
// arguments have been validated.  BH = B * H.  Each returns the HIP status of
// its launches (hipSuccess when everything was enqueued).
#pragma once

#include <hip/hip_runtime_api.h>

namespace fa {

// Dropout parameters (fa_dropout.h); a null pointer means no dropout.  The
// kernels with dropout exist for the square contract (Nq = Nk, dv = d).
struct Dropout;
// Packed variable-length sequences (fa_common.h); a null pointer means the
// dense [B, H, N, d] layout.  With sequences, BH is the number of (sequence,
// head) units B * H and N the longest sequence: it sizes the grid.
struct Seqs;

// Element strides of the forward's inputs: batch, head and row of Q, K and V
// (the head-dim stride is 1).  A null pointer means dense [B, H, N, d]
// tensors.  With strides, BH = B * H and H is needed to split it.
struct Strides {
  long long qb, qh, kb, kh, vb, vh;
  int qr, kr, vr;
  int H;
};

// The strides of dense [BH, Nq, d] / [BH, Nk, d] inputs in this layout (one
// head per batch entry).
inline Strides dense_strides(int Nq, int Nk, int d) {
  return Strides{(long long)Nq * d, 0, (long long)Nk * d, 0, (long long)Nk * d, 0, d, d, d, 1};
}

// Forward, bf16 inputs: Q [BH, Nq, d], K [BH, Nk, d], V [BH, Nk, dv].
// n_ksplit > 1 cuts the key tiles into that many ranges processed by separate
// workgroups; ws then holds n_ksplit * BH * Nq * (dv + 1) floats of partial
// results (fwd_splitkv_resolve gives the count actually used).
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq,
                           int Nk, int d, int dv, int causal, int n_ksplit, float* ws, float scale,
                           const Dropout* drop, const Seqs* seqs, hipStream_t stream,
                           const Strides* strides = nullptr);
// Forward for d = dv = 128 without dropout or split-KV ranges
// (fa_fwd_r64.hip), same arguments and layout as launch_fwd_bf16 with
// n_ksplit = 1; launch_fwd_bf16 routes these calls here.
bool fwd_r64_applies(int d, int dv);
hipError_t launch_fwd_r64(const void* q, const void* k, const void* v, float* o, float* lse, int BH, int Nq, int Nk,
                          int causal, float scale, const Seqs* seqs, const Strides& lay, hipStream_t stream);
// Number of key ranges a split-KV forward uses for n_splits requested
// (0: chosen for the grid); 1 means no split and no workspace.
int fwd_splitkv_resolve(int BH, int Nq, int Nk, int d, int dv, int n_splits);

// Split-KV forward for 1 .. kDecodeMaxRows query rows with d == dv on the
// vector ALUs (fa_decode.hip): one workgroup per (head, key range) of
// keys_per_split keys writes its partial O rows to opart ([n_split][BH * Nq]
// rows of d floats) and its logsumexp to lpart, the layout the split-KV merge
// reads.  c = scale * log2(e).  Dense [BH, N, d] inputs only.
constexpr int kDecodeMaxRows = 4;
bool decode_applies(int Nq, int d, int dv);
hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, float* opart, float* lpart, int BH, int Nq,
                              int Nk, int d, int n_split, int keys_per_split, float c, int causal,
                              hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N,
                          int d, float scale, int causal, hipStream_t stream);

// dQ only, query-stationary (fa_bwd_dq.hip); l2 and dsc are the per-row
// L log2(e) and scale * D written by the backward preprocess.  Nq query rows
// and Nk keys per head (upper-left causal mask when they differ).
hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout, const float* l2,
                              const float* dsc, float* dq, int BH, int Nq, int Nk, int d, float scale, int causal,
                              const Dropout* drop, const Seqs* seqs, hipStream_t stream,
                              const Strides* lay = nullptr);
// The dQ pass with the preprocess fused in: computes scale D = scale dO . O and
// L log2(e) of its rows from o and lse (bitwise as launch_bwd_prep does),
// stores them to l2 / dsc for a dK/dV launch that follows, and writes dq.
hipError_t launch_bwd_dq_fused(const void* q, const void* k, const void* v, const void* dout, const float* o,
                               const float* lse, float* l2, float* dsc, float* dq, int BH, int Nq, int Nk, int d,
                               float scale, int causal, const Dropout* drop, const Seqs* seqs, hipStream_t stream,
                               const Strides* lay = nullptr);

// Backward phases (fa_bwd.hip); ws holds [scale * D | L log2(e)], one float
// each per query row (BH * Nq).  The preprocess works on query rows only.
hipError_t launch_bwd_prep(const void* dout, const float* o, const float* lse, float* ws, int BH, int N, int d,
                           float scale, hipStream_t stream);
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* ws,
                           float* dk, float* dv, int BH, int Nq, int Nk, int d, float scale, int causal,
                           const Dropout* drop, const Seqs* seqs, hipStream_t stream,
                           const Strides* lay = nullptr);

// The allocation-free backward's scratch (fa_scratch.hip): its capacity in
// floats, and its device address on the current device (looked up once per
// device).
size_t scratch_floats();
hipError_t scratch_on_current_device(float** out);

// lay: element strides of strided Q, K, V (batch, head, row; K and V share
// the row stride), null for dense inputs; dO, O, L and the gradients are
// always dense.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, float* dvec, int BH, int Nq, int Nk,
                           int d, float scale, int causal, const Dropout* drop, const Seqs* seqs,
                           hipStream_t stream, const Strides* lay = nullptr);

}  // namespace fa

/*
 * fa.h -- C ABI of the exact IO-aware attention library (libfa.so, gfx950).
 *
 * The library computes exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T) V,      L = logsumexp(scale * Q K^T) (natural log),
 * block by block with an online softmax, so no N x N score or probability
 * matrix is ever written to device memory, and its gradient by recomputing
 * the probability tiles from Q, K and the saved L.
 *
 * Sources: "FlashAttention: The Matrix You Never Have to Write Down"
 * (maitreyasuin.github.io), sections "What attention computes", "The
 * identity", "From softmax to attention", "Build it", "Causal masking" and
 * "The forward pass is only half of it"; "Why FlashAttention Can Avoid a
 * Square Attention Array Without Making Attention Linear"
 * (leviathansystems.co), sections "Tiles need a shared softmax
 * normalization" and "Backward can recreate tiles instead of retaining the
 * square".
 *
 * Conventions shared by every entry point
 *  - Layout: every [B,H,N,d] tensor is dense row-major with d innermost
 *    (element (b,h,n,c) at ((b*H + h)*N + n)*d + c); L and the backward
 *    workspace rows are [B,H,N].  Q, K, V (and dO) are bf16 except for
 *    fa_fwd_f32; O, L, dQ, dK, dV are float32.
 *  - Causal masking is upper-left: query n sees keys 0..n (the
 *    is_causal=True convention of torch SDPA), "Build it" note on
 *    alignment.  causal is 0 or 1.
 *  - Memory: the caller allocates every buffer in device memory (hipMalloc or
 *    torch); the library never allocates, frees or synchronises.  Inputs are
 *    read only; outputs must not overlap inputs or each other.
 *  - Execution: work is enqueued on `stream` (NULL = the null stream) and
 *    the call returns at once; results are ready when the caller
 *    synchronises that stream.  Kernel faults surface at that point.
 *  - Errors: all arguments are checked on the host before anything is
 *    enqueued; on error nothing is launched and an fa_status code is
 *    returned.  B, H or N equal to 0 is a valid empty problem: FA_OK,
 *    nothing launched.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,     /* B, H or N negative, causal not 0/1, B*H above
                           INT32_MAX, or N*d*4 above INT32_MAX (one head of a
                           float32 tensor must be byte-addressable in 31 bits) */
  FA_ERR_HEADDIM = 3,   /* d is not a supported head width (64 or 128)         */
  FA_ERR_SCALE = 4,     /* scale is not finite (inf or NaN)                    */
  FA_ERR_WORKSPACE = 5, /* a required workspace is NULL                        */
  FA_ERR_HIP = 6,       /* a kernel launch was rejected by the HIP runtime     */
  FA_ERR_DROPOUT = 7,   /* dropout probability not in [0, 1)                   */
  FA_ERR_SCRATCH = 8    /* fa_bwd_noalloc: B*H*N above its scratch (2^21 rows) */
} fa_status;

/*
 * Forward pass, bf16 inputs ("From softmax to attention" and "Build it").
 *   q, k, v : device, bf16 [B,H,N,d]
 *   o       : device, float32 [B,H,N,d]  -- normalised output
 *   lse     : device, float32 [B,H,N]    -- per-row logsumexp of the scaled,
 *             masked scores, natural log; the statistic the backward needs
 *   d       : 64 or 128
 *   scale   : any finite value, usually 1/sqrt(d) ("Build it" fixes that
 *             choice; the caller may pass another).  0 weighs every visible
 *             key equally (O = their mean, L = ln of their count); a negative
 *             scale reverses the order of the scores.
 * Scores and the row sums stay on chip: S = Q K^T is formed one key tile at
 * a time on bf16 matrix cores with float32 accumulation; the weights are
 * taken against a per-row reference (the exact max of the row's first keys,
 * or of all its keys if float32 would overflow otherwise, "What it doesn't
 * solve" on the first page), rounded to bf16 for the P V product, and O is
 * divided by the row sum once, after the last tile.
 */
int fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * General forward, the first page's flash_attention contract ("Build it"):
 *   q : device, bf16 [B,H,Nq,d]      k : device, bf16 [B,H,Nk,d]
 *   v : device, bf16 [B,H,Nk,dv]     o : device, float32 [B,H,Nq,dv]
 *   lse : device, float32 [B,H,Nq]
 *   d, dv : 64 or 128 each.  Nq and Nk are independent; causal masking is
 *   upper-left for any Nq, Nk (key j visible to query i iff j <= i).
 *   Nk == 0 (no keys) gives o = 0 and lse = -inf for every row, per the
 *   page's empty-key policy ("Check it"); q, k, v may then be NULL.
 * fa_fwd(q,k,v,o,lse,B,H,N,d,...) is fa_fwd_ex(...,Nq=N,Nk=N,d,dv=d,...).
 * Per head, Nq*dv*4, Nk*d*2 and Nk*dv*2 bytes must stay below 2^31.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse,
              int B, int H, int Nq, int Nk, int d, int dv, float scale, int causal, hipStream_t stream);

/*
 * The general forward on strided inputs: Q, K, V may be views (for example
 * slices of one packed QKV projection), as the page's flash_attention takes
 * any tensor ("Build it").  Same contract and outputs as fa_fwd_ex, plus
 *   q_strides, k_strides, v_strides : host arrays of 3 element strides
 *     (batch, head, row) of Q, K, V; the head-dim stride is 1.
 * Each stride must be >= 0 and a multiple of 8 (16-byte rows), a row stride
 * at least the row width (d, or dv for V) and below 2^31, one head's rows
 * byte-addressable in 31 bits (N * row stride * 2 < 2^31), and q, k, v
 * 16-byte aligned; otherwise FA_ERR_SHAPE (NULL stride arrays: FA_ERR_NULL).
 * O and lse are dense [B,H,Nq,dv] and [B,H,Nq].
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, float* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, int dv,
                   const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                   float scale, int causal, hipStream_t stream);

/*
 * Split-KV forward (Flash-Decoding, "What it doesn't solve" on the first
 * page): for few query rows and long key sequences, the key tiles are cut
 * into contiguous ranges that separate workgroups process in parallel; each
 * writes a partial (O, L) into `workspace`, and a second kernel merges them
 * with the logsumexp identity ("The identity").  Same contract and results
 * (up to rounding) as fa_fwd_ex.  With one to four query rows and d == dv the
 * ranges run on the vector ALUs and weight V with unrounded float32
 * probabilities; otherwise the matrix-core kernel rounds them to bf16 first,
 * as fa_fwd_ex does.
 *   n_splits : 1 .. 256 ranges requested (capped at the number of key
 *              tiles), or 0 to let the library choose for the grid.
 *   workspace: device, >= fa_fwd_splitkv_workspace_bytes(...) bytes for the
 *              same arguments (0 bytes -- and NULL allowed -- when the
 *              request resolves to a single range).
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int dv, int n_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse, void* workspace,
                   int B, int H, int Nq, int Nk, int d, int dv, float scale, int causal, int n_splits,
                   hipStream_t stream);

/*
 * Forward pass with float32 inputs, computed entirely in float32 (same
 * contract as fa_fwd otherwise): the precision of the first page's own
 * exactness check ("Check it", float32 against a float64 reference at
 * 1e-5).  For small exact checks; not tuned.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: two float32 per query row
 * (scale * D_i with D_i = dO_i . O_i, and L_i log2(e)).  Returns 0 for an
 * empty or invalid shape.  Infrastructure (buffer sizing): no passage of the
 * pages defines it; D_i is the row sum of the chain-rule backward that
 * fa_bwd documents.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass by recomputation ("The forward pass is only half of it";
 * "Backward can recreate tiles instead of retaining the square").
 *   q, k, v, dout : device, bf16 [B,H,N,d]   (dout = dL/dO)
 *   o, lse        : device, float32, as written by fa_fwd for the same inputs
 *   dq, dk, dv    : device, float32 [B,H,N,d] -- fully overwritten
 *   workspace     : device, >= fa_bwd_workspace_bytes(B,H,N,d) bytes; its
 *                   contents on entry do not matter
 * The probability tiles are rebuilt from Q, K and lse; no N x N tensor is
 * stored.  Two kernels run on `stream`: a query-stationary pass for dq
 * (which recomputes the score tiles instead of summing partial dq with
 * atomics, and first computes the per-row statistics the backward needs,
 * storing them to the workspace), then a key-stationary pass for dk and dv.
 * Every output element is written once: results are deterministic.
 */
int fa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
           const void* dout, float* dq, float* dk, float* dv, void* workspace,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd for Nq query rows against Nk keys per head: the backward of fa_fwd_ex
 * with dv = d ("Build it": the query and key lengths may differ, and the
 * causal mask is anchored at the upper left, so row i sees keys j <= i).
 *   q, dout       : device, bf16 [B,H,Nq,d];  k, v : device, bf16 [B,H,Nk,d]
 *   o, lse        : device, float32 [B,H,Nq,d] and [B,H,Nq], as written by
 *                   fa_fwd_ex for the same inputs (dv = d)
 *   dq            : device, float32 [B,H,Nq,d];  dk, dv : float32 [B,H,Nk,d]
 *                   -- all fully overwritten
 *   workspace     : device, >= fa_bwd_workspace_bytes(B,H,Nq,d) bytes; may
 *                   be NULL when Nq or Nk is 0
 * A key that no query row sees (causal, j >= Nq) gets dk = dv = 0; with
 * Nk = 0, dq = 0; with Nq = 0, dk = dv = 0.  Pointers of tensors with no
 * elements may be NULL.  B, H, Nq or Nk negative, or B*H*max(Nq,Nk)*d past
 * the addressable range: FA_ERR_SHAPE.  d outside {64, 128}: FA_ERR_HEADDIM.
 * Same kernels, stream behaviour and determinism as fa_bwd (which is this
 * call with Nq = Nk).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
              const void* dout, float* dq, float* dk, float* dv, void* workspace,
              int B, int H, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd on strided Q, K, V: the backward of fa_fwd_strided with Nq = Nk = N
 * and dv = d (for example Q, K, V as slices of one packed QKV projection;
 * "Build it" takes any tensor).  Same arguments, results, stream behaviour
 * and errors as fa_bwd, plus
 *   q_strides, k_strides, v_strides : host arrays of 3 element strides
 *     (batch, head, row) of Q, K, V; the head-dim stride is 1.
 * Each stride must be >= 0 and a multiple of 8, a row stride at least d and
 * below 2^31, one head's rows byte-addressable in 31 bits, q, k, v 16-byte
 * aligned, and K and V must share their row stride; otherwise FA_ERR_SHAPE
 * (NULL stride arrays: FA_ERR_NULL).  dout, o, lse and dq, dk, dv are dense
 * [B,H,N,d] (lse [B,H,N]); the gradients are those of the viewed tensors.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const float* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv, void* workspace,
                   int B, int H, int N, int d, const int64_t* q_strides, const int64_t* k_strides,
                   const int64_t* v_strides, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layouts, results and
 * errors as fa_bwd, minus `workspace`: the two float32 per query row that
 * fa_bwd keeps in the caller's workspace live in a 16 MiB array inside the
 * library instead, one copy per GPU, held until the process ends.  The call
 * allocates and frees nothing.
 *   Limit: B*H*N <= 2^21 query rows, otherwise FA_ERR_SCRATCH (nothing is
 *   launched).  The array of the current device (hipGetDevice) is used:
 *   `stream` must belong to that device.
 *   Every call on one GPU shares that array and it keeps the last call's
 *   contents (each call writes every row it reads first, so nothing needs
 *   clearing): calls that overlap in time on one GPU -- on different streams,
 *   or from several host threads -- race and give undefined results; order
 *   them on one stream or synchronise between them.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const float* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Attention dropout whose mask the backward regenerates from the generator
 * state instead of storing it ("Backward can recreate tiles instead of
 * retaining the square", Why FlashAttention Can Avoid a Square Attention
 * Array Without Making Attention Linear).  Same arguments, layouts,
 * ownership and errors as fa_fwd / fa_bwd, plus:
 *   p_drop : dropout probability, 0 <= p_drop < 1, else FA_ERR_DROPOUT
 *   seed   : 64-bit generator key;  offset : 32-bit stream selector
 * Mask: for head bh = b*H + h, query row i, key j, the Philox4x32-10
 * generator (Salmon et al., SC 2011) with counter (j/4, i/4, bh, offset)
 * and key (seed mod 2^32, seed / 2^32) gives four words; the pair is kept
 * iff byte (j mod 4) of word (i mod 4) is >= t = min(255, round(256 p_drop)),
 * and kept weights are multiplied by 256 / (256 - t).  The softmax
 * normaliser and lse cover every weight (dropout acts on the normalised
 * probabilities): O = (P * keep * 256/(256-t)) V.  fa_bwd_dropout with the
 * same p_drop, seed and offset gives the gradients of that O; the workspace
 * is fa_bwd_workspace_bytes.  p_drop = 0 runs the plain kernels.
 */
/* The dropout probability the two calls above apply for p_drop: the
 * generator bytes are compared with t = min(255, round(256 p_drop)), so the
 * applied probability is t / 256 (p_drop = 0.1 applies 26/256 = 0.1015625).
 * Returns -1 for a p_drop outside [0, 1). */
float fa_dropout_applied_p(float p_drop);
int fa_fwd_dropout(const void* q, const void* k, const void* v, float* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const float* o, const float* lse,
                   const void* dout, float* dq, float* dk, float* dv, void* workspace,
                   int B, int H, int N, int d, float scale, int causal,
                   float p_drop, uint64_t seed, uint32_t offset, hipStream_t stream);

/*
 * Packed variable-length sequences: instead of padding every sequence to the
 * longest one, sequences share one token axis (the padding note among the
 * tips on PyTorch calls under "What it doesn't solve", FlashAttention: The
 * Matrix You Never Have to Write Down: padded positions cost work).
 *   q, k, v    : device, bf16 [H, total, d] head-major; sequence b occupies
 *                rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head
 *   o          : device, float32 [H, total, d];  lse : float32 [H, total]
 *   cu_seqlens : device, int32 [B+1], non-decreasing, cu[0] = 0, cu[B] = total
 *   max_seqlen : host bound on the longest sequence (sizes the launch; rows of
 *                a longer sequence beyond it are left unwritten); <= total
 * Each row attends to the keys of its own sequence; causal masking is
 * upper-left within the sequence; a sequence of length 0 has no rows.
 * Offsets that break the rules give unspecified values for the rows
 * involved, never a memory access outside the tensors (the kernels clamp
 * them into [0, total]).  fa_bwd_varlen returns the gradients in the same
 * layout; its workspace is fa_bwd_workspace_bytes(1, H, total, d).  Errors
 * as fa_fwd / fa_bwd (negative sizes or max_seqlen > total: FA_ERR_SHAPE;
 * NULL cu_seqlens: FA_ERR_NULL).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                  const int* cu_seqlens, int B, int H, int total, int max_seqlen, int d,
                  float scale, int causal, hipStream_t stream);
int fa_bwd_varlen(const void* q, const void* k, const void* v, const float* o, const float* lse,
                  const void* dout, float* dq, float* dk, float* dv, void* workspace,
                  const int* cu_seqlens, int B, int H, int total, int max_seqlen, int d,
                  float scale, int causal, hipStream_t stream);

/*
 * The backward in three phases, for callers that schedule or time them
 * separately (same arguments, layouts and errors as fa_bwd; workspace as
 * sized by fa_bwd_workspace_bytes).  On one stream
 *   fa_bwd_prep(...); fa_bwd_dkdv(...); fa_bwd_dq(...);
 * gives bitwise the results of fa_bwd, which runs the preprocess inside its
 * dQ pass (same summation order) and the dK/dV pass after it.
 *
 * fa_bwd_prep: per query row, scale * (dO_i . O_i) and L_i log2(e) into the
 *   workspace.  Reads dout, o, lse.
 * fa_bwd_dkdv: dK and dV, one pass per block of 128 keys over the query
 *   rows (causal: from the block's diagonal on).  Reads q, k, v, dout and
 *   the prepared workspace.
 * fa_bwd_dq: dQ, one pass per block of 128 query rows over the key tiles it
 *   sees, recomputing the probability tiles.  Reads q, k, v, dout and the
 *   prepared workspace.
 */
int fa_bwd_prep(const void* dout, const float* o, const float* lse, void* workspace,
                int B, int H, int N, int d, float scale, hipStream_t stream);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const void* workspace,
                float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                hipStream_t stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const void* workspace,
              float* dq, int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Static, human-readable text for an fa_status value (never NULL).
 * Infrastructure (error reporting): no passage of the pages defines it. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */

/*
 * fa.h -- C ABI of libfa.so: exact tiled scaled-dot-product attention on AMD
 * MI355X (gfx950), forward and backward, as hand-written HIP kernels.
 *
 * What is computed ("FlashAttention and online softmax", ML Systems Lesson 4):
 *   forward  -- section "The GPU picture: keep the tile on chip" and the tiled
 *               forward pass of "The online softmax theorem":
 *               O = softmax(scale * Q K^T [causal]) V, row by row, and per row
 *               lse_i = log sum_j exp(scale * q_i . k_j) over the visible keys
 *               (natural log, the scale included).  The N x N score matrix is
 *               never written to memory.
 *   causal   -- section "Causal masks and FlashAttention-3": query i sees key j
 *               iff j <= i; tiles wholly above the diagonal are skipped.
 *   backward -- section "Backward pass: recompute instead of store": the score
 *               tiles are recomputed from Q, K and lse (P = exp(S - lse)), then
 *               dV = P^T dO, dP = dO V^T, dS = P o (dP - D) with
 *               D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q.
 *               dQ, dK, dV are the gradients of sum(dO o O).
 *
 * Layout.  Every [B, H, N, d] tensor is dense and contiguous in that order
 * (row n of head (b, h) starts at element ((b * H + h) * N + n) * d).  lse is
 * [B, H, N] float32.  Element type: bf16 (FA_DTYPE_BF16, arithmetic in fp32 with
 * bf16 operands for the matrix products) or float32 (FA_DTYPE_FP32).
 *
 * Ownership.  All pointers are device memory owned by the caller.  The library
 * never allocates, frees or synchronises: work is enqueued on `stream` (a
 * hipStream_t; NULL = the legacy default stream) and the call returns at once.
 * Inputs are read only; outputs are fully overwritten (never accumulated into);
 * outputs must not alias inputs or each other.  The backward workspace is
 * scratch owned by the caller, at least fa_bwd_workspace_bytes() bytes; its
 * contents on entry do not matter and are undefined on exit.  Calls are
 * reentrant; calls on different streams that share no output run independently.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 * failed check launches nothing and returns:
 *   FA_ERR_INVALID_ARG  -- a null pointer, B, H or N < 1, B*H*N >= 2^31, a
 *                          tensor pointer not 16-byte aligned (lse: 4-byte),
 *                          softmax_scale not finite and > 0, causal not 0 or 1,
 *                          or a workspace shorter than fa_bwd_workspace_bytes();
 *   FA_ERR_UNSUPPORTED  -- d not 64 or 128, or an unknown dtype;
 *   FA_ERR_LAUNCH       -- the HIP runtime rejected a kernel launch (an error
 *                          that earlier, unrelated HIP calls left pending on the
 *                          calling thread is cleared first and never reported).
 * There is no fallback path of any kind: an unsupported request fails loudly
 * ("FlashAttention from Scratch", section "Pitfalls that turn into incidents").
 *
 * Numerics.  bf16: forward and backward are bitwise deterministic for given
 * inputs.  fp32: the backward accumulates dQ with float32 atomics, so dQ may
 * differ in the last bits from run to run.  Results agree with the exact ones up
 * to rounding, not bitwise ("FlashAttention from Scratch", "Bitwise mismatch is
 * not a bug").
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_LAUNCH = 3,
  FA_ERR_TOO_LARGE = 4 /* fa_bwd_noalloc only: the call does not fit its fixed scratch */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP32 = 1 } fa_dtype;

/* Forward pass.
 *   q, k, v : [B, H, N, d] inputs of `dtype`.
 *   o       : [B, H, N, d] output of `dtype`.
 *   lse     : [B, H, N] float32 output (natural-log logsumexp of the scaled,
 *             masked score row).
 *   softmax_scale : the factor tau in S = tau Q K^T (1/sqrt(d) for standard
 *             attention); must be finite and > 0.
 *   causal  : 1 = query i sees keys j <= i; 0 = every key.
 *   stream  : hipStream_t to enqueue on.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float softmax_scale, int causal,
                 int dtype, void* stream);

/* Bytes of device workspace fa_bwd needs: two float32 vectors of B*H*Npad values
 * (Npad = N rounded up to a multiple of 32: D_i and lse_i * log2(e)), for
 * FA_DTYPE_FP32 also a float32 dQ accumulator of [B, H, Npad, d], then an int32 block
 * plan of 16 + B*H*ceil(N/128) values (used by the variable-length and windowed bf16
 * calls of fa_bwd_ex); each region 256-byte aligned.  0 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/* Backward pass.
 *   q, k, v, o, dout : [B, H, N, d] of `dtype` (o is the forward output and dout
 *             the gradient of the loss with respect to it).
 *   lse     : [B, H, N] float32 from fa_fwd on the same q, k, v, scale, causal.
 *   dq, dk, dv : [B, H, N, d] outputs of `dtype`.
 *   workspace, workspace_bytes : caller-owned scratch (see above).
 *   Other arguments as for fa_fwd. */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                 float softmax_scale, int causal, int dtype, void* stream);

/* The three stages of the backward, to be run in this order on one stream; a caller
 * may run them separately (e.g. to time or overlap them).  Same argument rules and codes as
 * fa_bwd for the pointers each stage takes.
 *   fa_bwd_preprocess : D_i = dO_i . O_i (the row term of dS = P o (dP - D),
 *                       "Backward pass: recompute instead of store", step 3) and
 *                       lse_i in base 2 into the workspace (for FA_DTYPE_FP32 it also
 *                       clears the workspace's dQ accumulator).
 *   fa_bwd_main       : dK and dV.  Per block of keys, recomputes S and
 *                       P = exp(S - lse) for every visible query tile and
 *                       accumulates dV += P^T dO and dK += scale dS^T Q on chip
 *                       (steps 1-4 of the same passage).  For FA_DTYPE_FP32 it also
 *                       adds the unscaled dS K contributions to the accumulator.
 *   fa_bwd_dq         : dQ.  FA_DTYPE_BF16: per block of query rows, recomputes S,
 *                       P, dP and dS for every visible key tile and accumulates
 *                       dQ = scale dS K on chip (no atomics).  FA_DTYPE_FP32:
 *                       dQ = scale * accumulator.
 * fa_bwd_main and fa_bwd_dq read the workspace written by fa_bwd_preprocess.
 *
 * For FA_DTYPE_BF16, fa_bwd itself runs two launches: fa_bwd_dq_pre (below), then
 * fa_bwd_main.  The results equal those of the three stages bit for bit. */
fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            void* workspace, size_t workspace_bytes, int B, int H,
                            int N, int d, int dtype, void* stream);
fa_status fa_bwd_main(const void* q, const void* k, const void* v, const void* dout,
                      void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d, float softmax_scale, int causal,
                      int dtype, void* stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                    void* dq, void* workspace, size_t workspace_bytes, int B, int H,
                    int N, int d, float softmax_scale, int causal, int dtype,
                    void* stream);
/* fa_bwd_preprocess and fa_bwd_dq in one pass (FA_DTYPE_BF16 only; FA_ERR_UNSUPPORTED
 * for FA_DTYPE_FP32, whose dQ comes from fa_bwd_main's accumulator): each query row's
 * D_i = dO_i . O_i and lse_i * log2(e) are formed where the dQ pass loads that row,
 * used there, and written to the workspace for fa_bwd_main to run next.  Arguments as
 * fa_bwd's (o and lse read, dq written). */
fa_status fa_bwd_dq_pre(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* workspace,
                        size_t workspace_bytes, int B, int H, int N, int d,
                        float softmax_scale, int causal, int dtype, void* stream);

/* ---- Variable-length batches and sliding windows ---------------------------------
 * fa_fwd_ex / fa_bwd_ex take the arguments of fa_fwd / fa_bwd plus:
 *   cu_seqlens : NULL for dense [B, H, N, d] tensors (then `total` is ignored and
 *       the calls equal fa_fwd / fa_bwd with the window below).  Otherwise B+1 int32
 *       values in device memory, 0 = cu[0] <= cu[1] <= ... <= cu[B] = total: a batch
 *       of B sequences of lengths cu[b+1] - cu[b] (zero allowed) packed without
 *       padding ("FlashAttention from Scratch", "Pitfalls that turn into incidents":
 *       pass cu_seqlens instead of padded batches).  Tensors are then packed
 *       head-major, [H, total, d] (sequence b of head h in rows cu[b] .. cu[b+1]-1),
 *       lse is [H, total] float32, N is the longest length (max_seqlen) and every
 *       sequence attends only within itself.  The table is the caller's contract: the
 *       kernels read it on the device and this call cannot check it without a
 *       device-to-host copy.  A table outside these rules (including a length above N)
 *       gives wrong rows without an error, though never an access outside the
 *       tensors; the Python binding checks the table on a host copy before the call.
 *   window : 0 = no window.  W >= 1 (requires causal = 1): a causal band, query i
 *       sees key j iff i - W < j <= i ("FlashAttention and online softmax", "Where it
 *       shows up": sliding-window masks with tile skipping); tiles outside the band
 *       are skipped.
 * fa_bwd_ex's workspace: fa_bwd_workspace_bytes(B, H, N, d, dtype), N = max_seqlen.
 * Errors: as fa_fwd / fa_bwd, plus FA_ERR_INVALID_ARG for window < 0, window > 0
 * with causal = 0, a misaligned cu_seqlens, total < 1 or H * total >= 2^31. */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int B, int H, int N, int total, int d,
                    float softmax_scale, int causal, int window, int dtype, void* stream);
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, const int* cu_seqlens, int B,
                    int H, int N, int total, int d, float softmax_scale, int causal,
                    int window, int dtype, void* stream);

/* fa_bwd_ex's kernel launches one at a time (for timing them apart, or overlapping
 * them with other work): `launches` is a mask of the launches to enqueue, in fa_bwd's
 * order -- bf16: bit 0 fa_bwd_dq_pre's pass (dQ, and D and lse*log2(e) into the
 * workspace), bit 1 the dK/dV pass; fp32: bit 0 preprocess, bit 1 dK/dV pass (which
 * adds to the dQ accumulator), bit 2 dQ conversion.  Running the bits of
 * FA_BWD_ALL_LAUNCHES in increasing order on one stream equals fa_bwd_ex.  Other
 * arguments and errors as fa_bwd_ex; FA_ERR_INVALID_ARG for a mask outside 1..7. */
#define FA_BWD_ALL_LAUNCHES 7
fa_status fa_bwd_ex_launches(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, const int* cu_seqlens,
                             int B, int H, int N, int total, int d, float softmax_scale,
                             int causal, int window, int dtype, int launches, void* stream);

/* ---- Split-KV decoding ----------------------------------------------------------
 * "FlashAttention and online softmax" (Lesson 4), section "Split-KV for decoding
 * (flash-decoding)": the keys of each row are cut into chunks, each chunk is
 * reduced to a partial (o, lse) by workgroups of its own, and a second pass merges
 * the partials of each row with the formula of section "Merging two partial
 * results": lse = log sum_s e^{lse_s}, o = sum_s e^{lse_s - lse} o_s (an empty
 * chunk has lse_s = -inf and weight 0).
 *
 * A block of Nq query rows per (b, h) -- the newest Nq positions of a sequence whose
 * key/value cache holds Nk rows -- attends to that cache.
 *   q : [B, H, Nq, d]; k, v : [B, H, Nk, d]; o : [B, H, Nq, d], all of `dtype`;
 *   lse : [B, H, Nq] float32.  1 <= Nq <= 8, Nq <= Nk; d 64 or 128.
 *   causal : 1 = query i (0-based among the Nq) sees key j iff j <= i + (Nk - Nq)
 *            (for Nq = Nk the rule of fa_fwd; one decoding query sees every key);
 *            0 = every key.
 *   num_splits : 1..256 chunks.  With c = ceil(Nk / num_splits), chunk s holds keys
 *            [s c, min(Nk, (s+1) c)); chunks that start at or past Nk are empty.
 * Errors: as fa_fwd, plus FA_ERR_INVALID_ARG for Nk < Nq or num_splits < 1 and
 * FA_ERR_UNSUPPORTED for Nq > 8 (use fa_fwd for many query rows) or
 * num_splits > 256. */

/* Bytes of workspace fa_fwd_splitkv needs: the float32 partials
 * o_part [num_splits, B, H, Nq, d] and lse_part [num_splits, B, H, Nq], each region
 * 256-byte aligned.  0 for invalid sizes. */
size_t fa_splitkv_workspace_bytes(int B, int H, int Nq, int d, int num_splits);

/* Both passes (fa_fwd_partial into the workspace, then fa_merge) on one stream. */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Nq, int Nk, int d, float softmax_scale,
                         int causal, int num_splits, void* workspace,
                         size_t workspace_bytes, int dtype, void* stream);

/* First pass: for every chunk s, the attention of each query row over that chunk's
 * visible keys alone, normalised: o_part[s] (float32, [B, H, Nq, d]) and
 * lse_part[s] (float32, [B, H, Nq]); a row with no visible key in the chunk gets
 * o = 0, lse = -inf.  o_part 16-byte aligned, lse_part 4-byte aligned. */
fa_status fa_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                         float* lse_part, int B, int H, int Nq, int Nk, int d,
                         float softmax_scale, int causal, int num_splits, int dtype,
                         void* stream);

/* Second pass: merges num_splits partials of `rows` rows of length d
 * (o_part [num_splits, rows, d] float32, lse_part [num_splits, rows] float32) into
 * o [rows, d] of `dtype` and lse [rows] float32.  Any order of the chunks gives the
 * same result up to rounding.  1 <= d <= 1024, 1 <= num_splits <= 256; rows with
 * every lse_s = -inf get o = 0, lse = -inf.  Pointers need only their element
 * alignment; INVALID_ARG for null pointers or sizes out of range. */
fa_status fa_merge(const float* o_part, const float* lse_part, void* o, float* lse,
                   int num_splits, int rows, int d, int dtype, void* stream);

/* ---- Backward without a workspace argument -------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fa_bwd with the same arguments
 * except the workspace, which here is a fixed array of FA_NOALLOC_SCRATCH_BYTES inside
 * the library.  Each GPU the library runs on holds one such array from module load
 * until the process ends; its address is looked up once per device, on the first
 * call there.  The call allocates and frees nothing.
 *   - It fits iff fa_bwd_workspace_bytes(B, H, N, d, dtype) <= FA_NOALLOC_SCRATCH_BYTES
 *     (about 8 + 1/32 bytes per padded row for bf16, 8 + 4d + 1/32 for fp32, so bf16
 *     fits up to about 4.1M rows B*H*ceil32(N)); a larger call returns
 *     FA_ERR_TOO_LARGE before anything is enqueued.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in time on one
 *     GPU (different streams, threads or processes' shared contexts) race and give
 *     undefined results; serialise them, e.g. on one stream.  Nothing a previous call
 *     left in the array is read (the preprocess rewrites all of it that is used).
 *   - `stream` must belong to the current device.
 * Results equal fa_bwd's on the same inputs (bitwise for bf16).  Other errors as
 * fa_bwd; FA_ERR_LAUNCH also if the scratch address cannot be obtained. */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, float softmax_scale, int causal,
                         int dtype, void* stream);

/* Host-only argument checks of fa_fwd / fa_bwd (same rules, same codes); they
 * touch no device and enqueue nothing.  Pointers are checked for null and
 * alignment only. */
fa_status fa_fwd_check(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int B, int H, int N, int d,
                       float softmax_scale, int causal, int dtype);
fa_status fa_bwd_check(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, const void* dq,
                       const void* dk, const void* dv, const void* workspace,
                       size_t workspace_bytes, int B, int H, int N, int d,
                       float softmax_scale, int causal, int dtype);

/* Static text for a status code ("unknown status" for other values). */
const char* fa_status_string(int status);

/* ABI version of this header: (major << 16) | minor. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

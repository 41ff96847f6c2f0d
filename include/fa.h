/*
 * fa.h -- exact tiled attention forward pass (FlashAttention-style) for AMD MI355X (gfx950).
 *
 * The operation. For every batch b and head h independently, with Q, K, V the [N, d] slices:
 *
 *     S   = scale * Q K^T                      (a score per query i and key j)
 *     S[i][j] = -inf for j > i   when causal   (a query sees itself and earlier keys only)
 *     O   = softmax_rows(S) V                  (stable softmax: exponentials taken relative
 *                                               to the row maximum m, normalised by their sum l)
 *     LSE = m + ln(l)                          (one float per query row)
 *
 * This is ordinary scaled dot-product attention ("Understanding FlashAttention Pt 1", §0.2 and
 * §1.2; "Online Softmax & FlashAttention", Eq 26.1 and Listing 26.2). The library computes it
 * tile by tile with a running maximum, a running sum and an unnormalised accumulator that is
 * rescaled whenever the reference maximum moves, divides by the sum once after the last key
 * tile, and writes the logsumexp per row ("FlashAttention-2 -- Deeper Math", Fixes 1-5 and
 * "Causal masking: skip the blocks"). The N x N matrices S and P are never written to memory.
 * The result is exact up to floating-point rounding order; it is not an approximation.
 *
 * Conventions shared by every entry point:
 *   - q, k, v, o, lse are DEVICE pointers owned by the caller. The library never allocates,
 *     frees, copies or synchronises; it only enqueues kernels on `stream`.
 *   - Layout: contiguous row-major [B][H][N][d] for q, k, v and o; contiguous [B][H][N] for lse.
 *     Self-attention only: queries and keys have the same length N, and V has head dim d.
 *   - scale multiplies q.k in fp32 before the softmax (pass 1/sqrt(d) for the usual attention).
 *     It must be finite and >= 0.
 *   - causal is 0 (every query sees every key) or 1 (query i sees keys 0..i).
 *   - lse holds ln(sum_j exp(S[i][j] - m_i)) + m_i of the scaled scores, in natural-log units.
 *   - o must not overlap q, k, v or lse; lse must not overlap q, k, v or o.
 *   - stream is a hipStream_t (NULL = the default stream). The call is asynchronous: errors in
 *     argument checking are returned before any HIP call is made; a launch failure is reported
 *     as FA_ERR_LAUNCH (the launch call's own status).
 *   - Deterministic: the same inputs give bitwise-identical outputs run to run (no atomics, no
 *     cross-workgroup reductions).
 *   - Thread-safe: no global mutable state (the one exception, the per-device scratch of
 *     fa_fwd_splitkv_noalloc, is described with that function).
 *   - Limits: 1 <= N <= 2^22 and 1 <= B*H <= 65535.
 *
 * Grouped K/V heads ("Understanding FlashAttention Pt 1", §4.1): fa_fwd_gqa and fa_fwd_gqa_f32
 * take H query heads and H_kv key/value heads with H a multiple of H_kv. Query head h attends with
 * K/V head h / (H / H_kv), so consecutive groups of H / H_kv query heads share one K/V head:
 * H_kv = H is ordinary multi-head attention, H_kv = 1 is multi-query attention. They also take a
 * layout for q, k, v and o (lse stays [B][H][N]):
 *   FA_LAYOUT_BHND  q, o [B][H][N][d]     k, v [B][H_kv][N][d]   (the layout of fa_fwd)
 *   FA_LAYOUT_BNHD  q, o [B][N][H][d]     k, v [B][N][H_kv][d]   (tokens outermost, as in §4.1)
 * Each layout is contiguous row-major; every other convention above applies unchanged.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1) /* null pointer, B/H/N out of range, causal not 0/1, scale
                                   negative or not finite, or overlapping output buffers */
#define FA_ERR_UNSUPPORTED (-2) /* head dim d not in {64, 128} (the bf16 forward entry points
                                   fa_fwd, fa_fwd_gqa and fa_fwd_ext also take 256); split-KV:
                                   over 512 rows per K/V head */
#define FA_ERR_ALIGNMENT (-3)   /* a pointer is not 16-byte aligned */
#define FA_ERR_LAUNCH (-4)      /* the kernel launch call (or a HIP runtime query) returned an
                                   error */
#define FA_ERR_TOO_LARGE (-5)   /* fa_fwd_splitkv_noalloc: the shape needs more than the static
                                   scratch holds (FA_NOALLOC_SCRATCH_BYTES) */

/* Bytes of device scratch the library holds per GPU for fa_fwd_splitkv_noalloc (16 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES 16777216

#define FA_LAYOUT_BHND 0 /* [B][heads][N][d] */
#define FA_LAYOUT_BNHD 1 /* [B][N][heads][d] */

/*
 * fa_fwd -- bf16 inputs and outputs, fp32 arithmetic for the softmax and both accumulations.
 *   q, k, v : const bf16 (bfloat16, 2 bytes) [B][H][N][d]
 *   o       : bf16 [B][H][N][d], written (rounded to nearest even from fp32)
 *   lse     : float [B][H][N], written
 * The two contractions Q K^T and P V run on bf16 matrix cores with fp32 accumulation; P is
 * rounded to bf16 (nearest even) before P V, and the row sum l is taken from the fp32 P.
 * Returns FA_OK or one of the FA_ERR_* codes above.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_f32 -- fp32 inputs and outputs; every step in fp32 (no bf16 or reduced-precision
 * matrix arithmetic anywhere). Same layout, conventions and return codes as fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_gqa -- fa_fwd with H_kv key/value heads (H a multiple of H_kv) and a layout
 * (FA_LAYOUT_BHND or FA_LAYOUT_BNHD) for q, k, v, o. k and v hold B*H_kv*N*d elements, q and o
 * B*H*N*d, lse B*H*N floats. H_kv < 1, H not a multiple of H_kv or an unknown layout return
 * FA_ERR_INVALID_ARG. fa_fwd(q,k,v,o,lse,B,H,N,d,s,c,st) is fa_fwd_gqa(..., B, H, H, N, d, s, c,
 * FA_LAYOUT_BHND, st).
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int H_kv, int N, int d, float scale, int causal, int layout,
               void* stream);

/* fa_fwd_gqa_f32 -- the fp32 counterpart of fa_fwd_gqa (as fa_fwd_f32 is of fa_fwd). */
int fa_fwd_gqa_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal, int layout,
                   void* stream);

/*
 * Score variants ("Understanding FlashAttention Pt 1": S = QK^T / sqrt(d) + B with B an optional
 * additive mask or bias, §0.2; local/sliding-window attention and ALiBi-style bias, §3.5 and §4.2)
 * and head dim 256 ("Flash Attention": supported head dims 64, 128, 256). fa_fwd_ext is fa_fwd_gqa
 * (same layouts, head grouping, outputs and codes) with, for query row i and key j of one head:
 *   window_left, window_right: key j is visible iff i - window_left <= j <= i + window_right;
 *       -1 leaves that side unbounded (both -1: no window); the causal rule still applies when
 *       causal = 1. Tiles outside the window are skipped.
 *   alibi_slopes: NULL or device fp32[H], slope m_h of query head h: the score gets - m_h |i - j|.
 *   bias: NULL or device bf16 matrix per (batch, query head): the score gets bias[b][h][i][j] at
 *       element offset b * bias_batch_stride + h * bias_head_stride + i * bias_row_stride + j;
 *       a stride of 0 shares the matrix across batches or heads; bias_row_stride >= N, all three
 *       strides multiples of 8 and the pointer 16-byte aligned, so that every row starts 16-byte
 *       aligned (else FA_ERR_INVALID_ARG / FA_ERR_ALIGNMENT);
 *       one head's matrix must span under 2 GiB (else FA_ERR_UNSUPPORTED). -inf entries mask.
 * The bias and ALiBi terms are added to the scaled score: S_ij = scale q_i.k_j + B_ij - m_h|i-j|.
 * A row with no visible key (only possible through -inf bias entries) gets O = 0 and
 * LSE = -inf. d in {64, 128, 256}; bf16 only. fa_fwd and fa_fwd_gqa also accept d = 256 (bf16).
 */
int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int H_kv, int N, int d, float scale, int causal, int layout, int window_left,
               int window_right, const float* alibi_slopes, const void* bias,
               long long bias_batch_stride, long long bias_head_stride, long long bias_row_stride,
               void* stream);

/*
 * Split-KV decoding ("FlashAttention-2 -- Deeper Math", "What FA-2 does not fix": few queries
 * against a long K/V sequence are bound by reading K and V, so the keys are split across the GPU
 * and the partial softmaxes merged with the blockwise recurrence of "Understanding FlashAttention
 * Pt 1", §2.4). Shapes: q and o hold N_q query rows per head, k and v N_kv key rows per K/V head,
 * in the given layout (FA_LAYOUT_BHND: q, o [B][H][N_q][d], k, v [B][H_kv][N_kv][d];
 * FA_LAYOUT_BNHD: q, o [B][N_q][H][d], k, v [B][N_kv][H_kv][d]); lse [B][H][N_q]. Query head h uses
 * K/V head h / (H / H_kv), as in fa_fwd_gqa. Query i is token N_kv - N_q + i of the sequence: with
 * causal = 1 it sees keys j <= N_kv - N_q + i (then N_q <= N_kv is required), with causal = 0
 * every key. The result is the same function fa_fwd_gqa computes for those masks; only the order
 * of the floating-point operations differs.
 *
 * fa_splitkv_workspace_bytes -- bytes of device workspace fa_fwd_splitkv needs for this shape and
 *   split count (n_splits = 0: the library's choice, about 768 waves of one (batch, K/V head,
 *   split, 32-row tile) each, at least 128 keys per split; a given count is capped at one split
 *   per 32 keys).
 *   Returns 0 when the shape is not accepted by fa_fwd_splitkv.
 * fa_fwd_splitkv -- bf16 q, k, v, o; fp32 arithmetic; fp32 partial results of every split in
 *   `workspace` (caller-owned device memory of at least fa_splitkv_workspace_bytes(...) bytes,
 *   16-byte aligned, overlapping nothing else; its contents on entry do not matter and are
 *   overwritten). Two kernels are enqueued on `stream`; calls that share a workspace must not
 *   overlap. Limits: N_kv <= 2^22, (H / H_kv) * N_q <= 512 (the query rows that share one K/V
 *   head, stacked and cut into 32-row tiles; more return FA_ERR_UNSUPPORTED), d in {64, 128}.
 *   Other conventions and return codes as fa_fwd_gqa; a workspace that is NULL or too small
 *   returns FA_ERR_INVALID_ARG.
 */
size_t fa_splitkv_workspace_bytes(int B, int H, int H_kv, int N_q, int N_kv, int d, int causal,
                                  int n_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N_q, int N_kv, int d, float scale, int causal,
                   int layout, int n_splits, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate device memory (code
 *   under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 *   kernels, split plan, arguments (minus the workspace), result and return codes, with the split
 *   partials kept in a scratch array that the library holds in device memory, FA_NOALLOC_SCRATCH_BYTES
 *   per GPU for as long as the process lives. It calls no allocator. A shape whose partials
 *   (fa_splitkv_workspace_bytes(...) bytes) exceed the scratch returns FA_ERR_TOO_LARGE before any
 *   HIP call. The first call on a device looks the scratch's address up on that device (the
 *   current one, which `stream`, if not NULL, must belong to: else FA_ERR_INVALID_ARG). Every call
 *   on one GPU shares that GPU's scratch: calls that may overlap in time on one GPU (two streams,
 *   two host threads) race and must be serialised by the caller. The scratch needs no clearing:
 *   every partial a call reads was written by the same call.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int H_kv, int N_q, int N_kv, int d, float scale,
                           int causal, int layout, int n_splits, void* stream);

/*
 * Backward pass by recomputation ("Understanding FlashAttention Pt 1", §3.6; "Online Softmax &
 * FlashAttention", §26.4; the logsumexp form of the probabilities from "FlashAttention-2 -- Deeper
 * Math", Fix 2). Given the forward's inputs q, k, v, its output o and logsumexp lse (as written by
 * fa_fwd / fa_fwd_gqa for the same scale, mask and layout) and the upstream gradient dout = dL/dO,
 * writes the gradients of L:
 *     P = exp(scale q k^T - lse) (masked entries 0),   dV = P^T dout,   dP = dout v^T,
 *     D = rowsum(dout * o),   dS = P * (dP - D),   dQ = scale dS k,   dK = scale dS^T q.
 * With grouped K/V heads (H_kv < H) a K/V head's dk and dv are the sums over the query heads
 * that use it (query head h uses K/V head h / (H / H_kv)).
 *
 * fa_bwd_workspace_bytes -- bytes of device workspace fa_bwd needs: B * H * N floats (D), and,
 *   when the query heads of a K/V head are split over several workgroups to fill the GPU (grouped
 *   heads with few K/V heads), fp32 partial dK and dV of every split. Returns 0 for an invalid
 *   shape.
 * fa_bwd -- bf16 q, k, v, o, dout, dq, dk, dv in `layout` (q, o, dout, dq: H heads; k, v, dk, dv:
 *   H_kv heads; shapes as fa_fwd_gqa); fp32 lse [B][H][N]; fp32 arithmetic with the probabilities
 *   and dS rounded to bf16 as matrix-core operands. `workspace`: caller-owned device memory of at
 *   least fa_bwd_workspace_bytes(B, H, N) bytes, contents on entry irrelevant. Outputs must not
 *   overlap any input, each other or the workspace; all pointers 16-byte aligned. Two or three
 *   kernels are enqueued on `stream`; calls that share a workspace must not overlap. The result is
 *   deterministic (no atomics). Limits and return codes as fa_fwd_gqa (d in {64, 128}).
 */
size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d);
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
           float scale, int causal, int layout, void* workspace, size_t workspace_bytes,
           void* stream);

/* Human-readable text for a return code (static storage; never NULL). */
const char* fa_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

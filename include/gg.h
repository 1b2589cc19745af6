/*
 * gg.h -- C ABI of the grouped (ragged, per-expert) GEMM for MI355X
 * (gfx950): the bf16 passes below, then their scaled and accumulating
 * forms, the masked backward, the SiLU-mul gate/up forward, the grouped
 * bias and its backward, the [E, N, K] weight layout, the steps that
 * produce the grouped layout (offsets, routing, gather, combine), and the
 * fp8 block-scaled forward.
 *
 * The operation (PyTorch issue #152668, "Easy repro scenario", and its
 * backward): a 2-D activation X[M,K], a packed 3-D weight W[E,K,N] and int32
 * cumulative END offsets offs[E].  Expert g owns rows [end(g-1), end(g)) of
 * X, with end(-1) = 0, and
 *
 *   forward  Y[i, :]  = X[i, :] . W[g]            for each row i of expert g
 *   dgrad    dX[i, :] = dY[i, :] . W[g]^T          (the input gradient)
 *   wgrad    dW[g]    = X[rows of g]^T . dY[rows of g]   (the weight gradient)
 *
 * The masked variant (sglang PR #32385, "Evidence": A[E, max_m, K], a
 * per-expert active count masked_m[E], output D[E, max_m, N]) computes
 * D[e, r, :] = A[e, r, :] . W[e] for r < masked_m[e].
 *
 * Common contract of every entry point
 * ------------------------------------
 *  - Tensors are bf16 (uint16 storage), row-major and densely packed, in
 *    device memory the CALLER owns.  The library allocates nothing, frees
 *    nothing, needs no workspace, never copies device -> host and never
 *    synchronises: it validates the arguments on the host, then enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *    returns.  Group sizes stay on the device (TransformerEngine PR #3542,
 *    "Changes": expert counts remain on the GPU), so calls are safe to
 *    capture in a HIP graph.
 *  - offs / masked_m are int32 device arrays of num_groups entries.  The
 *    device clamps them: end(g) = min(max(offs[g], end(g-1)), M) and
 *    active(e) = min(max(masked_m[e], 0), max_m).  Bad values therefore give
 *    empty or shortened experts, never an out-of-range access or a hang.
 *  - Outputs are overwritten (alpha = 1, beta = 0; the *_ex forms below
 *    take other values): an output element is written without being read.  Elements the operation does not define
 *    are left untouched (TransformerEngine PR #3542, "Changes": unused
 *    capacity of caller-owned outputs is preserved; TileOPs issue #1566,
 *    "Summary": no output memset).
 *  - Host-checkable errors return a status before anything is enqueued;
 *    outputs are then untouched.  A failed kernel launch returns
 *    GG_ERR_HIP.  There is no fallback path of any kind.
 *  - Requirements: k % 8 == 0 and n % 8 == 0 (16-byte rows), every pointer
 *    16-byte aligned, 1 <= num_groups <= GG_MAX_GROUPS, m (or max_m) >= 0,
 *    8 <= k, n <= GG_MAX_KN, k * n < 2^31 (each expert's weight matrix
 *    under 4 GiB in bf16), and fewer than 2^31 - 2^16 rows (m, or
 *    num_groups * max_m for the masked layout).  An expert's rows may
 *    span any number of bytes.
 *  - Concurrent calls on different streams that write the same output race;
 *    calls on one stream are ordered.
 */
#ifndef GG_H
#define GG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GG_MAX_GROUPS 2048
#define GG_MAX_KN (1 << 20)   /* largest k and n */

typedef enum {
    GG_OK = 0,
    GG_ERR_NULL_PTR = 1,   /* a required pointer is NULL */
    GG_ERR_BAD_DIM = 2,    /* negative or zero size where not allowed, k or n not a multiple of 8, overflow */
    GG_ERR_ALIGNMENT = 3,  /* a pointer is not 16-byte aligned */
    GG_ERR_BAD_DTYPE = 4,  /* unknown output dtype */
    GG_ERR_LIMIT = 5,      /* num_groups outside [1, GG_MAX_GROUPS] */
    GG_ERR_HIP = 6         /* the HIP runtime reported an error (see gg_last_error) */
} gg_status;

typedef enum {
    GG_BF16 = 0,           /* bf16 output, fp32 result rounded to nearest even */
    GG_F32 = 1             /* fp32 output, the fp32 accumulator as is */
} gg_dtype;

/*
 * gg_forward -- Y = X . W[g] on the rows of each expert.
 *   x    [m, k]     bf16, rows grouped contiguously by expert
 *   w    [E, k, n]  bf16, one packed buffer (E = num_groups)
 *   offs [E]        int32 cumulative end offsets, device memory
 *   y    [m, n]     y_dtype; rows [0, end(E-1)) are written, rows at or
 *                   past end(E-1) are neither read nor written
 * Cited passage: PyTorch issue #152668, "Easy repro scenario" (the forward
 * of the grouped call on x[M,K], w[E,K,N], int32 offsets).
 */
gg_status gg_forward(const void* x, const void* w, const int32_t* offs,
                     void* y, gg_dtype y_dtype, int64_t m, int64_t k,
                     int64_t n, int32_t num_groups, void* stream);

/*
 * gg_dgrad -- dX = dY . W[g]^T on the rows of each expert.
 *   dy   [m, n]     bf16
 *   w    [E, k, n]  bf16
 *   offs [E]        int32 cumulative end offsets, device memory
 *   dx   [m, k]     dx_dtype; rows [0, end(E-1)) are written, the rest
 *                   untouched
 * Cited passage: PyTorch issue #152668, "Easy repro scenario" (the
 * backward through the grouped call), and TransformerEngine PR #3542,
 * "Changes" (the dgrad pass of the grouped GEMM).
 */
gg_status gg_dgrad(const void* dy, const void* w, const int32_t* offs,
                   void* dx, gg_dtype dx_dtype, int64_t m, int64_t k,
                   int64_t n, int32_t num_groups, void* stream);

/*
 * gg_wgrad -- dW[g] = X[rows of g]^T . dY[rows of g] for every expert.
 *   x    [m, k]     bf16
 *   dy   [m, n]     bf16
 *   offs [E]        int32 cumulative end offsets, device memory
 *   dw   [E, k, n]  dw_dtype; ALL of it is written (overwrite, not
 *                   accumulate); an expert with no rows gets +0.0 everywhere
 *   Rows of x and dy at or past end(E-1) are never read.
 * Cited passages: PyTorch issue #152668, "Describe the bug" (an expert with
 * zero tokens must not hang the backward) and TransformerEngine PR #3542,
 * "Changes" / "Validation" (overwrite wgrad; empty experts).
 */
gg_status gg_wgrad(const void* x, const void* dy, const int32_t* offs,
                   void* dw, gg_dtype dw_dtype, int64_t m, int64_t k,
                   int64_t n, int32_t num_groups, void* stream);

/*
 * gg_masked_forward -- Y[e, r, :] = X[e, r, :] . W[e] for r < masked_m[e].
 *   x        [E, max_m, k]  bf16; inactive rows are never read (they may
 *                           hold anything, NaN included)
 *   w        [E, k, n]      bf16
 *   masked_m [E]            int32 active-row counts, device memory
 *   y        [E, max_m, n]  y_dtype; only active rows are written
 * Cited passage: sglang PR #32385, "Evidence" (the masked grouped GEMM over
 * [E, max_m, K] with per-expert masked_m) and "Cause" (consumers must not
 * depend on inactive rows).
 */
gg_status gg_masked_forward(const void* x, const void* w,
                            const int32_t* masked_m, void* y,
                            gg_dtype y_dtype, int64_t max_m, int64_t k,
                            int64_t n, int32_t num_groups, void* stream);

/*
 * gg_masked_dgrad -- dX[e, r, :] = dY[e, r, :] . W[e]^T for r < masked_m[e].
 *   dy       [E, max_m, n]  bf16; inactive rows are never read
 *   w        [E, k, n]      bf16
 *   masked_m [E]            int32 active-row counts, device memory
 *   dx       [E, max_m, k]  dx_dtype; only active rows are written
 * gg_masked_wgrad -- dW[e] = X[e, :a]^T . dY[e, :a] with a = the clamped
 * masked_m[e], for every expert.
 *   x        [E, max_m, k]  bf16; inactive rows are never read
 *   dy       [E, max_m, n]  bf16; inactive rows are never read
 *   dw       [E, k, n]      dw_dtype; ALL of it is written, an expert with
 *                           no active rows gets +0.0 everywhere
 * The backward of gg_masked_forward on the same layout: the masked grouped
 * GEMM (sglang PR #32385, "Evidence") runs on the dispatched activations of
 * an expert-parallel MoE layer, whose training step needs the input and
 * weight gradients over the same active rows; inactive rows stay out of
 * every result ("Cause": consumers must not depend on them).
 */
gg_status gg_masked_dgrad(const void* dy, const void* w,
                          const int32_t* masked_m, void* dx,
                          gg_dtype dx_dtype, int64_t max_m, int64_t k,
                          int64_t n, int32_t num_groups, void* stream);
gg_status gg_masked_wgrad(const void* x, const void* dy,
                          const int32_t* masked_m, void* dw,
                          gg_dtype dw_dtype, int64_t max_m, int64_t k,
                          int64_t n, int32_t num_groups, void* stream);

/*
 * gg_forward_silu_mul -- the gate/up forward with the SiLU-mul activation
 * fused into its epilogue:
 *   out[i, c] = silu(G[i, c]) * U[i, c],  silu(z) = z / (1 + exp(-z)),
 *   G = X[rows of g] . W13[g][:, 0:I],  U = X[rows of g] . W13[g][:, I:2I]
 * for c < I = n / 2, evaluated in fp32 on the accumulators and rounded once.
 *   x    [m, k]       bf16
 *   w13  [E, k, n]    bf16, n = 2 I: the I gate columns, then the I up columns
 *   offs [E]          int32 cumulative end offsets, device memory
 *   out  [m, I]       out_dtype; rows [0, end(E-1)) are written, the rest
 *                     untouched
 * gg_masked_forward_silu_mul -- the same on the masked layout:
 *   x [E, max_m, k], out [E, max_m, I]; only active rows are read or written.
 * Requires n % 16 == 0 (I a multiple of 8).  The activation step between the
 * gate/up and down grouped GEMMs (sglang PR #32385, "Cause": the SiLU-mul
 * step on the masked layout writes only rows below masked_m), fused here so
 * the 2 I-wide gate/up product never reaches memory.
 */
gg_status gg_forward_silu_mul(const void* x, const void* w13,
                              const int32_t* offs, void* out,
                              gg_dtype out_dtype, int64_t m, int64_t k,
                              int64_t n, int32_t num_groups, void* stream);
gg_status gg_masked_forward_silu_mul(const void* x, const void* w13,
                                     const int32_t* masked_m, void* out,
                                     gg_dtype out_dtype, int64_t max_m,
                                     int64_t k, int64_t n,
                                     int32_t num_groups, void* stream);

/*
 * Scaled and accumulating forms of the six passes:
 *
 *   out = alpha * P + beta * out          (P = the pass's grouped product)
 *
 * over exactly the elements the plain entry point writes (rows of experts;
 * all of dW).  The combination happens in fp32 before the single rounding to
 * the output type -- fused accumulation, so accumulating into an fp32
 * main-grad (wgrad with beta = 1) loses nothing to an intermediate bf16
 * round (TransformerEngine PR #3542, "Changes": explicit alpha/beta and fused
 * accumulation into fp32 outputs are a distinct mode of the grouped GEMM).
 * When beta == 0 the output is not read (NaN in it is overwritten), and
 * alpha = 1, beta = 0 is the plain entry point.  When beta != 0 every element
 * written is read first; an expert with no rows gets beta * dW[g] in wgrad.
 * alpha and beta are IEEE fp32: NaN and infinity propagate.  Arguments,
 * layouts, ownership and errors are those of the plain entry point.
 */
gg_status gg_forward_ex(const void* x, const void* w, const int32_t* offs,
                        void* y, gg_dtype y_dtype, int64_t m, int64_t k,
                        int64_t n, int32_t num_groups, float alpha,
                        float beta, void* stream);
gg_status gg_dgrad_ex(const void* dy, const void* w, const int32_t* offs,
                      void* dx, gg_dtype dx_dtype, int64_t m, int64_t k,
                      int64_t n, int32_t num_groups, float alpha, float beta,
                      void* stream);
gg_status gg_wgrad_ex(const void* x, const void* dy, const int32_t* offs,
                      void* dw, gg_dtype dw_dtype, int64_t m, int64_t k,
                      int64_t n, int32_t num_groups, float alpha, float beta,
                      void* stream);
gg_status gg_masked_forward_ex(const void* x, const void* w,
                               const int32_t* masked_m, void* y,
                               gg_dtype y_dtype, int64_t max_m, int64_t k,
                               int64_t n, int32_t num_groups, float alpha,
                               float beta, void* stream);
gg_status gg_masked_dgrad_ex(const void* dy, const void* w,
                             const int32_t* masked_m, void* dx,
                             gg_dtype dx_dtype, int64_t max_m, int64_t k,
                             int64_t n, int32_t num_groups, float alpha,
                             float beta, void* stream);
gg_status gg_masked_wgrad_ex(const void* x, const void* dy,
                             const int32_t* masked_m, void* dw,
                             gg_dtype dw_dtype, int64_t max_m, int64_t k,
                             int64_t n, int32_t num_groups, float alpha,
                             float beta, void* stream);

/*
 * Backward of the grouped bias: with y[i, :] += s[i] * bias[g, :] over the
 * rows i of each expert g,
 *   gg_bias_grad        dbias[g, :] = sum_{i in g} s[i] dY[i, :]   (s = 1
 *                       when bias_scale is NULL); an expert with no rows
 *                       gets +0.0.  dbias fp32 [E, n], written entirely.
 *   gg_bias_scale_grad  ds[i] = sum_n bias[g, n] dY[i, n] for the rows an
 *                       expert owns; ds fp32 [m] (masked: [E * max_m]);
 *                       other entries untouched.
 * dY bf16 [m, n] (masked: [E, max_m, n]); sums in fp32 in a fixed order
 * (deterministic).  Errors as the GEMM entry points.
 * Cited passage: TransformerEngine PR #3542, "Validation" (the grouped
 * GEMM's tests cover bias in forward, dgrad and wgrad) and "Summary"
 * (grouped bias, scaled per token).
 */
gg_status gg_bias_grad(const void* dy, const int32_t* offs,
                       const float* bias_scale, float* dbias, int64_t m,
                       int64_t n, int32_t num_groups, void* stream);
gg_status gg_masked_bias_grad(const void* dy, const int32_t* masked_m,
                              const float* bias_scale, float* dbias,
                              int64_t max_m, int64_t n, int32_t num_groups,
                              void* stream);
gg_status gg_bias_scale_grad(const void* dy, const int32_t* offs,
                             const void* bias, float* ds, int64_t m,
                             int64_t n, int32_t num_groups, void* stream);
gg_status gg_masked_bias_scale_grad(const void* dy, const int32_t* masked_m,
                                    const void* bias, float* ds,
                                    int64_t max_m, int64_t n,
                                    int32_t num_groups, void* stream);

/*
 * [E, N, K] weight layout
 * -----------------------
 * The same passes with each expert's weight stored transposed, W[g] as
 * [n, k] (k contiguous) and dW as [E, n, k]: the "NT" / "TN" forms the
 * grouped GEMM dispatches besides "NN" (TransformerEngine PR #3542,
 * "Summary": TN, NN and NT dispatch), and the layout of the fp8 call's
 * weight (sglang PR #32385, "Evidence": the "nt" grouped GEMM).
 *
 *   gg_forward_nk         y[i, :]  = x[i, :] . W[g]^T        x [m, k], y [m, n]
 *   gg_dgrad_nk           dx[i, :] = dy[i, :] . W[g]         dy [m, n], dx [m, k]
 *   gg_wgrad_nk           dW[g]    = dy[rows of g]^T . x[rows of g]   dW [E, n, k]
 *   gg_masked_forward_nk  y[e, r, :] = x[e, r, :] . W[e]^T, r < masked_m[e]
 *
 * Arguments, requirements, ownership and errors are those of the [E, k, n]
 * entry point of the same pass; the _ex forms add alpha and beta as above.
 */
gg_status gg_forward_nk(const void* x, const void* w, const int32_t* offs,
                        void* y, gg_dtype y_dtype, int64_t m, int64_t k,
                        int64_t n, int32_t num_groups, void* stream);
gg_status gg_dgrad_nk(const void* dy, const void* w, const int32_t* offs,
                      void* dx, gg_dtype dx_dtype, int64_t m, int64_t k,
                      int64_t n, int32_t num_groups, void* stream);
gg_status gg_wgrad_nk(const void* x, const void* dy, const int32_t* offs,
                      void* dw, gg_dtype dw_dtype, int64_t m, int64_t k,
                      int64_t n, int32_t num_groups, void* stream);
gg_status gg_masked_forward_nk(const void* x, const void* w,
                               const int32_t* masked_m, void* y,
                               gg_dtype y_dtype, int64_t max_m, int64_t k,
                               int64_t n, int32_t num_groups, void* stream);
gg_status gg_forward_nk_ex(const void* x, const void* w, const int32_t* offs,
                           void* y, gg_dtype y_dtype, int64_t m, int64_t k,
                           int64_t n, int32_t num_groups, float alpha,
                           float beta, void* stream);
gg_status gg_dgrad_nk_ex(const void* dy, const void* w, const int32_t* offs,
                         void* dx, gg_dtype dx_dtype, int64_t m, int64_t k,
                         int64_t n, int32_t num_groups, float alpha,
                         float beta, void* stream);
gg_status gg_wgrad_nk_ex(const void* x, const void* dy, const int32_t* offs,
                         void* dw, gg_dtype dw_dtype, int64_t m, int64_t k,
                         int64_t n, int32_t num_groups, float alpha,
                         float beta, void* stream);
gg_status gg_masked_forward_nk_ex(const void* x, const void* w,
                                  const int32_t* masked_m, void* y,
                                  gg_dtype y_dtype, int64_t max_m, int64_t k,
                                  int64_t n, int32_t num_groups, float alpha,
                                  float beta, void* stream);

/*
 * Grouped bias with a per-token factor
 * ------------------------------------
 *   y[i, :] = alpha * (x[i, :] . W[g]) + beta * y[i, :] + s[i] * bias[g, :]
 * over the rows i of each expert g, combined in fp32 and rounded once.
 *   bias        bf16 [E, n], device memory, 16-byte aligned
 *   bias_scale  fp32 per-token factors s, device memory, or NULL for s = 1.
 *               Indexed by output row (masked: e * max_m + r); only rows
 *               an expert owns are read, so for the ragged layout it needs
 *               just end(E-1) entries -- the logical tokens -- however much
 *               unused capacity x and y carry (TransformerEngine PR #3542,
 *               review finding "Bias scaling breaks capacity": the scale
 *               vector covers the logical rows only and the capacity rows
 *               must be preserved).
 * Rows past end(E-1) (masked: at or past masked_m[e]) are neither read nor
 * written.  Otherwise as gg_forward_ex / gg_masked_forward_ex.
 * Cited passage: TransformerEngine PR #3542, "Summary" (grouped bias applied
 * to the grouped GEMM's output, optionally scaled per token) and the review
 * finding above.
 */
gg_status gg_forward_bias(const void* x, const void* w, const int32_t* offs,
                          const void* bias, const float* bias_scale, void* y,
                          gg_dtype y_dtype, int64_t m, int64_t k, int64_t n,
                          int32_t num_groups, float alpha, float beta,
                          void* stream);
gg_status gg_masked_forward_bias(const void* x, const void* w,
                                 const int32_t* masked_m, const void* bias,
                                 const float* bias_scale, void* y,
                                 gg_dtype y_dtype, int64_t max_m, int64_t k,
                                 int64_t n, int32_t num_groups, float alpha,
                                 float beta, void* stream);

/*
 * Producing the grouped layout
 * ----------------------------
 * The steps upstream and downstream of the grouped GEMM: offsets from
 * per-expert row counts, the permutation of token slots into expert-grouped
 * rows padded to min_alignment_m, the row gather, and the weighted combine
 * back to tokens.  All run on the device; none reads anything back to the
 * host (PyTorch issue #152668, "Describe the bug": offsets are created by a
 * permute-indices kernel with min_alignment_m 8 or 16, and padding empty
 * experts avoids the hang of that page's backend; TransformerEngine PR
 * #3224, discussion: m_splits live on the device).
 *
 * pad(c) = c rounded up to a multiple of min_alignment (>= 1), and at least
 * min_alignment when pad_empty != 0.
 *
 * gg_offsets_from_splits -- offs[g] = sum_{g' <= g} pad(m_splits[g']).
 *   m_splits  int64 [num_groups] device (negative counts count as 0)
 *   offs      int32 [num_groups] device, written.  A running sum at or past
 *             2^31 - 2^16 (the GEMMs' row limit) is saturated there instead
 *             of wrapping, so the offsets stay monotone and a GEMM clamps
 *             them to its own row count.
 *
 * gg_route -- token-slot -> expert assignment to the grouped layout.
 *   expert_of_slot  int32 [slots] device: the expert of each (token, k)
 *                   slot, slot = token * topk + k; values outside
 *                   [0, num_groups) drop the slot
 *   offs            int32 [num_groups]: padded end offsets, written
 *   row_slot        int32 [rows_cap]: for each row below offs[E-1] the slot
 *                   it holds, or -1 for a padding row; rows past it untouched.
 *                   Within an expert the slots keep their order.
 *   rows_cap        >= gg_route_rows_bound(slots, num_groups, min_alignment);
 *                   that bound must be below 2^31 - 2^16 (the GEMMs' row
 *                   limit), so every routed layout is one the GEMMs accept
 *   slot_row        int32 [slots]: the row each slot went to, -1 if dropped
 *   workspace       gg_route_workspace_bytes(slots, num_groups) bytes of
 *                   device memory, 16-byte aligned, the caller's; contents
 *                   on entry do not matter
 *
 * gg_gather_rows -- dst[r] = src[row_slot[r] / topk] for r below the last
 *   end offset, zeros for a padding row; rows past it untouched.  src has
 *   `tokens` rows and dst rows_cap rows of row_bytes (a multiple of 16) each:
 *   bf16 or e4m3 activations alike.
 *
 * gg_combine_rows -- out[t, :] = sum_k w[t, k] y[slot_row[t * topk + k], :]
 *   over the slots that were not dropped, in fp32, rounded once to out_dtype.
 *   y bf16 [rows_cap, n] (n % 8 == 0); weights fp32 [tokens, topk] or NULL
 *   for 1; out [tokens, n].
 * Cited passages: PyTorch issue #152668, "Describe the bug" (permute indices
 * with min_alignment_m; padding empty experts) and "Probably two
 * resolutions" (a); TransformerEngine PR #3224, discussion (device m_splits).
 */
gg_status gg_offsets_from_splits(const int64_t* m_splits, int32_t num_groups,
                                 int32_t min_alignment, int pad_empty,
                                 int32_t* offs, void* stream);
int64_t gg_route_rows_bound(int64_t slots, int32_t num_groups,
                            int32_t min_alignment);
int64_t gg_route_workspace_bytes(int64_t slots, int32_t num_groups);
gg_status gg_route(const int32_t* expert_of_slot, int64_t slots,
                   int32_t num_groups, int32_t min_alignment, int pad_empty,
                   int32_t* offs, int32_t* row_slot, int64_t rows_cap,
                   int32_t* slot_row, void* workspace, void* stream);
/*
 * gg_route_noalloc -- gg_route for callers that cannot allocate device
 *   memory (code under HIP graph capture, tight serving loops, harnesses
 *   that forbid hipMalloc): the same arguments and results without the
 *   workspace.  The route histograms go to a scratch array of
 *   GG_ROUTE_NOALLOC_SCRATCH_BYTES that the library holds per GPU until the
 *   process ends; gg_route_workspace_bytes(slots, num_groups) must not exceed
 *   it (GG_ERR_LIMIT otherwise: 4 MiB covers, for example, 4M slots with 256
 *   experts).  Allocates nothing.  Every call on one GPU shares that GPU's
 *   array, so calls whose executions overlap on one GPU (different streams,
 *   or host threads racing on one stream) race and may corrupt each other's
 *   results; calls ordered on one stream are safe.
 */
#define GG_ROUTE_NOALLOC_SCRATCH_BYTES (4 << 20)
gg_status gg_route_noalloc(const int32_t* expert_of_slot, int64_t slots,
                           int32_t num_groups, int32_t min_alignment,
                           int pad_empty, int32_t* offs, int32_t* row_slot,
                           int64_t rows_cap, int32_t* slot_row, void* stream);
gg_status gg_gather_rows(const void* src, int64_t tokens, int64_t row_bytes,
                         const int32_t* row_slot, int32_t topk,
                         const int32_t* offs, int32_t num_groups,
                         int64_t rows_cap, void* dst, void* stream);
gg_status gg_combine_rows(const void* y, int64_t n, const int32_t* slot_row,
                          const float* weights, int32_t topk, int64_t tokens,
                          int64_t rows_cap, void* out, gg_dtype out_dtype,
                          void* stream);

/*
 * FP8 (e4m3) block-scaled forward
 * -------------------------------
 * The fp8 form of the forward and masked forward (sglang PR #32385: the
 * masked MoE GEMMs of an fp8 rollout, "Evidence" operand table and "Cause"
 * model table): e4m3 operands (OCP E4M3, one byte each) with one power-of-
 * two scale per row and 128 reduction values,
 *
 *   Y[i, n] = sum_k x[i, k] sx[i, k/128] * w[g, n, k] sw[g, n, k/128]
 *
 * over the rows i of expert g.  The weight is [E, n, k] with k contiguous
 * (the "nt" operand of the page's call), and k must be a multiple of 128
 * (G = k / 128 scale blocks).  Each 64-deep scaled matrix instruction's
 * sum is added into an fp32 accumulator; the pages fix no precision for
 * this path, and the instruction's internal summation is not specified to
 * fp32 accuracy, so results are not promised to match an fp32 dot product
 * bit for bit.
 *
 * Scales are consumed as E8M0 bytes (2^(e-127)) in a packed, tile-major
 * layout that gg_fp8_pack_scales writes; a caller packs its weight scales
 * once and its activation scales per call (with the same offsets or
 * masked_m as the GEMM that reads them).
 */
typedef enum {
    GG_FP8_ACT_RAGGED = 0,  /* activation scales, ragged rows (groups = end offsets, rows = m) */
    GG_FP8_ACT_MASKED = 1,  /* activation scales, masked layout (groups = masked_m, rows = max_m) */
    GG_FP8_WEIGHT = 2       /* weight scales, rows = n per expert (groups unused, may be NULL) */
} gg_fp8_scale_layout;

/* Bytes of packed scales for an operand of `rows` rows (m, max_m or n) and
 * reduction length k (a multiple of 128): ceil(rows/256) * num_groups tiles
 * (ragged activations: ceil(rows/256) + num_groups, an upper bound), each
 * (k / 128) * 256 bytes.  Returns -1 for invalid arguments. */
int64_t gg_fp8_scale_bytes(gg_fp8_scale_layout layout, int64_t rows, int64_t k,
                           int32_t num_groups);

/*
 * gg_fp8_pack_scales -- write the packed scales of one operand.
 *   src      scales, one per (row, k-block) at src[row * ld_src + kb]:
 *            fp32 values (src_is_f32 = 1) or E8M0 bytes (src_is_f32 = 0;
 *            the page's packed int32 scales are 4 such bytes per word).
 *            Rows run over [m] (ragged), [E, max_m] or [E, n] flattened.
 *   ld_src   elements per source row, >= k / 128
 *   groups   the end offsets (ragged) or masked_m (masked), device memory;
 *            ignored for weights
 *   dst      gg_fp8_scale_bytes(...) bytes, device memory, 16-byte aligned
 *   bad_count  optional device int32: incremented by the number of ACTIVE
 *            scales that are not UE8M0 (an fp32 with its sign or mantissa
 *            bits set -- the page's "Problem" check -- or the byte 0xFF).
 *            Inactive rows (past an expert's end, at or past masked_m) are
 *            neither read nor validated, so garbage there is harmless (the
 *            fix the page names as the more correct one, "Rejected
 *            alternatives").  A non-UE8M0 active scale is packed as its
 *            exponent field (the mantissa dropped).
 * Cited passage: sglang PR #32385, "Problem", "Cause" and "Rejected
 * alternatives".
 */
gg_status gg_fp8_pack_scales(gg_fp8_scale_layout layout, const void* src,
                             int src_is_f32, int64_t ld_src,
                             const int32_t* groups, int64_t rows, int64_t k,
                             int32_t num_groups, void* dst,
                             int32_t* bad_count, void* stream);

/*
 * gg_fp8_forward -- the ragged fp8 forward.
 *   x         [m, k]     e4m3 bytes
 *   x_scales  packed (GG_FP8_ACT_RAGGED, same offs)
 *   w         [E, n, k]  e4m3 bytes
 *   w_scales  packed (GG_FP8_WEIGHT)
 *   offs      [E] int32 end offsets, device memory
 *   y         [m, n] y_dtype; rows past end(E-1) untouched
 * Requirements: those of gg_forward, and k % 128 == 0.
 * Cited passage: sglang PR #32385, "Evidence" (fp8 operands with per-128
 * scales) and "Cause" (G = k / 128).
 */
gg_status gg_fp8_forward(const void* x, const void* x_scales, const void* w,
                         const void* w_scales, const int32_t* offs, void* y,
                         gg_dtype y_dtype, int64_t m, int64_t k, int64_t n,
                         int32_t num_groups, void* stream);

/*
 * gg_fp8_masked_forward -- the same on the masked layout: x [E, max_m, k],
 * x_scales packed with GG_FP8_ACT_MASKED and the same masked_m, y
 * [E, max_m, n]; only active rows are read or written.
 * Cited passage: sglang PR #32385, "Evidence" (the masked fp8 call and its
 * operand table).
 */
gg_status gg_fp8_masked_forward(const void* x, const void* x_scales,
                                const void* w, const void* w_scales,
                                const int32_t* masked_m, void* y,
                                gg_dtype y_dtype, int64_t max_m, int64_t k,
                                int64_t n, int32_t num_groups, void* stream);

/* Static description of a status code. */
const char* gg_status_str(gg_status s);

/* Text of the last error seen by the calling thread (argument check or HIP
 * runtime message); "" when the last call succeeded. */
const char* gg_last_error(void);

/* Library version string. */
const char* gg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GG_H */

/*
 * moe.h -- C ABI of the dropless mixture-of-experts layer hot path on AMD Instinct MI355X
 * (gfx950): routing, dispatch (histogram, offsets, permutation, gather), grouped GEMMs over
 * ragged expert groups with a fused SwiGLU epilogue, weighted combine, and the MXFP8 group
 * quantiser.
 *
 * Sources (cited by page and section; the pages describe the method in words only):
 *   [Blog]    "Accelerating Dropless MoE Training in JAX with NVIDIA Transformer Engine",
 *             Chinese rendering on zhiding.cn.
 *   [Reading] paper-daily deep reading of arXiv 2603.07685.
 *   [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0.
 *
 * Conventions shared by every entry point
 *   - Pointers named in the signatures are DEVICE pointers unless a comment says "host".
 *     The caller allocates and frees all device memory (inputs, outputs, workspace); the
 *     library never allocates, frees or keeps per-call state, and is re-entrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call only
 *     enqueues work on it and returns: no host synchronisation, no device-to-host read, so
 *     group sizes never reach the host and every call can be captured in a HIP graph
 *     ([Blog] "Optimisations dropless MoE needs": kernels must work without the CPU knowing
 *     the shapes; [Reading] contribution 4: sync-free kernels for full graph coverage).
 *   - Matrices are row-major; a leading dimension is counted in elements.
 *   - Errors the host can see (null pointers, negative or unsupported sizes, misaligned
 *     pointers, workspace too small) return a status and enqueue nothing. A failed launch
 *     returns MOE_EHIP. Bad device-side data (an expert id outside [0, E), inconsistent
 *     offsets) gives unspecified results; every kernel clamps its indices, so it never
 *     reads or writes outside the buffers described here.
 *   - Sizes of zero (T = 0, every group empty) are valid and write only what is defined.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,      /* invalid argument (checked on the host; nothing enqueued) */
    MOE_ENOTSUP = 2,     /* valid but unsupported combination (e.g. dtype pair)       */
    MOE_EWORKSPACE = 3,  /* workspace pointer NULL or smaller than moe_workspace_bytes */
    MOE_EHIP = 4         /* a HIP launch failed                                        */
} moe_status_t;

typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_E4M3 = 2,   /* MXFP8 element: OCP FP8 E4M3, one byte                                    */
    MOE_E2M1 = 3    /* MXFP4 element: OCP FP4 E2M1, two per byte, the even element in bits 3..0 */
} moe_dtype_t;
typedef enum { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score_t;
typedef enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_SWIGLU_BWD = 2 } moe_epilogue_t;
typedef enum {
    MOE_OP_ROUTE = 0,
    MOE_OP_PERMUTE = 1,
    MOE_OP_GROUPED_GEMM = 2,
    MOE_OP_QUANT = 3,
    MOE_OP_ROUTE_BWD = 4,
    MOE_OP_COMBINE_BWD_QUANT = 5
} moe_op_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(int32_t status);

/* Device bytes of workspace an entry point needs (0 if none). Arguments that do not apply
 * to `op` are ignored: ROUTE uses (T, d, E); PERMUTE uses (T, E); GROUPED_GEMM and QUANT use
 * G (the group count); ROUTE_BWD uses (T, d, E, k); COMBINE_BWD_QUANT uses (T, k, G). The
 * result depends only on sizes, never
 * on data. An unknown op returns 0. */
size_t moe_workspace_bytes(int32_t op, int64_t T, int64_t d, int32_t E, int32_t k, int32_t G);

/*
 * moe_route -- the router: logits, expert bias, top-k selection and normalised weights.
 * [Blog] opening section: a learnable router picks the top-K experts of every token;
 * [Blog] "Optimisation 2": one fused router kernel assigns the experts.
 *
 *   L[t,e]   = sum_i x[t,i] * w_router[e,i]        (fp32 accumulation)
 *   key[t,e] = L[t,e] + bias[e]                    (fp32; bias may be NULL = 0)
 *   topk_idx[t,0..k-1] = the k experts with the largest keys, largest first; equal keys
 *                        go to the lower expert id
 *   topk_w[t,j]: score == MOE_SOFTMAX: exp(key_j - key_0) / sum_j' exp(key_j' - key_0)
 *                score == MOE_SIGMOID: s_j / sum_j' s_j',  s_j = 1 / (1 + exp(-key_j))
 *   keys_out (optional, may be NULL): key[t,e] as float32 [T, E].
 *
 *   x        [T, d] of dtype (MOE_BF16 or MOE_F32), leading dimension d
 *   w_router [E, d] same dtype (row e is expert e's router vector)
 *   1 <= k <= min(E, 16), 1 <= E <= 256, d % 8 == 0, x and w_router 16-byte aligned.
 *   Workspace: moe_workspace_bytes(MOE_OP_ROUTE, T, d, E, k, 0) bytes, 256-byte aligned (it
 *   is non-zero for large bf16 layers, whose projection runs as a K-split grouped GEMM with
 *   fp32 partial logits summed in a fixed order; workspace may be NULL when it is zero).
 *   Errors: MOE_EINVAL for bad sizes or pointers, MOE_EWORKSPACE for a missing or short
 *   workspace, MOE_ENOTSUP for an unsupported dtype or (K-split path) x or w_router of 4 GiB
 *   or more, MOE_EHIP for a failed launch.
 */
moe_status_t moe_route(const void* x, const void* w_router, int32_t dtype, const float* bias,
                       int64_t T, int64_t d, int32_t E, int32_t k, int32_t score,
                       int32_t* topk_idx, float* topk_w, float* keys_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_backward -- the router's backward: from the gradient of the loss with respect to
 * the normalised top-k weights to the gradients of the keys, the router weights, the expert
 * bias and the router's share of the input gradient.
 * [Blog] opening section: the router is learnable and trained with the layer. The top-k
 * selection is piecewise constant in the keys, so only the k selected keys of a token get
 * gradient (g = d_topk_w[t,:], w = topk_w as moe_route forms it, S = sum_j s_j):
 *   score == MOE_SOFTMAX: dkey_j = w_j * (g_j - sum_i w_i g_i)
 *   score == MOE_SIGMOID: dkey_j = (g_j - sum_i w_i g_i) / S * s_j * (1 - s_j)
 * and with key = x w_router^T + bias (dkey zero for unselected experts):
 *   d_keys_sel[t,j]  = dkey_j of expert topk_idx[t,j]                      [T, k] fp32
 *   d_x[t,:]         = sum_j dkey_j * w_router[topk_idx[t,j],:]  fp32 sum in slot order,
 *                      rounded once to dtype                                [T, d]
 *                      (accumulate_dx != 0: d_x[t,:] + that sum, the incoming value
 *                      read into the fp32 sum and the total rounded once, so the expert
 *                      path's input gradient and the router's join in one buffer;
 *                      d_x_perm != NULL: the incoming value is not read from d_x but formed
 *                      as the permutation's transpose of d_x_perm [T*k, d] (rows in expert
 *                      order, through row_of) plus d_x_perm_shared [T, d] if not NULL,
 *                      rounded once to dtype exactly as moe_combine(d_x_perm, NULL, row_of,
 *                      d_x_perm_shared) stores it, then the router's share is added as
 *                      above; accumulate_dx is then ignored)
 *   d_w_router[e,:]  = sum over tokens t that picked e of dkey * x[t,:]     [E, d] fp32
 *                      (rows of expert e in ascending token order, summed in
 *                      chunks of 256 rows whose partials are added in chunk order)
 *   d_bias[e]        = sum of the same dkey (fixed-order tree)              [E] fp32
 * Each of the four outputs may be NULL (not computed). The call overwrites the outputs it
 * computes (d_x as stated above).
 *
 *   x [T, d], w_router [E, d]: dtype MOE_BF16 or MOE_F32, 16-byte aligned, d % 8 == 0;
 *   keys [T, E] fp32: moe_route's keys_out; topk_idx [T, k]: moe_route's selection;
 *   d_topk_w [T, k] fp32; offsets [E+1 or more], row_of [T, k], src_token [T*k or more]:
 *   moe_permute's outputs for this topk_idx (needed when d_w_router or d_bias is wanted;
 *   row_of always). 1 <= k <= min(E, 16), 1 <= E <= 256.
 *   Workspace: moe_workspace_bytes(MOE_OP_ROUTE_BWD, T, d, E, k, 0) bytes, 256-byte aligned.
 *   Deterministic: no atomics. Errors: MOE_EINVAL for bad sizes or pointers (d_w_router
 *   must be 16-byte aligned), MOE_ENOTSUP for another dtype, MOE_EWORKSPACE for a missing or
 *   short workspace, MOE_EHIP for a failed launch.
 */
moe_status_t moe_route_backward(const void* x, const void* w_router, int32_t dtype, const float* keys,
                                const int32_t* topk_idx, const float* d_topk_w, const int32_t* offsets,
                                const int32_t* row_of, const int32_t* src_token, int64_t T, int64_t d,
                                int32_t E, int32_t k, int32_t score, float* d_keys_sel, void* d_x,
                                int32_t accumulate_dx, const void* d_x_perm, const void* d_x_perm_shared,
                                float* d_w_router, float* d_bias, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * moe_permute -- dispatch on one GPU: per-expert histogram, group offsets, permutation and
 * (optionally) the gather of token rows into expert-contiguous order.
 * [Blog] "Optimisation 2": dispatch reorders tokens so each expert's tokens are contiguous
 * and combine later restores the original order; [Blog] "Optimisation 1": group sizes are
 * never copied to the host.
 *
 *   offsets[e]   = number of (token, slot) pairs routed to experts < e; offsets[E] = T*k.
 *   row_of[t,j]  = the row of pair (t, j) in expert order; rows of one expert are
 *                  contiguous and in ascending token order (a stable counting sort).
 *   src_token[r] = the token of row r.
 *   x_perm[r,:]  = x[src_token[r],:]   (only if x_perm != NULL; x may be NULL otherwise)
 *   shared_group != 0 appends group E holding every token in order (the always-on shared
 *   expert): offsets has E+2 entries with offsets[E+1] = T*k + T, src_token and x_perm have
 *   T*k + T rows, rows T*k + t being token t.
 *
 *   topk_idx [T, k] int32 with distinct ids in [0, E) per token.
 *   x, x_perm: dtype MOE_BF16 or MOE_F32, leading dimension d, d % 8 == 0, 16-byte aligned.
 *   Workspace: moe_workspace_bytes(MOE_OP_PERMUTE, T, d, E, k, 0) bytes, 256-byte aligned.
 *   The result is deterministic (no floating point, no order-dependent atomics).
 */
moe_status_t moe_permute(const void* x, int32_t dtype, const int32_t* topk_idx,
                         int64_t T, int64_t d, int32_t E, int32_t k, int32_t shared_group,
                         int32_t* offsets, int32_t* row_of, int32_t* src_token, void* x_perm,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Arguments of a grouped GEMM over ragged row groups (the "grouped_gemm / ragged_dot"
 * contract of [Blog] "Optimisation 1": one call runs every expert's product at its actual
 * token count and computes only the rows that exist; [Blog] Figure 3 paragraph: two such
 * GEMMs form the grouped MLP).
 *
 * For each group g with rows r in [offsets[g], offsets[g+1]):
 *   epilogue NONE:   C[r, n] = sum_k A[a(r), k] * B_g[n, k]                  n < N
 *   epilogue SWIGLU: G = sum_k A[a(r),k] B_g[n,k], U = sum_k A[a(r),k] B_g[N+n,k]
 *                    C[r, n] = silu(G) * U,  silu(z) = z / (1 + exp(-z))     n < N
 *                    (B_g has 2N rows: gate rows first, then up rows); when aux != NULL
 *                    also aux[r, n] = G and aux[r, N+n] = U (in c_dtype).
 *   epilogue SWIGLU_BWD (the SwiGLU backward fused into the data-gradient GEMM dh = dY W_down^T;
 *                    MXFP8/MXFP4 operands, bf16 C): dh = bf16(sum_k A[a(r),k] B_g[n,k]) and, with
 *                    g = aux[r, n], u = aux[r, N+n] (the saved pre-activations, read), s = 1/(1+exp(-g)):
 *                    C[r, n] = bf16(dh u s (1 + g (1 - s))), C[r, N+n] = bf16(dh g s)   n < N
 *                    (C is [M, 2N]: the values moe_swiglu_backward writes from the stored dh;
 *                    the fused quantisation below then covers all 2N columns).
 * with a(r) = a_rows[r] if a_rows != NULL (a fused gather) else r, and
 * B_g = B + g * b_group_stride elements (groups may share or overlap B: it is only read).
 * Accumulation is fp32; C is rounded once.
 * Rows of C outside [offsets[0], offsets[G]) are not written. Empty groups cost nothing.
 *
 * Ragged-K mode (ragged_k = 1; the weight gradients, whose contraction runs over the tokens
 * of each group: [Reading] contribution 3 on group-wise low precision, [Blog]
 * "Optimisations dropless MoE needs" on group-aware MXFP8). Every group has the same
 * M x N output and its own K range of n_g = offsets[g+1] - offsets[g] blocks of 32:
 *   C_g[m, n] = sum over k < 32 n_g of A_g[m, k] * B_g[n, k]
 * for m < M, n < N, with C_g = C + g * c_group_stride elements. The operands are the
 * group-major output of moe_group_quant_mxfp8's column-wise mode: A_g is the row-major
 * [M, 32 n_g] matrix at A + 32*M*offsets[g], B_g the [N, 32 n_g] matrix at
 * B + 32*N*offsets[g], their scales [M, n_g] at a_scale + M*offsets[g] and [N, n_g] at
 * b_scale + N*offsets[g]. offsets is non-decreasing with offsets[G] <= K/32 and every entry
 * a multiple of 4 (128 elements), as the quantiser's block_start is; a group with an empty
 * range gets C_g = 0 written. The leading dimensions state the capacity: lda = ldb = K,
 * lda_scale = ldb_scale = K/32 (A holds M*K codes, B N*K). Only MXFP8 operands and epilogue
 * NONE; a_rows must be NULL, A_rows = M, b_group_stride and b_scale_group_stride 0,
 * c_group_stride >= M * ldc.
 */
typedef struct moe_gemm_args {
    int32_t G;                  /* number of groups (>= 1)                                  */
    const int32_t* offsets;     /* device [G+1], non-decreasing, offsets[G] <= M            */
    int64_t M;                  /* rows of C (and of a_rows); a host-known capacity         */
    int64_t N;                  /* output columns, N % 8 == 0                                */
    int64_t K;                  /* contraction length: K % 64 == 0 (bf16), % 128 (E4M3), % 256 (E2M1) */
    const void* A;              /* [A_rows, K], leading dimension lda                        */
    int32_t a_dtype;            /* MOE_BF16, MOE_F32, MOE_E4M3 or MOE_E2M1 (scales below)   */
    int64_t lda;
    int64_t A_rows;             /* rows of A (gather indices are clamped to it)              */
    const int32_t* a_rows;      /* optional device [M] gather index                          */
    const void* B;              /* group g: [N or 2N, K] at B + g*b_group_stride, ld = ldb   */
    int32_t b_dtype;            /* must equal a_dtype                                        */
    int64_t ldb;
    int64_t b_group_stride;
    void* C;                    /* [M, N], leading dimension ldc                             */
    int32_t c_dtype;            /* MOE_BF16 or MOE_F32                                       */
    int64_t ldc;
    int32_t epilogue;           /* moe_epilogue_t                                            */
    void* aux;                  /* SWIGLU: optional [M, 2N] pre-activation save; SWIGLU_BWD: its input */
    int64_t ld_aux;
    /* MXFP8 operands (a_dtype = b_dtype = MOE_E4M3, K % 128 == 0): A and B hold E4M3 codes and
     * every 32 consecutive K elements of a row share one E8M0 scale byte s, the element value
     * being code_value * 2^(s-127) ([OCP-MX]); products are exact and summed in fp32.
     * MXFP4 operands (MOE_E2M1, K % 256 == 0, ragged_k = 0): the same with E2M1
     * codes packed two per byte (element 2i of a row in bits 3..0 of byte i, as
     * moe_group_quant_mxfp4 writes them); lda, ldb and b_group_stride still count elements
     * (even numbers), so a row starts lda/2 bytes after the previous one. */
    const uint8_t* a_scale;     /* [A_rows, K/32], leading dimension lda_scale (a_rows applies) */
    int64_t lda_scale;
    const uint8_t* b_scale;     /* group g: [N or 2N, K/32] at b_scale + g*b_scale_group_stride  */
    int64_t ldb_scale;
    int64_t b_scale_group_stride;
    int32_t ragged_k;           /* 0: groups partition the rows of A and C; 1: ragged-K mode  */
    int64_t c_group_stride;     /* ragged-K mode: elements between consecutive groups' C      */
    /* Fused output quantisation ([Blog] "JAX plus Transformer Engine MoE training
     * performance": quantisation fused into the GEMM is the planned next step; [Blog]
     * "Optimisations dropless MoE needs": group-aware MXFP8). q_dtype 0: off. MOE_E4M3 or
     * MOE_E2M1 (ragged rows only, MXFP8 or MXFP4 operands, c_dtype MOE_BF16, N % 32 == 0;
     * MOE_ENOTSUP otherwise): the epilogue also quantises
     * the bf16 values of C it forms, so the bytes equal those moe_group_quant_mxfp8 (axis 0,
     * and axis 1 for q_col) or moe_group_quant_mxfp4 write when run on the stored C:
     *   q_row [M, N] E4M3 codes or [M, N/2] packed E2M1 (leading dimension ld_q_row bytes,
     *         16-byte aligned, ld_q_row % 16 == 0), s_row [M, N/32] scale bytes (ld_s_row);
     *   q_col, s_col (MOE_E4M3 only, optional): the group-aware column-wise copy in
     *         moe_group_quant_mxfp8's axis-1 layout, with capacity q_col_blocks >=
     *         4 (ceil(M/128) + G) blocks (q_col [N, 32 q_col_blocks], s_col [N, q_col_blocks]);
     *         the group block prefix is written to q_block_start [G+1].
     * Rows outside the groups are not written. C may be NULL when q_dtype != 0 (only the
     * quantised copies are written). */
    int32_t q_dtype;
    uint8_t* q_row;
    int64_t ld_q_row;
    uint8_t* s_row;
    int64_t ld_s_row;
    uint8_t* q_col;
    uint8_t* s_col;
    int32_t* q_block_start;
    int64_t q_col_blocks;
} moe_gemm_args_t;

/* Grouped GEMM (see moe_gemm_args_t). Workspace: moe_workspace_bytes(MOE_OP_GROUPED_GEMM,
 * 0, 0, 0, 0, G) bytes (a device-built tile schedule), G <= 2047 (1023 for MXFP8 and MXFP4
 * outside the ragged-K mode; MOE_ENOTSUP above it). A, B, C,
 * aux 16-byte aligned; A and B rows (lda, ldb, b_group_stride, in bytes) 16-byte multiples; ldc, ld_aux multiples
 * of 8; MXFP8 scale pointers and their strides 4-byte multiples. A (A_rows x lda) and one
 * group's B (N or 2N rows x ldb) must each span less than 4 GiB (MOE_ENOTSUP otherwise: the
 * loads use 32-bit offsets from the tile's base; MXFP8/MXFP4 outside the ragged-K mode: also
 * A_rows x lda_scale and one group's N (2N) x ldb_scale). The args struct is read on the host during
 * the call only. */
moe_status_t moe_grouped_gemm(const moe_gemm_args_t* args, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * moe_combine -- restore token order and accumulate the expert outputs.
 * [Blog] "Optimisation 2": combine returns each processed token to its original position
 * and sums the experts' results.
 *
 *   out[t,:] = sum_{j<k} topk_w[t,j] * y[row_of[t,j],:]  (+ y_shared[t,:] if not NULL)
 * summed in fp32 in the fixed order j = 0..k-1 then the shared expert, rounded once.
 *   y        [T*k, d] (rows in expert order), y_shared [T, d] or NULL, out [T, d];
 *   topk_w   [T, k] fp32, or NULL for weights of one: then the call is the transpose of the
 *            permutation's gather, dx[t] = sum_j dX_perm[row_of[t,j]] (+ the shared rows),
 *            which the backward uses to return the permuted input gradient to its tokens;
 *   dtype MOE_BF16 or MOE_F32 for y, y_shared and out; d % 8 == 0; 16-byte aligned.
 */
moe_status_t moe_combine(const void* y, int32_t dtype, const float* topk_w, const int32_t* row_of,
                         const void* y_shared, int64_t T, int64_t d, int32_t k, void* out,
                         void* stream);

/*
 * moe_combine_backward -- the transpose of moe_combine (the backward of [Blog]
 * "Optimisation 2"'s weighted combine):
 *   dy[row_of[t,j],:] = topk_w[t,j] * d_out[t,:]           exact product rounded once
 *   dy_shared[t,:]    = d_out[t,:]                         (if dy_shared != NULL)
 *   dw[t,j]           = sum_c d_out[t,c] * y[row_of[t,j],c] (if dw != NULL; fp32, fixed order)
 *   d_out [T, d], y [T*k, d] (the forward's expert outputs; read only when dw != NULL),
 *   dy [T*k, d] (every row written once, since row_of is a permutation; may be NULL when
 *   only dw or dy_shared are wanted), dy_shared [T, d],
 *   topk_w and dw [T, k] fp32; dtype MOE_BF16 or MOE_F32; d % 8 == 0; 16-byte aligned.
 */
moe_status_t moe_combine_backward(const void* d_out, int32_t dtype, const float* topk_w, const int32_t* row_of,
                                  const void* y, int64_t T, int64_t d, int32_t k, void* dy, void* dy_shared,
                                  float* dw, void* stream);

/*
 * moe_swiglu_backward -- gradient of the SwiGLU product h = silu(g) * u with respect to the
 * gate and up pre-activations the forward saved ([Blog] Figure 3 paragraph: the experts
 * are SwiGLU MLPs). With s = 1 / (1 + exp(-g)):
 *   dgu[r, c]     = dh[r,c] * u * s * (1 + g * (1 - s))    (gate part, c < f)
 *   dgu[r, f + c] = dh[r,c] * g * s                         (up part)
 * where g = gu[r, c] and u = gu[r, f + c] (the layout moe_grouped_gemm's SWIGLU aux writes).
 *   dh [rows, f] (ld_dh), gu [rows, 2f] (ld_gu), dgu [rows, 2f] (ld_dgu); dtype MOE_BF16 or
 *   MOE_F32; f and every leading dimension multiples of 8; 16-byte aligned. Math in fp32,
 *   one rounding per output.
 */
moe_status_t moe_swiglu_backward(const void* dh, int64_t ld_dh, const void* gu, int64_t ld_gu, int32_t dtype,
                                 int64_t rows, int64_t f, void* dgu, int64_t ld_dgu, void* stream);

/*
 * moe_group_quant_mxfp8 -- MXFP8 quantisation: E4M3 element codes plus one E8M0 scale byte
 * per block of 32 elements taken along a GEMM's contraction axis.
 * [Blog] "Optimisations dropless MoE needs": group-aware MXFP8 quantisation for the expert
 * GEMMs; [Reading] contribution 3: MoE low precision needs group quantisation.
 * Rule ([OCP-MX]): for a block with largest magnitude amax, scale byte
 *   s = clamp(floor(log2 amax) - 8 + 127, 0, 254)   (s = 0 for an all-zero block)
 * and each element x becomes the E4M3 code of x / 2^(s-127) rounded to nearest-even,
 * saturating at +-448 (bias 7, 3 mantissa bits, subnormal step 2^-9; the sign of zero kept).
 *
 *   in [rows, cols] (MOE_BF16 or MOE_F32, leading dimension ld_in); axis 0 needs cols % 32 == 0.
 *   row_index (device, [rows] int32, or NULL): logical row r is read from in row
 *     row_index[r] (clamped into [0, in_rows)), e.g. the permutation's src_token so that
 *     the permuted activations are quantised straight from the token-ordered input;
 *     in_rows is the number of rows of `in` (ignored when row_index is NULL).
 *   axis 0 (row-wise, for operands contracted along their rows' length):
 *     q [rows, ld_q >= cols] codes, scales [rows, ld_scales >= cols/32] bytes;
 *     group_offsets, G, block_start and workspace are ignored.
 *   axis 1 (group-aware column-wise, for the weight-gradient operands, contracted over
 *     the tokens of each group): rows are partitioned into G groups by group_offsets
 *     (device, [G+1]); each column is cut into blocks of 32 consecutive rows inside one
 *     group, the last block of a group possibly partial (its missing rows count as zero);
 *     blocks never straddle groups. Output is TRANSPOSED per group so the blocked axis is
 *     contiguous, and GROUP-MAJOR: group g owns nb_g = 4 * ceil(m_g/128) blocks, numbered
 *     block_start[g] .. block_start[g+1]-1 (block_start[g] = sum over g' < g of nb_g'), so
 *     every group starts on a 128-element boundary (one MXFP8 GEMM K slice); its codes are a
 *     row-major [cols, 32*nb_g] matrix at q + 32*cols*block_start[g] (block i of column c in
 *     columns 32i .. 32i+31; zero codes for the missing rows of a partial block) and its
 *     scales a [cols, nb_g] matrix at scales + cols*block_start[g]. Blocks past a group's
 *     last row are all zero (codes 0, scale byte 0) and add nothing to a product.
 *     block_start (device, [G+1]) is written when not NULL, else kept in workspace
 *     (moe_workspace_bytes(MOE_OP_QUANT, 0, 0, 0, 0, G) bytes). Capacity: ld_scales is the
 *     capacity in blocks, nblk <= ld_scales with nblk = 4 * (ceil(rows/128) + G), and
 *     ld_q == 32 * ld_scales; q holds 32 * cols * ld_scales bytes and scales
 *     cols * ld_scales bytes (the sizes of [cols, 32*nblk] and [cols, nblk] matrices);
 *     in 16-byte aligned with ld_in and cols spanning multiples of 16 bytes, scales 4-byte
 *     aligned.
 *   q 16-byte aligned (axis 0 also ld_q % 16 == 0). Deterministic; no floating-point atomics.
 */
moe_status_t moe_group_quant_mxfp8(const void* in, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_in,
                                   const int32_t* row_index, int64_t in_rows,
                                   const int32_t* group_offsets, int32_t G, int32_t axis,
                                   uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_scales,
                                   int32_t* block_start, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_group_quant_mxfp4 -- MXFP4 quantisation, row-wise: E2M1 element codes plus one E8M0
 * scale byte per block of 32 consecutive elements of a row (the layout a forward GEMM
 * contracting along the rows' length reads).
 * [Blog] "JAX plus Transformer Engine MoE training performance": a 4-bit block-scaled format
 * is the planned next precision; [Reading] contribution 3: FP8/FP4 recipes. [OCP-MX]: MXFP4
 * is E2M1 elements (bias 1, one mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6) with an E8M0
 * scale. Rule: for a block with largest magnitude amax, scale byte
 *   s = clamp(floor(log2 amax) - 2 + 127, 0, 254)   (s = 0 for an all-zero block)
 * and each element x becomes the E2M1 code of x / 2^(s-127) rounded to nearest, ties to the
 * even mantissa, saturating at +-6; code bit 3 is the sign (kept for zero), bits 2..0 the
 * magnitude index 0..7 of the values above.
 *
 *   in [rows (logical), cols] (MOE_BF16 or MOE_F32, leading dimension ld_in), cols % 32 == 0;
 *   row_index / in_rows as moe_group_quant_mxfp8 (logical row r reads in row row_index[r],
 *   clamped into [0, in_rows)).
 *   q [rows, ld_q >= cols/2] bytes: element 2i of a row in bits 3..0 of byte i, element 2i+1
 *   in bits 7..4 (the packing moe_grouped_gemm's MOE_E2M1 operands use);
 *   scales [rows, ld_scales >= cols/32] bytes.
 *   in and q 16-byte aligned, ld_q % 16 == 0, ld_in rows spanning multiples of 16 bytes.
 *   Deterministic. Errors: MOE_EINVAL for bad sizes or pointers, MOE_ENOTSUP for another
 *   dtype, MOE_EHIP for a failed launch.
 */
moe_status_t moe_group_quant_mxfp4(const void* in, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_in,
                                   const int32_t* row_index, int64_t in_rows, uint8_t* q, int64_t ld_q,
                                   uint8_t* scales, int64_t ld_scales, void* stream);

/*
 * moe_group_quant_mxfp8_dual -- both MXFP8 copies of one operand from a single read of it:
 * the row-wise copy (axis 0 above) and the group-aware column-wise copy (axis 1 above).
 * [Blog] "Optimisations dropless MoE needs": an expert GEMM operand of the MXFP8 training step
 * is contracted along its rows in one product and along its columns (each group's tokens) in
 * another, so both quantisations are needed; [Reading] contribution 3: group quantisation.
 *
 *   Arguments as in moe_group_quant_mxfp8 with axis 1 (in, dtype, rows, cols, ld_in,
 *   row_index, in_rows, group_offsets, G, block_start, workspace): q_col / ld_q_col /
 *   s_col / ld_s_col take the column-wise output with that mode's layout and capacity rules;
 *   q_row [rows, ld_q_row >= cols] and s_row [rows, ld_s_row >= cols/32] take the row-wise
 *   output of logical row r (read through row_index like the column-wise copy). cols % 32 == 0;
 *   q_row 16-byte aligned with ld_q_row % 16 == 0.
 *   Every code and scale byte equals what the two single-axis calls write. Rows outside
 *   every group (offsets[G] < rows) get neither copy.
 */
moe_status_t moe_group_quant_mxfp8_dual(const void* in, int32_t dtype, int64_t rows, int64_t cols, int64_t ld_in,
                                        const int32_t* row_index, int64_t in_rows, const int32_t* group_offsets,
                                        int32_t G, uint8_t* q_row, int64_t ld_q_row, uint8_t* s_row,
                                        int64_t ld_s_row, uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col,
                                        int64_t ld_s_col, int32_t* block_start, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * moe_swiglu_backward_quant_mxfp8_dual -- the SwiGLU backward and both MXFP8 copies of its
 * output in one pass, so the bf16 gate/up gradient never goes to memory.
 * [Blog] "Optimisations dropless MoE needs": the expert GEMMs' operands are MXFP8 with
 * group-aware quantisation, and the dgrad 1 / wgrad 1 GEMMs read only those copies of the
 * gate/up gradient; [Blog] Figure 3 paragraph: the experts are SwiGLU MLPs.
 *
 *   The output equals moe_swiglu_backward(dh, ld_dh, gu, ld_gu, dtype, rows, f, dgu, 2f)
 *   followed by moe_group_quant_mxfp8_dual(dgu, dtype, rows, 2f, 2f, NULL, rows,
 *   group_offsets, G, q_row, ..., s_col, ...) byte for byte: each dgu value is formed in
 *   fp32 as that kernel does, rounded to dtype, then quantised.
 *   dh [rows, f] (ld_dh), gu [rows, 2f] (ld_gu) as moe_swiglu_backward; dtype MOE_BF16 only
 *   (MOE_ENOTSUP otherwise); f % 128 == 0; q_row/s_row/q_col/s_col, block_start, workspace and
 *   their capacity rules as moe_group_quant_mxfp8_dual with cols = 2f. Errors as those two.
 */
moe_status_t moe_swiglu_backward_quant_mxfp8_dual(const void* dh, int64_t ld_dh, const void* gu, int64_t ld_gu,
                                                  int32_t dtype, int64_t rows, int64_t f,
                                                  const int32_t* group_offsets, int32_t G, uint8_t* q_row,
                                                  int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row,
                                                  uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col, int64_t ld_s_col,
                                                  int32_t* block_start, void* workspace, size_t workspace_bytes,
                                                  void* stream);

/*
 * moe_combine_backward_quant_mxfp8_dual -- the combine's transpose quantised straight into
 * both MXFP8 copies, so the bf16 dY never goes to memory ([Blog] "Optimisation 2": the combine
 * weights each expert row by its routing weight; [Blog] "Optimisations dropless MoE needs":
 * the expert GEMMs, whose data- and weight-gradient products read dY, run in MXFP8 with
 * group-aware quantisation).
 *
 *   The output equals moe_combine_backward(d_out, dtype, topk_w, row_of, ..., dy = dY,
 *   dy_shared = the shared rows of dY) followed by moe_group_quant_mxfp8_dual(dY, dtype,
 *   rows, d, d, NULL, rows, group_offsets, G, q_row, ..., s_col, ...) byte for byte, with
 *   rows = T*k (+ T when shared_group != 0, those rows being d_out itself): each dY row is
 *   topk_w[t,j] * d_out[t] rounded once to dtype, read through src_token.
 *   d_out [T, d] (leading dimension d); topk_w, row_of [T, k]; src_token [rows] as
 *   moe_permute writes them; d % 32 == 0; q_row/s_row/q_col/s_col/block_start and their
 *   capacity rules as moe_group_quant_mxfp8_dual with cols = d.
 *   Workspace: moe_workspace_bytes(MOE_OP_COMBINE_BWD_QUANT, T, 0, 0, k, G) bytes, 256-byte
 *   aligned (each permuted row's weight, then the quantiser's). Errors as those two calls.
 */
moe_status_t moe_combine_backward_quant_mxfp8_dual(const void* d_out, int32_t dtype, const float* topk_w,
                                                   const int32_t* row_of, const int32_t* src_token, int64_t T,
                                                   int64_t d, int32_t k, int32_t shared_group,
                                                   const int32_t* group_offsets, int32_t G, uint8_t* q_row,
                                                   int64_t ld_q_row, uint8_t* s_row, int64_t ld_s_row,
                                                   uint8_t* q_col, int64_t ld_q_col, uint8_t* s_col, int64_t ld_s_col,
                                                   int32_t* block_start, void* workspace, size_t workspace_bytes,
                                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

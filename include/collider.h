/*
 * collider.h - C ABI of libcollider: the backward pass of a transformer layer under token
 * filtering, in which the activations of filtered tokens are dropped in every layer and each
 * linear / attention backward runs as dense work over the kept tokens only.  MI355X (gfx950).
 *
 * Method: "Enhancing Token Filtering Efficiency in Large Language Model Training with Collider"
 * (arXiv 2502.00340).  Its abstract states the two parts built here: activations of filtered
 * tokens are filtered across all layers, and sparse GEMMs become dimension-reduced dense GEMMs.
 * Figure 2(b) defines backward token filtering (the loss of filtered tokens is dropped), Figure 3
 * why the attention softmax activation must be filtered too, Figure 5 that the Q/K backward
 * activations are filtered with it.
 *
 * Conventions shared by every entry point
 *  - Tokens are flattened t = b*S + s (B sequences of S tokens, M = B*S); tensors are row-major,
 *    one row per token; heads are interleaved in columns (q is [rows, nq*head_dim]).
 *  - Linear weights use the [out, in] layout, y = x @ w^T; weight gradients are [out, in] float32.
 *  - bf16 = bfloat16 (uint16 storage).  Every pointer is a device pointer unless said otherwise.
 *  - Ownership: the caller owns every buffer.  The library never allocates device memory; calls
 *    that need scratch space take a workspace sized by the matching *_workspace_bytes function.
 *  - Execution: every call enqueues work on `stream` and returns without waiting, except
 *    collider_index_count_host, which waits for one 4-byte copy.
 *  - Errors: arguments are checked on the host before anything is enqueued; a failed check returns
 *    a non-zero status and enqueues nothing.  A failed launch returns COLLIDER_ERR_HIP and leaves
 *    the outputs undefined.  Nothing throws across this interface.
 *  - Alignment: every bf16 tensor pointer must be 16-byte aligned and every bf16 leading dimension
 *    a multiple of 8 elements (COLLIDER_ERR_ALIGN otherwise).
 */
#ifndef COLLIDER_H
#define COLLIDER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  COLLIDER_OK = 0,
  COLLIDER_ERR_NULL = 1,        /* a required pointer is NULL */
  COLLIDER_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  COLLIDER_ERR_ALIGN = 3,       /* pointer / leading-dimension alignment violated */
  COLLIDER_ERR_UNSUPPORTED = 4, /* valid but not implemented (head_dim, dtype, ...) */
  COLLIDER_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  COLLIDER_ERR_HIP = 6          /* a HIP runtime call failed */
} collider_status;

typedef enum { COLLIDER_F32 = 0, COLLIDER_BF16 = 1 } collider_dtype;

/* Softmax-backward row term of the filtered attention backward.  The pages do not fix it.
 *  FILTERED: D~_i = sum_j P~_ij dP_ij over kept keys j (P~ = P with filtered-token columns
 *            removed) - the ordinary softmax backward run on the filtered activation; needs an
 *            extra pass over the kept pairs.
 *  FULL:     D_i = dO_i . O_i with the forward output O (the full softmax's identity). */
typedef enum { COLLIDER_ATTN_D_FILTERED = 0, COLLIDER_ATTN_D_FULL = 1 } collider_dmode;

/* Compacted index of a keep mask, produced by collider_build_index.  All arrays device-resident. */
typedef struct {
  const int32_t* idx;        /* [M]: idx[c], c < count, = c-th kept position (ascending);
                                entries c >= count list the filtered positions ascending */
  const int32_t* inv;        /* [M]: inv[t] = c if token t is kept, else -1 */
  const int32_t* cu_seqlens; /* [B+1]: kept tokens before sequence b; cu_seqlens[B] = count */
  const int32_t* count;      /* [1]: number of kept tokens M_kept */
  int32_t B, S;              /* batch and sequence length, M = B*S */
  int32_t M_kept;            /* host copy of *count (collider_index_count_host) */
} collider_index;

/* ---------------------------------------------------------------------------------------------
 * Mask -> index.  Backward token filtering selects tokens one by one (Figure 2(b)); the kept
 * tokens are what the dimension-reduced GEMMs run over (abstract).
 * keep: [B*S] bytes, non-zero = kept.  Outputs idx, inv [B*S], cu_seqlens [B+1], count [1] int32.
 * Deterministic; bit-exact.  B >= 1, S >= 1, B*S <= 2^30.
 * ------------------------------------------------------------------------------------------- */
collider_status collider_build_index(const uint8_t* keep, int32_t B, int32_t S, int32_t* idx,
                                     int32_t* inv, int32_t* cu_seqlens, int32_t* count,
                                     hipStream_t stream);

/* Mask -> index when the caller already knows how many tokens the mask keeps (a filter that keeps
 * a fixed number of tokens per batch, such as a top-k on per-token scores): the same outputs as
 * collider_build_index, without the host wait for the count.  expected_count becomes M_kept of the
 * index; on the device, compacted positions >= expected_count are left out of inv (-1) and
 * cu_seqlens (clamped), so that every consumer sized for expected_count rows stays in bounds
 * whatever the mask holds.  *mismatch (device int32, written by every call) = 1 if the mask keeps
 * another number of tokens - the gradients computed from such an index are then not the filtered
 * gradient and must be discarded - else 0; *count holds the true count either way.  On a mismatch
 * every output of a call that used the index is unspecified but the call stays within its buffers,
 * and collider_layer_bwd writes each full-layout dx row from one kernel only (the rows past the
 * true count are left to the zero fill of filtered rows).
 * COLLIDER_ERR_SHAPE if expected_count < 0 or > B*S; COLLIDER_ERR_NULL for a null pointer. */
collider_status collider_build_index_expect(const uint8_t* keep, int32_t B, int32_t S,
                                            int32_t expected_count, int32_t* idx, int32_t* inv,
                                            int32_t* cu_seqlens, int32_t* count, int32_t* mismatch,
                                            hipStream_t stream);

/* Copies *count_dev to *count_host (host pointer) and waits for it: the one host sync of a step. */
collider_status collider_index_count_host(const int32_t* count_dev, int32_t* count_host,
                                          hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Row gather (dimension reduction, abstract): dst[c, :] = src[idx[c], :] for c < n_rows.
 * row_elems elements of type dt per row; ld_* are row strides in elements.  Bit-exact copy.
 * ------------------------------------------------------------------------------------------- */
collider_status collider_gather_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                                     const int32_t* idx, int32_t n_rows, int32_t row_elems,
                                     collider_dtype dt, hipStream_t stream);

/* Row scatter back to the full token layout, for t < M:
 *   dst[t, :] = src[inv[t], :] if inv[t] >= 0; else +0.0 (zero_fill_filtered != 0, any non-zero
 *   value) or untouched (zero_fill_filtered == 0).
 * The rows of filtered tokens therefore stay exactly zero (abstract: sparsity is maintained). */
collider_status collider_scatter_rows(const void* src, int64_t ld_src, void* dst, int64_t ld_dst,
                                      const int32_t* inv, int32_t M, int32_t row_elems,
                                      int32_t zero_fill_filtered, collider_dtype dt,
                                      hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Linear-layer backward as dimension-reduced dense GEMMs (abstract) over M_kept compacted rows:
 *   dx = dy @ w        [M_kept, K]  (dtype dt; skipped when dx == NULL)
 *   dw = dy^T @ x      [N, K] float32 (overwritten, or added to when accumulate != 0)
 *   db = colsum(dy)    [N] float32 (optional, NULL to skip; same accumulate rule)
 * x [M_kept, K] (row stride ld_x), dy [M_kept, N] (ld_dy), w [N, K] dense, all of dtype dt
 * (COLLIDER_BF16: bf16 operands, fp32 accumulation; COLLIDER_F32: fp32 throughout).
 * M_kept = 0 gives dw = 0, db = 0.  With COLLIDER_BF16 the workspace also holds x transposed
 * (K x M_kept rounded up to 64, bf16), which the dw GEMM reads along the token reduction.
 * ------------------------------------------------------------------------------------------- */
size_t collider_linear_workspace_bytes(collider_dtype dt, int32_t M_kept, int32_t K, int32_t N);
collider_status collider_linear_bwd_reduced(collider_dtype dt, int32_t M_kept, int32_t K, int32_t N,
                                            const void* x, int64_t ld_x, const void* dy,
                                            int64_t ld_dy, const void* w, void* dx, float* dw,
                                            float* db, int32_t accumulate, void* ws,
                                            size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Filtered attention backward (Figures 3 and 5), causal, grouped-query, over compacted rows.
 * For each sequence b (rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the compacted tensors) and
 * query head h (KV head g = h / (nq/nkv)), with tau = softmax scale, for kept i >= j:
 *   P_ij = exp(tau q_i.k_j - lse_i)  (lse from the forward, over ALL causal keys, filtered too)
 *   dV_j = sum_i P_ij dO_i,  dP_ij = dO_i.v_j,  dS_ij = P_ij (dP_ij - D_i)  (D per dmode)
 *   dq_i = tau sum_j dS_ij k_j,  dk_j = tau sum_i dS_ij q_i, dK/dV summed over each KV group,
 * then the rotary-embedding backward on dq, dk (rotate-half on the first rot_dims dims of each
 * head, angle = pos * rope_base^(-2m/rot_dims), pos = idx[c] mod S).  Filtered keys never enter:
 * that is the removal of their softmax-activation columns.  q, k are post-rotary.
 * Inputs bf16 (lse float32 [M_kept, nq] natural-log); outputs bf16, each with its row stride.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
  int32_t n_q_heads, n_kv_heads, head_dim; /* head_dim 64 or 128; n_q_heads % n_kv_heads == 0 */
  int32_t rot_dims;                        /* 0 = no rotary; even, <= head_dim */
  float rope_base;
  float softmax_scale;                     /* 0 = 1/sqrt(head_dim) */
  int32_t dmode;                           /* collider_dmode */
} collider_attn_cfg;

typedef struct {
  const void* q; int64_t ld_q;     /* [M_kept, nq*d]  */
  const void* k; int64_t ld_k;     /* [M_kept, nkv*d] */
  const void* v; int64_t ld_v;     /* [M_kept, nkv*d] */
  const void* o; int64_t ld_o;     /* [M_kept, nq*d] forward output: required with
                                      COLLIDER_ATTN_D_FULL; optional with FILTERED, where it only
                                      improves the rounding of dq (NULL allowed) */
  const float* lse; int64_t ld_lse;/* [M_kept, nq] float32 */
  const void* dout; int64_t ld_do; /* [M_kept, nq*d] gradient of o */
  void* dq; int64_t ld_dq;         /* [M_kept, nq*d] out */
  void* dk; int64_t ld_dk;         /* [M_kept, nkv*d] out */
  void* dv; int64_t ld_dv;         /* [M_kept, nkv*d] out */
} collider_attn_io;

size_t collider_attn_workspace_bytes(const collider_attn_cfg* cfg, const collider_index* ix);
collider_status collider_attn_bwd_filtered(const collider_attn_cfg* cfg, const collider_index* ix,
                                           const collider_attn_io* io, void* ws, size_t ws_bytes,
                                           hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Whole-layer filtered backward (abstract: activations of filtered tokens filtered in every layer).
 * LLAMA: x -> RMSNorm(gamma1) -> QKV -> rotary -> causal GQA attention -> O; h = x + attn;
 *        h -> RMSNorm(gamma2) -> [gate|up] -> silu(gate)*up -> down; y = h + mlp.
 * PHI:   xn = LayerNorm(x; gamma, beta); y = x + O(attn(QKV(xn))) + fc2(gelu_tanh(fc1(xn))).
 * The upstream gradient rows of filtered tokens are never read (their loss is dropped, Figure
 * 2(b)); every GEMM runs over the M_kept kept rows; weight / gain gradients are sums over kept
 * tokens only; dx rows of filtered tokens are +0.0 (or absent when dx_compact != 0).
 * ------------------------------------------------------------------------------------------- */
typedef enum { COLLIDER_LAYER_LLAMA = 0, COLLIDER_LAYER_PHI = 1 } collider_layer_kind;

typedef struct {
  int32_t kind;                 /* collider_layer_kind */
  int32_t hidden;               /* H, multiple of 8 */
  int32_t n_q_heads, n_kv_heads, head_dim, rot_dims;
  int32_t inter;                /* I, multiple of 8 */
  float rope_base;
  int32_t dmode;                /* collider_dmode */
  int32_t accumulate;           /* != 0: weight / gain gradients are added to, not overwritten */
  int32_t unfiltered;           /* != 0: the ordinary dense backward over all M tokens, the baseline
                                   the method is measured against: the index arrays are not read
                                   (only B, S), nothing is gathered or scattered, every GEMM and
                                   the attention run on the full layout, dmode is taken as FULL */
  int32_t weight_layout;        /* collider_weight_layout: how the projection weights and their
                                   gradients are stored */
} collider_layer_cfg;

/* COLLIDER_WEIGHTS_OUT_IN: w [out, in], y = x w^T (torch nn.Linear), the layouts listed below.
 * COLLIDER_WEIGHTS_IN_OUT: W [in, out], y = x W (the notation of the Collider pages, dX = dY W^T):
 * every projection weight and its gradient is the transpose of the OUT_IN one - W_qkv [H, nqkv]
 * (q columns, then k, then v), W_o [nq*d, H], W_gateup [H, 2I] (gate columns then up), W_down
 * [I, H]; PHI: W_fc1 [H, I], W_fc2 [I, H] (the PHI layer then stacks W_qkv and W_fc1 into one
 * [H, nqkv + I] matrix in its workspace each call).  With IN_OUT each weight row is contiguous along the reduction of the activation-gradient
 * GEMM, so both of its operands are read with 16-byte LDS reads (OUT_IN needs the transposing
 * 8-byte reads, a third of the LDS bandwidth). */
typedef enum { COLLIDER_WEIGHTS_OUT_IN = 0, COLLIDER_WEIGHTS_IN_OUT = 1 } collider_weight_layout;

typedef struct {                /* bf16 weights, shapes for COLLIDER_WEIGHTS_OUT_IN (IN_OUT: the
                                   transposes); float32 norm parameters */
  const void* w_qkv;            /* [(nq+2nkv)*d, H]: q rows, then k, then v */
  const void* w_o;              /* [H, nq*d] */
  const void* w_gateup;         /* LLAMA [2I, H]: gate rows then up rows */
  const void* w_down;           /* LLAMA [H, I] */
  const void* w_fc1;            /* PHI [I, H] */
  const void* w_fc2;            /* PHI [H, I] */
  const float* gamma1;          /* LLAMA first RMSNorm gain [H] */
  const float* gamma2;          /* LLAMA second RMSNorm gain [H] */
  const float* ln_gamma;        /* PHI LayerNorm gain [H] */
  const float* ln_beta;         /* PHI LayerNorm bias [H] */
} collider_layer_weights;

typedef struct {                /* forward activations, full token layout [M, ...] */
  const void* x;                /* bf16 [M, H] layer input */
  const void* q;                /* bf16 [M, nq*d] post-rotary */
  const void* k;                /* bf16 [M, nkv*d] post-rotary */
  const void* v;                /* bf16 [M, nkv*d] */
  const void* o;                /* bf16 [M, nq*d] attention output (input of w_o) */
  const float* lse;             /* [M, nq] */
  const float* rstd1;           /* LLAMA: first RMSNorm 1/rms [M]; PHI: LayerNorm 1/std [M] */
  const float* mean;            /* PHI LayerNorm mean [M] */
  const void* h;                /* LLAMA bf16 [M, H] = x + attention output */
  const float* rstd2;           /* LLAMA second RMSNorm [M] */
  const void* gate;             /* LLAMA bf16 [M, I] */
  const void* up;               /* LLAMA bf16 [M, I] */
  const void* f;                /* PHI bf16 [M, I] fc1 pre-activation */
} collider_layer_saved;

typedef struct {                /* outputs (weight gradients in the weights' layout) */
  void* dx;                     /* bf16 [M, H] (dx_compact = 0) or [M_kept, H] (dx_compact != 0) */
  float* dw_qkv;                /* [(nq+2nkv)*d, H] */
  float* dw_o;                  /* [H, nq*d] */
  float* dw_gateup;             /* LLAMA [2I, H] */
  float* dw_down;               /* LLAMA [H, I] */
  float* dw_fc1;                /* PHI [I, H] */
  float* dw_fc2;                /* PHI [H, I] */
  float* dgamma1;               /* LLAMA [H] */
  float* dgamma2;               /* LLAMA [H] */
  float* dln_gamma;             /* PHI [H] */
  float* dln_beta;              /* PHI [H] */
} collider_layer_grads;

/* dy: bf16 [M, H] (dy_compact = 0) or already compacted [M_kept, H] (dy_compact != 0, e.g. the
 * dx of the layer above produced with dx_compact != 0).  The workspace must not alias any input
 * or output.  An index with M_kept = B*S (every token kept: its partition is the identity) runs the
 * dense path of unfiltered = 1, with the same results and no gather or index lookups; the
 * workspace size is queried with the same M_kept, so it follows. */
size_t collider_layer_workspace_bytes(const collider_layer_cfg* cfg, int32_t B, int32_t S,
                                      int32_t M_kept);
collider_status collider_layer_bwd(const collider_layer_cfg* cfg, const collider_layer_weights* w,
                                   const collider_layer_saved* saved, const void* dy,
                                   int32_t dy_compact, const collider_index* ix,
                                   collider_layer_grads* grads, int32_t dx_compact, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Loss side of the backward (Figure 2(b): the per-token training loss decides which tokens are
 * filtered; a filtered token's loss is dropped, so it sends no gradient into the LM head, the
 * layers or the token embedding).
 *
 * collider_ce_loss: per-token cross-entropy loss of every token from the LM head's logits (bf16
 * [M, V], row stride ld_logits, full token layout) and labels (int32 [M]):
 *   loss[t] = logsumexp(logits_t) - logits_t[labels[t]]   (natural log, float32 [M])
 *   loss[t] = 0 when labels[t] is outside [0, V) (no target, e.g. torch's ignore index -100).
 * This is the score token selection ranks by (collider_select_keep on `loss` keeps the tokens
 * with the largest loss).  Max and exp-sum in float32, one pass over each row; logits equal to
 * -inf (masked vocabulary entries) contribute nothing.  V and ld_logits multiples of 8, logits
 * 16-byte aligned (COLLIDER_ERR_ALIGN); M in [1, 2^30] (COLLIDER_ERR_SHAPE); NULL pointers
 * COLLIDER_ERR_NULL. */
collider_status collider_ce_loss(const void* logits, int64_t ld_logits, const int32_t* labels,
                                 int32_t M, int32_t V, float* loss, hipStream_t stream);

/*
 * collider_select_keep: token selection on per-token scores (float32 [M], e.g. the per-token loss
 * or any importance score).  keep[t] = 1 for the n_keep tokens with the largest score, else 0;
 * equal scores keep the lower position first; -0.0 ranks as +0.0; NaN ranks below every number.
 * n_keep <= 0 keeps nothing, n_keep >= M keeps every token.  keep is uint8 [M] (the mask
 * collider_build_index takes).  One workgroup, five passes over the scores: meant for per-batch
 * token counts (M <= 2^30 accepted; time grows linearly with M; collider_select_keep_ws below
 * spreads large counts over the GPU).  Bit-exact, deterministic.
 * Errors: NULL pointer, M < 1 or M > 2^30.
 * ------------------------------------------------------------------------------------------- */
collider_status collider_select_keep(const float* score, int32_t M, int32_t n_keep, uint8_t* keep,
                                     hipStream_t stream);

/* collider_select_keep_ws: the same selection, bit for bit, spread over many workgroups for large
 * token counts: four radix passes, each a histogram launch over contiguous chunks of the scores
 * and a one-workgroup launch that picks the next key byte, then a count of the threshold-equal
 * keys per chunk and the mask launch.  ws: 16-byte aligned device memory of
 * collider_select_workspace_bytes(M) bytes (0 for M <= 8192, where the one-workgroup kernel of
 * collider_select_keep runs; about 1 KB per 4096 tokens above it, at most 2 MB plus 8 KB), owned
 * by the caller, not kept after the call's work on `stream` ends; calls that share it must be
 * ordered.  Errors: NULL score or keep, M < 1 or M > 2^30, ws NULL or smaller than required,
 * ws not 16-byte aligned.
 * ------------------------------------------------------------------------------------------- */
size_t collider_select_workspace_bytes(int32_t M);
collider_status collider_select_keep_ws(const float* score, int32_t M, int32_t n_keep, uint8_t* keep,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/* collider_lm_head_bwd: per-token cross-entropy backward through the LM head, over kept tokens.
 * The forward computed logits = h @ w_lm^T (w_lm [V, H] bf16, [out, in]) and kept them, bf16
 * [M, V] in the full token layout (row stride ld_logits).  The loss is
 *   L = loss_scale * sum over kept t with 0 <= labels[t] < V of (logsumexp(logits_t) - logits_t[labels[t]])
 * (loss_scale = 1 / M_kept gives the mean over kept tokens; a label outside [0, V), such as
 * torch's ignore index -100, marks a token without a target).  Computes, for kept rows only:
 *   dlogits' = loss_scale * (softmax(logits') - onehot(labels'))   (bf16, in the workspace)
 *   dh' = dlogits' @ w_lm            -> dh: bf16 [M_kept, H] (dh_compact != 0; may be NULL when
 *                                       M_kept = 0) or [M, H] with the rows of filtered tokens +0.0
 *                                       (dh_compact == 0)
 *   dw_lm = dlogits'^T @ h'          -> float32 [V, H], overwritten (accumulate == 0) or added to
 * h is the bf16 [M, H] input of the LM head (full layout, row stride ld_h); labels int32 [M].
 * Requirements: H and V multiples of 8, 16-byte alignment of every bf16 pointer and leading
 * dimension (COLLIDER_ERR_ALIGN otherwise), ix from collider_build_index with M_kept set.
 * The workspace (collider_lm_head_workspace_bytes) holds h' transposed ([H, M_kept rounded up to
 * 64] bf16, the weight gradient's operand with its tokens contiguous), dlogits' ([M_kept, V] bf16)
 * and GEMM partials; it must not alias any input or output. */
size_t collider_lm_head_workspace_bytes(int32_t M_kept, int32_t H, int32_t V);
collider_status collider_lm_head_bwd(const void* logits, int64_t ld_logits, const int32_t* labels,
                                     const void* h, int64_t ld_h, const void* w_lm,
                                     const collider_index* ix, int32_t H, int32_t V,
                                     float loss_scale, void* dh, int32_t dh_compact, float* dw_lm,
                                     int32_t accumulate, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* collider_embedding_bwd: gradient of the token embedding table E [V, H] under x_t = E[ids[t]]:
 *   dE[v, :] = sum of dx[t, :] over the kept tokens t with ids[t] == v, summed in ascending t
 * (deterministic: the kept tokens are bucketed by id with a stable counting sort, then each row
 * is summed by one wavefront; no float atomics).  dx is bf16: compacted [M_kept, H] (dx_compact
 * != 0, e.g. the bottom layer's compact dx) or the full [M, H] layout (read at idx rows); ids is
 * int32 [M]; dE is float32 [V, H], every row written (rows no kept token uses: 0) unless
 * accumulate != 0 (then added to, and untouched rows left as they are).  Ids outside [0, V) are
 * skipped.  H a multiple of 8, 16-byte alignment as above.  Workspace:
 * collider_embedding_workspace_bytes. */
size_t collider_embedding_workspace_bytes(int32_t M_kept, int32_t V);
collider_status collider_embedding_bwd(const void* dx, int64_t ld_dx, int32_t dx_compact,
                                       const int32_t* ids, const collider_index* ix, int32_t H,
                                       int32_t V, float* dE, int32_t accumulate, void* ws,
                                       size_t ws_bytes, hipStream_t stream);

/* collider_embedding_bwd_noalloc: collider_embedding_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
 * same arguments without the workspace, the same kernels and the same result bit for bit; the
 * counting sort's scratch (per-id counts, offsets and cursors, the sorted token list) lives in a
 * library-owned device array of 7 MiB per GPU, held until the process ends.  Limits: V <=
 * 262144 and M_kept <= 1048576, else COLLIDER_ERR_WORKSPACE (nothing enqueued).  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).  Every call on a GPU
 * shares that GPU's scratch array and clears what it needs itself: calls that overlap on one GPU
 * (on different streams, or from several host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.  Other errors as collider_embedding_bwd. */
collider_status collider_embedding_bwd_noalloc(const void* dx, int64_t ld_dx, int32_t dx_compact,
                                               const int32_t* ids, const collider_index* ix,
                                               int32_t H, int32_t V, float* dE, int32_t accumulate,
                                               hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Measurement and diagnostics.
 * collider_profile_enable(1): from then on every kernel the library enqueues from the calling host
 * thread is bracketed by a pair of HIP events recorded on the same stream (the switch is per host
 * thread; other threads' launches are not timed).  collider_profile_collect waits for them and,
 * for each kernel name, returns the summed duration (ms) and the number of launches; it then
 * clears the record.  names receives up to max_kernels NUL-separated names (name_cap bytes).
 * Returns the number of distinct kernels, or -1 on error.
 * ------------------------------------------------------------------------------------------- */
collider_status collider_profile_enable(int32_t on);

/* Work decomposition of the bf16 GEMMs (a tuning and test control; results of every policy meet
 * the same tolerance, and each policy is deterministic):
 *   0  default: a cost model picks the tile shape and whole tiles, K-splits or stream-K;
 *   1  whole tiles and K-splits only;   2  stream-K wherever the direct-to-LDS kernel applies;
 *   3  whole tiles only.
 * Per host thread: it applies to the calls (and *_workspace_bytes queries) the calling thread
 * makes afterwards, and never to another thread's.  Workspace sizes depend on it: query
 * *_workspace_bytes after setting it.  Returns COLLIDER_ERR_SHAPE for any other value. */
collider_status collider_gemm_set_policy(int32_t policy);

/* The work decomposition the current policy picks for one bf16 GEMM C[M, N] = A B with reduction
 * length K, on the current device (host only, launches nothing).  layout 0: dX = dY w (A [M, K]
 * K-contiguous, B [K, N] N-contiguous, bf16 C); layout 1: dW = dY^T X (A and B token-major, fp32 C).
 * concurrent != 0: the plan for GEMMs that run beside another stream (the layer's).  out[7] receives
 * tile rows, tile columns, K-splits, whole tiles, stream-K tiles, workgroups, and 1 when the
 * direct-to-LDS kernel runs (0: register-staged).  COLLIDER_ERR_SHAPE for M or N <= 0, K < 0 or
 * N % 8 != 0; COLLIDER_ERR_NULL for out == NULL. */
collider_status collider_gemm_describe_plan(int32_t M, int32_t N, int32_t K, int32_t layout,
                                           int32_t concurrent, int32_t* out);
int32_t collider_profile_collect(char* names, int32_t name_cap, double* total_ms, int32_t* launches,
                                 int32_t max_kernels);

/* Library-held HIP objects.  collider_layer_bwd forks part of its work onto a side stream (default
 * priority) and joins it back to the caller's stream with events (created without the system-scope
 * fence: they only order the two streams; the host sees the results after synchronizing the
 * caller's stream, as for any work on it); it leases the stream and its events from a per-device
 * pool for the duration of one call and returns them when its launches are enqueued, so the pool
 * holds as many sets as calls have ever run at once on a device, however many host threads call
 * (a set still part of an open graph capture is not leased again until that capture ends).
 * collider_side_streams_live returns the number of sets alive (leased or idle, all devices).
 * collider_release_resources destroys every idle set and the pooled timing events (the next call
 * creates what it needs again); call it before unloading the library.  Sets leased by calls in
 * progress on other threads are left alone. */
int32_t collider_side_streams_live(void);
collider_status collider_release_resources(void);
const char* collider_status_string(collider_status s);

#ifdef __cplusplus
}
#endif
#endif /* COLLIDER_H */

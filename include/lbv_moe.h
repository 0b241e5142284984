/*
 * lbv_moe.h: C ABI of the routed-MoE feed-forward block of the LingBot-Video
 * MoE diffusion transformer, for AMD Instinct MI355X (gfx950).
 *
 * The block (sources: prhub.com.cn summary of sglang PR #32341, section
 * "实现拆解" step 1 and the excerpt of LingBotVideoSparseMoeBlock; the vLLM-Omni
 * LingBot-Video article, section "MoE 实现的源码级要点"):
 *
 *   tokens x [T, H]
 *   router (fp32): z = x W_r^T, s = sigmoid(z), c = s + e_score_correction_bias;
 *     group score = sum of the two largest c of each of n_group groups, keep
 *     the topk_group best groups, pick the top_k largest c inside them;
 *     weight_k = s[id_k] (raw score, no bias), divided by the sum over the
 *     chosen experts when norm_topk_prob, times routed_scaling_factor (once).
 *   experts: f_e(x) = W2_e (silu(W1_e x) * (W3_e x)), with W1 and W3 packed
 *     as w13_e = [W1_e; W3_e] (gate rows first, then up rows; not interleaved).
 *   out = sum_k weight_k f_{id_k}(x)  +  shared(x)   (the weight multiplies the
 *     expert output; the expert side applies no further scaling).
 *
 * Conventions shared by every call:
 *  - Ownership: the caller owns every buffer.  `cfg` points to host memory;
 *    every other pointer is device memory.  The library never allocates,
 *    frees or synchronises; each call only enqueues kernels on `stream`.
 *  - Errors: arguments are validated before anything is enqueued; a failed
 *    check returns a non-zero status and has no side effect.  A failed launch
 *    returns LBV_ERR_HIP.  Device-side faults surface at the caller's next
 *    synchronisation.  T == 0 is a successful no-op once the configuration
 *    is valid (no pointer is looked at, nothing is enqueued).
 *  - Layout: row-major, densely packed.  Pointers must be 16-byte aligned;
 *    hidden and intermediate must be multiples of 64.  With bf16 storage, x
 *    and each packed gate/up weight (one routed expert's w13, or shared_w13)
 *    must each be smaller than 4 GiB (LBV_ERR_SHAPE otherwise).
 *  - Precision: the router weight, correction bias, routing weights and all
 *    router arithmetic are fp32.  x, expert weights, `act` and `out` use
 *    `cfg->dtype` (bf16 or fp32); expert matmuls accumulate in fp32; the
 *    combine sums in fp32 and rounds once to the output type.
 *  - Padding: `mask` (u8 [T], NULL = all valid) marks padding tokens with 0.
 *    A padding token gets no routed expert (ids -1, weight 0) and its output
 *    is the shared expert alone.
 *  - Shared experts: n_shared_experts > 0 means one SwiGLU MLP of width
 *    I_s = intermediate * n_shared_experts with weight 1, packed as
 *    shared_w13 [2 I_s, H] (gate rows then up rows) and shared_w2 [H, I_s].
 *    Internally it runs as n_shared_experts pseudo-experts of width I.
 *  - Threading: calls keep no state; concurrent calls on different buffers
 *    are safe.
 */
#ifndef LBV_MOE_H
#define LBV_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LBV_OK = 0,
    LBV_ERR_NULL = 1,         /* a required pointer is NULL                        */
    LBV_ERR_SHAPE = 2,        /* a size or config field is out of range           */
    LBV_ERR_UNSUPPORTED = 3,  /* valid on the pages but not built here            */
    LBV_ERR_ALIAS = 4,        /* out overlaps x (the block is not in-place)        */
    LBV_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned                 */
    LBV_ERR_WORKSPACE = 6,    /* ws_bytes smaller than the size query returns     */
    LBV_ERR_HIP = 7           /* a kernel launch failed                           */
} lbv_status;

typedef enum { LBV_F32 = 0, LBV_BF16 = 1 } lbv_dtype;
typedef enum { LBV_SCORE_SIGMOID = 0, LBV_SCORE_SOFTMAX = 1 } lbv_score_func;

/*
 * Layer configuration (the constructor arguments of LingBotVideoSparseMoeBlock
 * in the PR #32341 excerpt).  LingBot-Video MoE 30B: hidden 2048,
 * num_experts 128, top_k 8, n_group 4, topk_group 2, intermediate 768,
 * n_shared_experts 1, norm_topk_prob 1, routed_scaling_factor 2.5, sigmoid.
 * Built here: sigmoid scores only; num_experts <= 256; top_k <= 16;
 * n_shared_experts <= 8; with P = the smallest power of two such that
 * 64 P >= num_experts, the group size num_experts / n_group must be >= 2, a
 * multiple of P, and (group size / P) a power of two.
 */
typedef struct {
    int32_t hidden;                  /* H                                   */
    int32_t num_experts;             /* E                                   */
    int32_t top_k;                   /* K                                   */
    int32_t n_group;
    int32_t topk_group;
    int32_t intermediate;            /* I, width of one routed expert        */
    int32_t n_shared_experts;        /* ns                                  */
    int32_t norm_topk_prob;          /* 0 or 1                              */
    float routed_scaling_factor;
    int32_t score_func;              /* lbv_score_func                      */
    int32_t dtype;                   /* lbv_dtype                           */
} lbv_moe_config;

/* Version of this ABI (bumped on any signature or layout change). */
int32_t lbv_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char *lbv_status_string(lbv_status status);

/* Checks a configuration without touching any device state. */
lbv_status lbv_moe_check_config(const lbv_moe_config *cfg);

/*
 * Workspace sizes in bytes.
 *   lbv_moe_workspace_size:          for lbv_moe_forward;
 *   lbv_moe_route_workspace_size:    for lbv_moe_route (does not depend on T;
 *                                    on the bf16 path 3 E H bf16 values, rounded
 *                                    up to 256 bytes, plus 4 x 4096 x EP fp32
 *                                    partial logits for calls of at most 4096
 *                                    tokens, EP = 64 if E <= 64 else 128; else 0);
 *   lbv_moe_permute_workspace_size:  for lbv_moe_permute;
 *   lbv_moe_w2_workspace_size:       for lbv_moe_gemm_w2_combine.
 * Sizes grow linearly with T (the forward one is dominated by the bf16 expert
 * output buffer, T (K + ns) H elements).
 */
lbv_status lbv_moe_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);
lbv_status lbv_moe_route_workspace_size(const lbv_moe_config *cfg, size_t *bytes);
lbv_status lbv_moe_permute_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);
lbv_status lbv_moe_w2_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);

/*
 * Router (PR #32341 summary, "实现拆解" step 1 and risk 4 under "风险与影响";
 * vLLM-Omni article, "MoE 实现的源码级要点").
 *   x        [T, H]   cfg->dtype
 *   router_w [E, H]   fp32
 *   e_bias   [E]      fp32, e_score_correction_bias (selection only)
 *   mask     [T]      u8 or NULL
 *   topk_ids [T, K]   int32 out: expert ids, slots ordered by biased score
 *                     descending then id ascending; -1 for padding tokens
 *   topk_w   [T, K]   fp32 out: routing weights, already scaled by
 *                     routed_scaling_factor; 0 for padding tokens
 *   ws, ws_bytes      scratch of lbv_moe_route_workspace_size bytes (may be
 *                     NULL when that size is 0).  With bf16 x the router
 *                     weight is split there into three bf16 planes whose sum
 *                     is exactly W_r, so the fp32 logits run on the bf16
 *                     matrix cores; finite W_r entries must stay below the
 *                     bf16 overflow threshold (about 3.39e38).  Calls of at
 *                     most 4096 tokens also keep partial logits there.
 * Ties between equal scores go to the lower group / expert index.
 */
lbv_status lbv_moe_route(const lbv_moe_config *cfg, int64_t T, const void *x,
                         const float *router_w, const float *e_bias, const uint8_t *mask,
                         int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Token-to-expert permutation (vLLM-Omni article, "MoE 实现的源码级要点":
 * token copies reordered by expert before the grouped matmuls).
 * A slot is (t, k) for k < K (routed) and (t, K + j) for j < ns (shared
 * pseudo-expert j); its id is t * (K + ns) + k.  Segments s = 0..E-1 are the
 * routed experts, s = E + j the shared pseudo-experts.
 *   topk_ids    [T, K]        int32 in.  Ids outside [0, E), and repeats of an
 *                             id already seen earlier in the same token, are
 *                             treated as "not routed".
 *   offsets     [E + ns + 1]  int32 out: segment s owns sorted rows
 *                             [offsets[s], offsets[s+1]); offsets[E+ns] = R,
 *                             the number of rows.
 *   sorted_rows [T (K + ns)]  int32 out: slot id of each sorted row (first R
 *                             entries); inside a segment rows follow slot id
 *                             order (a stable counting sort by expert).
 *   inv_rows    [T (K + ns)]  int32 out: sorted row of each slot, -1 for a
 *                             slot that is not routed.
 *   ws, ws_bytes              scratch, lbv_moe_permute_workspace_size bytes.
 */
lbv_status lbv_moe_permute(const lbv_moe_config *cfg, int64_t T, const int32_t *topk_ids,
                           int32_t *offsets, int32_t *sorted_rows, int32_t *inv_rows,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped gate/up matmul with fused SiLU gating (PR #32341 summary, runner
 * flags in the excerpt: silu, gated, gate and up not interleaved).  For every
 * sorted row r of segment s with slot id q and token t = q / (K + ns):
 *   act[r, i] = silu(g_i) * u_i,  g = W_gate_s x[t],  u = W_up_s x[t],
 * where for a routed expert W_gate = w13[s][0:I], W_up = w13[s][I:2I], and for
 * shared pseudo-expert j W_gate = shared_w13[jI:(j+1)I],
 * W_up = shared_w13[I_s + jI : I_s + (j+1)I].  fp32 accumulation, act rounded
 * once to cfg->dtype.
 *   x [T, H]; w13 [E, 2I, H]; shared_w13 [2 I_s, H] (NULL iff ns == 0);
 *   offsets, sorted_rows from lbv_moe_permute;
 *   act [T (K + ns), I] out (rows [0, R) written).
 */
lbv_status lbv_moe_gemm_w13_silu(const lbv_moe_config *cfg, int64_t T, const void *x,
                                 const void *w13, const void *shared_w13,
                                 const int32_t *offsets, const int32_t *sorted_rows,
                                 void *act, hipStream_t stream);

/*
 * Grouped down projection and weighted combine (PR #32341 summary, excerpt:
 * router weight applied on the output, no second scaling, shared expert added;
 * vLLM-Omni article: fp32 weighted restore).  Per sorted row r of segment s:
 * y_r = W2_s act[r] (W2_s = w2[s] for a routed expert, columns [jI,(j+1)I) of
 * shared_w2 for shared pseudo-expert j), stored in cfg->dtype; then per token
 *   out[t] = round( sum_k topk_w[t,k] * y[inv(t,k)] + sum_j y[inv(t,K+j)] )
 * summed in fp32 in slot order and rounded once to cfg->dtype.
 *   act [T (K + ns), I]; w2 [E, H, I]; shared_w2 [H, I_s] (NULL iff ns == 0);
 *   offsets, sorted_rows, inv_rows from lbv_moe_permute; topk_w [T, K];
 *   out [T, H]; ws, ws_bytes: lbv_moe_w2_workspace_size bytes.
 */
lbv_status lbv_moe_gemm_w2_combine(const lbv_moe_config *cfg, int64_t T, const void *act,
                                   const void *w2, const void *shared_w2,
                                   const int32_t *offsets, const int32_t *sorted_rows,
                                   const int32_t *inv_rows, const float *topk_w, void *out,
                                   void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The whole block (PR #32341 summary, LingBotVideoSparseMoeBlock.forward):
 * route, permute, gate/up + SiLU, down + combine, on `stream`, no host sync.
 *   x [T, H]; mask [T] or NULL; router_w [E, H]; e_bias [E]; w13 [E, 2I, H];
 *   w2 [E, H, I]; shared_w13 [2 I_s, H] and shared_w2 [H, I_s] (NULL iff
 *   ns == 0); out [T, H] (must not overlap x);
 *   topk_ids_out [T, K], topk_w_out [T, K]: optional copies of the routing
 *   (NULL to skip);
 *   ws, ws_bytes: lbv_moe_workspace_size bytes.
 */
lbv_status lbv_moe_forward(const lbv_moe_config *cfg, int64_t T, const void *x,
                           const uint8_t *mask, const float *router_w, const float *e_bias,
                           const void *w13, const void *w2, const void *shared_w13,
                           const void *shared_w2, void *out, int32_t *topk_ids_out,
                           float *topk_w_out, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LBV_MOE_H */

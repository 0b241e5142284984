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
    LBV_ERR_HIP = 7,          /* a kernel launch failed                           */
    LBV_ERR_SCRATCH = 8       /* an allocation-free call's fixed scratch is too small */
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

/* Version of this ABI (bumped on any signature or layout change; 2: the
 * gate/up call takes a workspace; 3: fp8 expert weights; 4: the attention
 * half; 5: the attention half with its AdaLN and gated residual). */
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
 *                                    up to 256 bytes, plus 4096 x EP fp32
 *                                    logits for calls of at most 4096 tokens,
 *                                    EP = 64 if E <= 64 else 128; else 0);
 *   lbv_moe_permute_workspace_size:  for lbv_moe_permute;
 *   lbv_moe_w13_workspace_size:      for lbv_moe_gemm_w13_silu (256 bytes of
 *                                    tile queue counters);
 *   lbv_moe_w2_workspace_size:       for lbv_moe_gemm_w2_combine.
 * Sizes grow linearly with T (the forward one is dominated by the bf16 expert
 * output buffer, T (K + ns) H elements).
 */
lbv_status lbv_moe_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);
lbv_status lbv_moe_route_workspace_size(const lbv_moe_config *cfg, size_t *bytes);
lbv_status lbv_moe_permute_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);
lbv_status lbv_moe_w13_workspace_size(const lbv_moe_config *cfg, int64_t T, size_t *bytes);
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
 *                     most 4096 tokens also keep their logits there.  A
 *                     token's ids and weights do not depend on the other
 *                     tokens of the call, nor on how many there are.
 * Ties between equal scores go to the lower group / expert index.
 */
lbv_status lbv_moe_route(const lbv_moe_config *cfg, int64_t T, const void *x,
                         const float *router_w, const float *e_bias, const uint8_t *mask,
                         int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Allocation-free router, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and errors as lbv_moe_route, minus
 * the workspace: its scratch is a fixed 8 MiB device array inside the library
 * (one per GPU, held until the process ends), so the call needs
 * lbv_moe_route_workspace_size(cfg) <= 8 MiB (3 E H bf16 planes plus
 * 4096 x 128 fp32 logits; H up to about 8192 with 128 experts), else
 * LBV_ERR_SCRATCH.  It allocates nothing; its first call on a device looks up
 * the array's address there (LBV_ERR_HIP if that fails).  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * host threads, other streams) race and must be serialised by the caller.
 * Nothing in the array needs to start at zero.
 */
lbv_status lbv_moe_route_noalloc(const lbv_moe_config *cfg, int64_t T, const void *x,
                                 const float *router_w, const float *e_bias,
                                 const uint8_t *mask, int32_t *topk_ids, float *topk_w,
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
 *   act [T (K + ns), I] out (rows [0, R) written);
 *   ws, ws_bytes: lbv_moe_w13_workspace_size bytes of scratch (tile queue
 *   counters, reset by the call itself on `stream`).
 */
lbv_status lbv_moe_gemm_w13_silu(const lbv_moe_config *cfg, int64_t T, const void *x,
                                 const void *w13, const void *shared_w13,
                                 const int32_t *offsets, const int32_t *sorted_rows,
                                 void *act, void *ws, size_t ws_bytes, hipStream_t stream);

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

/*
 * ---------------------------------------------------------------------------
 * FP8 expert weights.  The LingBot-Video recipe of vLLM-Omni ("Known
 * Limitations") names FP8 among the expert backends its first integration
 * leaves out; the pages give no recipe.  Reading taken here (weights only;
 * activations stay bf16, accumulation fp32): row r of a weight matrix (one
 * output channel) is stored as OCP e4m3fn codes q[r, :] (bias 7, largest
 * finite value 448, codes 0x7f / 0xff NaN) and one scale 2^e[r], e the
 * smallest integer with max|w[r, :]| <= 448 2^e (e = 0 for an all-zero row),
 * q the nearest e4m3fn value of w 2^-e with ties to the even code.  The block
 * computes exactly what the bf16 block computes with the weights
 * decode(q) 2^e (these are exact in bf16).
 * ---------------------------------------------------------------------------
 */

/*
 * Quantizes `rows` rows of `cols` weights (dtype LBV_BF16 or LBV_F32, finite
 * values) into q [rows, cols] e4m3fn codes and scale [rows] fp32 powers of
 * two.  cols must be a positive multiple of 16, rows below 2^32 and
 * rows * cols at most 2^40; w, q 16-byte aligned, scale
 * 4-byte aligned; q and scale must not overlap w.  rows == 0 is a no-op.
 * Expert weights quantize as [E * 2I, H] (w13), [E * H, I] (w2),
 * [2 I_s, H] (shared_w13) and [H, I_s] (shared_w2).
 */
lbv_status lbv_quantize_fp8_rows(const void *w, int32_t dtype, int64_t rows, int64_t cols,
                                 uint8_t *q, float *scale, hipStream_t stream);

/* FP8 expert weights of one layer (device pointers; the shared ones NULL iff
 * n_shared_experts == 0; codes 16-byte, scales 4-byte aligned). */
typedef struct {
    const uint8_t *w13;              /* [E, 2I, H] codes                     */
    const float *w13_scale;          /* [E, 2I]                              */
    const uint8_t *w2;               /* [E, H, I] codes                      */
    const float *w2_scale;           /* [E, H]                               */
    const uint8_t *shared_w13;       /* [2 I_s, H] codes                     */
    const float *shared_w13_scale;   /* [2 I_s]                              */
    const uint8_t *shared_w2;        /* [H, I_s] codes                       */
    const float *shared_w2_scale;    /* [H]; the scale of row n covers all   */
                                     /* I_s columns (every pseudo-expert)    */
} lbv_moe_fp8_weights;

/*
 * lbv_moe_forward with fp8 expert weights: cfg->dtype must be LBV_BF16
 * (LBV_ERR_UNSUPPORTED otherwise); x, out bf16; router in fp32 as before;
 * ws: lbv_moe_workspace_size bytes.  Per row the matmuls read 1 byte per
 * weight instead of 2 and form decode(q) 2^e exactly before the bf16 matrix
 * cores, so the result equals lbv_moe_forward's on the dequantized weights
 * up to the order of fp32 summation.
 */
lbv_status lbv_moe_forward_fp8(const lbv_moe_config *cfg, int64_t T, const void *x,
                               const uint8_t *mask, const float *router_w, const float *e_bias,
                               const lbv_moe_fp8_weights *wq, void *out, int32_t *topk_ids_out,
                               float *topk_w_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * lbv_moe_forward with fp8 expert weights and fp8 activations, both matmuls
 * on the fp8 matrix cores (same source and same silence about the recipe as
 * above).  Reading taken: the router runs on x as before; each x row is
 * quantized like a weight row (e4m3fn codes, one power-of-two scale per
 * token); act = silu(gate) * up is rounded to bf16, its storage type in the
 * block, then stored in MX blocks of 32 values along I (OCP Microscaling:
 * e4m3fn codes and one e8m0 scale byte 2^(b - 127) per block, the block's
 * exponent chosen like a weight row's, held to [-127, 127]); the down
 * matmul reads those blocks; the expert outputs and the combine are as in
 * lbv_moe_forward.  Products are exact, sums fp32.
 * cfg->dtype must be LBV_BF16 (LBV_ERR_UNSUPPORTED otherwise); hidden and
 * intermediate multiples of 128, intermediate at most 1024 (LBV_ERR_SHAPE
 * otherwise); x, out bf16; wq as for lbv_moe_forward_fp8; ws:
 * lbv_moe_workspace_size bytes (the quantized x and act live in it).
 */
lbv_status lbv_moe_forward_w8a8(const lbv_moe_config *cfg, int64_t T, const void *x,
                                const uint8_t *mask, const float *router_w, const float *e_bias,
                                const lbv_moe_fp8_weights *wq, void *out, int32_t *topk_ids_out,
                                float *topk_w_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * ---------------------------------------------------------------------------
 * The steps on either side of the block in a LingBot-Video DiT layer (prhub
 * summary of sglang PR #32341, "实现拆解" step 2: AdaLN through
 * scale_shift_table and a token-level temb6, the norms kept in fp32;
 * vLLM-Omni article, "MoE 实现的源码级要点": RMSNorm accumulates in fp32).
 * Reading taken (the pages give no formula): the FFN half of a layer is
 *   out = x + gate * block(h),   h = rmsnorm(x) * (1 + scale) + shift,
 *   rmsnorm(x) = x / sqrt(mean(x^2) + eps)   (no learnable weight),
 *   (shift, scale, gate) = rows 3, 4, 5 of table + temb6 row t (fp32; rows
 *   0-2 belong to the attention half),
 * with x and out the fp32 residual stream and h rounded once to cfg->dtype.
 *   x      [T, H]      fp32
 *   temb6  6 H fp32 values per token at temb6 + t * temb_stride (elements,
 *          a multiple of 4; 0 = one row for every token)
 *   table  [6, H]      fp32 (scale_shift_table)
 *   eps    >= 0, finite
 * ---------------------------------------------------------------------------
 */

/* h [T, H] (cfg->dtype) = rmsnorm(x) * (1 + scale) + shift, rounded once;
 * the sum of squares accumulates in fp32.  h must not overlap x. */
lbv_status lbv_adaln_rmsnorm(const lbv_moe_config *cfg, int64_t T, const float *x,
                             const float *temb6, int64_t temb_stride, const float *table,
                             float eps, void *h, hipStream_t stream);

/* Workspace of lbv_moe_ffn_adaln: lbv_moe_workspace_size plus h [T, H]. */
lbv_status lbv_moe_ffn_adaln_workspace_size(const lbv_moe_config *cfg, int64_t T,
                                            size_t *bytes);

/*
 * The FFN half of a DiT layer: h = AdaLN(x), the block on h (route, permute,
 * gate/up + SiLU, down + combine), and the gated residual
 *   out[t] = x[t] + gate[t] * (sum_k w[t,k] y[t,k] + shared y[t])
 * formed in fp32 from the combine's fp32 sum (the block output is not
 * rounded).  out [T, H] fp32 may be x itself (in place), but may not overlap
 * it otherwise.  mask, router and expert weights, topk_ids_out / topk_w_out
 * as in lbv_moe_forward; ws: lbv_moe_ffn_adaln_workspace_size bytes.
 */
lbv_status lbv_moe_ffn_adaln(const lbv_moe_config *cfg, int64_t T, const float *x,
                             const uint8_t *mask, const float *temb6, int64_t temb_stride,
                             const float *table, float eps, const float *router_w,
                             const float *e_bias, const void *w13, const void *w2,
                             const void *shared_w13, const void *shared_w2, float *out,
                             int32_t *topk_ids_out, float *topk_w_out, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * ---------------------------------------------------------------------------
 * The attention half of a DiT layer (prhub summary of sglang PR #32341, the
 * LingBotVideoAttention excerpt under "关键源码片段" and "实现拆解" step 2):
 * joint self-attention over each sample's video;text tokens.  Per layer:
 *   qkv = x [W_q; W_k; W_v]^T + b_qkv    (one fused projection, bf16 out)
 *   q, k: RMSNorm over each head's D = 128 channels with weights g_q, g_k
 *         (fp32, rounded to bf16), then the rotary embedding with neox style
 *         off: channels (2i, 2i+1) of token t turned by cos / sin [t, i]
 *         (fp32 tables, D/2 per token; rounded to bf16)
 *   o = softmax(q k^T / sqrt(D)) v per head, over the valid tokens of the
 *       query's own sample (samples are runs of S tokens; a padding query
 *       gives 0)
 *   out = o W_o^T + b_o                  (bf16)
 * Readings taken where the pages are silent: head_dim is 128 (hidden /
 * num_heads must be 128); rmsnorm(u) = u / sqrt(mean(u^2) + eps) * g; the
 * projections carry a bias (NULL for none); the roundings sit at the module
 * boundaries of a bf16 model.  Tokens are B samples of S rows each (padding
 * rows inside a sample marked 0 in mask), S <= 65536.
 * ---------------------------------------------------------------------------
 */
typedef struct {
    int32_t hidden;                  /* H = num_heads * 128                 */
    int32_t num_heads;
    float eps;                       /* of the q / k head norms             */
} lbv_attn_config;

/* Workspace of lbv_attn_forward for B samples of S tokens: 512 bytes plus
 * qkv [T, 3H], q, k, o [T, H] and vt [B, heads, 128, Sp] in bf16 (T = B S,
 * Sp = S rounded up to 64). */
lbv_status lbv_attn_workspace_size(const lbv_attn_config *cfg, int64_t B, int64_t S,
                                   size_t *bytes);

/*
 * Dense projection y [T, N] = x [T, K] w[N, K]^T (+ bias [N], fp32, or NULL),
 * bf16 in and out, fp32 accumulation, one rounding; on the grouped matmul
 * kernel with a single segment.  N, K multiples of 64; T < 2^24; x and w each
 * under 4 GiB.  ws: 512 bytes of device scratch (set on the stream).
 */
lbv_status lbv_linear_bf16(int64_t T, int32_t N, int32_t K, const void *x, const void *w,
                           const float *bias, void *y, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * q / k head norms and rotary embedding, and v transposed for the attention
 * kernel: from qkv [B S, 3H] (bf16) write q, k [B S, H] (bf16) and
 * vt [B, heads, 128, Sp] (bf16, key positions contiguous per channel; inside
 * every 16 keys the positions of keys 4-7 and 8-11 are swapped; zeros past S).
 * g_q, g_k [128] fp32; cos, sin [B S, 64] fp32.
 */
lbv_status lbv_attn_qk_prep(const lbv_attn_config *cfg, int64_t B, int64_t S, const void *qkv,
                            const float *g_q, const float *g_k, const float *cos_t,
                            const float *sin_t, void *q, void *k, void *vt, hipStream_t stream);

/*
 * Masked per-sample attention o [B S, H] (bf16) from q, k [B S, H] and vt as
 * lbv_attn_qk_prep writes them; mask u8 [B S] or NULL (every token valid).
 */
lbv_status lbv_attn_core(const lbv_attn_config *cfg, int64_t B, int64_t S, const void *q,
                         const void *k, const void *vt, const uint8_t *mask, void *o,
                         hipStream_t stream);

/*
 * The whole attention half: projection, prep, attention, output projection.
 *   x [B S, H] bf16 (the modulated layer input); mask u8 [B S] or NULL;
 *   w_qkv [3H, H] bf16 (rows of W_q, W_k, W_v); b_qkv [3H] fp32 or NULL;
 *   g_q, g_k [128] fp32; cos_t, sin_t [B S, 64] fp32; w_o [H, H] bf16;
 *   b_o [H] fp32 or NULL; out [B S, H] bf16 (must not overlap x or ws);
 *   ws: lbv_attn_workspace_size bytes.
 */
lbv_status lbv_attn_forward(const lbv_attn_config *cfg, int64_t B, int64_t S, const void *x,
                            const uint8_t *mask, const void *w_qkv, const float *b_qkv,
                            const float *g_q, const float *g_k, const float *cos_t,
                            const float *sin_t, const void *w_o, const float *b_o, void *out,
                            void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace of lbv_attn_half_adaln: lbv_attn_workspace_size plus h and the
 * block output, [B S, H] bf16 each. */
lbv_status lbv_attn_half_adaln_workspace_size(const lbv_attn_config *cfg, int64_t B, int64_t S,
                                              size_t *bytes);

/*
 * The attention half of a DiT layer with its modulation (prhub summary of
 * sglang PR #32341, "实现拆解" step 2; the same reading as the FFN half's,
 * with the first three rows): h = rmsnorm(x) * (1 + scale) + shift with
 * (shift, scale, gate) = rows 0, 1, 2 of table + temb6 row t (fp32), h
 * rounded to bf16; the attention half on h (lbv_attn_forward, bf16 block
 * output); out[t] = x[t] + gate[t] * block[t] in fp32.  x, out [B S, H] fp32
 * (out may be x itself, but may not overlap it otherwise); temb6 / table /
 * eps as for lbv_adaln_rmsnorm (eps of this norm; cfg->eps is the q/k head
 * norms'); the attention operands as for lbv_attn_forward; ws:
 * lbv_attn_half_adaln_workspace_size bytes.
 */
lbv_status lbv_attn_half_adaln(const lbv_attn_config *cfg, int64_t B, int64_t S, const float *x,
                               const uint8_t *mask, const float *temb6, int64_t temb_stride,
                               const float *table, float eps, const void *w_qkv,
                               const float *b_qkv, const float *g_q, const float *g_k,
                               const float *cos_t, const float *sin_t, const void *w_o,
                               const float *b_o, float *out, void *ws, size_t ws_bytes,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LBV_MOE_H */

/*
 * CPU oracle for the routed-MoE feed-forward block of the LingBot-Video MoE DiT.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * statement of what the block computes, written token by token from the pages.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * it; the library under test never does, and the two share no code.
 *
 * Sources (the pages), cited by page and section:
 *  [P1] prhub.com.cn summary of sglang PR #32341 (LingBot-Video MoE 30B):
 *       "实现拆解" step 1 (fp32 router, sigmoid scores plus
 *       e_score_correction_bias, group-limited top-k, routed scaling applied by
 *       the router and not again by the expert kernel; w13 packed [E, 2I, H]
 *       with gate then up, not interleaved), step 3 (48 layers, 128 experts,
 *       top-8, width 768, 4 groups, 2 kept, scaling 2.5), the moe.py excerpt
 *       of LingBotVideoSparseMoeBlock (SiLU-gated experts, router weight applied
 *       on the expert output, shared expert added to every token), and
 *       "风险与影响" risk 4 (a group's score is the sum of its two best scores).
 *  [P2] vLLM-Omni LingBot-Video article (m.xxqk.cn), "MoE 实现的源码级要点":
 *       selection on scores plus bias while the gate weights use the raw
 *       scores, norm_topk_prob, expert outputs restored with an FP32 weighted
 *       sum, padding mask applied to the routing scores, shared expert.
 *
 * Precision: the router (logits, sigmoid, bias, group scores, weights) is
 * fp32, as [P2] and the FP32 module list of [P1] step 2 fix it, with the
 * logit dot product summed sequentially over the hidden index.  The expert
 * MLPs and the combine, whose precision the pages leave to the kernel, are
 * evaluated in fp64 on the (bf16-exact) fp32 inputs, i.e. without the bf16
 * roundings a GPU takes.  Decision margins are fp64 differences of the fp32
 * selection values.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - the correction bias enters the group scores (group choice is selection);
 *  - experts of groups that are not kept are excluded from the top-k;
 *  - ties go to the lower group / expert index; slots are ordered by
 *    (biased score descending, expert index ascending);
 *  - normalisation is a plain division (sigmoid > 0, so the sum is > 0);
 *  - a padding token (mask 0) has no routed experts (ids -1, weights 0) and its
 *    output is the shared expert alone;
 *  - the shared expert is a SwiGLU MLP of width I * n_shared, weight 1,
 *    packed as [gate; up] = [2 I_s, H] and down [H, I_s]; w2 is [E, H, I].
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t hidden;          /* H */
    int32_t num_experts;     /* E */
    int32_t top_k;           /* K */
    int32_t n_group;
    int32_t topk_group;
    int32_t intermediate;    /* I, width of one routed expert */
    int32_t n_shared;        /* shared expert width is I * n_shared */
    int32_t norm_topk_prob;  /* 0 or 1 */
    float routed_scaling_factor;
} orc_cfg;

int orc_abi_version(void) { return 1; }

/* ---------------------------------------------------------------------------
 * Router, one token ([P1] step 1; [P2] "MoE 实现的源码级要点").
 * ------------------------------------------------------------------------- */

/* z[e] = sum_h x[h] * W_r[e,h], fp32, h ascending. */
static void router_logits(int H, int E, const float *x, const float *wr, float *z)
{
    for (int e = 0; e < E; ++e) {
        float acc = 0.0f;
        const float *w = wr + (size_t)e * H;
        for (int h = 0; h < H; ++h)
            acc += x[h] * w[h];
        z[e] = acc;
    }
}

/*
 * Route one token.  Outputs: ids[K] (int32), w[K] (fp32), the two decision
 * margins (fp64), and optionally z[E] (logits) and s[E] (sigmoid scores).
 * Returns 0 on success, -1 if the configuration is invalid.
 */
static int route_one(const orc_cfg *c, const float *x, const float *wr, const float *bias,
                     int valid, int32_t *ids, float *w, double *m_grp, double *m_sel,
                     float *z_out, float *s_out)
{
    const int E = c->num_experts, H = c->hidden, K = c->top_k;
    const int NG = c->n_group, TG = c->topk_group;
    if (NG <= 0 || E % NG != 0) return -1;
    const int G = E / NG;
    if (G < 2 || TG < 1 || TG > NG || K < 1 || K > TG * G) return -1;

    float *z = (float *)malloc(sizeof(float) * E * 3);
    float *s = z + E, *cs = z + 2 * E;
    float *gsc = (float *)malloc(sizeof(float) * NG);
    char *kept = (char *)calloc(NG, 1);
    char *taken = (char *)calloc(E, 1);

    router_logits(H, E, x, wr, z);
    for (int e = 0; e < E; ++e) {
        s[e] = 1.0f / (1.0f + expf(-z[e]));   /* sigmoid score */
        cs[e] = s[e] + bias[e];                /* selection value */
    }
    if (z_out) memcpy(z_out, z, sizeof(float) * E);
    if (s_out) memcpy(s_out, s, sizeof(float) * E);

    if (!valid) {
        for (int k = 0; k < K; ++k) { ids[k] = -1; w[k] = 0.0f; }
        *m_grp = INFINITY;
        *m_sel = INFINITY;
        goto done;
    }

    /* Group score: the two largest selection values inside the group, summed. */
    for (int j = 0; j < NG; ++j) {
        int b1 = -1, b2 = -1;
        for (int e = j * G; e < (j + 1) * G; ++e) {
            if (b1 < 0 || cs[e] > cs[b1]) { b2 = b1; b1 = e; }
            else if (b2 < 0 || cs[e] > cs[b2]) { b2 = e; }
        }
        gsc[j] = cs[b1] + cs[b2];
    }

    /* Keep the topk_group best groups: repeated arg-max, lower index on ties. */
    double last_kept_g = 0.0;
    for (int r = 0; r < TG; ++r) {
        int best = -1;
        for (int j = 0; j < NG; ++j)
            if (!kept[j] && (best < 0 || gsc[j] > gsc[best])) best = j;
        kept[best] = 1;
        last_kept_g = gsc[best];
    }
    {
        int best = -1;
        for (int j = 0; j < NG; ++j)
            if (!kept[j] && (best < 0 || gsc[j] > gsc[best])) best = j;
        *m_grp = best < 0 ? INFINITY : last_kept_g - (double)gsc[best];
    }

    /* Top-K experts inside the kept groups: repeated arg-max, lower index on ties. */
    double last_c = 0.0;
    for (int k = 0; k < K; ++k) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (kept[e / G] && !taken[e] && (best < 0 || cs[e] > cs[best])) best = e;
        taken[best] = 1;
        ids[k] = best;
        last_c = cs[best];
    }
    {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (kept[e / G] && !taken[e] && (best < 0 || cs[e] > cs[best])) best = e;
        *m_sel = best < 0 ? INFINITY : last_c - (double)cs[best];
    }

    /* Weights: raw scores at the chosen experts, optionally normalised, then
     * multiplied by the routed scaling factor once. */
    {
        float sum = 0.0f;
        for (int k = 0; k < K; ++k) sum += s[ids[k]];
        for (int k = 0; k < K; ++k) {
            float v = s[ids[k]];
            if (c->norm_topk_prob) v = v / sum;
            w[k] = v * c->routed_scaling_factor;
        }
    }

done:
    free(z);
    free(gsc);
    free(kept);
    free(taken);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Expert MLP ([P1] moe.py excerpt, runner flags: silu, gated, gate/up not
 * interleaved).  fp64 throughout.
 * ------------------------------------------------------------------------- */

static double silu_d(double u) { return u / (1.0 + exp(-u)); }

/*
 * act[i] = silu(gate_i) * up_i for i < width, where gate_i is row i and up_i
 * row up_off + i of the packed gate/up matrix w (rows of length H).
 */
static void swiglu_act(int H, int width, long up_off, const float *x, const float *w,
                       double *act)
{
    for (int i = 0; i < width; ++i) {
        const float *g = w + (size_t)i * H;
        const float *u = w + (size_t)(up_off + i) * H;
        double ga = 0.0, ua = 0.0;
        for (int h = 0; h < H; ++h) {
            ga += (double)g[h] * (double)x[h];
            ua += (double)u[h] * (double)x[h];
        }
        act[i] = silu_d(ga) * ua;
    }
}

/* y[n] = sum_i W[n, i] * act[i] for n < H; W has rows of length ld. */
static void down_proj(int H, int width, long ld, const float *W, const double *act, double *y)
{
    for (int n = 0; n < H; ++n) {
        const float *r = W + (size_t)n * ld;
        double acc = 0.0;
        for (int i = 0; i < width; ++i) acc += (double)r[i] * act[i];
        y[n] = acc;
    }
}

/* ---------------------------------------------------------------------------
 * Exported entry points.
 * ------------------------------------------------------------------------- */

/*
 * Route ntok tokens.  x [ntok,H] fp32; wr [E,H]; bias [E]; mask [ntok] or NULL.
 * ids/w [ntok,K]; m_grp/m_sel [ntok]; z/s [ntok,E] optional (NULL to skip).
 */
int orc_route(const orc_cfg *c, int64_t ntok, const float *x, const float *wr,
              const float *bias, const uint8_t *mask, int32_t *ids, float *w,
              double *m_grp, double *m_sel, float *z, float *s)
{
    int bad = 0;
    const int H = c->hidden, E = c->num_experts, K = c->top_k;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int64_t t = 0; t < ntok; ++t) {
        int r = route_one(c, x + t * H, wr, bias, mask ? mask[t] != 0 : 1, ids + t * K,
                          w + t * K, m_grp + t, m_sel + t, z ? z + t * E : NULL,
                          s ? s + t * E : NULL);
        bad |= (r != 0);
    }
    return bad ? -1 : 0;
}

/*
 * act [I] of routed expert e for one token: w13 is the full [E, 2I, H] array.
 */
void orc_expert_act(const orc_cfg *c, const float *x, const float *w13, int e, double *act)
{
    const int H = c->hidden, I = c->intermediate;
    swiglu_act(H, I, I, x, w13 + (size_t)e * 2 * I * H, act);
}

/* act [I*n_shared] of the shared expert for one token. */
void orc_shared_act(const orc_cfg *c, const float *x, const float *shared_w13, double *act)
{
    const int H = c->hidden, Is = c->intermediate * c->n_shared;
    swiglu_act(H, Is, Is, x, shared_w13, act);
}

/* y [H] of routed expert e applied to one token (unweighted). */
void orc_expert_out(const orc_cfg *c, const float *x, const float *w13, const float *w2,
                    int e, double *y)
{
    const int H = c->hidden, I = c->intermediate;
    double *act = (double *)malloc(sizeof(double) * I);
    swiglu_act(H, I, I, x, w13 + (size_t)e * 2 * I * H, act);
    down_proj(H, I, I, w2 + (size_t)e * H * I, act, y);
    free(act);
}

/*
 * Full block for ntok tokens (each token independent):
 *   out[t] = sum_k w[t,k] * f_{ids[t,k]}(x[t]) + f_shared(x[t])
 * x [ntok,H]; wr [E,H]; bias [E]; mask [ntok] or NULL; w13 [E,2I,H];
 * w2 [E,H,I]; shared_w13 [2 I_s,H] and shared_w2 [H,I_s] (NULL if n_shared=0).
 * out [ntok,H] fp64; ids/w [ntok,K]; m_grp/m_sel [ntok].
 */
int orc_moe_forward(const orc_cfg *c, int64_t ntok, const float *x, const uint8_t *mask,
                    const float *wr, const float *bias, const float *w13, const float *w2,
                    const float *shared_w13, const float *shared_w2, double *out,
                    int32_t *ids, float *w, double *m_grp, double *m_sel)
{
    const int H = c->hidden, K = c->top_k, I = c->intermediate;
    const int Is = c->intermediate * c->n_shared;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t t = 0; t < ntok; ++t) {
        const float *xt = x + t * H;
        int32_t *it = ids + t * K;
        float *wt = w + t * K;
        double *ot = out + t * H;
        int r = route_one(c, xt, wr, bias, mask ? mask[t] != 0 : 1, it, wt, m_grp + t,
                          m_sel + t, NULL, NULL);
        if (r != 0) { bad = 1; continue; }
        int wmax = I > Is ? I : Is;
        double *act = (double *)malloc(sizeof(double) * (wmax > 0 ? wmax : 1));
        double *y = (double *)malloc(sizeof(double) * H);
        for (int n = 0; n < H; ++n) ot[n] = 0.0;
        for (int k = 0; k < K; ++k) {
            if (it[k] < 0) continue;
            swiglu_act(H, I, I, xt, w13 + (size_t)it[k] * 2 * I * H, act);
            down_proj(H, I, I, w2 + (size_t)it[k] * H * I, act, y);
            for (int n = 0; n < H; ++n) ot[n] += (double)wt[k] * y[n];
        }
        if (Is > 0 && shared_w13 && shared_w2) {
            swiglu_act(H, Is, Is, xt, shared_w13, act);
            down_proj(H, Is, Is, shared_w2, act, y);
            for (int n = 0; n < H; ++n) ot[n] += y[n];
        }
        free(act);
        free(y);
    }
    return bad ? -1 : 0;
}

/*
 * Route with a given expert choice.  The scores s come from the oracle's own
 * router (steps above); the chosen experts are taken from ids_in [ntok, K]
 * instead of the group-limited top-k (an id outside [0, E) is an empty slot).
 * The weights follow the same rule as route_one on that choice: raw scores at
 * the given ids, summed in slot order, divided by the sum when
 * norm_topk_prob, times the routed scaling factor once; empty slots weigh 0.
 * The output is the block output for that choice (same expert MLPs and the
 * same combine as orc_moe_forward), so a token on which a kernel made another
 * near-equal choice can still be compared element by element.
 * out [ntok, H] fp64; w_out [ntok, K] fp32.
 */
int orc_moe_forward_ids(const orc_cfg *c, int64_t ntok, const float *x, const float *wr,
                        const int32_t *ids_in, const float *w13, const float *w2,
                        const float *shared_w13, const float *shared_w2, double *out,
                        float *w_out)
{
    const int H = c->hidden, K = c->top_k, I = c->intermediate, E = c->num_experts;
    const int Is = c->intermediate * c->n_shared;
    if (E <= 0 || K <= 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < ntok; ++t) {
        const float *xt = x + t * H;
        const int32_t *it = ids_in + t * K;
        float *wt = w_out + t * K;
        double *ot = out + t * H;
        float *z = (float *)malloc(sizeof(float) * E);
        router_logits(H, E, xt, wr, z);
        float sum = 0.0f;
        for (int k = 0; k < K; ++k) {
            if (it[k] < 0 || it[k] >= E) continue;
            sum += 1.0f / (1.0f + expf(-z[it[k]]));
        }
        for (int k = 0; k < K; ++k) {
            if (it[k] < 0 || it[k] >= E) { wt[k] = 0.0f; continue; }
            float v = 1.0f / (1.0f + expf(-z[it[k]]));
            if (c->norm_topk_prob) v = v / sum;
            wt[k] = v * c->routed_scaling_factor;
        }
        free(z);
        int wmax = I > Is ? I : Is;
        double *act = (double *)malloc(sizeof(double) * (wmax > 0 ? wmax : 1));
        double *y = (double *)malloc(sizeof(double) * H);
        for (int n = 0; n < H; ++n) ot[n] = 0.0;
        for (int k = 0; k < K; ++k) {
            if (it[k] < 0 || it[k] >= E) continue;
            swiglu_act(H, I, I, xt, w13 + (size_t)it[k] * 2 * I * H, act);
            down_proj(H, I, I, w2 + (size_t)it[k] * H * I, act, y);
            for (int n = 0; n < H; ++n) ot[n] += (double)wt[k] * y[n];
        }
        if (Is > 0 && shared_w13 && shared_w2) {
            swiglu_act(H, Is, Is, xt, shared_w13, act);
            down_proj(H, Is, Is, shared_w2, act, y);
            for (int n = 0; n < H; ++n) ot[n] += y[n];
        }
        free(act);
        free(y);
    }
    return 0;
}

/*
 * act rows of the gate/up stage for n (token, segment) pairs: segment s < E is
 * routed expert s, segment E + j the j-th width-I slice of the shared MLP
 * (gate rows jI .. jI+I-1 and up rows I_s + jI .. of shared_w13).
 * act[r, i] = silu(gate_i . x[tok[r]]) * (up_i . x[tok[r]]), fp64.
 * act [n, I].
 */
void orc_act_rows(const orc_cfg *c, int64_t n, const float *x, const float *w13,
                  const float *shared_w13, const int32_t *tok, const int32_t *seg, double *act)
{
    const int H = c->hidden, I = c->intermediate, E = c->num_experts;
    const long Is = (long)c->intermediate * c->n_shared;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < n; ++r) {
        const float *xt = x + (size_t)tok[r] * H;
        if (seg[r] < E) {
            swiglu_act(H, I, I, xt, w13 + (size_t)seg[r] * 2 * I * H, act + r * I);
        } else {
            const long j = seg[r] - E;
            /* gate rows start at j*I, up rows at I_s + j*I: offset between them I_s */
            swiglu_act(H, I, Is, xt, shared_w13 + (size_t)j * I * H, act + r * I);
        }
    }
}

/*
 * Down projection and weighted combine from given act values, per token:
 *   out[t] = sum_{k < K, ids[t,k] in [0,E)} w[t,k] * W2[ids[t,k]] act[t,k]
 *          + sum_{j < n_shared} W2_shared[:, jI:(j+1)I] act[t, K+j]
 * act [ntok, K + n_shared, I] (the act vector of each slot), ids/w [ntok, K],
 * w2 [E, H, I], shared_w2 [H, I_s]; out [ntok, H] fp64.
 */
void orc_down_combine(const orc_cfg *c, int64_t ntok, const float *act, const int32_t *ids,
                      const float *w, const float *w2, const float *shared_w2, double *out)
{
    const int H = c->hidden, I = c->intermediate, E = c->num_experts, K = c->top_k;
    const int NS = c->n_shared, KS = K + NS;
    const long Is = (long)I * NS;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < ntok; ++t) {
        double *ot = out + t * H;
        double *a = (double *)malloc(sizeof(double) * I);
        double *y = (double *)malloc(sizeof(double) * H);
        for (int n = 0; n < H; ++n) ot[n] = 0.0;
        for (int k = 0; k < KS; ++k) {
            const float *ak = act + ((size_t)t * KS + k) * I;
            for (int i = 0; i < I; ++i) a[i] = ak[i];
            if (k < K) {
                const int e = ids[t * K + k];
                if (e < 0 || e >= E) continue;
                down_proj(H, I, I, w2 + (size_t)e * H * I, a, y);
                for (int n = 0; n < H; ++n) ot[n] += (double)w[t * K + k] * y[n];
            } else {
                down_proj(H, I, Is, shared_w2 + (size_t)(k - K) * I, a, y);
                for (int n = 0; n < H; ++n) ot[n] += y[n];
            }
        }
        free(a);
        free(y);
    }
}

/* ---------------------------------------------------------------------------
 * The steps around the block in a DiT layer ([P1] step 2: AdaLN through
 * scale_shift_table and a token-level temb6, fp32-sensitive modules
 * including every norm; [P2] "MoE 实现的源码级要点": RMSNorm accumulates in
 * fp32).  Readings (the pages give no formula): the FFN half of a layer is
 *   out = x + gate * MoE(bf16(rmsnorm(x) * (1 + scale) + shift)),
 * with (shift, scale, gate) = rows 3, 4, 5 of scale_shift_table[6, H] +
 * temb6[t][6, H] (rows 0-2 belong to the attention half), RMSNorm
 * x / sqrt(mean(x^2) + eps) with no learnable weight (the modulation is the
 * affine part), the residual stream x in fp32, and the MoE input rounded once
 * to the experts' storage type.
 * ------------------------------------------------------------------------- */

/* Nearest bf16 value of d (ties to even), computed from d directly: the
 * 8 significant bits of the binary expansion of d, rounded by rint (the
 * default rounding mode is to nearest, ties to even).  Normal range only. */
static double bf16_round_d(double d)
{
    if (d == 0.0 || !isfinite(d)) return d;
    int e;
    const double m = frexp(d, &e);          /* d = m 2^e, 0.5 <= |m| < 1 */
    return ldexp(rint(ldexp(m, 8)), e - 8);
}

/*
 * h[t] = rmsnorm(x[t]) * (1 + scale[t]) + shift[t], fp64, then rounded to
 * bf16 when round_bf16 (stored as fp32, exact).  x [ntok, H] fp32;
 * temb6 row t at temb6 + t * temb_stride (6 H fp32 values; stride 0: one row
 * for all tokens); table [6, H].
 */
/* The same with the (shift, scale) rows given: 3, 4 in front of the FFN
 * block, 0, 1 in front of the attention block of a layer. */
void orc_adaln_rmsnorm_rows(int H, int64_t ntok, const float *x, const float *temb6,
                            int64_t temb_stride, const float *table, double eps, int round_bf16,
                            int shift_row, int scale_row, float *h)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        const float *xt = x + t * H;
        const float *et = temb6 + t * temb_stride;
        double ss = 0.0;
        for (int i = 0; i < H; ++i) ss += (double)xt[i] * (double)xt[i];
        const double r = 1.0 / sqrt(ss / H + eps);
        for (int i = 0; i < H; ++i) {
            const double shift = (double)table[shift_row * H + i] + (double)et[shift_row * H + i];
            const double scale = (double)table[scale_row * H + i] + (double)et[scale_row * H + i];
            const double v = (double)xt[i] * r * (1.0 + scale) + shift;
            h[t * H + i] = (float)(round_bf16 ? bf16_round_d(v) : v);
        }
    }
}

void orc_adaln_rmsnorm(int H, int64_t ntok, const float *x, const float *temb6,
                       int64_t temb_stride, const float *table, double eps, int round_bf16,
                       float *h)
{
    orc_adaln_rmsnorm_rows(H, ntok, x, temb6, temb_stride, table, eps, round_bf16, 3, 4, h);
}

/* The nearest bf16 value of each double (exposed for its pin). */
void orc_bf16_round(int64_t n, const double *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round_d(in[i]);
}

/* ---------------------------------------------------------------------------
 * FP8 expert weights.  The LingBot-Video recipe of vLLM-Omni ("Known
 * Limitations") names FP8 among the expert backends its first integration
 * leaves out; the pages give no recipe for it.  Reading: each weight row
 * (one output channel) is stored as OCP e4m3fn codes with one power-of-two
 * scale 2^e, e the smallest integer with max|w| <= 448 * 2^e (e = 0 for an
 * all-zero row), q = nearest e4m3fn value of w * 2^-e, ties to the even code.
 * The dequantized weight is decode(q) * 2^e.
 * ------------------------------------------------------------------------- */

/* Value of an OCP e4m3fn code (bias 7, no infinities, 0x7f / 0xff NaN). */
static double e4m3_decode(uint8_t c)
{
    const double s = (c & 0x80) ? -1.0 : 1.0;
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) return s * ldexp((double)m, -9);          /* subnormal: m * 2^-9 */
    return s * ldexp(8.0 + m, e - 10);                    /* (1 + m/8) 2^(e-7) */
}

/* Nearest e4m3fn code of a finite |v| <= 448, ties to the even code. */
static uint8_t e4m3_encode(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0;
    const double a = fabs(v);
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid of 2^-9; 8 * 2^-9 is the smallest normal, code 8 */
        return sign | (uint8_t)rint(ldexp(a, 9));
    }
    int ex;
    frexp(a, &ex);                                       /* a = f 2^ex, 0.5 <= f < 1 */
    int E = ex - 1;                                      /* a = (1 + r/8) 2^E */
    double r = rint(ldexp(a, 3 - E)) - 8.0;              /* mantissa steps of 2^(E-3) */
    if (r >= 8.0) { r = 0.0; ++E; }
    return sign | (uint8_t)(((E + 7) << 3) | (int)r);
}

/* Power-of-two exponent of a row with maximum magnitude amax. */
static int fp8_row_exponent(double amax)
{
    if (amax == 0.0) return 0;
    int x;
    const double f = frexp(amax, &x);                    /* amax = f 2^x, 448 = 0.875 2^9 */
    return f <= 0.875 ? x - 9 : x - 8;
}

/*
 * Quantize rows [rows, cols] of fp32 values: q [rows, cols] codes,
 * scale [rows] = 2^e as fp32.
 */
void orc_quantize_fp8_rows(int64_t rows, int64_t cols, const float *w, uint8_t *q, float *scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *wr = w + r * cols;
        double amax = 0.0;
        for (int64_t c = 0; c < cols; ++c) amax = fmax(amax, fabs((double)wr[c]));
        const int e = fp8_row_exponent(amax);
        scale[r] = (float)ldexp(1.0, e);
        for (int64_t c = 0; c < cols; ++c) q[r * cols + c] = e4m3_encode(ldexp((double)wr[c], -e));
    }
}

/* Dequantized rows: w[r, c] = decode(q[r, c]) * scale[r] (exact in fp32). */
void orc_dequantize_fp8_rows(int64_t rows, int64_t cols, const uint8_t *q, const float *scale,
                             float *w)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            w[r * cols + c] = (float)(e4m3_decode(q[r * cols + c]) * (double)scale[r]);
}

void orc_e4m3_decode_all(double *out)
{
    for (int c = 0; c < 256; ++c) out[c] = e4m3_decode((uint8_t)c);
}

/* ---------------------------------------------------------------------------
 * FP8 activations in MX blocks (OCP Microscaling, MXFP8 E4M3), for the
 * expert path with fp8 weights and fp8 activations.  The pages name FP8
 * expert backends but give no recipe (same source as above).  Reading: a row
 * is cut into blocks of 32 consecutive values; a block has one scale 2^e kept
 * as the e8m0 byte e + 127, e chosen by the rule of the weight rows above
 * (smallest e with max|v| <= 448 * 2^e, e = 0 for an all-zero block) and held
 * to [-127, 127], the byte's range; each value is the nearest e4m3fn code of
 * v * 2^-e, ties to the even code.  (The MX specification takes
 * e = floor(log2 max|v|) - 8 and saturates; the two agree unless
 * 448 * 2^e < max|v| < 512 * 2^e, where this rule takes the next e and
 * clips nothing.)
 * ------------------------------------------------------------------------- */

/* v [rows, cols] (cols a multiple of 32) -> codes q [rows, cols] and e8m0
 * bytes e8 [rows, cols / 32]. */
void orc_quantize_mx_rows(int64_t rows, int64_t cols, const double *v, uint8_t *q, uint8_t *e8)
{
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const double *vb = v + r * cols + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(vb[i]));
            int e = fp8_row_exponent(amax);
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            e8[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) q[r * cols + b * 32 + i] = e4m3_encode(ldexp(vb[i], -e));
        }
    }
}

/* v[r, c] = decode(q[r, c]) * 2^(e8[r, c / 32] - 127). */
void orc_dequantize_mx_rows(int64_t rows, int64_t cols, const uint8_t *q, const uint8_t *e8,
                            double *v)
{
    const int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            v[r * cols + c] = ldexp(e4m3_decode(q[r * cols + c]), (int)e8[r * nb + c / 32] - 127);
}

/* ---------------------------------------------------------------------------
 * The attention half of a LingBot-Video DiT layer (prhub summary of sglang PR
 * #32341, the LingBotVideoAttention excerpt under "关键源码片段" and "实现拆解"
 * step 2): q, k, v are linear projections of the layer input; q and k get an
 * RMSNorm over each head's D channels (fp32 module, learnable weight of D),
 * then the rotary embedding with neox style off (channels 2i and 2i + 1 form
 * a pair turned by the angle whose cos / sin the caller's tables hold for
 * that token and i); attention is non-causal with the default scale
 * 1 / sqrt(D), over the video;text tokens of the token's own sample, padding
 * keys excluded; the heads' outputs go through the output projection.
 * Readings (the pages give no formula): y = x W^T + b for the projections;
 * rmsnorm(u) = u / sqrt(mean(u^2) + eps) * g; a padding query's output is 0.
 * Everything here is fp64; the roundings to bf16 between the steps are the
 * caller's (oracle/__init__.py), at the module boundaries of a bf16 model.
 * ------------------------------------------------------------------------- */

/* y[t, n] = sum_c x[t, c] w[n, c] (+ b[n]): x [T, C], w [N, C], y [T, N]. */
void orc_linear(int64_t T, int N, int C, const float *x, const float *w, const float *b,
                double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *xr = x + t * C;
        for (int n = 0; n < N; ++n) {
            const float *wr = w + (int64_t)n * C;
            double acc = 0.0;
            for (int c = 0; c < C; ++c) acc += (double)xr[c] * (double)wr[c];
            y[t * N + n] = acc + (b ? (double)b[n] : 0.0);
        }
    }
}

/* RMSNorm of every row of D values: y = u / sqrt(mean(u^2) + eps) * g. */
void orc_head_rmsnorm(int64_t rows, int D, const double *u, const float *g, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *ur = u + r * D;
        double ss = 0.0;
        for (int i = 0; i < D; ++i) ss += ur[i] * ur[i];
        const double inv = 1.0 / sqrt(ss / D + eps);
        for (int i = 0; i < D; ++i) y[r * D + i] = ur[i] * inv * (double)g[i];
    }
}

/*
 * Rotary embedding, neox style off: for token t, head h and pair i < D/2,
 *   y[2i]   = u[2i] cos(t, i) - u[2i+1] sin(t, i)
 *   y[2i+1] = u[2i+1] cos(t, i) + u[2i] sin(t, i)
 * u, y [T, heads, D]; cs, sn [T, D/2].
 */
void orc_rope(int64_t T, int heads, int D, const double *u, const float *cs, const float *sn,
              double *y)
{
    const int P = D / 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < heads; ++h)
            for (int i = 0; i < P; ++i) {
                const double c = cs[t * P + i], s = sn[t * P + i];
                const double *ur = u + (t * heads + h) * D;
                double *yr = y + (t * heads + h) * D;
                yr[2 * i] = ur[2 * i] * c - ur[2 * i + 1] * s;
                yr[2 * i + 1] = ur[2 * i + 1] * c + ur[2 * i] * s;
            }
}

/*
 * Attention of the query rows qrows[0..nq) (all T rows when qrows is NULL):
 * token t belongs to sample t / S; its keys are the tokens of that sample
 * with mask 1 (every token when mask is NULL).  o[r, h] = sum_j p_j v[j, h],
 * p = softmax_j(q[t, h] . k[j, h] / sqrt(D)); 0 for a padding query or a
 * sample without keys.  q, k, v [T, heads, D]; o [nq, heads, D].
 */
void orc_attention(int64_t T, int64_t S, int heads, int D, const float *q, const float *k,
                   const float *v, const uint8_t *mask, int64_t nq, const int64_t *qrows,
                   double *o)
{
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel
    {
        double *sc = malloc(sizeof(double) * (size_t)S);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nq; ++r) {
            const int64_t t = qrows ? qrows[r] : r;
            const int64_t j0 = t / S * S, j1 = j0 + S < T ? j0 + S : T;
            for (int h = 0; h < heads; ++h) {
                double *orow = o + (r * heads + h) * D;
                for (int i = 0; i < D; ++i) orow[i] = 0.0;
                if (mask && !mask[t]) continue;
                const float *qr = q + (t * heads + h) * D;
                double mx = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    sc[j - j0] = -INFINITY;
                    if (mask && !mask[j]) continue;
                    const float *kr = k + (j * heads + h) * D;
                    double d = 0.0;
                    for (int i = 0; i < D; ++i) d += (double)qr[i] * (double)kr[i];
                    sc[j - j0] = d * scale;
                    if (sc[j - j0] > mx) mx = sc[j - j0];
                }
                if (mx == -INFINITY) continue;              /* no keys */
                double den = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    if (sc[j - j0] == -INFINITY) continue;
                    const double p = exp(sc[j - j0] - mx);
                    den += p;
                    const float *vr = v + (j * heads + h) * D;
                    for (int i = 0; i < D; ++i) orow[i] += p * (double)vr[i];
                }
                for (int i = 0; i < D; ++i) orow[i] /= den;
            }
        }
        free(sc);
    }
}

/*
 * Token copies sorted by expert ([P2] "MoE 实现的源码级要点": tokens are
 * reordered by expert before the grouped matmuls and restored after).
 * Plain stable counting sort of the slots by segment.  Slot (t, k), k < K, is
 * token t's k-th routed choice and belongs to segment ids[t,k]; slot (t, K+j)
 * belongs to shared segment E + j.  Slot id = t * (K + ns) + k.  An id outside
 * [0, E), or one already seen earlier in the same token, is not routed
 * (inv_rows = -1).  offsets [E + ns + 1]; sorted_rows, inv_rows [T (K + ns)].
 */
void orc_permute(const orc_cfg *c, int64_t T, const int32_t *ids, int32_t *offsets,
                 int32_t *sorted_rows, int32_t *inv_rows)
{
    const int E = c->num_experts, K = c->top_k, NS = c->n_shared;
    const int KS = K + NS, S = E + NS;
    int64_t *count = (int64_t *)calloc(S, sizeof(int64_t));
    int64_t *fill = (int64_t *)calloc(S, sizeof(int64_t));
    for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e = ids[t * K + k], first = 1;
            for (int j = 0; j < k; ++j)
                if (ids[t * K + j] == e) first = 0;
            if (e >= 0 && e < E && first) count[e]++;
        }
    for (int j = 0; j < NS; ++j) count[E + j] = T;
    offsets[0] = 0;
    for (int s = 0; s < S; ++s) {
        offsets[s + 1] = (int32_t)(offsets[s] + count[s]);
        fill[s] = offsets[s];
    }
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t slot = t * KS + k;
            int e = ids[t * K + k], first = 1;
            for (int j = 0; j < k; ++j)
                if (ids[t * K + j] == e) first = 0;
            if (e >= 0 && e < E && first) {
                int64_t pos = fill[e]++;
                sorted_rows[pos] = (int32_t)slot;
                inv_rows[slot] = (int32_t)pos;
            } else {
                inv_rows[slot] = -1;
            }
        }
        for (int j = 0; j < NS; ++j) {
            int64_t slot = t * KS + K + j;
            int64_t pos = fill[E + j]++;
            sorted_rows[pos] = (int32_t)slot;
            inv_rows[slot] = (int32_t)pos;
        }
    }
    free(count);
    free(fill);
}

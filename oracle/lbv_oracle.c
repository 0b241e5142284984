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

// Router of the LingBot-Video MoE block on gfx950.
//
// What it computes (prhub summary of sglang PR #32341, "实现拆解" step 1 and
// risk 4 under "风险与影响"; vLLM-Omni LingBot-Video article,
// "MoE 实现的源码级要点"):
//   z = x W_r^T (fp32), s = sigmoid(z), c = s + e_score_correction_bias;
//   group score = sum of the two largest c in each group; keep the topk_group
//   best groups; the top_k largest c inside the kept groups are the experts;
//   weight = s at those experts (no bias), normalised over the chosen experts
//   when norm_topk_prob, times routed_scaling_factor, once.
//
// Design:
//  * One workgroup (4 waves) routes 64 tokens.  The logits of the 64 tokens
//    against all experts are an fp32 matrix product done with
//    v_mfma_f32_32x32x2_f32 (exact fp32 products, fp32 accumulation) on
//    32-wide hidden chunks of x and W_r staged through LDS.  bf16 x is
//    widened exactly to fp32 when staged.
//  * The logits go to LDS; then each wave routes one token at a time with its
//    64 lanes: lane l owns experts [l*EPL, (l+1)*EPL).  A group then occupies
//    LG = G/EPL neighbouring lanes (16 lanes, one DPP row, for E=128), so the
//    in-group top-2 is a butterfly over LG lanes.  Group choice and expert
//    choice are repeated wave-wide arg-max reductions on 64-bit keys
//    (order-preserving score bits, inverted index), so ties go to the lower
//    index exactly as in a sequential scan.
#include "lbv_internal.h"
#include "lbv_pipe.h"

namespace lbv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int RT_TOK = 64;       // tokens per workgroup
constexpr int RT_HC = 32;        // hidden chunk staged per step
constexpr int RT_LD = RT_HC + 4; // LDS row stride (floats): rows shift by 4 banks
constexpr int RT_EMAX = 256;

struct RouteArgs {
    const void* x;
    const float* wr;
    const float* bias;
    const uint8_t* mask;
    int32_t* ids;
    float* w;
    int64_t T;
    int H, E, EP, K, NG, TG, G, EPL, LG, norm;
    float rsf;
};

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

template <bool XBF16>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    // LDS: staging of x / W_r chunks, later reused for the logits.
    constexpr int STAGE_FLOATS = (RT_TOK + RT_EMAX) * RT_LD;
    constexpr int Z_FLOATS = RT_TOK * (RT_EMAX + 1);
    __shared__ float smem[STAGE_FLOATS > Z_FLOATS ? STAGE_FLOATS : Z_FLOATS];
    float* xs = smem;                    // [RT_TOK][RT_LD]
    float* ws = smem + RT_TOK * RT_LD;   // [EP][RT_LD]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT_TOK;
    const int H = a.H, E = a.E, EP = a.EP;

    // ---- logits: z[64 tokens][EP experts] with fp32 MFMA -------------------
    // wave -> token half (32 rows) and every other 32-expert tile.
    const int th = wave & 1;
    const int eset = wave >> 1;
    const int ntile = EP / 32;
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;

    for (int h0 = 0; h0 < H; h0 += RT_HC) {
        // stage x: 64 rows x 32 values; thread -> row tid/4, 8 values
        {
            const int r = tid >> 2, c = (tid & 3) * 8;
            const int64_t t = t0 + r;
            float v[8];
            if (t < a.T) {
                if (XBF16) {
                    const uint4 q = *reinterpret_cast<const uint4*>(
                        static_cast<const uint16_t*>(a.x) + t * H + h0 + c);
                    const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = __uint_as_float(qq[i] << 16);
                        v[2 * i + 1] = __uint_as_float(qq[i] & 0xffff0000u);
                    }
                } else {
                    const float4* p = reinterpret_cast<const float4*>(
                        static_cast<const float*>(a.x) + t * H + h0 + c);
                    float4 p0 = p[0], p1 = p[1];
                    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
                    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.f;
            }
            float4* d = reinterpret_cast<float4*>(xs + r * RT_LD + c);
            d[0] = make_float4(v[0], v[1], v[2], v[3]);
            d[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        // stage W_r: EP rows x 32 values; 8 float4 per row
        for (int i = tid; i < EP * 8; i += 256) {
            const int r = i >> 3, c = (i & 7) * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < E) v = *reinterpret_cast<const float4*>(a.wr + static_cast<int64_t>(r) * H + h0 + c);
            *reinterpret_cast<float4*>(ws + r * RT_LD + c) = v;
        }
        __syncthreads();
        // 2 steps of 16 hidden values; each step is 8 MFMAs of k=2 in which
        // lanes 0-31 carry hidden index kk+i and lanes 32-63 kk+8+i (the same
        // pairing on both operands, so every product appears once).
#pragma unroll
        for (int kk = 0; kk < RT_HC; kk += 16) {
            const int koff = kk + (lane >> 5) * 8;
            const float* xr = xs + (th * 32 + (lane & 31)) * RT_LD + koff;
            const f32x4 xa = *reinterpret_cast<const f32x4*>(xr);
            const f32x4 xb = *reinterpret_cast<const f32x4*>(xr + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tile = eset + 2 * j;
                if (tile < ntile) {
                    const float* wrow = ws + (tile * 32 + (lane & 31)) * RT_LD + koff;
                    const f32x4 wa = *reinterpret_cast<const f32x4*>(wrow);
                    const f32x4 wb = *reinterpret_cast<const f32x4*>(wrow + 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[i], wa[i], acc[j], 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(xb[i], wb[i], acc[j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- logits to LDS: zs[token][expert], row stride EMAX+1 ----------------
    float* zs = smem;
    constexpr int ZLD = RT_EMAX + 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tile = eset + 2 * j;
        if (tile < ntile) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = th * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                const int col = tile * 32 + (lane & 31);
                zs[row * ZLD + col] = acc[j][i];
            }
        }
    }
    __syncthreads();

    // ---- selection: one wave per token --------------------------------------
    const int EPL = a.EPL, LG = a.LG, G = a.G, K = a.K;
    const int e0 = lane * EPL;                 // first expert of this lane
    const int grp = e0 / G;                    // this lane's group (>= NG: no experts)
    const bool lane_has = e0 < E;
    float bias_l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bias_l[q] = (q < EPL && e0 + q < E) ? a.bias[e0 + q] : 0.f;

    for (int r = wave; r < RT_TOK; r += 4) {
        const int64_t t = t0 + r;
        if (t >= a.T) break;
        const bool valid = a.mask == nullptr || a.mask[t] != 0;

        float s[4], c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < EPL && lane_has && e0 + q < E) {
                const float z = zs[r * ZLD + e0 + q];
                s[q] = 1.0f / (1.0f + expf(-z));
                c[q] = s[q] + bias_l[q];
            } else {
                s[q] = 0.f;
                c[q] = -INFINITY;
            }
        }

        // In-group top-2 over this lane's experts, then over the group's LG lanes.
        float b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < EPL) {
                const float v = c[q];
                if (v > b1) { b2 = b1; b1 = v; }
                else if (v > b2) { b2 = v; }
            }
        }
        for (int off = 1; off < LG; off <<= 1) {
            const float o1 = __shfl_xor(b1, off);
            const float o2 = __shfl_xor(b2, off);
            const float n1 = fmaxf(b1, o1);
            const float n2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
            b1 = n1;
            b2 = n2;
        }
        const float gscore = b1 + b2;

        // Keep TG groups: repeated arg-max over (score desc, group asc).
        uint32_t kept = 0;
        const bool grp_real = lane_has && grp < a.NG;
        for (int rr = 0; rr < a.TG; ++rr) {
            uint64_t key = 0;
            if (grp_real && !((kept >> grp) & 1u))
                key = (static_cast<uint64_t>(fkey(gscore)) << 32) | (0xffffffffu - static_cast<uint32_t>(grp));
            key = wave_max_u64(key);
            const int win = static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
            kept |= 1u << win;
        }
        const bool in_kept = grp_real && ((kept >> grp) & 1u);

        // Top-K experts in the kept groups: repeated arg-max over (c desc, id asc).
        uint32_t taken = 0;           // bit q: expert e0+q already chosen
        int my_id = -1;
        float my_s = 0.f;
        for (int k = 0; k < K; ++k) {
            uint64_t key = 0;
            if (in_kept) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q < EPL && !((taken >> q) & 1u) && e0 + q < E) {
                        const uint64_t kq = (static_cast<uint64_t>(fkey(c[q])) << 32) |
                                            (0xffffffffu - static_cast<uint32_t>(e0 + q));
                        key = kq > key ? kq : key;
                    }
                }
            }
            key = wave_max_u64(key);
            const int win = static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
            float sw = 0.f;
            if (win >= e0 && win < e0 + EPL) {
                const int q = win - e0;
                taken |= 1u << q;
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    if (qq == q) sw = s[qq];
            }
            // the owner lane's score, broadcast
            sw = __shfl(sw, win / EPL);
            if (lane == k) { my_id = win; my_s = sw; }
        }

        // Weights: sum of the chosen raw scores in slot order, then scale once.
        float sum = 0.f;
        for (int k = 0; k < K; ++k) sum += __shfl(my_s, k);
        if (lane < K) {
            float wv = a.norm ? my_s / sum : my_s;
            wv = wv * a.rsf;
            a.ids[t * K + lane] = valid ? my_id : -1;
            a.w[t * K + lane] = valid ? wv : 0.f;
        }
    }
}

// ===========================================================================
// bf16 path (x stored as bf16, E <= 128, n_group <= 8, G % 4 == 0, K <= 16)
// ===========================================================================
//
// Logits on the bf16 matrix cores, exactly in fp32 terms: the fp32 router
// weight is split once per call into three bf16 planes with
// W = hi + mid + lo exactly (hi = RNE(W), mid = RNE(W - hi), lo = W - hi - mid,
// which fits bf16 for every finite W below the bf16 overflow threshold).  x is
// bf16, so each product x*plane is exact in fp32 and the MFMA sums them in
// fp32: the logit is an fp32 dot product, in a different summation order.
//
// One workgroup routes 128 tokens.  Per 32-wide hidden slice a stage holds the
// 128 x rows and the 3 x EP plane rows (64 bytes each), filled by
// asynchronous copies three slices ahead.  Wave w owns expert tile w (32
// experts) against all 4 token tiles: 3 planes x 4 = 12 MFMAs per 16-deep
// step.  The epilogue turns logits into scores s = sigmoid(z) and selection
// values c = s + bias in LDS; then each lane routes one token by scanning
// its row: in-group top-2 sums, kept groups, and a sorted top-K insertion in
// (c descending, id ascending) order over the kept groups' experts.

constexpr int RV_TOK = 128;
constexpr int RV_BK = 32;
constexpr int RV_STAGES = 4;
constexpr int RV_NGMAX = 8;

struct RouteV2Args {
    const uint16_t* x;       // [T, H] bf16
    const uint16_t* planes;  // [3, E, H] bf16
    const float* bias;
    const uint8_t* mask;
    int32_t* ids;
    float* w;
    int64_t T;
    int H, E, K, NG, TG, G, norm;
    float rsf;
};

__global__ __launch_bounds__(256) void router_split_kernel(const float* wr, uint16_t* planes,
                                                           int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    const float w = wr[i];
    const uint16_t hi = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    planes[i] = hi;
    planes[n + i] = mid;
    planes[2 * n + i] = f32_to_bf16(r2);
}

__device__ __forceinline__ int rswz(int r) { return (r >> 2) & 3; }   // 64-byte rows

template <int EP, int KMAX>
__global__ __launch_bounds__(256) void route_bf16_kernel(RouteV2Args a) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    constexpr int ROWS = RV_TOK + 3 * EP;                 // stage rows
    constexpr int STAGE = ROWS * RV_BK;                   // bf16 elements
    constexpr int NI = ROWS / 64;                         // copies per wave per stage (16 rows each)
    static_assert(ROWS % 64 == 0, "stage rows split over 4 waves");
    constexpr int PITCH = EP + 4;                         // floats per token row of c / s
    constexpr int STAGE_BYTES = RV_STAGES * STAGE * 2;
    constexpr int CS_BYTES = 2 * RV_TOK * PITCH * 4;
    constexpr int SMEM = STAGE_BYTES > CS_BYTES ? STAGE_BYTES : CS_BYTES;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM / 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RV_TOK;
    const int H = a.H, E = a.E;

    // ---- copy sources: instruction i of this wave fills stage rows
    // wave * (ROWS/4) + 16 i + lane/4, logical chunk (lane%4) ^ rswz(row) ----
    const uint16_t* src[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = wave * (ROWS / 4) + i * 16 + (lane >> 2);
        const int c = (lane & 3) ^ rswz(r);
        if (r < RV_TOK) {
            int64_t t = t0 + r;
            if (t >= a.T) t = a.T - 1;
            src[i] = a.x + t * H + c * 8;
        } else {
            const int q = r - RV_TOK;
            const int p = q / EP;
            int e = q % EP;
            if (e >= E) e = E - 1;
            src[i] = a.planes + (static_cast<int64_t>(p) * E + e) * H + c * 8;
        }
    }
    auto issue = [&](int kt) {
        const uint32_t base = lds_addr(smem + (kt % RV_STAGES) * STAGE);
#pragma unroll
        for (int i = 0; i < NI; ++i)
            lds_dma16(src[i] + kt * RV_BK, base + (wave * (ROWS / 4) + i * 16) * RV_BK * 2);
    };

    const int khalf = lane >> 5;
    const bool has_tile = wave * 32 < EP;                 // EP = 64: waves 2, 3 idle in the MFMA
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;

    const int nk = H / RV_BK;
    issue(0);
    if (1 < nk) issue(1);
    if (2 < nk) issue(2);
    for (int kt = 0; kt < nk; ++kt) {
        const int ahead = nk - 1 - kt;
        if (ahead >= 2) wait_vmcnt<2 * NI>();
        else if (ahead == 1) wait_vmcnt<NI>();
        else wait_vmcnt<0>();
        block_barrier();
        if (kt + 3 < nk) issue(kt + 3);
        if (has_tile) {
            const uint16_t* st = smem + (kt % RV_STAGES) * STAGE;
#pragma unroll
            for (int kk = 0; kk < RV_BK / 16; ++kk) {
                const int ch = kk * 2 + khalf;
                bf16x8 tf[4], wf[3];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = i * 32 + (lane & 31);
                    tf[i] = *reinterpret_cast<const bf16x8*>(st + r * RV_BK + ((ch ^ rswz(r)) * 8));
                }
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    const int r = RV_TOK + p * EP + wave * 32 + (lane & 31);
                    wf[p] = *reinterpret_cast<const bf16x8*>(st + r * RV_BK + ((ch ^ rswz(r)) * 8));
                }
#pragma unroll
                for (int p = 0; p < 3; ++p)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[p], tf[i], acc[i], 0, 0, 0);
            }
        }
    }

    // ---- scores to LDS: lane holds experts 8q + 4*khalf + [0,4) of token (lane&31) ----
    block_barrier();
    float* Cs = reinterpret_cast<float*>(smem);
    float* Ss = Cs + RV_TOK * PITCH;
    if (has_tile) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = i * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = wave * 32 + 8 * q + 4 * khalf;
                float cv[4], sv[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int e = e0 + p;
                    const float z = acc[i][4 * q + p];
                    sv[p] = 1.0f / (1.0f + expf(-z));
                    cv[p] = e < E ? sv[p] + a.bias[e] : -INFINITY;
                }
                *reinterpret_cast<float4*>(Cs + tok * PITCH + e0) = make_float4(cv[0], cv[1], cv[2], cv[3]);
                *reinterpret_cast<float4*>(Ss + tok * PITCH + e0) = make_float4(sv[0], sv[1], sv[2], sv[3]);
            }
        }
    }
    __syncthreads();

    // ---- selection: lane-per-token (lanes 0-31 of every wave) -------------------
    if (lane >= 32) return;
    const int tok = wave * 32 + lane;
    const int64_t t = t0 + tok;
    if (t >= a.T) return;
    const float* crow = Cs + tok * PITCH;
    const int G = a.G, NG = a.NG;

    // in-group top-2 sums
    float gsc[RV_NGMAX];
#pragma unroll
    for (int j = 0; j < RV_NGMAX; ++j) {
        gsc[j] = -INFINITY;
        if (j < NG) {
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int e = j * G; e < (j + 1) * G; e += 4) {
                const float4 v4 = *reinterpret_cast<const float4*>(crow + e);
                const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float v = vv[u];
                    if (v > b1) { b2 = b1; b1 = v; }
                    else if (v > b2) { b2 = v; }
                }
            }
            gsc[j] = b1 + b2;
        }
    }
    // kept groups: repeated arg-max, lower index on ties; then their indices ascending
    uint32_t kept = 0;
    for (int r = 0; r < a.TG; ++r) {
        float bv = -INFINITY;
        int bj = -1;
#pragma unroll
        for (int j = 0; j < RV_NGMAX; ++j)
            if (j < NG && !((kept >> j) & 1u) && (bj < 0 || gsc[j] > bv)) { bv = gsc[j]; bj = j; }
        kept |= 1u << bj;
    }
    // top-K (first KMAX) over the kept groups' experts in ascending id order
    float v[KMAX];
    int id[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) { v[k] = -INFINITY; id[k] = -1; }
    uint32_t rem = kept;
    for (int r = 0; r < a.TG; ++r) {
        const int j = __builtin_ctz(rem);
        rem &= rem - 1;
        for (int e = j * G; e < (j + 1) * G; e += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(crow + e);
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float c = vv[u];
                const int ec = e + u;
#pragma unroll
                for (int k = KMAX - 1; k > 0; --k) {
                    const bool gp = c > v[k - 1];
                    const bool gk = c > v[k];
                    const float nv = gp ? v[k - 1] : (gk ? c : v[k]);
                    const int ni = gp ? id[k - 1] : (gk ? ec : id[k]);
                    v[k] = nv;
                    id[k] = ni;
                }
                if (c > v[0]) { v[0] = c; id[0] = ec; }
            }
        }
    }
    // weights from the raw scores, slot order sum, scaled once
    const float* srow = Ss + tok * PITCH;
    const bool valid = a.mask == nullptr || a.mask[t] != 0;
    float sk[KMAX];
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        sk[k] = 0.f;
        if (k < a.K) {
            sk[k] = srow[id[k]];
            sum += sk[k];
        }
    }
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < a.K) {
            float wv = a.norm ? sk[k] / sum : sk[k];
            wv = wv * a.rsf;
            a.ids[t * a.K + k] = valid ? id[k] : -1;
            a.w[t * a.K + k] = valid ? wv : 0.f;
        }
    }
}

}  // namespace

bool route_bf16_path(const Dims& d) {
    return d.bf16 && d.E <= 128 && d.NG <= RV_NGMAX && d.G % 4 == 0;
}

size_t route_ws_bytes(const Dims& d) {
    return route_bf16_path(d) ? static_cast<size_t>(3) * d.E * d.H * sizeof(uint16_t) : 0;
}

hipError_t launch_route(const Dims& d, const void* x, const float* router_w, const float* e_bias,
                        const uint8_t* mask, int32_t* topk_ids, float* topk_w, void* ws,
                        hipStream_t stream) {
    if (route_bf16_path(d)) {
        uint16_t* planes = static_cast<uint16_t*>(ws);
        const int64_t n = static_cast<int64_t>(d.E) * d.H;
        hipLaunchKernelGGL(router_split_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                           dim3(256), 0, stream, router_w, planes, n);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        RouteV2Args a;
        a.x = static_cast<const uint16_t*>(x);
        a.planes = planes;
        a.bias = e_bias;
        a.mask = mask;
        a.ids = topk_ids;
        a.w = topk_w;
        a.T = d.T;
        a.H = d.H;
        a.E = d.E;
        a.K = d.K;
        a.NG = d.NG;
        a.TG = d.TG;
        a.G = d.G;
        a.norm = d.norm;
        a.rsf = d.rsf;
        const dim3 grid(static_cast<unsigned>((d.T + RV_TOK - 1) / RV_TOK));
        if (d.E <= 64) {
            if (d.K <= 8) hipLaunchKernelGGL((route_bf16_kernel<64, 8>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((route_bf16_kernel<64, 16>), grid, dim3(256), 0, stream, a);
        } else {
            if (d.K <= 8) hipLaunchKernelGGL((route_bf16_kernel<128, 8>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((route_bf16_kernel<128, 16>), grid, dim3(256), 0, stream, a);
        }
        return hipGetLastError();
    }
    RouteArgs a;
    a.x = x;
    a.wr = router_w;
    a.bias = e_bias;
    a.mask = mask;
    a.ids = topk_ids;
    a.w = topk_w;
    a.T = d.T;
    a.H = d.H;
    a.E = d.E;
    a.EP = ((d.E + 31) / 32) * 32;
    a.K = d.K;
    a.NG = d.NG;
    a.TG = d.TG;
    a.G = d.G;
    a.EPL = d.EPL;
    a.LG = d.LG;
    a.norm = d.norm;
    a.rsf = d.rsf;
    const unsigned grid = static_cast<unsigned>((d.T + RT_TOK - 1) / RT_TOK);
    if (d.bf16)
        hipLaunchKernelGGL(route_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(route_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lbv

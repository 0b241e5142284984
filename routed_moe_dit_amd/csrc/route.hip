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
// Three paths:
//  * bf16 x, E <= 128 (the block's configuration), more than 4096 tokens:
//    route_bf16_kernel computes the fp32 logits on the bf16 matrix cores from
//    an exact three-plane split of W_r, then routes two lanes per token (see
//    the comment above it).
//  * bf16 x, E <= 128, at most 4096 tokens: route_logits_kernel forms the
//    same logits, in the same summation order, over many small workgroups,
//    and route_select_kernel routes one token per wave; a token's routing is
//    therefore the same on both sides of the switch.
//  * otherwise (fp32 x, more experts or groups): route_kernel, one workgroup
//    (4 waves) per 64 tokens, logits with v_mfma_f32_32x32x2_f32 on 32-wide
//    hidden chunks of x and W_r staged through LDS (bf16 x widened exactly),
//    then one token per wave.
// Wave-per-token routing (wave_route): lane l owns experts [l*EPL,
// (l+1)*EPL); a group occupies LG = G/EPL neighbouring lanes, so the in-group
// top-2 is a butterfly over LG lanes.  Group choice and expert choice are
// repeated wave-wide arg-max reductions on 64-bit keys (order-preserving
// score bits, inverted index), so ties go to the lower index exactly as in a
// sequential scan.
#include <mutex>

#include "lbv_internal.h"
#include "lbv_pipe.h"

// Scratch of the allocation-free router entry (lbv_moe_route_noalloc): the
// W_r planes and the few-token logits.  One copy per GPU, shared by every
// call on that GPU; host code never uses this name as an address (it is a
// host-side stand-in): route_scratch() looks up the device address once per
// device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[lbv::kRouteScratchBytes];

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

// Sigmoid score of a logit, fp32; every router path uses this one expression
// so that equal logits give equal scores whichever kernel computed them.
__device__ __forceinline__ float sigmoid_score(float z) { return 1.0f / (1.0f + expf(-z)); }

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

// Routes token t with one wave: lane l holds experts e0 = l*EPL + q (q < EPL,
// EPL <= 4) with raw scores s[q] and selection values c[q] (-inf past E);
// LG lanes cover one group of G experts.  Group top-2 sums by shuffles, kept
// groups and the top-K by repeated wave arg-max over (value desc, index asc),
// weights from the raw scores summed in slot order and scaled once.
__device__ __forceinline__ void wave_route(int64_t t, int lane, int E, int EPL, int LG, int G,
                                           int NG, int TG, int K, int norm, float rsf, bool valid,
                                           const float (&s)[4], const float (&c)[4],
                                           int32_t* ids, float* w) {
    const int e0 = lane * EPL;                 // first expert of this lane
    const int grp = e0 / G;                    // this lane's group (>= NG: no experts)
    const bool lane_has = e0 < E;
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
    const bool grp_real = lane_has && grp < NG;
    for (int rr = 0; rr < TG; ++rr) {
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
        float wv = norm ? my_s / sum : my_s;
        wv = wv * rsf;
        ids[t * K + lane] = valid ? my_id : -1;
        w[t * K + lane] = valid ? wv : 0.f;
    }
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
                s[q] = sigmoid_score(z);
                c[q] = s[q] + bias_l[q];
            } else {
                s[q] = 0.f;
                c[q] = -INFINITY;
            }
        }

        wave_route(t, lane, E, EPL, LG, G, a.NG, a.TG, K, a.norm, a.rsf, valid, s, c, a.ids, a.w);
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
// One workgroup (8 waves, two per SIMD) routes TOK = 32 TM tokens (TM chosen
// per call so that the grid fills the CUs in one round where it can).  Per
// 64-wide hidden slice a stage holds the TOK x rows and the 3 x EP plane rows
// (128 bytes each, laid out [X0|X1|W0|W1] over two stages), filled by
// asynchronous copies that waves 0-3 spread between their MFMAs.  Wave w owns
// expert tile (w % 4) % (EP/32) against all TM token tiles and the 16-deep
// slices 2g, 2g+1 (g = w / 4) of every hidden slice: 3 planes x TM MFMAs per
// step; the two halves of each logit are added through LDS at the end.  The
// epilogue turns logits into scores s = sigmoid(z) in LDS; then two lanes
// route one token with selection values c = s + bias: in-group top-2 sums,
// kept groups, and a sorted top-K in (c descending, id ascending) order over
// the kept groups' experts, kept as 64-bit keys so that the insertion has no
// branches.

constexpr int RV_NGMAX = 8;
constexpr int RV_BK = 64;

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

// The exact three-plane split of one fp32 router weight: hi = RNE(w),
// mid = RNE(w - hi), lo = RNE(w - hi - mid), with hi + mid + lo == w.  Every
// router path takes its planes from this one routine.
__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    hi = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(hi);
    mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    lo = f32_to_bf16(r2);
}

__global__ __launch_bounds__(256) void router_split_kernel(const float* wr, uint16_t* planes,
                                                           int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n) return;
    uint16_t hi, mid, lo;
    split3(wr[i], hi, mid, lo);
    planes[i] = hi;
    planes[n + i] = mid;
    planes[2 * n + i] = lo;
}

// 128-byte rows: chunk c of row r at c ^ ((r >> 1) & 7) (conflict-free reads)
__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }

// Routing of token t by a lane pair (u = 0, 1): srow holds its scores s
// (LDS), s_bias the correction bias (LDS).  Lane u takes experts 4b + 2u and
// 4b + 2u + 1 of every block of four; c = s + bias.  Writes ids and weights.
template <int KMAX>
__device__ __forceinline__ void select_token(const RouteV2Args& a, const float* srow,
                                             const float* s_bias, int u, int64_t t) {
    const int G = a.G, NG = a.NG;

    // in-group top-2 sums: each lane's top-2 over its half, then the top-2 of
    // the four (max / min, no branches); both lanes end with the same sums
    float gsc[RV_NGMAX];
#pragma unroll
    for (int j = 0; j < RV_NGMAX; ++j) {
        gsc[j] = -INFINITY;
        if (j < NG) {
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int e0 = j * G; e0 < (j + 1) * G; e0 += 4) {
                const int e = e0 + 2 * u;
                const float2 v2 = *reinterpret_cast<const float2*>(srow + e);
                const float2 bb = *reinterpret_cast<const float2*>(s_bias + e);
                const float c0 = v2.x + bb.x;
                const float c1 = v2.y + bb.y;
                b2 = fmaxf(b2, fminf(b1, c0));
                b1 = fmaxf(b1, c0);
                b2 = fmaxf(b2, fminf(b1, c1));
                b1 = fmaxf(b1, c1);
            }
            const float p1 = __shfl_xor(b1, 1), p2 = __shfl_xor(b2, 1);
            gsc[j] = fmaxf(b1, p1) + fmaxf(fminf(b1, p1), fmaxf(b2, p2));
        }
    }
    // kept groups: repeated arg-max, lower index on ties; then their indices ascending
    uint32_t kept = 0;
    for (int r = 0; r < a.TG; ++r) {
        float bv = -INFINITY;
        int bj = -1;
#pragma unroll
        for (int j = 0; j < RV_NGMAX; ++j) {
            const bool take = j < NG && !((kept >> j) & 1u) && (bj < 0 || gsc[j] > bv);
            bv = take ? gsc[j] : bv;
            bj = take ? j : bj;
        }
        kept |= 1u << bj;
    }
    // top-K (first KMAX) in (c descending, id ascending) order, as 64-bit
    // keys: an order-preserving image of c (with -0 taken as +0) above the
    // complement of the id, so that the larger key is the larger c, or the
    // lower id on equal c.  A sorted insertion is then
    // key[k] = max(key[k], min(key[k-1], new)).  Each lane inserts its half
    // of the kept groups' experts, then the partner's list.
    auto okey = [](float c, int e) -> uint64_t {
        uint32_t b = __float_as_uint(c + 0.0f);
        b ^= static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u;
        return (static_cast<uint64_t>(b) << 32) | static_cast<uint32_t>(~e);
    };
    uint64_t key[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) key[k] = 0;           // below every real key; decodes to id -1
    auto insert = [&](uint64_t nk) {
#pragma unroll
        for (int k = KMAX - 1; k > 0; --k) {
            const uint64_t lo = key[k - 1] < nk ? key[k - 1] : nk;
            key[k] = key[k] > lo ? key[k] : lo;
        }
        key[0] = key[0] > nk ? key[0] : nk;
    };
    uint32_t rem = kept;
    for (int r = 0; r < a.TG; ++r) {
        const int j = __builtin_ctz(rem);
        rem &= rem - 1;
        for (int e0 = j * G; e0 < (j + 1) * G; e0 += 4) {
            const int e = e0 + 2 * u;
            const float2 v2 = *reinterpret_cast<const float2*>(srow + e);
            const float2 bb = *reinterpret_cast<const float2*>(s_bias + e);
            insert(okey(v2.x + bb.x, e));
            insert(okey(v2.y + bb.y, e + 1));
        }
    }
    {
        uint64_t pk[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const uint32_t hi = __shfl_xor(static_cast<uint32_t>(key[k] >> 32), 1);
            const uint32_t lo = __shfl_xor(static_cast<uint32_t>(key[k]), 1);
            pk[k] = (static_cast<uint64_t>(hi) << 32) | lo;
        }
#pragma unroll
        for (int m = 0; m < KMAX; ++m) insert(pk[m]);
    }
    int id[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) id[k] = static_cast<int>(~static_cast<uint32_t>(key[k]));
    // weights from the raw scores, slot order sum, scaled once; lane u stores
    // the slots k with k % 2 == u
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
        if (k < a.K && (k & 1) == u) {
            float wv = a.norm ? sk[k] / sum : sk[k];
            wv = wv * a.rsf;
            a.ids[t * a.K + k] = valid ? id[k] : -1;
            a.w[t * a.K + k] = valid ? wv : 0.f;
        }
    }
}

template <int TM, int EP, int KMAX>
__global__ __launch_bounds__(512) void route_bf16_kernel(RouteV2Args a) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int BK = RV_BK;
    constexpr int TOK = 32 * TM;
    constexpr int XSZ = TOK * BK, WSZ = 3 * EP * BK;      // bf16 elements of one stage's parts
    constexpr int XI = TOK / 4 / 8, WI = 3 * EP / 4 / 8;  // copies per wave per k-tile (8 rows each)
    constexpr int NI = XI + WI;
    static_assert(TOK % 32 == 0 && (3 * EP) % 32 == 0, "rows split over 4 waves in 8-row copies");
    constexpr int PITCH = EP + 4;                         // floats per token row of s
    constexpr int SMEM = 2 * (XSZ + WSZ) * 2;
    static_assert(TOK * PITCH * 4 <= SMEM, "scores fit in the stage memory");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[SMEM / 2];
    __shared__ float s_bias[EP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TOK;
    const int H = a.H, E = a.E;
    if (tid < EP) s_bias[tid] = tid < E ? a.bias[tid] : 0.f;
    // 8 waves, two per SIMD: wave w handles expert tile (w % 4) % (EP / 32)
    // and the 16-deep slices 2g, 2g+1 (g = w / 4) of every 64-wide k-tile;
    // waves 0-3 also issue all the copies.  The two halves of the sum meet in
    // LDS at the end.
    const int grp = wave >> 2, ew = wave & 3;
    const bool copier = wave < 4;

    // ---- copy sources: a uniform base plus 32-bit per-lane byte offsets.  X
    // copy i of wave w fills x rows w*TOK/4 + 8i + lane/8; W copy i fills plane
    // rows w*3EP/4 + 8i + lane/8 (plane p = row / EP, expert row % EP); lane l
    // lands at physical chunk l%8, which holds logical chunk (l%8) ^ rswz(row).
    uint32_t xoff[XI], woff[WI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int r = ew * (TOK / 4) + i * 8 + (lane >> 3);
        const uint32_t c = (lane & 7) ^ rswz(r);
        int64_t t = t0 + r;
        if (t >= a.T) t = a.T - 1;
        xoff[i] = (__umul24(static_cast<uint32_t>(t), H) + c * 8) * 2;
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
        const int q = ew * (3 * EP / 4) + i * 8 + (lane >> 3);
        const uint32_t c = (lane & 7) ^ rswz(q);
        const int p = q / EP;
        int e = q % EP;
        if (e >= E) e = E - 1;
        woff[i] = (__umul24(p * E + e, H) + c * 8) * 2;
    }
    uint16_t* const xs = smem;                            // X0, X1
    uint16_t* const ws = smem + 2 * XSZ;                  // W0, W1
    auto copies = [&](auto S, int kt, int d0, int d1) {
        constexpr int s = decltype(S)::value;
        if (!copier) return;
        static_for<NI>([&](auto D) {
            constexpr int d = decltype(D)::value;
            if (d >= d0 && d < d1) {
                if constexpr (d < XI)
                    lds_dma16_sb<d * 8 * BK * 2>(a.x + kt * BK, xoff[d],
                                                 lds_addr(xs + s * XSZ + wave * (TOK / 4) * BK));
                else
                    lds_dma16_sb<(d - XI) * 8 * BK * 2>(a.planes + kt * BK, woff[d - XI],
                                                        lds_addr(ws + s * WSZ + wave * (3 * EP / 4) * BK));
            }
        });
    };
    auto zero_fill = [&](auto S) {
        constexpr int s = decltype(S)::value;
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4* px = reinterpret_cast<u32x4*>(xs + s * XSZ);
        u32x4* pw = reinterpret_cast<u32x4*>(ws + s * WSZ);
        for (int q = tid; q < XSZ / 8; q += 512) px[q] = z;
        for (int q = tid; q < WSZ / 8; q += 512) pw[q] = z;
    };

    // ---- fragments: plane rows are the MFMA's first operand, token rows the
    // second; slice kk of stage s: x fragment i at fx[kk] + s*XSZ + 32*i*BK,
    // plane p at fw[kk] + s*WSZ + p*EP*BK --------------------------------------
    const int kh = lane >> 5, rl = lane & 31;
    const int et = ew % (EP / 32);                        // expert tile (EP = 64: waves 2, 3 repeat 0, 1)
    const int ka = 2 * grp, kb = 2 * grp + 1;             // this wave's slices of a k-tile
    // fragment pointers of slice kk: fx + s*XSZ + 32*i*BK, fw + s*WSZ + p*EP*BK
    auto fxp = [&](int kk) { return xs + rl * BK + (((kk * 2 + kh) ^ rswz(rl)) * 8); };
    auto fwp = [&](int kk) { return ws + (et * 32 + rl) * BK + (((kk * 2 + kh) ^ rswz(rl)) * 8); };
    const uint16_t* const fxa = fxp(ka);
    const uint16_t* const fwa = fwp(ka);
    const uint16_t* const fxb = fxp(kb);
    const uint16_t* const fwb = fwp(kb);
    f32x16 acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[i] = f32x16{};
    bf16x8 tf0[TM], wf0[3], tf1[TM], wf1[3];

    const int nk = H / BK;
    const int nkp = (nk + 1) & ~1;                        // even: both steps of an iteration run
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    copies(S0{}, 0, 0, NI);
    wait_vmcnt<0>();
    block_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) tf0[i] = *reinterpret_cast<const bf16x8*>(fxa + i * 32 * BK);
#pragma unroll
    for (int p = 0; p < 3; ++p) wf0[p] = *reinterpret_cast<const bf16x8*>(fwa + p * EP * BK);

    constexpr int NQ = 3 * TM;                            // MFMAs per slice
    constexpr int NR = TM + 3;                            // fragment reads per slice
    constexpr int NPRE = NQ - NR;                         // MFMAs of the last slice before the barrier
    static_assert(NPRE >= 2, "reads fit between the MFMAs");
    // one slice: MFMAs from (CT, CW), after MFMA Q0 + r the fragment read r of
    // the slice at (FX, FW) of stage NB into (NT, NW), copies [D0, D1) of
    // k-tile KF spread over the MFMAs
#define RV_SLICE(CT, CW, NT_, NW_, NB, FX, FW, Q0, Q1, TS, KF, DO_COPY, D0, D1)                 \
    _Pragma("unroll") for (int q = (Q0); q < (Q1); ++q) {                                      \
        acc[q % TM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(CW[q / TM], CT[q % TM], acc[q % TM], 0, 0, 0); \
        const int r_ = q - (Q0);                                                                \
        if (r_ < TM)                                                                            \
            NT_[r_] = *reinterpret_cast<const bf16x8*>((FX) + (NB) * XSZ + r_ * 32 * BK);       \
        else if (r_ < NR)                                                                       \
            NW_[r_ - TM] = *reinterpret_cast<const bf16x8*>((FW) + (NB) * WSZ + (r_ - TM) * EP * BK); \
        if ((DO_COPY) && (D1) > (D0)) {                                                         \
            const int per = ((D1) - (D0) + (Q1) - (Q0) - 1) / ((Q1) - (Q0));                    \
            copies(TS, KF, (D0) + r_ * per, (D0) + r_ * per + per < (D1) ? (D0) + r_ * per + per : (D1)); \
        }                                                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                      \
    }
    // k-tile kt in stage S: the wave's first slice carries the copies of
    // k-tile kt + 1 into the other stage (freed by k-tile kt - 1); its second
    // slice brackets the hand-over (wait, barrier, then the reads of the
    // wave's first slice of k-tile kt + 1)
    auto step = [&](auto S, int kt) {
        constexpr int SI = decltype(S)::value;
        const auto TS = std::integral_constant<int, 1 - SI>{};
        const int kf = kt + 1;
        const bool do_copy = kf < nk;
        if (kf >= nk && kf < nkp) zero_fill(TS);
        RV_SLICE(tf0, wf0, tf1, wf1, SI, fxb, fwb, 0, NQ, TS, kf, do_copy, 0, NI)
#pragma unroll
        for (int q = 0; q < NPRE; ++q)
            acc[q % TM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf1[q / TM], tf1[q % TM], acc[q % TM], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kf < nkp) {
            wait_vmcnt<0>();
            wait_lgkmcnt0();
            block_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        RV_SLICE(tf1, wf1, tf0, wf0, 1 - SI, fxa, fwa, NPRE, NQ, TS, kf, false, 0, 0)
    };
#undef RV_SLICE
    for (int kt = 0; kt < nkp; kt += 2) {
        step(S0{}, kt);
        step(S1{}, kt + 1);
    }

    // ---- the two halves of the sum: waves 4-7 hand theirs to waves 0-3 ----
    wait_lgkmcnt0();
    block_barrier();
    {
        float* part = reinterpret_cast<float*>(smem);     // [4][TM][16][64]
        static_assert(4 * TM * 16 * 64 * 4 <= SMEM, "partial sums fit in the stage memory");
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) part[((ew * TM + i) * 16 + v) * 64 + lane] = acc[i][v];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][v] += part[((ew * TM + i) * 16 + v) * 64 + lane];
        }
        __syncthreads();
    }

    // ---- scores to LDS: lane holds experts 8q + 4*kh + [0,4) of token rl ----
    float* Ss = reinterpret_cast<float*>(smem);
    if (wave < EP / 32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int tok = i * 32 + rl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e0 = et * 32 + 8 * q + 4 * kh;
                float sv[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) sv[p] = sigmoid_score(acc[i][4 * q + p]);
                *reinterpret_cast<float4*>(Ss + tok * PITCH + e0) = make_float4(sv[0], sv[1], sv[2], sv[3]);
            }
        }
    }
    __syncthreads();

    // ---- selection: two lanes per token (u = 0, 1), lane u taking experts
    // 4b + 2u and 4b + 2u + 1 of every block of four; c = s + bias ---------------
    const int tok = tid >> 1, u = tid & 1;
    if (tok >= TOK) return;                               // both lanes of a token alike
    const int64_t t = t0 + tok;
    if (t >= a.T) return;
    select_token<KMAX>(a, Ss + tok * PITCH, s_bias, u, t);
}


// ---------------------------------------------------------------------------
// Few tokens (T <= RS_TMAX): one workgroup per 32 tokens and 32 experts, so
// that short batches spread over many CUs.  The logits are formed in exactly
// the order route_bf16_kernel uses: two accumulator chains, one over the
// 16-deep slices 0-1 and one over slices 2-3 of every 64-wide hidden k-tile,
// each applying the three planes in order, then one fp32 add of the two.  So
// a token's logits, and with them its routing, do not depend on how many
// tokens share the call.  A 4-deep ring of k-tiles keeps the walk over the
// hidden dimension ahead of the matrix cores.  The logits go to the
// workspace; a second kernel scores and routes each token with one wave.
// ---------------------------------------------------------------------------
constexpr int RS_TMAX = 4096;
constexpr int RS_STAGES = 4;

// grid: (ceil(T / 32), EP / 32); 2 waves, wave w accumulates slices 2w and
// 2w + 1 of every k-tile for 32 tokens x expert tile blockIdx.y (3 planes).
template <int EP>
__global__ __launch_bounds__(128) void route_logits_kernel(RouteV2Args a, float* zout) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    constexpr int BK = RV_BK;
    constexpr int TOK = 32, WR = 96, ROWS = TOK + WR;   // x rows, plane rows (3 x 32 experts)
    constexpr int STAGE = ROWS * BK;                    // bf16 elements per stage (16 KB)
    constexpr int CI = ROWS / 2 / 8;                    // copies per wave per k-tile (8 rows each)
    __shared__ __attribute__((aligned(1024))) uint16_t smem[RS_STAGES * STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TOK;
    const int et = blockIdx.y;
    const int H = a.H, E = a.E;
    const int nk = H / BK;

    // copy i of wave w: stage rows w*ROWS/2 + 8i + lane/8 (x rows first, then
    // plane rows p*32 + e of expert tile et); chunk (lane%8) ^ rswz(row)
    const uint16_t* src[CI];
#pragma unroll
    for (int i = 0; i < CI; ++i) {
        const int r = wave * (ROWS / 2) + i * 8 + (lane >> 3);
        const int c = (lane & 7) ^ rswz(r);
        if (r < TOK) {
            int64_t t = t0 + r;
            if (t >= a.T) t = a.T - 1;
            src[i] = a.x + t * H + c * 8;
        } else {
            const int q = r - TOK, p = q / 32;
            int e = et * 32 + q % 32;
            if (e >= E) e = E - 1;
            src[i] = a.planes + (static_cast<int64_t>(p) * E + e) * H + c * 8;
        }
    }
    auto issue = [&](int kt) {
        const uint32_t base = lds_addr(smem + (kt % RS_STAGES) * STAGE + wave * (ROWS / 2) * BK);
#pragma unroll
        for (int i = 0; i < CI; ++i) lds_dma16(src[i] + kt * BK, base + i * 8 * BK * 2);
    };
    const int kh = lane >> 5, rl = lane & 31;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int j = 0; j < RS_STAGES - 1; ++j)
        if (j < nk) issue(j);
    for (int kt = 0; kt < nk; ++kt) {
        // k-tile kt landed (the copies of up to two later k-tiles may be in flight)
        const int later = nk - 1 - kt < RS_STAGES - 2 ? nk - 1 - kt : RS_STAGES - 2;
        if (later >= 2) wait_vmcnt<2 * CI>();
        else if (later == 1) wait_vmcnt<CI>();
        else wait_vmcnt<0>();
        wait_lgkmcnt0();
        block_barrier();                                // every wave done with k-tile kt - 1
        if (kt + RS_STAGES - 1 < nk) issue(kt + RS_STAGES - 1);
        const uint16_t* st = smem + (kt % RS_STAGES) * STAGE;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int ch = (2 * wave + ss) * 2 + kh;
            const bf16x8 xf = *reinterpret_cast<const bf16x8*>(st + rl * BK + ((ch ^ rswz(rl)) * 8));
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const int rw = TOK + p * 32 + rl;
                const bf16x8 wf = *reinterpret_cast<const bf16x8*>(st + rw * BK + ((ch ^ rswz(rw)) * 8));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc, 0, 0, 0);
            }
        }
    }
    // the two chains meet: logit = (slices 0-1) + (slices 2-3)
    wait_lgkmcnt0();
    block_barrier();
    float* part = reinterpret_cast<float*>(smem);       // [16][64]
    if (wave == 1) {
#pragma unroll
        for (int v = 0; v < 16; ++v) part[v * 64 + lane] = acc[v];
    }
    __syncthreads();
    if (wave == 1) return;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += part[v * 64 + lane];
    // lane holds experts et*32 + 8q + 4*kh + [0, 4) of token t0 + rl
    const int64_t t = t0 + rl;
    if (t < a.T) {
        float* zrow = zout + t * EP + et * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(zrow + 8 * q + 4 * kh) =
                make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
}

// grid: ceil(T / 4); 4 waves, one token each: scores and routing by the wave.
__global__ __launch_bounds__(256) void route_select_kernel(RouteV2Args a, const float* z,
                                                           int EP, int EPL, int LG) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    const int e0 = lane * EPL;
    float s[4], c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        s[q] = 0.f;
        c[q] = -INFINITY;
        const int e = e0 + q;
        if (q < EPL && e < a.E) {
            s[q] = sigmoid_score(z[t * EP + e]);
            c[q] = s[q] + a.bias[e];
        }
    }
    const bool valid = a.mask == nullptr || a.mask[t] != 0;
    wave_route(t, lane, a.E, EPL, LG, a.G, a.NG, a.TG, a.K, a.norm, a.rsf, valid, s, c, a.ids, a.w);
}

}  // namespace

bool route_bf16_path(const Dims& d) {
    return d.bf16 && d.E <= 128 && d.NG <= RV_NGMAX && d.G % 4 == 0;
}

// planes of W_r, then the partial logits of the few-token path
static size_t route_planes_bytes(const Dims& d) {
    return (static_cast<size_t>(3) * d.E * d.H * sizeof(uint16_t) + 255) / 256 * 256;
}

size_t route_ws_bytes(const Dims& d) {
    if (!route_bf16_path(d)) return 0;
    const int EP = d.E <= 64 ? 64 : 128;
    return route_planes_bytes(d) + static_cast<size_t>(RS_TMAX) * EP * sizeof(float);
}

hipError_t route_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {nullptr};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
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
        if (d.T <= RS_TMAX) {
            // few tokens: logits over many small workgroups, then a scoring
            // and routing pass
            float* z = reinterpret_cast<float*>(static_cast<char*>(ws) + route_planes_bytes(d));
            const unsigned nt = static_cast<unsigned>((d.T + 31) / 32);
            const int EP = d.E <= 64 ? 64 : 128;
            if (EP == 64)
                hipLaunchKernelGGL(route_logits_kernel<64>, dim3(nt, 2), dim3(128), 0, stream, a, z);
            else
                hipLaunchKernelGGL(route_logits_kernel<128>, dim3(nt, 4), dim3(128), 0, stream, a, z);
            hipLaunchKernelGGL(route_select_kernel, dim3(static_cast<unsigned>((d.T + 3) / 4)), dim3(256), 0,
                               stream, a, z, EP, d.EPL, d.LG);
            return hipGetLastError();
        }
        // tokens per workgroup: the fewest (32 TM, TM = 4..6) whose grid fits
        // in one round over the CUs, else the most
        const int ncu = cu_count();
        int tm = 6;
        for (int c = 4; c <= 6; ++c) {
            if ((d.T + 32 * c - 1) / (32 * c) <= ncu) { tm = c; break; }
        }
        const dim3 grid(static_cast<unsigned>((d.T + 32 * tm - 1) / (32 * tm)));
#define RV_LAUNCH(TM_, EP_, KM_) \
        hipLaunchKernelGGL((route_bf16_kernel<TM_, EP_, KM_>), grid, dim3(512), 0, stream, a)
#define RV_BY_TM(EP_, KM_)                    \
        if (tm == 4) RV_LAUNCH(4, EP_, KM_);  \
        else if (tm == 5) RV_LAUNCH(5, EP_, KM_); \
        else RV_LAUNCH(6, EP_, KM_);
        if (d.E <= 64) {
            if (d.K <= 8) { RV_BY_TM(64, 8) } else { RV_BY_TM(64, 16) }
        } else {
            if (d.K <= 8) { RV_BY_TM(128, 8) } else { RV_BY_TM(128, 16) }
        }
#undef RV_BY_TM
#undef RV_LAUNCH
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

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

}  // namespace

hipError_t launch_route(const Dims& d, const void* x, const float* router_w, const float* e_bias,
                        const uint8_t* mask, int32_t* topk_ids, float* topk_w,
                        hipStream_t stream) {
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

// The attention half of a LingBot-Video DiT layer on gfx950: q/k head norms
// with the rotary embedding, and masked per-sample attention.
//
// What is computed (prhub summary of sglang PR #32341, the
// LingBotVideoAttention excerpt under "关键源码片段" and "实现拆解" step 2):
// q, k, v come from one fused projection (rows of q, then k, then v);
// q and k get an RMSNorm over each head's D = 128 channels with a weight
// (fp32), rounded to bf16, then the rotary embedding with neox style off
// (channels 2i and 2i+1 turned by the angle of the caller's cos / sin tables),
// rounded to bf16; attention is non-causal, scale 1 / sqrt(D), over the
// valid tokens of the query's own sample (samples are runs of S tokens; a
// padding query's output is 0).
//
// Prep (attn_prep_kernel): one workgroup per 64 tokens of one sample and one
// head; a wave normalises and rotates one (token, head) row of q and of k at
// a time (a lane owns the channel pair 2l, 2l+1), and the 64 tokens' v rows
// are transposed through LDS into vt [B][heads][D][Sp] (keys contiguous per
// channel, Sp = S rounded up to 64, zeros past S).  Inside every 16 keys the
// positions of keys 4-7 and 8-11 are swapped (bits 2 and 3 of the key index),
// which puts, for each half of a wave, the keys that its half of the score
// accumulator holds next to each other (see the attention kernel).
//
// Attention (attn_fwd_kernel): one workgroup of 8 waves per 256 queries of
// one (sample, head); a wave owns 32 queries.  Per 64-key tile the scores are
// formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (keys are the
// MFMA's rows, so a lane holds one query and 32 of the tile's keys, and the
// softmax statistics stay in the lane but for one exchange between the two
// half-waves); the online softmax runs in the exp2 domain with a lazy
// rescale (the running maximum moves only when a score exceeds it by 2^8);
// then O^T += V^T P^T, whose B operand is the score accumulator itself,
// rounded to bf16: the k order of that MFMA is the accumulator's key order,
// and vt's swapped positions give the V^T operand the same order.  K and V^T
// tiles come from global memory straight into LDS (global_load_lds_dwordx4,
// three stages, chunks XOR-swizzled per row), issued by waves 0-3 between
// their score MFMAs; waves 4-7 run half a tile behind waves 0-3 (see
// attn_fwd_kernel).
#include "lbv_internal.h"
#include "lbv_pipe.h"

namespace lbv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;           // head dim
constexpr int KT = 64;           // keys per tile
constexpr int QW = 32;           // queries per wave
constexpr int NWV = 8;           // waves per workgroup
constexpr int QB = QW * NWV;     // queries per workgroup
constexpr int MAXW = 1024;       // 64-key mask words per sample (S <= 65536)

// ---------------------------------------------------------------------------
// prep
// ---------------------------------------------------------------------------

struct PrepArgs {
    const uint16_t* qkv;   // [T, 3H] bf16
    const float* gq;       // [D]
    const float* gk;       // [D]
    const float* cs;       // [T, D/2]
    const float* sn;       // [T, D/2]
    uint16_t* q;           // [T, H] bf16
    uint16_t* k;           // [T, H] bf16
    uint16_t* vt;          // [B, heads, D, Sp] bf16
    float eps;
    int S, Sp, H, heads;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// RMSNorm of one head row (the lane's pair x0, x1 of 2 * 64 channels),
// rounded to bf16, then the pair's rotation, rounded to bf16 again.
__device__ __forceinline__ uint32_t norm_rope(uint32_t w, float g0, float g1, float c, float s,
                                              float eps) {
    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
    float ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    const uint32_t nw = pack_bf16x2(x0 * r * g0, x1 * r * g1);
    const float n0 = bf16_lo(nw), n1 = bf16_hi(nw);
    return pack_bf16x2(n0 * c - n1 * s, n1 * c + n0 * s);
}

__global__ __launch_bounds__(256) void attn_prep_kernel(PrepArgs a) {
    __shared__ uint16_t vs[64][D + 8];           // +8: rows 272 bytes apart
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y, c0 = blockIdx.x * 64;
    const int64_t tb = static_cast<int64_t>(b) * a.S;   // first token of the sample
    const int H3 = 3 * a.H;
    const float gq0 = a.gq[2 * lane], gq1 = a.gq[2 * lane + 1];
    const float gk0 = a.gk[2 * lane], gk1 = a.gk[2 * lane + 1];
    for (int i = 0; i < 16; ++i) {
        const int jj = c0 + wave * 16 + i;
        if (jj >= a.S) break;
        const int64_t t = tb + jj;
        const uint32_t* row = reinterpret_cast<const uint32_t*>(a.qkv + t * H3 + h * D);
        const uint32_t wq = row[lane];
        const uint32_t wk = row[a.H / 2 + lane];
        const float c = a.cs[t * (D / 2) + lane], s = a.sn[t * (D / 2) + lane];
        reinterpret_cast<uint32_t*>(a.q + t * a.H + h * D)[lane] = norm_rope(wq, gq0, gq1, c, s, a.eps);
        reinterpret_cast<uint32_t*>(a.k + t * a.H + h * D)[lane] = norm_rope(wk, gk0, gk1, c, s, a.eps);
    }
    // v rows of the 64 tokens (zeros past the sample) into LDS, 16 bytes a lane
    for (int u = tid; u < 64 * (D / 8); u += 256) {
        const int r = u / (D / 8), ch = u % (D / 8);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c0 + r < a.S)
            v = *reinterpret_cast<const u32x4*>(a.qkv + (tb + c0 + r) * H3 + 2 * a.H + h * D + ch * 8);
        *reinterpret_cast<uint2*>(&vs[r][ch * 8]) = uint2{v[0], v[1]};
        *reinterpret_cast<uint2*>(&vs[r][ch * 8 + 4]) = uint2{v[2], v[3]};
    }
    __syncthreads();
    // vt rows: channel d, 8 positions per 16-byte store; position p holds key
    // p with bits 2 and 3 swapped
    const int d = tid % D;
    uint16_t* vrow = a.vt + ((static_cast<int64_t>(b) * a.heads + h) * D + d) * a.Sp + c0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int p0 = (tid / D) * 32 + g * 8;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int pa = p0 + 2 * e, pb = pa + 1;
            const int ka = (pa & ~12) | ((pa & 4) << 1) | ((pa & 8) >> 1);
            const int kb = (pb & ~12) | ((pb & 4) << 1) | ((pb & 8) >> 1);
            w[e] = static_cast<uint32_t>(vs[ka][d]) | (static_cast<uint32_t>(vs[kb][d]) << 16);
        }
        *reinterpret_cast<u32x4*>(vrow + p0) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------

struct AttnArgs {
    const uint16_t* q;     // [T, H]
    const uint16_t* k;     // [T, H]
    const uint16_t* vt;    // [B, heads, D, Sp]
    const uint8_t* mask;   // [T] or null
    uint16_t* o;           // [T, H]
    int S, Sp, H, heads, B, nqt;
};

// LDS: three stages of [K tile: 64 rows x 256 bytes | V^T tile: 128 rows x 128
// bytes], then the sample's key mask, 64 keys per word.
constexpr int KBYTES = KT * D * 2;               // 16 KB
constexpr int VBYTES = D * KT * 2;               // 16 KB
constexpr int STAGE_BYTES = KBYTES + VBYTES;
constexpr int NSTG = 3;

// Two wave groups share each SIMD (wave w and w + 4): group A (waves 0-3)
// runs, between two barriers, the scores of tile j, their softmax and the PV
// product of tile j; group B (waves 4-7) runs the softmax and PV product of
// tile j - 1 and then the scores of tile j.  One barrier per tile holds the
// groups half a tile apart, so on every SIMD one wave's softmax (vector ALU)
// runs beside the other wave's matrix products.  Group A also issues the
// copies of tile j + 1 (into the stage that held tile j - 2, which both groups
// finished before the previous barrier) and waits for them before the
// barrier; B reads tile j - 1's V^T and tile j's K, both landed.
__global__ __launch_bounds__(NWV * 64) void attn_fwd_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) char lds[NSTG * STAGE_BYTES];
    __shared__ unsigned long long kmask[MAXW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool grpA = wave < 4;
    const int hl = lane >> 5, ql = lane & 31;
    // workgroups of one (sample, head) are consecutive in the logical order
    // and share an XCD (and its L2) for the K and V^T tiles
    const int lg = xcd_logical_block(blockIdx.x, gridDim.x);
    const int qt = lg % a.nqt;
    const int bh = lg / a.nqt;
    const int head = bh % a.heads, b = bh / a.heads;
    const int64_t tb = static_cast<int64_t>(b) * a.S;
    const int nkt = (a.S + KT - 1) / KT;

    // ---- the sample's key mask (bit j of word w: key 64 w + j is valid) ----
    for (int w = wave; w < nkt; w += NWV) {
        const int j = w * KT + lane;
        bool valid = j < a.S;
        if (valid && a.mask) valid = a.mask[tb + j] != 0;
        const unsigned long long bits = __ballot(valid);
        if (lane == 0) kmask[w] = bits;
    }

    // ---- this wave's 32 queries: q fragments for the 8 16-deep steps -------
    const int qrow = qt * QB + wave * QW + ql;           // query index in the sample
    const int qrc = qrow < a.S ? qrow : a.S - 1;
    bf16x8 qf[D / 16];
    {
        const uint16_t* qp = a.q + (tb + qrc) * a.H + head * D + hl * 8;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qp + st * 16);
    }

    // ---- copy sources (group A): K tile rows w*16 + 4i + lane/16, V^T rows
    // w*32 + 8i + lane/8; lane lands at physical chunk lane%16 (K) or lane%8
    // (V^T), holding logical chunk c ^ swizzle(row) ------------------------------
    const char* kbase = reinterpret_cast<const char*>(a.k + tb * a.H + head * D);
    const char* vbase = reinterpret_cast<const char*>(
        a.vt + (static_cast<int64_t>(b) * a.heads + head) * D * a.Sp);
    uint32_t koff_col[4], voff[4];
    int krow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rk = (wave & 3) * 16 + i * 4 + lane / 16;
        krow[i] = rk;
        koff_col[i] = ((lane % 16) ^ (rk & 15)) * 16;
        const int rv = (wave & 3) * 32 + i * 8 + lane / 8;
        voff[i] = rv * a.Sp * 2 + ((lane % 8) ^ ((rv >> 1) & 7)) * 16;
    }
    const uint32_t lds0 = lds_addr(lds);
    auto copy_k = [&](int stage, int kt, int i) {
        int j = kt * KT + krow[i];
        j = j < a.S ? j : a.S - 1;
        const uint32_t off = static_cast<uint32_t>(j) * a.H * 2 + koff_col[i];
        lds_dma16_sb<0>(kbase, off, lds0 + stage * STAGE_BYTES + (wave & 3) * 4096 + i * 1024);
    };
    auto copy_v = [&](int stage, int kt, int i) {
        lds_dma16_sb<0>(vbase + kt * KT * 2, voff[i],
                        lds0 + stage * STAGE_BYTES + KBYTES + (wave & 3) * 4096 + i * 1024);
    };

    // ---- fragment addresses ----------------------------------------------------
    // K (A operand of the score MFMA): key row 32 blk + ql, channels 16 st + 8 hl
    auto kfrag = [&](int stage, int blk, int st) -> bf16x8 {
        const int r = blk * 32 + ql;
        const char* p = lds + stage * STAGE_BYTES + r * 256 + (((2 * st + hl) ^ (r & 15)) * 16);
        return *reinterpret_cast<const bf16x8*>(p);
    };
    // V^T (A operand of the PV MFMA): channel row 32 dblk + ql, positions
    // 16 c + 8 hl .. + 7
    auto vfrag = [&](int stage, int dblk, int c) -> bf16x8 {
        const int r = dblk * 32 + ql;
        const char* p = lds + stage * STAGE_BYTES + KBYTES + r * 128 + (((2 * c + hl) ^ ((r >> 1) & 7)) * 16);
        return *reinterpret_cast<const bf16x8*>(p);
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
    f32x16 sacc[2];
    // running maximum (log2 domain, scaled) and this half-wave's running sum
    float mrun = -1e30f, lrun = 0.0f;
    const float csc = 1.4426950408889634f / sqrtf(static_cast<float>(D));   // log2(e) / sqrt(D)

    // scores S^T = K Q^T of tile kt; group A also copies tile kt + 1
    auto scores = [&](int kt, bool copy) {
        const int stg = kt % NSTG;
        const int cst = (kt + 1) % NSTG;
        bf16x8 kf0 = kfrag(stg, 0, 0), kf1 = kfrag(stg, 1, 0);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            bf16x8 nk0, nk1;
            if (st + 1 < D / 16) {
                nk0 = kfrag(stg, 0, st + 1);
                nk1 = kfrag(stg, 1, st + 1);
            }
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[st], st == 0 ? f32x16{} : sacc[0], 0, 0, 0);
            if (copy && st < 4) copy_k(cst, kt + 1, st);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf1, qf[st], st == 0 ? f32x16{} : sacc[1], 0, 0, 0);
            if (copy && st < 4) copy_v(cst, kt + 1, st);
            __builtin_amdgcn_sched_barrier(0);
            if (st + 1 < D / 16) {
                kf0 = nk0;
                kf1 = nk1;
            }
        }
    };

    // online softmax of tile kt's scores (exp2 domain, lazy rescale), then
    // O^T += V^T P^T
    auto softmax_pv = [&](int kt) {
        const int stg = kt % NSTG;
        const unsigned long long km = kmask[kt];
        if (km != ~0ull) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = blk * 32 + (r >> 2) * 8 + hl * 4 + (r & 3);
                    if (!((km >> key) & 1ull)) sacc[blk][r] = -3.0e38f;
                }
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[blk][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun, mx * csc);
        if (__ballot(mnew > mrun + 8.0f)) {
            // some query's scores rose past 2^8 times its reference: move the
            // reference of every query whose maximum rose
            const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
            lrun *= alpha;
#pragma unroll
            for (int i = 0; i < D / 32; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
            mrun = mnew;
        }
        bf16x8 pf[4];
        float psum = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[blk][half * 8 + e], csc, -mrun));
                    psum += p[e];
                }
                const u32x4 w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                 pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
                pf[blk * 2 + half] = __builtin_bit_cast(bf16x8, w);
            }
        lrun += psum;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            bf16x8 vf[D / 32];
#pragma unroll
            for (int dblk = 0; dblk < D / 32; ++dblk) vf[dblk] = vfrag(stg, dblk, c);
#pragma unroll
            for (int dblk = 0; dblk < D / 32; ++dblk)
                oacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dblk], pf[c], oacc[dblk], 0, 0, 0);
        }
    };

    // ---- prologue: tile 0 into stage 0 ----------------------------------------------
    if (grpA) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            copy_k(0, 0, i);
            copy_v(0, 0, i);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();                                  // mask words and stage 0 visible

    // each group passes nkt barriers, one per tile (separate loops keep each
    // group's registers to its own schedule)
    if (grpA) {
        for (int kt = 0; kt < nkt; ++kt) {
            scores(kt, kt + 1 < nkt);
            softmax_pv(kt);
            wait_vmcnt<0>();                          // tile kt + 1 landed
            wait_lgkmcnt0();
            block_barrier();
        }
    } else {
        scores(0, false);
        wait_lgkmcnt0();
        block_barrier();
        for (int kt = 1; kt < nkt; ++kt) {
            softmax_pv(kt - 1);
            scores(kt, false);
            wait_lgkmcnt0();
            block_barrier();
        }
        softmax_pv(nkt - 1);
    }

    // ---- output: O = O^T / l; lane holds its query's channels 32 dblk + 8 j +
    // 4 hl + [0, 4) ------------------------------------------------------------------
    const float ltot = lrun + __shfl_xor(lrun, 32);
    if (qrow >= a.S) return;
    const int64_t t = tb + qrow;
    const bool valid = (a.mask == nullptr || a.mask[t] != 0) && ltot > 0.0f;
    const float inv = valid ? 1.0f / ltot : 0.0f;
    uint16_t* orow = a.o + t * a.H + head * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint2 w = {pack_bf16x2(oacc[dblk][4 * j] * inv, oacc[dblk][4 * j + 1] * inv),
                             pack_bf16x2(oacc[dblk][4 * j + 2] * inv, oacc[dblk][4 * j + 3] * inv)};
            *reinterpret_cast<uint2*>(orow + dblk * 32 + j * 8 + hl * 4) = w;
        }
}

}  // namespace

int attn_sp(int S) { return (S + KT - 1) / KT * KT; }

hipError_t launch_attn_prep(int B, int S, int H, int heads, const void* qkv, const float* gq,
                            const float* gk, const float* cs, const float* sn, float eps, void* q,
                            void* k, void* vt, hipStream_t stream) {
    PrepArgs a;
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.gq = gq;
    a.gk = gk;
    a.cs = cs;
    a.sn = sn;
    a.q = static_cast<uint16_t*>(q);
    a.k = static_cast<uint16_t*>(k);
    a.vt = static_cast<uint16_t*>(vt);
    a.eps = eps;
    a.S = S;
    a.Sp = attn_sp(S);
    a.H = H;
    a.heads = heads;
    hipLaunchKernelGGL(attn_prep_kernel, dim3((S + 63) / 64, heads, B), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_attn_core(int B, int S, int H, int heads, const void* q, const void* k,
                            const void* vt, const uint8_t* mask, void* o, hipStream_t stream) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.vt = static_cast<const uint16_t*>(vt);
    a.mask = mask;
    a.o = static_cast<uint16_t*>(o);
    a.S = S;
    a.Sp = attn_sp(S);
    a.H = H;
    a.heads = heads;
    a.B = B;
    a.nqt = (S + QB - 1) / QB;
    const int64_t grid = static_cast<int64_t>(B) * heads * a.nqt;
    hipLaunchKernelGGL(attn_fwd_kernel, dim3(static_cast<unsigned>(grid)), dim3(NWV * 64), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace lbv

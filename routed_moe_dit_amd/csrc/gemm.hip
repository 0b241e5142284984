// Grouped expert matmuls and the weighted combine of the LingBot-Video MoE
// block on gfx950.
//
// What is computed (prhub summary of sglang PR #32341, "实现拆解" step 1 and
// the LingBotVideoSparseMoeBlock excerpt: SiLU-gated experts, w13 packed
// [E, 2I, H] with gate rows then up rows, router weight applied on the expert
// output, no second scaling, shared expert added; vLLM-Omni LingBot-Video
// article, "MoE 实现的源码级要点": grouped bf16 matmuls over expert-sorted
// token copies, fp32 weighted restore):
//   gate/up:  act[r] = silu(W_gate x[t]) * (W_up x[t])   per sorted row r
//   down:     y[r]   = W2 act[r]
//   combine:  out[t] = sum_k w[t,k] y[inv(t,k)] + sum_j y[inv(t,K+j)]
//
// Segments s < E are routed experts, s >= E shared pseudo-experts (a width
// I slice of the shared MLP, exact by linearity of the down projection).
//
// bf16 path: one workgroup (4 waves, 256 threads) computes a BM x BN tile of
// one segment with v_mfma_f32_32x32x16_bf16.  A and B tiles (K-contiguous,
// BK = 64 bf16 = 128 B per row) go global -> registers -> LDS, double-buffered
// so the next tile's loads are in flight while the current one is multiplied.
// LDS rows are 8 chunks of 16 B, chunk c of row r stored at c ^ (r & 7), so
// that the 16-byte fragment reads of 8 consecutive rows hit 8 different bank
// groups.  Tiles never cross a segment: the tile list is rebuilt from
// `offsets` by every workgroup (no host read-back of segment sizes), and
// the grid is sized for the worst case; surplus workgroups exit at once.
// For the gate/up matmul a B tile holds BN/2 gate rows and the matching BN/2
// up rows, and each wave's accumulators for gate column n and up column n sit
// in the same lane and register, so silu(g) * u is formed in registers.
#include "lbv_internal.h"

namespace lbv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const void* A;          // gate/up: x [T, H];  down: act [rows, I]
    const void* B;          // gate/up: w13 [E, 2I, H];  down: w2 [E, H, I]
    const void* Bsh;        // gate/up: shared_w13 [2 Is, H];  down: shared_w2 [H, Is]
    const int32_t* offsets; // [S + 1]
    const int32_t* rows;    // gate/up: sorted_rows (slot ids)
    void* C;                // gate/up: act [rows, I];  down: y [rows, H]
    int64_t T;
    int H, I, E, NS, KS, S;
    int kdim;               // reduction length: H (gate/up) or I (down)
    int ncols;              // output columns: I (gate/up) or H (down)
    int ntn;                // n-tiles per m-tile
};

// Finds the segment and first row of logical m-tile `mt` for tiles of BM rows
// (every segment is cut into ceil(rows / BM) tiles, in segment order).
// Returns false, uniformly over the block, if `mt` is past the last tile.
// Two block-wide scans over the segment tile counts (S <= 512).
// s_tmp: 8 ints of LDS, s_sel: 2 ints of LDS.
__device__ bool find_tile(const GemmArgs& a, int BM, int mt, int* seg_out, int* m0_out,
                          int* s_tmp, int* s_sel) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int c[2], inc[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int s = tid + p * 256;
        c[p] = 0;
        if (s < a.S) {
            const int n = a.offsets[s + 1] - a.offsets[s];
            c[p] = n > 0 ? (n + BM - 1) / BM : 0;
        }
        int v = c[p];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(v, off);
            if (lane >= off) v += o;
        }
        inc[p] = v;
        if (lane == 63) s_tmp[p * 4 + wave] = v;
    }
    if (tid == 0) s_sel[0] = -1;
    __syncthreads();
    int base0 = 0, base1 = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    for (int w = 0; w < wave; ++w) {
        base0 += s_tmp[w];
        base1 += s_tmp[4 + w];
    }
    const int st0 = base0 + inc[0] - c[0];
    const int st1 = base1 + inc[1] - c[1];
    if (c[0] > 0 && mt >= st0 && mt < st0 + c[0]) { s_sel[0] = tid; s_sel[1] = st0; }
    if (c[1] > 0 && mt >= st1 && mt < st1 + c[1]) { s_sel[0] = tid + 256; s_sel[1] = st1; }
    __syncthreads();
    const int seg = s_sel[0];
    if (seg < 0) return false;
    *seg_out = seg;
    *m0_out = (mt - s_sel[1]) * BM;
    return true;
}

template <int BM, int BN, int BK, int WM, int WN, int MODE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    static_assert(WM * WN == 4, "4 waves");
    static_assert(BK == 64, "LDS swizzle assumes 8 chunks of 16 B per row");
    constexpr int TM = BM / (WM * 32);
    constexpr int TN = BN / (WN * 32);
    static_assert(TM >= 1 && TN >= 1, "tile");
    static_assert(MODE == 1 || TN % 2 == 0, "gate/up tiles come in pairs");
    constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
    constexpr int AR = BM / 32, BR = BN / 32;   // load rounds (32 rows per round)

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_ELEMS + B_ELEMS)];
    __shared__ int s_tmp[8];
    __shared__ int s_sel[2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
    const int mt = lid / a.ntn;
    const int nt = lid % a.ntn;
    int seg, m0;
    if (!find_tile(a, BM, mt, &seg, &m0, s_tmp, s_sel)) return;

    const int seg_r0 = a.offsets[seg];
    const int seg_n = a.offsets[seg + 1] - seg_r0;
    const int kdim = a.kdim;
    const bool shared_seg = seg >= a.E;
    const int jsh = seg - a.E;
    const int Is = a.NS * a.I;

    // ---- per-thread global row pointers --------------------------------------
    const int lrow = tid >> 3;        // row within a 32-row round
    const int lchunk = tid & 7;       // 16-byte chunk within the 128-byte row slice
    const uint16_t* aptr[AR];
    const uint16_t* bptr[BR];
#pragma unroll
    for (int r = 0; r < AR; ++r) {
        int m = m0 + r * 32 + lrow;
        if (m >= seg_n) m = seg_n - 1;
        if (MODE == 0) {
            int slot = a.rows[seg_r0 + m];
            int64_t tok = slot / a.KS;
            if (tok < 0) tok = 0;
            if (tok >= a.T) tok = a.T - 1;
            aptr[r] = static_cast<const uint16_t*>(a.A) + tok * a.H + lchunk * 8;
        } else {
            aptr[r] = static_cast<const uint16_t*>(a.A) + static_cast<int64_t>(seg_r0 + m) * a.I +
                      lchunk * 8;
        }
    }
#pragma unroll
    for (int r = 0; r < BR; ++r) {
        const int br = r * 32 + lrow;    // B tile row
        if (MODE == 0) {
            const int half = br / (BN / 2);
            int n = nt * (BN / 2) + (br % (BN / 2));
            if (n >= a.I) n = a.I - 1;
            int64_t row;
            const uint16_t* base;
            if (!shared_seg) {
                base = static_cast<const uint16_t*>(a.B) + static_cast<int64_t>(seg) * 2 * a.I * a.H;
                row = half ? a.I + n : n;
            } else {
                base = static_cast<const uint16_t*>(a.Bsh);
                row = half ? Is + jsh * a.I + n : jsh * a.I + n;
            }
            bptr[r] = base + row * a.H + lchunk * 8;
        } else {
            int n = nt * BN + br;
            if (n >= a.H) n = a.H - 1;
            if (!shared_seg)
                bptr[r] = static_cast<const uint16_t*>(a.B) + static_cast<int64_t>(seg) * a.H * a.I +
                          static_cast<int64_t>(n) * a.I + lchunk * 8;
            else
                bptr[r] = static_cast<const uint16_t*>(a.Bsh) + static_cast<int64_t>(n) * Is +
                          jsh * a.I + lchunk * 8;
        }
    }

    // ---- LDS addressing (swizzled 16-byte chunks) ------------------------------
    // store: row lrow + 32 r, chunk lchunk  -> element offset
    const int st_off = lrow * BK + ((lchunk ^ (lrow & 7)) * 8);   // (r*32 + lrow) & 7 == lrow & 7

    u32x4 ra[AR], rb[BR];

    // ---- wave tile ----------------------------------------------------------------
    const int wm = wave / WN, wn = wave % WN;
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

    // fragment rows in LDS
    int arow[TM], brow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) arow[i] = wm * TM * 32 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (MODE == 0) {
            constexpr int HT = TN / 2;
            if (j < HT) brow[j] = wn * HT * 32 + j * 32 + (lane & 31);
            else brow[j] = BN / 2 + wn * HT * 32 + (j - HT) * 32 + (lane & 31);
        } else {
            brow[j] = wn * TN * 32 + j * 32 + (lane & 31);
        }
    }
    const int khalf = lane >> 5;

    const int nk = kdim / BK;
    // prologue: k-tile 0 -> registers -> LDS buffer 0
#pragma unroll
    for (int r = 0; r < AR; ++r) ra[r] = *reinterpret_cast<const u32x4*>(aptr[r]);
#pragma unroll
    for (int r = 0; r < BR; ++r) rb[r] = *reinterpret_cast<const u32x4*>(bptr[r]);
#pragma unroll
    for (int r = 0; r < AR; ++r) *reinterpret_cast<u32x4*>(smem + r * 32 * BK + st_off) = ra[r];
#pragma unroll
    for (int r = 0; r < BR; ++r)
        *reinterpret_cast<u32x4*>(smem + A_ELEMS + r * 32 * BK + st_off) = rb[r];
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) {   // next k-tile's global loads stay in flight during the MFMAs
            const int k0 = (kt + 1) * BK;
#pragma unroll
            for (int r = 0; r < AR; ++r) ra[r] = *reinterpret_cast<const u32x4*>(aptr[r] + k0);
#pragma unroll
            for (int r = 0; r < BR; ++r) rb[r] = *reinterpret_cast<const u32x4*>(bptr[r] + k0);
        }
        const uint16_t* As = smem + (kt & 1) * (A_ELEMS + B_ELEMS);
        const uint16_t* Bs = As + A_ELEMS;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + khalf;
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(As + arow[i] * BK + ((ch ^ (arow[i] & 7)) * 8));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + brow[j] * BK + ((ch ^ (brow[j] & 7)) * 8));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            uint16_t* An = smem + ((kt + 1) & 1) * (A_ELEMS + B_ELEMS);
#pragma unroll
            for (int r = 0; r < AR; ++r) *reinterpret_cast<u32x4*>(An + r * 32 * BK + st_off) = ra[r];
#pragma unroll
            for (int r = 0; r < BR; ++r)
                *reinterpret_cast<u32x4*>(An + A_ELEMS + r * 32 * BK + st_off) = rb[r];
        }
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------------
    uint16_t* C = static_cast<uint16_t*>(a.C);
    if (MODE == 0) {
        constexpr int HT = TN / 2;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < HT; ++j) {
                const int col = nt * (BN / 2) + wn * HT * 32 + j * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = wm * TM * 32 + i * 32 + 8 * (q >> 2) + 4 * khalf + (q & 3);
                    const int m = m0 + row;
                    if (m < seg_n && col < a.I) {
                        const float g = acc[i][j][q];
                        const float u = acc[i][j + HT][q];
                        const float v = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                        C[static_cast<int64_t>(seg_r0 + m) * a.I + col] = f32_to_bf16(v);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = nt * BN + wn * TN * 32 + j * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = wm * TM * 32 + i * 32 + 8 * (q >> 2) + 4 * khalf + (q & 3);
                    const int m = m0 + row;
                    if (m < seg_n && col < a.H)
                        C[static_cast<int64_t>(seg_r0 + m) * a.H + col] = f32_to_bf16(acc[i][j][q]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 storage path: plain LDS-tiled FMA (same segment tiling, 32 x 32 tiles).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
    constexpr int BM = 32, BN = 32, BK = 32;
    __shared__ float As[BM][BK + 1];
    __shared__ float Bg[BN][BK + 1];
    __shared__ float Bu[BN][BK + 1];
    __shared__ int s_tmp[8];
    __shared__ int s_sel[2];

    const int tid = threadIdx.x;
    const int mt = blockIdx.x / a.ntn, nt = blockIdx.x % a.ntn;
    int seg, m0;
    if (!find_tile(a, BM, mt, &seg, &m0, s_tmp, s_sel)) return;
    const int seg_r0 = a.offsets[seg];
    const int seg_n = a.offsets[seg + 1] - seg_r0;
    const bool shared_seg = seg >= a.E;
    const int jsh = seg - a.E;
    const int Is = a.NS * a.I;
    const float* A = static_cast<const float*>(a.A);
    const float* B = static_cast<const float*>(a.B);
    const float* Bsh = static_cast<const float*>(a.Bsh);

    const int tx = tid & 15, ty = tid >> 4;
    float accg[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, accu[2][2] = {{0.f, 0.f}, {0.f, 0.f}};

    for (int k0 = 0; k0 < a.kdim; k0 += BK) {
        for (int i = tid; i < BM * BK; i += 256) {
            const int r = i / BK, c = i % BK;
            int m = m0 + r;
            if (m >= seg_n) m = seg_n - 1;
            const float* rowp;
            if (MODE == 0) {
                int64_t tok = a.rows[seg_r0 + m] / a.KS;
                if (tok < 0) tok = 0;
                if (tok >= a.T) tok = a.T - 1;
                rowp = A + tok * a.H;
            } else {
                rowp = A + static_cast<int64_t>(seg_r0 + m) * a.I;
            }
            As[r][c] = rowp[k0 + c];
            int n = nt * BN + r;
            if (MODE == 0) {
                if (n >= a.I) n = a.I - 1;
                const float* g;
                const float* u;
                if (!shared_seg) {
                    const float* base = B + static_cast<int64_t>(seg) * 2 * a.I * a.H;
                    g = base + static_cast<int64_t>(n) * a.H;
                    u = base + static_cast<int64_t>(a.I + n) * a.H;
                } else {
                    g = Bsh + static_cast<int64_t>(jsh * a.I + n) * a.H;
                    u = Bsh + static_cast<int64_t>(Is + jsh * a.I + n) * a.H;
                }
                Bg[r][c] = g[k0 + c];
                Bu[r][c] = u[k0 + c];
            } else {
                if (n >= a.H) n = a.H - 1;
                const float* g = shared_seg
                    ? Bsh + static_cast<int64_t>(n) * Is + jsh * a.I
                    : B + static_cast<int64_t>(seg) * a.H * a.I + static_cast<int64_t>(n) * a.I;
                Bg[r][c] = g[k0 + c];
            }
        }
        __syncthreads();
        for (int k = 0; k < BK; ++k) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float xv = As[ty * 2 + i][k];
                    accg[i][j] += xv * Bg[tx * 2 + j][k];
                    if (MODE == 0) accu[i][j] += xv * Bu[tx * 2 + j][k];
                }
        }
        __syncthreads();
    }
    float* C = static_cast<float*>(a.C);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int m = m0 + ty * 2 + i;
            const int n = nt * BN + tx * 2 + j;
            if (m < seg_n && n < a.ncols) {
                float v = accg[i][j];
                if (MODE == 0) v = v * accu[i][j] / (1.0f + expf(-v));
                C[static_cast<int64_t>(seg_r0 + m) * a.ncols + n] = v;
            }
        }
}

// ---------------------------------------------------------------------------
// Combine: one wave per token, 8 consecutive outputs per lane per step.
// ---------------------------------------------------------------------------
struct CombArgs {
    const void* y;
    const int32_t* inv;
    const float* w;
    void* out;
    int64_t T;
    int H, K, NS, KS;
};

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(CombArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    constexpr int MAXS = 24;   // K <= 16 plus up to 8 shared pseudo-experts
    int rows[MAXS];
    float wt[MAXS];
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        rows[k] = -1;
        wt[k] = 1.0f;
        if (k < a.KS) {
            rows[k] = a.inv[t * a.KS + k];
            if (k < a.K) wt[k] = a.w[t * a.K + k];
        }
    }
    for (int h0 = lane * 8; h0 < a.H; h0 += 512) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            const int r = rows[k];
            if (r < 0) continue;
            if (BF16) {
                const uint4 q = *reinterpret_cast<const uint4*>(
                    static_cast<const uint16_t*>(a.y) + static_cast<int64_t>(r) * a.H + h0);
                const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += wt[k] * __uint_as_float(qq[i] << 16);
                    acc[2 * i + 1] += wt[k] * __uint_as_float(qq[i] & 0xffff0000u);
                }
            } else {
                const float4* p = reinterpret_cast<const float4*>(
                    static_cast<const float*>(a.y) + static_cast<int64_t>(r) * a.H + h0);
                const float4 p0 = p[0], p1 = p[1];
                const float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wt[k] * v[i];
            }
        }
        if (BF16) {
            uint4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + t * a.H + h0) = o;
        } else {
            float4* p = reinterpret_cast<float4*>(static_cast<float*>(a.out) + t * a.H + h0);
            p[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
            p[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
    }
}

// tile shapes of the bf16 path
constexpr int G1_BM = 128, G1_BN = 128, G1_WM = 2, G1_WN = 2;
constexpr int G2_BM = 128, G2_BN = 128, G2_WM = 2, G2_WN = 2;

GemmArgs make_args(const Dims& d) {
    GemmArgs a;
    a.T = d.T;
    a.H = d.H;
    a.I = d.I;
    a.E = d.E;
    a.NS = d.NS;
    a.KS = d.KS;
    a.S = d.S;
    return a;
}

int64_t max_mtiles(const Dims& d, int BM) {
    return (d.T * d.KS + BM - 1) / BM + d.S;
}

}  // namespace

hipError_t launch_gemm_w13(const Dims& d, const void* x, const void* w13,
                           const void* shared_w13, const int32_t* offsets,
                           const int32_t* sorted_rows, void* act, hipStream_t stream) {
    GemmArgs a = make_args(d);
    a.A = x;
    a.B = w13;
    a.Bsh = shared_w13;
    a.offsets = offsets;
    a.rows = sorted_rows;
    a.C = act;
    a.kdim = d.H;
    a.ncols = d.I;
    if (d.bf16) {
        a.ntn = (d.I + G1_BN / 2 - 1) / (G1_BN / 2);
        const int64_t grid = max_mtiles(d, G1_BM) * a.ntn;
        hipLaunchKernelGGL((gemm_bf16_kernel<G1_BM, G1_BN, 64, G1_WM, G1_WN, 0>),
                           dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
    } else {
        a.ntn = (d.I + 31) / 32;
        const int64_t grid = max_mtiles(d, 32) * a.ntn;
        hipLaunchKernelGGL(gemm_f32_kernel<0>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w2(const Dims& d, const void* act, const void* w2, const void* shared_w2,
                          const int32_t* offsets, void* y, hipStream_t stream) {
    GemmArgs a = make_args(d);
    a.A = act;
    a.B = w2;
    a.Bsh = shared_w2;
    a.offsets = offsets;
    a.rows = nullptr;
    a.C = y;
    a.kdim = d.I;
    a.ncols = d.H;
    if (d.bf16) {
        a.ntn = (d.H + G2_BN - 1) / G2_BN;
        const int64_t grid = max_mtiles(d, G2_BM) * a.ntn;
        hipLaunchKernelGGL((gemm_bf16_kernel<G2_BM, G2_BN, 64, G2_WM, G2_WN, 1>),
                           dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
    } else {
        a.ntn = (d.H + 31) / 32;
        const int64_t grid = max_mtiles(d, 32) * a.ntn;
        hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const void* y, const int32_t* inv_rows,
                          const float* topk_w, void* out, hipStream_t stream) {
    CombArgs a;
    a.y = y;
    a.inv = inv_rows;
    a.w = topk_w;
    a.out = out;
    a.T = d.T;
    a.H = d.H;
    a.K = d.K;
    a.NS = d.NS;
    a.KS = d.KS;
    const unsigned grid = static_cast<unsigned>((d.T + 3) / 4);
    if (d.bf16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lbv

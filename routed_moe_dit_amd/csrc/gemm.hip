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
#include <type_traits>

#include "lbv_internal.h"
#include "lbv_pipe.h"

// Compile-time shape of the bf16 path: workgroup tile BM x BN (2 x 2 waves;
// the gate/up GEMM's BN counts gate and up rows together, BN/2 act columns
// per tile), and the k-depth BK and number STAGES of the LDS ring.
#ifndef LBV_BK
#define LBV_BK 32
#endif
#ifndef LBV_STAGES
#define LBV_STAGES 4
#endif
#ifndef LBV_KK_UNROLL
#define LBV_KK_UNROLL 2
#endif
#ifndef LBV_G1_BM
#define LBV_G1_BM 256
#endif
#ifndef LBV_G1_BN
#define LBV_G1_BN 256
#endif
#ifndef LBV_G2_BM
#define LBV_G2_BM 256
#endif
#ifndef LBV_G2_BN
#define LBV_G2_BN 256
#endif

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

// 16-byte chunk swizzle of an LDS row of BK bf16: chunk c of row r is stored at
// c ^ swz<BK>(r).  Chosen by measurement on gfx950 for the MFMA fragment read
// (lanes 0-31 read rows r0 + lane, lanes 32-63 the next chunk), whose
// ds_read_b128 then runs at ~210 B/clk/CU (conflict-free):
//   64-byte rows:  c ^ ((r >> 2) & 3)   (unswizzled: ~62, c ^ ((r>>1)&3): ~120)
//   128-byte rows: c ^ ((r >> 1) & 7)   (c ^ (r & 7): ~120)
template <int BK>
__device__ __forceinline__ int swz(int r) {
    static_assert(BK == 32 || BK == 64, "row of 64 or 128 bytes");
    return BK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

template <int BM, int BN, int BK, int STAGES, int MODE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
    // BK: bf16 per row per stage (64 or 128 bytes); STAGES: LDS ring of
    // k-tiles, STAGES - 1 of them in flight while one is multiplied.
    static_assert(STAGES == 2 || STAGES == 4, "2 or 4 stages");
    constexpr int TM = BM / 64;                  // token tiles (32 rows) per wave
    constexpr int TN = BN / 64;                  // weight-row tiles (32 rows) per wave
    static_assert(MODE == 1 || TN % 2 == 0, "gate/up tiles come in pairs");
    constexpr int STAGE = (BM + BN) * BK;        // bf16 elements per stage
    constexpr int CPR = BK / 8;                  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                // rows per 1 KB copy instruction
    constexpr int AI = BM / 4 / RPI, BI = BN / 4 / RPI;  // copies per wave per stage
    constexpr int NI = AI + BI;

    // Four distinct LDS objects (not one array indexed by kt % 4): with the
    // stage named at compile time the compiler can prove that a stage being
    // read is not one being filled by the asynchronous loads, and does not
    // drain the whole load queue before every LDS read.
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[STAGES > 2 ? STAGE : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[STAGES > 3 ? STAGE : 8];
    __shared__ int s_tmp[8];
    __shared__ int s_sel[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lid = xcd_logical_block(blockIdx.x, gridDim.x);
    const int mt = lid / a.ntn;
    const int nt = lid % a.ntn;
    int seg, m0;
    if (!find_tile(a, BM, mt, &seg, &m0, s_tmp, s_sel)) return;

    const int seg_r0 = a.offsets[seg];
    const int seg_n = a.offsets[seg + 1] - seg_r0;
    const bool shared_seg = seg >= a.E;
    const int jsh = seg - a.E;
    const int Is = a.NS * a.I;

    // ---- global source of each lane's 16-byte chunk (per copy instruction) ----
    // Instruction i of wave w fills LDS rows w*(rows/4) + RPI i + [0, RPI) of
    // the stage; lane l lands at row +l/CPR, physical chunk l%CPR, which holds
    // logical chunk (l%CPR) ^ swz(row).
    const uint16_t* aptr[AI];
    const uint16_t* bptr[BI];
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const int r = wave * (BM / 4) + i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<BK>(r);
        int m = m0 + r;
        if (m >= seg_n) m = seg_n - 1;
        if (MODE == 0) {
            int64_t tok = a.rows[seg_r0 + m] / a.KS;
            tok = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            aptr[i] = static_cast<const uint16_t*>(a.A) + tok * a.H + c * 8;
        } else {
            aptr[i] = static_cast<const uint16_t*>(a.A) + static_cast<int64_t>(seg_r0 + m) * a.I +
                      c * 8;
        }
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const int r = wave * (BN / 4) + i * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz<BK>(r);
        if (MODE == 0) {
            const int half = r / (BN / 2);
            int n = nt * (BN / 2) + (r % (BN / 2));
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
            bptr[i] = base + row * a.H + c * 8;
        } else {
            int n = nt * BN + r;
            if (n >= a.H) n = a.H - 1;
            bptr[i] = shared_seg
                ? static_cast<const uint16_t*>(a.Bsh) + static_cast<int64_t>(n) * Is + jsh * a.I + c * 8
                : static_cast<const uint16_t*>(a.B) + static_cast<int64_t>(seg) * a.H * a.I +
                      static_cast<int64_t>(n) * a.I + c * 8;
        }
    }
    const int a_lds = wave * (BM / 4) * BK;          // element offsets inside a stage
    const int b_lds = BM * BK + wave * (BN / 4) * BK;

    const int nk = a.kdim / BK;

    auto stage_buf = [&](auto S) -> uint16_t* {
        static_assert(decltype(S)::value < STAGES, "stage index");
        if constexpr (decltype(S)::value == 0) return lds0;
        else if constexpr (decltype(S)::value == 1) return lds1;
        else if constexpr (decltype(S)::value == 2) return lds2;
        else return lds3;
    };
    // k-tile kt into stage S: NI copy instructions per wave
    auto issue = [&](auto S, int kt) {
        const int k0 = kt * BK;
        uint16_t* st = stage_buf(S);
        const uint32_t base = lds_addr(st);
#pragma unroll
        for (int i = 0; i < AI; ++i)
            lds_dma16(aptr[i] + k0, base + (a_lds + i * RPI * BK) * 2);
#pragma unroll
        for (int i = 0; i < BI; ++i)
            lds_dma16(bptr[i] + k0, base + (b_lds + i * RPI * BK) * 2);
    };

    // ---- fragments: weight rows are the MFMA's first operand, token rows the
    // second, so each lane ends up with 4 consecutive output columns ----------
    const int wm = wave >> 1, wn = wave & 1;
    int trow[TM], wrow[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) trow[i] = wm * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (MODE == 0) {
            constexpr int HT = TN / 2;
            wrow[j] = (j < HT ? 0 : BN / 2) + wn * (BN / 4) + (j % HT) * 32 + (lane & 31);
        } else {
            wrow[j] = wn * (BN / 2) + j * 32 + (lane & 31);
        }
    }
    const int khalf = lane >> 5;

    f32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.f;

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    issue(S0{}, 0);
    if constexpr (STAGES > 2) {
        if (1 < nk) issue(S1{}, 1);
    }
    if constexpr (STAGES > 3) {
        if (2 < nk) issue(S2{}, 2);
    }

    // one k-tile: wait for its stage, free the previous stage, refill it with
    // k-tile kt + 3, multiply
    auto step = [&](auto S, int kt) {
        constexpr int SI = decltype(S)::value;
        // copies of k-tile kt done; still in flight: the k-tiles issued after
        // it (at most STAGES - 2 of them)
        const int ahead = nk - 1 - kt;
        if constexpr (STAGES > 3) {
            if (ahead >= 2) wait_vmcnt<2 * NI>();
            else if (ahead == 1) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
        } else if constexpr (STAGES > 2) {
            if (ahead >= 1) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        block_barrier();
        if (kt + STAGES - 1 < nk)
            issue(std::integral_constant<int, (SI + STAGES - 1) % STAGES>{}, kt + STAGES - 1);
        const uint16_t* As = stage_buf(S);
        const uint16_t* Bs = As + BM * BK;
#pragma unroll LBV_KK_UNROLL
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + khalf;
            bf16x8 tf[TM], wf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                tf[i] = *reinterpret_cast<const bf16x8*>(As + trow[i] * BK + ((ch ^ swz<BK>(trow[i])) * 8));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                wf[j] = *reinterpret_cast<const bf16x8*>(Bs + wrow[j] * BK + ((ch ^ swz<BK>(wrow[j])) * 8));
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], tf[i], acc[j][i], 0, 0, 0);
        }
    };
    for (int kt = 0; kt < nk; kt += STAGES) {
        step(S0{}, kt);
        if (kt + 1 < nk) step(S1{}, kt + 1);
        if constexpr (STAGES > 2) {
            if (kt + 2 < nk) step(S2{}, kt + 2);
        }
        if constexpr (STAGES > 3) {
            if (kt + 3 < nk) step(S3{}, kt + 3);
        }
    }

    // ---- epilogue ---------------------------------------------------------------
    // Lane holds, for token tile i and weight tile j, output columns
    // 8q + 4*khalf + [0, 4) of token row (lane & 31).  Each wave first writes
    // its tile as bf16 into its own LDS region (row pitch = its column count,
    // 16-byte chunks XOR-swizzled by row), then reads it back 16 bytes per lane
    // so that every global store instruction writes whole contiguous rows.
    constexpr int WCOLS = MODE == 0 ? BN / 4 : BN / 2;   // output columns per wave
    constexpr int CHUNKS = WCOLS / 8;                    // 16-byte chunks per row
    block_barrier();                                     // all waves done with the stages
    uint16_t* ep;                                        // this wave's region (128 x WCOLS)
    if constexpr (STAGES == 4) {
        static_assert(128 * WCOLS <= STAGE, "one wave tile per stage buffer");
        ep = wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3;
    } else {
        static_assert(STAGES == 2 && 2 * 128 * WCOLS <= STAGE, "two wave tiles per stage buffer");
        ep = ((wave & 1) ? lds1 : lds0) + (wave >> 1) * 128 * WCOLS;
    }
    auto ep_off = [&](int row, int col) {                // element offset of (row, col) in the region
        return row * WCOLS + (((col >> 3) ^ (row % CHUNKS)) << 3) + (col & 7);
    };
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < (MODE == 0 ? TN / 2 : TN); ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = j * 32 + 8 * q + 4 * khalf;
                float v[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (MODE == 0) {
                        const float g = acc[j][i][4 * q + p];
                        const float u = acc[j + TN / 2][i][4 * q + p];
                        v[p] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                    } else {
                        v[p] = acc[j][i][4 * q + p];
                    }
                }
                uint2 o;
                o.x = pack_bf16x2(v[0], v[1]);
                o.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(ep + ep_off(row, col)) = o;
            }
        }
    }
    // read back: lane -> (row, chunk); a pass covers 64 / CHUNKS rows
    const int ncols = MODE == 0 ? a.I : a.H;
    const int col0 = MODE == 0 ? nt * (BN / 2) + wn * (BN / 4) : nt * BN + wn * (BN / 2);
    uint16_t* C = static_cast<uint16_t*>(a.C);
    constexpr int RPP = 64 / CHUNKS;                     // rows per pass
#pragma unroll 4
    for (int r0 = 0; r0 < 128; r0 += RPP) {
        const int row = r0 + lane / CHUNKS;
        const int ch = lane % CHUNKS;
        const int m = m0 + wm * (BM / 2) + row;
        const int col = col0 + ch * 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(ep + ep_off(row, ch * 8));
        if (m < seg_n && col < ncols)
            *reinterpret_cast<u32x4*>(C + static_cast<int64_t>(seg_r0 + m) * ncols + col) = v;
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

constexpr int G1_BM = LBV_G1_BM, G1_BN = LBV_G1_BN;
constexpr int G2_BM = LBV_G2_BM, G2_BN = LBV_G2_BN;

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
        hipLaunchKernelGGL((gemm_bf16_kernel<G1_BM, G1_BN, LBV_BK, LBV_STAGES, 0>),
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
        hipLaunchKernelGGL((gemm_bf16_kernel<G2_BM, G2_BN, LBV_BK, LBV_STAGES, 1>),
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

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
//   down:     y[slot(r)] = W2 act[r]   (stored back in slot order t*KS + k)
//   combine:  out[t] = sum_k w[t,k] y[t*KS+k] + sum_j y[t*KS+K+j]   (routed slots only)
//
// Segments s < E are routed experts, s >= E shared pseudo-experts (a width
// I slice of the shared MLP, exact by linearity of the down projection).
//
// bf16 path: a persistent workgroup per CU computes 256 x 256 tiles of one
// segment at a time with v_mfma_f32_32x32x16_bf16: 8 waves in 2 x 4, each
// with 128 x 64 fp32 accumulators, two waves per SIMD so that one can issue
// MFMAs while the other waits.  A and B tiles (K-contiguous, BK = 64 bf16 =
// 128 B per row, so every copy instruction moves whole 128-byte lines) go
// straight from global memory to LDS with global_load_lds_dwordx4 into two
// stages (three for the 64-row tiles used when segments hold few rows).
// Waves 0-3 (one per SIMD) issue the copies of the next k-tile one
// at a time between their MFMAs of the current one (a burst of copies stalls
// the issuing wave until the address unit takes them); the LDS reads of
// slice g + 1 sit between the MFMAs of slice g; one barrier per k-tile hands a
// stage over.  LDS rows are 16-byte chunks, chunk c of row r stored at
// c ^ ((r >> 1) & 7), which makes the fragment reads conflict-free.  Tiles
// never cross a segment; the tile table is built on the device from
// `offsets` (no host read-back of segment sizes).  For the gate/up matmul a B
// tile holds BN/2 gate rows and the matching BN/2 up rows, and each wave's
// accumulators for gate column n and up column n sit in the same lane and
// register, so silu(g) * u is formed in registers.
#include <type_traits>

#include "lbv_internal.h"
#include "lbv_pipe.h"

// Compile-time shape of the bf16 path: workgroup tile BM x BN (the gate/up
// GEMM's BN counts gate and up rows together, BN/2 act columns per tile);
// NPRE: MFMAs of a k-tile's last slice issued before its barrier;
// COPY_SLICES: slices of a k-tile that carry the next k-tile's copies;
// G*_EPI_NT: non-temporal output stores (act and y are written once and not
// reread while the matmul runs, so they need not displace operand lines);
// COMB_CHUNKS / COMB_NT: 16-byte chunks per lane per combine step, and
// non-temporal combine loads;
// G*_WAVES: waves per workgroup (4 or 8); G*_COPY_WAVES: waves that issue
// the stage copies; G*_ORDER: m-tiles per block of the tile order (1: m-tile
// major, the n-tiles of an m-tile adjacent; large: n-tile major inside each
// segment); G*_SMALL_ROWS (W8_G*_SMALL_ROWS with fp8 weights) / MID_ROWS /
// FEW_STAGES: below G*_SMALL_ROWS rows per segment on average the bf16-token
// matmuls use 64-row tiles, below MID_ROWS 128-row tiles, both with a
// FEW_STAGES-deep ring; A8_SMALL_ROWS / A8_MID_ROWS: the same for the
// fp8-token matmuls (two stages, A8_BM rows above).
#ifndef LBV_NPRE
#define LBV_NPRE 8
#endif
#ifndef LBV_COPY_SLICES
#define LBV_COPY_SLICES 2
#endif
#ifndef LBV_G1_COPY_WAVES
#define LBV_G1_COPY_WAVES 4
#endif
#ifndef LBV_G2_COPY_WAVES
#define LBV_G2_COPY_WAVES 4
#endif
#ifndef LBV_G1_WAVES
#define LBV_G1_WAVES 8
#endif
#ifndef LBV_G2_WAVES
#define LBV_G2_WAVES 8
#endif
#ifndef LBV_COMB_CHUNKS
#define LBV_COMB_CHUNKS 1
#endif
#ifndef LBV_COMB_NT
#define LBV_COMB_NT 1
#endif
#ifndef LBV_G1_EPI_NT
#define LBV_G1_EPI_NT 1
#endif
#ifndef LBV_G2_EPI_NT
#define LBV_G2_EPI_NT 1
#endif
#ifndef LBV_G1_ORDER
#define LBV_G1_ORDER 1
#endif
#ifndef LBV_G2_ORDER
#define LBV_G2_ORDER 1024
#endif
#ifndef LBV_G1_SMALL_ROWS
#define LBV_G1_SMALL_ROWS 20
#endif
#ifndef LBV_G2_SMALL_ROWS
#define LBV_G2_SMALL_ROWS 20
#endif
#ifndef LBV_W8_G1_SMALL_ROWS
#define LBV_W8_G1_SMALL_ROWS 80
#endif
#ifndef LBV_W8_G2_SMALL_ROWS
#define LBV_W8_G2_SMALL_ROWS 20
#endif
#ifndef LBV_MID_ROWS
#define LBV_MID_ROWS 480
#endif
#ifndef LBV_A8_SMALL_ROWS
#define LBV_A8_SMALL_ROWS 40
#endif
#ifndef LBV_A8_MID_ROWS
#define LBV_A8_MID_ROWS 80
#endif
#ifndef LBV_FEW_STAGES
#define LBV_FEW_STAGES 3
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
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// The 32-byte fp8 MFMA operand made of two 16-byte fragments (low, high).
__device__ __forceinline__ i32x8 op8(const bf16x8& lo8, const bf16x8& hi8) {
    const i32x4 l4 = __builtin_bit_cast(i32x4, lo8), h4 = __builtin_bit_cast(i32x4, hi8);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

struct GemmArgs {
    const void* A;          // gate/up: x [T, H];  down: act [rows, I]
    const void* B;          // gate/up: w13 [E, 2I, H];  down: w2 [E, H, I]
    const void* Bsh;        // gate/up: shared_w13 [2 Is, H];  down: shared_w2 [H, Is]
    const float* Bs;        // fp8 weights: row scales of B ([E, 2I] / [E, H])
    const float* Bshs;      // fp8 weights: row scales of Bsh ([2 Is] / [H])
    const float* bias;      // dense down-style matmul: [ncols] fp32 added before rounding, or null
    const float* xs;        // fp8 tokens, gate/up: x's power-of-two scale per token [T]
    uint8_t* asc;           // fp8 tokens: act's MX block scales [rows, kA8ScalePitch]
                            // (written by gate/up, read by down)
    const int32_t* offsets; // [S + 1]
    const int32_t* rows;    // sorted_rows: slot id of each sorted row
    void* C;                // gate/up: act [rows, I];  down: y [rows, H]
    int64_t T;
    int H, I, E, NS, KS, S;
    int kdim;               // reduction length: H (gate/up) or I (down)
    int ncols;              // output columns: I (gate/up) or H (down)
    int ntn;                // n-tiles per m-tile
    int* ctr;               // [8] tile queue counters, zero at launch (one per XCD)
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

// Segments the persistent kernel's LDS tile table holds (E + n_shared <= 264).
constexpr int kMaxSeg = 512;

// Persistent bf16 grouped matmul.  The grid is a multiple of 8 workgroups, one
// per CU; workgroup b serves XCD b % 8, which owns a contiguous eighth of the
// logical tiles (ordered segment by segment, inside a segment by ORDER),
// handed to its workgroups round-robin, so the tiles in flight on one XCD
// share operand rows in its L2.  Each workgroup builds the segment tile table
// once, then runs one continuous k-loop over all its tiles: the copies of the
// next tile's first STG-1 k-tiles are issued during the current tile's last
// k-tiles and land while its epilogue runs.
// DENSE (down-style only): one segment whose rows are stored in order (no
// slot ids) and an optional fp32 bias per output column: a plain linear layer
// y = x W^T + b.
template <int BM, int BN, int MODE, int NW, int CWV, int ORDER, int STG, bool W8, bool DENSE,
          bool A8 = false>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(GemmArgs a) {
    static_assert(!DENSE || MODE == 1, "dense rows: down-style only");
    // A8: fp8 tokens and fp8 weights on the scaled fp8 MFMA.  Weights: e4m3fn
    // codes with a power-of-two scale per row; gate/up tokens: x's codes with
    // a power-of-two scale per token; down tokens: act in MX blocks of 32
    // (e4m3fn codes, an e8m0 scale per block), which the gate/up epilogue
    // writes.  The row scales are applied in the epilogues, the act block
    // scales by the MFMA.  A k-tile holds 128 values per row, so its rows are
    // 128 bytes, as a bf16 k-tile of 64: the same stages and copies.
    static_assert(!A8 || (!W8 && !DENSE && (BM == 64 || BM == 128 || BM == 192 || BM == 256) && NW == 8 && CWV == 4 && STG == 2),
                  "fp8 tokens: 64- to 256-row tiles, 8 waves, 2 stages");
    // NW waves: 2 along the tokens x NW/2 along the weight rows (NW = 4: one
    // wave per SIMD with 128 x 128 accumulators; NW = 8: two per SIMD with
    // 128 x 64, so that one wave's MFMAs can cover the other's waits).
    constexpr int NTH = NW * 64;
    constexpr int WN = NW / 2;
    constexpr int BK = 64;                       // bf16 per row per k-tile: 128 bytes
    constexpr int TM = BM / 64;                  // token tiles (32 rows) per wave
    constexpr int TN = BN / WN / 32;             // weight-row tiles (32 rows) per wave
    static_assert(MODE == 1 || TN % 2 == 0, "gate/up tiles come in pairs");
    // B rows of a k-tile: BK bf16 (128 bytes) or, with fp8 weights (W8), BK
    // e4m3 codes (64 bytes); lengths below are in 16-bit LDS units
    constexpr int BKB = W8 ? BK / 2 : BK;
    constexpr int STAGE = BM * BK + BN * BKB;    // 16-bit units per stage
    constexpr int CPR = BK / 8;                  // 16-byte chunks per A row
    constexpr int RPI = 64 / CPR;                // A rows per 1 KB copy instruction
    constexpr int CPRB = BKB / 8;                // ... per B row
    constexpr int RPIB = 64 / CPRB;              // B rows per 1 KB copy instruction
    constexpr int EB = W8 || A8 ? 1 : 2;         // bytes per weight element in HBM
    // Waves 0 .. CW-1 issue the stage copies (with NW = 8 and CW = 4 one wave
    // per SIMD copies while the other only multiplies).
    constexpr int CW = CWV < NW ? CWV : NW;
    constexpr int AI = BM / CW / RPI, BI = BN / CW / RPIB;  // copies per copying wave per k-tile
    constexpr int NI = AI + BI;
    constexpr int KKS = BK / 16;                 // 16-deep k-slices per k-tile
    static_assert(BM % 64 == 0 && BM <= 256 && BN == 256, "slot ids: BM/64 waves x 64 rows");

    // STG stages (2, or 3 for short tiles) laid out [A0 | A1 (| A2) | B0 | B1
    // (| B2)] (A: token rows, B: weight rows), so that a fragment read is one
    // base register per slice plus an immediate offset for the stage and the
    // row group.  Stage STG-1 doubles as the epilogue's staging buffer.
    static_assert(STG == 2 || STG == 3, "2 or 3 stages");
    constexpr int ASZ = BM * BK, BSZ = BN * BKB;  // 16-bit units of one stage's A / B part
    // W8: the epilogue stages through a region of its own (EPW units per
    // wave) after the stages, since a stage's B part is half as large
    constexpr int EPW = 2048;
    __shared__ __attribute__((aligned(1024))) uint16_t lds[STG * STAGE + (W8 ? NW * EPW : 0)];
    __shared__ int s_pre[kMaxSeg + 1];           // m-tiles before segment s
    __shared__ int s_rid[BM];                    // slot ids of a tile's rows: gate/up: the next tile's; down: this tile's
    __shared__ int s_tmp[8];
    __shared__ int s_claim[2];
    // A8: the scales of a tile, two buffers (tile parity): its weight rows,
    // its token rows (gate/up: x's scale per token) and its act rows' block
    // scales (down: kA8ScalePitch bytes per row)
    __shared__ float s_sw[A8 ? 2 * BN : 1];
    __shared__ float s_sx[A8 && MODE == 0 ? 2 * BM : 1];
    __shared__ __attribute__((aligned(16))) uint8_t s_as[A8 && MODE == 1 ? 2 * BM * kA8ScalePitch : 16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int khalf = lane >> 5;
    const int Is = a.NS * a.I;

    // ---- segment tile table: s_pre[s] = sum over s' < s of ceil(n_s' / BM) ----
    {
        // threads 0..255 (waves 0..3) scan two values each
        int c[2] = {0, 0}, inc[2] = {0, 0};
        if (wave < 4) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int s = tid + p * 256;
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
        }
        __syncthreads();
        if (wave < 4) {
            int base0 = 0, base1 = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
            for (int w = 0; w < wave; ++w) {
                base0 += s_tmp[w];
                base1 += s_tmp[4 + w];
            }
            if (tid < a.S) s_pre[tid + 1] = base0 + inc[0];
            if (tid + 256 < a.S) s_pre[tid + 257] = base1 + inc[1];
        }
        if (tid == 0) s_pre[0] = 0;
        __syncthreads();
    }
    const int NT = __builtin_amdgcn_readfirstlane(s_pre[a.S]) * a.ntn;
    const int xcd = blockIdx.x % 8;
    constexpr int WOUT = MODE == 0 ? BN / 2 : BN;          // output columns of a tile
    const int ncols_all = MODE == 0 ? a.I : a.H;
    // ---- tile queues: XCD q owns the logical tiles NT q / 8 .. NT (q+1) / 8 - 1
    // (a contiguous range, so that the tiles in flight on one XCD share
    // operand rows in its L2) and hands them out in order through counter
    // a.ctr[q].  A workgroup takes tiles from its own XCD's queue, then,
    // once that is empty, from the other XCDs' queues in turn, so that the
    // XCDs finish together although tile costs differ (e.g. the shared
    // expert's contiguous rows run faster).  Which workgroup computes a tile
    // does not change its result.  Thread 0 claims; claims reach the other
    // threads through s_claim, one tile ahead: claim i + 2 is issued at the
    // start of tile i and resolved after its k-loop (so that the atomic's
    // round trip overlaps the MFMAs), into the slot tile i's claim came from.
    int qk = 0;                                            // queues found empty (thread 0)
    auto qrange = [&](int q, int& q0, int& q1) {
        q0 = static_cast<int>(static_cast<int64_t>(NT) * q / 8);
        q1 = static_cast<int>(static_cast<int64_t>(NT) * (q + 1) / 8);
    };
    auto claim = [&]() -> int {
        while (qk < 8) {
            const int q = (xcd + qk) & 7;
            int q0, q1;
            qrange(q, q0, q1);
            const int u = atomicAdd(&a.ctr[q], 1);
            if (u < q1 - q0) return q0 + u;
            ++qk;
        }
        return -1;
    };
    int pend_u = 0;                                        // thread 0: issued claim of queue
    auto claim_issue = [&]() {                             // (xcd + qk) & 7
        if (qk < 8) pend_u = atomicAdd(&a.ctr[(xcd + qk) & 7], 1);
    };
    auto claim_resolve = [&]() -> int {
        if (qk >= 8) return -1;
        int q0, q1;
        qrange((xcd + qk) & 7, q0, q1);
        if (pend_u < q1 - q0) return q0 + pend_u;
        ++qk;
        return claim();
    };
    if (tid == 0) {
        s_claim[0] = claim();
        s_claim[1] = claim();
    }
    __syncthreads();
    int t = __builtin_amdgcn_readfirstlane(s_claim[0]);
    if (t < 0) return;
    int it = 0;                                            // tiles done by this workgroup

    // ---- tile lookup: a forward walk over the segment table from the last
    // tile's segment (restarted from 0 if a tile index goes backwards) ----------
    int walk = 0;
    auto locate = [&](int tt, int& seg_, int& m0_, int& nt_, int& lo_, int& hi_) {
        // Inside a segment the m-tiles form blocks of ORDER (the last one
        // shorter); a block's tiles run n-tile major, so that the tiles that
        // share one weight slice are adjacent and those that share token rows
        // lie a block apart.  ORDER = 1 is m-tile major.
        if (__builtin_amdgcn_readfirstlane(s_pre[walk]) * a.ntn > tt) walk = 0;   // went backwards
        while (__builtin_amdgcn_readfirstlane(s_pre[walk + 1]) * a.ntn <= tt) ++walk;
        seg_ = walk;
        const int p0 = __builtin_amdgcn_readfirstlane(s_pre[walk]);
        const int nm = __builtin_amdgcn_readfirstlane(s_pre[walk + 1]) - p0;
        const int loc = tt - p0 * a.ntn;
        const int blk = loc / (ORDER * a.ntn);
        const int r = loc - blk * (ORDER * a.ntn);
        const int pb = nm - blk * ORDER < ORDER ? nm - blk * ORDER : ORDER;   // m-tiles in this block
        nt_ = r / pb;
        m0_ = (blk * ORDER + (r - nt_ * pb)) * BM;
        // output columns lo_ .. hi_ (the last n-tile may be partial)
        lo_ = nt_ * WOUT;
        hi_ = lo_ + WOUT - 1 < ncols_all - 1 ? lo_ + WOUT - 1 : ncols_all - 1;
    };

    // ---- copy sources: a wave-uniform base (scalar registers, advanced by BK
    // per k-tile) plus a 32-bit per-lane byte offset.  Instruction i of
    // copying wave w fills LDS rows w*(rows/CW) + RPI i + [0, RPI) of a stage's
    // A or B part; lane l lands at row +l/CPR, physical chunk l%CPR, which
    // holds logical chunk (l%CPR) ^ swz(row). ---------------------------------------
    const uint16_t* abase;
    const char* bbase;                            // weight rows, bytes
    uint32_t aoff[AI], boff[BI];
    // Slot ids of a tile's BM rows, copied into s_rid by waves 0 .. BM/64-1,
    // 64 rows each (a copy like the stage copies, counted by the same waits).  The
    // gate/up matmul gathers its x rows by them; the down matmul stores its
    // output rows to them.
    auto rid_copy = [&](int seg_r0_, int seg_n_, int m0_) {
        if (wave < BM / 64) {
            int m = m0_ + wave * 64 + lane;
            if (m >= seg_n_) m = seg_n_ - 1;
            lds_dma4_sb(a.rows, static_cast<uint32_t>(seg_r0_ + m) * 4, lds_addr(&s_rid[wave * 64]));
        }
    };
    // Points the copy sources at tile (seg_, m0_, nt_); gate/up reads the slot
    // ids from s_rid, which must have landed (and be visible: a barrier).
    auto set_sources = [&](int seg_, int seg_r0_, int seg_n_, int m0_, int nt_, int lo_, int hi_) {
        if (CW < NW && wave >= CW) return;       // not a copying wave
        // lane-derived terms are recomputed here rather than hoisted out of
        // the tile loop (where they would hold registers through the k-loop)
        const int lane = (threadIdx.x & 63) + opaque_zero();
        const bool shared_seg = seg_ >= a.E;
        const int jsh = seg_ - a.E;
        const char* B = static_cast<const char*>(a.B);
        const char* Bsh = static_cast<const char*>(a.Bsh);
        if (MODE == 0) {
            abase = static_cast<const uint16_t*>(a.A);
            bbase = shared_seg ? Bsh : B + static_cast<int64_t>(seg_) * 2 * a.I * a.H * EB;
        } else {
            abase = static_cast<const uint16_t*>(a.A) + static_cast<int64_t>(seg_r0_) * (A8 ? a.I / 2 : a.I);
            bbase = shared_seg ? Bsh + jsh * a.I * EB : B + static_cast<int64_t>(seg_) * a.H * a.I * EB;
        }
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            const int r = wave * (BM / CW) + i * RPI + lane / CPR;
            const uint32_t c = (lane % CPR) ^ swz<BK>(r);
            if (MODE == 0) {
                int tok = s_rid[r] / a.KS;
                tok = tok < 0 ? 0 : (tok >= a.T ? static_cast<int>(a.T) - 1 : tok);
                aoff[i] = A8 ? __umul24(tok, a.H) + c * 16 : (__umul24(tok, a.H) + c * 8) * 2;
            } else {
                int m = m0_ + r;
                if (m >= seg_n_) m = seg_n_ - 1;
                aoff[i] = A8 ? __umul24(m, a.I) + c * 16 : (__umul24(m, a.I) + c * 8) * 2;
            }
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int r = wave * (BN / CW) + i * RPIB + lane / CPRB;
            const uint32_t c = (lane % CPRB) ^ swz<BKB>(r);
            if (MODE == 0) {
                const int half = r / (BN / 2);
                int n = nt_ * (BN / 2) + (r % (BN / 2));
                // rows past the last column (a partial last n-tile) repeat
                // the last row: no extra HBM bytes
                n = n < lo_ ? lo_ : n;
                n = n > hi_ ? hi_ : n;
                if (n >= a.I) n = a.I - 1;
                const int row = shared_seg ? (half ? Is + jsh * a.I + n : jsh * a.I + n)
                                           : (half ? a.I + n : n);
                boff[i] = (__umul24(row, a.H) + c * (16 / EB)) * EB;
            } else {
                int n = nt_ * BN + r;
                n = n < lo_ ? lo_ : n;
                n = n > hi_ ? hi_ : n;
                if (n >= a.H) n = a.H - 1;
                boff[i] = (__umul24(n, shared_seg ? Is : a.I) + c * (16 / EB)) * EB;
            }
        }
    };

    // W8: the scale of the weight row of each of this lane's B fragments
    // (rows clamped as in the copies), loaded for a tile ahead of its k-loop
    constexpr int TNS = W8 ? TN : 1;
    float sc[TNS], nsc[TNS];
    auto load_scales = [&](int seg_, int nt_, int lo_, int hi_, float* dst) {
        if constexpr (W8) {
            const int ln = (threadIdx.x & 63) + opaque_zero();
            const int rl = ln & 31;
            const bool shared_seg = seg_ >= a.E;
            const int jsh = seg_ - a.E;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                int idx;
                if (MODE == 0) {
                    constexpr int HT = TN / 2;
                    const int half = j >= HT;
                    int n = nt_ * (BN / 2) + wn * (BN / 2 / WN) + rl + (half ? j - HT : j) * 32;
                    n = n < lo_ ? lo_ : n;
                    n = n > hi_ ? hi_ : n;
                    if (n >= a.I) n = a.I - 1;
                    idx = shared_seg ? (half ? Is + jsh * a.I + n : jsh * a.I + n)
                                     : seg_ * 2 * a.I + (half ? a.I + n : n);
                } else {
                    int n = nt_ * BN + wn * (BN / WN) + rl + j * 32;
                    n = n < lo_ ? lo_ : n;
                    n = n > hi_ ? hi_ : n;
                    if (n >= a.H) n = a.H - 1;
                    idx = shared_seg ? n : seg_ * a.H + n;
                }
                dst[j] = (shared_seg ? a.Bshs : a.Bs)[idx];
            }
        }
    };

    // A8: the scales tile (seg_, m0_, nt_) needs, copied into buffer buf by
    // the copying waves and counted by the same waits as the stage copies:
    // one 4-byte copy per weight row and per token row (gate/up: the token
    // ids come from s_rid, which must have landed), the act rows' block
    // scales (down) as 1 KB pieces of one contiguous run.  Rows past the
    // tile's segment take clamped rows (their outputs are not stored).
    auto scale_copy = [&](int buf, int seg_, int seg_r0_, int m0_, int nt_, int lo_, int hi_) {
        if constexpr (A8) {
            if (wave >= CW) return;
            const int ln = (threadIdx.x & 63) + opaque_zero();
            const bool shared_seg = seg_ >= a.E;
            const int jsh = seg_ - a.E;
            const int r = wave * 64 + ln;                     // row r of the tile's B (and A) rows
            int idx;
            if (MODE == 0) {
                const int half = r / (BN / 2);
                int n = nt_ * (BN / 2) + (r % (BN / 2));
                n = n < lo_ ? lo_ : (n > hi_ ? hi_ : n);
                if (n >= a.I) n = a.I - 1;
                idx = shared_seg ? (half ? Is + jsh * a.I + n : jsh * a.I + n)
                                 : seg_ * 2 * a.I + (half ? a.I + n : n);
            } else {
                int n = nt_ * BN + r;
                n = n < lo_ ? lo_ : (n > hi_ ? hi_ : n);
                if (n >= a.H) n = a.H - 1;
                idx = shared_seg ? n : seg_ * a.H + n;
            }
            lds_dma4_sb(shared_seg ? a.Bshs : a.Bs, static_cast<uint32_t>(idx) * 4,
                        lds_addr(&s_sw[buf * BN + wave * 64]));
            if constexpr (MODE == 0) {
                if (wave < BM / 64) {
                    int tok = s_rid[r] / a.KS;
                    tok = tok < 0 ? 0 : (tok >= a.T ? static_cast<int>(a.T) - 1 : tok);
                    lds_dma4_sb(a.xs, static_cast<uint32_t>(tok) * 4, lds_addr(&s_sx[buf * BM + wave * 64]));
                }
            } else {
                constexpr int NP = BM * kA8ScalePitch / 1024;   // 1 KB pieces
                const int64_t last = a.T * a.KS * kA8ScalePitch - 16;
#pragma unroll
                for (int d = 0; d < NP; ++d) {
                    if (d % CW != wave) continue;
                    int64_t off = (static_cast<int64_t>(seg_r0_) + m0_) * kA8ScalePitch + d * 1024 + ln * 16;
                    off = off < last ? off : last;
                    lds_dma16_sb<0>(a.asc, static_cast<uint32_t>(off),
                                    lds_addr(s_as + buf * BM * kA8ScalePitch + d * 1024));
                }
            }
        }
    };

    const int a_lds = wave * (BM / CW) * BK;     // this wave's rows inside an A / B part
    const int b_lds = wave * (BN / CW) * BKB;
    const int nk = a.kdim / (A8 ? 2 * BK : BK);  // k-tiles (A8: 128 one-byte values per row)
    // the k-loop of a tile runs over nkp = nk rounded up to a multiple of STG,
    // so that every step of an iteration is unconditional (no MFMA under a
    // branch); the k-tiles past nk are zero-filled stages, whose products add
    // exact zeros
    const int nkp = (nk + STG - 1) / STG * STG;

    auto a_part = [&](auto S) -> uint16_t* { return lds + decltype(S)::value * ASZ; };
    auto b_part = [&](auto S) -> uint16_t* { return lds + STG * ASZ + decltype(S)::value * BSZ; };
    auto zero_fill = [&](auto S) {
        u32x4* pa = reinterpret_cast<u32x4*>(a_part(S));
        u32x4* pb = reinterpret_cast<u32x4*>(b_part(S));
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < ASZ / 8 / NTH; ++q) pa[tid + NTH * q] = z;
#pragma unroll
        for (int q = 0; q < BSZ / 8 / NTH; ++q) pb[tid + NTH * q] = z;
    };
    // copy instruction D (A rows first, then B rows) of k-tile kt into stage S
    auto copy_const = [&](auto S, int kt, auto D) {
        constexpr int d = decltype(D)::value;
        if (CW < NW && wave >= CW) return;
        if constexpr (d < AI)
            lds_dma16_sb<d * RPI * BK * 2>(abase + kt * BK, aoff[d], lds_addr(a_part(S) + a_lds));
        else
            lds_dma16_sb<(d - AI) * RPIB * BKB * 2>(bbase + kt * BKB * 2, boff[d - AI],
                                                    lds_addr(b_part(S) + b_lds));
    };
    // the same for an index d that is a constant once the loops are unrolled
    auto copy_one = [&](auto S, int kt, int d) {
        static_for<NI>([&](auto D) {
            if (d == decltype(D)::value) copy_const(S, kt, D);
        });
    };

    // ---- fragments: weight rows are the MFMA's first operand, token rows the
    // second, so each lane ends up with 4 consecutive output columns ----------
    // A fragment i of slice kk in stage s: fa[kk] + s*ASZ + i*32*BK; B fragment
    // j: fb[kk] + s*BSZ + brow(j)*BKB.  Formed once per tile from a lane index
    // the compiler cannot see through, so that they are not held in registers
    // across the epilogue.
    // With fp8 weights a lane's 16-byte read of a B row holds its k values of
    // two slices: lanes 0-31 take k 0-31 of the k-tile, lanes 32-63 k 32-63,
    // slice kk using the lane's k values 8 kk .. 8 kk + 7 of its half; the A
    // fragments follow the same k order (chunk 4 khalf + kk).  fb[p], p = 0, 1:
    // the B chunk of slices 2p and 2p + 1.
    const uint16_t* fa[KKS];
    const uint16_t* fb[KKS];
    auto frag_offsets = [&]() {
        const int ln = (threadIdx.x & 63) + opaque_zero();
        const int kh = ln >> 5, rl = ln & 31;
        const int ra = wm * (BM / 2) + rl;                       // first A row (i = 0)
        const int rb = (MODE == 0 ? wn * (BN / 2 / WN) : wn * (BN / WN)) + rl;   // first B row (j = 0)
#pragma unroll
        for (int kk = 0; kk < KKS; ++kk) {
            const int ch = W8 ? kh * 4 + kk : kk * 2 + kh;     // swz(r) depends on r mod 32 only
            fa[kk] = lds + ra * BK + ((ch ^ swz<BK>(rl)) * 8);
            const int chb = W8 ? kh * 2 + (kk >> 1) : ch;
            fb[kk] = lds + STG * ASZ + rb * BKB + ((chb ^ swz<BKB>(rl)) * 8);
        }
    };
    // B row of fragment j relative to j = 0
    auto brow = [](int j) {
        constexpr int HT = TN / 2;
        return MODE == 0 ? (j < HT ? j * 32 : BN / 2 + (j - HT) * 32) : j * 32;
    };
    frag_offsets();

    f32x16 acc[TN][TM];
    // Two fragment sets: slice g is multiplied from set g % 2 while slice g + 1
    // is read into the other one.  W8: the raw B chunks (two slices each) and
    // the current slice's converted B fragments instead of wf0 / wf1.
    bf16x8 tf0[TM], wf0[TN], tf1[TM], wf1[TN];
    constexpr int TNR = W8 ? TN : 1;
    u32x4 raw[TNR];
    bf16x8 wcv[TNR];
    // W8: B fragments of slice ckk, decode(q) * 2^e of each lane's weight row
    // (exact in bf16), from the low (even ckk) or high half of the raw chunk
    auto conv = [&](int ckk) {
        if constexpr (W8) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t w0 = raw[j][(ckk & 1) * 2], w1 = raw[j][(ckk & 1) * 2 + 1];
                // each conversion yields the bf16 pair of bytes (0, 1) or (2, 3)
                // of its word as one 32-bit register; the pairs are moved as
                // whole words (no per-element extraction)
                const u32x4 v = {
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc[j], false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc[j], true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc[j], false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc[j], true))};
                wcv[j] = __builtin_bit_cast(bf16x8, v);
            }
        }
    };
    // B fragment read into set WS (bf16) or the raw chunk of an even slice (W8)
    auto read_b = [&](bf16x8* WS, int j, int stage, int nkk) {
        if constexpr (W8) {
            if ((nkk & 1) == 0)
                raw[j] = *reinterpret_cast<const u32x4*>(fb[nkk] + stage * BSZ + brow(j) * BKB);
        } else {
            WS[j] = *reinterpret_cast<const bf16x8*>(fb[nkk] + stage * BSZ + brow(j) * BKB);
        }
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    // ---- first tile: sources, k-tile 0 into stage 0, first slice read ----------
    int seg, m0, nt, lo, hi;
    locate(t, seg, m0, nt, lo, hi);
    int seg_r0 = a.offsets[seg];
    int seg_n = a.offsets[seg + 1] - seg_r0;
    if (MODE == 0) {
        rid_copy(seg_r0, seg_n, m0);
        wait_vmcnt<0>();
        block_barrier();
    }
    set_sources(seg, seg_r0, seg_n, m0, nt, lo, hi);
    load_scales(seg, nt, lo, hi, sc);
    scale_copy(0, seg, seg_r0, m0, nt, lo, hi);
    // k-tiles 0 .. STG-2 into stages 0 .. STG-2 (zero-filled past nk)
    auto pro_fill = [&](auto S, int kt) {
        if (kt < nk) {
#pragma unroll
            for (int d = 0; d < NI; ++d) copy_one(S, kt, d);
        } else {
            zero_fill(S);
        }
    };
    pro_fill(S0{}, 0);
    if constexpr (STG == 3) pro_fill(S1{}, 1);
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    block_barrier();
#pragma unroll
    for (int i = 0; i < TM; ++i) tf0[i] = *reinterpret_cast<const bf16x8*>(fa[0] + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < TN; ++j) read_b(wf0, j, 0, 0);
    // A8: slice 1 as well (a step multiplies two slices), and the act block
    // scales of k-tile 0
    uint32_t asc[TM], asn[TM];
    // The act row's block scales of k-tile kt, for step 0 (low byte) and
    // step 1 (next byte): blocks 4kt + khalf and 4kt + 2 + khalf, stored at
    // bytes 4kt + 2 khalf and 4kt + 2 khalf + 1 (the gate/up epilogue writes
    // each k-tile's four blocks in the order 0, 2, 1, 3).
    const uint8_t* const as_lane = s_as + (wm * (BM / 2) + (lane & 31)) * kA8ScalePitch + 2 * khalf;
    auto read_asc = [&](uint32_t* dst, int buf, int kt) {
        if constexpr (A8 && MODE == 1) {
            kt = kt < nk ? kt : nk - 1;
            const uint8_t* p = as_lane + buf * BM * kA8ScalePitch + 4 * kt;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                dst[i] = *reinterpret_cast<const uint16_t*>(p + i * 32 * kA8ScalePitch);
        }
    };
    // A8 fragments: 32-byte operands (slices 2s and 2s + 1 of a k-tile), two
    // sets: step 0 of a k-tile multiplies set P while set Q is read, step 1
    // multiplies Q while P is read (as the bf16 slices alternate), so the same
    // registers hold the same set at every step and across the loop.
    i32x8 tqP[TM], wqP[TN], tqQ[TM], wqQ[TN];
    auto rd8 = [](const uint16_t* p0, const uint16_t* p1) -> i32x8 {
        return op8(*reinterpret_cast<const bf16x8*>(p0), *reinterpret_cast<const bf16x8*>(p1));
    };
    // fragment read r (token fragments first) of step s2 / 2 of the k-tile
    // in `stage` into the set (T8, W8_)
    auto rd_frag = [&](i32x8* T8, i32x8* W8_, int r, int stage, int s2) {
        if (r < TM)
            T8[r] = rd8(fa[s2] + stage * ASZ + r * 32 * BK, fa[s2 + 1] + stage * ASZ + r * 32 * BK);
        else
            W8_[r - TM] = rd8(fb[s2] + stage * BSZ + brow(r - TM) * BKB,
                              fb[s2 + 1] + stage * BSZ + brow(r - TM) * BKB);
    };
    if constexpr (A8) {
#pragma unroll
        for (int r = 0; r < TM + TN; ++r) rd_frag(tqP, wqP, r, 0, 0);
        read_asc(asc, 0, 0);
    }

    constexpr int NQ = TM * TN;                  // MFMAs per slice
    constexpr int NR = TM + TN;                  // fragment reads per slice
    // MFMAs of the last slice before the barrier (0 when a slice has fewer
    // MFMAs than fragment reads)
    constexpr int NPRE = NQ - NR <= 0 ? 0 : (LBV_NPRE < NQ - NR ? LBV_NPRE : NQ - NR);
    constexpr int DSL = LBV_COPY_SLICES < KKS - 1 ? LBV_COPY_SLICES : KKS - 1;   // slices carrying copies

    // One slice: MFMAs [Q0, Q1) from set (CT, CW) (ZC: the tile's first slice,
    // accumulators start at zero); after MFMA Q0 + r, fragment read r of the
    // next slice (stage index NB, slice NKK) into set (NT, NW); copy instructions
    // [D0, D1) of k-tile KF into stage TS spread evenly over the MFMAs (when
    // DO_COPY).  The order is pinned: one MFMA, then its read and copy, then
    // a scheduling fence.
#define LBV_SLICE(CT, CW, NT_, NW_, NB, NKK, Q0, Q1, TS, KF, DO_COPY, D0, D1, ZC)              \
    _Pragma("unroll") for (int q = (Q0); q < (Q1); ++q) {                                     \
        if (ZC)                                                                                \
            acc[q / TM][q % TM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                    \
                W8 ? wcv[(q / TM) % TNR] : CW[q / TM], CT[q % TM], f32x16{}, 0, 0, 0);         \
        else                                                                                   \
            acc[q / TM][q % TM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                    \
                W8 ? wcv[(q / TM) % TNR] : CW[q / TM], CT[q % TM], acc[q / TM][q % TM], 0, 0, 0); \
        const int r_ = q - (Q0);                                                               \
        /* read rr goes after MFMA rr, the ones left over after the last MFMA */               \
        _Pragma("unroll") for (int rr = 0; rr < NR; ++rr) {                                   \
            if ((rr < (Q1) - (Q0) ? rr : (Q1) - (Q0) - 1) == r_) {                             \
                if (rr < TM)                                                                   \
                    NT_[rr] = *reinterpret_cast<const bf16x8*>(fa[NKK] + (NB) * ASZ + rr * 32 * BK); \
                else                                                                           \
                    read_b(NW_, rr - TM, NB, NKK);                                             \
            }                                                                                  \
        }                                                                                      \
        if ((D1) > (D0)) {                                                                     \
            _Pragma("unroll") for (int d = (D0); d < (D1); ++d) {                              \
                if ((d - (D0)) * ((Q1) - (Q0)) / ((D1) > (D0) ? (D1) - (D0) : 1) == r_ && (DO_COPY)) \
                    copy_one(TS, KF, d);                                                       \
            }                                                                                  \
        }                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                     \
    }

    // Next tile (valid when has_next): its lookup is done at the start of the
    // current tile, its slot ids are copied at step 0, its copy sources are set
    // right after the barrier of the second-to-last step.
    bool has_next = false;
    int nseg = 0, nm0 = 0, nnt = 0, nseg_r0 = 0, nseg_n = 0, nlo = 0, nhi = 0;

    // One k-tile kt held in stage S = kt % STG.  On entry slice 0 of it is in
    // set 0, and k-tiles kt+1 .. kt+STG-2 are in flight.  Slices 0 .. DSL-1
    // also carry the copies of k-tile kt + STG - 1 (past the tile's last
    // k-tile: of the next tile's first ones) into the stage that k-tile
    // kt - 1 freed.  The last slice brackets the hand-over: NPRE MFMAs, wait
    // for k-tile kt + 1's copies, barrier (every wave is done reading stage
    // S), then the remaining MFMAs with the reads of slice 0 of k-tile kt + 1
    // (unused after the tile's last k-tile).
    auto step = [&](auto S, int kt, auto First) {
        constexpr int SI = decltype(S)::value;
        constexpr bool FIRST = decltype(First)::value;
        const auto TS = std::integral_constant<int, (SI + STG - 1) % STG>{};
        constexpr int cur = SI, nxt = (SI + 1) % STG;   // stages read by this k-tile / the next
        const int kf = kt + STG - 1;             // k-tile copied during this step
        const bool nextc = kf >= nkp;            // ... a k-tile of the next tile
        const int kc = nextc ? kf - nkp : kf;    // its index within its tile
        const bool want = !nextc || has_next;    // that k-tile exists
        const bool do_copy = want && kc < nk;    // past nk it is a zero-filled stage
        if (want && kc >= nk) zero_fill(TS);
        if (MODE == 0 && kt == 0 && has_next) rid_copy(nseg_r0, nseg_n, nm0);
        if (MODE == 1 && !DENSE && kt == 0) rid_copy(seg_r0, seg_n, m0);
#pragma unroll
        for (int kk = 0; kk < KKS - 1; ++kk) {
            conv(kk);
            if (kk % 2 == 0) {
                LBV_SLICE(tf0, wf0, tf1, wf1, cur, kk + 1, 0, NQ, TS, kc, do_copy && kk < DSL,
                          kk < DSL ? kk * NI / DSL : 0, kk < DSL ? (kk + 1) * NI / DSL : 0,
                          FIRST && kk == 0)
            } else {
                LBV_SLICE(tf1, wf1, tf0, wf0, cur, kk + 1, 0, NQ, TS, kc, do_copy && kk < DSL,
                          kk < DSL ? kk * NI / DSL : 0, kk < DSL ? (kk + 1) * NI / DSL : 0,
                          false)
            }
        }
        // last slice (set 1)
        conv(KKS - 1);
#pragma unroll
        for (int q = 0; q < NPRE; ++q)
            acc[q / TM][q % TM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                W8 ? wcv[(q / TM) % TNR] : wf1[q / TM], tf1[q % TM], acc[q / TM][q % TM], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nkp) {
            // k-tile kt + 1 (and any slot-id copy) landed; with three stages
            // the copies issued in this step may stay in flight
            if (STG == 3 && do_copy) wait_vmcnt<NI>();
            else wait_vmcnt<0>();
        }
        wait_lgkmcnt0();
        block_barrier();
        if (kt == nkp - STG && has_next) {
            set_sources(nseg, nseg_r0, nseg_n, nm0, nnt, nlo, nhi);
            load_scales(nseg, nnt, nlo, nhi, nsc);
            wait_lgkmcnt0();
        }
        __builtin_amdgcn_sched_barrier(0);
        LBV_SLICE(tf1, wf1, tf0, wf0, nxt, 0, NPRE, NQ, TS, kc, false, 0, 0, false)
    };
#undef LBV_SLICE

    // A8: one k-tile (128 values per row) in stage S = kt % 2, two MFMA steps.
    // Step s multiplies 32-byte fragments made of slices 2s and 2s + 1: a
    // lane's chunks 4s + khalf and 4s + 2 + khalf, i.e. values k = 64s + 16
    // khalf + [0, 16) and 64s + 32 + 16 khalf + [0, 16), the instruction's own
    // order.  After MFMA r of a step comes fragment read r of the other set
    // (reads left over after the last MFMA).  Step 0 (set P) reads set Q from
    // slices 2, 3 and carries the copies of k-tile kt + 1; step 1 (set Q)
    // issues NPRE8 MFMAs, waits for k-tile kt + 1 and passes the barrier, then
    // issues the rest with the reads of k-tile kt + 1's slices 0, 1 into P.
    // The down matmul's act block scales: in step s, lane l provides the
    // scale of block 4kt + 2s + khalf of token row l % 32 in byte 0 of its
    // scale operand; read_asc brings both steps' bytes in one 16-bit word.
    constexpr int NR8 = TM + TN;                 // tuple reads per step
    constexpr int NPRE8 = NQ > NR8 ? NQ - NR8 : 0;
#define LBV_MFMA8(Q, SIDX, TS8, WS8)                                                          \
    {                                                                                          \
        const int sbv_ = MODE == 1 ? static_cast<int>(asc[(Q) % TM] >> (8 * (SIDX))) : 127;  \
        acc[(Q) / TM][(Q) % TM] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(              \
            WS8[(Q) / TM], TS8[(Q) % TM], acc[(Q) / TM][(Q) % TM], 0, 0, 0, 127, 0, sbv_);     \
    }
    // stage given at run time (one k-tile per loop iteration): its parts and
    // the copies and zero fill of stage s_
    auto copy8 = [&](int s_, int kt_, auto D) {
        constexpr int d = decltype(D)::value;
        if (wave >= CW) return;
        if constexpr (d < AI)
            lds_dma16_sb<d * RPI * BK * 2>(abase + kt_ * BK, aoff[d], lds_addr(lds + s_ * ASZ + a_lds));
        else
            lds_dma16_sb<(d - AI) * RPIB * BKB * 2>(bbase + kt_ * BKB * 2, boff[d - AI],
                                                    lds_addr(lds + STG * ASZ + s_ * BSZ + b_lds));
    };
    auto zero_fill8 = [&](int s_) {
        u32x4* pa = reinterpret_cast<u32x4*>(lds + s_ * ASZ);
        u32x4* pb = reinterpret_cast<u32x4*>(lds + STG * ASZ + s_ * BSZ);
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < ASZ / 8 / NTH; ++q) pa[tid + NTH * q] = z;
#pragma unroll
        for (int q = 0; q < BSZ / 8 / NTH; ++q) pb[tid + NTH * q] = z;
    };
    auto step8 = [&](int kt) {
        const int cur = kt & 1, nxt = cur ^ 1;   // STG == 2
        const int kf = kt + 1;                   // k-tile copied during this k-tile
        const bool nextc = kf >= nkp;            // ... a k-tile of the next tile
        const int kc = nextc ? kf - nkp : kf;
        const bool want = !nextc || has_next;
        const bool do_copy = want && kc < nk;
        if (want && kc >= nk) zero_fill8(nxt);
        if (MODE == 0 && kt == 0 && has_next) rid_copy(nseg_r0, nseg_n, nm0);
        if (MODE == 1 && kt == 0) rid_copy(seg_r0, seg_n, m0);
        // step 0: set P, reads of slices 2, 3 into Q, the copies
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            LBV_MFMA8(q, 0, tqP, wqP)
#pragma unroll
            for (int r = 0; r < NR8; ++r)
                if ((r < NQ ? r : NQ - 1) == q) rd_frag(tqQ, wqQ, r, cur, 2);
            static_for<NI>([&](auto D) {
                if (decltype(D)::value * NQ / NI == q && do_copy) copy8(nxt, kc, D);
            });
            __builtin_amdgcn_sched_barrier(0);
        }
        // step 1: set Q; the hand-over after NPRE8 MFMAs
#pragma unroll
        for (int q = 0; q < NPRE8; ++q) {
            LBV_MFMA8(q, 1, tqQ, wqQ)
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kt + 1 < nkp) wait_vmcnt<0>();       // k-tile kt + 1 (and any slot-id copy) landed
        wait_lgkmcnt0();
        block_barrier();
        if (kt == nkp - STG && has_next) {
            set_sources(nseg, nseg_r0, nseg_n, nm0, nnt, nlo, nhi);
            scale_copy((it + 1) & 1, nseg, nseg_r0, nm0, nnt, nlo, nhi);
        }
        read_asc(asn, it & 1, kt + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = NPRE8; q < NQ; ++q) {
            LBV_MFMA8(q, 1, tqQ, wqQ)
#pragma unroll
            for (int r = 0; r < NR8; ++r)
                if ((r < NQ - NPRE8 ? r : NQ - NPRE8 - 1) == q - NPRE8) rd_frag(tqP, wqP, r, nxt, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) asc[i] = asn[i];
    };
#undef LBV_MFMA8

    constexpr int WCOLS = MODE == 0 ? BN / 2 / WN : BN / WN;   // output columns per wave
    constexpr int CHUNKS = WCOLS / 8;                    // 16-byte chunks per row
    // staging regions in stage STG-1 (the last one a tile reads): its A and B
    // parts split evenly when they are the same size, else all in its B part;
    // W8: the region after the stages
    constexpr bool SPLIT = !W8 && ASZ == BSZ;
    constexpr int RSZ = W8 ? EPW : SPLIT ? 2 * ASZ / NW : BSZ / NW;   // staging elements per wave
    constexpr int PT0 = RSZ / WCOLS / 32;
    // token tiles per staging pass: the largest divisor of TM that fits
    constexpr int PT = (PT0 >= TM) ? TM : (TM % PT0 == 0 ? PT0 : (PT0 >= 2 && TM % 2 == 0 ? 2 : 1));
    constexpr int PROWS = PT * 32;                       // rows per staging pass
    static_assert(PT >= 1 && TM % PT == 0, "whole token tiles per pass");
    constexpr int SL = STG - 1;
    uint16_t* const ep0 = W8    ? lds + STG * STAGE + wave * RSZ
                          : SPLIT ? (wave < NW / 2 ? lds + SL * ASZ : lds + STG * ASZ + SL * BSZ) + (wave % (NW / 2)) * RSZ
                                  : lds + STG * ASZ + SL * BSZ + wave * RSZ;   // this wave's staging region
    auto ep_off = [&](int row, int col) {                // element offset of (row, col) in the region
        return row * WCOLS + (((col >> 3) ^ (row % CHUNKS)) << 3) + (col & 7);
    };
    uint16_t* C = static_cast<uint16_t*>(a.C);
    const int ncols = MODE == 0 ? a.I : a.H;

    for (;;) {
        const int tn = __builtin_amdgcn_readfirstlane(s_claim[(it + 1) & 1]);
        has_next = tn >= 0;
        if (tid == 0 && has_next) claim_issue();
        if (has_next) {
            locate(tn, nseg, nm0, nnt, nlo, nhi);
            nseg_r0 = a.offsets[nseg];
            nseg_n = a.offsets[nseg + 1] - nseg_r0;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[j][i] = f32x16{};
        if constexpr (A8) {
#pragma nounroll
            for (int kt = 0; kt < nkp; ++kt) step8(kt);
        } else {
            for (int kt = 0; kt < nkp; kt += STG) {
                step(S0{}, kt, std::false_type{});
                step(S1{}, kt + 1, std::false_type{});
                if constexpr (STG == 3) step(S2{}, kt + 2, std::false_type{});
            }
        }

        // the claim issued at this tile's start (read at the start of the next
        // tile, after the barrier that follows the epilogue)
        if (tid == 0 && has_next) s_claim[it & 1] = claim_resolve();
        // ---- epilogue: lane holds, for token tile i and weight tile j, output
        // columns 8q + 4*khalf + [0, 4) of token row (lane & 31).  Each wave
        // writes PROWS rows of its tile as bf16 into its staging region (row
        // pitch = its column count, 16-byte chunks XOR-swizzled by row), then
        // reads them back 16 bytes per lane, so that every global store
        // instruction writes whole contiguous rows.  Every wave passed the last
        // barrier after its final reads of stage STG-1.
        const int col0 = MODE == 0 ? nt * (BN / 2) + wn * (BN / 2 / WN) : nt * BN + wn * (BN / WN);
        // staging addresses are formed here, not hoisted out of the tile loop
        // (where they would hold registers through the whole k-loop)
        uint16_t* const ep = ep0;
        const int elane = (threadIdx.x & 63) + opaque_zero();
        const int ekh = elane >> 5;
#pragma unroll
        for (int p = 0; p < TM / PT; ++p) {
#pragma unroll
            for (int ii = 0; ii < PT; ++ii) {
                const int i = p * PT + ii;
                const int row = ii * 32 + (elane & 31);
#pragma unroll
                for (int j = 0; j < (MODE == 0 ? TN / 2 : TN); ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = j * 32 + 8 * q + 4 * ekh;
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (MODE == 0) {
                                float g = acc[j][i][4 * q + e];
                                float u = acc[j + TN / 2][i][4 * q + e];
                                if constexpr (A8) {
                                    // weight row scales (gate row, up row) and the token's scale
                                    const int wr = (it & 1) * BN + wn * (BN / 2 / WN) + col + e;
                                    const float sx = s_sx[(it & 1) * BM + wm * (BM / 2) + i * 32 + (elane & 31)];
                                    g *= s_sw[wr] * sx;
                                    u *= s_sw[wr + BN / 2] * sx;
                                }
                                v[e] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                            } else {
                                v[e] = acc[j][i][4 * q + e];
                                if constexpr (A8) v[e] *= s_sw[(it & 1) * BN + wn * (BN / WN) + col + e];
                                if (DENSE && a.bias) {
                                    const int bc = col0 + col + e;
                                    v[e] += a.bias[bc < ncols_all ? bc : ncols_all - 1];
                                }
                            }
                        }
                        uint2 o;
                        o.x = pack_bf16x2(v[0], v[1]);
                        o.y = pack_bf16x2(v[2], v[3]);
                        *reinterpret_cast<uint2*>(ep + ep_off(row, col)) = o;
                    }
                    __builtin_amdgcn_sched_barrier(0);   // bounds the accumulators read out at once
                }
            }
            if (p == 0) wait_vmcnt<0>();             // the next tile's first k-tiles landed
            // read back: lane -> (row, chunk); an instruction covers 64 / CHUNKS rows
            constexpr int RPP = 64 / CHUNKS;
#pragma unroll
            for (int r0 = 0; r0 < PROWS; r0 += RPP) {
                const int row = r0 + elane / CHUNKS;
                const int ch = elane % CHUNKS;
                const int m = m0 + wm * (BM / 2) + p * PROWS + row;
                const int col = col0 + ch * 8;
                const u32x4 v = *reinterpret_cast<const u32x4*>(ep + ep_off(row, ch * 8));
                // gate/up: act rows in segment order; down: y rows in slot order
                const int64_t orow = MODE == 0 || DENSE ? seg_r0 + m : s_rid[wm * (BM / 2) + p * PROWS + row];
                if constexpr (A8 && MODE == 0) {
                    // act in MX blocks: 4 consecutive lanes hold 32 columns of
                    // a row (4 chunks of 8), one block; its scale 2^e, e the
                    // smallest integer with max|act| <= 448 2^e (0 for an
                    // all-zero block, held to [-127, 127]); codes are the
                    // nearest e4m3fn values of act 2^-e (ties to even)
                    static_assert(CHUNKS % 4 == 0, "whole MX blocks per row and wave");
                    float f[8];
#pragma unroll
                    for (int wi = 0; wi < 4; ++wi) {
                        f[2 * wi] = __uint_as_float(v[wi] << 16);
                        f[2 * wi + 1] = __uint_as_float(v[wi] & 0xffff0000u);
                    }
                    float amax = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(f[k]));
                    amax = fmaxf(amax, __shfl_xor(amax, 1));
                    amax = fmaxf(amax, __shfl_xor(amax, 2));
                    int ex = 0;
                    if (amax > 0.0f) {
                        int x;
                        const float fr = frexpf(amax, &x);       // amax = fr 2^x, 448 = 0.875 2^9
                        ex = fr <= 0.875f ? x - 9 : x - 8;
                        ex = ex < -127 ? -127 : (ex > 127 ? 127 : ex);
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k) f[k] = fminf(fmaxf(ldexpf(f[k], -ex), -448.0f), 448.0f);
                    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
                    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
                    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
                    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 o8 = {static_cast<unsigned>(w0), static_cast<unsigned>(w1)};
                    if (m < seg_n && col >= lo && col <= hi) {
                        uint8_t* C8 = static_cast<uint8_t*>(a.C);
                        u32x2* dst = reinterpret_cast<u32x2*>(C8 + orow * ncols + col);
                        if (LBV_G1_EPI_NT) __builtin_nontemporal_store(o8, dst);
                        else *dst = o8;
                        // blocks 4g + (0, 1, 2, 3) of a row at bytes 4g + (0, 2, 1, 3)
                        const int kb = col / 32;
                        const int pos = (kb & ~3) | ((kb & 1) << 1) | ((kb >> 1) & 1);
                        if ((ch & 3) == 0) a.asc[orow * kA8ScalePitch + pos] = static_cast<uint8_t>(ex + 127);
                    }
                } else if (m < seg_n && col >= lo && col <= hi) {
                    u32x4* dst = reinterpret_cast<u32x4*>(C + orow * ncols + col);
                    if (MODE == 0 ? LBV_G1_EPI_NT : LBV_G2_EPI_NT) __builtin_nontemporal_store(v, dst);
                    else *dst = v;
                }
            }
        }
        if (!has_next) break;
        // every wave done with its staging reads (stage STG-1 may be refilled)
        // and every wave's copies of the next tile's first k-tiles landed
        wait_lgkmcnt0();
        block_barrier();
        // the next tile's copy sources again (they were set for its k-tile 0
        // copies before the epilogue; re-forming them here keeps them out of
        // the epilogue's registers), and the fragment offsets
        set_sources(nseg, nseg_r0, nseg_n, nm0, nnt, nlo, nhi);
        frag_offsets();
#pragma unroll
        for (int j = 0; j < TNS; ++j) sc[j] = nsc[j];
#pragma unroll
        for (int i = 0; i < TM; ++i) tf0[i] = *reinterpret_cast<const bf16x8*>(fa[0] + i * 32 * BK);
#pragma unroll
        for (int j = 0; j < TN; ++j) read_b(wf0, j, 0, 0);
        if constexpr (A8) {
#pragma unroll
            for (int r = 0; r < TM + TN; ++r) rd_frag(tqP, wqP, r, 0, 0);
            read_asc(asc, (it + 1) & 1, 0);
        }
        t = tn;
        ++it;
        seg = nseg;
        m0 = nm0;
        nt = nnt;
        lo = nlo;
        hi = nhi;
        seg_r0 = nseg_r0;
        seg_n = nseg_n;
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
                // gate/up: act rows in segment order; down: y rows in slot order
                const int64_t orow = MODE == 0 ? seg_r0 + m : a.rows[seg_r0 + m];
                C[orow * a.ncols + n] = v;
            }
        }
}

// ---------------------------------------------------------------------------
// Combine: one wave per token; the token's slot rows t*KS .. t*KS+KS-1 of y
// are contiguous (the down matmul stores them in slot order), so the step
// streams them, with non-temporal loads and stores (each byte is touched
// once; measured 319 -> 266 us at 38k tokens against cached loads).  Per step a lane owns 16 contiguous bytes of the output row
// and first issues the loads of all the token's routed slot rows, then sums
// them in slot order in fp32 and rounds once.  inv_rows only marks the empty
// slots (-1) of padding tokens.
// ---------------------------------------------------------------------------
struct CombArgs {
    const void* y;
    const int32_t* inv;
    const float* w;
    void* out;
    int64_t T;
    int H, K, NS, KS;
    // gated residual (RESID): out[t] = x[t] + gate[t] * sum, fp32, with
    // gate = table[5] + temb row t [5]
    const float* x;
    const float* temb;
    int64_t temb_stride;
    const float* table;
};

// RESID: the sum goes, unrounded, into the gated residual of the DiT layer
// (prhub summary of sglang PR #32341, "实现拆解" step 2: AdaLN with
// scale_shift_table and a token-level temb6): one read of the residual row
// and the gate, one fp32 write, instead of a round trip of the block output.
template <bool BF16, bool RESID>
__global__ __launch_bounds__(256) void combine_kernel(CombArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    constexpr int MAXS = 24;   // K <= 16 plus up to 8 shared pseudo-experts
    constexpr int EPL = BF16 ? 8 : 4;            // elements per 16-byte chunk
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int NC = LBV_COMB_CHUNKS;          // 16-byte chunks per lane per step
    int rows[MAXS];
    float wt[MAXS];
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        rows[k] = -1;
        wt[k] = 1.0f;
        if (k < a.KS) {
            rows[k] = a.inv[t * a.KS + k] < 0 ? -1 : static_cast<int>(t * a.KS + k);
            if (k < a.K) wt[k] = a.w[t * a.K + k];
        }
    }
    const char* y = static_cast<const char*>(a.y);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    for (int h0 = lane * EPL; h0 < a.H; h0 += 64 * EPL * NC) {
        u32x4 q[NC][MAXS];
        // RESID: the residual row and both gate parts are loaded with the
        // slot rows, so that all of a step's loads are in flight together
        f32x4 xv[NC][EPL / 4], ga[NC][EPL / 4], gb[NC][EPL / 4];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int h = h0 + c * 64 * EPL;
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k < a.KS && h < a.H) {
                    const int r = rows[k] < 0 ? 0 : rows[k];   // unused when the slot is empty
                    const u32x4* src = reinterpret_cast<const u32x4*>(y + (static_cast<int64_t>(r) * a.H + h) * ESZ);
                    q[c][k] = LBV_COMB_NT ? __builtin_nontemporal_load(src) : *src;
                }
            }
            if constexpr (RESID) {
                if (h < a.H) {
                    const f32x4* xr = reinterpret_cast<const f32x4*>(a.x + t * a.H + h);
                    const f32x4* g0 = reinterpret_cast<const f32x4*>(a.table + 5 * a.H + h);
                    const f32x4* g1 = reinterpret_cast<const f32x4*>(a.temb + t * a.temb_stride + 5 * a.H + h);
#pragma unroll
                    for (int j = 0; j < EPL / 4; ++j) {
                        xv[c][j] = __builtin_nontemporal_load(xr + j);
                        ga[c][j] = g0[j];
                        // one row for every token when the stride is 0: keep it cached
                        gb[c][j] = a.temb_stride ? __builtin_nontemporal_load(g1 + j) : g1[j];
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int h = h0 + c * 64 * EPL;
            if (h >= a.H) break;
            float acc[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k < a.KS && rows[k] >= 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // one fma per slot, written out (the compiler forms
                        // the same fma from a * b + c; explicit, the order of
                        // roundings does not depend on its choice)
                        if (BF16) {
                            acc[2 * i] = __builtin_fmaf(wt[k], __uint_as_float(q[c][k][i] << 16), acc[2 * i]);
                            acc[2 * i + 1] = __builtin_fmaf(wt[k], __uint_as_float(q[c][k][i] & 0xffff0000u), acc[2 * i + 1]);
                        } else {
                            acc[i] = __builtin_fmaf(wt[k], __uint_as_float(q[c][k][i]), acc[i]);
                        }
                    }
                }
            }
            if constexpr (RESID) {
                float* orow = static_cast<float*>(a.out) + t * a.H + h;
#pragma unroll
                for (int j = 0; j < EPL / 4; ++j) {
                    f32x4 ov;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ov[i] = xv[c][j][i] + (ga[c][j][i] + gb[c][j][i]) * acc[4 * j + i];
                    __builtin_nontemporal_store(ov, reinterpret_cast<f32x4*>(orow + 4 * j));
                }
            } else {
                u32x4 o;
                if (BF16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
                }
                __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<char*>(a.out) + (t * a.H + h) * ESZ));
            }
        }
    }
}

constexpr int G1_BM = LBV_G1_BM, G1_BN = LBV_G1_BN;
constexpr int G2_BM = LBV_G2_BM, G2_BN = LBV_G2_BN;

GemmArgs make_args(const Dims& d) {
    GemmArgs a{};
    a.T = d.T;
    a.H = d.H;
    a.I = d.I;
    a.E = d.E;
    a.NS = d.NS;
    a.KS = d.KS;
    a.S = d.S;
    a.ctr = nullptr;
    return a;
}

// Tile height of the grouped matmuls, from the rows per segment on average,
// T (K + ns) / S: 64 below `small`, 128 below `mid`, else `big`.  Shorter
// tiles pad each expert's few rows less; taller ones send each weight slice
// through a CU's copy path fewer times (128-row tiles hold a segment in about
// half as many tiles as 64-row ones).  With bf16 tokens the 64- and 128-row
// tiles have three stages (3 x 48 KB of LDS at 128 rows), which the
// HBM-bound small batches need, and 256-row tiles two.  The thresholds come
// from sweeps of the 128-expert layer (H 2048, I 768, top-8, one shared
// expert) over 50 to 38,000 tokens, forwards timed per tile height:
//   bf16 weights: 64 rows lead by ~1.5% up to 200 tokens (~14 rows per
//     segment), 128 rows from 400 to 6,000 tokens (28-420 rows; 1-14% ahead
//     of the better of the other two), 256 rows from 8,000 tokens (560 rows);
//   fp8 weights: 64-row gate/up tiles with 128-row down tiles lead by ~2%
//     from 600 to 1,000 tokens (42-70 rows), 128 rows for both by 9-12% at
//     1,600 and 3,000 tokens;
//   fp8 tokens (64, 128, 192 rows, two stages): 64 rows up to 400 tokens
//     (28 rows), 128 rows at 800 tokens (56 rows, 4% ahead), 192 rows from
//     1,600 tokens (112 rows; 12-19% ahead of 64 rows at 1,600 and 3,000).
// A row's sums do not depend on the tile height (same k order), so neither
// does the result.
int tile_rows(const Dims& d, int small, int mid, int big) {
    const int64_t rows = d.T * d.KS;
    if (rows < static_cast<int64_t>(small) * d.S) return 64;
    return rows < static_cast<int64_t>(mid) * d.S ? 128 : big;
}

// Zeroes the tile queue counters ahead of a grouped matmul on the same stream
// (a kernel rather than a memset, so that the call can be captured in a graph).
__global__ __launch_bounds__(64) void zero_ctr_kernel(int* ctr) {
    if (threadIdx.x < 8) ctr[threadIdx.x] = 0;
}

int64_t max_mtiles(const Dims& d, int BM) {
    return (d.T * d.KS + BM - 1) / BM + d.S;
}

template <bool W8>
void launch_w13_bf16(const Dims& d, const GemmArgs& a, hipStream_t stream) {
    const int bm = tile_rows(d, W8 ? LBV_W8_G1_SMALL_ROWS : LBV_G1_SMALL_ROWS, LBV_MID_ROWS, 256);
    if (bm == 64)
        hipLaunchKernelGGL((gemm_bf16_kernel<64, G1_BN, 0, LBV_G1_WAVES, LBV_G1_COPY_WAVES, LBV_G1_ORDER, LBV_FEW_STAGES, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G1_WAVES * 64), 0, stream, a);
    else if (bm == 128)
        hipLaunchKernelGGL((gemm_bf16_kernel<128, G1_BN, 0, LBV_G1_WAVES, LBV_G1_COPY_WAVES, LBV_G1_ORDER, LBV_FEW_STAGES, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G1_WAVES * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<G1_BM, G1_BN, 0, LBV_G1_WAVES, LBV_G1_COPY_WAVES, LBV_G1_ORDER, 2, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G1_WAVES * 64), 0, stream, a);
}

template <bool W8>
void launch_w2_bf16(const Dims& d, const GemmArgs& a, hipStream_t stream) {
    const int bm = tile_rows(d, W8 ? LBV_W8_G2_SMALL_ROWS : LBV_G2_SMALL_ROWS, LBV_MID_ROWS, 256);
    if (bm == 64)
        hipLaunchKernelGGL((gemm_bf16_kernel<64, G2_BN, 1, LBV_G2_WAVES, LBV_G2_COPY_WAVES, LBV_G2_ORDER, LBV_FEW_STAGES, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G2_WAVES * 64), 0, stream, a);
    else if (bm == 128)
        hipLaunchKernelGGL((gemm_bf16_kernel<128, G2_BN, 1, LBV_G2_WAVES, LBV_G2_COPY_WAVES, LBV_G2_ORDER, LBV_FEW_STAGES, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G2_WAVES * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<G2_BM, G2_BN, 1, LBV_G2_WAVES, LBV_G2_COPY_WAVES, LBV_G2_ORDER, 2, W8, false>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G2_WAVES * 64), 0, stream, a);
}

}  // namespace

hipError_t launch_gemm_w13(const Dims& d, const void* x, const void* w13,
                           const void* shared_w13, const int32_t* offsets,
                           const int32_t* sorted_rows, void* act, int* ctr, hipStream_t stream,
                           const float* w13_scale, const float* shared_w13_scale, bool zero_ctr) {
    GemmArgs a = make_args(d);
    a.ctr = ctr;
    a.A = x;
    a.B = w13;
    a.Bsh = shared_w13;
    a.Bs = w13_scale;
    a.Bshs = shared_w13_scale;
    a.offsets = offsets;
    a.rows = sorted_rows;
    a.C = act;
    a.kdim = d.H;
    a.ncols = d.I;
    if (d.bf16) {
        a.ntn = (d.I + G1_BN / 2 - 1) / (G1_BN / 2);
        if (zero_ctr) hipLaunchKernelGGL(zero_ctr_kernel, dim3(1), dim3(64), 0, stream, ctr);
        if (w13_scale) launch_w13_bf16<true>(d, a, stream);
        else launch_w13_bf16<false>(d, a, stream);
    } else {
        a.ntn = (d.I + 31) / 32;
        const int64_t grid = max_mtiles(d, 32) * a.ntn;
        hipLaunchKernelGGL(gemm_f32_kernel<0>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w2(const Dims& d, const void* act, const void* w2, const void* shared_w2,
                          const int32_t* offsets, const int32_t* sorted_rows, void* y, int* ctr,
                          hipStream_t stream, const float* w2_scale, const float* shared_w2_scale,
                          bool zero_ctr) {
    GemmArgs a = make_args(d);
    a.ctr = ctr;
    a.A = act;
    a.B = w2;
    a.Bsh = shared_w2;
    a.Bs = w2_scale;
    a.Bshs = shared_w2_scale;
    a.offsets = offsets;
    a.rows = sorted_rows;                        // slot of each sorted row: y is stored in slot order
    a.C = y;
    a.kdim = d.I;
    a.ncols = d.H;
    if (d.bf16) {
        a.ntn = (d.H + G2_BN - 1) / G2_BN;
        if (zero_ctr) hipLaunchKernelGGL(zero_ctr_kernel, dim3(1), dim3(64), 0, stream, ctr);
        if (w2_scale) launch_w2_bf16<true>(d, a, stream);
        else launch_w2_bf16<false>(d, a, stream);
    } else {
        a.ntn = (d.H + 31) / 32;
        const int64_t grid = max_mtiles(d, 32) * a.ntn;
        hipLaunchKernelGGL(gemm_f32_kernel<1>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           stream, a);
    }
    return hipGetLastError();
}

#ifndef LBV_A8_BM
#define LBV_A8_BM 192
#endif

hipError_t launch_gemm_w13_a8(const Dims& d, const uint8_t* xq, const float* xs,
                              const void* w13, const float* w13_scale, const void* shared_w13,
                              const float* shared_w13_scale, const int32_t* offsets,
                              const int32_t* sorted_rows, uint8_t* actq, uint8_t* act_scales,
                              int* ctr, hipStream_t stream) {
    GemmArgs a = make_args(d);
    a.ctr = ctr;
    a.A = xq;
    a.xs = xs;
    a.B = w13;
    a.Bsh = shared_w13;
    a.Bs = w13_scale;
    a.Bshs = shared_w13_scale;
    a.offsets = offsets;
    a.rows = sorted_rows;
    a.C = actq;
    a.asc = act_scales;
    a.kdim = d.H;
    a.ncols = d.I;
    a.ntn = (d.I + G1_BN / 2 - 1) / (G1_BN / 2);
    const int bm = tile_rows(d, LBV_A8_SMALL_ROWS, LBV_A8_MID_ROWS, LBV_A8_BM);
    if (bm == 64)
        hipLaunchKernelGGL((gemm_bf16_kernel<64, G1_BN, 0, 8, 4, LBV_G1_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    else if (bm == 128)
        hipLaunchKernelGGL((gemm_bf16_kernel<128, G1_BN, 0, 8, 4, LBV_G1_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<LBV_A8_BM, G1_BN, 0, 8, 4, LBV_G1_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_w2_a8(const Dims& d, const uint8_t* actq, uint8_t* act_scales,
                             const void* w2, const float* w2_scale, const void* shared_w2,
                             const float* shared_w2_scale, const int32_t* offsets,
                             const int32_t* sorted_rows, void* y, int* ctr, hipStream_t stream) {
    GemmArgs a = make_args(d);
    a.ctr = ctr;
    a.A = actq;
    a.asc = act_scales;
    a.B = w2;
    a.Bsh = shared_w2;
    a.Bs = w2_scale;
    a.Bshs = shared_w2_scale;
    a.offsets = offsets;
    a.rows = sorted_rows;                        // y is stored in slot order
    a.C = y;
    a.kdim = d.I;
    a.ncols = d.H;
    a.ntn = (d.H + G2_BN - 1) / G2_BN;         // a partial last n-tile (H = 128 mod 256) is clamped
    const int bm = tile_rows(d, LBV_A8_SMALL_ROWS, LBV_A8_MID_ROWS, LBV_A8_BM);
    if (bm == 64)
        hipLaunchKernelGGL((gemm_bf16_kernel<64, G2_BN, 1, 8, 4, LBV_G2_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    else if (bm == 128)
        hipLaunchKernelGGL((gemm_bf16_kernel<128, G2_BN, 1, 8, 4, LBV_G2_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<LBV_A8_BM, G2_BN, 1, 8, 4, LBV_G2_ORDER, 2, false, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(512), 0, stream, a);
    return hipGetLastError();
}

namespace {
// offsets of the one segment ([0, T]) and zeroed tile-queue counters
__global__ __launch_bounds__(64) void dense_setup_kernel(int32_t* offsets, int* ctr, int T) {
    const int l = threadIdx.x;
    if (l < 2) offsets[l] = l == 0 ? 0 : T;
    if (l < 8) ctr[l] = 0;
}
}  // namespace

hipError_t launch_linear(int64_t T, int N, int K, const void* x, const void* w, const float* bias,
                         void* y, void* ws, hipStream_t stream) {
    GemmArgs a{};
    a.T = T;
    a.H = N;
    a.I = K;
    a.E = 1;
    a.NS = 0;
    a.KS = 1;
    a.S = 1;
    a.A = x;
    a.B = w;
    a.Bsh = w;
    a.bias = bias;
    int32_t* offsets = static_cast<int32_t*>(ws);
    a.offsets = offsets;
    a.rows = nullptr;
    a.ctr = reinterpret_cast<int*>(static_cast<char*>(ws) + 256);
    a.C = y;
    a.kdim = K;
    a.ncols = N;
    a.ntn = (N + G2_BN - 1) / G2_BN;
    hipLaunchKernelGGL(dense_setup_kernel, dim3(1), dim3(64), 0, stream, offsets, a.ctr,
                       static_cast<int>(T));
    // 64-row tiles when 256-row ones would not give every CU a tile
    const int64_t tiles256 = (T + 255) / 256 * a.ntn;
    if (tiles256 < cu_count())
        hipLaunchKernelGGL((gemm_bf16_kernel<64, G2_BN, 1, LBV_G2_WAVES, LBV_G2_COPY_WAVES, LBV_G2_ORDER, LBV_FEW_STAGES, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G2_WAVES * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<G2_BM, G2_BN, 1, LBV_G2_WAVES, LBV_G2_COPY_WAVES, LBV_G2_ORDER, 2, false, true>),
                           dim3(cu_count() / 8 * 8), dim3(LBV_G2_WAVES * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const void* y, const int32_t* inv_rows,
                          const float* topk_w, void* out, hipStream_t stream) {
    CombArgs a{};
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
        hipLaunchKernelGGL((combine_kernel<true, false>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<false, false>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_combine_residual(const Dims& d, const void* y, const int32_t* inv_rows,
                                   const float* topk_w, const float* x, const float* temb,
                                   int64_t temb_stride, const float* table, float* out,
                                   hipStream_t stream) {
    CombArgs a{};
    a.y = y;
    a.inv = inv_rows;
    a.w = topk_w;
    a.out = out;
    a.T = d.T;
    a.H = d.H;
    a.K = d.K;
    a.NS = d.NS;
    a.KS = d.KS;
    a.x = x;
    a.temb = temb;
    a.temb_stride = temb_stride;
    a.table = table;
    const unsigned grid = static_cast<unsigned>((d.T + 3) / 4);
    if (d.bf16)
        hipLaunchKernelGGL((combine_kernel<true, true>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<false, true>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lbv

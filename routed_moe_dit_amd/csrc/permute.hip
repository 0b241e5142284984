// Token-to-expert permutation on gfx950 (vLLM-Omni LingBot-Video article,
// "MoE 实现的源码级要点": token copies are reordered by expert before the
// grouped matmuls and restored afterwards).
//
// A slot (t, k) with k < K is token t's k-th routed expert; slot (t, K + j) is
// shared pseudo-expert j.  The result is a stable counting sort of the slots
// by segment: inside a segment, rows follow slot id order.
//
// Three launches, all deterministic (no value depends on scheduling order):
//  1. count:   a block of 256 tokens builds, per wave and expert, a 64-bit
//              lane mask of the wave's tokens that chose the expert (LDS
//              ds_or_b64), and writes its per-expert token counts.
//  2. scan:    one block turns the counts into per-block starting offsets and
//              the segment offsets (shared pseudo-experts own T rows each);
//              a thread per expert walks its column of block counts.
//  3. scatter: every block rebuilds its masks; a token's rank inside its
//              expert's block range is the popcount of the lower lanes' bits
//              plus the counts of the lower waves, so the order is by token.
// Because the router never repeats an expert inside a token, one bit per
// (token, expert) is enough; ids out of range or repeated are skipped.
#include "lbv_internal.h"

namespace lbv {
namespace {

constexpr int PB = 256;        // tokens per block
constexpr int PMAX_E = 256;
constexpr int PMAX_K = 16;

struct PermArgs {
    const int32_t* ids;
    int32_t* blk;          // [nb][E] counts, then block offsets
    int32_t* offsets;      // [S+1]
    int32_t* sorted_rows;
    int32_t* inv_rows;
    int* ctr0;             // optional: tile queue counters of the matmuls that
    int* ctr1;             // follow on the stream, zeroed by the scan (8 ints each)
    int64_t T;
    int K, E, NS, KS, nb;
};

// Loads token t's ids, marking out-of-range ids and repeats as -1.
__device__ __forceinline__ void load_ids(const PermArgs& a, int64_t t, int* e) {
#pragma unroll
    for (int k = 0; k < PMAX_K; ++k) {
        e[k] = -1;
        if (k < a.K) {
            int v = a.ids[t * a.K + k];
            if (v < 0 || v >= a.E) v = -1;
#pragma unroll
            for (int j = 0; j < PMAX_K; ++j)
                if (j < k && e[j] == v) v = -1;
            e[k] = v;
        }
    }
}

__device__ __forceinline__ void build_masks(const PermArgs& a, unsigned long long (*bits)[PMAX_E],
                                            int* e, bool& has) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 4 * PMAX_E; i += PB) (&bits[0][0])[i] = 0ull;
    __syncthreads();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * PB + tid;
    has = t < a.T;
    if (has) {
        load_ids(a, t, e);
#pragma unroll
        for (int k = 0; k < PMAX_K; ++k)
            if (k < a.K && e[k] >= 0) atomicOr(&bits[wave][e[k]], 1ull << lane);
    }
    __syncthreads();
}

__global__ __launch_bounds__(PB) void perm_count_kernel(PermArgs a) {
    __shared__ unsigned long long bits[4][PMAX_E];
    int e[PMAX_K];
    bool has;
    build_masks(a, bits, e, has);
    for (int x = threadIdx.x; x < a.E; x += PB) {
        const int c = __popcll(bits[0][x]) + __popcll(bits[1][x]) + __popcll(bits[2][x]) +
                      __popcll(bits[3][x]);
        a.blk[static_cast<int64_t>(blockIdx.x) * a.E + x] = c;
    }
}

// Exclusive scan of one value per thread over a 256-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp /*[4]*/, int& total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += tmp[w];
    total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    __syncthreads();
    return base + inc - v;
}

__global__ __launch_bounds__(PB) void perm_scan_kernel(PermArgs a) {
    __shared__ int tmp[4];
    const int tid = threadIdx.x;
    if (tid < 8) {
        if (a.ctr0) a.ctr0[tid] = 0;
        if (a.ctr1) a.ctr1[tid] = 0;
    }
    // per expert: block offsets (in place) and the expert's total
    // (chunks of 16 independent loads, so that the column is not walked one
    // memory latency per block)
    int total_e = 0;
    if (tid < a.E) {
        constexpr int CH = 16;
        int run = 0;
        for (int b0 = 0; b0 < a.nb; b0 += CH) {
            int c[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i)
                c[i] = b0 + i < a.nb ? a.blk[static_cast<int64_t>(b0 + i) * a.E + tid] : 0;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (b0 + i < a.nb) a.blk[static_cast<int64_t>(b0 + i) * a.E + tid] = run;
                run += c[i];
            }
        }
        total_e = run;
    }
    // segment sizes: experts 0..E-1 (all in the first pass, since E <= 256),
    // then NS shared pseudo-experts of T rows.  S = E + NS <= 264 segments.
    int carry = 0;
    for (int base = 0; base < a.E + a.NS; base += PB) {
        const int s = base + tid;
        int v = 0;
        if (s < a.E) v = total_e;
        else if (s < a.E + a.NS) v = static_cast<int>(a.T);
        int tot;
        const int ex = block_exclusive_scan(v, tmp, tot);
        if (s < a.E + a.NS) a.offsets[s] = carry + ex;
        carry += tot;
    }
    if (tid == 0) a.offsets[a.E + a.NS] = carry;
}

__global__ __launch_bounds__(PB) void perm_scatter_kernel(PermArgs a) {
    __shared__ unsigned long long bits[4][PMAX_E];
    int e[PMAX_K];
    bool has;
    build_masks(a, bits, e, has);
    if (!has) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * PB + tid;
    const unsigned long long lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int k = 0; k < PMAX_K; ++k) {
        if (k < a.K) {
            const int64_t slot = t * a.KS + k;
            const int x = e[k];
            if (x < 0) {
                a.inv_rows[slot] = -1;
            } else {
                int rank = __popcll(bits[wave][x] & lower);
                for (int w = 0; w < wave; ++w) rank += __popcll(bits[w][x]);
                const int pos =
                    a.offsets[x] + a.blk[static_cast<int64_t>(blockIdx.x) * a.E + x] + rank;
                a.sorted_rows[pos] = static_cast<int32_t>(slot);
                a.inv_rows[slot] = pos;
            }
        }
    }
    for (int j = 0; j < a.NS; ++j) {
        const int64_t slot = t * a.KS + a.K + j;
        const int pos = a.offsets[a.E + j] + static_cast<int>(t);
        a.sorted_rows[pos] = static_cast<int32_t>(slot);
        a.inv_rows[slot] = pos;
    }
}

}  // namespace

size_t permute_ws_bytes(const Dims& d) {
    const int64_t nb = (d.T + PB - 1) / PB;
    return static_cast<size_t>(nb) * d.E * sizeof(int32_t);
}

hipError_t launch_permute(const Dims& d, const int32_t* topk_ids, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* inv_rows, void* ws,
                          hipStream_t stream, int* zero_ctr0, int* zero_ctr1) {
    PermArgs a;
    a.ctr0 = zero_ctr0;
    a.ctr1 = zero_ctr1;
    a.ids = topk_ids;
    a.blk = static_cast<int32_t*>(ws);
    a.offsets = offsets;
    a.sorted_rows = sorted_rows;
    a.inv_rows = inv_rows;
    a.T = d.T;
    a.K = d.K;
    a.E = d.E;
    a.NS = d.NS;
    a.KS = d.KS;
    a.nb = static_cast<int>((d.T + PB - 1) / PB);
    hipLaunchKernelGGL(perm_count_kernel, dim3(a.nb), dim3(PB), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(PB), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(a.nb), dim3(PB), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lbv

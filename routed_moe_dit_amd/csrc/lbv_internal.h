// Internal declarations shared by the HIP sources of liblbv_moe.
// Device helpers (bf16 storage, XCD-aware block order, segment lookup) and the
// launchers that the C ABI in abi.cpp calls after validating its arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace lbv {

// ---------------------------------------------------------------------------
// Problem description resolved on the host from lbv_moe_config.
// ---------------------------------------------------------------------------
struct Dims {
    int64_t T;      // tokens
    int H;          // hidden
    int E;          // routed experts
    int K;          // top_k
    int NG;         // n_group
    int TG;         // topk_group
    int G;          // experts per group
    int EPL;        // experts per lane in the router (1, 2 or 4)
    int LG;         // lanes per group in the router (G / EPL, a power of two)
    int I;          // routed expert width
    int NS;         // shared pseudo-experts (each of width I)
    int KS;         // slots per token: K + NS
    int S;          // segments: E + NS
    int norm;       // norm_topk_prob
    float rsf;      // routed_scaling_factor
    int bf16;       // 1: bf16 storage, 0: fp32 storage
};

// Compute units of the current device (cached per device; 256 if the query
// fails).
inline int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 8)
            cu = 256;
        cached[dev] = cu;
    }
    return cached[dev];
}

// Launchers (all enqueue on `stream`, return hipGetLastError()).
size_t route_ws_bytes(const Dims& d);
hipError_t launch_route(const Dims& d, const void* x, const float* router_w, const float* e_bias,
                        const uint8_t* mask, int32_t* topk_ids, float* topk_w, void* ws,
                        hipStream_t stream);

// Allocation-free router: the fixed per-device scratch (the router
// workspace must fit in it) and its device address on the current device.
constexpr size_t kRouteScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
hipError_t route_scratch(void** ptr);

// zero_ctr0 / zero_ctr1: optional tile queue counters (8 ints each) of the
// matmuls that follow on the stream, zeroed by the permutation's scan, so that
// those matmuls can be launched with zero_ctr = false.
size_t permute_ws_bytes(const Dims& d);
hipError_t launch_permute(const Dims& d, const int32_t* topk_ids, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* inv_rows, void* ws,
                          hipStream_t stream, int* zero_ctr0 = nullptr,
                          int* zero_ctr1 = nullptr);

// The grouped matmuls take `ctr`: 8 ints of device scratch for their tile
// queues, zero when the matmul starts: the launcher zeroes them on the stream
// unless zero_ctr is false (the caller has zeroed them earlier on the same
// stream, e.g. in the permutation).  With row scales (bf16 activations only)
// the weights are e4m3fn codes, one power-of-two scale per weight row.
constexpr size_t kGemmCtrBytes = 256;

hipError_t launch_gemm_w13(const Dims& d, const void* x, const void* w13,
                           const void* shared_w13, const int32_t* offsets,
                           const int32_t* sorted_rows, void* act, int* ctr, hipStream_t stream,
                           const float* w13_scale = nullptr,
                           const float* shared_w13_scale = nullptr, bool zero_ctr = true);

hipError_t launch_gemm_w2(const Dims& d, const void* act, const void* w2, const void* shared_w2,
                          const int32_t* offsets, const int32_t* sorted_rows, void* y, int* ctr,
                          hipStream_t stream, const float* w2_scale = nullptr,
                          const float* shared_w2_scale = nullptr, bool zero_ctr = true);

// e4m3fn codes and power-of-two scales of weight rows (bf16 or fp32 source)
hipError_t launch_quantize_fp8(const void* w, int src_bf16, int64_t rows, int cols, uint8_t* q,
                               float* scale, hipStream_t stream);

// fp8 tokens and fp8 weights (both matmuls on the scaled fp8 MFMA).  act's
// MX block scales take kA8ScalePitch bytes per act row (I / 32 of them used),
// so I <= 32 * kA8ScalePitch; H and I are multiples of 128.
constexpr int kA8ScalePitch = 32;

// gate/up: xq [T, H] e4m3fn codes with xs [T] power-of-two scales; weight
// codes and row scales as for the fp8-weight path; writes actq [rows, I]
// codes and act_scales [rows, kA8ScalePitch] e8m0 bytes.  The counters must
// be zero (the permutation's scan zeroes them).
hipError_t launch_gemm_w13_a8(const Dims& d, const uint8_t* xq, const float* xs,
                              const void* w13, const float* w13_scale, const void* shared_w13,
                              const float* shared_w13_scale, const int32_t* offsets,
                              const int32_t* sorted_rows, uint8_t* actq, uint8_t* act_scales,
                              int* ctr, hipStream_t stream);

// down: actq / act_scales as written above; y [rows, H] bf16 in slot order.
hipError_t launch_gemm_w2_a8(const Dims& d, const uint8_t* actq, uint8_t* act_scales,
                             const void* w2, const float* w2_scale, const void* shared_w2,
                             const float* shared_w2_scale, const int32_t* offsets,
                             const int32_t* sorted_rows, void* y, int* ctr, hipStream_t stream);

hipError_t launch_combine(const Dims& d, const void* y, const int32_t* inv_rows,
                          const float* topk_w, void* out, hipStream_t stream);

// Dense bf16 linear y [T, N] = x [T, K] W[N, K]^T (+ bias [N] fp32), rounded
// once to bf16, on the grouped matmul kernel with one segment; ws: 512 bytes
// (segment offsets and tile-queue counters, set on the stream).
constexpr size_t kLinearWsBytes = 512;
hipError_t launch_linear(int64_t T, int N, int K, const void* x, const void* w, const float* bias,
                         void* y, void* ws, hipStream_t stream);

// Attention half (head dim 128): q/k norms + rotary embedding + v transposed
// into vt [B][heads][128][attn_sp(S)], then masked per-sample attention.
int attn_sp(int S);
hipError_t launch_attn_prep(int B, int S, int H, int heads, const void* qkv, const float* gq,
                            const float* gk, const float* cs, const float* sn, float eps, void* q,
                            void* k, void* vt, hipStream_t stream);
hipError_t launch_attn_core(int B, int S, int H, int heads, const void* q, const void* k,
                            const void* vt, const uint8_t* mask, void* o, hipStream_t stream);

// AdaLN in front of the block and the gated residual after it.
struct AdalnArgs {
    const float* x;        // [T, H] fp32 residual stream
    const float* temb;     // temb6 rows: token t's 6 H values at temb + t * temb_stride
    int64_t temb_stride;   // 0: one row for every token
    const float* table;    // scale_shift_table [6, H]
    float eps;
    void* h;               // [T, H] block input (cfg dtype)
    int64_t T;
    int H;
    hipStream_t stream;
    int shift_row = 3;     // rows of table / temb6: 3, 4 in front of the FFN
    int scale_row = 4;     // block, 0, 1 in front of the attention block
};
hipError_t launch_adaln(const Dims& d, const AdalnArgs& a);
hipError_t launch_adaln_bf16(const AdalnArgs& a);

// out[t] = x[t] + (table[row] + temb row t [row]) * y[t], y bf16, fp32 in and
// out (out may be x)
hipError_t launch_gated_residual(int64_t T, int H, const float* x, const void* y,
                                 const float* temb, int64_t temb_stride, const float* table,
                                 int row, float* out, hipStream_t stream);

// combine + gated residual: out[t] = x[t] + gate[t] * (sum_k w y + shared y),
// gate = table[5] + temb6 row t [5], fp32 in and out (out may be x)
hipError_t launch_combine_residual(const Dims& d, const void* y, const int32_t* inv_rows,
                                   const float* topk_w, const float* x, const float* temb,
                                   int64_t temb_stride, const float* table, float* out,
                                   hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// bf16 is stored as its 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 with gfx950's v_cvt_pk_bf16_f32 (the
// rounding mode is the wave's default, nearest-even); NaN stays NaN.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Zero that the compiler cannot see through: a value derived from it is
// formed where it is written (the memory clobber also keeps it from moving
// across the surrounding loads and stores).
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z) : : "memory");
    return z;
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Renumber them so that each XCD walks a contiguous range of logical tiles:
// neighbouring tiles (which share operand rows) then meet in the same L2.
__device__ __forceinline__ int xcd_logical_block(int b, int nblocks) {
    constexpr int NX = 8;
    int xcd = b % NX;
    int idx = b / NX;
    int base = nblocks / NX;
    int rem = nblocks % NX;
    return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

}  // namespace lbv

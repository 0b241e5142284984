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

size_t permute_ws_bytes(const Dims& d);
hipError_t launch_permute(const Dims& d, const int32_t* topk_ids, int32_t* offsets,
                          int32_t* sorted_rows, int32_t* inv_rows, void* ws,
                          hipStream_t stream);

hipError_t launch_gemm_w13(const Dims& d, const void* x, const void* w13,
                           const void* shared_w13, const int32_t* offsets,
                           const int32_t* sorted_rows, void* act, hipStream_t stream);

hipError_t launch_gemm_w2(const Dims& d, const void* act, const void* w2, const void* shared_w2,
                          const int32_t* offsets, const int32_t* sorted_rows, void* y,
                          hipStream_t stream);

hipError_t launch_combine(const Dims& d, const void* y, const int32_t* inv_rows,
                          const float* topk_w, void* out, hipStream_t stream);

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

// FP8 expert weights: e4m3fn codes with one power-of-two scale per weight row.
//
// The LingBot-Video recipe of vLLM-Omni ("Known Limitations") names FP8 among
// the expert backends its first integration leaves out; the pages give no
// recipe for it.  This one keeps the pages' bf16 activations and fp32
// accumulation and stores only the weights in 8 bits: row r of a weight
// matrix becomes codes q[r, :] and a scale 2^e[r], e the smallest integer with
// max|w[r, :]| <= 448 * 2^e (448 is e4m3fn's largest finite value; e = 0 for
// an all-zero row), q the nearest e4m3fn value of w * 2^-e, ties to the even
// code.  The dequantized weight decode(q) * 2^e has at most 4 significant
// bits, so it is exact in bf16, and the matmuls' conversion instruction
// (v_cvt_scalef32_pk_bf16_fp8) forms it exactly from the code and the scale.
#include "lbv_internal.h"

namespace lbv {
namespace {

// One wave per row: the row's largest magnitude (exact: a max), its exponent,
// then the codes, 4 per lane per step.  cols % 4 == 0.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* w, int64_t rows, int cols,
                                                           uint8_t* q, float* scale) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    auto load4 = [&](int c, float* v) {
        if (BF16) {
            const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(w) + r * cols + c);
            v[0] = __uint_as_float(b.x << 16);
            v[1] = __uint_as_float(b.x & 0xffff0000u);
            v[2] = __uint_as_float(b.y << 16);
            v[3] = __uint_as_float(b.y & 0xffff0000u);
        } else {
            const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + r * cols + c);
            v[0] = f.x;
            v[1] = f.y;
            v[2] = f.z;
            v[3] = f.w;
        }
    };
    float amax = 0.0f;
    for (int c = lane * 4; c < cols; c += 256) {
        float v[4];
        load4(c, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    // amax = f 2^x with 0.5 <= f < 1; 448 = 0.875 2^9
    int e = 0;
    if (amax > 0.0f) {
        int x;
        const float f = frexpf(amax, &x);
        e = f <= 0.875f ? x - 9 : x - 8;
    }
    if (lane == 0) scale[r] = ldexpf(1.0f, e);
    for (int c = lane * 4; c < cols; c += 256) {
        float v[4];
        load4(c, v);
        // exact scaling by 2^-e; |v| <= 448, where the conversion rounds to
        // nearest even (it does not saturate, hence the no-op clamp)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(ldexpf(v[i], -e), -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
        *reinterpret_cast<int*>(q + r * cols + c) = p;
    }
}

typedef unsigned int u32x4q __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2q __attribute__((ext_vector_type(2)));

// bf16 rows of at most 512 NC values (cols % 8 == 0): one wave per row reads
// it once, chunk j of lane l (8 values) at column 8 (64 j + l), keeps it in
// registers for the conversion, and computes exactly what quantize_fp8_kernel
// computes (the same maximum, exponent, scaling, clamp and conversions).
template <int NC>
__global__ __launch_bounds__(256) void quantize_fp8_bf16_row_kernel(const uint16_t* w, int64_t rows,
                                                                    int cols, uint8_t* q,
                                                                    float* scale) {
    const int lane = threadIdx.x & 63;
    const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const uint16_t* row = w + r * cols;
    u32x4q v[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = 8 * (64 * j + lane);
        v[j] = c < cols ? *reinterpret_cast<const u32x4q*>(row + c) : u32x4q{0u, 0u, 0u, 0u};
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
            amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(v[j][k] << 16)),
                                     fabsf(__uint_as_float(v[j][k] & 0xffff0000u))));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    int e = 0;
    if (amax > 0.0f) {
        int x;
        const float f = frexpf(amax, &x);
        e = f <= 0.875f ? x - 9 : x - 8;
    }
    if (lane == 0) scale[r] = ldexpf(1.0f, e);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = 8 * (64 * j + lane);
        if (c >= cols) continue;
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = fminf(fmaxf(ldexpf(__uint_as_float(v[j][k] << 16), -e), -448.0f), 448.0f);
            f[2 * k + 1] = fminf(fmaxf(ldexpf(__uint_as_float(v[j][k] & 0xffff0000u), -e), -448.0f), 448.0f);
        }
        int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
        p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p0, true);
        int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
        p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], p1, true);
        *reinterpret_cast<u32x2q*>(q + r * cols + c) = u32x2q{static_cast<unsigned>(p0), static_cast<unsigned>(p1)};
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const void* w, int src_bf16, int64_t rows, int cols, uint8_t* q,
                               float* scale, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>((rows + 3) / 4);
    if (src_bf16 && cols % 8 == 0 && cols <= 4096) {
        const uint16_t* wb = static_cast<const uint16_t*>(w);
        if (cols <= 1024)
            hipLaunchKernelGGL(quantize_fp8_bf16_row_kernel<2>, dim3(grid), dim3(256), 0, stream, wb, rows, cols, q, scale);
        else if (cols <= 2048)
            hipLaunchKernelGGL(quantize_fp8_bf16_row_kernel<4>, dim3(grid), dim3(256), 0, stream, wb, rows, cols, q, scale);
        else
            hipLaunchKernelGGL(quantize_fp8_bf16_row_kernel<8>, dim3(grid), dim3(256), 0, stream, wb, rows, cols, q, scale);
    } else if (src_bf16)
        hipLaunchKernelGGL(quantize_fp8_kernel<true>, dim3(grid), dim3(256), 0, stream, w, rows, cols, q, scale);
    else
        hipLaunchKernelGGL(quantize_fp8_kernel<false>, dim3(grid), dim3(256), 0, stream, w, rows, cols, q, scale);
    return hipGetLastError();
}

}  // namespace lbv

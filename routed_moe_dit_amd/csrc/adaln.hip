// RMSNorm + AdaLN modulation in front of the routed-MoE block of a
// LingBot-Video DiT layer, on gfx950.
//
// What it computes (prhub summary of sglang PR #32341, "实现拆解" step 2:
// AdaLN through scale_shift_table and a token-level temb6, the norms among
// the fp32 modules; vLLM-Omni LingBot-Video article, "MoE 实现的源码级要点":
// RMSNorm accumulates in fp32):
//   h[t] = x[t] / sqrt(mean(x[t]^2) + eps) * (1 + scale[t]) + shift[t]
// with shift = table[3] + temb6[t][3] and scale = table[4] + temb6[t][4]
// (fp32) in front of the FFN block, rows 0 and 1 in front of the attention
// block, rounded once to the block's storage type.  The FFN block's gated
// residual is formed in the combine (gemm.hip); the attention block's here
// (gated_residual_kernel, gate row 2).
//
// One wave per token: each lane reads 16-byte pieces of the fp32 row, the sum
// of squares is reduced across the wave in fp32, and the lane writes its
// modulated values.  HBM-bound: per token 4 H bytes of x, 8 H of shift and
// scale when temb6 is per token, and 2 H (bf16) of h.
#include "lbv_internal.h"

namespace lbv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
__global__ __launch_bounds__(256) void adaln_rmsnorm_kernel(AdalnArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    const int H = a.H;
    const float* xr = a.x + t * H;
    const float* er = a.temb + t * a.temb_stride;
    float ss = 0.f;
    // first pass cached (the row is read again right below), second pass
    // streamed
    for (int i = lane * 4; i < H; i += 256) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(xr + i);
        ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(H) + a.eps);
    for (int i = lane * 4; i < H; i += 256) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr + i));
        const f32x4 sh0 = *reinterpret_cast<const f32x4*>(a.table + a.shift_row * H + i);
        const f32x4 sc0 = *reinterpret_cast<const f32x4*>(a.table + a.scale_row * H + i);
        const f32x4 sh1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(er + a.shift_row * H + i));
        const f32x4 sc1 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(er + a.scale_row * H + i));
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = v[j] * r * (1.0f + (sc0[j] + sc1[j])) + (sh0[j] + sh1[j]);
        if (BF16) {
            uint2 p;
            p.x = pack_bf16x2(o[0], o[1]);
            p.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.h) + t * H + i) = p;
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.h) + t * H + i) = f32x4{o[0], o[1], o[2], o[3]};
        }
    }
}

// One wave per token: out = x + gate * y, 4 values a lane per step (16 bytes
// of x and out, 8 of y); HBM-bound.
struct ResidArgs {
    const float* x;
    const uint16_t* y;
    const float* temb;
    int64_t temb_stride;
    const float* table;
    float* out;
    int64_t T;
    int H, row;
};

__global__ __launch_bounds__(256) void gated_residual_kernel(ResidArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (t >= a.T) return;
    const int H = a.H;
    const float* g0 = a.table + a.row * H;
    const float* g1 = a.temb + t * a.temb_stride + a.row * H;
    for (int i = lane * 4; i < H; i += 256) {
        const f32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.x + t * H + i));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 yw = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.y + t * H + i));
        const uint2 yv = {yw[0], yw[1]};
        const f32x4 ga = *reinterpret_cast<const f32x4*>(g0 + i);
        const f32x4 gb = *reinterpret_cast<const f32x4*>(g1 + i);
        const float y4[4] = {bf16_to_f32(static_cast<uint16_t>(yv.x)), bf16_to_f32(static_cast<uint16_t>(yv.x >> 16)),
                             bf16_to_f32(static_cast<uint16_t>(yv.y)), bf16_to_f32(static_cast<uint16_t>(yv.y >> 16))};
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = xv[j] + (ga[j] + gb[j]) * y4[j];
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(a.out + t * H + i));
    }
}

}  // namespace

hipError_t launch_adaln_bf16(const AdalnArgs& a) {
    const unsigned grid = static_cast<unsigned>((a.T + 3) / 4);
    hipLaunchKernelGGL(adaln_rmsnorm_kernel<true>, dim3(grid), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

hipError_t launch_gated_residual(int64_t T, int H, const float* x, const void* y,
                                 const float* temb, int64_t temb_stride, const float* table,
                                 int row, float* out, hipStream_t stream) {
    ResidArgs a{x, static_cast<const uint16_t*>(y), temb, temb_stride, table, out, T, H, row};
    const unsigned grid = static_cast<unsigned>((T + 3) / 4);
    hipLaunchKernelGGL(gated_residual_kernel, dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_adaln(const Dims& d, const AdalnArgs& a) {
    const unsigned grid = static_cast<unsigned>((d.T + 3) / 4);
    if (d.bf16)
        hipLaunchKernelGGL(adaln_rmsnorm_kernel<true>, dim3(grid), dim3(256), 0, a.stream, a);
    else
        hipLaunchKernelGGL(adaln_rmsnorm_kernel<false>, dim3(grid), dim3(256), 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace lbv

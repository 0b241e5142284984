// Host side of the lbv_moe C ABI: argument validation, workspace carving and
// kernel launches on the caller's stream.  Nothing here allocates device
// memory or synchronises; every check runs before the first launch, so a
// rejected call has no side effect.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "lbv_internal.h"
#include "lbv_moe.h"

using lbv::Dims;

namespace {

constexpr int32_t kAbiVersion = 6;
constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

lbv_status check_cfg(const lbv_moe_config* c) {
    if (!c) return LBV_ERR_NULL;
    if (c->score_func != LBV_SCORE_SIGMOID) return LBV_ERR_UNSUPPORTED;
    if (c->dtype != LBV_F32 && c->dtype != LBV_BF16) return LBV_ERR_UNSUPPORTED;
    if (c->hidden <= 0 || c->hidden % 64 != 0) return LBV_ERR_SHAPE;
    if (c->intermediate <= 0 || c->intermediate % 64 != 0) return LBV_ERR_SHAPE;
    if (c->num_experts <= 0 || c->n_group <= 0 || c->num_experts % c->n_group != 0)
        return LBV_ERR_SHAPE;
    if (c->topk_group <= 0 || c->topk_group > c->n_group) return LBV_ERR_SHAPE;
    const int G = c->num_experts / c->n_group;
    if (c->top_k <= 0 || c->top_k > c->topk_group * G) return LBV_ERR_SHAPE;
    if (c->n_shared_experts < 0) return LBV_ERR_SHAPE;
    if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1) return LBV_ERR_SHAPE;
    if (!isfinite(c->routed_scaling_factor)) return LBV_ERR_SHAPE;
    if (c->num_experts > 256 || c->top_k > 16 || c->n_shared_experts > 8 || c->n_group > 32)
        return LBV_ERR_UNSUPPORTED;
    if (G < 2) return LBV_ERR_UNSUPPORTED;
    int epl = 1;
    while (64 * epl < c->num_experts) epl *= 2;
    if (G % epl != 0 || !is_pow2(G / epl)) return LBV_ERR_UNSUPPORTED;
    // bf16 matmuls address their weight rows with 32-bit byte offsets
    if (c->dtype == LBV_BF16) {
        const int64_t w13_bytes = 2ll * c->intermediate * c->hidden * 2;
        const int64_t shared_bytes = w13_bytes * c->n_shared_experts;
        if (w13_bytes >= (1ll << 32) || shared_bytes >= (1ll << 32)) return LBV_ERR_SHAPE;
        // and form row offsets with 24-bit multiplies
        if (c->hidden >= (1 << 24) || 2ll * c->intermediate * (c->n_shared_experts > 1 ? c->n_shared_experts : 1) >= (1 << 24))
            return LBV_ERR_SHAPE;
    }
    return LBV_OK;
}

lbv_status make_dims(const lbv_moe_config* c, int64_t T, Dims* d) {
    lbv_status st = check_cfg(c);
    if (st != LBV_OK) return st;
    if (T < 0) return LBV_ERR_SHAPE;
    const int KS = c->top_k + c->n_shared_experts;
    // row indices and offsets are int32
    if (T > 0 && T > (int64_t)INT32_MAX / KS) return LBV_ERR_SHAPE;
    // the bf16 gate/up matmul gathers rows of x with 32-bit byte offsets
    // and the down matmul addresses act rows of a segment (at most T of them)
    // with 32-bit byte offsets
    if (c->dtype == LBV_BF16 && (T * c->hidden * 2 >= (1ll << 32) || T >= (1 << 24) ||
                                 T * c->intermediate * 2 >= (1ll << 32)))
        return LBV_ERR_SHAPE;
    d->T = T;
    d->H = c->hidden;
    d->E = c->num_experts;
    d->K = c->top_k;
    d->NG = c->n_group;
    d->TG = c->topk_group;
    d->G = c->num_experts / c->n_group;
    int epl = 1;
    while (64 * epl < c->num_experts) epl *= 2;
    d->EPL = epl;
    d->LG = d->G / epl;
    d->I = c->intermediate;
    d->NS = c->n_shared_experts;
    d->KS = KS;
    d->S = c->num_experts + c->n_shared_experts;
    d->norm = c->norm_topk_prob;
    d->rsf = c->routed_scaling_factor;
    d->bf16 = c->dtype == LBV_BF16 ? 1 : 0;
    return LBV_OK;
}

size_t elem_bytes(const Dims& d) { return d.bf16 ? 2 : 4; }

// Forward workspace layout (each part 256-byte aligned).
struct FwdLayout {
    size_t ids, w, offsets, sorted, inv, perm, route, ctr1, ctr2, act, y, total;
};

FwdLayout fwd_layout(const Dims& d) {
    FwdLayout L;
    const size_t T = static_cast<size_t>(d.T);
    size_t off = 0;
    L.ids = off;     off += round_up(T * d.K * sizeof(int32_t));
    L.w = off;       off += round_up(T * d.K * sizeof(float));
    L.offsets = off; off += round_up((d.S + 1) * sizeof(int32_t));
    L.sorted = off;  off += round_up(T * d.KS * sizeof(int32_t));
    L.inv = off;     off += round_up(T * d.KS * sizeof(int32_t));
    L.perm = off;    off += round_up(lbv::permute_ws_bytes(d));
    L.route = off;   off += round_up(lbv::route_ws_bytes(d));
    L.ctr1 = off;    off += round_up(lbv::kGemmCtrBytes);
    L.ctr2 = off;    off += round_up(lbv::kGemmCtrBytes);
    L.act = off;     off += round_up(T * d.KS * d.I * elem_bytes(d));
    L.y = off;       off += round_up(T * d.KS * d.H * elem_bytes(d));
    L.total = off;
    return L;
}

// down matmul workspace: the expert outputs y [T (K + ns), H], then the tile
// queue counters
size_t w2_y_bytes(const Dims& d) {
    return round_up(static_cast<size_t>(d.T) * d.KS * d.H * elem_bytes(d));
}
size_t w2_ws_bytes(const Dims& d) { return w2_y_bytes(d) + round_up(lbv::kGemmCtrBytes); }
size_t w13_ws_bytes(const Dims&) { return round_up(lbv::kGemmCtrBytes); }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

lbv_status hip_status(hipError_t e) { return e == hipSuccess ? LBV_OK : LBV_ERR_HIP; }

// The FFN half of a DiT layer: the forward workspace, then the block input h.
size_t ffn_h_offset(const Dims& d) { return fwd_layout(d).total; }
size_t ffn_ws_bytes(const Dims& d) {
    return ffn_h_offset(d) + round_up(static_cast<size_t>(d.T) * d.H * elem_bytes(d));
}

// Checks of the AdaLN operands shared by lbv_adaln_rmsnorm and lbv_moe_ffn_adaln.
lbv_status check_adaln(const Dims& d, const float* x, const float* temb6, int64_t temb_stride,
                       const float* table, float eps) {
    if (!x || !temb6 || !table) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(temb6) || !aligned16(table)) return LBV_ERR_ALIGN;
    if (temb_stride < 0 || temb_stride % 4 != 0) return LBV_ERR_ALIGN;
    if (!(eps >= 0.0f) || !isfinite(eps)) return LBV_ERR_SHAPE;
    (void)d;
    return LBV_OK;
}

}  // namespace

extern "C" {

int32_t lbv_abi_version(void) { return kAbiVersion; }

const char* lbv_status_string(lbv_status s) {
    switch (s) {
        case LBV_OK: return "ok";
        case LBV_ERR_NULL: return "a required pointer is NULL";
        case LBV_ERR_SHAPE: return "a size or configuration field is out of range";
        case LBV_ERR_UNSUPPORTED: return "configuration not supported by this build";
        case LBV_ERR_ALIAS: return "out overlaps x (the block is not in-place)";
        case LBV_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case LBV_ERR_WORKSPACE: return "workspace smaller than the size query returns";
        case LBV_ERR_HIP: return "a HIP kernel launch failed";
        case LBV_ERR_SCRATCH:
            return "the allocation-free call's fixed scratch is too small for this configuration";
    }
    return "unknown status";
}

lbv_status lbv_moe_check_config(const lbv_moe_config* cfg) { return check_cfg(cfg); }

lbv_status lbv_moe_workspace_size(const lbv_moe_config* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    *bytes = fwd_layout(d).total;
    return LBV_OK;
}

lbv_status lbv_moe_route_workspace_size(const lbv_moe_config* cfg, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, 0, &d);
    if (st != LBV_OK) return st;
    *bytes = round_up(lbv::route_ws_bytes(d));
    return LBV_OK;
}

lbv_status lbv_moe_permute_workspace_size(const lbv_moe_config* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    *bytes = round_up(lbv::permute_ws_bytes(d));
    return LBV_OK;
}

lbv_status lbv_moe_w13_workspace_size(const lbv_moe_config* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    *bytes = w13_ws_bytes(d);
    return LBV_OK;
}

lbv_status lbv_moe_w2_workspace_size(const lbv_moe_config* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    *bytes = w2_ws_bytes(d);
    return LBV_OK;
}

lbv_status lbv_moe_route(const lbv_moe_config* cfg, int64_t T, const void* x,
                         const float* router_w, const float* e_bias, const uint8_t* mask,
                         int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    const size_t need = round_up(lbv::route_ws_bytes(d));
    if (!x || !router_w || !e_bias || !topk_ids || !topk_w || (need > 0 && !ws))
        return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(e_bias) || !aligned4(topk_ids) ||
        !aligned4(topk_w) || !aligned16(ws))
        return LBV_ERR_ALIGN;
    if (ws_bytes < need) return LBV_ERR_WORKSPACE;
    return hip_status(lbv::launch_route(d, x, router_w, e_bias, mask, topk_ids, topk_w, ws, stream));
}

lbv_status lbv_moe_route_noalloc(const lbv_moe_config* cfg, int64_t T, const void* x,
                                 const float* router_w, const float* e_bias, const uint8_t* mask,
                                 int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!x || !router_w || !e_bias || !topk_ids || !topk_w) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(e_bias) || !aligned4(topk_ids) ||
        !aligned4(topk_w))
        return LBV_ERR_ALIGN;
    if (round_up(lbv::route_ws_bytes(d)) > lbv::kRouteScratchBytes) return LBV_ERR_SCRATCH;
    void* scratch = nullptr;
    if (lbv::route_scratch(&scratch) != hipSuccess) return LBV_ERR_HIP;
    return hip_status(lbv::launch_route(d, x, router_w, e_bias, mask, topk_ids, topk_w, scratch,
                                        stream));
}

lbv_status lbv_moe_permute(const lbv_moe_config* cfg, int64_t T, const int32_t* topk_ids,
                           int32_t* offsets, int32_t* sorted_rows, int32_t* inv_rows,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!topk_ids || !offsets || !sorted_rows || !inv_rows || !ws) return LBV_ERR_NULL;
    if (!aligned4(topk_ids) || !aligned4(offsets) || !aligned4(sorted_rows) ||
        !aligned4(inv_rows) || !aligned16(ws))
        return LBV_ERR_ALIGN;
    if (ws_bytes < round_up(lbv::permute_ws_bytes(d))) return LBV_ERR_WORKSPACE;
    return hip_status(lbv::launch_permute(d, topk_ids, offsets, sorted_rows, inv_rows, ws, stream));
}

lbv_status lbv_moe_gemm_w13_silu(const lbv_moe_config* cfg, int64_t T, const void* x,
                                 const void* w13, const void* shared_w13,
                                 const int32_t* offsets, const int32_t* sorted_rows,
                                 void* act, void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!x || !w13 || !offsets || !sorted_rows || !act || !ws) return LBV_ERR_NULL;
    if (d.NS > 0 && !shared_w13) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(w13) || !aligned16(shared_w13) || !aligned16(act) ||
        !aligned4(offsets) || !aligned4(sorted_rows) || !aligned16(ws))
        return LBV_ERR_ALIGN;
    if (ws_bytes < w13_ws_bytes(d)) return LBV_ERR_WORKSPACE;
    return hip_status(lbv::launch_gemm_w13(d, x, w13, shared_w13, offsets, sorted_rows, act,
                                           static_cast<int*>(ws), stream));
}

lbv_status lbv_moe_gemm_w2_combine(const lbv_moe_config* cfg, int64_t T, const void* act,
                                   const void* w2, const void* shared_w2,
                                   const int32_t* offsets, const int32_t* sorted_rows,
                                   const int32_t* inv_rows, const float* topk_w, void* out,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!act || !w2 || !offsets || !sorted_rows || !inv_rows || !topk_w || !out || !ws)
        return LBV_ERR_NULL;
    if (d.NS > 0 && !shared_w2) return LBV_ERR_NULL;
    if (!aligned16(act) || !aligned16(w2) || !aligned16(shared_w2) || !aligned16(out) ||
        !aligned16(ws) || !aligned4(offsets) || !aligned4(sorted_rows) || !aligned4(inv_rows) ||
        !aligned4(topk_w))
        return LBV_ERR_ALIGN;
    if (ws_bytes < w2_ws_bytes(d)) return LBV_ERR_WORKSPACE;
    int* ctr = reinterpret_cast<int*>(static_cast<char*>(ws) + w2_y_bytes(d));
    hipError_t e = lbv::launch_gemm_w2(d, act, w2, shared_w2, offsets, sorted_rows, ws, ctr, stream);
    if (e != hipSuccess) return LBV_ERR_HIP;
    return hip_status(lbv::launch_combine(d, ws, inv_rows, topk_w, out, stream));
}

lbv_status lbv_moe_ffn_adaln_workspace_size(const lbv_moe_config* cfg, int64_t T, size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    *bytes = ffn_ws_bytes(d);
    return LBV_OK;
}

lbv_status lbv_adaln_rmsnorm(const lbv_moe_config* cfg, int64_t T, const float* x,
                             const float* temb6, int64_t temb_stride, const float* table,
                             float eps, void* h, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    st = check_adaln(d, x, temb6, temb_stride, table, eps);
    if (st != LBV_OK) return st;
    if (!h) return LBV_ERR_NULL;
    if (!aligned16(h)) return LBV_ERR_ALIGN;
    const size_t xb = static_cast<size_t>(T) * d.H * 4;
    if (overlaps(x, xb, h, static_cast<size_t>(T) * d.H * elem_bytes(d))) return LBV_ERR_ALIAS;
    lbv::AdalnArgs a{x, temb6, temb_stride, table, eps, h, T, d.H, stream};
    return hip_status(lbv::launch_adaln(d, a));
}

lbv_status lbv_moe_ffn_adaln(const lbv_moe_config* cfg, int64_t T, const float* x,
                             const uint8_t* mask, const float* temb6, int64_t temb_stride,
                             const float* table, float eps, const float* router_w,
                             const float* e_bias, const void* w13, const void* w2,
                             const void* shared_w13, const void* shared_w2, float* out,
                             int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    st = check_adaln(d, x, temb6, temb_stride, table, eps);
    if (st != LBV_OK) return st;
    if (!router_w || !e_bias || !w13 || !w2 || !out || !ws) return LBV_ERR_NULL;
    if (d.NS > 0 && (!shared_w13 || !shared_w2)) return LBV_ERR_NULL;
    if (!aligned16(router_w) || !aligned4(e_bias) || !aligned16(w13) || !aligned16(w2) ||
        !aligned16(shared_w13) || !aligned16(shared_w2) || !aligned16(out) || !aligned16(ws) ||
        !aligned4(topk_ids_out) || !aligned4(topk_w_out))
        return LBV_ERR_ALIGN;
    const size_t xb = static_cast<size_t>(T) * d.H * 4;
    // in place (out == x) is allowed: each element is read, then written, by one lane
    if (out != x && overlaps(x, xb, out, xb)) return LBV_ERR_ALIAS;
    if (ws_bytes < ffn_ws_bytes(d)) return LBV_ERR_WORKSPACE;
    if (overlaps(ws, ws_bytes, out, xb) || overlaps(ws, ws_bytes, x, xb)) return LBV_ERR_ALIAS;

    const FwdLayout L = fwd_layout(d);
    char* base = static_cast<char*>(ws);
    int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
    float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
    int* ctr1 = reinterpret_cast<int*>(base + L.ctr1);
    int* ctr2 = reinterpret_cast<int*>(base + L.ctr2);
    void* h = base + ffn_h_offset(d);

    lbv::AdalnArgs a{x, temb6, temb_stride, table, eps, h, T, d.H, stream};
    hipError_t e = lbv::launch_adaln(d, a);
    if (e == hipSuccess) e = lbv::launch_route(d, h, router_w, e_bias, mask, ids, w, base + L.route, stream);
    // the permutation's scan zeroes both matmuls' tile queue counters
    if (e == hipSuccess)
        e = lbv::launch_permute(d, ids, offsets, sorted, inv, base + L.perm, stream, ctr1, ctr2);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w13(d, h, w13, shared_w13, offsets, sorted, base + L.act, ctr1, stream,
                                 nullptr, nullptr, false);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w2(d, base + L.act, w2, shared_w2, offsets, sorted, base + L.y, ctr2,
                                stream, nullptr, nullptr, false);
    if (e == hipSuccess)
        e = lbv::launch_combine_residual(d, base + L.y, inv, w, x, temb6, temb_stride, table, out, stream);
    return hip_status(e);
}

lbv_status lbv_quantize_fp8_rows(const void* w, int32_t dtype, int64_t rows, int64_t cols,
                                 uint8_t* q, float* scale, hipStream_t stream) {
    if (dtype != LBV_BF16 && dtype != LBV_F32) return LBV_ERR_UNSUPPORTED;
    if (rows < 0 || cols <= 0 || cols % 16 != 0 || cols > (1 << 30)) return LBV_ERR_SHAPE;
    // one wave per row, four rows per workgroup: the grid stays below 2^30
    if (rows >= (int64_t(1) << 32) || rows > (int64_t(1) << 40) / cols) return LBV_ERR_SHAPE;
    if (rows == 0) return LBV_OK;
    if (!w || !q || !scale) return LBV_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned4(scale)) return LBV_ERR_ALIGN;
    const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(cols);
    const size_t wb = n * (dtype == LBV_BF16 ? 2 : 4);
    if (overlaps(w, wb, q, n) || overlaps(w, wb, scale, static_cast<size_t>(rows) * 4) ||
        overlaps(q, n, scale, static_cast<size_t>(rows) * 4))
        return LBV_ERR_ALIAS;
    return hip_status(lbv::launch_quantize_fp8(w, dtype == LBV_BF16, rows, static_cast<int>(cols),
                                               q, scale, stream));
}

lbv_status lbv_moe_forward_fp8(const lbv_moe_config* cfg, int64_t T, const void* x,
                               const uint8_t* mask, const float* router_w, const float* e_bias,
                               const lbv_moe_fp8_weights* wq, void* out, int32_t* topk_ids_out,
                               float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (!d.bf16) return LBV_ERR_UNSUPPORTED;
    if (T == 0) return LBV_OK;
    if (!wq) return LBV_ERR_NULL;
    if (!x || !router_w || !e_bias || !wq->w13 || !wq->w13_scale || !wq->w2 || !wq->w2_scale ||
        !out || !ws)
        return LBV_ERR_NULL;
    if (d.NS > 0 && (!wq->shared_w13 || !wq->shared_w13_scale || !wq->shared_w2 ||
                     !wq->shared_w2_scale))
        return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(e_bias) || !aligned16(wq->w13) ||
        !aligned16(wq->w2) || !aligned16(wq->shared_w13) || !aligned16(wq->shared_w2) ||
        !aligned4(wq->w13_scale) || !aligned4(wq->w2_scale) || !aligned4(wq->shared_w13_scale) ||
        !aligned4(wq->shared_w2_scale) || !aligned16(out) || !aligned16(ws) ||
        !aligned4(topk_ids_out) || !aligned4(topk_w_out))
        return LBV_ERR_ALIGN;
    const size_t xbytes = static_cast<size_t>(T) * d.H * elem_bytes(d);
    if (overlaps(x, xbytes, out, xbytes)) return LBV_ERR_ALIAS;
    const FwdLayout L = fwd_layout(d);
    if (ws_bytes < L.total) return LBV_ERR_WORKSPACE;

    char* base = static_cast<char*>(ws);
    int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
    float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
    void* act = base + L.act;
    void* y = base + L.y;
    int* ctr1 = reinterpret_cast<int*>(base + L.ctr1);
    int* ctr2 = reinterpret_cast<int*>(base + L.ctr2);

    hipError_t e = lbv::launch_route(d, x, router_w, e_bias, mask, ids, w, base + L.route, stream);
    // the permutation's scan zeroes both matmuls' tile queue counters
    if (e == hipSuccess)
        e = lbv::launch_permute(d, ids, offsets, sorted, inv, base + L.perm, stream, ctr1, ctr2);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w13(d, x, wq->w13, wq->shared_w13, offsets, sorted, act, ctr1, stream,
                                 wq->w13_scale, wq->shared_w13_scale, false);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w2(d, act, wq->w2, wq->shared_w2, offsets, sorted, y, ctr2, stream,
                                wq->w2_scale, wq->shared_w2_scale, false);
    if (e == hipSuccess) e = lbv::launch_combine(d, y, inv, w, out, stream);
    return hip_status(e);
}

lbv_status lbv_moe_forward_w8a8(const lbv_moe_config* cfg, int64_t T, const void* x,
                                const uint8_t* mask, const float* router_w, const float* e_bias,
                                const lbv_moe_fp8_weights* wq, void* out, int32_t* topk_ids_out,
                                float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (!d.bf16) return LBV_ERR_UNSUPPORTED;
    // k-tiles of 128 values; act's block scales take kA8ScalePitch bytes per row
    if (d.H % 128 != 0 || d.I % 128 != 0 || d.I > 32 * lbv::kA8ScalePitch) return LBV_ERR_SHAPE;
    if (T == 0) return LBV_OK;
    if (!wq) return LBV_ERR_NULL;
    if (!x || !router_w || !e_bias || !wq->w13 || !wq->w13_scale || !wq->w2 || !wq->w2_scale ||
        !out || !ws)
        return LBV_ERR_NULL;
    if (d.NS > 0 && (!wq->shared_w13 || !wq->shared_w13_scale || !wq->shared_w2 ||
                     !wq->shared_w2_scale))
        return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(e_bias) || !aligned16(wq->w13) ||
        !aligned16(wq->w2) || !aligned16(wq->shared_w13) || !aligned16(wq->shared_w2) ||
        !aligned4(wq->w13_scale) || !aligned4(wq->w2_scale) || !aligned4(wq->shared_w13_scale) ||
        !aligned4(wq->shared_w2_scale) || !aligned16(out) || !aligned16(ws) ||
        !aligned4(topk_ids_out) || !aligned4(topk_w_out))
        return LBV_ERR_ALIGN;
    const size_t xbytes = static_cast<size_t>(T) * d.H * 2;
    if (overlaps(x, xbytes, out, xbytes)) return LBV_ERR_ALIAS;
    const FwdLayout L = fwd_layout(d);
    if (ws_bytes < L.total) return LBV_ERR_WORKSPACE;

    char* base = static_cast<char*>(ws);
    int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
    float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
    int* ctr1 = reinterpret_cast<int*>(base + L.ctr1);
    int* ctr2 = reinterpret_cast<int*>(base + L.ctr2);
    // fp8 act [R, I] and its block scales [R, kA8ScalePitch] in the bf16 act
    // region (R I + 32 R <= 2 R I bytes as I >= 128); fp8 x [T, H] and its
    // scales [T] in the y region, which the down matmul fills only after the
    // gate/up matmul has read them (R (K + ns) H 2 >= T H + 4 T bytes)
    const size_t R = static_cast<size_t>(T) * d.KS;
    uint8_t* actq = reinterpret_cast<uint8_t*>(base + L.act);
    uint8_t* act_scales = actq + R * d.I;
    uint8_t* xq = reinterpret_cast<uint8_t*>(base + L.y);
    float* xs = reinterpret_cast<float*>(xq + static_cast<size_t>(T) * d.H);
    void* y = base + L.y;

    hipError_t e = lbv::launch_route(d, x, router_w, e_bias, mask, ids, w, base + L.route, stream);
    // the permutation's scan zeroes both matmuls' tile queue counters
    if (e == hipSuccess)
        e = lbv::launch_permute(d, ids, offsets, sorted, inv, base + L.perm, stream, ctr1, ctr2);
    if (e == hipSuccess) e = lbv::launch_quantize_fp8(x, 1, T, d.H, xq, xs, stream);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w13_a8(d, xq, xs, wq->w13, wq->w13_scale, wq->shared_w13,
                                    wq->shared_w13_scale, offsets, sorted, actq, act_scales, ctr1,
                                    stream);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w2_a8(d, actq, act_scales, wq->w2, wq->w2_scale, wq->shared_w2,
                                   wq->shared_w2_scale, offsets, sorted, y, ctr2, stream);
    if (e == hipSuccess) e = lbv::launch_combine(d, y, inv, w, out, stream);
    return hip_status(e);
}

lbv_status lbv_moe_forward(const lbv_moe_config* cfg, int64_t T, const void* x,
                           const uint8_t* mask, const float* router_w, const float* e_bias,
                           const void* w13, const void* w2, const void* shared_w13,
                           const void* shared_w2, void* out, int32_t* topk_ids_out,
                           float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!x || !router_w || !e_bias || !w13 || !w2 || !out || !ws) return LBV_ERR_NULL;
    if (d.NS > 0 && (!shared_w13 || !shared_w2)) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(e_bias) || !aligned16(w13) ||
        !aligned16(w2) || !aligned16(shared_w13) || !aligned16(shared_w2) || !aligned16(out) ||
        !aligned16(ws) || !aligned4(topk_ids_out) || !aligned4(topk_w_out))
        return LBV_ERR_ALIGN;
    const size_t xbytes = static_cast<size_t>(T) * d.H * elem_bytes(d);
    if (overlaps(x, xbytes, out, xbytes)) return LBV_ERR_ALIAS;
    const FwdLayout L = fwd_layout(d);
    if (ws_bytes < L.total) return LBV_ERR_WORKSPACE;

    char* base = static_cast<char*>(ws);
    int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
    float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
    int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
    void* perm = base + L.perm;
    void* rws = base + L.route;
    void* act = base + L.act;
    void* y = base + L.y;
    int* ctr1 = reinterpret_cast<int*>(base + L.ctr1);
    int* ctr2 = reinterpret_cast<int*>(base + L.ctr2);

    hipError_t e = lbv::launch_route(d, x, router_w, e_bias, mask, ids, w, rws, stream);
    // the permutation's scan zeroes both matmuls' tile queue counters
    if (e == hipSuccess) e = lbv::launch_permute(d, ids, offsets, sorted, inv, perm, stream, ctr1, ctr2);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w13(d, x, w13, shared_w13, offsets, sorted, act, ctr1, stream, nullptr,
                                 nullptr, false);
    if (e == hipSuccess)
        e = lbv::launch_gemm_w2(d, act, w2, shared_w2, offsets, sorted, y, ctr2, stream, nullptr,
                                nullptr, false);
    if (e == hipSuccess) e = lbv::launch_combine(d, y, inv, w, out, stream);
    return hip_status(e);
}

}  // extern "C"

// ---- attention half ----------------------------------------------------------

namespace {

constexpr int kHeadDim = 128;

lbv_status check_attn(const lbv_attn_config* c, int64_t B, int64_t S) {
    if (!c) return LBV_ERR_NULL;
    if (c->num_heads <= 0 || c->hidden != c->num_heads * kHeadDim) return LBV_ERR_UNSUPPORTED;
    if (!(c->eps >= 0.0f) || !isfinite(c->eps)) return LBV_ERR_SHAPE;
    if (B < 0 || S < 0 || S > 65536) return LBV_ERR_SHAPE;
    const int64_t T = B * S;
    if (B > 0 && S > 0 && (T >= (1 << 24) || T * 3 * c->hidden * 2 >= (1ll << 32) ||
                           int64_t(c->hidden) * 3 * c->hidden * 2 >= (1ll << 32)))
        return LBV_ERR_SHAPE;
    return LBV_OK;
}

struct AttnLayout {
    size_t lin, qkv, q, k, vt, o, total;
};

AttnLayout attn_layout(const lbv_attn_config* c, int64_t B, int64_t S) {
    AttnLayout L;
    const size_t T = static_cast<size_t>(B * S), H = static_cast<size_t>(c->hidden);
    size_t off = 0;
    L.lin = off; off += round_up(lbv::kLinearWsBytes);
    L.qkv = off; off += round_up(T * 3 * H * 2);
    L.q = off;   off += round_up(T * H * 2);
    L.k = off;   off += round_up(T * H * 2);
    L.vt = off;  off += round_up(static_cast<size_t>(B) * H * lbv::attn_sp(static_cast<int>(S)) * 2);
    L.o = off;   off += round_up(T * H * 2);
    L.total = off;
    return L;
}

}  // namespace

extern "C" {

lbv_status lbv_attn_workspace_size(const lbv_attn_config* cfg, int64_t B, int64_t S,
                                   size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    *bytes = attn_layout(cfg, B, S).total;
    return LBV_OK;
}

lbv_status lbv_linear_bf16(int64_t T, int32_t N, int32_t K, const void* x, const void* w,
                           const float* bias, void* y, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    if (T < 0 || N <= 0 || K <= 0 || N % 64 != 0 || K % 64 != 0) return LBV_ERR_SHAPE;
    if (T >= (1 << 24) || T * K * 2 >= (1ll << 32) || int64_t(N) * K * 2 >= (1ll << 32) ||
        N >= (1 << 24) || K >= (1 << 24))
        return LBV_ERR_SHAPE;
    if (T == 0) return LBV_OK;
    if (!x || !w || !y || !ws) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || !aligned16(ws) || !aligned4(bias))
        return LBV_ERR_ALIGN;
    if (ws_bytes < lbv::kLinearWsBytes) return LBV_ERR_WORKSPACE;
    const size_t xb = static_cast<size_t>(T) * K * 2, yb = static_cast<size_t>(T) * N * 2;
    if (overlaps(x, xb, y, yb) || overlaps(w, static_cast<size_t>(N) * K * 2, y, yb) ||
        overlaps(ws, lbv::kLinearWsBytes, y, yb))
        return LBV_ERR_ALIAS;
    return hip_status(lbv::launch_linear(T, N, K, x, w, bias, y, ws, stream));
}

lbv_status lbv_attn_qk_prep(const lbv_attn_config* cfg, int64_t B, int64_t S, const void* qkv,
                            const float* g_q, const float* g_k, const float* cos_t,
                            const float* sin_t, void* q, void* k, void* vt, hipStream_t stream) {
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    if (B == 0 || S == 0) return LBV_OK;
    if (!qkv || !g_q || !g_k || !cos_t || !sin_t || !q || !k || !vt) return LBV_ERR_NULL;
    if (!aligned16(qkv) || !aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned4(g_q) ||
        !aligned4(g_k) || !aligned4(cos_t) || !aligned4(sin_t))
        return LBV_ERR_ALIGN;
    return hip_status(lbv::launch_attn_prep(static_cast<int>(B), static_cast<int>(S), cfg->hidden,
                                            cfg->num_heads, qkv, g_q, g_k, cos_t, sin_t, cfg->eps,
                                            q, k, vt, stream));
}

lbv_status lbv_attn_core(const lbv_attn_config* cfg, int64_t B, int64_t S, const void* q,
                         const void* k, const void* vt, const uint8_t* mask, void* o,
                         hipStream_t stream) {
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    if (B == 0 || S == 0) return LBV_OK;
    if (!q || !k || !vt || !o) return LBV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(o)) return LBV_ERR_ALIGN;
    return hip_status(lbv::launch_attn_core(static_cast<int>(B), static_cast<int>(S), cfg->hidden,
                                            cfg->num_heads, q, k, vt, mask, o, stream));
}

lbv_status lbv_attn_half_adaln_workspace_size(const lbv_attn_config* cfg, int64_t B, int64_t S,
                                              size_t* bytes) {
    if (!bytes) return LBV_ERR_NULL;
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    const size_t hb = round_up(static_cast<size_t>(B * S) * cfg->hidden * 2);
    *bytes = attn_layout(cfg, B, S).total + 2 * hb;
    return LBV_OK;
}

lbv_status lbv_attn_half_adaln(const lbv_attn_config* cfg, int64_t B, int64_t S, const float* x,
                               const uint8_t* mask, const float* temb6, int64_t temb_stride,
                               const float* table, float eps, const void* w_qkv,
                               const float* b_qkv, const float* g_q, const float* g_k,
                               const float* cos_t, const float* sin_t, const void* w_o,
                               const float* b_o, float* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    if (B == 0 || S == 0) return LBV_OK;
    if (!x || !temb6 || !table || !w_qkv || !g_q || !g_k || !cos_t || !sin_t || !w_o || !out ||
        !ws)
        return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(temb6) || !aligned16(table) || !aligned16(out) ||
        !aligned16(w_qkv) || !aligned16(w_o) || !aligned16(ws) || !aligned4(b_qkv) ||
        !aligned4(b_o) || !aligned4(g_q) || !aligned4(g_k) || !aligned4(cos_t) || !aligned4(sin_t))
        return LBV_ERR_ALIGN;
    if (temb_stride < 0 || temb_stride % 4 != 0) return LBV_ERR_ALIGN;
    if (!(eps >= 0.0f) || !isfinite(eps)) return LBV_ERR_SHAPE;
    const AttnLayout L = attn_layout(cfg, B, S);
    const int64_t T = B * S;
    const int H = cfg->hidden;
    const size_t hb = round_up(static_cast<size_t>(T) * H * 2);
    if (ws_bytes < L.total + 2 * hb) return LBV_ERR_WORKSPACE;
    const size_t xb = static_cast<size_t>(T) * H * 4;
    // in place (out == x) is allowed: each element is read, then written, by one lane
    if (out != x && overlaps(x, xb, out, xb)) return LBV_ERR_ALIAS;
    if (overlaps(ws, ws_bytes, out, xb) || overlaps(ws, ws_bytes, x, xb)) return LBV_ERR_ALIAS;
    char* base = static_cast<char*>(ws);
    void* h = base + L.total;
    void* blk = base + L.total + hb;
    lbv::AdalnArgs a{x, temb6, temb_stride, table, eps, h, T, H, stream};
    a.shift_row = 0;
    a.scale_row = 1;
    hipError_t e = lbv::launch_adaln_bf16(a);
    if (e == hipSuccess)
        e = lbv::launch_linear(T, 3 * H, H, h, w_qkv, b_qkv, base + L.qkv, base + L.lin, stream);
    if (e == hipSuccess)
        e = lbv::launch_attn_prep(static_cast<int>(B), static_cast<int>(S), H, cfg->num_heads,
                                  base + L.qkv, g_q, g_k, cos_t, sin_t, cfg->eps, base + L.q,
                                  base + L.k, base + L.vt, stream);
    if (e == hipSuccess)
        e = lbv::launch_attn_core(static_cast<int>(B), static_cast<int>(S), H, cfg->num_heads,
                                  base + L.q, base + L.k, base + L.vt, mask, base + L.o, stream);
    if (e == hipSuccess)
        e = lbv::launch_linear(T, H, H, base + L.o, w_o, b_o, blk, base + L.lin, stream);
    if (e == hipSuccess)
        e = lbv::launch_gated_residual(T, H, x, blk, temb6, temb_stride, table, 2, out, stream);
    return hip_status(e);
}

lbv_status lbv_attn_forward(const lbv_attn_config* cfg, int64_t B, int64_t S, const void* x,
                            const uint8_t* mask, const void* w_qkv, const float* b_qkv,
                            const float* g_q, const float* g_k, const float* cos_t,
                            const float* sin_t, const void* w_o, const float* b_o, void* out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
    lbv_status st = check_attn(cfg, B, S);
    if (st != LBV_OK) return st;
    if (B == 0 || S == 0) return LBV_OK;
    if (!x || !w_qkv || !g_q || !g_k || !cos_t || !sin_t || !w_o || !out || !ws)
        return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(w_o) || !aligned16(out) ||
        !aligned16(ws) || !aligned4(b_qkv) || !aligned4(b_o) || !aligned4(g_q) ||
        !aligned4(g_k) || !aligned4(cos_t) || !aligned4(sin_t))
        return LBV_ERR_ALIGN;
    const AttnLayout L = attn_layout(cfg, B, S);
    if (ws_bytes < L.total) return LBV_ERR_WORKSPACE;
    const int64_t T = B * S;
    const int H = cfg->hidden;
    const size_t xb = static_cast<size_t>(T) * H * 2;
    if (overlaps(x, xb, out, xb) || overlaps(ws, ws_bytes, out, xb) || overlaps(ws, ws_bytes, x, xb))
        return LBV_ERR_ALIAS;
    char* base = static_cast<char*>(ws);
    hipError_t e = lbv::launch_linear(T, 3 * H, H, x, w_qkv, b_qkv, base + L.qkv, base + L.lin,
                                      stream);
    if (e == hipSuccess)
        e = lbv::launch_attn_prep(static_cast<int>(B), static_cast<int>(S), H, cfg->num_heads,
                                  base + L.qkv, g_q, g_k, cos_t, sin_t, cfg->eps, base + L.q,
                                  base + L.k, base + L.vt, stream);
    if (e == hipSuccess)
        e = lbv::launch_attn_core(static_cast<int>(B), static_cast<int>(S), H, cfg->num_heads,
                                  base + L.q, base + L.k, base + L.vt, mask, base + L.o, stream);
    if (e == hipSuccess)
        e = lbv::launch_linear(T, H, H, base + L.o, w_o, b_o, out, base + L.lin, stream);
    return hip_status(e);
}

}  // extern "C"

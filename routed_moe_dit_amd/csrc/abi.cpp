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

constexpr int32_t kAbiVersion = 1;
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
    if (c->dtype == LBV_BF16 && (T * c->hidden * 2 >= (1ll << 32) || T >= (1 << 24))) return LBV_ERR_SHAPE;
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
    size_t ids, w, offsets, sorted, inv, perm, route, act, y, total;
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
    L.act = off;     off += round_up(T * d.KS * d.I * elem_bytes(d));
    L.y = off;       off += round_up(T * d.KS * d.H * elem_bytes(d));
    L.total = off;
    return L;
}

size_t w2_ws_bytes(const Dims& d) {
    return round_up(static_cast<size_t>(d.T) * d.KS * d.H * elem_bytes(d));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

lbv_status hip_status(hipError_t e) { return e == hipSuccess ? LBV_OK : LBV_ERR_HIP; }

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
                                 void* act, hipStream_t stream) {
    Dims d;
    lbv_status st = make_dims(cfg, T, &d);
    if (st != LBV_OK) return st;
    if (T == 0) return LBV_OK;
    if (!x || !w13 || !offsets || !sorted_rows || !act) return LBV_ERR_NULL;
    if (d.NS > 0 && !shared_w13) return LBV_ERR_NULL;
    if (!aligned16(x) || !aligned16(w13) || !aligned16(shared_w13) || !aligned16(act) ||
        !aligned4(offsets) || !aligned4(sorted_rows))
        return LBV_ERR_ALIGN;
    return hip_status(lbv::launch_gemm_w13(d, x, w13, shared_w13, offsets, sorted_rows, act, stream));
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
    hipError_t e = lbv::launch_gemm_w2(d, act, w2, shared_w2, offsets, sorted_rows, ws, stream);
    if (e != hipSuccess) return LBV_ERR_HIP;
    return hip_status(lbv::launch_combine(d, ws, inv_rows, topk_w, out, stream));
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

    hipError_t e = lbv::launch_route(d, x, router_w, e_bias, mask, ids, w, rws, stream);
    if (e == hipSuccess) e = lbv::launch_permute(d, ids, offsets, sorted, inv, perm, stream);
    if (e == hipSuccess) e = lbv::launch_gemm_w13(d, x, w13, shared_w13, offsets, sorted, act, stream);
    if (e == hipSuccess) e = lbv::launch_gemm_w2(d, act, w2, shared_w2, offsets, sorted, y, stream);
    if (e == hipSuccess) e = lbv::launch_combine(d, y, inv, w, out, stream);
    return hip_status(e);
}

}  // extern "C"

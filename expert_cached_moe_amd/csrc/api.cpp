// libmoecache: context, validation, expert blob packing, pool binding, fills and
// the dispatch of the GPU entry points.  The declarations and their contracts are
// in include/moe.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <functional>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace moe {

int fail(moe_ctx* ctx, int code, const std::string& msg) {
    if (ctx) ctx->err = msg;
    return code;
}

int hip_fail(moe_ctx* ctx, hipError_t e, const char* what) {
    return fail(ctx, MOE_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int validate_config(const moe_config* c, std::string* why) {
    auto bad = [&](int code, const char* m) { if (why) *why = m; return code; };
    if (!c) return bad(MOE_EINVAL, "null config");
    if (c->hidden <= 0 || c->hidden % 64) return bad(MOE_ESHAPE, "hidden must be a positive multiple of 64");
    if (c->w_dtype == MOE_W_MXFP4 && c->hidden % 256)
        return bad(MOE_ESHAPE, "hidden must be a multiple of 256 for MXFP4 weights");
    if (c->inter <= 0 || c->inter % 32) return bad(MOE_ESHAPE, "inter must be a positive multiple of 32");
    if (c->n_experts < 1 || c->n_experts > kMaxExperts) return bad(MOE_ESHAPE, "n_experts must be in 1..512");
    if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > kMaxTopK)
        return bad(MOE_ESHAPE, "top_k must be in 1..min(n_experts, 16)");
    if (c->n_shared != 0 && c->n_shared != 1) return bad(MOE_ESHAPE, "n_shared must be 0 or 1");
    if (c->n_slots < 0 || c->n_slots > (1 << 21)) return bad(MOE_ESHAPE, "n_slots out of range");
    if (c->n_layers < 1 || int64_t(c->n_layers) * c->n_experts > (1 << 24))
        return bad(MOE_ESHAPE, "n_layers out of range");
    if (c->w_dtype != MOE_W_F32 && c->w_dtype != MOE_W_BF16 && c->w_dtype != MOE_W_MXFP4)
        return bad(MOE_EUNSUPPORTED, "unknown weight dtype");
    if (c->renormalize != 0 && c->renormalize != 1) return bad(MOE_EINVAL, "renormalize must be 0 or 1");
    if (c->q_round != MOE_Q_NEAREST && c->q_round != MOE_Q_ARGMIN) return bad(MOE_EINVAL, "unknown q_round");
    if (!(c->bp_gbps > 0) || !(c->bh_gbps > 0) || !std::isfinite(c->bp_gbps) || !std::isfinite(c->bh_gbps))
        return bad(MOE_EINVAL, "bandwidths must be positive and finite");
    return MOE_OK;
}

BlobLayout blob_layout(const moe_config& c) {
    BlobLayout L;
    const int64_t H = c.hidden, I = c.inter;
    if (c.w_dtype == MOE_W_MXFP4) {
        L.gu = 0;
        L.gu_scale = align256(2 * I * H / 2);
        L.d = align256(L.gu_scale + 2 * I * H / 32);
        L.d_scale = align256(L.d + H * I / 2);
        L.bytes = align256(L.d_scale + H * I / 32);
    } else {
        const int64_t es = c.w_dtype == MOE_W_F32 ? 4 : 2;
        L.gu = 0;
        L.d = align256(2 * I * H * es);
        L.bytes = align256(L.d + H * I * es);
        L.gu_scale = L.d_scale = 0;
    }
    return L;
}

WsLayout ws_layout(const moe_config& c, int32_t max_T) {
    WsLayout W;
    const int64_t T = max_T < 1 ? 1 : max_T;
    const int64_t pairs = T * c.top_k;
    const int64_t chunks = (pairs + kPermChunk - 1) / kPermChunk;
    const int64_t rows = pairs + (c.n_shared ? T : 0);
    W.hist = 0;
    W.base = align256(W.hist + chunks * c.n_experts * 4);
    W.tiles = align256(W.base + chunks * c.n_experts * 4);
    W.h = align256(W.tiles + gemm_tile_ints(c, int32_t(T)) * 4);
    // pair outputs of moe_expert_ffn_merge when it does not fuse (decode batches only)
    const int64_t Td = T < kDecodeMaxT ? T : kDecodeMaxT;
    const int64_t rows_d = Td * c.top_k + (c.n_shared ? Td : 0);
    W.o = align256(W.h + rows * int64_t(c.inter) * act_bytes(c));
    W.bytes = align256(W.o + rows_d * int64_t(c.hidden) * act_bytes(c));
    return W;
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_EINVAL: return "MOE_EINVAL";
        case MOE_ESHAPE: return "MOE_ESHAPE";
        case MOE_ECAPACITY: return "MOE_ECAPACITY";
        case MOE_EHIP: return "MOE_EHIP";
        case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED";
        case MOE_ESTATE: return "MOE_ESTATE";
        default: return "MOE_UNKNOWN";
    }
}

int moe_create(const moe_config* cfg, moe_ctx** out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    int st = validate_config(cfg, nullptr);
    if (st != MOE_OK) return st;
    moe_ctx* ctx = new (std::nothrow) moe_ctx();
    if (!ctx) return MOE_EINVAL;
    try {
        ctx->cfg = *cfg;
        ctx->lay = blob_layout(*cfg);
        const int64_t keys = int64_t(cfg->n_layers) * cfg->n_experts;
        ctx->key_of_slot.assign(cfg->n_slots, -1);
        ctx->recency.assign(cfg->n_slots, 0);
        ctx->slot_of_key.assign(keys, -1);
        ctx->in_step.assign(keys, 0);
        ctx->count_scratch.assign(cfg->n_experts, 0);
    } catch (...) {
        delete ctx;
        return MOE_EINVAL;
    }
    *out = ctx;
    return MOE_OK;
}

void moe_destroy(moe_ctx* ctx) {
    if (!ctx) return;
    if (ctx->fill_event) (void)hipEventDestroy(ctx->fill_event);
    for (hipEvent_t ev : ctx->stream_ev)
        if (ev) (void)hipEventDestroy(ev);
    delete ctx;
}

const char* moe_last_error(const moe_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

int64_t moe_expert_bytes(const moe_config* cfg) {
    int st = validate_config(cfg, nullptr);
    return st != MOE_OK ? st : blob_layout(*cfg).bytes;
}

int64_t moe_workspace_bytes(const moe_config* cfg, int32_t max_T) {
    int st = validate_config(cfg, nullptr);
    if (st != MOE_OK) return st;
    if (max_T < 0) return MOE_EINVAL;
    return ws_layout(*cfg, max_T).bytes;
}

int64_t moe_pair_rows(const moe_config* cfg, int32_t T) {
    int st = validate_config(cfg, nullptr);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_EINVAL;
    return int64_t(T) * cfg->top_k + (cfg->n_shared ? T : 0);
}

int moe_pack_expert(const moe_config* cfg, const void* wg, const void* wu, const void* wd, const uint8_t* sg,
                    const uint8_t* su, const uint8_t* sd, void* blob) {
    int st = validate_config(cfg, nullptr);
    if (st != MOE_OK) return st;
    if (!wg || !wu || !wd || !blob) return MOE_EINVAL;
    const BlobLayout L = blob_layout(*cfg);
    const int64_t H = cfg->hidden, I = cfg->inter;
    uint8_t* out = static_cast<uint8_t*>(blob);
    if (cfg->w_dtype == MOE_W_MXFP4) {
        if (!sg || !su || !sd) return MOE_EINVAL;
        for (int64_t i = 0; i < I * H / 32; ++i)
            if (sg[i] == 0xFF || su[i] == 0xFF) return MOE_EINVAL;
        for (int64_t i = 0; i < H * I / 32; ++i)
            if (sd[i] == 0xFF) return MOE_EINVAL;
        std::memset(out, 0, L.bytes);
        const int64_t cb = H / 2, sb = H / 32;  // bytes per Wgu row: codes, scales
        for (int64_t r = 0; r < 2 * I; ++r) {
            const int64_t blk = r / 32, w = r % 32;
            const bool up = w >= 16;
            const int64_t src = blk * 16 + (up ? w - 16 : w);
            std::memcpy(out + L.gu + r * cb, static_cast<const uint8_t*>(up ? wu : wg) + src * cb, cb);
            std::memcpy(out + L.gu_scale + r * sb, (up ? su : sg) + src * sb, sb);
        }
        std::memcpy(out + L.d, wd, H * I / 2);
        std::memcpy(out + L.d_scale, sd, H * I / 32);
        return MOE_OK;
    }
    if (sg || su || sd) return MOE_EINVAL;
    std::memset(out, 0, L.bytes);
    const int64_t es = cfg->w_dtype == MOE_W_F32 ? 4 : 2;
    const int64_t rb = H * es;
    for (int64_t r = 0; r < 2 * I; ++r) {
        const int64_t blk = r / 32, w = r % 32;
        const bool up = w >= 16;
        const int64_t src = blk * 16 + (up ? w - 16 : w);
        std::memcpy(out + L.gu + r * rb, static_cast<const uint8_t*>(up ? wu : wg) + src * rb, rb);
    }
    std::memcpy(out + L.d, wd, H * I * es);
    return MOE_OK;
}

int moe_bind_pools(moe_ctx* ctx, void* d_slots, int32_t n_slots, const void* h_pool, int32_t n_pool) {
    if (!ctx) return MOE_EINVAL;
    if (n_slots < 0 || n_slots > ctx->cfg.n_slots || (n_slots > 0 && !d_slots))
        return fail(ctx, MOE_EINVAL, "n_slots must be in 0..cfg.n_slots with a device pool");
    const int64_t keys = int64_t(ctx->cfg.n_layers) * ctx->cfg.n_experts;
    if (h_pool && n_pool != keys) return fail(ctx, MOE_EINVAL, "host pool must hold n_layers*E blobs");
    ctx->d_slots = d_slots;
    ctx->n_bound_slots = n_slots;
    ctx->h_pool = h_pool;
    ctx->n_pool = h_pool ? n_pool : 0;
    return MOE_OK;
}

int moe_router_logits(moe_ctx* ctx, const void* d_x, int32_t T, const float* d_wr, float* d_logits, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (T == 0) return MOE_OK;
    if (!d_x || !d_wr || !d_logits) return fail(ctx, MOE_EINVAL, "null router buffer");
    hipError_t e = launch_router_logits(ctx->cfg, d_x, T, d_wr, d_logits, s);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_router_logits launch");
}

int moe_route(moe_ctx* ctx, const float* d_logits, int32_t T, int32_t* d_topk_ids, float* d_topk_w,
              int32_t* d_counts, int32_t* d_offsets, int32_t* d_perm, int32_t* d_inv, void* d_ws,
              hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (!d_counts || !d_offsets) return fail(ctx, MOE_EINVAL, "null counts/offsets");
    if (T > 0 && (!d_logits || !d_topk_ids || !d_topk_w || !d_perm || !d_inv))
        return fail(ctx, MOE_EINVAL, "null route buffer");
    if (int64_t(T) * ctx->cfg.top_k > kSmallRouteMaxPairs && !d_ws)
        return fail(ctx, MOE_EINVAL, "workspace required for this T");
    hipError_t e = launch_route(ctx->cfg, d_logits, T, d_topk_ids, d_topk_w, d_counts, d_offsets, d_perm,
                                d_inv, d_ws, s);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_route launch");
}

int moe_fill(moe_ctx* ctx, const moe_plan* plan, hipStream_t side) {
    if (!ctx || !plan) return MOE_EINVAL;
    if (plan->n_fill > 0 && (!ctx->d_slots || !ctx->h_pool))
        return fail(ctx, MOE_ESTATE, "moe_fill needs bound device slots and host pool");
    if (plan->n_fill < 0 || (plan->n_fill > 0 && (!plan->fill || !plan->fill_slot)))
        return fail(ctx, MOE_EINVAL, "bad plan");
    const int64_t bytes = ctx->lay.bytes;
    for (int i = 0; i < plan->n_fill; ++i) {
        const int64_t key = int64_t(plan->layer) * ctx->cfg.n_experts + plan->fill[i];
        if (plan->fill[i] < 0 || plan->fill[i] >= ctx->cfg.n_experts || key >= ctx->n_pool ||
            plan->fill_slot[i] < 0 || plan->fill_slot[i] >= ctx->n_bound_slots)
            return fail(ctx, MOE_EINVAL, "fill expert/slot out of range");
    }
    if (!ctx->fill_event) {
        hipError_t e = hipEventCreateWithFlags(&ctx->fill_event, hipEventDisableTiming);
        if (e != hipSuccess) { ctx->fill_event = nullptr; return hip_fail(ctx, e, "hipEventCreateWithFlags"); }
    }
    for (int i = 0; i < plan->n_fill; ++i) {
        const int64_t key = int64_t(plan->layer) * ctx->cfg.n_experts + plan->fill[i];
        const uint8_t* src = static_cast<const uint8_t*>(ctx->h_pool) + key * bytes;
        uint8_t* dst = static_cast<uint8_t*>(ctx->d_slots) + int64_t(plan->fill_slot[i]) * bytes;
        hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, side);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync (fill)");
    }
    hipError_t e = hipEventRecord(ctx->fill_event, side);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "hipEventRecord (fill)");
}

int moe_upload(moe_ctx* ctx, void* d_dst, const void* h_src, int64_t bytes, hipStream_t side) {
    if (!ctx) return MOE_EINVAL;
    if (bytes < 0 || (bytes > 0 && (!d_dst || !h_src))) return fail(ctx, MOE_EINVAL, "bad upload");
    if (!ctx->fill_event) {
        hipError_t e = hipEventCreateWithFlags(&ctx->fill_event, hipEventDisableTiming);
        if (e != hipSuccess) { ctx->fill_event = nullptr; return hip_fail(ctx, e, "hipEventCreateWithFlags"); }
    }
    if (bytes > 0) {
        hipError_t e = hipMemcpyAsync(d_dst, h_src, bytes, hipMemcpyHostToDevice, side);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync (upload)");
    }
    hipError_t e = hipEventRecord(ctx->fill_event, side);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "hipEventRecord (upload)");
}

int moe_move_slots(moe_ctx* ctx, const moe_resize* r, hipStream_t s) {
    if (!ctx || !r) return MOE_EINVAL;
    if (r->n_move < 0 || (r->n_move > 0 && (!r->move_src || !r->move_dst))) return fail(ctx, MOE_EINVAL, "bad resize");
    if (r->n_move > 0 && !ctx->d_slots) return fail(ctx, MOE_ESTATE, "moe_move_slots needs a bound device pool");
    for (int i = 0; i < r->n_move; ++i)
        if (r->move_src[i] < 0 || r->move_src[i] >= ctx->n_bound_slots || r->move_dst[i] < 0 ||
            r->move_dst[i] >= ctx->n_bound_slots || r->move_src[i] == r->move_dst[i])
            return fail(ctx, MOE_EINVAL, "move outside the bound device pool");
    const int64_t bytes = ctx->lay.bytes;
    uint8_t* base = static_cast<uint8_t*>(ctx->d_slots);
    for (int i = 0; i < r->n_move; ++i) {
        hipError_t e = hipMemcpyAsync(base + int64_t(r->move_dst[i]) * bytes, base + int64_t(r->move_src[i]) * bytes,
                                      bytes, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync (slot move)");
    }
    return MOE_OK;
}

int moe_fill_wait(moe_ctx* ctx, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    if (!ctx->fill_event) return MOE_OK;  // nothing was ever filled
    hipError_t e = hipStreamWaitEvent(s, ctx->fill_event, 0);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "hipStreamWaitEvent");
}

// Decode expert list from the host's copy of the top-k ids: per listed expert that some
// token of the step uses, its tokens (bit t) and each token's slot j among its k picks; the
// shared expert (last) takes all.  Listed experts without a token produce no pair and are
// left out, so the list holds at most T*k routed entries plus the shared one
// (kMaxDecodeList), however many experts the caller lists.  where[e] = index of expert e in
// h_experts or -1.
static int build_decode_list(moe_ctx* ctx, int32_t T, const int32_t* h_topk_ids, const int32_t* h_experts,
                             const int32_t* h_slots, int32_t with_shared, const std::vector<int32_t>& where,
                             DecodeList* dl) {
    const moe_config& c = ctx->cfg;
    if (T < 1 || T > kDecodeMaxT) return fail(ctx, MOE_ESHAPE, "decode list needs 1 <= T <= 8");
    // list position of each listed expert with tokens, in first-use order (t, j)
    std::vector<int32_t> pos(c.n_experts, -1);
    dl->n = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < c.top_k; ++j) {
            const int id = h_topk_ids[t * c.top_k + j];
            if (id < 0 || id >= c.n_experts) return fail(ctx, MOE_EINVAL, "top-k id out of range");
            for (int jj = 0; jj < j; ++jj)
                if (h_topk_ids[t * c.top_k + jj] == id) return fail(ctx, MOE_EINVAL, "repeated expert in a token");
            const int i = where[id];
            if (i < 0) continue;
            if (pos[id] < 0) {
                if (dl->n >= kMaxDecodeList - 1) return fail(ctx, MOE_ESHAPE, "decode list overflow");
                pos[id] = dl->n++;
                dl->ent[pos[id]] = h_experts[i] | (h_slots[i] << 10);
                dl->tokmask[pos[id]] = 0;
                dl->jpack[pos[id]] = 0;
            }
            dl->tokmask[pos[id]] |= 1u << t;
            dl->jpack[pos[id]] |= uint32_t(j) << (4 * t);
        }
    if (with_shared) {
        const int n = dl->n++;
        dl->ent[n] = kSharedTag;
        dl->tokmask[n] = (1u << T) - 1u;
        dl->jpack[n] = 0;
    }
    return MOE_OK;
}

int moe_expert_ffn(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids, const int32_t* d_offsets,
                   const int32_t* d_perm, const void* d_slot_base, const int32_t* h_experts, const int32_t* h_slots,
                   int32_t n, const void* d_shared, int32_t with_shared, void* d_o, void* d_ws, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    const moe_config& c = ctx->cfg;
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (n < 0 || n > c.n_experts) return fail(ctx, MOE_EINVAL, "n must be in 0..E");
    if (with_shared != 0 && with_shared != 1) return fail(ctx, MOE_EINVAL, "with_shared must be 0 or 1");
    if (with_shared && (!c.n_shared || !d_shared)) return fail(ctx, MOE_EINVAL, "no shared expert");
    if (T == 0 || (n == 0 && !with_shared)) return MOE_OK;
    if (!d_x || !d_o || !d_ws) return fail(ctx, MOE_EINVAL, "null x/o/workspace");
    const bool host_lists = h_topk_ids && T <= kDecodeMaxT && decode_shape_supported(c);
    if (n > 0 && (!h_experts || !h_slots || !d_slot_base)) return fail(ctx, MOE_EINVAL, "null routed-expert argument");
    if (n > 0 && !host_lists && (!d_offsets || !d_perm)) return fail(ctx, MOE_EINVAL, "need d_offsets and d_perm");
    std::vector<int32_t> where(c.n_experts, -1);
    for (int i = 0; i < n; ++i) {
        const int e = h_experts[i], sl = h_slots[i];
        if (e < 0 || e >= c.n_experts || where[e] >= 0) return fail(ctx, MOE_EINVAL, "expert id out of range or repeated");
        if (sl < 0 || sl >= (1 << 21)) return fail(ctx, MOE_EINVAL, "slot out of range");
        where[e] = i;
    }
    hipError_t e;
    if (host_lists) {
        DecodeList dl;
        const int st = build_decode_list(ctx, T, h_topk_ids, h_experts, h_slots, with_shared, where, &dl);
        if (st != MOE_OK) return st;
        e = launch_ffn_decode(c, ctx->lay, d_x, T, d_slot_base, d_shared, dl, d_o, d_ws, s);
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_expert_ffn launch");
    }
    ExpertList list;
    list.n = 0;
    for (int i = 0; i < n; ++i) list.ent[list.n++] = h_experts[i] | (h_slots[i] << 10);
    if (with_shared) list.ent[list.n++] = kSharedTag;
    if (T <= kDecodeMaxT || !gemm_shape_supported(c)) {
        if (!gemv_shape_supported(c)) return fail(ctx, MOE_ESHAPE, "no GEMV kernel for this hidden/inter");
        e = launch_ffn_gemv(c, ctx->lay, d_x, T, d_offsets, d_perm, d_slot_base, d_shared, list, d_o, d_ws, s);
    } else {
        e = launch_ffn_gemm(c, ctx->lay, d_x, T, d_offsets, d_perm, d_slot_base, d_shared, list, d_o, d_ws, s);
    }
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_expert_ffn launch");
}

int moe_expert_ffn_merge(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids,
                         const int32_t* d_topk_ids, const float* d_topk_w, const void* d_slot_base,
                         const int32_t* h_experts, const int32_t* h_slots, int32_t n, const void* d_shared,
                         int32_t with_shared, const float* d_y_host, void* d_out, void* d_ws, hipStream_t s) {
    return moe::expert_ffn_merge(ctx, d_x, T, h_topk_ids, d_topk_ids, d_topk_w, d_slot_base, h_experts, h_slots, n,
                                 d_shared, with_shared, d_y_host, d_out, [&](int32_t, void** ws) {
                                     *ws = d_ws;
                                     return d_ws ? MOE_OK : fail(ctx, MOE_EINVAL, "null workspace");
                                 }, s);
}

}  // extern "C"

namespace moe {

int expert_ffn_merge(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids, const int32_t* d_topk_ids,
                     const float* d_topk_w, const void* d_slot_base, const int32_t* h_experts, const int32_t* h_slots,
                     int32_t n, const void* d_shared, int32_t with_shared, const float* d_y_host, void* d_out,
                     const std::function<int(int32_t, void**)>& workspace, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    const moe_config& c = ctx->cfg;
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (n < 0 || n > c.n_experts) return fail(ctx, MOE_EINVAL, "n must be in 0..E");
    if (with_shared != 0 && with_shared != 1) return fail(ctx, MOE_EINVAL, "with_shared must be 0 or 1");
    if (with_shared && (!c.n_shared || !d_shared)) return fail(ctx, MOE_EINVAL, "no shared expert");
    if (T == 0) return MOE_OK;
    if (T > kDecodeMaxT || !decode_shape_supported(c))
        return fail(ctx, MOE_ESHAPE, "moe_expert_ffn_merge takes decode batches (T <= 8) of the decode shapes");
    if (!d_x || !d_out || !h_topk_ids || !d_topk_ids || !d_topk_w)
        return fail(ctx, MOE_EINVAL, "null x/out/top-k argument");
    if (n > 0 && (!h_experts || !h_slots || !d_slot_base)) return fail(ctx, MOE_EINVAL, "null routed-expert argument");
    std::vector<int32_t> where(c.n_experts, -1);
    uint32_t mask[kMaxExperts / 32] = {0};
    for (int i = 0; i < n; ++i) {
        const int e = h_experts[i], sl = h_slots[i];
        if (e < 0 || e >= c.n_experts || where[e] >= 0) return fail(ctx, MOE_EINVAL, "expert id out of range or repeated");
        if (sl < 0 || sl >= (1 << 21)) return fail(ctx, MOE_EINVAL, "slot out of range");
        where[e] = i;
        mask[e >> 5] |= 1u << (e & 31);
    }
    DecodeList dl;
    const int st = build_decode_list(ctx, T, h_topk_ids, h_experts, h_slots, with_shared, where, &dl);
    if (st != MOE_OK) return st;
    void* d_ws = nullptr;
    const int wst = workspace(T, &d_ws);     // after validation: an error leaves nothing behind
    if (wst != MOE_OK) return wst;
    hipError_t e = launch_ffn_decode_merge(c, ctx->lay, d_x, T, d_slot_base, d_shared, dl, d_topk_ids, d_topk_w, mask,
                                           with_shared, d_y_host, d_out, d_ws, s);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_expert_ffn_merge launch");
}

}  // namespace moe

extern "C" {

int moe_merge_partial(moe_ctx* ctx, const void* d_o, const int32_t* d_topk_ids, const float* d_topk_w,
                      const int32_t* h_gpu_experts, int32_t n_gpu, int32_t with_shared, const float* d_y_host,
                      int32_t T, void* d_out, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    const moe_config& c = ctx->cfg;
    if (T < 0 || n_gpu < 0 || n_gpu > c.n_experts) return fail(ctx, MOE_EINVAL, "bad T or n_gpu");
    if (with_shared != 0 && with_shared != 1) return fail(ctx, MOE_EINVAL, "with_shared must be 0 or 1");
    if (with_shared && !c.n_shared) return fail(ctx, MOE_EINVAL, "no shared expert");
    if (T == 0) return MOE_OK;
    if (!d_out || !d_topk_ids || !d_topk_w) return fail(ctx, MOE_EINVAL, "null merge buffer");
    if ((n_gpu > 0 || with_shared) && !d_o) return fail(ctx, MOE_EINVAL, "null pair outputs");
    if (n_gpu > 0 && !h_gpu_experts) return fail(ctx, MOE_EINVAL, "null expert list");
    uint32_t mask[kMaxExperts / 32] = {0};
    for (int i = 0; i < n_gpu; ++i) {
        const int e = h_gpu_experts[i];
        if (e < 0 || e >= c.n_experts) return fail(ctx, MOE_EINVAL, "expert id out of range");
        mask[e >> 5] |= 1u << (e & 31);
    }
    hipError_t e = launch_merge(c, d_o, d_topk_ids, d_topk_w, mask, with_shared, d_y_host, T, d_out, s);
    return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "moe_merge_partial launch");
}

}  // extern "C"

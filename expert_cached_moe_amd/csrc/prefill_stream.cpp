// Layer streaming for prefill: a chunk of tokens goes through every MoE layer while
// the layers' expert pools cross PCIe from pinned host memory.
//
// asapai.co.kr, "Running 753B GLM-5.2 on a single workstation GPU", section
// "Abandoning fixed offloading in favor of measured bandwidth": prefill streams the
// whole expert pool of each layer, and a second device buffer lets the next layer's
// transfer overlap the current layer's compute (turning the second buffer off costs
// about a fifth to a quarter of the prefill rate there).
//
// Schedule with two buffers (U = upload on `side`, C = compute on `s`):
//   U0 -> buf0;  for l: [U(l+1) -> buf((l+1)%2) after C(l-1)] ; C(l) on buf(l%2) after U(l)
// With one buffer every upload waits for the previous layer's compute.
#include <hip/hip_runtime.h>

#include <vector>

#include "internal.h"

using namespace moe;

extern "C" {

int moe_prefill_stream(moe_ctx* ctx, void* d_layer_bufs, int32_t n_buffers, const float* d_logits, const void* d_x,
                       int32_t T, const void* d_shared, int32_t* d_topk_ids, float* d_topk_w, int32_t* d_counts,
                       int32_t* d_offsets, int32_t* d_perm, int32_t* d_inv, void* d_o, void* d_ws, void* d_out,
                       hipStream_t s, hipStream_t side) {
    if (!ctx) return MOE_EINVAL;
    const moe_config& c = ctx->cfg;
    const int L = c.n_layers, E = c.n_experts;
    if (n_buffers != 1 && n_buffers != 2) return fail(ctx, MOE_EINVAL, "n_buffers must be 1 or 2");
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (!ctx->h_pool || ctx->n_pool != int64_t(L) * E)
        return fail(ctx, MOE_ESTATE, "moe_prefill_stream needs a bound host pool of n_layers*E blobs");
    if (!d_layer_bufs || !d_out || !d_counts || !d_offsets) return fail(ctx, MOE_EINVAL, "null buffer");
    if (c.n_shared && !d_shared) return fail(ctx, MOE_EINVAL, "shared expert blobs required");
    if (T > 0 && (!d_logits || !d_x || !d_topk_ids || !d_topk_w || !d_perm || !d_inv || !d_o || !d_ws))
        return fail(ctx, MOE_EINVAL, "null route/ffn buffer");
    if (side == s) return fail(ctx, MOE_EINVAL, "uploads need a stream of their own");
    if (T > 0 && !(T > kDecodeMaxT && gemm_shape_supported(c)) && !gemv_shape_supported(c))
        return fail(ctx, MOE_ESHAPE, "no expert kernel for this hidden/inter");
    for (hipEvent_t& ev : ctx->stream_ev) {
        if (ev) continue;
        hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            ev = nullptr;
            return hip_fail(ctx, e, "hipEventCreateWithFlags");
        }
    }
    hipEvent_t ev_start = ctx->stream_ev[0];
    hipEvent_t* up_done = ctx->stream_ev + 1;
    hipEvent_t* comp_done = ctx->stream_ev + 3;

    const int64_t blob = ctx->lay.bytes, layer_bytes = blob * E;
    const uint8_t* hpool = static_cast<const uint8_t*>(ctx->h_pool);
    uint8_t* bufs = static_cast<uint8_t*>(d_layer_bufs);
    std::vector<int32_t> all(E);
    for (int e = 0; e < E; ++e) all[e] = e;
    const int with_shared = c.n_shared ? 1 : 0;
    const int64_t out_layer = int64_t(T) * c.hidden * act_bytes(c);

    auto upload = [&](int l) -> int {
        const int b = l % n_buffers;
        hipError_t e = hipMemcpyAsync(bufs + b * layer_bytes, hpool + l * layer_bytes, layer_bytes,
                                      hipMemcpyHostToDevice, side);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipMemcpyAsync (layer upload)");
        e = hipEventRecord(up_done[b], side);
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "hipEventRecord (upload)");
    };
    auto side_waits = [&](hipEvent_t ev) -> int {
        hipError_t e = hipStreamWaitEvent(side, ev, 0);
        return e == hipSuccess ? MOE_OK : hip_fail(ctx, e, "hipStreamWaitEvent (side)");
    };

    hipError_t he = hipEventRecord(ev_start, s);
    if (he != hipSuccess) return hip_fail(ctx, he, "hipEventRecord (start)");
    int st = side_waits(ev_start);
    if (st == MOE_OK && L > 0) st = upload(0);
    for (int l = 0; st == MOE_OK && l < L; ++l) {
        const int b = l % n_buffers;
        if (n_buffers == 2 && l + 1 < L) {
            if (l >= 1 && (st = side_waits(comp_done[(l + 1) % 2])) != MOE_OK) break;
            if ((st = upload(l + 1)) != MOE_OK) break;
        }
        he = hipStreamWaitEvent(s, up_done[b], 0);
        if (he != hipSuccess) { st = hip_fail(ctx, he, "hipStreamWaitEvent (compute)"); break; }
        const uint8_t* sh = with_shared ? static_cast<const uint8_t*>(d_shared) + int64_t(l) * blob : nullptr;
        void* out = static_cast<uint8_t*>(d_out) + l * out_layer;
        if ((st = moe_route(ctx, d_logits + int64_t(l) * T * E, T, d_topk_ids, d_topk_w, d_counts, d_offsets,
                            d_perm, d_inv, d_ws, s)) != MOE_OK)
            break;
        if ((st = moe_expert_ffn(ctx, d_x, T, nullptr, d_offsets, d_perm, bufs + b * layer_bytes, all.data(),
                                 all.data(), E, sh, with_shared, d_o, d_ws, s)) != MOE_OK)
            break;
        if ((st = moe_merge_partial(ctx, d_o, d_topk_ids, d_topk_w, all.data(), E, with_shared, nullptr, T, out,
                                    s)) != MOE_OK)
            break;
        he = hipEventRecord(comp_done[b], s);
        if (he != hipSuccess) { st = hip_fail(ctx, he, "hipEventRecord (compute)"); break; }
        if (n_buffers == 1 && l + 1 < L) {
            if ((st = side_waits(comp_done[0])) != MOE_OK) break;
            if ((st = upload(l + 1)) != MOE_OK) break;
        }
    }
    return st;
}

}  // extern "C"

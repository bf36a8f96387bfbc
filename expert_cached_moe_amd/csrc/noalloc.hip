// moe_expert_ffn_merge_noalloc: the decode experts + merge with the library's own scratch.
//
// For callers that may not allocate device memory (code under HIP graph capture, serving loops
// and harnesses that forbid hipMalloc).  The scratch the decode kernels need (SwiGLU
// activations, and the pair outputs when the down projection and the merge run as separate
// kernels) lives in one file-scope device array, which each GPU the library runs on holds
// until the process ends.  Its device address is taken once per device with
// hipGetSymbolAddress (host code never passes the array's own name to a kernel: on the host
// that name is a stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace moe {
namespace {

constexpr int64_t kScratchBytes = int64_t(8) << 20;     // 8 MiB: decode batches of up to 8 tokens, 136 pair rows of 16 K values
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array, looked up on the first call on the device.
int scratch_ptr(moe_ctx* ctx, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(ctx, MOE_EUNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(ctx, e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

int64_t moe_noalloc_scratch_bytes(void) { return moe::kScratchBytes; }

int moe_expert_ffn_merge_noalloc(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids,
                                 const int32_t* d_topk_ids, const float* d_topk_w, const void* d_slot_base,
                                 const int32_t* h_experts, const int32_t* h_slots, int32_t n, const void* d_shared,
                                 int32_t with_shared, const float* d_y_host, void* d_out, hipStream_t s) {
    if (!ctx) return MOE_EINVAL;
    return moe::expert_ffn_merge(ctx, d_x, T, h_topk_ids, d_topk_ids, d_topk_w, d_slot_base, h_experts, h_slots, n,
                                 d_shared, with_shared, d_y_host, d_out, [&](int32_t t, void** ws) {
                                     const int64_t need = moe::ws_layout(ctx->cfg, t).bytes;
                                     if (need > moe::kScratchBytes)
                                         return moe::fail(ctx, MOE_ECAPACITY,
                                                          "decode scratch of " + std::to_string(need) +
                                                              " bytes exceeds the library's " +
                                                              std::to_string(moe::kScratchBytes) + "-byte array");
                                     return moe::scratch_ptr(ctx, ws);
                                 }, s);
}

}  // extern "C"

// Gate-weighted un-permute and exact merge of the GPU and CPU partial sums (gfx950).
//
// banandre.com, "The 284B Model on a 32GB GPU Trick", section "The q* Policy:
// Math Instead of Guesses": the GPU and CPU partial sums are added after the
// layer, with no approximation.  For token t:
//   y[t] = sum_{j=0..k-1, expert on the GPU} w[t][j] * o[t*k+j]  (+ shared o[T*k+t])
//          (+ y_host[t]),
// accumulated in fp32 in that fixed order, then stored as fp32 or bf16.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

struct MergeArgs {
    const float* o;
    const int32_t* ids;
    const float* w;
    const float* y_host;
    void* out;
    int32_t T, k, H, with_shared, out_bf16;
    uint32_t mask[kMaxExperts / 32];
};

__global__ void __launch_bounds__(256) k_merge(const MergeArgs a) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= a.H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; ++j) {
        const int p = t * a.k + j;
        const int e = a.ids[p];
        if (!((a.mask[e >> 5] >> (e & 31)) & 1u)) continue;
        const float g = a.w[p];
        const float4 v = *reinterpret_cast<const float4*>(a.o + int64_t(p) * a.H + c);
        acc.x = fmaf(g, v.x, acc.x);
        acc.y = fmaf(g, v.y, acc.y);
        acc.z = fmaf(g, v.z, acc.z);
        acc.w = fmaf(g, v.w, acc.w);
    }
    if (a.with_shared) {
        const float4 v = *reinterpret_cast<const float4*>(a.o + (int64_t(a.T) * a.k + t) * a.H + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (a.y_host) {
        const float4 v = *reinterpret_cast<const float4*>(a.y_host + int64_t(t) * a.H + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if (a.out_bf16) {
        uint2 r;
        r.x = dev::pack_bf16x2(acc.x, acc.y);
        r.y = dev::pack_bf16x2(acc.z, acc.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + int64_t(t) * a.H + c) = r;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + int64_t(t) * a.H + c) = acc;
    }
}

}  // namespace

hipError_t launch_merge(const moe_config& c, const float* o, const int32_t* ids, const float* w,
                        const uint32_t* gpu_mask, int32_t with_shared, const float* y_host, int32_t T, void* out,
                        hipStream_t s) {
    MergeArgs a;
    a.o = o;
    a.ids = ids;
    a.w = w;
    a.y_host = y_host;
    a.out = out;
    a.T = T;
    a.k = c.top_k;
    a.H = c.hidden;
    a.with_shared = with_shared;
    a.out_bf16 = c.w_dtype != MOE_W_F32;
    for (int i = 0; i < kMaxExperts / 32; ++i) a.mask[i] = gpu_mask[i];
    const dim3 grid((c.hidden / 4 + 255) / 256, T);
    hipLaunchKernelGGL(k_merge, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

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
    const void* o;            // pair outputs in the activation dtype (fp32, or bf16 when out_bf16)
    const int32_t* ids;
    const float* w;
    const float* y_host;
    void* out;
    int32_t T, k, H, with_shared, out_bf16;
    uint32_t mask[kMaxExperts / 32];
};

// Four consecutive values of a pair-output row, raw (16 bytes of fp32 or 8 of bf16); they are
// loaded first and widened after every load of the thread is in flight.
template <bool BF16> struct Raw4;
template <> struct Raw4<true> { typedef uint2 T; };
template <> struct Raw4<false> { typedef float4 T; };

template <bool BF16>
__device__ __forceinline__ typename Raw4<BF16>::T load_raw4(const void* o, int64_t idx) {
    if constexpr (BF16) return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(o) + idx);
    else return *reinterpret_cast<const float4*>(static_cast<const float*>(o) + idx);
}

__device__ __forceinline__ float4 widen(uint2 r) {
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u), __uint_as_float(r.y << 16),
                       __uint_as_float(r.y & 0xFFFF0000u));
}
__device__ __forceinline__ float4 widen(float4 r) { return r; }

template <bool BF16>
__global__ void __launch_bounds__(256) k_merge(const MergeArgs a) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= a.H) return;
    // every partial row of the token is loaded at once (rows of CPU experts hold stale
    // values and are dropped by a select, never multiplied), next to the ids and gates
    typename Raw4<BF16>::T v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
        v[j] = (a.o && j < a.k) ? load_raw4<BF16>(a.o, (int64_t(t) * a.k + j) * a.H + c) : typename Raw4<BF16>::T{};
    float g[kMaxTopK];
    int64_t row[kMaxTopK];
    // the mask words are read up front and picked by compare, so the only memory access
    // that waits for an id is none
    uint32_t mw[kMaxExperts / 32];
#pragma unroll
    for (int q = 0; q < kMaxExperts / 32; ++q) mw[q] = a.mask[q];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        row[j] = -1;
        g[j] = 0.0f;
        if (j < a.k) {
            const int p = t * a.k + j;
            const int e = a.ids[p];
            uint32_t word = 0;
#pragma unroll
            for (int q = 0; q < kMaxExperts / 32; ++q) word = (e >> 5) == q ? mw[q] : word;
            if ((word >> (e & 31)) & 1u) {
                row[j] = p;
                g[j] = a.w[p];
            }
        }
    }
    float4 sh = make_float4(0.f, 0.f, 0.f, 0.f), yh = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.with_shared) sh = widen(load_raw4<BF16>(a.o, (int64_t(a.T) * a.k + t) * a.H + c));
    if (a.y_host) yh = *reinterpret_cast<const float4*>(a.y_host + int64_t(t) * a.H + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (row[j] >= 0) {
            const float4 f = widen(v[j]);
            acc.x = fmaf(g[j], f.x, acc.x);
            acc.y = fmaf(g[j], f.y, acc.y);
            acc.z = fmaf(g[j], f.z, acc.z);
            acc.w = fmaf(g[j], f.w, acc.w);
        }
    }
    acc.x += sh.x; acc.y += sh.y; acc.z += sh.z; acc.w += sh.w;
    acc.x += yh.x; acc.y += yh.y; acc.z += yh.z; acc.w += yh.w;
    if (BF16) {
        uint2 r;
        r.x = dev::pack_bf16x2(acc.x, acc.y);
        r.y = dev::pack_bf16x2(acc.z, acc.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + int64_t(t) * a.H + c) = r;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + int64_t(t) * a.H + c) = acc;
    }
}

}  // namespace

hipError_t launch_merge(const moe_config& c, const void* o, const int32_t* ids, const float* w,
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
    if (a.out_bf16) hipLaunchKernelGGL((k_merge<true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_merge<false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

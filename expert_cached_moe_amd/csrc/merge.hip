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

// N consecutive values of a pair-output row per thread, raw: 8 bf16 (16 bytes) or 4 fp32 (16
// bytes), so every load instruction of a wave moves 1 KiB.  They are loaded first and widened
// after every load of the thread is in flight.
template <bool BF16> struct Piece;
template <> struct Piece<true> {
    typedef uint4 T;
    static constexpr int N = 8;
};
template <> struct Piece<false> {
    typedef float4 T;
    static constexpr int N = 4;
};

template <bool BF16>
__device__ __forceinline__ typename Piece<BF16>::T load_piece(const void* o, int64_t idx) {
    if constexpr (BF16) return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(o) + idx);
    else return *reinterpret_cast<const float4*>(static_cast<const float*>(o) + idx);
}

__device__ __forceinline__ void widen(uint4 r, float (&f)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void widen(float4 r, float (&f)[4]) {
    f[0] = r.x;
    f[1] = r.y;
    f[2] = r.z;
    f[3] = r.w;
}

template <bool BF16>
__global__ void __launch_bounds__(256) k_merge(const MergeArgs a) {
    constexpr int N = Piece<BF16>::N;
    typedef typename Piece<BF16>::T Raw;
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * N;
    if (c >= a.H) return;
    // every partial row of the token is loaded at once (rows of CPU experts hold stale
    // values and are dropped by a select, never multiplied), next to the ids and gates
    Raw v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) v[j] = (a.o && j < a.k) ? load_piece<BF16>(a.o, (int64_t(t) * a.k + j) * a.H + c) : Raw{};
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
    Raw shr{};
    if (a.with_shared) shr = load_piece<BF16>(a.o, (int64_t(a.T) * a.k + t) * a.H + c);
    float yh[N];
#pragma unroll
    for (int i = 0; i < N; ++i) yh[i] = 0.0f;
    if (a.y_host) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 q = *reinterpret_cast<const float4*>(a.y_host + int64_t(t) * a.H + c + i);
            yh[i] = q.x;
            yh[i + 1] = q.y;
            yh[i + 2] = q.z;
            yh[i + 3] = q.w;
        }
    }
    float acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (row[j] >= 0) {
            float f[N];
            widen(v[j], f);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] = fmaf(g[j], f[i], acc[i]);
        }
    }
    float sh[N];
    widen(shr, sh);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        acc[i] += sh[i];
        acc[i] += yh[i];
    }
    if constexpr (BF16) {
        uint4 r;
        r.x = dev::pack_bf16x2(acc[0], acc[1]);
        r.y = dev::pack_bf16x2(acc[2], acc[3]);
        r.z = dev::pack_bf16x2(acc[4], acc[5]);
        r.w = dev::pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + int64_t(t) * a.H + c) = r;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + int64_t(t) * a.H + c) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
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
    const int per_thread = a.out_bf16 ? 8 : 4;           // values per thread (16 bytes of pair output)
    const dim3 grid((c.hidden / per_thread + 255) / 256, T);
    if (a.out_bf16) hipLaunchKernelGGL((k_merge<true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_merge<false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe

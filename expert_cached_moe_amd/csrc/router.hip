// Router logits l[t][e] = sum_h x[t][h] * W_r[e][h] on gfx950, accumulated in fp32.
//
// banandre.com, "The 284B Model on a 32GB GPU Trick", section "Sparsity Is a Lie (But a
// Useful One)": a small router scores every expert for each token before the top-k.  W_r
// is stored per expert ([E][H], each expert's weights contiguous), so a decode token reads
// every router row once, coalesced.
//
// T <= 8: one wave per expert streams its row and keeps one partial sum per token; a
// butterfly over the wave finishes each dot product.  Larger T: 64-token x 64-expert tiles
// with both operands staged in LDS 16 columns of H at a time; every output sums h in
// ascending order.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

using dev::kWave;

constexpr int kGemvT = 8;

template <bool BF16>
__device__ __forceinline__ float4 load_x4(const void* x, int64_t off) {
    if (BF16) {
        const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + off);
        return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                           __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
    }
    return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
}

template <bool BF16>
__global__ void __launch_bounds__(256) k_router_gemv(const void* __restrict__ x, int T, int H, int E,
                                                     const float* __restrict__ wr, float* __restrict__ out) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int e = blockIdx.x * 4 + wave;
    if (e >= E) return;
    const float* row = wr + int64_t(e) * H;
    float acc[kGemvT];
#pragma unroll
    for (int t = 0; t < kGemvT; ++t) acc[t] = 0.0f;
    for (int h = lane * 4; h < H; h += kWave * 4) {
        const float4 w = *reinterpret_cast<const float4*>(row + h);
#pragma unroll
        for (int t = 0; t < kGemvT; ++t) {
            if (t < T) {
                const float4 v = load_x4<BF16>(x, int64_t(t) * H + h);
                acc[t] = fmaf(v.x, w.x, acc[t]);
                acc[t] = fmaf(v.y, w.y, acc[t]);
                acc[t] = fmaf(v.z, w.z, acc[t]);
                acc[t] = fmaf(v.w, w.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kGemvT; ++t) {
        if (t >= T) break;
        float s = acc[t];
#pragma unroll
        for (int d = kWave / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
        if (lane == 0) out[int64_t(t) * E + e] = s;
    }
}

// 64 tokens x 64 experts per workgroup; thread (tr, ec) owns tokens 4tr..4tr+3 and experts
// 4ec..4ec+3.  LDS holds the tiles K-major (xs[h][t], ws[h][e]) so each K step is two
// 16-byte reads for 16 FMAs.
constexpr int kTT = 64, kTE = 64, kTK = 16;

template <bool BF16>
__global__ void __launch_bounds__(256) k_router_gemm(const void* __restrict__ x, int T, int H, int E,
                                                     const float* __restrict__ wr, float* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) float xs[kTK][kTT + 4];
    __shared__ __attribute__((aligned(16))) float ws[kTK][kTE + 4];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * kTT, e0 = blockIdx.y * kTE;
    const int tr = tid / 16, ec = tid % 16;
    float acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[a][q] = 0.0f;
    for (int h0 = 0; h0 < H; h0 += kTK) {
        // x tile and w tile: 64 rows x kTK columns each, 4 values per thread
        {
            const int r = tid / 4, c = (tid % 4) * 4;
            const bool ok = t0 + r < T;
            const float4 v = ok ? load_x4<BF16>(x, int64_t(t0 + r) * H + h0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
            xs[c][r] = v.x;
            xs[c + 1][r] = v.y;
            xs[c + 2][r] = v.z;
            xs[c + 3][r] = v.w;
        }
        {
            const int r = tid / 4, c = (tid % 4) * 4;
            const float4 v = e0 + r < E ? *reinterpret_cast<const float4*>(wr + int64_t(e0 + r) * H + h0 + c)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
            ws[c][r] = v.x;
            ws[c + 1][r] = v.y;
            ws[c + 2][r] = v.z;
            ws[c + 3][r] = v.w;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kTK; ++c) {
            const float4 xv = *reinterpret_cast<const float4*>(&xs[c][4 * tr]);
            const float4 w0 = *reinterpret_cast<const float4*>(&ws[c][4 * ec]);
            const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
            const float wb[4] = {w0.x, w0.y, w0.z, w0.w};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[a][q] = fmaf(xa[a], wb[q], acc[a][q]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int t = t0 + 4 * tr + a;
        if (t >= T) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = e0 + 4 * ec + q;
            if (e < E) out[int64_t(t) * E + e] = acc[a][q];
        }
    }
}

}  // namespace

hipError_t launch_router_logits(const moe_config& c, const void* x, int32_t T, const float* wr, float* out,
                                hipStream_t s) {
    const bool bf16 = c.w_dtype != MOE_W_F32;
    const int H = c.hidden, E = c.n_experts;
    if (T <= kGemvT) {
        const dim3 grid((E + 3) / 4);
        if (bf16) hipLaunchKernelGGL((k_router_gemv<true>), grid, dim3(256), 0, s, x, T, H, E, wr, out);
        else hipLaunchKernelGGL((k_router_gemv<false>), grid, dim3(256), 0, s, x, T, H, E, wr, out);
    } else {
        const dim3 grid((T + kTT - 1) / kTT, (E + kTE - 1) / kTE);
        if (bf16) hipLaunchKernelGGL((k_router_gemm<true>), grid, dim3(256), 0, s, x, T, H, E, wr, out);
        else hipLaunchKernelGGL((k_router_gemm<false>), grid, dim3(256), 0, s, x, T, H, E, wr, out);
    }
    return hipGetLastError();
}

}  // namespace moe

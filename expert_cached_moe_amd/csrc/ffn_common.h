// Element formats and per-chunk arithmetic shared by the GEMV-style decode kernels.
//
// A weight "chunk" is 16 bytes of one row: 4 fp32, 8 bf16 or 32 MXFP4 elements (one
// e8m0 scale block).  The matching activation chunk holds the same elements of x
// (or h) in the activation format (fp32 for fp32 weights, else bf16).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace moe {
namespace ffn {

enum { WT_F32 = 0, WT_BF16 = 1, WT_FP4 = 2 };


template <int WT> struct Fmt;
template <> struct Fmt<WT_F32> {
    static constexpr int EPC = 4, ABYTES = 4;
    __device__ static int64_t row_bytes(int K) { return int64_t(K) * 4; }
};
template <> struct Fmt<WT_BF16> {
    static constexpr int EPC = 8, ABYTES = 2;
    __device__ static int64_t row_bytes(int K) { return int64_t(K) * 2; }
};
template <> struct Fmt<WT_FP4> {
    static constexpr int EPC = 32, ABYTES = 2;
    __device__ static int64_t row_bytes(int K) { return int64_t(K) / 2; }
};

// Activation chunk matching one 16-byte weight chunk.
template <int WT> struct ActChunk { uint4 v[Fmt<WT>::EPC * Fmt<WT>::ABYTES / 16]; };

template <int WT>
__device__ __forceinline__ void load_act(ActChunk<WT>& a, const uint8_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < int(sizeof(a.v) / 16); ++i) a.v[i] = q[i];
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t a, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dev::bf16x2, w), __builtin_bit_cast(dev::bf16x2, a), c,
                                           false);
}

// Partial dot product of one weight chunk with one activation chunk.
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4& w, const ActChunk<WT>& a, uint8_t scale, float acc);

template <>
__device__ __forceinline__ float chunk_dot<WT_F32>(const uint4& w, const ActChunk<WT_F32>& a, uint8_t, float acc) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(a.v[0].x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(a.v[0].y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(a.v[0].z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(a.v[0].w), acc);
    return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<WT_BF16>(const uint4& w, const ActChunk<WT_BF16>& a, uint8_t, float acc) {
    acc = dot2(w.x, a.v[0].x, acc);
    acc = dot2(w.y, a.v[0].y, acc);
    acc = dot2(w.z, a.v[0].z, acc);
    acc = dot2(w.w, a.v[0].w, acc);
    return acc;
}

// MXFP4: 32 e2m1 elements of one scale block.  The unscaled products are summed in
// fp32 and the block sum is multiplied by the power-of-two scale 2^(s-127).
template <>
__device__ __forceinline__ float chunk_dot<WT_FP4>(const uint4& w, const ActChunk<WT_FP4>& a, uint8_t s, float acc) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float part = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 av = a.v[q];  // 8 bf16 activations: elements 8q .. 8q+7
        const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
        // byte b of the word holds elements 2b (low nibble) and 2b + 1 (high nibble)
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ww[q], 1.0f, 0),
                                               __builtin_bit_cast(dev::bf16x2, aw[0]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ww[q], 1.0f, 1),
                                               __builtin_bit_cast(dev::bf16x2, aw[1]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ww[q], 1.0f, 2),
                                               __builtin_bit_cast(dev::bf16x2, aw[2]), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(ww[q], 1.0f, 3),
                                               __builtin_bit_cast(dev::bf16x2, aw[3]), part, false);
    }
    const float sc = s ? __uint_as_float(uint32_t(s) << 23) : __uint_as_float(0x00400000u);
    return fmaf(part, sc, acc);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// silu from the hardware exp2 and reciprocal (about 1 ulp each), for values that are
// rounded to bf16 (8 significant bits) right after.
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}


// Hides a weight chunk from the optimiser at the top of each token iteration, so the
// MXFP4 decode to bf16 stays inside the token loop: hoisted out of it, the decoded
// copies hold four times the weight registers live and cut the waves per SIMD.
template <int WT>
__device__ __forceinline__ void keep_packed(uint4& w) {
    if constexpr (WT == WT_FP4) asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}

// 16-byte weight chunk `ch` of a row, streamed (non-temporal: read once per step).
__device__ __forceinline__ uint4 load_w(const uint8_t* row, int ch) {
    const dev::u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const dev::u32x4*>(row) + ch);
    return make_uint4(t.x, t.y, t.z, t.w);
}

template <int WT>
// Store in the activation dtype (fp32 for fp32 weights, bf16 otherwise): h and pair outputs.
__device__ __forceinline__ void store_act(uint8_t* h, int64_t idx, float v) {
    if (WT == WT_F32)
        reinterpret_cast<float*>(h)[idx] = v;
    else
        reinterpret_cast<uint16_t*>(h)[idx] = dev::f32_to_bf16_bits(v);
}

inline int chunks_per_row(int wt, int K) { return wt == WT_F32 ? K / 4 : wt == WT_BF16 ? K / 8 : K / 32; }

}  // namespace ffn
}  // namespace moe

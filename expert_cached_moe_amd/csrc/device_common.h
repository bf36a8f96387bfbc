// Device helpers shared by the gfx950 kernels of libmoecache.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {
namespace dev {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Two fp32 values to packed bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Sum of NV values held by every lane of a group of G consecutive lanes (G a power of
// two, 2 <= G <= 64).  Halving exchange: at the step with distance d the lane keeps
// one half of its values and adds the partner's copy of that half, so NV values cost
// about NV + log2(G) shuffles instead of NV * log2(G).  On return v[0] holds the
// group sum of value index vidx(lane), where vidx is returned; every lane of the
// group that holds the same index holds the same (bitwise) sum.
template <int NV, int G>
__device__ __forceinline__ int group_reduce_split(float (&v)[NV], int lane) {
    int idx = 0;
    int n = NV;
#pragma unroll
    for (int d = G / 2; d >= 1; d >>= 1) {
        if (n > 1) {
            const bool upper = (lane & d) != 0;
            const int h = n / 2;
#pragma unroll
            for (int i = 0; i < NV / 2; ++i) {
                if (i < h) {
                    // both values as registers before the select: a select of the two array
                    // loads is otherwise folded into a load through a selected address, which
                    // puts the array in scratch memory
                    float lo = v[i], hi = v[i + h];
                    asm("" : "+v"(lo), "+v"(hi));
                    const float send = upper ? lo : hi;
                    const float keep = upper ? hi : lo;
                    v[i] = keep + __shfl_xor(send, d, kWave);
                }
            }
            if (upper) idx += h;
            n = h;
        } else {
            v[0] += __shfl_xor(v[0], d, kWave);
        }
    }
    return idx;
}

}  // namespace dev
}  // namespace moe

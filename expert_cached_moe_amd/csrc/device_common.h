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

// Value of the partner lane across bit D of the lane index.  D <= 8: DPP inside each row of
// 16 lanes (quad swaps for 1 and 2; the half-row and row mirrors, i <-> 7 - i and i <-> 15 - i,
// for 4 and 8: each pairs a lane with one whose bit D differs and whose higher bits agree).
template <int D>
__device__ __forceinline__ float dpp_partner(float x) {
    static_assert(D == 1 || D == 2 || D == 4 || D == 8, "row-local partner");
    constexpr int kCtrl = D == 1 ? 0xB1 : D == 2 ? 0x4E : D == 4 ? 0x141 : 0x140;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// (lo, hi) held by every lane -> lo + partner's lo in the lanes whose bit D (16 or 32) is clear,
// hi + partner's hi in the others: one permlane swap of the two registers hands each lane its
// own kept value and the partner's copy, in the two halves of the result.
template <int D>
__device__ __forceinline__ float swap_add(float lo, float hi) {
    static_assert(D == 16 || D == 32, "cross-row partner");
    const auto sw = D == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false)
                            : __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Sum of NV values held by every lane of a group of G consecutive lanes (G a power of
// two, 2 <= G <= 64, groups aligned to G).  Halving exchange: at the step with distance d
// each lane keeps one half of its values and adds its partner's copy of that half (partner:
// a lane of the group whose bit d differs and whose other bits above d agree), so NV values
// cost about NV + log2(G) exchanges instead of NV * log2(G).  The exchanges are DPP moves
// and permlane swaps, register to register (no LDS round trip).  On return v[0] holds the
// group sum of value index vidx(lane), where vidx is returned; every lane of the group that
// holds the same index holds the same (bitwise) sum.
template <int D, int NV>
__device__ __forceinline__ void reduce_step(float (&v)[NV], int& n, int& idx, int lane) {
    if (n > 1) {
        const bool upper = (lane & D) != 0;
        const int h = n / 2;
#pragma unroll
        for (int i = 0; i < NV / 2; ++i) {
            if (i < h) {
                // both values as registers before the select: a select of the two array
                // loads is otherwise folded into a load through a selected address, which
                // puts the array in scratch memory
                float lo = v[i], hi = v[i + h];
                asm("" : "+v"(lo), "+v"(hi));
                if constexpr (D >= 16) {
                    v[i] = swap_add<D>(lo, hi);
                } else {
                    const float send = upper ? lo : hi;
                    const float keep = upper ? hi : lo;
                    v[i] = keep + dpp_partner<D>(send);
                }
            }
        }
        if (upper) idx += h;
        n = h;
    } else {
        if constexpr (D >= 16)
            v[0] = swap_add<D>(v[0], v[0]);
        else
            v[0] += dpp_partner<D>(v[0]);
    }
}

template <int NV, int G>
__device__ __forceinline__ int group_reduce_split(float (&v)[NV], int lane) {
    static_assert(G >= 2 && G <= 64 && (G & (G - 1)) == 0, "group size");
    int idx = 0;
    int n = NV;
    if constexpr (G >= 64) reduce_step<32>(v, n, idx, lane);
    if constexpr (G >= 32) reduce_step<16>(v, n, idx, lane);
    if constexpr (G >= 16) reduce_step<8>(v, n, idx, lane);
    if constexpr (G >= 8) reduce_step<4>(v, n, idx, lane);
    if constexpr (G >= 4) reduce_step<2>(v, n, idx, lane);
    reduce_step<1>(v, n, idx, lane);
    return idx;
}

// Value of lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((__lane_id() & 32) ? sw[0] : sw[1]);
}

}  // namespace dev
}  // namespace moe

// Router softmax + top-k and the token-by-expert permutation (gfx950).
//
// banandre.com, "The 284B Model on a 32GB GPU Trick", section "Sparsity Is a Lie
// (But a Useful One)": a small router selects a handful of experts per token; in
// prefill thousands of tokens route to nearly every expert (section "The Three
// Failure Modes of Existing Engines"), so the pairs are grouped by expert before
// the grouped GEMM.
//
// Selection order: logit descending, lower expert id on equal logits (-0 == +0).
// Gates: softmax renormalised over the k selected logits (or over all experts).
// Selection: k rounds of a wave-wide maximum over an order-preserving 32-bit key of
// the logit; ballots over the lanes holding that key then name the lowest expert id,
// whose key is cleared for the next round.
// Grouping: stable counting sort of pairs p = t*k + j by expert (ascending p
// within an expert), with its inverse.  Integer work is exact and deterministic:
// counts use integer LDS atomics, ranks use wave ballots.
#include <hip/hip_runtime.h>


#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

using dev::kWave;

constexpr int kRouteWaves = 16;              // tokens per workgroup in the large-T route kernel
constexpr int kBlock = kRouteWaves * kWave;  // 1024 threads
static_assert(kBlock == kPermChunk, "one pair per thread per permutation chunk");

// Order-preserving key of a logit: larger logit -> larger unsigned key; -0 and +0 share a key.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide maximum of an unsigned key, left in every lane: butterflies inside each row of
// 16 lanes (DPP quad swaps, rotations by 4 and 8), then row pairs and wave halves exchanged
// with permlane16_swap / permlane32_swap.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t a) {
    return max(a, uint32_t(__builtin_amdgcn_mov_dpp(int(a), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t a) {
    a = dpp_umax<0xB1>(a);   // quad_perm [1,0,3,2]
    a = dpp_umax<0x4E>(a);   // quad_perm [2,3,0,1]
    a = dpp_umax<0x124>(a);  // row_ror:4
    a = dpp_umax<0x128>(a);  // row_ror:8
    const auto h16 = __builtin_amdgcn_permlane16_swap(a, a, false, false);
    a = max(h16[0], h16[1]);
    const auto h32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return max(h32[0], h32[1]);
}

// Route one token with one wave.  EPL = experts per lane (ceil(E/64)); lane l holds experts
// l + 64 i.  k rounds: the wave-wide maximum of the logit keys, then the lowest expert id
// holding it (ballots per slot i, lowest slot first, then lowest lane, since the id is
// l + 64 i), whose key is cleared to 0; lane j keeps the j-th pick.  Keys of finite logits
// are nonzero, so 0 marks an expert out of the running.
template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ lrow, int E, int k, int renorm,
                                            int32_t* __restrict__ ids_out, float* __restrict__ w_out,
                                            int32_t* __restrict__ lds_ids) {
    const int lane = dev::lane_id();
    float v[EPL];
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        const bool live = e < E;
        v[i] = live ? lrow[e] : 0.0f;
        key[i] = live ? order_key(v[i]) : 0u;
    }
    uint32_t mine = 0u;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        uint32_t best = key[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) best = max(best, key[i]);
        best = wave_umax(best);
        uint64_t hit = 0;
        int slot = 0;
#pragma unroll
        for (int i = EPL - 1; i >= 0; --i) {
            const uint64_t b = __ballot(key[i] == best);
            if (b) {
                hit = b;
                slot = i;
            }
        }
        const int wl = __builtin_ctzll(hit);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == slot && lane == wl) key[i] = 0u;
        if (lane == j) {
            mine = best;
            my_e = wl + kWave * slot;
        }
    }
    const float my_v = key_value(mine);
    const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_v), 0));
    // softmax over the selected logits (or over all E), shifted by the largest logit
    const float ex = lane < k ? expf(my_v - v0) : 0.0f;
    float den = 0.0f;
    if (renorm) {
        for (int j = 0; j < k; ++j) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
    } else {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i < E) s += expf(v[i] - v0);
#pragma unroll
        for (int d = kWave / 2; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
        den = s;
    }
    if (lane < k) {
        ids_out[lane] = my_e;
        w_out[lane] = ex / den;
        if (lds_ids) lds_ids[lane] = my_e;
    }
}

template <int EPL>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int T, int E, int k, int renorm, int t0,
                             int tstride, int32_t* __restrict__ ids, float* __restrict__ w,
                             int32_t* __restrict__ lds_ids) {
    const int wave = threadIdx.x / kWave;
    for (int t = t0 + wave; t < T; t += tstride)
        route_token<EPL>(logits + int64_t(t) * E, E, k, renorm, ids + int64_t(t) * k, w + int64_t(t) * k,
                         lds_ids ? lds_ids + int64_t(t) * k : nullptr);
}

__device__ __forceinline__ void route_dispatch(const float* logits, int T, int E, int k, int renorm, int t0, int tstride,
                               int32_t* ids, float* w, int32_t* lds_ids) {
    const int epl = (E + kWave - 1) / kWave;
    switch (epl) {
        case 1: route_tokens<1>(logits, T, E, k, renorm, t0, tstride, ids, w, lds_ids); break;
        case 2: route_tokens<2>(logits, T, E, k, renorm, t0, tstride, ids, w, lds_ids); break;
        case 3:
        case 4: route_tokens<4>(logits, T, E, k, renorm, t0, tstride, ids, w, lds_ids); break;
        default: route_tokens<8>(logits, T, E, k, renorm, t0, tstride, ids, w, lds_ids); break;
    }
}

// Lanes of the wave holding the same expert id (10-bit ids), among lanes with valid = 1.
__device__ __forceinline__ uint64_t match_expert(int e, bool valid) {
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0;
}

// Exclusive prefix sum of cnt[0..E) by wave 0 into off[0..E]; other waves idle.
__device__ void wave0_scan(const int32_t* __restrict__ cnt, int E, int32_t* __restrict__ off_lds,
                           int32_t* __restrict__ off_global, int32_t* __restrict__ counts_global) {
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    constexpr int kPer = kMaxExperts / kWave;  // 8 experts per lane
    int local[kPer];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane * kPer + i;
        local[i] = e < E ? cnt[e] : 0;
        sum += local[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane * kPer + i;
        if (e < E) {
            off_lds[e] = run;
            if (off_global) off_global[e] = run;
            if (counts_global) counts_global[e] = local[i];
        }
        run += local[i];
    }
    if (lane == kWave - 1) {
        off_lds[E] = run;
        if (off_global) off_global[E] = run;
    }
}

// Stable scatter of one chunk of up to 1024 pairs: pair p = p0 + tid with expert
// e = ids[tid].  run[e] is the output position of the chunk's first pair of expert
// e; it is advanced by the chunk's count.  wc: [16][E] per-wave counts (LDS).
__device__ void scatter_chunk(const int32_t* __restrict__ ids_src, int p0, int n_valid, int E,
                              int32_t* __restrict__ run, int32_t (*wc)[kMaxExperts],
                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const bool valid = tid < n_valid;
    const int e = valid ? ids_src[tid] : 0;
    const uint64_t m = match_expert(e, valid);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int rank = __popcll(m & lt);
    const int cw = __popcll(m);
    for (int i = tid; i < kRouteWaves * E; i += kBlock) wc[i / E][i % E] = 0;
    __syncthreads();
    if (valid && rank == 0) wc[wave][e] = cw;
    __syncthreads();
    if (valid) {
        int pos = run[e] + rank;
        for (int w2 = 0; w2 < wave; ++w2) pos += wc[w2][e];
        perm[pos] = p0 + tid;
        inv[p0 + tid] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kBlock) {
        int s = 0;
#pragma unroll
        for (int w2 = 0; w2 < kRouteWaves; ++w2) s += wc[w2][ee];
        run[ee] += s;
    }
    __syncthreads();
}

// T*k <= 4096: route, count, scan and scatter in one workgroup.
__global__ __launch_bounds__(kBlock) void k_route_small(const float* __restrict__ logits, int T, int E, int k,
                                                        int renorm, int32_t* __restrict__ ids, float* __restrict__ w,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int32_t s_ids[kSmallRouteMaxPairs];
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_run[kMaxExperts + 1];
    __shared__ int32_t s_wc[kRouteWaves][kMaxExperts];
    const int tid = threadIdx.x;
    route_dispatch(logits, T, E, k, renorm, 0, kRouteWaves, ids, w, s_ids);
    for (int e = tid; e < E; e += kBlock) s_cnt[e] = 0;
    __syncthreads();
    const int n = T * k;
    for (int p = tid; p < n; p += kBlock) atomicAdd(&s_cnt[s_ids[p]], 1);
    __syncthreads();
    wave0_scan(s_cnt, E, s_run, offsets, counts);
    __syncthreads();
    for (int p0 = 0; p0 < n; p0 += kBlock) scatter_chunk(s_ids + p0, p0, n - p0, E, s_run, s_wc, perm, inv);
}

// T*k <= 64 (decode): route, then the whole grouping by wave 0 with ballots.  For the
// pair of lane p with expert e: eq = lanes with expert e, lt = lanes with a smaller
// expert (bit-serial compare of the 10-bit ids, most significant bit first), so
// its position is |lt| + |eq below p|.
__global__ __launch_bounds__(1024) void k_route_tiny(const float* __restrict__ logits, int T, int E, int k,
                                                     int renorm, int32_t* __restrict__ ids, float* __restrict__ w,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int32_t s_ids[kWave];
    const int tid = threadIdx.x;
    route_dispatch(logits, T, E, k, renorm, 0, blockDim.x / kWave, ids, w, s_ids);
    __syncthreads();
    const int n = T * k;
    for (int e = tid; e < E; e += blockDim.x) {
        int c = 0, lt = 0;
        for (int p = 0; p < n; ++p) {
            const int v = s_ids[p];
            c += v == e;
            lt += v < e;
        }
        counts[e] = c;
        offsets[e] = lt;
    }
    if (tid == 0) offsets[E] = n;
    if (tid < kWave) {
        const bool valid = tid < n;
        const int e = valid ? s_ids[tid] : 0;
        uint64_t eq = __ballot(valid), lt = 0;
#pragma unroll
        for (int b = 9; b >= 0; --b) {
            const bool bit = (e >> b) & 1;
            const uint64_t b1 = __ballot(valid && bit);
            if (bit) {
                lt |= eq & ~b1;
                eq &= b1;
            } else {
                eq &= ~b1;
            }
        }
        const uint64_t below = tid == 0 ? 0ull : (~0ull >> (kWave - tid));
        if (valid) {
            const int pos = __popcll(lt) + __popcll(eq & below);
            perm[pos] = tid;
            inv[tid] = pos;
        }
    }
}

// Large T: one wave per token.
__global__ __launch_bounds__(kBlock) void k_route(const float* __restrict__ logits, int T, int E, int k, int renorm,
                                                  int32_t* __restrict__ ids, float* __restrict__ w) {
    route_dispatch(logits, T, E, k, renorm, blockIdx.x * kRouteWaves, T, ids, w, nullptr);
}

// Per-chunk expert histograms hist[chunk][E].
__global__ __launch_bounds__(kBlock) void k_perm_hist(const int32_t* __restrict__ ids, int n, int E,
                                                      int32_t* __restrict__ hist) {
    __shared__ int32_t s_cnt[kMaxExperts];
    const int tid = threadIdx.x, c = blockIdx.x;
    for (int e = tid; e < E; e += kBlock) s_cnt[e] = 0;
    __syncthreads();
    const int p = c * kBlock + tid;
    if (p < n) atomicAdd(&s_cnt[ids[p]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) hist[int64_t(c) * E + e] = s_cnt[e];
}

// counts, offsets, and base[chunk][e] = offsets[e] + pairs of e in earlier chunks.  The
// workgroup's threads form G = 1024 / E groups per expert (thread e + E q: expert e, group q);
// group q owns a contiguous range of chunks, sums its column of hist over that range in one
// round of loads, and after the group partials and the experts' totals are scanned in LDS
// writes its base values once (from the values still in registers when the range is at most
// 8 chunks).  One thread per expert walking all the chunks took two dependent global round
// trips per 8 chunks.
__global__ __launch_bounds__(kBlock) void k_perm_scan(const int32_t* __restrict__ hist, int nchunks, int E,
                                                      int32_t* __restrict__ base, int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ offsets) {
    __shared__ int32_t s_part[kBlock];           // [G][E] partial sums
    __shared__ int32_t s_cnt[kMaxExperts];
    __shared__ int32_t s_off[kMaxExperts + 1];
    constexpr int U = 8;
    const int tid = threadIdx.x;
    const int G = kBlock / E;                     // E <= 512, so G >= 2
    const int span = (nchunks + G - 1) / G;       // chunks per group
    const int e = tid % E, q = tid / E;
    const bool act = q < G;
    const int c0 = act ? q * span : 0, c1 = act ? min(nchunks, c0 + span) : 0;
    int h[U];
#pragma unroll
    for (int u = 0; u < U; ++u) h[u] = 0;
    int part = 0;
    for (int b = c0; b < c1; b += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) h[u] = b + u < c1 ? hist[int64_t(b + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) part += h[u];
    }
    if (act) s_part[q * E + e] = part;
    __syncthreads();
    for (int x = tid; x < E; x += kBlock) {
        int total = 0;
        for (int g = 0; g < G; ++g) total += s_part[g * E + x];
        s_cnt[x] = total;
    }
    __syncthreads();
    wave0_scan(s_cnt, E, s_off, offsets, counts);
    __syncthreads();
    if (!act) return;
    int run = s_off[e];
    for (int g = 0; g < q; ++g) run += s_part[g * E + e];
    for (int b = c0; b < c1; b += U) {
        if (span > U) {
#pragma unroll
            for (int u = 0; u < U; ++u) h[u] = b + u < c1 ? hist[int64_t(b + u) * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (b + u < c1) base[int64_t(b + u) * E + e] = run;
            run += h[u];
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_perm_scatter(const int32_t* __restrict__ ids, int n, int E,
                                                         const int32_t* __restrict__ base, int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv) {
    __shared__ int32_t s_run[kMaxExperts];
    __shared__ int32_t s_wc[kRouteWaves][kMaxExperts];
    const int tid = threadIdx.x, c = blockIdx.x;
    for (int e = tid; e < E; e += kBlock) s_run[e] = base[int64_t(c) * E + e];
    __syncthreads();
    const int p0 = c * kBlock;
    scatter_chunk(ids + p0, p0, n - p0, E, s_run, s_wc, perm, inv);
}

}  // namespace

hipError_t launch_route(const moe_config& c, const float* logits, int32_t T, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                        hipStream_t s) {
    const int E = c.n_experts, k = c.top_k;
    const int64_t n = int64_t(T) * k;
    if (n <= kWave) {
        const int waves = T < 1 ? 1 : T > 16 ? 16 : int(T);   // one wave per token
        hipLaunchKernelGGL(k_route_tiny, dim3(1), dim3(waves * kWave), 0, s, logits, T, E, k, c.renormalize, ids, w,
                           counts, offsets, perm, inv);
        return hipGetLastError();
    }
    if (n <= kSmallRouteMaxPairs) {
        hipLaunchKernelGGL(k_route_small, dim3(1), dim3(kBlock), 0, s, logits, T, E, k, c.renormalize, ids, w,
                           counts, offsets, perm, inv);
        return hipGetLastError();
    }
    const WsLayout L = ws_layout(c, T);
    int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.hist);
    int32_t* base = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.base);
    const int nchunks = int((n + kPermChunk - 1) / kPermChunk);
    hipLaunchKernelGGL(k_route, dim3((T + kRouteWaves - 1) / kRouteWaves), dim3(kBlock), 0, s, logits, T, E, k,
                       c.renormalize, ids, w);
    hipLaunchKernelGGL(k_perm_hist, dim3(nchunks), dim3(kBlock), 0, s, ids, int(n), E, hist);
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(kBlock), 0, s, hist, nchunks, E, base, counts, offsets);
    hipLaunchKernelGGL(k_perm_scatter, dim3(nchunks), dim3(kBlock), 0, s, ids, int(n), E, base, perm, inv);
    return hipGetLastError();
}

}  // namespace moe

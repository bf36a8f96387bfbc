// Decode expert FFN (T <= 8 tokens): batched GEMV over the expert slots (gfx950).
//
// Decode reads every weight of every selected expert once per step while only a
// handful of tokens use it, so the step is bound by HBM bandwidth.  Each lane
// streams 16-byte chunks of weight rows into registers (consecutive lanes read
// consecutive chunks: 1 KiB per wave load instruction); the tokens routed to the
// expert are applied to the registers and each row sum is reduced across the lanes
// of the row with a halving exchange (DPP moves and permlane swaps).  The gate/up kernel
// copies the activation rows (x) into LDS once per workgroup for bf16 and MXFP4 weights (one
// barrier per group of rows), as does the MXFP4 down kernel for h; the fp32 kernels and the
// bf16 down kernel read them straight from memory with independent waves, and the fused
// down + merge kernel keeps its pair outputs in LDS.  Which tokens use which expert comes from the host's copy of the
// step's top-k ids (the host needs them anyway to plan the cache), packed into the
// kernel arguments, so these kernels do not wait for the router kernel.
//
// Two launches:
//   gate/up: each wave owns a few intermediate columns (their gate rows and up rows
//            of the interleaved [2I][H] matrix); after the reduction lanes l and l^32
//            hold (gate, up) of one column, and h = silu(gate) * up is stored (bf16,
//            or fp32 for fp32 weights);
//   down:    rows of [H][I]: o[p][row] = Wd[row] . h[p] in fp32, stored in the activation
//            dtype; or, in the fused kernel, merged into the layer output in the same launch.
// Expert form: SwiGLU without biases (banandre.com, "The 284B Model on a 32GB GPU
// Trick", section "Sparsity Is a Lie": experts are small feed-forward networks).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "ffn_common.h"
#include "internal.h"

namespace moe {
namespace {

using dev::kWave;
using namespace ffn;

// Layer output of the fused down + merge kernel (the arguments of moe_merge_partial).
struct MergeTarget {
    const int32_t* ids;    // device top-k ids [T][k]
    const float* w;        // device gates [T][k]
    const float* y_host;   // host-expert partial sums, fp32 [T][H], or null
    void* out;             // [T][H]: bf16 (bf16 and MXFP4 weights) or fp32
    uint32_t mask[kMaxExperts / 32];  // experts whose pair outputs count
    int32_t with_shared;
};

struct DecodeArgs {
    const uint8_t* slot_base;
    const uint8_t* shared_blob;
    int64_t blob_bytes;
    int64_t off_w, off_s;  // matrix and MXFP4 scale offsets inside a blob
    const uint8_t* act;    // gate/up: x [T][H]; down: h [pair rows][I]
    uint8_t* out;          // gate/up: h; down: o [pair rows][H] in the activation dtype
    int32_t K, nrows, T, k, I, H;
    int32_t nt;            // MXFP4: activation rows staged in LDS per group
    MergeTarget m;         // fused down + merge: gates, mask and layer output
    DecodeList list;
};

// MXFP4 activations through LDS.  A lane's 16-byte weight chunk holds 32 elements, whose
// activations are 64 contiguous bytes; read straight from global memory, the four 16-byte
// pieces of consecutive lanes lie 64 bytes apart, so every load instruction touches four
// times the cache granules of a dense one, and each wave repeats them.  Instead the
// workgroup copies each activation row once into LDS with direct-to-LDS loads, stored
// piece-major: piece i of chunk j at 16-byte slot i*(K/32) + j, so lane reads of piece i
// for consecutive chunks are consecutive 16-byte slots (measured on MI355X: 3% off the
// MXFP4 decode FFN).  The copies are issued after the weight loads: fetching the
// activations first and letting the products start as each weight chunk lands
// (per-chunk waits) measured 15-20% slower than streaming the weights at once and
// waiting for everything.  bf16 activations take the same path with the row copied as is:
// one copy per workgroup instead of one global read per wave (decode FFN at batch 8: 1-2%
// faster on MI355X).
__device__ __forceinline__ void barrier_loads() {
    __builtin_amdgcn_s_waitcnt(0);      // vmcnt(0) expcnt(0) lgkmcnt(0): own LDS-bound loads landed
    __syncthreads();
}

// Issues the copy of activation row `row` (K bf16 values) into staging slot `slot` of
// `xs`; K/512 instructions of 64 lanes, spread over the workgroup's nw waves.
__device__ __forceinline__ void stage_row(uint4* xs, const uint8_t* act, int row, int K, int slot, int wave, int nw,
                                          int lane) {
    const int units = K / 8, cpr = K / 32;
    const uint8_t* src = act + int64_t(row) * K * 2;
    for (int u = wave; u * kWave < units; u += nw) {
        const int S = u * kWave + lane, i = S / cpr, j = S - i * cpr;
        __builtin_amdgcn_global_load_lds(src + 64 * j + 16 * i, xs + slot * units + u * kWave, 16, 0, 0);
    }
}

// bf16: row `row` copied as is (chunk j at 16-byte slot j of the row's staging slot)
__device__ __forceinline__ void stage_row_plain(uint4* xs, const uint8_t* act, int row, int K, int slot, int wave, int nw,
                                                int lane) {
    const int units = K / 8;
    const uint8_t* src = act + int64_t(row) * K * 2;
    for (int u = wave; u * kWave < units; u += nw)
        __builtin_amdgcn_global_load_lds(src + 16 * (u * kWave + lane), xs + slot * units + u * kWave, 16, 0, 0);
}
__device__ __forceinline__ void read_staged(ActChunk<WT_BF16>& av, const uint4* xs, int K, int slot, int chunk) {
    av.v[0] = xs[slot * (K / 8) + chunk];
}

__device__ __forceinline__ void read_staged(ActChunk<WT_FP4>& av, const uint4* xs, int K, int slot, int chunk) {
    const int units = K / 8, cpr = K / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) av.v[i] = xs[slot * units + i * cpr + chunk];
}

// MXFP4 block scales of consecutive weight rows.  The scale bytes of rows [r0, r0 + n) are
// contiguous (K/32 bytes a row); lane l loads dword l of every 64-dword piece of that run, and
// a lane that needs byte b of the run takes it from the lane holding dword b/4 (ds_bpermute).
// One dword load a lane per piece replaces one byte load per weight chunk: a vector memory
// instruction costs the address pipeline about the same whatever it moves, and byte loads of
// 64 bytes a wave made the MXFP4 decode kernels 7-8% slower (measured on MI355X).
template <int ND>
struct ScaleRun {
    uint32_t d[ND];
    // run: the run's first scale byte; ndw: dwords readable from it
    __device__ __forceinline__ void load(const uint8_t* run, int ndw, int lane) {
#pragma unroll
        for (int k = 0; k < ND; ++k) {
            const int i = 64 * k + lane;
            d[k] = *reinterpret_cast<const uint32_t*>(run + 4 * (i < ndw ? i : 0));
        }
    }
    // byte b of the run, from piece k = b / 256 (the same in every lane of the call)
    __device__ __forceinline__ uint8_t byte(int k, int b) const {
        const int v = __builtin_amdgcn_ds_bpermute(b & 252, int(d[k]));
        return uint8_t(uint32_t(v) >> (8 * (b & 3)));
    }
};

// Keeps the loads issued above it ahead of the code below it (the scale permutes below wait
// for the scale loads, which were issued first, and must not hold back the weight loads).
__device__ __forceinline__ void loads_issued() { asm volatile("" ::: "memory"); }

// Pair row and activation row of the i-th set bit of the expert's token mask.
struct TokenIter {
    uint32_t mask, jpack;
    bool shared;
    int T, k;
    __device__ bool next(int& p, int& t) {
        if (!mask) return false;
        t = __builtin_ctz(mask);
        mask &= mask - 1;
        p = shared ? T * k + t : t * k + int((jpack >> (4 * t)) & 15u);
        return true;
    }
};

// Rows per wave of the gate/up kernel: small waves keep many loads in flight across
// the chip (measured on MI355X: one gate+up row pair per wave streams the 50 MB of a
// 1-token step 20% faster than 8 rows per wave); at least 8 loads per lane.
// (MXFP4 with 16 loads per lane, or 4 down passes, measured 7-12% slower.)
constexpr int kGateUpWaves = 4;
template <int CPL> struct GateUpShape {
    static constexpr int RPW = CPL >= 4 ? 2 : 8 / CPL;  // rows per wave: RPW/2 gate + RPW/2 up
    static constexpr int WPB = kGateUpWaves;            // waves per workgroup
    static constexpr int COLS = RPW / 2 * WPB;          // intermediate columns per workgroup
};

template <int WT, int CPL>
__global__ void __launch_bounds__(64 * kGateUpWaves) k_decode_gate_up(const DecodeArgs a) {
    constexpr int EPC = Fmt<WT>::EPC;
    constexpr int AB = Fmt<WT>::ABYTES;
    constexpr int RPW = GateUpShape<CPL>::RPW, HALF = RPW / 2, WPB = GateUpShape<CPL>::WPB;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int ei = blockIdx.y;
    const int entry = a.list.ent[ei];
    const bool shared = (entry & 1023) == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    TokenIter it{a.list.tokmask[ei], a.list.jpack[ei], shared, a.T, a.k};
    const int64_t row_bytes = Fmt<WT>::row_bytes(a.H);
    const int col0 = (blockIdx.x * WPB + wave) * HALF;       // first intermediate column of the wave
    // interleaved layout: column i has its gate row at (i/16)*32 + i%16 and its up row 16 further
    auto row_of = [&](int q) {
        const int i = col0 + (q < HALF ? q : q - HALF);
        return (i / 16) * 32 + (i % 16) + (q < HALF ? 0 : 16);
    };
    // MXFP4: the scales of the gate rows and of the up rows (HALF consecutive rows each)
    constexpr int NDW = HALF * 16 * CPL, ND = (NDW + 63) / 64;
    ScaleRun<ND> sr[2];
    if constexpr (WT == WT_FP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) sr[h].load(blob + a.off_s + int64_t(row_of(h * HALF)) * (a.H / 32), NDW, lane);
    }
    uint4 wv[RPW][CPL];
    uint8_t sv[RPW][CPL];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const int64_t r = row_of(q);
#pragma unroll
        for (int c = 0; c < CPL; ++c) wv[q][c] = load_w(blob + a.off_w + r * row_bytes, c * kWave + lane);
    }
    if constexpr (WT == WT_FP4) loads_issued();
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int base = (q % HALF) * 64 * CPL + c * kWave;   // run byte of chunk c * 64 of row q
            sv[q][c] = WT == WT_FP4 ? sr[q / HALF].byte(base / 256, base + lane) : uint8_t(0);
        }
    // one token: dot products of the wave's rows with x[t], SwiGLU, store h[p]
    auto token = [&](int p, auto&& act_chunk) {
#pragma unroll
        for (int q = 0; q < RPW; ++q)
#pragma unroll
            for (int c = 0; c < CPL; ++c) keep_packed<WT>(wv[q][c]);
        float part[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) part[q] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ActChunk<WT> av;
            act_chunk(av, c);
#pragma unroll
            for (int q = 0; q < RPW; ++q) part[q] = chunk_dot<WT>(wv[q][c], av, sv[q][c], part[q]);
        }
        // after the halving reduction lanes l and l^32 hold (gate, up) of one column
        const int qi = dev::group_reduce_split<RPW, 64>(part, lane);
        const float up = dev::other_half(part[0]);
        if ((lane & 32) == 0 && (lane & (64 / RPW - 1)) == 0)
            store_act<WT>(a.out, int64_t(p) * a.I + col0 + qi, silu(part[0]) * up);
    };
    int p, t;
    if constexpr (WT == WT_F32) {
        while (it.next(p, t))
            token(p, [&](ActChunk<WT>& av, int c) {
                load_act<WT>(av, a.act + (int64_t(t) * a.H + int64_t(c * kWave + lane) * EPC) * AB);
            });
    } else {
        // groups of up to nt token rows of x, staged after the weight loads are issued; every
        // wave takes the same token sequence, so the barriers are uniform.  The first group's
        // copies are issued ahead of the loop: at the loop's entry the compiler waits for the
        // weight loads (register copies), which would otherwise put the activation fetch
        // behind the whole weight stream.
        extern __shared__ __attribute__((aligned(16))) uint4 xs[];
        auto stage_group = [&](TokenIter g, int gp, int gt) {
            int n = 0;
            for (bool gh = true; n < a.nt && gh; ++n) {
                if constexpr (WT == WT_FP4) stage_row(xs, a.act, gt, a.H, n, wave, WPB, lane);
                else stage_row_plain(xs, a.act, gt, a.H, n, wave, WPB, lane);
                gh = g.next(gp, gt);
            }
            return n;
        };
        bool have = it.next(p, t);
        int n = have ? stage_group(it, p, t) : 0;
        while (have) {
            barrier_loads();
            for (int s = 0; s < n; ++s) {
                token(p, [&](ActChunk<WT>& av, int c) { read_staged(av, xs, a.H, s, c * kWave + lane); });
                have = it.next(p, t);
            }
            __syncthreads();            // group read before the next one lands
            if (have) n = stage_group(it, p, t);
        }
    }
}

// Down rows: LPR lanes per row, CPL chunks per lane, NPASS passes of 64/LPR rows.
constexpr int kDownPasses = 2, kDownWaves = 8;

template <int WT, int LPR, int CPL>
__global__ void __launch_bounds__(64 * kDownWaves) k_decode_down(const DecodeArgs a) {
    constexpr int EPC = Fmt<WT>::EPC;
    constexpr int AB = Fmt<WT>::ABYTES;
    constexpr int RPP = kWave / LPR;
    constexpr int NPASS = kDownPasses;
    constexpr int RPW = NPASS * RPP;
    constexpr int RPB = RPW * kDownWaves;
    static_assert(NPASS <= LPR, "pass layout");
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = lane / LPR, lr = lane % LPR;
    const int ei = blockIdx.y;
    const int entry = a.list.ent[ei];
    const bool shared = (entry & 1023) == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    TokenIter it{a.list.tokmask[ei], a.list.jpack[ei], shared, a.T, a.k};
    const int64_t row_bytes = Fmt<WT>::row_bytes(a.I);
    const int row0 = blockIdx.x * RPB + wave * RPW;

    int p, t;
    bool have = it.next(p, t);
    ActChunk<WT> av0[CPL];
    if (WT != WT_FP4 && have) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) load_act<WT>(av0[c], a.act + (int64_t(p) * a.I + int64_t(c * LPR + lr) * EPC) * AB);
    }
    // MXFP4 with at most 4 chunks a lane: the scales of each pass's RPP rows (64 * CPL bytes) as
    // one run, clipped at the matrix end; wider rows load a scale byte per chunk
    constexpr bool kRun = WT == WT_FP4 && 16 * CPL <= 64;
    ScaleRun<1> sr[NPASS];
    if constexpr (kRun) {
#pragma unroll
        for (int q = 0; q < NPASS; ++q) {
            const int rs = row0 + q * RPP;
            const int avail = rs < a.nrows ? min(16 * CPL, (a.nrows - rs) * (a.I / 128)) : 0;
            sr[q].load(blob + a.off_s + (avail ? int64_t(rs) * (a.I / 32) : 0), avail ? avail : 1, lane);
        }
    }
    uint4 wv[NPASS][CPL];
    uint8_t sv[NPASS][CPL];
#pragma unroll
    for (int q = 0; q < NPASS; ++q) {
        const int r = row0 + q * RPP + g;
        const bool ok = r < a.nrows;
        const int rl = ok ? r : a.nrows - 1;     // unconditional loads (a loaded register copied inside
                                                 // a branch waits for every load): rows past the end
                                                 // reread the last row, and are not stored
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            wv[q][c] = load_w(blob + a.off_w + int64_t(rl) * row_bytes, c * LPR + lr);
            if constexpr (!kRun)
                sv[q][c] = (WT == WT_FP4 && ok) ? blob[a.off_s + int64_t(r) * (a.I / 32) + c * LPR + lr] : uint8_t(127);
        }
    }
    if constexpr (kRun) {
        loads_issued();
#pragma unroll
        for (int q = 0; q < NPASS; ++q)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                sv[q][c] = row0 + q * RPP + g < a.nrows ? sr[q].byte(0, g * LPR * CPL + c * LPR + lr) : uint8_t(127);
    }
    // one pair row: dot products of the wave's rows with h[p], store o[p]
    auto token = [&](int p, auto&& act_chunk) {
#pragma unroll
        for (int q = 0; q < NPASS; ++q)
#pragma unroll
            for (int c = 0; c < CPL; ++c) keep_packed<WT>(wv[q][c]);
        float part[NPASS];
#pragma unroll
        for (int q = 0; q < NPASS; ++q) part[q] = 0.0f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ActChunk<WT> av;
            act_chunk(av, c);
#pragma unroll
            for (int q = 0; q < NPASS; ++q) part[q] = chunk_dot<WT>(wv[q][c], av, sv[q][c], part[q]);
        }
        const int qi = dev::group_reduce_split<NPASS, LPR>(part, lane);
        const int r = row0 + qi * RPP + g;
        if ((lr & (LPR / NPASS - 1)) == 0 && r < a.nrows)
            store_act<WT>(a.out, int64_t(p) * a.H + r, part[0]);
    };
    if constexpr (WT != WT_FP4) {
        if (have) token(p, [&](ActChunk<WT>& av, int c) { av = av0[c]; });
        while (it.next(p, t))
            token(p, [&](ActChunk<WT>& av, int c) {
                load_act<WT>(av, a.act + (int64_t(p) * a.I + int64_t(c * LPR + lr) * EPC) * AB);
            });
    } else {
        // groups of up to nt pair rows of h (uniform over the workgroup; the first group's
        // copies issued ahead of the loop, as above)
        extern __shared__ __attribute__((aligned(16))) uint4 xs[];
        auto stage_group = [&](TokenIter g, int gp, int gt) {
            int n = 0;
            for (bool gh = true; n < a.nt && gh; ++n) {
                stage_row(xs, a.act, gp, a.I, n, wave, kDownWaves, lane);
                gh = g.next(gp, gt);
            }
            return n;
        };
        int n = have ? stage_group(it, p, t) : 0;
        while (have) {
            barrier_loads();
            for (int s = 0; s < n; ++s) {
                token(p, [&](ActChunk<WT>& av, int c) { read_staged(av, xs, a.I, s, c * LPR + lr); });
                have = it.next(p, t);
            }
            __syncthreads();            // group read before the next one lands
            if (have) n = stage_group(it, p, t);
        }
    }
}

// Down projection and gate-weighted merge in one launch.  A workgroup owns RPW rows of the
// output for every listed expert: wave w computes the pair outputs of entry w for those rows
// exactly as k_decode_down does (same lanes, chunks and reduction order),
// rounds them to the activation dtype and keeps them in LDS; after one barrier each
// (token, row) is merged exactly as k_merge does: gate-weighted pair outputs of the GPU
// experts in order j = 0..k-1 (fmaf), then the shared expert's row, then the host part.
// The result is therefore bit-identical to moe_expert_ffn followed by moe_merge_partial,
// without the pair outputs going through memory or a third launch.  Used when the list
// has at most one entry per wave (decode at batch 1 of the workloads' shapes: 7-8 experts).
constexpr int kFusedWaves = 8, kFusedTopK = 8;

template <int WT, int LPR, int CPL>
__global__ void __launch_bounds__(64 * kFusedWaves) k_decode_down_merge(const DecodeArgs a) {
    constexpr int EPC = Fmt<WT>::EPC;
    constexpr int AB = Fmt<WT>::ABYTES;
    constexpr int RPP = kWave / LPR;
    constexpr int NPASS = kDownPasses;
    constexpr int RPW = NPASS * RPP;
    static_assert(NPASS <= LPR && RPW <= 8, "pass layout");
    __shared__ float s_o[(kDecodeMaxT * kFusedTopK + kDecodeMaxT) * RPW];
    // wave index made uniform, so the list reads (ent, tokmask, jpack at [ei]) are scalar loads:
    // as vector loads their waits also waited for the merge inputs issued ahead of them
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int g = lane / LPR, lr = lane % LPR;
    const int64_t row_bytes = Fmt<WT>::row_bytes(a.I);
    const int row0 = blockIdx.x * RPW;
    // the merge's ids, gates and host part, issued first so their latency hides under the
    // weight stream.  Thread i < T*RPW (all in wave 0) merges token i / RPW, row i % RPW; only
    // wave 0 loads them (17 loads a wave in every wave would crowd the weight loads in the
    // address path), inside wave 0 unconditionally (index 0 for the other threads; the host
    // part through a valid stand-in address), so no load waits behind a branch
    const bool merger = tid < a.T * RPW;
    const int mt = merger ? tid / RPW : 0, mrl = tid % RPW, mrow = row0 + mrl;
    int mid[kFusedTopK];
    float mw[kFusedTopK];
    float myh;
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < kFusedTopK; ++j) {
            const int pj = merger && j < a.k ? mt * a.k + j : 0;
            mid[j] = a.m.ids[pj];
            mw[j] = a.m.w[pj];
        }
        const float* yh = a.m.y_host ? a.m.y_host + int64_t(mt) * a.H + (mrow < a.H ? mrow : 0) : a.m.w;
        myh = *yh;
    }
    // one entry per wave (the host launches this kernel for lists of at most kFusedWaves
    // entries); no loop over entries, whose back edge would make the compiler wait for the
    // merge inputs before the weight loads (register reuse across iterations)
    if (wave < a.list.n) {
        const int ei = wave;
        const int entry = a.list.ent[ei];
        const bool shared = (entry & 1023) == kSharedTag;
        const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
        TokenIter it{a.list.tokmask[ei], a.list.jpack[ei], shared, a.T, a.k};
        int p, t;
        bool have = it.next(p, t);
        // first token's h prefetched ahead of the weights (not for MXFP4: 64 bytes per chunk)
        ActChunk<WT> av0[WT == WT_FP4 ? 1 : CPL];
        if (WT != WT_FP4 && have) {
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                load_act<WT>(av0[c], a.act + (int64_t(p) * a.I + int64_t(c * LPR + lr) * EPC) * AB);
        }
        // MXFP4 with at most 4 chunks a lane: the scales of each pass's RPP rows (64 * CPL bytes) as
        // one run, clipped at the matrix end; wider rows load a scale byte per chunk
        constexpr bool kRun = WT == WT_FP4 && 16 * CPL <= 64;
        ScaleRun<1> sr[NPASS];
        if constexpr (kRun) {
#pragma unroll
            for (int q = 0; q < NPASS; ++q) {
                const int rs = row0 + q * RPP;
                const int avail = rs < a.nrows ? min(16 * CPL, (a.nrows - rs) * (a.I / 128)) : 0;
                sr[q].load(blob + a.off_s + (avail ? int64_t(rs) * (a.I / 32) : 0), avail ? avail : 1, lane);
            }
        }
        uint4 wv[NPASS][CPL];
        uint8_t sv[NPASS][CPL];
#pragma unroll
        for (int q = 0; q < NPASS; ++q) {
            const int r = row0 + q * RPP + g;
            const bool ok = r < a.nrows;
            const int rl = ok ? r : a.nrows - 1;     // unconditional loads (a loaded register copied inside
                                                     // a branch waits for every load): rows past the end
                                                     // reread the last row, and are not stored
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                wv[q][c] = load_w(blob + a.off_w + int64_t(rl) * row_bytes, c * LPR + lr);
                if constexpr (!kRun)
                    sv[q][c] = (WT == WT_FP4 && ok) ? blob[a.off_s + int64_t(r) * (a.I / 32) + c * LPR + lr] : uint8_t(127);
            }
        }
        if constexpr (kRun) {
            loads_issued();
#pragma unroll
            for (int q = 0; q < NPASS; ++q)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    sv[q][c] = row0 + q * RPP + g < a.nrows ? sr[q].byte(0, g * LPR * CPL + c * LPR + lr) : uint8_t(127);
        }
        auto token = [&](int p, auto&& act_chunk) {
#pragma unroll
            for (int q = 0; q < NPASS; ++q)
#pragma unroll
                for (int c = 0; c < CPL; ++c) keep_packed<WT>(wv[q][c]);
            float part[NPASS];
#pragma unroll
            for (int q = 0; q < NPASS; ++q) part[q] = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                ActChunk<WT> av;
                act_chunk(av, c);
#pragma unroll
                for (int q = 0; q < NPASS; ++q) part[q] = chunk_dot<WT>(wv[q][c], av, sv[q][c], part[q]);
            }
            const int qi = dev::group_reduce_split<NPASS, LPR>(part, lane);
            if ((lr & (LPR / NPASS - 1)) == 0)   // the value a pair-output store would write, read back
                s_o[p * RPW + qi * RPP + g] =
                    WT == WT_F32 ? part[0] : __uint_as_float(uint32_t(dev::f32_to_bf16_bits(part[0])) << 16);
        };
        if (WT != WT_FP4 && have) token(p, [&](ActChunk<WT>& av, int c) { av = av0[WT == WT_FP4 ? 0 : c]; });
        else if (have)
            token(p, [&](ActChunk<WT>& av, int c) {
                load_act<WT>(av, a.act + (int64_t(p) * a.I + int64_t(c * LPR + lr) * EPC) * AB);
            });
        while (it.next(p, t))
            token(p, [&](ActChunk<WT>& av, int c) {
                load_act<WT>(av, a.act + (int64_t(p) * a.I + int64_t(c * LPR + lr) * EPC) * AB);
            });
    }
    __syncthreads();
    if (wave == 0 && merger && mrow < a.H) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kFusedTopK; ++j) {
            const int e = mid[j];
            if (j < a.k && ((a.m.mask[e >> 5] >> (e & 31)) & 1u))
                acc = fmaf(mw[j], s_o[(mt * a.k + j) * RPW + mrl], acc);
        }
        const float sh = a.m.with_shared ? s_o[(a.T * a.k + mt) * RPW + mrl] : 0.0f;
        acc += sh;
        acc += a.m.y_host ? myh : 0.0f;
        if (WT == WT_F32)
            static_cast<float*>(a.m.out)[int64_t(mt) * a.H + mrow] = acc;
        else
            static_cast<uint16_t*>(a.m.out)[int64_t(mt) * a.H + mrow] = uint16_t(dev::pack_bf16x2(acc, 0.0f));
    }
}

// Lanes per down row (LPR) and 16-byte chunks per lane (CPL) with LPR * CPL = chunks per row.
// At most 32 lanes a row where the row allows it: the fused down + merge kernel then covers at
// least 4 rows per workgroup (v4flash bf16, 192 chunks a row, batch 1: 1 us off the 52 us step
// against 64 lanes with separate down and merge kernels), and the separate down kernel uses
// the same lanes and chunks, so both give the same bits (0.3% slower at batch 8 than 64 lanes).
bool pick_down(int d_ch, int* lpr, int* cpl) {
    for (int l : {32, 16, 64})
        for (int c : {1, 2, 3, 4, 6, 8})
            if (l * c == d_ch) { *lpr = l; *cpl = c; return true; }
    return false;
}

template <int WT, int CPL>
hipError_t launch_gu1(const DecodeArgs& a, int n_list, hipStream_t s) {
    using S = GateUpShape<CPL>;
    if (a.I % S::COLS) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_decode_gate_up<WT, CPL>), dim3(a.I / S::COLS, n_list), dim3(64 * S::WPB),
                       WT != WT_F32 ? a.nt * a.H * 2 : 0, s, a);
    return hipGetLastError();
}

template <int WT>
hipError_t launch_gu(const DecodeArgs& a, int cpl, int n_list, hipStream_t s) {
    switch (cpl) {
        case 1: return launch_gu1<WT, 1>(a, n_list, s);
        case 2: return launch_gu1<WT, 2>(a, n_list, s);
        case 4: return launch_gu1<WT, 4>(a, n_list, s);
        case 8: return launch_gu1<WT, 8>(a, n_list, s);
        default: return hipErrorInvalidValue;
    }
}

template <int WT>
hipError_t launch_d(const DecodeArgs& a, int lpr, int cpl, int n_list, hipStream_t s) {
    const int rpb = kDownPasses * (kWave / lpr) * kDownWaves;
    const dim3 grid((a.nrows + rpb - 1) / rpb, n_list);
#define MOE_D(L, C) \
    if (lpr == L && cpl == C) { \
        hipLaunchKernelGGL((k_decode_down<WT, L, C>), grid, dim3(64 * kDownWaves), WT == WT_FP4 ? a.nt * a.I * 2 : 0, \
                           s, a);                                                                                  \
        return hipGetLastError(); \
    }
#define MOE_DL(L) MOE_D(L, 1) MOE_D(L, 2) MOE_D(L, 3) MOE_D(L, 4) MOE_D(L, 6) MOE_D(L, 8)
    MOE_DL(64) MOE_DL(32) MOE_DL(16)
#undef MOE_DL
#undef MOE_D
    return hipErrorInvalidValue;
}

template <int WT>
hipError_t launch_dm(const DecodeArgs& a, int lpr, int cpl, hipStream_t s) {
    const int rpw = kDownPasses * (kWave / lpr);
    const dim3 grid((a.nrows + rpw - 1) / rpw);
#define MOE_DM(L, C) \
    if (lpr == L && cpl == C) { \
        hipLaunchKernelGGL((k_decode_down_merge<WT, L, C>), grid, dim3(64 * kFusedWaves), 0, s, a); \
        return hipGetLastError(); \
    }
#define MOE_DML(L) MOE_DM(L, 1) MOE_DM(L, 2) MOE_DM(L, 3) MOE_DM(L, 4) MOE_DM(L, 6) MOE_DM(L, 8)
    MOE_DML(64) MOE_DML(32) MOE_DML(16)
#undef MOE_DML
#undef MOE_DM
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_shape_supported(const moe_config& c) {
    const int gu = ffn::chunks_per_row(c.w_dtype, c.hidden), d = ffn::chunks_per_row(c.w_dtype, c.inter);
    int l, cc;
    // MXFP4 staging copies whole 64-lane instructions: rows of H and I bf16 are multiples of 1 KiB
    const bool stage_ok = c.w_dtype != MOE_W_MXFP4 || (c.hidden % 512 == 0 && c.inter % 512 == 0);
    return c.inter % 16 == 0 && gu % kWave == 0 && (gu / kWave == 1 || gu / kWave == 2 || gu / kWave == 4 ||
                                                     gu / kWave == 8) && pick_down(d, &l, &cc) && stage_ok;
}

// Activation rows staged per group: the most tokens any listed expert takes, within a
// 32 KiB LDS budget per workgroup.
static int staged_rows(const DecodeList& list, int K) {
    int most = 1;
    for (int i = 0; i < list.n; ++i) most = std::max(most, __builtin_popcount(list.tokmask[i]));
    return std::max(1, std::min(most, (32 << 10) / (2 * K)));
}

// o != null: gate/up, then down into the pair outputs o; else gate/up, then the fused
// down + merge into out.
static hipError_t launch_ffn_decode_impl(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                                         const void* slot_base, const void* shared, const DecodeList& list, void* o,
                                         void* ws, hipStream_t s, const int32_t* ids, const float* w,
                                         const uint32_t* mask, int32_t with_shared, const float* y_host, void* out) {
    const int gu_ch = ffn::chunks_per_row(c.w_dtype, c.hidden), d_ch = ffn::chunks_per_row(c.w_dtype, c.inter);
    int lpr, cpld;
    if (!pick_down(d_ch, &lpr, &cpld)) return hipErrorInvalidValue;
    const WsLayout W = ws_layout(c, T);
    uint8_t* hbuf = static_cast<uint8_t*>(ws) + W.h;
    DecodeArgs a;
    a.slot_base = static_cast<const uint8_t*>(slot_base);
    a.shared_blob = static_cast<const uint8_t*>(shared);
    a.blob_bytes = lay.bytes;
    a.T = T;
    a.k = c.top_k;
    a.I = c.inter;
    a.H = c.hidden;
    // Entries with the most tokens first: workgroups start in blockIdx.y order, and an
    // expert's workgroups take time in proportion to its tokens (the shared expert has all
    // of them), so last in line they would form the kernel's tail.
    int order[kMaxDecodeList];
    for (int i = 0; i < list.n; ++i) order[i] = i;
    std::stable_sort(order, order + list.n, [&](int x, int y) {
        return __builtin_popcount(list.tokmask[x]) > __builtin_popcount(list.tokmask[y]);
    });
    a.list.n = list.n;
    for (int i = 0; i < list.n; ++i) {
        a.list.ent[i] = list.ent[order[i]];
        a.list.tokmask[i] = list.tokmask[order[i]];
        a.list.jpack[i] = list.jpack[order[i]];
    }
    a.off_w = lay.gu;
    a.off_s = lay.gu_scale;
    a.act = static_cast<const uint8_t*>(x);
    a.out = hbuf;
    a.K = c.hidden;
    a.nrows = 2 * c.inter;
    a.nt = staged_rows(list, c.hidden);
    hipError_t e;
    switch (c.w_dtype) {
        case MOE_W_F32: e = launch_gu<WT_F32>(a, gu_ch / kWave, list.n, s); break;
        case MOE_W_BF16: e = launch_gu<WT_BF16>(a, gu_ch / kWave, list.n, s); break;
        default: e = launch_gu<WT_FP4>(a, gu_ch / kWave, list.n, s); break;
    }
    if (e != hipSuccess) return e;
    a.off_w = lay.d;
    a.off_s = lay.d_scale;
    a.act = hbuf;
    a.out = static_cast<uint8_t*>(o);
    a.K = c.inter;
    a.nrows = c.hidden;
    a.nt = staged_rows(list, c.inter);
    if (!o) {
        a.m.ids = ids;
        a.m.w = w;
        a.m.y_host = y_host;
        a.m.out = out;
        for (int i = 0; i < kMaxExperts / 32; ++i) a.m.mask[i] = mask[i];
        a.m.with_shared = with_shared;
        switch (c.w_dtype) {
            case MOE_W_F32: return launch_dm<WT_F32>(a, lpr, cpld, s);
            case MOE_W_BF16: return launch_dm<WT_BF16>(a, lpr, cpld, s);
            default: return launch_dm<WT_FP4>(a, lpr, cpld, s);
        }
    }
    switch (c.w_dtype) {
        case MOE_W_F32: return launch_d<WT_F32>(a, lpr, cpld, list.n, s);
        case MOE_W_BF16: return launch_d<WT_BF16>(a, lpr, cpld, list.n, s);
        default: return launch_d<WT_FP4>(a, lpr, cpld, list.n, s);
    }
}

hipError_t launch_ffn_decode_merge(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                                   const void* slot_base, const void* shared, const DecodeList& list,
                                   const int32_t* ids, const float* w, const uint32_t* mask, int32_t with_shared,
                                   const float* y_host, void* out, void* ws, hipStream_t s) {
    // The fused kernel when every wave takes one entry and a workgroup covers at least 4
    // output rows (at most 32 lanes per down row; rows of 192 chunks, bf16 with I = 1536, run
    // 32 lanes of 6 chunks).  Measured on MI355X: with more entries a wave takes several
    // experts one after another, and with 2 rows per workgroup (64 lanes per row) the
    // per-workgroup merge outweighs the saved launch; both run slower fused than the separate
    // down and merge kernels (pair outputs in the workspace).
    // no listed expert has a token (and no shared expert): the output is the host part, or zero
    if (list.n == 0) return launch_merge(c, nullptr, ids, w, mask, 0, y_host, T, out, s);
    int lpr = 64, cpl = 0;
    pick_down(ffn::chunks_per_row(c.w_dtype, c.inter), &lpr, &cpl);
    if (list.n <= kFusedWaves && c.top_k <= kFusedTopK && lpr <= 32)
        return launch_ffn_decode_impl(c, lay, x, T, slot_base, shared, list, nullptr, ws, s, ids, w, mask,
                                      with_shared, y_host, out);
    void* o = static_cast<uint8_t*>(ws) + ws_layout(c, T).o;
    hipError_t e = launch_ffn_decode_impl(c, lay, x, T, slot_base, shared, list, o, ws, s, nullptr, nullptr, nullptr,
                                          0, nullptr, nullptr);
    if (e != hipSuccess) return e;
    return launch_merge(c, o, ids, w, mask, with_shared, y_host, T, out, s);
}

hipError_t launch_ffn_decode(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                             const void* slot_base, const void* shared, const DecodeList& list, void* o, void* ws,
                             hipStream_t s) {
    if (list.n == 0) return hipSuccess;       // no listed expert has a token: no pair output to write
    return launch_ffn_decode_impl(c, lay, x, T, slot_base, shared, list, o, ws, s, nullptr, nullptr, nullptr, 0,
                                  nullptr, nullptr);
}

}  // namespace moe

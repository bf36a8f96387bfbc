// Decode expert FFN (T <= 8 tokens): batched GEMV over the expert slots (gfx950).
//
// Decode reads every weight of every selected expert once per step while only a
// handful of tokens use it, so the work is bound by HBM bandwidth, not by the
// matrix cores.  Each lane streams 16-byte chunks of weight rows into registers
// (consecutive lanes read consecutive chunks: 1 KiB per wave load), the tokens
// routed to the expert are then applied to the registers, and the row sums are
// reduced across the lanes of a row with a halving shuffle exchange.
//
// Two launches per call:
//   gate/up: rows of the interleaved [2I][H] matrix; a workgroup owns one block of
//            16 gate rows and the 16 matching up rows and writes
//            h = silu(gate) * up for its 16 columns (bf16, or fp32 for fp32 weights);
//   down:    rows of [H][I]; o[p][row] = Wd[row] . h[p] in fp32.
// The SwiGLU expert and the silu form follow the layer definition used throughout
// (banandre.com, "The 284B Model on a 32GB GPU Trick", section "Sparsity Is a
// Lie": experts are small feed-forward networks).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ffn_common.h"
#include "internal.h"

namespace moe {
namespace {

using dev::kWave;

using namespace ffn;

struct GemvArgs {
    const uint8_t* slot_base;
    const uint8_t* shared_blob;
    int64_t blob_bytes;
    int64_t off_w;       // matrix offset inside a blob
    int64_t off_s;       // MXFP4 scale offset inside a blob
    const uint8_t* act;  // gate/up: x [T][H]; down: h [pair rows][I]
    uint8_t* out;        // gate/up: h [pair rows][I]; down: o fp32 [pair rows][H]
    const int32_t* offsets;
    const int32_t* perm;
    int32_t K;           // row length in elements
    int32_t nrows;       // rows of the matrix
    int32_t T, k, I, H;
    ExpertList list;
};

constexpr int kMaxBatch = 8;  // tokens buffered between workgroup barriers (gate/up)

// LPR: lanes per row; CPL: 16-byte chunks per lane per row (row = LPR*CPL chunks);
// RPW: rows per wave; GU: gate/up mode (else down mode).
template <int WT, int LPR, int CPL, int RPW, bool GU>
__global__ void __launch_bounds__(GU ? 64 * (32 / RPW) : 256)
k_gemv(const GemvArgs a) {
    constexpr int EPC = Fmt<WT>::EPC;
    constexpr int ROWS_PER_PASS = kWave / LPR;
    constexpr int NPASS = RPW / ROWS_PER_PASS;
    constexpr int WAVES = GU ? 32 / RPW : 4;
    constexpr int RPB = WAVES * RPW;
    static_assert(NPASS >= 1 && NPASS <= LPR, "pass layout");
    constexpr int ACT_CHUNK_BYTES = EPC * Fmt<WT>::ABYTES;

    __shared__ float s_sum[GU ? kMaxBatch : 1][GU ? 32 : 1];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int g = lane / LPR, lr = lane % LPR;
    const int entry = a.list.ent[blockIdx.y];
    const int e = entry & 1023;
    const bool shared = e == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    const int64_t row_bytes = int64_t(a.K) * (WT == WT_F32 ? 4 : WT == WT_BF16 ? 2 : 1) / (WT == WT_FP4 ? 2 : 1);
    const int row0 = blockIdx.x * RPB + wave * RPW;

    // ---- stream this wave's weight rows into registers ----
    uint4 wv[NPASS][CPL];
    uint8_t sv[NPASS][CPL];
#pragma unroll
    for (int q = 0; q < NPASS; ++q) {
        const int row = row0 + q * ROWS_PER_PASS + g;
        const bool ok = row < a.nrows;
        const dev::u32x4* rp = reinterpret_cast<const dev::u32x4*>(blob + a.off_w + int64_t(row) * row_bytes);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            if (ok) {
                const dev::u32x4 t = __builtin_nontemporal_load(rp + c * LPR + lr);
                wv[q][c] = make_uint4(t.x, t.y, t.z, t.w);
            } else {
                wv[q][c] = make_uint4(0, 0, 0, 0);
            }
            if (WT == WT_FP4)
                sv[q][c] = ok ? blob[a.off_s + int64_t(row) * (a.K / 32) + c * LPR + lr] : uint8_t(127);
            else
                sv[q][c] = 0;
        }
    }

    // ---- tokens routed to this expert ----
    int cnt, base = 0;
    if (shared) {
        cnt = a.T;
    } else {
        base = a.offsets[e];
        cnt = a.offsets[e + 1] - base;
    }
    const int64_t act_stride = int64_t(GU ? a.H : a.I) * Fmt<WT>::ABYTES;
    for (int b0 = 0; b0 < cnt; b0 += kMaxBatch) {
        const int nb = min(kMaxBatch, cnt - b0);
        for (int bi = 0; bi < nb; ++bi) {
            const int i = b0 + bi;
            const int p = shared ? a.T * a.k + i : a.perm[base + i];
            const int arow = GU ? (shared ? i : p / a.k) : p;
            const uint8_t* ap = a.act + int64_t(arow) * act_stride;
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
                load_act<WT>(av, ap + int64_t(c * LPR + lr) * ACT_CHUNK_BYTES);
#pragma unroll
                for (int q = 0; q < NPASS; ++q) part[q] = chunk_dot<WT>(wv[q][c], av, sv[q][c], part[q]);
            }
            const int qi = dev::group_reduce_split<NPASS, LPR>(part, lane);
            const bool writer = (lr & (LPR / NPASS - 1)) == 0;
            const int row = row0 + qi * ROWS_PER_PASS + g;
            if (writer) {
                if (GU) {
                    s_sum[bi][row - blockIdx.x * RPB] = part[0];
                } else if (row < a.nrows) {
                    store_act<WT>(a.out, int64_t(p) * a.H + row, part[0]);
                }
            }
        }
        if (GU) {
            __syncthreads();
            // h for the block's 16 intermediate columns: gate row r, up row r + 16
            for (int idx = tid; idx < nb * 16; idx += WAVES * kWave) {
                const int bi = idx / 16, r = idx % 16;
                const int i = b0 + bi;
                const int p = shared ? a.T * a.k + i : a.perm[base + i];
                const float hv = silu(s_sum[bi][r]) * s_sum[bi][r + 16];
                const int64_t col = int64_t(blockIdx.x) * 16 + r;
                store_act<WT>(a.out, int64_t(p) * a.I + col, hv);
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------- dispatch
struct Variant {
    int lpr, cpl;
};

bool pick(int nch, Variant* v) {
    static const int lprs[3] = {64, 32, 16};
    static const int cpls[6] = {1, 2, 3, 4, 6, 8};
    for (int li = 0; li < 3; ++li)
        for (int ci = 0; ci < 6; ++ci)
            if (lprs[li] * cpls[ci] == nch) { *v = {lprs[li], cpls[ci]}; return true; }
    return false;
}

template <int WT, int LPR, int CPL, bool GU>
hipError_t launch_one(const GemvArgs& a, dim3 grid, hipStream_t s) {
    constexpr int RPW = CPL <= 4 ? 8 : 4;
    constexpr int WAVES = GU ? 32 / RPW : 4;
    hipLaunchKernelGGL((k_gemv<WT, LPR, CPL, RPW, GU>), grid, dim3(WAVES * kWave), 0, s, a);
    return hipGetLastError();
}

template <int WT, bool GU>
hipError_t launch_variant(const GemvArgs& a, Variant v, int n_list, hipStream_t s) {
    const int rpw = v.cpl <= 4 ? 8 : 4;
    const int rpb = GU ? 32 : 4 * rpw;
    const dim3 grid((a.nrows + rpb - 1) / rpb, n_list);
#define MOE_GEMV_CASE(L, C) \
    if (v.lpr == L && v.cpl == C) return launch_one<WT, L, C, GU>(a, grid, s);
#define MOE_GEMV_LPR(L) \
    MOE_GEMV_CASE(L, 1) MOE_GEMV_CASE(L, 2) MOE_GEMV_CASE(L, 3) MOE_GEMV_CASE(L, 4) MOE_GEMV_CASE(L, 6) MOE_GEMV_CASE(L, 8)
    MOE_GEMV_LPR(64)
    MOE_GEMV_LPR(32)
    MOE_GEMV_LPR(16)
#undef MOE_GEMV_LPR
#undef MOE_GEMV_CASE
    return hipErrorInvalidValue;
}

template <bool GU>
hipError_t launch_wt(int wt, const GemvArgs& a, Variant v, int n_list, hipStream_t s) {
    switch (wt) {
        case WT_F32: return launch_variant<WT_F32, GU>(a, v, n_list, s);
        case WT_BF16: return launch_variant<WT_BF16, GU>(a, v, n_list, s);
        default: return launch_variant<WT_FP4, GU>(a, v, n_list, s);
    }
}

}  // namespace

bool gemv_shape_supported(const moe_config& c) {
    Variant v;
    return pick(chunks_per_row(c.w_dtype, c.hidden), &v) && pick(chunks_per_row(c.w_dtype, c.inter), &v) &&
           c.inter % 16 == 0;
}

hipError_t launch_ffn_gemv(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                           const int32_t* offsets, const int32_t* perm, const void* slot_base,
                           const void* shared, const ExpertList& list, void* o, void* ws, hipStream_t s) {
    Variant vgu, vd;
    if (!pick(chunks_per_row(c.w_dtype, c.hidden), &vgu) || !pick(chunks_per_row(c.w_dtype, c.inter), &vd))
        return hipErrorInvalidValue;
    const WsLayout W = ws_layout(c, T);
    uint8_t* hbuf = static_cast<uint8_t*>(ws) + W.h;
    GemvArgs a;
    a.slot_base = static_cast<const uint8_t*>(slot_base);
    a.shared_blob = static_cast<const uint8_t*>(shared);
    a.blob_bytes = lay.bytes;
    a.offsets = offsets;
    a.perm = perm;
    a.T = T;
    a.k = c.top_k;
    a.I = c.inter;
    a.H = c.hidden;
    a.list = list;
    // gate/up
    a.off_w = lay.gu;
    a.off_s = lay.gu_scale;
    a.act = static_cast<const uint8_t*>(x);
    a.out = hbuf;
    a.K = c.hidden;
    a.nrows = 2 * c.inter;
    hipError_t e = launch_wt<true>(c.w_dtype, a, vgu, list.n, s);
    if (e != hipSuccess) return e;
    // down
    a.off_w = lay.d;
    a.off_s = lay.d_scale;
    a.act = hbuf;
    a.out = static_cast<uint8_t*>(o);
    a.K = c.inter;
    a.nrows = c.hidden;
    return launch_wt<false>(c.w_dtype, a, vd, list.n, s);
}

}  // namespace moe

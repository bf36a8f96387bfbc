// Prefill expert FFN (T > 8 tokens): grouped GEMM on MFMA (gfx950).
//
// Prefill routes thousands of tokens to nearly every expert (banandre.com, "The
// 284B Model on a 32GB GPU Trick", section "The Three Failure Modes of Existing
// Engines"), so each expert's work is a dense product over the rows routed to it.
// Pairs are grouped by expert (moe_route's stable permutation); per expert
//   GEMM 1:  G = A_e . Wgu^T  (A_e = x rows of the expert's pairs, gathered)
//            epilogue h = silu(gate) * up, stored as bf16 at the pair's sorted row;
//   GEMM 2:  O = h_e . Wd^T, accumulated in fp32 and stored as bf16 at the pair's row
//            p = perm[pos] (the merge reads the pair outputs).
// bf16 operands and fp32 accumulation on v_mfma_f32_32x32x16_bf16; MXFP4 weights are
// decoded to bf16 operands (exactly) on their way from LDS to the MFMAs.
//
// Four kernels, chosen per GEMM from N and K:
//   k_gemm_big  persistent 256 x 256 tiles, K slices of 64 loaded straight into two LDS
//               stages (bf16 GEMMs with K >= 512, and every MXFP4 GEMM whose tile scales
//               fit its LDS region);
//   k_gemm_b3   persistent 128 x 256 tiles, K slices of 64 in a ring of three LDS stages
//               (bf16 GEMMs with K = 256 or 384);
//   k_gemm_dma  128 x 256 tiles, a ring of 3 stages of K = 32 loaded straight into LDS, two
//               workgroups per CU (bf16 GEMMs with K = 64 or 128);
//   k_gemm      register-staged tiles (MXFP4 shapes the large tile does not take).
// Gate and up rows are interleaved in blocks of 16 in the weight layout, so the gate and up
// values of a column are one lane exchange apart in a 32-wide fragment and the SwiGLU
// epilogue needs no extra pass.  Tiles are numbered expert-major and each of the 8 XCDs takes
// a contiguous range of the real tile count, so the A rows and weights of an expert are
// re-read from that XCD's L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "ffn_common.h"
#include "internal.h"

namespace moe {
namespace {

using dev::kWave;

// Tile configuration (chosen by measurement on MI355X; see the kernel comment).
#ifndef MOE_GEMM_BM
#define MOE_GEMM_BM 128
#endif
#ifndef MOE_GEMM_BN
#define MOE_GEMM_BN 256
#endif
#ifndef MOE_GEMM_WM
#define MOE_GEMM_WM 2
#endif
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN 4
#endif
#ifndef MOE_GEMM_MF
#define MOE_GEMM_MF 32
#endif
#ifndef MOE_GEMM_DB
#define MOE_GEMM_DB 0
#endif
constexpr int BM = MOE_GEMM_BM, BN = MOE_GEMM_BN, BK = 64;
constexpr int WM = MOE_GEMM_WM, WN = MOE_GEMM_WN;   // wave grid
constexpr int MF = MOE_GEMM_MF;                     // MFMA tile: 16 (16x16x32) or 32 (32x32x16)
constexpr bool DB = MOE_GEMM_DB;                    // two LDS stages, one barrier per K step
constexpr int KMF = MF == 16 ? 32 : 16;             // K per MFMA
constexpr int NACC = MF == 16 ? 4 : 16;             // accumulator floats per lane per tile
constexpr int kThreads = WM * WN * 64;
constexpr int TM = BM / WM, TN = BN / WN;           // wave tile
constexpr int FM = TM / MF, FN = TN / MF;           // MFMA tiles per wave
constexpr int ACH = BM * 8 / kThreads;              // 16-byte A chunks per thread per K step
constexpr int FCH = BN * 2 / kThreads > 0 ? BN * 2 / kThreads : 1;  // MXFP4 code chunks per thread
constexpr int LDS_STRIDE = BK + 8;                  // bf16 elements per LDS row (16-byte pad)
constexpr int kStages = DB ? 2 : 1;
constexpr int kLdsBytes = kStages * (BM + BN) * LDS_STRIDE * 2;
constexpr int kXcds = 8;
static_assert(ACH * kThreads == BM * 8 && FCH * kThreads >= BN * 2, "chunking");
static_assert(FM * MF == TM && FN * MF == TN, "wave tile");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
template <int M> struct AccT;
template <> struct AccT<16> { typedef f32x4 T; };
template <> struct AccT<32> { typedef f32x16 T; };

struct TileMapArgs {
    const int32_t* offsets;
    int32_t T, bm;            // bm: row-tile height of the GEMM kernel that reads the list
    int32_t* tiles;   // [0]: count, then (entry << 16) | m_tile
    int4* rec;        // per row tile: list entry, first row (in perm order), rows, m_tile
    ExpertList list;
};

// Tiles of every listed expert in list order: ceil(rows / bm) m-tiles each.
__global__ void __launch_bounds__(1024) k_tile_map(const TileMapArgs a) {
    __shared__ int32_t s_cnt[kMaxExperts + 1];
    __shared__ int32_t s_base[kMaxExperts + 2];
    const int tid = threadIdx.x;
    const int n = a.list.n;
    for (int i = tid; i < n; i += blockDim.x) {
        const int e = a.list.ent[i] & 1023;
        const int rows = e == kSharedTag ? a.T : a.offsets[e + 1] - a.offsets[e];
        s_cnt[i] = (rows + a.bm - 1) / a.bm;
    }
    __syncthreads();
    if (tid < kWave) {                        // exclusive scan, 9 entries per lane
        constexpr int kPer = (kMaxExperts + 1 + kWave - 1) / kWave;
        int loc[kPer], sum = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = tid * kPer + q;
            loc[q] = i < n ? s_cnt[i] : 0;
            sum += loc[q];
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int v = __shfl_up(incl, d, kWave);
            if (tid >= d) incl += v;
        }
        int run = incl - sum;
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int i = tid * kPer + q;
            if (i < n) s_base[i] = run;
            run += loc[q];
        }
        if (tid == kWave - 1) {
            s_base[n] = run;
            a.tiles[0] = run;
        }
    }
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
        const int ent = a.list.ent[i], e = ent & 1023;
        const int base = e == kSharedTag ? 0 : a.offsets[e];
        const int rows = e == kSharedTag ? a.T : a.offsets[e + 1] - base;
        for (int m = 0; m < s_cnt[i]; ++m) {
            a.tiles[1 + s_base[i] + m] = (i << 16) | m;
            a.rec[s_base[i] + m] = make_int4(ent, base, rows, m);
        }
    }
}

struct GemmArgs {
    const uint8_t* slot_base;
    const uint8_t* shared_blob;
    int64_t blob_bytes;
    int64_t off_w, off_s;      // weight matrix (and MXFP4 scales) inside a blob
    const uint8_t* a_src;      // GEMM 1: x [T][H] bf16; GEMM 2: h [rows][I] bf16
    void* out;                 // GEMM 1: h bf16 [rows][I]; GEMM 2: o bf16 [pair rows][H]
    const int32_t* offsets;
    const int32_t* perm;
    const int32_t* tiles;
    const int4* rec;           // per row tile: list entry, first row, rows, m_tile (one load)
    int32_t T, k, K, N;        // K: reduction length, N: output columns of the matrix
    int32_t I, H;
    int32_t grid;              // launched workgroups (a multiple of the XCD count)
    int32_t mode;              // 0: GEMM 1 (A rows gathered from x), 1: GEMM 2 (A = h)
    ExpertList list;
};

// Logical tile of workgroup b, or -1.  The real tile count (the list's row tiles times
// the column tiles) is cut into kXcds contiguous ranges, one per XCD (workgroups are dealt
// round-robin to the XCDs), so each XCD's L2 holds the A rows and weights of a few
// experts at a time and every XCD gets an equal share.  The grid is sized for the most
// row tiles a list can have; the workgroups past an XCD's share exit at once.
__device__ __forceinline__ int xcd_tile(int b, int n_slots, int n_tiles) {
    const int total = n_slots * n_tiles;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int i = b / kXcds;
    const int lid = (b % kXcds) * per_xcd + i;
    return i < per_xcd && lid < total ? lid : -1;
}

// MXFP4 -> bf16 of 32 elements (16 code bytes) with the block scale folded in.
__device__ __forceinline__ void fp4_to_bf16(const uint4 codes, uint8_t s, uint4 out[4]) {
    const float sc = s ? __uint_as_float(uint32_t(s) << 23) : __uint_as_float(0x00400000u);
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const dev::bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 0);
        const dev::bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 1);
        const dev::bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 2);
        const dev::bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[q], sc, 3);
        out[q] = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                            __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
    }
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t bf16_bits(float v) { return uint16_t(dev::pack_bf16x2(v, 0.0f)); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Register-staged GEMM for MXFP4 weights at shapes the large-tile kernel does not take
// (K above the LDS room for a tile's scales, or K not a multiple of 128; bf16 weights always
// run the pipelined or large-tile kernels).  MODE 0: gate/up GEMM with SwiGLU epilogue;
// MODE 1: down GEMM.  WM x WN waves, each TM x TN = FM x FN MFMA tiles.  The next K step's
// global tiles (A rows, weight codes and scales) are loaded into registers while the
// current LDS stage is consumed; the codes are dequantised to bf16 on their way into LDS.
template <int MODE>
__global__ void __launch_bounds__(kThreads) k_gemm(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t* As = lds;                                 // [stages][BM][LDS_STRIDE]
    uint16_t* Bs = lds + kStages * BM * LDS_STRIDE;     // [stages][BN][LDS_STRIDE]
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / WN, wn = wave % WN;

    const int n_tiles = a.N / BN;
    const int lid = xcd_tile(blockIdx.x, a.tiles[0], n_tiles);
    if (lid < 0) return;
    const int slot = lid / n_tiles, nt = lid % n_tiles;
    const int tinfo = a.tiles[1 + slot];
    const int ei = tinfo >> 16, mt = tinfo & 0xFFFF;
    const int entry = a.list.ent[ei];
    const int e = entry & 1023;
    const bool shared = e == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    const int base = shared ? 0 : a.offsets[e];
    const int rows = shared ? a.T : a.offsets[e + 1] - base;
    const int m0 = mt * BM, n0 = nt * BN;
    const int K = a.K;

    // ---- per K step each thread moves ACH 16-byte chunks of A (row = c / 8, column c % 8) and FCH
    //      16-byte runs of weight codes with their scale bytes (row = c / 2, half c % 2)
    const uint8_t* arow[ACH];
    bool avalid[ACH];
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int c = tid + kThreads * i;
        const int r = c / 8;
        avalid[i] = m0 + r < rows;
        int64_t src_row = 0;
        if (avalid[i]) {
            if (MODE == 0)
                src_row = shared ? (m0 + r) : a.perm[base + m0 + r] / a.k;        // token of the pair
            else
                src_row = shared ? int64_t(a.T) * a.k + m0 + r : base + m0 + r;  // h row
        }
        arow[i] = a.a_src + src_row * int64_t(K) * 2 + (c % 8) * 16;
    }
    const int64_t wrow_bytes = K / 2;
    const uint8_t* wbase = blob + a.off_w;
    const uint8_t* sbase = blob + a.off_s;

    uint4 ra[ACH];
    uint4 rbq[FCH];
    uint8_t rbs[FCH];

#define MOE_GEMM_LOAD(k0)                                                                                    \
    {                                                                                                        \
        _Pragma("unroll") for (int i = 0; i < ACH; ++i) ra[i] =                                              \
            avalid[i] ? *reinterpret_cast<const uint4*>(arow[i] + int64_t(k0) * 2) : make_uint4(0, 0, 0, 0); \
        _Pragma("unroll") for (int i = 0; i < FCH; ++i) {                                                    \
            const int c = tid + kThreads * i, r = c >> 1, half = c & 1;                                      \
            if (c < BN * 2) {                                                                                \
                rbq[i] = *reinterpret_cast<const uint4*>(wbase + int64_t(n0 + r) * wrow_bytes + (k0) / 2 + half * 16); \
                rbs[i] = sbase[int64_t(n0 + r) * (K / 32) + (k0) / 32 + half];                               \
            }                                                                                                \
        }                                                                                                    \
    }
#define MOE_GEMM_STORE(st)                                                                                   \
    {                                                                                                        \
        uint16_t* as_ = As + (st) * BM * LDS_STRIDE;                                                         \
        uint16_t* bs_ = Bs + (st) * BN * LDS_STRIDE;                                                         \
        _Pragma("unroll") for (int i = 0; i < ACH; ++i) {                                                    \
            const int c = tid + kThreads * i;                                                                \
            *reinterpret_cast<uint4*>(&as_[(c / 8) * LDS_STRIDE + (c % 8) * 8]) = ra[i];                     \
        }                                                                                                    \
        _Pragma("unroll") for (int i = 0; i < FCH; ++i) {                                                    \
            const int c = tid + kThreads * i, r = c >> 1, half = c & 1;                                      \
            if (c < BN * 2) {                                                                                \
                uint4 v[4];                                                                                  \
                fp4_to_bf16(rbq[i], rbs[i], v);                                                              \
                _Pragma("unroll") for (int q = 0; q < 4; ++q)                                                \
                    *reinterpret_cast<uint4*>(&bs_[r * LDS_STRIDE + half * 32 + q * 8]) = v[q];              \
            }                                                                                                \
        }                                                                                                    \
    }

    typename AccT<MF>::T acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < NACC; ++q) acc[i][j][q] = 0.0f;

#define MOE_GEMM_COMPUTE(st)                                                                                 \
    {                                                                                                        \
        const uint16_t* as_ = As + (st) * BM * LDS_STRIDE;                                                   \
        const uint16_t* bs_ = Bs + (st) * BN * LDS_STRIDE;                                                   \
        _Pragma("unroll") for (int kk = 0; kk < BK / KMF; ++kk) {                                            \
            bf16x8 af[FM], bfr[FN];                                                                          \
            const int kc = kk * KMF + (lane / MF) * 8;                                                       \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) af[i] =                                           \
                *reinterpret_cast<const bf16x8*>(&as_[(wm * TM + i * MF + lane % MF) * LDS_STRIDE + kc]);    \
            _Pragma("unroll") for (int j = 0; j < FN; ++j) bfr[j] =                                          \
                *reinterpret_cast<const bf16x8*>(&bs_[(wn * TN + j * MF + lane % MF) * LDS_STRIDE + kc]);    \
            _Pragma("unroll") for (int i = 0; i < FM; ++i) _Pragma("unroll") for (int j = 0; j < FN; ++j)    \
                acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);                                                  \
        }                                                                                                    \
    }

    const int nk = K / BK;
    if (DB) {
        MOE_GEMM_LOAD(0)
        MOE_GEMM_STORE(0)
        __syncthreads();
        for (int ks = 0; ks < nk; ++ks) {
            const int st = ks & 1;
            if (ks + 1 < nk) MOE_GEMM_LOAD((ks + 1) * BK)
            MOE_GEMM_COMPUTE(st)
            if (ks + 1 < nk) MOE_GEMM_STORE(st ^ 1)
            __syncthreads();
        }
    } else {
        MOE_GEMM_LOAD(0)
        for (int ks = 0; ks < nk; ++ks) {
            __syncthreads();                 // previous step's LDS reads are done
            MOE_GEMM_STORE(0)
            __syncthreads();
            if (ks + 1 < nk) MOE_GEMM_LOAD((ks + 1) * BK)
            MOE_GEMM_COMPUTE(0)
        }
    }
#undef MOE_GEMM_COMPUTE
#undef MOE_GEMM_LOAD
#undef MOE_GEMM_STORE

    // ---- epilogue.  MF = 16: lane holds column lane%16, value q at row (lane/16)*4 + q.
    //      MF = 32: lane holds column lane%32, value q at row 8*(q/4) + (lane/32)*4 + q%4.
    auto row_of = [&](int i, int q) {
        return MF == 16 ? m0 + wm * TM + i * 16 + (lane / 16) * 4 + q
                        : m0 + wm * TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
    };
    if (MODE == 0) {
        // gate/up interleave of 16: a 16-wide tile pair (MF=16) or one 32-wide tile (MF=32)
        // holds the gate and up values of 16 intermediate columns
        uint16_t* h = static_cast<uint16_t*>(a.out);
        if (MF == 16) {
#pragma unroll
            for (int jj = 0; jj < FN / 2; ++jj) {
                const int col = (n0 + wn * TN + jj * 32) / 32 * 16 + lane % 16;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int q = 0; q < NACC; ++q) {
                        const int row = row_of(i, q);
                        if (row < rows) {
                            const int64_t hrow = shared ? int64_t(a.T) * a.k + row : base + row;
                            h[hrow * a.I + col] = dev::f32_to_bf16_bits(ffn::silu_fast(acc[i][2 * jj][q]) * acc[i][2 * jj + 1][q]);
                        }
                    }
            }
        } else {
            const bool gate_lane = (lane % 32) < 16;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = (n0 + wn * TN + j * 32) / 32 * 16 + lane % 16;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int q = 0; q < NACC; ++q) {
                        const float up = __shfl_xor(acc[i][j][q], 16, kWave);
                        const int row = row_of(i, q);
                        if (gate_lane && row < rows) {
                            const int64_t hrow = shared ? int64_t(a.T) * a.k + row : base + row;
                            h[hrow * a.I + col] = dev::f32_to_bf16_bits(ffn::silu_fast(acc[i][j][q]) * up);
                        }
                    }
            }
        }
    } else {
        uint16_t* o = static_cast<uint16_t*>(a.out);       // pair outputs, bf16
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int q = 0; q < NACC; ++q) {
                const int row = row_of(i, q);
                if (row < rows) {
                    const int64_t p = shared ? int64_t(a.T) * a.k + row : a.perm[base + row];
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        o[p * a.H + n0 + wn * TN + j * MF + lane % MF] = dev::f32_to_bf16_bits(acc[i][j][q]);
                }
            }
    }
}

// ---------------------------------------------------------------- pipelined bf16 GEMM
// Direct global->LDS loads (global_load_lds_dwordx4: lane i of a wave writes 16
// bytes at the wave's LDS base + 16 i) into a ring of NSTAGE stages of BK = 32, so
// the loads run NSTAGE - 1 steps ahead of the MFMAs and need no staging registers.
// LDS rows are 64 bytes (4 chunks of 8 bf16); chunk c of row r is stored at slot
// c ^ ((r >> 2) & 3), which keeps the 16 lanes of a fragment read on distinct banks.
// A rows past the expert's end load row 0 of the expert (their outputs are dropped).
#ifndef MOE_DMA_BM
#define MOE_DMA_BM MOE_GEMM_BM
#endif
#ifndef MOE_DMA_BN
#define MOE_DMA_BN 256
#endif
#ifndef MOE_DMA_STAGES
#define MOE_DMA_STAGES 3
#endif
#ifndef MOE_DMA_BK
#define MOE_DMA_BK 32
#endif
#ifndef MOE_DMA_WSKIP
#define MOE_DMA_WSKIP 1
#endif
#ifndef MOE_DMA_WM
#define MOE_DMA_WM 2
#endif
#ifndef MOE_DMA_WN
#define MOE_DMA_WN 4
#endif
#ifndef MOE_DMA_NMAJOR
#define MOE_DMA_NMAJOR 0
#endif
namespace dma {
constexpr int BM = MOE_DMA_BM, BN = MOE_DMA_BN, WM = MOE_DMA_WM, WN = MOE_DMA_WN, MF = 32, BK = MOE_DMA_BK,
              NSTAGE = MOE_DMA_STAGES;
constexpr int kThreads = WM * WN * 64, NW = WM * WN;
constexpr int TM = BM / WM, TN = BN / WN, FM = TM / MF, FN = TN / MF;
constexpr int ROWB = BK * 2;                              // bytes per LDS row
constexpr int CPR = ROWB / 16;                            // 16-byte chunks per row
static_assert(CPR == 4 || CPR == 8, "K slice of 32 or 64");
constexpr int STAGE_BYTES = (BM + BN) * ROWB;
constexpr int Q = (BM + BN) * ROWB / 1024 / NW;           // 1 KiB load instructions per wave per stage
constexpr int kStageLds = NSTAGE * STAGE_BYTES;
// Epilogue staging.  GEMM 1: the tile's h values, BM rows of BN/2 bf16; the row stride is
// 16 bytes past a multiple of 64 so the four rows one store instruction touches fall in
// different bank groups.  GEMM 2: fp32 rows in passes of PR rows (stride 32 bytes past a
// multiple of 64: the two rows of one store land in opposite bank halves) and the rows'
// destinations.  The staging may not push the workgroup past the LDS that keeps its
// occupancy (80 KiB when the stages allow two workgroups per CU, else 160 KiB).
constexpr int HSTR = BN + 16;
constexpr int OSTR = BN * 4 + 32;
constexpr int kLdsCap = kStageLds <= 80 * 1024 ? 80 * 1024 : 160 * 1024;
constexpr int pass_rows() {
    int pr = BM;
    while (pr > 32 && pr * OSTR + BM * 4 > (kStageLds > kLdsCap ? kStageLds : kLdsCap)) pr /= 2;
    return pr;
}
constexpr int PR = pass_rows();
constexpr int kEpiLds = BM * HSTR > PR * OSTR + BM * 4 ? BM * HSTR : PR * OSTR + BM * 4;
constexpr int kLdsBytes = kStageLds > kEpiLds ? kStageLds : kEpiLds;
static_assert(PR % 32 == 0 && BM % PR == 0, "epilogue passes hold whole fragments");
static_assert(Q * NW * 1024 == STAGE_BYTES, "stage split");
static_assert(FM * MF == TM && FN * MF == TN, "wave tile");
static_assert((NSTAGE - 1) * Q < 64, "vmcnt range");
static_assert((BM * ROWB) % 1024 == 0, "A/B boundary on a load block");

// LDS position of 16-byte chunk c of row r: 64 B rows put 4 rows side by side in the 256 B
// bank window, 128 B rows 2, so the XOR spreads the 32 rows of a fragment read over all banks.
__device__ __forceinline__ int swz(int r, int c) { return CPR == 4 ? c ^ ((r >> 2) & 3) : c ^ ((r >> 1) & 7); }

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
}  // namespace dma

template <int MODE>
__global__ void __launch_bounds__(dma::kThreads) k_gemm_dma(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / dma::WN, wn = wave % dma::WN;
    const int n_tiles = a.N / dma::BN;
    const int lid = xcd_tile(blockIdx.x, a.tiles[0], n_tiles);
    if (lid < 0) return;
    const int slot = lid / n_tiles;
    const int tinfo = a.tiles[1 + slot];
    const int ei = tinfo >> 16;
    int mt = tinfo & 0xFFFF, nt = lid % n_tiles;
    const int entry = a.list.ent[ei];
    const int e = entry & 1023;
    const bool shared = e == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    const int base = shared ? 0 : a.offsets[e];
    const int rows = shared ? a.T : a.offsets[e + 1] - base;
    if (MOE_DMA_NMAJOR) {
        // within an expert, walk its m-tiles fastest: consecutive workgroups share a weight slice
        const int mte = (rows + dma::BM - 1) / dma::BM;
        const int off = lid - n_tiles * (slot - mt);
        nt = off / mte;
        mt = off % mte;
    }
    const int m0 = mt * dma::BM, n0 = nt * dma::BN;
    const int K = a.K;
    const int64_t wrow_bytes = int64_t(K) * 2;

    // per load instruction q of this wave: the lane's global source (k0 = 0) and the wave's LDS offset
    const uint8_t* src[dma::Q];
    int ldsoff[dma::Q];
#pragma unroll
    for (int q = 0; q < dma::Q; ++q) {
        const int blk = wave + dma::NW * q;
        const int J = blk * 64 + lane;                      // 16-byte chunk index within the stage
        ldsoff[q] = blk * 1024;
        if (J < dma::BM * dma::CPR) {
            const int r = J / dma::CPR, c = dma::swz(r, J % dma::CPR);
            int64_t srow;
            const int rr = m0 + r < rows ? m0 + r : 0;
            if (MODE == 0)
                srow = shared ? rr : a.perm[base + rr] / a.k;
            else
                srow = shared ? int64_t(a.T) * a.k + rr : base + rr;
            src[q] = a.a_src + srow * int64_t(K) * 2 + c * 16;
        } else {
            const int j = J - dma::BM * dma::CPR;
            const int r = j / dma::CPR, c = dma::swz(r, j % dma::CPR);
            src[q] = blob + a.off_w + int64_t(n0 + r) * wrow_bytes + c * 16;
        }
    }
    auto issue = [&](int ks) {
        uint8_t* st = lds8 + (ks % dma::NSTAGE) * dma::STAGE_BYTES;
#pragma unroll
        for (int q = 0; q < dma::Q; ++q)
            __builtin_amdgcn_global_load_lds(src[q] + ks * dma::BK * 2, st + ldsoff[q], 16, 0, 0);
    };

    typename AccT<dma::MF>::T acc[dma::FM][dma::FN];
#pragma unroll
    for (int i = 0; i < dma::FM; ++i)
#pragma unroll
        for (int j = 0; j < dma::FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    const int nk = K / dma::BK;
    // a wave whose rows all lie past the expert's last row only helps load and keeps the barriers
    const bool active = !MOE_DMA_WSKIP || m0 + wm * dma::TM < rows;
#pragma unroll
    for (int s = 0; s < dma::NSTAGE - 1; ++s)
        if (s < nk) issue(s);
    for (int ks = 0; ks < nk; ++ks) {
        // this wave's loads of stage ks have landed; the barrier makes that true for every
        // wave, and every wave has finished reading stage ks-1 (refilled just below).  A bare
        // s_barrier: __syncthreads() would also wait for the loads still in flight.
        if (ks + dma::NSTAGE - 2 < nk) dma::wait_vm<(dma::NSTAGE - 2) * dma::Q>();
        else dma::wait_vm<0>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (ks + dma::NSTAGE - 1 < nk) issue(ks + dma::NSTAGE - 1);
        const uint8_t* as_ = lds8 + (ks % dma::NSTAGE) * dma::STAGE_BYTES;
        const uint8_t* bs_ = as_ + dma::BM * dma::ROWB;
        if (!active) continue;
#pragma unroll
        for (int kk = 0; kk < dma::BK / 16; ++kk) {
            bf16x8 af[dma::FM], bfr[dma::FN];
            const int c = kk * 2 + lane / 32;
#pragma unroll
            for (int i = 0; i < dma::FM; ++i) {
                const int R = wm * dma::TM + i * 32 + lane % 32;
                af[i] = *reinterpret_cast<const bf16x8*>(as_ + R * dma::ROWB + (dma::swz(R, c) << 4));
            }
#pragma unroll
            for (int j = 0; j < dma::FN; ++j) {
                const int R = wn * dma::TN + j * 32 + lane % 32;
                bfr[j] = *reinterpret_cast<const bf16x8*>(bs_ + R * dma::ROWB + (dma::swz(R, c) << 4));
            }
#pragma unroll
            for (int i = 0; i < dma::FM; ++i)
#pragma unroll
                for (int j = 0; j < dma::FN; ++j) acc[i][j] = mfma(af[i], bfr[j], acc[i][j]);
        }
    }

    // Epilogue through LDS: once every wave is past the last K step (no loads in flight) the
    // stages are free; the tile is staged there and written out as whole rows, 16 bytes a lane.
    const int tid_ = threadIdx.x;
    __syncthreads();
    if (MODE == 0) {
        // SwiGLU: in a 32-wide fragment lanes 0-15 hold gate and lanes 16-31 up for the same 16
        // h columns.  permlane16_swap of elements q1 and q1+4 hands every lane a (gate, up)
        // pair: lanes 0-15 of each half those of q1, lanes 16-31 those of q1+4.
        uint8_t* ht = lds8;
        if (active) {
#pragma unroll
            for (int i = 0; i < dma::FM; ++i)
#pragma unroll
                for (int j = 0; j < dma::FN; ++j) {
                    const int col = (wn * dma::TN + j * 32) / 2 + lane % 16;
#pragma unroll
                    for (int qq = 0; qq < 8; ++qq) {
                        const int q1 = (qq / 4) * 8 + qq % 4;
                        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][q1]),
                                                                         __float_as_uint(acc[i][j][q1 + 4]), false, false);
                        const float g = __uint_as_float(sw[0]), u = __uint_as_float(sw[1]);
                        const int q = (lane % 32) < 16 ? q1 : q1 + 4;
                        const int r = wm * dma::TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                        *reinterpret_cast<uint16_t*>(ht + r * dma::HSTR + col * 2) =
                            dev::f32_to_bf16_bits(ffn::silu_fast(g) * u);
                    }
                }
        }
        __syncthreads();
        constexpr int CH = dma::BN / 16;                     // 16-byte chunks per h row of the tile
        uint16_t* h = static_cast<uint16_t*>(a.out);
        for (int idx = tid_; idx < dma::BM * CH; idx += dma::kThreads) {
            const int r = idx / CH, c = idx % CH;
            if (m0 + r < rows) {
                const int64_t hrow = shared ? int64_t(a.T) * a.k + m0 + r : base + m0 + r;
                *reinterpret_cast<dev::u32x4*>(h + hrow * a.I + n0 / 2 + c * 8) =
                    *reinterpret_cast<const dev::u32x4*>(ht + r * dma::HSTR + c * 16);
            }
        }
    } else {
        uint8_t* ot = lds8;
        int32_t* dst = reinterpret_cast<int32_t*>(lds8 + dma::PR * dma::OSTR);
        for (int r = tid_; r < dma::BM; r += dma::kThreads)
            dst[r] = m0 + r >= rows ? -1 : shared ? a.T * a.k + m0 + r : a.perm[base + m0 + r];
        uint16_t* o = static_cast<uint16_t*>(a.out);        // pair outputs, bf16
        constexpr int CH = dma::BN / 8;                      // 8-value chunks (16 bytes of bf16) per row
        for (int pass = 0; pass < dma::BM / dma::PR; ++pass) {
            if (active) {
#pragma unroll
                for (int i = 0; i < dma::FM; ++i) {
                    const int r0 = wm * dma::TM + i * 32;
                    if (r0 / dma::PR != pass) continue;
#pragma unroll
                    for (int j = 0; j < dma::FN; ++j)
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int r = r0 - pass * dma::PR + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                            *reinterpret_cast<float*>(ot + r * dma::OSTR + (wn * dma::TN + j * 32 + lane % 32) * 4) =
                                acc[i][j][q];
                        }
                }
            }
            __syncthreads();
            for (int idx = tid_; idx < dma::PR * CH; idx += dma::kThreads) {
                const int r = idx / CH, c = idx % CH;
                const int d = dst[pass * dma::PR + r];
                if (d >= 0) {
                    const float4 u = *reinterpret_cast<const float4*>(ot + r * dma::OSTR + c * 32);
                    const float4 v = *reinterpret_cast<const float4*>(ot + r * dma::OSTR + c * 32 + 16);
                    dev::u32x4 pk;
                    pk[0] = dev::pack_bf16x2(u.x, u.y);
                    pk[1] = dev::pack_bf16x2(u.z, u.w);
                    pk[2] = dev::pack_bf16x2(v.x, v.y);
                    pk[3] = dev::pack_bf16x2(v.z, v.w);
                    *reinterpret_cast<dev::u32x4*>(o + int64_t(d) * a.H + n0 + c * 8) = pk;
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------- large-tile GEMM (bf16 or MXFP4 weights)
// 256 x 256 output tiles, 8 waves (2 x 4) of 128 x 64 = 4 x 2 fragments of 32x32x16 MFMA,
// two waves per SIMD (measured on the 8K-token chunk of the 2048 x 768 layer: 547 us for
// GEMM 1 against 604 us with 4 waves of 128 x 128; a wave that stalls issuing its
// direct-to-LDS loads leaves the SIMD to the other).  K slices of BK = 64 (128-byte rows,
// so every row segment a load touches is a whole cache line) are filled by direct
// global->LDS loads into two 64 KiB stage buffers; the 256 x 256 accumulators fill the
// register file, so this is one workgroup per CU.  The workgroups are persistent: each
// walks its XCD's share of the tiles, and the first K slice of its next tile is loaded
// while the current tile's last slice and epilogue run (the epilogue is staged in the LDS
// above the first buffer), so the per-tile start-up and the output stores overlap the
// MFMAs.  Waves whose rows lie partly past the expert's last row run only the fragments
// that hold rows (FA of FM).
// MXFP4 weights travel as codes: a slice holds 32 code bytes per weight row (a quarter of
// bf16), and the tile's e8m0 scales sit in LDS.  The K order inside a slice is permuted the
// same way for both operands (lane half h, sub-step kk covers K = 32 h + 8 kk .. + 7), so
// one 16-byte LDS read gives a lane the codes of all four sub-steps and one scale covers
// them; the codes become bf16 MFMA operands in registers (v_cvt_scalef32_pk_bf16_fp4,
// exact: every e2m1 value times a power of two fits bf16).
namespace big {
#ifndef MOE_BIG_WN
#define MOE_BIG_WN 4
#endif
constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = MOE_BIG_WN, MF = 32;
constexpr int NW = WM * WN, kThreads = NW * kWave;
constexpr int TM = BM / WM, TN = BN / WN, FM = TM / MF, FN = TN / MF;
constexpr int ROWB = BK * 2, CPR = ROWB / 16;       // A rows (and bf16 weight rows): 128 bytes, 8 chunks
constexpr int A_BYTES = BM * ROWB;                  // 32 KiB of A per slice
constexpr int QA = A_BYTES / 1024 / NW;             // 1 KiB A load instructions per wave per slice
constexpr int HSTR = BN + 16;                       // staging row: BN/2 bf16 + 16 bytes
constexpr int kMaxKFp4 = 4096;                      // MXFP4: the tile's scales (BM x K/32 bytes) in LDS
// LDS layout: stage buffers 0 and 1 (A rows, then weight rows), the epilogue staging from
// buffer 1 up (buffer 0 is taking the next tile's first slice by then), the row table and,
// for MXFP4, the scales.
template <bool FP4> struct Lay {
    static constexpr int BROWB = FP4 ? BK / 2 : BK * 2;   // weight bytes per row and slice
    static constexpr int STAGE = A_BYTES + BN * BROWB;    // 64 KiB (bf16), 40 KiB (MXFP4)
    static constexpr int QB = BN * BROWB / 1024 / NW;     // weight load instructions per wave per slice
    static constexpr int Q = QA + QB;
    static constexpr int EPI = STAGE;
    static constexpr int ROWTAB = EPI + BM * HSTR;        // output row of each tile row (GEMM 2)
    static constexpr int SCALES = ROWTAB + BM * 4;
    static constexpr int kLdsBytes = FP4 ? SCALES + BM * (kMaxKFp4 / 32 + 16) : ROWTAB + BM * 4;
    static_assert(kLdsBytes <= 160 * 1024 && ROWTAB >= 2 * STAGE, "LDS per CU; the row table is outside the stages");
    static_assert(QB * NW * 1024 == BN * BROWB && QB >= 1, "weight loads split over the waves");
};
static_assert(QA * NW * 1024 == A_BYTES, "A loads split over the waves");
static_assert(FM * MF == TM && FN * MF == TN && FM == 4, "wave tile (the FA dispatch covers 0..4)");
static_assert(kThreads >= BM, "one output row per thread in the epilogue bookkeeping");
constexpr int kWavesPerSimd = NW / 4;               // 4 SIMDs per CU, one workgroup per CU
// chunk c of row r sits at slot c ^ ((r >> 1) & 7): two 128-byte rows share a 256-byte
// bank window, and the 32 rows of a fragment read land on distinct banks
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }
// MXFP4 code rows (32 bytes, 2 chunks): rows r and r + 8 of a 16-row read group are apart
__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 3) & 1); }

// One tile as this thread sees it.
struct Tile {
    int m0, n0, rows, fa;
    int obase;                  // output row of tile row 0 when the rows are consecutive (h; shared expert)
    int orow;                   // output row of this thread's tile row (epilogue), -1 past the end
    const uint8_t* bbase;       // weight row n0 at K offset 0 (wave-uniform)
    const uint8_t* sbase;       // MXFP4: the e8m0 scales of weight row n0 (wave-uniform)
    uint32_t ao[QA];            // byte offsets (from a_src) of the A rows of this lane's QA load chunks
    uint32_t alive;             // bit q: A load q of this wave covers a row of the tile (wave-uniform)
};

// Byte offset of this lane's chunk within a weight-row block: load QA + q reads weight row
// (wave + NW (QA + q)) * 64 + lane) / 8 - BM = rb + 32 q; the chunk (source-side swizzle: the
// LDS side of a load is linear) is the same for every q, and for the A loads too.
__device__ __forceinline__ int lane_chunk() {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    return swz((wave * 64 + lane) / CPR, lane % CPR);
}

template <int MODE, bool FP4>
__device__ __forceinline__ Tile make_tile(const GemmArgs& a, int lid, int n_tiles) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / WN;
    Tile t;
    const int slot = lid / n_tiles;
    int nt = lid % n_tiles;
    const int4 rec = a.rec[slot];                   // one load instead of a chain of four
    const int entry = rec.x;
    int mt = rec.w;
    const int e = entry & 1023;
    const bool shared = e == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    const int base = rec.y;
    t.rows = rec.z;
    if (int64_t(t.rows) * 64 <= int64_t(a.N) * (FP4 ? 17 : 64)) {
        // the expert's activation rows take fewer bytes than its weights (bf16: 2 bytes an
        // element; MXFP4: 17/32): its m-tiles run fastest, so the tiles that share a weight
        // block are adjacent and run together on one XCD, and the expert's rows stay in that
        // XCD's L2 between weight blocks (a3b 8K gate/up GEMM: 1.30x the algorithmic bytes
        // fetched, against 1.65x with the n-tiles fastest).  Experts with more rows than that
        // (the shared expert in prefill) keep the n-tiles fastest, sharing each row block.
        const int mte = (t.rows + BM - 1) / BM;
        const int off = lid - n_tiles * (slot - mt);   // the expert's tiles start at slot - mt
        nt = off / mte;
        mt = off % mte;
    }
    t.m0 = mt * BM;
    t.n0 = nt * BN;
    const int fa = (t.rows - t.m0 - wm * TM + 31) / 32;   // fragment rows of this wave that hold rows
    t.fa = __builtin_amdgcn_readfirstlane(fa < 0 ? 0 : fa > FM ? FM : fa);
    const uint32_t arow_bytes = uint32_t(a.K) * 2;
    const uint32_t c16 = uint32_t(lane_chunk()) * 16;
    int pv[QA], rrs[QA];
    t.alive = 0;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int r = ((wave + NW * q) * 64 + lane) / CPR;
        // A load q of the wave fills tile rows 8 (wave + NW q) .. + 7; one wholly past the
        // expert's rows is skipped (its LDS rows feed only output rows that are dropped)
        if (t.m0 + (wave + NW * q) * (64 / CPR) < t.rows) t.alive |= 1u << q;
        const int rr = t.m0 + r < t.rows ? t.m0 + r : 0;        // rows past the end load row 0 (dropped)
        if constexpr (MODE == 0) {
            rrs[q] = rr;
            pv[q] = a.perm[shared ? 0 : base + rr];     // a valid index either way
        } else {
            t.ao[q] = uint32_t(shared ? a.T * a.k + rr : base + rr) * arow_bytes + c16;
        }
    }
    if constexpr (MODE == 0) {
        // the QA perm loads are all issued before the first of them is waited for
#pragma unroll
        for (int q = 0; q < QA; ++q) asm volatile("" : "+v"(pv[q]));
#pragma unroll
        for (int q = 0; q < QA; ++q)
            t.ao[q] = (shared ? uint32_t(rrs[q]) : uint32_t(pv[q]) / uint32_t(a.k)) * arow_bytes + c16;
    }
    t.alive = __builtin_amdgcn_readfirstlane(t.alive);
    t.bbase = blob + a.off_w + int64_t(t.n0) * (FP4 ? a.K / 2 : a.K * 2);
    t.sbase = blob + a.off_s + int64_t(t.n0) * (a.K / 32);
    t.obase = (shared ? a.T * a.k : base) + t.m0;
    const int r = tid;                                           // epilogue: tile row tid
    const bool live = r < BM && t.m0 + r < t.rows;
    if constexpr (MODE == 0)
        t.orow = live ? t.obase + r : -1;
    else
        t.orow = !live ? -1 : shared ? t.obase + r : a.perm[live && !shared ? base + t.m0 + r : 0];
    return t;
}

// This lane's byte offset in the tile's weight rows for its first weight load, and the
// step between its weight loads (QB > 1).  bf16: load QA + q fills chunk (wave + NW (QA + q))
// * 64 + lane of the stage, weight row that / 8 - BM; MXFP4: load QA fills code chunk
// wave * 64 + lane, row that / 2.
template <bool FP4>
__device__ __forceinline__ uint32_t b_lane_off(int K) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (FP4) {
        const int r = (wave * 64 + lane) / 2;
        return uint32_t(r) * uint32_t(K / 2) + uint32_t(swz4(r, lane % 2)) * 16;
    }
    return uint32_t(((wave + NW * QA) * 64 + lane) / CPR - BM) * uint32_t(K) * 2 + uint32_t(lane_chunk()) * 16;
}
template <bool FP4>
__device__ __forceinline__ uint32_t b_stride(int K) {
    return FP4 ? 0u : uint32_t(K) * 2 * (NW * 64 / CPR);
}

// Loads of one K slice into stage buffer buf: A rows at a_src + ao[q] + koa (with SKIP, the
// loads in alive only), weight rows at bbase + boff + kob.  The slice is handed over by a
// barrier that waits for every load, so the number issued may vary.  Skipping is used by the
// down GEMMs (MXFP4 8K chunk: 843-850 us against 895-899 us) and the MXFP4 gate/up GEMM (1,318-
// 1,320 against 1,331-1,333 us); the bf16 gate/up GEMM measured slower with it (451-454 against
// 442 us), so it loads every row group.
template <bool FP4, bool SKIP>
__device__ __forceinline__ void issue(uint8_t* lds8, const uint8_t* a_src, const uint32_t (&ao)[QA], uint32_t alive,
                                      const uint8_t* bbase, uint32_t boff, uint32_t bstride, uint32_t koa, uint32_t kob,
                                      int buf) {
    const int wave = threadIdx.x / kWave;
    uint8_t* st = lds8 + buf * Lay<FP4>::STAGE;
#pragma unroll
    for (int q = 0; q < Lay<FP4>::Q; ++q) {
        if (SKIP && q < QA && !((alive >> q) & 1u)) continue;
        const uint8_t* src = q < QA ? a_src + (ao[q] + koa) : bbase + (boff + (q - QA) * bstride + kob);
        __builtin_amdgcn_global_load_lds(src, st + (wave + NW * q) * 1024, 16, 0, 0);
    }
}

// MXFP4: LDS row stride of the tile's scales.  The 32 lanes of a fragment read one scale byte
// each from 32 consecutive rows; rows of an even number of 16-byte chunks (K/32 = 64 or 128
// bytes) would put those bytes in 2 or 4 banks, so such rows get one 16-byte pad chunk, which
// spreads them over 16 banks.  Rows that are not whole chunks (K not a multiple of 512) are
// copied back to back.
__device__ __forceinline__ int scale_stride(int K) {
    const int rb = K / 32;
    return rb % 16 == 0 && (rb / 16) % 2 == 0 ? rb + 16 : rb;
}

// MXFP4: the tile's scales (BM rows x K/32 bytes, contiguous in the blob) into LDS, rows
// scale_stride(K) bytes apart (the pad chunk of a row repeats its last chunk; never read).
__device__ __forceinline__ void issue_scales(uint8_t* lds8, const uint8_t* sbase, int K) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int rb = K / 32, stride = scale_stride(K);
    const int chunks = BM * stride / 16;                 // a multiple of 64 (K a multiple of 128)
    uint8_t* dst = lds8 + Lay<true>::SCALES;
    for (int c0 = wave * 64; c0 < chunks; c0 += kThreads) {
        const int c = c0 + lane;
        int src = c * 16;                                // rows back to back
        if (stride != rb) {
            const int cpr = stride / 16, r = c / cpr, j = c - r * cpr;
            src = r * rb + min(j, rb / 16 - 1) * 16;
        }
        __builtin_amdgcn_global_load_lds(sbase + src, dst + c0 * 16, 16, 0, 0);
    }
}

// 8 MXFP4 codes (low nibble first) times the block scale, as bf16 MFMA operands
__device__ __forceinline__ bf16x8 fp4x8_bf16(uint32_t w, float sc) {
    const dev::bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    const dev::bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    const dev::bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    const dev::bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
}  // namespace big

// Barrier that hands direct-to-LDS data to the other waves: every wave first waits for its
// own loads (they write blocks the other waves read; a plain __syncthreads() only waits for
// what this wave's own later code reads, so it may leave them in flight).
__device__ __forceinline__ void barrier_loads() {
    __builtin_amdgcn_s_waitcnt(0);      // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();
}

// Barrier over LDS only: this wave's LDS operations have completed, vector memory operations
// (the epilogue's global stores) may still be in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One tile for a wave that computes FA fragment rows (0..FM).  On entry the tile's slice 0
// is in flight into buffer 0 (first tile of the workgroup) or has landed (later tiles: the
// previous tile waited for it before its epilogue's stores, so the stores are left to drain
// under this tile's first slice); before the last slice the next tile's slice 0 is issued
// into buffer 0 (for the last tile of the workgroup, a harmless reload of this tile's last
// slice).  The epilogue also builds nn, the descriptor of tile nn_lid (if >= 0), while no
// store is in flight.
template <int MODE, int FA, bool FP4>
__device__ __forceinline__ void big_tile(const GemmArgs& a, uint8_t* lds8, const big::Tile& t, const big::Tile& nx,
                                         bool has_next, bool first, int nn_lid, big::Tile& nn) {
    using L = big::Lay<FP4>;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / big::WN, wn = wave % big::WN;
    const int nk = a.K / big::BK;
    const uint32_t bstride = big::b_stride<FP4>(a.K);
    const uint32_t boff = big::b_lane_off<FP4>(a.K);
    constexpr int NA = FA > 0 ? FA : 1;
    f32x16 acc[NA][big::FN];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < big::FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // fragments of K sub-step kk (16 wide) of slice ks in stage as_; two register sets, so
    // the reads of sub-step kk + 1 are in flight while the MFMAs of kk run.  MXFP4: the
    // codes and scale of the whole slice are read with sub-step 0 (permuted K order).
    uint4 bq[big::FN];
    float bsc[big::FN];
    auto frag = [&](const uint8_t* as_, int kk, int ks, bf16x8 (&fa)[NA], bf16x8 (&fb)[big::FN]) {
        const uint8_t* bs_ = as_ + big::A_BYTES;
        const int c = FP4 ? (lane / 32) * 4 + kk : kk * 2 + lane / 32;
#pragma unroll
        for (int i = 0; i < FA; ++i) {
            const int R = wm * big::TM + i * 32 + lane % 32;
            fa[i] = *reinterpret_cast<const bf16x8*>(as_ + R * big::ROWB + (big::swz(R, c) << 4));
        }
        if constexpr (FP4) {
            if (kk == 0) {
#pragma unroll
                for (int j = 0; j < big::FN; ++j) {
                    const int R = wn * big::TN + j * 32 + lane % 32;
                    bq[j] = *reinterpret_cast<const uint4*>(bs_ + R * 32 + (big::swz4(R, lane / 32) << 4));
                    const uint32_t sc = lds8[L::SCALES + R * big::scale_stride(a.K) + ks * 2 + lane / 32];
                    bsc[j] = sc ? __uint_as_float(sc << 23) : __uint_as_float(0x00400000u);
                }
            }
#pragma unroll
            for (int j = 0; j < big::FN; ++j)
                fb[j] = big::fp4x8_bf16(kk == 0 ? bq[j].x : kk == 1 ? bq[j].y : kk == 2 ? bq[j].z : bq[j].w, bsc[j]);
        } else {
#pragma unroll
            for (int j = 0; j < big::FN; ++j) {
                const int R = wn * big::TN + j * 32 + lane % 32;
                fb[j] = *reinterpret_cast<const bf16x8*>(bs_ + R * big::ROWB + (big::swz(R, c) << 4));
            }
        }
    };
    auto mma = [&](const bf16x8 (&fa)[NA], const bf16x8 (&fb)[big::FN]) {
#pragma unroll
        for (int i = 0; i < FA; ++i)
#pragma unroll
            for (int j = 0; j < big::FN; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
    };
    // schedule of one sub-step: its MFMAs with the next sub-step's NR LDS reads placed one
    // after each of the first MFMAs
    constexpr int NM = FA * big::FN;
    constexpr int NR_B = FP4 ? 0 : big::FN, NR0 = FA + (FP4 ? 2 * big::FN : big::FN);
    auto sched = [&](auto nr_) {
        constexpr int NR = decltype(nr_)::value;
        if constexpr (NM >= NR) {
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
        }
    };
    using RdK = std::integral_constant<int, FA + NR_B>;   // reads of sub-steps 1..3
    using Rd0 = std::integral_constant<int, NR0>;         // reads of sub-step 0

    // Slice ks is read from buffer ks & 1 (nk is even).  The barrier of slice ks sits
    // before its last sub-step: by then every wave has read all of slice ks (so its buffer
    // can take slice ks + 2) and the loads of slice ks + 1, issued one slice earlier, have
    // landed (so the last sub-step's MFMAs overlap the reads of the next slice's first
    // sub-step).  The loop body is straight-line and the last slice is peeled, which keeps
    // the accumulators in place across iterations.
    bf16x8 fa0[NA], fb0[big::FN], fa1[NA], fb1[big::FN];
    if (first) barrier_loads();     // slice 0 (and the scales) landed
    big::issue<FP4, MODE == 1 || FP4>(lds8, a.a_src, t.ao, t.alive, t.bbase, boff, bstride, big::ROWB, L::BROWB, 1);
    if (MODE == 1 && tid < big::BM) reinterpret_cast<int32_t*>(lds8 + L::ROWTAB)[tid] = t.orow;   // read after later barriers
    if constexpr (FA > 0) frag(lds8, 0, 0, fa0, fb0);
    for (int ks = 0; ks + 1 < nk; ++ks) {
        const uint8_t* as_ = lds8 + (ks & 1) * L::STAGE;
        if constexpr (FA > 0) {
            frag(as_, 1, ks, fa1, fb1);
            mma(fa0, fb0);
            frag(as_, 2, ks, fa0, fb0);
            mma(fa1, fb1);
            frag(as_, 3, ks, fa1, fb1);
            mma(fa0, fb0);
            sched(RdK{});
            sched(RdK{});
            sched(RdK{});
        }
        barrier_loads();            // (in the first slice of a later tile, also the previous epilogue's stores)
        // MXFP4: the next slice's first reads go before the loads that refill this slice's
        // buffer (in program order, so the code reads are not taken to depend on those
        // loads); bf16 issues the loads first (measured faster)
        if constexpr (FA > 0 && FP4) frag(lds8 + ((ks + 1) & 1) * L::STAGE, 0, ks + 1, fa0, fb0);
        {
            // slice ks + 2 into the buffer slice ks leaves; past the end, the next tile's slice 0
            // (or, after the last tile, this tile's last slice again: never read)
            const bool nxt = ks + 2 >= nk;
            const bool other = nxt && has_next;
            const uint32_t kn = uint32_t(nxt ? (has_next ? 0 : nk - 1) : ks + 2);
            uint32_t ao[big::QA];
#pragma unroll
            for (int q = 0; q < big::QA; ++q) ao[q] = other ? nx.ao[q] : t.ao[q];
            big::issue<FP4, MODE == 1 || FP4>(lds8, a.a_src, ao, other ? nx.alive : t.alive, other ? nx.bbase : t.bbase, boff, bstride,
                            kn * big::ROWB, kn * L::BROWB,
                            ks & 1);
        }
        if constexpr (FA > 0) {
            if constexpr (!FP4) frag(lds8 + ((ks + 1) & 1) * L::STAGE, 0, ks + 1, fa0, fb0);
            mma(fa1, fb1);
            sched(Rd0{});
        }
    }
    if constexpr (FA > 0) {
        const uint8_t* as_ = lds8 + L::STAGE;       // slice nk - 1 (odd)
        frag(as_, 1, nk - 1, fa1, fb1);
        mma(fa0, fb0);
        frag(as_, 2, nk - 1, fa0, fb0);
        mma(fa1, fb1);
        frag(as_, 3, nk - 1, fa1, fb1);
        mma(fa0, fb0);
        mma(fa1, fb1);
    }

    // Epilogue through the LDS above buffer 0 (buffer 0 holds the next tile's first slice):
    // the tile is staged there and written out as whole rows, 16 bytes a lane.
    uint8_t* stg = lds8 + L::EPI;
    // Every wave is done with slice nk - 1 (buffer 1) and the scales, and the next tile's slice
    // 0 has landed: the only vector memory operations in flight are loads here, so this wait
    // costs their tail.  Loads and stores share one completion counter, so the loads the next
    // tile needs first are waited for before any store is issued; the stores then drain under
    // the next tile's first slice.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (FP4 && has_next) big::issue_scales(lds8, nx.sbase, a.K);   // the next tile's, while this one finishes
    // the descriptor of the tile after next, and the scales, complete before the first store
    auto next_desc = [&]() {
        if (nn_lid >= 0) nn = big::make_tile<MODE, FP4>(a, nn_lid, a.N / big::BN);
        __builtin_amdgcn_s_waitcnt(0);
    };
    if (MODE == 0) {
        // SwiGLU: in a 32-wide fragment lanes 0-15 hold gate and lanes 16-31 up for the
        // same 16 h columns; permlane16_swap of elements q1 and q1+4 hands every lane a
        // (gate, up) pair: lanes 0-15 of each half those of q1, lanes 16-31 those of q1+4.
#pragma unroll
        for (int i = 0; i < FA; ++i)
#pragma unroll
            for (int j = 0; j < big::FN; ++j) {
                const int col = (wn * big::TN + j * 32) / 2 + lane % 16;
                float hv[8];
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int q1 = (qq / 4) * 8 + qq % 4;
                    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][q1]),
                                                                     __float_as_uint(acc[i][j][q1 + 4]), false, false);
                    hv[qq] = ffn::silu_fast(__uint_as_float(sw[0])) * __uint_as_float(sw[1]);
                }
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int q1 = (qq / 4) * 8 + qq % 4;
                    const int q = (lane % 32) < 16 ? q1 : q1 + 4;
                    const int r = wm * big::TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                    *reinterpret_cast<uint16_t*>(stg + r * big::HSTR + col * 2) = bf16_bits(hv[qq]);
                }
            }
        next_desc();
        lds_barrier();
        constexpr int CH = big::BN / 16;                     // 16-byte chunks per h row of the tile
        constexpr int PER = big::BM * CH / big::kThreads;
        uint16_t* h = static_cast<uint16_t*>(a.out);
        dev::u32x4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * big::kThreads, r = idx / CH, c = idx % CH;
            v[k] = *reinterpret_cast<const dev::u32x4*>(stg + r * big::HSTR + c * 16);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * big::kThreads, r = idx / CH, c = idx % CH;
            if (t.m0 + r < t.rows)
                *reinterpret_cast<dev::u32x4*>(h + int64_t(t.obase + r) * a.I + t.n0 / 2 + c * 8) = v[k];
        }
    } else {
        // pair outputs, bf16, staged in two passes of half the tile's columns (pass p: columns
        // BN/2 p .. BN/2 p + BN/2 - 1, those of wave columns WN/2 p .. WN/2 p + WN/2 - 1), then
        // each row's BN/2 contiguous columns written as whole lines to the row from the tile's
        // row table
        uint16_t* o = static_cast<uint16_t*>(a.out);
        const int32_t* orow = reinterpret_cast<const int32_t*>(lds8 + L::ROWTAB);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wn / (big::WN / 2) == pass) {
#pragma unroll
                for (int i = 0; i < FA; ++i)
#pragma unroll
                    for (int j = 0; j < big::FN; ++j) {
                        const int col = (wn % (big::WN / 2)) * big::TN + j * 32 + lane % 32;     // staged column
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int r = wm * big::TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                            *reinterpret_cast<uint16_t*>(stg + r * big::HSTR + col * 2) = bf16_bits(acc[i][j][q]);
                        }
                    }
            }
            if (pass == 0) next_desc();
            lds_barrier();
            // 16 chunks of 16 bytes per staged row: 256 contiguous bytes of the output row; the
            // LDS reads first, then the stores
            constexpr int PER = big::BM * 16 / big::kThreads;
            int32_t d[PER];
            dev::u32x4 v[PER];
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int idx = tid + k * big::kThreads, r = idx / 16, c = idx % 16;
                d[k] = orow[r];
                v[k] = *reinterpret_cast<const dev::u32x4*>(stg + r * big::HSTR + c * 16);
            }
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int c = (tid + k * big::kThreads) % 16;
                if (d[k] >= 0)
                    *reinterpret_cast<dev::u32x4*>(o + int64_t(d[k]) * a.H + t.n0 + pass * (big::BN / 2) + c * 8) = v[k];
            }
            if (pass == 0) lds_barrier();
        }
    }
    lds_barrier();              // the staging is read: the next tile's slice 1 goes into buffer 1
}

// Persistent: workgroup b serves XCD b % 8 and walks tiles b / 8, b / 8 + G / 8, ... of that
// XCD's contiguous share of the real tiles (G workgroups in all).
template <int MODE, bool FP4>
__global__ void __launch_bounds__(big::kThreads) __attribute__((amdgpu_waves_per_eu(big::kWavesPerSimd, big::kWavesPerSimd)))
k_gemm_big(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const int n_tiles = a.N / big::BN;
    const int total = a.tiles[0] * n_tiles;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds, stride = gridDim.x / kXcds;
    int i = blockIdx.x / kXcds;
    if (i >= per_xcd || x * per_xcd + i >= total) return;
    // the descriptors of the first two tiles are read before any load is issued; later ones
    // in the epilogue two tiles ahead
    big::Tile cur = big::make_tile<MODE, FP4>(a, x * per_xcd + i, n_tiles);
    int in = i + stride;
    bool has_next = in < per_xcd && x * per_xcd + in < total;
    big::Tile nx = has_next ? big::make_tile<MODE, FP4>(a, x * per_xcd + in, n_tiles) : cur;
    big::issue<FP4, MODE == 1 || FP4>(lds8, a.a_src, cur.ao, cur.alive, cur.bbase, big::b_lane_off<FP4>(a.K), big::b_stride<FP4>(a.K), 0, 0, 0);
    if (FP4) big::issue_scales(lds8, cur.sbase, a.K);
    bool first = true;
    while (true) {
        const int in2 = in + stride;
        const bool has_next2 = has_next && in2 < per_xcd && x * per_xcd + in2 < total;
        const int nn_lid = has_next2 ? x * per_xcd + in2 : -1;
        big::Tile nn = nx;
        switch (cur.fa) {
            case 4: big_tile<MODE, 4, FP4>(a, lds8, cur, nx, has_next, first, nn_lid, nn); break;
            case 3: big_tile<MODE, 3, FP4>(a, lds8, cur, nx, has_next, first, nn_lid, nn); break;
            case 2: big_tile<MODE, 2, FP4>(a, lds8, cur, nx, has_next, first, nn_lid, nn); break;
            case 1: big_tile<MODE, 1, FP4>(a, lds8, cur, nx, has_next, first, nn_lid, nn); break;
            default: big_tile<MODE, 0, FP4>(a, lds8, cur, nx, has_next, first, nn_lid, nn); break;
        }
        if (!has_next) break;
        cur = nx;
        nx = nn;
        has_next = has_next2;
        in = in2;
        first = false;
    }
}

// ---------------------------------------------------------------- three-stage bf16 GEMM
// 128 x 256 tiles, K slices of 64 (whole 128-byte row segments) loaded straight into a ring
// of three 48 KiB LDS stages, so the loads of a slice have two slices of MFMA time to land
// (the 256 x 256 tile's 64 KiB stages leave room for two).  8 waves (2 x 4) of 64 x 64 = 2 x 2
// fragments of 32x32x16 MFMA.  Persistent like the large tile: a workgroup walks its XCD's
// share of the tiles, the stage ring continues across its tiles, and the next tile's first two
// slices are loaded under the current tile's last slices; its third after the epilogue, which
// is staged in the buffer the last slice leaves.
namespace b3 {
constexpr int BM = 128, BN = 256, BK = 64, NS = 3, WM = 2, WN = 4, MF = 32;
constexpr int NW = WM * WN, kThreads = NW * kWave;
constexpr int TM = BM / WM, TN = BN / WN, FM = TM / MF, FN = TN / MF;
constexpr int ROWB = BK * 2, CPR = ROWB / 16;
constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB, STAGE = A_BYTES + B_BYTES;
constexpr int QA = A_BYTES / 1024 / NW, QB = B_BYTES / 1024 / NW, Q = QA + QB;
constexpr int HSTR = BN + 16;                       // staged row: BN/2 bf16 + 16 bytes
constexpr int ROWTAB = NS * STAGE;                  // output row of each tile row (GEMM 2)
constexpr int kLdsBytes = ROWTAB + BM * 4;
static_assert(BM * HSTR <= STAGE, "the epilogue is staged in one stage buffer");
static_assert(kLdsBytes <= 160 * 1024, "LDS per CU");
static_assert(QA * NW * 1024 == A_BYTES && QB * NW * 1024 == B_BYTES, "loads split over the waves");
static_assert(FM * MF == TM && FN * MF == TN && FM == 2 && FN == 2, "wave tile");
static_assert(kThreads >= BM, "one tile row per thread in the row table");
static_assert(Q < 16, "vmcnt immediates");
constexpr int kWavesPerSimd = NW / 4;
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

struct Tile {
    int m0, n0, rows, fa, obase, orow;
    const uint8_t* bbase;
    uint32_t ao[QA];
};

template <int MODE>
__device__ __forceinline__ Tile make_tile(const GemmArgs& a, int lid, int n_tiles) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / WN;
    Tile t;
    const int slot = lid / n_tiles;
    int nt = lid % n_tiles;
    const int4 rec = a.rec[slot];
    const int entry = rec.x;
    int mt = rec.w;
    const int e = entry & 1023;
    const bool shared = e == kSharedTag;
    const uint8_t* blob = shared ? a.shared_blob : a.slot_base + int64_t(entry >> 10) * a.blob_bytes;
    const int base = rec.y;
    t.rows = rec.z;
    if (t.rows <= a.N) {                        // rows in fewer bytes than the weights: m-tiles fastest
        const int mte = (t.rows + BM - 1) / BM;
        const int off = lid - n_tiles * (slot - mt);
        nt = off / mte;
        mt = off % mte;
    }
    t.m0 = mt * BM;
    t.n0 = nt * BN;
    const int fa = (t.rows - t.m0 - wm * TM + 31) / 32;
    t.fa = __builtin_amdgcn_readfirstlane(fa < 0 ? 0 : fa > FM ? FM : fa);
    const uint32_t arow_bytes = uint32_t(a.K) * 2;
    const uint32_t c16 = uint32_t(swz((wave * 64 + lane) / CPR, lane % CPR)) * 16;
    int pv[QA], rrs[QA];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int r = ((wave + NW * q) * 64 + lane) / CPR;
        const int rr = t.m0 + r < t.rows ? t.m0 + r : 0;
        if constexpr (MODE == 0) {
            rrs[q] = rr;
            pv[q] = a.perm[shared ? 0 : base + rr];     // a valid index either way
        } else {
            t.ao[q] = uint32_t(shared ? a.T * a.k + rr : base + rr) * arow_bytes + c16;
        }
    }
    if constexpr (MODE == 0) {
        // the QA perm loads are all issued before the first of them is waited for
#pragma unroll
        for (int q = 0; q < QA; ++q) asm volatile("" : "+v"(pv[q]));
#pragma unroll
        for (int q = 0; q < QA; ++q)
            t.ao[q] = (shared ? uint32_t(rrs[q]) : uint32_t(pv[q]) / uint32_t(a.k)) * arow_bytes + c16;
    }
    t.bbase = blob + a.off_w + int64_t(t.n0) * a.K * 2;
    t.obase = (shared ? a.T * a.k : base) + t.m0;
    const int r = tid;
    const bool live = r < BM && t.m0 + r < t.rows;
    if constexpr (MODE == 0)
        t.orow = live ? t.obase + r : -1;
    else
        t.orow = !live ? -1 : shared ? t.obase + r : a.perm[live && !shared ? base + t.m0 + r : 0];
    return t;
}

// Loads of K slice ks of tile t into stage buffer buf (Q instructions a wave).
__device__ __forceinline__ void issue(uint8_t* lds8, const GemmArgs& a, const Tile& t, int ks, int buf) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    uint8_t* st = lds8 + buf * STAGE;
    const uint32_t koff = uint32_t(ks) * ROWB;
    const uint32_t brow = uint32_t((wave * 64 + lane) / CPR);             // weight row of load QA
    const uint32_t boff = brow * uint32_t(a.K) * 2 + uint32_t(swz(int(brow), lane % CPR)) * 16;
    const uint32_t bstride = uint32_t(a.K) * 2 * (NW * 64 / CPR);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint8_t* src = q < QA ? a.a_src + (t.ao[q] + koff) : t.bbase + (boff + (q - QA) * bstride + koff);
        __builtin_amdgcn_global_load_lds(src, st + (wave + NW * q) * 1024, 16, 0, 0);
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
}  // namespace b3

// One tile for a wave that computes FA fragment rows (0..2); slice ks is in buffer (g0 + ks) % 3.
// First tile of the workgroup: on entry slices 0, 1 and 2 have been issued, in that order, and
// nothing else is in flight.  Later tiles: slices 0 and 1 have landed (the previous tile waited
// for them before its epilogue's stores), and slice 2 and those stores are in flight; the first
// slice waits for all of them (loads and stores share one completion counter), so the stores
// drain under its MFMAs.  On exit this tile's stores may be in flight; the caller issues the
// next tile's slice 2 into buffer (g0 + nk - 1) % 3 (its slices 0 and 1 were issued here).
// The epilogue also builds nn, the descriptor of tile nn_lid (if >= 0), before its stores.
template <int MODE, int FA>
__device__ __forceinline__ void b3_tile(const GemmArgs& a, uint8_t* lds8, const b3::Tile& t, const b3::Tile& nx,
                                        bool has_next, int g0, bool first, int nn_lid, b3::Tile& nn) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / b3::WN, wn = wave % b3::WN;
    const int nk = a.K / b3::BK;
    constexpr int NA = FA > 0 ? FA : 1;
    f32x16 acc[NA][b3::FN];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < b3::FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    auto buf_of = [&](int ks) { int b = g0 + ks; b -= 3 * (b / 3); return b; };
    auto frag = [&](const uint8_t* as_, int kk, bf16x8 (&fa)[NA], bf16x8 (&fb)[b3::FN]) {
        const uint8_t* bs_ = as_ + b3::A_BYTES;
        const int c = kk * 2 + lane / 32;
#pragma unroll
        for (int i = 0; i < FA; ++i) {
            const int R = wm * b3::TM + i * 32 + lane % 32;
            fa[i] = *reinterpret_cast<const bf16x8*>(as_ + R * b3::ROWB + (b3::swz(R, c) << 4));
        }
#pragma unroll
        for (int j = 0; j < b3::FN; ++j) {
            const int R = wn * b3::TN + j * 32 + lane % 32;
            fb[j] = *reinterpret_cast<const bf16x8*>(bs_ + R * b3::ROWB + (b3::swz(R, c) << 4));
        }
    };
    auto mma = [&](const bf16x8 (&fa)[NA], const bf16x8 (&fb)[b3::FN]) {
#pragma unroll
        for (int i = 0; i < FA; ++i)
#pragma unroll
            for (int j = 0; j < b3::FN; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
    };
    constexpr int NM = FA * b3::FN, NR = FA + b3::FN;
    auto sched = [&]() {
        if constexpr (NM >= NR && NR > 0) {
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
        }
    };
    bf16x8 fa0[NA], fb0[b3::FN], fa1[NA], fb1[b3::FN];
    if (first) {
        b3::wait_vm<2 * b3::Q>();       // slice 0 landed (slices 1 and 2 may still be in flight)
        b3::bare_barrier();
    }
    if (MODE == 1 && tid < b3::BM) reinterpret_cast<int32_t*>(lds8 + b3::ROWTAB)[tid] = t.orow;   // read after later barriers
    if constexpr (FA > 0) frag(lds8 + buf_of(0) * b3::STAGE, 0, fa0, fb0);
    for (int ks = 0; ks + 1 < nk; ++ks) {
        const uint8_t* as_ = lds8 + buf_of(ks) * b3::STAGE;
        if constexpr (FA > 0) {
            frag(as_, 1, fa1, fb1);
            mma(fa0, fb0);
            frag(as_, 2, fa0, fb0);
            mma(fa1, fb1);
            frag(as_, 3, fa1, fb1);
            mma(fa0, fb0);
            sched();
            sched();
            sched();
        }
        // every wave has read slice ks (its buffer can take slice ks + 3) and slice ks + 1 has
        // landed (slice ks + 2, issued one slice later, may still be in flight; in the first
        // slice of a later tile everything in flight is waited for, the previous stores too)
        if (!first && ks == 0) {
            __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0) lgkmcnt(0)
        } else {
            b3::wait_vm<b3::Q>();
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the fragment reads of this wave done
        }
        b3::bare_barrier();
        {
            // slice ks + 3 into the buffer slice ks leaves: this tile's, else the next tile's slice
            // 0 or 1 (or, after the last tile, slice ks again: the same bytes, never read)
            const int kn = ks + 3;
            if (kn < nk) b3::issue(lds8, a, t, kn, buf_of(ks));
            else if (has_next) b3::issue(lds8, a, nx, kn - nk, buf_of(ks));
            else b3::issue(lds8, a, t, ks, buf_of(ks));
        }
        if constexpr (FA > 0) {
            frag(lds8 + buf_of(ks + 1) * b3::STAGE, 0, fa0, fb0);
            mma(fa1, fb1);
            sched();
        }
    }
    if constexpr (FA > 0) {
        const uint8_t* as_ = lds8 + buf_of(nk - 1) * b3::STAGE;
        frag(as_, 1, fa1, fb1);
        mma(fa0, fb0);
        frag(as_, 2, fa0, fb0);
        mma(fa1, fb1);
        frag(as_, 3, fa1, fb1);
        mma(fa0, fb0);
        mma(fa1, fb1);
    }
    // Epilogue staged in the buffer of the last slice (the next tile's slices 0 and 1 are in
    // the other two); afterwards the next tile's slice 2 goes there.
    uint8_t* stg = lds8 + buf_of(nk - 1) * b3::STAGE;
    // every wave is done with slice nk - 1, and the next tile's slices 0 and 1 have landed
    // (only loads are in flight here: the wait costs their tail, before any store is issued)
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    auto next_desc = [&]() {
        if (nn_lid >= 0) nn = b3::make_tile<MODE>(a, nn_lid, a.N / b3::BN);
    };
    if (MODE == 0) {
#pragma unroll
        for (int i = 0; i < FA; ++i)
#pragma unroll
            for (int j = 0; j < b3::FN; ++j) {
                const int col = (wn * b3::TN + j * 32) / 2 + lane % 16;
                float hv[8];
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int q1 = (qq / 4) * 8 + qq % 4;
                    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][j][q1]),
                                                                     __float_as_uint(acc[i][j][q1 + 4]), false, false);
                    hv[qq] = ffn::silu_fast(__uint_as_float(sw[0])) * __uint_as_float(sw[1]);
                }
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int q1 = (qq / 4) * 8 + qq % 4;
                    const int q = (lane % 32) < 16 ? q1 : q1 + 4;
                    const int r = wm * b3::TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                    *reinterpret_cast<uint16_t*>(stg + r * b3::HSTR + col * 2) = bf16_bits(hv[qq]);
                }
            }
        next_desc();
        lds_barrier();
        constexpr int CH = b3::BN / 16;
        constexpr int PER = b3::BM * CH / b3::kThreads;
        uint16_t* h = static_cast<uint16_t*>(a.out);
        dev::u32x4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * b3::kThreads, r = idx / CH, c = idx % CH;
            v[k] = *reinterpret_cast<const dev::u32x4*>(stg + r * b3::HSTR + c * 16);
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * b3::kThreads, r = idx / CH, c = idx % CH;
            if (t.m0 + r < t.rows)
                *reinterpret_cast<dev::u32x4*>(h + int64_t(t.obase + r) * a.I + t.n0 / 2 + c * 8) = v[k];
        }
    } else {
        uint16_t* o = static_cast<uint16_t*>(a.out);
        const int32_t* orow = reinterpret_cast<const int32_t*>(lds8 + b3::ROWTAB);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            if (wn / (b3::WN / 2) == pass) {
#pragma unroll
                for (int i = 0; i < FA; ++i)
#pragma unroll
                    for (int j = 0; j < b3::FN; ++j) {
                        const int col = (wn % (b3::WN / 2)) * b3::TN + j * 32 + lane % 32;     // staged column
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int r = wm * b3::TM + i * 32 + 8 * (q / 4) + (lane / 32) * 4 + (q % 4);
                            *reinterpret_cast<uint16_t*>(stg + r * b3::HSTR + col * 2) = bf16_bits(acc[i][j][q]);
                        }
                    }
            }
            if (pass == 0) next_desc();
            lds_barrier();
            // the LDS reads first, then the stores
            constexpr int PER = b3::BM * 16 / b3::kThreads;
            int32_t d[PER];
            dev::u32x4 v[PER];
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int idx = tid + k * b3::kThreads, r = idx / 16, c = idx % 16;
                d[k] = orow[r];
                v[k] = *reinterpret_cast<const dev::u32x4*>(stg + r * b3::HSTR + c * 16);
            }
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int c = (tid + k * b3::kThreads) % 16;
                if (d[k] >= 0)
                    *reinterpret_cast<dev::u32x4*>(o + int64_t(d[k]) * a.H + t.n0 + pass * (b3::BN / 2) + c * 8) = v[k];
            }
            if (pass == 0) lds_barrier();
        }
    }
    lds_barrier();              // the staging is read: the next tile's slice 2 goes into its buffer
}

template <int MODE>
__global__ void __launch_bounds__(b3::kThreads) __attribute__((amdgpu_waves_per_eu(b3::kWavesPerSimd, b3::kWavesPerSimd)))
k_gemm_b3(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const int n_tiles = a.N / b3::BN;
    const int total = a.tiles[0] * n_tiles;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int x = blockIdx.x % kXcds, stride = gridDim.x / kXcds;
    int i = blockIdx.x / kXcds;
    if (i >= per_xcd || x * per_xcd + i >= total) return;
    const int nk = a.K / b3::BK;
    // the descriptors of the first two tiles are read while no slice is in flight (their
    // loads would otherwise wait for the slices ahead of them); later ones in the epilogue two
    // tiles ahead, before its stores
    b3::Tile cur = b3::make_tile<MODE>(a, x * per_xcd + i, n_tiles);
    int in = i + stride;
    bool has_next = in < per_xcd && x * per_xcd + in < total;
    b3::Tile nx = has_next ? b3::make_tile<MODE>(a, x * per_xcd + in, n_tiles) : cur;
#pragma unroll
    for (int s = 0; s < 3; ++s) b3::issue(lds8, a, cur, s, s);
    int g0 = 0;
    bool first = true;
    while (true) {
        const int in2 = in + stride;
        const bool has_next2 = has_next && in2 < per_xcd && x * per_xcd + in2 < total;
        const int nn_lid = has_next2 ? x * per_xcd + in2 : -1;
        b3::Tile nn = nx;
        switch (cur.fa) {
            case 2: b3_tile<MODE, 2>(a, lds8, cur, nx, has_next, g0, first, nn_lid, nn); break;
            case 1: b3_tile<MODE, 1>(a, lds8, cur, nx, has_next, g0, first, nn_lid, nn); break;
            default: b3_tile<MODE, 0>(a, lds8, cur, nx, has_next, g0, first, nn_lid, nn); break;
        }
        if (!has_next) break;
        g0 = (g0 + nk) % 3;
        b3::issue(lds8, a, nx, 2, (g0 + 2) % 3);       // the new tile's slices 0 and 1 have landed
        cur = nx;
        nx = nn;
        has_next = has_next2;
        in = in2;
        first = false;
    }
}

// The GEMM stages use more than the default 64 KiB of LDS per workgroup.
hipError_t allow_lds() {
    static hipError_t once = [] {
        const void* ks[2] = {reinterpret_cast<const void*>(&k_gemm<0>), reinterpret_cast<const void*>(&k_gemm<1>)};
        for (const void* k : ks) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
            if (e != hipSuccess) return e;
        }
        const void* kd[2] = {reinterpret_cast<const void*>(&k_gemm_dma<0>), reinterpret_cast<const void*>(&k_gemm_dma<1>)};
        for (const void* k : kd) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, dma::kLdsBytes);
            if (e != hipSuccess) return e;
        }
        const void* kb[2] = {reinterpret_cast<const void*>(&k_gemm_big<0, false>),
                             reinterpret_cast<const void*>(&k_gemm_big<1, false>)};
        for (const void* k : kb) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, big::Lay<false>::kLdsBytes);
            if (e != hipSuccess) return e;
        }
        const void* k3[2] = {reinterpret_cast<const void*>(&k_gemm_b3<0>), reinterpret_cast<const void*>(&k_gemm_b3<1>)};
        for (const void* k : k3) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, b3::kLdsBytes);
            if (e != hipSuccess) return e;
        }
        const void* kf[2] = {reinterpret_cast<const void*>(&k_gemm_big<0, true>),
                             reinterpret_cast<const void*>(&k_gemm_big<1, true>)};
        for (const void* k : kf) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, big::Lay<true>::kLdsBytes);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    return once;
}

// Upper bound on the tile count of a list built with row-tile height bm (every expert may
// add one partial tile, and the shared expert's T rows one more).
int max_tiles(const moe_config& c, int32_t T, int bm) {
    const int64_t pairs = int64_t(T) * c.top_k;
    return int((pairs + bm - 1) / bm + c.n_experts + 1 + (T + bm - 1) / bm + 1);
}

}  // namespace

// Tile list: [0] count, [1 .. max] (entry << 16) | m_tile, then from a 16-byte boundary one
// int4 record per row tile.
int64_t tile_rec_index(const moe_config& c, int32_t T) {
    return (1 + int64_t(max_tiles(c, T, BM < dma::BM ? BM : dma::BM)) + 3) / 4 * 4;
}
int64_t gemm_tile_ints(const moe_config& c, int32_t T) {
    return tile_rec_index(c, T) + 4 * int64_t(max_tiles(c, T, BM < dma::BM ? BM : dma::BM));
}

bool gemm_shape_supported(const moe_config& c) {
    if (c.w_dtype == MOE_W_F32) return false;
    return c.hidden % BK == 0 && c.inter % BK == 0 && (2 * c.inter) % BN == 0 && c.hidden % BN == 0 &&
           c.hidden >= BK && c.inter >= BK;
}

hipError_t launch_ffn_gemm(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                           const int32_t* offsets, const int32_t* perm, const void* slot_base,
                           const void* shared, const ExpertList& list, void* o, void* ws, hipStream_t s) {
    const WsLayout W = ws_layout(c, T);
    int32_t* tiles = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + W.tiles);
    const bool fp4 = c.w_dtype == MOE_W_MXFP4;
    // kernel per GEMM: 2 large-tile, 3 three-stage 128 x 256, 1 pipelined 128 x 256 (bf16 with
    // fewer than three K slices of 64), 0 register-staged (MXFP4 shapes the large tile does not
    // take; every bf16 shape gemm_shape_supported accepts fits 3 or 1).  The large tile needs
    // K loops long enough to pay for its per-tile start and epilogue; on the 8K-token chunk of
    // the 2048 x 768 layer it runs GEMM 1 (K = 2048) in 430-438 us against 496 us on the
    // three-stage kernel, and GEMM 2 (K = 768) in 292-294 us against 300-302 us.  Below K = 512
    // the three-stage kernel (persistent, two slices of lookahead) takes bf16 GEMMs.
    auto kind = [&](int N, int K) {
        // large tile: an even slice count, A row offsets (rows of x or h times the row bytes)
        // in 32 bits and, for MXFP4, the tile's scales within their LDS region
        const int64_t a_rows = int64_t(T) * c.top_k + T;
        const bool big_ok = N % big::BN == 0 && K % (2 * big::BK) == 0 &&
                            a_rows * K * 2 < (int64_t(1) << 32) && (!fp4 || K <= big::kMaxKFp4);
        if (fp4) return big_ok ? 2 : 0;
        const bool b3_ok = N % b3::BN == 0 && K % b3::BK == 0 && K / b3::BK >= 3 && a_rows * K * 2 < (int64_t(1) << 32);
        if (K >= 512 && big_ok) return 2;
        return b3_ok ? 3 : 1;
    };
    auto bm_of = [](int kd) { return kd == 3 ? b3::BM : kd == 2 ? big::BM : kd == 1 ? dma::BM : BM; };
    const int kind1 = kind(2 * c.inter, c.hidden), kind2 = kind(c.hidden, c.inter);
    TileMapArgs tm;
    tm.offsets = offsets;
    tm.T = T;
    tm.bm = bm_of(kind1);
    tm.tiles = tiles;
    tm.rec = reinterpret_cast<int4*>(tiles + tile_rec_index(c, T));
    tm.list = list;
    hipLaunchKernelGGL(k_tile_map, dim3(1), dim3(1024), 0, s, tm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmArgs a;
    a.slot_base = static_cast<const uint8_t*>(slot_base);
    a.shared_blob = static_cast<const uint8_t*>(shared);
    a.blob_bytes = lay.bytes;
    a.offsets = offsets;
    a.perm = perm;
    a.tiles = tiles;
    a.rec = tm.rec;
    a.T = T;
    a.k = c.top_k;
    a.I = c.inter;
    a.H = c.hidden;
    a.list = list;
    if ((e = allow_lds()) != hipSuccess) return e;
    auto launch = [&](int kd, int mode, int bm) {
        const int bn = kd == 3 ? b3::BN : kd == 2 ? big::BN : kd == 1 ? dma::BN : BN;
        a.grid = (max_tiles(c, T, bm) * (a.N / bn) + kXcds - 1) / kXcds * kXcds;
        a.mode = mode;
        if (kd == 2 || kd == 3) {
            // persistent: at most one workgroup per CU (a multiple of the XCD count)
            static const int n_cu = [] {
                int dev = 0, n = 0;
                if (hipGetDevice(&dev) != hipSuccess ||
                    hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
                    n = 0;
                return n;
            }();
            const int cap = n_cu >= kXcds ? n_cu / kXcds * kXcds : kXcds;
            a.grid = a.grid < cap ? a.grid : cap;
            const dim3 g(a.grid), b(big::kThreads);
            if (kd == 3) {
                if (mode == 0) hipLaunchKernelGGL((k_gemm_b3<0>), g, dim3(b3::kThreads), b3::kLdsBytes, s, a);
                else hipLaunchKernelGGL((k_gemm_b3<1>), g, dim3(b3::kThreads), b3::kLdsBytes, s, a);
            } else if (fp4) {
                if (mode == 0) hipLaunchKernelGGL((k_gemm_big<0, true>), g, b, big::Lay<true>::kLdsBytes, s, a);
                else hipLaunchKernelGGL((k_gemm_big<1, true>), g, b, big::Lay<true>::kLdsBytes, s, a);
            } else {
                if (mode == 0) hipLaunchKernelGGL((k_gemm_big<0, false>), g, b, big::Lay<false>::kLdsBytes, s, a);
                else hipLaunchKernelGGL((k_gemm_big<1, false>), g, b, big::Lay<false>::kLdsBytes, s, a);
            }
        } else if (kd == 1) {
            if (mode == 0)
                hipLaunchKernelGGL((k_gemm_dma<0>), dim3(a.grid), dim3(dma::kThreads), dma::kLdsBytes, s, a);
            else
                hipLaunchKernelGGL((k_gemm_dma<1>), dim3(a.grid), dim3(dma::kThreads), dma::kLdsBytes, s, a);
        } else {
            if (!fp4) return hipErrorInvalidValue;          // the register-staged kernel takes MXFP4 only
            if (mode == 0)
                hipLaunchKernelGGL((k_gemm<0>), dim3(a.grid), dim3(kThreads), kLdsBytes, s, a);
            else
                hipLaunchKernelGGL((k_gemm<1>), dim3(a.grid), dim3(kThreads), kLdsBytes, s, a);
        }
        return hipGetLastError();
    };
    uint8_t* hbuf = static_cast<uint8_t*>(ws) + W.h;
    // GEMM 1: [rows x H] . [2I x H]^T -> h [rows x I]
    a.off_w = lay.gu;
    a.off_s = lay.gu_scale;
    a.a_src = static_cast<const uint8_t*>(x);
    a.out = hbuf;
    a.K = c.hidden;
    a.N = 2 * c.inter;
    if ((e = launch(kind1, 0, tm.bm)) != hipSuccess) return e;
    // GEMM 2: h [rows x I] . [H x I]^T -> o [pair rows x H]
    a.off_w = lay.d;
    a.off_s = lay.d_scale;
    a.a_src = hbuf;
    a.out = o;
    a.K = c.inter;
    a.N = c.hidden;
    const int bm2 = bm_of(kind2);
    if (bm2 != tm.bm) {            // the list is rebuilt after GEMM 1 has read it (same stream)
        tm.bm = bm2;
        hipLaunchKernelGGL(k_tile_map, dim3(1), dim3(1024), 0, s, tm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return launch(kind2, 1, bm2);
}

}  // namespace moe

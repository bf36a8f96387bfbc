// Internal declarations shared by the host-side C++ and the HIP launchers of
// libmoecache.  Not part of the public ABI (include/moe.h).
#pragma once

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 512;       // E limit: ids fit in 10 bits, masks in 16 words
constexpr int kMaxTopK = 16;
constexpr int kDecodeMaxT = 8;         // T <= 8: batched GEMV path; larger T: grouped GEMM
constexpr int kSharedTag = 1023;       // list entry tag of the shared expert
constexpr int kPermChunk = 1024;       // pairs per permutation chunk (one workgroup)
constexpr int kSmallRouteMaxPairs = 4096;  // fused route+permute in one workgroup up to here

inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Byte layout of one expert blob (identical in the host pool and the device slots).
//   fp32 / bf16: Wgu [2I][H] then Wd [H][I], K contiguous.  Wgu interleaves gate and
//                up rows in blocks of 16: row r holds gate row (r/32)*16 + r%32 when
//                r%32 < 16, else up row (r/32)*16 + r%32 - 16.
//   MXFP4:       Wgu codes [2I][H/2], Wgu scales [2I][H/32], Wd codes [H][I/2],
//                Wd scales [H][I/32]; same row interleave.
struct BlobLayout {
    int64_t gu = 0, gu_scale = 0, d = 0, d_scale = 0, bytes = 0;
};

int validate_config(const moe_config* c, std::string* why);
BlobLayout blob_layout(const moe_config& c);
inline int act_bytes(const moe_config& c) { return c.w_dtype == MOE_W_F32 ? 4 : 2; }

// Scratch layout inside the caller's workspace (pure scratch: nothing in it needs a value
// before a call).  hist/base: permutation histograms of the large-T route; tiles: the grouped
// GEMM's tile list; h: SwiGLU activations; o: decode pair outputs of moe_expert_ffn_merge
// when its down projection and merge run as separate kernels.
struct WsLayout {
    int64_t hist = 0, base = 0, tiles = 0, h = 0, o = 0, bytes = 0;
};
int64_t gemm_tile_ints(const moe_config& c, int32_t T);  // tile-list entries of the grouped GEMM
WsLayout ws_layout(const moe_config& c, int32_t max_T);

// A small persistent worker pool for the host FFN.
class ThreadPool {
public:
    ~ThreadPool();
    void run(int n_items, int n_threads, const std::function<void(int)>& fn);

private:
    void resize(int n);
    std::vector<std::thread> threads_;
    std::mutex mu_;
    std::condition_variable cv_, done_cv_;
    const std::function<void(int)>* job_ = nullptr;
    int n_items_ = 0;
    std::atomic<int> next_{0};
    int busy_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

}  // namespace moe

struct moe_ctx {
    moe_config cfg;
    moe::BlobLayout lay;
    // global LRU over (layer, expert) keys
    std::vector<int32_t> key_of_slot;    // [C] cache key held by a slot, -1 = free
    std::vector<int64_t> recency;        // [C] (step counter << 20) | (n - rank)
    std::vector<int32_t> slot_of_key;    // [L*E]
    std::vector<int64_t> in_step;        // [L*E] counter stamp of the step using the key
    std::vector<int32_t> count_scratch;  // [E]
    int64_t counter = 0;
    moe_stats stats{};
    // bound pools
    void* d_slots = nullptr;
    int32_t n_bound_slots = 0;
    const void* h_pool = nullptr;
    int32_t n_pool = 0;
    hipEvent_t fill_event = nullptr;
    // layer streaming: [0] start, [1..2] upload into buffer b done, [3..4] compute on buffer b done
    hipEvent_t stream_ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    // host FFN workers and scratch
    moe::ThreadPool pool;
    std::vector<float> hx, hh, ho;
    std::string err;
};

namespace moe {

int fail(moe_ctx* ctx, int code, const std::string& msg);
int hip_fail(moe_ctx* ctx, hipError_t e, const char* what);

// moe_expert_ffn_merge with the workspace supplied by `workspace(T, &ptr)` once the arguments
// are valid; a status other than MOE_OK from it is returned as is (it sets the message).
int expert_ffn_merge(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids, const int32_t* d_topk_ids,
                     const float* d_topk_w, const void* d_slot_base, const int32_t* h_experts, const int32_t* h_slots,
                     int32_t n, const void* d_shared, int32_t with_shared, const float* d_y_host, void* d_out,
                     const std::function<int(int32_t, void**)>& workspace, hipStream_t s);

// ---- kernel launchers (defined in the .hip files) ----
struct ExpertList {
    int32_t n;                 // entries used
    int32_t ent[kMaxExperts + 1];  // expert | slot << 10; expert == kSharedTag: shared
};

// Decode (T <= kDecodeMaxT) expert list with per-expert token sets from the host's
// top-k ids: token t uses the expert when bit t of tokmask is set, as pair
// t*k + ((jpack >> 4t) & 15).  The shared expert uses every token.
constexpr int kMaxDecodeList = kDecodeMaxT * kMaxTopK + 1;
struct DecodeList {
    int32_t n;
    int32_t ent[kMaxDecodeList];      // expert | slot << 10; kSharedTag: shared expert
    uint32_t tokmask[kMaxDecodeList];
    uint32_t jpack[kMaxDecodeList];
};

hipError_t launch_ffn_decode(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                             const void* slot_base, const void* shared, const DecodeList& list, void* o, void* ws,
                             hipStream_t s);
// Decode FFN with the gate-weighted merge fused into the down kernel: out = the result of
// moe_merge_partial over the pair outputs launch_ffn_decode would write (bit-identical).
hipError_t launch_ffn_decode_merge(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                                   const void* slot_base, const void* shared, const DecodeList& list,
                                   const int32_t* ids, const float* w, const uint32_t* mask, int32_t with_shared,
                                   const float* y_host, void* out, void* ws, hipStream_t s);
bool decode_shape_supported(const moe_config& c);

hipError_t launch_route(const moe_config& c, const float* logits, int32_t T, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv, void* ws,
                        hipStream_t s);

// Returns hipSuccess, or hipErrorInvalidValue when no kernel variant fits the shape.
hipError_t launch_ffn_gemv(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                           const int32_t* offsets, const int32_t* perm, const void* slot_base,
                           const void* shared, const ExpertList& list, void* o, void* ws,
                           hipStream_t s);
bool gemv_shape_supported(const moe_config& c);


hipError_t launch_ffn_gemm(const moe_config& c, const BlobLayout& lay, const void* x, int32_t T,
                           const int32_t* offsets, const int32_t* perm, const void* slot_base,
                           const void* shared, const ExpertList& list, void* o, void* ws,
                           hipStream_t s);
bool gemm_shape_supported(const moe_config& c);

hipError_t launch_router_logits(const moe_config& c, const void* x, int32_t T, const float* wr, float* out,
                                hipStream_t s);
hipError_t launch_merge(const moe_config& c, const void* o, const int32_t* ids, const float* w,
                        const uint32_t* gpu_mask, int32_t with_shared, const float* y_host,
                        int32_t T, void* out, hipStream_t s);

}  // namespace moe

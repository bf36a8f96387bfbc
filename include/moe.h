/*
 * moe.h — C ABI of libmoecache: one MoE layer's forward pass over a
 * slot-limited expert cache, for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes comes from the FreeToken pages:
 *   [A] asapai.co.kr, "Running 753B GLM-5.2 on a single workstation GPU:
 *       FreeToken doubles llama.cpp's throughput"
 *   [B] banandre.com, "The 284B Model on a 32GB GPU Trick: How FreeToken Proves
 *       Hardware Is a Software Problem"
 *   [Z] zubnet.ai, news item on FreeToken and Unsloth GGUF
 * A router picks k experts per token ([B] "Sparsity Is a Lie"); on a decode
 * step the experts that miss the GPU cache are split by q* ~= m*B_P/B_H into
 * experts uploaded to GPU slots and experts computed on the host CPU; the two
 * partial sums are added after the layer ([B] "The q* Policy").  The cache is
 * one LRU over all layers, updated on misses, starting empty ([A] "Abandoning
 * fixed offloading ...", [B] "Semantic-Aware Caching", [B] "Elastic Memory").
 * Prefill streams whole layers through two device buffers ([A] same section).
 *
 * Conventions (all entry points):
 *   - Return an int status (MOE_OK = 0, negative on error).  Nothing aborts and
 *     no C++ exception crosses the ABI.  A call that returns an error has no side
 *     effect on the context, the cache or any output (inputs are validated first).
 *   - The caller owns every buffer (device memory from hipMalloc or torch, host
 *     memory from hipHostMalloc or pinned torch tensors).  The library owns only
 *     the context, its cache state and its HIP events.
 *   - d_ = device pointer, h_ = host pointer.  GPU calls are asynchronous on the
 *     given stream; faults in asynchronous work surface at the caller's sync.
 *   - A context is not thread-safe.  Results are bitwise deterministic run to
 *     run (no floating-point atomics).
 *   - Element formats: weights fp32, bf16 or MXFP4 (OCP MX v1.0: e2m1 codes,
 *     element 2i in the low nibble of byte i, one e8m0 scale per 32 elements
 *     along K); activations and outputs are fp32 for fp32 weights and bf16
 *     otherwise; router logits, gates and partial sums are fp32.
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* bad argument (null pointer, out-of-range id, NaN scale) */
#define MOE_ESHAPE (-2)        /* shape not supported by the config or the kernels */
#define MOE_ECAPACITY (-3)     /* caller array too small */
#define MOE_EHIP (-4)          /* a HIP runtime call failed; moe_last_error has its string */
#define MOE_EUNSUPPORTED (-5)  /* valid request that this library does not implement */
#define MOE_ESTATE (-6)        /* pools not bound, or a call out of order */

/* weight element formats */
#define MOE_W_F32 0
#define MOE_W_BF16 1
#define MOE_W_MXFP4 2

/* integer readings of q* ~= m*B_P/B_H ([B] "The q* Policy") */
#define MOE_Q_NEAREST 0  /* floor((m*B_P)/B_H + 1/2) in IEEE double, clamped to [0, m] */
#define MOE_Q_ARGMIN 1   /* smallest q minimising max(q/B_P, (m-q)/(B_H-B_P)) */

typedef struct moe_config {
    int32_t hidden;        /* H: model width; multiple of 64 (of 256 for MXFP4) */
    int32_t inter;         /* I: expert intermediate width; multiple of 32 */
    int32_t n_experts;     /* E: routed experts per layer, 1..512 */
    int32_t top_k;         /* k: experts per token, 1..min(E, 16) */
    int32_t n_shared;      /* 0 or 1 always-on shared expert (gate 1, never cached) */
    int32_t n_slots;       /* C: device expert slots of the global LRU cache (>= 0) */
    int32_t n_layers;      /* layers sharing the cache, key = (layer, expert); >= 1 */
    int32_t w_dtype;       /* MOE_W_F32 | MOE_W_BF16 | MOE_W_MXFP4 */
    int32_t renormalize;   /* 1: gates are the softmax renormalised over the top k;
                              0: softmax over all E experts */
    int32_t q_round;       /* MOE_Q_NEAREST | MOE_Q_ARGMIN */
    double bp_gbps;        /* B_P: host->GPU link bandwidth (e.g. 52.7) */
    double bh_gbps;        /* B_H: host memory bandwidth available to experts (e.g. 77.3) */
} moe_config;

/* One decode step's cache plan ([B] "The q* Policy"; [A] "Abandoning fixed
 * offloading ...").  The caller allocates every array; each set array needs
 * `cap` >= the number of distinct experts of the step (min(E, T*k) suffices),
 * slot_of_expert needs E entries (it may be NULL).  All sets are in step order:
 * more tokens first, then lower expert id. */
typedef struct moe_plan {
    int32_t cap;
    int32_t n_distinct;       /* |S_t| */
    int32_t n_hit;
    int32_t n_miss;           /* m */
    int32_t n_fill;           /* q = min(q*(m), C - n_hit) */
    int32_t n_host;           /* m - q */
    int32_t layer;
    int32_t* distinct;        /* [cap] S_t */
    int32_t* hit;             /* [cap] resident experts */
    int32_t* hit_slot;        /* [cap] their slots */
    int32_t* fill;            /* [cap] misses uploaded to the GPU (first q misses) */
    int32_t* fill_slot;       /* [cap] destination slots */
    int32_t* fill_victim;     /* [cap] evicted cache key (layer*E + expert), -1 for a free slot */
    int32_t* host;            /* [cap] misses computed on the CPU (not inserted) */
    int32_t* slot_of_expert;  /* [E] this layer's slot table after the step, -1 = absent */
} moe_plan;

typedef struct moe_stats {
    int64_t steps;
    int64_t distinct;        /* distinct (expert, step) reads */
    int64_t hits;
    int64_t misses;
    int64_t fills;
    int64_t host;
    int64_t evictions;
} moe_stats;

/* Result of a cache resize (moe_lru_resize); arrays are caller-owned with capacity cap. */
typedef struct moe_resize {
    int32_t cap;        /* capacity of each array */
    int32_t n_move;     /* kept entries that leave a slot past the new size */
    int32_t n_evict;    /* entries dropped by a shrink */
    int32_t* move_src;  /* [cap] slot an entry leaves (>= new size) */
    int32_t* move_dst;  /* [cap] free slot below the new size it moves to */
    int32_t* evicted;   /* [cap] cache keys (layer*E + expert) dropped, in slot order */
} moe_resize;

typedef struct moe_ctx moe_ctx;

/* ---------------------------------------------------------------- context */
/* Validate *cfg and create a context.  Makes no HIP call (usable on a host
 * without a GPU for the planner and the host FFN).  Errors: MOE_EINVAL (null),
 * MOE_ESHAPE (sizes), MOE_EUNSUPPORTED (dtype).  *out is NULL on error. */
int moe_create(const moe_config* cfg, moe_ctx** out);
/* Free the context and its HIP events; NULL is a no-op.  Never frees caller memory. */
void moe_destroy(moe_ctx* ctx);
/* Message of the last failed call on ctx (owned by ctx, valid until the next call). */
const char* moe_last_error(const moe_ctx* ctx);
/* Static name of a status code. */
const char* moe_status_string(int status);

/* Bytes of one expert blob (the slot stride; a multiple of 256), or a negative
 * status for an invalid config.  The blob is the library's own layout, the same
 * in the host pool and in the device slots, so a fill is one contiguous copy
 * ([B] "Elastic Memory": experts are read into their final host layout). */
int64_t moe_expert_bytes(const moe_config* cfg);
/* Device scratch bytes needed by moe_route + moe_expert_ffn (+ moe_expert_ffn_merge) for
 * up to max_T tokens.  The workspace is scratch (caller-owned, no initial value needed);
 * calls that share a workspace must be ordered (one stream, or events). */
int64_t moe_workspace_bytes(const moe_config* cfg, int32_t max_T);
/* Rows of the pair-output buffer d_o for T tokens: T*k (+ T with a shared expert).  Each
 * row holds H values in the activation dtype (fp32 for fp32 weights, else bf16). */
int64_t moe_pair_rows(const moe_config* cfg, int32_t T);

/* Pack one expert from natural layout into a blob (host memory, moe_expert_bytes).
 *   fp32 / bf16: wg, wu [I][H] and wd [H][I] row-major, elements float or bf16 bits;
 *                sg, su, sd must be NULL.
 *   MXFP4:       wg, wu [I][H/2] and wd [H][I/2] code bytes; sg, su [I][H/32] and
 *                sd [H][I/32] e8m0 scales (0xFF = NaN is rejected: MOE_EINVAL). */
int moe_pack_expert(const moe_config* cfg, const void* wg, const void* wu, const void* wd,
                    const uint8_t* sg, const uint8_t* su, const uint8_t* sd, void* blob);

/* Bind the pools used by moe_fill and moe_host_ffn ([A] "Abandoning fixed offloading ...":
 * a GPU expert cache of limited capacity in front of the full expert pool in host memory;
 * [B] "Elastic Memory": the host copy is kept in its final layout, and the GPU holds as
 * many expert slots as its memory budget allows).
 *   d_slots: device, n_slots blobs (n_slots <= cfg->n_slots), caller-owned; slot i is
 *            the blob at d_slots + i*moe_expert_bytes;
 *   h_pool:  host (pinned for asynchronous fills), n_pool = n_layers*E blobs in
 *            key order (layer*E + expert), caller-owned.
 * The library keeps the pointers, never frees them, and reads / writes them only in
 * moe_fill, moe_move_slots, moe_prefill_stream and moe_host_ffn.  Either pointer may be
 * NULL when the corresponding calls are not used.  Errors (no state change): MOE_EINVAL
 * (n_slots out of range, a device pool missing, n_pool != n_layers*E).  Makes no HIP call
 * (the fill event is created by the first moe_fill / moe_upload). */
int moe_bind_pools(moe_ctx* ctx, void* d_slots, int32_t n_slots, const void* h_pool, int32_t n_pool);

/* ---------------------------------------------------------------- router */
/* Router logits of T tokens (async on s): d_logits[t][e] = sum_h d_x[t][h] * d_wr[e][h],
 * accumulated in fp32.  d_x [T][H] in the activation dtype (fp32 for fp32 weights, else
 * bf16); d_wr [E][H] fp32, one contiguous row of router weights per expert; d_logits [T][E]
 * fp32 (the input of moe_route).  T == 0 is a valid no-op.  ([B] "Sparsity Is a Lie": a
 * small router scores the experts of each token.) */
int moe_router_logits(moe_ctx* ctx, const void* d_x, int32_t T, const float* d_wr, float* d_logits,
                      hipStream_t s);
/* Softmax + top-k and token-by-expert permutation of T tokens (async on s).
 *   d_logits [T][E] fp32 (finite; NaN order is unspecified);
 *   d_topk_ids [T][k] int32 (logit descending, lower id first on equal logits);
 *   d_topk_w [T][k] fp32 gates; d_counts [E]; d_offsets [E+1] exclusive prefix
 *   sums; d_perm [T*k] pair ids p = t*k + j grouped by expert, ascending p within
 *   an expert; d_inv [T*k] with inv[perm[i]] = i.  d_ws: moe_workspace_bytes.
 *   T == 0 is a valid no-op.  ([B] "Sparsity Is a Lie") */
int moe_route(moe_ctx* ctx, const float* d_logits, int32_t T, int32_t* d_topk_ids, float* d_topk_w,
              int32_t* d_counts, int32_t* d_offsets, int32_t* d_perm, int32_t* d_inv, void* d_ws,
              hipStream_t s);

/* ---------------------------------------------------------------- cache planner (host) */
/* q* for m misses ([B] "The q* Policy").  Pure; negative m gives 0. */
int32_t moe_qstar(int32_t m, double bp, double bh, int32_t rounding);
/* Plan one decode step of `layer` from the host copy of its top-k ids
 * h_topk_ids [T][k] and update the cache: hits, q* fills (evicting the least
 * recently used expert not used in this step), host set.  ([A] "Abandoning fixed
 * offloading ...": the decode cache is one LRU over the experts of all layers, updated on
 * misses; [B] "The q* Policy": of the m misses, about m*B_P/B_H are copied to the GPU and
 * the rest computed on the CPU; [B] "Elastic Memory": the cache starts empty.)  The ids
 * are caller-owned and only read; the plan's arrays are caller-owned and written.
 * Synchronous, host only.  Errors (no state change): MOE_EINVAL (ids out of range or
 * repeated within a token, bad layer), MOE_ECAPACITY (plan->cap too small). */
int moe_lru_step(moe_ctx* ctx, int32_t layer, const int32_t* h_topk_ids, int32_t T, moe_plan* plan);
/* Replay n_steps decode steps of `layer` (ids [n_steps][T][k], host, read only) in order,
 * exactly as n_steps calls of moe_lru_step would ([A] "Abandoning fixed offloading ...":
 * the pages measure their miss rates by replaying routing traces against the cache).
 * plans may be NULL (then only *stats is filled), else a caller-owned array of n_steps
 * plans; stats (may be NULL) receives the cumulative statistics after the replay.  All ids
 * are validated before the cache is touched (errors as moe_lru_step, no state change). */
int moe_lru_replay(moe_ctx* ctx, int32_t layer, const int32_t* h_topk_ids, int32_t n_steps, int32_t T,
                   moe_plan* plans, moe_stats* stats);
/* Empty the cache (cold start) and zero the statistics. */
int moe_lru_reset(moe_ctx* ctx);
/* This layer's current slot table (h_slot_of_expert [E], -1 = absent). */
int moe_lru_slots(const moe_ctx* ctx, int32_t layer, int32_t* h_slot_of_expert);
/* Elastic slot pool ([B] "Elastic Memory": at a scheduler safe point the GPU expert
 * cache is rebuilt under a new VRAM budget without reloading the host pool).  Host only,
 * between steps.  Shrink (new_slots < current): the new_slots most recently used entries
 * stay, the others are evicted; kept entries in slots >= new_slots move to the lowest free
 * slots below new_slots (in ascending source-slot order).  Grow: every entry stays and
 * slots are added free.  The returned moves are applied to the device pool with
 * moe_move_slots before the pool is rebound at the new size (moe_bind_pools).  0 <=
 * new_slots <= 2^21.  Errors (no state change): MOE_EINVAL, MOE_ECAPACITY (cap below the
 * moves or evictions). */
int moe_lru_resize(moe_ctx* ctx, int32_t new_slots, moe_resize* out);
/* Copy every move of a resize inside the bound device slot pool (device to device, async
 * on s).  Every source and destination must lie in the bound pool. */
int moe_move_slots(moe_ctx* ctx, const moe_resize* r, hipStream_t s);
/* Cumulative statistics since create/reset. */
int moe_lru_stats(const moe_ctx* ctx, moe_stats* stats);

/* ---------------------------------------------------------------- miss fills */
/* Upload the plan's fills from the bound host pool into the bound device slots:
 * one hipMemcpyAsync per fill on `side`, then the context's fill event is
 * recorded on `side` ([B] "The q* Policy": copy the weights across PCIe and
 * execute on the GPU).  Requires moe_bind_pools with both pools. */
int moe_fill(moe_ctx* ctx, const moe_plan* plan, hipStream_t side);
/* Make stream s wait for the last moe_fill / moe_upload of this context. */
int moe_fill_wait(moe_ctx* ctx, hipStream_t s);
/* Asynchronous copy of `bytes` from host to device on `side` followed by the
 * fill event (whole-layer streaming into a prefill buffer, [A] "Abandoning fixed
 * offloading ...": full-layer double buffering). */
int moe_upload(moe_ctx* ctx, void* d_dst, const void* h_src, int64_t bytes, hipStream_t side);

/* ---------------------------------------------------------------- expert FFN */
/* GPU SwiGLU experts over device slots (async on s) ([B] "Sparsity Is a Lie": each routed
 * expert is a small feed-forward network; [B] "The q* Policy": experts resident in the GPU
 * cache, or just copied there, are computed on the GPU):
 *   o[p] = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)) for every pair p = t*k + j whose
 *   expert e = topk_ids[t][j] is listed in h_experts, read from the blob at
 *   d_slot_base + h_slots[i]*moe_expert_bytes; with with_shared = 1 also
 *   o[T*k + t] for the shared expert blob d_shared (all tokens).
 *   d_x [T][H] activations; h_experts / h_slots: host arrays of n (<= E) distinct
 *   expert ids and slot indices (listed experts that no token uses are skipped);
 *   d_o [moe_pair_rows][H] in the activation dtype, each pair's result rounded once
 *   (rows of unlisted experts are not written);
 *   d_ws: moe_workspace_bytes(max_T >= T).
 *   Which tokens use an expert comes from h_topk_ids (host copy [T][k] of the
 *   step's ids, as moe_lru_step consumes) when given and T <= 8; the kernels then
 *   do not read d_offsets / d_perm and need not wait for moe_route.  Otherwise
 *   d_offsets / d_perm from moe_route are read on the device.
 * T <= 8 runs the decode path (HBM-bound batched GEMV); larger T runs the
 * grouped GEMM on MFMA.  Errors: MOE_EINVAL (ids, null), MOE_ESHAPE. */
int moe_expert_ffn(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids,
                   const int32_t* d_offsets, const int32_t* d_perm, const void* d_slot_base,
                   const int32_t* h_experts, const int32_t* h_slots, int32_t n, const void* d_shared,
                   int32_t with_shared, void* d_o, void* d_ws, hipStream_t s);

/* CPU SwiGLU experts of the plan's host set from the bound host pool:
 * h_y[t] = sum over j with topk_ids[t][j] in plan->host of w[t][j]*FFN(x_t),
 * fp32 [T][H] (fully written; zero rows where nothing is on the host), with
 * n_threads worker threads (<= 0: hardware concurrency).  ([B] "The q* Policy":
 * leave the weights in system RAM and execute on the CPU.)  Synchronous. */
int moe_host_ffn(moe_ctx* ctx, const void* h_x, int32_t T, const int32_t* h_topk_ids,
                 const float* h_topk_w, const moe_plan* plan, float* h_y, int32_t n_threads);

/* ---------------------------------------------------------------- merge */
/* Gate-weighted un-permute and exact merge of the partial sums (async on s):
 *   out[t] = cast( sum_{j=0..k-1, topk_ids[t][j] in h_gpu_experts} w[t][j]*o[t*k+j]
 *                  + (with_shared ? o[T*k+t] : 0) + (d_y_host ? y_host[t] : 0) )
 * in fp32, in that order; d_o as written by moe_expert_ffn (activation dtype);
 * out is fp32 (fp32 weights) or bf16 [T][H].
 * ([B] "The q* Policy": the partial sums merge exactly after the layer.) */
int moe_merge_partial(moe_ctx* ctx, const void* d_o, const int32_t* d_topk_ids, const float* d_topk_w,
                      const int32_t* h_gpu_experts, int32_t n_gpu, int32_t with_shared,
                      const float* d_y_host, int32_t T, void* d_out, hipStream_t s);

/* Decode expert FFN and merge in one call (async on s): out as moe_merge_partial would
 * write it from the pair outputs moe_expert_ffn would write for the same arguments
 * (h_experts doubles as h_gpu_experts), bit for bit, without the pair outputs going
 * through memory when the call lists at most 8 entries (routed experts + the shared
 * one), k <= 8 and the decode kernel reads a down-projection row with at most 32 lanes
 * (the workloads' shapes do: bf16 with I = 768 or 1536, MXFP4 with I = 1536): the down
 * projection and the gate-weighted merge then share one kernel; otherwise the separate
 * kernels run with the pair outputs in d_ws.
 * Decode batches only: T <= 8, h_topk_ids given, and the shapes of the decode kernels
 * (else MOE_ESHAPE); d_topk_ids / d_topk_w are moe_route's outputs for the same step
 * (read on the device, so the call must follow moe_route on s).  Same buffers and
 * errors as the two calls otherwise; d_y_host may be null.  ([B] "The q* Policy": the
 * GPU experts' partial sum, merged exactly with the host part after the layer.) */
int moe_expert_ffn_merge(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids,
                         const int32_t* d_topk_ids, const float* d_topk_w, const void* d_slot_base,
                         const int32_t* h_experts, const int32_t* h_slots, int32_t n, const void* d_shared,
                         int32_t with_shared, const float* d_y_host, void* d_out, void* d_ws, hipStream_t s);

/* moe_expert_ffn_merge without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the scratch lives in one file-scope device array of moe_noalloc_scratch_bytes() bytes
 * (8 MiB) that each GPU the library runs on holds until the process ends.  Same arguments,
 * results (bit for bit) and errors as moe_expert_ffn_merge, without d_ws; the call makes no
 * device allocation and needs no initialised scratch.  Every call on one GPU uses that GPU's
 * array (it keeps the last call's contents), so calls that overlap on one GPU (other streams,
 * other threads or contexts) race: order them.  A batch whose workspace
 * (moe_workspace_bytes(cfg, T)) exceeds the array is refused with MOE_ECAPACITY before any
 * GPU work; MOE_EHIP if the array's device address cannot be obtained. */
int moe_expert_ffn_merge_noalloc(moe_ctx* ctx, const void* d_x, int32_t T, const int32_t* h_topk_ids,
                                 const int32_t* d_topk_ids, const float* d_topk_w, const void* d_slot_base,
                                 const int32_t* h_experts, const int32_t* h_slots, int32_t n, const void* d_shared,
                                 int32_t with_shared, const float* d_y_host, void* d_out, hipStream_t s);
/* Bytes of the scratch array moe_expert_ffn_merge_noalloc uses on each GPU. */
int64_t moe_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------- layer streaming (prefill) */
/* One T-token prefill chunk through cfg.n_layers MoE layers whose expert pools
 * stream from the bound host pool (n_layers*E blobs, layer-major, pinned) into
 * device layer buffers of E blobs each ([A] "Abandoning fixed offloading in favor
 * of measured bandwidth": full-layer double buffering, the next layer's experts
 * cross PCIe while the current layer computes).  Layer l runs moe_route on
 * d_logits + l*T*E, moe_expert_ffn over all E experts of its buffer (slot =
 * expert) plus, when cfg.n_shared, the shared blob d_shared + l*moe_expert_bytes,
 * and moe_merge_partial into d_out + l*T*H (activation dtype).
 *   n_buffers = 2: the upload of layer l+1 runs on `side` while layer l computes
 *     on `s`; it waits only for the compute of layer l-1 (its buffer's last user).
 *   n_buffers = 1: the single-buffer ablation; each upload waits for the compute
 *     of the previous layer.
 *   d_layer_bufs: n_buffers*E blobs (device, caller-owned);
 *   d_x [T][H]: the input of every layer (activation dtype);
 *   d_topk_ids, d_topk_w, d_counts, d_offsets, d_perm, d_inv, d_o, d_ws: as for
 *     moe_route / moe_expert_ffn with max_T >= T, reused by every layer;
 *   d_out [n_layers][T][H].
 * The first upload starts after the work already enqueued on `s`; on return the
 * whole chunk is enqueued and `s` ends with the last layer's merge.  Requires
 * moe_bind_pools with a host pool.  Errors found before anything is enqueued:
 * MOE_EINVAL, MOE_ESTATE (no host pool), MOE_ESHAPE; a HIP error (MOE_EHIP) can
 * leave part of the chunk enqueued. */
int moe_prefill_stream(moe_ctx* ctx, void* d_layer_bufs, int32_t n_buffers, const float* d_logits,
                       const void* d_x, int32_t T, const void* d_shared, int32_t* d_topk_ids, float* d_topk_w,
                       int32_t* d_counts, int32_t* d_offsets, int32_t* d_perm, int32_t* d_inv, void* d_o,
                       void* d_ws, void* d_out, hipStream_t s, hipStream_t side);

#ifdef __cplusplus
}
#endif
#endif /* MOE_CACHE_H */

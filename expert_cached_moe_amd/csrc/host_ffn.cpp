// Host-expert execution: the CPU side of the q* split.
//
// banandre.com, "The 284B Model on a 32GB GPU Trick", section "The q* Policy:
// Math Instead of Guesses": a missed expert that is not copied to the GPU keeps
// its weights in system RAM and is computed on the CPU; its partial sum is added
// to the GPU's after the layer.  The weights are read from the pinned host pool
// in the same blob layout as the device slots (section "Elastic Memory": experts
// are read into their final host layout).
//
// Three parallel phases on a persistent worker pool, each item computed by one
// thread in a fixed order (results do not depend on the thread count):
//   1. h = silu(Wg x) * (Wu x) for blocks of 16 intermediate columns,
//   2. o = Wd h for blocks of 64 output rows,
//   3. y[t] = sum over the token's CPU experts, in top-k order, of gate * o.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "internal.h"

namespace moe {

ThreadPool::~ThreadPool() { resize(0); }

void ThreadPool::resize(int n) {
    if (int(threads_.size()) == n) return;
    {
        std::lock_guard<std::mutex> lk(mu_);
        stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : threads_) t.join();
    threads_.clear();
    stop_ = false;
    for (int i = 0; i < n; ++i) {
        uint64_t g;
        {
            std::lock_guard<std::mutex> lk(mu_);
            g = gen_;
        }
        threads_.emplace_back([this, g]() {
            uint64_t seen = g;
            for (;;) {
                const std::function<void(int)>* job;
                int n_items;
                {
                    std::unique_lock<std::mutex> lk(mu_);
                    cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
                    if (stop_) return;
                    seen = gen_;
                    job = job_;
                    n_items = n_items_;
                }
                for (int it; (it = next_.fetch_add(1)) < n_items;) (*job)(it);
                {
                    std::lock_guard<std::mutex> lk(mu_);
                    if (--busy_ == 0) done_cv_.notify_all();
                }
            }
        });
    }
}

void ThreadPool::run(int n_items, int n_threads, const std::function<void(int)>& fn) {
    if (n_threads <= 1 || n_items <= 1) {
        for (int i = 0; i < n_items; ++i) fn(i);
        return;
    }
    resize(n_threads - 1);
    {
        std::lock_guard<std::mutex> lk(mu_);
        job_ = &fn;
        n_items_ = n_items;
        next_.store(0);
        busy_ = int(threads_.size());
        ++gen_;
    }
    cv_.notify_all();
    for (int it; (it = next_.fetch_add(1)) < n_items;) fn(it);
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [&] { return busy_ == 0; });
    job_ = nullptr;
}

namespace {

inline float bf16_to_f32(uint16_t b) {
    uint32_t u = uint32_t(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// OCP MX v1.0 FP4 E2M1 magnitudes indexed by the three low bits of a code.
constexpr float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

// Decode K weights of one row (format w) into fp32.
void decode_row(int w, const uint8_t* row, const uint8_t* scales, int K, float* out) {
    if (w == MOE_W_F32) {
        std::memcpy(out, row, size_t(K) * 4);
    } else if (w == MOE_W_BF16) {
        const uint16_t* r = reinterpret_cast<const uint16_t*>(row);
        for (int i = 0; i < K; ++i) out[i] = bf16_to_f32(r[i]);
    } else {
        for (int b = 0; b < K / 32; ++b) {
            const float sc = std::ldexp(1.0f, int(scales[b]) - 127);
            for (int i = 0; i < 16; ++i) {
                const uint8_t byte = row[b * 16 + i];
                const uint8_t lo = byte & 15, hi = byte >> 4;
                out[b * 32 + 2 * i] = (lo & 8 ? -kE2M1[lo & 7] : kE2M1[lo & 7]) * sc;
                out[b * 32 + 2 * i + 1] = (hi & 8 ? -kE2M1[hi & 7] : kE2M1[hi & 7]) * sc;
            }
        }
    }
}

// Eight interleaved fp32 partial sums; a fixed summation order.
inline float dot(const float* a, const float* b, int K) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < K; i += 8)
        for (int l = 0; l < 8; ++l) acc[l] += a[i + l] * b[i + l];
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
}

inline float silu(float z) { return z / (1.0f + std::exp(-z)); }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_host_ffn(moe_ctx* ctx, const void* h_x, int32_t T, const int32_t* h_topk_ids,
                            const float* h_topk_w, const moe_plan* plan, float* h_y, int32_t n_threads) {
    if (!ctx || !plan) return MOE_EINVAL;
    const moe_config& c = ctx->cfg;
    const int H = c.hidden, I = c.inter, k = c.top_k, E = c.n_experts;
    if (T < 0) return fail(ctx, MOE_EINVAL, "T < 0");
    if (T == 0) return MOE_OK;
    if (!h_x || !h_topk_ids || !h_topk_w || !h_y) return fail(ctx, MOE_EINVAL, "null host buffer");
    const int nh = plan->n_host;
    if (nh < 0 || nh > E || (nh > 0 && !plan->host)) return fail(ctx, MOE_EINVAL, "bad plan host set");
    if (plan->layer < 0 || plan->layer >= c.n_layers) return fail(ctx, MOE_EINVAL, "bad plan layer");
    if (nh > 0 && !ctx->h_pool) return fail(ctx, MOE_ESTATE, "host pool not bound");
    std::vector<int32_t> he_of(E, -1);
    for (int i = 0; i < nh; ++i) {
        const int e = plan->host[i];
        if (e < 0 || e >= E || he_of[e] >= 0) return fail(ctx, MOE_EINVAL, "host expert out of range or repeated");
        he_of[e] = i;
    }
    for (int64_t p = 0; p < int64_t(T) * k; ++p)
        if (h_topk_ids[p] < 0 || h_topk_ids[p] >= E) return fail(ctx, MOE_EINVAL, "expert id out of range");
    if (n_threads <= 0) n_threads = int(std::max(1u, std::thread::hardware_concurrency()));

    // tokens of each host expert, and the o-row of every host pair
    std::vector<std::vector<int32_t>> toks(nh);
    std::vector<int32_t> orow(size_t(T) * k, -1);
    std::vector<int32_t> row0(nh + 1, 0);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int he = he_of[h_topk_ids[t * k + j]];
            if (he >= 0) toks[he].push_back(t);
        }
    for (int i = 0; i < nh; ++i) row0[i + 1] = row0[i] + int(toks[i].size());
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int he = he_of[h_topk_ids[t * k + j]];
            if (he < 0) continue;
            const auto& v = toks[he];
            orow[t * k + j] = row0[he] + int(std::lower_bound(v.begin(), v.end(), t) - v.begin());
        }
    const int nrows = row0[nh];

    // activations to fp32
    ctx->hx.resize(size_t(T) * H);
    if (c.w_dtype == MOE_W_F32) std::memcpy(ctx->hx.data(), h_x, size_t(T) * H * 4);
    else
        for (int64_t i = 0; i < int64_t(T) * H; ++i)
            ctx->hx[i] = bf16_to_f32(static_cast<const uint16_t*>(h_x)[i]);
    ctx->hh.assign(size_t(std::max(nrows, 1)) * I, 0.0f);
    ctx->ho.assign(size_t(std::max(nrows, 1)) * H, 0.0f);

    const BlobLayout& L = ctx->lay;
    const int wdt = c.w_dtype;
    const int64_t esz = wdt == MOE_W_F32 ? 4 : 2;
    auto blob_of = [&](int he) {
        const int64_t key = int64_t(plan->layer) * E + plan->host[he];
        return static_cast<const uint8_t*>(ctx->h_pool) + key * L.bytes;
    };
    auto row_ptr = [&](const uint8_t* blob, bool gu, int64_t r, int K, const uint8_t** sc) {
        if (wdt == MOE_W_MXFP4) {
            *sc = blob + (gu ? L.gu_scale : L.d_scale) + r * (K / 32);
            return blob + (gu ? L.gu : L.d) + r * (K / 2);
        }
        *sc = nullptr;
        return blob + (gu ? L.gu : L.d) + r * K * esz;
    };

    // phase 1: h for (host expert, block of 16 intermediate columns)
    const int ib = I / 16;
    ctx->pool.run(nh * ib, n_threads, [&](int item) {
        const int he = item / ib, blk = item % ib;
        const uint8_t* blob = blob_of(he);
        const auto& tv = toks[he];
        std::vector<float> wg(H), wu(H);
        for (int r = 0; r < 16; ++r) {
            const int i = blk * 16 + r;
            const uint8_t* sc;
            const uint8_t* pg = row_ptr(blob, true, int64_t(blk) * 32 + r, H, &sc);
            decode_row(wdt, pg, sc, H, wg.data());
            const uint8_t* pu = row_ptr(blob, true, int64_t(blk) * 32 + 16 + r, H, &sc);
            decode_row(wdt, pu, sc, H, wu.data());
            for (size_t q = 0; q < tv.size(); ++q) {
                const float* x = ctx->hx.data() + size_t(tv[q]) * H;
                const float g = dot(wg.data(), x, H), u = dot(wu.data(), x, H);
                ctx->hh[size_t(row0[he] + int(q)) * I + i] = silu(g) * u;
            }
        }
    });
    // phase 2: o = Wd h for (host expert, block of 64 output rows)
    const int rb = (H + 63) / 64;
    ctx->pool.run(nh * rb, n_threads, [&](int item) {
        const int he = item / rb, blk = item % rb;
        const uint8_t* blob = blob_of(he);
        const int ntok = row0[he + 1] - row0[he];
        std::vector<float> wd(I);
        for (int r = blk * 64; r < std::min(H, blk * 64 + 64); ++r) {
            const uint8_t* sc;
            const uint8_t* pd = row_ptr(blob, false, r, I, &sc);
            decode_row(wdt, pd, sc, I, wd.data());
            for (int q = 0; q < ntok; ++q)
                ctx->ho[size_t(row0[he] + q) * H + r] = dot(wd.data(), ctx->hh.data() + size_t(row0[he] + q) * I, I);
        }
    });
    // phase 3: y[t] = sum_j gate * o in top-k order
    ctx->pool.run(T, n_threads, [&](int t) {
        float* y = h_y + size_t(t) * H;
        std::fill(y, y + H, 0.0f);
        for (int j = 0; j < k; ++j) {
            const int r = orow[t * k + j];
            if (r < 0) continue;
            const float w = h_topk_w[t * k + j];
            const float* o = ctx->ho.data() + size_t(r) * H;
            for (int cc = 0; cc < H; ++cc) y[cc] += w * o[cc];
        }
    });
    return MOE_OK;
}

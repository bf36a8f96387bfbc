// Host-side cache planner: the global LRU expert cache and the q* split.
//
// banandre.com, "The 284B Model on a 32GB GPU Trick", section "The q* Policy:
// Math Instead of Guesses": for a step with m cache misses, fill about
// m*B_P/B_H of them into the GPU cache and compute the rest on the CPU, because
// DMA and CPU expert reads share the host memory bandwidth.
// asapai.co.kr, "Running 753B GLM-5.2 on a single workstation GPU", section
// "Abandoning fixed offloading in favor of measured bandwidth": the decode cache
// is a global LRU updated on misses; banandre.com, same page, "Semantic-Aware
// Caching": one LRU spans all MoE layers; "Elastic Memory": the first request
// runs with a cold (empty) cache.
//
// Readings where the pages are open: experts of a step are handled in step
// order (more tokens first, then lower id); the first q misses are filled;
// CPU-computed misses are not inserted; an expert used in step s with rank r of
// n gets recency (s, n - r); a fill takes the lowest free slot, else the slot of
// the least recent resident not used in this step.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "internal.h"

using namespace moe;

extern "C" int32_t moe_qstar(int32_t m, double bp, double bh, int32_t rounding) {
    if (m <= 0) return 0;
    if (!(bh > bp)) return m;  // no residual host bandwidth for the CPU: fill every miss
    if (rounding == MOE_Q_ARGMIN) {
        int32_t best_q = 0;
        double best = 0.0;
        for (int32_t q = 0; q <= m; ++q) {
            const double c = std::max(double(q) / bp, double(m - q) / (bh - bp));
            if (q == 0 || c < best) { best = c; best_q = q; }
        }
        return best_q;
    }
    const double v = std::floor(double(m) * bp / bh + 0.5);
    return v < 0 ? 0 : (v > m ? m : int32_t(v));
}

namespace {

// Validate one step's ids: in range and distinct within each token.
bool step_ids_ok(const moe_ctx* ctx, const int32_t* ids, int32_t T) {
    const int k = ctx->cfg.top_k, E = ctx->cfg.n_experts;
    for (int t = 0; t < T; ++t) {
        const int32_t* r = ids + int64_t(t) * k;
        for (int j = 0; j < k; ++j) {
            if (r[j] < 0 || r[j] >= E) return false;
            for (int i = 0; i < j; ++i)
                if (r[i] == r[j]) return false;
        }
    }
    return true;
}

// Distinct experts of the step in step order.
void step_order(moe_ctx* ctx, const int32_t* ids, int32_t T, std::vector<int32_t>& S) {
    const int k = ctx->cfg.top_k;
    std::vector<int32_t>& cnt = ctx->count_scratch;
    S.clear();
    for (int64_t p = 0; p < int64_t(T) * k; ++p) {
        if (cnt[ids[p]]++ == 0) S.push_back(ids[p]);
    }
    std::sort(S.begin(), S.end(), [&](int32_t a, int32_t b) {
        return cnt[a] != cnt[b] ? cnt[a] > cnt[b] : a < b;
    });
    for (int32_t e : S) cnt[e] = 0;
}

int plan_step(moe_ctx* ctx, int32_t layer, const int32_t* ids, int32_t T, moe_plan* plan) {
    const moe_config& c = ctx->cfg;
    const int E = c.n_experts;
    const int64_t kbase = int64_t(layer) * E;
    std::vector<int32_t> S;
    step_order(ctx, ids, T, S);
    const int n = int(S.size());
    if (plan && plan->cap < n) return fail(ctx, MOE_ECAPACITY, "plan capacity below the distinct experts of the step");

    std::vector<int32_t> hit, hit_slot, miss;
    for (int32_t e : S) {
        const int32_t sl = ctx->slot_of_key[kbase + e];
        if (sl >= 0) { hit.push_back(e); hit_slot.push_back(sl); }
        else miss.push_back(e);
    }
    const int m = int(miss.size());
    int q = moe_qstar(m, c.bp_gbps, c.bh_gbps, c.q_round);
    q = std::min(q, c.n_slots - int(hit.size()));
    if (q < 0) q = 0;

    // ---- mutate the cache (all checks are done) ----
    const int64_t step = ++ctx->counter;
    for (int r = 0; r < n; ++r) ctx->in_step[kbase + S[r]] = step;
    auto key_of = [&](int r) { return (step << 20) | int64_t(n - r); };
    // rank of each expert in S
    std::vector<std::pair<int32_t, int32_t>> rk;
    for (int r = 0; r < n; ++r) rk.emplace_back(S[r], r);
    auto rank_of = [&](int32_t e) {
        for (auto& pr : rk) if (pr.first == e) return pr.second;
        return 0;
    };
    for (size_t i = 0; i < hit.size(); ++i) ctx->recency[hit_slot[i]] = key_of(rank_of(hit[i]));
    std::vector<int32_t> fill_slot, fill_victim;
    int64_t evictions = 0;
    for (int i = 0; i < q; ++i) {
        const int32_t e = miss[i];
        int32_t s_free = -1;
        for (int s = 0; s < c.n_slots; ++s)
            if (ctx->key_of_slot[s] < 0) { s_free = s; break; }
        int32_t victim = -1, slot = s_free;
        if (slot < 0) {
            int64_t best = 0;
            for (int s = 0; s < c.n_slots; ++s) {
                const int32_t key = ctx->key_of_slot[s];
                if (ctx->in_step[key] == step) continue;
                if (slot < 0 || ctx->recency[s] < best) { best = ctx->recency[s]; slot = s; }
            }
            victim = ctx->key_of_slot[slot];
            ctx->slot_of_key[victim] = -1;
            ++evictions;
        }
        ctx->key_of_slot[slot] = int32_t(kbase + e);
        ctx->slot_of_key[kbase + e] = slot;
        ctx->recency[slot] = key_of(rank_of(e));
        fill_slot.push_back(slot);
        fill_victim.push_back(victim);
    }

    ctx->stats.steps += 1;
    ctx->stats.distinct += n;
    ctx->stats.hits += int64_t(hit.size());
    ctx->stats.misses += m;
    ctx->stats.fills += q;
    ctx->stats.host += m - q;
    ctx->stats.evictions += evictions;

    if (plan) {
        plan->layer = layer;
        plan->n_distinct = n;
        plan->n_hit = int32_t(hit.size());
        plan->n_miss = m;
        plan->n_fill = q;
        plan->n_host = m - q;
        auto put = [](int32_t* dst, const int32_t* src, size_t cnt) { if (dst && cnt) std::memcpy(dst, src, cnt * 4); };
        put(plan->distinct, S.data(), S.size());
        put(plan->hit, hit.data(), hit.size());
        put(plan->hit_slot, hit_slot.data(), hit_slot.size());
        put(plan->fill, miss.data(), size_t(q));
        put(plan->fill_slot, fill_slot.data(), fill_slot.size());
        put(plan->fill_victim, fill_victim.data(), fill_victim.size());
        put(plan->host, miss.data() + q, size_t(m - q));
        if (plan->slot_of_expert)
            for (int e = 0; e < E; ++e) plan->slot_of_expert[e] = ctx->slot_of_key[kbase + e];
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_lru_step(moe_ctx* ctx, int32_t layer, const int32_t* h_topk_ids, int32_t T, moe_plan* plan) {
    if (!ctx) return MOE_EINVAL;
    if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, MOE_EINVAL, "layer out of range");
    if (T < 0 || (T > 0 && !h_topk_ids)) return fail(ctx, MOE_EINVAL, "bad ids");
    if (!step_ids_ok(ctx, h_topk_ids, T)) return fail(ctx, MOE_EINVAL, "expert id out of range or repeated within a token");
    return plan_step(ctx, layer, h_topk_ids, T, plan);
}

int moe_lru_replay(moe_ctx* ctx, int32_t layer, const int32_t* h_topk_ids, int32_t n_steps, int32_t T,
                   moe_plan* plans, moe_stats* stats) {
    if (!ctx) return MOE_EINVAL;
    if (layer < 0 || layer >= ctx->cfg.n_layers) return fail(ctx, MOE_EINVAL, "layer out of range");
    if (n_steps < 0 || T < 0 || (n_steps > 0 && T > 0 && !h_topk_ids)) return fail(ctx, MOE_EINVAL, "bad ids");
    const int64_t per = int64_t(T) * ctx->cfg.top_k;
    for (int32_t s = 0; s < n_steps; ++s)
        if (!step_ids_ok(ctx, h_topk_ids + s * per, T))
            return fail(ctx, MOE_EINVAL, "expert id out of range or repeated within a token");
    if (plans) {
        const int need = int(std::min<int64_t>(ctx->cfg.n_experts, per));
        for (int32_t s = 0; s < n_steps; ++s)
            if (plans[s].cap < need) return fail(ctx, MOE_ECAPACITY, "plan capacity below min(E, T*k)");
    }
    for (int32_t s = 0; s < n_steps; ++s) {
        int st = plan_step(ctx, layer, h_topk_ids + s * per, T, plans ? plans + s : nullptr);
        if (st != MOE_OK) return st;
    }
    if (stats) *stats = ctx->stats;
    return MOE_OK;
}

int moe_lru_reset(moe_ctx* ctx) {
    if (!ctx) return MOE_EINVAL;
    std::fill(ctx->key_of_slot.begin(), ctx->key_of_slot.end(), -1);
    std::fill(ctx->recency.begin(), ctx->recency.end(), 0);
    std::fill(ctx->slot_of_key.begin(), ctx->slot_of_key.end(), -1);
    std::fill(ctx->in_step.begin(), ctx->in_step.end(), 0);
    ctx->counter = 0;
    ctx->stats = moe_stats{};
    return MOE_OK;
}

int moe_lru_slots(const moe_ctx* ctx, int32_t layer, int32_t* h_slot_of_expert) {
    if (!ctx || !h_slot_of_expert) return MOE_EINVAL;
    if (layer < 0 || layer >= ctx->cfg.n_layers) return MOE_EINVAL;
    const int E = ctx->cfg.n_experts;
    std::memcpy(h_slot_of_expert, ctx->slot_of_key.data() + int64_t(layer) * E, size_t(E) * 4);
    return MOE_OK;
}

int moe_lru_resize(moe_ctx* ctx, int32_t new_slots, moe_resize* out) {
    if (!ctx || !out) return MOE_EINVAL;
    if (new_slots < 0 || new_slots > (1 << 21)) return fail(ctx, MOE_EINVAL, "new_slots out of range");
    const int C = ctx->cfg.n_slots;
    std::vector<int32_t> moves_src, moves_dst, evicted;
    std::vector<char> keep(size_t(C), 0);
    if (new_slots < C) {
        std::vector<int32_t> resident;
        for (int s = 0; s < C; ++s)
            if (ctx->key_of_slot[s] >= 0) resident.push_back(s);
        std::vector<int32_t> by_recency = resident;
        std::sort(by_recency.begin(), by_recency.end(),
                  [&](int32_t a, int32_t b) { return ctx->recency[a] > ctx->recency[b]; });
        const size_t n_keep = std::min(by_recency.size(), size_t(new_slots));
        for (size_t i = 0; i < n_keep; ++i) keep[by_recency[i]] = 1;
        for (int32_t s : resident)
            if (!keep[s]) evicted.push_back(ctx->key_of_slot[s]);
        int32_t next_free = 0;
        for (int s = new_slots; s < C; ++s) {
            if (!keep[s]) continue;
            while (keep[next_free]) ++next_free;   // a free slot below new_slots exists: kept <= new_slots
            moves_src.push_back(s);
            moves_dst.push_back(next_free);
            ++next_free;
        }
    }
    if (out->cap < int32_t(moves_src.size()) || out->cap < int32_t(evicted.size()))
        return fail(ctx, MOE_ECAPACITY, "resize arrays below the moves or evictions");
    if ((!moves_src.empty() && (!out->move_src || !out->move_dst)) || (!evicted.empty() && !out->evicted))
        return fail(ctx, MOE_EINVAL, "null resize array");

    // ---- mutate (all checks are done) ----
    if (new_slots < C) {
        for (int32_t key : evicted) {
            const int32_t s = ctx->slot_of_key[key];
            ctx->slot_of_key[key] = -1;
            ctx->key_of_slot[s] = -1;
            ctx->recency[s] = 0;
        }
        for (size_t i = 0; i < moves_src.size(); ++i) {
            const int32_t a = moves_src[i], b = moves_dst[i], key = ctx->key_of_slot[a];
            ctx->key_of_slot[b] = key;
            ctx->recency[b] = ctx->recency[a];
            ctx->slot_of_key[key] = b;
            ctx->key_of_slot[a] = -1;
            ctx->recency[a] = 0;
        }
    }
    ctx->key_of_slot.resize(size_t(new_slots), -1);
    ctx->recency.resize(size_t(new_slots), 0);
    ctx->cfg.n_slots = new_slots;   // the bound device pool stays bound (moves run in it) until rebound
    out->n_move = int32_t(moves_src.size());
    out->n_evict = int32_t(evicted.size());
    if (!moves_src.empty()) {
        std::memcpy(out->move_src, moves_src.data(), moves_src.size() * 4);
        std::memcpy(out->move_dst, moves_dst.data(), moves_dst.size() * 4);
    }
    if (!evicted.empty()) std::memcpy(out->evicted, evicted.data(), evicted.size() * 4);
    return MOE_OK;
}

int moe_lru_stats(const moe_ctx* ctx, moe_stats* stats) {
    if (!ctx || !stats) return MOE_EINVAL;
    *stats = ctx->stats;
    return MOE_OK;
}

}  // extern "C"

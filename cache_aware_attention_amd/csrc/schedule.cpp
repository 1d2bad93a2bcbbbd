// schedule.cpp -- host-side step planning for KV-cached MAR decoding.
//
// "MARche" paper-notes page, flowchart and Key Design 3: a periodic full
// refresh runs when step % 3 == 0 (the initial step included), recomputing
// every layer and rewriting the caches; on the other steps layers 1-2 run full
// attention, layer 2 selects the refreshing tokens (Key Design 1) and the
// deeper layers run cache-aware attention over the active set, whose size is a
// fixed budget shared by generating, previous and refreshing tokens.
// "LazyMAR" paper-notes page: warm-up steps run in full; the token gate
// applies past the first three layers; fully computed steps re-store the
// condition-cache residual.
#include "mar_cache_attn.h"

extern "C" int mar_plan_step(const int32_t* counts, int n_steps, int step, int n_tokens,
                             int budget, int period, int warmup, mar_step_plan* out) {
    if (counts == nullptr || out == nullptr) return MAR_E_NULL;
    if (n_steps < 1 || n_tokens < 1 || period < 1) return MAR_E_SHAPE;
    if (step < 0 || step >= n_steps || budget < 0 || warmup < 0) return MAR_E_RANGE;
    long long begin = 0;
    for (int s = 0; s < step; ++s) {
        if (counts[s] < 0) return MAR_E_RANGE;
        begin += counts[s];
    }
    if (counts[step] < 0) return MAR_E_RANGE;
    const int n_gen = counts[step];
    const int n_prev = step > 0 ? counts[step - 1] : 0;
    if (begin + n_gen > n_tokens) return MAR_E_RANGE;
    mar_step_plan p;
    p.step = step;
    p.gen_begin = static_cast<int32_t>(begin);
    p.n_gen = n_gen;
    p.prev_begin = static_cast<int32_t>(begin - n_prev);
    p.n_prev = n_prev;
    p.refresh = (step < warmup || step % period == 0) ? 1 : 0;
    if (p.refresh) {
        p.n_refresh = 0;
        p.n_active = n_tokens;
        p.n_cached = 0;
    } else {
        int k = budget - n_gen - n_prev;
        if (k < 0) k = 0;
        const int room = n_tokens - n_gen - n_prev;
        if (k > room) k = room;
        p.n_refresh = k;
        p.n_active = n_gen + n_prev + k;
        p.n_cached = n_tokens - p.n_active;
    }
    *out = p;
    return MAR_OK;
}

extern "C" int mar_layer_flags(const mar_step_plan* plan, int layer, int n_full_layers,
                               int select_layer, int ungated_layers) {
    if (plan == nullptr) return MAR_E_NULL;
    if (layer < 1 || n_full_layers < 0 || ungated_layers < 0) return MAR_E_RANGE;
    if (plan->refresh) return 0;
    int flags = 0;
    if (layer > n_full_layers) flags |= MAR_LAYER_CACHE;
    if (layer == select_layer) flags |= MAR_LAYER_SELECT;
    if (layer > ungated_layers) flags |= MAR_LAYER_GATE;
    return flags;
}

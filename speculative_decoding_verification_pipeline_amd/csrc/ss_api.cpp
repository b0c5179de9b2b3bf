// Host side of the C ABI: handle lifetime, workspace, argument validation and
// kernel launches. Nothing here allocates or synchronises after create.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>

#include "ss_device.h"
#include "ss_internal.h"

struct ss_sampler {
    ss_sampler_config cfg;
    int n_tiles;       // 8192-entry tiles per row
    int n_wt;          // wave tiles per row (WPT per 8192-entry tile)
    int n_vtiles;      // 128-row LM-head vocabulary tiles
    int max_rows;      // rows of the row kernels (verification: B * (G + 1))
    void* ws_base;
    int64_t ws_bytes;
    ss::Workspace ws;
    float2* lm_partials;
    ss::LaunchEvents events;
    // defaults substituted for absent per-request parameters, [max_batch] each
    int32_t* def_zero_i;
    float* def_zero_f;
    float* def_one_f;
    int32_t* def_iota;
};

namespace {

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device pointers for every per-request parameter: an absent one points at the
// handle's default array (so the kernels read every parameter unconditionally).
ss::ParamPtrs to_ptrs(const ss_sampler* s, const ss_params* p) {
    ss::ParamPtrs q;
    q.temperature = p->temperature;
    q.top_k = p->top_k ? p->top_k : s->def_zero_i;
    q.top_p = p->top_p ? p->top_p : s->def_one_f;
    q.min_p = p->min_p ? p->min_p : s->def_zero_f;
    q.rep = p->repetition_penalty ? p->repetition_penalty : s->def_one_f;
    q.freq = p->frequency_penalty ? p->frequency_penalty : s->def_zero_f;
    q.pres = p->presence_penalty ? p->presence_penalty : s->def_zero_f;
    const bool hist = p->history_len && p->history_ids;
    q.hist_ids = hist ? p->history_ids : s->def_zero_i;
    q.hist_len = hist ? p->history_len : s->def_zero_i;
    q.hist_stride = hist ? p->history_stride : 0;
    const bool bias = p->bias_len && p->bias_ids && p->bias_values;
    q.bias_ids = bias ? p->bias_ids : s->def_zero_i;
    q.bias_vals = bias ? p->bias_values : s->def_zero_f;
    q.bias_len = bias ? p->bias_len : s->def_zero_i;
    q.bias_stride = bias ? p->bias_stride : 0;
    q.mask = p->grammar_mask;
    q.mask_stride = p->mask_stride;
    q.request_ids = p->request_ids ? p->request_ids : s->def_iota;
    q.positions = p->positions ? p->positions : s->def_zero_i;
    q.seed = p->seed;
    return q;
}

ss_status check_params(const ss_sampler* s, const ss_params* p) {
    if (!p || !p->temperature) return SS_ERR_INVALID_ARG;
    const int V = s->cfg.vocab_size;
    if (p->history_len) {
        if (!p->history_ids || p->history_stride < 0 || p->history_stride > 65000)
            return SS_ERR_INVALID_ARG;
    }
    if (p->bias_len) {
        if (!p->bias_ids || !p->bias_values || p->bias_stride < 0) return SS_ERR_INVALID_ARG;
    }
    if (p->grammar_mask) {
        if (p->mask_stride < (V + 31) / 32) return SS_ERR_INVALID_ARG;
    }
    return SS_OK;
}

ss_status check_logits(const ss_sampler* s, const void* logits, ss_dtype dtype, int64_t row_stride) {
    if (!logits) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_INVALID_ARG;
    if (row_stride < s->cfg.vocab_size) return SS_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(logits) & (dtype == SS_F32 ? 3u : 1u)) != 0)
        return SS_ERR_INVALID_ARG;  // not even element-aligned
    return SS_OK;
}

}  // namespace

extern "C" {

const char* ss_status_string(ss_status st) {
    switch (st) {
        case SS_OK: return "ok";
        case SS_ERR_INVALID_ARG: return "invalid argument";
        case SS_ERR_UNSUPPORTED: return "unsupported argument";
        case SS_ERR_OUT_OF_MEMORY: return "out of device memory";
        case SS_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

ss_status ss_sampler_create(const ss_sampler_config* cfg, ss_sampler** out) {
    if (!cfg || !out) return SS_ERR_INVALID_ARG;
    *out = nullptr;
    if (cfg->max_batch < 1 || cfg->vocab_size < 1 || cfg->vocab_size > ss::MAX_VOCAB ||
        cfg->max_draft < 0 || cfg->max_draft > 16 || cfg->hidden_size < 0 ||
        cfg->hidden_size % 64 != 0 || cfg->device < 0)
        return SS_ERR_INVALID_ARG;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) return SS_ERR_HIP;
    if (hipSetDevice(cfg->device) != hipSuccess) return SS_ERR_HIP;

    ss_sampler* s = new (std::nothrow) ss_sampler();
    if (!s) return SS_ERR_OUT_OF_MEMORY;
    s->cfg = *cfg;
    const int V = cfg->vocab_size;
    const int B = cfg->max_batch;
    s->n_tiles = (V + ss::TILE - 1) / ss::TILE;
    s->n_wt = s->n_tiles * ss::WPT;  // a wave's entries interleave across its whole tile
    s->n_vtiles = (V + 127) / 128;
    s->max_rows = B * (cfg->max_draft + 1);
    const int64_t R = s->max_rows;
    const int64_t nt = s->n_tiles;

    // carve one allocation; nothing in it needs clearing between calls
    int64_t off = 0;
    auto take = [&off](int64_t bytes) {
        const int64_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const int64_t nw = s->n_wt;
    const int64_t o_stats = take(R * nw * (int64_t)sizeof(ss::WaveStat));
    const int64_t o_cand = take(R * nw * ss::WCAP * (int64_t)sizeof(unsigned long long));
    const int64_t o_info = take(R * (int64_t)sizeof(ss::RowInfo));
    const int64_t o_acc = take(R * 4);
    const int64_t o_restile = take((int64_t)B * nt * (int64_t)sizeof(double2));
    const int64_t o_scratch = take(R * (int64_t)V * 4);
    const int64_t o_lmpart = cfg->hidden_size > 0 ? take(64 * (int64_t)s->n_vtiles * sizeof(float2)) : 0;
    const int64_t o_defaults = take(4 * (int64_t)B * 4);
    s->ws_bytes = off;
    if (hipMalloc(&s->ws_base, (size_t)off) != hipSuccess) {
        (void)hipGetLastError();
        delete s;
        return SS_ERR_OUT_OF_MEMORY;
    }
    char* b = static_cast<char*>(s->ws_base);
    ss::Workspace& w = s->ws;
    w.wstats = reinterpret_cast<ss::WaveStat*>(b + o_stats);
    w.cand = reinterpret_cast<unsigned long long*>(b + o_cand);
    w.rowinfo = reinterpret_cast<ss::RowInfo*>(b + o_info);
    w.row_accept = reinterpret_cast<int32_t*>(b + o_acc);
    w.resid_tile = reinterpret_cast<double2*>(b + o_restile);
    w.scratch_z = reinterpret_cast<float*>(b + o_scratch);
    w.n_tiles = s->n_tiles;
    w.n_wt = s->n_wt;
    w.V = V;
    s->lm_partials = cfg->hidden_size > 0 ? reinterpret_cast<float2*>(b + o_lmpart) : nullptr;
    {
        int32_t* d = reinterpret_cast<int32_t*>(b + o_defaults);
        s->def_zero_i = d;
        s->def_zero_f = reinterpret_cast<float*>(d + B);
        s->def_one_f = reinterpret_cast<float*>(d + 2 * B);
        s->def_iota = d + 3 * B;
        int32_t* h = new (std::nothrow) int32_t[4 * (size_t)B];
        if (!h) {
            (void)hipFree(s->ws_base);
            delete s;
            return SS_ERR_OUT_OF_MEMORY;
        }
        for (int i = 0; i < B; ++i) {
            const float one = 1.0f;
            h[i] = 0;
            h[B + i] = 0;  // +0.0f
            std::memcpy(&h[2 * B + i], &one, 4);
            h[3 * B + i] = i;
        }
        const bool ok = hipMemcpy(d, h, 4 * (size_t)B * 4, hipMemcpyHostToDevice) == hipSuccess;
        delete[] h;
        if (!ok) {
            (void)hipFree(s->ws_base);
            delete s;
            return SS_ERR_HIP;
        }
    }
    *out = s;
    return SS_OK;
}

void ss_sampler_destroy(ss_sampler* s) {
    if (!s) return;
    (void)hipSetDevice(s->cfg.device);
    (void)hipFree(s->ws_base);
    delete s;
}

int64_t ss_sampler_workspace_bytes(const ss_sampler* s) { return s ? s->ws_bytes : 0; }

ss_status ss_sampler_set_launch_events(ss_sampler* s, void* const* events, int32_t n_events) {
    if (!s || n_events < 0 || n_events > 8) return SS_ERR_INVALID_ARG;
    s->events.n = events ? n_events : 0;
    for (int k = 0; k < 8; ++k)
        s->events.ev[k] = (events && k < n_events) ? static_cast<hipEvent_t>(events[k]) : nullptr;
    return SS_OK;
}

ss_status ss_sample(ss_sampler* s, const void* logits, ss_dtype dtype, int64_t row_stride,
                    int32_t B, const ss_params* params, int32_t* out_tokens, const ss_debug* debug,
                    void* stream) {
    if (!s || B < 0 || B > s->cfg.max_batch) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!out_tokens) return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(s, logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(s, params);
    if (st != SS_OK) return st;
    if (debug && debug->topk_ids && debug->topk_stride < 1) return SS_ERR_INVALID_ARG;
    ss::SampleArgs a;
    std::memset(&a, 0, sizeof(a));
    a.logits = logits;
    a.row_stride = row_stride;
    a.B = B;
    a.V = s->cfg.vocab_size;
    a.p = to_ptrs(s, params);
    a.out_tokens = out_tokens;
    if (debug) {
        a.dbg_processed = debug->processed_logits;
        a.dbg_topk = debug->topk_ids;
        a.dbg_topk_stride = debug->topk_ids ? debug->topk_stride : 0;
        a.dbg_kept = debug->kept_count;
        a.dbg_probs = debug->probs;
        a.dbg_path = debug->path;
    }
    a.ws = s->ws;
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_sample(a, dtype, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                       : SS_ERR_HIP;
}

ss_status ss_spec_verify(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                         int64_t row_stride, const float* draft_probs, int64_t draft_stride,
                         const int32_t* draft_tokens, int32_t B, int32_t G,
                         const ss_params* params, int32_t* out_tokens,
                         int32_t* out_num_accepted, void* stream) {
    if (!s || B < 0 || B > s->cfg.max_batch) return SS_ERR_INVALID_ARG;
    if (G < 1 || G > s->cfg.max_draft) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!draft_probs || !draft_tokens || !out_tokens || !out_num_accepted) return SS_ERR_INVALID_ARG;
    if (draft_stride < s->cfg.vocab_size) return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(s, target_logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(s, params);
    if (st != SS_OK) return st;
    ss::SpecArgs a;
    std::memset(&a, 0, sizeof(a));
    a.target = target_logits;
    a.row_stride = row_stride;
    a.draft_probs = draft_probs;
    a.draft_stride = draft_stride;
    a.draft_tokens = draft_tokens;
    a.B = B;
    a.G = G;
    a.V = s->cfg.vocab_size;
    a.p = to_ptrs(s, params);
    a.out_tokens = out_tokens;
    a.out_num_accepted = out_num_accepted;
    a.ws = s->ws;
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_spec(a, dtype, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                     : SS_ERR_HIP;
}

ss_status ss_lmhead_sample(ss_sampler* s, const uint16_t* hidden, const uint16_t* weight,
                           int32_t B, const float* temperature, const int32_t* request_ids,
                           const int32_t* positions, uint64_t seed, int32_t* out_tokens,
                           float* debug_logits, void* stream) {
    if (!s || s->cfg.hidden_size <= 0) return SS_ERR_INVALID_ARG;
    if (B < 1 || B > s->cfg.max_batch || B > 64) return SS_ERR_INVALID_ARG;
    if (!hidden || !weight || !temperature || !out_tokens) return SS_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(weight)) return SS_ERR_UNSUPPORTED;
    ss::LmheadArgs a;
    std::memset(&a, 0, sizeof(a));
    a.hidden = hidden;
    a.weight = weight;
    a.B = B;
    a.K = s->cfg.hidden_size;
    a.V = s->cfg.vocab_size;
    a.temperature = temperature;
    a.request_ids = request_ids;
    a.positions = positions;
    a.seed = seed;
    a.out_tokens = out_tokens;
    a.debug_logits = debug_logits;
    a.partials = s->lm_partials;
    a.n_vtiles = s->n_vtiles;
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_lmhead(a, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                : SS_ERR_HIP;
}

}  // extern "C"

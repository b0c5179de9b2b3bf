// Host side of the C ABI: handle lifetime, workspace, argument validation and
// kernel launches. Nothing here allocates or synchronises after create; the
// handle-free ss_sample_noalloc never allocates at all (its scratch is a static
// device array of this file).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>
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
    ss::LmTileStat* lm_stats;
    int32_t* lm_unres;
    ss::LmCut* lm_cut;
    ss::LaunchEvents events;
    // defaults substituted for absent per-request parameters, [max_batch] each
    int32_t* def_zero_i;
    float* def_zero_f;
    float* def_one_f;
    int32_t* def_iota;
};

namespace {

// Device arrays read in place of absent per-request parameters.
struct Defaults {
    const int32_t* zero_i;
    const float* zero_f;
    const float* one_f;
    const int32_t* iota;
};

Defaults defaults_of(const ss_sampler* s) {
    return {s->def_zero_i, s->def_zero_f, s->def_one_f, s->def_iota};
}

}  // namespace

namespace {

constexpr int64_t kAlign = 256;

constexpr int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device pointers for every per-request parameter: an absent one points at the
// handle's default array (so the kernels read every parameter unconditionally).
ss::ParamPtrs to_ptrs(const Defaults& d, const ss_params* p) {
    ss::ParamPtrs q;
    q.temperature = p->temperature;
    q.top_k = p->top_k ? p->top_k : d.zero_i;
    q.top_p = p->top_p ? p->top_p : d.one_f;
    q.min_p = p->min_p ? p->min_p : d.zero_f;
    q.rep = p->repetition_penalty ? p->repetition_penalty : d.one_f;
    q.freq = p->frequency_penalty ? p->frequency_penalty : d.zero_f;
    q.pres = p->presence_penalty ? p->presence_penalty : d.zero_f;
    const bool hist = p->history_len && p->history_ids;
    q.hist_ids = hist ? p->history_ids : d.zero_i;
    q.hist_len = hist ? p->history_len : d.zero_i;
    q.hist_stride = hist ? p->history_stride : 0;
    const bool bias = p->bias_len && p->bias_ids && p->bias_values;
    q.bias_ids = bias ? p->bias_ids : d.zero_i;
    q.bias_vals = bias ? p->bias_values : d.zero_f;
    q.bias_len = bias ? p->bias_len : d.zero_i;
    q.bias_stride = bias ? p->bias_stride : 0;
    q.mask = p->grammar_mask;
    q.mask_stride = p->mask_stride;
    q.request_ids = p->request_ids ? p->request_ids : d.iota;
    q.positions = p->positions ? p->positions : d.zero_i;
    q.seed = p->seed;
    return q;
}

ss_status check_params(int V, const ss_params* p) {
    if (!p || !p->temperature) return SS_ERR_INVALID_ARG;
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

ss_status check_logits(int V, const void* logits, ss_dtype dtype, int64_t row_stride) {
    if (!logits) return SS_ERR_INVALID_ARG;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_INVALID_ARG;
    if (row_stride < V) return SS_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(logits) & (dtype == SS_F32 ? 3u : 1u)) != 0)
        return SS_ERR_INVALID_ARG;  // not even element-aligned
    return SS_OK;
}

// ---------------------------------------------------------------------------
// ss_sample_noalloc: the same kernels as ss_sample, with the workspace carved
// from a static device array instead of a handle's allocation.

// Per-row workspace of a sampling call over B rows of V entries (the buffers a
// handle gives ss_sample, sized for exactly B rows); with base set, points w at
// them. Returns the bytes used.
constexpr int64_t sample_scratch_layout(int64_t B, int64_t V, char* base, ss::Workspace* w) {
    const int64_t n_tiles = (V + ss::TILE - 1) / ss::TILE;
    const int64_t n_wt = n_tiles * ss::WPT;
    int64_t off = 0;
    const int64_t o_stats = off;
    off = align_up(off + B * n_wt * (int64_t)sizeof(ss::WaveStat));
    const int64_t o_cand = off;
    off = align_up(off + B * n_wt * ss::WCAP * (int64_t)sizeof(unsigned long long));
    const int64_t o_info = off;
    off = align_up(off + B * (int64_t)sizeof(ss::RowInfo));
    const int64_t o_z = off;
    off = align_up(off + B * V * 4);
    if (base && w) {
        w->wstats = reinterpret_cast<ss::WaveStat*>(base + o_stats);
        w->cand = reinterpret_cast<unsigned long long*>(base + o_cand);
        w->rowinfo = reinterpret_cast<ss::RowInfo*>(base + o_info);
        w->row_accept = nullptr;  // verification only
        w->resid_tile = nullptr;
        w->scratch_z = reinterpret_cast<float*>(base + o_z);
        w->bins = nullptr;  // no binned tails: such rows take the whole-row path
        w->n_tiles = (int)n_tiles;
        w->n_wt = (int)n_wt;
        w->V = (int)V;
    }
    return off;
}

// The layout grows with V for a fixed B, so its largest size under the limits
// is at the largest V each B allows.
constexpr int64_t largest_sample_scratch() {
    int64_t m = 0;
    for (int64_t b = 1; b <= SS_NOALLOC_MAX_BATCH; ++b) {
        int64_t v = SS_NOALLOC_MAX_ENTRIES / b;
        if (v > ss::MAX_VOCAB) v = ss::MAX_VOCAB;
        const int64_t n = sample_scratch_layout(b, v, nullptr, nullptr);
        if (n > m) m = n;
    }
    return m;
}
static_assert(largest_sample_scratch() <= SS_NOALLOC_SCRATCH_BYTES,
              "the static scratch must hold the largest call the limits admit");

// Values read in place of absent per-request parameters (one row each).
struct DefaultTable {
    int32_t zero_i[SS_NOALLOC_MAX_BATCH];
    float zero_f[SS_NOALLOC_MAX_BATCH];
    float one_f[SS_NOALLOC_MAX_BATCH];
    int32_t iota[SS_NOALLOC_MAX_BATCH];
};

constexpr DefaultTable make_default_table() {
    DefaultTable t{};
    for (int i = 0; i < SS_NOALLOC_MAX_BATCH; ++i) {
        t.zero_i[i] = 0;
        t.zero_f[i] = 0.0f;
        t.one_f[i] = 1.0f;
        t.iota[i] = i;
    }
    return t;
}

}  // namespace

// One copy of each per GPU, reserved with the library's code object. Host code
// never passes these names to a kernel: it uses the device addresses that
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_SCRATCH_BYTES];
static __device__ __align__(256) DefaultTable noalloc_defaults = make_default_table();

namespace {

constexpr int kMaxDevices = 64;

struct NoAllocDevice {
    std::atomic<char*> scratch;
    std::atomic<const DefaultTable*> defaults;
};
NoAllocDevice g_noalloc[kMaxDevices];  // static storage: starts null
std::mutex g_noalloc_mutex;

// This GPU's addresses of the two arrays, looked up once per device with that
// device current (the first call on a device; later calls read the cache).
ss_status noalloc_arrays(int dev, char** scr, const DefaultTable** defs) {
    char* p = g_noalloc[dev].scratch.load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_noalloc_mutex);
        p = g_noalloc[dev].scratch.load(std::memory_order_relaxed);
        if (!p) {
            void* sp = nullptr;
            void* dp = nullptr;
            if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) != hipSuccess || !sp ||
                hipGetSymbolAddress(&dp, HIP_SYMBOL(noalloc_defaults)) != hipSuccess || !dp) {
                (void)hipGetLastError();
                return SS_ERR_HIP;
            }
            g_noalloc[dev].defaults.store(static_cast<const DefaultTable*>(dp),
                                          std::memory_order_relaxed);
            p = static_cast<char*>(sp);
            g_noalloc[dev].scratch.store(p, std::memory_order_release);
        }
    }
    *scr = p;
    *defs = g_noalloc[dev].defaults.load(std::memory_order_relaxed);
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
        cfg->max_draft < 0 || cfg->max_draft > 63 || cfg->hidden_size < 0 ||
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
    const int64_t o_bins = take((int64_t)B * nw * ss::NBIN * 4);
    const int64_t dmax = cfg->max_draft > 0 ? cfg->max_draft : 1;
    const int64_t o_tpath = take(R * dmax * 4);
    const int64_t o_tdepth = take(R * 4);
    const int64_t o_tnext = take(R * 4);
    const int64_t o_lmpart = cfg->hidden_size > 0 ? take(64 * (int64_t)s->n_vtiles * sizeof(float2)) : 0;
    const int64_t o_lmstat =
        cfg->hidden_size > 0 ? take(64 * (int64_t)s->n_vtiles * (int64_t)sizeof(ss::LmTileStat)) : 0;
    const int64_t o_lmunres = cfg->hidden_size > 0 ? take(64 * 4) : 0;
    const int64_t o_lmcut = cfg->hidden_size > 0 ? take(64 * (int64_t)sizeof(ss::LmCut)) : 0;
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
    w.bins = reinterpret_cast<float*>(b + o_bins);
    w.tree_path = reinterpret_cast<int32_t*>(b + o_tpath);
    w.tree_depth = reinterpret_cast<int32_t*>(b + o_tdepth);
    w.tree_next = reinterpret_cast<int32_t*>(b + o_tnext);
    w.tree_dmax = (int)dmax;
    w.n_tiles = s->n_tiles;
    w.n_wt = s->n_wt;
    w.V = V;
    s->lm_partials = cfg->hidden_size > 0 ? reinterpret_cast<float2*>(b + o_lmpart) : nullptr;
    s->lm_stats = cfg->hidden_size > 0 ? reinterpret_cast<ss::LmTileStat*>(b + o_lmstat) : nullptr;
    s->lm_unres = cfg->hidden_size > 0 ? reinterpret_cast<int32_t*>(b + o_lmunres) : nullptr;
    s->lm_cut = cfg->hidden_size > 0 ? reinterpret_cast<ss::LmCut*>(b + o_lmcut) : nullptr;
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
    if (!s || n_events < 0 || n_events > 16) return SS_ERR_INVALID_ARG;
    s->events.n = events ? n_events : 0;
    for (int k = 0; k < 16; ++k)
        s->events.ev[k] = (events && k < n_events) ? static_cast<hipEvent_t>(events[k]) : nullptr;
    return SS_OK;
}

ss_status ss_sample(ss_sampler* s, const void* logits, ss_dtype dtype, int64_t row_stride,
                    int32_t B, const ss_params* params, int32_t* out_tokens, const ss_debug* debug,
                    void* stream) {
    if (!s || B < 0 || B > s->cfg.max_batch) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!out_tokens) return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(s->cfg.vocab_size, logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(s->cfg.vocab_size, params);
    if (st != SS_OK) return st;
    if (debug && debug->topk_ids && debug->topk_stride < 1) return SS_ERR_INVALID_ARG;
    ss::SampleArgs a;
    std::memset(&a, 0, sizeof(a));
    a.logits = logits;
    a.row_stride = row_stride;
    a.B = B;
    a.V = s->cfg.vocab_size;
    a.p = to_ptrs(defaults_of(s), params);
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
    // Binned tails serve unfiltered rows without penalty or bias lists: a batch
    // that carries such lists takes the kernels without them (their code alone
    // slows the merge a little).
    if (params && (params->history_ids || params->bias_ids)) a.ws.bins = nullptr;
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_sample(a, dtype, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                       : SS_ERR_HIP;
}

ss_status ss_spec_verify(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                         int64_t row_stride, const float* draft_probs, int64_t draft_stride,
                         const int32_t* draft_tokens, int32_t B, int32_t G,
                         const ss_params* params, int32_t* out_tokens,
                         int32_t* out_num_accepted, void* stream) {
    return ss_spec_verify_scatter(s, target_logits, dtype, row_stride, draft_probs, draft_stride,
                                  draft_tokens, B, G, params, out_tokens, out_num_accepted,
                                  nullptr, stream);
}

ss_status ss_spec_verify_scatter(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                                 int64_t row_stride, const float* draft_probs,
                                 int64_t draft_stride, const int32_t* draft_tokens, int32_t B,
                                 int32_t G, const ss_params* params, int32_t* out_tokens,
                                 int32_t* out_num_accepted, const ss_sequences* seq,
                                 void* stream) {
    if (!s || B < 0 || B > s->cfg.max_batch) return SS_ERR_INVALID_ARG;
    if (G < 1 || G > s->cfg.max_draft) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!draft_tokens || !out_tokens || !out_num_accepted) return SS_ERR_INVALID_ARG;
    if (draft_probs && draft_stride < s->cfg.vocab_size) return SS_ERR_INVALID_ARG;
    if (seq && (!seq->tokens || !seq->len || seq->capacity < 0 || seq->stride < seq->capacity))
        return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(s->cfg.vocab_size, target_logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(s->cfg.vocab_size, params);
    if (st != SS_OK) return st;
    ss::SpecArgs a;
    std::memset(&a, 0, sizeof(a));
    a.target = target_logits;
    a.row_stride = row_stride;
    a.draft_probs = draft_probs;
    a.draft_stride = draft_probs ? draft_stride : 0;
    a.draft_tokens = draft_tokens;
    a.B = B;
    a.G = G;
    a.V = s->cfg.vocab_size;
    a.p = to_ptrs(defaults_of(s), params);
    a.out_tokens = out_tokens;
    a.out_num_accepted = out_num_accepted;
    if (seq) {
        a.seq_tokens = seq->tokens;
        a.seq_stride = seq->stride;
        a.seq_capacity = seq->capacity;
        a.seq_len = seq->len;
    }
    a.ws = s->ws;
    a.ws.bins = nullptr;  // verification rows draw from their candidates or the whole row
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_spec(a, dtype, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                     : SS_ERR_HIP;
}

ss_status ss_tree_verify(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                         int64_t row_stride, const int32_t* parents, const int32_t* tokens,
                         int32_t B, int32_t N, const ss_params* params, int32_t* out_tokens,
                         int32_t* out_nodes, int32_t* out_num_accepted, void* stream) {
    if (!s || B < 0 || B > s->cfg.max_batch) return SS_ERR_INVALID_ARG;
    if (N < 2 || N > s->cfg.max_draft + 1) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!parents || !tokens || !out_tokens || !out_nodes || !out_num_accepted)
        return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(s->cfg.vocab_size, target_logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(s->cfg.vocab_size, params);
    if (st != SS_OK) return st;
    ss::TreeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.target = target_logits;
    a.row_stride = row_stride;
    a.parents = parents;
    a.tokens = tokens;
    a.B = B;
    a.N = N;
    a.V = s->cfg.vocab_size;
    a.p = to_ptrs(defaults_of(s), params);
    a.out_tokens = out_tokens;
    a.out_nodes = out_nodes;
    a.out_num_accepted = out_num_accepted;
    a.ws = s->ws;
    a.ws.bins = nullptr;  // verification rows draw from their candidates or the whole row
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_tree(a, dtype, static_cast<hipStream_t>(stream), s->events) == hipSuccess ? SS_OK
                                                                                     : SS_ERR_HIP;
}

ss_status ss_lmhead_sample_params(ss_sampler* s, const uint16_t* hidden, const uint16_t* weight,
                                  int32_t B, const ss_params* params, int32_t* out_tokens,
                                  int32_t* debug_path, void* stream) {
    if (!s || s->cfg.hidden_size <= 0) return SS_ERR_INVALID_ARG;
    if (B < 1 || B > s->cfg.max_batch || B > 64) return SS_ERR_INVALID_ARG;
    if (!hidden || !weight || !out_tokens) return SS_ERR_INVALID_ARG;
    if (!aligned16(hidden) || !aligned16(weight)) return SS_ERR_UNSUPPORTED;
    const ss_status st = check_params(s->cfg.vocab_size, params);
    if (st != SS_OK) return st;
    ss::LmheadArgs a;
    std::memset(&a, 0, sizeof(a));
    a.hidden = hidden;
    a.weight = weight;
    a.B = B;
    a.K = s->cfg.hidden_size;
    a.V = s->cfg.vocab_size;
    a.temperature = params->temperature;
    a.seed = params->seed;
    a.out_tokens = out_tokens;
    a.partials = s->lm_partials;
    a.n_vtiles = s->n_vtiles;
    a.p = to_ptrs(defaults_of(s), params);
    a.stats = s->lm_stats;
    a.unres = s->lm_unres;
    a.cut = s->lm_cut;
    a.zmat = s->ws.scratch_z;
    a.dbg_path = debug_path;
    if (hipSetDevice(s->cfg.device) != hipSuccess) return SS_ERR_HIP;
    return ss::launch_lmhead_params(a, static_cast<hipStream_t>(stream), s->events) == hipSuccess
               ? SS_OK
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

ss_status ss_sample_noalloc(const void* logits, ss_dtype dtype, int64_t row_stride, int32_t B,
                            int32_t V, const ss_params* params, int32_t* out_tokens,
                            void* stream) {
    if (B < 0 || V < 1 || V > ss::MAX_VOCAB) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (B > SS_NOALLOC_MAX_BATCH || (int64_t)B * V > SS_NOALLOC_MAX_ENTRIES) return SS_ERR_UNSUPPORTED;
    if (!out_tokens) return SS_ERR_INVALID_ARG;
    ss_status st = check_logits(V, logits, dtype, row_stride);
    if (st != SS_OK) return st;
    st = check_params(V, params);
    if (st != SS_OK) return st;
    if (sample_scratch_layout(B, V, nullptr, nullptr) > SS_NOALLOC_SCRATCH_BYTES)
        return SS_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SS_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SS_ERR_UNSUPPORTED;
    char* scr = nullptr;
    const DefaultTable* defs = nullptr;
    st = noalloc_arrays(dev, &scr, &defs);
    if (st != SS_OK) return st;
    ss::SampleArgs a;
    std::memset(&a, 0, sizeof(a));
    a.logits = logits;
    a.row_stride = row_stride;
    a.B = B;
    a.V = V;
    a.p = to_ptrs(Defaults{defs->zero_i, defs->zero_f, defs->one_f, defs->iota}, params);
    a.out_tokens = out_tokens;
    sample_scratch_layout(B, V, scr, &a.ws);
    ss::LaunchEvents none;
    std::memset(&none, 0, sizeof(none));
    return ss::launch_sample(a, dtype, static_cast<hipStream_t>(stream), none) == hipSuccess
               ? SS_OK
               : SS_ERR_HIP;
}

}  // extern "C"

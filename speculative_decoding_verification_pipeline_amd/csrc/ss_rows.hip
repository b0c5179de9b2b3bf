// Row kernels: the fused sampler and speculative verification (gfx950).
//
// The pipeline and its order follow the SonicSampler abstract (arxivdaily page,
// English abstract): per request, grammar mask, repetition / frequency /
// presence penalties, logit bias, temperature, then top-k, top-p and min-p, all
// in one batched launch, with a hierarchical two-stage top-k. Verification
// follows "Accelerating Sonar through speculation" (Perplexity blog, sections
// on speculative decoding and target-draft decoding).
//
// Design (MI355X-first, not a translation of the pages' Triton kernels):
//  * One workgroup (256 threads, 4 wave64s) per 8192-entry vocabulary tile of a
//    row; the grid is rows x tiles and depends only on (B, V), so one launch
//    serves any mix of per-request parameters and can be graph-captured.
//  * Stage 1 streams the tile once with 16-byte loads (float4 / 8 x bf16),
//    applies penalties (multiplicities counted in LDS), bias and the packed
//    mask in registers, and reduces: tile max, softmax partial sum, and a
//    candidate list -- every entry above a threshold taken from the sorted
//    per-thread maxima, so the list is always an exact prefix of the tile in
//    key order, capped at CW entries. Low-entropy rows leave only a handful of
//    entries near the top of each tile, which keeps the lists short.
//  * The last workgroup to finish a row (agent-scope release/acquire on a
//    per-row counter, reset for the next launch) merges the tiles: the union of
//    candidates above the highest tile threshold is an exact prefix of the
//    whole row; it is sorted in LDS and top-k / top-p / min-p and the
//    inverse-CDF draw are resolved on it with binary64 prefix sums. When a
//    request needs more of the row than the prefix holds, the same workgroup
//    runs an exact whole-row fallback (radix selection by count or by mass over
//    the row's recomputed z), so results never depend on the fast path's reach.
#include <float.h>
#include <limits.h>

#include "ss_device.h"
#include "ss_internal.h"

#pragma clang fp contract(off)

namespace ss {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr double MASS_SCALE = 17592186044416.0;  // 2^44 fixed-point weights in the fallback

struct RowCtx {
    const void* logits;
    int V;
    float T;
    int top_k;
    float top_p;
    float min_p;
    float rep, freq, pres;
    const int32_t* hist;
    int hist_len;
    const int32_t* extra;  // draft tokens that precede this row (verification)
    int extra_len;
    const int32_t* bias_ids;
    const float* bias_vals;
    int bias_len;
    const uint32_t* mask;  // this row's mask words or null
    uint32_t req, pos;
    uint64_t seed;
};

__device__ RowCtx make_ctx(const ParamPtrs& p, int b, const void* logits, int V,
                           const int32_t* extra, int extra_len, const uint32_t* mask_row,
                           uint32_t pos_offset) {
    RowCtx c;
    c.logits = logits;
    c.V = V;
    c.T = p.temperature[b];
    c.top_k = p.top_k ? p.top_k[b] : 0;
    c.top_p = p.top_p ? p.top_p[b] : 1.0f;
    c.min_p = p.min_p ? p.min_p[b] : 0.0f;
    c.rep = p.rep ? p.rep[b] : 1.0f;
    c.freq = p.freq ? p.freq[b] : 0.0f;
    c.pres = p.pres ? p.pres[b] : 0.0f;
    c.hist_len = p.hist_len ? p.hist_len[b] : 0;
    c.hist = p.hist_ids ? p.hist_ids + (int64_t)b * p.hist_stride : nullptr;
    if (!c.hist) c.hist_len = 0;
    c.extra = extra;
    c.extra_len = extra ? extra_len : 0;
    c.bias_len = p.bias_len ? p.bias_len[b] : 0;
    c.bias_ids = p.bias_ids ? p.bias_ids + (int64_t)b * p.bias_stride : nullptr;
    c.bias_vals = p.bias_vals ? p.bias_vals + (int64_t)b * p.bias_stride : nullptr;
    if (!c.bias_ids || !c.bias_vals) c.bias_len = 0;
    c.mask = mask_row;
    c.req = p.request_ids ? (uint32_t)p.request_ids[b] : (uint32_t)b;
    c.pos = (p.positions ? (uint32_t)p.positions[b] : 0u) + pos_offset;
    c.seed = p.seed;
    return c;
}

// ---------------------------------------------------------------------------
// LDS layouts (one union per workgroup; phases are separated by barriers)

struct SmemTile {
    uint32_t cnt[TILE / 2];   // u16 history multiplicities of the tile's entries
    uint32_t bias[TILE / 32]; // bit set: some bias entry targets this vocabulary entry
    float sorted[NT];         // sorted per-thread maxima
};

struct SmemPool {
    float z[POOL];
    int id[POOL];
    TileStat st[MAX_TILES];
};

struct SmemRadix {
    uint32_t hc[256];
    unsigned long long hm[256];
};

union SmemU {
    SmemTile t;
    SmemPool p;
    SmemRadix r;
};

struct SmemS {
    RedScratch red;
    int npool;
    int is_last;
    int sel;
    int take_last;
    unsigned long long rem;
    int flag;
};

// ---------------------------------------------------------------------------
// tile geometry: thread tid owns NG groups of VEC consecutive entries

template <int DT>
struct Lay {
    static constexpr int VEC = DT == SS_F32 ? 4 : 8;
    static constexpr int NG = EPT / VEC;
    static constexpr int GSTRIDE = NT * VEC;
};

template <int DT>
__device__ __forceinline__ int slot_id(int tb, int s) {
    using L = Lay<DT>;
    return tb + (s / L::VEC) * L::GSTRIDE + (int)threadIdx.x * L::VEC + (s % L::VEC);
}

template <int DT>
__device__ __forceinline__ float read_logit(const void* row, int id) {
    if (DT == SS_F32) return ((const float*)row)[id];
    const uint32_t b = ((const uint16_t*)row)[id];
    return __uint_as_float(b << 16);
}

template <int DT>
__device__ __forceinline__ void load_tile(const RowCtx& c, int tb, float v[EPT]) {
    using L = Lay<DT>;
    // 16-byte loads need a 16-byte aligned row; other rows take element loads
    const bool vec = ((uintptr_t)c.logits & 15u) == 0;
#pragma unroll
    for (int g = 0; g < L::NG; ++g) {
        const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
        if (DT == SS_F32) {
            const float* p = (const float*)c.logits + e0;
            if (vec && e0 + 4 <= c.V) {
                const float4 q = *(const float4*)p;
                v[g * 4 + 0] = q.x;
                v[g * 4 + 1] = q.y;
                v[g * 4 + 2] = q.z;
                v[g * 4 + 3] = q.w;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[g * 4 + j] = (e0 + j < c.V) ? p[j] : NEG_INF;
            }
        } else {
            const uint16_t* p = (const uint16_t*)c.logits + e0;
            if (vec && e0 + 8 <= c.V) {
                const uint4 q = *(const uint4*)p;
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[g * 8 + 2 * k] = __uint_as_float(w[k] << 16);
                    v[g * 8 + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[g * 8 + j] = (e0 + j < c.V) ? __uint_as_float((uint32_t)p[j] << 16) : NEG_INF;
            }
        }
    }
}

// Penalties -> bias -> mask for one entry. Shared by every path that forms x'
// so all of them produce the same binary32 value.
__device__ __forceinline__ float process_entry(const RowCtx& c, int id, float x, uint32_t count,
                                               bool bias_hit, bool allowed) {
    if (count) {
        x = (x > 0.0f) ? x / c.rep : x * c.rep;
        const float fc = c.freq * (float)count;
        x = x - fc;
        x = x - c.pres;
    }
    if (bias_hit) {
        for (int k = 0; k < c.bias_len; ++k)
            if (c.bias_ids[k] == id) x = x + c.bias_vals[k];
    }
    return allowed ? x : NEG_INF;
}

// Builds the tile's multiplicity counts and bias bitmap in LDS (two barriers).
__device__ __forceinline__ void build_tables(const RowCtx& c, int tb, SmemTile& t) {
    const int tid = threadIdx.x;
    const bool has_cnt = (c.hist_len + c.extra_len) > 0;
    if (has_cnt) {
        uint4* c4 = (uint4*)t.cnt;
#pragma unroll
        for (int k = 0; k < TILE / 8 / NT; ++k) c4[tid + k * NT] = make_uint4(0, 0, 0, 0);
    }
    if (c.bias_len > 0) t.bias[tid] = 0;
    __syncthreads();
    if (has_cnt) {
        for (int i = tid; i < c.hist_len + c.extra_len; i += NT) {
            const int id = i < c.hist_len ? c.hist[i] : c.extra[i - c.hist_len];
            const int l = id - tb;
            if (id >= 0 && id < c.V && l >= 0 && l < TILE)
                atomicAdd(&t.cnt[l >> 1], 1u << ((l & 1) * 16));
        }
    }
    for (int i = tid; i < c.bias_len; i += NT) {
        const int id = c.bias_ids[i];
        const int l = id - tb;
        if (id >= 0 && id < c.V && l >= 0 && l < TILE) atomicOr(&t.bias[l >> 5], 1u << (l & 31));
    }
    __syncthreads();
}

template <int DT>
__device__ __forceinline__ void process_tile(const RowCtx& c, int tb, float v[EPT], const SmemTile& t) {
    using L = Lay<DT>;
    const bool has_cnt = (c.hist_len + c.extra_len) > 0;
    const bool has_bias = c.bias_len > 0;
#pragma unroll
    for (int g = 0; g < L::NG; ++g) {
        const int l0 = g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
        const int e0 = tb + l0;
        uint32_t cw[L::VEC / 2];
        if (has_cnt) {
            if constexpr (L::VEC == 4) {
                const uint2 q = *(const uint2*)&t.cnt[l0 >> 1];
                cw[0] = q.x;
                cw[1] = q.y;
            } else {
                const uint4 q = *(const uint4*)&t.cnt[l0 >> 1];
                cw[0] = q.x;
                cw[1] = q.y;
                cw[2] = q.z;
                cw[3] = q.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < L::VEC / 2; ++k) cw[k] = 0;
        }
        const uint32_t bb = has_bias ? (t.bias[l0 >> 5] >> (l0 & 31)) : 0u;
        const uint32_t mw = (c.mask && e0 < c.V) ? (c.mask[e0 >> 5] >> (e0 & 31)) : 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < L::VEC; ++j) {
            const int id = e0 + j;
            if (id >= c.V) continue;
            const uint32_t cnt = (cw[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const bool hit = (bb >> j) & 1u;
            const bool allowed = (mw >> j) & 1u;
            float x = v[g * L::VEC + j];
            if (cnt | hit | !allowed) x = process_entry(c, id, x, cnt, hit, allowed);
            v[g * L::VEC + j] = x;
        }
    }
}

// x' for a single entry (used by acceptance tests). Whole workgroup participates.
template <int DT>
__device__ float single_entry(const RowCtx& c, int id, SmemS& sh) {
    int cnt = 0;
    for (int i = threadIdx.x; i < c.hist_len + c.extra_len; i += NT) {
        const int h = i < c.hist_len ? c.hist[i] : c.extra[i - c.hist_len];
        cnt += (h == id);
    }
    cnt = block_sum_i(cnt, sh.red);
    bool hit = false;
    for (int k = 0; k < c.bias_len; ++k) hit |= (c.bias_ids[k] == id);
    const bool allowed = c.mask ? ((c.mask[id >> 5] >> (id & 31)) & 1u) : true;
    const float x = read_logit<DT>(c.logits, id);
    return process_entry(c, id, x, (uint32_t)cnt, hit, allowed);
}

// ---------------------------------------------------------------------------
// stage 1: one tile of one row

template <int DT>
__device__ void tile_stage1(const RowCtx& c, int row, int tile, const Workspace& ws, SmemU& su,
                            SmemS& sh, float* dbg_proc_row, float* dbg_probs_row) {
    const int tid = threadIdx.x;
    const int tb = tile * TILE;
    float v[EPT];
    load_tile<DT>(c, tb, v);
    build_tables(c, tb, su.t);
    process_tile<DT>(c, tb, v, su.t);

    if (dbg_proc_row || dbg_probs_row) {
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int id = slot_id<DT>(tb, s);
            if (id < c.V) {
                if (dbg_proc_row) dbg_proc_row[id] = v[s];
                if (dbg_probs_row) dbg_probs_row[id] = 0.0f;
            }
        }
    }

    float lm = NEG_INF;
    int nf = 0;
#pragma unroll
    for (int s = 0; s < EPT; ++s) {
        lm = fmaxf(lm, v[s]);
        nf += v[s] > NEG_INF;
    }
    TileStat st;
    st.pad = 0;
    if (c.T == 0.0f) {
        const float m = block_max(lm, sh.red);
        int am = INT_MAX;
        if (m > NEG_INF) {
#pragma unroll
            for (int s = EPT - 1; s >= 0; --s)
                if (v[s] == m) am = slot_id<DT>(tb, s);
        }
        am = block_min_i(am, sh.red);
        nf = block_sum_i(nf, sh.red);
        st.m = m;
        st.argmax = m > NEG_INF ? am : -1;
        st.s = 0.0;
        st.beta = NEG_INF;
        st.ncand = 0;
        st.nfinite = nf;
    } else {
        const float srt = block_sort_desc(lm, su.t.sorted);
        su.t.sorted[tid] = srt;
        __syncthreads();
        const float m = su.t.sorted[0];
        nf = block_sum_i(nf, sh.red);
        float theta = NEG_INF;
        int ncand = nf;
        if (nf > CW) {
            int L = LTARGET;
            for (;;) {
                theta = su.t.sorted[L];
                int cnt = 0;
#pragma unroll
                for (int s = 0; s < EPT; ++s) cnt += v[s] > theta;
                cnt = block_sum_i(cnt, sh.red);
                if (cnt <= CW) {
                    ncand = cnt;
                    break;
                }
                L = L > 16 ? L - 16 : 0;  // L = 0 puts theta at the tile max: no candidates
            }
        }
        double ssum = 0.0;
        if (m > NEG_INF) {
            const float c2 = 1.4426950408889634f / c.T;
            float acc = 0.0f;
#pragma unroll
            for (int s = 0; s < EPT; ++s) acc += exp2f((v[s] - m) * c2);
            ssum = acc;
        }
        ssum = block_sum_d(ssum, sh.red);
        int mine = 0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) mine += v[s] > theta;
        int tot;
        int off = block_excl_scan_i(mine, sh.red, tot);
        float2* cand = ws.cand + ((size_t)row * ws.n_tiles + tile) * CW;
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            if (v[s] > theta) {
                cand[off] = make_float2(v[s], __int_as_float(slot_id<DT>(tb, s)));
                ++off;
            }
        }
        st.m = m;
        st.argmax = -1;
        st.s = ssum;
        st.beta = theta;
        st.ncand = ncand;
        st.nfinite = nf;
    }
    if (tid == 0) ws.stats[(size_t)row * ws.n_tiles + tile] = st;
}

// Release this workgroup's stage-1 writes and count it in; true for the last
// workgroup of the group (which then sees every other workgroup's writes and
// leaves the counter at zero for the next launch or graph replay).
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, SmemS& sh) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        sh.is_last = (prev == expected - 1);
        if (sh.is_last)
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const bool last = sh.is_last != 0;
    if (last) __threadfence();
    return last;
}

// ---------------------------------------------------------------------------
// stage 2: row finaliser

struct RowDbg {
    int32_t* topk;     // row of [topk_stride] or null
    int topk_stride;
    int32_t* kept;     // scalar or null
    float* probs;      // row of [V] or null
    int32_t* path;     // scalar or null
};

struct RowSummary {
    float m;
    int argmax;
    int nfinite;
    float beta;
    double W;
};

__device__ RowSummary summarize_tiles(const TileStat* st, int n_tiles, float T) {
    const int lane = threadIdx.x & (WAVE - 1);
    TileStat t;
    if (lane < n_tiles) {
        t = st[lane];
    } else {
        t.m = NEG_INF;
        t.argmax = INT_MAX;
        t.s = 0.0;
        t.beta = NEG_INF;
        t.ncand = 0;
        t.nfinite = 0;
    }
    RowSummary r;
    r.m = wave_max(t.m);
    r.argmax = wave_min_i((t.m == r.m && t.argmax >= 0) ? t.argmax : INT_MAX);
    r.nfinite = wave_sum_i(t.nfinite);
    const bool incomplete = t.ncand < t.nfinite;
    r.beta = wave_max(incomplete ? t.beta : NEG_INF);
    double s = 0.0;
    if (T > 0.0f && t.m > NEG_INF && r.m > NEG_INF) {
        const float c2 = 1.4426950408889634f / T;
        s = t.s * (double)exp2f((t.m - r.m) * c2);
    }
    r.W = wave_sum_d(s);
    return r;
}

__device__ __forceinline__ uint64_t wq(float w) { return (uint64_t)((double)w * MASS_SCALE); }

// Radix selection over the row's z (scratch), 8 passes of 8-bit digits on key64.
// by_mass = false: the key of the rank-`target` element (1-based) in key order.
// by_mass = true: the key of the first element whose inclusive mass exceeds
// `target` (fixed point); the smallest key if none does.
template <class Pred>
__device__ unsigned long long radix_select(const float* zr, int V, float zmax, Pred pred,
                                           bool by_mass, unsigned long long target, SmemRadix& h,
                                           SmemS& sh) {
    const int tid = threadIdx.x;
    unsigned long long prefix = 0, pmask = 0, rem = target;
    int take_last = 0;
    for (int d = 7; d >= 0; --d) {
        for (int b = tid; b < 256; b += NT) {
            h.hc[b] = 0;
            h.hm[b] = 0;
        }
        __syncthreads();
        const int sft = d * 8;
        for (int v = tid; v < V; v += NT) {
            const float z = zr[v];
            if (!(z > NEG_INF)) continue;
            const unsigned long long k = key64(z, v);
            if ((k & pmask) != prefix) continue;
            const float w = expf(z - zmax);
            if (!pred(k, w)) continue;
            const int b = (int)((k >> sft) & 255ull);
            atomicAdd(&h.hc[b], 1u);
            if (by_mass) atomicAdd(&h.hm[b], (unsigned long long)wq(w));
        }
        __syncthreads();
        if (tid == 0) {
            unsigned long long cum = 0;
            int sel = -1, lastnz = -1;
            for (int b = 255; b >= 0; --b) {
                if (h.hc[b] == 0) continue;
                lastnz = b;
                const unsigned long long amt = by_mass ? h.hm[b] : (unsigned long long)h.hc[b];
                const bool hit = by_mass ? (cum + amt > rem) : (cum + amt >= rem);
                if (!take_last && hit) {
                    sel = b;
                    rem -= cum;
                    break;
                }
                cum += amt;
            }
            if (sel < 0) {
                sel = lastnz < 0 ? 0 : lastnz;
                take_last = 1;
            }
            sh.sel = sel;
            sh.take_last = take_last;
            sh.rem = rem;
        }
        __syncthreads();
        const int sel = sh.sel;
        take_last = sh.take_last;
        rem = sh.rem;
        prefix |= (unsigned long long)sel << sft;
        pmask |= 255ull << sft;
        __syncthreads();
    }
    return prefix;
}

template <class Pred>
__device__ void count_and_mass(const float* zr, int V, float zmax, Pred pred, int& count,
                               unsigned long long& mass, SmemS& sh) {
    int cnt = 0;
    unsigned long long ms = 0;
    for (int v = threadIdx.x; v < V; v += NT) {
        const float z = zr[v];
        if (!(z > NEG_INF)) continue;
        const float w = expf(z - zmax);
        if (pred(key64(z, v), w)) {
            ++cnt;
            ms += wq(w);
        }
    }
    count = block_sum_i(cnt, sh.red);
    // u64 sum: exact in any order
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ms += __shfl_xor(ms, o);
    __shared__ unsigned long long part[NT / WAVE];
    if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = ms;
    __syncthreads();
    unsigned long long t = 0;
#pragma unroll
    for (int k = 0; k < NT / WAVE; ++k) t += part[k];
    __syncthreads();
    mass = t;
}

// Exact whole-row resolution: recompute z for the whole row into scratch, then
// select by count (top-k) and by mass (top-p, the draw) with radix passes.
template <int DT>
__device__ void finalize_slow(const RowCtx& c, int row, const Workspace& ws, int n_tiles,
                              const RowSummary& rs, float u, SmemU& su, SmemS& sh, RowInfo& info,
                              const RowDbg& dbg) {
    const int tid = threadIdx.x;
    const int V = c.V;
    float* zr = ws.scratch_z + (size_t)row * V;
    for (int t = 0; t < n_tiles; ++t) {
        float v[EPT];
        load_tile<DT>(c, t * TILE, v);
        build_tables(c, t * TILE, su.t);
        process_tile<DT>(c, t * TILE, v, su.t);
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int id = slot_id<DT>(t * TILE, s);
            if (id < V) zr[id] = v[s] > NEG_INF ? canon_zero(v[s] / c.T) : NEG_INF;
        }
        __syncthreads();
    }
    const float zmax = canon_zero(rs.m / c.T);
    const int total = rs.nfinite;
    const bool topk_on = c.top_k > 0 && c.top_k < V;
    const int K_eff = topk_on ? min(c.top_k, total) : total;
    unsigned long long kK = 0;
    if (topk_on && K_eff < total)
        kK = radix_select(zr, V, zmax, [](unsigned long long, float) { return true; }, false,
                          (unsigned long long)K_eff, su.r, sh);
    int nK;
    unsigned long long WK;
    count_and_mass(zr, V, zmax, [kK](unsigned long long k, float) { return k >= kK; }, nK, WK, sh);
    unsigned long long kP = kK;
    if (c.top_p < 1.0f) {
        const unsigned long long tgt = (unsigned long long)((double)c.top_p * (double)WK);
        kP = radix_select(zr, V, zmax, [kK](unsigned long long k, float) { return k >= kK; }, true,
                          tgt, su.r, sh);
    }
    const float mp = c.min_p;
    auto kept = [kP, mp](unsigned long long k, float w) { return k >= kP && (mp <= 0.0f || w >= mp); };
    int n_kept;
    unsigned long long Wk;
    count_and_mass(zr, V, zmax, kept, n_kept, Wk, sh);
    const unsigned long long tgt = (unsigned long long)((double)u * (double)Wk);
    const unsigned long long kt = radix_select(zr, V, zmax, kept, true, tgt, su.r, sh);
    if (tid == 0) {
        info.kappa = kP;
        info.W = (double)Wk / MASS_SCALE;
        info.zmax = zmax;
        info.min_p = mp;
        info.n_kept = n_kept;
        info.token = key64_id(kt);
        info.argmax = -1;
        info.path = 1;
    }
    if (dbg.probs) {
        const double Wd = (double)Wk / MASS_SCALE;
        for (int v = tid; v < V; v += NT) {
            const float z = zr[v];
            float p = 0.0f;
            if (z > NEG_INF) {
                const float w = expf(z - zmax);
                if (kept(key64(z, v), w)) p = (float)((double)w / Wd);
            }
            dbg.probs[v] = p;
        }
    }
    if (dbg.topk) {
        int base = 0;
        for (int v0 = 0; v0 < V; v0 += NT) {
            const int v = v0 + tid;
            bool f = false;
            if (topk_on && v < V) {
                const float z = zr[v];
                f = z > NEG_INF && key64(z, v) >= kK;
            }
            int tot;
            const int off = block_excl_scan_i(f ? 1 : 0, sh.red, tot);
            if (f && base + off < dbg.topk_stride) dbg.topk[base + off] = v;
            base += tot;
        }
        for (int i = (topk_on ? min(base, dbg.topk_stride) : 0) + tid; i < dbg.topk_stride; i += NT)
            dbg.topk[i] = -1;
    }
    if (tid == 0) {
        if (dbg.kept) *dbg.kept = n_kept;
        if (dbg.path) *dbg.path = 1;
    }
    __syncthreads();
}

// Finds the first index i in [0, lim) of the sorted pool satisfying pred(i, excl,
// incl, w), scanning each thread's chunk in order with binary64 prefix sums.
template <class Pred>
__device__ int pool_first(int lim, int cs, const float* wl, double base, Pred pred, SmemS& sh) {
    int found = INT_MAX;
    double run = base;
    const int i0 = (int)threadIdx.x * cs;
    for (int k = 0; k < cs; ++k) {
        const int i = i0 + k;
        if (i >= lim) break;
        const double w = (double)wl[k];
        if (pred(i, run, run + w, wl[k])) {
            found = i;
            break;
        }
        run += w;
    }
    return block_min_i(found, sh.red);
}

template <int DT>
__device__ void finalize_row(const RowCtx& c, int row, const Workspace& ws, float u, SmemU& su,
                             SmemS& sh, const RowDbg& dbg, RowInfo& info_out) {
    const int tid = threadIdx.x;
    const int n_tiles = ws.n_tiles;
    const int V = c.V;
    // issue the stats and every candidate slot together: one round trip
    constexpr int PER = POOL / NT;
    const float2* cand = ws.cand + (size_t)row * n_tiles * CW;
    float2 cv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int g = tid + k * NT;
        cv[k] = g < n_tiles * CW ? cand[g] : make_float2(NEG_INF, 0.0f);
    }
    if (tid < n_tiles) su.p.st[tid] = ws.stats[(size_t)row * n_tiles + tid];
    if (tid == 0) sh.npool = 0;
    __syncthreads();
    const RowSummary rs = summarize_tiles(su.p.st, n_tiles, c.T);

    __shared__ RowInfo info;
    if (tid == 0) {
        info.kappa = 0;
        info.W = 1.0;
        info.zmax = rs.m;
        info.min_p = 0.0f;
        info.n_kept = rs.m > NEG_INF ? 1 : 0;
        info.token = rs.m > NEG_INF ? rs.argmax : -1;
        info.argmax = rs.m > NEG_INF ? rs.argmax : -1;
        info.path = 0;
    }
    if (c.T == 0.0f || !(rs.m > NEG_INF)) {
        __syncthreads();
        if (dbg.topk)
            for (int i = tid; i < dbg.topk_stride; i += NT) dbg.topk[i] = -1;
        if (tid == 0) {
            if (dbg.probs && info.token >= 0) dbg.probs[info.token] = 1.0f;
            if (dbg.kept) *dbg.kept = info.n_kept;
            if (dbg.path) *dbg.path = 0;
        }
        __syncthreads();
        info_out = info;
        return;
    }
    // the union of candidates above the highest tile threshold is exact
    const float zmax = canon_zero(rs.m / c.T);
    const float zb = rs.beta > NEG_INF ? canon_zero(rs.beta / c.T) : NEG_INF;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int g = tid + k * NT;
        const int t = g / CW;
        if (g < n_tiles * CW && (g % CW) < su.p.st[t].ncand) {
            const float z = canon_zero(cv[k].x / c.T);
            if (z > zb) {
                const int pos = atomicAdd(&sh.npool, 1);
                su.p.z[pos] = z;
                su.p.id[pos] = __float_as_int(cv[k].y);
            }
        }
    }
    __syncthreads();
    const int n = sh.npool;
    int n_pad = 1;
    while (n_pad < n) n_pad <<= 1;
    for (int i = n + tid; i < n_pad; i += NT) {
        su.p.z[i] = NEG_INF;
        su.p.id[i] = INT_MAX;
    }
    __syncthreads();
    // bitonic sort of the pool into key order (z descending, id ascending)
    for (int k = 2; k <= n_pad; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n_pad; i += NT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const float za = su.p.z[i], zb2 = su.p.z[ixj];
                    const int ia = su.p.id[i], ib = su.p.id[ixj];
                    const bool a_first = key_before(za, ia, zb2, ib);
                    const bool desc = (i & k) == 0;
                    if (desc ? !a_first : a_first) {
                        su.p.z[i] = zb2;
                        su.p.z[ixj] = za;
                        su.p.id[i] = ib;
                        su.p.id[ixj] = ia;
                    }
                }
            }
            __syncthreads();
        }
    }
    // per-thread contiguous chunks, weights, binary64 exclusive prefix
    const int cs = n_pad > NT ? n_pad / NT : 1;
    float wl[POOL / NT];
    double loc = 0.0;
#pragma unroll
    for (int k = 0; k < POOL / NT; ++k) {
        const int i = tid * cs + k;
        wl[k] = (k < cs && i < n) ? expf(su.p.z[i] - zmax) : 0.0f;
        loc += (double)wl[k];
    }
    double totw;
    const double base = block_excl_scan_d(loc, sh.red, totw);

    const int total = rs.nfinite;
    const bool topk_on = c.top_k > 0 && c.top_k < V;
    const int K_eff = topk_on ? min(c.top_k, total) : total;
    const bool cut_k = topk_on && K_eff < total;
    // the debug top-k list needs the whole set when top-k keeps every finite entry
    bool fallback = n == 0 || (cut_k && K_eff > n) || (dbg.topk && topk_on && !cut_k && total > n);
    double WK = rs.W;
    int n_topp = cut_k ? K_eff : total;
    int n_kept = n_topp;
    int token = -1;
    double Wk = rs.W;
    if (!fallback && cut_k) {
        double part = 0.0;
#pragma unroll
        for (int k = 0; k < POOL / NT; ++k)
            if (tid * cs + k < K_eff) part += (double)wl[k];
        WK = block_sum_d(part, sh.red);
    }
    if (!fallback && c.top_p < 1.0f) {
        const double thr = (double)c.top_p * WK;
        const int lim = min(n, n_topp);
        const int f = pool_first(lim, cs, wl, base,
                                 [thr](int, double ex, double, float) { return ex >= thr; }, sh);
        if (f != INT_MAX) n_topp = f;
        else if (n_topp > n) fallback = true;
        n_kept = n_topp;
    }
    if (!fallback && c.min_p > 0.0f) {
        const float mp = c.min_p;
        const int lim = min(n, n_topp);
        const int f = pool_first(lim, cs, wl, base,
                                 [mp](int, double, double, float w) { return w < mp; }, sh);
        if (f != INT_MAX) n_kept = f;
        else if (n_topp > n) fallback = true;
        else n_kept = n_topp;
    }
    if (!fallback && dbg.probs && n_kept > n) fallback = true;
    if (!fallback) {
        if (n_kept < total) {
            double part = 0.0;
#pragma unroll
            for (int k = 0; k < POOL / NT; ++k)
                if (tid * cs + k < n_kept) part += (double)wl[k];
            Wk = block_sum_d(part, sh.red);
        }
        const double tgt = (double)u * Wk;
        const int lim = min(n, n_kept);
        const int f = pool_first(lim, cs, wl, base,
                                 [tgt](int, double, double in, float) { return in > tgt; }, sh);
        if (f != INT_MAX) token = su.p.id[f];
        else if (n_kept <= n) token = su.p.id[n_kept - 1];
        else fallback = true;
    }
    if (fallback) {
        __syncthreads();
        finalize_slow<DT>(c, row, ws, n_tiles, rs, u, su, sh, info, dbg);
        __syncthreads();
        info_out = info;
        return;
    }
    if (tid == 0) {
        info.kappa = n_kept < total ? key64(su.p.z[n_kept - 1], su.p.id[n_kept - 1]) : 0ull;
        info.W = Wk;
        info.zmax = zmax;
        info.min_p = 0.0f;
        info.n_kept = n_kept;
        info.token = token;
        info.argmax = -1;
        info.path = 0;
        if (dbg.kept) *dbg.kept = n_kept;
        if (dbg.path) *dbg.path = 0;
    }
    if (dbg.probs) {
        for (int i = tid; i < n_kept; i += NT)
            dbg.probs[su.p.id[i]] = (float)((double)expf(su.p.z[i] - zmax) / Wk);
    }
    if (dbg.topk) {
        const int lim = cut_k ? K_eff : (topk_on ? total : 0);
        for (int i = tid; i < dbg.topk_stride; i += NT)
            dbg.topk[i] = (i < lim && i < n) ? su.p.id[i] : -1;
    }
    __syncthreads();
    info_out = info;
}

// ---------------------------------------------------------------------------
// kernels

// Maps the linear workgroup index to a (row, tile) pair so that the tiles of a
// row run on the same XCD (dispatch places workgroup i on XCD i mod 8), which
// keeps the last-block merge's reads in that XCD's L2.
__device__ __forceinline__ int xcd_linear(int n) {
    const int i = blockIdx.x;
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

template <int DT>
__global__ __launch_bounds__(NT) void k_sample(SampleArgs a) {
    __shared__ SmemU su;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int lin = xcd_linear(a.B * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const void* logits = (const char*)a.logits + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    const RowCtx c = make_ctx(a.p, row, logits, a.V, nullptr, 0, mrow, 0);
    tile_stage1<DT>(c, row, tile, a.ws, su, sh,
                    a.dbg_processed ? a.dbg_processed + (size_t)row * a.V : nullptr,
                    a.dbg_probs ? a.dbg_probs + (size_t)row * a.V : nullptr);
    if (!arrive_last(a.ws.row_counter + row, (uint32_t)n_tiles, sh)) return;
    const float u = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_SAMPLE));
    RowDbg dbg;
    dbg.topk = a.dbg_topk ? a.dbg_topk + (size_t)row * a.dbg_topk_stride : nullptr;
    dbg.topk_stride = a.dbg_topk_stride;
    dbg.kept = a.dbg_kept ? a.dbg_kept + row : nullptr;
    dbg.probs = a.dbg_probs ? a.dbg_probs + (size_t)row * a.V : nullptr;
    dbg.path = a.dbg_path ? a.dbg_path + row : nullptr;
    RowInfo info;
    finalize_row<DT>(c, row, a.ws, u, su, sh, dbg, info);
    if (threadIdx.x == 0) a.out_tokens[row] = info.token;
}

// Verification, kernel 1: every target row of every request runs stage 1 and
// the row finaliser; each draft row then takes its accept decision, the bonus
// row samples its token, and the last row of a request assembles the output.
template <int DT>
__global__ __launch_bounds__(NT) void k_spec_rows(SpecArgs a) {
    __shared__ SmemU su;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int G1 = a.G + 1;
    const int lin = xcd_linear(a.B * G1 * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const int b = row / G1;
    const int j = row % G1;
    const void* logits = (const char*)a.target + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    const int32_t* drafts = a.draft_tokens + (size_t)b * a.G;
    const RowCtx c = make_ctx(a.p, b, logits, a.V, drafts, j, mrow, (uint32_t)j);
    tile_stage1<DT>(c, row, tile, a.ws, su, sh, nullptr, nullptr);
    if (!arrive_last(a.ws.row_counter + row, (uint32_t)n_tiles, sh)) return;
    RowDbg dbg = {nullptr, 0, nullptr, nullptr, nullptr};
    const float u = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_SAMPLE));
    RowInfo info;
    finalize_row<DT>(c, row, a.ws, u, su, sh, dbg, info);
    if (j < a.G) {
        const int d = drafts[j];
        int acc;
        if (c.T == 0.0f || info.n_kept == 0) {
            acc = (info.argmax >= 0 && d == info.argmax) ? 1 : 0;
        } else if (d < 0 || d >= a.V) {
            acc = 0;
        } else {
            const float xd = single_entry<DT>(c, d, sh);
            double pi = 0.0;
            if (xd > NEG_INF) {
                const float zd = canon_zero(xd / c.T);
                const float w = expf(zd - info.zmax);
                const bool kept = key64(zd, d) >= info.kappa && (info.min_p <= 0.0f || w >= info.min_p);
                if (kept) pi = (double)w / info.W;
            }
            const double q = (double)a.draft_probs[((size_t)b * a.G + j) * a.draft_stride + d];
            const float ua = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_ACCEPT));
            acc = q > 0.0 ? ((double)ua < pi / q ? 1 : 0) : (pi > 0.0 ? 1 : 0);
        }
        if (threadIdx.x == 0) a.ws.row_accept[row] = acc;
    }
    if (threadIdx.x == 0) a.ws.rowinfo[row] = info;
    if (!arrive_last(a.ws.req_counter + b, (uint32_t)G1, sh)) return;
    if (threadIdx.x == 0) {
        int n = a.G;
        for (int k = 0; k < a.G; ++k)
            if (!a.ws.row_accept[(size_t)b * G1 + k]) {
                n = k;
                break;
            }
        int32_t* out = a.out_tokens + (size_t)b * G1;
        for (int k = 0; k < n; ++k) out[k] = drafts[k];
        const RowInfo ri = a.ws.rowinfo[(size_t)b * G1 + n];
        int resid = -1;
        if (n == a.G) out[n] = ri.token;
        else if (c.T == 0.0f || ri.n_kept == 0) out[n] = ri.argmax;
        else {
            out[n] = -1;
            resid = n;
        }
        for (int k = n + 1; k < G1; ++k) out[k] = -1;
        a.out_num_accepted[b] = n;
        a.ws.resid_row[b] = resid;
    }
}

// Residual mass of one tile of a rejected row: r = max(0, pi - q) per entry (or
// pi itself when use_pi), in token-id order within each thread group.
template <int DT>
__device__ void residual_values(const RowCtx& c, const RowInfo& ri, const float* q, int tb,
                                bool use_pi, SmemU& su, double r[EPT]) {
    float v[EPT];
    load_tile<DT>(c, tb, v);
    build_tables(c, tb, su.t);
    process_tile<DT>(c, tb, v, su.t);
#pragma unroll
    for (int s = 0; s < EPT; ++s) {
        const int id = slot_id<DT>(tb, s);
        double val = 0.0;
        if (id < c.V && v[s] > NEG_INF) {
            const float z = canon_zero(v[s] / c.T);
            const float w = expf(z - ri.zmax);
            const bool kept = key64(z, id) >= ri.kappa && (ri.min_p <= 0.0f || w >= ri.min_p);
            const float pi = kept ? (float)((double)w / ri.W) : 0.0f;
            val = use_pi ? (double)pi : (double)fmaxf(0.0f, pi - q[id]);
        }
        r[s] = val;
    }
}

template <int DT>
__global__ __launch_bounds__(NT) void k_spec_residual(SpecArgs a) {
    __shared__ SmemU su;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x % n_tiles;
    const int j = a.ws.resid_row[b];
    if (j < 0) return;
    const int G1 = a.G + 1;
    const int row = b * G1 + j;
    const void* logits = (const char*)a.target + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    const int32_t* drafts = a.draft_tokens + (size_t)b * a.G;
    const RowCtx c = make_ctx(a.p, b, logits, a.V, drafts, j, mrow, (uint32_t)j);
    const RowInfo ri = a.ws.rowinfo[row];
    const float* q = a.draft_probs + ((size_t)b * a.G + j) * a.draft_stride;
    double r[EPT];
    {
        residual_values<DT>(c, ri, q, tile * TILE, false, su, r);
        double sr = 0.0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) sr += r[s];
        sr = block_sum_d(sr, sh.red);
        __syncthreads();
        // pi alone, for a residual that sums to zero
        double rp[EPT];
        residual_values<DT>(c, ri, q, tile * TILE, true, su, rp);
        double sp = 0.0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) sp += rp[s];
        sp = block_sum_d(sp, sh.red);
        if (threadIdx.x == 0) a.ws.resid_tile[(size_t)b * n_tiles + tile] = make_double2(sr, sp);
    }
    if (!arrive_last(a.ws.resid_counter + b, (uint32_t)n_tiles, sh)) return;
    // last tile of this request: locate the tile, then the entry, in id order
    __shared__ int s_tile;
    __shared__ int s_usepi;
    __shared__ double s_rem;
    if (threadIdx.x == 0) {
        double R = 0.0, P = 0.0;
        for (int t = 0; t < n_tiles; ++t) {
            const double2 x = a.ws.resid_tile[(size_t)b * n_tiles + t];
            R += x.x;
            P += x.y;
        }
        const int use_pi = !(R > 0.0);
        const double tot = use_pi ? P : R;
        const float ur = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_RESIDUAL));
        const double tgt = (double)ur * tot;
        double cum = 0.0;
        int sel = -1, lastnz = -1;
        double rem = 0.0;
        for (int t = 0; t < n_tiles; ++t) {
            const double2 x = a.ws.resid_tile[(size_t)b * n_tiles + t];
            const double amt = use_pi ? x.y : x.x;
            if (amt > 0.0) lastnz = t;
            if (sel < 0 && cum + amt > tgt && amt > 0.0) {
                sel = t;
                rem = tgt - cum;
            }
            cum += amt;
        }
        if (sel < 0) {
            sel = lastnz;
            rem = DBL_MAX;
        }
        s_tile = sel;
        s_usepi = use_pi;
        s_rem = rem;
    }
    __syncthreads();
    const int st = s_tile;
    int token = -1;
    if (st >= 0) {
        residual_values<DT>(c, ri, q, st * TILE, s_usepi != 0, su, r);
        using L = Lay<DT>;
        double carry = 0.0;
        int found = INT_MAX, lastpos = -1;
        const double rem = s_rem;
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            double gs = 0.0;
#pragma unroll
            for (int k = 0; k < L::VEC; ++k) gs += r[g * L::VEC + k];
            double gt;
            const double gb = block_excl_scan_d(gs, sh.red, gt);
            double run = carry + gb;
#pragma unroll
            for (int k = 0; k < L::VEC; ++k) {
                const double x = r[g * L::VEC + k];
                const int id = slot_id<DT>(st * TILE, g * L::VEC + k);
                if (x > 0.0) {
                    lastpos = max(lastpos, id);
                    if (found == INT_MAX && run + x > rem) found = id;
                }
                run += x;
            }
            carry += gt;
        }
        found = block_min_i(found, sh.red);
        lastpos = -block_min_i(-lastpos, sh.red);
        token = found != INT_MAX ? found : lastpos;
    }
    if (threadIdx.x == 0) a.out_tokens[(size_t)b * G1 + j] = token;
}

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_sample(const SampleArgs& a, ss_dtype dt, hipStream_t st) {
    const dim3 grid(a.B * a.ws.n_tiles);
    if (dt == SS_F32) hipLaunchKernelGGL(k_sample<SS_F32>, grid, dim3(NT), 0, st, a);
    else hipLaunchKernelGGL(k_sample<SS_BF16>, grid, dim3(NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_spec(const SpecArgs& a, ss_dtype dt, hipStream_t st) {
    const dim3 grid1(a.B * (a.G + 1) * a.ws.n_tiles);
    const dim3 grid2(a.B * a.ws.n_tiles);
    if (dt == SS_F32) {
        hipLaunchKernelGGL(k_spec_rows<SS_F32>, grid1, dim3(NT), 0, st, a);
        hipLaunchKernelGGL(k_spec_residual<SS_F32>, grid2, dim3(NT), 0, st, a);
    } else {
        hipLaunchKernelGGL(k_spec_rows<SS_BF16>, grid1, dim3(NT), 0, st, a);
        hipLaunchKernelGGL(k_spec_residual<SS_BF16>, grid2, dim3(NT), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace ss

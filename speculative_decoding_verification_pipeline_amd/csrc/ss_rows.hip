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
//  * Stage 1 streams the tile once with 16-byte global loads (float4 / 8 x
//    bf16), applies penalties (multiplicities counted in LDS), bias and the
//    packed mask in registers, and reduces: tile max, softmax partial sum, and a
//    candidate list -- every entry above a threshold taken from the sorted
//    per-thread maxima, so the list is always an exact prefix of the tile in
//    key order. Its length is capped per request: greedy rows need none, a
//    top-k row never more than k from one tile, other rows a short head (the
//    low-entropy structure of LLM logits puts nearly all mass there).
//  * A second launch, one workgroup per row, merges (the kernel boundary is the
//    only synchronisation, so stage 1 carries no fences and only its own
//    registers): candidates above the highest tile threshold form an exact
//    prefix of the whole row (the pool, in LDS). Its first 256 entries are
//    sorted across the workgroup with a bitonic network in registers; the
//    top-k boundary deeper than that comes from a radix selection over the
//    pool; top-p, min-p and the inverse-CDF draw are ballots over binary64
//    prefix sums of the sorted head. Requests that reach
//    past the head sort the whole pool ("deep" path), and requests that reach
//    past the pool run an exact whole-row fallback (radix selection by count
//    and by mass over the row's recomputed z). Results never depend on which
//    path resolved them.
#include <float.h>
#include <limits.h>

#include "ss_device.h"
#include "ss_internal.h"

#pragma clang fp contract(off)

namespace ss {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr double MASS_SCALE = 17592186044416.0;  // 2^44 fixed-point weights in the fallback
constexpr int CAP_FREE = 32;   // candidates per tile for rows without top-k
constexpr int CAP_MIN = 8;     // smallest cap for a top-k row

// Loads through the global address space (16-byte vector loads, no flat path).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ T gld(const T* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}
template <>
__device__ __forceinline__ uint4 gld<uint4>(const uint4* p) {
    const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ float2 gld<float2>(const float2* p) {
    const f32x2_t v = *(const __attribute__((address_space(1))) f32x2_t*)p;
    return make_float2(v.x, v.y);
}

struct RowCtx {
    const void* logits;
    int V;
    float T;
    int top_k;
    float top_p;
    float min_p;
    float rep, freq, pres;
    const int32_t* hist;
    int hist_len;          // clamped to hist_cap
    int hist_cap;          // row stride of the history ids (entries readable for this row)
    const int32_t* extra;  // draft tokens that precede this row (verification)
    int extra_len;
    const int32_t* bias_ids;
    const float* bias_vals;
    int bias_len;          // clamped to bias_cap
    int bias_cap;
    const uint32_t* mask;  // this row's mask words or null
    uint32_t req, pos;
    uint64_t seed;
};

// Every parameter pointer is valid (the host substitutes defaults for absent
// ones), so all reads are unconditional and issue together.
__device__ __forceinline__ RowCtx make_ctx(const ParamPtrs& p, int b, const void* logits, int V,
                                           const int32_t* extra, int extra_len,
                                           const uint32_t* mask_row, uint32_t pos_offset) {
    RowCtx c;
    c.logits = logits;
    c.V = V;
    c.T = p.temperature[b];
    c.top_k = p.top_k[b];
    c.top_p = p.top_p[b];
    c.min_p = p.min_p[b];
    c.rep = p.rep[b];
    c.freq = p.freq[b];
    c.pres = p.pres[b];
    c.hist_cap = p.hist_stride;
    c.hist_len = min(p.hist_len[b], p.hist_stride);
    c.hist = p.hist_ids + (int64_t)b * p.hist_stride;
    c.extra = extra;
    c.extra_len = extra ? extra_len : 0;
    c.bias_cap = p.bias_stride;
    c.bias_len = min(p.bias_len[b], p.bias_stride);
    c.bias_ids = p.bias_ids + (int64_t)b * p.bias_stride;
    c.bias_vals = p.bias_vals + (int64_t)b * p.bias_stride;
    c.mask = mask_row;
    c.req = (uint32_t)p.request_ids[b];
    c.pos = (uint32_t)p.positions[b] + pos_offset;
    c.seed = p.seed;
    return c;
}

// ---------------------------------------------------------------------------
// LDS layouts (one union per workgroup; phases are separated by barriers)

struct SmemTile {
    uint32_t cnt[TILE / 2];   // u16 history multiplicities of the tile's entries
    uint32_t bias[TILE / 32]; // bit set: some bias entry targets this vocabulary entry
    int32_t bid[NT];          // the row's first NT bias entries, in array order
    float bval[NT];
    union {
        struct {
            float lmax[NT];    // per-wave sorted thread maxima
            float sorted[NT];  // all thread maxima in descending order
        };
        unsigned long long keys[CW];  // the candidates' keys (z, id), once the threshold is set
    };
    unsigned long long list[CW];  // the tile's candidates (x' bits, id), unordered
};

// The row merge runs one 1024-thread workgroup per row (four waves per SIMD).
constexpr int NTR = 1024;
constexpr int PERR = POOL / NTR;  // candidate slots per merge thread
constexpr int OCT = NTR / CW;     // tiles covered by one slot round
constexpr int MERGE_LG_MAX = 12;  // log2 of the largest merge segment (POOL slots)

// A pointer into LDS that the compiler keeps in the LDS address space (32-bit
// addresses, ds_read), also through the merge's unrolled pointer walks.
typedef const unsigned long long __attribute__((address_space(3)))* lds_key_ptr;

struct SmemPool {
    unsigned long long buf[2][POOL];  // merge-tree ping-pong buffers (keys, zero = empty slot)
    int wcnt[PERR][NTR / WAVE];       // kept candidates per (slot round, wave)
    int len[2][MAX_TILES];            // segment lengths per merge level
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

template <int NB>
struct SmemST {
    RedT<NB> red;
    RedT<NB> red2;
    int sel;
    int take_last;
    unsigned long long rem;
};
using SmemS = SmemST<NT>;   // tile workgroups
using SmemR = SmemST<NTR>;  // row-merge workgroups

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
    if (DT == SS_F32) return gld((const float*)row + id);
    const uint32_t b = gld((const uint16_t*)row + id);
    return __uint_as_float(b << 16);
}

template <int DT>
__device__ __forceinline__ void unpack_group(const uint4 q, float* out) {
    if constexpr (DT == SS_F32) {
        out[0] = __uint_as_float(q.x);
        out[1] = __uint_as_float(q.y);
        out[2] = __uint_as_float(q.z);
        out[3] = __uint_as_float(q.w);
    } else {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = __uint_as_float(w[k] << 16);
            out[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
}

template <int DT, bool ALIGNED = false>
__device__ __forceinline__ void load_tile(const RowCtx& c, int tb, float v[EPT]) {
    using L = Lay<DT>;
    constexpr int ES = DT == SS_F32 ? 4 : 2;
    const char* row = (const char*)c.logits;
    if constexpr (ALIGNED) {
        // Rows 16-byte aligned and V a multiple of VEC (checked by the host):
        // a group lies wholly inside or wholly past V, and a group past V reads
        // the row's last group instead and is set to -inf. Branch-free, so the
        // compiler can count these loads exactly behind earlier ones.
        uint4 q[L::NG];
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
            // the logits are read once: non-temporal, so they do not push the
            // row's history ids and the tile summaries out of L2
            const u32x4_t* src = (const u32x4_t*)(row + (size_t)min(e0, c.V - L::VEC) * ES);
            const u32x4_t qv = __builtin_nontemporal_load(src);
            q[g] = make_uint4(qv.x, qv.y, qv.z, qv.w);
        }
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
            unpack_group<DT>(q[g], v + g * L::VEC);
#pragma unroll
            for (int j = 0; j < L::VEC; ++j) v[g * L::VEC + j] = e0 < c.V ? v[g * L::VEC + j] : NEG_INF;
        }
        return;
    }
    // 16-byte loads need a 16-byte aligned row; a full tile needs no bounds checks
    const bool vec = ((uintptr_t)row & 15u) == 0;
    if (vec && tb + TILE <= c.V) {
        uint4 q[L::NG];
#pragma unroll
        for (int g = 0; g < L::NG; ++g)
            q[g] = gld((const uint4*)(row + (size_t)(tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC) * ES));
#pragma unroll
        for (int g = 0; g < L::NG; ++g) unpack_group<DT>(q[g], v + g * L::VEC);
        return;
    }
#pragma unroll
    for (int g = 0; g < L::NG; ++g) {
        const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
        if (vec && e0 + L::VEC <= c.V) {
            unpack_group<DT>(gld((const uint4*)(row + (size_t)e0 * ES)), v + g * L::VEC);
        } else {
#pragma unroll
            for (int j = 0; j < L::VEC; ++j)
                v[g * L::VEC + j] = (e0 + j < c.V) ? read_logit<DT>(row, e0 + j) : NEG_INF;
        }
    }
}

// Penalties -> bias -> mask for one entry. Shared by every path that forms x'
// so all of them produce the same binary32 value. Bias entries are applied in
// array order; with tables, the first NT of them come from LDS.
__device__ __forceinline__ float penalize(const RowCtx& c, float x, uint32_t count) {
    if (count) {
        x = (x > 0.0f) ? x / c.rep : x * c.rep;
        const float fc = c.freq * (float)count;
        x = x - fc;
        x = x - c.pres;
    }
    return x;
}

__device__ __forceinline__ float process_entry(const RowCtx& c, int id, float x, uint32_t count,
                                               bool bias_hit, bool allowed) {
    x = penalize(c, x, count);
    if (bias_hit) {
        for (int k = 0; k < c.bias_len; ++k)
            if (gld(c.bias_ids + k) == id) x = x + gld(c.bias_vals + k);
    }
    return allowed ? x : NEG_INF;
}

__device__ __forceinline__ float process_entry_t(const RowCtx& c, int id, float x, uint32_t count,
                                                 bool bias_hit, bool allowed, const SmemTile& t) {
    x = penalize(c, x, count);
    if (bias_hit) {
        const int nl = min(c.bias_len, NT);
        for (int k = 0; k < nl; ++k)
            if (t.bid[k] == id) x = x + t.bval[k];
        for (int k = NT; k < c.bias_len; ++k)
            if (gld(c.bias_ids + k) == id) x = x + gld(c.bias_vals + k);
    }
    return allowed ? x : NEG_INF;
}

// The row's history and bias lists are small and shared by all its tiles. Each
// thread fetches its first two history ids, its draft token and one bias
// entry with addresses that depend on kernel arguments only (the row strides
// bound what is readable), so the loads issue ahead of the tile's logits
// without waiting for the per-request lengths.
// A 4-byte global load the optimiser keeps in program order (a relaxed
// workgroup-scope atomic load: the same instruction as a plain load).
__device__ __forceinline__ int pinned_load(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct TablePrefetch {
    int hist[2];
    int extra;
    int bias_id;
    float bias_val;
};

__device__ __forceinline__ TablePrefetch prefetch_tables(const RowCtx& c) {
    TablePrefetch f;
    const int tid = threadIdx.x;
    // Unconditional loads at clamped indices (entry 0 of every list is
    // readable: absent lists point at default arrays), so every path issues the
    // same loads in the same order and the loads issued after these (the
    // tile's) need not complete before the tables are built.
    // They are relaxed atomic loads only so that the compiler keeps them here,
    // ahead of the tile's, instead of sinking them into the table build.
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = tid + k * NT;
        const int h = pinned_load(c.hist + min(i, max(c.hist_cap - 1, 0)));
        f.hist[k] = i < c.hist_cap ? h : -1;
    }
    int e = -1;  // no draft list (sampling): no load at all
    if (c.extra) e = pinned_load(c.extra + min(tid, max(c.extra_len - 1, 0)));
    f.extra = tid < c.extra_len ? e : -1;
    const int bi = min(tid, max(c.bias_cap - 1, 0));
    const int bid = pinned_load(c.bias_ids + bi);
    const float bv = __int_as_float(pinned_load((const int32_t*)c.bias_vals + bi));
    f.bias_id = tid < c.bias_cap ? bid : -1;
    f.bias_val = tid < c.bias_cap ? bv : 0.0f;
    return f;
}

// Builds the tile's multiplicity counts, bias bitmap and bias list in LDS (two
// barriers). Threads with active = false only take part in the barriers.
__device__ __forceinline__ void build_tables(const RowCtx& c, int tb, SmemTile& t,
                                             const TablePrefetch& f, bool active = true) {
    const int tid = threadIdx.x;
    const bool has_cnt = active && (c.hist_len + c.extra_len) > 0;
    const bool has_bias = active && c.bias_len > 0;
    if (has_cnt) {
        uint4* c4 = (uint4*)t.cnt;
#pragma unroll
        for (int k = 0; k < TILE / 8 / NT; ++k) c4[tid + k * NT] = make_uint4(0, 0, 0, 0);
    }
    if (has_bias) {
        t.bias[tid] = 0;
        t.bid[tid] = f.bias_id;
        t.bval[tid] = f.bias_val;
    }
    __syncthreads();
    auto count = [&](int id) {
        const int l = id - tb;
        if (id >= 0 && id < c.V && l >= 0 && l < TILE) atomicAdd(&t.cnt[l >> 1], 1u << ((l & 1) * 16));
    };
    if (has_cnt) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (tid + k * NT < c.hist_len) count(f.hist[k]);
        for (int i = tid + 2 * NT; i < c.hist_len; i += NT) count(gld(c.hist + i));
        if (tid < c.extra_len) count(f.extra);
    }
    auto mark = [&](int id) {
        const int l = id - tb;
        if (id >= 0 && id < c.V && l >= 0 && l < TILE) atomicOr(&t.bias[l >> 5], 1u << (l & 31));
    };
    if (has_bias && tid < c.bias_len) mark(f.bias_id);
    for (int i = tid + NT; has_bias && i < c.bias_len; i += NT) mark(gld(c.bias_ids + i));
    __syncthreads();
}

// This thread's grammar-mask words (one per group of VEC entries), fetched with
// the tile's logits; all-ones without a mask.
template <int DT>
__device__ __forceinline__ void load_mask(const RowCtx& c, int tb, uint32_t mw[Lay<DT>::NG]) {
    using L = Lay<DT>;
#pragma unroll
    for (int g = 0; g < L::NG; ++g) {
        const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
        mw[g] = (c.mask && e0 < c.V) ? gld(c.mask + (e0 >> 5)) : 0xFFFFFFFFu;
    }
}

template <int DT>
__device__ __forceinline__ void process_tile(const RowCtx& c, int tb, float v[EPT], const SmemTile& t,
                                             const uint32_t mwords[Lay<DT>::NG]) {
    using L = Lay<DT>;
    const bool has_cnt = (c.hist_len + c.extra_len) > 0;
    const bool has_bias = c.bias_len > 0;
    if (!has_cnt && !has_bias && !c.mask) return;
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
        const uint32_t mw = mwords[g] >> (e0 & 31);
        // most groups hold no history hit, bias or masked entry: skip them whole
        constexpr uint32_t vm = (1u << L::VEC) - 1u;
        uint32_t anyc = 0;
#pragma unroll
        for (int k = 0; k < L::VEC / 2; ++k) anyc |= cw[k];
        if ((anyc | (bb & vm) | (~mw & vm)) == 0u) continue;
#pragma unroll
        for (int j = 0; j < L::VEC; ++j) {
            const int id = e0 + j;
            if (id >= c.V) continue;
            const uint32_t cnt = (cw[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
            const bool hit = (bb >> j) & 1u;
            const bool allowed = (mw >> j) & 1u;
            float x = v[g * L::VEC + j];
            if (cnt | hit | !allowed) x = process_entry_t(c, id, x, cnt, hit, allowed, t);
            v[g * L::VEC + j] = x;
        }
    }
}

// x' for a single entry (used by acceptance tests). Whole workgroup participates.
template <int DT, int NB>
__device__ __forceinline__ float single_entry(const RowCtx& c, int id, SmemST<NB>& sh) {
    int cnt = 0;
    for (int i = threadIdx.x; i < c.hist_len + c.extra_len; i += NB) {
        const int h = i < c.hist_len ? gld(c.hist + i) : gld(c.extra + (i - c.hist_len));
        cnt += (h == id);
    }
    cnt = block_sum_i(cnt, sh.red);
    bool hit = false;
    for (int k = 0; k < c.bias_len; ++k) hit |= (gld(c.bias_ids + k) == id);
    const bool allowed = c.mask ? ((gld(c.mask + (id >> 5)) >> (id & 31)) & 1u) : true;
    const float x = read_logit<DT>(c.logits, id);
    return process_entry(c, id, x, (uint32_t)cnt, hit, allowed);
}

// Candidate cap of one tile for this request: no tile can hold more than k of a
// row's top-k; rows without top-k keep a short head.
__device__ __forceinline__ int row_cap(const RowCtx& c) {
    if (c.T == 0.0f) return 0;
    if (c.top_k > 0 && c.top_k < c.V) return min(CW, max(c.top_k, CAP_MIN));
    return CAP_FREE;
}

// ---------------------------------------------------------------------------
// stage 1: one tile of one row

template <int DT, bool ALIGNED>
__device__ __forceinline__ void tile_stage1(const RowCtx& c, int row, int tile, const Workspace& ws, SmemTile& tt,
                            SmemS& sh, float* dbg_proc_row, float* dbg_probs_row) {
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int tb = tile * TILE;
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    // issue order: mask words and history / bias (needed first), then the
    // tile, which the tables' build does not wait for
    load_mask<DT>(c, tb, mw);
    const TablePrefetch f = prefetch_tables(c);
    __builtin_amdgcn_sched_barrier(0);
    load_tile<DT, ALIGNED>(c, tb, v);
    if (c.hist_len + c.extra_len + c.bias_len > 0) build_tables(c, tb, tt, f);
    process_tile<DT>(c, tb, v, tt, mw);

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

    // lane maximum and minimum; entries are counted one by one only in waves
    // where some lane holds a -inf
    float lm = v[0], lmin = v[0];
#pragma unroll
    for (int s = 1; s < EPT; ++s) {
        lm = fmaxf(lm, v[s]);
        lmin = fminf(lmin, v[s]);
    }
    int nf = EPT;
    if (__ballot(!(lmin > NEG_INF))) {
        nf = 0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) nf += v[s] > NEG_INF;
    }
    TileStat st;
    st.pad = 0;
    const int cap = row_cap(c);
    if (cap == 0) {
        const float m = block_max(lm, sh.red);
        int am = INT_MAX;
        // only lanes holding the maximum look for its lowest index
        if (m > NEG_INF && lm == m) {
#pragma unroll
            for (int s = EPT - 1; s >= 0; --s)
                if (v[s] == m) am = slot_id<DT>(tb, s);
        }
        // argmin and finite count share one exchange
        am = wave_min_i(am);
        nf = wave_sum_i(nf);
        if (lane == 0) {
            sh.red.i[wv] = am;
            sh.red2.i[wv] = nf;
        }
        __syncthreads();
        am = sh.red.i[0];
        nf = sh.red2.i[0];
#pragma unroll
        for (int k = 1; k < NT / WAVE; ++k) {
            am = min(am, sh.red.i[k]);
            nf += sh.red2.i[k];
        }
        st.m = m;
        st.argmax = m > NEG_INF ? am : -1;
        st.s = 0.0;
        st.beta = NEG_INF;
        st.ncand = 0;
        st.nfinite = nf;
    } else {
        // the lane maxima, sorted descending, seed the candidate threshold: each
        // wave sorts its 64 through DPP, then every maximum finds its place
        // among the other waves' sorted lists (ties: lower wave first)
        nf = wave_sum_i(nf);
        if (lane == 0) sh.red.i[wv] = nf;
        const float srt = wave_sort_desc(lm);
        tt.lmax[tid] = srt;
        __syncthreads();
        nf = sh.red.i[0] + sh.red.i[1] + sh.red.i[2] + sh.red.i[3];
        {
            int pos[NT / WAVE - 1];
            const float* lst[NT / WAVE - 1];
            bool ge[NT / WAVE - 1];
#pragma unroll
            for (int q = 0; q < NT / WAVE - 1; ++q) {
                const int w2 = q < wv ? q : q + 1;
                lst[q] = tt.lmax + w2 * WAVE;
                ge[q] = w2 < wv;
                pos[q] = 0;
            }
#pragma unroll
            for (int b = 5; b >= 0; --b) {
                float x[NT / WAVE - 1];
#pragma unroll
                for (int q = 0; q < NT / WAVE - 1; ++q) x[q] = lst[q][pos[q] + (1 << b) - 1];
#pragma unroll
                for (int q = 0; q < NT / WAVE - 1; ++q)
                    pos[q] += (x[q] > srt || (ge[q] && x[q] == srt)) ? (1 << b) : 0;
            }
            int rank = lane;
#pragma unroll
            for (int q = 0; q < NT / WAVE - 1; ++q) {
                const float x = lst[q][pos[q]];
                rank += pos[q] + ((x > srt || (ge[q] && x == srt)) ? 1 : 0);
            }
            tt.sorted[rank] = srt;
        }
        __syncthreads();
        const float m = tt.sorted[0];
        // first threshold try and the softmax partial sum in one exchange
        const int step = max(1, cap / 8);
        int L = cap - step;
        const bool cut = nf > cap;
        float theta = cut ? tt.sorted[L] : NEG_INF;
        int mine = 0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) mine += v[s] > theta;
        int cnt = mine;
        double ssum = 0.0;
        // The tile sum only feeds the row's normaliser, which a top-k cut makes
        // unused: a tile with more than k finite entries proves the cut.
        const bool need_s = !(c.top_k > 0 && c.top_k < c.V && nf > c.top_k);
        if (need_s && m > NEG_INF) {
            // raw v_exp_f32: terms below 2^-126 flush to zero, which cannot move
            // a sum whose largest term is 1
            const float c2 = 1.4426950408889634f / c.T;
            float acc = 0.0f;
#pragma unroll
            for (int s = 0; s < EPT; ++s) acc += __builtin_amdgcn_exp2f((v[s] - m) * c2);
            ssum = acc;
        }
        cnt = wave_sum_i(cnt);
        ssum = wave_sum_d(ssum);
        if (lane == 0) {
            sh.red2.i[wv] = cnt;
            sh.red2.d[wv] = ssum;
        }
        __syncthreads();
        cnt = sh.red2.i[0] + sh.red2.i[1] + sh.red2.i[2] + sh.red2.i[3];
        const int* wcnt = sh.red2.i;  // per-wave candidate counts of the final threshold
        ssum = ((sh.red2.d[0] + sh.red2.d[1]) + sh.red2.d[2]) + sh.red2.d[3];
        // lower the threshold until the candidates fit (L = 0 puts it at the
        // tile maximum: no candidates)
        while (cnt > cap) {
            L = L > step ? L - step : 0;
            theta = tt.sorted[L];
            mine = 0;
#pragma unroll
            for (int s = 0; s < EPT; ++s) mine += v[s] > theta;
            cnt = block_sum_i(mine, sh.red);
            wcnt = sh.red.i;
        }
        // candidates (x', id) into LDS: each wave's slice starts after the
        // earlier waves' counts; within it, slot by slot, lanes in order (a
        // ballot per slot, skipped when no lane of the wave has a candidate)
        int base = 0;
#pragma unroll
        for (int w = 0; w < NT / WAVE - 1; ++w) base += w < wv ? wcnt[w] : 0;
        base = __builtin_amdgcn_readfirstlane(base);
        if (__builtin_amdgcn_readfirstlane(wcnt[wv]) > 0) {
#pragma unroll
            for (int s = 0; s < EPT; ++s) {
                const bool hit = v[s] > theta;
                const unsigned long long bm = __ballot(hit);
                if (bm) {
                    if (hit)
                        tt.list[base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u))] =
                            ((unsigned long long)__float_as_uint(v[s]) << 32) | (uint32_t)slot_id<DT>(tb, s);
                    base += __popcll(bm);
                }
            }
        }
        __syncthreads();
        // one key (z = x'/T, id) per thread of the waves holding candidates
        // (0, below every key, past cnt); each such wave sorts its keys in
        // registers, and with more than 64 candidates every key also counts the
        // larger keys of the other wave's sorted list: the list goes out sorted
        unsigned long long* cand = ws.cand + ((size_t)row * ws.n_tiles + tile) * CW;
        const int nw = (cnt + WAVE - 1) / WAVE;  // at most CW / WAVE = 2
        unsigned long long my = 0;
        if (wv < nw) {
            if (tid < cnt) {
                const unsigned long long e = tt.list[tid];
                my = key64(canon_zero(__uint_as_float((uint32_t)(e >> 32)) / c.T), (int)(uint32_t)e);
            }
            my = wave_sort_desc_u64(my);
            if (nw > 1) tt.keys[tid] = my;
        }
        if (nw > 1) __syncthreads();
        if (wv < nw) {
            int r = lane;
            if (nw > 1) {
                const unsigned long long* other = tt.keys + (wv ^ 1) * WAVE;
                int pos = 0;
#pragma unroll
                for (int b = 5; b >= 0; --b) pos += other[pos + (1 << b) - 1] > my ? (1 << b) : 0;
                r += pos + (other[pos] > my ? 1 : 0);
            }
            if (my != 0) cand[r] = my;
        }
        st.m = m;
        st.argmax = -1;
        st.s = ssum;
        st.beta = theta;
        st.ncand = cnt;
        st.nfinite = nf;
    }
    if (tid == 0) ws.stats[(size_t)row * ws.n_tiles + tile] = st;
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

// Lane t of every wave holds tile t's summary (the others an empty one); each
// wave reduces them identically, so no exchange between waves is needed.
__device__ __forceinline__ TileStat load_tile_stat(const Workspace& ws, int row) {
    const int lane = threadIdx.x & (WAVE - 1);
    TileStat t;
    if (lane < ws.n_tiles) {
        t = ws.stats[(size_t)row * ws.n_tiles + lane];
    } else {
        t.m = NEG_INF;
        t.argmax = INT_MAX;
        t.s = 0.0;
        t.beta = NEG_INF;
        t.ncand = 0;
        t.nfinite = 0;
        t.pad = 0;
    }
    return t;
}

// The row's maximum, finite count and highest incomplete-tile threshold. Every
// wave of the merge needs these before the pool is laid out; the argmax (greedy
// rows) and the row mass (rows not cut by top-k) are formed only where needed.
__device__ __forceinline__ RowSummary summarize_tiles(const TileStat t) {
    RowSummary r;
    r.m = wave_max(t.m);
    r.nfinite = wave_sum_i(t.nfinite);
    const bool incomplete = t.ncand < t.nfinite;
    r.beta = wave_max(incomplete ? t.beta : NEG_INF);
    r.argmax = -1;
    r.W = 0.0;
    return r;
}

__device__ __forceinline__ int row_argmax(const TileStat t, float m) {
    return wave_min_i((t.m == m && t.argmax >= 0) ? t.argmax : INT_MAX);
}

// Σ exp((x' - m) / T) over the row from the tiles' partial sums.
__device__ __forceinline__ double row_mass(const TileStat t, float m, float T) {
    double s = 0.0;
    if (T > 0.0f && t.m > NEG_INF && m > NEG_INF) {
        const float c2 = 1.4426950408889634f / T;
        s = t.s * (double)exp2f((t.m - m) * c2);
    }
    return wave_sum_d(s);
}

__device__ __forceinline__ uint64_t wq(float w) { return (uint64_t)((double)w * MASS_SCALE); }

// Radix selection over the row's z (scratch), 8 passes of 8-bit digits on key64.
// by_mass = false: the key of the rank-`target` element (1-based) in key order.
// by_mass = true: the key of the first element whose inclusive mass exceeds
// `target` (fixed point); the smallest key if none does.
template <class Pred>
__device__ unsigned long long radix_select(const float* zr, int V, float zmax, Pred pred,
                                           bool by_mass, unsigned long long target, SmemRadix& h,
                                           SmemR& sh) {
    const int tid = threadIdx.x;
    unsigned long long prefix = 0, pmask = 0, rem = target;
    int take_last = 0;
    for (int d = 7; d >= 0; --d) {
        for (int b = tid; b < 256; b += NTR) {
            h.hc[b] = 0;
            h.hm[b] = 0;
        }
        __syncthreads();
        const int sft = d * 8;
        for (int v = tid; v < V; v += NTR) {
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
                               unsigned long long& mass, SmemR& sh) {
    int cnt = 0;
    unsigned long long ms = 0;
    for (int v = threadIdx.x; v < V; v += NTR) {
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
    __shared__ unsigned long long part[NTR / WAVE];
    if ((threadIdx.x & (WAVE - 1)) == 0) part[threadIdx.x / WAVE] = ms;
    __syncthreads();
    unsigned long long t = 0;
#pragma unroll
    for (int k = 0; k < NTR / WAVE; ++k) t += part[k];
    __syncthreads();
    mass = t;
}

// Exact whole-row resolution: recompute z for the whole row into scratch (the
// first NT threads, one tile at a time), then select by count (top-k) and by
// mass (top-p, the draw) with radix passes over the whole workgroup.
template <int DT>
__device__ __forceinline__ void finalize_slow(const RowCtx& c, int row, const Workspace& ws,
                                           int n_tiles, const RowSummary& rs, float u, SmemU& su,
                                           SmemR& sh, RowInfo& info, const RowDbg& dbg) {
    const int tid = threadIdx.x;
    const int V = c.V;
    const bool tl = tid < NT;
    float* zr = ws.scratch_z + (size_t)row * V;
    const bool tables = c.hist_len + c.extra_len + c.bias_len > 0;
    TablePrefetch f = {{-1, -1}, -1, -1, 0.0f};
    if (tables && tl) f = prefetch_tables(c);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        float v[EPT];
        uint32_t mw[Lay<DT>::NG];
        if (tl) {
            load_tile<DT>(c, t * TILE, v);
            load_mask<DT>(c, t * TILE, mw);
        }
        if (tables) build_tables(c, t * TILE, su.t, f, tl);
        if (tl) {
            process_tile<DT>(c, t * TILE, v, su.t, mw);
#pragma unroll
            for (int s = 0; s < EPT; ++s) {
                const int id = slot_id<DT>(t * TILE, s);
                if (id < V) zr[id] = v[s] > NEG_INF ? canon_zero(v[s] / c.T) : NEG_INF;
            }
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
        for (int v = tid; v < V; v += NTR) {
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
        for (int v0 = 0; v0 < V; v0 += NTR) {
            const int v = v0 + tid;
            bool fl = false;
            if (topk_on && v < V) {
                const float z = zr[v];
                fl = z > NEG_INF && key64(z, v) >= kK;
            }
            int tot;
            const int off = block_excl_scan_i(fl ? 1 : 0, sh.red, tot);
            if (fl && base + off < dbg.topk_stride) dbg.topk[base + off] = v;
            base += tot;
        }
        for (int i = (topk_on ? min(base, dbg.topk_stride) : 0) + tid; i < dbg.topk_stride; i += NTR)
            dbg.topk[i] = -1;
    }
    if (tid == 0) {
        if (dbg.kept) *dbg.kept = n_kept;
        if (dbg.path) *dbg.path = 1;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// the sorted pool

__device__ __forceinline__ float key_z(unsigned long long k) {
    const uint32_t m = (uint32_t)(k >> 32);
    return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// What the merge reads from stage 1: the row's candidate slots and the tile
// summaries (lane t holds tile t). Issued before anything else so the row's
// loads share one round trip.
struct RowLoad {
    unsigned long long cv[PERR];
    TileStat ts;
};

__device__ __forceinline__ RowLoad row_load(const Workspace& ws, int row) {
    RowLoad l;
    const int n_tiles = ws.n_tiles;
    const unsigned long long* cand = ws.cand + (size_t)row * n_tiles * CW;
#pragma unroll
    for (int k = 0; k < PERR; ++k) {
        const int g = (int)threadIdx.x + k * NTR;
        l.cv[k] = g < n_tiles * CW ? gld(cand + g) : 0ull;
    }
    l.ts = load_tile_stat(ws, row);
    return l;
}

// One merge level over slots tid + r NTR, r < R (slot layout, segments of C
// slots padded with zero keys): each kept entry moves to its index plus the
// number of partner entries before it, each empty slot to the tail of its
// merged segment. The R searches advance together so their LDS reads overlap.
template <int R>
__device__ __forceinline__ void merge_level(const unsigned long long* in, unsigned long long* out,
                                            const int* len, int C, int lg, int nslots) {
    const int tid = threadIdx.x;
    unsigned long long key[R];
    int pos[R], pb[R], ob[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int g = tid + r * NTR;
        const int gg = g < nslots ? g : 0;
        key[r] = in[gg];
        const int sg = gg >> lg;
        const int i = gg & (C - 1);
        const int lo = len[sg];
        const int le = len[sg & ~1], lr = len[sg | 1];
        pb[r] = (sg ^ 1) * C;
        pos[r] = 0;
        if (g >= nslots) ob[r] = -1;
        else if (i < lo) ob[r] = (sg & ~1) * C + i;  // plus the partner count
        else ob[r] = -2 - ((sg & ~1) * C + le + lr + ((sg & 1) ? (C - le) : 0) + (i - lo));
    }
    const lds_key_ptr lin = (lds_key_ptr)in;
    lds_key_ptr sp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sp[r] = lin + pb[r];
    bool kept = false;
#pragma unroll
    for (int r = 0; r < R; ++r) kept |= ob[r] >= 0;
    if (__ballot(kept)) {  // waves holding only empty slots skip the searches
#pragma unroll
        for (int bit = MERGE_LG_MAX - 1; bit >= 0; --bit) {
            if (bit >= lg) continue;
            unsigned long long x[R];
#pragma unroll
            for (int r = 0; r < R; ++r) x[r] = sp[r][(1 << bit) - 1];
#pragma unroll
            for (int r = 0; r < R; ++r) sp[r] += x[r] > key[r] ? (1 << bit) : 0;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) pos[r] = (int)(sp[r] - (lin + pb[r])) + (sp[r][0] > key[r] ? 1 : 0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (ob[r] >= 0) out[ob[r] + pos[r]] = key[r];
        else if (ob[r] <= -2) out[-2 - ob[r]] = 0ull;
    }
}

// A four-way merge level: each group of four segments of C = 2^lg slots becomes
// one segment of 4C. A kept entry moves to its index plus, for each of its three
// partner segments, the number of partner entries before it (binary searches
// over the padded partners, all 3R in lockstep); empty slots fill the group's
// tail in segment order. Half the levels of pairwise merging, so half the chain
// of dependent LDS reads.
template <int R>
__device__ __forceinline__ void merge_level4(const unsigned long long* in, unsigned long long* out,
                                             const int* len, int C, int lg, int nslots) {
    const int tid = threadIdx.x;
    unsigned long long key[R];
    int pos[R][3], pb[R][3], ob[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int g = tid + r * NTR;
        const int gg = g < nslots ? g : 0;
        key[r] = in[gg];
        const int sg = gg >> lg;
        const int q = sg & 3, g0 = sg & ~3;
        const int i = gg & (C - 1);
        const int lo = len[sg];
        int tot = 0, before = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int lp = len[g0 + p];
            tot += lp;
            before += p < q ? C - lp : 0;
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            pb[r][k] = (g0 + k + (k >= q ? 1 : 0)) << lg;
            pos[r][k] = 0;
        }
        if (g >= nslots) ob[r] = -1;
        else if (i < lo) ob[r] = (g0 << lg) + i;  // plus the partner counts
        else ob[r] = -2 - ((g0 << lg) + tot + before + (i - lo));
    }
    // kept entries sit at the front of each segment, so whole waves of slots
    // are often empty: their searches are skipped (a wave-uniform branch)
    // each search walks a pointer into its partner; the probe distance of a
    // step is a constant, so it rides in the LDS instruction's offset field
    const lds_key_ptr lin = (lds_key_ptr)in;
    lds_key_ptr sp[R][3];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < 3; ++k) sp[r][k] = lin + pb[r][k];
    bool kept = false;
#pragma unroll
    for (int r = 0; r < R; ++r) kept |= ob[r] >= 0;
    if (__ballot(kept)) {  // waves holding only empty slots skip the searches
#pragma unroll
        for (int bit = MERGE_LG_MAX - 1; bit >= 0; --bit) {
            if (bit >= lg) continue;
            unsigned long long x[R][3];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < 3; ++k) x[r][k] = sp[r][k][(1 << bit) - 1];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int k = 0; k < 3; ++k) sp[r][k] += x[r][k] > key[r] ? (1 << bit) : 0;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < 3; ++k)
                pos[r][k] = (int)(sp[r][k] - (lin + pb[r][k])) + (sp[r][k][0] > key[r] ? 1 : 0);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (ob[r] >= 0) out[ob[r] + pos[r][0] + pos[r][1] + pos[r][2]] = key[r];
        else if (ob[r] <= -2) out[-2 - ob[r]] = 0ull;
    }
}

// Outcome of resolving a row on its sorted pool.
struct RowOut {
    unsigned long long kappa;
    double Wk;
    int n_kept;
    int token;
    int lim_list;
    int slow;
};

// One wave answers top-k mass, top-p, min-p and the draw on the sorted pool
// F[0, n), 64 entries per step: entry i's weight w_i = exp(z_i - zmax) (binary32,
// as everywhere on this path), masses in binary64 with a running carry.
// slow = 1 when a request reaches past the pool.
__device__ __forceinline__ RowOut resolve_wave(const unsigned long long* F, int n, float zmax, const RowSummary& rs,
                               const RowCtx& c, float u, int K_eff, bool cut_k, int total,
                               bool topk_on, bool want_probs, bool want_topk, double WK_block) {
    const int lane = threadIdx.x & (WAVE - 1);
    RowOut o;
    o.slow = 0;
    o.kappa = 0;
    o.Wk = rs.W;
    o.n_kept = 0;
    o.token = -1;
    o.lim_list = cut_k ? K_eff : (topk_on ? total : 0);
    auto wat = [&](int i, int lim) -> float {
        return i < lim ? expf(key_z(F[i]) - zmax) : 0.0f;
    };
    // mass of the top-k set (summed by the whole workgroup when it spans more
    // than one chunk)
    double WK = rs.W;
    unsigned long long kK = 0;
    if (cut_k) {
        if (K_eff > WAVE) {
            WK = WK_block;
        } else {
            WK = wave_sum_d((double)wat(lane, K_eff));
        }
        kK = F[K_eff - 1];
    }
    // top-p (first entry whose exclusive mass reaches top_p W_K) and min-p
    // (first entry with w < min_p), scanned together
    const int lim_p = cut_k ? K_eff : total;
    const bool use_p = c.top_p < 1.0f, use_m = c.min_p > 0.0f;
    const double thr = (double)c.top_p * WK;
    const int end_p = min(n, lim_p);
    int fp = INT_MAX, fm = INT_MAX;
    {
        double carry = 0.0;
        for (int c0 = 0;; c0 += WAVE) {
            const bool need_p = use_p && fp == INT_MAX && c0 < end_p;
            const int n_topp_now = fp != INT_MAX ? fp : lim_p;
            const bool need_m = use_m && fm == INT_MAX && c0 < min(n, n_topp_now);
            if (!need_p && !need_m) break;
            const int i = c0 + lane;
            const float w = wat(i, n);
            const double in = wave_incl_scan_d((double)w);
            const double excl = carry + (in - (double)w);
            if (need_p) {
                const unsigned long long m = __ballot(i < end_p && excl >= thr);
                if (m) fp = c0 + __ffsll((long long)m) - 1;
            }
            if (need_m) {
                const unsigned long long m = __ballot(i < n && w < c.min_p);
                if (m) fm = c0 + __ffsll((long long)m) - 1;
            }
            carry += __shfl(in, WAVE - 1);
        }
    }
    int n_topp = lim_p;
    if (use_p) {
        if (fp != INT_MAX) n_topp = fp;
        else if (lim_p > n) o.slow = 1;
    }
    int n_kept = n_topp;
    if (!o.slow && use_m) {
        if (fm < n_topp) n_kept = fm;
        else if (fm == INT_MAX && n_topp > n) o.slow = 1;
    }
    if (o.slow) return o;
    // kept mass and the cut key
    double Wk;
    unsigned long long kappa;
    if (n_kept == total) {
        Wk = rs.W;
        kappa = 0;
    } else if (cut_k && n_kept == K_eff) {
        Wk = WK;
        kappa = kK;
    } else {
        double carry = 0.0;
        for (int c0 = 0; c0 < n_kept; c0 += WAVE) carry += wave_sum_d((double)wat(c0 + lane, n_kept));
        Wk = carry;
        kappa = F[n_kept - 1];
    }
    // the draw: first kept entry whose inclusive mass exceeds u Wk
    const double tgt = (double)u * Wk;
    const int lim = min(n, n_kept);
    int fd = INT_MAX;
    {
        double carry = 0.0;
        for (int c0 = 0; c0 < lim && fd == INT_MAX; c0 += WAVE) {
            const int i = c0 + lane;
            const double in = carry + wave_incl_scan_d((double)wat(i, lim));
            const unsigned long long m = __ballot(i < lim && in > tgt);
            if (m) fd = c0 + __ffsll((long long)m) - 1;
            carry = __shfl(in, WAVE - 1);
        }
    }
    const int pick = fd != INT_MAX ? fd : (n_kept <= n ? n_kept - 1 : -1);
    if (pick < 0 || (want_probs && n_kept > n) || (want_topk && o.lim_list > n)) {
        o.slow = 1;
        return o;
    }
    o.kappa = kappa;
    o.Wk = Wk;
    o.n_kept = n_kept;
    o.token = key64_id(F[pick]);
    return o;
}

template <int DT>
__device__ __forceinline__ void finalize_row(const RowCtx& c, int row, const Workspace& ws,
                                             const RowLoad& rl, SmemU& su, SmemR& sh,
                                             const RowDbg& dbg, RowInfo& info_out) {
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int n_tiles = ws.n_tiles;
    const int V = c.V;
    SmemPool& P = su.p;
    const TileStat ts = rl.ts;
    RowSummary rs = summarize_tiles(ts);

    __shared__ RowInfo info;
    if (c.T == 0.0f || !(rs.m > NEG_INF)) {
        rs.argmax = row_argmax(ts, rs.m);
        RowInfo r;
        r.kappa = 0;
        r.W = 1.0;
        r.zmax = rs.m;
        r.min_p = 0.0f;
        r.n_kept = rs.m > NEG_INF ? 1 : 0;
        r.token = rs.m > NEG_INF ? rs.argmax : -1;
        r.argmax = r.token;
        r.path = 0;
        if (dbg.topk)
            for (int i = tid; i < dbg.topk_stride; i += NTR) dbg.topk[i] = -1;
        if (tid == 0) {
            if (dbg.probs && r.token >= 0) dbg.probs[r.token] = 1.0f;
            if (dbg.kept) *dbg.kept = r.n_kept;
            if (dbg.path) *dbg.path = 0;
        }
        info_out = r;
        return;
    }
    // The pool: every entry with z above the highest tile threshold. It is a
    // prefix of each tile's sorted list and, as a whole, an exact prefix of the
    // row in key order. Slot layout: tile t owns slots [t CW, (t + 1) CW), its
    // kept entries first and zero keys after them, up to a power-of-two number
    // of tiles, so every merge segment is padded with keys that precede none.
    const float zmax = canon_zero(rs.m / c.T);
    const float zb = rs.beta > NEG_INF ? canon_zero(rs.beta / c.T) : NEG_INF;
    const uint32_t mzb = mono32(zb);
    int npad = 1;
    while (npad < n_tiles) npad *= 2;
    // slots per tile: the row's candidate cap rounded up to a power of two
    int sw = 8;
    while (sw < row_cap(c)) sw *= 2;
    int lsw = 3;
    while ((1 << lsw) < sw) ++lsw;
    const int nslots = npad * sw;
    const int oct = __builtin_amdgcn_readfirstlane(tid / CW);
#pragma unroll
    for (int k = 0; k < PERR; ++k) {
        const int g = tid + k * NTR;
        const int t = OCT * k + oct;  // tile of candidate slot g
        const int i = g % CW;
        bool keep = false;
        if (t < n_tiles) {
            const int nc = __builtin_amdgcn_readlane(ts.ncand, t);
            keep = i < nc && (uint32_t)(rl.cv[k] >> 32) > mzb;
        }
        if (t < npad && i < sw) P.buf[0][t * sw + i] = keep ? rl.cv[k] : 0ull;
        const int wc = __popcll(__ballot(keep));
        if (lane == 0) P.wcnt[k][wv] = wc;
    }
    __syncthreads();
    if (tid < MAX_TILES) {
        const int t = tid;
        const int k = t / OCT, o = t % OCT;
        P.len[0][t] = t < n_tiles ? P.wcnt[k][2 * o] + P.wcnt[k][2 * o + 1] : 0;
    }
    __syncthreads();
    // Merge tree: level l merges segments of 2^l tiles. An entry's output
    // position is its index in its segment plus the number of partner entries
    // that precede it (binary search over the padded partner segment); empty
    // slots fill the tail of each merged segment with zero keys.
    // Four-way levels while a group of four segments exists in the padded
    // layout, then at most one pairwise level.
    int src = 0;
    for (int seg_tiles = 1, lg = lsw; seg_tiles < n_tiles;) {
        const int C = seg_tiles * sw;
        const unsigned long long* in = P.buf[src];
        unsigned long long* out = P.buf[src ^ 1];
        const int* len = P.len[src];
        const bool four = seg_tiles * 4 <= npad;
        if (four) {
            if (nslots <= NTR)
                merge_level4<1>(in, out, len, C, lg, nslots);
            else if (nslots <= 2 * NTR)
                merge_level4<2>(in, out, len, C, lg, nslots);
            else
                merge_level4<PERR>(in, out, len, C, lg, nslots);
        } else {
            if (nslots <= NTR)
                merge_level<1>(in, out, len, C, lg, nslots);
            else if (nslots <= 2 * NTR)
                merge_level<2>(in, out, len, C, lg, nslots);
            else
                merge_level<PERR>(in, out, len, C, lg, nslots);
        }
        if (tid < MAX_TILES) {
            const int j = tid;
            if (four)
                P.len[src ^ 1][j] = 4 * j + 3 < MAX_TILES
                                        ? (len[4 * j] + len[4 * j + 1]) + (len[4 * j + 2] + len[4 * j + 3])
                                        : 0;
            else
                P.len[src ^ 1][j] = 2 * j + 1 < MAX_TILES ? len[2 * j] + len[2 * j + 1] : 0;
        }
        __syncthreads();
        src ^= 1;
        seg_tiles *= four ? 4 : 2;
        lg += four ? 2 : 1;
    }
    const int n = P.len[src][0];
    const unsigned long long* F = P.buf[src];

    const int total = rs.nfinite;
    const bool topk_on = c.top_k > 0 && c.top_k < V;
    const int K_eff = topk_on ? min(c.top_k, total) : total;
    const bool cut_k = topk_on && K_eff < total;
    bool slow = n == 0 || (cut_k && K_eff > n);
    if (!slow) {
        // Wave 0 resolves the row on the sorted pool, 64 entries at a time with
        // a running binary64 carry (every cut is a prefix question, and on
        // low-entropy rows all of them fall in the first chunk or two); the
        // rest of the workgroup waits at one barrier.
        __shared__ RowOut s_out;
        double WK_block = 0.0;
        if (cut_k && K_eff > WAVE) {
            double part = 0.0;
            for (int i = tid; i < K_eff; i += NTR) part += (double)expf(key_z(F[i]) - zmax);
            WK_block = block_sum_d(part, sh.red);
        }
        if (wv == 0) {
            // the draw's uniform and the row mass, in the resolving wave only
            const float u = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_SAMPLE));
            RowSummary rw = rs;
            if (!cut_k) rw.W = row_mass(ts, rs.m, c.T);
            const RowOut o = resolve_wave(F, n, zmax, rw, c, u, K_eff, cut_k, total, topk_on,
                                          dbg.probs != nullptr, dbg.topk != nullptr, WK_block);
            if (lane == 0) s_out = o;
        }
        __syncthreads();
        const RowOut o = s_out;
        if (!o.slow) {
            RowInfo r;
            r.kappa = o.kappa;
            r.W = o.Wk;
            r.zmax = zmax;
            r.min_p = 0.0f;
            r.n_kept = o.n_kept;
            r.token = o.token;
            r.argmax = -1;
            r.path = 0;
            if (tid == 0) {
                if (dbg.kept) *dbg.kept = o.n_kept;
                if (dbg.path) *dbg.path = 0;
            }
            if (dbg.probs)
                for (int i = tid; i < o.n_kept; i += NTR)
                    dbg.probs[key64_id(F[i])] = (float)((double)expf(key_z(F[i]) - zmax) / o.Wk);
            if (dbg.topk)
                for (int i = tid; i < dbg.topk_stride; i += NTR)
                    dbg.topk[i] = i < o.lim_list ? key64_id(F[i]) : -1;
            info_out = r;
            return;
        }
    }
    const float u = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_SAMPLE));
    finalize_slow<DT>(c, row, ws, n_tiles, rs, u, su, sh, info, dbg);
    __syncthreads();
    info_out = info;
}

// ---------------------------------------------------------------------------
// kernels
//
// Each pass is a short chain of launches on one stream: the kernel boundary is
// the only synchronisation between stages (no cross-workgroup fences or
// counters), and each kernel carries only the registers and LDS of its stage.

// Workgroup i runs on XCD i mod 8. Stage 1 and the row merge both map their
// linear index so that a row's tiles and its merge land on the same XCD, which
// keeps the merge's reads of the stage-1 results in that XCD's L2.
__device__ __forceinline__ int xcd_linear(int n) {
    const int i = blockIdx.x;
    if ((n & 7) != 0) return i;
    return (i & 7) * (n >> 3) + (i >> 3);
}

template <int DT>
__device__ __forceinline__ RowCtx sample_ctx(const SampleArgs& a, int row) {
    const void* logits = (const char*)a.logits + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    return make_ctx(a.p, row, logits, a.V, nullptr, 0, mrow, 0);
}

// Target row j of request b is scored after the draft tokens d_0..d_{j-1}: they
// extend the penalty history and the position.
template <int DT>
__device__ __forceinline__ RowCtx spec_ctx(const SpecArgs& a, int b, int j) {
    const int row = b * (a.G + 1) + j;
    const void* logits = (const char*)a.target + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    return make_ctx(a.p, b, logits, a.V, a.draft_tokens + (size_t)b * a.G, j, mrow, (uint32_t)j);
}

// Tile kernels: seven 256-thread workgroups per CU fit the LDS (about 23 KB
// each); the register budget is held to the same seven waves per SIMD.
#define SS_TILE_OCC __attribute__((amdgpu_waves_per_eu(7)))

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_sample_tiles(SampleArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int lin = xcd_linear(a.B * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const RowCtx c = sample_ctx<DT>(a, row);
    tile_stage1<DT, ALIGNED>(c, row, tile, a.ws, tt, sh,
                    a.dbg_processed ? a.dbg_processed + (size_t)row * a.V : nullptr,
                    a.dbg_probs ? a.dbg_probs + (size_t)row * a.V : nullptr);
}

template <int DT>
__global__ __launch_bounds__(NTR) void k_sample_rows(SampleArgs a) {
    __shared__ SmemU su;
    __shared__ SmemR sh;
    const int row = xcd_linear(a.B);
    const RowLoad rl = row_load(a.ws, row);
    const RowCtx c = sample_ctx<DT>(a, row);
    RowDbg dbg;
    dbg.topk = a.dbg_topk ? a.dbg_topk + (size_t)row * a.dbg_topk_stride : nullptr;
    dbg.topk_stride = a.dbg_topk_stride;
    dbg.kept = a.dbg_kept ? a.dbg_kept + row : nullptr;
    dbg.probs = a.dbg_probs ? a.dbg_probs + (size_t)row * a.V : nullptr;
    dbg.path = a.dbg_path ? a.dbg_path + row : nullptr;
    RowInfo info;
    finalize_row<DT>(c, row, a.ws, rl, su, sh, dbg, info);
    if (threadIdx.x == 0) a.out_tokens[row] = info.token;
}

// Verification, stage 1 over every target row of every request.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(NT) void k_spec_tiles(SpecArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int G1 = a.G + 1;
    const int lin = xcd_linear(a.B * G1 * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const RowCtx c = spec_ctx<DT>(a, row / G1, row % G1);
    tile_stage1<DT, ALIGNED>(c, row, tile, a.ws, tt, sh, nullptr, nullptr);
}

// Verification, per target row: the filtered distribution, then the accept
// test of the draft token at that position (draft rows) or the bonus token
// (last row).
template <int DT>
__global__ __launch_bounds__(NTR) void k_spec_rows(SpecArgs a) {
    __shared__ SmemU su;
    __shared__ SmemR sh;
    const int G1 = a.G + 1;
    const int row = xcd_linear(a.B * G1);
    const int b = row / G1;
    const int j = row % G1;
    const RowLoad rl = row_load(a.ws, row);
    const RowCtx c = spec_ctx<DT>(a, b, j);
    RowDbg dbg = {nullptr, 0, nullptr, nullptr, nullptr};
    RowInfo info;
    finalize_row<DT>(c, row, a.ws, rl, su, sh, dbg, info);
    if (j < a.G) {
        const int d = a.draft_tokens[(size_t)b * a.G + j];
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
}

// Accepted draft count of request b: the first rejected position, or G.
__device__ __forceinline__ int accepted_prefix(const SpecArgs& a, int b) {
    const int G1 = a.G + 1;
    int n = a.G;
    for (int k = a.G - 1; k >= 0; --k)
        if (!a.ws.row_accept[(size_t)b * G1 + k]) n = k;
    return n;
}

// Position of request b whose token comes from the residual distribution, or -1.
__device__ __forceinline__ int residual_position(const SpecArgs& a, int b, RowInfo& ri) {
    const int n = accepted_prefix(a, b);
    ri = a.ws.rowinfo[(size_t)b * (a.G + 1) + n];
    if (n == a.G || a.p.temperature[b] == 0.0f || ri.n_kept == 0) return -1;
    return n;
}

// pi(v) of the filtered distribution described by ri, for processed logit x.
__device__ __forceinline__ float filtered_prob(const RowCtx& c, const RowInfo& ri, int id, float x) {
    if (!(x > NEG_INF)) return 0.0f;
    const float z = canon_zero(x / c.T);
    const float w = expf(z - ri.zmax);
    const bool kept = key64(z, id) >= ri.kappa && (ri.min_p <= 0.0f || w >= ri.min_p);
    return kept ? (float)((double)w / ri.W) : 0.0f;
}

// Residual mass of one tile of a rejected row: r = max(0, pi - q) per entry (or
// pi itself when use_pi), in token-id order within each thread group.
template <int DT>
__device__ void residual_values(const RowCtx& c, const RowInfo& ri, const float* q, int tb,
                                bool use_pi, SmemTile& tt, double r[EPT]) {
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    const TablePrefetch f = prefetch_tables(c);
    load_tile<DT>(c, tb, v);
    load_mask<DT>(c, tb, mw);
    if (c.hist_len + c.extra_len + c.bias_len > 0) build_tables(c, tb, tt, f);
    process_tile<DT>(c, tb, v, tt, mw);
#pragma unroll
    for (int s = 0; s < EPT; ++s) {
        const int id = slot_id<DT>(tb, s);
        double val = 0.0;
        if (id < c.V) {
            const float pi = filtered_prob(c, ri, id, v[s]);
            val = use_pi ? (double)pi : (double)fmaxf(0.0f, pi - gld(q + id));
        }
        r[s] = val;
    }
}

// Verification, residual stage 1: per tile of each rejected row, the sums of the
// residual max(0, pi - q) and of pi (the fallback when the residual is zero).
template <int DT>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_spec_resid_tiles(SpecArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    const int n_tiles = a.ws.n_tiles;
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x % n_tiles;
    RowInfo ri;
    const int j = residual_position(a, b, ri);
    if (j < 0) return;
    const RowCtx c = spec_ctx<DT>(a, b, j);
    const float* q = a.draft_probs + ((size_t)b * a.G + j) * a.draft_stride;
    const int tb = tile * TILE;
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    const TablePrefetch f = prefetch_tables(c);
    load_tile<DT>(c, tb, v);
    load_mask<DT>(c, tb, mw);
    if (c.hist_len + c.extra_len + c.bias_len > 0) build_tables(c, tb, tt, f);
    process_tile<DT>(c, tb, v, tt, mw);
    double sr = 0.0, sp = 0.0;
#pragma unroll
    for (int s = 0; s < EPT; ++s) {
        const int id = slot_id<DT>(tb, s);
        if (id < c.V) {
            const float pi = filtered_prob(c, ri, id, v[s]);
            sr += (double)fmaxf(0.0f, pi - gld(q + id));
            sp += (double)pi;
        }
    }
    sr = block_sum_d(sr, sh.red);
    sp = block_sum_d(sp, sh.red);
    if (threadIdx.x == 0) a.ws.resid_tile[(size_t)b * n_tiles + tile] = make_double2(sr, sp);
}

// Verification, per request: the output row. Accepted drafts, then the bonus
// token, the greedy target token, or a draw from the residual distribution in
// token-id order (tile by the per-tile sums, then the entry within the tile).
template <int DT>
__global__ __launch_bounds__(NT) void k_spec_finish(SpecArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    __shared__ int s_tile;
    __shared__ int s_usepi;
    __shared__ double s_rem;
    const int n_tiles = a.ws.n_tiles;
    const int b = blockIdx.x;
    const int G1 = a.G + 1;
    const int n = accepted_prefix(a, b);
    RowInfo ri;
    const int j = residual_position(a, b, ri);
    int32_t* out = a.out_tokens + (size_t)b * G1;
    if (threadIdx.x == 0) {
        for (int k = 0; k < n; ++k) out[k] = a.draft_tokens[(size_t)b * a.G + k];
        for (int k = n + 1; k < G1; ++k) out[k] = -1;
        a.out_num_accepted[b] = n;
        if (j < 0) out[n] = n == a.G ? ri.token : ri.argmax;
    }
    if (j < 0) return;
    const RowCtx c = spec_ctx<DT>(a, b, j);
    const float* q = a.draft_probs + ((size_t)b * a.G + j) * a.draft_stride;
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
        double r[EPT];
        residual_values<DT>(c, ri, q, st * TILE, s_usepi != 0, tt, r);
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
    if (threadIdx.x == 0) out[j] = token;
}

// ---------------------------------------------------------------------------
// launchers

// Every row starts 16-byte aligned and V is a whole number of 16-byte groups:
// the tile kernels then take the branch-free load.
template <int DT>
static bool rows_aligned(const void* base, int64_t row_stride, int V) {
    constexpr int VEC = DT == SS_F32 ? 4 : 8;
    return ((uintptr_t)base & 15u) == 0 && row_stride % VEC == 0 && V % VEC == 0 && V >= VEC;
}

template <int DT>
static void sample_chain(const SampleArgs& a, hipStream_t st, const LaunchEvents& le) {
    if (rows_aligned<DT>(a.logits, a.row_stride, a.V))
        launch_k(le, 0, k_sample_tiles<DT, true>, dim3(a.B * a.ws.n_tiles), dim3(NT), st, a);
    else
        launch_k(le, 0, k_sample_tiles<DT, false>, dim3(a.B * a.ws.n_tiles), dim3(NT), st, a);
    launch_k(le, 1, k_sample_rows<DT>, dim3(a.B), dim3(NTR), st, a);
}

template <int DT>
static void spec_chain(const SpecArgs& a, hipStream_t st, const LaunchEvents& le) {
    const int rows = a.B * (a.G + 1);
    if (rows_aligned<DT>(a.target, a.row_stride, a.V))
        launch_k(le, 0, k_spec_tiles<DT, true>, dim3(rows * a.ws.n_tiles), dim3(NT), st, a);
    else
        launch_k(le, 0, k_spec_tiles<DT, false>, dim3(rows * a.ws.n_tiles), dim3(NT), st, a);
    launch_k(le, 1, k_spec_rows<DT>, dim3(rows), dim3(NTR), st, a);
    launch_k(le, 2, k_spec_resid_tiles<DT>, dim3(a.B * a.ws.n_tiles), dim3(NT), st, a);
    launch_k(le, 3, k_spec_finish<DT>, dim3(a.B), dim3(NT), st, a);
}

hipError_t launch_sample(const SampleArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le) {
    if (dt == SS_F32) sample_chain<SS_F32>(a, st, le);
    else sample_chain<SS_BF16>(a, st, le);
    return hipGetLastError();
}

hipError_t launch_spec(const SpecArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le) {
    if (dt == SS_F32) spec_chain<SS_F32>(a, st, le);
    else spec_chain<SS_BF16>(a, st, le);
    return hipGetLastError();
}

}  // namespace ss

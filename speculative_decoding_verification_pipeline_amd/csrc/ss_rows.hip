// Row kernels: the fused sampler, linear and tree verification, and the row
// stage of LM-head sampling with the per-request pipeline (gfx950).
//
// The pipeline and its order follow the SonicSampler abstract (arxivdaily page,
// English abstract): per request, grammar mask, repetition / frequency /
// presence penalties, logit bias, temperature, then top-k, top-p and min-p, all
// in one batched pass, with a hierarchical two-stage top-k that exploits the
// low entropy of LLM outputs. Verification follows "Accelerating Sonar through
// speculation" (Perplexity blog, sections on speculative decoding and
// target-draft decoding).
//
// Design (MI355X-first, not a translation of the pages' Triton kernels):
//  * Stage 1: one workgroup (256 threads, 4 wave64s) per 8192-entry vocabulary
//    tile of a row; the grid is rows x tiles and depends only on (B, V), so one
//    launch serves any mix of per-request parameters and can be graph-captured.
//    The tile is streamed once with 16-byte non-temporal loads; penalties
//    (multiplicities counted in LDS while the tile is in flight), bias and the
//    packed mask are applied in registers, and only threads whose slots hold a
//    penalised or biased entry do any per-entry work.
//  * After the data lands every wave works alone on its 2048-entry share (a
//    wave tile): no workgroup barrier, only DPP / permlane reductions and
//    ballots. Its candidates are every entry whose z lies within DELTA of the
//    wave maximum when those fit 64 slots, so on low-entropy rows the wave
//    holding the row maximum keeps everything that can matter; a wave deep in
//    a steep tail that overflows modestly takes a narrower window; a flat wave
//    keeps its head by count (sorted lane maxima and a binary search of the
//    cut). Rows that top-k may leave uncut also get the mass outside the
//    candidates: exact for count-cut waves, a bounded approximation otherwise.
//  * Stage 2, one workgroup per row: the pool -- every candidate above the
//    highest wave-tile bound -- is an exact prefix of the row in key order. It
//    is sorted by a counting sort over buckets of (zmax - z), which are
//    monotone in key order, followed by a rank within each bucket; top-k,
//    top-p, min-p and the inverse-CDF draw are then wave scans over binary64
//    prefix sums. Requests that reach past the pool run an exact whole-row
//    path: z of the whole row into scratch, then each selection (top-k by
//    count, top-p and the draw by mass) as one histogram pass over buckets of
//    (zmax - z) and an exact resolve of the one bucket that holds the answer.
//    Between the two, an unfiltered row without penalty or bias lists whose
//    draw lies past its pool is drawn from binned tails: its count-cut waves
//    also bin their other entries' masses by z in stage 1, and stage 2 finds
//    the bin that holds the draw, then that bin's entries in one pass over the
//    row. Results never depend on which path resolved them.
//  * Verification reuses both stages over every target row; its residual stage
//    keeps each entry's residual with the per-tile sums so that the draw reads
//    the chosen tile's residuals. The LM-head rows left open by the GEMM's
//    tile candidates fix their kept set on one workgroup per row, then run the
//    Gumbel pass over it on the whole GPU.
#include <float.h>
#include <limits.h>

#include "ss_device.h"
#include "ss_internal.h"

#pragma clang fp contract(off)

namespace ss {

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr int NTR_MAX = 1024;  // largest workgroup of the row kernels
constexpr double MASS_SCALE = 17592186044416.0;  // 2^44 fixed-point weights in the fallback
// Widest candidate window below a wave tile's maximum, in units of z = x' / T:
// on the wave holding the row maximum it keeps every entry weighing more than
// e^-24 = 3.8e-11 of it.
constexpr float DELTA = 24.0f;
// Largest share of the top-k mass a top-k set deeper than the pool may leave
// out of its normaliser (each probability and CDF breakpoint moves by at most
// this much; the parity rule allows 1e-6).
constexpr double TAIL_EPS = 2e-7;


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

// T > 0 a (normal) power of two: then x / T is exactly x (1 / T), with no
// rounding step of its own, and a product replaces the division.
__device__ __forceinline__ bool pow2_temp(float T) {
    return (__float_as_uint(T) & 0x7FFFFFu) == 0u && T >= FLT_MIN;
}

// ---------------------------------------------------------------------------
// LDS layouts (one union per workgroup; phases are separated by barriers)

struct SmemTile {
    uint32_t cnt[TILE / 2];   // u16 history multiplicities of the tile's entries
    uint32_t xw[NT];          // per thread: bit s set when its slot s is penalised or biased
    uint32_t bw[NT];          // per thread: bit s set when its slot s is biased
    int32_t bl[NT];           // the tile's bias hits (local index, value), in no fixed order
    float bv[NT];
    int nbh;                  // bias hits appended (the list holds the first NT)
    int bfull;                // 1: some entry is biased more than once, or the list overflowed
    unsigned long long wl[WPT][WCAP];  // per wave: its candidates (x' bits, id) in slot order
};
static_assert(WPT * NBIN * sizeof(double) <= sizeof(SmemTile::cnt), "wave bins fit the tables' LDS");

// The row merge runs one 1024-thread workgroup per row (16 waves): the
// candidate loads, the pool compaction and the sort spread over all of them.
constexpr int NTR = NTR_MAX;
constexpr int NWR = NTR / WAVE;                // waves of the merge workgroup
constexpr int MSLOT = MAX_WT * WCAP / NTR;     // candidate slots per merge thread
constexpr int POOL = 4096;                     // largest pool the merge sorts
constexpr int NBK = 2048;                      // buckets of the pool's counting sort
constexpr int BKPT = NBK / NTR;                // buckets per merge thread
constexpr int BK_MAX = 1024;                   // largest bucket ranked by direct comparison

// Arrays of the sorting phase and of the resolving phase share storage: a
// barrier separates the last read of the first from the first write of the
// second.
struct SmemPool {
    unsigned long long F[POOL];       // the pool in key order
    union {
        unsigned long long bk[POOL];  // sorting: the pool in bucket order (arrival order within a bucket)
        struct {
            double P2[POOL / 2];      // resolving: second half of the inclusive prefix masses
            float w[POOL];            // resolving: weights exp(z - zmax) in key order
        };
    };
    union {
        struct {
            uint32_t cnt[NBK];        // sorting: bucket sizes
            uint32_t start[NBK];      // sorting: bucket offsets
        };
        double P[POOL / 2];           // resolving: first half of the inclusive prefix masses
    };
};
constexpr int EPTR = POOL / NTR;  // pool entries per merge thread in the prefix pass
constexpr int AREG = POOL / NWR;  // per-wave region of the unsorted pool

struct SmemRadix {
    uint32_t hc[256];
    unsigned long long hm[256];
};

// Whole-row selection by buckets of d = zmax - z: HB1 buckets of width 1/HSCALE
// over d in [0, HD1), then HB - HB1 buckets of equal width over [HD1, zmax -
// zlo] when the row's lowest finite z, zlo, lies deeper (one more bucket, HB,
// holds everything past HD1 when zlo is not known): per-bucket counts and
// fixed-point masses, then the one bucket that holds the answer.
constexpr int HB = 4096;
constexpr int HB1 = 3072;
constexpr float HSCALE = 128.0f;
constexpr float HD1 = HB1 / HSCALE;  // 24
constexpr int HCAP = 2048;  // largest bucket resolved in LDS (else the radix passes)

struct SmemHist {
    uint32_t hc[HB + 1];
    unsigned long long hm[HB + 1];
};

struct SmemBucket {
    unsigned long long key[HCAP];
    unsigned long long wq[HCAP];
};

struct SmemHistState {
    unsigned long long wsum[NTR_MAX / WAVE];
    unsigned long long wsum2[NTR_MAX / WAVE];
    unsigned long long cum;     // count or mass of the buckets before the selected one
    unsigned long long target;
    unsigned long long key;
    unsigned long long total_mass;
    int total_count;
    int sel;                    // selected bucket (INT_MAX: none crosses)
    int lastnz;                 // deepest non-empty bucket
    int n;                      // entries collected from the selected bucket
};

constexpr int RQ = 4;            // 16-byte loads per thread in flight in vector row passes
constexpr int LIST_CAP = 8192;  // history + draft + bias ids staged in LDS by the fallback

// The workgroup visits every entry v of a float row in memory, f(v, zr[v]).
// The passes of the whole-row path are bound by the bytes each thread keeps in
// flight, so the 16-byte-aligned body goes four floats per load, RQ loads at a
// time (NQ of them; a pass with little work per entry takes more); the
// unaligned head and the tail take one entry per thread.
template <int NQ = RQ, class F>
__device__ __forceinline__ void row_visit(const float* zr, int V, F f) {
    const int tid = threadIdx.x;
    const int head = min(V, (int)(((16u - ((uint32_t)(uintptr_t)zr & 15u)) & 15u) >> 2));
    if (tid < head) f(tid, zr[tid]);
    const int nq = (V - head) >> 2;
    const uint4* q = (const uint4*)(zr + head);
    for (int i0 = tid; i0 < nq; i0 += NTR * NQ) {
        uint4 t[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) t[k] = i0 + k * NTR < nq ? gld(q + i0 + k * NTR) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const int i = i0 + k * NTR;
            if (i < nq) {
                const int v = head + 4 * i;
                f(v, __uint_as_float(t[k].x));
                f(v + 1, __uint_as_float(t[k].y));
                f(v + 2, __uint_as_float(t[k].z));
                f(v + 3, __uint_as_float(t[k].w));
            }
        }
    }
    const int v = head + 4 * nq + tid;
    if (v < V) f(v, zr[v]);
}

// Per-chunk tables of the whole-row path's patches: multiplicities (u16 pairs),
// bias marks, claim flags, and which chunks any list entry touches.
constexpr int PCH = 16384;     // vocabulary entries per chunk
constexpr int PMASKW = 1;      // chunk mask words
static_assert(MAX_VOCAB <= PMASKW * 32 * PCH, "patch chunk mask");

struct SmemPatch {
    uint32_t cnt[PCH / 2];
    uint32_t bias[PCH / 32];
    uint32_t flag[PCH / 32];
    uint32_t touched[PMASKW];
};

constexpr int BV_CAP = 1024;  // bias values staged in LDS by the fallback

struct SmemList {
    int32_t ids[LIST_CAP];      // the history, draft and bias ids
    uint32_t work[LIST_CAP];    // claimed entries: list index | multiplicity << 13 | bias << 27
    float bvals[BV_CAP];        // the bias values
    int nwork;
    SmemPatch pt;
};
static_assert(LIST_CAP <= (1 << 13), "work item layout");

// The draw of an unfiltered row over its binned tail: the row's non-pool mass
// by bin of z, the entries of the bin that holds the draw, and their masses by
// sub-bin.
constexpr int NRB = 1024;  // row bins (the last one also holds everything deeper)
constexpr int NSB = 64;    // sub-bins of the drawn bin
constexpr int BCAP = 8192;  // entries of the drawn bin
constexpr int SBCAP = 512; // entries of the drawn sub-bin
static_assert(NSB == WAVE && NRB % WAVE == 0, "one sub-bin per lane; whole bins per lane");
constexpr int UBCAP = 8;   // wave tiles without bins that the draw bins itself
struct SmemBins {
    double rb[NRB];
    double sb[NSB];
    unsigned long long key[BCAP];
    unsigned long long sk[SBCAP];
    double part[NTR_MAX / WAVE];
    int toff[MAX_WT];          // row bin of each wave tile's bin 0 (INT_MAX: no bins)
    float tscale[MAX_WT];      // exp(zm - zmax) of each wave tile
    int tnc[MAX_WT];           // candidates of each wave tile
    double base, tgt;
    float xlo, xhi;            // bin beta's entries: x in (xlo, xhi]
    int n, beta, sub, ns, pick;
};

static_assert(sizeof(SmemBins) <= sizeof(SmemList), "the binned draw adds no LDS");
union SmemU {
    SmemTile t;
    SmemPool p;
    SmemRadix r;
    SmemHist h;
    SmemBucket k;
    SmemList l;
    SmemBins b;
};

template <int NB>
struct SmemST {
    RedT<NB> red;
    RedT<NB> red2;
    float fmin[NB / WAVE];
    int imax[NB / WAVE];
    double dg[EPT / 4][NB / WAVE];  // per wave: one total per group of the tile's threads
    int sel;
    int take_last;
    unsigned long long rem;
    SmemHistState hs;
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

// Slot s's id formed from one base register at the point of use: the empty asm
// hides the base's value so the compiler does not keep one id register per
// group alive across the kernel (it has no memory operands).
template <int DT>
__device__ __forceinline__ int slot_id_late(int base, int s) {
    using L = Lay<DT>;
    asm volatile("" : "+v"(base));
    return base + (s / L::VEC) * L::GSTRIDE + (s % L::VEC);
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

// The branch-free tile load of aligned rows, kept as raw 16-byte words so that
// work issued after it (the tables' build) need not wait for the data: the
// unpack comes later.
template <int DT>
struct RawTile {
    uint4 q[Lay<DT>::NG];
};

template <int DT>
__device__ __forceinline__ RawTile<DT> load_tile_raw(const RowCtx& c, int tb) {
    using L = Lay<DT>;
    constexpr int ES = DT == SS_F32 ? 4 : 2;
    const char* row = (const char*)c.logits;
    RawTile<DT> r;
#pragma unroll
    for (int g = 0; g < L::NG; ++g) {
        const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
        // the logits are read once: non-temporal, so they do not push the
        // row's history ids out of L2; a 32-bit offset from the row's
        // (uniform) base keeps one register per load; a group past V reads the
        // row's last group instead (rows are 16-byte aligned, V a multiple of
        // the group) and is set to -inf when unpacked
        const uint32_t off = (uint32_t)min(e0, c.V - L::VEC) * (uint32_t)ES;
        const u32x4_t qv = __builtin_nontemporal_load((const u32x4_t*)(row + off));
        r.q[g] = make_uint4(qv.x, qv.y, qv.z, qv.w);
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void unpack_tile(const RowCtx& c, int tb, const RawTile<DT>& r, float v[EPT]) {
    using L = Lay<DT>;
#pragma unroll
    for (int g = 0; g < L::NG; ++g) unpack_group<DT>(r.q[g], v + g * L::VEC);
    if (tb + TILE > c.V) {  // only the row's last tile reaches past V
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
#pragma unroll
            for (int j = 0; j < L::VEC; ++j) v[g * L::VEC + j] = e0 < c.V ? v[g * L::VEC + j] : NEG_INF;
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
            // row's history ids and the tile summaries out of L2; a 32-bit
            // offset from the row's (uniform) base keeps one register per load
            const uint32_t off = (uint32_t)min(e0, c.V - L::VEC) * (uint32_t)ES;
            const u32x4_t* src = (const u32x4_t*)(row + off);
            const u32x4_t qv = __builtin_nontemporal_load(src);
            q[g] = make_uint4(qv.x, qv.y, qv.z, qv.w);
        }
#pragma unroll
        for (int g = 0; g < L::NG; ++g) unpack_group<DT>(q[g], v + g * L::VEC);
        if (tb + TILE > c.V) {  // only the row's last tile reaches past V
#pragma unroll
            for (int g = 0; g < L::NG; ++g) {
                const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
#pragma unroll
                for (int j = 0; j < L::VEC; ++j) v[g * L::VEC + j] = e0 < c.V ? v[g * L::VEC + j] : NEG_INF;
            }
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

// The bias of tile entry l (id tb + l), known to be biased. When each biased
// entry of the tile has one bias entry and the tile's hits fit the list, the
// single value comes from the LDS hit list; otherwise the row's whole list is
// applied in array order.
__device__ __forceinline__ float add_bias_t(const RowCtx& c, float x, int id, int l, const SmemTile& t,
                                           int nbh, bool bfull) {
    if (!bfull) {
        for (int k = 0; k < nbh; ++k)
            if (t.bl[k] == l) x = x + t.bv[k];
        return x;
    }
    for (int k = 0; k < c.bias_len; ++k)
        if (gld(c.bias_ids + k) == id) x = x + gld(c.bias_vals + k);
    return x;
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

// Builds the tile's multiplicity counts in LDS, for every thread a word with
// bit s set when its slot s holds a penalised or biased entry and a word with
// bit s set when it is biased, and the list of the tile's bias hits (two
// barriers). Threads with active = false only take part in the barriers.
template <int DT>
__device__ __forceinline__ void build_tables(const RowCtx& c, int tb, SmemTile& t,
                                             const TablePrefetch& f, bool active = true) {
    using L = Lay<DT>;
    const int tid = threadIdx.x;
    const bool has_cnt = active && (c.hist_len + c.extra_len) > 0;
    const bool has_bias = active && c.bias_len > 0;
    if (has_cnt) {
        uint4* c4 = (uint4*)t.cnt;
#pragma unroll
        for (int k = 0; k < TILE / 8 / NT; ++k) c4[tid + k * NT] = make_uint4(0, 0, 0, 0);
    }
    if (active) {
        t.xw[tid] = 0;
        t.bw[tid] = 0;
        if (tid == 0) {
            t.nbh = 0;
            t.bfull = 0;
        }
    }
    __syncthreads();
    // owner thread and slot bit of local entry l (the inverse of slot_id)
    auto owner = [&](int l) { return (l % L::GSTRIDE) / L::VEC; };
    auto bit = [&](int l) { return 1u << ((l / L::GSTRIDE) * L::VEC + (l % L::GSTRIDE) % L::VEC); };
    auto count = [&](int id) {
        const int l = id - tb;
        if (id >= 0 && id < c.V && l >= 0 && l < TILE) {
            atomicAdd(&t.cnt[l >> 1], 1u << ((l & 1) * 16));
            atomicOr(&t.xw[owner(l)], bit(l));
        }
    };
    if (has_cnt) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if (tid + k * NT < c.hist_len) count(f.hist[k]);
        for (int i = tid + 2 * NT; i < c.hist_len; i += NT) count(gld(c.hist + i));
        if (tid < c.extra_len) count(f.extra);
    }
    auto mark = [&](int id, float val) {
        const int l = id - tb;
        if (id >= 0 && id < c.V && l >= 0 && l < TILE) {
            const int o = owner(l);
            const uint32_t b = bit(l);
            atomicOr(&t.xw[o], b);
            const uint32_t old = atomicOr(&t.bw[o], b);
            const int p = atomicAdd(&t.nbh, 1);
            if (p < NT) {
                t.bl[p] = l;
                t.bv[p] = val;
            }
            if ((old & b) || p >= NT) t.bfull = 1;
        }
    };
    if (has_bias && tid < c.bias_len) mark(f.bias_id, f.bias_val);
    for (int i = tid + NT; has_bias && i < c.bias_len; i += NT) mark(gld(c.bias_ids + i), gld(c.bias_vals + i));
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

// a where the mask m is all ones, b where it is zero (a bit select)
__device__ __forceinline__ float bsel(uint32_t m, float a, float b) {
    return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

// All ones when bit b of s is set (the empty asm hides that the value is 0 or
// all ones, so the compiler keeps the bit selects instead of rewriting them
// into an indexed access, which would move the slot array to scratch).
__device__ __forceinline__ uint32_t bit_mask(uint32_t s, int b) {
    uint32_t m = 0u - ((s >> b) & 1u);
    asm volatile("" : "+v"(m));
    return m;
}

// Slot s of this thread's entries, s held per lane (registers cannot be
// indexed by a per-lane value): a select tree over the bits of s.
__device__ __forceinline__ float slot_get(const float v[EPT], int s) {
    float a[EPT / 2];
    const uint32_t m0 = bit_mask((uint32_t)s, 0);
#pragma unroll
    for (int i = 0; i < EPT / 2; ++i) a[i] = bsel(m0, v[2 * i + 1], v[2 * i]);
#pragma unroll
    for (int w = EPT / 4, b = 1; w >= 1; w >>= 1, ++b) {
        const uint32_t m = bit_mask((uint32_t)s, b);
#pragma unroll
        for (int i = 0; i < w; ++i) a[i] = bsel(m, a[2 * i + 1], a[2 * i]);
    }
    return a[0];
}

__device__ __forceinline__ void slot_set(float v[EPT], int s, float x) {
    const uint32_t oh = 1u << s;
#pragma unroll
    for (int i = 0; i < EPT; ++i) v[i] = bsel(bit_mask(oh, i), x, v[i]);
}

// Penalties, bias and mask on this thread's entries. The mask comes first, as
// a bit select per slot; then each lane walks the set bits of its exception
// word (penalised or biased entries that the mask allows), one entry per
// step, so the wave takes as many steps as its busiest lane has exceptions and
// the code holds one copy of the per-entry work (its size matters: the whole
// kernel competes for the instruction cache).
template <int DT>
__device__ __forceinline__ void process_tile(const RowCtx& c, int tb, float v[EPT], const SmemTile& t,
                                             const uint32_t mwords[Lay<DT>::NG], bool tables) {
    using L = Lay<DT>;
    constexpr uint32_t vm = (1u << L::VEC) - 1u;
    uint32_t aw = 0xFFFFFFFFu;  // bit s: slot s is allowed by the mask
    if (c.mask) {
        aw = 0u;
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            const int e0 = tb + g * L::GSTRIDE + (int)threadIdx.x * L::VEC;
            aw |= ((mwords[g] >> (e0 & 31)) & vm) << (g * L::VEC);
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) v[k] = ((aw >> k) & 1u) ? v[k] : NEG_INF;
    }
    uint32_t ex = tables ? t.xw[threadIdx.x] & aw : 0u;
    if (ex == 0u) return;
    const uint32_t bw = c.bias_len > 0 ? t.bw[threadIdx.x] : 0u;
    const int nbh = bw ? t.nbh : 0;
    const bool bfull = bw ? t.bfull != 0 : false;
    const bool has_cnt = (c.hist_len + c.extra_len) > 0;
    do {
        const int sl = __builtin_ctz(ex);
        ex &= ex - 1u;
        const int l = (sl / L::VEC) * L::GSTRIDE + (int)threadIdx.x * L::VEC + (sl % L::VEC);
        const int id = tb + l;
        if (id < c.V) {
            const uint32_t cnt = has_cnt ? (t.cnt[l >> 1] >> ((l & 1) * 16)) & 0xFFFFu : 0u;
            float x = penalize(c, slot_get(v, sl), cnt);
            if ((bw >> sl) & 1u) x = add_bias_t(c, x, id, l, t, nbh, bfull);
            slot_set(v, sl, x);
        }
    } while (ex != 0u);
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

// ---------------------------------------------------------------------------
// stage 1: one tile of one row; each wave summarises its own wave tile

__device__ __forceinline__ float wave_min_f(float v) {
    return wave_allreduce32(v, [](float a, float b) { return fminf(a, b); });
}

__device__ __forceinline__ int wave_max_i(int v) {
    return wave_allreduce32(v, [](int a, int b) { return max(a, b); });
}


template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// Entries of this lane above theta (strict) or at or above it, counted over the
// wave (the ballot counts stay in scalar registers).
__device__ __forceinline__ int wave_count_above(const float v[EPT], float theta, bool strict) {
    int n = 0;
#pragma unroll
    for (int s = 0; s < EPT; ++s) n += __popcll(__ballot(strict ? v[s] > theta : v[s] >= theta));
    return n;
}

// BINS: the binned tails of unfiltered rows (the SAMPLE draw only)
template <int DT, bool ALIGNED, bool BINS>
__device__ __forceinline__ void tile_stage1(const RowCtx& c, int row, int tile, const Workspace& ws,
                                            SmemTile& tt, float* dbg_proc_row, float* dbg_probs_row) {
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int tb = tile * TILE;
    const int sid0 = tb + tid * Lay<DT>::VEC;  // id of this thread's slot 0
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    // issue order: mask words and history / bias (needed first), then the
    // tile, which the tables' build does not wait for
    load_mask<DT>(c, tb, mw);
    const TablePrefetch f = prefetch_tables(c);
    __builtin_amdgcn_sched_barrier(0);
    const bool tables = c.hist_len + c.extra_len + c.bias_len > 0;
    if constexpr (ALIGNED) {
        const RawTile<DT> raw = load_tile_raw<DT>(c, tb);
        if (tables) build_tables<DT>(c, tb, tt, f);
        unpack_tile<DT>(c, tb, raw, v);
    } else {
        load_tile<DT, false>(c, tb, v);
        if (tables) build_tables<DT>(c, tb, tt, f);
    }
    process_tile<DT>(c, tb, v, tt, mw, tables);

    if (dbg_proc_row || dbg_probs_row) {
        // 32-bit offsets from the row's (uniform) base: no per-lane 64-bit
        // addresses are kept for this cold path
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int id = slot_id_late<DT>(sid0, s);
            if (id < c.V) {
                const uint32_t off = (uint32_t)id * 4u;
                if (dbg_proc_row) *(float*)((char*)dbg_proc_row + off) = v[s];
                if (dbg_probs_row) *(float*)((char*)dbg_probs_row + off) = 0.0f;
            }
        }
    }

    // From here on each wave works alone on its wave tile (its entries
    // interleave across the workgroup tile, so every wave tile of the last
    // tile may hold entries below V).
    const int wt = tile * WPT + __builtin_amdgcn_readfirstlane(wv);  // uniform per wave
    unsigned long long* const cand = ws.cand + ((size_t)row * ws.n_wt + wt) * WCAP;
    float lm = v[0], lmin = v[0];
#pragma unroll
    for (int s = 1; s < EPT; ++s) {
        lm = fmaxf(lm, v[s]);
        lmin = fminf(lmin, v[s]);
    }
    // entries are counted one by one only in waves where some lane holds a -inf
    int nf = EPT;
    if (__ballot(!(lmin > NEG_INF))) {
        nf = 0;
#pragma unroll
        for (int s = 0; s < EPT; ++s) nf += v[s] > NEG_INF;
    }
    const float m = wave_max(lm);
    WaveStat st;
    st.m = m;
    st.argmax = -1;
    st.zbeta = NEG_INF;
    st.ncand = 0;
    st.nfinite = wave_sum_i(nf);
    st.flags = 0;
    st.zmin = __builtin_huge_valf();
    st.zm = NEG_INF;
    st.s = 0.0;
    st.sc = 0.0;
    if (c.T == 0.0f) {
        // greedy: lowest id among the maxima; only lanes holding the maximum scan
        int am = INT_MAX;
        if (m > NEG_INF && lm == m) {
#pragma unroll
            for (int s = EPT - 1; s >= 0; --s)
                if (v[s] == m) am = slot_id_late<DT>(sid0, s);
        }
        am = wave_min_i(am);
        st.argmax = m > NEG_INF ? am : -1;
    } else if (m > NEG_INF) {
        // Windows x' >= m - d T for d = DELTA, DELTA / 2, DELTA / 4: the first
        // whose entries fit the wave's WCAP slots gives the candidates. On a
        // low-entropy row the wave holding the row maximum keeps everything
        // within DELTA of it; a wave deep in the tail sees a locally dense
        // region and settles for a narrower window. The window is chosen on
        // counts alone (a compare and a ballot per slot); the candidates are
        // written once, for the chosen threshold.
        unsigned long long* wl = tt.wl[wv];
        float theta = fmaxf(m - DELTA * c.T, -FLT_MAX);
        int n = wave_count_above(v, theta, false);
        // A narrower window only shortens the search: the head by count always
        // cuts lower. It is worth taking where the wide window overflowed
        // modestly (a locally dense stretch of a steep tail, whose narrower
        // cut still lies far below the row maximum); a wave with three quarters
        // of its entries inside the wide window is flat and goes to the count cut.
        if (n > WCAP && n <= 3 * (WT / 4)) {
            theta = fmaxf(m - (0.5f * DELTA) * c.T, -FLT_MAX);
            n = wave_count_above(v, theta, false);
            if (n > WCAP) {
                theta = fmaxf(m - (0.25f * DELTA) * c.T, -FLT_MAX);
                n = wave_count_above(v, theta, false);
            }
        }
        const bool strict = n > WCAP;
        if (strict) {
            // Even the narrowest window overflows (a flat wave): keep the head by
            // count. With the lane maxima sorted descending, count(x' > sorted[L])
            // grows with L; take the largest L whose count fits (L = 0 always
            // does: nothing exceeds the maximum).
            const float srt = wave_sort_desc(lm);
            int lo = 0, hi = WAVE - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                const float th = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(srt), mid));
                if (wave_count_above(v, th, true) <= WCAP) lo = mid;
                else hi = mid - 1;
            }
            theta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(srt), lo));
            st.flags |= WS_OVF;
        }
        // The candidates in slot order, to the wave's LDS list: at most WCAP
        // of them, the count above having used the same comparisons.
        auto write = [&](auto strict_c) -> int {
            constexpr bool STRICT = decltype(strict_c)::value;
            int k = 0;
#pragma unroll
            for (int sl = 0; sl < EPT; ++sl) {
                const bool hit = STRICT ? v[sl] > theta : v[sl] >= theta;
                const unsigned long long bm = __ballot(hit);
                if (bm) {
                    const int p = k + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
                    if (hit)
                        wl[p] = ((unsigned long long)__float_as_uint(v[sl]) << 32) | (uint32_t)slot_id_late<DT>(sid0, sl);
                    k += __popcll(bm);
                }
            }
            return k;
        };
        const int base = strict ? write(BoolC<true>{}) : write(BoolC<false>{});
        st.ncand = base;
        st.zm = canon_zero(m / c.T);
        // non-candidates have x' below (or at) theta, so z at most RN(theta / T)
        st.zbeta = base < st.nfinite ? canon_zero(theta / c.T) : NEG_INF;
        // the LDS list was written by other lanes of this wave: LDS operations
        // of one wave complete in order, the fences keep the compiler's order
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // each lane below the count turns one candidate into its key (z, id)
        // and weighs it against the wave maximum: the merge takes the tile's
        // candidate mass whole instead of re-forming every weight
        {
            const float zm = st.zm;
            float zc = __builtin_huge_valf();
            float wcand = 0.0f;
            if (lane < base) {
                const unsigned long long e = wl[lane];
                const float x = __uint_as_float((uint32_t)(e >> 32));
                zc = canon_zero(x / c.T);
                wcand = expf(zc - zm);
                *(unsigned long long*)((char*)cand + (uint32_t)lane * 8u) = key64(zc, (int)(uint32_t)e);
            }
            st.zmin = wave_min_f(zc);
            st.sc = wave_sum_d((double)wcand);
        }
        // The mass outside the candidates. A wave tile with more than k finite
        // entries proves the row is cut by top-k: its mass outside the
        // candidates is not needed (the top-k set's is bounded by count in the
        // merge). Otherwise a count-cut (flat) wave tile sums its whole mass
        // exactly, z = x' / T entry by entry (the row's normaliser may rest on
        // it), and every other wave tile sums its non-candidates with exp2 on
        // x' log2(e) / T - m log2(e) / T, an approximation whose error the
        // merge bounds: it serves as the normaliser's far tail.
        const bool certainly_cut = c.top_k > 0 && c.top_k < c.V && st.nfinite > c.top_k;
        if (certainly_cut) {
            // no tail sum
        } else if (strict) {
            const float zm = st.zm;
            // A count-cut wave tile of an unfiltered row without penalty or
            // bias tables also bins its non-candidates' masses by z: the
            // row's draw can then skip the whole-row passes. The tables' LDS,
            // unused then, holds the wave's bins.
            const bool bin = BINS && ws.bins != nullptr && !tables && st.zbeta > NEG_INF && c.top_p >= 1.0f &&
                             c.min_p <= 0.0f && (c.top_k <= 0 || c.top_k >= c.V);  // uniform
            double* wb = (double*)tt.cnt + wv * NBIN;
            const float a0 = floorf(-st.zbeta * (float)BIN_S);
            if (bin) {
                for (int i = lane; i < NBIN; i += WAVE) wb[i] = 0.0;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            // separate copies of the loop: the one without bins stays free of
            // them, and where T is a power of two (T = 1 above all) x' / T is
            // the exact product x' (1 / T), without a division per entry
            const float rT = 1.0f / c.T;
            const bool pow2 = pow2_temp(c.T);  // uniform
            auto sum_tile = [&](auto bin_c, auto p2_c) {
                constexpr bool BIN = decltype(bin_c)::value;
                constexpr bool P2 = decltype(p2_c)::value;
                double acc = 0.0;
#pragma unroll
                for (int s = 0; s < EPT; ++s) {
                    if (v[s] > NEG_INF) {
                        const float z = canon_zero(P2 ? v[s] * rT : v[s] / c.T);
                        const float w = expf(z - zm);
                        acc += (double)w;
                        // non-candidates: x' <= theta, so z <= zbeta and the bin is >= 0
                        if (BIN && v[s] <= theta)
                            atomicAdd(&wb[(int)fminf(floorf(-z * (float)BIN_S) - a0, (float)(NBIN - 1))], (double)w);
                    }
                }
                return acc;
            };
            double acc;
            if constexpr (BINS) {
                if (bin) acc = pow2 ? sum_tile(BoolC<true>{}, BoolC<true>{}) : sum_tile(BoolC<true>{}, BoolC<false>{});
                else acc = pow2 ? sum_tile(BoolC<false>{}, BoolC<true>{}) : sum_tile(BoolC<false>{}, BoolC<false>{});
            } else {
                acc = pow2 ? sum_tile(BoolC<false>{}, BoolC<true>{}) : sum_tile(BoolC<false>{}, BoolC<false>{});
            }
            st.s = wave_sum_d(acc);
            st.flags |= WS_SUM;
            if (bin) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                float* gb = ws.bins + ((size_t)row * ws.n_wt + wt) * NBIN;
                for (int i = lane; i < NBIN; i += WAVE) gb[i] = (float)wb[i];
                st.flags |= WS_BIN;
            }
        } else {
            float acc = 0.0f;
            if (base < st.nfinite) {
                const float c2 = 1.4426950408889634f / c.T;
                const float mc = m * c2;
#pragma unroll
                for (int s = 0; s < EPT; ++s) {
                    // one fused rounding: x' c2 - m c2
                    const float t = __builtin_amdgcn_exp2f(__builtin_fmaf(v[s], c2, -mc));
                    acc += v[s] >= theta ? 0.0f : t;
                }
            }
            st.s = wave_sum_d((double)acc);
            st.flags |= WS_APX;
        }
    }
    if (lane == 0) ws.wstats[(size_t)row * ws.n_wt + wt] = st;
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
    int nfinite;
};

__device__ __forceinline__ WaveStat empty_stat() {
    WaveStat s;
    s.m = NEG_INF;
    s.argmax = -1;
    s.zbeta = NEG_INF;
    s.ncand = 0;
    s.nfinite = 0;
    s.flags = 0;
    s.zmin = __builtin_huge_valf();
    s.zm = NEG_INF;
    s.s = 0.0;
    s.sc = 0.0;
    return s;
}

// What the merge reads from stage 1, issued before anything else so the row's
// loads share one round trip: lane t of every wave holds the summaries of wave
// tiles t and t + 64, and thread (wave w, lane l) candidate slot l of wave
// tiles w, w + 16, ... (read whether or not the slot is filled).
struct RowLoad {
    unsigned long long cv[MSLOT];
    WaveStat s0, s1;
};

__device__ __forceinline__ RowLoad row_load(const Workspace& ws, int row) {
    RowLoad l;
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    const unsigned long long* cand = ws.cand + (size_t)row * ws.n_wt * WCAP;
#pragma unroll
    for (int k = 0; k < MSLOT; ++k) {
        const int wt = wv + NWR * k;
        l.cv[k] = wt < ws.n_wt ? gld(cand + (size_t)wt * WCAP + lane) : 0ull;
    }
    const WaveStat* st = ws.wstats + (size_t)row * ws.n_wt;
    l.s0 = lane < ws.n_wt ? st[lane] : empty_stat();
    l.s1 = lane + WAVE < ws.n_wt ? st[lane + WAVE] : empty_stat();
    return l;
}

// A field of wave tile wt's summary (wt uniform across the wave).
__device__ __forceinline__ int stat_ncand(const RowLoad& l, int wt) {
    return wt < WAVE ? __builtin_amdgcn_readlane(l.s0.ncand, wt) : __builtin_amdgcn_readlane(l.s1.ncand, wt - WAVE);
}
__device__ __forceinline__ int stat_flags(const RowLoad& l, int wt) {
    return wt < WAVE ? __builtin_amdgcn_readlane(l.s0.flags, wt) : __builtin_amdgcn_readlane(l.s1.flags, wt - WAVE);
}

// The row as the wave-tile summaries describe it (formed by every wave alike).
struct RowView {
    float zmax;    // z of the row maximum
    float zb;      // the pool is every candidate with z > zb (-inf: every finite entry)
    float zlo;     // a lower bound of the pool's z
    double W;      // the row mass: candidates, WS_SUM tiles whole, WS_APX non-candidates
    double Wc;     // the candidates' mass: at least the pool's
    double err;    // bound on the error of the approximate part of W
    int missing;   // some tile leaves mass outside its candidates that no sum covers
                   // (only where the row is cut by top-k)
    unsigned long long ub[2];  // wave tiles that leave non-candidates no WS_BIN bins cover
};

// Relative error bound of a window-cut tile's approximate non-candidate mass:
// each term exp2(fma(x', c2, -m c2)) differs from exp(RN(x'/T) - RN(m/T)) by
// the roundings of m c2, the fused product-difference and the reciprocal (each
// 2^-24 of terms up to |z| + d, d <= 104 for any term that is not zero in
// binary32), exp2's own error and the binary32 sum of 32 terms.
__device__ __forceinline__ double apx_eps(float zm) {
    return 0x1p-21 * ((double)fabsf(zm) + 104.0) + 0x1p-19;
}

__device__ __forceinline__ RowView row_view(const RowLoad& l, float m, float T) {
    RowView r;
    r.zmax = canon_zero(m / T);
    float zb[2];
    double sum = 0.0, err = 0.0, csum = 0.0;
    float zmin = __builtin_huge_valf();
    int missing = 0;
    bool ub[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const WaveStat& s = h ? l.s1 : l.s0;
        const bool incomplete = s.ncand < s.nfinite;
        zb[h] = incomplete ? s.zbeta : NEG_INF;
        ub[h] = incomplete && !(s.flags & WS_BIN);
        zmin = fminf(zmin, s.zmin);
        if (s.nfinite > 0) {
            const float zm = s.zm;
            // binary32 exp of a binary32 difference: relative error ~1e-7 on
            // each tile's share of the mass
            const double scale = (double)expf(zm - r.zmax);
            csum += s.sc * scale;
            if (s.flags & WS_SUM) {
                sum += s.s * scale;  // the whole tile, candidates included
            } else {
                sum += s.sc * scale;
                if (s.flags & WS_APX) {
                    sum += s.s * scale;
                    err += s.s * scale * apx_eps(zm);
                } else if (incomplete) {
                    missing = 1;
                }
            }
        }
    }
    r.zb = wave_max(fmaxf(zb[0], zb[1]));
    r.zlo = r.zb > NEG_INF ? r.zb : wave_min_f(zmin);
    r.W = wave_sum_d(sum);
    r.Wc = wave_sum_d(csum);
    r.err = wave_sum_d(err);
    r.missing = wave_max_i(missing);
    r.ub[0] = __ballot(ub[0]);
    r.ub[1] = __ballot(ub[1]);
    return r;
}

__device__ __forceinline__ int row_argmax(const RowLoad& l, float m) {
    const int a = (l.s0.m == m && l.s0.argmax >= 0) ? l.s0.argmax : INT_MAX;
    const int b = (l.s1.m == m && l.s1.argmax >= 0) ? l.s1.argmax : INT_MAX;
    return wave_min_i(min(a, b));
}

// floor(w 2^44) for a binary32 weight w in [0, 1], by integer shifts of its
// significand: the same value as truncating the binary64 product w * 2^44
// (exact: 24 bits), without the binary64-to-integer conversion sequence.
__device__ __forceinline__ uint64_t wq(float w) {
    static_assert(MASS_SCALE == 0x1p44, "the shift below assumes 2^44");
    const uint32_t b = __float_as_uint(w);
    const int e = (int)(b >> 23);  // biased exponent (w >= 0)
    const uint64_t m = (uint64_t)((b & 0x7FFFFFu) | 0x800000u);
    const int sh = e - 106;        // w 2^44 = m 2^(e - 127 - 23 + 44)
    if (e == 0) return 0;          // zero or subnormal: below 2^-82
    return sh >= 0 ? m << sh : (sh > -64 ? m >> -sh : 0);
}


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

// Scale of the deep buckets for a row whose finite z lie in [zlo, zmax] (0:
// none, zlo unknown or the row is shallower than HD1).
__device__ __forceinline__ float hdeep_scale(float zmax, float zlo) {
    const float r = zmax - zlo;
    return r > HD1 ? fminf((float)(HB - HB1) / (r - HD1), 1.0e30f) : 0.0f;
}

__device__ __forceinline__ int hbucket(float z, float zmax, float s2) {
    // d = zmax - z >= 0 rounded, then scaled exactly (near part) or shifted
    // and scaled (deep part): every step is monotone in z, so bucket order
    // follows key order
    const float d = zmax - z;
    const float dn = d * HSCALE;
    if (dn < (float)HB1) return (int)dn;
    if (s2 > 0.0f) return HB1 + (int)fminf((d - HD1) * s2, (float)(HB - HB1 - 1));
    return HB;
}

// Exclusive prefix of one u64 per thread in thread order (exact); total too.
__device__ unsigned long long block_excl_scan_u64(unsigned long long v, SmemHistState& hs,
                                                  unsigned long long& total) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = threadIdx.x / WAVE;
    const unsigned long long inc = wave_incl_scan_u64(v);
    if (lane == WAVE - 1) hs.wsum[w] = inc;
    __syncthreads();
    unsigned long long base = 0, tot = 0;
    for (int k = 0; k < NTR / WAVE; ++k) {
        if (k < w) base += hs.wsum[k];
        tot += hs.wsum[k];
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

// The same for two values at once (one pair of barriers).
__device__ void block_excl_scan2_u64(unsigned long long a, unsigned long long b, SmemHistState& hs,
                                     unsigned long long& pre_a, unsigned long long& pre_b,
                                     unsigned long long& tot_a, unsigned long long& tot_b) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = threadIdx.x / WAVE;
    const unsigned long long ia = wave_incl_scan_u64(a), ib = wave_incl_scan_u64(b);
    if (lane == WAVE - 1) {
        hs.wsum[w] = ia;
        hs.wsum2[w] = ib;
    }
    __syncthreads();
    unsigned long long ba = 0, bb = 0, ta = 0, tb = 0;
    for (int k = 0; k < NTR / WAVE; ++k) {
        const unsigned long long x = hs.wsum[k], y = hs.wsum2[k];
        if (k < w) {
            ba += x;
            bb += y;
        }
        ta += x;
        tb += y;
    }
    __syncthreads();
    pre_a = ba + ia - a;
    pre_b = bb + ib - b;
    tot_a = ta;
    tot_b = tb;
}

// An entry's weight exp(z - zmax). With deep_zero, entries more than
// HW_DEEP below the maximum weigh 0 without the exponential: their fixed-point
// weight is 0 either way (exp(-HW_DEEP) 2^44 < 1), and the caller's predicate
// does not tell such small weights from 0.
constexpr float HW_DEEP = 31.0f;
__device__ __forceinline__ float entry_w(float z, float zmax, bool deep_zero) {
    return deep_zero && zmax - z > HW_DEEP ? 0.0f : expf(z - zmax);
}

// Totals of the entries that pass (key >= kmin, and w >= wmin when wmin > 0: the
// predicate of every selection here) (count, and with by_mass the fixed-point
// mass) and, when want_key, the key selected among them exactly as radix_select
// defines it (an entry's weight is formed only where the mass or wmin needs it):
// by count, the key of rank `target` (1-based); by mass, the key of the first
// entry whose inclusive mass exceeds target = frac x total mass (frac > 0) or
// `target` (frac = 0); the smallest such key if none does. One pass builds the
// bucket histogram; a second collects the selected bucket's entries, which are
// resolved by pairwise comparison. A bucket too large for LDS, or the deepest
// bucket, is left to radix_select.
__device__ __forceinline__ void hist_select(const float* zr, int V, float zmax, float s2, bool w_deep_zero,
                                            unsigned long long kmin, float wmin, bool by_mass, bool want_key,
                                            unsigned long long target, double frac, SmemU& su, SmemR& sh,
                                            int& count, unsigned long long& mass, unsigned long long& key) {
    const int tid = threadIdx.x;
    const bool need_w = by_mass || wmin > 0.0f;  // uniform
    // the entry's key when it passes (0 otherwise: no finite z has key 0), and its weight
    auto pass = [&](int v, float z, float& w) -> unsigned long long {
        const unsigned long long kk = key64(z, v);
        if (kk < kmin) return 0ull;
        w = 0.0f;
        if (need_w) {
            w = entry_w(z, zmax, w_deep_zero);
            if (wmin > 0.0f && !(w >= wmin)) return 0ull;
        }
        return kk;
    };
    SmemHist& h = su.h;
    SmemHistState& hs = sh.hs;
    for (int b = tid; b <= HB; b += NTR) {
        h.hc[b] = 0;
        h.hm[b] = 0;
    }
    __syncthreads();
    row_visit(zr, V, [&](int v, float z) {
        if (!(z > NEG_INF)) return;
        // the key only where kmin can exclude the entry
        if (kmin != 0ull && key64(z, v) < kmin) return;
        float w = 0.0f;
        if (need_w) {
            w = entry_w(z, zmax, w_deep_zero);
            if (wmin > 0.0f && !(w >= wmin)) return;
        }
        const int b = hbucket(z, zmax, s2);
        atomicAdd(&h.hc[b], 1u);
        if (by_mass) atomicAdd(&h.hm[b], (unsigned long long)wq(w));
    });
    __syncthreads();
    // thread t owns buckets 4t .. 4t + 3; the last thread also the deepest one
    constexpr int PER = HB / NTR;
    static_assert(PER * NTR == HB, "bucket ownership");
    const int b0 = tid * PER;
    const int nb = PER + (tid == NTR - 1 ? 1 : 0);
    unsigned long long mine_c = 0, mine_m = 0;
    int lastnz = -1;
    for (int i = 0; i < nb; ++i) {
        mine_c += h.hc[b0 + i];
        mine_m += h.hm[b0 + i];
        if (h.hc[b0 + i]) lastnz = b0 + i;
    }
    unsigned long long tot_c, tot_m, pre_c, pre_m;
    block_excl_scan2_u64(mine_c, mine_m, hs, pre_c, pre_m, tot_c, tot_m);
    count = (int)tot_c;
    mass = tot_m;
    if (!want_key) return;
    const unsigned long long tgt =
        by_mass && frac > 0.0 ? (unsigned long long)(frac * (double)tot_m) : target;
    if (tid == 0) {
        hs.sel = INT_MAX;
        hs.lastnz = -1;
        hs.n = 0;
    }
    __syncthreads();
    {
        unsigned long long cum = by_mass ? pre_m : pre_c;
        for (int i = 0; i < nb; ++i) {
            const int b = b0 + i;
            if (h.hc[b] == 0) continue;
            const unsigned long long amt = by_mass ? h.hm[b] : (unsigned long long)h.hc[b];
            if (by_mass ? (cum + amt > tgt) : (cum + amt >= tgt)) {
                atomicMin(&hs.sel, b);
                break;
            }
            cum += amt;
        }
        if (lastnz >= 0) atomicMax(&hs.lastnz, lastnz);
    }
    __syncthreads();
    int sel = hs.sel;
    const bool take_last = sel == INT_MAX;
    if (take_last) sel = hs.lastnz;
    if (sel < 0) {  // nothing satisfies pred
        key = 0;
        return;
    }
    if (sel >= b0 && sel < b0 + nb) {  // the owner records what precedes the bucket
        unsigned long long cum = by_mass ? pre_m : pre_c;
        for (int b = b0; b < sel; ++b) cum += by_mass ? h.hm[b] : (unsigned long long)h.hc[b];
        hs.cum = cum;
        hs.target = tgt;
        hs.total_count = (int)h.hc[sel];
    }
    __syncthreads();
    const int csel = hs.total_count;
    if (sel == HB || csel > HCAP) {
        key = radix_select(zr, V, zmax,
                           [kmin, wmin](unsigned long long k, float w) { return k >= kmin && (wmin <= 0.0f || w >= wmin); },
                           by_mass, tgt, su.r, sh);
        return;
    }
    const unsigned long long cum = hs.cum;
    __syncthreads();  // the histogram is dead from here: its memory holds the bucket
    SmemBucket& kb = su.k;
    row_visit(zr, V, [&](int v, float z) {
        if (!(z > NEG_INF) || hbucket(z, zmax, s2) != sel) return;
        float w;
        const unsigned long long kk = pass(v, z, w);
        if (!kk) return;
        const int slot = atomicAdd(&hs.n, 1);
        if (slot < HCAP) {  // the histogram counted exactly these entries
            kb.key[slot] = kk;
            kb.wq[slot] = wq(w);
        }
    });
    __syncthreads();
    const int n = min(hs.n, HCAP);
    if (tid == 0) hs.key = ~0ull;
    __syncthreads();
    if (take_last) {
        for (int i = tid; i < n; i += NTR) atomicMin(&hs.key, kb.key[i]);
    } else {
        // count and mass of the bucket's entries that precede entry i in key
        // order: G lanes of one wave share entry i, each over every G-th entry
        int G = 1;
        while (G < WAVE && n * (2 * G) <= NTR) G *= 2;
        const unsigned long long rem = tgt - cum;
        for (int base = 0; base < n; base += NTR / G) {  // the same trip count in every lane
            const int i = base + tid / G;
            const bool live = i < n;
            const unsigned long long ki = live ? kb.key[i] : 0ull;
            unsigned long long before = 0;
            if (live)
                for (int j = tid % G; j < n; j += G) {
                    const unsigned long long kj = kb.key[j];
                    if (kj > ki) before += by_mass ? kb.wq[j] : 1ull;
                }
            for (int o = 1; o < G; o <<= 1) {
                const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)before, o);
                const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(before >> 32), o);
                before += ((unsigned long long)hi << 32) | lo;
            }
            if (live && tid % G == 0) {
                const bool hit = by_mass ? (before <= rem && rem < before + kb.wq[i]) : (before + 1 == rem);
                if (hit) hs.key = ki;  // exactly one entry qualifies
            }
        }
    }
    __syncthreads();
    key = hs.key;
    __syncthreads();
}

// z of every entry of the row into scratch, by the whole workgroup: first from
// the raw logits and the mask alone, then the entries a history, draft or bias
// entry touches are formed again with their multiplicity and bias, through the
// same process_entry as every other path.
// Entry i of the concatenated history, draft and bias id lists.
__device__ __forceinline__ int list_id(const RowCtx& c, int nh, int i) {
    if (i < c.hist_len) return gld(c.hist + i);
    if (i < nh) return gld(c.extra + (i - c.hist_len));
    return gld(c.bias_ids + (i - nh));
}

// z again for each distinct id of the n list entries (LDS copy `ids` and the
// bias values in `bv`, or null to read them from memory), the vocabulary taken
// PCH entries at a time: the chunk's multiplicities and bias marks are counted
// in LDS from the whole list, then the first thread to claim an entry's flag
// forms its z (from memory) or, with the lists staged, appends it to a work
// list that is formed after the last chunk, all its loads in flight together.
// Chunks no list entry touches are skipped. Returns the least z it wrote.
template <int DT>
__device__ __forceinline__ float patch_entries(const RowCtx& c, float* zr, int nh, int n, SmemList& sl, bool staged) {
    const int tid = threadIdx.x;
    SmemPatch& pt = sl.pt;
    float lo = __builtin_huge_valf();
    auto id_at = [&](int i) { return staged ? sl.ids[i] : list_id(c, nh, i); };
    // x' of entry id from its raw logit, multiplicity and bias mark (the same
    // steps, in the same order, as process_entry)
    auto form = [&](int id, uint32_t cnt, bool hit) {
        const bool allowed = c.mask ? ((gld(c.mask + (id >> 5)) >> (id & 31)) & 1u) : true;
        float x = penalize(c, read_logit<DT>(c.logits, id), cnt);
        if (hit) {
            for (int k = 0; k < c.bias_len; ++k)
                if (id_at(nh + k) == id) x = x + (staged && k < BV_CAP ? sl.bvals[k] : gld(c.bias_vals + k));
        }
        x = allowed ? x : NEG_INF;
        const float z = x > NEG_INF ? canon_zero(x / c.T) : NEG_INF;
        zr[id] = z;
        if (z > NEG_INF) lo = fminf(lo, z);
    };
    const int nch = (c.V + PCH - 1) / PCH;
    if (tid < PMASKW) pt.touched[tid] = 0u;
    if (tid == 0) sl.nwork = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NTR) {
        const int id = id_at(i);
        if (id >= 0 && id < c.V) atomicOr(&pt.touched[(id / PCH) >> 5], 1u << ((id / PCH) & 31));
    }
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        if (!((pt.touched[ch >> 5] >> (ch & 31)) & 1u)) continue;  // uniform
        const int c0 = ch * PCH;
        for (int k = tid; k < PCH / 2; k += NTR) pt.cnt[k] = 0u;
        for (int k = tid; k < PCH / 32; k += NTR) {
            pt.bias[k] = 0u;
            pt.flag[k] = 0u;
        }
        __syncthreads();
        for (int i = tid; i < n; i += NTR) {
            const int l = id_at(i) - c0;
            if (l < 0 || l >= PCH || l + c0 >= c.V) continue;
            if (i < nh) atomicAdd(&pt.cnt[l >> 1], 1u << ((l & 1) * 16));
            else atomicOr(&pt.bias[l >> 5], 1u << (l & 31));
        }
        __syncthreads();
        for (int i = tid; i < n; i += NTR) {
            const int id = id_at(i);
            const int l = id - c0;
            if (l < 0 || l >= PCH || id >= c.V) continue;
            const uint32_t b = 1u << (l & 31);
            if (atomicOr(&pt.flag[l >> 5], b) & b) continue;  // another thread has it
            const uint32_t cnt = (pt.cnt[l >> 1] >> ((l & 1) * 16)) & 0xFFFFu;
            const bool hit = (pt.bias[l >> 5] & b) != 0u;
            if (staged) {
                // distinct ids number at most n <= LIST_CAP: the list cannot overflow
                sl.work[atomicAdd(&sl.nwork, 1)] = (uint32_t)i | (cnt << 13) | ((hit ? 1u : 0u) << 27);
            } else {
                form(id, cnt, hit);
            }
        }
        __syncthreads();  // the tables are cleared for the next chunk; the work list is whole
    }
    if (staged) {
        for (int w = tid; w < sl.nwork; w += NTR) {
            const uint32_t it = sl.work[w];
            form(sl.ids[it & 0x1FFFu], (it >> 13) & 0x3FFFu, (it >> 27) & 1u);
        }
    }
    return lo;
}

// Returns a lower bound of the row's finite z (+inf: none is finite): the
// least z written by either pass.
template <int DT>
__device__ __forceinline__ float row_z(const RowCtx& c, float* zr, SmemU& su, SmemR& sh) {
    const int tid = threadIdx.x;
    const int V = c.V;
    float lo = __builtin_huge_valf();
    // the raw pass: 16-byte loads of the aligned body, RQ in flight per
    // thread (the loop is bound by memory latency), single entries for the
    // unaligned head and the tail
    constexpr int VEC = Lay<DT>::VEC;
    constexpr int ES = DT == SS_F32 ? 4 : 2;
    auto one = [&](int v, float x, uint32_t mword) {
        const float xv = ((mword >> (v & 31)) & 1u) ? x : NEG_INF;
        const float z = xv > NEG_INF ? canon_zero(xv / c.T) : NEG_INF;
        zr[v] = z;
        if (z > NEG_INF) lo = fminf(lo, z);
    };
    auto mask_word = [&](int v) { return c.mask ? gld(c.mask + (v >> 5)) : 0xFFFFFFFFu; };
    const char* row = (const char*)c.logits;
    const int head = min(V, (int)(((16u - ((uint32_t)(uintptr_t)row & 15u)) & 15u) / ES));
    if (tid < head) one(tid, read_logit<DT>(c.logits, tid), mask_word(tid));
    const int nq = (V - head) / VEC;
    const uint4* q = (const uint4*)(row + (size_t)head * ES);
    for (int i0 = tid; i0 < nq; i0 += NTR * RQ) {
        uint4 t[RQ];
        uint32_t m0[RQ], m1[RQ];
#pragma unroll
        for (int k = 0; k < RQ; ++k) {
            const int i = i0 + k * NTR;
            const int v = head + VEC * min(i, nq - 1);
            t[k] = i < nq ? gld(q + i) : make_uint4(0, 0, 0, 0);
            m0[k] = mask_word(v);               // the group may straddle two mask words
            m1[k] = mask_word(v + VEC - 1);
        }
#pragma unroll
        for (int k = 0; k < RQ; ++k) {
            const int i = i0 + k * NTR;
            if (i >= nq) continue;
            const int v = head + VEC * i;
            float x[VEC];
            unpack_group<DT>(t[k], x);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                one(v + j, x[j], ((v + j) >> 5) == (v >> 5) ? m0[k] : m1[k]);
        }
    }
    for (int v = head + VEC * nq + tid; v < V; v += NTR) one(v, read_logit<DT>(c.logits, v), mask_word(v));
    const int nh = c.hist_len + c.extra_len;
    const int n = nh + c.bias_len;
    if (n > 0) {
        const bool staged = n <= LIST_CAP;
        if (staged) {
            for (int i = tid; i < n; i += NTR) su.l.ids[i] = list_id(c, nh, i);
            for (int k = tid; k < min(c.bias_len, BV_CAP); k += NTR) su.l.bvals[k] = gld(c.bias_vals + k);
        }
        __syncthreads();  // also orders the raw pass before the patches
        lo = fminf(lo, patch_entries<DT>(c, zr, nh, n, su.l, staged));
    }
    return -block_max(-lo, sh.red);  // its barriers also end the patches
}

// Exact whole-row resolution: z for the whole row into scratch, then select by
// count (top-k) and by mass (top-p, the draw) over bucket histograms of the
// distance below the row maximum.
template <int DT>
__device__ __forceinline__ void finalize_slow(const RowCtx& c, int row, const Workspace& ws,
                                           int n_tiles, const RowSummary& rs, float u, SmemU& su,
                                           SmemR& sh, RowInfo& info, const RowDbg& dbg) {
    const int tid = threadIdx.x;
    const int V = c.V;
    float* zr = ws.scratch_z + (size_t)row * V;
    const float zlo = row_z<DT>(c, zr, su, sh);
    const float zmax = canon_zero(rs.m / c.T);
    const float s2 = hdeep_scale(zmax, zlo);
    const int total = rs.nfinite;
    const bool topk_on = c.top_k > 0 && c.top_k < V;
    const int K_eff = topk_on ? min(c.top_k, total) : total;
    int cnt;
    unsigned long long ms;
    unsigned long long kK = 0;
    if (topk_on && K_eff < total)
        hist_select(zr, V, zmax, s2, true, 0ull, 0.0f, false, true, (unsigned long long)K_eff, 0.0, su, sh, cnt,
                    ms, kK);
    unsigned long long kP = kK;
    if (c.top_p < 1.0f)  // the first entry whose inclusive mass exceeds top_p x (top-k mass)
        hist_select(zr, V, zmax, s2, true, kK, 0.0f, true, true, 0, (double)c.top_p, su, sh, cnt, ms, kP);
    const float mp = c.min_p;
    auto kept = [kP, mp](unsigned long long k, float w) { return k >= kP && (mp <= 0.0f || w >= mp); };
    // the draw: the first kept entry whose inclusive mass exceeds u x (kept mass)
    int n_kept;
    unsigned long long Wk, kt;
    // min_p at or below the deepest nonzero fixed-point weight needs every w
    const bool dz = mp <= 0.0f || mp > 1e-13f;
    hist_select(zr, V, zmax, s2, dz, kP, mp, true, true, 0, (double)u, su, sh, n_kept, Wk, kt);
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


// Outcome of resolving a row on its sorted pool.
struct RowOut {
    unsigned long long kappa;
    double Wk;
    int n_kept;
    int token;
    int lim_list;
    int slow;
};

// Inclusive prefix mass of sorted-pool entry i (binary64).
__device__ __forceinline__ double pool_prefix(const SmemPool& P, int i) {
    return i < POOL / 2 ? P.P[i] : P.P2[i - POOL / 2];
}

// First index i in [0, lim) whose predicate holds (INT_MAX if none), 64
// entries per step; pred(i) reads only LDS.
template <class Pred>
__device__ __forceinline__ int wave_first(int lim, Pred pred) {
    const int lane = threadIdx.x & (WAVE - 1);
    for (int c0 = 0; c0 < lim; c0 += WAVE) {
        const int i = c0 + lane;
        const unsigned long long m = __ballot(i < lim && pred(i));
        if (m) return c0 + __ffsll((long long)m) - 1;
    }
    return INT_MAX;
}

// One wave answers top-k mass, top-p, min-p and the draw on the sorted pool
// F[0, n) from the weights w_i = exp(z_i - zmax) (binary32, as everywhere on
// this path) and their binary64 inclusive prefix sums, both already in LDS.
// W is the row mass (used when top-k does not cut) and err a bound on its
// error; missing: some tile's mass outside its candidates is not in W (rows
// cut by top-k only); every entry past the pool weighs at most exp(zb - zmax).
// slow = 1 when a request needs entries past the pool.
__device__ __forceinline__ RowOut resolve_wave(const SmemPool& P, int n, float zmax, float zb, double W,
                                               double err, bool missing, const RowCtx& c, float u, int K_eff,
                                               bool cut_k, int total, bool topk_on, bool want_probs,
                                               bool want_topk) {
    RowOut o;
    o.slow = 0;
    o.kappa = 0;
    o.Wk = W;
    o.n_kept = 0;
    o.token = -1;
    o.lim_list = cut_k ? K_eff : (topk_on ? total : 0);
    // mass of the top-k set; a top-k set deeper than the pool adds only
    // entries the caller has shown to be negligible
    double WK = W;
    unsigned long long kK = 0;
    if (cut_k) {
        WK = pool_prefix(P, min(K_eff, n) - 1);
        kK = K_eff <= n ? P.F[K_eff - 1] : 0ull;
        // A top-k set deeper than the pool takes the pool's mass as its own:
        // the K_eff - n entries it holds past the pool must weigh at most
        // TAIL_EPS of it. Each weighs at most exp(zb - zmax); where every tile
        // summed its mass outside the candidates, all entries past the pool
        // together weigh at most (W - WK) + err.
        if (K_eff > n) {
            double past = (double)(K_eff - n) * exp((double)zb - (double)zmax);
            if (!missing) past = fmin(past, (W - WK) + err);
            if (past > TAIL_EPS * WK) {
                o.slow = 1;
                return o;
            }
        }
    }
    // top-p: the first entry whose exclusive mass reaches top_p W_K
    const int lim_p = cut_k ? K_eff : total;
    int n_topp = lim_p;
    if (c.top_p < 1.0f) {
        const double thr = (double)c.top_p * WK;
        const int fp = wave_first(min(n, lim_p), [&](int i) { return i > 0 && pool_prefix(P, i - 1) >= thr; });
        if (fp != INT_MAX) n_topp = fp;
        else if (lim_p > n) o.slow = 1;
    }
    // min-p: the first entry with w < min_p (w is non-increasing along the
    // pool up to rounding; entries near the cut are boundary cases)
    int n_kept = n_topp;
    if (!o.slow && c.min_p > 0.0f) {
        const int fm = wave_first(min(n, n_topp), [&](int i) { return P.w[i] < c.min_p; });
        if (fm != INT_MAX) {
            n_kept = fm;
        } else if (n_topp > n) {
            // every pool entry passes min-p; one past the pool passes only if
            // its weight, at most exp(zb - zmax), could reach min_p
            if ((double)c.min_p > exp((double)zb - (double)zmax)) n_kept = n;
            else o.slow = 1;
        }
    }
    if (o.slow) return o;
    // kept mass and the cut key (0: every finite entry, or a top-k set deeper
    // than the pool)
    double Wk;
    unsigned long long kappa;
    if (n_kept == total) {
        Wk = W;
        kappa = 0;
    } else if (cut_k && n_kept == K_eff) {
        Wk = WK;
        kappa = kK;
    } else {
        Wk = pool_prefix(P, n_kept - 1);
        kappa = P.F[n_kept - 1];
    }
    // the draw: first kept entry whose inclusive mass exceeds u Wk
    const double tgt = (double)u * Wk;
    const int lim = min(n, n_kept);
    const int fd = wave_first(lim, [&](int i) { return pool_prefix(P, i) > tgt; });
    const int pick = fd != INT_MAX ? fd : (n_kept <= n ? n_kept - 1 : -1);
    if (pick < 0 || (want_probs && n_kept > n) || (want_topk && o.lim_list > n)) {
        o.slow = 1;
        return o;
    }
    o.kappa = kappa;
    o.Wk = Wk;
    o.n_kept = n_kept;
    o.token = key64_id(P.F[pick]);
    return o;
}

// The largest binary32 x with RN(x / T) <= c (c finite, T > 0): x / T is
// correctly rounded, so RN(x / T) <= c holds exactly for x up to that value.
// A 65-way search over the ordered bit patterns of the non-NaN floats, one
// wave: each step tests 64 points of (lo, hi) at once, P(lo) true and P(hi)
// false throughout.
__device__ __forceinline__ float x_at_most(float c, float T) {
    const int lane = threadIdx.x & (WAVE - 1);
    auto ord = [](float x) {
        const uint32_t b = __float_as_uint(x);
        return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    };
    auto unord = [](uint32_t u) { return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u); };
    const uint32_t olo = ord(NEG_INF), ohi = ord(__builtin_huge_valf());
    {
        // the answer lies within a few units in the last place of c T unless
        // that product over- or underflows: 64 consecutive floats around it
        const uint32_t g = ord(c * T);
        const uint32_t p = min(max(g, olo + 32u) - 32u + (uint32_t)lane, ohi);
        const unsigned long long ok = __ballot(unord(p) / T <= c);
        const int k = __popcll(ok);
        if (k > 0 && k < WAVE && (ok & 1ull)) return unord(__builtin_amdgcn_readlane(p, k - 1));
    }
    uint32_t lo = olo, hi = ohi;
    while (hi - lo > 1) {
        const uint32_t p = lo + (uint32_t)(((unsigned long long)(hi - lo) * (unsigned)(lane + 1)) / (WAVE + 1));
        const unsigned long long ok = __ballot(p == lo || unord(p) / T <= c);  // monotone in lane
        const int k = __popcll(ok);  // lanes 0 .. k-1 hold points where P holds
        const uint32_t nlo = __builtin_amdgcn_readlane(p, max(k - 1, 0));
        const uint32_t nhi = k < WAVE ? __builtin_amdgcn_readlane(p, min(k, WAVE - 1)) : hi;
        lo = k > 0 ? nlo : lo;
        hi = nhi;
    }
    return unord(lo);
}

// The SAMPLE draw of an unfiltered row (no top-k, top-p or min-p) without
// penalty or bias tables, when the draw lies past the pool's mass. Entries
// above zb (the pool) come first in key order; every other entry has z <= zb
// and lies in row bin floor(-z BIN_S) - floor(-zb BIN_S), which does not
// decrease along key order. The row bins' masses come from stage 1's bins of
// the count-cut wave tiles (scaled to zmax), the candidates at or below zb, and
// the entries of every other wave tile that leaves entries outside its
// candidates (at most UBCAP such tiles), formed again from the logits. The bin
// that holds u W is then searched entry by entry: one pass over the row
// collects its entries (by the range of x that maps into the bin's range of z),
// their masses by sub-bin give the sub-bin, and pairwise ranks in the sub-bin
// give the entry. Masses are binary32 weights summed in binary64, as on the
// pool path. Returns false, leaving the row to the whole-row path, when the bin
// also holds a tile's deepest bin (whose entries may lie deeper), when the bin
// holds more than BCAP entries or its sub-bin more than SBCAP, or when more
// than UBCAP wave tiles lack bins.
template <int DT>
__device__ __forceinline__ bool bin_draw(const RowCtx& c, int row, const Workspace& ws, const RowView& rv, float u,
                                         int total, SmemBins& B, RowInfo& out) {
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    if (__popcll(rv.ub[0]) + __popcll(rv.ub[1]) > UBCAP) return false;  // uniform
    const float zmax = rv.zmax, zb = rv.zb;
    const float atop = floorf(-zb * (float)BIN_S);
    auto rbin = [&](float z) { return (int)fminf(floorf(-z * (float)BIN_S) - atop, (float)(NRB - 1)); };
    auto unbinned = [&](int wt) { return (rv.ub[wt >> 6] >> (wt & 63)) & 1ull; };
    const int n_wt = ws.n_wt;
    const WaveStat* stats = ws.wstats + (size_t)row * n_wt;
    // the wave tiles' bins: where each starts among the row bins, its scale
    if (tid < n_wt) {
        const WaveStat st = stats[tid];
        const bool has = st.flags & WS_BIN;
        B.toff[tid] = has ? (int)fminf(floorf(-st.zbeta * (float)BIN_S) - atop, (float)NRB) : INT_MAX;
        B.tscale[tid] = has ? expf(st.zm - zmax) : 0.0f;
        B.tnc[tid] = st.ncand;
    }
    for (int i = tid; i < NRB; i += NTR) B.rb[i] = 0.0;
    if (tid < NSB) B.sb[tid] = 0.0;
    if (tid == 0) B.n = 0;
    __syncthreads();
    // the tiles' bins, scaled to zmax, onto the row bins (the last row bin also
    // takes everything deeper); all loads of a thread in flight at once
    {
        const float* bins = ws.bins + (size_t)row * n_wt * NBIN;
        const int nb = n_wt * NBIN;
        constexpr int UB = MAX_WT * NBIN / NTR;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (g == 1 && nb <= (UB / 2) * NTR) break;  // uniform
            float m[UB / 2];
#pragma unroll
            for (int k = 0; k < UB / 2; ++k) {
                const int i = tid + (g * (UB / 2) + k) * NTR;
                m[k] = i < nb ? gld(bins + i) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < UB / 2; ++k) {
                const int i = tid + (g * (UB / 2) + k) * NTR;
                if (m[k] > 0.0f) {
                    const int off = B.toff[i / NBIN];
                    if (off != INT_MAX)
                        atomicAdd(&B.rb[min(off + i % NBIN, NRB - 1)], (double)m[k] * (double)B.tscale[i / NBIN]);
                }
            }
        }
    }
    // the candidates (read again: the merge's copy is not kept this long): the
    // pool's mass, and the bins of those at or below zb (a wave tile without
    // bins gives all its entries below)
    double wp = 0.0;
    {
        const unsigned long long* cand = ws.cand + (size_t)row * n_wt * WCAP;
        static_assert(NTR % WCAP == 0, "a thread keeps its lane of the candidate lists");
        unsigned long long kc[MSLOT];
#pragma unroll
        for (int k = 0; k < MSLOT; ++k) {
            const int wt = wv + NWR * k;
            kc[k] = wt < n_wt && lane < B.tnc[wt] ? gld(cand + (size_t)wt * WCAP + lane) : 0ull;
        }
#pragma unroll
        for (int k = 0; k < MSLOT; ++k) {
            const int wt = wv + NWR * k;
            if (kc[k] != 0ull) {
                const float z = key_z(kc[k]);
                const double w = (double)expf(z - zmax);
                if (z > zb) wp += w;
                else if (!unbinned(wt)) atomicAdd(&B.rb[rbin(z)], w);
            }
        }
    }
    // wave tiles without bins: every entry at or below zb, from the logits
    // (the wave tile's entries: WAVE VEC consecutive ids per group of the tile)
    {
        constexpr int VEC = Lay<DT>::VEC;
        static_assert(WT == 2 * NTR, "two entries of a wave tile per thread");
        for (int h = 0; h < 2; ++h) {
            unsigned long long m = rv.ub[h];
            while (m) {
                const int wt = h * WAVE + (int)__builtin_ctzll(m);
                m &= m - 1;
                const int tb = (wt / WPT) * TILE + (wt % WPT) * (WAVE * VEC);
#pragma unroll
                for (int e0 = 0; e0 < 2; ++e0) {
                    const int e = tid + e0 * NTR;
                    const int id = tb + (e / (WAVE * VEC)) * Lay<DT>::GSTRIDE + e % (WAVE * VEC);
                    if (id >= c.V) continue;
                    if (c.mask && !((gld(c.mask + (id >> 5)) >> (id & 31)) & 1u)) continue;
                    const float x = read_logit<DT>(c.logits, id);
                    if (!(x > NEG_INF)) continue;
                    const float z = canon_zero(x / c.T);
                    if (z <= zb) atomicAdd(&B.rb[rbin(z)], (double)expf(z - zmax));
                }
            }
        }
    }
    wp = wave_sum_d(wp);
    if (lane == 0) B.part[wv] = wp;
    __syncthreads();
    // wave 0: the row's mass, the draw's target, the bin that holds it and
    // the range of x that maps into that bin
    if (wv == 0) {
        double Wp = 0.0;
#pragma unroll
        for (int w = 0; w < NWR; ++w) Wp += B.part[w];
        constexpr int PER = NRB / WAVE;
        // lane l sums bins l PER .. l PER + PER - 1 (read in a rotated order:
        // the lanes then meet different LDS banks)
        double loc = 0.0;
#pragma unroll
        for (int k = 0; k < PER; ++k) loc += B.rb[lane * PER + ((k + lane) & (PER - 1))];
        const double inc = wave_incl_scan_d(loc);
        const double W = Wp + __shfl(inc, WAVE - 1);
        const double tgt = (double)u * W;
        const double before = Wp + inc - loc;  // mass above this lane's first bin
        // the lane whose bins hold the target, then the bin within them
        const unsigned long long hit = __ballot(before <= tgt && tgt < before + loc && loc > 0.0);
        int beta = -1;
        double base = 0.0;
        if (hit) {
            // that lane's bins, one per lane: the first non-empty one whose
            // inclusive mass passes the target
            const int l0 = (int)__builtin_ctzll(hit);
            const double b0 = __shfl(before, l0);
            const double m = lane < PER ? B.rb[l0 * PER + lane] : 0.0;
            const double run = b0 + wave_incl_scan_d(m);
            const unsigned long long h2 = __ballot(lane < PER && m > 0.0 && tgt < run);
            if (h2) {
                const int k = (int)__builtin_ctzll(h2);
                beta = l0 * PER + k;
                base = __shfl(run - m, k);
            }
        }
        // row bins from the shallowest tile's deepest bin on may hold deeper entries
        int deep = NRB - 1;
        for (int t = lane; t < n_wt; t += WAVE) {
            const int off = B.toff[t];
            if (off != INT_MAX) deep = min(deep, off + NBIN - 1);
        }
        deep = wave_min_i(deep);
        beta = (beta >= 0 && beta < deep && tgt >= Wp) ? beta : -1;
        float xlo = 0.0f, xhi = 0.0f;
        if (beta >= 0) {
            // bin beta is z in (-(atop + beta + 1) / BIN_S, -(atop + beta) / BIN_S]
            // (exact: integers below 2^24 over a power of two)
            xhi = x_at_most(fminf(-(atop + (float)beta) / (float)BIN_S, zb), c.T);
            xlo = x_at_most(-(atop + (float)(beta + 1)) / (float)BIN_S, c.T);
        }
        if (lane == 0) {
            B.beta = beta;
            B.base = base;
            B.tgt = tgt;
            B.part[0] = W;
            B.xlo = xlo;
            B.xhi = xhi;
        }
    }
    __syncthreads();
    const int beta = B.beta;
    if (beta < 0) return false;
    const float xlo = B.xlo, xhi = B.xhi;
    // one pass over the row: the entries of bin beta
    const char* rowp = (const char*)c.logits;
    constexpr int VEC = Lay<DT>::VEC;
    constexpr int ES = DT == SS_F32 ? 4 : 2;
    // (ids only: their keys, and the grammar mask, come after the pass)
    auto visit = [&](int v, float x) {
        if (!(x > xlo && x <= xhi)) return;
        const int slot = atomicAdd(&B.n, 1);
        if (slot < BCAP) B.key[slot] = (unsigned long long)v;
    };
    const int V = c.V;
    const int head = min(V, (int)(((16u - ((uint32_t)(uintptr_t)rowp & 15u)) & 15u) / ES));
    if (tid < head) visit(tid, read_logit<DT>(c.logits, tid));
    const int nq = (V - head) / VEC;
    const uint4* q = (const uint4*)(rowp + (size_t)head * ES);
    // One workgroup per row: 64 entries per thread in flight (16-byte loads),
    // tested into a bit mask without branches; the few entries in range leave
    // their ids.
    constexpr int RC = 64 / VEC;
    for (int i0 = tid; i0 < nq; i0 += NTR * RC) {
        uint4 t[RC];
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            const int i = i0 + k * NTR;
            t[k] = i < nq ? gld(q + i) : make_uint4(0, 0, 0, 0);
        }
        unsigned long long hm = 0;
#pragma unroll
        for (int k = 0; k < RC; ++k) {
            float x[VEC];
            unpack_group<DT>(t[k], x);
            uint32_t b = 0;
#pragma unroll
            for (int j = 0; j < VEC; ++j) b |= (x[j] > xlo && x[j] <= xhi) ? 1u << j : 0u;
            if (i0 + k * NTR >= nq) b = 0;
            hm |= (unsigned long long)b << (k * VEC);
        }
        if (hm) {
            int slot = atomicAdd(&B.n, __popcll(hm));
            for (; hm; hm &= hm - 1, ++slot) {
                const int bit = (int)__builtin_ctzll(hm);
                if (slot < BCAP) B.key[slot] = (unsigned long long)(head + VEC * (i0 + (bit / VEC) * NTR) + bit % VEC);
            }
        }
    }
    for (int v = head + VEC * nq + tid; v < V; v += NTR) visit(v, read_logit<DT>(c.logits, v));
    __syncthreads();
    const int n = B.n;
    if (n > BCAP || n == 0) return false;
    // sub-bins of bin beta (monotone in key order), their masses, and the one
    // that holds the target
    const float sb0 = (atop + (float)beta) * (float)NSB;
    auto sbin = [&](float z) {
        return (int)fminf(fmaxf(floorf(-z * (float)(BIN_S * NSB)) - sb0, 0.0f), (float)(NSB - 1));
    };
    // each collected id becomes its key (0: not allowed by the grammar mask;
    // no finite z has key 0) and adds its mass to its sub-bin
    for (int i0 = tid; i0 < n; i0 += 4 * NTR) {
        int v[4];
        float x[4];
        bool ok[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + k * NTR;
            v[k] = i < n ? (int)B.key[i] : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = read_logit<DT>(c.logits, v[k]);
            ok[k] = !c.mask || ((gld(c.mask + (v[k] >> 5)) >> (v[k] & 31)) & 1u);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + k * NTR;
            if (i >= n) continue;
            const float z = canon_zero(x[k] / c.T);
            B.key[i] = ok[k] ? key64(z, v[k]) : 0ull;
            if (ok[k]) atomicAdd(&B.sb[sbin(z)], (double)expf(z - zmax));
        }
    }
    __syncthreads();
    if (wv == 0) {
        const double m = B.sb[lane];
        const double inc = wave_incl_scan_d(m);
        const double before = B.base + inc - m;
        const double tgt = B.tgt;
        const unsigned long long hit = __ballot(m > 0.0 && before <= tgt && tgt < before + m);
        const unsigned long long nz = __ballot(m > 0.0);
        // past every sub-bin (rounding of the bins' masses): the last one
        const int sub = hit ? (int)__builtin_ctzll(hit) : nz ? 63 - (int)__builtin_clzll(nz) : -1;
        const double sbase = __shfl(before, max(sub, 0));
        if (lane == 0) {
            B.sub = sub;
            B.base = sbase;
            B.ns = 0;
            B.pick = -1;
        }
    }
    __syncthreads();
    const int sub = B.sub;
    if (sub < 0) return false;
    const double sbase = B.base, tgt = B.tgt;
    // the sub-bin's entries, then the first of them in key order whose
    // inclusive mass passes the target (else the last of them)
    for (int i = tid; i < n; i += NTR) {
        const unsigned long long ki = B.key[i];
        if (ki != 0 && sbin(key_z(ki)) == sub) {
            const int slot = atomicAdd(&B.ns, 1);
            if (slot < SBCAP) B.sk[slot] = ki;
        }
    }
    __syncthreads();
    const int ns = B.ns;
    if (ns > SBCAP) return false;
    if (ns <= WAVE) {
        // one entry per lane, the others' keys and weights by lane reads
        if (wv == 0) {
            const unsigned long long ki = lane < ns ? B.sk[lane] : 0ull;
            const double wi = lane < ns ? (double)expf(key_z(ki) - zmax) : 0.0;
            double before = sbase;
            int below = 0;
            for (int j = 0; j < ns; ++j) {
                const unsigned long long kj = ((unsigned long long)__builtin_amdgcn_readlane((uint32_t)(ki >> 32), j) << 32) |
                                              (uint32_t)__builtin_amdgcn_readlane((uint32_t)ki, j);
                const double wj = __shfl(wi, j);
                if (kj > ki) before += wj;
                below += kj < ki ? 1 : 0;
            }
            const bool pass = lane < ns && before <= tgt && tgt < before + wi;
            const bool last = lane < ns && below == 0 && !(tgt < before + wi);
            const unsigned long long pm = __ballot(pass), lm = __ballot(last);
            if (lane == 0) B.pick = pm ? SBCAP + 63 - (int)__builtin_clzll(pm) : lm ? (int)__builtin_ctzll(lm) : -1;
        }
    } else for (int i = tid; i < ns; i += NTR) {
        const unsigned long long ki = B.sk[i];
        double before = sbase;
        int below = 0;
        for (int j = 0; j < ns; ++j) {
            const unsigned long long kj = B.sk[j];
            if (kj > ki) before += (double)expf(key_z(kj) - zmax);
            below += kj < ki ? 1 : 0;
        }
        const double wi = (double)expf(key_z(ki) - zmax);
        // exactly one entry passes; without one the target lies past the
        // sub-bin's mass (rounding of the bins) and the last entry is taken
        if (before <= tgt && tgt < before + wi) atomicMax(&B.pick, SBCAP + i);
        else if (below == 0 && !(tgt < before + wi)) atomicMax(&B.pick, i);
    }
    __syncthreads();
    const int pick = B.pick;
    if (pick < 0) return false;
    out.token = key64_id(B.sk[pick >= SBCAP ? pick - SBCAP : pick]);
    out.kappa = 0;
    out.W = B.part[0];
    out.zmax = zmax;
    out.min_p = 0.0f;
    out.n_kept = total;
    out.argmax = -1;
    out.path = 2;
    return true;
}

// BINS: the binned tail draw of unfiltered rows (the SAMPLE draw only)
template <int DT, bool BINS>
__device__ __forceinline__ void finalize_row(const RowCtx& c, int row, const Workspace& ws,
                                             const RowLoad& rl, SmemU& su, SmemR& sh,
                                             const RowDbg& dbg, RowInfo& info_out) {
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int V = c.V;
    SmemPool& P = su.p;
    RowSummary rs;
    rs.m = wave_max(fmaxf(rl.s0.m, rl.s1.m));
    rs.nfinite = wave_sum_i(rl.s0.nfinite + rl.s1.nfinite);

    __shared__ RowInfo info;
    if (c.T == 0.0f || !(rs.m > NEG_INF)) {
        const int am = rs.m > NEG_INF ? row_argmax(rl, rs.m) : -1;
        RowInfo r;
        r.kappa = 0;
        r.W = 1.0;
        r.zmax = rs.m;
        r.min_p = 0.0f;
        r.n_kept = am >= 0 ? 1 : 0;
        r.token = am;
        r.argmax = am;
        r.path = 0;
        if (dbg.topk)
            for (int i = tid; i < dbg.topk_stride; i += NTR) dbg.topk[i] = -1;
        if (tid == 0) {
            if (dbg.probs && am >= 0) dbg.probs[am] = 1.0f;
            if (dbg.kept) *dbg.kept = r.n_kept;
            if (dbg.path) *dbg.path = 0;
        }
        info_out = r;
        return;
    }
    // the draw's uniform, formed while the row's loads are in flight
    const float u = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_SAMPLE));
    // the row view, formed by wave 0 alone (sixteen waves forming it side by
    // side on four SIMDs took longer than the exchange) and shared through LDS
    __shared__ RowView s_rv;
    if (wv == 0) {
        const RowView r = row_view(rl, rs.m, c.T);
        if (lane == 0) s_rv = r;
    }
    __syncthreads();
    const RowView rv = s_rv;
    const float zmax = rv.zmax;
    const uint32_t mzb = mono32(rv.zb);

    // The pool: every candidate with z above zb. It is an exact prefix of the
    // row in key order (no entry outside the candidates lies above zb). Each
    // wave appends its pool entries, one ballot per slot round, to its own
    // region of A (A shares storage with F, which is written only after every
    // read of A).
    unsigned long long* A = P.F;
    unsigned long long* Aw = A + wv * AREG;
    int cw = 0;
#pragma unroll
    for (int k = 0; k < MSLOT; ++k) {
        const int wt = wv + NWR * k;
        if (wt < ws.n_wt) {
            const int nc = stat_ncand(rl, wt);
            const bool inp = lane < nc && (uint32_t)(rl.cv[k] >> 32) > mzb;
            const unsigned long long bm = __ballot(inp);
            if (bm) {
                const int p = cw + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
                if (inp && p < AREG) Aw[p] = rl.cv[k];
                cw += __popcll(bm);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < BKPT; ++j) P.cnt[tid * BKPT + j] = 0u;
    if (lane == 0) sh.red.i[wv] = cw;
    __syncthreads();
    // wave w's entries occupy A[w AREG, w AREG + cnt_w); entry j of the pool in
    // wave order sits in region r at j - (entries of the regions before r)
    // off[w]: entries of the regions before region w (uniform)
    int n = 0, regmax = 0;
    int off[NWR];
#pragma unroll
    for (int w = 0; w < NWR; ++w) {
        const int cw_w = __builtin_amdgcn_readfirstlane(sh.red.i[w]);
        off[w] = n;
        n += cw_w;
        regmax = max(regmax, cw_w);
    }
    auto pool_entry = [&](int j) -> unsigned long long {
        int r = 0, base = 0;
#pragma unroll
        for (int w = 1; w < NWR; ++w) {
            const bool past = j >= off[w];
            r += past ? 1 : 0;
            base = past ? off[w] : base;
        }
        return A[r * AREG + (j - base)];
    };
    const float zlo = rv.zlo;
    const double W = rv.W;
    const int total = rs.nfinite;
    const bool topk_on = c.top_k > 0 && c.top_k < V;
    const int K_eff = topk_on ? min(c.top_k, total) : total;
    const bool cut_k = topk_on && K_eff < total;
    bool slow = n == 0 || regmax > AREG || (rv.missing != 0 && !cut_k);
    // An uncut row's normaliser must be accurate: a relative error e of W moves
    // every probability and every CDF breakpoint by at most e, and the parity
    // rule allows 1e-6. (A top-k set deeper than the pool is checked once the
    // pool's mass is known.)
    if (!slow && !cut_k) slow = rv.err > 5e-7 * W;
    // An uncut row whose draw (no top-p, no min-p) or top-p cut lies deeper
    // than all the candidates' mass cannot resolve on the pool: skip building
    // it. (The margin covers the binary32 scaling of each tile's candidate sum.)
    if (!slow && !cut_k && c.min_p <= 0.0f) {
        const double need = c.top_p < 1.0f ? (double)c.top_p * W : (double)u * W;
        slow = need > rv.Wc * (1.0 + 1e-5);
    }

    if (!slow) {
        if (n <= WAVE) {
            // A pool of one wave's size: wave 0 sorts it in registers (a bitonic
            // network over lane exchanges) and forms its weights and binary64
            // prefix masses; it alone reads them, so no barrier follows.
            if (wv == 0) {
                unsigned long long key = lane < n ? pool_entry(lane) : 0ull;
                key = wave_sort_desc_u64(key);  // zero keys (empty lanes) sort last
                const float w = lane < n ? expf(key_z(key) - zmax) : 0.0f;
                const double pre = wave_incl_scan_d((double)w);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                if (lane < n) {
                    P.F[lane] = key;
                    P.w[lane] = w;
                    P.P[lane] = pre;
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
        } else {
            // Counting sort by bucket b = (zmax - z) S, non-decreasing along key
            // order, then each entry's rank among its bucket's entries.
            const float R = zmax - zlo;
            const float S = R > 0.0f ? fminf((float)NBK / R, 3.0e38f) : 0.0f;
            unsigned long long key[EPTR];
            int bkt[EPTR], arr[EPTR];
#pragma unroll
            for (int j = 0; j < EPTR; ++j) {
                const int e = tid + j * NTR;
                key[j] = 0ull;
                bkt[j] = 0;
                arr[j] = 0;
                if (e < n) {
                    key[j] = pool_entry(e);
                    bkt[j] = (int)fminf((zmax - key_z(key[j])) * S, (float)(NBK - 1));
                    arr[j] = (int)atomicAdd(&P.cnt[bkt[j]], 1u);
                }
            }
            __syncthreads();
            {
                uint32_t cb[BKPT];
                int tot = 0, mx = 0;
#pragma unroll
                for (int j = 0; j < BKPT; ++j) {
                    cb[j] = P.cnt[tid * BKPT + j];
                    tot += (int)cb[j];
                    mx = max(mx, (int)cb[j]);
                }
                const int inc = wave_incl_scan_i(tot);
                const int wmx = wave_max_i(mx);
                if (lane == WAVE - 1) sh.red2.i[wv] = inc;
                if (lane == 0) sh.imax[wv] = wmx;
                __syncthreads();
                int base = inc - tot, bmax = 0;
#pragma unroll
                for (int w = 0; w < NWR; ++w) {
                    base += w < wv ? sh.red2.i[w] : 0;
                    bmax = max(bmax, sh.imax[w]);
                }
#pragma unroll
                for (int j = 0; j < BKPT; ++j) {
                    P.start[tid * BKPT + j] = (uint32_t)base;
                    base += (int)cb[j];
                }
                slow = bmax > BK_MAX;
            }
            __syncthreads();
            if (!slow) {
#pragma unroll
                for (int j = 0; j < EPTR; ++j)
                    if (tid + j * NTR < n) P.bk[P.start[bkt[j]] + arr[j]] = key[j];
                __syncthreads();
#pragma unroll
                for (int j = 0; j < EPTR; ++j) {
                    if (tid + j * NTR < n) {
                        const int s0 = (int)P.start[bkt[j]], cbk = (int)P.cnt[bkt[j]];
                        int r = 0;
                        for (int q = 0; q < cbk; ++q) r += P.bk[s0 + q] > key[j] ? 1 : 0;
                        P.F[s0 + r] = key[j];
                    }
                }
                __syncthreads();
                // Weights and binary64 inclusive prefix masses of the sorted pool
                // (each thread sums EPTR consecutive entries, then the thread
                // totals are scanned in thread order); the bucket arrays they
                // overwrite are dead. A pool of up to EPTR waves' worth of
                // entries is summed by wave 0 alone, which also resolves the
                // row, so no barrier follows.
                if (n <= EPTR * WAVE) {
                    if (wv == 0) {
                        float wl[EPTR];
                        double run = 0.0, pre[EPTR];
#pragma unroll
                        for (int j = 0; j < EPTR; ++j) {
                            const int i = lane * EPTR + j;
                            wl[j] = i < n ? expf(key_z(P.F[i]) - zmax) : 0.0f;
                            run += (double)wl[j];
                            pre[j] = run;
                        }
                        const double base = wave_incl_scan_d(run) - run;
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
                        for (int j = 0; j < EPTR; ++j) {
                            const int i = lane * EPTR + j;
                            if (i < n) {
                                P.w[i] = wl[j];
                                P.P[i] = base + pre[j];
                            }
                        }
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    }
                } else {
                float wl[EPTR];
                double pre[EPTR];
                double run = 0.0;
#pragma unroll
                for (int j = 0; j < EPTR; ++j) {
                    const int i = tid * EPTR + j;
                    wl[j] = i < n ? expf(key_z(P.F[i]) - zmax) : 0.0f;
                    run += (double)wl[j];
                    pre[j] = run;
                }
                double tot;
                const double base = block_excl_scan_d(run, sh.red, tot);
#pragma unroll
                for (int j = 0; j < EPTR; ++j) {
                    const int i = tid * EPTR + j;
                    if (i < n) {
                        P.w[i] = wl[j];
                        if (i < POOL / 2) P.P[i] = base + pre[j];
                        else P.P2[i - POOL / 2] = base + pre[j];
                    }
                }
                __syncthreads();
                }
            }
        }
    }
    if (!slow) {
        const unsigned long long* F = P.F;
        __shared__ RowOut s_out;
        if (wv == 0) {
            const RowOut o = resolve_wave(P, n, zmax, rv.zb, W, rv.err, rv.missing != 0, c, u, K_eff, cut_k,
                                          total, topk_on,
                                          dbg.probs != nullptr, dbg.topk != nullptr);
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
                    dbg.probs[key64_id(F[i])] = (float)((double)P.w[i] / o.Wk);
            if (dbg.topk)
                for (int i = tid; i < dbg.topk_stride; i += NTR)
                    dbg.topk[i] = i < o.lim_list ? key64_id(F[i]) : -1;
            info_out = r;
            return;
        }
    }
    // an unfiltered row without penalty or bias tables whose draw lies past
    // its pool: the binned tail
    if (BINS && (c.top_k <= 0 || c.top_k >= V)) {
        // (laid out apart from the hot path: most rows never come here)
        if (__builtin_expect(c.top_p >= 1.0f && c.min_p <= 0.0f && c.hist_len + c.extra_len + c.bias_len == 0 &&
                                 !dbg.probs && !dbg.topk && ws.bins && rv.zb > NEG_INF &&
                                 fabsf(rv.zb) < 0x1p18f,  // bins near zb are exact integers in binary32
                             0)) {
            RowInfo r;
            const bool done = bin_draw<DT>(c, row, ws, s_rv, u, rs.nfinite, su.b, r);  // the view read again from LDS
            __syncthreads();  // every thread has read the outcome before the LDS is reused
            if (done) {
                if (tid == 0) {
                    if (dbg.kept) *dbg.kept = r.n_kept;
                    if (dbg.path) *dbg.path = 2;
                }
                info_out = r;
                return;
            }
        }
    }
    finalize_slow<DT>(c, row, ws, ws.n_tiles, rs, u, su, sh, info, dbg);
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

// Tile kernels: six 256-thread workgroups per CU (about 23 KB of LDS each);
// the register budget is held to six waves per SIMD, which keeps the tile's 32
// values per lane and the window passes in registers without spilling.
#define SS_TILE_OCC __attribute__((amdgpu_waves_per_eu(6)))

// BINS: kernels that keep binned tails for unfiltered rows (batches without
// penalty or bias lists: rows with lists never use them)
template <int DT, bool ALIGNED, bool BINS>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_sample_tiles(SampleArgs a) {
    __shared__ SmemTile tt;
    const int n_tiles = a.ws.n_tiles;
    const int lin = xcd_linear(a.B * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const RowCtx c = sample_ctx<DT>(a, row);
    tile_stage1<DT, ALIGNED, BINS>(c, row, tile, a.ws, tt,
                    a.dbg_processed ? a.dbg_processed + (size_t)row * a.V : nullptr,
                    a.dbg_probs ? a.dbg_probs + (size_t)row * a.V : nullptr);
}

template <int DT, bool BINS>
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
    finalize_row<DT, BINS>(c, row, a.ws, rl, su, sh, dbg, info);
    if (threadIdx.x == 0) a.out_tokens[row] = info.token;
}

// Verification, stage 1 over every target row of every request.
template <int DT, bool ALIGNED>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_spec_tiles(SpecArgs a) {
    __shared__ SmemTile tt;
    const int n_tiles = a.ws.n_tiles;
    const int G1 = a.G + 1;
    const int lin = xcd_linear(a.B * G1 * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const RowCtx c = spec_ctx<DT>(a, row / G1, row % G1);
    tile_stage1<DT, ALIGNED, false>(c, row, tile, a.ws, tt, nullptr, nullptr);
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
    finalize_row<DT, false>(c, row, a.ws, rl, su, sh, dbg, info);
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
            // a greedy draft puts all its mass on d
            const double q = a.draft_probs
                                 ? (double)a.draft_probs[((size_t)b * a.G + j) * a.draft_stride + d]
                                 : 1.0;
            const float ua = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_ACCEPT));
            acc = q > 0.0 ? ((double)ua < pi / q ? 1 : 0) : (pi > 0.0 ? 1 : 0);
        }
        if (threadIdx.x == 0) a.ws.row_accept[row] = acc;
    }
    if (threadIdx.x == 0) a.ws.rowinfo[row] = info;
}

// Accepted draft count of request b: the first rejected position, or G. Lane k
// of each wave reads position k's decision (G <= 16), so the loads overlap.
__device__ __forceinline__ int accepted_prefix(const SpecArgs& a, int b) {
    const int lane = threadIdx.x & (WAVE - 1);
    const bool rej = lane < a.G && !a.ws.row_accept[(size_t)b * (a.G + 1) + lane];
    const unsigned long long m = __ballot(rej);
    return m ? (int)__builtin_ctzll(m) : a.G;
}

// Position of request b whose token comes from the residual distribution, or -1.
__device__ __forceinline__ int residual_position(const SpecArgs& a, int b, RowInfo& ri) {
    const int n = accepted_prefix(a, b);
    ri = a.ws.rowinfo[(size_t)b * (a.G + 1) + n];
    if (n == a.G || a.p.temperature[b] == 0.0f || ri.n_kept == 0) return -1;
    return n;
}

// pi(v) of the filtered distribution described by ri, for processed logit x
// (invW = 1 / ri.W: the binary64 product differs from the quotient by at most
// one unit in its last place, far below the binary32 rounding of pi).
// (P2: T is a power of two, and x' / T the exact product x' rT.)
template <bool P2>
__device__ __forceinline__ float filtered_prob(const RowCtx& c, const RowInfo& ri, double invW, float rT, int id,
                                               float x) {
    if (!(x > NEG_INF)) return 0.0f;
    const float z = canon_zero(P2 ? x * rT : x / c.T);
    const float w = expf(z - ri.zmax);
    const bool kept = key64(z, id) >= ri.kappa && (ri.min_p <= 0.0f || w >= ri.min_p);
    return kept ? (float)((double)w * invW) : 0.0f;
}

// Residual mass of one tile of a rejected row: r = max(0, pi - q) per entry (or
// pi itself when use_pi), in token-id order within each thread group.
// q(id) of the draft distribution at a rejected node: a dense draft row, or
// for deterministic drafts one at each proposed token (d0, and n more tokens in
// `set`) and zero elsewhere.
struct DraftQ {
    const float* q;
    int d0;
    const int32_t* set;
    int n;
    __device__ __forceinline__ float operator()(int id) const {
        if (q) return gld(q + id);
        bool one = id == d0;
        for (int k = 0; k < n; ++k) one |= set[k] == id;
        return one ? 1.0f : 0.0f;
    }
};

// The residual max(0, pi - q) (or pi itself when use_pi) of this thread's
// entries of tile tb, pi being the filtered distribution described by ri.
template <int DT>
__device__ __forceinline__ void residual_values(const RowCtx& c, const RowInfo& ri, const DraftQ& qf,
                                                int tb, bool use_pi, SmemTile& tt, double r[EPT]) {
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    const TablePrefetch f = prefetch_tables(c);
    load_tile<DT>(c, tb, v);
    load_mask<DT>(c, tb, mw);
    const bool tables = c.hist_len + c.extra_len + c.bias_len > 0;
    if (tables) build_tables<DT>(c, tb, tt, f);
    process_tile<DT>(c, tb, v, tt, mw, tables);
    const double invW = 1.0 / ri.W;
    const float rT = 1.0f / c.T;
    auto fill = [&](auto p2_c) {
        constexpr bool P2 = decltype(p2_c)::value;
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int id = slot_id<DT>(tb, s);
            double val = 0.0;
            if (id < c.V) {
                const float pi = filtered_prob<P2>(c, ri, invW, rT, id, v[s]);
                val = use_pi ? (double)pi : (double)fmaxf(0.0f, pi - qf(id));
            }
            r[s] = val;
        }
    };
    if (pow2_temp(c.T)) fill(BoolC<true>{});
    else fill(BoolC<false>{});
}

// Sums over tile tb of the residual and of pi (the fallback when the residual
// is zero), by the whole workgroup. With `keep`, each entry's residual (a
// binary32 value) also goes to keep[id], so that the draw within the tile
// reads it instead of forming the tile again.
template <int DT>
__device__ __forceinline__ double2 residual_sums(const RowCtx& c, const RowInfo& ri, const DraftQ& qf,
                                                 int tb, SmemTile& tt, SmemS& sh, float* keep) {
    float v[EPT];
    uint32_t mw[Lay<DT>::NG];
    const TablePrefetch f = prefetch_tables(c);
    load_tile<DT>(c, tb, v);
    load_mask<DT>(c, tb, mw);
    const bool tables = c.hist_len + c.extra_len + c.bias_len > 0;
    if (tables) build_tables<DT>(c, tb, tt, f);
    process_tile<DT>(c, tb, v, tt, mw, tables);
    double sr = 0.0, sp = 0.0;
    const double invW = 1.0 / ri.W;
    const float rT = 1.0f / c.T;
    auto sum = [&](auto p2_c) {
        constexpr bool P2 = decltype(p2_c)::value;
#pragma unroll
        for (int s = 0; s < EPT; ++s) {
            const int id = slot_id<DT>(tb, s);
            if (id < c.V) {
                const float pi = filtered_prob<P2>(c, ri, invW, rT, id, v[s]);
                const float rv = fmaxf(0.0f, pi - qf(id));
                if (keep) keep[id] = rv;
                sr += (double)rv;
                sp += (double)pi;
            }
        }
    };
    if (pow2_temp(c.T)) sum(BoolC<true>{});
    else sum(BoolC<false>{});
    // both sums in one exchange of the wave totals
    sr = wave_sum_d(sr);
    sp = wave_sum_d(sp);
    const int wv = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) {
        sh.red.d[wv] = sr;
        sh.red2.d[wv] = sp;
    }
    __syncthreads();
    sr = 0.0;
    sp = 0.0;
#pragma unroll
    for (int w = 0; w < NT / WAVE; ++w) {
        sr += sh.red.d[w];
        sp += sh.red2.d[w];
    }
    return make_double2(sr, sp);
}

// Verification, residual stage 1: per tile of each rejected row, the sums of the
// residual max(0, pi - q) and of pi.
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
    DraftQ qf;
    qf.q = a.draft_probs ? a.draft_probs + ((size_t)b * a.G + j) * a.draft_stride : nullptr;
    qf.d0 = a.draft_tokens[(size_t)b * a.G + j];
    qf.set = nullptr;
    qf.n = 0;
    const double2 x = residual_sums<DT>(c, ri, qf, tile * TILE, tt, sh,
                                        a.ws.scratch_z + ((size_t)b * (a.G + 1) + j) * a.V);
    if (threadIdx.x == 0) a.ws.resid_tile[(size_t)b * n_tiles + tile] = x;
}

// A draw from the residual distribution of the row described by c and ri, in
// token-id order: the tile by the per-tile sums `tiles`, then the entry within
// the tile (u from the residual domain at c's position). The entries'
// residuals come from `kept` (written with the sums) when the draw uses the
// residual, else they are formed again. Called by the whole workgroup; lane t
// of wave 0 brings tile t's sums in `x` (loaded early by the caller: they do
// not depend on which row is drawn).
template <int DT>
__device__ __forceinline__ int residual_draw(const RowCtx& c, const RowInfo& ri, const DraftQ& qf,
                                             double2 x, int n_tiles, const float* kept, SmemTile& tt,
                                             SmemS& sh, int& s_tile, int& s_usepi, double& s_rem) {
    if (threadIdx.x < WAVE) {
        // lane t holds tile t's sums (n_tiles <= 32): the totals, then the
        // tile where the running sum in tile order passes u x total
        const int t = threadIdx.x;
        const double R = wave_sum_d(x.x);
        const double P = wave_sum_d(x.y);
        const int use_pi = !(R > 0.0);
        const double tot = use_pi ? P : R;
        const float ur = u24(philox_word(c.seed, c.req, c.pos, 0, DOM_RESIDUAL));
        const double tgt = (double)ur * tot;
        const double amt = use_pi ? x.y : x.x;
        const double inc = wave_incl_scan_d(amt);
        const double cum = inc - amt;
        const unsigned long long hit = __ballot(t < n_tiles && amt > 0.0 && cum + amt > tgt);
        const unsigned long long nz = __ballot(t < n_tiles && amt > 0.0);
        int sel;
        double rem;
        if (hit) {
            sel = (int)__builtin_ctzll(hit);
            rem = tgt - __shfl(cum, sel);
        } else {
            sel = nz ? 63 - (int)__builtin_clzll(nz) : -1;
            rem = DBL_MAX;
        }
        if (t == 0) {
            s_tile = sel;
            s_usepi = use_pi;
            s_rem = rem;
        }
    }
    __syncthreads();
    const int st = s_tile;
    int token = -1;
    if (st >= 0) {
        double r[EPT];
        if (kept && s_usepi == 0) {
#pragma unroll
            for (int s = 0; s < EPT; ++s) {
                const int id = slot_id<DT>(st * TILE, s);
                r[s] = id < c.V ? (double)gld(kept + id) : 0.0;
            }
        } else {
            residual_values<DT>(c, ri, qf, st * TILE, s_usepi != 0, tt, r);
        }
        using L = Lay<DT>;
        static_assert(L::NG <= EPT / 4, "group totals");
        const int lane = threadIdx.x & (WAVE - 1);
        const int wv = threadIdx.x / WAVE;
        // Id order in the tile is group, then thread, then entry: every
        // group's sums are scanned across the threads at once (one wave scan
        // per group, one exchange of the wave totals).
        double gs[L::NG], wex[L::NG];
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            gs[g] = 0.0;
#pragma unroll
            for (int k = 0; k < L::VEC; ++k) gs[g] += r[g * L::VEC + k];
            const double inc = wave_incl_scan_d(gs[g]);
            wex[g] = inc - gs[g];
            if (lane == WAVE - 1) sh.dg[g][wv] = inc;
        }
        __syncthreads();
        double carry = 0.0;
        int found = INT_MAX, lastpos = -1;
        const double rem = s_rem;
#pragma unroll
        for (int g = 0; g < L::NG; ++g) {
            double run = carry + wex[g], gt = 0.0;
#pragma unroll
            for (int w = 0; w < NT / WAVE; ++w) {
                const double t = sh.dg[g][w];
                run += w < wv ? t : 0.0;
                gt += t;
            }
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
        // the smallest id that passes, else the largest id with residual mass
        found = wave_min_i(found);
        lastpos = wave_max_i(lastpos);
        if (lane == 0) {
            sh.red.i[wv] = found;
            sh.red2.i[wv] = lastpos;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NT / WAVE; ++w) {
            found = min(found, sh.red.i[w]);
            lastpos = max(lastpos, sh.red2.i[w]);
        }
        token = found != INT_MAX ? found : lastpos;
    }
    return token;
}

// The token of rejected position j of request b.
template <int DT>
__device__ __forceinline__ int residual_token(const SpecArgs& a, int b, int j, const RowInfo& ri, double2 xt,
                                              SmemTile& tt, SmemS& sh, int& s_tile, int& s_usepi,
                                              double& s_rem) {
    const RowCtx c = spec_ctx<DT>(a, b, j);
    DraftQ qf;
    qf.q = a.draft_probs ? a.draft_probs + ((size_t)b * a.G + j) * a.draft_stride : nullptr;
    qf.d0 = a.draft_tokens[(size_t)b * a.G + j];
    qf.set = nullptr;
    qf.n = 0;
    return residual_draw<DT>(c, ri, qf, xt, a.ws.n_tiles, a.ws.scratch_z + ((size_t)b * (a.G + 1) + j) * a.V, tt,
                             sh, s_tile, s_usepi, s_rem);
}

// Verification, per request: the output row (accepted drafts, then the bonus
// token, the greedy target token, or the residual draw) and, when the caller
// keeps per-request token sequences on the device, their append: the emitted
// tokens go into the slots after each sequence's length, which then advances,
// so the host need not read the accepted counts before the next step.
template <int DT>
__global__ __launch_bounds__(NT) void k_spec_finish(SpecArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    __shared__ int s_tile;
    __shared__ int s_usepi;
    __shared__ double s_rem;
    const int b = blockIdx.x;
    const int G1 = a.G + 1;
    // the residual tile sums, issued first (used only if a position is rejected)
    const double2 xt = threadIdx.x < a.ws.n_tiles ? a.ws.resid_tile[(size_t)b * a.ws.n_tiles + threadIdx.x]
                                                  : make_double2(0.0, 0.0);
    const int n = accepted_prefix(a, b);
    RowInfo ri;
    const int j = residual_position(a, b, ri);
    int32_t* out = a.out_tokens + (size_t)b * G1;
    int final_token = n == a.G ? ri.token : ri.argmax;
    if (threadIdx.x == 0) {
        for (int k = 0; k < n; ++k) out[k] = a.draft_tokens[(size_t)b * a.G + k];
        for (int k = n + 1; k < G1; ++k) out[k] = -1;
        a.out_num_accepted[b] = n;
        if (j < 0) out[n] = final_token;
    }
    if (j >= 0) {  // uniform over the workgroup
        final_token = residual_token<DT>(a, b, j, ri, xt, tt, sh, s_tile, s_usepi, s_rem);
        if (threadIdx.x == 0) out[j] = final_token;
    }
    if (a.seq_tokens) {
        // every read of this request's parameters (its position may be the
        // length array itself) precedes the length update
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t* seq = a.seq_tokens + (size_t)b * a.seq_stride;
            const int L = a.seq_len[b];
            for (int k = 0; k <= n; ++k) {
                const int slot = L + k;
                if (slot >= 0 && slot < a.seq_capacity)
                    seq[slot] = k < n ? a.draft_tokens[(size_t)b * a.G + k] : final_token;
            }
            a.seq_len[b] = min(L + n + 1, a.seq_capacity);
        }
    }
}


// ---------------------------------------------------------------------------
// tree verification: node n of request b is row b * N + n; its penalty history
// is the request's followed by the tokens on the path from the root to n, and
// its position is the request's plus the node's depth.

template <int DT>
__device__ __forceinline__ RowCtx tree_ctx(const TreeArgs& a, int b, int n, int depth) {
    const int row = b * a.N + n;
    const void* logits = (const char*)a.target + (size_t)row * a.row_stride * (DT == SS_F32 ? 4 : 2);
    const uint32_t* mrow = a.p.mask ? a.p.mask + (size_t)row * a.p.mask_stride : nullptr;
    const int d = max(depth, 0);
    return make_ctx(a.p, b, logits, a.V, a.ws.tree_path + (size_t)row * a.ws.tree_dmax, d, mrow,
                    (uint32_t)d);
}

// Depth and root path of every node, one wave per request (lane n = node n).
// Node n >= 1 hangs below parents[n] when 0 <= parents[n] < n; a node that
// breaks this, or lies below such a node, is unreachable (depth -1).
__global__ __launch_bounds__(WAVE) void k_tree_paths(TreeArgs a) {
    const int b = blockIdx.x;
    const int n = threadIdx.x;
    const int N = a.N;
    const int par = n < N ? a.parents[(size_t)b * N + n] : -1;
    const int tok = n < N ? a.tokens[(size_t)b * N + n] : -1;
    const bool edge = n >= 1 && n < N && par >= 0 && par < n;
    int d = n == 0 ? 0 : -1;
    for (int r = 1; r < N; ++r) {  // depth r is settled after round r
        const int pd = __shfl(d, edge ? par : 0);
        const bool set = d < 0 && edge && pd >= 0;
        if (set) d = pd + 1;
        if (!__ballot(set)) break;  // a round that settles nothing ends the walk (uniform)
    }
    if (n < N) a.ws.tree_depth[(size_t)b * N + n] = d;
    int32_t* path = a.ws.tree_path + ((size_t)b * N + min(n, N - 1)) * a.ws.tree_dmax;
    int at = n;
    const int dmax = wave_max_i(n < N ? d : 0);
    for (int r = 0; r < dmax; ++r) {  // path[d - 1 - r] = token of the r-th ancestor-or-self
        const int t = __shfl(tok, at);
        const int p = __shfl(par, at);
        if (n < N && r < d) path[d - 1 - r] = t;
        at = r < d ? p : at;
    }
}

template <int DT, bool ALIGNED>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_tree_tiles(TreeArgs a) {
    __shared__ SmemTile tt;
    const int n_tiles = a.ws.n_tiles;
    const int lin = xcd_linear(a.B * a.N * n_tiles);
    const int row = lin / n_tiles;
    const int tile = lin % n_tiles;
    const RowCtx c = tree_ctx<DT>(a, row / a.N, row % a.N, a.ws.tree_depth[row]);
    tile_stage1<DT, ALIGNED, false>(c, row, tile, a.ws, tt, nullptr, nullptr);
}

// Per node x: its filtered distribution, then its children tested in index
// order against the residual target (one-hot proposals): child i with token d
// is accepted iff u_i < p(d) / (1 - p of the siblings rejected before it), or
// for greedy rows iff d is the greedy token. Records the accepted child.
template <int DT>
__global__ __launch_bounds__(NTR) void k_tree_rows(TreeArgs a) {
    __shared__ SmemU su;
    __shared__ SmemR sh;
    const int row = xcd_linear(a.B * a.N);
    const int b = row / a.N;
    const int x = row % a.N;
    const int depth = a.ws.tree_depth[row];
    const RowLoad rl = row_load(a.ws, row);
    const RowCtx c = tree_ctx<DT>(a, b, x, depth);
    RowDbg dbg = {nullptr, 0, nullptr, nullptr, nullptr};
    RowInfo info;
    finalize_row<DT, false>(c, row, a.ws, rl, su, sh, dbg, info);
    // every wave holds the request's tree (lane = node), so the children and
    // their tokens are the same in every wave: the loop below is uniform
    const int lane = threadIdx.x & (WAVE - 1);
    const int par = lane < a.N ? a.parents[(size_t)b * a.N + lane] : -1;
    const int tok = lane < a.N ? a.tokens[(size_t)b * a.N + lane] : -1;
    unsigned long long kids = __ballot(depth >= 0 && lane >= 1 && lane < a.N && par == x && x < lane);
    int next = -1;
    if (kids) {
        if (c.T == 0.0f || info.n_kept == 0) {
            const unsigned long long m = kids & __ballot(info.argmax >= 0 && tok == info.argmax);
            next = m ? (int)__builtin_ctzll(m) : -1;
        } else {
            double remaining = 1.0;
            unsigned long long rejected = 0;  // children rejected so far with a new token
            for (int i = 0; kids; ++i) {
                const int ch = (int)__builtin_ctzll(kids);
                kids &= kids - 1;
                const int d = __shfl(tok, ch);
                const bool fresh = d >= 0 && d < a.V && (rejected & __ballot(tok == d)) == 0;
                double pi = 0.0;
                if (fresh) {
                    const float xd = single_entry<DT>(c, d, sh);
                    if (xd > NEG_INF) {
                        const float zd = canon_zero(xd / c.T);
                        const float w = expf(zd - info.zmax);
                        const bool kept = key64(zd, d) >= info.kappa &&
                                          (info.min_p <= 0.0f || w >= info.min_p);
                        if (kept) pi = (double)w / info.W;
                    }
                }
                const float ua = u24(philox_word(c.seed, c.req, c.pos, (uint32_t)i, DOM_ACCEPT));
                const double ratio = remaining > 0.0 ? pi / remaining : 0.0;
                if ((double)ua < ratio) {
                    next = ch;
                    break;
                }
                if (fresh) {
                    rejected |= 1ull << ch;
                    remaining -= pi;
                }
            }
        }
    }
    if (threadIdx.x == 0) {
        a.ws.tree_next[row] = next;
        a.ws.rowinfo[row] = info;
    }
}

// The accepted path of request b, walked in every wave from the root through
// the accepted children (each deeper than the last, so at most N - 1 steps):
// returns its length and the node it ends at; writer() sees each step.
template <class F>
__device__ __forceinline__ int tree_walk(const TreeArgs& a, int b, int& end, F writer) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nx = lane < a.N ? a.ws.tree_next[(size_t)b * a.N + lane] : -1;
    int cur = 0, k = 0;
    for (int r = 0; r < a.N; ++r) {
        const int nn = __shfl(nx, cur);
        if (nn <= cur || nn >= a.N) break;
        writer(k, nn);
        cur = nn;
        ++k;
    }
    end = cur;
    return k;
}

// The tokens of node e's children (all rejected when e ends the path) into
// set; returns their count. Whole workgroup; every wave computes the same.
__device__ __forceinline__ int tree_kids(const TreeArgs& a, int b, int e, int32_t* set) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int par = lane < a.N ? a.parents[(size_t)b * a.N + lane] : -1;
    const int tok = lane < a.N ? a.tokens[(size_t)b * a.N + lane] : -1;
    const bool kid = lane >= 1 && lane < a.N && par == e && e < lane;
    const unsigned long long m = __ballot(kid);
    if (threadIdx.x < WAVE && kid)
        set[__popcll(m & ((1ull << lane) - 1ull))] = tok;
    __syncthreads();
    return __popcll(m);
}

// Residual stage 1 of a request whose path ends at a node with children.
template <int DT>
__global__ __launch_bounds__(NT) SS_TILE_OCC void k_tree_resid_tiles(TreeArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    __shared__ int32_t set[WAVE];
    const int n_tiles = a.ws.n_tiles;
    const int b = blockIdx.x / n_tiles;
    const int tile = blockIdx.x % n_tiles;
    int e;
    tree_walk(a, b, e, [](int, int) {});
    const int row = b * a.N + e;
    const RowInfo ri = a.ws.rowinfo[row];
    const int nk = tree_kids(a, b, e, set);
    if (nk == 0 || a.p.temperature[b] == 0.0f || ri.n_kept == 0) return;
    const RowCtx c = tree_ctx<DT>(a, b, e, a.ws.tree_depth[row]);
    DraftQ qf;
    qf.q = nullptr;
    qf.d0 = -1;
    qf.set = set;
    qf.n = nk;
    const double2 x = residual_sums<DT>(c, ri, qf, tile * TILE, tt, sh, a.ws.scratch_z + (size_t)row * a.V);
    if (threadIdx.x == 0) a.ws.resid_tile[(size_t)b * n_tiles + tile] = x;
}

// Per request: the accepted path (tokens and nodes), then the final token: the
// greedy token, the residual draw after the end node's children were all
// rejected, or the end node's own draw at a leaf.
template <int DT>
__global__ __launch_bounds__(NT) void k_tree_finish(TreeArgs a) {
    __shared__ SmemTile tt;
    __shared__ SmemS sh;
    __shared__ int32_t set[WAVE];
    __shared__ int s_tile;
    __shared__ int s_usepi;
    __shared__ double s_rem;
    const int b = blockIdx.x;
    const int N = a.N;
    int32_t* out_t = a.out_tokens + (size_t)b * N;
    int32_t* out_n = a.out_nodes + (size_t)b * N;
    const int lane = threadIdx.x & (WAVE - 1);
    const int tok = lane < N ? a.tokens[(size_t)b * N + lane] : -1;
    // the residual tile sums, issued first (used only if the end node's children were rejected)
    const double2 xt = threadIdx.x < a.ws.n_tiles ? a.ws.resid_tile[(size_t)b * a.ws.n_tiles + threadIdx.x]
                                                  : make_double2(0.0, 0.0);
    int e;
    const int k = tree_walk(a, b, e, [&](int i, int node) {
        const int t = __shfl(tok, node);
        if (threadIdx.x == 0) {
            out_t[i] = t;
            out_n[i] = node;
        }
    });
    const int row = b * N + e;
    const RowInfo ri = a.ws.rowinfo[row];
    const int nk = tree_kids(a, b, e, set);
    int final_token;
    if (a.p.temperature[b] == 0.0f || ri.n_kept == 0) {
        final_token = ri.argmax;
    } else if (nk == 0) {
        final_token = ri.token;
    } else {
        const RowCtx c = tree_ctx<DT>(a, b, e, a.ws.tree_depth[row]);
        DraftQ qf;
        qf.q = nullptr;
        qf.d0 = -1;
        qf.set = set;
        qf.n = nk;
        final_token = residual_draw<DT>(c, ri, qf, xt, a.ws.n_tiles, a.ws.scratch_z + (size_t)row * a.V, tt, sh,
                                        s_tile, s_usepi, s_rem);
    }
    if (threadIdx.x == 0) {
        out_t[k] = final_token;
        for (int i = k + 1; i < N; ++i) out_t[i] = -1;
        for (int i = k; i < N; ++i) out_n[i] = -1;
        a.out_num_accepted[b] = k;
    }
}

// ---------------------------------------------------------------------------
// LM-head sampling with the per-request pipeline: the row stage.
//
// Every (row, tile) summary gives the tile's LM_NC largest keys and the next
// one. Let R be the largest of the next keys over all tiles: every entry with a
// key above R is among the tiles' candidates (an entry left out of its tile's
// list is at most that tile's next key). These certified entries, sorted, are
// an exact prefix of the row in key order; when the top-k, top-p and min-p
// cuts all fall inside it, the kept support is known and the token is the best
// z' + g over it. Otherwise the row is marked open: its z', which the GEMM
// kernel wrote to the workspace, go through the whole-row selection below.

constexpr int LM_CAP = 4096;  // certified entries sorted in LDS

struct SmemLm {
    unsigned long long key[LM_CAP];
    union {
        unsigned long long sorted[LM_CAP];  // the keys in bucket order, while they are ranked
        double pre[LM_CAP];                 // inclusive prefix mass in key order
    };
    uint32_t cnt[NBK];                      // bucket sizes
    uint32_t start[NBK];                    // bucket offsets
};

__device__ __forceinline__ bool lm_better(float sa, int ia, float sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// Block-wide (score, id) argmax, the lowest id among equal scores.
__device__ __forceinline__ void lm_block_best(float& s, int& i, SmemR& sh) {
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const float os = __shfl_xor(s, o);
        const int oi = __shfl_xor(i, o);
        if (lm_better(os, oi, s, i)) {
            s = os;
            i = oi;
        }
    }
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) {
        sh.fmin[w] = s;
        sh.imax[w] = i;
    }
    __syncthreads();
    s = sh.fmin[0];
    i = sh.imax[0];
    for (int k = 1; k < NTR / WAVE; ++k)
        if (lm_better(sh.fmin[k], sh.imax[k], s, i)) {
            s = sh.fmin[k];
            i = sh.imax[k];
        }
    __syncthreads();
}

__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, SmemR& sh) {
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
        const unsigned long long x = ((unsigned long long)hi << 32) | lo;
        v = x > v ? x : v;
    }
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) sh.hs.wsum[w] = v;
    __syncthreads();
    unsigned long long m = 0;
    for (int k = 0; k < NTR / WAVE; ++k) m = sh.hs.wsum[k] > m ? sh.hs.wsum[k] : m;
    __syncthreads();
    return m;
}

__device__ __forceinline__ float lm_gumbel_score(const LmheadArgs& a, int j, int v, float z) {
    const uint4 w = philox4x32_10(make_uint4((uint32_t)a.p.request_ids[j], (uint32_t)a.p.positions[j],
                                             (uint32_t)v >> 2, DOM_GUMBEL),
                                  (uint32_t)a.p.seed, (uint32_t)(a.p.seed >> 32));
    const uint32_t s = (uint32_t)v & 3u;
    return z + gumbel32(s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w);
}

__global__ __launch_bounds__(NTR) void k_lm_merge(LmheadArgs a) {
    __shared__ SmemLm L;
    __shared__ SmemR sh;
    __shared__ int s_n;
    const int j = blockIdx.x;
    const int tid = threadIdx.x;
    const ParamPtrs& p = a.p;
    const LmTileStat* st = a.stats + (size_t)j * a.n_vtiles;
    const float T = p.temperature[j];
    // the row's maximum, the best Gumbel score, the deepest certifying bound
    // and the finite count
    unsigned long long kmax = 0, rest = 0;
    float bs = -FLT_MAX;
    int bi = INT_MAX, nfin = 0;
    for (int t = tid; t < a.n_vtiles; t += NTR) {
        const LmTileStat x = st[t];
        kmax = x.key[0] > kmax ? x.key[0] : kmax;
        rest = x.rest > rest ? x.rest : rest;
        if (lm_better(x.best_s, x.best_i, bs, bi)) {
            bs = x.best_s;
            bi = x.best_i;
        }
        nfin += x.nfinite;
    }
    kmax = block_max_u64(kmax, sh);
    rest = block_max_u64(rest, sh);
    lm_block_best(bs, bi, sh);
    const int total = block_sum_i(nfin, sh.red);
    const int V = a.V;
    const bool topk_on = p.top_k[j] > 0 && p.top_k[j] < V;
    const float tp = p.top_p[j];
    const float mp = p.min_p[j];
    const bool filtered = topk_on || tp < 1.0f || mp > 0.0f;
    if (total == 0 || T == 0.0f || !filtered) {
        if (tid == 0) {
            // no finite entry: -1; greedy: the largest key; else the best score
            a.out_tokens[j] = total == 0 ? -1 : T == 0.0f ? key64_id(kmax) : (bi == INT_MAX ? -1 : bi);
            a.unres[j] = 0;
            if (a.dbg_path) a.dbg_path[j] = 2;
        }
        return;
    }
    const float zmax = key_z(kmax);
    // the row mass
    double wsum = 0.0;
    for (int t = tid; t < a.n_vtiles; t += NTR) {
        const LmTileStat x = st[t];
        if (x.key[0]) wsum += (double)x.mass * (double)expf(key_z(x.key[0]) - zmax);
    }
    const double W = block_sum_d(wsum, sh.red);
    // the certified entries: keys above every tile's next key
    if (tid == 0) s_n = 0;
    __syncthreads();
    for (int t = tid; t < a.n_vtiles; t += NTR) {
        const LmTileStat x = st[t];
#pragma unroll
        for (int i = 0; i < LM_NC; ++i)
            if (x.key[i] > rest) {
                const int slot = atomicAdd(&s_n, 1);
                if (slot < LM_CAP) L.key[slot] = x.key[i];
            }
    }
    __syncthreads();
    const int nc = s_n;
    bool open = nc > LM_CAP;
    int n3 = 0;
    // Counting sort of the certified keys by bucket b = (zmax - z) S, which
    // does not decrease along key order, then each key's rank among its
    // bucket's keys (a bitonic network when a bucket is too large).
    bool bitonic = false;
    if (!open && nc > 1) {
        float zl = __builtin_huge_valf();
        for (int i = tid; i < nc; i += NTR) zl = fminf(zl, key_z(L.key[i]));
        zl = -block_max(-zl, sh.red);
        const float R = zmax - zl;
        const float S = R > 0.0f ? fminf((float)NBK / R, 3.0e38f) : 0.0f;
        for (int i = tid; i < NBK; i += NTR) L.cnt[i] = 0u;
        __syncthreads();
        constexpr int PE = LM_CAP / NTR;
        unsigned long long kk[PE];
        int bk[PE], ar[PE];
#pragma unroll
        for (int q = 0; q < PE; ++q) {
            const int e = tid + q * NTR;
            kk[q] = 0ull;
            bk[q] = 0;
            ar[q] = 0;
            if (e < nc) {
                kk[q] = L.key[e];
                bk[q] = (int)fminf((zmax - key_z(kk[q])) * S, (float)(NBK - 1));
                ar[q] = (int)atomicAdd(&L.cnt[bk[q]], 1u);
            }
        }
        __syncthreads();
        uint32_t cb[BKPT];
        unsigned long long mine = 0, mx = 0;
#pragma unroll
        for (int q = 0; q < BKPT; ++q) {
            cb[q] = L.cnt[tid * BKPT + q];
            mine += cb[q];
            mx = cb[q] > mx ? cb[q] : mx;
        }
        unsigned long long all;
        unsigned long long base = block_excl_scan_u64(mine, sh.hs, all);
        mx = block_max_u64(mx, sh);
#pragma unroll
        for (int q = 0; q < BKPT; ++q) {
            L.start[tid * BKPT + q] = (uint32_t)base;
            base += cb[q];
        }
        bitonic = mx > BK_MAX;  // uniform
        __syncthreads();
        if (!bitonic) {
#pragma unroll
            for (int q = 0; q < PE; ++q)
                if (tid + q * NTR < nc) L.sorted[L.start[bk[q]] + ar[q]] = kk[q];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < PE; ++q) {
                if (tid + q * NTR < nc) {
                    const int s0 = (int)L.start[bk[q]], cq = (int)L.cnt[bk[q]];
                    int r = 0;
                    for (int i = 0; i < cq; ++i) r += L.sorted[s0 + i] > kk[q] ? 1 : 0;
                    L.key[s0 + r] = kk[q];
                }
            }
            __syncthreads();
        }
    }
    if (!open && bitonic) {
        // bitonic sort, descending, over the next power of two (zero keys last)
        int P2 = WAVE;
        while (P2 < nc) P2 <<= 1;
        for (int i = nc + tid; i < P2; i += NTR) L.key[i] = 0ull;
        __syncthreads();
        for (int k = 2; k <= P2; k <<= 1) {
            for (int h = k >> 1; h > 0; h >>= 1) {
                for (int i = tid; i < P2 / 2; i += NTR) {
                    const int lo = 2 * h * (i / h) + (i % h);
                    const int hi = lo + h;
                    const bool desc = (lo & k) == 0;
                    const unsigned long long x = L.key[lo], y = L.key[hi];
                    if ((x < y) == desc) {
                        L.key[lo] = y;
                        L.key[hi] = x;
                    }
                }
                __syncthreads();
            }
        }
    }
    if (!open) {
        // weights and binary64 inclusive prefix masses in key order
        constexpr int PER = LM_CAP / NTR;
        double run = 0.0;
        double pre[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int i = tid * PER + q;
            const double w = i < nc ? (double)expf(key_z(L.key[i]) - zmax) : 0.0;
            run += w;
            pre[q] = run;
        }
        double tot;
        const double base = block_excl_scan_d(run, sh.red, tot);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int i = tid * PER + q;
            if (i < nc) L.pre[i] = base + pre[q];
        }
        __syncthreads();
        // the cuts, as the sampler makes them: top-k, top-p over the top-k
        // mass, min-p against the maximum
        const int K_eff = topk_on ? min(p.top_k[j], total) : total;
        int n1 = total;
        double Wk = W;
        if (topk_on && K_eff < total) {
            if (K_eff > nc) open = true;
            else {
                n1 = K_eff;
                Wk = L.pre[K_eff - 1];
            }
        }
        int n2 = n1;
        if (!open && tp < 1.0f) {
            // keep i while the mass before it is below top_p x Wk
            const double thr = (double)tp * Wk;
            const int lim = min(n1, nc);
            int cnt = 0;
            for (int i = tid; i < lim; i += NTR) cnt += (i == 0 || L.pre[i - 1] < thr) ? 1 : 0;
            cnt = block_sum_i(cnt, sh.red);
            if (cnt == lim && n1 > nc) open = true;  // the cut lies past the certified entries
            else n2 = cnt;
        }
        if (!open) {
            if (mp > 0.0f) {
                if (n2 > nc) {
                    // every uncertified entry must weigh below min_p
                    if (rest && expf(key_z(rest) - zmax) >= mp) open = true;
                    n2 = nc;
                }
                int cnt = 0;
                for (int i = tid; i < n2; i += NTR)
                    cnt += expf(key_z(L.key[i]) - zmax) >= mp ? 1 : 0;
                n3 = block_sum_i(cnt, sh.red);
            } else {
                if (n2 > nc) open = true;
                n3 = n2;
            }
        }
    }
    if (open) {
        // what the whole-row selection needs of the row: its extent and count
        float lo = __builtin_huge_valf();
        for (int t = tid; t < a.n_vtiles; t += NTR) lo = fminf(lo, st[t].zmin);
        lo = -block_max(-lo, sh.red);
        if (tid == 0) {
            a.unres[j] = 1;
            if (a.dbg_path) a.dbg_path[j] = 1;
            LmCut q;
            q.kP = 0;
            q.best = 0;
            q.zmax = zmax;
            q.mp = mp;
            q.zlo = lo;
            q.total = total;
            a.cut[j] = q;
        }
        return;
    }
    // Gumbel-max over the kept support
    float s2 = -FLT_MAX;
    int i2 = INT_MAX;
    for (int i = tid; i < n3; i += NTR) {
        const unsigned long long k = L.key[i];
        const int v = key64_id(k);
        const float sc = lm_gumbel_score(a, j, v, key_z(k));
        if (lm_better(sc, v, s2, i2)) {
            s2 = sc;
            i2 = v;
        }
    }
    lm_block_best(s2, i2, sh);
    if (tid == 0) {
        a.out_tokens[j] = i2 == INT_MAX ? -1 : i2;
        a.unres[j] = 0;
        if (a.dbg_path) a.dbg_path[j] = 0;
    }
}

// Rows left open: their z' (written by the GEMM kernel) through the whole-row
// selection of the kept set (top-k, then top-p; min-p is tested entry by entry
// in the Gumbel pass that follows).
__global__ __launch_bounds__(NTR) void k_lm_slow(LmheadArgs a) {
    __shared__ SmemU su;
    __shared__ SmemR sh;
    const int j = blockIdx.x;
    if (!a.unres[j]) return;
    const int tid = threadIdx.x;
    const ParamPtrs& p = a.p;
    const int V = a.V;
    const float* zr = a.zmat + (size_t)j * V;
    // the row's maximum, least entry and count, from the tiles' summaries
    const LmCut c0 = a.cut[j];
    const float zmax = c0.zmax;
    const float s2 = hdeep_scale(zmax, c0.zlo);
    const int total = c0.total;
    const bool topk_on = p.top_k[j] > 0 && p.top_k[j] < V;
    const int K_eff = topk_on ? min(p.top_k[j], total) : total;
    int cnt;
    unsigned long long ms, kK = 0;
    if (topk_on && K_eff < total)
        hist_select(zr, V, zmax, s2, true, 0ull, 0.0f, false, true,
                    (unsigned long long)K_eff, 0.0, su, sh, cnt, ms, kK);
    unsigned long long kP = kK;
    if (p.top_p[j] < 1.0f)
        hist_select(zr, V, zmax, s2, true, kK, 0.0f, true, true,
                    0, (double)p.top_p[j], su, sh, cnt, ms, kP);
    // the kept set; the Gumbel pass over it runs over the whole GPU (k_lm_gumbel)
    if (tid == 0) {
        LmCut q = c0;
        q.kP = kP;
        q.best = 0;
        a.cut[j] = q;
    }
}

// The Gumbel-max over an open row's kept set, LM_GCH chunks of the row per row
// (one workgroup each): every workgroup takes the best (z' + g, id) of its
// chunk and folds it into the row's key with a 64-bit atomic maximum (higher
// score first, then the lower id: the order the candidate paths use).
constexpr int LM_GCH = 32;
constexpr int LM_GNT = 256;

__global__ __launch_bounds__(LM_GNT) void k_lm_gumbel(LmheadArgs a) {
    const int j = blockIdx.y;
    if (!a.unres[j]) return;
    const int tid = threadIdx.x;
    const ParamPtrs& p = a.p;
    const int V = a.V;
    const LmCut q = a.cut[j];
    const float* zr = a.zmat + (size_t)j * V;
    const int ng = (V + 3) / 4;  // groups of four entries, one Philox block each
    const int per = (ng + LM_GCH - 1) / LM_GCH;
    const int gb = blockIdx.x * per, ge = min(ng, gb + per);
    float bs = -FLT_MAX;
    int bi = INT_MAX;
    const uint32_t req = (uint32_t)p.request_ids[j], pos = (uint32_t)p.positions[j];
    const bool al = ((uint32_t)(uintptr_t)zr & 15u) == 0u;
    for (int g0 = gb + tid; g0 < ge; g0 += LM_GNT * RQ) {
        float zs[RQ][4];
#pragma unroll
        for (int h = 0; h < RQ; ++h) {
            const int g = g0 + h * LM_GNT;
            if (g < ge && al && g * 4 + 3 < V) {
                const uint4 t = gld((const uint4*)zr + g);
                zs[h][0] = __uint_as_float(t.x);
                zs[h][1] = __uint_as_float(t.y);
                zs[h][2] = __uint_as_float(t.z);
                zs[h][3] = __uint_as_float(t.w);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int v = g * 4 + k;
                    zs[h][k] = g < ge && v < V ? zr[v] : NEG_INF;
                }
            }
        }
#pragma unroll
        for (int h = 0; h < RQ; ++h) {
            const int g = g0 + h * LM_GNT;
            bool any = false;
            bool keep[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float z = zs[h][k];
                const int v = g * 4 + k;
                keep[k] = z > NEG_INF && key64(z, v) >= q.kP && (q.mp <= 0.0f || expf(z - q.zmax) >= q.mp);
                any |= keep[k];
            }
            if (!any) continue;
            const uint4 w = philox4x32_10(make_uint4(req, pos, (uint32_t)g, DOM_GUMBEL),
                                          (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (!keep[k]) continue;
                const float sc = zs[h][k] + gumbel32(ws[k]);
                if (lm_better(sc, g * 4 + k, bs, bi)) {
                    bs = sc;
                    bi = g * 4 + k;
                }
            }
        }
    }
    // the workgroup's best, then the row's
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const float os = __shfl_xor(bs, o);
        const int oi = __shfl_xor(bi, o);
        if (lm_better(os, oi, bs, bi)) {
            bs = os;
            bi = oi;
        }
    }
    __shared__ float s_s[LM_GNT / WAVE];
    __shared__ int s_i[LM_GNT / WAVE];
    if ((tid & (WAVE - 1)) == 0) {
        s_s[tid / WAVE] = bs;
        s_i[tid / WAVE] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < LM_GNT / WAVE; ++w)
            if (lm_better(s_s[w], s_i[w], bs, bi)) {
                bs = s_s[w];
                bi = s_i[w];
            }
        if (bi != INT_MAX)
            atomicMax(&a.cut[j].best, key64(bs, bi));
    }
}

// The open rows' tokens from their best keys (-1: an empty kept set).
__global__ __launch_bounds__(WAVE) void k_lm_pick(LmheadArgs a) {
    for (int j = threadIdx.x; j < a.B; j += WAVE) {
        if (!a.unres[j]) continue;
        const unsigned long long k = a.cut[j].best;
        a.out_tokens[j] = k ? key64_id(k) : -1;
    }
}

void launch_lm_merge(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k) {
    launch_k(le, k, k_lm_merge, dim3(a.B), dim3(NTR), st, a);
}

void launch_lm_slow(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k) {
    launch_k(le, k, k_lm_slow, dim3(a.B), dim3(NTR), st, a);
}

void launch_lm_gumbel(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k) {
    launch_k(le, k, k_lm_gumbel, dim3(LM_GCH, a.B), dim3(LM_GNT), st, a);
    launch_k(le, k + 1, k_lm_pick, dim3(1), dim3(WAVE), st, a);
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
    const dim3 g(a.B * a.ws.n_tiles);
    const bool al = rows_aligned<DT>(a.logits, a.row_stride, a.V);
    if (a.ws.bins) {
        if (al) launch_k(le, 0, k_sample_tiles<DT, true, true>, g, dim3(NT), st, a);
        else launch_k(le, 0, k_sample_tiles<DT, false, true>, g, dim3(NT), st, a);
        launch_k(le, 1, k_sample_rows<DT, true>, dim3(a.B), dim3(NTR), st, a);
    } else {
        if (al) launch_k(le, 0, k_sample_tiles<DT, true, false>, g, dim3(NT), st, a);
        else launch_k(le, 0, k_sample_tiles<DT, false, false>, g, dim3(NT), st, a);
        launch_k(le, 1, k_sample_rows<DT, false>, dim3(a.B), dim3(NTR), st, a);
    }
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

template <int DT>
static void tree_chain(const TreeArgs& a, hipStream_t st, const LaunchEvents& le) {
    const int rows = a.B * a.N;
    launch_k(le, 0, k_tree_paths, dim3(a.B), dim3(WAVE), st, a);
    if (rows_aligned<DT>(a.target, a.row_stride, a.V))
        launch_k(le, 1, k_tree_tiles<DT, true>, dim3(rows * a.ws.n_tiles), dim3(NT), st, a);
    else
        launch_k(le, 1, k_tree_tiles<DT, false>, dim3(rows * a.ws.n_tiles), dim3(NT), st, a);
    launch_k(le, 2, k_tree_rows<DT>, dim3(rows), dim3(NTR), st, a);
    launch_k(le, 3, k_tree_resid_tiles<DT>, dim3(a.B * a.ws.n_tiles), dim3(NT), st, a);
    launch_k(le, 4, k_tree_finish<DT>, dim3(a.B), dim3(NT), st, a);
}

hipError_t launch_tree(const TreeArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le) {
    if (dt == SS_F32) tree_chain<SS_F32>(a, st, le);
    else tree_chain<SS_BF16>(a, st, le);
    return hipGetLastError();
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

// Fused LM-head GEMM + exact Gumbel-max sampling (gfx950 bf16 MFMA).
//
// Follows the FlashSampling news item (meineki.news, body): logits are formed
// in on-chip tiles, Gumbel noise is added, only a per-row maximum of each
// vocabulary tile is kept, and a small reduction over tiles yields the token;
// argmax decomposes over partitions, so the result is exact. The kept item is a
// (score, index) pair.
//
// Design for MI355X:
//  * One workgroup (4 wave64s) owns a 128-row vocabulary tile for all (up to
//    64) batch rows and walks K in steps of 64. Each step's operands -- 128 x 64
//    of W and 64 x 64 of H, bf16 -- are copied straight from global memory into
//    LDS by global_load_lds_dwordx4 (every instruction moves 1 KB: 8 rows x 128
//    contiguous bytes), three steps deep, so the W stream keeps many bytes in
//    flight without holding them in registers. Each LDS stage is a separate
//    object, waits are explicit (vmcnt for the copies, lgkmcnt for the LDS reads
//    of the stage being overwritten) and the barrier is a bare s_barrier.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r sits in slot
//    c ^ (r & 7) so the MFMA operand reads spread over the banks.
//  * z = W h^T with v_mfma_f32_32x32x16_bf16, W as the A operand (vocabulary
//    rows as M), H as B (batch as N): wave w computes vocabulary rows
//    [32w, 32w + 32) x 64 batch rows in two f32 accumulators. Each lane's
//    accumulators then cover four consecutive vocabulary entries of one batch
//    row, which is exactly one Philox block (4 words).
//  * Each workgroup starts K at its own step so concurrent workgroups spread
//    their weight reads over the row span. W is read once from HBM; the logits
//    never leave registers.
//  * Epilogue: s = z / T + g, per-row (max, lowest index) over the tile, written
//    as one pair per row per tile; a second launch reduces the pairs of every
//    row.
#include <float.h>
#include <limits.h>

#include "ss_device.h"
#include "ss_internal.h"

#pragma clang fp contract(off)

namespace ss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int LM_NT = 256;
constexpr int LM_ROWS = 128;   // vocabulary rows per workgroup tile
constexpr int LM_KSTEP = 64;   // K per pipeline step (4 MFMAs of K = 16)
constexpr int LM_MAXB = 64;
constexpr int LM_W_BYTES = LM_ROWS * LM_KSTEP * 2;   // 16 KB per stage
constexpr int LM_H_BYTES = LM_MAXB * LM_KSTEP * 2;   // 8 KB per stage

#define LDS_PTR(x) ((__attribute__((address_space(3))) void*)(x))

// s_waitcnt immediates (gfx9 encoding): vmcnt N with lgkmcnt 0, expcnt free.
constexpr int WAIT_VM6_LGK0 = 0x0076;
constexpr int WAIT_VM0_LGK0 = 0x0070;
// Cache policy of the weight copies: the non-temporal (streaming) bit.
constexpr int LM_W_CPOL = 2;

// Copies step `ks` of the operands into one LDS stage: wave w moves W rows
// [32w, 32w + 32) (4 instructions) and H rows [16w, 16w + 16) (2 instructions).
__device__ __forceinline__ void lm_copy(uint8_t* wbuf, uint8_t* hbuf, const uint16_t* __restrict__ weight,
                                        const uint16_t* __restrict__ hidden, int K, int V, int B,
                                        int tile, int ks) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int sub = lane >> 3;             // row within the 8 rows of an instruction
    const int slot = lane & 7;             // destination 16-byte slot in the LDS row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = wave * 32 + q * 8 + sub;                // row in the tile
        const int c = slot ^ (r & 7);                          // global chunk held by this slot
        int v = tile * LM_ROWS + r;
        v = v < V ? v : V - 1;
        const uint16_t* src = weight + (size_t)v * K + ks * LM_KSTEP + c * 8;
        // the weight is read once: non-temporal, so it does not push the
        // hidden states (re-read by every workgroup) out of L2
        __builtin_amdgcn_global_load_lds((const void*)src, LDS_PTR(wbuf + (wave * 32 + q * 8) * 128),
                                         16, 0, LM_W_CPOL);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int r = wave * 16 + q * 8 + sub;
        const int c = slot ^ (r & 7);
        const int j = r < B ? r : B - 1;
        const uint16_t* src = hidden + (size_t)j * K + ks * LM_KSTEP + c * 8;
        __builtin_amdgcn_global_load_lds((const void*)src, LDS_PTR(hbuf + (wave * 16 + q * 8) * 128),
                                         16, 0, 0);
    }
}

// One step's MFMA operands from an LDS stage (read before the next copy is
// issued, so nothing of the stage being read is in flight behind them).
struct LmOps {
    bf16x8 a[4];
    bf16x8 b0[4];
    bf16x8 b1[4];
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// The reads are issued as ds_read_b128 in inline assembly, and one explicit
// lgkmcnt(0) that takes every result as an operand orders them before their
// uses: the compiler then sees no LDS read it would have to order against the
// copies still in flight into the other stages.
__device__ __forceinline__ void lm_read(const uint8_t* wbuf, const uint8_t* hbuf, LmOps& o) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int wave = threadIdx.x / WAVE;
    const int half = lane >> 5;
    const int r = wave * 32 + (lane & 31);
    const int j0 = lane & 31, j1 = j0 + 32;
    const uint32_t wb = lds_addr(wbuf), hb = lds_addr(hbuf);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + half;
        const uint32_t aa = wb + r * 128 + ((c ^ (r & 7)) << 4);
        const uint32_t ab0 = hb + j0 * 128 + ((c ^ (j0 & 7)) << 4);
        const uint32_t ab1 = hb + j1 * 128 + ((c ^ (j1 & 7)) << 4);
        asm volatile("ds_read_b128 %0, %1" : "=v"(o.a[s]) : "v"(aa));
        asm volatile("ds_read_b128 %0, %1" : "=v"(o.b0[s]) : "v"(ab0));
        asm volatile("ds_read_b128 %0, %1" : "=v"(o.b1[s]) : "v"(ab1));
    }
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(o.a[0]), "+v"(o.a[1]), "+v"(o.a[2]), "+v"(o.a[3]), "+v"(o.b0[0]),
                   "+v"(o.b0[1]), "+v"(o.b0[2]), "+v"(o.b0[3]), "+v"(o.b1[0]), "+v"(o.b1[1]),
                   "+v"(o.b1[2]), "+v"(o.b1[3]));
}

__device__ __forceinline__ void lm_mfma(const LmOps& o, floatx16 acc[2]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[s], o.b0[s], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[s], o.b1[s], acc[1], 0, 0, 0);
    }
}

__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// The GEMM of vocabulary tile `tile` into the two accumulators (the operand
// stages are the six LDS buffers).
__device__ __forceinline__ void lm_gemm(const LmheadArgs& a, int tile, floatx16 acc[2], uint8_t* w0,
                                        uint8_t* w1, uint8_t* w2, uint8_t* h0, uint8_t* h1,
                                        uint8_t* h2) {
    const int K = a.K;
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[y][r] = 0.0f;

    // each workgroup walks K from its own starting step
    const int nsteps = K / LM_KSTEP;
    const int rot = (int)(((unsigned)tile * 2654435761u) % (unsigned)nsteps);
    auto ks_of = [&](int it) {
        int s = it + rot;
        return s >= nsteps ? s - nsteps : s;
    };
    lm_copy(w0, h0, a.weight, a.hidden, K, a.V, a.B, tile, ks_of(0));
    if (nsteps > 1) lm_copy(w1, h1, a.weight, a.hidden, K, a.V, a.B, tile, ks_of(1));
    // step i: wait for its copies (the next stage's may stay in flight) and for
    // this wave's reads of the stage about to be overwritten, barrier, read the
    // operands, start the copy two steps ahead, multiply.
#define LM_STEP(WB, HB, WN, HN, I)                                                        \
    {                                                                                     \
        const int i_ = (I);                                                               \
        if (i_ >= nsteps) break;                                                          \
        if (i_ + 1 < nsteps) __builtin_amdgcn_s_waitcnt(WAIT_VM6_LGK0);                   \
        else __builtin_amdgcn_s_waitcnt(WAIT_VM0_LGK0);                                   \
        __builtin_amdgcn_s_barrier();                                                     \
        LmOps o_;                                                                         \
        lm_read(WB, HB, o_);                                                              \
        if (i_ + 2 < nsteps) lm_copy(WN, HN, a.weight, a.hidden, K, a.V, a.B, tile, ks_of(i_ + 2)); \
        lm_mfma(o_, acc);                                                                 \
    }
    for (int it = 0; it < nsteps; it += 3) {
        LM_STEP(w0, h0, w2, h2, it)
        LM_STEP(w1, h1, w0, h0, it + 1)
        LM_STEP(w2, h2, w1, h1, it + 2)
    }
#undef LM_STEP
}

__global__ __launch_bounds__(LM_NT) void k_lmhead(LmheadArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t w0[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t w1[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t w2[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h0[LM_H_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h1[LM_H_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h2[LM_H_BYTES];
    __shared__ float s_score[LM_NT / WAVE][LM_MAXB];
    __shared__ int s_idx[LM_NT / WAVE][LM_MAXB];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid / WAVE;
    const int tile = blockIdx.x;
    const int half = lane >> 5;
    const int r32 = lane & 31;
    floatx16 acc[2];
    lm_gemm(a, tile, acc, w0, w1, w2, h0, h1, h2);

    // epilogue: lane holds, for batch column j = bb*32 + r32, vocabulary entries
    // tile*128 + wave*32 + 8*(r/4) + 4*half + (r%4)
    float best_s[2];
    int best_i[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const int j = bb * 32 + r32;
        best_s[bb] = -FLT_MAX;
        best_i[bb] = INT_MAX;
        if (j >= a.B) continue;
        const float T = a.temperature[j];
        const uint32_t req = a.request_ids ? (uint32_t)a.request_ids[j] : (uint32_t)j;
        const uint32_t pos = a.positions ? (uint32_t)a.positions[j] : 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int vbase = tile * LM_ROWS + wave * 32 + 8 * g + 4 * half;
            if (vbase >= a.V) continue;
            uint4 wv = make_uint4(0, 0, 0, 0);
            if (T != 0.0f)
                wv = philox4x32_10(make_uint4(req, pos, (uint32_t)vbase >> 2, DOM_GUMBEL),
                                   (uint32_t)a.seed, (uint32_t)(a.seed >> 32));
            const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = vbase + q;
                if (v >= a.V) continue;
                const float z = acc[bb][4 * g + q];
                if (a.debug_logits) a.debug_logits[(size_t)j * a.V + v] = z;
                const float s = (T != 0.0f) ? z / T + gumbel32(ws[q]) : z;
                if (better(s, v, best_s[bb], best_i[bb])) {
                    best_s[bb] = s;
                    best_i[bb] = v;
                }
            }
        }
    }
    // the two K-halves of a column hold different vocabulary entries: combine
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const float os = __shfl_xor(best_s[bb], 32);
        const int oi = __shfl_xor(best_i[bb], 32);
        if (better(os, oi, best_s[bb], best_i[bb])) {
            best_s[bb] = os;
            best_i[bb] = oi;
        }
        if (half == 0) {
            s_score[wave][bb * 32 + r32] = best_s[bb];
            s_idx[wave][bb * 32 + r32] = best_i[bb];
        }
    }
    __syncthreads();
    if (tid < a.B) {
        float bs = s_score[0][tid];
        int bi = s_idx[0][tid];
#pragma unroll
        for (int w = 1; w < LM_NT / WAVE; ++w)
            if (better(s_score[w][tid], s_idx[w][tid], bs, bi)) {
                bs = s_score[w][tid];
                bi = s_idx[w][tid];
            }
        a.partials[(size_t)tid * a.n_vtiles + tile] = make_float2(bs, __int_as_float(bi));
    }
}

// ---------------------------------------------------------------------------
// The per-request pipeline in the epilogue (ss_lmhead_sample_params).
//
// After the GEMM the stage buffers hold the tile's tables: per batch row, the
// multiplicity of each of the tile's 128 entries in the row's history (u16)
// and a bit per entry that some logit-bias entry names. Each entry's logit then
// goes through penalties, bias (entries applied in array order), mask and
// temperature as in the sampler, giving z'. The kernel summarises each
// (row, tile): its LM_NC largest keys (z', id), the next key, the mass below
// its maximum, the best Gumbel score and the count of finite entries. For rows
// with a filter it also writes z' to the workspace (4 bytes per entry against
// the weight's 2 K per vocabulary row): the rows the summaries cannot settle
// are then selected over the whole row without forming the GEMM again.

constexpr int LM_NK = LM_NC + 1;  // keys kept per list: the candidates and the next one

__device__ __forceinline__ float lm_penalize(float x, uint32_t count, float rep, float freq, float pres) {
    x = (x > 0.0f) ? x / rep : x * rep;
    const float fc = freq * (float)count;
    x = x - fc;
    x = x - pres;
    return x;
}

// Inserts key k into the descending list t[0..LM_NK) (0 = empty slot).
__device__ __forceinline__ void lm_insert(unsigned long long t[LM_NK], unsigned long long k) {
#pragma unroll
    for (int i = 0; i < LM_NK; ++i) {
        const unsigned long long hi = t[i] > k ? t[i] : k;
        const unsigned long long lo = t[i] > k ? k : t[i];
        t[i] = hi;
        k = lo;
    }
}

// One list's summary while lists are merged.
struct LmPart {
    unsigned long long t[LM_NK];
    float mass;      // relative to z of t[0]
    float best_s;
    int best_i;
    int nfinite;
    float zmin;      // the least finite z'
};

__device__ __forceinline__ void lm_combine(LmPart& x, const LmPart& y) {
    const float zx = x.t[0] ? key_z(x.t[0]) : -FLT_MAX;
    const float zy = y.t[0] ? key_z(y.t[0]) : -FLT_MAX;
    const float zc = fmaxf(zx, zy);
    float m = 0.0f;
    if (x.t[0]) m += x.mass * expf(zx - zc);
    if (y.t[0]) m += y.mass * expf(zy - zc);
    x.mass = m;
#pragma unroll
    for (int i = 0; i < LM_NK; ++i)
        if (y.t[i]) lm_insert(x.t, y.t[i]);
    if (better(y.best_s, y.best_i, x.best_s, x.best_i)) {
        x.best_s = y.best_s;
        x.best_i = y.best_i;
    }
    x.nfinite += y.nfinite;
    x.zmin = fminf(x.zmin, y.zmin);
}

__device__ __forceinline__ LmPart lm_shfl_xor32(const LmPart& x) {
    LmPart y;
#pragma unroll
    for (int i = 0; i < LM_NK; ++i) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x.t[i], 32);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x.t[i] >> 32), 32);
        y.t[i] = ((unsigned long long)hi << 32) | lo;
    }
    y.mass = __shfl_xor(x.mass, 32);
    y.best_s = __shfl_xor(x.best_s, 32);
    y.best_i = __shfl_xor(x.best_i, 32);
    y.nfinite = __shfl_xor(x.nfinite, 32);
    y.zmin = __shfl_xor(x.zmin, 32);
    return y;
}

__global__ __launch_bounds__(LM_NT) void k_lmhead_proc(LmheadArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t w0[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t w1[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t w2[LM_W_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h0[LM_H_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h1[LM_H_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t h2[LM_H_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid / WAVE;
    const int tile = blockIdx.x;
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const ParamPtrs& p = a.p;
    floatx16 acc[2];
    lm_gemm(a, tile, acc, w0, w1, w2, h0, h1, h2);

    // the tables (every wave is past its last read of the stage buffers)
    __syncthreads();
    uint32_t* cnt = (uint32_t*)w0;       // [64][64]: two u16 multiplicities per word
    uint32_t* bbits = (uint32_t*)w1;     // [64][4]: bias bit per entry
    int* hl = (int*)(w1 + 1024);         // [64] history lengths
    int* bl = hl + LM_MAXB;              // [64] bias lengths
    for (int i = tid; i < LM_MAXB * LM_ROWS / 2; i += LM_NT) cnt[i] = 0u;
    bbits[tid] = 0u;
    if (tid < LM_MAXB) {
        hl[tid] = tid < a.B ? min(p.hist_len[tid], p.hist_stride) : 0;
        bl[tid] = tid < a.B ? min(p.bias_len[tid], p.bias_stride) : 0;
    }
    __syncthreads();
    const int v0 = tile * LM_ROWS;
    const int Hs = p.hist_stride;
    if (Hs > 0) {
        const int total = a.B * Hs;
        constexpr int U = 8;  // loads in flight per thread
        for (int f0 = tid; f0 < total; f0 += LM_NT * U) {
            int ids[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = f0 + u * LM_NT;
                const int j = f / Hs;
                ids[u] = (f < total && f - j * Hs < hl[j]) ? p.hist_ids[f] : -1;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int f = f0 + u * LM_NT;
                const int e = ids[u] - v0;
                if (ids[u] >= 0 && ids[u] < a.V && e >= 0 && e < LM_ROWS)
                    atomicAdd(&cnt[(f / Hs) * (LM_ROWS / 2) + (e >> 1)], 1u << ((e & 1) * 16));
            }
        }
    }
    const int Bs = p.bias_stride;
    if (Bs > 0) {
        for (int f = tid; f < a.B * Bs; f += LM_NT) {
            const int j = f / Bs;
            if (f - j * Bs >= bl[j]) continue;
            const int id = p.bias_ids[f];
            const int e = id - v0;
            if (id >= 0 && id < a.V && e >= 0 && e < LM_ROWS) atomicOr(&bbits[j * 4 + (e >> 5)], 1u << (e & 31));
        }
    }
    __syncthreads();

    // each lane: for batch row j = bb*32 + r32, tile entries wave*32 + 8g + 4half + q
    LmPart part[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        LmPart& P = part[bb];
#pragma unroll
        for (int i = 0; i < LM_NK; ++i) P.t[i] = 0ull;
        P.mass = 0.0f;
        P.best_s = -FLT_MAX;
        P.best_i = INT_MAX;
        P.nfinite = 0;
        P.zmin = __builtin_huge_valf();
        const int j = bb * 32 + r32;
        if (j >= a.B) continue;
        const float T = p.temperature[j];
        // z' to the workspace: rows with a filter (the others never need it)
        const bool mat = T != 0.0f && ((p.top_k[j] > 0 && p.top_k[j] < a.V) || p.top_p[j] < 1.0f ||
                                       p.min_p[j] > 0.0f);
        const float rep = p.rep[j], freq = p.freq[j], pres = p.pres[j];
        const uint32_t req = (uint32_t)p.request_ids[j];
        const uint32_t pos = (uint32_t)p.positions[j];
        const int wbase = v0 + wave * 32;
        const uint32_t mw = (p.mask && wbase < a.V) ? p.mask[(size_t)j * p.mask_stride + (wbase >> 5)] : ~0u;
        const int32_t* bids = p.bias_ids + (size_t)j * Bs;
        const float* bvals = p.bias_vals + (size_t)j * Bs;
        const int nb = bl[j];
        float zz[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int vb = wbase + 8 * g + 4 * half;
            uint4 wv = make_uint4(0, 0, 0, 0);
            if (T != 0.0f && vb < a.V)
                wv = philox4x32_10(make_uint4(req, pos, (uint32_t)vb >> 2, DOM_GUMBEL),
                                   (uint32_t)p.seed, (uint32_t)(p.seed >> 32));
            const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = vb + q;
                const int e = v - v0;
                float x = acc[bb][4 * g + q];
                if (v >= a.V) {
                    zz[4 * g + q] = -__builtin_huge_valf();
                    continue;
                }
                const uint32_t c = (cnt[j * (LM_ROWS / 2) + (e >> 1)] >> ((e & 1) * 16)) & 0xFFFFu;
                if (c) x = lm_penalize(x, c, rep, freq, pres);
                if ((bbits[j * 4 + (e >> 5)] >> (e & 31)) & 1u)
                    for (int k = 0; k < nb; ++k)
                        if (bids[k] == v) x = x + bvals[k];
                if (!((mw >> (e & 31)) & 1u)) x = -__builtin_huge_valf();
                const bool fin = x > -__builtin_huge_valf();
                const float zp = fin ? (T != 0.0f ? canon_zero(x / T) : canon_zero(x)) : x;
                zz[4 * g + q] = zp;
                if (!fin) continue;
                lm_insert(P.t, key64(zp, v));
                const float sc = T != 0.0f ? zp + gumbel32(ws[q]) : zp;
                if (better(sc, v, P.best_s, P.best_i)) {
                    P.best_s = sc;
                    P.best_i = v;
                }
                ++P.nfinite;
            }
        }
        if (mat) {
            float* zr = a.zmat + (size_t)j * a.V;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int vb = wbase + 8 * g + 4 * half;
                if ((a.V & 3) == 0 && vb + 3 < a.V) {
                    *(float4*)(zr + vb) = make_float4(zz[4 * g], zz[4 * g + 1], zz[4 * g + 2], zz[4 * g + 3]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (vb + q < a.V) zr[vb + q] = zz[4 * g + q];
                }
            }
        }
        if (P.t[0]) {
            const float zt = key_z(P.t[0]);
            float m = 0.0f, lo = __builtin_huge_valf();
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (zz[i] > -__builtin_huge_valf()) {
                    m += expf(zz[i] - zt);
                    lo = fminf(lo, zz[i]);
                }
            P.mass = m;
            P.zmin = lo;
        }
    }
    // the two halves of a column hold different entries: combine, then the
    // four waves through LDS
    struct alignas(16) Slot {
        unsigned long long t[LM_NK];
        float mass, best_s;
        int best_i, nfinite;
        float zmin;
    };
    static_assert(sizeof(Slot) * LM_MAXB * (LM_NT / WAVE) <= LM_W_BYTES, "slots fit a stage buffer");
    Slot* slots = (Slot*)w2;  // [wave][row]
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        const LmPart y = lm_shfl_xor32(part[bb]);
        lm_combine(part[bb], y);
        if (half == 0) {
            Slot& sl = slots[wave * LM_MAXB + bb * 32 + r32];
#pragma unroll
            for (int i = 0; i < LM_NK; ++i) sl.t[i] = part[bb].t[i];
            sl.mass = part[bb].mass;
            sl.best_s = part[bb].best_s;
            sl.best_i = part[bb].best_i;
            sl.nfinite = part[bb].nfinite;
            sl.zmin = part[bb].zmin;
        }
    }
    __syncthreads();
    if (tid < a.B) {
        LmPart x;
        {
            const Slot& sl = slots[tid];
#pragma unroll
            for (int i = 0; i < LM_NK; ++i) x.t[i] = sl.t[i];
            x.mass = sl.mass;
            x.best_s = sl.best_s;
            x.best_i = sl.best_i;
            x.nfinite = sl.nfinite;
            x.zmin = sl.zmin;
        }
#pragma unroll
        for (int w = 1; w < LM_NT / WAVE; ++w) {
            const Slot& sl = slots[w * LM_MAXB + tid];
            LmPart y;
#pragma unroll
            for (int i = 0; i < LM_NK; ++i) y.t[i] = sl.t[i];
            y.mass = sl.mass;
            y.best_s = sl.best_s;
            y.best_i = sl.best_i;
            y.nfinite = sl.nfinite;
            y.zmin = sl.zmin;
            lm_combine(x, y);
        }
        LmTileStat st;
#pragma unroll
        for (int i = 0; i < LM_NC; ++i) st.key[i] = x.t[i];
        st.rest = x.t[LM_NC];
        st.mass = x.mass;
        st.best_s = x.best_s;
        st.best_i = x.best_i;
        st.nfinite = x.nfinite;
        st.zmin = x.zmin;
        st.pad = 0;
        a.stats[(size_t)tid * a.n_vtiles + tile] = st;
    }
}

// Cross-tile reduction: one workgroup per batch row; each thread takes a
// strided share of the tiles, then (max, lowest index) across the wave through
// DPP / permlane exchanges and across the four waves through LDS.
template <int J>
__device__ __forceinline__ void better_xor(float& s, int& i) {
    const float os = xor_lane_f<J>(s);
    const int oi = xor_lane_i<J>(i);
    if (better(os, oi, s, i)) {
        s = os;
        i = oi;
    }
}

__global__ __launch_bounds__(LM_NT) void k_lmhead_reduce(LmheadArgs a) {
    __shared__ float s_score[LM_NT / WAVE];
    __shared__ int s_idx[LM_NT / WAVE];
    const int tid = threadIdx.x;
    const int j = blockIdx.x;
    float bs = -FLT_MAX;
    int bi = INT_MAX;
    const float2* pr = a.partials + (size_t)j * a.n_vtiles;
    for (int t = tid; t < a.n_vtiles; t += LM_NT) {
        const float2 x = pr[t];
        const int xi = __float_as_int(x.y);
        if (better(x.x, xi, bs, bi)) {
            bs = x.x;
            bi = xi;
        }
    }
    better_xor<1>(bs, bi);
    better_xor<2>(bs, bi);
    better_xor<4>(bs, bi);
    better_xor<8>(bs, bi);
    better_xor<16>(bs, bi);
    better_xor<32>(bs, bi);
    if ((tid & (WAVE - 1)) == 0) {
        s_score[tid / WAVE] = bs;
        s_idx[tid / WAVE] = bi;
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int w = 1; w < LM_NT / WAVE; ++w)
            if (better(s_score[w], s_idx[w], bs, bi)) {
                bs = s_score[w];
                bi = s_idx[w];
            }
        a.out_tokens[j] = bi == INT_MAX ? -1 : bi;
    }
}

hipError_t launch_lmhead_params(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le) {
    launch_k(le, 0, k_lmhead_proc, dim3(a.n_vtiles), dim3(LM_NT), st, a);
    launch_lm_merge(a, st, le, 1);
    launch_lm_slow(a, st, le, 2);
    launch_lm_gumbel(a, st, le, 3);
    return hipGetLastError();
}

hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le) {
    launch_k(le, 0, k_lmhead, dim3(a.n_vtiles), dim3(LM_NT), st, a);
    launch_k(le, 1, k_lmhead_reduce, dim3(a.B), dim3(LM_NT), st, a);
    return hipGetLastError();
}

}  // namespace ss

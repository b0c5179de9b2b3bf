// Device-side building blocks shared by the sampling kernels (gfx950, wave64).
//
// Philox4x32-10 follows Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3" (SC'11): per round, words 0 and 2 are
// multiplied by two fixed 32-bit constants, the high halves are mixed with the
// other two words and the key, and the key advances by two Weyl increments.
// The pages describe no generator; this one is keyed by the seed with counter
// (request, position, draw >> 2, domain).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ss {

constexpr int WAVE = 64;
constexpr int NT = 256;            // threads per workgroup of the row kernels
constexpr int EPT = 32;            // logits per thread
constexpr int TILE = NT * EPT;     // 8192 vocabulary entries per workgroup tile
constexpr int WT = WAVE * EPT;     // 2048 entries per wave tile (one wave's share of a tile)
constexpr int WPT = NT / WAVE;     // wave tiles per workgroup tile
constexpr int WCAP = 64;           // candidate slots per wave tile
constexpr int MAX_TILES = 32;      // V <= 262144
constexpr int MAX_WT = MAX_TILES * WPT;
constexpr int MAX_VOCAB = MAX_TILES * TILE;

constexpr uint32_t PH_M0 = 0xD2511F53u;
constexpr uint32_t PH_M1 = 0xCD9E8D57u;
constexpr uint32_t PH_W0 = 0x9E3779B9u;
constexpr uint32_t PH_W1 = 0xBB67AE85u;

enum : uint32_t { DOM_SAMPLE = 0, DOM_ACCEPT = 1, DOM_RESIDUAL = 2, DOM_GUMBEL = 3 };

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = PH_M0 * c.x;
        const uint32_t hi0 = __umulhi(PH_M0, c.x);
        const uint32_t lo1 = PH_M1 * c.z;
        const uint32_t hi1 = __umulhi(PH_M1, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += PH_W0;
        k1 += PH_W1;
    }
    return c;
}

__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint32_t request, uint32_t position,
                                                uint32_t draw, uint32_t domain) {
    const uint4 o = philox4x32_10(make_uint4(request, position, draw >> 2, domain),
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t s = draw & 3u;
    return s == 0 ? o.x : s == 1 ? o.y : s == 2 ? o.z : o.w;
}

// Top 24 bits scaled by 2^-24: a uniform on [0, 1), exact in binary32.
__device__ __forceinline__ float u24(uint32_t w) { return (float)(w >> 8) * 0x1p-24f; }

// -ln(-ln U), U = 1 - (w + 0.5) 2^-32, kept accurate over the whole range: for
// small w the argument of log1p is small; for large w, U itself is formed from
// the complement (2^32 - 1 - w) so nothing cancels.
__device__ __forceinline__ float gumbel32(uint32_t w) {
    float e;
    if (w < 0x80000000u) {
        const float x = ((float)w + 0.5f) * 0x1p-32f;
        e = -log1pf(-x);
    } else {
        const float u = ((float)(~w) + 0.5f) * 0x1p-32f;
        e = -logf(u);
    }
    return -logf(e);
}

// ---------------------------------------------------------------------------
// ordering helpers: key order is (z descending, token id ascending)

__device__ __forceinline__ float canon_zero(float z) { return z + 0.0f; }  // -0 -> +0

__device__ __forceinline__ uint32_t mono32(float z) {
    const uint32_t b = __float_as_uint(z);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Larger key64 = earlier in key order. z must be canonical (no -0).
__device__ __forceinline__ unsigned long long key64(float z, int id) {
    return ((unsigned long long)mono32(z) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ int key64_id(unsigned long long k) {
    return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

// z of a key (the inverse of mono32 on its upper half).
__device__ __forceinline__ float key_z(unsigned long long k) {
    const uint32_t m = (uint32_t)(k >> 32);
    return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}

// ---------------------------------------------------------------------------
// wave64 lane exchange through DPP and the gfx950 permlane swaps (VALU, no LDS
// round trip). Reductions pair lanes by mirrors (quad swap, half-row and row
// mirror, then the 16- and 32-lane swaps); scans shift within rows of 16 and
// broadcast row ends across rows.

template <int CTRL, int ROWMASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xF, BOUND_ZERO);
}

// A DPP move whose lanes all read a lane of their own row (or whose edge lanes
// are discarded by the caller): no old value is needed, so none is materialised.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

enum : int {
    DPP_QUAD_X1 = 0xB1,      // quad_perm [1,0,3,2]: lane ^ 1
    DPP_QUAD_X2 = 0x4E,      // quad_perm [2,3,0,1]: lane ^ 2
    DPP_ROW_SHL4 = 0x104,
    DPP_ROW_SHR1 = 0x111,
    DPP_ROW_SHR2 = 0x112,
    DPP_ROW_SHR4 = 0x114,
    DPP_ROW_SHR8 = 0x118,
    DPP_ROW_ROR8 = 0x128,    // lane ^ 8 within a row of 16
    DPP_ROW_MIRROR = 0x140,  // lane -> 15 - lane within a row
    DPP_HALF_MIRROR = 0x141, // lane -> 7 - lane within 8
    DPP_BCAST15 = 0x142,     // lane 15 of each row -> the next row
    DPP_BCAST31 = 0x143,     // lane 31 -> rows 2 and 3
};

// Lanes of a wave whose index has bit B set (B a power of two; 0 for B >= 64).
__host__ __device__ constexpr unsigned long long lanes_with_bit(int b) {
    return b == 1 ? 0xAAAAAAAAAAAAAAAAull : b == 2 ? 0xCCCCCCCCCCCCCCCCull
         : b == 4 ? 0xF0F0F0F0F0F0F0F0ull : b == 8 ? 0xFF00FF00FF00FF00ull
         : b == 16 ? 0xFFFF0000FFFF0000ull : b == 32 ? 0xFFFFFFFF00000000ull : 0ull;
}

// A lane-constant condition given as a wave mask: the mask stays in scalar
// registers and feeds the select directly (no per-lane arithmetic).
__device__ __forceinline__ bool lane_in(unsigned long long mask) {
    return __builtin_amdgcn_inverse_ballot_w64(mask);
}

// The value held by lane ^ J (J a power of two below 64).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    if constexpr (J == 1) {
        return dpp_mov<DPP_QUAD_X1>(v);
    } else if constexpr (J == 2) {
        return dpp_mov<DPP_QUAD_X2>(v);
    } else if constexpr (J == 4) {
        const uint32_t up = dpp_mov<DPP_ROW_SHL4>(v);
        const uint32_t dn = dpp_mov<DPP_ROW_SHR4>(v);
        return lane_in(lanes_with_bit(4)) ? dn : up;
    } else if constexpr (J == 8) {
        return dpp_mov<DPP_ROW_ROR8>(v);
    } else if constexpr (J == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return lane_in(lanes_with_bit(16)) ? p[0] : p[1];
    } else {
        static_assert(J == 32, "lane exchange distance");
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return lane_in(lanes_with_bit(32)) ? p[0] : p[1];
    }
}

template <int J>
__device__ __forceinline__ float xor_lane_f(float v) {
    return __uint_as_float(xor_lane<J>(__float_as_uint(v)));
}

template <int J>
__device__ __forceinline__ int xor_lane_i(int v) {
    return (int)xor_lane<J>((uint32_t)v);
}

// Butterfly all-reduce: after the step with mirror M every lane holds the
// reduction over its aligned group of 2M lanes.
template <class T, class Op>
__device__ __forceinline__ T wave_allreduce32(T v, Op op) {
    auto sw = [](T x, auto tag) -> T {
        constexpr int C = decltype(tag)::value;
        uint32_t u;
        __builtin_memcpy(&u, &x, 4);
        u = dpp_mov<C>(u);
        T r;
        __builtin_memcpy(&r, &u, 4);
        return r;
    };
    v = op(v, sw(v, std::integral_constant<int, DPP_QUAD_X1>()));
    v = op(v, sw(v, std::integral_constant<int, DPP_QUAD_X2>()));
    v = op(v, sw(v, std::integral_constant<int, DPP_HALF_MIRROR>()));
    v = op(v, sw(v, std::integral_constant<int, DPP_ROW_MIRROR>()));
    {
        uint32_t u;
        __builtin_memcpy(&u, &v, 4);
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        T a, b;
        const uint32_t pa = p[0], pb = p[1];
        __builtin_memcpy(&a, &pa, 4);
        __builtin_memcpy(&b, &pb, 4);
        v = op(a, b);
    }
    {
        uint32_t u;
        __builtin_memcpy(&u, &v, 4);
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        T a, b;
        const uint32_t pa = p[0], pb = p[1];
        __builtin_memcpy(&a, &pa, 4);
        __builtin_memcpy(&b, &pb, 4);
        v = op(a, b);
    }
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_allreduce32(v, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ int wave_min_i(int v) {
    return wave_allreduce32(v, [](int a, int b) { return min(a, b); });
}

__device__ __forceinline__ int wave_sum_i(int v) {
    return wave_allreduce32(v, [](int a, int b) { return a + b; });
}

template <int C>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long u = __double_as_longlong(v);
    const uint32_t lo = dpp_mov<C>((uint32_t)u);
    const uint32_t hi = dpp_mov<C>((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Binary64 sum over the wave in a fixed pairing order (the same in every lane).
__device__ __forceinline__ double wave_sum_d(double v) {
    // a + b and b + a round identically, so the mirrored partners agree exactly
    v = v + dpp_f64<DPP_QUAD_X1>(v);
    v = v + dpp_f64<DPP_QUAD_X2>(v);
    v = v + dpp_f64<DPP_HALF_MIRROR>(v);
    v = v + dpp_f64<DPP_ROW_MIRROR>(v);
    {
        const unsigned long long u = __double_as_longlong(v);
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
        const double a = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0]));
        const double b = __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
        v = a + b;
    }
    {
        const unsigned long long u = __double_as_longlong(v);
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
        const double a = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0]));
        const double b = __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
        v = a + b;
    }
    return v;
}

// Inclusive prefix sums across the wave (Hillis-Steele within rows of 16, then
// the row ends carried across rows).
__device__ __forceinline__ int wave_incl_scan_i(int v) {
    uint32_t u = (uint32_t)v;
    u += dpp_mov<DPP_ROW_SHR1>(u);
    u += dpp_mov<DPP_ROW_SHR2>(u);
    u += dpp_mov<DPP_ROW_SHR4>(u);
    u += dpp_mov<DPP_ROW_SHR8>(u);
    u += dpp_u32<DPP_BCAST15, 0xA, false>(0u, u);
    u += dpp_u32<DPP_BCAST31, 0xC, false>(0u, u);
    return (int)u;
}

template <int C, int ROWMASK, bool BZ>
__device__ __forceinline__ double dpp_f64_masked(double v) {
    const unsigned long long u = __double_as_longlong(v);
    const uint32_t lo = dpp_u32<C, ROWMASK, BZ>(0u, (uint32_t)u);
    const uint32_t hi = dpp_u32<C, ROWMASK, BZ>(0u, (uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ double wave_incl_scan_d(double v) {
    v = v + dpp_f64_masked<DPP_ROW_SHR1, 0xF, true>(v);
    v = v + dpp_f64_masked<DPP_ROW_SHR2, 0xF, true>(v);
    v = v + dpp_f64_masked<DPP_ROW_SHR4, 0xF, true>(v);
    v = v + dpp_f64_masked<DPP_ROW_SHR8, 0xF, true>(v);
    v = v + dpp_f64_masked<DPP_BCAST15, 0xA, false>(v);
    v = v + dpp_f64_masked<DPP_BCAST31, 0xC, false>(v);
    return v;
}

template <int C, int ROWMASK, bool BZ>
__device__ __forceinline__ unsigned long long dpp_u64_masked(unsigned long long u) {
    const uint32_t lo = dpp_u32<C, ROWMASK, BZ>(0u, (uint32_t)u);
    const uint32_t hi = dpp_u32<C, ROWMASK, BZ>(0u, (uint32_t)(u >> 32));
    return ((unsigned long long)hi << 32) | lo;
}

// Inclusive prefix sum of a u64 over the wave (lane order), by the same DPP
// steps as wave_incl_scan_d.
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
    v += dpp_u64_masked<DPP_ROW_SHR1, 0xF, true>(v);
    v += dpp_u64_masked<DPP_ROW_SHR2, 0xF, true>(v);
    v += dpp_u64_masked<DPP_ROW_SHR4, 0xF, true>(v);
    v += dpp_u64_masked<DPP_ROW_SHR8, 0xF, true>(v);
    v += dpp_u64_masked<DPP_BCAST15, 0xA, false>(v);
    v += dpp_u64_masked<DPP_BCAST31, 0xC, false>(v);
    return v;
}

// Scratch for workgroup-level reductions over NB threads (NB / WAVE waves).
template <int NB>
struct RedT {
    float f[NB / WAVE];
    int i[NB / WAVE];
    double d[NB / WAVE];
};

template <int NB>
__device__ __forceinline__ float block_max(float v, RedT<NB>& r) {
    v = wave_max(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.f[w] = v;
    __syncthreads();
    float m = r.f[0];
#pragma unroll
    for (int k = 1; k < NB / WAVE; ++k) m = fmaxf(m, r.f[k]);
    __syncthreads();
    return m;
}

template <int NB>
__device__ __forceinline__ int block_min_i(int v, RedT<NB>& r) {
    v = wave_min_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.i[w] = v;
    __syncthreads();
    int m = r.i[0];
#pragma unroll
    for (int k = 1; k < NB / WAVE; ++k) m = min(m, r.i[k]);
    __syncthreads();
    return m;
}

template <int NB>
__device__ __forceinline__ int block_sum_i(int v, RedT<NB>& r) {
    v = wave_sum_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.i[w] = v;
    __syncthreads();
    int m = 0;
#pragma unroll
    for (int k = 0; k < NB / WAVE; ++k) m += r.i[k];
    __syncthreads();
    return m;
}

// Deterministic: fixed pairing within each wave, then the wave sums in wave order.
template <int NB>
__device__ __forceinline__ double block_sum_d(double v, RedT<NB>& r) {
    v = wave_sum_d(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.d[w] = v;
    __syncthreads();
    double m = 0.0;
#pragma unroll
    for (int k = 0; k < NB / WAVE; ++k) m += r.d[k];
    __syncthreads();
    return m;
}

// Exclusive scan of one int per thread in thread order; returns the total too.
template <int NB>
__device__ __forceinline__ int block_excl_scan_i(int v, RedT<NB>& r, int& total) {
    const int inc = wave_incl_scan_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) r.i[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NB / WAVE; ++k) {
        if (k < w) base += r.i[k];
        tot += r.i[k];
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

template <int NB>
__device__ __forceinline__ double block_excl_scan_d(double v, RedT<NB>& r, double& total) {
    const double inc = wave_incl_scan_d(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) r.d[w] = inc;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int k = 0; k < NB / WAVE; ++k) {
        if (k < w) base += r.d[k];
        tot += r.d[k];
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

__device__ __forceinline__ uint32_t xor_lane_dyn_u(uint32_t v, int j) {
    switch (j) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
    }
}

// Sorts one float per lane across the wave, descending (bitonic network over
// DPP / permlane exchanges; lane i ends with the i-th largest). The network runs
// on order-preserving u32 images of the floats, and which lanes of a pair keep
// the larger value is a constant lane mask per step, so a step costs one lane
// exchange, one compare and one select.
__device__ __forceinline__ float wave_sort_desc(float v) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
#pragma unroll
    for (int k = 2; k <= WAVE; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const uint32_t o = xor_lane_dyn_u(u, j);
            // the lower lane of a pair keeps the larger value in descending blocks
            const bool keep_max = lane_in(~(lanes_with_bit(k) ^ lanes_with_bit(j)));
            u = ((u >= o) == keep_max) ? u : o;
        }
    }
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}

// The same network on one 64-bit key per lane (descending; both halves move
// with each exchange): lane i ends with the i-th largest key.
__device__ __forceinline__ unsigned long long wave_sort_desc_u64(unsigned long long k) {
#pragma unroll
    for (int kk = 2; kk <= WAVE; kk <<= 1) {
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            const uint32_t lo = xor_lane_dyn_u((uint32_t)k, j);
            const uint32_t hi = xor_lane_dyn_u((uint32_t)(k >> 32), j);
            const unsigned long long o = ((unsigned long long)hi << 32) | lo;
            const bool keep_max = lane_in(~(lanes_with_bit(kk) ^ lanes_with_bit(j)));
            k = ((k >= o) == keep_max) ? k : o;
        }
    }
    return k;
}

}  // namespace ss

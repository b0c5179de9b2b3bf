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

namespace ss {

constexpr int WAVE = 64;
constexpr int NT = 256;            // threads per workgroup of the row kernels
constexpr int EPT = 32;            // logits per thread
constexpr int TILE = NT * EPT;     // 8192 vocabulary entries per workgroup tile
constexpr int CW = 128;            // candidate slots per tile
constexpr int LTARGET = 112;       // lane maxima that seed a tile's candidate threshold
constexpr int MAX_TILES = 32;      // V <= 262144
constexpr int POOL = MAX_TILES * CW;
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

__device__ __forceinline__ bool key_before(float za, int ia, float zb, int ib) {
    return za > zb || (za == zb && ia < ib);
}

// ---------------------------------------------------------------------------
// wave64 / workgroup reductions (xor shuffles lower to DPP / ds_swizzle)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    return v;
}

__device__ __forceinline__ double wave_incl_scan_d(double v) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const double y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    return v;
}

// Scratch for workgroup-level reductions (NT / WAVE = 4 waves).
struct RedScratch {
    float f[NT / WAVE];
    int i[NT / WAVE];
    double d[NT / WAVE];
};

__device__ __forceinline__ float block_max(float v, RedScratch& r) {
    v = wave_max(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.f[w] = v;
    __syncthreads();
    float m = r.f[0];
#pragma unroll
    for (int k = 1; k < NT / WAVE; ++k) m = fmaxf(m, r.f[k]);
    __syncthreads();
    return m;
}

__device__ __forceinline__ int block_min_i(int v, RedScratch& r) {
    v = wave_min_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.i[w] = v;
    __syncthreads();
    int m = r.i[0];
#pragma unroll
    for (int k = 1; k < NT / WAVE; ++k) m = min(m, r.i[k]);
    __syncthreads();
    return m;
}

__device__ __forceinline__ int block_sum_i(int v, RedScratch& r) {
    v = wave_sum_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.i[w] = v;
    __syncthreads();
    int m = 0;
#pragma unroll
    for (int k = 0; k < NT / WAVE; ++k) m += r.i[k];
    __syncthreads();
    return m;
}

// Deterministic: fixed shuffle tree, then the four wave sums in wave order.
__device__ __forceinline__ double block_sum_d(double v, RedScratch& r) {
    v = wave_sum_d(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0) r.d[w] = v;
    __syncthreads();
    double m = 0.0;
#pragma unroll
    for (int k = 0; k < NT / WAVE; ++k) m += r.d[k];
    __syncthreads();
    return m;
}

// Exclusive scan of one int per thread in thread order; returns the total too.
__device__ __forceinline__ int block_excl_scan_i(int v, RedScratch& r, int& total) {
    const int inc = wave_incl_scan_i(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) r.i[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < NT / WAVE; ++k) {
        if (k < w) base += r.i[k];
        tot += r.i[k];
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

__device__ __forceinline__ double block_excl_scan_d(double v, RedScratch& r, double& total) {
    const double inc = wave_incl_scan_d(v);
    const int w = threadIdx.x / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == WAVE - 1) r.d[w] = inc;
    __syncthreads();
    double base = 0.0, tot = 0.0;
#pragma unroll
    for (int k = 0; k < NT / WAVE; ++k) {
        if (k < w) base += r.d[k];
        tot += r.d[k];
    }
    __syncthreads();
    total = tot;
    return base + inc - v;
}

// Sorts one float per thread across the workgroup, descending (bitonic network;
// strides below the wave width exchange through shuffles, the rest through LDS).
__device__ __forceinline__ float block_sort_desc(float v, float* tmp) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 2; k <= NT; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            float o;
            if (j >= WAVE) {
                tmp[tid] = v;
                __syncthreads();
                o = tmp[tid ^ j];
                __syncthreads();
            } else {
                o = __shfl_xor(v, j);
            }
            const bool desc = (tid & k) == 0;
            const bool lower = (tid & j) == 0;
            v = (lower == desc) ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return v;
}

}  // namespace ss

// Fused LM-head GEMM + exact Gumbel-max sampling (gfx950 bf16 MFMA).
//
// Follows the FlashSampling news item (meineki.news, body): logits are formed
// in on-chip tiles, Gumbel noise is added, only a per-row maximum of each
// vocabulary tile is kept, and a small reduction over tiles yields the token;
// argmax decomposes over partitions, so the result is exact. The kept item is a
// (score, index) pair.
//
// Design for MI355X:
//  * The product z = W H^T is computed with W as the MFMA A operand (vocabulary
//    rows as M) and H^T as B (batch as N), v_mfma_f32_32x32x16_bf16 with fp32
//    accumulators. With that orientation each lane's accumulators cover four
//    consecutive vocabulary entries of one batch row, which is exactly one
//    Philox block (4 words), so the noise costs one generator call per 4 logits.
//  * One workgroup (4 wave64s) owns a 256-column vocabulary tile for all (up to
//    64) batch rows: wave w streams vocabulary rows [64w, 64w + 64) of the tile.
//    Each lane reads 64 contiguous bytes of a W row per step (the two lanes of a
//    row cover a whole 128-byte line), and the K index of each MFMA is permuted
//    consistently on both operands so the loads stay contiguous. The next
//    step's operands are loaded before the current step's MFMAs (register
//    double buffering) to keep the W stream in flight; W is read once from HBM
//    and never written back, and the logits never leave registers.
//  * Epilogue: s = z / T + g, per-row (max, lowest index) over the tile, written
//    as one pair per row per tile; a second, single-workgroup launch reduces
//    the pairs of every row.
#include <float.h>
#include <limits.h>

#include "ss_device.h"
#include "ss_internal.h"

#pragma clang fp contract(off)

namespace ss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int LM_NT = 256;
constexpr int LM_COLS = 256;   // vocabulary entries per workgroup tile
constexpr int LM_KSTEP = 64;   // K consumed per pipeline step (4 MFMAs of K = 16)
constexpr int LM_MAXB = 64;

struct Ops {
    uint4 a[2][4];  // W rows: [vocab block][sub-step]
    uint4 b[2][4];  // H rows: [batch block][sub-step]
};

__device__ __forceinline__ void load_ops(Ops& o, const uint16_t* __restrict__ wrow0,
                                         const uint16_t* __restrict__ wrow1,
                                         const uint16_t* __restrict__ hrow0,
                                         const uint16_t* __restrict__ hrow1, int koff) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o.a[0][i] = wrow0 ? *(const uint4*)(wrow0 + koff + 8 * i) : make_uint4(0, 0, 0, 0);
        o.a[1][i] = wrow1 ? *(const uint4*)(wrow1 + koff + 8 * i) : make_uint4(0, 0, 0, 0);
        o.b[0][i] = hrow0 ? *(const uint4*)(hrow0 + koff + 8 * i) : make_uint4(0, 0, 0, 0);
        o.b[1][i] = hrow1 ? *(const uint4*)(hrow1 + koff + 8 * i) : make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void mfma_ops(const Ops& o, floatx16 acc[2][2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, o.a[vb][i]);
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, o.b[bb][i]);
                acc[vb][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[vb][bb], 0, 0, 0);
            }
        }
    }
}

__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

__global__ __launch_bounds__(LM_NT) void k_lmhead(LmheadArgs a) {
    __shared__ float s_score[LM_NT / WAVE][LM_MAXB];
    __shared__ int s_idx[LM_NT / WAVE][LM_MAXB];
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wave = tid / WAVE;
    const int tile = blockIdx.x;
    const int half = lane >> 5;      // which 32-wide K half this lane feeds
    const int r32 = lane & 31;
    const int K = a.K;

    // vocabulary rows of this lane (A operand) and batch rows (B operand)
    const int v0 = tile * LM_COLS + wave * 64 + r32;
    const int v1 = v0 + 32;
    const int koff_lane = 32 * half;
    const uint16_t* w0 = v0 < a.V ? a.weight + (size_t)v0 * K + koff_lane : nullptr;
    const uint16_t* w1 = v1 < a.V ? a.weight + (size_t)v1 * K + koff_lane : nullptr;
    const uint16_t* h0 = r32 < a.B ? a.hidden + (size_t)r32 * K + koff_lane : nullptr;
    const uint16_t* h1 = r32 + 32 < a.B ? a.hidden + (size_t)(r32 + 32) * K + koff_lane : nullptr;

    floatx16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.0f;

    // each workgroup walks K from its own starting step, so concurrent
    // workgroups spread their weight reads over the whole row span
    const int nsteps = K / LM_KSTEP;
    const int rot = (int)(((unsigned)tile * 2654435761u) % (unsigned)nsteps);
    auto koff = [&](int it) {
        int s = it + rot;
        s = s >= nsteps ? s - nsteps : s;
        return s * LM_KSTEP;
    };
    Ops o0, o1;
    load_ops(o0, w0, w1, h0, h1, koff(0));
    int it = 0;
    for (; it + 2 <= nsteps; it += 2) {
        load_ops(o1, w0, w1, h0, h1, koff(it + 1));
        mfma_ops(o0, acc);
        if (it + 2 < nsteps) load_ops(o0, w0, w1, h0, h1, koff(it + 2));
        mfma_ops(o1, acc);
    }
    if (it < nsteps) mfma_ops(o0, acc);

    // epilogue: lane holds, for batch column j = bb*32 + r32, vocabulary entries
    // tile*256 + wave*64 + vb*32 + 8*(r/4) + 4*half + (r%4)
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
        for (int vb = 0; vb < 2; ++vb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int vbase = tile * LM_COLS + wave * 64 + vb * 32 + 8 * g + 4 * half;
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
                    const float z = acc[vb][bb][4 * g + q];
                    if (a.debug_logits) a.debug_logits[(size_t)j * a.V + v] = z;
                    const float s = (T != 0.0f) ? z / T + gumbel32(ws[q]) : z;
                    if (better(s, v, best_s[bb], best_i[bb])) {
                        best_s[bb] = s;
                        best_i[bb] = v;
                    }
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

hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le) {
    launch_k(le, 0, k_lmhead, dim3(a.n_vtiles), dim3(LM_NT), st, a);
    launch_k(le, 1, k_lmhead_reduce, dim3(a.B), dim3(LM_NT), st, a);
    return hipGetLastError();
}

}  // namespace ss

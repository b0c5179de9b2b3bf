// Internal structures shared by the host side of the library and its kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_sampler.h"

namespace ss {

// Stage-1 summary of one 2048-entry wave tile of one row (32 bytes).
//  * Candidates are written as keys (z, id), unsorted, in cand[row][wave tile].
//  * Every finite entry of the wave tile that is not a candidate has
//    z <= zbeta; zbeta = -inf when every finite entry is a candidate.
struct WaveStat {
    float m;        // max processed logit x' (-inf if none is finite)
    int argmax;     // greedy rows: lowest id attaining m; -1 otherwise
    float zbeta;    // RN(beta / T) of the cut beta in x' (x' < beta, window; x' <= beta, count)
    int ncand;      // candidates written (<= WCAP)
    int nfinite;    // finite processed logits
    int flags;      // WS_OVF, WS_SUM, WS_APX
    float zmin;     // smallest z among the candidates (+inf: none)
    float zm;       // RN(m / T), the z of the maximum (T > 0)
    double s;       // WS_SUM / WS_APX: a mass relative to exp(zm)
    double sc;      // the candidates' mass relative to exp(zm) (binary32 terms)
};
static_assert(sizeof(WaveStat) == 48, "WaveStat layout");

// The window held more than WCAP entries: the candidates are the head of the
// wave tile by count instead.
constexpr int WS_OVF = 1;
// s holds the wave tile's whole mass, exact (count-cut tiles of rows top-k may
// not cut).
constexpr int WS_SUM = 2;
// s holds the mass of the wave tile's non-candidates, relative to RN(m / T) and
// approximate (window-cut tiles of rows top-k may not cut).
constexpr int WS_APX = 4;
// Neither flag: the tile holds more finite entries than the row's top-k, so the
// row is cut by top-k and the mass outside the candidates is not summed (the
// merge bounds what a top-k set deeper than the pool can miss by count).
// With WS_SUM: the tile's non-candidates' mass is also binned by z (Workspace::bins).
constexpr int WS_BIN = 8;
// Bins of a WS_BIN tile: BIN_S per unit of z on the absolute grid floor(-z BIN_S),
// NBIN of them from the one holding the tile's zbeta down; the last also holds
// everything deeper.
constexpr int BIN_S = 32;
constexpr int NBIN = 256;

// What the row finaliser knows about one row's filtered distribution.
// kept(v) <=> key64(z_v, v) >= kappa and (min_p <= 0 or exp(z_v - zmax) >= min_p),
// pi(v) = kept(v) ? exp(z_v - zmax) / W : 0.
struct RowInfo {
    unsigned long long kappa;
    double W;
    float zmax;
    float min_p;
    int n_kept;
    int token;      // sampled token (ss_sample and the bonus row), greedy token for T = 0
    int argmax;     // lowest id among the maxima of x'
    int path;       // 0 tile candidates, 1 whole-row fallback
    int pad[2];
};
static_assert(sizeof(RowInfo) == 48, "RowInfo layout");

// Per-row view of the caller's parameters, as device pointers (host-built;
// every pointer but mask is valid: absent parameters point at defaults).
struct ParamPtrs {
    const float* temperature;
    const int32_t* top_k;
    const float* top_p;
    const float* min_p;
    const float* rep;
    const float* freq;
    const float* pres;
    const int32_t* hist_ids;
    const int32_t* hist_len;
    int32_t hist_stride;
    const int32_t* bias_ids;
    const float* bias_vals;
    const int32_t* bias_len;
    int32_t bias_stride;
    const uint32_t* mask;
    int32_t mask_stride;
    const int32_t* request_ids;
    const int32_t* positions;
    uint64_t seed;
};

struct Workspace {
    WaveStat* wstats;        // [max_rows * n_wt]
    unsigned long long* cand;  // [max_rows * n_wt * WCAP]  candidate keys per wave tile
    RowInfo* rowinfo;        // [max_rows]
    int32_t* row_accept;     // [max_rows]: spec decision per draft row
    double2* resid_tile;     // [max_batch * n_tiles]: residual / target mass per tile
    float* scratch_z;        // [max_rows * V] fallback rows
    float* bins;             // [max_batch * n_wt * NBIN] WS_BIN tiles' masses by z, or null
    int32_t* tree_path;      // [max_rows * tree_dmax]: tokens from the root to each tree node
    int32_t* tree_depth;     // [max_rows]: depth of each tree node (-1: unreachable)
    int32_t* tree_next;      // [max_rows]: accepted child of each tree node (-1: none)
    int tree_dmax;           // path stride (the deepest path a tree of the handle can have)
    int n_tiles;             // 8192-entry workgroup tiles per row
    int n_wt;                // wave tiles per row (WPT per workgroup tile)
    int V;
};

struct SampleArgs {
    const void* logits;
    int64_t row_stride;
    int B;
    int V;
    ParamPtrs p;
    int32_t* out_tokens;
    float* dbg_processed;
    int32_t* dbg_topk;
    int32_t dbg_topk_stride;
    int32_t* dbg_kept;
    float* dbg_probs;
    int32_t* dbg_path;
    Workspace ws;
};

struct SpecArgs {
    const void* target;
    int64_t row_stride;
    const float* draft_probs;  // null: greedy draft, q one-hot at the draft token
    int64_t draft_stride;
    const int32_t* draft_tokens;
    int B;
    int G;
    int V;
    ParamPtrs p;
    int32_t* out_tokens;
    int32_t* out_num_accepted;
    int32_t* seq_tokens;       // null: no append to the request sequences
    int64_t seq_stride;
    int32_t seq_capacity;
    int32_t* seq_len;
    Workspace ws;
};

struct TreeArgs {
    const void* target;        // [B * N] rows: row b * N + n after the path root -> n
    int64_t row_stride;
    const int32_t* parents;    // [B, N]
    const int32_t* tokens;     // [B, N]
    int B;
    int N;
    int V;
    ParamPtrs p;
    int32_t* out_tokens;       // [B, N]
    int32_t* out_nodes;        // [B, N]
    int32_t* out_num_accepted; // [B]
    Workspace ws;
};

// Per (batch row, LM-head vocabulary tile) summary left by the processed
// epilogue: the tile's LM_NC largest keys (z', id) in key order, the next one
// (every other entry of the tile is at most it), the mass below the tile
// maximum, the best Gumbel score and the count of finite entries.
constexpr int LM_NC = 4;
struct LmTileStat {
    unsigned long long key[LM_NC];  // descending; 0 = none
    unsigned long long rest;        // 0 = none
    float mass;                     // sum of exp(z' - z'(key[0])) over the finite entries
    float best_s;                   // the largest z' + g (T > 0) or x' (T = 0)
    int best_i;                     // its id (the lowest among equals), INT_MAX if none
    int nfinite;
    float zmin;                     // the least finite z' (+inf if none)
    int pad;
};
static_assert(sizeof(LmTileStat) == 64, "LmTileStat layout");

// The kept set of an open LM-head row, fixed by the whole-row selection, and
// the best (z' + g, id) key its chunks have found (0 = none yet).
struct LmCut {
    unsigned long long kP;    // kept: key64(z', v) >= kP ...
    unsigned long long best;  // mono32(z' + g) << 32 | ~id, the maximum over the chunks
    float zmax;               // ... and, with min_p > 0, exp(z' - zmax) >= min_p
    float mp;
    float zlo;                // the row's least finite z'
    int total;                // its finite entries
};
static_assert(sizeof(LmCut) == 32, "LmCut layout");

struct LmheadArgs {
    const uint16_t* hidden;
    const uint16_t* weight;
    int B;
    int K;
    int V;
    const float* temperature;
    const int32_t* request_ids;
    const int32_t* positions;
    uint64_t seed;
    int32_t* out_tokens;
    float* debug_logits;
    float2* partials;        // [64 * n_vtiles] (score, id bits)
    int n_vtiles;
    // the per-request pipeline in the epilogue (ss_lmhead_sample_params)
    ParamPtrs p;
    LmTileStat* stats;       // [64 * n_vtiles]
    int32_t* unres;          // [64]: rows the candidates could not resolve
    LmCut* cut;              // [64]: their kept sets and best keys
    float* zmat;             // [64 * V]: z' of those rows, formed again
    int32_t* dbg_path;       // [B] or null: 0 candidates, 1 whole row, 2 no filter or greedy
};

// Optional timing events of a call (see ss_sampler_set_launch_events): launch
// k is bracketed by ev[2k] (its start) and ev[2k + 1] (its end), recorded by
// the dispatch itself.
struct LaunchEvents {
    hipEvent_t ev[16];
    int n;
    hipEvent_t start(int k) const { return 2 * k + 1 < n ? ev[2 * k] : nullptr; }
    hipEvent_t stop(int k) const { return 2 * k + 1 < n ? ev[2 * k + 1] : nullptr; }
};

// Launches kernel k of a call, with its timing events when they are set.
template <class F, class... A>
inline void launch_k(const LaunchEvents& le, int k, F kernel, dim3 grid, dim3 block,
                     hipStream_t st, A... args) {
    if (le.start(k))
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, le.start(k), le.stop(k), 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

hipError_t launch_sample(const SampleArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le);
hipError_t launch_spec(const SpecArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le);
hipError_t launch_tree(const TreeArgs& a, ss_dtype dt, hipStream_t st, const LaunchEvents& le);
hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le);
hipError_t launch_lmhead_params(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le);
// the row kernels of ss_lmhead_sample_params (in the row-kernel source)
void launch_lm_merge(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k);
void launch_lm_slow(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k);
void launch_lm_gumbel(const LmheadArgs& a, hipStream_t st, const LaunchEvents& le, int k);

}  // namespace ss

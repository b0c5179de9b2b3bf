/*
 * ss_sampler.h -- C ABI of the MI355X (gfx950) batched sampling library.
 *
 * One library serves three hot paths that the source pages describe:
 *
 *  - ss_sample: per-request logit processing and token selection in one
 *    batched, graph-capturable launch (SonicSampler abstract, arxivdaily page,
 *    English abstract: grammar-constrained decoding; repetition, frequency and
 *    presence penalties; logit bias; temperature; top-k / top-p / min-p
 *    filtering; hierarchical two-stage top-k; per-request behaviour in one
 *    batch).
 *  - ss_spec_verify: verification of a linear draft by rejection sampling
 *    ("Accelerating Sonar through speculation", Perplexity blog, sections on
 *    speculative decoding and on target-draft decoding: up to n + 1 tokens per
 *    step, acceptance compares the full distributions, the target supplies an
 *    extra token; the accepted count is what the engine must read back).
 *  - ss_lmhead_sample: LM-head GEMM fused with exact Gumbel-max sampling, the
 *    logits never reaching memory (FlashSampling news item, meineki.news, body:
 *    logits formed in on-chip tiles, Gumbel noise added, a per-row maximum per
 *    vocabulary tile kept, a small cross-tile reduction; exact because argmax
 *    decomposes over partitions).
 *
 * Conventions
 *  - Every pointer passed to ss_sample, ss_spec_verify and ss_lmhead_sample
 *    (inputs, outputs, parameter arrays) is a DEVICE pointer on the sampler's
 *    device, except the ss_params / ss_debug structs themselves, which live in
 *    host memory and are read during the call. The caller owns every buffer.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return. They never allocate, copy to the host or synchronise,
 *    so they may be captured in a HIP graph; the launch shape depends only on
 *    (B, G, V, K), never on parameter values.
 *  - Host-detectable argument errors are returned before anything is launched.
 *    Values inside device parameter arrays cannot be checked without a
 *    synchronisation; their ranges are a caller contract stated per field.
 *  - Row-level degenerate data is encoded in the outputs: a row with no
 *    finite processed logit yields token -1.
 *  - Random numbers come from a counter-based Philox4x32-10 generator keyed by
 *    (seed) with counter (request, position, draw >> 2, domain); a draw is
 *    therefore a pure function of those values (domains: 0 sampling,
 *    1 acceptance, 2 residual, 3 Gumbel noise).
 *  - A sampler handle is not thread-safe; use one handle per concurrent stream.
 */
#ifndef SS_SAMPLER_H
#define SS_SAMPLER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ss_sampler ss_sampler; /* opaque; owns its device workspace */

typedef enum {
    SS_OK = 0,
    SS_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, size out of range */
    SS_ERR_UNSUPPORTED = -2,   /* a valid request the library does not serve */
    SS_ERR_OUT_OF_MEMORY = -3, /* workspace allocation failed (create only) */
    SS_ERR_HIP = -4            /* a HIP runtime call or launch failed */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/* Host struct. Limits fixed for the handle's lifetime; workspace is sized from
 * them once, in ss_sampler_create. */
typedef struct {
    int32_t max_batch;   /* max rows (ss_sample) / requests (spec, lmhead), >= 1 */
    int32_t vocab_size;  /* V, 1 .. 262144 */
    int32_t max_draft;   /* max G for ss_spec_verify and N - 1 for ss_tree_verify,
                            0 .. 63 (0: verification unused) */
    int32_t hidden_size; /* K for ss_lmhead_sample, 0 or a multiple of 64 (0: unused) */
    int32_t device;      /* HIP device ordinal */
} ss_sampler_config;

/* Per-request parameters: a host struct holding DEVICE pointers, one entry per
 * row (ss_sample) or per request (ss_spec_verify). NULL disables a feature and
 * takes the stated default. */
typedef struct {
    const float* temperature;        /* [B] required; >= 0 and finite; 0 = greedy */
    const int32_t* top_k;            /* [B]; <= 0 or >= V: off; any k in between is served:
                                        a top-k set reaching past the tile candidates with
                                        non-negligible mass takes the exact whole-row path */
    const float* top_p;              /* [B]; in (0, 1]; 1 = off (NULL: 1) */
    const float* min_p;              /* [B]; in [0, 1]; 0 = off (NULL: 0) */
    const float* repetition_penalty; /* [B]; > 0 (NULL: 1) */
    const float* frequency_penalty;  /* [B] (NULL: 0) */
    const float* presence_penalty;   /* [B] (NULL: 0) */
    const int32_t* history_ids;      /* [B, history_stride]; ids outside [0,V) ignored */
    const int32_t* history_len;      /* [B], each in [0, history_stride]; NULL: no history */
    int32_t history_stride;          /* >= 0, <= 65000 (multiplicities are counted in 16 bits,
                                        with room for up to 63 draft tokens) */
    const int32_t* bias_ids;         /* [B, bias_stride]; ids outside [0,V) ignored */
    const float* bias_values;        /* [B, bias_stride]; applied in array order */
    const int32_t* bias_len;         /* [B], each in [0, bias_stride]; NULL: no bias */
    int32_t bias_stride;             /* >= 0; bias_ids and bias_values share it */
    const uint32_t* grammar_mask;    /* [B, mask_stride] (verify: [B, G+1, mask_stride]);
                                        bit (v & 31) of word (v >> 5), 1 = allowed */
    int32_t mask_stride;             /* words between consecutive rows, >= ceil(V / 32) when
                                        grammar_mask is set (verification: between positions,
                                        row b * (G + 1) + j) */
    const int32_t* request_ids;      /* [B] Philox counter word 0 (NULL: row index) */
    const int32_t* positions;        /* [B] Philox counter word 1 (NULL: 0) */
    uint64_t seed;                   /* Philox key (host value) */
} ss_params;

/* Optional per-call debug outputs of ss_sample (DEVICE pointers, each may be
 * NULL). They cost extra memory traffic; leave them NULL when timing. */
typedef struct {
    float* processed_logits; /* [B, V]: logits after penalties, bias and mask */
    int32_t* topk_ids;       /* [B, topk_stride]: the top-k set (any order), -1 padded;
                                all -1 for rows where top-k is off or T = 0 */
    int32_t topk_stride;     /* columns of topk_ids; the set is cut at this many */
    int32_t* kept_count;     /* [B]: size of the sampling support after all filters */
    float* probs;            /* [B, V]: filtered probabilities (0 outside the support) */
    int32_t* path;           /* [B]: 0 = resolved from the tile candidates,
                                1 = resolved by the exact whole-row fallback (top-k ids and
                                probabilities asked for here can send rows there that
                                would otherwise resolve from the candidates),
                                2 = an unfiltered row drawn from its binned tail (calls
                                without history or bias lists; never with topk_ids or
                                probs asked for) */
} ss_debug;

/* Creates a sampler on cfg->device and allocates its workspace (the only call
 * that allocates). Returns SS_ERR_INVALID_ARG for out-of-range limits (checked
 * before any HIP call), SS_ERR_OUT_OF_MEMORY if the workspace does not fit,
 * SS_ERR_HIP otherwise (for instance a device ordinal that does not exist). */
ss_status ss_sampler_create(const ss_sampler_config* cfg, ss_sampler** out);

/* Frees the workspace. The caller must ensure no enqueued call is pending. */
void ss_sampler_destroy(ss_sampler* s);

/* Static description of a status code. */
const char* ss_status_string(ss_status st);

/* Bytes of device workspace the handle holds. */
int64_t ss_sampler_workspace_bytes(const ss_sampler* s);

/* ss_sampler_set_launch_events -- measurement hook (timing of the kernels).
 *   events    array of n_events hipEvent_t handles created by the caller, or
 *             NULL to clear the hook. The library copies the handles.
 *   n_events  0 .. 16.
 * While set, every ss_sample / ss_spec_verify / ss_lmhead_sample call launches
 * its k-th kernel (k = 0, 1, ...) with events[2k] as its start and
 * events[2k + 1] as its stop event (hipExtLaunchKernel: the dispatch records
 * them when the kernel begins and ends), for every k with 2k + 1 < n_events.
 * ss_sample launches 2 kernels (tile scan, row merge), ss_spec_verify 4 (tile
 * scan, row merge, residual tile sums, per-request finish), ss_tree_verify 5
 * (tree paths, tile scan, row merge and child tests, residual tile sums,
 * per-request finish), ss_lmhead_sample 2 (fused GEMM tiles, cross-tile
 * reduction) and ss_lmhead_sample_params 5 (as listed there).
 * Returns SS_ERR_INVALID_ARG for a null handle or n_events outside 0 .. 16.
 * Not meant for graph capture. */
ss_status ss_sampler_set_launch_events(ss_sampler* s, void* const* events, int32_t n_events);

/* ss_sample -- sample one token per row of a [B, V] logits matrix.
 *   logits      [B, row_stride] of dtype (SS_F32 or SS_BF16), element-aligned,
 *               row_stride >= V. Rows whose start is 16-byte aligned are read
 *               with 16-byte vector loads, others element by element.
 *               Entries are finite or -inf (-inf = never sampled); NaN and
 *               +inf are outside the contract (the result is unspecified).
 *   B           0 .. max_batch (0 is a no-op).
 *   params      per-row parameters (host struct of device pointers).
 *   out_tokens  [B] int32: sampled token, or -1 when a row has no finite logit.
 *   debug       NULL or optional debug outputs.
 * Per row: penalties -> bias -> grammar mask -> temperature (T = 0: greedy,
 * lowest id among the maxima) -> top-k -> top-p -> min-p -> inverse-CDF draw in
 * (z descending, id ascending) order with u = u24(Philox(seed; request,
 * position, 0, domain 0)). Ties always go to the lower token id. */
/* Errors (returned before any launch): SS_ERR_INVALID_ARG for a null handle,
 * B < 0 or B > max_batch, null logits / out_tokens / params / temperature, a
 * dtype other than SS_F32 / SS_BF16, row_stride < V, logits not aligned to
 * their element size, history_stride outside 0 .. 65000, bias or history
 * pointers given without their companions, mask_stride < ceil(V / 32) with a
 * mask, or topk_ids given with topk_stride < 1; SS_ERR_HIP if the launch fails.
 * B = 0 returns SS_OK without touching any pointer but the handle. */
ss_status ss_sample(ss_sampler* s, const void* logits, ss_dtype dtype, int64_t row_stride,
                    int32_t B, const ss_params* params, int32_t* out_tokens,
                    const ss_debug* debug, void* stream);

/* ss_spec_verify -- verify a linear draft of G tokens per request.
 *   target_logits [B, G+1, row_stride] of dtype: target logits at the G draft
 *                 positions and the bonus position (same layout rules as above).
 *   draft_probs   [B, G, draft_stride] float32 draft probabilities (draft_stride >= V),
 *                 or NULL for a greedy draft, one that takes its top token at every
 *                 step ("Accelerating Sonar through speculation", target-draft
 *                 section): q is then one-hot at each draft token, so draft j is
 *                 accepted iff u < p(d_j) and a rejection resamples from p with d_j
 *                 removed; no draft row is read (draft_stride is ignored).
 *   draft_tokens  [B, G] int32 draft tokens.
 *   B, G          0 .. max_batch, 1 .. max_draft.
 *   out_tokens    [B, G+1] int32: accepted drafts, then the final (corrected or
 *                 bonus) token, then -1 padding.
 *   out_num_accepted [B] int32 in [0, G]; stays on the device (reading it back
 *                 is the caller's synchronisation point).
 * Row j of a request uses the request's parameters and, as penalty history, the
 * request history followed by draft tokens 0 .. j-1. Greedy requests (T = 0)
 * accept on exact match with the greedy token; others accept draft j with
 * probability min(1, p/q) (u from domain 1 at position + j), on rejection
 * resample from the normalised max(0, p - q) in token-id order (domain 2), and
 * after full acceptance draw the bonus token as ss_sample would at position + G.
 * Launches four kernels: the tile scan over every target row, the row merge and
 * accept tests, the residual tile sums and the per-request finish (the last
 * two only do work for rejected requests). */
/* Errors: as ss_sample, plus SS_ERR_INVALID_ARG for G outside 1 .. max_draft,
 * null draft_tokens / out_tokens / out_num_accepted, or draft_probs given with
 * draft_stride < V. */
ss_status ss_spec_verify(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                         int64_t row_stride, const float* draft_probs, int64_t draft_stride,
                         const int32_t* draft_tokens, int32_t B, int32_t G,
                         const ss_params* params, int32_t* out_tokens,
                         int32_t* out_num_accepted, void* stream);

/* Per-request token sequences kept on the device (all pointers device). */
typedef struct {
    int32_t* tokens;   /* [B, stride] int32: request b's tokens, slots 0 .. capacity-1 */
    int64_t stride;    /* >= capacity */
    int32_t capacity;  /* slots per request, >= 0 */
    int32_t* len;      /* [B] int32: tokens already in each sequence, 0 .. capacity;
                          read and advanced in place */
} ss_sequences;

/* ss_spec_verify_scatter -- ss_spec_verify, then the emitted tokens placed into
 * the request sequences on the device ("Accelerating Sonar through
 * speculation", section on single-token MTP scheduling: after acceptance a
 * kernel puts the next target tokens into their slots, so no GPU-to-CPU
 * synchronisation follows acceptance). Request b's accepted drafts and final
 * token, out_tokens[b, 0 .. n_b], go to seq->tokens[b, len_b .. len_b + n_b]
 * and len_b becomes len_b + n_b + 1; slots at or beyond capacity are not
 * written and len_b stops at capacity (keep capacity >= len_b + G + 1 to lose
 * nothing). params->positions may be seq->len itself: every read of a
 * request's position precedes its length update, so consecutive calls on one
 * stream advance the Philox positions with the sequences, and nothing needs
 * to be read back between steps. Same kernels as ss_spec_verify (the append is
 * part of the last launch); seq = NULL is ss_spec_verify.
 * Errors: as ss_spec_verify, plus SS_ERR_INVALID_ARG for a seq with null
 * tokens or len, capacity < 0 or stride < capacity. */
ss_status ss_spec_verify_scatter(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                                 int64_t row_stride, const float* draft_probs,
                                 int64_t draft_stride, const int32_t* draft_tokens, int32_t B,
                                 int32_t G, const ss_params* params, int32_t* out_tokens,
                                 int32_t* out_num_accepted, const ss_sequences* seq,
                                 void* stream);

/* ss_tree_verify -- verify a draft tree per request ("Accelerating Sonar
 * through speculation", EAGLE section: the draft explores a tree in which each
 * node holds its draft's top-K candidates for the next token; the longest
 * acceptable path is kept and the target adds one token).
 *   target_logits [B, N, row_stride] of dtype: row b * N + n holds the target's
 *                 logits after the path from the root to node n (node 0 = the
 *                 root, the last committed token).
 *   parents       [B, N] int32: parent node of each node (entry 0 ignored).
 *                 Node n >= 1 hangs below parents[n] when 0 <= parents[n] < n;
 *                 otherwise it, and everything below it, is unreachable.
 *   tokens        [B, N] int32: draft token of each node (entry 0 ignored).
 *   B, N          0 .. max_batch, 2 .. max_draft + 1.
 *   params        as ss_sample; a grammar mask, when given, has one row per
 *                 node (row b * N + n, mask_stride words apart).
 *   out_tokens    [B, N] int32: the accepted path's tokens, then the final
 *                 token, then -1 padding.
 *   out_nodes     [B, N] int32: the tree node of each accepted token, then -1.
 *   out_num_accepted [B] int32: the accepted path's length (0 .. N - 1).
 * Node n uses the request's parameters, the request history followed by the
 * tokens on its root path as penalty history, and position + depth(n). Walking
 * down from the root, the children of the current node are tested in index
 * order as one-hot proposals against the residual target: child i with token d
 * is accepted iff u < p(d) / (1 - p of the siblings rejected before it), u from
 * domain 1 (acceptance) at position + depth, draw i; greedy rows (T = 0) accept
 * the child holding the greedy token. The final token is the greedy token, a
 * draw from p without the rejected children's tokens in token-id order (domain
 * 2) when the end node has children, or the end node's own draw as ss_sample
 * would make it when it is a leaf. A chain (one child per node) gives exactly
 * ss_spec_verify with a greedy draft (draft_probs NULL).
 * Launches five kernels. Errors: as ss_sample, plus SS_ERR_INVALID_ARG for N
 * outside 2 .. max_draft + 1 or null parents / tokens / outputs. */
ss_status ss_tree_verify(ss_sampler* s, const void* target_logits, ss_dtype dtype,
                         int64_t row_stride, const int32_t* parents, const int32_t* tokens,
                         int32_t B, int32_t N, const ss_params* params, int32_t* out_tokens,
                         int32_t* out_nodes, int32_t* out_num_accepted, void* stream);

/* ss_lmhead_sample -- fused LM-head GEMM + Gumbel-max sampling.
 *   hidden        [B, K] bfloat16 bits (row-major), 16-byte aligned.
 *   weight        [V, K] bfloat16 bits (row-major), 16-byte aligned.
 *   B             1 .. min(max_batch, 64); K = hidden_size of the handle.
 *   temperature   [B] float32 (>= 0; 0 = argmax of the logits, no noise).
 *   request_ids, positions  [B] int32 Philox counter words (NULL: row index / 0).
 *   out_tokens    [B] int32.
 *   debug_logits  NULL, or [B, V] float32 to receive the unscaled logits.
 * Token = lowest v attaining max_v (z[b,v] / T_b + g(Philox(seed; request,
 * position, v >> 2, domain 3)[v & 3])), g = -ln(-ln U), U = 1 - (w + 0.5) 2^-32.
 * Per 128-row vocabulary tile the GEMM kernel keeps only a (max, argmax) pair
 * per batch row; a second launch reduces the pairs of each row (the result does
 * not depend on the tiling: argmax decomposes over any partition).
 * Errors: SS_ERR_INVALID_ARG for a null handle, a handle created with
 * hidden_size 0, B outside 1 .. min(max_batch, 64), or null hidden / weight /
 * temperature / out_tokens; SS_ERR_UNSUPPORTED for hidden or weight not 16-byte
 * aligned; SS_ERR_HIP if a launch fails. */
ss_status ss_lmhead_sample(ss_sampler* s, const uint16_t* hidden, const uint16_t* weight,
                           int32_t B, const float* temperature, const int32_t* request_ids,
                           const int32_t* positions, uint64_t seed, int32_t* out_tokens,
                           float* debug_logits, void* stream);

/* ss_sample_noalloc -- ss_sample without a handle, for callers that cannot
 * allocate device memory: code recorded under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It runs the same kernels as
 * ss_sample, but for the binned tail of unfiltered rows (its scratch holds no
 * bins: such rows take the whole-row path), and returns the same tokens for the
 * same arguments, up to draws within rounding (1e-6 of the row's mass) of a
 * boundary of the cumulative distribution, which the two paths sum in different
 * orders.
 *   Device:   the current HIP device; `stream` must belong to it.
 *   Scratch:  a static device array of SS_NOALLOC_SCRATCH_BYTES per GPU,
 *             reserved with the library's code object (held until the process
 *             ends). The first call on a device looks up its address there
 *             (make that first call outside graph capture); no call allocates
 *             or frees memory.
 *   Limits:   B <= SS_NOALLOC_MAX_BATCH and B * V <= SS_NOALLOC_MAX_ENTRIES
 *             (every size up to B = 64 rows of a 131072-entry vocabulary);
 *             larger requests return SS_ERR_UNSUPPORTED before any launch.
 *   Arguments as for ss_sample, with V (1 .. 262144) passed per call; no
 *   debug outputs. Nothing in the scratch needs clearing between calls.
 *   Every call on one GPU shares that GPU's scratch: two calls whose work
 *   overlaps in time on the same GPU (different streams, or different host
 *   threads) race and may return wrong tokens. Calls ordered on one stream do
 *   not race.
 * Errors: SS_ERR_INVALID_ARG for B < 0, V outside 1 .. 262144, or any check
 * ss_sample makes on logits, params and out_tokens; SS_ERR_UNSUPPORTED beyond
 * the limits above or on a device ordinal >= 64; SS_ERR_HIP if the address
 * lookup or a launch fails. B = 0 returns SS_OK at once. */
#define SS_NOALLOC_MAX_BATCH 64
#define SS_NOALLOC_MAX_ENTRIES 8388608
#define SS_NOALLOC_SCRATCH_BYTES 37748736
ss_status ss_sample_noalloc(const void* logits, ss_dtype dtype, int64_t row_stride, int32_t B,
                            int32_t V, const ss_params* params, int32_t* out_tokens,
                            void* stream);

/* ss_lmhead_sample_params -- the fused LM-head GEMM with the whole per-request
 * pipeline in its epilogue (SonicSampler abstract: penalties, bias, grammar
 * mask, temperature and top-k / top-p / min-p per request in one batched pass;
 * FlashSampling news item: Gumbel-max sampling folded into the GEMM so the
 * logits stay on chip).
 *   hidden, weight, B   as ss_lmhead_sample (K = hidden_size of the handle).
 *   params              as ss_sample: temperature, filters, penalties over the
 *                       history, logit bias, grammar mask (row b, mask_stride
 *                       words apart), request ids, positions and seed.
 *   out_tokens          [B] int32.
 *   debug_path          NULL, or [B] int32: 0 = decided on the tile candidates,
 *                       1 = decided over the whole row of z',
 *                       2 = no filter or greedy (the tiles' best scores).
 * Each GEMM tile applies penalties, bias, mask and temperature to its logits
 * (z' = x'/T as in ss_sample) and keeps, per batch row, its 4 largest keys, the
 * next key, the mass below its maximum and its best Gumbel score. T = 0: the
 * greedy token of x'. No filter: the lowest id attaining max z' + g (g from
 * domain 3 at the token's id, as ss_lmhead_sample). With filters: the same
 * maximum over the kept support (top-k, then top-p over the top-k mass, then
 * min-p), which Gumbel-max samples from the filtered distribution exactly. The
 * support is taken from the tiles' candidates whenever the cuts fall among the
 * entries they certify (every key above the largest next key); other rows are
 * selected over their whole row of z', which the GEMM kernel also writes to the
 * workspace for every row with a filter (4 bytes per entry, against the 2 K of
 * weight per vocabulary entry the GEMM reads; rows without a filter never
 * leave the chip). Launches five kernels: GEMM with summaries, row merge, the
 * whole-row selection of the kept set, the Gumbel pass over the kept set (32
 * workgroups per row) and the token write; the last three return at once for
 * rows the candidates resolved. Errors: as ss_lmhead_sample, and the checks
 * ss_sample makes on params. */
ss_status ss_lmhead_sample_params(ss_sampler* s, const uint16_t* hidden, const uint16_t* weight,
                                  int32_t B, const ss_params* params, int32_t* out_tokens,
                                  int32_t* debug_path, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_SAMPLER_H */

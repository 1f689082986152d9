/*
 * zha.h - C ABI of libzha: the decode hot path of Zyphra Hierarchical
 * Attention (ZHA) on MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *  - "Subquadratic Attention with a Hierarchical Tree-Structured Indexer"
 *    (summary page of the technical report), §Tree Construction: every chunk
 *    of b contiguous keys is compressed to a summary key, the attention of a
 *    reference query over the chunk with the chunk as keys and values; higher
 *    levels are built the same way from their children's summaries.
 *  - same page, §Routing: at each level keep the smallest score-ordered prefix
 *    of candidate nodes holding a fraction p of the softmax mass, expand the
 *    kept nodes' children, down to leaf chunks; attend exactly over
 *    {token 0} U kept leaf chunks U the query's current chunk.
 *  - "Zyphra Hierarchical Attention: The End of Quadratic Attention?",
 *    §How the tree is built and searched: contiguous chunks, the full KV
 *    cache stays at the leaves, token 0 is always kept as a sink.
 *
 * Fixed readings (the pages leave these open):
 *  - one reference query per (level, kv head); a summary is the
 *    softmax(r . c * scale)-weighted mean of its children c;
 *  - a node's score is q . summary * scale, computed in fp32; the cut orders
 *    candidates by (score desc, node id asc) and keeps the smallest prefix
 *    with cumulative mass >= p of the candidates' total; p >= 1 keeps all;
 *  - only complete nodes exist (node i of level l covers tokens
 *    [i*b^l, (i+1)*b^l)); complete nodes whose parent is incomplete enter as
 *    candidates at their own level; at the top level every complete node is a
 *    candidate;
 *  - a query that sees N tokens attends {0} U kept leaf chunks U
 *    [b*floor((N-1)/b), N), each token once.
 *
 * Conventions for every function:
 *  - All tensor pointers are DEVICE pointers, owned by the caller, and must
 *    stay valid until the work enqueued on `stream` has finished. The library
 *    never allocates or frees memory and keeps no pointer after returning; the
 *    one memory it owns is the static scratch of zha_attend_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued asynchronously on it; no call synchronises except
 *    zha_read_device_status.
 *  - Host-detectable errors (null pointers, unsupported shapes, a workspace
 *    that is too small) are returned before anything is enqueued. Conditions
 *    only the device can see (a selection larger than sel_capacity, an append
 *    past capacity) set bits in a status word inside the workspace, read with
 *    zha_read_device_status.
 *  - Layouts (row-major, innermost last):
 *      K, V           [B, H_kv, capacity, d]   bf16 or fp32 (geom.kv_dtype)
 *      ref_q          [L, H_kv, R, d]          fp32 (R = n_refs, 1 for SUMMARY)
 *      summaries      fp32; level l (1-based) starts at element
 *                     sizes.level_offset[l-1]; tangent r of node i of (batch
 *                     s, kv head h) is row ((s*H_kv + h)*sizes.level_nodes[l-1]
 *                     + i)*R + r (R = 1 for SUMMARY scoring); with TANGENT
 *                     scoring its offset is element level_bias_offset[l-1] +
 *                     that row index
 *      q, out         [B, T, H_q, d]           fp32
 *      lse            [B, T, H_q]              fp32 (natural log, scale included)
 *      seq_lens       [B]                      int32, tokens present per sequence
 *      q_pos          [B, T]                   int32 position of each query row,
 *                     or NULL for the last T positions (seq_lens[s]-T+t); a
 *                     row at position t sees tokens [0, t] and only the tree
 *                     nodes complete within them
 *      sel_blocks     [B, T, H_q, sel_capacity] int32 kept leaf-chunk ids, ascending
 *      n_sel          [B, T, H_q]              int32 true number kept
 *    Query head h reads kv head h / (H_q / H_kv).
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define ZHA_API __attribute__((visibility("default")))
#else
#define ZHA_API
#endif

typedef int32_t zha_status;

#define ZHA_OK               0
#define ZHA_ERR_NULL         1  /* a required pointer is NULL */
#define ZHA_ERR_SHAPE        2  /* inconsistent sizes (H_q % H_kv, T, capacity, ...) */
#define ZHA_ERR_UNSUPPORTED  3  /* a size this build has no kernel for */
#define ZHA_ERR_WORKSPACE    4  /* workspace smaller than zha_query_sizes asks for */
#define ZHA_ERR_CAPACITY     5  /* device: selection or append exceeded a capacity */
#define ZHA_ERR_HIP          6  /* the HIP runtime reported an error */

/* Device status bits (zha_read_device_status). */
#define ZHA_DEV_SEL_OVERFLOW     1u  /* some n_sel exceeded sel_capacity: list truncated */
#define ZHA_DEV_APPEND_OVERFLOW  2u  /* an append would pass capacity: nothing written */

#define ZHA_KV_BF16 0
#define ZHA_KV_F32  1

#define ZHA_MAX_LEVELS 8

typedef struct zha_geom {
    int32_t batch;       /* B >= 1 */
    int32_t n_q_heads;   /* H_q, a multiple of H_kv, H_q / H_kv <= 16 */
    int32_t n_kv_heads;  /* H_kv >= 1 */
    int32_t head_dim;    /* d: 64 or 128 */
    int32_t branching;   /* b: a power of two in [2, 256] */
    int32_t n_levels;    /* L: 1..ZHA_MAX_LEVELS */
    int64_t capacity;    /* tokens allocated per sequence, < 2^31 */
    int32_t kv_dtype;    /* ZHA_KV_BF16 or ZHA_KV_F32 */
    float   scale;       /* score scale; 0 selects 1/sqrt(d) */
    /* Per-level top-p schedule ("Subquadratic Attention with a Hierarchical
     * Tree-Structured Indexer", Future Directions: scaling p with depth, since
     * a fixed p < 1 keeps about p^L of the mass after L levels). Entry l-1 in
     * (0, 1] is the cut fraction at level l and overrides a call's top_p
     * there; 0 keeps the call's top_p. Entries at levels past n_levels must
     * be 0. A zero-initialised struct routes every level with top_p. */
    float   level_p[ZHA_MAX_LEVELS];
    /* Node scoring ("Subquadratic Attention with a Hierarchical
     * Tree-Structured Indexer", §Tree Construction):
     *  ZHA_SCORE_SUMMARY (0): one reference query per (level, kv head); a node
     *    stores the softmax(r . c * scale)-weighted mean of its children and
     *    scores q . summary * scale. n_refs must be 0 or 1.
     *  ZHA_SCORE_TANGENT (1): n_refs = R reference queries per (level, kv
     *    head); a node stores R tangents (key k_r, offset b_r) and scores
     *    max_r (q . k_r * scale + b_r). At level 1, k_r is the attention of
     *    reference query r over the chunk (keys as values) and b_r the chunk's
     *    log-sum-exp at r minus r . k_r * scale. Above, each child enters with
     *    its best tangent at r (lowest index on ties) and its offset added to
     *    the pooling logit: the tangent at r of the log-sum-exp of the
     *    children's estimates. Routing then runs the same top-p cut.
     * ref_q is [L, H_kv, n_refs, d]. */
    int32_t n_refs;      /* R: 0 or 1 for SUMMARY, 1..16 for TANGENT */
    int32_t scoring;     /* ZHA_SCORE_SUMMARY or ZHA_SCORE_TANGENT */
    /* Compressed value summaries ("Subquadratic Attention with a Hierarchical
     * Tree-Structured Indexer", Future Directions: pruned subtrees contribute
     * coarse attention outputs). 1: every node also stores a value summary,
     * its children's values pooled with its key summary's weights (build and
     * append then read V), and zha_attend / zha_attend_noalloc add one
     * pseudo-token per candidate a level's cut did not keep: logit its score
     * plus ln(its tokens outside the sink and the current chunk), value its
     * value summary; out and lse are the softmax over the exact tokens and the
     * pseudo-tokens. zha_sparse_attend stays exact over I. SUMMARY scoring
     * only. 0: off. */
    int32_t value_summaries;
} zha_geom;

#define ZHA_SCORE_SUMMARY 0
#define ZHA_SCORE_TANGENT 1
#define ZHA_MAX_REFS 16

typedef struct zha_sizes {
    size_t  summaries_bytes;                 /* fp32 summary buffer for all levels */
    size_t  workspace_bytes;                 /* scratch for every call with up to max_rows query rows */
    int64_t level_nodes[ZHA_MAX_LEVELS];     /* node slots per (batch, kv head) and level: capacity / b^l */
    int64_t level_offset[ZHA_MAX_LEVELS];    /* element offset of each level's keys inside summaries */
    int64_t level_bias_offset[ZHA_MAX_LEVELS];/* element offset of each level's tangent offsets (TANGENT only) */
    int64_t level_value_offset[ZHA_MAX_LEVELS];/* element offset of each level's value summaries [B, H_kv, nodes, d]
                                                  (value_summaries only) */
    int64_t level_sel_offset[ZHA_MAX_LEVELS];/* element offset of each level inside a level_sel buffer */
    size_t  level_sel_bytes;                 /* bytes of a level_sel buffer for max_rows rows */
    int32_t max_rows;                        /* B*T rows the workspace was sized for */
    /* Row tiles (one sequence, B = 1): zha_route, zha_attend, zha_sparse_attend
     * and zha_dense_attend accept a workspace smaller than workspace_bytes and
     * then run their rows in tiles, the largest halving of t whose layout fits
     * (not with level_sel, whose layout follows the whole call). For max_t rows
     * a workspace of workspace_bytes_tiled (at most 4 GiB where the whole call
     * needs more) runs tiles of tile_rows rows. */
    int32_t tile_rows;
    size_t  workspace_bytes_tiled;
} zha_sizes;

/* Sizes of the summary buffer and workspace for `geom` and calls with at most
 * `max_t` query rows per sequence (max_t >= 1). Host only, enqueues nothing. */
ZHA_API zha_status zha_query_sizes(const zha_geom* geom, int32_t max_t, zha_sizes* out);

/* Build every complete node of every level for the first seq_lens[s] tokens of
 * each sequence [Tree Construction]. K is read, summaries are written. V is
 * read only with geom.value_summaries (else it may be NULL). ws must hold
 * zha_query_sizes(...).workspace_bytes (any max_t). */
ZHA_API zha_status zha_build_tree(const zha_geom* geom, const void* K, const void* V, const float* ref_q,
                          const int32_t* seq_lens, float* summaries,
                          void* ws, size_t ws_bytes, void* stream);

/* Append t_new tokens to every sequence: k_new, v_new are [B, H_kv, t_new, d]
 * in the cache dtype. Rows are written at seq_lens[s] .. seq_lens[s]+t_new-1,
 * every node they complete is summarised (bit-identical to zha_build_tree),
 * then seq_lens[s] += t_new. A sequence that would pass capacity is left
 * untouched and ZHA_DEV_APPEND_OVERFLOW is raised. [the tree is built on the
 * fly as the context grows: A query's path through the tree, step by step] */
ZHA_API zha_status zha_append(const zha_geom* geom, void* K, void* V, const void* k_new, const void* v_new,
                      int32_t t_new, int32_t* seq_lens, const float* ref_q, float* summaries,
                      void* ws, size_t ws_bytes, void* stream);

/* Route T query rows per sequence top-down through the tree [Routing].
 * Writes sel_blocks / n_sel. level_stats (nullable) receives
 * [B, T, H_q, L, 2] int32 (candidates, kept) per level (index l-1).
 * level_sel (nullable) receives every level's kept ids, ascending: with
 * R = B*T rows, level l of row r = s*T + t, head h starts at element
 * R*H_q*sizes.level_sel_offset[l-1] + (r*H_q + h) * sizes.level_nodes[l-1]
 * (sizes from zha_query_sizes for the same geom; R*H_q*sum(level_nodes)
 * elements in all).
 * top_p in (0, 1]. sel_capacity >= 1. */
ZHA_API zha_status zha_route(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos,
                     const float* summaries, const int32_t* seq_lens, float top_p,
                     int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel,
                     int32_t* level_stats, int32_t* level_sel,
                     void* ws, size_t ws_bytes, void* stream);

/* Exact attention of each query row over {0} U its kept leaf chunks U its
 * current chunk [Routing, o(q)]. Uses the first min(n_sel, sel_capacity)
 * entries of each list. out and lse as in the layouts above. */
ZHA_API zha_status zha_sparse_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos,
                             const void* K, const void* V, const int32_t* seq_lens,
                             const int32_t* sel_blocks, const int32_t* n_sel, int32_t sel_capacity,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* zha_route followed by zha_sparse_attend on one stream (identical results).
 * One difference: if a kept list overflows sel_capacity (ZHA_DEV_SEL_OVERFLOW),
 * the list is truncated but the attention still covers every kept chunk. */
ZHA_API zha_status zha_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos,
                      const void* K, const void* V, const float* summaries, const int32_t* seq_lens,
                      float top_p, int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel,
                      int32_t* level_stats, int32_t* level_sel, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* zha_attend for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels and results, with no workspace argument. Its scratch is a static
 * 64 MiB array inside the library, one per GPU the library runs on, held until
 * the process ends; the call allocates and frees nothing. A call whose layout
 * needs more (zha_query_sizes(geom, t).workspace_bytes > 64 MiB) returns
 * ZHA_ERR_WORKSPACE before anything is enqueued. The first call on a device
 * zeroes the whole array; every call zeroes its status word. dev_status
 * (nullable, a device pointer) receives the call's ZHA_DEV_* bits, written
 * after its last kernel on `stream`. Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents: calls that overlap on one GPU
 * (concurrent streams or threads) race and must be serialised by the caller. */
ZHA_API zha_status zha_attend_noalloc(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos,
                              const void* K, const void* V, const float* summaries, const int32_t* seq_lens,
                              float top_p, int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel,
                              int32_t* level_stats, int32_t* level_sel, float* out, float* lse,
                              uint32_t* dev_status, void* stream);

/* Dense baseline: exact attention of each row over all tokens it sees
 * [The Quadratic Bottleneck: decode re-reads the whole cache per token]. */
ZHA_API zha_status zha_dense_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos,
                            const void* K, const void* V, const int32_t* seq_lens,
                            float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Wait for `stream`, then read (and, if clear != 0, reset) the device status
 * word of workspace `ws` into *out (ZHA_DEV_* bits). The only synchronising call. */
ZHA_API zha_status zha_read_device_status(void* ws, void* stream, uint32_t* out, int32_t clear);

/* Kernel timing for benchmarks, the per-kernel terms of the latency model
 * ("Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
 * §Latency Scaling, eqs. (3)-(4)). While active, every launch whose label
 * matches `label` is bracketed by two HIP events on its own stream. Labels:
 * build_level@l, append_fused, append_rows, advance_seq, route_score@l,
 * route_cut@l, attn_bitmap, attn_items, attend, attend_combine; a label without "@l"
 * matches every level. NULL stops recording. At most 8192 launches are kept
 * (later ones are counted as dropped). Host-side state shared by all threads:
 * for single-threaded benchmarks only. Creating the event pool is the only
 * allocation; it happens here, never in the timed calls. */
ZHA_API zha_status zha_profile_start(const char* label);

/* Wait for the recorded events, return the summed kernel time in milliseconds,
 * the number of launches timed and the number dropped, then clear the record
 * (recording stays active). */
ZHA_API zha_status zha_profile_collect(double* total_ms, int64_t* launches, int64_t* dropped);

/* Static text for a status code. */
ZHA_API const char* zha_status_string(zha_status s);

/* Text of the last error raised on the calling thread ("" if none). */
ZHA_API const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */

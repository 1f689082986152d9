// zha_internal.h - layout arithmetic and kernel parameter blocks shared by the
// host entry points and the kernel launchers of libzha. Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/zha.h"

namespace zha {

constexpr int kWave = 64;
constexpr int kMaxGroup = 16;          // H_q / H_kv handled by one kernel group
constexpr int kAttnWorkgroups = 512;   // attention workgroups when pairs are few (launch and partial slots: this + pairs)
constexpr size_t kAlign = 256;
constexpr int kScoreThreads = 64;      // scoring workgroup: one wave, its active parents one at a time
constexpr int kScoreWaves = 2048;      // scoring waves per launch: what the chip holds at once

// Scoring workgroups per (row, kv head) for a level with `slots` parent slots:
// about kScoreWaves in all over `pairs` (row, kv head) pairs, each with at
// most 64 slots (the wave's lanes build their masks).
inline int64_t score_groups(int64_t slots, int64_t pairs) {
    const int64_t target = (kScoreWaves + pairs - 1) / (pairs > 0 ? pairs : 1);
    int64_t w = target < slots ? target : slots;
    const int64_t need = (slots + 63) / 64;
    w = w > need ? w : need;
    return w > 0 ? w : 1;
}

// Launch shape of a level's scoring. With at most 64 (row, kv head) pairs the
// waves are dealt out in the kernel by each pair's parent count (the kept
// counts of the level above), `need` at least per pair so that no wave holds
// more than 64 slots: the heavy pairs, whose parents would otherwise queue up
// one after another in a few waves, get most of the chip. With more pairs
// every pair gets score_groups waves (a grid of runs x pairs).
struct ScoreShape {
    bool balanced;
    int64_t waves;      // balanced: the 1-D grid; otherwise runs per pair
    int64_t need;       // balanced: waves every pair gets at least
    int64_t max_runs;   // most waves one pair can get (columns of the split cut's maxima)
};
inline ScoreShape score_shape(int64_t slots, int64_t pairs) {
    ScoreShape s{};
    if (pairs <= 64) {
        s.balanced = true;
        s.need = slots > 0 ? (slots + 63) / 64 : 1;
        s.waves = kScoreWaves > 2 * s.need * pairs ? kScoreWaves : 2 * s.need * pairs;
        s.max_runs = s.waves - (pairs - 1) * s.need;
    } else {
        s.balanced = false;
        s.waves = score_groups(slots, pairs);
        s.need = s.waves;
        s.max_runs = s.waves;
    }
    return s;
}
constexpr int kCutBins = 2048;         // mass bins of a cut's first pass
constexpr int kSplitSlice = 2048;      // candidates per workgroup of the split cut
constexpr int kSplitSliceLog2 = 11;
constexpr int kSplitMaxPairs = 128;    // (row, head) pairs up to which a level's cut is split over workgroups
constexpr int kSplitMaxSlices = 1024;  // slices per (row, head) the split cut's boundary kernel can scan

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Geometry after validation, with everything the kernels need precomputed.
struct Geo {
    int B, Hq, Hkv, G, D, b, lb, L, kv_dtype;   // lb = log2(b)
    int64_t cap;                       // tokens per sequence
    float scale;
    int64_t nodes[ZHA_MAX_LEVELS];     // node slots per (batch, kv) per level
    int64_t span[ZHA_MAX_LEVELS + 1];  // tokens per node of level l (index l-1); span[L] = b^(L+1)
    int64_t sum_off[ZHA_MAX_LEVELS];   // element offset of each level in the summary buffer
    int64_t sel_off[ZHA_MAX_LEVELS];   // element offset of each level in a level_sel buffer (per row count)
    int64_t nodes_total;               // sum of nodes[l]
    float level_p[ZHA_MAX_LEVELS];     // per-level cut fraction, 0 = the call's top_p
    int R;                             // tangents per node (reference queries per level and kv head)
    bool tangent;                      // tangent scoring: offsets stored, score = max over the R tangents
    int64_t bias_off[ZHA_MAX_LEVELS];  // element offset of each level's tangent offsets in the summary buffer
    bool vsum;                         // compressed value summaries
    int64_t val_off[ZHA_MAX_LEVELS];   // element offset of each level's value summaries
    int64_t summ_total;                // elements of the summary buffer
};

// Level-1 bitmap words -> attention items: a pair's words in segments, one
// workgroup per segment (kItemsSegFew words with few pairs, else one per thread).
constexpr int kItemsThreads = 256;
constexpr int kItemsSegFew = kWave;
constexpr int kItemsFewPairs = 64;
constexpr int kItemsRecountSegs = 32;  // more segments per pair than this: count them in a pass of their own
inline int items_seg_words(int64_t pairs) { return pairs <= kItemsFewPairs ? kItemsSegFew : kItemsThreads; }
inline int64_t items_segments(const Geo& g, int64_t pairs) {
    const int64_t words = (g.nodes[0] + 1 + 31) / 32;     // chunks incl. the current one
    const int sw = items_seg_words(pairs);
    const int64_t n = (words + sw - 1) / sw;
    return n > 1 ? n : 1;
}

constexpr int kPseudoMaxRuns = 64;     // pseudo-token waves per (row, kv head) and level

// Byte layout of the workspace for `rows` query rows.
struct WsLayout {
    size_t status;        // uint32 device status word (256-byte header)
    size_t qpos;          // int32  [rows] positions of a row tile's rows when the caller passes none
    size_t scores;        // float  [rows, Hq, nodes_total] dense-by-node scores, level offsets = sel_off
    size_t kept;          // int32  [rows, Hq, nodes_total] kept lists per level (level 1 unused)
    size_t kept_cnt;      // int32  [rows, Hq, L]
    size_t bitmap;        // uint32 [rows, Hq, bm_words_total] kept bitmaps per level (a spare bit for index nodes[l])
    size_t bm_off[ZHA_MAX_LEVELS];    // word offset of each level inside a row-head bitmap
    int64_t bm_words_total;
    size_t aitems;        // int2   [rows, Hkv, nodes[0] + 2] attention items (block, head mask)
    size_t acnt;          // int32  [rows, Hkv]
    size_t segcnt;        // int32  [rows, Hkv, items_segments] items per bitmap segment (long bitmaps only)
    size_t plan;          // int64  [2, rows * Hkv + 1] exclusive prefixes of attention groups and workgroup shares per (row, kv head)
    size_t partial;       // float  [kAttnWorkgroups + rows * Hkv, G, D + 4] split-K partial state per workgroup (max, sum, 2 pad, acc)
    size_t pseudo;        // float  [L, rows * Hkv, pseudo_runs, G, D + 4] pseudo-token partials (value summaries only)
    int pseudo_runs;
    // split cut (rows * Hq <= kSplitMaxPairs and every level small enough); absent otherwise
    bool split;
    size_t rank;          // int32  [rows, Hq, nodes_total] a kept node's place in its head's kept list
    size_t cand_sc;       // float  [rows, Hq, cand_stride] a level's candidate scores in candidate order
    size_t cand_nd;       // int32  [rows, Hq, cand_stride] their node ids
    size_t srt_k;         // uint32 [rows, Hq, cand_stride] per slice, candidates grouped by bin
    size_t srt_s;         // float  [rows, Hq, cand_stride] and their scores
    int64_t cand_stride;
    size_t pmax;          // float  [rows, Hq, pmax_stride] per scoring workgroup maxima of a level
    int64_t pmax_stride;
    size_t pruns;         // int32  [rows, Hq] scoring workgroups of the head's (row, kv head) pair
    size_t chist;         // uint64 [rows, Hq, kCutBins] a level's mass per bin
    size_t cum;           // uint32 [rows, Hq, slice_stride, kCutBins + 1] per slice, candidates before each bin
    int64_t slice_stride;
    size_t total;
};

// Parameters shared by every kernel that reads queries.
struct RowInfo {
    const int32_t* seq_lens;  // [B]
    const int32_t* q_pos;     // [B, T] or null
    int T;                    // rows per sequence
};

__host__ __device__ inline int row_visible(const RowInfo& ri, int row) {
    const int s = row / ri.T, t = row % ri.T;
    const int pos = ri.q_pos ? ri.q_pos[row] : (ri.seq_lens[s] - ri.T + t);
    return pos + 1;
}

// Tokens a row sees, clamped to its sequence's length and the capacity. Its
// two loads (length, and position or again the length) go out together.
__device__ __forceinline__ int clamp_visible(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T, t = row % ri.T;
    const int len = ri.seq_lens[s];
    const int pv = *(ri.q_pos ? ri.q_pos + row : ri.seq_lens + s);
    const int n = (ri.q_pos ? pv : len - ri.T + t) + 1;
    const int lim = static_cast<int>(len < cap ? len : cap);
    return n < 0 ? 0 : (n > lim ? lim : n);
}

// Opt-in kernel timing (zha_profile_start): brackets a launch with two events
// when `label` (optionally "label@level") matches the active target.
class ProfScope {
   public:
    ProfScope(const char* label, int level, hipStream_t st);
    ~ProfScope();
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;

   private:
    int slot_ = -1;
    hipStream_t st_;
};

// Launchers (defined in the kernel translation units). All return hipError_t.
hipError_t launch_build_level(const Geo& g, int level, const void* K, const void* V, const float* ref_q,
                              float* summaries, const int32_t* seq_lens, int mode, int t_new, hipStream_t st);
hipError_t launch_append_rows(const Geo& g, void* K, void* V, const void* k_new, const void* v_new, int t_new,
                              const int32_t* seq_lens, uint32_t* status, hipStream_t st);
hipError_t launch_append_fused(const Geo& g, void* K, void* V, const void* k_new, const void* v_new, int t_new,
                               int32_t* seq_lens, const float* ref_q, float* summaries, uint32_t* status,
                               hipStream_t st);
hipError_t launch_advance_seq(const Geo& g, int32_t* seq_lens, int t_new, hipStream_t st);

struct RouteArgs {
    const float* q;
    RowInfo ri;
    int rows;
    const float* summaries;
    float top_p;
    float top_p_l[ZHA_MAX_LEVELS];   // the cut fraction of each level (top_p or the geometry's schedule)
    int sel_cap;
    int32_t* sel_blocks;
    int32_t* n_sel;
    int32_t* level_stats;
    int32_t* level_sel;
    char* ws;
    const WsLayout* lay;
};
hipError_t launch_route(const Geo& g, const RouteArgs& a, hipStream_t st);

// Rows per sequence from which every level is scored densely on the matrix
// cores (route_dense.hip) instead of by gathering the kept parents' children.
constexpr int kDenseMinRows = 64;
bool dense_scores_fit(const Geo& g, int T);
hipError_t launch_dense_scores(const Geo& g, const RowInfo& ri, const float* q, const float* summaries,
                               float* scores, int li_lo, int li_hi, hipStream_t st);

struct AttendArgs {
    const float* q;
    RowInfo ri;
    int rows;
    const void* K;
    const void* V;
    const int32_t* sel_blocks;
    const int32_t* n_sel;
    int sel_cap;
    float* out;
    float* lse;
    char* ws;
    const WsLayout* lay;
    bool dense;
    bool bitmaps_ready;       // the route already wrote the level-1 kept bitmaps
};
hipError_t launch_attend(const Geo& g, const AttendArgs& a, hipStream_t st);

// Pseudo-tokens of the pruned candidates of every level, merged into out / lse
// (value summaries). Needs the route's kept bitmaps and every level's scores.
hipError_t launch_pseudo(const Geo& g, const AttendArgs& a, const float* summaries, hipStream_t st);

}  // namespace zha

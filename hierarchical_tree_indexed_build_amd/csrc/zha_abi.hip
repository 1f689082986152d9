// zha_abi.hip - the extern "C" entry points of libzha: argument validation,
// size and offset arithmetic, workspace layout, and kernel sequencing on the
// caller's stream. Every host-detectable error is returned before any launch.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "zha_internal.h"

namespace zha {
namespace {

thread_local std::string g_last_error;

zha_status fail(zha_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
zha_status fail(zha_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

zha_status hip_fail(hipError_t e, const char* what) {
    return fail(ZHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

zha_status make_geo(const zha_geom* in, Geo* g) {
    if (!in) return fail(ZHA_ERR_NULL, "geom is NULL");
    if (in->batch < 1 || in->n_kv_heads < 1 || in->n_q_heads < 1)
        return fail(ZHA_ERR_SHAPE, "batch, n_q_heads and n_kv_heads must be >= 1");
    if (in->n_q_heads % in->n_kv_heads)
        return fail(ZHA_ERR_SHAPE, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", in->n_q_heads,
                    in->n_kv_heads);
    const int G = in->n_q_heads / in->n_kv_heads;
    if (!is_pow2_in(G, 1, kMaxGroup))
        return fail(ZHA_ERR_UNSUPPORTED, "query heads per kv head must be 1, 2, 4, 8 or 16 (got %d)", G);
    if (in->head_dim != 64 && in->head_dim != 128)
        return fail(ZHA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", in->head_dim);
    if (!is_pow2_in(in->branching, 2, 256))
        return fail(ZHA_ERR_UNSUPPORTED, "branching must be a power of two in [2, 256] (got %d)", in->branching);
    if (in->n_levels < 1 || in->n_levels > ZHA_MAX_LEVELS)
        return fail(ZHA_ERR_SHAPE, "n_levels must be in [1, %d] (got %d)", ZHA_MAX_LEVELS, in->n_levels);
    if (in->capacity < 1 || in->capacity >= (int64_t(1) << 31))
        return fail(ZHA_ERR_SHAPE, "capacity must be in [1, 2^31) (got %lld)", static_cast<long long>(in->capacity));
    if (in->kv_dtype != ZHA_KV_BF16 && in->kv_dtype != ZHA_KV_F32)
        return fail(ZHA_ERR_UNSUPPORTED, "kv_dtype must be ZHA_KV_BF16 or ZHA_KV_F32");
    if (!(in->scale >= 0.f) || std::isinf(in->scale)) return fail(ZHA_ERR_SHAPE, "scale must be finite and >= 0");
    if (in->scoring != ZHA_SCORE_SUMMARY && in->scoring != ZHA_SCORE_TANGENT)
        return fail(ZHA_ERR_UNSUPPORTED, "scoring must be ZHA_SCORE_SUMMARY or ZHA_SCORE_TANGENT (got %d)", in->scoring);
    if (in->value_summaries != 0 && in->value_summaries != 1)
        return fail(ZHA_ERR_SHAPE, "value_summaries must be 0 or 1 (got %d)", in->value_summaries);
    if (in->value_summaries && in->scoring != ZHA_SCORE_SUMMARY)
        return fail(ZHA_ERR_UNSUPPORTED, "value summaries need summary scoring");
    const int R = in->n_refs > 0 ? in->n_refs : 1;
    if (in->n_refs < 0 || R > ZHA_MAX_REFS || (in->scoring == ZHA_SCORE_SUMMARY && R != 1))
        return fail(ZHA_ERR_UNSUPPORTED, "n_refs must be 0 or 1 for summary scoring and 1..%d for tangent scoring (got %d)",
                    ZHA_MAX_REFS, in->n_refs);
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
        const float v = in->level_p[l];
        if (l < in->n_levels ? !(v == 0.f || (v > 0.f && v <= 1.f)) : v != 0.f)
            return fail(ZHA_ERR_SHAPE, "level_p[%d] must be 0 or in (0, 1] for a level of the tree, 0 past it (got %g)",
                        l, static_cast<double>(v));
        g->level_p[l] = v;
    }
    g->B = in->batch;
    g->Hq = in->n_q_heads;
    g->Hkv = in->n_kv_heads;
    g->G = G;
    g->D = in->head_dim;
    g->b = in->branching;
    g->lb = 0;
    while ((1 << g->lb) < g->b) ++g->lb;
    g->L = in->n_levels;
    g->R = R;
    g->tangent = in->scoring == ZHA_SCORE_TANGENT;
    g->vsum = in->value_summaries != 0;
    g->kv_dtype = in->kv_dtype;
    g->cap = in->capacity;
    g->scale = in->scale > 0.f ? in->scale : 1.0f / std::sqrt(static_cast<float>(in->head_dim));
    int64_t span = 1;
    int64_t soff = 0, loff = 0;
    for (int l = 0; l < ZHA_MAX_LEVELS + 1; ++l) {
        // spans beyond 2^62 are clamped: no node of such a level can be complete
        span = (span > (int64_t(1) << 56)) ? span : span * g->b;
        g->span[l] = span;
        if (l < ZHA_MAX_LEVELS) {
            g->nodes[l] = (l < g->L) ? g->cap / span : 0;
            g->sum_off[l] = soff;
            g->sel_off[l] = loff;
            soff += static_cast<int64_t>(g->B) * g->Hkv * g->nodes[l] * g->R * g->D;
            loff += g->nodes[l];
        }
    }
    g->nodes_total = loff;
    // tangent offsets follow every level's keys
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
        g->bias_off[l] = soff;
        if (g->tangent) soff += static_cast<int64_t>(g->B) * g->Hkv * g->nodes[l] * g->R;
    }
    // then the value summaries
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
        g->val_off[l] = soff;
        if (g->vsum) soff += static_cast<int64_t>(g->B) * g->Hkv * g->nodes[l] * g->D;
    }
    g->summ_total = soff;
    return ZHA_OK;
}


WsLayout layout(const Geo& g, int rows) {
    WsLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    const size_t R = static_cast<size_t>(rows);
    L.status = take(256);
    L.qpos = take(R * 4);
    L.scores = take(R * g.Hq * g.nodes_total * 4);
    L.kept = take(R * g.Hq * g.nodes_total * 4);
    L.kept_cnt = take(R * g.Hq * g.L * 4);
    int64_t bw = 0;
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
        L.bm_off[l] = static_cast<size_t>(bw);
        bw += (l < g.L) ? (g.nodes[l] + 32) / 32 : 0;     // one spare bit for index nodes[l]
    }
    L.bm_words_total = bw;
    L.bitmap = take(R * g.Hq * static_cast<size_t>(bw) * 4);
    L.aitems = take(R * g.Hkv * static_cast<size_t>(g.nodes[0] + 2) * 8);
    L.acnt = take(R * g.Hkv * 4);
    {
        const int64_t nseg = items_segments(g, static_cast<int64_t>(R) * g.Hkv);
        L.segcnt = take(nseg > kItemsRecountSegs ? R * g.Hkv * static_cast<size_t>(nseg) * 4 : 0);
    }
    L.plan = take(2 * (R * g.Hkv + 1) * 8);
    L.partial = take((static_cast<size_t>(kAttnWorkgroups) + R * g.Hkv) * g.G * (g.D + 4) * 4);
    if (g.vsum) {
        const int64_t pairs = static_cast<int64_t>(R) * g.Hkv;
        L.pseudo_runs = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kPseudoMaxRuns, 2048 / pairs)));
        L.pseudo = take(static_cast<size_t>(g.L) * pairs * L.pseudo_runs * g.G * (g.D + 4) * 4);
    }
    // the split cut: candidates of a level are at most its node slots
    const int64_t cand = g.nodes[0];
    const int64_t slices = (cand + kSplitSlice - 1) / kSplitSlice;
    L.split = R * g.Hq <= static_cast<size_t>(kSplitMaxPairs) && slices <= kSplitMaxSlices;
    if (L.split) {
        int64_t pm = 1;
        for (int l = 0; l < g.L; ++l) {
            const int64_t slots = (l == g.L - 1) ? (g.nodes[l] + g.b - 1) / g.b : g.nodes[l + 1] + 1;
            pm = std::max<int64_t>(pm, score_shape(slots, static_cast<int64_t>(R) * g.Hkv).max_runs);
        }
        L.cand_stride = cand;
        L.pmax_stride = pm;
        L.slice_stride = slices;
        L.rank = take(R * g.Hq * static_cast<size_t>(g.nodes_total) * 4);
        L.cand_sc = take(R * g.Hq * static_cast<size_t>(cand) * 4);
        L.cand_nd = take(R * g.Hq * static_cast<size_t>(cand) * 4);
        L.srt_k = take(R * g.Hq * static_cast<size_t>(cand) * 4);
        L.srt_s = take(R * g.Hq * static_cast<size_t>(cand) * 4);
        L.pmax = take(R * g.Hq * static_cast<size_t>(pm) * 4);
        L.pruns = take(R * g.Hq * 4);
        L.chist = take(R * g.Hq * static_cast<size_t>(kCutBins) * 8);
        L.cum = take(R * g.Hq * static_cast<size_t>(slices) * (kCutBins + 1) * 4);
    }
    L.total = off;
    return L;
}

zha_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return fail(ZHA_ERR_NULL, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(ZHA_ERR_SHAPE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(ZHA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return ZHA_OK;
}

zha_status check_rows(const Geo& g, int32_t t, int* rows) {
    if (t < 1) return fail(ZHA_ERR_SHAPE, "t (query rows per sequence) must be >= 1 (got %d)", t);
    const int64_t r = static_cast<int64_t>(g.B) * t;
    if (r > (int64_t(1) << 24)) return fail(ZHA_ERR_SHAPE, "too many query rows (%lld)", static_cast<long long>(r));
    *rows = static_cast<int>(r);
    return ZHA_OK;
}

// ---- row tiles ----
// A call of t rows of one sequence whose workspace holds only part of the
// layout runs in tiles of rows (the largest halving of t whose layout fits),
// each a complete route and attention of its rows; a tiled workspace for
// max_t rows (zha_query_sizes) keeps under kTileBytes.
constexpr size_t kTileBytes = size_t(4) << 30;

int tile_rows_fitting(const Geo& g, int t, size_t bytes) {
    int r = t;
    while (r > 1 && layout(g, r).total > bytes) r = (r + 1) / 2;
    return layout(g, r).total <= bytes ? r : 0;
}

// Default positions of a tile's rows (seq_lens[0] - t + t0 + i), written into the workspace.
__global__ void tile_positions_kernel(int32_t* pos, const int32_t* seq_lens, int t, int t0, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) pos[i] = seq_lens[0] - t + t0 + i;
}

// Runs body(t0, rows, q_pos, layout) once with every row, or over row tiles
// when the workspace is smaller than the full layout and tiling is allowed
// (one sequence; the caller asked for no per-call buffer laid out by row count).
template <class Body>
zha_status run_rows(const Geo& g, int32_t t, const int32_t* q_pos, const int32_t* seq_lens, void* ws,
                    size_t ws_bytes, bool can_tile, hipStream_t s, Body&& body) {
    int rows;
    zha_status st = check_rows(g, t, &rows);
    if (st) return st;
    const WsLayout full = layout(g, rows);
    if (ws_bytes >= full.total || !can_tile || g.B != 1 || !ws) {
        if ((st = check_ws(ws, ws_bytes, full.total))) return st;
        return body(0, t, q_pos, full);
    }
    const int tile = tile_rows_fitting(g, t, ws_bytes);
    if (tile == 0) return check_ws(ws, ws_bytes, layout(g, 1).total);
    for (int t0 = 0; t0 < t; t0 += tile) {
        const int tt = std::min(tile, t - t0);
        const WsLayout Lt = layout(g, tt);
        if ((st = check_ws(ws, ws_bytes, Lt.total))) return st;
        const int32_t* qp = q_pos ? q_pos + t0 : nullptr;
        if (!qp) {
            int32_t* pos = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + Lt.qpos);
            hipLaunchKernelGGL(tile_positions_kernel, dim3((tt + 255) / 256), dim3(256), 0, s, pos, seq_lens, t, t0, tt);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return hip_fail(e, "tile positions launch");
            qp = pos;
        }
        if ((st = body(t0, tt, qp, Lt))) return st;
    }
    return ZHA_OK;
}

// ---- opt-in kernel timing ----
struct Profiler {
    std::string target;          // empty: inactive
    std::vector<hipEvent_t> ev;  // pairs (start, stop)
    int used = 0;
    int64_t dropped = 0;
};
Profiler g_prof;
constexpr int kProfSlots = 8192;

// ---- the static scratch of zha_attend_noalloc ----
// Device memory the library owns, for callers that cannot allocate. Each GPU
// the library runs on holds its own copy until the process ends. In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    void* ptr = nullptr;       // device address of this device's scratch
    bool cleared = false;      // the whole array was zeroed once (its first call)
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Clears `words` 32-bit words (a fill kernel rather than a memset, so that the
// call stays valid under stream capture).
__global__ void zero_words_kernel(uint32_t* p, size_t words) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

__global__ void copy_word_kernel(const uint32_t* src, uint32_t* dst) { *dst = *src; }

bool prof_matches(const char* label, int level) {
    if (g_prof.target.empty()) return false;
    const std::string& t = g_prof.target;
    const size_t at = t.find('@');
    if (at == std::string::npos) return t == label;
    return t.compare(0, at, label) == 0 && std::strlen(label) == at && std::atoi(t.c_str() + at + 1) == level;
}

}  // namespace

ProfScope::ProfScope(const char* label, int level, hipStream_t st) : st_(st) {
    if (!prof_matches(label, level)) return;
    if (g_prof.used >= kProfSlots) {
        ++g_prof.dropped;
        return;
    }
    slot_ = g_prof.used++;
    (void)hipEventRecord(g_prof.ev[2 * slot_], st_);
}

ProfScope::~ProfScope() {
    if (slot_ >= 0) (void)hipEventRecord(g_prof.ev[2 * slot_ + 1], st_);
}

}  // namespace zha

using namespace zha;

extern "C" {

zha_status zha_query_sizes(const zha_geom* geom, int32_t max_t, zha_sizes* out) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if (!out) return fail(ZHA_ERR_NULL, "out is NULL");
    int rows;
    if ((st = check_rows(g, max_t, &rows))) return st;
    const WsLayout L = layout(g, rows);
    *out = zha_sizes{};
    out->summaries_bytes = static_cast<size_t>(g.summ_total) * 4;
    out->workspace_bytes = L.total;
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
        out->level_nodes[l] = g.nodes[l];
        out->level_offset[l] = g.sum_off[l];
        out->level_bias_offset[l] = g.bias_off[l];
        out->level_value_offset[l] = g.val_off[l];
        out->level_sel_offset[l] = g.sel_off[l];
    }
    out->level_sel_bytes = static_cast<size_t>(rows) * g.Hq * g.nodes_total * 4;
    out->max_rows = rows;
    out->tile_rows = max_t;
    out->workspace_bytes_tiled = L.total;
    if (g.B == 1 && L.total > kTileBytes) {
        const int tile = std::max(tile_rows_fitting(g, max_t, kTileBytes), 1);
        out->tile_rows = tile;
        out->workspace_bytes_tiled = layout(g, tile).total;
    }
    return ZHA_OK;
}

zha_status zha_build_tree(const zha_geom* geom, const void* K, const void* V, const float* ref_q,
                          const int32_t* seq_lens, float* summaries, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if (!K || !ref_q || !seq_lens || !summaries) return fail(ZHA_ERR_NULL, "K, ref_q, seq_lens and summaries are required");
    if (g.vsum && !V) return fail(ZHA_ERR_NULL, "V is required with value summaries");
    if ((st = check_ws(ws, ws_bytes, 256))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int level = 1; level <= g.L; ++level) {
        const hipError_t e = launch_build_level(g, level, K, V, ref_q, summaries, seq_lens, 0, 0, s);
        if (e != hipSuccess) return hip_fail(e, "build level launch");
    }
    return ZHA_OK;
}

zha_status zha_append(const zha_geom* geom, void* K, void* V, const void* k_new, const void* v_new, int32_t t_new,
                      int32_t* seq_lens, const float* ref_q, float* summaries, void* ws, size_t ws_bytes,
                      void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if (!K || !V || !k_new || !v_new || !seq_lens || !ref_q || !summaries)
        return fail(ZHA_ERR_NULL, "K, V, k_new, v_new, seq_lens, ref_q and summaries are required");
    if (t_new < 1 || t_new > g.cap) return fail(ZHA_ERR_SHAPE, "t_new must be in [1, capacity] (got %d)", t_new);
    if ((st = check_ws(ws, ws_bytes, 256))) return st;
    uint32_t* status = static_cast<uint32_t*>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (t_new <= 64) {
        e = launch_append_fused(g, K, V, k_new, v_new, t_new, seq_lens, ref_q, summaries, status, s);
        if (e != hipSuccess) return hip_fail(e, "append launch");
        return ZHA_OK;
    }
    e = launch_append_rows(g, K, V, k_new, v_new, t_new, seq_lens, status, s);
    if (e != hipSuccess) return hip_fail(e, "append rows launch");
    for (int level = 1; level <= g.L; ++level) {
        e = launch_build_level(g, level, K, V, ref_q, summaries, seq_lens, 1, t_new, s);
        if (e != hipSuccess) return hip_fail(e, "append level launch");
    }
    e = launch_advance_seq(g, seq_lens, t_new, s);
    if (e != hipSuccess) return hip_fail(e, "append advance launch");
    return ZHA_OK;
}

static zha_status route_impl(const Geo& g, const float* q, int32_t t, const int32_t* q_pos, const float* summaries,
                             const int32_t* seq_lens, float top_p, int32_t sel_capacity, int32_t* sel_blocks,
                             int32_t* n_sel, int32_t* level_stats, int32_t* level_sel, void* ws, const WsLayout& L,
                             int rows, hipStream_t s) {
    RouteArgs a{};
    a.q = q;
    a.ri = RowInfo{seq_lens, q_pos, t};
    a.rows = rows;
    a.summaries = summaries;
    a.top_p = top_p;
    for (int l = 0; l < ZHA_MAX_LEVELS; ++l) a.top_p_l[l] = g.level_p[l] > 0.f ? g.level_p[l] : top_p;
    a.sel_cap = sel_capacity;
    a.sel_blocks = sel_blocks;
    a.n_sel = n_sel;
    a.level_stats = level_stats;
    a.level_sel = level_sel;
    a.ws = static_cast<char*>(ws);
    a.lay = &L;
    const hipError_t e = launch_route(g, a, s);
    if (e != hipSuccess) return hip_fail(e, "route launch");
    return ZHA_OK;
}

static zha_status check_route_args(const float* q, const float* summaries, const int32_t* seq_lens, float top_p,
                                   int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel) {
    if (!q || !summaries || !seq_lens || !sel_blocks || !n_sel)
        return fail(ZHA_ERR_NULL, "q, summaries, seq_lens, sel_blocks and n_sel are required");
    if (!(top_p > 0.f && top_p <= 1.f)) return fail(ZHA_ERR_SHAPE, "top_p must be in (0, 1]");
    if (sel_capacity < 1) return fail(ZHA_ERR_SHAPE, "sel_capacity must be >= 1");
    return ZHA_OK;
}

zha_status zha_route(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos, const float* summaries,
                     const int32_t* seq_lens, float top_p, int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel,
                     int32_t* level_stats, int32_t* level_sel, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if ((st = check_route_args(q, summaries, seq_lens, top_p, sel_capacity, sel_blocks, n_sel))) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_rows(g, t, q_pos, seq_lens, ws, ws_bytes, level_sel == nullptr, s,
                    [&](int t0, int tt, const int32_t* qp, const WsLayout& L) {
                        const int64_t r0 = static_cast<int64_t>(t0) * g.Hq;
                        return route_impl(g, q + r0 * g.D, tt, qp, summaries, seq_lens, top_p, sel_capacity,
                                          sel_blocks + r0 * sel_capacity, n_sel + r0,
                                          level_stats ? level_stats + r0 * g.L * 2 : nullptr, level_sel, ws, L,
                                          g.B * tt, s);
                    });
}

static zha_status attend_impl(const Geo& g, const float* q, int32_t t, const int32_t* q_pos, const void* K,
                              const void* V, const int32_t* seq_lens, const int32_t* sel_blocks, const int32_t* n_sel,
                              int32_t sel_capacity, float* out, float* lse, void* ws, const WsLayout& L, int rows,
                              bool dense, bool bitmaps_ready, hipStream_t s, const float* summaries = nullptr) {
    AttendArgs a{};
    a.q = q;
    a.ri = RowInfo{seq_lens, q_pos, t};
    a.rows = rows;
    a.K = K;
    a.V = V;
    a.sel_blocks = sel_blocks;
    a.n_sel = n_sel;
    a.sel_cap = sel_capacity;
    a.out = out;
    a.lse = lse;
    a.ws = static_cast<char*>(ws);
    a.lay = &L;
    a.dense = dense;
    a.bitmaps_ready = bitmaps_ready;
    hipError_t e = launch_attend(g, a, s);
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    // after a route in the same call: the pruned candidates as pseudo-tokens
    if (g.vsum && summaries && bitmaps_ready) {
        e = launch_pseudo(g, a, summaries, s);
        if (e != hipSuccess) return hip_fail(e, "pseudo-token launch");
    }
    return ZHA_OK;
}

zha_status zha_sparse_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos, const void* K,
                             const void* V, const int32_t* seq_lens, const int32_t* sel_blocks, const int32_t* n_sel,
                             int32_t sel_capacity, float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if (!q || !K || !V || !seq_lens || !sel_blocks || !n_sel || !out || !lse)
        return fail(ZHA_ERR_NULL, "q, K, V, seq_lens, sel_blocks, n_sel, out and lse are required");
    if (sel_capacity < 1) return fail(ZHA_ERR_SHAPE, "sel_capacity must be >= 1");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_rows(g, t, q_pos, seq_lens, ws, ws_bytes, true, s,
                    [&](int t0, int tt, const int32_t* qp, const WsLayout& L) {
                        const int64_t r0 = static_cast<int64_t>(t0) * g.Hq;
                        return attend_impl(g, q + r0 * g.D, tt, qp, K, V, seq_lens, sel_blocks + r0 * sel_capacity,
                                           n_sel + r0, sel_capacity, out + r0 * g.D, lse + r0, ws, L, g.B * tt,
                                           false, false, s);
                    });
}

zha_status zha_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos, const void* K,
                      const void* V, const float* summaries, const int32_t* seq_lens, float top_p,
                      int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel, int32_t* level_stats,
                      int32_t* level_sel, float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if ((st = check_route_args(q, summaries, seq_lens, top_p, sel_capacity, sel_blocks, n_sel))) return st;
    if (!K || !V || !out || !lse) return fail(ZHA_ERR_NULL, "K, V, out and lse are required");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_rows(g, t, q_pos, seq_lens, ws, ws_bytes, level_sel == nullptr, s,
                    [&](int t0, int tt, const int32_t* qp, const WsLayout& L) {
                        const int64_t r0 = static_cast<int64_t>(t0) * g.Hq;
                        int32_t* sb = sel_blocks + r0 * sel_capacity;
                        int32_t* ns = n_sel + r0;
                        zha_status e = route_impl(g, q + r0 * g.D, tt, qp, summaries, seq_lens, top_p, sel_capacity,
                                                  sb, ns, level_stats ? level_stats + r0 * g.L * 2 : nullptr,
                                                  level_sel, ws, L, g.B * tt, s);
                        if (e) return e;
                        return attend_impl(g, q + r0 * g.D, tt, qp, K, V, seq_lens, sb, ns, sel_capacity,
                                           out + r0 * g.D, lse + r0, ws, L, g.B * tt, false, true, s, summaries);
                    });
}

zha_status zha_attend_noalloc(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos, const void* K,
                              const void* V, const float* summaries, const int32_t* seq_lens, float top_p,
                              int32_t sel_capacity, int32_t* sel_blocks, int32_t* n_sel, int32_t* level_stats,
                              int32_t* level_sel, float* out, float* lse, uint32_t* dev_status, void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if ((st = check_route_args(q, summaries, seq_lens, top_p, sel_capacity, sel_blocks, n_sel))) return st;
    if (!K || !V || !out || !lse) return fail(ZHA_ERR_NULL, "K, V, out and lse are required");
    int rows;
    if ((st = check_rows(g, t, &rows))) return st;
    const WsLayout L = layout(g, rows);
    if (L.total > kScratchBytes)
        return fail(ZHA_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the static scratch holds %zu: use zha_attend with a "
                    "workspace",
                    L.total, kScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "current device");
    if (dev < 0 || dev >= kMaxDevices) return fail(ZHA_ERR_UNSUPPORTED, "device %d is past the %d the scratch table holds", dev, kMaxDevices);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    bool first = false;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ScratchSlot& slot = g_scratch[dev];
        if (!slot.ptr) {
            void* ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "scratch address");
            if (!ptr) return fail(ZHA_ERR_HIP, "scratch address is NULL");
            slot.ptr = ptr;
        }
        ws = slot.ptr;
        first = !slot.cleared;
        slot.cleared = true;
    }
    // the status word starts every call at zero; the whole array once, on its first call
    const size_t words = first ? kScratchBytes / 4 : 1;
    hipLaunchKernelGGL(zero_words_kernel, dim3(first ? 1024 : 1), dim3(256), 0, s, static_cast<uint32_t*>(ws), words);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "scratch clear launch");
    if ((st = route_impl(g, q, t, q_pos, summaries, seq_lens, top_p, sel_capacity, sel_blocks, n_sel, level_stats,
                         level_sel, ws, L, rows, s)))
        return st;
    if ((st = attend_impl(g, q, t, q_pos, K, V, seq_lens, sel_blocks, n_sel, sel_capacity, out, lse, ws, L, rows,
                          false, true, s, summaries)))
        return st;
    if (dev_status) {
        hipLaunchKernelGGL(copy_word_kernel, dim3(1), dim3(1), 0, s, static_cast<const uint32_t*>(ws), dev_status);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "status copy launch");
    }
    return ZHA_OK;
}

zha_status zha_dense_attend(const zha_geom* geom, const float* q, int32_t t, const int32_t* q_pos, const void* K,
                            const void* V, const int32_t* seq_lens, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
    Geo g;
    zha_status st = make_geo(geom, &g);
    if (st) return st;
    if (!q || !K || !V || !seq_lens || !out || !lse)
        return fail(ZHA_ERR_NULL, "q, K, V, seq_lens, out and lse are required");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return run_rows(g, t, q_pos, seq_lens, ws, ws_bytes, true, s,
                    [&](int t0, int tt, const int32_t* qp, const WsLayout& L) {
                        const int64_t r0 = static_cast<int64_t>(t0) * g.Hq;
                        return attend_impl(g, q + r0 * g.D, tt, qp, K, V, seq_lens, nullptr, nullptr, 1,
                                           out + r0 * g.D, lse + r0, ws, L, g.B * tt, true, false, s);
                    });
}

zha_status zha_read_device_status(void* ws, void* stream, uint32_t* out, int32_t clear) {
    if (!ws || !out) return fail(ZHA_ERR_NULL, "ws and out are required");
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    e = hipMemcpy(out, ws, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "status read");
    if (clear) {
        const uint32_t zero = 0;
        e = hipMemcpy(ws, &zero, sizeof(uint32_t), hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, "status clear");
    }
    return ZHA_OK;
}

const char* zha_status_string(zha_status s) {
    switch (s) {
        case ZHA_OK: return "ok";
        case ZHA_ERR_NULL: return "null pointer";
        case ZHA_ERR_SHAPE: return "inconsistent shape";
        case ZHA_ERR_UNSUPPORTED: return "unsupported size";
        case ZHA_ERR_WORKSPACE: return "workspace too small";
        case ZHA_ERR_CAPACITY: return "capacity exceeded";
        case ZHA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* zha_last_error(void) { return g_last_error.c_str(); }

zha_status zha_profile_start(const char* label) {
    if (!label || !*label) {
        g_prof.target.clear();
        return ZHA_OK;
    }
    if (g_prof.ev.empty()) {
        g_prof.ev.resize(2 * kProfSlots);
        for (auto& e : g_prof.ev) {
            const hipError_t r = hipEventCreate(&e);
            if (r != hipSuccess) {
                g_prof.ev.clear();
                return hip_fail(r, "profile event pool");
            }
        }
    }
    g_prof.target = label;
    g_prof.used = 0;
    g_prof.dropped = 0;
    return ZHA_OK;
}

zha_status zha_profile_collect(double* total_ms, int64_t* launches, int64_t* dropped) {
    if (!total_ms || !launches || !dropped) return fail(ZHA_ERR_NULL, "outputs are required");
    double tot = 0.0;
    for (int i = 0; i < g_prof.used; ++i) {
        hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "profile event wait");
        float ms = 0.f;
        r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "profile event time");
        tot += ms;
    }
    *total_ms = tot;
    *launches = g_prof.used;
    *dropped = g_prof.dropped;
    g_prof.used = 0;
    g_prof.dropped = 0;
    return ZHA_OK;
}

}  // extern "C"

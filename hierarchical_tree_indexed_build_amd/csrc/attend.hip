// attend.hip - exact attention over the selected tokens, and the dense baseline.
//
// A query row that sees N tokens attends I = {0} U (kept leaf chunks) U
// [b*floor((N-1)/b), N) ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", §Routing, I(q) and o(q); token 0 is the sink of
// "Zyphra Hierarchical Attention: The End of Quadratic Attention?", §How the
// tree is built and searched). The dense baseline attends [0, N).
//
// The kept leaf chunks arrive as one bitmap per query head: the level-1 cut
// writes them in zha_attend, attn_bitmap_kernel builds them from id lists for a
// standalone sparse call. Kernels:
//  * attn_items_kernel  - per (row, kv head): OR the g query heads' bitmaps,
//    add chunk 0 (sink) and the current chunk, and compact them into one
//    ascending list of (chunk, head mask) items; K/V of a chunk are then read
//    once for the whole GQA group.
//  * attend_kernel      - split-K flash decoding. Workgroup = one share of a
//    (row, kv head) pair's groups; each wave streams 16-token groups of it through a two-stage
//    register pipeline with an online softmax for all g heads; lanes own a
//    slice of d; waves merge in LDS and write one (max, sum, acc[d]) partial
//    per head and split.
//  * attend_combine_kernel - per (row, head): LSE merge of the splits.
// The attention's work plan is the prefix of the groups and of the workgroup
// shares over the (row, kv head) pairs: attn_plan_kernel writes it for more
// than 64 pairs; with fewer, the attention and combine kernels take it from
// the pairs' counts themselves.
#include <algorithm>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

constexpr uint32_t kAllHeads = 1u << 30;     // item flag: every head attends the chunk (current chunk)

// An item read through the scalar data cache: the list is not written while
// the attention runs, so it can be read as constant memory.
typedef __attribute__((address_space(4))) const int const_i32;
__device__ __forceinline__ int2 scalar_item(const int2* items, int64_t i) {
    const const_i32* c = (const const_i32*)(items);
    return make_int2(c[2 * i], c[2 * i + 1]);
}

__device__ __forceinline__ int visible_clamped(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T;
    int n = row_visible(ri, row);
    const int lim = static_cast<int>(imin(ri.seq_lens[s], cap));
    n = n < 0 ? 0 : n;
    return n > lim ? lim : n;
}

// ----------------------------------------------------------------------------
// kept leaf chunks -> per-head bitmaps (standalone sparse calls only; the cut
// of zha_attend writes these bitmaps itself)
// ----------------------------------------------------------------------------
struct BitmapParams {
    const int32_t* sel_blocks;
    const int32_t* n_sel;
    int sel_cap;
    uint32_t* bm;              // level-1 bitmaps, (row*Hq + hq)*stride
    int64_t stride;            // words per row-head
    int64_t words;             // words of the level-1 bitmap
};

__global__ __launch_bounds__(256) void attn_bitmap_kernel(BitmapParams p) {
    const int64_t rh = blockIdx.x;
    uint32_t* bm = p.bm + rh * p.stride;
    for (int64_t w = threadIdx.x; w < p.words; w += blockDim.x) bm[w] = 0u;
    __threadfence_block();
    __syncthreads();
    const int n = max(0, min(p.n_sel[rh], p.sel_cap));
    const int32_t* lst = p.sel_blocks + rh * p.sel_cap;
    for (int j = threadIdx.x; j < n; j += blockDim.x) {
        const int64_t node = lst[j];
        if (node >= 0 && (node >> 5) < p.words)
            __hip_atomic_fetch_or(bm + (node >> 5), 1u << (node & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
}

// ----------------------------------------------------------------------------
// the group's attention items
// Workgroup = (segment of seg_words bitmap words, (row, kv head)). The
// union of the g heads' level-1 bitmaps, plus the sink chunk and the current
// chunk, is compacted in ascending chunk order into (chunk, head mask) items.
// A segment's first item position is the popcount of the union before it,
// which each workgroup takes itself from the (few) earlier words, all its
// threads counting, so the segments of a pair run in parallel. A thread owns
// one word of the segment. With few pairs a segment is 64 words, owned by
// the first wave: one wave's worth of scattered item stores, so a dense
// stretch of kept chunks spreads over many compute units. With many pairs
// (the rows of a prefill chunk) the chip is full anyway and a segment is
// 256 words, one per thread, so that fewer workgroups re-count the words
// before theirs.
// ----------------------------------------------------------------------------
struct ItemsParams {
    RowInfo ri;
    const uint32_t* bm;        // level-1 bitmaps, (row*Hq + hq)*stride
    int64_t stride;
    int2* items;               // [rows, Hkv, item_stride]
    int64_t item_stride;
    int32_t* acnt;             // [rows, Hkv]
    int32_t* segcnt;           // [rows, Hkv, seg_stride] items per segment, or null: each segment re-counts
    int64_t seg_stride;
    int64_t cap;
    int lb, Hq, Hkv;
    int seg_words;             // words per segment: kItemsSegFew or kItemsThreads
};

// One pair's view of the level-1 bitmaps: complete chunks are valid below nc1,
// the sink and the current chunk are always in.
template <int G>
struct ItemsView {
    const uint32_t* bm0;
    int64_t stride, nc1, nblk, cur;

    __device__ __forceinline__ ItemsView(const ItemsParams& p, int row, int kv) {
        const int N = visible_clamped(p.ri, row, p.cap);
        nc1 = static_cast<int64_t>(N) >> p.lb;                                    // complete leaf chunks
        nblk = N > 0 ? ((static_cast<int64_t>(N) - 1) >> p.lb) + 1 : 0;          // chunks incl. the current one
        cur = nblk - 1;
        stride = p.stride;
        bm0 = p.bm + (static_cast<int64_t>(row) * p.Hq + static_cast<int64_t>(kv) * G) * p.stride;
    }
    __device__ __forceinline__ int64_t words() const { return (nblk + 31) >> 5; }
    // word wd of the union: kept complete chunks of any head, the sink, the current chunk
    __device__ __forceinline__ uint32_t word(int64_t wd, uint32_t (&heads)[G]) const {
        const int64_t base = wd << 5;
        const uint32_t valid = base >= nc1 ? 0u : (nc1 - base >= 32 ? 0xffffffffu : ((1u << (nc1 - base)) - 1u));
        uint32_t u = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            heads[h] = bm0[static_cast<int64_t>(h) * stride + wd] & valid;
            u |= heads[h];
        }
        if (wd == 0 && nblk > 0) u |= 1u;
        if ((cur >> 5) == wd) u |= 1u << (cur & 31);
        return u;
    }
};

// Items per segment, for pairs whose bitmaps span many segments: the items
// kernel then adds the counts before its segment instead of re-reading every
// earlier word, which for a 16M-token row costs O(segments^2) word reads.
template <int G>
__global__ __launch_bounds__(kItemsThreads) void attn_segcount_kernel(ItemsParams p) {
    constexpr int NW = kItemsThreads / kWave;
    __shared__ uint32_t red[NW];
    const int seg = blockIdx.x, y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const ItemsView<G> v(p, row, kv);
    const int64_t words = v.words();
    const int64_t nseg = (words + p.seg_words - 1) / p.seg_words;
    if (seg >= nseg) return;
    const int64_t wd = static_cast<int64_t>(seg) * p.seg_words + tid;
    uint32_t heads[G];
    const uint64_t c = wave_scan_u64((tid < p.seg_words && wd < words) ? __popc(v.word(wd, heads)) : 0u);
    if (lane == 63) red[w] = static_cast<uint32_t>(c);
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) t += red[i];
        p.segcnt[static_cast<int64_t>(y) * p.seg_stride + seg] = static_cast<int32_t>(t);
    }
}

template <int G>
__global__ __launch_bounds__(kItemsThreads) void attn_items_kernel(ItemsParams p) {
    constexpr int NW = kItemsThreads / kWave;
    __shared__ uint64_t red[NW];
    __shared__ uint64_t red2[NW];
    const int seg = blockIdx.x, y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const ItemsView<G> v(p, row, kv);
    const int64_t words = v.words();
    const int64_t nseg = (words + p.seg_words - 1) / p.seg_words;
    const int64_t last = nseg > 0 ? nseg - 1 : 0;      // the last segment writes the count
    if (seg > last) return;
    const int64_t w0 = static_cast<int64_t>(seg) * p.seg_words;
    const int64_t wd = w0 + tid;
    uint32_t heads[G];
    const uint32_t mine = (tid < p.seg_words && wd < words) ? v.word(wd, heads) : 0u;
    // items before the segment
    uint64_t pre = 0;
    if (p.segcnt) {
        const int32_t* sc = p.segcnt + static_cast<int64_t>(y) * p.seg_stride;
        for (int64_t x = tid; x < seg; x += kItemsThreads) pre += static_cast<uint32_t>(sc[x]);
    } else {
#pragma unroll 4
        for (int64_t x = tid; x < w0; x += kItemsThreads) {
            uint32_t hx[G];
            pre += __popc(v.word(x, hx));
        }
    }
    const uint64_t cnt = __popc(mine);
    const uint64_t inc = wave_scan_u64(cnt);
    const uint64_t pinc = wave_scan_u64(pre);
    if (lane == 63) {
        red[w] = inc;
        red2[w] = pinc;
    }
    __syncthreads();
    uint64_t before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) before += red[i];
        total += red[i] + red2[i];
    }
    uint64_t seg_before = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) seg_before += red2[i];
    int2* items = p.items + static_cast<int64_t>(y) * p.item_stride;
    int64_t pos = static_cast<int64_t>(seg_before + before + inc - cnt);
    uint32_t u = mine;
    while (u) {
        const int bit = __ffs(static_cast<int>(u)) - 1;
        u &= u - 1;
        const int64_t chunk = (wd << 5) + bit;
        uint32_t mask = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) mask |= ((heads[h] >> bit) & 1u) << h;
        if (chunk == v.cur) mask |= kAllHeads;
        items[pos++] = make_int2(static_cast<int>(chunk), static_cast<int>(mask));
    }
    if (seg == last && tid == 0) p.acnt[y] = static_cast<int32_t>(total);
}

// ----------------------------------------------------------------------------
// split-K attention, balanced over the whole chip
// Work unit: a group of kGroupTokens tokens of one item (chunk) of one (row,
// kv head) pair. Each pair's groups are cut into shares of the same size
// (attn_chunk), one workgroup per share: a heavy pair is spread over many
// workgroups, and no workgroup spans two pairs, so each one loads a single
// q, starts a single pipeline and writes a single partial state, at slot
// = its workgroup index. attn_plan_kernel writes the prefixes of the groups
// and of the shares over the pairs (or the kernels build them, for at most
// 64 pairs). Scores are kept in log2 units (q is pre-scaled by
// scale * log2(e)), so every exponential is one native exp2.
// ----------------------------------------------------------------------------
constexpr int kGroupTokens = 16;          // tokens a wave handles per pipeline stage

constexpr int kMinChunk = 8;              // a workgroup gets at least 8 groups (128 tokens) of work
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
    const float* q;
    RowInfo ri;
    const void* K;
    const void* V;
    const int2* items;         // [pairs, item_stride] (sparse)
    const int32_t* acnt;       // [pairs] items per pair (sparse)
    int64_t item_stride;
    int64_t* plan;             // [2 (pairs + 1)] exclusive prefixes of groups, then of workgroup shares, per pair
    float* partial;            // [nwg + pairs, G, D + 4] by workgroup: max, sum, 2 pad, acc[D]
    int64_t cap;
    int b, lb, lgpi, Hq, Hkv, pairs, nwg, dense;
    int wave_plan;             // pairs <= 64: kernels take the plan from the counts themselves
    float qscale;              // scale * log2(e)
    float* out;                // [rows, Hq, D]: written here for a pair of one share, else by the combine
    float* lse;                // [rows, Hq] or null
};

// Each (row, kv head) pair's groups are cut into workgroup shares of `chunk`
// groups (a pair's last share may be shorter), so no workgroup spans two
// pairs: one q load, one online-softmax state and one partial per workgroup.
// With fewer pairs than workgroups, chunk is large enough that every pair's
// shares fit in nwg workgroups together: sum ceil(n / chunk) <= total / chunk
// + pairs <= nwg.
__device__ __forceinline__ int64_t attn_chunk(int64_t total, int nwg, int pairs) {
    const int64_t avail = static_cast<int64_t>(nwg) - pairs;
    const int64_t d = avail > 0 ? avail : nwg;
    const int64_t c = (total + d - 1) / d;
    return c < kMinChunk ? kMinChunk : c;
}

// groups of one pair: its items (sparse) or all its chunks (dense), times groups per chunk
__device__ __forceinline__ int64_t pair_groups(const AttnParams& p, int pr) {
    const int row = pr / p.Hkv;
    int64_t nitems;
    if (p.dense) {
        const int N = visible_clamped(p.ri, row, p.cap);
        nitems = N > 0 ? ((static_cast<int64_t>(N) - 1) >> p.lb) + 1 : 0;
    } else {
        nitems = p.acnt[pr];
    }
    return nitems << p.lgpi;
}

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void attn_plan_kernel(AttnParams p) {
    __shared__ int64_t red[kPlanThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nt = blockDim.x;
    int64_t carry = 0;
    for (int base = 0; base < p.pairs; base += nt) {
        const int pr = base + tid;
        const int64_t v = pr < p.pairs ? pair_groups(p, pr) : 0;
        const uint64_t inc = wave_scan_u64(static_cast<uint64_t>(v));
        if (lane == 63) red[w] = static_cast<int64_t>(inc);
        __syncthreads();
        int64_t before = 0, total = 0;
        for (int i = 0; i < nt / kWave; ++i) {
            if (i < w) before += red[i];
            total += red[i];
        }
        if (pr < p.pairs) p.plan[pr] = carry + before + static_cast<int64_t>(inc) - v;
        carry += total;
        __syncthreads();
    }
    if (tid == 0) p.plan[p.pairs] = carry;
    // second pass: the prefix of the pairs' workgroup shares
    const int64_t chunk = attn_chunk(carry, p.nwg, p.pairs);
    int64_t* wplan = p.plan + p.pairs + 1;
    carry = 0;
    for (int base = 0; base < p.pairs; base += nt) {
        const int pr = base + tid;
        const int64_t v = pr < p.pairs ? (pair_groups(p, pr) + chunk - 1) / chunk : 0;
        const uint64_t inc = wave_scan_u64(static_cast<uint64_t>(v));
        if (lane == 63) red[w] = static_cast<int64_t>(inc);
        __syncthreads();
        int64_t before = 0, total = 0;
        for (int i = 0; i < nt / kWave; ++i) {
            if (i < w) before += red[i];
            total += red[i];
        }
        if (pr < p.pairs) wplan[pr] = carry + before + static_cast<int64_t>(inc) - v;
        carry += total;
        __syncthreads();
    }
    if (tid == 0) wplan[p.pairs] = carry;
}

// The work plan as the attention and combine kernels see it: the prefix of
// the groups over the pairs, and the prefix of their workgroup shares. With at
// most 64 pairs every wave builds both itself: lane pr loads pair pr's group
// count and wave scans give the prefixes on lane pr, read back with readlane
// (pr is uniform). Otherwise they are the plan kernel's output.
struct PlanView {
    const int64_t* plan;       // [pairs + 1] group prefix, then [pairs + 1] workgroup prefix
    uint64_t incl;             // wave plan: inclusive group prefix on lane pr
    uint64_t wincl;            // wave plan: inclusive workgroup prefix on lane pr
    int64_t chunk;             // groups per workgroup share
    int pairs;
    bool wave;
    __device__ __forceinline__ PlanView(const AttnParams& p)
        : plan(p.plan), incl(0), wincl(0), chunk(0), pairs(p.pairs), wave(p.wave_plan != 0) {
        if (wave) {
            const int lane = threadIdx.x & (kWave - 1);
            const int64_t n = lane < pairs ? pair_groups(p, lane) : 0;
            incl = wave_scan_u64(static_cast<uint64_t>(n));
            chunk = attn_chunk(at(pairs), p.nwg, pairs);
            wincl = wave_scan_u64(static_cast<uint64_t>((n + chunk - 1) / chunk));
        } else {
            chunk = attn_chunk(plan[pairs], p.nwg, pairs);
        }
    }
    static __device__ __forceinline__ int64_t lane_read(uint64_t v, int l) {
        const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
        const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
        return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    }
    __device__ __forceinline__ int64_t at(int pr) const {     // first group of pair pr, 0 <= pr <= pairs
        if (!wave) return plan[pr];
        return pr == 0 ? 0 : lane_read(incl, pr - 1);
    }
    __device__ __forceinline__ int64_t wat(int pr) const {    // first workgroup of pair pr, 0 <= pr <= pairs
        if (!wave) return plan[pairs + 1 + pr];
        return pr == 0 ? 0 : lane_read(wincl, pr - 1);
    }
    __device__ __forceinline__ int64_t total() const { return at(pairs); }
    // the pair whose shares include workgroup w, or -1 past the last share
    __device__ __forceinline__ int pair_of_wg(int64_t w) const {
        if (w >= wat(pairs)) return -1;
        if (wave) {
            const int lane = threadIdx.x & (kWave - 1);
            const uint64_t prev = __shfl_up(wincl, 1);
            const int64_t excl = lane == 0 ? 0 : static_cast<int64_t>(prev);
            const unsigned long long bal = __ballot(lane < pairs && excl <= w);
            return __popcll(bal) - 1;                       // a prefix of lanes; the last one owns w
        }
        const int64_t* wp = plan + pairs + 1;
        int lo = 0, hi = pairs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (wp[mid] <= w) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
};

template <typename KT, int D, int G>
struct AttnCfg {
    // dims per lane: q and the accumulators of all G heads take 2*G*DPL <= 64 registers
    static constexpr int DPL = (32 / G < 4) ? (32 / G < 2 ? 2 : 32 / G) : (32 / G > D / 4 ? D / 4 : 32 / G);
    static constexpr int LPT = D / DPL;                              // lanes per token
    static constexpr int TPP = kWave / LPT;                          // tokens per pass
    static constexpr int NP = kGroupTokens / TPP;                    // passes per group
    static constexpr int WPP = DPL * static_cast<int>(sizeof(KT)) / 4;  // 32-bit words per lane per pass
};

template <int W>
__device__ __forceinline__ void load_words(const void* __restrict__ ptr, uint32_t (&w)[W]) {
    if constexpr (W % 4 == 0) {
        const uint4* v = static_cast<const uint4*>(ptr);
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
            const uint4 u = v[i];
            w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
        }
    } else if constexpr (W == 2) {
        const uint2 u = *static_cast<const uint2*>(ptr);
        w[0] = u.x; w[1] = u.y;
    } else {
        static_assert(W == 1, "one-, two- or four-word multiples");
        w[0] = *static_cast<const uint32_t*>(ptr);
    }
}

template <typename KT, int N, int W>
__device__ __forceinline__ void widen(const uint32_t (&w)[W], float (&x)[N]) {
    if constexpr (sizeof(KT) == 2) {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) x[i] = __uint_as_float(w[i]);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename KT, int D, int G>
__global__ __launch_bounds__(256) void attend_kernel(AttnParams p) {
    using C = AttnCfg<KT, D, G>;
    constexpr int NW = 4;
    constexpr int NP = C::NP, WPP = C::WPP, DPL = C::DPL, LPT = C::LPT, TPP = C::TPP;
    __shared__ float sm_m[NW][G], sm_l[NW][G];
    __shared__ float sm_acc[NW][G][D];

    const int wg = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform in the wave
    const int part = lane % LPT, tsub = lane / LPT;
    const PlanView pv(p);
    const int pr = pv.pair_of_wg(wg);           // the one pair this workgroup works on
    if (pr < 0) return;
    const int gpi = 1 << p.lgpi;
    const int tg = p.b >= kGroupTokens ? kGroupTokens : p.b;

    {
        // this workgroup's share of the pair's groups
        const int64_t ga = (wg - pv.wat(pr)) * pv.chunk, gb = imin(ga + pv.chunk, pv.at(pr + 1) - pv.at(pr));
        const int row = pr / p.Hkv, kv = pr % p.Hkv;
        const int s = row / p.ri.T;
        const int N = visible_clamped(p.ri, row, p.cap);

        float qv[G][DPL];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            load_vec<DPL>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + h) * D + part * DPL, qv[h]);
#pragma unroll
            for (int e = 0; e < DPL; ++e) qv[h][e] *= p.qscale;
        }
        const KT* Kb = static_cast<const KT*>(p.K) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + part * DPL;
        const KT* Vb = static_cast<const KT*>(p.V) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + part * DPL;
        const int2* items = p.items + static_cast<int64_t>(pr) * p.item_stride;

        float m[G], l[G], acc[G][DPL];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
        }

        // group g -> (chunk id, head mask): a scalar load (the address is
        // wave-uniform), issued two groups ahead of its use; its wait counts
        // scalar loads only, so the K/V rows in flight stay in flight
        auto item_of = [&](int64_t g) -> int2 {
            const int64_t it = g >> p.lgpi;
            if (p.dense) return make_int2(static_cast<int>(it), static_cast<int>(kAllHeads));
            return scalar_item(items, it);
        };
        auto first_token = [&](int64_t g, int2 e) -> int64_t {
            return (static_cast<int64_t>(e.x) << p.lb) + (g & (gpi - 1)) * kGroupTokens;
        };
        auto issue = [&](int64_t t0, uint32_t (&kb)[NP][WPP], uint32_t (&vb)[NP][WPP]) {
#pragma unroll
            for (int ps = 0; ps < NP; ++ps) {
                const int j = min(ps * TPP + tsub, tg - 1);
                const int64_t t = imin(t0 + j, N - 1);     // always a present row
                load_words<WPP>(Kb + t * D, kb[ps]);
                load_words<WPP>(Vb + t * D, vb[ps]);
            }
        };
        auto consume = [&](int64_t t0, uint32_t mask, const uint32_t (&kb)[NP][WPP], const uint32_t (&vb)[NP][WPP]) {
            float sc[NP][G];
#pragma unroll
            for (int ps = 0; ps < NP; ++ps) {
                const int j = ps * TPP + tsub;
                const int64_t t = t0 + j;
                const bool inb = (j < tg) && (t < N);
                float x[DPL];
                widen<KT, DPL, WPP>(kb[ps], x);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) a = fmaf(qv[h][e], x[e], a);
                    a = fast_group_sum<LPT>(a);
                    const bool ok = inb && ((mask & kAllHeads) || ((mask >> h) & 1u) || t == 0);
                    sc[ps][h] = ok ? a : -INFINITY;
                }
            }
            float mn[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float gm = sc[0][h];
#pragma unroll
                for (int ps = 1; ps < NP; ++ps) gm = fmaxf(gm, sc[ps][h]);
                mn[h] = fmaxf(m[h], gm);
                const float alpha = (mn[h] == -INFINITY) ? 1.f : fast_exp2(m[h] - mn[h]);   // 0 while nothing was seen
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] *= alpha;
                m[h] = mn[h];
            }
#pragma unroll
            for (int ps = 0; ps < NP; ++ps) {
                float v[DPL];
                widen<KT, DPL, WPP>(vb[ps], v);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float pr_ = (mn[h] == -INFINITY) ? 0.f : fast_exp2(sc[ps][h] - mn[h]);   // 0 when masked
                    l[h] += pr_;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(pr_, v[e], acc[h][e]);
                }
            }
        };

        // Software pipeline over this wave's groups ga+wave, +NW, +2NW, ...: while a
        // group is consumed, the K/V rows of the next one and the chunk id of the
        // one after are already in flight. Buffers A and B alternate. Every load
        // in the loop is unconditional (past the wave's last group the indices
        // stay on that group, whose rows the caches hold), so the waits before a
        // group's use leave the loads issued after it in flight.
        uint32_t kA[NP][WPP], vA[NP][WPP], kB[NP][WPP], vB[NP][WPP];
        const int64_t g0 = ga + wave;
        // this wave's groups (32-bit counters: their compares stay on the scalar unit)
        const int nk = g0 < gb ? static_cast<int>((gb - g0 + NW - 1) / NW) : 0;
        auto grp = [&](int k) { return g0 + static_cast<int64_t>(k < nk ? k : nk - 1) * NW; };
        if (nk > 0) {
            int2 e0 = item_of(grp(0));
            int2 e1 = item_of(grp(1));
            issue(first_token(grp(0), e0), kA, vA);
            // one exit, at the top: a path that left the loop from its middle
            // would reach the loop head with B's loads unwaited, and the wait
            // placed for it there would drain every load each iteration
            int k = 0;
            for (; k + 1 < nk; k += 2) {
                int2 e2 = item_of(grp(k + 2));
                issue(first_token(grp(k + 1), e1), kB, vB);
                consume(first_token(grp(k), e0), static_cast<uint32_t>(e0.y), kA, vA);
                e0 = e1;
                e1 = e2;
                e2 = item_of(grp(k + 3));
                issue(first_token(grp(k + 2), e1), kA, vA);
                consume(first_token(grp(k + 1), e0), static_cast<uint32_t>(e0.y), kB, vB);
                e0 = e1;
                e1 = e2;
            }
            if (k < nk) consume(first_token(grp(k), e0), static_cast<uint32_t>(e0.y), kA, vA);   // odd count
        }

        // ---- merge the token slots of each wave, then the waves ----
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float M = strided_max<LPT>(m[h]);
            const float f = (m[h] == -INFINITY) ? 0.f : fast_exp2(m[h] - M);
            const float lw = strided_sum<LPT>(l[h] * f);
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e] * f);
            if (lane < LPT) {
#pragma unroll
                for (int e = 0; e < DPL; ++e) sm_acc[wave][h][part * DPL + e] = acc[h][e];
            }
            if (lane == 0) {
                sm_m[wave][h] = M;
                sm_l[wave][h] = lw;
            }
        }
        __syncthreads();
        if (pv.wat(pr + 1) - pv.wat(pr) == 1) {
            // the pair's only share: normalise here (the combine skips the pair)
            const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * G;
            for (int idx = threadIdx.x; idx < G * (D + 1); idx += blockDim.x) {
                const int h = idx / (D + 1), c = idx % (D + 1);
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
                float L = 0.f, A = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - M);
                    L += f * sm_l[w][h];
                    if (c < D) A += f * sm_acc[w][h][c];
                }
                if (c < D) p.out[(rh0 + h) * D + c] = A * (L > 0.f ? 1.f / L : 0.f);
                else if (p.lse) p.lse[rh0 + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
            }
        } else {
            float* pout = p.partial + static_cast<int64_t>(wg) * G * (D + 4);
            for (int idx = threadIdx.x; idx < G * (D + 4); idx += blockDim.x) {
                const int h = idx / (D + 4), c = idx % (D + 4);
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
                float out = 0.f;
                if (c == 0) {
                    out = M;
                } else if (c == 1 || c >= 4) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - M);
                        out += f * (c == 1 ? sm_l[w][h] : sm_acc[w][h][c - 4]);
                    }
                }
                pout[idx] = out;
            }
        }
    }
}

// ----------------------------------------------------------------------------
// split-K attention for bf16 caches with the scores on the matrix cores
// Same work split, pipeline, partial slots and merge as attend_kernel; the
// group's 16 x g score tile is one 16x16x32 bf16 MFMA per 32 dimensions:
//   S^T[token][head] = sum_d K[token][d] * q[head][d],
// A = the group's K rows (lane l: token l % 16, dims [(l/16) D/4, +D/4), read
// straight from HBM as bf16), B = q (lane l: head l % 16, same dims; heads
// >= g are zero). The scaled q is split into three bf16 parts, hi + mid + lo,
// that sum to it exactly but for the last part's rounding (about 2^-25 of
// |q|): every product of a bf16 key with a bf16 part is exact in fp32 and the
// MFMA accumulates in fp32, so q . k is an fp32 dot product of the bf16 key
// and the fp32 query (three MFMAs per slice). The result holds token
// 4 (l/16) + r, head l % 16 in lane l, register r: the online softmax runs in
// that layout, and the probabilities go through LDS to the value pass, which
// stays on the VALU (lanes own 4 tokens x D/LPT dims as in attend_kernel).
// ----------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_bits_rn(float x) {   // round to nearest even
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// NW waves a workgroup: 8 when the pairs are few and g <= 4 (half the
// workgroups, so half the partial slots for the combine to merge), else 4.
template <int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void attend_mfma_kernel(AttnParams p) {
    using C = AttnCfg<uint16_t, D, G>;
    constexpr int NP = C::NP, WPP = C::WPP, DPL = C::DPL, LPT = C::LPT, TPP = C::TPP;
    constexpr int KW = D / 8;                    // 32-bit words of K per lane (D/4 bf16)
    constexpr int NS = D / 32;                   // MFMA slices of 32 dimensions
    static_assert(G <= 16 && kGroupTokens == 16, "16 x 16 score tile");
    __shared__ float sm_m[NW][G], sm_l[NW][G];
    __shared__ float sm_acc[NW][G][D];
    __shared__ float sm_p[NW][kGroupTokens][G];   // a group's probabilities, token-major

    const int wg = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // uniform in the wave
    const int part = lane % LPT, tsub = lane / LPT;       // value-pass layout
    const int mrow = lane & 15, mblk = lane >> 4;          // MFMA layout: token/head, dim block
    const PlanView pv(p);
    const int pr = pv.pair_of_wg(wg);           // the one pair this workgroup works on
    if (pr < 0) return;
    const int gpi = 1 << p.lgpi;
    const int tg = p.b >= kGroupTokens ? kGroupTokens : p.b;

    {
        // this workgroup's share of the pair's groups
        const int64_t ga = (wg - pv.wat(pr)) * pv.chunk, gb = imin(ga + pv.chunk, pv.at(pr + 1) - pv.at(pr));
        const int row = pr / p.Hkv, kv = pr % p.Hkv;
        const int s = row / p.ri.T;
        const int N = visible_clamped(p.ri, row, p.cap);

        // q of head mrow (zero beyond g): its load is issued here, its split into
        // scaled bf16 hi + mid + lo parts waits until the first K/V rows are in flight
        bf16x8_t qh[NS], qm[NS], ql[NS];
        float qf[D / 4];
        if (mrow < G) {
            load_vec<D / 4>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + mrow) * D + mblk * (D / 4), qf);
        } else {
#pragma unroll
            for (int e = 0; e < D / 4; ++e) qf[e] = 0.f;
        }
        auto split_q = [&]() {
#pragma unroll
            for (int sl = 0; sl < NS; ++sl)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    // x - hi and x - hi - mid are exact in fp32; hi + mid + lo
                    // equals x up to lo's rounding
                    const float x = qf[sl * 8 + j] * p.qscale;
                    const uint32_t hb = bf16_bits_rn(x);
                    const float r1 = x - __uint_as_float(hb << 16);
                    const uint32_t mb = bf16_bits_rn(r1);
                    const uint32_t lb = bf16_bits_rn(r1 - __uint_as_float(mb << 16));
                    qh[sl][j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hb));
                    qm[sl][j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(mb));
                    ql[sl][j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(lb));
                }
        };
        const uint16_t* Kr = static_cast<const uint16_t*>(p.K) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + mblk * (D / 4);
        const uint16_t* Vb = static_cast<const uint16_t*>(p.V) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + part * DPL;
        const int2* items = p.items + static_cast<int64_t>(pr) * p.item_stride;

        // softmax state: in the MFMA layout (head mrow) m and this lane's share of l;
        // the accumulators in the value-pass layout
        float m = -INFINITY, l = 0.f;
        float acc[G][DPL];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;

        // group g -> (chunk id, head mask): a scalar load (the address is
        // wave-uniform), issued two groups ahead of its use; its wait counts
        // scalar loads only, so the K/V rows in flight stay in flight
        auto item_of = [&](int64_t g) -> int2 {
            const int64_t it = g >> p.lgpi;
            if (p.dense) return make_int2(static_cast<int>(it), static_cast<int>(kAllHeads));
            return scalar_item(items, it);
        };
        auto first_token = [&](int64_t g, int2 e) -> int64_t {
            return (static_cast<int64_t>(e.x) << p.lb) + (g & (gpi - 1)) * kGroupTokens;
        };
        auto issue = [&](int64_t t0, uint32_t (&kb)[KW], uint32_t (&vb)[NP][WPP]) {
            {
                const int j = min(mrow, tg - 1);
                const int64_t t = imin(t0 + j, N - 1);        // always a present row
                load_words<KW>(Kr + t * D, kb);
            }
#pragma unroll
            for (int ps = 0; ps < NP; ++ps) {
                const int j = min(ps * TPP + tsub, tg - 1);
                const int64_t t = imin(t0 + j, N - 1);
                load_words<WPP>(Vb + t * D, vb[ps]);
            }
        };
        auto consume = [&](int64_t t0, uint32_t mask, const uint32_t (&kb)[KW], const uint32_t (&vb)[NP][WPP]) {
            // scores: 16 tokens x 16 heads
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                bf16x8_t a;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = kb[sl * 4 + j];
                    a[2 * j] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w & 0xffffu));
                    a[2 * j + 1] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(w >> 16));
                }
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[sl], sc, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qm[sl], sc, 0, 0, 0);
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[sl], sc, 0, 0, 0);
            }
            // online softmax of head mrow over tokens 4 * mblk + r
            const bool hv = mrow < G;
            const bool hm = hv && ((mask & kAllHeads) || ((mask >> mrow) & 1u));
            float sv[4], gm = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 4 * mblk + r;
                const int64_t t = t0 + j;
                const bool ok = hv && (j < tg) && (t < N) && (hm || t == 0);
                sv[r] = ok ? sc[r] : -INFINITY;
                gm = fmaxf(gm, sv[r]);
            }
            gm = fmaxf(gm, __shfl_xor(gm, 16));
            gm = fmaxf(gm, __shfl_xor(gm, 32));
            const float mn = fmaxf(m, gm);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);   // 0 while nothing was seen
            float ps_sum = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pr_ = (mn == -INFINITY) ? 0.f : fast_exp2(sv[r] - mn);   // 0 when masked
                ps_sum += pr_;
                if (hv) sm_p[wave][4 * mblk + r][mrow] = pr_;
            }
            l = l * alpha + ps_sum;
            m = mn;
            __builtin_amdgcn_wave_barrier();
            // value pass: rescale, then accumulate p * v for the lane's tokens
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] *= ah;
            }
#pragma unroll
            for (int ps = 0; ps < NP; ++ps) {
                float v[DPL];
                widen<uint16_t, DPL, WPP>(vb[ps], v);
                const float* pp = &sm_p[wave][ps * TPP + tsub][0];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float ph = pp[h];
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(ph, v[e], acc[h][e]);
                }
            }
            __builtin_amdgcn_wave_barrier();                       // sm_p is rewritten by the next group
        };

        // the pipeline of attend_kernel: unconditional loads, A and B alternating
        uint32_t kA[KW], vA[NP][WPP], kB[KW], vB[NP][WPP];
        const int64_t g0 = ga + wave;
        // this wave's groups (32-bit counters: their compares stay on the scalar unit)
        const int nk = g0 < gb ? static_cast<int>((gb - g0 + NW - 1) / NW) : 0;
        auto grp = [&](int k) { return g0 + static_cast<int64_t>(k < nk ? k : nk - 1) * NW; };
        if (nk > 0) {
            int2 e0 = item_of(grp(0));
            int2 e1 = item_of(grp(1));
            issue(first_token(grp(0), e0), kA, vA);
            split_q();
            int k = 0;
            for (; k + 1 < nk; k += 2) {          // one exit, at the top (see attend_kernel)
                int2 e2 = item_of(grp(k + 2));
                issue(first_token(grp(k + 1), e1), kB, vB);
                consume(first_token(grp(k), e0), static_cast<uint32_t>(e0.y), kA, vA);
                e0 = e1;
                e1 = e2;
                e2 = item_of(grp(k + 3));
                issue(first_token(grp(k + 2), e1), kA, vA);
                consume(first_token(grp(k + 1), e0), static_cast<uint32_t>(e0.y), kB, vB);
                e0 = e1;
                e1 = e2;
            }
            if (k < nk) consume(first_token(grp(k), e0), static_cast<uint32_t>(e0.y), kA, vA);   // odd count
        }

        // ---- merge: the four dim blocks' shares of l, the token slots of the
        // accumulators, then the waves ----
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (lane < G) {
            sm_m[wave][lane] = m;
            sm_l[wave][lane] = l;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e]);
            if (lane < LPT) {
#pragma unroll
                for (int e = 0; e < DPL; ++e) sm_acc[wave][h][part * DPL + e] = acc[h][e];
            }
        }
        __syncthreads();
        if (pv.wat(pr + 1) - pv.wat(pr) == 1) {
            // the pair's only share: normalise here (the combine skips the pair)
            const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * G;
            for (int idx = threadIdx.x; idx < G * (D + 1); idx += blockDim.x) {
                const int h = idx / (D + 1), c = idx % (D + 1);
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
                float L = 0.f, A = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - M);
                    L += f * sm_l[w][h];
                    if (c < D) A += f * sm_acc[w][h][c];
                }
                if (c < D) p.out[(rh0 + h) * D + c] = A * (L > 0.f ? 1.f / L : 0.f);
                else if (p.lse) p.lse[rh0 + h] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
            }
        } else {
            float* pout = p.partial + static_cast<int64_t>(wg) * G * (D + 4);
            for (int idx = threadIdx.x; idx < G * (D + 4); idx += blockDim.x) {
                const int h = idx / (D + 4), c = idx % (D + 4);
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
                float out = 0.f;
                if (c == 0) {
                    out = M;
                } else if (c == 1 || c >= 4) {
#pragma unroll
                    for (int w = 0; w < NW; ++w) {
                        const float f = (sm_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sm_m[w][h] - M);
                        out += f * (c == 1 ? sm_l[w][h] : sm_acc[w][h][c - 4]);
                    }
                }
                pout[idx] = out;
            }
        }
    }
}

// ----------------------------------------------------------------------------
// LSE merge of a pair's segments: one workgroup per (row, query head)
// Thread (group, quad) merges every NGRP-th slot of the pair for four
// dimensions: a slot's max, sum and float4 of the accumulator arrive in one
// round of loads, kCombineUnroll slots at a time, into a private online LSE
// state. The NGRP states then merge through LDS.
// ----------------------------------------------------------------------------
constexpr int kCombineThreads = 1024;
constexpr int kCombineUnroll = 16;

template <int D, int G>
__global__ __launch_bounds__(kCombineThreads) void attend_combine_kernel(AttnParams p, float* out, float* lse) {
    constexpr int Q = D / 4;                        // float4 quads of a row
    constexpr int NGRP = kCombineThreads / Q;       // slot groups
    constexpr int U = kCombineUnroll;
    constexpr int64_t SS = static_cast<int64_t>(G) * (D + 4);   // floats per slot
    __shared__ float sm_m[NGRP], sm_l[NGRP];
    __shared__ float4 sm_a[NGRP][Q];
    const int64_t rh = blockIdx.x;
    const int row = static_cast<int>(rh / p.Hq), hq = static_cast<int>(rh % p.Hq);
    const int kv = hq / G, h = hq % G;
    const int pr = row * p.Hkv + kv;
    const int tid = threadIdx.x, quad = tid % Q, grp = tid / Q;
    const PlanView pv(p);
    const int64_t w0 = pv.wat(pr), w1 = pv.wat(pr + 1);       // the pair's workgroups = its slots
    if (w0 >= w1) {                                              // nothing visible
        if (tid < D) out[rh * D + tid] = 0.f;
        if (tid == 0 && lse) lse[rh] = -INFINITY;
        return;
    }
    if (w1 - w0 == 1) return;                                    // its one workgroup wrote the output
    const int nslot = static_cast<int>(w1 - w0);
    const float* pp = p.partial + (w0 * G + h) * (D + 4);       // slot i at pp + i * SS
    float M = -INFINITY, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = grp; i0 < nslot; i0 += NGRP * U) {
        float mi[U], li[U];
        float4 ai[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * NGRP;
            if (i < nslot) {
                const float* sp = pp + i * SS;
                mi[u] = sp[0];
                li[u] = sp[1];
                ai[u] = *reinterpret_cast<const float4*>(sp + 4 + 4 * quad);
            } else {
                mi[u] = -INFINITY;
                li[u] = 0.f;
                ai[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (mi[u] == -INFINITY) continue;
            const float Mn = fmaxf(M, mi[u]);
            const float fo = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
            const float fi = fast_exp2(mi[u] - Mn);
            L = L * fo + li[u] * fi;
            A.x = A.x * fo + ai[u].x * fi;
            A.y = A.y * fo + ai[u].y * fi;
            A.z = A.z * fo + ai[u].z * fi;
            A.w = A.w * fo + ai[u].w * fi;
            M = Mn;
        }
    }
    if (quad == 0) {
        sm_m[grp] = M;
        sm_l[grp] = L;
    }
    sm_a[grp][quad] = A;
    __syncthreads();
    if (tid < Q) {
        float Mx = -INFINITY;
#pragma unroll 8
        for (int g = 0; g < NGRP; ++g) Mx = fmaxf(Mx, sm_m[g]);
        float Lt = 0.f;
        float4 At = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int g = 0; g < NGRP; ++g) {
            const float mg = sm_m[g];
            const float f = (mg == -INFINITY) ? 0.f : fast_exp2(mg - Mx);
            Lt += f * sm_l[g];
            const float4 a = sm_a[g][tid];
            At.x += f * a.x;
            At.y += f * a.y;
            At.z += f * a.z;
            At.w += f * a.w;
        }
        const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
        float* o = out + rh * D + 4 * tid;            // caller memory: no alignment assumed
        o[0] = At.x * inv;
        o[1] = At.y * inv;
        o[2] = At.z * inv;
        o[3] = At.w * inv;
        if (tid == 0 && lse) lse[rh] = (Lt > 0.f) ? (Mx + __log2f(Lt)) * kLn2 : -INFINITY;
    }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
// Attention workgroups of one launch: what the chip holds at once at the
// kernel's register use (blocks per compute unit x compute units), at most
// kAttnWorkgroups. A kernel that holds one block per compute unit then runs
// its shares in one round rather than two with a tail. Read once per device.
template <auto Kernel>
static int resident_workgroups(int block) {
    static int cached[64] = {0};        // per kernel and device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kAttnWorkgroups;
    int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (n > 0) return n;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(Kernel), block, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1) {
        (void)hipGetLastError();
        return kAttnWorkgroups;
    }
    n = per_cu * cus < kAttnWorkgroups ? per_cu * cus : kAttnWorkgroups;
    __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
    return n;
}

// Eight-wave bf16 workgroups: few pairs (the kernels build the plan
// themselves) and g <= 4, where the kernel holds two waves a SIMD.
static bool attn_wide(bool bf16, int G, int pairs) { return bf16 && G <= 4 && pairs <= kWave; }

template <typename KT, int D, int G>
static int attn_workgroups_t(bool wide) {
    if constexpr (sizeof(KT) == 2) {
        if constexpr (G <= 4)
            if (wide) return resident_workgroups<attend_mfma_kernel<D, G, 8>>(8 * kWave);
        return resident_workgroups<attend_mfma_kernel<D, G, 4>>(4 * kWave);
    } else {
        return resident_workgroups<attend_kernel<KT, D, G>>(256);
    }
}

template <typename KT, int D>
static int attn_workgroups_g(int G, bool wide) {
    switch (G) {
        case 1: return attn_workgroups_t<KT, D, 1>(wide);
        case 2: return attn_workgroups_t<KT, D, 2>(wide);
        case 4: return attn_workgroups_t<KT, D, 4>(wide);
        case 8: return attn_workgroups_t<KT, D, 8>(wide);
        case 16: return attn_workgroups_t<KT, D, 16>(wide);
        default: return kAttnWorkgroups;
    }
}

template <typename KT, int D, int G>
static hipError_t launch_attn_t(const AttnParams& ap, int rows, int Hq, float* out, float* lse, bool wide,
                                hipStream_t st) {
    {
        ProfScope ps("attend", 0, st);
        if constexpr (sizeof(KT) == 2)       // bf16 cache: scores on the matrix cores
        {
            bool launched = false;
            if constexpr (G <= 4) {
                if (wide) {
                    hipLaunchKernelGGL((attend_mfma_kernel<D, G, 8>), dim3(ap.nwg + ap.pairs), dim3(8 * kWave), 0, st, ap);
                    launched = true;
                }
            }
            if (!launched)
                hipLaunchKernelGGL((attend_mfma_kernel<D, G, 4>), dim3(ap.nwg + ap.pairs), dim3(4 * kWave), 0, st, ap);
        }
        else
            hipLaunchKernelGGL((attend_kernel<KT, D, G>), dim3(ap.nwg + ap.pairs), dim3(256), 0, st, ap);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ProfScope ps("attend_combine", 0, st);
    hipLaunchKernelGGL((attend_combine_kernel<D, G>), dim3(rows * Hq), dim3(kCombineThreads), 0, st, ap, out, lse);
    return hipGetLastError();
}

template <typename KT, int D>
static hipError_t attn_g(int G, const AttnParams& ap, int rows, int Hq, float* out, float* lse, bool wide,
                         hipStream_t st) {
    switch (G) {
        case 1: return launch_attn_t<KT, D, 1>(ap, rows, Hq, out, lse, wide, st);
        case 2: return launch_attn_t<KT, D, 2>(ap, rows, Hq, out, lse, wide, st);
        case 4: return launch_attn_t<KT, D, 4>(ap, rows, Hq, out, lse, wide, st);
        case 8: return launch_attn_t<KT, D, 8>(ap, rows, Hq, out, lse, wide, st);
        case 16: return launch_attn_t<KT, D, 16>(ap, rows, Hq, out, lse, wide, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attend(const Geo& g, const AttendArgs& a, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    const int pairs = a.rows * g.Hkv;
    if (!a.dense) {
        uint32_t* bm1 = reinterpret_cast<uint32_t*>(ws + lay.bitmap) + lay.bm_off[0];
        const int64_t leaf_words = (g.nodes[0] + 32) / 32;
        if (!a.bitmaps_ready) {
            BitmapParams bp{a.sel_blocks, a.n_sel, a.sel_cap, bm1, lay.bm_words_total, leaf_words};
            ProfScope ps("attn_bitmap", 0, st);
            hipLaunchKernelGGL(attn_bitmap_kernel, dim3(a.rows * g.Hq), dim3(256), 0, st, bp);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        ItemsParams ip{};
        ip.ri = a.ri;
        ip.bm = bm1;
        ip.stride = lay.bm_words_total;
        ip.items = reinterpret_cast<int2*>(ws + lay.aitems);
        ip.item_stride = g.nodes[0] + 2;
        ip.acnt = reinterpret_cast<int32_t*>(ws + lay.acnt);
        ip.cap = g.cap;
        ip.lb = g.lb;
        ip.Hq = g.Hq;
        ip.Hkv = g.Hkv;
        ip.seg_words = items_seg_words(pairs);
        const int64_t nseg = items_segments(g, pairs);
        if (nseg > kItemsRecountSegs) {
            ip.segcnt = reinterpret_cast<int32_t*>(ws + lay.segcnt);
            ip.seg_stride = nseg;
        }
        const dim3 gi(static_cast<unsigned>(nseg), pairs), bi(kItemsThreads);
        if (ip.segcnt) {
            ProfScope ps("attn_segcount", 0, st);
            switch (g.G) {
                case 1: hipLaunchKernelGGL(attn_segcount_kernel<1>, gi, bi, 0, st, ip); break;
                case 2: hipLaunchKernelGGL(attn_segcount_kernel<2>, gi, bi, 0, st, ip); break;
                case 4: hipLaunchKernelGGL(attn_segcount_kernel<4>, gi, bi, 0, st, ip); break;
                case 8: hipLaunchKernelGGL(attn_segcount_kernel<8>, gi, bi, 0, st, ip); break;
                case 16: hipLaunchKernelGGL(attn_segcount_kernel<16>, gi, bi, 0, st, ip); break;
                default: return hipErrorInvalidValue;
            }
        }
        {
            ProfScope ps("attn_items", 0, st);
            switch (g.G) {
                case 1: hipLaunchKernelGGL(attn_items_kernel<1>, gi, bi, 0, st, ip); break;
                case 2: hipLaunchKernelGGL(attn_items_kernel<2>, gi, bi, 0, st, ip); break;
                case 4: hipLaunchKernelGGL(attn_items_kernel<4>, gi, bi, 0, st, ip); break;
                case 8: hipLaunchKernelGGL(attn_items_kernel<8>, gi, bi, 0, st, ip); break;
                case 16: hipLaunchKernelGGL(attn_items_kernel<16>, gi, bi, 0, st, ip); break;
                default: return hipErrorInvalidValue;
            }
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    AttnParams ap{};
    ap.q = a.q;
    ap.ri = a.ri;
    ap.K = a.K;
    ap.V = a.V;
    ap.items = reinterpret_cast<const int2*>(ws + lay.aitems);
    ap.acnt = reinterpret_cast<const int32_t*>(ws + lay.acnt);
    ap.item_stride = g.nodes[0] + 2;
    ap.plan = reinterpret_cast<int64_t*>(ws + lay.plan);
    ap.partial = reinterpret_cast<float*>(ws + lay.partial);
    ap.cap = g.cap;
    ap.b = g.b;
    ap.lb = g.lb;
    ap.lgpi = g.lb > 4 ? g.lb - 4 : 0;          // groups of kGroupTokens per chunk
    ap.Hq = g.Hq;
    ap.Hkv = g.Hkv;
    ap.pairs = pairs;
    const bool wide = attn_wide(g.kv_dtype == ZHA_KV_BF16, g.G, pairs);
    {
        const bool bf16 = g.kv_dtype == ZHA_KV_BF16;
        ap.nwg = g.D == 128 ? (bf16 ? attn_workgroups_g<uint16_t, 128>(g.G, wide) : attn_workgroups_g<float, 128>(g.G, wide))
                            : (bf16 ? attn_workgroups_g<uint16_t, 64>(g.G, wide) : attn_workgroups_g<float, 64>(g.G, wide));
    }
    ap.dense = a.dense ? 1 : 0;
    ap.wave_plan = pairs <= kWave ? 1 : 0;
    ap.qscale = g.scale * kLog2e;
    ap.out = a.out;
    ap.lse = a.lse;
    if (!ap.wave_plan) {
        {
            ProfScope ps("attn_plan", 0, st);
            hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, ap);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool bf = g.kv_dtype == ZHA_KV_BF16;
    if (g.D == 128)
        return bf ? attn_g<uint16_t, 128>(g.G, ap, a.rows, g.Hq, a.out, a.lse, wide, st)
                  : attn_g<float, 128>(g.G, ap, a.rows, g.Hq, a.out, a.lse, wide, st);
    return bf ? attn_g<uint16_t, 64>(g.G, ap, a.rows, g.Hq, a.out, a.lse, wide, st)
              : attn_g<float, 64>(g.G, ap, a.rows, g.Hq, a.out, a.lse, wide, st);
}

}  // namespace zha

// route.hip - top-down routing of queries through the ZHA tree.
//
// Per level l, from the top ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", §Routing):
//   candidates = children of the nodes kept at l+1, plus the level's complete
//                nodes whose parent is incomplete (at the top: every complete
//                node);
//   score      = scale * q . summary, fp32;
//   keep       = the smallest prefix in (score desc, node id asc) order whose
//                softmax mass is >= top_p of the candidates' total.
//
// Kernels, ordered by kernel boundaries alone: no device-scope fences (on this
// part every XCD has its own L2, and a device-scope release writes L2 back).
// The one cross-workgroup atomic is the split cut's u64 add into a pair's
// mass bins (route_split_hist_kernel): integer sums are exact in any order,
// and only the next kernel reads them.
//  * route_upper_kernel - one workgroup per (row, query head) walks the small
//    upper levels in one launch: candidates, scores and the cut stay in LDS
//    from level to level. When the levels above the lowest fused one hold at
//    most 64 nodes each, every node of the fused levels is scored up front:
//    wave 0 scores and cuts the small levels while the other waves score the
//    lowest one, so its scoring no longer waits for the cuts above it.
//  * per remaining level (the leaf level always):
//    - route_score_kernel - a workgroup owns up to 64 interleaved parent slots of one
//      (row, kv head). It ORs the group's kept bitmaps of level l+1 over its
//      slots (plus the incomplete parent, whose complete children are the
//      orphans) and scores each such parent's b children once for all g query
//      heads: a summary row is read once per kv group. Scores land in a
//      dense-by-node array per (row, query head).
//    - the cut: with few (row, head) pairs, route_split_hist_kernel and
//      route_split_emit_kernel spread each pair's cut over slices of its
//      candidates; otherwise route_cut_kernel, one workgroup per (row, query
//      head), with the scores staged in LDS when they fit.
// The cut itself: masses exp(s - max) are held in 2^-40 fixed point, so their
// sums are exact and independent of order. The masses are binned by the
// score's distance below the max; the bin where the running mass reaches
// ceil(top_p * total) holds the boundary, which a ranking or a radix select
// over that bin's members (an order-preserving score key) pins down exactly.
// Ties at the boundary go to the lower node ids; a stable compaction writes
// the kept ids in ascending order and the head's kept bitmap. The small upper
// levels use a radix select over all their candidates.
#include <algorithm>
#include <type_traits>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

// ----------------------------------------------------------------------------
// scoring
// ----------------------------------------------------------------------------
struct ScoreParams {
    const float* q;            // [rows, Hq, D]
    RowInfo ri;
    const float* summ;         // summaries of this level (R tangent rows per node with tangent scoring)
    const float* offs;         // tangent scoring: this level's offsets (R per node), else null
    int R;                     // tangent rows per node (1 without tangent scoring)
    int64_t nodes_l;           // node slots per (batch, kv) at this level
    float* scores;             // ws scores base
    int64_t nodes_total;       // per (row, head) stride of the scores
    int64_t lvl_off;           // offset of this level in a (row, head) score array
    const uint32_t* bm_up;     // kept bitmaps of level l+1 (row-head stride bm_words_total)
    int64_t bm_words_total;
    int64_t cap;
    int b, lb, li, L, Hq, Hkv, T;
    float scale;
    // split cut of this level (pmax null otherwise): every workgroup leaves the
    // maximum of each head's own candidates it scored and writes their scores
    // and ids in the head's candidate order; the workgroups of a (row, kv
    // head) clear the heads' mass bins and this level's bitmaps between them
    float* pmax;               // [rows, Hq, pmax_stride], column = the workgroup's run within its pair
    int64_t pmax_stride;
    int32_t* pruns;            // [rows, Hq]: runs (workgroups) of the head's pair
    // waves dealt by parent counts (ScoreShape): the 1-D grid's size, 0 for a
    // grid of runs x pairs; the pairs, and the waves each gets at least
    int64_t bal_waves;
    int pairs;
    int64_t bal_need;
    unsigned long long* chist; // [rows, Hq, kCutBins]
    uint32_t* bm_cur;          // this level's kept bitmaps (row-head stride bm_words_total)
    const int32_t* rank_up;    // [rows, Hq, nodes_total]: a kept node's place in its head's kept list (level l+1)
    int64_t lvl_off_up;
    const int32_t* kept_cnt;   // [rows, Hq, L]
    float* cand_sc;            // [rows, Hq, cand_stride]
    int32_t* cand_nd;
    int64_t cand_stride;
};

// The pair and run of this scoring wave when the waves are dealt by parent
// counts: lane l < pairs weighs pair l by the parents its heads kept at the
// level above (their summed counts capped at the level's complete parents;
// all its slots at the top), and pair l owns waves
// [end(l-1), end(l)) with end(l) = need (l+1) + extra * (weights of pairs
// 0..l) / (all weights), extra = the waves beyond need per pair. Every wave
// derives the same split from the same counts.
// Tokens a row sees (clamp_visible) with its two loads issued together.
__device__ __forceinline__ int score_visible(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T, t = row % ri.T;
    const int len = ri.seq_lens[s];
    const int pos = ri.q_pos ? ri.q_pos[row] : len - ri.T + t;
    const int n = pos + 1;
    const int lim = static_cast<int>(len < cap ? len : cap);
    return n < 0 ? 0 : (n > lim ? lim : n);
}

template <int G>
__device__ __forceinline__ void score_deal(const ScoreParams& p, int* y_out, int* run_out, int64_t* w_out,
                                           int* n_out) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool top = (p.li == p.L - 1);
    uint64_t wgt = 0;
    int nl = 0;
    if (lane < p.pairs) {
        // one round of loads, every address valid whatever the level: the
        // row's length and position, and its heads' kept counts
        const int row = lane / p.Hkv, kv = lane % p.Hkv;
        const int sq = row / p.ri.T, t = row % p.ri.T;
        const int32_t* pp = p.ri.q_pos ? p.ri.q_pos + row : p.ri.seq_lens + sq;
        const int len = p.ri.seq_lens[sq];
        const int pv = *pp;
        const int64_t r0 = static_cast<int64_t>(row) * p.Hq + kv * G;
        const int lup = p.li + 1 < p.L ? p.li + 1 : p.L - 1;
        int32_t kcs[G];
#pragma unroll
        for (int h = 0; h < G; ++h) kcs[h] = p.kept_cnt[(r0 + h) * p.L + lup];
        __asm__ volatile("" ::: "memory");               // not sunk into the branch below
        const int n = (p.ri.q_pos ? pv : len - p.ri.T + t) + 1;
        const int lim = static_cast<int>(len < p.cap ? len : p.cap);
        nl = n < 0 ? 0 : (n > lim ? lim : n);
        if (top) {
            wgt = static_cast<uint64_t>((((static_cast<int64_t>(nl) >> (p.lb * (p.li + 1))) + p.b - 1) >> p.lb));
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h) wgt += static_cast<uint64_t>(kcs[h]);
            // the pair's active parents are the union of its heads' kept sets:
            // at most their summed counts and at most the complete parents
            // (heads that keep most of a level overlap, and the sum overstates)
            const uint64_t ncu = static_cast<uint64_t>(static_cast<int64_t>(nl) >> (p.lb * (p.li + 2)));
            wgt = wgt < ncu ? wgt : ncu;
            wgt += 1;                                    // the incomplete parent
        }
    }
    const uint64_t cum = wave_scan_u64(wgt);
    const uint64_t tot = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                             static_cast<int>(static_cast<uint32_t>(cum)), p.pairs - 1))) |
                         (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(
                              static_cast<int>(static_cast<uint32_t>(cum >> 32)), p.pairs - 1))) << 32);
    const int64_t extra = p.bal_waves - p.bal_need * p.pairs;
    const int64_t share = tot ? static_cast<int64_t>(static_cast<uint64_t>(extra) * cum / tot)
                              : extra * (lane + 1) / p.pairs;
    const int end = static_cast<int>(p.bal_need * (lane + 1) + share);
    const int gw = blockIdx.x;
    const int y = __popcll(__ballot(lane < p.pairs && end <= gw));
    const int start = y ? __builtin_amdgcn_readlane(end, y - 1) : 0;
    *y_out = y;
    *run_out = gw - start;
    *w_out = __builtin_amdgcn_readlane(end, y) - start;
    *n_out = __builtin_amdgcn_readlane(nl, y);
}

// Workgroup = one wave = at most 64 parent slots of one (row, kv head), taken
// every W-th of the pair's W waves, its active parents one at a time. The
// wave builds the slots' masks with ballots (lane = slot): the slots some head
// of the group kept, and for each head the slots it takes candidates from.
// About 2048 waves in all, what the chip holds at once at this kernel's
// register use; with few pairs they are dealt by parent counts (score_deal),
// so a heavy pair's parents are spread as wide as the chip allows.
template <int D, int G, bool TAN>
__global__ __launch_bounds__(kScoreThreads) void route_score_kernel(ScoreParams p) {
    static_assert(kScoreThreads == kWave, "a scoring workgroup is one wave");
    int y, run, N;
    int64_t W;
    if (p.bal_waves) {
        score_deal<G>(p, &y, &run, &W, &N);
    } else {
        y = blockIdx.y;
        run = blockIdx.x;
        W = gridDim.x;
        N = score_visible(p.ri, y / p.Hkv, p.cap);
    }
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.T;
    const bool top = (p.li == p.L - 1);
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (p.li + 2)));
    const int64_t orphans = nc - (nc_up << p.lb);
    const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * G;      // the group's first (row, head)
    const bool split = p.pmax != nullptr;
    if (split && run == 0 && threadIdx.x < G) p.pruns[rh0 + threadIdx.x] = static_cast<int32_t>(W);
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int DPL = (G <= 4) ? 16 : (G == 8 ? 8 : 4);   // dims per lane
    constexpr int LPR = D / DPL;                             // lanes per summary row
    constexpr int RPP = kWave / LPR;                         // rows per pass
    constexpr int UNR = 4;                                   // passes issued together
    static_assert(G <= LPR, "one lane per head writes the head's score");
    const int sub = lane / LPR, part = lane % LPR;

    // The pair's active parents, in node order: at the top every block of b
    // nodes; below, the complete parents some head of the group kept at the
    // level above, then the incomplete parent holding the orphans (taken by
    // every head). The wave takes active parents run, run + W, run + 2W, ...,
    // so a pair's parents spread evenly over its waves however the cut
    // clustered them. Below the top the wave finds them from the union of
    // the heads' kept bits, kWpl words a lane per pass.
    constexpr int kWpl = 4;
    const int64_t nwords = top ? 0 : (nc_up + 31) >> 5;
    // first round of loads, every address valid whatever the level: the
    // heads' queries, the first pass's kept bits, and the heads' kept counts
    // at the level above (the incomplete parent's children follow the kept
    // parents' in a head's candidate order)
    float qv[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) load_row_il<DPL, LPR>(p.q + (rh0 + h) * D + part * 4, qv[h]);
    const int lup = p.li + 1 < p.L ? p.li + 1 : p.L - 1;
    int32_t kc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) kc[h] = p.kept_cnt[(rh0 + h) * p.L + lup];
    uint32_t u[kWpl];
    auto load_union = [&](int64_t w0) {
#pragma unroll
        for (int k = 0; k < kWpl; ++k) {
            const int64_t wd = w0 + static_cast<int64_t>(lane) * kWpl + k;
            const int64_t wc = wd < nwords ? wd : 0;
            uint32_t x = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) x |= p.bm_up[(rh0 + h) * p.bm_words_total + wc];
            // only bits of complete parents count
            const int64_t lo = wd << 5;
            const uint32_t valid = wd >= nwords ? 0u : (nc_up - lo >= 32 ? ~0u : ((1u << (nc_up - lo)) - 1u));
            u[k] = x & valid;
        }
    };
    load_union(0);
    __asm__ volatile("" ::: "memory");      // keeps the loads above here, in one round

    const int RT = TAN ? p.R : 1;                            // tangent rows per node
    const int64_t nbase = (static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes_l;   // this pair's first node
    const float* summ = p.summ + nbase * RT * D;
    const float* offs = TAN ? p.offs + nbase * RT : nullptr;
    float* sc0 = p.scores + rh0 * p.nodes_total + p.lvl_off;
    float hmx[G];                                            // per head: max over its own candidates
#pragma unroll
    for (int h = 0; h < G; ++h) hmx[h] = -INFINITY;
    // Active parents are scored in groups: with b below the S = UNR * RPP
    // rows of a pass, one pass holds min(PPM, S / b) parents, so each of the
    // wave's round trips to memory carries S summary rows instead of b. Slot
    // (u2, sub) of a pass is row u2 * RPP + sub of the group; with b >= S the
    // group is one parent and the passes step through its children. Every
    // head's score of every child is written; for the split cut, the heads
    // that take a parent (all of them at the top and for the incomplete
    // parent, else those that kept it at the level above) also get its
    // children as candidates, at the parent's place in their candidate order.
    constexpr int S = UNR * RPP;
    // (at most two: each parent's values are named variables, since an array
    // selected by the lane's slot would be indexed dynamically and leave registers)
    constexpr int PPM = (G <= 4 && !TAN) ? 2 : 1;
    const int pp = p.b >= S ? 1 : imin(PPM, S >> p.lb);    // parents per group
    int64_t gpar0 = 0, gpar1 = 0;
    int gn = 0;
    auto score_group = [&]() {
        const int np = gn;
        gn = 0;
        // rows of the group past its first child's (b >= S: the parent's children)
        const int64_t ext = p.b >= S ? imin((gpar0 << p.lb) + p.b, nc) - (gpar0 << p.lb) : S;
        // the slot's parent within the group
        auto slot_parent = [&](int u2) { return p.b >= S ? 0 : ((u2 * RPP + sub) >> p.lb); };
        int32_t c_[UNR];                                 // the slot's node, or -1 where the slot is empty
        auto slot_rows = [&](int64_t cb) {
#pragma unroll
            for (int u2 = 0; u2 < UNR; ++u2) {
                const int slot = u2 * RPP + sub;
                const int pi = slot_parent(u2);
                const int64_t co = p.b >= S ? cb + slot : static_cast<int64_t>(slot & (p.b - 1));
                const int64_t par = (PPM > 1 && pi == 1 && np > 1) ? gpar1 : gpar0;
                const int64_t c = (par << p.lb) + co;
                c_[u2] = (pi < np && c < imin((par << p.lb) + p.b, nc)) ? static_cast<int32_t>(c) : -1;
            }
        };
        float x[UNR][DPL];
        float xo[UNR];                                   // tangent scoring: the rows' offsets
        auto load_pass = [&](int rr) {
#pragma unroll
            for (int u2 = 0; u2 < UNR; ++u2) {
                // an empty slot reads the group's first row; its results are dropped
                const int64_t c = c_[u2] >= 0 ? static_cast<int64_t>(c_[u2]) : (gpar0 << p.lb);
                load_row_il<DPL, LPR>(summ + (c * RT + rr) * D + part * 4, x[u2]);
                if constexpr (TAN) xo[u2] = offs[c * RT + rr];
            }
        };
        slot_rows(0);
        load_pass(0);
        // split: each parent's candidate base per head, read with the first summaries
        int32_t cbp0[G], cbp1[G];
        auto cand_base = [&](int64_t par, int32_t (&cbp)[G]) {
            const bool orph = !top && par == nc_up;
            const int64_t pr = (top || nc_up == 0) ? 0 : imin(par, nc_up - 1);
            const int32_t* rp = p.rank_up + rh0 * p.nodes_total + p.lvl_off_up + pr;
            const uint32_t* bp = p.bm_up + rh0 * p.bm_words_total + (pr >> 5);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const int32_t rk = rp[h * p.nodes_total];
                const uint32_t bw = bp[h * p.bm_words_total];
                int32_t cb = -1;
                if (top) cb = static_cast<int32_t>(par << p.lb);
                else if (orph) cb = kc[h] << p.lb;
                else if ((bw >> (pr & 31)) & 1u) cb = rk << p.lb;
                cbp[h] = cb;
            }
        };
        if (split) {
            cand_base(gpar0, cbp0);
            if (PPM > 1 && pp > 1) {
                cand_base(np > 1 ? gpar1 : gpar0, cbp1);
            } else {
#pragma unroll
                for (int h = 0; h < G; ++h) cbp1[h] = cbp0[h];
            }
        }
        for (int64_t cb = 0;;) {
            // a node's score: q . summary * scale, or the largest of its R tangents
            float best[UNR][G];
            for (int rr = 0;;) {
#pragma unroll
                for (int u2 = 0; u2 < UNR; ++u2) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        float t = 0.f;
#pragma unroll
                        for (int e = 0; e < DPL; ++e) t = fmaf(qv[h][e], x[u2][e], t);
                        t = fast_group_sum<LPR>(t) * p.scale;
                        if constexpr (TAN) best[u2][h] = rr == 0 ? t + xo[u2] : fmaxf(best[u2][h], t + xo[u2]);
                        else best[u2][h] = t;
                    }
                }
                if (++rr >= RT) break;
                load_pass(rr);
            }
#pragma unroll
            for (int u2 = 0; u2 < UNR; ++u2) {
                const int64_t c = c_[u2];
                const int pi = slot_parent(u2);
                if (c >= 0) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float sv = best[u2][h];
                        if (part == h) sc0[static_cast<int64_t>(h) * p.nodes_total + c] = sv;
                        if (split) {
                            const int32_t cbh = (PPM > 1 && pi == 1) ? cbp1[h] : cbp0[h];
                            if (cbh >= 0) {
                                hmx[h] = fmaxf(hmx[h], sv);
                                if (part == h) {
                                    const int64_t at = (rh0 + h) * p.cand_stride + cbh + (c & (p.b - 1));
                                    p.cand_sc[at] = sv;
                                    p.cand_nd[at] = static_cast<int32_t>(c);
                                }
                            }
                        }
                    }
                }
            }
            cb += S;
            if (cb >= ext) break;
            slot_rows(cb);
            load_pass(0);
        }
    };
    // The wave's active parents one after another: at the top every b-block
    // of nodes; below, the kept parents from the union bits, then the
    // incomplete parent.
    int64_t j = run;                       // the next active parent this wave takes
    int64_t base = 0;                      // active parents before the current pass of union words
    int64_t w0 = 0;                        // the pass's first word
    int64_t pass_n = 0;                    // active parents in the pass
    uint64_t incl = 0;                     // the lane's inclusive count of them
    bool orph_left = !top && orphans > 0;
    const int64_t blocks = top ? (nc + p.b - 1) >> p.lb : 0;
    auto count_pass = [&]() {
        uint32_t cnt = 0;
#pragma unroll
        for (int k = 0; k < kWpl; ++k) cnt += __popc(u[k]);
        incl = wave_scan_u64(cnt);
        pass_n = static_cast<int64_t>(lane63_u64(incl));
    };
    if (!top && nwords > 0) count_pass();
    auto next_parent = [&]() -> int64_t {
        if (top) {
            if (j >= blocks) return -1;
            const int64_t r = j;
            j += W;
            return r;
        }
        while (w0 < nwords) {
            if (j < base + pass_n) {
                // the lane whose words hold active parent j, then the word and the bit
                const uint64_t rel = static_cast<uint64_t>(j - base);
                const int L = __popcll(__ballot(incl <= rel));
                const uint64_t before = L ? static_cast<uint64_t>(
                    static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(incl)), L - 1))) : 0;
                uint32_t r = static_cast<uint32_t>(rel - before);
                int64_t par = -1;
#pragma unroll
                for (int k = 0; k < kWpl; ++k) {
                    uint32_t xw = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u[k]), L));
                    const uint32_t c = static_cast<uint32_t>(__popc(xw));
                    if (par < 0) {
                        if (r < c) {
                            for (uint32_t i = 0; i < r; ++i) xw &= xw - 1u;
                            par = ((w0 + static_cast<int64_t>(L) * kWpl + k) << 5) + __builtin_ctz(xw);
                        } else {
                            r -= c;
                        }
                    }
                }
                j += W;
                return par;
            }
            base += pass_n;
            w0 += static_cast<int64_t>(kWave) * kWpl;
            pass_n = 0;
            if (w0 < nwords) {
                load_union(w0);
                count_pass();
            }
        }
        // the incomplete parent is active parent `base`
        if (orph_left && j == base) {
            orph_left = false;
            return nc_up;
        }
        return -1;
    };
    for (;;) {
        int n = 0;
        for (; n < pp; ++n) {
            const int64_t par = next_parent();
            if (par < 0) break;
            if (n == 0) gpar0 = par;
            else gpar1 = par;
        }
        if (n == 0) break;
        gn = n;
        score_group();
        if (n < pp) break;
    }
    if (split) {
        float m = -INFINITY;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_max_f(hmx[h])), 63));
            if (lane == h) m = mh;
        }
        if (lane < G) p.pmax[(rh0 + lane) * p.pmax_stride + run] = m;
        // the runs of the pair clear its heads' bins and this level's bitmaps
        // between them, for the cut's kernels (nothing here reads them). Done
        // last: stores issued before the first loads would hold up the wait
        // for those loads, which counts stores too.
        const int64_t stride = W * blockDim.x, first = static_cast<int64_t>(run) * blockDim.x + threadIdx.x;
        for (int64_t i = first; i < G * kCutBins; i += stride) p.chist[rh0 * kCutBins + i] = 0ull;
        const int64_t words = (nc + 31) >> 5;
        for (int64_t i = first; i < G * words; i += stride)
            p.bm_cur[(rh0 + i / words) * p.bm_words_total + i % words] = 0u;
    }
}

// ----------------------------------------------------------------------------
// the cut: block primitives and the two phases shared by both cut kernels
// ----------------------------------------------------------------------------
constexpr int kCutThreads = 1024;
constexpr int kCutWaves = kCutThreads / kWave;
constexpr float kCutBinScale = 2048.0f / 28.0f;     // bins per unit of score (a 2^-40 mass is 0 beyond 27.8)
constexpr int kCutList = 256;                       // boundary-bin members resolved from an LDS list

struct BlockScratch {
    uint64_t hist[2][256];      // radix histograms (crowded boundary bins), alternating between rounds
    uint64_t red_u64[kCutWaves];
    float red_f[kCutWaves];
    uint64_t wcnt[kCutWaves];   // per-wave (tie << 32 | below) counts of the compaction
    uint64_t bcast_u64[2];
    uint32_t bcast_u32[2];
    uint32_t red_u32[kCutWaves];
    uint32_t list[kCutList];    // candidates of the boundary bin
    float list_s[kCutList];     // and their scores
    uint32_t list_n;
    int32_t wcount;
    uint64_t rk[2][kWave];      // one wave's (key, mass) pairs for mass_ranked_before
};

// For lanes 0..m-1 holding distinct sort keys pk (m <= 64, wave-uniform) and
// masses F (lanes m..63 hold pk = ~0 and F = 0): the sum of the masses of the
// members whose key is below the lane's own, i.e. the mass ranked before it in
// key order. Every lane stores its (key, mass) in the wave's scratch; each
// lane then reads the members back eight at a time (every lane reads the same
// address, a broadcast) and sums the masses of the smaller keys. The scratch
// belongs to one wave at a time.
template <class Scratch>
__device__ __forceinline__ uint64_t mass_ranked_before(uint64_t pk, uint64_t F, int m, Scratch& bs) {
    const int lane = threadIdx.x & 63;
    bs.rk[0][lane] = pk;
    bs.rk[1][lane] = F;
    __builtin_amdgcn_wave_barrier();
    uint64_t pre = 0;
    for (int j0 = 0; j0 < m; j0 += 8) {        // j0 + 8 <= 64: entries past m never count
        uint64_t pj[8], fj[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            pj[u] = bs.rk[0][j0 + u];
            fj[u] = bs.rk[1][j0 + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) pre += pj[u] < pk ? fj[u] : 0ull;
    }
    __builtin_amdgcn_wave_barrier();           // the scratch is rewritten by the next call
    return pre;
}

// The boundary bin's members resolved by one wave (m <= 64, member i on lane
// i, candidate ids lk[] and scores ls[]): each lane ranks its member in (key,
// candidate) order, the masses are laid out in rank order and prefix-summed,
// and a member is kept while the mass ranked before it is below rem. Leaves
// the largest kept key (the boundary key) in bs.bcast_u32[1] and the number
// of kept members with that key in bs.bcast_u64[1].
template <class Scratch>
__device__ __forceinline__ void wave_resolve(const uint32_t* lk, const float* ls, int m, float mx, uint64_t rem,
                                             Scratch& bs) {
    const int lane = threadIdx.x & 63;
    const bool valid = lane < m;
    const uint32_t k = valid ? lk[lane] : 0u;
    const float s = valid ? ls[lane] : 0.f;
    const uint32_t key = valid ? desc_key(s) : 0xffffffffu;
    const uint64_t F = valid ? mass_fx(s, mx) : 0;
    const uint64_t pk = valid ? ((static_cast<uint64_t>(key) << 32) | k) : ~0ull;   // distinct per member
    // the mass ranked before each member, summed over the members in registers
    const uint64_t pre = mass_ranked_before(pk, F, m, bs);
    const bool kept = valid && pre < rem;
    const uint32_t kap = static_cast<uint32_t>(
        __builtin_amdgcn_readlane(static_cast<int>(wave_scan_max_u32(kept ? key : 0u)), 63));
    const uint64_t ties = __popcll(__ballot(kept && key == kap));
    if (lane == 0) {
        bs.bcast_u32[1] = kap;
        bs.bcast_u64[1] = ties;
    }
}

// LDS histogram updates from a whole wave (every lane calls, `active` or
// not). Lanes that share an index with at least 7 others are combined first
// and updated by one lane: many candidates of a cut can fall in one bin, and
// LDS atomics on one address serialise. The remaining lanes update directly.
__device__ __forceinline__ void wave_add_u64(unsigned long long* base, int idx, uint64_t v, bool active) {
    const int lane = threadIdx.x & 63;
    unsigned long long pend = __ballot(active);
    for (int it = 0; it < 4 && pend; ++it) {
        const int leader = __ffsll(static_cast<long long>(pend)) - 1;
        const int li = __builtin_amdgcn_readlane(idx, leader);
        const unsigned long long grp = __ballot(active && idx == li) & pend;
        if (__popcll(grp) < 8) break;
        const uint64_t sum = lane63_u64(wave_scan_u64(((grp >> lane) & 1ull) ? v : 0ull));
        if (lane == leader) atomicAdd(base + li, static_cast<unsigned long long>(sum));
        pend &= ~grp;
    }
    if ((pend >> lane) & 1ull) atomicAdd(base + idx, static_cast<unsigned long long>(v));
}

// Block reductions: a DPP scan per wave (lane 63 holds the wave's result),
// one LDS slot per wave, one barrier to publish and one to free the slots.
// NW: waves in the block (blockDim.x / 64).
template <int NW = kCutWaves>
__device__ __forceinline__ float block_max_f(float v, BlockScratch& bs) {
    v = wave_scan_max_f(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) bs.red_f[w] = v;
    __syncthreads();
    float r = bs.red_f[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) r = fmaxf(r, bs.red_f[i]);
    __syncthreads();
    return r;
}

template <int NW = kCutWaves>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, BlockScratch& bs) {
    v = wave_scan_u64(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) bs.red_u64[w] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) r += bs.red_u64[i];
    __syncthreads();
    return r;
}

// Sum of a u64 and max of a u32 over the block, in one round of barriers.
template <int NW = kCutWaves>
__device__ __forceinline__ void block_sum_max(uint64_t& sum, uint32_t& mx, BlockScratch& bs) {
    const uint64_t s = wave_scan_u64(sum);
    const uint32_t m = wave_scan_max_u32(mx);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) {
        bs.red_u64[w] = s;
        bs.red_u32[w] = m;
    }
    __syncthreads();
    uint64_t rs = 0;
    uint32_t rm = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        rs += bs.red_u64[i];
        rm = max(rm, bs.red_u32[i]);
    }
    __syncthreads();
    sum = rs;
    mx = rm;
}

// Exclusive prefix sum over the block in thread order; *total receives the sum.
template <int NW = kCutWaves>
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, BlockScratch& bs, uint64_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t inc = wave_scan_u64(v);
    if (lane == 63) bs.red_u64[w] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) before += bs.red_u64[i];
        all += bs.red_u64[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Bin of a score by its distance below the maximum. It never decreases along
// the descending key order, so each bin holds a contiguous run of that order
// (and equal scores share a bin).
__device__ __forceinline__ int cut_bin(float s, float mx) {
    const float d = (mx - s) * kCutBinScale;
    return d < static_cast<float>(kCutBins - 1) ? static_cast<int>(d) : kCutBins - 1;
}

// Where a cut ends: every candidate whose key is below kappa is kept, plus the
// first need_ties (in candidate order) of those whose key equals kappa.
struct CutBoundary {
    bool take_all;
    uint32_t kappa;
    uint64_t need_ties;
};

// MSB-first radix select, 8 bits a round, over the entries e < cnt that
// entry(e, key, F) accepts: returns the key at which the mass of the smaller
// keys, plus its own, first reaches rem, and lowers rem by the mass of the
// smaller keys. hist[0] must be zero and published before the call. Rounds
// alternate between two histograms, so a round needs two barriers. The
// entries' keys usually share their top digits (they come from one narrow
// score bin): a first pass finds their smallest and largest key, and the
// rounds start at the digit where those differ (a digit all entries share
// would hold all the mass and nothing before it).
template <int NW, class Entry>
__device__ __forceinline__ uint32_t radix_kappa(Entry entry, int64_t cnt, uint64_t& rem, BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    uint32_t kmin_n = 0u, kmax = 0u;           // largest ~key and largest key of the entries with mass
    for (int64_t e = tid; e < cnt; e += nt) {
        uint32_t key;
        uint64_t F;
        if (!entry(e, key, F) || F == 0) continue;
        kmin_n = max(kmin_n, ~key);
        kmax = max(kmax, key);
    }
    kmin_n = wave_scan_max_u32(kmin_n);
    kmax = wave_scan_max_u32(kmax);
    if (lane == 63) {
        bs.red_u32[wave] = kmax;
        bs.red_u64[wave] = kmin_n;
    }
    __syncthreads();
    uint32_t a = 0u, b = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        a = max(a, static_cast<uint32_t>(bs.red_u64[i]));
        b = max(b, bs.red_u32[i]);
    }
    __syncthreads();
    const uint32_t kmin = ~a;
    const int common = (kmin == b) ? 32 : __clz(static_cast<int>(kmin ^ b));
    int known = (common / 8) * 8;
    uint32_t prefix = kmin & top_bits_mask(known);
    int cur = 0;
    for (; known < 32; known += 8) {
        const int shift = 24 - known;
        const uint32_t hmask = top_bits_mask(known);
        uint64_t* hist = bs.hist[cur];
        for (int64_t e = tid; e < cnt; e += nt) {
            uint32_t key;
            uint64_t F;
            if (!entry(e, key, F) || F == 0 || ((key ^ prefix) & hmask) != 0u) continue;
            atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(key >> shift) & 255u]),
                      static_cast<unsigned long long>(F));
        }
        for (int i = tid; i < 256; i += nt) bs.hist[cur ^ 1][i] = 0;   // the next round's histogram
        __syncthreads();
        if (wave == 0) {
            // lanes own 4 consecutive digits; scan in digit order
            uint64_t v[4], lsum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = hist[lane * 4 + j];
                lsum += v[j];
            }
            const uint64_t inc = wave_scan_u64(lsum);
            uint64_t c = inc - lsum;
            int found = -1;
            uint64_t before = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (found < 0 && v[j] != 0 && c + v[j] >= rem) {
                    found = lane * 4 + j;
                    before = c;
                }
                c += v[j];
            }
            const unsigned long long bal = __ballot(found >= 0);
            // the entries hold the remaining mass (>= rem), so some lane finds the digit
            const int first = bal ? __ffsll(static_cast<long long>(bal)) - 1 : 0;
            if (lane == first) {
                bs.bcast_u32[cur] = static_cast<uint32_t>(found >= 0 ? found : 0);
                bs.bcast_u64[cur] = found >= 0 ? before : 0;
            }
        }
        __syncthreads();
        rem -= bs.bcast_u64[cur];
        prefix |= bs.bcast_u32[cur] << shift;
        cur ^= 1;
    }
    return prefix;
}

// The boundary of the top-p cut over candidates 0..n-1 with scores score(k)
// and maximum mx, by radix select over every candidate (small sets). Masses exp(s - mx) are 2^-40 fixed point; the total and
// every partial sum are exact. An MSB-first radix select, 8 bits a round,
// finds the key at which the mass of the keys before it first reaches
// ceil(top_p * total). Rounds alternate between two histograms, so a round
// needs two barriers: after the histogram, and after the digit is published.
template <int NW = kCutWaves, class ScoreAt>
__device__ __forceinline__ CutBoundary cut_boundary_radix(ScoreAt score, int64_t n, float mx, float top_p,
                                                    BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    CutBoundary cb{(top_p >= 1.0f) || n == 0, 0u, 0u};
    if (cb.take_all) return cb;
    // the first kRadixCache candidates of each thread keep their key and mass in
    // registers for every round; any beyond them are recomputed per round
    constexpr int kRadixCache = 4;
    uint32_t ck[kRadixCache];
    uint64_t cF[kRadixCache];
    uint64_t E = 0;
    uint32_t kmax = 0;
#pragma unroll
    for (int j = 0; j < kRadixCache; ++j) {
        const int64_t k = tid + static_cast<int64_t>(j) * nt;
        ck[j] = 0u;
        cF[j] = 0;
        if (k < n) {
            const float s = score(k);
            ck[j] = desc_key(s);
            cF[j] = mass_fx(s, mx);
            E += cF[j];
            if (cF[j]) kmax = max(kmax, ck[j]);
        }
    }
    const int64_t cached = static_cast<int64_t>(kRadixCache) * nt;
    for (int64_t k = cached + tid; k < n; k += nt) {
        const float s = score(k);
        const uint64_t F = mass_fx(s, mx);
        E += F;
        if (F) kmax = max(kmax, desc_key(s));
    }
    for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;      // published by the barriers below
    block_sum_max<NW>(E, kmax, bs);
    const uint32_t kmin = desc_key(mx);
    uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(top_p) * static_cast<double>(E)));
    if (rem == 0) rem = 1;
    int known = (kmin == kmax) ? 32 : __clz(static_cast<int>(kmin ^ kmax));
    uint32_t prefix = kmin & top_bits_mask(known);
    int cur = 0;
    while (known < 32) {
        const int nb = min(8, 32 - known);
        const int shift = 32 - known - nb;
        const uint32_t hmask = top_bits_mask(known);
        uint64_t* hist = bs.hist[cur];
        // the first rounds put most candidates in one digit: wave_add_u64 combines them per wave
#pragma unroll
        for (int j = 0; j < kRadixCache; ++j) {                  // whole waves update
            const uint64_t F = ((ck[j] ^ prefix) & hmask) == 0u ? cF[j] : 0;
            wave_add_u64(reinterpret_cast<unsigned long long*>(hist), static_cast<int>((ck[j] >> shift) & ((1u << nb) - 1u)),
                         F, F != 0);
        }
        for (int64_t kb = cached; kb < n; kb += nt) {             // uniform trip count
            const int64_t k = kb + tid;
            uint32_t key = 0;
            uint64_t F = 0;
            if (k < n) {
                const float s = score(k);
                key = desc_key(s);
                if (((key ^ prefix) & hmask) == 0u) F = mass_fx(s, mx);
            }
            wave_add_u64(reinterpret_cast<unsigned long long*>(hist), static_cast<int>((key >> shift) & ((1u << nb) - 1u)),
                         F, F != 0);
        }
        for (int i = tid; i < 256; i += nt) bs.hist[cur ^ 1][i] = 0;   // the next round's histogram
        __syncthreads();
        if (wave == 0) {
            // lanes own 4 consecutive digits; scan in digit order
            uint64_t v[4], lsum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = hist[lane * 4 + j];
                lsum += v[j];
            }
            const uint64_t inc = wave_scan_u64(lsum);
            uint64_t c = inc - lsum;
            int found = -1;
            uint64_t before = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (found < 0 && v[j] != 0 && c + v[j] >= rem) {
                    found = lane * 4 + j;
                    before = c;
                }
                c += v[j];
            }
            const unsigned long long bal = __ballot(found >= 0);
            // the bins hold the remaining mass (>= rem), so some lane finds the digit
            const int first = bal ? __ffsll(static_cast<long long>(bal)) - 1 : 0;
            if (lane == first) {
                bs.bcast_u32[cur] = static_cast<uint32_t>(found >= 0 ? found : 0);
                bs.bcast_u64[cur] = found >= 0 ? before : 0;
            }
        }
        __syncthreads();
        rem -= bs.bcast_u64[cur];
        prefix |= bs.bcast_u32[cur] << shift;
        known += nb;
        cur ^= 1;
    }
    cb.kappa = prefix;
    const uint64_t Fk = mass_fx(desc_key_to_float(prefix), mx);
    cb.need_ties = Fk ? (rem + Fk - 1) / Fk : 0;
    return cb;
}

// The boundary of the top-p cut over candidates 0..n-1 with scores score(k)
// and maximum mx (blockDim == kCutThreads). Masses exp(s - mx) are 2^-40
// fixed point, so the total and every partial sum are exact integers.
//  1. One pass adds each mass into the bin of its score (bins[], kCutBins
//     entries of LDS) and into the total; rem = ceil(top_p * total).
//  2. A block scan over the bins finds the bin where the running mass first
//     reaches rem: every bin before it is kept whole.
//  3. A second pass lists the members of that bin. One wave ranks up to 64 of
//     them in (key, index) order and keeps them while the mass ranked before
//     is below what rem still needs; a longer list goes through a radix select.
// The result is the same key and tie count as a radix select over all the
// candidates: bins only narrow the search.
// kBinsClear: the caller cleared bins[] and published it with a barrier.
template <int NW = kCutWaves, bool kBinsClear = false, class ScoreAt>
__device__ __forceinline__ CutBoundary cut_boundary(ScoreAt score, int64_t n, float mx, float top_p,
                                                    uint64_t* bins, BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    CutBoundary cb{(top_p >= 1.0f) || n == 0, 0u, 0u};
    if (cb.take_all) return cb;
    if constexpr (!kBinsClear) {
        for (int i = tid; i < kCutBins; i += nt) bins[i] = 0;
        __syncthreads();
    }
    uint64_t E = 0;
    for (int64_t kb = 0; kb < n; kb += nt) {                  // uniform trip count: whole waves update
        const int64_t k = kb + tid;
        float s = 0.f;
        uint64_t F = 0;
        if (k < n) {
            s = score(k);
            F = mass_fx(s, mx);
        }
        E += F;
        wave_add_u64(reinterpret_cast<unsigned long long*>(bins), cut_bin(s, mx), F, F != 0);
    }
    if (tid == 0) bs.list_n = 0;
    for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;
    E = block_sum_u64<NW>(E, bs);                   // its barriers also publish the bins
    uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(top_p) * static_cast<double>(E)));
    if (rem == 0) rem = 1;

    constexpr int BPT = kCutBins / (NW * kWave);    // bins per thread, in bin order
    uint64_t v[BPT], lsum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        v[j] = bins[tid * BPT + j];
        lsum += v[j];
    }
    uint64_t tot;
    uint64_t c = block_excl_scan_u64<NW>(lsum, bs, &tot);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        if (v[j] != 0 && c < rem && c + v[j] >= rem) {  // exactly one bin crosses rem (tot >= rem)
            bs.bcast_u32[0] = static_cast<uint32_t>(tid * BPT + j);
            bs.bcast_u64[0] = c;
        }
        c += v[j];
    }
    __syncthreads();
    const int bstar = static_cast<int>(bs.bcast_u32[0]);
    rem -= bs.bcast_u64[0];

    // members of the boundary bin (those with a nonzero mass), appended a wave at a time
    for (int64_t kb = 0; kb < n; kb += nt) {
        const int64_t k = kb + tid;
        bool mem = false;
        if (k < n) {
            const float s = score(k);
            mem = cut_bin(s, mx) == bstar && mass_fx(s, mx) != 0;
        }
        const unsigned long long bal = __ballot(mem);
        if (bal) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&bs.list_n, static_cast<uint32_t>(__popcll(bal)));
            base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
            const uint32_t pos = base + static_cast<uint32_t>(__popcll(bal & ((1ull << lane) - 1ull)));
            if (mem && pos < kCutList) {
                bs.list[pos] = static_cast<uint32_t>(k);
                bs.list_s[pos] = score(k);
            }
        }
    }
    __syncthreads();
    const uint32_t m = bs.list_n;

    if (m <= kWave) {
        if (wave == 0) wave_resolve(bs.list, bs.list_s, static_cast<int>(m), mx, rem, bs);
        __syncthreads();
        cb.kappa = bs.bcast_u32[1];
        cb.need_ties = bs.bcast_u64[1];
        return cb;
    }
    uint32_t kap;
    if (m <= kCutList) {
        kap = radix_kappa<NW>([&](int64_t e, uint32_t& key, uint64_t& F) {
            const float s = bs.list_s[e];
            key = desc_key(s);
            F = mass_fx(s, mx);
            return true;
        }, m, rem, bs);
    } else {
        kap = radix_kappa<NW>([&](int64_t k, uint32_t& key, uint64_t& F) {
            const float s = score(k);
            if (cut_bin(s, mx) != bstar) return false;
            key = desc_key(s);
            F = mass_fx(s, mx);
            return true;
        }, n, rem, bs);
    }
    cb.kappa = kap;
    const uint64_t Fk = mass_fx(desc_key_to_float(kap), mx);
    cb.need_ties = Fk ? (rem + Fk - 1) / Fk : 0;
    return cb;
}

// The same cut for n <= 64 candidates, run by one wave with candidate k on
// lane k and no block barriers: each lane ranks its candidate in (key asc,
// index asc) order against the others' keys, the masses are laid out in rank
// order and prefix-summed, and a candidate is kept when the mass ranked before
// it is still below ceil(top_p * total). This keeps exactly the candidates the
// boundary search keeps: all keys below the boundary key, and of the boundary
// key's ties the first in index order. emit(pos, k) for every kept one, pos
// ascending in k. Returns the number kept (on every lane).
template <class ScoreAt, class Emit, class Scratch>
__device__ __forceinline__ int wave_cut_small(ScoreAt score, int n, float top_p, Scratch& bs, Emit emit) {
    const int lane = threadIdx.x & 63;
    const bool valid = lane < n;
    const float s = valid ? score(lane) : -INFINITY;
    const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_max_f(s)), 63));
    const uint64_t F = valid ? mass_fx(s, mx) : 0;
    const uint32_t key = desc_key(s);
    const uint64_t E = lane63_u64(wave_scan_u64(F));
    const bool take_all = (top_p >= 1.0f) || n == 0;
    uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(top_p) * static_cast<double>(E)));
    if (rem == 0) rem = 1;
    const uint64_t pk = valid ? ((static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(lane)) : ~0ull;
    const uint64_t pre = mass_ranked_before(pk, F, n, bs);
    const bool kept = valid && (take_all || pre < rem);
    const unsigned long long bal = __ballot(kept);
    if (kept) emit(static_cast<int64_t>(__popcll(bal & ((1ull << lane) - 1ull))), static_cast<int64_t>(lane));
    return __popcll(bal);
}

// Stable compaction of the kept candidates, 64 at a time: each wave owns a
// contiguous range of 64-candidate blocks, and a count pass plus a scan over
// the waves gives each wave its first output position. emit(pos, k) for every
// kept k, pos its rank among the kept (ascending k). mark(k, bits) once per
// aligned run of (1 << run_lg) <= 32 candidates starting at k that keeps any,
// bit i set when k + i is kept (a run maps to consecutive node ids inside one
// bitmap word). Returns the number kept.
template <int NW = kCutWaves, class ScoreAt, class Emit, class Mark>
__device__ __forceinline__ int64_t cut_compact(ScoreAt score, int64_t n, const CutBoundary& cb, int run_lg,
                                               BlockScratch& bs, Emit emit, Mark mark) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t nblk = (n + 63) >> 6;
    const int64_t per = (nblk + NW - 1) / NW;
    const int64_t b0 = imin(static_cast<int64_t>(w) * per, nblk), b1 = imin(b0 + per, nblk);
    const unsigned long long below = (1ull << lane) - 1ull;
    auto classify = [&](int64_t k, bool& lt, bool& tie) {
        const bool valid = k < n;
        if (cb.take_all) {
            lt = valid;
            tie = false;
            return;
        }
        const uint32_t key = valid ? desc_key(score(k)) : 0u;
        lt = valid && key < cb.kappa;
        tie = valid && key == cb.kappa;
    };
    uint64_t c_lt = 0, c_tie = 0;
    for (int64_t blk = b0; blk < b1; ++blk) {
        bool lt, tie;
        classify((blk << 6) + lane, lt, tie);
        c_lt += __popcll(__ballot(lt));
        c_tie += __popcll(__ballot(tie));
    }
    if (lane == 0) bs.wcnt[w] = (c_tie << 32) | c_lt;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint64_t x = bs.wcnt[i];
        if (i < w) before += x;
        all += x;
    }
    uint64_t lt_b = before & 0xffffffffu, tie_b = before >> 32;
    const uint64_t need = cb.need_ties;
    const int run = 1 << run_lg;
    const unsigned long long run_mask = (1ull << run) - 1ull;
    for (int64_t blk = b0; blk < b1; ++blk) {
        const int64_t k = (blk << 6) + lane;
        bool lt, tie;
        classify(k, lt, tie);
        const unsigned long long blt = __ballot(lt), btie = __ballot(tie);
        const uint64_t my_lt = lt_b + __popcll(blt & below), my_tie = tie_b + __popcll(btie & below);
        const bool keep = lt || (tie && my_tie < need);
        if (keep) emit(static_cast<int64_t>(my_lt + (lt ? (my_tie < need ? my_tie : need) : my_tie)), k);
        const unsigned long long bkeep = __ballot(keep);
        if ((lane & (run - 1)) == 0) {
            const uint32_t bits = static_cast<uint32_t>((bkeep >> lane) & run_mask);
            if (bits) mark(k, bits);
        }
        lt_b += __popcll(blt);
        tie_b += __popcll(btie);
    }
    __syncthreads();                                // wcnt is free for the next cut
    const uint64_t tot_lt = all & 0xffffffffu, tot_tie = all >> 32;
    return static_cast<int64_t>(tot_lt + (tot_tie < need ? tot_tie : need));
}

// ----------------------------------------------------------------------------
// per-level cut kernel (levels scored by route_score_kernel)
// ----------------------------------------------------------------------------
struct CutParams {
    RowInfo ri;
    const float* scores;
    int64_t nodes_total, lvl_off, lvl_off_up;
    int32_t* kept;             // ws kept lists (levels >= 2)
    int32_t* kept_cnt;         // [rows, Hq, L]
    uint32_t* bitmap;          // ws kept bitmaps: (row*Hq + hq)*bm_words_total + bm_off
    int64_t bm_words_total, bm_off;
    int32_t* sel_blocks;
    int32_t* n_sel;
    int sel_cap;
    int32_t* level_stats;
    int32_t* level_sel;
    int64_t lsel_off, nodes_l;
    uint32_t* status;
    int64_t cap;
    int b, lb, li, L, Hq, T;
    float top_p;
    int64_t pairs;             // rows * Hq (the one-wave-per-pair kernel)
};

constexpr int kCutStage = 32768;      // candidate scores staged in LDS (128 KiB)
constexpr int kCutUpStage = 2048;     // kept parents staged in LDS with them
constexpr int kCutBmWords = 4096;     // kept bitmap built in LDS (levels up to 131072 nodes)

template <int kStage, int kUpStage, int kBmWords>
struct CutSharedT {
    static constexpr int stage = kStage, up_stage = kUpStage, bm_words = kBmWords;
    float sc[kStage];
    int32_t up[kUpStage];
    union {
        uint64_t bins[kCutBins];      // the cut's first pass
        uint32_t bm[kBmWords];        // then the kept bitmap
    };
    BlockScratch bs;
};
using CutShared = CutSharedT<kCutStage, kCutUpStage, kCutBmWords>;

// The candidates of one (row, head) at one level, in ascending node order:
// k < nkids are the children of the kept parents up[0..kc), then the orphans.
struct CutCands {
    const float* sc;           // this level's scores of the (row, head)
    const int32_t* up;         // kept parents (ascending)
    int64_t nkids, nc_up, ncand;
    int lb;
    __device__ __forceinline__ int64_t node(int64_t k) const {
        return k < nkids ? ((static_cast<int64_t>(up[k >> lb]) << lb) | (k & ((int64_t(1) << lb) - 1)))
                         : (nc_up << lb) + (k - nkids);
    }
};

// kStaged: the candidates' scores and parents sit in LDS (read from HBM
// once); otherwise each pass re-reads them from global memory. The two
// variants are separate instantiations, so each only addresses one space.
template <bool kStaged, int NW, class Sh>
__device__ __forceinline__ void cut_level(const CutParams& p, Sh& sh, CutCands cc, int64_t rh,
                                          int64_t nc) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const bool leaf = (p.li == 0);
    const int64_t ncand = cc.ncand;
    auto score = [&](int64_t k) -> float {
        if constexpr (kStaged) return sh.sc[k];
        else return cc.sc[cc.node(k)];
    };

    // ---- stage the parents, then the scores; max ----
    float mx = -INFINITY;
    if constexpr (kStaged) {
        const int64_t kc = cc.nkids >> cc.lb;
        for (int64_t i = tid; i < kc; i += nt) sh.up[i] = cc.up[i];
        __syncthreads();
        cc.up = sh.up;
        // every candidate of the thread in flight at once: at most stage / threads
        constexpr int U = Sh::stage / (NW * kWave);
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = tid + static_cast<int64_t>(u) * nt;
            v[u] = k < ncand ? cc.sc[cc.node(k)] : -INFINITY;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = tid + static_cast<int64_t>(u) * nt;
            if (k < ncand) sh.sc[k] = v[u];
            mx = fmaxf(mx, v[u]);
        }
    } else {
        // kStageUnroll candidates per thread in flight: their parent ids
        // first, then their scores
        constexpr int kStageUnroll = 8;
        for (int64_t kb = tid; kb < ncand; kb += static_cast<int64_t>(kStageUnroll) * nt) {
            int64_t node[kStageUnroll];
            float v[kStageUnroll];
#pragma unroll
            for (int u = 0; u < kStageUnroll; ++u) {
                const int64_t k = kb + static_cast<int64_t>(u) * nt;
                node[u] = k < ncand ? cc.node(k) : -1;
            }
#pragma unroll
            for (int u = 0; u < kStageUnroll; ++u) v[u] = node[u] >= 0 ? cc.sc[node[u]] : -INFINITY;
#pragma unroll
            for (int u = 0; u < kStageUnroll; ++u) mx = fmaxf(mx, v[u]);
        }
    }

    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    // kept bitmap of this head at this level: the level below ORs the group's
    // bitmaps to find the parents to score; the attention reads level 1
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int64_t words = (nc + 31) >> 5;
    const bool lds_bm = words <= Sh::bm_words;
    auto emit = [&](int64_t pos, int64_t k) {
        const int32_t node = static_cast<int32_t>(cc.node(k));
        if (kept_out) kept_out[pos] = node;
        if (sel_out && pos < p.sel_cap) sel_out[pos] = node;
        if (lsel_out) lsel_out[pos] = node;
    };
    auto mark = [&](int64_t k, uint32_t bits) {
        const int64_t node = cc.node(k);
        if (lds_bm) atomicOr(&sh.bm[node >> 5], bits << (node & 31));
        else __hip_atomic_fetch_or(bm + (node >> 5), bits << (node & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto clear_bm = [&]() {      // the bitmap shares LDS with the bins: clear it once they are done
        if (lds_bm) {
            for (int64_t w = tid; w < words; w += nt) sh.bm[w] = 0u;
        } else {
            for (int64_t w = tid; w < words; w += nt) bm[w] = 0u;
            __threadfence_block();
        }
    };
    int64_t m;
    if (ncand <= kWave) {
        clear_bm();
        __syncthreads();                                   // also publishes the staged scores
        if ((tid >> 6) == 0) {
            const int mw = wave_cut_small(score, static_cast<int>(ncand), p.top_p, sh.bs,
                                          [&](int64_t pos, int64_t k) { emit(pos, k); mark(k, 1u); });
            if (tid == 0) sh.bs.wcount = mw;
        }
        __syncthreads();
        m = sh.bs.wcount;
    } else {
        mx = block_max_f<NW>(mx, sh.bs);                  // its barriers also publish the staged scores
        const CutBoundary cb = cut_boundary<NW>(score, ncand, mx, p.top_p, sh.bins, sh.bs);
        clear_bm();                                        // published by the compaction's first barrier
        m = cut_compact<NW>(score, ncand, cb, cc.lb < 5 ? cc.lb : 5, sh.bs, emit, mark);
    }
    if (lds_bm) {
        __syncthreads();
        for (int64_t w = tid; w < words; w += nt) bm[w] = sh.bm[w];
    }
    if (tid == 0) {
        p.kept_cnt[rh * p.L + p.li] = static_cast<int32_t>(m);
        if (leaf) {
            p.n_sel[rh] = static_cast<int32_t>(m);
            if (m > p.sel_cap) atomicOr(p.status, ZHA_DEV_SEL_OVERFLOW);
        }
        if (p.level_stats) {
            p.level_stats[(rh * p.L + p.li) * 2 + 0] = static_cast<int32_t>(ncand);
            p.level_stats[(rh * p.L + p.li) * 2 + 1] = static_cast<int32_t>(m);
        }
    }
}

template <int NW, class Sh>
__global__ __launch_bounds__(NW * kWave) void route_cut_kernel(CutParams p) {
    __shared__ Sh sh;
    const int hq = blockIdx.x, row = blockIdx.y;
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    CutCands cc;
    cc.sc = p.scores + rh * p.nodes_total + p.lvl_off;
    cc.lb = p.lb;
    cc.up = nullptr;
    int64_t kc = 0;
    cc.nc_up = 0;
    if (p.li != p.L - 1) {
        cc.nc_up = static_cast<int64_t>(N) >> (p.lb * (p.li + 2));
        kc = p.kept_cnt[rh * p.L + p.li + 1];
        cc.up = p.kept + rh * p.nodes_total + p.lvl_off_up;
    }
    cc.nkids = kc << p.lb;
    cc.ncand = cc.nkids + (nc - (cc.nc_up << p.lb));
    if (cc.ncand <= Sh::stage && kc <= Sh::up_stage) cut_level<true, NW>(p, sh, cc, rh, nc);
    else cut_level<false, NW>(p, sh, cc, rh, nc);
}

// ----------------------------------------------------------------------------
// one wave per (row, head): a level's cut for many pairs at once
// When thousands of (row, head) pairs route together (the rows of a prefill
// chunk), a workgroup per pair spends most of its time starting up and
// synchronising. Here each wave cuts one pair's level on its own, with its
// candidates' scores in its own 8 KiB of LDS and no block barriers:
//  1. the candidates' maximum; their 2^-40 fixed-point masses, summed in total
//     and per bin of the score's distance below the maximum (kWaveBins bins);
//  2. a scan of the bins finds the bin where the running mass reaches
//     ceil(top_p * total); its members, if at most 64, are ranked exactly by
//     wave_resolve, else an MSB-first radix select over their keys pins the
//     boundary key and the ties it needs;
//  3. the kept ids in ascending order and the kept bitmap: when the pass that
//     gathers the boundary bin's members also lists every candidate of the
//     earlier bins (at most kWaveSure), from those two lists; otherwise a
//     stable ballot compaction over all candidates.
// The kept set is the one cut_boundary and cut_compact produce.
// ----------------------------------------------------------------------------
constexpr int kWaveCutThreads = 256;
constexpr int kWaveCutWaves = kWaveCutThreads / kWave;
constexpr int kWaveBins = 256;
constexpr float kWaveBinScale = 256.0f / 28.0f;
constexpr int kWaveStage = 2048;        // candidate scores staged per wave: levels of up to 2048 nodes
constexpr int kWaveBmWords = kWaveStage / 32 + 1;          // the level's kept bitmap, in LDS
constexpr int kWaveSure = 128;          // candidates above the boundary bin listed in LDS (more: a compaction pass)

struct WaveScratch {
    static constexpr bool staged = true;
    static constexpr int bm_words = kWaveBmWords;
    uint64_t bcast_u64[2];
    uint32_t bcast_u32[2];
    uint64_t bins[kWaveBins];  // mass per bin, then per radix digit
    uint32_t list[kWave];      // members of the boundary bin
    float list_s[kWave];
    uint32_t sure[kWaveSure];  // candidates in earlier bins (all kept), in candidate order
    uint32_t kmem[kWave];      // the kept members, in candidate order
    uint32_t bm[kWaveBmWords];
    float sc[kWaveStage];      // the candidates' scores, in candidate order
    uint64_t rk[2][kWave];     // (key, mass) pairs for mass_ranked_before
};

__device__ __forceinline__ int wave_bin(float s, float mx) {
    const float d = (mx - s) * kWaveBinScale;
    return d < static_cast<float>(kWaveBins - 1) ? static_cast<int>(d) : kWaveBins - 1;
}

__device__ __forceinline__ int64_t lane_read_u64(uint64_t v, int l) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The digit (lane-owned runs of 4 in order) at which the running mass of
// hist[0..256) first reaches rem; *before receives the mass of the earlier
// digits. hist holds at least rem in total.
__device__ __forceinline__ int wave_find_digit(const uint64_t* hist, uint64_t rem, uint64_t* before) {
    const int lane = threadIdx.x & 63;
    uint64_t v[4], lsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = hist[lane * 4 + j];
        lsum += v[j];
    }
    const uint64_t inc = wave_scan_u64(lsum);
    uint64_t c = inc - lsum;
    int found = -1;
    uint64_t bf = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (found < 0 && v[j] != 0 && c + v[j] >= rem) {
            found = lane * 4 + j;
            bf = c;
        }
        c += v[j];
    }
    const unsigned long long bal = __ballot(found >= 0);
    const int first = bal ? __ffsll(static_cast<long long>(bal)) - 1 : 0;
    *before = static_cast<uint64_t>(lane_read_u64(bf, first));
    return __builtin_amdgcn_readlane(found, first);
}

// WS::staged: the candidates' scores are staged in the wave's LDS (a level
// of at most kWaveStage nodes), so every pass after the load runs on LDS.
// Otherwise every pass re-reads them from global memory, kPassU blocks of 64
// in flight per lane; that variant keeps only the small scratch in LDS, so
// many more waves share a compute unit.
constexpr int kPassU = 8;

struct WaveScratchU {           // the unstaged variant's scratch
    static constexpr bool staged = false;
    static constexpr int bm_words = 576;     // levels of up to 18432 nodes keep the bitmap in LDS
    uint64_t bcast_u64[2];
    uint32_t bcast_u32[2];
    uint64_t bins[kWaveBins];
    uint32_t list[kWave];
    float list_s[kWave];
    uint32_t sure[kWaveSure];
    uint32_t kmem[kWave];
    uint32_t bm[bm_words];
    uint64_t rk[2][kWave];
};

// Entries of the ascending list a[0..cnt) below x (a binary search).
__device__ __forceinline__ int count_below(const uint32_t* a, int cnt, uint32_t x) {
    int lo = 0, hi = cnt;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

template <class WS>
__global__ __launch_bounds__(kWaveCutThreads) void route_wave_cut_kernel(CutParams p) {
    constexpr bool kStaged = WS::staged;
    __shared__ WS wsh[kWaveCutWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rh = static_cast<int64_t>(blockIdx.x) * kWaveCutWaves + wave;
    if (rh >= p.pairs) return;                       // the whole wave: nothing below syncs the block
    WS& ws = wsh[wave];
    const int row = static_cast<int>(rh / p.Hq);
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    CutCands cc;
    cc.sc = p.scores + rh * p.nodes_total + p.lvl_off;
    cc.lb = p.lb;
    cc.up = nullptr;
    cc.nc_up = 0;
    int64_t kc = 0;
    if (p.li != p.L - 1) {
        cc.nc_up = static_cast<int64_t>(N) >> (p.lb * (p.li + 2));
        kc = p.kept_cnt[rh * p.L + p.li + 1];
        cc.up = p.kept + rh * p.nodes_total + p.lvl_off_up;
    }
    cc.nkids = kc << p.lb;
    cc.ncand = cc.nkids + (nc - (cc.nc_up << p.lb));
    const int n = static_cast<int>(cc.ncand);        // staged: <= nodes of the level <= kWaveStage
    const bool leaf = (p.li == 0);
    // Candidate k's node id without a branch: every lane loads a kept parent's
    // id (its index clamped into the list), so the loads of a whole group of
    // blocks go out together; lanes past the children take the uncovered tail.
    // With no kept parents (the top level) the pair's count slot stands in as
    // a valid address whose value is never used.
    const int lbw = p.lb;
    const int32_t lmask = (1 << lbw) - 1;
    const int32_t nkids32 = static_cast<int32_t>(cc.nkids);
    const int32_t tail0 = static_cast<int32_t>(cc.nc_up << lbw) - nkids32;
    const int32_t* upp = kc > 0 ? cc.up : p.kept_cnt + rh * p.L;
    const int32_t plast = kc > 0 ? static_cast<int32_t>(kc) - 1 : 0;
    auto node_of = [&](int k) -> int32_t {
        const int32_t par = upp[min(k >> lbw, plast)];
        return k < nkids32 ? ((par << lbw) | (k & lmask)) : k + tail0;
    };

    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int64_t words = (nc + 31) >> 5;
    const bool lds_bm = words <= WS::bm_words;       // always, staged
    if (lds_bm) {
        for (int64_t w = lane; w < words; w += kWave) ws.bm[w] = 0u;
    } else {
        for (int64_t w = lane; w < words; w += kWave) bm[w] = 0u;
        __threadfence_block();
    }
    __builtin_amdgcn_wave_barrier();
    auto emit_node = [&](int64_t pos, int32_t node) {
        if (kept_out) kept_out[pos] = node;
        if (sel_out && pos < p.sel_cap) sel_out[pos] = node;
        if (lsel_out) lsel_out[pos] = node;
    };
    auto mark_node = [&](int32_t node, uint32_t bits) {
        if (lds_bm) atomicOr(&ws.bm[node >> 5], bits << (node & 31));
        else __hip_atomic_fetch_or(bm + (node >> 5), bits << (node & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    };

    int64_t m;
    if (n <= kWave) {
        m = wave_cut_small([&](int64_t k) -> float { return cc.sc[cc.node(k)]; }, n, p.top_p, ws,
                           [&](int64_t pos, int64_t k) {
                               const int32_t node = static_cast<int32_t>(cc.node(k));
                               emit_node(pos, node);
                               mark_node(node, 1u);
                           });
    } else {
        const int nblk = (n + kWave - 1) / kWave;
        // blocks r0 .. r0 + kPassU - 1 of the candidates (block r holds k = 64 r + lane);
        // lanes past the candidates get node 0 (a valid address) and are masked by the caller
        // (the parent index is clamped, so the loads of blocks past the end are valid too)
        auto load_parents = [&](int r0, int32_t (&par)[kPassU]) {
#pragma unroll
            for (int u = 0; u < kPassU; ++u) {
                const int k = lane + (r0 + u) * kWave;
                par[u] = upp[min(k >> lbw, plast)];
            }
        };
        auto nodes_from = [&](int r0, int32_t (&par)[kPassU], int32_t (&nd)[kPassU]) {
            // taken as used here, so no load is sunk into a branch of the select below
#pragma unroll
            for (int u = 0; u < kPassU; ++u) asm volatile("" : "+v"(par[u]));
#pragma unroll
            for (int u = 0; u < kPassU; ++u) {
                const int k = lane + (r0 + u) * kWave;
                const int32_t node = k < nkids32 ? ((par[u] << lbw) | (k & lmask)) : k + tail0;
                nd[u] = k < n ? node : 0;
            }
        };
        auto fetch_nodes = [&](int r0, int32_t (&nd)[kPassU]) {
            int32_t par[kPassU];
            load_parents(r0, par);
            nodes_from(r0, par, nd);
        };
        auto fetch_global = [&](int r0, float (&v)[kPassU], int32_t (&nd)[kPassU]) {
            fetch_nodes(r0, nd);
#pragma unroll
            for (int u = 0; u < kPassU; ++u) v[u] = cc.sc[nd[u]];
        };
        // body(r, score, node): whole waves, blocks in order; WithNodes: the
        // staged variant also looks up the node ids (the unstaged one has them).
        // Unstaged, the next group's parent ids are loaded while this group's
        // scores are in flight, so a group waits for one round trip, not two.
        auto pass_impl = [&](auto with_nodes, auto&& body) {
            int32_t par[kPassU];
            if constexpr (!kStaged) load_parents(0, par);
            for (int r0 = 0; r0 < nblk; r0 += kPassU) {
                float v[kPassU];
                int32_t nd[kPassU];
                if constexpr (kStaged) {
                    if constexpr (decltype(with_nodes)::value) fetch_nodes(r0, nd);
#pragma unroll
                    for (int u = 0; u < kPassU; ++u) {
                        const int k = lane + (r0 + u) * kWave;
                        v[u] = k < n ? ws.sc[k] : 0.f;
                    }
                } else {
                    nodes_from(r0, par, nd);
#pragma unroll
                    for (int u = 0; u < kPassU; ++u) v[u] = cc.sc[nd[u]];
                    load_parents(r0 + kPassU, par);
                }
#pragma unroll
                for (int u = 0; u < kPassU; ++u)     // block r0 always exists: its load stays out of a branch
                    if (u == 0 || r0 + u < nblk) body(r0 + u, v[u], nd[u]);
            }
        };
        auto pass = [&](auto&& body) {
            pass_impl(std::false_type{}, [&](int r, float sv, int32_t) { body(r, sv); });
        };
        auto pass_nodes = [&](auto&& body) { pass_impl(std::true_type{}, body); };
        // the maximum (staged: while the scores go to LDS)
        float mx = -INFINITY;
        if constexpr (kStaged) {
            for (int r0 = 0; r0 < nblk; r0 += kPassU) {
                float v[kPassU];
                int32_t nd[kPassU];
                fetch_global(r0, v, nd);
#pragma unroll
                for (int u = 0; u < kPassU; ++u) {
                    const int k = lane + (r0 + u) * kWave;
                    if (k < n) {
                        ws.sc[k] = v[u];
                        mx = fmaxf(mx, v[u]);
                    }
                }
            }
        } else {
            pass([&](int r, float sv) {
                if (lane + r * kWave < n) mx = fmaxf(mx, sv);
            });
        }
        mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_max_f(mx)), 63));
        __builtin_amdgcn_wave_barrier();
        const bool take_all = p.top_p >= 1.0f;
        uint32_t kappa = 0;
        uint64_t need = 0;
        bool listed = false;             // the kept set is in the two LDS lists: no compaction pass
        uint32_t lnm = 0, lns = 0;       // members of the boundary bin, candidates of earlier bins
        if (!take_all) {
            // 1. masses, in total and per bin
            for (int i = lane; i < kWaveBins; i += kWave) ws.bins[i] = 0;
            __builtin_amdgcn_wave_barrier();
            uint64_t E = 0;
            pass([&](int r, float sv) {
                const bool valid = lane + r * kWave < n;
                const uint64_t F = valid ? mass_fx(sv, mx) : 0;
                E += F;
                wave_add_u64(reinterpret_cast<unsigned long long*>(ws.bins), valid ? wave_bin(sv, mx) : 0, F, F != 0);
            });
            E = lane63_u64(wave_scan_u64(E));
            uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(p.top_p) * static_cast<double>(E)));
            if (rem == 0) rem = 1;
            __builtin_amdgcn_wave_barrier();
            // 2. the boundary bin and its members
            uint64_t before;
            const int bstar = wave_find_digit(ws.bins, rem, &before);
            rem -= before;
            // Members may include candidates of zero mass (only the last bins
            // hold any): ranked after every member of nonzero mass above them,
            // they leave the boundary key and its ties as they are, and one
            // ranked before the boundary is kept, as the compaction keeps it.
            // Candidates of earlier bins rank above every member: all kept.
            uint32_t nm = 0, ns = 0;
            pass([&](int r, float sv) {
                const int k = lane + r * kWave;
                const int bin = wave_bin(sv, mx);
                const bool mem = k < n && bin == bstar;
                const bool sure = k < n && bin < bstar;
                const unsigned long long bal = __ballot(mem), bsu = __ballot(sure);
                const uint32_t pos = nm + static_cast<uint32_t>(__popcll(bal & ((1ull << lane) - 1ull)));
                const uint32_t spos = ns + static_cast<uint32_t>(__popcll(bsu & ((1ull << lane) - 1ull)));
                if (mem && pos < kWave) {
                    ws.list[pos] = static_cast<uint32_t>(k);
                    ws.list_s[pos] = sv;
                }
                if (sure && spos < kWaveSure) ws.sure[spos] = static_cast<uint32_t>(k);
                nm += static_cast<uint32_t>(__popcll(bal));
                ns += static_cast<uint32_t>(__popcll(bsu));
            });
            __builtin_amdgcn_wave_barrier();
            listed = nm <= kWave && ns <= kWaveSure;
            lnm = nm;
            lns = ns;
            if (nm <= kWave) {
                wave_resolve(ws.list, ws.list_s, static_cast<int>(nm), mx, rem, ws);
                __builtin_amdgcn_wave_barrier();
                kappa = ws.bcast_u32[1];
                need = ws.bcast_u64[1];
            } else {
                // a crowded bin: radix select over its members' keys, 8 bits a round
                uint32_t prefix = 0;
                for (int known = 0; known < 32; known += 8) {
                    const int shift = 24 - known;
                    const uint32_t hmask = known ? ~0u << (32 - known) : 0u;
                    for (int i = lane; i < kWaveBins; i += kWave) ws.bins[i] = 0;
                    __builtin_amdgcn_wave_barrier();
                    pass([&](int r, float sv) {
                        const uint32_t key = desc_key(sv);
                        const bool in = lane + r * kWave < n && wave_bin(sv, mx) == bstar &&
                                        ((key ^ prefix) & hmask) == 0u;
                        const uint64_t F = in ? mass_fx(sv, mx) : 0;
                        wave_add_u64(reinterpret_cast<unsigned long long*>(ws.bins), static_cast<int>((key >> shift) & 255u),
                                     F, F != 0);
                    });
                    __builtin_amdgcn_wave_barrier();
                    uint64_t bd;
                    const int d = wave_find_digit(ws.bins, rem, &bd);
                    rem -= bd;
                    prefix |= static_cast<uint32_t>(d) << shift;
                    __builtin_amdgcn_wave_barrier();
                }
                kappa = prefix;
                const uint64_t Fk = mass_fx(desc_key_to_float(kappa), mx);
                need = Fk ? (rem + Fk - 1) / Fk : 0;
            }
        }
        if (listed) {
            // 3'. the kept members (key below the boundary key, or among the
            // first `need` ties in candidate order) merged with the list of the
            // earlier bins: an entry's place is its rank in its own list plus
            // the entries of the other list before it (candidate order is node
            // order, so the ids come out ascending as the compaction writes them)
            const unsigned long long below = (1ull << lane) - 1ull;
            const bool valid = lane < static_cast<int>(lnm);
            const uint32_t k = valid ? ws.list[lane] : 0u;
            const uint32_t key = desc_key(valid ? ws.list_s[lane] : 0.f);
            const unsigned long long btie = __ballot(valid && key == kappa);
            const bool keep = valid && (key < kappa || (key == kappa && static_cast<uint64_t>(__popcll(btie & below)) < need));
            const unsigned long long bkeep = __ballot(keep);
            const int km = __popcll(bkeep & below), nkm = __popcll(bkeep);
            if (keep) ws.kmem[km] = k;
            __builtin_amdgcn_wave_barrier();
            if (keep) {
                const int32_t node = node_of(static_cast<int>(k));
                emit_node(km + count_below(ws.sure, static_cast<int>(lns), k), node);
                mark_node(node, 1u);
            }
            for (int j = lane; j < static_cast<int>(lns); j += kWave) {
                const uint32_t ks = ws.sure[j];
                const int32_t node = node_of(static_cast<int>(ks));
                emit_node(j + count_below(ws.kmem, nkm, ks), node);
                mark_node(node, 1u);
            }
            m = static_cast<int64_t>(lns) + nkm;
        } else {
            // 3. stable compaction, 64 candidates (one block) at a time
            const int run_lg = p.lb < 5 ? p.lb : 5;
            const int run = 1 << run_lg;
            const unsigned long long run_mask = (1ull << run) - 1ull;
            const unsigned long long below = (1ull << lane) - 1ull;
            uint64_t lt_b = 0, tie_b = 0;
            pass_nodes([&](int r, float sv, int32_t node) {
                const int64_t k = lane + r * kWave;
                const bool valid = k < n;
                const uint32_t key = valid ? desc_key(sv) : 0u;
                const bool lt = valid && (take_all || key < kappa);
                const bool tie = valid && !take_all && key == kappa;
                const unsigned long long blt = __ballot(lt), btie = __ballot(tie);
                const uint64_t my_lt = lt_b + __popcll(blt & below), my_tie = tie_b + __popcll(btie & below);
                const bool keep = lt || (tie && my_tie < need);
                if (keep) emit_node(static_cast<int64_t>(my_lt + (lt ? (my_tie < need ? my_tie : need) : my_tie)), node);
                const unsigned long long bkeep = __ballot(keep);
                if ((lane & (run - 1)) == 0) {
                    const uint32_t bits = static_cast<uint32_t>((bkeep >> lane) & run_mask);
                    if (bits) mark_node(node, bits);
                }
                lt_b += __popcll(blt);
                tie_b += __popcll(btie);
            });
            m = static_cast<int64_t>(lt_b + (tie_b < need ? tie_b : need));
        }
    }
    if (lds_bm) {
        __builtin_amdgcn_wave_barrier();
        for (int64_t w = lane; w < words; w += kWave) bm[w] = ws.bm[w];
    }
    if (lane == 0) {
        p.kept_cnt[rh * p.L + p.li] = static_cast<int32_t>(m);
        if (leaf) {
            p.n_sel[rh] = static_cast<int32_t>(m);
            if (m > p.sel_cap) atomicOr(p.status, ZHA_DEV_SEL_OVERFLOW);
        }
        if (p.level_stats) {
            p.level_stats[(rh * p.L + p.li) * 2 + 0] = static_cast<int32_t>(n);
            p.level_stats[(rh * p.L + p.li) * 2 + 1] = static_cast<int32_t>(m);
        }
    }
}

// ----------------------------------------------------------------------------
// the split cut: a level's cut spread over many workgroups per (row, head)
// When few (row, head) pairs route at once, one workgroup per pair leaves most
// of the chip idle while the largest candidate sets (tens of thousands) are
// cut. The same cut then runs over slices of kSplitSlice candidates, in two
// kernels ordered by their boundary:
//  * route_split_hist_kernel: the level max from the scoring workgroups'
//    partial maxima; the slice's node ids and scores copied in candidate
//    order and again grouped by bin, with each bin's start; its masses added
//    into the (row, head)'s global bins.
//  * route_split_emit_kernel: every slice finds the boundary bin from the
//    global bins, gathers that bin's members from the slices' bin groups,
//    resolves the boundary exactly (as cut_boundary does), counts the kept
//    candidates of the earlier slices, and writes its own kept ids and bits.
// The scoring kernel clears the bins and the level's bitmap beforehand. The
// kept set is the one cut_boundary and cut_compact produce.
// ----------------------------------------------------------------------------
struct SplitParams {
    RowInfo ri;
    const float* scores;       // dense-by-node scores, (row, head) stride nodes_total
    int64_t nodes_total, lvl_off, lvl_off_up;
    int32_t* kept;             // ws kept lists (levels >= 2)
    int32_t* kept_cnt;         // [rows, Hq, L]
    uint32_t* bitmap;
    int64_t bm_words_total, bm_off;
    int32_t* sel_blocks;
    int32_t* n_sel;
    int sel_cap;
    int32_t* level_stats;
    int32_t* level_sel;
    int64_t lsel_off, nodes_l;
    uint32_t* status;
    int64_t cap;
    int b, lb, li, L, Hq, T;
    float top_p;
    const float* pmax;
    const int32_t* pruns;      // [rows, Hq]: the scoring runs of the head's pair (columns of pmax)
    int64_t pmax_stride;
    const float* cand_sc;      // [rows, Hq, cand_stride] scores in candidate order (from the scoring kernel)
    const int32_t* cand_nd;    // node ids in candidate order
    int32_t* rank;             // [rows, Hq, nodes_total] kept node -> its place in the kept list (levels >= 2)
    uint32_t* srt_k;           // per slice, the slice's candidates grouped by bin: candidate index
    float* srt_s;              //   and score
    int64_t cand_stride;
    uint32_t* cum;             // [rows, Hq, slice_stride, kCutBins + 1] per slice: candidates in earlier bins
    unsigned long long* chist; // [rows, Hq, kCutBins] masses per bin
    int64_t slice_stride;
};

// This thread's share of the maximum over a head's scoring maxima (columns
// [0, pruns[rh]) of its pmax row). When the row stride allows, every column
// is loaded at once, in the same round as the count (columns past it hold
// stale values and are masked), rather than after it.
template <int NT>
__device__ __forceinline__ float split_pmax(const SplitParams& p, int64_t rh, int tid) {
    constexpr int kSpec = 8;
    const float* col = p.pmax + rh * p.pmax_stride;
    const int n = p.pruns[rh];
    float mx = -INFINITY;
    if (p.pmax_stride <= static_cast<int64_t>(kSpec) * NT) {
        float v[kSpec];
#pragma unroll
        for (int j = 0; j < kSpec; ++j) {
            const int64_t i = tid + static_cast<int64_t>(j) * NT;
            v[j] = col[i < p.pmax_stride ? i : 0];
        }
#pragma unroll
        for (int j = 0; j < kSpec; ++j)
            if (tid + j * NT < n) mx = fmaxf(mx, v[j]);
        return mx;
    }
    for (int i = tid; i < n; i += NT) mx = fmaxf(mx, col[i]);
    return mx;
}

__device__ __forceinline__ CutCands split_cands(const SplitParams& p, int row, int64_t rh, int64_t* nc_out) {
    // one round of loads, every address valid whatever the level: the row's
    // length and position, and the head's kept count at the level above
    const bool top = (p.li == p.L - 1);
    const int N = clamp_visible(p.ri, row, p.cap);
    const int32_t kc_up = p.kept_cnt[rh * p.L + (top ? p.li : p.li + 1)];
    __asm__ volatile("" ::: "memory");         // issued here, not sunk into the branches below
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    CutCands cc;
    cc.sc = p.scores + rh * p.nodes_total + p.lvl_off;
    cc.lb = p.lb;
    cc.up = nullptr;
    cc.nc_up = 0;
    int64_t kc = 0;
    if (!top) {
        cc.nc_up = static_cast<int64_t>(N) >> (p.lb * (p.li + 2));
        kc = kc_up;
        cc.up = p.kept + rh * p.nodes_total + p.lvl_off_up;
    }
    cc.nkids = kc << p.lb;
    cc.ncand = cc.nkids + (nc - (cc.nc_up << p.lb));
    *nc_out = nc;
    return cc;
}

constexpr int kSplitThreads = 256;
constexpr int kSplitWaves = kSplitThreads / kWave;
constexpr int kSplitPer = kSplitSlice / kSplitThreads;       // candidates per thread
constexpr int kBinsPerThread = kCutBins / kSplitThreads;

// Slice workgroup: the level max; the slice's candidates grouped by bin (a
// counting sort in LDS) with each bin's start; its masses added into the
// (row, head)'s bins. The scoring kernel wrote the scores in candidate order.
__global__ __launch_bounds__(kSplitThreads) void route_split_hist_kernel(SplitParams p) {
    __shared__ unsigned long long mbin[kCutBins];
    __shared__ uint32_t cbin[kCutBins];
    __shared__ BlockScratch bs;
    const int sl = blockIdx.x, hq = blockIdx.y, row = blockIdx.z;
    const int tid = threadIdx.x;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    const int64_t k0 = static_cast<int64_t>(sl) << kSplitSliceLog2;
    const int64_t cbase = rh * p.cand_stride;
    // issued together: the candidate count, the scoring maxima, the slice's scores
    int64_t nc;
    const CutCands cc = split_cands(p, row, rh, &nc);
    float mx = split_pmax<kSplitThreads>(p, rh, tid);
    float v[kSplitPer];
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        const int64_t k = k0 + tid + u * kSplitThreads;
        v[u] = k < p.cand_stride ? p.cand_sc[cbase + k] : -INFINITY;
    }
    if (k0 >= cc.ncand) return;
    bool val[kSplitPer];
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) val[u] = k0 + tid + u * kSplitThreads < cc.ncand;
    for (int i = tid; i < kCutBins; i += kSplitThreads) {
        mbin[i] = 0ull;
        cbin[i] = 0u;
    }
    mx = block_max_f<kSplitWaves>(mx, bs);            // its barriers also publish the cleared bins
    if (p.top_p >= 1.0f) return;                      // everything is kept: no bins needed
    int bn[kSplitPer];
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        bn[u] = cut_bin(v[u], mx);
        if (!val[u]) continue;
        atomicAdd(&cbin[bn[u]], 1u);
        const uint64_t F = mass_fx(v[u], mx);
        if (F) atomicAdd(&mbin[bn[u]], static_cast<unsigned long long>(F));
    }
    __syncthreads();
    // bin start offsets within the slice: thread t owns bins [t*BPT, t*BPT + BPT)
    uint32_t c[kBinsPerThread], lsum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) {
        c[j] = cbin[tid * kBinsPerThread + j];
        lsum += c[j];
    }
    uint64_t tot;
    uint32_t run = static_cast<uint32_t>(block_excl_scan_u64<kSplitWaves>(lsum, bs, &tot));
    uint32_t* cum = p.cum + (rh * p.slice_stride + sl) * (kCutBins + 1);
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) {
        cum[tid * kBinsPerThread + j] = run;
        cbin[tid * kBinsPerThread + j] = run;            // becomes the bin's write cursor
        run += c[j];
    }
    if (tid == kSplitThreads - 1) cum[kCutBins] = run;
    __syncthreads();
    uint32_t* sk = p.srt_k + cbase + k0;
    float* ss = p.srt_s + cbase + k0;
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        if (!val[u]) continue;
        const uint32_t at = atomicAdd(&cbin[bn[u]], 1u);
        sk[at] = static_cast<uint32_t>(k0 + tid + u * kSplitThreads);
        ss[at] = v[u];
    }
    unsigned long long* gb = p.chist + rh * kCutBins;
    for (int i = tid; i < kCutBins; i += kSplitThreads) {
        const unsigned long long x = mbin[i];
        if (x) atomicAdd(gb + i, x);                  // device scope: slices of a (row, head) sit on any XCD
    }
}

struct SplitEmitShared {
    uint32_t s_lt[kSplitMaxSlices];                   // per slice: kept below the boundary key
    uint32_t s_tie[kSplitMaxSlices];                  // per slice: at the boundary key
    uint32_t s_mb[kSplitMaxSlices + 1];               // per slice: first member's place in the member order
    uint32_t s_mo[kSplitMaxSlices];                   // per slice: members' offset in the slice's bin order
    uint64_t wcnt[kSplitWaves];
    BlockScratch bs;
};

// Slice workgroup: the level's boundary, worked out again by every slice of
// the (row, head) from the bins and the boundary bin's members, then the
// slice's kept ids at their ranks. Slice 0 also writes the level's counts.
__global__ __launch_bounds__(kSplitThreads) void route_split_emit_kernel(SplitParams p) {
    __shared__ SplitEmitShared sh;
    BlockScratch& bs = sh.bs;
    constexpr int BPW = kSplitSlice / kSplitThreads;           // 64-candidate blocks per wave
    const int sl = blockIdx.x, hq = blockIdx.y, row = blockIdx.z;
    const int tid = threadIdx.x, nt = kSplitThreads, lane = tid & 63, w = tid >> 6;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    const int64_t k0 = static_cast<int64_t>(sl) << kSplitSliceLog2;
    const int64_t cbase = rh * p.cand_stride;
    // issued together: the candidate count and this wave's blocks of the slice,
    // [kw, kw + 64 * BPW) (entries past the count are never used)
    int64_t nc;
    const CutCands cc = split_cands(p, row, rh, &nc);
    const int64_t kw = k0 + static_cast<int64_t>(w) * 64 * BPW;
    float sv[BPW];
    int32_t nd[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int64_t k = kw + j * 64 + lane;
        sv[j] = k < p.cand_stride ? p.cand_sc[cbase + k] : 0.f;
        nd[j] = k < p.cand_stride ? p.cand_nd[cbase + k] : 0;
    }
    // and, in the same round, the head's mass bins and scoring maxima (read
    // whether or not the cut needs them)
    const unsigned long long* gb = p.chist + rh * kCutBins;
    uint64_t v[kBinsPerThread], lsum = 0;
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) v[j] = gb[tid * kBinsPerThread + j];
    float mx = split_pmax<kSplitThreads>(p, rh, tid);
    const int64_t ncand = cc.ncand;
    const int nsl = static_cast<int>((ncand + kSplitSlice - 1) >> kSplitSliceLog2);
    if (sl >= nsl && sl != 0) return;
    const bool take_all = (p.top_p >= 1.0f) || ncand == 0;
    uint32_t kappa = 0u;
    uint64_t need = 0;
    for (int i = tid; i < nsl; i += nt) {
        sh.s_lt[i] = 0u;
        sh.s_tie[i] = 0u;
    }
    if (!take_all) {
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) lsum += v[j];
        mx = block_max_f<kSplitWaves>(mx, bs);
        if (tid == 0) bs.list_n = 0;
        for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;
        // the bin where the running mass first reaches ceil(top_p * total)
        uint64_t E;
        uint64_t c = block_excl_scan_u64<kSplitWaves>(lsum, bs, &E);
        uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(p.top_p) * static_cast<double>(E)));
        if (rem == 0) rem = 1;
#pragma unroll
        for (int j = 0; j < kBinsPerThread; ++j) {
            if (v[j] != 0 && c < rem && c + v[j] >= rem) {
                bs.bcast_u32[0] = static_cast<uint32_t>(tid * kBinsPerThread + j);
                bs.bcast_u64[0] = c;
            }
            c += v[j];
        }
        __syncthreads();
        const int bstar = static_cast<int>(bs.bcast_u32[0]);
        rem -= bs.bcast_u64[0];
        // per slice: candidates in earlier bins (all kept) and the boundary bin's members
        const uint32_t* cum = p.cum + rh * p.slice_stride * (kCutBins + 1);
        constexpr int SPT = kSplitMaxSlices / kSplitThreads;   // slices per thread, contiguous
        uint32_t mc[SPT], msum = 0;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int s2 = tid * SPT + j;
            mc[j] = 0u;
            if (s2 < nsl) {
                const uint32_t a = cum[static_cast<int64_t>(s2) * (kCutBins + 1) + bstar];
                const uint32_t b = cum[static_cast<int64_t>(s2) * (kCutBins + 1) + bstar + 1];
                sh.s_lt[s2] = a;
                sh.s_mo[s2] = a;
                mc[j] = b - a;
            }
            msum += mc[j];
        }
        uint64_t mall;
        uint32_t mb = static_cast<uint32_t>(block_excl_scan_u64<kSplitWaves>(msum, bs, &mall));
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int s2 = tid * SPT + j;
            if (s2 < nsl) sh.s_mb[s2] = mb;
            mb += mc[j];
        }
        if (tid == 0) sh.s_mb[nsl] = static_cast<uint32_t>(mall);
        __syncthreads();
        const uint32_t m = static_cast<uint32_t>(mall);
        // member e -> (candidate, score): its slice by binary search over the member offsets
        auto member = [&](uint32_t e, uint32_t& k, float& s) {
            int lo = 0, hi = nsl - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.s_mb[mid] <= e) lo = mid;
                else hi = mid - 1;
            }
            const int64_t at = cbase + (static_cast<int64_t>(lo) << kSplitSliceLog2) + sh.s_mo[lo] + (e - sh.s_mb[lo]);
            k = p.srt_k[at];
            s = p.srt_s[at];
        };
        if (m <= kCutList) {
            for (uint32_t e = tid; e < m; e += nt) {
                uint32_t k;
                float s;
                member(e, k, s);
                bs.list[e] = k;
                bs.list_s[e] = s;
            }
            __syncthreads();
        }
        if (m <= kWave) {
            if (w == 0) wave_resolve(bs.list, bs.list_s, static_cast<int>(m), mx, rem, bs);
            __syncthreads();
            kappa = bs.bcast_u32[1];
            need = bs.bcast_u64[1];
        } else {
            if (m <= kCutList) {
                kappa = radix_kappa<kSplitWaves>([&](int64_t e, uint32_t& key, uint64_t& F) {
                    const float s = bs.list_s[e];
                    key = desc_key(s);
                    F = mass_fx(s, mx);
                    return true;
                }, m, rem, bs);
            } else {
                kappa = radix_kappa<kSplitWaves>([&](int64_t e, uint32_t& key, uint64_t& F) {
                    uint32_t k;
                    float s;
                    member(static_cast<uint32_t>(e), k, s);
                    key = desc_key(s);
                    F = mass_fx(s, mx);
                    return true;
                }, m, rem, bs);
            }
            const uint64_t Fk = mass_fx(desc_key_to_float(kappa), mx);
            need = Fk ? (rem + Fk - 1) / Fk : 0;
        }
        // members below the boundary key, and the ties, per slice
        for (uint32_t e = tid; e < m; e += nt) {
            uint32_t k;
            float s;
            if (m <= kCutList) {
                k = bs.list[e];
                s = bs.list_s[e];
            } else {
                member(e, k, s);
            }
            const uint32_t key = desc_key(s);
            if (key < kappa) atomicAdd(&sh.s_lt[k >> kSplitSliceLog2], 1u);
            else if (key == kappa) atomicAdd(&sh.s_tie[k >> kSplitSliceLog2], 1u);
        }
    } else {
        for (int i = tid; i < nsl; i += nt) {
            const int64_t a = static_cast<int64_t>(i) << kSplitSliceLog2;
            sh.s_lt[i] = static_cast<uint32_t>(imin(ncand - a, kSplitSlice));
        }
    }
    __syncthreads();
    // (ties << 32 | below) before this slice, and the totals
    uint64_t mine = 0;
    for (int i = tid; i < nsl; i += nt)
        if (i < sl) mine += (static_cast<uint64_t>(sh.s_tie[i]) << 32) | sh.s_lt[i];
    uint64_t mine_all = 0;
    for (int i = tid; i < nsl; i += nt) mine_all += (static_cast<uint64_t>(sh.s_tie[i]) << 32) | sh.s_lt[i];
    const uint64_t before_sl = block_sum_u64<kSplitWaves>(mine, bs);
    const uint64_t all = block_sum_u64<kSplitWaves>(mine_all, bs);
    const uint64_t tot_lt = all & 0xffffffffu, tot_tie = all >> 32;
    const int64_t m_kept = static_cast<int64_t>(tot_lt + (tot_tie < need ? tot_tie : need));
    const bool leaf = (p.li == 0);
    if (sl == 0 && tid == 0) {
        p.kept_cnt[rh * p.L + p.li] = static_cast<int32_t>(m_kept);
        if (leaf) {
            p.n_sel[rh] = static_cast<int32_t>(m_kept);
            if (m_kept > p.sel_cap) atomicOr(p.status, ZHA_DEV_SEL_OVERFLOW);
        }
        if (p.level_stats) {
            p.level_stats[(rh * p.L + p.li) * 2 + 0] = static_cast<int32_t>(ncand);
            p.level_stats[(rh * p.L + p.li) * 2 + 1] = static_cast<int32_t>(m_kept);
        }
    }
    if (sl >= nsl) return;
    // ---- the slice's kept ids ----
    auto classify = [&](int j, bool& lt, bool& tie) {
        const int64_t k = kw + j * 64 + lane;
        const bool valid = k < ncand;
        if (take_all) {
            lt = valid;
            tie = false;
            return;
        }
        const uint32_t key = desc_key(sv[j]);
        lt = valid && key < kappa;
        tie = valid && key == kappa;
    };
    // the blocks' below / tie masks, kept for the writing pass (wave-uniform)
    unsigned long long mlt[BPW], mtie[BPW];
    uint64_t c_lt = 0, c_tie = 0;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        bool lt, tie;
        classify(j, lt, tie);
        mlt[j] = __ballot(lt);
        mtie[j] = __ballot(tie);
        c_lt += __popcll(mlt[j]);
        c_tie += __popcll(mtie[j]);
    }
    if (lane == 0) sh.wcnt[w] = (c_tie << 32) | c_lt;
    __syncthreads();
    uint64_t before = before_sl;
#pragma unroll
    for (int i = 0; i < kSplitWaves; ++i)
        if (i < w) before += sh.wcnt[i];
    uint64_t lt_b = before & 0xffffffffu, tie_b = before >> 32;
    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* rank_out = leaf ? nullptr : p.rank + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int run = 1 << (p.lb < 5 ? p.lb : 5);
    const unsigned long long run_mask = (1ull << run) - 1ull;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const unsigned long long blt = mlt[j], btie = mtie[j];
        const bool lt = (blt >> lane) & 1ull, tie = (btie >> lane) & 1ull;
        const uint64_t my_lt = lt_b + __popcll(blt & below), my_tie = tie_b + __popcll(btie & below);
        const bool keep = lt || (tie && my_tie < need);
        if (keep) {
            const int64_t pos = static_cast<int64_t>(my_lt + (lt ? (my_tie < need ? my_tie : need) : my_tie));
            const int32_t node = nd[j];
            if (kept_out) {
                kept_out[pos] = node;
                rank_out[node] = static_cast<int32_t>(pos);
            }
            if (sel_out && pos < p.sel_cap) sel_out[pos] = node;
            if (lsel_out) lsel_out[pos] = node;
        }
        const unsigned long long bkeep = __ballot(keep);
        if ((lane & (run - 1)) == 0) {
            const uint32_t bits = static_cast<uint32_t>((bkeep >> lane) & run_mask);
            // a run's nodes are consecutive and share one word. With b >= 32 a run is
            // a whole, aligned word that no other run touches: a plain store. With
            // smaller b, runs of other slices may share the word.
            if (bits && run == 32) bm[nd[j] >> 5] = bits;
            else if (bits)
                __hip_atomic_fetch_or(bm + (nd[j] >> 5), bits << (nd[j] & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        lt_b += __popcll(blt);
        tie_b += __popcll(btie);
    }
}

// ----------------------------------------------------------------------------
// fused traversal of the upper levels
// One workgroup per (row, query head) walks every level from the top down to
// level li_lo in one launch (every fused level has at most kUpperNodes nodes
// per (sequence, kv head)). Per level: the candidate ids are built in LDS from
// the kept nodes of the level above, each candidate's summary row is scored
// against the head's query (8 waves, a row per LPR lanes, 4 passes of rows in
// flight per wave), and the same
// exact cut runs on the LDS-resident scores. The kept set stays in LDS for the
// next level and is written out (kept list, count, bitmap) for the levels
// below li_lo. With small levels above li_lo (at most 64 nodes each) and at
// most kUpperPre nodes in all, the scores of every complete node of the fused
// levels are computed first instead (see "scoring up front" below), the
// levels above li_lo are cut by wave 0 alone meanwhile, and level li_lo's
// candidates then take their scores from LDS.
// ----------------------------------------------------------------------------
constexpr int kUpperNodes = 8192;
constexpr int kUpperPre = 4096;        // fused levels' nodes scored up front
constexpr int kUpperThreads = 512;     // 8 waves: rows in flight for the scoring, cheap barriers for the cut
constexpr int kUpperWaves = kUpperThreads / kWave;

struct UpperParams {
    const float* q;            // [rows, Hq, D]
    RowInfo ri;
    const float* summaries;
    int64_t sum_off[ZHA_MAX_LEVELS];
    int64_t nodes[ZHA_MAX_LEVELS];
    int64_t sel_off[ZHA_MAX_LEVELS];
    int64_t bm_off[ZHA_MAX_LEVELS];
    int64_t nodes_total;
    int32_t* kept;             // ws kept lists
    int32_t* kept_cnt;         // [rows, Hq, L]
    uint32_t* bitmap;          // ws kept bitmaps
    int32_t* rank;             // ws kept node -> place in its head's kept list (split cut only, else null)
    int64_t bm_words_total;
    int32_t* level_stats;
    int32_t* level_sel;
    int64_t rows;
    int64_t cap;
    int b, lb, L, li_lo, Hq, Hkv, G, T;
    float top_p_l[ZHA_MAX_LEVELS];   // cut fraction per level
    float scale;
    int64_t bias_off[ZHA_MAX_LEVELS];  // tangent scoring: each level's offsets
    int R;                             // tangent rows per node (1 without tangent scoring)
    float* scores;                     // value summaries: the dense-by-node scores its levels also go to (else null)
};

struct UpperShared {
    float sc[kUpperNodes];
    int32_t cid[kUpperNodes];          // candidate node ids, ascending
    int32_t par[kUpperNodes];          // kept nodes of the level above, ascending
    uint32_t bm[kUpperNodes / 32 + 1];
    uint64_t bins[kCutBins];           // mass bins of the boundary search
    float nsc[kUpperPre];              // scores of every complete node of the fused levels, top level first
    int64_t npar;                      // kept nodes of the level above the lowest fused one (wave 0's cuts)
    BlockScratch bs;
};

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave));
    return v;
}

template <int D, bool TAN>
__global__ __launch_bounds__(kUpperThreads) void route_upper_kernel(UpperParams p) {
    __shared__ UpperShared sh;
    constexpr int NW = kUpperWaves;
    constexpr int DPL = 16;                    // dims per lane
    constexpr int LPR = D / DPL;               // lanes per summary row
    constexpr int RPP = kWave / LPR;           // rows per wave pass
    constexpr int UNR = 4;                     // passes issued together: 4 * RPP rows in flight per wave
    // Workgroups go to the eight XCDs in turn (linear id mod 8 = blockIdx.x
    // mod 8 when H_q is a multiple of 8): XCD c takes query heads
    // [c H_q/8, (c + 1) H_q/8), so the heads of a kv group, which read the
    // same summary rows, share one XCD's L2.
    const int hq = (p.Hq & 7) ? static_cast<int>(blockIdx.x)
                              : static_cast<int>(blockIdx.x & 7) * (p.Hq >> 3) + static_cast<int>(blockIdx.x >> 3);
    const int row = blockIdx.y;
    const int kv = hq / p.G, s = row / p.T;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = NW;
    const int sub = lane / LPR, part = lane % LPR;
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    float qv[DPL];
    load_row_il<DPL, LPR>(p.q + rh * D + part * 4, qv);
    const int RT = TAN ? p.R : 1;                  // tangent rows per node
    const int64_t pair_sk = static_cast<int64_t>(s) * p.Hkv + kv;

    // ---- scoring up front ----
    // When every level above the lowest fused one has at most a wave's worth
    // of nodes and all fused levels together fit kUpperPre, every complete
    // node of those levels is scored at once (level l's node n at
    // sh.nsc[off(l) + n], levels top first): wave 0 scores the small levels and
    // runs their one-wave cuts while the other waves score the lowest level,
    // whose cut then only picks its candidates' scores. A level of one node
    // is never scored (its lone candidate is kept unscored). Scores are
    // computed exactly as below, so the cuts are the same.
    int64_t hi_tot = 0;                        // nsc slots of the levels above li_lo
    bool pre = p.li_lo + 1 < p.L;
    for (int l = p.L - 1; l > p.li_lo; --l) {
        const int64_t n_l = static_cast<int64_t>(N) >> (p.lb * (l + 1));
        pre = pre && n_l <= kWave;
        hi_tot += n_l;
    }
    const int64_t n_lo = static_cast<int64_t>(N) >> (p.lb * (p.li_lo + 1));
    pre = pre && hi_tot + n_lo <= kUpperPre;
    // scores of nodes [0, n) of level l into sh.nsc[at + node], by wave wi of nw2
    auto score_level = [&](int l, int64_t at, int64_t n, int wi, int nw2) {
        const int64_t nb = pair_sk * p.nodes[l];
        const float* summ = p.summaries + p.sum_off[l] + nb * RT * D;
        const float* offs = TAN ? p.summaries + p.bias_off[l] + nb * RT : nullptr;
        for (int64_t kb = static_cast<int64_t>(wi) * RPP * UNR; kb < n; kb += static_cast<int64_t>(nw2) * RPP * UNR) {
            float best[UNR];
            for (int rr = 0; rr < RT; ++rr) {
                float x[UNR][DPL], xo[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t row = imin(kb + u * RPP + sub, n - 1) * RT + rr;   // a present row
                    load_row_il<DPL, LPR>(summ + row * D + part * 4, x[u]);
                    if constexpr (TAN) xo[u] = offs[row];
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    float t = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) t = fmaf(qv[e], x[u][e], t);
                    t = fast_group_sum<LPR>(t) * p.scale;
                    if constexpr (TAN) best[u] = rr == 0 ? t + xo[u] : fmaxf(best[u], t + xo[u]);
                    else best[u] = t;
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t k = kb + u * RPP + sub;
                if (k < n && part == 0) sh.nsc[at + k] = best[u];
            }
        }
    };

    int64_t npar = 0;                          // kept nodes of the level above
    int32_t par0 = -1;                         // their one id when a lone candidate was kept (not in LDS)
    int li_first = p.L - 1;                    // the first level the block loop below takes
    if (pre) {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        if (wv == 0) {
            {
                int64_t at = 0;
                for (int l = p.L - 1; l > p.li_lo; --l) {
                    const int64_t n_l = static_cast<int64_t>(N) >> (p.lb * (l + 1));
                    if (n_l > 1) score_level(l, at, n_l, 0, 1);
                    at += n_l;
                }
            }
            __builtin_amdgcn_wave_barrier();
            // the small levels' cuts, one wave each; their kept lists go to sh.par
            int64_t off = 0;
            for (int li = p.L - 1; li > p.li_lo; --li) {
                const bool top = (li == p.L - 1);
                const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (li + 1));
                const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (li + 2)));
                const int64_t nkids = npar << p.lb;
                const int ncand = static_cast<int>(nkids + (nc - (nc_up << p.lb)));   // <= nc <= 64
                int32_t* kept_out = p.kept + rh * p.nodes_total + p.sel_off[li];
                int32_t* lsel_out = p.level_sel ? p.level_sel + p.rows * p.Hq * p.sel_off[li] + rh * p.nodes[li] : nullptr;
                int32_t* rank_out = p.rank ? p.rank + rh * p.nodes_total + p.sel_off[li] : nullptr;
                // candidate k on lane k: its node and score
                int32_t node = 0;
                float t = -INFINITY;
                if (lane < ncand) {
                    node = static_cast<int32_t>(lane < nkids ? ((static_cast<int64_t>(sh.par[lane >> p.lb]) << p.lb) | (lane & (p.b - 1)))
                                                             : (nc_up << p.lb) + (lane - nkids));
                    t = sh.nsc[off + node];
                    if (p.scores && ncand > 1) p.scores[rh * p.nodes_total + p.sel_off[li] + node] = t;
                }
                bool kl = false;                   // this lane's candidate is kept
                int m;
                if (ncand == 1) {
                    // a lone candidate carries the whole mass and is kept unscored
                    if (lane == 0) {
                        kept_out[0] = node;
                        if (rank_out) rank_out[node] = 0;
                        if (lsel_out) lsel_out[0] = node;
                    }
                    m = 1;
                    kl = lane == 0;
                    __builtin_amdgcn_wave_barrier();
                    if (lane == 0) sh.par[0] = node;
                } else {
                    __builtin_amdgcn_wave_barrier();   // sh.par is read above and rewritten below
                    // wave_cut_small asks each lane for its own candidate (k == lane)
                    m = wave_cut_small([&](int64_t) { return t; }, ncand, p.top_p_l[li], sh.bs,
                                       [&](int64_t pos, int64_t) {
                        const int32_t nd = node;
                        kl = true;
                        sh.par[pos] = nd;
                        kept_out[pos] = nd;
                        if (rank_out) rank_out[nd] = static_cast<int32_t>(pos);
                        if (lsel_out) lsel_out[pos] = nd;
                    });
                    __builtin_amdgcn_wave_barrier();
                }
                // the level's kept bits (nc <= 64: two words), OR-reduced over the kept lanes
                const uint32_t b0 = wave_or_u32(kl && node < 32 ? 1u << (node & 31) : 0u);
                const uint32_t b1 = wave_or_u32(kl && node >= 32 ? 1u << (node & 31) : 0u);
                uint32_t* bmg = p.bitmap + rh * p.bm_words_total + p.bm_off[li];
                if (lane < ((nc + 31) >> 5)) bmg[lane] = lane == 0 ? b0 : b1;
                if (lane == 0) {
                    p.kept_cnt[rh * p.L + li] = m;
                    if (p.level_stats) {
                        p.level_stats[(rh * p.L + li) * 2 + 0] = ncand;
                        p.level_stats[(rh * p.L + li) * 2 + 1] = m;
                    }
                }
                npar = m;
                off += nc;
                __builtin_amdgcn_wave_barrier();
            }
            if (lane == 0) sh.npar = npar;
        } else {
            if (n_lo > 1) score_level(p.li_lo, hi_tot, n_lo, wv - 1, nw - 1);
        }
        __syncthreads();
        npar = sh.npar;
        li_first = p.li_lo;
    }
    for (int li = li_first; li >= p.li_lo; --li) {
        const bool top = (li == p.L - 1);
        const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (li + 1));
        const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (li + 2)));
        const int64_t nkids = npar << p.lb;
        const int64_t ncand = nkids + (nc - (nc_up << p.lb));   // <= nc <= nodes[li] <= kUpperNodes
        if (ncand == 1) {
            // A lone candidate carries the whole mass and is kept unscored, with
            // no block step. With b >= 2 a kept parent brings b candidates, so
            // the lone one is the level's first node past the complete parents'
            // children (at the top: node 0).
            const int32_t node = static_cast<int32_t>(nc_up << p.lb);
            uint32_t* bmg = p.bitmap + rh * p.bm_words_total + p.bm_off[li];
            const int64_t words = (nc + 31) >> 5;
            for (int64_t w = tid; w < words; w += nt) bmg[w] = (w == (node >> 5)) ? (1u << (node & 31)) : 0u;
            if (tid == 0) {
                p.kept[rh * p.nodes_total + p.sel_off[li]] = node;
                if (p.rank) p.rank[rh * p.nodes_total + p.sel_off[li] + node] = 0;
                if (p.level_sel) p.level_sel[p.rows * p.Hq * p.sel_off[li] + rh * p.nodes[li]] = node;
                p.kept_cnt[rh * p.L + li] = 1;
                if (p.level_stats) {
                    p.level_stats[(rh * p.L + li) * 2 + 0] = 1;
                    p.level_stats[(rh * p.L + li) * 2 + 1] = 1;
                }
            }
            npar = 1;
            par0 = node;
            continue;
        }
        // scored up front: each thread picks the scores of the candidates it
        // lists, and clears the cut's bins; the barriers of the block max
        // below publish all of it (no thread reads another's candidates before)
        float mx = -INFINITY;
        for (int64_t k = tid; k < ncand; k += nt) {
            const int64_t pk = k >> p.lb;
            const int32_t par = par0 >= 0 ? par0 : sh.par[pk];
            const int32_t c = static_cast<int32_t>(k < nkids ? ((static_cast<int64_t>(par) << p.lb) | (k & (p.b - 1)))
                                                            : (nc_up << p.lb) + (k - nkids));
            sh.cid[k] = c;
            if (pre) {
                const float t = sh.nsc[hi_tot + c];
                sh.sc[k] = t;
                mx = fmaxf(mx, t);
                if (p.scores) p.scores[rh * p.nodes_total + p.sel_off[li] + c] = t;
            }
        }
        par0 = -1;
        const int64_t words = (nc + 31) >> 5;
        for (int64_t w = tid; w < words; w += nt) sh.bm[w] = 0u;
        if (pre) {
            for (int i = tid; i < kCutBins; i += nt) sh.bins[i] = 0;
        } else {
            __syncthreads();                   // the scoring below reads every thread's candidates
        }
        // ---- score the candidates: a row per LPR lanes, RPP rows per wave pass ----
        const int64_t nbase = pair_sk * p.nodes[li];
        const float* summ = p.summaries + p.sum_off[li] + nbase * RT * D;
        const float* offs = TAN ? p.summaries + p.bias_off[li] + nbase * RT : nullptr;
        for (int64_t kb = static_cast<int64_t>(wave) * RPP * UNR; !pre && kb < ncand; kb += static_cast<int64_t>(nw) * RPP * UNR) {
            float best[UNR];
            for (int rr = 0; rr < RT; ++rr) {
                float x[UNR][DPL], xo[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int64_t k = imin(kb + u * RPP + sub, ncand - 1);   // a present row; extra results are dropped
                    const int64_t row = static_cast<int64_t>(sh.cid[k]) * RT + rr;
                    load_row_il<DPL, LPR>(summ + row * D + part * 4, x[u]);
                    if constexpr (TAN) xo[u] = offs[row];
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    float t = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) t = fmaf(qv[e], x[u][e], t);
                    t = fast_group_sum<LPR>(t) * p.scale;
                    if constexpr (TAN) best[u] = rr == 0 ? t + xo[u] : fmaxf(best[u], t + xo[u]);
                    else best[u] = t;
                }
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const float t = best[u];
                const int64_t k = kb + u * RPP + sub;
                if (k < ncand) {
                    mx = fmaxf(mx, t);
                    if (part == 0) {
                        sh.sc[k] = t;
                        if (p.scores) p.scores[rh * p.nodes_total + p.sel_off[li] + sh.cid[k]] = t;
                    }
                }
            }
        }
        // ---- the cut ----
        auto score = [&](int64_t k) -> float { return sh.sc[k]; };
        int32_t* kept_out = p.kept + rh * p.nodes_total + p.sel_off[li];
        int32_t* lsel_out = p.level_sel ? p.level_sel + p.rows * p.Hq * p.sel_off[li] + rh * p.nodes[li] : nullptr;
        int32_t* rank_out = p.rank ? p.rank + rh * p.nodes_total + p.sel_off[li] : nullptr;
        auto emit = [&](int64_t pos, int64_t k) {
            const int32_t node = sh.cid[k];
            sh.par[pos] = node;                 // parents of the next level (cid holds this level's ids)
            kept_out[pos] = node;
            if (rank_out) rank_out[node] = static_cast<int32_t>(pos);
            if (lsel_out) lsel_out[pos] = node;
        };
        auto mark = [&](int64_t k, uint32_t bits) {
            const int32_t node = sh.cid[k];
            atomicOr(&sh.bm[node >> 5], bits << (node & 31));
        };
        int64_t m;
        if (ncand <= kWave) {                  // one wave, no block steps
            __syncthreads();                   // publishes sc[]
            if (wave == 0) {
                const int mw = wave_cut_small(score, static_cast<int>(ncand), p.top_p_l[li], sh.bs,
                                              [&](int64_t pos, int64_t k) { emit(pos, k); mark(k, 1u); });
                if (lane == 0) sh.bs.wcount = mw;
            }
            __syncthreads();
            m = sh.bs.wcount;
        } else {
            mx = block_max_f<NW>(mx, sh.bs);   // its barriers also publish sc[] (and, scored up front, the cleared bins)
            const CutBoundary cb = pre ? cut_boundary<NW, true>(score, ncand, mx, p.top_p_l[li], sh.bins, sh.bs)
                                       : cut_boundary<NW, false>(score, ncand, mx, p.top_p_l[li], sh.bins, sh.bs);
            m = cut_compact<NW>(score, ncand, cb, p.lb < 5 ? p.lb : 5, sh.bs, emit, mark);
        }
        uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off[li];
        for (int64_t w = tid; w < words; w += nt) bm[w] = sh.bm[w];
        if (tid == 0) {
            p.kept_cnt[rh * p.L + li] = static_cast<int32_t>(m);
            if (p.level_stats) {
                p.level_stats[(rh * p.L + li) * 2 + 0] = static_cast<int32_t>(ncand);
                p.level_stats[(rh * p.L + li) * 2 + 1] = static_cast<int32_t>(m);
            }
        }
        npar = m;
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <int D, int G>
static void launch_score_t(dim3 grid, const ScoreParams& sp, hipStream_t st) {
    ProfScope ps("route_score", sp.li + 1, st);
    if (sp.offs)
        hipLaunchKernelGGL((route_score_kernel<D, G, true>), grid, dim3(kScoreThreads), 0, st, sp);
    else
        hipLaunchKernelGGL((route_score_kernel<D, G, false>), grid, dim3(kScoreThreads), 0, st, sp);
}

template <int D>
static hipError_t launch_score_g(int G, dim3 grid, const ScoreParams& sp, hipStream_t st) {
    switch (G) {
        case 1: launch_score_t<D, 1>(grid, sp, st); break;
        case 2: launch_score_t<D, 2>(grid, sp, st); break;
        case 4: launch_score_t<D, 4>(grid, sp, st); break;
        case 8: launch_score_t<D, 8>(grid, sp, st); break;
        case 16: launch_score_t<D, 16>(grid, sp, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Lowest level (0-based, >= 1) from which every level up to the top is handled
// by the fused traversal; g.L when none is (the leaf level is never fused: its
// scan needs the whole chip and the group's shared reads).
static int upper_from(const Geo& g) {
    int lo = g.L;
    while (lo - 1 >= 1 && g.nodes[lo - 1] <= kUpperNodes) --lo;
    return lo;
}

// Level li's cut from the dense-by-node scores: one workgroup per (row, query
// head), or one wave per pair when the pairs are many (many = true): with the
// candidates staged in the wave's LDS when the level fits (wave = true), else
// re-read from global memory in every pass.
static hipError_t launch_cut(const Geo& g, const RouteArgs& a, int li, hipStream_t st, bool wave = false,
                             bool many = false) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    const bool top = (li == g.L - 1);
    CutParams cp{};
    cp.ri = a.ri;
    cp.scores = reinterpret_cast<float*>(ws + lay.scores);
    cp.nodes_total = g.nodes_total;
    cp.lvl_off = g.sel_off[li];
    cp.lvl_off_up = top ? 0 : g.sel_off[li + 1];
    cp.kept = reinterpret_cast<int32_t*>(ws + lay.kept);
    cp.kept_cnt = reinterpret_cast<int32_t*>(ws + lay.kept_cnt);
    cp.bitmap = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
    cp.bm_words_total = lay.bm_words_total;
    cp.bm_off = static_cast<int64_t>(lay.bm_off[li]);
    cp.sel_blocks = a.sel_blocks;
    cp.n_sel = a.n_sel;
    cp.sel_cap = a.sel_cap;
    cp.level_stats = a.level_stats;
    cp.level_sel = a.level_sel;
    cp.lsel_off = static_cast<int64_t>(a.rows) * g.Hq * g.sel_off[li];
    cp.nodes_l = g.nodes[li];
    cp.status = reinterpret_cast<uint32_t*>(ws + lay.status);
    cp.cap = g.cap;
    cp.b = g.b;
    cp.lb = g.lb;
    cp.li = li;
    cp.L = g.L;
    cp.Hq = g.Hq;
    cp.T = a.ri.T;
    cp.top_p = a.top_p_l[li];
    cp.pairs = static_cast<int64_t>(a.rows) * g.Hq;
    {
        ProfScope ps("route_cut", li + 1, st);
        const dim3 wgrid(static_cast<unsigned>((cp.pairs + kWaveCutWaves - 1) / kWaveCutWaves));
        if (wave) {
            hipLaunchKernelGGL(route_wave_cut_kernel<WaveScratch>, wgrid, dim3(kWaveCutThreads), 0, st, cp);
        } else if (many) {
            hipLaunchKernelGGL(route_wave_cut_kernel<WaveScratchU>, wgrid, dim3(kWaveCutThreads), 0, st, cp);
        } else {
            hipLaunchKernelGGL((route_cut_kernel<kCutWaves, CutShared>), dim3(g.Hq, a.rows), dim3(kCutThreads), 0, st, cp);
        }
    }
    return hipGetLastError();
}

hipError_t launch_route(const Geo& g, const RouteArgs& a, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    float* scores = reinterpret_cast<float*>(ws + lay.scores);
    int32_t* kept = reinterpret_cast<int32_t*>(ws + lay.kept);
    int32_t* kept_cnt = reinterpret_cast<int32_t*>(ws + lay.kept_cnt);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + lay.status);
    const int pairs = a.rows * g.Hkv;

    // many rows per sequence: every level's scores on the matrix cores at
    // once, then the levels' cuts from the top
    if (a.ri.T >= kDenseMinRows && dense_scores_fit(g, a.ri.T) && !g.tangent) {
        hipError_t e = launch_dense_scores(g, a.ri, a.q, a.summaries, scores, 0, g.L - 1, st);
        // one wave per pair while a level's candidates fit a wave's LDS
        for (int li = g.L - 1; e == hipSuccess && li >= 0; --li)
            e = launch_cut(g, a, li, st, g.nodes[li] <= kWaveStage, true);
        return e;
    }

    const int li_lo = upper_from(g);

    if (li_lo < g.L) {
        UpperParams up{};
        up.q = a.q;
        up.ri = a.ri;
        up.summaries = a.summaries;
        for (int l = 0; l < ZHA_MAX_LEVELS; ++l) {
            up.sum_off[l] = g.sum_off[l];
            up.nodes[l] = g.nodes[l];
            up.sel_off[l] = g.sel_off[l];
            up.bm_off[l] = static_cast<int64_t>(lay.bm_off[l]);
        }
        up.nodes_total = g.nodes_total;
        up.kept = kept;
        up.kept_cnt = kept_cnt;
        up.bitmap = bitmap;
        up.rank = lay.split ? reinterpret_cast<int32_t*>(ws + lay.rank) : nullptr;
        up.bm_words_total = lay.bm_words_total;
        up.level_stats = a.level_stats;
        up.level_sel = a.level_sel;
        up.rows = a.rows;
        up.cap = g.cap;
        up.b = g.b;
        up.lb = g.lb;
        up.L = g.L;
        up.li_lo = li_lo;
        up.Hq = g.Hq;
        up.Hkv = g.Hkv;
        up.G = g.G;
        up.T = a.ri.T;
        for (int l = 0; l < ZHA_MAX_LEVELS; ++l) up.top_p_l[l] = a.top_p_l[l];
        up.scale = g.scale;
        for (int l = 0; l < ZHA_MAX_LEVELS; ++l) up.bias_off[l] = g.bias_off[l];
        up.R = g.R;
        up.scores = g.vsum ? scores : nullptr;
        {
            ProfScope ps("route_upper", 0, st);
            const dim3 grid(g.Hq, a.rows), block(kUpperThreads);
            if (g.D == 128) {
                if (g.tangent) hipLaunchKernelGGL((route_upper_kernel<128, true>), grid, block, 0, st, up);
                else hipLaunchKernelGGL((route_upper_kernel<128, false>), grid, block, 0, st, up);
            } else {
                if (g.tangent) hipLaunchKernelGGL((route_upper_kernel<64, true>), grid, block, 0, st, up);
                else hipLaunchKernelGGL((route_upper_kernel<64, false>), grid, block, 0, st, up);
            }
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    for (int li = li_lo - 1; li >= 0; --li) {
        const bool top = (li == g.L - 1);
        ScoreParams sp{};
        sp.q = a.q;
        sp.ri = a.ri;
        sp.summ = a.summaries + g.sum_off[li];
        sp.offs = g.tangent ? a.summaries + g.bias_off[li] : nullptr;
        sp.R = g.R;
        sp.nodes_l = g.nodes[li];
        sp.scores = scores;
        sp.nodes_total = g.nodes_total;
        sp.lvl_off = g.sel_off[li];
        sp.bm_up = bitmap + (top ? 0 : lay.bm_off[li + 1]);
        sp.bm_words_total = lay.bm_words_total;
        sp.cap = g.cap;
        sp.b = g.b;
        sp.lb = g.lb;
        sp.li = li;
        sp.L = g.L;
        sp.Hq = g.Hq;
        sp.Hkv = g.Hkv;
        sp.T = a.ri.T;
        sp.scale = g.scale;
        // parent slots of the level: blocks of b nodes at the top; below, every
        // node of level l+1 plus the incomplete one
        const int64_t slots = top ? (g.nodes[li] + g.b - 1) / g.b : g.nodes[li + 1] + 1;
        const ScoreShape shp = score_shape(slots, pairs);
        sp.kept_cnt = kept_cnt;
        sp.pairs = static_cast<int>(pairs);
        sp.bal_waves = shp.balanced ? shp.waves : 0;
        sp.bal_need = shp.need;
        const dim3 sgrid = shp.balanced ? dim3(static_cast<unsigned>(shp.waves), 1)
                                        : dim3(static_cast<unsigned>(shp.waves), static_cast<unsigned>(pairs));
        if (lay.split) {
            sp.pmax = reinterpret_cast<float*>(ws + lay.pmax);
            sp.pmax_stride = lay.pmax_stride;
            sp.pruns = reinterpret_cast<int32_t*>(ws + lay.pruns);
            sp.chist = reinterpret_cast<unsigned long long*>(ws + lay.chist);
            sp.bm_cur = bitmap + lay.bm_off[li];
            sp.rank_up = reinterpret_cast<const int32_t*>(ws + lay.rank);
            sp.lvl_off_up = top ? 0 : g.sel_off[li + 1];
            sp.cand_sc = reinterpret_cast<float*>(ws + lay.cand_sc);
            sp.cand_nd = reinterpret_cast<int32_t*>(ws + lay.cand_nd);
            sp.cand_stride = lay.cand_stride;
        }
        hipError_t e = (g.D == 128) ? launch_score_g<128>(g.G, sgrid, sp, st)
                                    : launch_score_g<64>(g.G, sgrid, sp, st);
        if (e != hipSuccess) return e;

        if (lay.split) {
            SplitParams xp{};
            xp.ri = a.ri;
            xp.scores = scores;
            xp.nodes_total = g.nodes_total;
            xp.lvl_off = g.sel_off[li];
            xp.lvl_off_up = top ? 0 : g.sel_off[li + 1];
            xp.kept = kept;
            xp.kept_cnt = kept_cnt;
            xp.bitmap = bitmap;
            xp.bm_words_total = lay.bm_words_total;
            xp.bm_off = static_cast<int64_t>(lay.bm_off[li]);
            xp.sel_blocks = a.sel_blocks;
            xp.n_sel = a.n_sel;
            xp.sel_cap = a.sel_cap;
            xp.level_stats = a.level_stats;
            xp.level_sel = a.level_sel;
            xp.lsel_off = static_cast<int64_t>(a.rows) * g.Hq * g.sel_off[li];
            xp.nodes_l = g.nodes[li];
            xp.status = status;
            xp.cap = g.cap;
            xp.b = g.b;
            xp.lb = g.lb;
            xp.li = li;
            xp.L = g.L;
            xp.Hq = g.Hq;
            xp.T = a.ri.T;
            xp.top_p = a.top_p_l[li];
            xp.pmax = reinterpret_cast<const float*>(ws + lay.pmax);
            xp.pruns = reinterpret_cast<const int32_t*>(ws + lay.pruns);
            xp.pmax_stride = lay.pmax_stride;
            xp.cand_sc = reinterpret_cast<const float*>(ws + lay.cand_sc);
            xp.cand_nd = reinterpret_cast<const int32_t*>(ws + lay.cand_nd);
            xp.rank = reinterpret_cast<int32_t*>(ws + lay.rank);
            xp.srt_k = reinterpret_cast<uint32_t*>(ws + lay.srt_k);
            xp.srt_s = reinterpret_cast<float*>(ws + lay.srt_s);
            xp.cand_stride = lay.cand_stride;
            xp.cum = reinterpret_cast<uint32_t*>(ws + lay.cum);
            xp.chist = reinterpret_cast<unsigned long long*>(ws + lay.chist);
            xp.slice_stride = lay.slice_stride;
            // candidates of a level are at most its node slots
            const unsigned nsl = static_cast<unsigned>((g.nodes[li] + kSplitSlice - 1) / kSplitSlice);
            {
                ProfScope ps("route_cut", li + 1, st);
                hipLaunchKernelGGL(route_split_hist_kernel, dim3(nsl, g.Hq, a.rows), dim3(kSplitThreads), 0, st, xp);
                hipLaunchKernelGGL(route_split_emit_kernel, dim3(nsl, g.Hq, a.rows), dim3(kSplitThreads), 0, st, xp);
            }
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }

        e = launch_cut(g, a, li, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zha

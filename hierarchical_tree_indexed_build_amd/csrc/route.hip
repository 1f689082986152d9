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
// Kernels, ordered by kernel boundaries alone: no device-scope fences and no
// cross-workgroup atomics (on this part every XCD has its own L2, and a
// device-scope release writes L2 back).
//  * route_upper_kernel - one workgroup per (row, query head) walks the small
//    upper levels in one launch: candidates, scores and the cut stay in LDS
//    from level to level.
//  * per remaining level (the leaf level always):
//    - route_score_kernel - a workgroup owns kScoreParents parent slots of one
//      (row, kv head). It ORs the group's kept bitmaps of level l+1 over its
//      slots (plus the incomplete parent, whose complete children are the
//      orphans) and scores each such parent's b children once for all g query
//      heads: a summary row is read once per kv group. Scores land in a
//      dense-by-node array per (row, query head).
//    - route_cut_kernel - one workgroup per (row, query head); the candidates'
//      scores are staged in LDS when they fit.
// The cut itself (both cut kernels): masses exp(s - max) are held in 2^-40
// fixed point, so their sums are exact and independent of order; an MSB-first
// radix select over an order-preserving score key finds the boundary score;
// ties at the boundary go to the lower node ids; a stable compaction writes the
// kept ids in ascending order and the head's kept bitmap.
#include <algorithm>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

__device__ __forceinline__ int clamp_visible(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T;
    int n = row_visible(ri, row);
    const int lim = static_cast<int>(imin(ri.seq_lens[s], cap));
    n = n < 0 ? 0 : n;
    return n > lim ? lim : n;
}

// ----------------------------------------------------------------------------
// scoring
// ----------------------------------------------------------------------------
struct ScoreParams {
    const float* q;            // [rows, Hq, D]
    RowInfo ri;
    const float* summ;         // summaries of this level
    int64_t nodes_l;           // node slots per (batch, kv) at this level
    float* scores;             // ws scores base
    int64_t nodes_total;       // per (row, head) stride of the scores
    int64_t lvl_off;           // offset of this level in a (row, head) score array
    const uint32_t* bm_up;     // kept bitmaps of level l+1 (row-head stride bm_words_total)
    int64_t bm_words_total;
    int64_t cap;
    int b, lb, li, L, Hq, Hkv, T;
    float scale;
};

constexpr int kScoreParents = 8;     // parent slots per workgroup (one byte of a bitmap word)

template <int D, int G>
__global__ __launch_bounds__(256) void route_score_kernel(ScoreParams p) {
    const int y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.T;
    const int N = clamp_visible(p.ri, row, p.cap);
    const bool top = (p.li == p.L - 1);
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (p.li + 2)));
    const int64_t orphans = nc - (nc_up << p.lb);
    // parent slots: at the top, blocks of b nodes; below, the complete parents
    // (scored when some head of the group kept them) and the incomplete parent
    // holding the orphans
    const int64_t slots = top ? ((nc + p.b - 1) >> p.lb) : (nc_up + (orphans > 0 ? 1 : 0));
    const int64_t P0 = static_cast<int64_t>(blockIdx.x) * kScoreParents;
    if (P0 >= slots) return;
    const int nact = static_cast<int>(imin(slots - P0, kScoreParents));
    uint32_t act = (1u << nact) - 1u;
    if (!top) {
        const uint32_t* bw = p.bm_up + (static_cast<int64_t>(row) * p.Hq + kv * G) * p.bm_words_total + (P0 >> 5);
        uint32_t kept = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) kept |= bw[h * p.bm_words_total];
        kept = (kept >> (P0 & 31)) & ((1u << kScoreParents) - 1u);
        const uint32_t orph = (orphans > 0 && nc_up >= P0 && nc_up < P0 + kScoreParents) ? (1u << (nc_up - P0)) : 0u;
        act &= kept | orph;
    }
    if (!act) return;

    constexpr int DPL = (G <= 4) ? 16 : (G == 8 ? 8 : 4);   // dims per lane
    constexpr int LPR = D / DPL;                             // lanes per summary row
    constexpr int RPP = kWave / LPR;                         // rows per pass
    constexpr int UNR = 4;                                   // passes issued together
    static_assert(G <= LPR, "one lane per head writes the head's score");
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane / LPR, part = lane % LPR;
    const int wave = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;

    const float* summ = p.summ + (static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes_l * D;
    float* sc0 = p.scores + (static_cast<int64_t>(row) * p.Hq + kv * G) * p.nodes_total + p.lvl_off;
    float qv[G][DPL];
    bool have_q = false;
    int nth = 0;
    for (uint32_t a = act; a; a &= a - 1, ++nth) {
        if (nth % nw != wave) continue;                      // parents dealt round-robin to the waves
        if (!have_q) {                                       // only waves with work read q
#pragma unroll
            for (int h = 0; h < G; ++h)
                load_row<DPL>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + h) * D + part * DPL, qv[h]);
            have_q = true;
        }
        const int64_t par = P0 + (__ffs(static_cast<int>(a)) - 1);
        const int64_t c0 = par << p.lb;
        const int64_t c1 = imin(c0 + p.b, nc);
        for (int64_t cb = c0; cb < c1; cb += UNR * RPP) {
            float x[UNR][DPL];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t c = imin(cb + u * RPP + sub, c1 - 1);   // a present row; extra results are dropped
                load_row<DPL>(summ + c * D + part * DPL, x[u]);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t c = cb + u * RPP + sub;
                float acc[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float t = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) t = fmaf(qv[h][e], x[u][e], t);
                    acc[h] = fast_group_sum<LPR>(t);
                }
                if (c < c1) {
#pragma unroll
                    for (int h = 0; h < G; ++h)
                        if (part == h) sc0[static_cast<int64_t>(h) * p.nodes_total + c] = acc[h] * p.scale;
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------
// the cut: block primitives and the two phases shared by both cut kernels
// ----------------------------------------------------------------------------
constexpr int kCutThreads = 1024;
constexpr int kCutWaves = kCutThreads / kWave;

struct BlockScratch {
    uint64_t hist[2][256];      // radix histograms, alternating between rounds
    uint64_t red_u64[kCutWaves];
    float red_f[kCutWaves];
    uint32_t red_u32[kCutWaves];
    uint64_t bcast_u64[2];
    uint32_t bcast_u32[2];
    uint32_t wkey[kWave];       // single-wave cut: keys, masses in rank order, prefix masses
    uint64_t wmass[kWave];
    uint64_t wpre[kWave];
    int32_t wcount;
};

// Block reductions: a DPP scan per wave (lane 63 holds the wave's result),
// one LDS slot per wave, one barrier to publish and one to free the slots.
__device__ __forceinline__ float block_max_f(float v, BlockScratch& bs) {
    v = wave_scan_max_f(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) bs.red_f[w] = v;
    __syncthreads();
    float r = bs.red_f[0];
#pragma unroll
    for (int i = 1; i < kCutWaves; ++i) r = fmaxf(r, bs.red_f[i]);
    __syncthreads();
    return r;
}

// Sum of a u64 and max of a u32 over the block, in one round of barriers.
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
    for (int i = 0; i < kCutWaves; ++i) {
        rs += bs.red_u64[i];
        rm = max(rm, bs.red_u32[i]);
    }
    __syncthreads();
    sum = rs;
    mx = rm;
}

// Exclusive prefix sum over the block in thread order; *total receives the sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, BlockScratch& bs, uint64_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t inc = wave_scan_u64(v);
    if (lane == 63) bs.red_u64[w] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kCutWaves; ++i) {
        if (i < w) before += bs.red_u64[i];
        all += bs.red_u64[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Where a cut ends: every candidate whose key is below kappa is kept, plus the
// first need_ties (in candidate order) of those whose key equals kappa.
struct CutBoundary {
    bool take_all;
    uint32_t kappa;
    uint64_t need_ties;
};

// The boundary of the top-p cut over candidates 0..n-1 with scores score(k)
// and maximum mx. Masses exp(s - mx) are 2^-40 fixed point; the total and
// every partial sum are exact. An MSB-first radix select, 8 bits a round,
// finds the key at which the mass of the keys before it first reaches
// ceil(top_p * total). Rounds alternate between two histograms, so a round
// needs two barriers: after the histogram, and after the digit is published.
template <class ScoreAt>
__device__ __forceinline__ CutBoundary cut_boundary(ScoreAt score, int64_t n, float mx, float top_p,
                                                    BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    CutBoundary cb{(top_p >= 1.0f) || n == 0, 0u, 0u};
    if (cb.take_all) return cb;
    uint64_t E = 0;
    uint32_t kmax = 0;
    for (int64_t k = tid; k < n; k += nt) {
        const float s = score(k);
        const uint64_t F = mass_fx(s, mx);
        E += F;
        if (F) kmax = max(kmax, desc_key(s));
    }
    for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;      // published by the barriers below
    block_sum_max(E, kmax, bs);
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
        for (int64_t k = tid; k < n; k += nt) {
            const float s = score(k);
            const uint32_t key = desc_key(s);
            if (((key ^ prefix) & hmask) != 0u) continue;
            const uint64_t F = mass_fx(s, mx);
            if (F) atomicAdd(reinterpret_cast<unsigned long long*>(&hist[(key >> shift) & ((1u << nb) - 1u)]),
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

// The same cut for n <= 64 candidates, run by one wave with candidate k on
// lane k and no block barriers: each lane ranks its candidate in (key asc,
// index asc) order against the others' keys, the masses are laid out in rank
// order and prefix-summed, and a candidate is kept when the mass ranked before
// it is still below ceil(top_p * total). This keeps exactly the candidates the
// boundary search keeps: all keys below the boundary key, and of the boundary
// key's ties the first in index order. emit(pos, k) for every kept one, pos
// ascending in k. Returns the number kept (on every lane).
template <class ScoreAt, class Emit>
__device__ __forceinline__ int wave_cut_small(ScoreAt score, int n, float top_p, BlockScratch& bs, Emit emit) {
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
    bs.wkey[lane] = key;
    __builtin_amdgcn_wave_barrier();
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const uint32_t kj = bs.wkey[j];
        rank += (kj < key) || (kj == key && j < lane);
    }
    if (valid) bs.wmass[rank] = F;
    __builtin_amdgcn_wave_barrier();
    const uint64_t mj = lane < n ? bs.wmass[lane] : 0;
    bs.wpre[lane] = wave_scan_u64(mj) - mj;
    __builtin_amdgcn_wave_barrier();
    const bool kept = valid && (take_all || bs.wpre[rank] < rem);
    const unsigned long long bal = __ballot(kept);
    if (kept) emit(static_cast<int64_t>(__popcll(bal & ((1ull << lane) - 1ull))), static_cast<int64_t>(lane));
    return __popcll(bal);
}

// Stable compaction of the kept candidates: emit(pos, k) for each kept k, pos
// its rank among the kept (ascending k). Threads own contiguous ranges of k.
// Returns the number kept.
template <class ScoreAt, class Emit>
__device__ __forceinline__ int64_t cut_compact(ScoreAt score, int64_t n, const CutBoundary& cb, BlockScratch& bs,
                                               Emit emit) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t chunk = (n + nt - 1) / nt;
    const int64_t k0 = imin(static_cast<int64_t>(tid) * chunk, n);
    const int64_t k1 = imin(k0 + chunk, n);
    uint32_t c_nt = 0, c_tie = 0;
    if (!cb.take_all) {
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t key = desc_key(score(k));
            c_nt += key < cb.kappa;
            c_tie += key == cb.kappa;
        }
    } else {
        c_nt = static_cast<uint32_t>(k1 - k0);
    }
    uint64_t tot;
    const uint64_t pre = block_excl_scan_u64((static_cast<uint64_t>(c_tie) << 32) | c_nt, bs, &tot);
    uint64_t nt_before = pre & 0xffffffffu, tie_before = pre >> 32;
    const uint64_t tot_nt = tot & 0xffffffffu, tot_tie = tot >> 32;
    const uint64_t ties_kept = tot_tie < cb.need_ties ? tot_tie : cb.need_ties;
    for (int64_t k = k0; k < k1; ++k) {
        int64_t pos;
        if (cb.take_all) {
            pos = k;
        } else {
            const uint32_t key = desc_key(score(k));
            if (key < cb.kappa) {
                pos = static_cast<int64_t>(nt_before + (tie_before < cb.need_ties ? tie_before : cb.need_ties));
                ++nt_before;
            } else if (key == cb.kappa) {
                const bool keep = tie_before < cb.need_ties;
                pos = static_cast<int64_t>(nt_before + tie_before);
                ++tie_before;
                if (!keep) continue;
            } else {
                continue;
            }
        }
        emit(pos, k);
    }
    return static_cast<int64_t>(tot_nt + ties_kept);
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
};

constexpr int kCutStage = 32768;      // candidate scores staged in LDS (128 KiB)
constexpr int kCutBmWords = 4096;     // kept bitmap built in LDS (levels up to 131072 nodes)

struct CutShared {
    float sc[kCutStage];
    uint32_t bm[kCutBmWords];
    BlockScratch bs;
};

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

// kStaged: every candidate score sits in sh.sc (read from HBM once);
// otherwise each pass re-reads the scores from global memory. The two
// variants are separate instantiations, so each only addresses one space.
template <bool kStaged>
__device__ __forceinline__ void cut_level(const CutParams& p, CutShared& sh, const CutCands& cc, int64_t rh,
                                          int64_t nc) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const bool leaf = (p.li == 0);
    const int64_t ncand = cc.ncand;
    auto score = [&](int64_t k) -> float {
        if constexpr (kStaged) return sh.sc[k];
        else return cc.sc[cc.node(k)];
    };

    // kept bitmap of this head at this level: the level below ORs the group's
    // bitmaps to find the parents to score; the attention reads level 1
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int64_t words = (nc + 31) >> 5;
    const bool lds_bm = words <= kCutBmWords;
    if (lds_bm) {
        for (int64_t w = tid; w < words; w += nt) sh.bm[w] = 0u;
    } else {
        for (int64_t w = tid; w < words; w += nt) bm[w] = 0u;
        __threadfence_block();
    }

    // ---- stage the scores, max ----
    // kStageUnroll candidates per thread are in flight at once: their parent
    // ids first, then their scores, so the two dependent loads of one
    // candidate do not serialise the loop.
    constexpr int kStageUnroll = 8;
    float mx = -INFINITY;
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
        for (int u = 0; u < kStageUnroll; ++u) {
            const int64_t k = kb + static_cast<int64_t>(u) * nt;
            if (k < ncand) {
                if constexpr (kStaged) sh.sc[k] = v[u];
                mx = fmaxf(mx, v[u]);
            }
        }
    }
    mx = block_max_f(mx, sh.bs);

    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    // a thread's candidates are contiguous, so its parent id changes every b of them:
    // keep the last one instead of reloading it per candidate
    int64_t last_pi = -1, last_par = 0;
    const int64_t kid_mask = (int64_t(1) << cc.lb) - 1;
    auto emit = [&](int64_t pos, int64_t k) {
        int64_t node;
        if (k < cc.nkids) {
            const int64_t pi = k >> cc.lb;
            if (pi != last_pi) {
                last_pi = pi;
                last_par = cc.up[pi];
            }
            node = (last_par << cc.lb) | (k & kid_mask);
        } else {
            node = (cc.nc_up << cc.lb) + (k - cc.nkids);
        }
        if (kept_out) kept_out[pos] = static_cast<int32_t>(node);
        if (sel_out && pos < p.sel_cap) sel_out[pos] = static_cast<int32_t>(node);
        if (lsel_out) lsel_out[pos] = static_cast<int32_t>(node);
        if (lds_bm) atomicOr(&sh.bm[node >> 5], 1u << (node & 31));
        else __hip_atomic_fetch_or(bm + (node >> 5), 1u << (node & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int64_t m;
    if (ncand <= kWave) {
        if ((tid >> 6) == 0) {
            const int mw = wave_cut_small(score, static_cast<int>(ncand), p.top_p, sh.bs, emit);
            if (tid == 0) sh.bs.wcount = mw;
        }
        __syncthreads();
        m = sh.bs.wcount;
    } else {
        const CutBoundary cb = cut_boundary(score, ncand, mx, p.top_p, sh.bs);
        m = cut_compact(score, ncand, cb, sh.bs, emit);
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

__global__ __launch_bounds__(kCutThreads) void route_cut_kernel(CutParams p) {
    __shared__ CutShared sh;
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
    if (cc.ncand <= kCutStage) cut_level<true>(p, sh, cc, rh, nc);
    else cut_level<false>(p, sh, cc, rh, nc);
}

// ----------------------------------------------------------------------------
// fused traversal of the upper levels
// One workgroup per (row, query head) walks every level from the top down to
// level li_lo in one launch (every fused level has at most kUpperNodes nodes
// per (sequence, kv head)). Per level: the candidate ids are built in LDS from
// the kept nodes of the level above, each candidate's summary row is scored
// against the head's query (16 waves, a row per LPR lanes), and the same
// exact cut runs on the LDS-resident scores. The kept set stays in LDS for the
// next level and is written out (kept list, count, bitmap) for the levels
// below li_lo.
// ----------------------------------------------------------------------------
constexpr int kUpperNodes = 8192;

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
    int64_t bm_words_total;
    int32_t* level_stats;
    int32_t* level_sel;
    int64_t rows;
    int64_t cap;
    int b, lb, L, li_lo, Hq, Hkv, G, T;
    float top_p, scale;
};

struct UpperShared {
    float sc[kUpperNodes];
    int32_t cid[kUpperNodes];          // candidate node ids, ascending
    int32_t par[kUpperNodes];          // kept nodes of the level above, ascending
    uint32_t bm[kUpperNodes / 32 + 1];
    BlockScratch bs;
};

template <int D>
__global__ __launch_bounds__(kCutThreads) void route_upper_kernel(UpperParams p) {
    __shared__ UpperShared sh;
    constexpr int DPL = 16;                    // dims per lane
    constexpr int LPR = D / DPL;               // lanes per summary row
    constexpr int RPP = kWave / LPR;           // rows per wave pass
    constexpr int UNR = 2;                     // passes issued together (1024 threads: <= 128 VGPRs)
    const int hq = blockIdx.x, row = blockIdx.y;
    const int kv = hq / p.G, s = row / p.T;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt / kWave;
    const int sub = lane / LPR, part = lane % LPR;
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    float qv[DPL];
    load_row<DPL>(p.q + rh * D + part * DPL, qv);

    int64_t npar = 0;                          // kept nodes of the level above
    for (int li = p.L - 1; li >= p.li_lo; --li) {
        const bool top = (li == p.L - 1);
        const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (li + 1));
        const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (li + 2)));
        const int64_t nkids = npar << p.lb;
        const int64_t ncand = nkids + (nc - (nc_up << p.lb));   // <= nc <= nodes[li] <= kUpperNodes
        for (int64_t k = tid; k < ncand; k += nt) {
            sh.cid[k] = static_cast<int32_t>(k < nkids ? ((static_cast<int64_t>(sh.par[k >> p.lb]) << p.lb) |
                                                          (k & (p.b - 1)))
                                                       : (nc_up << p.lb) + (k - nkids));
        }
        const int64_t words = (nc + 31) >> 5;
        for (int64_t w = tid; w < words; w += nt) sh.bm[w] = 0u;
        __syncthreads();

        // ---- score the candidates: a row per LPR lanes, RPP rows per wave pass ----
        const float* summ = p.summaries + p.sum_off[li] + (static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes[li] * D;
        float mx = -INFINITY;
        for (int64_t kb = static_cast<int64_t>(wave) * RPP * UNR; kb < ncand; kb += static_cast<int64_t>(nw) * RPP * UNR) {
            float x[UNR][DPL];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t k = imin(kb + u * RPP + sub, ncand - 1);   // a present row; extra results are dropped
                load_row<DPL>(summ + static_cast<int64_t>(sh.cid[k]) * D + part * DPL, x[u]);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                float t = 0.f;
#pragma unroll
                for (int e = 0; e < DPL; ++e) t = fmaf(qv[e], x[u][e], t);
                t = fast_group_sum<LPR>(t) * p.scale;
                const int64_t k = kb + u * RPP + sub;
                if (k < ncand) {
                    mx = fmaxf(mx, t);
                    if (part == 0) sh.sc[k] = t;
                }
            }
        }
        // ---- the cut ----
        auto score = [&](int64_t k) -> float { return sh.sc[k]; };
        int32_t* kept_out = p.kept + rh * p.nodes_total + p.sel_off[li];
        int32_t* lsel_out = p.level_sel ? p.level_sel + p.rows * p.Hq * p.sel_off[li] + rh * p.nodes[li] : nullptr;
        auto emit = [&](int64_t pos, int64_t k) {
            const int32_t node = sh.cid[k];
            sh.par[pos] = node;                 // parents of the next level (cid holds this level's ids)
            kept_out[pos] = node;
            if (lsel_out) lsel_out[pos] = node;
            atomicOr(&sh.bm[node >> 5], 1u << (node & 31));
        };
        int64_t m;
        if (ncand <= kWave) {                  // one wave, no block steps
            __syncthreads();                   // publishes sc[]
            if (wave == 0) {
                const int mw = wave_cut_small(score, static_cast<int>(ncand), p.top_p, sh.bs, emit);
                if (lane == 0) sh.bs.wcount = mw;
            }
            __syncthreads();
            m = sh.bs.wcount;
        } else {
            mx = block_max_f(mx, sh.bs);       // its barriers also publish sc[]
            const CutBoundary cb = cut_boundary(score, ncand, mx, p.top_p, sh.bs);
            m = cut_compact(score, ncand, cb, sh.bs, emit);
            __syncthreads();
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
    hipLaunchKernelGGL((route_score_kernel<D, G>), grid, dim3(256), 0, st, sp);
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

hipError_t launch_route(const Geo& g, const RouteArgs& a, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    float* scores = reinterpret_cast<float*>(ws + lay.scores);
    int32_t* kept = reinterpret_cast<int32_t*>(ws + lay.kept);
    int32_t* kept_cnt = reinterpret_cast<int32_t*>(ws + lay.kept_cnt);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + lay.status);
    const int pairs = a.rows * g.Hkv;
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
        up.top_p = a.top_p;
        up.scale = g.scale;
        {
            ProfScope ps("route_upper", 0, st);
            if (g.D == 128)
                hipLaunchKernelGGL(route_upper_kernel<128>, dim3(g.Hq, a.rows), dim3(kCutThreads), 0, st, up);
            else
                hipLaunchKernelGGL(route_upper_kernel<64>, dim3(g.Hq, a.rows), dim3(kCutThreads), 0, st, up);
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
        const int64_t gx = std::max<int64_t>(1, (slots + kScoreParents - 1) / kScoreParents);
        hipError_t e = (g.D == 128) ? launch_score_g<128>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st)
                                    : launch_score_g<64>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st);
        if (e != hipSuccess) return e;

        CutParams cp{};
        cp.ri = a.ri;
        cp.scores = scores;
        cp.nodes_total = g.nodes_total;
        cp.lvl_off = g.sel_off[li];
        cp.lvl_off_up = top ? 0 : g.sel_off[li + 1];
        cp.kept = kept;
        cp.kept_cnt = kept_cnt;
        cp.bitmap = bitmap;
        cp.bm_words_total = lay.bm_words_total;
        cp.bm_off = static_cast<int64_t>(lay.bm_off[li]);
        cp.sel_blocks = a.sel_blocks;
        cp.n_sel = a.n_sel;
        cp.sel_cap = a.sel_cap;
        cp.level_stats = a.level_stats;
        cp.level_sel = a.level_sel;
        cp.lsel_off = static_cast<int64_t>(a.rows) * g.Hq * g.sel_off[li];
        cp.nodes_l = g.nodes[li];
        cp.status = status;
        cp.cap = g.cap;
        cp.b = g.b;
        cp.lb = g.lb;
        cp.li = li;
        cp.L = g.L;
        cp.Hq = g.Hq;
        cp.T = a.ri.T;
        cp.top_p = a.top_p;
        {
            ProfScope ps("route_cut", li + 1, st);
            hipLaunchKernelGGL(route_cut_kernel, dim3(g.Hq, a.rows), dim3(kCutThreads), 0, st, cp);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace zha

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
//    - the cut: with few (row, head) pairs, route_split_hist_kernel,
//      route_split_bound_kernel and route_split_emit_kernel spread each pair's
//      cut over slices of its candidates; otherwise route_cut_kernel, one
//      workgroup per (row, query head), with the scores staged in LDS when
//      they fit.
// The cut itself: masses exp(s - max) are held in 2^-40 fixed point, so their
// sums are exact and independent of order. The masses are binned by the
// score's distance below the max; the bin where the running mass reaches
// ceil(top_p * total) holds the boundary, which a ranking or a radix select
// over that bin's members (an order-preserving score key) pins down exactly.
// Ties at the boundary go to the lower node ids; a stable compaction writes
// the kept ids in ascending order and the head's kept bitmap. The small upper
// levels use a radix select over all their candidates.
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
    // split cut of this level (null otherwise): each workgroup leaves the
    // maximum of every head's candidates it scored, and workgroup 0 of a
    // (row, kv head) clears the heads' mass bins
    float* pmax;               // [rows, Hq, pmax_stride], column blockIdx.x
    int64_t pmax_stride;
    unsigned long long* chist; // [rows, Hq, kCutBins]
};


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
    const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * G;      // the group's first (row, head)
    if (p.chist && blockIdx.x == 0) {
        for (int i = threadIdx.x; i < G * kCutBins; i += blockDim.x) p.chist[rh0 * kCutBins + i] = 0ull;
    }
    const int nact = P0 < slots ? static_cast<int>(imin(slots - P0, kScoreParents)) : 0;
    uint32_t act = nact ? (1u << nact) - 1u : 0u;
    uint32_t mine[G];                                        // parent slots each head takes candidates from
    uint32_t orph = 0;
#pragma unroll
    for (int h = 0; h < G; ++h) mine[h] = act;
    if (!top && act) {
        const uint32_t* bw = p.bm_up + rh0 * p.bm_words_total + (P0 >> 5);
        uint32_t kept = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mine[h] = (bw[h * p.bm_words_total] >> (P0 & 31)) & ((1u << kScoreParents) - 1u);
            kept |= mine[h];
        }
        orph = (orphans > 0 && nc_up >= P0 && nc_up < P0 + kScoreParents) ? (1u << (nc_up - P0)) : 0u;
        act &= kept | orph;
#pragma unroll
        for (int h = 0; h < G; ++h) mine[h] |= orph;
    }
    if (!act) {
        if (p.pmax && threadIdx.x < G) p.pmax[(rh0 + threadIdx.x) * p.pmax_stride + blockIdx.x] = -INFINITY;
        return;
    }

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
    float hmx[G];                                            // per head: max over its own candidates
#pragma unroll
    for (int h = 0; h < G; ++h) hmx[h] = -INFINITY;
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
        const int slot = __ffs(static_cast<int>(a)) - 1;
        const int64_t par = P0 + slot;
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
                    for (int h = 0; h < G; ++h) {
                        const float sv = acc[h] * p.scale;
                        if (part == h) sc0[static_cast<int64_t>(h) * p.nodes_total + c] = sv;
                        if ((mine[h] >> slot) & 1u) hmx[h] = fmaxf(hmx[h], sv);
                    }
                }
            }
        }
    }
    if (p.pmax) {
        __shared__ float red[G][4];
        const int lane64 = threadIdx.x & 63;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_scan_max_f(hmx[h])), 63));
            if (lane64 == 0) red[h][wave] = m;
        }
        __syncthreads();
        if (threadIdx.x < G) {
            float m = red[threadIdx.x][0];
            for (int w = 1; w < nw; ++w) m = fmaxf(m, red[threadIdx.x][w]);
            p.pmax[(rh0 + threadIdx.x) * p.pmax_stride + blockIdx.x] = m;
        }
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
    uint32_t list_n;
    uint32_t wkey[kWave];       // single-wave ranking: keys, candidate ids, masses in rank order, prefixes
    uint32_t wk[kWave];
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

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, BlockScratch& bs) {
    v = wave_scan_u64(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 63) bs.red_u64[w] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < kCutWaves; ++i) r += bs.red_u64[i];
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
// alternate between two histograms, so a round needs two barriers.
template <class Entry>
__device__ __forceinline__ uint32_t radix_kappa(Entry entry, int64_t cnt, uint64_t& rem, BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    uint32_t prefix = 0;
    int cur = 0;
    for (int known = 0; known < 32; known += 8) {
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
template <class ScoreAt>
__device__ __forceinline__ CutBoundary cut_boundary_radix(ScoreAt score, int64_t n, float mx, float top_p,
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
template <class ScoreAt>
__device__ __forceinline__ CutBoundary cut_boundary(ScoreAt score, int64_t n, float mx, float top_p,
                                                    uint64_t* bins, BlockScratch& bs) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    CutBoundary cb{(top_p >= 1.0f) || n == 0, 0u, 0u};
    if (cb.take_all) return cb;
    for (int i = tid; i < kCutBins; i += nt) bins[i] = 0;
    __syncthreads();
    uint64_t E = 0;
    for (int64_t k = tid; k < n; k += nt) {
        const float s = score(k);
        const uint64_t F = mass_fx(s, mx);
        if (F) {
            E += F;
            atomicAdd(reinterpret_cast<unsigned long long*>(&bins[cut_bin(s, mx)]), static_cast<unsigned long long>(F));
        }
    }
    if (tid == 0) bs.list_n = 0;
    for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;
    E = block_sum_u64(E, bs);                       // its barriers also publish the bins
    uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(top_p) * static_cast<double>(E)));
    if (rem == 0) rem = 1;

    constexpr int BPT = kCutBins / kCutThreads;     // bins per thread, in bin order
    uint64_t v[BPT], lsum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        v[j] = bins[tid * BPT + j];
        lsum += v[j];
    }
    uint64_t tot;
    uint64_t c = block_excl_scan_u64(lsum, bs, &tot);
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
            if (mem && pos < kCutList) bs.list[pos] = static_cast<uint32_t>(k);
        }
    }
    __syncthreads();
    const uint32_t m = bs.list_n;

    if (m <= kWave) {
        if (wave == 0) {
            const bool valid = lane < static_cast<int>(m);
            const uint32_t k = valid ? bs.list[lane] : 0u;
            const float s = valid ? score(k) : 0.f;
            const uint32_t key = valid ? desc_key(s) : 0xffffffffu;
            const uint64_t F = valid ? mass_fx(s, mx) : 0;
            bs.wkey[lane] = key;
            bs.wk[lane] = k;
            __builtin_amdgcn_wave_barrier();
            int rank = 0;
            for (int j = 0; j < static_cast<int>(m); ++j) {
                const uint32_t kj = bs.wkey[j], ij = bs.wk[j];
                rank += (kj < key) || (kj == key && ij < k);
            }
            if (valid) bs.wmass[rank] = F;
            __builtin_amdgcn_wave_barrier();
            const uint64_t mj = lane < static_cast<int>(m) ? bs.wmass[lane] : 0;
            bs.wpre[lane] = wave_scan_u64(mj) - mj;
            __builtin_amdgcn_wave_barrier();
            const bool kept = valid && bs.wpre[rank] < rem;
            const uint32_t kap = static_cast<uint32_t>(
                __builtin_amdgcn_readlane(static_cast<int>(wave_scan_max_u32(kept ? key : 0u)), 63));
            const uint64_t ties = __popcll(__ballot(kept && key == kap));
            if (lane == 0) {
                bs.bcast_u32[1] = kap;
                bs.bcast_u64[1] = ties;
            }
        }
        __syncthreads();
        cb.kappa = bs.bcast_u32[1];
        cb.need_ties = bs.bcast_u64[1];
        return cb;
    }
    uint32_t kap;
    if (m <= kCutList) {
        kap = radix_kappa([&](int64_t e, uint32_t& key, uint64_t& F) {
            const float s = score(static_cast<int64_t>(bs.list[e]));
            key = desc_key(s);
            F = mass_fx(s, mx);
            return true;
        }, m, rem, bs);
    } else {
        kap = radix_kappa([&](int64_t k, uint32_t& key, uint64_t& F) {
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

// Stable compaction of the kept candidates, 64 at a time: each wave owns a
// contiguous range of 64-candidate blocks, and a count pass plus a scan over
// the waves gives each wave its first output position. emit(pos, k) for every
// kept k, pos its rank among the kept (ascending k). mark(k, bits) once per
// aligned run of (1 << run_lg) <= 32 candidates starting at k that keeps any,
// bit i set when k + i is kept (a run maps to consecutive node ids inside one
// bitmap word). Returns the number kept.
template <class ScoreAt, class Emit, class Mark>
__device__ __forceinline__ int64_t cut_compact(ScoreAt score, int64_t n, const CutBoundary& cb, int run_lg,
                                               BlockScratch& bs, Emit emit, Mark mark) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t nblk = (n + 63) >> 6;
    const int64_t per = (nblk + kCutWaves - 1) / kCutWaves;
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
    for (int i = 0; i < kCutWaves; ++i) {
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
};

constexpr int kCutStage = 32768;      // candidate scores staged in LDS (128 KiB)
constexpr int kCutUpStage = 2048;     // kept parents staged in LDS with them
constexpr int kCutBmWords = 4096;     // kept bitmap built in LDS (levels up to 131072 nodes)

struct CutShared {
    float sc[kCutStage];
    int32_t up[kCutUpStage];
    union {
        uint64_t bins[kCutBins];      // the cut's first pass
        uint32_t bm[kCutBmWords];     // then the kept bitmap
    };
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

// kStaged: the candidates' scores and parents sit in LDS (read from HBM
// once); otherwise each pass re-reads them from global memory. The two
// variants are separate instantiations, so each only addresses one space.
template <bool kStaged>
__device__ __forceinline__ void cut_level(const CutParams& p, CutShared& sh, CutCands cc, int64_t rh,
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
        // every candidate of the thread in flight at once: at most kCutStage / kCutThreads
        constexpr int U = kCutStage / kCutThreads;
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
    const bool lds_bm = words <= kCutBmWords;
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
        mx = block_max_f(mx, sh.bs);                      // its barriers also publish the staged scores
        const CutBoundary cb = cut_boundary(score, ncand, mx, p.top_p, sh.bins, sh.bs);
        clear_bm();                                        // published by the compaction's first barrier
        m = cut_compact(score, ncand, cb, cc.lb < 5 ? cc.lb : 5, sh.bs, emit, mark);
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
    if (cc.ncand <= kCutStage && kc <= kCutUpStage) cut_level<true>(p, sh, cc, rh, nc);
    else cut_level<false>(p, sh, cc, rh, nc);
}

// ----------------------------------------------------------------------------
// the split cut: a level's cut spread over many workgroups per (row, head)
// When few (row, head) pairs route at once, one workgroup per pair leaves most
// of the chip idle while the largest candidate sets (tens of thousands) are
// cut. The same cut then runs as three kernels over slices of kSplitSlice
// candidates, ordered by kernel boundaries:
//  * route_split_hist_kernel  (slice): the level max from the scoring
//    workgroups' partial maxima; the slice's node ids and scores copied in
//    candidate order; each mass added into the (row, head)'s global bins.
//  * route_split_bound_kernel (row, head): the boundary bin from the bins, its
//    members listed and resolved exactly (as in cut_boundary), and the count of
//    kept candidates and of boundary ties before every slice.
//  * route_split_emit_kernel  (slice): the kept ids written at their ranks and
//    their bitmap bits set.
// The kept set is the one cut_boundary and cut_compact produce.
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
    int pmax_n;                // scoring workgroups of the level
    int64_t pmax_stride;
    float* cand_sc;
    int32_t* cand_nd;
    int64_t cand_stride;
    unsigned long long* chist;
    SplitInfo* info;
    unsigned long long* slice;
    int64_t slice_stride;
};

__device__ __forceinline__ CutCands split_cands(const SplitParams& p, int row, int64_t rh, int64_t* nc_out) {
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
    *nc_out = nc;
    return cc;
}

constexpr int kSplitThreads = 256;
constexpr int kSplitPer = kSplitSlice / kSplitThreads;       // candidates per thread

__global__ __launch_bounds__(kSplitThreads) void route_split_hist_kernel(SplitParams p) {
    __shared__ unsigned long long bins[kCutBins];
    __shared__ float red[kSplitThreads / kWave];
    const int sl = blockIdx.x, hq = blockIdx.y, row = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    int64_t nc;
    const CutCands cc = split_cands(p, row, rh, &nc);
    const int64_t k0 = static_cast<int64_t>(sl) << kSplitSliceLog2;
    if (k0 >= cc.ncand) return;
    float mx = -INFINITY;
    for (int i = tid; i < p.pmax_n; i += kSplitThreads) mx = fmaxf(mx, p.pmax[rh * p.pmax_stride + i]);
    int32_t nd[kSplitPer];
    float v[kSplitPer];
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        const int64_t k = k0 + tid + u * kSplitThreads;
        nd[u] = k < cc.ncand ? static_cast<int32_t>(cc.node(k)) : -1;
    }
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) v[u] = nd[u] >= 0 ? cc.sc[nd[u]] : -INFINITY;
    float* csc = p.cand_sc + rh * p.cand_stride;
    int32_t* cnd = p.cand_nd + rh * p.cand_stride;
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        const int64_t k = k0 + tid + u * kSplitThreads;
        if (nd[u] >= 0) {
            csc[k] = v[u];
            cnd[k] = nd[u];
        }
    }
    for (int i = tid; i < kCutBins; i += kSplitThreads) bins[i] = 0ull;
    mx = wave_scan_max_f(mx);
    if (lane == 63) red[w] = mx;
    __syncthreads();                                  // also publishes the cleared bins
    mx = red[0];
#pragma unroll
    for (int i = 1; i < kSplitThreads / kWave; ++i) mx = fmaxf(mx, red[i]);
    if (p.top_p >= 1.0f) return;                      // everything is kept: no bins needed
#pragma unroll
    for (int u = 0; u < kSplitPer; ++u) {
        if (nd[u] < 0) continue;
        const uint64_t F = mass_fx(v[u], mx);
        if (F) atomicAdd(&bins[cut_bin(v[u], mx)], static_cast<unsigned long long>(F));
    }
    __syncthreads();
    unsigned long long* gb = p.chist + rh * kCutBins;
    for (int i = tid; i < kCutBins; i += kSplitThreads) {
        const unsigned long long x = bins[i];
        if (x) atomicAdd(gb + i, x);                  // device scope: slices of a (row, head) sit on any XCD
    }
}

constexpr int kSplitBoundBatch = 16;                  // candidate scores per thread in flight

struct SplitBoundShared {
    uint32_t s_lt[kSplitMaxSlices];                   // per slice: candidates below the boundary key
    uint32_t s_tie[kSplitMaxSlices];                  // per slice: candidates at the boundary key
    BlockScratch bs;
};

__global__ __launch_bounds__(kCutThreads) void route_split_bound_kernel(SplitParams p) {
    __shared__ SplitBoundShared sh;
    BlockScratch& bs = sh.bs;
    const int hq = blockIdx.x, row = blockIdx.y;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    int64_t nc;
    const CutCands cc = split_cands(p, row, rh, &nc);
    const int64_t ncand = cc.ncand;
    const int nsl = static_cast<int>((ncand + kSplitSlice - 1) >> kSplitSliceLog2);
    const bool leaf = (p.li == 0);
    // this level's bitmap starts empty; the emit kernel ORs the kept bits in
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int64_t words = (nc + 31) >> 5;
    for (int64_t i = tid; i < words; i += nt) bm[i] = 0u;
    for (int i = tid; i < nsl; i += nt) {
        sh.s_lt[i] = 0u;
        sh.s_tie[i] = 0u;
    }
    const bool take_all = (p.top_p >= 1.0f) || ncand == 0;
    uint32_t kappa = 0u;
    uint64_t need = 0;
    const float* csc = p.cand_sc + rh * p.cand_stride;
    if (!take_all) {
        // issued together: the bins, the scoring maxima, the first batch of candidate scores
        constexpr int BPT = kCutBins / kCutThreads;
        constexpr int U = kSplitBoundBatch;
        const unsigned long long* gb = p.chist + rh * kCutBins;
        uint64_t v[BPT], lsum = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) v[j] = gb[tid * BPT + j];
        float mx = -INFINITY;
        for (int i = tid; i < p.pmax_n; i += nt) mx = fmaxf(mx, p.pmax[rh * p.pmax_stride + i]);
        float sb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t k = tid + static_cast<int64_t>(u) * nt;
            sb[u] = k < ncand ? csc[k] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < BPT; ++j) lsum += v[j];
        mx = block_max_f(mx, bs);                     // its barriers also publish the cleared slice counts
        if (tid == 0) bs.list_n = 0;
        for (int i = tid; i < 256; i += nt) bs.hist[0][i] = 0;
        uint64_t E;
        uint64_t c = block_excl_scan_u64(lsum, bs, &E);
        uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(p.top_p) * static_cast<double>(E)));
        if (rem == 0) rem = 1;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            if (v[j] != 0 && c < rem && c + v[j] >= rem) {
                bs.bcast_u32[0] = static_cast<uint32_t>(tid * BPT + j);
                bs.bcast_u64[0] = c;
            }
            c += v[j];
        }
        __syncthreads();
        const int bstar = static_cast<int>(bs.bcast_u32[0]);
        rem -= bs.bcast_u64[0];
        // one pass, U candidates per thread in flight: members of the boundary bin,
        // and per slice the candidates in earlier bins
        const int nc32 = static_cast<int>(ncand);         // a level holds fewer than 2^31 candidates
        for (int kb = 0; kb < nc32; kb += U * nt) {
            if (kb) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = kb + tid + u * nt;
                    sb[u] = k < nc32 ? csc[k] : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int kw = kb + u * nt + (wave << 6);   // the wave's first candidate
                const int k = kw + lane;
                bool lt = false, mem = false;
                if (k < nc32) {
                    const int bn = cut_bin(sb[u], mx);
                    lt = bn < bstar;
                    mem = bn == bstar;                 // with any mass, so counts by key and by bin agree
                }
                const unsigned long long blt = __ballot(lt);
                if (lane == 0 && blt) atomicAdd(&sh.s_lt[kw >> kSplitSliceLog2], static_cast<uint32_t>(__popcll(blt)));
                const unsigned long long bal = __ballot(mem);
                if (bal) {
                    uint32_t base = 0;
                    if (lane == 0) base = atomicAdd(&bs.list_n, static_cast<uint32_t>(__popcll(bal)));
                    base = static_cast<uint32_t>(__shfl(static_cast<int>(base), 0));
                    const uint32_t pos = base + static_cast<uint32_t>(__popcll(bal & ((1ull << lane) - 1ull)));
                    if (mem && pos < kCutList) bs.list[pos] = static_cast<uint32_t>(k);
                }
            }
        }
        __syncthreads();
        const uint32_t m = bs.list_n;
        auto score = [&](int64_t k) -> float { return csc[k]; };
        if (m <= kWave) {
            if (wave == 0) {
                const bool valid = lane < static_cast<int>(m);
                const uint32_t k = valid ? bs.list[lane] : 0u;
                const float s = valid ? score(k) : 0.f;
                const uint32_t key = valid ? desc_key(s) : 0xffffffffu;
                const uint64_t F = valid ? mass_fx(s, mx) : 0;
                bs.wkey[lane] = key;
                bs.wk[lane] = k;
                __builtin_amdgcn_wave_barrier();
                int rank = 0;
                for (int j = 0; j < static_cast<int>(m); ++j) {
                    const uint32_t kj = bs.wkey[j], ij = bs.wk[j];
                    rank += (kj < key) || (kj == key && ij < k);
                }
                if (valid) bs.wmass[rank] = F;
                __builtin_amdgcn_wave_barrier();
                const uint64_t mj = lane < static_cast<int>(m) ? bs.wmass[lane] : 0;
                bs.wpre[lane] = wave_scan_u64(mj) - mj;
                __builtin_amdgcn_wave_barrier();
                const bool kept = valid && bs.wpre[rank] < rem;
                const uint32_t kap = static_cast<uint32_t>(
                    __builtin_amdgcn_readlane(static_cast<int>(wave_scan_max_u32(kept ? key : 0u)), 63));
                const uint64_t ties = __popcll(__ballot(kept && key == kap));
                if (lane == 0) {
                    bs.bcast_u32[1] = kap;
                    bs.bcast_u64[1] = ties;
                }
            }
            __syncthreads();
            kappa = bs.bcast_u32[1];
            need = bs.bcast_u64[1];
        } else {
            if (m <= kCutList) {
                kappa = radix_kappa([&](int64_t e, uint32_t& key, uint64_t& F) {
                    const float s = score(static_cast<int64_t>(bs.list[e]));
                    key = desc_key(s);
                    F = mass_fx(s, mx);
                    return true;
                }, m, rem, bs);
            } else {
                kappa = radix_kappa([&](int64_t k, uint32_t& key, uint64_t& F) {
                    const float s = score(k);
                    if (cut_bin(s, mx) != bstar) return false;
                    key = desc_key(s);
                    F = mass_fx(s, mx);
                    return true;
                }, ncand, rem, bs);
            }
            const uint64_t Fk = mass_fx(desc_key_to_float(kappa), mx);
            need = Fk ? (rem + Fk - 1) / Fk : 0;
        }
        // the boundary bin's members below the boundary key, and its ties, per slice
        if (m <= kCutList) {
            for (uint32_t i = tid; i < m; i += nt) {
                const uint32_t k = bs.list[i];
                const uint32_t key = desc_key(score(k));
                if (key < kappa) atomicAdd(&sh.s_lt[k >> kSplitSliceLog2], 1u);
                else if (key == kappa) atomicAdd(&sh.s_tie[k >> kSplitSliceLog2], 1u);
            }
        } else {                                       // a crowded bin: count every slice by key
            for (int i = tid; i < nsl; i += nt) sh.s_lt[i] = 0u;
            __syncthreads();
            for (int64_t kb = 0; kb < ncand; kb += nt) {
                const int64_t k = kb + tid;
                const uint32_t key = k < ncand ? desc_key(csc[k]) : 0xffffffffu;
                const unsigned long long blt = __ballot(k < ncand && key < kappa);
                const unsigned long long bti = __ballot(k < ncand && key == kappa);
                const int sidx = static_cast<int>((kb + (wave << 6)) >> kSplitSliceLog2);
                if (lane == 0 && blt) atomicAdd(&sh.s_lt[sidx], __popcll(blt));
                if (lane == 0 && bti) atomicAdd(&sh.s_tie[sidx], __popcll(bti));
            }
        }
    } else {
        for (int i = tid; i < nsl; i += nt) {
            const int64_t a = static_cast<int64_t>(i) << kSplitSliceLog2;
            sh.s_lt[i] = static_cast<uint32_t>(imin(ncand - a, kSplitSlice));
        }
    }
    __syncthreads();
    // (ties << 32 | below) before each slice: one slice per thread, in slice order
    const uint64_t mine = tid < nsl ? ((static_cast<uint64_t>(sh.s_tie[tid]) << 32) | sh.s_lt[tid]) : 0ull;
    uint64_t all;
    const uint64_t before = block_excl_scan_u64(mine, bs, &all);
    if (tid < nsl) p.slice[rh * p.slice_stride + tid] = before;
    const uint64_t tot_lt = all & 0xffffffffu, tot_tie = all >> 32;
    const int64_t m_kept = static_cast<int64_t>(tot_lt + (tot_tie < need ? tot_tie : need));
    if (tid == 0) {
        SplitInfo si;
        si.need_ties = need;
        si.kappa = kappa;
        si.take_all = take_all ? 1 : 0;
        si.ncand = ncand;
        p.info[rh] = si;
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
}

__global__ __launch_bounds__(kSplitThreads) void route_split_emit_kernel(SplitParams p) {
    constexpr int NW = kSplitThreads / kWave;
    constexpr int BPW = kSplitSlice / kSplitThreads;           // 64-candidate blocks per wave
    __shared__ uint64_t wcnt[NW];
    const int sl = blockIdx.x, hq = blockIdx.y, row = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    const SplitInfo si = p.info[rh];
    const int64_t ncand = si.ncand;
    const int64_t k0 = static_cast<int64_t>(sl) << kSplitSliceLog2;
    if (k0 >= ncand) return;
    const float* csc = p.cand_sc + rh * p.cand_stride;
    const int32_t* cnd = p.cand_nd + rh * p.cand_stride;
    // this wave's blocks: [kw, kw + 64 * BPW)
    const int64_t kw = k0 + static_cast<int64_t>(w) * 64 * BPW;
    float s[BPW];
    int32_t nd[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int64_t k = kw + j * 64 + lane;
        s[j] = k < ncand ? csc[k] : 0.f;
        nd[j] = k < ncand ? cnd[k] : 0;
    }
    auto classify = [&](int j, bool& lt, bool& tie) {
        const int64_t k = kw + j * 64 + lane;
        const bool valid = k < ncand;
        if (si.take_all) {
            lt = valid;
            tie = false;
            return;
        }
        const uint32_t key = desc_key(s[j]);
        lt = valid && key < si.kappa;
        tie = valid && key == si.kappa;
    };
    uint64_t c_lt = 0, c_tie = 0;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        bool lt, tie;
        classify(j, lt, tie);
        c_lt += __popcll(__ballot(lt));
        c_tie += __popcll(__ballot(tie));
    }
    if (lane == 0) wcnt[w] = (c_tie << 32) | c_lt;
    __syncthreads();
    uint64_t before = p.slice[rh * p.slice_stride + sl];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        if (i < w) before += wcnt[i];
    uint64_t lt_b = before & 0xffffffffu, tie_b = before >> 32;
    const uint64_t need = si.need_ties;
    const bool leaf = (p.li == 0);
    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int run = 1 << (p.lb < 5 ? p.lb : 5);
    const unsigned long long run_mask = (1ull << run) - 1ull;
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        bool lt, tie;
        classify(j, lt, tie);
        const unsigned long long blt = __ballot(lt), btie = __ballot(tie);
        const uint64_t my_lt = lt_b + __popcll(blt & below), my_tie = tie_b + __popcll(btie & below);
        const bool keep = lt || (tie && my_tie < need);
        if (keep) {
            const int64_t pos = static_cast<int64_t>(my_lt + (lt ? (my_tie < need ? my_tie : need) : my_tie));
            const int32_t node = nd[j];
            if (kept_out) kept_out[pos] = node;
            if (sel_out && pos < p.sel_cap) sel_out[pos] = node;
            if (lsel_out) lsel_out[pos] = node;
        }
        const unsigned long long bkeep = __ballot(keep);
        if ((lane & (run - 1)) == 0) {
            const uint32_t bits = static_cast<uint32_t>((bkeep >> lane) & run_mask);
            if (bits)   // a run's nodes are consecutive and share one word; runs of other slices may share it too
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
        };
        auto mark = [&](int64_t k, uint32_t bits) {
            const int32_t node = sh.cid[k];
            atomicOr(&sh.bm[node >> 5], bits << (node & 31));
        };
        int64_t m;
        if (ncand <= kWave) {                  // one wave, no block steps
            __syncthreads();                   // publishes sc[]
            if (wave == 0) {
                const int mw = wave_cut_small(score, static_cast<int>(ncand), p.top_p, sh.bs,
                                              [&](int64_t pos, int64_t k) { emit(pos, k); mark(k, 1u); });
                if (lane == 0) sh.bs.wcount = mw;
            }
            __syncthreads();
            m = sh.bs.wcount;
        } else {
            mx = block_max_f(mx, sh.bs);       // its barriers also publish sc[]
            const CutBoundary cb = cut_boundary_radix(score, ncand, mx, p.top_p, sh.bs);
            m = cut_compact(score, ncand, cb, p.lb < 5 ? p.lb : 5, sh.bs, emit, mark);
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
        if (lay.split) {
            sp.pmax = reinterpret_cast<float*>(ws + lay.pmax);
            sp.pmax_stride = lay.pmax_stride;
            sp.chist = reinterpret_cast<unsigned long long*>(ws + lay.chist);
        }
        hipError_t e = (g.D == 128) ? launch_score_g<128>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st)
                                    : launch_score_g<64>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st);
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
            xp.top_p = a.top_p;
            xp.pmax = reinterpret_cast<const float*>(ws + lay.pmax);
            xp.pmax_n = static_cast<int>(gx);
            xp.pmax_stride = lay.pmax_stride;
            xp.cand_sc = reinterpret_cast<float*>(ws + lay.cand_sc);
            xp.cand_nd = reinterpret_cast<int32_t*>(ws + lay.cand_nd);
            xp.cand_stride = lay.cand_stride;
            xp.chist = reinterpret_cast<unsigned long long*>(ws + lay.chist);
            xp.info = reinterpret_cast<SplitInfo*>(ws + lay.cinfo);
            xp.slice = reinterpret_cast<unsigned long long*>(ws + lay.cslice);
            xp.slice_stride = lay.slice_stride;
            // candidates of a level are at most its node slots
            const unsigned nsl = static_cast<unsigned>((g.nodes[li] + kSplitSlice - 1) / kSplitSlice);
            {
                ProfScope ps("route_cut", li + 1, st);
                hipLaunchKernelGGL(route_split_hist_kernel, dim3(nsl, g.Hq, a.rows), dim3(kSplitThreads), 0, st, xp);
                hipLaunchKernelGGL(route_split_bound_kernel, dim3(g.Hq, a.rows), dim3(kCutThreads), 0, st, xp);
                hipLaunchKernelGGL(route_split_emit_kernel, dim3(nsl, g.Hq, a.rows), dim3(kSplitThreads), 0, st, xp);
            }
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            continue;
        }

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

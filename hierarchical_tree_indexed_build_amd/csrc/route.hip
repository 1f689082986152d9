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
// Two kernels per level, ordered by the kernel boundary alone: no device-scope
// fences and no cross-workgroup atomics (on this part every XCD has its own L2,
// and a device-scope release writes L2 back).
//  * route_score_kernel - a workgroup owns kScoreParents parent slots of one
//    (row, kv head). It ORs the group's kept bitmaps of level l+1 over its
//    slots (plus the incomplete parent, whose complete children are the
//    orphans) and scores each such parent's b children once for all g query
//    heads: a summary row is read once per kv group. Scores land in a
//    dense-by-node array per (row, query head).
//  * route_cut_kernel - one workgroup per (row, query head). The candidates'
//    scores are staged in LDS when they fit; masses exp(s - max) are held in
//    2^-40 fixed point, so their sums are exact and independent of order; an
//    MSB-first radix select over an order-preserving score key finds the
//    boundary score; ties at the boundary go to the lower node ids; a stable
//    compaction writes the kept ids in ascending order and the head's kept
//    bitmap (built in LDS when it fits).
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
// cut
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

constexpr int kCutThreads = 1024;
constexpr int kCutWaves = kCutThreads / kWave;
constexpr int kCutStage = 32768;      // candidate scores staged in LDS (128 KiB)
constexpr int kCutBmWords = 4096;     // kept bitmap built in LDS (levels up to 131072 nodes)

struct CutShared {
    float sc[kCutStage];
    uint32_t bm[kCutBmWords];
    uint64_t hist[256];
    uint64_t red_u64[kCutWaves];
    float red_f[kCutWaves];
    uint32_t red_u32[kCutWaves];
    uint64_t bcast_u64;
    uint32_t bcast_u32;
};

__device__ __forceinline__ float block_max_f(float v, CutShared& sh) {
    v = group_max<kWave>(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh.red_f[w] = v;
    __syncthreads();
    float r = sh.red_f[0];
#pragma unroll
    for (int i = 1; i < kCutWaves; ++i) r = fmaxf(r, sh.red_f[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, CutShared& sh) {
    v = wave_sum_u64(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh.red_u64[w] = v;
    __syncthreads();
    uint64_t r = 0;
#pragma unroll
    for (int i = 0; i < kCutWaves; ++i) r += sh.red_u64[i];
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, CutShared& sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, 64)));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) sh.red_u32[w] = v;
    __syncthreads();
    uint32_t r = sh.red_u32[0];
#pragma unroll
    for (int i = 1; i < kCutWaves; ++i) r = max(r, sh.red_u32[i]);
    __syncthreads();
    return r;
}

// Exclusive prefix sum over the block in thread order; *total receives the sum.
__device__ __forceinline__ uint64_t block_excl_scan_u64(uint64_t v, CutShared& sh, uint64_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t inc = wave_incl_scan_u64(v, lane);
    if (lane == 63) sh.red_u64[w] = inc;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kCutWaves; ++i) {
        if (i < w) before += sh.red_u64[i];
        all += sh.red_u64[i];
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

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

// The cut proper. kStaged: every candidate score sits in sh.sc (read from HBM
// once); otherwise each pass re-reads the scores from global memory. The two
// variants are separate instantiations, so each only ever addresses one space.
template <bool kStaged>
__device__ __forceinline__ void cut_body(const CutParams& p, CutShared& sh, const CutCands& cc, int64_t rh,
                                         int64_t nc) {
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const bool leaf = (p.li == 0);
    const int64_t ncand = cc.ncand;
    auto score = [&](int64_t k) -> float {
        if constexpr (kStaged) return sh.sc[k];
        else return cc.sc[cc.node(k)];
    };

    // kept bitmap of this head at this level: the level below ORs the group's
    // bitmaps to find the parents to score
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
    float mx = -INFINITY;
    for (int64_t k = tid; k < ncand; k += nt) {
        const float v = cc.sc[cc.node(k)];
        if constexpr (kStaged) sh.sc[k] = v;
        mx = fmaxf(mx, v);
    }
    mx = block_max_f(mx, sh);

    // ---- fixed-point total mass; least significant key with mass ----
    const bool take_all = (p.top_p >= 1.0f) || ncand == 0;
    uint32_t kappa = 0;
    uint64_t need_ties = 0;
    if (!take_all) {
        uint64_t E = 0;
        uint32_t kmax = 0;
        for (int64_t k = tid; k < ncand; k += nt) {
            const float s = score(k);
            const uint64_t F = mass_fx(s, mx);
            E += F;
            if (F) kmax = max(kmax, desc_key(s));
        }
        E = block_sum_u64(E, sh);
        kmax = block_max_u32(kmax, sh);
        const uint32_t kmin = desc_key(mx);
        uint64_t rem = static_cast<uint64_t>(ceil(static_cast<double>(p.top_p) * static_cast<double>(E)));
        if (rem == 0) rem = 1;
        int known = (kmin == kmax) ? 32 : __clz(static_cast<int>(kmin ^ kmax));
        uint32_t prefix = kmin & top_bits_mask(known);
        // ---- radix select of the boundary key, 8 bits at a time ----
        while (known < 32) {
            const int nb = min(8, 32 - known);
            const int shift = 32 - known - nb;
            const uint32_t hmask = top_bits_mask(known);
            for (int i = tid; i < 256; i += nt) sh.hist[i] = 0;
            __syncthreads();
            for (int64_t k = tid; k < ncand; k += nt) {
                const float s = score(k);
                const uint32_t key = desc_key(s);
                if (((key ^ prefix) & hmask) != 0u) continue;
                const uint64_t F = mass_fx(s, mx);
                if (F) atomicAdd(reinterpret_cast<unsigned long long*>(&sh.hist[(key >> shift) & ((1u << nb) - 1u)]),
                                 static_cast<unsigned long long>(F));
            }
            __syncthreads();
            if (wave == 0) {
                // lanes own 4 consecutive digits; scan in digit order
                uint64_t v[4], lsum = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[j] = sh.hist[lane * 4 + j];
                    lsum += v[j];
                }
                const uint64_t inc = wave_incl_scan_u64(lsum, lane);
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
                    sh.bcast_u32 = static_cast<uint32_t>(found >= 0 ? found : 0);
                    sh.bcast_u64 = found >= 0 ? before : 0;
                }
            }
            __syncthreads();
            rem -= sh.bcast_u64;
            prefix |= sh.bcast_u32 << shift;
            known += nb;
            __syncthreads();
        }
        kappa = prefix;
        const uint64_t Fk = mass_fx(desc_key_to_float(kappa), mx);
        need_ties = Fk ? (rem + Fk - 1) / Fk : 0;
    }

    // ---- stable selection: contiguous candidate ranges per thread ----
    const int64_t chunk = (ncand + nt - 1) / nt;
    const int64_t k0 = imin(static_cast<int64_t>(tid) * chunk, ncand);
    const int64_t k1 = imin(k0 + chunk, ncand);
    uint32_t c_nt = 0, c_tie = 0;
    if (!take_all) {
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t key = desc_key(score(k));
            c_nt += key < kappa;
            c_tie += key == kappa;
        }
    } else {
        c_nt = static_cast<uint32_t>(k1 - k0);
    }
    uint64_t tot;
    const uint64_t pre = block_excl_scan_u64((static_cast<uint64_t>(c_tie) << 32) | c_nt, sh, &tot);
    uint64_t nt_before = pre & 0xffffffffu, tie_before = pre >> 32;
    const uint64_t tot_nt = tot & 0xffffffffu, tot_tie = tot >> 32;
    const uint64_t ties_kept = tot_tie < need_ties ? tot_tie : need_ties;
    const int64_t m = static_cast<int64_t>(tot_nt + ties_kept);

    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    for (int64_t k = k0; k < k1; ++k) {
        const int64_t node = cc.node(k);
        bool keep;
        int64_t pos;
        if (take_all) {
            keep = true;
            pos = k;
        } else {
            const uint32_t key = desc_key(score(k));
            if (key < kappa) {
                keep = true;
                pos = static_cast<int64_t>(nt_before + (tie_before < need_ties ? tie_before : need_ties));
                ++nt_before;
            } else if (key == kappa) {
                keep = tie_before < need_ties;
                pos = static_cast<int64_t>(nt_before + tie_before);
                ++tie_before;
            } else {
                keep = false;
                pos = 0;
            }
        }
        if (!keep) continue;
        if (kept_out) kept_out[pos] = static_cast<int32_t>(node);
        if (sel_out && pos < p.sel_cap) sel_out[pos] = static_cast<int32_t>(node);
        if (lsel_out) lsel_out[pos] = static_cast<int32_t>(node);
        if (lds_bm) atomicOr(&sh.bm[node >> 5], 1u << (node & 31));
        else __hip_atomic_fetch_or(bm + (node >> 5), 1u << (node & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
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
    if (cc.ncand <= kCutStage) cut_body<true>(p, sh, cc, rh, nc);
    else cut_body<false>(p, sh, cc, rh, nc);
}

// ----------------------------------------------------------------------------
// launcher
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

hipError_t launch_route(const Geo& g, const RouteArgs& a, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    float* scores = reinterpret_cast<float*>(ws + lay.scores);
    int32_t* kept = reinterpret_cast<int32_t*>(ws + lay.kept);
    int32_t* kept_cnt = reinterpret_cast<int32_t*>(ws + lay.kept_cnt);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + lay.status);
    const int pairs = a.rows * g.Hkv;

    for (int li = g.L - 1; li >= 0; --li) {
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

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
// Two kernels per level:
//  * route_score_kernel - one wave per candidate block (the b children of a
//    kept parent). The g query heads of a kv group share one read of every
//    summary row: a block is scored once for all g heads if any of them kept
//    its parent (the union of the group's kept sets, built by the previous
//    level's cut). Scores land in a dense-by-node array per (row, head).
//  * route_cut_kernel - one workgroup per (row, query head). Exact cut with
//    softmax masses in 2^-40 fixed point (exp in fp32, integer sums: exact and
//    independent of summation order), an MSB-first radix select over the
//    order-preserving score key to find the boundary score, index-ascending
//    tie handling, and a stable compaction that emits kept ids in ascending
//    order. The last workgroup of each kv group to finish ORs the group's
//    kept bitmaps into the union list the next level's scoring walks.
#include <algorithm>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

// ----------------------------------------------------------------------------
// scoring
// ----------------------------------------------------------------------------
struct ScoreParams {
    const float* q;            // [rows, Hq, D]
    RowInfo ri;
    const float* summ;         // summaries of this level
    int64_t nodes_l;           // node slots per (batch, kv) at this level
    float* scores;             // ws scores base
    int64_t nodes_total;       // per (row, head) stride of scores / kept / ulist
    int64_t lvl_off;           // offset of this level in the per-(row,head) arrays
    int64_t lvl_off_up;        // offset of level l+1
    const int32_t* ulist;      // union of kept nodes at l+1 per (row, kv)
    const int32_t* ucnt;       // [rows, Hkv, L]
    uint32_t* grp_ctr;         // zeroed by the top-level launch
    int64_t n_ctr;
    int64_t span_l, span_up, cap;
    int b, li, L, Hq, Hkv, T;
    float scale;
};

__device__ __forceinline__ int clamp_visible(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T;
    int n = row_visible(ri, row);
    const int lim = static_cast<int>(min<int64_t>(ri.seq_lens[s], cap));
    n = n < 0 ? 0 : n;
    return n > lim ? lim : n;
}

template <int D, int G>
__global__ __launch_bounds__(256) void route_score_kernel(ScoreParams p) {
    if (p.grp_ctr) {
        for (int64_t i = static_cast<int64_t>(blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
             i < p.n_ctr; i += static_cast<int64_t>(gridDim.x) * gridDim.y * blockDim.x)
            p.grp_ctr[i] = 0;
    }
    const int y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.T;
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t nc = N / p.span_l;
    const bool top = (p.li == p.L - 1);
    int64_t ucount = 0, nc_up = 0, nitems;
    if (top) {
        nitems = (nc + p.b - 1) / p.b;
    } else {
        nc_up = N / p.span_up;
        ucount = p.ucnt[(static_cast<int64_t>(row) * p.Hkv + kv) * p.L + p.li + 1];
        nitems = ucount + ((nc > nc_up * p.b) ? 1 : 0);
    }
    if (nitems == 0) return;

    constexpr int DPL = (G <= 4) ? 16 : (G == 8 ? 8 : 4);   // dims per lane
    constexpr int LPR = D / DPL;                             // lanes per summary row
    constexpr int RPP = kWave / LPR;                         // rows per pass
    constexpr int UNR = 4;                                   // passes issued together
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane / LPR, part = lane % LPR;
    const int wave = threadIdx.x / kWave, nw = blockDim.x / kWave;

    float qv[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
        load_row<DPL>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + h) * D + part * DPL, qv[h]);

    const float* summ = p.summ + (static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes_l * D;
    const int32_t* ul = p.ulist + (static_cast<int64_t>(row) * p.Hkv + kv) * p.nodes_total + p.lvl_off_up;
    float* sc0 = p.scores + (static_cast<int64_t>(row) * p.Hq + kv * G) * p.nodes_total + p.lvl_off;

    for (int64_t it = static_cast<int64_t>(blockIdx.x) * nw + wave; it < nitems;
         it += static_cast<int64_t>(gridDim.x) * nw) {
        const int64_t par = top ? it : (it < ucount ? static_cast<int64_t>(ul[it]) : nc_up);
        const int64_t c0 = par * p.b;
        const int64_t c1 = min(c0 + p.b, nc);
        for (int64_t cb = c0; cb < c1; cb += UNR * RPP) {
            float x[UNR][DPL];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t c = cb + u * RPP + sub;
                if (c < c1) load_row<DPL>(summ + c * D + part * DPL, x[u]);
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int64_t c = cb + u * RPP + sub;
                if (c >= c1) continue;       // uniform across the LPR lanes of a row
                float acc[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) a = fmaf(qv[h][e], x[u][e], a);
                    acc[h] = group_sum<LPR>(a);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
                    if (h % LPR == part) sc0[static_cast<int64_t>(h) * p.nodes_total + c] = acc[h] * p.scale;
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
    uint32_t* bitmap;          // ws bitmaps: (row*Hq + hq)*bm_words_total + bm_off
    int64_t bm_words_total, bm_off;
    int32_t* ulist;            // union list output for this level
    int32_t* ucnt;
    uint32_t* grp_ctr;         // [rows, Hkv, L]
    int32_t* sel_blocks;
    int32_t* n_sel;
    int sel_cap;
    int32_t* level_stats;
    int32_t* level_sel;
    int64_t lsel_off, nodes_l;
    uint32_t* status;
    int64_t span_l, span_up, cap;
    int b, li, L, Hq, Hkv, G, T;
    float top_p;
};

constexpr int kCutThreads = 512;
constexpr int kCutWaves = kCutThreads / kWave;

struct CutShared {
    uint64_t hist[256];
    uint64_t red_u64[kCutWaves];
    float red_f[kCutWaves];
    uint32_t red_u32[kCutWaves];
    uint64_t bcast_u64[2];
    uint32_t bcast_u32[2];
    int flag;
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

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kCutThreads) void route_cut_kernel(CutParams p) {
    __shared__ CutShared sh;
    const int hq = blockIdx.x, row = blockIdx.y, kv = hq / p.G;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int N = clamp_visible(p.ri, row, p.cap);
    const int64_t nc = N / p.span_l;
    const int64_t rh = static_cast<int64_t>(row) * p.Hq + hq;
    const bool top = (p.li == p.L - 1);
    const bool leaf = (p.li == 0);
    const float* sc = p.scores + rh * p.nodes_total + p.lvl_off;

    int64_t kc = 0, nc_up = 0;
    const int32_t* up = nullptr;
    if (!top) {
        nc_up = N / p.span_up;
        kc = p.kept_cnt[rh * p.L + p.li + 1];
        up = p.kept + rh * p.nodes_total + p.lvl_off_up;
    }
    const int64_t b = p.b;
    const int64_t nkids = kc * b;
    const int64_t ncand = nkids + (nc - nc_up * b);
    auto cand = [&](int64_t k) -> int64_t {
        return k < nkids ? static_cast<int64_t>(up[k / b]) * b + (k % b) : nc_up * b + (k - nkids);
    };

    // this head's kept bitmap for the level (consumed by the level below's scoring)
    uint32_t* bm = p.bitmap + rh * p.bm_words_total + p.bm_off;
    const int64_t words = (nc + 31) / 32;
    if (!leaf)
        for (int64_t w = tid; w < words; w += nt) bm[w] = 0u;

    // ---- pass A: max score ----
    float mx = -INFINITY;
    for (int64_t k = tid; k < ncand; k += nt) mx = fmaxf(mx, sc[cand(k)]);
    mx = block_max_f(mx, sh);

    // ---- pass B: fixed-point total mass, least significant key with mass ----
    const bool take_all = (p.top_p >= 1.0f) || ncand == 0;
    uint32_t kappa = 0;
    uint64_t need_ties = 0;
    if (!take_all) {
        uint64_t E = 0;
        uint32_t kmax = 0;
        for (int64_t k = tid; k < ncand; k += nt) {
            const float s = sc[cand(k)];
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
        // ---- radix select: find the boundary key, 8 bits at a time ----
        while (known < 32) {
            const int nb = min(8, 32 - known);
            const int shift = 32 - known - nb;
            const uint32_t hmask = top_bits_mask(known);
            for (int i = tid; i < 256; i += nt) sh.hist[i] = 0;
            __syncthreads();
            for (int64_t k = tid; k < ncand; k += nt) {
                const float s = sc[cand(k)];
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
                    if (found < 0 && c + v[j] >= rem && v[j] != 0) {
                        found = lane * 4 + j;
                        before = c;
                    }
                    c += v[j];
                }
                const unsigned long long bal = __ballot(found >= 0);
                const int first = bal ? __ffsll(static_cast<long long>(bal)) - 1 : 63;
                if (lane == first) {
                    sh.bcast_u32[0] = static_cast<uint32_t>(found >= 0 ? found : 255);
                    sh.bcast_u64[0] = (found >= 0) ? before : c - v[3];
                }
            }
            __syncthreads();
            const uint32_t digit = sh.bcast_u32[0];
            rem -= sh.bcast_u64[0];
            prefix |= digit << shift;
            known += nb;
            __syncthreads();
        }
        kappa = prefix;
        const uint64_t Fk = mass_fx(desc_key_to_float(kappa), mx);
        need_ties = Fk ? (rem + Fk - 1) / Fk : 0;
    }

    // ---- stable selection: contiguous ranges per thread ----
    const int64_t chunk = (ncand + nt - 1) / nt;
    const int64_t k0 = min<int64_t>(static_cast<int64_t>(tid) * chunk, ncand);
    const int64_t k1 = min<int64_t>(k0 + chunk, ncand);
    uint32_t c_nt = 0, c_tie = 0;
    if (!take_all) {
        for (int64_t k = k0; k < k1; ++k) {
            const uint32_t key = desc_key(sc[cand(k)]);
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
    const int64_t m = static_cast<int64_t>(tot_nt + min(tot_tie, need_ties));

    int32_t* kept_out = leaf ? nullptr : p.kept + rh * p.nodes_total + p.lvl_off;
    int32_t* sel_out = leaf ? p.sel_blocks + rh * p.sel_cap : nullptr;
    int32_t* lsel_out = p.level_sel ? p.level_sel + p.lsel_off + rh * p.nodes_l : nullptr;
    if (!leaf) __threadfence();   // the zeroed bitmap is visible device-wide before any atomicOr
    __syncthreads();
    for (int64_t k = k0; k < k1; ++k) {
        const int64_t node = cand(k);
        bool keep;
        int64_t pos;
        if (take_all) {
            keep = true;
            pos = k;
        } else {
            const uint32_t key = desc_key(sc[node]);
            if (key < kappa) {
                keep = true;
                pos = static_cast<int64_t>(nt_before + min(tie_before, need_ties));
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
        if (kept_out) {
            kept_out[pos] = static_cast<int32_t>(node);
            atomicOr(bm + (node >> 5), 1u << (node & 31));
        }
        if (sel_out && pos < p.sel_cap) sel_out[pos] = static_cast<int32_t>(node);
        if (lsel_out) lsel_out[pos] = static_cast<int32_t>(node);
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
    if (leaf) return;

    // ---- last head of the kv group builds the group's union of kept nodes ----
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        uint32_t* ctr = p.grp_ctr + (static_cast<int64_t>(row) * p.Hkv + kv) * p.L + p.li;
        const uint32_t old = atomicAdd(ctr, 1u);
        const int last = (old == static_cast<uint32_t>(p.G - 1));
        if (last) atomicExch(ctr, 0u);
        sh.flag = last;
    }
    __syncthreads();
    if (!sh.flag) return;
    __threadfence();
    const uint32_t* gb = p.bitmap + (static_cast<int64_t>(row) * p.Hq + kv * p.G) * p.bm_words_total + p.bm_off;
    const int64_t wchunk = (words + nt - 1) / nt;
    const int64_t w0 = min<int64_t>(static_cast<int64_t>(tid) * wchunk, words);
    const int64_t w1 = min<int64_t>(w0 + wchunk, words);
    uint32_t cnt = 0;
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t u = 0;
        for (int h = 0; h < p.G; ++h) u |= ld_relaxed(gb + static_cast<int64_t>(h) * p.bm_words_total + w);
        cnt += __popc(u);
    }
    uint64_t utot;
    uint64_t upos = block_excl_scan_u64(cnt, sh, &utot);
    int32_t* ul = p.ulist + (static_cast<int64_t>(row) * p.Hkv + kv) * p.nodes_total + p.lvl_off;
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t u = 0;
        for (int h = 0; h < p.G; ++h) u |= ld_relaxed(gb + static_cast<int64_t>(h) * p.bm_words_total + w);
        while (u) {
            const int bit = __ffs(static_cast<int>(u)) - 1;
            u &= u - 1;
            ul[upos++] = static_cast<int32_t>(w * 32 + bit);
        }
    }
    if (tid == 0) p.ucnt[(static_cast<int64_t>(row) * p.Hkv + kv) * p.L + p.li] = static_cast<int32_t>(utot);
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
    int32_t* ulist = reinterpret_cast<int32_t*>(ws + lay.ulist);
    int32_t* ucnt = reinterpret_cast<int32_t*>(ws + lay.ucnt);
    uint32_t* grp_ctr = reinterpret_cast<uint32_t*>(ws + lay.grp_ctr);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws + lay.status);
    const int pairs = a.rows * g.Hkv;

    for (int li = g.L - 1; li >= 0; --li) {
        ScoreParams sp{};
        sp.q = a.q;
        sp.ri = a.ri;
        sp.summ = a.summaries + g.sum_off[li];
        sp.nodes_l = g.nodes[li];
        sp.scores = scores;
        sp.nodes_total = g.nodes_total;
        sp.lvl_off = g.sel_off[li];
        sp.lvl_off_up = (li + 1 < g.L) ? g.sel_off[li + 1] : 0;
        sp.ulist = ulist;
        sp.ucnt = ucnt;
        sp.grp_ctr = (li == g.L - 1) ? grp_ctr : nullptr;
        sp.n_ctr = static_cast<int64_t>(a.rows) * g.Hkv * g.L;
        sp.span_l = g.span[li];
        sp.span_up = g.span[li + 1];
        sp.cap = g.cap;
        sp.b = g.b;
        sp.li = li;
        sp.L = g.L;
        sp.Hq = g.Hq;
        sp.Hkv = g.Hkv;
        sp.T = a.ri.T;
        sp.scale = g.scale;
        const int64_t max_items = (g.nodes[li] + g.b - 1) / g.b + 1;
        const int64_t want = std::max<int64_t>(1, (4096 + pairs - 1) / pairs);
        const int64_t gx = std::max<int64_t>(1, std::min<int64_t>((max_items + 3) / 4, want));
        hipError_t e = (g.D == 128) ? launch_score_g<128>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st)
                                    : launch_score_g<64>(g.G, dim3(static_cast<unsigned>(gx), pairs), sp, st);
        if (e != hipSuccess) return e;

        CutParams cp{};
        cp.ri = a.ri;
        cp.scores = scores;
        cp.nodes_total = g.nodes_total;
        cp.lvl_off = g.sel_off[li];
        cp.lvl_off_up = sp.lvl_off_up;
        cp.kept = kept;
        cp.kept_cnt = kept_cnt;
        cp.bitmap = bitmap;
        cp.bm_words_total = lay.bm_words_total;
        cp.bm_off = static_cast<int64_t>(lay.bm_off[li]);
        cp.ulist = ulist;
        cp.ucnt = ucnt;
        cp.grp_ctr = grp_ctr;
        cp.sel_blocks = a.sel_blocks;
        cp.n_sel = a.n_sel;
        cp.sel_cap = a.sel_cap;
        cp.level_stats = a.level_stats;
        cp.level_sel = a.level_sel;
        cp.lsel_off = static_cast<int64_t>(a.rows) * g.Hq * g.sel_off[li];
        cp.nodes_l = g.nodes[li];
        cp.status = status;
        cp.span_l = g.span[li];
        cp.span_up = g.span[li + 1];
        cp.cap = g.cap;
        cp.b = g.b;
        cp.li = li;
        cp.L = g.L;
        cp.Hq = g.Hq;
        cp.Hkv = g.Hkv;
        cp.G = g.G;
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

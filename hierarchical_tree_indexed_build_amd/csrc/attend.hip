// attend.hip - exact attention over the selected tokens, and the dense baseline.
//
// A query row that sees N tokens attends I = {0} U (kept leaf chunks) U
// [b*floor((N-1)/b), N) ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", §Routing, I(q) and o(q); token 0 is the sink of
// "Zyphra Hierarchical Attention: The End of Quadratic Attention?", §How the
// tree is built and searched). The dense baseline attends [0, N).
//
// Kernels:
//  * attn_union_kernel  - per (row, kv head): OR the g query heads' kept leaf
//    chunks into one ascending list of (chunk, head mask) items, adding chunk
//    0 (sink) and the current chunk; K/V of a chunk are then read once for the
//    whole GQA group.
//  * attend_kernel      - split-K flash decoding. Workgroup = (split, row, kv
//    head); each wave streams 16-token groups of its split with an online
//    softmax for all g heads (scores: lanes own a slice of d, reduced within
//    the token's lanes; values: lanes own d/64 dimensions); waves merge in LDS
//    and write one (max, sum, acc[d]) partial per head and split.
//  * attend_combine_kernel - per (row, head): LSE merge of the splits.
#include <algorithm>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

constexpr uint32_t kAllHeads = 1u << 30;     // item flag: every head attends the chunk (current chunk)

__device__ __forceinline__ int visible_clamped(const RowInfo& ri, int row, int64_t cap) {
    const int s = row / ri.T;
    int n = row_visible(ri, row);
    const int lim = static_cast<int>(min<int64_t>(ri.seq_lens[s], cap));
    n = n < 0 ? 0 : n;
    return n > lim ? lim : n;
}

__device__ __forceinline__ uint32_t ld_relaxed_a(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------
// union of the group's kept leaf chunks
// One workgroup per (row, kv head). Leaf ids are walked in chunks of
// kUnionChunk ids: each head's ascending list is cut at the chunk end by a
// binary search, bits are set in LDS, and the chunk's words are compacted with
// a block scan. No global atomics, no device-scope fences.
// ----------------------------------------------------------------------------
struct UnionParams {
    RowInfo ri;
    const int32_t* sel_blocks;
    const int32_t* n_sel;
    int sel_cap;
    int2* items;               // [rows, Hkv, item_stride]
    int64_t item_stride;
    int32_t* acnt;             // [rows, Hkv]
    int64_t cap;
    int b, Hq, Hkv, G;
};

constexpr int kUnionThreads = 1024;
constexpr int kUnionWords = 512;                  // bitmap words per head per chunk
constexpr int64_t kUnionChunk = kUnionWords * 32; // leaf ids per chunk

__global__ __launch_bounds__(kUnionThreads) void attn_union_kernel(UnionParams p) {
    __shared__ uint32_t bm[kMaxGroup][kUnionWords];
    __shared__ int cur_pos[kMaxGroup], end_pos[kMaxGroup];
    __shared__ uint32_t wsum[kUnionThreads / kWave];
    const int y = blockIdx.x;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int N = visible_clamped(p.ri, row, p.cap);
    if (N <= 0) {
        if (tid == 0) p.acnt[y] = 0;
        return;
    }
    const int64_t cur = (N - 1) / p.b;
    const int64_t nblk = cur + 1;
    const int64_t nc1 = N / p.b;
    const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * p.G;
    if (tid < p.G) cur_pos[tid] = 0;
    int2* items = p.items + static_cast<int64_t>(y) * p.item_stride;
    uint32_t total = 0;
    for (int64_t cb = 0; cb < nblk; cb += kUnionChunk) {
        const int64_t ce = cb + kUnionChunk;
        for (int i = tid; i < p.G * kUnionWords; i += nt) (&bm[0][0])[i] = 0u;
        if (tid < p.G) {
            const int32_t* lst = p.sel_blocks + (rh0 + tid) * p.sel_cap;
            int lo = cur_pos[tid], hi = max(0, min(p.n_sel[rh0 + tid], p.sel_cap));
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (lst[mid] < ce) lo = mid + 1;
                else hi = mid;
            }
            end_pos[tid] = lo;
        }
        __syncthreads();
        for (int h = 0; h < p.G; ++h) {
            const int32_t* lst = p.sel_blocks + (rh0 + h) * p.sel_cap;
            for (int j = cur_pos[h] + tid; j < end_pos[h]; j += nt) {
                const int64_t node = lst[j];
                if (node >= cb && node < ce && node < nc1)
                    atomicOr(&bm[h][(node - cb) >> 5], 1u << (node & 31));
            }
        }
        __syncthreads();
        uint32_t u = 0;
        const int w = tid;
        const int64_t wbase = cb + static_cast<int64_t>(w) * 32;
        if (w < kUnionWords && wbase < nblk) {
            for (int h = 0; h < p.G; ++h) u |= bm[h][w];
            if (wbase == 0) u |= 1u;                                         // sink chunk
            if (cur >= wbase && cur < wbase + 32) u |= 1u << (cur - wbase);  // current chunk
        }
        const uint32_t cnt = __popc(u);
        // block exclusive scan of cnt
        uint32_t inc = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t v = __shfl_up(inc, o, 64);
            if (lane >= o) inc += v;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        uint32_t before = 0, ctot = 0;
        for (int i = 0; i < nt / kWave; ++i) {
            if (i < wave) before += wsum[i];
            ctot += wsum[i];
        }
        uint32_t pos = total + before + inc - cnt;
        while (u) {
            const int bit = __ffs(static_cast<int>(u)) - 1;
            u &= u - 1;
            const int64_t node = wbase + bit;
            uint32_t mask = 0;
            for (int h = 0; h < p.G; ++h) mask |= ((bm[h][w] >> bit) & 1u) << h;
            if (node == cur) mask |= kAllHeads;
            items[pos++] = make_int2(static_cast<int>(node), static_cast<int>(mask));
        }
        total += ctot;
        __syncthreads();
        if (tid < p.G) cur_pos[tid] = end_pos[tid];
        __syncthreads();
    }
    if (tid == 0) p.acnt[y] = static_cast<int32_t>(total);
}

// ----------------------------------------------------------------------------
// split-K attention
// ----------------------------------------------------------------------------
struct AttnParams {
    const float* q;
    RowInfo ri;
    const void* K;
    const void* V;
    const int2* items;
    const int32_t* acnt;
    int64_t item_stride;
    float* partial;            // [rows, Hq, S, D + 2]
    int64_t cap;
    int b, Hq, Hkv, S, dense;
    float scale;
};

constexpr int kGroupTokens = 16;          // tokens a wave handles per pipeline stage
constexpr int kMinGroupsPerSplit = 8;     // a split gets at least 8 groups (128 tokens) of work

// Items (chunks) of one (row, kv head) and the number of splits that share them;
// the attention and the combine must agree on both.
__device__ __forceinline__ void attn_work(const AttnParams& p, int row, int kv, int N, int64_t* groups, int* seff) {
    const int64_t U = p.dense ? (N + p.b - 1) / p.b : p.acnt[static_cast<int64_t>(row) * p.Hkv + kv];
    const int gpi = p.b >= kGroupTokens ? p.b / kGroupTokens : 1;
    const int64_t ng = U * gpi;
    const int64_t s = (ng + kMinGroupsPerSplit - 1) / kMinGroupsPerSplit;
    *groups = ng;
    *seff = static_cast<int>(s < 1 ? 1 : (s > p.S ? p.S : s));
}

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

template <typename KT, int D, int G>
__global__ __launch_bounds__(256) void attend_kernel(AttnParams p) {
    using C = AttnCfg<KT, D, G>;
    constexpr int NW = 4;
    constexpr int NP = C::NP, WPP = C::WPP, DPL = C::DPL, LPT = C::LPT, TPP = C::TPP;
    __shared__ float sm_m[NW][G], sm_l[NW][G];
    __shared__ float sm_acc[NW][G][D];

    const int split = blockIdx.x;
    const int y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.ri.T;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int N = visible_clamped(p.ri, row, p.cap);
    int64_t ng;
    int seff;
    attn_work(p, row, kv, N, &ng, &seff);
    if (split >= seff) return;                       // the combine reads only seff partials
    const int64_t g0 = ng * split / seff, g1 = ng * (split + 1) / seff;
    const int gpi = p.b >= kGroupTokens ? p.b / kGroupTokens : 1;
    const int tg = p.b >= kGroupTokens ? kGroupTokens : p.b;

    const int part = lane % LPT, tsub = lane / LPT;
    float qv[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
        load_vec<DPL>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + h) * D + part * DPL, qv[h]);

    const KT* Kb = static_cast<const KT*>(p.K) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + part * DPL;
    const KT* Vb = static_cast<const KT*>(p.V) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D + part * DPL;
    const int2* items = p.items + static_cast<int64_t>(y) * p.item_stride;

    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    }

    // group g -> (chunk id, head mask). For the sparse path the chunk ids of 64
    // of this wave's upcoming groups are loaded at once, one per lane, and read
    // back with readlane, so no dependent load sits in the pipeline.
    int64_t batch_k0 = -1;
    int2 batch = make_int2(0, 0);
    auto item_of = [&](int64_t g) -> int2 {
        const int64_t it = g / gpi;
        if (p.dense) return make_int2(static_cast<int>(it), static_cast<int>(kAllHeads));
        const int64_t k = (g - g0 - wave) / NW;                 // this wave's k-th group
        if (batch_k0 < 0 || k >= batch_k0 + kWave) {
            batch_k0 = k;
            const int64_t gl = g + static_cast<int64_t>(lane) * NW;
            batch = gl < g1 ? items[gl / gpi] : make_int2(0, 0);
        }
        const int src = static_cast<int>(k - batch_k0);
        return make_int2(__builtin_amdgcn_readlane(batch.x, src), __builtin_amdgcn_readlane(batch.y, src));
    };
    auto first_token = [&](int64_t g, int2 e) -> int64_t {
        return static_cast<int64_t>(e.x) * p.b + (g % gpi) * kGroupTokens;
    };
    auto issue = [&](int64_t t0, uint32_t (&kb)[NP][WPP], uint32_t (&vb)[NP][WPP]) {
#pragma unroll
        for (int ps = 0; ps < NP; ++ps) {
            const int j = min(ps * TPP + tsub, tg - 1);
            const int64_t t = min<int64_t>(t0 + j, N - 1);     // always a present row
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
                a = fast_group_sum<LPT>(a) * p.scale;
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
            const float alpha = (mn[h] == -INFINITY) ? 1.f : expf(m[h] - mn[h]);   // 0 while nothing was seen
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
                const float pr = (mn[h] == -INFINITY) ? 0.f : expf(sc[ps][h] - mn[h]);   // 0 when masked
                l[h] += pr;
#pragma unroll
                for (int e = 0; e < DPL; ++e) acc[h][e] = fmaf(pr, v[e], acc[h][e]);
            }
        }
    };

    // Software pipeline over this wave's groups g0+wave, +NW, +2NW, ...: while a
    // group is consumed, the K/V rows of the next one and the chunk id of the
    // one after are already in flight. Buffers A and B alternate.
    uint32_t kA[NP][WPP], vA[NP][WPP], kB[NP][WPP], vB[NP][WPP];
    int64_t g = g0 + wave;
    if (g < g1) {
        int2 e0 = item_of(g);                                          // chunk of group g
        int2 e1 = (g + NW < g1) ? item_of(g + NW) : make_int2(0, 0);   // chunk of group g + NW
        issue(first_token(g, e0), kA, vA);
        for (;;) {
            int64_t gn = g + NW;
            int2 e2 = make_int2(0, 0);
            if (gn < g1) {
                issue(first_token(gn, e1), kB, vB);
                if (gn + NW < g1) e2 = item_of(gn + NW);
            }
            consume(first_token(g, e0), static_cast<uint32_t>(e0.y), kA, vA);
            if (gn >= g1) break;
            g = gn;
            e0 = e1;
            e1 = e2;
            gn = g + NW;
            e2 = make_int2(0, 0);
            if (gn < g1) {
                issue(first_token(gn, e1), kA, vA);
                if (gn + NW < g1) e2 = item_of(gn + NW);
            }
            consume(first_token(g, e0), static_cast<uint32_t>(e0.y), kB, vB);
            if (gn >= g1) break;
            g = gn;
            e0 = e1;
            e1 = e2;
        }
    }

    // ---- merge the token slots of each wave ----
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float M = strided_max<LPT>(m[h]);
        const float f = (m[h] == -INFINITY) ? 0.f : expf(m[h] - M);
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
    for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
        const int h = idx / (D + 2), c = idx % (D + 2);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
        float out = 0.f;
        if (c == 0) {
            out = M;
        } else {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = (sm_m[w][h] == -INFINITY) ? 0.f : expf(sm_m[w][h] - M);
                out += f * (c == 1 ? sm_l[w][h] : sm_acc[w][h][c - 2]);
            }
        }
        const int64_t rh = static_cast<int64_t>(row) * p.Hq + kv * G + h;
        p.partial[(rh * p.S + split) * (D + 2) + c] = out;
    }
}

// ----------------------------------------------------------------------------
// LSE merge of the splits: one workgroup per (row, query head)
// ----------------------------------------------------------------------------
constexpr int kCombineThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void attend_combine_kernel(AttnParams p, float* out, float* lse, int G) {
    __shared__ float fs[kAttnSplitsMax];
    __shared__ float red[kCombineThreads / kWave];
    __shared__ float part_acc[kCombineThreads];
    const int64_t rh = blockIdx.x;
    const int row = static_cast<int>(rh / p.Hq), kv = static_cast<int>((rh % p.Hq) / G);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = visible_clamped(p.ri, row, p.cap);
    int64_t ng;
    int seff;
    attn_work(p, row, kv, N, &ng, &seff);
    const float* pp = p.partial + rh * p.S * (D + 2);
    const float ms = tid < seff ? pp[tid * (D + 2)] : -INFINITY;
    float M = group_max<kWave>(ms);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int i = 1; i < kCombineThreads / kWave; ++i) M = fmaxf(M, red[i]);
    __syncthreads();
    const float f = (ms == -INFINITY) ? 0.f : expf(ms - M);
    if (tid < kAttnSplitsMax) fs[tid] = f;
    float Lp = group_sum<kWave>(tid < seff ? f * pp[tid * (D + 2) + 1] : 0.f);
    if (lane == 0) red[wave] = Lp;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kCombineThreads / kWave; ++i) L += red[i];
    constexpr int R = kCombineThreads / D;         // split subsets per dimension
    const int dim = tid % D, sub = tid / D;
    float a = 0.f;
#pragma unroll 4
    for (int sp = sub; sp < seff; sp += R) a = fmaf(fs[sp], pp[sp * (D + 2) + 2 + dim], a);
    part_acc[tid] = a;
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) t += part_acc[r * D + tid];
        out[rh * D + tid] = (L > 0.f) ? t / L : 0.f;
    }
    if (tid == 0 && lse) lse[rh] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename KT, int D, int G>
static void launch_attn_t(dim3 grid, const AttnParams& ap, hipStream_t st) {
    ProfScope ps("attend", 0, st);
    hipLaunchKernelGGL((attend_kernel<KT, D, G>), grid, dim3(256), 0, st, ap);
}

template <typename KT, int D>
static hipError_t attn_g(int G, dim3 grid, const AttnParams& ap, hipStream_t st) {
    switch (G) {
        case 1: launch_attn_t<KT, D, 1>(grid, ap, st); break;
        case 2: launch_attn_t<KT, D, 2>(grid, ap, st); break;
        case 4: launch_attn_t<KT, D, 4>(grid, ap, st); break;
        case 8: launch_attn_t<KT, D, 8>(grid, ap, st); break;
        case 16: launch_attn_t<KT, D, 16>(grid, ap, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attend(const Geo& g, const AttendArgs& a, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    const int pairs = a.rows * g.Hkv;
    if (!a.dense) {
        UnionParams up{};
        up.ri = a.ri;
        up.sel_blocks = a.sel_blocks;
        up.n_sel = a.n_sel;
        up.sel_cap = a.sel_cap;
        up.items = reinterpret_cast<int2*>(ws + lay.aitems);
        up.item_stride = g.nodes[0] + 2;
        up.acnt = reinterpret_cast<int32_t*>(ws + lay.acnt);
        up.cap = g.cap;
        up.b = g.b;
        up.Hq = g.Hq;
        up.Hkv = g.Hkv;
        up.G = g.G;
        {
            ProfScope ps("attn_union", 0, st);
            hipLaunchKernelGGL(attn_union_kernel, dim3(pairs), dim3(kUnionThreads), 0, st, up);
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
    ap.partial = reinterpret_cast<float*>(ws + lay.partial);
    ap.cap = g.cap;
    ap.b = g.b;
    ap.Hq = g.Hq;
    ap.Hkv = g.Hkv;
    ap.S = lay.splits;
    ap.dense = a.dense ? 1 : 0;
    ap.scale = g.scale;
    const dim3 grid(lay.splits, pairs);
    hipError_t e;
    const bool bf = g.kv_dtype == ZHA_KV_BF16;
    if (g.D == 128) e = bf ? attn_g<uint16_t, 128>(g.G, grid, ap, st) : attn_g<float, 128>(g.G, grid, ap, st);
    else e = bf ? attn_g<uint16_t, 64>(g.G, grid, ap, st) : attn_g<float, 64>(g.G, grid, ap, st);
    if (e != hipSuccess) return e;
    ProfScope ps("attend_combine", 0, st);
    if (g.D == 128)
        hipLaunchKernelGGL(attend_combine_kernel<128>, dim3(a.rows * g.Hq), dim3(kCombineThreads), 0, st, ap, a.out,
                           a.lse, g.G);
    else
        hipLaunchKernelGGL(attend_combine_kernel<64>, dim3(a.rows * g.Hq), dim3(kCombineThreads), 0, st, ap, a.out,
                           a.lse, g.G);
    return hipGetLastError();
}

}  // namespace zha

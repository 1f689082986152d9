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
// ----------------------------------------------------------------------------
struct UnionParams {
    RowInfo ri;
    const int32_t* sel_blocks;
    const int32_t* n_sel;
    int sel_cap;
    uint32_t* abm;             // [rows, Hq, abm_words]
    int64_t abm_words;
    int2* items;               // [rows, Hkv, item_stride]
    int64_t item_stride;
    int32_t* acnt;             // [rows, Hkv]
    int64_t cap;
    int b, Hq, Hkv, G;
};

constexpr int kUnionThreads = 256;

__global__ __launch_bounds__(kUnionThreads) void attn_union_kernel(UnionParams p) {
    __shared__ uint64_t red[kUnionThreads / kWave];
    const int y = blockIdx.x;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int N = visible_clamped(p.ri, row, p.cap);
    if (N <= 0) {
        if (tid == 0) p.acnt[y] = 0;
        return;
    }
    const int64_t cur = (N - 1) / p.b;
    const int64_t words = cur / 32 + 1;
    const int64_t nc1 = N / p.b;
    uint32_t* bm0 = p.abm + (static_cast<int64_t>(row) * p.Hq + kv * p.G) * p.abm_words;
    for (int h = 0; h < p.G; ++h)
        for (int64_t w = tid; w < words; w += nt) bm0[h * p.abm_words + w] = 0u;
    __threadfence();     // zeroes are visible device-wide before the atomics below
    __syncthreads();
    for (int h = 0; h < p.G; ++h) {
        const int64_t rh = static_cast<int64_t>(row) * p.Hq + kv * p.G + h;
        const int n = min(p.n_sel[rh], p.sel_cap);
        const int32_t* lst = p.sel_blocks + rh * p.sel_cap;
        for (int j = tid; j < n; j += nt) {
            const int64_t node = lst[j];
            if (node >= 0 && node < nc1) atomicOr(bm0 + h * p.abm_words + (node >> 5), 1u << (node & 31));
        }
    }
    __threadfence();
    __syncthreads();
    const int64_t chunk = (words + nt - 1) / nt;
    const int64_t w0 = min<int64_t>(static_cast<int64_t>(tid) * chunk, words);
    const int64_t w1 = min<int64_t>(w0 + chunk, words);
    auto word_union = [&](int64_t w) -> uint32_t {
        uint32_t u = 0;
        for (int h = 0; h < p.G; ++h) u |= ld_relaxed_a(bm0 + h * p.abm_words + w);
        if (w == 0) u |= 1u;                                   // sink chunk
        if (w == (cur >> 5)) u |= 1u << (cur & 31);            // current chunk
        return u;
    };
    uint64_t cnt = 0;
    for (int64_t w = w0; w < w1; ++w) cnt += __popc(word_union(w));
    // block exclusive scan
    const uint64_t inc = wave_incl_scan_u64(cnt, lane);
    if (lane == 63) red[wave] = inc;
    __syncthreads();
    uint64_t pos = inc - cnt, total = 0;
    for (int i = 0; i < nt / kWave; ++i) {
        if (i < wave) pos += red[i];
        total += red[i];
    }
    int2* it = p.items + static_cast<int64_t>(y) * p.item_stride;
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t u = word_union(w);
        while (u) {
            const int bit = __ffs(static_cast<int>(u)) - 1;
            u &= u - 1;
            const int64_t node = w * 32 + bit;
            uint32_t mask = 0;
            for (int h = 0; h < p.G; ++h) mask |= ((ld_relaxed_a(bm0 + h * p.abm_words + w) >> bit) & 1u) << h;
            if (node == cur) mask |= kAllHeads;
            it[pos++] = make_int2(static_cast<int>(node), static_cast<int>(mask));
        }
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

template <int D, int G>
struct AttnCfg {
    static constexpr int DPL = (G <= 4) ? 16 : (G == 8 ? 8 : 4);  // score dims per lane
    static constexpr int LPT = D / DPL;                             // lanes per token (score phase)
    static constexpr int TPP = kWave / LPT;                         // tokens per pass
    static constexpr int TG = 16;                                   // tokens per group
    static constexpr int NP = TG / TPP;                             // passes per group
    static constexpr int DPV = D / kWave;                           // value dims per lane
};

template <typename KT, int D, int G>
__global__ __launch_bounds__(256) void attend_kernel(AttnParams p) {
    using C = AttnCfg<D, G>;
    constexpr int NW = 4;
    __shared__ float sm_m[NW][G], sm_l[NW][G];
    __shared__ float sm_acc[NW][G][D];

    const int split = blockIdx.x;
    const int y = blockIdx.y;
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.ri.T;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int N = visible_clamped(p.ri, row, p.cap);
    const int64_t U = p.dense ? (N + p.b - 1) / p.b : p.acnt[y];
    const int64_t i0 = U * split / p.S, i1 = U * (split + 1) / p.S;
    const int gpi = p.b >= C::TG ? p.b / C::TG : 1;          // groups per item
    const int tg = p.b >= C::TG ? C::TG : p.b;                // valid tokens per group
    const int64_t ngroups = (i1 - i0) * gpi;

    const int part = lane % C::LPT, tsub = lane / C::LPT;
    float qv[G][C::DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
        load_row<C::DPL>(p.q + (static_cast<int64_t>(row) * p.Hq + kv * G + h) * D + part * C::DPL, qv[h]);

    const KT* Kb = static_cast<const KT*>(p.K) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D;
    const KT* Vb = static_cast<const KT*>(p.V) + (static_cast<int64_t>(s) * p.Hkv + kv) * p.cap * D;
    const int2* items = p.items + static_cast<int64_t>(y) * p.item_stride;

    float m[G], l[G], acc[G][C::DPV];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int k = 0; k < C::DPV; ++k) acc[h][k] = 0.f;
    }

    for (int64_t gi = wave; gi < ngroups; gi += NW) {
        const int64_t item = i0 + gi / gpi;
        int64_t blk;
        uint32_t mask;
        if (p.dense) {
            blk = item;
            mask = kAllHeads;
        } else {
            const int2 e = items[item];
            blk = e.x;
            mask = static_cast<uint32_t>(e.y);
        }
        const int64_t t0 = blk * p.b + (gi % gpi) * C::TG;
        // ---- scores for the group's tokens ----
        float sc[C::NP][G];
        float kx[C::NP][C::DPL];
#pragma unroll
        for (int ps = 0; ps < C::NP; ++ps) {
            const int j = ps * C::TPP + tsub;
            const int64_t t = t0 + j;
            if (j < tg && t < N) load_row<C::DPL>(Kb + t * D + part * C::DPL, kx[ps]);
            else {
#pragma unroll
                for (int e = 0; e < C::DPL; ++e) kx[ps][e] = 0.f;
            }
        }
        float gmax[G];
#pragma unroll
        for (int h = 0; h < G; ++h) gmax[h] = -INFINITY;
#pragma unroll
        for (int ps = 0; ps < C::NP; ++ps) {
            const int j = ps * C::TPP + tsub;
            const int64_t t = t0 + j;
            const bool inb = (j < tg) && (t < N);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a = 0.f;
#pragma unroll
                for (int e = 0; e < C::DPL; ++e) a = fmaf(qv[h][e], kx[ps][e], a);
                a = group_sum<C::LPT>(a) * p.scale;
                const bool ok = inb && ((mask & kAllHeads) || ((mask >> h) & 1u) || t == 0);
                sc[ps][h] = ok ? a : -INFINITY;
                gmax[h] = fmaxf(gmax[h], sc[ps][h]);
            }
        }
        // ---- online softmax update ----
        float pr[C::NP][G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float gm = strided_max<C::LPT>(gmax[h]);
            const float mn = fmaxf(m[h], gm);
            const float alpha = (mn == -INFINITY) ? 1.f : expf(m[h] - mn);
            float ls = 0.f;
#pragma unroll
            for (int ps = 0; ps < C::NP; ++ps) {
                pr[ps][h] = (sc[ps][h] == -INFINITY) ? 0.f : expf(sc[ps][h] - mn);
                ls += pr[ps][h];
            }
            ls = strided_sum<C::LPT>(ls);
            l[h] = l[h] * alpha + ls;
            m[h] = mn;
#pragma unroll
            for (int k = 0; k < C::DPV; ++k) acc[h][k] *= alpha;
        }
        // ---- values ----
#pragma unroll
        for (int j = 0; j < C::TG; ++j) {
            const int64_t t = t0 + j;
            if (j >= tg || t >= N) break;      // uniform across the wave
            float v[C::DPV];
            load_few<C::DPV>(Vb + t * D + lane * C::DPV, v);
            const int src = (j % C::TPP) * C::LPT;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pj =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr[j / C::TPP][h]), src));
#pragma unroll
                for (int k = 0; k < C::DPV; ++k) acc[h][k] = fmaf(pj, v[k], acc[h][k]);
            }
        }
    }

    // ---- merge the waves, write the split's partial ----
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            sm_m[wave][h] = m[h];
            sm_l[wave][h] = l[h];
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int k = 0; k < C::DPV; ++k) sm_acc[wave][h][lane * C::DPV + k] = acc[h][k];
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

struct CombineParams {
    const float* partial;
    float* out;
    float* lse;
    int S, D;
};

__global__ __launch_bounds__(128) void attend_combine_kernel(CombineParams p) {
    const int64_t rh = blockIdx.x;
    const float* pp = p.partial + rh * p.S * (p.D + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < p.S; ++sp) M = fmaxf(M, pp[sp * (p.D + 2)]);
    for (int c = threadIdx.x; c < p.D + 1; c += blockDim.x) {
        float L = 0.f, a = 0.f;
        for (int sp = 0; sp < p.S; ++sp) {
            const float ms = pp[sp * (p.D + 2)];
            if (ms == -INFINITY) continue;
            const float f = expf(ms - M);
            L += f * pp[sp * (p.D + 2) + 1];
            if (c < p.D) a += f * pp[sp * (p.D + 2) + 2 + c];
        }
        if (c < p.D) p.out[rh * p.D + c] = (L > 0.f) ? a / L : 0.f;
        else if (p.lse) p.lse[rh] = (L > 0.f) ? M + logf(L) : -INFINITY;
    }
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename KT, int D, int G>
static void launch_attn_t(dim3 grid, const AttnParams& ap, hipStream_t st) {
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
        up.abm = reinterpret_cast<uint32_t*>(ws + lay.abm);
        up.abm_words = lay.abm_words;
        up.items = reinterpret_cast<int2*>(ws + lay.aitems);
        up.item_stride = g.nodes[0] + 2;
        up.acnt = reinterpret_cast<int32_t*>(ws + lay.acnt);
        up.cap = g.cap;
        up.b = g.b;
        up.Hq = g.Hq;
        up.Hkv = g.Hkv;
        up.G = g.G;
        hipLaunchKernelGGL(attn_union_kernel, dim3(pairs), dim3(kUnionThreads), 0, st, up);
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
    CombineParams cp{ap.partial, a.out, a.lse, lay.splits, g.D};
    hipLaunchKernelGGL(attend_combine_kernel, dim3(a.rows * g.Hq), dim3(128), 0, st, cp);
    return hipGetLastError();
}

}  // namespace zha

// pseudo.hip - compressed value summaries: the pruned subtrees' coarse share
// of the attention ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", Future Directions: compressed value summaries;
// §Key Insight, eq. (1): the output splits into the kept set's share and the
// rest's).
//
// After a route, every candidate a level's cut did not keep stands for its
// subtree as one pseudo-token: logit = its routing score + ln(the tokens of
// its span the exact part does not attend, i.e. the span less the sink and the
// current chunk), value = its value summary (the children's values pooled
// with the key summary's weights, built with the tree). zha_attend then
// returns the softmax over the exact tokens and these pseudo-tokens.
//
// Kernels:
//  * pseudo_level_kernel - per level: one wave per (run, (row, kv head)) pair
//    takes every W-th active parent of the pair (at the top every block of b
//    nodes; below, the parents some head of the group kept, then the
//    incomplete parent whose complete children are the orphans). For each
//    child and each head of the group that took it as a candidate and did not
//    keep it, the wave folds exp(logit) * value into that head's online
//    softmax state (natural log units), and writes one partial per head.
//  * pseudo_merge_kernel - per (row, query head): the exact attention's
//    (out, lse) and every partial of every level, merged by their log-sum-exp.
// The scores are the route's (the dense-by-node array; the upper-level kernel
// writes its levels' scores there when value summaries are on), the kept sets
// its bitmaps.
#include <algorithm>

#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

struct PseudoParams {
    RowInfo ri;
    const float* scores;       // dense-by-node scores, (row, head) stride nodes_total, this level at lvl_off
    const uint32_t* bitmap;    // kept bitmaps, (row, head) stride bm_words_total
    const float* vals;         // this level's value summaries [B, Hkv, nodes_l, D]
    float* partial;            // this level's partials [pairs, runs, G, D + 4]
    int64_t nodes_total, lvl_off, bm_words_total, bm_off, bm_off_up, nodes_l, cap;
    int b, lb, li, L, Hq, Hkv, T, runs;
};

template <int D, int G>
__global__ __launch_bounds__(kWave) void pseudo_level_kernel(PseudoParams p) {
    constexpr int DPL = (G <= 4) ? 16 : (G == 8 ? 8 : 4);   // dims per lane
    constexpr int LPR = D / DPL;                             // lanes per value row
    constexpr int RPP = kWave / LPR;                         // rows per pass
    const int lane = threadIdx.x;
    const int sub = lane / LPR, part = lane % LPR;
    const int run = blockIdx.x, y = blockIdx.y;              // y = (row, kv head)
    const int row = y / p.Hkv, kv = y % p.Hkv;
    const int s = row / p.T;
    const int N = clamp_visible(p.ri, row, p.cap);
    const bool top = (p.li == p.L - 1);
    const int64_t nc = static_cast<int64_t>(N) >> (p.lb * (p.li + 1));
    const int64_t nc_up = top ? 0 : (static_cast<int64_t>(N) >> (p.lb * (p.li + 2)));
    const int64_t span_lg = static_cast<int64_t>(p.lb) * (p.li + 1);
    const int64_t cur = N > 0 ? ((static_cast<int64_t>(N) - 1) >> p.lb) << p.lb : 0;   // first token of the current chunk
    const int64_t rh0 = static_cast<int64_t>(row) * p.Hq + kv * G;
    const float* sc0 = p.scores + rh0 * p.nodes_total + p.lvl_off;
    const float* vals = p.vals + (static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes_l * D;

    // online softmax state per (row slot sub, head): max, sum, this lane's dims
    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
    }
    auto bit = [&](int64_t base_off, int h, int64_t node) -> uint32_t {
        return (p.bitmap[(rh0 + h) * p.bm_words_total + base_off + (node >> 5)] >> (node & 31)) & 1u;
    };
    // the children of parent par (every head takes them where `every`, else the
    // heads whose kept set at the level above holds par)
    auto fold_parent = [&](int64_t par, bool every) {
        uint32_t takes = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) takes |= (every ? 1u : bit(p.bm_off_up, h, par)) << h;
        const int64_t c0 = par << p.lb, c1 = imin(c0 + p.b, nc);
        for (int64_t cb = c0; cb < c1; cb += RPP) {
            const int64_t c = cb + sub;
            const bool in = c < c1;
            const int64_t cc = in ? c : c1 - 1;              // a present row; its result is dropped
            float v[DPL];
            load_row<DPL>(vals + cc * D + part * DPL, v);
            // tokens of the node outside the sink and the current chunk
            const int64_t lo = cc << span_lg, hi = (cc + 1) << span_lg;
            int64_t count = (hi - lo) - (lo == 0 ? 1 : 0) - imax(0, imin(N, hi) - imax(cur, lo));
            if (lo == 0 && cur == 0) count += 1;              // the sink lies in the current chunk: once
            const float lnc = count > 0 ? logf(static_cast<float>(count)) : 0.f;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const bool pruned = in && count > 0 && ((takes >> h) & 1u) && !bit(p.bm_off, h, cc);
                if (!pruned) continue;
                const float z = sc0[static_cast<int64_t>(h) * p.nodes_total + cc] + lnc;
                const float mn = fmaxf(m[h], z);
                const float a = expf(m[h] - mn);             // 0 while nothing was folded
                const float e = expf(z - mn);
                l[h] = l[h] * a + e;
#pragma unroll
                for (int k = 0; k < DPL; ++k) acc[h][k] = fmaf(e, v[k], acc[h][k] * a);
                m[h] = mn;
            }
        }
    };

    const int W = p.runs;
    if (top) {
        const int64_t blocks = (nc + p.b - 1) >> p.lb;
        for (int64_t j = run; j < blocks; j += W) fold_parent(j, true);
    } else {
        // active parents: the complete parents some head kept, in node order, then the incomplete one
        int64_t base = 0, j = run;
        const int64_t nwords = (nc_up + 31) >> 5;
        for (int64_t w0 = 0; w0 < nwords; w0 += kWave) {
            const int64_t wd = w0 + lane;
            uint32_t u = 0;
            if (wd < nwords) {
#pragma unroll
                for (int h = 0; h < G; ++h) u |= p.bitmap[(rh0 + h) * p.bm_words_total + p.bm_off_up + wd];
                const int64_t lo = wd << 5;
                u &= nc_up - lo >= 32 ? ~0u : ((1u << (nc_up - lo)) - 1u);
            }
            const uint64_t incl = wave_scan_u64(__popc(u));
            const int64_t pass_n = static_cast<int64_t>(lane63_u64(incl));
            for (; j < base + pass_n; j += W) {
                const uint64_t rel = static_cast<uint64_t>(j - base);
                const int L = __popcll(__ballot(incl <= rel));           // the lane whose word holds it
                const uint64_t before = L ? static_cast<uint64_t>(static_cast<uint32_t>(
                    __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(incl)), L - 1))) : 0;
                uint32_t xw = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u), L));
                for (uint32_t r = static_cast<uint32_t>(rel - before); r > 0; --r) xw &= xw - 1u;
                fold_parent(((w0 + L) << 5) + __builtin_ctz(xw), false);
            }
            base += pass_n;
        }
        if (nc > (nc_up << p.lb) && j == base) fold_parent(nc_up, true);   // the orphans
    }

    // merge the row slots (lanes of equal part), then write one partial per head
    float* out = p.partial + (static_cast<int64_t>(y) * p.runs + run) * G * (D + 4);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float M = strided_max<LPR>(m[h]);
        const float f = (m[h] == -INFINITY) ? 0.f : expf(m[h] - M);
        const float Ls = strided_sum<LPR>(l[h] * f);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[h][k] = strided_sum<LPR>(acc[h][k] * f);
        float* o = out + h * (D + 4);
        if (lane == 0) {
            o[0] = M;
            o[1] = Ls;
        }
        if (lane < LPR) {
#pragma unroll
            for (int k = 0; k < DPL; ++k) o[4 + part * DPL + k] = acc[h][k];
        }
    }
}

// Per (row, query head): the exact part (out, lse; natural log) and the
// partials of every level, merged; out and lse are rewritten.
__global__ __launch_bounds__(128) void pseudo_merge_kernel(const float* __restrict__ partial, float* out, float* lse,
                                                           int L, int64_t level_stride, int runs, int G, int D, int Hq,
                                                           int Hkv) {
    const int64_t rh = blockIdx.x;
    const int row = static_cast<int>(rh / Hq), hq = static_cast<int>(rh % Hq);
    const int kv = hq / G, h = hq % G;
    const int64_t y = static_cast<int64_t>(row) * Hkv + kv;
    const int tid = threadIdx.x;
    const float l0 = lse[rh];
    float M = l0;
    for (int li = 0; li < L; ++li)
        for (int r = 0; r < runs; ++r)
            M = fmaxf(M, partial[li * level_stride + ((y * runs + r) * G + h) * (D + 4)]);
    if (M == -INFINITY) return;                               // nothing at all: out and lse stay as they are
    const float f0 = (l0 == -INFINITY) ? 0.f : expf(l0 - M);
    float S = f0;
    for (int li = 0; li < L; ++li)
        for (int r = 0; r < runs; ++r) {
            const float* pp = partial + li * level_stride + ((y * runs + r) * G + h) * (D + 4);
            if (pp[0] != -INFINITY) S += expf(pp[0] - M) * pp[1];
        }
    for (int c = tid; c < D; c += blockDim.x) {
        float a = f0 * out[rh * D + c];
        for (int li = 0; li < L; ++li)
            for (int r = 0; r < runs; ++r) {
                const float* pp = partial + li * level_stride + ((y * runs + r) * G + h) * (D + 4);
                if (pp[0] != -INFINITY) a += expf(pp[0] - M) * pp[4 + c];
            }
        out[rh * D + c] = a / S;
    }
    __syncthreads();
    if (tid == 0) lse[rh] = M + logf(S);
}

template <int D, int G>
static hipError_t launch_pseudo_t(const PseudoParams& pp, int pairs, hipStream_t st) {
    hipLaunchKernelGGL((pseudo_level_kernel<D, G>), dim3(pp.runs, pairs), dim3(kWave), 0, st, pp);
    return hipGetLastError();
}

template <int D>
static hipError_t pseudo_g(int G, const PseudoParams& pp, int pairs, hipStream_t st) {
    switch (G) {
        case 1: return launch_pseudo_t<D, 1>(pp, pairs, st);
        case 2: return launch_pseudo_t<D, 2>(pp, pairs, st);
        case 4: return launch_pseudo_t<D, 4>(pp, pairs, st);
        case 8: return launch_pseudo_t<D, 8>(pp, pairs, st);
        case 16: return launch_pseudo_t<D, 16>(pp, pairs, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_pseudo(const Geo& g, const AttendArgs& a, const float* summaries, hipStream_t st) {
    const WsLayout& lay = *a.lay;
    char* ws = a.ws;
    const int pairs = a.rows * g.Hkv;
    const int64_t level_stride = static_cast<int64_t>(pairs) * lay.pseudo_runs * g.G * (g.D + 4);
    float* partial = reinterpret_cast<float*>(ws + lay.pseudo);
    {
        ProfScope ps("pseudo", 0, st);
        for (int li = 0; li < g.L; ++li) {
            PseudoParams pp{};
            pp.ri = a.ri;
            pp.scores = reinterpret_cast<const float*>(ws + lay.scores);
            pp.bitmap = reinterpret_cast<const uint32_t*>(ws + lay.bitmap);
            pp.vals = summaries + g.val_off[li];
            pp.partial = partial + li * level_stride;
            pp.nodes_total = g.nodes_total;
            pp.lvl_off = g.sel_off[li];
            pp.bm_words_total = lay.bm_words_total;
            pp.bm_off = static_cast<int64_t>(lay.bm_off[li]);
            pp.bm_off_up = li + 1 < g.L ? static_cast<int64_t>(lay.bm_off[li + 1]) : 0;
            pp.nodes_l = g.nodes[li];
            pp.cap = g.cap;
            pp.b = g.b;
            pp.lb = g.lb;
            pp.li = li;
            pp.L = g.L;
            pp.Hq = g.Hq;
            pp.Hkv = g.Hkv;
            pp.T = a.ri.T;
            pp.runs = lay.pseudo_runs;
            const hipError_t e = (g.D == 128) ? pseudo_g<128>(g.G, pp, pairs, st) : pseudo_g<64>(g.G, pp, pairs, st);
            if (e != hipSuccess) return e;
        }
    }
    ProfScope ps("pseudo_merge", 0, st);
    hipLaunchKernelGGL(pseudo_merge_kernel, dim3(a.rows * g.Hq), dim3(128), 0, st, partial, a.out, a.lse, g.L,
                       level_stride, lay.pseudo_runs, g.G, g.D, g.Hq, g.Hkv);
    return hipGetLastError();
}

}  // namespace zha

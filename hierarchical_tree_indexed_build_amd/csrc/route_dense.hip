// route_dense.hip - node scores of whole levels for many query rows at once,
// on the fp32 matrix cores.
//
// The routing score of a node is scale * q . summary, in fp32
// ("Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
// §Routing). When a sequence routes many rows together (a causal prefill
// chunk), the rows' candidate sets cover most of each level, and scoring the
// children of kept parents one (row, head) at a time would read every summary
// row once per (row, head). Here the scores of every complete node of a level
// are one contraction per (sequence, kv head): the g query heads of the group
// and all the sequence's rows form the rows of Q, the level's summaries the
// columns, d the inner dimension. Each summary tile is then read once per 128
// query rows. A row's cut later reads only its own candidates (nodes complete
// at its position), so scores of nodes it cannot see are written and ignored.
//
// Tile: 128 query rows x 128 nodes per workgroup of 4 waves (2 x 2), each
// wave 64 x 64 = 4 x 4 blocks of v_mfma_f32_16x16x4_f32. The inner dimension
// is staged through LDS in chunks of 32 with the next chunk loaded into
// registers during the current one's products. In a chunk, the lane group
// j = lane / 16 owns dims [8j, 8j + 8) of both operands, so every lane reads
// its operands as two 16-byte LDS loads per block; the product sums the same
// dims over both operands, in an order different from the VALU dot product.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

namespace {

constexpr int kDenseThreads = 256;
constexpr int kDenseTM = 128;          // query rows per tile
constexpr int kDenseTN = 128;          // nodes per tile
constexpr int kDenseTK = 32;           // inner dims per staged chunk
constexpr int kDenseLd = kDenseTK + 4; // LDS row stride in floats (16-byte aligned, offsets the banks)

typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct DenseParams {
    const float* q;            // [rows, Hq, D]
    RowInfo ri;
    const float* summaries;
    float* scores;             // [rows, Hq, nodes_total] by node id, level offsets sc_off
    int64_t nodes_total;
    int64_t cap;
    int Hq, Hkv, G, lgG, lb, nlev;   // G = 1 << lgG <= 16
    int64_t mrows;             // T * G: contraction rows per (sequence, kv head)
    float scale;
    int li[ZHA_MAX_LEVELS];            // level (0-based) of each handled entry
    int64_t sum_off[ZHA_MAX_LEVELS];   // its summaries' element offset
    int64_t nodes[ZHA_MAX_LEVELS];     // its node slots per (sequence, kv head)
    int64_t sc_off[ZHA_MAX_LEVELS];    // its offset inside a (row, head) score array
    int tile0[ZHA_MAX_LEVELS + 1];     // first column tile of each entry; tile0[nlev] = all tiles
};

struct DenseShared {
    alignas(16) float a[kDenseTM * kDenseLd];   // query rows x staged dims
    alignas(16) float b[kDenseTN * kDenseLd];   // summary rows x staged dims
    int vis_max;
};

// Contraction row r of (sequence s, kv head kv) is query head kv*G + r % G of
// the sequence's row r / G.
__device__ __forceinline__ int64_t dense_rh(const DenseParams& p, int s, int kv, int64_t r) {
    const int64_t row = static_cast<int64_t>(s) * p.ri.T + (r >> p.lgG);
    return row * p.Hq + (static_cast<int64_t>(kv) << p.lgG) + (r & (p.G - 1));
}

template <int D>
__global__ __launch_bounds__(kDenseThreads) void route_dense_score_kernel(DenseParams p) {
    __shared__ DenseShared sh;
    float* sa = sh.a;
    float* sb = sh.b;
    const int x = blockIdx.x;
    if (x >= p.tile0[p.nlev]) return;                  // padding of the column grid
    int e = 0;
    while (x >= p.tile0[e + 1]) ++e;
    const int li = p.li[e];
    const int sk = blockIdx.z, s = sk / p.Hkv, kv = sk % p.Hkv;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kDenseTM;
    const int64_t n0 = static_cast<int64_t>(x - p.tile0[e]) * kDenseTN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // columns: nodes complete for the tile's furthest-seeing row
    if (tid == 0) sh.vis_max = 0;
    __syncthreads();
    if (tid < kDenseTM && m0 + tid < p.mrows) {
        const int row = static_cast<int>(static_cast<int64_t>(s) * p.ri.T + (m0 + tid) / p.G);
        atomicMax(&sh.vis_max, clamp_visible(p.ri, row, p.cap));
    }
    __syncthreads();
    const int64_t ncols = imin(static_cast<int64_t>(sh.vis_max) >> (p.lb * (li + 1)), p.nodes[e]);
    if (n0 >= ncols) return;                           // uniform: every thread read the same vis_max

    // staging: 128 rows x 32 dims per operand = 1024 float4, four per thread:
    // rows tr + 32u (u < 4) at dims [4 c4, 4 c4 + 4) of the chunk. Row tr + 32u
    // of Q is query row tr + 32u of the same head (32 is a multiple of G), so
    // the four A rows are one pointer apart by a fixed stride.
    constexpr int kPer = kDenseTM * kDenseTK / 4 / kDenseThreads;
    constexpr int kRowStep = kDenseThreads / (kDenseTK / 4);      // 32 rows between a thread's rows
    const int tr = tid / (kDenseTK / 4), c4 = tid % (kDenseTK / 4);
    const int st0 = tr * kDenseLd + c4 * 4;
    const int64_t mr0 = m0 + tr, nr0 = n0 + tr;
    const int na = static_cast<int>(imax(0, imin(kPer, (p.mrows - mr0 + kRowStep - 1) / kRowStep)));
    const int nb = static_cast<int>(imax(0, imin(kPer, (ncols - nr0 + kRowStep - 1) / kRowStep)));
    const float* a0 = p.q + (na ? dense_rh(p, s, kv, mr0) : 0) * D + c4 * 4;
    const int64_t a_step = (static_cast<int64_t>(kRowStep) >> p.lgG) * p.Hq * D;
    const float* b0 = p.summaries + p.sum_off[e] + ((static_cast<int64_t>(s) * p.Hkv + kv) * p.nodes[e] + nr0) * D + c4 * 4;
    f32x4_t ra[kPer], rb[kPer];
    auto fetch = [&](int c) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            ra[u] = u < na ? *reinterpret_cast<const f32x4_t*>(a0 + u * a_step + c * kDenseTK) : z;
            rb[u] = u < nb ? *reinterpret_cast<const f32x4_t*>(b0 + static_cast<int64_t>(u) * kRowStep * D + c * kDenseTK) : z;
        }
    };
    fetch(0);

    const int wm = wave >> 1, wn = wave & 1;
    const int i16 = lane & 15, j4 = lane >> 4;
    f32x4_t acc[4][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int kChunks = D / kDenseTK;
#pragma unroll 1
    for (int c = 0; c < kChunks; ++c) {
        if (c) __syncthreads();                        // the previous chunk's products are done
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            *reinterpret_cast<f32x4_t*>(sa + st0 + u * kRowStep * kDenseLd) = ra[u];
            *reinterpret_cast<f32x4_t*>(sb + st0 + u * kRowStep * kDenseLd) = rb[u];
        }
        __syncthreads();
        if (c + 1 < kChunks) fetch(c + 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x4_t fa[4], fb[4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
                fa[bi] = *reinterpret_cast<const f32x4_t*>(sa + (wm * 64 + bi * 16 + i16) * kDenseLd + j4 * 8 + kk * 4);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                fb[bj] = *reinterpret_cast<const f32x4_t*>(sb + (wn * 64 + bj * 16 + i16) * kDenseLd + j4 * 8 + kk * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int bj = 0; bj < 4; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[bi][q], fb[bj][q], acc[bi][bj], 0, 0, 0);
        }
    }

    // block (bi, bj): lane holds rows 4 * j4 + {0..3}, column i16
#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t mr = m0 + wm * 64 + bi * 16 + j4 * 4 + i;
            if (mr >= p.mrows) continue;
            float* dst = p.scores + dense_rh(p, s, kv, mr) * p.nodes_total + p.sc_off[e];
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t col = n0 + wn * 64 + bj * 16 + i16;
                if (col < ncols) dst[col] = acc[bi][bj][i] * p.scale;
            }
        }
    }
}

}  // namespace

bool dense_scores_fit(const Geo& g, int T) {
    const int64_t mt = (static_cast<int64_t>(T) * g.G + kDenseTM - 1) / kDenseTM;
    int64_t tiles = 0;
    for (int l = 0; l < g.L; ++l) tiles += (g.nodes[l] + kDenseTN - 1) / kDenseTN;
    return mt <= 65535 && static_cast<int64_t>(g.B) * g.Hkv <= 65535 && tiles + 8 <= (int64_t(1) << 30);
}

hipError_t launch_dense_scores(const Geo& g, const RowInfo& ri, const float* q, const float* summaries,
                               float* scores, int li_lo, int li_hi, hipStream_t st) {
    DenseParams p{};
    p.q = q;
    p.ri = ri;
    p.summaries = summaries;
    p.scores = scores;
    p.nodes_total = g.nodes_total;
    p.cap = g.cap;
    p.Hq = g.Hq;
    p.Hkv = g.Hkv;
    p.G = g.G;
    p.lgG = 0;
    while ((1 << p.lgG) < g.G) ++p.lgG;
    p.lb = g.lb;
    p.mrows = static_cast<int64_t>(ri.T) * g.G;
    p.scale = g.scale;
    int64_t tiles = 0;
    int n = 0;
    for (int li = li_hi; li >= li_lo; --li, ++n) {
        p.li[n] = li;
        p.sum_off[n] = g.sum_off[li];
        p.nodes[n] = g.nodes[li];
        p.sc_off[n] = g.sel_off[li];
        p.tile0[n] = static_cast<int>(tiles);
        tiles += (g.nodes[li] + kDenseTN - 1) / kDenseTN;
    }
    p.nlev = n;
    p.tile0[n] = static_cast<int>(tiles);
    if (n == 0 || tiles == 0) return hipSuccess;
    // a column tile keeps one XCD for all its row tiles (workgroups go to the
    // XCDs in turn): pad the column count to a multiple of 8
    const unsigned gx = static_cast<unsigned>((tiles + 7) / 8 * 8);
    const unsigned gy = static_cast<unsigned>((p.mrows + kDenseTM - 1) / kDenseTM);
    const dim3 grid(gx, gy, static_cast<unsigned>(g.B * g.Hkv));
    ProfScope ps("route_dense", 0, st);
    if (g.D == 128)
        hipLaunchKernelGGL(route_dense_score_kernel<128>, grid, dim3(kDenseThreads), 0, st, p);
    else
        hipLaunchKernelGGL(route_dense_score_kernel<64>, grid, dim3(kDenseThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace zha

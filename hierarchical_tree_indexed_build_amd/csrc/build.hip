// build.hip - summary reduction for the ZHA tree and its incremental append path.
//
// A node of level l summarises its b children (raw keys at level 1, level l-1
// summaries above): weights softmax(scale * r_l . c_j) and summary
// sum_j w_j c_j, i.e. the attention of the level's reference query over the
// children with the children as keys and values ("Subquadratic Attention with
// a Hierarchical Tree-Structured Indexer", §Tree Construction). Only complete
// nodes are built, each exactly once; appends complete nodes in the same
// device function, so append-built and build-built summaries are bit-identical.
//
// Mapping: one wave64 per node. Up to 64 bf16 children (level 1, the bulk of
// the bytes): each 16-byte load instruction reads whole child rows (a row
// spread over d/8 lanes) and the node stays in registers for the dot products
// with r and the weighted sum. fp32 children (levels above): pass 1 gives each
// child row 64/b lanes for the dot products and pass 2 walks the rows again
// (re-read from L1/L2) with d/64 dimensions a lane. More children (b = 128,
// 256): each lane owns b/64 rows, and pass 2 walks them again. The node is
// read from HBM once and every store is a coalesced 4*d-byte row.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

template <int N, typename T>
__device__ __forceinline__ void load_n(const T* __restrict__ p, float (&x)[N]) {
    if constexpr (N <= 4) load_few<N>(p, x);
    else load_row<N>(p, x);
}

// More children than lanes (b = 128, 256): lane l owns child rows l, l + 64,
// ...; each row's dot product with r is taken 8 elements at a time (r is the
// same for every lane). The softmax and the weighted sum are as below.
template <typename CT, int B, int D, bool VAL = false>
__device__ __forceinline__ void reduce_node_wide(const CT* __restrict__ ch, const float* __restrict__ r,
                                                 float scale, float* __restrict__ out, int lane,
                                                 const CT* __restrict__ vch = nullptr, float* __restrict__ vout = nullptr) {
    constexpr int RPL = B / kWave;   // child rows per lane
    constexpr int DPL = D / kWave;   // dimensions per lane in pass 2
    float z[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) z[i] = 0.f;
#pragma unroll 2
    for (int e0 = 0; e0 < D; e0 += 8) {
        float rr[8];
        load_row<8>(r + e0, rr);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float x[8];
            load_row<8>(ch + static_cast<int64_t>(i * kWave + lane) * D + e0, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) z[i] = fmaf(rr[e], x[e], z[i]);
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        z[i] *= scale;
        mloc = fmaxf(mloc, z[i]);
    }
    const float m = group_max<kWave>(mloc);
    float w[RPL], sloc = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        w[i] = expf(z[i] - m);
        sloc += w[i];
    }
    const float tot = group_sum<kWave>(sloc);

    float acc[DPL], vacc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = vacc[k] = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
#pragma unroll 8
        for (int j = 0; j < kWave; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[i]), j));
            float v[DPL];
            load_n<DPL>(ch + static_cast<int64_t>(i * kWave + j) * D + lane * DPL, v);
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, v[k], acc[k]);
            if constexpr (VAL) {
                float y[DPL];
                load_n<DPL>(vch + static_cast<int64_t>(i * kWave + j) * D + lane * DPL, y);
#pragma unroll
                for (int k = 0; k < DPL; ++k) vacc[k] = fmaf(wj, y[k], vacc[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        out[lane * DPL + k] = acc[k] / tot;
        if constexpr (VAL) vout[lane * DPL + k] = vacc[k] / tot;
    }
}

// Up to 64 bf16 children (raw keys). Each load instruction covers whole child rows: a row is
// read by LPW lanes, 16 bytes each (EPW elements), so one instruction reads
// RPI = 64 / LPW complete rows, and lane (sub, col) holds column block col of
// rows sub, sub + RPI, ... The node's rows stay in registers for both passes:
// the dot products with r are summed over each row's LPW lanes, and the
// weighted sum is formed per lane over its rows and then summed over the RPI
// lanes that share a column block.
template <typename CT, int B, int D, bool VAL = false>
__device__ __forceinline__ void reduce_node_rows(const CT* __restrict__ ch, const float* __restrict__ r,
                                                 float scale, float* __restrict__ out, int lane,
                                                 const CT* __restrict__ vch = nullptr, float* __restrict__ vout = nullptr) {
    constexpr int EPW = 16 / static_cast<int>(sizeof(CT));   // elements in one 16-byte piece
    constexpr int LPW = D / EPW;                             // lanes per row
    constexpr int RPI = kWave / LPW;                         // rows per load instruction
    constexpr int NI = (B + RPI - 1) / RPI;                  // rows per lane
    static_assert(LPW >= 1 && LPW <= kWave && kWave % LPW == 0, "a row spans a power-of-two lane group");
    const int col = lane % LPW, sub = lane / LPW;

    // the pieces as loaded (16 bytes a row), widened where they are used
    uint4 x[NI], y[VAL ? NI : 1];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int row = i * RPI + sub;
        const int rw = row < B ? row : B - 1;                // a present row; its weight is 0
        x[i] = *reinterpret_cast<const uint4*>(ch + rw * D + col * EPW);
        if constexpr (VAL) y[i] = *reinterpret_cast<const uint4*>(vch + rw * D + col * EPW);
    }
    auto elem = [](const uint4& q, int e) -> float {
        const uint32_t w = e / (EPW / 4) == 0 ? q.x : e / (EPW / 4) == 1 ? q.y : e / (EPW / 4) == 2 ? q.z : q.w;
        if constexpr (sizeof(CT) == 2) return (e & 1) ? bf16_hi(w) : bf16_lo(w);
        else return __uint_as_float(w);
    };
    float rr[EPW];
    load_n<EPW>(r + col * EPW, rr);
    float z[NI], mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < EPW; ++e) t = fmaf(rr[e], elem(x[i], e), t);
        z[i] = fast_group_sum<LPW>(t) * scale;
        if (i * RPI + sub < B) mloc = fmaxf(mloc, z[i]);
    }
    // pass 2 widens the pieces again rather than keeping pass 1's floats live
#pragma unroll
    for (int i = 0; i < NI; ++i) __asm__ volatile("" : "+v"(x[i].x), "+v"(x[i].y), "+v"(x[i].z), "+v"(x[i].w));
    const float m = strided_max<LPW>(mloc);
    float w[NI], sloc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        w[i] = (i * RPI + sub < B) ? expf(z[i] - m) : 0.f;
        sloc += w[i];
    }
    const float tot = strided_sum<LPW>(sloc);
    float acc[EPW], vacc[EPW];
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[e] = vacc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
            acc[e] = fmaf(w[i], elem(x[i], e), acc[e]);
            if constexpr (VAL) vacc[e] = fmaf(w[i], elem(y[i], e), vacc[e]);
        }
#pragma unroll
    for (int e = 0; e < EPW; ++e) {
        acc[e] = strided_sum<LPW>(acc[e]);
        if constexpr (VAL) vacc[e] = strided_sum<LPW>(vacc[e]);
    }
    if (sub == 0) {
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
            out[col * EPW + e] = acc[e] / tot;
            if constexpr (VAL) vout[col * EPW + e] = vacc[e] / tot;
        }
    }
}

// Up to 64 fp32 children (summaries of the level below): pass 1 gives each
// child row 64/b lanes, each holding d*b/64 contiguous elements, for the b
// dot products with r; pass 2 gives each lane d/64 dimensions and walks the b
// rows (re-read from L1/L2) to form the weighted sum. It holds fewer registers
// than the row layout with 512-byte rows, which matters in the 1024-thread
// append kernel.
template <typename CT, int B, int D, bool VAL = false>
__device__ __forceinline__ void reduce_node_narrow(const CT* __restrict__ ch, const float* __restrict__ r,
                                                   float scale, float* __restrict__ out, int lane,
                                                   const CT* __restrict__ vch = nullptr, float* __restrict__ vout = nullptr) {
    constexpr int LPR = kWave / B;   // lanes per child row
    constexpr int EPL = D / LPR;     // elements per lane in pass 1
    constexpr int DPL = D / kWave;   // dimensions per lane in pass 2
    const int row = lane / LPR, part = lane % LPR;

    float x[EPL], rr[EPL];
    load_n<EPL>(ch + row * D + part * EPL, x);
    load_n<EPL>(r + part * EPL, rr);
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) z = fmaf(rr[e], x[e], z);
    z = group_sum<LPR>(z) * scale;
    const float m = group_max<kWave>(z);
    const float w = expf(z - m);
    const float tot = group_sum<kWave>(w) * (1.0f / LPR);   // each row is held by LPR lanes

    float acc[DPL], vacc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = vacc[k] = 0.f;
#pragma unroll 8
    for (int j = 0; j < B; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j * LPR));
        float v[DPL];
        load_n<DPL>(ch + j * D + lane * DPL, v);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, v[k], acc[k]);
        if constexpr (VAL) {
            float y[DPL];
            load_n<DPL>(vch + j * D + lane * DPL, y);
#pragma unroll
            for (int k = 0; k < DPL; ++k) vacc[k] = fmaf(wj, y[k], vacc[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        out[lane * DPL + k] = acc[k] / tot;
        if constexpr (VAL) vout[lane * DPL + k] = vacc[k] / tot;
    }
}

// The node's key summary; with VAL also its value summary (the children's
// values vch pooled with the same weights) into vout.
template <typename CT, int B, int D, bool VAL = false>
__device__ __forceinline__ void reduce_node_wave(const CT* __restrict__ ch, const float* __restrict__ r,
                                                 float scale, float* __restrict__ out, int lane,
                                                 const CT* __restrict__ vch = nullptr, float* __restrict__ vout = nullptr) {
    if constexpr (B > kWave) reduce_node_wide<CT, B, D, VAL>(ch, r, scale, out, lane, vch, vout);
    else if constexpr (sizeof(CT) == 2) reduce_node_rows<CT, B, D, VAL>(ch, r, scale, out, lane, vch, vout);
    else reduce_node_narrow<CT, B, D, VAL>(ch, r, scale, out, lane, vch, vout);
}

// ---- tangent scoring ----
// One tangent of a node: the first-order expansion, at reference query r, of
// the log-sum-exp of its children's estimates. Child j offers Rc tangents
// (key row (j Rc + r') of ch, offset choff[j Rc + r']; raw keys with no offset
// at level 1) and enters with the one largest at r (lowest r' on ties):
// z_j = scale r . key + off, w = softmax(z), key = sum_j w_j key_j, offset =
// LSE(z) - scale r . key ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", §Tree Construction: k_hat_r, b_hat_r).
template <typename CT, int B, int D>
__device__ __forceinline__ void tangent_node_narrow(const CT* __restrict__ ch, const float* __restrict__ choff, int Rc,
                                                    const float* __restrict__ r, float scale, float* __restrict__ okey,
                                                    float* __restrict__ ooff, int lane) {
    // no implicit contraction: the append kernel (child count known to be 1)
    // and the build kernel must round every step alike (explicit fmaf only)
#pragma clang fp contract(off)
    constexpr int LPR = kWave / B;   // lanes per child
    constexpr int EPL = D / LPR;     // elements per lane in pass 1
    constexpr int DPL = D / kWave;   // dimensions per lane in pass 2
    const int row = lane / LPR, part = lane % LPR;
    float rr[EPL];
    load_n<EPL>(r + part * EPL, rr);
    float z = -INFINITY;
    int rs = 0;
    for (int rc = 0; rc < Rc; ++rc) {
        float x[EPL];
        load_n<EPL>(ch + static_cast<int64_t>(row * Rc + rc) * D + part * EPL, x);
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) t = fmaf(rr[e], x[e], t);
        t = group_sum<LPR>(t) * scale;
        if (choff) t += choff[row * Rc + rc];
        if (rc == 0 || t > z) {       // strict: the lowest index keeps a tie
            z = t;
            rs = rc;
        }
    }
    const float m = group_max<kWave>(z);
    const float w = expf(z - m);
    const float tot = group_sum<kWave>(w) * (1.0f / LPR);   // each child is held by LPR lanes
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll 4
    for (int j = 0; j < B; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j * LPR));
        const int rj = __builtin_amdgcn_readlane(rs, j * LPR);
        float v[DPL];
        load_n<DPL>(ch + static_cast<int64_t>(j * Rc + rj) * D + lane * DPL, v);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, v[k], acc[k]);
    }
    float rq[DPL];
    load_n<DPL>(r + lane * DPL, rq);
    float dq = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        acc[k] = acc[k] / tot;
        okey[lane * DPL + k] = acc[k];
        dq = fmaf(rq[k], acc[k], dq);
    }
    dq = group_sum<kWave>(dq);
    if (lane == 0) *ooff = (m + logf(tot)) - scale * dq;
}

// The same with more children than lanes: lane l owns children l, l + 64, ...
template <typename CT, int B, int D>
__device__ __forceinline__ void tangent_node_wide(const CT* __restrict__ ch, const float* __restrict__ choff, int Rc,
                                                  const float* __restrict__ r, float scale, float* __restrict__ okey,
                                                  float* __restrict__ ooff, int lane) {
    // no implicit contraction: the append kernel (child count known to be 1)
    // and the build kernel must round every step alike (explicit fmaf only)
#pragma clang fp contract(off)
    constexpr int RPL = B / kWave;
    constexpr int DPL = D / kWave;
    float z[RPL];
    int rs[RPL];
    for (int rc = 0; rc < Rc; ++rc) {
        float t[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) t[i] = 0.f;
#pragma unroll 2
        for (int e0 = 0; e0 < D; e0 += 8) {
            float rr[8];
            load_row<8>(r + e0, rr);
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                float x[8];
                load_row<8>(ch + static_cast<int64_t>((i * kWave + lane) * Rc + rc) * D + e0, x);
#pragma unroll
                for (int e = 0; e < 8; ++e) t[i] = fmaf(rr[e], x[e], t[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float v = t[i] * scale;
            if (choff) v += choff[(i * kWave + lane) * Rc + rc];
            if (rc == 0 || v > z[i]) {
                z[i] = v;
                rs[i] = rc;
            }
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) mloc = fmaxf(mloc, z[i]);
    const float m = group_max<kWave>(mloc);
    float w[RPL], sloc = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        w[i] = expf(z[i] - m);
        sloc += w[i];
    }
    const float tot = group_sum<kWave>(sloc);
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
#pragma unroll 4
        for (int j = 0; j < kWave; ++j) {
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[i]), j));
            const int rj = __builtin_amdgcn_readlane(rs[i], j);
            float v[DPL];
            load_n<DPL>(ch + static_cast<int64_t>((i * kWave + j) * Rc + rj) * D + lane * DPL, v);
#pragma unroll
            for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, v[k], acc[k]);
        }
    }
    float rq[DPL];
    load_n<DPL>(r + lane * DPL, rq);
    float dq = 0.f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
        acc[k] = acc[k] / tot;
        okey[lane * DPL + k] = acc[k];
        dq = fmaf(rq[k], acc[k], dq);
    }
    dq = group_sum<kWave>(dq);
    if (lane == 0) *ooff = (m + logf(tot)) - scale * dq;
}

template <typename CT, int B, int D>
__device__ __forceinline__ void tangent_node_wave(const CT* __restrict__ ch, const float* __restrict__ choff, int Rc,
                                                  const float* __restrict__ r, float scale, float* __restrict__ okey,
                                                  float* __restrict__ ooff, int lane) {
    if constexpr (B > kWave) tangent_node_wide<CT, B, D>(ch, choff, Rc, r, scale, okey, ooff, lane);
    else tangent_node_narrow<CT, B, D>(ch, choff, Rc, r, scale, okey, ooff, lane);
}

struct BuildParams {
    const void* children;      // level-1: K; else summaries of level l-1
    float* out;                // summaries of level l
    const float* r;            // ref_q + (l-1)*Hkv*D
    const int32_t* seq_lens;
    int64_t child_rows;        // row slots per (batch, kv) in `children` (capacity or nodes[l-2])
    int64_t out_rows;          // node slots per (batch, kv) at level l
    int64_t span;              // tokens per node at level l
    int64_t cap;
    int Hkv, BH, slots, mode, t_new;
    float scale;
    // tangent scoring: R tangents per node, Rc per child (1 at level 1); offsets of the children
    // (null at level 1) and of this level; r points at the level's [Hkv, R, D] reference queries
    const float* child_off;
    float* out_off;
    int R, Rc;
    // value summaries: the children's values (V at level 1, value summaries above) and this level's
    const void* values;
    float* out_val;
};

enum { kBuildPlain = 0, kBuildTangent = 1, kBuildValues = 2 };

enum { kModeBuild = 0, kModeAppend = 1 };

template <typename CT, int B, int D, int MODE>
__global__ __launch_bounds__(256) void build_level_kernel(BuildParams p) {
    constexpr bool TAN = MODE == kBuildTangent;
    const int lane = threadIdx.x & (kWave - 1);
    const int RW = TAN ? p.R : 1;                        // waves per node: one per tangent
    const int64_t total = static_cast<int64_t>(p.BH) * p.slots * RW;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
    for (int64_t wv = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave; wv < total;
         wv += stride) {
        const int64_t nw = wv / RW;
        const int rr = static_cast<int>(wv % RW);
        const int bh = static_cast<int>(nw / p.slots);
        const int64_t k = nw % p.slots;
        const int s = bh / p.Hkv, h = bh % p.Hkv;
        const int64_t len = imin(imax(p.seq_lens[s], 0), p.cap);
        int64_t i, hi;
        if (p.mode == kModeBuild) {
            i = k;
            hi = len / p.span;
        } else {
            if (p.seq_lens[s] < 0 || len + p.t_new > p.cap) continue;
            i = len / p.span + k;
            hi = (len + p.t_new) / p.span;
        }
        if (i >= hi) continue;
        if constexpr (TAN) {
            const int64_t c0 = (static_cast<int64_t>(bh) * p.child_rows + i * B) * p.Rc;   // first child row
            const CT* ch = static_cast<const CT*>(p.children) + c0 * D;
            const float* co = p.child_off ? p.child_off + c0 : nullptr;
            const int64_t orow = (static_cast<int64_t>(bh) * p.out_rows + i) * p.R + rr;
            tangent_node_wave<CT, B, D>(ch, co, p.Rc, p.r + (static_cast<int64_t>(h) * p.R + rr) * D, p.scale,
                                        p.out + orow * D, p.out_off + orow, lane);
        } else if constexpr (MODE == kBuildValues) {
            const int64_t c0 = (bh * p.child_rows + i * B) * D;
            const int64_t o0 = (bh * p.out_rows + i) * D;
            reduce_node_wave<CT, B, D, true>(static_cast<const CT*>(p.children) + c0, p.r + h * D, p.scale, p.out + o0,
                                             lane, static_cast<const CT*>(p.values) + c0, p.out_val + o0);
        } else {
            const CT* ch = static_cast<const CT*>(p.children) + (bh * p.child_rows + i * B) * D;
            float* o = p.out + (bh * p.out_rows + i) * D;
            reduce_node_wave<CT, B, D>(ch, p.r + h * D, p.scale, o, lane);
        }
    }
}

// ----------------------------------------------------------------------------
// append: copy rows (multi-token path)
// ----------------------------------------------------------------------------
struct CopyParams {
    char* K;
    char* V;
    const char* kn;
    const char* vn;
    const int32_t* seq_lens;
    uint32_t* status;
    int64_t cap;
    int64_t row_bytes;   // D * element size
    int Hkv, t_new;
};

__global__ __launch_bounds__(256) void append_rows_kernel(CopyParams p) {
    const int bh = blockIdx.y;
    const int s = bh / p.Hkv;
    const int64_t len = p.seq_lens[s];
    if (len < 0 || len + p.t_new > p.cap) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && bh % p.Hkv == 0) atomicOr(p.status, ZHA_DEV_APPEND_OVERFLOW);
        return;
    }
    const int64_t nbytes = p.row_bytes * p.t_new;       // a multiple of 16
    const int64_t dst0 = (static_cast<int64_t>(bh) * p.cap + len) * p.row_bytes;
    const int64_t src0 = static_cast<int64_t>(bh) * p.t_new * p.row_bytes;
    for (int64_t o = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 16; o < nbytes;
         o += static_cast<int64_t>(gridDim.x) * blockDim.x * 16) {
        *reinterpret_cast<uint4*>(p.K + dst0 + o) = *reinterpret_cast<const uint4*>(p.kn + src0 + o);
        *reinterpret_cast<uint4*>(p.V + dst0 + o) = *reinterpret_cast<const uint4*>(p.vn + src0 + o);
    }
}

__global__ void advance_seq_kernel(int32_t* seq_lens, int B, int t_new, int64_t cap) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < B && seq_lens[s] >= 0 && seq_lens[s] + static_cast<int64_t>(t_new) <= cap) seq_lens[s] += t_new;
}

// ----------------------------------------------------------------------------
// append: fused single-launch path for short appends (decode)
// One workgroup per sequence, one wave per kv head: copy the new rows, then
// complete nodes level by level (each level reads the nodes the wave just
// wrote, after a fence), then advance seq_lens once every head is done.
// ----------------------------------------------------------------------------
struct FusedParams {
    char* K;
    char* V;
    const char* kn;
    const char* vn;
    int32_t* seq_lens;
    const float* ref_q;
    float* summaries;
    uint32_t* status;
    int64_t cap;
    int64_t nodes[ZHA_MAX_LEVELS];
    int64_t sum_off[ZHA_MAX_LEVELS];
    int64_t span[ZHA_MAX_LEVELS];
    int64_t bias_off[ZHA_MAX_LEVELS];   // tangent scoring: each level's offsets in the summary buffer
    int64_t val_off[ZHA_MAX_LEVELS];    // value summaries: each level's in the summary buffer
    int Hkv, L, t_new, R;
    bool tangent, values;
    float scale;
};

template <typename KT, int B, int D, int MODE>
__global__ __launch_bounds__(512) void append_fused_kernel(FusedParams p) {
    constexpr bool TAN = MODE == kBuildTangent, VAL = MODE == kBuildValues;
    const int s = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave, nwaves = blockDim.x / kWave;
    const int64_t len = p.seq_lens[s];
    if (len < 0 || len + p.t_new > p.cap) {
        if (threadIdx.x == 0) atomicOr(p.status, ZHA_DEV_APPEND_OVERFLOW);
        return;
    }
    constexpr int64_t row_bytes = static_cast<int64_t>(D) * sizeof(KT);
    for (int h = wave; h < p.Hkv; h += nwaves) {
        const int64_t bh = static_cast<int64_t>(s) * p.Hkv + h;
        const int64_t nbytes = row_bytes * p.t_new;
        const int64_t dst0 = (bh * p.cap + len) * row_bytes;
        const int64_t src0 = bh * p.t_new * row_bytes;
        for (int64_t o = lane * 16; o < nbytes; o += kWave * 16) {
            // both loads before either store (the compiler cannot tell the
            // new rows from the cache apart)
            const uint4 kx = *reinterpret_cast<const uint4*>(p.kn + src0 + o);
            const uint4 vx = *reinterpret_cast<const uint4*>(p.vn + src0 + o);
            *reinterpret_cast<uint4*>(p.K + dst0 + o) = kx;
            *reinterpret_cast<uint4*>(p.V + dst0 + o) = vx;
        }
        for (int l = 0; l < p.L; ++l) {
            const int64_t lo = len / p.span[l], hi = (len + p.t_new) / p.span[l];
            if (lo >= hi) break;      // nothing completes here, so nothing above either
            // what the wave wrote last (the new rows, or the level below's
            // summaries) is read back next, by other lanes; a step that
            // completes no node needs no fence
            __threadfence();
            float* lvl = p.summaries + p.sum_off[l];
            if constexpr (TAN) {
                const float* r0 = p.ref_q + (static_cast<int64_t>(l) * p.Hkv + h) * p.R * D;
                for (int64_t i = lo; i < hi; ++i) {
                    for (int rr = 0; rr < p.R; ++rr) {
                        const int64_t orow = (bh * p.nodes[l] + i) * p.R + rr;
                        float* ok = lvl + orow * D;
                        float* oo = p.summaries + p.bias_off[l] + orow;
                        if (l == 0) {
                            const KT* ch = reinterpret_cast<const KT*>(p.K) + (bh * p.cap + i * B) * D;
                            tangent_node_wave<KT, B, D>(ch, nullptr, 1, r0 + rr * D, p.scale, ok, oo, lane);
                        } else {
                            const int64_t c0 = (bh * p.nodes[l - 1] + i * B) * p.R;
                            tangent_node_wave<float, B, D>(p.summaries + p.sum_off[l - 1] + c0 * D,
                                                           p.summaries + p.bias_off[l - 1] + c0, p.R, r0 + rr * D,
                                                           p.scale, ok, oo, lane);
                        }
                    }
                }
            } else {
                const float* r = p.ref_q + (static_cast<int64_t>(l) * p.Hkv + h) * D;
                for (int64_t i = lo; i < hi; ++i) {
                    float* o = lvl + (bh * p.nodes[l] + i) * D;
                    float* vo = VAL ? p.summaries + p.val_off[l] + (bh * p.nodes[l] + i) * D : nullptr;
                    if (l == 0) {
                        const int64_t c0 = (bh * p.cap + i * B) * D;
                        reduce_node_wave<KT, B, D, VAL>(reinterpret_cast<const KT*>(p.K) + c0, r, p.scale, o, lane,
                                                        reinterpret_cast<const KT*>(p.V) + c0, vo);
                    } else {
                        const int64_t c0 = (bh * p.nodes[l - 1] + i * B) * D;
                        reduce_node_wave<float, B, D, VAL>(p.summaries + p.sum_off[l - 1] + c0, r, p.scale, o, lane,
                                                           VAL ? p.summaries + p.val_off[l - 1] + c0 : nullptr, vo);
                    }
                }
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) p.seq_lens[s] = static_cast<int32_t>(len + p.t_new);
}

// ----------------------------------------------------------------------------
// launchers
// ----------------------------------------------------------------------------
template <typename CT, int B, int D>
static hipError_t launch_level_t(const BuildParams& bp, int64_t total_waves, int level, hipStream_t st) {
    const bool tan = bp.out_off != nullptr;
    const int64_t waves = total_waves * (tan ? bp.R : 1);
    const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 16384);
    if (blocks <= 0) return hipSuccess;
    ProfScope ps("build_level", level, st);
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (tan) hipLaunchKernelGGL((build_level_kernel<CT, B, D, kBuildTangent>), grid, block, 0, st, bp);
    else if (bp.out_val) hipLaunchKernelGGL((build_level_kernel<CT, B, D, kBuildValues>), grid, block, 0, st, bp);
    else hipLaunchKernelGGL((build_level_kernel<CT, B, D, kBuildPlain>), grid, block, 0, st, bp);
    return hipGetLastError();
}

template <typename CT, int D>
static hipError_t dispatch_b(int b, const BuildParams& bp, int64_t tw, int lv, hipStream_t st) {
    switch (b) {
        case 2: return launch_level_t<CT, 2, D>(bp, tw, lv, st);
        case 4: return launch_level_t<CT, 4, D>(bp, tw, lv, st);
        case 8: return launch_level_t<CT, 8, D>(bp, tw, lv, st);
        case 16: return launch_level_t<CT, 16, D>(bp, tw, lv, st);
        case 32: return launch_level_t<CT, 32, D>(bp, tw, lv, st);
        case 64: return launch_level_t<CT, 64, D>(bp, tw, lv, st);
        case 128: return launch_level_t<CT, 128, D>(bp, tw, lv, st);
        case 256: return launch_level_t<CT, 256, D>(bp, tw, lv, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_build_level(const Geo& g, int level, const void* K, const void* V, const float* ref_q,
                              float* summaries, const int32_t* seq_lens, int mode, int t_new, hipStream_t st) {
    BuildParams bp{};
    const int l = level - 1;
    bp.children = (level == 1) ? K : static_cast<const void*>(summaries + g.sum_off[l - 1]);
    bp.out = summaries + g.sum_off[l];
    bp.r = ref_q + static_cast<int64_t>(l) * g.Hkv * g.R * g.D;
    bp.R = g.R;
    bp.Rc = (level == 1) ? 1 : g.R;
    bp.child_off = (g.tangent && level > 1) ? summaries + g.bias_off[l - 1] : nullptr;
    bp.out_off = g.tangent ? summaries + g.bias_off[l] : nullptr;
    bp.values = g.vsum ? ((level == 1) ? V : static_cast<const void*>(summaries + g.val_off[l - 1])) : nullptr;
    bp.out_val = g.vsum ? summaries + g.val_off[l] : nullptr;
    bp.seq_lens = seq_lens;
    bp.child_rows = (level == 1) ? g.cap : g.nodes[l - 1];
    bp.out_rows = g.nodes[l];
    bp.span = g.span[l];
    bp.cap = g.cap;
    bp.Hkv = g.Hkv;
    bp.BH = g.B * g.Hkv;
    bp.mode = mode;
    bp.t_new = t_new;
    bp.scale = g.scale;
    if (mode == kModeBuild) {
        bp.slots = static_cast<int>(g.nodes[l]);
    } else {
        bp.slots = static_cast<int>((t_new + g.span[l] - 1) / g.span[l] + 1);
    }
    if (bp.slots <= 0) return hipSuccess;
    const int64_t tw = static_cast<int64_t>(bp.BH) * bp.slots;
    const bool f32 = (level > 1) || g.kv_dtype == ZHA_KV_F32;
    if (g.D == 128) {
        return f32 ? dispatch_b<float, 128>(g.b, bp, tw, level, st) : dispatch_b<uint16_t, 128>(g.b, bp, tw, level, st);
    }
    return f32 ? dispatch_b<float, 64>(g.b, bp, tw, level, st) : dispatch_b<uint16_t, 64>(g.b, bp, tw, level, st);
}

hipError_t launch_append_rows(const Geo& g, void* K, void* V, const void* k_new, const void* v_new, int t_new,
                              const int32_t* seq_lens, uint32_t* status, hipStream_t st) {
    CopyParams cp{};
    cp.K = static_cast<char*>(K);
    cp.V = static_cast<char*>(V);
    cp.kn = static_cast<const char*>(k_new);
    cp.vn = static_cast<const char*>(v_new);
    cp.seq_lens = seq_lens;
    cp.status = status;
    cp.cap = g.cap;
    cp.row_bytes = static_cast<int64_t>(g.D) * (g.kv_dtype == ZHA_KV_BF16 ? 2 : 4);
    cp.Hkv = g.Hkv;
    cp.t_new = t_new;
    const int64_t chunks = (cp.row_bytes * t_new / 16 + 255) / 256;
    const unsigned gx = static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(chunks, 1), 1024));
    ProfScope ps("append_rows", 0, st);
    hipLaunchKernelGGL(append_rows_kernel, dim3(gx, g.B * g.Hkv), dim3(256), 0, st, cp);
    return hipGetLastError();
}

hipError_t launch_advance_seq(const Geo& g, int32_t* seq_lens, int t_new, hipStream_t st) {
    ProfScope ps("advance_seq", 0, st);
    hipLaunchKernelGGL(advance_seq_kernel, dim3((g.B + 255) / 256), dim3(256), 0, st, seq_lens, g.B, t_new, g.cap);
    return hipGetLastError();
}

template <typename KT, int B, int D>
static hipError_t launch_fused_t(const FusedParams& fp, int B_, int Hkv, hipStream_t st) {
    const int waves = std::min(Hkv, 8);             // more kv heads: a wave takes several in turn
    ProfScope ps("append_fused", 0, st);
    const dim3 grid(B_), block(waves * kWave);
    if (fp.tangent) hipLaunchKernelGGL((append_fused_kernel<KT, B, D, kBuildTangent>), grid, block, 0, st, fp);
    else if (fp.values) hipLaunchKernelGGL((append_fused_kernel<KT, B, D, kBuildValues>), grid, block, 0, st, fp);
    else hipLaunchKernelGGL((append_fused_kernel<KT, B, D, kBuildPlain>), grid, block, 0, st, fp);
    return hipGetLastError();
}

template <typename KT, int D>
static hipError_t fused_b(int b, const FusedParams& fp, int B_, int Hkv, hipStream_t st) {
    switch (b) {
        case 2: return launch_fused_t<KT, 2, D>(fp, B_, Hkv, st);
        case 4: return launch_fused_t<KT, 4, D>(fp, B_, Hkv, st);
        case 8: return launch_fused_t<KT, 8, D>(fp, B_, Hkv, st);
        case 16: return launch_fused_t<KT, 16, D>(fp, B_, Hkv, st);
        case 32: return launch_fused_t<KT, 32, D>(fp, B_, Hkv, st);
        case 64: return launch_fused_t<KT, 64, D>(fp, B_, Hkv, st);
        case 128: return launch_fused_t<KT, 128, D>(fp, B_, Hkv, st);
        case 256: return launch_fused_t<KT, 256, D>(fp, B_, Hkv, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_append_fused(const Geo& g, void* K, void* V, const void* k_new, const void* v_new, int t_new,
                               int32_t* seq_lens, const float* ref_q, float* summaries, uint32_t* status,
                               hipStream_t st) {
    FusedParams fp{};
    fp.K = static_cast<char*>(K);
    fp.V = static_cast<char*>(V);
    fp.kn = static_cast<const char*>(k_new);
    fp.vn = static_cast<const char*>(v_new);
    fp.seq_lens = seq_lens;
    fp.ref_q = ref_q;
    fp.summaries = summaries;
    fp.status = status;
    fp.cap = g.cap;
    for (int l = 0; l < g.L; ++l) {
        fp.nodes[l] = g.nodes[l];
        fp.sum_off[l] = g.sum_off[l];
        fp.span[l] = g.span[l];
        fp.bias_off[l] = g.bias_off[l];
        fp.val_off[l] = g.val_off[l];
    }
    fp.R = g.R;
    fp.tangent = g.tangent;
    fp.values = g.vsum;
    fp.Hkv = g.Hkv;
    fp.L = g.L;
    fp.t_new = t_new;
    fp.scale = g.scale;
    const bool bf = g.kv_dtype == ZHA_KV_BF16;
    if (g.D == 128) return bf ? fused_b<uint16_t, 128>(g.b, fp, g.B, g.Hkv, st) : fused_b<float, 128>(g.b, fp, g.B, g.Hkv, st);
    return bf ? fused_b<uint16_t, 64>(g.b, fp, g.B, g.Hkv, st) : fused_b<float, 64>(g.b, fp, g.B, g.Hkv, st);
}

}  // namespace zha

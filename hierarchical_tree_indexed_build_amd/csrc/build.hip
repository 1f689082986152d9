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
// Mapping: one wave64 per node. Pass 1 gives each child row 64/b lanes, each
// holding d*b/64 contiguous elements, for the b dot products with r; pass 2
// gives each lane d/64 dimensions and walks the b rows (re-read from L1/L2) to
// form the weighted sum, so the node is read from HBM once and every store is a
// coalesced 4*d-byte row.
#include "zha_device.h"
#include "zha_internal.h"

namespace zha {

template <int N, typename T>
__device__ __forceinline__ void load_n(const T* __restrict__ p, float (&x)[N]) {
    if constexpr (N <= 4) load_few<N>(p, x);
    else load_row<N>(p, x);
}

template <typename CT, int B, int D>
__device__ __forceinline__ void reduce_node_wave(const CT* __restrict__ ch, const float* __restrict__ r,
                                                 float scale, float* __restrict__ out, int lane) {
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

    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int j = 0; j < B; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j * LPR));
        float v[DPL];
        load_n<DPL>(ch + j * D + lane * DPL, v);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wj, v[k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < DPL; ++k) out[lane * DPL + k] = acc[k] / tot;
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
};

enum { kModeBuild = 0, kModeAppend = 1 };

template <typename CT, int B, int D>
__global__ __launch_bounds__(256) void build_level_kernel(BuildParams p) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t total = static_cast<int64_t>(p.BH) * p.slots;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * (blockDim.x / kWave);
    for (int64_t wv = static_cast<int64_t>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave; wv < total;
         wv += stride) {
        const int bh = static_cast<int>(wv / p.slots);
        const int64_t k = wv % p.slots;
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
        const CT* ch = static_cast<const CT*>(p.children) + (bh * p.child_rows + i * B) * D;
        float* o = p.out + (bh * p.out_rows + i) * D;
        reduce_node_wave<CT, B, D>(ch, p.r + h * D, p.scale, o, lane);
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
    int Hkv, L, t_new;
    float scale;
};

template <typename KT, int B, int D>
__global__ __launch_bounds__(1024) void append_fused_kernel(FusedParams p) {
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
            const float* r = p.ref_q + (static_cast<int64_t>(l) * p.Hkv + h) * D;
            for (int64_t i = lo; i < hi; ++i) {
                float* o = lvl + (bh * p.nodes[l] + i) * D;
                if (l == 0) {
                    const KT* ch = reinterpret_cast<const KT*>(p.K) + (bh * p.cap + i * B) * D;
                    reduce_node_wave<KT, B, D>(ch, r, p.scale, o, lane);
                } else {
                    const float* ch = p.summaries + p.sum_off[l - 1] + (bh * p.nodes[l - 1] + i * B) * D;
                    reduce_node_wave<float, B, D>(ch, r, p.scale, o, lane);
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
    const int64_t blocks = std::min<int64_t>((total_waves + 3) / 4, 16384);
    if (blocks <= 0) return hipSuccess;
    ProfScope ps("build_level", level, st);
    hipLaunchKernelGGL((build_level_kernel<CT, B, D>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, bp);
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
    }
    return hipErrorInvalidValue;
}

hipError_t launch_build_level(const Geo& g, int level, const void* K, const float* ref_q, float* summaries,
                              const int32_t* seq_lens, int mode, int t_new, hipStream_t st) {
    BuildParams bp{};
    const int l = level - 1;
    bp.children = (level == 1) ? K : static_cast<const void*>(summaries + g.sum_off[l - 1]);
    bp.out = summaries + g.sum_off[l];
    bp.r = ref_q + static_cast<int64_t>(l) * g.Hkv * g.D;
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
    const int waves = std::min(Hkv, 16);
    ProfScope ps("append_fused", 0, st);
    hipLaunchKernelGGL((append_fused_kernel<KT, B, D>), dim3(B_), dim3(waves * kWave), 0, st, fp);
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
    }
    fp.Hkv = g.Hkv;
    fp.L = g.L;
    fp.t_new = t_new;
    fp.scale = g.scale;
    const bool bf = g.kv_dtype == ZHA_KV_BF16;
    if (g.D == 128) return bf ? fused_b<uint16_t, 128>(g.b, fp, g.B, g.Hkv, st) : fused_b<float, 128>(g.b, fp, g.B, g.Hkv, st);
    return bf ? fused_b<uint16_t, 64>(g.b, fp, g.B, g.Hkv, st) : fused_b<float, 64>(g.b, fp, g.B, g.Hkv, st);
}

}  // namespace zha

// zha_device.h - device helpers for the gfx950 kernels of libzha:
// wave64 reductions with a fixed butterfly order (deterministic results),
// exact bf16 widening and vectorised row loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zha {

// Integer min / max written out, so 64-bit operands stay in integer registers.
__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Load N consecutive elements (N a multiple of 4) of a row into fp32 registers.
// Element type uint16_t means bf16 bits, widened exactly.
template <int N>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ p, float (&x)[N]) {
    static_assert(N % 8 == 0 || N == 4, "bf16 rows load in groups of 8 (or 4)");
    if constexpr (N % 8 == 0) {
        const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            const uint4 u = v[i];
            x[8 * i + 0] = bf16_lo(u.x); x[8 * i + 1] = bf16_hi(u.x);
            x[8 * i + 2] = bf16_lo(u.y); x[8 * i + 3] = bf16_hi(u.y);
            x[8 * i + 4] = bf16_lo(u.z); x[8 * i + 5] = bf16_hi(u.z);
            x[8 * i + 6] = bf16_lo(u.w); x[8 * i + 7] = bf16_hi(u.w);
        }
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    }
}

template <int N>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&x)[N]) {
    static_assert(N % 4 == 0, "fp32 rows load in groups of 4");
    const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const float4 u = v[i];
        x[4 * i + 0] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
    }
}

// A row of an fp32 matrix shared by LPR lanes, interleaved: lane `part` holds
// float4 number part, part + LPR, part + 2 LPR, ... of the row, so each load
// instruction covers LPR * 16 contiguous bytes of every row it touches. `p`
// points at the lane's first float4 (row + 4 * part).
template <int N, int LPR>
__device__ __forceinline__ void load_row_il(const float* __restrict__ p, float (&x)[N]) {
    static_assert(N % 4 == 0, "fp32 rows load in groups of 4");
    const float4* v = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const float4 u = v[i * LPR];
        x[4 * i + 0] = u.x; x[4 * i + 1] = u.y; x[4 * i + 2] = u.z; x[4 * i + 3] = u.w;
    }
}

// Load M (1, 2 or 4) consecutive elements.
template <int M>
__device__ __forceinline__ void load_few(const uint16_t* __restrict__ p, float (&x)[M]) {
    if constexpr (M == 1) {
        x[0] = __uint_as_float(uint32_t(*p) << 16);
    } else if constexpr (M == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        x[0] = bf16_lo(w); x[1] = bf16_hi(w);
    } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    }
}
template <int M>
__device__ __forceinline__ void load_few(const float* __restrict__ p, float (&x)[M]) {
    if constexpr (M == 1) {
        x[0] = *p;
    } else if constexpr (M == 2) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        x[0] = u.x; x[1] = u.y;
    } else {
        const float4 u = *reinterpret_cast<const float4*>(p);
        x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    }
}

// Load N consecutive elements, N in {1, 2, 4} or a multiple of 8 (bf16) / 4 (fp32).
template <int N, typename T>
__device__ __forceinline__ void load_vec(const T* __restrict__ p, float (&x)[N]) {
    if constexpr (N <= 2 || (N == 4 && sizeof(T) == 2)) load_few<N>(p, x);
    else load_row<N>(p, x);
}

// Sum / max over aligned groups of W lanes (W a power of two <= 64). Every lane
// of a group ends with the group's result; the combination order is fixed.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
// Sum over aligned groups of W <= 16 lanes with DPP lane permutes (one VALU op
// per step: swap within pairs, within quads, mirror within 8, mirror within 16).
// Every lane of a group ends with the group's sum; the order is fixed.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16, "DPP groups of 1..16 lanes");
    if constexpr (W >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (W >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if constexpr (W >= 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if constexpr (W >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Sum over aligned groups of any W <= 64 lanes: DPP inside rows of 16, then
// cross-row exchanges.
template <int W>
__device__ __forceinline__ float fast_group_sum(float v) {
    if constexpr (W <= 16) {
        return dpp_group_sum<W>(v);
    } else {
        v = dpp_group_sum<16>(v);
#pragma unroll
        for (int o = 16; o < W; o <<= 1) v += __shfl_xor(v, o, 64);
        return v;
    }
}

// Reduce over lanes that differ only in the bits of [LO, 64): sums across the
// lane index's high part, keeping the low part (lanes with equal lane % LO).
template <int LO>
__device__ __forceinline__ float strided_sum(float v) {
#pragma unroll
    for (int o = 32; o >= LO; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
template <int LO>
__device__ __forceinline__ float strided_max(float v) {
#pragma unroll
    for (int o = 32; o >= LO; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, 64);
        v += (static_cast<uint64_t>(hi) << 32) | lo;
    }
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele, fixed order).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t lo = __shfl_up(static_cast<uint32_t>(v), o, 64);
        const uint32_t hi = __shfl_up(static_cast<uint32_t>(v >> 32), o, 64);
        if (lane >= o) v += (static_cast<uint64_t>(hi) << 32) | lo;
    }
    return v;
}

// Inclusive scans over the 64 lanes of a wave in lane order, built from DPP
// row shifts (within rows of 16 lanes) and row broadcasts (lane 15 of a row to
// the next row, lane 31 to rows 2 and 3): six VALU steps, no LDS traffic.
// Lane 63 ends with the wave's total (or maximum).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_scan_add_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, ROW_MASK, 0xF, false);
    return v + ((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
    v = dpp_scan_add_u64<0x111, 0xF>(v);   // row_shr:1
    v = dpp_scan_add_u64<0x112, 0xF>(v);   // row_shr:2
    v = dpp_scan_add_u64<0x114, 0xF>(v);   // row_shr:4
    v = dpp_scan_add_u64<0x118, 0xF>(v);   // row_shr:8
    v = dpp_scan_add_u64<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_scan_add_u64<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_scan_max_f(float v) {
    const int t = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false);
    return fmaxf(v, __int_as_float(t));
}
__device__ __forceinline__ float wave_scan_max_f(float v) {
    v = dpp_scan_max_f<0x111, 0xF>(v);
    v = dpp_scan_max_f<0x112, 0xF>(v);
    v = dpp_scan_max_f<0x114, 0xF>(v);
    v = dpp_scan_max_f<0x118, 0xF>(v);
    v = dpp_scan_max_f<0x142, 0xA>(v);
    v = dpp_scan_max_f<0x143, 0xC>(v);
    return v;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_scan_max_u32(uint32_t v) {
    const uint32_t t = __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, ROW_MASK, 0xF, false);
    return v > t ? v : t;
}
__device__ __forceinline__ uint32_t wave_scan_max_u32(uint32_t v) {
    v = dpp_scan_max_u32<0x111, 0xF>(v);
    v = dpp_scan_max_u32<0x112, 0xF>(v);
    v = dpp_scan_max_u32<0x114, 0xF>(v);
    v = dpp_scan_max_u32<0x118, 0xF>(v);
    v = dpp_scan_max_u32<0x142, 0xA>(v);
    v = dpp_scan_max_u32<0x143, 0xC>(v);
    return v;
}
__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Order-preserving map of a float to uint32 that sorts DESCENDING scores first:
// a < b as keys  <=>  score a > score b.
__device__ __forceinline__ uint32_t desc_key(float s) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}
__device__ __forceinline__ float desc_key_to_float(uint32_t k) {
    const uint32_t asc = ~k;
    const uint32_t u = (asc & 0x80000000u) ? (asc & 0x7fffffffu) : ~asc;
    return __uint_as_float(u);
}

// Mask of the top n bits of a 32-bit word, for n in [0, 32]. Uses a 64-bit
// shift so that no shift amount ever reaches the operand width.
__device__ __forceinline__ uint32_t top_bits_mask(int n) {
    return static_cast<uint32_t>(0xffffffff00000000ull >> n);
}

// Fixed-point softmax mass: exp(s - m) in fp32 scaled by 2^40 and truncated.
// Integer sums of these are exact and independent of the summation order.
__device__ __forceinline__ uint64_t mass_fx(float s, float m) {
    const float e = expf(s - m);
    return static_cast<uint64_t>(e * 0x1p40f);
}

}  // namespace zha

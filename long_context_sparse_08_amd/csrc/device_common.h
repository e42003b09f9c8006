// device_common.h — storage formats, vector loads and wave helpers shared by the libcsa kernels.
// Target: CDNA4 (gfx950), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace csa {

// DT_KV_FP8_BF16: KV rows of c values stored as c - 64 e4m3 bytes, then 64 bf16 values
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3, DT_KV_FP8_BF16 = 4 };

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ scalar formats
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn byte -> fp32 (exact).  exponent bias 7; e == 0 is subnormal (mant * 2^-9);
// S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, mant = b & 7u;
    float v = (e == 0) ? (float)mant * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (mant << 20));
    if (e == 15u && mant == 7u) v = __builtin_nanf("");
    return (b & 0x80u) ? -v : v;
}

// fp32 -> OCP e4m3fn byte: round to nearest, ties to even, saturating at +-448 (finite input).
// The grid's quantum at |x| is 2^(floor(log2|x|) - 3) for normal values (exponent >= -6) and
// 2^-9 below; dividing by it is exact, rintf rounds to nearest even.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float f) {
    const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
    const float a = fminf(fabsf(f), 448.f);
    const int ea = (int)((__float_as_uint(a) >> 23) & 255u) - 127;
    const float q = __uint_as_float((uint32_t)((ea > -6 ? ea : -6) - 3 + 127) << 23);
    const float r = rintf(a / q) * q;
    if (r == 0.f) return sign;
    const uint32_t rb = __float_as_uint(r);
    const int er = (int)((rb >> 23) & 255u) - 127;
    if (er < -6) return sign | (uint32_t)(r * 512.f);   // subnormal: r = mant * 2^-9
    return sign | ((uint32_t)(er + 7) << 3) | ((rb >> 20) & 7u);
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 and +0 map together.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ 8-wide loads / stores
// Load 8 consecutive elements (element offset `i`, 8-aligned) of dtype DT as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t i, float (&v)[8]) {
    if constexpr (DT == DT_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else if constexpr (DT == DT_BF16) {
        uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    } else {
        uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + i);
        const uint32_t w[2] = {r.x, r.y};
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * j + e] = e4m3_to_f32((w[j] >> (8 * e)) & 0xffu);
    }
}

// Load one element of dtype DT as float.
template <int DT>
__device__ __forceinline__ float load1(const void* __restrict__ base, int64_t i) {
    if constexpr (DT == DT_F32) return static_cast<const float*>(base)[i];
    else if constexpr (DT == DT_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
    else return e4m3_to_f32(static_cast<const uint8_t*>(base)[i]);
}

// Store 8 floats at element offset i (8-aligned) as DT (F32, BF16 or FP8).
template <int DT>
__device__ __forceinline__ void store8(void* __restrict__ base, int64_t i, const float (&v)[8]) {
    if constexpr (DT == DT_F32) {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + i);
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else if constexpr (DT == DT_FP8) {
        uint2 r;
        r.x = f32_to_e4m3_rne(v[0]) | (f32_to_e4m3_rne(v[1]) << 8) | (f32_to_e4m3_rne(v[2]) << 16) |
              (f32_to_e4m3_rne(v[3]) << 24);
        r.y = f32_to_e4m3_rne(v[4]) | (f32_to_e4m3_rne(v[5]) << 8) | (f32_to_e4m3_rne(v[6]) << 16) |
              (f32_to_e4m3_rne(v[7]) << 24);
        *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + i) = r;
    } else {
        uint4 r;
        r.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
        r.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
        r.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
        r.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + i) = r;
    }
}

template <int DT>
__device__ __forceinline__ void store1(void* __restrict__ base, int64_t i, float v) {
    if constexpr (DT == DT_F32) static_cast<float*>(base)[i] = v;
    else static_cast<uint16_t*>(base)[i] = (uint16_t)f32_to_bf16_rne(v);
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// ------------------------------------------------------------------ VALU-only wave scans
// Cross-lane steps through DPP and the gfx950 lane swaps: no LDS round trip (a __shfl is a
// ds_bpermute), so a chain of them costs a few cycles per step instead of an LDS latency.

// x of the lane the DPP control CTRL names, in the rows of ROW_MASK; 0 elsewhere and where
// the named lane is outside the row
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes: row_shr 1, 2, 4, 8 scan each row of 16 lanes,
// row_bcast:15 adds row 0's total to row 1 (and row 2's to row 3), row_bcast:31 adds the
// total of rows 0-1 to rows 2-3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u32<0x111, 0xF>(x);
    x += dpp_u32<0x112, 0xF>(x);
    x += dpp_u32<0x114, 0xF>(x);
    x += dpp_u32<0x118, 0xF>(x);
    x += dpp_u32<0x142, 0xA>(x);
    x += dpp_u32<0x143, 0xC>(x);
    return x;
}

// max / min over the wave, every lane gets it: lane ^ 1, lane ^ 2 (quad_perm), the other quad
// of 8 (row_half_mirror), the other half of 16 (row_mirror), then lanes l ^ 16 and l ^ 32
// (permlane16 / permlane32 swaps return the pair {x[l], x[l ^ 16 or 32]})
template <bool MAX>
__device__ __forceinline__ float wave_ext(float x) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    auto dp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    x = op(x, dp(x, std::integral_constant<int, 0xB1>{}));
    x = op(x, dp(x, std::integral_constant<int, 0x4E>{}));
    x = op(x, dp(x, std::integral_constant<int, 0x141>{}));
    x = op(x, dp(x, std::integral_constant<int, 0x140>{}));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Number of compressed entries (ratio r) visible to the query at absolute position p:
// entry s is visible iff r*(s+1)-1 <= p.
__device__ __forceinline__ int64_t visible_entries(int64_t p, int r, int64_t N) {
    int64_t v = (p + 1) / r;
    if (p + 1 < 0) v = 0;
    return v < N ? v : N;
}

}  // namespace csa

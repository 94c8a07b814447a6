// Device helpers shared by the scan kernels (gfx950).
#pragma once

#include "sdm_internal.h"

#include <utility>

namespace sdm {

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), each index a constant expression
template <class F, int... Js>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, Js...>)
{
    (f(std::integral_constant<int, Js>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kOOB = 0xFFFFFFF0u; // a buffer offset past every buffer's end

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void st128(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, off, 0, 0);
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding)
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// x + (x of lane ^ D), identical in both lanes of every pair (an exactly
// commutative add): DPP row_ror:8 for D = 8, the gfx950 permlane swaps for 16
// and 32, ds_bpermute below 8.
template <int D> __device__ __forceinline__ uint32_t partner32(uint32_t u)
{
    static_assert(D == 8, "DPP partner only for D = 8");
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false);
}
template <int D> __device__ __forceinline__ float bfly(float x)
{
    if constexpr (D < 8) {
        return x + __shfl_xor(x, D);
    } else if constexpr (D == 8) {
        return x + __uint_as_float(partner32<8>(__float_as_uint(x)));
    } else if constexpr (D == 16) {
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(s[0]) + __uint_as_float(s[1]);
    } else {
        static_assert(D == 32, "butterfly distance");
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
}
template <int D> __device__ __forceinline__ double bfly(double x)
{
    if constexpr (D < 8) {
        return x + __shfl_xor(x, D);
    } else {
        const uint64_t b = (uint64_t)__double_as_longlong(x);
        const uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
        if constexpr (D == 8) {
            const uint64_t p = ((uint64_t)partner32<8>(hi) << 32) | partner32<8>(lo);
            return x + __longlong_as_double((long long)p);
        } else {
            uint32_t a_lo, b_lo, a_hi, b_hi;
            if constexpr (D == 16) {
                const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
                const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
                a_lo = sl[0]; b_lo = sl[1]; a_hi = sh[0]; b_hi = sh[1];
            } else {
                static_assert(D == 32, "butterfly distance");
                const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
                const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
                a_lo = sl[0]; b_lo = sl[1]; a_hi = sh[0]; b_hi = sh[1];
            }
            return __longlong_as_double((long long)(((uint64_t)a_hi << 32) | a_lo)) +
                   __longlong_as_double((long long)(((uint64_t)b_hi << 32) | b_lo));
        }
    }
}

// Four per-lane values, each summed over the 8 lane groups of a wave (LPS = 8):
// one DPP stage, then two transposing permlane16 swaps and one permlane32 swap,
// so that row r (lanes 16r..16r+15) ends with the total of value r.  Every value
// goes through the same tree ((g0+g1)+(g2+g3))+((g4+g5)+(g6+g7)).
__device__ __forceinline__ float reduce4_to_rows(float v0, float v1, float v2, float v3)
{
    v0 = bfly<8>(v0);
    v1 = bfly<8>(v1);
    v2 = bfly<8>(v2);
    v3 = bfly<8>(v3);
    const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
    const float t01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]); // rows 0,2: v0; rows 1,3: v1
    const float t23 = __uint_as_float(s23[0]) + __uint_as_float(s23[1]); // rows 0,2: v2; rows 1,3: v3
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(t01), __float_as_uint(t23), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Two values through the same tree: row r ends with the total of value r & 1 (the
// last level pairs each row's partial with itself two rows away, which is the
// tree's last addition for that value; addition is commutative, so every total
// is the one reduce4_to_rows gives).
__device__ __forceinline__ float reduce2_to_rows(float v0, float v1)
{
    v0 = bfly<8>(v0);
    v1 = bfly<8>(v1);
    const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const float t01 = __uint_as_float(s01[0]) + __uint_as_float(s01[1]); // rows 0,2: v0; rows 1,3: v1
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(t01), __float_as_uint(t01), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// The float whose nearest-even bf16 rounding is that of the double x (one
// rounding of x to bf16).  x rounds to float
// first; that can only go wrong when the float lands exactly on a bf16 tie while
// x was not on it, and then moving the float one ulp towards x settles the tie
// the way x lies (rounding is monotone and the bf16 tie is a float value).
__device__ __forceinline__ float settle_bf16_tie(double x)
{
    const float f = (float)x;
    uint32_t u = __float_as_uint(f);
    if ((u & 0xFFFFu) == 0x8000u) {
        const double fd = (double)f;
        if (fd != x)
            u = (__builtin_fabs(fd) > __builtin_fabs(x)) ? u - 1u : u + 1u;
    }
    return __uint_as_float(u);
}

// reduce4_to_rows for doubles: the same tree, the permlane swaps applied to
// both 32-bit halves of every value.
__device__ __forceinline__ void swap_rows_d(double a, double b, bool rows32, double& x, double& y)
{
    const uint64_t ua = (uint64_t)__double_as_longlong(a), ub = (uint64_t)__double_as_longlong(b);
    uint32_t xl, yl, xh, yh;
    if (rows32) {
        const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)ua, (uint32_t)ub, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32), false, false);
        xl = lo[0]; yl = lo[1]; xh = hi[0]; yh = hi[1];
    } else {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)ua, (uint32_t)ub, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(ua >> 32), (uint32_t)(ub >> 32), false, false);
        xl = lo[0]; yl = lo[1]; xh = hi[0]; yh = hi[1];
    }
    x = __longlong_as_double((long long)(((uint64_t)xh << 32) | xl));
    y = __longlong_as_double((long long)(((uint64_t)yh << 32) | yl));
}

__device__ __forceinline__ double reduce2_to_rows(double v0, double v1)
{
    v0 = bfly<8>(v0);
    v1 = bfly<8>(v1);
    double a, b;
    swap_rows_d(v0, v1, false, a, b);
    const double t01 = a + b; // rows 0,2: v0; rows 1,3: v1
    swap_rows_d(t01, t01, true, a, b);
    return a + b;
}

__device__ __forceinline__ double reduce4_to_rows(double v0, double v1, double v2, double v3)
{
    v0 = bfly<8>(v0);
    v1 = bfly<8>(v1);
    v2 = bfly<8>(v2);
    v3 = bfly<8>(v3);
    double a, b;
    swap_rows_d(v0, v1, false, a, b);
    const double t01 = a + b; // rows 0,2: v0; rows 1,3: v1
    swap_rows_d(v2, v3, false, a, b);
    const double t23 = a + b; // rows 0,2: v2; rows 1,3: v3
    swap_rows_d(t01, t23, true, a, b);
    return a + b;
}

} // namespace sdm

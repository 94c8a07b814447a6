// State cells and cross-lane sums shared by the staged scan and the decode step.
//
// A workgroup owns 128 bytes of every slot row; lane (g, e) of a wave holds the
// 16 bytes e of two slot positions, the wave's 8 lane groups g covering 8
// positions at a time.  A float32 state is updated in float32; a bf16 state is
// updated in double and rounded once to bf16 when stored.
#pragma once

#include "scan_device.h"

namespace sdm {

// The 16 bytes of state a lane owns in one slot segment: 4 float32 or 8 bf16
// values, unpacked to float32 for the arithmetic and packed back with one
// nearest-even rounding per value.
template <class ST> struct Cell;
template <> struct Cell<float> {
    static constexpr int E = 4;
    using CT = float; // type of the write arithmetic
    __device__ static uint4 pack(const float (&x)[4])
    {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
    __device__ static void unpack(const uint4& u, float (&x)[4])
    {
        x[0] = __uint_as_float(u.x);
        x[1] = __uint_as_float(u.y);
        x[2] = __uint_as_float(u.z);
        x[3] = __uint_as_float(u.w);
    }
};
template <> struct Cell<uint16_t> {
    static constexpr int E = 8;
    using CT = double;
    __device__ static void unpack(const uint4& u, float (&x)[8])
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(w[i]);
            x[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    // v_cvt_pk_bf16_f32: nearest-even, NaN stays a quiet NaN
    __device__ static uint32_t pack2(float lo, float hi)
    {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
    }
    // One rounding of each double to bf16: through float, which is exact unless
    // the float lands on a bf16 tie (1 in 2^16); only then, for the whole wave,
    // the tie is settled the way the double lies.
    __device__ static uint4 pack(const double (&x)[8])
    {
        float f[8];
        bool tie = false;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            f[q] = (float)x[q];
            tie |= (__float_as_uint(f[q]) & 0xFFFFu) == 0x8000u;
        }
        if (__builtin_amdgcn_ballot_w64(tie) != 0u) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
                f[q] = settle_bf16_tie(x[q]);
        }
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
};

// A lane's 8 bytes of a bf16 state in a 64-byte slot segment (4 values), for
// memories too few to fill the device with 128-byte segments: the same
// arithmetic and rounding as Cell<uint16_t>, held in the low half of a uint4.
template <class ST> struct CellHalf;
template <> struct CellHalf<uint16_t> {
    static constexpr int E = 4;
    using CT = double;
    __device__ static void unpack(const uint4& u, float (&x)[4])
    {
        x[0] = bf16_lo(u.x);
        x[1] = bf16_hi(u.x);
        x[2] = bf16_lo(u.y);
        x[3] = bf16_hi(u.y);
    }
    __device__ static uint4 pack(const double (&x)[4])
    {
        float f[4];
        bool tie = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[q] = (float)x[q];
            tie |= (__float_as_uint(f[q]) & 0xFFFFu) == 0x8000u;
        }
        if (__builtin_amdgcn_ballot_w64(tie) != 0u) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                f[q] = settle_bf16_tie(x[q]);
        }
        return make_uint4(Cell<uint16_t>::pack2(f[0], f[1]), Cell<uint16_t>::pack2(f[2], f[3]), 0u, 0u);
    }
};

// A lane's 4 bytes of a bf16 state in a 32-byte slot segment (2 values), for a
// single long sequence: twice the workgroups of 64-byte segments again, the same
// arithmetic and rounding, held in the low word of a uint4.
template <class ST> struct CellQuarter;
template <> struct CellQuarter<uint16_t> {
    static constexpr int E = 2;
    using CT = double;
    __device__ static void unpack(const uint4& u, float (&x)[2])
    {
        x[0] = bf16_lo(u.x);
        x[1] = bf16_hi(u.x);
    }
    __device__ static uint4 pack(const double (&x)[2])
    {
        float f[2];
        bool tie = false;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f[q] = (float)x[q];
            tie |= (__float_as_uint(f[q]) & 0xFFFFu) == 0x8000u;
        }
        if (__builtin_amdgcn_ballot_w64(tie) != 0u) {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                f[q] = settle_bf16_tie(x[q]);
        }
        return make_uint4(Cell<uint16_t>::pack2(f[0], f[1]), 0u, 0u, 0u);
    }
};

// Totals over the 4 waves of the per-wave partials ([wave][el][E] values of
// type X) of element lane el, in the same order in every lane.
template <int E, class X>
__device__ __forceinline__ void sum_waves(const float4* part, int el, X (&t)[E])
{
    const X* p = reinterpret_cast<const X*>(part);
#pragma unroll
    for (int q = 0; q < E; ++q)
        t[q] = (p[(0 * 8 + el) * E + q] + p[(1 * 8 + el) * E + q]) + (p[(2 * 8 + el) * E + q] + p[(3 * 8 + el) * E + q]);
}

// The wave's totals over its 8 lane groups of the E values of every lane, left
// in part ([wave][el][E] values of type X); lanes l and l ^ 8 write the same.
template <int E, class X>
__device__ __forceinline__ void reduce_to_part(const X (&v)[E], float4* part, int wave, int el, int lane)
{
    X* p = reinterpret_cast<X*>(part);
    if constexpr (E == 2) {
        // rows 0 and 2 end with the total of value 0, rows 1 and 3 with value 1's
        const X t = reduce2_to_rows(v[0], v[1]);
        p[(wave * 8 + el) * E + ((lane >> 4) & 1)] = t;
    } else {
#pragma unroll
        for (int c = 0; c < E / 4; ++c) {
            // row r (lanes 16r .. 16r+15) ends with the total of value 4c + r
            const X t = reduce4_to_rows(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
            p[(wave * 8 + el) * E + 4 * c + (lane >> 4)] = t;
        }
    }
}

// The arithmetic of one element, shared by every kernel that writes or reads
// the state so that they agree to the last bit: each fused multiply-add is
// written out and the compiler may fuse nothing else here.
// A lane's share of the prediction, for its two write slots (values m, weights w).
template <class CT>
__device__ __forceinline__ CT predict2(CT al, CT w0, float m0, CT w1, float m1)
{
#pragma clang fp contract(off)
    if constexpr (sizeof(CT) == 8) // w m is exact in double: the decay comes out of the sum
        return al * __builtin_fma(w1, (CT)m1, w0 * (CT)m0);
    else
        return __builtin_fmaf(w1, al * m1, w0 * (al * m0));
}
// The delta-rule step beta * (v - vhat).
template <class CT> __device__ __forceinline__ CT delta(CT be, float v, CT vh)
{
#pragma clang fp contract(off)
    return be * ((CT)v - vh);
}
// A write slot after the update: its decayed value plus its weight times the step.
template <class CT> __device__ __forceinline__ CT updated(CT al, float m, CT w, CT dlt)
{
#pragma clang fp contract(off)
    if constexpr (sizeof(CT) == 8)
        return __builtin_fma(w, dlt, al * (CT)m);
    else
        return __builtin_fmaf(w, dlt, al * m);
}
// A lane's share of the read, for its two read slots.
__device__ __forceinline__ float read2(float r0, float q0, float r1, float q1)
{
#pragma clang fp contract(off)
    return __builtin_fmaf(r1, q1, r0 * q0);
}

} // namespace sdm

// Internal declarations shared by the gfx950 kernels and the host API of libsdm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, nearest with ties to even; NaN stays a (quiet) NaN,
// values past the largest finite bfloat16 round to infinity.
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return bf16_rne(lo) | (bf16_rne(hi) << 16); }

// order-preserving map from float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t ordered_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// buffer resources: raw (byte-addressed) buffers; an access past num_records
// reads zeros and drops writes instead of faulting.
// ---------------------------------------------------------------------------

constexpr int kBufferWord3 = 0x00020000; // gfx9-family raw buffer format word

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// ---------------------------------------------------------------------------
// launchers (all asynchronous on `stream`; they return the launch status)
// ---------------------------------------------------------------------------

// Half scores of the rows of q ([rows_per_head * H, dk], row r belongs to head r % H)
// against subkeys [H, 2, S, dh]: scores [rows, 2, S] float32.
hipError_t launch_pk_score(const void* q, const void* subkeys, float* scores, long rows_per_head, int H,
                           int S, int dh, bool in_bf16, hipStream_t stream);

// Per-half top-k, outer-sum top-W and softmax weights for `rows` rows of scores.
hipError_t launch_pk_topk(const float* scores, int32_t* idx, float* wt, long rows, int S, int k, int W,
                          hipStream_t stream);

// The scan's plan: one 16-byte record per (b, h, t, position) packing the write
// and read slot ids, their weights, where in the scan's LDS ring a slot written
// too recently to be read from memory is found, and whether a store is superseded.
// Also writes (alpha, beta) of every token next to each other for the scan.
size_t plan_bytes(int B, int H, int T, int W); // records followed by the (alpha, beta) pairs
hipError_t launch_sdm_plan(const int32_t* idx_w, const float* wt_w, const int32_t* idx_r, const float* wt_r,
                           const float* alpha, const float* beta, uint4* plan, float2* ab, int B, int T, int H, int W,
                           hipStream_t stream);

struct ScanArgs {
    const uint4* plan;  // [B*H, T, W] records
    const float2* ab;   // [B*H, T] (alpha, beta)
    const void* v;
    void* mem;
    float* out;
    int B, T, H, d, W;
    long N;
};

// Scan launch geometry chosen for a shape.
struct ScanPlan {
    int lps;       // lanes sharing one slot (16 bytes each)
    int rw;        // slot positions per lane
    int waves;     // waves per workgroup
    int lookahead; // tokens between a slot read's issue and its use
    int grid;      // workgroups
    int lds;       // dynamic LDS bytes
};

bool plan_scan(int B, int H, int d, int W, bool state_bf16, ScanPlan* plan);
hipError_t launch_sdm_scan(const ScanArgs& a, const ScanPlan& plan, bool state_bf16, bool in_bf16,
                           hipStream_t stream);

} // namespace sdm

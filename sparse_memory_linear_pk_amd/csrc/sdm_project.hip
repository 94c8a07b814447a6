// sdm_project: the layer's input projections, on the matrix cores.
//
// The SDM blog post (section "How does SDM work?", its "Write & Read"
// subsection) projects the token embedding to the write keys and, separately,
// to the query of the read; the value and the two gates of the gated delta
// rule come from the same embedding.  For every row r (token) of a call and
// every output column c of the H heads' blocks [wq | rq | v | alpha | beta]
// (C = 2 dk + d + 2 columns per head):
//   y[r, c] = sum_k x[r, k] * w[c, k]
// with x [rows, D] and w [H*C, D] in bf16 (w has an output's D weights
// contiguous, the usual out x in layout of a linear layer).  Both operands are
// therefore contiguous along the reduction, and one kernel computes the whole
// product on v_mfma_f32_32x32x16_bf16 with float32 accumulation; its epilogue
// stores each column where it belongs: wq, rq and v rounded to bf16 (nearest
// even), alpha and beta as sigmoid(y + bias) in float32.
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 tile of y, each wave a
// 64 x 64 quarter (2 x 2 MFMA tiles of 32 x 32); the k loop stages 64-wide
// slices of both operands through LDS (rows padded to 144 bytes, so the 16
// lanes of a 128-bit LDS read phase hit distinct banks), double-buffered so
// that the next slice's global loads are in flight during this slice's MFMAs.
//
// sdm_broadcast_memory copies a learned initial memory [H, N, d] into each of
// the B sequences' memories.
#include "sdm_internal.h"

namespace sdm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8; // bf16 elements per LDS row (144 bytes)

struct ProjArgs {
    const uint16_t* x;  // [R, D]
    const uint16_t* w;  // [NC, D]
    const float* bias;  // [H, 2]
    uint16_t* wq;       // [R, H, dk]
    uint16_t* rq;       // [R, H, dk]
    uint16_t* v;        // [R, H, d]
    float* alpha;       // [R, H]
    float* beta;        // [R, H]
    int R, D, H, dk, d;
};

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    const bf16x2v_t b = __builtin_convertvector((f32x2v_t){f, 0.f}, bf16x2v_t); // nearest even
    return (uint16_t)(__builtin_bit_cast(uint32_t, b) & 0xFFFFu);
}

// 16 bytes of row `row` (of `rows`) at column k (of D): zero past either end.
__device__ __forceinline__ uint4 ld_row16(const uint16_t* base, int rows, int D, int row, int k)
{
    return (row < rows && k < D) ? *reinterpret_cast<const uint4*>(base + (size_t)row * D + k)
                                 : make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(256) void project_kernel(ProjArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDK];
    const int C = 2 * a.dk + a.d + 2, NC = a.H * C;
    const int r0 = blockIdx.y * BM, c0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // staging: 1024 16-byte chunks per operand tile, 4 per thread; chunk -> (row, 8-element k group)
    int srow[4], skc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ch = tid + 256 * i;
        srow[i] = ch >> 3;
        skc[i] = (ch & 7) * 8;
    }
    uint4 ra[4], rb[4];
    auto fetch = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = ld_row16(a.x, a.R, a.D, r0 + srow[i], k0 + skc[i]);
            rb[i] = ld_row16(a.w, NC, a.D, c0 + srow[i], k0 + skc[i]);
        }
    };
    auto stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<uint4*>(&sA[buf][srow[i] * LDK + skc[i]]) = ra[i];
            *reinterpret_cast<uint4*>(&sB[buf][srow[i] * LDK + skc[i]]) = rb[i];
        }
    };

    f32x16_t acc[2][2] = {};
    const int ksl = (a.D + BK - 1) / BK;
    fetch(0);
    stage(0);
    __syncthreads();
    for (int s = 0; s < ksl; ++s) {
        const int buf = s & 1;
        if (s + 1 < ksl)
            fetch((s + 1) * BK); // in flight during this slice's MFMAs
        const uint16_t* A = sA[buf];
        const uint16_t* Bm = sB[buf];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kofs = kk * 16 + (lane >> 5) * 8;
            bf16x8_t av[2], bv[2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                av[m] = *reinterpret_cast<const bf16x8_t*>(&A[(wm * 64 + m * 32 + (lane & 31)) * LDK + kofs]);
#pragma unroll
            for (int n = 0; n < 2; ++n)
                bv[n] = *reinterpret_cast<const bf16x8_t*>(&Bm[(wn * 64 + n * 32 + (lane & 31)) * LDK + kofs]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[m], bv[n], acc[m][n], 0, 0, 0);
        }
        if (s + 1 < ksl) {
            stage(buf ^ 1); // the other buffer: last read one slice ago, before the barrier below
            __syncthreads();
        }
    }

    // epilogue: lane holds column (lane % 32) of rows 8*(e/4) + 4*(lane/32) + e%4 of each 32 x 32 tile
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int c = c0 + wn * 64 + n * 32 + (lane & 31);
        if (c >= NC)
            continue;
        const int h = c / C, o = c % C;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = r0 + wm * 64 + m * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (r >= a.R)
                    continue;
                const float y = acc[m][n][e];
                const size_t rh = (size_t)r * a.H + h;
                if (o < a.dk)
                    a.wq[rh * a.dk + o] = to_bf16(y);
                else if (o < 2 * a.dk)
                    a.rq[rh * a.dk + (o - a.dk)] = to_bf16(y);
                else if (o < 2 * a.dk + a.d)
                    a.v[rh * a.d + (o - 2 * a.dk)] = to_bf16(y);
                else {
                    const int gi = o - 2 * a.dk - a.d; // 0: alpha, 1: beta
                    const double z = (double)y + (double)a.bias[2 * h + gi];
                    const float g = (float)(1.0 / (1.0 + exp(-z)));
                    (gi == 0 ? a.alpha : a.beta)[rh] = g;
                }
            }
        }
    }
}

// dst[b] = src for b < B: 16-byte copies, grid-stride (bytes a multiple of 16)
__global__ __launch_bounds__(256) void broadcast_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        long n16, int B)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) {
        const uint4 u = src[i];
        for (int b = 0; b < B; ++b)
            dst[(size_t)b * n16 + i] = u;
    }
}

} // namespace

hipError_t launch_project(const void* x, const void* w, const float* bias, void* wq, void* rq, void* v, float* alpha,
                          float* beta, int R, int D, int H, int dk, int d, hipStream_t stream)
{
    if (R < 1 || D < 8 || D % 8 || H < 1 || dk < 1 || d < 1)
        return hipErrorInvalidValue;
    ProjArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias, static_cast<uint16_t*>(wq),
               static_cast<uint16_t*>(rq), static_cast<uint16_t*>(v), alpha, beta, R, D, H, dk, d};
    const long NC = (long)H * (2 * dk + d + 2);
    dim3 grid((unsigned)((NC + BN - 1) / BN), (unsigned)((R + BM - 1) / BM)), block(256);
    hipLaunchKernelGGL(project_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_broadcast(const void* m0, void* mem, size_t bytes_all_heads, int B, hipStream_t stream)
{
    if (bytes_all_heads % 16 || B < 1)
        return hipErrorInvalidValue;
    const long n16 = (long)(bytes_all_heads / 16);
    const long blocks = (n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096;
    hipLaunchKernelGGL(broadcast_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(m0), static_cast<uint4*>(mem), n16, B);
    return hipGetLastError();
}

} // namespace sdm

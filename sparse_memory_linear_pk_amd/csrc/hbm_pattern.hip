// A measurement kernel, not part of the layer: the memory traffic of the scan
// with its arithmetic taken out.
//
// The scan moves, per token and memory, W random slot rows read for the write,
// W random rows read for the read and the W write rows stored back, each as one
// 128-byte segment per workgroup (the workgroup owns 128 bytes of every row).
// This kernel issues exactly that pattern with the scan's geometry (one
// workgroup of four waves per memory and 128-byte column of the rows, eight
// lanes of 16 bytes per segment, two positions per lane, three tokens of loads
// in flight) on rows drawn by a hash, with no dependence between tokens and no
// barriers.  Its bandwidth is the ceiling that random 128-byte reads and writes
// in a 2:1 mix reach on the device: the scan cannot beat it, so the scan's
// achieved bandwidth is judged against it as well as against the HBM peak.
// The reverse scan of the backward pass reads 4 segments per slot position and
// token (the read slot's memory and gradient, the write slot's gradient, its
// logged value) and writes 3 (both gradients and the restored memory): the same
// kernel with 4 reads and 3 writes per position gives its ceiling.
// Every loaded value feeds a stored value, so the compiler removes no load; the
// memory's contents are scrambled.
#include "sdm_internal.h"

#include <utility>

namespace sdm {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld(__amdgpu_buffer_rsrc_t r, uint32_t o)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0));
}
__device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t o, uint4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, o, 0, 0);
}
template <int N> __device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ uint32_t mix(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) { return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w); }

template <class F, int... J> __device__ __forceinline__ void unroll_impl(F& f, std::integer_sequence<int, J...>)
{
    (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void unroll(F&& f)
{
    unroll_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kP = 3;                           // tokens of loads in flight
constexpr int kZ = kP + 1;                      // register stages
constexpr uint32_t kPast = 0xFFFFFFF0u;         // an offset past every buffer: reads zero, drops the store

// NR row sets read and the first NW of them written back, per slot position and token.
template <int NR, int NW>
__global__ __launch_bounds__(256) void hbm_pattern_kernel(char* mem, int T, int W, uint32_t rows, uint32_t row_stride,
                                                          int nchunk, uint32_t seed)
{
    constexpr int kOps = 2 * NR + 2 * NW;           // per token and wave (two positions per lane)
    constexpr int kWait = (kP - 1) * kOps + 2 * NW; // after a token's stores: the last kP - 1 tokens may be in flight
    static_assert(NW <= NR && kWait <= 63, "vmcnt");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 3, el = lane & 7;
    const int m = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const uint32_t lane_off = (uint32_t)(chunk * 8 + el) * 16u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(mem + (size_t)m * rows * row_stride, rows * row_stride);
    const int pos[2] = {wave * 16 + g, wave * 16 + 8 + g};
    auto offset = [&](int t, int p, uint32_t set) -> uint32_t {
        if (t < 0 || t >= T || p >= W)
            return kPast;
        const uint32_t row = mix((seed + (uint32_t)m * 7919u + (uint32_t)t * 131u + set) * 1024u + (uint32_t)p) % rows;
        return row * row_stride + lane_off;
    };
    uint4 v[kZ][NR][2];
    for (int z = 0; z < kZ; ++z)
        for (int i = 0; i < NR; ++i)
            for (int q = 0; q < 2; ++q)
                v[z][i][q] = make_uint4(0u, 0u, 0u, 0u);
    const int blocks = (T + kP + 1 + kZ - 1) / kZ;
    for (int blk = 0; blk < blocks; ++blk) {
        unroll<kZ>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            const int s = -kP - 1 + blk * kZ + j; // token whose rows are in stage j
            uint4 k = make_uint4(0u, 0u, 0u, 0u);  // every loaded value feeds the stores
#pragma unroll
            for (int i = NW; i < NR; ++i)
                k = xor4(k, xor4(v[j][i][0], v[j][i][1]));
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                st(r, offset(s, pos[0], (uint32_t)i), xor4(v[j][i][0], k));
                st(r, offset(s, pos[1], (uint32_t)i), xor4(v[j][i][1], k));
            }
            wait_vm<kWait>();
            const int u = s + kZ;
#pragma unroll
            for (int i = 0; i < NR; ++i)
                for (int q = 0; q < 2; ++q)
                    v[j][i][q] = ld(r, offset(u, pos[q], (uint32_t)i));
        });
    }
}

} // namespace

hipError_t launch_hbm_pattern(void* mem, int memories, long rows, int row_bytes, long row_stride, int T, int W,
                              int reads, int writes, uint32_t seed, hipStream_t stream)
{
    const int nchunk = row_bytes / 128;
    dim3 grid((unsigned)(memories * nchunk)), block(256);
    if (reads == 2 && writes == 1)
        hipLaunchKernelGGL((hbm_pattern_kernel<2, 1>), grid, block, 0, stream, (char*)mem, T, W, (uint32_t)rows,
                           (uint32_t)row_stride, nchunk, seed);
    else if (reads == 4 && writes == 3)
        hipLaunchKernelGGL((hbm_pattern_kernel<4, 3>), grid, block, 0, stream, (char*)mem, T, W, (uint32_t)rows,
                           (uint32_t)row_stride, nchunk, seed);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

} // namespace sdm

// sdm_scan: the sequential memory scan of the SDM layer, and its plan.
//
// Per token t of memory (b, h), with write slots n_i, weights w_i, decay alpha,
// step beta, value v and read slots m_j, weights r_j (SDM blog post, section
// "How does SDM work?" and the caption of the figure "The SDM mechanism, end
// to end": decay the selected slots, then the delta-rule write, then a
// softmax-weighted read of the read-selected slots):
//   x_i = alpha * M[n_i];  vhat = sum_i w_i x_i;  M[n_i] = x_i + w_i * beta * (v - vhat)
//   out = sum_j r_j * M[m_j]                     (after the write of the same token)
// Addressing never reads the memory, so every slot element evolves on its own:
// the scan is parallel over (b, h, element) and sequential over t.
//
// Work split.  A workgroup owns one (b, h) and a chunk of DC consecutive slot
// elements and walks all T tokens alone.  Memory is slot-major, so one slot's
// chunk is DC*sizeof(state) contiguous bytes, read by LPS lanes with one 16-byte
// access each.  The W slots of a token spread over the wave's 64/LPS lane groups
// and over the workgroup's waves; the sums over slots (vhat, out) are xor
// butterflies across lane groups (DPP row_ror:8 and the gfx950 permlane16/32
// swaps) and one LDS exchange across waves.
//
// Pipelining.  A token's slot reads are issued P tokens ahead and its plan
// record 2P tokens ahead.  Every wave issues the same vector-memory operations
// for every token (reads for inactive lanes and for tokens outside [0, T) use
// offsets past the end of their buffer, which read zeros and drop writes), so
// one `s_waitcnt vmcnt(K)` per token retires exactly the reads issued P tokens
// earlier together with everything issued before them: vmcnt counts loads and
// stores in issue order on this target.  A barrier after that wait means the
// reads issued next, for token u, see every store of tokens <= u - 2P - 1.  A
// slot written later than that (up to u itself, for the read set) is taken from
// an LDS ring holding the stored values of the last R = 2P + 1 tokens; the plan
// kernel below works out which reads need it and where from.  Two stores of one
// slot at most P tokens apart may both be in flight, so only the later one is
// issued; every reader between them is inside the forwarding window.
#include "sdm_internal.h"

#include <utility>

namespace sdm {
namespace {

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

constexpr int kLookahead = 6;               // P
constexpr int kRing = 2 * kLookahead + 1;   // R
constexpr uint32_t kOOB = 0xFFFFFFF0u;      // a buffer offset past every buffer's end

// Plan record for (b, h, t, position i), 16 bytes:
//   x: write slot (20 bits) | (1 + ring position of its latest unsettled write) << 20 (11 bits)
//      | skip-store << 31
//   y: read slot (20 bits)  | (1 + ring position of its latest unsettled write) << 20 (12 bits)
//   z: write weight, w: read weight (float bits)
constexpr uint32_t kSlotMask = 0xFFFFFu;

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

constexpr int kPlanTokens = 32;
constexpr int kPlanThreads = 256;

__device__ __forceinline__ int lower_bound64(const int32_t* s, int n)
{
    int lo = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1)
        if (s[lo + step - 1] < n)
            lo += step;
    return lo;
}

// For every token t and position i: the write slot's latest write by a token in
// [t - 2P, t) and the read slot's latest write in [t - 2P, t], as ring positions
// ((t' mod R) * W + i'), and whether a token in (t, t + P] writes the same slot.
// Write sets are sorted by slot once per token so each lookup is a binary search.
__global__ __launch_bounds__(kPlanThreads) void sdm_plan_kernel(const int32_t* __restrict__ idx_w,
                                                              const float* __restrict__ wt_w,
                                                              const int32_t* __restrict__ idx_r,
                                                              const float* __restrict__ wt_r,
                                                              uint4* __restrict__ plan, int T, int H, int W)
{
    constexpr int P = kLookahead;
    extern __shared__ int32_t s_plan[]; // [span][64] sorted slots, then [span][64] their positions
    const int tiles = (T + kPlanTokens - 1) / kPlanTokens;
    const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bh / H, h = bh % H;
    const int t0 = tile * kPlanTokens, t1 = min(T, t0 + kPlanTokens);
    const int lo = max(0, t0 - 2 * P), hi = min(T, t1 + P);
    const int span = hi - lo;
    int32_t* s_slot = s_plan;
    int32_t* s_pos = s_plan + span * 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;

    // each wave sorts whole write sets by slot (bitonic network across the wave)
    for (int tt = wave; tt < span; tt += nw) {
        const int t = lo + tt;
        int key = 0x7FFFFFFF, pos = lane;
        if (lane < W)
            key = idx_w[((long)(b * T + t) * H + h) * W + lane];
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const int ok = __shfl_xor(key, stride), op = __shfl_xor(pos, stride);
                const bool up = (lane & size) == 0, lower = (lane & stride) == 0;
                const bool take_other = (up == lower) ? (ok < key) : (ok > key);
                if (take_other) {
                    key = ok;
                    pos = op;
                }
            }
        }
        s_slot[tt * 64 + lane] = key;
        s_pos[tt * 64 + lane] = pos;
    }
    __syncthreads();

    const int items = (t1 - t0) * W;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int t = t0 + it / W, i = it % W;
        const long o = ((long)(b * T + t) * H + h) * W + i;
        const int n = idx_w[o], m = idx_r[o];
        uint32_t fw = 0, fr = 0, skip = 0;
        for (int tp = t; tp >= max(0, t - 2 * P) && (fw == 0 || fr == 0); --tp) {
            const int32_t* ss = s_slot + (tp - lo) * 64;
            if (fw == 0 && tp < t) {
                const int k = lower_bound64(ss, n);
                if (k < 64 && ss[k] == n)
                    fw = (uint32_t)((tp % kRing) * W + s_pos[(tp - lo) * 64 + k]) + 1u;
            }
            if (fr == 0) {
                const int k = lower_bound64(ss, m);
                if (k < 64 && ss[k] == m)
                    fr = (uint32_t)((tp % kRing) * W + s_pos[(tp - lo) * 64 + k]) + 1u;
            }
        }
        for (int tq = t + 1; tq <= min(T - 1, t + P) && !skip; ++tq) {
            const int32_t* ss = s_slot + (tq - lo) * 64;
            const int k = lower_bound64(ss, n);
            skip = k < 64 && ss[k] == n;
        }
        uint4 rec;
        rec.x = ((uint32_t)n & kSlotMask) | (fw << 20) | (skip << 31);
        rec.y = ((uint32_t)m & kSlotMask) | (fr << 20);
        rec.z = __float_as_uint(wt_w[o]);
        rec.w = __float_as_uint(wt_r[o]);
        plan[((long)bh * T + t) * W + i] = rec;
    }
}

// ---------------------------------------------------------------------------
// the scan
// ---------------------------------------------------------------------------

constexpr int kScanMaxThreads = 512;

template <class ST> struct StateFmt;
template <> struct StateFmt<float> {
    static constexpr int VEC = 4;
    __device__ static void unpack(const uint4& r, float (&x)[4])
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
    __device__ static uint4 pack(const float (&x)[4])
    {
        return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
    }
};
template <> struct StateFmt<uint16_t> { // bfloat16 bits
    static constexpr int VEC = 8;
    __device__ static void unpack(const uint4& r, float (&x)[8])
    {
        x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
        x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
        x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
        x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
    }
    __device__ static uint4 pack(const float (&x)[8])
    {
        return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                          pack_bf16x2(x[6], x[7]));
    }
};

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void st128(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r, off, 0, 0);
}

// VEC consecutive values of v (bf16 or float) as raw words, read with V_OPS loads
template <class VT, int VEC> struct VSlice {
    static constexpr int WORDS = VEC * (int)sizeof(VT) / 4;
    static constexpr int V_OPS = WORDS <= 4 ? 1 : WORDS / 4;
    uint32_t w[WORDS];
    __device__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        if constexpr (WORDS == 2) {
            const i32x2_t u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
            w[0] = (uint32_t)u[0];
            w[1] = (uint32_t)u[1];
        } else {
#pragma unroll
            for (int q = 0; q < WORDS / 4; ++q) {
                const uint4 u = ld128(r, off == kOOB ? kOOB : off + 16u * q);
                w[4 * q] = u.x; w[4 * q + 1] = u.y; w[4 * q + 2] = u.z; w[4 * q + 3] = u.w;
            }
        }
    }
    __device__ float get(int i) const
    {
        if constexpr (sizeof(VT) == 4)
            return __uint_as_float(w[i]);
        else
            return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
    }
};

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

__device__ __forceinline__ float xor8(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16(float x)
{
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor32(float x)
{
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Sum over the lanes that share `lane % LPS` (the 64/LPS lane groups), the same
// value in every lane: a xor butterfly, so every lane adds in the same order.
template <int LPS> __device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int m = LPS; m < 8; m <<= 1)
        x += __shfl_xor(x, m);
    x = xor8(x);
    x = xor16(x);
    return xor32(x);
}

template <class ST, class VT, int LPS>
__global__ __launch_bounds__(kScanMaxThreads) void sdm_scan_kernel(ScanArgs a)
{
    static_assert(LPS <= 8, "lane groups are summed with a butterfly from distance LPS up");
    using F = StateFmt<ST>;
    using VS = VSlice<VT, F::VEC>;
    constexpr int P = kLookahead, R = kRing;
    constexpr int VEC = F::VEC;       // slot elements per lane
    constexpr int DC = LPS * VEC;     // slot elements per workgroup
    constexpr int GPW = 64 / LPS;     // slot positions per wave
    constexpr int O_OPS = VEC / 4;    // 16-byte stores per lane for `out`
    // vector-memory operations per token: reads issued ahead, then stores
    constexpr int L_OPS = 2 + VS::V_OPS + 2 + 1; // write slot, read slot, v, alpha, beta, plan record
    constexpr int C_OPS = O_OPS + 1;             // out (previous token), slot store
    constexpr int K = (P - 1) * (L_OPS + C_OPS) + C_OPS;

    const int nwv = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPS, el = lane % LPS;
    const int pos = wave * GPW + g;     // this lane's position in the token's write and read sets
    const bool act = pos < a.W;
    const int T = a.T, H = a.H, W = a.W, d = a.d;
    const int nchunk = d / DC;
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int b = bh / H, h = bh % H;
    const uint32_t row_bytes = (uint32_t)d * (uint32_t)sizeof(ST);
    const uint32_t lane_off = (uint32_t)(chunk * DC + el * VEC) * (uint32_t)sizeof(ST);

    const __amdgpu_buffer_rsrc_t r_mem = make_rsrc(static_cast<const char*>(a.mem) + (size_t)bh * a.N * row_bytes,
                                                   (uint32_t)((size_t)a.N * row_bytes));
    const __amdgpu_buffer_rsrc_t r_plan = make_rsrc(a.plan + (size_t)bh * T * W, (uint32_t)((size_t)T * W * 16));
    // v, out: [B, T, H, d], alpha, beta: [B, T, H]; each resource spans sequence b
    const size_t tok0 = (size_t)b * T * H;
    const __amdgpu_buffer_rsrc_t r_v = make_rsrc(static_cast<const VT*>(a.v) + tok0 * d,
                                                 (uint32_t)((size_t)T * H * d * sizeof(VT)));
    const __amdgpu_buffer_rsrc_t r_out = make_rsrc(a.out + tok0 * d, (uint32_t)((size_t)T * H * d * 4));
    const __amdgpu_buffer_rsrc_t r_al = make_rsrc(a.alpha + tok0, (uint32_t)((size_t)T * H * 4));
    const __amdgpu_buffer_rsrc_t r_be = make_rsrc(a.beta + tok0, (uint32_t)((size_t)T * H * 4));
    const uint32_t v_lane = (uint32_t)(chunk * DC + el * VEC) * (uint32_t)sizeof(VT);
    const uint32_t o_lane = (uint32_t)(chunk * DC + el * VEC) * 4u;

    extern __shared__ uint4 lds[];
    uint4* ring = lds;                                           // [R*W][LPS]
    float* red = reinterpret_cast<float*>(lds + R * W * LPS);    // [nwv][LPS][VEC]
    float* ored = red + nwv * LPS * VEC;                         // [nwv][LPS][VEC]

    // per-token offsets; tokens outside [0, T) and inactive lanes read past the end
    auto tok_ok = [&](int t) { return t >= 0 && t < T; };
    auto plan_off = [&](int t) -> uint32_t { return (tok_ok(t) && act) ? (uint32_t)(t * W + pos) * 16u : kOOB; };

    // Ring buffers in registers (indices are compile-time after unrolling):
    //   slot chunks of token t in [t mod (P+1)], loaded at the end of body t-P-1, used in body t;
    //   plan record of token t in rec[t mod (2P+2)], loaded at the end of body t-2P-1, used by the
    //   issue at the end of body t-P-1 (slot ids) and in body t (weights, ring positions).
    constexpr int ZS = P + 1, ZR = 2 * P + 2;
    uint4 rec[ZR];
    uint4 sw[ZS], sr[ZS];
    VS vv[ZS];
    float al[ZS], be[ZS];
#pragma unroll
    for (int z = 0; z < ZR; ++z)
        rec[z] = make_uint4(0, 0, 0, 0);

    // End of body s: reads for token s+P+1 (slot chunks, v, gates) and the plan
    // record of token s+2P+1.  With s = s0 + ZR*blk + j and s0 = -(2P+1):
    // s mod ZS = (j+1) mod ZS, (s+P+1) mod ZR = (j+P+2) mod ZR, (s+2P+1) mod ZR = j.
#define SDM_ISSUE(S_, J_)                                                                                           \
    {                                                                                                              \
        const int u_ = (S_) + P + 1;                                                                               \
        const uint4 ru_ = rec[((J_) + P + 2) % ZR];                                                                \
        const bool ok_ = tok_ok(u_);                                                                               \
        const bool oka_ = ok_ && act;                                                                              \
        constexpr int zs_ = ((J_) + 1) % ZS;                                                                       \
        sw[zs_] = ld128(r_mem, oka_ ? (ru_.x & kSlotMask) * row_bytes + lane_off : kOOB);                          \
        sr[zs_] = ld128(r_mem, oka_ ? (ru_.y & kSlotMask) * row_bytes + lane_off : kOOB);                          \
        const uint32_t ro_ = (uint32_t)(u_ * H + h);                                                               \
        vv[zs_].load(r_v, ok_ ? ro_ * (uint32_t)d * (uint32_t)sizeof(VT) + v_lane : kOOB);                          \
        al[zs_] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_al, ok_ ? ro_ * 4u : kOOB, 0, 0));          \
        be[zs_] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_be, ok_ ? ro_ * 4u : kOOB, 0, 0));          \
        rec[(J_) % ZR] = ld128(r_plan, plan_off((S_) + 2 * P + 1));                                                 \
    }

    // Bodies run from the virtual token s0 = -(2P+1), so the first real records
    // and slot chunks arrive through the same uniform pattern as every later one;
    // virtual tokens (s < 0 or s >= T) read zeros and store nothing.  Body T
    // stores the output of token T-1.
    constexpr int S0 = -(2 * P + 1);
    const int blocks = (T + 1 - S0 + ZR - 1) / ZR;
    for (int blk = 0; blk < blocks; ++blk) {
        static_for<ZR>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const int s = S0 + blk * ZR + j;
            const bool real = tok_ok(s);
            const uint4 rs = rec[(j + 1) % ZR];
            const int sp = (j + 1) % ZS;

            // ---- write: decay this lane's slot, its share of the prediction
            float x[VEC];
            {
                uint4 raw = sw[sp];
                const uint32_t fpos = (rs.x >> 20) & 0x7FFu;
                if (fpos && fpos <= (uint32_t)(R * W))
                    raw = ring[(fpos - 1) * LPS + el];
                F::unpack(raw, x);
                const float w = __uint_as_float(rs.z), alpha = al[sp];
                float acc[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    x[q] = alpha * x[q];
                    acc[q] = group_sum<LPS>(w * x[q]);
                }
                if (g == 0) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        red[(wave * LPS + el) * VEC + q] = acc[q];
                }
            }
            lds_barrier();
            // ---- the previous token's read is complete in `ored`: every wave sums it, wave 0 stores
            {
                float o[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    o[q] = group_sum<LPS>(g < nwv ? ored[(g * LPS + el) * VEC + q] : 0.f);
                const bool st_ = wave == 0 && g == 0 && tok_ok(s - 1);
                const uint32_t oo = st_ ? (uint32_t)((s - 1) * H + h) * (uint32_t)d * 4u + o_lane : kOOB;
#pragma unroll
                for (int q = 0; q < O_OPS; ++q)
                    st128(r_out, oo == kOOB ? kOOB : oo + 16u * q,
                          make_uint4(__float_as_uint(o[4 * q]), __float_as_uint(o[4 * q + 1]),
                                     __float_as_uint(o[4 * q + 2]), __float_as_uint(o[4 * q + 3])));
            }
            // ---- delta-rule write of this lane's slot
            {
                const float w = __uint_as_float(rs.z), beta = be[sp];
                float y[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    const float vh = group_sum<LPS>(g < nwv ? red[(g * LPS + el) * VEC + q] : 0.f);
                    y[q] = x[q] + w * (beta * (vv[sp].get(q) - vh));
                }
                const uint4 packed = F::pack(y);
                if (act)
                    ring[(((s + 2 * R) % R) * W + pos) * LPS + el] = packed;
                const bool st_ = real && act && !(rs.x >> 31);
                st128(r_mem, st_ ? (rs.x & kSlotMask) * row_bytes + lane_off : kOOB, packed);
            }
            // the reads for token s+1 were issued at the end of body s-P: retire them
            // and everything issued before them, in every wave
            wait_vmcnt<K>();
            lds_barrier();
            // ---- read: this lane's read slot, after this token's write
            {
                uint4 raw = sr[sp];
                const uint32_t rpos = rs.y >> 20;
                if (rpos && rpos <= (uint32_t)(R * W))
                    raw = ring[(rpos - 1) * LPS + el];
                float y[VEC];
                F::unpack(raw, y);
                const float r = __uint_as_float(rs.w);
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    y[q] = group_sum<LPS>(r * y[q]);
                if (g == 0) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        ored[(wave * LPS + el) * VEC + q] = y[q];
                }
            }
            SDM_ISSUE(s, j);
        });
    }
#undef SDM_ISSUE
}

template <class ST, class VT>
hipError_t launch_typed(const ScanArgs& a, const ScanPlan& p, hipStream_t stream)
{
    dim3 grid((unsigned)p.grid), block((unsigned)(p.waves * 64));
    switch (p.lps) {
    case 1: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 1>), grid, block, p.lds, stream, a); break;
    case 2: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 2>), grid, block, p.lds, stream, a); break;
    case 4: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 4>), grid, block, p.lds, stream, a); break;
    case 8: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 8>), grid, block, p.lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

bool plan_scan(int B, int H, int d, int W, bool state_bf16, ScanPlan* plan)
{
    const int vec = state_bf16 ? 8 : 4;
    const long units = (long)B * H;
    int lps = 8;
    // largest chunk that divides d, shrunk while the grid would leave CUs idle
    while (lps > 1 && (d % (lps * vec) != 0 || (lps > 2 && units * (d / (lps * vec)) < 256)))
        lps >>= 1;
    if (d % (lps * vec) != 0)
        return false;
    const int gpw = 64 / lps;
    const int waves = (W + gpw - 1) / gpw;
    if (waves * 64 > kScanMaxThreads || waves > gpw || kRing * W > 2047)
        return false;
    plan->lps = lps;
    plan->waves = waves;
    plan->lookahead = kLookahead;
    plan->grid = (int)(units * (d / (lps * vec)));
    plan->lds = kRing * W * lps * 16 + 2 * waves * lps * vec * 4;
    return plan->lds <= 160 * 1024;
}

size_t plan_bytes(int B, int H, int T, int W) { return (size_t)B * H * T * W * sizeof(uint4); }

hipError_t launch_sdm_plan(const int32_t* idx_w, const float* wt_w, const int32_t* idx_r, const float* wt_r,
                           uint4* plan, int B, int T, int H, int W, hipStream_t stream)
{
    const int tiles = (T + kPlanTokens - 1) / kPlanTokens;
    const int span = kPlanTokens + 3 * kLookahead;
    const size_t lds = (size_t)span * 64 * 2 * sizeof(int32_t);
    hipLaunchKernelGGL(sdm_plan_kernel, dim3((unsigned)(tiles * B * H)), dim3(kPlanThreads), lds, stream, idx_w, wt_w,
                       idx_r, wt_r, plan, T, H, W);
    return hipGetLastError();
}

hipError_t launch_sdm_scan(const ScanArgs& a, const ScanPlan& plan, bool state_bf16, bool in_bf16,
                           hipStream_t stream)
{
    if (state_bf16)
        return in_bf16 ? launch_typed<uint16_t, uint16_t>(a, plan, stream) : launch_typed<uint16_t, float>(a, plan, stream);
    return in_bf16 ? launch_typed<float, uint16_t>(a, plan, stream) : launch_typed<float, float>(a, plan, stream);
}

} // namespace sdm

// sdm_scan: the sequential memory scan of the SDM layer, and its forwarding plan.
//
// Per token t of memory (b, h), with write slots n_i, weights w_i, decay alpha,
// step beta, value v and read slots m_j, weights r_j (SDM blog post, section
// "How does SDM work?" and the caption of the figure "The SDM mechanism, end
// to end": decay the selected slots, then the delta-rule write, then a
// softmax-weighted read of the read-selected slots):
//   x_i = alpha * M[n_i];  vhat = sum_i w_i x_i;  M[n_i] = x_i + w_i * beta * (v - vhat)
//   out = sum_j r_j * M[m_j]                     (after the write of the same token)
// Addressing never reads the memory, so every slot element e evolves on its
// own: the scan is parallel over (b, h, e) and sequential over t.
//
// Work split.  A workgroup owns one (b, h) and a chunk of DC consecutive slot
// elements; it walks all T tokens with no other workgroup involved.  Memory is
// slot-major, so a slot's chunk is DC*sizeof(state) contiguous bytes, read by
// LPS lanes with one 16-byte access each.  The W slots of a token are spread
// over the wave's 64/LPS lane groups and over the workgroup's waves: the sums
// over slots (vhat and out) are butterfly shuffles inside a wave plus one pass
// through LDS across waves.
//
// Latency hiding.  One token moves 3*W*DC*sizeof(state) bytes per workgroup and
// depends on the previous token, so slot reads are issued ahead: tokens go in
// epochs of E.  At the start of epoch e every wave drains its outstanding
// memory operations (s_waitcnt 0) and the workgroup meets at a barrier; then
// the slot reads of epoch e+1 are issued and epoch e is computed from the reads
// issued one epoch earlier.  A slot read for token t therefore sees every store
// of tokens before (t/E - 1)*E.  A slot written by a later token (up to t itself
// for the read set) cannot be trusted from memory; its value is taken from an
// LDS ring that keeps the stored values of the last 2E tokens.  Which reads must
// be forwarded, and from where, is worked out once per token by sdm_hazard
// (below) from the slot indices alone.  Two writes of one slot in one epoch are
// not ordered in memory, so only the later one is stored.
#include "sdm_internal.h"

namespace sdm {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// forwarding plan
// ---------------------------------------------------------------------------

constexpr int kHazTokens = 32;   // tokens per workgroup
constexpr int kHazThreads = 256;

// For every token t (epoch e = t/E, ring of 2E tokens) and every position of its
// write and read sets, fwd = 1 + ring position ((t' mod 2E)*W + i') of the latest
// write of the same slot by a token t' in [max(0, (e-1)E), t) for the write set,
// [.., t] for the read set; 0 when there is none.  Write positions also get
// kFwdSkipStore when a later token of epoch e writes the same slot.
__global__ __launch_bounds__(kHazThreads) void sdm_hazard_kernel(const int32_t* __restrict__ idx_w,
                                                               const int32_t* __restrict__ idx_r,
                                                               int32_t* __restrict__ fwd_w,
                                                               int32_t* __restrict__ fwd_r, int T, int H, int W,
                                                               int E)
{
    extern __shared__ int32_t s_w[]; // write sets of tokens [lo, hi)
    const int tiles = (T + kHazTokens - 1) / kHazTokens;
    const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bh / H, h = bh % H;
    const int t0 = tile * kHazTokens, t1 = min(T, t0 + kHazTokens);
    const int lo = max(0, (t0 / E - 1) * E);
    const int hi = min(T, ((t1 - 1) / E + 1) * E);
    const int ring = 2 * E;

    for (int x = threadIdx.x; x < (hi - lo) * W; x += blockDim.x) {
        const int t = lo + x / W, i = x % W;
        s_w[x] = idx_w[((long)(b * T + t) * H + h) * W + i];
    }
    __syncthreads();

    const int items = (t1 - t0) * 2 * W;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int t = t0 + it / (2 * W);
        const int rem = it % (2 * W);
        const bool rd = rem >= W;
        const int i = rem % W;
        const long o = ((long)(b * T + t) * H + h) * W + i;
        const int n = rd ? idx_r[o] : s_w[(t - lo) * W + i];
        const int ws = max(0, (t / E - 1) * E);
        uint32_t code = 0;
        for (int tp = rd ? t : t - 1; tp >= ws && code == 0; --tp) {
            const int32_t* set = s_w + (tp - lo) * W;
            for (int ip = 0; ip < W; ++ip) {
                if (set[ip] == n) {
                    code = (uint32_t)((tp % ring) * W + ip) + 1u;
                    break;
                }
            }
        }
        if (!rd) {
            const int ee = min(T, (t / E + 1) * E);
            bool later = false;
            for (int tq = t + 1; tq < ee && !later; ++tq) {
                const int32_t* set = s_w + (tq - lo) * W;
                for (int ip = 0; ip < W; ++ip)
                    later |= set[ip] == n;
            }
            if (later)
                code |= kFwdSkipStore;
        }
        (rd ? fwd_r : fwd_w)[o] = (int32_t)code;
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

// VEC consecutive values of v, as raw words
template <class VT, int VEC> struct VSlice {
    static constexpr int WORDS = VEC * (int)sizeof(VT) / 4;
    uint32_t w[WORDS];
    __device__ void load(const VT* p)
    {
        if constexpr (WORDS == 2) {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            w[0] = u.x; w[1] = u.y;
        } else {
#pragma unroll
            for (int q = 0; q < WORDS / 4; ++q) {
                const uint4 u = reinterpret_cast<const uint4*>(p)[q];
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

__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Every memory operation this wave has issued completes, then the workgroup meets.
__device__ __forceinline__ void drain_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <class ST, class VT, int LPS, int E>
__global__ __launch_bounds__(kScanMaxThreads) void sdm_scan_kernel(ScanArgs a)
{
    using F = StateFmt<ST>;
    constexpr int VEC = F::VEC;        // slot elements per lane
    constexpr int DC = LPS * VEC;      // slot elements per workgroup
    constexpr int GPW = 64 / LPS;      // slot positions per wave
    constexpr int RING = 2 * E;

    const int nwv = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPS, el = lane % LPS;
    const int pos = wave * GPW + g;    // this lane's position in the token's write and read sets
    const bool act = pos < a.W;
    const int T = a.T, H = a.H, W = a.W, d = a.d;
    const int nchunk = d / DC;
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int b = bh / H, h = bh % H;
    const uint32_t row_bytes = (uint32_t)d * (uint32_t)sizeof(ST);
    const uint32_t lane_off = (uint32_t)(chunk * DC + el * VEC) * (uint32_t)sizeof(ST);
    const char* mbase = static_cast<const char*>(a.mem) + (size_t)bh * (size_t)a.N * row_bytes;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(mbase, (uint32_t)((size_t)a.N * row_bytes));

    extern __shared__ uint4 lds[];
    uint4* ring = lds;                                            // [RING*W][LPS]
    float* red = reinterpret_cast<float*>(lds + RING * W * LPS);  // [nwv][LPS][VEC]
    float* ored = red + nwv * LPS * VEC;                          // [nwv][LPS][VEC]

    auto meta_off = [&](int t) -> long { return ((long)(b * T + t) * H + h) * W + pos; };
    auto tok_row = [&](int t) -> long { return (long)(b * T + t) * H + h; };

    // registers: c* = epoch being computed, n* = next epoch (in flight), nn* = slot ids two ahead
    uint4 cw[E], cr[E], nw[E], nr[E];
    uint32_t cfw[E], crf[E], nfw[E], nrf[E];
    float cwt[E], crt[E], nwt[E], nrt[E], ca[E], cb[E], na[E], nb[E];
    int32_t cwi[E], nwi[E], nri[E], nnwi[E], nnri[E];
    VSlice<VT, VEC> cv[E], nv[E];

    auto load_ids = [&](int ep, int32_t (&wi)[E], int32_t (&ri)[E]) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int t = ep * E + k;
            if (act && t < T) {
                wi[k] = a.idx_w[meta_off(t)];
                ri[k] = a.idx_r[meta_off(t)];
            } else {
                wi[k] = 0;
                ri[k] = 0;
            }
        }
    };
    auto issue = [&](int ep) {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int t = ep * E + k;
            if (t < T) {
                if (act) {
                    nw[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rsrc, (uint32_t)nwi[k] * row_bytes + lane_off, 0, 0));
                    nr[k] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rsrc, (uint32_t)nri[k] * row_bytes + lane_off, 0, 0));
                    const long mo = meta_off(t);
                    nfw[k] = (uint32_t)a.fwd_w[mo];
                    nwt[k] = a.wt_w[mo];
                    nrf[k] = (uint32_t)a.fwd_r[mo];
                    nrt[k] = a.wt_r[mo];
                } else {
                    nw[k] = nr[k] = make_uint4(0, 0, 0, 0);
                    nfw[k] = nrf[k] = 0;
                    nwt[k] = nrt[k] = 0.f;
                }
                nv[k].load(static_cast<const VT*>(a.v) + tok_row(t) * d + chunk * DC + el * VEC);
                na[k] = a.alpha[tok_row(t)];
                nb[k] = a.beta[tok_row(t)];
            }
        }
    };

    const int nep = (T + E - 1) / E;
    load_ids(0, nwi, nri);
    if (nep > 1)
        load_ids(1, nnwi, nnri);
    drain_barrier();
    issue(0);

    int pend = -1; // token whose read partials wait in `ored`
    for (int ep = 0; ep < nep; ++ep) {
        drain_barrier();
#pragma unroll
        for (int k = 0; k < E; ++k) {
            cw[k] = nw[k]; cr[k] = nr[k];
            cfw[k] = nfw[k]; crf[k] = nrf[k];
            cwt[k] = nwt[k]; crt[k] = nrt[k];
            ca[k] = na[k]; cb[k] = nb[k];
            cwi[k] = nwi[k];
            cv[k] = nv[k];
            nwi[k] = nnwi[k];
            nri[k] = nnri[k];
        }
        if (ep + 1 < nep)
            issue(ep + 1);
        if (ep + 2 < nep)
            load_ids(ep + 2, nnwi, nnri);

#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int t = ep * E + k;
            if (t >= T)
                break;
            // ---- write: decay the slot, form its share of the prediction
            uint4 raw = cw[k];
            const uint32_t fpos = cfw[k] & kFwdPosMask;
            if (fpos && fpos <= (uint32_t)(RING * W))
                raw = ring[(fpos - 1) * LPS + el];
            float x[VEC], acc[VEC];
            F::unpack(raw, x);
            const float al = ca[k], w = cwt[k];
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                x[q] = al * x[q];
                acc[q] = w * x[q];
            }
#pragma unroll
            for (int m = LPS; m < 64; m <<= 1)
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    acc[q] += __shfl_xor(acc[q], m);
            if (g == 0) {
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    red[(wave * LPS + el) * VEC + q] = acc[q];
            }
            lds_barrier();
            // the previous token's read is complete in `ored`
            if (pend >= 0 && wave == 0 && g == 0) {
                float o[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    o[q] = 0.f;
                for (int ww = 0; ww < nwv; ++ww)
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        o[q] += ored[(ww * LPS + el) * VEC + q];
                float4* dst = reinterpret_cast<float4*>(a.out + tok_row(pend) * d + chunk * DC + el * VEC);
#pragma unroll
                for (int q = 0; q < VEC / 4; ++q)
                    dst[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
            }
            float vh[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                vh[q] = 0.f;
            for (int ww = 0; ww < nwv; ++ww)
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    vh[q] += red[(ww * LPS + el) * VEC + q];
            const float be = cb[k];
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                x[q] = x[q] + w * (be * (cv[k].get(q) - vh[q]));
            const uint4 packed = F::pack(x);
            if (act) {
                ring[((t % RING) * W + pos) * LPS + el] = packed;
                if (!(cfw[k] & kFwdSkipStore))
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, packed),
                                                           rsrc, (uint32_t)cwi[k] * row_bytes + lane_off, 0, 0);
            }
            lds_barrier();
            // ---- read: weighted sum of the read slots, after this token's write
            uint4 rraw = cr[k];
            const uint32_t rpos = crf[k] & kFwdPosMask;
            if (rpos && rpos <= (uint32_t)(RING * W))
                rraw = ring[(rpos - 1) * LPS + el];
            float y[VEC];
            F::unpack(rraw, y);
            const float rw = crt[k];
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                y[q] = rw * y[q];
#pragma unroll
            for (int m = LPS; m < 64; m <<= 1)
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    y[q] += __shfl_xor(y[q], m);
            if (g == 0) {
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    ored[(wave * LPS + el) * VEC + q] = y[q];
            }
            pend = t;
        }
    }
    lds_barrier();
    if (pend >= 0 && wave == 0 && g == 0) {
        float o[VEC];
#pragma unroll
        for (int q = 0; q < VEC; ++q)
            o[q] = 0.f;
        for (int ww = 0; ww < nwv; ++ww)
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                o[q] += ored[(ww * LPS + el) * VEC + q];
        float4* dst = reinterpret_cast<float4*>(a.out + tok_row(pend) * d + chunk * DC + el * VEC);
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q)
            dst[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    }
}

constexpr int kEpoch = 4;

template <class ST, class VT>
hipError_t launch_typed(const ScanArgs& a, const ScanPlan& p, hipStream_t stream)
{
    dim3 grid((unsigned)p.grid), block((unsigned)(p.waves * 64));
    switch (p.lps) {
    case 1: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 1, kEpoch>), grid, block, p.lds, stream, a); break;
    case 2: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 2, kEpoch>), grid, block, p.lds, stream, a); break;
    case 4: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 4, kEpoch>), grid, block, p.lds, stream, a); break;
    case 8: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 8, kEpoch>), grid, block, p.lds, stream, a); break;
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
    if (waves * 64 > kScanMaxThreads)
        return false;
    plan->lps = lps;
    plan->waves = waves;
    plan->epoch = kEpoch;
    plan->grid = (int)(units * (d / (lps * vec)));
    plan->lds = 2 * kEpoch * W * lps * 16 + 2 * waves * lps * vec * 4;
    return plan->lds <= 160 * 1024;
}

hipError_t launch_sdm_hazard(const int32_t* idx_w, const int32_t* idx_r, int32_t* fwd_w, int32_t* fwd_r, int B,
                             int T, int H, int W, int epoch, hipStream_t stream)
{
    const int tiles = (T + kHazTokens - 1) / kHazTokens;
    const int span = kHazTokens + 3 * epoch; // tokens staged per workgroup, at most
    const size_t lds = (size_t)span * W * sizeof(int32_t);
    hipLaunchKernelGGL(sdm_hazard_kernel, dim3((unsigned)(tiles * B * H)), dim3(kHazThreads), lds, stream, idx_w,
                       idx_r, fwd_w, fwd_r, T, H, W, epoch);
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

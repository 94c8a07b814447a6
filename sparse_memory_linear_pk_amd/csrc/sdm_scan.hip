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
#include "scan_device.h"

namespace sdm {
namespace {

constexpr int kLookahead = 6;               // P
constexpr int kRing = 2 * kLookahead + 1;   // R

// Plan record for (b, h, t, position i), 16 bytes:
//   x: write slot (20 bits) | (1 + ring position of its latest unsettled write) << 20 (11 bits)
//      | skip-store << 31
//   y: read slot (20 bits)  | (1 + ring position of its latest unsettled write) << 20 (12 bits)
//   z: write weight, w: read weight (float bits)
constexpr uint32_t kSlotMask = 0xFFFFFu;

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

constexpr int kPlanTokens = 32;  // tokens per plan workgroup (at most; 16 when 32 leave CUs idle)
constexpr int kPlanThreads = 512;
constexpr int kFilterWords = 4096; // a 2^17-bit hashed filter of the slots written near a tile

__device__ __forceinline__ uint32_t filter_bit(int n) { return ((uint32_t)n * 2654435761u) >> 15; }

__device__ __forceinline__ int lower_bound64(const int32_t* s, int n)
{
    int lo = 0;
#pragma unroll
    for (int step = 32; step > 0; step >>= 1)
        if (s[lo + step - 1] < n)
            lo += step;
    return lo;
}

struct PlanArgs {
    const int32_t* idx_w;
    const float* wt_w;
    const int32_t* idx_r;
    const float* wt_r;
    const float* alpha;
    const float* beta;
    uint4* plan;
    float2* ab;        // register-ring format only
    int T, H, W, d, Tp;
    int Ts, t0;        // tokens per sequence of idx, wt, alpha, beta; the chunk's first token
    uint32_t N;        // slots per memory (the staged sentinel slot id)
    uint32_t v_bytes;  // bytes of one value element (staged header offsets)
    int tile;          // tokens per workgroup, at most kPlanTokens
};

// For every token t and position i: the write slot's latest write by a token in
// [t - 2P, t) and the read slot's latest write in [t - 2P, t], as (1 + ring
// position) with ring position (ring slot of t') * stride + i', and whether a
// token in (t, t + P] writes the same slot.  Write sets are sorted by slot once
// per token so each lookup is a binary search.
//   register-ring format: ring slot t' mod (2P+1), stride W, fields 20 + 11/12 bits;
//   staged format: window kWindow, ring slot (t' - S0) mod 8, stride 64, fields 21 + 10 bits; a
//   forwarded read names the sentinel slot (nothing to load), bit 31 of y marks a
//   forwarded write slot (load nothing, still store); sentinel records for
//   positions >= W and tokens >= T, then a header per token (bit 0 of its out
//   offset: the token writes a slot the previous token wrote).
template <int P, int WIN, bool STAGED>
__global__ __launch_bounds__(kPlanThreads) void sdm_plan_kernel(PlanArgs a)
{
    constexpr int kSpanMax = kPlanTokens + WIN + P;
    // [span][64] sorted slots, [span][64] their positions, the slot filter, the tile's dependence flags
    extern __shared__ int32_t s_plan[];
    const int T = a.T, H = a.H, W = a.W;
    const int Tout = STAGED ? a.Tp : T; // tokens written per memory
    const int tiles = (Tout + a.tile - 1) / a.tile;
    const int bh = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bh / H, h = bh % H;
    const int t0 = tile * a.tile, t1 = min(Tout, t0 + a.tile);
    const int lo = max(0, min(T, t0) - WIN), hi = min(T, t1 + P);
    const int span = max(0, hi - lo);
    int32_t* s_slot = s_plan;
    int32_t* s_pos = s_plan + span * 64;
    uint32_t* s_filter = reinterpret_cast<uint32_t*>(s_plan + 2 * kSpanMax * 64);
    uint32_t* s_dep = s_filter + kFilterWords;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    constexpr int kSlotShift = STAGED ? staged::kSlotBits : 20;
    constexpr uint32_t kSlotField = (1u << kSlotShift) - 1u;
    const int stride = STAGED ? staged::kPos : W;
    auto ring_slot = [](int tp) { return STAGED ? (tp - staged::kS0) % staged::kRing : tp % (2 * P + 1); };
    auto in_filter = [&](int n) {
        const uint32_t f = filter_bit(n);
        return (s_filter[f >> 5] >> (f & 31u)) & 1u;
    };

    for (int i = threadIdx.x; i < kFilterWords; i += blockDim.x)
        s_filter[i] = 0u;
    __syncthreads();

    // each wave sorts whole write sets by slot (bitonic network across the wave)
    // and enters their slots in the filter
    for (int tt = wave; tt < span; tt += nw) {
        const int t = lo + tt;
        int key = 0x7FFFFFFF, pos = lane;
        if (lane < W)
            key = a.idx_w[((long)b * a.Ts + a.t0 + t) * H * W + (long)h * W + lane];
        if (lane < W) {
            const uint32_t f = filter_bit(key);
            atomicOr(&s_filter[f >> 5], 1u << (f & 31u));
        }
#pragma unroll
        for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
            for (int stride_ = size >> 1; stride_ > 0; stride_ >>= 1) {
                const int ok = __shfl_xor(key, stride_), op = __shfl_xor(pos, stride_);
                const bool up = (lane & size) == 0, lower = (lane & stride_) == 0;
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

    if constexpr (STAGED) {
        // does token t write a slot token t - 1 wrote?  one wave per token, one slot per lane
        for (int t = t0 + wave; t < t1; t += nw) {
            bool hit = false;
            if (t < T && t > 0 && lane < W) {
                const int n = s_slot[(t - lo) * 64 + lane];
                const int32_t* prev = s_slot + (t - 1 - lo) * 64;
                const int k = lower_bound64(prev, n);
                hit = k < 64 && prev[k] == n;
            }
            const bool dep = __builtin_amdgcn_ballot_w64(hit) != 0u;
            if (lane == 0)
                s_dep[t - t0] = dep ? 1u : 0u;
        }
        __syncthreads();
    } else {
        for (int t = t0 + (int)threadIdx.x; t < t1; t += blockDim.x) {
            const long o = ((long)b * a.Ts + a.t0 + t) * H + h;
            a.ab[(long)bh * T + t] = make_float2(a.alpha[o], a.beta[o]);
        }
    }
    const int per_tok = STAGED ? staged::kRecs : W;
    const int items = (t1 - t0) * per_tok;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int t = t0 + it / per_tok, i = it % per_tok;
        uint4 rec;
        if (STAGED && i == staged::kPos) { // header
            const long o = ((long)b * a.Ts + a.t0 + t) * H + h;
            const uint32_t row = (uint32_t)(t * H + h) * (uint32_t)a.d;
            const bool real = t < T;
            rec.x = real ? __float_as_uint(a.alpha[o]) : 0u;
            rec.y = real ? __float_as_uint(a.beta[o]) : 0u;
            rec.z = (real ? row : (uint32_t)T * H * a.d) * a.v_bytes;
            rec.w = (real ? row : (uint32_t)T * H * a.d) * 4u;
            rec.w |= s_dep[t - t0] ? staged::kDepFlag : 0u;
        } else if (STAGED && (t >= T || i >= W)) { // sentinel: slot past the memory, no store, weight 0
            rec = make_uint4(a.N | (1u << 31), a.N, 0u, 0u);
        } else {
            const long o = (((long)b * a.Ts + a.t0 + t) * H + h) * W + i;
            const int n = a.idx_w[o], m = a.idx_r[o];
            uint32_t fw = 0, fr = 0, skip = 0;
            // the filter holds every slot written in [lo, hi): a slot outside it
            // was written by no token the searches below would find
            if (in_filter(n)) {
                for (int tp = t - 1; tp >= max(0, t - WIN) && fw == 0; --tp) {
                    const int32_t* ss = s_slot + (tp - lo) * 64;
                    const int k = lower_bound64(ss, n);
                    if (k < 64 && ss[k] == n)
                        fw = (uint32_t)(ring_slot(tp) * stride + s_pos[(tp - lo) * 64 + k]) + 1u;
                }
                for (int tq = t + 1; tq <= min(T - 1, t + P) && !skip; ++tq) {
                    const int32_t* ss = s_slot + (tq - lo) * 64;
                    const int k = lower_bound64(ss, n);
                    skip = k < 64 && ss[k] == n;
                }
            }
            if (in_filter(m)) {
                for (int tp = t; tp >= max(0, t - WIN) && fr == 0; --tp) {
                    const int32_t* ss = s_slot + (tp - lo) * 64;
                    const int k = lower_bound64(ss, m);
                    if (k < 64 && ss[k] == m)
                        fr = (uint32_t)(ring_slot(tp) * stride + s_pos[(tp - lo) * 64 + k]) + 1u;
                }
            }
            rec.x = ((uint32_t)n & kSlotField) | (fw << kSlotShift) | (skip << 31);
            if constexpr (STAGED)
                rec.y = (fr ? a.N : (uint32_t)m) | (fr << kSlotShift) | ((uint32_t)(fw != 0) << 31);
            else
                rec.y = ((uint32_t)m & kSlotField) | (fr << kSlotShift);
            rec.z = __float_as_uint(a.wt_w[o]);
            rec.w = __float_as_uint(a.wt_r[o]);
        }
        a.plan[((long)bh * Tout + t) * per_tok + i] = rec;
    }
}

// ---------------------------------------------------------------------------
// the scan
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t)); // v_cvt_pk_bf16_f32
}

// State formats.  `compute_t` is the type of the write path: float for a float32
// state, double for a bf16 state so that every stored value is the single
// nearest-even rounding of (nearly) the exact value, as a double reference has it.
template <class ST> struct StateFmt;
template <> struct StateFmt<float> {
    static constexpr int VEC = 4;
    using compute_t = float;
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
    using compute_t = double;
    __device__ static void unpack(const uint4& r, float (&x)[8])
    {
        x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
        x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
        x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
        x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
    }
    __device__ static uint4 pack(const double (&x)[8])
    {
        float f[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            f[q] = settle_bf16_tie(x[q]);
        return make_uint4(pack2_bf16(f[0], f[1]), pack2_bf16(f[2], f[3]), pack2_bf16(f[4], f[5]),
                          pack2_bf16(f[6], f[7]));
    }
};

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

// Sum over all 64/LPS lane groups of a wave (lanes sharing lane % LPS).
template <int LPS, class T> __device__ __forceinline__ T wave_sum(T x)
{
    if constexpr (LPS < 64)
        x = bfly<LPS>(x);
    if constexpr (2 * LPS < 64)
        x = bfly<2 * LPS>(x);
    if constexpr (4 * LPS < 64)
        x = bfly<4 * LPS>(x);
    if constexpr (8 * LPS < 64)
        x = bfly<8 * LPS>(x);
    if constexpr (16 * LPS < 64)
        x = bfly<16 * LPS>(x);
    if constexpr (32 * LPS < 64)
        x = bfly<32 * LPS>(x);
    return x;
}

// Sum of the per-wave partials: lane group g holds partial (g mod p2) (zero past
// the last wave) and a butterfly over log2(p2) group bits adds them.
template <int LPS, class T> __device__ __forceinline__ T waves_sum(T x, int p2)
{
    if constexpr (LPS < 64)
        if (p2 > 1) x = bfly<LPS>(x);
    if constexpr (2 * LPS < 64)
        if (p2 > 2) x = bfly<2 * LPS>(x);
    if constexpr (4 * LPS < 64)
        if (p2 > 4) x = bfly<4 * LPS>(x);
    if constexpr (8 * LPS < 64)
        if (p2 > 8) x = bfly<8 * LPS>(x);
    if constexpr (16 * LPS < 64)
        if (p2 > 16) x = bfly<16 * LPS>(x);
    if constexpr (32 * LPS < 64)
        if (p2 > 32) x = bfly<32 * LPS>(x);
    return x;
}

// ds_swizzle in bit mode: lane l of each 32-lane half reads lane ((l & AND) within that half).
template <int AND> __device__ __forceinline__ uint32_t swz(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, AND);
}
template <int AND> __device__ __forceinline__ uint4 swz4(const uint4& v)
{
    return make_uint4(swz<AND>(v.x), swz<AND>(v.y), swz<AND>(v.z), swz<AND>(v.w));
}

// At most 4 waves per workgroup (1 when a wave holds every position with one
// position per lane), so each wave may use the whole register file of its SIMD.
// FAST: float arithmetic, 8 lanes per slot chunk, two positions per lane and
// exactly 4 waves; sums over slots then use reduce4_to_rows.
template <class ST, class VT, int LPS, int RW, bool FAST>
__global__ __launch_bounds__(RW == 2 ? 256 : 64) void sdm_scan_kernel(ScanArgs a)
{
    using F = StateFmt<ST>;
    using CT = typename F::compute_t;
    using VS = VSlice<VT, F::VEC>;
    constexpr int P = kLookahead, R = kRing, ZS = P + 1, ZR = 2 * P + 2;
    constexpr int VEC = F::VEC;       // slot elements per lane
    constexpr int DC = LPS * VEC;     // slot elements per workgroup
    constexpr int GPW = 64 / LPS;     // lane groups per wave
    static_assert(!FAST || (VEC == 4 && LPS == 8 && RW == 2 && sizeof(CT) == 4), "fast path shape");
    static_assert(VEC / 4 <= GPW, "out is stored by the first VEC/4 lane groups");
    // vector-memory operations per token: reads issued ahead, then stores
    constexpr int L_OPS = 2 * RW + VS::V_OPS + 1 + RW; // slot reads (write, read), v, alpha|beta, plan records
    constexpr int C_OPS = RW + 1;                      // slot stores, out
    constexpr int K = (P - 1) * (L_OPS + C_OPS) + C_OPS;
    static_assert(K <= 63, "more operations in flight than vmcnt can count");
    // metadata is read by one lane per group (records) or per half-wave (v) and broadcast
    constexpr int REC_SWZ = 0x1F & ~(LPS - 1); // lane -> first lane of its group
    constexpr int V_SWZ = LPS - 1;             // lane -> same element in the first group of its half

    const int nwv = blockDim.x >> 6;
    int p2 = 1;
    while (p2 < nwv)
        p2 <<= 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / LPS, el = lane % LPS;
    const bool rec_lead = el == 0;
    const bool v_lead = g % (GPW / 2 > 0 ? GPW / 2 : 1) == 0;
    const int T = a.T, H = a.H, W = a.W, d = a.d;
    int pos[RW];
    bool act[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        pos[r] = (wave * RW + r) * GPW + g; // this lane's positions in the token's write and read sets
        act[r] = pos[r] < W;
    }
    const int nchunk = d / DC;
    const int bh = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int b = bh / H, h = bh % H;
    const uint32_t row_bytes = (uint32_t)a.ms * (uint32_t)sizeof(ST); // slot row to slot row in memory
    const uint32_t lane_off = (uint32_t)(chunk * DC + el * VEC) * (uint32_t)sizeof(ST);

    const __amdgpu_buffer_rsrc_t r_mem = make_rsrc(static_cast<const char*>(a.mem) + (size_t)bh * a.N * row_bytes,
                                                   (uint32_t)((size_t)a.N * row_bytes));
    const __amdgpu_buffer_rsrc_t r_plan = make_rsrc(a.plan + (size_t)bh * T * W, (uint32_t)((size_t)T * W * 16));
    const __amdgpu_buffer_rsrc_t r_ab = make_rsrc(a.ab + (size_t)bh * T, (uint32_t)((size_t)T * 8));
    // v, out: [B, T, H, d]; each resource spans sequence b
    const size_t tok0 = (size_t)b * a.Ts * H;
    const __amdgpu_buffer_rsrc_t r_v = make_rsrc(static_cast<const VT*>(a.v) + tok0 * d,
                                                 (uint32_t)((size_t)T * H * d * sizeof(VT)));
    const __amdgpu_buffer_rsrc_t r_out = make_rsrc(a.out + tok0 * d, (uint32_t)((size_t)T * H * d * 4));
    const uint32_t v_lane = (uint32_t)(chunk * DC + el * VEC) * (uint32_t)sizeof(VT);

    extern __shared__ uint4 lds[];
    uint4* ring = lds;                                             // [R*W][LPS] stored slot chunks
    CT* red = reinterpret_cast<CT*>(lds + R * W * LPS);            // [nwv][LPS][VEC] write partials
    float* ored = reinterpret_cast<float*>(red + nwv * LPS * VEC); // [nwv][LPS][VEC] read partials

    auto tok_ok = [&](int t) { return t >= 0 && t < T; };

    // Register rings (indices are constants after unrolling):
    //   slot chunks, v, gates of token t in [t mod (P+1)]: read at the end of body t-P-1, broadcast
    //   in body t-1, used in body t;
    //   plan records of token t in rec[t mod (2P+2)]: read at the end of body t-2P-1, broadcast
    //   within lane groups in body t-P-1 and used there (slot ids) and in body t.
    constexpr int S0 = -(2 * P + 1);
    uint4 rec[ZR][RW];
    uint4 sw[ZS][RW], sr[ZS][RW];
    VS vv[ZS];
    f32x2_t gab[ZS];
#pragma unroll
    for (int z = 0; z < ZR; ++z)
#pragma unroll
        for (int r = 0; r < RW; ++r)
            rec[z][r] = make_uint4(0, 0, 0, 0);

    // End of body s = S0 + ZR*blk + J: reads for token s+P+1 and the plan records of token s+2P+1.
    // s mod ZS = (J+1) mod ZS, (s+P+1) mod ZR = (J+P+2) mod ZR, (s+2P+1) mod ZR = J mod ZR.
    auto issue = [&](int s, auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int zs = (J + 1) % ZS, zu = (J + P + 2) % ZR, zl = J % ZR;
        const int u = s + P + 1;
        const bool ok = tok_ok(u);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint4 ru = rec[zu][r];
            const bool oka = ok && act[r];
            sw[zs][r] = ld128(r_mem, oka ? (ru.x & kSlotMask) * row_bytes + lane_off : kOOB);
            sr[zs][r] = ld128(r_mem, oka ? (ru.y & kSlotMask) * row_bytes + lane_off : kOOB);
        }
        const uint32_t ro = (uint32_t)(u * H + h);
        vv[zs].load(r_v, (ok && v_lead) ? ro * (uint32_t)d * (uint32_t)sizeof(VT) + v_lane : kOOB);
        gab[zs] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                                  r_ab, (ok && lane == 0) ? (uint32_t)u * 8u : kOOB, 0, 0));
        const int un = s + 2 * P + 1;
#pragma unroll
        for (int r = 0; r < RW; ++r)
            rec[zl][r] = ld128(r_plan, (tok_ok(un) && act[r] && rec_lead) ? (uint32_t)(un * W + pos[r]) * 16u : kOOB);
    };
    // After the wait in body s: the records of token s+P+1 and v, gates of token s+1 have
    // arrived in their leader lanes; hand them to every lane.
    auto broadcast = [&](auto jc) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int zu = (J + P + 2) % ZR, z1 = (J + 2) % ZS;
#pragma unroll
        for (int r = 0; r < RW; ++r)
            rec[zu][r] = swz4<REC_SWZ>(rec[zu][r]);
#pragma unroll
        for (int q = 0; q < VS::WORDS; ++q)
            vv[z1].w[q] = swz<V_SWZ>(vv[z1].w[q]);
        gab[z1] = (f32x2_t){__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gab[z1][0]))),
                            __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gab[z1][1])))};
    };

    // Bodies run from the virtual token S0, so the first real records and slot
    // chunks arrive through the same uniform pattern as every later one; virtual
    // tokens (s < 0 or s >= T) read zeros and store nothing.  Body T stores the
    // output of token T-1.
    const int blocks = (T + 1 - S0 + ZR - 1) / ZR;
    for (int blk = 0; blk < blocks; ++blk) {
        static_for<ZR>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            constexpr int sp = (j + 1) % ZS, zr = (j + 1) % ZR;
            const int s = S0 + blk * ZR + j;
            const bool real = tok_ok(s);

            // ---- write: decay this lane's slots, their share of the prediction
            CT x[RW][VEC];
            CT acc[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q)
                acc[q] = 0;
            const CT alpha = (CT)gab[sp][0];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const uint4 rs = rec[zr][r];
                uint4 raw = sw[sp][r];
                const uint32_t fpos = (rs.x >> 20) & 0x7FFu;
                if (fpos && fpos <= (uint32_t)(R * W))
                    raw = ring[(fpos - 1) * LPS + el];
                float m[VEC];
                F::unpack(raw, m);
                const CT w = (CT)__uint_as_float(rs.z);
#pragma unroll
                for (int q = 0; q < VEC; ++q) {
                    x[r][q] = alpha * (CT)m[q];
                    acc[q] += w * x[r][q];
                }
            }
            if constexpr (FAST) {
                const float t = reduce4_to_rows(acc[0], acc[1], acc[2], acc[3]);
                if ((lane & 8) == 0)
                    red[(wave * LPS + el) * VEC + (lane >> 4)] = t;
            } else {
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    acc[q] = wave_sum<LPS>(acc[q]);
                if (g == 0) {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        red[(wave * LPS + el) * VEC + q] = acc[q];
                }
            }
            lds_barrier();
            // ---- the previous token's read sits in `ored`: wave 0 sums and stores it
            if constexpr (FAST) {
                // waves 0..3 read into groups g mod 4; a DPP stage and two transposing
                // permlane16 swaps leave (o0, o1) in row 0 and (o2, o3) in row 1
                float o01 = 0.f;
                if (wave == 0) {
                    const float4 pv = *reinterpret_cast<const float4*>(ored + ((g & 3) * LPS + el) * VEC);
                    const float o0 = bfly<8>(pv.x), o1 = bfly<8>(pv.y), o2 = bfly<8>(pv.z), o3 = bfly<8>(pv.w);
                    const auto s02 = __builtin_amdgcn_permlane16_swap(__float_as_uint(o0), __float_as_uint(o2), false, false);
                    const auto s13 = __builtin_amdgcn_permlane16_swap(__float_as_uint(o1), __float_as_uint(o3), false, false);
                    const float t02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
                    const float t13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
                    o01 = t02;
                    const float o_b = t13;
                    const int row = lane >> 4;
                    const bool st_ = (lane & 8) == 0 && row < 2 && tok_ok(s - 1);
                    const uint32_t oo = st_ ? ((uint32_t)((s - 1) * H + h) * (uint32_t)d + (uint32_t)(chunk * DC + el * VEC + 2 * row)) * 4u : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2_t, (f32x2_t){o01, o_b}), r_out, oo, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2_t, (f32x2_t){o01, o01}), r_out, kOOB, 0, 0);
                }
            } else {
                float o[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    o[q] = 0.f;
                if (wave == 0) {
                    const int pg = g & (p2 - 1);
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        o[q] = waves_sum<LPS>(pg < nwv ? ored[(pg * LPS + el) * VEC + q] : 0.f, p2);
                }
                const bool st_ = wave == 0 && g < VEC / 4 && tok_ok(s - 1);
                const uint32_t oo = st_ ? ((uint32_t)((s - 1) * H + h) * (uint32_t)d + (uint32_t)(chunk * DC + el * VEC)) * 4u + 16u * (uint32_t)(g & 1) : kOOB;
                uint4 ov;
                if constexpr (VEC == 8) {
                    ov = (g & 1) ? make_uint4(__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7]))
                                 : make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
                } else {
                    ov = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
                }
                st128(r_out, oo, ov);
            }
            // ---- delta-rule write of this lane's slots
            {
                CT vh[VEC];
                if constexpr (FAST) {
                    const float4 pv = *reinterpret_cast<const float4*>(red + ((g & 3) * LPS + el) * VEC);
                    vh[0] = bfly<16>(bfly<8>(pv.x));
                    vh[1] = bfly<16>(bfly<8>(pv.y));
                    vh[2] = bfly<16>(bfly<8>(pv.z));
                    vh[3] = bfly<16>(bfly<8>(pv.w));
                } else {
                    const int pg = g & (p2 - 1);
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        vh[q] = waves_sum<LPS>(pg < nwv ? red[(pg * LPS + el) * VEC + q] : (CT)0, p2);
                }
                const CT beta = (CT)gab[sp][1];
                CT dlt[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    dlt[q] = beta * ((CT)vv[sp].get(q) - vh[q]);
                const int ring_tok = ((s + 2 * R) % R) * W;
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    const uint4 rs = rec[zr][r];
                    const CT w = (CT)__uint_as_float(rs.z);
                    CT y[VEC];
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        y[q] = x[r][q] + w * dlt[q];
                    const uint4 packed = F::pack(y);
                    if (act[r])
                        ring[(ring_tok + pos[r]) * LPS + el] = packed;
                    const bool st_ = real && act[r] && !(rs.x >> 31);
                    st128(r_mem, st_ ? (rs.x & kSlotMask) * row_bytes + lane_off : kOOB, packed);
                }
            }
            // the reads for token s+1 were issued at the end of body s-P: retire them
            // and everything issued before them, in every wave
            wait_vmcnt<K>();
            lds_barrier();
            broadcast(jc);
            // ---- read: this lane's read slots, after this token's write
            {
                float oa[VEC];
#pragma unroll
                for (int q = 0; q < VEC; ++q)
                    oa[q] = 0.f;
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    const uint4 rs = rec[zr][r];
                    uint4 raw = sr[sp][r];
                    const uint32_t rpos = rs.y >> 20;
                    if (rpos && rpos <= (uint32_t)(R * W))
                        raw = ring[(rpos - 1) * LPS + el];
                    float m[VEC];
                    F::unpack(raw, m);
                    const float rw = __uint_as_float(rs.w);
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        oa[q] += rw * m[q];
                }
                if constexpr (FAST) {
                    const float t = reduce4_to_rows(oa[0], oa[1], oa[2], oa[3]);
                    if ((lane & 8) == 0)
                        ored[(wave * LPS + el) * VEC + (lane >> 4)] = t;
                } else {
#pragma unroll
                    for (int q = 0; q < VEC; ++q)
                        oa[q] = wave_sum<LPS>(oa[q]);
                    if (g == 0) {
#pragma unroll
                        for (int q = 0; q < VEC; ++q)
                            ored[(wave * LPS + el) * VEC + q] = oa[q];
                    }
                }
            }
            issue(s, jc);
        });
    }
}

template <class ST, class VT, int RW, bool FAST>
hipError_t launch_rw(const ScanArgs& a, const ScanPlan& p, hipStream_t stream)
{
    dim3 grid((unsigned)p.grid), block((unsigned)(p.waves * 64));
    if constexpr (FAST) {
        hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 8, 2, true>), grid, block, p.lds, stream, a);
        return hipGetLastError();
    }
    switch (p.lps) {
    case 1: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 1, RW, false>), grid, block, p.lds, stream, a); break;
    case 2: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 2, RW, false>), grid, block, p.lds, stream, a); break;
    case 4: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 4, RW, false>), grid, block, p.lds, stream, a); break;
    case 8: hipLaunchKernelGGL((sdm_scan_kernel<ST, VT, 8, RW, false>), grid, block, p.lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class ST, class VT>
hipError_t launch_typed(const ScanArgs& a, const ScanPlan& p, hipStream_t stream)
{
    if constexpr (sizeof(ST) == 4) {
        if (p.lps == 8 && p.rw == 2 && p.waves == 4)
            return launch_rw<ST, VT, 2, true>(a, p, stream);
    }
    return p.rw == 2 ? launch_rw<ST, VT, 2, false>(a, p, stream) : launch_rw<ST, VT, 1, false>(a, p, stream);
}

} // namespace

bool plan_scan(int B, int H, int T, int d, int ms, int W, long N, bool state_bf16, bool in_bf16, ScanPlan* plan)
{
    const long units = (long)B * H;
    const uint64_t v_bytes = in_bf16 ? 2 : 4;
    const uint64_t s_bytes = state_bf16 ? 2 : 4;
    if (ms < d || (ms * s_bytes) % 16 || (uint64_t)N * ms * s_bytes >= (1ull << 32))
        return false;
    if ((d * s_bytes) % 128 == 0 && W <= staged::kPos && N < (1l << staged::kSlotBits) &&
        (uint64_t)(N + 1) * ms * s_bytes <= (1ull << 32) && ((uint64_t)T * H + 1) * d * 4 <= (1ull << 32) &&
        ((uint64_t)T * H + 1) * d * v_bytes <= (1ull << 32)) {
        plan->staged = true;
        plan->lps = 8;
        plan->rw = 2;
        plan->waves = 4;
        plan->lookahead = staged::kP;
        // 64-byte (4 bf16 values per lane) or 32-byte segments (2 values) when 128-byte
        // ones leave most CUs idle
        const long cols = units * (d * s_bytes / 128);
        plan->seg_bytes = !state_bf16 || cols >= 128 ? 128 : cols >= 64 ? 64 : 32;
        plan->grid = (int)(units * (d * s_bytes / plan->seg_bytes));
        plan->lds = 0;
        // pairs run from S0 to the pair after the one holding T-1; each loads the
        // records of the pair four ahead
        const int blocks = (T + 2 - staged::kS0 + staged::kRecSlots - 1) / staged::kRecSlots;
        plan->Tp = staged::kS0 + blocks * staged::kRecSlots + 8;
        return true;
    }
    // the register-ring kernel addresses one sequence's v and out rows of a chunk with 32-bit offsets
    if (((uint64_t)T * H + 1) * d * 4 > (1ull << 32))
        return false;
    const int vec = state_bf16 ? 8 : 4;
    const int ct = state_bf16 ? 8 : 4; // bytes of the write path's arithmetic type
    int lps = 8;
    // largest chunk that divides d, shrunk while the grid would leave CUs idle
    while (lps > 1 && (d % (lps * vec) != 0 || (lps > 2 && units * (d / (lps * vec)) < 256)))
        lps >>= 1;
    if (d % (lps * vec) != 0)
        return false;
    const int gpw = 64 / lps;
    const int rw = W > gpw ? 2 : 1; // slot positions per lane
    const int waves = (W + gpw * rw - 1) / (gpw * rw);
    if (waves * 64 > (rw == 2 ? 256 : 64) || waves > gpw || kRing * W > 2047)
        return false;
    plan->staged = false;
    plan->lps = lps;
    plan->rw = rw;
    plan->waves = waves;
    plan->lookahead = kLookahead;
    plan->grid = (int)(units * (d / (lps * vec)));
    plan->lds = kRing * W * lps * 16 + waves * lps * vec * (ct + 4);
    plan->Tp = T;
    return plan->lds <= 160 * 1024;
}

size_t plan_bytes(const ScanPlan& p, int B, int H, int T, int W)
{
    if (p.staged)
        return (size_t)B * H * p.Tp * staged::kRecs * sizeof(uint4);
    return (size_t)B * H * T * (W * sizeof(uint4) + sizeof(float2));
}

hipError_t launch_sdm_plan(const ScanPlan& p, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                           const float* wt_r, const float* alpha, const float* beta, void* plan, const Rows& r,
                           int W, int d, long N, bool in_bf16, hipStream_t stream)
{
    const int B = r.B, H = r.H, T = r.Tc;
    PlanArgs a;
    a.idx_w = idx_w;
    a.wt_w = wt_w;
    a.idx_r = idx_r;
    a.wt_r = wt_r;
    a.alpha = alpha;
    a.beta = beta;
    a.plan = static_cast<uint4*>(plan);
    a.ab = p.staged ? nullptr : reinterpret_cast<float2*>(a.plan + (size_t)B * H * T * W);
    a.T = T;
    a.Ts = r.Ts;
    a.t0 = r.t0;
    a.H = H;
    a.W = W;
    a.d = d;
    a.Tp = p.Tp;
    a.N = (uint32_t)N;
    a.v_bytes = in_bf16 ? 2u : 4u;
    const int P = p.staged ? staged::kP : kLookahead, WIN = p.staged ? staged::kWindow : 2 * kLookahead;
    // 32 tokens a workgroup, or 16 when that leaves most CUs without one (short chunks)
    const int Tout = p.staged ? p.Tp : T;
    a.tile = (long)((Tout + kPlanTokens - 1) / kPlanTokens) * B * H < 512 ? kPlanTokens / 2 : kPlanTokens;
    const int tiles = (Tout + a.tile - 1) / a.tile;
    const size_t lds = ((size_t)(kPlanTokens + WIN + P) * 64 * 2 + kFilterWords + kPlanTokens) * sizeof(int32_t);
    if (p.staged)
        hipLaunchKernelGGL((sdm_plan_kernel<staged::kP, staged::kWindow, true>), dim3((unsigned)(tiles * B * H)),
                           dim3(kPlanThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((sdm_plan_kernel<kLookahead, 2 * kLookahead, false>), dim3((unsigned)(tiles * B * H)),
                           dim3(kPlanThreads), lds, stream, a);
    return hipGetLastError();
}

hipError_t launch_sdm_scan(const ScanArgs& a, const ScanPlan& plan, bool state_bf16, bool in_bf16,
                           hipStream_t stream)
{
    if (plan.staged)
        return launch_sdm_scan_staged(a, plan, state_bf16, in_bf16, stream);
    if (state_bf16)
        return in_bf16 ? launch_typed<uint16_t, uint16_t>(a, plan, stream) : launch_typed<uint16_t, float>(a, plan, stream);
    return in_bf16 ? launch_typed<float, uint16_t>(a, plan, stream) : launch_typed<float, float>(a, plan, stream);
}

} // namespace sdm

// sdm_scan, staged form: the memory scan of the SDM layer for a float32 or a
// bf16 state.
//
// Per token t of memory (b, h), with write slots n_i, weights w_i, decay alpha,
// step beta, value v and read slots m_j, weights r_j (SDM blog post, section
// "How does SDM work?" and the caption of the figure "The SDM mechanism, end
// to end"):
//   x_i = alpha * M[n_i];  vhat = sum_i w_i x_i;  M[n_i] = x_i + w_i * beta * (v - vhat)
//   out = sum_j r_j * M[m_j]                     (after the write of the same token)
// A float32 state is updated in float32.  A bf16 state is updated in double
// and rounded once, to nearest-even, when a slot is stored (every stored value
// is then the correctly rounded exact result, as the double reference has it);
// the read sees the stored values and sums in float32.
//
// Work split.  A workgroup of 4 waves owns one (b, h) and 128 bytes of every
// slot row (32 float32 or 64 bf16 elements) and walks all T tokens.  When the
// memories are too few to fill the device that way (one long sequence), a
// bf16 state is split into 64-byte segments (8 lanes x 8 bytes, 4 values per
// lane) or 32-byte ones (8 lanes x 4 bytes, 2 values): more workgroups, less
// arithmetic per token each.  A token's 64 positions (the W selected slots,
// padded with sentinels) spread over the waves, 16 each: lane (g, e) of wave w
// holds the bytes e of positions 16w + g and 16w + 8 + g (E = 2, 4 or 8 elements).  Sums over positions are a
// transposing reduction inside the wave and one LDS exchange across the waves.
//
// Pipeline.  Tokens go in pairs.  At the start of pair k: the read of pair k-1
// (after its write), then the loads of pair k+2 (its slot rows and v into
// registers; the plan records of pair k+4 into registers, parked in LDS two pairs
// later, where the 8 lanes sharing a position read them as a broadcast), then the
// write of pair k: both tokens' partial sums, one barrier, both updates.  When
// token 2k+1 writes a slot token 2k writes (a plan flag), its write is redone
// after token 2k's has landed in the ring.  Two pairs of slot reads stay in
// flight per wave, enough to cover the memory latency at full bandwidth.
//
// Forwarding.  A slot written too recently for its load to see the store comes
// from a ring of the values stored by the last 12 tokens, which the plan names;
// such a slot is not loaded (its load reads past the buffer, zeros) and an
// unforwarded slot names the ring's zero entry, so a read is the sum of a
// register and, when any lane of the wave forwards, one LDS load.
//
// Log.  For training, the kernel can also store every write slot's value before
// its write (the staged segment, or the ring entry it was forwarded from, bit for
// bit) to a log that the reverse pass restores the memory from: four more stores
// per pair, issued after the slot stores.
//
// Ordering.  Every wave issues the same vector-memory operations in the same
// order for every pair (sentinel records and headers of the virtual tokens
// before 0 and after T-1 give offsets past their buffers, which read zeros and
// drop writes), so counted waits (s_waitcnt vmcnt) retire exactly the intended
// operations: loads and stores retire in issue order.  A barrier after a wait
// makes every wave's retired stores visible to the loads issued after it.  Two
// stores of one slot that may be in flight together are never both issued: the
// plan drops the earlier.
#include "scan_cell.h"

namespace sdm {
namespace {

using namespace staged;

constexpr int kWaves = 4;
constexpr int kRecPerWave = 17;                  // 16 records and the header
constexpr int kEntryU4 = 8;                      // one slot segment: 8 lanes x 16 bytes
constexpr int kPartU4 = kWaves * 8 * 4;          // room for one token's partials ([wave][el][E], <= 8 doubles)

__shared__ __attribute__((aligned(16))) uint4 g_ring[(kRing * kPos + 1) * kEntryU4]; // zero entry, stored segments
__shared__ __attribute__((aligned(16))) uint4 g_rec[kRecSlots * kWaves * kRecPerWave + kWaves]; // records, headers; a spare entry per wave
__shared__ __attribute__((aligned(16))) float4 g_red[2 * kPartU4];                  // write partials of a pair
__shared__ __attribute__((aligned(16))) float4 g_ored[2 * kPartU4];                 // read partials of a pair
static_assert(kStages == 6, "register rings of three pairs");

// Ring entry a record field names: entry f - 1 of the ring for f > 0, the zero
// entry for f = 0 (then the staged segment holds the value).
__device__ __forceinline__ const uint4* ring_src(uint32_t field, const uint4* ring_lane)
{
    return ring_lane + ((field >> kSlotBits) & 0x3FFu) * kEntryU4;
}

// Whether any lane of the wave takes one of its two slots from the ring (a
// wave-uniform answer; most tokens forward nothing and skip the ring loads).
__device__ __forceinline__ bool forwards(uint32_t f0, uint32_t f1)
{
    constexpr uint32_t kField = 0x3FFu << kSlotBits;
    return __builtin_amdgcn_ballot_w64(((f0 | f1) & kField) != 0u) != 0u;
}

// Workgroup barrier after this wave's own LDS loads and stores have completed.
// The loads into the stage buffers are not waited for here: those buffers are
// private to each wave, and the per-token vmcnt wait retires them.  (A release
// fence would wait for them.)  The memory clobber keeps the compiler from moving
// memory accesses across.
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A segment's 16, 8 or 4 bytes of one lane (held in the low part of the uint4).
template <int SEGB> __device__ __forceinline__ uint4 ldseg(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    if constexpr (SEGB == 128) {
        return ld128(r, off);
    } else if constexpr (SEGB == 64) {
        const i32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_uint4((uint32_t)v[0], (uint32_t)v[1], 0u, 0u);
    } else {
        return make_uint4((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0), 0u, 0u, 0u);
    }
}
template <int SEGB> __device__ __forceinline__ void stseg(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v)
{
    if constexpr (SEGB == 128)
        st128(r, off, v);
    else if constexpr (SEGB == 64)
        __builtin_amdgcn_raw_buffer_store_b64((i32x2_t){(int)v.x, (int)v.y}, r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b32((int)v.x, r, off, 0, 0);
}

// ST: state element (float or bf16 bits), VT: v element (float or bf16 bits),
// LOG: also store the write slots' values before the write to a.log,
// SEGB: bytes of every slot row the workgroup owns (128, or 64 or 32 for a bf16 state).
template <class ST, class VT, bool LOG, int SEGB>
__global__ __launch_bounds__(256) void sdm_scan_staged_kernel(ScanArgs a)
{
    static_assert(SEGB == 128 || ((SEGB == 64 || SEGB == 32) && sizeof(ST) == 2), "segment width");
    using C = std::conditional_t<SEGB == 128, Cell<ST>, std::conditional_t<SEGB == 64, CellHalf<ST>, CellQuarter<ST>>>;
    using CT = typename C::CT;                       // type of the write arithmetic
    constexpr int E = C::E;                          // state elements per lane
    constexpr int SEG = SEGB / (int)sizeof(ST);      // state elements of a workgroup's segment
    constexpr int VB = E * (int)sizeof(VT);          // bytes of v per lane and token: 4, 8, 16 or 32
    constexpr int NV = VB <= 16 ? 1 : 2;             // v loads per token
    constexpr int NO = E >= 4 ? E / 4 : 1;           // out stores per token (16 bytes each, or one of 8)
    constexpr int ZS = kStages, ZR = kRecSlots, ZL = 4;
    // Vector-memory operations of a pair, in issue order: at its start the loads
    // (per token of pair k+2 4 slot loads and NV of v; the records of pair k+4),
    // then 2*NO out stores, 4 slot stores and, with LOG, 4 log stores.  vmcnt(K)
    // at the start of pair k leaves only pair k-1's operations in flight: pair
    // k's data and pair k+2's records have landed and pair k-2's stores are done.
    constexpr int K = 2 * (4 + NV) + 2 + 2 * NO + 4 + (LOG ? 4 : 0);
    static_assert(K <= 63, "vmcnt");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int g = lane >> 3, el = lane & 7;
    const int T = a.T, H = a.H, d = a.d;
    const uint32_t N = (uint32_t)a.N;
    const int nchunk = d / SEG;
    // Workgroups go to the 8 XCDs in turn (blockIdx mod 8).  Narrow segments share a
    // 128-byte line with their neighbours: each XCD then takes a contiguous run of
    // segments, so that the workgroups reading one line share one L2.
    int lin = blockIdx.x;
    if constexpr (SEGB < 128) {
        if (gridDim.x % 8 == 0)
            lin = (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8);
    }
    const int bh = lin / nchunk, chunk = lin % nchunk;
    const int b = bh / H;
    const uint32_t row_bytes = (uint32_t)d * (uint32_t)sizeof(ST);      // a log row
    const uint32_t mem_row = (uint32_t)a.ms * (uint32_t)sizeof(ST);     // slot row to slot row in memory
    const uint32_t lane_off = (uint32_t)chunk * SEGB + (uint32_t)el * (SEGB / 8);
    const uint32_t tok_elems = (uint32_t)T * H * d;

    const __amdgpu_buffer_rsrc_t r_mem = make_rsrc(static_cast<const char*>(a.mem) + (size_t)bh * a.N * mem_row,
                                                   N * mem_row);
    const __amdgpu_buffer_rsrc_t r_plan = make_rsrc(a.plan + (size_t)bh * a.Tp * kRecs,
                                                    (uint32_t)a.Tp * kRecs * 16u);
    const size_t tok0 = (size_t)b * a.Ts * H;
    const __amdgpu_buffer_rsrc_t r_v = make_rsrc(static_cast<const VT*>(a.v) + tok0 * d, tok_elems * sizeof(VT));
    const __amdgpu_buffer_rsrc_t r_out = make_rsrc(a.out + tok0 * d, tok_elems * 4u);
    // the log of this memory's tokens of the call: one row of W segments per token
    const uint32_t log_tok = (uint32_t)a.W * row_bytes;
    const __amdgpu_buffer_rsrc_t r_log =
        make_rsrc(LOG ? static_cast<const char*>(a.log) + (size_t)bh * a.Ts * log_tok : nullptr,
                  LOG ? (uint32_t)T * log_tok : 0u);

    // positions of this lane
    const int pos0 = (wave * 2) * 8 + g, pos1 = pos0 + 8;
    const uint32_t lpos0 = pos0 < a.W ? (uint32_t)pos0 * row_bytes + lane_off : kOOB;
    const uint32_t lpos1 = pos1 < a.W ? (uint32_t)pos1 * row_bytes + lane_off : kOOB;
    const uint4* ring_lane = g_ring + el;   // the zero entry
    uint4* ring_w = g_ring + kEntryU4 + el; // entry 0 of the stored segments
    // record loads: lane i < 16 fetches record 16w + i of a token, lane 16 the header
    const uint32_t rec_lane = lane < 16 ? (uint32_t)(16 * wave + lane) * 16u : (uint32_t)kPos * 16u;
    const uint32_t elem0 = (uint32_t)(chunk * SEG + el * E);  // this lane's first element
    const uint32_t v_lane = elem0 * (uint32_t)sizeof(VT);
    const uint32_t o_lane = elem0 * 4u; // out: the 8 lanes of group 0 of one wave store E floats each
    // lanes >= 17 park their (unused) record load in the wave's spare entry; an
    // index into the one array (not a choice of pointers) keeps the compiler
    // certain that the store does not touch the stage buffers
    const bool parks = lane < kRecPerWave;
    const int spare = kRecSlots * kWaves * kRecPerWave + wave;

    // Sentinels for the virtual tokens before 0: a slot past the memory, no
    // store, weight 0, nothing forwarded; gates 0 and v, out offsets past their buffers.
    const uint4 sent_rec = make_uint4(N | (1u << 31), N, 0u, 0u);
    const uint4 sent_hdr = make_uint4(0u, 0u, tok_elems * (uint32_t)sizeof(VT), tok_elems * 4u);
    const uint4 sent_lane = lane < 16 ? sent_rec : sent_hdr;
    if (lane < kRecPerWave) {
#pragma unroll
        for (int z = 0; z < ZR; ++z)
            g_rec[(z * kWaves + wave) * kRecPerWave + lane] = sent_lane;
    }
    const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
    if (wave == 0 && lane < kEntryU4)
        g_ring[lane] = zero4;
    __syncthreads();

    // Per-token state on its way through the pipeline, token t in [(t - S0) mod 6]
    // (records in [(t - S0) mod 4]):
    uint4 rl[ZL];          // record loads (lanes < 17), issued four pairs ahead, parked two pairs later
    uint4 vr[ZS][NV];      // this lane's values of v (8 bytes: the first half), issued two pairs ahead
    uint4 wset[ZS][2];     // its write slots' segments (zero when forwarded), issued two pairs ahead
    uint4 rset[ZS][2];     // its read slots' segments (zero when forwarded), issued two pairs ahead
    uint32_t soff[ZS][2];  // store offsets of the write slots (past the memory: no store)
#pragma unroll
    for (int z = 0; z < ZL; ++z)
        rl[z] = sent_lane;
#pragma unroll
    for (int z = 0; z < ZS; ++z) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            vr[z][i] = zero4;
        wset[z][0] = wset[z][1] = rset[z][0] = rset[z][1] = zero4;
        soff[z][0] = soff[z][1] = kOOB;
    }

    // this lane's records and the header of the token in record slot Z
    auto records = [&](auto zc, uint4& r0, uint4& r1, uint4& hd) __attribute__((always_inline)) {
        const uint4* rw = g_rec + (decltype(zc)::value * kWaves + wave) * kRecPerWave;
        r0 = rw[g];
        r1 = rw[8 + g];
        hd = rw[16];
    };

    // The values of this lane's two slots: the staged segments plus, for a
    // forwarded slot, its ring entry (one of the two is zero).
    auto slot_values = [&](const uint4 (&ss)[2], uint32_t f0, uint32_t f1, float (&m0)[E], float (&m1)[E])
        __attribute__((always_inline)) {
        C::unpack(ss[0], m0);
        C::unpack(ss[1], m1);
        if (forwards(f0, f1)) {
            float r0[E], r1[E];
            C::unpack(*ring_src(f0, ring_lane), r0);
            C::unpack(*ring_src(f1, ring_lane), r1);
#pragma unroll
            for (int q = 0; q < E; ++q) {
                m0[q] += r0[q];
                m1[q] += r1[q];
            }
        }
    };

    // Write, first half: this lane's share of the prediction of the decayed
    // slots, summed over the wave into red; the slots' values are left in m0, m1
    // for the second half (no ring entry they come from changes in between: a
    // pair overwrites the entries of tokens 11 and 12 back, a slot forwards from
    // at most 7 back).
    auto partials = [&](const uint4 (&ws)[2], const uint4& r0, const uint4& r1, float alpha, float4* red,
                        float (&m0)[E], float (&m1)[E]) __attribute__((always_inline)) {
        slot_values(ws, r0.x, r1.x, m0, m1);
        const CT w0 = __uint_as_float(r0.z), w1 = __uint_as_float(r1.z), al = alpha;
        CT acc[E];
#pragma unroll
        for (int q = 0; q < E; ++q)
            acc[q] = predict2<CT>(al, w0, m0[q], w1, m1[q]);
        reduce_to_part<E, CT>(acc, red, wave, el, lane);
    };

    // The stored bits of this lane's two write slots before the write: the staged
    // segment, or the ring entry a forwarded slot comes from.
    auto old_bits = [&](const uint4 (&ss)[2], uint32_t f0, uint32_t f1, uint4& o0, uint4& o1)
        __attribute__((always_inline)) {
        constexpr uint32_t kField = 0x3FFu << kSlotBits;
        o0 = ss[0];
        o1 = ss[1];
        if (forwards(f0, f1)) {
            if (f0 & kField)
                o0 = *ring_src(f0, ring_lane);
            if (f1 & kField)
                o1 = *ring_src(f1, ring_lane);
        }
    };

    // Write, second half (after the barrier that publishes red): the delta-rule
    // update of this lane's slots (values m0, m1 from the first half, decayed
    // exactly as there), stored into the ring entry of the token in ring slot J;
    // with LOG, the slots' bits before the update in o0, o1.
    auto update = [&](auto jc, const uint4 (&ws)[2], const uint4& r0, const uint4& r1, float alpha, float beta,
                      const uint4 (&vraw)[NV], const float4* red, const float (&m0)[E], const float (&m1)[E],
                      uint4& p0, uint4& p1, uint4& o0, uint4& o1) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        CT vh[E];
        sum_waves<E, CT>(red, el, vh);
        // pin the use of v here: unpacking it earlier (the compiler would, at the
        // top of the loop) waits for a load still in flight
        uint4 u[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            u[i] = vraw[i];
            asm volatile("" : "+v"(u[i].x), "+v"(u[i].y), "+v"(u[i].z), "+v"(u[i].w));
        }
        float vv[E];
        if constexpr (sizeof(VT) == 2) {
            const uint32_t w[4] = {u[0].x, u[0].y, u[0].z, u[0].w};
#pragma unroll
            for (int i = 0; i < E / 2; ++i) {
                vv[2 * i] = bf16_lo(w[i]);
                vv[2 * i + 1] = bf16_hi(w[i]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const uint4& w = u[q / 4];
                vv[q] = __uint_as_float(q % 4 == 0 ? w.x : q % 4 == 1 ? w.y : q % 4 == 2 ? w.z : w.w);
            }
        }
        if constexpr (LOG)
            old_bits(ws, r0.x, r1.x, o0, o1);
        const CT w0 = __uint_as_float(r0.z), w1 = __uint_as_float(r1.z), al = alpha, be = beta;
        CT y0[E], y1[E];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const CT dlt = delta<CT>(be, vv[q], vh[q]);
            y0[q] = updated<CT>(al, m0[q], w0, dlt);
            y1[q] = updated<CT>(al, m1[q], w1, dlt);
        }
        p0 = C::pack(y0);
        p1 = C::pack(y1);
        ring_w[J * kPos * kEntryU4 + pos0 * kEntryU4] = p0;
        ring_w[J * kPos * kEntryU4 + pos1 * kEntryU4] = p1;
    };

    // Read: this lane's read slots of the token in record slot Z (after its write),
    // the wave's share of out left in ored.
    auto read_phase = [&](auto zc, const uint4 (&rs)[2], float4* ored) __attribute__((always_inline)) {
        uint4 r0, r1, hd;
        records(zc, r0, r1, hd);
        float q0[E], q1[E];
        slot_values(rs, r0.y, r1.y, q0, q1);
        const float rw0 = __uint_as_float(r0.w), rw1 = __uint_as_float(r1.w);
        float oa[E];
#pragma unroll
        for (int q = 0; q < E; ++q)
            oa[q] = read2(rw0, q0[q], rw1, q1[q]);
        reduce_to_part<E, float>(oa, ored, wave, el, lane);
    };

    // Issue for token u (record slot Z, register slot S): its slot rows and v, and
    // the records of token u + 4 into rl[(u - S0) mod 4].
    auto issue = [&](auto zc, auto sc, int u) __attribute__((always_inline)) {
        constexpr int S = decltype(sc)::value;
        uint4 u0, u1, hu;
        records(zc, u0, u1, hu);
        const uint32_t ow0 = __umul24(u0.x & ((1u << kSlotBits) - 1u), mem_row) + lane_off;
        const uint32_t ow1 = __umul24(u1.x & ((1u << kSlotBits) - 1u), mem_row) + lane_off;
        const uint32_t or0 = __umul24(u0.y & ((1u << kSlotBits) - 1u), mem_row) + lane_off;
        const uint32_t or1 = __umul24(u1.y & ((1u << kSlotBits) - 1u), mem_row) + lane_off;
        // a forwarded write slot is not loaded (top bit of y); a forwarded read slot is the sentinel
        wset[S][0] = ldseg<SEGB>(r_mem, (u0.y >> 31) ? kOOB : ow0);
        wset[S][1] = ldseg<SEGB>(r_mem, (u1.y >> 31) ? kOOB : ow1);
        rset[S][0] = ldseg<SEGB>(r_mem, or0);
        rset[S][1] = ldseg<SEGB>(r_mem, or1);
        soff[S][0] = (u0.x >> 31) ? kOOB : ow0;
        soff[S][1] = (u1.x >> 31) ? kOOB : ow1;
        if constexpr (VB == 4) {
            vr[S][0] = make_uint4((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r_v, hu.z + v_lane, 0, 0), 0u, 0u, 0u);
        } else if constexpr (VB == 8) {
            const i32x2_t w2 = __builtin_amdgcn_raw_buffer_load_b64(r_v, hu.z + v_lane, 0, 0);
            vr[S][0] = make_uint4((uint32_t)w2[0], (uint32_t)w2[1], 0u, 0u);
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                vr[S][i] = ld128(r_v, hu.z + v_lane + 16u * i);
        }
        const uint32_t ro = (uint32_t)(u + 4) * (uint32_t)(kRecs * 16) + rec_lane;
        rl[decltype(zc)::value % ZL] = ld128(r_plan, lane < kRecPerWave ? ro : kOOB);
    };

    // out of the token in record slot Z from the partials in ored: wave `owner`
    // sums and its group 0 stores; every wave still issues the stores (past the
    // buffer elsewhere), so all waves count the same memory operations
    auto store_out = [&](auto zc, const float4* ored, int owner) __attribute__((always_inline)) {
        float o[E];
#pragma unroll
        for (int q = 0; q < E; ++q)
            o[q] = 0.f;
        uint32_t off = kOOB;
        if (wave == owner) {
            const uint4 hd = g_rec[(decltype(zc)::value * kWaves + wave) * kRecPerWave + 16];
            sum_waves<E, float>(ored, el, o);
            off = g == 0 ? (hd.w & ~kDepFlag) + o_lane : kOOB;
        }
        if constexpr (E == 2) {
            __builtin_amdgcn_raw_buffer_store_b64((i32x2_t){(int)__float_as_uint(o[0]), (int)__float_as_uint(o[1])},
                                                  r_out, off, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NO; ++i)
                st128(r_out, off == kOOB ? kOOB : off + 16u * i,
                      make_uint4(__float_as_uint(o[4 * i]), __float_as_uint(o[4 * i + 1]),
                                 __float_as_uint(o[4 * i + 2]), __float_as_uint(o[4 * i + 3])));
        }
    };

    // Pair (s, s+1), s = S0 + ZR*blk + j0: record and ring slots j0, j0+1, register
    // slots j0 mod 6, j0+1 mod 6.
    const int blocks = (T + 2 - kS0 + ZR - 1) / ZR;
    for (int blk = 0; blk < blocks; ++blk) {
        static_for<ZR / 2>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j0 = 2 * decltype(jc)::value, j1 = j0 + 1;
            constexpr int n0 = (j0 + 4) % ZR, n1 = (j0 + 5) % ZR;   // pair k+2
            constexpr int p0 = (j0 + ZR - 2) % ZR, p1 = (j0 + ZR - 1) % ZR; // pair k-1
            const int s = kS0 + blk * ZR + j0;

            // this pair's slot rows and v and pair k+2's records have landed; every
            // store of pair k-2 is done and, after the barrier, visible to every wave,
            // as are pair k-1's ring entries
            wait_vmcnt<K>();
            barrier_lds();
            g_rec[parks ? (n0 * kWaves + wave) * kRecPerWave + lane : spare] = rl[n0 % ZL];
            g_rec[parks ? (n1 * kWaves + wave) * kRecPerWave + lane : spare] = rl[n1 % ZL];

            // ---- read of pair k-1 (its register slots are then free)
            read_phase(std::integral_constant<int, p0>{}, rset[p0 % ZS], g_ored);
            read_phase(std::integral_constant<int, p1>{}, rset[p1 % ZS], g_ored + kPartU4);

            // ---- issue pair k+2 into those register slots
            issue(std::integral_constant<int, n0>{}, std::integral_constant<int, n0 % ZS>{}, s + 4);
            issue(std::integral_constant<int, n1>{}, std::integral_constant<int, n1 % ZS>{}, s + 5);

            // ---- write of this pair
            uint4 a0, a1, ha, b0, b1, hb;
            records(std::integral_constant<int, j0>{}, a0, a1, ha);
            records(std::integral_constant<int, j1>{}, b0, b1, hb);
            uint4 ya0, ya1, yb0, yb1, oa0, oa1, ob0, ob1;
            float ma0[E], ma1[E], mb0[E], mb1[E];
            partials(wset[j0 % ZS], a0, a1, __uint_as_float(ha.x), g_red, ma0, ma1);
            partials(wset[j1 % ZS], b0, b1, __uint_as_float(hb.x), g_red + kPartU4, mb0, mb1);
            barrier_lds();
            store_out(std::integral_constant<int, p0>{}, g_ored, 0);
            store_out(std::integral_constant<int, p1>{}, g_ored + kPartU4, 1);
            update(std::integral_constant<int, j0>{}, wset[j0 % ZS], a0, a1, __uint_as_float(ha.x),
                   __uint_as_float(ha.y), vr[j0 % ZS], g_red, ma0, ma1, ya0, ya1, oa0, oa1);
            update(std::integral_constant<int, j1>{}, wset[j1 % ZS], b0, b1, __uint_as_float(hb.x),
                   __uint_as_float(hb.y), vr[j1 % ZS], g_red + kPartU4, mb0, mb1, yb0, yb1, ob0, ob1);
            if (__builtin_amdgcn_readfirstlane(hb.w) & kDepFlag) {
                // token s+1 writes a slot token s writes: redo its write now that
                // token s's values are in the ring
                barrier_lds();
                partials(wset[j1 % ZS], b0, b1, __uint_as_float(hb.x), g_red + kPartU4, mb0, mb1);
                barrier_lds();
                update(std::integral_constant<int, j1>{}, wset[j1 % ZS], b0, b1, __uint_as_float(hb.x),
                       __uint_as_float(hb.y), vr[j1 % ZS], g_red + kPartU4, mb0, mb1, yb0, yb1, ob0, ob1);
            }
            stseg<SEGB>(r_mem, soff[j0 % ZS][0], ya0);
            stseg<SEGB>(r_mem, soff[j0 % ZS][1], ya1);
            stseg<SEGB>(r_mem, soff[j1 % ZS][0], yb0);
            stseg<SEGB>(r_mem, soff[j1 % ZS][1], yb1);
            if constexpr (LOG) {
                // tokens outside [0, T) and positions past W log nothing (offsets past the buffer)
                const uint32_t la = (s >= 0 && s < T) ? (uint32_t)s * log_tok : kOOB;
                const uint32_t lb = (s + 1 >= 0 && s + 1 < T) ? (uint32_t)(s + 1) * log_tok : kOOB;
                stseg<SEGB>(r_log, la == kOOB || lpos0 == kOOB ? kOOB : la + lpos0, oa0);
                stseg<SEGB>(r_log, la == kOOB || lpos1 == kOOB ? kOOB : la + lpos1, oa1);
                stseg<SEGB>(r_log, lb == kOOB || lpos0 == kOOB ? kOOB : lb + lpos0, ob0);
                stseg<SEGB>(r_log, lb == kOOB || lpos1 == kOOB ? kOOB : lb + lpos1, ob1);
            }
        });
    }
}

} // namespace

namespace {
template <class ST, class VT, int SEGB>
void launch_typed_staged(const ScanArgs& a, dim3 grid, dim3 block, hipStream_t stream)
{
    if (a.log)
        hipLaunchKernelGGL((sdm_scan_staged_kernel<ST, VT, true, SEGB>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((sdm_scan_staged_kernel<ST, VT, false, SEGB>), grid, block, 0, stream, a);
}
} // namespace

hipError_t launch_sdm_scan_staged(const ScanArgs& a, const ScanPlan& p, bool state_bf16, bool in_bf16,
                                  hipStream_t stream)
{
    const int seg = p.seg_bytes / (state_bf16 ? 2 : 4);
    if (!p.staged || p.waves != kWaves || a.d % seg != 0 || a.W > kPos ||
        (p.seg_bytes != 128 && !((p.seg_bytes == 64 || p.seg_bytes == 32) && state_bf16)))
        return hipErrorInvalidValue;
    // the log of a call: one memory's tokens of a chunk addressable by 32-bit offsets
    if (a.log && (uint64_t)a.T * a.W * a.d * (state_bf16 ? 2u : 4u) >= (1ull << 32) - 16u)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)p.grid), block(kWaves * 64);
    if (state_bf16) {
        if (p.seg_bytes == 32)
            in_bf16 ? launch_typed_staged<uint16_t, uint16_t, 32>(a, grid, block, stream)
                    : launch_typed_staged<uint16_t, float, 32>(a, grid, block, stream);
        else if (p.seg_bytes == 64)
            in_bf16 ? launch_typed_staged<uint16_t, uint16_t, 64>(a, grid, block, stream)
                    : launch_typed_staged<uint16_t, float, 64>(a, grid, block, stream);
        else
            in_bf16 ? launch_typed_staged<uint16_t, uint16_t, 128>(a, grid, block, stream)
                    : launch_typed_staged<uint16_t, float, 128>(a, grid, block, stream);
    } else {
        in_bf16 ? launch_typed_staged<float, uint16_t, 128>(a, grid, block, stream)
                : launch_typed_staged<float, float, 128>(a, grid, block, stream);
    }
    return hipGetLastError();
}

} // namespace sdm

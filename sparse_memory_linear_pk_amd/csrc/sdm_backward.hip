// The backward pass of the SDM layer (float32 or bf16 state): reverse-mode
// differentiation of the forward (SDM blog post, section "How does SDM
// work?", its "Write & Read" subsection and the caption of the figure "The SDM
// mechanism, end to end"), with the selected slots held fixed and the state
// rounding passed straight through.
//
// Per token, the forward decays the W write slots (x_i = a M[n_i]), predicts
// vhat = sum_i w_i x_i, writes M[n_i] = x_i + w_i delta with
// delta = beta (v - vhat), then reads out = sum_j r_j M[m_j].  Walking the
// tokens backwards with G = dL/dM after the token:
//   read:  dr_j = <dout, M[m_j]>,  G[m_j] += r_j dout
//   write: g_i = G[n_i], ddelta = sum_i w_i g_i, dv = beta ddelta,
//          dbeta = <ddelta, v - vhat>, dvhat = -beta ddelta,
//          dw_i = <g_i, delta> + <dvhat, x_i>, dx_i = g_i + w_i dvhat,
//          dalpha = sum_i <dx_i, M_old[n_i]>, G[n_i] = a dx_i,
//          and M[n_i] is restored to M_old[n_i] from the forward's log.
// The state gradient is independent per slot element, like the forward, so
// grad_scan_kernel keeps the forward's decomposition: one workgroup per
// (memory, 128-byte column) walks all tokens in reverse.  It loads token t-1's
// slots while it works on token t; grad_conflict_kernel flags the tokens whose
// slots meet the next token's, and only those load again after token t's stores.  Its dot products over
// d (dr, dw, dalpha, dbeta) leave as per-column partial sums; grad_rows_kernel
// adds them in column order, applies the softmax's derivative
// dsigma_i = w_i (dw_i - sum_k w_k dw_k) and sends dsigma to the query halves
// (dq) and, as dense rows over the sub-keys, to grad_subkey_kernel, which
// forms dK[h][half] = sum over the rows of head h of dsigma-row x query-half.
#include "scan_cell.h"

namespace sdm {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ void load4(const float* p, float (&x)[4])
{
    const float4 u = *reinterpret_cast<const float4*>(p);
    x[0] = u.x;
    x[1] = u.y;
    x[2] = u.z;
    x[3] = u.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&x)[4])
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_lo(u.x);
    x[1] = bf16_hi(u.x);
    x[2] = bf16_lo(u.y);
    x[3] = bf16_hi(u.y);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8])
{
    const float4 u = *reinterpret_cast<const float4*>(p), w = *reinterpret_cast<const float4*>(p + 4);
    x[0] = u.x;
    x[1] = u.y;
    x[2] = u.z;
    x[3] = u.w;
    x[4] = w.x;
    x[5] = w.y;
    x[6] = w.z;
    x[7] = w.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8])
{
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(q[i]);
        x[2 * i + 1] = bf16_hi(q[i]);
    }
}
template <int E, class T> __device__ __forceinline__ void loadE(const T* p, float (&x)[E])
{
    if constexpr (E == 4)
        load4(p, x);
    else
        load8(p, x);
}
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// E float32 gradient values of a lane from / into GU 16-byte pieces
template <int GU, int E> __device__ __forceinline__ void unpack_g(const uint4 (&u)[GU], float (&x)[E])
{
    static_assert(E == 4 * GU, "gradient pieces");
#pragma unroll
    for (int i = 0; i < GU; ++i) {
        x[4 * i] = __uint_as_float(u[i].x);
        x[4 * i + 1] = __uint_as_float(u[i].y);
        x[4 * i + 2] = __uint_as_float(u[i].z);
        x[4 * i + 3] = __uint_as_float(u[i].w);
    }
}
template <int E> __device__ __forceinline__ uint4 pack_g(const float (&x)[E], int i)
{
    return make_uint4(__float_as_uint(x[4 * i]), __float_as_uint(x[4 * i + 1]), __float_as_uint(x[4 * i + 2]),
                      __float_as_uint(x[4 * i + 3]));
}

// the sum over the 8 lanes of a lane group (lanes differing in bits 0..2), in a fixed tree
__device__ __forceinline__ float sum8(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x;
}

// 16 gradient bytes at a 64-bit address (global memory instructions, one per access)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4_t global_u32x4;
__device__ __forceinline__ uint4 gld(const float* p)
{
    return __builtin_bit_cast(uint4, *(const global_u32x4*)(p));
}
__device__ __forceinline__ void gst(float* p, const uint4& v) { *(global_u32x4*)(p) = __builtin_bit_cast(u32x4_t, v); }

// ST: state element (float or bf16 bits); the gradient is float32 either way.
// A workgroup owns 128 bytes of every memory row (E = 4 float32 or 8 bf16
// values per lane) and the matching E float32 values per lane of the gradient
// rows (16 or 32 bytes).
// WIDE: one memory's gradient is 4 GiB or more (the 8B shape's float32 gradient
// of a bf16 state, 6.3 GB), past what a buffer offset reaches: it is then read
// and written with 64-bit addresses, and a position past W (whose slot is -1)
// addresses the lane's own entry of a small workspace sink instead of a place
// past the buffer, so every access is still issued on every path.
template <class ST, class VT, bool WIDE>
__global__ __launch_bounds__(kWaves * 64) void grad_scan_kernel(GradArgs a)
{
    constexpr int E = 16 / (int)sizeof(ST);
    constexpr int GU = E / 4; // 16-byte gradient pieces per lane and position
    __shared__ __attribute__((aligned(16))) uint4 s_g[64 * 8 * GU]; // read slots' gradients after the read
    __shared__ int32_t s_rslot[64];
    __shared__ __attribute__((aligned(16))) float s_y[kWaves * 8 * E];
    __shared__ __attribute__((aligned(16))) float s_d[kWaves * 8 * E];
    __shared__ float s_al[kWaves];

    const int ncol = a.ncol; // d * sizeof(ST) / 128
    const int bh = blockIdx.x / ncol, col = blockIdx.x % ncol;
    const int b = bh / a.H, h = bh % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, el = lane & 7;
    const int W = a.W, P = 2 * a.W + 2;
    const long N = (long)a.S * a.S;
    // slot row to slot row in the memory and in the gradient (ms elements of each)
    const uint32_t row_bytes = (uint32_t)a.ms * (uint32_t)sizeof(ST), grow_bytes = (uint32_t)a.ms * 4u;
    const uint32_t lane_off = (uint32_t)col * 128u + (uint32_t)el * 16u;
    const uint32_t glane_off = (uint32_t)col * (128u * GU) + (uint32_t)el * (16u * GU);
    const size_t mem_el = (size_t)bh * N * a.ms; // first element of memory bh
    ST* const mem = static_cast<ST*>(a.mem);
    const ST* const log = static_cast<const ST*>(a.log);
    const __amdgpu_buffer_rsrc_t r_mem = make_rsrc(mem + mem_el, (uint32_t)(N * row_bytes));
    const __amdgpu_buffer_rsrc_t r_g = make_rsrc(a.G + mem_el, WIDE ? 0u : (uint32_t)(N * grow_bytes));
    const int pos[2] = {wave * 16 + g, wave * 16 + 8 + g};
    const bool live[2] = {pos[0] < W, pos[1] < W};
    float* const g_mem = a.G + mem_el + glane_off / 4u;       // this lane's gradient values of slot 0 (WIDE)
    float* const g_sink = a.sink + threadIdx.x * (4u * GU);   // where a position past W goes (WIDE)
    // gradient piece u of slot `slot` at position p: load and store
    auto gload = [&](int p, int32_t slot, int u) __attribute__((always_inline)) -> uint4 {
        if constexpr (WIDE)
            return gld((live[p] ? g_mem + (size_t)(uint32_t)slot * a.ms : g_sink) + 4 * u);
        else
            return ld128(r_g, live[p] ? (uint32_t)slot * grow_bytes + glane_off + 16u * u : kOOB);
    };
    auto gstore = [&](int p, int32_t slot, int u, const uint4& v) __attribute__((always_inline)) {
        if constexpr (WIDE)
            gst((live[p] ? g_mem + (size_t)(uint32_t)slot * a.ms : g_sink) + 4 * u, v);
        else
            st128(r_g, live[p] ? (uint32_t)slot * grow_bytes + glane_off + 16u * u : kOOB, v);
    };
    const int e0 = col * (128 / (int)sizeof(ST)) + el * E; // this lane's first element of the row

    // A token's slots are fetched two tokens ahead, its other state-independent
    // inputs (weights, the log of its write slots, dout, v, the gates) and its
    // slot rows one token ahead.  The rows are loaded before the next token's
    // stores, which is correct unless the two tokens share a slot (the conflict
    // flag): then they are loaded again once the next token's stores are
    // visible.  Buffers alternate between even and odd steps (the loop is
    // unrolled by two), so no value still in flight is ever copied: a copy would
    // make the compiler wait for every memory operation issued before it,
    // stores included.  Every load is issued on every path (a position past W
    // or a token before 0 reads a valid entry whose value is then dropped): a
    // load skipped on some path makes the compiler's count of loads in flight
    // conservative at the join, and it then waits for the newest loads too.
    struct Ids {
        int32_t ws[2], rs[2];
    };
    struct Meta {
        float ww[2], rw[2];
        uint4 wo[2];
        float go[E], vv[E];
        float al, be;
        int conflict;
    };
    struct Rows4 {
        uint4 rv[2], rg[2][GU], wg[2][GU]; // read slots' memory and gradient, write slots' gradient
    };
    const int posc[2] = {min(pos[0], W - 1), min(pos[1], W - 1)}; // a valid position to read
    auto fetch_ids = [&](int t, Ids& m) __attribute__((always_inline)) {
        const long row = ((long)b * a.T + t) * a.H + h;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int32_t w = a.idx[0][row * W + posc[p]], r = a.idx[1][row * W + posc[p]];
            m.ws[p] = live[p] ? w : -1;
            m.rs[p] = live[p] ? r : -1;
        }
    };
    auto fetch_meta = [&](int t, Meta& m) __attribute__((always_inline)) {
        const long row = ((long)b * a.T + t) * a.H + h;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // raw values: a position past W is zeroed where it is used (a select here
            // would wait for the load)
            m.ww[p] = a.wt[0][row * W + posc[p]];
            m.rw[p] = a.wt[1][row * W + posc[p]];
            m.wo[p] = *reinterpret_cast<const uint4*>(log + (((size_t)bh * a.T + t) * W + posc[p]) * a.d + e0);
        }
        loadE<E>(a.dout + (size_t)row * a.d + e0, m.go);
        loadE<E>(static_cast<const VT*>(a.v) + (size_t)row * a.d + e0, m.vv);
        m.al = a.alpha[row];
        m.be = a.beta[row];
        m.conflict = a.conflict[row];
    };
    auto issue = [&](const Ids& m, Rows4& st) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            st.rv[p] = ld128(r_mem, live[p] ? (uint32_t)m.rs[p] * row_bytes + lane_off : kOOB);
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                st.rg[p][u] = gload(p, m.rs[p], u);
                st.wg[p][u] = gload(p, m.ws[p], u);
            }
        }
    };
    // step t of parity X = (T-1-t) & 1 starts with: I[X] = slots of t, I[1-X] = slots of
    // t-1, Mt[X] = the rest of t, St[X] = t's rows (in flight)
    Ids I[2];
    Meta Mt[2];
    Rows4 St[2];
    fetch_ids(a.T - 1, I[0]);
    fetch_meta(a.T - 1, Mt[0]);
    issue(I[0], St[0]);
    fetch_ids(max(a.T - 2, 0), I[1]);

    for (int tp = a.T - 1; tp >= 0; tp -= 2)
      static_for<2>([&](auto pc) __attribute__((always_inline)) {
        constexpr int X = decltype(pc)::value, Y = 1 - X; // this step's buffers, the next step's
        const int t = tp - X;
        if (t < 0)
            return;
        const Ids cur = I[X]; // fetched two steps ago
        fetch_ids(max(t - 2, 0), I[X]);
        issue(I[Y], St[Y]); // token t-1's rows (for t = 0, token 0's again, unused)
        fetch_meta(max(t - 1, 0), Mt[Y]);
        const long row = ((long)b * a.T + t) * a.H + h;
        const int32_t ws[2] = {cur.ws[0], cur.ws[1]}, rs[2] = {cur.rs[0], cur.rs[1]};
        const Meta& m = Mt[X];
        const float ww[2] = {live[0] ? m.ww[0] : 0.f, live[1] ? m.ww[1] : 0.f};
        const float rw[2] = {live[0] ? m.rw[0] : 0.f, live[1] ? m.rw[1] : 0.f};
        const uint4 wo[2] = {m.wo[0], m.wo[1]}; // dead positions: zeroed when unpacked below
        const Rows4& sc = St[X];
        float go[E], vv[E];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            go[q] = m.go[q];
            vv[q] = m.vv[q];
        }
        const float al = m.al, be = m.be;
        float* part = a.part + ((size_t)row * ncol + col) * P;
        // the read: the memory holds its state after token t's write
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float m[E], gr[E];
            Cell<ST>::unpack(sc.rv[p], m);
            unpack_g<GU>(sc.rg[p], gr);
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < E; ++q) {
                s = __builtin_fmaf(go[q], m[q], s);
                gr[q] = __builtin_fmaf(rw[p], go[q], gr[q]);
            }
            s = sum8(s);
            if (el == 0 && live[p])
                part[pos[p]] = s;
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const uint4 pk = pack_g(gr, u);
                s_g[(pos[p] * 8 + el) * GU + u] = pk;
                gstore(p, rs[p], u, pk);
            }
        }
        if (el == 0) {
            s_rslot[pos[0]] = rs[0];
            s_rslot[pos[1]] = rs[1];
        }
        // a token that reads one of its own write slots (flag bit 1, the same for the whole
        // workgroup) waits for every wave's read gradients in LDS; the others skip the wait
        const bool intra = (__builtin_amdgcn_readfirstlane(m.conflict) & 2) != 0;
        if (intra)
            __syncthreads();

        // the write: a write slot also read by this token takes its gradient after the read
        float gw[2][E], x[2][E], old[2][E];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // branch-free (every entry read, the tests combined bitwise): the short-circuit
            // form of this select has been compiled wrongly here, keeping the candidate
            // index on lanes that did not match
            int hit = -1;
            const int32_t wsp = ws[p];
            if (intra) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = el * 8 + u;
                    const int32_t sv = s_rslot[j];
                    hit = ((j < W) & (sv == wsp) & (wsp >= 0)) ? j : hit;
                }
#pragma unroll
                for (int m = 1; m < 8; m <<= 1)
                    hit = max(hit, __shfl_xor(hit, m));
            }
            if (hit >= 0) {
                uint4 hv[GU];
#pragma unroll
                for (int u = 0; u < GU; ++u)
                    hv[u] = s_g[(hit * 8 + el) * GU + u];
                unpack_g<GU>(hv, gw[p]);
            } else {
                unpack_g<GU>(sc.wg[p], gw[p]);
            }
            Cell<ST>::unpack(live[p] ? wo[p] : make_uint4(0u, 0u, 0u, 0u), old[p]);
#pragma unroll
            for (int q = 0; q < E; ++q)
                x[p][q] = al * old[p][q];
        }
        {
            float ay[E], ad[E];
#pragma unroll
            for (int q = 0; q < E; ++q) {
                ay[q] = __builtin_fmaf(ww[1], x[1][q], ww[0] * x[0][q]);
                ad[q] = __builtin_fmaf(ww[1], gw[1][q], ww[0] * gw[0][q]);
            }
            reduce_to_part<E, float>(ay, reinterpret_cast<float4*>(s_y), wave, el, lane);
            reduce_to_part<E, float>(ad, reinterpret_cast<float4*>(s_d), wave, el, lane);
        }
        __syncthreads();
        float yh[E], dd[E], dl[E], dyh[E];
        sum_waves<E, float>(reinterpret_cast<const float4*>(s_y), el, yh);
        sum_waves<E, float>(reinterpret_cast<const float4*>(s_d), el, dd);
#pragma unroll
        for (int q = 0; q < E; ++q) {
            dl[q] = be * (vv[q] - yh[q]);
            dyh[q] = -be * dd[q];
        }
        float pa = 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float ng[E];
            float sw = 0.f;
#pragma unroll
            for (int q = 0; q < E; ++q) {
                const float dx = __builtin_fmaf(ww[p], dyh[q], gw[p][q]);
                sw = __builtin_fmaf(gw[p][q], dl[q], sw);
                sw = __builtin_fmaf(dyh[q], x[p][q], sw);
                pa = __builtin_fmaf(dx, old[p][q], pa);
                ng[q] = al * dx;
            }
            sw = sum8(sw);
            if (el == 0 && live[p])
                part[W + pos[p]] = sw;
#pragma unroll
            for (int u = 0; u < GU; ++u)
                gstore(p, ws[p], u, pack_g(ng, u));
            st128(r_mem, live[p] ? (uint32_t)ws[p] * row_bytes + lane_off : kOOB, wo[p]); // the slot before the token
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1)
            pa += __shfl_xor(pa, m);
        if (lane == 0)
            s_al[wave] = pa;
        if (wave == 0 && g == 0) {
            float sb = 0.f;
            float4 o;
#pragma unroll
            for (int q = 0; q < E; ++q)
                sb = __builtin_fmaf(dd[q], vv[q] - yh[q], sb);
            sb = sum8(sb);
            if (el == 0)
                part[2 * W + 1] = sb;
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                o.x = be * dd[4 * u];
                o.y = be * dd[4 * u + 1];
                o.z = be * dd[4 * u + 2];
                o.w = be * dd[4 * u + 3];
                *reinterpret_cast<float4*>(a.dv + (size_t)row * a.d + e0 + 4 * u) = o;
            }
        }
        __syncthreads(); // token t's stores are visible to the workgroup's loads from here on
        if (threadIdx.x == 0)
            part[2 * W] = (s_al[0] + s_al[1]) + (s_al[2] + s_al[3]);
        if (t >= 1 && (Mt[Y].conflict & 1))
            issue(I[Y], St[Y]);
      });
}

// flag[row] of token u of memory (b, h): bit 0 when a slot token u writes or
// reads is also written or read by token u + 1 (never for the last token), bit 1
// when token u reads one of the slots it writes.  One wave per row: each of token
// u's slots is broadcast and compared with token u + 1's and with u's own.
__global__ __launch_bounds__(256) void grad_conflict_kernel(const int32_t* idx_w, const int32_t* idx_r,
                                                            int32_t* flag, long R, int T, int H, int W)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long row = (long)blockIdx.x * 4 + wave;
    if (row >= R)
        return; // the whole wave
    const int u = (int)((row / H) % T);
    const bool last = u == T - 1;
    const long nrow = last ? row : row + H; // (b, u + 1, h)
    const bool live = lane < W;
    const int32_t aw = live ? idx_w[row * W + lane] : -1, ar = live ? idx_r[row * W + lane] : -1;
    const int32_t nw = live && !last ? idx_w[nrow * W + lane] : -2;
    const int32_t nr = live && !last ? idx_r[nrow * W + lane] : -2;
    bool hit = false, own = false;
    for (int k = 0; k < W; ++k) {
        const int32_t x = __shfl(aw, k), y = __shfl(ar, k);
        hit = hit || nw == x || nr == x || nw == y || nr == y;
        own = own || (live && aw == y);
    }
    const bool any = __builtin_amdgcn_ballot_w64(hit) != 0u;
    const bool any_own = __builtin_amdgcn_ballot_w64(own) != 0u;
    if (lane == 0)
        flag[row] = (any ? 1 : 0) | (any_own ? 2 : 0);
}

constexpr int kRowsPerBlock = 4;

// One wave per row: the column partials added in column order, the softmax's
// derivative for the write and the read weights, dq, and the dense dsigma rows.
template <class VT>
__global__ __launch_bounds__(kRowsPerBlock * 64) void grad_rows_kernel(GradArgs a, long R)
{
    extern __shared__ float s_dsrow[]; // [kRowsPerBlock][S]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long row = (long)blockIdx.x * kRowsPerBlock + wave;
    if (row >= R)
        return; // the whole wave; no block barriers below
    const int W = a.W, P = 2 * a.W + 2, S = a.S, dh = a.dh, dk = 2 * a.dh, ncol = a.ncol;
    const int h = (int)(row % a.H);
    float* my = s_dsrow + wave * S;
    const bool live = lane < W;

    float up[2] = {0.f, 0.f}; // dL/d(write weight), dL/d(read weight) of this lane's position
    float sa = 0.f, sb = 0.f;
    const float* pr = a.part + (size_t)row * ncol * P;
    for (int c = 0; c < ncol; ++c, pr += P) {
        if (live) {
            up[1] += pr[lane];
            up[0] += pr[W + lane];
        }
        if (lane == 0) {
            sa += pr[2 * W];
            sb += pr[2 * W + 1];
        }
    }
    if (lane == 0) {
        a.dalpha[row] = sa;
        a.dbeta[row] = sb;
    }
    const VT* K = static_cast<const VT*>(a.subkeys) + (size_t)h * 2 * S * dh;
    for (int set = 0; set < 2; ++set) {
        const double w = live ? (double)a.wt[set][row * W + lane] : 0.0;
        const int32_t n = live ? a.idx[set][row * W + lane] : 0;
        double mean = w * (double)up[set];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1)
            mean += __shfl_xor(mean, o);
        const float dsig = live ? (float)(w * ((double)up[set] - mean)) : 0.f;
        const int key[2] = {n / S, n % S};
        for (int half = 0; half < 2; ++half) {
            // dq: sum over the selected slots of dsigma times the slot's sub-key of this half
            // (the shuffles run on the whole wave: a half narrower than 64 leaves lanes idle in the sum only)
            const VT* Kh = K + (size_t)half * S * dh;
            for (int j0 = 0; j0 < dh; j0 += 64) {
                const int j = j0 + lane;
                float acc = 0.f;
                for (int k = 0; k < W; ++k) {
                    const float dsk = __shfl(dsig, k);
                    const int kk = __shfl(key[half], k);
                    if (j < dh)
                        acc = __builtin_fmaf(dsk, load1(Kh + (size_t)kk * dh + j), acc);
                }
                if (j < dh)
                    a.dq[set][(size_t)row * dk + half * dh + j] = acc;
            }
            // the dense row of dsigma summed per sub-key, for the sub-key gradient
            for (int s2 = lane; s2 < S; s2 += 64)
                my[s2] = 0.f;
            float tot = 0.f;
            bool first = true;
            for (int k = 0; k < W; ++k) {
                const int kk = __shfl(key[half], k);
                const float dk_ = __shfl(dsig, k);
                if (kk == key[half]) {
                    tot += dk_;
                    first = first && k >= lane;
                }
            }
            if (live && first)
                my[key[half]] = tot;
            float* dst = a.ds + (((size_t)set * R + row) * 2 + half) * S;
            for (int s2 = lane; s2 < S; s2 += 64)
                dst[s2] = my[s2];
        }
    }
}

// dK[h][half][s][j] = sum over k of ds[k][s] q[k][j], k running over both
// query sets and every row of head h; split over k, one 64 x 64 tile of (s, j)
// per workgroup, 4 x 4 outputs per thread.
constexpr int kTile = 64, kKB = 16;

template <class VT>
__global__ __launch_bounds__(256) void grad_subkey_kernel(GradArgs a, long R, long rows_per_split)
{
    __shared__ __attribute__((aligned(16))) float As[kKB][kTile];
    __shared__ __attribute__((aligned(16))) float Bs[kKB][kTile];
    const int S = a.S, dh = a.dh, dk = 2 * a.dh, H = a.H;
    const int s0 = blockIdx.x * kTile, j0 = blockIdx.y * kTile;
    const int z = blockIdx.z; // (split, h, half)
    const int half = z & 1, h = (z >> 1) % H, split = (z >> 1) / H;
    const long BT = (long)a.B * a.T, K = 2 * BT;
    const long k0 = (long)split * rows_per_split, k1 = k0 + rows_per_split < K ? k0 + rows_per_split : K;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int lk = tid >> 4, l4 = (tid & 15) * 4;
    float acc[4][4] = {};
    for (long kb = k0; kb < k1; kb += kKB) {
        {
            const long k = kb + lk;
            const bool ok = k < k1;
            const int set = ok ? (int)(k / BT) : 0;
            const long r = ok ? (k % BT) * H + h : 0;
            const float* dsr = a.ds + (((size_t)set * R + r) * 2 + half) * S;
            const VT* qr = static_cast<const VT*>(a.q[set]) + (size_t)r * dk + (size_t)half * dh;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + l4 + u, j = j0 + l4 + u;
                As[lk][l4 + u] = ok && s < S ? dsr[s] : 0.f;
                Bs[lk][l4 + u] = ok && j < dh ? load1(qr + j) : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kKB; ++kk) {
            const float4 av = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
            const float4 bv = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
            const float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[u][v] = __builtin_fmaf(ar[u], br[v], acc[u][v]);
        }
        __syncthreads();
    }
    float* out = a.sub_part + (((size_t)split * H + h) * 2 + half) * S * dh;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int s = s0 + ty * 4 + u;
        if (s >= S)
            continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int j = j0 + tx * 4 + v;
            if (j < dh)
                out[(size_t)s * dh + j] = acc[u][v];
        }
    }
}

// the splits added in split order
__global__ __launch_bounds__(256) void grad_subkey_sum_kernel(const float* part, float* dsub, long n, int nsplit)
{
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float s = 0.f;
    for (int k = 0; k < nsplit; ++k)
        s += part[(size_t)k * n + i];
    dsub[i] = s;
}

} // namespace

size_t grad_part_floats(int B, int H, int T, int d, int W, bool state_bf16)
{
    return (size_t)B * T * H * (size_t)(d / (state_bf16 ? 64 : 32)) * (size_t)(2 * W + 2);
}

int grad_sub_splits(int B, int H, int T, int S, int dh)
{
    const long tiles = (long)((S + kTile - 1) / kTile) * ((dh + kTile - 1) / kTile) * H * 2;
    const long K = 2L * B * T;
    long n = (1024 + tiles - 1) / tiles;
    const long by_rows = (K + 255) / 256; // at least 256 rows of k per split
    n = n < by_rows ? n : by_rows;
    n = n < 64 ? n : 64;
    return (int)(n < 1 ? 1 : n);
}

hipError_t launch_grad_conflicts(const GradArgs& a, hipStream_t stream)
{
    const long R = (long)a.B * a.T * a.H;
    hipLaunchKernelGGL(grad_conflict_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream, a.idx[0], a.idx[1],
                       a.conflict, R, a.T, a.H, a.W);
    return hipGetLastError();
}

hipError_t launch_grad_scan(const GradArgs& a, hipStream_t stream)
{
    const int seg = a.state_bf16 ? 64 : 32;
    if (a.d % seg || a.ncol != a.d / seg || a.W > 64 || a.W < 1 || a.ms < a.d || a.ms % 4)
        return hipErrorInvalidValue;
    // one memory's state rows are addressed with 32-bit buffer offsets; its float32
    // gradient too unless it reaches 4 GiB (then 64-bit addresses and the sink)
    const uint64_t N = (uint64_t)a.S * a.S;
    if (N * a.ms * (a.state_bf16 ? 2u : 4u) >= (1ull << 32))
        return hipErrorInvalidValue;
    const bool wide = N * a.ms * 4u >= (1ull << 32);
    if (wide && !a.sink)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.B * a.H * a.ncol)), block(kWaves * 64);
#define SDM_GRAD_SCAN(ST, VT)                                                                                        \
    do {                                                                                                             \
        if (wide)                                                                                                    \
            hipLaunchKernelGGL((grad_scan_kernel<ST, VT, true>), grid, block, 0, stream, a);                         \
        else                                                                                                         \
            hipLaunchKernelGGL((grad_scan_kernel<ST, VT, false>), grid, block, 0, stream, a);                        \
    } while (0)
    if (a.state_bf16) {
        if (a.in_bf16)
            SDM_GRAD_SCAN(uint16_t, uint16_t);
        else
            SDM_GRAD_SCAN(uint16_t, float);
    } else {
        if (a.in_bf16)
            SDM_GRAD_SCAN(float, uint16_t);
        else
            SDM_GRAD_SCAN(float, float);
    }
#undef SDM_GRAD_SCAN
    return hipGetLastError();
}

hipError_t launch_grad_rows(const GradArgs& a, hipStream_t stream)
{
    const long R = (long)a.B * a.T * a.H;
    dim3 grid((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * 64);
    const size_t lds = (size_t)kRowsPerBlock * a.S * sizeof(float);
    if (a.in_bf16)
        hipLaunchKernelGGL((grad_rows_kernel<uint16_t>), grid, block, lds, stream, a, R);
    else
        hipLaunchKernelGGL((grad_rows_kernel<float>), grid, block, lds, stream, a, R);
    return hipGetLastError();
}

hipError_t launch_grad_subkeys(const GradArgs& a, hipStream_t stream)
{
    const long R = (long)a.B * a.T * a.H, K = 2L * a.B * a.T;
    const long per = (K + a.nsplit - 1) / a.nsplit;
    dim3 grid((unsigned)((a.S + kTile - 1) / kTile), (unsigned)((a.dh + kTile - 1) / kTile),
              (unsigned)(a.nsplit * a.H * 2)),
        block(256);
    if (a.in_bf16)
        hipLaunchKernelGGL((grad_subkey_kernel<uint16_t>), grid, block, 0, stream, a, R, per);
    else
        hipLaunchKernelGGL((grad_subkey_kernel<float>), grid, block, 0, stream, a, R, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const long n = (long)a.H * 2 * a.S * a.dh;
    hipLaunchKernelGGL(grad_subkey_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a.sub_part,
                       a.dsub, n, a.nsplit);
    return hipGetLastError();
}

} // namespace sdm

// The backward pass of the SDM layer (float32 state): reverse-mode
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
// (memory, 128-byte column) walks all tokens in reverse.  Its dot products over
// d (dr, dw, dalpha, dbeta) leave as per-column partial sums; grad_rows_kernel
// adds them in column order, applies the softmax's derivative
// dsigma_i = w_i (dw_i - sum_k w_k dw_k) and sends dsigma to the query halves
// (dq) and, as dense rows over the sub-keys, to grad_subkey_kernel, which
// forms dK[h][half] = sum over the rows of head h of dsigma-row x query-half.
#include "scan_cell.h"

namespace sdm {
namespace {

constexpr int kWaves = 4;
constexpr int E = 4; // float32 state: 4 values per lane, 32 per 128-byte column

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
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// the sum over the 8 lanes of a lane group (lanes differing in bits 0..2), in a fixed tree
__device__ __forceinline__ float sum8(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x;
}

template <class VT>
__global__ __launch_bounds__(kWaves * 64) void grad_scan_kernel(GradArgs a)
{
    __shared__ __attribute__((aligned(16))) uint4 s_g[64 * 8]; // read slots' gradients after the read
    __shared__ int32_t s_rslot[64];
    __shared__ __attribute__((aligned(16))) float s_y[kWaves * 8 * E];
    __shared__ __attribute__((aligned(16))) float s_d[kWaves * 8 * E];
    __shared__ float s_al[kWaves];

    const int ncol = a.d / 32;
    const int bh = blockIdx.x / ncol, col = blockIdx.x % ncol;
    const int b = bh / a.H, h = bh % a.H;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, el = lane & 7;
    const int W = a.W, P = 2 * a.W + 2;
    const long N = (long)a.S * a.S;
    const uint32_t row_bytes = (uint32_t)a.d * 4u;
    const uint32_t lane_off = (uint32_t)col * 128u + (uint32_t)el * 16u;
    const size_t mem_off = (size_t)bh * N * a.d;
    const __amdgpu_buffer_rsrc_t r_mem = make_rsrc(a.mem + mem_off, (uint32_t)(N * row_bytes));
    const __amdgpu_buffer_rsrc_t r_g = make_rsrc(a.G + mem_off, (uint32_t)(N * row_bytes));
    const int pos[2] = {wave * 16 + g, wave * 16 + 8 + g};
    const bool live[2] = {pos[0] < W, pos[1] < W};
    const int e0 = col * 32 + el * E; // this lane's first element of the row

    // Everything of a token that does not depend on the state (its slots and
    // weights, the log of its write slots, dout, v and the gates) is fetched one
    // token ahead, so that a token starts with its slot loads.
    struct Meta {
        int32_t ws[2], rs[2];
        float ww[2], rw[2];
        uint4 wo[2];
        float go[E], vv[E];
        float al, be;
    };
    auto fetch = [&](int t, Meta& m) __attribute__((always_inline)) {
        const long row = ((long)b * a.T + t) * a.H + h;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            m.ws[p] = live[p] ? a.idx[0][row * W + pos[p]] : -1;
            m.rs[p] = live[p] ? a.idx[1][row * W + pos[p]] : -1;
            m.ww[p] = live[p] ? a.wt[0][row * W + pos[p]] : 0.f;
            m.rw[p] = live[p] ? a.wt[1][row * W + pos[p]] : 0.f;
            m.wo[p] = live[p] ? *reinterpret_cast<const uint4*>(a.log + (((size_t)bh * a.T + t) * W + pos[p]) * a.d + e0)
                              : make_uint4(0u, 0u, 0u, 0u);
        }
        load4(a.dout + (size_t)row * a.d + e0, m.go);
        load4(static_cast<const VT*>(a.v) + (size_t)row * a.d + e0, m.vv);
        m.al = a.alpha[row];
        m.be = a.beta[row];
    };
    Meta cur;
    fetch(a.T - 1, cur);

    for (int t = a.T - 1; t >= 0; --t) {
        const long row = ((long)b * a.T + t) * a.H + h;
        const int32_t ws[2] = {cur.ws[0], cur.ws[1]}, rs[2] = {cur.rs[0], cur.rs[1]};
        const float ww[2] = {cur.ww[0], cur.ww[1]}, rw[2] = {cur.rw[0], cur.rw[1]};
        const uint4 wo[2] = {cur.wo[0], cur.wo[1]};
        uint4 rv[2], rg[2], wg[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            rv[p] = ld128(r_mem, live[p] ? (uint32_t)rs[p] * row_bytes + lane_off : kOOB);
            rg[p] = ld128(r_g, live[p] ? (uint32_t)rs[p] * row_bytes + lane_off : kOOB);
            wg[p] = ld128(r_g, live[p] ? (uint32_t)ws[p] * row_bytes + lane_off : kOOB);
        }
        float go[E], vv[E];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            go[q] = cur.go[q];
            vv[q] = cur.vv[q];
        }
        const float al = cur.al, be = cur.be;
        if (t > 0)
            fetch(t - 1, cur);
        float* part = a.part + ((size_t)row * ncol + col) * P;

        // the read: the memory holds its state after token t's write
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float m[E], gr[E];
            Cell<float>::unpack(rv[p], m);
            Cell<float>::unpack(rg[p], gr);
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < E; ++q) {
                s = __builtin_fmaf(go[q], m[q], s);
                gr[q] = __builtin_fmaf(rw[p], go[q], gr[q]);
            }
            s = sum8(s);
            if (el == 0 && live[p])
                part[pos[p]] = s;
            const uint4 pk = Cell<float>::pack(gr);
            s_g[pos[p] * 8 + el] = pk;
            st128(r_g, live[p] ? (uint32_t)rs[p] * row_bytes + lane_off : kOOB, pk);
        }
        if (el == 0) {
            s_rslot[pos[0]] = rs[0];
            s_rslot[pos[1]] = rs[1];
        }
        __syncthreads();

        // the write: a write slot also read by this token takes its gradient after the read
        float gw[2][E], x[2][E], old[2][E];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            int hit = -1;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                hit = (ws[p] >= 0 && el * 8 + u < W && s_rslot[el * 8 + u] == ws[p]) ? el * 8 + u : hit;
#pragma unroll
            for (int m = 1; m < 8; m <<= 1)
                hit = max(hit, __shfl_xor(hit, m));
            Cell<float>::unpack(hit >= 0 ? s_g[hit * 8 + el] : wg[p], gw[p]);
            Cell<float>::unpack(wo[p], old[p]);
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
            const uint32_t off = live[p] ? (uint32_t)ws[p] * row_bytes + lane_off : kOOB;
            st128(r_g, off, Cell<float>::pack(ng));
            st128(r_mem, off, wo[p]); // the slot's value before the token
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
            o.x = be * dd[0];
            o.y = be * dd[1];
            o.z = be * dd[2];
            o.w = be * dd[3];
            *reinterpret_cast<float4*>(a.dv + (size_t)row * a.d + e0) = o;
        }
        __syncthreads();
        if (threadIdx.x == 0)
            part[2 * W] = (s_al[0] + s_al[1]) + (s_al[2] + s_al[3]);
    }
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
    const int W = a.W, P = 2 * a.W + 2, S = a.S, dh = a.dh, dk = 2 * a.dh, ncol = a.d / 32;
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

size_t grad_part_floats(int B, int H, int T, int d, int W)
{
    return (size_t)B * T * H * (size_t)(d / 32) * (size_t)(2 * W + 2);
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

hipError_t launch_grad_scan(const GradArgs& a, hipStream_t stream)
{
    if (a.d % 32 || a.W > 64 || a.W < 1)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)(a.B * a.H * (a.d / 32))), block(kWaves * 64);
    if (a.in_bf16)
        hipLaunchKernelGGL((grad_scan_kernel<uint16_t>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((grad_scan_kernel<float>), grid, block, 0, stream, a);
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

// Host side of libsdm: the C ABI declared in include/sdm.h.
//
// Validates arguments on the host before anything reaches the device, owns the
// addressing workspace, and launches the kernels in pipeline order on the
// caller's stream: pk_score + pk_topk for the write queries, the same for the
// read queries, sdm_plan, then sdm_scan.  Addressing never reads the memory,
// so the pipeline has no feedback from the scan.
#include "sdm.h"
#include "sdm_internal.h"

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

namespace {

constexpr uint32_t kMagic = 0x53444d31u; // "SDM1"
thread_local char g_err[512] = "";

sdm_status fail(sdm_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

enum Kind { K_SCORE = 0, K_SELECT = 1, K_PLAN = 2, K_SCAN = 3, K_STEP = 4, K_TRAIN = 5, K_BWD_SCAN = 6,
            K_BWD_ROWS = 7, K_BWD_SUB = 8, K_PROJ = 9 };

struct TimedLaunch {
    Kind kind;
    hipEvent_t start, stop;
};

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// sdm_step_static's scratch: on the step's two-launch path, the slot ids then
// (256-byte aligned) the weights of both query sets, 2*B*H*W of each.  One copy
// per device, kept until the process ends; host code reaches it only through the
// device address hipGetSymbolAddress returns for the current device.
constexpr size_t kStepScratchBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kStepScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// A forward longer than kOneChunk tokens runs its scan in chunks: kFirstChunk
// tokens first, then each chunk 3/2 of the one before (rounded down to a
// multiple of 64 tokens) up to kMaxChunk.  A remainder shorter than
// kMaxChunk / 2 joins the chunk before it where the two fit in kMaxChunk;
// otherwise those tokens form two chunks of about half each, so no chunk
// exceeds kMaxChunk tokens.  The addressing and plan of chunk c + 1 run on a
// second stream while chunk c scans; beside a running scan they get only the
// CU resources the scan leaves free and stretch to most of its time, so a
// chunk may be only a little longer than the one before it.  The first chunk,
// whose preparation nothing hides, is short; the later ones are long, since
// every scan launch costs about 50 us of pipeline fill and drain.
constexpr int kOneChunk = 2048;
constexpr int kFirstChunk = 640;
constexpr int kMaxChunk = 3072;

struct Chunking {
    std::vector<int> start; // first token of each chunk, then T
    int C() const { return (int)start.size() - 1; }
    int t0(int ci) const { return start[ci]; }
    int len(int ci) const { return start[ci + 1] - start[ci]; }
};

Chunking chunking_of(const sdm_config& c)
{
    Chunking k;
    k.start.push_back(0);
    int t = 0, len = c.T <= kOneChunk ? c.T : kFirstChunk;
    while (true) {
        int next = t + len;
        if (next >= c.T || c.T - next < kMaxChunk / 2)
            next = c.T - t <= kMaxChunk ? c.T : t + (((c.T - t) / 2) & ~63);
        k.start.push_back(next);
        if (next == c.T)
            return k;
        t = next;
        len = std::min(kMaxChunk, (len * 3 / 2) & ~63);
    }
}

struct Layout {
    size_t scores, idx, wt, plan, frag, kmax, kstat, step, total;
    std::vector<size_t> plan_off; // byte offset of each chunk's plan
};

Layout layout_of(const sdm_config& c, const Chunking& k, const std::vector<sdm::ScanPlan>& plans)
{
    const size_t rows = (size_t)c.B * c.T * c.H;
    Layout L;
    // the forward's scores: binary16 for bf16 inputs (they only locate the
    // candidates of the exact selection), float32 otherwise
    L.scores = align_up(rows * 2 * (size_t)c.n_sub * (c.in_dtype == SDM_BF16 ? 2u : 4u));
    L.idx = align_up(rows * (size_t)c.W * sizeof(int32_t));
    L.wt = align_up(rows * (size_t)c.W * sizeof(float));
    L.plan = 0;
    for (int ci = 0; ci < k.C(); ++ci) {
        L.plan_off.push_back(L.plan);
        L.plan += align_up(sdm::plan_bytes(plans[ci], c.B, c.H, k.len(ci), c.W));
    }
    L.frag = align_up(sdm::pk_score_frag_bytes(c.H, c.n_sub, c.dk / 2));
    // sdm_step's slot ids and weights, write then read set: 2*B*H*W of each,
    // apart from the forward's buffers (which hold B*T*H*W and T may be 1)
    L.step = align_up(2 * (size_t)c.B * c.H * c.W * sizeof(int32_t));
    L.kmax = align_up(2 * (size_t)c.H * sdm::kAbsmaxParts * sizeof(float)); // partial max |K| per sub-key table
    // the tables' mean rows and spreads, for the fused scoring's thresholds
    L.kstat = align_up(sdm::subkey_stats_floats(c.H, c.dk / 2) * sizeof(float));
    L.total = 2 * L.scores + 2 * (L.idx + L.wt) + L.plan + L.frag + L.kmax + L.kstat + 2 * L.step;
    return L;
}

// Elements from one slot row of a memory to the next in the state tensors.
int mem_stride_of(const sdm_config& c) { return c.mem_stride ? c.mem_stride : c.d; }

// The integer a caller stored in a dtype field.  A C caller (or a binding) may
// store any int there, and loading an enum object that holds a value outside its
// enumerators is undefined in C++, so unchecked configs are read through this.
static_assert(sizeof(sdm_dtype) == sizeof(int) && sizeof(sdm_status) == sizeof(int),
              "sdm_dtype and sdm_status are int-sized in the C ABI");

int dtype_bits(const sdm_dtype& f)
{
    int v;
    memcpy(&v, &f, sizeof v);
    return v;
}

// The shape checks that need no scan plan (and allocate nothing).
sdm_status check_shape(const sdm_config* c)
{
    if (!c)
        return fail(SDM_ERR_INVALID_ARG, "config is NULL");
    if (c->B < 1 || c->H < 1 || c->T < 1 || c->d < 1 || c->n_sub < 1 || c->dk < 1 || c->k < 1 || c->W < 1)
        return fail(SDM_ERR_INVALID_ARG, "every size must be >= 1 (B=%d H=%d T=%d d=%d S=%d dk=%d k=%d W=%d)", c->B,
                    c->H, c->T, c->d, c->n_sub, c->dk, c->k, c->W);
    const int in_dt = dtype_bits(c->in_dtype), st_dt = dtype_bits(c->state_dtype);
    if ((in_dt != SDM_F32 && in_dt != SDM_BF16) || (st_dt != SDM_F32 && st_dt != SDM_BF16))
        return fail(SDM_ERR_INVALID_ARG, "unknown dtype (in %d, state %d)", in_dt, st_dt);
    if (c->dk % 2)
        return fail(SDM_ERR_INVALID_ARG, "dk=%d must be even (two halves)", c->dk);
    if (c->k > c->n_sub)
        return fail(SDM_ERR_INVALID_ARG, "k=%d exceeds the %d sub-keys of a half", c->k, c->n_sub);
    if ((long)c->W > (long)c->k * c->k)
        return fail(SDM_ERR_INVALID_ARG, "W=%d exceeds the k*k=%d candidates", c->W, c->k * c->k);
    const int dh = c->dk / 2;
    static const int kHalfWidths[] = {16, 32, 48, 64, 96, 128, 192, 256};
    bool dh_ok = false;
    for (int w : kHalfWidths)
        dh_ok |= dh == w;
    if (!dh_ok)
        return fail(SDM_ERR_UNSUPPORTED, "dk/2=%d: supported half widths are 16, 32, 48, 64, 96, 128, 192, 256", dh);
    if (c->k > 64 || c->W > 64)
        return fail(SDM_ERR_UNSUPPORTED, "k=%d, W=%d: at most 64 each", c->k, c->W);
    if (c->n_sub > 1024)
        return fail(SDM_ERR_UNSUPPORTED, "S=%d: at most 1024 sub-keys per half", c->n_sub);
    if (c->d % 8)
        return fail(SDM_ERR_UNSUPPORTED, "d=%d must be a multiple of 8", c->d);
    const size_t s = c->state_dtype == SDM_BF16 ? 2 : 4;
    if (c->mem_stride != 0 && (c->mem_stride < c->d || (c->mem_stride * s) % 16 != 0))
        return fail(SDM_ERR_INVALID_ARG, "mem_stride=%d: 0 (dense rows), or at least d=%d with rows a multiple of 16 "
                    "bytes", c->mem_stride, c->d);
    const int ms = mem_stride_of(*c);
    const size_t mem_bytes = (size_t)c->n_sub * c->n_sub * ms * s;
    if (mem_bytes >= (1ull << 32))
        return fail(SDM_ERR_UNSUPPORTED, "one memory is %zu bytes; at most 2^32 - 1", mem_bytes);
    if ((long)c->H * c->n_sub * 2 * 4 * 128 >= (1l << 31))
        return fail(SDM_ERR_UNSUPPORTED, "H*S=%ld: at most 2^21 - 1", (long)c->H * c->n_sub);
    if ((long)c->B * c->T * c->H > (1l << 31) / 64)
        return fail(SDM_ERR_UNSUPPORTED, "B*T*H=%ld rows is too many", (long)c->B * c->T * c->H);
    return SDM_OK;
}

sdm_status check_config(const sdm_config* c, std::vector<sdm::ScanPlan>* plans)
{
    const sdm_status s = check_shape(c);
    if (s != SDM_OK)
        return s;
    const Chunking k = chunking_of(*c);
    const long N = (long)c->n_sub * c->n_sub;
    const int ms = mem_stride_of(*c);
    plans->assign(k.C(), sdm::ScanPlan{});
    for (int ci = 0; ci < k.C(); ++ci)
        if (!sdm::plan_scan(c->B, c->H, k.len(ci), c->d, ms, c->W, N, c->state_dtype == SDM_BF16,
                            c->in_dtype == SDM_BF16, &(*plans)[ci]))
            return fail(SDM_ERR_UNSUPPORTED, "no scan layout for d=%d W=%d", c->d, c->W);
    return SDM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

} // namespace

struct sdm_ctx {
    uint32_t magic;
    sdm_config cfg;
    hipStream_t stream;  // the caller's: scans run here
    hipStream_t aux;     // addressing and plans of a chunked forward after its first chunk (default priority)
    std::vector<hipEvent_t> e_plan; // chunk c's plan is written
    int device;
    Chunking ck;
    std::vector<sdm::ScanPlan> plans; // scan layout of each chunk
    void* block;
    Layout L;
    void* scores[2]; // the forward's scores of each query set (binary16 for bf16 inputs)
    int32_t* idx[2];
    float* wt[2];
    uint4* plan_buf;
    void* frag;
    int32_t* step_idx;   // [2][B*H][W] (sdm_step)
    float* step_wt;      // [2][B*H][W]
    float* kmax;         // [H][2][kAbsmaxParts]: partial max |K| of each sub-key table (the exact selection's bound)
    float* kstat;        // [H][2][dh + 4]: mean row and spread of each table (the fused scoring's thresholds)
    bool timing;
    std::vector<TimedLaunch> pending;
    sdm_timing totals;
    // backward workspace, allocated by the first sdm_backward call
    void* bwd_block;
    float* part;
    float* ds;
    float* sub_part;
    int32_t* conflict;
    float* sink;
    int nsplit;
};

namespace {

sdm_status check_handle(sdm_handle h)
{
    if (!h || h->magic != kMagic)
        return fail(SDM_ERR_INVALID_ARG, "invalid or destroyed handle");
    return SDM_OK;
}

sdm_status hip_fail(hipError_t e, const char* what)
{
    return fail(SDM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Records events around one launch, on the stream it runs on, when timing is on.
struct Timer {
    sdm_ctx* h;
    Kind kind;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    Timer(sdm_ctx* h_, Kind k, hipStream_t s) : h(h_), kind(k), st(s)
    {
        if (h->timing && hipEventCreate(&a) == hipSuccess && hipEventCreate(&b) == hipSuccess)
            (void)hipEventRecord(a, st);
    }
    ~Timer()
    {
        if (a && b) {
            (void)hipEventRecord(b, st);
            h->pending.push_back({kind, a, b});
        }
    }
};

sdm::Rows all_rows(const sdm_config& c) { return sdm::Rows{c.B, c.H, c.T, c.T, 0}; }

sdm::Rows chunk_rows(const sdm_ctx* h, int ci)
{
    const sdm_config& c = h->cfg;
    return sdm::Rows{c.B, c.H, h->ck.len(ci), c.T, h->ck.t0(ci)};
}

// Whether the forward's addressing scores with the fused candidate search.
bool cand_path(const sdm_config& c) { return sdm::pk_cand_path(c.n_sub, c.dk / 2, c.k, c.in_dtype == SDM_BF16); }

// The per-call preparation of the sub-key tables: their MFMA operand order (bf16
// inputs), the largest magnitude of each table (the exact selection's bound)
// and, for the fused scoring, each table's mean row and spread.
hipError_t prepare_subkeys(sdm_ctx* h, const void* subkeys, hipStream_t st)
{
    const sdm_config& c = h->cfg;
    const bool bf16 = c.in_dtype == SDM_BF16;
    if (cand_path(c)) // all three in one pass over the tables
        return sdm::launch_subkey_prepare(subkeys, h->frag, h->kstat, h->kmax, c.H, c.n_sub, c.dk / 2, st);
    hipError_t e = hipSuccess;
    if (bf16)
        e = sdm::launch_pk_subkey_frag(subkeys, h->frag, c.H, c.n_sub, c.dk / 2, st);
    if (e == hipSuccess)
        e = sdm::launch_subkey_absmax(subkeys, h->kmax, c.H, c.n_sub, c.dk / 2, bf16, st);
    return e;
}

// frag: prepare the sub-key tables first (once per call that scores).
// exact: scores for the exact selection (run_select with q), stored as binary16
// for bf16 inputs; otherwise float32 (the stage seam).
sdm_status run_score(sdm_ctx* h, const void* q, const void* subkeys, void* scores, const sdm::Rows& r,
                     hipStream_t st, bool frag, bool exact = true)
{
    const sdm_config& c = h->cfg;
    const bool bf16 = c.in_dtype == SDM_BF16;
    hipError_t e = hipSuccess;
    if (frag)
        e = prepare_subkeys(h, subkeys, st);
    if (e == hipSuccess) {
        Timer t(h, K_SCORE, st); // pk_score alone
        e = exact && cand_path(c)
                ? sdm::launch_pk_score_cand(q, q, h->frag, h->kstat, scores, scores, 1, r, c.n_sub, c.dk / 2, c.k, st)
                : sdm::launch_pk_score(q, subkeys, h->frag, scores, r, c.n_sub, c.dk / 2, bf16, exact && bf16, st);
    }
    return e == hipSuccess ? SDM_OK : hip_fail(e, "pk_score launch");
}

// q and subkeys given (the forward's path): the scores that can reach a half's
// top k are made exact from them (h->kmax must be prepared; the scores are
// those of run_score with exact); q null: the float32 scores are taken as given
// (the stage seam).
sdm_status run_select(sdm_ctx* h, const void* scores, int32_t* idx, float* wt, const sdm::Rows& r, hipStream_t st,
                      const void* q, const void* subkeys)
{
    const sdm_config& c = h->cfg;
    Timer t(h, K_SELECT, st);
    hipError_t e = q && cand_path(c)
                       ? sdm::launch_pk_topk_cand(scores, scores, idx, idx, wt, wt, 1, r, c.n_sub, c.k, c.W, q, q,
                                                  subkeys, h->kmax, c.dk / 2, st)
                       : sdm::launch_pk_topk(scores, idx, wt, r, c.n_sub, c.k, c.W, q, subkeys, h->kmax, c.dk / 2,
                                             c.in_dtype == SDM_BF16, st);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "pk_topk launch");
}

const sdm::ScanPlan& plan_of(const sdm_ctx* h, int ci) { return h->plans[ci]; }

uint4* plan_region(const sdm_ctx* h, int ci)
{
    return reinterpret_cast<uint4*>(reinterpret_cast<char*>(h->plan_buf) + h->L.plan_off[ci]);
}

sdm_status run_plan(sdm_ctx* h, int ci, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                    const float* wt_r, const float* alpha, const float* beta, hipStream_t st)
{
    const sdm_config& c = h->cfg;
    Timer t(h, K_PLAN, st);
    hipError_t e = sdm::launch_sdm_plan(plan_of(h, ci), idx_w, wt_w, idx_r, wt_r, alpha, beta, plan_region(h, ci),
                                        chunk_rows(h, ci), c.W, c.d, (long)c.n_sub * c.n_sub, c.in_dtype == SDM_BF16,
                                        st);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_plan launch");
}

sdm_status run_scan(sdm_ctx* h, int ci, const void* v, void* mem, float* out, hipStream_t st, void* log = nullptr,
                    Kind kind = K_SCAN)
{
    const sdm_config& c = h->cfg;
    const sdm::ScanPlan& p = plan_of(h, ci);
    const sdm::Rows r = chunk_rows(h, ci);
    const size_t first = (size_t)r.t0 * c.H * c.d; // element of token t0 in sequence 0
    sdm::ScanArgs a;
    a.plan = plan_region(h, ci);
    a.ab = p.staged ? nullptr : reinterpret_cast<const float2*>(a.plan + (size_t)c.B * c.H * r.Tc * c.W);
    a.v = static_cast<const char*>(v) + first * (c.in_dtype == SDM_BF16 ? 2 : 4);
    a.mem = mem;
    a.out = out + first;
    a.log = log ? static_cast<char*>(log) + (size_t)r.t0 * c.W * c.d * (c.state_dtype == SDM_BF16 ? 2u : 4u) : nullptr;
    a.B = c.B;
    a.T = r.Tc;
    a.Ts = c.T;
    a.H = c.H;
    a.d = c.d;
    a.W = c.W;
    a.Tp = p.Tp;
    a.N = (long)c.n_sub * c.n_sub;
    a.ms = mem_stride_of(c);
    Timer t(h, kind, st);
    hipError_t e = sdm::launch_sdm_scan(a, p, c.state_dtype == SDM_BF16, c.in_dtype == SDM_BF16, st);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_scan launch");
}

// Scores and exact selection of both query sets for rows r, one launch each,
// into h->idx and h->wt, or into idx/wt (both sets) when given.
sdm_status run_address_pair(sdm_ctx* h, const sdm::Rows& r, const void* wq, const void* rq, const void* subkeys,
                            hipStream_t st, bool prepare, int32_t* const* idx = nullptr, float* const* wt = nullptr)
{
    int32_t* io0 = idx ? idx[0] : h->idx[0];
    int32_t* io1 = idx ? idx[1] : h->idx[1];
    float* wo0 = wt ? wt[0] : h->wt[0];
    float* wo1 = wt ? wt[1] : h->wt[1];
    const sdm_config& c = h->cfg;
    const bool bf16 = c.in_dtype == SDM_BF16;
    hipError_t e = prepare ? prepare_subkeys(h, subkeys, st) : hipSuccess;
    const bool cand = cand_path(c);
    if (e == hipSuccess) {
        Timer t(h, K_SCORE, st);
        e = cand ? sdm::launch_pk_score_cand(wq, rq, h->frag, h->kstat, h->scores[0], h->scores[1], 2, r, c.n_sub,
                                             c.dk / 2, c.k, st)
                 : sdm::launch_pk_score_pair(wq, rq, subkeys, h->frag, h->scores[0], h->scores[1], r, c.n_sub,
                                             c.dk / 2, bf16, st);
    }
    if (e != hipSuccess)
        return hip_fail(e, "pk_score launch");
    Timer t(h, K_SELECT, st);
    e = cand ? sdm::launch_pk_topk_cand(h->scores[0], h->scores[1], io0, io1, wo0, wo1, 2, r, c.n_sub, c.k, c.W, wq,
                                        rq, subkeys, h->kmax, c.dk / 2, st)
             : sdm::launch_pk_topk_pair(h->scores[0], h->scores[1], io0, io1, wo0, wo1, r, c.n_sub, c.k, c.W, wq, rq,
                                        subkeys, h->kmax, c.dk / 2, bf16, st);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "pk_topk launch");
}

// The addressing of both query sets for chunk ci, then its plan.
sdm_status run_chunk_front(sdm_ctx* h, int ci, const void* wq, const void* rq, const float* alpha, const float* beta,
                           const void* subkeys, hipStream_t st)
{
    const sdm_status s = run_address_pair(h, chunk_rows(h, ci), wq, rq, subkeys, st, ci == 0);
    return s == SDM_OK ? run_plan(h, ci, h->idx[0], h->wt[0], h->idx[1], h->wt[1], alpha, beta, st) : s;
}

// Scores and selection of both query sets for every row of the call, on st.
sdm_status run_address_all(sdm_ctx* h, const void* wq, const void* rq, const void* subkeys, hipStream_t st)
{
    return run_address_pair(h, all_rows(h->cfg), wq, rq, subkeys, st, true);
}

sdm_status forward_impl(sdm_ctx* h, const void* wq, const void* rq, const void* v, const float* alpha,
                        const float* beta, const void* subkeys, void* mem_inout, float* out, void* log);

sdm_status check_train_shape(const sdm_config& c, const char* who)
{
    const int seg = c.state_dtype == SDM_BF16 ? 64 : 32;
    if (c.d % seg)
        return fail(SDM_ERR_UNSUPPORTED, "%s: d=%d must be a multiple of %d (128-byte slot columns)", who, c.d, seg);
    const unsigned sb = c.state_dtype == SDM_BF16 ? 2u : 4u;
    const Chunking k = chunking_of(c);
    for (int ci = 0; ci < k.C(); ++ci)
        if ((uint64_t)k.len(ci) * c.W * c.d * sb >= (1ull << 32) - 16u)
            return fail(SDM_ERR_UNSUPPORTED, "%s: one memory's log of a %d-token chunk exceeds 4 GiB", who, k.len(ci));
    return SDM_OK;
}

} // namespace

extern "C" {

const char* sdm_status_str(sdm_status s)
{
    int code; // any int a C caller passed (an enum object out of its range may not be loaded in C++)
    memcpy(&code, &s, sizeof code);
    switch (code) {
    case SDM_OK: return "ok";
    case SDM_ERR_INVALID_ARG: return "invalid argument";
    case SDM_ERR_UNSUPPORTED: return "unsupported shape";
    case SDM_ERR_OOM: return "out of device memory";
    case SDM_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char* sdm_last_error(void) { return g_err; }

int sdm_mem_stride_hint(const sdm_config* cfg)
{
    if (!cfg)
        return 0;
    const long s = dtype_bits(cfg->state_dtype) == SDM_BF16 ? 2 : 4;
    const long row = (long)cfg->d * s; // bytes of a dense row (d is not validated here)
    if (row % 128 || row < 1024 || row >= (1l << 30))
        return cfg->d;
    const long units = row / 128; // 128-byte units of a dense row
    return (int)((units | 1) * 128 / s);
}

sdm_status sdm_workspace_bytes(const sdm_config* cfg, size_t* bytes)
{
    std::vector<sdm::ScanPlan> plans;
    sdm_status s = check_config(cfg, &plans);
    if (s != SDM_OK)
        return s;
    if (!bytes)
        return fail(SDM_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout_of(*cfg, chunking_of(*cfg), plans).total;
    return SDM_OK;
}

sdm_status sdm_create(const sdm_config* cfg, void* hip_stream, sdm_handle* out)
{
    g_err[0] = 0;
    if (!out)
        return fail(SDM_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    std::vector<sdm::ScanPlan> plans;
    sdm_status s = check_config(cfg, &plans);
    if (s != SDM_OK)
        return s;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    sdm_ctx* h = new (std::nothrow) sdm_ctx();
    if (!h)
        return fail(SDM_ERR_OOM, "host allocation failed");
    h->cfg = *cfg;
    h->stream = (hipStream_t)hip_stream;
    h->device = dev;
    h->plans = plans;
    h->ck = chunking_of(*cfg);
    h->L = layout_of(*cfg, h->ck, plans);
    h->aux = nullptr;
    h->timing = false;
    h->bwd_block = nullptr;
    h->part = h->ds = h->sub_part = h->sink = nullptr;
    h->conflict = nullptr;
    h->nsplit = 0;
    memset(&h->totals, 0, sizeof h->totals);
    e = hipMalloc(&h->block, h->L.total);
    if (e != hipSuccess) {
        const size_t total = h->L.total;
        delete h;
        (void)hipGetLastError();
        return fail(SDM_ERR_OOM, "workspace of %zu bytes: %s", total, hipGetErrorString(e));
    }
    char* p = (char*)h->block;
    for (int set = 0; set < 2; ++set) {
        h->scores[set] = p;
        p += h->L.scores;
    }
    for (int set = 0; set < 2; ++set) {
        h->idx[set] = (int32_t*)p;
        p += h->L.idx;
        h->wt[set] = (float*)p;
        p += h->L.wt;
    }
    h->plan_buf = (uint4*)p;
    p += h->L.plan;
    h->frag = p;
    p += h->L.frag;
    h->kmax = (float*)p;
    p += h->L.kmax;
    h->kstat = (float*)p;
    p += h->L.kstat;
    h->step_idx = (int32_t*)p;
    p += h->L.step;
    h->step_wt = (float*)p;
    if (h->ck.C() > 1) {
        e = hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking);
        h->e_plan.assign(h->ck.C(), nullptr);
        for (int ci = 0; ci < h->ck.C() && e == hipSuccess; ++ci)
            e = hipEventCreateWithFlags(&h->e_plan[ci], hipEventDisableTiming);
        if (e != hipSuccess) {
            for (hipEvent_t ev : h->e_plan)
                if (ev)
                    (void)hipEventDestroy(ev);
            if (h->aux)
                (void)hipStreamDestroy(h->aux);
            (void)hipFree(h->block);
            delete h;
            return hip_fail(e, "stream or event creation");
        }
    }
    h->magic = kMagic;
    *out = h;
    return SDM_OK;
}

sdm_status sdm_destroy(sdm_handle h)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    hipError_t e = hipStreamSynchronize(h->stream);
    if (h->aux) {
        const hipError_t ea = hipStreamSynchronize(h->aux);
        e = e == hipSuccess ? ea : e;
        for (hipEvent_t ev : h->e_plan)
            (void)hipEventDestroy(ev);
        (void)hipStreamDestroy(h->aux);
    }
    for (auto& tl : h->pending) {
        (void)hipEventDestroy(tl.start);
        (void)hipEventDestroy(tl.stop);
    }
    hipError_t e2 = hipFree(h->block);
    if (h->bwd_block) {
        const hipError_t e3 = hipFree(h->bwd_block);
        e2 = e2 == hipSuccess ? e3 : e2;
    }
    h->magic = 0;
    delete h;
    if (e != hipSuccess)
        return hip_fail(e, "hipStreamSynchronize");
    if (e2 != hipSuccess)
        return hip_fail(e2, "hipFree");
    return SDM_OK;
}

sdm_status sdm_score(sdm_handle h, const void* q, const void* subkeys, float* scores)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!q || !subkeys || !scores)
        return fail(SDM_ERR_INVALID_ARG, "sdm_score: NULL pointer");
    if (!aligned16(q) || !aligned16(subkeys) || !aligned4(scores))
        return fail(SDM_ERR_INVALID_ARG, "sdm_score: q and subkeys must be 16-byte aligned");
    return run_score(h, q, subkeys, scores, all_rows(h->cfg), h->stream, true, false);
}

sdm_status sdm_select(sdm_handle h, const float* scores, int32_t* idx, float* wt)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!scores || !idx || !wt)
        return fail(SDM_ERR_INVALID_ARG, "sdm_select: NULL pointer");
    if (!aligned4(scores) || !aligned4(idx) || !aligned4(wt))
        return fail(SDM_ERR_INVALID_ARG, "sdm_select: pointers must be 4-byte aligned");
    return run_select(h, scores, idx, wt, all_rows(h->cfg), h->stream, nullptr, nullptr);
}

sdm_status sdm_address(sdm_handle h, const void* q, const void* subkeys, int32_t* idx, float* wt)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!q || !subkeys || !idx || !wt)
        return fail(SDM_ERR_INVALID_ARG, "sdm_address: NULL pointer");
    if (!aligned16(q) || !aligned16(subkeys) || !aligned4(idx) || !aligned4(wt))
        return fail(SDM_ERR_INVALID_ARG, "sdm_address: misaligned pointer");
    s = run_score(h, q, subkeys, h->scores[0], all_rows(h->cfg), h->stream, true);
    return s != SDM_OK ? s : run_select(h, h->scores[0], idx, wt, all_rows(h->cfg), h->stream, q, subkeys);
}

sdm_status sdm_address_pair(sdm_handle h, const void* wq, const void* rq, const void* subkeys, int32_t* idx_w,
                            float* wt_w, int32_t* idx_r, float* wt_r)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !subkeys || !idx_w || !wt_w || !idx_r || !wt_r)
        return fail(SDM_ERR_INVALID_ARG, "sdm_address_pair: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(subkeys) || !aligned4(idx_w) || !aligned4(wt_w) ||
        !aligned4(idx_r) || !aligned4(wt_r))
        return fail(SDM_ERR_INVALID_ARG, "sdm_address_pair: misaligned pointer");
    int32_t* const idx[2] = {idx_w, idx_r};
    float* const wt[2] = {wt_w, wt_r};
    return run_address_pair(h, all_rows(h->cfg), wq, rq, subkeys, h->stream, true, idx, wt);
}

sdm_status sdm_scan_with(sdm_handle h, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r,
                         const float* wt_r, const void* v, const float* alpha, const float* beta, void* mem_inout,
                         float* out)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!idx_w || !wt_w || !idx_r || !wt_r || !v || !alpha || !beta || !mem_inout || !out)
        return fail(SDM_ERR_INVALID_ARG, "sdm_scan_with: NULL pointer");
    if (!aligned16(v) || !aligned16(mem_inout) || !aligned16(out) || !aligned4(idx_w) || !aligned4(wt_w) ||
        !aligned4(idx_r) || !aligned4(wt_r) || !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_scan_with: misaligned pointer");
    for (int ci = 0; ci < h->ck.C() && s == SDM_OK; ++ci) {
        s = run_plan(h, ci, idx_w, wt_w, idx_r, wt_r, alpha, beta, h->stream);
        if (s == SDM_OK)
            s = run_scan(h, ci, v, mem_inout, out, h->stream);
    }
    return s;
}

sdm_status sdm_forward(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                       const float* beta, const void* subkeys, void* mem_inout, float* out)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !v || !alpha || !beta || !subkeys || !mem_inout || !out)
        return fail(SDM_ERR_INVALID_ARG, "sdm_forward: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(v) || !aligned16(subkeys) || !aligned16(mem_inout) ||
        !aligned16(out) || !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_forward: misaligned pointer");
    return forward_impl(h, wq, rq, v, alpha, beta, subkeys, mem_inout, out, nullptr);
}

} // extern "C"

namespace {

// The forward's launches; with log, the scans also keep every write slot's old value.
sdm_status forward_impl(sdm_ctx* h, const void* wq, const void* rq, const void* v, const float* alpha,
                        const float* beta, const void* subkeys, void* mem_inout, float* out, void* log)
{
    sdm_status s = SDM_OK;
    const Kind kind = log ? K_TRAIN : K_SCAN;
    if (h->ck.C() == 1) {
        s = run_chunk_front(h, 0, wq, rq, alpha, beta, subkeys, h->stream);
        return s == SDM_OK ? run_scan(h, 0, v, mem_inout, out, h->stream, log, kind) : s;
    }
    // Chunked: the first chunk, whose preparation nothing hides, is addressed and
    // planned on the caller's stream (no wait between streams before its scan);
    // the addressing and plan of every later chunk go, in order, to the aux
    // stream, which starts after the first plan (so after everything the
    // caller's stream held before this call: its inputs and earlier calls' scans
    // of the plans about to be rewritten).  The scan of chunk c waits for its
    // plan on the caller's stream, so chunk c + 1's addressing runs while chunk
    // c scans.
    s = run_chunk_front(h, 0, wq, rq, alpha, beta, subkeys, h->stream);
    if (s != SDM_OK)
        return s;
    hipError_t e = hipEventRecord(h->e_plan[0], h->stream);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(h->aux, h->e_plan[0], 0);
    if (e != hipSuccess)
        return hip_fail(e, "stream ordering");
    for (int ci = 1; ci < h->ck.C(); ++ci) {
        if ((s = run_chunk_front(h, ci, wq, rq, alpha, beta, subkeys, h->aux)) != SDM_OK)
            return s;
        if ((e = hipEventRecord(h->e_plan[ci], h->aux)) != hipSuccess)
            return hip_fail(e, "stream ordering");
    }
    for (int ci = 0; ci < h->ck.C(); ++ci) {
        if (ci > 0 && (e = hipStreamWaitEvent(h->stream, h->e_plan[ci], 0)) != hipSuccess)
            return hip_fail(e, "stream ordering");
        if ((s = run_scan(h, ci, v, mem_inout, out, h->stream, log, kind)) != SDM_OK)
            return s;
    }
    return SDM_OK;
}

} // namespace

extern "C" {

sdm_status sdm_step(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                    const float* beta, const void* subkeys, void* mem_inout, float* out)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !v || !alpha || !beta || !subkeys || !mem_inout || !out)
        return fail(SDM_ERR_INVALID_ARG, "sdm_step: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(v) || !aligned16(subkeys) || !aligned16(mem_inout) ||
        !aligned16(out) || !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_step: misaligned pointer");
    const sdm_config& c = h->cfg;
    if (!sdm::step_supported(c.d, c.state_dtype == SDM_BF16))
        return fail(SDM_ERR_UNSUPPORTED, "sdm_step: d=%d: a slot row must be a multiple of 128 bytes", c.d);
    // the slot ids and weights of both query sets (two-launch path) go to the
    // step's own 2*B*H*W entries of the workspace
    Timer t(h, K_STEP, h->stream);
    hipError_t e = sdm::launch_sdm_step(wq, rq, v, alpha, beta, subkeys, mem_inout, out, h->step_idx, h->step_wt, c.B,
                                        c.H, c.d, mem_stride_of(c), c.n_sub, c.dk / 2, c.k, c.W, c.in_dtype == SDM_BF16,
                                        c.state_dtype == SDM_BF16, h->stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_step launch");
}

} // extern "C"

namespace {

// The device address of `scratch` on the current device, resolved on the first
// call on that device and kept.
sdm_status step_scratch(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SDM_ERR_UNSUPPORTED, "sdm_step_static: device %d (at most %d devices)", dev, kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return hip_fail(e, "hipGetSymbolAddress of the step scratch");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return SDM_OK;
}

} // namespace

extern "C" {

sdm_status sdm_step_static(const sdm_config* cfg, void* hip_stream, const void* wq, const void* rq, const void* v,
                           const float* alpha, const float* beta, const void* subkeys, void* mem_inout, float* out)
{
    sdm_status s = check_shape(cfg);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !v || !alpha || !beta || !subkeys || !mem_inout || !out)
        return fail(SDM_ERR_INVALID_ARG, "sdm_step_static: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(v) || !aligned16(subkeys) || !aligned16(mem_inout) ||
        !aligned16(out) || !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_step_static: misaligned pointer");
    const sdm_config& c = *cfg;
    if (!sdm::step_supported(c.d, c.state_dtype == SDM_BF16))
        return fail(SDM_ERR_UNSUPPORTED, "sdm_step_static: d=%d: a slot row must be a multiple of 128 bytes", c.d);
    const size_t n = 2 * (size_t)c.B * c.H * c.W; // slot ids (and weights) of both query sets
    if (2 * align_up(n * sizeof(int32_t)) > kStepScratchBytes)
        return fail(SDM_ERR_UNSUPPORTED, "sdm_step_static: B*H*W=%zu exceeds the %zu-byte scratch (at most 65536)",
                    n / 2, kStepScratchBytes);
    void* base = nullptr;
    if ((s = step_scratch(&base)) != SDM_OK)
        return s;
    int32_t* idx = static_cast<int32_t*>(base);
    float* wt = reinterpret_cast<float*>(static_cast<char*>(base) + align_up(n * sizeof(int32_t)));
    hipError_t e = sdm::launch_sdm_step(wq, rq, v, alpha, beta, subkeys, mem_inout, out, idx, wt, c.B, c.H, c.d,
                                        mem_stride_of(c), c.n_sub, c.dk / 2, c.k, c.W, c.in_dtype == SDM_BF16,
                                        c.state_dtype == SDM_BF16, (hipStream_t)hip_stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sdm_step_static launch");
}

sdm_status sdm_forward_train(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                             const float* beta, const void* subkeys, void* mem_inout, float* out, void* log)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !v || !alpha || !beta || !subkeys || !mem_inout || !out || !log)
        return fail(SDM_ERR_INVALID_ARG, "sdm_forward_train: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(v) || !aligned16(subkeys) || !aligned16(mem_inout) ||
        !aligned16(out) || !aligned16(log) || !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_forward_train: misaligned pointer");
    const sdm_config& c = h->cfg;
    if ((s = check_train_shape(c, "sdm_forward_train")) != SDM_OK)
        return s;
    return forward_impl(h, wq, rq, v, alpha, beta, subkeys, mem_inout, out, log);
}

sdm_status sdm_backward_workspace_bytes(const sdm_config* cfg, size_t* bytes)
{
    std::vector<sdm::ScanPlan> plans;
    sdm_status s = check_config(cfg, &plans);
    if (s != SDM_OK)
        return s;
    if (!bytes)
        return fail(SDM_ERR_INVALID_ARG, "bytes is NULL");
    if ((s = check_train_shape(*cfg, "sdm_backward_workspace_bytes")) != SDM_OK)
        return s;
    const sdm_config& c = *cfg;
    const size_t rows = (size_t)c.B * c.T * c.H;
    const int nsplit = sdm::grad_sub_splits(c.B, c.H, c.T, c.n_sub, c.dk / 2);
    *bytes = align_up(sdm::grad_part_floats(c.B, c.H, c.T, c.d, c.W, c.state_dtype == SDM_BF16) * 4) +
             align_up(2 * rows * 2 * c.n_sub * 4) +
             align_up((size_t)nsplit * c.H * 2 * c.n_sub * (c.dk / 2) * 4) + align_up(rows * 4) +
             align_up(sdm::kGradSinkBytes);
    return SDM_OK;
}

sdm_status sdm_backward(sdm_handle h, const void* wq, const void* rq, const void* v, const float* alpha,
                        const float* beta, const void* subkeys, void* mem_inout, const void* log, const float* dout,
                        float* dmem_inout, float* dwq, float* drq, float* dv, float* dalpha, float* dbeta,
                        float* dsubkeys)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!wq || !rq || !v || !alpha || !beta || !subkeys || !mem_inout || !log || !dout || !dmem_inout || !dwq ||
        !drq || !dv || !dalpha || !dbeta || !dsubkeys)
        return fail(SDM_ERR_INVALID_ARG, "sdm_backward: NULL pointer");
    if (!aligned16(wq) || !aligned16(rq) || !aligned16(v) || !aligned16(subkeys) || !aligned16(mem_inout) ||
        !aligned16(log) || !aligned16(dout) || !aligned16(dmem_inout) || !aligned16(dv) || !aligned4(dwq) ||
        !aligned4(drq) || !aligned4(alpha) || !aligned4(beta) || !aligned4(dalpha) || !aligned4(dbeta) ||
        !aligned4(dsubkeys))
        return fail(SDM_ERR_INVALID_ARG, "sdm_backward: misaligned pointer");
    const sdm_config& c = h->cfg;
    if ((s = check_train_shape(c, "sdm_backward")) != SDM_OK)
        return s;
    const size_t rows = (size_t)c.B * c.T * c.H;
    if (!h->bwd_block) {
        size_t bytes = 0;
        if ((s = sdm_backward_workspace_bytes(&c, &bytes)) != SDM_OK)
            return s;
        hipError_t e = hipMalloc(&h->bwd_block, bytes);
        if (e != hipSuccess) {
            h->bwd_block = nullptr;
            (void)hipGetLastError();
            return fail(SDM_ERR_OOM, "backward workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
        }
        char* p = (char*)h->bwd_block;
        h->part = (float*)p;
        p += align_up(sdm::grad_part_floats(c.B, c.H, c.T, c.d, c.W, c.state_dtype == SDM_BF16) * 4);
        h->ds = (float*)p;
        p += align_up(2 * rows * 2 * c.n_sub * 4);
        h->sub_part = (float*)p;
        h->nsplit = sdm::grad_sub_splits(c.B, c.H, c.T, c.n_sub, c.dk / 2);
        p += align_up((size_t)h->nsplit * c.H * 2 * c.n_sub * (c.dk / 2) * 4);
        h->conflict = (int32_t*)p;
        p += align_up(rows * 4);
        h->sink = (float*)p;
    }
    // the forward's slots and weights, recomputed by the same kernels
    if ((s = run_address_all(h, wq, rq, subkeys, h->stream)) != SDM_OK)
        return s;
    sdm::GradArgs a;
    a.B = c.B;
    a.H = c.H;
    a.T = c.T;
    a.d = c.d;
    a.ms = mem_stride_of(c);
    a.S = c.n_sub;
    a.dh = c.dk / 2;
    a.W = c.W;
    a.in_bf16 = c.in_dtype == SDM_BF16;
    a.state_bf16 = c.state_dtype == SDM_BF16;
    a.ncol = c.d * (a.state_bf16 ? 2 : 4) / 128;
    a.mem = mem_inout;
    a.G = dmem_inout;
    a.log = log;
    for (int set = 0; set < 2; ++set) {
        a.idx[set] = h->idx[set];
        a.wt[set] = h->wt[set];
    }
    a.q[0] = wq;
    a.q[1] = rq;
    a.v = v;
    a.alpha = alpha;
    a.beta = beta;
    a.subkeys = subkeys;
    a.dout = dout;
    a.dv = dv;
    a.dalpha = dalpha;
    a.dbeta = dbeta;
    a.dq[0] = dwq;
    a.dq[1] = drq;
    a.dsub = dsubkeys;
    a.part = h->part;
    a.ds = h->ds;
    a.sub_part = h->sub_part;
    a.conflict = h->conflict;
    a.sink = h->sink;
    a.nsplit = h->nsplit;
    hipError_t e;
    {
        Timer t(h, K_BWD_ROWS, h->stream);
        e = sdm::launch_grad_conflicts(a, h->stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "conflict flags launch");
    {
        Timer t(h, K_BWD_SCAN, h->stream);
        e = sdm::launch_grad_scan(a, h->stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "backward scan launch");
    {
        Timer t(h, K_BWD_ROWS, h->stream);
        e = sdm::launch_grad_rows(a, h->stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "backward rows launch");
    {
        Timer t(h, K_BWD_SUB, h->stream);
        e = sdm::launch_grad_subkeys(a, h->stream);
    }
    return e == hipSuccess ? SDM_OK : hip_fail(e, "sub-key gradient launch");
}

sdm_status sdm_project(sdm_handle h, int D, const void* x, const void* w, const float* gate_bias, void* wq, void* rq,
                       void* v, float* alpha, float* beta)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!x || !w || !gate_bias || !wq || !rq || !v || !alpha || !beta)
        return fail(SDM_ERR_INVALID_ARG, "sdm_project: NULL pointer");
    if (!aligned16(x) || !aligned16(w) || !aligned4(gate_bias) || !aligned4(wq) || !aligned4(rq) || !aligned4(v) ||
        !aligned4(alpha) || !aligned4(beta))
        return fail(SDM_ERR_INVALID_ARG, "sdm_project: misaligned pointer");
    const sdm_config& c = h->cfg;
    if (c.in_dtype != SDM_BF16)
        return fail(SDM_ERR_UNSUPPORTED, "sdm_project: built for bf16 embeddings and weights");
    if (D < 8 || D % 8 || D > (1 << 20))
        return fail(SDM_ERR_UNSUPPORTED, "sdm_project: D=%d must be a multiple of 8 in [8, 2^20]", D);
    Timer t(h, K_PROJ, h->stream);
    hipError_t e = sdm::launch_project(x, w, gate_bias, wq, rq, v, alpha, beta, c.B * c.T, D, c.H, c.dk, c.d,
                                       h->stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "projection launch");
}

sdm_status sdm_broadcast_memory(sdm_handle h, const void* m0, void* mem_out)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!m0 || !mem_out)
        return fail(SDM_ERR_INVALID_ARG, "sdm_broadcast_memory: NULL pointer");
    if (!aligned16(m0) || !aligned16(mem_out))
        return fail(SDM_ERR_INVALID_ARG, "sdm_broadcast_memory: misaligned pointer");
    const sdm_config& c = h->cfg;
    // rows of mem_stride elements in both (the padding is copied along)
    const size_t bytes = (size_t)c.H * c.n_sub * c.n_sub * mem_stride_of(c) * (c.state_dtype == SDM_BF16 ? 2 : 4);
    hipError_t e = sdm::launch_broadcast(m0, mem_out, bytes, c.B, h->stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "broadcast launch");
}

sdm_status sdm_overlap(sdm_handle h, const int32_t* idx_w, const float* wt_w, const int32_t* idx_r, const float* wt_r,
                       int buckets, float* write_cum, float* read, int n_queries, const int32_t* queries,
                       float* overlap)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!idx_w || !wt_w || !idx_r || !wt_r || !write_cum || !read || (n_queries > 0 && (!queries || !overlap)))
        return fail(SDM_ERR_INVALID_ARG, "sdm_overlap: NULL pointer");
    if (!aligned4(idx_w) || !aligned4(wt_w) || !aligned4(idx_r) || !aligned4(wt_r) || !aligned4(write_cum) ||
        !aligned4(read) || (n_queries > 0 && (!aligned4(queries) || !aligned4(overlap))))
        return fail(SDM_ERR_INVALID_ARG, "sdm_overlap: misaligned pointer");
    const sdm_config& c = h->cfg;
    const long N = (long)c.n_sub * c.n_sub;
    if (buckets < 1 || buckets > N || n_queries < 0 || n_queries > (1 << 20))
        return fail(SDM_ERR_INVALID_ARG, "sdm_overlap: buckets=%d must be in [1, N=%ld], n_queries=%d in [0, 2^20]",
                    buckets, N, n_queries);
    hipError_t e = sdm::launch_overlap(idx_w, wt_w, idx_r, wt_r, buckets, write_cum, read, n_queries, queries, overlap,
                                       c.B, c.T, c.H, c.W, N, h->stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "overlap launch");
}

sdm_status sdm_set_timing(sdm_handle h, int enable)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    for (auto& tl : h->pending) {
        (void)hipEventDestroy(tl.start);
        (void)hipEventDestroy(tl.stop);
    }
    h->pending.clear();
    memset(&h->totals, 0, sizeof h->totals);
    h->timing = enable != 0;
    return SDM_OK;
}

sdm_status sdm_get_timing(sdm_handle h, sdm_timing* t)
{
    sdm_status s = check_handle(h);
    if (s != SDM_OK)
        return s;
    if (!t)
        return fail(SDM_ERR_INVALID_ARG, "sdm_get_timing: NULL pointer");
    sdm_status rc = SDM_OK;
    for (auto& tl : h->pending) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(tl.stop);
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, tl.start, tl.stop);
        if (e != hipSuccess && rc == SDM_OK)
            rc = hip_fail(e, "timing event");
        switch (tl.kind) {
        case K_SCORE: h->totals.ms_score += ms; h->totals.n_score++; break;
        case K_SELECT: h->totals.ms_select += ms; h->totals.n_select++; break;
        case K_PLAN: h->totals.ms_plan += ms; h->totals.n_plan++; break;
        case K_SCAN: h->totals.ms_scan += ms; h->totals.n_scan++; break;
        case K_STEP: h->totals.ms_step += ms; h->totals.n_step++; break;
        case K_TRAIN: h->totals.ms_train += ms; h->totals.n_train++; break;
        case K_BWD_SCAN: h->totals.ms_bwd_scan += ms; h->totals.n_bwd_scan++; break;
        case K_BWD_ROWS: h->totals.ms_bwd_rows += ms; h->totals.n_bwd_rows++; break;
        case K_BWD_SUB: h->totals.ms_bwd_sub += ms; h->totals.n_bwd_sub++; break;
        case K_PROJ: h->totals.ms_project += ms; h->totals.n_project++; break;
        }
        (void)hipEventDestroy(tl.start);
        (void)hipEventDestroy(tl.stop);
    }
    h->pending.clear();
    *t = h->totals;
    return rc;
}

sdm_status sdm_pattern_probe_mix(void* mem, int memories, long rows, int row_bytes, long row_stride, int T, int W,
                                 int reads, int writes, unsigned seed, void* hip_stream)
{
    if (!mem || ((uintptr_t)mem & 15u))
        return fail(SDM_ERR_INVALID_ARG, "sdm_pattern_probe: mem is NULL or not 16-byte aligned");
    if (memories < 1 || rows < 1 || T < 1 || W < 1 || W > 64)
        return fail(SDM_ERR_INVALID_ARG, "sdm_pattern_probe: memories=%d rows=%ld T=%d W=%d", memories, rows, T, W);
    if (row_stride == 0)
        row_stride = row_bytes;
    if (row_bytes < 128 || row_bytes % 128 != 0 || row_stride < row_bytes || row_stride % 16 != 0 ||
        (unsigned long long)rows * (unsigned long long)row_stride >= (1ull << 32) - 16)
        return fail(SDM_ERR_INVALID_ARG, "sdm_pattern_probe: row_bytes=%d must be a multiple of 128, row_stride=%ld "
                    "at least row_bytes and a multiple of 16, and one memory below 4 GiB", row_bytes, row_stride);
    if (!((reads == 2 && writes == 1) || (reads == 4 && writes == 3)))
        return fail(SDM_ERR_INVALID_ARG, "sdm_pattern_probe: reads:writes %d:%d; built for 2:1 and 4:3", reads, writes);
    hipError_t e = sdm::launch_hbm_pattern(mem, memories, rows, row_bytes, row_stride, T, W, reads, writes, seed,
                                           (hipStream_t)hip_stream);
    return e == hipSuccess ? SDM_OK : hip_fail(e, "hbm_pattern launch");
}

sdm_status sdm_pattern_probe(void* mem, int memories, long rows, int row_bytes, int T, int W, unsigned seed,
                             void* hip_stream)
{
    return sdm_pattern_probe_mix(mem, memories, rows, row_bytes, 0, T, W, 2, 1, seed, hip_stream);
}

} // extern "C"

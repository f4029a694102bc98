// sk_api.hip -- host side of the C ABI declared in include/sk.h: argument
// validation, workspace carve-up and the launch sequence of each entry point.
// All work is enqueued on the caller's stream; nothing here synchronises
// except sk_check_inputs and the convergence checks of sk_solve_ex.
#include "sk.h"
#include "sk_internal.hpp"

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <optional>
#include <tuple>
#include <utility>
#include <vector>

namespace sk {
namespace {

constexpr int kAbiVersion = 2;
#ifndef SK_SMALL_PAIRS
#define SK_SMALL_PAIRS 2.0e6
#endif
// Passes with at most this many (query, key) pairs use the single-kernel
// small-problem path (d <= 8).
constexpr double kSmallPairs = SK_SMALL_PAIRS;
constexpr int64_t kTargetGroups = 2048;  // workgroups per pass: 8 per CU on 256 CUs
// Stop-rule checks are read one interval late below this many pairs per pass (about 2048 x 2048,
// where an iteration takes ~10 us and a check's host round trip ~25 us).
constexpr double kDeferPairs = 4.2e6;
constexpr int64_t kMinColsPerSplit = 512;
constexpr int kMfmaGradSplitRows = 64;  // rows per block that bound the matrix-core gradient's key splits

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Split {
    int nsplit;
    int cols;
};

Split split_for(int64_t nq, int64_t nk, int rows_per_block) {
    int64_t row_blocks = (nq + rows_per_block - 1) / rows_per_block;
    int64_t sp = (kTargetGroups + row_blocks - 1) / row_blocks;
    sp = std::min<int64_t>(sp, (nk + kMinColsPerSplit - 1) / kMinColsPerSplit);
    sp = std::min<int64_t>(sp, kMaxSplit);
    sp = std::max<int64_t>(sp, 1);
    int64_t cols = (nk + sp - 1) / sp;
    sp = (nk + cols - 1) / cols;
    return Split{(int)sp, (int)cols};
}

// The split of a transport pass: no more key splits than split_for allows (the
// workspace is sized by it), but when the row blocks fit the GPU's resident
// workgroups (cap) at once, only as many splits as keep them all resident, so
// the grid runs as one full wave instead of a full wave and a ragged one.
// The same split with its key columns per split rounded up to a multiple of
// align (never more splits than before, so the workspace still holds them).
Split align_split(Split s, int64_t nk, int align) {
    const int64_t cols = ((int64_t)s.cols + align - 1) / align * align;
    return Split{(int)((nk + cols - 1) / cols), (int)cols};
}

Split split_resident(int64_t nq, int64_t nk, int rows_per_block, int cap) {
    const Split base = split_for(nq, nk, rows_per_block);
    const int64_t row_blocks = (nq + rows_per_block - 1) / rows_per_block;
    if (cap <= 0 || row_blocks >= cap) return base;
    int64_t sp = std::min<int64_t>(base.nsplit, std::max<int64_t>(1, cap / row_blocks));
    const int64_t cols = (nk + sp - 1) / sp;
    sp = (nk + cols - 1) / cols;
    return Split{(int)sp, (int)cols};
}

// Resident workgroups of a transport kernel, per device (cached).
int transport_capacity_cached(const Layout& L, int mode, int kwidth) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int dim = L.mfma ? L.P : L.d;
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_tuple(dev, (L.mfma ? 1000 : 0) + dim, mode, kwidth);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    const int c = L.mfma ? mfma_transport_capacity(dim, mode, kwidth) : transport_capacity(dim, mode, kwidth);
    if (c > 0) cache[key] = c;
    return c;
}

int rows_per_block(int d) {
    return d <= kValuMaxD ? valu_rows_per_block() : mfma_rows_per_block(packed_stride(d));
}

// Key-range split of the gradient pass (a plain split grid: it runs once per solve).
Split grad_split(int64_t n, int64_t m, int d) {
    // d > 8: the bound of the matrix-core gradient's key splits (64-row blocks), which sizes its partials; the
    // kernel runs as few splits as keep its workgroups resident, at most this many
    return split_for(n, m, d <= kValuMaxD ? valu_block_rows() : kMfmaGradSplitRows);
}

// Upper bound on the workgroups of a streamed pass, from the sizes alone (the
// workspace is sized with it): at most kMaxGroups (kMaxGroupsValu for the
// vector-ALU pass, d <= 8), each with >= kMinKeysPerGroup keys.
int64_t groups_bound(int64_t nq, int64_t nk, int rpb, bool valu) {
    const int64_t total = (nq + rpb - 1) / rpb * nk;
    int64_t w = (total + kMinKeysPerGroup - 1) / kMinKeysPerGroup;
    w = std::min<int64_t>(w, valu ? kMaxGroupsValu : kMaxGroups);
    w = std::min<int64_t>(w, ((int64_t)1 << 62) / total);  // keeps w * total in int64
    return std::max<int64_t>(w, 1);
}

// Workgroups of a streamed pass.  The matrix-core pass takes one resident
// round (capacity).  The vector-ALU pass takes a whole number of resident
// rounds: one more for every kRoundKeys (row block, key) units that a single
// round would give each workgroup, at most kValuRounds.  Short problems keep
// one round (more ranges would only add partials and merge work); long ones
// run several rounds of shorter ranges, which the hardware hands out as slots
// free up.  A fractional round would leave a ragged last one.  Measured per
// 100-iteration solve at d = 3 (ms): 30,000^2 33.6 with one round, 33.1 with
// two, 35.6 with 1.3; 50,000^2 88.6 / 86.6 / 85.9 / 86.3 with 1 / 2 / 3 / 4;
// 50,000 x 40,000 71.4 / 70.1 / 69.5 / 70.0; 100,000^2 347.5 against 334.8
// with 4; 10,000^2 at d = 2 (200 iterations) 10.9 against 11.9 with 2.
int pass_groups(int64_t nq, int64_t nk, int rpb, int capacity, bool valu) {
    const int64_t bound = groups_bound(nq, nk, rpb, valu);
    const int64_t cap = std::max(capacity, 1);
    int64_t rounds = 1;
    if (valu) {
        const int64_t total = (nq + rpb - 1) / rpb * nk;
        rounds = std::min<int64_t>(std::max<int64_t>(total / (cap * kRoundKeys), 1), kValuRounds);
    }
    return (int)std::min<int64_t>(bound, rounds * cap);
}

// Workgroups the GPU holds at once for the d-dimensional pass, per device.
int pass_capacity(int d) {
    static std::mutex mu;
    static std::map<std::pair<int, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    auto key = std::make_pair(dev, d);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    const int c = d <= kValuMaxD ? valu_pass_capacity(d) : mfma_pass_capacity(packed_stride(d));
    if (c > 0) cache[key] = c;
    return c;
}

int check_sizes(int64_t n, int64_t m, int32_t d) {
    if (n < 1 || m < 1 || d < 1 || n > INT32_MAX || m > INT32_MAX) return SK_ERR_SHAPE;
    if (d > kMaxD) return SK_ERR_UNSUPPORTED_D;
    return SK_OK;
}

int check_eps(float eps) {
    if (!std::isfinite(eps) || eps <= 0.0f) return SK_ERR_EPS;
    // the pre-scaled query 2 log2e / eps must stay finite in fp32
    if (!(2.0 * (double)kLog2e / (double)eps < (double)FLT_MAX)) return SK_ERR_EPS;
    return SK_OK;
}

struct Ws {
    Layout L;
    char* base;
    float* f(size_t off) const { return reinterpret_cast<float*>(base + off); }
    uint16_t* h(size_t off) const { return reinterpret_cast<uint16_t*>(base + off); }
    double* dbl(size_t off) const { return reinterpret_cast<double*>(base + off); }
};

int check_ws(void* ws, size_t ws_bytes, const Layout& L) {
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < L.total)
        return SK_ERR_WORKSPACE;
    return SK_OK;
}

#define SK_TRY(expr)                              \
    do {                                          \
        if ((expr) != hipSuccess) return SK_ERR_HIP; \
    } while (0)

// The scale of both clouds' fp16 split parts: fl(sqrt(2 log2e / eps)), from
// the same float 2 log2e / eps every pass takes, so that the split kernel and
// the passes agree on every bit.
float split_root(float eps) { return (float)std::sqrt((double)(2.0f * kLog2e / eps)); }

// Shifts both clouds by their common centre and packs them.  x_bias / y_bias:
// 0 = none, 1 = zero potential, 2 = from the given potential.
// u_x / u_y (may be null) receive the states that the initial biases encode.
int prepare(const Ws& W, const float* x, const float* y, const float* a, const float* b, float eps,
            int x_bias, const float* f, int y_bias, const float* g, hipStream_t s, float* u_x = nullptr,
            float* u_y = nullptr) {
    const Layout& L = W.L;
    float* centre = W.f(L.centre);
    SK_TRY(launch_centre(x, y, (int)L.n, (int)L.m, L.d, W.dbl(L.cen), centre, s));
    SK_TRY(launch_pack(x, (int)L.n, L.d, L.P, L.mfma, centre, a, W.f(L.xp), W.f(L.nx), W.f(L.l2a), W.f(L.hx),
                       1.0f / eps, x_bias, f, u_x, s));
    SK_TRY(launch_pack(y, (int)L.m, L.d, L.P, L.mfma, centre, b, W.f(L.yp), W.f(L.ny), W.f(L.l2b), W.f(L.hy),
                       1.0f / eps, y_bias, g, u_y, s));
    if (L.split) {  // scales and keys of the fp16 matrix-core pass
        SK_TRY(launch_absmax(W.f(L.xp), L.n * L.P, W.f(L.yp), L.m * L.P, W.f(L.amax_part), W.f(L.amax), s));
        const float rq = split_root(eps);
        SK_TRY(launch_split2(W.f(L.xp), L.n, L.P, W.f(L.amax), rq, W.h(L.xb), s));
        SK_TRY(launch_split2(W.f(L.yp), L.m, L.P, W.f(L.amax) + 1, rq, W.h(L.yb), s));
    }
    return SK_OK;
}

// A streamed pass with queries from one side and keys from the other.
// row_side = true: queries x (n), keys y (m); otherwise the transpose.
PassArgs make_pass(const Ws& W, bool row_side, float eps, const float* w_q, int capacity) {
    const Layout& L = W.L;
    PassArgs p{};
    const int64_t nq = row_side ? L.n : L.m, nk = row_side ? L.m : L.n;
    p.rpb = rows_per_block(L.d);
    p.total = (nq + p.rpb - 1) / p.rpb * nk;
    p.W = pass_groups(nq, nk, p.rpb, capacity, !L.mfma);
    p.q = W.f(row_side ? L.xp : L.yp);
    p.k = W.f(row_side ? L.yp : L.xp);
    p.kbias = L.mfma ? W.f(row_side ? L.hy : L.hx) : nullptr;
    p.kb = L.split ? W.h(row_side ? L.yb : L.xb) : nullptr;
    p.qb = L.split ? W.h(row_side ? L.xb : L.yb) : nullptr;
    p.rq = split_root(eps);
    p.qmax = L.split ? W.f(L.amax) + (row_side ? 0 : 1) : nullptr;
    p.kmax = L.split ? W.f(L.amax) + (row_side ? 1 : 0) : nullptr;
    p.nq = (int)nq;
    p.nk = (int)nk;
    p.P = L.P;
    p.qscale = 2.0f * kLog2e / eps;
    p.part = reinterpret_cast<float2*>(W.base + L.part);
    p.small = (!L.mfma && (double)nq * (double)nk <= kSmallPairs) ? 1 : 0;
    Fin& F = p.fin;
    F.mode = kFinSolve;
    F.P = L.P;
    F.d = L.d;
    F.eps_ln2 = eps * kLn2;
    F.inv_eps = 1.0f / eps;
    F.alpha = 1.0f;
    F.lse = W.f(row_side ? L.lse_r : L.lse_c);
    F.lse_out = F.lse;
    F.l2w = W.f(row_side ? L.l2a : L.l2b);
    F.w = w_q;
    F.nrm = W.f(row_side ? L.nx : L.ny);
    F.pot = nullptr;
    F.bias_packed = L.mfma ? nullptr : W.f(row_side ? L.xp : L.yp);
    F.bias_sep = L.mfma ? W.f(row_side ? L.hx : L.hy) : nullptr;
    F.rbuf = nullptr;
    F.pot_in = nullptr;
    return p;
}

// Points a pass at other query / key arrays (same packed layout) and resizes
// its stream-K decomposition; nq <= n and nk <= m of the layout keep the
// partials within the workspace.
void retarget(PassArgs& p, const float* q, int64_t nq, const float* k, int64_t nk, int capacity) {
    p.q = q;
    p.k = k;
    p.kb = p.qb = nullptr;  // no split copy of other keys
    p.qmax = p.kmax = nullptr;
    p.nq = (int)nq;
    p.nk = (int)nk;
    p.total = (nq + p.rpb - 1) / p.rpb * nk;
    p.W = pass_groups(nq, nk, p.rpb, capacity, !p.kbias);
    p.small = (!(p.kbias) && (double)nq * (double)nk <= kSmallPairs) ? 1 : 0;
}

// Optional event timing of the pass kernels (sk_timing_enable / sk_timing_read).
struct Timing {
    std::mutex mu;
    bool on = false;
    int stride = 1;                // time every stride-th pass launch
    int64_t seen = 0;              // pass launches since enable
    std::vector<hipEvent_t> pool;  // pairs: [2k] start, [2k + 1] stop
    size_t used = 0;               // pairs recorded since enable
    double pairs = 0.0;
    int paused = 0;                // > 0: launches are not timed (TimingPause)
};
Timing& timing() {
    static Timing t;
    return t;
}

// Takes the event pair for the next streamed-pass launch of `pairs` point
// pairs when timing is on, the stream is not being captured and the stride
// selects it; otherwise leaves both null.
int timing_events_pairs(double pairs, hipStream_t s, hipEvent_t* e0, hipEvent_t* e1) {
    Timing& T = timing();
    *e0 = *e1 = nullptr;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return SK_ERR_HIP;
    std::lock_guard<std::mutex> lk(T.mu);
    // no event nodes inside a captured graph
    if (T.on && T.paused == 0 && cap == hipStreamCaptureStatusNone && (T.seen++ % T.stride) == 0) {
        while (T.pool.size() < 2 * (T.used + 1)) {
            hipEvent_t e;
            SK_TRY(hipEventCreate(&e));
            T.pool.push_back(e);
        }
        *e0 = T.pool[2 * T.used];
        *e1 = T.pool[2 * T.used + 1];
        ++T.used;
        T.pairs += pairs;
    }
    return SK_OK;
}

int timing_events(int64_t nq, int64_t nk, hipStream_t s, hipEvent_t* e0, hipEvent_t* e1) {
    return timing_events_pairs((double)nq * (double)nk, s, e0, e1);
}

bool timing_on() {
    Timing& T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    return T.on;
}

// Leaves the pass launches made during its lifetime untimed (auxiliary passes
// that would blur the average of the kernel being measured).
struct TimingPause {
    TimingPause() {
        std::lock_guard<std::mutex> lk(timing().mu);
        ++timing().paused;
    }
    ~TimingPause() {
        std::lock_guard<std::mutex> lk(timing().mu);
        --timing().paused;
    }
    TimingPause(const TimingPause&) = delete;
    TimingPause& operator=(const TimingPause&) = delete;
};

int run_pass(const Ws& W, const PassArgs& p, hipStream_t s) {
    hipEvent_t e0, e1;
    int st = timing_events(p.nq, p.nk, s, &e0, &e1);
    if (st) return st;
    if (W.L.mfma)
        SK_TRY(launch_pass_mfma(p, s, e0, e1));
    else
        SK_TRY(launch_pass_valu(p, W.L.d, s, e0, e1));
    return SK_OK;
}

}  // namespace

Layout make_layout(int64_t n, int64_t m, int d) {
    Layout L{};
    L.d = d;
    L.P = packed_stride(d);
    L.mfma = d > kValuMaxD;
    L.n = n;
    L.m = m;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return o;
    };
    const size_t P = (size_t)L.P, un = (size_t)n, um = (size_t)m, umx = (size_t)std::max(n, m);
    L.xp = take(un * P * 4);
    L.yp = take(um * P * 4);
    L.hx = take(un * 4);
    L.hy = take(um * 4);
    L.nx = take(un * 4);
    L.ny = take(um * 4);
    L.l2a = take(un * 4);
    L.l2b = take(um * 4);
    L.lse_r = take(un * 4);
    L.lse_c = take(um * 4);
    L.rbuf = take(umx * 4);
    const int rpb = rows_per_block(d);
    const Split sr = grad_split(n, m, d);
    const bool valu = d <= kValuMaxD;
    const size_t stream_k = (size_t)std::max(groups_bound(n, m, rpb, valu), groups_bound(m, n, rpb, valu)) * 2 * rpb;
    const size_t part_rows = std::max((size_t)sr.nsplit * un, stream_k);
    L.part = take(part_rows * sizeof(float2));
    L.partA = take(sr.nsplit > 1 ? (size_t)sr.nsplit * un * P * 4 : 0);
    L.red = take((size_t)4 * kRedBlocks * 3 * sizeof(double));
    L.cen = take((size_t)2 * kRedBlocks * d * sizeof(double));
    L.centre = take((size_t)d * 4);
    L.chk = take(8 * sizeof(double));
    L.lse_r2 = take(un * 4);
    L.lse_c2 = take(um * 4);
    L.snap_f = take(un * 4);
    L.snap_g = take(um * 4);
    L.split = L.mfma;
    L.xb = take(L.split ? un * 2 * P * 2 : 0);
    L.yb = take(L.split ? um * 2 * P * 2 : 0);
    L.amax = take(L.split ? 2 * sizeof(float) : 0);
    L.amax_part = take(L.split ? 2 * kAbsMaxBlocks * sizeof(float) : 0);
    L.kt = take(L.mfma ? (umx + kTransColAlign - 1) / kTransColAlign * kTransColAlign * 2 * P * 2 : 0);
    L.pmax = take(L.mfma ? 64 * sizeof(float) : 0);
    L.total = off;
    return L;
}

int plan_split(int64_t nq, int64_t nk, int rpb) { return split_for(nq, nk, rpb).nsplit; }

namespace {

// Options of sk_solve_ex (validated by the caller).
struct ExOpts {
    int variant;     // 0 alternating, 1 symmetric
    float alpha;     // blend of the symmetric variant
    int stop_mode;   // 0 fixed, 1 marginal, 2 potential
    float tol;
    int max_iter;
    int check_every;
};

struct ExResult {
    int iters;
    int converged;   // -1 under the fixed rule
    float viol;      // NaN when no check ran
};

// Check values travel through pinned, mapped host memory: the reduction kernel
// stores them there directly, then raises a sequence flag behind a
// system-scope fence, and the host polls the flag instead of synchronising
// the stream (a stream synchronisation costs far more than a small pass).
// The poll also asks the stream whether it is idle, so it ends even if the
// flag never comes (a failed launch).  Slots of 16 words are taken from a pool
// that grows on demand (one slot per call in flight) and is kept for the life
// of the process.
constexpr int kSlotWords = 16;
constexpr int kFlagWord = kSlotWords - 1;

struct HostSlots {
    std::mutex mu;
    std::vector<float*> free;
};
HostSlots& host_slots() {
    static HostSlots h;
    return h;
}

class HostSlot {
  public:
    int acquire() {
        HostSlots& H = host_slots();
        std::lock_guard<std::mutex> lk(H.mu);
        if (!H.free.empty()) {
            host_ = H.free.back();
            H.free.pop_back();
        } else if (hipHostMalloc(reinterpret_cast<void**>(&host_), kSlotWords * sizeof(float),
                                 hipHostMallocMapped | hipHostMallocPortable | hipHostMallocCoherent) != hipSuccess) {
            host_ = nullptr;
            return SK_ERR_HIP;
        }
        if (hipHostGetDevicePointer(reinterpret_cast<void**>(&dev_), host_, 0) != hipSuccess) return SK_ERR_HIP;
        seq_ = reinterpret_cast<volatile int*>(host_)[kFlagWord];
        return SK_OK;
    }
    ~HostSlot() {
        if (!host_) return;
        HostSlots& H = host_slots();
        std::lock_guard<std::mutex> lk(H.mu);
        H.free.push_back(host_);
    }
    float* dev() const { return dev_; }
    int* flag() const { return reinterpret_cast<int*>(dev_ + kFlagWord); }
    // the sequence number the next check's kernel raises
    int next() { return ++seq_; }
    // waits until the check numbered seq_ has been published, then reads it
    int read(float* out, int n, hipStream_t s) const {
        volatile int* f = reinterpret_cast<volatile int*>(host_) + kFlagWord;
        for (;;) {
            bool seen = false;
            for (int k = 0; k < 4096 && !seen; ++k) seen = *f == seq_;
            if (seen) break;
            const hipError_t q = hipStreamQuery(s);
            if (q == hipSuccess) {
                if (*f != seq_) return SK_ERR_HIP;  // stream idle without the flag
                break;
            }
            if (q != hipErrorNotReady) return SK_ERR_HIP;
        }
        std::atomic_thread_fence(std::memory_order_acquire);
        for (int k = 0; k < n; ++k) out[k] = reinterpret_cast<volatile float*>(host_)[k];
        return SK_OK;
    }

  private:
    float* host_ = nullptr;
    float* dev_ = nullptr;
    int seq_ = 0;
};

// The larger of two check values, NaN if either is NaN (a NaN check is never met).
float max_nan(float a, float b) { return (std::isnan(a) || std::isnan(b)) ? NAN : std::max(a, b); }

// Sinkhorn with an update variant and a stop rule (SinkSLOT README, API
// Reference).  Iteration k of the alternating variant is a row pass from the
// current g then a column pass from the new f; the symmetric variant runs both
// passes from the state before the iteration, blends each result into its
// side's state and then rewrites both key biases.
//
// Checks come after every check_every-th iteration and after the last.  The
// marginal residual of the state after iteration k falls out of the passes of
// iteration k + 1 (the row pass for the alternating variant, whose column sums
// are exact by construction; both passes for the symmetric one), so a check
// costs no extra pass except after the last iteration, where a probe pass
// (which changes nothing) takes its place.  Passes that produce a residual
// write their new state into the second state buffer, so the state that was
// checked is still at hand when it meets the tolerance: its potentials are
// then rewritten from it and the run ends with iters = k.  The potential rule
// compares the output potentials with a snapshot taken at the previous check.
int solve_ex(const Ws& W, const float* x, const float* y, const float* a, const float* b, float eps,
             const ExOpts& o, float* f, float* g, ExResult* res, hipStream_t s) {
    const Layout& L = W.L;
    res->iters = o.max_iter;
    res->converged = o.stop_mode == 0 ? -1 : 0;
    res->viol = NAN;
    if (o.max_iter == 0) {
        SK_TRY(launch_fill(f, L.n, 0.0f, s));
        SK_TRY(launch_fill(g, L.m, 0.0f, s));
        return SK_OK;
    }
    const int cap = pass_capacity(L.d);
    if (cap <= 0) return SK_ERR_HIP;
    const bool sym = o.variant == 1;
    float* ur[2] = {W.f(L.lse_r), W.f(L.lse_r2)};
    float* uc[2] = {W.f(L.lse_c), W.f(L.lse_c2)};
    int cr = 0, cc = 0;
    int st;
    if ((st = prepare(W, x, y, a, b, eps, sym ? 1 : 0, nullptr, 1, nullptr, s, sym ? ur[0] : nullptr,
                      sym ? uc[0] : nullptr)))
        return st;

    PassArgs row = make_pass(W, true, eps, a, cap);
    row.fin.pot = f;
    PassArgs col = make_pass(W, false, eps, b, cap);
    col.fin.pot = g;
    if (sym) {  // biases are rewritten once both passes have read the old ones
        row.fin.alpha = col.fin.alpha = o.alpha;
        row.fin.bias_packed = row.fin.bias_sep = nullptr;
        col.fin.bias_packed = col.fin.bias_sep = nullptr;
    }
    float* rbuf = W.f(L.rbuf);
    HostSlot slot;
    if (o.stop_mode != 0 && (st = slot.acquire())) return st;
    float* chk = slot.dev();
    float host[2] = {0.0f, 0.0f};
    if (o.stop_mode == 2) {
        SK_TRY(launch_fill(W.f(L.snap_f), L.n, 0.0f, s));
        SK_TRY(launch_fill(W.f(L.snap_g), L.m, 0.0f, s));
    }
    auto is_check = [&](int k) { return o.stop_mode != 0 && k >= 1 && (k % o.check_every == 0 || k == o.max_iter); };
    // the state after iteration k met the tolerance: restore its potentials and stop
    auto stop_at = [&](int k, bool restore_f, bool restore_g) -> int {
        if (restore_f) SK_TRY(launch_pot_from_state(ur[cr], W.f(L.nx), eps * kLn2, f, (int)L.n, s));
        if (restore_g) SK_TRY(launch_pot_from_state(uc[cc], W.f(L.ny), eps * kLn2, g, (int)L.m, s));
        res->iters = k;
        res->converged = 1;
        return SK_OK;
    };

    // Deferred checks on small problems, where a check's host round trip costs as much as several
    // iterations: a check value is read only when the next check is due (or after the loop), so
    // the host keeps the GPU fed meanwhile.  The checked iteration's potentials stay restorable
    // until then -- f's state in the buffer the fused pass did not overwrite and g in snap_g
    // (marginal rule), both potentials in snap_f / snap_g (potential rule) -- and a stop
    // returns exactly what the immediate check returns; only the iterations enqueued past the
    // stopping one run in vain.  The symmetric variant's marginal check stays immediate.
    // (Marginal rule: the column pass of a check iteration writes its state to the other buffer,
    // so g's checked state survives in uc like f's in ur.)
    const bool defer = o.stop_mode != 0 && (double)L.n * (double)L.m <= kDeferPairs && !(o.stop_mode == 1 && sym);
    struct Pending {
        bool on = false;
        int k = 0;   // the checked iteration
        int cr = 0;  // marginal rule: the buffers holding the checked row and column states
        int cc = 0;
    } pend;
    // reads the pending check; *stopped = its iteration met the tolerance (potentials restored)
    auto settle = [&](bool* stopped) -> int {
        *stopped = false;
        if (!pend.on) return SK_OK;
        pend.on = false;
        int rc;
        if ((rc = slot.read(host, 1, s))) return rc;
        res->viol = host[0];
        const bool met = o.stop_mode == 1 ? host[0] <= o.tol : host[0] < o.tol;
        if (!met) return SK_OK;
        if (o.stop_mode == 1) {
            SK_TRY(launch_pot_from_state(ur[pend.cr], W.f(L.nx), eps * kLn2, f, (int)L.n, s));
            SK_TRY(launch_pot_from_state(uc[pend.cc], W.f(L.ny), eps * kLn2, g, (int)L.m, s));
        } else {
            SK_TRY(hipMemcpyAsync(f, W.f(L.snap_f), (size_t)L.n * sizeof(float), hipMemcpyDeviceToDevice, s));
            SK_TRY(hipMemcpyAsync(g, W.f(L.snap_g), (size_t)L.m * sizeof(float), hipMemcpyDeviceToDevice, s));
        }
        res->iters = pend.k;
        res->converged = 1;
        *stopped = true;
        return SK_OK;
    };

    for (int k = 1; k <= o.max_iter; ++k) {
        const bool fused = o.stop_mode == 1 && is_check(k - 1);
        if (defer && fused) {
            // the previous check's buffers are about to be reused: settle it first
            bool stopped;
            if ((st = settle(&stopped))) return st;
            if (stopped) return SK_OK;
        }
        row.fin.lse = ur[cr];
        row.fin.lse_out = fused ? ur[cr ^ 1] : ur[cr];
        row.fin.rbuf = fused ? rbuf : nullptr;
        if ((st = run_pass(W, row, s))) return st;
        if (fused) {
            const bool last = !sym;  // the row value alone is the check
            SK_TRY(launch_max_reduce(rbuf, (int)L.n, chk + 0, s, last ? slot.flag() : nullptr, last ? slot.next() : 0));
        }
        if (fused && !sym) {
            if (defer) {
                pend.on = true;
                pend.k = k - 1;
                pend.cr = cr;
                pend.cc = cc;
            } else {
                if ((st = slot.read(host, 1, s))) return st;
                res->viol = host[0];
                if (host[0] <= o.tol) return stop_at(k - 1, true, false);
            }
            cr ^= 1;
        }
        const bool fused_col = fused && sym;
        const bool keep_col = fused && defer;  // keep g's checked state for a deferred stop
        col.fin.lse = uc[cc];
        col.fin.lse_out = (fused_col || keep_col) ? uc[cc ^ 1] : uc[cc];
        col.fin.rbuf = fused_col ? rbuf : nullptr;
        if ((st = run_pass(W, col, s))) return st;
        if (keep_col) cc ^= 1;
        if (fused_col) {
            SK_TRY(launch_max_reduce(rbuf, (int)L.m, chk + 1, s, slot.flag(), slot.next()));
            if ((st = slot.read(host, 2, s))) return st;
            res->viol = max_nan(host[0], host[1]);
            if (res->viol <= o.tol) return stop_at(k - 1, true, true);
            cr ^= 1;
            cc ^= 1;
        }
        if (sym) {
            BiasSide bx{ur[cr], W.f(L.l2a), L.mfma ? nullptr : W.f(L.xp), L.mfma ? W.f(L.hx) : nullptr, (int)L.n};
            BiasSide by{uc[cc], W.f(L.l2b), L.mfma ? nullptr : W.f(L.yp), L.mfma ? W.f(L.hy) : nullptr, (int)L.m};
            SK_TRY(launch_apply_bias(bx, by, L.P, L.d, s));
        }
        if (o.stop_mode == 2 && is_check(k)) {
            if (defer) {  // the snapshots are about to be replaced: settle the previous check first
                bool stopped;
                if ((st = settle(&stopped))) return st;
                if (stopped) return SK_OK;
            }
            SK_TRY(launch_pot_change(f, W.f(L.snap_f), (int)L.n, g, W.f(L.snap_g), (int)L.m, chk, s, slot.flag(),
                                     slot.next()));
            if (defer) {
                pend.on = true;
                pend.k = k;
            } else {
                if ((st = slot.read(host, 1, s))) return st;
                res->viol = host[0];
                if (host[0] < o.tol) return stop_at(k, false, false);
            }
        }
    }
    if (defer) {
        bool stopped;
        if ((st = settle(&stopped))) return st;
        if (stopped) return SK_OK;
    }
    if (o.stop_mode == 1) {  // the check after the last iteration: probe passes
        PassArgs probe = row;
        probe.fin.mode = kFinProbe;
        probe.fin.lse = ur[cr];
        probe.fin.rbuf = rbuf;
        if ((st = run_pass(W, probe, s))) return st;
        SK_TRY(launch_max_reduce(rbuf, (int)L.n, chk + 0, s, sym ? nullptr : slot.flag(), sym ? 0 : slot.next()));
        int cnt = 1;
        if (sym) {
            probe = col;
            probe.fin.mode = kFinProbe;
            probe.fin.lse = uc[cc];
            probe.fin.rbuf = rbuf;
            if ((st = run_pass(W, probe, s))) return st;
            SK_TRY(launch_max_reduce(rbuf, (int)L.m, chk + 1, s, slot.flag(), slot.next()));
            cnt = 2;
        }
        if ((st = slot.read(host, cnt, s))) return st;
        res->viol = cnt == 2 ? max_nan(host[0], host[1]) : host[0];
        if (res->viol <= o.tol) res->converged = 1;
    }
    return SK_OK;
}

// Fixed-count alternating solve with the optional fused residual trace (sk_solve).
// g_init (may be null, may alias g): the starting g of the iteration (0 when null).
int solve_fixed(const Ws& W, const float* x, const float* y, const float* a, const float* b, float eps,
                int n_iters, float* f, float* g, int check_every, float* resid_trace, hipStream_t s,
                const float* g_init = nullptr) {
    const Layout& L = W.L;
    const int64_t n = L.n, m = L.m;
    int st;
    if (n_iters == 0) {
        SK_TRY(launch_fill(f, n, 0.0f, s));
        if (g_init == nullptr)
            SK_TRY(launch_fill(g, m, 0.0f, s));
        else if (g_init != g)
            SK_TRY(hipMemcpyAsync(g, g_init, (size_t)m * sizeof(float), hipMemcpyDeviceToDevice, s));
        return SK_OK;
    }
    const int cap = pass_capacity(L.d);
    if (cap <= 0) return SK_ERR_HIP;
    // the key biases of the first row pass encode the starting g; g itself is first written by a column pass
    if ((st = prepare(W, x, y, a, b, eps, 0, nullptr, g_init ? 2 : 1, g_init, s))) return st;

    PassArgs row = make_pass(W, true, eps, a, cap);
    row.fin.pot = f;
    PassArgs col = make_pass(W, false, eps, b, cap);
    col.fin.pot = g;
    float* rbuf = W.f(L.rbuf);

    for (int k = 1; k <= n_iters; ++k) {
        // the row pass of iteration k also yields the residual of iteration k-1's plan
        const bool check_prev = check_every > 0 && k > 1 && (k - 1) % check_every == 0;
        row.fin.rbuf = check_prev ? rbuf : nullptr;
        if ((st = run_pass(W, row, s))) return st;
        if (check_prev) SK_TRY(launch_resid_reduce(rbuf, (int)n, resid_trace + (k - 1) / check_every - 1, nullptr, s));
        if ((st = run_pass(W, col, s))) return st;
    }
    if (check_every > 0 && n_iters % check_every == 0) {
        PassArgs probe = row;
        probe.fin.mode = kFinProbe;
        probe.fin.rbuf = rbuf;
        if ((st = run_pass(W, probe, s))) return st;
        SK_TRY(launch_resid_reduce(rbuf, (int)n, resid_trace + n_iters / check_every - 1, nullptr, s));
    }
    return SK_OK;
}

// Gradient with respect to x at fixed g (sk_grad_x).
int grad_core(const Ws& W, const float* x, const float* y, const float* a, const float* b, float eps,
              const float* g, float* grad, hipStream_t s) {
    const Layout& L = W.L;
    const int64_t n = L.n, m = L.m;
    const int d = L.d;
    int st;
    int cap = 0;
    if (L.mfma && (cap = pass_capacity(d)) <= 0) return SK_ERR_HIP;
    if ((st = prepare(W, x, y, a, b, eps, 0, nullptr, 2, g, s))) return st;

    if (!L.mfma) {
        GradArgs ga{};
        const Split sp = grad_split(n, m, d);
        ga.q = W.f(L.xp);
        ga.k = W.f(L.yp);
        ga.kbias = nullptr;
        ga.nq = (int)n;
        ga.nk = (int)m;
        ga.P = L.P;
        ga.d = d;
        ga.qscale = 2.0f * kLog2e / eps;
        ga.cols_per_split = sp.cols;
        ga.nsplit = sp.nsplit;
        ga.part = reinterpret_cast<float2*>(W.base + L.part);
        ga.partA = W.f(L.partA);
        ga.w = a;
        ga.grad = grad;
        SK_TRY(launch_grad_valu(ga, s));
        return SK_OK;
    }
    // d > 8: first the row lse of the same scores, then the weighted key sums
    // (transport mode 4), with no more key splits than the workspace holds
    PassArgs lse_pass = make_pass(W, true, eps, a, cap);
    lse_pass.fin.mode = kFinStore;
    {
        TimingPause pause;  // the pass timing covers the gradient kernel
        if ((st = run_pass(W, lse_pass, s))) return st;
    }
    const int rpb = mfma_grad_rows_per_block(L.P);
    const int gcap = transport_capacity_cached(L, 4, 16);
    if (gcap <= 0) return SK_ERR_HIP;
    Split sp = split_resident(n, m, rpb, gcap);
    const Split lim = grad_split(n, m, d);  // the workspace holds this many splits' partials
    if (sp.nsplit > lim.nsplit) {
        const int64_t cols = (m + lim.nsplit - 1) / lim.nsplit;
        sp = Split{(int)((m + cols - 1) / cols), (int)cols};
    }
    sp = align_split(sp, m, kTransColAlign);
    TransArgs t{};
    t.q = W.f(L.xp);
    t.k = W.f(L.yp);
    t.kbias = W.f(L.hy);
    t.kb = W.h(L.yb);
    t.qb = W.h(L.xb);
    t.rq = split_root(eps);
    t.qmax = W.f(L.amax);
    t.kmax = W.f(L.amax) + 1;
    t.lse = W.f(L.lse_r);
    t.nq = (int)n;
    t.nk = (int)m;
    t.P = L.P;
    t.d = d;
    t.qscale = 2.0f * kLog2e / eps;
    t.cols_per_split = sp.cols;
    t.nsplit = sp.nsplit;
    t.part = reinterpret_cast<float2*>(W.base + L.part);
    t.partA = W.f(L.partA);
    t.out = grad;
    t.ldo = d;
    t.kout = d;
    t.gw = a;
    t.kt = W.h(L.kt);
    hipEvent_t e0, e1;
    if ((st = timing_events(n, m, s, &e0, &e1))) return st;
    SK_TRY(launch_transport_mfma(t, 4, 16, s, e0, e1));
    return SK_OK;
}

// Dual objective at arbitrary potentials: one row pass for the plan's row sums.
int dual_cost(const Ws& W, const float* x, const float* y, const float* a, const float* b, float eps,
              const float* f, const float* g, double* out, hipStream_t s) {
    const Layout& L = W.L;
    const int cap = pass_capacity(L.d);
    if (cap <= 0) return SK_ERR_HIP;
    int st;
    if ((st = prepare(W, x, y, a, b, eps, 0, nullptr, 2, g, s))) return st;
    PassArgs row = make_pass(W, true, eps, a, cap);
    row.fin.mode = kFinMass;
    row.fin.pot_in = f;
    row.fin.rbuf = W.f(L.rbuf);
    if ((st = run_pass(W, row, s))) return st;
    SK_TRY(launch_cost_mass(a, b, f, g, W.f(L.rbuf), (int)L.n, (int)L.m, eps, out, s));
    return SK_OK;
}

// Workspace of the transport products and the Hessian-vector product: the
// solver layout, then the split partials of the transport passes and the
// vectors of the product (all O((n + m) d)).
struct TLayout {
    Layout L;
    size_t part, partA;
    size_t A, st, U, B, E, diag, rhs, z, zb, res, p, prod, scal, pv;
    size_t total;
};
constexpr int kTransMaxK = 9;  // payload columns per vector-ALU transport pass

// Payload columns per transport pass, and accumulators per row of a split partial.
int trans_chunk(const Layout& L) { return !L.mfma ? kTransMaxK : (L.P >= 64 ? 64 : 16); }
int trans_acc(const Layout& L) { return !L.mfma ? kTransMaxK : std::max(64, L.P); }
// Rows per workgroup: the largest over the kernel's modes (workspace sizing),
// or those of one mode and payload width.
int trans_rows(const Layout& L) { return L.mfma ? mfma_transport_max_rows_per_block(L.P) : transport_rows_per_block(); }

TLayout make_tlayout(int64_t n, int64_t m, int d) {
    TLayout T{};
    T.L = make_layout(n, m, d);
    size_t off = align_up(T.L.total, 256);
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return o;
    };
    const int rpb = trans_rows(T.L);
    const size_t nsr = (size_t)split_for(n, m, rpb).nsplit, nsc = (size_t)split_for(m, n, rpb).nsplit;
    const size_t prow = std::max(nsr > 1 ? nsr * n : 0, nsc > 1 ? nsc * m : 0);
    const size_t un = (size_t)n, um = (size_t)m, N = un + um, ud = (size_t)d;
    T.part = take(prow * sizeof(float2));
    T.partA = take(prow * (size_t)trans_acc(T.L) * 4);
    T.A = take(un * ud * 4);
    T.st = take(un * 4);
    T.U = take(un * (ud + 1) * 4);
    T.B = take(um * (ud + 1) * 4);
    T.E = take(un * ud * 4);
    T.diag = take(N * 4);
    T.rhs = take(N * 4);
    T.z = take(N * 4);
    T.zb = take(N * 4);
    T.res = take(N * 4);
    T.p = take(N * 4);
    T.prod = take(N * 4);
    T.scal = take((4 + 3 * kCgBlocks) * sizeof(double));
    T.pv = take(un * sizeof(double));  // the primal value's per-row terms
    T.total = off;
    return T;
}

// The row log-sum-exp of the scores of one side, for the matrix-core
// transport kernels (their weights 2^{s - lse} are then <= 1).
int store_lse(const Ws& W, bool row_side, float eps, const float* w_q, hipStream_t s) {
    const int cap = pass_capacity(W.L.d);
    if (cap <= 0) return SK_ERR_HIP;
    PassArgs p = make_pass(W, row_side, eps, w_q, cap);
    p.fin.mode = kFinStore;
    return run_pass(W, p, s);
}

// One transport pass over the packed clouds of W (both packed from their
// potentials): row_side = queries x, keys y; otherwise the transpose.  mode 0
// takes kin <= trans_chunk payload columns; modes 1 and 2 write d columns.
int transport_pass(const Ws& W, const TLayout& T, bool row_side, float eps, int mode, const float* pay, int ldp,
                   int kin, const float* rowv, float* out, int ldo, int kout, float* mass, hipStream_t s) {
    const Layout& L = W.L;
    TransArgs t{};
    t.nq = (int)(row_side ? L.n : L.m);
    t.nk = (int)(row_side ? L.m : L.n);
    t.q = W.f(row_side ? L.xp : L.yp);
    t.k = W.f(row_side ? L.yp : L.xp);
    t.kbias = L.mfma ? W.f(row_side ? L.hy : L.hx) : nullptr;
    t.kb = L.split ? W.h(row_side ? L.yb : L.xb) : nullptr;
    t.qb = L.split ? W.h(row_side ? L.xb : L.yb) : nullptr;
    t.rq = split_root(eps);
    t.qmax = L.split ? W.f(L.amax) + (row_side ? 0 : 1) : nullptr;
    t.kmax = L.split ? W.f(L.amax) + (row_side ? 1 : 0) : nullptr;
    t.qbias = L.mfma ? W.f(row_side ? L.hx : L.hy) : nullptr;
    t.lse = L.mfma ? W.f(row_side ? L.lse_r : L.lse_c) : nullptr;
    t.pay = pay;
    t.rowv = rowv;
    t.P = L.P;
    t.d = L.d;
    t.qscale = 2.0f * kLog2e / eps;
    // a single payload column runs on the vector ALUs inside the matrix-core kernel
    const int kmode = (L.mfma && mode == 0 && kin == 1) ? 3 : mode;
    const int kwidth = L.mfma ? (kin <= 16 ? 16 : 64) : (kin <= 1 ? 1 : (kin <= 4 ? 4 : kTransMaxK));
    Split sp = split_resident(t.nq, t.nk,
                              L.mfma ? mfma_transport_rows_per_block(L.P, kmode, kwidth)
                                     : transport_rows_per_block(),
                              transport_capacity_cached(L, kmode, kwidth));
    if (L.mfma) {
        sp = align_split(sp, t.nk, kTransColAlign);
        t.kt = W.h(L.kt);
        t.pmax = W.f(L.pmax);
    }
    t.cols_per_split = sp.cols;
    t.nsplit = sp.nsplit;
    t.part = reinterpret_cast<float2*>(W.base + T.part);
    t.partA = W.f(T.partA);
    t.out = out;
    t.ldo = ldo;
    t.kout = kout;
    t.ldp = ldp;
    t.kin = kin;
    t.mass = mass;
    hipEvent_t e0, e1;
    int st = timing_events(t.nq, t.nk, s, &e0, &e1);
    if (st) return st;
    if (L.mfma) {
        SK_TRY(launch_transport_mfma(t, kmode, kwidth, s, e0, e1));
    } else {
        SK_TRY(launch_transport(t, mode, kwidth, s, e0, e1));
    }
    return SK_OK;
}

// out (rows x k) = P v or P^T v in chunks of payload columns; mass (may be null)
// receives the plan's row (or column) sums with the first chunk.
int transport_cols(const Ws& W, const TLayout& T, bool row_side, float eps, const float* v, int k, float* out,
                   float* mass, hipStream_t s) {
    const int chunk = trans_chunk(W.L);
    int st;
    for (int c0 = 0; c0 < k; c0 += chunk) {
        const int kin = std::min(chunk, k - c0);
        if ((st = transport_pass(W, T, row_side, eps, 0, v + c0, k, kin, nullptr, out + c0, k, kin,
                                 c0 == 0 ? mass : nullptr, s)))
            return st;
    }
    return SK_OK;
}

int check_transport_sizes(int64_t n, int64_t m, int32_t d) { return check_sizes(n, m, d); }

// ---------------------------------------------------------------- two-stage block-sparse solver
// Workspace: the solver layout of the problem in block order, the layout of
// the centroid problem, and the sort, block, lift, sample and tile arrays.
struct FLayout {
    Layout L, Lc;
    int B, nbx, nby, ns, bits;
    size_t coarse;
    size_t box, boxpart, code_in, code_out, idx_in, idx_out, sort_temp, sort_bytes;
    size_t xs, ys, as, bs, permx, permy;
    size_t amass, bmass, xcen, ycen, xlo, xhi, ylo, yhi, fmax, gmax, F, G;
    size_t ky, kx, knrm, kl2w;
    size_t sq, sf, sa, snrm, slse;
    size_t fs, gs;
    size_t srx, sry, rowbest, colbest, rcnt, rptr, ridx, ccnt, cptr, cidx, spart;
    int64_t list_cap;  // entries of each kept-tile list
    int sparse_groups;
    size_t total;
};

constexpr int64_t kMaxTiles = (int64_t)1 << 36;     // block pairs the screening scores
constexpr int64_t kMaxKeptTiles = (int64_t)1 << 28;  // entries of each kept-tile list
constexpr int kSparseGroups = 2048;              // workgroups of a sparse pass (8 per CU on 256 CUs)

int morton_bits_for(int d) { return std::max(1, std::min(10, 30 / d)); }

// false when the sort's scratch size cannot be queried
bool make_flayout(int64_t n, int64_t m, int d, int B, int n_sample, FLayout* out) {
    FLayout F{};
    F.L = make_layout(n, m, d);
    F.B = B;
    F.nbx = (int)((n + B - 1) / B);
    F.nby = (int)((m + B - 1) / B);
    F.Lc = make_layout(F.nbx, F.nby, d);
    F.ns = (int)std::min<int64_t>(n, n_sample);
    F.bits = morton_bits_for(d);
    size_t off = align_up(F.L.total, 256);
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + std::max<size_t>(bytes, 1), 256);
        return o;
    };
    const size_t un = (size_t)n, um = (size_t)m, ud = (size_t)d, umx = (size_t)std::max(n, m);
    const size_t bx = (size_t)F.nbx, by = (size_t)F.nby, bmx = std::max(bx, by), P = (size_t)F.L.P;
    F.coarse = take(F.Lc.total);
    F.box = take(2 * ud * 4);
    F.boxpart = take((size_t)kRedBlocks * 2 * ud * 4);
    F.code_in = take(umx * 4);
    F.code_out = take(umx * 4);
    F.idx_in = take(umx * 4);
    F.idx_out = take(umx * 4);
    F.sort_bytes = sort_temp_bytes((int)umx, F.bits * d);
    if (F.sort_bytes == 0) return false;
    F.sort_temp = take(F.sort_bytes);
    F.xs = take(un * ud * 4);
    F.ys = take(um * ud * 4);
    F.as = take(un * 4);
    F.bs = take(um * 4);
    F.permx = take(un * 4);
    F.permy = take(um * 4);
    F.amass = take(bx * 4);
    F.bmass = take(by * 4);
    F.xcen = take(bx * ud * 4);
    F.ycen = take(by * ud * 4);
    F.xlo = take(bx * ud * 4);
    F.xhi = take(bx * ud * 4);
    F.ylo = take(by * ud * 4);
    F.yhi = take(by * ud * 4);
    F.fmax = take(bx * 4);
    F.gmax = take(by * 4);
    F.F = take(bx * 4);
    F.G = take(by * 4);
    F.ky = take(by * P * 4);
    F.kx = take(bx * P * 4);
    F.knrm = take(bmx * 4);
    F.kl2w = take(bmx * 4);
    F.sq = take((size_t)F.ns * P * 4);
    F.sf = take((size_t)F.ns * 4);
    F.sa = take((size_t)F.ns * 4);
    F.snrm = take((size_t)F.ns * 4);
    F.slse = take((size_t)F.ns * 4);
    F.fs = take(un * 4);
    F.gs = take(um * 4);
    F.list_cap = std::min<int64_t>((int64_t)bx * (int64_t)by, kMaxKeptTiles);
    F.srx = take(bx * (size_t)screen_stride_of(d) * 4);
    F.sry = take(by * (size_t)screen_stride_of(d) * 4);
    F.rowbest = take(bx * 4);
    F.colbest = take(by * 4);
    F.rcnt = take(bx * 4);
    F.rptr = take((bx + 1) * 4);
    F.ridx = take((size_t)F.list_cap * 4);
    F.ccnt = take(by * 4);
    F.cptr = take((by + 1) * 4);
    F.cidx = take((size_t)F.list_cap * 4);
    F.sparse_groups = kSparseGroups;
    F.spart = take((size_t)F.sparse_groups * 2 * B * sizeof(float2));
    F.total = off;
    *out = F;
    return true;
}

struct Fs2Opts {
    int B;
    float tol, delta;
    int coarse_iters, max_rounds;
    float coarse_gain;
    int n_sample, max_iters, check_every, screen_every;
};

struct Fs2Info {
    int rounds = 0, fine_iters = 0, kept = 0, converged = 0;
    float residual = NAN, last_check = NAN;
};

// Morton order of one cloud: codes, stable radix sort of (code, index), gather.
int morton_sort(char* base, const FLayout& F, const float* p, const float* w, int npts, int d, float* ps, float* ws,
                int* perm, hipStream_t s) {
    uint32_t *cin = reinterpret_cast<uint32_t*>(base + F.code_in), *cout = reinterpret_cast<uint32_t*>(base + F.code_out);
    uint32_t *iin = reinterpret_cast<uint32_t*>(base + F.idx_in), *iout = reinterpret_cast<uint32_t*>(base + F.idx_out);
    SK_TRY(launch_morton(p, npts, d, F.bits, reinterpret_cast<float*>(base + F.box), cin, iin, s));
    SK_TRY(launch_sort_pairs(base + F.sort_temp, F.sort_bytes, cin, cout, iin, iout, npts, F.bits * d, s));
    SK_TRY(launch_gather_points(p, w, iout, npts, d, ps, ws, perm, s));
    return SK_OK;
}

int fs2_solve(char* base, const FLayout& F, const float* x, const float* y, const float* a, const float* b, float eps,
              const Fs2Opts& o, float* f_out, float* g_out, int* perm_x, int* perm_y, Fs2Info* info, hipStream_t s) {
    const Layout& L = F.L;
    const int n = (int)L.n, m = (int)L.m, d = L.d;
    Ws W{L, base};
    Ws Wc{F.Lc, base + F.coarse};
    auto fp = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
    auto ip = [&](size_t off) { return reinterpret_cast<int*>(base + off); };
    float *xs = fp(F.xs), *ys = fp(F.ys), *as = fp(F.as), *bs = fp(F.bs);
    float *fs = fp(F.fs), *gs = fp(F.gs), *Fc = fp(F.F), *Gc = fp(F.G);
    int st;
    const int cap = pass_capacity(d);
    if (cap <= 0) return SK_ERR_HIP;
    HostSlot slot;
    if ((st = slot.acquire())) return st;
    float host[2];

    // 1-2: Morton order and blocks
    SK_TRY(launch_bbox(x, n, y, m, d, fp(F.boxpart), fp(F.box), s));
    if ((st = morton_sort(base, F, x, a, n, d, xs, as, ip(F.permx), s))) return st;
    if ((st = morton_sort(base, F, y, b, m, d, ys, bs, ip(F.permy), s))) return st;
    if ((st = prepare(W, xs, ys, as, bs, eps, 0, nullptr, 1, nullptr, s))) return st;
    SK_TRY(launch_block_stats(xs, as, n, d, F.B, fp(F.amass), fp(F.xcen), fp(F.xlo), fp(F.xhi), s));
    SK_TRY(launch_block_stats(ys, bs, m, d, F.B, fp(F.bmass), fp(F.ycen), fp(F.ylo), fp(F.yhi), s));

    // 3: coarse stage on the centroids, lifted to the points after every round
    // (untimed: the pass timing covers the block-sparse passes of the fine stage).
    // The check of a round needs the lifted g at every point but the lifted f
    // only at its sampled rows, so a round lifts f at those rows alone and f
    // is lifted at every point once, from the accepted round.
    std::optional<TimingPause> pause;
    pause.emplace();
    PassArgs lift_f = make_pass(W, true, eps, as, cap);
    lift_f.fin.pot = fs;
    retarget(lift_f, W.f(L.xp), n, fp(F.ky), F.nby, cap);
    const int stride = n / F.ns;
    // the sampled rows: coordinates, weights and norms (the potential gathered with them, from fs, is not
    // yet set and is overwritten by every round's lift before the check reads it)
    SK_TRY(launch_gather_rows(W.f(L.xp), L.P, fs, as, W.f(L.nx), F.ns, stride, fp(F.sq), fp(F.sf), fp(F.sa),
                              fp(F.snrm), s));
    PassArgs lift_fs = make_pass(W, true, eps, fp(F.sa), cap);
    retarget(lift_fs, fp(F.sq), F.ns, fp(F.ky), F.nby, cap);
    lift_fs.fin.lse = lift_fs.fin.lse_out = fp(F.slse);
    lift_fs.fin.l2w = nullptr;  // no bias is written for the sampled rows
    lift_fs.fin.nrm = fp(F.snrm);
    lift_fs.fin.pot = fp(F.sf);
    lift_fs.fin.bias_packed = nullptr;
    lift_fs.fin.bias_sep = nullptr;
    PassArgs lift_g = make_pass(W, false, eps, bs, cap);
    lift_g.fin.pot = gs;
    retarget(lift_g, W.f(L.yp), m, fp(F.kx), F.nbx, cap);
    PassArgs check = make_pass(W, true, eps, as, cap);
    check.fin.mode = kFinResidLog2;  // the lift can be far off: log2 of the residual stays finite
    check.fin.w = fp(F.sa);
    check.fin.nrm = fp(F.snrm);
    check.fin.pot_in = fp(F.sf);
    check.fin.rbuf = W.f(L.rbuf);
    retarget(check, fp(F.sq), F.ns, W.f(L.yp), m, cap);
    // decisions on log2 of the check value: the same comparisons as on the value itself
    const double log2_tol = o.tol > 0.0f ? std::log2((double)o.tol) : -INFINITY;
    const double log2_keep = 1.0 - (double)o.coarse_gain > 0.0 ? std::log2(1.0 - (double)o.coarse_gain) : INFINITY;
    double prev = NAN;
    for (int round = 1;; ++round) {
        if ((st = prepare(Wc, fp(F.xcen), fp(F.ycen), fp(F.amass), fp(F.bmass), eps, 0, nullptr, round == 1 ? 1 : 2,
                          Gc, s)))
            return st;
        PassArgs row = make_pass(Wc, true, eps, fp(F.amass), cap);
        row.fin.pot = Fc;
        PassArgs col = make_pass(Wc, false, eps, fp(F.bmass), cap);
        col.fin.pot = Gc;
        for (int k = 0; k < o.coarse_iters; ++k) {
            if ((st = run_pass(Wc, row, s))) return st;
            if ((st = run_pass(Wc, col, s))) return st;
        }
        // lift: one c-transform of each side against the other side's centroids
        // (f at the sampled rows only)
        SK_TRY(launch_pack(fp(F.ycen), F.nby, d, L.P, false, W.f(L.centre), fp(F.bmass), fp(F.ky), fp(F.knrm),
                           fp(F.kl2w), nullptr, 1.0f / eps, 2, Gc, nullptr, s));
        if ((st = run_pass(W, lift_fs, s))) return st;
        SK_TRY(launch_pack(fp(F.xcen), F.nbx, d, L.P, false, W.f(L.centre), fp(F.amass), fp(F.kx), fp(F.knrm),
                           fp(F.kl2w), nullptr, 1.0f / eps, 2, Fc, nullptr, s));
        if ((st = run_pass(W, lift_g, s))) return st;
        // sampled check of the lifted plan's rows over all points
        if ((st = run_pass(W, check, s))) return st;
        SK_TRY(launch_max_reduce(W.f(L.rbuf), F.ns, slot.dev(), s, slot.flag(), slot.next()));
        if ((st = slot.read(host, 1, s))) return st;
        const double lc = host[0];  // log2 of the largest sampled |(P1)_i - a_i|
        info->rounds = round;
        info->last_check = (float)std::exp2(lc);
        if (lc <= log2_tol || round >= o.max_rounds) break;
        // stop when the check fell by less than the fraction coarse_gain: c > (1 - gain) c_prev
        // (a fall of 100% or more is impossible: then always)
        if (round >= 2 && (log2_keep == INFINITY || lc > log2_keep + prev)) break;
        prev = lc;
    }
    // f at every point from the accepted round (the packed centroids ky are still that round's)
    if ((st = run_pass(W, lift_f, s))) return st;

    // 4-5: block-sparse fine stage from the lifted potentials
    pause.reset();
    ScreenArgs sa{};
    sa.fmax = fp(F.fmax);
    sa.gmax = fp(F.gmax);
    sa.amass = fp(F.amass);
    sa.bmass = fp(F.bmass);
    sa.xlo = fp(F.xlo);
    sa.xhi = fp(F.xhi);
    sa.ylo = fp(F.ylo);
    sa.yhi = fp(F.yhi);
    sa.nbx = F.nbx;
    sa.nby = F.nby;
    sa.d = d;
    sa.eps = eps;
    sa.delta = o.delta;
    sa.log_delta = o.delta > 0.0f ? (float)std::log((double)o.delta) : -INFINITY;
    sa.dx = fp(F.srx);
    sa.dy = fp(F.sry);
    sa.rowbest = ip(F.rowbest);
    sa.colbest = ip(F.colbest);
    sa.cap = F.list_cap;
    SparseArgs rowp{}, colp{};
    rowp.q = W.f(L.xp);
    rowp.k = W.f(L.yp);
    rowp.nq = n;
    rowp.nk = m;
    rowp.B = F.B;
    rowp.qscale = 2.0f * kLog2e / eps;
    rowp.ptr = ip(F.rptr);
    rowp.idx = ip(F.ridx);
    rowp.fin = make_pass(W, true, eps, as, cap).fin;
    rowp.fin.pot = fs;
    rowp.nqb = F.nbx;
    rowp.W = F.sparse_groups;
    rowp.part = reinterpret_cast<float2*>(base + F.spart);
    colp = rowp;
    colp.q = W.f(L.yp);
    colp.k = W.f(L.xp);
    colp.nq = m;
    colp.nk = n;
    colp.ptr = ip(F.cptr);
    colp.idx = ip(F.cidx);
    colp.fin = make_pass(W, false, eps, bs, cap).fin;
    colp.fin.pot = gs;
    colp.nqb = F.nby;
    SparseArgs probe = rowp;
    probe.fin.mode = kFinProbe;
    probe.fin.rbuf = W.f(L.rbuf);
    double kept_pairs = 0.0;
    for (int it = 1; it <= o.max_iters; ++it) {
        if ((it - 1) % o.screen_every == 0) {
            SK_TRY(launch_block_max(fs, as, n, F.B, fp(F.fmax), s));
            SK_TRY(launch_block_max(gs, bs, m, F.B, fp(F.gmax), s));
            SK_TRY(launch_screen(sa, ip(F.rcnt), ip(F.rptr), ip(F.ridx), ip(F.ccnt), ip(F.cptr), ip(F.cidx), s));
            // the kept total must fit the lists before any sparse pass reads them (a host
            // read per screening); the last row block's list and the last column block's
            // count give the point pairs of the kept tiles for the pass timing
            int rp[2], cp[2], last = -1;
            SK_TRY(hipMemcpyAsync(rp, ip(F.rptr) + F.nbx - 1, sizeof rp, hipMemcpyDeviceToHost, s));
            SK_TRY(hipMemcpyAsync(cp, ip(F.cptr) + F.nby - 1, sizeof cp, hipMemcpyDeviceToHost, s));
            SK_TRY(hipStreamSynchronize(s));
            if ((int64_t)rp[1] > F.list_cap) return SK_ERR_SHAPE;  // more kept tiles than the lists hold
            if (timing_on()) {
                // full B x B tiles, less the short last row / column block
                if (rp[1] > rp[0]) {
                    SK_TRY(hipMemcpyAsync(&last, ip(F.ridx) + rp[1] - 1, sizeof last, hipMemcpyDeviceToHost, s));
                    SK_TRY(hipStreamSynchronize(s));
                }
                const double Bd = F.B, sr = Bd - (double)(n - (int64_t)(F.nbx - 1) * F.B),
                             sc = Bd - (double)(m - (int64_t)(F.nby - 1) * F.B);
                kept_pairs = Bd * Bd * rp[1] - Bd * sr * (rp[1] - rp[0]) - Bd * sc * (cp[1] - cp[0]) +
                             sr * sc * (last == F.nby - 1 ? 1.0 : 0.0);
            }
        }
        hipEvent_t e0, e1;
        if ((st = timing_events_pairs(kept_pairs, s, &e0, &e1))) return st;
        SK_TRY(launch_pass_sparse(rowp, d, s, e0, e1));
        if ((st = timing_events_pairs(kept_pairs, s, &e0, &e1))) return st;
        SK_TRY(launch_pass_sparse(colp, d, s, e0, e1));
        info->fine_iters = it;
        if (it % o.check_every == 0 || it == o.max_iters) {
            SK_TRY(launch_pass_sparse(probe, d, s));
            SK_TRY(launch_resid_reduce(W.f(L.rbuf), n, slot.dev(), nullptr, s, slot.flag(), slot.next()));
            if ((st = slot.read(host, 1, s))) return st;
            info->residual = host[0];
            if (host[0] <= o.tol) {
                info->converged = 1;
                break;
            }
        }
    }
    if (o.max_iters > 0) {
        int kept = 0;
        SK_TRY(hipMemcpyAsync(&kept, ip(F.rptr) + F.nbx, sizeof(int), hipMemcpyDeviceToHost, s));
        SK_TRY(hipStreamSynchronize(s));
        info->kept = kept;
    }
    SK_TRY(launch_scatter(fs, ip(F.permx), n, f_out, s));
    SK_TRY(launch_scatter(gs, ip(F.permy), m, g_out, s));
    if (perm_x) SK_TRY(hipMemcpyAsync(perm_x, ip(F.permx), (size_t)n * 4, hipMemcpyDeviceToDevice, s));
    if (perm_y) SK_TRY(hipMemcpyAsync(perm_y, ip(F.permy), (size_t)m * 4, hipMemcpyDeviceToDevice, s));
    return SK_OK;
}

int check_fs2(int64_t n, int64_t m, int32_t d, const Fs2Opts& o) {
    int st = check_sizes(n, m, d);
    if (st) return st;
    if (d > kValuMaxD) return SK_ERR_UNSUPPORTED_D;
    if (o.B < 1 || o.B > valu_block_rows()) return SK_ERR_SHAPE;
    const int64_t nbx = (n + o.B - 1) / o.B, nby = (m + o.B - 1) / o.B;
    if (nbx * nby > kMaxTiles) return SK_ERR_SHAPE;
    if (o.delta <= 0.0f && nbx * nby > kMaxKeptTiles) return SK_ERR_SHAPE;  // delta 0 keeps every tile
    if (!(o.tol >= 0.0f) || !std::isfinite(o.tol) || !(o.delta >= 0.0f) || !std::isfinite(o.delta) ||
        !std::isfinite(o.coarse_gain))
        return SK_ERR_STOP;
    if (o.coarse_iters < 1 || o.max_rounds < 1 || o.n_sample < 1 || o.max_iters < 0 || o.check_every < 1 ||
        o.screen_every < 1)
        return SK_ERR_ITERS;
    return SK_OK;
}


int check_ex(int variant, float alpha, int stop_mode, float tol, int max_iter, int check_every) {
    if (variant != 0 && variant != 1) return SK_ERR_VARIANT;
    if (variant == 1 && !(alpha > 0.0f && alpha <= 1.0f)) return SK_ERR_VARIANT;
    if (max_iter < 0) return SK_ERR_ITERS;
    if (stop_mode < 0 || stop_mode > 2) return SK_ERR_STOP;
    if (stop_mode != 0 && (!(tol >= 0.0f) || !std::isfinite(tol) || check_every < 1)) return SK_ERR_STOP;
    return SK_OK;
}

// Workspace of sk_divergence: the largest of the three solver layouts, then
// one potential pair of max(n, m) floats each.
struct DivLayout {
    size_t solver, f, g, total;
};
DivLayout div_layout(int64_t n, int64_t m, int d) {
    DivLayout D{};
    D.solver = std::max({make_layout(n, m, d).total, make_layout(n, n, d).total, make_layout(m, m, d).total});
    D.solver = align_up(D.solver, 256);
    const size_t pot = align_up((size_t)std::max(n, m) * 4, 256);
    D.f = D.solver;
    D.g = D.f + pot;
    D.total = D.g + pot;
    return D;
}

}  // namespace

}  // namespace sk

// Device scratch of sk_solve_noalloc, for callers that cannot allocate: one
// copy per GPU, held until the process ends.  In host code this name stands
// for a host-side shadow, not device memory; the device address is taken once
// per device with hipGetSymbolAddress (scratch_address below) and only that
// address reaches kernels.
static __device__ __align__(256) unsigned char scratch[SK_NOALLOC_SCRATCH_BYTES];

namespace sk {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device (null until first taken)

// The current device's address of `scratch`, taken on the first call on that device.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SK_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SK_ERR_HIP;
        if (reinterpret_cast<uintptr_t>(p) % 256 != 0) return SK_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SK_OK;
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int sk_abi_version(void) { return kAbiVersion; }

const char* sk_status_string(int status) {
    switch (status) {
        case SK_OK: return "ok";
        case SK_ERR_NULL: return "a required pointer is NULL";
        case SK_ERR_SHAPE:
            return "invalid sizes or shape arguments (n, m, d >= 1 and n, m < 2^31; payload widths, block sizes and "
                   "block-pair counts within the entry point's limits)";
        case SK_ERR_UNSUPPORTED_D: return "unsupported dimension d";
        case SK_ERR_EPS: return "eps must be finite and > 0 (and 2*log2(e)/eps finite in fp32)";
        case SK_ERR_ITERS: return "an iteration or step count is out of range";
        case SK_ERR_CHECK_EVERY: return "check_every must be >= 0, with resid_trace when > 0";
        case SK_ERR_NEG_WEIGHT: return "weights must be nonnegative";
        case SK_ERR_MASS_MISMATCH: return "sum(a) must equal sum(b)";
        case SK_ERR_EMPTY_MEASURE: return "sum(a) and sum(b) must be > 0";
        case SK_ERR_NONFINITE: return "inputs contain NaN or Inf";
        case SK_ERR_WORKSPACE: return "workspace missing, misaligned (256 B) or too small";
        case SK_ERR_HIP: return "HIP runtime or kernel launch failure";
        case SK_ERR_VARIANT: return "variant must be 0 (alternating) or 1 (symmetric, 0 < alpha <= 1)";
        case SK_ERR_STOP:
            return "invalid stop or threshold arguments (stop_mode 0, 1 or 2; tolerances and thresholds finite and "
                   ">= 0; check_every >= 1)";
        case SK_ERR_CAPTURE: return "this call synchronises the stream and cannot run under graph capture";
        case SK_ERR_LR: return "the step size must be finite";
        case SK_ERR_SCRATCH:
            return "the problem needs more workspace than the static scratch of sk_solve_noalloc holds "
                   "(sk_workspace_bytes(n, m, d) > SK_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int sk_timing_enable(int enable) {
    Timing& T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    T.on = enable > 0;
    T.stride = enable > 0 ? enable : 1;
    T.seen = 0;
    T.used = 0;
    T.pairs = 0.0;
    return SK_OK;
}

int sk_timing_read(double* total_ms, int64_t* launches, double* pairs) {
    if (!total_ms || !launches || !pairs) return SK_ERR_NULL;
    Timing& T = timing();
    std::lock_guard<std::mutex> lk(T.mu);
    double tot = 0.0;
    for (size_t k = 0; k < T.used; ++k) {
        SK_TRY(hipEventSynchronize(T.pool[2 * k + 1]));
        float ms = 0.0f;
        SK_TRY(hipEventElapsedTime(&ms, T.pool[2 * k], T.pool[2 * k + 1]));
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int64_t)T.used;
    *pairs = T.pairs;
    return SK_OK;
}

size_t sk_workspace_bytes(int64_t n, int64_t m, int32_t d) {
    if (n < 1 || m < 1 || d < 1 || d > kMaxD || n > INT32_MAX || m > INT32_MAX) return 0;
    return make_layout(n, m, d).total;
}

int sk_check_inputs(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m,
                    int32_t d, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{L, static_cast<char*>(ws)};
    SK_TRY(launch_check(x, y, a, b, (int)n, (int)m, d, W.dbl(L.red), W.dbl(L.chk), s));
    double res[4];
    SK_TRY(hipMemcpyAsync(res, W.dbl(L.chk), sizeof(res), hipMemcpyDeviceToHost, s));
    SK_TRY(hipStreamSynchronize(s));
    if (res[0] != 0.0) return SK_ERR_NONFINITE;
    if (res[1] != 0.0) return SK_ERR_NEG_WEIGHT;
    if (!(res[2] > 0.0) || !(res[3] > 0.0)) return SK_ERR_EMPTY_MEASURE;
    if (std::fabs(res[2] - res[3]) > 1e-5 * std::max(res[2], res[3])) return SK_ERR_MASS_MISMATCH;
    return SK_OK;
}

int sk_solve(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
             float eps, int32_t n_iters, float* f, float* g, int32_t check_every, float* resid_trace, void* ws,
             size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (n_iters < 0) return SK_ERR_ITERS;
    if (check_every < 0 || (check_every > 0 && n_iters / check_every > 0 && !resid_trace))
        return SK_ERR_CHECK_EVERY;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    Ws W{L, static_cast<char*>(ws)};
    return solve_fixed(W, x, y, a, b, eps, n_iters, f, g, check_every, resid_trace,
                       reinterpret_cast<hipStream_t>(stream));
}

int sk_solve_warm(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                  float eps, int32_t n_iters, const float* g_init, float* f, float* g, int32_t check_every,
                  float* resid_trace, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !g_init || !f || !g) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (n_iters < 0) return SK_ERR_ITERS;
    if (check_every < 0 || (check_every > 0 && n_iters / check_every > 0 && !resid_trace))
        return SK_ERR_CHECK_EVERY;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    Ws W{L, static_cast<char*>(ws)};
    return solve_fixed(W, x, y, a, b, eps, n_iters, f, g, check_every, resid_trace,
                       reinterpret_cast<hipStream_t>(stream), g_init);
}

int sk_primal_cost(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                   float eps, const float* f, const float* g, double* out, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !out) return SK_ERR_NULL;
    int st = check_transport_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    const TLayout T = make_tlayout(n, m, d);
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < T.total) return SK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{T.L, static_cast<char*>(ws)};
    const Layout& L = T.L;
    const int cap = pass_capacity(d);
    if (cap <= 0) return SK_ERR_HIP;
    if ((st = prepare(W, x, y, a, b, eps, 2, f, 2, g, s))) return st;
    float* U = W.f(T.B);        // m x (d + 1): [y~_j, |y~_j|^2]
    float* Tr = W.f(T.U);       // n x (d + 1): per-row sums of P U
    float* r = W.f(T.diag);     // P 1
    float* c = r + n;           // P^T 1
    SK_TRY(launch_primal_payload(W.f(L.yp), L.P, d, W.f(L.ny), (int)m, U, s));
    if (L.mfma) {
        TimingPause pause;
        if ((st = store_lse(W, true, eps, a, s))) return st;
    }
    if ((st = transport_cols(W, T, true, eps, U, d + 1, Tr, r, s))) return st;
    PassArgs col = make_pass(W, false, eps, b, cap);
    col.fin.mode = kFinMass;
    col.fin.pot_in = g;
    col.fin.rbuf = c;
    if ((st = run_pass(W, col, s))) return st;
    SK_TRY(launch_primal(a, b, f, g, r, c, W.f(L.xp), L.P, d, W.f(L.nx), Tr, (int)n, (int)m, eps,
                         reinterpret_cast<double*>(W.f(T.pv)), out, s));
    return SK_OK;
}

int sk_solve_noalloc(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m,
                     int32_t d, float eps, int32_t n_iters, float* f, float* g, int32_t check_every,
                     float* resid_trace, void* stream) {
    if (!x || !y || !a || !b || !f || !g) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (n_iters < 0) return SK_ERR_ITERS;
    if (check_every < 0 || (check_every > 0 && n_iters / check_every > 0 && !resid_trace))
        return SK_ERR_CHECK_EVERY;
    const Layout L = make_layout(n, m, d);
    if (L.total > (size_t)SK_NOALLOC_SCRATCH_BYTES) return SK_ERR_SCRATCH;
    void* ptr = nullptr;
    if ((st = scratch_address(&ptr))) return st;
    // every region the solve reads is written first by the same call: nothing needs clearing
    Ws W{L, static_cast<char*>(ptr)};
    return solve_fixed(W, x, y, a, b, eps, n_iters, f, g, check_every, resid_trace,
                       reinterpret_cast<hipStream_t>(stream));
}

int sk_cost(const float* a, const float* b, const float* f, const float* g, int64_t n, int64_t m, float eps,
            double* out, void* stream) {
    if (!a || !b || !f || !g || !out) return SK_ERR_NULL;
    if (n < 1 || m < 1 || n > INT32_MAX || m > INT32_MAX) return SK_ERR_SHAPE;
    int st = check_eps(eps);
    if (st) return st;
    SK_TRY(launch_cost(a, b, f, g, (int)n, (int)m, eps, out, reinterpret_cast<hipStream_t>(stream)));
    return SK_OK;
}

int sk_marginal_residual(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m,
                         int32_t d, float eps, const float* f, const float* g, float* out, void* ws,
                         size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !out) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{L, static_cast<char*>(ws)};
    const int cap = pass_capacity(d);
    if (cap <= 0) return SK_ERR_HIP;
    if ((st = prepare(W, x, y, a, b, eps, 2, f, 2, g, s))) return st;
    float* rbuf = W.f(L.rbuf);

    PassArgs row = make_pass(W, true, eps, a, cap);
    row.fin.mode = kFinResid;
    row.fin.pot_in = f;
    row.fin.rbuf = rbuf;
    if ((st = run_pass(W, row, s))) return st;
    SK_TRY(launch_resid_reduce(rbuf, (int)n, out + 0, out + 2, s));

    PassArgs col = make_pass(W, false, eps, b, cap);
    col.fin.mode = kFinResid;
    col.fin.pot_in = g;
    col.fin.rbuf = rbuf;
    if ((st = run_pass(W, col, s))) return st;
    SK_TRY(launch_resid_reduce(rbuf, (int)m, out + 1, out + 3, s));
    return SK_OK;
}

int sk_grad_x(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
              float eps, const float* g, float* grad, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !g || !grad) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    Ws W{L, static_cast<char*>(ws)};
    return grad_core(W, x, y, a, b, eps, g, grad, reinterpret_cast<hipStream_t>(stream));
}
int sk_solve_ex(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                float eps, int32_t variant, float alpha, int32_t stop_mode, float stop_tol, int32_t max_iter,
                int32_t check_every, float* f, float* g, int32_t* iters_run, int32_t* converged,
                float* final_viol, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !iters_run || !converged || !final_viol) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if ((st = check_ex(variant, alpha, stop_mode, stop_tol, max_iter, check_every))) return st;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (stop_mode != 0) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cap) != hipSuccess) return SK_ERR_HIP;
        if (cap != hipStreamCaptureStatusNone) return SK_ERR_CAPTURE;
    }
    Ws W{L, static_cast<char*>(ws)};
    ExOpts o{variant, variant == 1 ? alpha : 1.0f, stop_mode, stop_tol, max_iter, check_every};
    ExResult r{};
    if ((st = solve_ex(W, x, y, a, b, eps, o, f, g, &r, s))) return st;
    *iters_run = r.iters;
    *converged = r.converged;
    *final_viol = r.viol;
    return SK_OK;
}

int sk_dual_cost(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                 float eps, const float* f, const float* g, double* out, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !out) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    Ws W{L, static_cast<char*>(ws)};
    return dual_cost(W, x, y, a, b, eps, f, g, out, reinterpret_cast<hipStream_t>(stream));
}

size_t sk_divergence_workspace_bytes(int64_t n, int64_t m, int32_t d) {
    if (check_sizes(n, m, d) != SK_OK) return 0;
    return div_layout(n, m, d).total;
}

int sk_divergence(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                  float eps, int32_t variant, float alpha, int32_t n_iters, double* out, void* ws, size_t ws_bytes,
                  void* stream) {
    if (!x || !y || !a || !b || !out) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if ((st = check_ex(variant, alpha, 0, 0.0f, n_iters, 1))) return st;
    const DivLayout D = div_layout(n, m, d);
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < D.total) return SK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    float* fb = reinterpret_cast<float*>(base + D.f);
    float* gb = reinterpret_cast<float*>(base + D.g);
    const ExOpts o{variant, variant == 1 ? alpha : 1.0f, 0, 0.0f, n_iters, 1};
    struct Term {
        const float *p, *q, *wp, *wq;
        int64_t np, nq;
    };
    const Term terms[3] = {{x, y, a, b, n, m}, {x, x, a, a, n, n}, {y, y, b, b, m, m}};
    for (int t = 0; t < 3; ++t) {
        const Term& T = terms[t];
        Ws W{make_layout(T.np, T.nq, d), base};
        ExResult r{};
        if ((st = solve_ex(W, T.p, T.q, T.wp, T.wq, eps, o, fb, gb, &r, s))) return st;
        if ((st = dual_cost(W, T.p, T.q, T.wp, T.wq, eps, fb, gb, out + 1 + t, s))) return st;
    }
    SK_TRY(launch_div_combine(out, s));
    return SK_OK;
}

int sk_gradient_flow(float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                     float eps, int32_t n_iters, int32_t n_steps, float lr, float* f, float* g, float* grad,
                     double* cost_trace, void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !grad) return SK_ERR_NULL;
    int st = check_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (n_iters < 0 || n_steps < 0) return SK_ERR_ITERS;
    if (!std::isfinite(lr)) return SK_ERR_LR;
    const Layout L = make_layout(n, m, d);
    if ((st = check_ws(ws, ws_bytes, L))) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{L, static_cast<char*>(ws)};
    for (int k = 0; k < n_steps; ++k) {
        if ((st = solve_fixed(W, x, y, a, b, eps, n_iters, f, g, 0, nullptr, s))) return st;
        if (cost_trace) SK_TRY(launch_cost(a, b, f, g, (int)n, (int)m, eps, cost_trace + k, s));
        if ((st = grad_core(W, x, y, a, b, eps, g, grad, s))) return st;
        SK_TRY(launch_axpy(x, grad, n * d, -lr, s));
    }
    return SK_OK;
}

size_t sk_transport_workspace_bytes(int64_t n, int64_t m, int32_t d) {
    if (check_transport_sizes(n, m, d) != SK_OK) return 0;
    return make_tlayout(n, m, d).total;
}

int sk_transport(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                 float eps, const float* f, const float* g, int32_t transpose, const float* v, int32_t k, float* out,
                 void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !v || !out) return SK_ERR_NULL;
    int st = check_transport_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (k < 1 || (transpose != 0 && transpose != 1)) return SK_ERR_SHAPE;
    const TLayout T = make_tlayout(n, m, d);
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < T.total) return SK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{T.L, static_cast<char*>(ws)};
    const bool row_side = transpose == 0;
    if ((st = prepare(W, x, y, a, b, eps, 2, f, 2, g, s))) return st;
    if (T.L.mfma) {
        TimingPause pause;  // the pass timing covers the transport kernel
        if ((st = store_lse(W, row_side, eps, row_side ? a : b, s))) return st;
    }
    return transport_cols(W, T, row_side, eps, v, k, out, nullptr, s);
}

int sk_hvp(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
           float eps, const float* f, const float* g, const float* v, int32_t cg_iters, float* out, float* cg_resid,
           void* ws, size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !v || !out) return SK_ERR_NULL;
    int st = check_transport_sizes(n, m, d);
    if (st) return st;
    if ((st = check_eps(eps))) return st;
    if (cg_iters < 0) return SK_ERR_ITERS;
    const TLayout T = make_tlayout(n, m, d);
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < T.total) return SK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Ws W{T.L, static_cast<char*>(ws)};
    const Layout& L = T.L;
    const int in = (int)n, im = (int)m, N = in + im;
    float *A = W.f(T.A), *stv = W.f(T.st), *U = W.f(T.U), *B = W.f(T.B), *E = W.f(T.E);
    float *diag = W.f(T.diag), *rhs = W.f(T.rhs), *z = W.f(T.z), *zb = W.f(T.zb), *res = W.f(T.res), *p = W.f(T.p);
    float* prod = W.f(T.prod);
    double* scal = W.dbl(T.scal);
    if ((st = prepare(W, x, y, a, b, eps, 2, f, 2, g, s))) return st;
    {
        // the pass timing covers the single-column products of the CG steps
        TimingPause pause;
        if (L.mfma) {  // the plan is fixed: one lse pass per side serves every product below
            if ((st = store_lse(W, true, eps, a, s))) return st;
            if ((st = store_lse(W, false, eps, b, s))) return st;
        }
        // A = P y~ and r = P 1
        if (L.mfma) {
            if ((st = transport_pass(W, T, true, eps, 1, nullptr, 0, 0, nullptr, A, d, d, diag, s))) return st;
        } else {
            if ((st = transport_pass(W, T, true, eps, 0, W.f(L.yp), L.P, d, nullptr, A, d, d, diag, s))) return st;
        }
        SK_TRY(launch_hvp_rows(W.f(L.xp), L.P, d, in, v, A, diag, stv, rhs, U, s));
        // B = P^T [st, v] and c = P^T 1
        if ((st = transport_cols(W, T, false, eps, U, d + 1, B, diag + in, s))) return st;
        SK_TRY(launch_hvp_cols(W.f(L.yp), L.P, d, im, B, rhs + in, s));
    }
    SK_TRY(launch_cg_init(N, in, diag, rhs, z, zb, res, p, scal, s));
    for (int it = 0; it < cg_iters; ++it) {
        if ((st = transport_pass(W, T, true, eps, 0, p + in, 1, 1, nullptr, prod, 1, 1, nullptr, s))) return st;
        if ((st = transport_pass(W, T, false, eps, 0, p, 1, 1, nullptr, prod + in, 1, 1, nullptr, s))) return st;
        SK_TRY(launch_cg_step(N, in, diag, prod, z, zb, res, p, scal, s));
    }
    if (cg_resid) SK_TRY(launch_cg_report(scal, cg_resid, s));
    // E = sum_j P_ij (psi_j + 2 <y~_j, v_i>) y~_j, then the product
    {
        TimingPause pause;
        if ((st = transport_pass(W, T, true, eps, 2, zb + in, 1, 1, v, E, d, d, nullptr, s))) return st;
    }
    SK_TRY(launch_hvp_final(in, d, eps, v, diag, stv, zb, A, E, out, s));
    return SK_OK;
}

size_t sk_fs2_workspace_bytes(int64_t n, int64_t m, int32_t d, int32_t block, int32_t n_sample) {
    // the workspace does not depend on the thresholds: a positive delta stands in for any
    Fs2Opts o{block, 0.0f, 1e-6f, 1, 1, 0.0f, std::max(n_sample, 1), 0, 1, 1};
    if (check_fs2(n, m, d, o) != SK_OK) return 0;
    FLayout F;
    if (!make_flayout(n, m, d, block, std::max(n_sample, 1), &F)) return 0;
    return F.total;
}

int sk_fs2_solve(const float* x, const float* y, const float* a, const float* b, int64_t n, int64_t m, int32_t d,
                 float eps, int32_t block, float tol, float delta, int32_t coarse_iters, int32_t max_rounds,
                 float coarse_gain, int32_t n_sample, int32_t max_iters, int32_t check_every, int32_t screen_every,
                 float* f, float* g, int32_t* info_i, float* info_f, int32_t* perm_x, int32_t* perm_y, void* ws,
                 size_t ws_bytes, void* stream) {
    if (!x || !y || !a || !b || !f || !g || !info_i || !info_f) return SK_ERR_NULL;
    int st;
    if ((st = check_eps(eps))) return st;
    const Fs2Opts o{block, tol, delta, coarse_iters, max_rounds, coarse_gain, n_sample, max_iters, check_every,
                    screen_every};
    if ((st = check_fs2(n, m, d, o))) return st;
    FLayout F;
    if (!make_flayout(n, m, d, block, n_sample, &F)) return SK_ERR_HIP;
    if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) % 256) != 0 || ws_bytes < F.total) return SK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return SK_ERR_HIP;
    if (cap != hipStreamCaptureStatusNone) return SK_ERR_CAPTURE;
    Fs2Info info;
    if ((st = fs2_solve(static_cast<char*>(ws), F, x, y, a, b, eps, o, f, g, perm_x, perm_y, &info, s))) return st;
    info_i[0] = info.rounds;
    info_i[1] = info.fine_iters;
    info_i[2] = info.kept;
    info_i[3] = info.converged;
    info_f[0] = info.residual;
    info_f[1] = info.last_check;
    return SK_OK;
}

}  // extern "C"

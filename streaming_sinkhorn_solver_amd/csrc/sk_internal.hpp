// sk_internal.hpp -- shared definitions of the HIP implementation behind sk.h.
//
// Notation follows "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
// (technical summary, Methodology 1): for squared-Euclidean cost the row
// half-step f_i = -eps LSE_j[(g_j - C_ij)/eps + log b_j] is a log-sum-exp of a
// biased dot-product score.  With C_ij = |x_i|^2 + |y_j|^2 - 2<x_i, y_j> and
// everything in base 2 (log2e = 1/ln 2):
//
//     s_ij  = <q_i, y_j> + h_j,     q_i = (2 log2e / eps) x_i,
//     h_j   = log2 b_j + log2e (g_j - |y_j|^2) / eps      (the "bias" of key j),
//     lse_i = log2 sum_j 2^{s_ij}    (running max M and rescaled sum S),
//     f_i   = |x_i|^2 - eps ln2 lse_i.
//
// The column half-step is the same with the roles of (x, a, f) and (y, b, g)
// swapped.  Inside a solve the bias of the next pass is simply
// h_i = log2 a_i - lse_i, because g (or f) enters only through lse.
//
// Both clouds are first shifted by a common centre c = (mean x + mean y)/2,
// which leaves every C_ij unchanged and keeps |x|^2, |y|^2 small so the
// expanded form loses little to fp32 cancellation.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

// Launches a kernel; when the event pair e0 / e1 is given, the two events take
// the kernel's own start and end times, recorded with its dispatch (no marker
// packets of their own that would lengthen the measured interval of a short
// kernel).  Timed launches never occur under graph capture.
#define SK_LAUNCH_TIMED(kernel, grid, block, stream, e0, e1, ...)                                \
    do {                                                                                          \
        if (e0)                                                                                   \
            hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e0, e1, 0, __VA_ARGS__);        \
        else                                                                                      \
            hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                      \
    } while (0)

namespace sk {

constexpr int kBlock = 256;               // threads per workgroup (4 wave64s)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -3.402823466e38f;  // running-max start: -FLT_MAX, never -inf
constexpr int kXcds = 8;                     // XCDs (each with its own L2) that workgroups are dealt to
constexpr int kMaxD = 256;
constexpr int kValuMaxD = 8;              // d <= 8: vector-ALU kernels; else matrix cores
constexpr int kRedBlocks = 512;           // fixed partial count of the 2-stage reductions
constexpr int kMaxSplit = 64;             // column splits of one gradient pass
constexpr int kMaxGroups = 2048;          // workgroups of one matrix-core streamed pass (upper bound)
constexpr int kMaxGroupsValu = 8192;      // workgroups of one vector-ALU streamed pass (upper bound)
constexpr int kValuRounds = 4;            // resident rounds of workgroups a vector-ALU pass may take
constexpr int kRoundKeys = 1800;          // per-workgroup units of one round that call for another round
#ifndef SK_MIN_KEYS
#define SK_MIN_KEYS 64
#endif
constexpr int kMinKeysPerGroup = SK_MIN_KEYS;  // smallest key range a workgroup is given

// Packed stride (floats) of one point in the workspace.
//  VALU layout:  [coords (d) | bias | zero pad] to a multiple of 4 (float4 loads).
//  MFMA layout:  [coords (d) | zero pad] to max(16, next power of two >= d);
//                the bias is kept in a separate array.
inline int packed_stride(int d) {
    if (d <= kValuMaxD) return ((d + 1 + 3) / 4) * 4;
    int p = 16;
    while (p < d) p *= 2;
    return p;
}

// What a streamed pass does with each finished row's log-sum-exp.
enum FinMode : int {
    kFinSolve = 0,   // store lse, next-pass bias, output potential; optional fused residual
    kFinProbe = 1,   // residual of the previous state only (no state change)
    kFinResid = 2,   // residual against a caller-supplied potential
    kFinStore = 3,   // store lse only
    kFinMass = 4,    // row sums of the plan at a caller-supplied potential
    kFinResidLog2 = 5,  // log2 |residual| against a caller-supplied potential (finite beyond float32 range)
};

// kFinSolve keeps the state as u_i = (|q~_i|^2 - f_i) / (eps ln 2), the base-2
// log-sum-exp of the last pass for a plain update.  A blended update (the
// symmetric variant) stores u' = u + alpha (lse - u), i.e. f' = (1 - alpha) f +
// alpha f~ in cost units; alpha = 1 is the plain update and reads no old state.
struct Fin {
    int mode;
    int P;               // packed stride of the query cloud (bias slot at index d)
    int d;
    float eps_ln2;       // eps * ln 2
    float inv_eps;       // 1 / eps
    float alpha;         // blend weight of kFinSolve (1 = replace)
    float* lse;          // [nq] state u before the pass (read for a residual or a blend)
    float* lse_out;      // [nq] state after the pass (may equal lse)
    const float* l2w;    // [nq] log2 of the query-side weights (-inf for zero weight); read when a bias is written
    const float* w;      // [nq] query-side weights
    const float* nrm;    // [nq] |q~|^2 of the centred query points
    float* pot;          // [nq] output potential in cost units, or null
    float* bias_packed;  // query packed base (bias slot = index d), or null
    float* bias_sep;     // separate bias array (matrix-core layout), or null
    float* rbuf;         // [nq] |residual_i| (kFinSolve, kFinProbe, kFinResid) or (P1)_i (kFinMass)
    const float* pot_in; // [nq] caller potential (kFinResid, kFinMass)
};

// Arguments of one streamed log-sum-exp pass over all (query, key) pairs.
//
// Work decomposition ("stream-K"): the queries are cut into row blocks of
// rpb rows; the flattened space of (row block, key) units u = rb * nk + j,
// total = n_row_blocks * nk, is cut into W equal contiguous ranges
// [w * total / W, (w + 1) * total / W), one per workgroup, with W the number
// of workgroups the GPU holds at once.  A range covering a whole row block
// finishes it in place; a range that starts or ends inside a row block leaves
// a partial (M, S) for it in slot 0 (its first segment) or slot 1 (its last),
// and a merge kernel combines the partials of each row block in workgroup
// order.  (Merging inside the pass by the last workgroup to arrive was
// measured slower: every contributor then pays a device-scope release fence,
// and the merging workgroup's loop over all partials is serial.)
struct PassArgs {
    const float* q;      // query cloud, packed [nq][P]
    const float* k;      // key cloud, packed [nk][P]
    const float* kbias;  // separate key bias [nk] (matrix-core layout), else null
    const uint16_t* kb;  // matrix-core layout: fp16 parts of the scaled keys [nk][2][P] (h, l), else null
    const uint16_t* qb;  // matrix-core layout: the same parts of the queries [nq][2][P], else null
    const float* qmax;   // matrix-core layout: largest |packed coordinate| of the query cloud (device)
    const float* kmax;   // matrix-core layout: the same of the key cloud (device)
    int nq, nk, P;
    float qscale;        // 2 log2e / eps
    float rq;            // matrix-core layout: fl(sqrt(qscale)), the scale of both clouds' split parts
    int rpb;             // rows per block
    int W;               // workgroups
    int64_t total;       // n_row_blocks * nk
    float2* part;        // [W][2][rpb] partial (M, S)
    int small;           // d <= 8 and small: one workgroup per few rows, whole key range, no merge
    Fin fin;
};

// Arguments of the streamed gradient pass.
struct GradArgs {
    const float* q;      // x packed [n][P]
    const float* k;      // y packed [m][P] with bias slot holding h_j from g
    const float* kbias;  // separate key bias (matrix-core layout), else null
    int nq, nk, P, d;
    float qscale;
    int cols_per_split;
    int nsplit;
    float2* part;        // [nsplit][nq] partial (M, S)
    float* partA;        // [nsplit][nq][P] partial weighted key sums
    const float* w;      // a
    float* grad;         // [nq][d] output
    const float* lse;    // [nq] row log-sum-exp (matrix-core gradient, from a first pass)
};

// Arguments of a block-sparse pass (d <= 8): query block I (rows
// [I B, (I + 1) B)) scans the key blocks idx[ptr[I] .. ptr[I + 1]) (keys
// [J B, (J + 1) B)); rows and keys are in block (Morton) order.  The kept
// tiles are shared out stream-K style over W workgroups.
struct SparseArgs {
    const float* q;      // query cloud, packed [nq][P]
    const float* k;      // key cloud, packed [nk][P]
    int nq, nk, B, nqb;  // nqb = ceil(nq / B) query blocks
    float qscale;        // 2 log2e / eps
    const int* ptr;      // [nqb + 1]
    const int* idx;      // kept key blocks
    int W;               // workgroups
    float2* part;        // [W][2][B] partial (M, S) of split blocks
    Fin fin;
};

// Tile bounds of the block-sparse fine stage (sk_fs2.hip).
struct ScreenArgs {
    const float *fmax, *gmax;    // per-block maxima of the potentials (points of positive weight)
    const float *amass, *bmass;  // block masses
    const float *xlo, *xhi, *ylo, *yhi;  // block boxes [blocks][d]
    float *dx, *dy;              // per-block records [blocks][screen_stride_of(d)] (written by the screening)
    int nbx, nby, d;
    float eps, delta, log_delta;
    float inv_eps;               // 1 / eps (set by the screening)
    int* rowbest;                // [nbx] the tile of largest bound in each row block
    int* colbest;                // [nby] ... in each column block
    int64_t cap;                 // capacity of each tile list (entries)
};

// Floats per block record of the screening: box lo[d], hi[d], potential
// maximum, log mass term, padded to whole float4s.
constexpr int screen_stride_of(int d) { return (2 * d + 2 + 3) / 4 * 4; }

// Arguments of a streamed transport product (d <= 8; see sk_transport.hip).
struct TransArgs {
    const float* q;      // query cloud, packed [nq][P], bias slot = log2 w + log2e (pot - |q~|^2)/eps
    const float* k;      // key cloud, packed [nk][P], same bias from the key-side potential
    const float* kbias;  // matrix-core layout: key biases [nk], else null
    const uint16_t* kb;  // matrix-core layout: fp16 parts of the scaled keys [nk][2][P]
    const uint16_t* qb;  // matrix-core layout: the same parts of the queries [nq][2][P]
    const float* qmax;   // matrix-core layout: largest |packed coordinate| of the query cloud (device)
    const float* kmax;   // matrix-core layout: the same of the key cloud (device)
    float rq;            // matrix-core layout: fl(sqrt(2 log2e / eps)), the scale of the split parts
    const float* qbias;  // matrix-core layout: query biases [nq], else null
    const float* lse;    // matrix-core layout: row log-sum-exp of the scores [nq] (a first pass)
    const float* pay;    // payload: key j's columns at pay[j * ldp + c], c < kin
    const float* rowv;   // per-row direction [nq][d] (weighted mode), else null
    int nq, nk, P, d;
    float qscale;        // 2 log2e / eps
    int cols_per_split, nsplit;
    float2* part;        // [nsplit][nq] partial (M, S)
    float* partA;        // [nsplit][nq][accumulators] partial payload sums
    float* out;          // out[i * ldo + c], c < kout
    int ldo, kout, ldp, kin;
    float* mass;         // [nq] row sums of the plan, or null
    const float* gw;     // matrix-core gradient (mode 4): the row weights a [nq], else null
    uint16_t* kt;        // matrix-core layout: room for the payload's fp16 parts (the key coordinates in modes 1
                         // and 4, the payload columns in mode 0) transposed in blocks of 32 keys,
                         // [ceil(nk / 32)][2][columns][32] (written by the launch)
    float* pmax;         // matrix-core layout: room for the payload columns' largest magnitudes (64 floats, mode 0)
};

// Workspace carve-up, a pure function of (n, m, d).
struct Layout {
    int d, P;
    bool mfma;
    int64_t n, m;
    size_t xp, yp, hx, hy, nx, ny, l2a, l2b, lse_r, lse_c, rbuf, part, partA, red, cen, centre, chk;
    size_t xb, yb;            // fp16 parts of the scaled packed clouds (matrix-core layout)
    bool split;               // xb, yb are in use
    size_t amax, amax_part;   // largest |packed coordinate| of x and y (2 floats), and its per-block maxima
    size_t lse_r2, lse_c2;    // second state buffers (a check keeps the previous state)
    size_t snap_f, snap_g;    // potentials at the previous check (potential stop rule)
    size_t kt;                // matrix-core layout: transposed fp16 payload parts of the weighted sums (TransArgs::kt)
    size_t pmax;              // matrix-core layout: largest magnitude of each payload column (TransArgs::pmax)
    size_t total;
};

Layout make_layout(int64_t n, int64_t m, int d);

// Split policy of a streamed pass: number of column splits for nq queries
// against nk keys when one workgroup covers rows_per_block queries.
int plan_split(int64_t nq, int64_t nk, int rows_per_block);
// Key columns per split of the matrix-core transport kernels are a multiple of
// this (the transposed key parts are staged in whole blocks of 32 keys).
constexpr int kTransColAlign = 32;

// ----- launchers (return hipError_t of the launch) --------------------------------
hipError_t launch_centre(const float* x, const float* y, int n, int m, int d, double* partials,
                         float* centre, hipStream_t s);
// u_out (may be null): the state u matching the initial bias (0 for bias_mode 0).
hipError_t launch_pack(const float* pts, int npts, int d, int P, bool mfma, const float* centre,
                       const float* w, float* packed, float* nrm, float* l2w, float* bias_sep,
                       float inv_eps, int bias_mode, const float* pot, float* u_out, hipStream_t s);
hipError_t launch_fill(float* p, int64_t count, float value, hipStream_t s);
// Key bias h = log2 w - u of both clouds from their states (one launch).
struct BiasSide {
    const float* u;
    const float* l2w;
    float* packed;  // VALU layout: bias slot at index d of each packed row, else null
    float* sep;     // matrix-core layout: separate bias array, else null
    int npts;
};
hipError_t launch_apply_bias(const BiasSide& x, const BiasSide& y, int P, int d, hipStream_t s);
// pot_i = nrm_i - eps ln2 u_i (the potential of a stored state).
hipError_t launch_pot_from_state(const float* u, const float* nrm, float eps_ln2, float* pot, int npts,
                                 hipStream_t s);
// out[0] = max(max_i |f_i - sf_i|, max_j |g_j - sg_j|), then sf = f, sg = g.
// flag (may be null): set to seq once out[0] is visible to the host.
hipError_t launch_pot_change(const float* f, float* sf, int n, const float* g, float* sg, int m, float* out,
                             hipStream_t s, int* flag = nullptr, int seq = 0);
// mass (may be null): per-row plan sums (P1)_i; the cost then uses their float64
// sum as the plan mass instead of sum(b).
hipError_t launch_cost_mass(const float* a, const float* b, const float* f, const float* g, const float* mass,
                            int n, int m, float eps, double* out, hipStream_t s);
// U (m x (d + 1)) = [y~_j, |y~_j|^2], the payload of the plan's transport cost.
hipError_t launch_primal_payload(const float* yp, int P, int d, const float* ny, int m, float* U, hipStream_t s);
// out[0] = <P,C> + eps KL(P | a x b), out[1] = <P,C> from the plan's row sums r, column sums c and per-row
// payload sums T (n x (d + 1)) of U; pv is scratch for n doubles (each row's share of <P,C>).
hipError_t launch_primal(const float* a, const float* b, const float* f, const float* g, const float* r,
                         const float* c, const float* xp, int P, int d, const float* nx, const float* T, int n,
                         int m, float eps, double* pv, double* out, hipStream_t s);
// Transport products (sk_transport.hip).  mode 0: K-column payload, kwidth in
// {1, 4, 9} (>= kin); mode 2: the Hessian-vector product's weighted pass.
int transport_rows_per_block();
// Matrix-core transport products (d > 8, sk_pass_mfma.hip): mode 0 with up to
// 64 payload columns (kwidth 16 or 64), mode 1 (payload = the key coordinates),
// mode 2 (weighted pass); needs lse from a kFinStore pass over the same scores.
// Rows per workgroup of the matrix-core transport kernel for padded width P,
// mode and payload width (16 or 64); the largest over modes and widths.
int mfma_transport_rows_per_block(int P, int mode, int kwidth);
int mfma_transport_max_rows_per_block(int P);
// Workgroups of one transport kernel the GPU holds at once (current device; 0 on error).
int mfma_transport_capacity(int P, int mode, int kwidth);
int transport_capacity(int d, int mode, int kwidth);
hipError_t launch_transport_mfma(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0 = nullptr,
                                 hipEvent_t ev1 = nullptr);
// ev0 / ev1 (may be null): recorded right before and after the pass kernel (not the merge).
hipError_t launch_transport(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr);
hipError_t launch_hvp_rows(const float* xp, int P, int d, int n, const float* v, const float* A, const float* r,
                           float* st, float* rho, float* U, hipStream_t s);
hipError_t launch_hvp_cols(const float* yp, int P, int d, int m, const float* B, float* gam, hipStream_t s);
hipError_t launch_hvp_final(int n, int d, float eps, const float* v, const float* r, const float* st,
                            const float* phi, const float* A, const float* E, float* out, hipStream_t s);
hipError_t launch_cg_init(int N, int n, const float* diag, const float* rhs, float* z, float* zb, float* res, float* p,
                          double* scal, hipStream_t s);
hipError_t launch_cg_step(int N, int n, const float* diag, const float* prod, float* z, float* zb, float* res, float* p,
                          double* scal, hipStream_t s);
hipError_t launch_cg_report(const double* scal, float* out, hipStream_t s);
// Workgroups of a CG step's kernels; the step's scalars take 4 + 3 kCgBlocks doubles.
constexpr int kCgBlocks = 128;

// Two-stage block-sparse solver pieces (sk_fs2.hip).
hipError_t launch_bbox(const float* x, int n, const float* y, int m, int d, float* part, float* box, hipStream_t s);
hipError_t launch_morton(const float* p, int n, int d, int bits, const float* box, uint32_t* code, uint32_t* idx,
                         hipStream_t s);
size_t sort_temp_bytes(int n, int end_bit);  // 0 when the size cannot be queried
hipError_t launch_sort_pairs(void* temp, size_t temp_bytes, const uint32_t* kin, uint32_t* kout, const uint32_t* vin,
                             uint32_t* vout, int n, int end_bit, hipStream_t s);
hipError_t launch_gather_points(const float* p, const float* w, const uint32_t* idx, int n, int d, float* ps, float* ws,
                                int* perm, hipStream_t s);
hipError_t launch_block_stats(const float* ps, const float* ws, int n, int d, int B, float* mass, float* cen,
                              float* blo, float* bhi, hipStream_t s);
hipError_t launch_gather_rows(const float* qp, int P, const float* pot, const float* w, const float* nrm, int ns,
                              int stride, float* qs, float* pots, float* ws, float* nrms, hipStream_t s);
hipError_t launch_block_max(const float* pot, const float* w, int n, int B, float* out, hipStream_t s);
hipError_t launch_screen(const ScreenArgs& a, int* rcnt, int* rptr, int* ridx, int* ccnt, int* cptr, int* cidx,
                         hipStream_t s);
hipError_t launch_scatter(const float* in, const int* perm, int n, float* out, hipStream_t s);

// v <- v + alpha * u over count floats.
hipError_t launch_axpy(float* v, const float* u, int64_t count, float alpha, hipStream_t s);
// out[0] = out[1] - out[2] / 2 - out[3] / 2.
hipError_t launch_div_combine(double* out, hipStream_t s);
hipError_t launch_check(const float* x, const float* y, const float* a, const float* b, int n, int m,
                        int d, double* partials, double* result, hipStream_t s);
hipError_t launch_cost(const float* a, const float* b, const float* f, const float* g, int n, int m,
                       float eps, double* out, hipStream_t s);
// flag (may be null): set to seq once out_max[0] is visible to the host.
// max of v[0..cnt) (-inf when empty) into out[0], then the flag as in launch_resid_reduce
hipError_t launch_max_reduce(const float* v, int cnt, float* out, hipStream_t s, int* flag, int seq);
hipError_t launch_resid_reduce(const float* rbuf, int cnt, float* out_max, float* out_sum, hipStream_t s,
                               int* flag = nullptr, int seq = 0);
// Vector-ALU passes (d <= 8): a streamed pass, plus the exact merge of the
// split partials when nsplit > 1.
// ev0 / ev1 (may be null): events recorded on s right before and right after
// the pass kernel itself (not the merge).
hipError_t launch_pass_valu(const PassArgs& a, int d, hipStream_t s, hipEvent_t ev0 = nullptr,
                            hipEvent_t ev1 = nullptr);
hipError_t launch_grad_valu(const GradArgs& a, hipStream_t s);
int valu_rows_per_block();  // rows per row block of the dense pass
int valu_block_rows();      // rows per workgroup of the gradient and block-sparse passes
// Block-sparse vector-ALU pass (B <= 512 rows per query block).
hipError_t launch_pass_sparse(const SparseArgs& a, int d, hipStream_t s, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr);
// Merges the partial (M, S) pairs of row blocks split across workgroups (no
// launch when every row block was finished by one workgroup).
hipError_t launch_merge(const PassArgs& a, hipStream_t s);
// Matrix-core passes (9 <= d <= 256), by packed stride P in {16, 32, 64, 128, 256}.
hipError_t launch_pass_mfma(const PassArgs& a, hipStream_t s, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
int mfma_rows_per_block(int P);
int mfma_pass_capacity(int P);
// fp16 parts (h, l) of rows x P packed floats times rq and a power of two into
// out [rows][2][P], the exponent from the cloud's largest |coordinate| *cmax
// (device) times rq.
hipError_t launch_split2(const float* in, int64_t rows, int P, const float* cmax, float rq, uint16_t* out,
                         hipStream_t s);
// out[0] = max |x[e]| over nx floats, out[1] = the same over y (nx, ny multiples
// of 4); part holds 2 * kAbsMaxBlocks floats.
constexpr int kAbsMaxBlocks = 256;
hipError_t launch_absmax(const float* x, int64_t nx, const float* y, int64_t ny, float* part, float* out,
                         hipStream_t s);
// Matrix-core gradient pass (needs the row lse of the same scores); rows per workgroup.
// Rows per workgroup of the matrix-core gradient (transport mode 4) at padded stride P.
int mfma_grad_rows_per_block(int P);
// Workgroups of the d-dimensional pass kernel resident at once on the current
// device (CUs x occupancy), 0 on failure.
int valu_pass_capacity(int d);

}  // namespace sk

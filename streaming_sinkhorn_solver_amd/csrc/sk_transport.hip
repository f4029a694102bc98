// sk_transport.hip -- streamed transport products and the pieces of the
// Hessian-vector product, on the vector ALUs (d <= 8).
//
// "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodology 3:
// the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) is applied to vectors and
// matrices by the same streamed, row-stationary traversal as the Sinkhorn
// half-steps, never stored; the Hessian-vector product is assembled from such
// products.
//
// With both clouds packed from their potentials (bias slot h = log2 w +
// log2e (pot - |p~|^2)/eps) the plan entry of query i and key j is
// 2^{s_ij + h_i}, s_ij = <q_i, k_j> + h_j the usual score.  A pass keeps, per
// query row, the running max M of s_ij, the rescaled sum S = sum_j 2^{s_ij - M}
// and the rescaled payload sums Acc = sum_j 2^{s_ij - M} w_ij psi_j, and ends with
// P psi = 2^{M + h_i} Acc and the row mass 2^{M + h_i} S.
//
//  MODE 0: w_ij = 1, psi_j = K payload columns of key j (a strided array: the
//          caller's matrix, or the packed keys themselves for P Y~);
//  MODE 2: psi_j = y~_j (the key's centred coordinates) and the per-pair weight
//          w_ij = pay_j + <y~_j, 2 v_i> with v_i a per-row direction: the last
//          pass of the Hessian-vector product.
//
// The key range may be split across workgroups (a split grid, as in the
// gradient); partial (M, S, Acc) are merged exactly afterwards.
#include "sk_internal.hpp"
#include "sk_pass_common.hpp"

namespace sk {
namespace {

constexpr int kTR = 2;     // query rows per lane
constexpr int kTTL = 256;  // keys per LDS tile
constexpr int kTTJ = 8;    // keys per register chunk

template <int D>
__device__ __forceinline__ void stage_keys(float4* tile, const float4* __restrict__ kp, int base, int c1) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    for (int e = threadIdx.x; e < kTTL * V; e += kBlock) {
        const int col = base + e / V;
        const int part = e % V;
        float4 v;
        if (col < c1) {
            v = kp[(size_t)col * V + part];
        } else {  // past the range: zero coordinates, bias -inf (adds nothing)
            v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (part == D / 4) reinterpret_cast<float*>(&v)[D % 4] = -INFINITY;
        }
        tile[e] = v;
    }
}

template <int D, int K, int MODE>
__global__ __launch_bounds__(kBlock) void k_transport(TransArgs A) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    constexpr int KA = MODE == 0 ? K : D;   // accumulators per row
    constexpr int KL = MODE == 0 ? K : 1;   // payload floats per key in LDS
    __shared__ float4 tile[kTTL * V];
    __shared__ float ptile[kTTL * KL];

    const int split = blockIdx.y;
    const int row0 = blockIdx.x * (kBlock * kTR) + threadIdx.x;

    float q[kTR][D], vd[kTR][D];
    float M[kTR], S[kTR], Acc[kTR][KA];
#pragma unroll
    for (int r = 0; r < kTR; ++r) {
        const int i = row0 + r * kBlock;
        const int ic = i < A.nq ? i : A.nq - 1;
#pragma unroll
        for (int t = 0; t < D; ++t) {
            q[r][t] = A.q[(size_t)ic * P + t] * A.qscale;
            vd[r][t] = MODE == 2 ? 2.0f * A.rowv[(size_t)ic * D + t] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < KA; ++c) Acc[r][c] = 0.0f;
        M[r] = kNegBig;
        S[r] = 0.0f;
    }

    const int c0 = split * A.cols_per_split;
    const int c1 = min(c0 + A.cols_per_split, A.nk);
    const float4* kp = reinterpret_cast<const float4*>(A.k);

    for (int base = c0; base < c1; base += kTTL) {
        __syncthreads();
        stage_keys<D>(tile, kp, base, c1);
        for (int e = threadIdx.x; e < kTTL * KL; e += kBlock) {
            const int col = base + e / KL;
            const int c = e % KL;
            ptile[e] = (col < c1 && c < A.kin) ? A.pay[(size_t)col * A.ldp + c] : 0.0f;
        }
        __syncthreads();
        const int ntile = min(kTTL, c1 - base);
        for (int c = 0; c < ntile; c += kTTJ) {
            float kk[kTTJ][P];
#pragma unroll
            for (int t = 0; t < kTTJ; ++t)
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    const float4 v = tile[(c + t) * V + u];
                    kk[t][4 * u + 0] = v.x;
                    kk[t][4 * u + 1] = v.y;
                    kk[t][4 * u + 2] = v.z;
                    kk[t][4 * u + 3] = v.w;
                }
#pragma unroll
            for (int r = 0; r < kTR; ++r) {
                float s[kTTJ];
#pragma unroll
                for (int t = 0; t < kTTJ; ++t) {
                    float acc = kk[t][D];
#pragma unroll
                    for (int dd = 0; dd < D; ++dd) acc = fmaf(q[r][dd], kk[t][dd], acc);
                    s[t] = acc;
                }
                float mt = s[0];
#pragma unroll
                for (int t = 1; t < kTTJ; ++t) mt = fmaxf(mt, s[t]);
                const float mn = fmaxf(M[r], mt);
                const float sc = ex2(M[r] - mn);
                float sum = S[r] * sc;
#pragma unroll
                for (int cc = 0; cc < KA; ++cc) Acc[r][cc] *= sc;
#pragma unroll
                for (int t = 0; t < kTTJ; ++t) {
                    const float e = ex2(s[t] - mn);
                    sum += e;
                    if (MODE == 0) {
#pragma unroll
                        for (int cc = 0; cc < K; ++cc) Acc[r][cc] = fmaf(e, ptile[(c + t) * KL + cc], Acc[r][cc]);
                    } else {
                        float w = ptile[c + t];
#pragma unroll
                        for (int dd = 0; dd < D; ++dd) w = fmaf(vd[r][dd], kk[t][dd], w);
                        const float ew = e * w;
#pragma unroll
                        for (int dd = 0; dd < D; ++dd) Acc[r][dd] = fmaf(ew, kk[t][dd], Acc[r][dd]);
                    }
                }
                S[r] = sum;
                M[r] = mn;
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kTR; ++r) {
        const int i = row0 + r * kBlock;
        if (i >= A.nq) continue;
        if (A.nsplit == 1) {
            const float scale = ex2(M[r] + A.q[(size_t)i * P + D]);
#pragma unroll
            for (int cc = 0; cc < KA; ++cc)
                if (cc < A.kout) A.out[(size_t)i * A.ldo + cc] = Acc[r][cc] * scale;
            if (A.mass) A.mass[i] = S[r] * scale;
        } else {
            A.part[(size_t)split * A.nq + i] = make_float2(M[r], S[r]);
            float* pa = A.partA + ((size_t)split * A.nq + i) * KA;
#pragma unroll
            for (int cc = 0; cc < KA; ++cc) pa[cc] = Acc[r][cc];
        }
    }
}

// Exact merge of the split partials of each row, then the plan scale.
template <int KA>
__global__ __launch_bounds__(kBlock) void k_transport_merge(TransArgs A) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= A.nq) return;
    float M = kNegBig;
    for (int s = 0; s < A.nsplit; ++s) M = fmaxf(M, A.part[(size_t)s * A.nq + i].x);
    float S = 0.0f, acc[KA];
#pragma unroll
    for (int c = 0; c < KA; ++c) acc[c] = 0.0f;
    for (int s = 0; s < A.nsplit; ++s) {
        const float2 p = A.part[(size_t)s * A.nq + i];
        const float sc = ex2(p.x - M);
        S += p.y * sc;
        const float* pa = A.partA + ((size_t)s * A.nq + i) * KA;
#pragma unroll
        for (int c = 0; c < KA; ++c) acc[c] = fmaf(pa[c], sc, acc[c]);
    }
    const float scale = ex2(M + A.q[(size_t)i * A.P + A.d]);
#pragma unroll
    for (int c = 0; c < KA; ++c)
        if (c < A.kout) A.out[(size_t)i * A.ldo + c] = acc[c] * scale;
    if (A.mass) A.mass[i] = S * scale;
}

template <int D, int K, int MODE>
hipError_t launch_t(const TransArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int KA = MODE == 0 ? K : D;
    const int rpb = kBlock * kTR;
    dim3 grid((a.nq + rpb - 1) / rpb, a.nsplit);
    SK_LAUNCH_TIMED((k_transport<D, K, MODE>), grid, dim3(kBlock), s, ev0, ev1, a);
    if (a.nsplit > 1)
        hipLaunchKernelGGL(k_transport_merge<KA>, dim3((a.nq + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

template <int D, int K, int MODE>
int capacity_t() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_transport<D, K, MODE>, kBlock, 0) != hipSuccess)
        return 0;
    return cus * per_cu;
}

template <int D>
int capacity_t_d(int mode, int kwidth) {
    if (mode == 2) return capacity_t<D, 1, 2>();
    switch (kwidth) {
        case 1: return capacity_t<D, 1, 0>();
        case 4: return capacity_t<D, 4, 0>();
        case 9: return capacity_t<D, 9, 0>();
        default: return 0;
    }
}

template <int D>
hipError_t launch_t_d(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (mode == 2) return launch_t<D, 1, 2>(a, s, ev0, ev1);
    switch (kwidth) {
        case 1: return launch_t<D, 1, 0>(a, s, ev0, ev1);
        case 4: return launch_t<D, 4, 0>(a, s, ev0, ev1);
        case 9: return launch_t<D, 9, 0>(a, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- HVP pieces
// The Hessian-vector product of the entropic cost in x at the plan of (f, g)
// (implicit differentiation, centred coordinates x~, y~):
//   rho_i = 2 (r_i st_i - <A_i, v_i>),  st_i = <x~_i, v_i>,  A = P Y~,  r = P 1,
//   gam_j = 2 (B_j0 - <y~_j, B_j[1..d]>),  B = P^T [st, v],
//   [[diag r, P], [P^T, diag c]] (phi, psi) = (rho, gam)   (preconditioned CG),
//   (H v)_i = 2 r_i v_i - (2/eps) ((phi_i - 2 st_i) A_i + E_i),
//   E_i = sum_j P_ij (psi_j + 2 <y~_j, v_i>) y~_j.

// st, rho and the column payload U = [st, v] (row stride d + 1).
__global__ __launch_bounds__(kBlock) void k_hvp_rows(const float* __restrict__ xp, int P, int d, int n,
                                                     const float* __restrict__ v, const float* __restrict__ A,
                                                     const float* __restrict__ r, float* __restrict__ st,
                                                     float* __restrict__ rho, float* __restrict__ U) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float sx = 0.0f, av = 0.0f;
    for (int t = 0; t < d; ++t) {
        const float vt = v[(size_t)i * d + t];
        sx = fmaf(xp[(size_t)i * P + t], vt, sx);
        av = fmaf(A[(size_t)i * d + t], vt, av);
        U[(size_t)i * (d + 1) + 1 + t] = vt;
    }
    U[(size_t)i * (d + 1)] = sx;
    st[i] = sx;
    rho[i] = 2.0f * (r[i] * sx - av);
}

__global__ __launch_bounds__(kBlock) void k_hvp_cols(const float* __restrict__ yp, int P, int d, int m,
                                                     const float* __restrict__ B, float* __restrict__ gam) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= m) return;
    float yb = 0.0f;
    for (int t = 0; t < d; ++t) yb = fmaf(yp[(size_t)j * P + t], B[(size_t)j * (d + 1) + 1 + t], yb);
    gam[j] = 2.0f * (B[(size_t)j * (d + 1)] - yb);
}

__global__ __launch_bounds__(kBlock) void k_hvp_final(int n, int d, float eps, const float* __restrict__ v,
                                                      const float* __restrict__ r, const float* __restrict__ st,
                                                      const float* __restrict__ phi, const float* __restrict__ A,
                                                      const float* __restrict__ E, float* __restrict__ out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float c = phi[i] - 2.0f * st[i];
    const float k2 = 2.0f / eps;
    for (int t = 0; t < d; ++t) {
        const size_t e = (size_t)i * d + t;
        out[e] = 2.0f * r[i] * v[e] - k2 * fmaf(c, A[e], E[e]);
    }
}

// Preconditioned conjugate gradients on K z = rhs, K = [[diag r, P], [P^T, diag c]],
// preconditioner diag(r, c)^-1, over N = n + m unknowns, all in one workgroup
// (float64 dot products, fixed order).  K is singular along the gauge
// direction e = (1_n, -1_m) (K e = (r - P 1, P^T 1 - c) = 0); the right-hand
// side is consistent in exact arithmetic, but float32 products are not exactly
// symmetric, so the residual is projected onto the complement of e at every
// step (keeping the iterates from wandering along e), and the iterate with the
// smallest residual so far is kept in zb: steps past convergence, where the
// step sizes are made of rounding noise, cannot spoil the result.
// scal: [0] rz = <res, D^-1 res>, [1] rz at the start, [2] smallest rz so far.
// Each step reads Kp = diag * p + (P p_psi ; P^T p_phi), the two streamed
// products being in prod (n + m floats), computed from the current p.
__device__ inline double wg_sum(double v, double* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (t < w) sh[t] += sh[t + w];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

// The CG kernels run in one workgroup: unrolling each strided loop by 8 keeps
// eight elements' loads in flight per thread instead of one (each thread still
// takes its elements, and sums them, in the same order).
#define CG_UNROLL _Pragma("unroll 8")

// res <- res - (<res, e> / N) e, then p = D^-1 res (init) and rz.
__device__ inline double project_and_precondition(int N, int n, const float* __restrict__ diag, float* __restrict__ res,
                                                  float* __restrict__ pre_out, double* sh) {
    double re = 0.0;
    CG_UNROLL
    for (int k = threadIdx.x; k < N; k += blockDim.x) re += k < n ? (double)res[k] : -(double)res[k];
    re = wg_sum(re, sh);
    const float mu = (float)(re / N);
    double rz = 0.0;
    CG_UNROLL
    for (int k = threadIdx.x; k < N; k += blockDim.x) {
        const float rk = res[k] - (k < n ? mu : -mu);
        res[k] = rk;
        const float dk = diag[k];
        const float pre = dk > 0.0f ? rk / dk : 0.0f;
        if (pre_out) pre_out[k] = pre;
        rz += (double)rk * (double)pre;
    }
    return wg_sum(rz, sh);
}

__global__ __launch_bounds__(1024) void k_cg_init(int N, int n, const float* __restrict__ diag,
                                                  const float* __restrict__ rhs, float* __restrict__ z,
                                                  float* __restrict__ zb, float* __restrict__ res,
                                                  float* __restrict__ p, double* __restrict__ scal) {
    __shared__ double sh[1024];
    CG_UNROLL
    for (int k = threadIdx.x; k < N; k += blockDim.x) {
        z[k] = 0.0f;
        zb[k] = 0.0f;
        res[k] = rhs[k];
    }
    __syncthreads();
    const double rz = project_and_precondition(N, n, diag, res, p, sh);
    if (threadIdx.x == 0) {
        scal[0] = rz;
        scal[1] = rz;
        scal[2] = rz;
        scal[3] = rz;
    }
}

// One CG step in four kernels over kCgBlocks workgroups (a single workgroup
// is bound by one CU's bandwidth: 57 us per step at N = 32,768, 159 us at
// 100,000).  Each kernel writes one partial per workgroup, and every
// workgroup of the next reduces all of them with the same fixed tree, so the
// scalars are bit-identical across workgroups and runs.  scal: [0] rz,
// [1] rz at the start, [2] the best rz so far, [3] the step's new rz (committed
// into [0] and [2] by the next step's first kernel, which reads neither),
// [4 ..] the partials.
static_assert(kCgBlocks <= kBlock, "a workgroup reduces all partials in one pass");
__device__ inline double cg_total(const double* part, double* sh) {
    return wg_sum(threadIdx.x < kCgBlocks ? part[threadIdx.x] : 0.0, sh);
}

// Commit the previous step's rz, then <p, K p> per workgroup.
__global__ __launch_bounds__(kBlock) void k_cg_a(int N, const float* __restrict__ diag, const float* __restrict__ prod,
                                                 const float* __restrict__ p, double* __restrict__ scal) {
    __shared__ double sh[kBlock];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const double rzn = scal[3];
        if (rzn < scal[2]) scal[2] = rzn;
        scal[0] = rzn;
    }
    double pkp = 0.0;
    CG_UNROLL
    for (int k = blockIdx.x * kBlock + threadIdx.x; k < N; k += kCgBlocks * kBlock) {
        const float kp = fmaf(diag[k], p[k], prod[k]);
        pkp += (double)p[k] * (double)kp;
    }
    pkp = wg_sum(pkp, sh);
    if (threadIdx.x == 0) scal[4 + blockIdx.x] = pkp;
}

// z += alpha p, res -= alpha K p, then <res, e> per workgroup (e = +1 on the
// first n entries, -1 on the rest).
__global__ __launch_bounds__(kBlock) void k_cg_b(int N, int n, const float* __restrict__ diag,
                                                 const float* __restrict__ prod, const float* __restrict__ p,
                                                 float* __restrict__ z, float* __restrict__ res,
                                                 double* __restrict__ scal) {
    __shared__ double sh[kBlock];
    const double pkp = cg_total(scal + 4, sh);
    const double rz = scal[0];
    const float alpha = (pkp > 0.0 && rz > 0.0) ? (float)(rz / pkp) : 0.0f;
    double re = 0.0;
    CG_UNROLL
    for (int k = blockIdx.x * kBlock + threadIdx.x; k < N; k += kCgBlocks * kBlock) {
        const float kp = fmaf(diag[k], p[k], prod[k]);
        z[k] = fmaf(alpha, p[k], z[k]);
        const float r = fmaf(-alpha, kp, res[k]);
        res[k] = r;
        re += k < n ? (double)r : -(double)r;
    }
    re = wg_sum(re, sh);
    if (threadIdx.x == 0) scal[4 + kCgBlocks + blockIdx.x] = re;
}

// res <- res - (<res, e> / N) e, then <res, D^-1 res> per workgroup.
__global__ __launch_bounds__(kBlock) void k_cg_c(int N, int n, const float* __restrict__ diag, float* __restrict__ res,
                                                 double* __restrict__ scal) {
    __shared__ double sh[kBlock];
    const float mu = (float)(cg_total(scal + 4 + kCgBlocks, sh) / N);
    double rz = 0.0;
    CG_UNROLL
    for (int k = blockIdx.x * kBlock + threadIdx.x; k < N; k += kCgBlocks * kBlock) {
        const float rk = res[k] - (k < n ? mu : -mu);
        res[k] = rk;
        const float dk = diag[k];
        const float pre = dk > 0.0f ? rk / dk : 0.0f;
        rz += (double)rk * (double)pre;
    }
    rz = wg_sum(rz, sh);
    if (threadIdx.x == 0) scal[4 + 2 * kCgBlocks + blockIdx.x] = rz;
}

// p <- D^-1 res + beta p, keep z if this step's rz is the best so far, and
// leave the new rz in scal[3].
__global__ __launch_bounds__(kBlock) void k_cg_d(int N, const float* __restrict__ diag, const float* __restrict__ res,
                                                 const float* __restrict__ z, float* __restrict__ p,
                                                 float* __restrict__ zb, double* __restrict__ scal) {
    __shared__ double sh[kBlock];
    const double rz_new = cg_total(scal + 4 + 2 * kCgBlocks, sh);
    const double rz = scal[0];
    const float beta = rz > 0.0 ? (float)(rz_new / rz) : 0.0f;
    const bool best = rz_new < scal[2];
    CG_UNROLL
    for (int k = blockIdx.x * kBlock + threadIdx.x; k < N; k += kCgBlocks * kBlock) {
        const float dk = diag[k];
        const float pre = dk > 0.0f ? res[k] / dk : 0.0f;
        p[k] = fmaf(beta, p[k], pre);
    }
    if (best) {  // the same in every workgroup
        CG_UNROLL
        for (int k = blockIdx.x * kBlock + threadIdx.x; k < N; k += kCgBlocks * kBlock) zb[k] = z[k];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) scal[3] = rz_new;
}

// sqrt(rz_best / rz0): the preconditioned residual of the kept iterate relative to the start.
// The last step's rz is still pending in scal[3].
__global__ void k_cg_report(const double* __restrict__ scal, float* __restrict__ out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const double best = scal[3] < scal[2] ? scal[3] : scal[2];
        out[0] = scal[1] > 0.0 ? (float)sqrt(fmax(best, 0.0) / scal[1]) : 0.0f;
    }
}

inline int grid_of(int64_t count) { return (int)((count + kBlock - 1) / kBlock); }

}  // namespace

int transport_rows_per_block() { return kBlock * kTR; }

int transport_capacity(int d, int mode, int kwidth) {
    switch (d) {
        case 1: return capacity_t_d<1>(mode, kwidth);
        case 2: return capacity_t_d<2>(mode, kwidth);
        case 3: return capacity_t_d<3>(mode, kwidth);
        case 4: return capacity_t_d<4>(mode, kwidth);
        case 5: return capacity_t_d<5>(mode, kwidth);
        case 6: return capacity_t_d<6>(mode, kwidth);
        case 7: return capacity_t_d<7>(mode, kwidth);
        case 8: return capacity_t_d<8>(mode, kwidth);
        default: return 0;
    }
}

hipError_t launch_transport(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (a.d) {
        case 1: return launch_t_d<1>(a, mode, kwidth, s, ev0, ev1);
        case 2: return launch_t_d<2>(a, mode, kwidth, s, ev0, ev1);
        case 3: return launch_t_d<3>(a, mode, kwidth, s, ev0, ev1);
        case 4: return launch_t_d<4>(a, mode, kwidth, s, ev0, ev1);
        case 5: return launch_t_d<5>(a, mode, kwidth, s, ev0, ev1);
        case 6: return launch_t_d<6>(a, mode, kwidth, s, ev0, ev1);
        case 7: return launch_t_d<7>(a, mode, kwidth, s, ev0, ev1);
        case 8: return launch_t_d<8>(a, mode, kwidth, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_hvp_rows(const float* xp, int P, int d, int n, const float* v, const float* A, const float* r,
                           float* st, float* rho, float* U, hipStream_t s) {
    hipLaunchKernelGGL(k_hvp_rows, dim3(grid_of(n)), dim3(kBlock), 0, s, xp, P, d, n, v, A, r, st, rho, U);
    return hipGetLastError();
}

hipError_t launch_hvp_cols(const float* yp, int P, int d, int m, const float* B, float* gam, hipStream_t s) {
    hipLaunchKernelGGL(k_hvp_cols, dim3(grid_of(m)), dim3(kBlock), 0, s, yp, P, d, m, B, gam);
    return hipGetLastError();
}

hipError_t launch_hvp_final(int n, int d, float eps, const float* v, const float* r, const float* st,
                            const float* phi, const float* A, const float* E, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_hvp_final, dim3(grid_of(n)), dim3(kBlock), 0, s, n, d, eps, v, r, st, phi, A, E, out);
    return hipGetLastError();
}

hipError_t launch_cg_init(int N, int n, const float* diag, const float* rhs, float* z, float* zb, float* res, float* p,
                          double* scal, hipStream_t s) {
    hipLaunchKernelGGL(k_cg_init, dim3(1), dim3(1024), 0, s, N, n, diag, rhs, z, zb, res, p, scal);
    return hipGetLastError();
}

hipError_t launch_cg_step(int N, int n, const float* diag, const float* prod, float* z, float* zb, float* res, float* p,
                          double* scal, hipStream_t s) {
    hipLaunchKernelGGL(k_cg_a, dim3(kCgBlocks), dim3(kBlock), 0, s, N, diag, prod, p, scal);
    hipLaunchKernelGGL(k_cg_b, dim3(kCgBlocks), dim3(kBlock), 0, s, N, n, diag, prod, p, z, res, scal);
    hipLaunchKernelGGL(k_cg_c, dim3(kCgBlocks), dim3(kBlock), 0, s, N, n, diag, res, scal);
    hipLaunchKernelGGL(k_cg_d, dim3(kCgBlocks), dim3(kBlock), 0, s, N, diag, res, z, p, zb, scal);
    return hipGetLastError();
}

hipError_t launch_cg_report(const double* scal, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_cg_report, dim3(1), dim3(64), 0, s, scal, out);
    return hipGetLastError();
}

}  // namespace sk

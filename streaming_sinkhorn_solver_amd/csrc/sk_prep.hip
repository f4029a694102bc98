// sk_prep.hip -- once-per-call preparation and the small deterministic reductions:
// common centre, packing of the clouds with norms and log-weights, data checks,
// the dual cost, the residual max / sum, the state-to-bias and state-to-potential
// maps of the stop rules and blended updates, and the potential-change check.
//
// Every reduction is two-stage with a fixed partition (kRedBlocks partials, or
// one workgroup walking the data in a fixed order) and a fixed-order final
// sum, so results are bit-identical from run to run.
#include "sk_internal.hpp"

#include <algorithm>

#include <cmath>

namespace sk {
namespace {

__device__ inline double block_sum_f64(double v, double* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (t < w) sh[t] += sh[t + w];
        __syncthreads();
    }
    double r = sh[0];
    __syncthreads();
    return r;
}

// Maximum that propagates NaN (fmaxf returns the other operand): a check value
// read from a NaN state must not look like a met tolerance.
__device__ __forceinline__ float max_nan(float a, float b) { return (a != a || b != b) ? a + b : fmaxf(a, b); }

__device__ inline float block_max_f32(float v, float* sh) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (t < w) sh[t] = max_nan(sh[t], sh[t + w]);
        __syncthreads();
    }
    float r = sh[0];
    __syncthreads();
    return r;
}

// Per-block column sums of a (npts, d) cloud in float64.  Thread t < span owns
// coordinate t % d and walks the flat array with stride span (a multiple of d),
// so loads stay contiguous across threads.
__global__ __launch_bounds__(kBlock) void k_colsum_partial(const float* __restrict__ pts, int64_t total,
                                                           int d, double* __restrict__ partial) {
    __shared__ double sh[kBlock];
    const int span = (kBlock / d) * d;
    const int t = threadIdx.x;
    const int64_t per_block = ((total + gridDim.x - 1) / gridDim.x + d - 1) / d * d;
    const int64_t lo = (int64_t)blockIdx.x * per_block;
    const int64_t hi = lo + per_block < total ? lo + per_block : total;
    double acc = 0.0;
    if (t < span)
        for (int64_t e = lo + t; e < hi; e += span) acc += (double)pts[e];
    sh[t] = acc;
    __syncthreads();
    if (t < d) {
        double s = 0.0;
        for (int u = t; u < span; u += d) s += sh[u];
        partial[(size_t)blockIdx.x * d + t] = s;
    }
}

// One workgroup per coordinate t: the partial sums of each cloud joined by a
// fixed-shape tree (deterministic), then c_t = (mean_x + mean_y) / 2.
__global__ __launch_bounds__(kBlock) void k_centre_final(const double* __restrict__ px, int nbx,
                                                         const double* __restrict__ py, int nby, int d,
                                                         int n, int m, float* __restrict__ centre) {
    __shared__ double sh[kBlock];
    const int t = blockIdx.x;
    double sx = 0.0, sy = 0.0;
    for (int b = threadIdx.x; b < nbx; b += blockDim.x) sx += px[(size_t)b * d + t];
    for (int b = threadIdx.x; b < nby; b += blockDim.x) sy += py[(size_t)b * d + t];
    sx = block_sum_f64(sx, sh);
    sy = block_sum_f64(sy, sh);
    if (threadIdx.x == 0) centre[t] = (float)(0.5 * (sx / n + sy / m));
}

// Pack one cloud: centred coordinates, zero padding, |p~|^2, log2 w and the
// initial bias.  bias_mode: 0 = none (0), 1 = zero potential, 2 = from pot.
// u_out (may be null) receives the state u = (|p~|^2 - pot) log2e / eps that
// the bias encodes (h = log2 w - u); 0 for bias_mode 0.
__global__ __launch_bounds__(kBlock) void k_pack(const float* __restrict__ pts, int npts, int d, int P,
                                                 int mfma, const float* __restrict__ centre,
                                                 const float* __restrict__ w, float* __restrict__ packed,
                                                 float* __restrict__ nrm, float* __restrict__ l2w,
                                                 float* __restrict__ bias_sep, float inv_eps, int bias_mode,
                                                 const float* __restrict__ pot, float* __restrict__ u_out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= npts) return;
    float s = 0.0f;
    float* row = packed + (size_t)i * P;
    for (int t = 0; t < d; ++t) {
        float v = pts[(size_t)i * d + t] - centre[t];
        row[t] = v;
        s = fmaf(v, v, s);
    }
    for (int t = d; t < P; ++t) row[t] = 0.0f;
    const float wi = w[i];
    const float lw = wi > 0.0f ? log2f(wi) : -INFINITY;
    nrm[i] = s;
    l2w[i] = lw;
    float u = 0.0f;
    if (bias_mode == 1) u = s * kLog2e * inv_eps;
    if (bias_mode == 2) u = (s - pot[i]) * kLog2e * inv_eps;
    const float h = bias_mode == 0 ? 0.0f : lw - u;
    if (u_out) u_out[i] = u;
    if (mfma)
        bias_sep[i] = h;
    else
        row[d] = h;
}

__global__ __launch_bounds__(kBlock) void k_fill(float* __restrict__ p, int64_t count, float v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = v;
}

// Key bias of both clouds from their states: threads [0, x.npts) serve x, the rest y.
__global__ __launch_bounds__(kBlock) void k_apply_bias(BiasSide x, BiasSide y, int P, int d) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    const BiasSide& S = i < x.npts ? x : y;
    if (i >= x.npts) i -= x.npts;
    if (i >= S.npts) return;
    const float h = S.l2w[i] - S.u[i];
    if (S.sep)
        S.sep[i] = h;
    else
        S.packed[(size_t)i * P + d] = h;
}

// Potential of a stored state; the same expression as the pass epilogue.
__global__ __launch_bounds__(kBlock) void k_pot_from_state(const float* __restrict__ u,
                                                           const float* __restrict__ nrm, float eps_ln2,
                                                           float* __restrict__ pot, int npts) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < npts) pot[i] = nrm[i] - eps_ln2 * u[i];
}

// v <- v + alpha * u (the descent step of the gradient flow).
__global__ __launch_bounds__(kBlock) void k_axpy(float* __restrict__ v, const float* __restrict__ u, int64_t count,
                                                 float alpha) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) v[i] += alpha * u[i];
}

// Data checks of one flat array: [nonfinite flag, negative flag, float64 sum].
__global__ __launch_bounds__(kBlock) void k_check_partial(const float* __restrict__ v, int64_t total,
                                                          double* __restrict__ partial) {
    __shared__ double sh[kBlock];
    const int64_t per_block = (total + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per_block;
    const int64_t hi = lo + per_block < total ? lo + per_block : total;
    double bad = 0.0, neg = 0.0, sum = 0.0;
    for (int64_t e = lo + threadIdx.x; e < hi; e += blockDim.x) {
        float x = v[e];
        if (!isfinite(x)) bad = 1.0;
        if (x < 0.0f) neg = 1.0;
        sum += (double)x;
    }
    bad = block_sum_f64(bad, sh);
    neg = block_sum_f64(neg, sh);
    sum = block_sum_f64(sum, sh);
    if (threadIdx.x == 0) {
        partial[3 * blockIdx.x + 0] = bad;
        partial[3 * blockIdx.x + 1] = neg;
        partial[3 * blockIdx.x + 2] = sum;
    }
}

// result: [nonfinite, negative weight, sum a, sum b]; partials holds 4 arrays x, y, a, b.
// One workgroup: each thread folds a fixed stride of the 4 nblk partial records, then fixed-order trees.
__global__ __launch_bounds__(kBlock) void k_check_final(const double* __restrict__ partial, int nblk,
                                                        double* __restrict__ result) {
    __shared__ double sh[kBlock];
    double bad = 0.0, neg = 0.0, sa = 0.0, sb = 0.0;
    for (int e = threadIdx.x; e < 4 * nblk; e += blockDim.x) {
        const int arr = e / nblk;
        const double* p = partial + (size_t)e * 3;
        bad += p[0];
        if (arr >= 2) neg += p[1];
        if (arr == 2) sa += p[2];
        if (arr == 3) sb += p[2];
    }
    bad = block_sum_f64(bad, sh);
    neg = block_sum_f64(neg, sh);
    sa = block_sum_f64(sa, sh);
    sb = block_sum_f64(sb, sh);
    if (threadIdx.x == 0) {
        result[0] = bad;
        result[1] = neg;
        result[2] = sa;
        result[3] = sb;
    }
}

// Elements a thread of the single-workgroup reductions loads before it folds
// them in: their loads are in flight together instead of one latency each.
constexpr int kRedUnroll = 8;

// Cost: one workgroup walks both vectors in a fixed order with float64 sums.
// With `mass` (per-row plan sums) the plan mass is their sum; without it the
// potentials are taken to come out of a column half-step, whose plan mass is sum(b).
__global__ __launch_bounds__(1024) void k_cost(const float* __restrict__ a, const float* __restrict__ b,
                                               const float* __restrict__ f, const float* __restrict__ g,
                                               const float* __restrict__ mass, int n, int m, float eps,
                                               double* __restrict__ out) {
    __shared__ double sh[1024];
    double af = 0.0, sa = 0.0, bg = 0.0, sb = 0.0, mp = 0.0;
    const int T = blockDim.x;
    int i = threadIdx.x;
    // kRedUnroll elements per thread in flight at once, summed in the same order as one at a time
    for (; i + (kRedUnroll - 1) * T < n; i += kRedUnroll * T) {
        float av[kRedUnroll], fv[kRedUnroll], mv[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            av[k] = a[i + k * T];
            fv[k] = f[i + k * T];
            mv[k] = mass ? mass[i + k * T] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            if (av[k] != 0.0f) af += (double)av[k] * (double)fv[k];
            sa += (double)av[k];
            if (mass) mp += (double)mv[k];
        }
    }
    for (; i < n; i += T) {
        float ai = a[i];
        if (ai != 0.0f) af += (double)ai * (double)f[i];
        sa += (double)ai;
        if (mass) mp += (double)mass[i];
    }
    int j = threadIdx.x;
    for (; j + (kRedUnroll - 1) * T < m; j += kRedUnroll * T) {
        float bv[kRedUnroll], gv[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            bv[k] = b[j + k * T];
            gv[k] = g[j + k * T];
        }
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            if (bv[k] != 0.0f) bg += (double)bv[k] * (double)gv[k];
            sb += (double)bv[k];
        }
    }
    for (; j < m; j += T) {
        float bj = b[j];
        if (bj != 0.0f) bg += (double)bj * (double)g[j];
        sb += (double)bj;
    }
    af = block_sum_f64(af, sh);
    sa = block_sum_f64(sa, sh);
    bg = block_sum_f64(bg, sh);
    sb = block_sum_f64(sb, sh);
    if (mass) mp = block_sum_f64(mp, sh);
    if (threadIdx.x == 0)
        out[0] = mass ? af + bg - (double)eps * (mp - sa * sb) : af + bg - (double)eps * sb * (1.0 - sa);
}

// Payload of the plan's transport cost: U_j = [y~_j (d values), |y~_j|^2], from the packed cloud.
__global__ __launch_bounds__(kBlock) void k_primal_payload(const float* __restrict__ yp, int P, int d,
                                                           const float* __restrict__ ny, int m,
                                                           float* __restrict__ U) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= m) return;
    float* u = U + (size_t)j * (d + 1);
    for (int t = 0; t < d; ++t) u[t] = yp[(size_t)j * P + t];
    u[d] = ny[j];
}

// Primal value of the plan P_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) from its row sums r, column sums c
// and per-row sums T_i = [sum_j P_ij y~_j, sum_j P_ij |y~_j|^2] (centred coordinates; C is unchanged by the
// common shift).  With log(P_ij / (a_i b_j)) = (f_i + g_j - C_ij)/eps the generalised KL term collapses:
//   out[0] = <P,C> + eps KL(P | a x b) = sum_i f_i r_i + sum_j g_j c_j - eps (sum_i r_i - sum(a) sum(b)),
//   out[1] = <P,C> = sum_i (r_i |x~_i|^2 - 2 <x~_i, T_i> + T_i[d]).
// Each row's term of out[1] is formed by one thread per row over the whole grid (k_primal_rows, the
// coordinates in order); one workgroup then takes all the float64 sums in a fixed order (k_primal). Rows
// and columns of zero weight carry no plan mass.
__global__ __launch_bounds__(kBlock) void k_primal_rows(const float* __restrict__ a, const float* __restrict__ r,
                                                        const float* __restrict__ xp, int P, int d,
                                                        const float* __restrict__ nx, const float* __restrict__ T,
                                                        int n, double* __restrict__ pv) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    if (a[i] == 0.0f) {
        pv[i] = 0.0;
        return;
    }
    const double ri = (double)r[i];
    const float* t = T + (size_t)i * (d + 1);
    double dot = 0.0;
    for (int k = 0; k < d; ++k) dot += (double)xp[(size_t)i * P + k] * (double)t[k];
    pv[i] = ri * (double)nx[i] - 2.0 * dot + (double)t[d];
}

__global__ __launch_bounds__(1024) void k_primal(const float* __restrict__ a, const float* __restrict__ b,
                                                 const float* __restrict__ f, const float* __restrict__ g,
                                                 const float* __restrict__ r, const float* __restrict__ c,
                                                 const double* __restrict__ pv, int n, int m, float eps,
                                                 double* __restrict__ out) {
    __shared__ double sh[1024];
    double fr = 0.0, gc = 0.0, mp = 0.0, sa = 0.0, sb = 0.0, pc = 0.0;
    const int T = blockDim.x;
    int i = threadIdx.x;
    for (; i + (kRedUnroll - 1) * T < n; i += kRedUnroll * T) {
        float av[kRedUnroll], rv[kRedUnroll], fv[kRedUnroll];
        double pw[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            av[k] = a[i + k * T];
            rv[k] = r[i + k * T];
            fv[k] = f[i + k * T];
            pw[k] = pv[i + k * T];
        }
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            sa += (double)av[k];
            if (av[k] == 0.0f) continue;
            fr += (double)fv[k] * (double)rv[k];
            mp += (double)rv[k];
            pc += pw[k];
        }
    }
    for (; i < n; i += T) {
        const float ai = a[i];
        sa += (double)ai;
        if (ai == 0.0f) continue;
        const double ri = (double)r[i];
        fr += (double)f[i] * ri;
        mp += ri;
        pc += pv[i];
    }
    int j = threadIdx.x;
    for (; j + (kRedUnroll - 1) * T < m; j += kRedUnroll * T) {
        float bv[kRedUnroll], gv[kRedUnroll], cv[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            bv[k] = b[j + k * T];
            gv[k] = g[j + k * T];
            cv[k] = c[j + k * T];
        }
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            sb += (double)bv[k];
            if (bv[k] != 0.0f) gc += (double)gv[k] * (double)cv[k];
        }
    }
    for (; j < m; j += T) {
        const float bj = b[j];
        sb += (double)bj;
        if (bj != 0.0f) gc += (double)g[j] * (double)c[j];
    }
    fr = block_sum_f64(fr, sh);
    gc = block_sum_f64(gc, sh);
    mp = block_sum_f64(mp, sh);
    sa = block_sum_f64(sa, sh);
    sb = block_sum_f64(sb, sh);
    pc = block_sum_f64(pc, sh);
    if (threadIdx.x == 0) {
        out[0] = fr + gc - (double)eps * (mp - sa * sb);
        out[1] = pc;
    }
}

// Largest change of the potentials since the snapshot, then the snapshot is refreshed.
// A check value may go to host memory: then `flag` (may be null) is set to
// `seq` after it, behind a system-scope fence, so a host that sees the flag
// sees the value.
__device__ inline void publish(float* out, float v, int* flag, int seq) {
    out[0] = v;
    if (flag) {
        __threadfence_system();
        reinterpret_cast<volatile int*>(flag)[0] = seq;
    }
}

__global__ __launch_bounds__(1024) void k_pot_change(const float* __restrict__ f, float* __restrict__ sf, int n,
                                                     const float* __restrict__ g, float* __restrict__ sg, int m,
                                                     float* __restrict__ out, int* flag, int seq) {
    __shared__ float shf[1024];
    float mx = 0.0f;
    const int T = blockDim.x;
    // each side: kRedUnroll elements per thread loaded at once (a max does not depend on the order)
    for (int side = 0; side < 2; ++side) {
        const float* __restrict__ v = side ? g : f;
        float* __restrict__ sv = side ? sg : sf;
        const int cnt = side ? m : n;
        int i = threadIdx.x;
        for (; i + (kRedUnroll - 1) * T < cnt; i += kRedUnroll * T) {
            float cur[kRedUnroll], old[kRedUnroll];
#pragma unroll
            for (int k = 0; k < kRedUnroll; ++k) {
                cur[k] = v[i + k * T];
                old[k] = sv[i + k * T];
            }
#pragma unroll
            for (int k = 0; k < kRedUnroll; ++k) {
                mx = max_nan(mx, fabsf(cur[k] - old[k]));
                sv[i + k * T] = cur[k];
            }
        }
        for (; i < cnt; i += T) {
            const float c = v[i];
            mx = max_nan(mx, fabsf(c - sv[i]));
            sv[i] = c;
        }
    }
    mx = block_max_f32(mx, shf);
    if (threadIdx.x == 0) publish(out, mx, flag, seq);
}

__global__ void k_div_combine(double* out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) out[0] = out[1] - 0.5 * out[2] - 0.5 * out[3];
}

// Residual reduction: max and float64 sum of |r_i|.
__global__ __launch_bounds__(1024) void k_resid_reduce(const float* __restrict__ r, int cnt,
                                                       float* __restrict__ out_max,
                                                       float* __restrict__ out_sum, int* flag, int seq) {
    __shared__ double sh[1024];
    __shared__ float shf[1024];
    float mx = 0.0f;
    double sm = 0.0;
    const int T = blockDim.x;
    int i = threadIdx.x;
    for (; i + (kRedUnroll - 1) * T < cnt; i += kRedUnroll * T) {
        float v[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) v[k] = r[i + k * T];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) {
            mx = max_nan(mx, v[k]);
            sm += (double)v[k];
        }
    }
    for (; i < cnt; i += T) {
        float v = r[i];
        mx = max_nan(mx, v);
        sm += (double)v;
    }
    mx = block_max_f32(mx, shf);
    sm = block_sum_f64(sm, sh);
    if (threadIdx.x == 0) {
        if (out_sum) out_sum[0] = (float)sm;
        publish(out_max, mx, flag, seq);
    }
}

// Maximum of v[0..cnt), -inf when cnt == 0, NaN if any v is NaN (one workgroup): lane maxima, then
// a shuffle tree per wave and one more across the waves (max is exact in any order).
__global__ __launch_bounds__(1024) void k_max_reduce(const float* __restrict__ v, int cnt, float* __restrict__ out,
                                                     int* flag, int seq) {
    __shared__ float shw[16];
    float mx = -INFINITY;
    const int T = blockDim.x;
    int i = threadIdx.x;
    for (; i + (kRedUnroll - 1) * T < cnt; i += kRedUnroll * T) {
        float w[kRedUnroll];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) w[k] = v[i + k * T];
#pragma unroll
        for (int k = 0; k < kRedUnroll; ++k) mx = max_nan(mx, w[k]);
    }
    for (; i < cnt; i += T) mx = max_nan(mx, v[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max_nan(mx, __shfl_xor(mx, off));
    const int wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    if ((threadIdx.x & 63) == 0) shw[wave] = mx;
    __syncthreads();
    if (threadIdx.x < 64) {
        mx = threadIdx.x < nw ? shw[threadIdx.x] : -INFINITY;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = max_nan(mx, __shfl_xor(mx, off));
        if (threadIdx.x == 0) publish(out, mx, flag, seq);
    }
}

inline int grid_for(int64_t count, int block) { return (int)((count + block - 1) / block); }

}  // namespace

hipError_t launch_centre(const float* x, const float* y, int n, int m, int d, double* partials,
                         float* centre, hipStream_t s) {
    double* px = partials;
    double* py = partials + (size_t)kRedBlocks * d;
    // partial sums: as many workgroups as give each about 8 elements per thread, at most kRedBlocks
    auto blocks = [](int64_t total) {
        return (int)std::min<int64_t>(kRedBlocks, std::max<int64_t>(1, (total + 8 * kBlock - 1) / (8 * kBlock)));
    };
    const int nbx = blocks((int64_t)n * d), nby = blocks((int64_t)m * d);
    hipLaunchKernelGGL(k_colsum_partial, dim3(nbx), dim3(kBlock), 0, s, x, (int64_t)n * d, d, px);
    hipLaunchKernelGGL(k_colsum_partial, dim3(nby), dim3(kBlock), 0, s, y, (int64_t)m * d, d, py);
    hipLaunchKernelGGL(k_centre_final, dim3(d), dim3(kBlock), 0, s, px, nbx, py, nby, d, n, m, centre);
    return hipGetLastError();
}

hipError_t launch_pack(const float* pts, int npts, int d, int P, bool mfma, const float* centre,
                       const float* w, float* packed, float* nrm, float* l2w, float* bias_sep,
                       float inv_eps, int bias_mode, const float* pot, float* u_out, hipStream_t s) {
    hipLaunchKernelGGL(k_pack, dim3(grid_for(npts, kBlock)), dim3(kBlock), 0, s, pts, npts, d, P,
                       mfma ? 1 : 0, centre, w, packed, nrm, l2w, bias_sep, inv_eps, bias_mode, pot, u_out);
    return hipGetLastError();
}

hipError_t launch_apply_bias(const BiasSide& x, const BiasSide& y, int P, int d, hipStream_t s) {
    hipLaunchKernelGGL(k_apply_bias, dim3(grid_for((int64_t)x.npts + y.npts, kBlock)), dim3(kBlock), 0, s, x, y,
                       P, d);
    return hipGetLastError();
}

hipError_t launch_pot_from_state(const float* u, const float* nrm, float eps_ln2, float* pot, int npts,
                                 hipStream_t s) {
    hipLaunchKernelGGL(k_pot_from_state, dim3(grid_for(npts, kBlock)), dim3(kBlock), 0, s, u, nrm, eps_ln2, pot,
                       npts);
    return hipGetLastError();
}

hipError_t launch_pot_change(const float* f, float* sf, int n, const float* g, float* sg, int m, float* out,
                             hipStream_t s, int* flag, int seq) {
    hipLaunchKernelGGL(k_pot_change, dim3(1), dim3(1024), 0, s, f, sf, n, g, sg, m, out, flag, seq);
    return hipGetLastError();
}

hipError_t launch_cost_mass(const float* a, const float* b, const float* f, const float* g, const float* mass,
                            int n, int m, float eps, double* out, hipStream_t s) {
    hipLaunchKernelGGL(k_cost, dim3(1), dim3(1024), 0, s, a, b, f, g, mass, n, m, eps, out);
    return hipGetLastError();
}

hipError_t launch_primal_payload(const float* yp, int P, int d, const float* ny, int m, float* U, hipStream_t s) {
    hipLaunchKernelGGL(k_primal_payload, dim3(grid_for(m, kBlock)), dim3(kBlock), 0, s, yp, P, d, ny, m, U);
    return hipGetLastError();
}

hipError_t launch_primal(const float* a, const float* b, const float* f, const float* g, const float* r,
                         const float* c, const float* xp, int P, int d, const float* nx, const float* T, int n,
                         int m, float eps, double* pv, double* out, hipStream_t s) {
    hipLaunchKernelGGL(k_primal_rows, dim3(grid_for(n, kBlock)), dim3(kBlock), 0, s, a, r, xp, P, d, nx, T, n, pv);
    hipLaunchKernelGGL(k_primal, dim3(1), dim3(1024), 0, s, a, b, f, g, r, c, pv, n, m, eps, out);
    return hipGetLastError();
}

hipError_t launch_axpy(float* v, const float* u, int64_t count, float alpha, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_axpy, dim3(grid_for(count, kBlock)), dim3(kBlock), 0, s, v, u, count, alpha);
    return hipGetLastError();
}

hipError_t launch_div_combine(double* out, hipStream_t s) {
    hipLaunchKernelGGL(k_div_combine, dim3(1), dim3(64), 0, s, out);
    return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t count, float value, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill, dim3(grid_for(count, kBlock)), dim3(kBlock), 0, s, p, count, value);
    return hipGetLastError();
}

hipError_t launch_check(const float* x, const float* y, const float* a, const float* b, int n, int m,
                        int d, double* partials, double* result, hipStream_t s) {
    const float* arrs[4] = {x, y, a, b};
    const int64_t lens[4] = {(int64_t)n * d, (int64_t)m * d, n, m};
    for (int k = 0; k < 4; ++k)
        hipLaunchKernelGGL(k_check_partial, dim3(kRedBlocks), dim3(kBlock), 0, s, arrs[k], lens[k],
                           partials + (size_t)k * kRedBlocks * 3);
    hipLaunchKernelGGL(k_check_final, dim3(1), dim3(kBlock), 0, s, partials, kRedBlocks, result);
    return hipGetLastError();
}

hipError_t launch_cost(const float* a, const float* b, const float* f, const float* g, int n, int m,
                       float eps, double* out, hipStream_t s) {
    hipLaunchKernelGGL(k_cost, dim3(1), dim3(1024), 0, s, a, b, f, g, nullptr, n, m, eps, out);
    return hipGetLastError();
}

hipError_t launch_max_reduce(const float* v, int cnt, float* out, hipStream_t s, int* flag, int seq) {
    // one wave per 64 values up to 16 waves: small problems need no more than their count
    const int threads = (int)std::min<int64_t>(1024, std::max<int64_t>(64, ((int64_t)cnt + 63) / 64 * 64));
    hipLaunchKernelGGL(k_max_reduce, dim3(1), dim3(threads), 0, s, v, cnt, out, flag, seq);
    return hipGetLastError();
}

hipError_t launch_resid_reduce(const float* rbuf, int cnt, float* out_max, float* out_sum, hipStream_t s,
                               int* flag, int seq) {
    hipLaunchKernelGGL(k_resid_reduce, dim3(1), dim3(1024), 0, s, rbuf, cnt, out_max, out_sum, flag, seq);
    return hipGetLastError();
}

}  // namespace sk

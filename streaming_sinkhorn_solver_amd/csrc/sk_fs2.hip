// sk_fs2.hip -- kernels of the two-stage block-sparse solver (d <= 8).
//
// "FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport" (abstract): Morton
// ordered blocks of points, a coarse solve on block centroids lifted to the
// points, and a fine stage restricted to block pairs whose mass bound is above
// a threshold.  This file holds the data-parallel pieces around the streamed
// passes: the bounding box and Morton codes (the sort itself is hipCUB's radix
// sort), gathers into block order, per-block mass / centroid / box, the
// sampled rows of the lift check, per-block potential maxima, the tile bounds
// and their CSR / CSC lists, and the scatter back to the caller's order.
// The streamed passes themselves are the dense pass kernels (coarse stage,
// lift, sampled check) and k_pass_sparse (fine stage).
#include "sk_internal.hpp"

#include <hipcub/device/device_radix_sort.hpp>

#include <cfloat>
#include <climits>

namespace sk {
namespace {

inline int grid_of(int64_t count) { return (int)((count + kBlock - 1) / kBlock); }

// Per-coordinate min / max of a flat (npts, d) array into part[blk][0 | 1][d]:
// thread t < span owns coordinate t % d and walks the array with stride span.
__global__ __launch_bounds__(kBlock) void k_bbox_partial(const float* __restrict__ x, int64_t nx, const float* __restrict__ y,
                                                         int64_t ny, int d, float* __restrict__ part) {
    __shared__ float smin[kBlock], smax[kBlock];
    const int span = (kBlock / d) * d;
    const int t = threadIdx.x;
    float lo = FLT_MAX, hi = -FLT_MAX;
    if (t < span) {
        for (int64_t e = (int64_t)blockIdx.x * span + t; e < nx; e += (int64_t)gridDim.x * span) {
            lo = fminf(lo, x[e]);
            hi = fmaxf(hi, x[e]);
        }
        for (int64_t e = (int64_t)blockIdx.x * span + t; e < ny; e += (int64_t)gridDim.x * span) {
            lo = fminf(lo, y[e]);
            hi = fmaxf(hi, y[e]);
        }
    }
    smin[t] = lo;
    smax[t] = hi;
    __syncthreads();
    if (t < d) {
        for (int u = t + d; u < span; u += d) {
            lo = fminf(lo, smin[u]);
            hi = fmaxf(hi, smax[u]);
        }
        part[((size_t)blockIdx.x * 2 + 0) * d + t] = lo;
        part[((size_t)blockIdx.x * 2 + 1) * d + t] = hi;
    }
}

__global__ void k_bbox_final(const float* __restrict__ part, int nblk, int d, float* __restrict__ box) {
    const int t = threadIdx.x;
    if (t >= d) return;
    float lo = FLT_MAX, hi = -FLT_MAX;
    for (int b = 0; b < nblk; ++b) {
        lo = fminf(lo, part[((size_t)b * 2 + 0) * d + t]);
        hi = fmaxf(hi, part[((size_t)b * 2 + 1) * d + t]);
    }
    box[t] = lo;
    box[d + t] = hi;
}

// Morton code of each point: q_t = min(2^bits - 1, floor((p_t - lo_t) * (2^bits / (hi_t - lo_t)))) in float32,
// bit k of q_t at position k d + t.
__global__ __launch_bounds__(kBlock) void k_morton(const float* __restrict__ p, int n, int d, int bits,
                                                   const float* __restrict__ box, uint32_t* __restrict__ code,
                                                   uint32_t* __restrict__ idx) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int top = (1 << bits) - 1;
    uint32_t c = 0;
    for (int t = 0; t < d; ++t) {
        const float lo = box[t];
        const float span = box[d + t] - lo;
        const float scale = span > 0.0f ? (float)(1 << bits) / span : 0.0f;
        const float v = floorf((p[(size_t)i * d + t] - lo) * scale);
        const int q = v < 0.0f ? 0 : (v > (float)top ? top : (int)v);
        for (int k = 0; k < bits; ++k) c |= (uint32_t)((q >> k) & 1) << (k * d + t);
    }
    code[i] = c;
    idx[i] = (uint32_t)i;
}

// Points and weights in sorted order; perm[i] = original index of sorted point i.
__global__ __launch_bounds__(kBlock) void k_gather_points(const float* __restrict__ p, const float* __restrict__ w,
                                                          const uint32_t* __restrict__ idx, int n, int d,
                                                          float* __restrict__ ps, float* __restrict__ ws,
                                                          int* __restrict__ perm) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int o = (int)idx[i];
    for (int t = 0; t < d; ++t) ps[(size_t)i * d + t] = p[(size_t)o * d + t];
    ws[i] = w[o];
    perm[i] = o;
}

__device__ inline double wg_sum_d(double v, double* sh) {
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

__device__ inline float wg_min_max(float v, float* sh, bool is_max) {
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (t < w) sh[t] = is_max ? fmaxf(sh[t], sh[t + w]) : fminf(sh[t], sh[t + w]);
        __syncthreads();
    }
    const float r = sh[0];
    __syncthreads();
    return r;
}

// One workgroup per block of B sorted points: mass (float64 sum), centroid
// (weighted mean, plain mean for a massless block), box min / max.
__global__ __launch_bounds__(kBlock) void k_block_stats(const float* __restrict__ ps, const float* __restrict__ ws,
                                                        int n, int d, int B, float* __restrict__ mass,
                                                        float* __restrict__ cen, float* __restrict__ blo,
                                                        float* __restrict__ bhi) {
    __shared__ double shd[kBlock];
    __shared__ float shf[kBlock];
    const int I = blockIdx.x;
    const int r0 = I * B, r1 = min(r0 + B, n);
    double m = 0.0;
    for (int i = r0 + threadIdx.x; i < r1; i += blockDim.x) m += (double)ws[i];
    m = wg_sum_d(m, shd);
    for (int t = 0; t < d; ++t) {
        double sw = 0.0, sp = 0.0;
        float lo = FLT_MAX, hi = -FLT_MAX;
        for (int i = r0 + threadIdx.x; i < r1; i += blockDim.x) {
            const float v = ps[(size_t)i * d + t];
            sw += (double)ws[i] * (double)v;
            sp += (double)v;
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
        sw = wg_sum_d(sw, shd);
        sp = wg_sum_d(sp, shd);
        lo = wg_min_max(lo, shf, false);
        hi = wg_min_max(hi, shf, true);
        if (threadIdx.x == 0) {
            cen[(size_t)I * d + t] = (float)(m > 0.0 ? sw / m : sp / (double)(r1 - r0));
            blo[(size_t)I * d + t] = lo;
            bhi[(size_t)I * d + t] = hi;
        }
    }
    if (threadIdx.x == 0) mass[I] = (float)m;
}

// Sampled rows r * stride (r < ns): packed query row, potential, weight, |p~|^2.
__global__ __launch_bounds__(kBlock) void k_gather_rows(const float* __restrict__ qp, int P, const float* __restrict__ pot,
                                                        const float* __restrict__ w, const float* __restrict__ nrm,
                                                        int ns, int stride, float* __restrict__ qs,
                                                        float* __restrict__ pots, float* __restrict__ wsx,
                                                        float* __restrict__ nrms) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= ns) return;
    const size_t i = (size_t)r * stride;
    for (int t = 0; t < P; ++t) qs[(size_t)r * P + t] = qp[i * P + t];
    pots[r] = pot[i];
    wsx[r] = w[i];
    nrms[r] = nrm[i];
}

// Largest potential over a block's points of positive weight (-inf if none).
__global__ __launch_bounds__(kBlock) void k_block_max(const float* __restrict__ pot, const float* __restrict__ w, int n,
                                                      int B, float* __restrict__ out) {
    __shared__ float shf[kBlock];
    const int I = blockIdx.x;
    const int r0 = I * B, r1 = min(r0 + B, n);
    float mx = -INFINITY;
    for (int i = r0 + threadIdx.x; i < r1; i += blockDim.x)
        if (w[i] > 0.0f) mx = fmaxf(mx, pot[i]);
    mx = wg_min_max(mx, shf, true);
    if (threadIdx.x == 0) out[I] = mx;
}

// The tile bound of (I, J):
//   score = (fmax_I + gmax_J - dmin_IJ^2)/eps + log max(B_J NBy, A_I NBx),
// dmin from the two boxes; kept iff score > log delta (every tile when delta <= 0).
__device__ inline float tile_score(const ScreenArgs& A, int I, int J) {
    float gap2 = 0.0f;
    for (int t = 0; t < A.d; ++t) {
        const float g1 = A.ylo[(size_t)J * A.d + t] - A.xhi[(size_t)I * A.d + t];
        const float g2 = A.xlo[(size_t)I * A.d + t] - A.yhi[(size_t)J * A.d + t];
        const float g = fmaxf(0.0f, fmaxf(g1, g2));
        gap2 = fmaf(g, g, gap2);
    }
    const float E = (A.fmax[I] + A.gmax[J] - gap2) / A.eps;
    return E + logf(fmaxf(A.bmass[J] * (float)A.nby, A.amass[I] * (float)A.nbx));
}

// argmax with ties to the smaller index (numpy's first maximum); -inf scores tie too.
__device__ inline void better(float& bs, int& bi, float s, int i) {
    if (s > bs || (s == bs && i < bi)) {
        bs = s;
        bi = i;
    }
}

__device__ inline void wg_argmax(float& bs, int& bi, float* shs, int* shi) {
    const int t = threadIdx.x;
    shs[t] = bs;
    shi[t] = bi;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (t < w) {
            float s = shs[t];
            int i = shi[t];
            better(s, i, shs[t + w], shi[t + w]);
            shs[t] = s;
            shi[t] = i;
        }
        __syncthreads();
    }
    bs = shs[0];
    bi = shi[0];
    __syncthreads();
}

// The tile bounds are recomputed wherever they are needed instead of being
// stored: evaluating one is a box distance and two logarithms, and an
// NBx x NBy matrix of them would bound the problem size by memory.

// One workgroup per line o (a row block when rows, else a column block): the
// other index of the line's tile of largest bound (ties to the smaller index).
__global__ __launch_bounds__(kBlock) void k_screen_best(ScreenArgs A, int rows) {
    __shared__ float shs[kBlock];
    __shared__ int shi[kBlock];
    const int o = blockIdx.x;
    const int len = rows ? A.nby : A.nbx;
    float bs = -INFINITY;
    int bi = INT_MAX;
    for (int u = threadIdx.x; u < len; u += blockDim.x) better(bs, bi, rows ? tile_score(A, o, u) : tile_score(A, u, o), u);
    wg_argmax(bs, bi, shs, shi);
    if (threadIdx.x == 0) (rows ? A.rowbest : A.colbest)[o] = bi < len ? bi : 0;
}

// Whether tile (I, J) is kept: its bound is above log delta (every tile when
// delta <= 0), or it is the best tile of its row block or of its column block.
// Not inlined: the row lists and the column lists then take every decision
// with the same machine code, so they hold the same tiles.
__device__ __noinline__ bool tile_kept(const ScreenArgs& A, int I, int J) {
    return A.delta <= 0.0f || A.rowbest[I] == J || A.colbest[J] == I || tile_score(A, I, J) > A.log_delta;
}

// Kept tiles of line o (a row block when rows, else a column block), in
// increasing order of the other index: count (idx == null) or write at ptr[o]
// (entries at or beyond cap are not written; the caller checks the total).
// Each thread takes a contiguous run of the line, so a workgroup prefix sum
// keeps the order.
__global__ __launch_bounds__(kBlock) void k_tile_list(ScreenArgs A, int rows, const int* __restrict__ ptr,
                                                      int* __restrict__ cnt, int* __restrict__ idx) {
    __shared__ int sh[kBlock];
    const int o = blockIdx.x;
    const int len = rows ? A.nby : A.nbx;
    const int per = (len + kBlock - 1) / kBlock;
    const int u0 = min(threadIdx.x * per, len), u1 = min(u0 + per, len);
    auto at = [&](int u) { return rows ? tile_kept(A, o, u) : tile_kept(A, u, o); };
    int c = 0;
    for (int u = u0; u < u1; ++u) c += at(u) ? 1 : 0;
    sh[threadIdx.x] = c;
    __syncthreads();
    // inclusive scan (Hillis-Steele) over the workgroup
    for (int w = 1; w < kBlock; w <<= 1) {
        const int v = threadIdx.x >= w ? sh[threadIdx.x - w] : 0;
        __syncthreads();
        sh[threadIdx.x] += v;
        __syncthreads();
    }
    if (!idx) {
        if (threadIdx.x == kBlock - 1) cnt[o] = sh[kBlock - 1];
        return;
    }
    int64_t pos = (int64_t)ptr[o] + sh[threadIdx.x] - c;
    for (int u = u0; u < u1; ++u)
        if (at(u)) {
            if (pos < A.cap) idx[pos] = u;
            ++pos;
        }
}

// Exclusive prefix sum of cnt[0..len) into ptr[0..len] in one workgroup (fixed
// order), summed in 64 bits; values above cap are stored as cap + 1, so a total
// beyond the lists' capacity shows as ptr[len] > cap however large it is.
__global__ __launch_bounds__(kBlock) void k_exclusive_scan(const int* __restrict__ cnt, int len, int64_t cap,
                                                           int* __restrict__ ptr) {
    __shared__ long long sh[kBlock];
    const int per = (len + kBlock - 1) / kBlock;
    const int u0 = min(threadIdx.x * per, len), u1 = min(u0 + per, len);
    long long c = 0;
    for (int u = u0; u < u1; ++u) c += cnt[u];
    sh[threadIdx.x] = c;
    __syncthreads();
    for (int w = 1; w < kBlock; w <<= 1) {
        const long long v = threadIdx.x >= w ? sh[threadIdx.x - w] : 0;
        __syncthreads();
        sh[threadIdx.x] += v;
        __syncthreads();
    }
    auto clamp = [&](long long v) { return (int)(v > cap ? cap + 1 : v); };
    long long run = sh[threadIdx.x] - c;
    for (int u = u0; u < u1; ++u) {
        ptr[u] = clamp(run);
        run += cnt[u];
    }
    if (threadIdx.x == kBlock - 1) ptr[len] = clamp(sh[kBlock - 1]);
}

__global__ __launch_bounds__(kBlock) void k_scatter(const float* __restrict__ in, const int* __restrict__ perm, int n,
                                                    float* __restrict__ out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[perm[i]] = in[i];
}

}  // namespace

hipError_t launch_bbox(const float* x, int n, const float* y, int m, int d, float* part, float* box, hipStream_t s) {
    hipLaunchKernelGGL(k_bbox_partial, dim3(kRedBlocks), dim3(kBlock), 0, s, x, (int64_t)n * d, y, (int64_t)m * d, d,
                       part);
    hipLaunchKernelGGL(k_bbox_final, dim3(1), dim3(64), 0, s, part, kRedBlocks, d, box);
    return hipGetLastError();
}

hipError_t launch_morton(const float* p, int n, int d, int bits, const float* box, uint32_t* code, uint32_t* idx,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_morton, dim3(grid_of(n)), dim3(kBlock), 0, s, p, n, d, bits, box, code, idx);
    return hipGetLastError();
}

size_t sort_temp_bytes(int n, int end_bit) {
    size_t bytes = 0;
    if (hipcub::DeviceRadixSort::SortPairs(nullptr, bytes, (const uint32_t*)nullptr, (uint32_t*)nullptr,
                                           (const uint32_t*)nullptr, (uint32_t*)nullptr, n, 0, end_bit) != hipSuccess)
        return 0;
    return bytes;
}

hipError_t launch_sort_pairs(void* temp, size_t temp_bytes, const uint32_t* kin, uint32_t* kout, const uint32_t* vin,
                             uint32_t* vout, int n, int end_bit, hipStream_t s) {
    return hipcub::DeviceRadixSort::SortPairs(temp, temp_bytes, kin, kout, vin, vout, n, 0, end_bit, s);
}

hipError_t launch_gather_points(const float* p, const float* w, const uint32_t* idx, int n, int d, float* ps, float* ws,
                                int* perm, hipStream_t s) {
    hipLaunchKernelGGL(k_gather_points, dim3(grid_of(n)), dim3(kBlock), 0, s, p, w, idx, n, d, ps, ws, perm);
    return hipGetLastError();
}

hipError_t launch_block_stats(const float* ps, const float* ws, int n, int d, int B, float* mass, float* cen,
                              float* blo, float* bhi, hipStream_t s) {
    hipLaunchKernelGGL(k_block_stats, dim3((n + B - 1) / B), dim3(kBlock), 0, s, ps, ws, n, d, B, mass, cen, blo, bhi);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const float* qp, int P, const float* pot, const float* w, const float* nrm, int ns,
                              int stride, float* qs, float* pots, float* ws, float* nrms, hipStream_t s) {
    hipLaunchKernelGGL(k_gather_rows, dim3(grid_of(ns)), dim3(kBlock), 0, s, qp, P, pot, w, nrm, ns, stride, qs, pots,
                       ws, nrms);
    return hipGetLastError();
}

hipError_t launch_block_max(const float* pot, const float* w, int n, int B, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_block_max, dim3((n + B - 1) / B), dim3(kBlock), 0, s, pot, w, n, B, out);
    return hipGetLastError();
}

hipError_t launch_screen(const ScreenArgs& a, int* rcnt, int* rptr, int* ridx, int* ccnt, int* cptr, int* cidx,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_screen_best, dim3(a.nbx), dim3(kBlock), 0, s, a, 1);
    hipLaunchKernelGGL(k_screen_best, dim3(a.nby), dim3(kBlock), 0, s, a, 0);
    hipLaunchKernelGGL(k_tile_list, dim3(a.nbx), dim3(kBlock), 0, s, a, 1, nullptr, rcnt, nullptr);
    hipLaunchKernelGGL(k_tile_list, dim3(a.nby), dim3(kBlock), 0, s, a, 0, nullptr, ccnt, nullptr);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kBlock), 0, s, rcnt, a.nbx, a.cap, rptr);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kBlock), 0, s, ccnt, a.nby, a.cap, cptr);
    hipLaunchKernelGGL(k_tile_list, dim3(a.nbx), dim3(kBlock), 0, s, a, 1, rptr, rcnt, ridx);
    hipLaunchKernelGGL(k_tile_list, dim3(a.nby), dim3(kBlock), 0, s, a, 0, cptr, ccnt, cidx);
    return hipGetLastError();
}

hipError_t launch_scatter(const float* in, const int* perm, int n, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_scatter, dim3(grid_of(n)), dim3(kBlock), 0, s, in, perm, n, out);
    return hipGetLastError();
}

}  // namespace sk

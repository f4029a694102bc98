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
//   score = (fmax_I + gmax_J - dmin_IJ^2)/eps + log max(A_I NBx, B_J NBy),
// dmin from the two boxes; kept iff score > log delta (every tile when delta <= 0).
// Each block is first packed into one record (its box, its potential maximum
// and log(mass x block count)), so a bound is a box distance, an add and one
// fma; the logarithm of the larger mass term is the larger logarithm.
// The bounds are recomputed wherever they are needed instead of being stored:
// an NBx x NBy matrix of them would bound the problem size by memory.
template <int D>
struct Rec {
    float lo[D], hi[D], pot, lam;
};

template <int D>
__device__ inline Rec<D> load_rec(const float* __restrict__ recs, int b) {
    constexpr int S = screen_stride_of(D);
    float v[S];
    const float4* p = reinterpret_cast<const float4*>(recs + (size_t)b * S);
#pragma unroll
    for (int k = 0; k < S / 4; ++k) {
        const float4 t = p[k];
        v[4 * k] = t.x;
        v[4 * k + 1] = t.y;
        v[4 * k + 2] = t.z;
        v[4 * k + 3] = t.w;
    }
    Rec<D> r;
#pragma unroll
    for (int t = 0; t < D; ++t) {
        r.lo[t] = v[t];
        r.hi[t] = v[D + t];
    }
    r.pot = v[2 * D];
    r.lam = v[2 * D + 1];
    return r;
}

// X is always the row (x) block and Y the column (y) block, and every step is
// an IEEE operation with no multiply-add left to the compiler's choice, so a
// tile's bound has the same bits in every kernel that evaluates it: the row
// lists and the column lists hold the same tiles.
template <int D>
__device__ inline float rec_score(const Rec<D>& X, const Rec<D>& Y, float inv_eps) {
    float gap2 = 0.0f;
#pragma unroll
    for (int t = 0; t < D; ++t) {
        const float g = fmaxf(0.0f, fmaxf(Y.lo[t] - X.hi[t], X.lo[t] - Y.hi[t]));
        gap2 = fmaf(g, g, gap2);
    }
    return fmaf((X.pot + Y.pot) - gap2, inv_eps, fmaxf(X.lam, Y.lam));
}

// One record per block: lo[d], hi[d], the potential maximum, log(mass * nb),
// zero padding up to the stride.
__global__ __launch_bounds__(kBlock) void k_screen_rec(const float* __restrict__ pmax, const float* __restrict__ mass,
                                                       const float* __restrict__ lo, const float* __restrict__ hi,
                                                       int nb, int d, int S, float* __restrict__ rec) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nb) return;
    float* r = rec + (size_t)b * S;
    for (int t = 0; t < d; ++t) {
        r[t] = lo[(size_t)b * d + t];
        r[d + t] = hi[(size_t)b * d + t];
    }
    r[2 * d] = pmax[b];
    r[2 * d + 1] = logf(mass[b] * (float)nb);
    for (int t = 2 * d + 2; t < S; ++t) r[t] = 0.0f;
}

// argmax with ties to the smaller index (numpy's first maximum); -inf scores tie too.
__device__ inline void better(float& bs, int& bi, float s, int i) {
    if (s > bs || (s == bs && i < bi)) {
        bs = s;
        bi = i;
    }
}

// Lines (row or column blocks) per workgroup: the line records stay in
// registers, so fewer lines at larger d.
constexpr int lines_of(int D) { return D <= 4 ? 8 : 4; }
constexpr int kWaves = kBlock / 64;

// The lines o0 .. o0 + NL - 1 of a workgroup: row blocks when ROWS, else
// column blocks; a line past the end repeats the last one and is not stored.
// The line records pass through LDS, so each lane holds its own copy in vector
// registers instead of the compiler keeping them in scalar registers, which
// it runs out of and spills.
template <int D, bool ROWS>
struct Lines {
    static constexpr int NL = lines_of(D);
    Rec<D> r[NL];
    int best[NL];  // the line's own best tile (list kernels)
    int o0, nl, no;
    const float* other;
    const int* obest;  // the other side's best tiles

    __device__ Lines(const ScreenArgs& A, bool with_best, float* stage) {
        constexpr int S = screen_stride_of(D);
        o0 = blockIdx.x * NL;
        nl = ROWS ? A.nbx : A.nby;
        no = ROWS ? A.nby : A.nbx;
        other = ROWS ? A.dy : A.dx;
        obest = ROWS ? A.colbest : A.rowbest;
        const float* own = ROWS ? A.dx : A.dy;
        const int* lbest = ROWS ? A.rowbest : A.colbest;
        for (int k = threadIdx.x; k < NL * S; k += blockDim.x)
            stage[k] = own[(size_t)min(o0 + k / S, nl - 1) * S + k % S];
        __syncthreads();
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            r[l] = load_rec<D>(stage, l);
            best[l] = with_best ? lbest[min(o0 + l, nl - 1)] : 0;
        }
    }
    __device__ float score(int l, const Rec<D>& q, float inv_eps) const {
        return ROWS ? rec_score<D>(r[l], q, inv_eps) : rec_score<D>(q, r[l], inv_eps);
    }
    // tile (line l, other block u) kept: its bound is above log delta (every
    // tile when delta <= 0), or it is the best tile of its row or its column
    __device__ bool kept(const ScreenArgs& A, int l, int u, const Rec<D>& q, int obu) const {
        return A.delta <= 0.0f || best[l] == u || obu == o0 + l || score(l, q, A.inv_eps) > A.log_delta;
    }
};

// Per line, the other index of its tile of largest bound (ties to the smaller
// index) into rowbest (ROWS) or colbest.
template <int D, bool ROWS>
__global__ __launch_bounds__(kBlock) void k_screen_best(ScreenArgs A) {
    constexpr int NL = lines_of(D);
    __shared__ float shs[NL][kWaves];
    __shared__ int shi[NL][kWaves];
    __shared__ float4 stage[NL * screen_stride_of(D) / 4];
    const Lines<D, ROWS> L(A, false, reinterpret_cast<float*>(stage));
    float bs[NL];
    int bi[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        bs[l] = -INFINITY;
        bi[l] = INT_MAX;
    }
    for (int u = threadIdx.x; u < L.no; u += kBlock) {
        const Rec<D> q = load_rec<D>(L.other, u);
#pragma unroll
        for (int l = 0; l < NL; ++l) better(bs[l], bi[l], L.score(l, q, A.inv_eps), u);
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
        for (int k = 32; k > 0; k >>= 1) better(bs[l], bi[l], __shfl_xor(bs[l], k), __shfl_xor(bi[l], k));
        if (lane == 0) {
            shs[l][wv] = bs[l];
            shi[l][wv] = bi[l];
        }
    }
    __syncthreads();
    const int l = threadIdx.x;
    if (l < NL && L.o0 + l < L.nl) {
        float s = shs[l][0];
        int i = shi[l][0];
        for (int w = 1; w < kWaves; ++w) better(s, i, shs[l][w], shi[l][w]);
        (ROWS ? A.rowbest : A.colbest)[L.o0 + l] = i < L.no ? i : 0;
    }
}

// Kept tiles per line: counted into cnt (idx == null), else written at
// ptr[line] in increasing order of the other index (entries at or beyond cap
// are not written; the caller checks the total).  The workgroup walks the
// other blocks in chunks of kBlock, one per thread, and places each chunk's
// kept entries with a ballot and the wave totals, which keeps the order.
template <int D, bool ROWS>
__global__ __launch_bounds__(kBlock) void k_tile_list(ScreenArgs A, const int* __restrict__ ptr,
                                                      int* __restrict__ cnt, int* __restrict__ idx) {
    constexpr int NL = lines_of(D);
    __shared__ int wt[NL][kWaves];
    __shared__ float4 stage[NL * screen_stride_of(D) / 4];
    const Lines<D, ROWS> L(A, true, reinterpret_cast<float*>(stage));
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (!idx) {
        int c[NL] = {};
        for (int u = threadIdx.x; u < L.no; u += kBlock) {
            const Rec<D> q = load_rec<D>(L.other, u);
            const int obu = L.obest[u];
#pragma unroll
            for (int l = 0; l < NL; ++l) c[l] += L.kept(A, l, u, q, obu) ? 1 : 0;
        }
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            for (int k = 32; k > 0; k >>= 1) c[l] += __shfl_xor(c[l], k);
            if (lane == 0) wt[l][wv] = c[l];
        }
        __syncthreads();
        const int l = threadIdx.x;
        if (l < NL && L.o0 + l < L.nl) {
            int t = 0;
            for (int w = 0; w < kWaves; ++w) t += wt[l][w];
            cnt[L.o0 + l] = t;
        }
        return;
    }
    int64_t base[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) base[l] = L.o0 + l < L.nl ? ptr[L.o0 + l] : 0;
    const unsigned long long below_me = (1ull << lane) - 1ull;
    for (int ub = 0; ub < L.no; ub += kBlock) {
        const int u = ub + threadIdx.x;
        const bool in = u < L.no;
        const int uc = in ? u : L.no - 1;
        const Rec<D> q = load_rec<D>(L.other, uc);
        const int obu = L.obest[uc];
        unsigned mine = 0;
        int pre[NL];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const bool k = in && L.o0 + l < L.nl && L.kept(A, l, u, q, obu);
            const unsigned long long bal = __ballot(k);
            pre[l] = __popcll(bal & below_me);
            mine |= (k ? 1u : 0u) << l;
            if (lane == 0) wt[l][wv] = __popcll(bal);
        }
        __syncthreads();
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            int lower = 0, tot = 0;
            for (int w = 0; w < kWaves; ++w) {
                const int c = wt[l][w];
                lower += w < wv ? c : 0;
                tot += c;
            }
            if ((mine >> l) & 1u) {
                const int64_t pos = base[l] + lower + pre[l];
                if (pos < A.cap) idx[pos] = u;
            }
            base[l] += tot;
        }
        __syncthreads();
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

template <int D>
void screen_d(const ScreenArgs& a, int* rcnt, int* rptr, int* ridx, int* ccnt, int* cptr, int* cidx, hipStream_t s) {
    constexpr int NL = lines_of(D);
    const dim3 gx((a.nbx + NL - 1) / NL), gy((a.nby + NL - 1) / NL);
    hipLaunchKernelGGL((k_screen_best<D, true>), gx, dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL((k_screen_best<D, false>), gy, dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL((k_tile_list<D, true>), gx, dim3(kBlock), 0, s, a, nullptr, rcnt, nullptr);
    hipLaunchKernelGGL((k_tile_list<D, false>), gy, dim3(kBlock), 0, s, a, nullptr, ccnt, nullptr);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kBlock), 0, s, rcnt, a.nbx, a.cap, rptr);
    hipLaunchKernelGGL(k_exclusive_scan, dim3(1), dim3(kBlock), 0, s, ccnt, a.nby, a.cap, cptr);
    hipLaunchKernelGGL((k_tile_list<D, true>), gx, dim3(kBlock), 0, s, a, rptr, rcnt, ridx);
    hipLaunchKernelGGL((k_tile_list<D, false>), gy, dim3(kBlock), 0, s, a, cptr, ccnt, cidx);
}

hipError_t launch_screen(const ScreenArgs& a_in, int* rcnt, int* rptr, int* ridx, int* ccnt, int* cptr, int* cidx,
                         hipStream_t s) {
    ScreenArgs a = a_in;
    a.inv_eps = 1.0f / a.eps;
    const int S = screen_stride_of(a.d);
    hipLaunchKernelGGL(k_screen_rec, dim3(grid_of(a.nbx)), dim3(kBlock), 0, s, a.fmax, a.amass, a.xlo, a.xhi, a.nbx,
                       a.d, S, a.dx);
    hipLaunchKernelGGL(k_screen_rec, dim3(grid_of(a.nby)), dim3(kBlock), 0, s, a.gmax, a.bmass, a.ylo, a.yhi, a.nby,
                       a.d, S, a.dy);
    switch (a.d) {
        case 1: screen_d<1>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 2: screen_d<2>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 3: screen_d<3>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 4: screen_d<4>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 5: screen_d<5>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 6: screen_d<6>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 7: screen_d<7>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        case 8: screen_d<8>(a, rcnt, rptr, ridx, ccnt, cptr, cidx, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scatter(const float* in, const int* perm, int n, float* out, hipStream_t s) {
    hipLaunchKernelGGL(k_scatter, dim3(grid_of(n)), dim3(kBlock), 0, s, in, perm, n, out);
    return hipGetLastError();
}

}  // namespace sk

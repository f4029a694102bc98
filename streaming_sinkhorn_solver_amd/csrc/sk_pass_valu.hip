// sk_pass_valu.hip -- streamed log-sum-exp passes on the vector ALUs (d <= 8).
//
// One pass computes, for every query point i, lse_i = log2 sum_j 2^{s_ij} with
// s_ij = <q_i, k_j> + h_j over all keys j, without storing any s_ij
// ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodology 2:
// no materialisation, online running max / sum-exp, fused score + bias + LSE +
// potential update, row-stationary traversal).
//
// Mapping to CDNA4:
//  * row-stationary: each lane owns R query rows in registers (pre-scaled
//    coordinates, running max M and sum S); rows are strided by the workgroup
//    size so a wave's loads are contiguous;
//  * keys (coordinates + bias, one float4 for d <= 3) are staged tile by tile
//    in LDS and read back as wave-wide broadcasts;
//  * per (row, key) the work is d FMAs, one max, one subtract, one exp2 and one
//    add; the running max is updated once per chunk of TJ keys, so the
//    rescale of S costs one exp2 per chunk rather than per pair (R = 2 rows
//    per lane and TJ = 16 keys per chunk were the fastest of 20 measured
//    tilings at n = m = 50,000, d = 3);
//  * when the rows alone cannot fill 256 CUs the key range is split across
//    workgroups and the partial (M, S) pairs are merged exactly afterwards:
//    M = max_s M_s, S = sum_s S_s 2^{M_s - M}.
// The running max starts at -FLT_MAX, not -inf, so keys with zero weight
// (bias -inf) never produce (-inf) - (-inf).
#include "sk_internal.hpp"
#include "sk_pass_common.hpp"

#ifndef SK_VALU_R
#define SK_VALU_R 2
#endif
#ifndef SK_VALU_TJ
#define SK_VALU_TJ 16
#endif
#ifndef SK_VALU_TL
#define SK_VALU_TL 256
#endif

namespace sk {
namespace {

constexpr int kR = SK_VALU_R;     // query rows per lane
constexpr int kTJ = SK_VALU_TJ;   // keys per register chunk
constexpr int kTL = SK_VALU_TL;   // keys per LDS tile

// Stages keys [base, base + kTL) of the split [.., c1) into LDS; keys past c1
// get zero coordinates and bias -inf, so they add exactly nothing.
template <int D>
__device__ __forceinline__ void stage_tile(float4* tile, const float4* __restrict__ kp, int base, int c1) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    for (int e = threadIdx.x; e < kTL * V; e += kBlock) {
        const int col = base + e / V;
        const int part = e % V;
        float4 v;
        if (col < c1) {
            v = kp[(size_t)col * V + part];
        } else {
            v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (part == D / 4) {
                float* c = reinterpret_cast<float*>(&v);
                c[D % 4] = -INFINITY;
            }
        }
        tile[e] = v;
    }
}

// One chunk of kTJ keys, read from an LDS tile at key offset c (broadcast:
// every lane reads the same key), against the R query rows each lane holds:
// scores, one running-max update per row and the rescaled sum (base 2).
template <int D>
__device__ __forceinline__ void lse_chunk(const float4* tile, int c, const float (&q)[kR][D], float (&M)[kR],
                                          float (&S)[kR]) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    float kk[kTJ][P];
#pragma unroll
    for (int t = 0; t < kTJ; ++t)
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const float4 v = tile[(c + t) * V + u];
            kk[t][4 * u + 0] = v.x;
            kk[t][4 * u + 1] = v.y;
            kk[t][4 * u + 2] = v.z;
            kk[t][4 * u + 3] = v.w;
        }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        float s[kTJ];
#pragma unroll
        for (int t = 0; t < kTJ; ++t) {
            float acc = kk[t][D];
#pragma unroll
            for (int dd = 0; dd < D; ++dd) acc = fmaf(q[r][dd], kk[t][dd], acc);
            s[t] = acc;
        }
        float mt = s[0];
#pragma unroll
        for (int t = 1; t < kTJ; ++t) mt = fmaxf(mt, s[t]);
        const float mn = fmaxf(M[r], mt);
        float acc = S[r] * ex2(M[r] - mn);
#pragma unroll
        for (int t = 0; t < kTJ; ++t) acc += ex2(s[t] - mn);
        S[r] = acc;
        M[r] = mn;
    }
}

// Streams keys [j0, j1) past the R query rows each lane holds, updating the
// running max M and rescaled sum S of every row (base 2).  The whole
// workgroup stages each tile (the block-sparse pass, whose lanes hold
// kBlock * kR rows).
template <int D>
__device__ __forceinline__ void scan_keys(float4* tile, const float4* __restrict__ kp, const float (&q)[kR][D],
                                          float (&M)[kR], float (&S)[kR], int j0, int j1) {
    for (int base = j0; base < j1; base += kTL) {
        __syncthreads();
        stage_tile<D>(tile, kp, base, j1);
        __syncthreads();
        const int ntile = min(kTL, j1 - base);
        for (int c = 0; c < ntile; c += kTJ) lse_chunk<D>(tile, c, q, M, S);
    }
}

// Keys per wave-private LDS tile of the dense pass: at most 256 float4 (4 KB)
// whatever d, a multiple of 64 keys (whole chunks, so a chunk never reads past
// the tile, and whole float4s per lane when the wave stages it).
template <int D>
constexpr int wave_tile_keys() {
    return 256 / (((D + 1 + 3) / 4) * 4 / 4) / 64 * 64;
}
static_assert(wave_tile_keys<8>() == 64 && wave_tile_keys<4>() == 128 && wave_tile_keys<3>() == 256, "tiles");
static_assert(64 % kTJ == 0, "a tile holds whole chunks");

// Orders one wave's LDS stores before its later LDS loads.  The lanes of a
// wave issue LDS instructions in program order and the LDS performs them in
// order, so no hardware barrier is needed; the fences keep the compiler from
// moving the loads above the stores.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same scan by one wave alone, through its own LDS tile: keys past j1 are
// staged with zero coordinates and bias -inf and add exactly nothing.
template <int D>
__device__ __forceinline__ void scan_keys_wave(float4* tile, const float4* __restrict__ kp, const float (&q)[kR][D],
                                               float (&M)[kR], float (&S)[kR], int j0, int j1, int lane) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    constexpr int TK = wave_tile_keys<D>();
    static_assert((TK * V) % 64 == 0, "a tile is whole float4s per lane");
    for (int base = j0; base < j1; base += TK) {
        wave_lds_sync();
        // all of a lane's loads in flight at once: clamped addresses, padding selected afterwards
        float4 v[TK * V / 64];
#pragma unroll
        for (int k = 0; k < TK * V / 64; ++k) {
            const int e = lane + 64 * k;
            const int col = min(base + e / V, j1 - 1);
            v[k] = kp[(size_t)col * V + e % V];
        }
#pragma unroll
        for (int k = 0; k < TK * V / 64; ++k) {
            const int e = lane + 64 * k;
            if (base + e / V >= j1) {
                v[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (e % V == D / 4) reinterpret_cast<float*>(&v[k])[D % 4] = -INFINITY;
            }
            tile[e] = v[k];
        }
        wave_lds_sync();
        const int ntile = min(TK, j1 - base);
        for (int c = 0; c < ntile; c += kTJ) lse_chunk<D>(tile, c, q, M, S);
    }
}

// Block-sparse pass, stream-K over the kept tiles.  The kept (query block,
// key block) tiles, in CSR order (query block I owns tiles ptr[I] ..
// ptr[I + 1]), are cut into W equal contiguous ranges, one per workgroup,
// whatever the query blocks, so the work balances however unevenly the
// tiles fall.  A workgroup walks its range query block by query block; a
// segment that covers a block's whole list finishes it in place, a first or
// last segment that does not leaves partial (M, S) in slot 0 or 1 for the
// merge.  Both clouds are in block order, so a key block is a contiguous key
// range and each tile is one call of the dense key scan.
template <int D>
__global__ __launch_bounds__(kBlock) void k_pass_sparse(SparseArgs A) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    __shared__ float4 tile[kTL * (P / 4)];
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const int w = blockIdx.x;
    const int64_t nnz = A.ptr[A.nqb];
    int64_t t = range_lo(w, nnz, A.W);
    const int64_t u1 = range_lo(w + 1, nnz, A.W);
    if (t >= u1) return;
    // query block of tile t: the largest I with ptr[I] <= t (empty blocks never qualify last)
    int lo = 0, hi = A.nqb - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (A.ptr[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    int I = lo;
    bool first = true;
    while (t < u1) {
        const int64_t b0 = A.ptr[I], b1 = A.ptr[I + 1];
        const int64_t seg_hi = min(u1, b1);
        const int r0 = I * A.B;
        const int r1 = min(r0 + A.B, A.nq);
        float q[kR][D], M[kR], S[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int i = r0 + threadIdx.x + r * kBlock;
            const int ic = i < r1 ? i : r1 - 1;
#pragma unroll
            for (int c = 0; c < D; ++c) q[r][c] = A.q[(size_t)ic * P + c] * A.qscale;
            M[r] = kNegBig;
            S[r] = 0.0f;
        }
        for (int64_t tt = t; tt < seg_hi; ++tt) {
            const int j0 = A.idx[tt] * A.B;
            scan_keys<D>(tile, kp, q, M, S, j0, min(j0 + A.B, A.nk));
        }
        const bool whole = t == b0 && seg_hi == b1;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int i = r0 + threadIdx.x + r * kBlock;
            if (i >= r1) continue;
            if (whole)
                finalize(A.fin, i, M[r] + lg2(S[r]));
            else
                A.part[((size_t)w * 2 + (first ? 0 : 1)) * A.B + (i - r0)] = make_float2(M[r], S[r]);
        }
        first = false;
        t = seg_hi;
        while (I + 1 < A.nqb && A.ptr[I + 1] <= t) ++I;
    }
}

// Rows of query blocks split across workgroups: combine the partials of the
// workgroups whose ranges meet the block's tile list, in workgroup order.
__global__ __launch_bounds__(kBlock) void k_sparse_merge(SparseArgs A) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= A.nq) return;
    const int I = i / A.B;
    const int64_t nnz = A.ptr[A.nqb];
    const int64_t p0 = A.ptr[I], p1 = A.ptr[I + 1];
    if (p0 >= p1) return;  // no tiles (every block keeps one, so this does not occur)
    const int w0 = range_owner(p0, nnz, A.W), w1 = range_owner(p1 - 1, nnz, A.W);
    if (w0 == w1) return;  // finished in place
    const FinIn pre = fin_load(A.fin, i);  // issued before the partials' loads
    float M = kNegBig, S = 0.0f;
    for (int w = w0; w <= w1; ++w) {
        const int64_t lo = range_lo(w, nnz, A.W);
        if (lo == range_lo(w + 1, nnz, A.W)) continue;  // an empty range wrote nothing
        const int slot = (w == w0 && lo < p0) ? 1 : 0;
        const float2 p = A.part[((size_t)w * 2 + slot) * A.B + (i - I * A.B)];
        const float mn = fmaxf(M, p.x);
        S = S * ex2(M - mn) + p.y * ex2(p.x - mn);
        M = mn;
    }
    finalize(A.fin, i, M + lg2(S), pre);
}

// The dense pass.  A row block is the kPassRows = 64 R rows of one wave's
// lanes, and all kWaves waves of a workgroup hold the same rows: each wave
// scans a chunk-aligned quarter of the segment's keys through its own LDS
// tile (no workgroup barrier inside the scan), then the waves' (M, S) are
// merged through LDS and one thread per row finishes the row or writes its
// partial.  Sharing rows across the waves cuts the partials a stream-K range
// leaves, and the merge that reads them, by kWaves against a workgroup of
// kWaves * 64 R distinct rows, for the same work per lane.
constexpr int kWaves = kBlock / 64;
constexpr int kPassRows = 64 * kR;

// Occupancy asked of the compiler (waves per SIMD).  Left to itself it
// schedules the chunk loop for 5 waves at d = 2, 3 (87 and 95 VGPRs): 3.4%
// slower at 50,000^2 than the 7 waves the previous layout of this pass ran
// at.  Held to 6 (80 VGPRs) it needs no scratch.  Held to 7 (72 VGPRs) it
// spills a few values of the segment set-up (none in the key loop); with
// several resident rounds of workgroups those scratch lines reach HBM.
// Measured with the round rule, per 100-iteration solve: 50,000^2 85.8 ms
// at 6 waves against 86.4 at 7, with 6.5 against 23.0 MB written per pass
// launch; 50,000 x 40,000 69.5 against 69.8 ms.  The larger d keep the
// occupancy the previous layout had.
template <int D>
constexpr int pass_min_waves() {
    return D <= 3 ? 6 : (D == 4 ? 5 : (D <= 7 ? 4 : 3));
}

template <int D>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(pass_min_waves<D>(), 8)))
void k_pass_valu(PassArgs A) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    constexpr int TK = wave_tile_keys<D>();
    __shared__ float4 tiles[kWaves][TK * V];
    __shared__ float2 red[kWaves][kPassRows];
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

    const int w = xcd_range(blockIdx.x, A.W);
    const int64_t lo = range_lo(w, A.total, A.W), hi = range_lo(w + 1, A.total, A.W);
    for (int64_t u = lo; u < hi;) {
        const int rb = (int)(u / A.nk);
        const int j0 = (int)(u - (int64_t)rb * A.nk);
        const int j1 = (int)min<int64_t>((int64_t)A.nk, (int64_t)j0 + (hi - u));
        const int row0 = rb * kPassRows + lane;

        float q[kR][D];
        float M[kR], S[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int i = row0 + r * 64;
            const int ic = i < A.nq ? i : A.nq - 1;
            const float* qr = A.q + (size_t)ic * P;
#pragma unroll
            for (int t = 0; t < D; ++t) q[r][t] = qr[t] * A.qscale;
            M[r] = kNegBig;
            S[r] = 0.0f;
        }
        // this wave's share of [j0, j1): whole chunks, the last wave taking the remainder
        const int per = (j1 - j0 + kWaves * kTJ - 1) / (kWaves * kTJ) * kTJ;
        const int wj0 = min(j1, j0 + wave * per), wj1 = min(j1, wj0 + per);
        scan_keys_wave<D>(tiles[wave], kp, q, M, S, wj0, wj1, lane);
#pragma unroll
        for (int r = 0; r < kR; ++r) red[wave][lane + r * 64] = make_float2(M[r], S[r]);
        __syncthreads();
        if (threadIdx.x < kPassRows) {
            const int lr = threadIdx.x;
            float m = red[0][lr].x, sum = red[0][lr].y;
#pragma unroll
            for (int k = 1; k < kWaves; ++k) {
                const float2 p = red[k][lr];
                const float mn = fmaxf(m, p.x);
                sum = sum * ex2(m - mn) + p.y * ex2(p.x - mn);
                m = mn;
            }
            const int i = rb * kPassRows + lr;
            if (i < A.nq) {
                if (j0 == 0 && j1 == A.nk)
                    finalize(A.fin, i, m + lg2(sum));
                else
                    A.part[((size_t)w * 2 + (u == lo ? 0 : 1)) * A.rpb + lr] = make_float2(m, sum);
            }
        }
        __syncthreads();  // red is rewritten by the next segment
        u += j1 - j0;
    }
}

// Small problems (at most 2e6 pairs per pass, e.g. 1000 x 1000): one pass
// kernel per half-step, no partials and no merge launch, which is what bounds
// such passes (measured 7.1 us vs 7.8 us + the merge at 1000 x 1000; at
// 10,000 x 10,000 the stream-K pass is faster, 27 us vs 44 us).
// kSmallG consecutive lanes share a query row; lane `sub` of the group takes
// keys sub, sub + G, sub + 2G, ... of each LDS tile (the lanes of a wave read
// G consecutive keys per step, conflict-free), keeps its own running (M, S),
// and the group joins them with a fixed xor-shuffle tree.
#ifndef SK_SMALL_G
#define SK_SMALL_G 64
#endif
constexpr int kSmallG = SK_SMALL_G;
constexpr int kSmallRows = kBlock / kSmallG;   // query rows per workgroup
// keys per lane per chunk: 16 covers 1024 keys in one chunk, so a 1000-key pass
// issues all its key loads before the first use (3.26 against 3.45 us per
// graph-replayed pass at 1000 x 1000 with 8)
constexpr int kSmallTJ = 16;
constexpr int kSmallTile = 1024;               // keys per LDS tile (multiple of G * TJ)
static_assert(kSmallTile % (kSmallG * kSmallTJ) == 0, "tile must hold whole chunks");

template <int D>
__global__ __launch_bounds__(kBlock) void k_pass_small(PassArgs A) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    __shared__ float4 tile[kSmallTile * V];
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const int sub = threadIdx.x % kSmallG;
    const int i = blockIdx.x * kSmallRows + threadIdx.x / kSmallG;
    const int ic = i < A.nq ? i : A.nq - 1;
    float q[D];
#pragma unroll
    for (int t = 0; t < D; ++t) q[t] = A.q[(size_t)ic * P + t] * A.qscale;
    // the row's finalisation inputs, loaded now so that their latency overlaps the key loads
    const FinIn pre = fin_load(A.fin, ic);
    float M = kNegBig, S = 0.0f;

    if (A.nk <= kSmallTile) {
        // one tile's worth of keys: each lane reads its own straight from global
        // memory (cached, and shared by the workgroup's rows), skipping the LDS
        // round trip and barrier that dominate so short a kernel (1000 x 1000:
        // 7.7 us per iteration instead of 9.0)
        for (int t0 = 0; kSmallG * t0 < A.nk; t0 += kSmallTJ) {
            float s[kSmallTJ];
#pragma unroll
            for (int tt = 0; tt < kSmallTJ; ++tt) {
                const int col = sub + kSmallG * (t0 + tt);
                const int cc = col < A.nk ? col : A.nk - 1;
                float kk[P];
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    const float4 v = kp[(size_t)cc * V + u];
                    kk[4 * u + 0] = v.x;
                    kk[4 * u + 1] = v.y;
                    kk[4 * u + 2] = v.z;
                    kk[4 * u + 3] = v.w;
                }
                float acc = col < A.nk ? kk[D] : -INFINITY;  // past the keys: bias -inf, adds nothing
#pragma unroll
                for (int dd = 0; dd < D; ++dd) acc = fmaf(q[dd], kk[dd], acc);
                s[tt] = acc;
            }
            float mt = s[0];
#pragma unroll
            for (int tt = 1; tt < kSmallTJ; ++tt) mt = fmaxf(mt, s[tt]);
            const float mn = fmaxf(M, mt);
            float acc = S * ex2(M - mn);
#pragma unroll
            for (int tt = 0; tt < kSmallTJ; ++tt) acc += ex2(s[tt] - mn);
            S = acc;
            M = mn;
        }
    } else
    for (int base = 0; base < A.nk; base += kSmallTile) {
        __syncthreads();
        for (int e = threadIdx.x; e < kSmallTile * V; e += kBlock) {
            const int col = base + e / V, part = e % V;
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (col < A.nk) {
                v = kp[(size_t)col * V + part];
            } else if (part == D / 4) {
                reinterpret_cast<float*>(&v)[D % 4] = -INFINITY;
            }
            tile[e] = v;
        }
        __syncthreads();
        const int ntile = min(kSmallTile, A.nk - base);
        for (int t0 = 0; t0 < kSmallTile / kSmallG && kSmallG * t0 < ntile; t0 += kSmallTJ) {
            float s[kSmallTJ];
#pragma unroll
            for (int tt = 0; tt < kSmallTJ; ++tt) {
                float kk[P];
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    const float4 v = tile[(sub + kSmallG * (t0 + tt)) * V + u];
                    kk[4 * u + 0] = v.x;
                    kk[4 * u + 1] = v.y;
                    kk[4 * u + 2] = v.z;
                    kk[4 * u + 3] = v.w;
                }
                float acc = kk[D];
#pragma unroll
                for (int dd = 0; dd < D; ++dd) acc = fmaf(q[dd], kk[dd], acc);
                s[tt] = acc;
            }
            float mt = s[0];
#pragma unroll
            for (int tt = 1; tt < kSmallTJ; ++tt) mt = fmaxf(mt, s[tt]);
            const float mn = fmaxf(M, mt);
            float acc = S * ex2(M - mn);
#pragma unroll
            for (int tt = 0; tt < kSmallTJ; ++tt) acc += ex2(s[tt] - mn);
            S = acc;
            M = mn;
        }
    }
#pragma unroll
    for (int off = kSmallG / 2; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(M, off), s2 = __shfl_xor(S, off);
        const float mn = fmaxf(M, m2);
        S = S * ex2(M - mn) + s2 * ex2(m2 - mn);
        M = mn;
    }
    if (sub == 0 && i < A.nq) finalize(A.fin, i, M + lg2(S), pre);
}

// Combines, for every row of a row block split across workgroups, the partial
// (M, S) pairs: M = max M_w, S = sum S_w 2^{M_w - M}.  kMergeLanes lanes share
// a row, each taking every kMergeLanes-th contributing workgroup, then a fixed
// xor-shuffle tree joins them (the order is fixed, so results are repeatable).
constexpr int kMergeLanes = 8;

//
// A wave's 64 lanes hold 64 / kMergeLanes consecutive rows from a multiple of
// that count, and a row block (rpb rows, a multiple of it) never splits such a
// group, so the row block and its range bookkeeping are wave-uniform: taken
// from the first lane, they are computed once per wave on the scalar unit
// instead of as 64-bit divisions in every lane. Of the ranges that meet the
// block only the first, wf, can start before it (the owner of u0 is the last
// range starting at or before u0), so its range start decides the one slot
// that is not 0.
static_assert(kPassRows % kMergeLanes == 0 && 64 % kMergeLanes == 0, "a lane group never splits a row block");

__global__ __launch_bounds__(kBlock) void k_merge(PassArgs A) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int i = t / kMergeLanes, sub = t % kMergeLanes;
    const bool live = i < A.nq;
    const int ic = live ? i : A.nq - 1;
    const int rb = __builtin_amdgcn_readfirstlane(ic / A.rpb), lr = ic - rb * A.rpb;
    const int64_t u0 = (int64_t)rb * A.nk, u1 = u0 + A.nk;
    const int wf = range_owner(u0, A.total, A.W), wl = range_owner(u1 - 1, A.total, A.W);
    const bool first_starts_before = range_lo(wf, A.total, A.W) < u0;
    // the row's finalisation inputs, loaded now so that their latency overlaps the partials' loads
    const FinIn pre = fin_load(A.fin, ic);
    float M = kNegBig, S = 0.0f;
    for (int w = wf + sub; w <= wl; w += kMergeLanes) {
        const int slot = (w == wf && first_starts_before) ? 1 : 0;
        const float2 p = A.part[((size_t)w * 2 + slot) * A.rpb + lr];
        const float mn = fmaxf(M, p.x);
        S = S * ex2(M - mn) + p.y * ex2(p.x - mn);
        M = mn;
    }
#pragma unroll
    for (int off = kMergeLanes / 2; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(M, off), s2 = __shfl_xor(S, off);
        const float mn = fmaxf(M, m2);
        S = S * ex2(M - mn) + s2 * ex2(m2 - mn);
        M = mn;
    }
    // a row block held whole by one workgroup was finished by the pass itself
    if (live && sub == 0 && wf != wl) finalize(A.fin, i, M + lg2(S), pre);
}

// Gradient pass: the same traversal with the running weighted key sum
// A_i = sum_j 2^{s_ij - M_i} k_j (rescaled with S on every max change);
// grad_i = 2 a_i (x~_i - A_i / S_i), where x~ and k are centred alike.
template <int D>
__global__ __launch_bounds__(kBlock) void k_grad_valu(GradArgs A) {
    constexpr int P = ((D + 1 + 3) / 4) * 4;
    constexpr int V = P / 4;
    __shared__ float4 tile[kTL * V];

    const int split = blockIdx.y;
    const int row0 = blockIdx.x * (kBlock * kR) + threadIdx.x;

    float q[kR][D];
    float M[kR], S[kR], Acc[kR][D];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int i = row0 + r * kBlock;
        const int ic = i < A.nq ? i : A.nq - 1;
        const float* qr = A.q + (size_t)ic * P;
#pragma unroll
        for (int t = 0; t < D; ++t) {
            q[r][t] = qr[t] * A.qscale;
            Acc[r][t] = 0.0f;
        }
        M[r] = kNegBig;
        S[r] = 0.0f;
    }

    const int c0 = split * A.cols_per_split;
    const int c1 = min(c0 + A.cols_per_split, A.nk);
    const float4* kp = reinterpret_cast<const float4*>(A.k);

    for (int base = c0; base < c1; base += kTL) {
        __syncthreads();
        stage_tile<D>(tile, kp, base, c1);
        __syncthreads();
        const int ntile = min(kTL, c1 - base);
        for (int c = 0; c < ntile; c += kTJ) {
            float kk[kTJ][P];
#pragma unroll
            for (int t = 0; t < kTJ; ++t)
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    const float4 v = tile[(c + t) * V + u];
                    kk[t][4 * u + 0] = v.x;
                    kk[t][4 * u + 1] = v.y;
                    kk[t][4 * u + 2] = v.z;
                    kk[t][4 * u + 3] = v.w;
                }
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                float s[kTJ];
#pragma unroll
                for (int t = 0; t < kTJ; ++t) {
                    float acc = kk[t][D];
#pragma unroll
                    for (int dd = 0; dd < D; ++dd) acc = fmaf(q[r][dd], kk[t][dd], acc);
                    s[t] = acc;
                }
                float mt = s[0];
#pragma unroll
                for (int t = 1; t < kTJ; ++t) mt = fmaxf(mt, s[t]);
                const float mn = fmaxf(M[r], mt);
                const float sc = ex2(M[r] - mn);
                float acc = S[r] * sc;
#pragma unroll
                for (int dd = 0; dd < D; ++dd) Acc[r][dd] *= sc;
#pragma unroll
                for (int t = 0; t < kTJ; ++t) {
                    const float e = ex2(s[t] - mn);
                    acc += e;
#pragma unroll
                    for (int dd = 0; dd < D; ++dd) Acc[r][dd] = fmaf(e, kk[t][dd], Acc[r][dd]);
                }
                S[r] = acc;
                M[r] = mn;
            }
        }
    }

#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int i = row0 + r * kBlock;
        if (i >= A.nq) continue;
        if (A.nsplit == 1) {
            const float two_w = 2.0f * A.w[i];
            const float inv = 1.0f / S[r];
#pragma unroll
            for (int dd = 0; dd < D; ++dd)
                A.grad[(size_t)i * D + dd] = two_w * (A.q[(size_t)i * P + dd] - Acc[r][dd] * inv);
        } else {
            A.part[(size_t)split * A.nq + i] = make_float2(M[r], S[r]);
            float* pa = A.partA + ((size_t)split * A.nq + i) * P;
#pragma unroll
            for (int dd = 0; dd < D; ++dd) pa[dd] = Acc[r][dd];
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_grad_merge(GradArgs A) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= A.nq) return;
    float M = kNegBig;
    for (int s = 0; s < A.nsplit; ++s) M = fmaxf(M, A.part[(size_t)s * A.nq + i].x);
    float S = 0.0f;
    float acc[kMaxD > 8 ? 8 : kMaxD];
    for (int dd = 0; dd < A.d; ++dd) acc[dd] = 0.0f;
    for (int s = 0; s < A.nsplit; ++s) {
        const float2 p = A.part[(size_t)s * A.nq + i];
        const float sc = ex2(p.x - M);
        S += p.y * sc;
        const float* pa = A.partA + ((size_t)s * A.nq + i) * A.P;
        for (int dd = 0; dd < A.d; ++dd) acc[dd] += pa[dd] * sc;
    }
    const float two_w = 2.0f * A.w[i];
    const float inv = 1.0f / S;
    for (int dd = 0; dd < A.d; ++dd)
        A.grad[(size_t)i * A.d + dd] = two_w * (A.q[(size_t)i * A.P + dd] - acc[dd] * inv);
}

template <int D>
hipError_t launch_pass_d(const PassArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.small) {
        SK_LAUNCH_TIMED(k_pass_small<D>, dim3((a.nq + kSmallRows - 1) / kSmallRows), dim3(kBlock), s, ev0, ev1, a);
        return hipGetLastError();
    }
    SK_LAUNCH_TIMED(k_pass_valu<D>, dim3(a.W), dim3(kBlock), s, ev0, ev1, a);
    return launch_merge(a, s);
}

template <int D>
int capacity_d() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pass_valu<D>, kBlock, 0) != hipSuccess) return 0;
    return cus * per_cu;
}

template <int D>
hipError_t launch_grad_d(const GradArgs& a, hipStream_t s) {
    const int rpb = kBlock * kR;
    dim3 grid((a.nq + rpb - 1) / rpb, a.nsplit);
    hipLaunchKernelGGL(k_grad_valu<D>, grid, dim3(kBlock), 0, s, a);
    if (a.nsplit > 1)
        hipLaunchKernelGGL(k_grad_merge, dim3((a.nq + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int valu_rows_per_block() { return kPassRows; }
int valu_block_rows() { return kBlock * kR; }

hipError_t launch_merge(const PassArgs& a, hipStream_t s) {
    if (a.rpb % (64 / kMergeLanes) != 0) return hipErrorInvalidValue;  // k_merge takes a wave's row block as uniform
    const int64_t n_row_blocks = a.total / a.nk;
    if (a.W > n_row_blocks || a.total % a.W != 0 || (a.total / a.W) % a.nk != 0)
        hipLaunchKernelGGL(k_merge, dim3(((int64_t)a.nq * kMergeLanes + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}


int valu_pass_capacity(int d) {
    switch (d) {
        case 1: return capacity_d<1>();
        case 2: return capacity_d<2>();
        case 3: return capacity_d<3>();
        case 4: return capacity_d<4>();
        case 5: return capacity_d<5>();
        case 6: return capacity_d<6>();
        case 7: return capacity_d<7>();
        case 8: return capacity_d<8>();
        default: return 0;
    }
}

hipError_t launch_pass_valu(const PassArgs& a, int d, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (d) {
        case 1: return launch_pass_d<1>(a, s, ev0, ev1);
        case 2: return launch_pass_d<2>(a, s, ev0, ev1);
        case 3: return launch_pass_d<3>(a, s, ev0, ev1);
        case 4: return launch_pass_d<4>(a, s, ev0, ev1);
        case 5: return launch_pass_d<5>(a, s, ev0, ev1);
        case 6: return launch_pass_d<6>(a, s, ev0, ev1);
        case 7: return launch_pass_d<7>(a, s, ev0, ev1);
        case 8: return launch_pass_d<8>(a, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_sparse_d(const SparseArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    SK_LAUNCH_TIMED(k_pass_sparse<D>, dim3(a.W), dim3(kBlock), s, ev0, ev1, a);
    hipLaunchKernelGGL(k_sparse_merge, dim3((a.nq + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pass_sparse(const SparseArgs& a, int d, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (a.B < 1 || a.B > kBlock * kR || a.W < 1 || !a.part || a.nqb != (a.nq + a.B - 1) / a.B)
        return hipErrorInvalidValue;
    switch (d) {
        case 1: return launch_sparse_d<1>(a, s, ev0, ev1);
        case 2: return launch_sparse_d<2>(a, s, ev0, ev1);
        case 3: return launch_sparse_d<3>(a, s, ev0, ev1);
        case 4: return launch_sparse_d<4>(a, s, ev0, ev1);
        case 5: return launch_sparse_d<5>(a, s, ev0, ev1);
        case 6: return launch_sparse_d<6>(a, s, ev0, ev1);
        case 7: return launch_sparse_d<7>(a, s, ev0, ev1);
        case 8: return launch_sparse_d<8>(a, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_grad_valu(const GradArgs& a, hipStream_t s) {
    switch (a.d) {
        case 1: return launch_grad_d<1>(a, s);
        case 2: return launch_grad_d<2>(a, s);
        case 3: return launch_grad_d<3>(a, s);
        case 4: return launch_grad_d<4>(a, s);
        case 5: return launch_grad_d<5>(a, s);
        case 6: return launch_grad_d<6>(a, s);
        case 7: return launch_grad_d<7>(a, s);
        case 8: return launch_grad_d<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sk

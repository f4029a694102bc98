// sk_pass_mfma.hip -- streamed log-sum-exp passes with the cross term on
// matrix cores (9 <= d <= 256).
//
// The score of a (query, key) pair is s_ij = <q_i, k_j> + h_j (base 2, see
// sk_internal.hpp): a dense contraction over the padded dimension P, followed
// by a per-row online log-sum-exp ("FlashSinkhorn: IO-Aware Entropic Optimal
// Transport on GPU", Methodology 1-2: biased dot-product scores, streamed
// tiles, running max / sum-exp, no materialisation).
//
// Mapping to CDNA4 (wave64, D = A B + C, keys as A, queries as B):
//  * lane l = 16 g + c; D is 16 keys x 16 queries with lane l holding keys
//    4g..4g+3 of query c, for both instructions used here:
//    v_mfma_f32_16x16x4f32 (lane: key / query c, k slot g) and
//    v_mfma_f32_16x16x32_f16 (lane: key / query c, k slots 8g..8g+7);
//  * the contraction index is permuted so that lane group g owns the
//    contiguous coordinate range [g P/4, (g+1) P/4). Each lane keeps its
//    query's split coordinates in registers for a whole segment
//    (row-stationary) and reads its key's from a padded LDS tile;
//  * the accumulator starts at the key biases, so the bias add is free;
//  * each lane runs an online (M, S) over the keys it sees; the four lane
//    groups that share a query are merged with two cross-lane exchanges at
//    the end of a segment;
//  * NQB independent 16-query blocks per wave interleave their MFMA chains.
// Work is split across workgroups with the same stream-K ranges as the vector
// passes; a row block here is 4 waves x NQB x 16 queries.
//
// The solver pass and every transport mode (the d > 8 gradient among them)
// take the cross term on fp16 matrix cores from a scaled two-part split of
// every fp32 coordinate, within a few fp32 unit roundoffs per term (split2,
// split_scores).  The weighted sums of the payload modes 0, 1 and 4 take the
// same split form up to P = 128 (weights and payload in two fp16 parts each);
// MODE 2 and P = 256 keep fp32 matrix instructions for them.
#include "sk_internal.hpp"
#include "sk_pass_common.hpp"

#include <algorithm>
#include <cfloat>
#include <type_traits>

namespace sk {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kBlock / 64;

#ifndef SK_MFMA_NQB
#define SK_MFMA_NQB 4
#endif

// 16-query blocks per wave (register budget: NQB * P / 4 query VGPRs)
template <int P>
constexpr int mfma_nqb() {
    return P <= 64 ? SK_MFMA_NQB : (P == 128 ? 2 : 1);
}

// Register staging of one fp32 LDS tile of TL keys (coordinates only; the
// payload modes read a key's coordinates as their second operand): each
// thread holds F4 float4s.  Loads are unconditional (clamped to the last valid
// key) and issued back to back, so a tile costs one memory latency, and the
// loads for the next tile are issued before the current tile is computed.
template <int P, int TL>
struct TileStageF {
    static constexpr int F4 = TL * (P / 4) / kBlock;
    static_assert(TL * (P / 4) % kBlock == 0, "tile must split evenly over the workgroup");
    float4 v[F4];

    __device__ __forceinline__ void load(const float4* __restrict__ kp, int base, int j1) {
#pragma unroll
        for (int r = 0; r < F4; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / (P / 4), part = e - key * (P / 4);
            const int col = base + key;
            const float4 x = kp[(size_t)min(col, j1 - 1) * (P / 4) + part];
            v[r] = col < j1 ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

    __device__ __forceinline__ void store(float* ktile) const {
        constexpr int PS = P + 4;
#pragma unroll
        for (int r = 0; r < F4; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / (P / 4), part = e - key * (P / 4);
            *reinterpret_cast<float4*>(&ktile[key * PS + part * 4]) = v[r];
        }
    }
};

// Row stride (halves) of a transposed split key tile of TL keys: a multiple of
// 4, so that a lane group's 4 keys are one 8-byte read, padded so that the 16
// rows a wave reads at once start in different banks.
template <int TL>
constexpr int ysplit_stride() {
    return TL + 8;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

#ifndef SK_MFMA2_TILE
#define SK_MFMA2_TILE 4096
#endif

// ---- two-part fp16 split of scaled fp32 values
//
// Both clouds are scaled by rq = fl(sqrt(2 log2e / eps)), so that the score's
// cross term <q, k> = (2 log2e / eps) <x~, y~> is the product of the two
// scaled clouds, and each cloud once more by a power of two 2^e chosen from
// its largest scaled magnitude (split_exp), so that its operands lie below
// 2^14, within fp16's range and near its top. One split per cloud and solve
// then serves it as queries in one half-step and as keys in the other.
// Then v = h + l with h = fp16(v) and l = fp16(v - h), both rounded to
// nearest even: the remainder v - h is exact
// in fp32 and |v - h - l| <= 2^-22 |v| + 2^-25, the second term from fp16's
// subnormal spacing (it matters only for |v| below about 2^-3 at the scaled
// size, against largest operands of 2^13 to 2^14). The score takes
// hq hk + hq lk + lq hk: each product of two fp16 values is
// exact in fp32, the matrix cores add in fp32, and the dropped product lq lk
// is below 2^-22 |q_t k_t|. This is the fp16 splitting of Ootomo and Yokota
// ("Recovering single precision accuracy from Tensor Cores while surpassing
// the FP32 theoretical peak performance", IJHPCA 2022), with a common scale
// per side in place of their per-part scaling. Its error per term is a few
// fp32 unit roundoffs (2^-22 against 2^-24). One v_mfma_f32_16x16x32_f16
// (16 keys x 16 queries x 32 coordinates) runs at the bf16 rate, 16x the
// fp32 matrix rate, so the three products of 32 coordinates take 3/16 of the
// matrix-core time of the eight fp32 steps they replace.
//
// The matrix cores then return 2^(eq + ek) times the score (the key biases
// are scaled the same way when a tile is staged); the log-sum-exp takes the
// scale off inside its exponent with one fma, fma(D, r, -M r), r = 2^-(eq+ek).
// Each scaled coordinate carries one rounding, and rq^2 is 2 log2e / eps to
// within an fp32 roundoff, the same order as the rounding of an unsplit
// fl(x~ 2 log2e / eps).

// The exponent e that puts the largest magnitude mx at mx 2^e in [2^13, 2^14)
// (0 for a zero or non-finite mx).
__device__ __forceinline__ int split_exp(float mx) {
    if (!(mx > 0.0f) || !(mx <= FLT_MAX)) return 0;
    int e;
    (void)frexpf(mx, &e);  // mx = f 2^e, f in [0.5, 1)
    return 14 - e;
}

// The power-of-two exponent of a cloud whose largest |coordinate| is cmax,
// scaled by rq. Capped at 48, so that the score scale 2^(eq + ek) stays at
// most 2^96 and staged biases up to 2^32 in magnitude stay finite. The cap
// binds only for a cloud whose scaled coordinates all lie below 2^-34; its
// parts then carry an absolute error of at most 2^-73 beside the relative
// 2^-22, for each coordinate of it.
__device__ __forceinline__ int cloud_exp(float cmax, float rq) { return min(split_exp(cmax * rq), 48); }

// The scales of one pass: query parts are those of fl(v rq) 2^eq, key parts
// those of fl(v rq) 2^ek (each cloud's own exponent).
struct SplitScale {
    float t;   // 2^(eq + ek): score scale of the matrix-core results and staged biases
    float r;   // 2^-(eq + ek)
    float m0;  // running-max start, kNegBig min(t, 1), so that -m0 r stays finite
};

__device__ __forceinline__ SplitScale split_scale(const float* qmax, const float* kmax, float rq) {
    const int e = cloud_exp(*qmax, rq) + cloud_exp(*kmax, rq);
    SplitScale z;
    z.t = ldexpf(1.0f, e);
    z.r = ldexpf(1.0f, -e);
    z.m0 = z.t < 1.0f ? kNegBig * z.t : kNegBig;
    return z;
}

__device__ __forceinline__ unsigned f16_bits(float x) {
    return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)x);
}
__device__ __forceinline__ float f16_value(unsigned h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}
__device__ __forceinline__ void split2(float v, unsigned& h, unsigned& l) {
    h = f16_bits(v);
    l = f16_bits(v - f16_value(h));
}

// ---- the weighted sums of the key-payload transports in the split form
//
// The key coordinates are split once per launch by k_split_cols_t into fp16
// parts times 2^ey (payload_exp: the cloud's largest |coordinate| into
// [2^13, 2^14), capped so that 2^ey and 2^-(ey + kWScaleExp) stay normal
// floats), transposed in blocks of 32 keys: kt[(j / 32) 2P + part P + t][j % 32],
// keys past nk zero.  A workgroup stages a tile of them with plain 16-byte
// copies (TileStageT) into yt[part P + t][key] (rows YS halves apart).
__device__ __forceinline__ int payload_exp(const float* kmax) { return min(split_exp(*kmax), 100); }

// The general payload of mode 0 takes the same layout with KA columns (zero
// past its kin) and a power of two per column, from that column's largest
// magnitude (k_col_absmax), so a column of small values keeps its precision.
__global__ __launch_bounds__(kBlock) void k_split_cols_t(const float* __restrict__ v, int nk, int ld, int ncols,
                                                         int KA, const float* __restrict__ cmax, int per_col,
                                                         uint16_t* __restrict__ kt) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nkp = (int64_t)(nk + kTransColAlign - 1) / kTransColAlign * kTransColAlign;
    if (e >= nkp * KA) return;
    // 32 consecutive threads take the 32 keys of one block at one column: each wave writes two 64-byte runs
    const int jj = (int)(e % kTransColAlign);
    const int64_t rest = e / kTransColAlign;
    const int t = (int)(rest % KA);
    const int64_t blk = rest / KA;
    const int64_t j = blk * kTransColAlign + jj;
    unsigned h = 0, l = 0;
    if (j < nk && t < ncols) split2(v[j * ld + t] * ldexpf(1.0f, payload_exp(per_col ? cmax + t : cmax)), h, l);
    kt[((blk * 2) * KA + t) * kTransColAlign + jj] = (uint16_t)h;
    kt[((blk * 2 + 1) * KA + t) * kTransColAlign + jj] = (uint16_t)l;
}

// Largest |v[j ld + t]| over the nk rows of each column t < ncols (0 for
// ncols <= t < KS; out cleared to 0 first).  Thread x takes column x % KS of
// every (kBlock / KS)-th row, so a wave reads whole rows; each workgroup then
// folds its row lanes and adds its maxima with an integer atomicMax on the
// bits of the non-negative floats, which orders them as the floats (the
// result does not depend on the order of the workgroups).
__global__ __launch_bounds__(kBlock) void k_col_absmax(const float* __restrict__ v, int nk, int ld, int ncols, int KS,
                                                       unsigned* __restrict__ out) {
    __shared__ float sh[kBlock];
    const int c = threadIdx.x % KS, r0 = threadIdx.x / KS, rstep = kBlock / KS;
    float mx = 0.0f;
    if (c < ncols)
        for (int j = blockIdx.x * rstep + r0; j < nk; j += gridDim.x * rstep)
            mx = fmaxf(mx, fabsf(v[(size_t)j * ld + c]));
    sh[threadIdx.x] = mx;
    __syncthreads();
    if (r0 == 0) {
        for (int r = 1; r < rstep; ++r) mx = fmaxf(mx, sh[r * KS + c]);
        atomicMax(out + c, __float_as_uint(mx));
    }
}

// Register staging of one tile of TL keys of the transposed parts of P
// columns (TL a multiple of 32, the tile's first key a multiple of 32): TL / 32
// blocks of 2P rows of 32 halves (four 16-byte units each).  Blocks past the
// array read as zero; keys past the segment inside a block carry weight 0.
template <int P, int TL>
struct TileStageT {
    static constexpr int UNITS = TL / 32 * 2 * P * 4;
    static constexpr int U = (UNITS + kBlock - 1) / kBlock;  // the last round may be partial (16 columns, P = 128)
    static_assert(TL % 32 == 0 && (UNITS % kBlock == 0 || UNITS < kBlock), "tile must split over the workgroup");
    u4v v[U];

    __device__ __forceinline__ void load(const u4v* __restrict__ kt, int base, int nk) {
        const int nblk = (nk + 31) / 32;
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int e = threadIdx.x + r * kBlock;
            if (UNITS % kBlock != 0 && e >= UNITS) continue;
            const int blk = e / (2 * P * 4), rem = e - blk * (2 * P * 4);
            const int b = base / 32 + blk;
            const u4v x = kt[((size_t)min(b, nblk - 1) * 2 * P) * 4 + rem];
            v[r] = b < nblk ? x : u4v{0u, 0u, 0u, 0u};
        }
    }

    __device__ __forceinline__ void store(uint16_t* yt) const {
        constexpr int YS = ysplit_stride<TL>();
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int e = threadIdx.x + r * kBlock;
            if (UNITS % kBlock != 0 && e >= UNITS) continue;
            const int blk = e / (2 * P * 4), rem = e - blk * (2 * P * 4);
            const int row = rem / 4, q = rem - row * 4;
            *reinterpret_cast<u4v*>(yt + row * YS + blk * 32 + q * 8) = v[r];
        }
    }
};

// Whether a transport mode takes its weighted sums in the split form: the
// key-payload modes and the general payload (mode 0) up to P = 128 (a key tile
// then holds at least 32 keys); not MODE 2, whose weights carry a signed factor.
constexpr bool split_sums(int P, int MODE) { return (MODE == 0 || MODE == 1 || MODE == 4) && P <= 128; }

// The parts of packed rows: out[i][part][t] (parts h, l) of fl(in[i][t] rq) 2^e,
// e = cloud_exp of the cloud's largest |coordinate| *cmax.
__global__ __launch_bounds__(kBlock) void k_split2(const float* __restrict__ in, int64_t count, int P,
                                                   const float* __restrict__ cmax, float rq,
                                                   uint16_t* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= count) return;
    const float sc = ldexpf(1.0f, cloud_exp(*cmax, rq));
    const int64_t i = e / P;
    const int t = (int)(e - i * P);
    unsigned h, l;
    split2((in[e] * rq) * sc, h, l);
    uint16_t* o = out + i * 2 * P + t;
    o[0] = (uint16_t)h;
    o[P] = (uint16_t)l;
}

// The largest |value| of each of two packed clouds: per-block maxima
// (blockIdx.y picks the cloud), then one workgroup joins them.
__global__ __launch_bounds__(kBlock) void k_absmax_part(const float4* __restrict__ x4, int64_t nx4,
                                                        const float4* __restrict__ y4, int64_t ny4,
                                                        float* __restrict__ part) {
    const float4* v = blockIdx.y == 0 ? x4 : y4;
    const int64_t cnt = blockIdx.y == 0 ? nx4 : ny4;
    float mx = 0.0f;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < cnt; e += (int64_t)gridDim.x * kBlock) {
        const float4 w = v[e];
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w))));
    }
    __shared__ float red[kBlock];
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kBlock) void k_absmax_final(const float* __restrict__ part, int nb,
                                                         float* __restrict__ out) {
    __shared__ float red[kBlock];
    for (int side = 0; side < 2; ++side) {
        float mx = 0.0f;
        for (int e = threadIdx.x; e < nb; e += kBlock) mx = fmaxf(mx, part[side * nb + e]);
        red[threadIdx.x] = mx;
        __syncthreads();
        for (int off = kBlock / 2; off > 0; off >>= 1) {
            if ((int)threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
            __syncthreads();
        }
        if (threadIdx.x == 0) out[side] = red[0];
        __syncthreads();
    }
}

// keys per LDS tile of the split pass (SK_MFMA2_TILE coordinates: 2 x 2 bytes each)
template <int P>
constexpr int mfma2_tile_keys() {
    return SK_MFMA2_TILE / P < 16 ? 16 : SK_MFMA2_TILE / P;
}

// Register staging of one LDS tile of split keys: a key row is RU 16-byte
// units (h, l parts of P coordinates), stored RU + 1 apart in LDS, an odd
// number of units, so 16 lanes reading 16 rows at one offset do not conflict.
// The key biases are staged times the pass's score scale t.
template <int P>
struct TileStage2 {
    static constexpr int TL = mfma2_tile_keys<P>();
    static constexpr int RU = P / 4;
    static constexpr int RS = RU + 1;
    static constexpr int U = TL * RU / kBlock;
    static constexpr int NB = (TL + kBlock - 1) / kBlock;
    static_assert(TL * RU % kBlock == 0, "tile must split evenly over the workgroup");
    static_assert(RS % 2 == 1, "odd row stride in 16-byte units");
    u4v v[U];
    float b[NB];

    __device__ __forceinline__ void load(const u4v* __restrict__ kb, const float* __restrict__ kbias, float t,
                                         int base, int j1) {
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / RU, part = e - key * RU;
            const int col = base + key;
            const u4v x = kb[(size_t)min(col, j1 - 1) * RU + part];
            v[r] = col < j1 ? x : u4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int col = base + threadIdx.x + r * kBlock;
            const float x = kbias[min(col, j1 - 1)];
            b[r] = col < j1 ? x * t : -INFINITY;
        }
    }

    __device__ __forceinline__ void store(u4v* ktile, float* btile) const {
#pragma unroll
        for (int r = 0; r < U; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / RU, part = e - key * RU;
            ktile[key * RS + part] = v[r];
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int k = threadIdx.x + r * kBlock;
            if (k < TL) btile[k] = b[r];
        }
    }
};

__device__ __forceinline__ f4 mfma_f16(const u4v a, const u4v b, const f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// Query operands per lane in the split form: P >= 32 keeps one (h, l) pair of
// 8-coordinate chunks per chunk; P = 16 (4 coordinates per lane group, half an
// operand) keeps two ready operands, (h, h) and (l, l).
template <int P>
constexpr int split_qops() {
    return P >= 32 ? P / 32 : 1;
}

// A lane's query operands for the split form, from the query's row of split
// parts (parts h, l, P/8 16-byte units apart; the same layout and lane-group
// map as a key row). P >= 32: chunk kc of qh, ql holds the h, l parts of
// coordinates 8 kc .. 8 kc + 7 of the lane group. P = 16: qh = (h, h),
// ql = (l, l) over the lane group's 4 coordinates, the B operands of
// split_scores<16>.
template <int P>
__device__ __forceinline__ void load_query_parts(const u4v* __restrict__ row, int g, u4v (&qh)[split_qops<P>()],
                                                 u4v (&ql)[split_qops<P>()]) {
    if constexpr (P == 16) {
        const uint2* r2 = reinterpret_cast<const uint2*>(row);
        const uint2 h = r2[g], l = r2[4 + g];
        qh[0] = u4v{h.x, h.y, h.x, h.y};
        ql[0] = u4v{l.x, l.y, l.x, l.y};
    } else {
        constexpr int KC = P / 32;
        const u4v* kr = row + g * KC;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            qh[kc] = kr[kc];
            ql[kc] = kr[P / 8 + kc];
        }
    }
}

// Scores (times the pass's scale t) of one 16-key block for NQB query blocks
// in the split form: row is the lane's key row in the LDS tile (parts h, l,
// P/8 units apart) and g its lane group. P >= 32: three products per
// 8-coordinate chunk. P = 16: the lane group's 4 coordinates fill half an
// operand, so A = (kh, kl) against B = (qh, qh) and then (ql, ql) gives all
// four products in two instructions. With four query blocks the four
// accumulator chains keep the matrix pipe busy; with fewer, the small products
// go to a second accumulator per block (from zero).
template <int P, int NQB>
__device__ __forceinline__ void split_scores(const u4v* row, int g, const u4v (&qh)[NQB][split_qops<P>()],
                                             const u4v (&ql)[NQB][split_qops<P>()], const f4 bias,
                                             f4 (&acc)[NQB]) {
    constexpr bool kTwoAcc = NQB < 4;
    f4 acc2[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        acc[qb] = bias;
        acc2[qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    f4(&small)[NQB] = kTwoAcc ? acc2 : acc;
    if constexpr (P == 16) {
        // 8 bytes per part and lane group: part p at uint2 index 4 p + g of the row
        const uint2* r2 = reinterpret_cast<const uint2*>(row);
        const uint2 kh = r2[g], kl = r2[4 + g];
        const u4v a = {kh.x, kh.y, kl.x, kl.y};
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_f16(a, qh[qb][0], acc[qb]);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_f16(a, ql[qb][0], small[qb]);
    } else {
        constexpr int KC = P / 32;
        const u4v* kr = row + g * KC;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u4v kh = kr[kc], kl = kr[P / 8 + kc];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_f16(kh, qh[qb][kc], acc[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_f16(kh, ql[qb][kc], small[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_f16(kl, qh[qb][kc], acc[qb]);
        }
    }
    if constexpr (kTwoAcc) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[qb] += acc2[qb];
    }
}

// A lane's KT key coordinates of one 16-key block, from the padded LDS tile.
template <int KT>
__device__ __forceinline__ void load_keys(float (&kf)[KT], const float* ktile, int off) {
    const float4* kr = reinterpret_cast<const float4*>(&ktile[off]);
#pragma unroll
    for (int t4 = 0; t4 < KT / 4; ++t4) {
        const float4 v = kr[t4];
        kf[4 * t4 + 0] = v.x;
        kf[4 * t4 + 1] = v.y;
        kf[4 * t4 + 2] = v.z;
        kf[4 * t4 + 3] = v.w;
    }
}

// The larger of two scores, NaN-propagating (IEEE 754-2019 maximum). On
// gfx950 this is v_maximum3_f32, which takes three operands and reads matrix
// results as they are; fmaxf, whose NaN rule drops a quiet NaN, first quiets
// each matrix result with one v_max_f32 of its own (nine instructions for the
// nine candidates of one update instead of four).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Online log-sum-exp over the four scores a lane holds for one 16-key block.
// Scores, M and the candidates are in the pass's scaled units (times t); the
// exponents are taken back to base-2 units with one fma each, fma(x, r, -mn r)
// = (x - mn) r rounded once, the same value as x r - mn r of unscaled scores.
// M starts at SplitScale::m0, so -mn r is finite and an empty key set gives
// fma(-inf, r, finite) = -inf, never inf - inf.
__device__ __forceinline__ void lse_block(float& M, float& S, const f4 acc, float r) {
    const float mn = vmax3(vmax3(acc[0], acc[1], acc[2]), acc[3], M);
    const float nm = -mn * r;
    float s = S * ex2(fmaf(M, r, nm));
#pragma unroll
    for (int v = 0; v < 4; ++v) s += ex2(fmaf(acc[v], r, nm));
    S = s;
    M = mn;
}

// The same over the eight scores of two 16-key blocks (one rescale for both).
__device__ __forceinline__ void lse_block2(float& M, float& S, const f4 a, const f4 b, float r) {
    const float mn = vmax3(vmax3(a[0], a[1], a[2]), vmax3(a[3], b[0], b[1]), vmax3(b[2], b[3], M));
    const float nm = -mn * r;
    float s = S * ex2(fmaf(M, r, nm));
#pragma unroll
    for (int v = 0; v < 4; ++v) s += ex2(fmaf(a[v], r, nm));
#pragma unroll
    for (int v = 0; v < 4; ++v) s += ex2(fmaf(b[v], r, nm));
    S = s;
    M = mn;
}

__device__ __forceinline__ void lse_merge(float& M, float& S, float m2, float s2, float r) {
    const float mn = vmax(M, m2);
    const float nm = -mn * r;
    S = S * ex2(fmaf(M, r, nm)) + s2 * ex2(fmaf(m2, r, nm));
    M = mn;
}

// The solver pass: the cross term on fp16 matrix cores from the two-part
// split (both clouds split in memory by k_split2; a lane loads its query's
// parts once per segment and keeps them in registers). Lane group g owns the
// coordinates [g P/4, (g+1) P/4).
// Waves per SIMD the solver pass is compiled for: four at P = 16 (128 VGPRs)
// and P = 256, three otherwise (165 VGPRs at P = 64, where the compiler left
// alone takes 175 and two). No spills at any P; at 16384^2 d = 16 and 32 ran
// 2% faster than without the bound, d = 64 the same.
template <int P>
constexpr int pass_waves() {
    return (P == 16 || P == 256) ? 4 : 3;
}

template <int P>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(pass_waves<P>()))) void k_pass_mfma(
    PassArgs A) {
    constexpr int KQ = split_qops<P>();  // query operands per part
    constexpr int NQB = mfma_nqb<P>();   // 16-query blocks per wave
    using Stage = TileStage2<P>;
    constexpr int TL = Stage::TL;
    constexpr int RS = Stage::RS;
    __shared__ u4v ktile[TL * RS];
    __shared__ __align__(16) float btile[TL];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const u4v* kb = reinterpret_cast<const u4v*>(A.kb);
    const u4v* qbp = reinterpret_cast<const u4v*>(A.qb);
    const SplitScale sc = split_scale(A.qmax, A.kmax, A.rq);

    const int w = xcd_range(blockIdx.x, A.W);
    const int64_t lo = range_lo(w, A.total, A.W), hi = range_lo(w + 1, A.total, A.W);
    for (int64_t u = lo; u < hi;) {
        const int rb = (int)(u / A.nk);
        const int j0 = (int)(u - (int64_t)rb * A.nk);
        const int j1 = (int)min<int64_t>((int64_t)A.nk, (int64_t)j0 + (hi - u));
        const int qrow0 = rb * A.rpb + wave * (NQB * 16);

        // queries, scaled, as h, l parts
        u4v qh[NQB][KQ], ql[NQB][KQ];
        float M[NQB], S[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int i = qrow0 + qb * 16 + c;
            const int ic = i < A.nq ? i : A.nq - 1;
            load_query_parts<P>(qbp + (size_t)ic * (P / 4), g, qh[qb], ql[qb]);
            M[qb] = sc.m0;
            S[qb] = 0.0f;
        }

        Stage stage;
        stage.load(kb, A.kbias, sc.t, j0, j1);
        for (int base = j0; base < j1; base += TL) {
            __syncthreads();
            stage.store(ktile, btile);
            __syncthreads();
            if (base + TL < j1) stage.load(kb, A.kbias, sc.t, base + TL, j1);
            const int ntile = min(TL, j1 - base);
            if constexpr (TL >= 32) {
                // two 16-key blocks per step, one rescale for both (3.5% faster at d = 64 than one block per
                // step); rows past the segment's keys hold bias -inf and add nothing
                for (int kb32 = 0; kb32 < ntile; kb32 += 32) {
                    const f4 bias0 = *reinterpret_cast<const f4*>(&btile[kb32 + 4 * g]);
                    const f4 bias1 = *reinterpret_cast<const f4*>(&btile[kb32 + 16 + 4 * g]);
                    f4 acc0[NQB], acc1[NQB];
                    split_scores<P, NQB>(ktile + (kb32 + c) * RS, g, qh, ql, bias0, acc0);
                    split_scores<P, NQB>(ktile + (kb32 + 16 + c) * RS, g, qh, ql, bias1, acc1);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) lse_block2(M[qb], S[qb], acc0[qb], acc1[qb], sc.r);
                }
            } else {
                for (int kb16 = 0; kb16 < ntile; kb16 += 16) {
                    const f4 bias = *reinterpret_cast<const f4*>(&btile[kb16 + 4 * g]);
                    f4 acc[NQB];
                    split_scores<P, NQB>(ktile + (kb16 + c) * RS, g, qh, ql, bias, acc);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) lse_block(M[qb], S[qb], acc[qb], sc.r);
                }
            }
        }

        // the four lane groups hold disjoint key subsets of the same queries
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            lse_merge(M[qb], S[qb], __shfl_xor(M[qb], 16), __shfl_xor(S[qb], 16), sc.r);
            lse_merge(M[qb], S[qb], __shfl_xor(M[qb], 32), __shfl_xor(S[qb], 32), sc.r);
        }
        const bool complete = (j0 == 0 && j1 == A.nk);
        float2* slot = A.part + ((size_t)w * 2 + (u == lo ? 0 : 1)) * A.rpb;
        if (g == 0) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int i = qrow0 + qb * 16 + c;
                if (i >= A.nq) continue;
                const float mu = M[qb] * sc.r;  // the running max in base-2 units (exact: a power-of-two scale)
                if (complete)
                    finalize(A.fin, i, mu + lg2(S[qb]));
                else
                    slot[wave * (NQB * 16) + qb * 16 + c] = make_float2(mu, S[qb]);
            }
        }
        u += j1 - j0;
    }
}

// Transport products for d > 8 (see sk_transport.hip for the d <= 8 kernel and
// the quantities).  w_ij = 2^{s_ij - lse_i} <= 1 with lse from a first pass
// over the same scores, and the payload sums accumulate with a second matrix
// contraction over the keys whose A operand is the lane's own weights (eight
// fp16 parts per 32 keys in the split form, four fp32 values per 16 keys
// otherwise):
//   T_i[col] = sum_j w_ij psi_j[col],   P psi = 2^{lse_i + h_i} T_i,
//   row mass = 2^{lse_i + h_i} sum_j w_ij.
//  MODE 0: psi_j = NP payload columns (16 * NP, zero-padded);
//  MODE 1: psi_j = the key's coordinates;
//  MODE 2: the key's coordinates with w_ij (pay_j + <y~_j, 2 v_i>), the inner
//          product taken on fp32 matrix instructions like the weighted sums;
//  MODE 3: one payload column, summed with four vector FMAs per lane and
//          16 keys (a 16-column MFMA tile would be 15/16 padding);
//  MODE 4: the gradient in x at fixed g: T_i as in MODE 1, then
//          grad_i = 2 a_i (x~_i - T_i / S_i), S_i = sum_j w_ij (the plan's
//          barycentric map; the plan scale cancels).
// Every mode forms its scores in the fp16 split form of the solver pass (same
// helpers and scales).  The weighted sums of MODES 0, 1 and 4 up to P = 128
// take the fp16 split form too (split_sums: weights and payload as two fp16
// parts each, three products, the payload split per launch by k_split_cols_t);
// MODE 2 and P = 256 keep fp32 matrix instructions, the key coordinates read
// from an fp32 key tile and a general payload from an fp32 payload tile.
// 16-query blocks per wave of the transport kernel: their MFMA chains
// interleave, at a register cost of NQB * P / 8 query VGPRs plus NQB output
// tiles.
// Exponent of the power of two the split weighted sums scale their weights by:
// a weight w <= 1 becomes w 2^14 <= 2^14, within fp16's range, and the parts of
// weights down to 2^-28 stay normal fp16 numbers (smaller ones add at most
// 2^-39 each in absolute terms).
constexpr int kWScaleExp = 14;

constexpr int transport_nqb(int P, int NP, int MODE) {
    // the one-column kernel: 4 blocks, 151 against 171 us with 2 at 16384^2, d = 64 (bf16 split form); an
    // HVP at d = 16 4.93 against 5.18 ms
    const int base = ((MODE == 0 && NP > 1) || MODE == 3) ? 4 : 2;
    return P <= 64 ? base : (P == 128 ? base / 2 : 1);
}

template <int P, int NP, int MODE>
__global__ __launch_bounds__(kBlock) void k_transport_mfma(TransArgs A) {
    constexpr int KT = P / 4;
    constexpr int KQ = split_qops<P>();
    constexpr int PS = P + 4;
    constexpr bool KEYS = MODE == 1 || MODE == 2 || MODE == 4;  // the fp32 key coordinates are an operand
    constexpr int NB = KEYS ? P / 16 : NP;                       // 16-column output blocks (unused in MODE 3)
    constexpr int KP = MODE == 0 ? 16 * NP : 1;                  // payload floats per key in LDS
    using Stage = TileStage2<P>;
    using FStage = TileStageF<P, Stage::TL>;
    constexpr int TL = Stage::TL;
    constexpr int RS = Stage::RS;
    constexpr int NQB = transport_nqb(P, NP, MODE);
    // Modes whose payload is the key cloud (1, 4) take the weighted sums on fp16
    // matrix instructions too, up to P = 128: weights and key coordinates as
    // two fp16 parts each (three products), 32 keys per step.
    constexpr bool SPLITW = split_sums(P, MODE);
    static_assert(!SPLITW || TL >= 32, "the split weighted sums take 32 keys per step");
    constexpr int YS = ysplit_stride<TL>();
    constexpr int KA = KEYS ? P : 16 * NP;                        // columns of the weighted sums
    constexpr bool PAY = (MODE == 0 && !SPLITW) || MODE == 2 || MODE == 3;  // an fp32 payload tile
    __shared__ u4v ktile[TL * RS];
    __shared__ __align__(16) float ftile[KEYS && !SPLITW ? TL * PS : 1];
    __shared__ __align__(16) uint16_t ytile[SPLITW ? 2 * KA * YS : 1];
    __shared__ __align__(16) float btile[TL];
    __shared__ __align__(16) float ptile[PAY ? TL * KP : 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const u4v* kb = reinterpret_cast<const u4v*>(A.kb);
    const int split = blockIdx.y;
    const int c0 = split * A.cols_per_split;
    const int c1 = min(c0 + A.cols_per_split, A.nk);
    const int qrow0 = blockIdx.x * (kWaves * 16 * NQB) + wave * (16 * NQB);
    // scores come back times sc.t (key biases staged the same way)
    const SplitScale sc = split_scale(A.qmax, A.kmax, A.rq);
    const u4v* qbp = reinterpret_cast<const u4v*>(A.qb);
    // SPLITW: the key coordinates come split times 2^ey (k_split_cols_t) and the
    // weights are split times 2^kWScaleExp, exact scalings taken off T and S
    // before the epilogue
    const int ey = SPLITW && KEYS ? payload_exp(A.kmax) : 0;
    const u4v* ktp = reinterpret_cast<const u4v*>(A.kt);
    const float wofs = SPLITW ? (float)kWScaleExp : 0.0f;

    float vf[MODE == 2 ? NQB : 1][KT];
    u4v qh[NQB][KQ], ql[NQB][KQ];
    float lse_c[NQB], S[NQB], Tv[NQB];
    f4 T[NQB][NB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int i = qrow0 + qb * 16 + c;
        const int ic = i < A.nq ? i : A.nq - 1;
        load_query_parts<P>(qbp + (size_t)ic * (P / 4), g, qh[qb], ql[qb]);
        if (MODE == 2) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int dim = g * KT + t;
                vf[MODE == 2 ? qb : 0][t] = dim < A.d ? 2.0f * A.rowv[(size_t)ic * A.d + dim] : 0.0f;
            }
        }
        lse_c[qb] = A.lse[ic] - wofs;
        S[qb] = 0.0f;
        Tv[qb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) T[qb][nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    Stage stage;
    FStage fstage;
    struct NoStage {};
    std::conditional_t<SPLITW, TileStageT<KA, TL>, NoStage> tstage;
    if (c0 < c1) {
        stage.load(kb, A.kbias, sc.t, c0, c1);
        if constexpr (SPLITW)
            tstage.load(ktp, c0, A.nk);
        else if constexpr (KEYS)
            fstage.load(kp, c0, c1);
    }
    for (int base = c0; base < c1; base += TL) {
        __syncthreads();
        stage.store(ktile, btile);
        if constexpr (SPLITW)
            tstage.store(ytile);
        else if constexpr (KEYS)
            fstage.store(ftile);
        if constexpr (PAY)
            for (int e = threadIdx.x; e < TL * KP; e += kBlock) {
                const int col = base + e / KP;
                const int cc = e % KP;
                ptile[e] = (col < c1 && cc < A.kin) ? A.pay[(size_t)col * A.ldp + cc] : 0.0f;
            }
        __syncthreads();
        if (base + TL < c1) {
            stage.load(kb, A.kbias, sc.t, base + TL, c1);
            if constexpr (SPLITW)
                tstage.load(ktp, base + TL, A.nk);
            else if constexpr (KEYS)
                fstage.load(kp, base + TL, c1);
        }
        const int ntile = min(TL, c1 - base);
        if constexpr (SPLITW) {
            // Two 16-key blocks per step.  Contraction slot 8g + e of the weighted
            // sums is key 4g + e of the first block (e < 4) and 16 + 4g + e - 4 of
            // the second: the A operand is the lane's own eight weights (query c),
            // the B operand 8 of those keys' parts of one coordinate, two 8-byte
            // runs of the transposed tile.  Keys past the segment hold bias -inf,
            // weight 0.
            for (int k0 = 0; k0 < ntile; k0 += 32) {
                f4 acc0[NQB], acc1[NQB];
                const f4 bias0 = *reinterpret_cast<const f4*>(&btile[k0 + 4 * g]);
                const f4 bias1 = *reinterpret_cast<const f4*>(&btile[k0 + 16 + 4 * g]);
                split_scores<P, NQB>(ktile + (k0 + c) * RS, g, qh, ql, bias0, acc0);
                split_scores<P, NQB>(ktile + (k0 + 16 + c) * RS, g, qh, ql, bias1, acc1);
                u4v wh[NQB], wl[NQB];
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    float wv8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = e < 4 ? acc0[qb][e] : acc1[qb][e - 4];
                        wv8[e] = ex2(fmaf(x, sc.r, -lse_c[qb]));  // the weight times 2^kWScaleExp
                        S[qb] += wv8[e];
                    }
                    // the parts of split2, two weights per packed conversion (v_cvt_pk_f16_f32, rounding to
                    // nearest even): h = fp16(w), l = fp16(w - h)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const f2v p = {wv8[2 * j], wv8[2 * j + 1]};
                        const h2v hp = __builtin_convertvector(p, h2v);
                        const h2v lp = __builtin_convertvector(p - __builtin_convertvector(hp, f2v), h2v);
                        wh[qb][j] = __builtin_bit_cast(unsigned, hp);
                        wl[qb][j] = __builtin_bit_cast(unsigned, lp);
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const uint16_t* rh = ytile + (nb * 16 + c) * YS + k0 + 4 * g;
                    const uint16_t* rl = rh + KA * YS;
                    const uint2 h0 = *reinterpret_cast<const uint2*>(rh), h1 = *reinterpret_cast<const uint2*>(rh + 16);
                    const uint2 l0 = *reinterpret_cast<const uint2*>(rl), l1 = *reinterpret_cast<const uint2*>(rl + 16);
                    const u4v yh = {h0.x, h0.y, h1.x, h1.y}, yl = {l0.x, l0.y, l1.x, l1.y};
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) T[qb][nb] = mfma_f16(wh[qb], yh, T[qb][nb]);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) T[qb][nb] = mfma_f16(wh[qb], yl, T[qb][nb]);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) T[qb][nb] = mfma_f16(wl[qb], yh, T[qb][nb]);
                }
            }
            continue;
        }
        for (int kb16 = 0; kb16 < ntile; kb16 += 16) {
            const f4 bias = *reinterpret_cast<const f4*>(&btile[kb16 + 4 * g]);
            f4 acc[NQB], dv[NQB];
            split_scores<P, NQB>(ktile + (kb16 + c) * RS, g, qh, ql, bias, acc);
            if constexpr (MODE == 2) {
                float kf[KT];
                load_keys<KT>(kf, ftile, (kb16 + c) * PS + g * KT);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) dv[qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
                        dv[qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], vf[MODE == 2 ? qb : 0][t], dv[qb], 0, 0,
                                                                      0);
            }
            float wv[NQB][4];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float w = ex2(fmaf(acc[qb][v], sc.r, -lse_c[qb]));
                    S[qb] += w;
                    if constexpr (MODE == 2)
                        wv[qb][v] = w * (ptile[kb16 + 4 * g + v] + dv[qb][v]);
                    else
                        wv[qb][v] = w;
                }
            if constexpr (MODE == 3) {
                // one payload column: four FMAs per lane beat a 16-column MFMA tile
                const f4 pv = *reinterpret_cast<const f4*>(&ptile[kb16 + 4 * g]);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) Tv[qb] = fmaf(wv[qb][v], pv[v], Tv[qb]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float b = MODE == 0 ? ptile[(kb16 + 4 * g + v) * KP + nb * 16 + c]
                                                  : ftile[(kb16 + 4 * g + v) * PS + nb * 16 + c];
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb)
                            T[qb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[qb][v], b, T[qb][nb], 0, 0, 0);
                    }
            }
        }
    }
    static_assert(KA == 16 * NB, "one 16-column block per output tile");
    if constexpr (SPLITW) {
        // take off the exact scalings: weights 2^kWScaleExp, payload 2^ey (mode 0:
        // per column, this lane's column nb 16 + c)
        const float rw = ldexpf(1.0f, -kWScaleExp);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int e = MODE == 0 ? payload_exp(A.pmax + nb * 16 + c) : ey;
            const float rt = ldexpf(1.0f, -kWScaleExp - e);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) T[qb][nb] *= rt;
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) S[qb] *= rw;
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int q0 = qrow0 + qb * 16;
        // S: lane (g, c) summed keys 4g.. of query c; join the four groups
        float Sq = S[qb];
        Sq += __shfl_xor(Sq, 16);
        Sq += __shfl_xor(Sq, 32);
        float Tq = Tv[qb];
        if (MODE == 3) {
            Tq += __shfl_xor(Tq, 16);
            Tq += __shfl_xor(Tq, 32);
        }
        if (A.nsplit == 1 && MODE == 4) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int qi = 4 * g + v;        // query of T[qb][nb][v] in this lane
                const float Si = __shfl(Sq, qi);  // lane qi holds query qi's sum
                const int i = q0 + qi;
                if (i >= A.nq) continue;
                const float two_w = 2.0f * A.gw[i];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int dim = nb * 16 + c;
                    if (dim < A.kout)
                        A.out[(size_t)i * A.ldo + dim] = two_w * (A.q[(size_t)i * P + dim] - T[qb][nb][v] / Si);
                }
            }
        } else if (A.nsplit == 1) {
            if (g == 0 && q0 + c < A.nq) {
                const int i = q0 + c;
                const float scale = ex2(A.lse[i] + A.qbias[i]);
                if (A.mass) A.mass[i] = Sq * scale;
                if (MODE == 3) A.out[(size_t)i * A.ldo] = Tq * scale;
            }
#pragma unroll
            for (int v = 0; v < 4 && MODE != 3; ++v) {
                const int i = q0 + 4 * g + v;
                if (i >= A.nq) continue;
                const float scale = ex2(A.lse[i] + A.qbias[i]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int col = nb * 16 + c;
                    if (col < A.kout) A.out[(size_t)i * A.ldo + col] = T[qb][nb][v] * scale;
                }
            }
        } else {
            if (g == 0 && q0 + c < A.nq) {
                A.part[(size_t)split * A.nq + q0 + c] = make_float2(0.0f, Sq);
                if (MODE == 3) A.partA[((size_t)split * A.nq + q0 + c) * KA] = Tq;
            }
#pragma unroll
            for (int v = 0; v < 4 && MODE != 3; ++v) {
                const int i = q0 + 4 * g + v;
                if (i >= A.nq) continue;
                float* pa = A.partA + ((size_t)split * A.nq + i) * KA;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) pa[nb * 16 + c] = T[qb][nb][v];
            }
        }
    }
}

// Sums the split partials (S, T) in split order, then applies the plan scale.
__global__ __launch_bounds__(kBlock) void k_transport_mfma_merge(TransArgs A, int KA) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cols = A.kout + 1;  // the payload columns, then the row mass
    if (t >= (int64_t)A.nq * cols) return;
    const int i = (int)(t / cols), col = (int)(t - (int64_t)i * cols);
    const float scale = ex2(A.lse[i] + A.qbias[i]);
    float acc = 0.0f;
    if (col < A.kout) {
        for (int s = 0; s < A.nsplit; ++s) acc += A.partA[((size_t)s * A.nq + i) * KA + col];
        A.out[(size_t)i * A.ldo + col] = acc * scale;
    } else if (A.mass) {
        for (int s = 0; s < A.nsplit; ++s) acc += A.part[(size_t)s * A.nq + i].y;
        A.mass[i] = acc * scale;
    }
}

// MODE 4 with a split key range: sums the partials (S, T) in split order and
// writes grad_i = 2 a_i (x~_i - T_i / S_i).
__global__ __launch_bounds__(kBlock) void k_transport_grad_merge(TransArgs A) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)A.nq * A.kout) return;
    const int i = (int)(t / A.kout), dim = (int)(t - (int64_t)i * A.kout);
    float S = 0.0f, T = 0.0f;
    for (int s = 0; s < A.nsplit; ++s) {
        S += A.part[(size_t)s * A.nq + i].y;
        T += A.partA[((size_t)s * A.nq + i) * A.P + dim];
    }
    A.out[(size_t)i * A.ldo + dim] = 2.0f * A.gw[i] * (A.q[(size_t)i * A.P + dim] - T / S);
}

template <int P, int NP, int MODE>
hipError_t launch_transport_mfma_p(const TransArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int KA = (MODE == 1 || MODE == 2 || MODE == 4) ? P : 16 * NP;
    constexpr int rpb = kWaves * 16 * transport_nqb(P, NP, MODE);
    // the split keys and the clouds' largest magnitudes are written by every set-up
    if (!a.kb || !a.qb || !a.qmax || !a.kmax) return hipErrorInvalidValue;
    if (MODE == 4 && (!a.gw || a.kout > P)) return hipErrorInvalidValue;
    if constexpr (split_sums(P, MODE)) {
        // the split weighted sums stage whole 32-key blocks: every key split starts on a block
        if (!a.kt || (a.nsplit > 1 && a.cols_per_split % kTransColAlign != 0)) return hipErrorInvalidValue;
        constexpr int KS = MODE == 0 ? 16 * NP : P;  // columns of the split payload (<= P)
        const int64_t elems = (int64_t)(a.nk + kTransColAlign - 1) / kTransColAlign * kTransColAlign * KS;
        const dim3 sgrid((unsigned)((elems + kBlock - 1) / kBlock));
        if constexpr (MODE == 0) {
            if (!a.pay || !a.pmax || a.kin < 1 || a.kin > KS) return hipErrorInvalidValue;
            static_assert(kBlock % KS == 0, "whole row lanes per workgroup");
            const int rows = kBlock / KS;
            const int gblocks = (int)std::min<int64_t>(256, ((int64_t)a.nk + rows - 1) / rows);
            if (launch_fill(a.pmax, KS, 0.0f, s) != hipSuccess) return hipGetLastError();
            hipLaunchKernelGGL(k_col_absmax, dim3(gblocks), dim3(kBlock), 0, s, a.pay, a.nk, a.ldp, a.kin, KS,
                               reinterpret_cast<unsigned*>(a.pmax));
            hipLaunchKernelGGL(k_split_cols_t, sgrid, dim3(kBlock), 0, s, a.pay, a.nk, a.ldp, a.kin, KS,
                               (const float*)a.pmax, 1, a.kt);
        } else {
            hipLaunchKernelGGL(k_split_cols_t, sgrid, dim3(kBlock), 0, s, a.k, a.nk, P, P, P, a.kmax, 0, a.kt);
        }
    }
    dim3 grid((a.nq + rpb - 1) / rpb, a.nsplit);
    SK_LAUNCH_TIMED((k_transport_mfma<P, NP, MODE>), grid, dim3(kBlock), s, ev0, ev1, a);
    if (a.nsplit > 1 && MODE == 4)
        hipLaunchKernelGGL(k_transport_grad_merge, dim3((unsigned)(((int64_t)a.nq * a.kout + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, s, a);
    else if (a.nsplit > 1)
        hipLaunchKernelGGL(k_transport_mfma_merge, dim3((unsigned)(((int64_t)a.nq * (a.kout + 1) + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, s, a, KA);
    return hipGetLastError();
}

template <int P>
hipError_t launch_transport_mfma_pp(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0,
                                    hipEvent_t ev1) {
    if (mode == 1) return launch_transport_mfma_p<P, 1, 1>(a, s, ev0, ev1);
    if (mode == 2) return launch_transport_mfma_p<P, 1, 2>(a, s, ev0, ev1);
    if (mode == 3) return launch_transport_mfma_p<P, 1, 3>(a, s, ev0, ev1);
    if (mode == 4) return launch_transport_mfma_p<P, 1, 4>(a, s, ev0, ev1);
    if (kwidth == 16) return launch_transport_mfma_p<P, 1, 0>(a, s, ev0, ev1);
    if constexpr (P >= 64) {  // a 64-column payload tile fits LDS beside the key tile from P = 64 on
        if (kwidth == 64) return launch_transport_mfma_p<P, 4, 0>(a, s, ev0, ev1);
    }
    return hipErrorInvalidValue;
}

template <int P>
hipError_t launch_mfma_p(const PassArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    // the split keys and the clouds' largest magnitudes are written by every solver set-up
    if (!a.kb || !a.qb || !a.qmax || !a.kmax) return hipErrorInvalidValue;
    SK_LAUNCH_TIMED(k_pass_mfma<P>, dim3(a.W), dim3(kBlock), s, ev0, ev1, a);
    return launch_merge(a, s);
}

template <int P, int NP, int MODE>
int capacity_tp() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_transport_mfma<P, NP, MODE>, kBlock, 0) != hipSuccess)
        return 0;
    return cus * per_cu;
}

template <int P>
int capacity_tpp(int mode, int kwidth) {
    if (mode == 1) return capacity_tp<P, 1, 1>();
    if (mode == 2) return capacity_tp<P, 1, 2>();
    if (mode == 3) return capacity_tp<P, 1, 3>();
    if (mode == 4) return capacity_tp<P, 1, 4>();
    if (kwidth == 16) return capacity_tp<P, 1, 0>();
    if constexpr (P >= 64) {
        if (kwidth == 64) return capacity_tp<P, 4, 0>();
    }
    return 0;
}

template <int P>
int capacity_p() {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pass_mfma<P>, kBlock, 0) != hipSuccess)
        return 0;
    return cus * per_cu;
}

}  // namespace

int mfma_rows_per_block(int P) {
    switch (P) {
        case 16: return kWaves * mfma_nqb<16>() * 16;
        case 32: return kWaves * mfma_nqb<32>() * 16;
        case 64: return kWaves * mfma_nqb<64>() * 16;
        case 128: return kWaves * mfma_nqb<128>() * 16;
        case 256: return kWaves * mfma_nqb<256>() * 16;
        default: return 0;
    }
}

hipError_t launch_pass_mfma(const PassArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    switch (a.P) {
        case 16: return launch_mfma_p<16>(a, s, ev0, ev1);
        case 32: return launch_mfma_p<32>(a, s, ev0, ev1);
        case 64: return launch_mfma_p<64>(a, s, ev0, ev1);
        case 128: return launch_mfma_p<128>(a, s, ev0, ev1);
        case 256: return launch_mfma_p<256>(a, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

int mfma_grad_rows_per_block(int P) { return kWaves * 16 * transport_nqb(P, 1, 4); }

int mfma_transport_rows_per_block(int P, int mode, int kwidth) {
    return kWaves * 16 * transport_nqb(P, kwidth > 16 ? 4 : 1, mode);
}

int mfma_transport_capacity(int P, int mode, int kwidth) {
    switch (P) {
        case 16: return capacity_tpp<16>(mode, kwidth);
        case 32: return capacity_tpp<32>(mode, kwidth);
        case 64: return capacity_tpp<64>(mode, kwidth);
        case 128: return capacity_tpp<128>(mode, kwidth);
        case 256: return capacity_tpp<256>(mode, kwidth);
        default: return 0;
    }
}

int mfma_transport_max_rows_per_block(int P) {
    int r = 0;
    for (int mode = 0; mode <= 4; ++mode)
        for (int kw : {16, 64}) r = std::max(r, mfma_transport_rows_per_block(P, mode, kw));
    return r;
}

hipError_t launch_transport_mfma(const TransArgs& a, int mode, int kwidth, hipStream_t s, hipEvent_t ev0,
                                 hipEvent_t ev1) {
    switch (a.P) {
        case 16: return launch_transport_mfma_pp<16>(a, mode, kwidth, s, ev0, ev1);
        case 32: return launch_transport_mfma_pp<32>(a, mode, kwidth, s, ev0, ev1);
        case 64: return launch_transport_mfma_pp<64>(a, mode, kwidth, s, ev0, ev1);
        case 128: return launch_transport_mfma_pp<128>(a, mode, kwidth, s, ev0, ev1);
        case 256: return launch_transport_mfma_pp<256>(a, mode, kwidth, s, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split2(const float* in, int64_t rows, int P, const float* cmax, float rq, uint16_t* out,
                         hipStream_t s) {
    const int64_t count = rows * P;
    hipLaunchKernelGGL(k_split2, dim3((unsigned)((count + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, in, count, P,
                       cmax, rq, out);
    return hipGetLastError();
}

hipError_t launch_absmax(const float* x, int64_t nx, const float* y, int64_t ny, float* part, float* out,
                         hipStream_t s) {
    if (nx % 4 != 0 || ny % 4 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_absmax_part, dim3(kAbsMaxBlocks, 2), dim3(kBlock), 0, s, reinterpret_cast<const float4*>(x),
                       nx / 4, reinterpret_cast<const float4*>(y), ny / 4, part);
    hipLaunchKernelGGL(k_absmax_final, dim3(1), dim3(kBlock), 0, s, part, kAbsMaxBlocks, out);
    return hipGetLastError();
}

int mfma_pass_capacity(int P) {
    switch (P) {
        case 16: return capacity_p<16>();
        case 32: return capacity_p<32>();
        case 64: return capacity_p<64>();
        case 128: return capacity_p<128>();
        case 256: return capacity_p<256>();
        default: return 0;
    }
}

}  // namespace sk

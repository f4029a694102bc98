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
//    v_mfma_f32_16x16x32_bf16 (lane: key / query c, k slots 8g..8g+7);
//  * the contraction index is permuted so that lane group g owns the
//    contiguous coordinate range [g P/4, (g+1) P/4). Each lane keeps its
//    query's coordinates in registers for the whole pass (row-stationary) and
//    reads its key's from a padded LDS tile;
//  * the accumulator starts at the key biases, so the bias add is free;
//  * each lane runs an online (M, S) over the keys it sees; the four lane
//    groups that share a query are merged with two cross-lane exchanges at
//    the end of a segment;
//  * NQB independent 16-query blocks per wave interleave their MFMA chains.
// Work is split across workgroups with the same stream-K ranges as the vector
// passes; a row block here is 4 waves x NQB x 16 queries.
//
// The solver pass and the one-column transport kernel take the cross term on
// bf16 matrix cores from a three-part split of every fp32 coordinate that is
// as exact as an fp32 dot product (split3, split_scores); the gradient and the
// payload-carrying transport modes use fp32 instructions.
#include "sk_internal.hpp"
#include "sk_pass_common.hpp"

#include <algorithm>
#include <type_traits>

namespace sk {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kBlock / 64;

#ifndef SK_MFMA_NQB
#define SK_MFMA_NQB 4
#endif
#ifndef SK_MFMA_TILE_FLOATS
#define SK_MFMA_TILE_FLOATS 8192
#endif

// 16-query blocks per wave (register budget: NQB * P / 4 query VGPRs)
template <int P>
constexpr int mfma_nqb() {
    return P <= 64 ? SK_MFMA_NQB : (P == 128 ? 2 : 1);
}

// keys per LDS tile (about SK_MFMA_TILE_FLOATS floats of coordinates)
template <int P>
constexpr int mfma_tile_keys() {
    return SK_MFMA_TILE_FLOATS / P < 16 ? 16 : SK_MFMA_TILE_FLOATS / P;
}

// Register staging of one LDS tile of TL keys: each thread holds kStageF4
// float4s of coordinates and up to kStageB biases.  Loads are unconditional
// (clamped to the last valid key) and issued back to back, so a tile costs one
// memory latency, and the loads for the next tile are issued before the
// current tile is computed.
template <int P>
struct TileStage {
    static constexpr int TL = mfma_tile_keys<P>();
    static constexpr int F4 = TL * (P / 4) / kBlock;
    static constexpr int NB = (TL + kBlock - 1) / kBlock;
    static_assert(TL * (P / 4) % kBlock == 0, "tile must split evenly over the workgroup");
    float4 v[F4];
    float b[NB];

    __device__ __forceinline__ void load(const float4* __restrict__ kp, const float* __restrict__ kbias, int base,
                                         int j1) {
#pragma unroll
        for (int r = 0; r < F4; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / (P / 4), part = e - key * (P / 4);
            const int col = base + key;
            const float4 x = kp[(size_t)min(col, j1 - 1) * (P / 4) + part];
            v[r] = col < j1 ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int col = base + threadIdx.x + r * kBlock;
            const float x = kbias[min(col, j1 - 1)];
            b[r] = col < j1 ? x : -INFINITY;
        }
    }

    __device__ __forceinline__ void store(float* ktile, float* btile) const {
        constexpr int PS = P + 4;
#pragma unroll
        for (int r = 0; r < F4; ++r) {
            const int e = threadIdx.x + r * kBlock;
            const int key = e / (P / 4), part = e - key * (P / 4);
            *reinterpret_cast<float4*>(&ktile[key * PS + part * 4]) = v[r];
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
            const int k = threadIdx.x + r * kBlock;
            if (k < TL) btile[k] = b[r];
        }
    }
};

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

#ifndef SK_MFMA3_TILE
#define SK_MFMA3_TILE 4096
#endif

// ---- three-part bf16 split of fp32 values
//
// v = h + m + l with h = bf16(v), m = bf16(v - h), l = bf16(v - h - m), each
// rounded to nearest even. The two remainders are exact in fp32 (each part is
// within a factor 2 of what it rounds), and |v - h - m - l| <= 2^-27 |v|. Then
//   q.k ~ hq hk + hq mk + mq hk + hq lk + lq hk + mq mk:
// every product of two bf16 values is exact in fp32, the matrix cores add in
// fp32, and the dropped products (m l, l m, l l) are below 2^-26 of
// |q_t k_t|, under the unit roundoff 2^-24 of an fp32 dot product. On gfx950
// one v_mfma_f32_16x16x32_bf16 (16 keys x 16 queries x 32 coordinates) costs
// half the issue time of one v_mfma_f32_16x16x4f32 (the bf16 rate is 16x the
// fp32 rate), so the six products of 32 coordinates take 3/8 of the
// matrix-core time of the eight fp32 steps they replace.
__device__ __forceinline__ unsigned bf16_rne(float x) {  // finite x
    unsigned u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_value(unsigned h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ void split3(float v, unsigned& h, unsigned& m, unsigned& l) {
    h = bf16_rne(v);
    const float r = v - bf16_value(h);
    m = bf16_rne(r);
    l = bf16_rne(r - bf16_value(m));
}

// The parts of packed rows: out[i][part][t] (parts h, m, l) from in[i][t].
__global__ __launch_bounds__(kBlock) void k_split3(const float* __restrict__ in, int64_t count, int P,
                                                   uint16_t* __restrict__ out) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= count) return;
    const int64_t i = e / P;
    const int t = (int)(e - i * P);
    unsigned h, m, l;
    split3(in[e], h, m, l);
    uint16_t* o = out + i * 3 * P + t;
    o[0] = (uint16_t)h;
    o[P] = (uint16_t)m;
    o[2 * P] = (uint16_t)l;
}

// keys per LDS tile of the split pass (SK_MFMA3_TILE coordinates: 3 x 2 bytes each)
template <int P>
constexpr int mfma3_tile_keys() {
    return SK_MFMA3_TILE / P < 16 ? 16 : SK_MFMA3_TILE / P;
}

// Register staging of one LDS tile of split keys: a key row is RU 16-byte
// units (h, m, l parts of P coordinates), stored RU + 1 apart in LDS, an odd
// number of units, so 16 lanes reading 16 rows at one offset do not conflict.
template <int P>
struct TileStage3 {
    static constexpr int TL = mfma3_tile_keys<P>();
    static constexpr int RU = 3 * P / 8;
    static constexpr int RS = RU + 1;
    static constexpr int U = TL * RU / kBlock;
    static constexpr int NB = (TL + kBlock - 1) / kBlock;
    static_assert(TL * RU % kBlock == 0, "tile must split evenly over the workgroup");
    u4v v[U];
    float b[NB];

    __device__ __forceinline__ void load(const u4v* __restrict__ kb, const float* __restrict__ kbias, int base,
                                         int j1) {
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
            b[r] = col < j1 ? x : -INFINITY;
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

__device__ __forceinline__ f4 mfma_bf16(const u4v a, const u4v b, const f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0,
                                                   0);
}

// Query operands per lane in the split form: P >= 32 keeps one (h, m, l)
// triple of 8-coordinate chunks per chunk; P = 16 (4 coordinates per lane
// group, half an operand) keeps three ready operands that pair two parts each.
template <int P>
constexpr int split_qops() {
    return P >= 32 ? P / 32 : 1;
}

// A lane's query row for the split form, from its P/4 coordinates at qr,
// scaled. P >= 32: chunk kc of qh, qm, ql holds the h, m, l parts of
// coordinates 8 kc .. 8 kc + 7. P = 16: qh = (h, h), qm = (m, h), ql = (l, m)
// over the lane group's 4 coordinates, the B operands of the three products
// split_scores<16> forms.
template <int P>
__device__ __forceinline__ void load_query_split(const float* __restrict__ qr, float qscale,
                                                 u4v (&qh)[split_qops<P>()], u4v (&qm)[split_qops<P>()],
                                                 u4v (&ql)[split_qops<P>()]) {
    const float4* q4 = reinterpret_cast<const float4*>(qr);
    if constexpr (P == 16) {
        const float4 v = q4[0];
        const float x[4] = {v.x * qscale, v.y * qscale, v.z * qscale, v.w * qscale};
        unsigned hw[2], mw[2], lw[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            unsigned h0, m0, l0, h1, m1, l1;
            split3(x[2 * e], h0, m0, l0);
            split3(x[2 * e + 1], h1, m1, l1);
            hw[e] = h0 | (h1 << 16);
            mw[e] = m0 | (m1 << 16);
            lw[e] = l0 | (l1 << 16);
        }
        qh[0] = u4v{hw[0], hw[1], hw[0], hw[1]};
        qm[0] = u4v{mw[0], mw[1], hw[0], hw[1]};
        ql[0] = u4v{lw[0], lw[1], mw[0], mw[1]};
    } else {
#pragma unroll
        for (int t4 = 0; t4 < P / 16; ++t4) {
            const float4 v = q4[t4];
            const float x[4] = {v.x * qscale, v.y * qscale, v.z * qscale, v.w * qscale};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                unsigned h0, m0, l0, h1, m1, l1;
                split3(x[2 * e], h0, m0, l0);
                split3(x[2 * e + 1], h1, m1, l1);
                const int kc = t4 / 2, wd = 2 * (t4 % 2) + e;
                qh[kc][wd] = h0 | (h1 << 16);
                qm[kc][wd] = m0 | (m1 << 16);
                ql[kc][wd] = l0 | (l1 << 16);
            }
        }
    }
}

// Scores of one 16-key block for NQB query blocks in the split form: row is
// the lane's key row in the LDS tile (parts h, m, l, P/8 units apart) and g its
// lane group. P >= 32: six products per 8-coordinate chunk. P = 16: the lane
// group's 4 coordinates fill half an operand, so the six products go in pairs
// into three instructions, (h, m) x (h, h), (h, l) x (m, h), (h, m) x (l, m).
// With four query blocks the four accumulator chains keep the matrix pipe busy;
// with fewer, the small products go to a second accumulator per block (from
// zero).
template <int P, int NQB>
__device__ __forceinline__ void split_scores(const u4v* row, int g, const u4v (&qh)[NQB][split_qops<P>()],
                                             const u4v (&qm)[NQB][split_qops<P>()],
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
        const uint2 kh = r2[g], km = r2[4 + g], kl = r2[8 + g];
        const u4v a1 = {kh.x, kh.y, km.x, km.y}, a2 = {kh.x, kh.y, kl.x, kl.y};
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_bf16(a1, qh[qb][0], acc[qb]);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_bf16(a2, qm[qb][0], small[qb]);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_bf16(a1, ql[qb][0], acc[qb]);
    } else {
        constexpr int KC = P / 32;
        const u4v* kr = row + g * KC;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u4v kh = kr[kc], km = kr[P / 8 + kc], kl = kr[2 * (P / 8) + kc];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_bf16(kh, qh[qb][kc], acc[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_bf16(kh, ql[qb][kc], small[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_bf16(kh, qm[qb][kc], acc[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_bf16(kl, qh[qb][kc], small[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) acc[qb] = mfma_bf16(km, qh[qb][kc], acc[qb]);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) small[qb] = mfma_bf16(km, qm[qb][kc], small[qb]);
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

// Online log-sum-exp over the four scores a lane holds for one 16-key block.
__device__ __forceinline__ void lse_block(float& M, float& S, const f4 acc) {
    const float mt = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
    const float mn = fmaxf(M, mt);
    float s = S * ex2(M - mn);
    s += ex2(acc[0] - mn);
    s += ex2(acc[1] - mn);
    s += ex2(acc[2] - mn);
    s += ex2(acc[3] - mn);
    S = s;
    M = mn;
}

// The same over the eight scores of two 16-key blocks (one rescale for both).
__device__ __forceinline__ void lse_block2(float& M, float& S, const f4 a, const f4 b) {
    const float mt = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3])));
    const float mn = fmaxf(M, mt);
    float s = S * ex2(M - mn);
#pragma unroll
    for (int v = 0; v < 4; ++v) s += ex2(a[v] - mn);
#pragma unroll
    for (int v = 0; v < 4; ++v) s += ex2(b[v] - mn);
    S = s;
    M = mn;
}

__device__ __forceinline__ void lse_merge(float& M, float& S, float m2, float s2) {
    const float mn = fmaxf(M, m2);
    S = S * ex2(M - mn) + s2 * ex2(m2 - mn);
    M = mn;
}

// The solver pass: the cross term on bf16 matrix cores from the three-part
// split (keys split in memory by k_split3, queries split in registers when a
// segment starts). Lane group g owns the coordinates [g P/4, (g+1) P/4).
template <int P>
__global__ __launch_bounds__(kBlock) void k_pass_mfma(PassArgs A) {
    constexpr int KT = P / 4;            // coordinates per lane group
    constexpr int KQ = split_qops<P>();  // query operands per part
    constexpr int NQB = mfma_nqb<P>();   // 16-query blocks per wave
    using Stage = TileStage3<P>;
    constexpr int TL = Stage::TL;
    constexpr int RS = Stage::RS;
    __shared__ u4v ktile[TL * RS];
    __shared__ __align__(16) float btile[TL];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const u4v* kb = reinterpret_cast<const u4v*>(A.kb);

    const int w = blockIdx.x;
    const int64_t lo = range_lo(w, A.total, A.W), hi = range_lo(w + 1, A.total, A.W);
    for (int64_t u = lo; u < hi;) {
        const int rb = (int)(u / A.nk);
        const int j0 = (int)(u - (int64_t)rb * A.nk);
        const int j1 = (int)min<int64_t>((int64_t)A.nk, (int64_t)j0 + (hi - u));
        const int qrow0 = rb * A.rpb + wave * (NQB * 16);

        // queries, scaled, as h, m, l parts
        u4v qh[NQB][KQ], qm[NQB][KQ], ql[NQB][KQ];
        float M[NQB], S[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int i = qrow0 + qb * 16 + c;
            const int ic = i < A.nq ? i : A.nq - 1;
            load_query_split<P>(A.q + (size_t)ic * P + g * KT, A.qscale, qh[qb], qm[qb], ql[qb]);
            M[qb] = kNegBig;
            S[qb] = 0.0f;
        }

        Stage stage;
        stage.load(kb, A.kbias, j0, j1);
        for (int base = j0; base < j1; base += TL) {
            __syncthreads();
            stage.store(ktile, btile);
            __syncthreads();
            if (base + TL < j1) stage.load(kb, A.kbias, base + TL, j1);
            const int ntile = min(TL, j1 - base);
            if constexpr (TL >= 32) {
                // two 16-key blocks per step, one rescale for both (3.5% faster at d = 64 than one block per
                // step); rows past the segment's keys hold bias -inf and add nothing
                for (int kb32 = 0; kb32 < ntile; kb32 += 32) {
                    const f4 bias0 = *reinterpret_cast<const f4*>(&btile[kb32 + 4 * g]);
                    const f4 bias1 = *reinterpret_cast<const f4*>(&btile[kb32 + 16 + 4 * g]);
                    f4 acc0[NQB], acc1[NQB];
                    split_scores<P, NQB>(ktile + (kb32 + c) * RS, g, qh, qm, ql, bias0, acc0);
                    split_scores<P, NQB>(ktile + (kb32 + 16 + c) * RS, g, qh, qm, ql, bias1, acc1);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) lse_block2(M[qb], S[qb], acc0[qb], acc1[qb]);
                }
            } else {
                for (int kb16 = 0; kb16 < ntile; kb16 += 16) {
                    const f4 bias = *reinterpret_cast<const f4*>(&btile[kb16 + 4 * g]);
                    f4 acc[NQB];
                    split_scores<P, NQB>(ktile + (kb16 + c) * RS, g, qh, qm, ql, bias, acc);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) lse_block(M[qb], S[qb], acc[qb]);
                }
            }
        }

        // the four lane groups hold disjoint key subsets of the same queries
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            lse_merge(M[qb], S[qb], __shfl_xor(M[qb], 16), __shfl_xor(S[qb], 16));
            lse_merge(M[qb], S[qb], __shfl_xor(M[qb], 32), __shfl_xor(S[qb], 32));
        }
        const bool complete = (j0 == 0 && j1 == A.nk);
        float2* slot = A.part + ((size_t)w * 2 + (u == lo ? 0 : 1)) * A.rpb;
        if (g == 0) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int i = qrow0 + qb * 16 + c;
                if (i >= A.nq) continue;
                if (complete)
                    finalize(A.fin, i, M[qb] + lg2(S[qb]));
                else
                    slot[wave * (NQB * 16) + qb * 16 + c] = make_float2(M[qb], S[qb]);
            }
        }
        u += j1 - j0;
    }
}

// Gradient for d > 8: T_i = sum_j w_ij y_j with w_ij = 2^{s_ij - lse_i}, the
// row lse coming from a first streamed pass over the same scores (so every
// w_ij <= 1 and no rescaling is needed).  Per 16-key block the scores are
// recomputed on the matrix cores exactly as in the pass, and T accumulates
// with a second MFMA: A = weights (16 queries x 4 keys per step; a lane's own
// four weights, keys 4g + v, are exactly its A operand for steps v = 0..3),
// B = the block's key coordinates (4 keys x 16 dims, read from the LDS tile).
// The output tile of dims [16 nb, 16 nb + 16) leaves lane l holding
// T[query 4(l/16) + v][dim 16 nb + l%16].  grad_i = 2 a_i (x~_i - T_i / S_i)
// with S_i = sum_j w_ij (1 up to rounding).  One 16-query block per wave; the
// key range is split across workgroups (blockIdx.y) and partial (S, T) are
// plain sums.
template <int P>
__global__ __launch_bounds__(kBlock) void k_grad_mfma(GradArgs A) {
    constexpr int KT = P / 4;
    constexpr int PS = P + 4;
    constexpr int NB = P / 16;  // 16-dim output blocks
    constexpr int TL = mfma_tile_keys<P>();
    __shared__ __align__(16) float ktile[TL * PS];
    __shared__ __align__(16) float btile[TL];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const int split = blockIdx.y;
    const int c0 = split * A.cols_per_split;
    const int c1 = min(c0 + A.cols_per_split, A.nk);
    const int qrow0 = blockIdx.x * (kWaves * 16) + wave * 16;

    float qf[KT];
    {
        const int i = qrow0 + c;
        const int ic = i < A.nq ? i : A.nq - 1;
        const float4* qr = reinterpret_cast<const float4*>(A.q + (size_t)ic * P + g * KT);
#pragma unroll
        for (int t4 = 0; t4 < KT / 4; ++t4) {
            const float4 v = qr[t4];
            qf[4 * t4 + 0] = v.x * A.qscale;
            qf[4 * t4 + 1] = v.y * A.qscale;
            qf[4 * t4 + 2] = v.z * A.qscale;
            qf[4 * t4 + 3] = v.w * A.qscale;
        }
    }
    const float lse_c = A.lse[min(qrow0 + c, A.nq - 1)];
    float S = 0.0f;
    f4 T[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) T[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    TileStage<P> stage;
    if (c0 < c1) stage.load(kp, A.kbias, c0, c1);
    for (int base = c0; base < c1; base += TL) {
        __syncthreads();
        stage.store(ktile, btile);
        __syncthreads();
        if (base + TL < c1) stage.load(kp, A.kbias, base + TL, c1);
        const int ntile = min(TL, c1 - base);
        for (int kb = 0; kb < ntile; kb += 16) {
            float kf[KT];
            const float4* kr = reinterpret_cast<const float4*>(&ktile[(kb + c) * PS + g * KT]);
#pragma unroll
            for (int t4 = 0; t4 < KT / 4; ++t4) {
                const float4 v = kr[t4];
                kf[4 * t4 + 0] = v.x;
                kf[4 * t4 + 1] = v.y;
                kf[4 * t4 + 2] = v.z;
                kf[4 * t4 + 3] = v.w;
            }
            f4 acc = *reinterpret_cast<const f4*>(&btile[kb + 4 * g]);
#pragma unroll
            for (int t = 0; t < KT; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], qf[t], acc, 0, 0, 0);
            float wv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                wv[v] = ex2(acc[v] - lse_c);
                S += wv[v];
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    T[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[v], ktile[(kb + 4 * g + v) * PS + nb * 16 + c],
                                                                 T[nb], 0, 0, 0);
        }
    }
    // S: lane (g, c) summed keys 4g.. of query c; join the four groups
    S += __shfl_xor(S, 16);
    S += __shfl_xor(S, 32);
    if (A.nsplit == 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int qi = 4 * g + v;                 // query of T[nb][v] in this lane
            const float Sq = __shfl(S, qi);           // lane qi holds query qi's S
            const int i = qrow0 + qi;
            if (i >= A.nq) continue;
            const float two_w = 2.0f * A.w[i];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int dim = nb * 16 + c;
                if (dim < A.d) A.grad[(size_t)i * A.d + dim] = two_w * (A.q[(size_t)i * P + dim] - T[nb][v] / Sq);
            }
        }
    } else {
        if (g == 0 && qrow0 + c < A.nq) A.part[(size_t)split * A.nq + qrow0 + c] = make_float2(0.0f, S);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = qrow0 + 4 * g + v;
            if (i >= A.nq) continue;
            float* pa = A.partA + ((size_t)split * A.nq + i) * P;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) pa[nb * 16 + c] = T[nb][v];
        }
    }
}

// Sums the split partials (S, T) of the matrix-core gradient in split order.
__global__ __launch_bounds__(kBlock) void k_grad_mfma_merge(GradArgs A) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)A.nq * A.d) return;
    const int i = (int)(t / A.d), dim = (int)(t - (int64_t)i * A.d);
    float S = 0.0f, T = 0.0f;
    for (int s = 0; s < A.nsplit; ++s) {
        S += A.part[(size_t)s * A.nq + i].y;
        T += A.partA[((size_t)s * A.nq + i) * A.P + dim];
    }
    A.grad[t] = 2.0f * A.w[i] * (A.q[(size_t)i * A.P + dim] - T / S);
}

template <int P>
hipError_t launch_grad_mfma_p(const GradArgs& a, hipStream_t s) {
    dim3 grid((a.nq + kWaves * 16 - 1) / (kWaves * 16), a.nsplit);
    hipLaunchKernelGGL(k_grad_mfma<P>, grid, dim3(kBlock), 0, s, a);
    if (a.nsplit > 1)
        hipLaunchKernelGGL(k_grad_mfma_merge, dim3((unsigned)(((int64_t)a.nq * a.d + kBlock - 1) / kBlock)),
                           dim3(kBlock), 0, s, a);
    return hipGetLastError();
}


// Transport products for d > 8 (see sk_transport.hip for the d <= 8 kernel and
// the quantities).  As in the gradient, w_ij = 2^{s_ij - lse_i} <= 1 with lse
// from a first pass over the same scores, and the payload sums accumulate with
// a second MFMA whose A operand is the lane's own four weights:
//   T_i[col] = sum_j w_ij psi_j[col],   P psi = 2^{lse_i + h_i} T_i,
//   row mass = 2^{lse_i + h_i} sum_j w_ij.
//  MODE 0: psi_j = NP payload columns (16 * NP, zero-padded) staged in LDS;
//  MODE 1: psi_j = the key's coordinates (read from the key tile);
//  MODE 2: the key's coordinates with w_ij (pay_j + <y~_j, 2 v_i>), the inner
//          product taken on the matrix cores like the score;
//  MODE 3: one payload column, summed with four vector FMAs per lane and
//          16 keys (a 16-column MFMA tile would be 15/16 padding).
// 16-query blocks per wave of the transport kernel: their MFMA chains
// interleave, at a register cost of NQB * P / 4 query VGPRs plus NQB output
// tiles.  Measured at d = 64 (16384 x 16384): the 64-column product takes
// 1019 / 727 / 606 us with 1 / 2 / 4 blocks, the per-row-direction pass
// (MODE 2, 2 NQB P / 4 query VGPRs) 797 / 785 / 902 us, the single-column
// product 402 / 355 / 358 us.
constexpr int transport_nqb(int P, int NP, int MODE) {
    // the one-column kernel (split form): 4 blocks, 151 against 171 us with 2 at 16384^2, d = 64; an HVP
    // at d = 16 4.93 against 5.18 ms
    const int base = ((MODE == 0 && NP > 1) || MODE == 3) ? 4 : 2;
    return P <= 64 ? base : (P == 128 ? base / 2 : 1);
}

template <int P, int NP, int MODE>
__global__ __launch_bounds__(kBlock) void k_transport_mfma(TransArgs A) {
    // one payload column (MODE 3, the conjugate-gradient product) takes the split form from P = 32
    constexpr bool SPLIT = MODE == 3;
    constexpr int KT = P / 4;
    constexpr int KQ = split_qops<P>();
    constexpr int PS = P + 4;
    constexpr int NB = (MODE == 1 || MODE == 2) ? P / 16 : NP;  // 16-column output blocks (unused in MODE 3)
    constexpr int KP = MODE == 0 ? 16 * NP : 1;  // payload floats per key in LDS
    using Stage = std::conditional_t<SPLIT, TileStage3<P>, TileStage<P>>;
    constexpr int TL = Stage::TL;
    constexpr int NQB = transport_nqb(P, NP, MODE);
    constexpr int LDS_WORDS = SPLIT ? TL * TileStage3<P>::RS * 4 : TL * PS;
    __shared__ __align__(16) float ktile[LDS_WORDS];
    __shared__ __align__(16) float btile[TL];
    __shared__ __align__(16) float ptile[MODE == 1 ? 1 : TL * KP];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const float4* kp = reinterpret_cast<const float4*>(A.k);
    const u4v* kb = reinterpret_cast<const u4v*>(A.kb);
    const int split = blockIdx.y;
    const int c0 = split * A.cols_per_split;
    const int c1 = min(c0 + A.cols_per_split, A.nk);
    const int qrow0 = blockIdx.x * (kWaves * 16 * NQB) + wave * (16 * NQB);

    float qf[SPLIT ? 1 : NQB][SPLIT ? 1 : KT], vf[MODE == 2 ? NQB : 1][KT];
    u4v qh[SPLIT ? NQB : 1][SPLIT ? KQ : 1], qm[SPLIT ? NQB : 1][SPLIT ? KQ : 1], ql[SPLIT ? NQB : 1][SPLIT ? KQ : 1];
    float lse_c[NQB], S[NQB], Tv[NQB];
    f4 T[NQB][NB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int i = qrow0 + qb * 16 + c;
        const int ic = i < A.nq ? i : A.nq - 1;
        if constexpr (SPLIT) {
            load_query_split<P>(A.q + (size_t)ic * P + g * KT, A.qscale, qh[qb], qm[qb], ql[qb]);
        } else {
            const float4* qr = reinterpret_cast<const float4*>(A.q + (size_t)ic * P + g * KT);
#pragma unroll
            for (int t4 = 0; t4 < KT / 4; ++t4) {
                const float4 v = qr[t4];
                qf[qb][4 * t4 + 0] = v.x * A.qscale;
                qf[qb][4 * t4 + 1] = v.y * A.qscale;
                qf[qb][4 * t4 + 2] = v.z * A.qscale;
                qf[qb][4 * t4 + 3] = v.w * A.qscale;
            }
        }
        if (MODE == 2) {
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int dim = g * KT + t;
                vf[MODE == 2 ? qb : 0][t] = dim < A.d ? 2.0f * A.rowv[(size_t)ic * A.d + dim] : 0.0f;
            }
        }
        lse_c[qb] = A.lse[ic];
        S[qb] = 0.0f;
        Tv[qb] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) T[qb][nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    Stage stage;
    if (c0 < c1) {
        if constexpr (SPLIT)
            stage.load(kb, A.kbias, c0, c1);
        else
            stage.load(kp, A.kbias, c0, c1);
    }
    for (int base = c0; base < c1; base += TL) {
        __syncthreads();
        if constexpr (SPLIT)
            stage.store(reinterpret_cast<u4v*>(ktile), btile);
        else
            stage.store(ktile, btile);
        if (MODE != 1)
            for (int e = threadIdx.x; e < TL * KP; e += kBlock) {
                const int col = base + e / KP;
                const int cc = e % KP;
                ptile[e] = (col < c1 && cc < A.kin) ? A.pay[(size_t)col * A.ldp + cc] : 0.0f;
            }
        __syncthreads();
        if (base + TL < c1) {
            if constexpr (SPLIT)
                stage.load(kb, A.kbias, base + TL, c1);
            else
                stage.load(kp, A.kbias, base + TL, c1);
        }
        const int ntile = min(TL, c1 - base);
        for (int kb16 = 0; kb16 < ntile; kb16 += 16) {
            const f4 bias = *reinterpret_cast<const f4*>(&btile[kb16 + 4 * g]);
            f4 acc[NQB], dv[NQB];
            if constexpr (SPLIT) {
                constexpr int RS = TileStage3<P>::RS;
                split_scores<P, NQB>(reinterpret_cast<const u4v*>(ktile) + (kb16 + c) * RS, g, qh, qm, ql, bias, acc);
            } else {
                float kf[KT];
                load_keys<KT>(kf, ktile, (kb16 + c) * PS + g * KT);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    acc[qb] = bias;
                    dv[qb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
                        acc[qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], qf[qb][t], acc[qb], 0, 0, 0);
                if (MODE == 2) {
#pragma unroll
                    for (int t = 0; t < KT; ++t)
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb)
                            dv[qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], vf[MODE == 2 ? qb : 0][t], dv[qb], 0,
                                                                          0, 0);
                }
            }
            float wv[NQB][4];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float w = ex2(acc[qb][v] - lse_c[qb]);
                    S[qb] += w;
                    wv[qb][v] = MODE == 2 ? w * (ptile[kb16 + 4 * g + v] + dv[qb][v]) : w;
                }
            if (MODE == 3) {
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
                                                  : ktile[(kb16 + 4 * g + v) * PS + nb * 16 + c];
#pragma unroll
                        for (int qb = 0; qb < NQB; ++qb)
                            T[qb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[qb][v], b, T[qb][nb], 0, 0, 0);
                    }
            }
        }
    }
    constexpr int KA = 16 * NB;
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
        if (A.nsplit == 1) {
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

template <int P, int NP, int MODE>
hipError_t launch_transport_mfma_p(const TransArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    constexpr int KA = (MODE == 1 || MODE == 2) ? P : 16 * NP;
    constexpr int rpb = kWaves * 16 * transport_nqb(P, NP, MODE);
    dim3 grid((a.nq + rpb - 1) / rpb, a.nsplit);
    if (ev0) (void)hipEventRecord(ev0, s);
    hipLaunchKernelGGL((k_transport_mfma<P, NP, MODE>), grid, dim3(kBlock), 0, s, a);
    if (ev1) (void)hipEventRecord(ev1, s);
    if (a.nsplit > 1)
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
    if (kwidth == 16) return launch_transport_mfma_p<P, 1, 0>(a, s, ev0, ev1);
    if constexpr (P >= 64) {  // a 64-column payload tile fits LDS beside the key tile from P = 64 on
        if (kwidth == 64) return launch_transport_mfma_p<P, 4, 0>(a, s, ev0, ev1);
    }
    return hipErrorInvalidValue;
}

template <int P>
hipError_t launch_mfma_p(const PassArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (ev0) (void)hipEventRecord(ev0, s);
    if (!a.kb) return hipErrorInvalidValue;  // the split keys are written by every solver set-up
    hipLaunchKernelGGL(k_pass_mfma<P>, dim3(a.W), dim3(kBlock), 0, s, a);
    if (ev1) (void)hipEventRecord(ev1, s);
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

int mfma_grad_rows_per_block() { return kWaves * 16; }

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
    for (int mode = 0; mode <= 3; ++mode)
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

hipError_t launch_grad_mfma(const GradArgs& a, hipStream_t s) {
    switch (a.P) {
        case 16: return launch_grad_mfma_p<16>(a, s);
        case 32: return launch_grad_mfma_p<32>(a, s);
        case 64: return launch_grad_mfma_p<64>(a, s);
        case 128: return launch_grad_mfma_p<128>(a, s);
        case 256: return launch_grad_mfma_p<256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split3(const float* in, int64_t rows, int P, uint16_t* out, hipStream_t s) {
    const int64_t count = rows * P;
    hipLaunchKernelGGL(k_split3, dim3((unsigned)((count + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, in, count, P,
                       out);
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

// sk_ubench.hip -- issue-rate micro-benchmarks that fix the vector-ALU ceiling
// of the streamed passes on gfx950: fp32 FMA, the transcendental exp2
// (v_exp_f32), and the per-pair instruction mix of a d = 3 pass.  Built as a
// separate library (libsk_ubench.so); the solver does not use it.
//
// Each thread runs kChains independent dependency chains so issue rate, not
// latency, is measured.  The kernels write one value per thread so the work
// cannot be removed.
#include <hip/hip_cooperative_groups.h>
#include <hip/hip_runtime.h>

namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void k_fma(float* out, int iters, float a, float b) {
    float v[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) v[c] = threadIdx.x * 1e-3f + c;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) v[c] = fmaf(v[c], a, b);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_exp(float* out, int iters) {
    float v[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) v[c] = -(threadIdx.x * 1e-3f + c * 0.1f);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) v[c] = __builtin_amdgcn_exp2f(-v[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One "pair" = 3 FMA (score), 1 max, 1 subtract, 1 exp2, 1 add, as in a d = 3
// pass.  The key coordinate advances once per 8 pairs (one extra add per
// chain group) so nothing is loop-invariant.
__global__ __launch_bounds__(256) void k_mix(float* out, int iters, float k0, float k1, float k2, float h) {
    const float q1 = threadIdx.x * 1e-5f + 0.5f, q2 = -0.25f - threadIdx.x * 1e-5f;
    float q0[kChains], m[kChains], s[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        q0[c] = threadIdx.x * 1e-4f + c;
        m[c] = -1.0f;
        s[c] = 0.0f;
    }
    float kx = k0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            kx += 1e-7f;
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                const float sc = fmaf(q2, k2, fmaf(q1, k1, fmaf(q0[c], kx, h)));
                m[c] = fmaxf(m[c], sc);
                s[c] += __builtin_amdgcn_exp2f(sc - m[c]);
            }
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += s[c] + m[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// NF FMAs and NE exp2 per chain and step, on independent chains (the exp2
// chains never feed the FMA chains): does a v_exp_f32 take a vector-ALU issue
// slot of its own, or does it run beside the FMAs?  Compare (6, 1) with (6, 0)
// and (7, 0).
template <int NF, int NE>
__global__ __launch_bounds__(256) void k_fma_exp(float* out, int iters, float a, float b) {
    float v[kChains], e[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        v[c] = threadIdx.x * 1e-3f + c;
        e[c] = threadIdx.x * 1e-4f + c * 0.1f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
#pragma unroll
                for (int f = 0; f < NF; ++f) v[c] = fmaf(v[c], a, b);
#pragma unroll
                for (int x = 0; x < NE; ++x) e[c] = __builtin_amdgcn_exp2f(-e[c]);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c] + e[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same with the exp2 in its plain (VOP1) form, as the streamed passes issue
// it: the chain e <- exp2(e) carries no source modifier (its values run to
// +inf, which the units process at full rate).
template <int NF, int NE>
__global__ __launch_bounds__(256) void k_fma_exp_plain(float* out, int iters, float a, float b) {
    float v[kChains], e[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        v[c] = threadIdx.x * 1e-3f + c;
        e[c] = threadIdx.x * 1e-4f + c * 0.1f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
#pragma unroll
                for (int f = 0; f < NF; ++f) v[c] = fmaf(v[c], a, b);
#pragma unroll
                for (int x = 0; x < NE; ++x) e[c] = __builtin_amdgcn_exp2f(e[c]);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c] + e[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// (6, 1) with the scheduler told to interleave: each chain step is issued as
// six FMAs then one exp2 (left alone, the compiler gathers all exp2 of an
// unrolled step into one block, and a block of back-to-back exp2 runs at the
// transcendental unit's half rate with nothing beside it).  In the streamed
// passes the exp2 sit between the subtracts, adds and FMAs, as here.
__global__ __launch_bounds__(256) void k_fma_exp_interleaved(float* out, int iters, float a, float b) {
    float v[kChains], e[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        v[c] = threadIdx.x * 1e-3f + c;
        e[c] = threadIdx.x * 1e-4f + c * 0.1f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
#pragma unroll
                for (int f = 0; f < 6; ++f) v[c] = fmaf(v[c], a, b);
                e[c] = __builtin_amdgcn_exp2f(e[c]);
            }
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                __builtin_amdgcn_sched_group_barrier(0x0002, 6, 0);  // six VALU
                __builtin_amdgcn_sched_group_barrier(0x0400, 1, 0);  // one TRANS
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c] + e[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Six fp32 operations of one kind per chain step on independent chains
// (OP 0 add, 1 subtract, 2 multiply): the issue cost of the non-FMA
// instructions of a pass, against k_fma_exp<6, 0>.
template <int OP>
__global__ __launch_bounds__(256) void k_valu_op(float* out, int iters, float a, float b) {
    float v[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) v[c] = threadIdx.x * 1e-3f + c;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c)
#pragma unroll
                for (int f = 0; f < 6; ++f) v[c] = OP == 0 ? v[c] + b : (OP == 1 ? v[c] - a : v[c] * a);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += v[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Cost of a device-wide barrier: iters grid-wide synchronisations of a
// cooperative launch (every workgroup resident), each preceded by one store
// per thread, as a persistent solver would pay between its half-steps.
__global__ __launch_bounds__(256) void k_grid_sync(float* out, int iters) {
    cooperative_groups::grid_group grid = cooperative_groups::this_grid();
    float v = threadIdx.x * 1e-3f;
    for (int it = 0; it < iters; ++it) {
        v = fmaf(v, 0.999f, 1e-3f);
        out[blockIdx.x * blockDim.x + threadIdx.x] = v;
        grid.sync();
    }
}

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// fp32 matrix-core rate: kChains independent v_mfma_f32_16x16x4f32 chains per wave.
__global__ __launch_bounds__(256) void k_mfma16(float* out, int iters) {
    const float a = threadIdx.x * 1e-3f, b = 1.0f - threadIdx.x * 1e-4f;
    f4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4{0.0f, 0.0f, 0.0f, (float)c};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// fp32 matrix-core rate with the 32x32x2 shape (4 independent chains, 16 accumulators each).
__global__ __launch_bounds__(256) void k_mfma32(float* out, int iters) {
    const float a = threadIdx.x * 1e-3f, b = 1.0f - threadIdx.x * 1e-4f;
    f16v acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = (float)(c + e);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][15];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

// bf16 matrix-core rate: kChains independent v_mfma_f32_16x16x32_bf16 chains per wave.
__global__ __launch_bounds__(256) void k_mfma_bf16(float* out, int iters) {
    const unsigned t = threadIdx.x;
    const u4v ua = {0x3F803F80u + t, 0x3F003F00u, 0x3E803E80u, 0x3F803F00u};
    const u4v ub = {0x3F803F80u, 0x3F003F80u + t, 0x3E803E80u, 0x3F003F00u};
    const bf8 a = __builtin_bit_cast(bf8, ua), b = __builtin_bit_cast(bf8, ub);
    f4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4{0.0f, 0.0f, 0.0f, (float)c};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same bf16 chains with 8 independent vector FMAs after every matrix
// instruction: whether the vector ALU runs under the matrix pipe (time near
// the larger of the two) or not (near their sum).
__global__ __launch_bounds__(256) void k_mfma_bf16_valu(float* out, int iters) {
    const unsigned t = threadIdx.x;
    const u4v ua = {0x3F803F80u + t, 0x3F003F00u, 0x3E803E80u, 0x3F803F00u};
    const u4v ub = {0x3F803F80u, 0x3F003F80u + t, 0x3E803E80u, 0x3F003F00u};
    const bf8 a = __builtin_bit_cast(bf8, ua), b = __builtin_bit_cast(bf8, ub);
    f4 acc[kChains];
    float v[8];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4{0.0f, 0.0f, 0.0f, (float)c};
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t * 1e-3f + e;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fmaf(v[e], 0.999f, 1e-3f);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One v_mfma_f32_16x16x32_f16 per chain step with NF FMAs and NE exp2 beside
// it: independent of the matrix results (DEP = 0), or reading the accumulator
// of the chain issued kChains / 2 instructions earlier (DEP = 1, as a log-sum-
// exp over the previous block's scores would).  Whether transcendentals and
// consumers of matrix results co-execute with the fp16 matrix pipe.
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
template <int NF, int NE, int DEP>
__global__ __launch_bounds__(256) void k_mfma_f16_mix(float* out, int iters) {
    const unsigned t = threadIdx.x;
    const u4v ua = {0x3C003C00u + (t & 7u), 0x38003800u, 0x34003400u, 0x3C003800u};
    const u4v ub = {0x34003400u, 0x3C003800u + (t & 7u), 0x38003800u, 0x30003000u};
    const h8 a = __builtin_bit_cast(h8, ua), b = __builtin_bit_cast(h8, ub);
    f4 acc[kChains];
    float v[NF > 0 ? NF : 1], e[NE > 0 ? NE : 1];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f4{0.0f, 0.0f, 0.0f, (float)c};
#pragma unroll
    for (int x = 0; x < (NF > 0 ? NF : 1); ++x) v[x] = t * 1e-3f + x;
#pragma unroll
    for (int x = 0; x < (NE > 0 ? NE : 1); ++x) e[x] = t * 1e-4f + 0.25f * x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
                const f4 src = acc[(c + kChains / 2) % kChains];
#pragma unroll
                for (int x = 0; x < NF; ++x) v[x] = DEP ? fmaf(src[x & 3], 1e-12f, v[x]) : fmaf(v[x], 0.999f, 1e-3f);
#pragma unroll
                for (int x = 0; x < NE; ++x)
                    e[x] = DEP ? __builtin_amdgcn_exp2f(fmaf(src[x & 3], -1e-12f, -e[x])) : __builtin_amdgcn_exp2f(-e[x]);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
#pragma unroll
    for (int x = 0; x < NF; ++x) s += v[x];
#pragma unroll
    for (int x = 0; x < NE; ++x) s += e[x];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// kind 0: fp32 FMA, 1: exp2, 2: d = 3 pair mix; each thread performs
// iters * 8 * 8 operations (FMAs, exp2s or pairs).  kind 3: each wave issues
// iters * 64 v_mfma_f32_16x16x4f32 (2048 flops each); kind 4: each wave issues
// iters * 64 v_mfma_f32_32x32x2f32 (4096 flops each); kind 5: each wave issues
// iters * 64 v_mfma_f32_16x16x32_bf16 (16384 flops each); kind 6: as kind 5
// with 8 vector FMAs per matrix instruction.  kinds 19-24: each wave issues
// iters * 64 v_mfma_f32_16x16x32_f16 with (FMAs, exp2) beside each: (0, 0),
// (8, 0), (0, 4), (3, 1), and (3, 1), (3, 0) reading earlier matrix results.
// kind 18: iters device-wide
// barriers under a cooperative launch (refused with an error when the grid
// cannot be resident at once).  Launches `blocks` x 256 threads; out must
// hold blocks * 256 floats.  Returns a hipError_t.
int sku_launch(int kind, int blocks, int iters, float* out, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(k_fma, dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 1)
        hipLaunchKernelGGL(k_exp, dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 2)
        hipLaunchKernelGGL(k_mix, dim3(blocks), dim3(256), 0, s, out, iters, 0.3f, 0.2f, 0.1f, 0.05f);
    else if (kind == 3)
        hipLaunchKernelGGL(k_mfma16, dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 4)
        hipLaunchKernelGGL(k_mfma32, dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 5)
        hipLaunchKernelGGL(k_mfma_bf16, dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 6)
        hipLaunchKernelGGL(k_mfma_bf16_valu, dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 7)
        hipLaunchKernelGGL((k_fma_exp<6, 0>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 8)
        hipLaunchKernelGGL((k_fma_exp<6, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 9)
        hipLaunchKernelGGL((k_fma_exp<7, 0>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 10)
        hipLaunchKernelGGL((k_fma_exp<4, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 11)
        hipLaunchKernelGGL((k_fma_exp<2, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 12)
        hipLaunchKernelGGL((k_fma_exp_plain<6, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 13)
        hipLaunchKernelGGL((k_fma_exp_plain<2, 1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 14)
        hipLaunchKernelGGL(k_fma_exp_interleaved, dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 15)
        hipLaunchKernelGGL((k_valu_op<0>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 16)
        hipLaunchKernelGGL((k_valu_op<1>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 17)
        hipLaunchKernelGGL((k_valu_op<2>), dim3(blocks), dim3(256), 0, s, out, iters, 0.999f, 1e-3f);
    else if (kind == 19)
        hipLaunchKernelGGL((k_mfma_f16_mix<0, 0, 0>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 20)
        hipLaunchKernelGGL((k_mfma_f16_mix<8, 0, 0>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 21)
        hipLaunchKernelGGL((k_mfma_f16_mix<0, 4, 0>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 22)
        hipLaunchKernelGGL((k_mfma_f16_mix<3, 1, 0>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 23)
        hipLaunchKernelGGL((k_mfma_f16_mix<3, 1, 1>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 24)
        hipLaunchKernelGGL((k_mfma_f16_mix<3, 0, 1>), dim3(blocks), dim3(256), 0, s, out, iters);
    else if (kind == 18) {
        void* args[] = {&out, &iters};
        return (int)hipLaunchCooperativeKernel(reinterpret_cast<void*>(k_grid_sync), dim3(blocks), dim3(256), args,
                                               0, s);
    }
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // extern "C"

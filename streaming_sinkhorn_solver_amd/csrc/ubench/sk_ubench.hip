// sk_ubench.hip -- issue-rate micro-benchmarks that fix the vector-ALU ceiling
// of the streamed passes on gfx950: fp32 FMA, the transcendental exp2
// (v_exp_f32), and the per-pair instruction mix of a d = 3 pass.  Built as a
// separate library (libsk_ubench.so); the solver does not use it.
//
// Each thread runs kChains independent dependency chains so issue rate, not
// latency, is measured.  The kernels write one value per thread so the work
// cannot be removed.
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

}  // namespace

extern "C" {

// kind 0: fp32 FMA, 1: exp2, 2: d = 3 pair mix; each thread performs
// iters * 8 * 8 operations (FMAs, exp2s or pairs).  kind 3: each wave issues
// iters * 64 v_mfma_f32_16x16x4f32 (2048 flops each); kind 4: each wave issues
// iters * 64 v_mfma_f32_32x32x2f32 (4096 flops each); kind 5: each wave issues
// iters * 64 v_mfma_f32_16x16x32_bf16 (16384 flops each); kind 6: as kind 5
// with 8 vector FMAs per matrix instruction.  Launches `blocks` x 256
// threads; out must hold blocks * 256 floats.  Returns a hipError_t.
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
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

}  // extern "C"

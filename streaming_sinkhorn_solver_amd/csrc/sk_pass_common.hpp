// sk_pass_common.hpp -- device helpers shared by the streamed-pass kernels:
// base-2 exp/log, the per-row finalisation of a pass, and the stream-K range
// arithmetic (see PassArgs in sk_internal.hpp).
#pragma once

#include "sk_internal.hpp"

namespace sk {
namespace {

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Applies a finished row's log-sum-exp (base 2) to the pass outputs.
__device__ __forceinline__ void finalize(const Fin& F, int i, float lse) {
    if (F.mode == kFinSolve) {
        const float old = (F.rbuf || F.alpha != 1.0f) ? F.lse[i] : 0.0f;
        if (F.rbuf) {
            const float wi = F.w[i];
            const float r = wi > 0.0f ? wi * expm1f((lse - old) * kLn2) : 0.0f;
            F.rbuf[i] = fabsf(r);
        }
        const float u = F.alpha == 1.0f ? lse : fmaf(F.alpha, lse - old, old);
        F.lse_out[i] = u;
        const float h = F.l2w[i] - u;
        if (F.bias_packed) F.bias_packed[(size_t)i * F.P + F.d] = h;
        if (F.bias_sep) F.bias_sep[i] = h;
        if (F.pot) F.pot[i] = F.nrm[i] - F.eps_ln2 * u;
    } else if (F.mode == kFinProbe) {
        const float wi = F.w[i];
        const float r = wi > 0.0f ? wi * expm1f((lse - F.lse[i]) * kLn2) : 0.0f;
        F.rbuf[i] = fabsf(r);
    } else if (F.mode == kFinStore) {
        F.lse[i] = lse;
    } else if (F.mode == kFinMass) {  // (P1)_i = a_i exp((f_i - f~_i)/eps)
        const float wi = F.w[i];
        const float e = (F.pot_in[i] - F.nrm[i]) * F.inv_eps + kLn2 * lse;
        F.rbuf[i] = wi > 0.0f ? wi * expf(e) : 0.0f;
    } else if (F.mode == kFinResidLog2) {
        // log2 |a_i (exp(e) - 1)|, e = (f_i - f~_i)/eps, without forming exp(e):
        // for e > 0, log2(exp(e) - 1) = e / ln 2 + log2(1 - exp(-e)); -inf for a zero residual
        const float wi = F.w[i];
        const float e = (F.pot_in[i] - F.nrm[i]) * F.inv_eps + kLn2 * lse;
        const float l = e > 0.0f ? fmaf(e, kLog2e, log2f(-expm1f(-e))) : log2f(-expm1f(e));
        F.rbuf[i] = wi > 0.0f ? log2f(wi) + l : -INFINITY;
    } else {  // kFinResid: (P1)_i / a_i - 1 = exp((f_i - f~_i)/eps) - 1
        const float wi = F.w[i];
        const float e = (F.pot_in[i] - F.nrm[i]) * F.inv_eps + kLn2 * lse;
        const float r = wi > 0.0f ? wi * expm1f(e) : 0.0f;
        F.rbuf[i] = fabsf(r);
    }
}

__device__ __forceinline__ int64_t range_lo(int w, int64_t total, int W) { return (int64_t)w * total / W; }

// The workgroup whose range holds unit u: the largest w with range_lo(w) <= u.
__device__ __forceinline__ int range_owner(int64_t u, int64_t total, int W) {
    return (int)(((u + 1) * W + total - 1) / total) - 1;
}

}  // namespace
}  // namespace sk

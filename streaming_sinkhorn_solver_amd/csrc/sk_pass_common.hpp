// sk_pass_common.hpp -- device helpers shared by the streamed-pass kernels:
// base-2 exp/log, the per-row finalisation of a pass, and the stream-K range
// arithmetic (see PassArgs in sk_internal.hpp).
#pragma once

#include "sk_internal.hpp"

namespace sk {
namespace {

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// What finalize reads of row i besides the log-sum-exp: loaded ahead by a
// kernel that can overlap these loads with its own work (the small-problem
// pass, whose duration is mostly memory latency).
struct FinIn {
    float w;    // query weight
    float old;  // state before the pass
    float l2w;  // log2 weight
    float nrm;  // |q~|^2
    float pin;  // caller potential
};

__device__ __forceinline__ FinIn fin_load(const Fin& F, int i) {
    FinIn p{0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (F.mode == kFinSolve) {
        if (F.rbuf || F.alpha != 1.0f) p.old = F.lse[i];
        if (F.rbuf) p.w = F.w[i];
        if (F.bias_packed || F.bias_sep) p.l2w = F.l2w[i];  // only the next bias needs it
        if (F.pot) p.nrm = F.nrm[i];
    } else if (F.mode == kFinProbe) {
        p.w = F.w[i];
        p.old = F.lse[i];
    } else if (F.mode != kFinStore) {  // kFinMass, kFinResid, kFinResidLog2
        p.w = F.w[i];
        p.pin = F.pot_in[i];
        p.nrm = F.nrm[i];
    }
    return p;
}

// Applies a finished row's log-sum-exp (base 2) to the pass outputs, with the
// row's inputs p = fin_load(F, i).
__device__ __forceinline__ void finalize(const Fin& F, int i, float lse, const FinIn& p) {
    if (F.mode == kFinSolve) {
        if (F.rbuf) {
            const float r = p.w > 0.0f ? p.w * expm1f((lse - p.old) * kLn2) : 0.0f;
            F.rbuf[i] = fabsf(r);
        }
        const float u = F.alpha == 1.0f ? lse : fmaf(F.alpha, lse - p.old, p.old);
        F.lse_out[i] = u;
        const float h = p.l2w - u;
        if (F.bias_packed) F.bias_packed[(size_t)i * F.P + F.d] = h;
        if (F.bias_sep) F.bias_sep[i] = h;
        if (F.pot) F.pot[i] = p.nrm - F.eps_ln2 * u;
    } else if (F.mode == kFinProbe) {
        const float r = p.w > 0.0f ? p.w * expm1f((lse - p.old) * kLn2) : 0.0f;
        F.rbuf[i] = fabsf(r);
    } else if (F.mode == kFinStore) {
        F.lse[i] = lse;
    } else if (F.mode == kFinMass) {  // (P1)_i = a_i exp((f_i - f~_i)/eps)
        const float e = (p.pin - p.nrm) * F.inv_eps + kLn2 * lse;
        F.rbuf[i] = p.w > 0.0f ? p.w * expf(e) : 0.0f;
    } else if (F.mode == kFinResidLog2) {
        // log2 |a_i (exp(e) - 1)|, e = (f_i - f~_i)/eps, without forming exp(e):
        // for e > 0, log2(exp(e) - 1) = e / ln 2 + log2(1 - exp(-e)); -inf for a zero residual
        const float e = (p.pin - p.nrm) * F.inv_eps + kLn2 * lse;
        const float l = e > 0.0f ? fmaf(e, kLog2e, log2f(-expm1f(-e))) : log2f(-expm1f(e));
        F.rbuf[i] = p.w > 0.0f ? log2f(p.w) + l : -INFINITY;
    } else {  // kFinResid: (P1)_i / a_i - 1 = exp((f_i - f~_i)/eps) - 1
        const float e = (p.pin - p.nrm) * F.inv_eps + kLn2 * lse;
        const float r = p.w > 0.0f ? p.w * expm1f(e) : 0.0f;
        F.rbuf[i] = fabsf(r);
    }
}

__device__ __forceinline__ void finalize(const Fin& F, int i, float lse) { finalize(F, i, lse, fin_load(F, i)); }

__device__ __forceinline__ int64_t range_lo(int w, int64_t total, int W) { return (int64_t)w * total / W; }

// The stream-K range that workgroup b of W takes. The hardware deals
// workgroups to the chip's kXcds XCDs round-robin (b mod kXcds), and each XCD
// has its own L2; numbering the ranges XCD by XCD gives every XCD a contiguous
// run of ranges, so a row block's query rows are fetched into one or two L2s
// instead of all of them. A bijection on [0, W); partial slots and the merge
// use the range index, so results do not depend on it.
__device__ __forceinline__ int xcd_range(int b, int W) {
    const int q = W / kXcds, r = W % kXcds, x = b % kXcds;
    return x * q + min(x, r) + b / kXcds;
}

// The workgroup whose range holds unit u: the largest w with range_lo(w) <= u.
__device__ __forceinline__ int range_owner(int64_t u, int64_t total, int W) {
    return (int)(((u + 1) * W + total - 1) / total) - 1;
}

}  // namespace
}  // namespace sk

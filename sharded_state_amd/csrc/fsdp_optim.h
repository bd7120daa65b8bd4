// fsdp_optim.h -- the pointwise optimizers of the unit kernel, as policy types.
// Not installed.
//
// "fairseq 中的 Fully Sharded Data Parallel (FSDP) 实战指南" (zskr.cn),
// "限制与兼容性说明": FSDP supports the pointwise optimizers (Adam, AdamW,
// Adadelta, Adamax, SGD, ...) because every element of a rank's shard is
// updated from that element's gradient and state alone.  "Data Parallelism"
// (vanos001 notes), "The Basic Protocol": W = W - lr * Adam(G_avg, m, v).
//
// Each policy holds its per-launch scalars (computed on the host: fp32
// hyper-parameters, 1 - beta one fp32 operation, bias terms in double rounded
// once) and updates one element: p is the parameter (fp32 master), a and b the
// first and second state values; kStates says how many of them the optimizer
// keeps (the kernel neither loads nor stores the others).  Every fp32
// operation is a single IEEE operation (no contraction), divide and square
// root correctly rounded.  Weight decay: decoupled (p * (1 - lr*wd)) for AdamW,
// added to the gradient (d = g + wd*p, skipped when wd == 0) for the others.
#pragma once

#include <hip/hip_runtime.h>

#include "fsdp_kernels.h"

#pragma clang fp contract(off)

namespace fsdp {

__device__ __forceinline__ float l2_grad(float g, float p, float wd) { return wd != 0.0f ? g + (wd * p) : g; }

// AdamW: bias-corrected Adam, eps after the square root, decoupled decay.
struct OptAdamW {
    static constexpr int kStorePace = 0;
    static constexpr int kStates = 2;
    static constexpr bool kState16 = true;   // also runs on 16-bit parameter / m / v
    AdamScalars s;
    __device__ __forceinline__ void operator()(float g, float& p, float& m, float& v) const {
        float p1 = p * s.decay;
        float m1 = (s.b1 * m) + (s.omb1 * g);
        float v1 = (s.b2 * v) + (s.omb2 * (g * g));
        float den = (__builtin_sqrtf(v1) / s.bc2_sqrt) + s.eps;
        float p2 = p1 - (s.step_size * (m1 / den));
        p = p2;
        m = m1;
        v = v1;
    }
};

// SGD without momentum: p <- p - lr*d.
struct OptSgd {
    static constexpr int kStorePace = 0;
    static constexpr int kStates = 0;
    static constexpr bool kState16 = false;
    float lr, wd;
    __device__ __forceinline__ void operator()(float g, float& p, float&, float&) const {
        const float d = l2_grad(g, p, wd);
        p = p - (lr * d);
    }
};

// SGD with heavy-ball momentum: b <- d on the first step, else
// mu*b + (1 - dampening)*d; the step is d + mu*b (Nesterov) or b.
struct OptSgdMomentum {
    static constexpr int kStorePace = 0;
    static constexpr int kStates = 1;
    static constexpr bool kState16 = false;
    float lr, wd, mu, omd;
    int first, nesterov;
    __device__ __forceinline__ void operator()(float g, float& p, float& buf, float&) const {
        float d = l2_grad(g, p, wd);
        const float b = first ? d : (mu * buf) + (omd * d);
        buf = b;
        d = nesterov ? d + (mu * b) : b;
        p = p - (lr * d);
    }
};

// Adamax: m <- b1*m + (1-b1)*d; u <- max(b2*u, |d| + eps) (NaN if either
// operand is NaN); p <- p - clr * (m / u) with clr = lr / (1 - b1^t).
struct OptAdamax {
    // Adamax's arithmetic is short (one divide, no square root), so with N <= 2
    // its waves reach their stores while the memory system is still saturated
    // with the other waves' reads; idling 16 x 64 cycles before the stores
    // (unit_vec) measured +1.6 points on GPT-2 Large x36 and +1.5 on GPT-2 XL
    // (and took XL's run-to-run spread from 75.0-80.0% to 79.0-79.3%), same
    // box, four repetitions; the N = 8 shapes lost 0.6 with it and AdamW, whose
    // two divides and square root already space its stores, lost too.
    static constexpr int kStorePace = 16;
    static constexpr int kStates = 2;
    static constexpr bool kState16 = false;
    float clr, b1, omb1, b2, eps, wd;
    __device__ __forceinline__ void operator()(float g, float& p, float& m, float& u) const {
        const float d = l2_grad(g, p, wd);
        const float m1 = (b1 * m) + (omb1 * d);
        const float x = b2 * u, y = __builtin_fabsf(d) + eps;
        const float u1 = (__builtin_isnan(x) || __builtin_isnan(y)) ? __builtin_nanf("") : (y > x ? y : x);
        m = m1;
        u = u1;
        p = p - (clr * (m1 / u1));
    }
};

// Adadelta: v <- rho*v + (1-rho)*d*d; delta = sqrt(acc + eps) / sqrt(v + eps) * d;
// acc <- rho*acc + (1-rho)*delta*delta; p <- p - lr*delta.
struct OptAdadelta {
    static constexpr int kStorePace = 0;
    static constexpr int kStates = 2;
    static constexpr bool kState16 = false;
    float lr, rho, omr, eps, wd;
    __device__ __forceinline__ void operator()(float g, float& p, float& v, float& acc) const {
        const float d = l2_grad(g, p, wd);
        const float v1 = (rho * v) + (omr * (d * d));
        const float delta = (__builtin_sqrtf(acc + eps) / __builtin_sqrtf(v1 + eps)) * d;
        const float a1 = (rho * acc) + (omr * (delta * delta));
        v = v1;
        acc = a1;
        p = p - (lr * delta);
    }
};

}  // namespace fsdp

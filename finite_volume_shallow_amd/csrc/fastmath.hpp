// Reciprocal, reciprocal square root and square root for the kernels.
//
// float:  the hardware approximations (v_rcp_f32, v_rsq_f32, v_sqrt_f32,
//         about 1 ulp), well inside the float32 tolerance of the method.
// double: the hardware estimate (v_rcp_f64 / v_rsq_f64, relative error
//         about 5e-8 on this hardware) refined by one Newton step with fused
//         multiply-adds (quadratic convergence: a few 1e-15 relative), in
//         place of the longer IEEE division and square-root sequences; that
//         is four orders of magnitude inside the 1e-10 tolerance of the
//         float64 path.  The bare estimates (rcp_est, rsq_est) serve where a
//         surrounding Newton iteration corrects any error (root finding) or
//         only a starting point is needed.  Inputs are positive normal
//         numbers (depths, wave speeds); a depth <= 0 gives NaN and is
//         flagged by the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace swe {

template <typename T> struct FM;

template <> struct FM<float> {
    static __device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
    static __device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }
    static __device__ __forceinline__ float sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
    static __device__ __forceinline__ float rsq_est(float x) { return __builtin_amdgcn_rsqf(x); }
    static __device__ __forceinline__ float rcp_est(float x) { return __builtin_amdgcn_rcpf(x); }
};

template <> struct FM<double> {
    static __device__ __forceinline__ double rcp(double x)
    {
        const double r = __builtin_amdgcn_rcp(x);
        return __builtin_fma(r, __builtin_fma(-x, r, 1.0), r);
    }
    static __device__ __forceinline__ double rsq(double x)
    {
        const double y = __builtin_amdgcn_rsq(x);
        // y (3/2 - x/2 y^2)
        return y * __builtin_fma(-0.5 * x, y * y, 1.5);
    }
    static __device__ __forceinline__ double sqrt(double x) { return x * rsq(x); }
    // the bare hardware estimates: starting points and Newton corrections
    static __device__ __forceinline__ double rsq_est(double x) { return __builtin_amdgcn_rsq(x); }
    static __device__ __forceinline__ double rcp_est(double x) { return __builtin_amdgcn_rcp(x); }
};

} // namespace swe

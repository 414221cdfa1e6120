// Reciprocal, reciprocal square root and square root for the kernels.
//
// float:  the hardware approximations (v_rcp_f32, v_rsq_f32, v_sqrt_f32,
//         about 1 ulp), well inside the float32 tolerance of the method.
// double: the hardware estimate (v_rcp_f64 / v_rsq_f64) refined by two
//         Newton steps with fused multiply-adds, a few ulp at most, instead
//         of the longer IEEE division and square-root sequences.  Inputs are
//         positive normal numbers (depths, wave speeds); a depth <= 0 gives
//         NaN and is flagged by the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace swe {

template <typename T> struct FM;

template <> struct FM<float> {
    static __device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
    static __device__ __forceinline__ float rsq(float x) { return __builtin_amdgcn_rsqf(x); }
    static __device__ __forceinline__ float sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
    static __device__ __forceinline__ float rsq_est(float x) { return __builtin_amdgcn_rsqf(x); }
};

template <> struct FM<double> {
    static __device__ __forceinline__ double rcp(double x)
    {
        double r = __builtin_amdgcn_rcp(x);
        double e = __builtin_fma(-x, r, 1.0);
        r = __builtin_fma(r, e, r);
        e = __builtin_fma(-x, r, 1.0);
        return __builtin_fma(r, e, r);
    }
    static __device__ __forceinline__ double rsq(double x)
    {
        double y = __builtin_amdgcn_rsq(x);
        const double h = 0.5 * x;
        // y <- y (3/2 - x/2 y^2), twice
        double e = __builtin_fma(-h, y * y, 1.5);
        y = y * e;
        e = __builtin_fma(-h, y * y, 1.5);
        return y * e;
    }
    static __device__ __forceinline__ double sqrt(double x) { return x * rsq(x); }
    // the bare hardware estimate, for starting points only
    static __device__ __forceinline__ double rsq_est(double x) { return __builtin_amdgcn_rsq(x); }
};

} // namespace swe

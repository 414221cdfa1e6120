// Global time-step minimum ([IR] Eq. (5): dt = min_i dt_i).
//
// A wavefront (64 lanes) reduces with cross-lane shuffles, the waves of a
// block through LDS, and one lane per block folds the result into a device
// slot with an atomic min on the IEEE bit pattern: for non-negative doubles
// the unsigned 64-bit order is the numeric order, so the result is exact and
// independent of the order in which blocks arrive.  NaN candidates are
// dropped by fmin (non-finite states are flagged separately).
#pragma once

#include <hip/hip_runtime.h>

namespace swe {

__device__ __forceinline__ double wave_min(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmin(v, __shfl_xor(v, off, 64));
    return v;
}

// Every thread of the block must call this (it contains a barrier).
__device__ __forceinline__ void block_min_to_slot(double v, double *slot)
{
    __shared__ double part[16];
    v = wave_min(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    if (lane == 0) part[wid] = v;
    __syncthreads();
    if (wid == 0) {
        double w = lane < nw ? part[lane] : __builtin_inf();
        w = wave_min(w);
        if (lane == 0 && w >= 0.0 && w < __builtin_inf())
            atomicMin(reinterpret_cast<unsigned long long *>(slot), (unsigned long long)__double_as_longlong(w));
    }
}

} // namespace swe

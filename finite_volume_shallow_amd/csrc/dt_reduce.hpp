// Global time-step minimum ([IR] Eq. (5): dt = min_i dt_i).
//
// A wavefront (64 lanes) reduces with DPP lane moves (VALU, no LDS
// traffic), the waves of a block through LDS, and one lane per block folds
// the result into a device slot with an atomic min on the IEEE bit pattern:
// for non-negative doubles the unsigned 64-bit order is the numeric order,
// so the result is exact and independent of the order in which blocks
// arrive.  NaN candidates are dropped by fmin (non-finite states are flagged
// separately).
#pragma once

#include <hip/hip_runtime.h>

namespace swe {

// v of the lane selected by DPP control CTRL; lanes outside ROWS keep old.
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ double dpp_double(double old, double v)
{
    const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(v), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(v), CTRL, ROWS, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Minimum over the 64 lanes, returned to every lane.  All 64 lanes must be
// active.  Quad permutations, then the half-row and row mirrors leave each
// row of 16 lanes holding its minimum; the row broadcasts of lanes 15 and
// 31 carry it into the upper rows, so lane 63 ends with the wave minimum.
__device__ __forceinline__ double wave_min(double v)
{
    const double inf = __builtin_inf();
    v = fmin(v, dpp_double<0xB1>(inf, v));       // quad_perm [1, 0, 3, 2]
    v = fmin(v, dpp_double<0x4E>(inf, v));       // quad_perm [2, 3, 0, 1]
    v = fmin(v, dpp_double<0x141>(inf, v));      // row_half_mirror
    v = fmin(v, dpp_double<0x140>(inf, v));      // row_mirror
    v = fmin(v, dpp_double<0x142, 0xA>(inf, v)); // row_bcast:15 into rows 1, 3
    v = fmin(v, dpp_double<0x143, 0xC>(inf, v)); // row_bcast:31 into rows 2, 3
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), 63);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), 63);
    return __hiloint2double(hi, lo);
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

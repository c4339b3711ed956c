// newton_iter.hpp -- pieces shared by the Newton paths that run one launch
// per iteration: whether an iteration still runs (every launch reads the
// previous iteration's max|delta|, so the host can enqueue the whole cap
// without waiting for the device), and the workgroup fold of max|delta|.
#pragma once

#include "common.hpp"

namespace prn {

__device__ __forceinline__ bool newton_active(const uint32_t *maxd, int k, float tol) {
    // maxd holds |delta| bits; iterations not run hold 0.
    return k == 1 || !(__uint_as_float(maxd[k - 2]) <= tol);
}

// Fold the per-thread max|delta| (bits of non-negative floats; NaN above
// +inf) over the workgroup and merge it into *dst.  All workgroups of an
// iteration share *dst, so same-address atomics would serialise: only the
// workgroup's first thread updates it, and only when its value exceeds the
// value it reads there (maxima only grow, so a stale read can only cause an
// unnecessary update, never a lost one).
template <int NW>
__device__ __forceinline__ void wg_max_to(uint32_t mx, uint32_t *dst) {
    __shared__ uint32_t s_wmax[NW];
    mx = wave_max_u32(clamp_nan_to_inf(mx));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) s_wmax[w] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = 0;
        for (int k = 0; k < NW; ++k) m = s_wmax[k] > m ? s_wmax[k] : m;
        const uint32_t cur = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (m > cur) __hip_atomic_fetch_max(dst, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace prn

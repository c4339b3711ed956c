// common.hpp -- device primitives shared by the gfx950 kernels:
// fast sigmoid/tanh, the affine-map monoid that the linear-recurrence scans
// compose, wave-level shuffles and the decoupled look-back descriptors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prn {

// ---------------------------------------------------------------- math
// sigmoid(x) = 1 / (1 + 2^(-x log2 e)) with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each).  Saturates correctly: x -> -inf
// gives rcp(inf) = 0, x -> +inf gives rcp(1) = 1.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoid(float x) {
    return fast_rcp(1.0f + fast_exp2(-kLog2e * x));
}
// tanh(x) = 2 sigmoid(2x) - 1; absolute error a few 1e-8.
__device__ __forceinline__ float tanh_fast(float x) {
    return fmaf(2.0f, sigmoid(2.0f * x), -1.0f);
}

// |x| as ordered bits: for non-negative floats the unsigned order equals the
// float order, and every NaN compares above +inf, so an unsigned max keeps
// NaN visible (a float max would drop it).
__device__ __forceinline__ uint32_t abs_bits(float x) {
    return __float_as_uint(x) & 0x7fffffffu;
}
constexpr uint32_t kInfBits = 0x7f800000u;
__device__ __forceinline__ uint32_t clamp_nan_to_inf(uint32_t b) {
    return b > kInfBits ? kInfBits : b;
}

// ---------------------------------------------------------------- monoid
// Affine maps x -> A x + b of a linear recurrence.  then(e, l) is "e first,
// then l": (A_l A_e, A_l b_e + b_l).  Composition is associative, which is
// what lets the recurrence be evaluated by a parallel scan.
struct Aff1 {
    float a, b;
};
struct Aff2 {
    float a00, a01, a10, a11, b0, b1;
};

template <int S> struct MonoidT;

template <> struct MonoidT<1> {
    using Map = Aff1;
    using State = float;
    __device__ __forceinline__ static Map id() { return {1.0f, 0.0f}; }
    __device__ __forceinline__ static Map then(Map e, Map l) {
        return {l.a * e.a, fmaf(l.a, e.b, l.b)};
    }
    __device__ __forceinline__ static State apply(Map m, State x) { return fmaf(m.a, x, m.b); }
    __device__ __forceinline__ static State zero() { return 0.0f; }
    __device__ __forceinline__ static Map shfl_up(Map m, int d) {
        return {__shfl_up(m.a, d, 64), __shfl_up(m.b, d, 64)};
    }
};

struct float2s {
    float x, y;
};

template <> struct MonoidT<2> {
    using Map = Aff2;
    using State = float2s;
    __device__ __forceinline__ static Map id() { return {1.0f, 0.0f, 0.0f, 1.0f, 0.0f, 0.0f}; }
    __device__ __forceinline__ static Map then(Map e, Map l) {
        Map r;
        r.a00 = fmaf(l.a00, e.a00, l.a01 * e.a10);
        r.a01 = fmaf(l.a00, e.a01, l.a01 * e.a11);
        r.a10 = fmaf(l.a10, e.a00, l.a11 * e.a10);
        r.a11 = fmaf(l.a10, e.a01, l.a11 * e.a11);
        r.b0 = fmaf(l.a00, e.b0, fmaf(l.a01, e.b1, l.b0));
        r.b1 = fmaf(l.a10, e.b0, fmaf(l.a11, e.b1, l.b1));
        return r;
    }
    __device__ __forceinline__ static State apply(Map m, State x) {
        return {fmaf(m.a00, x.x, fmaf(m.a01, x.y, m.b0)), fmaf(m.a10, x.x, fmaf(m.a11, x.y, m.b1))};
    }
    __device__ __forceinline__ static State zero() { return {0.0f, 0.0f}; }
    __device__ __forceinline__ static Map shfl_up(Map m, int d) {
        return {__shfl_up(m.a00, d, 64), __shfl_up(m.a01, d, 64), __shfl_up(m.a10, d, 64),
                __shfl_up(m.a11, d, 64), __shfl_up(m.b0, d, 64),  __shfl_up(m.b1, d, 64)};
    }
};

// ---------------------------------------------------------------- look-back
// Decoupled look-back descriptors, one per (chunk, batch, channel).  Each
// descriptor is a few 64-bit words that are written exactly once per launch
// (from the sentinel to a value) with agent-scope atomic stores, and polled
// with agent-scope atomic loads, which the compiler emits as device-coherent
// (sc1) accesses, so they are seen across the XCDs' separate L2 caches.  A
// word that is no longer the sentinel therefore already holds its final
// value and no flag or fence is needed.  The sentinel is a signalling-NaN
// pair that arithmetic never produces; published values are canonicalised so
// that an input NaN cannot mimic it.
//   agg : the chunk's aggregate map (S=1: 1 word; S=2: 3 words)
//   inc : the state after the chunk, i.e. the inclusive prefix applied to the
//         initial state (S=1: low half of 1 word; S=2: 1 word)
constexpr uint32_t kSentinel32 = 0x7f800001u;
constexpr uint64_t kSentinel64 = 0x7f8000017f800001ull;

__device__ __forceinline__ float canon(float x) { return x != x ? __uint_as_float(0x7fc00000u) : x; }
__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
    return (uint64_t)__float_as_uint(canon(lo)) | ((uint64_t)__float_as_uint(canon(hi)) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float hi_f(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }

__device__ __forceinline__ uint64_t ld_coherent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int S> __device__ __forceinline__ typename MonoidT<S>::State nan_state();
template <> __device__ __forceinline__ float nan_state<1>() { return __uint_as_float(0x7fc00000u); }
template <> __device__ __forceinline__ float2s nan_state<2>() {
    return {__uint_as_float(0x7fc00000u), __uint_as_float(0x7fc00000u)};
}

template <int S> struct Desc;

template <> struct Desc<1> {
    static constexpr int kAggWords = 1;
    static constexpr int kIncWords = 1;
    __device__ static void put_agg(uint64_t *w, Aff1 m) { st_coherent(w, pack2(m.a, m.b)); }
    __device__ static void put_inc(uint64_t *w, float x) { st_coherent(w, pack2(x, 0.0f)); }
    __device__ static bool get_inc(const uint64_t *w, float &x) {
        uint64_t v = ld_coherent(w);
        if (v == kSentinel64) return false;
        x = lo_f(v);
        return true;
    }
    __device__ static bool get_agg(const uint64_t *w, Aff1 &m) {
        uint64_t v = ld_coherent(w);
        if (v == kSentinel64) return false;
        m = {lo_f(v), hi_f(v)};
        return true;
    }
};

template <> struct Desc<2> {
    static constexpr int kAggWords = 3;
    static constexpr int kIncWords = 1;
    __device__ static void put_agg(uint64_t *w, Aff2 m) {
        st_coherent(w + 0, pack2(m.a00, m.a01));
        st_coherent(w + 1, pack2(m.a10, m.a11));
        st_coherent(w + 2, pack2(m.b0, m.b1));
    }
    __device__ static void put_inc(uint64_t *w, float2s x) { st_coherent(w, pack2(x.x, x.y)); }
    __device__ static bool get_inc(const uint64_t *w, float2s &x) {
        uint64_t v = ld_coherent(w);
        if (v == kSentinel64) return false;
        x = {lo_f(v), hi_f(v)};
        return true;
    }
    __device__ static bool get_agg(const uint64_t *w, Aff2 &m) {
        uint64_t v0 = ld_coherent(w + 0), v1 = ld_coherent(w + 1), v2 = ld_coherent(w + 2);
        if (v0 == kSentinel64 || v1 == kSentinel64 || v2 == kSentinel64) return false;
        m = {lo_f(v0), hi_f(v0), lo_f(v1), hi_f(v1), lo_f(v2), hi_f(v2)};
        return true;
    }
};

// Bound on the polls of one unpublished descriptor.  Every predecessor of a
// chunk holds a smaller dynamic ticket, so it is already resident and will
// publish and the wait ends; the bound is only a guard against a broken
// invariant: when it is hit the error word is set and NaN is returned, so
// the failure shows in the output instead of hanging the device.
constexpr uint32_t kMaxPolls = 1u << 20;

// ---------------------------------------------------------------- indexing
__device__ __forceinline__ int64_t idx3(int64_t b, int64_t t, int64_t j, int64_t L, int64_t H) {
    return (b * L + t) * H + j;
}

// Wave-wide max of unsigned values (butterfly over the 64 lanes).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint32_t o = __shfl_xor(v, d, 64);
        v = v > o ? v : o;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

}  // namespace prn

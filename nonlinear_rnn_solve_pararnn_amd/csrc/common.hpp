// common.hpp -- device primitives shared by the gfx950 kernels:
// fast sigmoid/tanh, the affine-map monoid that the linear-recurrence scans
// compose, wave-level shuffles and the decoupled look-back descriptors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "tags.hpp"

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

// k x k blocks (k >= 3): A row-major, a[i * k + l] takes component l into i.
template <int K>
struct AffK {
    float a[K * K];
    float b[K];
};
template <int K>
struct VecK {
    float v[K];
};

// The primary template serves k x k blocks; k = 1 and k = 2 are specialised
// below with named fields.
template <int S>
struct MonoidT {
    static_assert(S >= 3 && S <= 8, "k x k blocks for 3 <= k <= 8");
    using Map = AffK<S>;
    using State = VecK<S>;
    __device__ __forceinline__ static Map id() {
        Map m;
#pragma unroll
        for (int i = 0; i < S; ++i) {
#pragma unroll
            for (int l = 0; l < S; ++l) m.a[i * S + l] = i == l ? 1.0f : 0.0f;
            m.b[i] = 0.0f;
        }
        return m;
    }
    __device__ __forceinline__ static Map then(const Map &e, const Map &l) {
        Map r;
#pragma unroll
        for (int i = 0; i < S; ++i) {
#pragma unroll
            for (int c = 0; c < S; ++c) {
                float acc = l.a[i * S] * e.a[c];
#pragma unroll
                for (int m = 1; m < S; ++m) acc = fmaf(l.a[i * S + m], e.a[m * S + c], acc);
                r.a[i * S + c] = acc;
            }
            float acc = l.b[i];
#pragma unroll
            for (int m = 0; m < S; ++m) acc = fmaf(l.a[i * S + m], e.b[m], acc);
            r.b[i] = acc;
        }
        return r;
    }
    __device__ __forceinline__ static State apply(const Map &m, const State &x) {
        State y;
#pragma unroll
        for (int i = 0; i < S; ++i) {
            float acc = m.b[i];
#pragma unroll
            for (int l = 0; l < S; ++l) acc = fmaf(m.a[i * S + l], x.v[l], acc);
            y.v[i] = acc;
        }
        return y;
    }
    __device__ __forceinline__ static State zero() {
        State x;
#pragma unroll
        for (int i = 0; i < S; ++i) x.v[i] = 0.0f;
        return x;
    }
    __device__ __forceinline__ static Map shfl_up(const Map &m, int d) {
        Map r;
#pragma unroll
        for (int i = 0; i < S * S; ++i) r.a[i] = __shfl_up(m.a[i], d, 64);
#pragma unroll
        for (int i = 0; i < S; ++i) r.b[i] = __shfl_up(m.b[i], d, 64);
        return r;
    }
};

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
// Decoupled look-back descriptors, one per (chunk, batch, channel).  Every
// word is 64 bits: a float payload in the low half and the tag of the launch
// that wrote it in the high half.  Words are written once per launch with
// agent-scope atomic stores and polled with agent-scope atomic loads, which
// the compiler emits as device-coherent (sc1) accesses, so they are seen
// across the XCDs' separate L2 caches.  A word whose tag is this launch's
// already holds its final value, so no flag, fence or clearing pass is
// needed: words left over from earlier launches carry other tags.
//   agg : the chunk's aggregate map (S=1: a, b; S=2: a00, a01, a10, a11, b0, b1)
//   inc : the state after the chunk, i.e. the inclusive prefix applied to the
//         initial state (S components)
//
// Launch tags and the epochs that number the launches on one workspace are
// defined in tags.hpp: no two launches of one period share a tag, and the
// last launch of a period clears the workspace (finish_launch below).
__device__ __forceinline__ uint64_t tagged(float x, uint32_t tag) {
    return (uint64_t)__float_as_uint(x) | ((uint64_t)tag << 32);
}
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ bool has_tag(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

__device__ __forceinline__ uint64_t ld_coherent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int S> __device__ __forceinline__ typename MonoidT<S>::State nan_state() {
    typename MonoidT<S>::State x;
#pragma unroll
    for (int i = 0; i < S; ++i) x.v[i] = __uint_as_float(0x7fc00000u);
    return x;
}
template <> __device__ __forceinline__ float nan_state<1>() { return __uint_as_float(0x7fc00000u); }
template <> __device__ __forceinline__ float2s nan_state<2>() {
    return {__uint_as_float(0x7fc00000u), __uint_as_float(0x7fc00000u)};
}

// k x k blocks: the k*k entries of A then the k offsets; the state's k components.
template <int S>
struct Desc {
    static constexpr int kAggWords = desc_agg_words(S);
    static constexpr int kIncWords = desc_inc_words(S);
    static_assert(kAggWords == S * S + S && kIncWords == S, "one word per float");
    __device__ static void put_agg(uint64_t *w, const AffK<S> &m, uint32_t tag) {
#pragma unroll
        for (int i = 0; i < S * S; ++i) st_coherent(w + i, tagged(m.a[i], tag));
#pragma unroll
        for (int i = 0; i < S; ++i) st_coherent(w + S * S + i, tagged(m.b[i], tag));
    }
    __device__ static void put_inc(uint64_t *w, const VecK<S> &x, uint32_t tag) {
#pragma unroll
        for (int i = 0; i < S; ++i) st_coherent(w + i, tagged(x.v[i], tag));
    }
    __device__ static bool get_inc(const uint64_t *w, VecK<S> &x, uint32_t tag) {
        uint64_t v[S];
#pragma unroll
        for (int i = 0; i < S; ++i) v[i] = ld_coherent(w + i);
        bool ok = true;
#pragma unroll
        for (int i = 0; i < S; ++i) ok = ok && has_tag(v[i], tag);
        if (!ok) return false;
#pragma unroll
        for (int i = 0; i < S; ++i) x.v[i] = lo_f(v[i]);
        return true;
    }
    __device__ static bool get_agg(const uint64_t *w, AffK<S> &m, uint32_t tag) {
        uint64_t v[S * S + S];
#pragma unroll
        for (int i = 0; i < S * S + S; ++i) v[i] = ld_coherent(w + i);
        bool ok = true;
#pragma unroll
        for (int i = 0; i < S * S + S; ++i) ok = ok && has_tag(v[i], tag);
        if (!ok) return false;
#pragma unroll
        for (int i = 0; i < S * S; ++i) m.a[i] = lo_f(v[i]);
#pragma unroll
        for (int i = 0; i < S; ++i) m.b[i] = lo_f(v[S * S + i]);
        return true;
    }
};

template <> struct Desc<1> {
    static constexpr int kAggWords = desc_agg_words(1);
    static constexpr int kIncWords = desc_inc_words(1);
    static_assert(kAggWords == 2 && kIncWords == 1, "one word per float");
    __device__ static void put_agg(uint64_t *w, Aff1 m, uint32_t tag) {
        st_coherent(w + 0, tagged(m.a, tag));
        st_coherent(w + 1, tagged(m.b, tag));
    }
    __device__ static void put_inc(uint64_t *w, float x, uint32_t tag) { st_coherent(w, tagged(x, tag)); }
    __device__ static bool get_inc(const uint64_t *w, float &x, uint32_t tag) {
        const uint64_t v = ld_coherent(w);
        if (!has_tag(v, tag)) return false;
        x = lo_f(v);
        return true;
    }
    __device__ static bool get_agg(const uint64_t *w, Aff1 &m, uint32_t tag) {
        const uint64_t v0 = ld_coherent(w + 0), v1 = ld_coherent(w + 1);
        if (!has_tag(v0, tag) || !has_tag(v1, tag)) return false;
        m = {lo_f(v0), lo_f(v1)};
        return true;
    }
};

template <> struct Desc<2> {
    static constexpr int kAggWords = desc_agg_words(2);
    static constexpr int kIncWords = desc_inc_words(2);
    static_assert(kAggWords == 6 && kIncWords == 2, "one word per float");
    __device__ static void put_agg(uint64_t *w, Aff2 m, uint32_t tag) {
        st_coherent(w + 0, tagged(m.a00, tag));
        st_coherent(w + 1, tagged(m.a01, tag));
        st_coherent(w + 2, tagged(m.a10, tag));
        st_coherent(w + 3, tagged(m.a11, tag));
        st_coherent(w + 4, tagged(m.b0, tag));
        st_coherent(w + 5, tagged(m.b1, tag));
    }
    __device__ static void put_inc(uint64_t *w, float2s x, uint32_t tag) {
        st_coherent(w + 0, tagged(x.x, tag));
        st_coherent(w + 1, tagged(x.y, tag));
    }
    __device__ static bool get_inc(const uint64_t *w, float2s &x, uint32_t tag) {
        const uint64_t v0 = ld_coherent(w + 0), v1 = ld_coherent(w + 1);
        if (!has_tag(v0, tag) || !has_tag(v1, tag)) return false;
        x = {lo_f(v0), lo_f(v1)};
        return true;
    }
    __device__ static bool get_agg(const uint64_t *w, Aff2 &m, uint32_t tag) {
        uint64_t v[6];
#pragma unroll
        for (int k = 0; k < 6; ++k) v[k] = ld_coherent(w + k);
        bool ok = true;
#pragma unroll
        for (int k = 0; k < 6; ++k) ok = ok && has_tag(v[k], tag);
        if (!ok) return false;
        m = {lo_f(v[0]), lo_f(v[1]), lo_f(v[2]), lo_f(v[3]), lo_f(v[4]), lo_f(v[5])};
        return true;
    }
};

// Ticket header of a workspace (its first two words, tags.hpp): tickets
// drawn in the current launch and the launch epoch, then the count of
// finished workgroups of the last launch of a period.  The workgroup that
// draws a launch's last ticket resets the count and advances the epoch, so
// the next launch on the stream finds the header ready; a zero-filled
// workspace is ready for its first launch.  Every draw of one launch sees
// the same epoch.
struct Ticket {
    uint32_t index, tag;
    bool wrap;  // this launch uses the last tag of the period
};
__device__ __forceinline__ Ticket draw_ticket(uint64_t *hdr, uint32_t draws) {
    const uint64_t old = __hip_atomic_fetch_add(hdr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t idx = (uint32_t)old, epoch = (uint32_t)(old >> 32);
    if (epoch >= kTagPeriod) epoch = kTagPeriod - 1u;  // only a header the library did not write
    if (idx + 1u == draws)
        __hip_atomic_store(hdr, header_after_draw(idx, epoch, draws), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return {idx, launch_tag(epoch), is_wrap_launch(epoch)};
}

// Where a launch's caller workspace is and what it must keep.  At the end of
// the last launch of a period (Ticket::wrap) the workgroup that finishes last
// zeroes every word past the header except [keep_lo, keep_hi): state that a
// later launch of the same call reads (the per-iteration path's max|delta|
// slots and boundary states, the adjoint's dL/du partials), which holds no
// tagged words.
struct WsSpan {
    uint64_t *hdr;
    uint64_t words;            // 64-bit words of the caller's whole buffer
    uint64_t keep_lo, keep_hi;
};

// Zero words [lo, hi) of w (w 16-byte aligned) with every thread of the
// workgroup: an odd word at either end alone, 16-byte stores in between.
__device__ __forceinline__ void clear_words(uint64_t *w, uint64_t lo, uint64_t hi) {
    if (lo >= hi) return;
    if (lo & 1) {
        if (threadIdx.x == 0) w[lo] = 0;
        ++lo;
    }
    if (hi > lo && (hi & 1)) {
        if (threadIdx.x == 0) w[hi - 1] = 0;
        --hi;
    }
    uint4 *v = reinterpret_cast<uint4 *>(w + lo);
    for (uint64_t i = threadIdx.x; i < (hi - lo) / 2; i += blockDim.x) v[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Called by every thread of every workgroup of a launch that draws tickets,
// after the workgroup's last draw and last access to records; `t` is any of
// its tickets.  Outside the last launch of a period it does nothing.  In that
// launch every workgroup counts itself out (its record stores released
// first), and the one that finishes last clears the workspace; the next
// launch on the stream starts after it.  No workgroup waits for another.
// The wrap step is a call, not inlined: its loops would otherwise raise the
// register count of every kernel that ends with it.
__device__ __noinline__ void finish_wrap_launch(const WsSpan ws) {
    __shared__ int s_last;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // this thread's record stores first
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint64_t before =
            __hip_atomic_fetch_add(ws.hdr + 1, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = before + 1 == (uint64_t)gridDim.x ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const ClearRanges r = clear_ranges(ws.words, ws.keep_lo, ws.keep_hi);
    clear_words(ws.hdr, r.lo0, r.hi0);
    clear_words(ws.hdr, r.lo1, r.hi1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(ws.hdr + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void finish_launch(const Ticket &t, const WsSpan &ws) {
    if (t.wrap) finish_wrap_launch(ws);  // the same for every workgroup of the launch
}

// Bound on the polls of one unpublished descriptor.  Every predecessor of a
// chunk holds a smaller dynamic ticket, so it is already resident and will
// publish and the wait ends; the bound is only a guard against a broken
// invariant (such as a workspace that was not zero-filled before its first
// use): when it is hit NaN is returned, so the failure shows in the output
// instead of hanging the device.
constexpr uint32_t kMaxPolls = 1u << 20;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations but not for its outstanding global memory operations (loads
// issued early stay in flight across it).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left alone
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- streamed inputs
// Inputs that a launch reads exactly once are loaded with the non-temporal
// hint.  It changes only how the caches keep the lines: streamed operands
// then do not push the look-back records and the lines still being written
// out of L2 (the diagonal scan at B=16, L=4096, H=1024 gains about 12%).
// Operands read twice (a state that is also the next position's previous
// state) keep ordinary loads, and so do two patterns where streaming was
// measured to lose: the 64-byte runs of the Newton forward kernels (one
// thread's four 16-byte loads share a line with its neighbour's; the GRU
// forward at B=16, L=2^20, H=1 went from 0.30 to 0.40 ms per step) and the
// 64-byte row pieces of the fused GRU tiles (11% more bytes fetched, no
// gain).  The adjoint's 32-byte runs gain from it (0.166 -> 0.149 ms).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float ld_once(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float2 ld_once(const float2 *p) {
    const f32x2 v = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(p));
    return make_float2(v.x, v.y);
}
__device__ __forceinline__ float4 ld_once(const float4 *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- runs
// C consecutive floats at a 16-byte aligned address, moved with one 16-byte
// access per four floats: the sequence of a single channel (H = 1) walked by
// one thread in the time-lane layout.  ONCE selects the streamed load.
template <int C, bool ONCE = false>
__device__ __forceinline__ void load_run(const float *p, float (&v)[C]) {
    static_assert(C % 4 == 0, "runs are whole float4s");
#pragma unroll
    for (int k = 0; k < C / 4; ++k) {
        const float4 q = ONCE ? ld_once(reinterpret_cast<const float4 *>(p) + k) : reinterpret_cast<const float4 *>(p)[k];
        v[4 * k + 0] = q.x;
        v[4 * k + 1] = q.y;
        v[4 * k + 2] = q.z;
        v[4 * k + 3] = q.w;
    }
}
template <int C>
__device__ __forceinline__ void store_run(float *p, const float (&v)[C]) {
    static_assert(C % 4 == 0, "runs are whole float4s");
#pragma unroll
    for (int k = 0; k < C / 4; ++k)
        reinterpret_cast<float4 *>(p)[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
}

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

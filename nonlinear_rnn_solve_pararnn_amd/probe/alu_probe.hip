// alu_probe.hip -- measurement only, not part of the C ABI of libpararnn:
// the issue rates of plain fp32 multiply-adds and of the transcendental pair
// (exp2, reciprocal) that the Newton kernels are built from, measured on the
// device with the same compiler flags (packed fp32 disabled), so the
// arithmetic rooflines can be given against a measured basis beside the
// published fp32 vector peak; and the rate of dense 8x8 map compositions in
// the block scans' vector form against the matrix cores' bound for the same
// work.  Each thread runs independent chains held in registers; nothing is
// read from memory and one float per thread is written so the chains are
// kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../csrc/lanegroup.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

__global__ __launch_bounds__(kThreads) void fma_probe_kernel(int iters, float *out) {
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = 1e-3f * (threadIdx.x + k);
    const float m = 0.9999f, c = 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += a[k];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// a <- 1 / (1 + 2^a): one exp2, one add and one reciprocal per step; the
// iterate stays in (0, 1).
__global__ __launch_bounds__(kThreads) void trans_probe_kernel(int iters, float *out) {
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = 1e-3f * (threadIdx.x + k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a[k]));
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += a[k];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Per step: four chains of (exp2, add, reciprocal) and M multiply-adds on
// eight other chains, the mix of the Newton cells (transcendentals among
// plain instructions), to see how the two share the issue of a SIMD.
template <int M>
__global__ __launch_bounds__(kThreads) void mix_probe_kernel(int iters, float *out) {
    float t[4], a[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = 1e-3f * (threadIdx.x + k);
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = 1e-3f * (threadIdx.x + k);
    const float m = 0.9999f, c = 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
            for (int k = 0; k < 4; ++k) t[k] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t[k]));
#pragma unroll
            for (int r = 0; r < M; ++r) a[r & 7] = fmaf(a[r & 7], m, c);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += t[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) s += a[k];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// ---------------------------------------------------------------- 8x8 maps
// The block scans compose dense 8x8 affine maps (A, b), one per position.
// Vector form, as the scans do it (lanegroup.hpp): lane c of a group of 8
// lanes holds row c of a map in xor order and a composition is row_then,
// multiply-adds with DPP operands.  Four independent chains per lane group;
// the fixed map contracts, so the values stay small.
constexpr int kComposeChains = 4, kComposeUnroll = 4;
__global__ __launch_bounds__(kThreads) void lg8_compose_probe_kernel(int iters, float *out) {
    using prn::lg::RowK;
    RowK<8> m;
#pragma unroll
    for (int p = 0; p < 8; ++p) m.a[p] = p == 0 ? 0.5f : 1e-3f * (float)((threadIdx.x + p) & 7);
    m.b = 1e-3f;
    RowK<8> acc[kComposeChains];
#pragma unroll
    for (int k = 0; k < kComposeChains; ++k) {
        acc[k] = m;
        acc[k].b = 1e-3f * (float)(k + 1);
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kComposeUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < kComposeChains; ++k) acc[k] = prn::lg::row_then<8>(acc[k], m);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kComposeChains; ++k) {
#pragma unroll
        for (int p = 0; p < 8; ++p) s += acc[k].a[p];
        s += acc[k].b;
    }
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Matrix-core bound for the same work: v_mfma_f32_16x16x4_f32 (a 16x4 by
// 4x16 fp32 product per wave).  Two 8x8 maps packed block-diagonally into a
// 16x16 matrix compose with another such pair in one 16x16x16 product, four
// of these instructions.  Eight independent accumulators per wave, operands
// held in registers: the lane permutes a chain of products would need between
// steps (the product's layout is not the next operand's) are left out, and
// so is the b part of the maps, so this bounds the matrix cores from above.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kThreads) void mfma_probe_kernel(int iters, float *out) {
    const float a = 1e-3f * (float)(threadIdx.x & 63), b = 1e-3f;
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k].x + acc[k].y + acc[k].z + acc[k].w;
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Lane operations one launch performs: blocks * 256 threads * iters * 16 * 8
// multiply-adds (fma) or exp2/reciprocal pairs (trans).  out: device float
// [blocks * 256].  Returns 0, or the HIP error code of the launch.
int alu_probe_threads_per_block(void) { return kThreads; }
int alu_probe_steps_per_iter(void) { return kUnroll * 8; }

int alu_probe_fma(int64_t blocks, int32_t iters, float *out, void *stream) {
    hipLaunchKernelGGL(fma_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return (int)hipGetLastError();
}

int alu_probe_trans(int64_t blocks, int32_t iters, float *out, void *stream) {
    hipLaunchKernelGGL(trans_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return (int)hipGetLastError();
}

// Steps per iteration of the mix probe (each: 4 x (exp2, add, reciprocal)
// and m multiply-adds, m in {0, 4, 8, 16, 32}); returns -1 for another m.
int alu_probe_mix_steps_per_iter(void) { return 8; }

int alu_probe_mix(int64_t blocks, int32_t iters, int32_t m, float *out, void *stream) {
    const dim3 g((unsigned)blocks), b(kThreads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (m) {
        case 0: hipLaunchKernelGGL(mix_probe_kernel<0>, g, b, 0, s, iters, out); break;
        case 4: hipLaunchKernelGGL(mix_probe_kernel<4>, g, b, 0, s, iters, out); break;
        case 8: hipLaunchKernelGGL(mix_probe_kernel<8>, g, b, 0, s, iters, out); break;
        case 16: hipLaunchKernelGGL(mix_probe_kernel<16>, g, b, 0, s, iters, out); break;
        case 32: hipLaunchKernelGGL(mix_probe_kernel<32>, g, b, 0, s, iters, out); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

// 8x8 compositions per thread and iteration of the vector probe (each lane
// group of 8 threads composes kComposeChains maps kComposeUnroll times per
// iteration: per lane group, 8 times this); MFMA instructions per wave and
// iteration of the matrix-core probe (2048 flops each).
int alu_probe_lg8_compose_per_group_iter(void) { return kComposeChains * kComposeUnroll; }
int alu_probe_mfma_per_wave_iter(void) { return kUnroll * 8; }

int alu_probe_lg8_compose(int64_t blocks, int32_t iters, float *out, void *stream) {
    hipLaunchKernelGGL(lg8_compose_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return (int)hipGetLastError();
}

int alu_probe_mfma(int64_t blocks, int32_t iters, float *out, void *stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"

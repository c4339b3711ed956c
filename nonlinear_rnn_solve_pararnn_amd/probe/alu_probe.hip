// alu_probe.hip -- measurement only, not part of the C ABI of libpararnn:
// the issue rates of plain fp32 multiply-adds and of the transcendental pair
// (exp2, reciprocal) that the Newton kernels are built from, measured on the
// device with the same compiler flags (packed fp32 disabled), so the
// arithmetic rooflines can be given against a measured basis beside the
// published fp32 vector peak.  Each thread runs 8 independent chains held in
// registers; nothing is read from memory and one float per thread is written
// so the chains are kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // extern "C"

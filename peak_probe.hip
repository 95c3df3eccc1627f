// Microbenchmarks of this GPU's own peaks, for the roofline fractions the benchmark reports: the
// dense bf16 matrix-core rate and the HBM read rate. Not part of the retention library or its ABI;
// bench.py (beside this file) loads the small library built from it.
//
//   mfma_peak_kernel  every wave issues 32x32x16 bf16 MFMAs on four independent accumulators (so
//                     that no issue waits on a result; distinct start values, or the compiler merges
//                     the chains), operands in registers, no memory traffic inside the loop. One
//                     launch = blocks * 4 waves * iters * 4 MFMAs of 32768 flop.
//   hbm_read_kernel   a grid-stride sum over a buffer with 16-byte non-temporal loads, four loads in
//                     flight per thread; the buffer is read once per launch.
#include <hip/hip_runtime.h>

#include <cstddef>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 4;

__global__ __launch_bounds__(kThreads) void mfma_peak_kernel(int iters, float* __restrict__ out) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)(threadIdx.x + j));
        b[j] = (__bf16)(1e-3f * (float)(j + 1));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        acc[c] = f32x16{};
        acc[c][0] = (float)c;  // distinct chains (identical ones would merge)
    }
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[c][j];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;  // one float per thread: the work is used
}

__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const f32x4* __restrict__ src, size_t n4, float* __restrict__ out) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const f32x4 x0 = __builtin_nontemporal_load(src + i), x1 = __builtin_nontemporal_load(src + i + stride);
        const f32x4 x2 = __builtin_nontemporal_load(src + i + 2 * stride), x3 = __builtin_nontemporal_load(src + i + 3 * stride);
        acc += (x0 + x1) + (x2 + x3);
    }
    for (; i < n4; i += stride) acc += __builtin_nontemporal_load(src + i);
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

}  // namespace

extern "C" {

// Threads per block of both probes; out must hold blocks * probe_threads() floats.
int probe_threads(void) { return kThreads; }

// Launch the MFMA probe on stream (NULL: default): blocks workgroups of 4 waves, iters loop trips.
// Returns the hipError_t of the launch (0 on success).
int probe_mfma_bf16(int blocks, int iters, float* out, void* stream) {
    if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream), iters, out);
    return (int)hipGetLastError();
}

// Launch the HBM read probe over bytes (a multiple of 16) at src (16-byte aligned).
int probe_hbm_read(const void* src, size_t bytes, int blocks, float* out, void* stream) {
    if (!src || !out || blocks <= 0 || bytes % 16 || reinterpret_cast<size_t>(src) % 16) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(hbm_read_kernel, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const f32x4*>(src), bytes / 16, out);
    return (int)hipGetLastError();
}

}  // extern "C"

// fp32-input retention on the vector ALU: the chunkwise form, the parallel form, and a row-wise
// per-head GroupNorm pass. On gfx950 the fp32 matrix cores and the fp32 vector units have the
// same peak rate, so this path uses plain fused multiply-adds with LDS-staged operands. It serves
// fp32 workloads (small, tolerance 1e-4), where accuracy rather than throughput is the point.
//
// Chunkwise form (abeam.tech RetNet summary, "Chunk recursion for long-sequence training"), for a
// chunk of length L with carried state R and local row j:
//     o_j = sum_{t<=j} g^(j-t) (q_j . k_t) v_t + g^(j+1) q_j R,    R <- g^L R + sum_t g^(L-1-t) k_t^T v_t
// Parallel form (same page, retention definition): o_n = sum_{m<=n} g^(n-m) (q_n . k_m) v_m.
#include "common.hpp"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;  // d_v columns per workgroup

// Grid: B*H*(DV/64) workgroups. Dynamic LDS: R [DK][64] fp32 then S [C][C] fp32.
// Thread t: column t % 64, row group t / 64 (rows strided by 4).
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(int H, int N, int DK, int DV, int C,
                                                             const float* __restrict__ q, const float* __restrict__ k,
                                                             const float* __restrict__ v, const float* __restrict__ state_in,
                                                             float* __restrict__ state_out, float* __restrict__ out,
                                                             HeadConsts hc, const float* __restrict__ vpre, int vsplit, int vshift) {
    extern __shared__ float smem[];
    const int nsl = DV / kCols;
    const int bh = blockIdx.x / nsl, slice = blockIdx.x % nsl, h = bh % H;
    const int col = threadIdx.x % kCols, rgp = threadIdx.x / kCols;
    const int c = slice * kCols + col;
    float* R = smem;             // [DK][64]
    float* S = smem + DK * kCols;  // [C][C]
    const float l2g = hc.log2g[h];
    const float* qh = q + (size_t)bh * N * DK;
    const float* kh = k + (size_t)bh * N * DK;
    const float* vh = v + (size_t)bh * N * DV;
    // value row t: row t of the prefix buffer below vsplit, else row t - vshift of v (VShift)
    auto vat = [&](int t) __attribute__((always_inline)) {
        return t < vsplit ? vpre[((size_t)bh * vsplit + t) * DV + c] : vh[(size_t)(t - vshift) * DV + c];
    };

    for (int i = rgp; i < DK; i += 4) R[i * kCols + col] = state_in ? state_in[((size_t)bh * DK + i) * DV + c] : 0.f;
    __syncthreads();

    for (int c0 = 0; c0 < N; c0 += C) {
        const int L = min(C, N - c0);
        if (out) {
            for (int idx = threadIdx.x; idx < L * L; idx += kThreads) {
                const int j = idx / L, t = idx % L;
                float s = 0.f;
                if (t <= j) {
                    const float* qj = qh + (size_t)(c0 + j) * DK;
                    const float* kt = kh + (size_t)(c0 + t) * DK;
                    for (int i = 0; i < DK; ++i) s += qj[i] * kt[i];
                    s *= decay_pow(l2g, (float)(j - t));
                }
                S[j * C + t] = s;
            }
            __syncthreads();
            for (int j = rgp; j < L; j += 4) {
                const float* qj = qh + (size_t)(c0 + j) * DK;
                float inter = 0.f;
                for (int i = 0; i < DK; ++i) inter += qj[i] * R[i * kCols + col];
                float intra = 0.f;
                for (int t = 0; t <= j; ++t) intra += S[j * C + t] * vat(c0 + t);
                out[((size_t)bh * N + c0 + j) * DV + c] = intra + decay_pow(l2g, (float)(j + 1)) * inter;
            }
            __syncthreads();  // R is read above and rewritten below
        }
        const float gL = decay_pow(l2g, (float)L);
        for (int i = rgp; i < DK; i += 4) {
            float acc = 0.f;
            for (int t = 0; t < L; ++t)
                acc += decay_pow(l2g, (float)(L - 1 - t)) * kh[(size_t)(c0 + t) * DK + i] * vat(c0 + t);
            R[i * kCols + col] = gL * R[i * kCols + col] + acc;
        }
        __syncthreads();
    }
    if (state_out)
        for (int i = rgp; i < DK; i += 4) state_out[((size_t)bh * DK + i) * DV + c] = R[i * kCols + col];
}

// Grid: (ceil(N/64), B*H*(DV/64)). Thread t: column t % 64, query rows rgp, rgp+4, ... (16 rows).
// LDS: S [64][64] for one key block.
__global__ __launch_bounds__(kThreads) void parallel_f32_kernel(int H, int N, int DK, int DV, const float* __restrict__ q,
                                                                const float* __restrict__ k, const float* __restrict__ v,
                                                                float* __restrict__ out, HeadConsts hc) {
    __shared__ float S[64][65];
    const int nsl = DV / kCols;
    const int qb = blockIdx.x, bh = blockIdx.y / nsl, slice = blockIdx.y % nsl, h = bh % H;
    const int col = threadIdx.x % kCols, rgp = threadIdx.x / kCols;
    const int c = slice * kCols + col;
    const float l2g = hc.log2g[h];
    const float* qh = q + (size_t)bh * N * DK;
    const float* kh = k + (size_t)bh * N * DK;
    const float* vh = v + (size_t)bh * N * DV;
    const int n0 = qb * 64;
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    for (int m0 = 0; m0 <= n0; m0 += 64) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < 64 * 64; idx += kThreads) {
            const int a = idx / 64, b = idx % 64;
            const int n = n0 + a, m = m0 + b;
            float s = 0.f;
            if (n < N && m < N && m <= n) {
                const float* qn = qh + (size_t)n * DK;
                const float* km = kh + (size_t)m * DK;
                for (int i = 0; i < DK; ++i) s += qn[i] * km[i];
                s *= decay_pow(l2g, (float)(n - m));
            }
            S[a][b] = s;
        }
        __syncthreads();
        const int mlim = min(64, N - m0);
        for (int b = 0; b < mlim; ++b) {
            const float vv = vh[(size_t)(m0 + b) * DV + c];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] += S[rgp + 4 * r][b] * vv;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int n = n0 + rgp + 4 * r;
        if (n < N) out[((size_t)bh * N + n) * DV + c] = acc[r];
    }
}

// One wave per (b, h, n) row: y = (x - mean) / sqrt(var + eps) * w + b over DV channels, times
// swish(gate) when a gate is given.
template <typename TOUT>
__global__ __launch_bounds__(kThreads) void groupnorm_rows_kernel(long rows, int H, int N, int DV, const float* __restrict__ x,
                                                                  TOUT* __restrict__ y, GnArgs gn) {
    const long row = (long)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= rows) return;
    const int h = (int)((row / N) % H);
    const float* xr = x + (size_t)row * DV;
    float s = 0.f;
    for (int c = lane; c < DV; c += kWave) s += xr[c];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s / (float)DV;
    float m2 = 0.f;
    for (int c = lane; c < DV; c += kWave) m2 += (xr[c] - mean) * (xr[c] - mean);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m2 += __shfl_xor(m2, off, 64);
    const float inv = rsqrtf(m2 / (float)DV + gn.eps);
    for (int c = lane; c < DV; c += kWave) {
        const float wv = gn.weight ? gn.weight[(size_t)h * DV + c] : 1.f;
        const float bv = gn.bias ? gn.bias[(size_t)h * DV + c] : 0.f;
        const float gs = gn.gate ? swish(gate_at(gn, (size_t)row * DV + c)) : 1.f;
        y[(size_t)row * DV + c] = from_float<TOUT>(((xr[c] - mean) * inv * wv + bv) * gs);
    }
}

__global__ void cast_rows_kernel(size_t n, const float* __restrict__ x, bf16* __restrict__ y) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) y[i] = (bf16)x[i];
}

// Where the pre-norm fp32 output goes: into `out` itself when out is fp32, else the workspace.
bool needs_staging(int gn, int out_bf16) { return gn || out_bf16; }

hipError_t finish(const LaunchArgs& a, float* pre) {
    const long rows = (long)a.B * a.H * a.N;
    if (a.gn.enabled) {
        const unsigned grid = (unsigned)((rows + 3) / 4);
        if (a.out_bf16)
            hipLaunchKernelGGL(groupnorm_rows_kernel<bf16>, dim3(grid), dim3(kThreads), 0, a.stream, rows, a.H, a.N, a.DV, pre,
                               (bf16*)a.out, a.gn);
        else
            hipLaunchKernelGGL(groupnorm_rows_kernel<float>, dim3(grid), dim3(kThreads), 0, a.stream, rows, a.H, a.N, a.DV, pre,
                               (float*)a.out, a.gn);
    } else if (a.out_bf16) {
        hipLaunchKernelGGL(cast_rows_kernel, dim3(1024), dim3(kThreads), 0, a.stream, (size_t)rows * a.DV, pre, (bf16*)a.out);
    }
    return hipGetLastError();
}

}  // namespace

bool chunkwise_f32_supported(int DK, int DV, int chunk) {
    return (DK == 64 || DK == 128 || DK == 256) && DV % kCols == 0 && DV <= 512 && (chunk == 64 || chunk == 128);
}
bool parallel_f32_supported(int DK, int DV) { return DK >= 1 && DK <= 512 && DV % kCols == 0 && DV <= 512; }

size_t chunkwise_f32_workspace(int B, int H, int N, int DV, int gn, int out_bf16) {
    return needs_staging(gn, out_bf16) ? (size_t)B * H * N * DV * sizeof(float) : 0;
}
size_t parallel_f32_workspace(int B, int H, int N, int DV, int gn, int out_bf16) {
    return chunkwise_f32_workspace(B, H, N, DV, gn, out_bf16);
}

hipError_t launch_chunkwise_f32(const LaunchArgs& a) {
    const bool stage = a.out && needs_staging(a.gn.enabled, a.out_bf16);
    float* pre = a.out ? (stage ? (float*)a.ws : (float*)a.out) : nullptr;
    const size_t lds = ((size_t)a.DK * kCols + (size_t)a.chunk * a.chunk) * sizeof(float);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_f32_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_f32_kernel, dim3(a.B * a.H * (a.DV / kCols)), dim3(kThreads), lds, a.stream, a.H, a.N, a.DK, a.DV,
                       a.chunk, (const float*)a.q, (const float*)a.k, (const float*)a.v, a.state_in, a.state_out, pre, a.hc,
                       (const float*)a.vs.pre, a.vs.split, a.vs.shift);
    e = hipGetLastError();
    if (e != hipSuccess || !stage) return e;
    return finish(a, pre);
}

hipError_t launch_parallel_f32(const LaunchArgs& a) {
    const bool stage = needs_staging(a.gn.enabled, a.out_bf16);
    float* pre = stage ? (float*)a.ws : (float*)a.out;
    hipLaunchKernelGGL(parallel_f32_kernel, dim3((a.N + 63) / 64, a.B * a.H * (a.DV / kCols)), dim3(kThreads), 0, a.stream, a.H,
                       a.N, a.DK, a.DV, (const float*)a.q, (const float*)a.k, (const float*)a.v, pre, a.hc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !stage) return e;
    return finish(a, pre);
}

}  // namespace ret

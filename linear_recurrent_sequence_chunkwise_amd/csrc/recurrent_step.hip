// Recurrent decode step (abeam.tech RetNet summary, "Training in parallel, generation by state
// update"): per (b, h), S <- gamma_h S + k^T v in place, then o = q S with the updated S, plus an
// optional per-head GroupNorm of o (mlnews.online RetNet page, bullet summary).
//
// HBM-bound: the fp32 state (d_k x d_v per head) is read once and written once; q, k, v and o
// are tiny. One workgroup owns one (b, h) state so the GroupNorm row stays inside it. Each thread
// streams float4 column groups of the state rows with non-temporal 16-byte loads and stores,
// eight rows in flight, and the per-thread partial products q_i * S_i are reduced across row
// groups through LDS in a fixed order.
#include "common.hpp"

namespace ret {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) red[w] = x;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) s += red[i];
    return s;
}

template <typename TIN> __device__ __forceinline__ f32x4 load4(const TIN* p);
template <> __device__ __forceinline__ f32x4 load4<float>(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <> __device__ __forceinline__ f32x4 load4<bf16>(const bf16* p) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// Grid: B*H workgroups of 256 threads. DV/4 column groups (CG) must divide 256; the
// 256/CG row groups (RG) stride over the d_k rows. Dynamic LDS: q and k (2*DK floats) and
// RG*DV floats for the cross-row-group reduction.
template <typename TIN, typename TOUT>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(
    int H, int DK, int DV, const TIN* __restrict__ q, const TIN* __restrict__ k, const TIN* __restrict__ v,
    float* __restrict__ state, TOUT* __restrict__ out, HeadConsts hc, GnArgs gn) {
    extern __shared__ float smem[];
    __shared__ float red[kThreads / kWave];
    const int bh = blockIdx.x, h = bh % H, t = threadIdx.x;
    const int CG = DV >> 2, RG = kThreads / CG;
    const int cg = t % CG, rg = t / CG;
    float* qs = smem;
    float* ks = smem + DK;
    float* part = smem + 2 * DK;  // [RG][DV]

    for (int i = t; i < DK; i += kThreads) {
        qs[i] = to_float(q[(size_t)bh * DK + i]);
        ks[i] = to_float(k[(size_t)bh * DK + i]);
    }
    const f32x4 vv = load4<TIN>(v + (size_t)bh * DV + 4 * cg);
    __syncthreads();

    const float g = hc.gamma[h];
    f32x4* S = reinterpret_cast<f32x4*>(state + (size_t)bh * DK * DV);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int i = rg;
    // eight rows in flight per thread
    for (; i + 7 * RG < DK; i += 8 * RG) {
        f32x4 s[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] = __builtin_nontemporal_load(S + (size_t)(i + u * RG) * CG + cg);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = i + u * RG;
            const f32x4 n = g * s[u] + ks[r] * vv;
            __builtin_nontemporal_store(n, S + (size_t)r * CG + cg);
            acc += qs[r] * n;
        }
    }
    for (; i < DK; i += RG) {
        const f32x4 s = __builtin_nontemporal_load(S + (size_t)i * CG + cg);
        const f32x4 n = g * s + ks[i] * vv;
        __builtin_nontemporal_store(n, S + (size_t)i * CG + cg);
        acc += qs[i] * n;
    }
    if (out == nullptr) return;

    reinterpret_cast<f32x4*>(part)[rg * CG + cg] = acc;
    __syncthreads();
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (rg == 0) {
        for (int r = 0; r < RG; ++r) {  // fixed order
            const f32x4 p = reinterpret_cast<const f32x4*>(part)[r * CG + cg];
            o[0] += p[0]; o[1] += p[1]; o[2] += p[2]; o[3] += p[3];
        }
    }
    if (gn.enabled) {
        const float mean = block_sum(rg == 0 ? (o[0] + o[1]) + (o[2] + o[3]) : 0.f, red) / (float)DV;
        float m2 = 0.f;
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m2 += (o[j] - mean) * (o[j] - mean);
        }
        const float var = block_sum(m2, red) / (float)DV;
        const float inv = rsqrtf(var + gn.eps);
        if (rg == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 4 * cg + j;
                const float w = gn.weight ? gn.weight[(size_t)h * DV + c] : 1.f;
                const float b = gn.bias ? gn.bias[(size_t)h * DV + c] : 0.f;
                o[j] = (o[j] - mean) * inv * w + b;
            }
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[(size_t)bh * DV + 4 * cg + j] = from_float<TOUT>(o[j]);
    }
}

template <typename TIN, typename TOUT>
hipError_t launch_typed(const LaunchArgs& a) {
    const int CG = a.DV / 4, RG = kThreads / CG;
    const size_t lds = (size_t)(2 * a.DK + RG * a.DV) * sizeof(float);
    hipLaunchKernelGGL((recurrent_step_kernel<TIN, TOUT>), dim3(a.B * a.H), dim3(kThreads), lds, a.stream, a.H, a.DK,
                       a.DV, (const TIN*)a.q, (const TIN*)a.k, (const TIN*)a.v, a.state_out, (TOUT*)a.out, a.hc, a.gn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent_step(const LaunchArgs& a) {
    if (a.in_bf16) return a.out_bf16 ? launch_typed<bf16, bf16>(a) : launch_typed<bf16, float>(a);
    return a.out_bf16 ? launch_typed<float, bf16>(a) : launch_typed<float, float>(a);
}

}  // namespace ret

// Recurrent decode step (abeam.tech RetNet summary, "Training in parallel, generation by state
// update"): per (b, h), S <- gamma_h S + k^T v in place, then o = q S with the updated S, plus an
// optional per-head GroupNorm of o (mlnews.online RetNet page, bullet summary).
//
// HBM-bound: the fp32 state (d_k x d_v per head) is read once and written once; q, k, v and o
// are tiny. One 512-thread workgroup owns one (b, h) state so the GroupNorm row stays inside it.
// Each thread streams float4 column groups of the state rows through 16-byte buffer loads and
// stores with the non-temporal cache policy (stores also sc1: written through, not kept in L2),
// eight rows in flight, and the per-thread partial products q_i * S_i are reduced across row
// groups through LDS in a fixed order. Measured on MI355X with a random state: this shape streams
// at about 6.0 TB/s; 1024-thread workgroups, 256-thread workgroups, software-pipelined batches and
// 16-byte global (not buffer) accesses with the non-temporal builtins are all slower.
#include "common.hpp"

namespace ret {
namespace {

constexpr int kThreads = 512;
constexpr int kLoadNT = 2;        // buffer cache policy: nt
constexpr int kStoreNT = 2 | 16;  // nt | sc1

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

// Grid: B*H workgroups of kThreads. DV/4 column groups (CG) must divide kThreads; the
// kThreads/CG row groups (RG) stride over the d_k rows. Dynamic LDS: q and k (2*DK floats) and
// RG*DV floats for the cross-row-group reduction. One state is at most 32 MiB (d_k <= 8192,
// d_v <= 1024), so byte offsets fit the 32-bit buffer range.
// DV is a template parameter so that the row strides of the eight loads in flight are
// compile-time constants: the loads are then issued in the order they are consumed and each
// wait drains only the oldest one.
// ROT: q and k are turned by the positional rotation at this step's position (the offset) as they
// come into LDS, in fp32 (pair (2i, 2i+1) by the cos and sin that the host formed in double
// precision), so the turned values are never rounded to the input dtype. Wave w turns pairs
// 64 w + lane. The wave reads its 64 pairs' cos and sin out of the kernel arguments at
// compile-time offsets (scalar loads) and writes each into its lane (v_writelane), in uniform
// control flow: indexing the argument block by lane would make every workgroup fetch the whole
// table with vector loads.
template <bool ROT>
__device__ __forceinline__ void pick_turn(const typename IfRot<ROT, StepRot>::type& rc, int w, float& cs, float& sn) {
    if constexpr (ROT) {
        static_assert(kMaxPairs == 2 * kWave, "two waves cover the pairs");
        int c = 0, s = 0;
        // the wave index made scalar, so that the branch and every offset below are wave-uniform
        if (__builtin_amdgcn_readfirstlane(w) == 0) {
#pragma unroll
            for (int j = 0; j < kWave; ++j) {
                asm("v_writelane_b32 %0, %1, %2" : "+v"(c) : "s"(__builtin_bit_cast(int, rc.cs[j])), "i"(j));
                asm("v_writelane_b32 %0, %1, %2" : "+v"(s) : "s"(__builtin_bit_cast(int, rc.sn[j])), "i"(j));
            }
        } else {
#pragma unroll
            for (int j = 0; j < kWave; ++j) {
                asm("v_writelane_b32 %0, %1, %2" : "+v"(c) : "s"(__builtin_bit_cast(int, rc.cs[kWave + j])), "i"(j));
                asm("v_writelane_b32 %0, %1, %2" : "+v"(s) : "s"(__builtin_bit_cast(int, rc.sn[kWave + j])), "i"(j));
            }
        }
        cs = __builtin_bit_cast(float, c);
        sn = __builtin_bit_cast(float, s);
    }
}

template <typename TIN, typename TOUT, int DV, bool ROT>
__global__ __launch_bounds__(kThreads) void recurrent_step_kernel(
    int H, int DK, const TIN* __restrict__ q, const TIN* __restrict__ k, const TIN* __restrict__ v,
    float* __restrict__ state, TOUT* __restrict__ out, HeadConsts hc, GnArgs gn, typename IfRot<ROT, StepRot>::type rc) {
    extern __shared__ float smem[];
    __shared__ float red[kThreads / kWave];
    const int bh = blockIdx.x, h = bh % H, t = threadIdx.x;
    constexpr int CG = DV >> 2, RG = kThreads / CG;
    const int cg = t % CG, rg = t / CG;
    float* qs = smem;
    float* ks = smem + DK;
    float* part = smem + 2 * DK;  // [RG][DV]

    if constexpr (ROT) {
        if (t < DK / 2) {  // DK / 2 <= kMaxPairs = 2 waves
            const int i = t;
            float sn, cs;
            pick_turn<ROT>(rc, t >> 6, cs, sn);
            const size_t e = (size_t)bh * DK + 2 * i;
            const float qa = to_float(q[e]), qb = to_float(q[e + 1]), ka = to_float(k[e]), kb = to_float(k[e + 1]);
            qs[2 * i] = qa * cs - qb * sn;
            qs[2 * i + 1] = qa * sn + qb * cs;
            ks[2 * i] = ka * cs - kb * sn;
            ks[2 * i + 1] = ka * sn + kb * cs;
        }
    } else {
        for (int i = t; i < DK; i += kThreads) {
            qs[i] = to_float(q[(size_t)bh * DK + i]);
            ks[i] = to_float(k[(size_t)bh * DK + i]);
        }
    }
    const f32x4 vv = load4<TIN>(v + (size_t)bh * DV + 4 * cg);
    __syncthreads();

    const float g = hc.gamma[h];
    // The state's base address passes through readfirstlane: it is wave-uniform anyway, but after
    // the rotation's lane-divergent prologue the compiler cannot prove it, and a descriptor it
    // takes for divergent gets a readfirstlane loop around every buffer access (measured: the
    // rotated step 14% slower than the plain one).
    const uint64_t sb = reinterpret_cast<uint64_t>(state + (size_t)bh * DK * DV);
    const uint64_t sbu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(sb >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(sbu), 0, (unsigned)__builtin_amdgcn_readfirstlane(DK * DV * 4), 0x00020000);
    auto ld = [&](int r) __attribute__((always_inline)) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)((r * CG + cg) * 16), 0, kLoadNT));
    };
    auto st = [&](int r, f32x4 x) __attribute__((always_inline)) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, (unsigned)((r * CG + cg) * 16), 0, kStoreNT);
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int i = rg;
    // eight rows in flight per thread: all eight loads, then the updates and stores
    for (; i + 7 * RG < DK; i += 8 * RG) {
        f32x4 s[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) s[u] = ld(i + u * RG);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int r = i + u * RG;
            const f32x4 n = g * s[u] + ks[r] * vv;
            st(r, n);
            acc += qs[r] * n;
        }
    }
    for (; i < DK; i += RG) {
        const f32x4 n = g * ld(i) + ks[i] * vv;
        st(i, n);
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
                if (gn.gate) o[j] *= swish(gate_at(gn, (size_t)bh * DV + c));  // the swish gate after GroupNorm
            }
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[(size_t)bh * DV + 4 * cg + j] = from_float<TOUT>(o[j]);
    }
}

template <typename TIN, typename TOUT, int DV, bool ROT>
hipError_t launch_dv_r(const LaunchArgs& a, typename IfRot<ROT, StepRot>::type rc) {
    constexpr int CG = DV / 4, RG = kThreads / CG;
    const size_t lds = (size_t)(2 * a.DK + RG * DV) * sizeof(float);
    const void* kern = reinterpret_cast<const void*>(recurrent_step_kernel<TIN, TOUT, DV, ROT>);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((recurrent_step_kernel<TIN, TOUT, DV, ROT>), dim3(a.B * a.H), dim3(kThreads), lds, a.stream, a.H, a.DK,
                       (const TIN*)a.q, (const TIN*)a.k, (const TIN*)a.v, a.state_out, (TOUT*)a.out, a.hc, a.gn, rc);
    return hipGetLastError();
}

template <typename TIN, typename TOUT, int DV>
hipError_t launch_dv(const LaunchArgs& a) {
    if (a.step_rot) {
        if (a.DK % 2 || a.DK / 2 > kMaxPairs) return hipErrorInvalidValue;
        return launch_dv_r<TIN, TOUT, DV, true>(a, *a.step_rot);
    }
    return launch_dv_r<TIN, TOUT, DV, false>(a, NoRot{});
}

// d_v / 4 divides 256 (checked by the caller): d_v in {4, 8, ..., 1024}
template <typename TIN, typename TOUT>
hipError_t launch_typed(const LaunchArgs& a) {
    switch (a.DV) {
        case 4: return launch_dv<TIN, TOUT, 4>(a);
        case 8: return launch_dv<TIN, TOUT, 8>(a);
        case 16: return launch_dv<TIN, TOUT, 16>(a);
        case 32: return launch_dv<TIN, TOUT, 32>(a);
        case 64: return launch_dv<TIN, TOUT, 64>(a);
        case 128: return launch_dv<TIN, TOUT, 128>(a);
        case 256: return launch_dv<TIN, TOUT, 256>(a);
        case 512: return launch_dv<TIN, TOUT, 512>(a);
        case 1024: return launch_dv<TIN, TOUT, 1024>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent_step(const LaunchArgs& a) {
    if (a.in_bf16) return a.out_bf16 ? launch_typed<bf16, bf16>(a) : launch_typed<bf16, float>(a);
    return a.out_bf16 ? launch_typed<float, bf16>(a) : launch_typed<float, float>(a);
}

}  // namespace ret

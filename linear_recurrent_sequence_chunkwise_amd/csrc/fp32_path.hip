// fp32-input retention on the vector ALU: the chunkwise form, the parallel form, and a row-wise
// per-head GroupNorm pass. On gfx950 the fp32 matrix cores and the fp32 vector units have the
// same peak rate, so this path uses plain fused multiply-adds with LDS-staged operands and register
// blocking. It serves fp32 inputs (tolerance 1e-4): every product and sum in fp32.
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

// Grid: B*H*(DV/64) workgroups of 256 threads, one (b, h, 64-column slice) each, walking the
// chunks in order. Thread (ty, tx) = (t / 16, t % 16) owns rows j = ty + 16 r of a chunk (r < C/16)
// and columns 4 tx .. 4 tx + 3 of the slice; for the scores also keys tx + 16 c; for the state
// rows d = ty + 16 r of R. Per chunk, with register blocking and operands staged in LDS:
//   A  S = Q K^T and Q R together, over d_k in 16-wide tiles of Q and K (rows padded to 17 floats,
//      so the 16 key rows a wave reads sit in distinct banks); then S (.) D into LDS and
//      g^(j+1) Q R kept in registers;
//   B  + S V over 16-token tiles of V; the rows go out as 16-byte stores;
//   C  R <- g^L R + K^T (V (.) zeta) over 16-token tiles of K and zeta-scaled V.
// LDS: R [DK][64], S [C][C+1], and one tile region shared by the phases.
template <int DK, int C>
__global__ __launch_bounds__(kThreads) void chunk_f32_kernel(int H, int N, int DV, const float* __restrict__ q,
                                                             const float* __restrict__ k, const float* __restrict__ v,
                                                             const float* __restrict__ state_in, float* __restrict__ state_out,
                                                             float* __restrict__ out, HeadConsts hc, const float* __restrict__ vpre,
                                                             int vsplit, int vshift) {
    constexpr int RB = C / 16;    // chunk rows per thread (and key columns of S per thread)
    constexpr int RD = DK / 16;   // state rows per thread
    constexpr int TK = 16;        // d_k tile of phase A, token tile of phases B and C
    constexpr int LQ = TK + 1;    // padded row of the Q and K tiles
    extern __shared__ float smem[];
    float* R = smem;                                  // [DK][64]
    float* S = R + DK * kCols;                        // [C][C + 1]
    float* U = S + C * (C + 1);                       // tiles
    float* Qs = U;                                    // A: [C][LQ]
    float* Ks = U + C * LQ;                           // A: [C][LQ]
    float* Vs = U;                                    // B: [TK][64]
    float* Kt = U;                                    // C: [TK][DK]
    float* Vt = U + TK * DK;                          // C: [TK][64]
    const int nsl = DV / kCols;
    const int bh = blockIdx.x / nsl, slice = blockIdx.x % nsl, h = bh % H;
    const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
    const int col0 = slice * kCols;
    const float l2g = hc.log2g[h];
    const float* qh = q + (size_t)bh * N * DK;
    const float* kh = k + (size_t)bh * N * DK;
    const float* vh = v + (size_t)bh * N * DV;
    // value row t, columns col0 + c .. + 3: row t of the prefix buffer below vsplit, else row t - vshift of v
    auto vrow4 = [&](int t, int c) __attribute__((always_inline)) {
        const float* p = t < vsplit ? vpre + ((size_t)bh * vsplit + t) * DV : vh + (size_t)(t - vshift) * DV;
        return *reinterpret_cast<const float4*>(p + col0 + c);
    };

    for (int i = tid; i < DK * kCols; i += kThreads) {
        const int d = i / kCols, c = i % kCols;
        R[i] = state_in ? state_in[((size_t)bh * DK + d) * DV + col0 + c] : 0.f;
    }
    __syncthreads();

    for (int c0 = 0; c0 < N; c0 += C) {
        const int L = min(C, N - c0);
        if (out) {
            // ---- A: S = Q K^T and Q R
            float acc[RB][RB], aq[RB][4];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
#pragma unroll
                for (int c = 0; c < RB; ++c) acc[r][c] = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) aq[r][c] = 0.f;
            }
            for (int d0 = 0; d0 < DK; d0 += TK) {
                for (int f = tid; f < C * TK / 4; f += kThreads) {
                    const int j = f / (TK / 4), kq = f % (TK / 4);
                    float4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
                    if (j < L) {
                        a = *reinterpret_cast<const float4*>(qh + (size_t)(c0 + j) * DK + d0 + 4 * kq);
                        b = *reinterpret_cast<const float4*>(kh + (size_t)(c0 + j) * DK + d0 + 4 * kq);
                    }
                    float* qd = Qs + j * LQ + 4 * kq;
                    float* kd = Ks + j * LQ + 4 * kq;
                    qd[0] = a.x; qd[1] = a.y; qd[2] = a.z; qd[3] = a.w;
                    kd[0] = b.x; kd[1] = b.y; kd[2] = b.z; kd[3] = b.w;
                }
                __syncthreads();
#pragma unroll 4
                for (int kk = 0; kk < TK; ++kk) {
                    float a[RB], b[RB];
#pragma unroll
                    for (int r = 0; r < RB; ++r) a[r] = Qs[(ty + 16 * r) * LQ + kk];
#pragma unroll
                    for (int c = 0; c < RB; ++c) b[c] = Ks[(tx + 16 * c) * LQ + kk];
                    const float4 rr = *reinterpret_cast<const float4*>(R + (d0 + kk) * kCols + 4 * tx);
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
#pragma unroll
                        for (int c = 0; c < RB; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
                        aq[r][0] = fmaf(a[r], rr.x, aq[r][0]);
                        aq[r][1] = fmaf(a[r], rr.y, aq[r][1]);
                        aq[r][2] = fmaf(a[r], rr.z, aq[r][2]);
                        aq[r][3] = fmaf(a[r], rr.w, aq[r][3]);
                    }
                }
                __syncthreads();
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int j = ty + 16 * r;
#pragma unroll
                for (int c = 0; c < RB; ++c) {
                    const int t = tx + 16 * c;
                    S[j * (C + 1) + t] = t <= j && j < L ? acc[r][c] * decay_pow(l2g, (float)(j - t)) : 0.f;
                }
                const float dj = decay_pow(l2g, (float)(j + 1));
#pragma unroll
                for (int c = 0; c < 4; ++c) aq[r][c] *= dj;
            }
            __syncthreads();
            // ---- B: + S V
            for (int t0 = 0; t0 < L; t0 += TK) {
                {
                    const int tt = tid / 16, cq = tid % 16;
                    const float4 x = t0 + tt < L ? vrow4(c0 + t0 + tt, 4 * cq) : float4{0.f, 0.f, 0.f, 0.f};
                    *reinterpret_cast<float4*>(Vs + tt * kCols + 4 * cq) = x;
                }
                __syncthreads();
#pragma unroll 4
                for (int tt = 0; tt < TK; ++tt) {
                    const float4 vv = *reinterpret_cast<const float4*>(Vs + tt * kCols + 4 * tx);
#pragma unroll
                    for (int r = 0; r < RB; ++r) {
                        const float sv = S[(ty + 16 * r) * (C + 1) + t0 + tt];
                        aq[r][0] = fmaf(sv, vv.x, aq[r][0]);
                        aq[r][1] = fmaf(sv, vv.y, aq[r][1]);
                        aq[r][2] = fmaf(sv, vv.z, aq[r][2]);
                        aq[r][3] = fmaf(sv, vv.w, aq[r][3]);
                    }
                }
                __syncthreads();
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int j = ty + 16 * r;
                if (j < L)
                    *reinterpret_cast<float4*>(out + ((size_t)bh * N + c0 + j) * DV + col0 + 4 * tx) =
                        float4{aq[r][0], aq[r][1], aq[r][2], aq[r][3]};
            }
        }
        // ---- C: R <- g^L R + K^T (V (.) zeta), zeta_t = g^(L-1-t)
        float ar[RD][4];
        const float gL = decay_pow(l2g, (float)L);
#pragma unroll
        for (int r = 0; r < RD; ++r) {
            const float4 x = *reinterpret_cast<const float4*>(R + (ty + 16 * r) * kCols + 4 * tx);
            ar[r][0] = gL * x.x; ar[r][1] = gL * x.y; ar[r][2] = gL * x.z; ar[r][3] = gL * x.w;
        }
        for (int t0 = 0; t0 < L; t0 += TK) {
            for (int f = tid; f < TK * DK / 4; f += kThreads) {
                const int tt = f / (DK / 4), dq = f % (DK / 4);
                const float4 x = t0 + tt < L ? *reinterpret_cast<const float4*>(kh + (size_t)(c0 + t0 + tt) * DK + 4 * dq)
                                             : float4{0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<float4*>(Kt + tt * DK + 4 * dq) = x;
            }
            {
                const int tt = tid / 16, cq = tid % 16, t = t0 + tt;
                float4 x = {0.f, 0.f, 0.f, 0.f};
                if (t < L) {
                    x = vrow4(c0 + t, 4 * cq);
                    const float z = decay_pow(l2g, (float)(L - 1 - t));
                    x.x *= z; x.y *= z; x.z *= z; x.w *= z;
                }
                *reinterpret_cast<float4*>(Vt + tt * kCols + 4 * cq) = x;
            }
            __syncthreads();
#pragma unroll 4
            for (int tt = 0; tt < TK; ++tt) {
                const float4 vv = *reinterpret_cast<const float4*>(Vt + tt * kCols + 4 * tx);
#pragma unroll
                for (int r = 0; r < RD; ++r) {
                    const float kv = Kt[tt * DK + ty + 16 * r];
                    ar[r][0] = fmaf(kv, vv.x, ar[r][0]);
                    ar[r][1] = fmaf(kv, vv.y, ar[r][1]);
                    ar[r][2] = fmaf(kv, vv.z, ar[r][2]);
                    ar[r][3] = fmaf(kv, vv.w, ar[r][3]);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int r = 0; r < RD; ++r)
            *reinterpret_cast<float4*>(R + (ty + 16 * r) * kCols + 4 * tx) = float4{ar[r][0], ar[r][1], ar[r][2], ar[r][3]};
        __syncthreads();
    }
    if (state_out)
        for (int i = tid; i < DK * kCols; i += kThreads) {
            const int d = i / kCols, c = i % kCols;
            state_out[((size_t)bh * DK + d) * DV + col0 + c] = R[i];
        }
}

template <int DK, int C>
size_t chunk_f32_lds() {
    constexpr size_t tiles = (2 * C * 17 > 16 * DK + 16 * kCols) ? 2 * C * 17 : 16 * DK + 16 * kCols;
    return ((size_t)DK * kCols + (size_t)C * (C + 1) + tiles) * sizeof(float);
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

template <int DK, int C>
hipError_t launch_chunk_f32_t(const LaunchArgs& a, float* pre) {
    const size_t lds = chunk_f32_lds<DK, C>();
    const void* kern = reinterpret_cast<const void*>(chunk_f32_kernel<DK, C>);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((chunk_f32_kernel<DK, C>), dim3(a.B * a.H * (a.DV / kCols)), dim3(kThreads), lds, a.stream, a.H, a.N, a.DV,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, a.state_in, a.state_out, pre, a.hc,
                       (const float*)a.vs.pre, a.vs.split, a.vs.shift);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_chunk_f32_dk(const LaunchArgs& a, float* pre) {
    return a.chunk == 64 ? launch_chunk_f32_t<DK, 64>(a, pre) : launch_chunk_f32_t<DK, 128>(a, pre);
}

hipError_t launch_chunkwise_f32(const LaunchArgs& a) {
    const bool stage = a.out && needs_staging(a.gn.enabled, a.out_bf16);
    float* pre = a.out ? (stage ? (float*)a.ws : (float*)a.out) : nullptr;
    hipError_t e = a.DK == 64 ? launch_chunk_f32_dk<64>(a, pre) : a.DK == 128 ? launch_chunk_f32_dk<128>(a, pre)
                                                                             : launch_chunk_f32_dk<256>(a, pre);
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

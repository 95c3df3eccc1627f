// Positional rotation of q and k before retention (abeam.tech RetNet summary, "Technical
// mechanism": Q and K get a positional rotation after the projections; eulerwa.com "3. RetNet
// 상세": RoPE with the exponential decay). The reading is the rotary position embedding of Su et al.
// (RoFormer): feature pair (2i, 2i+1) at absolute position p turns by p * theta_i,
// theta_i = base^(-2i/d).
//
//   rotate_kernel   one pass over [rows][N][d]: each thread takes 4 consecutive pairs (8 features,
//                   one 16-byte bf16 load or two fp32 loads), or one pair when d is not a multiple
//                   of 8, at 8 consecutive positions, and writes the turned pairs in the output
//                   dtype. HBM-bound: it reads and writes each element once.
#include "common.hpp"

namespace ret {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
    static __device__ __forceinline__ void load(const bf16* p, float* x) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
    }
    static __device__ __forceinline__ void store(bf16* p, const float* x) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (bf16)x[j];
        *reinterpret_cast<bf16x8*>(p) = v;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float* x) {
        const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
    }
    static __device__ __forceinline__ void store(float* p, const float* x) {
        f32x4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = x[j];
            b[j] = x[4 + j];
        }
        reinterpret_cast<f32x4*>(p)[0] = a;
        reinterpret_cast<f32x4*>(p)[1] = b;
    }
};

// A thread takes PAIRS consecutive pairs (4: 8 features, one 16-byte bf16 load; 1 when d is not a
// multiple of 8) of RB consecutive positions n0 .. n0+RB-1 of one (b, h) row block. sin and cos are
// evaluated at n0 and at the per-position step, then advanced by angle addition (each step adds
// about one rounding to them, so about 1e-6 after RB = 8 steps). All loads are issued first.
// sgn = -1 turns the other way (sin negated). x and y may be the same buffer: each thread reads its
// elements before writing them, and no two threads share an element.
constexpr int RB = 8;

// Two tensors in one launch: units [0, units) turn x0 into y0, units [units, 2 units) x1 into y1
// (x1 null: one tensor). With bf16 outputs, lo0 / lo1 (when given) receive the low parts of the
// turned values, value - bf16(value) rounded to bf16, laid out like y0 / y1.
template <typename TI, typename TO, int PAIRS>
__global__ __launch_bounds__(256) void rotate_kernel(long units, int N, int d, const TI* x0, TO* y0, const TI* x1, TO* y1,
                                                     TO* lo0, TO* lo1, RotConsts rc, float sgn) {
    const int per_row = d / (2 * PAIRS);
    const int nblk = (N + RB - 1) / RB;
    const long all = x1 ? 2 * units : units;
    for (long uu = (long)blockIdx.x * blockDim.x + threadIdx.x; uu < all; uu += (long)gridDim.x * blockDim.x) {
        const bool second = uu >= units;
        const long u = second ? uu - units : uu;
        const TI* x = second ? x1 : x0;
        TO* y = second ? y1 : y0;
        TO* lo = second ? lo1 : lo0;
        const int i0 = (int)(u % per_row) * PAIRS;  // first pair
        const long blk = u / per_row;
        const long bh = blk / nblk;
        const int n0 = (int)(blk % nblk) * RB;
        const int rows = min(RB, N - n0);
        const size_t base = ((size_t)bh * N + n0) * d + 2 * i0;
        float v[RB][2 * PAIRS];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (r < rows) {
                if constexpr (PAIRS == 4) {
                    Vec8<TI>::load(x + base + (size_t)r * d, v[r]);
                } else {
                    v[r][0] = (float)x[base + (size_t)r * d];
                    v[r][1] = (float)x[base + (size_t)r * d + 1];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < PAIRS; ++j) {
            const float fhi = rc.fhi[i0 + j], flo = rc.flo[i0 + j];
            float s, c, ss, cs;
            rot_sincos(n0, fhi, flo, rc.ph[i0 + j], s, c);
            sincospif(fhi + flo, &ss, &cs);
            s *= sgn;
            ss *= sgn;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float a = v[r][2 * j], b = v[r][2 * j + 1];
                v[r][2 * j] = a * c - b * s;
                v[r][2 * j + 1] = a * s + b * c;
                const float c2 = c * cs - s * ss;
                s = s * cs + c * ss;
                c = c2;
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (r < rows) {
                if constexpr (PAIRS == 4) {
                    Vec8<TO>::store(y + base + (size_t)r * d, v[r]);
                } else {
                    y[base + (size_t)r * d] = from_float<TO>(v[r][0]);
                    y[base + (size_t)r * d + 1] = from_float<TO>(v[r][1]);
                }
                if (sizeof(TO) == 2 && lo) {
                    float l[2 * PAIRS];
#pragma unroll
                    for (int j = 0; j < 2 * PAIRS; ++j) l[j] = v[r][j] - (float)from_float<TO>(v[r][j]);
                    if constexpr (PAIRS == 4) {
                        Vec8<TO>::store(lo + base + (size_t)r * d, l);
                    } else {
                        lo[base + (size_t)r * d] = from_float<TO>(l[0]);
                        lo[base + (size_t)r * d + 1] = from_float<TO>(l[1]);
                    }
                }
            }
        }
    }
}

template <typename TI, typename TO>
hipError_t launch_t(long rows, int N, int d, const void* x0, void* y0, const void* x1, void* y1, void* lo0, void* lo1,
                    const RotConsts& rc, float sgn, hipStream_t st) {
    const bool vec = d % 8 == 0;
    const long units = rows / N * ((N + RB - 1) / RB) * (long)(d / (vec ? 8 : 2));
    const long blocks = ((x1 ? 2 : 1) * units + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
    if (vec)
        hipLaunchKernelGGL((rotate_kernel<TI, TO, 4>), dim3(grid), dim3(256), 0, st, units, N, d, static_cast<const TI*>(x0),
                           static_cast<TO*>(y0), static_cast<const TI*>(x1), static_cast<TO*>(y1), static_cast<TO*>(lo0),
                           static_cast<TO*>(lo1), rc, sgn);
    else
        hipLaunchKernelGGL((rotate_kernel<TI, TO, 1>), dim3(grid), dim3(256), 0, st, units, N, d, static_cast<const TI*>(x0),
                           static_cast<TO*>(y0), static_cast<const TI*>(x1), static_cast<TO*>(y1), static_cast<TO*>(lo0),
                           static_cast<TO*>(lo1), rc, sgn);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate2(long rows, int N, int d, const void* x0, void* y0, const void* x1, void* y1, int x_bf16, int y_bf16,
                          const RotConsts& rc, int inverse, hipStream_t stream, void* lo0, void* lo1) {
    if (rows <= 0) return hipSuccess;
    const float sgn = inverse ? -1.f : 1.f;
    if (x_bf16 && y_bf16) return launch_t<bf16, bf16>(rows, N, d, x0, y0, x1, y1, lo0, lo1, rc, sgn, stream);
    if (x_bf16) return launch_t<bf16, float>(rows, N, d, x0, y0, x1, y1, nullptr, nullptr, rc, sgn, stream);
    if (y_bf16) return launch_t<float, bf16>(rows, N, d, x0, y0, x1, y1, lo0, lo1, rc, sgn, stream);
    return launch_t<float, float>(rows, N, d, x0, y0, x1, y1, nullptr, nullptr, rc, sgn, stream);
}

hipError_t launch_rotate(long rows, int N, int d, const void* x, int x_bf16, void* y, int y_bf16, const RotConsts& rc, int inverse,
                         hipStream_t stream) {
    return launch_rotate2(rows, N, d, x, y, nullptr, nullptr, x_bf16, y_bf16, rc, inverse, stream);
}

}  // namespace ret

// Residual linear attention (mengro1102.github.io RAttention post, section 4, RLA formula):
//   S_t = S_(t-1) + phi(k_t)^T v_t,   o_t = phi(q_t) S_(t-w-1)
// is retention with gamma = 1 on shifted keys and values: with K'[n] = phi(k[n - w - 1]) and
// V'[n] = v[n - w - 1] (tokens before the segment from the caller's window rows, absent tokens as
// zero rows), o_n = phi(q_n) . sum_(m <= n) K'[m]^T V'[m], and the final state is the sum over the
// tokens that have left the window. phi is the identity or the softmax over the d_k features of a
// row (the page's "softmax-based" feature map).
//
//   rla_prepare_kernel   one wave per (b*h, n) row: phi(q[n]) (unless phi is the identity, where q
//                        is used in place), phi of the shifted key row and the shifted value row,
//                        in the input dtype. d_k <= 256 (4 features per lane in registers); the
//                        softmax in double precision. HBM-bound.
// The retention itself runs in the chunkwise kernels (N > 1) or the decode-step kernel (N = 1).
#include "common.hpp"

namespace ret {
namespace {

__device__ __forceinline__ double wave_max_d(double x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// y = phi(x) over d <= 256 features, lane l holding features l, l + 64, l + 128, l + 192. The
// softmax runs in double precision (exp(x - max) / sum) and is rounded once to fp32, then to the
// output dtype: the rounded features then equal the exactly computed ones rounded the same way,
// except where a value lies within about 1e-16 relative of a rounding boundary.
template <typename T>
__device__ __forceinline__ void feature_row(int fmap, int d, const T* x, T* y, int lane) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = lane + 64 * j;
        v[j] = i < d ? to_float(x[i]) : -INFINITY;
    }
    if (fmap == 1) {
        const double m = wave_max_d((double)fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
        double e[4], s = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            e[j] = lane + 64 * j < d ? exp((double)v[j] - m) : 0.0;
            s += e[j];
        }
        s = wave_sum_d(s);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (float)(e[j] / s);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = lane + 64 * j;
        if (i < d) y[i] = from_float<T>(v[j]);
    }
}

template <typename T>
__device__ __forceinline__ void copy_row(int d, const T* x, T* y, int lane) {
    if ((d * sizeof(T)) % 16 == 0) {
        const int n16 = d * (int)sizeof(T) / 16;
        for (int c = lane; c < n16; c += 64) reinterpret_cast<u32x4*>(y)[c] = reinterpret_cast<const u32x4*>(x)[c];
    } else {
        for (int i = lane; i < d; i += 64) y[i] = x[i];
    }
}

template <typename T>
__device__ __forceinline__ void zero_row(int d, T* y, int lane) {
    for (int i = lane; i < d; i += 64) y[i] = from_float<T>(0.f);
}

template <typename T>
__global__ __launch_bounds__(256) void rla_prepare_kernel(long rows, int N, int dk, int dv, int P, int prev_len, int fmap,
                                                          const T* q, const T* k, const T* v, const T* kp, const T* vp, T* qo,
                                                          T* ko, T* vo) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // the whole wave leaves together
    const int lane = threadIdx.x & 63;
    const long bh = row / N;
    const int n = (int)(row % N);
    if (qo) feature_row(fmap, dk, q + (size_t)row * dk, qo + (size_t)row * dk, lane);
    const int p = n - P;  // position of the token whose key and value land in row n
    const T* ks = nullptr;
    const T* vs = nullptr;
    if (p >= 0) {
        ks = k + ((size_t)bh * N + p) * dk;
        vs = v + ((size_t)bh * N + p) * dv;
    } else if (p >= -prev_len) {
        ks = kp + ((size_t)bh * P + (p + P)) * dk;
        vs = vp + ((size_t)bh * P + (p + P)) * dv;
    }
    if (ks) {
        feature_row(fmap, dk, ks, ko + (size_t)row * dk, lane);
        copy_row(dv, vs, vo + (size_t)row * dv, lane);
    } else {
        zero_row(dk, ko + (size_t)row * dk, lane);
        zero_row(dv, vo + (size_t)row * dv, lane);
    }
}

// dst = src (or zero when src is null), n floats, 16-byte aligned.
__global__ __launch_bounds__(256) void copy_state_kernel(size_t n4, const float* src, float* dst) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
        reinterpret_cast<f32x4*>(dst)[i] = src ? reinterpret_cast<const f32x4*>(src)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

hipError_t launch_rla_prepare(const RlaPrep& r, hipStream_t stream) {
    const long rows = r.rows;
    if (rows <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((rows + 3) / 4);
    if (r.bf16)
        hipLaunchKernelGGL(rla_prepare_kernel<bf16>, dim3(grid), dim3(256), 0, stream, rows, r.N, r.dk, r.dv, r.P, r.prev_len, r.fmap,
                           static_cast<const bf16*>(r.q), static_cast<const bf16*>(r.k), static_cast<const bf16*>(r.v),
                           static_cast<const bf16*>(r.kp), static_cast<const bf16*>(r.vp), static_cast<bf16*>(r.qo),
                           static_cast<bf16*>(r.ko), static_cast<bf16*>(r.vo));
    else
        hipLaunchKernelGGL(rla_prepare_kernel<float>, dim3(grid), dim3(256), 0, stream, rows, r.N, r.dk, r.dv, r.P, r.prev_len, r.fmap,
                           static_cast<const float*>(r.q), static_cast<const float*>(r.k), static_cast<const float*>(r.v),
                           static_cast<const float*>(r.kp), static_cast<const float*>(r.vp), static_cast<float*>(r.qo),
                           static_cast<float*>(r.ko), static_cast<float*>(r.vo));
    return hipGetLastError();
}

hipError_t launch_copy_state(size_t n, const float* src, float* dst, hipStream_t stream) {
    const size_t n4 = n / 4;
    const size_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, n4, src, dst);
    return hipGetLastError();
}

}  // namespace ret

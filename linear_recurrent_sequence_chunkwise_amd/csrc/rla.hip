// Residual linear attention (mengro1102.github.io RAttention post, section 4, RLA formula):
//   S_t = S_(t-1) + phi(k_t)^T v_t,   o_t = phi(q_t) S_(t-w-1)
// is retention with gamma = 1 on shifted keys and values: with K'[n] = phi(k[n - w - 1]) and
// V'[n] = v[n - w - 1] (tokens before the segment from the caller's window rows, absent tokens as
// zero rows), o_n = phi(q_n) . sum_(m <= n) K'[m]^T V'[m], and the final state is the sum over the
// tokens that have left the window. phi is the identity or the softmax over the d_k features of a
// row (the page's "softmax-based" feature map).
//
//   rla_prepare_kernel   grid-stride, one wave per row: first the shifted value rows for n below a
//                        split (w + 1 rounded up to a 32-token stage, at most N), into a prefix
//                        buffer; then, row by row, phi(q[n]) (unless phi is the identity, where q is
//                        used in place) and phi of the shifted key row, in the input dtype, with the
//                        next row's loads in flight. d_k <= 256, a multiple of 4 (4 consecutive
//                        features per lane, one 8- or 16-byte access); the softmax in double
//                        precision for fp32 features, in single precision for bf16 features (stored
//                        as high and low parts).
// The retention itself runs in the chunkwise kernels (N > 1), which read value rows at and past the
// split from v itself, shifted by w + 1 rows (VShift), or the decode-step kernel (N = 1).
#include <algorithm>

#include "common.hpp"

namespace ret {
namespace {

// A lane move within each row of 16 lanes (DPP; all 64 lanes active): quad_perm [1,0,3,2] (lane
// xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror (lane i of 8 from 7 - i), row_mirror (lane i
// of 16 from 15 - i). After the two quad steps every lane of a quad holds the same value, so the
// mirrors pair each lane with the other quad (half-row) as xor 4 (xor 8) would.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xF, 0xF, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Two independent wave reductions at once, so that their moves overlap: four DPP steps within rows
// of 16 lanes, then two shuffles across rows. Every lane ends with the same value (each step adds
// or compares the same two operands in every lane).
__device__ __forceinline__ void wave_max2(float& a, float& b) {
    a = fmaxf(a, dpp_f<0xB1>(a)); b = fmaxf(b, dpp_f<0xB1>(b));
    a = fmaxf(a, dpp_f<0x4E>(a)); b = fmaxf(b, dpp_f<0x4E>(b));
    a = fmaxf(a, dpp_f<0x141>(a)); b = fmaxf(b, dpp_f<0x141>(b));
    a = fmaxf(a, dpp_f<0x140>(a)); b = fmaxf(b, dpp_f<0x140>(b));
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const float x = __shfl_xor(a, o, 64), y = __shfl_xor(b, o, 64);
        a = fmaxf(a, x);
        b = fmaxf(b, y);
    }
}
__device__ __forceinline__ void wave_sum2(double& a, double& b) {
    a += dpp_d<0xB1>(a); b += dpp_d<0xB1>(b);
    a += dpp_d<0x4E>(a); b += dpp_d<0x4E>(b);
    a += dpp_d<0x141>(a); b += dpp_d<0x141>(b);
    a += dpp_d<0x140>(a); b += dpp_d<0x140>(b);
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const double x = __shfl_xor(a, o, 64), y = __shfl_xor(b, o, 64);
        a += x;
        b += y;
    }
}

// Features 4l .. 4l+3 of a row of d <= 256 (lane l, one 8- or 16-byte access; d a multiple of 4);
// -inf past the end or without a row.
template <typename T> struct Vec4;
template <> struct Vec4<bf16> {
    static __device__ __forceinline__ void store(bf16* p, const float* v) {
        bf16x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (bf16)v[j];
        *reinterpret_cast<bf16x4*>(p) = x;
    }
};
template <> struct Vec4<float> {
    static __device__ __forceinline__ void store(float* p, const float* v) {
        *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    }
};

template <typename T>
__device__ __forceinline__ void store_row4(T* y, int d, int lane, const float* v) {
    if (4 * lane < d) Vec4<T>::store(y + 4 * lane, v);
}

// 2^(j/32), j = 0 .. 31, rounded to double (computed to 60 digits)
__constant__ double kExp2Frac[32] = {1.0, 1.0218971486541166, 1.0442737824274138, 1.0671404006768237, 1.0905077326652577, 1.1143867425958924, 1.1387886347566916, 1.1637248587775775, 1.189207115002721, 1.215247359980469, 1.241857812073484, 1.2690509571917332, 1.2968395546510096, 1.3252366431597413, 1.3542555469368927, 1.383909881963832, 1.4142135623730951, 1.4451808069770467, 1.4768261459394993, 1.5091644275934228, 1.5422108254079407, 1.5759808451078865, 1.6104903319492543, 1.645755478153965, 1.681792830507429, 1.718619298122478, 1.7562521603732995, 1.7947090750031072, 1.8340080864093424, 1.8741676341103, 1.9152065613971474, 1.9571441241754002};

// exp(z) for z <= 0 in double precision: z = (32 m + j) ln2/32 + r with ln2/32 split in two (Cody
// and Waite; the two parts of ln 2 are the high/low split published with Sun's fdlibm, whose high
// part has its low bits zero, so n = 32 m + j times it is exact for |n| < 2^21), |r| <= ln2/64, exp(r) by its
// Taylor series to degree 6 (truncation below 4e-18 relative), times 2^(j/32) from the table in
// LDS, scaled by 2^m (ldexp, which flushes to zero below the double range). z is clamped at -746,
// below which exp is zero in double precision. Measured against libm's exp on [-700, 0]: relative
// error below 4e-16.
__device__ __forceinline__ double exp_nonpos(double z, const double* tab) {
    z = fmax(z, -746.0);
    const double n = rint(z * 46.166241308446828);             // 32 / ln 2
    double r = fma(-n, 6.93147180369123816490e-01 / 32, z);     // ln 2 / 32, high part
    r = fma(-n, 1.90821492927058770002e-10 / 32, r);            // ln 2 / 32, low part
    double p = 1.0 / 720.0;
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    const int ni = (int)n;  // in [-34500, 0]
    return ldexp(p * tab[ni & 31], ni >> 5);
}

// phi over two rows at once (a: the q row, b: the key row), in place. The softmax runs in double
// precision, exp(x - max) times the reciprocal of the sum, rounded once to fp32: the rounded
// features then equal the exactly computed ones rounded the same way, except where a value lies
// within about 1e-16 relative of a rounding boundary.
__device__ __forceinline__ void softmax2(int d, int lane, float* a, float* b, const double* tab) {
    float fa = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));  // the maximum of fp32 values is exact in fp32
    float fb = fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3]));
    wave_max2(fa, fb);
    const double ma = fa, mb = fb;
    double ea[4], eb[4], sa = 0.0, sb = 0.0;
    const bool in = 4 * lane < d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ea[j] = in ? exp_nonpos((double)a[j] - ma, tab) : 0.0;
        eb[j] = in ? exp_nonpos((double)b[j] - mb, tab) : 0.0;
        sa += ea[j];
        sb += eb[j];
    }
    wave_sum2(sa, sb);
    const double ia = 1.0 / sa, ib = 1.0 / sb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = (float)(ea[j] * ia);
        b[j] = (float)(eb[j] * ib);
    }
}


__device__ __forceinline__ void wave_sum2f(float& a, float& b) {
    a += dpp_f<0xB1>(a); b += dpp_f<0xB1>(b);
    a += dpp_f<0x4E>(a); b += dpp_f<0x4E>(b);
    a += dpp_f<0x141>(a); b += dpp_f<0x141>(b);
    a += dpp_f<0x140>(a); b += dpp_f<0x140>(b);
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
        const float x = __shfl_xor(a, o, 64), y = __shfl_xor(b, o, 64);
        a += x;
        b += y;
    }
}

// phi over two rows in single precision, for features that are then stored as bf16 high and low
// parts (about 2^-17 relative): exp(x - max) by the device library's expf (about 1 ulp), a
// pairwise sum over the wave (8 levels, below 1e-6 relative), times the reciprocal of the sum.
__device__ __forceinline__ void softmax2_f32(int d, int lane, float* a, float* b) {
    float ma = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
    float mb = fmaxf(fmaxf(b[0], b[1]), fmaxf(b[2], b[3]));
    wave_max2(ma, mb);
    float ea[4], eb[4];
    const bool in = 4 * lane < d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ea[j] = in ? expf(a[j] - ma) : 0.f;
        eb[j] = in ? expf(b[j] - mb) : 0.f;
    }
    float sa = (ea[0] + ea[1]) + (ea[2] + ea[3]), sb = (eb[0] + eb[1]) + (eb[2] + eb[3]);
    wave_sum2f(sa, sb);
    const float ia = 1.f / sa, ib = 1.f / sb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = ea[j] * ia;
        b[j] = eb[j] * ib;
    }
}

// The q and key features 4l .. 4l+3 of one row, as loaded (bf16x4 or f32x4).
template <typename T> struct Raw4;
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <> struct Raw4<float> { typedef f32x4 type; };

// Where row (bh, n) of the prepare pass reads and writes. ks is null where no key row lands (a
// token before the caller's window rows); vs then is null too.
template <typename T>
struct RowAt {
    long row;
    int bh, n;
    const T* ks;
    const T* vs;
};

template <typename T>
__device__ __forceinline__ RowAt<T> locate(int bh, int n, int N, int dk, int dv, int P, int prev_len, const T* k,
                                           const T* v, const T* kp, const T* vp) {
    RowAt<T> r{(long)bh * N + n, bh, n, nullptr, nullptr};
    const int p = n - P;  // position of the token whose key and value land in row n
    if (p >= 0) {
        r.ks = k + ((size_t)bh * N + p) * dk;
        r.vs = v + ((size_t)bh * N + p) * dv;
    } else if (p >= -prev_len) {
        r.ks = kp + ((size_t)bh * P + (p + P)) * dk;
        r.vs = vp + ((size_t)bh * P + (p + P)) * dv;
    }
    return r;
}

// Issues the q and key loads of a row without a condition, so that the compiler's load waits stay
// exact while the loads are in flight across the previous row's work. Lanes past d_k read feature
// 0; an absent key row reads the q row, and with the identity map (want_q false) the q load reads
// the key row again. finish_row discards what these stand-ins read.
template <typename T>
__device__ __forceinline__ void load_row(const RowAt<T>& r, const T* q, int dk, int lane, bool want_q,
                                         typename Raw4<T>::type& xq, typename Raw4<T>::type& xk) {
    const int off = 4 * lane < dk ? 4 * lane : 0;
    const T* qrow = q + (size_t)r.row * dk;
    const T* krow = r.ks ? r.ks : qrow;
    xq = *reinterpret_cast<const typename Raw4<T>::type*>((want_q ? qrow : krow) + off);
    xk = *reinterpret_cast<const typename Raw4<T>::type*>(krow + off);
}

// The rest of one row: phi(q[n]) (unless phi is the identity) and phi of the key row that lands at n
// (zero where none does).
// Stores the bf16 low parts of 4 features (x - bf16(x), rounded) when y is given.
__device__ __forceinline__ void store_lo4(bf16* y, int d, int lane, const float* v) {
    if (!y || 4 * lane >= d) return;
    float lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lo[j] = v[j] - (float)(bf16)v[j];
    Vec4<bf16>::store(y + 4 * lane, lo);
}
__device__ __forceinline__ void store_lo4(float*, int, int, const float*) {}

template <typename T, typename TO>
__device__ __forceinline__ void finish_row(const RowAt<T>& r, const typename Raw4<T>::type& xq,
                                           const typename Raw4<T>::type& xk, int dk, int fmap, int lane,
                                           const double* tab, TO* qo, TO* ko, TO* qlo, TO* klo) {
    const bool live = 4 * lane < dk;
    float fq[4], fk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        fq[j] = live ? (float)xq[j] : -INFINITY;
        fk[j] = live && r.ks ? (float)xk[j] : -INFINITY;
    }
    if (fmap == 1) {
        if constexpr (sizeof(TO) == 2)
            softmax2_f32(dk, lane, fq, fk);  // bf16 features with low parts
        else
            softmax2(dk, lane, fq, fk, tab);
    }
    if (qo) store_row4(qo + (size_t)r.row * dk, dk, lane, fq);
    if (qlo) store_lo4(qlo + (size_t)r.row * dk, dk, lane, fq);
    if (!r.ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fk[j] = 0.f;
    }
    store_row4(ko + (size_t)r.row * dk, dk, lane, fk);
    if (klo) store_lo4(klo + (size_t)r.row * dk, dk, lane, fk);
}

// The next row of a wave's stride after r, or r itself past the end (more false).
template <typename T>
__device__ __forceinline__ RowAt<T> advance(const RowAt<T>& r, int BH, int N, int dk, int dv, int P, int prev_len,
                                            int step_bh, int step_n, const T* k, const T* v, const T* kp, const T* vp,
                                            bool& more) {
    int bh = r.bh + step_bh, n = r.n + step_n;  // step_n < N, so one carry at most
    if (n >= N) {
        n -= N;
        ++bh;
    }
    more = bh < BH;
    return more ? locate<T>(bh, n, N, dk, dv, P, prev_len, k, v, kp, vp) : r;
}

// T: the input dtype; TO: the dtype of the features and value rows written (T, or fp32 for bf16
// inputs whose features the fp32 kernels consume).
template <typename T, typename TO>
__global__ __launch_bounds__(256) void rla_prepare_kernel(int BH, int N, int dk, int dv, int P, int prev_len, int fmap,
                                                          int vsplit, int step_bh, int step_n, const T* q, const T* k,
                                                          const T* v, const T* kp, const T* vp, TO* qo, TO* ko, TO* vo,
                                                          TO* qlo, TO* klo) {
    __shared__ double tab[32];
    if (threadIdx.x < 32) tab[threadIdx.x] = kExp2Frac[threadIdx.x];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    // Rows are wave-uniform, so their index and address arithmetic runs on the scalar unit.
    const int wave = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = (int)gridDim.x * 4;
    // The shifted value rows below vsplit, [B*H][vsplit][d_v] (the chunk kernels read the later rows
    // from v itself): one wave per row, d_v * size / 16 whole 16-byte chunks (bf16 to fp32: 4 values
    // per chunk written).
    const int n16 = dv * (int)sizeof(TO) / 16;
    for (long vr = wave; vr < (long)BH * vsplit; vr += waves) {
        const int bh = (int)(vr / vsplit), n = (int)(vr % vsplit);
        const RowAt<T> r = locate<T>(bh, n, N, dk, dv, P, prev_len, k, v, kp, vp);
        u32x4* dst = reinterpret_cast<u32x4*>(vo + (size_t)vr * dv);
        for (int c = lane; c < n16; c += 64) {
            if constexpr (sizeof(T) == sizeof(TO)) {
                dst[c] = r.vs ? reinterpret_cast<const u32x4*>(r.vs)[c] : u32x4{0u, 0u, 0u, 0u};
            } else {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (r.vs) {
                    const bf16x4 b = reinterpret_cast<const bf16x4*>(r.vs)[c];
                    x = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
                }
                reinterpret_cast<f32x4*>(dst)[c] = x;
            }
        }
    }
    // phi(q) and the shifted phi(k). A wave takes every waves-th row, (step_bh, step_n) in (b*h, n)
    // form: one division per wave, then an add and a carry per row. The next row's loads are issued
    // before this row's softmax, into the other of two register sets (a copy between them would be
    // a use that waits for the load).
    if (wave >= (long)BH * N) return;  // the whole wave leaves together
    RowAt<T> ra = locate<T>(wave / N, wave % N, N, dk, dv, P, prev_len, k, v, kp, vp), rb;
    typename Raw4<T>::type aq, ak, bq, bk;
    const bool want_q = qo != nullptr;
    load_row(ra, q, dk, lane, want_q, aq, ak);
    bool more;
    for (;;) {
        rb = advance(ra, BH, N, dk, dv, P, prev_len, step_bh, step_n, k, v, kp, vp, more);
        load_row(rb, q, dk, lane, want_q, bq, bk);
        finish_row(ra, aq, ak, dk, fmap, lane, tab, qo, ko, qlo, klo);
        if (!more) break;
        ra = advance(rb, BH, N, dk, dv, P, prev_len, step_bh, step_n, k, v, kp, vp, more);
        load_row(ra, q, dk, lane, want_q, aq, ak);
        finish_row(rb, bq, bk, dk, fmap, lane, tab, qo, ko, qlo, klo);
        if (!more) break;
    }
}

// out = a + b + c, four values per thread and step (b and c may be null; out may alias a).
template <typename TOUT>
__global__ __launch_bounds__(256) void add_rows_kernel(size_t n4, const float* a, const float* b, const float* c, TOUT* out) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        f32x4 x = reinterpret_cast<const f32x4*>(a)[i];
        if (b) x += reinterpret_cast<const f32x4*>(b)[i];
        if (c) x += reinterpret_cast<const f32x4*>(c)[i];
        if constexpr (sizeof(TOUT) == 4) {
            reinterpret_cast<f32x4*>(out)[i] = x;
        } else {
            reinterpret_cast<bf16x4*>(out)[i] = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
        }
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
    // 16 four-wave blocks per CU on 256 CUs: 8 of them fill the 8 wave slots of each SIMD and the
    // rest start as those finish, which evens out the tail (measured faster than 4 or 8 per CU);
    // larger inputs loop
    const long grid = std::min<long>((rows + 3) / 4, 256 * 16);
    const long step = 4 * grid;
    const int BH = (int)(rows / r.N), step_bh = (int)(step / r.N), step_n = (int)(step % r.N);
    if (r.bf16 && r.feat_f32)
        hipLaunchKernelGGL((rla_prepare_kernel<bf16, float>), dim3((unsigned)grid), dim3(256), 0, stream, BH, r.N, r.dk, r.dv, r.P,
                           r.prev_len, r.fmap, r.vsplit, step_bh, step_n,
                           static_cast<const bf16*>(r.q), static_cast<const bf16*>(r.k), static_cast<const bf16*>(r.v),
                           static_cast<const bf16*>(r.kp), static_cast<const bf16*>(r.vp), static_cast<float*>(r.qo),
                           static_cast<float*>(r.ko), static_cast<float*>(r.vo), nullptr, nullptr);
    else if (r.bf16)
        hipLaunchKernelGGL((rla_prepare_kernel<bf16, bf16>), dim3((unsigned)grid), dim3(256), 0, stream, BH, r.N, r.dk, r.dv, r.P,
                           r.prev_len, r.fmap, r.vsplit, step_bh, step_n,
                           static_cast<const bf16*>(r.q), static_cast<const bf16*>(r.k), static_cast<const bf16*>(r.v),
                           static_cast<const bf16*>(r.kp), static_cast<const bf16*>(r.vp), static_cast<bf16*>(r.qo),
                           static_cast<bf16*>(r.ko), static_cast<bf16*>(r.vo), static_cast<bf16*>(r.qlo),
                           static_cast<bf16*>(r.klo));
    else
        hipLaunchKernelGGL((rla_prepare_kernel<float, float>), dim3((unsigned)grid), dim3(256), 0, stream, BH, r.N, r.dk, r.dv, r.P,
                           r.prev_len, r.fmap, r.vsplit, step_bh, step_n,
                           static_cast<const float*>(r.q), static_cast<const float*>(r.k), static_cast<const float*>(r.v),
                           static_cast<const float*>(r.kp), static_cast<const float*>(r.vp), static_cast<float*>(r.qo),
                           static_cast<float*>(r.ko), static_cast<float*>(r.vo), nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_add_rows(size_t n, const float* a, const float* b, const float* c, void* out, bool out_bf16, hipStream_t stream) {
    const size_t n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 256 * 8);
    if (out_bf16)
        hipLaunchKernelGGL(add_rows_kernel<bf16>, dim3(grid), dim3(256), 0, stream, n4, a, b, c, static_cast<bf16*>(out));
    else
        hipLaunchKernelGGL(add_rows_kernel<float>, dim3(grid), dim3(256), 0, stream, n4, a, b, c, static_cast<float*>(out));
    return hipGetLastError();
}

hipError_t launch_copy_state(size_t n, const float* src, float* dst, hipStream_t stream) {
    const size_t n4 = n / 4;
    const size_t blocks = (n4 + 255) / 256;
    hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream, n4, src, dst);
    return hipGetLastError();
}

}  // namespace ret

// Backward of chunkwise retention (dq, dk, dv, dstate_in for dL/dout = dout) on the forward chunk
// kernels.
//
// Method (abeam.tech RetNet summary, "Training in parallel, generation by state update": the state
// recurrence S_n = g S_(n-1) + k_n^T v_n, o_n = q_n S_n; training is what the pages measure).
// Retention is linear in each of q, k and v, and its gradients are retentions themselves. With
// t -> N-1-t the time reversal of a [B][H][N][d] tensor:
//   dq_n = sum_{m<=n} g^(n-m) (dout_n . v_m) k_m + g^(n+1) dout_n S_in^T
//        = forward(q' = dout, k' = v, v' = k, state_in' = S_in^T)_n
//   dv_m = sum_{n>=m} g^(n-m) (q_n . k_m) dout_n      = rev(forward(rev k, rev q, rev dout))_m
//   dk_m = sum_{n>=m} g^(n-m) (dout_n . v_m) q_n      = rev(forward(rev v, rev dout, rev q))_m
//   dstate_in = g U_0, U_0 = sum_n g^n q_n^T dout_n   = g * state_out of the dv forward
// A forward whose contraction width (d_v here) has no kernel runs as s forwards over column
// blocks of width d_v / s, whose outputs add (the scores are sums over the contraction index).
// The gradients come out in fp32; the forwards accumulate in fp32 with the operand precision of
// the forward path (bf16 scores and bf16 hi + lo state and scaled values for bf16 inputs).
#include "common.hpp"

namespace ret {
namespace {

constexpr int kCopyThreads = 256;

// dst[bh][n][c] = src[bh][rev ? N-1-n : n][c0 + c], c < w (src rows of d elements), 16 bytes
// per thread. w * sizeof(T) and c0 * sizeof(T) are multiples of 16 (checked by the caller).
template <typename T>
__global__ __launch_bounds__(kCopyThreads) void gather_rows_kernel(long BH, int N, int d, int c0, int w, int rev,
                                                                   const T* __restrict__ src, T* __restrict__ dst) {
    constexpr int EV = 16 / (int)sizeof(T);
    const int vpr = w / EV;  // vectors per output row
    const size_t total = (size_t)BH * N * vpr;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads) {
        const size_t row = i / vpr;
        const int cv = (int)(i % vpr);
        const long bh = (long)(row / N);
        const int n = (int)(row % N);
        const int ns = rev ? N - 1 - n : n;
        const uint4 x = *reinterpret_cast<const uint4*>(src + ((size_t)bh * N + ns) * d + c0 + cv * EV);
        *reinterpret_cast<uint4*>(dst + row * w + cv * EV) = x;
    }
}

// dst[bh][rev ? N-1-n : n][c0 + c] = src[bh][n][c] (+ the old value when accumulating), fp32,
// 16 bytes per thread; the reverse of gather_rows_kernel.
__global__ __launch_bounds__(kCopyThreads) void scatter_rows_kernel(long BH, int N, int d, int c0, int w, int rev, int accumulate,
                                                                    const float* __restrict__ src, float* __restrict__ dst) {
    const int vpr = w / 4;
    const size_t total = (size_t)BH * N * vpr;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads) {
        const size_t row = i / vpr;
        const int cv = (int)(i % vpr);
        const long bh = (long)(row / N);
        const int n = (int)(row % N);
        const int nd = rev ? N - 1 - n : n;
        float4* o = reinterpret_cast<float4*>(dst + ((size_t)bh * N + nd) * d + c0 + 4 * cv);
        float4 x = *reinterpret_cast<const float4*>(src + row * w + 4 * cv);
        if (accumulate) {
            const float4 y = *o;
            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
        *o = x;
    }
}

// t[bh][r][c] = s[bh][c][r0 + r] for r < rw, c < dk: column block r0 .. r0 + rw of S^T, S [dk][dv]
__global__ __launch_bounds__(kCopyThreads) void transpose_state_kernel(long BH, int dk, int dv, int r0, int rw,
                                                                       const float* __restrict__ s, float* __restrict__ t) {
    const size_t total = (size_t)BH * rw * dk;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads) {
        const long bh = (long)(i / ((size_t)rw * dk));
        const int r = (int)((i / dk) % rw), c = (int)(i % dk);
        t[i] = s[((size_t)bh * dk + c) * dv + r0 + r];
    }
}

// x[bh][...] *= gamma_h for each of the per-head blocks of `per` elements
__global__ __launch_bounds__(kCopyThreads) void scale_heads_kernel(long BH, int H, size_t per, HeadConsts hc, float* __restrict__ x) {
    const size_t total = (size_t)BH * per;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads)
        x[i] *= hc.gamma[(i / per) % H];
}

unsigned grid_for(size_t work) {
    const size_t g = (work + kCopyThreads - 1) / kCopyThreads;
    return (unsigned)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

bool fwd_supported(int in_bf16, int dk, int dv, int chunk) {
    return in_bf16 ? chunkwise_bf16_supported(dk, dv, chunk) : chunkwise_f32_supported(dk, dv, chunk);
}

size_t fwd_workspace(int in_bf16, int B, int H, int N, int dk, int dv, int chunk) {
    return in_bf16 ? chunkwise_bf16_workspace(B, H, N, dk, dv, chunk, 0, 1) : chunkwise_f32_workspace(B, H, N, dv, 0, 0);
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace regions, each 256-aligned.
struct BwdLayout {
    int split;  // column blocks of d_v in the dq and dk forwards
    size_t fwd, rq, rk, rdo, dqo, dqv, rv, rdh, tmp, st, total;
};

BwdLayout bwd_layout(int in_bf16, int B, int H, int N, int DK, int DV, int chunk) {
    BwdLayout l{};
    l.split = bwd_split(in_bf16, DK, DV, chunk);
    const int w = l.split ? DV / l.split : DV;
    const size_t rows = (size_t)B * H * N, sz = in_bf16 ? 2 : 4;
    size_t fw = fwd_workspace(in_bf16, B, H, N, DK, DV, chunk);
    const size_t f2 = fwd_workspace(in_bf16, B, H, N, w, DK, chunk);
    if (f2 > fw) fw = f2;
    size_t o = 0;
    l.fwd = o; o += al(fw);
    l.rq = o; o += al(rows * DK * sz);                     // rev q
    l.rk = o; o += al(rows * DK * sz);                     // rev k
    l.rdo = o; o += al(rows * DV * sz);                    // rev dout
    l.dqo = o; o += al(l.split > 1 ? rows * w * sz : 0);   // a column block of dout
    l.dqv = o; o += al(l.split > 1 ? rows * w * sz : 0);   // ... of v
    l.rv = o; o += al(rows * w * sz);                      // a column block of rev v
    l.rdh = o; o += al(l.split > 1 ? rows * w * sz : 0);   // ... of rev dout
    l.tmp = o; o += al(rows * (size_t)(DK > DV ? DK : DV) * 4);
    l.st = o; o += al((size_t)B * H * w * DK * 4);         // a block of S_in^T
    l.total = o;
    return l;
}

template <typename T>
void gather(const LaunchArgs& a, const void* src, int d, int c0, int w, int rev, void* dst) {
    const size_t work = (size_t)a.B * a.H * a.N * w / (16 / sizeof(T));
    hipLaunchKernelGGL(gather_rows_kernel<T>, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d, c0,
                       w, rev, reinterpret_cast<const T*>(src), reinterpret_cast<T*>(dst));
}

void gather_any(const LaunchArgs& a, const void* src, int d, int c0, int w, int rev, void* dst) {
    if (a.in_bf16) gather<bf16>(a, src, d, c0, w, rev, dst);
    else gather<float>(a, src, d, c0, w, rev, dst);
}

void scatter(const LaunchArgs& a, const float* src, int d, int c0, int w, int rev, int acc, float* dst) {
    const size_t work = (size_t)a.B * a.H * a.N * w / 4;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d, c0, w,
                       rev, acc, src, dst);
}

// one forward on the given operands (d_k = dk, d_v = dv), fp32 out, no GroupNorm
hipError_t forward(const LaunchArgs& base, int dk, int dv, const void* q, const void* k, const void* v, const float* state_in,
                   float* out, float* state_out, void* ws, size_t ws_bytes) {
    LaunchArgs a = base;
    a.DK = dk;
    a.DV = dv;
    a.out_bf16 = 0;
    a.gn = GnArgs{};
    a.q = q; a.k = k; a.v = v;
    a.state_in = state_in;
    a.out = out;
    a.state_out = state_out;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    return a.in_bf16 ? launch_chunkwise_bf16(a) : launch_chunkwise_f32(a);
}

}  // namespace

int bwd_split(int in_bf16, int DK, int DV, int chunk) {
    if (!fwd_supported(in_bf16, DK, DV, chunk)) return 0;
    for (int s = 1; s <= 2; s *= 2)
        if (DV % s == 0 && fwd_supported(in_bf16, DV / s, DK, chunk) && ((DV / s) * (in_bf16 ? 2 : 4)) % 16 == 0) return s;
    return 0;
}

size_t chunkwise_bwd_workspace(int in_bf16, int B, int H, int N, int DK, int DV, int chunk) {
    return bwd_layout(in_bf16, B, H, N, DK, DV, chunk).total;
}

hipError_t launch_chunkwise_bwd(const BwdArgs& b) {
    const LaunchArgs& a = b.base;
    const BwdLayout l = bwd_layout(a.in_bf16, a.B, a.H, a.N, a.DK, a.DV, a.chunk);
    const int DK = a.DK, DV = a.DV, s = l.split, w = DV / s;
    char* ws = reinterpret_cast<char*>(a.ws);
    void* fws = ws + l.fwd;
    const size_t fwb = l.rq - l.fwd;
    float* tmp = reinterpret_cast<float*>(ws + l.tmp);
    hipError_t e;
    // reversed operands
    gather_any(a, b.q, DK, 0, DK, 1, ws + l.rq);
    gather_any(a, b.k, DK, 0, DK, 1, ws + l.rk);
    gather_any(a, b.dout, DV, 0, DV, 1, ws + l.rdo);

    // dq = sum over column blocks j of forward(dout_j, v_j, k, (S_in^T)_j)
    if (b.dq) {
        for (int j = 0; j < s; ++j) {
            const void* qo = b.dout;
            const void* kv = b.v;
            if (s > 1) {
                gather_any(a, b.dout, DV, j * w, w, 0, ws + l.dqo);
                gather_any(a, b.v, DV, j * w, w, 0, ws + l.dqv);
                qo = ws + l.dqo;
                kv = ws + l.dqv;
            }
            const float* st = nullptr;
            if (b.state_in) {
                const size_t work = (size_t)a.B * a.H * w * DK;
                hipLaunchKernelGGL(transpose_state_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, DK, DV,
                                   j * w, w, b.state_in, reinterpret_cast<float*>(ws + l.st));
                st = reinterpret_cast<const float*>(ws + l.st);
            }
            e = forward(a, w, DK, qo, kv, b.k, st, j == 0 ? b.dq : tmp, nullptr, fws, fwb);
            if (e != hipSuccess) return e;
            if (j > 0) scatter(a, tmp, DK, 0, DK, 0, 1, b.dq);
        }
    }
    // dv = rev(forward(rev k, rev q, rev dout)); its final state is U_0
    if (b.dv || b.dstate_in) {
        e = forward(a, DK, DV, ws + l.rk, ws + l.rq, ws + l.rdo, nullptr, b.dv ? tmp : nullptr, b.dstate_in, fws, fwb);
        if (e != hipSuccess) return e;
        if (b.dv) scatter(a, tmp, DV, 0, DV, 1, 0, b.dv);
        if (b.dstate_in) {
            const size_t per = (size_t)DK * DV;
            hipLaunchKernelGGL(scale_heads_kernel, dim3(grid_for((size_t)a.B * a.H * per)), dim3(kCopyThreads), 0, a.stream,
                               (long)a.B * a.H, a.H, per, a.hc, b.dstate_in);
        }
    }
    // dk = rev(sum over column blocks j of forward(rev v_j, rev dout_j, rev q))
    if (b.dk) {
        for (int j = 0; j < s; ++j) {
            gather_any(a, b.v, DV, j * w, w, 1, ws + l.rv);
            const void* rdo = ws + l.rdo;
            if (s > 1) {
                gather_any(a, b.dout, DV, j * w, w, 1, ws + l.rdh);
                rdo = ws + l.rdh;
            }
            e = forward(a, w, DK, ws + l.rv, rdo, ws + l.rq, nullptr, tmp, nullptr, fws, fwb);
            if (e != hipSuccess) return e;
            scatter(a, tmp, DK, 0, DK, 1, j > 0, b.dk);
        }
    }
    return hipGetLastError();
}

}  // namespace ret

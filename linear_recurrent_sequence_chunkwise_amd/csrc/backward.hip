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
// A forward whose contraction width (d_v here) has no kernel runs over s column blocks of width
// d_v / s, whose outputs add (the scores are sums over the contraction index). The blocks are
// stacked along the batch (B' = s B), so one launch covers them with s times the workgroups.
// bf16 inputs: the forwards read every operand in place (OpAddr: the time reversal, the row stride
// and column block of a 512-wide operand, the source head of a stacked block) and write every
// gradient in place; the s = 2 column blocks add their rows atomically into the zeroed gradient.
// fp32 inputs: the reversed and stacked operands are copied into the workspace first, and a last
// pass sums the s outputs.
// The gradients come out in fp32; the forwards accumulate in fp32 with the operand precision of
// the forward path (bf16 scores and bf16 hi + lo state and scaled values for bf16 inputs).
#include "common.hpp"

namespace ret {
namespace {

constexpr int kCopyThreads = 256;

// Up to six copies of the rows of one [BH][N][d] source, read once: output o receives the column
// block c0 .. c0 + w of every row, time-reversed or not, `copies` times (copies after the first at
// copy_stride elements), as dst[copy][bh][n][c]. 16 bytes per thread; c0, w and d hold whole
// 16-byte units (checked by the caller).
struct RowCopy {
    void* dst;
    int c0, w, rev, copies;
    size_t copy_stride;
};
struct RowCopies {
    RowCopy o[6];
    int n;
};

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void copy_rows_kernel(long BH, int N, int d, const T* __restrict__ src, RowCopies cp) {
    constexpr int EV = 16 / (int)sizeof(T);
    const int vpr = d / EV;
    const size_t total = (size_t)BH * N * vpr;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads) {
        const size_t row = i / vpr;
        const int c = (int)(i % vpr) * EV;
        const long bh = (long)(row / N);
        const int n = (int)(row % N);
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + row * d + c));
        for (int k = 0; k < cp.n; ++k) {
            const RowCopy& o = cp.o[k];
            if (c < o.c0 || c >= o.c0 + o.w) continue;
            const size_t at = ((size_t)bh * N + (o.rev ? N - 1 - n : n)) * o.w + (c - o.c0);
            for (int j = 0; j < o.copies; ++j) *reinterpret_cast<u32x4*>(reinterpret_cast<T*>(o.dst) + j * o.copy_stride + at) = x;
        }
    }
}

// dst[bh][rev ? N-1-n : n][c0 + c] = src[bh][n][c] (+ the old value when accumulating), fp32,
// 16 bytes per thread.
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

// dst[bh][rev ? N-1-n : n][c] = sum over j < s of src[j][bh][n][c] (fp32, rows of d, 16 bytes per
// thread), the s column-block outputs of a stacked forward added in block order
__global__ __launch_bounds__(kCopyThreads) void sum_blocks_kernel(long BH, int N, int d, int s, int rev, const float* __restrict__ src,
                                                                  float* __restrict__ dst) {
    const int vpr = d / 4;
    const size_t rows = (size_t)BH * N, total = rows * vpr;
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kCopyThreads) {
        const size_t row = i / vpr;
        const int cv = (int)(i % vpr);
        const long bh = (long)(row / N);
        const int n = (int)(row % N);
        float4 x = *reinterpret_cast<const float4*>(src + row * d + 4 * cv);
        for (int j = 1; j < s; ++j) {
            const float4 y = *reinterpret_cast<const float4*>(src + ((size_t)j * rows + row) * d + 4 * cv);
            x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
        *reinterpret_cast<float4*>(dst + ((size_t)bh * N + (rev ? N - 1 - n : n)) * d + 4 * cv) = x;
    }
}

// x[0 .. n4*4) = 0, 16 bytes per thread (a kernel, so that a captured call records no memset node)
__global__ __launch_bounds__(kCopyThreads) void zero_kernel(size_t n4, float* __restrict__ x) {
    for (size_t i = blockIdx.x * (size_t)kCopyThreads + threadIdx.x; i < n4; i += (size_t)gridDim.x * kCopyThreads)
        reinterpret_cast<float4*>(x)[i] = float4{0.f, 0.f, 0.f, 0.f};
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

// Workspace regions, each 256-aligned. With s column blocks, "stacked" buffers hold s copies one
// after another (the batch of the stacked forward). bf16 inputs need only fwd and st.
struct BwdLayout {
    int split;  // column blocks of d_v in the dq and dk forwards
    size_t fwd, rq, rk, rdo, sa, sb, sc, ta, tb, tc, tmp, st, pa, total;
    bool share;  // the dk forward takes the dq forward's scores, anti-transposed (at pa)
};

BwdLayout bwd_layout(int in_bf16, int B, int H, int N, int DK, int DV, int chunk) {
    BwdLayout l{};
    l.split = bwd_split(in_bf16, DK, DV, chunk);
    const int s = l.split ? l.split : 1, w = DV / s;
    const size_t rows = (size_t)B * H * N, sz = in_bf16 ? 2 : 4;
    size_t fw = fwd_workspace(in_bf16, B, H, N, DK, DV, chunk);
    const size_t f2 = fwd_workspace(in_bf16, s * B, H, N, w, DK, chunk);
    if (f2 > fw) fw = f2;
    size_t o = 0;
    l.fwd = o; o += al(fw);
    if (in_bf16) {                                      // operands read in place, column blocks added in place
        l.rq = l.rk = l.rdo = l.sa = l.sb = l.sc = l.ta = l.tb = l.tc = l.tmp = o;
        l.st = o; o += al((size_t)s * B * H * w * DK * 4);
        l.share = chunk > 0 && N % chunk == 0 && chunkwise_bf16_supported(w, DK, chunk) && chunkwise_bf16_scores_split(w, chunk);
        l.pa = o; o += l.share ? al(chunkwise_bf16_scores_bytes(s * B, H, N, w, chunk)) : 0;
        l.total = o;
        return l;
    }
    l.rq = o; o += al(rows * DK * sz);                  // rev q
    l.rk = o; o += al(rows * DK * sz);                  // rev k
    l.rdo = o; o += al(rows * DV * sz);                 // rev dout
    l.sa = o; o += al(s > 1 ? s * rows * w * sz : 0);   // dq forward: stacked column blocks of dout
    l.sb = o; o += al(s > 1 ? s * rows * w * sz : 0);   // ... of v
    l.sc = o; o += al(s > 1 ? s * rows * DK * sz : 0);  // ... k once per block
    l.ta = o; o += al(s * rows * w * sz);               // dk forward: stacked reversed blocks of v
    l.tb = o; o += al(s > 1 ? s * rows * w * sz : 0);   // ... of dout
    l.tc = o; o += al(s > 1 ? s * rows * DK * sz : 0);  // ... rev q once per block
    const size_t t1 = rows * (size_t)DV * 4, t2 = s * rows * (size_t)DK * 4;
    l.tmp = o; o += al(t1 > t2 ? t1 : t2);              // fp32 forward output
    l.st = o; o += al((size_t)s * B * H * w * DK * 4);  // stacked blocks of S_in^T
    l.total = o;
    return l;
}

void copy_rows(const LaunchArgs& a, const void* src, int d, const RowCopies& cp) {
    const size_t work = (size_t)a.B * a.H * a.N * d * (a.in_bf16 ? 2 : 4) / 16;
    if (a.in_bf16)
        hipLaunchKernelGGL(copy_rows_kernel<bf16>, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d,
                           reinterpret_cast<const bf16*>(src), cp);
    else
        hipLaunchKernelGGL(copy_rows_kernel<float>, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d,
                           reinterpret_cast<const float*>(src), cp);
}

void scatter(const LaunchArgs& a, const float* src, int d, int c0, int w, int rev, int acc, float* dst) {
    const size_t work = (size_t)a.B * a.H * a.N * w / 4;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d, c0, w,
                       rev, acc, src, dst);
}

// one forward on the given operands (d_k = dk, d_v = dv), fp32 out, no GroupNorm
hipError_t forward(const LaunchArgs& base, int dk, int dv, const void* q, const void* k, const void* v, const float* state_in,
                   float* out, float* state_out, void* ws, size_t ws_bytes, OpAddr addr = OpAddr{}) {
    LaunchArgs a = base;
    a.addr = addr;
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

// bf16: every forward reads its operands in place. With two column blocks the stacked forward adds
// both blocks' rows into the gradient (zeroed first): a + b in either order is the same fp32 value.
hipError_t bwd_in_place(const BwdArgs& b) {
    const LaunchArgs& a = b.base;
    const BwdLayout l = bwd_layout(1, a.B, a.H, a.N, a.DK, a.DV, a.chunk);
    const int DK = a.DK, DV = a.DV, s = l.split, w = DV / s, BH = a.B * a.H;
    const size_t rows = (size_t)BH * a.N;
    char* ws = reinterpret_cast<char*>(a.ws);
    void* fws = ws + l.fwd;
    const size_t fwb = l.st - l.fwd;
    LaunchArgs stacked = a;  // the column blocks stacked along the batch
    stacked.B = s * a.B;
    const int acc = s > 1;
    auto zero = [&](float* dst) {
        const size_t n4 = rows * DK / 4;
        hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n4)), dim3(kCopyThreads), 0, a.stream, n4, dst);
    };
    hipError_t e;
    // dq = sum over column blocks j of forward(dout_j, v_j, k, (S_in^T)_j): dout and v rows DV apart,
    // block j from column j w; k shared by the blocks
    if (b.dq) {
        const float* st = nullptr;
        if (b.state_in) {
            for (int j = 0; j < s; ++j) {
                const size_t work = (size_t)BH * w * DK;
                hipLaunchKernelGGL(transpose_state_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)BH, DK, DV, j * w,
                                   w, b.state_in, reinterpret_cast<float*>(ws + l.st) + (size_t)j * BH * w * DK);
            }
            st = reinterpret_cast<const float*>(ws + l.st);
        }
        if (acc) zero(b.dq);
        LaunchArgs sq = stacked;
        if (l.share && b.dk) sq.p_anti = ws + l.pa;  // the dk forward's scores, written on the way
        e = forward(sq, w, DK, b.dout, b.v, b.k, st, b.dq, nullptr, fws, fwb, OpAddr{0, DV, w, BH, acc});
        if (e != hipSuccess) return e;
    }
    // dv = rev(forward(rev k, rev q, rev dout)), written in place; its final state is U_0
    if (b.dv || b.dstate_in) {
        e = forward(a, DK, DV, b.k, b.q, b.dout, nullptr, b.dv, b.dstate_in, fws, fwb, OpAddr{1, DK, 0, BH, 0});
        if (e != hipSuccess) return e;
        if (b.dstate_in) {
            const size_t per = (size_t)DK * DV;
            hipLaunchKernelGGL(scale_heads_kernel, dim3(grid_for((size_t)BH * per)), dim3(kCopyThreads), 0, a.stream, (long)BH, a.H, per,
                               a.hc, b.dstate_in);
        }
    }
    // dk = rev(sum over column blocks j of forward(rev v_j, rev dout_j, rev q)); the reversed
    // forward writes its rows back in time order
    if (b.dk) {
        if (acc) zero(b.dk);
        LaunchArgs sk = stacked;
        if (l.share && b.dq) sk.p_given = ws + l.pa;
        e = forward(sk, w, DK, b.v, b.dout, b.q, nullptr, b.dk, nullptr, fws, fwb, OpAddr{1, DV, w, BH, acc});
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

hipError_t launch_chunkwise_bwd(const BwdArgs& b) {
    if (b.base.in_bf16) return bwd_in_place(b);
    const LaunchArgs& a = b.base;
    const BwdLayout l = bwd_layout(a.in_bf16, a.B, a.H, a.N, a.DK, a.DV, a.chunk);
    const int DK = a.DK, DV = a.DV, s = l.split, w = DV / s;
    const size_t rows = (size_t)a.B * a.H * a.N, sz = a.in_bf16 ? 2 : 4;
    char* ws = reinterpret_cast<char*>(a.ws);
    void* fws = ws + l.fwd;
    const size_t fwb = l.rq - l.fwd;
    float* tmp = reinterpret_cast<float*>(ws + l.tmp);
    LaunchArgs stacked = a;  // the column blocks stacked along the batch
    stacked.B = s * a.B;
    auto blk = [&](size_t off, int j, size_t width) { return ws + off + (size_t)j * rows * width * sz; };
    auto sum_blocks = [&](int d, int rev, float* dst) {
        const size_t work = rows * d / 4;
        hipLaunchKernelGGL(sum_blocks_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, a.N, d, s, rev, tmp,
                           dst);
    };
    hipError_t e;
    // The operands of every forward, each source read once: reversed q, k and dout (dv forward);
    // with s > 1 the column blocks of dout and v and s copies of k, stacked (dq forward); reversed
    // column blocks of v (and with s > 1 of dout) and s copies of rev q, stacked (dk forward).
    auto rc = [](void* dst, int c0, int w_, int rev, int copies, size_t stride) { return RowCopy{dst, c0, w_, rev, copies, stride}; };
    const size_t kst = rows * DK;  // element stride of stacked copies
    const bool sq = s > 1 && b.dq, sk = s > 1 && b.dk;
    {
        RowCopies cq{}, ck{}, cd{}, cv{};
        cq.o[cq.n++] = rc(ws + l.rq, 0, DK, 1, 1, 0);
        if (sk) cq.o[cq.n++] = rc(ws + l.tc, 0, DK, 1, s, kst);
        ck.o[ck.n++] = rc(ws + l.rk, 0, DK, 1, 1, 0);
        if (sq) ck.o[ck.n++] = rc(ws + l.sc, 0, DK, 0, s, kst);
        cd.o[cd.n++] = rc(ws + l.rdo, 0, DV, 1, 1, 0);
        for (int j = 0; j < s; ++j) {
            if (sq) cd.o[cd.n++] = rc(blk(l.sa, j, w), j * w, w, 0, 1, 0);
            if (sk) cd.o[cd.n++] = rc(blk(l.tb, j, w), j * w, w, 1, 1, 0);
            if (sq) cv.o[cv.n++] = rc(blk(l.sb, j, w), j * w, w, 0, 1, 0);
            if (b.dk) cv.o[cv.n++] = rc(blk(l.ta, j, w), j * w, w, 1, 1, 0);
        }
        copy_rows(a, b.q, DK, cq);
        copy_rows(a, b.k, DK, ck);
        copy_rows(a, b.dout, DV, cd);
        if (cv.n) copy_rows(a, b.v, DV, cv);
    }

    // dq = sum over column blocks j of forward(dout_j, v_j, k, (S_in^T)_j)
    if (b.dq) {
        const void *qo = b.dout, *kv = b.v, *vk = b.k;
        if (s > 1) {
            qo = ws + l.sa;
            kv = ws + l.sb;
            vk = ws + l.sc;
        }
        const float* st = nullptr;
        if (b.state_in) {
            for (int j = 0; j < s; ++j) {
                const size_t work = (size_t)a.B * a.H * w * DK;
                hipLaunchKernelGGL(transpose_state_kernel, dim3(grid_for(work)), dim3(kCopyThreads), 0, a.stream, (long)a.B * a.H, DK, DV,
                                   j * w, w, b.state_in, reinterpret_cast<float*>(ws + l.st) + (size_t)j * a.B * a.H * w * DK);
            }
            st = reinterpret_cast<const float*>(ws + l.st);
        }
        e = forward(stacked, w, DK, qo, kv, vk, st, s > 1 ? tmp : b.dq, nullptr, fws, fwb);
        if (e != hipSuccess) return e;
        if (s > 1) sum_blocks(DK, 0, b.dq);
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
        const void *qv = ws + l.ta, *kd = ws + l.rdo, *vq = ws + l.rq;
        if (s > 1) {
            kd = ws + l.tb;
            vq = ws + l.tc;
        }
        e = forward(stacked, w, DK, qv, kd, vq, nullptr, tmp, nullptr, fws, fwb);
        if (e != hipSuccess) return e;
        sum_blocks(DK, 1, b.dk);
    }
    return hipGetLastError();
}

}  // namespace ret

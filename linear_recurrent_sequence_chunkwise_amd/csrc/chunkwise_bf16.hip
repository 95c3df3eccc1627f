// Chunkwise recurrent retention, bf16 inputs, fp32 accumulation, on the gfx950 matrix cores.
//
// Method (abeam.tech RetNet summary, "Chunk recursion for long-sequence training"; mlnews.online
// RetNet abstract: chunks encoded in parallel, summarised recurrently). Unrolling the recurrence
// S_n = g S_(n-1) + k_n^T v_n over one chunk of length L with carried state R gives, for local row j,
//     o_j = [(Q K^T (.) D) V]_j + g^(j+1) [Q R]_j,      D[j][t] = g^(j-t) for t <= j
//     R  <- g^L R + K^T (V (.) zeta),                    zeta_t = g^(L-1-t)
//
// Two kernels:
//   chunk_scores_kernel   fully parallel over (row band, chunk, b*h): P = (Q K^T) (.) D on MFMA,
//                         decay and causal mask applied in registers, stored as bf16 in the
//                         workspace (32x32 blocks on and below the diagonal).
//   chunk_main_kernel     one workgroup per (b, h, 32-column slice of d_v), looping over the chunks
//                         in order. It keeps its d_k x 32 slice of R in fp32 accumulators, and per
//                         chunk computes the inter-chunk term Q R (R as bf16 hi + lo, both MFMA),
//                         scales it by g^(j+1), adds P V (V from LDS through transposing reads),
//                         applies the optional per-head GroupNorm through a fixed-order exchange of
//                         per-slice row statistics with the other slices of the same head, stores
//                         the output, and advances R with K^T (V (.) zeta) (V (.) zeta as bf16
//                         hi + lo). Every slice of a head needs all of Q and K, so the slices of one
//                         head are placed on one XCD to share its L2.
#include "common.hpp"


namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kW = 32;     // d_v columns per workgroup
constexpr int kTK = 64;    // K rows staged per state-update sub-block
constexpr int kRing = 4;   // GroupNorm statistics ring depth (>= 3 needed, see publish/finalize)
constexpr unsigned kSpinLimit = 1u << 24;

// ---------------------------------------------------------------------------------------------
// P = (Q K^T) (.) D for one chunk. Grid (C/64 bands, nchunks, B*H); wave w computes row tile
// t = 4*band + w (16 rows) against key tiles 0 .. (t|1): the second key tile of a diagonal 32x32
// block is all zero for even t but is written so that the consumer can read whole 32-key steps.
template <int DK>
__global__ __launch_bounds__(kThreads) void chunk_scores_kernel(int H, int N, int C, int nchunks,
                                                                const bf16* __restrict__ q,
                                                                const bf16* __restrict__ k,
                                                                bf16* __restrict__ P, HeadConsts hc) {
    const int band = blockIdx.x, chunk = blockIdx.y, bh = blockIdx.z, h = bh % H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = 4 * band + w;
    const int c0 = chunk * C;
    const int L = min(C, N - c0);
    const bf16* qb = q + ((size_t)bh * N + c0) * DK;
    const bf16* kb = k + ((size_t)bh * N + c0) * DK;
    bf16* Pc = P + ((size_t)bh * nchunks + chunk) * (size_t)C * C;
    const float l2g = hc.log2g[h];

    const int qrow = 16 * t + (lane & 15);
    bf16x8 qa[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
        qa[ks] = qrow < L ? frag_rowmajor(qb, DK, 16 * t, 32 * ks, lane) : zero_bf16x8();

    const int nkt = (t | 1) + 1;
    for (int kt = 0; kt < nkt; ++kt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        const int krow = 16 * kt + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const bf16x8 kf = krow < L ? frag_rowmajor(kb, DK, 16 * kt, 32 * ks, lane) : zero_bf16x8();
            s = mfma16(qa[ks], kf, s);
        }
        const int key = 16 * kt + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * t + 4 * (lane >> 4) + i;
            const float d = row >= key ? decay_pow(l2g, (float)(row - key)) : 0.f;
            Pc[(size_t)row * C + key] = (bf16)(s[i] * d);
        }
    }
}

// ---------------------------------------------------------------------------------------------
struct MainParams {
    int H, N, C, NS, nchunks, nteams_launch, team_base;
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const bf16* P;
    const float* state_in;
    float* state_out;
    void* out;
    float2* stats;       // [teams][kRing][NS][64]
    unsigned* counters;  // [teams]
    unsigned* err_flag;
    GnArgs gn;
};

template <int DK>
struct MainLds {
    static constexpr int LDK = DK + 16;  // K rows: transposing reads of 4 rows hit distinct banks
    static constexpr int LR = DK + 8;    // R^T rows: 16-byte reads of 16 rows hit distinct banks
    static constexpr int LV = kW + 16;   // V rows
    bf16 Ks[kTK * LDK];
    bf16 Rhi[kW * LR];
    bf16 Rlo[kW * LR];
    float zeta[512];
};

// One (b, h, d_v slice) per workgroup. Wave w owns R rows [w*DK/4, (w+1)*DK/4) (state update) and,
// for each 64-row group of a chunk, output row tile 4*rg + w (16 rows x 32 columns).
template <int DK, typename TOUT, bool GN, bool WANT_OUT>
__global__ __launch_bounds__(kThreads) void chunk_main_kernel(MainParams p, HeadConsts hc) {
    using Lds = MainLds<DK>;
    constexpr int LDK = Lds::LDK, LR = Lds::LR, LV = Lds::LV;
    constexpr int RTR = DK / 64;  // 16-row R tiles per wave
    __shared__ Lds sm;
    extern __shared__ bf16 Vs[];  // [C][LV]

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    // XCD-aware placement: workgroup i runs on XCD i % 8. With a multiple of 8 teams per launch,
    // all slices of a team share i % 8, so they share one L2 for that head's Q, K and P.
    int team_local, slice;
    if (p.nteams_launch % 8 == 0) {
        const int i = blockIdx.x;
        team_local = (i % 8) + 8 * (i / (8 * p.NS));
        slice = (i / 8) % p.NS;
    } else {
        team_local = blockIdx.x / p.NS;
        slice = blockIdx.x % p.NS;
    }
    const int bh = p.team_base + team_local;
    const int h = bh % p.H;
    const int N = p.N, C = p.C, DV = p.NS * kW;
    const float l2g = hc.log2g[h];
    const int col0 = slice * kW;

    // ---- initial state
    f32x4 accR[RTR][2];
#pragma unroll
    for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = w * (DK / 4) + 16 * rt + 4 * g4 + i;
                const int col = col0 + 16 * ct + c16;
                accR[rt][ct][i] = p.state_in ? p.state_in[((size_t)bh * DK + row) * DV + col] : 0.f;
            }

    auto write_R = [&]() {
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bf16x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16 a, b;
                    split_hi_lo(accR[rt][ct][i], a, b);
                    hi[i] = a;
                    lo[i] = b;
                }
                const int col = 16 * ct + c16;
                const int row = w * (DK / 4) + 16 * rt + 4 * g4;
                *reinterpret_cast<bf16x4*>(&sm.Rhi[col * LR + row]) = hi;
                *reinterpret_cast<bf16x4*>(&sm.Rlo[col * LR + row]) = lo;
            }
    };
    write_R();

    // ---- GroupNorm exchange state
    const int team = bh;
    float2* st_team = p.stats + (size_t)team * kRing * p.NS * 64;
    int gidx = 0;
    bool pend = false;
    int pend_g = 0, pend_c0 = 0, pend_L = 0, pend_tile = 0;
    f32x4 pend_acc[2];
    pend_acc[0] = pend_acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

    TOUT* out = reinterpret_cast<TOUT*>(p.out);

    auto store_tile = [&](int c0, int L, int tile, const f32x4* a) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * tile + 4 * g4 + i;
                if (r < L) out[((size_t)bh * N + c0 + r) * DV + col0 + 16 * ct + c16] = from_float<TOUT>(a[ct][i]);
            }
    };

    auto publish = [&](int g, const f32x4* a) {
        float2* dst = st_team + (size_t)(g % kRing) * p.NS * 64 + (size_t)slice * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = sum16(a[0][i] + a[1][i]);
            const float mean = s * (1.0f / kW);
            const float d0 = a[0][i] - mean, d1 = a[1][i] - mean;
            const float m2 = sum16(d0 * d0 + d1 * d1);
            if (c16 == 0) dst[16 * w + 4 * g4 + i] = make_float2(mean, m2);
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_fetch_add(p.counters + team, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    };

    auto finalize = [&](int g, int c0, int L, int tile, f32x4* a) {
        if (threadIdx.x == 0) {
            const unsigned target = (unsigned)p.NS * (unsigned)(g + 1);
            unsigned spins = 0;
            while (__hip_atomic_load(p.counters + team, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinLimit) {
                    atomicOr(p.err_flag, 1u);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const float2* src = st_team + (size_t)(g % kRing) * p.NS * 64;
        const int myslice = c16 % p.NS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = 16 * w + 4 * g4 + i;
            const float2 sv = src[(size_t)myslice * 64 + rr];
            float mean = sv.x, m2 = sv.y;
            float n = (float)kW;
            for (int off = 1; off < p.NS; off <<= 1) {
                const float om = __shfl_xor(mean, off, 64);
                const float o2 = __shfl_xor(m2, off, 64);
                const float d = om - mean;
                m2 = (m2 + o2) + d * d * (n * 0.5f);
                mean = (mean + om) * 0.5f;
                n *= 2.f;
            }
            const float var = m2 / (float)DV;
            const float inv = rsqrtf(var + p.gn.eps);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int c = col0 + 16 * ct + c16;
                const float wv = p.gn.weight ? p.gn.weight[(size_t)h * DV + c] : 1.f;
                const float bv = p.gn.bias ? p.gn.bias[(size_t)h * DV + c] : 0.f;
                a[ct][i] = (a[ct][i] - mean) * inv * wv + bv;
            }
        }
        store_tile(c0, L, tile, a);
    };

    __syncthreads();

    for (int chunk = 0; chunk < p.nchunks; ++chunk) {
        const int c0 = chunk * C;
        const int L = min(C, N - c0);
        const int Lpad = (L + 63) & ~63;

        // ---- stage V[c0 .. c0+Lpad) x slice columns, and zeta
        for (int idx = threadIdx.x; idx < Lpad * (kW / 8); idx += kThreads) {
            const int r = idx / (kW / 8), sg = idx % (kW / 8);
            bf16x8 val = zero_bf16x8();
            if (r < L) val = *reinterpret_cast<const bf16x8*>(p.v + ((size_t)bh * N + c0 + r) * DV + col0 + 8 * sg);
            *reinterpret_cast<bf16x8*>(&Vs[r * LV + 8 * sg]) = val;
        }
        for (int j = threadIdx.x; j < Lpad; j += kThreads)
            sm.zeta[j] = j < L ? decay_pow(l2g, (float)(L - 1 - j)) : 0.f;
        __syncthreads();

        if constexpr (WANT_OUT) {
            const bf16* Pc = p.P + ((size_t)bh * p.nchunks + chunk) * (size_t)C * C;
            const bf16* qc = p.q + ((size_t)bh * N + c0) * DK;
            for (int rg = 0; rg < Lpad / 64; ++rg) {
                const int tile = 4 * rg + w;
                f32x4 acc[2];
                acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
                // inter-chunk: Q R with R = hi + lo
                const bool qok = 16 * tile + c16 < L;
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const bf16x8 a = qok ? frag_rowmajor(qc, DK, 16 * tile, 32 * ks, lane) : zero_bf16x8();
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const bf16x8 bhi = *reinterpret_cast<const bf16x8*>(&sm.Rhi[(16 * ct + c16) * LR + 32 * ks + 8 * g4]);
                        const bf16x8 blo = *reinterpret_cast<const bf16x8*>(&sm.Rlo[(16 * ct + c16) * LR + 32 * ks + 8 * g4]);
                        acc[ct] = mfma16(a, bhi, acc[ct]);
                        acc[ct] = mfma16(a, blo, acc[ct]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xi = decay_pow(l2g, (float)(16 * tile + 4 * g4 + i + 1));
                    acc[0][i] *= xi;
                    acc[1][i] *= xi;
                }
                // intra-chunk: P V over key steps of 32 up to the diagonal block
                const int nks = (16 * tile + 15) / 32 + 1;
                for (int ks = 0; ks < nks; ++ks) {
                    const bf16x8 a = frag_rowmajor(Pc, C, 16 * tile, 32 * ks, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        const bf16x8 b = lds_frag_kmajor(Vs, LV, 32 * ks, 16 * ct, lane);
                        acc[ct] = mfma16(a, b, acc[ct]);
                    }
                }
                if constexpr (GN) {
                    publish(gidx, acc);
                    if (pend) finalize(pend_g, pend_c0, pend_L, pend_tile, pend_acc);
                    pend = true;
                    pend_g = gidx;
                    pend_c0 = c0;
                    pend_L = L;
                    pend_tile = tile;
                    pend_acc[0] = acc[0];
                    pend_acc[1] = acc[1];
                    ++gidx;
                } else {
                    store_tile(c0, L, tile, acc);
                }
            }
        }

        // ---- state update: R <- g^L R + K^T (V (.) zeta)
        const float gL = decay_pow(l2g, (float)L);
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) accR[rt][ct] *= gL;
        for (int sb = 0; sb < Lpad / kTK; ++sb) {
            __syncthreads();  // Ks free
            for (int idx = threadIdx.x; idx < kTK * (DK / 8); idx += kThreads) {
                const int r = idx / (DK / 8), sg = idx % (DK / 8);
                const int tok = sb * kTK + r;
                bf16x8 val = zero_bf16x8();
                if (tok < L) val = *reinterpret_cast<const bf16x8*>(p.k + ((size_t)bh * N + c0 + tok) * DK + 8 * sg);
                *reinterpret_cast<bf16x8*>(&sm.Ks[r * LDK + 8 * sg]) = val;
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < kTK / 32; ++ks) {
                const int tok0 = sb * kTK + 32 * ks;
                float z[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = sm.zeta[tok0 + 8 * g4 + j];
                bf16x8 bhi[2], blo[2];
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const bf16x8 vb = lds_frag_kmajor(Vs, LV, tok0, 16 * ct, lane);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        bf16 hi, lo;
                        split_hi_lo((float)vb[j] * z[j], hi, lo);
                        bhi[ct][j] = hi;
                        blo[ct][j] = lo;
                    }
                }
#pragma unroll
                for (int rt = 0; rt < RTR; ++rt) {
                    const bf16x8 ak = lds_frag_kmajor(sm.Ks, LDK, 32 * ks, w * (DK / 4) + 16 * rt, lane);
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        accR[rt][ct] = mfma16(ak, bhi[ct], accR[rt][ct]);
                        accR[rt][ct] = mfma16(ak, blo[ct], accR[rt][ct]);
                    }
                }
            }
        }
        __syncthreads();  // every wave is done reading R (phase A) and Vs
        write_R();
        __syncthreads();
    }
    if constexpr (GN) {
        if (pend) finalize(pend_g, pend_c0, pend_L, pend_tile, pend_acc);
    }
    if (p.state_out) {
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = w * (DK / 4) + 16 * rt + 4 * g4 + i;
                    const int col = col0 + 16 * ct + c16;
                    p.state_out[((size_t)bh * DK + row) * DV + col] = accR[rt][ct][i];
                }
    }
}

__global__ void zero_words_kernel(unsigned* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Workspace layout (bytes, each part 256-aligned):
//   P         B*H*nchunks*C*C bf16     (only when the output is wanted)
//   counters  B*H uint32 + 1 error flag
//   stats     B*H*kRing*NS*64 float2   (only with GroupNorm)
struct WsLayout {
    size_t p_off, p_bytes, cnt_off, cnt_bytes, st_off, st_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int B, int H, int N, int DV, int C, int gn, int want_out) {
    WsLayout l{};
    const size_t nchunks = (size_t)(N + C - 1) / C;
    l.p_off = 0;
    l.p_bytes = want_out ? align256((size_t)B * H * nchunks * C * C * sizeof(bf16)) : 0;
    l.cnt_off = l.p_off + l.p_bytes;
    l.cnt_bytes = gn ? align256(((size_t)B * H + 1) * sizeof(unsigned)) : 0;
    l.st_off = l.cnt_off + l.cnt_bytes;
    l.st_bytes = gn ? align256((size_t)B * H * kRing * (DV / kW) * 64 * sizeof(float2)) : 0;
    l.total = l.st_off + l.st_bytes;
    return l;
}

template <int DK, typename TOUT, bool GN, bool WANT_OUT>
hipError_t launch_main(const LaunchArgs& a, MainParams mp) {
    const void* kern = reinterpret_cast<const void*>(chunk_main_kernel<DK, TOUT, GN, WANT_OUT>);
    const size_t dyn = (size_t)a.chunk * MainLds<DK>::LV * sizeof(bf16);
    const int teams = a.B * a.H;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    if (!GN) {
        mp.team_base = 0;
        mp.nteams_launch = teams;
        hipLaunchKernelGGL((chunk_main_kernel<DK, TOUT, GN, WANT_OUT>), dim3(teams * mp.NS), dim3(kThreads), dyn, a.stream, mp, a.hc);
        return hipGetLastError();
    }
    // GroupNorm: the slices of a head exchange statistics, so they must be co-resident. Launch
    // cooperatively, in batches of whole teams that fit on the device at once.
    int dev = 0, ncu = 0, per_cu = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, dyn);
    if (e != hipSuccess) return e;
    const int fit_blocks = ncu * per_cu;
    int teams_per_launch = fit_blocks / mp.NS;
    if (teams_per_launch < 1) return hipErrorCooperativeLaunchTooLarge;
    if (teams_per_launch >= 8) teams_per_launch &= ~7;
    for (int base = 0; base < teams; base += teams_per_launch) {
        MainParams lp = mp;
        lp.team_base = base;
        lp.nteams_launch = teams - base < teams_per_launch ? teams - base : teams_per_launch;
        HeadConsts hc = a.hc;
        void* args[] = {&lp, &hc};
        e = hipLaunchCooperativeKernel(kern, dim3(lp.nteams_launch * mp.NS), dim3(kThreads),
                                       args, (unsigned)dyn, a.stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, typename TOUT>
hipError_t launch_dk(const LaunchArgs& a) {
    const int C = a.chunk;
    const int nchunks = (a.N + C - 1) / C;
    const bool want_out = a.out != nullptr;
    const WsLayout l = ws_layout(a.B, a.H, a.N, a.DV, C, a.gn.enabled, want_out);
    char* ws = reinterpret_cast<char*>(a.ws);
    MainParams mp{};
    mp.H = a.H; mp.N = a.N; mp.C = C; mp.NS = a.DV / kW; mp.nchunks = nchunks;
    mp.q = (const bf16*)a.q; mp.k = (const bf16*)a.k; mp.v = (const bf16*)a.v;
    mp.P = want_out ? reinterpret_cast<const bf16*>(ws + l.p_off) : nullptr;
    mp.state_in = a.state_in; mp.state_out = a.state_out; mp.out = a.out;
    mp.gn = a.gn;
    if (a.gn.enabled && want_out) {
        mp.counters = reinterpret_cast<unsigned*>(ws + l.cnt_off);
        mp.err_flag = mp.counters + (size_t)a.B * a.H;
        mp.stats = reinterpret_cast<float2*>(ws + l.st_off);
        const size_t nwords = (size_t)a.B * a.H + 1;
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((nwords + 255) / 256)), dim3(256), 0, a.stream, mp.counters, nwords);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (want_out) {
        hipLaunchKernelGGL(chunk_scores_kernel<DK>, dim3(C / 64, nchunks, a.B * a.H), dim3(kThreads), 0, a.stream, a.H, a.N,
                           C, nchunks, mp.q, mp.k, const_cast<bf16*>(mp.P), a.hc);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.gn.enabled) return launch_main<DK, TOUT, true, true>(a, mp);
        return launch_main<DK, TOUT, false, true>(a, mp);
    }
    return launch_main<DK, TOUT, false, false>(a, mp);
}

}  // namespace

bool chunkwise_bf16_supported(int DK, int DV, int chunk) {
    const bool dk_ok = DK == 64 || DK == 256;
    const bool dv_ok = DV % kW == 0 && DV / kW >= 1 && DV / kW <= 16 && ((DV / kW) & (DV / kW - 1)) == 0;
    const bool c_ok = chunk == 64 || chunk == 128 || chunk == 256 || chunk == 512;
    return dk_ok && dv_ok && c_ok;
}

size_t chunkwise_bf16_workspace(int B, int H, int N, int DK, int DV, int chunk, int gn, int want_out) {
    (void)DK;
    return ws_layout(B, H, N, DV, chunk, gn && want_out, want_out).total;
}

hipError_t launch_chunkwise_bf16(const LaunchArgs& a) {
    if (a.DK == 64) return a.out_bf16 ? launch_dk<64, bf16>(a) : launch_dk<64, float>(a);
    return a.out_bf16 ? launch_dk<256, bf16>(a) : launch_dk<256, float>(a);
}

}  // namespace ret

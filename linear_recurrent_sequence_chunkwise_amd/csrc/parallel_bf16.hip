// Parallel form of retention on the gfx950 matrix cores, bf16 inputs, fp32 accumulation
// (abeam.tech RetNet summary, retention as content-based reference times distance-based
// forgetting; "Training in parallel"): O = (Q K^T (.) D) V, D[n][m] = g^(n-m) for n >= m.
//
// One workgroup of eight waves per (64 query rows, b, h) owns all d_v output columns, so the
// optional per-head GroupNorm is computed inside it. Workgroups run longest first (query blocks
// from the end of the sequence), which balances the causal triangle's unequal rows over the CUs.
// The keys go by in 32-key blocks up to the diagonal, software-pipelined with one barrier per block:
//   - K and V blocks come in through unconditional buffer loads into registers one iteration
//     ahead, and are written to double-buffered, swizzled LDS tiles;
//   - each wave computes one 16 x 16 tile of S^T = K Q^T (Q fragments stay in registers and serve
//     as the B operand), so that each lane holds 4 consecutive keys of one query row; it applies
//     the causal mask and the decay g^(n-m) in registers and writes P to LDS as a bf16 high part and
//     a bf16 low part (P spans the whole sequence here, so a single bf16 rounding of P would
//     dominate the error);
//   - the scores of block kb + 1 are computed in the same iteration as P V of block kb: the eight
//     waves, arranged 2 x 4 over (rows, column quarters), accumulate P V with both parts; two waves
//     per SIMD, so that one's LDS and load latencies overlap the other's work.
#include "common.hpp"

namespace ret {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKB = 32;  // keys per block

template <int DK, int DV>
struct ParLds {
    // K and V rows unpadded, their 16-byte chunks swizzled (SwzTile): fragment reads of 16 rows and
    // transposing reads then touch distinct banks
    bf16 Ks[2][kKB * DK];  // K blocks kb + 1 and kb + 2 (by parity)
    bf16 Vs[2][kKB * DV];  // V blocks kb and kb + 1
    // P of blocks kb and kb + 1: row r holds the 32 high parts then the 32 low parts (128 bytes),
    // swizzled like K and V
    bf16 P[2][64 * 2 * kKB];
    float red[4][64];
};

// Eight waves, two per SIMD. Scores: wave w computes the 16 x 16 tile S^T of query tile w & 3 and
// key tile w >> 2 of the block. P V: wave w owns rows 32 (w >> 2) .. +32 and the column quarter
// (w & 3) * DV / 4 .. +DV/4.
// chunk > 0: only the keys of the query's own chunk of that many tokens (a multiple of 64), the
// intra-chunk term of the chunkwise form.
template <int DK, int DV, typename TOUT, bool GN>
__global__ __launch_bounds__(kThreads) void parallel_kernel(int H, int N, const bf16* __restrict__ q,
                                                            const bf16* __restrict__ k, const bf16* __restrict__ v,
                                                            TOUT* __restrict__ out, HeadConsts hc, GnArgs gn, int chunk) {
    using Lds = ParLds<DK, DV>;
    using KT = SwzTile<DK * 2>;
    using VT = SwzTile<DV * 2>;
    using PT = SwzTile<4 * kKB>;  // P rows: 32 high then 32 low bf16 parts
    constexpr int CQ = DV / 4;   // columns per wave in P V
    constexpr int CT = CQ / 16;  // 16-column tiles per wave
    static_assert(CQ % 16 == 0, "d_v must split into four groups of 16-column tiles");
    extern __shared__ char smem_raw[];
    Lds& sm = *reinterpret_cast<Lds*>(smem_raw);

    // Workgroup order: longest first (query block nqb - 1 has the most key blocks), and within one
    // query block the heads in turn. Workgroup i runs on XCD i % 8, so with B*H a multiple of 8 an
    // XCD holds the heads bh = XCD (mod 8), and its concurrent workgroups stream the same K and V
    // blocks through its L2.
    const int nqb = (N + 63) / 64, BH = gridDim.x / nqb;
    const int qb = nqb - 1 - (int)(blockIdx.x / BH), bh = blockIdx.x % BH, h = bh % H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    const int qt = w & 3, kt = w >> 2;  // scores tile
    const int wr = w >> 2, wc = w & 3;  // P V rows and column quarter
    const int n0 = qb * 64;
    const float l2g = hc.log2g[h];
    const bf16* qh = q + (size_t)bh * N * DK;
    const bf16* kh = k + (size_t)bh * N * DK;
    const bf16* vh = v + (size_t)bh * N * DV;

    bf16x8 qa[DK / 32];
    const bool qok = n0 + 16 * qt + c16 < N;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qa[ks] = qok ? frag_rowmajor(qh, DK, n0 + 16 * qt, 32 * ks, lane) : zero_bf16x8();

    f32x4 acc[2][CT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkb = min((n0 + 64 + kKB - 1) / kKB, (N + kKB - 1) / kKB);  // key blocks up to the diagonal
    const int kbs = chunk > 0 ? (n0 / chunk) * chunk / kKB : 0;             // first key block
    // K and V rows of a block go through registers (16-byte pieces, idx = threadIdx.x + kThreads * j
    // < pieces; rows past the sequence read as zero): loaded one iteration before they are written
    // to LDS, so that a whole iteration hides the load latency.
    constexpr int KP = kKB * (DK / 8), VP = kKB * (DV / 8);  // 16-byte pieces of a block
    constexpr int NKR = (KP + kThreads - 1) / kThreads, NVR = (VP + kThreads - 1) / kThreads;
    bf16x8 kr[NKR], vr[NVR];
    // Buffer loads over the block's rows (the resource ends at the sequence, so rows past N and
    // pieces past the block read as zero): no branches, so the compiler's load waits stay exact.
    auto load_k = [&](int kb) __attribute__((always_inline)) {
        const int m0 = kb * kKB, rows = min(kKB, N - m0);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kh + (size_t)m0 * DK), 0, (unsigned)(rows * DK * 2), 0x00020000);
#pragma unroll
        for (int j = 0; j < NKR; ++j) {
            const int idx = threadIdx.x + kThreads * j;
            kr[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)(idx * 16), 0, 0));
        }
    };
    auto load_v = [&](int kb) __attribute__((always_inline)) {
        const int m0 = kb * kKB, rows = min(kKB, N - m0);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vh + (size_t)m0 * DV), 0, (unsigned)(rows * DV * 2), 0x00020000);
#pragma unroll
        for (int j = 0; j < NVR; ++j) {
            const int idx = threadIdx.x + kThreads * j;
            vr[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)(idx * 16), 0, 0));
        }
    };
    auto store_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NKR; ++j) {
            const int idx = threadIdx.x + kThreads * j, r = idx / (DK / 8), sg = idx % (DK / 8);
            if (idx < KP) *reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(sm.Ks[buf]) + KT::off(r, sg)) = kr[j];
        }
    };
    auto store_v = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NVR; ++j) {
            const int idx = threadIdx.x + kThreads * j, r = idx / (DV / 8), sg = idx % (DV / 8);
            if (idx < VP) *reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(sm.Vs[buf]) + VT::off(r, sg)) = vr[j];
        }
    };
    // S^T tile of block kb: lane (g4, c16) ends with keys m0 + 16kt + 4g4 + i of query row
    // n0 + 16qt + c16; P = S (.) D goes to LDS as bf16 high and low parts.
    auto scores = [&](int kb) __attribute__((always_inline)) {
        const int m0 = kb * kKB, buf = kb & 1;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (m0 + 16 * kt <= n0 + 16 * qt + 15) {  // a tile wholly above the diagonal stays zero
            constexpr int G = DK / 32 < 4 ? DK / 32 : 4;  // K fragments read together
#pragma unroll
            for (int k0 = 0; k0 < DK / 32; k0 += G) {
                bf16x8 kf[G];
#pragma unroll
                for (int i = 0; i < G; ++i) kf[i] = frag_rowmajor_swz<DK * 2>(reinterpret_cast<const char*>(sm.Ks[buf]), 16 * kt, 32 * (k0 + i), lane);
#pragma unroll
                for (int i = 0; i < G; ++i) s = mfma16(kf[i], qa[k0 + i], s);
            }
        }
        const int n = n0 + 16 * qt + c16;
        bf16x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 16 * kt + 4 * g4 + i;
            const float d = n >= m ? decay_pow(l2g, (float)(n - m)) : 0.f;
            bf16 a, c;
            split_hi_lo(s[i] * d, a, c);
            hi[i] = a;
            lo[i] = c;
        }
        char* prow = reinterpret_cast<char*>(sm.P[buf]);
        const int pr = 16 * qt + c16, pc = 2 * kt + (g4 >> 1), ps = 8 * (g4 & 1);  // row, 16-byte chunk, byte in it
        *reinterpret_cast<bf16x4*>(prow + PT::off(pr, pc) + ps) = hi;
        *reinterpret_cast<bf16x4*>(prow + PT::off(pr, pc + kKB / 8) + ps) = lo;
    };
    // P V of block kb for rows 32wr .. +32, columns wc*CQ .. +CQ
    auto pv = [&](int kb) __attribute__((always_inline)) {
        const int buf = kb & 1;
        bf16x8 ahi[2], alo[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            ahi[rt] = frag_rowmajor_swz<4 * kKB>(reinterpret_cast<const char*>(sm.P[buf]), 32 * wr + 16 * rt, 0, lane);
            alo[rt] = frag_rowmajor_swz<4 * kKB>(reinterpret_cast<const char*>(sm.P[buf]), 32 * wr + 16 * rt, kKB, lane);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const bf16x8 b = lds_frag_kmajor_swz<DV * 2>(reinterpret_cast<const char*>(sm.Vs[buf]), 0, wc * CQ + 16 * ct, lane);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                acc[rt][ct] = mfma16(ahi[rt], b, acc[rt][ct]);
                acc[rt][ct] = mfma16(alo[rt], b, acc[rt][ct]);
            }
        }
    };

    // Software pipeline, one barrier per block. Entering iteration kb, LDS holds K(kb+1), V(kb) and
    // P(kb), and the registers hold K(kb+2) and V(kb+1). Iteration kb writes those registers to the
    // buffers that iteration kb-1 finished reading, loads K(kb+3) and V(kb+2), and computes the
    // scores of block kb+1 together with P V of block kb.
    load_k(kbs);
    load_v(kbs);
    store_k(kbs & 1);
    store_v(kbs & 1);
    if (nkb > kbs + 1) load_k(kbs + 1);
    if (nkb > kbs + 1) load_v(kbs + 1);
    __syncthreads();
    scores(kbs);
    if (nkb > kbs + 1) store_k((kbs + 1) & 1);
    if (nkb > kbs + 2) load_k(kbs + 2);
    for (int kb = kbs; kb < nkb; ++kb) {
        __syncthreads();  // iteration kb-1's reads and writes are done and visible
        if (kb + 2 < nkb) store_k(kb & 1);
        if (kb + 1 < nkb) store_v((kb + 1) & 1);
        if (kb + 3 < nkb) load_k(kb + 3);
        if (kb + 2 < nkb) load_v(kb + 2);
        if (kb + 1 < nkb) scores(kb + 1);
        pv(kb);
    }

    if constexpr (GN) {
        // row statistics over all DV columns: each wave holds a quarter of them
        float mean[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = 0.f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) s += acc[rt][ct][i];
                s = sum16(s);
                if (c16 == 0) sm.red[wc][32 * wr + 16 * rt + 4 * g4 + i] = s;
            }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * wr + 16 * rt + 4 * g4 + i;
                mean[rt][i] = ((sm.red[0][r] + sm.red[1][r]) + (sm.red[2][r] + sm.red[3][r])) * (1.0f / DV);
            }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = 0.f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const float d = acc[rt][ct][i] - mean[rt][i];
                    s += d * d;
                }
                s = sum16(s);
                if (c16 == 0) sm.red[wc][32 * wr + 16 * rt + 4 * g4 + i] = s;
            }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 32 * wr + 16 * rt + 4 * g4 + i;
                const float var = ((sm.red[0][r] + sm.red[1][r]) + (sm.red[2][r] + sm.red[3][r])) * (1.0f / DV);
                const float inv = rsqrtf(var + gn.eps);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int c = wc * CQ + 16 * ct + c16;
                    const float wv = gn.weight ? gn.weight[(size_t)h * DV + c] : 1.f;
                    const float bv = gn.bias ? gn.bias[(size_t)h * DV + c] : 0.f;
                    acc[rt][ct][i] = (acc[rt][ct][i] - mean[rt][i]) * inv * wv + bv;
                }
            }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + 32 * wr + 16 * rt + 4 * g4 + i;
            if (n < N) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const size_t e = ((size_t)bh * N + n) * DV + wc * CQ + 16 * ct + c16;
                    float val = acc[rt][ct][i];
                    if constexpr (GN) {
                        if (gn.gate) val *= swish(gate_at(gn, e));  // the swish gate after GroupNorm
                    }
                    out[e] = from_float<TOUT>(val);
                }
            }
        }
}

template <int DK, int DV, typename TOUT, bool GN>
hipError_t launch_typed(const LaunchArgs& a) {
    const size_t lds = sizeof(ParLds<DK, DV>);
    const void* kern = reinterpret_cast<const void*>(parallel_kernel<DK, DV, TOUT, GN>);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((parallel_kernel<DK, DV, TOUT, GN>), dim3((a.N + 63) / 64 * a.B * a.H), dim3(kThreads), lds, a.stream,
                       a.H, a.N, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (TOUT*)a.out, a.hc, a.gn, a.intra_chunk);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_shape(const LaunchArgs& a) {
    if (a.out_bf16) return a.gn.enabled ? launch_typed<DK, DV, bf16, true>(a) : launch_typed<DK, DV, bf16, false>(a);
    return a.gn.enabled ? launch_typed<DK, DV, float, true>(a) : launch_typed<DK, DV, float, false>(a);
}

}  // namespace

// d_k 64 or 256 (K rows of whole 128-byte lines); d_v 64 .. 512, four column groups of 16-column tiles
bool parallel_bf16_supported(int DK, int DV) {
    return (DK == 64 || DK == 256) && (DV == 64 || DV == 128 || DV == 256 || DV == 512);
}

template <int DK>
hipError_t launch_dk(const LaunchArgs& a) {
    switch (a.DV) {
        case 64: return launch_shape<DK, 64>(a);
        case 128: return launch_shape<DK, 128>(a);
        case 256: return launch_shape<DK, 256>(a);
        default: return launch_shape<DK, 512>(a);
    }
}

hipError_t launch_parallel_bf16(const LaunchArgs& a) { return a.DK == 64 ? launch_dk<64>(a) : launch_dk<256>(a); }

}  // namespace ret

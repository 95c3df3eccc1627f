// Chunkwise recurrent retention, bf16 inputs, fp32 accumulation, on the gfx950 matrix cores.
//
// Method (abeam.tech RetNet summary, "Chunk recursion for long-sequence training"; mlnews.online
// RetNet abstract: chunks encoded in parallel, summarised recurrently). Unrolling the recurrence
// S_n = g S_(n-1) + k_n^T v_n over one chunk of length L with carried state R gives, for local row j,
//     o_j = [(Q K^T (.) D) V]_j + g^(j+1) [Q R]_j,      D[j][t] = g^(j-t) for t <= j
//     R  <- g^L R + K^T (V (.) zeta),                    zeta_t = g^(L-1-t)
//
// Two kernels:
//   chunk_scores_kernel   parallel over (64-row band, chunk, b*h): P = (Q K^T) (.) D on MFMA with the
//                         decay and causal mask applied in registers, stored as bf16 in the workspace
//                         (32-key blocks on and below the diagonal). Q and K go through LDS with all
//                         loads of a block issued together; the next key block is prefetched.
//   chunk_main_kernel     one workgroup per (b, h, 32-column slice of d_v), walking the sequence in
//                         32-token stages. Each stage's Q, K, V and P rows are prefetched into
//                         registers two stages ahead, then written to LDS. Per stage:
//                           out  = g^(j+1) Q R + P V      (R from the previous chunk, as bf16 hi + lo,
//                                                         held in registers for the whole chunk)
//                           R   += K^T (V (.) zeta)       (V (.) zeta as bf16 hi + lo; R fp32 in
//                                                         accumulators, scaled by g^L at chunk start)
//                         The optional per-head GroupNorm needs statistics over all d_v columns,
//                         which 16 workgroups share: they exchange tagged per-row partial
//                         statistics through global memory (see the kernel), with workgroups
//                         co-resident through a cooperative launch. The slices of one head sit on
//                         one XCD to share L2.
#include "common.hpp"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kW = 32;     // d_v columns per workgroup
constexpr int kST = 32;    // tokens per pipeline stage
constexpr int kRingP = 8;  // GroupNorm partials ring (stages); >= 6 needed for the reuse argument
constexpr int kRingM = 8;  // GroupNorm merged-statistics ring (stages); >= 4 needed
constexpr int kRedLag = 2; // the reducer of stage x merges its partials during stage x + kRedLag
constexpr int kGnLag = 5;  // stage x is normalised and stored during stage x + kGnLag
constexpr unsigned kSpinLimit = 1u << 24;

// ---------------------------------------------------------------------------------------------
// P = (Q K^T) (.) D. Grid (C/64 bands, nchunks, B*H). Wave w owns row tile t = 4*band + w and
// writes key tiles 0 .. (t|1): for even t the second tile of the diagonal 32-key block is all
// zero but written, so that the consumer reads whole 32-key steps.
template <int DK>
__global__ __launch_bounds__(kThreads) void chunk_scores_kernel(int H, int N, int C, int nchunks,
                                                                const bf16* __restrict__ q,
                                                                const bf16* __restrict__ k,
                                                                bf16* __restrict__ P, HeadConsts hc) {
    constexpr int LD = DK + 8;           // 16-byte fragment reads of 16 rows: distinct banks
    constexpr int NCH = 64 * DK / 8 / kThreads;  // 16-byte chunks per thread for a 64-row block
    __shared__ bf16 Qs[64 * LD];
    __shared__ bf16 Ks[2][64 * LD];
    const int band = blockIdx.x, chunk = blockIdx.y, bh = blockIdx.z, h = bh % H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    const int c0 = chunk * C;
    const int L = min(C, N - c0);
    const bf16* qb = q + ((size_t)bh * N + c0) * DK;
    const bf16* kb = k + ((size_t)bh * N + c0) * DK;
    bf16* Pc = P + ((size_t)bh * nchunks + chunk) * (size_t)C * C;
    const float l2g = hc.log2g[h];

    auto load_block = [&](const bf16* base, int row0, bf16x8* r) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int j = threadIdx.x + kThreads * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            r[u] = row0 + row < L ? *reinterpret_cast<const bf16x8*>(base + (size_t)(row0 + row) * DK + 8 * sg)
                                  : zero_bf16x8();
        }
    };
    auto store_block = [&](bf16* dst, const bf16x8* r) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int j = threadIdx.x + kThreads * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            *reinterpret_cast<bf16x8*>(dst + row * LD + 8 * sg) = r[u];
        }
    };

    bf16x8 rq[NCH], rk[NCH];
    load_block(qb, 64 * band, rq);
    load_block(kb, 0, rk);
    store_block(Qs, rq);
    store_block(Ks[0], rk);
    if (band > 0) load_block(kb, 64, rk);
    __syncthreads();

    const int t = 4 * band + w;  // row tile of this wave
    bf16x8 qa[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) qa[ks] = frag_rowmajor(Qs, LD, 16 * w, 32 * ks, lane);

    for (int kbk = 0; kbk <= band; ++kbk) {
        const bf16* Kc = Ks[kbk & 1];
        // key tiles of this block that the row tile needs: up to (t|1)
        const int last = min(3, (t | 1) - 4 * kbk);
        for (int kt = 0; kt <= last; ++kt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) s = mfma16(qa[ks], frag_rowmajor(Kc, LD, 16 * kt, 32 * ks, lane), s);
            const int key = 64 * kbk + 16 * kt + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * t + 4 * g4 + i;
                const float d = row >= key ? decay_pow(l2g, (float)(row - key)) : 0.f;
                Pc[(size_t)row * C + key] = (bf16)(s[i] * d);
            }
        }
        if (kbk < band) {
            store_block(Ks[(kbk + 1) & 1], rk);
            if (kbk + 2 <= band) load_block(kb, 64 * (kbk + 2), rk);
            __syncthreads();
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
    unsigned long long* part;    // [teams][kRingP][NP][32] x 2 tagged words: per-16-column row partials
    unsigned long long* merged;  // [teams][kRingM][32] x 2 tagged words: (mean, 1/std) per row
    unsigned* err_flag;
    GnArgs gn;
};

template <int DK, int C>
struct MainGeom {
    static constexpr int LQ = DK + 8;    // Q rows (16-byte reads)
    static constexpr int LK = DK + 16;   // K rows (transposing reads)
    static constexpr int LP = C + 8;     // P rows (16-byte reads)
    static constexpr int LV = kW + 16;   // V rows (transposing reads)
    static constexpr int LR = DK + 8;    // R^T rows (16-byte reads)
    static constexpr int QCH = kST * DK / 8;                    // 16-byte chunks of Q (or K) per stage
    static constexpr int QN = (QCH + kThreads - 1) / kThreads;  // ... per thread
    static constexpr int PN = kST * C / 8 / kThreads;           // P chunk slots per thread: 32 rows x C/8
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + (size_t)kST * LQ * 2;
    static constexpr size_t OFF_P = OFF_K + (size_t)kST * LK * 2;
    static constexpr size_t OFF_V = OFF_P + (size_t)kST * LP * 2;
    static constexpr size_t OFF_RH = OFF_V + (size_t)C * LV * 2;
    static constexpr size_t OFF_RL = OFF_RH + (size_t)kW * LR * 2;
    static constexpr size_t OFF_ZH = OFF_RL + (size_t)kW * LR * 2;   // V (.) zeta, bf16 high part, this stage
    static constexpr size_t OFF_ZL = OFF_ZH + (size_t)kST * LV * 2;  // ... low part
    static constexpr size_t BYTES = OFF_ZL + (size_t)kST * LV * 2;
};

template <int DK, int C>
struct StageRegs {
    bf16x8 q[MainGeom<DK, C>::QN];
    bf16x8 k[MainGeom<DK, C>::QN];
    bf16x8 p[MainGeom<DK, C>::PN > 0 ? MainGeom<DK, C>::PN : 1];
    bf16x8 v;
};

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ unsigned long long tagged(float x, unsigned tag) {
    return ((unsigned long long)tag << 32) | __builtin_bit_cast(unsigned, x);
}
__device__ __forceinline__ float untag(unsigned long long w) { return __builtin_bit_cast(float, (unsigned)w); }
__device__ __forceinline__ unsigned long long ld_tagged(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(unsigned long long* p, unsigned long long w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge two (mean, M2) summaries of n values each. Symmetric in its arguments, so every lane of a
// butterfly ends with the bitwise-same result.
__device__ __forceinline__ void merge_eq(float& mean, float& m2, float om, float o2, float n) {
    const float d = om - mean;
    m2 = (m2 + o2) + d * d * (n * 0.5f);
    mean = (mean + om) * 0.5f;
}

// One (b, h, d_v slice) per workgroup. Wave w owns R rows [w*DK/4, (w+1)*DK/4) (state update) and,
// in every 32-token stage, the 16 x 16 output tile (rows 16*(w>>1), columns 16*(w&1)).
//
// GroupNorm exchange (no counters, no fences): every value is published as a 64-bit atomic store
// whose high half is a tag (stage + 1), so a reader knows whether it sees the current stage.
//   stage g, end:   each wave publishes per-row (mean, M2) of its 16 columns for stage g;
//   stage g, end:   the slice (g-2) % NS ("reducer") merges all partials of stage g-2 in a fixed
//                   order and publishes (mean, 1/std) per row;
//   stage g, end:   every workgroup normalises and stores its stage g-5 tile, using the merged
//                   statistics it loaded during stage g-1.
// The loads feeding these steps are issued at the start of a stage, ahead of the prefetch, so that
// waiting for them never waits for the prefetch; a stale tag (rare) makes the lane re-load until
// the tag matches.
template <int DK, int C, typename TOUT, bool GN, bool WANT_OUT>
__global__ __launch_bounds__(kThreads) void chunk_main_kernel(MainParams p, HeadConsts hc) {
    using G = MainGeom<DK, C>;
    constexpr int RTR = DK / 64;  // 16-row R tiles per wave
    constexpr int SPC = C / kST;  // stages per full chunk
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* Qs = reinterpret_cast<bf16*>(smem + G::OFF_Q);
    bf16* Ks = reinterpret_cast<bf16*>(smem + G::OFF_K);
    bf16* Ps = reinterpret_cast<bf16*>(smem + G::OFF_P);
    bf16* Vs = reinterpret_cast<bf16*>(smem + G::OFF_V);
    bf16* Rhi = reinterpret_cast<bf16*>(smem + G::OFF_RH);
    bf16* Rlo = reinterpret_cast<bf16*>(smem + G::OFF_RL);
    bf16* VZh = reinterpret_cast<bf16*>(smem + G::OFF_ZH);
    bf16* VZl = reinterpret_cast<bf16*>(smem + G::OFF_ZL);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    // XCD-aware placement: workgroup i runs on XCD i % 8. With a multiple of 8 teams per launch,
    // all slices of a team share i % 8 and therefore one L2.
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
    const int N = p.N, DV = p.NS * kW, NS = p.NS;
    const float l2g = hc.log2g[h];
    const int col0 = slice * kW;
    const int nchunks = p.nchunks;
    const int L_last = N - (nchunks - 1) * C;
    const int total = (nchunks - 1) * SPC + (L_last + kST - 1) / kST;
    const int rt_o = w >> 1, ct_o = w & 1;  // output tile of this wave within a stage

    // Buffer resources: loads past the end of a head's data return zero (tail rows, padding).
    const unsigned q_bytes = (unsigned)((size_t)N * DK * 2), v_bytes = (unsigned)((size_t)N * DV * 2);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + (size_t)bh * N * DK), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)bh * N * DK), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)bh * N * DV), 0, v_bytes, 0x00020000);
    const unsigned p_bytes = WANT_OUT ? (unsigned)((size_t)nchunks * C * C * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(WANT_OUT ? p.P + (size_t)bh * nchunks * C * C : p.q), 0, p_bytes, 0x00020000);

    // ---- stage loads: global -> registers (unconditional instructions), registers -> LDS
    auto load_stage = [&](StageRegs<DK, C>& r, int g) __attribute__((always_inline)) {
        const int gg = g < total ? g : total - 1;  // past the end: reload the last stage (unused)
        const int ci = gg / SPC, s = gg % SPC;
        const int tok0 = ci * C + kST * s;
#pragma unroll
        for (int u = 0; u < G::QN; ++u) {
            const int j = threadIdx.x + kThreads * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            const unsigned off = j < G::QCH ? (unsigned)((tok0 + row) * DK + 8 * sg) * 2u : q_bytes;
            if constexpr (WANT_OUT) r.q[u] = buf_load16(rq, off);
            r.k[u] = buf_load16(rk, off);
        }
        {
            const int row = threadIdx.x >> 2, sg = threadIdx.x & 3;  // 32 rows x 4 chunks of 8 columns
            const unsigned off = threadIdx.x < kST * 4 ? (unsigned)((tok0 + row) * DV + col0 + 8 * sg) * 2u : v_bytes;
            r.v = buf_load16(rv, off);
        }
        if constexpr (WANT_OUT) {
            const int per_row = 4 * (s + 1);  // 16-byte chunks needed per row: keys [0, 32(s+1))
            const unsigned base = (unsigned)((ci * C + kST * s) * C);
#pragma unroll
            for (int u = 0; u < G::PN; ++u) {
                const int j = threadIdx.x + kThreads * u;
                const int row = j / (C / 8), sg = j % (C / 8);
                const unsigned off = sg < per_row ? (base + (unsigned)(row * C + 8 * sg)) * 2u : p_bytes;
                r.p[u] = buf_load16(rp, off);
            }
        }
    };
    auto store_stage = [&](const StageRegs<DK, C>& r, int s, int L) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < G::QN; ++u) {
            const int j = threadIdx.x + kThreads * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            if (G::QCH % kThreads == 0 || j < G::QCH) {
                if constexpr (WANT_OUT) *reinterpret_cast<bf16x8*>(Qs + row * G::LQ + 8 * sg) = r.q[u];
                *reinterpret_cast<bf16x8*>(Ks + row * G::LK + 8 * sg) = r.k[u];
            }
        }
        if (threadIdx.x < kST * 4) {
            const int row = threadIdx.x >> 2, sg = threadIdx.x & 3;
            *reinterpret_cast<bf16x8*>(Vs + (kST * s + row) * G::LV + 8 * sg) = r.v;
            // V (.) zeta for the state update, split once here into bf16 high and low parts
            const int t = kST * s + row;
            const float z = t < L ? decay_pow(l2g, (float)(L - 1 - t)) : 0.f;
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 a, b;
                split_hi_lo((float)r.v[e] * z, a, b);
                hi[e] = a;
                lo[e] = b;
            }
            *reinterpret_cast<bf16x8*>(VZh + row * G::LV + 8 * sg) = hi;
            *reinterpret_cast<bf16x8*>(VZl + row * G::LV + 8 * sg) = lo;
        }
        if constexpr (WANT_OUT) {
            const int per_row = 4 * (s + 1);
#pragma unroll
            for (int u = 0; u < G::PN; ++u) {
                const int j = threadIdx.x + kThreads * u;
                const int row = j / (C / 8), sg = j % (C / 8);
                if (sg < per_row) *reinterpret_cast<bf16x8*>(Ps + row * G::LP + 8 * sg) = r.p[u];
            }
        }
    };

    // ---- carried state: wave w owns R rows [w*DK/4, (w+1)*DK/4) x 32 columns, fp32
    f32x4 accR[RTR][2];
#pragma unroll
    for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = w * (DK / 4) + 16 * rt + 4 * g4 + i;
                accR[rt][ct][i] = p.state_in ? p.state_in[((size_t)bh * DK + row) * DV + col0 + 16 * ct + c16] : 0.f;
            }
    auto write_R = [&]() __attribute__((always_inline)) {
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
                const int col = 16 * ct + c16, row = w * (DK / 4) + 16 * rt + 4 * g4;
                *reinterpret_cast<bf16x4*>(Rhi + col * G::LR + row) = hi;
                *reinterpret_cast<bf16x4*>(Rlo + col * G::LR + row) = lo;
            }
    };
    // R^T fragments (B operand of Q R) for this wave's output column tile, for one whole chunk
    bf16x8 rfh[DK / 32], rfl[DK / 32];
    auto read_R_frags = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            rfh[ks] = frag_rowmajor(Rhi, G::LR, 16 * ct_o, 32 * ks, lane);
            rfl[ks] = frag_rowmajor(Rlo, G::LR, 16 * ct_o, 32 * ks, lane);
        }
    };

    TOUT* out = reinterpret_cast<TOUT*>(p.out);
    auto store_tile = [&](const f32x4& a, int g) __attribute__((always_inline)) {
        const int ci = g / SPC, s = g % SPC, c0 = ci * C;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = c0 + kST * s + 16 * rt_o + 4 * g4 + i;
            if (r < N) out[((size_t)bh * N + r) * DV + col0 + 16 * ct_o + c16] = from_float<TOUT>(a[i]);
        }
    };

    // ---- GroupNorm exchange state (see the comment above the kernel)
    const int NP = 2 * NS;                 // 16-column partials per row
    const int LPR = NP < 8 ? NP : 8;       // reducer lanes per row
    const int PPL = NP < 8 ? 1 : NP / 8;   // partials merged locally per reducer lane (<= 4)
    unsigned long long* part_team = p.part + (size_t)bh * kRingP * NP * kST * 2;
    unsigned long long* merged_team = p.merged + (size_t)bh * kRingM * kST * 2;
    // affine parameters of this lane's output column, loaded once
    float gw = 1.f, gb = 0.f;
    if constexpr (GN) {
        const int c = col0 + 16 * ct_o + c16;
        if (p.gn.weight) gw = p.gn.weight[(size_t)h * DV + c];
        if (p.gn.bias) gb = p.gn.bias[(size_t)h * DV + c];
    }
    f32x4 pend[kGnLag];  // output tiles of stages g-1 .. g-kGnLag (pend[k] = stage g-1-k)
#pragma unroll
    for (int k = 0; k < kGnLag; ++k) pend[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    unsigned long long red_w[4][2];   // reducer: this lane's loaded partials
    unsigned long long mrg_w[2][2];   // (mean, 1/std) of row 4*g4 + (c16 & 3), for two stages in flight
    const int rrow = 8 * w + (lane >> 3), rk8 = lane & 7;  // reducer: row and lane within the row
    const int mrow = 16 * rt_o + 4 * g4 + (c16 & 3);       // row whose merged statistics this lane loads

    auto spin_fail = [&]() __attribute__((always_inline)) { atomicOr(p.err_flag, 1u); };
    auto reducer_issue = [&](int gr) __attribute__((always_inline)) {
        const unsigned long long* src = part_team + (size_t)(gr % kRingP) * NP * kST * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pi = (NP < 8 ? rk8 % NP : rk8 + 8 * j);
            if (j < PPL) {
                red_w[j][0] = ld_tagged(src + ((size_t)pi * kST + rrow) * 2);
                red_w[j][1] = ld_tagged(src + ((size_t)pi * kST + rrow) * 2 + 1);
            }
        }
    };
    auto reducer_finish = [&](int gr) __attribute__((always_inline)) {
        const unsigned tag = (unsigned)gr + 1u;
        const unsigned long long* src = part_team + (size_t)(gr % kRingP) * NP * kST * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < PPL) {
                const int pi = (NP < 8 ? rk8 % NP : rk8 + 8 * j);
                if ((unsigned)(red_w[j][0] >> 32) != tag || (unsigned)(red_w[j][1] >> 32) != tag) {
                    unsigned spins = 0;
                    do {
                        __builtin_amdgcn_s_sleep(1);
                        red_w[j][0] = ld_tagged(src + ((size_t)pi * kST + rrow) * 2);
                        red_w[j][1] = ld_tagged(src + ((size_t)pi * kST + rrow) * 2 + 1);
                        if (++spins > kSpinLimit) { spin_fail(); break; }
                    } while ((unsigned)(red_w[j][0] >> 32) != tag || (unsigned)(red_w[j][1] >> 32) != tag);
                }
            }
        }
        // fixed merge tree: ((p0, p1), (p2, p3)) locally, then across the row's lanes
        float pm[4], p2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) { pm[j] = untag(red_w[j][0]); p2[j] = untag(red_w[j][1]); }
        float mean = pm[0], m2 = p2[0], n = 16.f;
        if (PPL == 4) {
            merge_eq(pm[0], p2[0], pm[1], p2[1], 16.f);
            merge_eq(pm[2], p2[2], pm[3], p2[3], 16.f);
            merge_eq(pm[0], p2[0], pm[2], p2[2], 32.f);
            mean = pm[0]; m2 = p2[0]; n = 64.f;
        } else if (PPL == 2) {
            merge_eq(pm[0], p2[0], pm[1], p2[1], 16.f);
            mean = pm[0]; m2 = p2[0]; n = 32.f;
        }
        for (int off = 1; off < LPR; off <<= 1) {
            const float om = __shfl_xor(mean, off, 64), o2 = __shfl_xor(m2, off, 64);
            merge_eq(mean, m2, om, o2, n);
            n *= 2.f;
        }
        if (rk8 == 0) {
            const float rstd = rsqrtf(m2 / (float)DV + p.gn.eps);
            unsigned long long* dst = merged_team + (size_t)(gr % kRingM) * kST * 2 + (size_t)rrow * 2;
            st_tagged(dst, tagged(mean, tag));
            st_tagged(dst + 1, tagged(rstd, tag));
        }
    };
    auto merged_issue = [&](int gf, int b) __attribute__((always_inline)) {
        const unsigned long long* src = merged_team + (size_t)(gf % kRingM) * kST * 2 + (size_t)mrow * 2;
        mrg_w[b][0] = ld_tagged(src);
        mrg_w[b][1] = ld_tagged(src + 1);
    };
    auto finalize = [&](f32x4 a, int gf, int b) __attribute__((always_inline)) {
        const unsigned tag = (unsigned)gf + 1u;
        if ((unsigned)(mrg_w[b][0] >> 32) != tag || (unsigned)(mrg_w[b][1] >> 32) != tag) {
            const unsigned long long* src = merged_team + (size_t)(gf % kRingM) * kST * 2 + (size_t)mrow * 2;
            unsigned spins = 0;
            do {
                __builtin_amdgcn_s_sleep(1);
                mrg_w[b][0] = ld_tagged(src);
                mrg_w[b][1] = ld_tagged(src + 1);
                if (++spins > kSpinLimit) { spin_fail(); break; }
            } while ((unsigned)(mrg_w[b][0] >> 32) != tag || (unsigned)(mrg_w[b][1] >> 32) != tag);
        }
        const float mean_l = untag(mrg_w[b][0]), rstd_l = untag(mrg_w[b][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mean = __shfl(mean_l, 16 * g4 + i, 64), rstd = __shfl(rstd_l, 16 * g4 + i, 64);
            a[i] = (a[i] - mean) * rstd * gw + gb;
        }
        store_tile(a, gf);
    };
    auto publish = [&](const f32x4& a, int g) __attribute__((always_inline)) {
        const unsigned tag = (unsigned)g + 1u;
        unsigned long long* dst = part_team + ((size_t)(g % kRingP) * NP + 2 * slice + ct_o) * kST * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mean = sum16(a[i]) * (1.0f / 16.0f);
            const float d = a[i] - mean;
            const float m2 = sum16(d * d);
            if (c16 == 0) {
                const int rr = 16 * rt_o + 4 * g4 + i;
                st_tagged(dst + (size_t)rr * 2, tagged(mean, tag));
                st_tagged(dst + (size_t)rr * 2 + 1, tagged(m2, tag));
            }
        }
    };
    // GroupNorm bookkeeping for step g (a pipeline stage, or a drain step after the last one). The
    // loads are issued at the start of a step, before that step's prefetch, so that waiting for them
    // never waits for the prefetch; merged statistics are used one step after they are loaded.
    //   reducer of stage g-kRedLag: load its partials now, merge and publish at the end of this step
    //   merged statistics of stage g-kGnLag+1: load now (buffer b), use next step
    //   stage g-kGnLag: normalise with the statistics loaded last step (buffer b^1) and store
    auto gn_issue = [&](int g, int b) __attribute__((always_inline)) {
        const int gr = g - kRedLag;
        if (gr >= 0 && gr < total && gr % NS == slice) reducer_issue(gr);
        const int gm = g - kGnLag + 1;
        if (gm >= 0 && gm < total) merged_issue(gm, b);
    };
    auto gn_finish = [&](int g, int b) __attribute__((always_inline)) {
        const int gr = g - kRedLag;
        if (gr >= 0 && gr < total && gr % NS == slice) reducer_finish(gr);
        const int gf = g - kGnLag;
        if (gf >= 0 && gf < total) finalize(pend[kGnLag - 1], gf, b ^ 1);
    };

    // ---- one pipeline stage
    auto stage = [&](StageRegs<DK, C>& r, int g) __attribute__((always_inline)) {
        const int ci = g / SPC, s = g % SPC;
        const int L = min(C, N - ci * C);
        const bool chunk_end = (s == SPC - 1) || (g == total - 1);
        __syncthreads();  // (A) the previous stage's LDS reads are done
        if (s == 0) {
            const float gL = decay_pow(l2g, (float)L);
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) accR[rt][ct] *= gL;
        }
        store_stage(r, s, L);
        if constexpr (WANT_OUT && GN) gn_issue(g, g & 1);
        load_stage(r, g + 2);
        __syncthreads();  // (B)
        if (s == 0 && WANT_OUT) read_R_frags();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (WANT_OUT) {
            // inter-chunk: Q R with R = hi + lo, in four independent accumulator chains so the
            // matrix core is not held up by the latency of one long dependent chain
            f32x4 qa[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) qa[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const bf16x8 a = frag_rowmajor(Qs, G::LQ, 16 * rt_o, 32 * ks, lane);
                qa[2 * (ks & 1)] = mfma16(a, rfh[ks], qa[2 * (ks & 1)]);
                qa[2 * (ks & 1) + 1] = mfma16(a, rfl[ks], qa[2 * (ks & 1) + 1]);
            }
            const f32x4 qr = (qa[0] + qa[2]) + (qa[1] + qa[3]);
            // intra-chunk: P V over the 32-key steps up to this stage
            f32x4 pv = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks <= s; ++ks) {
                const bf16x8 a = frag_rowmajor(Ps, G::LP, 16 * rt_o, 32 * ks, lane);
                const bf16x8 b = lds_frag_kmajor(Vs, G::LV, 32 * ks, 16 * ct_o, lane);
                pv = mfma16(a, b, pv);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = qr[i] * decay_pow(l2g, (float)(kST * s + 16 * rt_o + 4 * g4 + i + 1)) + pv[i];
        }
        // state: R += K^T (V (.) zeta) for the 32 tokens of this stage
        {
            bf16x8 bhi[2], blo[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bhi[ct] = lds_frag_kmajor(VZh, G::LV, 0, 16 * ct, lane);
                blo[ct] = lds_frag_kmajor(VZl, G::LV, 0, 16 * ct, lane);
            }
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) {
                const bf16x8 ak = lds_frag_kmajor(Ks, G::LK, 0, w * (DK / 4) + 16 * rt, lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    accR[rt][ct] = mfma16(ak, bhi[ct], accR[rt][ct]);
                    accR[rt][ct] = mfma16(ak, blo[ct], accR[rt][ct]);
                }
            }
        }
        if constexpr (WANT_OUT) {
            if constexpr (GN) {
                publish(acc, g);
                gn_finish(g, g & 1);
#pragma unroll
                for (int k = kGnLag - 1; k > 0; --k) pend[k] = pend[k - 1];
                pend[0] = acc;
            } else {
                store_tile(acc, g);
            }
        }
        if (chunk_end) {
            __syncthreads();  // (C) all reads of R^T for this chunk are done
            write_R();
        }
    };

    write_R();
    StageRegs<DK, C> r0, r1;
    load_stage(r0, 0);
    load_stage(r1, 1);
    for (int g = 0; g < total; g += 2) {
        stage(r0, g);
        if (g + 1 < total) stage(r1, g + 1);
    }
    if constexpr (WANT_OUT && GN) {
        // drain: the last reductions and normalisations, no compute
        for (int g = total; g < total + kGnLag; ++g) {
            gn_issue(g, g & 1);
            gn_finish(g, g & 1);
#pragma unroll
            for (int k = kGnLag - 1; k > 0; --k) pend[k] = pend[k - 1];
        }
    }
    if (p.state_out) {
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = w * (DK / 4) + 16 * rt + 4 * g4 + i;
                    p.state_out[((size_t)bh * DK + row) * DV + col0 + 16 * ct + c16] = accR[rt][ct][i];
                }
    }
}


// GroupNorm statistics exchange between the workgroups (slices) of one head. Every value is a 64-bit
// atomic store whose high half is a tag (stage + 1), so a reader can tell whether it sees the
// current stage; the rings are cleared before each call. No counters, no fences:
//   stage x, end:            each output wave publishes per-row (mean, M2) of its 16 columns;
//   stage x + kRedLag, end:  slice x % NS merges all partials of stage x in a fixed order and
//                            publishes (mean, 1/std) per row;
//   stage x + kGnLag - 1:    every output wave loads the merged statistics of its rows;
//   stage x + kGnLag, end:   it normalises and stores its stage-x tile.
// Loads are issued at the start of a step, before that step's prefetch, so waiting for them never
// waits for the prefetch; a stale tag (rare) makes the lane re-load until the tag matches.
// One output wave owns one 16 x 16 tile per stage: rows 16*rt_o .. of the stage, 16 columns.
template <typename TOUT>
struct GnExchange {
    int NS, NP, LPR, PPL, total, slice, part_idx, rt_o, lane, g4, c16, bh, N, DV, col_out, SPC, C;
    float eps, gw, gb;
    unsigned long long* part_team;
    unsigned long long* merged_team;
    unsigned* err_flag;
    TOUT* out;
    unsigned long long red_w[4][2];  // reducer: this lane's loaded partials
    unsigned long long mrg_a[2], mrg_b[2];  // merged (mean, 1/std) of row mrow, two steps in flight (by parity)
    int rrow, rk8, mrow;

    __device__ __forceinline__ void init(const MainParams& p, int bh_, int h, int slice_, int wave_in_group, int lane_, int total_,
                                         int spc, int C_) {
        NS = p.NS; NP = 2 * NS; LPR = NP < 8 ? NP : 8; PPL = NP < 8 ? 1 : NP / 8;
        total = total_; slice = slice_; bh = bh_; N = p.N; DV = NS * 32; SPC = spc; C = C_;
        lane = lane_; g4 = lane >> 4; c16 = lane & 15;
        rt_o = wave_in_group >> 1;
        const int ct_o = wave_in_group & 1;
        part_idx = 2 * slice + ct_o;
        col_out = slice * 32 + 16 * ct_o + c16;
        eps = p.gn.eps;
        gw = p.gn.weight ? p.gn.weight[(size_t)h * DV + col_out] : 1.f;
        gb = p.gn.bias ? p.gn.bias[(size_t)h * DV + col_out] : 0.f;
        part_team = p.part + (size_t)bh * kRingP * NP * kST * 2;
        merged_team = p.merged + (size_t)bh * kRingM * kST * 2;
        err_flag = p.err_flag;
        out = reinterpret_cast<TOUT*>(p.out);
        rrow = 8 * wave_in_group + (lane >> 3);
        rk8 = lane & 7;
        mrow = 16 * rt_o + 4 * g4 + (c16 & 3);
    }
    __device__ __forceinline__ void store_tile(f32x4 a, int g) const {
        const int c0 = (g / SPC) * C, s = g % SPC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = c0 + kST * s + 16 * rt_o + 4 * g4 + i;
            if (r < N) out[((size_t)bh * N + r) * DV + col_out] = from_float<TOUT>(a[i]);
        }
    }
    __device__ __forceinline__ const unsigned long long* part_at(int g, int pi, int row) const {
        return part_team + (((size_t)(g % kRingP) * NP + pi) * kST + row) * 2;
    }
    __device__ __forceinline__ void publish(f32x4 a, int g) const {
        const unsigned tag = (unsigned)g + 1u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mean = sum16(a[i]) * (1.0f / 16.0f);
            const float d = a[i] - mean;
            const float m2 = sum16(d * d);
            if (c16 == 0) {
                unsigned long long* dst = const_cast<unsigned long long*>(part_at(g, part_idx, 16 * rt_o + 4 * g4 + i));
                st_tagged(dst, tagged(mean, tag));
                st_tagged(dst + 1, tagged(m2, tag));
            }
        }
    }
    __device__ __forceinline__ bool is_reducer(int gr) const { return gr >= 0 && gr < total && gr % NS == slice; }
    __device__ __forceinline__ int red_pi(int j) const { return NP < 8 ? rk8 % NP : rk8 + 8 * j; }
    __device__ __forceinline__ void reducer_issue(int gr) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < PPL) {
                const unsigned long long* src = part_at(gr, red_pi(j), rrow);
                red_w[j][0] = ld_tagged(src);
                red_w[j][1] = ld_tagged(src + 1);
            }
    }
    __device__ __forceinline__ void reducer_finish(int gr) {
        const unsigned tag = (unsigned)gr + 1u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < PPL && ((unsigned)(red_w[j][0] >> 32) != tag || (unsigned)(red_w[j][1] >> 32) != tag)) {
                const unsigned long long* src = part_at(gr, red_pi(j), rrow);
                unsigned spins = 0;
                do {
                    __builtin_amdgcn_s_sleep(1);
                    red_w[j][0] = ld_tagged(src);
                    red_w[j][1] = ld_tagged(src + 1);
                    if (++spins > kSpinLimit) { atomicOr(err_flag, 1u); break; }
                } while ((unsigned)(red_w[j][0] >> 32) != tag || (unsigned)(red_w[j][1] >> 32) != tag);
            }
        }
        // fixed merge tree: ((p0, p1), (p2, p3)) locally, then across the row's lanes
        float pm[4], p2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) { pm[j] = untag(red_w[j][0]); p2[j] = untag(red_w[j][1]); }
        float mean = pm[0], m2 = p2[0], n = 16.f;
        if (PPL == 4) {
            merge_eq(pm[0], p2[0], pm[1], p2[1], 16.f);
            merge_eq(pm[2], p2[2], pm[3], p2[3], 16.f);
            merge_eq(pm[0], p2[0], pm[2], p2[2], 32.f);
            mean = pm[0]; m2 = p2[0]; n = 64.f;
        } else if (PPL == 2) {
            merge_eq(pm[0], p2[0], pm[1], p2[1], 16.f);
            mean = pm[0]; m2 = p2[0]; n = 32.f;
        }
        for (int off = 1; off < LPR; off <<= 1) {
            const float om = __shfl_xor(mean, off, 64), o2 = __shfl_xor(m2, off, 64);
            merge_eq(mean, m2, om, o2, n);
            n *= 2.f;
        }
        if (rk8 == 0) {
            const float rstd = rsqrtf(m2 / (float)DV + eps);
            unsigned long long* dst = merged_team + ((size_t)(gr % kRingM) * kST + rrow) * 2;
            st_tagged(dst, tagged(mean, tag));
            st_tagged(dst + 1, tagged(rstd, tag));
        }
    }
    __device__ __forceinline__ void merged_issue(int gf, int b) {
        const unsigned long long* src = merged_team + ((size_t)(gf % kRingM) * kST + mrow) * 2;
        const unsigned long long w0 = ld_tagged(src), w1 = ld_tagged(src + 1);
        if (b) { mrg_b[0] = w0; mrg_b[1] = w1; } else { mrg_a[0] = w0; mrg_a[1] = w1; }
    }
    __device__ __forceinline__ void finalize(f32x4 a, int gf, int b) {
        const unsigned tag = (unsigned)gf + 1u;
        unsigned long long w0 = b ? mrg_b[0] : mrg_a[0], w1 = b ? mrg_b[1] : mrg_a[1];
        if ((unsigned)(w0 >> 32) != tag || (unsigned)(w1 >> 32) != tag) {
            const unsigned long long* src = merged_team + ((size_t)(gf % kRingM) * kST + mrow) * 2;
            unsigned spins = 0;
            do {
                __builtin_amdgcn_s_sleep(1);
                w0 = ld_tagged(src);
                w1 = ld_tagged(src + 1);
                if (++spins > kSpinLimit) { atomicOr(err_flag, 1u); break; }
            } while ((unsigned)(w0 >> 32) != tag || (unsigned)(w1 >> 32) != tag);
        }
        const float mean_l = untag(w0), rstd_l = untag(w1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mean = __shfl(mean_l, 16 * g4 + i, 64), rstd = __shfl(rstd_l, 16 * g4 + i, 64);
            a[i] = (a[i] - mean) * rstd * gw + gb;
        }
        store_tile(a, gf);
    }
    // Step g (a pipeline stage, or a drain step after the last one), with the output-tile ring pend
    // (pend[k] = tile of stage g-1-k).
    __device__ __forceinline__ void issue(int g, int b) {
        if (is_reducer(g - kRedLag)) reducer_issue(g - kRedLag);
        const int gm = g - kGnLag + 1;
        if (gm >= 0 && gm < total) merged_issue(gm, b);
    }
    __device__ __forceinline__ void finish(int g, int b, const f32x4 (&pend)[kGnLag]) {
        if (is_reducer(g - kRedLag)) reducer_finish(g - kRedLag);
        const int gf = g - kGnLag;
        if (gf >= 0 && gf < total) finalize(pend[kGnLag - 1], gf, b ^ 1);
    }
};

// ---------------------------------------------------------------------------------------------
// Warp-specialised chunk kernel (chunks up to 256): 512 threads = 4 output waves + 4 state waves,
// one of each per SIMD, so that loads, LDS traffic and matrix-core work of the two overlap.
//   state waves  (w = 4..7): prefetch each 32-token stage's Q, K, V and P rows into registers two
//                stages ahead, store stage g+1 into the idle LDS buffer while stage g is computed,
//                split V (.) zeta into bf16 hi + lo, and accumulate R += K^T (V (.) zeta) for their
//                d_k quarter of R (fp32, scaled by g^L at each chunk start).
//   output waves (w = 0..3): per stage, the 16 x 16 tile (rows 16*(w>>1), columns 16*(w&1)) of
//                g^(j+1) Q R + P V, with R^T (hi + lo) held in registers for the chunk, then the
//                GroupNorm exchange and the store.
// At each chunk end the state waves write R as bf16 hi + lo into the Q/K region of the LDS buffer
// that the finished stage used; the output waves read their fragments from it at the next stage.
template <int DK, int C>
struct WsGeom {
    static constexpr int LQ = DK + 8, LK = DK + 16, LP = C + 8, LV = kW + 16, LR = DK + 8;
    static constexpr size_t Q_BYTES = (size_t)kST * LQ * 2;
    static constexpr size_t K_BYTES = (size_t)kST * LK * 2;
    static constexpr size_t P_BYTES = (size_t)kST * LP * 2;
    static constexpr size_t Z_BYTES = (size_t)kST * LV * 2;
    static constexpr size_t BUF = Q_BYTES + K_BYTES + P_BYTES + 2 * Z_BYTES;  // one stage buffer
    // V rows of the chunk, double-buffered by chunk parity: during a chunk's last stage the state
    // waves already store the next chunk's first V rows while the output waves still read these
    static constexpr size_t V_BYTES = (size_t)C * LV * 2;
    static constexpr size_t OFF_V = 2 * BUF;
    static constexpr size_t BYTES = OFF_V + 2 * V_BYTES;
    static constexpr size_t R_BYTES = 2 * (size_t)kW * LR * 2;
    static_assert(R_BYTES <= Q_BYTES + K_BYTES, "R^T must fit in a stage buffer's Q/K region");
    static constexpr int QCH = kST * DK / 8;
    static constexpr int QN = QCH / 256;       // Q (and K) chunks per state thread
    static constexpr int PN = kST * C / 8 / 256;  // P slots per state thread
};

template <int DK, int C>
struct WsRegs {
    bf16x8 q[WsGeom<DK, C>::QN > 0 ? WsGeom<DK, C>::QN : 1];
    bf16x8 k[WsGeom<DK, C>::QN > 0 ? WsGeom<DK, C>::QN : 1];
    bf16x8 p[WsGeom<DK, C>::PN > 0 ? WsGeom<DK, C>::PN : 1];
    bf16x8 v;
};

template <int DK, int C, typename TOUT, bool GN>
__global__ __launch_bounds__(512) void chunk_ws_kernel(MainParams p, HeadConsts hc) {
    using G = WsGeom<DK, C>;
    constexpr int RTR = DK / 64;  // 16-row R tiles per state wave
    constexpr int SPC = C / kST;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto Qb = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<bf16*>(smem + b * G::BUF); };
    auto Kb = [&](int b) __attribute__((always_inline)) { return reinterpret_cast<bf16*>(smem + b * G::BUF + G::Q_BYTES); };
    auto Pb = [&](int b) __attribute__((always_inline)) {
        return reinterpret_cast<bf16*>(smem + b * G::BUF + G::Q_BYTES + G::K_BYTES);
    };
    auto Zh = [&](int b) __attribute__((always_inline)) {
        return reinterpret_cast<bf16*>(smem + b * G::BUF + G::Q_BYTES + G::K_BYTES + G::P_BYTES);
    };
    auto Zl = [&](int b) __attribute__((always_inline)) {
        return reinterpret_cast<bf16*>(smem + b * G::BUF + G::Q_BYTES + G::K_BYTES + G::P_BYTES + G::Z_BYTES);
    };
    auto Vc = [&](int ci) __attribute__((always_inline)) { return reinterpret_cast<bf16*>(smem + G::OFF_V + (ci & 1) * G::V_BYTES); };

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    const bool state_wave = w >= 4;
    const int wl = w & 3;          // wave index within its group
    const int st = threadIdx.x - 256;  // state-group thread index (valid for state waves)
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
    const int N = p.N, DV = p.NS * kW;
    const float l2g = hc.log2g[h];
    const int col0 = slice * kW;
    const int nchunks = p.nchunks;
    const int L_last = N - (nchunks - 1) * C;
    const int total = (nchunks - 1) * SPC + (L_last + kST - 1) / kST;
    const int rt_o = wl >> 1, ct_o = wl & 1;

    const unsigned q_bytes = (unsigned)((size_t)N * DK * 2), v_bytes = (unsigned)((size_t)N * DV * 2);
    const unsigned p_bytes = (unsigned)((size_t)nchunks * C * C * 2);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + (size_t)bh * N * DK), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)bh * N * DK), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)bh * N * DV), 0, v_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc((void*)(p.P + (size_t)bh * nchunks * C * C), 0, p_bytes, 0x00020000);

    // ---- state waves: stage loads and stores
    auto load_stage = [&](WsRegs<DK, C>& r, int g) __attribute__((always_inline)) {
        const int gg = g < total ? g : total - 1;
        const int ci = gg / SPC, s = gg % SPC;
        const int tok0 = ci * C + kST * s;
#pragma unroll
        for (int u = 0; u < G::QN; ++u) {
            const int j = st + 256 * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            const unsigned off = (unsigned)((tok0 + row) * DK + 8 * sg) * 2u;
            r.q[u] = buf_load16(rq, off);
            r.k[u] = buf_load16(rk, off);
        }
        {
            const int row = st >> 2, sg = st & 3;
            const unsigned off = st < kST * 4 ? (unsigned)((tok0 + row) * DV + col0 + 8 * sg) * 2u : v_bytes;
            r.v = buf_load16(rv, off);
        }
        const int per_row = 4 * (s + 1);
        const unsigned base = (unsigned)((ci * C + kST * s) * C);
#pragma unroll
        for (int u = 0; u < G::PN; ++u) {
            const int j = st + 256 * u;
            const int row = j / (C / 8), sg = j % (C / 8);
            const unsigned off = sg < per_row ? (base + (unsigned)(row * C + 8 * sg)) * 2u : p_bytes;
            r.p[u] = buf_load16(rp, off);
        }
    };
    auto store_stage = [&](const WsRegs<DK, C>& r, int g, int b) __attribute__((always_inline)) {
        const int ci = g / SPC, s = g % SPC;
        const int L = min(C, N - ci * C);
        bf16* Qs = Qb(b);
        bf16* Ks = Kb(b);
        bf16* Ps = Pb(b);
#pragma unroll
        for (int u = 0; u < G::QN; ++u) {
            const int j = st + 256 * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            *reinterpret_cast<bf16x8*>(Qs + row * G::LQ + 8 * sg) = r.q[u];
            *reinterpret_cast<bf16x8*>(Ks + row * G::LK + 8 * sg) = r.k[u];
        }
        if (st < kST * 4) {
            const int row = st >> 2, sg = st & 3;
            *reinterpret_cast<bf16x8*>(Vc(ci) + (kST * s + row) * G::LV + 8 * sg) = r.v;
            const int t = kST * s + row;
            const float z = t < L ? decay_pow(l2g, (float)(L - 1 - t)) : 0.f;
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 a, c;
                split_hi_lo((float)r.v[e] * z, a, c);
                hi[e] = a;
                lo[e] = c;
            }
            *reinterpret_cast<bf16x8*>(Zh(b) + row * G::LV + 8 * sg) = hi;
            *reinterpret_cast<bf16x8*>(Zl(b) + row * G::LV + 8 * sg) = lo;
        }
        const int per_row = 4 * (s + 1);
#pragma unroll
        for (int u = 0; u < G::PN; ++u) {
            const int j = st + 256 * u;
            const int row = j / (C / 8), sg = j % (C / 8);
            if (sg < per_row) *reinterpret_cast<bf16x8*>(Ps + row * G::LP + 8 * sg) = r.p[u];
        }
    };

    // Barrier sequence, identical for both roles (each role runs its own loop with its own
    // registers): one after the prologue; per stage g: one at a chunk start (s == 0), one at the
    // end of the stage, and one more after a chunk end that is not the last stage.
    TOUT* out = reinterpret_cast<TOUT*>(p.out);
    if (state_wave) {
        // ---------------- state waves: R rows [wl*DK/4, (wl+1)*DK/4) x 32 columns, fp32
        f32x4 accR[RTR][2];
#pragma unroll
        for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = wl * (DK / 4) + 16 * rt + 4 * g4 + i;
                    accR[rt][ct][i] = p.state_in ? p.state_in[((size_t)bh * DK + row) * DV + col0 + 16 * ct + c16] : 0.f;
                }
        auto write_R = [&](int b) __attribute__((always_inline)) {  // R^T as bf16 hi + lo into buffer b's Q/K region
            bf16* Rhi = Qb(b);
            bf16* Rlo = Qb(b) + kW * G::LR;
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    bf16x4 hi, lo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bf16 a, c;
                        split_hi_lo(accR[rt][ct][i], a, c);
                        hi[i] = a;
                        lo[i] = c;
                    }
                    const int col = 16 * ct + c16, row = wl * (DK / 4) + 16 * rt + 4 * g4;
                    *reinterpret_cast<bf16x4*>(Rhi + col * G::LR + row) = hi;
                    *reinterpret_cast<bf16x4*>(Rlo + col * G::LR + row) = lo;
                }
        };
        auto scale_R = [&](int L) __attribute__((always_inline)) {
            const float gL = decay_pow(l2g, (float)L);
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) accR[rt][ct] *= gL;
        };
        // prologue: stage 0 into buffer 0, R_{-1} into buffer 1's Q/K region, loads for stages 1, 2
        WsRegs<DK, C> r0, r1;  // r0 holds even stages, r1 odd stages
        load_stage(r0, 0);
        load_stage(r1, 1);
        store_stage(r0, 0, 0);
        write_R(1);
        load_stage(r0, 2);
        scale_R(min(C, N));
        __syncthreads();
        auto stage = [&](WsRegs<DK, C>& rn, int g) __attribute__((always_inline)) {  // rn holds stage g+1
            const int b = g & 1, s = g % SPC;
            const bool chunk_end = (s == SPC - 1) || (g == total - 1);
            if (s == 0) __syncthreads();  // the output waves have taken R from buffer b^1
            const bf16* Ks = Kb(b);
            bf16x8 bhi[2], blo[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bhi[ct] = lds_frag_kmajor(Zh(b), G::LV, 0, 16 * ct, lane);
                blo[ct] = lds_frag_kmajor(Zl(b), G::LV, 0, 16 * ct, lane);
            }
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) {
                const bf16x8 ak = lds_frag_kmajor(Ks, G::LK, 0, wl * (DK / 4) + 16 * rt, lane);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    accR[rt][ct] = mfma16(ak, bhi[ct], accR[rt][ct]);
                    accR[rt][ct] = mfma16(ak, blo[ct], accR[rt][ct]);
                }
            }
            if (g + 1 < total) {  // stage g+1 into the idle buffer, then loads for stage g+3
                store_stage(rn, g + 1, b ^ 1);
                load_stage(rn, g + 3);
            }
            __syncthreads();  // stage g consumed; stage g+1 stored
            if (chunk_end && g + 1 < total) {
                write_R(b);  // R of this chunk into buffer b's (now idle) Q/K region
                scale_R(min(C, N - ((g + 1) / SPC) * C));
                __syncthreads();
            }
        };
        for (int g = 0; g < total; g += 2) {
            stage(r1, g);
            if (g + 1 < total) stage(r0, g + 1);
        }
        if (p.state_out) {
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = wl * (DK / 4) + 16 * rt + 4 * g4 + i;
                        p.state_out[((size_t)bh * DK + row) * DV + col0 + 16 * ct + c16] = accR[rt][ct][i];
                    }
        }
    } else {
        // ---------------- output waves: 16 x 16 tile of each stage
        bf16x8 rfh[DK / 32], rfl[DK / 32];
        GnExchange<TOUT> gx;
        f32x4 pend[kGnLag];
        if constexpr (GN) gx.init(p, bh, h, slice, wl, lane, total, SPC, C);
#pragma unroll
        for (int k = 0; k < kGnLag; ++k) pend[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto store_plain = [&](f32x4 a, int g) __attribute__((always_inline)) {
            const int c0 = (g / SPC) * C, s = g % SPC;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = c0 + kST * s + 16 * rt_o + 4 * g4 + i;
                if (r < N) out[((size_t)bh * N + r) * DV + col0 + 16 * ct_o + c16] = from_float<TOUT>(a[i]);
            }
        };
        __syncthreads();
        for (int g = 0; g < total; ++g) {
            const int b = g & 1, s = g % SPC;
            const bool chunk_end = (s == SPC - 1) || (g == total - 1);
            if (s == 0) {
                // R of the previous chunk sits in buffer b^1's Q/K region until the barrier
                const bf16* Rhi = Qb(b ^ 1);
                const bf16* Rlo = Qb(b ^ 1) + kW * G::LR;
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    rfh[ks] = frag_rowmajor(Rhi, G::LR, 16 * ct_o, 32 * ks, lane);
                    rfl[ks] = frag_rowmajor(Rlo, G::LR, 16 * ct_o, 32 * ks, lane);
                }
                __syncthreads();
            }
            if constexpr (GN) gx.issue(g, g & 1);
            const bf16* Qs = Qb(b);
            const bf16* Ps = Pb(b);
            f32x4 qa[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) qa[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const bf16x8 a = frag_rowmajor(Qs, G::LQ, 16 * rt_o, 32 * ks, lane);
                qa[2 * (ks & 1)] = mfma16(a, rfh[ks], qa[2 * (ks & 1)]);
                qa[2 * (ks & 1) + 1] = mfma16(a, rfl[ks], qa[2 * (ks & 1) + 1]);
            }
            const f32x4 qr = (qa[0] + qa[2]) + (qa[1] + qa[3]);
            f32x4 pv = {0.f, 0.f, 0.f, 0.f};
            const bf16* Vs = Vc(g / SPC);
            for (int ks = 0; ks <= s; ++ks) {
                const bf16x8 a = frag_rowmajor(Ps, G::LP, 16 * rt_o, 32 * ks, lane);
                const bf16x8 bv = lds_frag_kmajor(Vs, G::LV, 32 * ks, 16 * ct_o, lane);
                pv = mfma16(a, bv, pv);
            }
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = qr[i] * decay_pow(l2g, (float)(kST * s + 16 * rt_o + 4 * g4 + i + 1)) + pv[i];
            if constexpr (GN) {
                gx.publish(acc, g);
                gx.finish(g, g & 1, pend);
#pragma unroll
                for (int k = kGnLag - 1; k > 0; --k) pend[k] = pend[k - 1];
                pend[0] = acc;
            } else {
                store_plain(acc, g);
            }
            __syncthreads();  // stage g consumed; stage g+1 stored
            if (chunk_end && g + 1 < total) __syncthreads();  // R of this chunk written
        }
        if constexpr (GN) {
            for (int g = total; g < total + kGnLag; ++g) {
                gx.issue(g, g & 1);
                gx.finish(g, g & 1, pend);
#pragma unroll
                for (int k = kGnLag - 1; k > 0; --k) pend[k] = pend[k - 1];
            }
        }
    }
}

__global__ void zero_words_kernel(unsigned* p, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// ---------------------------------------------------------------------------------------------
// Workspace layout (bytes, each part 256-aligned):
//   P         B*H*nchunks*C*C bf16                  (only when the output is wanted)
//   flag      one uint32 error flag                 (only with GroupNorm)
//   partials  B*H*kRingP*(2*NS)*32 x 2 uint64       (only with GroupNorm)
//   merged    B*H*kRingM*32 x 2 uint64              (only with GroupNorm)
struct WsLayout {
    size_t p_off, p_bytes, flag_off, part_off, part_bytes, mrg_off, mrg_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int B, int H, int N, int DV, int C, int gn, int want_out) {
    WsLayout l{};
    const size_t nchunks = (size_t)(N + C - 1) / C;
    l.p_off = 0;
    l.p_bytes = want_out ? align256((size_t)B * H * nchunks * C * C * sizeof(bf16)) : 0;
    l.flag_off = l.p_off + l.p_bytes;
    const size_t flag_bytes = gn ? 256 : 0;
    l.part_off = l.flag_off + flag_bytes;
    l.part_bytes = gn ? align256((size_t)B * H * kRingP * (2 * (DV / kW)) * kST * 2 * sizeof(unsigned long long)) : 0;
    l.mrg_off = l.part_off + l.part_bytes;
    l.mrg_bytes = gn ? align256((size_t)B * H * kRingM * kST * 2 * sizeof(unsigned long long)) : 0;
    l.total = l.mrg_off + l.mrg_bytes;
    return l;
}

// Chunks up to 256 with an output use the warp-specialised kernel; 512-token chunks (whose stage
// buffers do not fit twice in LDS) and state-only prefills use the single-group kernel.
template <int DK, int C, bool WANT_OUT>
constexpr bool use_ws() { return WANT_OUT && C <= 256; }

template <int DK, int C, typename TOUT, bool GN, bool WANT_OUT>
const void* main_kernel_ptr() {
    if constexpr (use_ws<DK, C, WANT_OUT>()) return reinterpret_cast<const void*>(chunk_ws_kernel<DK, C, TOUT, GN>);
    else return reinterpret_cast<const void*>(chunk_main_kernel<DK, C, TOUT, GN, WANT_OUT>);
}

template <int DK, int C, typename TOUT, bool GN, bool WANT_OUT>
hipError_t launch_main(const LaunchArgs& a, MainParams mp) {
    constexpr bool ws = use_ws<DK, C, WANT_OUT>();
    const void* kern = main_kernel_ptr<DK, C, TOUT, GN, WANT_OUT>();
    const size_t dyn = ws ? WsGeom<DK, C>::BYTES : MainGeom<DK, C>::BYTES;
    const int threads = ws ? 512 : kThreads;
    const int teams = a.B * a.H;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    if (!GN) {
        mp.team_base = 0;
        mp.nteams_launch = teams;
        HeadConsts hc = a.hc;
        void* args[] = {&mp, &hc};
        return hipLaunchKernel(kern, dim3(teams * mp.NS), dim3(threads), args, dyn, a.stream);
    }
    // GroupNorm: the slices of a head wait for each other's statistics, so they must be
    // co-resident. Launch cooperatively, in batches of whole teams that fit on the device at once.
    int dev = 0, ncu = 0, per_cu = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, dyn);
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
        e = hipLaunchCooperativeKernel(kern, dim3(lp.nteams_launch * mp.NS), dim3(threads), args, (unsigned)dyn, a.stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int C, typename TOUT>
hipError_t launch_dk_c(const LaunchArgs& a) {
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
        mp.err_flag = reinterpret_cast<unsigned*>(ws + l.flag_off);
        mp.part = reinterpret_cast<unsigned long long*>(ws + l.part_off);
        mp.merged = reinterpret_cast<unsigned long long*>(ws + l.mrg_off);
        // tags must not match anything left by an earlier call: clear flag, partials and merged
        const size_t nwords = (l.total - l.flag_off) / sizeof(unsigned);
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((nwords + 1023) / 1024 < 2048 ? (nwords + 1023) / 1024 : 2048)),
                           dim3(256), 0, a.stream, mp.err_flag, nwords);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (want_out) {
        hipLaunchKernelGGL(chunk_scores_kernel<DK>, dim3(C / 64, nchunks, a.B * a.H), dim3(kThreads), 0, a.stream, a.H, a.N, C,
                           nchunks, mp.q, mp.k, const_cast<bf16*>(mp.P), a.hc);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.gn.enabled) return launch_main<DK, C, TOUT, true, true>(a, mp);
        return launch_main<DK, C, TOUT, false, true>(a, mp);
    }
    return launch_main<DK, C, TOUT, false, false>(a, mp);
}

template <int DK, typename TOUT>
hipError_t launch_dk(const LaunchArgs& a) {
    switch (a.chunk) {
        case 64: return launch_dk_c<DK, 64, TOUT>(a);
        case 128: return launch_dk_c<DK, 128, TOUT>(a);
        case 256: return launch_dk_c<DK, 256, TOUT>(a);
        default: return launch_dk_c<DK, 512, TOUT>(a);
    }
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

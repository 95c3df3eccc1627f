// Chunkwise recurrent retention, bf16 inputs, fp32 accumulation, on the gfx950 matrix cores.
//
// Method (abeam.tech RetNet summary, "Chunk recursion for long-sequence training"; mlnews.online
// RetNet abstract: chunks encoded in parallel, summarised recurrently). Unrolling the recurrence
// S_n = g S_(n-1) + k_n^T v_n over one chunk of length L with carried state R gives, for local row j,
//     o_j = [(Q K^T (.) D) V]_j + g^(j+1) [Q R]_j,      D[j][t] = g^(j-t) for t <= j
//     R  <- g^L R + K^T (V (.) zeta),                    zeta_t = g^(L-1-t)
//
// Kernels:
//   chunk_scores_kernel   parallel over (chunk, b*h): P = (Q K^T) (.) D on MFMA with the decay and
//                         causal mask applied in registers, stored in the workspace as bf16 hi and,
//                         in a second plane, lo = P - hi rounded (32-key blocks on and below the
//                         diagonal). A single bf16 P moves the output by about 1e-2 of its RMS.
//   chunk_ws_kernel       (chunks up to 256 whose stage buffers fit, output wanted) one workgroup
//                         per (b, h, 32-column slice of d_v), walking the sequence in 32-token
//                         stages, with loader waves, state waves and output waves (see the kernel):
//                           out  = g^(j+1) Q R + P V      (R of the previous chunk and P as bf16
//                                                         hi + lo)
//                           R   += K^T (V (.) zeta)       (V (.) zeta as bf16 hi + lo; R fp32 in
//                                                         accumulators, scaled by g^L at chunk start)
//   chunk_main_kernel     the same per stage with every wave doing both parts (512-token chunks,
//                         and state-only calls that read their operands in place, which have no
//                         output part).
//   gn_rows_kernel        the optional per-head GroupNorm over d_v, on fp32 pre-norm rows that the
//                         chunk kernel writes to the workspace.
// The d_v slices of one head sit on one XCD to share its L2. Plain calls whose (b, h, slice)
// workgroups would leave compute units idle run on the segmented kernels of chunk_seg.hip instead.
#include <algorithm>

#include "common.hpp"

namespace ret {
namespace {

constexpr int kThreads = 256;
constexpr int kW = 32;     // d_v columns per workgroup
constexpr int kST = 32;    // tokens per pipeline stage

// ---------------------------------------------------------------------------------------------
// P = (Q K^T) (.) D for every chunk, into the workspace as [B*H][nchunks][C][C] bf16, its high
// part in P and, when Plo is given, the low part (P - hi, rounded) in Plo, same layout. With qlo
// (the low part of a q that bf16 does not hold) Q K^T is q K^T + qlo K^T, each in fp32. With Pa
// (no qlo) the kernel also writes the scores anti-transposed, P'[C-1-m][C-1-r] = P[r][m], for chunk
// nchunks-1-c at Pa (high parts, then the low parts one plane of P further): these are the scores
// of the time-reversed walk with the roles of q and k exchanged, when N is a multiple of C. Grid
// (nchunks, B*H), 256 threads. The MFMAs compute P^T = K Q^T per 16 x 16 tile so that each lane
// ends with 4 consecutive keys of one row (one 8-byte store). K rows go through LDS in 128-key
// blocks (buffer-to-LDS loads, swizzled rows); each wave reads the Q fragments of its row tile
// straight from global memory into registers. Row tile t (16 rows) gets key tiles 0 .. (t|1): the
// consumer reads whole 32-key steps up to the diagonal one, whose upper part is written as zero.
// Waves take row tiles in mirrored pairs (t, T-1-t) so that the causal work is balanced.
// KLO: k comes as two parts too (k + klo), and Q K^T = q K^T + qlo K^T + q Klo^T (the qlo Klo^T
// term, about 2^-16 relative, dropped): the K and Klo blocks of 64 keys sit side by side in LDS.
// ROT (with KLO, plain operand addressing): q and k come unrotated, and the kernel applies the
// positional rotation itself (abeam.tech RetNet summary, "Technical mechanism": Q and K are turned
// after the projections), split into bf16 high and low parts, which the scores use as above and
// which are also written out (rf.qh, rf.ql, rf.kh, rf.kl, [B*H][N][DK]) for the chunk passes that
// follow. First the chunk's q rows pass through the K blocks' LDS, 128 rows at a time, are turned
// and written out; the Q fragments are then read back from there. Each K block is turned in LDS
// after its load. Each thread turns one 16-byte piece (4 pairs) of consecutive rows: sin and cos
// at the first row and of the one-position step, then angle addition (as the rotation pass does;
// about one rounding per step).
struct RotFuse {
    bf16 *qh, *ql, *kh, *kl;
    RotConsts rc;
};

// Turns piece c (features 8c .. 8c+7, pairs 4c .. 4c+3) of rows r0 .. r0+nr-1 of a block in LDS
// (rows of QRB bytes, swizzled as SwzTile<QRB>) holding sequence positions pos0 + r: high and low
// parts to hi_at / lo_at (LDS; lo_at null: not kept) and, for positions below N, to the planes
// gh / gl (row pos of [N][DK] at this head).
template <int QRB>
__device__ __forceinline__ void turn_rows(char* blk, char* hi_at, char* lo_at, int c, int r0, int nr, int pos0, int N,
                                          const RotConsts& rc, bf16* gh, bf16* gl) {
    constexpr int DK = QRB / 2;
    float sn[4], cn[4], ss[4], cs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = 4 * c + j;
        rot_sincos(pos0 + r0, rc.fhi[i], rc.flo[i], rc.ph[i], sn[j], cn[j]);
        sincospif(rc.fhi[i] + rc.flo[i], &ss[j], &cs[j]);
    }
    for (int rr = 0; rr < nr; ++rr) {
        const int r = r0 + rr, pos = pos0 + r;
        const int byte = r * QRB + 16 * (c ^ (r & SwzTile<QRB>::M));
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(blk + byte);
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = (float)x[2 * j], b = (float)x[2 * j + 1];
            bf16 h, l;
            split_hi_lo(a * cn[j] - b * sn[j], h, l);
            hi[2 * j] = h;
            lo[2 * j] = l;
            split_hi_lo(a * sn[j] + b * cn[j], h, l);
            hi[2 * j + 1] = h;
            lo[2 * j + 1] = l;
            const float c2 = cn[j] * cs[j] - sn[j] * ss[j];
            sn[j] = sn[j] * cs[j] + cn[j] * ss[j];
            cn[j] = c2;
        }
        if (hi_at) *reinterpret_cast<bf16x8*>(hi_at + byte) = hi;
        if (lo_at) *reinterpret_cast<bf16x8*>(lo_at + byte) = lo;
        if (pos < N) {
            *reinterpret_cast<bf16x8*>(gh + (size_t)pos * DK + 8 * c) = hi;
            *reinterpret_cast<bf16x8*>(gl + (size_t)pos * DK + 8 * c) = lo;
        }
    }
}

template <int DK, bool KLO = false, bool ROT = false>
__global__ __launch_bounds__(256) void chunk_scores_kernel(int H, int N, int C, int nchunks, const bf16* __restrict__ q,
                                                           const bf16* __restrict__ qlo, const bf16* __restrict__ k,
                                                           const bf16* __restrict__ klo, bf16* __restrict__ P,
                                                           bf16* __restrict__ Plo, bf16* __restrict__ Pa, HeadConsts hc, int rev,
                                                           int ldqk, int qcol_blk, int srcBH, typename IfRot<ROT, RotFuse>::type rf) {
    static_assert(!ROT || KLO, "the rotated scores use both parts of k");
    constexpr int KB = KLO ? 64 : 128;  // keys per LDS block
    constexpr int QRB = DK * 2;   // bytes per K row
    constexpr int NKB = KB * QRB / 1024;  // kilobytes of a K block
    __shared__ __attribute__((aligned(1024))) char Ks[(KLO ? 2 : 1) * KB * QRB];
    const int chunk = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    const int c0 = chunk * C;
    const float l2g = hc.log2g[h];
    // rows of this head's q and k (in place: stride ldqk, a column block, reversed); rows past the
    // sequence fall outside the resource and read as zero
    const unsigned q_bytes = (unsigned)(((size_t)(N - 1) * ldqk + DK) * 2);
    const size_t qbase = (size_t)(bh % srcBH) * N * ldqk + (size_t)(bh / srcBH) * qcol_blk;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + qbase), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + qbase), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rql = __builtin_amdgcn_make_buffer_rsrc((void*)((qlo ? qlo : q) + qbase), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rkl = __builtin_amdgcn_make_buffer_rsrc((void*)((KLO && !ROT ? klo : k) + qbase), 0, q_bytes, 0x00020000);
    auto row_of = [&](int t) __attribute__((always_inline)) { return rev ? N - 1 - t : t; };
    bf16* Pc = P + ((size_t)bh * nchunks + chunk) * (size_t)C * C;
    bf16* Plc = Plo ? Plo + ((size_t)bh * nchunks + chunk) * (size_t)C * C : nullptr;
    // the anti-transposed scores (both parts), chunk nchunks-1-chunk of the time-reversed walk
    bf16* Pac = Pa ? Pa + ((size_t)bh * nchunks + (nchunks - 1 - chunk)) * (size_t)C * C : nullptr;
    bf16* Palc = Pa ? Pac + (size_t)gridDim.y * nchunks * C * C : nullptr;
    const int T = C / 16;  // row tiles of the chunk
    constexpr int UPR = QRB / 16;  // 16-byte pieces per row
    if constexpr (ROT) {
        // the chunk's q rows, 2 KB at a time through the K blocks' LDS, turned and written out
        for (int rb = 0; rb < C; rb += 2 * KB) {
            const int rows = min(2 * KB, C - rb);
            if (rb > 0) __syncthreads();
            for (int j = w; j < rows * QRB / 1024; j += 4) {
                const int byte = 1024 * j + 16 * lane, r = byte / QRB;
                const int c = ((byte % QRB) >> 4) ^ (r & SwzTile<QRB>::M);
                const unsigned off = (unsigned)(((c0 + rb + r) * DK + 8 * c) * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(Ks + 1024 * j), 16, off, 0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            __syncthreads();
            const int rpt = rows * UPR / 256;
            turn_rows<QRB>(Ks, nullptr, nullptr, threadIdx.x % UPR, (threadIdx.x / UPR) * rpt, rpt, c0 + rb, N, rf.rc,
                           rf.qh + (size_t)bh * N * DK, rf.ql + (size_t)bh * N * DK);
        }
        __syncthreads();  // the q rows are read and written out
    }
    // ROT: the turned q rows, as written out (rows past the sequence read as zero)
    const bf16 *qp = q, *qlp = q;
    if constexpr (ROT) {
        qp = rf.qh + (size_t)bh * N * DK;
        qlp = rf.ql + (size_t)bh * N * DK;
    }
    const __amdgpu_buffer_rsrc_t rqh = __builtin_amdgcn_make_buffer_rsrc((void*)qp, 0, (unsigned)((size_t)N * DK * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rqhl = __builtin_amdgcn_make_buffer_rsrc((void*)qlp, 0, (unsigned)((size_t)N * DK * 2), 0x00020000);

    for (int kb0 = 0; kb0 < C; kb0 += KB) {
        // K rows kb0 .. kb0+KB-1 of the chunk (rows past the sequence read as zero)
        if (kb0 > 0) __syncthreads();  // the previous block's reads are done
        for (int j = w; j < NKB; j += 4) {
            const int byte = 1024 * j + 16 * lane, r = byte / QRB;
            const int c = ((byte % QRB) >> 4) ^ (r & SwzTile<QRB>::M);
            const unsigned off = (unsigned)((row_of(c0 + kb0 + r) * ldqk + 8 * c) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Ks + 1024 * j), 16, off, 0, 0, 0);
            if constexpr (KLO && !ROT)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rkl, (__attribute__((address_space(3))) void*)(Ks + KB * QRB + 1024 * j), 16, off,
                                                         0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if constexpr (ROT) {
            // the K block turned in place (high part), its low part into the Klo block
            constexpr int RPT = KB * UPR / 256;
            turn_rows<QRB>(Ks, Ks, Ks + KB * QRB, threadIdx.x % UPR, (threadIdx.x / UPR) * RPT, RPT, c0 + kb0, N, rf.rc,
                           rf.kh + (size_t)bh * N * DK, rf.kl + (size_t)bh * N * DK);
            __syncthreads();
        }
        for (int m = 0; m < T / 4; ++m) {
            const int t = (m & 1) ? 4 * m + 3 - w : 4 * m + w;  // mirrored within each group of 8
            const int last = min((t | 1), (kb0 + KB) / 16 - 1);  // last key tile of this block
            if (last * 16 < kb0) continue;
            bf16x8 qf[DK / 32];
            bf16x8 qlf[DK / 32];
            if constexpr (ROT) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const unsigned off = (unsigned)(((c0 + 16 * t + c16) * DK + 32 * ks + 8 * g4) * 2);
                    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rqh, off, 0, 0));
                    qlf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rqhl, off, 0, 0));
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const unsigned off = (unsigned)((row_of(c0 + 16 * t + c16) * ldqk + 32 * ks + 8 * g4) * 2);
                    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
                }
            }
            if (!ROT && qlo) {
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const unsigned off = (unsigned)((row_of(c0 + 16 * t + c16) * ldqk + 32 * ks + 8 * g4) * 2);
                    qlf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rql, off, 0, 0));
                }
            }
            for (int kt = kb0 / 16; kt <= last; ++kt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc_t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    const bf16x8 kf = frag_rowmajor_swz<QRB>(Ks, 16 * kt - kb0, 32 * ks, lane);
                    acc = mfma16(kf, qf[ks], acc);
                    // the same tile untransposed (the two operands' lane layouts coincide): lane
                    // holds rows 16t + 4g4 + i of key 16kt + c16
                    if (Pa) acc_t = mfma16(qf[ks], kf, acc_t);
                }
                if (Pa) {
                    // anti-transposed: element (row r, key m) at (C-1-m, C-1-r), so this lane's four
                    // rows are four consecutive columns, in reverse order
                    const int m = 16 * kt + c16, r0 = 16 * t + 4 * g4;
                    bf16x4 o, ol;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bf16 hi, lo;
                        split_hi_lo(r0 + i >= m ? acc_t[i] * decay_pow(l2g, (float)(r0 + i - m)) : 0.f, hi, lo);
                        o[3 - i] = hi;
                        ol[3 - i] = lo;
                    }
                    const size_t at = (size_t)(C - 1 - m) * C + (C - 4 - r0);
                    *reinterpret_cast<bf16x4*>(Pac + at) = o;
                    *reinterpret_cast<bf16x4*>(Palc + at) = ol;
                }
                if (qlo || KLO) {
                    f32x4 al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < DK / 32; ++ks) {
                        if (ROT || qlo) al = mfma16(frag_rowmajor_swz<QRB>(Ks, 16 * kt - kb0, 32 * ks, lane), qlf[ks], al);
                        if constexpr (KLO) al = mfma16(frag_rowmajor_swz<QRB>(Ks + KB * QRB, 16 * kt - kb0, 32 * ks, lane), qf[ks], al);
                    }
                    acc += al;
                }
                // lane: row 16t + c16, keys 16kt + 4g4 + i
                const int row = 16 * t + c16;
                bf16x4 o, ol;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g4 + i;
                    bf16 hi, lo;
                    split_hi_lo(row >= key ? acc[i] * decay_pow(l2g, (float)(row - key)) : 0.f, hi, lo);
                    o[i] = hi;
                    ol[i] = lo;
                }
                *reinterpret_cast<bf16x4*>(Pc + (size_t)row * C + 16 * kt + 4 * g4) = o;
                if (Plc) *reinterpret_cast<bf16x4*>(Plc + (size_t)row * C + 16 * kt + 4 * g4) = ol;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// The buffer resource of the value rows of one stage (VShift): the prefix buffer of head src when
// pre, else v of head src. Built from selected scalars, so that it stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t value_rsrc(bool pre, const bf16* v, const bf16* vpre, int src, int N, int vsplit,
                                                             int DV) {
    const bf16* base = pre ? vpre + (size_t)src * vsplit * DV : v + (size_t)src * N * DV;
    const unsigned bytes = (unsigned)((size_t)(pre ? vsplit : N) * DV * 2);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, 0x00020000);
}

struct MainParams {
    int H, N, C, NS, nchunks, teams;
    int rev, ldqk, qcol_blk, srcBH;  // operand addressing (OpAddr, defaults resolved)
    int out_acc;                     // fp32 out added atomically to the rows of head bh % srcBH
    int vsplit, vshift;              // value rows through VShift (vsplit = 0: plain)
    const bf16* q;
    const bf16* qlo;  // low part of q (same addressing), added to Q R and to the scores; or null
    const bf16* k;
    const bf16* v;
    const bf16* vpre;
    const bf16* P;
    const bf16* Plo;  // low part of P (same layout), when the kernel uses it
    const float* state_in;
    float* state_out;
    void* out;
};

template <int DK, int C, bool PLO = false>
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
    static constexpr size_t OFF_PL = OFF_P + (size_t)kST * LP * 2;                // P low part (PLO)
    static constexpr size_t OFF_V = OFF_PL + (PLO ? (size_t)kST * LP * 2 : 0);
    static constexpr size_t V_END = OFF_V + (size_t)C * LV * 2;
    static constexpr size_t R_BYTES = (size_t)kW * LR * 2;  // R^T, one part
    static constexpr size_t Z_BYTES = (size_t)kST * LV * 2;
    // R^T (hi, lo) is written at a chunk end and read at the next chunk's first stage, before the
    // second stage stores V rows 32.. of the chunk: where the separate layout does not fit in LDS it
    // lives in those rows
    static constexpr bool R_IN_V =
        V_END + 2 * R_BYTES + 2 * Z_BYTES > 160 * 1024 && (size_t)(C - kST) * LV * 2 >= 2 * R_BYTES;
    static constexpr size_t OFF_RH = R_IN_V ? OFF_V + (size_t)kST * LV * 2 : V_END;
    static constexpr size_t OFF_RL = OFF_RH + R_BYTES;
    static constexpr size_t OFF_ZH = R_IN_V ? V_END : OFF_RL + R_BYTES;  // V (.) zeta, bf16 high part, this stage
    static constexpr size_t OFF_ZL = OFF_ZH + (size_t)kST * LV * 2;  // ... low part
    static constexpr size_t BYTES = OFF_ZL + (size_t)kST * LV * 2;
};

template <int DK, int C, bool PLO>
struct StageRegs {
    bf16x8 q[MainGeom<DK, C>::QN];
    bf16x8 k[MainGeom<DK, C>::QN];
    bf16x8 p[MainGeom<DK, C>::PN > 0 ? MainGeom<DK, C>::PN : 1];
    bf16x8 pl[PLO && MainGeom<DK, C>::PN > 0 ? MainGeom<DK, C>::PN : 1];
    bf16x8 v;
};

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Team and slice of this workgroup. Workgroup i runs on XCD i % 8: with a multiple of 8 teams,
// all slices of a team share i % 8 and therefore one L2.
__device__ __forceinline__ void team_slice(int teams, int NS, int& team, int& slice) {
    const int i = blockIdx.x;
    if (teams % 8 == 0) {
        team = (i % 8) + 8 * (i / (8 * NS));
        slice = (i / 8) % NS;
    } else {
        team = i / NS;
        slice = i % NS;
    }
}

// One (b, h, d_v slice) per workgroup. Wave w owns R rows [w*DK/4, (w+1)*DK/4) (state update) and,
// in every 32-token stage, the 16 x 16 output tile (rows 16*(w>>1), columns 16*(w&1)).
// VSH: value rows through VShift (residual linear attention); the plain instantiation has none of it.
// PLO: P arrives as bf16 hi + lo (P V runs on both parts).
template <int DK, int C, typename TOUT, bool WANT_OUT, bool VSH, bool PLO>
__global__ __launch_bounds__(kThreads) void chunk_main_kernel(MainParams p, HeadConsts hc) {
    using G = MainGeom<DK, C, PLO>;
    constexpr int RTR = DK / 64;  // 16-row R tiles per wave
    constexpr int SPC = C / kST;  // stages per full chunk
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* Qs = reinterpret_cast<bf16*>(smem + G::OFF_Q);
    bf16* Ks = reinterpret_cast<bf16*>(smem + G::OFF_K);
    bf16* Ps = reinterpret_cast<bf16*>(smem + G::OFF_P);
    bf16* Pls = reinterpret_cast<bf16*>(smem + G::OFF_PL);
    bf16* Vs = reinterpret_cast<bf16*>(smem + G::OFF_V);
    bf16* Rhi = reinterpret_cast<bf16*>(smem + G::OFF_RH);
    bf16* Rlo = reinterpret_cast<bf16*>(smem + G::OFF_RL);
    bf16* VZh = reinterpret_cast<bf16*>(smem + G::OFF_ZH);
    bf16* VZl = reinterpret_cast<bf16*>(smem + G::OFF_ZL);

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    int bh, slice;
    team_slice(p.teams, p.NS, bh, slice);
    const int h = bh % p.H;
    const int N = p.N, DV = p.NS * kW;
    const float l2g = hc.log2g[h];
    const int col0 = slice * kW;
    const int nchunks = p.nchunks;
    const int L_last = N - (nchunks - 1) * C;
    const int total = (nchunks - 1) * SPC + (L_last + kST - 1) / kST;
    const int rt_o = w >> 1, ct_o = w & 1;  // output tile of this wave within a stage

    // Buffer resources: loads past the end of a head's data return zero (tail rows, padding). q, k
    // and v of source head bh % srcBH (q and k: rows ldqk apart, from a column block; all rows in
    // reverse with rev).
    const int ldqk = p.ldqk, src = bh % p.srcBH;
    auto row_of = [&](int t) __attribute__((always_inline)) { return p.rev ? N - 1 - t : t; };
    const unsigned q_bytes = (unsigned)(((size_t)(N - 1) * ldqk + DK) * 2), v_bytes = (unsigned)((size_t)N * DV * 2);
    const size_t qbase = (size_t)src * N * ldqk + (size_t)(bh / p.srcBH) * p.qcol_blk;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qbase), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + qbase), 0, q_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)src * N * DV), 0, v_bytes, 0x00020000);
    // value rows below vsplit come from the prefix buffer, the others from v shifted by vshift rows;
    // a stage lies wholly on one side
    const unsigned vp_bytes = (unsigned)((size_t)p.vsplit * DV * 2);
    const unsigned p_bytes = WANT_OUT ? (unsigned)((size_t)nchunks * C * C * 2) : 0u;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(WANT_OUT ? p.P + (size_t)bh * nchunks * C * C : p.q), 0, p_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rpl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(WANT_OUT && PLO ? p.Plo + (size_t)bh * nchunks * C * C : p.q), 0, PLO ? p_bytes : 0u, 0x00020000);

    // ---- stage loads: global -> registers (unconditional instructions), registers -> LDS
    auto load_stage = [&](StageRegs<DK, C, PLO>& r, int g) __attribute__((always_inline)) {
        const int gg = g < total ? g : total - 1;  // past the end: reload the last stage (unused)
        const int ci = gg / SPC, s = gg % SPC;
        const int tok0 = ci * C + kST * s;
#pragma unroll
        for (int u = 0; u < G::QN; ++u) {
            const int j = threadIdx.x + kThreads * u;
            const int row = j / (DK / 8), sg = j % (DK / 8);
            const unsigned off = j < G::QCH ? (unsigned)((row_of(tok0 + row) * ldqk + 8 * sg) * 2) : q_bytes;
            if constexpr (WANT_OUT) r.q[u] = buf_load16(rq, off);
            r.k[u] = buf_load16(rk, off);
        }
        {
            const int row = threadIdx.x >> 2, sg = threadIdx.x & 3;  // 32 rows x 4 chunks of 8 columns
            if constexpr (VSH) {
                const bool pre = __builtin_amdgcn_readfirstlane((int)(tok0 < p.vsplit)) != 0;  // wave-uniform: a scalar resource
                const int t = tok0 + row, vr = pre ? t : row_of(t) - p.vshift;
                const unsigned off = threadIdx.x < kST * 4 && t < N ? (unsigned)((vr * DV + col0 + 8 * sg) * 2) : (pre ? vp_bytes : v_bytes);
                r.v = buf_load16(value_rsrc(pre, p.v, p.vpre, src, N, p.vsplit, DV), off);
            } else {
                const unsigned off = threadIdx.x < kST * 4 ? (unsigned)((row_of(tok0 + row) * DV + col0 + 8 * sg) * 2) : v_bytes;
                r.v = buf_load16(rv, off);
            }
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
                if constexpr (PLO) r.pl[u] = buf_load16(rpl, off);
            }
        }
    };
    auto store_stage = [&](const StageRegs<DK, C, PLO>& r, int s, int L) __attribute__((always_inline)) {
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
                if (sg < per_row) {
                    *reinterpret_cast<bf16x8*>(Ps + row * G::LP + 8 * sg) = r.p[u];
                    if constexpr (PLO) *reinterpret_cast<bf16x8*>(Pls + row * G::LP + 8 * sg) = r.pl[u];
                }
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
    const int obh = p.out_acc ? bh % p.srcBH : bh;  // output head
    auto store_tile = [&](const f32x4& a, int g) __attribute__((always_inline)) {
        const int ci = g / SPC, s = g % SPC, c0 = ci * C;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = c0 + kST * s + 16 * rt_o + 4 * g4 + i;
            if (r >= N) continue;
            TOUT* o = out + ((size_t)obh * N + row_of(r)) * DV + col0 + 16 * ct_o + c16;
            if constexpr (sizeof(TOUT) == 4) {
                if (p.out_acc)
                    __builtin_amdgcn_global_atomic_fadd_f32(o, a[i]);
                else
                    *o = a[i];
            } else {
                *o = from_float<TOUT>(a[i]);
            }
        }
    };

    // ---- one pipeline stage
    auto stage = [&](StageRegs<DK, C, PLO>& r, int g) __attribute__((always_inline)) {
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
                if constexpr (PLO) pv = mfma16(frag_rowmajor(Pls, G::LP, 16 * rt_o, 32 * ks, lane), b, pv);
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
        if constexpr (WANT_OUT) store_tile(acc, g);
        if (chunk_end) {
            __syncthreads();  // (C) all reads of R^T for this chunk are done
            write_R();
        }
    };

    write_R();
    StageRegs<DK, C, PLO> r0, r1;
    load_stage(r0, 0);
    load_stage(r1, 1);
    for (int g = 0; g < total; g += 2) {
        stage(r0, g);
        if (g + 1 < total) stage(r1, g + 1);
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


// ---------------------------------------------------------------------------------------------
// Warp-specialised chunk kernel (chunks up to 256): 768 threads = 4 output waves, 4 state waves and
// 4 loader waves (one of each per SIMD), so that loads, LDS traffic and matrix-core work overlap.
//   loader waves (w = 8..11): bring the Q, K and P rows of stage g + NB - 1 from global memory
//                straight into LDS buffer (g + NB - 1) % NB with buffer-to-LDS loads (no registers,
//                no LDS write instructions), NB - 1 stages ahead, then wait for their loads of stage
//                g + 1. Four waves keep four times the loads in flight that one wave's counter
//                allows. They also pull the lines of stage g + 4 into L2 with one more load each
//                into a scratch kilobyte of LDS that nobody reads: the slices of a head run in step,
//                so without it every slice would wait for the same lines to come from memory. The
//                loader waves never read LDS, so the compiler adds no waits for these loads.
//   state waves  (w = 4..7): per 32-token stage g, accumulate R += K^T (V (.) zeta) for their d_k
//                quarter of R (fp32, scaled by g^L at each chunk start), V (.) zeta formed as bf16
//                hi + lo in registers from the stage's V block, and write stage g+1's V rows into
//                the V ring (V loaded into registers two stages ahead). No V (.) zeta planes in the
//                stage buffers leaves room for three buffers at d_k = 256, chunk 128.
//   output waves (w = 0..3): per stage, the 16 x 16 tile (rows 16*(w>>1), columns 16*(w&1)) of
//                g^(j+1) Q R + P V, with R^T (hi + lo) held in registers for the chunk, and its store.
// Q, K, P and R^T tiles are swizzled (SwzTile). At each chunk end the state waves write R^T as bf16
// hi + lo into the Q/K region of the buffer that the finished stage used; the output waves read
// their fragments from it at the next stage, before the loaders refill that buffer. PLO: P comes
// as bf16 hi + lo, both parts loaded, P V on both. QLO: q comes as two bf16 parts (q + qlo, the
// high and low parts of an operand that bf16 does not hold), both loaded, Q R on both (qlo times
// the high part of R; the scores kernel forms P from both parts). NOP: no intra-chunk term (no P,
// no P V): the output is g^(j+1) Q R alone, for split calls whose P V another call carries.
template <int DK, int C, bool PLO = false, bool QLO = false, bool NOP = false>
struct WsGeom {
    static constexpr int QRB = DK * 2;            // bytes per Q / K tile row
    static constexpr int PRB = C * 2;             // bytes per P tile row
    static constexpr int LV = kW;                 // V and V (.) zeta rows: 32 bf16, dense
    static constexpr size_t Q_BYTES = (size_t)kST * QRB;
    static constexpr size_t P_BYTES = NOP ? 0 : (size_t)kST * PRB;
    static constexpr size_t OFF_K = Q_BYTES, OFF_P = 2 * Q_BYTES, OFF_PL = OFF_P + P_BYTES;
    static constexpr size_t OFF_QL = OFF_PL + (PLO ? P_BYTES : 0);
    static constexpr size_t BUF = OFF_QL + (QLO ? Q_BYTES : 0);  // one stage buffer
    // V rows in a ring of C / 32 + 1 blocks of 32 rows: block s of chunk ci sits in slot
    // (ci * C / 32 + s) mod (C / 32 + 1), so during a chunk's last stage the state waves store the
    // next chunk's first rows into the one slot that the chunk's own blocks leave free
    static constexpr int V_SLOTS = C / kST + 1;
    static constexpr size_t V_BLK = (size_t)kST * LV * 2;
    static constexpr size_t V_RING = V_SLOTS * V_BLK;
    static constexpr size_t SCRATCH = 1024;  // target of the L2 warm-up loads
    // three stage buffers when they fit in the 160 KiB of LDS, else two
    static constexpr int NB = 3 * BUF + V_RING + SCRATCH <= 160 * 1024 ? 3 : 2;
    static constexpr size_t OFF_V = NB * BUF;
    static constexpr size_t OFF_SCRATCH = OFF_V + V_RING;
    static constexpr size_t BYTES = OFF_SCRATCH + SCRATCH;
    // R^T (kW rows of DK bf16, swizzled like Q) hi part in the Q region, lo part in the K region
    static_assert((size_t)kW * QRB == Q_BYTES, "R^T hi / lo fill the Q / K regions");
    static_assert(Q_BYTES % 4096 == 0 && P_BYTES % 4096 == 0, "tiles are split over four loader waves in kilobytes");
    static constexpr int Q_KB = (int)(Q_BYTES / 1024), P_KB = (int)(P_BYTES / 1024);
    static constexpr int NDMA = ((QLO ? 3 : 2) * Q_KB + (PLO ? 2 : 1) * P_KB) / 4;  // buffer-to-LDS loads per stage and loader wave
    static_assert(NDMA + 2 <= 63, "the loads of one stage must fit the vmcnt counter");
};

// s_waitcnt immediate (gfx9 encoding) for vmcnt(n), expcnt and lgkmcnt not waited on
template <int n>
constexpr int wait_vm() { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Workgroup barrier for LDS hand-offs: this wave's LDS accesses complete (lgkmcnt(0)), then
// s_barrier. Unlike __syncthreads() it does not wait for outstanding global loads and stores, so
// prefetches stay in flight across it. The empty asm statements keep the compiler from moving
// memory accesses across the barrier. Loads into LDS are waited for explicitly by their issuer.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LT: the state term of a correction call (the (q_hi, k_lo) call of a two-call split, whose k is
// the low part of a k that bf16 does not hold, 2^-8 of it or less): V (.) zeta and R enter the
// matrix cores as single bf16 values (about 2^-9 relative of a term that is itself about 2^-8 of
// the result); P V keeps P as hi + lo.
template <int DK, int C, typename TOUT, bool VSH, bool PLO, bool QLO = false, bool NOP = false, bool LT = false>
__global__ __launch_bounds__(768) void chunk_ws_kernel(MainParams p, HeadConsts hc) {
    using G = WsGeom<DK, C, PLO, QLO, NOP>;
    constexpr int NB = G::NB;
    constexpr int RTR = DK / 64;  // 16-row R tiles per state wave
    constexpr int SPC = C / kST;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    auto buf = [&](int g) __attribute__((always_inline)) { return smem + (g % NB) * G::BUF; };  // buffer of stage g
    // V ring slot of chunk ci's first block, and the block s slots after a first slot f
    auto vfirst = [&](int ci) __attribute__((always_inline)) { return (ci * SPC) % G::V_SLOTS; };
    auto Vblk = [&](int f, int s) __attribute__((always_inline)) {
        const int i = f + s;
        return reinterpret_cast<bf16*>(smem + G::OFF_V + (i >= G::V_SLOTS ? i - G::V_SLOTS : i) * G::V_BLK);
    };

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, c16 = lane & 15;
    const int wl = w & 3;  // wave index within the output or state group
    int bh, slice;
    team_slice(p.teams, p.NS, bh, slice);
    const int h = bh % p.H;
    const int N = p.N, DV = p.NS * kW;
    const float l2g = hc.log2g[h];
    const int col0 = slice * kW;
    const int nchunks = p.nchunks;
    const int L_last = N - (nchunks - 1) * C;
    const int total = (nchunks - 1) * SPC + (L_last + kST - 1) / kST;
    const int rt_o = wl >> 1, ct_o = wl & 1;

    // Buffer resources: loads past the end of a head's data return zero (tail rows, padding). q, k
    // and v of source head bh % srcBH (q and k: rows ldqk apart, from a column block; all rows in
    // reverse with rev); P, out and the states of head bh.
    const int ldqk = p.ldqk, src = bh % p.srcBH;
    auto row_of = [&](int t) __attribute__((always_inline)) { return p.rev ? N - 1 - t : t; };
    const unsigned q_bytes = (unsigned)(((size_t)(N - 1) * ldqk + DK) * 2), v_bytes = (unsigned)((size_t)N * DV * 2);
    const unsigned vp_bytes = (unsigned)((size_t)p.vsplit * DV * 2);  // value rows below vsplit (VShift)
    const size_t qbase = (size_t)src * N * ldqk + (size_t)(bh / p.srcBH) * p.qcol_blk;
    const unsigned p_bytes = (unsigned)((size_t)nchunks * C * C * 2);

    // Barrier sequence, identical for all roles (each role runs its own loop with its own
    // registers): one after the prologue; per stage g: one at a chunk start (s == 0), one at the
    // end of the stage, and one more after a chunk end that is not the last stage.
    if (w >= 8) {
        // ---------------- loader waves
        // first claim on instruction issue in their SIMD, so that each stage's loads go out as soon
        // as the buffer is free (measured 5-7 us faster at the N=8192 layer than equal priorities)
        __builtin_amdgcn_s_setprio(3);
        const int lw = __builtin_amdgcn_readfirstlane(w - 8);  // wave-uniform: one buffer resource per wave
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qbase), 0, q_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + qbase), 0, q_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rql =
            __builtin_amdgcn_make_buffer_rsrc((void*)((QLO ? p.qlo : p.q) + qbase), 0, q_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)src * N * DV), 0, v_bytes, 0x00020000);
        // (no scores without P V: empty resources that no load uses)
        const __amdgpu_buffer_rsrc_t rp =
            __builtin_amdgcn_make_buffer_rsrc((void*)(p.P + (size_t)bh * nchunks * C * C), 0, NOP ? 0u : p_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rpl = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((PLO ? p.Plo : p.P) + (size_t)bh * nchunks * C * C), 0, NOP ? 0u : p_bytes, 0x00020000);
        // This wave's share (kilobytes j = lw mod 4) of the Q, K and P rows of stage g, into its
        // buffer; lane l fills bytes [16l, 16l+16) of each kilobyte. P: only the 32-key steps up to
        // this stage; the rest read as zero, no traffic.
        auto dma_stage = [&](int g) __attribute__((always_inline)) {
            const int ci = g / SPC, s = g % SPC;
            const int tok0 = ci * C + kST * s;
            char* bq = buf(g);
#pragma unroll
            for (int jj = 0; jj < G::Q_KB / 4; ++jj) {
                const int j = 4 * jj + lw;
                const int byte = 1024 * j + 16 * lane, r = byte / G::QRB;
                const int c = ((byte % G::QRB) >> 4) ^ (r & SwzTile<G::QRB>::M);
                const unsigned off = (unsigned)((row_of(tok0 + r) * ldqk + 8 * c) * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)(bq + 1024 * j), 16, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(bq + G::OFF_K + 1024 * j), 16, off, 0, 0, 0);
                if constexpr (QLO)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rql, (__attribute__((address_space(3))) void*)(bq + G::OFF_QL + 1024 * j), 16, off, 0, 0, 0);
            }
            const int per_row = 4 * (s + 1);
            const unsigned base = (unsigned)((ci * C + kST * s) * C);
#pragma unroll
            for (int jj = 0; jj < G::P_KB / 4; ++jj) {
                const int j = 4 * jj + lw;
                const int byte = 1024 * j + 16 * lane, r = byte / G::PRB;
                const int c = ((byte % G::PRB) >> 4) ^ (r & SwzTile<G::PRB>::M);
                const unsigned off = c < per_row ? (base + (unsigned)(r * C + 8 * c)) * 2u : p_bytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (__attribute__((address_space(3))) void*)(bq + G::OFF_P + 1024 * j), 16, off, 0, 0, 0);
                if constexpr (PLO)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rpl, (__attribute__((address_space(3))) void*)(bq + G::OFF_PL + 1024 * j), 16, off, 0, 0, 0);
            }
        };
        // L2 warm-up of stage g: one 16-byte load per 128-byte line, this slice's share (lines
        // i = slice mod NS) of the head's Q (loader 0), K (loader 1) and P (loader 2) lines, and
        // this slice's own V row segments (loader 3). Lanes without a line load past the end.
        auto warm = [&](int g) __attribute__((always_inline)) {
            const int ci = g / SPC, s = g % SPC;
            const int tok0 = ci * C + kST * s;
            constexpr int LPR = G::QRB / 128;  // lines per Q (or K) row
            const int i = slice + p.NS * lane;
            unsigned off;
            __amdgpu_buffer_rsrc_t r = rq;
            if (lw < 2) {
                off = g < total && i < kST * LPR ? (unsigned)(row_of(tok0 + i / LPR) * ldqk * 2 + 128 * (i % LPR)) : q_bytes;
                if (lw == 1) r = rk;
            } else if (NOP && lw == 2) {
                // no P: the lines of q's low part (with QLO), else a load past the end
                off = QLO && g < total && i < kST * LPR ? (unsigned)(row_of(tok0 + i / LPR) * ldqk * 2 + 128 * (i % LPR)) : q_bytes;
                r = rql;
            } else if (lw == 2) {
                const int plr = (kST * (s + 1) * 2 + 127) / 128;  // P lines per row up to this stage
                off = g < total && i < kST * plr ? (unsigned)(((ci * C + kST * s + i / plr) * C) * 2 + 128 * (i % plr)) : p_bytes;
                r = rp;
            } else if constexpr (VSH) {
                const bool pre = __builtin_amdgcn_readfirstlane((int)(tok0 < p.vsplit)) != 0;  // wave-uniform: a scalar resource
                const int t = tok0 + lane, vr = pre ? t : row_of(t) - p.vshift;
                off = g < total && lane < kST && t < N ? (unsigned)((vr * DV + col0) * 2) : (pre ? vp_bytes : v_bytes);
                r = value_rsrc(pre, p.v, p.vpre, src, N, p.vsplit, DV);
            } else {
                off = g < total && lane < kST ? (unsigned)((row_of(tok0 + lane) * DV + col0) * 2) : v_bytes;
                r = rv;
            }
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(smem + G::OFF_SCRATCH), 16, off, 0, 0, 0);
        };
        // Wait for this wave's loads of one stage: the loads issued after them are one stage of
        // loads and two warm-up loads (NB == 3), or one warm-up load (NB == 2).
        constexpr int kAfter = NB == 3 ? G::NDMA + 2 : 1;
        // prologue: stages 0 .. NB-2, warm-up of stages NB .. 2NB-2 ... (see the loop)
        dma_stage(0);
        warm(2);
        if (NB == 3 && total > 1) {
            dma_stage(1);
            warm(3);
            __builtin_amdgcn_s_waitcnt(wait_vm<kAfter>());  // stage 0 landed
        } else {
            __builtin_amdgcn_s_waitcnt(wait_vm<1>());
        }
        lds_barrier();
        for (int g = 0; g < total; ++g) {
            const int s = g % SPC;
            const bool chunk_end = (s == SPC - 1) || (g == total - 1);
            if (s == 0) lds_barrier();  // the output waves have taken R from the buffer refilled next
            if (g + NB - 1 < total) {
                dma_stage(g + NB - 1);
                warm(g + NB + 1);
                __builtin_amdgcn_s_waitcnt(wait_vm<kAfter>());  // stage g+1 landed
            } else {
                __builtin_amdgcn_s_waitcnt(wait_vm<0>());
            }
            lds_barrier();  // stage g consumed; stage g+1 in LDS
            if (chunk_end && g + 1 < total) lds_barrier();
        }
    } else if (w >= 4) {
        // ---------------- state waves: R rows [wl*DK/4, (wl+1)*DK/4) x 32 columns, fp32
        const int st = threadIdx.x - 256;  // 0..255
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)src * N * DV), 0, v_bytes, 0x00020000);
        // V rows of stage g: 32 rows x 4 groups of 8 columns, one 16-byte load per thread < 128 (rows
        // below vsplit from the prefix buffer, the others from v shifted by vshift rows)
        auto load_v = [&](int g) __attribute__((always_inline)) {
            const int gg = g < total ? g : total - 1;
            const int tok0 = (gg / SPC) * C + kST * (gg % SPC);
            const int row = st >> 2, sg = st & 3;
            if constexpr (VSH) {
                const bool pre = __builtin_amdgcn_readfirstlane((int)(tok0 < p.vsplit)) != 0;  // wave-uniform: a scalar resource
                const int t = tok0 + row, vr = pre ? t : row_of(t) - p.vshift;
                const unsigned off =
                    st < kST * 4 && g < total && t < N ? (unsigned)((vr * DV + col0 + 8 * sg) * 2) : (pre ? vp_bytes : v_bytes);
                return buf_load16(value_rsrc(pre, p.v, p.vpre, src, N, p.vsplit, DV), off);
            } else {
                const unsigned off = st < kST * 4 && g < total ? (unsigned)((row_of(tok0 + row) * DV + col0 + 8 * sg) * 2) : v_bytes;
                return buf_load16(rv, off);
            }
        };
        auto store_v = [&](const bf16x8& v, int g) __attribute__((always_inline)) {
            if (st < kST * 4) {
                const int row = st >> 2, sg = st & 3;
                *reinterpret_cast<bf16x8*>(Vblk(vfirst(g / SPC), g % SPC) + row * G::LV + 8 * sg) = v;
            }
        };
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
        auto write_R = [&](char* b) __attribute__((always_inline)) {  // R^T as bf16 hi + lo into a buffer's Q/K region
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
                    const int o = SwzTile<G::QRB>::off(col, row >> 3) + (row & 7) * 2;
                    *reinterpret_cast<bf16x4*>(b + o) = hi;
                    if constexpr (!LT) *reinterpret_cast<bf16x4*>(b + G::OFF_K + o) = lo;
                }
        };
        auto scale_R = [&](int L) __attribute__((always_inline)) {
            const float gL = decay_pow(l2g, (float)L);
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) accR[rt][ct] *= gL;
        };
        // prologue: V of stage 0 into LDS, R_{-1} where the output waves look for it at stage 0
        // (the buffer of stage -1), V of stages 1 and 2 in registers
        store_v(load_v(0), 0);
        write_R(buf(NB - 1));
        bf16x8 va = load_v(1), vb = load_v(2);  // V of stage g+1 for even g (va) and odd g (vb)
        scale_R(min(C, N));
        lds_barrier();
        auto sstage = [&](int g, bf16x8& vn) __attribute__((always_inline)) {
            const int s = g % SPC;
            const bool chunk_end = (s == SPC - 1) || (g == total - 1);
            if (s == 0) lds_barrier();
            const char* Ks = buf(g) + G::OFF_K;
            bf16x8 bhi[2], blo[2], ak[RTR];
            {
                // V (.) zeta of this stage as bf16 hi + lo, formed in registers from the stage's V
                // block: this lane's tokens t = 32 s + 8 g4 + j, zeta = g^(L-1-t) (0 past the chunk)
                const int L = min(C, N - (g / SPC) * C);
                float z[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = kST * s + 8 * g4 + j;
                    z[j] = t < L ? decay_pow(l2g, (float)(L - 1 - t)) : 0.f;
                }
                const bf16* Vb = Vblk(vfirst(g / SPC), s);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const bf16x8 vv = lds_frag_kmajor(Vb, G::LV, 0, 16 * ct, lane);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if constexpr (LT) {
                            bhi[ct][j] = (bf16)((float)vv[j] * z[j]);
                        } else {
                            bf16 a, c;
                            split_hi_lo((float)vv[j] * z[j], a, c);
                            bhi[ct][j] = a;
                            blo[ct][j] = c;
                        }
                    }
                }
            }
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt) ak[rt] = lds_frag_kmajor_swz<G::QRB>(Ks, 0, wl * (DK / 4) + 16 * rt, lane);
            if (g + 1 < total) {
                store_v(vn, g + 1);  // into the V ring (stage g+1's Q/K/P come from the loader)
                vn = load_v(g + 3);
            }
#pragma unroll
            for (int rt = 0; rt < RTR; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    accR[rt][ct] = mfma16(ak[rt], bhi[ct], accR[rt][ct]);
                    if constexpr (!LT) accR[rt][ct] = mfma16(ak[rt], blo[ct], accR[rt][ct]);
                }
            lds_barrier();  // stage g consumed; stage g+1 in LDS
            if (chunk_end && g + 1 < total) {
                write_R(buf(g));  // R of this chunk into stage g's (now idle) Q/K region
                scale_R(min(C, N - ((g + 1) / SPC) * C));
                lds_barrier();
            }
        };
        for (int g = 0; g < total; g += 2) {
            sstage(g, va);
            if (g + 1 < total) sstage(g + 1, vb);
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
        // output rows of this head through a buffer resource: stores past row N are dropped
        const int obh = p.out_acc ? bh % p.srcBH : bh;  // output head
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<TOUT*>(p.out) + (size_t)obh * N * DV), 0, (unsigned)((size_t)N * DV * sizeof(TOUT)), 0x00020000);
        bf16x8 rfh[DK / 32], rfl[DK / 32];
        // g^(r+1) for this lane's rows r = 16 rt_o + 4 g4 + i of a stage
        float row_decay[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) row_decay[i] = decay_pow(l2g, (float)(16 * rt_o + 4 * g4 + i + 1));
        // zero the V ring slots that the state waves do not write before the first stage (all but
        // slot 0): P V reads every block of a chunk, zero P times these rows
        for (int i = threadIdx.x; i < (int)((G::V_RING - G::V_BLK) / 16); i += 256)
            *reinterpret_cast<f32x4*>(smem + G::OFF_V + G::V_BLK + 16 * i) = f32x4{0.f, 0.f, 0.f, 0.f};
        lds_barrier();
        for (int g = 0; g < total; ++g) {
            const int s = g % SPC;
            const bool chunk_end = (s == SPC - 1) || (g == total - 1);
            if (s == 0) {
                // R of the previous chunk sits in the Q/K region of stage g-1's buffer until the barrier
                const char* Rb = buf(g + NB - 1);
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) {
                    rfh[ks] = frag_rowmajor_swz<G::QRB>(Rb, 16 * ct_o, 32 * ks, lane);
                    if constexpr (!LT) rfl[ks] = frag_rowmajor_swz<G::QRB>(Rb + G::OFF_K, 16 * ct_o, 32 * ks, lane);
                }
                lds_barrier();
            }
            const char* Qs = buf(g);
            const char* Ps = buf(g) + G::OFF_P;
            const char* Pls = buf(g) + G::OFF_PL;
            const int vf0 = vfirst(g / SPC);
            // the Q fragments and the first two P V steps' fragments first (their read latencies
            // overlap), then the QR chains; the other P and V reads go out while those run
            bf16x8 qf[DK / 32], pf[2], vf[2];
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) qf[ks] = frag_rowmajor_swz<G::QRB>(Qs, 16 * rt_o, 32 * ks, lane);
            if constexpr (!NOP) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    pf[ks] = frag_rowmajor_swz<G::PRB>(Ps, 16 * rt_o, 32 * ks, lane);
                    vf[ks] = lds_frag_kmajor(Vblk(vf0, ks), G::LV, 0, 16 * ct_o, lane);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 qa[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) qa[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                qa[2 * (ks & 1)] = mfma16(qf[ks], rfh[ks], qa[2 * (ks & 1)]);
                if constexpr (!LT) qa[2 * (ks & 1) + 1] = mfma16(qf[ks], rfl[ks], qa[2 * (ks & 1) + 1]);
            }
            if constexpr (QLO) {
                const char* Qls = buf(g) + G::OFF_QL;
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks)
                    qa[2 * (ks & 1) + 1] = mfma16(frag_rowmajor_swz<G::QRB>(Qls, 16 * rt_o, 32 * ks, lane), rfh[ks], qa[2 * (ks & 1) + 1]);
            }
            // P V over the 32-key steps up to this stage's own, in two chains. The first two steps
            // run at every stage (their fragments are read with Q above): P is zero past the
            // stage's keys (its rows are loaded as zero there) and the V rows there are finite
            // (zeroed at the start, or rows of an earlier chunk); the later steps stop at the
            // stage (measured 10-20 us faster at the N=8192 layer than running every step)
            f32x4 pa[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            if constexpr (!NOP) {
                pa[0] = mfma16(pf[0], vf[0], pa[0]);
                pa[1] = mfma16(pf[1], vf[1], pa[1]);
                if constexpr (PLO) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) pa[ks] = mfma16(frag_rowmajor_swz<G::PRB>(Pls, 16 * rt_o, 32 * ks, lane), vf[ks], pa[ks]);
                }
#pragma unroll
                for (int ks = 2; ks < SPC; ++ks) {
                    if (ks > s) break;  // P is zero past this stage's keys
                    const bf16x8 vk = lds_frag_kmajor(Vblk(vf0, ks), G::LV, 0, 16 * ct_o, lane);
                    pa[ks & 1] = mfma16(frag_rowmajor_swz<G::PRB>(Ps, 16 * rt_o, 32 * ks, lane), vk, pa[ks & 1]);
                    if constexpr (PLO) pa[ks & 1] = mfma16(frag_rowmajor_swz<G::PRB>(Pls, 16 * rt_o, 32 * ks, lane), vk, pa[ks & 1]);
                }
            }
            const f32x4 qr = (qa[0] + qa[2]) + (qa[1] + qa[3]);
            const f32x4 pv = pa[0] + pa[1];
            // g^(j+1) for row j = 32 s + r of the chunk: g^(32 s) (one per stage) times g^(r+1)
            const float gs = decay_pow(l2g, (float)(kST * s));
            const int c0 = (g / SPC) * C;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = kST * s + 16 * rt_o + 4 * g4 + i;  // row within the chunk
                const float acc = qr[i] * (gs * row_decay[i]) + pv[i];
                const unsigned off = (unsigned)((row_of(c0 + j) * DV + col0 + 16 * ct_o + c16) * (int)sizeof(TOUT));
                // output rows with the non-temporal policy (2): they are not read again by this kernel,
                // and the L2 keeps the lines of Q, K and P that the head's slices share (measured
                // 4 us faster per call at the N=8192 layer, five interleaved runs each)
                if constexpr (sizeof(TOUT) == 4) {
                    if (p.out_acc)
                        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc, ro, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, acc), ro, off, 0, 2);
                } else
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_float<TOUT>(acc)), ro, off, 0, 2);
            }
            lds_barrier();  // stage g consumed; stage g+1 in LDS
            if (chunk_end && g + 1 < total) lds_barrier();  // R of this chunk written
        }
    }
}

// Per-head GroupNorm of fp32 pre-norm rows: one wave per (b, h, n) row of DV <= 512 channels, held
// in registers (lane l owns channels 4l..4l+3 and 256+4l..256+4l+3). Mean first, then the biased
// variance from the centred values, so no cancellation; y = (x - mean) / sqrt(var + eps) * w + b,
// times swish(gate) when a (bf16) gate is given.
template <typename TOUT>
__global__ __launch_bounds__(256) void gn_rows_kernel(long rows, int H, int N, int DV, const float* __restrict__ x,
                                                      TOUT* __restrict__ y, GnArgs gn) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float* xr = x + (size_t)row * DV;
    f32x4 xv[2];
    bf16x4 gv[2];  // the gate's values, loaded together with the rows
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 4 * lane + 256 * i;
        xv[i] = c < DV ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr + c)) : f32x4{0.f, 0.f, 0.f, 0.f};
        if (gn.gate && c < DV)
            gv[i] = __builtin_nontemporal_load(reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(gn.gate) + (size_t)row * DV + c));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) s += (xv[i][0] + xv[i][1]) + (xv[i][2] + xv[i][3]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s / (float)DV;
    float m2 = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (4 * lane + 256 * i < DV) {
#pragma unroll
            for (int j = 0; j < 4; ++j) m2 += (xv[i][j] - mean) * (xv[i][j] - mean);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m2 += __shfl_xor(m2, off, 64);
    const float inv = rsqrtf(m2 / (float)DV + gn.eps);
    const int h = (int)((row / N) % H);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = 4 * lane + 256 * i;
        if (c >= DV) continue;
        f32x4 w = {1.f, 1.f, 1.f, 1.f}, bb = {0.f, 0.f, 0.f, 0.f};
        if (gn.weight) w = *reinterpret_cast<const f32x4*>(gn.weight + (size_t)h * DV + c);
        if (gn.bias) bb = *reinterpret_cast<const f32x4*>(gn.bias + (size_t)h * DV + c);
        f32x4 gs = {1.f, 1.f, 1.f, 1.f};
        if (gn.gate) {
#pragma unroll
            for (int j = 0; j < 4; ++j) gs[j] = swish((float)gv[i][j]);
        }
        TOUT o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = from_float<TOUT>(((xv[i][j] - mean) * inv * w[j] + bb[j]) * gs[j]);
        TOUT* yr = y + (size_t)row * DV + c;
        // the normalised rows with non-temporal stores: written once and not read again here
        // (measured 8 us off the N=8192 layer call, four interleaved runs each)
        if constexpr (sizeof(TOUT) == 4)
            __builtin_nontemporal_store(f32x4{(float)o[0], (float)o[1], (float)o[2], (float)o[3]}, reinterpret_cast<f32x4*>(yr));
        else
            __builtin_nontemporal_store(bf16x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<bf16x4*>(yr));
    }
}

// ---------------------------------------------------------------------------------------------
// Workspace layout (bytes, each part 256-aligned):
//   P     B*H*nchunks*C*C bf16      scores of every chunk (only when the output is wanted), followed
//                                   by their low parts in the same layout when the kernel uses them
//   pre   B*H*N*DV fp32             pre-norm output rows (only with GroupNorm)
struct WsLayout {
    size_t p_off, p_bytes, pre_off, pre_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int B, int H, int N, int DV, int C, int gn, int want_out, bool plo) {
    WsLayout l{};
    const size_t nchunks = (size_t)(N + C - 1) / C;
    l.p_off = 0;
    l.p_bytes = want_out ? align256((plo ? 2 : 1) * (size_t)B * H * nchunks * C * C * sizeof(bf16)) : 0;
    l.pre_off = l.p_off + l.p_bytes;
    // fp32 rows: the GroupNorm's pre-norm staging, and at chunks of 256 and 512 (two kernels, see
    // launch_intra_split) the staging of any output that is not fp32 out itself
    l.pre_bytes = want_out && (gn || C >= 256) ? align256((size_t)B * H * N * DV * sizeof(float)) : 0;
    l.total = l.pre_off + l.pre_bytes;
    return l;
}

// Workspace of the segmented kernels (chunk_seg.hip), when they serve the call:
//   sin   B*H*DK*DV fp32   a copy of state_in when the call updates the state in place
//   U     the segments' own final states
//   pre   B*H*N*DV fp32    pre-norm output rows (only with GroupNorm)
struct SegWsLayout {
    size_t sin_off, u_off, pre_off, total;
};

SegWsLayout seg_ws_layout(int B, int H, int N, int DK, int DV, int C, int gn) {
    SegWsLayout l{};
    l.sin_off = 0;
    l.u_off = align256((size_t)B * H * DK * DV * sizeof(float));
    l.pre_off = l.u_off + align256(chunkwise_seg_state_bytes(B, H, N, DK, DV, C));
    l.total = l.pre_off + (gn ? align256((size_t)B * H * N * DV * sizeof(float)) : 0);
    return l;
}

// Whether a plain call (operands contiguous, in time order) at this shape runs on the segmented kernels
bool seg_shape(int DK, int DV, int C, int want_out) {
    LaunchArgs a{};
    a.B = a.H = 1; a.DK = DK; a.DV = DV; a.chunk = C; a.in_bf16 = 1;
    a.out = want_out ? reinterpret_cast<void*>(16) : nullptr;
    return chunkwise_seg_supported(a);
}

// Chunks up to 256 with an output use the warp-specialised kernel, with P as bf16 hi + lo (its
// stage buffers fit in LDS for every supported d_k); 512-token chunks use the single-group kernel,
// with P as hi + lo as well, and state-only calls that reach this point (operands read in place)
// use the single-group kernel without P.
constexpr size_t kLdsBytes = 160 * 1024;
template <int DK, int C, bool WANT_OUT>
constexpr bool use_ws() { return WANT_OUT && C <= 256 && WsGeom<DK, C, true>::BYTES <= kLdsBytes; }
template <int DK, int C>
constexpr bool p_lo() { return use_ws<DK, C, true>() || MainGeom<DK, C, true>::BYTES <= kLdsBytes; }
// whether the warp-specialised kernel takes q as two parts (q + qlo) at (DK, C)
template <int DK, int C>
constexpr bool q_lo_fits() { return C <= 256 && WsGeom<DK, C, true, true>::BYTES <= kLdsBytes; }
// ... and with no intra-chunk term (no P)
template <int DK, int C>
constexpr bool q_lo_nop_fits() { return C <= 256 && WsGeom<DK, C, true, true, true>::BYTES <= kLdsBytes; }

template <int DK>
bool p_lo_dk(int C) {
    switch (C) {
        case 64: return p_lo<DK, 64>();
        case 128: return p_lo<DK, 128>();
        case 256: return p_lo<DK, 256>();
        default: return p_lo<DK, 512>();
    }
}
// whether a call with an output at (DK, C) keeps the low part of P
bool p_lo_used(int DK, int C) { return DK == 64 ? p_lo_dk<64>(C) : p_lo_dk<256>(C); }

template <int DK, int C, typename TOUT, bool WANT_OUT, bool VSH, bool QLO = false, bool NOP = false, bool LT = false>
hipError_t launch_main_v(const LaunchArgs& a, const MainParams& mp) {
    constexpr bool ws = use_ws<DK, C, WANT_OUT>();
    constexpr bool plo = WANT_OUT && p_lo<DK, C>();
    static_assert(!QLO || (ws && (NOP ? q_lo_nop_fits<DK, C>() : q_lo_fits<DK, C>())),
                  "q as two parts on the warp-specialised kernel only");
    static_assert(!NOP || QLO, "no intra-chunk term only with q as two parts");
    static_assert(!LT || (ws && !QLO), "the correction call's single-part state on the warp-specialised kernel only");
    const void* kern;
    if constexpr (ws) kern = reinterpret_cast<const void*>(chunk_ws_kernel<DK, C, TOUT, VSH, true, QLO, NOP, LT>);
    else kern = reinterpret_cast<const void*>(chunk_main_kernel<DK, C, TOUT, WANT_OUT, VSH, plo>);
    size_t dyn;
    if constexpr (ws) dyn = WsGeom<DK, C, true, QLO, NOP>::BYTES;
    else dyn = MainGeom<DK, C, plo>::BYTES;
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    MainParams lp = mp;
    HeadConsts hc = a.hc;
    void* args[] = {&lp, &hc};
    return hipLaunchKernel(kern, dim3(mp.teams * mp.NS), dim3(ws ? 768 : kThreads), args, dyn, a.stream);
}

// value rows through VShift, and q as two parts (fp32 output only), only in the instantiations
// that need them
template <int DK, int C, typename TOUT, bool WANT_OUT>
hipError_t launch_main(const LaunchArgs& a, const MainParams& mp) {
    if constexpr (WANT_OUT && sizeof(TOUT) == 4 && use_ws<DK, C, WANT_OUT>() && q_lo_nop_fits<DK, C>()) {
        if (mp.qlo && a.no_pv)
            return mp.vsplit ? launch_main_v<DK, C, TOUT, WANT_OUT, true, true, true>(a, mp)
                             : launch_main_v<DK, C, TOUT, WANT_OUT, false, true, true>(a, mp);
    }
    if constexpr (WANT_OUT && sizeof(TOUT) == 4 && use_ws<DK, C, WANT_OUT>() && q_lo_fits<DK, C>()) {
        if (mp.qlo && !a.no_pv)
            return mp.vsplit ? launch_main_v<DK, C, TOUT, WANT_OUT, true, true>(a, mp)
                             : launch_main_v<DK, C, TOUT, WANT_OUT, false, true>(a, mp);
    }
    if constexpr (WANT_OUT && sizeof(TOUT) == 4 && use_ws<DK, C, WANT_OUT>()) {
        if (a.lo_state && !mp.qlo && !a.no_pv)
            return mp.vsplit ? launch_main_v<DK, C, TOUT, WANT_OUT, true, false, false, true>(a, mp)
                             : launch_main_v<DK, C, TOUT, WANT_OUT, false, false, false, true>(a, mp);
    }
    if (mp.qlo || a.no_pv || a.lo_state) return hipErrorInvalidValue;
    return mp.vsplit ? launch_main_v<DK, C, TOUT, WANT_OUT, true>(a, mp) : launch_main_v<DK, C, TOUT, WANT_OUT, false>(a, mp);
}

// The segmented kernels, then the GroupNorm row pass when there is one.
template <typename TOUT>
hipError_t launch_seg(const LaunchArgs& a) {
    const SegWsLayout l = seg_ws_layout(a.B, a.H, a.N, a.DK, a.DV, a.chunk, a.gn.enabled);
    char* ws = reinterpret_cast<char*>(a.ws);
    LaunchArgs b = a;
    hipError_t e;
    if (a.state_in && a.state_in == a.state_out) {
        // the last segment writes state_out while workgroups of other segments may still be about to
        // read state_in: they read a copy
        float* cp = reinterpret_cast<float*>(ws + l.sin_off);
        e = launch_copy_state((size_t)a.B * a.H * a.DK * a.DV, a.state_in, cp, a.stream);
        if (e != hipSuccess) return e;
        b.state_in = cp;
    }
    float* U = reinterpret_cast<float*>(ws + l.u_off);
    if (!a.gn.enabled) return launch_chunkwise_seg(b, U, a.out, false);
    float* pre = reinterpret_cast<float*>(ws + l.pre_off);
    e = launch_chunkwise_seg(b, U, pre, true);
    if (e != hipSuccess) return e;
    const long rows = (long)a.B * a.H * a.N;
    hipLaunchKernelGGL(gn_rows_kernel<TOUT>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, a.stream, rows, a.H, a.N, a.DV, pre,
                       reinterpret_cast<TOUT*>(a.out), a.gn);
    return hipGetLastError();
}

// The segmented kernels take a plain call when one workgroup per (head, 32-column slice of d_v)
// would leave compute units idle: they spread the same work over segments of the sequence too.
bool seg_preferred(const LaunchArgs& a) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return chunkwise_seg_supported(a) && (long)a.B * a.H * (a.DV / kW) < cus;
}

// Chunks of 512 (and 256) with an output and plain operands: the two terms of the chunkwise form in
// two kernels. The intra-chunk term (Q K^T (.) D) V runs on the parallel-form kernel restricted to each
// query's own chunk (fp32 rows; P as hi + lo there too); then the warp-specialised kernel without
// an intra-chunk term adds g^(j+1) Q R to them (atomic fp32 adds, one per element) and carries the
// state. Its stage buffers hold Q and K only (32 KiB at d_k = 256), so three fit beside the
// 34 KiB V ring, where the stage buffers with the 512-key scores would not fit twice. With a
// GroupNorm or a bf16 output the rows go through the fp32 pre-norm staging in the workspace.
bool intra_split_ok(const LaunchArgs& a, int DK) {
    const bool plain = a.addr.rev == 0 && (a.addr.ldqk == 0 || a.addr.ldqk == DK) && a.addr.qcol_blk == 0 &&
                       (a.addr.srcBH == 0 || a.addr.srcBH == a.B * a.H) && a.addr.out_acc == 0;
    return plain && a.in_bf16 && a.out != nullptr && !a.qlo && !a.p_anti && !a.p_given && !a.no_pv && !a.lo_state && a.vs.split == 0 &&
           parallel_bf16_supported(DK, a.DV);
}

template <int DK, int C, typename TOUT>
hipError_t launch_intra_split(const LaunchArgs& a) {
    using G = WsGeom<DK, C, true, false, true>;
    static_assert(G::BYTES <= kLdsBytes && p_lo<DK, C>(), "intra-chunk split: stage buffers and staging fit");
    const int nchunks = (a.N + C - 1) / C;
    const WsLayout l = ws_layout(a.B, a.H, a.N, a.DV, C, a.gn.enabled, true, true);
    const bool direct = !a.gn.enabled && sizeof(TOUT) == 4;
    // fp32 staging of a GroupNorm or bf16 output: the pre-norm rows
    float* o32 = direct ? static_cast<float*>(a.out) : reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + l.pre_off);
    LaunchArgs pa = a;  // the intra-chunk term: parallel form within each chunk, fp32 rows
    pa.out = o32;
    pa.out_bf16 = 0;
    pa.gn = GnArgs{};
    pa.intra_chunk = C;
    hipError_t e = launch_parallel_bf16(pa);
    if (e != hipSuccess) return e;
    MainParams mp{};
    mp.H = a.H; mp.N = a.N; mp.C = C; mp.NS = a.DV / kW; mp.nchunks = nchunks; mp.teams = a.B * a.H;
    mp.rev = 0; mp.ldqk = DK; mp.qcol_blk = 0; mp.srcBH = a.B * a.H;
    mp.out_acc = 1;
    mp.q = (const bf16*)a.q; mp.k = (const bf16*)a.k; mp.v = (const bf16*)a.v;
    mp.state_in = a.state_in; mp.state_out = a.state_out; mp.out = o32;
    const void* kern = reinterpret_cast<const void*>(chunk_ws_kernel<DK, C, float, false, true, false, true>);
    if ((e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::BYTES)) != hipSuccess) return e;
    HeadConsts hc = a.hc;
    void* args[] = {&mp, &hc};
    if ((e = hipLaunchKernel(kern, dim3(mp.teams * mp.NS), dim3(768), args, G::BYTES, a.stream)) != hipSuccess) return e;
    const long rows = (long)a.B * a.H * a.N;
    if (a.gn.enabled) return launch_gn_rows(rows, a.H, a.N, a.DV, o32, a.out, sizeof(TOUT) == 2, a.gn, a.stream);
    if (!direct) return launch_add_rows((size_t)rows * a.DV, o32, nullptr, nullptr, a.out, true, a.stream);
    return hipSuccess;
}

template <int DK, int C, typename TOUT>
hipError_t launch_dk_c(const LaunchArgs& a) {
    if (seg_preferred(a)) return launch_seg<TOUT>(a);
    // chunks of 512 and 256 (measured 3.08 against 3.22 ms at N = 65536, chunk 256; at chunk 128 the
    // split is slower, 480 against 427 us at the N = 8192 layer, and the fused kernel stays)
    if constexpr (C == 512 || C == 256) {
        if (intra_split_ok(a, DK)) return launch_intra_split<DK, C, TOUT>(a);
    }
    if (chunkwise_seg_state_supported(a)) return launch_chunkwise_seg_state(a, reinterpret_cast<float*>(a.ws));
    const int nchunks = (a.N + C - 1) / C;
    const bool want_out = a.out != nullptr;
    const bool plo = want_out && p_lo<DK, C>();
    const WsLayout l = ws_layout(a.B, a.H, a.N, a.DV, C, a.gn.enabled, want_out, plo);
    char* ws = reinterpret_cast<char*>(a.ws);
    MainParams mp{};
    mp.H = a.H; mp.N = a.N; mp.C = C; mp.NS = a.DV / kW; mp.nchunks = nchunks; mp.teams = a.B * a.H;
    mp.rev = a.addr.rev;
    mp.ldqk = a.addr.ldqk ? a.addr.ldqk : DK;
    mp.qcol_blk = a.addr.qcol_blk;
    mp.srcBH = a.addr.srcBH ? a.addr.srcBH : a.B * a.H;
    mp.out_acc = a.addr.out_acc;
    if (mp.out_acc && (!want_out || a.gn.enabled || sizeof(TOUT) != 4)) return hipErrorInvalidValue;
    if (a.qlo && (!want_out || a.gn.enabled || sizeof(TOUT) != 4)) return hipErrorInvalidValue;
    if (a.p_anti && (!want_out || !plo || a.qlo || a.N % C != 0)) return hipErrorInvalidValue;
    if (a.p_given && (!want_out || !plo || a.qlo)) return hipErrorInvalidValue;
    if (a.no_pv && (!a.qlo || a.p_anti || a.p_given)) return hipErrorInvalidValue;
    if (a.lo_state && (!want_out || a.gn.enabled || sizeof(TOUT) != 4 || a.qlo || a.no_pv || !use_ws<DK, C, true>())) return hipErrorInvalidValue;
    mp.q = (const bf16*)a.q;
    mp.qlo = (const bf16*)a.qlo; mp.k = (const bf16*)a.k; mp.v = (const bf16*)a.v;
    mp.vpre = (const bf16*)a.vs.pre; mp.vsplit = a.vs.split; mp.vshift = a.vs.shift;
    mp.P = want_out ? reinterpret_cast<const bf16*>(a.p_given ? a.p_given : ws + l.p_off) : nullptr;
    mp.Plo = plo ? mp.P + (size_t)a.B * a.H * nchunks * C * C : nullptr;
    mp.state_in = a.state_in; mp.state_out = a.state_out; mp.out = a.out;
    if (!want_out) return launch_main<DK, C, TOUT, false>(a, mp);

    if (!a.p_given && !a.no_pv) {
        hipLaunchKernelGGL(chunk_scores_kernel<DK>, dim3(nchunks, a.B * a.H), dim3(256), 0, a.stream, a.H, a.N, C, nchunks, mp.q,
                           mp.qlo, mp.k, nullptr, const_cast<bf16*>(mp.P), const_cast<bf16*>(mp.Plo), static_cast<bf16*>(a.p_anti),
                           a.hc, mp.rev, mp.ldqk, mp.qcol_blk, mp.srcBH, NoRot{});
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!a.gn.enabled) return launch_main<DK, C, TOUT, true>(a, mp);
    // GroupNorm: fp32 pre-norm rows into the workspace, then normalise them into out
    float* pre = reinterpret_cast<float*>(ws + l.pre_off);
    mp.out = pre;
    e = launch_main<DK, C, float, true>(a, mp);
    if (e != hipSuccess) return e;
    const long rows = (long)a.B * a.H * a.N;
    hipLaunchKernelGGL(gn_rows_kernel<TOUT>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, a.stream, rows, a.H, a.N, a.DV,
                       pre, reinterpret_cast<TOUT*>(a.out), a.gn);
    return hipGetLastError();
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
    // enough for either kernel family: callers that read operands in place (the backward, residual
    // linear attention) run the warp-specialised kernels at shapes the segmented ones also serve
    const size_t t = ws_layout(B, H, N, DV, chunk, gn && want_out, want_out, want_out && p_lo_used(DK, chunk)).total;
    if (!want_out) {
        // state-only calls with plain operands run on the segment-state kernel (callers that read
        // operands in place run the single-group kernel, which needs no workspace)
        LaunchArgs a{};
        a.B = B; a.H = H; a.N = N; a.DK = DK; a.DV = DV; a.chunk = chunk; a.in_bf16 = 1;
        a.state_out = reinterpret_cast<float*>(16);
        return chunkwise_seg_state_supported(a) ? std::max(t, chunkwise_seg_state_only_bytes(B, H, N, DK, DV)) : t;
    }
    if (!seg_shape(DK, DV, chunk, want_out)) return t;
    const size_t u = seg_ws_layout(B, H, N, DK, DV, chunk, gn && want_out).total;
    return t > u ? t : u;
}

hipError_t launch_gn_rows(long rows, int H, int N, int DV, const float* pre, void* y, bool y_bf16, const GnArgs& gn,
                          hipStream_t stream) {
    if (rows <= 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
    if (y_bf16)
        hipLaunchKernelGGL(gn_rows_kernel<bf16>, grid, dim3(256), 0, stream, rows, H, N, DV, pre, static_cast<bf16*>(y), gn);
    else
        hipLaunchKernelGGL(gn_rows_kernel<float>, grid, dim3(256), 0, stream, rows, H, N, DV, pre, static_cast<float*>(y), gn);
    return hipGetLastError();
}

template <int DK>
bool q_lo_dk(int C) {
    switch (C) {
        case 64: return q_lo_fits<DK, 64>();
        case 128: return q_lo_fits<DK, 128>();
        case 256: return q_lo_fits<DK, 256>();
        default: return false;
    }
}
template <int DK>
bool split2_dk(int C) {
    switch (C) {
        case 64: return q_lo_nop_fits<DK, 64>() && p_lo<DK, 64>();
        case 128: return q_lo_nop_fits<DK, 128>() && p_lo<DK, 128>();
        case 256: return q_lo_nop_fits<DK, 256>() && p_lo<DK, 256>();
        default: return false;
    }
}
bool chunkwise_bf16_split2_supported(int DK, int chunk) { return DK == 64 ? split2_dk<64>(chunk) : DK == 256 && split2_dk<256>(chunk); }

hipError_t launch_chunkwise_bf16_scores(const LaunchArgs& a, const void* q, const void* qlo, const void* k, const void* klo, void* P) {
    const int C = a.chunk, nchunks = (a.N + C - 1) / C;
    if (a.N <= 0 || a.B * a.H <= 0) return hipSuccess;
    if (!(a.DK == 64 || a.DK == 256) || !p_lo_used(a.DK, C)) return hipErrorInvalidValue;
    bf16* ph = static_cast<bf16*>(P);
    bf16* pl = ph + (size_t)a.B * a.H * nchunks * C * C;
    const bf16 *q_ = static_cast<const bf16*>(q), *ql = static_cast<const bf16*>(qlo), *k_ = static_cast<const bf16*>(k),
               *kl = static_cast<const bf16*>(klo);
    const dim3 grid(nchunks, a.B * a.H);
    const int BH = a.B * a.H;
    if (a.DK == 64) {
        if (kl) hipLaunchKernelGGL((chunk_scores_kernel<64, true>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, ql, k_, kl, ph, pl, nullptr, a.hc, 0, 64, 0, BH, NoRot{});
        else hipLaunchKernelGGL((chunk_scores_kernel<64, false>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, ql, k_, nullptr, ph, pl, nullptr, a.hc, 0, 64, 0, BH, NoRot{});
    } else {
        if (kl) hipLaunchKernelGGL((chunk_scores_kernel<256, true>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, ql, k_, kl, ph, pl, nullptr, a.hc, 0, 256, 0, BH, NoRot{});
        else hipLaunchKernelGGL((chunk_scores_kernel<256, false>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, ql, k_, nullptr, ph, pl, nullptr, a.hc, 0, 256, 0, BH, NoRot{});
    }
    return hipGetLastError();
}

hipError_t launch_chunkwise_bf16_scores_rot(const LaunchArgs& a, const void* q, const void* k, const RotConsts& rc, void* const planes[4],
                                            void* P) {
    const int C = a.chunk, nchunks = (a.N + C - 1) / C;
    if (a.N <= 0 || a.B * a.H <= 0) return hipSuccess;
    if (!(a.DK == 64 || a.DK == 256) || !p_lo_used(a.DK, C)) return hipErrorInvalidValue;
    bf16* ph = static_cast<bf16*>(P);
    bf16* pl = ph + (size_t)a.B * a.H * nchunks * C * C;
    RotFuse rf;
    rf.qh = static_cast<bf16*>(planes[0]);
    rf.ql = static_cast<bf16*>(planes[1]);
    rf.kh = static_cast<bf16*>(planes[2]);
    rf.kl = static_cast<bf16*>(planes[3]);
    rf.rc = rc;
    const bf16 *q_ = static_cast<const bf16*>(q), *k_ = static_cast<const bf16*>(k);
    const dim3 grid(nchunks, a.B * a.H);
    const int BH = a.B * a.H;
    if (a.DK == 64)
        hipLaunchKernelGGL((chunk_scores_kernel<64, true, true>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, nullptr, k_,
                           nullptr, ph, pl, nullptr, a.hc, 0, 64, 0, BH, rf);
    else
        hipLaunchKernelGGL((chunk_scores_kernel<256, true, true>), grid, dim3(256), 0, a.stream, a.H, a.N, C, nchunks, q_, nullptr, k_,
                           nullptr, ph, pl, nullptr, a.hc, 0, 256, 0, BH, rf);
    return hipGetLastError();
}

size_t chunkwise_bf16_scores_bytes(int B, int H, int N, int DK, int chunk) {
    const size_t nchunks = (size_t)(N + chunk - 1) / chunk;
    return (p_lo_used(DK, chunk) ? 2 : 1) * (size_t)B * H * nchunks * chunk * chunk * sizeof(bf16);
}

bool chunkwise_bf16_scores_split(int DK, int chunk) { return p_lo_used(DK, chunk); }

bool chunkwise_bf16_qlo_supported(int DK, int C) { return DK == 64 ? q_lo_dk<64>(C) : DK == 256 && q_lo_dk<256>(C); }

hipError_t launch_chunkwise_bf16(const LaunchArgs& a) {
    if (a.DK == 64) return a.out_bf16 ? launch_dk<64, bf16>(a) : launch_dk<64, float>(a);
    return a.out_bf16 ? launch_dk<256, bf16>(a) : launch_dk<256, float>(a);
}

}  // namespace ret

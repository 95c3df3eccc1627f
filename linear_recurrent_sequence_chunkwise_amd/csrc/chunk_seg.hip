// Chunkwise retention, bf16 inputs, split over sequence segments as well as d_v slices.
//
// Method (abeam.tech RetNet summary, "Chunk recursion for long-sequence training"; mlnews.online
// RetNet abstract: chunks encoded in parallel, summarised recurrently). Unrolling the recurrence
// S_n = g S_(n-1) + k_n^T v_n over one chunk of length L with carried state R gives, for local row j,
//     o_j = [(Q K^T (.) D) V]_j + g^(j+1) [Q R]_j,      D[j][t] = g^(j-t) for t <= j
//     R  <- g^L R + K^T (V (.) zeta),                    zeta_t = g^(L-1-t)
// and over a whole segment of tokens [a, b] started from zero,
//     U = sum_{t in [a, b]} g^(b-t) k_t^T v_t,
// so that the state entering a later segment that starts at token c is
//     R_c = g^c state_in + sum over earlier segments of g^(c-1-b) U.
//
// A head has only one chain of states, and the state of one head (d_k x d_v fp32) fills a CU's
// register file, so the work is spread over (head, segment of whole chunks, slice of d_v). Two
// launches:
//   seg_states_kernel  every segment but the last: its U (state-only, fully parallel), into the
//                      workspace.
//   seg_main_kernel    every (head, segment, slice): R_c from state_in and the U of the earlier
//                      segments, then the segment's chunks in 32-token stages:
//                        scores  P = (Q K^T) (.) D on the matrix cores, decay and causal mask in
//                                registers, kept in fp32 and handed to P V as bf16 hi + lo;
//                        out     g^(j+1) Q R + P V, R (of the previous chunk) as bf16 hi + lo
//                                operands held in registers for the chunk;
//                        state   R += K^T (V (.) zeta), V (.) zeta as bf16 hi + lo, R fp32 in
//                                accumulator registers.
// Both kernels run 8 waves, two per SIMD. Wave w = (c, r), c = w % 4, r = w / 4, belongs to the
// slice's column group c (16 CT columns); the two waves of a group sit on one SIMD. The state
// update is split by halves of d_k: wave (c, r) accumulates rows r*DK/2 .. of R over the group's
// columns. The products for the output run over all of d_k and are split by the group's column
// tiles (CT = 2: tile r, both row tiles of a stage) or, with one column tile, by row tiles (row
// tile r): each wave then needs R of the previous chunk over all of d_k for its column tile, so at
// each chunk start the pair swaps their halves of it (as bf16 hi + lo operands) through LDS. Q, K
// and V of each stage pass global -> registers (one stage ahead) -> LDS; the chunk's K and V stay
// in LDS rings for the scores and P V.
#include <type_traits>

#include <algorithm>

#include "common.hpp"

namespace ret {
namespace {

constexpr int kST = 32;  // tokens per stage
constexpr int kNW = 8;   // waves per workgroup
constexpr int kNT = 64 * kNW;

typedef unsigned u32;

template <int DK, int C, int W>
struct SegGeom {
    static constexpr int SPC = C / kST;   // stages per full chunk
    static constexpr int NKS = SPC;       // K ring slots: the chunk's stages (the next stage's K
                                          // lands in the slot whose scores are finished)
    static constexpr int NVS = SPC + 1;   // V ring slots: the chunk's stages and the one being filled
    static constexpr int QRB = DK * 2;    // bytes per Q / K tile row
    static constexpr int VRB = W * 2;     // bytes per V tile row
    static constexpr int PRB = C * 2;     // bytes per P tile row (one bf16 part)
    static constexpr int CT = W / 64;     // 16-column tiles per column group (4 groups)
    static constexpr int RTW = CT;        // row tiles of a stage in one wave's output products
    static constexpr int DKH = DK / 2;    // d_k half of one wave's state update
    static constexpr int KS = DK / 32;    // 32-wide contraction steps over d_k
    static constexpr int KSH = KS / 2;    // ... over the half
    static constexpr int DTH = DKH / 16;  // 16-row tiles of R in the half
    static constexpr size_t Q_BYTES = (size_t)kST * QRB;
    static constexpr size_t V_BYTES = (size_t)kST * VRB;
    static constexpr size_t P_BYTES = (size_t)kST * PRB;
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + Q_BYTES;
    static constexpr size_t OFF_V = OFF_K + NKS * Q_BYTES;
    static constexpr size_t OFF_PH = OFF_V + NVS * V_BYTES;
    static constexpr size_t OFF_PL = OFF_PH + P_BYTES;
    // the chunk-start swap of R halves: 2 KSH operand fragments (hi, lo) of 1 KiB per wave, in a
    // region of its own when LDS has room, else in the P tile and the three K ring slots the new
    // chunk has not filled yet (all idle at a chunk start)
    static constexpr size_t XR_BYTES = (size_t)kNW * 2 * KSH * 1024;
    static constexpr size_t BASE = OFF_PL + P_BYTES;
    static constexpr bool XR_OWN = BASE + XR_BYTES <= 160 * 1024;
    static constexpr size_t BYTES = XR_OWN ? BASE + XR_BYTES : BASE;
    static_assert(XR_OWN || (NKS == 4 && XR_BYTES == 3 * Q_BYTES + 2 * P_BYTES), "chunk-start swap fits the idle tiles");
    static constexpr int QCH = (int)(Q_BYTES / 16), VCH = (int)(V_BYTES / 16);  // 16-byte chunks per tile
    static constexpr int QL = (QCH + kNT - 1) / kNT, VL = (VCH + kNT - 1) / kNT;  // ... per thread
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(KSH >= 1 && (CT == 1 || CT == 2) && SPC >= 2, "tile shapes");
    static_assert(QCH % 64 == 0 && VCH % 64 == 0, "whole waves load each tile");
};

// Segment s of `segs` covers the chunks [s * nchunks / segs, (s+1) * nchunks / segs).
__device__ __forceinline__ int seg_chunk(int s, int nchunks, int segs) { return (int)(((long)s * nchunks) / segs); }

// Workgroup i -> (team = b*h, segment, slice). Workgroup i runs on XCD i % 8: when the number of
// (team, segment) groups is a multiple of 8, the slices of one group share i % 8 (and so one L2,
// which then serves their common Q and K rows).
__device__ __forceinline__ void seg_place(int groups, int NS, int segs, int& team, int& seg, int& slice) {
    const int i = blockIdx.x;
    int grp;
    if (groups % 8 == 0) {
        grp = (i % 8) + 8 * (i / (8 * NS));
        slice = (i / 8) % NS;
    } else {
        grp = i / NS;
        slice = i % NS;
    }
    team = grp / segs;
    seg = grp % segs;
}

// Workgroup barrier for LDS hand-offs: this wave's LDS accesses complete (lgkmcnt(0)), then
// s_barrier. Unlike __syncthreads() it does not wait for outstanding global loads and stores, so
// the next stage's loads stay in flight across it. The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// fp32 pair -> packed bf16 pair (round to nearest even), element 0 in the low half
__device__ __forceinline__ u32 pack_bf16(float a, float b) {
    const bf16 x = (bf16)a, y = (bf16)b;
    return (u32)__builtin_bit_cast(unsigned short, x) | ((u32)__builtin_bit_cast(unsigned short, y) << 16);
}

// The B operand of one 32-row contraction step (rows 32 ks .. 32 ks + 31 of R, 16 columns), high or
// low bf16 part, from the two accumulator tiles X (rows 0..15 of the step) and Y (rows 16..31): in
// accumulator layout lane group G = l/16 holds rows 4G..4G+3 of each tile; the operand wants rows
// 8G..8G+7 of the step. Two lane swaps per register pair regroup them without LDS:
//   32-lane swap: X groups 2,3 <-> Y groups 0,1;  16-lane swap: X groups 1,3 <-> Y groups 0,2,
// after which X holds rows 8G..8G+3 and Y rows 8G+4..8G+7 of lane group G.
__device__ __forceinline__ bf16x8 acc_to_bop(const f32x4& X, const f32x4& Y, bool lo_part) {
    float x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (lo_part) {
            x[i] = X[i] - (float)(bf16)X[i];
            y[i] = Y[i] - (float)(bf16)Y[i];
        } else {
            x[i] = X[i];
            y[i] = Y[i];
        }
    }
    u32 x0 = pack_bf16(x[0], x[1]), x1 = pack_bf16(x[2], x[3]);
    u32 y0 = pack_bf16(y[0], y[1]), y1 = pack_bf16(y[2], y[3]);
    auto a = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(b[0], b[1], false, false);
    u32x4 r = {c[0], d[0], c[1], d[1]};
    return __builtin_bit_cast(bf16x8, r);
}

// The workgroup's loads of one 32-token stage, global -> registers: Q and K rows tok0 .. tok0+31
// (DK columns) and V rows (the slice's W columns). 16-byte chunk j of a tile is loaded by thread
// j % 512 (its slot j / 512); threads past a tile's chunks (whole waves) load nothing. Rows past
// the sequence, and every load of a stage that is not live, read as zero.
template <int DK, int C, int W>
struct StageLoad {
    using G = SegGeom<DK, C, W>;
    bf16x8 q[G::QL], k[G::QL], v[G::VL];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int tok0,
                                         bool live, int DV, int col0, bool want_q) {
        constexpr int QC = G::QRB / 16, VC = G::VRB / 16;  // 16-byte chunks per row
#pragma unroll
        for (int u = 0; u < G::QL; ++u) {
            const int j = threadIdx.x + kNT * u, row = j / QC, c = j % QC;
            const unsigned off = live && j < G::QCH ? (unsigned)(((tok0 + row) * DK + 8 * c) * 2) : 0x80000000u;
            if (want_q) q[u] = buf_load16(rq, off);
            k[u] = buf_load16(rk, off);
        }
#pragma unroll
        for (int u = 0; u < G::VL; ++u) {
            const int j = threadIdx.x + kNT * u, row = j / VC, c = j % VC;
            const unsigned off = live && j < G::VCH ? (unsigned)(((tok0 + row) * DV + col0 + 8 * c) * 2) : 0x80000000u;
            v[u] = buf_load16(rv, off);
        }
    }
    // registers -> the stage's LDS tiles (swizzled rows)
    __device__ __forceinline__ void store(char* qs, char* ks, char* vs, bool want_q) const {
        constexpr int QC = G::QRB / 16, VC = G::VRB / 16;
#pragma unroll
        for (int u = 0; u < G::QL; ++u) {
            const int j = threadIdx.x + kNT * u, row = j / QC, c = j % QC;
            if (G::QCH % kNT == 0 || j < G::QCH) {
                const int o = SwzTile<G::QRB>::off(row, c);
                if (want_q) *reinterpret_cast<bf16x8*>(qs + o) = q[u];
                *reinterpret_cast<bf16x8*>(ks + o) = k[u];
            }
        }
#pragma unroll
        for (int u = 0; u < G::VL; ++u) {
            const int j = threadIdx.x + kNT * u, row = j / VC, c = j % VC;
            if (G::VCH % kNT == 0 || j < G::VCH) *reinterpret_cast<bf16x8*>(vs + SwzTile<G::VRB>::off(row, c)) = v[u];
        }
    }
};

struct SegParams {
    int H, N, C, NS, segs, nchunks, teams, DV;
    const bf16* q;
    const bf16* k;
    const bf16* v;
    const float* state_in;
    float* state_out;
    float* U;    // [teams][segs - 1][DK][DV] fp32: the segments' own final states ([teams][segs][DK][DV] for
                 // a state-only call with more than one segment)
    void* out;   // [teams][N][DV] in TOUT (pre-norm fp32 rows when GroupNorm follows)
    int state_only;  // seg_states_kernel covers every segment, the last one ending at N
};

// V (.) zeta of one B fragment (8 consecutive tokens of one column), split into bf16 hi + lo
__device__ __forceinline__ void scale_split(const bf16x8& v, const float* z, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (float)v[e] * z[e];
        const bf16 a = (bf16)x;
        hi[e] = a;
        lo[e] = (bf16)(x - (float)a);
    }
}

// The wave's state update over one 32-token tile in LDS: R[half r rows][its columns] +=
// K^T (V (.) zeta), with z the decay factors of this lane's 8 tokens (8 g4 .. 8 g4 + 7 of the tile).
template <int DK, int C, int W, int DTH_, int CT_>
__device__ __forceinline__ void state_update(f32x4 (&accR)[DTH_][CT_], const char* Ks, const char* Vs, const float* z, int r, int cc0,
                                             int lane) {
    using G = SegGeom<DK, C, W>;
    static_assert(DTH_ == G::DTH && CT_ == G::CT, "accumulator shape");
    bf16x8 bh[G::CT], bl[G::CT];
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) scale_split(lds_frag_kmajor_swz<G::VRB>(Vs, 0, cc0 + 16 * ct, lane), z, bh[ct], bl[ct]);
#pragma unroll
    for (int dt = 0; dt < G::DTH; ++dt) {
        const bf16x8 a = lds_frag_kmajor_swz<G::QRB>(Ks, 0, r * G::DKH + 16 * dt, lane);
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) accR[dt][ct] = mfma16(a, bh[ct], accR[dt][ct]);
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) accR[dt][ct] = mfma16(a, bl[ct], accR[dt][ct]);
        if (dt % 4 == 3) __builtin_amdgcn_sched_barrier(0);  // bounds the fragment reads in flight
    }
}

// ---------------------------------------------------------------------------------------------
// U of segment s < segs - 1 for one (team, slice): sum over the segment's tokens t of
// g^(b - t) k_t^T v_t, b its last token. Grid: teams * (segs - 1) * NS workgroups of 8 waves, laid
// out as in the main kernel (wave (c, r): column group c, d_k half r). Three K and V tile buffers:
// each step's tiles are stored two steps ahead of use.
// A state-only call (state_only) takes every segment, the last one ending at token N - 1 (its
// last step reads rows past N as zero); with one segment the workgroup writes the final state
// g^N state_in + U itself, else the segments' U for seg_final_kernel.
template <int DK, int C, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(kNT, kNT), amdgpu_waves_per_eu(2, 2))) void seg_states_kernel(SegParams p,
                                                                                                                   HeadConsts hc) {
    using G = SegGeom<DK, C, W>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    // w is the same in every lane of a wave: readfirstlane keeps it in scalar registers
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g4 = lane >> 4, c16 = lane & 15;
    const int c = w & 3, r = w >> 2;
    const int S1 = p.state_only ? p.segs : p.segs - 1;
    const int i = blockIdx.x;
    const int team = i / (S1 * p.NS), seg = (i / p.NS) % S1, slice = i % p.NS;
    const int N = p.N, DV = p.DV, h = team % p.H;
    const float l2g = hc.log2g[h];
    const int col0 = slice * W, cc0 = c * 16 * G::CT;
    const int t0 = seg_chunk(seg, p.nchunks, p.segs) * C, t1 = min(seg_chunk(seg + 1, p.nchunks, p.segs) * C, N);  // [t0, t1)
    const int steps = (t1 - t0 + kST - 1) / kST;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)team * N * DK), 0,
                                                                        (unsigned)((size_t)N * DK * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)team * N * DV), 0,
                                                                        (unsigned)((size_t)N * DV * 2), 0x00020000);
    auto Kb = [&](int b) __attribute__((always_inline)) { return smem + (size_t)b * G::Q_BYTES; };
    auto Vb = [&](int b) __attribute__((always_inline)) { return smem + 3 * G::Q_BYTES + (size_t)b * G::V_BYTES; };

    f32x4 acc[G::DTH][G::CT];
#pragma unroll
    for (int dt = 0; dt < G::DTH; ++dt)
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) acc[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    // log2 of the decay of this lane's token 8 g4 + e of a step, relative to the step's first token
    float zl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) zl[e] = -(float)(8 * g4 + e) * l2g;

    StageLoad<DK, C, W> st;
    st.load(rk, rk, rv, t0, steps > 0, DV, col0, false);
    st.store(nullptr, Kb(0), Vb(0), false);
    st.load(rk, rk, rv, t0 + kST, steps > 1, DV, col0, false);
    st.store(nullptr, Kb(1), Vb(1), false);
    st.load(rk, rk, rv, t0 + 2 * kST, steps > 2, DV, col0, false);
    for (int g = 0; g < steps; ++g) {
        lds_barrier();  // step g's tiles written; step g-1's reads done
        // step g + 2's tiles into the buffer step g - 1 used; step g + 3's loads
        st.store(nullptr, Kb((g + 2) % 3), Vb((g + 2) % 3), false);
        st.load(rk, rk, rv, t0 + kST * (g + 3), g + 3 < steps, DV, col0, false);
        // decay to the segment's last token t1 - 1 of token t0 + 32 g + 8 g4 + e
        const float zs = (float)(t1 - 1 - t0 - kST * g) * l2g;
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = __builtin_amdgcn_exp2f(zs + zl[e]);
        state_update<DK, C, W>(acc, Kb(g % 3), Vb(g % 3), z, r, cc0, lane);
    }
    if (p.state_only && p.segs == 1) {
        // the final state: g^N state_in + U (each lane reads the state_in elements it writes, so
        // state_out may be state_in)
        const float gN = decay_pow(l2g, (float)N);
        const size_t base = (size_t)team * DK * DV;
#pragma unroll
        for (int dt = 0; dt < G::DTH; ++dt)
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t o = base + (size_t)(r * G::DKH + 16 * dt + 4 * g4 + e) * DV + col0 + cc0 + 16 * ct + c16;
                    p.state_out[o] = (p.state_in ? gN * p.state_in[o] : 0.f) + acc[dt][ct][e];
                }
        return;
    }
    float* U = p.U + ((size_t)team * S1 + seg) * DK * DV;
#pragma unroll
    for (int dt = 0; dt < G::DTH; ++dt)
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                U[(size_t)(r * G::DKH + 16 * dt + 4 * g4 + e) * DV + col0 + cc0 + 16 * ct + c16] = acc[dt][ct][e];
}

// The final state of a state-only call over several segments: g^N state_in + sum over segments s
// of g^(N - 1 - b_s) U_s, b_s the segment's last token. Grid-stride over groups of four elements
// (DK * DV a multiple of 4); each thread reads the state_in elements it writes.
__global__ __launch_bounds__(256) void seg_final_kernel(SegParams p, HeadConsts hc, int DK, int C) {
    const size_t per = (size_t)DK * p.DV / 4, n4 = (size_t)p.teams * per;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
        const int team = (int)(i / per);
        const float l2g = hc.log2g[team % p.H];
        f32x4 acc = p.state_in ? reinterpret_cast<const f32x4*>(p.state_in)[i] * decay_pow(l2g, (float)p.N) : f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < p.segs; ++s) {
            const int b = min(seg_chunk(s + 1, p.nchunks, p.segs) * C, p.N) - 1;
            acc += reinterpret_cast<const f32x4*>(p.U + ((size_t)team * p.segs + s) * DK * p.DV)[i % per] *
                   decay_pow(l2g, (float)(p.N - 1 - b));
        }
        reinterpret_cast<f32x4*>(p.state_out)[i] = acc;
    }
}

// ---------------------------------------------------------------------------------------------
// One (team, segment, slice) per workgroup; see the file comment. Each chunk starts with the swap
// of R halves (two barriers); stage s of the chunk (s a compile-time constant: the chunk's stages
// are unrolled, so no branch sits among the matrix products) runs with two:
//   (B1) Q, K and V of the stage in LDS, the previous stage's P reads done
//   Q R (over all of d_k, the wave's output tiles) and its score tiles in one pass over Q; the
//     decayed, masked scores into the P tile as bf16 hi + lo
//   (B2) the next stage's registers -> LDS, its next loads issued; P V; the state update of the
//     wave's d_k half; output rows g^(j+1) Q R + P V.
// Scores of stage s: the 2 (s + 1) key tiles of 16 keys up to the stage, both row tiles each; wave
// w takes key tile w mod 2 (s + 1), so that every wave issues the same products (waves with the
// same key tile compute and write the same values).
template <int DK, int C, int W, typename TOUT>
__global__ __attribute__((amdgpu_flat_work_group_size(kNT, kNT), amdgpu_waves_per_eu(2, 2))) void seg_main_kernel(SegParams p,
                                                                                                                 HeadConsts hc) {
    using G = SegGeom<DK, C, W>;
    constexpr int SPC = G::SPC, NKS = G::NKS, NVS = G::NVS, KS = G::KS, KSH = G::KSH, DTH = G::DTH, CT = G::CT, RTW = G::RTW;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    char* Qs = smem + G::OFF_Q;
    auto Kslot = [&](int g) __attribute__((always_inline)) { return smem + G::OFF_K + (size_t)(g % NKS) * G::Q_BYTES; };
    auto Vslot = [&](int g) __attribute__((always_inline)) { return smem + G::OFF_V + (size_t)(g % NVS) * G::V_BYTES; };
    char* Ph = smem + G::OFF_PH;
    char* Pl = smem + G::OFF_PL;

    const int lane_ = threadIdx.x & 63, w_ = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), g4 = lane_ >> 4, c16 = lane_ & 15;
    const int w = w_, c = w & 3, r = w >> 2;
    const int qct = CT == 2 ? r : 0;   // the group's column tile of this wave's output products
    int team, seg, slice;
    seg_place(p.teams * p.segs, p.NS, p.segs, team, seg, slice);
    const int N = p.N, DV = p.DV, h = team % p.H;
    const float l2g = hc.log2g[h];
    const int col0 = slice * W, cc0 = c * 16 * CT;  // the slice's first column; the group's first column in it
    const int oc = col0 + cc0 + 16 * qct;          // first output column of this wave
    const int cb = seg_chunk(seg, p.nchunks, p.segs), ce = seg_chunk(seg + 1, p.nchunks, p.segs);
    const int total = (ce - cb) * SPC;  // stages of this segment (the last chunk's past N read as zero)
    const int tokA = cb * C;            // first token of the segment

    const unsigned qk_bytes = (unsigned)((size_t)N * DK * 2);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + (size_t)team * N * DK), 0, qk_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + (size_t)team * N * DK), 0, qk_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + (size_t)team * N * DV), 0,
                                                                        (unsigned)((size_t)N * DV * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(reinterpret_cast<TOUT*>(p.out) + (size_t)team * N * DV), 0, (unsigned)((size_t)N * DV * sizeof(TOUT)), 0x00020000);
    auto stage_tok0 = [&](int g) __attribute__((always_inline)) { return (cb + g / SPC) * C + kST * (g % SPC); };

    // ---- the state entering the segment: g^tokA state_in + sum over earlier segments of
    // g^(tokA - 1 - b) U (b = that segment's last token), for this wave's rows and columns
    f32x4 accR[DTH][CT];
    auto r_off = [&](int dt, int ct, int e) __attribute__((always_inline)) {
        return (size_t)(r * G::DKH + 16 * dt + 4 * g4 + e) * DV + col0 + cc0 + 16 * ct + c16;
    };
    {
        const float a = decay_pow(l2g, (float)tokA);
        const float* si = p.state_in ? p.state_in + (size_t)team * DK * DV : nullptr;
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) accR[dt][ct][e] = si ? a * si[r_off(dt, ct, e)] : 0.f;
    }
    for (int s2 = 0; s2 < seg; ++s2) {
        const int b = seg_chunk(s2 + 1, p.nchunks, p.segs) * C - 1;  // last token of segment s2
        const float a = decay_pow(l2g, (float)(tokA - 1 - b));
        const float* U = p.U + ((size_t)team * (p.segs - 1) + s2) * DK * DV;
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) accR[dt][ct][e] += a * U[r_off(dt, ct, e)];
    }

    // per-lane parts of the decay exponents (each exponent is one of these plus a wave-uniform part):
    //   g^(j+1) of this lane's output rows j = 32 s + 16 rt + 4 g4 + e: 2^(x4 + (32 s + 16 rt + e + 1) l2g)
    //   the scores' g^(j - t), row j = 16 rt + c16 of the stage, key t = 16 kt + 4 g4 + e of the chunk:
    //     j - t = pd + A - e with A = 32 s + 16 rt - 16 kt
    //   zeta of this lane's tokens t = 32 s + 8 g4 + e: 2^(z8 + (L - 1 - 32 s - e) l2g)
    const int pd = c16 - 4 * g4;
    const float x4_ = (float)(4 * g4) * l2g, p4_ = (float)pd * l2g, z8_ = -(float)(8 * g4) * l2g;

    // the chunk-start swap area of wave w: 2 KSH fragments of 1 KiB
    auto xr = [&](int wv, int ch, int ks, int lo) __attribute__((always_inline)) {
        const int f = (ks * 2 + lo);  // fragment within the wave's part
        char* base;
        if constexpr (G::XR_OWN) {
            base = smem + G::BASE + (size_t)wv * 2 * KSH * 1024;
        } else {
            // 8 KiB per wave: pairs of waves share the P tile (hi + lo) or one of the three K slots
            // the chunk's first stage does not use
            const int reg = wv >> 1;
            base = (reg == 3 ? Ph : Kslot(ch + 1 + reg)) + (size_t)(wv & 1) * 2 * KSH * 1024;
        }
        return reinterpret_cast<bf16x8*>(base + (size_t)f * 1024);
    };

    StageLoad<DK, C, W> st;
    st.load(rq, rk, rv, stage_tok0(0), total > 0, DV, col0, true);
    st.store(Qs, Kslot(0), Vslot(0), true);
    st.load(rq, rk, rv, stage_tok0(1), total > 1, DV, col0, true);

    bf16x8 rbh[KS], rbl[KS];  // R of the previous chunk, all of d_k, column tile qct: B operands
    for (int ci = cb; ci < ce; ++ci) {
        const int L = min(C, N - ci * C);
        const int g0 = (ci - cb) * SPC;  // segment stage index of the chunk's first stage
        // ---- swap of R halves: operands of this wave's half for its own column tile, and for the
        // partner's (into LDS); then the partner's half of its own column tile (from LDS)
        lds_barrier();  // every wave's reads of the previous stage's P and K done
        {
            // (register arrays are indexed by compile-time values only; r picks through selects)
            const int lane = lane_;
            bf16x8 oh[KSH], ol[KSH];  // this wave's half, its own column tile
#pragma unroll
            for (int ks = 0; ks < KSH; ++ks) {
                const f32x4 x0 = CT == 2 && r ? accR[2 * ks][CT - 1] : accR[2 * ks][0];
                const f32x4 x1 = CT == 2 && r ? accR[2 * ks + 1][CT - 1] : accR[2 * ks + 1][0];
                oh[ks] = acc_to_bop(x0, x1, false);
                ol[ks] = acc_to_bop(x0, x1, true);
                // the partner's column tile (the other one, or the same with one tile)
                const f32x4 y0 = CT == 2 && !r ? accR[2 * ks][CT - 1] : accR[2 * ks][0];
                const f32x4 y1 = CT == 2 && !r ? accR[2 * ks + 1][CT - 1] : accR[2 * ks + 1][0];
                xr(w, g0, ks, 0)[lane] = acc_to_bop(y0, y1, false);
                xr(w, g0, ks, 1)[lane] = acc_to_bop(y0, y1, true);
            }
            lds_barrier();
#pragma unroll
            for (int ks = 0; ks < KSH; ++ks) {
                const bf16x8 ph = xr(w ^ 4, g0, ks, 0)[lane], pl = xr(w ^ 4, g0, ks, 1)[lane];
                rbh[ks] = r ? ph : oh[ks];
                rbl[ks] = r ? pl : ol[ks];
                rbh[KSH + ks] = r ? oh[ks] : ph;
                rbl[KSH + ks] = r ? ol[ks] : pl;
            }
        }
        {
            const float gL = decay_pow(l2g, (float)L);
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) accR[dt][ct] *= gL;
        }

        auto stage = [&](auto s_c) __attribute__((always_inline)) {
            constexpr int s = decltype(s_c)::value;
            constexpr int NKT = 2 * (s + 1);  // key tiles of 16 keys up to this stage
            const int g = g0 + s;
            // the lane index, opaque to the compiler within each stage: the swizzled LDS addresses of
            // the stage's fragments are then recomputed per stage (a few instructions each) instead of
            // each being held in a register across the chunk loop
            // The same for the decay base: the stage's decay factors are then computed here (a few
            // transcendental instructions) rather than hoisted out of the chunk loop as dozens of
            // loop-invariant registers.
            int lane = lane_, w = w_;
            float l2 = l2g, p4 = p4_, x4 = x4_, z8 = z8_;
            asm volatile("" : "+v"(lane), "+v"(l2), "+v"(p4), "+v"(x4), "+v"(z8), "+s"(w));
            const int r = w >> 2, rt0 = CT == 2 ? 0 : r;
            lds_barrier();  // (B1)

            // ---- Q R over all of d_k for this wave's output tiles, and the scores of its key tile
            // kt = w mod NKT for both row tiles
            const int kt = w % NKT;
            f32x4 qr[RTW], sc[2];
#pragma unroll
            for (int t = 0; t < RTW; ++t) qr[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            sc[0] = sc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 qa[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) qa[rt] = frag_rowmajor_swz<G::QRB>(Qs, 16 * rt, 32 * ks, lane);
#pragma unroll
                for (int t = 0; t < RTW; ++t) qr[t] = mfma16(CT == 2 ? qa[t] : (r ? qa[1] : qa[0]), rbh[ks], qr[t]);
                {
                    const bf16x8 ka = frag_rowmajor_swz<G::QRB>(Kslot(g - s + kt / 2), 16 * (kt & 1), 32 * ks, lane);
                    sc[0] = mfma16(ka, qa[0], sc[0]);
                    sc[1] = mfma16(ka, qa[1], sc[1]);
                }
#pragma unroll
                for (int t = 0; t < RTW; ++t) qr[t] = mfma16(CT == 2 ? qa[t] : (r ? qa[1] : qa[0]), rbl[ks], qr[t]);
                // keep the next steps' fragment reads from being hoisted far ahead (registers)
                if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
            // decayed, masked scores -> P (hi, lo): lane holds keys 16 kt + 4 g4 + e of stage row
            // 16 rt + c16 (waves with the same key tile write the same values)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int A = kST * s + 16 * rt - 16 * kt;  // j - t = pd + A - e
                float x[4], y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = __builtin_amdgcn_exp2f(p4 + (float)(A - e) * l2);
                    x[e] = pd + A - e >= 0 ? sc[rt][e] * d : 0.f;
                    y[e] = x[e] - (float)(bf16)x[e];
                }
                const int o = SwzTile<G::PRB>::off(16 * rt + c16, 2 * kt + (g4 >> 1)) + 8 * (g4 & 1);
                *reinterpret_cast<uint2*>(Ph + o) = uint2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
                *reinterpret_cast<uint2*>(Pl + o) = uint2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
            }
            lds_barrier();  // (B2)

            // ---- the next stage's tiles into LDS (Q buffer, K slot g+1 (its scores are done), V slot
            // g+1), and the loads of stage g + 2
            st.store(Qs, Kslot(g + 1), Vslot(g + 1), true);
            st.load(rq, rk, rv, stage_tok0(g + 2), g + 2 < total, DV, col0, true);

            // ---- P V of this wave's output tiles over the chunk's key steps 0..s
            f32x4 pv[RTW];
#pragma unroll
            for (int t = 0; t < RTW; ++t) pv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k2 = 0; k2 <= s; ++k2) {
                const bf16x8 vb = lds_frag_kmajor_swz<G::VRB>(Vslot(g - s + k2), 0, cc0 + 16 * qct, lane);
#pragma unroll
                for (int t = 0; t < RTW; ++t) {
                    const int rt = rt0 + t;
                    pv[t] = mfma16(frag_rowmajor_swz<G::PRB>(Ph, 16 * rt, 32 * k2, lane), vb, pv[t]);
                    pv[t] = mfma16(frag_rowmajor_swz<G::PRB>(Pl, 16 * rt, 32 * k2, lane), vb, pv[t]);
                }
            }

            // ---- state: R (rows of d_k half r, the group's columns) += K^T (V (.) zeta), zeta_t =
            // g^(L - 1 - t) for this lane's tokens t = 32 s + 8 g4 + e, 0 past the chunk
            {
                float z[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    z[e] = kST * s + 8 * g4 + e < L ? __builtin_amdgcn_exp2f(z8 + (float)(L - 1 - kST * s - e) * l2) : 0.f;
                state_update<DK, C, W>(accR, Kslot(g), Vslot(g), z, r, cc0, lane);
            }

            // ---- output rows j = 32 s + 16 rt + 4 g4 + e: g^(j+1) Q R + P V
#pragma unroll
            for (int t = 0; t < RTW; ++t) {
                const int rt = rt0 + t;
                const int r0 = ci * C + kST * s + 16 * rt;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float o = qr[t][e] * __builtin_amdgcn_exp2f(x4 + (float)(kST * s + 16 * rt + e + 1) * l2) + pv[t][e];
                    const int row = r0 + 4 * g4 + e;
                    const unsigned off = (unsigned)(((size_t)row * DV + oc + c16) * sizeof(TOUT));
                    if constexpr (sizeof(TOUT) == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, o), ro, off, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_float<TOUT>(o)), ro, off, 0, 0);
                }
            }
        };
        stage(std::integral_constant<int, 0>{});
        stage(std::integral_constant<int, 1>{});
        if constexpr (SPC > 2) {
            stage(std::integral_constant<int, 2>{});
            stage(std::integral_constant<int, 3>{});
        }
    }
    if (p.state_out && seg == p.segs - 1) {
        float* so = p.state_out + (size_t)team * DK * DV;
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) so[r_off(dt, ct, e)] = accR[dt][ct][e];
    }
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Host side: shape support, segment count, workspace, launches.
namespace {

// Slice width: 128 columns when d_v allows, else 64.
int seg_width(int DV) { return DV % 128 == 0 ? 128 : (DV % 64 == 0 ? 64 : 0); }

// Segments per head: enough (team, segment, slice) workgroups to fill the 256 CUs once, in whole
// chunks, at least one chunk per segment.
int seg_count(int teams, int NS, int nchunks) {
    const int per = teams * NS;
    if (per >= 256) return 1;
    int s = 256 / per;
    return s < nchunks ? s : nchunks;
}

template <int DK, int C, int W, typename TOUT>
hipError_t seg_launch_t(const LaunchArgs& a, float* U, void* out) {
    using G = SegGeom<DK, C, W>;
    SegParams p{};
    p.H = a.H; p.N = a.N; p.C = C; p.DV = a.DV; p.NS = a.DV / W; p.teams = a.B * a.H;
    p.nchunks = (a.N + C - 1) / C;
    p.segs = seg_count(p.teams, p.NS, p.nchunks);
    p.q = (const bf16*)a.q; p.k = (const bf16*)a.k; p.v = (const bf16*)a.v;
    p.state_in = a.state_in; p.state_out = a.state_out; p.U = U; p.out = out;
    HeadConsts hc = a.hc;
    hipError_t e;
    if (p.segs > 1) {
        const void* kern = reinterpret_cast<const void*>(seg_states_kernel<DK, C, W>);
        const size_t dyn = 3 * (G::Q_BYTES + G::V_BYTES);
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
        void* args[] = {&p, &hc};
        e = hipLaunchKernel(kern, dim3(p.teams * (p.segs - 1) * p.NS), dim3(kNT), args, dyn, a.stream);
        if (e != hipSuccess) return e;
    }
    const void* kern = reinterpret_cast<const void*>(seg_main_kernel<DK, C, W, TOUT>);
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)G::BYTES);
    if (e != hipSuccess) return e;
    void* args[] = {&p, &hc};
    return hipLaunchKernel(kern, dim3(p.teams * p.segs * p.NS), dim3(kNT), args, G::BYTES, a.stream);
}

// A state-only call: every segment's U in one launch (128-token chunk geometry: the chunk length
// only sets where segments may split), then their decayed sum when there are several.
template <int DK, int W>
hipError_t seg_state_launch_t(const LaunchArgs& a, float* U) {
    constexpr int C = 128;
    using G = SegGeom<DK, C, W>;
    SegParams p{};
    p.H = a.H; p.N = a.N; p.C = C; p.DV = a.DV; p.NS = a.DV / W; p.teams = a.B * a.H;
    p.nchunks = (a.N + C - 1) / C;
    p.segs = seg_count(p.teams, p.NS, p.nchunks);
    p.k = (const bf16*)a.k; p.v = (const bf16*)a.v;
    p.state_in = a.state_in; p.state_out = a.state_out; p.U = U;
    p.state_only = 1;
    HeadConsts hc = a.hc;
    const void* kern = reinterpret_cast<const void*>(seg_states_kernel<DK, C, W>);
    const size_t dyn = 3 * (G::Q_BYTES + G::V_BYTES);
    hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    void* args[] = {&p, &hc};
    e = hipLaunchKernel(kern, dim3(p.teams * p.segs * p.NS), dim3(kNT), args, dyn, a.stream);
    if (e != hipSuccess || p.segs == 1) return e;
    const size_t n4 = (size_t)p.teams * DK * p.DV / 4;
    const unsigned grid = (unsigned)std::min<size_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(seg_final_kernel, dim3(grid), dim3(256), 0, a.stream, p, hc, DK, C);
    return hipGetLastError();
}

template <int DK, int C, typename TOUT>
hipError_t seg_launch_c(const LaunchArgs& a, float* U, void* out) {
    return seg_width(a.DV) == 128 ? seg_launch_t<DK, C, 128, TOUT>(a, U, out) : seg_launch_t<DK, C, 64, TOUT>(a, U, out);
}

template <int DK, typename TOUT>
hipError_t seg_launch_dk(const LaunchArgs& a, float* U, void* out) {
    return a.chunk == 64 ? seg_launch_c<DK, 64, TOUT>(a, U, out) : seg_launch_c<DK, 128, TOUT>(a, U, out);
}

}  // namespace

bool chunkwise_seg_supported(const LaunchArgs& a) {
    const bool plain = a.addr.rev == 0 && (a.addr.ldqk == 0 || a.addr.ldqk == a.DK) && a.addr.qcol_blk == 0 &&
                       (a.addr.srcBH == 0 || a.addr.srcBH == a.B * a.H) && a.addr.out_acc == 0 && a.qlo == nullptr && !a.p_anti && !a.p_given && !a.lo_state && a.vs.split == 0;
    return plain && a.in_bf16 && a.out != nullptr && (a.DK == 64 || a.DK == 256) && (a.chunk == 64 || a.chunk == 128) &&
           seg_width(a.DV) != 0;
}

// A state-only call (no output) with plain operands that the segment-state kernel serves.
bool chunkwise_seg_state_supported(const LaunchArgs& a) {
    const bool plain = a.addr.rev == 0 && (a.addr.ldqk == 0 || a.addr.ldqk == a.DK) && a.addr.qcol_blk == 0 &&
                       (a.addr.srcBH == 0 || a.addr.srcBH == a.B * a.H) && a.addr.out_acc == 0 && a.qlo == nullptr && !a.p_anti && !a.p_given && !a.lo_state && a.vs.split == 0;
    return plain && a.in_bf16 && a.out == nullptr && a.state_out != nullptr && (a.DK == 64 || a.DK == 256) && seg_width(a.DV) != 0;
}

// Bytes of the segment states of a state-only call (none with a single segment).
size_t chunkwise_seg_state_only_bytes(int B, int H, int N, int DK, int DV) {
    const int W = seg_width(DV);
    if (!W) return 0;
    const int segs = seg_count(B * H, DV / W, (N + 127) / 128);
    return segs > 1 ? (size_t)B * H * segs * DK * DV * sizeof(float) : 0;
}

hipError_t launch_chunkwise_seg_state(const LaunchArgs& a, float* U) {
    if (a.DK == 64) return seg_width(a.DV) == 128 ? seg_state_launch_t<64, 128>(a, U) : seg_state_launch_t<64, 64>(a, U);
    return seg_width(a.DV) == 128 ? seg_state_launch_t<256, 128>(a, U) : seg_state_launch_t<256, 64>(a, U);
}

// Bytes of the segment states U (the call's pre-norm rows, if any, are laid out by the caller).
size_t chunkwise_seg_state_bytes(int B, int H, int N, int DK, int DV, int chunk) {
    const int W = seg_width(DV);
    if (!W) return 0;
    const int nchunks = (N + chunk - 1) / chunk;
    const int segs = seg_count(B * H, DV / W, nchunks);
    return (size_t)B * H * (segs - 1) * DK * DV * sizeof(float);
}

// out: the call's output, or the fp32 pre-norm rows when a GroupNorm pass follows (out_f32 set).
hipError_t launch_chunkwise_seg(const LaunchArgs& a, float* U, void* out, bool out_f32) {
    if (a.DK == 64) return out_f32 || !a.out_bf16 ? seg_launch_dk<64, float>(a, U, out) : seg_launch_dk<64, bf16>(a, U, out);
    return out_f32 || !a.out_bf16 ? seg_launch_dk<256, float>(a, U, out) : seg_launch_dk<256, bf16>(a, U, out);
}

}  // namespace ret

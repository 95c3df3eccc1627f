// Internal header of the gfx950 retention library: types, MFMA wrappers, LDS transpose reads,
// decay helpers and the launch-argument block shared by the kernels and the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ret {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxHeads = 128;
constexpr int kWave = 64;

// Per-head decay constants, passed by value as a kernel argument. gamma is the fp32 rounding of
// the caller's fp64 value; log2g = log2(gamma) computed in fp64 on the host, then rounded.
struct HeadConsts {
    float gamma[kMaxHeads];
    float log2g[kMaxHeads];
};

struct GnArgs {
    int enabled;
    float eps;
    const float* weight;  // [H][dv] or nullptr
    const float* bias;    // [H][dv] or nullptr
    const void* gate;     // laid out like the output, input dtype, or nullptr
    int gate_bf16;
};

// Everything a launcher needs; filled and validated by the C-ABI layer.
// Operand addressing of a bf16 chunkwise forward, for callers that read operands in place (the
// backward). Zero fields mean the defaults: contiguous [B][H][N][d] tensors walked in time order.
//   rev       token t of the walk is row N-1-t of q, k, v and out
//   ldqk      elements between consecutive q rows (and k rows); 0: d_k
//   qcol_blk  the workgroups of stacked head index bh read q and k from column (bh / srcBH) * qcol_blk
//   srcBH     q, k and v of stacked head index bh are those of head bh % srcBH; 0: B * H
//   out_acc   fp32 out only: out rows of stacked head index bh are those of head bh % srcBH, and
//             the forward adds its values to them atomically instead of storing them. out must
//             start at zero; with two stacked blocks the result is order independent (a + b).
// P, the states and (without out_acc) out are laid out by the stacked head index.
struct OpAddr {
    int rev, ldqk, qcol_blk, srcBH, out_acc;
};

// Value rows read with a shift (chunkwise kernels; residual linear attention): row t of the value
// operand is row t of pre (laid out [B*H][split][DV]) for t < split, and row t - shift of v for
// t >= split. split is a multiple of 32 (a stage) or N, and split >= shift. split = 0: plain v.
struct VShift {
    const void* pre;
    int split, shift;
};

struct RotConsts;
struct StepRot;
struct LaunchArgs {
    int B, H, N, DK, DV;
    int in_bf16, out_bf16;
    int chunk;
    OpAddr addr;  // bf16 chunkwise only
    VShift vs;    // chunkwise only
    const void* q;
    const void* qlo;  // bf16 chunkwise with an fp32 output only: low part of q, or null
    // bf16 chunkwise with an output, N a multiple of the chunk: p_anti receives the scores of this
    // call anti-transposed (the scores of the time-reversed call with q and k exchanged), laid out
    // as the workspace's scores (chunkwise_bf16_scores_bytes); p_given supplies such scores instead
    // of computing them. Both null: the call computes its own.
    void* p_anti;
    const void* p_given;
    // bf16 chunkwise, q as two parts (qlo), fp32 out: no intra-chunk term (no scores, no P V): the
    // output is g^(j+1) Q R alone, for a split call whose intra-chunk term another call carries
    int no_pv;
    // bf16 chunkwise, fp32 out, no GroupNorm, chunks up to 256: the call is the correction term of a
    // split whose k is the low part of a k that bf16 does not hold; its state term (V (.) zeta and R)
    // enters the matrix cores as single bf16 values, P V as before
    int lo_state;
    // decode step: cos and sin of each pair's angle at the step's position (host memory; null: no
    // rotation); the kernel turns q and k with them
    const StepRot* step_rot;
    // bf16 parallel form: > 0 keeps only the keys of each query's own chunk of this many tokens (a
    // multiple of 64): the intra-chunk term of the chunkwise form
    int intra_chunk;
    const void* k;
    const void* v;
    void* out;              // may be null (chunkwise state-only)
    const float* state_in;  // may be null
    float* state_out;       // may be null; the decode step uses it as its in/out state
    GnArgs gn;
    HeadConsts hc;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

// g^e for a per-head log2(g), with the hardware exp2 (v_exp_f32, about 1 ulp): exactly 1 at e = 0;
// results below the normal range flush to 0, which is below anything they are added to here.
__device__ __forceinline__ float decay_pow(float log2g, float e) { return __builtin_amdgcn_exp2f(e * log2g); }

// 16x16x32 bf16 MFMA, fp32 accumulate. Operand layouts (lane l of 64, checked on gfx950):
//   A[m][k]: lane holds m = l%16, k = 8*(l/16) + j (j = 0..7)
//   B[k][n]: lane holds k = 8*(l/16) + j, n = l%16
//   D[m][n]: lane holds m = 4*(l/16) + i (i = 0..3), n = l%16
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the 4-element
// rows addressed by lanes 4r + i/4, for r = 0..3 (checked on gfx950).
__device__ __forceinline__ s16x4 lds_read_tr16(const bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// An MFMA operand whose contraction index runs down the rows of a row-major bf16 matrix X in LDS
// (X[r][c] at base[r*ld + c]): the fragment for rows r0..r0+31 and columns c0..c0+15, i.e.
// lane l gets X[r0 + 8*(l/16) + j][c0 + l%16], j = 0..7. Serves as the B operand of X (k = rows)
// or as the A operand of X^T (m = columns). Two transposing 8-byte reads per lane.
__device__ __forceinline__ bf16x8 lds_frag_kmajor(const bf16* base, int ld, int r0, int c0, int lane) {
    const int g = lane >> 4, p = lane & 15;
    const bf16* a0 = base + (size_t)(r0 + 8 * g + (p >> 2)) * ld + c0 + 4 * (p & 3);
    s16x4 lo = lds_read_tr16(a0);
    s16x4 hi = lds_read_tr16(a0 + 4 * ld);
    bf16x8 r;
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
    r[0] = l4[0]; r[1] = l4[1]; r[2] = l4[2]; r[3] = l4[3];
    r[4] = h4[0]; r[5] = h4[1]; r[6] = h4[2]; r[7] = h4[3];
    return r;
}

// The operand whose contraction index runs along the rows' contiguous dimension: lane l gets
// X[r0 + l%16][c0 + 8*(l/16) + j], j = 0..7 (one 16-byte read). A operand of X (m = rows) or
// B operand of X^T (n = rows).
__device__ __forceinline__ bf16x8 frag_rowmajor(const bf16* base, size_t ld, int r0, int c0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (size_t)(r0 + (lane & 15)) * ld + c0 + 8 * (lane >> 4));
}

// Swizzled LDS tiles: rows of RB bytes (RB a multiple of 128), the 16-byte chunk c of row r stored
// at byte r*RB + 16*(c ^ (r & M)), M = min(RB/16, 16) - 1. A fragment read of 16 rows at one chunk,
// or a transposing read of 4 rows x 2 chunks, then touches distinct banks (measured on gfx950:
// padding rows by 16 bytes instead still conflicts for 16-row reads). A tile is filled 1 KB at a
// time by buffer-to-LDS loads, lane l of a wave writing bytes [16l, 16l + 16) of its kilobyte.
template <int RB>
struct SwzTile {
    static_assert(RB % 128 == 0, "rows of whole 128-byte lines");
    static constexpr int M = (RB / 16 < 16 ? RB / 16 : 16) - 1;
    __device__ static __forceinline__ int off(int r, int c) { return r * RB + 16 * (c ^ (r & M)); }
};

// frag_rowmajor on a swizzled tile (c0 a multiple of 8).
template <int RB>
__device__ __forceinline__ bf16x8 frag_rowmajor_swz(const char* base, int r0, int c0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + SwzTile<RB>::off(r0 + (lane & 15), (c0 >> 3) + (lane >> 4)));
}

// lds_frag_kmajor on a swizzled tile (c0 a multiple of 16).
template <int RB>
__device__ __forceinline__ bf16x8 lds_frag_kmajor_swz(const char* base, int r0, int c0, int lane) {
    const int g = lane >> 4, p = lane & 15;
    const int row = r0 + 8 * g + (p >> 2), col = c0 + 4 * (p & 3);
    const int sub = (col & 7) * 2;
    s16x4 lo = lds_read_tr16(reinterpret_cast<const bf16*>(base + SwzTile<RB>::off(row, col >> 3) + sub));
    s16x4 hi = lds_read_tr16(reinterpret_cast<const bf16*>(base + SwzTile<RB>::off(row + 4, col >> 3) + sub));
    bf16x8 r;
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
    const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
    r[0] = l4[0]; r[1] = l4[1]; r[2] = l4[2]; r[3] = l4[3];
    r[4] = h4[0]; r[5] = h4[1]; r[6] = h4[2]; r[7] = h4[3];
    return r;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = (bf16)0.0f;
    return z;
}

__device__ __forceinline__ void split_hi_lo(float x, bf16& hi, bf16& lo) {
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
}

// Swish gate of the GroupNorm output (abeam.tech RetNet summary, "Multi-timescale decay, gate and
// normalisation"): x * sigmoid(x), with the hardware exp2 and reciprocal (about 1 ulp each);
// exp overflow for very negative x gives 0 * x, the limit.
__device__ __forceinline__ float swish(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}
// Element i of the gate tensor, in its dtype
__device__ __forceinline__ float gate_at(const struct GnArgs& gn, size_t i) {
    return gn.gate_bf16 ? (float)reinterpret_cast<const __bf16*>(gn.gate)[i] : reinterpret_cast<const float*>(gn.gate)[i];
}

template <typename T> __device__ __forceinline__ T from_float(float x);
template <> __device__ __forceinline__ float from_float<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_float<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ float to_float(T x) { return (float)x; }

// Sum over the 16 lanes that share l/16 (lanes differing in bits 0..3). Symmetric butterfly:
// every lane ends with the bitwise-same value.
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

// Positional rotation (rotary embedding) of q and k: feature pair i of the row at position
// offset + n turns by (offset + n) * theta_i. Formed on the host in double precision per call:
// fhi + flo = theta_i / pi (half-turns per position, split into two floats) and
// ph = (offset * theta_i / pi) mod 2.
constexpr int kMaxPairs = 128;
struct RotConsts {
    float fhi[kMaxPairs];
    float flo[kMaxPairs];
    float ph[kMaxPairs];
};

// The decode step's rotation: one position (the offset) per call, so each pair's turn is a fixed
// cos and sin, evaluated on the host in double precision from the same angle as RotConsts and
// rounded once to float.
struct StepRot {
    float cs[kMaxPairs];
    float sn[kMaxPairs];
};

// A kernel parameter that only instantiations with a rotation carry: IfRot<ROT, T>::type is T when
// ROT, else an empty struct.
struct NoRot {};
template <bool ROT, typename T> struct IfRot { typedef NoRot type; };
template <typename T> struct IfRot<true, T> { typedef T type; };

// sin and cos of the angle of pair (fhi, flo, ph) at local position n (0 <= n < 2^24, exact in
// fp32). The phase in half-turns is ph + n * (fhi + flo) mod 2: the product n * fhi is split into
// its rounded value and its exact rounding error (fma), the rounded value is reduced mod 2 exactly,
// and sincospif gives sin and cos of pi times the phase. Contraction is off so that the split
// stays exact as written.
__device__ __forceinline__ void rot_sincos(int n, float fhi, float flo, float ph, float& s, float& c) {
#pragma clang fp contract(off)
    const float nf = (float)n;
    float p = nf * fhi;
    const float e = __builtin_fmaf(nf, fhi, -p);
    p = p - 2.f * __builtin_floorf(0.5f * p);
    const float h = p + (e + __builtin_fmaf(nf, flo, ph));
    sincospif(h, &s, &c);
}

}  // namespace ret

// Backward of the chunkwise form: gradients for dL/dout = dout, in fp32.
namespace ret {
struct BwdArgs {
    LaunchArgs base;  // shape, input dtype, chunk, decay constants, workspace, stream
    const void* q;
    const void* k;
    const void* v;
    const void* dout;       // laid out like v, input dtype
    const float* state_in;  // may be null
    float* dq;              // each may be null
    float* dk;
    float* dv;
    float* dstate_in;
};
}  // namespace ret

// Launchers (one per kernel family), called by the C-ABI layer after validation.
namespace ret {
void set_last_error(const char* msg);  // the message retention_last_error() returns
hipError_t launch_recurrent_step(const LaunchArgs& a);
hipError_t launch_chunkwise_bf16(const LaunchArgs& a);
hipError_t launch_parallel_bf16(const LaunchArgs& a);
hipError_t launch_chunkwise_f32(const LaunchArgs& a);
hipError_t launch_parallel_f32(const LaunchArgs& a);
size_t chunkwise_bf16_workspace(int B, int H, int N, int DK, int DV, int chunk, int gn, int want_out);
size_t chunkwise_f32_workspace(int B, int H, int N, int DV, int gn, int out_bf16);
size_t parallel_f32_workspace(int B, int H, int N, int DV, int gn, int out_bf16);
bool chunkwise_bf16_supported(int DK, int DV, int chunk);
// Whether a bf16 chunkwise call with an fp32 output and no GroupNorm takes q as two parts
// (LaunchArgs::qlo) at this d_k and chunk: the warp-specialised kernel, when its stage buffers with
// the second q plane fit in LDS.
bool chunkwise_bf16_qlo_supported(int DK, int chunk);
// Bytes of the scores (both parts) a bf16 chunkwise call with an output keeps, for p_anti / p_given,
// and whether it keeps them as high and low parts (p_anti and p_given need that).
size_t chunkwise_bf16_scores_bytes(int B, int H, int N, int DK, int chunk);
bool chunkwise_bf16_scores_split(int DK, int chunk);
// The two-call split of a bf16 chunkwise call on (q_hi + q_lo, k_hi + k_lo) at this d_k and chunk:
// the scores of all three products from one kernel (launch_chunkwise_bf16_scores with qlo and klo)
// go to the (q_hi, k_lo) call (p_given), and the (q_hi + q_lo, k_hi) call runs without P (no_pv).
bool chunkwise_bf16_split2_supported(int DK, int chunk);
// The scores kernel alone (plain operands, a.B, a.H, a.N, a.DK, a.chunk, a.hc): P = q k^T (+ qlo k^T
// with qlo, + q klo^T with klo) as bf16 high and low planes at P (chunkwise_bf16_scores_bytes).
hipError_t launch_chunkwise_bf16_scores(const LaunchArgs& a, const void* q, const void* qlo, const void* k, const void* klo, void* P);
// The same scores of the rotated q and k from unrotated q and k (plain addressing): the kernel
// turns them itself and also writes the rotated operands as bf16 high and low parts, planes =
// {q_hi, q_lo, k_hi, k_lo}, each [B*H][N][DK].
hipError_t launch_chunkwise_bf16_scores_rot(const LaunchArgs& a, const void* q, const void* k, const RotConsts& rc, void* const planes[4],
                                            void* P);
// The segmented bf16 chunkwise kernels (chunk_seg.hip): plain operands, an output, d_k 64 or 256,
// chunk 64 or 128, d_v a multiple of 64. U: the segment states in the workspace; out: the call's
// output, or fp32 pre-norm rows when out_f32 (a GroupNorm pass follows).
bool chunkwise_seg_supported(const LaunchArgs& a);
size_t chunkwise_seg_state_bytes(int B, int H, int N, int DK, int DV, int chunk);
hipError_t launch_chunkwise_seg(const LaunchArgs& a, float* U, void* out, bool out_f32);
// State-only calls (no output, state_out given) on the segment-state kernel: plain operands, bf16,
// d_k 64 or 256, d_v a multiple of 64, any chunk length. U: the segment states in the workspace.
bool chunkwise_seg_state_supported(const LaunchArgs& a);
size_t chunkwise_seg_state_only_bytes(int B, int H, int N, int DK, int DV);
hipError_t launch_chunkwise_seg_state(const LaunchArgs& a, float* U);
bool chunkwise_f32_supported(int DK, int DV, int chunk);
bool parallel_bf16_supported(int DK, int DV);
bool parallel_f32_supported(int DK, int DV);
int bwd_split(int in_bf16, int DK, int DV, int chunk);  // 0: unsupported
size_t chunkwise_bwd_workspace(int in_bf16, int B, int H, int N, int DK, int DV, int chunk);
hipError_t launch_chunkwise_bwd(const BwdArgs& b);
// y = rotation of x ([rows][N][d], d even, row r at local position r % N); x and y may be the same
// buffer. inverse != 0 turns by the opposite angles.
hipError_t launch_rotate(long rows, int N, int d, const void* x, int x_bf16, void* y, int y_bf16, const RotConsts& rc,
                         int inverse, hipStream_t stream);
// Two tensors of the same shape in one launch (x0 -> y0, x1 -> y1; x1 may be null). With bf16
// outputs, lo0 / lo1 (when not null) also receive the low parts of the turned values (value minus
// its bf16 rounding, rounded to bf16).
hipError_t launch_rotate2(long rows, int N, int d, const void* x0, void* y0, const void* x1, void* y1, int x_bf16, int y_bf16,
                          const RotConsts& rc, int inverse, hipStream_t stream, void* lo0 = nullptr, void* lo1 = nullptr);
// The per-head GroupNorm (and gate) over fp32 pre-norm rows [rows][DV], into y (fp32 or bf16).
hipError_t launch_gn_rows(long rows, int H, int N, int DV, const float* pre, void* y, bool y_bf16, const GnArgs& gn,
                          hipStream_t stream);
// Residual linear attention operands: qo = phi(q) (qo null: phi is the identity and q is used as
// is), ko = phi(k) shifted by P = window + 1 rows, and vo = the first vsplit rows of v shifted the
// same way ([rows / N][vsplit][dv]; the chunk kernels read the later rows from v, see VShift); the
// first P rows come from the window rows kp, vp ([rows / N][P][d], of which the last prev_len hold
// tokens) or are zero.
struct RlaPrep {
    long rows;  // B * H * N
    int N, dk, dv, P, prev_len, fmap, bf16;
    int feat_f32;  // bf16 inputs: features and value rows written in fp32 (else in the input dtype)
    int vsplit;    // shifted value rows written per head ([B*H][vsplit][dv] at vo)
    const void *q, *k, *v, *kp, *vp;
    void *qo, *ko, *vo;
    void *qlo, *klo;  // bf16 features: the low parts (feature - its bf16 rounding, rounded), or null
};
hipError_t launch_rla_prepare(const RlaPrep& r, hipStream_t stream);
// out = a + b + c over n values (c may be null; out may be a), fp32 sums, stored in fp32 or bf16;
// n a multiple of 4, every pointer 16-byte aligned.
hipError_t launch_add_rows(size_t n, const float* a, const float* b, const float* c, void* out, bool out_bf16, hipStream_t stream);
// dst = src, or zero when src is null (n floats, a multiple of 4, 16-byte aligned).
hipError_t launch_copy_state(size_t n, const float* src, float* dst, hipStream_t stream);
}  // namespace ret

// C-ABI entry points of the retention library (declared in include/retention.h): argument
// validation on the host before any HIP call, per-head decay constants in fp64, workspace sizing,
// and dispatch to the kernel launchers. No exception crosses the boundary; errors are returned
// as ret_status with a thread-local message.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/retention.h"
#include "common.hpp"
#include "entry.hpp"

namespace {

thread_local char g_err[512] = "";

ret_status fail(ret_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int32_t dt) { return dt == RET_BF16 ? 2 : 4; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

ret_status check_shape(const ret_shape* s, bool step) {
    if (!s) return fail(RET_ERR_INVALID_ARG, "shape is NULL");
    if (s->batch <= 0 || s->heads <= 0 || s->seq_len <= 0 || s->d_k <= 0 || s->d_v <= 0)
        return fail(RET_ERR_INVALID_ARG, "non-positive dimension (batch %d heads %d seq_len %d d_k %d d_v %d)", s->batch, s->heads,
                    s->seq_len, s->d_k, s->d_v);
    if ((s->in_dtype != RET_F32 && s->in_dtype != RET_BF16) || (s->out_dtype != RET_F32 && s->out_dtype != RET_BF16))
        return fail(RET_ERR_INVALID_ARG, "dtype must be RET_F32 (0) or RET_BF16 (1) (in %d out %d)", s->in_dtype, s->out_dtype);
    if (step && s->seq_len != 1) return fail(RET_ERR_INVALID_ARG, "recurrent step needs seq_len == 1 (got %d)", s->seq_len);
    const double elems = (double)s->batch * s->heads * s->seq_len * (double)(s->d_k > s->d_v ? s->d_k : s->d_v);
    const double states = (double)s->batch * s->heads * (double)s->d_k * s->d_v;
    if (elems > 9.0e15 || states > 9.0e15) return fail(RET_ERR_INVALID_ARG, "tensor sizes overflow");
    if (s->heads > RETENTION_MAX_HEADS)
        return fail(RET_ERR_UNSUPPORTED, "heads %d exceeds RETENTION_MAX_HEADS (%d)", s->heads, RETENTION_MAX_HEADS);
    return RET_OK;
}

// The bf16 chunk kernels address one head's rows (q, k, v and out up to 4 bytes per element, or rows
// of the wider operand in the backward) and its scores in 32-bit byte offsets: every such extent,
// with the sequence padded to whole chunks, must stay below 2^31 bytes.
bool bf16_head_fits(const ret_shape* s, int chunk) {
    const double n_pad = std::ceil((double)s->seq_len / chunk) * chunk;
    const double widest = (double)(s->d_k > s->d_v ? s->d_k : s->d_v);
    return n_pad * widest * 4.0 < 2147483648.0 && n_pad * chunk * 2.0 < 2147483648.0;
}

ret_status check_bf16_head(const ret_shape* s, int chunk) {
    if (s->in_dtype != RET_BF16 || chunk <= 0 || bf16_head_fits(s, chunk)) return RET_OK;
    return fail(RET_ERR_UNSUPPORTED, "seq_len %d is too long for the bf16 chunk kernels at d_k %d, d_v %d, chunk %d: one head's rows "
                "and scores must stay below 2^31 bytes (about 1M tokens at d_v 512)", s->seq_len, s->d_k, s->d_v, chunk);
}

ret_status check_gamma(const ret_shape* s, const double* gamma, ret::HeadConsts* hc) {
    if (!gamma) return fail(RET_ERR_INVALID_ARG, "gamma is NULL");
    for (int h = 0; h < s->heads; ++h) {
        const double g = gamma[h];
        if (!(g > 0.0 && g <= 1.0)) return fail(RET_ERR_INVALID_ARG, "gamma[%d] = %g is not in (0, 1]", h, g);
        hc->gamma[h] = (float)g;
        hc->log2g[h] = (float)std::log2(g);
    }
    for (int h = s->heads; h < ret::kMaxHeads; ++h) {
        hc->gamma[h] = 1.f;
        hc->log2g[h] = 0.f;
    }
    return RET_OK;
}

ret_status check_gn(const ret_groupnorm* gn, int in_bf16, ret::GnArgs* out) {
    out->enabled = 0;
    out->eps = 0.f;
    out->weight = nullptr;
    out->bias = nullptr;
    out->gate = nullptr;
    out->gate_bf16 = in_bf16;
    if (gn && !gn->enabled && gn->gate) return fail(RET_ERR_INVALID_ARG, "a gate needs the GroupNorm epilogue (enabled = 1)");
    if (!gn || !gn->enabled) return RET_OK;
    if (!(gn->eps > 0.f) || !std::isfinite(gn->eps)) return fail(RET_ERR_INVALID_ARG, "groupnorm eps must be finite and > 0");
    if ((gn->weight && !aligned16(gn->weight)) || (gn->bias && !aligned16(gn->bias)))
        return fail(RET_ERR_INVALID_ARG, "groupnorm weight/bias must be 16-byte aligned");
    if (gn->gate && !aligned16(gn->gate)) return fail(RET_ERR_INVALID_ARG, "gate must be 16-byte aligned");
    out->enabled = 1;
    out->eps = gn->eps;
    out->weight = gn->weight;
    out->bias = gn->bias;
    out->gate = gn->gate;
    return RET_OK;
}

// Rotation constants per feature pair, in double precision: theta_i / pi split into two floats,
// and the offset's phase (offset * theta_i / pi mod 2) from an exact two-product and an exact fmod.
// step (optional): cos and sin of pi times that phase, for the decode step's single position.
ret_status check_rotation(const ret_rotation* r, const ret_shape* s, ret::RotConsts* rc, bool* on,
                          ret::StepRot* step = nullptr) {
    *on = false;
    if (!r || !r->enabled) return RET_OK;
    if (!(r->base > 0.0) || !std::isfinite(r->base)) return fail(RET_ERR_INVALID_ARG, "rotation base must be finite and > 0");
    if (r->offset < 0 || r->offset >= (1LL << 31))
        return fail(RET_ERR_INVALID_ARG, "rotation offset must be in [0, 2^31) (got %lld)", (long long)r->offset);
    if (s->d_k % 2) return fail(RET_ERR_INVALID_ARG, "rotation needs an even d_k (got %d)", s->d_k);
    if (s->d_k / 2 > ret::kMaxPairs) return fail(RET_ERR_UNSUPPORTED, "rotation supports d_k <= %d (got %d)", 2 * ret::kMaxPairs, s->d_k);
    if (s->seq_len >= (1 << 24)) return fail(RET_ERR_UNSUPPORTED, "rotation supports seq_len < 2^24 (got %d)", s->seq_len);
    const int d = s->d_k;
    const double off = (double)r->offset;
    for (int i = 0; i < ret::kMaxPairs; ++i) {
        if (i >= d / 2) {
            rc->fhi[i] = rc->flo[i] = rc->ph[i] = 0.f;
            if (step) step->cs[i] = step->sn[i] = 0.f;
            continue;
        }
        const double f = std::pow(r->base, -2.0 * i / d) / M_PI;
        const float hi = (float)f;
        rc->fhi[i] = hi;
        rc->flo[i] = (float)(f - (double)hi);
        const double p = off * f;
        const double e = std::fma(off, f, -p);
        double ph = std::fmod(p, 2.0) + e;
        ph -= 2.0 * std::floor(0.5 * ph);
        rc->ph[i] = (float)ph;
        if (step) {
            step->cs[i] = (float)std::cos(M_PI * ph);
            step->sn[i] = (float)std::sin(M_PI * ph);
        }
    }
    *on = true;
    return RET_OK;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Workspace for the rotated q and k, in front of the call's own workspace.
size_t rotation_ws(const ret_shape* s) {
    return 2 * align256((size_t)s->batch * s->heads * s->seq_len * s->d_k * elem_size(s->in_dtype));
}

// Rotate q and k into the front of the workspace; q, k and the workspace then point at the
// rotated copies and the rest of the workspace.
hipError_t stage_rotation(const ret_shape* s, const ret::RotConsts& rc, const void** q, const void** k, void** ws, size_t* wsb,
                          hipStream_t st) {
    const size_t A = rotation_ws(s) / 2;
    char* base = static_cast<char*>(*ws);
    const long rows = (long)s->batch * s->heads * s->seq_len;
    const int bf = s->in_dtype == RET_BF16;
    const hipError_t e = ret::launch_rotate2(rows, s->seq_len, s->d_k, *q, base, *k, base + A, bf, bf, rc, 0, st);
    if (e != hipSuccess) return e;
    *q = base;
    *k = base + A;
    *ws = base + 2 * A;
    *wsb -= 2 * A;
    return hipSuccess;
}

// ---- q and k carried as bf16 high + low parts (rotated operands of the bf16 forward forms, and
// RLA's softmax features). A retention call is bilinear in (q, k) and linear in state_in, so three
// bf16 calls on the parts give
//     out = A(q_hi, k_hi) + A(q_hi, k_lo) + A(q_lo, k_hi)     (lo x lo, about 2^-16 relative, dropped)
// with state_in entering the calls on q_hi and q_lo once each, and the final state the sum of the
// states of the calls on k_hi and k_lo. The partial outputs are fp32; a GroupNorm (and gate)
// follows their sum. The chunkwise kernels add the second and third calls' rows into the first's
// (OpAddr::out_acc: one atomic add per element and call, the calls in stream order, so the sum is
// the same every time); the parallel kernel writes three partial outputs that a last pass adds.

// Bytes of the partial results. Summed by a last pass (acc false): the fp32 partial outputs (two;
// three when the sum cannot go to out directly, i.e. a bf16 output or a GroupNorm after it). Added
// in place (acc true): one fp32 output when the sum cannot go to out directly, else none. Then the
// second partial state, then (acc, two calls at this chunk) the scores of the three products.
size_t split_parts_bytes(const ret_shape* s, bool gn, bool acc, int chunk) {
    const size_t rows = (size_t)s->batch * s->heads * s->seq_len;
    const size_t o = align256(rows * s->d_v * sizeof(float));
    const bool staged = s->out_dtype == RET_BF16 || gn;
    const size_t outs = acc ? (staged ? 1 : 0) : (staged ? 3 : 2);
    const size_t p = acc && ret::chunkwise_bf16_split2_supported(s->d_k, chunk)
                         ? align256(ret::chunkwise_bf16_scores_bytes(s->batch, s->heads, s->seq_len, s->d_k, chunk))
                         : 0;
    return outs * o + align256((size_t)s->batch * s->heads * s->d_k * s->d_v * sizeof(float)) + p;
}

// Rotated q and k of a bf16 forward call as high and low parts: four planes.
size_t rotation_split_ws(const ret_shape* s) { return 2 * rotation_ws(s); }

// Places the four planes (q_hi, q_lo, k_hi, k_lo) at the front of *ws and advances it past them.
void place_rotation_split(const ret_shape* s, void* parts[4], void** ws, size_t* wsb) {
    const size_t A = rotation_ws(s) / 2;
    char* base = static_cast<char*>(*ws);
    for (int i = 0; i < 4; ++i) parts[i] = base + i * A;
    *ws = base + 4 * A;
    *wsb -= 4 * A;
}

// Writes the four planes (q_hi, q_lo, k_hi, k_lo) at the front of *ws and advances it past them.
hipError_t stage_rotation_split(const ret_shape* s, const ret::RotConsts& rc, const void* q, const void* k, const void* parts[4],
                                void** ws, size_t* wsb, hipStream_t st) {
    void* pl[4];
    place_rotation_split(s, pl, ws, wsb);
    const long rows = (long)s->batch * s->heads * s->seq_len;
    const hipError_t e = ret::launch_rotate2(rows, s->seq_len, s->d_k, q, pl[0], k, pl[2], 1, 1, rc, 0, st, pl[1], pl[3]);
    if (e != hipSuccess) return e;
    for (int i = 0; i < 4; ++i) parts[i] = pl[i];
    return hipSuccess;
}

// The rotation of a split call done by its scores kernel: the unrotated q and k, the constants,
// and the planes that kernel writes (then read by the chunk passes as qh, ql, kh, kl).
struct FusedRot {
    const void* q;
    const void* k;
    const ret::RotConsts* rc;
    void* planes[4];
};

// The partial calls and the sums. a: the call (q and k unset; out, state_in, state_out, gn and
// out_bf16 as the caller asked), parts: split_parts_bytes(shape, gn, acc, chunk) of workspace; launch: the
// bf16 kernel family (chunkwise, which adds the partial outputs in place (acc), or parallel). Where
// the chunkwise kernel takes q as two parts, A(q_hi, k_hi) + A(q_lo, k_hi) is one call on
// (q_hi + q_lo, k_hi). An in-place state_in is read by the calls that need it before the last call
// writes state_out.
hipError_t run_split(const ret::LaunchArgs& a, const void* qh, const void* ql, const void* kh, const void* kl, char* parts,
                     hipError_t (*launch)(const ret::LaunchArgs&), bool acc, const FusedRot* fr = nullptr) {
    const size_t rows = (size_t)a.B * a.H * a.N;
    const size_t ob = align256(rows * a.DV * sizeof(float));
    const bool staged = a.out_bf16 || a.gn.enabled;  // the sum goes through the workspace
    ret::LaunchArgs c = a;
    c.out_bf16 = 0;
    c.gn = ret::GnArgs{};
    hipError_t e;
    if (acc) {
        float* o = staged ? reinterpret_cast<float*>(parts) : static_cast<float*>(a.out);
        float* s2 = reinterpret_cast<float*>(parts + (staged ? ob : 0));
        char* sc = parts + (staged ? ob : 0) + align256((size_t)a.B * a.H * a.DK * a.DV * sizeof(float));
        if (a.out && ret::chunkwise_bf16_split2_supported(a.DK, a.chunk)) {
            // two calls sharing one scores pass over all three products: (q_hi, k_lo) with those
            // scores stores its rows and its state; (q_hi + q_lo, k_hi) without an intra-chunk term
            // adds its rows and writes the state from state_in
            e = fr ? ret::launch_chunkwise_bf16_scores_rot(a, fr->q, fr->k, *fr->rc, fr->planes, sc)
                   : ret::launch_chunkwise_bf16_scores(a, qh, ql, kh, kl, sc);
            if (e != hipSuccess) return e;
            c.q = qh; c.k = kl; c.p_given = sc; c.out = o; c.state_in = nullptr; c.state_out = a.state_out ? s2 : nullptr;
            c.lo_state = 1;  // its state term is about 2^-8 of the result: single bf16 parts suffice
            if ((e = launch(c)) != hipSuccess) return e;
            c.p_given = nullptr;
            c.lo_state = 0;
            c.addr.out_acc = 1;
            c.no_pv = 1;
            c.q = qh; c.qlo = ql; c.k = kh; c.state_in = a.state_in; c.state_out = a.state_out;
            if ((e = launch(c)) != hipSuccess) return e;
        } else if (fr) {
            return hipErrorInvalidValue;  // the planes are written only by the two-call split's scores
        } else if (a.out && ret::chunkwise_bf16_qlo_supported(a.DK, a.chunk)) {
            // two calls: (q_hi, k_lo) stores its rows and its state; (q_hi + q_lo, k_hi), on the
            // kernel that takes q as two parts, adds its rows and writes the state from state_in
            c.q = qh; c.k = kl; c.out = o; c.state_in = nullptr; c.state_out = a.state_out ? s2 : nullptr;
            if ((e = launch(c)) != hipSuccess) return e;
            c.addr.out_acc = 1;
            c.q = qh; c.qlo = ql; c.k = kh; c.state_in = a.state_in; c.state_out = a.state_out;
            if ((e = launch(c)) != hipSuccess) return e;
        } else {
            // three calls: the first stores its rows, the next two add theirs:
            // ((q_lo, k_hi) + (q_hi, k_lo)) + (q_hi, k_hi)
            if (a.out) {
                c.q = ql; c.k = kh; c.out = o; c.state_in = a.state_in; c.state_out = nullptr;
                if ((e = launch(c)) != hipSuccess) return e;
            }
            c.addr.out_acc = a.out != nullptr;
            if (a.out || a.state_out) {
                c.q = qh; c.k = kl; c.out = a.out ? o : nullptr; c.state_in = nullptr; c.state_out = a.state_out ? s2 : nullptr;
                if ((e = launch(c)) != hipSuccess) return e;
            }
            c.q = qh; c.k = kh; c.out = a.out ? o : nullptr; c.state_in = a.state_in; c.state_out = a.state_out;
            if ((e = launch(c)) != hipSuccess) return e;
        }
        if (a.out && a.gn.enabled) {
            if ((e = ret::launch_gn_rows((long)rows, a.H, a.N, a.DV, o, a.out, a.out_bf16, a.gn, a.stream)) != hipSuccess) return e;
        } else if (a.out && staged) {
            if ((e = ret::launch_add_rows(rows * a.DV, o, nullptr, nullptr, a.out, true, a.stream)) != hipSuccess) return e;
        }
        if (a.state_out)
            return ret::launch_add_rows((size_t)a.B * a.H * a.DK * a.DV, a.state_out, s2, nullptr, a.state_out, false, a.stream);
        return hipSuccess;
    }
    float* o2 = reinterpret_cast<float*>(parts);
    float* o3 = reinterpret_cast<float*>(parts + ob);
    float* o1 = staged ? reinterpret_cast<float*>(parts + 2 * ob) : static_cast<float*>(a.out);
    float* s2 = reinterpret_cast<float*>(parts + (staged ? 3 : 2) * ob);
    if (a.out) {
        c.q = ql; c.k = kh; c.out = o3; c.state_in = a.state_in; c.state_out = nullptr;
        if ((e = launch(c)) != hipSuccess) return e;
    }
    if (a.out || a.state_out) {
        c.q = qh; c.k = kl; c.out = a.out ? o2 : nullptr; c.state_in = nullptr; c.state_out = a.state_out ? s2 : nullptr;
        if ((e = launch(c)) != hipSuccess) return e;
    }
    c.q = qh; c.k = kh; c.out = a.out ? o1 : nullptr; c.state_in = a.state_in; c.state_out = a.state_out;
    if ((e = launch(c)) != hipSuccess) return e;
    if (a.out) {
        if (a.gn.enabled) {
            if ((e = ret::launch_add_rows(rows * a.DV, o1, o2, o3, o1, false, a.stream)) != hipSuccess) return e;
            if ((e = ret::launch_gn_rows((long)rows, a.H, a.N, a.DV, o1, a.out, a.out_bf16, a.gn, a.stream)) != hipSuccess) return e;
        } else if ((e = ret::launch_add_rows(rows * a.DV, o1, o2, o3, a.out, a.out_bf16, a.stream)) != hipSuccess) {
            return e;
        }
    }
    if (a.state_out)
        return ret::launch_add_rows((size_t)a.B * a.H * a.DK * a.DV, a.state_out, s2, nullptr, a.state_out, false, a.stream);
    return hipSuccess;
}

// Workspace of the forward forms with a rotation: bf16 inputs carry the rotated q and k as high and
// low parts (three calls, partial results), fp32 inputs one rotated copy.
size_t chunkwise_rot_ws(const ret_shape* s, int chunk, bool gn, int want_out);
size_t parallel_rot_ws(const ret_shape* s, bool gn);

ret_status check_ptr(const void* p, const char* name, bool required) {
    if (!p) return required ? fail(RET_ERR_INVALID_ARG, "%s is NULL", name) : RET_OK;
    if (!aligned16(p)) return fail(RET_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return RET_OK;
}

ret_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return RET_OK;
    return fail(RET_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define RET_TRY(x)                         \
    do {                                   \
        const ret_status _s = (x);         \
        if (_s != RET_OK) return _s;       \
    } while (0)

ret::LaunchArgs base_args(const ret_shape* s, int chunk, const ret::HeadConsts& hc, const ret::GnArgs& gn, void* ws,
                          size_t wsb, void* stream) {
    ret::LaunchArgs a{};
    a.B = s->batch; a.H = s->heads; a.N = s->seq_len; a.DK = s->d_k; a.DV = s->d_v;
    a.in_bf16 = s->in_dtype == RET_BF16;
    a.out_bf16 = s->out_dtype == RET_BF16;
    a.chunk = chunk;
    a.hc = hc;
    a.gn = gn;
    a.ws = ws;
    a.ws_bytes = wsb;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    return a;
}

// The chunkwise call's workspace: with want_out, enough for a call with an output or without one
// (a state-only bf16 call on the segment-state kernel can need more than the call with an output).
size_t chunkwise_ws(const ret_shape* s, int chunk, int gn, int want_out) {
    if (s->in_dtype == RET_BF16) {
        const size_t st = ret::chunkwise_bf16_workspace(s->batch, s->heads, s->seq_len, s->d_k, s->d_v, chunk, gn, 0);
        if (!want_out) return st;
        return std::max(st, ret::chunkwise_bf16_workspace(s->batch, s->heads, s->seq_len, s->d_k, s->d_v, chunk, gn, 1));
    }
    return want_out ? ret::chunkwise_f32_workspace(s->batch, s->heads, s->seq_len, s->d_v, gn, s->out_dtype == RET_BF16) : 0;
}

// Residual linear attention with bf16 inputs and the softmax map keeps more than bf16 of its
// features: the softmax concentrates a row's weight on a few features, and their bf16 rounding alone
// moves the output by 2e-2 to 5e-2 of its RMS. A decode step (N = 1) takes them in fp32 on the fp32
// decode kernel. A segment (N > 1) runs the bf16 chunkwise kernels three times on the features'
// bf16 high and low parts: the output is bilinear in (phi(q), phi(k)), so
//   o = A(q_hi, k_hi) + A(q_hi, k_lo) + A(q_lo, k_hi) + (the lo x lo term, about 2^-16 relative),
// with state_in entering the calls on q_hi and q_lo once each and the state from the k_hi and k_lo
// calls added (rla_split_features).
bool rla_f32_features(const ret_shape* s, int fmap) { return s->in_dtype == RET_BF16 && fmap == RET_FMAP_SOFTMAX && s->seq_len == 1; }
bool rla_split_features(const ret_shape* s, int fmap) { return s->in_dtype == RET_BF16 && fmap == RET_FMAP_SOFTMAX && s->seq_len > 1; }

// Residual linear attention: phi(q), the shifted phi(k) and v (input dtype, fp32 for
// rla_f32_features, bf16 high and low feature parts for rla_split_features; each 256-byte aligned),
// the split call's partial results, then the chunkwise workspace for N > 1 (no GroupNorm).
size_t rla_ws(const ret_shape* s, int chunk, int fmap) {
    const size_t rows = (size_t)s->batch * s->heads * s->seq_len;
    const bool f32 = rla_f32_features(s, fmap), split = rla_split_features(s, fmap);
    const size_t es = f32 ? sizeof(float) : elem_size(s->in_dtype);
    const size_t ops = (split ? 4 : 2) * align256(rows * s->d_k * es) + align256(rows * s->d_v * es);
    if (s->seq_len == 1) return ops;
    return ops + (split ? split_parts_bytes(s, false, true, chunk) : 0) + chunkwise_ws(s, chunk, 0, 1);
}

size_t parallel_ws(const ret_shape* s, int gn) {
    if (s->in_dtype == RET_BF16) return 0;
    return ret::parallel_f32_workspace(s->batch, s->heads, s->seq_len, s->d_v, gn, s->out_dtype == RET_BF16);
}

// The backward's partial gradients of the split: dq (k_lo) and dk (q_lo), dv twice, dstate_in.
size_t bwd_split_parts_bytes(const ret_shape* s) {
    const size_t rows = (size_t)s->batch * s->heads * s->seq_len;
    return 2 * align256(rows * s->d_k * 4) + 2 * align256(rows * s->d_v * 4) +
           align256((size_t)s->batch * s->heads * s->d_k * s->d_v * 4);
}

// The backward with a rotation: bf16 inputs carry the rotated q and k as high and low parts (three
// backward calls, partial gradients), fp32 inputs one rotated copy.
size_t bwd_rot_ws(const ret_shape* s, int chunk) {
    const size_t b = ret::chunkwise_bwd_workspace(s->in_dtype == RET_BF16, s->batch, s->heads, s->seq_len, s->d_k, s->d_v, chunk);
    if (s->in_dtype != RET_BF16) return rotation_ws(s) + b;
    return rotation_split_ws(s) + bwd_split_parts_bytes(s) + b;
}

size_t chunkwise_rot_ws(const ret_shape* s, int chunk, bool gn, int want_out) {
    if (s->in_dtype != RET_BF16) return rotation_ws(s) + chunkwise_ws(s, chunk, gn, want_out);
    return rotation_split_ws(s) + split_parts_bytes(s, gn, true, chunk) + chunkwise_ws(s, chunk, 0, want_out);
}

size_t parallel_rot_ws(const ret_shape* s, bool gn) {
    if (s->in_dtype != RET_BF16) return rotation_ws(s) + parallel_ws(s, gn);
    return rotation_split_ws(s) + split_parts_bytes(s, gn, false, 0) + parallel_ws(s, 0);
}

ret_status check_ws(size_t need, const void* ws, size_t wsb) {
    if (need == 0) return RET_OK;
    if (!ws) return fail(RET_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (!aligned16(ws)) return fail(RET_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    if (wsb < need) return fail(RET_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", wsb, need);
    return RET_OK;
}

}  // namespace

// Sets the thread-local message that retention_last_error() returns (for entry points defined in
// other files of the library).
void ret::set_last_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }

extern "C" {

int32_t retention_abi_version(void) { return RETENTION_ABI_VERSION; }

const char* retention_last_error(void) { return g_err; }

const char* retention_status_string(int32_t status) {
    switch (status) {
        case RET_OK: return "RET_OK: success";
        case RET_ERR_INVALID_ARG: return "RET_ERR_INVALID_ARG: invalid argument";
        case RET_ERR_UNSUPPORTED: return "RET_ERR_UNSUPPORTED: no kernel for these shapes or dtypes";
        case RET_ERR_WORKSPACE: return "RET_ERR_WORKSPACE: workspace missing or too small";
        case RET_ERR_DEVICE: return "RET_ERR_DEVICE: HIP error";
        default: return "unknown status";
    }
}

// Whether a kernel exists for call fn at this shape, chunk and rotation setting: the same tests as
// the entry points make (which also report the reason).
bool shape_supported(int32_t fn, const ret_shape* s, int chunk, bool rot) {
    const bool bf = s->in_dtype == RET_BF16;
    const int dk = s->d_k, dv = s->d_v;
    if (rot && (dk % 2 || dk / 2 > ret::kMaxPairs)) return false;
    const bool step_ok = dv % 4 == 0 && dv / 4 <= 256 && 256 % (dv / 4) == 0;
    switch (fn) {
        case RET_FN_CHUNKWISE:
            return bf ? ret::chunkwise_bf16_supported(dk, dv, chunk) && bf16_head_fits(s, chunk) : ret::chunkwise_f32_supported(dk, dv, chunk);
        case RET_FN_RECURRENT_STEP: return step_ok && dk <= 8192;
        case RET_FN_PARALLEL: return bf ? ret::parallel_bf16_supported(dk, dv) : ret::parallel_f32_supported(dk, dv);
        case RET_FN_CHUNKWISE_BWD: return ret::bwd_split(bf, dk, dv, chunk) != 0 && (!bf || bf16_head_fits(s, chunk));
        case RET_FN_RLA: {
            const size_t vrow = (size_t)dv * elem_size(s->in_dtype);
            if (rot || dk > 256 || dk % 4 || vrow % 16 != 0 || vrow > 4096) return false;
            if (s->seq_len == 1) return step_ok;
            return bf ? ret::chunkwise_bf16_supported(dk, dv, chunk) && bf16_head_fits(s, chunk)
                      : ret::chunkwise_f32_supported(dk, dv, chunk);
        }
        default: return false;
    }
}

size_t retention_workspace_bytes(int32_t fn, const ret_shape* shape, int32_t chunk, int32_t flags) {
    if (check_shape(shape, fn == RET_FN_RECURRENT_STEP) != RET_OK) return (size_t)-1;
    if (flags & ~(RET_WS_GROUPNORM | RET_WS_ROTATION)) return (size_t)-1;
    if (!shape_supported(fn, shape, chunk, (flags & RET_WS_ROTATION) != 0)) return (size_t)-1;
    const bool gn = (flags & RET_WS_GROUPNORM) != 0;
    const size_t rot = (flags & RET_WS_ROTATION) ? rotation_ws(shape) : 0;
    switch (fn) {
        case RET_FN_CHUNKWISE:
            if (chunk <= 0) return (size_t)-1;
            return rot ? chunkwise_rot_ws(shape, chunk, gn, 1) : chunkwise_ws(shape, chunk, gn, 1);
        case RET_FN_RECURRENT_STEP: return 0;  // a rotation is applied inside the step kernel
        case RET_FN_PARALLEL: return rot ? parallel_rot_ws(shape, gn) : parallel_ws(shape, gn);
        case RET_FN_CHUNKWISE_BWD:
            if (chunk <= 0) return (size_t)-1;
            if (rot) return bwd_rot_ws(shape, chunk);
            return ret::chunkwise_bwd_workspace(shape->in_dtype == RET_BF16, shape->batch, shape->heads, shape->seq_len,
                                                shape->d_k, shape->d_v, chunk);
        case RET_FN_RLA:
            if (shape->seq_len > 1 && chunk <= 0) return (size_t)-1;
            return std::max(rla_ws(shape, chunk, RET_FMAP_IDENTITY), rla_ws(shape, chunk, RET_FMAP_SOFTMAX));
        default: return (size_t)-1;
    }
}

ret_status retention_chunkwise_fwd(const ret_shape* shape, int32_t chunk, const void* q, const void* k, const void* v,
                                   const double* gamma, const ret_rotation* rotation, const float* state_in,
                                   const ret_groupnorm* groupnorm, void* out, float* state_out, void* workspace,
                                   size_t workspace_bytes, void* hip_stream) {
    return (ret_status)ret::chunkwise_fwd_entry(shape, chunk, q, k, v, gamma, rotation, state_in, groupnorm, out, state_out, workspace,
                                                workspace_bytes, nullptr, hip_stream);
}

}  // extern "C"

// The chunkwise forward behind both entry points. provide (may be null) is asked for the
// workspace after every argument has been validated, with the bytes the call needs, only when it
// needs some; it returns RET_OK with the buffer, or a status (its message already set).
int ret::chunkwise_fwd_entry(const ret_shape* shape, int32_t chunk, const void* q, const void* k, const void* v,
                             const double* gamma, const ret_rotation* rotation, const float* state_in,
                             const ret_groupnorm* groupnorm, void* out, float* state_out, void* workspace,
                             size_t workspace_bytes, int (*provide)(size_t need, void** ws, size_t* bytes), void* hip_stream) {
    g_err[0] = '\0';
    RET_TRY(check_shape(shape, false));
    RET_TRY(check_ptr(q, "q", true));
    RET_TRY(check_ptr(k, "k", true));
    RET_TRY(check_ptr(v, "v", true));
    RET_TRY(check_ptr(state_in, "state_in", false));
    RET_TRY(check_ptr(out, "out", false));
    RET_TRY(check_ptr(state_out, "state_out", false));
    if (!out && !state_out) return fail(RET_ERR_INVALID_ARG, "out and state_out are both NULL");
    ret::HeadConsts hc;
    RET_TRY(check_gamma(shape, gamma, &hc));
    ret::GnArgs gn;
    RET_TRY(check_gn(groupnorm, shape->in_dtype == RET_BF16, &gn));
    ret::RotConsts rc;
    bool rot = false;
    RET_TRY(check_rotation(rotation, shape, &rc, &rot));
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    const bool bf = shape->in_dtype == RET_BF16;
    if (bf ? !ret::chunkwise_bf16_supported(shape->d_k, shape->d_v, chunk)
           : !ret::chunkwise_f32_supported(shape->d_k, shape->d_v, chunk))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise: no kernel for %s inputs with d_k %d, d_v %d, chunk %d", bf ? "bf16" : "fp32",
                    shape->d_k, shape->d_v, chunk);
    RET_TRY(check_bf16_head(shape, chunk));
    const size_t rows = (size_t)shape->batch * shape->heads * shape->seq_len;
    const size_t in_sz = elem_size(shape->in_dtype);
    const size_t out_bytes = rows * shape->d_v * elem_size(shape->out_dtype);
    if (out && (overlaps(out, out_bytes, q, rows * shape->d_k * in_sz) || overlaps(out, out_bytes, k, rows * shape->d_k * in_sz) ||
                overlaps(out, out_bytes, v, rows * shape->d_v * in_sz)))
        return fail(RET_ERR_INVALID_ARG, "out must not alias q, k or v");
    const size_t st_bytes = (size_t)shape->batch * shape->heads * shape->d_k * shape->d_v * sizeof(float);
    if (state_out && out && overlaps(out, out_bytes, state_out, st_bytes))
        return fail(RET_ERR_INVALID_ARG, "out must not alias state_out");
    if (state_out && state_in && state_in != state_out && overlaps(state_in, st_bytes, state_out, st_bytes))
        return fail(RET_ERR_INVALID_ARG, "state_out may equal state_in but must not partly overlap it");
    if (!out) {
        gn.enabled = 0;
        gn.gate = nullptr;
    }
    const size_t need = rot ? chunkwise_rot_ws(shape, chunk, gn.enabled, out != nullptr)
                            : chunkwise_ws(shape, chunk, gn.enabled, out != nullptr);
    if (provide && need > 0) RET_TRY((ret_status)provide(need, &workspace, &workspace_bytes));
    RET_TRY(check_ws(need, workspace, workspace_bytes));
    const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    if (rot && bf) {
        // rotated bf16 operands as high and low parts, three products (the rotated values rounded
        // once to bf16 would move the output by up to 2.4e-2 of its RMS). With an output at the
        // chunks of the two-call split, its scores kernel turns q and k itself and writes the
        // planes; else a rotation pass writes them first.
        const void* pq[4];
        FusedRot fr;
        const bool fuse = out && ret::chunkwise_bf16_split2_supported(shape->d_k, chunk);
        hipError_t e = hipSuccess;
        if (fuse) {
            place_rotation_split(shape, fr.planes, &workspace, &workspace_bytes);
            fr.q = q; fr.k = k; fr.rc = &rc;
            for (int i = 0; i < 4; ++i) pq[i] = fr.planes[i];
        } else if ((e = stage_rotation_split(shape, rc, q, k, pq, &workspace, &workspace_bytes, st)) != hipSuccess) {
            return device_status(e, "retention_chunkwise_fwd rotation launch");
        }
        char* parts = static_cast<char*>(workspace);
        const size_t pb = split_parts_bytes(shape, gn.enabled, true, chunk);
        ret::LaunchArgs a = base_args(shape, chunk, hc, gn, parts + pb, workspace_bytes - pb, hip_stream);
        a.v = v; a.out = out; a.state_in = state_in; a.state_out = state_out;
        e = run_split(a, pq[0], pq[1], pq[2], pq[3], parts, ret::launch_chunkwise_bf16, true, fuse ? &fr : nullptr);
        return device_status(e, "retention_chunkwise_fwd launch");
    }
    if (rot) {
        const hipError_t e = stage_rotation(shape, rc, &q, &k, &workspace, &workspace_bytes, st);
        if (e != hipSuccess) return device_status(e, "retention_chunkwise_fwd rotation launch");
    }
    ret::LaunchArgs a = base_args(shape, chunk, hc, gn, workspace, workspace_bytes, hip_stream);
    a.q = q; a.k = k; a.v = v; a.out = out; a.state_in = state_in; a.state_out = state_out;
    hipError_t e = bf ? ret::launch_chunkwise_bf16(a) : ret::launch_chunkwise_f32(a);
    return device_status(e, "retention_chunkwise_fwd launch");
}

extern "C" {

ret_status retention_chunkwise_bwd(const ret_shape* shape, int32_t chunk, const void* q, const void* k, const void* v,
                                   const double* gamma, const ret_rotation* rotation, const float* state_in, const void* dout,
                                   float* dq, float* dk, float* dv, float* dstate_in, void* workspace, size_t workspace_bytes,
                                   void* hip_stream) {
    g_err[0] = '\0';
    RET_TRY(check_shape(shape, false));
    RET_TRY(check_ptr(q, "q", true));
    RET_TRY(check_ptr(k, "k", true));
    RET_TRY(check_ptr(v, "v", true));
    RET_TRY(check_ptr(dout, "dout", true));
    RET_TRY(check_ptr(state_in, "state_in", false));
    RET_TRY(check_ptr(dq, "dq", false));
    RET_TRY(check_ptr(dk, "dk", false));
    RET_TRY(check_ptr(dv, "dv", false));
    RET_TRY(check_ptr(dstate_in, "dstate_in", false));
    if (!dq && !dk && !dv && !dstate_in) return fail(RET_ERR_INVALID_ARG, "dq, dk, dv and dstate_in are all NULL");
    if (shape->out_dtype != RET_F32) return fail(RET_ERR_UNSUPPORTED, "the gradients are fp32 (out_dtype must be RET_F32)");
    ret::HeadConsts hc;
    RET_TRY(check_gamma(shape, gamma, &hc));
    ret::RotConsts rc;
    bool rot = false;
    RET_TRY(check_rotation(rotation, shape, &rc, &rot));
    if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
    const bool bf = shape->in_dtype == RET_BF16;
    if (!ret::bwd_split(bf, shape->d_k, shape->d_v, chunk))
        return fail(RET_ERR_UNSUPPORTED, "chunkwise backward: no kernels for %s inputs with d_k %d, d_v %d, chunk %d", bf ? "bf16" : "fp32",
                    shape->d_k, shape->d_v, chunk);
    RET_TRY(check_bf16_head(shape, chunk));
    const size_t rows = (size_t)shape->batch * shape->heads * shape->seq_len;
    const size_t in_sz = elem_size(shape->in_dtype);
    const size_t st_bytes = (size_t)shape->batch * shape->heads * shape->d_k * shape->d_v * sizeof(float);
    const void* ins[5] = {q, k, v, dout, state_in};
    const size_t in_b[5] = {rows * shape->d_k * in_sz, rows * shape->d_k * in_sz, rows * shape->d_v * in_sz, rows * shape->d_v * in_sz,
                            st_bytes};
    const void* outs[4] = {dq, dk, dv, dstate_in};
    const size_t out_b[4] = {rows * shape->d_k * 4, rows * shape->d_k * 4, rows * shape->d_v * 4, st_bytes};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], out_b[i], ins[j], in_b[j])) return fail(RET_ERR_INVALID_ARG, "gradient outputs must not alias the inputs");
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], out_b[i], outs[j], out_b[j])) return fail(RET_ERR_INVALID_ARG, "gradient outputs must not alias each other");
    }
    const size_t need = rot ? bwd_rot_ws(shape, chunk)
                            : ret::chunkwise_bwd_workspace(bf, shape->batch, shape->heads, shape->seq_len, shape->d_k, shape->d_v, chunk);
    RET_TRY(check_ws(need, workspace, workspace_bytes));
    const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (rot && bf) {
        // rotated bf16 q and k as high and low parts: dq is linear in k, dk and dstate_in in q, dv
        // bilinear in both, so (q_hi, k_hi) gives every gradient, (q_hi, k_lo) adds to dq (without the
        // state_in term, which does not involve k) and dv, and (q_lo, k_hi) adds to dk, dv and dstate_in
        const void* pq[4];
        e = stage_rotation_split(shape, rc, q, k, pq, &workspace, &workspace_bytes, st);
        if (e != hipSuccess) return device_status(e, "retention_chunkwise_bwd rotation launch");
        char* parts = static_cast<char*>(workspace);
        const size_t gk = align256(rows * shape->d_k * 4), gv = align256(rows * shape->d_v * 4);
        float* dq2 = reinterpret_cast<float*>(parts);
        float* dk3 = reinterpret_cast<float*>(parts + gk);
        float* dv2 = reinterpret_cast<float*>(parts + 2 * gk);
        float* dv3 = reinterpret_cast<float*>(parts + 2 * gk + gv);
        float* ds3 = reinterpret_cast<float*>(parts + 2 * gk + 2 * gv);
        const size_t pb = bwd_split_parts_bytes(shape);
        ret::BwdArgs b{};
        b.base = base_args(shape, chunk, hc, ret::GnArgs{}, parts + pb, workspace_bytes - pb, hip_stream);
        b.v = v; b.dout = dout;
        ret::BwdArgs c = b;
        c.q = pq[0]; c.k = pq[3]; c.dq = dq ? dq2 : nullptr; c.dv = dv ? dv2 : nullptr;
        if ((c.dq || c.dv) && (e = ret::launch_chunkwise_bwd(c)) != hipSuccess) return device_status(e, "retention_chunkwise_bwd launch");
        c = b;
        c.q = pq[1]; c.k = pq[2]; c.dk = dk ? dk3 : nullptr; c.dv = dv ? dv3 : nullptr; c.dstate_in = dstate_in ? ds3 : nullptr;
        if ((c.dk || c.dv || c.dstate_in) && (e = ret::launch_chunkwise_bwd(c)) != hipSuccess)
            return device_status(e, "retention_chunkwise_bwd launch");
        c = b;
        c.q = pq[0]; c.k = pq[2]; c.state_in = state_in; c.dq = dq; c.dk = dk; c.dv = dv; c.dstate_in = dstate_in;
        if ((e = ret::launch_chunkwise_bwd(c)) != hipSuccess) return device_status(e, "retention_chunkwise_bwd launch");
        if (dq && (e = ret::launch_add_rows(rows * shape->d_k, dq, dq2, nullptr, dq, false, st)) != hipSuccess)
            return device_status(e, "retention_chunkwise_bwd sum launch");
        if (dk && (e = ret::launch_add_rows(rows * shape->d_k, dk, dk3, nullptr, dk, false, st)) != hipSuccess)
            return device_status(e, "retention_chunkwise_bwd sum launch");
        if (dv && (e = ret::launch_add_rows(rows * shape->d_v, dv, dv2, dv3, dv, false, st)) != hipSuccess)
            return device_status(e, "retention_chunkwise_bwd sum launch");
        if (dstate_in && (e = ret::launch_add_rows(st_bytes / 4, dstate_in, ds3, nullptr, dstate_in, false, st)) != hipSuccess)
            return device_status(e, "retention_chunkwise_bwd sum launch");
    } else {
        if (rot) {
            e = stage_rotation(shape, rc, &q, &k, &workspace, &workspace_bytes, st);
            if (e != hipSuccess) return device_status(e, "retention_chunkwise_bwd rotation launch");
        }
        ret::BwdArgs b{};
        b.base = base_args(shape, chunk, hc, ret::GnArgs{}, workspace, workspace_bytes, hip_stream);
        b.q = q; b.k = k; b.v = v; b.dout = dout; b.state_in = state_in;
        b.dq = dq; b.dk = dk; b.dv = dv; b.dstate_in = dstate_in;
        e = ret::launch_chunkwise_bwd(b);
    }
    // gradients at the rotated q and k, turned back by the inverse rotation (in place)
    const long rrows = (long)shape->batch * shape->heads * shape->seq_len;
    if (e == hipSuccess && rot && (dq || dk))
        e = ret::launch_rotate2(rrows, shape->seq_len, shape->d_k, dq ? dq : dk, dq ? dq : dk, dq && dk ? dk : nullptr,
                                dq && dk ? dk : nullptr, 0, 0, rc, 1, st);
    return device_status(e, "retention_chunkwise_bwd launch");
}

ret_status retention_recurrent_step(const ret_shape* shape, const void* q, const void* k, const void* v, const double* gamma,
                                    const ret_rotation* rotation, float* state, const ret_groupnorm* groupnorm, void* out,
                                    void* workspace, size_t workspace_bytes, void* hip_stream) {
    g_err[0] = '\0';
    RET_TRY(check_shape(shape, true));
    RET_TRY(check_ptr(q, "q", true));
    RET_TRY(check_ptr(k, "k", true));
    RET_TRY(check_ptr(v, "v", true));
    RET_TRY(check_ptr(state, "state", true));
    RET_TRY(check_ptr(out, "out", false));
    ret::HeadConsts hc;
    RET_TRY(check_gamma(shape, gamma, &hc));
    ret::GnArgs gn;
    RET_TRY(check_gn(groupnorm, shape->in_dtype == RET_BF16, &gn));
    const int dv = shape->d_v;
    if (dv % 4 != 0 || dv / 4 > 256 || 256 % (dv / 4) != 0)
        return fail(RET_ERR_UNSUPPORTED, "recurrent step needs d_v a multiple of 4 with d_v/4 dividing 256 (got %d)", dv);
    if (shape->d_k > 8192) return fail(RET_ERR_UNSUPPORTED, "recurrent step supports d_k <= 8192 (got %d)", shape->d_k);
    const size_t bh = (size_t)shape->batch * shape->heads;
    const size_t st_bytes = bh * shape->d_k * dv * sizeof(float);
    const size_t out_bytes = bh * dv * elem_size(shape->out_dtype);
    if (out && overlaps(out, out_bytes, state, st_bytes)) return fail(RET_ERR_INVALID_ARG, "out must not alias state");
    ret::RotConsts rc;
    ret::StepRot sr;
    bool rot = false;
    RET_TRY(check_rotation(rotation, shape, &rc, &rot, &sr));
    (void)workspace;
    (void)workspace_bytes;  // the step needs none: a rotation is applied inside the kernel
    ret::LaunchArgs a = base_args(shape, 1, hc, gn, nullptr, 0, hip_stream);
    a.q = q; a.k = k; a.v = v; a.out = out; a.state_out = state;
    a.step_rot = rot ? &sr : nullptr;
    return device_status(ret::launch_recurrent_step(a), "retention_recurrent_step launch");
}

ret_status retention_parallel_fwd(const ret_shape* shape, const void* q, const void* k, const void* v, const double* gamma,
                                  const ret_rotation* rotation, const ret_groupnorm* groupnorm, void* out, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
    g_err[0] = '\0';
    RET_TRY(check_shape(shape, false));
    RET_TRY(check_ptr(q, "q", true));
    RET_TRY(check_ptr(k, "k", true));
    RET_TRY(check_ptr(v, "v", true));
    RET_TRY(check_ptr(out, "out", true));
    ret::HeadConsts hc;
    RET_TRY(check_gamma(shape, gamma, &hc));
    ret::GnArgs gn;
    RET_TRY(check_gn(groupnorm, shape->in_dtype == RET_BF16, &gn));
    const bool bf = shape->in_dtype == RET_BF16;
    if (bf ? !ret::parallel_bf16_supported(shape->d_k, shape->d_v) : !ret::parallel_f32_supported(shape->d_k, shape->d_v))
        return fail(RET_ERR_UNSUPPORTED, "parallel: no kernel for %s inputs with d_k %d, d_v %d", bf ? "bf16" : "fp32", shape->d_k,
                    shape->d_v);
    const size_t rows = (size_t)shape->batch * shape->heads * shape->seq_len;
    const size_t in_sz = elem_size(shape->in_dtype);
    const size_t out_bytes = rows * shape->d_v * elem_size(shape->out_dtype);
    if (overlaps(out, out_bytes, q, rows * shape->d_k * in_sz) || overlaps(out, out_bytes, k, rows * shape->d_k * in_sz) ||
        overlaps(out, out_bytes, v, rows * shape->d_v * in_sz))
        return fail(RET_ERR_INVALID_ARG, "out must not alias q, k or v");
    ret::RotConsts rc;
    bool rot = false;
    RET_TRY(check_rotation(rotation, shape, &rc, &rot));
    const size_t need = rot ? parallel_rot_ws(shape, gn.enabled) : parallel_ws(shape, gn.enabled);
    RET_TRY(check_ws(need, workspace, workspace_bytes));
    if (rot && bf) {
        // rotated bf16 operands as high and low parts, three calls
        const void* pq[4];
        hipError_t e = stage_rotation_split(shape, rc, q, k, pq, &workspace, &workspace_bytes, reinterpret_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return device_status(e, "retention_parallel_fwd rotation launch");
        char* parts = static_cast<char*>(workspace);
        const size_t pb = split_parts_bytes(shape, gn.enabled, false, 0);
        ret::LaunchArgs a = base_args(shape, 0, hc, gn, parts + pb, workspace_bytes - pb, hip_stream);
        a.v = v; a.out = out;
        e = run_split(a, pq[0], pq[1], pq[2], pq[3], parts, ret::launch_parallel_bf16, false);
        return device_status(e, "retention_parallel_fwd launch");
    }
    if (rot) {
        const hipError_t e = stage_rotation(shape, rc, &q, &k, &workspace, &workspace_bytes, reinterpret_cast<hipStream_t>(hip_stream));
        if (e != hipSuccess) return device_status(e, "retention_parallel_fwd rotation launch");
    }
    ret::LaunchArgs a = base_args(shape, 0, hc, gn, workspace, workspace_bytes, hip_stream);
    a.q = q; a.k = k; a.v = v; a.out = out;
    hipError_t e = bf ? ret::launch_parallel_bf16(a) : ret::launch_parallel_f32(a);
    return device_status(e, "retention_parallel_fwd launch");
}

ret_status retention_rla_fwd(const ret_shape* shape, int32_t chunk, int32_t window, int32_t feature_map, const void* q,
                             const void* k, const void* v, const void* k_prev, const void* v_prev, int32_t prev_len,
                             const float* state_in, void* out, float* state_out, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
    g_err[0] = '\0';
    RET_TRY(check_shape(shape, false));
    RET_TRY(check_ptr(q, "q", true));
    RET_TRY(check_ptr(k, "k", true));
    RET_TRY(check_ptr(v, "v", true));
    RET_TRY(check_ptr(state_in, "state_in", false));
    RET_TRY(check_ptr(out, "out", false));
    RET_TRY(check_ptr(state_out, "state_out", false));
    if (window < 0 || window > (1 << 30)) return fail(RET_ERR_INVALID_ARG, "window must be in [0, 2^30] (got %d)", window);
    if (feature_map != RET_FMAP_IDENTITY && feature_map != RET_FMAP_SOFTMAX)
        return fail(RET_ERR_INVALID_ARG, "feature_map must be RET_FMAP_IDENTITY or RET_FMAP_SOFTMAX (got %d)", feature_map);
    const int P = window + 1;
    if (prev_len < 0 || prev_len > P) return fail(RET_ERR_INVALID_ARG, "prev_len must be in [0, window + 1] (got %d)", prev_len);
    RET_TRY(check_ptr(k_prev, "k_prev", prev_len > 0));
    RET_TRY(check_ptr(v_prev, "v_prev", prev_len > 0));
    if (!out && !state_out) return fail(RET_ERR_INVALID_ARG, "out and state_out are both NULL");
    if (shape->d_k > 256 || shape->d_k % 4)
        return fail(RET_ERR_UNSUPPORTED, "residual linear attention supports d_k <= 256, a multiple of 4 (got %d)", shape->d_k);
    const size_t vrow = (size_t)shape->d_v * elem_size(shape->in_dtype);
    if (vrow % 16 != 0 || vrow > 4096)
        return fail(RET_ERR_UNSUPPORTED, "residual linear attention needs value rows of a multiple of 16 bytes, at most 4 KiB (d_v %d)",
                    shape->d_v);
    const bool bf = shape->in_dtype == RET_BF16;
    const int N = shape->seq_len, dv = shape->d_v;
    if (N == 1) {
        if (!state_out) return fail(RET_ERR_INVALID_ARG, "a one-token segment (decode step) needs state_out");
        if (dv % 4 != 0 || dv / 4 > 256 || 256 % (dv / 4) != 0)
            return fail(RET_ERR_UNSUPPORTED, "a one-token segment needs d_v a multiple of 4 with d_v/4 dividing 256 (got %d)", dv);
    } else {
        if (chunk <= 0) return fail(RET_ERR_INVALID_ARG, "chunk must be positive (got %d)", chunk);
        if (bf ? !ret::chunkwise_bf16_supported(shape->d_k, dv, chunk) : !ret::chunkwise_f32_supported(shape->d_k, dv, chunk))
            return fail(RET_ERR_UNSUPPORTED, "residual linear attention: no chunkwise kernel for %s inputs with d_k %d, d_v %d, chunk %d",
                        bf ? "bf16" : "fp32", shape->d_k, dv, chunk);
        RET_TRY(check_bf16_head(shape, chunk));
    }
    const size_t rows = (size_t)shape->batch * shape->heads * N;
    const size_t es = elem_size(shape->in_dtype);
    const size_t out_bytes = rows * dv * elem_size(shape->out_dtype);
    const size_t pk = (size_t)shape->batch * shape->heads * P * shape->d_k * es, pv = (size_t)shape->batch * shape->heads * P * dv * es;
    if (out && (overlaps(out, out_bytes, q, rows * shape->d_k * es) || overlaps(out, out_bytes, k, rows * shape->d_k * es) ||
                overlaps(out, out_bytes, v, rows * dv * es) || (prev_len && overlaps(out, out_bytes, k_prev, pk)) ||
                (prev_len && overlaps(out, out_bytes, v_prev, pv))))
        return fail(RET_ERR_INVALID_ARG, "out must not alias q, k, v, k_prev or v_prev");
    const size_t st_bytes = (size_t)shape->batch * shape->heads * shape->d_k * dv * sizeof(float);
    if (state_out && out && overlaps(out, out_bytes, state_out, st_bytes)) return fail(RET_ERR_INVALID_ARG, "out must not alias state_out");
    if (state_out && state_in && state_in != state_out && overlaps(state_in, st_bytes, state_out, st_bytes))
        return fail(RET_ERR_INVALID_ARG, "state_out may equal state_in but must not partly overlap it");
    RET_TRY(check_ws(rla_ws(shape, chunk, feature_map), workspace, workspace_bytes));

    // operands: phi(q), shifted phi(k) and v, in the front of the workspace
    const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    char* w = static_cast<char*>(workspace);
    const bool f32feat = rla_f32_features(shape, feature_map), split = rla_split_features(shape, feature_map);
    const size_t eo = f32feat ? sizeof(float) : es;  // bytes per prepared element
    const size_t Aq = align256(rows * shape->d_k * eo), Av = align256(rows * dv * eo);
    const size_t nq = split ? 4 : 2;  // feature planes: q and k, or their high and low parts
    ret::RlaPrep r{};
    r.rows = (long)rows; r.N = N; r.dk = shape->d_k; r.dv = dv; r.P = P; r.prev_len = prev_len; r.fmap = feature_map; r.bf16 = bf;
    r.feat_f32 = f32feat;
    r.q = q; r.k = k; r.v = v; r.kp = k_prev; r.vp = v_prev;
    r.qo = feature_map == RET_FMAP_IDENTITY ? nullptr : w;
    r.ko = w + Aq;
    if (split) {
        r.qlo = w + 2 * Aq;
        r.klo = w + 3 * Aq;
    }
    r.vo = w + nq * Aq;
    // shifted value rows in the workspace only up to vsplit (w + 1 rounded up to a 32-token stage,
    // at most N); the chunkwise kernels read the later rows from v, w + 1 rows back. With fp32
    // features (a decode step) the one value row is written there in fp32.
    r.vsplit = f32feat ? N : (int)std::min<long long>(((long long)P + 31) / 32 * 32, N);
    hipError_t e = ret::launch_rla_prepare(r, st);
    if (e != hipSuccess) return device_status(e, "retention_rla_fwd prepare launch");
    ret::HeadConsts hc;
    for (int h = 0; h < ret::kMaxHeads; ++h) {
        hc.gamma[h] = 1.f;
        hc.log2g[h] = 0.f;
    }
    char* rest = w + nq * Aq + Av;  // after the operands
    char* parts = rest;             // split calls: partial outputs and state
    if (split) rest += split_parts_bytes(shape, false, true, chunk);
    ret::LaunchArgs a = base_args(shape, N == 1 ? 1 : chunk, hc, ret::GnArgs{}, rest,
                                  workspace_bytes - (size_t)(rest - w), hip_stream);
    if (f32feat) a.in_bf16 = 0;  // the fp32 decode kernel, on the fp32 features and value row
    a.q = r.qo ? r.qo : q; a.k = r.ko; a.out = out;
    if (r.vsplit == N) {
        a.v = r.vo;  // every value row is in the prefix buffer (laid out like v)
    } else {
        a.v = v;
        a.vs = ret::VShift{r.vo, r.vsplit, P};
    }
    if (N == 1) {
        if (state_in != state_out) {
            e = ret::launch_copy_state(st_bytes / sizeof(float), state_in, state_out, st);
            if (e != hipSuccess) return device_status(e, "retention_rla_fwd state copy launch");
        }
        a.state_out = state_out;
        return device_status(ret::launch_recurrent_step(a), "retention_rla_fwd step launch");
    }
    if (!split) {
        a.state_in = state_in; a.state_out = state_out;
        return device_status(a.in_bf16 ? ret::launch_chunkwise_bf16(a) : ret::launch_chunkwise_f32(a), "retention_rla_fwd launch");
    }
    a.state_in = state_in; a.state_out = state_out;
    return device_status(run_split(a, r.qo, r.qlo, r.ko, r.klo, parts, ret::launch_chunkwise_bf16, true), "retention_rla_fwd launch");
}

}  // extern "C"

/*
 * retention.h: C ABI of the MI355X (gfx950) multi-scale retention library.
 *
 * Multi-scale retention, per head h with a fixed decay gamma_h (0 < gamma_h <= 1):
 *   parallel form    O = (Q K^T (.) D) V,  D[n][m] = gamma^(n-m) for n >= m, else 0
 *   recurrent form   S_n = gamma * S_(n-1) + k_n^T v_n,   o_n = q_n S_n
 *   chunkwise form   each chunk computed in parallel inside, the state carried between chunks
 * Sources: abeam.tech RetNet paper summary, section "Technical mechanism" (retention as
 * content-based reference times distance-based forgetting; training in parallel, generation by
 * state update; chunk recursion for long-sequence training); mlnews.online "Retentive Network:
 * A Successor to Transformer for Large Language Models" (three computation paradigms; per-head
 * decay; per-head GroupNorm of the retention outputs); eulerwa.com "3. RetNet in detail"
 * ("How does it work?": the three modes compute the same values).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts (row-major, contiguous, last index fastest):
 *   q, k      [B][H][N][d_k]          v, out   [B][H][N][d_v]
 *   state     [B][H][d_k][d_v] fp32   (the recurrent state S, one d_k x d_v matrix per head)
 *   decode-step vectors: q, k [B][H][d_k], v and out [B][H][d_v]
 * Positions are 0-based and o_n includes token n (diagonal decay gamma^0 = 1). No 1/sqrt(d_k)
 * scaling is applied: the result is exactly (Q K^T (.) D) V.
 * Pointers: q, k, v, out, state*, groupnorm weight/bias and workspace are DEVICE pointers owned
 * by the caller. `gamma` is a HOST pointer to H doubles, and `rotation` and `groupnorm` HOST
 * pointers to structs; all three are read during the call only. The library
 * never allocates device memory and keeps no state between calls except a thread-local error
 * string and, for retention_chunkwise_fwd_noalloc only, its fixed per-GPU scratch array (part of
 * the loaded code object) and the address of it on each device. All device pointers must be
 * 16-byte aligned.
 * Streams: all work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream) and the
 * call returns without synchronising. Errors found during execution surface at the caller's
 * next synchronisation.
 * Errors: every argument is validated on the host before any HIP call. No C++ exception
 * crosses this boundary. On a non-OK return, retention_last_error() describes the problem.
 * Determinism: for the same inputs, shapes and chunk, results are bitwise identical from run
 * to run (fixed reduction orders; no floating-point atomics).
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RETENTION_ABI_VERSION 4
#define RETENTION_MAX_HEADS 128

typedef enum {
    RET_OK = 0,
    RET_ERR_INVALID_ARG = 1,  /* null required pointer, bad dimension, gamma not in (0,1], eps <= 0,
                                 misaligned pointer, out and state_out both NULL, ...          */
    RET_ERR_UNSUPPORTED = 2,  /* valid arguments, but no kernel specialisation for them        */
    RET_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than retention_workspace_bytes()    */
    RET_ERR_DEVICE = 4        /* a HIP call or kernel launch failed; see retention_last_error  */
} ret_status;

typedef enum { RET_F32 = 0, RET_BF16 = 1 } ret_dtype;

typedef enum {
    RET_FN_CHUNKWISE = 0,
    RET_FN_RECURRENT_STEP = 1,
    RET_FN_PARALLEL = 2,
    RET_FN_CHUNKWISE_BWD = 3,
    RET_FN_RLA = 4
} ret_fn;

/* Feature maps of residual linear attention. */
typedef enum { RET_FMAP_IDENTITY = 0, RET_FMAP_SOFTMAX = 1 } ret_feature_map;

/* Flags of retention_workspace_bytes(): the epilogue and prologue settings of the call. */
#define RET_WS_GROUPNORM 1
#define RET_WS_ROTATION 2

/* Problem shape. in_dtype applies to q, k and v; out_dtype to out. */
typedef struct {
    int32_t batch, heads, seq_len, d_k, d_v;
    int32_t in_dtype;   /* ret_dtype */
    int32_t out_dtype;  /* ret_dtype */
} ret_shape;

/* Optional per-head GroupNorm epilogue (mlnews.online RetNet page, bullet summary: outputs are
 * normalised per head before concatenation). One group = the d_v channels of one head at one
 * position: y = (o - mean) / sqrt(var + eps) * weight[h][c] + bias[h][c], biased variance,
 * statistics in fp32 from the fp32 pre-norm output. weight/bias: device fp32 [H][d_v], or NULL
 * for 1 / 0. Pass NULL (or enabled = 0) for no normalisation.
 * Optional swish gate after it (abeam.tech RetNet summary, "Multi-timescale decay, gate and
 * normalisation": a Swish gate adds non-linearity, GroupNorm handles the heads' differing
 * variance): out = swish(g) * y with swish(x) = x * sigmoid(x), g = gate[b][h][n][c], a device
 * tensor in the input dtype laid out like out ([B][H][d_v] for the decode step), or NULL. A gate
 * needs enabled = 1 (RET_ERR_INVALID_ARG otherwise). */
typedef struct {
    int32_t enabled;
    float eps;           /* > 0 */
    const float* weight; /* [H][d_v] or NULL */
    const float* bias;   /* [H][d_v] or NULL */
    const void* gate;    /* like out, input dtype, or NULL */
} ret_groupnorm;

/* Optional positional rotation of q and k before retention (abeam.tech RetNet summary, "Technical
 * mechanism": Q and K get a positional rotation after the projections; eulerwa.com "3. RetNet
 * 상세": RoPE is the position encoding used with the decay). The pages give no formula; this is
 * the rotary position embedding of Su et al. (RoFormer): at absolute position p = offset + n, each
 * feature pair (2i, 2i+1) of q_n and of k_n is turned by p * theta_i, theta_i = base^(-2i/d_k):
 *   (a, b) -> (a cos(p theta_i) - b sin(p theta_i), a sin(p theta_i) + b cos(p theta_i)).
 * Retention then runs on the rotated q and k, so scores depend on relative positions only.
 * offset is the absolute position of token 0 of this call (the number of tokens before it, e.g.
 * the prefill length for a decode step). Needs d_k even (d_k <= 256), base > 0 finite,
 * 0 <= offset < 2^31 and seq_len < 2^24. Pass NULL (or enabled = 0) for none. The chunkwise, parallel and
 * backward calls keep the rotated q and k in the workspace (flag RET_WS_ROTATION of
 * retention_workspace_bytes); the decode step needs none. fp32 inputs: one fp32 copy each.
 * bf16 inputs: the turned values are not bf16 numbers, and rounding them once would move the
 * output by up to 2.4e-2 of its RMS, so the chunkwise and parallel forms and the backward keep
 * them as bf16 high and low parts and run on (q_hi, k_hi), (q_hi, k_lo) and (q_lo, k_hi) (the
 * lo x lo term, about 2^-16 relative, is dropped). The chunkwise forward with an output at chunks
 * 64 to 256 forms the scores of the three products in one kernel, which also turns q and k and
 * writes their parts to the workspace, then runs (q_hi, k_lo) on those scores and
 * (q_hi + q_lo, k_hi) without an intra-chunk term, adding fp32 rows in place; its other calls
 * (chunk 512, state only) turn q and k in a pass of their own first and run two or three calls. The
 * parallel and backward calls keep fp32 partial results in the workspace and add them.
 * The decode step turns q and k in fp32 inside its kernel, with no rounding of the turned values.
 * Angles: the per-pair frequency theta_i / pi and the offset's phase are formed on the host in
 * double precision; the device adds n times the frequency with an exact two-product and
 * evaluates sin and cos of pi times the phase in fp32 (error about 1e-6 rad at any allowed
 * position). */
typedef struct {
    int32_t enabled;
    double base;    /* e.g. 10000 */
    int64_t offset; /* absolute position of token 0 */
} ret_rotation;

/*
 * Chunkwise recurrent form (abeam.tech summary, "Chunk recursion for long-sequence training";
 * mlnews abstract: chunks encoded in parallel, summarised recurrently).
 * With chunk length C (positions c*C .. c*C+L-1, L = C or N mod C for the last chunk) and R the
 * state carried in (state_in, or zero when NULL), for local row j:
 *   o_j = sum_{t<=j} gamma^(j-t) (q_j . k_t) v_t + gamma^(j+1) q_j R
 *   R  <- gamma^L R + sum_t gamma^(L-1-t) k_t^T v_t
 * chunk: 64, 128, 256 or 512 (bf16 inputs); 64 or 128 (fp32 inputs).
 * state_in: fp32 [B][H][d_k][d_v] or NULL (zero). state_out: fp32, or NULL. state_out may equal
 * state_in (in place). out may be NULL only when state_out is not NULL (state-only prefill);
 * out must not alias q, k or v.
 * Supported: d_k in {64, 256} and d_v in {32, 64, 128, 256, 512} for bf16; d_k in {64,128,256}, d_v a
 * multiple of 64 up to 512 for fp32. H <= RETENTION_MAX_HEADS. bf16 inputs also need one head's
 * padded extent within 32-bit offsets: P = ceil(N / chunk) * chunk, P * max(d_k, d_v) * 4 < 2^31 and
 * P * chunk * 2 < 2^31 (about 1M tokens at d_v = 512); longer sequences return RET_ERR_UNSUPPORTED
 * (run them as segments through state_in / state_out).
 * Precision (bf16 inputs): products accumulate in fp32; the carried state is fp32 and enters the
 * matrix cores as a bf16 high part plus a bf16 low part, as does v scaled by its decay.
 */
ret_status retention_chunkwise_fwd(const ret_shape* shape, int32_t chunk,
                                   const void* q, const void* k, const void* v,
                                   const double* gamma, const ret_rotation* rotation, const float* state_in,
                                   const ret_groupnorm* groupnorm, void* out, float* state_out,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One recurrent step (abeam.tech summary, "Training in parallel, generation by state update"):
 *   S <- gamma_h S + k^T v  (in place, fp32),   o = q S  (with the updated S)
 * shape->seq_len must be 1. q, k: [B][H][d_k]; v: [B][H][d_v]; state: fp32 [B][H][d_k][d_v],
 * read and written in place; out: [B][H][d_v] (may be NULL to only advance the state).
 * Supported: d_v a multiple of 4 with d_v / 4 dividing 256 (d_v <= 1024), any d_k >= 1.
 * With a rotation, rotation->offset is the position of this token; the kernel turns q and k in
 * fp32 as it reads them (no rounding of the turned values), so the step needs no workspace
 * (workspace may be NULL; retention_workspace_bytes returns 0).
 */
ret_status retention_recurrent_step(const ret_shape* shape,
                                    const void* q, const void* k, const void* v,
                                    const double* gamma, const ret_rotation* rotation, float* state,
                                    const ret_groupnorm* groupnorm, void* out,
                                    void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Parallel form (abeam.tech summary, retention as content-based reference times distance-based
 * forgetting): O = (Q K^T (.) D) V over the whole sequence, causal, no state.
 * Supported: d_k in {64, 256} and d_v in {64, 128, 256, 512} for bf16; d_k <= 512 and d_v a multiple
 * of 64 up to 512 for fp32. H <= RETENTION_MAX_HEADS.
 */
ret_status retention_parallel_fwd(const ret_shape* shape,
                                  const void* q, const void* k, const void* v,
                                  const double* gamma, const ret_rotation* rotation,
                                  const ret_groupnorm* groupnorm, void* out,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Backward of the chunkwise form: the gradients of a loss L for dL/dout = dout (abeam.tech
 * summary, "Training in parallel, generation by state update": differentiating
 * S_n = gamma S_(n-1) + k_n^T v_n, o_n = q_n S_n with the reverse-time state
 * U_n = gamma U_(n+1) + q_n^T dout_n gives dq_n = dout_n S_n^T, dk_n = U_n v_n^T, dv_n = k_n U_n
 * and dstate_in = gamma U_0). The pre-norm output: no GroupNorm or gate.
 * q, k: [B][H][N][d_k]; v, dout: [B][H][N][d_v], in shape->in_dtype; state_in: fp32
 * [B][H][d_k][d_v] or NULL (zero). Outputs, each fp32 and each optional: dq, dk like q; dv like v;
 * dstate_in like state_in. shape->out_dtype must be RET_F32. Outputs must not alias inputs or each
 * other. Supported where the forwards it runs exist: retention_chunkwise_fwd at (d_k, d_v) and at
 * contraction width d_v with value width d_k; a d_v with no forward kernel of contraction width d_v
 * runs as two column blocks of d_v / 2 (bf16 (64, 32), for one, has neither and returns
 * RET_ERR_UNSUPPORTED). The same bound on one head's extent as retention_chunkwise_fwd.
 * With a rotation, dq and dk are the gradients with respect to the unrotated q and k: the
 * gradients at the rotated inputs turned back by the inverse rotation (its transpose).
 * Workspace: retention_workspace_bytes(RET_FN_CHUNKWISE_BWD, ...): the workspace of the forward
 * calls and the blocks of state_in^T (bf16 inputs, whose forwards read every operand in place and
 * add the two column blocks' rows of dq and dk into those outputs; with seq_len a multiple of the
 * chunk also the dq forward's scores, anti-transposed, which the dk forward reads in place of its
 * own); for fp32 inputs also the fp32
 * outputs of the column blocks and time-reversed and block copies of q, k, v and dout (plus the
 * rotated q and k with RET_WS_ROTATION). With bf16 inputs and two column blocks, dq and dk are
 * zeroed and then written by atomic fp32 adds: each element receives exactly two, so the result
 * does not depend on their order.
 */
ret_status retention_chunkwise_bwd(const ret_shape* shape, int32_t chunk,
                                   const void* q, const void* k, const void* v,
                                   const double* gamma, const ret_rotation* rotation,
                                   const float* state_in, const void* dout,
                                   float* dq, float* dk, float* dv, float* dstate_in,
                                   void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Residual linear attention, RLA (mengro1102.github.io RAttention post, section 4, RLA formula and
 * notes): the undecayed linear-attention state read w + 1 tokens late,
 *   S_t = S_(t-1) + phi(k_t)^T v_t,   o_t = phi(q_t) S_(t-w-1)
 * so that o_t sees only the tokens that have left a sliding window of the last w tokens and t
 * itself (the window's own attention is out of scope). phi (feature_map): RET_FMAP_SOFTMAX, the
 * softmax over the d_k features of each row (the page calls the best map softmax-based and gives
 * no formula), or RET_FMAP_IDENTITY.
 * One call covers a segment of N tokens, positions 0 .. N-1:
 *   k_prev, v_prev: [B][H][window+1][d_k] and [B][H][window+1][d_v], the window+1 positions before
 *     the segment (rows in time order); only the last prev_len rows hold tokens (the sequence
 *     starts after the others, which are never read). prev_len = 0 at the start of a sequence,
 *     where k_prev and v_prev may be NULL. 0 <= prev_len <= window + 1.
 *   state_in: fp32 [B][H][d_k][d_v], the sum of phi(k)^T v over every token before the window
 *     rows (NULL: zero).
 *   state_out: the sum over every token that has left the window at the end of the segment, i.e.
 *     the state the last output read. With the last window+1 tokens as the next k_prev, v_prev, it
 *     is the next segment's state_in. A decode step is a segment of N = 1 whose k_prev row 0 is the
 *     token leaving the window; it runs on the decode-step kernel and needs state_out (which may
 *     equal state_in: the state is then advanced in place).
 * q, k, v, out: as retention_chunkwise_fwd. window >= 0. d_k <= 256, a multiple of 4; a value row (d_v elements of
 * the input dtype) a multiple of 16 bytes and at most 4 KiB. N > 1 takes the chunkwise
 * kernels (chunk and (d_k, d_v) as there); N = 1 the decode-step kernel (d_v as there).
 * Workspace: retention_workspace_bytes(RET_FN_RLA, ...), the larger of the two maps' needs: phi(q),
 * the shifted phi(k) and room for the shifted v, plus the chunkwise workspace. With the identity
 * map (or fp32 inputs) they are in the input dtype and only the first
 * min(ceil((window + 1) / 32) * 32, N) shifted value rows of each head are written there (the
 * kernels read the later ones from v itself). With bf16 inputs and the softmax map the features
 * keep more than bf16 (the softmax puts most of a row's weight on a few features, whose bf16
 * rounding alone would move the output by 2e-2 to 5e-2 of its RMS): a segment (N > 1) writes their
 * bf16 high and low parts and runs the bf16 chunkwise kernels on (q_hi, k_hi), (q_hi, k_lo) and
 * (q_lo, k_hi) (the first and last as one call on q_hi + q_lo where the chunk kernel takes q as
 * two parts): the later calls add their fp32 rows into the first's (into out for an fp32 output,
 * else through one fp32 buffer in the workspace) and the second partial state is added after
 * them; a decode step (N = 1) takes the features and the value row in fp32.
 */
ret_status retention_rla_fwd(const ret_shape* shape, int32_t chunk, int32_t window, int32_t feature_map,
                             const void* q, const void* k, const void* v,
                             const void* k_prev, const void* v_prev, int32_t prev_len,
                             const float* state_in, void* out, float* state_out,
                             void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * The chunkwise forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results as retention_chunkwise_fwd, with its scratch taken
 * from a fixed array inside the library instead of a caller workspace. The call allocates nothing.
 * The array holds RETENTION_NOALLOC_SCRATCH_BYTES; a call whose workspace
 * (retention_workspace_bytes(RET_FN_CHUNKWISE, ...)) exceeds it returns RET_ERR_WORKSPACE before any
 * HIP call. Each GPU holds one copy of the array from the library's first use on it until the
 * process ends; its address is looked up once per device, on the first call with that device
 * current. The stream must belong to the current device. Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents: calls that overlap in time on one GPU (different
 * streams, or host threads) race on it and must be ordered by the caller.
 */
#define RETENTION_NOALLOC_SCRATCH_BYTES (64ull << 20)
ret_status retention_chunkwise_fwd_noalloc(const ret_shape* shape, int32_t chunk,
                                           const void* q, const void* k, const void* v,
                                           const double* gamma, const ret_rotation* rotation, const float* state_in,
                                           const ret_groupnorm* groupnorm, void* out, float* state_out,
                                           void* hip_stream);

/* Bytes of device workspace the call `fn` needs for this shape, chunk and flags (a bitwise OR of
 * RET_WS_GROUPNORM when a GroupNorm epilogue is enabled and RET_WS_ROTATION when a rotation is).
 * Returns 0 when none is needed, and (size_t)-1 when the arguments are invalid or no kernel
 * supports the shape, chunk and flags (the call itself would return RET_ERR_UNSUPPORTED; residual
 * linear attention takes no rotation).
 * Chunkwise with bf16 inputs: the larger of what a call with an output and a state-only call
 * need. With an output: the intra-chunk scores as bf16 high and low parts
 * (2*B*H*ceil(N/chunk)*chunk^2*2 bytes), plus fp32 pre-norm rows (B*H*N*d_v*4 bytes) with
 * GroupNorm; or, where one workgroup per (b, h, 32 columns of d_v) would leave compute units idle,
 * the fp32 states of the sequence segments the call is split into (up to B*H*S*d_k*d_v*4 bytes for
 * S segments) plus the pre-norm rows. State-only: the segments' states when there are several.
 * Other calls: fp32 staging rows when GroupNorm or a bf16 output needs them. A rotation adds the
 * rotated q and k (2*B*H*N*d_k elements of the input dtype, each copy 256-byte aligned) in front.
 * The caller owns it; its contents are scratch and need no initialisation. */
size_t retention_workspace_bytes(int32_t fn, const ret_shape* shape, int32_t chunk, int32_t flags);

/* Static description of a status code. */
const char* retention_status_string(int32_t status);

/* Thread-local detail for the last non-OK return on this thread ("" if none). */
const char* retention_last_error(void);

/* RETENTION_ABI_VERSION of the built library. */
int32_t retention_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RETENTION_H */

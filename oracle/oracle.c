/*
 * Multi-scale retention: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load this library. The GPU library never links it and
 * shares no code, header or table with it.
 *
 * Every function follows the definitions on the pages, written out directly
 * in double precision with no blocking, fusion or reordering beyond what the
 * definition states:
 *
 *   - abeam.tech RetNet paper summary, section "Technical mechanism",
 *     subsection "Retention multiplies content-based reference and
 *     distance-based forgetting": the output at position n weights each
 *     past value v_m by the content affinity q_n . k_m times the decay
 *     gamma^(n-m); future positions are masked.
 *   - same page, subsection "Training in parallel, generation by state
 *     update": per head, S_n = gamma * S_{n-1} + k_n^T v_n and o_n = q_n S_n.
 *   - same page, subsection "Chunk recursion for long-sequence training":
 *     inside a chunk the interactions are computed in parallel, earlier
 *     chunks arrive through the state matrix, and the state is updated at
 *     the end of each chunk.
 *   - mlnews.online "Retentive Network: A Successor to Transformer for
 *     Large Language Models", bullet summary: each head has its own gamma;
 *     retention outputs are normalised per head with GroupNorm.
 *
 * Tensor layout (all row-major, contiguous, last index fastest):
 *   q, k: [B][H][N][dk]   v, out: [B][H][N][dv]   state: [B][H][dk][dv]
 * Positions n are 0-based; o_n includes token n (the decay of the diagonal
 * term is gamma^0 = 1).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Recurrent form (abeam.tech summary, "Training in parallel, generation by
 * state update"). For every (b, h), starting from state_in (or zero):
 *     S <- gamma_h * S + k_n^T v_n      (d_k x d_v rank-1 update)
 *     o_n = q_n S                       (read after the update)
 * out and state_out may each be NULL.
 */
void oracle_recurrent(int B, int H, int N, int dk, int dv,
                      const double* q, const double* k, const double* v,
                      const double* gamma, const double* state_in,
                      double* out, double* state_out) {
    /* Output columns j and state columns j depend only on state column j, so the work is
       split into independent blocks of columns; each element sees the same operations in the
       same order as in a single pass. */
    const int CB = 64;
    const int ncb = (dv + CB - 1) / CB;
#pragma omp parallel for schedule(dynamic, 1)
    for (long task = 0; task < (long)B * H * ncb; ++task) {
        const int bh = (int)(task / ncb);
        const int j0 = (int)(task % ncb) * CB;
        const int j1 = (j0 + CB < dv) ? j0 + CB : dv;
        const int w = j1 - j0;
        const double g = gamma[bh % H];
        double* S = (double*)malloc((size_t)dk * w * sizeof(double));  /* S[i][j - j0] */
        for (int i = 0; i < dk; ++i)
            for (int j = j0; j < j1; ++j)
                S[(size_t)i * w + (j - j0)] = state_in ? state_in[((size_t)bh * dk + i) * dv + j] : 0.0;
        for (int n = 0; n < N; ++n) {
            const double* qn = q + ((size_t)bh * N + n) * dk;
            const double* kn = k + ((size_t)bh * N + n) * dk;
            const double* vn = v + ((size_t)bh * N + n) * dv;
            double* on = out ? out + ((size_t)bh * N + n) * dv : NULL;
            if (on)
                for (int j = j0; j < j1; ++j) on[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                double* Si = S + (size_t)i * w;  /* Si[j - j0] holds S[i][j] */
                for (int j = j0; j < j1; ++j) Si[j - j0] = g * Si[j - j0] + kn[i] * vn[j];
                if (on)
                    for (int j = j0; j < j1; ++j) on[j] += qn[i] * Si[j - j0];
            }
        }
        if (state_out)
            for (int i = 0; i < dk; ++i)
                for (int j = j0; j < j1; ++j)
                    state_out[((size_t)bh * dk + i) * dv + j] = S[(size_t)i * w + (j - j0)];
        free(S);
    }
}

/*
 * Gradients of the recurrent form (the backward pass of training, which is what
 * the pages measure: abeam.tech summary, "Training in parallel, generation by
 * state update"). For a loss L with dL/do_n = dout_n, differentiating
 *     S_n = gamma S_{n-1} + k_n^T v_n,   o_n = q_n S_n   (S_-1 = state_in or 0)
 * with the reverse-time state
 *     U_n = gamma U_{n+1} + q_n^T dout_n,   U_N = 0      (d_k x d_v)
 * gives, for every (b, h),
 *     dq_n = dout_n S_n^T,   dk_n = U_n v_n^T,   dv_n = k_n U_n,
 *     dstate_in = gamma U_0.
 * dq, dk, dv (laid out like q, k, v) and dstate_in ([B][H][dk][dv]) may be NULL.
 */
void oracle_recurrent_bwd(int B, int H, int N, int dk, int dv,
                          const double* q, const double* k, const double* v,
                          const double* gamma, const double* state_in, const double* dout,
                          double* dq, double* dkk, double* dvv, double* dstate_in) {
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const double g = gamma[bh % H];
        double* S = (double*)malloc((size_t)dk * dv * sizeof(double));
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = state_in ? state_in[(size_t)bh * dk * dv + e] : 0.0;
        for (int n = 0; n < N; ++n) {
            const double* kn = k + ((size_t)bh * N + n) * dk;
            const double* vn = v + ((size_t)bh * N + n) * dv;
            const double* gn = dout + ((size_t)bh * N + n) * dv;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kn[i] * vn[j];
            if (dq)
                for (int i = 0; i < dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < dv; ++j) a += gn[j] * S[(size_t)i * dv + j];
                    dq[((size_t)bh * N + n) * dk + i] = a;
                }
        }
        double* U = S;  /* reused: the forward state is no longer needed */
        for (size_t e = 0; e < (size_t)dk * dv; ++e) U[e] = 0.0;
        for (int n = N - 1; n >= 0; --n) {
            const double* qn = q + ((size_t)bh * N + n) * dk;
            const double* kn = k + ((size_t)bh * N + n) * dk;
            const double* vn = v + ((size_t)bh * N + n) * dv;
            const double* gn = dout + ((size_t)bh * N + n) * dv;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) U[(size_t)i * dv + j] = g * U[(size_t)i * dv + j] + qn[i] * gn[j];
            if (dkk)
                for (int i = 0; i < dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < dv; ++j) a += U[(size_t)i * dv + j] * vn[j];
                    dkk[((size_t)bh * N + n) * dk + i] = a;
                }
            if (dvv)
                for (int j = 0; j < dv; ++j) {
                    double a = 0.0;
                    for (int i = 0; i < dk; ++i) a += kn[i] * U[(size_t)i * dv + j];
                    dvv[((size_t)bh * N + n) * dv + j] = a;
                }
        }
        if (dstate_in)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) dstate_in[(size_t)bh * dk * dv + e] = g * U[e];
        free(S);
    }
}

/*
 * Parallel form (abeam.tech summary, "Retention multiplies content-based
 * reference and distance-based forgetting" and "Training in parallel"):
 *     o_n = sum_{m <= n} gamma^(n-m) (q_n . k_m) v_m
 * i.e. O = (Q K^T (.) D) V with D_nm = gamma^(n-m) for n >= m, else 0.
 * Quadratic in N: for small inputs only.
 */
void oracle_parallel(int B, int H, int N, int dk, int dv,
                     const double* q, const double* k, const double* v,
                     const double* gamma, double* out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        for (int n = 0; n < N; ++n) {
            const double* qn = q + ((size_t)bh * N + n) * dk;
            double* on = out + ((size_t)bh * N + n) * dv;
            memset(on, 0, (size_t)dv * sizeof(double));
            for (int m = 0; m <= n; ++m) {
                const double* km = k + ((size_t)bh * N + m) * dk;
                const double* vm = v + ((size_t)bh * N + m) * dv;
                double a = 0.0;
                for (int i = 0; i < dk; ++i) a += qn[i] * km[i];
                const double w = pow(g, (double)(n - m)) * a;
                for (int j = 0; j < dv; ++j) on[j] += w * vm[j];
            }
        }
    }
}

/*
 * Chunkwise recurrent form (abeam.tech summary, "Chunk recursion for
 * long-sequence training"; mlnews abstract: each chunk is encoded in
 * parallel while the chunks are summarised recurrently).
 * Chunk c covers positions c*C ... c*C+L-1 with L = C, or N mod C for a
 * short last chunk. With R the state carried in from earlier chunks
 * (state_in or zero), for local row j of the chunk:
 *     o_j = sum_{t <= j} gamma^(j-t) (q_j . k_t) v_t      (inside the chunk)
 *         + gamma^(j+1) q_j R                             (earlier chunks)
 * and at the end of the chunk
 *     R <- gamma^L R + sum_t gamma^(L-1-t) k_t^T v_t.
 * These are the recurrence unrolled over one chunk.
 */
void oracle_chunkwise(int B, int H, int N, int dk, int dv, int C,
                      const double* q, const double* k, const double* v,
                      const double* gamma, const double* state_in,
                      double* out, double* state_out) {
    const size_t sd = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const double g = gamma[bh % H];
        double* R = (double*)malloc(sd * sizeof(double));
        if (state_in) memcpy(R, state_in + (size_t)bh * sd, sd * sizeof(double));
        else memset(R, 0, sd * sizeof(double));
        for (int c0 = 0; c0 < N; c0 += C) {
            const int L = (N - c0 < C) ? (N - c0) : C;
            if (out) {
                for (int j = 0; j < L; ++j) {
                    const double* qj = q + ((size_t)bh * N + c0 + j) * dk;
                    double* oj = out + ((size_t)bh * N + c0 + j) * dv;
                    memset(oj, 0, (size_t)dv * sizeof(double));
                    const double xi = pow(g, (double)(j + 1));
                    for (int i = 0; i < dk; ++i) {
                        const double* Ri = R + (size_t)i * dv;
                        for (int col = 0; col < dv; ++col) oj[col] += xi * qj[i] * Ri[col];
                    }
                    for (int t = 0; t <= j; ++t) {
                        const double* kt = k + ((size_t)bh * N + c0 + t) * dk;
                        const double* vt = v + ((size_t)bh * N + c0 + t) * dv;
                        double a = 0.0;
                        for (int i = 0; i < dk; ++i) a += qj[i] * kt[i];
                        const double w = pow(g, (double)(j - t)) * a;
                        for (int col = 0; col < dv; ++col) oj[col] += w * vt[col];
                    }
                }
            }
            const double gL = pow(g, (double)L);
            for (size_t e = 0; e < sd; ++e) R[e] *= gL;
            for (int t = 0; t < L; ++t) {
                const double* kt = k + ((size_t)bh * N + c0 + t) * dk;
                const double* vt = v + ((size_t)bh * N + c0 + t) * dv;
                const double z = pow(g, (double)(L - 1 - t));
                for (int i = 0; i < dk; ++i) {
                    double* Ri = R + (size_t)i * dv;
                    for (int col = 0; col < dv; ++col) Ri[col] += z * kt[i] * vt[col];
                }
            }
        }
        if (state_out) memcpy(state_out + (size_t)bh * sd, R, sd * sizeof(double));
        free(R);
    }
}

/*
 * Per-head GroupNorm (mlnews bullet summary: retention outputs are
 * normalised per head with GroupNorm before the heads are concatenated;
 * abeam.tech summary, "Multi-timescale decay, gate and normalisation").
 * One group = the d_v channels of one head at one position, so each
 * row x of x[B][H][N][dv] is normalised on its own:
 *     mu = mean(x), var = mean((x - mu)^2)   (biased)
 *     y  = (x - mu) / sqrt(var + eps) * w[h][c] + b[h][c]
 * weight and bias are [H][dv]; NULL means 1 and 0.
 * Then the swish gate (same abeam.tech section: a Swish gate adds
 * non-linearity), read here as multiplying the normalised output by
 * swish(g) = g * sigmoid(g) = g / (1 + exp(-g)) of a given gate tensor g
 * laid out like x; NULL means no gate.
 */
void oracle_groupnorm(int B, int H, int N, int dv, double eps,
                      const double* weight, const double* bias, const double* gate,
                      const double* x, double* y) {
    const long rows = (long)B * H * N;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const int h = (int)((r / N) % H);
        const double* xr = x + (size_t)r * dv;
        double* yr = y + (size_t)r * dv;
        double mu = 0.0;
        for (int c = 0; c < dv; ++c) mu += xr[c];
        mu /= dv;
        double var = 0.0;
        for (int c = 0; c < dv; ++c) var += (xr[c] - mu) * (xr[c] - mu);
        var /= dv;
        const double inv = 1.0 / sqrt(var + eps);
        for (int c = 0; c < dv; ++c) {
            const double w = weight ? weight[(size_t)h * dv + c] : 1.0;
            const double b = bias ? bias[(size_t)h * dv + c] : 0.0;
            yr[c] = (xr[c] - mu) * inv * w + b;
            if (gate) {
                const double g = gate[(size_t)r * dv + c];
                yr[c] *= g / (1.0 + exp(-g));
            }
        }
    }
}

/*
 * Positional rotation of q and k (abeam.tech summary, "Technical mechanism",
 * subsection "Retention multiplies content-based reference and
 * distance-based forgetting": Q and K get a positional rotation after the
 * projections; eulerwa.com "3. RetNet 상세", list of advantages and the
 * comparison table: RoPE is the position encoding used with the decay).
 * The pages give no formula; the reading taken is the rotary position
 * embedding as published by Su et al. (RoFormer): at absolute position
 * p = offset + n, each pair of features (2i, 2i+1), i < d/2, is turned by
 * the angle p * theta_i with theta_i = base^(-2i/d):
 *     y[2i]   = x[2i] cos(p theta_i) - x[2i+1] sin(p theta_i)
 *     y[2i+1] = x[2i] sin(p theta_i) + x[2i+1] cos(p theta_i)
 * x, y: [rows][N][d] (rows = B*H), d even. direction = -1 turns by the
 * opposite angle (the inverse, which is the transpose: used for gradients).
 */
void oracle_rotate(long rows, int N, int d, double base, long long offset, int direction,
                   const double* x, double* y) {
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        for (int n = 0; n < N; ++n) {
            const double p = (double)(offset + n) * (direction < 0 ? -1.0 : 1.0);
            const double* xn = x + ((size_t)r * N + n) * d;
            double* yn = y + ((size_t)r * N + n) * d;
            for (int i = 0; i < d / 2; ++i) {
                const double theta = pow(base, -2.0 * i / d);
                const double c = cos(p * theta), s = sin(p * theta);
                const double a = xn[2 * i], b = xn[2 * i + 1];
                yn[2 * i] = a * c - b * s;
                yn[2 * i + 1] = a * s + b * c;
            }
        }
    }
}

/*
 * Feature map of residual linear attention (mengro1102.github.io RAttention post, section 4, the
 * RLA formula and its notes: phi is a feature map, softmax-based works best). The page gives no
 * formula; the reading taken is the softmax over the d features of one row,
 *     phi(x)_i = exp(x_i) / sum_j exp(x_j),
 * evaluated as exp(x_i - max x) / sum_j exp(x_j - max x). fmap 0 is the identity.
 */
static void rla_phi(int fmap, int d, const double* x, double* y) {
    if (fmap == 0) {
        for (int i = 0; i < d; ++i) y[i] = x[i];
        return;
    }
    double m = x[0];
    for (int i = 1; i < d; ++i) m = x[i] > m ? x[i] : m;
    double s = 0.0;
    for (int i = 0; i < d; ++i) {
        y[i] = exp(x[i] - m);
        s += y[i];
    }
    for (int i = 0; i < d; ++i) y[i] /= s;
}

void oracle_rla_phi(long rows, int d, int fmap, const double* x, double* y) {
    for (long r = 0; r < rows; ++r) rla_phi(fmap, d, x + (size_t)r * d, y + (size_t)r * d);
}

/*
 * Residual linear attention (same page, section 4, RLA formula):
 *     S_t = S_(t-1) + phi(k_t)^T v_t,     o_t = phi(q_t) S_(t-w-1)
 * i.e. the undecayed linear-attention state read w + 1 tokens late, so that o_t sees only the
 * tokens that have left the sliding window of the last w tokens and t itself.
 * One call covers positions 0 .. N-1 of a segment. The w + 1 positions before it (-(w+1) .. -1)
 * are rows 0 .. w of kp, vp ([B][H][w+1][dk], [B][H][w+1][dv]), of which only the last prev_len
 * hold tokens (positions -prev_len .. -1; the sequence starts after the others; prev_len = 0 and
 * NULL kp, vp at the start of a sequence), and state_in (or 0) is S_(-w-2), the sum over every
 * earlier token. With S_(t-w-1) = S_(t-w-2) + phi(k_(t-w-1))^T v_(t-w-1), the state read by o_t gains one
 * token per step. state_out is the state the last output read, S_(N-w-2): every token that has
 * left the window. It is the state_in of a following segment whose kp, vp are the last w + 1
 * tokens of this one (positions N-w-1 .. N-1, which the next segment adds one per step). w >= 0.
 */
void oracle_rla(int B, int H, int N, int dk, int dv, int w, int fmap,
                const double* q, const double* k, const double* v, const double* kp, const double* vp, int prev_len,
                const double* state_in, double* out, double* state_out) {
    const int P = w + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        double* S = (double*)malloc((size_t)dk * dv * sizeof(double));
        double* fq = (double*)malloc((size_t)dk * sizeof(double));
        double* fk = (double*)malloc((size_t)dk * sizeof(double));
        for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = state_in ? state_in[(size_t)bh * dk * dv + e] : 0.0;
        for (int t = 0; t < N; ++t) {
            /* the token at position t - w - 1 joins the state that o_t reads */
            const int p = t - P;
            const double* kt = NULL;
            const double* vt = NULL;
            if (p < 0) {
                if (kp && p >= -prev_len) {
                    kt = kp + ((size_t)bh * P + (p + P)) * dk;
                    vt = vp + ((size_t)bh * P + (p + P)) * dv;
                }
            } else {
                kt = k + ((size_t)bh * N + p) * dk;
                vt = v + ((size_t)bh * N + p) * dv;
            }
            if (kt) {
                rla_phi(fmap, dk, kt, fk);
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += fk[i] * vt[j];
            }
            rla_phi(fmap, dk, q + ((size_t)bh * N + t) * dk, fq);
            double* ot = out + ((size_t)bh * N + t) * dv;
            for (int j = 0; j < dv; ++j) {
                double a = 0.0;
                for (int i = 0; i < dk; ++i) a += fq[i] * S[(size_t)i * dv + j];
                ot[j] = a;
            }
        }
        if (state_out)
            for (size_t e = 0; e < (size_t)dk * dv; ++e) state_out[(size_t)bh * dk * dv + e] = S[e];
        free(S);
        free(fq);
        free(fk);
    }
}

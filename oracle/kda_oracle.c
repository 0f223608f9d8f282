/*
 * kda_oracle.c -- CPU fp64 reference for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * it.  It shares no source, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section; the pages are web articles about Kimi K3):
 *   [K3 note]  "Kimi K3: Architecture, Training, and Million-Token Agentic RL"
 *              (Awesome-LLM-Research-Collections note on the K3 technical report)
 *   [K3 hood]  "Kimi K3 Under the Hood: A 2.8T MoE Built for Million-Token Agents" (dev.to)
 *
 * What is computed, for every (sequence n, head h), token by token, in fp64:
 *   gate      g = g_min * Sigmoid(exp(A[h]) * z_t)  with g_min = -5, alpha = exp(g)
 *             ([K3 note] §3.3, lower-bounded decay equation; [K3 hood] "Sequence mixing",
 *             the retention parameterization)
 *   decay     Sbar = Diag(alpha) S_{t-1}        -- rows of S are key channels
 *   predict   vhat = Sbar^T k_t
 *   write     S_t  = Sbar + beta_t k_t (v_t - vhat)^T
 *   read      o_t  = S_t^T q_t                  -- after the write
 *             ([K3 note] §3.2, the rearranged edit/read order; §3.1, full KDA recurrence
 *             S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, o_t = S_t^T q_t)
 * The state S is d_k x d_v per head and starts from a caller-given state or from zero
 * ([K3 note] §3.1 fixed-shape state; prefix-cache restore in [K3 hood] "Serving two
 * incompatible cache types").  No scale is applied to q: o = S^T q exactly as printed.
 *
 * Inputs are the exact values the GPU receives (bf16 values are passed widened to fp32),
 * so input quantisation is not counted as kernel error.  Arithmetic is plain IEEE double,
 * compiled without fast-math.  OpenMP runs independent (n, h) pairs in parallel; each
 * pair's token loop is serial.
 *
 * Every function here is pinned by the CPU tests (closed forms, invariants, brute force,
 * an independent chunked derivation and planted-mistake detection); none is "parity
 * unpinned".
 *
 * KDA_ORACLE_MUTANT (compile-time, tests only): plants one known mistake so the tests
 * can show that their pins catch it.  0 (default) is the correct oracle.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0
#endif

#define KDA_ORACLE_OK 0
#define KDA_ORACLE_EINVAL (-1)
#define KDA_ORACLE_ENOMEM (-2)

int kda_oracle_mutant(void) { return KDA_ORACLE_MUTANT; }

/* Lower-bounded gate, one element.  [K3 note] §3.3: g = g_min * Sigmoid(e^A z). */
static double gate_one(double a_log, double z, double g_min)
{
#if KDA_ORACLE_MUTANT == 6
    double x = a_log * z;            /* planted: e^A replaced by A */
#else
    double x = exp(a_log) * z;
#endif
#if KDA_ORACLE_MUTANT == 7
    double s = 1.0 / (1.0 + exp(x)); /* planted: Sigmoid(-x) */
#else
    /* Sigmoid(x) = 1 / (1 + e^-x).  For x -> -inf, e^-x = inf and the quotient is 0;
     * for x -> +inf it is 1.  No NaN for finite x. */
    double s = 1.0 / (1.0 + exp(-x));
#endif
    return g_min * s;
}

/* g[t,h,c] for a [T, H, dk] block of decay logits z and per-(head, channel) A [H, dk]. */
void kda_oracle_gate(const float *z, const float *A, double g_min, int64_t n_tokens, int H,
                     int dk, double *g_out)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n_tokens; ++t) {
        for (int h = 0; h < H; ++h) {
            for (int c = 0; c < dk; ++c) {
                size_t i = ((size_t)t * H + h) * dk + c;
                g_out[i] = gate_one((double)A[(size_t)h * dk + c], (double)z[i], g_min);
            }
        }
    }
}

/* Start token of sequence n: cu_seqlens[n] if given, else n * T (equal-length batch). */
static int64_t seq_start(const int32_t *cu, int64_t T, int n)
{
    return cu ? (int64_t)cu[n] : (int64_t)n * T;
}

/*
 * Chunk-local inclusive cumulative log-decay: out[t] = sum of g over the tokens of t's chunk
 * up to and including t.  Chunks have `chunk` tokens and restart at every sequence start;
 * the last chunk of a sequence may be shorter.  This is the quantity whose reciprocal the
 * lower bound keeps finite ([K3 note] §3.3, reciprocal cumulative decay and the 16-token
 * tile bound).
 */
int kda_oracle_chunk_cumsum(const double *g, const int32_t *cu, int N, int64_t T, int H, int dk,
                            int chunk, double *out)
{
    if (!g || !out || N < 0 || H <= 0 || dk <= 0 || chunk <= 0) return KDA_ORACLE_EINVAL;
    int n;
#pragma omp parallel for schedule(dynamic)
    for (n = 0; n < N; ++n) {
        int64_t s0 = seq_start(cu, T, n), s1 = seq_start(cu, T, n + 1);
        if (!cu) s1 = s0 + T;
        size_t row = (size_t)H * dk;
        for (size_t col = 0; col < row; ++col) {
            double acc = 0.0;
            for (int64_t t = s0; t < s1; ++t) {
#if KDA_ORACLE_MUTANT == 8
                if ((t - s0) % chunk == 0) acc = 0.0;
                out[(size_t)t * row + col] = acc;           /* planted: exclusive sum */
                acc += g[(size_t)t * row + col];
#elif KDA_ORACLE_MUTANT == 9
                if (t % chunk == 0) acc = 0.0;             /* planted: global alignment */
                acc += g[(size_t)t * row + col];
                out[(size_t)t * row + col] = acc;
#else
                if ((t - s0) % chunk == 0) acc = 0.0;
                acc += g[(size_t)t * row + col];
                out[(size_t)t * row + col] = acc;
#endif
            }
        }
    }
    return KDA_ORACLE_OK;
}

/*
 * One token of the recurrence on a single head's state S [dk, dv] (row-major, rows = key
 * channels).  alpha[c] = exp(g[c]).  Writes o[dv] = S_t^T q after the update.
 * [K3 note] §3.2: decay, predict at the edit address, write the error, then read.
 */
static void recur_token(double *S, int dk, int dv, const double *alpha, const float *q,
                        const float *k, const float *v, double beta, double *vhat, double *o)
{
    int c, j;
#if KDA_ORACLE_MUTANT == 1
    /* planted: decay columns (value channels) instead of rows; needs dk == dv */
    for (c = 0; c < dk; ++c)
        for (j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= alpha[j % dk];
#elif KDA_ORACLE_MUTANT == 2
    /* planted: decay applied after the edit instead of before it (below) */
#else
    for (c = 0; c < dk; ++c) {
        double a = alpha[c];
        double *row = S + (size_t)c * dv;
        for (j = 0; j < dv; ++j) row[j] *= a;          /* Sbar = Diag(alpha) S */
    }
#endif
#if KDA_ORACLE_MUTANT == 3
    /* planted: read before the write */
    for (j = 0; j < dv; ++j) o[j] = 0.0;
    for (c = 0; c < dk; ++c) {
        double qc = (double)q[c];
        const double *row = S + (size_t)c * dv;
        for (j = 0; j < dv; ++j) o[j] += row[j] * qc;
    }
#endif
    for (j = 0; j < dv; ++j) vhat[j] = 0.0;
    for (c = 0; c < dk; ++c) {                          /* vhat = Sbar^T k */
#if KDA_ORACLE_MUTANT == 12
        double kc = (double)q[c];                       /* planted: predicted at q, not k */
#else
        double kc = (double)k[c];
#endif
        const double *row = S + (size_t)c * dv;
        for (j = 0; j < dv; ++j) vhat[j] += row[j] * kc;
    }
    for (j = 0; j < dv; ++j) {
#if KDA_ORACLE_MUTANT == 4
        vhat[j] = beta * (double)v[j] - vhat[j];       /* planted: erase not scaled by beta */
#elif KDA_ORACLE_MUTANT == 5
        vhat[j] = -beta * ((double)v[j] - vhat[j]);     /* planted: sign of the write */
#else
        vhat[j] = beta * ((double)v[j] - vhat[j]);      /* u = beta (v - vhat) */
#endif
    }
    for (c = 0; c < dk; ++c) {                          /* S = Sbar + k u^T */
        double kc = (double)k[c];
        double *row = S + (size_t)c * dv;
        for (j = 0; j < dv; ++j) row[j] += kc * vhat[j];
    }
#if KDA_ORACLE_MUTANT == 2
    for (c = 0; c < dk; ++c)
        for (j = 0; j < dv; ++j) S[(size_t)c * dv + j] *= alpha[c];
#endif
#if KDA_ORACLE_MUTANT != 3
    for (j = 0; j < dv; ++j) o[j] = 0.0;
    for (c = 0; c < dk; ++c) {                          /* o = S_t^T q (read after write) */
#if KDA_ORACLE_MUTANT == 10
        double qc = (double)k[c];                       /* planted: read with k, not q */
#else
        double qc = (double)q[c];
#endif
        const double *row = S + (size_t)c * dv;
        for (j = 0; j < dv; ++j) o[j] += row[j] * qc;
    }
#endif
}

/*
 * Per-token alpha for head h: from the given log-decay g (fp64, [*, H, dk]) when g is not
 * NULL, else from the gate on z and A.
 */
static void token_alpha(const double *g, const float *z, const float *A, double g_min,
                        size_t tok_off, int h, int dk, double *alpha)
{
    for (int c = 0; c < dk; ++c) {
        double gc = g ? g[tok_off + c]
                      : gate_one((double)A[(size_t)h * dk + c], (double)z[tok_off + c], g_min);
#if KDA_ORACLE_MUTANT == 11
        alpha[c] = exp(-gc);                             /* planted: e^-g, growth, not decay */
#else
        alpha[c] = exp(gc);                              /* alpha = e^g */
#endif
    }
}

/*
 * Prefill / token recurrence over packed sequences.
 *
 *   q, k, z : [total, H, dk]  fp32 (bf16 inputs passed widened)
 *   v       : [total, H, dv]
 *   beta    : [total, H]
 *   A       : [H, dk]         used only when g == NULL
 *   g       : [total, H, dk]  fp64 log-decay, or NULL to apply the gate to z and A
 *   S0      : [N, H, dk, dv]  fp32 initial state, or NULL for zeros
 *   cu      : [N + 1] host int32 sequence starts, or NULL for N sequences of length T
 *   pairs   : [n_pairs, 2] (n, h) pairs to compute, or NULL for all N*H in (n, h) order
 *   o_out   : packed per pair: pair p's outputs are rows [off_p, off_p + L_n) of a
 *             [sum L, dv] fp64 array, off_p = sum of the lengths of the earlier pairs
 *   S_out   : [n_pairs, dk, dv] fp64 final states, or NULL
 *   n_threads <= 0 keeps the OpenMP default.
 */
int kda_oracle_prefill(const float *q, const float *k, const float *v, const float *beta,
                       const float *z, const float *A, const double *g, double g_min,
                       const float *S0, const int32_t *cu, int N, int64_t T, int H, int dk,
                       int dv, const int32_t *pairs, int n_pairs, double *o_out,
                       double *S_out, int n_threads)
{
    if (!q || !k || !v || !beta || !o_out || N < 0 || H <= 0 || dk <= 0 || dv <= 0)
        return KDA_ORACLE_EINVAL;
    if (!g && (!z || !A)) return KDA_ORACLE_EINVAL;
    if (!cu && T < 0) return KDA_ORACLE_EINVAL;
    int np = pairs ? n_pairs : N * H;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * ((size_t)np + 1));
    if (!off) return KDA_ORACLE_ENOMEM;
    off[0] = 0;
    for (int p = 0; p < np; ++p) {
        int n = pairs ? pairs[2 * p] : p / H;
        int h = pairs ? pairs[2 * p + 1] : p % H;
        if (n < 0 || n >= N || h < 0 || h >= H) { free(off); return KDA_ORACLE_EINVAL; }
        int64_t s0 = seq_start(cu, T, n), s1 = cu ? seq_start(cu, T, n + 1) : s0 + T;
        if (s1 < s0) { free(off); return KDA_ORACLE_EINVAL; }
        off[p + 1] = off[p] + (s1 - s0);
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int failed = 0;
    int p;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (p = 0; p < np; ++p) {
        int n = pairs ? pairs[2 * p] : p / H;
        int h = pairs ? pairs[2 * p + 1] : p % H;
        int64_t s0 = seq_start(cu, T, n), s1 = cu ? seq_start(cu, T, n + 1) : s0 + T;
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !alpha || !tmp) {
            free(S); free(alpha); free(tmp);
            failed |= 1;
            continue;
        }
        if (S0) {
            const float *src = S0 + ((size_t)n * H + h) * (size_t)dk * dv;
            for (size_t i = 0; i < (size_t)dk * dv; ++i) S[i] = (double)src[i];
        } else {
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
        }
        for (int64_t t = s0; t < s1; ++t) {
            size_t tk = ((size_t)t * H + h) * dk;
            size_t tv = ((size_t)t * H + h) * dv;
            token_alpha(g, z, A, g_min, tk, h, dk, alpha);
            recur_token(S, dk, dv, alpha, q + tk, k + tk, v + tv,
                        (double)beta[(size_t)t * H + h], tmp,
                        o_out + (size_t)(off[p] + (t - s0)) * dv);
        }
        if (S_out) memcpy(S_out + (size_t)p * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(alpha); free(tmp);
    }
    free(off);
    return failed ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * One decode step: every listed (n, h) pair advances its fp64 state by one token.
 * [K3 note] §3.2, the per-token map (x_t, S_{t-1}) -> (y_t, S_t); §3.3 recurrent decoding.
 *
 *   q, k, z : [N, H, dk]; v : [N, H, dv]; beta : [N, H]; A : [H, dk]
 *   S       : [n_pairs, dk, dv] fp64, read and written in place
 *   o_out   : [n_pairs, dv] fp64
 */
int kda_oracle_decode_step(const float *q, const float *k, const float *v, const float *beta,
                           const float *z, const float *A, double g_min, double *S, int N,
                           int H, int dk, int dv, const int32_t *pairs, int n_pairs,
                           double *o_out, int n_threads)
{
    if (!q || !k || !v || !beta || !z || !A || !S || !o_out || N < 0 || H <= 0 || dk <= 0 ||
        dv <= 0)
        return KDA_ORACLE_EINVAL;
    int np = pairs ? n_pairs : N * H;
    for (int p = 0; p < np; ++p) {
        int n = pairs ? pairs[2 * p] : p / H;
        int h = pairs ? pairs[2 * p + 1] : p % H;
        if (n < 0 || n >= N || h < 0 || h >= H) return KDA_ORACLE_EINVAL;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int failed = 0;
    int p;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (p = 0; p < np; ++p) {
        int n = pairs ? pairs[2 * p] : p / H;
        int h = pairs ? pairs[2 * p + 1] : p % H;
        double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!alpha || !tmp) {
            free(alpha); free(tmp);
            failed |= 1;
            continue;
        }
        size_t tk = ((size_t)n * H + h) * dk;
        size_t tv = ((size_t)n * H + h) * dv;
        token_alpha(NULL, z, A, g_min, tk, h, dk, alpha);
        recur_token(S + (size_t)p * dk * dv, dk, dv, alpha, q + tk, k + tk, v + tv,
                    (double)beta[(size_t)n * H + h], tmp, o_out + (size_t)p * dv);
        free(alpha); free(tmp);
    }
    return failed ? KDA_ORACLE_ENOMEM : KDA_ORACLE_OK;
}

/*
 * Output epilogue, per row (one token of one head): y = Sigmoid(gate) * RMSNorm(o) with
 * RMSNorm(o) = o / sqrt(mean(o^2) + eps) * w.  [K3 note] §3.2: the K3 output path is
 * W_o[Sigmoid(W_g x_t) (.) RMSNorm(o~_t)]; the projections need trained weights, so the gate
 * logits (W_g x_t) arrive as an input.  The pages do not spell out RMSNorm; the plain
 * reading taken here: root mean square over the head's d_v readout channels, a per-channel
 * weight w, and an additive eps inside the root.
 */
void kda_oracle_output_gate(const float *o, const float *gate, const float *w, double eps,
                            int64_t rows, int dv, double *y)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float *orow = o + r * dv, *grow = gate + r * dv;
        double ss = 0.0;
        for (int c = 0; c < dv; ++c) ss += (double)orow[c] * (double)orow[c];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int c = 0; c < dv; ++c) {
            const double sg = 1.0 / (1.0 + exp(-(double)grow[c]));
            y[r * dv + c] = (double)orow[c] * inv * (double)w[c] * sg;
        }
    }
}

/*
 * Input prologue ([K3 note] §3.2): q, k = L2Norm(Swish(ShortConv(W x))) and
 * v = Swish(ShortConv(W_v x)); during decoding ShortConv also reads the layer's short
 * convolution cache C^conv of the few most recent inputs, and writes it back.  The
 * projections W x need trained weights, so the projected inputs x arrive as an input.
 * Readings of what the pages leave open: ShortConv is a causal depthwise convolution over
 * time of width Wk per channel, out_t[c] = sum_i w[c][i] * x_{t-Wk+1+i}[c] (the last tap
 * multiplies the current token); inputs before a sequence's first token come from cache_in
 * (the Wk-1 most recent earlier inputs, oldest first) or are zero; Swish(u) = u Sigmoid(u);
 * L2Norm divides each group of l2_group channels (one head) by sqrt(sum u^2 + 1e-6).
 * cache_out receives the last Wk-1 inputs of each sequence, reaching back into cache_in
 * for short sequences.
 *
 * x [total, C] (fp32 values), w [C, Wk], cache_in/out [N, C, Wk-1] (nullable), y [total, C].
 */
int kda_oracle_short_conv(const float *x, const float *w, int Wk, const float *cache_in,
                          double *cache_out, const int32_t *cu, int N, int64_t T, int C,
                          int l2_group, double *y)
{
    if (Wk < 1 || C <= 0 || N <= 0 || (l2_group > 0 && C % l2_group != 0)) return KDA_ORACLE_EINVAL;
    const int hist = Wk - 1;
    for (int n = 0; n < N; ++n) {
        const int64_t s0 = seq_start(cu, T, n), s1 = seq_start(cu, T, n + 1);
        const int64_t L = s1 - s0;
        for (int64_t t = 0; t < L; ++t) {
            double *yrow = y + (s0 + t) * C;
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int i = 0; i < Wk; ++i) {
                    const int64_t p = t - hist + i;  /* position inside the sequence */
                    double xv;
                    if (p >= 0) xv = x[(s0 + p) * C + c];
                    else xv = cache_in ? cache_in[((int64_t)n * C + c) * hist + (hist + p)] : 0.0;
                    acc += (double)w[(int64_t)c * Wk + i] * xv;
                }
                yrow[c] = acc / (1.0 + exp(-acc));  /* Swish */
            }
            if (l2_group > 0) {
                for (int g0 = 0; g0 < C; g0 += l2_group) {
                    double ss = 0.0;
                    for (int c = g0; c < g0 + l2_group; ++c) ss += yrow[c] * yrow[c];
                    const double inv = 1.0 / sqrt(ss + 1e-6);
                    for (int c = g0; c < g0 + l2_group; ++c) yrow[c] *= inv;
                }
            }
        }
        if (cache_out && hist > 0) {
            for (int c = 0; c < C; ++c)
                for (int j = 0; j < hist; ++j) {
                    const int64_t p = L - hist + j;
                    double xv;
                    if (p >= 0) xv = x[(s0 + p) * C + c];
                    else xv = cache_in ? cache_in[((int64_t)n * C + c) * hist + (hist + p)] : 0.0;
                    cache_out[((int64_t)n * C + c) * hist + j] = xv;
                }
        }
    }
    return KDA_ORACLE_OK;
}

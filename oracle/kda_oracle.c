/*
 * kda_oracle.c - plain float64 CPU oracle of the Kimi Delta Attention (KDA)
 * gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with
 * the HIP library; both sides only see the same seeded inputs.
 *
 * What it computes (token by token, in float64, no blocking or reordering):
 *
 *   Prologue, per token and head (AWS Neuron "KDA TKG Kernel API Reference",
 *   parameter list of kda_tkg: q/k are raw "pre-L2-norm", the scale is folded
 *   into the normalised query, g is activated as
 *   lower_bound * sigmoid(exp(a_log) * (g + dt_bias)), beta arrives as logits):
 *       qh = scale * q / sqrt(sum q^2 + eps)     (without L2 norm: scale * q)
 *       kh = k / sqrt(sum k^2 + eps)             (without L2 norm: k)
 *       gamma_i = lb * sigmoid(exp(a_log[h]) * (g_i + dt_bias[i,h]))
 *       beta = sigmoid(beta_logit)
 *
 *   KDA step (decay first, residual against the decayed state, then output):
 *       S    <- Diag(exp(gamma)) S
 *       u    =  S^T kh
 *       S    <- S + beta * kh (v - u)^T
 *       o    =  S^T qh
 *
 *   EJK step (ejkernel "kernel_delta_attention" page, "The core recurrence":
 *   scalar per-head decay d, beta used as given, residual against the
 *   undecayed state):
 *       u    =  S^T kh
 *       S    <- exp(d) S + beta * kh (v - u)^T
 *       o    =  S^T qh
 *
 *   The page writes h_{t-1} @ k_t and h_t @ q_t; with a [dk, dv] state and a
 *   [.., v_head_dim] output the contraction is over dk, i.e. S^T k and S^T q.
 *
 *   Variable-length packing (ejkernel "recurrent" page, run() parameter
 *   cu_seqlens, cumulative sequence lengths): sequence n covers tokens
 *   [cu[n], cu[n+1]); each sequence starts from its own initial state (or
 *   zeros) and returns its own final state.
 *
 *   Grouped heads (ejkernel "recurrent" page, run(): query has num_heads,
 *   key and value num_kv_heads; gates, state and output num_heads): head h
 *   takes the key and value of head h / (H / Hkv).
 *
 * Layouts (row-major): q [Ntok, H, dk]; k [Ntok, Hkv, dk]; v [Ntok, Hkv, dv];
 * g [Ntok, H, dk] (KDA) or [Ntok, H] (EJK, may be NULL = no decay);
 * beta [Ntok, H]; a_log [H]; dt_bias [dk, H]; states [N, H, dk, dv];
 * o [Ntok, H, dv].  Decode uses the kda_tkg layouts: q, g [B, dk, H];
 * k [B, dk, Hkv]; v [B, Hkv, dv]; beta [B, H]; out [B, H, dv];
 * S [B, H, dk, dv] advanced in place.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Query/key normalisation (ejkernel use_qk_l2norm; kda_tkg raw q/k). */
static void oracle_normalise(const double* x, long stride, int d, int use_l2norm,
                             double eps, double mult, double* out)
{
    double ss = 0.0;
    if (use_l2norm) {
        for (int i = 0; i < d; ++i) ss += x[i * stride] * x[i * stride];
        mult = mult / sqrt(ss + eps);
    }
    for (int i = 0; i < d; ++i) out[i] = mult * x[i * stride];
}

/* Per-channel log-decay gamma (kda_tkg parameter "g"). */
static void oracle_gate(const double* g, long stride, const double* dt_bias, int H, int h,
                        double a_log_h, double lb, int dk, double* gamma)
{
    const double ea = exp(a_log_h);
    for (int i = 0; i < dk; ++i)
        gamma[i] = lb * oracle_sigmoid(ea * (g[i * stride] + (dt_bias ? dt_bias[(long)i * H + h] : 0.0)));
}

/* One recurrence step on S[dk][dv]; writes o[dv].  u is dv scratch. */
static void oracle_step(double* S, int dk, int dv, const double* qh, const double* kh,
                        const double* v, long vstride, const double* gamma, double d_ejk,
                        double beta, int ejk, double* o, long ostride, double* u)
{
    if (!ejk) {
        for (int i = 0; i < dk; ++i) {
            const double a = exp(gamma[i]);
            for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= a;
        }
    }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * kh[i];
        u[j] = acc;
    }
    const double a = ejk ? exp(d_ejk) : 1.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(long)i * dv + j] = a * S[(long)i * dv + j] + beta * kh[i] * (v[j * vstride] - u[j]);
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * qh[i];
        o[j * ostride] = acc;
    }
}

static double oracle_resolve_scale(double scale, int dk)
{
    /* ejkernel softmax_scale: None means head_dim^-0.5 */
    if (!(scale > 0.0)) return 1.0 / sqrt((double)dk);
    return scale;
}

int kda_oracle_prefill(const double* q, const double* k, const double* v, const double* g,
                       const double* beta, const double* a_log, const double* dt_bias,
                       const double* initial_state, const int64_t* cu_seqlens, int n_seqs,
                       int H, int Hkv, int dk, int dv, double scale, double lower_bound, double eps,
                       int use_l2norm, int ejk, const int32_t* units, int n_units,
                       double* o, double* final_state, int n_threads)
{
    if (n_seqs < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    scale = oracle_resolve_scale(scale, dk);
    const int total = units ? n_units : n_seqs * H;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int w = 0; w < total; ++w) {
        const int unit = units ? units[w] : w;
        const int n = unit / H, h = unit % H;
        const int hk = h / (H / Hkv);   /* key/value head of head h */
        if (n < 0 || n >= n_seqs) { bad |= 1; continue; }
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gam = (double*)malloc(sizeof(double) * (size_t)dk);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        const size_t sz = (size_t)dk * dv;
        const size_t soff = ((size_t)n * H + h) * sz;
        if (initial_state) memcpy(S, initial_state + soff, sizeof(double) * sz);
        else memset(S, 0, sizeof(double) * sz);
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const size_t th = (size_t)t * H + h;
            const size_t tkv = (size_t)t * Hkv + hk;
            oracle_normalise(q + th * dk, 1, dk, use_l2norm, eps, scale, qh);
            oracle_normalise(k + tkv * dk, 1, dk, use_l2norm, eps, 1.0, kh);
            double b, d = 0.0;
            if (!ejk) {
                oracle_gate(g + th * dk, 1, dt_bias, H, h, a_log[h], lower_bound, dk, gam);
                b = oracle_sigmoid(beta[th]);
            } else {
                d = g ? g[th] : 0.0;
                b = beta[th];
            }
            oracle_step(S, dk, dv, qh, kh, v + tkv * dv, 1, gam, d, b, ejk, o + th * dv, 1, u);
        }
        if (final_state) memcpy(final_state + soff, S, sizeof(double) * sz);
        free(S); free(qh); free(kh); free(gam); free(u);
    }
    return bad ? 1 : 0;
}

int kda_oracle_decode(const double* q, const double* k, const double* g, const double* v,
                      const double* beta, const double* a_log, const double* dt_bias,
                      double scale, double lower_bound, double eps, int B, int H, int Hkv, int dk,
                      int dv, int use_l2norm, int ejk, double* out, double* S, int n_threads)
{
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || dk <= 0 || dv <= 0) return 1;
    scale = oracle_resolve_scale(scale, dk);
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(static)
    for (int w = 0; w < B * H; ++w) {
        const int b = w / H, h = w % H;
        const int hk = h / (H / Hkv);   /* key/value head of head h */
        double* qv = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kv = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gam = (double*)malloc(sizeof(double) * (size_t)dk);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        /* q, g are [B, dk, H]: element i of item (b, h) sits at (b*dk + i)*H + h;
           k is [B, dk, Hkv] and v [B, Hkv, dv] */
        const double* qb = q + (size_t)b * dk * H + h;
        const double* kb = k + (size_t)b * dk * Hkv + hk;
        oracle_normalise(qb, H, dk, use_l2norm, eps, scale, qv);
        oracle_normalise(kb, Hkv, dk, use_l2norm, eps, 1.0, kv);
        double bt, d = 0.0;
        if (!ejk) {
            oracle_gate(g + (size_t)b * dk * H + h, H, dt_bias, H, h, a_log[h], lower_bound, dk, gam);
            bt = oracle_sigmoid(beta[(size_t)b * H + h]);
        } else {
            d = g ? g[(size_t)b * H + h] : 0.0;
            bt = beta[(size_t)b * H + h];
        }
        oracle_step(S + (size_t)w * dk * dv, dk, dv, qv, kv, v + ((size_t)b * Hkv + hk) * dv, 1, gam, d, bt, ejk,
                    out + (size_t)w * dv, 1, u);
        free(qv); free(kv); free(gam); free(u);
    }
    return 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

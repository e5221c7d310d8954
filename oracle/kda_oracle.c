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

/*
 * Backward pass (reverse-mode gradient) of kda_oracle_prefill, token by token
 * in float64.  The forward pass is the one above; the reverse sweep runs the
 * chain rule back through each step, in reverse token order, then through the
 * prologue.  Given dO = dL/do [Ntok, H, dv] and dS_T = dL/d(final state)
 * (NULL = 0), it returns dL/d of every input: q, k, v, the raw gate g (KDA) or
 * the decay d (EJK), the beta logits (KDA) or beta (EJK), a_log, dt_bias and
 * the initial state.
 *
 * Per token, with S_prev the state before the step and S the state after it:
 *   KDA forward: a = exp(gamma); Sd = Diag(a) S_prev; u = Sd^T kh; e = v - u;
 *                S = Sd + beta kh e^T; o = S^T qh
 *   reverse:     dS += qh dO^T;            dqh = S dO
 *                de = beta dS^T kh;         dbeta = kh^T dS e;   dkh = beta dS e
 *                dv = de;                   dSd = dS - kh de^T;  dkh -= Sd de
 *                dgamma_i = a_i sum_j S_prev_ij dSd_ij;           dS <- Diag(a) dSd
 *   EJK forward: u = S_prev^T kh; e = v - u; S = exp(d) S_prev + beta kh e^T; o = S^T qh
 *   reverse:     as above with Sd = S_prev in the residual and
 *                dd = exp(d) sum_ij S_prev_ij dS_ij;  dS <- exp(d) dS - kh de^T
 *   prologue:    qh = s q / n_q, n_q = sqrt(q.q + eps): dq = s (dqh / n_q - q (q.dqh) / n_q^3)
 *                kh = k / n_k:                        dk = dkh / n_k - k (k.dkh) / n_k^3
 *                (without the L2 norm: dq = s dqh, dk = dkh)
 *                gamma = lb sigmoid(x), x = exp(a_log) (g + dt_bias):
 *                    dx = dgamma lb sigmoid(x) (1 - sigmoid(x));  dg = dx exp(a_log);
 *                    d dt_bias += dg;  d a_log += dx x
 *                beta = sigmoid(l): dl = dbeta beta (1 - beta)
 * The states a reverse step needs are recomputed from checkpoints taken every
 * 64 tokens by the forward pass (the same forward step, rerun).
 * Grouped heads: dk and dv of a key/value head sum over the heads that read it.
 */
#define ORACLE_CKPT 64

int kda_oracle_backward(const double* q, const double* k, const double* v, const double* g,
                        const double* beta, const double* a_log, const double* dt_bias,
                        const double* initial_state, const int64_t* cu_seqlens, int n_seqs,
                        int H, int Hkv, int dk, int dv, double scale, double lower_bound, double eps,
                        int use_l2norm, int ejk, const double* dO, const double* dS_final,
                        double* dq, double* dk_out, double* dv_out, double* dg, double* dbeta,
                        double* da_log, double* ddt_bias, double* dS0, int n_threads)
{
    if (n_seqs < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    scale = oracle_resolve_scale(scale, dk);
    const int64_t ntok = n_seqs > 0 ? cu_seqlens[n_seqs] : 0;
    const int G = H / Hkv;
    /* per query head: dk and dv before the group sum; per unit: parameter partials */
    double* dkq = (double*)calloc((size_t)(ntok > 0 ? ntok : 1) * H * dk, sizeof(double));
    double* dvq = (double*)calloc((size_t)(ntok > 0 ? ntok : 1) * H * dv, sizeof(double));
    double* da_part = (double*)calloc((size_t)(n_seqs > 0 ? n_seqs : 1) * H, sizeof(double));
    double* ddt_part = (double*)calloc((size_t)(n_seqs > 0 ? n_seqs : 1) * H * dk, sizeof(double));
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int w = 0; w < n_seqs * H; ++w) {
        const int n = w / H, h = w % H;
        const int hk = h / G;
        const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
        const int64_t L = t1 - t0;
        const size_t sz = (size_t)dk * dv;
        const size_t soff = ((size_t)n * H + h) * sz;
        const int nck = (int)((L + ORACLE_CKPT - 1) / ORACLE_CKPT);
        double* ck = (double*)malloc(sizeof(double) * sz * (size_t)(nck + 1));
        double* Sb = (double*)malloc(sizeof(double) * sz * (ORACLE_CKPT + 1));
        double* dS = (double*)malloc(sizeof(double) * sz);
        double* dSd = (double*)malloc(sizeof(double) * sz);
        double* qh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* gam = (double*)malloc(sizeof(double) * (size_t)dk);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        double* e = (double*)malloc(sizeof(double) * (size_t)dv);
        double* de = (double*)malloc(sizeof(double) * (size_t)dv);
        double* otmp = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dqh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* dkh = (double*)malloc(sizeof(double) * (size_t)dk);
        double* dgam = (double*)malloc(sizeof(double) * (size_t)dk);
        /* the prologue of token t (the same functions as the forward pass) */
#define PROLOGUE(t)                                                                              \
        const size_t th = (size_t)(t) * H + h, tkv = (size_t)(t) * Hkv + hk;                    \
        oracle_normalise(q + th * dk, 1, dk, use_l2norm, eps, scale, qh);                        \
        oracle_normalise(k + tkv * dk, 1, dk, use_l2norm, eps, 1.0, kh);                         \
        double bt, dd = 0.0;                                                                     \
        if (!ejk) {                                                                              \
            oracle_gate(g + th * dk, 1, dt_bias, H, h, a_log[h], lower_bound, dk, gam);          \
            bt = oracle_sigmoid(beta[th]);                                                       \
        } else {                                                                                 \
            dd = g ? g[th] : 0.0;                                                                \
            bt = beta[th];                                                                       \
        }
        /* forward: checkpoints of the state before tokens 0, 64, 128, ... */
        if (initial_state) memcpy(ck, initial_state + soff, sizeof(double) * sz);
        else memset(ck, 0, sizeof(double) * sz);
        memcpy(Sb, ck, sizeof(double) * sz);
        for (int64_t j = 0; j < L; ++j) {
            if (j > 0 && j % ORACLE_CKPT == 0) memcpy(ck + (size_t)(j / ORACLE_CKPT) * sz, Sb, sizeof(double) * sz);
            PROLOGUE(t0 + j)
            (void)dd;
            oracle_step(Sb, dk, dv, qh, kh, v + tkv * dv, 1, gam, dd, bt, ejk, otmp, 1, u);
        }
        /* reverse sweep */
        if (dS_final) memcpy(dS, dS_final + soff, sizeof(double) * sz);
        else memset(dS, 0, sizeof(double) * sz);
        double da = 0.0;
        double* ddt = ddt_part + (size_t)w * dk;
        for (int c = nck - 1; c >= 0; --c) {
            const int64_t j0 = (int64_t)c * ORACLE_CKPT;
            const int64_t j1 = (j0 + ORACLE_CKPT < L) ? j0 + ORACLE_CKPT : L;
            /* Sb[m] = state before token j0 + m, Sb[j1 - j0] = state after the block */
            memcpy(Sb, ck + (size_t)c * sz, sizeof(double) * sz);
            for (int64_t j = j0; j < j1; ++j) {
                double* Sn = Sb + (size_t)(j - j0 + 1) * sz;
                memcpy(Sn, Sb + (size_t)(j - j0) * sz, sizeof(double) * sz);
                PROLOGUE(t0 + j)
                oracle_step(Sn, dk, dv, qh, kh, v + tkv * dv, 1, gam, dd, bt, ejk, otmp, 1, u);
            }
            for (int64_t j = j1 - 1; j >= j0; --j) {
                const double* Sp = Sb + (size_t)(j - j0) * sz;      /* before the step */
                const double* Sa = Sb + (size_t)(j - j0 + 1) * sz;  /* after the step */
                PROLOGUE(t0 + j)
                const double* vt = v + tkv * dv;
                const double* dot = dO + th * dv;
                /* Sd: the state the residual is taken against */
                if (!ejk) {
                    for (int i = 0; i < dk; ++i) {
                        const double a = exp(gam[i]);
                        for (int jj = 0; jj < dv; ++jj) dSd[(size_t)i * dv + jj] = a * Sp[(size_t)i * dv + jj];
                    }
                } else {
                    memcpy(dSd, Sp, sizeof(double) * sz);
                }
                const double* Sd = dSd;   /* holds Sd until it is overwritten below */
                for (int jj = 0; jj < dv; ++jj) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i) acc += Sd[(size_t)i * dv + jj] * kh[i];
                    e[jj] = vt[jj] - acc;
                }
                /* o = S^T qh */
                for (int i = 0; i < dk; ++i)
                    for (int jj = 0; jj < dv; ++jj) dS[(size_t)i * dv + jj] += qh[i] * dot[jj];
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int jj = 0; jj < dv; ++jj) acc += Sa[(size_t)i * dv + jj] * dot[jj];
                    dqh[i] = acc;
                }
                /* S = Sd' + beta kh e^T (Sd' = Sd for KDA, exp(d) S_prev for EJK) */
                double dbt = 0.0;
                for (int jj = 0; jj < dv; ++jj) {
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i) acc += kh[i] * dS[(size_t)i * dv + jj];
                    de[jj] = bt * acc;
                    dbt += acc * e[jj];
                }
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0, acc2 = 0.0;
                    for (int jj = 0; jj < dv; ++jj) {
                        acc += dS[(size_t)i * dv + jj] * e[jj];
                        acc2 += Sd[(size_t)i * dv + jj] * de[jj];
                    }
                    dkh[i] = bt * acc - acc2;   /* e = v - Sd^T kh */
                }
                double* dvt = dvq + th * dv;
                for (int jj = 0; jj < dv; ++jj) dvt[jj] = de[jj];
                if (!ejk) {
                    /* dSd = dS - kh de^T; dgamma_i = a_i sum_j S_prev_ij dSd_ij; dS <- Diag(a) dSd */
                    for (int i = 0; i < dk; ++i) {
                        const double a = exp(gam[i]);
                        double acc = 0.0;
                        for (int jj = 0; jj < dv; ++jj) {
                            const double x = dS[(size_t)i * dv + jj] - kh[i] * de[jj];
                            acc += Sp[(size_t)i * dv + jj] * x;
                            dS[(size_t)i * dv + jj] = a * x;
                        }
                        dgam[i] = a * acc;
                    }
                } else {
                    /* S = exp(d) S_prev + beta kh (v - S_prev^T kh)^T */
                    const double a = exp(dd);
                    double acc = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int jj = 0; jj < dv; ++jj) {
                            acc += Sp[(size_t)i * dv + jj] * dS[(size_t)i * dv + jj];
                            dS[(size_t)i * dv + jj] = a * dS[(size_t)i * dv + jj] - kh[i] * de[jj];
                        }
                    if (dg) dg[th] = a * acc;
                }
                /* prologue */
                {
                    const double* qr = q + th * dk;
                    const double* kr = k + tkv * dk;
                    double* dqr = dq + th * dk;
                    double* dkr = dkq + th * dk;
                    if (use_l2norm) {
                        double ssq = 0.0, ssk = 0.0, pq = 0.0, pk = 0.0;
                        for (int i = 0; i < dk; ++i) {
                            ssq += qr[i] * qr[i]; ssk += kr[i] * kr[i];
                            pq += qr[i] * dqh[i]; pk += kr[i] * dkh[i];
                        }
                        const double nq = sqrt(ssq + eps), nk = sqrt(ssk + eps);
                        for (int i = 0; i < dk; ++i) {
                            dqr[i] = scale * (dqh[i] / nq - qr[i] * pq / (nq * nq * nq));
                            dkr[i] = dkh[i] / nk - kr[i] * pk / (nk * nk * nk);
                        }
                    } else {
                        for (int i = 0; i < dk; ++i) { dqr[i] = scale * dqh[i]; dkr[i] = dkh[i]; }
                    }
                    if (!ejk) {
                        const double ea = exp(a_log[h]);
                        const double* gr = g + th * dk;
                        for (int i = 0; i < dk; ++i) {
                            const double x = ea * (gr[i] + (dt_bias ? dt_bias[(size_t)i * H + h] : 0.0));
                            const double sg = oracle_sigmoid(x);
                            const double dx = dgam[i] * lower_bound * sg * (1.0 - sg);
                            dg[th * dk + i] = dx * ea;
                            ddt[i] += dx * ea;
                            da += dx * x;
                        }
                        dbeta[th] = dbt * bt * (1.0 - bt);
                    } else {
                        dbeta[th] = dbt;
                    }
                }
            }
        }
        if (dS0) memcpy(dS0 + soff, dS, sizeof(double) * sz);
        da_part[w] = da;
#undef PROLOGUE
        free(ck); free(Sb); free(dS); free(dSd); free(qh); free(kh); free(gam); free(u); free(e);
        free(de); free(otmp); free(dqh); free(dkh); free(dgam);
    }
    /* group sums for k and v; parameter sums over sequences (fixed order) */
    for (int64_t t = 0; t < ntok; ++t)
        for (int hv = 0; hv < Hkv; ++hv) {
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int r = 0; r < G; ++r) acc += dkq[((size_t)t * H + hv * G + r) * dk + i];
                dk_out[((size_t)t * Hkv + hv) * dk + i] = acc;
            }
            for (int jj = 0; jj < dv; ++jj) {
                double acc = 0.0;
                for (int r = 0; r < G; ++r) acc += dvq[((size_t)t * H + hv * G + r) * dv + jj];
                dv_out[((size_t)t * Hkv + hv) * dv + jj] = acc;
            }
        }
    if (!ejk) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int n = 0; n < n_seqs; ++n) acc += da_part[(size_t)n * H + h];
            if (da_log) da_log[h] = acc;
            for (int i = 0; i < dk; ++i) {
                double a2 = 0.0;
                for (int n = 0; n < n_seqs; ++n) a2 += ddt_part[((size_t)n * H + h) * dk + i];
                if (ddt_bias) ddt_bias[(size_t)i * H + h] = a2;
            }
        }
    }
    free(dkq); free(dvq); free(da_part); free(ddt_part);
    return 0;
}

/*
 * Gated recurrent attention (ejkernel "recurrent" page, recurrent_attention():
 * query, key, value, the gates g, g_gamma, gk, gv, softmax_scale,
 * initial_state, reverse, cu_seqlens), token by token in float64.  The page
 * gives no formula; the reading taken (every gate a log-space factor, used
 * as given):
 *     S <- exp(g_gamma[b, h]) * Diag(exp(gk_t)) S Diag(exp(gv_t))   (layer, key and value gates)
 *     S <- S + k_t v_t^T
 *     o_t = S^T (scale * exp(g_t) * q_t)                              (query gate)
 * with tokens taken in order, or from the last to the first with reverse.
 * Absent gates are 0 (no decay).  Layouts: q, g, gk [Ntok, H, dk]; k
 * [Ntok, Hkv, dk]; v [Ntok, Hkv, dv]; gv [Ntok, H, dv]; g_gamma [Bg, H] with
 * row min(n, Bg - 1) for sequence n (Bg = B for a dense batch, 1 packed);
 * states [N, H, dk, dv]; o [Ntok, H, dv].
 */
int kda_oracle_gated_recurrent(const double* q, const double* k, const double* v, const double* g,
                               const double* g_gamma, int g_gamma_rows, const double* gk,
                               const double* gv, const double* initial_state,
                               const int64_t* cu_seqlens, int n_seqs, int H, int Hkv, int dk, int dv,
                               double scale, int reverse, double* o, double* final_state, int n_threads)
{
    if (n_seqs < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    scale = oracle_resolve_scale(scale, dk);
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int w = 0; w < n_seqs * H; ++w) {
        const int n = w / H, h = w % H;
        const int hk = h / (H / Hkv);
        const size_t sz = (size_t)dk * dv;
        const size_t soff = ((size_t)n * H + h) * sz;
        double* S = (double*)malloc(sizeof(double) * sz);
        double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
        if (initial_state) memcpy(S, initial_state + soff, sizeof(double) * sz);
        else memset(S, 0, sizeof(double) * sz);
        const double lg = g_gamma ? g_gamma[(size_t)(n < g_gamma_rows ? n : g_gamma_rows - 1) * H + h] : 0.0;
        const int64_t t0 = cu_seqlens[n], t1 = cu_seqlens[n + 1];
        for (int64_t m = 0; m < t1 - t0; ++m) {
            const int64_t t = reverse ? t1 - 1 - m : t0 + m;
            const size_t th = (size_t)t * H + h, tkv = (size_t)t * Hkv + hk;
            for (int i = 0; i < dk; ++i) {
                const double ri = lg + (gk ? gk[th * dk + i] : 0.0);
                for (int j = 0; j < dv; ++j) {
                    const double f = exp(ri + (gv ? gv[th * dv + j] : 0.0));
                    S[(size_t)i * dv + j] = f * S[(size_t)i * dv + j] + k[tkv * dk + i] * v[tkv * dv + j];
                }
            }
            for (int i = 0; i < dk; ++i) qt[i] = scale * exp(g ? g[th * dk + i] : 0.0) * q[th * dk + i];
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * qt[i];
                o[th * dv + j] = acc;
            }
        }
        if (final_state) memcpy(final_state + soff, S, sizeof(double) * sz);
        free(S); free(qt);
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

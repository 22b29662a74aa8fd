/*
 * gdn_oracle.c - CPU oracle for the Gated DeltaNet speculative-verify path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only the tests, the smoke check and the benchmark's cpu_baseline leg use it.  It shares no
 * code, header, table or helper with the HIP library; both sides only consume the same seeded
 * inputs.
 *
 * Everything is evaluated token by token in fp64 from the (already rounded) fp32 inputs,
 * in the order the definitions state, with no blocking or reordering:
 *
 *   conv    Depthwise causal conv1d, kernel 4, over concat(old conv state, new qkv rows)
 *           (lucebox-hub internal.h, struct TargetCache: conv_state and conv_input_cache
 *           comments; struct TargetLayer: ssm_conv1d, a depthwise causal conv weight).
 *           xhat[t][c] = sum_j w[c][j] * xext[t+j][c], tap 3 multiplies the current token.
 *   gate    g = -exp(A_log) * softplus(alpha + dt_bias), rho = exp(g)  (gated delta rule of
 *           Yang, Kautz & Hatamizadeh, "Gated Delta Networks", 2024; per-head A and dt_bias
 *           parameters in lucebox-hub internal.h, struct TargetLayer).
 *   update  S_t = rho_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, written out as
 *           S_t[i][j] = rho * (S[i][j] - beta * p_i * k_j) + beta * v_i * k_j with p = S k,
 *           which is the product with (I - beta k k^T) expanded by distributivity.
 *   readout o_t = S_t q_t.
 *   norm    y = o / sqrt(mean(o^2) + eps) * norm_w * z * sigmoid(z)  (ssm_norm [head_v_dim],
 *           rms_eps and the z projection in lucebox-hub internal.h, TargetLayer/TargetWeights).
 *   capture cap[t] = S_t for every verify position t (lucebox-hub internal.h, TargetCache:
 *           ssm_intermediate, whose element t is the state after verify token t).
 *   tree    the state of node i is the chain evaluated along the root path of i, starting
 *           from the committed state; the conv window is taken along the same path
 *           (lucebox-hub internal.h, QwenGraphInputs::parent_ids, which switches the forward to
 *           tree verification).
 *
 * Layouts (row-major, last index fastest):
 *   qkv [B][T][C] with C = 2*H_k*d_k + H_v*d_v, channel blocks q | k | v, head-major;
 *   z [B][T][H_v][d_v]; alpha, beta [B][T][H_v]; state [P][H_v][d_v][d_k];
 *   conv_state [P][3][C] oldest row first; conv_w [C][4]; norm_w [d_v]; A_log, dt_bias [H_v].
 *   Value head h reads key head h / (H_v / H_k).
 *
 * Parity pins: every function here is checked in tests/ against closed forms, invariants,
 * exact rational brute force and library routines; see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int32_t n_kh, n_vh, d_k, d_v, d_conv;
    int32_t flags; /* bit 0: SiLU after the conv, q and k scaled to unit length, q * d_k^-1/2 */
    double eps;    /* RMS-norm epsilon */
} ora_dims;

#define ORA_F_QK_NORM_SILU 1
#define ORA_L2_EPS 1e-6

static int channels(const ora_dims *d) { return 2 * d->n_kh * d->d_k + d->n_vh * d->d_v; }

double ora_softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

double ora_gate(double A_log, double dt_bias, double alpha)
{
    return -exp(A_log) * ora_softplus(alpha + dt_bias);
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* y[i] = o[i] / sqrt(mean(o^2) + eps) * w[i] * silu(z[i]) over n values. */
void ora_norm_gate(int n, const double *o, const float *z, const float *w, double eps, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += o[i] * o[i];
    double inv = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) {
        double zi = z[i];
        y[i] = o[i] * inv * (double)w[i] * (zi * sigmoid(zi));
    }
}

/* Row r of the extended conv input of a token path: rows 0..2 are the slot's conv state,
 * row 3+m is the qkv row of the m-th token on the path. */
static const float *ext_row(const ora_dims *d, const float *qkv_b, const float *cs_s,
                            const int32_t *path, int r)
{
    int C = channels(d);
    if (r < d->d_conv - 1) return cs_s + (size_t)r * C;
    return qkv_b + (size_t)path[r - (d->d_conv - 1)] * C;
}

/* Post-conv value of channel c at path position m. */
static double conv_at(const ora_dims *d, const float *qkv_b, const float *cs_s, const float *conv_w,
                      const int32_t *path, int m, int c)
{
    double acc = 0.0;
    for (int j = 0; j < d->d_conv; ++j)
        acc += (double)conv_w[(size_t)c * d->d_conv + j] *
               (double)ext_row(d, qkv_b, cs_s, path, m + j)[c];
    return acc;
}

/* xhat for every channel of one batch entry along the chain 0..T-1: out [T][C] fp64. */
void ora_conv(const ora_dims *d, int T, const float *qkv_b, const float *cs_s,
              const float *conv_w, double *out)
{
    int C = channels(d);
    int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
    for (int t = 0; t < T; ++t) path[t] = t;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < C; ++c) out[(size_t)t * C + c] = conv_at(d, qkv_b, cs_s, conv_w, path, t, c);
    free(path);
}

/*
 * Run one (batch entry, value head) unit along a token path of length L.
 *   S      [d_v][d_k] fp64: in = start state, out = state after the last path token
 *   cap    [L][d_v][d_k] fp64 or NULL: state after each path token
 *   y      [L][d_v] fp64 or NULL: gated, normalised output of each path token
 *   o_raw  [L][d_v] fp64 or NULL: readout before the norm
 */
static void run_path(const ora_dims *d, int T, int b, int h, const int32_t *path, int L,
                     const float *qkv, const float *z, const float *alpha, const float *beta,
                     const float *A_log, const float *dt_bias, const float *conv_w,
                     const float *norm_w, const float *cs_s, double *S, double *cap, double *y,
                     double *o_raw)
{
    const int C = channels(d);
    const int dk = d->d_k, dv = d->d_v, Hv = d->n_vh;
    const int hk = h / (d->n_vh / d->n_kh);
    const int q0 = hk * dk, k0 = d->n_kh * dk + hk * dk, v0 = 2 * d->n_kh * dk + h * dv;
    const float *qkv_b = qkv + (size_t)b * T * C;
    double *q = (double *)malloc(sizeof(double) * dk);
    double *k = (double *)malloc(sizeof(double) * dk);
    double *v = (double *)malloc(sizeof(double) * dv);
    double *p = (double *)malloc(sizeof(double) * dv);
    double *o = (double *)malloc(sizeof(double) * dv);

    for (int m = 0; m < L; ++m) {
        const int t = path[m];
        for (int i = 0; i < dk; ++i) {
            q[i] = conv_at(d, qkv_b, cs_s, conv_w, path, m, q0 + i);
            k[i] = conv_at(d, qkv_b, cs_s, conv_w, path, m, k0 + i);
        }
        for (int i = 0; i < dv; ++i) v[i] = conv_at(d, qkv_b, cs_s, conv_w, path, m, v0 + i);
        if (d->flags & ORA_F_QK_NORM_SILU) {
            double nq = 0.0, nk = 0.0;
            for (int i = 0; i < dk; ++i) {
                q[i] = q[i] * sigmoid(q[i]);
                k[i] = k[i] * sigmoid(k[i]);
                nq += q[i] * q[i];
                nk += k[i] * k[i];
            }
            for (int i = 0; i < dv; ++i) v[i] = v[i] * sigmoid(v[i]);
            double sq = 1.0 / sqrt(nq + ORA_L2_EPS) / sqrt((double)dk);
            double sk = 1.0 / sqrt(nk + ORA_L2_EPS);
            for (int i = 0; i < dk; ++i) {
                q[i] *= sq;
                k[i] *= sk;
            }
        }
        const size_t tok = ((size_t)b * T + t) * Hv + h;
        const double bt = beta[tok];
        const double rho = exp(ora_gate(A_log[h], dt_bias[h], alpha[tok]));

        /* p = S k, then S <- rho (S - beta p k^T) + beta v k^T */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * k[j];
            p[i] = acc;
        }
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j) {
                double *sij = &S[(size_t)i * dk + j];
                *sij = rho * (*sij - bt * p[i] * k[j]) + bt * v[i] * k[j];
            }
        /* o = S_t q */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * q[j];
            o[i] = acc;
        }
        if (cap) memcpy(cap + (size_t)m * dv * dk, S, sizeof(double) * dv * dk);
        if (o_raw) memcpy(o_raw + (size_t)m * dv, o, sizeof(double) * dv);
        if (y) ora_norm_gate(dv, o, z + tok * dv, norm_w, d->eps, y + (size_t)m * dv);
    }
    free(q);
    free(k);
    free(v);
    free(p);
    free(o);
}

static void load_state(const ora_dims *d, const float *state, int s, int h, double *S)
{
    const size_t n = (size_t)d->d_v * d->d_k;
    const float *src = state + ((size_t)s * d->n_vh + h) * n;
    for (size_t i = 0; i < n; ++i) S[i] = src[i];
}

/*
 * Chain verify for a list of (batch entry, value head) units.  Unit u covers batch entry
 * unit_b[u] (slot slot_ids[unit_b[u]]) and value head unit_h[u]:
 *   st_out [n_units][d_v][d_k]      state after the last token
 *   cap_out [n_units][T][d_v][d_k]  state after every token, or NULL
 *   y_out  [n_units][T][d_v]        gated output, or NULL
 *   o_out  [n_units][T][d_v]        raw readout, or NULL
 * Returns 0, or -1 on an out-of-range index.
 */
int ora_verify(const ora_dims *d, int T, int B, int P, const float *qkv, const float *z,
               const float *alpha, const float *beta, const float *A_log, const float *dt_bias,
               const float *conv_w, const float *norm_w, const float *state,
               const float *conv_state, const int32_t *slot_ids, int n_units,
               const int32_t *unit_b, const int32_t *unit_h, double *st_out, double *cap_out,
               double *y_out, double *o_out, int n_threads)
{
    const int C = channels(d);
    const size_t nS = (size_t)d->d_v * d->d_k;
    for (int u = 0; u < n_units; ++u) {
        if (unit_b[u] < 0 || unit_b[u] >= B || unit_h[u] < 0 || unit_h[u] >= d->n_vh) return -1;
        int s = slot_ids[unit_b[u]];
        if (s < 0 || s >= P) return -1;
    }
    int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
    for (int t = 0; t < T; ++t) path[t] = t;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (int u = 0; u < n_units; ++u) {
        const int b = unit_b[u], h = unit_h[u], s = slot_ids[b];
        double *S = st_out + (size_t)u * nS;
        load_state(d, state, s, h, S);
        run_path(d, T, b, h, path, T, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                 conv_state + (size_t)s * (d->d_conv - 1) * C, S,
                 cap_out ? cap_out + (size_t)u * T * nS : NULL,
                 y_out ? y_out + (size_t)u * T * d->d_v : NULL,
                 o_out ? o_out + (size_t)u * T * d->d_v : NULL);
    }
    free(path);
    return 0;
}

/*
 * Tree verify for a list of (batch entry, value head) units.  parent [B][T]: parent[0] = -1 is
 * the root; a node with parent -1 starts from the committed state, any other node from its
 * parent.  For every node the chain is re-run along the node's root path.
 *   cap_out [n_units][T][d_v][d_k] state after each node (required)
 *   y_out   [n_units][T][d_v]      gated output of each node, or NULL
 * Returns 0, or -1 on a malformed parent array or index.
 */
int ora_tree(const ora_dims *d, int T, int B, int P, const float *qkv, const float *z,
             const float *alpha, const float *beta, const float *A_log, const float *dt_bias,
             const float *conv_w, const float *norm_w, const float *state,
             const float *conv_state, const int32_t *slot_ids, const int32_t *parent,
             int n_units, const int32_t *unit_b, const int32_t *unit_h, double *cap_out,
             double *y_out, int n_threads)
{
    const int C = channels(d);
    const size_t nS = (size_t)d->d_v * d->d_k;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < T; ++i) {
            int p = parent[(size_t)b * T + i];
            if (p < -1 || p >= i) return -1;
        }
    for (int u = 0; u < n_units; ++u) {
        if (unit_b[u] < 0 || unit_b[u] >= B || unit_h[u] < 0 || unit_h[u] >= d->n_vh) return -1;
        int s = slot_ids[unit_b[u]];
        if (s < 0 || s >= P) return -1;
    }
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
#endif
    for (int u = 0; u < n_units; ++u) {
        const int b = unit_b[u], h = unit_h[u], s = slot_ids[b];
        const int32_t *par = parent + (size_t)b * T;
        int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
        double *S = (double *)malloc(sizeof(double) * nS);
        double *ys = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * d->d_v);
        for (int i = 0; i < T; ++i) {
            int L = 0;
            for (int n = i; n >= 0; n = par[n]) ++L;
            int m = L;
            for (int n = i; n >= 0; n = par[n]) path[--m] = n;
            load_state(d, state, s, h, S);
            run_path(d, T, b, h, path, L, qkv, z, alpha, beta, A_log, dt_bias, conv_w, norm_w,
                     conv_state + (size_t)s * (d->d_conv - 1) * C, S, NULL,
                     y_out ? ys : NULL, NULL);
            memcpy(cap_out + ((size_t)u * T + i) * nS, S, sizeof(double) * nS);
            if (y_out)
                memcpy(y_out + ((size_t)u * T + i) * d->d_v, ys + (size_t)(L - 1) * d->d_v,
                       sizeof(double) * d->d_v);
        }
        free(path);
        free(S);
        free(ys);
    }
    return 0;
}

/* The tree's per-node conv state: cap [B][T][3][C] holds the last three rows of the conv
 * window that ends at each node (a pure copy of inputs along the node's root path). */
int ora_tree_conv(const ora_dims *d, int T, int B, int P, const float *qkv,
                  const float *conv_state, const int32_t *slot_ids, const int32_t *parent,
                  float *cap)
{
    const int C = channels(d), K1 = d->d_conv - 1;
    int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
    for (int b = 0; b < B; ++b) {
        int s = slot_ids[b];
        if (s < 0 || s >= P) {
            free(path);
            return -1;
        }
        const int32_t *par = parent + (size_t)b * T;
        for (int i = 0; i < T; ++i) {
            int L = 0;
            for (int n = i; n >= 0; n = par[n]) ++L;
            int m = L;
            for (int n = i; n >= 0; n = par[n]) path[--m] = n;
            for (int r = 0; r < K1; ++r)
                memcpy(cap + (((size_t)b * T + i) * K1 + r) * C,
                       ext_row(d, qkv + (size_t)b * T * C, conv_state + (size_t)s * K1 * C, path,
                               L + r),
                       sizeof(float) * C);
        }
    }
    free(path);
    return 0;
}

int ora_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

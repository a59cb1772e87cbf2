/*
 * oal_oracle.c -- CPU reference for OAL causal attention. TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may call this
 * library. The product path (the HIP library) shares no code, header, table or constant
 * with it.
 *
 * Everything is fp64, in plain loops, with no blocking, feature maps or reordering beyond
 * what the definitions state. Sources (daiwk.github.io reproduction notes of arXiv
 * 2610.13674, "OAL: 按 QK 离群贡献分组的正二次注意力核", section "核心公式"):
 *
 *  - group partial scores: s_g = sum_{r in group g} q_r k_r / sqrt(d_h), s-bar = [1, s_1..s_G]
 *    (second display of the section);
 *  - kernel: kappa(q,k) = eps + s-bar^T L L^T s-bar > 0 (third display);
 *  - prefix states H0, H1, H2 over j <= i of [v_j;1], k_{j,r}[v_j;1], k_{j,r}k_{j,t}[v_j;1]
 *    (fourth display);
 *  - readout u~_i = a H0 + (1/sqrt d_h) sum_r b_r q_r H1_r + (1/d_h) sum_{r,t} C_rt q_r q_t H2_rt,
 *    y^_i = u~_{i,1:dv} / u~_{i,dv+1} (fifth display).
 *
 * The dense routine is the definition itself: for every causal pair (j <= i) it evaluates
 * kappa and forms the kappa-weighted average of v. The recurrence routine follows the
 * H-state equations of the pages with a full d x d H2 and (a, b, C) obtained from (eps, L)
 * by expanding s-bar^T M s-bar with M = L L^T:
 *     a = eps + M_00,  b_r = 2 M_{0, g(r)},  C_rt = M_{g(r), g(t)}
 * where g(r) is the s-bar index of dim r's group. The pages do not print this map; it is
 * the reading the two displays force, and the tests pin it by requiring the two routines
 * to agree.
 *
 * Group ids in group_of_dim are config ids 0..G-1; config group g is s-bar entry g+1, and
 * row/column 0 of L belong to the constant entry. L is given per head as a
 * (g_max+1) x (g_max+1) row-major array whose lower triangle is read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oal_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* kappa for one (query, key) pair of one head: eps + || L^T s-bar ||^2. */
double oal_oracle_kappa(int d, int G, int g_max, const uint8_t *group_of_dim,
                        const double *L, double eps, const double *q, const double *k) {
    double sbar[65 + 1];   /* G <= d <= 64 */
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    sbar[0] = 1.0;
    for (int g = 1; g <= G; ++g) sbar[g] = 0.0;
    for (int r = 0; r < d; ++r) sbar[1 + group_of_dim[r]] += q[r] * k[r];
    for (int g = 1; g <= G; ++g) sbar[g] *= inv_sqrt_d;
    double kap = eps;
    for (int m = 0; m <= G; ++m) {
        double z = 0.0;                          /* (L^T s-bar)_m = sum_g L[g][m] s-bar_g */
        for (int g = m; g <= G; ++g) z += L[g * (g_max + 1) + m] * sbar[g];
        kap += z * z;
    }
    return kap;
}

static int check_args(int B, int Hq, int Hkv, int T, int d, int dv, const int *n_groups,
                      const uint8_t *group_of_dim, int g_max) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || T < 0 || d <= 0 || d > 64 || dv <= 0) return 1;
    if (Hq % Hkv) return 2;
    for (int h = 0; h < Hq; ++h) {
        if (n_groups[h] < 1 || n_groups[h] > d || n_groups[h] > g_max) return 3;
        for (int r = 0; r < d; ++r)
            if (group_of_dim[h * d + r] >= n_groups[h]) return 4;
    }
    return 0;
}

/* One output row (b, h, i) of the dense definition: y[dv] and the denominator. */
static void dense_row(int Hq, int Hkv, int T, int d, int dv, int b, int h, int i,
                      const double *q, const double *k, const double *v, const int *n_groups,
                      const uint8_t *group_of_dim, int g_max, const double *L, const double *eps,
                      double *y_row, double *den_out) {
    int kv = h / (Hq / Hkv);                     /* query head h reads KV head h / n_rep */
    const double *qi = q + (((size_t)b * Hq + h) * T + i) * d;
    const double *kb = k + ((size_t)b * Hkv + kv) * T * d;
    const double *vb = v + ((size_t)b * Hkv + kv) * T * dv;
    const double *Lh = L + (size_t)h * (g_max + 1) * (g_max + 1);
    const uint8_t *gam = group_of_dim + (size_t)h * d;
    double num[1024];
    double den = 0.0;
    for (int c = 0; c < dv; ++c) num[c] = 0.0;
    for (int j = 0; j <= i; ++j) {               /* causal, inclusive: j <= i */
        double kap = oal_oracle_kappa(d, n_groups[h], g_max, gam, Lh, eps[h], qi, kb + (size_t)j * d);
        for (int c = 0; c < dv; ++c) num[c] += kap * vb[(size_t)j * dv + c];
        den += kap;
    }
    for (int c = 0; c < dv; ++c) y_row[c] = num[c] / den;
    if (den_out) *den_out = den;
}

/*
 * Dense O(T^2) kernel sum for all rows.
 *   q [B,Hq,T,d], k [B,Hkv,T,d], v [B,Hkv,T,dv]; n_groups [Hq]; group_of_dim [Hq,d];
 *   L [Hq,(g_max+1)^2]; eps [Hq]; y [B,Hq,T,dv] out; den [B,Hq,T] out (may be NULL).
 * Returns 0 on success, a positive code on bad arguments.
 */
int oal_oracle_dense(int B, int Hq, int Hkv, int T, int d, int dv, const double *q,
                     const double *k, const double *v, const int *n_groups,
                     const uint8_t *group_of_dim, int g_max, const double *L, const double *eps,
                     double *y, double *den) {
    int rc = check_args(B, Hq, Hkv, T, d, dv, n_groups, group_of_dim, g_max);
    if (rc || dv > 1024) return rc ? rc : 5;
    long long rows = (long long)B * Hq * T;
#pragma omp parallel for schedule(dynamic, 16)
    for (long long idx = 0; idx < rows; ++idx) {
        int i = (int)(idx % T);
        int h = (int)((idx / T) % Hq);
        int b = (int)(idx / ((long long)T * Hq));
        dense_row(Hq, Hkv, T, d, dv, b, h, i, q, k, v, n_groups, group_of_dim, g_max, L, eps,
                  y + (size_t)idx * dv, den ? den + idx : NULL);
    }
    return 0;
}

/* Dense definition for a list of rows (b, h, i) given as int64 triples. */
int oal_oracle_dense_rows(int B, int Hq, int Hkv, int T, int d, int dv, const double *q,
                          const double *k, const double *v, const int *n_groups,
                          const uint8_t *group_of_dim, int g_max, const double *L,
                          const double *eps, int n_rows, const int64_t *rows, double *y,
                          double *den) {
    int rc = check_args(B, Hq, Hkv, T, d, dv, n_groups, group_of_dim, g_max);
    if (rc || dv > 1024) return rc ? rc : 5;
    for (int n = 0; n < n_rows; ++n) {
        if (rows[3 * n] < 0 || rows[3 * n] >= B || rows[3 * n + 1] < 0 || rows[3 * n + 1] >= Hq ||
            rows[3 * n + 2] < 0 || rows[3 * n + 2] >= T)
            return 6;
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < n_rows; ++n) {
        dense_row(Hq, Hkv, T, d, dv, (int)rows[3 * n], (int)rows[3 * n + 1], (int)rows[3 * n + 2],
                  q, k, v, n_groups, group_of_dim, g_max, L, eps, y + (size_t)n * dv,
                  den ? den + n : NULL);
    }
    return 0;
}

/* The causal kappa matrix of one (b, h): kap[i*T + j] for j <= i, 0 above the diagonal. */
int oal_oracle_kappa_matrix(int B, int Hq, int Hkv, int T, int d, const double *q,
                            const double *k, const int *n_groups, const uint8_t *group_of_dim,
                            int g_max, const double *L, const double *eps, int b, int h,
                            double *kap) {
    int rc = check_args(B, Hq, Hkv, T, d, 1, n_groups, group_of_dim, g_max);
    if (rc) return rc;
    if (b < 0 || b >= B || h < 0 || h >= Hq) return 6;
    int kv = h / (Hq / Hkv);
    for (int i = 0; i < T; ++i)
        for (int j = 0; j < T; ++j)
            kap[(size_t)i * T + j] = (j <= i)
                ? oal_oracle_kappa(d, n_groups[h], g_max, group_of_dim + (size_t)h * d,
                                   L + (size_t)h * (g_max + 1) * (g_max + 1), eps[h],
                                   q + (((size_t)b * Hq + h) * T + i) * d,
                                   k + (((size_t)b * Hkv + kv) * T + j) * d)
                : 0.0;
    return 0;
}

/*
 * Naive H0/H1/H2 recurrence (full d x d H2) with readout, following the pages' equations
 * step by step. Self-test companion of the dense routine; O(T d^2 dv).
 *   H_final (optional) [B, Hkv, 1 + d + d*d, dv+1]: the states after the last token,
 *   ordered H0, then H1_r (r = 0..d-1), then H2_rt (r-major).
 */
int oal_oracle_recurrence(int B, int Hq, int Hkv, int T, int d, int dv, const double *q,
                          const double *k, const double *v, const int *n_groups,
                          const uint8_t *group_of_dim, int g_max, const double *L,
                          const double *eps, double *y, double *H_final) {
    int rc = check_args(B, Hq, Hkv, T, d, dv, n_groups, group_of_dim, g_max);
    if (rc) return rc;
    int n_rep = Hq / Hkv, W = dv + 1, gm1 = g_max + 1;
    size_t nfeat = 1 + (size_t)d + (size_t)d * d;
    double *H = (double *)malloc(nfeat * W * sizeof(double));
    double *a = (double *)malloc(Hq * sizeof(double));
    double *bco = (double *)malloc((size_t)Hq * d * sizeof(double));
    double *C = (double *)malloc((size_t)Hq * d * d * sizeof(double));
    double *M = (double *)malloc((size_t)gm1 * gm1 * sizeof(double));
    double *u = (double *)malloc(W * sizeof(double));
    if (!H || !a || !bco || !C || !M || !u) {
        free(H); free(a); free(bco); free(C); free(M); free(u);
        return 7;
    }
    /* (eps, L) -> (a, b, C): expand s-bar^T (L L^T) s-bar. */
    for (int h = 0; h < Hq; ++h) {
        const double *Lh = L + (size_t)h * gm1 * gm1;
        int G = n_groups[h];
        for (int x = 0; x <= G; ++x)
            for (int y2 = 0; y2 <= G; ++y2) {
                double s = 0.0;
                for (int m = 0; m <= G; ++m)
                    if (m <= x && m <= y2) s += Lh[x * gm1 + m] * Lh[y2 * gm1 + m];
                M[x * gm1 + y2] = s;
            }
        const uint8_t *gam = group_of_dim + (size_t)h * d;
        a[h] = eps[h] + M[0];
        for (int r = 0; r < d; ++r) {
            bco[(size_t)h * d + r] = 2.0 * M[0 * gm1 + 1 + gam[r]];
            for (int t = 0; t < d; ++t)
                C[((size_t)h * d + r) * d + t] = M[(1 + gam[r]) * gm1 + 1 + gam[t]];
        }
    }
    double inv_sqrt_d = 1.0 / sqrt((double)d), inv_d = 1.0 / (double)d;
    for (int b = 0; b < B; ++b)
        for (int kv = 0; kv < Hkv; ++kv) {
            memset(H, 0, nfeat * W * sizeof(double));
            const double *kb = k + ((size_t)b * Hkv + kv) * T * d;
            const double *vb = v + ((size_t)b * Hkv + kv) * T * dv;
            for (int i = 0; i < T; ++i) {
                /* H_i = H_{i-1} + term_i, with term_i built from [v_i; 1] */
                const double *ki = kb + (size_t)i * d;
                for (int c = 0; c < W; ++c) {
                    double vc = (c < dv) ? vb[(size_t)i * dv + c] : 1.0;
                    H[0 * W + c] += vc;
                    for (int r = 0; r < d; ++r) H[(1 + r) * W + c] += ki[r] * vc;
                    for (int r = 0; r < d; ++r)
                        for (int t = 0; t < d; ++t)
                            H[(1 + d + (size_t)r * d + t) * W + c] += ki[r] * ki[t] * vc;
                }
                /* readout for every query head sharing this KV head */
                for (int hh = 0; hh < n_rep; ++hh) {
                    int h = kv * n_rep + hh;
                    const double *qi = q + (((size_t)b * Hq + h) * T + i) * d;
                    for (int c = 0; c < W; ++c) {
                        double acc = a[h] * H[0 * W + c];
                        double lin = 0.0;
                        for (int r = 0; r < d; ++r) lin += bco[(size_t)h * d + r] * qi[r] * H[(1 + r) * W + c];
                        double quad = 0.0;
                        for (int r = 0; r < d; ++r)
                            for (int t = 0; t < d; ++t)
                                quad += C[((size_t)h * d + r) * d + t] * qi[r] * qi[t] *
                                        H[(1 + d + (size_t)r * d + t) * W + c];
                        u[c] = acc + inv_sqrt_d * lin + inv_d * quad;
                    }
                    double *yi = y + (((size_t)b * Hq + h) * T + i) * dv;
                    for (int c = 0; c < dv; ++c) yi[c] = u[c] / u[dv];
                }
            }
            if (H_final)
                memcpy(H_final + ((size_t)b * Hkv + kv) * nfeat * W, H, nfeat * W * sizeof(double));
        }
    free(H); free(a); free(bco); free(C); free(M); free(u);
    return 0;
}

/*
 * Prefix states with H2 kept as its upper triangle (r <= t), the layout of the library's
 * state: row 0 = H0, rows 1..d = H1_r, then H2_rt for r <= t in row-major order of the
 * upper triangle; column c < dv is v's component c, column dv is the "1" of [v;1].
 *   H [B, Hkv, 1 + d + d(d+1)/2, dv+1] out. Sums over tokens j < T (all of them).
 */
int oal_oracle_state(int B, int Hkv, int T, int d, int dv, const double *k, const double *v,
                     double *H) {
    if (B < 0 || Hkv <= 0 || T < 0 || d <= 0 || d > 64 || dv <= 0) return 1;
    int W = dv + 1;
    size_t nfeat = 1 + (size_t)d + (size_t)d * (d + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int bk = 0; bk < B * Hkv; ++bk) {
        double *Hb = H + (size_t)bk * nfeat * W;
        memset(Hb, 0, nfeat * W * sizeof(double));
        const double *kb = k + (size_t)bk * T * d;
        const double *vb = v + (size_t)bk * T * dv;
        for (int j = 0; j < T; ++j) {
            const double *kj = kb + (size_t)j * d;
            for (int c = 0; c < W; ++c) {
                double vc = (c < dv) ? vb[(size_t)j * dv + c] : 1.0;
                size_t f = 0;
                Hb[f++ * W + c] += vc;
                for (int r = 0; r < d; ++r) Hb[f++ * W + c] += kj[r] * vc;
                for (int r = 0; r < d; ++r)
                    for (int t = r; t < d; ++t) Hb[f++ * W + c] += kj[r] * kj[t] * vc;
            }
        }
    }
    return 0;
}

/*
 * Causal contribution score of every q/k dim (section "核心公式", first display; the
 * "逐 prompt 因果贡献统计" node of the flowchart), for each prompt p (a sequence of the
 * batch) and query head h with KV head kv = h / (Hq / Hkv):
 *   chi[p,h,r]   = (1/|Omega_p|) * sum over causal pairs (i, j <= i) of |q[p,h,i,r] k[p,kv,j,r] / sqrt(d)|
 *   chi_mean[h,r] = (1/B) * sum_p chi[p,h,r]
 * |Omega_p| is read as the number of causal pairs of the prompt, T (T+1) / 2. The sum is
 * the plain double loop over pairs, O(T^2 d) per (p, h).
 *   q [B, Hq, T, d], k [B, Hkv, T, d]; chi [B, Hq, d] out; chi_mean [Hq, d] out (may be NULL).
 */
int oal_oracle_contribution(int B, int Hq, int Hkv, int T, int d, const double *q,
                            const double *k, double *chi, double *chi_mean) {
    if (B < 1 || Hq <= 0 || Hkv <= 0 || T < 1 || d <= 0 || d > 64) return 1;
    if (Hq % Hkv) return 2;
    int rep = Hq / Hkv;
    double n_pairs = (double)T * (double)(T + 1) / 2.0;
    double sqrt_d = sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * Hq; ++bh) {
        int b = bh / Hq, h = bh % Hq, kv = h / rep;
        const double *qb = q + (size_t)bh * T * d;
        const double *kb = k + ((size_t)b * Hkv + kv) * T * d;
        double acc[64];
        for (int r = 0; r < d; ++r) acc[r] = 0.0;
        for (int i = 0; i < T; ++i)
            for (int j = 0; j <= i; ++j)
                for (int r = 0; r < d; ++r)
                    acc[r] += fabs(qb[(size_t)i * d + r] * kb[(size_t)j * d + r] / sqrt_d);
        for (int r = 0; r < d; ++r) chi[(size_t)bh * d + r] = acc[r] / n_pairs;
    }
    if (chi_mean) {
        for (int h = 0; h < Hq; ++h)
            for (int r = 0; r < d; ++r) {
                double s = 0.0;
                for (int b = 0; b < B; ++b) s += chi[((size_t)b * Hq + h) * d + r];
                chi_mean[(size_t)h * d + r] = s / B;
            }
    }
    return 0;
}

/*
 * Gradients of the dense definition (section "核心公式": s-bar, kappa and readout displays)
 * for an upstream gradient dy = dLoss/dy, by the chain rule through every causal pair:
 *   y_i = num_i / den_i,  num_i = sum_{j<=i} kappa_ij v_j,  den_i = sum_{j<=i} kappa_ij
 *   dnum_i = dy_i / den_i,  dden_i = -(dy_i . y_i) / den_i
 *   per pair (j <= i):  dkappa = dnum_i . v_j + dden_i;  dv_j += kappa_ij dnum_i;  deps += dkappa
 *   kappa = eps + sum_m z_m^2,  z_m = sum_{g >= m} L[g][m] s-bar_g
 *     dz_m = 2 z_m dkappa;  dL[g][m] += s-bar_g dz_m (g >= m);  ds-bar_g = sum_{m <= g} L[g][m] dz_m
 *   s-bar_{1+gamma(r)} collects q_r k_r / sqrt(d):  dq_ir += ds-bar_{1+gamma(r)} k_jr / sqrt(d),
 *                                                   dk_jr += ds-bar_{1+gamma(r)} q_ir / sqrt(d)
 * Inputs as in oal_oracle_dense plus dy [B,Hq,T,dv]. Outputs: dq [B,Hq,T,d], dk [B,Hkv,T,d],
 * dv_out [B,Hkv,T,dv], dL [Hq,(g_max+1)^2] (lower triangle rows/cols 0..G_h; the rest zero),
 * deps [Hq]. Parallel over (sequence, KV head); per-(sequence, head) partials of dL and deps
 * are summed in sequence order afterwards.
 */
int oal_oracle_backward(int B, int Hq, int Hkv, int T, int d, int dv, const double *q,
                        const double *k, const double *v, const int *n_groups,
                        const uint8_t *group_of_dim, int g_max, const double *L, const double *eps,
                        const double *dy, double *dq, double *dk, double *dv_out, double *dL,
                        double *deps) {
    int rc = check_args(B, Hq, Hkv, T, d, dv, n_groups, group_of_dim, g_max);
    if (rc || dv > 1024) return rc ? rc : 5;
    const int rep = Hq / Hkv, gm1 = g_max + 1;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double *dL_part = (double *)calloc((size_t)B * Hq * gm1 * gm1, sizeof(double));
    double *de_part = (double *)calloc((size_t)B * Hq, sizeof(double));
    if (!dL_part || !de_part) { free(dL_part); free(de_part); return 6; }
    memset(dq, 0, (size_t)B * Hq * T * d * sizeof(double));
    memset(dk, 0, (size_t)B * Hkv * T * d * sizeof(double));
    memset(dv_out, 0, (size_t)B * Hkv * T * dv * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int bk = 0; bk < B * Hkv; ++bk) {
        const int b = bk / Hkv, kv = bk % Hkv;
        const double *kb = k + (size_t)bk * T * d;
        const double *vb = v + (size_t)bk * T * dv;
        double *dkb = dk + (size_t)bk * T * d;
        double *dvb = dv_out + (size_t)bk * T * dv;
        double yrow[1024], dnum[1024];
        for (int h = kv * rep; h < (kv + 1) * rep; ++h) {
            const int G = n_groups[h];
            const double *Lh = L + (size_t)h * gm1 * gm1;
            const uint8_t *gam = group_of_dim + (size_t)h * d;
            double *dLh = dL_part + ((size_t)b * Hq + h) * gm1 * gm1;
            double de = 0.0;
            for (int i = 0; i < T; ++i) {
                const double *qi = q + (((size_t)b * Hq + h) * T + i) * d;
                double *dqi = dq + (((size_t)b * Hq + h) * T + i) * d;
                const double *dyi = dy + (((size_t)b * Hq + h) * T + i) * dv;
                double den;
                dense_row(Hq, Hkv, T, d, dv, b, h, i, q, k, v, n_groups, group_of_dim, g_max, L,
                          eps, yrow, &den);
                double dden = 0.0;
                for (int c = 0; c < dv; ++c) {
                    dnum[c] = dyi[c] / den;
                    dden -= dyi[c] * yrow[c];
                }
                dden /= den;
                for (int j = 0; j <= i; ++j) {
                    const double *kj = kb + (size_t)j * d;
                    double sbar[65 + 1], z[65 + 1], dsbar[65 + 1];
                    sbar[0] = 1.0;
                    for (int g = 1; g <= G; ++g) sbar[g] = 0.0;
                    for (int r = 0; r < d; ++r) sbar[1 + gam[r]] += qi[r] * kj[r] * inv_sqrt_d;
                    double kap = eps[h];
                    for (int m = 0; m <= G; ++m) {
                        z[m] = 0.0;
                        for (int g = m; g <= G; ++g) z[m] += Lh[g * gm1 + m] * sbar[g];
                        kap += z[m] * z[m];
                    }
                    double dkap = dden;
                    for (int c = 0; c < dv; ++c) {
                        dkap += dnum[c] * vb[(size_t)j * dv + c];
                        dvb[(size_t)j * dv + c] += kap * dnum[c];
                    }
                    de += dkap;
                    for (int g = 0; g <= G; ++g) dsbar[g] = 0.0;
                    for (int m = 0; m <= G; ++m) {
                        const double dz = 2.0 * z[m] * dkap;
                        for (int g = m; g <= G; ++g) {
                            dLh[g * gm1 + m] += sbar[g] * dz;
                            dsbar[g] += Lh[g * gm1 + m] * dz;
                        }
                    }
                    double *dkj = dkb + (size_t)j * d;
                    for (int r = 0; r < d; ++r) {
                        const double ds = dsbar[1 + gam[r]] * inv_sqrt_d;
                        dqi[r] += ds * kj[r];
                        dkj[r] += ds * qi[r];
                    }
                }
            }
            de_part[(size_t)b * Hq + h] = de;
        }
    }
    for (int h = 0; h < Hq; ++h) {
        double de = 0.0;
        for (int e = 0; e < gm1 * gm1; ++e) dL[(size_t)h * gm1 * gm1 + e] = 0.0;
        for (int b = 0; b < B; ++b) {
            de += de_part[(size_t)b * Hq + h];
            for (int e = 0; e < gm1 * gm1; ++e)
                dL[(size_t)h * gm1 * gm1 + e] += dL_part[((size_t)b * Hq + h) * gm1 * gm1 + e];
        }
        deps[h] = de;
    }
    free(dL_part);
    free(de_part);
    return 0;
}

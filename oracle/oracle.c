/*
 * fp64 CPU oracle for fused CSR neighbourhood attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may call,
 * link or load this file; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code, header or table with the
 * HIP library.
 *
 * What it computes follows "On Efficient Scaling of GNNs via IO-Aware Layers
 * Implementations" (technical summary, Methodology: attention-based layers,
 * forward pass and backward pass). The pages name the computation (score,
 * softmax normalisation over the neighbourhood, value aggregation; backward
 * recomputes weights from a per-node log-sum-exp) without writing formulas;
 * the formulas below are the standard definitions of the two layers the pages
 * name: Graph-Transformer scaled dot-product attention and GATv2 scoring.
 *
 * This oracle deliberately does NOT use the fused method: for each destination
 * row it materialises every edge logit in fp64, takes the max in one pass and
 * the normalising sum in a second, then forms the weights explicitly.
 *
 * Graph convention: CSR by destination. Row i lists the sources j of edges
 * j -> i; the softmax runs over those in-neighbours. A row may be empty
 * (output 0, LSE = -inf, zero gradients).
 *
 * All inputs are fp64 arrays [N,H,D] row-major (element (i,h,d) at
 * ((i*H)+h)*D+d). Each function may be restricted to a list of rows
 * (rows == NULL means every row, in order). Rows are processed in parallel
 * with OpenMP; inside a row the order is serial and fixed.
 *
 * Besides each result the oracle returns its summation scale: the sum of the
 * absolute values of the terms reduced into that output element (Higham's
 * condition scale). Tests divide the GPU-vs-oracle difference by it.
 *
 * The last function, the neighbourhood max/min reduction, is exact by nature
 * and decides integers (the winning source), so it works in fp32, the
 * precision its messages are formed in; see its own comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX3(i, h, d, H, D) ((((int64_t)(i) * (H)) + (h)) * (int64_t)(D) + (d))

static int64_t row_of(const int64_t *rows, int64_t r) { return rows ? rows[r] : r; }

/* Per-thread growable scratch for one row's logits. */
typedef struct {
    double *s;
    int64_t cap;
} rowbuf;

static int rowbuf_need(rowbuf *b, int64_t n) {
    if (n <= b->cap) return 0;
    double *p = (double *)realloc(b->s, (size_t)n * sizeof(double));
    if (!p) return -1;
    b->s = p;
    b->cap = n;
    return 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of later oracle calls (n >= 1); only changes how rows are shared out. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Graph-Transformer logit s_ij^h = scale * <q_i^h, k_j^h>. */
static double gt_logit(const double *Q, const double *K, int64_t i, int64_t j, int h, int H, int D,
                       double scale) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += Q[IDX3(i, h, d, H, D)] * K[IDX3(j, h, d, H, D)];
    return scale * acc;
}

/* GATv2 logit s_ij^h = sum_d a[h,d] * LeakyReLU(xs_j + xd_i), LeakyReLU(x) = x (x >= 0), slope*x (x < 0). */
static double gatv2_logit(const double *XD, const double *XS, const double *att, int64_t i, int64_t j,
                          int h, int H, int D, double slope) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) {
        double z = XS[IDX3(j, h, d, H, D)] + XD[IDX3(i, h, d, H, D)];
        double lr = (z >= 0.0) ? z : slope * z;
        acc += att[(int64_t)h * D + d] * lr;
    }
    return acc;
}

/*
 * Shared softmax-aggregate over one row once its logits s[0..deg) are known:
 * two passes (max, then sum of exp), explicit weights, weighted sum of V rows.
 */
static void softmax_aggregate(const double *s, int64_t deg, const int32_t *nbr, const double *V,
                              int h, int H, int D, double *o /*[D]*/, double *lse, double *so /*[D] or NULL*/,
                              double *sl) {
    for (int d = 0; d < D; ++d) {
        o[d] = 0.0;
        if (so) so[d] = 0.0;
    }
    if (deg == 0) {
        *lse = -INFINITY;
        if (sl) *sl = 1.0;
        return;
    }
    double m = -INFINITY, amax = 0.0;
    for (int64_t e = 0; e < deg; ++e) {
        if (s[e] > m) m = s[e];
        if (fabs(s[e]) > amax) amax = fabs(s[e]);
    }
    double z = 0.0;
    for (int64_t e = 0; e < deg; ++e) z += exp(s[e] - m);
    for (int64_t e = 0; e < deg; ++e) {
        double a = exp(s[e] - m) / z;
        int64_t j = nbr[e];
        for (int d = 0; d < D; ++d) {
            double v = V[IDX3(j, h, d, H, D)];
            o[d] += a * v;
            if (so) so[d] += a * fabs(v);
        }
    }
    *lse = m + log(z);
    if (sl) *sl = 1.0 + amax;
}

/*
 * Graph-Transformer forward.
 * Out (per listed row r, head h): O[r,h,:], LSE[r,h]; optional SO[r,h,:]
 * (sum_j alpha_ij |v_jd|) and SL[r,h] (1 + max_j |s_ij|).
 */
int orc_gt_fwd(int64_t N, const int64_t *indptr, const int32_t *indices, int H, int D, const double *Q,
               const double *K, const double *V, double scale, int64_t nr, const int64_t *rows, double *O,
               double *LSE, double *SO, double *SL) {
    if (!rows) nr = N;
    int err = 0;
#pragma omp parallel
    {
        rowbuf b = {0, 0};
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nr; ++r) {
            int64_t i = row_of(rows, r);
            int64_t e0 = indptr[i], deg = indptr[i + 1] - e0;
            if (rowbuf_need(&b, deg)) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                for (int64_t e = 0; e < deg; ++e) b.s[e] = gt_logit(Q, K, i, indices[e0 + e], h, H, D, scale);
                softmax_aggregate(b.s, deg, indices + e0, V, h, H, D, O + IDX3(r, h, 0, H, D),
                                  LSE + r * H + h, SO ? SO + IDX3(r, h, 0, H, D) : NULL,
                                  SL ? SL + r * H + h : NULL);
            }
        }
        free(b.s);
    }
    return err;
}

/* GATv2 forward: the same softmax-aggregate with GATv2 logits; V is usually XS itself. */
int orc_gatv2_fwd(int64_t N, const int64_t *indptr, const int32_t *indices, int H, int D, const double *XD,
                  const double *XS, const double *V, const double *att, double slope, int64_t nr,
                  const int64_t *rows, double *O, double *LSE, double *SO, double *SL) {
    if (!rows) nr = N;
    int err = 0;
#pragma omp parallel
    {
        rowbuf b = {0, 0};
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nr; ++r) {
            int64_t i = row_of(rows, r);
            int64_t e0 = indptr[i], deg = indptr[i + 1] - e0;
            if (rowbuf_need(&b, deg)) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                for (int64_t e = 0; e < deg; ++e)
                    b.s[e] = gatv2_logit(XD, XS, att, i, indices[e0 + e], h, H, D, slope);
                softmax_aggregate(b.s, deg, indices + e0, V, h, H, D, O + IDX3(r, h, 0, H, D),
                                  LSE + r * H + h, SO ? SO + IDX3(r, h, 0, H, D) : NULL,
                                  SL ? SL + r * H + h : NULL);
            }
        }
        free(b.s);
    }
    return err;
}

/*
 * Graph-Transformer backward, per destination row (FlashAttention-2 style
 * gradient of softmax attention, written from its definition):
 *   alpha_ij    = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i)     (two passes)
 *   dalpha_ij   = <dO_i, v_j>
 *   Delta_i     = sum_j alpha_ij dalpha_ij          (from the weights, not <dO_i, O_i>)
 *   ds_ij       = alpha_ij (dalpha_ij - Delta_i)
 *   dQ_i        = scale * sum_j ds_ij k_j
 * Outputs per listed row: dQ [nr,H,D], Delta [nr,H], and the row statistics
 * M [nr,H] (max logit) and Z [nr,H] (sum of exp(s - M)) that the source-side
 * pass reuses. SdQ (optional) = scale * sum_j alpha_ij (|dalpha_ij| + |Delta_i|) |k_jd|.
 */
int orc_gt_bwd_rows(int64_t N, const int64_t *indptr, const int32_t *indices, int H, int D,
                    const double *Q, const double *K, const double *V, const double *dO, double scale,
                    int64_t nr, const int64_t *rows, double *dQ, double *Delta, double *M, double *Z,
                    double *SdQ) {
    if (!rows) nr = N;
    int err = 0;
#pragma omp parallel
    {
        rowbuf b = {0, 0};
        rowbuf da = {0, 0};
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nr; ++r) {
            int64_t i = row_of(rows, r);
            int64_t e0 = indptr[i], deg = indptr[i + 1] - e0;
            if (rowbuf_need(&b, deg) || rowbuf_need(&da, deg)) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                double *dq = dQ + IDX3(r, h, 0, H, D);
                double *sdq = SdQ ? SdQ + IDX3(r, h, 0, H, D) : NULL;
                for (int d = 0; d < D; ++d) {
                    dq[d] = 0.0;
                    if (sdq) sdq[d] = 0.0;
                }
                if (deg == 0) {
                    Delta[r * H + h] = 0.0;
                    M[r * H + h] = -INFINITY;
                    Z[r * H + h] = 0.0;
                    continue;
                }
                double m = -INFINITY;
                for (int64_t e = 0; e < deg; ++e) {
                    b.s[e] = gt_logit(Q, K, i, indices[e0 + e], h, H, D, scale);
                    if (b.s[e] > m) m = b.s[e];
                }
                double z = 0.0;
                for (int64_t e = 0; e < deg; ++e) z += exp(b.s[e] - m);
                /* b.s now becomes alpha; da holds dalpha */
                double delta = 0.0;
                for (int64_t e = 0; e < deg; ++e) {
                    int64_t j = indices[e0 + e];
                    b.s[e] = exp(b.s[e] - m) / z;
                    double t = 0.0;
                    for (int d = 0; d < D; ++d) t += dO[IDX3(i, h, d, H, D)] * V[IDX3(j, h, d, H, D)];
                    da.s[e] = t;
                    delta += b.s[e] * t;
                }
                for (int64_t e = 0; e < deg; ++e) {
                    int64_t j = indices[e0 + e];
                    double ds = b.s[e] * (da.s[e] - delta);
                    double cs = b.s[e] * (fabs(da.s[e]) + fabs(delta));
                    for (int d = 0; d < D; ++d) {
                        double k = K[IDX3(j, h, d, H, D)];
                        dq[d] += ds * k;
                        if (sdq) sdq[d] += cs * fabs(k);
                    }
                }
                for (int d = 0; d < D; ++d) {
                    dq[d] *= scale;
                    if (sdq) sdq[d] *= scale;
                }
                Delta[r * H + h] = delta;
                M[r * H + h] = m;
                Z[r * H + h] = z;
            }
        }
        free(b.s);
        free(da.s);
    }
    return err;
}

/*
 * Graph-Transformer backward, per source node j, over its out-edges j -> i
 * (the transposed adjacency, CSC: cindptr/cindices list the destinations i):
 *   dK_j = scale * sum_i ds_ij q_i,   dV_j = sum_i alpha_ij dO_i
 * with alpha_ij and ds_ij formed from the destination-row statistics M, Z,
 * Delta of orc_gt_bwd_rows. slot[i] gives the position of row i in those
 * arrays (-1: missing, an error). Optional scales:
 *   SdK = scale * sum_i alpha_ij (|dalpha_ij| + |Delta_i|) |q_id|,  SdV = sum_i alpha_ij |dO_id|.
 */
int orc_gt_bwd_srcs(int64_t N, const int64_t *cindptr, const int32_t *cindices, int H, int D,
                    const double *Q, const double *K, const double *V, const double *dO, double scale,
                    const int64_t *slot, const double *M, const double *Z, const double *Delta, int64_t ns,
                    const int64_t *srcs, double *dK, double *dV, double *SdK, double *SdV) {
    if (!srcs) ns = N;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < ns; ++r) {
        int64_t j = row_of(srcs, r);
        int64_t e0 = cindptr[j], e1 = cindptr[j + 1];
        for (int h = 0; h < H; ++h) {
            double *dk = dK + IDX3(r, h, 0, H, D), *dv = dV + IDX3(r, h, 0, H, D);
            double *sdk = SdK ? SdK + IDX3(r, h, 0, H, D) : NULL;
            double *sdv = SdV ? SdV + IDX3(r, h, 0, H, D) : NULL;
            for (int d = 0; d < D; ++d) {
                dk[d] = dv[d] = 0.0;
                if (sdk) sdk[d] = 0.0;
                if (sdv) sdv[d] = 0.0;
            }
            for (int64_t e = e0; e < e1; ++e) {
                int64_t i = cindices[e];
                int64_t si = slot[i];
                if (si < 0) {
#pragma omp atomic write
                    err = -2;
                    continue;
                }
                double s = gt_logit(Q, K, i, j, h, H, D, scale);
                double a = exp(s - M[si * H + h]) / Z[si * H + h];
                double t = 0.0;
                for (int d = 0; d < D; ++d) t += dO[IDX3(i, h, d, H, D)] * V[IDX3(j, h, d, H, D)];
                double dlt = Delta[si * H + h];
                double ds = a * (t - dlt);
                double cs = a * (fabs(t) + fabs(dlt));
                for (int d = 0; d < D; ++d) {
                    double q = Q[IDX3(i, h, d, H, D)], g = dO[IDX3(i, h, d, H, D)];
                    dk[d] += ds * q;
                    dv[d] += a * g;
                    if (sdk) sdk[d] += cs * fabs(q);
                    if (sdv) sdv[d] += a * fabs(g);
                }
            }
            for (int d = 0; d < D; ++d) {
                dk[d] *= scale;
                if (sdk) sdk[d] *= scale;
            }
        }
    }
    return err;
}

/*
 * GATv2 backward, written from the definition. Per head h, with
 * z_ijd = xs_jd + xd_id, phi = LeakyReLU(slope), phi'(z) = 1 (z >= 0) or slope,
 * s_ij = sum_d a_d phi(z_ijd), alpha_ij = softmax_j s_ij, O_i = sum_j alpha_ij v_j:
 *   dalpha_ij = <dO_i, v_j>,  Delta_i = sum_j alpha_ij dalpha_ij,
 *   ds_ij = alpha_ij (dalpha_ij - Delta_i),  dz_ijd = ds_ij a_d phi'(z_ijd)
 *   dXD_i = sum_j dz_ij,   dXS_j = sum_i dz_ij,   dV_j = sum_i alpha_ij dO_i,
 *   da_d  = sum_ij ds_ij phi(z_ijd).
 * Destination side (per listed row): dXD, Delta, the row statistics M, Z, the
 * row's da contribution DA [nr,H,D], and scales SdXD, SDA.
 */
int orc_gatv2_bwd_rows(int64_t N, const int64_t *indptr, const int32_t *indices, int H, int D,
                       const double *XD, const double *XS, const double *V, const double *att, double slope,
                       const double *dO, int64_t nr, const int64_t *rows, double *dXD, double *Delta, double *M,
                       double *Z, double *DA, double *SdXD, double *SDA) {
    if (!rows) nr = N;
    int err = 0;
#pragma omp parallel
    {
        rowbuf b = {0, 0};
        rowbuf da = {0, 0};
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nr; ++r) {
            int64_t i = row_of(rows, r);
            int64_t e0 = indptr[i], deg = indptr[i + 1] - e0;
            if (rowbuf_need(&b, deg) || rowbuf_need(&da, deg)) {
#pragma omp atomic write
                err = -1;
                continue;
            }
            for (int h = 0; h < H; ++h) {
                double *gx = dXD + IDX3(r, h, 0, H, D), *ga = DA + IDX3(r, h, 0, H, D);
                double *sx = SdXD ? SdXD + IDX3(r, h, 0, H, D) : NULL, *sa = SDA ? SDA + IDX3(r, h, 0, H, D) : NULL;
                for (int d = 0; d < D; ++d) {
                    gx[d] = ga[d] = 0.0;
                    if (sx) sx[d] = 0.0;
                    if (sa) sa[d] = 0.0;
                }
                if (deg == 0) {
                    Delta[r * H + h] = 0.0;
                    M[r * H + h] = -INFINITY;
                    Z[r * H + h] = 0.0;
                    continue;
                }
                double m = -INFINITY;
                for (int64_t e = 0; e < deg; ++e) {
                    b.s[e] = gatv2_logit(XD, XS, att, i, indices[e0 + e], h, H, D, slope);
                    if (b.s[e] > m) m = b.s[e];
                }
                double z = 0.0;
                for (int64_t e = 0; e < deg; ++e) z += exp(b.s[e] - m);
                double delta = 0.0;
                for (int64_t e = 0; e < deg; ++e) {
                    int64_t j = indices[e0 + e];
                    b.s[e] = exp(b.s[e] - m) / z;
                    double t = 0.0;
                    for (int d = 0; d < D; ++d) t += dO[IDX3(i, h, d, H, D)] * V[IDX3(j, h, d, H, D)];
                    da.s[e] = t;
                    delta += b.s[e] * t;
                }
                for (int64_t e = 0; e < deg; ++e) {
                    int64_t j = indices[e0 + e];
                    double ds = b.s[e] * (da.s[e] - delta);
                    double cs = b.s[e] * (fabs(da.s[e]) + fabs(delta));
                    for (int d = 0; d < D; ++d) {
                        double zz = XS[IDX3(j, h, d, H, D)] + XD[IDX3(i, h, d, H, D)];
                        double ph = (zz >= 0.0) ? zz : slope * zz;
                        double dph = (zz >= 0.0) ? 1.0 : slope;
                        double ad = att[(int64_t)h * D + d];
                        gx[d] += ds * ad * dph;
                        ga[d] += ds * ph;
                        if (sx) sx[d] += cs * fabs(ad * dph);
                        if (sa) sa[d] += cs * fabs(ph);
                    }
                }
                Delta[r * H + h] = delta;
                M[r * H + h] = m;
                Z[r * H + h] = z;
            }
        }
        free(b.s);
        free(da.s);
    }
    return err;
}

/*
 * GATv2 backward, source side over the transposed adjacency: dXS_j (the
 * score path only) and dV_j, with scales. Row statistics from
 * orc_gatv2_bwd_rows through slot[] as in orc_gt_bwd_srcs.
 */
int orc_gatv2_bwd_srcs(int64_t N, const int64_t *cindptr, const int32_t *cindices, int H, int D,
                       const double *XD, const double *XS, const double *V, const double *att, double slope,
                       const double *dO, const int64_t *slot, const double *M, const double *Z, const double *Delta,
                       int64_t ns, const int64_t *srcs, double *dXS, double *dV, double *SdXS, double *SdV) {
    if (!srcs) ns = N;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < ns; ++r) {
        int64_t j = row_of(srcs, r);
        for (int h = 0; h < H; ++h) {
            double *gs = dXS + IDX3(r, h, 0, H, D), *gv = dV + IDX3(r, h, 0, H, D);
            double *ss = SdXS ? SdXS + IDX3(r, h, 0, H, D) : NULL, *sv = SdV ? SdV + IDX3(r, h, 0, H, D) : NULL;
            for (int d = 0; d < D; ++d) {
                gs[d] = gv[d] = 0.0;
                if (ss) ss[d] = 0.0;
                if (sv) sv[d] = 0.0;
            }
            for (int64_t e = cindptr[j]; e < cindptr[j + 1]; ++e) {
                int64_t i = cindices[e];
                int64_t si = slot[i];
                if (si < 0) {
#pragma omp atomic write
                    err = -2;
                    continue;
                }
                double a = exp(gatv2_logit(XD, XS, att, i, j, h, H, D, slope) - M[si * H + h]) / Z[si * H + h];
                double t = 0.0;
                for (int d = 0; d < D; ++d) t += dO[IDX3(i, h, d, H, D)] * V[IDX3(j, h, d, H, D)];
                double dlt = Delta[si * H + h];
                double ds = a * (t - dlt), cs = a * (fabs(t) + fabs(dlt));
                for (int d = 0; d < D; ++d) {
                    double zz = XS[IDX3(j, h, d, H, D)] + XD[IDX3(i, h, d, H, D)];
                    double dph = (zz >= 0.0) ? 1.0 : slope;
                    double ad = att[(int64_t)h * D + d], g = dO[IDX3(i, h, d, H, D)];
                    gs[d] += ds * ad * dph;
                    gv[d] += a * g;
                    if (ss) ss[d] += cs * fabs(ad * dph);
                    if (sv) sv[d] += a * fabs(g);
                }
            }
        }
    }
    return err;
}

/*
 * Degree-aware reduction layer ("On Efficient Scaling of GNNs via IO-Aware
 * Layers Implementations", technical summary, Methodology: reduction-based
 * aggregations, a per-edge computation followed by a neighbourhood min/max).
 *
 * Message of entry (i, j) of row i: m_ij[f] = X[j][f] (msg 0) or the
 * difference X[j][f] - X[i][f] (msg 1). out[i][f] is the maximum (op 0) or
 * minimum (op 1) of m_ij[f] over the entries of row i, and arg[i][f] the
 * smallest source index j attaining it; values compare as floats, so -0 and
 * +0 are equal. An empty row gives out 0 and arg -1.
 *
 * Unlike the attention functions this one works in fp32: the winner is an
 * integer decided by comparing messages, so it is decided in the precision the
 * messages are formed in. X holds fp32 values (bf16 inputs widened exactly);
 * the difference is one correctly rounded fp32 subtraction. Rows in parallel,
 * entries of a row in CSR order.
 */
int orc_segment_reduce(int64_t N, const int64_t *indptr, const int32_t *indices, int64_t F, const float *X,
                       int op, int msg, int64_t n_rows, const int64_t *rows, float *out, int32_t *arg) {
    (void)N;
    int err = 0;
#pragma omp parallel
    {
        float *best = (float *)malloc((size_t)(F > 0 ? F : 1) * sizeof(float));
        int32_t *bj = (int32_t *)malloc((size_t)(F > 0 ? F : 1) * sizeof(int32_t));
        if (!best || !bj) {
#pragma omp atomic write
            err = -1;
        }
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!best || !bj) continue;
            const int64_t i = row_of(rows, r);
            for (int64_t f = 0; f < F; ++f) {
                best[f] = 0.0f;
                bj[f] = -1;
            }
            for (int64_t e = indptr[i]; e < indptr[i + 1]; ++e) {
                const int32_t j = indices[e];
                for (int64_t f = 0; f < F; ++f) {
                    const float v = msg ? X[(int64_t)j * F + f] - X[i * F + f] : X[(int64_t)j * F + f];
                    int take;
                    if (bj[f] < 0)
                        take = 1;
                    else if (v == best[f])
                        take = j < bj[f];
                    else
                        take = op == 0 ? (v > best[f]) : (v < best[f]);
                    if (take) {
                        best[f] = v;
                        bj[f] = j;
                    }
                }
            }
            for (int64_t f = 0; f < F; ++f) {
                out[r * F + f] = bj[f] < 0 ? 0.0f : best[f];
                arg[r * F + f] = bj[f];
            }
        }
        free(best);
        free(bj);
    }
    return err;
}

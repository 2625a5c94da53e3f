/*
 * Driver for the AddressSanitizer build of the fp64 oracle (oracle/oracle.c):
 * every exported function on a small graph with empty rows, nodes whose
 * only in-edge is their self-loop, a repeated source and a high-degree row,
 * over all rows and over a row subset, plus the source pass's missing-row
 * error. It checks one hand-worked value per function family so that a
 * broken build is not mistaken for a clean run. Exit 0 and "oracle ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_gt_fwd(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *, const double *,
               double, int64_t, const int64_t *, double *, double *, double *, double *);
int orc_gatv2_fwd(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *, const double *,
                  const double *, double, int64_t, const int64_t *, double *, double *, double *, double *);
int orc_gt_bwd_rows(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *,
                    const double *, const double *, double, int64_t, const int64_t *, double *, double *, double *,
                    double *, double *);
int orc_gt_bwd_srcs(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *,
                    const double *, const double *, double, const int64_t *, const double *, const double *,
                    const double *, int64_t, const int64_t *, double *, double *, double *, double *);
int orc_gatv2_bwd_rows(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *,
                       const double *, const double *, double, const double *, int64_t, const int64_t *, double *,
                       double *, double *, double *, double *, double *, double *);
int orc_gatv2_bwd_srcs(int64_t, const int64_t *, const int32_t *, int, int, const double *, const double *,
                       const double *, const double *, double, const double *, const int64_t *, const double *,
                       const double *, const double *, int64_t, const int64_t *, double *, double *, double *,
                       double *);
int orc_segment_reduce(int64_t, const int64_t *, const int32_t *, int64_t, const float *, int, int, int64_t,
                       const int64_t *, float *, int32_t *);
void orc_set_threads(int);

#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
            return 1;                                              \
        }                                                          \
    } while (0)

enum { N = 7, H = 2, D = 3, E = 14 };

int main(void) {
    /* rows: 0 {0,1,2,3,4,5,6}  1 {}  2 {2}  3 {1,1,3}  4 {0,4}  5 {5}  6 {}  (CSR by destination) */
    const int64_t ip[N + 1] = {0, 7, 7, 8, 11, 13, 14, 14};
    const int32_t ix[E] = {0, 1, 2, 3, 4, 5, 6, 2, 1, 1, 3, 0, 4, 5};
    /* transposed adjacency of the same entries */
    int64_t cip[N + 1] = {0};
    int32_t cix[E];
    for (int i = 0; i < N; ++i)
        for (int64_t e = ip[i]; e < ip[i + 1]; ++e) ++cip[ix[e] + 1];
    for (int j = 0; j < N; ++j) cip[j + 1] += cip[j];
    int64_t fill[N];
    for (int j = 0; j < N; ++j) fill[j] = cip[j];
    for (int i = 0; i < N; ++i)
        for (int64_t e = ip[i]; e < ip[i + 1]; ++e) cix[fill[ix[e]]++] = i;
    const int nf = N * H * D;
    double *Q = malloc(sizeof(double) * nf), *K = malloc(sizeof(double) * nf), *V = malloc(sizeof(double) * nf);
    double *dO = malloc(sizeof(double) * nf), *att = malloc(sizeof(double) * H * D);
    for (int k = 0; k < nf; ++k) {
        Q[k] = sin(1.0 + k);
        K[k] = cos(2.0 * k);
        V[k] = 0.5 * k - 3.0;
        dO[k] = sin(0.3 * k);
    }
    for (int k = 0; k < H * D; ++k) att[k] = 0.25 * (k - 2);
    double *O = malloc(sizeof(double) * nf), *SO = malloc(sizeof(double) * nf);
    double LSE[N * H], SL[N * H];
    orc_set_threads(3);
    CHECK(orc_gt_fwd(N, ip, ix, H, D, Q, K, V, 0.5, 0, NULL, O, LSE, SO, SL) == 0);
    CHECK(isinf(LSE[1 * H]) && LSE[1 * H] < 0 && O[1 * H * D] == 0.0);  /* empty row */
    CHECK(O[2 * H * D] == V[2 * H * D]);                                 /* self-loop only: O = v */
    const int64_t rows[3] = {3, 1, 0};
    double Os[3 * H * D], Ls[3 * H], SOs[3 * H * D], SLs[3 * H];
    CHECK(orc_gt_fwd(N, ip, ix, H, D, Q, K, V, 0.5, 3, rows, Os, Ls, SOs, SLs) == 0);
    CHECK(Os[0] == O[3 * H * D] && Ls[2 * H] == LSE[0]);
    CHECK(orc_gatv2_fwd(N, ip, ix, H, D, Q, K, V, att, 0.2, 0, NULL, O, LSE, NULL, NULL) == 0);
    CHECK(O[5 * H * D + 1] == V[5 * H * D + 1]);
    /* backward: destination rows, then sources, then a missing destination row */
    double *dQ = malloc(sizeof(double) * nf), *SdQ = malloc(sizeof(double) * nf);
    double Dl[N * H], M[N * H], Z[N * H];
    CHECK(orc_gt_bwd_rows(N, ip, ix, H, D, Q, K, V, dO, 0.5, 0, NULL, dQ, Dl, M, Z, SdQ) == 0);
    CHECK(dQ[2 * H * D] == 0.0 && Dl[1 * H] == 0.0);                    /* single neighbour; empty row */
    int64_t slot[N];
    for (int i = 0; i < N; ++i) slot[i] = i;
    double *dK = malloc(sizeof(double) * nf), *dV = malloc(sizeof(double) * nf);
    double *SdK = malloc(sizeof(double) * nf), *SdV = malloc(sizeof(double) * nf);
    CHECK(orc_gt_bwd_srcs(N, cip, cix, H, D, Q, K, V, dO, 0.5, slot, M, Z, Dl, 0, NULL, dK, dV, SdK, SdV) == 0);
    double s = 0.0;                                                      /* sum_j dK_j = 0 per (h, d) */
    for (int j = 0; j < N; ++j) s += dK[j * H * D];
    CHECK(fabs(s) < 1e-12);
    slot[0] = -1;
    CHECK(orc_gt_bwd_srcs(N, cip, cix, H, D, Q, K, V, dO, 0.5, slot, M, Z, Dl, 0, NULL, dK, dV, NULL, NULL) == -2);
    slot[0] = 0;
    double *DA = malloc(sizeof(double) * nf), *SDA = malloc(sizeof(double) * nf);
    CHECK(orc_gatv2_bwd_rows(N, ip, ix, H, D, Q, K, V, att, 0.2, dO, 3, rows, dQ, Dl, M, Z, DA, SdQ, SDA) == 0);
    CHECK(orc_gatv2_bwd_rows(N, ip, ix, H, D, Q, K, V, att, 0.2, dO, 0, NULL, dQ, Dl, M, Z, DA, SdQ, SDA) == 0);
    const int64_t srcs[2] = {6, 1};
    CHECK(orc_gatv2_bwd_srcs(N, cip, cix, H, D, Q, K, V, att, 0.2, dO, slot, M, Z, Dl, 2, srcs, dK, dV, SdK, SdV) ==
          0);
    /* source 6 feeds only row 0, whose dO[0][0] is sin 0 = 0; source 1 feeds rows 0 and 3 */
    CHECK(dV[0] == 0.0 && dV[H * D] != 0.0);
    /* reduction: max of x_j, smallest winning source */
    float X[N * 4], out[N * 4];
    int32_t arg[N * 4];
    for (int k = 0; k < N * 4; ++k) X[k] = (float)((k * 7) % 5);
    CHECK(orc_segment_reduce(N, ip, ix, 4, X, 0, 0, N, NULL, out, arg) == 0);
    CHECK(arg[1 * 4] == -1 && out[1 * 4] == 0.0f);                       /* empty row */
    CHECK(orc_segment_reduce(N, ip, ix, 4, X, 1, 1, 3, rows, out, arg) == 0);
    free(Q); free(K); free(V); free(dO); free(att); free(O); free(SO); free(dQ); free(SdQ);
    free(dK); free(dV); free(SdK); free(SdV); free(DA); free(SDA);
    printf("oracle ok\n");
    return 0;
}

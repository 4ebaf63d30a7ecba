/*
 * cgtp_oracle.c -- plain FP64 CPU oracle for the Clebsch-Gordan tensor
 * product (CG TP) and the graph convolution built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no
 * code, header, table or helper with it.
 *
 * What it computes, and where that is defined:
 *  - "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep
 *    Networks" (abstract): the CG tensor product contracts two dense
 *    feature vectors with a structured sparse tensor; the fused kernel
 *    combines it with a graph convolution; the gradient and the higher
 *    derivatives needed for forces are provided.  The pages give no
 *    formula, so every routine below is the plain textbook definition:
 *      * complex CG coefficients from the Racah formula;
 *      * real coupling tensors obtained by changing each index to the real
 *        spherical-harmonic basis;
 *      * real spherical harmonics in component normalisation and their
 *        Jacobian with respect to the (unnormalised) edge vector;
 *      * the tensor product, convolution, its adjoints (backward) and
 *        forces written as explicit nested loops.
 *  - "Faster training and inference with NVIDIA's open-source
 *    SE(3)-Transformer" (TFN section): a degree-d feature has 2d+1
 *    components; contributions to one output degree are summed.
 *
 * Nothing here is blocked, fused or reordered beyond the definitions.
 * Parallelism: OpenMP over independent output rows only; every output
 * element is summed by one thread in a fixed order.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Thread count of the loops below (timing only; results do not depend on
 * it: every output element is summed by one thread in a fixed order).
 * Returns the count in effect. */
int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

#define ORC_LMAX 12

/* ------------------------------------------------------------------ */
/* Complex-basis Clebsch-Gordan coefficients (Racah formula).          */
/* ------------------------------------------------------------------ */

static double fact(int n) {
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= (double)i;
    return f;
}

/* <j1 m1 j2 m2 | J M> with the Condon-Shortley phase convention
 * (integer angular momenta only). */
double orc_cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
    if (M != m1 + m2) return 0.0;
    if (J < abs(j1 - j2) || J > j1 + j2) return 0.0;
    if (abs(m1) > j1 || abs(m2) > j2 || abs(M) > J) return 0.0;
    double pre = (2.0 * J + 1.0) * fact(J + j1 - j2) * fact(J - j1 + j2) *
                 fact(j1 + j2 - J) / fact(j1 + j2 + J + 1);
    pre = sqrt(pre);
    double pre2 = sqrt(fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) *
                       fact(j2 - m2) * fact(j2 + m2));
    double s = 0.0;
    for (int k = 0; k <= j1 + j2 + J; ++k) {
        int a = j1 + j2 - J - k;
        int b = j1 - m1 - k;
        int c = j2 + m2 - k;
        int d = J - j2 + m1 + k;
        int e = J - j1 - m2 + k;
        if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
        double term = 1.0 / (fact(k) * fact(a) * fact(b) * fact(c) * fact(d) * fact(e));
        s += (k % 2 == 0) ? term : -term;
    }
    return pre * pre2 * s;
}

/* ------------------------------------------------------------------ */
/* Real basis.                                                          */
/* ------------------------------------------------------------------ */

/* Row m (real index, -l..l) of the unitary matrix taking complex
 * spherical harmonics (Condon-Shortley phase) to real ones:
 *   m<0 : (i/sqrt2) (Y^m - (-1)^m Y^-m)
 *   m=0 : Y^0
 *   m>0 : (1/sqrt2) (Y^-m + (-1)^m Y^m)
 * U[(m+l)*(2l+1) + (mu+l)]. */
static void real_basis_matrix(int l, double complex *U) {
    int d = 2 * l + 1;
    for (int i = 0; i < d * d; ++i) U[i] = 0.0;
    const double r2 = 1.0 / sqrt(2.0);
    for (int m = -l; m <= l; ++m) {
        double sgn = (abs(m) % 2 == 0) ? 1.0 : -1.0; /* (-1)^m */
        if (m < 0) {
            U[(m + l) * d + (m + l)] += I * r2;
            U[(m + l) * d + (-m + l)] += -I * r2 * sgn;
        } else if (m == 0) {
            U[l * d + l] = 1.0;
        } else {
            U[(m + l) * d + (-m + l)] += r2;
            U[(m + l) * d + (m + l)] += r2 * sgn;
        }
    }
}

/* Real coupling tensor R[i][j][k] (i over 2l1+1, j over 2l2+1, k over
 * 2l3+1, all in real order m=-l..l):
 *   R = sum_mu U3[k,mu3] C[mu1,mu2,mu3] conj(U1[i,mu1]) conj(U2[j,mu2])
 * The real part is kept when l1+l2+l3 is even, the imaginary part when it
 * is odd (the other part vanishes).  Returns 0, or -1 for a forbidden
 * triple. */
int orc_real_cg(int l1, int l2, int l3, double *R) {
    if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > ORC_LMAX || l2 > ORC_LMAX || l3 > ORC_LMAX)
        return -1;
    if (l3 < abs(l1 - l2) || l3 > l1 + l2) return -1;
    int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
    double complex *U1 = malloc(sizeof(double complex) * d1 * d1);
    double complex *U2 = malloc(sizeof(double complex) * d2 * d2);
    double complex *U3 = malloc(sizeof(double complex) * d3 * d3);
    real_basis_matrix(l1, U1);
    real_basis_matrix(l2, U2);
    real_basis_matrix(l3, U3);
    int odd = (l1 + l2 + l3) % 2;
    for (int i = 0; i < d1; ++i)
        for (int j = 0; j < d2; ++j)
            for (int k = 0; k < d3; ++k) {
                double complex acc = 0.0;
                for (int a = 0; a < d1; ++a)
                    for (int b = 0; b < d2; ++b)
                        for (int c = 0; c < d3; ++c) {
                            double cg = orc_cg_complex(l1, a - l1, l2, b - l2, l3, c - l3);
                            if (cg == 0.0) continue;
                            acc += U3[k * d3 + c] * cg * conj(U1[i * d1 + a]) *
                                   conj(U2[j * d2 + b]);
                        }
                R[(i * d2 + j) * d3 + k] = odd ? cimag(acc) : creal(acc);
            }
    free(U1);
    free(U2);
    free(U3);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Real spherical harmonics, component normalisation.                   */
/*   Y_{l,0}  = sqrt(2l+1) P_l(cos t)                                   */
/*   Y_{l,+m} = sqrt(2l+1) sqrt(2 (l-m)!/(l+m)!) P_l^m(cos t) cos(m p)  */
/*   Y_{l,-m} = same with sin(m p)                                      */
/* P_l^m without the Condon-Shortley phase; index l*l + (m+l).          */
/* ------------------------------------------------------------------ */

/* Associated Legendre functions (no C-S phase) and their theta
 * derivatives, P[l][m], Q[l][m] = dP/dtheta, for 0<=m<=l<=lmax. */
static void legendre(int lmax, double ct, double st, double P[][ORC_LMAX + 1],
                     double Q[][ORC_LMAX + 1]) {
    for (int m = 0; m <= lmax; ++m) {
        /* P_m^m = (2m-1)!! s^m ; dP_m^m/dtheta = (2m-1)!! m c s^(m-1) */
        double dfact = 1.0;
        for (int k = 1; k <= 2 * m - 1; k += 2) dfact *= (double)k;
        double sm = 1.0;
        for (int k = 0; k < m; ++k) sm *= st;
        double sm1 = 1.0;
        for (int k = 0; k < m - 1; ++k) sm1 *= st;
        P[m][m] = dfact * sm;
        Q[m][m] = (m == 0) ? 0.0 : dfact * m * ct * sm1;
        if (m + 1 <= lmax) {
            /* P_{m+1}^m = (2m+1) c P_m^m ; derivative via d c/dtheta = -s */
            P[m + 1][m] = (2 * m + 1) * ct * P[m][m];
            Q[m + 1][m] = (2 * m + 1) * (-st * P[m][m] + ct * Q[m][m]);
        }
        for (int l = m + 2; l <= lmax; ++l) {
            P[l][m] = ((2 * l - 1) * ct * P[l - 1][m] - (l + m - 1) * P[l - 2][m]) / (l - m);
            Q[l][m] = ((2 * l - 1) * (-st * P[l - 1][m] + ct * Q[l - 1][m]) -
                       (l + m - 1) * Q[l - 2][m]) /
                      (l - m);
        }
    }
}

static double sh_norm(int l, int m) {
    int am = abs(m);
    double n = sqrt(2.0 * l + 1.0);
    if (am == 0) return n;
    return n * sqrt(2.0 * fact(l - am) / fact(l + am));
}

/* Y[n][(lmax+1)^2] of the directions r[n][3] (r need not be unit). */
void orc_sh(int lmax, int64_t n, const double *r, double *Y) {
    int nsh = (lmax + 1) * (lmax + 1);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        double x = r[3 * e], y = r[3 * e + 1], z = r[3 * e + 2];
        double rr = sqrt(x * x + y * y + z * z);
        double ct = z / rr, st = sqrt(x * x + y * y) / rr;
        double ph = atan2(y, x);
        double P[ORC_LMAX + 1][ORC_LMAX + 1], Q[ORC_LMAX + 1][ORC_LMAX + 1];
        legendre(lmax, ct, st, P, Q);
        for (int l = 0; l <= lmax; ++l)
            for (int m = -l; m <= l; ++m) {
                int am = abs(m);
                double t = (m > 0) ? cos(am * ph) : (m < 0 ? sin(am * ph) : 1.0);
                Y[e * nsh + l * l + m + l] = sh_norm(l, m) * P[l][am] * t;
            }
    }
}

/* J[n][(lmax+1)^2][3] = dY/dr at r (r unnormalised).  Chain rule through
 * spherical angles: grad Y = (1/|r|) (dY/dtheta e_theta + (1/sin t) dY/dphi
 * e_phi).  Valid away from the poles (sin t = 0). */
void orc_sh_jacobian(int lmax, int64_t n, const double *r, double *Jac) {
    int nsh = (lmax + 1) * (lmax + 1);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        double x = r[3 * e], y = r[3 * e + 1], z = r[3 * e + 2];
        double rr = sqrt(x * x + y * y + z * z);
        double ct = z / rr, st = sqrt(x * x + y * y) / rr;
        double ph = atan2(y, x);
        double cp = cos(ph), sp = sin(ph);
        double eth[3] = {ct * cp, ct * sp, -st};
        double eph[3] = {-sp, cp, 0.0};
        double P[ORC_LMAX + 1][ORC_LMAX + 1], Q[ORC_LMAX + 1][ORC_LMAX + 1];
        legendre(lmax, ct, st, P, Q);
        for (int l = 0; l <= lmax; ++l)
            for (int m = -l; m <= l; ++m) {
                int am = abs(m);
                double t, dt; /* angular factor and its phi derivative */
                if (m > 0) {
                    t = cos(am * ph);
                    dt = -am * sin(am * ph);
                } else if (m < 0) {
                    t = sin(am * ph);
                    dt = am * cos(am * ph);
                } else {
                    t = 1.0;
                    dt = 0.0;
                }
                double nrm = sh_norm(l, m);
                double dth = nrm * Q[l][am] * t;
                double dph_over_s = (am == 0) ? 0.0 : nrm * (P[l][am] / st) * dt;
                for (int c = 0; c < 3; ++c)
                    Jac[(e * nsh + l * l + m + l) * 3 + c] =
                        (dth * eth[c] + dph_over_s * eph[c]) / rr;
            }
    }
}

/* ------------------------------------------------------------------ */
/* Tensor product: one item.                                            */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t l1, l2, l3;
    int32_t mul1, mul2, mul3;
    int64_t off1, off2, off3; /* element offsets of the blocks in the rows */
    int64_t woff;             /* offset of this path's weights in a weight row */
} orc_path;

enum { ORC_UVU = 0, ORC_UVW = 1 };

typedef struct {
    const orc_path *paths;
    int np;
    int mode;
    double **R; /* R[p] dense real coupling tensor of path p */
} orc_plan;

static int plan_init(orc_plan *pl, const orc_path *paths, int np, int mode) {
    pl->paths = paths;
    pl->np = np;
    pl->mode = mode;
    pl->R = calloc((size_t)(np > 0 ? np : 1), sizeof(double *));
    for (int p = 0; p < np; ++p) {
        const orc_path *q = &paths[p];
        if (mode == ORC_UVU && q->mul3 != q->mul1) return -1;
        size_t sz = (size_t)(2 * q->l1 + 1) * (2 * q->l2 + 1) * (2 * q->l3 + 1);
        pl->R[p] = malloc(sizeof(double) * sz);
        if (orc_real_cg(q->l1, q->l2, q->l3, pl->R[p]) != 0) return -1;
    }
    return 0;
}

static void plan_free(orc_plan *pl) {
    for (int p = 0; p < pl->np; ++p) free(pl->R[p]);
    free(pl->R);
}

/* For path q, the weight index of the triple (u, v, o) where o is the
 * output multiplicity index (o == u in uvu mode). */
static int64_t widx(const orc_path *q, int mode, int u, int v, int o) {
    if (mode == ORC_UVU) return q->woff + (int64_t)u * q->mul2 + v;
    return q->woff + ((int64_t)u * q->mul2 + v) * q->mul3 + o;
}

/* z += f(x, y, w) for one item:
 *   z[off3 + o*d3 + k] += sum W(u,v,o) R[i,j,k] x[off1+u*d1+i] y[off2+v*d2+j] */
static void tp_item(const orc_plan *pl, const double *x, const double *y, const double *w,
                    double *z) {
    for (int p = 0; p < pl->np; ++p) {
        const orc_path *q = &pl->paths[p];
        const double *R = pl->R[p];
        int d1 = 2 * q->l1 + 1, d2 = 2 * q->l2 + 1, d3 = 2 * q->l3 + 1;
        for (int u = 0; u < q->mul1; ++u)
            for (int v = 0; v < q->mul2; ++v) {
                int olo = (pl->mode == ORC_UVU) ? u : 0;
                int ohi = (pl->mode == ORC_UVU) ? u + 1 : q->mul3;
                for (int o = olo; o < ohi; ++o) {
                    double wt = w[widx(q, pl->mode, u, v, o)];
                    for (int i = 0; i < d1; ++i)
                        for (int j = 0; j < d2; ++j)
                            for (int k = 0; k < d3; ++k)
                                z[q->off3 + (int64_t)o * d3 + k] +=
                                    wt * R[(i * d2 + j) * d3 + k] *
                                    x[q->off1 + (int64_t)u * d1 + i] *
                                    y[q->off2 + (int64_t)v * d2 + j];
                }
            }
    }
}

/* Adjoints of tp_item for one item with output cotangent g:
 *   gx[off1+u*d1+i] += sum W R y g ;  gy[...] += sum W R x g ;
 *   gw[widx]        += sum R x y g.    Any of gx, gy, gw may be NULL. */
static void tp_item_adjoint(const orc_plan *pl, const double *x, const double *y,
                            const double *w, const double *g, double *gx, double *gy,
                            double *gw) {
    for (int p = 0; p < pl->np; ++p) {
        const orc_path *q = &pl->paths[p];
        const double *R = pl->R[p];
        int d1 = 2 * q->l1 + 1, d2 = 2 * q->l2 + 1, d3 = 2 * q->l3 + 1;
        for (int u = 0; u < q->mul1; ++u)
            for (int v = 0; v < q->mul2; ++v) {
                int olo = (pl->mode == ORC_UVU) ? u : 0;
                int ohi = (pl->mode == ORC_UVU) ? u + 1 : q->mul3;
                for (int o = olo; o < ohi; ++o) {
                    int64_t wi = widx(q, pl->mode, u, v, o);
                    double wt = w[wi];
                    for (int i = 0; i < d1; ++i)
                        for (int j = 0; j < d2; ++j)
                            for (int k = 0; k < d3; ++k) {
                                double r = R[(i * d2 + j) * d3 + k];
                                double xi = x[q->off1 + (int64_t)u * d1 + i];
                                double yj = y[q->off2 + (int64_t)v * d2 + j];
                                double gk = g[q->off3 + (int64_t)o * d3 + k];
                                if (gx) gx[q->off1 + (int64_t)u * d1 + i] += wt * r * yj * gk;
                                if (gy) gy[q->off2 + (int64_t)v * d2 + j] += wt * r * xi * gk;
                                if (gw) gw[wi] += r * xi * yj * gk;
                            }
                }
            }
    }
}

/* ------------------------------------------------------------------ */
/* Public TP entry points.  wrow = weights per item; wrow == 0 means one  */
/* weight vector shared by all items.  Outputs are overwritten.          */
/* ------------------------------------------------------------------ */

int orc_tp_forward(const orc_path *paths, int np, int mode, int64_t batch, int64_t dim1,
                   int64_t dim2, int64_t dim3, int64_t wrow, const double *x, const double *y,
                   const double *w, double *out) {
    orc_plan pl;
    if (plan_init(&pl, paths, np, mode) != 0) {
        plan_free(&pl);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < batch; ++b) {
        double *z = out + b * dim3;
        for (int64_t k = 0; k < dim3; ++k) z[k] = 0.0;
        tp_item(&pl, x + b * dim1, y + b * dim2, w + b * wrow, z);
    }
    plan_free(&pl);
    return 0;
}

int orc_tp_backward(const orc_path *paths, int np, int mode, int64_t batch, int64_t dim1,
                    int64_t dim2, int64_t dim3, int64_t wrow, int64_t wnumel,
                    const double *x, const double *y, const double *w, const double *g,
                    double *gx, double *gy, double *gw) {
    orc_plan pl;
    if (plan_init(&pl, paths, np, mode) != 0) {
        plan_free(&pl);
        return -1;
    }
    if (gx) memset(gx, 0, sizeof(double) * batch * dim1);
    if (gy) memset(gy, 0, sizeof(double) * batch * dim2);
    if (gw) memset(gw, 0, sizeof(double) * (wrow ? batch * wrow : wnumel));
    if (wrow) {
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < batch; ++b)
            tp_item_adjoint(&pl, x + b * dim1, y + b * dim2, w + b * wrow, g + b * dim3,
                            gx ? gx + b * dim1 : NULL, gy ? gy + b * dim2 : NULL,
                            gw ? gw + b * wrow : NULL);
    } else {
        /* shared weights: the weight gradient sums over items, in item order */
        for (int64_t b = 0; b < batch; ++b)
            tp_item_adjoint(&pl, x + b * dim1, y + b * dim2, w, g + b * dim3,
                            gx ? gx + b * dim1 : NULL, gy ? gy + b * dim2 : NULL, gw);
    }
    plan_free(&pl);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Graph convolution.  Edges in any order; edge e carries y[e], w[e] and */
/* sends x[src[e]] to node dst[e]:                                       */
/*   out[n] = sum_{e : dst[e] == n} f(x[src[e]], y[e], w[e])             */
/* ------------------------------------------------------------------ */

/* Lists of edge ids grouped by key, each list in increasing edge id. */
typedef struct {
    int64_t *start; /* [n+1] */
    int64_t *ids;   /* [E]  */
} orc_groups;

static int groups_build(const int32_t *key, int64_t E, int64_t n, orc_groups *g) {
    g->start = calloc((size_t)n + 1, sizeof(int64_t));
    g->ids = malloc(sizeof(int64_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) {
        if (key[e] < 0 || key[e] >= n) return -1;
        g->start[key[e] + 1]++;
    }
    for (int64_t i = 0; i < n; ++i) g->start[i + 1] += g->start[i];
    int64_t *fill = calloc((size_t)n + 1, sizeof(int64_t));
    for (int64_t e = 0; e < E; ++e) g->ids[g->start[key[e]] + fill[key[e]]++] = e;
    free(fill);
    return 0;
}

static void groups_free(orc_groups *g) {
    free(g->start);
    free(g->ids);
}

int orc_conv_forward(const orc_path *paths, int np, int mode, int64_t n_nodes, int64_t n_edges,
                     const int32_t *src, const int32_t *dst, int64_t dim1, int64_t dim2,
                     int64_t dim3, int64_t wrow, const double *x, const double *y,
                     const double *w, double *out) {
    orc_plan pl;
    orc_groups gd;
    if (plan_init(&pl, paths, np, mode) != 0) {
        plan_free(&pl);
        return -1;
    }
    for (int64_t e = 0; e < n_edges; ++e)
        if (src[e] < 0 || src[e] >= n_nodes) {
            plan_free(&pl);
            return -1;
        }
    if (groups_build(dst, n_edges, n_nodes, &gd) != 0) {
        groups_free(&gd);
        plan_free(&pl);
        return -1;
    }
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t n = 0; n < n_nodes; ++n) {
        double *z = out + n * dim3;
        for (int64_t k = 0; k < dim3; ++k) z[k] = 0.0;
        for (int64_t t = gd.start[n]; t < gd.start[n + 1]; ++t) {
            int64_t e = gd.ids[t];
            tp_item(&pl, x + (int64_t)src[e] * dim1, y + e * dim2, w + e * wrow, z);
        }
    }
    groups_free(&gd);
    plan_free(&pl);
    return 0;
}

/* Adjoint of the convolution for output cotangent g_out[n_nodes][dim3]:
 *   g_x[s] = sum_{e : src[e]==s} (d/dx) ;  g_y[e], g_w[e] per edge.
 * Any output may be NULL.  With shared weights (wrow == 0) g_w has wnumel
 * entries summed over edges in edge order. */
int orc_conv_backward(const orc_path *paths, int np, int mode, int64_t n_nodes,
                      int64_t n_edges, const int32_t *src, const int32_t *dst, int64_t dim1,
                      int64_t dim2, int64_t dim3, int64_t wrow, int64_t wnumel,
                      const double *x, const double *y, const double *w, const double *g_out,
                      double *g_x, double *g_y, double *g_w) {
    orc_plan pl;
    orc_groups gs;
    if (plan_init(&pl, paths, np, mode) != 0) {
        plan_free(&pl);
        return -1;
    }
    for (int64_t e = 0; e < n_edges; ++e)
        if (dst[e] < 0 || dst[e] >= n_nodes) {
            plan_free(&pl);
            return -1;
        }
    if (groups_build(src, n_edges, n_nodes, &gs) != 0) {
        groups_free(&gs);
        plan_free(&pl);
        return -1;
    }
    if (g_x) {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t s = 0; s < n_nodes; ++s) {
            double *gx = g_x + s * dim1;
            for (int64_t k = 0; k < dim1; ++k) gx[k] = 0.0;
            for (int64_t t = gs.start[s]; t < gs.start[s + 1]; ++t) {
                int64_t e = gs.ids[t];
                tp_item_adjoint(&pl, x + s * dim1, y + e * dim2, w + e * wrow,
                                g_out + (int64_t)dst[e] * dim3, gx, NULL, NULL);
            }
        }
    }
    if (g_y || (g_w && wrow)) {
#pragma omp parallel for schedule(static)
        for (int64_t e = 0; e < n_edges; ++e) {
            double *gy = g_y ? g_y + e * dim2 : NULL;
            double *gw = (g_w && wrow) ? g_w + e * wrow : NULL;
            if (gy)
                for (int64_t k = 0; k < dim2; ++k) gy[k] = 0.0;
            if (gw)
                for (int64_t k = 0; k < wrow; ++k) gw[k] = 0.0;
            tp_item_adjoint(&pl, x + (int64_t)src[e] * dim1, y + e * dim2, w + e * wrow,
                            g_out + (int64_t)dst[e] * dim3, NULL, gy, gw);
        }
    }
    if (g_w && !wrow) {
        memset(g_w, 0, sizeof(double) * wnumel);
        for (int64_t e = 0; e < n_edges; ++e)
            tp_item_adjoint(&pl, x + (int64_t)src[e] * dim1, y + e * dim2, w,
                            g_out + (int64_t)dst[e] * dim3, NULL, NULL, g_w);
    }
    groups_free(&gs);
    plan_free(&pl);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Forces.  r_e = pos[dst] - pos[src], sh_e = Y(r_e).  For an energy     */
/* with gradient g_sh[e] = dE/dsh_e:                                      */
/*   F_a = -dE/dpos_a = -sum_{e:dst=a} J_e^T g_e + sum_{e:src=a} J_e^T g_e */
/* Summed per atom over edges in edge order.                             */
/* ------------------------------------------------------------------ */

int orc_forces(int lmax, int64_t n_nodes, int64_t n_edges, const int32_t *src,
               const int32_t *dst, const double *r, const double *g_sh, double *F) {
    int nsh = (lmax + 1) * (lmax + 1);
    double *Jac = malloc(sizeof(double) * (size_t)(n_edges > 0 ? n_edges : 1) * nsh * 3);
    orc_sh_jacobian(lmax, n_edges, r, Jac);
    memset(F, 0, sizeof(double) * n_nodes * 3);
    for (int64_t e = 0; e < n_edges; ++e) {
        if (src[e] < 0 || src[e] >= n_nodes || dst[e] < 0 || dst[e] >= n_nodes) {
            free(Jac);
            return -1;
        }
        for (int c = 0; c < 3; ++c) {
            double v = 0.0;
            for (int k = 0; k < nsh; ++k) v += Jac[(e * nsh + k) * 3 + c] * g_sh[e * nsh + k];
            F[(int64_t)dst[e] * 3 + c] -= v;
            F[(int64_t)src[e] * 3 + c] += v;
        }
    }
    free(Jac);
    return 0;
}

/* Cotangent on sh of the force loss L = 1/2 sum_a |F_a|^2:
 *   gg_sh[e] = dL/dg_sh[e] = -J_e (F[dst_e] - F[src_e]). */
int orc_force_loss_cotangent(int lmax, int64_t n_nodes, int64_t n_edges, const int32_t *src,
                             const int32_t *dst, const double *r, const double *F,
                             double *gg_sh) {
    int nsh = (lmax + 1) * (lmax + 1);
    double *Jac = malloc(sizeof(double) * (size_t)(n_edges > 0 ? n_edges : 1) * nsh * 3);
    orc_sh_jacobian(lmax, n_edges, r, Jac);
    for (int64_t e = 0; e < n_edges; ++e) {
        if (src[e] < 0 || src[e] >= n_nodes || dst[e] < 0 || dst[e] >= n_nodes) {
            free(Jac);
            return -1;
        }
        for (int k = 0; k < nsh; ++k) {
            double v = 0.0;
            for (int c = 0; c < 3; ++c)
                v += Jac[(e * nsh + k) * 3 + c] *
                     (F[(int64_t)dst[e] * 3 + c] - F[(int64_t)src[e] * 3 + c]);
            gg_sh[e * nsh + k] = -v;
        }
    }
    free(Jac);
    return 0;
}

/* ------------------------------------------------------------------ */
/* CSR: stable sort of edge ids by key.                                  */
/*   perm[t] = t-th edge id in (key, edge id) order                      */
/*   row_ptr[n] = number of edges with key < n                           */
/* ------------------------------------------------------------------ */

int orc_csr(const int32_t *key, int64_t n_edges, int64_t n_nodes, int32_t *perm,
            int32_t *row_ptr) {
    int64_t *cnt = calloc((size_t)n_nodes + 1, sizeof(int64_t));
    for (int64_t e = 0; e < n_edges; ++e) {
        if (key[e] < 0 || key[e] >= n_nodes) {
            free(cnt);
            return -1;
        }
        cnt[key[e] + 1]++;
    }
    for (int64_t n = 0; n < n_nodes; ++n) cnt[n + 1] += cnt[n];
    for (int64_t n = 0; n <= n_nodes; ++n) row_ptr[n] = (int32_t)cnt[n];
    for (int64_t e = 0; e < n_edges; ++e) perm[cnt[key[e]]++] = (int32_t)e;
    free(cnt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Sparse attention over a graph: "Fused3S: Fast Sparse Attention on    */
/* Tensor Cores" (abstract) splits it into sampled dense-dense matrix    */
/* multiplication, softmax normalisation and sparse matrix               */
/* multiplication.  Written here as those three steps, per head h:       */
/*   s_e   = scale * <q[dst e][h], k[src e][h]>          (SDDMM)         */
/*   p_e   = exp(s_e) / sum_{e': dst e' = dst e} exp(s_e')   (softmax)   */
/*   out[i][h] = sum_{e: dst e = i} p_e v[src e][h]      (SpMM)          */
/* Rows with no edge are zero.  q [n_rows][H][d], k and v [n_cols][H][d], */
/* out [n_rows][H][d]; edges in any order.                               */
/* ------------------------------------------------------------------ */

int orc_sparse_attention(int64_t n_rows, int64_t n_cols, int64_t n_edges, const int32_t *src,
                         const int32_t *dst, int n_heads, int head_dim, double scale, const double *q,
                         const double *k, const double *v, double *out) {
    /* edges of each row, in edge order */
    int64_t *start = calloc((size_t)n_rows + 1, sizeof(int64_t));
    int64_t *idx = malloc(sizeof(int64_t) * (size_t)(n_edges > 0 ? n_edges : 1));
    for (int64_t e = 0; e < n_edges; ++e) {
        if (src[e] < 0 || src[e] >= n_cols || dst[e] < 0 || dst[e] >= n_rows) {
            free(start);
            free(idx);
            return -1;
        }
        start[dst[e] + 1]++;
    }
    for (int64_t i = 0; i < n_rows; ++i) start[i + 1] += start[i];
    {
        int64_t *fill = malloc(sizeof(int64_t) * (size_t)(n_rows + 1));
        memcpy(fill, start, sizeof(int64_t) * (size_t)(n_rows + 1));
        for (int64_t e = 0; e < n_edges; ++e) idx[fill[dst[e]]++] = e;
        free(fill);
    }
    const int64_t rowlen = (int64_t)n_heads * head_dim;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t deg = start[i + 1] - start[i];
        double *s = malloc(sizeof(double) * (size_t)(deg > 0 ? deg : 1));
        for (int h = 0; h < n_heads; ++h) {
            double *o = out + i * rowlen + (int64_t)h * head_dim;
            for (int c = 0; c < head_dim; ++c) o[c] = 0.0;
            if (deg == 0) continue;
            const double *qi = q + i * rowlen + (int64_t)h * head_dim;
            /* SDDMM: scores of the row's edges */
            double smax = -HUGE_VAL;
            for (int64_t t = 0; t < deg; ++t) {
                const double *kj = k + (int64_t)src[idx[start[i] + t]] * rowlen + (int64_t)h * head_dim;
                double dot = 0.0;
                for (int c = 0; c < head_dim; ++c) dot += qi[c] * kj[c];
                s[t] = scale * dot;
                if (s[t] > smax) smax = s[t];
            }
            /* softmax over the row (shifted by the row maximum) */
            double z = 0.0;
            for (int64_t t = 0; t < deg; ++t) {
                s[t] = exp(s[t] - smax);
                z += s[t];
            }
            /* SpMM */
            for (int64_t t = 0; t < deg; ++t) {
                const double *vj = v + (int64_t)src[idx[start[i] + t]] * rowlen + (int64_t)h * head_dim;
                const double p = s[t] / z;
                for (int c = 0; c < head_dim; ++c) o[c] += p * vj[c];
            }
        }
        free(s);
    }
    free(start);
    free(idx);
    return 0;
}

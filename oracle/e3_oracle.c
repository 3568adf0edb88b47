/*
 * e3_oracle.c -- plain, slow, fp64 CPU oracle for the fused equivariant
 * message-passing convolution and the channel-wise Clebsch-Gordan tensor
 * product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library; the only common ground is the convention
 * it implements, restated below from the sources it follows.
 *
 * Sources (page titles; sections / equations):
 *   [e3j]  "e3j: An Efficient and Open-Source Backend for Euclidean
 *          Equivariant Operations on GPU and TPU" (arXiv html version).
 *     - A.3 Eq.4   bank of real harmonics Y_l(r), l = 0..lmax
 *     - A.3 Eq.6   CG coupling (x (x)_C y)^{LM} = sum_{m+m'=M} C x^{lm} y^{l'm'}
 *     - A.3 Eq.7, E.1 Eq.12-13  message passing m_b = sum_a s_ab (x_a (x) Y(r_ab))
 *     - E.1 Eq.10-11  sparse bilinear TP with per-block edge scalars
 *     - E.1 Eq.16  VJP of the convolution (dx, dy, ds)
 *     - B.1        parity selection rule p1 p2 = p3
 *     - G.1 Eq.19-21 spin / ladder structure of the harmonics
 *   [Tessera] "Ab Initio Accuracy Beyond the Cutoff: Distributed
 *          Message-Passing Equivariant Attention at Tens-of-Millions-of-Atom
 *          Scale" (html version).
 *     - 2.2 Eq.3   forces as the negative analytic gradient of the energy
 *   Textbook material used where the pages stay silent (normalisation and
 *   phase are left open there, G.1 and G.2): Racah's closed form for the
 *   complex CG coefficients with the Condon-Shortley phase, and the standard
 *   complex-to-real change of basis of the spherical harmonics.
 *
 * Conventions (the specification both this oracle and the GPU library obey):
 *   - irreps are (l, parity); a feature block of irrep l has 2l+1 components
 *     ordered m = -l..l; channels are the innermost axis;
 *   - real harmonics are component-normalised: sum_m Y_lm(r)^2 = 2l+1;
 *   - real CG block T^{(l1,l2,L)}[M][m1][m2] = U_L C (U_l1^dag (x) U_l2^dag),
 *     which is purely real when l1+l2+L is even and purely imaginary when it
 *     is odd; the oracle keeps Re T (even) or Im T (odd);
 *   - paths are enumerated x-irrep major, then y-irrep, then output irrep,
 *     keeping (ix,iy,io) iff |lx-ly| <= lo <= lx+ly and px*py == po;
 *   - outputs of paths that land on the same output irrep are summed after
 *     their per-path weights are applied (collapsed output);
 *   - r_e = pos[receiver] - pos[sender]; a negative sender marks a padding
 *     edge, which contributes nothing and has zero gradients.
 *
 * Precision: fp64 throughout, plain loops, OpenMP over independent output
 * rows only (no reordering of any sum).
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_IRREPS 16
#define ORACLE_MAX_L 8 /* harmonics; CG blocks up to twice this */
#define ORACLE_MAX_DY 128 /* y components per row (the per-edge y buffer) */
#define ORACLE_MAX_PATHS 256

typedef struct {
  int nx, ny, no;
  int xl[ORACLE_MAX_IRREPS], xp[ORACLE_MAX_IRREPS];
  int yl[ORACLE_MAX_IRREPS], yp[ORACLE_MAX_IRREPS];
  int ol[ORACLE_MAX_IRREPS], op[ORACLE_MAX_IRREPS];
  int C; /* channels (multiplicity of every x and output irrep) */
  /* 0: paths landing on the same output irrep are summed (collapsed);
   * 1: every path keeps its own output block, in path order (e3j's
   *    default, one output block per path: A.3, E.1) */
  int per_path;
} oracle_desc;

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the later parallel loops (n > 0); used to time the oracle
 * on one thread.  No arithmetic depends on it: every output row is computed
 * by one thread in a fixed order. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static long double factorial(int n) {
  long double r = 1.0L;
  for (int i = 2; i <= n; ++i) r *= (long double)i;
  return r;
}

/* <l1 m1 l2 m2 | L M> by Racah's closed form (Condon-Shortley phase), in
 * long double: the alternating sum cancels more with the degree, and the
 * factorials stay exact up to 20!. */
double oracle_cg_complex(int l1, int m1, int l2, int m2, int L, int M) {
  if (M != m1 + m2) return 0.0;
  if (L < abs(l1 - l2) || L > l1 + l2) return 0.0;
  if (abs(m1) > l1 || abs(m2) > l2 || abs(M) > L) return 0.0;
  long double pre = sqrtl((2.0L * L + 1.0L) * factorial(L + l1 - l2) * factorial(L - l1 + l2) *
                          factorial(l1 + l2 - L) / factorial(l1 + l2 + L + 1));
  pre *= sqrtl(factorial(L + M) * factorial(L - M) * factorial(l1 - m1) * factorial(l1 + m1) *
               factorial(l2 - m2) * factorial(l2 + m2));
  long double s = 0.0L;
  for (int k = 0;; ++k) {
    int d1 = l1 + l2 - L - k, d2 = l1 - m1 - k, d3 = l2 + m2 - k;
    int d4 = L - l2 + m1 + k, d5 = L - l1 - m2 + k;
    if (d1 < 0 || d2 < 0 || d3 < 0) break; /* these only shrink with k */
    if (d4 < 0 || d5 < 0) continue;        /* these only grow with k */
    long double t = factorial(k) * factorial(d1) * factorial(d2) * factorial(d3) *
                    factorial(d4) * factorial(d5);
    s += ((k & 1) ? -1.0L : 1.0L) / t;
  }
  return (double)(pre * s);
}

/* Complex -> real change of basis U_l (row = real m, column = complex m'),
 * so that real harmonics = U_l * complex harmonics:
 *   m > 0 :  Y_{l,m}  = (Y_l^{-m} + (-1)^m Y_l^{m}) / sqrt2
 *   m = 0 :  Y_{l,0}  =  Y_l^0
 *   m < 0 :  Y_{l,m}  = i (Y_l^{m} - (-1)^m Y_l^{-m}) / sqrt2            */
static void umat(int l, double complex *U) {
  int n = 2 * l + 1;
  const double s = 1.0 / sqrt(2.0);
  memset(U, 0, sizeof(double complex) * n * n);
  for (int m = -l; m <= l; ++m) {
    int r = m + l;
    double sgn = (m & 1) ? -1.0 : 1.0;
    if (m == 0) {
      U[r * n + l] = 1.0;
    } else if (m > 0) {
      U[r * n + (-m + l)] = s;
      U[r * n + (m + l)] = sgn * s;
    } else {
      U[r * n + (m + l)] = I * s;
      U[r * n + (-m + l)] = -I * sgn * s;
    }
  }
}

void oracle_umat(int l, double *re, double *im) {
  if (l < 0 || l > 2 * ORACLE_MAX_L) return;
  int n = 2 * l + 1;
  double complex U[(2 * ORACLE_MAX_L + 1) * (2 * ORACLE_MAX_L + 1) * 4];
  umat(l, U);
  for (int i = 0; i < n * n; ++i) {
    re[i] = creal(U[i]);
    im[i] = cimag(U[i]);
  }
}

/* Real CG block out[(M*(2l1+1) + m1)*(2l2+1) + m2], indices shifted by +l.
 * Returns 0 on success, -1 if the triple is not coupled. */
int oracle_cg_real(int l1, int l2, int L, double *out) {
  if (l1 < 0 || l2 < 0 || L < abs(l1 - l2) || L > l1 + l2 || l1 > 2 * ORACLE_MAX_L ||
      l2 > 2 * ORACLE_MAX_L || L > 2 * ORACLE_MAX_L)
    return -1;
  int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, nL = 2 * L + 1;
  double complex *U1 = malloc(sizeof(double complex) * n1 * n1);
  double complex *U2 = malloc(sizeof(double complex) * n2 * n2);
  double complex *UL = malloc(sizeof(double complex) * nL * nL);
  umat(l1, U1);
  umat(l2, U2);
  umat(L, UL);
  int odd = (l1 + l2 + L) & 1;
  for (int M = 0; M < nL; ++M)
    for (int a = 0; a < n1; ++a)
      for (int b = 0; b < n2; ++b) {
        double complex t = 0.0;
        for (int Mp = 0; Mp < nL; ++Mp)
          for (int ap = 0; ap < n1; ++ap)
            for (int bp = 0; bp < n2; ++bp) {
              double c = oracle_cg_complex(l1, ap - l1, l2, bp - l2, L, Mp - L);
              if (c == 0.0) continue;
              t += UL[M * nL + Mp] * c * conj(U1[a * n1 + ap]) * conj(U2[b * n2 + bp]);
            }
        out[(M * n1 + a) * n2 + b] = odd ? cimag(t) : creal(t);
      }
  free(U1);
  free(U2);
  free(UL);
  return 0;
}

/* Component-normalised real harmonics of any degree l from the textbook
 * construction: complex Y_l^m = N_lm P_l^m(cos t) e^{i m phi} with the
 * Condon-Shortley phase, moved to the real basis of umat() and scaled by
 * sqrt(4 pi).  The phase factors cancel, leaving for m > 0
 *   Y_{l, m} = sqrt(2 (2l+1) (l-m)!/(l+m)!) Q_l^m(z) Re (x + i y)^m
 *   Y_{l,-m} = sqrt(2 (2l+1) (l-m)!/(l+m)!) Q_l^m(z) Im (x + i y)^m
 *   Y_{l, 0} = sqrt(2l+1) P_l(z)
 * with Q_l^m = P_l^m / sin^m t (without the phase) a polynomial in z:
 * Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m,
 * (l-m) Q_l^m = (2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m.
 * Used for l >= 4 (and checked against the polynomials below for l <= 3). */
int oracle_sh_general(int l, const double r[3], double *out) {
  if (l < 0 || l > ORACLE_MAX_L) return -1;
  double n = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  if (n == 0.0) { /* no direction: 1 at l = 0, zeros above (as the closed forms) */
    for (int m = 0; m < 2 * l + 1; ++m) out[m] = (l == 0) ? 1.0 : 0.0;
    return 0;
  }
  double x = 0, y = 0, z = 0;
  if (n > 0) {
    x = r[0] / n;
    y = r[1] / n;
    z = r[2] / n;
  }
  double cr = 1.0, ci = 0.0; /* (x + i y)^m */
  for (int m = 0; m <= l; ++m) {
    double q_mm = 1.0; /* (2m-1)!! */
    for (int k = 2 * m - 1; k > 1; k -= 2) q_mm *= k;
    double q = q_mm;
    if (l > m) {
      double q_prev = q_mm, q_cur = (2 * m + 1) * z * q_mm;
      for (int ll = m + 2; ll <= l; ++ll) {
        double q_next = ((2 * ll - 1) * z * q_cur - (ll + m - 1) * q_prev) / (ll - m);
        q_prev = q_cur;
        q_cur = q_next;
      }
      q = q_cur;
    }
    double ratio = 1.0; /* (l-m)!/(l+m)! */
    for (int k = l - m + 1; k <= l + m; ++k) ratio /= k;
    if (m == 0) {
      out[l] = sqrt(2.0 * l + 1.0) * q;
    } else {
      double c = sqrt(2.0 * (2.0 * l + 1.0) * ratio) * q;
      out[l + m] = c * cr;
      out[l - m] = c * ci;
    }
    double nr = cr * x - ci * y, ni = cr * y + ci * x;
    cr = nr;
    ci = ni;
  }
  return 0;
}

/* Component-normalised real harmonics of the unit vector r/|r|, written out
 * as polynomials for l <= 3, by oracle_sh_general above for l = 4..8.
 * out has 2l+1 entries, m = -l..l.  A zero vector yields the l = 0 value
 * only (higher degrees are 0). */
int oracle_sh_l(int l, const double r[3], double *out) {
  double n = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  double x = 0, y = 0, z = 0;
  if (n > 0) {
    x = r[0] / n;
    y = r[1] / n;
    z = r[2] / n;
  }
  switch (l) {
    case 0:
      out[0] = 1.0;
      return 0;
    case 1: {
      double s3 = sqrt(3.0);
      out[0] = s3 * y;
      out[1] = s3 * z;
      out[2] = s3 * x;
      return 0;
    }
    case 2: {
      double s15 = sqrt(15.0), s5 = sqrt(5.0);
      out[0] = s15 * x * y;
      out[1] = s15 * y * z;
      out[2] = 0.5 * s5 * (2 * z * z - x * x - y * y);
      out[3] = s15 * x * z;
      out[4] = 0.5 * s15 * (x * x - y * y);
      return 0;
    }
    case 3: {
      double a = sqrt(35.0 / 8.0), b = sqrt(105.0), c = sqrt(21.0 / 8.0), d = sqrt(7.0);
      out[0] = a * (3 * x * x - y * y) * y;
      out[1] = b * x * y * z;
      out[2] = c * y * (4 * z * z - x * x - y * y);
      out[3] = 0.5 * d * z * (2 * z * z - 3 * x * x - 3 * y * y);
      out[4] = c * x * (4 * z * z - x * x - y * y);
      out[5] = 0.5 * b * (x * x - y * y) * z;
      out[6] = a * (x * x - 3 * y * y) * x;
      return 0;
    }
    default:
      return oracle_sh_general(l, r, out);
  }
}

/* Harmonics for l = 0..lmax concatenated: out has (lmax+1)^2 entries. */
int oracle_sh(int lmax, const double r[3], double *out) {
  if (lmax < 0 || lmax > ORACLE_MAX_L) return -1;
  int o = 0;
  for (int l = 0; l <= lmax; ++l) {
    oracle_sh_l(l, r, out + o);
    o += 2 * l + 1;
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Path enumeration and CG blocks for one descriptor.                      */

typedef struct {
  int ix, iy, io, l1, l2, L;
  int xoff, yoff, ooff;
  double *T; /* dense real CG block, (2L+1) x (2l1+1) x (2l2+1) */
} opath;

typedef struct {
  int np;
  opath p[ORACLE_MAX_PATHS];
  int dx, dy, dout;
  int yoff[ORACLE_MAX_IRREPS];
} oplan;

static int plan_build(const oracle_desc *d, oplan *pl) {
  int xoff[ORACLE_MAX_IRREPS], ooff[ORACLE_MAX_IRREPS];
  if (d->nx < 0 || d->ny < 0 || d->no < 0 || d->nx > ORACLE_MAX_IRREPS ||
      d->ny > ORACLE_MAX_IRREPS || d->no > ORACLE_MAX_IRREPS)
    return -1;
  pl->dx = pl->dy = pl->dout = 0;
  for (int i = 0; i < d->nx; ++i) {
    xoff[i] = pl->dx;
    pl->dx += 2 * d->xl[i] + 1;
  }
  for (int i = 0; i < d->ny; ++i) {
    pl->yoff[i] = pl->dy;
    pl->dy += 2 * d->yl[i] + 1;
  }
  for (int i = 0; i < d->no; ++i) {
    ooff[i] = pl->dout;
    pl->dout += 2 * d->ol[i] + 1;
  }
  if (pl->dy > ORACLE_MAX_DY) return -1; /* per-edge y buffer below */
  pl->np = 0;
  for (int ix = 0; ix < d->nx; ++ix)
    for (int iy = 0; iy < d->ny; ++iy)
      for (int io = 0; io < d->no; ++io) {
        int l1 = d->xl[ix], l2 = d->yl[iy], L = d->ol[io];
        if (L < abs(l1 - l2) || L > l1 + l2) continue;
        if (d->xp[ix] * d->yp[iy] != d->op[io]) continue;
        if (pl->np >= ORACLE_MAX_PATHS) return -1;
        opath *p = &pl->p[pl->np++];
        p->ix = ix;
        p->iy = iy;
        p->io = io;
        p->l1 = l1;
        p->l2 = l2;
        p->L = L;
        p->xoff = xoff[ix];
        p->yoff = pl->yoff[iy];
        p->ooff = ooff[io];
        p->T = malloc(sizeof(double) * (2 * L + 1) * (2 * l1 + 1) * (2 * l2 + 1));
        if (oracle_cg_real(l1, l2, L, p->T) != 0) return -1;
      }
  if (d->per_path) { /* one output block per path, in path order */
    pl->dout = 0;
    for (int i = 0; i < pl->np; ++i) {
      pl->p[i].ooff = pl->dout;
      pl->dout += 2 * pl->p[i].L + 1;
    }
  }
  return 0;
}

static void plan_free(oplan *pl) {
  for (int i = 0; i < pl->np; ++i) free(pl->p[i].T);
  pl->np = 0;
}

int oracle_num_paths(const oracle_desc *d) {
  oplan *pl = malloc(sizeof(oplan));
  int r = plan_build(d, pl);
  int n = r == 0 ? pl->np : -1;
  plan_free(pl);
  free(pl);
  return n;
}

/* (ix, iy, io) of path i in canonical order; returns -1 when out of range. */
int oracle_path_info(const oracle_desc *d, int i, int *ix, int *iy, int *io) {
  oplan *pl = malloc(sizeof(oplan));
  int r = plan_build(d, pl);
  if (r == 0 && i >= 0 && i < pl->np) {
    *ix = pl->p[i].ix;
    *iy = pl->p[i].iy;
    *io = pl->p[i].io;
  } else {
    r = -1;
  }
  plan_free(pl);
  free(pl);
  return r;
}

/* The y operand of edge e: either given (Yg[e][dy]) or the harmonics of the
 * edge vector, one bank per y irrep (each must have the harmonic parity). */
static int edge_y(const oracle_desc *d, const oplan *pl, int64_t e, const double *evec,
                  const double *Yg, double *Ye) {
  if (Yg) {
    memcpy(Ye, Yg + e * pl->dy, sizeof(double) * pl->dy);
    return 0;
  }
  for (int iy = 0; iy < d->ny; ++iy) {
    int l = d->yl[iy];
    if (l > ORACLE_MAX_L) return -1;
    if (d->yp[iy] != ((l & 1) ? -1 : 1)) return -1;
    oracle_sh_l(l, evec + 3 * e, Ye + pl->yoff[iy]);
  }
  return 0;
}

static int check_y(const oracle_desc *d, const double *Yg) {
  if (Yg) return 0;
  for (int iy = 0; iy < d->ny; ++iy) {
    int l = d->yl[iy];
    if (l > ORACLE_MAX_L || d->yp[iy] != ((l & 1) ? -1 : 1)) return -1;
  }
  return 0;
}

/* Conv forward, [e3j] E.1 Eq.13 with one scalar block per path:
 *   m[b][ooff+M][q] = sum_{e in row b, sender >= 0} sum_P w[e][P][q]
 *                       sum_{m1,m2} T_P[M][m1][m2] x[sender][xoff+m1][q] Y_e[yoff+m2]
 * Computed for receivers rows[0..nrows-1]; m is [nrows][dout][C]. */
int oracle_conv_forward(const oracle_desc *d, int n_nodes, int64_t n_edges, const int *rowptr,
                        const int *sender, const double *evec, const double *Yg, const double *x,
                        const double *w, int nrows, const int *rows, double *m) {
  (void)n_edges;
  oplan *pl = malloc(sizeof(oplan));
  if (plan_build(d, pl) != 0 || check_y(d, Yg) != 0) {
    plan_free(pl);
    free(pl);
    return -1;
  }
  const int C = d->C, P = pl->np, dx = pl->dx, dout = pl->dout;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (int i = 0; i < nrows; ++i) {
    int b = rows[i];
    double *mb = m + (int64_t)i * dout * C;
    memset(mb, 0, sizeof(double) * dout * C);
    if (b < 0 || b >= n_nodes) {
      bad = 1;
      continue;
    }
    double Ye[ORACLE_MAX_DY];
    for (int64_t e = rowptr[b]; e < rowptr[b + 1]; ++e) {
      int a = sender[e];
      if (a < 0) continue; /* padding edge */
      edge_y(d, pl, e, evec, Yg, Ye);
      const double *xa = x + (int64_t)a * dx * C;
      const double *we = w + e * P * C;
      for (int pi = 0; pi < P; ++pi) {
        const opath *p = &pl->p[pi];
        int n1 = 2 * p->l1 + 1, n2 = 2 * p->l2 + 1, nL = 2 * p->L + 1;
        for (int M = 0; M < nL; ++M)
          for (int m1 = 0; m1 < n1; ++m1)
            for (int m2 = 0; m2 < n2; ++m2) {
              double c = p->T[(M * n1 + m1) * n2 + m2];
              if (c == 0.0) continue;
              double cy = c * Ye[p->yoff + m2];
              for (int q = 0; q < C; ++q)
                mb[(p->ooff + M) * C + q] +=
                    we[pi * C + q] * cy * xa[(p->xoff + m1) * C + q];
            }
      }
    }
  }
  plan_free(pl);
  free(pl);
  return bad ? -1 : 0;
}

/* Standalone TP forward, [e3j] E.1 Eq.10-11 applied row by row:
 *   z[r][ooff+M][q] = sum_P w[r][P][q] sum_{m1,m2} T_P[M][m1][m2] x[r][xoff+m1][q] y[r][yoff+m2]
 * for rows[0..nrows-1]; z is [nrows][dout][C]. */
int oracle_tp_forward(const oracle_desc *d, int64_t n_rows, const double *x, const double *y,
                      const double *w, int nrows, const int64_t *rows, double *z) {
  oplan *pl = malloc(sizeof(oplan));
  if (plan_build(d, pl) != 0) {
    plan_free(pl);
    free(pl);
    return -1;
  }
  const int C = d->C, P = pl->np, dx = pl->dx, dy = pl->dy, dout = pl->dout;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int i = 0; i < nrows; ++i) {
    int64_t r = rows[i];
    double *zr = z + (int64_t)i * dout * C;
    memset(zr, 0, sizeof(double) * dout * C);
    if (r < 0 || r >= n_rows) {
      bad = 1;
      continue;
    }
    const double *xr = x + r * dx * C, *yr = y + r * dy, *wr = w + r * P * C;
    for (int pi = 0; pi < P; ++pi) {
      const opath *p = &pl->p[pi];
      int n1 = 2 * p->l1 + 1, n2 = 2 * p->l2 + 1, nL = 2 * p->L + 1;
      for (int M = 0; M < nL; ++M)
        for (int m1 = 0; m1 < n1; ++m1)
          for (int m2 = 0; m2 < n2; ++m2) {
            double c = p->T[(M * n1 + m1) * n2 + m2];
            if (c == 0.0) continue;
            double cy = c * yr[p->yoff + m2];
            for (int q = 0; q < C; ++q)
              zr[(p->ooff + M) * C + q] += wr[pi * C + q] * cy * xr[(p->xoff + m1) * C + q];
          }
    }
  }
  plan_free(pl);
  free(pl);
  return bad ? -1 : 0;
}

/* Receiver of every edge from the CSR row pointers (plain scan). */
static int *edge_receivers(int n_nodes, int64_t n_edges, const int *rowptr) {
  int *recv = malloc(sizeof(int) * (n_edges > 0 ? n_edges : 1));
  for (int b = 0; b < n_nodes; ++b)
    for (int64_t e = rowptr[b]; e < rowptr[b + 1]; ++e) recv[e] = b;
  return recv;
}

/* Conv backward, node cotangent, [e3j] E.1 Eq.16 (first line) with per-path
 * scalars:  dx[a][xoff+m1][q] = sum_{e: sender(e)=a} sum_P w[e][P][q]
 *             sum_{M,m2} T_P[M][m1][m2] Y_e[yoff+m2] dm[recv(e)][ooff+M][q]
 * for senders rows[0..nrows-1]; dx is [nrows][dx][C]. */
int oracle_conv_backward_dx(const oracle_desc *d, int n_nodes, int64_t n_edges, const int *rowptr,
                            const int *sender, const double *evec, const double *Yg,
                            const double *w, const double *dm, int nrows, const int *rows,
                            double *dxo) {
  oplan *pl = malloc(sizeof(oplan));
  if (plan_build(d, pl) != 0 || check_y(d, Yg) != 0) {
    plan_free(pl);
    free(pl);
    return -1;
  }
  const int C = d->C, P = pl->np, dx = pl->dx, dout = pl->dout;
  int *recv = edge_receivers(n_nodes, n_edges, rowptr);
  /* out-edges of each requested sender, by one pass over all edges */
  int *slot = malloc(sizeof(int) * (n_nodes > 0 ? n_nodes : 1));
  for (int a = 0; a < n_nodes; ++a) slot[a] = -1;
  int bad = 0;
  for (int i = 0; i < nrows; ++i) {
    if (rows[i] < 0 || rows[i] >= n_nodes) bad = 1;
    else slot[rows[i]] = i;
  }
  int64_t *cnt = calloc(nrows + 1, sizeof(int64_t));
  for (int64_t e = 0; e < n_edges; ++e)
    if (sender[e] >= 0 && slot[sender[e]] >= 0) cnt[slot[sender[e]] + 1]++;
  for (int i = 0; i < nrows; ++i) cnt[i + 1] += cnt[i];
  int64_t *lst = malloc(sizeof(int64_t) * (cnt[nrows] > 0 ? cnt[nrows] : 1));
  int64_t *fill = calloc(nrows + 1, sizeof(int64_t));
  for (int64_t e = 0; e < n_edges; ++e)
    if (sender[e] >= 0 && slot[sender[e]] >= 0) {
      int i = slot[sender[e]];
      lst[cnt[i] + fill[i]++] = e;
    }
  /* a sender listed twice in rows gets its result in the last slot only;
   * fill the others the same way for consistency */
#pragma omp parallel for schedule(dynamic, 4)
  for (int i = 0; i < nrows; ++i) {
    double *out = dxo + (int64_t)i * dx * C;
    memset(out, 0, sizeof(double) * dx * C);
    int a = rows[i];
    if (a < 0 || a >= n_nodes) continue;
    int s = slot[a];
    double Ye[ORACLE_MAX_DY];
    for (int64_t k = cnt[s]; k < cnt[s + 1]; ++k) {
      int64_t e = lst[k];
      int b = recv[e];
      edge_y(d, pl, e, evec, Yg, Ye);
      const double *we = w + e * P * C;
      const double *dmb = dm + (int64_t)b * dout * C;
      for (int pi = 0; pi < P; ++pi) {
        const opath *p = &pl->p[pi];
        int n1 = 2 * p->l1 + 1, n2 = 2 * p->l2 + 1, nL = 2 * p->L + 1;
        for (int M = 0; M < nL; ++M)
          for (int m1 = 0; m1 < n1; ++m1)
            for (int m2 = 0; m2 < n2; ++m2) {
              double c = p->T[(M * n1 + m1) * n2 + m2];
              if (c == 0.0) continue;
              double cy = c * Ye[p->yoff + m2];
              for (int q = 0; q < C; ++q)
                out[(p->xoff + m1) * C + q] +=
                    we[pi * C + q] * cy * dmb[(p->ooff + M) * C + q];
            }
      }
    }
  }
  free(recv);
  free(slot);
  free(cnt);
  free(lst);
  free(fill);
  plan_free(pl);
  free(pl);
  return bad ? -1 : 0;
}

/* Conv backward, edge cotangents, [e3j] E.1 Eq.16 (second and third lines)
 * with per-path scalars:
 *   dw[e][P][q]   = sum_M z_P[M][q] dm[recv][ooff+M][q],
 *                   z_P[M][q] = sum_{m1,m2} T_P[M][m1][m2] x[sender][xoff+m1][q] Y_e[yoff+m2]
 *   dY[e][yoff+m2] = sum_q sum_{P on that y irrep} w[e][P][q]
 *                   sum_{M,m1} T_P[M][m1][m2] x[sender][xoff+m1][q] dm[recv][ooff+M][q]
 * for edges rows[0..nrows-1]; dw is [nrows][P][C], dY is [nrows][dy].
 * Padding edges get dw = 0 and dY = 0. */
int oracle_conv_backward_edge(const oracle_desc *d, int n_nodes, int64_t n_edges,
                              const int *rowptr, const int *sender, const double *evec,
                              const double *Yg, const double *x, const double *w,
                              const double *dm, int nrows, const int64_t *rows, double *dw,
                              double *dY) {
  oplan *pl = malloc(sizeof(oplan));
  if (plan_build(d, pl) != 0 || check_y(d, Yg) != 0) {
    plan_free(pl);
    free(pl);
    return -1;
  }
  const int C = d->C, P = pl->np, dx = pl->dx, dy = pl->dy, dout = pl->dout;
  int *recv = edge_receivers(n_nodes, n_edges, rowptr);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int i = 0; i < nrows; ++i) {
    double *dwe = dw + (int64_t)i * P * C;
    double *dYe = dY + (int64_t)i * dy;
    memset(dwe, 0, sizeof(double) * P * C);
    memset(dYe, 0, sizeof(double) * dy);
    int64_t e = rows[i];
    if (e < 0 || e >= n_edges) {
      bad = 1;
      continue;
    }
    int a = sender[e];
    if (a < 0) continue;
    int b = recv[e];
    double Ye[ORACLE_MAX_DY];
    edge_y(d, pl, e, evec, Yg, Ye);
    const double *xa = x + (int64_t)a * dx * C;
    const double *we = w + e * P * C;
    const double *dmb = dm + (int64_t)b * dout * C;
    for (int pi = 0; pi < P; ++pi) {
      const opath *p = &pl->p[pi];
      int n1 = 2 * p->l1 + 1, n2 = 2 * p->l2 + 1, nL = 2 * p->L + 1;
      for (int M = 0; M < nL; ++M)
        for (int m1 = 0; m1 < n1; ++m1)
          for (int m2 = 0; m2 < n2; ++m2) {
            double c = p->T[(M * n1 + m1) * n2 + m2];
            if (c == 0.0) continue;
            for (int q = 0; q < C; ++q) {
              double xd = xa[(p->xoff + m1) * C + q] * dmb[(p->ooff + M) * C + q];
              dwe[pi * C + q] += c * Ye[p->yoff + m2] * xd;
              dYe[p->yoff + m2] += c * we[pi * C + q] * xd;
            }
          }
    }
  }
  free(recv);
  plan_free(pl);
  free(pl);
  return bad ? -1 : 0;
}

/* Harmonics of n vectors r[n][3] -> out[n][(lmax+1)^2]. */
int oracle_sh_batch(int lmax, int64_t n, const double *r, double *out) {
  if (lmax < 0 || lmax > ORACLE_MAX_L) return -1;
  const int d = (lmax + 1) * (lmax + 1);
  for (int64_t i = 0; i < n; ++i) oracle_sh(lmax, r + 3 * i, out + i * d);
  return 0;
}

/* Batched TP backward, the VJP of oracle_tp_forward ([e3j] E.1 Eq.14-15:
 * each cotangent is the tensor product with the coefficient records
 * permuted, here with the per-path scalars of Eq.11):
 *   dx[r][xoff+m1][q] = sum_P w[r][P][q] sum_{M,m2} T_P[M][m1][m2] y[r][yoff+m2] dz[r][ooff+M][q]
 *   dw[r][P][q]       = sum_M (sum_{m1,m2} T_P[M][m1][m2] x[r][xoff+m1][q] y[r][yoff+m2]) dz[r][ooff+M][q]
 *   dy[r][yoff+m2]    = sum_q sum_P w[r][P][q] sum_{M,m1} T_P[M][m1][m2] x[r][xoff+m1][q] dz[r][ooff+M][q]
 * for rows[0..nrows-1]; dx [nrows][dx][C], dw [nrows][P][C], dy [nrows][dy]. */
int oracle_tp_backward(const oracle_desc *d, int64_t n_rows, const double *x, const double *y,
                       const double *w, const double *dz, int nrows, const int64_t *rows,
                       double *dxo, double *dwo, double *dyo) {
  oplan *pl = malloc(sizeof(oplan));
  if (plan_build(d, pl) != 0) {
    plan_free(pl);
    free(pl);
    return -1;
  }
  const int C = d->C, P = pl->np, dx = pl->dx, dy = pl->dy, dout = pl->dout;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16)
  for (int i = 0; i < nrows; ++i) {
    double *dxr = dxo + (int64_t)i * dx * C, *dwr = dwo + (int64_t)i * P * C;
    double *dyr = dyo + (int64_t)i * dy;
    memset(dxr, 0, sizeof(double) * dx * C);
    memset(dwr, 0, sizeof(double) * P * C);
    memset(dyr, 0, sizeof(double) * dy);
    int64_t r = rows[i];
    if (r < 0 || r >= n_rows) {
      bad = 1;
      continue;
    }
    const double *xr = x + r * dx * C, *yr = y + r * dy, *wr = w + r * P * C;
    const double *dzr = dz + r * dout * C;
    for (int pi = 0; pi < P; ++pi) {
      const opath *p = &pl->p[pi];
      int n1 = 2 * p->l1 + 1, n2 = 2 * p->l2 + 1, nL = 2 * p->L + 1;
      for (int M = 0; M < nL; ++M)
        for (int m1 = 0; m1 < n1; ++m1)
          for (int m2 = 0; m2 < n2; ++m2) {
            double c = p->T[(M * n1 + m1) * n2 + m2];
            if (c == 0.0) continue;
            for (int q = 0; q < C; ++q) {
              double g = dzr[(p->ooff + M) * C + q];
              double xv = xr[(p->xoff + m1) * C + q], yv = yr[p->yoff + m2];
              dxr[(p->xoff + m1) * C + q] += wr[pi * C + q] * c * yv * g;
              dwr[pi * C + q] += c * xv * yv * g;
              dyr[p->yoff + m2] += wr[pi * C + q] * c * xv * g;
            }
          }
    }
  }
  plan_free(pl);
  free(pl);
  return bad ? -1 : 0;
}

/* Gradient of the harmonics with respect to the (unnormalised) vector:
 * out[k] = sum_m dY[m] dY_lm/dr_k for l = 0..lmax, i.e. J^T dY with
 * J = dY/dr.  Written from the closed forms of oracle_sh_l: with
 * u = r/|r| the harmonics are polynomials P(u), and
 * dP/dr = (I - u u^T) grad_u P / |r|.  A zero vector gives 0. */
#define ORACLE_MAX_L_GRAD 3 /* the closed-form partials below */
int oracle_sh_grad(int lmax, const double r[3], const double *dY, double out[3]) {
  if (lmax < 0 || lmax > ORACLE_MAX_L_GRAD) return -1;
  out[0] = out[1] = out[2] = 0.0;
  double n = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  if (n == 0.0) return 0;
  double x = r[0] / n, y = r[1] / n, z = r[2] / n;
  double g[3] = {0, 0, 0}; /* sum_m dY[m] grad_u P_lm(u) */
  int o = 0;
  for (int l = 0; l <= lmax; ++l) {
    const double *w = dY + o;
    /* partial derivatives of each component polynomial, (d/dx, d/dy, d/dz) */
    double d[7][3];
    int nm = 2 * l + 1;
    switch (l) {
      case 0:
        d[0][0] = d[0][1] = d[0][2] = 0.0;
        break;
      case 1: {
        double s3 = sqrt(3.0);
        double t[3][3] = {{0, s3, 0}, {0, 0, s3}, {s3, 0, 0}}; /* y, z, x */
        memcpy(d, t, sizeof(t));
        break;
      }
      case 2: {
        double s15 = sqrt(15.0), s5 = sqrt(5.0);
        double t[5][3] = {{s15 * y, s15 * x, 0},
                          {0, s15 * z, s15 * y},
                          {-s5 * x, -s5 * y, 2 * s5 * z},
                          {s15 * z, 0, s15 * x},
                          {s15 * x, -s15 * y, 0}};
        memcpy(d, t, sizeof(t));
        break;
      }
      case 3: {
        double a = sqrt(35.0 / 8.0), b = sqrt(105.0), c = sqrt(21.0 / 8.0), e = sqrt(7.0);
        double q = 4 * z * z - x * x - y * y;
        double t[7][3] = {
            {a * 6 * x * y, a * (3 * x * x - 3 * y * y), 0},
            {b * y * z, b * x * z, b * x * y},
            {c * y * (-2 * x), c * (q - 2 * y * y), c * y * 8 * z},
            {0.5 * e * z * (-6 * x), 0.5 * e * z * (-6 * y), 0.5 * e * (6 * z * z - 3 * x * x - 3 * y * y)},
            {c * (q - 2 * x * x), c * x * (-2 * y), c * x * 8 * z},
            {0.5 * b * 2 * x * z, -0.5 * b * 2 * y * z, 0.5 * b * (x * x - y * y)},
            {a * (3 * x * x - 3 * y * y), a * (-6 * x * y), 0}};
        memcpy(d, t, sizeof(t));
        break;
      }
    }
    for (int m = 0; m < nm; ++m)
      for (int k = 0; k < 3; ++k) g[k] += w[m] * d[m][k];
    o += nm;
  }
  /* project out the radial part and scale by 1/|r| */
  double u[3] = {x, y, z};
  double ug = u[0] * g[0] + u[1] * g[1] + u[2] * g[2];
  for (int k = 0; k < 3; ++k) out[k] = (g[k] - u[k] * ug) / n;
  return 0;
}

int oracle_sh_grad_batch(int lmax, int64_t n, const double *r, const double *dY, double *out) {
  if (lmax < 0 || lmax > ORACLE_MAX_L_GRAD) return -1;
  const int d = (lmax + 1) * (lmax + 1);
  for (int64_t i = 0; i < n; ++i) oracle_sh_grad(lmax, r + 3 * i, dY + i * d, out + 3 * i);
  return 0;
}

/* Position gradient from edge-vector gradients.  With r_e = pos[recv(e)] -
 * pos[sender(e)], a scalar E that depends on the positions only through the
 * r_e has dE/dpos[b] = sum_{e: recv(e)=b} g_e - sum_{e: sender(e)=b} g_e,
 * g_e = dE/dr_e; the force is F_b = -dE/dpos[b] ([Tessera] 2.2 Eq.3).
 * Padding edges (sender outside [0,N)) are skipped.
 * dpos [N][3]. */
int oracle_edge_grad_to_nodes(int n_nodes, int64_t n_edges, const int *rowptr, const int *sender,
                              const double *g, double *dpos) {
  if (n_nodes < 0 || n_edges < 0 || rowptr[0] != 0 || rowptr[n_nodes] != n_edges) return -1;
  memset(dpos, 0, sizeof(double) * 3 * (size_t)n_nodes);
  for (int b = 0; b < n_nodes; ++b)
    for (int e = rowptr[b]; e < rowptr[b + 1]; ++e) {
      int a = sender[e];
      if (a < 0 || a >= n_nodes) continue;
      for (int k = 0; k < 3; ++k) {
        dpos[3 * b + k] += g[3 * e + k];
        dpos[3 * a + k] -= g[3 * e + k];
      }
    }
  return 0;
}

/* Equivariant channel mixing within each irrep ([e3j] A.3 Eq.5).  The
 * equivariant choice of the mixing tensor is W^{km}_{k'm'} = W^{k}_{k'}
 * delta_{mm'} for every pair of blocks of equal (l, parity) (a map between
 * blocks of different type cannot commute with all rotations and the
 * inversion); so
 *   y[r][o, m][k] = sum over input blocks i with (l_i, p_i) = (l_o, p_o) of
 *                   sum_{k'} x[r][i, m][k'] W_io[k'][k],
 * with x [rows][dx][Cin], y [rows][dy][Cout], and W holding, for every such
 * (i, o) pair in i-major then o order, a row-major Cin x Cout matrix.
 * Output blocks without a matching input block are zero.  Returns the
 * number of weight matrices (>= 0), or -1 on bad arguments; when y is NULL
 * only the count is computed. */
int oracle_linear(int nin, const int *in_l, const int *in_p, int cin, int nout, const int *out_l,
                  const int *out_p, int cout, int64_t n_rows, const double *x, const double *W,
                  double *y) {
  if (nin < 0 || nout < 0 || cin < 1 || cout < 1 || n_rows < 0) return -1;
  int din = 0, dout = 0, inoff[ORACLE_MAX_IRREPS], outoff[ORACLE_MAX_IRREPS];
  if (nin > ORACLE_MAX_IRREPS || nout > ORACLE_MAX_IRREPS) return -1;
  for (int i = 0; i < nin; ++i) {
    inoff[i] = din;
    din += 2 * in_l[i] + 1;
  }
  for (int o = 0; o < nout; ++o) {
    outoff[o] = dout;
    dout += 2 * out_l[o] + 1;
  }
  /* pair index of (i, o), -1 when the types differ */
  int pair[ORACLE_MAX_IRREPS][ORACLE_MAX_IRREPS], np = 0;
  for (int i = 0; i < nin; ++i)
    for (int o = 0; o < nout; ++o)
      pair[i][o] = (in_l[i] == out_l[o] && in_p[i] == out_p[o]) ? np++ : -1;
  if (!y) return np;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double *yr = y + r * dout * cout;
    const double *xr = x + r * din * cin;
    memset(yr, 0, sizeof(double) * dout * cout);
    for (int o = 0; o < nout; ++o)
      for (int i = 0; i < nin; ++i) {
        if (pair[i][o] < 0) continue;
        const double *Wio = W + (int64_t)pair[i][o] * cin * cout;
        for (int m = 0; m < 2 * out_l[o] + 1; ++m)
          for (int k = 0; k < cout; ++k) {
            double s = 0.0;
            for (int kp = 0; kp < cin; ++kp) s += xr[(inoff[i] + m) * cin + kp] * Wio[kp * cout + k];
            yr[(outoff[o] + m) * cout + k] += s;
          }
      }
  }
  return np;
}

/* VJP of oracle_linear for the cotangent dy [rows][dout][Cout]:
 *   dx[r][i, m][k'] = sum over output blocks o of the type of i of
 *                     sum_k dy[r][o, m][k] W_io[k'][k]
 *   dW_io[k'][k]    = sum_r sum_m x[r][i, m][k'] dy[r][o, m][k]
 * (dx [rows][din][Cin], dW like W).  Returns the pair count or -1. */
int oracle_linear_backward(int nin, const int *in_l, const int *in_p, int cin, int nout,
                           const int *out_l, const int *out_p, int cout, int64_t n_rows,
                           const double *x, const double *W, const double *dy, double *dx,
                           double *dW) {
  if (nin < 0 || nout < 0 || cin < 1 || cout < 1 || n_rows < 0) return -1;
  if (nin > ORACLE_MAX_IRREPS || nout > ORACLE_MAX_IRREPS) return -1;
  int din = 0, dout = 0, inoff[ORACLE_MAX_IRREPS], outoff[ORACLE_MAX_IRREPS];
  for (int i = 0; i < nin; ++i) {
    inoff[i] = din;
    din += 2 * in_l[i] + 1;
  }
  for (int o = 0; o < nout; ++o) {
    outoff[o] = dout;
    dout += 2 * out_l[o] + 1;
  }
  int pair[ORACLE_MAX_IRREPS][ORACLE_MAX_IRREPS], np = 0;
  for (int i = 0; i < nin; ++i)
    for (int o = 0; o < nout; ++o)
      pair[i][o] = (in_l[i] == out_l[o] && in_p[i] == out_p[o]) ? np++ : -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    double *dxr = dx + r * din * cin;
    const double *dyr = dy + r * dout * cout;
    memset(dxr, 0, sizeof(double) * din * cin);
    for (int i = 0; i < nin; ++i)
      for (int o = 0; o < nout; ++o) {
        if (pair[i][o] < 0) continue;
        const double *Wio = W + (int64_t)pair[i][o] * cin * cout;
        for (int m = 0; m < 2 * in_l[i] + 1; ++m)
          for (int kp = 0; kp < cin; ++kp) {
            double s = 0.0;
            for (int k = 0; k < cout; ++k) s += dyr[(outoff[o] + m) * cout + k] * Wio[kp * cout + k];
            dxr[(inoff[i] + m) * cin + kp] += s;
          }
      }
  }
  /* dW: one pair and one weight entry per task, rows summed in order */
  for (int i = 0; i < nin; ++i)
    for (int o = 0; o < nout; ++o) {
      if (pair[i][o] < 0) continue;
      double *dWio = dW + (int64_t)pair[i][o] * cin * cout;
#pragma omp parallel for schedule(static)
      for (int kp = 0; kp < cin; ++kp)
        for (int k = 0; k < cout; ++k) {
          double s = 0.0;
          for (int64_t r = 0; r < n_rows; ++r)
            for (int m = 0; m < 2 * in_l[i] + 1; ++m)
              s += x[(r * din + inoff[i] + m) * cin + kp] * dy[(r * dout + outoff[o] + m) * cout + k];
          dWio[kp * cout + k] = s;
        }
    }
  return np;
}

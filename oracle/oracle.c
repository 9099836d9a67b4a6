/*
 * oracle.c -- plain, slow, fp64 CPU reference of the fast-multipole gravity
 * evaluation.  TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and
 * the CPU-baseline leg of the benchmark; never by the product library, with
 * which it shares no code, header or table.
 *
 * It follows the jz-fmm project page step by step:
 *   - direct sum with the self term omitted ("From particle pairs to node
 *     pairs", the equation for Phi(x_i));
 *   - Cartesian mass moments about the cell centre ("Describing the source and
 *     the receiving region", the moment equations M, M^(1), M^(2), "higher
 *     moments follow the same pattern");
 *   - the local Taylor polynomial about the receiving centre and a = -grad Phi
 *     (same section, the Taylor equation);
 *   - the multipole-to-local translation from the moments and R = c_A - c_B
 *     ("Calculating a node-node interaction", the two closed forms);
 *   - the opening criterion theta = |l_A + l_B| / |c_A - c_B|, open iff
 *     theta >= theta_max (same section, the criterion equation);
 *   - upward pass, interaction stage, downward pass ("Combining near and far
 *     interactions");
 *   - the reversible integer-lattice kick-drift-kick step ("Why
 *     reversibility matters");
 *   - the vector-Jacobian product of the force calculation ("Following
 *     sensitivities backwards"): exactly, by the chain rule, for the direct
 *     sum, and in the page's fast multipole form (the next higher derivative
 *     of the original evaluation plus an FMM whose sources are the
 *     sensitivities as monopoles and dipoles).
 *
 * Readings taken where the page is silent (each repeated at its code):
 *   R1  "order p": every expansion keeps total degree <= p; the translation
 *       keeps |n| + |m| <= p (the widget keeps "terms through total degree p").
 *   R2  expansion centre = geometric centre of the octree cell.
 *   R3  half-widths l = (h, h, h), h = half the cell side.
 *   R4  root cube anchored at the per-axis minimum, side = smallest power of two
 *       >= the largest extent (1 if all extents are 0).
 *   R5  21 bits per axis, x the most significant bit of each triple, upper edge
 *       clamped.   R6  key arithmetic in fp64, no fused multiply-add.
 *   R7  stable sort (equal keys keep input order).
 *   R8  a node is a leaf iff count <= leaf_size or its level is 21.
 *   R9  nodes numbered breadth first (level, then key prefix); empty octants
 *       have no node.
 *   R10 walk: accept -> M2L; two leaves -> P2P; otherwise split the coarser
 *       non-leaf, both if the levels are equal (a node paired with itself is
 *       split into all ordered child pairs).
 *   R11 the criterion is evaluated in integer cell units: accept iff
 *       3 (hA + hB)^2 < fl(theta*theta) * |cA - cB|^2, so ties are opened.
 *   R12 lists are directed and sorted by (target, source).
 *   R13 the self term is omitted by index.
 *
 * The build flags must not contract a*b+c into one rounding (-ffp-contract=off)
 * so that the key and criterion arithmetic stays bit-exact.
 */
#include "oracle.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MAXP 10
#define MAXK 286 /* C(13,3) */
#define KEYBITS 21

static double wall(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* multi-index bookkeeping                                             */
/* ------------------------------------------------------------------ */
typedef struct {
  int p, K;
  int e[MAXK][3];
  int idx[MAXP + 1][MAXP + 1][MAXP + 1]; /* -1 beyond degree p */
} mtab;

static void mtab_init(mtab* t, int p) {
  int k = 0;
  t->p = p;
  memset(t->idx, 0xff, sizeof(t->idx));
  for (int d = 0; d <= p; d++)
    for (int a = d; a >= 0; a--)
      for (int b = d - a; b >= 0; b--) {
        int c = d - a - b;
        t->e[k][0] = a;
        t->e[k][1] = b;
        t->e[k][2] = c;
        t->idx[a][b][c] = k;
        k++;
      }
  t->K = k;
}

int oracle_ncoef(int order) {
  if (order < 0 || order > MAXP) return -1;
  return (order + 1) * (order + 2) * (order + 3) / 6;
}

static double fact(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; i++) f *= (double)i;
  return f;
}

static double dfact_odd(int q) { /* (2q-1)!!, with (-1)!! = 1 */
  double f = 1.0;
  for (int i = 2 * q - 1; i > 1; i -= 2) f *= (double)i;
  return f;
}

static double ipow(double x, int n) {
  double r = 1.0;
  for (int i = 0; i < n; i++) r *= x;
  return r;
}

static double binom(int n, int k) { return fact(n) / (fact(k) * fact(n - k)); }

/* ------------------------------------------------------------------ */
/* single operators                                                    */
/* ------------------------------------------------------------------ */

/* Moments of a particle set about centre c (moment equations of the jz-fmm
 * page: M = sum m, M1 = sum m s, M2_ab = sum m s_a s_b, higher ones alike). */
static void p2m_set(const mtab* t, int64_t n, const double* pos, const double* mass,
                    const double* c, double* M) {
  for (int64_t j = 0; j < n; j++) {
    double s[3] = {pos[3 * j] - c[0], pos[3 * j + 1] - c[1], pos[3 * j + 2] - c[2]};
    for (int k = 0; k < t->K; k++)
      M[k] += mass[j] * ipow(s[0], t->e[k][0]) * ipow(s[1], t->e[k][1]) *
              ipow(s[2], t->e[k][2]);
  }
}

/* Moments about a parent centre from moments about a child centre, d = c_child
 * - c_parent: (s + d)^m = sum_{k<=m} C(m,k) s^k d^(m-k), per axis. */
static void m2m_one(const mtab* t, const double* Mc, const double* d, double* Mp) {
  for (int i = 0; i < t->K; i++) {
    const int* m = t->e[i];
    double acc = 0.0;
    for (int ka = 0; ka <= m[0]; ka++)
      for (int kb = 0; kb <= m[1]; kb++)
        for (int kc = 0; kc <= m[2]; kc++) {
          int k = t->idx[ka][kb][kc];
          acc += binom(m[0], ka) * binom(m[1], kb) * binom(m[2], kc) *
                 ipow(d[0], m[0] - ka) * ipow(d[1], m[1] - kb) * ipow(d[2], m[2] - kc) * Mc[k];
        }
    Mp[i] += acc;
  }
}

/* Derivatives of 1/|r| up to total degree p, from the closed form
 *   d^a_x d^b_y d^c_z f(u), u = |r|^2/2, f(u) = (2u)^(-1/2):
 *   sum_{i,j,l} H(a,i) H(b,j) H(c,l) x^(a-2i) y^(b-2j) z^(c-2l) f^(a+b+c-i-j-l)(u),
 *   H(a,i) = a! / (2^i i! (a-2i)!),  f^(q)(u) = (-1)^q (2q-1)!! / |r|^(2q+1).
 * (Each axis contributes a Hermite-polynomial factor because u is a sum of
 * per-axis squares.) */
static void dtensor(const mtab* t, const double* r, double* D) {
  double r2 = r[0] * r[0] + r[1] * r[1] + r[2] * r[2];
  double rn = sqrt(r2);
  double g[2 * MAXP + 2];
  for (int q = 0; q <= t->p; q++) {
    double sgn = (q % 2) ? -1.0 : 1.0;
    g[q] = sgn * dfact_odd(q) / ipow(rn, 2 * q + 1);
  }
  for (int k = 0; k < t->K; k++) {
    int a = t->e[k][0], b = t->e[k][1], c = t->e[k][2];
    double acc = 0.0;
    for (int i = 0; 2 * i <= a; i++)
      for (int j = 0; 2 * j <= b; j++)
        for (int l = 0; 2 * l <= c; l++) {
          double h = fact(a) / (ipow(2.0, i) * fact(i) * fact(a - 2 * i)) * fact(b) /
                     (ipow(2.0, j) * fact(j) * fact(b - 2 * j)) * fact(c) /
                     (ipow(2.0, l) * fact(l) * fact(c - 2 * l));
          acc += h * ipow(r[0], a - 2 * i) * ipow(r[1], b - 2 * j) * ipow(r[2], c - 2 * l) *
                 g[a + b + c - i - j - l];
        }
    D[k] = acc;
  }
}

/* Multipole-to-local, G = 1.  Taylor-expanding -m_j / |R + dx - s_j| in dx and
 * s_j gives L_n = -sum_m (-1)^|m| / m! M_m D^(n+m)(R); reading R1 keeps
 * |n| + |m| <= p.  For M, M1 only this reduces to the two closed forms on the
 * jz-fmm page. */
static void m2l_one(const mtab* t, const double* M, const double* R, double* L) {
  double D[MAXK];
  dtensor(t, R, D);
  for (int i = 0; i < t->K; i++) {
    const int* n = t->e[i];
    int dn = n[0] + n[1] + n[2];
    double acc = 0.0;
    for (int j = 0; j < t->K; j++) {
      const int* m = t->e[j];
      int dm = m[0] + m[1] + m[2];
      if (dn + dm > t->p) continue;
      double sgn = (dm % 2) ? -1.0 : 1.0;
      int k = t->idx[n[0] + m[0]][n[1] + m[1]][n[2] + m[2]];
      acc += sgn / (fact(m[0]) * fact(m[1]) * fact(m[2])) * M[j] * D[k];
    }
    L[i] -= acc;
  }
}

/* Local-to-local: re-centre the Taylor polynomial, d = c_child - c_parent:
 * L_n(child) = sum_{|n|+|k|<=p} L_(n+k)(parent) d^k / k!. */
static void l2l_one(const mtab* t, const double* Lp, const double* d, double* Lc) {
  for (int i = 0; i < t->K; i++) {
    const int* n = t->e[i];
    int dn = n[0] + n[1] + n[2];
    double acc = 0.0;
    for (int j = 0; j < t->K; j++) {
      const int* k = t->e[j];
      int dk = k[0] + k[1] + k[2];
      if (dn + dk > t->p) continue;
      int nk = t->idx[n[0] + k[0]][n[1] + k[1]][n[2] + k[2]];
      acc += Lp[nk] * ipow(d[0], k[0]) * ipow(d[1], k[1]) * ipow(d[2], k[2]) /
             (fact(k[0]) * fact(k[1]) * fact(k[2]));
    }
    Lc[i] += acc;
  }
}

/* Local evaluation: Phi = sum_n L_n dx^n / n!, a = -grad Phi (Taylor equation of
 * the jz-fmm page and "Differentiating this polynomial gives the acceleration"). */
static void l2p_one(const mtab* t, const double* L, const double* dx, double* phi,
                    double* acc) {
  double p = 0.0, a[3] = {0.0, 0.0, 0.0};
  for (int i = 0; i < t->K; i++) {
    const int* n = t->e[i];
    double nf = fact(n[0]) * fact(n[1]) * fact(n[2]);
    p += L[i] * ipow(dx[0], n[0]) * ipow(dx[1], n[1]) * ipow(dx[2], n[2]) / nf;
    for (int al = 0; al < 3; al++) {
      if (n[al] == 0) continue;
      int e[3] = {n[0], n[1], n[2]};
      e[al] -= 1;
      a[al] -= L[i] * ipow(dx[0], e[0]) * ipow(dx[1], e[1]) * ipow(dx[2], e[2]) /
               (fact(e[0]) * fact(e[1]) * fact(e[2]));
    }
  }
  *phi += p;
  acc[0] += a[0];
  acc[1] += a[1];
  acc[2] += a[2];
}

/* Moments of monopoles q_j and point dipoles d_j about c.  A point dipole d
 * at x has the potential d . grad_y G(y - x), G = -1/|r| (the field of a
 * monopole, differentiated with respect to its position and negated), so with
 * s = x - c its raw moments are the negated derivative of s^m along d:
 *   M_m += q s^m - sum_a d_a m_a s^(m - e_a).
 * These are the sources of the FMM inside the VJP (jz-fmm page, "Following
 * sensitivities backwards": the force sensitivities act as dipole moments). */
static void p2m_dip_set(const mtab* t, int64_t n, const double* pos, const double* q,
                        const double* dip, const double* c, double* M) {
  for (int64_t j = 0; j < n; j++) {
    double s[3] = {pos[3 * j] - c[0], pos[3 * j + 1] - c[1], pos[3 * j + 2] - c[2]};
    for (int k = 0; k < t->K; k++) {
      const int* m = t->e[k];
      double v = q[j] * ipow(s[0], m[0]) * ipow(s[1], m[1]) * ipow(s[2], m[2]);
      for (int a = 0; a < 3; a++) {
        if (m[a] == 0) continue;
        int e[3] = {m[0], m[1], m[2]};
        e[a] -= 1;
        v -= dip[3 * j + a] * (double)m[a] * ipow(s[0], e[0]) * ipow(s[1], e[1]) *
             ipow(s[2], e[2]);
      }
      M[k] += v;
    }
  }
}

/* Second derivatives of the local Taylor polynomial at offset dx (the "next
 * higher derivative" of the original evaluation that the VJP needs):
 *   H_ab = sum_n L_(n + e_a + e_b) dx^n / n!,   order xx, yy, zz, xy, xz, yz. */
static void l2p_hess_one(const mtab* t, const double* L, const double* dx, double* H6) {
  static const int pa[6] = {0, 1, 2, 0, 0, 1}, pb[6] = {0, 1, 2, 1, 2, 2};
  for (int i = 0; i < t->K; i++) {
    const int* n = t->e[i];
    if (n[0] + n[1] + n[2] + 2 > t->p) continue;
    double w = ipow(dx[0], n[0]) * ipow(dx[1], n[1]) * ipow(dx[2], n[2]) /
               (fact(n[0]) * fact(n[1]) * fact(n[2]));
    for (int h = 0; h < 6; h++) {
      int e[3] = {n[0], n[1], n[2]};
      e[pa[h]] += 1;
      e[pb[h]] += 1;
      H6[h] += L[t->idx[e[0]][e[1]][e[2]]] * w;
    }
  }
}

int oracle_p2m_dipole(int order, int64_t n, const double* pos, const double* q,
                      const double* dip, const double* centre, double* mpole) {
  if (order < 0 || order > MAXP || n < 0) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  memset(mpole, 0, sizeof(double) * (size_t)t.K);
  p2m_dip_set(&t, n, pos, q, dip, centre, mpole);
  return ORACLE_OK;
}
int oracle_l2p_hessian(int order, const double* L, const double* dx, double* H6) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  for (int h = 0; h < 6; h++) H6[h] = 0.0;
  l2p_hess_one(&t, L, dx, H6);
  return ORACLE_OK;
}
int oracle_p2m(int order, int64_t n, const double* pos, const double* mass,
               const double* centre, double* mpole) {
  if (order < 0 || order > MAXP || n < 0) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  memset(mpole, 0, sizeof(double) * (size_t)t.K);
  p2m_set(&t, n, pos, mass, centre, mpole);
  return ORACLE_OK;
}
int oracle_m2m(int order, const double* mc, const double* d, double* mp) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  m2m_one(&t, mc, d, mp);
  return ORACLE_OK;
}
int oracle_dtensor(int order, const double* r, double* D) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  dtensor(&t, r, D);
  return ORACLE_OK;
}
int oracle_m2l(int order, const double* M, const double* r, double* L) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  m2l_one(&t, M, r, L);
  return ORACLE_OK;
}
int oracle_l2l(int order, const double* Lp, const double* d, double* Lc) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  l2l_one(&t, Lp, d, Lc);
  return ORACLE_OK;
}
int oracle_l2p(int order, const double* L, const double* dx, double* phi, double* acc) {
  if (order < 0 || order > MAXP) return ORACLE_ERR_ARG;
  mtab t;
  mtab_init(&t, order);
  l2p_one(&t, L, dx, phi, acc);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* direct sum                                                          */
/* ------------------------------------------------------------------ */
int oracle_direct(int64_t n, const double* pos, const double* mass, int64_t nt,
                  const int64_t* tg, double* phi, double* acc) {
  if (n < 0 || nt < 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t q = 0; q < nt; q++) {
    int64_t i = tg[q];
    double p = 0.0, a0 = 0.0, a1 = 0.0, a2 = 0.0;
    for (int64_t j = 0; j < n; j++) {
      if (j == i) continue; /* self term omitted */
      double dx = pos[3 * i] - pos[3 * j], dy = pos[3 * i + 1] - pos[3 * j + 1],
             dz = pos[3 * i + 2] - pos[3 * j + 2];
      double r = sqrt(dx * dx + dy * dy + dz * dz);
      double r3 = r * r * r;
      p -= mass[j] / r;
      a0 -= mass[j] * dx / r3;
      a1 -= mass[j] * dy / r3;
      a2 -= mass[j] * dz / r3;
    }
    phi[q] = p;
    acc[3 * q] = a0;
    acc[3 * q + 1] = a1;
    acc[3 * q + 2] = a2;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* vector-Jacobian product, direct sum                                 */
/* ------------------------------------------------------------------ */
/* The VJP carries the sensitivities pb_i = dS/dphi_i and ab_i = dS/da_i of a
 * scalar S back to the positions and masses ("Following sensitivities
 * backwards" on the jz-fmm page).  Here it is the exact gradient of
 * S = sum_i pb_i phi_i + ab_i . a_i for the direct sum, by the plain chain
 * rule over ordered pairs.  With r = x_i - x_j and f(r) = -1/|r|:
 *   grad f = r/|r|^3,   Hess f = I/|r|^3 - 3 r r^T/|r|^5,
 *   phi_i = sum_j m_j f(r),   a_i = -sum_j m_j grad f(r),
 * so pair (i, j) adds  l_ij = m_j (pb_i f(r) - ab_i . grad f(r))  to S, and
 *   dl_ij/dm_j = pb_i f - ab_i . grad f,
 *   dl_ij/dr   = m_j (pb_i grad f - Hess f ab_i),
 * which goes to x_i with a plus and to x_j with a minus sign.  Each particle
 * gathers the terms of the pairs it is part of, so the loop runs over i
 * without shared writes. */
static void pair_vjp_grad(const double* r, double mj, double pbi, const double* abi,
                          double* g) { /* g = dl_ij/dr */
  double rr = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  double r3 = rr * rr * rr, r5 = r3 * rr * rr;
  double ra = r[0] * abi[0] + r[1] * abi[1] + r[2] * abi[2];
  for (int a = 0; a < 3; a++) {
    double gradf = r[a] / r3;
    double hab = abi[a] / r3 - 3.0 * r[a] * ra / r5; /* (Hess f) ab */
    g[a] = mj * (pbi * gradf - hab);
  }
}
static double pair_vjp_mass(const double* r, double pbi, const double* abi) {
  double rr = sqrt(r[0] * r[0] + r[1] * r[1] + r[2] * r[2]);
  double r3 = rr * rr * rr;
  double f = -1.0 / rr;
  double ag = (r[0] * abi[0] + r[1] * abi[1] + r[2] * abi[2]) / r3; /* ab . grad f */
  return pbi * f - ag;
}

int oracle_direct_vjp(int64_t n, const double* pos, const double* mass, const double* pb,
                      const double* ab, double* xbar, double* mbar) {
  if (n < 0) return ORACLE_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < n; i++) {
    double gx[3] = {0.0, 0.0, 0.0}, gm = 0.0, g[3];
    for (int64_t j = 0; j < n; j++) {
      if (j == i) continue;
      double r[3] = {pos[3 * i] - pos[3 * j], pos[3 * i + 1] - pos[3 * j + 1],
                     pos[3 * i + 2] - pos[3 * j + 2]};
      /* pair (i, j): i is the target, r = x_i - x_j */
      pair_vjp_grad(r, mass[j], pb[i], ab + 3 * i, g);
      for (int a = 0; a < 3; a++) gx[a] += g[a];
      /* pair (j, i): i is the source, r' = x_j - x_i = -r */
      double rn[3] = {-r[0], -r[1], -r[2]};
      pair_vjp_grad(rn, mass[i], pb[j], ab + 3 * j, g);
      for (int a = 0; a < 3; a++) gx[a] -= g[a];
      gm += pair_vjp_mass(rn, pb[j], ab + 3 * j);
    }
    for (int a = 0; a < 3; a++) xbar[3 * i + a] = gx[a];
    mbar[i] = gm;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* keys                                                                */
/* ------------------------------------------------------------------ */

/* R4: root cube.  R5/R6: keys. */
static void root_cube(int64_t n, const double* pos, double* lo, double* side) {
  double hi[3];
  for (int a = 0; a < 3; a++) lo[a] = hi[a] = pos[a];
  for (int64_t i = 1; i < n; i++)
    for (int a = 0; a < 3; a++) {
      double v = pos[3 * i + a];
      if (v < lo[a]) lo[a] = v;
      if (v > hi[a]) hi[a] = v;
    }
  double ext = 0.0;
  for (int a = 0; a < 3; a++) {
    double e = hi[a] - lo[a];
    if (e > ext) ext = e;
  }
  if (ext == 0.0) {
    *side = 1.0;
    return;
  }
  int ex;
  double f = frexp(ext, &ex); /* ext = f 2^ex, f in [0.5, 1) */
  *side = (f == 0.5) ? ext : ldexp(1.0, ex);
}

static uint64_t interleave(uint32_t ux, uint32_t uy, uint32_t uz) {
  uint64_t key = 0;
  for (int b = 0; b < KEYBITS; b++) {
    key |= (uint64_t)((ux >> b) & 1u) << (3 * b + 2);
    key |= (uint64_t)((uy >> b) & 1u) << (3 * b + 1);
    key |= (uint64_t)((uz >> b) & 1u) << (3 * b);
  }
  return key;
}

static void keys_of(int64_t n, const double* pos, const double* lo, double side,
                    uint64_t* keys) {
  int e;
  frexp(side, &e);                           /* side = 2^(e-1) */
  double scale = ldexp(1.0, KEYBITS - (e - 1)); /* 2^21 / side, exact */
  const double umax = (double)((1u << KEYBITS) - 1u);
  for (int64_t i = 0; i < n; i++) {
    uint32_t u[3];
    for (int a = 0; a < 3; a++) {
      double s = pos[3 * i + a] - lo[a]; /* one rounding */
      double v = floor(s * scale);        /* exact power-of-two scale */
      if (v < 0.0) v = 0.0;
      if (v > umax) v = umax;
      u[a] = (uint32_t)v;
    }
    keys[i] = interleave(u[0], u[1], u[2]);
  }
}

int oracle_morton(int64_t n, const double* pos, double* lo, double* side, uint64_t* keys) {
  if (n < 1) return ORACLE_ERR_ARG;
  root_cube(n, pos, lo, side);
  keys_of(n, pos, lo, *side, keys);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* result object                                                       */
/* ------------------------------------------------------------------ */
struct oracle_result {
  int64_t n;
  int p, K, leaf;
  double theta;
  double lo[3], side;
  uint64_t* key; /* sorted */
  int32_t* perm; /* perm[k] = input index of sorted particle k */
  double* xs;    /* sorted positions */
  double* ms;    /* sorted masses */
  int64_t n_nodes, n_leaves, n_marked;
  int depth;
  uint8_t* level;
  uint64_t* prefix;
  int32_t *begin, *count, *parent, *first_child;
  uint8_t* n_child;
  uint8_t* mark;
  double* centre;
  int64_t n_m2l, n_p2p;
  int64_t *m2l_off, *p2p_off;
  int32_t *m2l_src, *p2p_src;
  uint64_t *dcnt[2], *dhash[2]; /* digest mode: per-target list digests */
  double *M, *L;
  double *phi, *acc; /* caller's order */
  double times[8];
};

void oracle_free(oracle_result* r) {
  if (!r) return;
  free(r->key);
  free(r->perm);
  free(r->xs);
  free(r->ms);
  free(r->level);
  free(r->prefix);
  free(r->begin);
  free(r->count);
  free(r->parent);
  free(r->first_child);
  free(r->n_child);
  free(r->mark);
  free(r->centre);
  free(r->m2l_off);
  free(r->p2p_off);
  free(r->m2l_src);
  free(r->p2p_src);
  for (int k = 0; k < 2; k++) {
    free(r->dcnt[k]);
    free(r->dhash[k]);
  }
  free(r->M);
  free(r->L);
  free(r->phi);
  free(r->acc);
  free(r);
}

/* ------------------------------------------------------------------ */
/* sort (R7)                                                           */
/* ------------------------------------------------------------------ */
typedef struct {
  uint64_t key;
  int64_t idx;
} kidx;

static int kidx_cmp(const void* a, const void* b) {
  const kidx* x = (const kidx*)a;
  const kidx* y = (const kidx*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  if (x->idx != y->idx) return x->idx < y->idx ? -1 : 1; /* stable */
  return 0;
}

/* ------------------------------------------------------------------ */
/* tree (R8, R9)                                                       */
/* ------------------------------------------------------------------ */
typedef struct {
  int64_t n, cap;
  uint8_t* level;
  uint64_t* prefix;
  int32_t *begin, *count, *parent, *first_child;
  uint8_t* n_child;
} nodevec;

static int nv_push(nodevec* v, int lev, uint64_t pre, int32_t b, int32_t c, int32_t par) {
  if (v->n == v->cap) {
    int64_t nc = v->cap ? 2 * v->cap : 1024;
    void* p;
#define GROW(f, T)                                  \
  p = realloc(v->f, sizeof(T) * (size_t)nc);        \
  if (!p) return -1;                                \
  v->f = (T*)p;
    GROW(level, uint8_t)
    GROW(prefix, uint64_t)
    GROW(begin, int32_t)
    GROW(count, int32_t)
    GROW(parent, int32_t)
    GROW(first_child, int32_t)
    GROW(n_child, uint8_t)
#undef GROW
    v->cap = nc;
  }
  int64_t i = v->n++;
  v->level[i] = (uint8_t)lev;
  v->prefix[i] = pre;
  v->begin[i] = b;
  v->count[i] = c;
  v->parent[i] = par;
  v->first_child[i] = -1;
  v->n_child[i] = 0;
  return 0;
}

static int build_tree(oracle_result* r) {
  nodevec v;
  memset(&v, 0, sizeof(v));
  if (nv_push(&v, 0, 0, 0, (int32_t)r->n, -1)) return ORACLE_ERR_OOM;
  /* Nodes are appended in the order they are split, and each node's children
   * in ascending octant order, so processing ids in order is breadth first. */
  for (int64_t i = 0; i < v.n; i++) {
    int lev = v.level[i];
    if (v.count[i] <= r->leaf || lev == KEYBITS) continue; /* leaf */
    int sh = 3 * (KEYBITS - (lev + 1));
    int32_t b = v.begin[i], e = v.begin[i] + v.count[i];
    int64_t first = v.n;
    int nchild = 0;
    int32_t k = b;
    while (k < e) {
      uint64_t cp = r->key[k] >> sh;
      int32_t k2 = k;
      while (k2 < e && (r->key[k2] >> sh) == cp) k2++;
      if (nv_push(&v, lev + 1, cp, k, k2 - k, (int32_t)i)) return ORACLE_ERR_OOM;
      nchild++;
      k = k2;
    }
    v.first_child[i] = (int32_t)first;
    v.n_child[i] = (uint8_t)nchild;
  }
  r->n_nodes = v.n;
  r->level = v.level;
  r->prefix = v.prefix;
  r->begin = v.begin;
  r->count = v.count;
  r->parent = v.parent;
  r->first_child = v.first_child;
  r->n_child = v.n_child;
  r->n_leaves = 0;
  r->depth = 0;
  for (int64_t i = 0; i < v.n; i++) {
    if (v.n_child[i] == 0) r->n_leaves++;
    if (v.level[i] > r->depth) r->depth = v.level[i];
  }
  /* geometry: integer cell coordinates from the key prefix (R2, R3) */
  r->centre = (double*)malloc(sizeof(double) * 3 * (size_t)v.n);
  if (!r->centre) return ORACLE_ERR_OOM;
  for (int64_t i = 0; i < v.n; i++) {
    int lev = v.level[i];
    uint64_t q[3] = {0, 0, 0};
    for (int b = 0; b < lev; b++) {
      q[0] |= ((v.prefix[i] >> (3 * b + 2)) & 1u) << b;
      q[1] |= ((v.prefix[i] >> (3 * b + 1)) & 1u) << b;
      q[2] |= ((v.prefix[i] >> (3 * b)) & 1u) << b;
    }
    double w = ldexp(r->side, -lev); /* cell side */
    for (int a = 0; a < 3; a++) r->centre[3 * i + a] = r->lo[a] + ((double)q[a] + 0.5) * w;
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* dual tree walk (R10 - R12)                                          */
/* ------------------------------------------------------------------ */
typedef struct {
  int64_t n, cap;
  int32_t* t;
  int32_t* s;
} pairvec;

static int pv_push(pairvec* v, int32_t t, int32_t s) {
  if (v->n == v->cap) {
    int64_t nc = v->cap ? 2 * v->cap : 4096;
    int32_t* a = (int32_t*)realloc(v->t, sizeof(int32_t) * (size_t)nc);
    if (!a) return -1;
    v->t = a;
    a = (int32_t*)realloc(v->s, sizeof(int32_t) * (size_t)nc);
    if (!a) return -1;
    v->s = a;
    v->cap = nc;
  }
  v->t[v->n] = t;
  v->s[v->n] = s;
  v->n++;
  return 0;
}

typedef struct {
  const oracle_result* r;
  double t2;
  pairvec m2l, p2p;
  int err;
  /* digest mode: entries are counted and hashed per target (below) instead of
   * stored; pairs that reach level split_at are set aside in `tasks` and
   * walked afterwards, in parallel (every pair is walked exactly once either
   * way, so the entries emitted are the same) */
  int digest;
  uint64_t *dcnt[2], *dhash[2]; /* [0] M2L, [1] P2P; per target node */
  pairvec* tasks;
  int split_at;
} walkctx;

/* Digest of a list: its entry count and the sum (mod 2^64) of h(s) over its
 * sources s, which does not depend on their order.  h(s) is the (s+1)-th
 * output of SplitMix64 (S. Vigna) seeded with 0: state (s+1) * 0x9e3779b97f4a7c15,
 * then the generator's finalizer. */
static uint64_t digest_h(int32_t s) {
  uint64_t z = ((uint64_t)(uint32_t)s + 1u) * 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

/* kind 0: M2L(A <- B); kind 1: P2P(A <- B) */
static void emit(walkctx* w, int kind, int32_t A, int32_t B) {
  if (w->digest) {
    const uint64_t h = digest_h(B);
    uint64_t* c = w->dcnt[kind] + A;
    uint64_t* d = w->dhash[kind] + A;
#pragma omp atomic
    *c += 1u;
#pragma omp atomic
    *d += h;
    return;
  }
  if (pv_push(kind == 0 ? &w->m2l : &w->p2p, A, B)) w->err = 1;
}

static void cell_coords(const oracle_result* r, int32_t i, int64_t* q) {
  int lev = r->level[i];
  q[0] = q[1] = q[2] = 0;
  for (int b = 0; b < lev; b++) {
    q[0] |= (int64_t)((r->prefix[i] >> (3 * b + 2)) & 1u) << b;
    q[1] |= (int64_t)((r->prefix[i] >> (3 * b + 1)) & 1u) << b;
    q[2] |= (int64_t)((r->prefix[i] >> (3 * b)) & 1u) << b;
  }
}

/* Opening criterion of the jz-fmm page, theta = |l_A + l_B| / |c_A - c_B| with
 * l = (h,h,h) (R3); accept iff theta < theta_max.  Evaluated in units of half
 * the finer cell's side (R11): centres and half-widths are then integers, and
 * the only rounding is the product fl(theta^2) * R^2. */
static int accept(const walkctx* w, int32_t A, int32_t B) {
  const oracle_result* r = w->r;
  int la = r->level[A], lb = r->level[B];
  int lm = la > lb ? la : lb;
  int64_t qa[3], qb[3];
  cell_coords(r, A, qa);
  cell_coords(r, B, qb);
  int64_t ha = (int64_t)1 << (lm - la), hb = (int64_t)1 << (lm - lb);
  int64_t r2 = 0;
  for (int a = 0; a < 3; a++) {
    int64_t ca = ha * (2 * qa[a] + 1), cb = hb * (2 * qb[a] + 1);
    r2 += (ca - cb) * (ca - cb);
  }
  double lhs = 3.0 * (double)((ha + hb) * (ha + hb));
  return lhs < w->t2 * (double)r2;
}

static int is_leaf(const oracle_result* r, int32_t i) { return r->n_child[i] == 0; }

static void walk(walkctx* w, int32_t A, int32_t B) {
  const oracle_result* r = w->r;
  if (w->err) return;
  if (r->mark && !r->mark[A]) return; /* sampled mode: no requested target below A */
  if (w->tasks && (r->level[A] >= w->split_at || r->level[B] >= w->split_at)) {
    if (pv_push(w->tasks, A, B)) w->err = 1; /* walked later, in parallel */
    return;
  }
  if (A == B) {
    if (is_leaf(r, A)) {
      emit(w, 1, A, A);
    } else {
      for (int i = 0; i < r->n_child[A]; i++)
        for (int j = 0; j < r->n_child[A]; j++)
          walk(w, r->first_child[A] + i, r->first_child[A] + j);
    }
    return;
  }
  if (accept(w, A, B)) {
    emit(w, 0, A, B);
    return;
  }
  int canA = !is_leaf(r, A), canB = !is_leaf(r, B);
  int la = r->level[A], lb = r->level[B];
  if (canA && canB) {
    if (la < lb) {
      for (int i = 0; i < r->n_child[A]; i++) walk(w, r->first_child[A] + i, B);
    } else if (lb < la) {
      for (int j = 0; j < r->n_child[B]; j++) walk(w, A, r->first_child[B] + j);
    } else {
      for (int i = 0; i < r->n_child[A]; i++)
        for (int j = 0; j < r->n_child[B]; j++)
          walk(w, r->first_child[A] + i, r->first_child[B] + j);
    }
  } else if (canA) {
    for (int i = 0; i < r->n_child[A]; i++) walk(w, r->first_child[A] + i, B);
  } else if (canB) {
    for (int j = 0; j < r->n_child[B]; j++) walk(w, A, r->first_child[B] + j);
  } else {
    emit(w, 1, A, B);
  }
}

/* Digest mode: the walk from (root, root) down to the pairs that reach level
 * split_at, then those pairs' walks in parallel. */
static int walk_digests(walkctx* w) {
  pairvec tasks;
  memset(&tasks, 0, sizeof(tasks));
  w->tasks = &tasks;
  w->split_at = 4;
  walk(w, 0, 0);
  w->tasks = NULL;
  int err = w->err;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : err)
  for (int64_t k = 0; k < tasks.n; k++) {
    walkctx lw = *w;
    lw.err = 0;
    walk(&lw, tasks.t[k], tasks.s[k]);
    err |= lw.err;
  }
  free(tasks.t);
  free(tasks.s);
  return err;
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* R12: CSR by target, sources ascending. */
static int to_csr(int64_t n_nodes, pairvec* v, int64_t** off_out, int32_t** src_out) {
  int64_t* off = (int64_t*)calloc((size_t)n_nodes + 1, sizeof(int64_t));
  int32_t* src = (int32_t*)malloc(sizeof(int32_t) * (size_t)(v->n ? v->n : 1));
  int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_nodes + 1));
  if (!off || !src || !cur) {
    free(off);
    free(src);
    free(cur);
    return ORACLE_ERR_OOM;
  }
  for (int64_t e = 0; e < v->n; e++) off[v->t[e] + 1]++;
  for (int64_t i = 0; i < n_nodes; i++) off[i + 1] += off[i];
  memcpy(cur, off, sizeof(int64_t) * (size_t)(n_nodes + 1));
  for (int64_t e = 0; e < v->n; e++) src[cur[v->t[e]]++] = v->s[e];
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < n_nodes; i++)
    qsort(src + off[i], (size_t)(off[i + 1] - off[i]), sizeof(int32_t), cmp_i32);
  free(cur);
  *off_out = off;
  *src_out = src;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* the whole evaluation                                                */
/* ------------------------------------------------------------------ */
int oracle_fmm(int64_t n, const double* pos, const double* mass, int order, double theta,
               int leaf_size, int64_t n_sample, const int64_t* sample, int stage_mask,
               oracle_result** out) {
  *out = NULL;
  if (n < 1 || n >= ((int64_t)1 << 31) || order < 0 || order > MAXP || !(theta > 0.0) ||
      !(theta < 1.0) || leaf_size < 1 || n_sample < 0)
    return ORACLE_ERR_ARG;
  for (int64_t i = 0; i < 3 * n; i++)
    if (!isfinite(pos[i])) return ORACLE_ERR_NONFINITE;
  for (int64_t i = 0; i < n; i++)
    if (!isfinite(mass[i])) return ORACLE_ERR_NONFINITE;
  for (int64_t s = 0; s < n_sample; s++)
    if (sample[s] < 0 || sample[s] >= n) return ORACLE_ERR_ARG;

  oracle_result* r = (oracle_result*)calloc(1, sizeof(oracle_result));
  if (!r) return ORACLE_ERR_OOM;
  r->n = n;
  r->p = order;
  r->K = oracle_ncoef(order);
  r->leaf = leaf_size;
  r->theta = theta;
  mtab tab;
  mtab_init(&tab, order);
  int rc = ORACLE_OK;
  double t0 = wall(), t1;

  /* keys + stable sort */
  uint64_t* keys = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)n);
  kidx* ki = (kidx*)malloc(sizeof(kidx) * (size_t)n);
  r->key = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)n);
  r->perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  r->xs = (double*)malloc(sizeof(double) * 3 * (size_t)n);
  r->ms = (double*)malloc(sizeof(double) * (size_t)n);
  if (!keys || !ki || !r->key || !r->perm || !r->xs || !r->ms) {
    free(keys);
    free(ki);
    oracle_free(r);
    return ORACLE_ERR_OOM;
  }
  root_cube(n, pos, r->lo, &r->side);
  keys_of(n, pos, r->lo, r->side, keys);
  for (int64_t i = 0; i < n; i++) {
    ki[i].key = keys[i];
    ki[i].idx = i;
  }
  qsort(ki, (size_t)n, sizeof(kidx), kidx_cmp);
  for (int64_t k = 0; k < n; k++) {
    int64_t i = ki[k].idx;
    r->key[k] = ki[k].key;
    r->perm[k] = (int32_t)i;
    for (int a = 0; a < 3; a++) r->xs[3 * k + a] = pos[3 * i + a];
    r->ms[k] = mass[i];
  }
  free(keys);
  free(ki);
  t1 = wall();
  r->times[0] = t1 - t0;
  t0 = t1;

  rc = build_tree(r);
  if (rc) {
    oracle_free(r);
    return rc;
  }
  t1 = wall();
  r->times[1] = t1 - t0;
  t0 = t1;

  /* sampled mode: mark the leaves that hold a requested particle and their
   * ancestors; everything else is computed only as a source */
  if (n_sample > 0) {
    r->mark = (uint8_t*)calloc((size_t)r->n_nodes, 1);
    int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* leaf_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!r->mark || !inv || !leaf_of) {
      free(inv);
      free(leaf_of);
      oracle_free(r);
      return ORACLE_ERR_OOM;
    }
    for (int64_t k = 0; k < n; k++) inv[r->perm[k]] = (int32_t)k;
    for (int64_t i = 0; i < r->n_nodes; i++)
      if (r->n_child[i] == 0)
        for (int32_t k = r->begin[i]; k < r->begin[i] + r->count[i]; k++) leaf_of[k] = (int32_t)i;
    for (int64_t s = 0; s < n_sample; s++) {
      int32_t i = leaf_of[inv[sample[s]]];
      while (i >= 0 && !r->mark[i]) {
        r->mark[i] = 1;
        i = r->parent[i];
      }
    }
    free(inv);
    free(leaf_of);
    r->n_marked = 0;
    for (int64_t i = 0; i < r->n_nodes; i++) r->n_marked += r->mark[i];
  } else {
    r->n_marked = r->n_nodes;
  }

  walkctx w;
  memset(&w, 0, sizeof(w));
  w.r = r;
  w.t2 = theta * theta; /* fl(theta^2), one rounding (R11) */
  if (stage_mask & 2) { /* digest mode: no lists, no numeric passes */
    w.digest = 1;
    for (int k = 0; k < 2; k++) {
      r->dcnt[k] = (uint64_t*)calloc((size_t)r->n_nodes, sizeof(uint64_t));
      r->dhash[k] = (uint64_t*)calloc((size_t)r->n_nodes, sizeof(uint64_t));
      if (!r->dcnt[k] || !r->dhash[k]) {
        oracle_free(r);
        return ORACLE_ERR_OOM;
      }
      w.dcnt[k] = r->dcnt[k];
      w.dhash[k] = r->dhash[k];
    }
    if (walk_digests(&w)) {
      oracle_free(r);
      return ORACLE_ERR_OOM;
    }
    r->n_m2l = r->n_p2p = 0;
    for (int64_t i = 0; i < r->n_nodes; i++) {
      r->n_m2l += (int64_t)r->dcnt[0][i];
      r->n_p2p += (int64_t)r->dcnt[1][i];
    }
    r->times[2] = wall() - t0;
    *out = r;
    return ORACLE_OK;
  }
  walk(&w, 0, 0);
  if (w.err) {
    free(w.m2l.t);
    free(w.m2l.s);
    free(w.p2p.t);
    free(w.p2p.s);
    oracle_free(r);
    return ORACLE_ERR_OOM;
  }
  r->n_m2l = w.m2l.n;
  r->n_p2p = w.p2p.n;
  rc = to_csr(r->n_nodes, &w.m2l, &r->m2l_off, &r->m2l_src);
  if (!rc) rc = to_csr(r->n_nodes, &w.p2p, &r->p2p_off, &r->p2p_src);
  free(w.m2l.t);
  free(w.m2l.s);
  free(w.p2p.t);
  free(w.p2p.s);
  if (rc) {
    oracle_free(r);
    return rc;
  }
  t1 = wall();
  r->times[2] = t1 - t0;
  t0 = t1;

  if (!(stage_mask & 1)) {
    *out = r;
    return ORACLE_OK;
  }

  const int K = r->K;
  const int64_t nn = r->n_nodes;
  r->M = (double*)calloc((size_t)(nn * K), sizeof(double));
  r->L = (double*)calloc((size_t)(nn * K), sizeof(double));
  double* phs = (double*)calloc((size_t)n, sizeof(double));
  double* acs = (double*)calloc((size_t)(3 * n), sizeof(double));
  r->phi = (double*)malloc(sizeof(double) * (size_t)n);
  r->acc = (double*)malloc(sizeof(double) * 3 * (size_t)n);
  if (!r->M || !r->L || !phs || !acs || !r->phi || !r->acc) {
    free(phs);
    free(acs);
    oracle_free(r);
    return ORACLE_ERR_OOM;
  }

  /* upward pass: leaf moments, then children into parents, deepest level first */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < nn; i++)
    if (r->n_child[i] == 0)
      p2m_set(&tab, r->count[i], r->xs + 3 * (int64_t)r->begin[i], r->ms + r->begin[i],
              r->centre + 3 * i, r->M + i * K);
  for (int lev = r->depth - 1; lev >= 0; lev--) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < nn; i++) {
      if (r->level[i] != lev || r->n_child[i] == 0) continue;
      for (int c = 0; c < r->n_child[i]; c++) {
        int64_t ch = r->first_child[i] + c;
        double d[3] = {r->centre[3 * ch] - r->centre[3 * i],
                       r->centre[3 * ch + 1] - r->centre[3 * i + 1],
                       r->centre[3 * ch + 2] - r->centre[3 * i + 2]};
        m2m_one(&tab, r->M + ch * K, d, r->M + i * K);
      }
    }
  }
  t1 = wall();
  r->times[3] = t1 - t0;
  t0 = t1;

  /* interaction stage: every accepted pair translated into the target's local */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nn; a++) {
    for (int64_t e = r->m2l_off[a]; e < r->m2l_off[a + 1]; e++) {
      int64_t b = r->m2l_src[e];
      double R[3] = {r->centre[3 * a] - r->centre[3 * b],
                     r->centre[3 * a + 1] - r->centre[3 * b + 1],
                     r->centre[3 * a + 2] - r->centre[3 * b + 2]};
      m2l_one(&tab, r->M + b * K, R, r->L + a * K);
    }
  }
  t1 = wall();
  r->times[4] = t1 - t0;
  t0 = t1;

  /* downward pass: parents before children (breadth-first ids), then leaves */
  for (int lev = 1; lev <= r->depth; lev++) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < nn; i++) {
      if (r->level[i] != lev) continue;
      if (r->mark && !r->mark[i]) continue;
      int64_t pa = r->parent[i];
      double d[3] = {r->centre[3 * i] - r->centre[3 * pa],
                     r->centre[3 * i + 1] - r->centre[3 * pa + 1],
                     r->centre[3 * i + 2] - r->centre[3 * pa + 2]};
      l2l_one(&tab, r->L + pa * K, d, r->L + i * K);
    }
  }
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < nn; i++) {
    if (r->n_child[i] != 0 || (r->mark && !r->mark[i])) continue;
    for (int32_t k = r->begin[i]; k < r->begin[i] + r->count[i]; k++) {
      double dx[3] = {r->xs[3 * k] - r->centre[3 * i], r->xs[3 * k + 1] - r->centre[3 * i + 1],
                      r->xs[3 * k + 2] - r->centre[3 * i + 2]};
      l2p_one(&tab, r->L + i * K, dx, phs + k, acs + 3 * k);
    }
  }
  t1 = wall();
  r->times[5] = t1 - t0;
  t0 = t1;

  /* near field: leaf pairs summed directly, self term omitted by index (R13) */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nn; a++) {
    if (r->n_child[a] != 0) continue;
    for (int32_t i = r->begin[a]; i < r->begin[a] + r->count[a]; i++) {
      double p = 0.0, a0 = 0.0, a1 = 0.0, a2 = 0.0;
      for (int64_t e = r->p2p_off[a]; e < r->p2p_off[a + 1]; e++) {
        int32_t b = r->p2p_src[e];
        for (int32_t j = r->begin[b]; j < r->begin[b] + r->count[b]; j++) {
          if (j == i) continue;
          double dx = r->xs[3 * i] - r->xs[3 * j], dy = r->xs[3 * i + 1] - r->xs[3 * j + 1],
                 dz = r->xs[3 * i + 2] - r->xs[3 * j + 2];
          double rr = sqrt(dx * dx + dy * dy + dz * dz);
          double r3 = rr * rr * rr;
          p -= r->ms[j] / rr;
          a0 -= r->ms[j] * dx / r3;
          a1 -= r->ms[j] * dy / r3;
          a2 -= r->ms[j] * dz / r3;
        }
      }
      phs[i] += p;
      acs[3 * i] += a0;
      acs[3 * i + 1] += a1;
      acs[3 * i + 2] += a2;
    }
  }
  t1 = wall();
  r->times[6] = t1 - t0;

  /* back to the caller's order; in sampled mode unmarked leaves give NaN */
  for (int64_t k = 0; k < n; k++) {
    int64_t i = r->perm[k];
    r->phi[i] = phs[k];
    for (int a = 0; a < 3; a++) r->acc[3 * i + a] = acs[3 * k + a];
  }
  if (r->mark) {
    for (int64_t i = 0; i < nn; i++) {
      if (r->n_child[i] != 0 || r->mark[i]) continue;
      for (int32_t k = r->begin[i]; k < r->begin[i] + r->count[i]; k++) {
        int64_t q = r->perm[k];
        r->phi[q] = NAN;
        r->acc[3 * q] = r->acc[3 * q + 1] = r->acc[3 * q + 2] = NAN;
      }
    }
  }
  free(phs);
  free(acs);
  double tot = 0.0;
  for (int s = 0; s < 7; s++) tot += r->times[s];
  r->times[7] = tot;
  *out = r;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* vector-Jacobian product, fast multipole form                        */
/* ------------------------------------------------------------------ */
/* The jz-fmm page ("Following sensitivities backwards") evaluates the VJP of
 * the FMM with two contributions.  Written out for S = sum_i pb_i phi_i +
 * ab_i . a_i, with Phi the potential of the masses and
 *   Psi(y) = sum_k [ pb_k G(y - x_k) + ab_k . grad_y G(y - x_k) ],  G = -1/|r|,
 * the potential of monopoles pb_k and dipoles ab_k (self term omitted):
 *   dS/dx_i = -pb_i a_i - Hess Phi(x_i) ab_i + m_i grad Psi(x_i),
 *   dS/dm_i = Psi(x_i).
 * The first two terms are the "next higher derivative in the original
 * evaluation" (Hess Phi from the forward's leaf locals plus the near field),
 * the last ones "an FMM with the force sensitivities acting as dipole
 * moments": the same tree, lists and translations, with the moments of the
 * monopoles and dipoles.  Every sum runs over the same near and far split as
 * the forward.  In sampled mode only the marked leaves are targets (the
 * others get NaN), exactly as in the forward. */
static int fmm_vjp_on(const oracle_result* r, const double* pb, const double* ab,
                      double* xbar, double* mbar) {
  const int64_t n = r->n, nn = r->n_nodes;
  const int K = r->K;
  mtab tab;
  mtab_init(&tab, r->p);
  double* pbs = (double*)malloc(sizeof(double) * (size_t)n);
  double* abs_ = (double*)malloc(sizeof(double) * 3 * (size_t)n);
  double* Mb = (double*)calloc((size_t)(nn * K), sizeof(double));
  double* Lb = (double*)calloc((size_t)(nn * K), sizeof(double));
  double* H = (double*)calloc((size_t)(6 * n), sizeof(double));
  double* psi = (double*)calloc((size_t)n, sizeof(double));
  double* mg = (double*)calloc((size_t)(3 * n), sizeof(double)); /* -grad Psi */
  if (!pbs || !abs_ || !Mb || !Lb || !H || !psi || !mg) {
    free(pbs);
    free(abs_);
    free(Mb);
    free(Lb);
    free(H);
    free(psi);
    free(mg);
    return ORACLE_ERR_OOM;
  }
  for (int64_t k = 0; k < n; k++) {
    int64_t i = r->perm[k];
    pbs[k] = pb[i];
    for (int a = 0; a < 3; a++) abs_[3 * k + a] = ab[3 * i + a];
  }

  /* upward pass of the sensitivity sources */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < nn; i++)
    if (r->n_child[i] == 0)
      p2m_dip_set(&tab, r->count[i], r->xs + 3 * (int64_t)r->begin[i], pbs + r->begin[i],
                  abs_ + 3 * (int64_t)r->begin[i], r->centre + 3 * i, Mb + i * K);
  for (int lev = r->depth - 1; lev >= 0; lev--) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < nn; i++) {
      if (r->level[i] != lev || r->n_child[i] == 0) continue;
      for (int c = 0; c < r->n_child[i]; c++) {
        int64_t ch = r->first_child[i] + c;
        double d[3] = {r->centre[3 * ch] - r->centre[3 * i],
                       r->centre[3 * ch + 1] - r->centre[3 * i + 1],
                       r->centre[3 * ch + 2] - r->centre[3 * i + 2]};
        m2m_one(&tab, Mb + ch * K, d, Mb + i * K);
      }
    }
  }
  /* interaction stage over the forward's accepted pairs */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nn; a++) {
    for (int64_t e = r->m2l_off[a]; e < r->m2l_off[a + 1]; e++) {
      int64_t b = r->m2l_src[e];
      double R[3] = {r->centre[3 * a] - r->centre[3 * b],
                     r->centre[3 * a + 1] - r->centre[3 * b + 1],
                     r->centre[3 * a + 2] - r->centre[3 * b + 2]};
      m2l_one(&tab, Mb + b * K, R, Lb + a * K);
    }
  }
  /* downward pass */
  for (int lev = 1; lev <= r->depth; lev++) {
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < nn; i++) {
      if (r->level[i] != lev) continue;
      if (r->mark && !r->mark[i]) continue;
      int64_t pa = r->parent[i];
      double d[3] = {r->centre[3 * i] - r->centre[3 * pa],
                     r->centre[3 * i + 1] - r->centre[3 * pa + 1],
                     r->centre[3 * i + 2] - r->centre[3 * pa + 2]};
      l2l_one(&tab, Lb + pa * K, d, Lb + i * K);
    }
  }
  /* far parts at the particles: Hess Phi from the forward's locals, Psi and
   * -grad Psi from the sensitivity locals */
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t i = 0; i < nn; i++) {
    if (r->n_child[i] != 0 || (r->mark && !r->mark[i])) continue;
    for (int32_t k = r->begin[i]; k < r->begin[i] + r->count[i]; k++) {
      double dx[3] = {r->xs[3 * k] - r->centre[3 * i], r->xs[3 * k + 1] - r->centre[3 * i + 1],
                      r->xs[3 * k + 2] - r->centre[3 * i + 2]};
      l2p_hess_one(&tab, r->L + i * K, dx, H + 6 * (int64_t)k);
      l2p_one(&tab, Lb + i * K, dx, psi + k, mg + 3 * (int64_t)k);
    }
  }
  /* near field, self term omitted by index */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t a = 0; a < nn; a++) {
    if (r->n_child[a] != 0 || (r->mark && !r->mark[a])) continue;
    for (int32_t i = r->begin[a]; i < r->begin[a] + r->count[a]; i++) {
      double h[6] = {0, 0, 0, 0, 0, 0}, ps = 0.0, gp[3] = {0, 0, 0};
      for (int64_t e = r->p2p_off[a]; e < r->p2p_off[a + 1]; e++) {
        int32_t b = r->p2p_src[e];
        for (int32_t j = r->begin[b]; j < r->begin[b] + r->count[b]; j++) {
          if (j == i) continue;
          double d[3] = {r->xs[3 * i] - r->xs[3 * j], r->xs[3 * i + 1] - r->xs[3 * j + 1],
                         r->xs[3 * i + 2] - r->xs[3 * j + 2]};
          double rr = sqrt(d[0] * d[0] + d[1] * d[1] + d[2] * d[2]);
          double r3 = rr * rr * rr, r5 = r3 * rr * rr;
          double mj = r->ms[j];
          /* Hess Phi: m_j (I/r^3 - 3 d d^T/r^5) */
          h[0] += mj * (1.0 / r3 - 3.0 * d[0] * d[0] / r5);
          h[1] += mj * (1.0 / r3 - 3.0 * d[1] * d[1] / r5);
          h[2] += mj * (1.0 / r3 - 3.0 * d[2] * d[2] / r5);
          h[3] -= mj * 3.0 * d[0] * d[1] / r5;
          h[4] -= mj * 3.0 * d[0] * d[2] / r5;
          h[5] -= mj * 3.0 * d[1] * d[2] / r5;
          /* Psi and grad Psi of monopole pb_j and dipole ab_j at x_j */
          const double* aj = abs_ + 3 * (int64_t)j;
          double ad = aj[0] * d[0] + aj[1] * d[1] + aj[2] * d[2];
          ps += -pbs[j] / rr + ad / r3;
          for (int c = 0; c < 3; c++) gp[c] += pbs[j] * d[c] / r3 + aj[c] / r3 - 3.0 * d[c] * ad / r5;
        }
      }
      for (int c = 0; c < 6; c++) H[6 * (int64_t)i + c] += h[c];
      psi[i] += ps;
      for (int c = 0; c < 3; c++) mg[3 * (int64_t)i + c] -= gp[c];
    }
  }
  /* combine in the caller's order */
  for (int64_t k = 0; k < n; k++) {
    int64_t i = r->perm[k];
    const double* h = H + 6 * k;
    const double* b = abs_ + 3 * k;
    double hb[3] = {h[0] * b[0] + h[3] * b[1] + h[4] * b[2],
                    h[3] * b[0] + h[1] * b[1] + h[5] * b[2],
                    h[4] * b[0] + h[5] * b[1] + h[2] * b[2]};
    for (int a = 0; a < 3; a++)
      xbar[3 * i + a] = -pbs[k] * r->acc[3 * i + a] - hb[a] - r->ms[k] * mg[3 * k + a];
    mbar[i] = psi[k];
  }
  if (r->mark) {
    for (int64_t i = 0; i < nn; i++) {
      if (r->n_child[i] != 0 || r->mark[i]) continue;
      for (int32_t k = r->begin[i]; k < r->begin[i] + r->count[i]; k++) {
        int64_t q = r->perm[k];
        mbar[q] = NAN;
        xbar[3 * q] = xbar[3 * q + 1] = xbar[3 * q + 2] = NAN;
      }
    }
  }
  free(pbs);
  free(abs_);
  free(Mb);
  free(Lb);
  free(H);
  free(psi);
  free(mg);
  return ORACLE_OK;
}

int oracle_fmm_vjp(int64_t n, const double* pos, const double* mass, int order, double theta,
                   int leaf_size, int64_t n_sample, const int64_t* sample, const double* pb,
                   const double* ab, double* xbar, double* mbar) {
  for (int64_t i = 0; i < n; i++)
    if (!isfinite(pb[i]) || !isfinite(ab[3 * i]) || !isfinite(ab[3 * i + 1]) ||
        !isfinite(ab[3 * i + 2]))
      return ORACLE_ERR_NONFINITE;
  oracle_result* r = NULL;
  int rc = oracle_fmm(n, pos, mass, order, theta, leaf_size, n_sample, sample, 1, &r);
  if (rc) return rc;
  rc = fmm_vjp_on(r, pb, ab, xbar, mbar);
  oracle_free(r);
  return rc;
}

/* ------------------------------------------------------------------ */
/* reversible integer-lattice kick-drift-kick step                     */
/* ------------------------------------------------------------------ */
/* The jz-fmm page ("Why reversibility matters") keeps positions and velocities
 * on an integer lattice while the force stays floating point; undoing an
 * update subtracts the increment the forward update added.  Readings: the
 * time-symmetric scheme is kick-drift-kick leapfrog; x = q dx and v = u dv
 * with q, u integer; increments are rounded half to even in fp64:
 *   kick:  u += s rint(a(q) (dt/2) / dv),    drift: q += s rint(u (dt dv / dx)),
 * with s = +1 forward and -1 backward.  A backward step runs kick, drift, kick
 * with s = -1, starting from the force at its starting state, so it undoes a
 * forward step exactly.  Forces come from oracle_fmm (G = 1).  *min_margin
 * receives the smallest distance of a kick's rounded quantity to a rounding
 * boundary (x.5), relative to max(1, |quantity|), over all kicks. */
static int lattice_force(int64_t n, const int64_t* q, const double* mass, double dx, int order,
                         double theta, int leaf, double* pos, double* acc) {
  for (int64_t i = 0; i < 3 * n; i++) pos[i] = (double)q[i] * dx;
  oracle_result* r = NULL;
  int rc = oracle_fmm(n, pos, mass, order, theta, leaf, 0, NULL, 1, &r);
  if (rc) return rc;
  memcpy(acc, r->acc, sizeof(double) * 3 * (size_t)n);
  oracle_free(r);
  return ORACLE_OK;
}

static void lattice_kick(int64_t n, int64_t* u, const double* acc, double c, int s,
                         double* min_margin) {
  for (int64_t i = 0; i < 3 * n; i++) {
    double k = acc[i] * c;
    double m = fabs(k - floor(k) - 0.5) / fmax(1.0, fabs(k));
    if (m < *min_margin) *min_margin = m;
    u[i] += (int64_t)s * (int64_t)rint(k);
  }
}

int oracle_lattice_steps(int64_t n, int64_t* q, int64_t* u, const double* mass, double dx,
                         double dv, double dt, int n_steps, int direction, int order,
                         double theta, int leaf_size, double* min_margin) {
  if (n < 1 || n_steps < 0 || (direction != 1 && direction != -1) || !(dx > 0.0) ||
      !(dv > 0.0) || !isfinite(dt))
    return ORACLE_ERR_ARG;
  double* pos = (double*)malloc(sizeof(double) * 3 * (size_t)n);
  double* acc = (double*)malloc(sizeof(double) * 3 * (size_t)n);
  if (!pos || !acc) {
    free(pos);
    free(acc);
    return ORACLE_ERR_OOM;
  }
  const double ck = 0.5 * dt / dv, cd = dt * dv / dx;
  *min_margin = INFINITY;
  int rc = n_steps > 0 ? lattice_force(n, q, mass, dx, order, theta, leaf_size, pos, acc) : 0;
  for (int st = 0; st < n_steps && !rc; st++) {
    lattice_kick(n, u, acc, ck, direction, min_margin);
    for (int64_t i = 0; i < 3 * n; i++)
      q[i] += (int64_t)direction * (int64_t)rint((double)u[i] * cd);
    rc = lattice_force(n, q, mass, dx, order, theta, leaf_size, pos, acc);
    if (!rc) lattice_kick(n, u, acc, ck, direction, min_margin);
  }
  free(pos);
  free(acc);
  return rc;
}

/* ------------------------------------------------------------------ */
/* copy-out                                                            */
/* ------------------------------------------------------------------ */
void oracle_sizes(const oracle_result* r, int64_t* s) {
  s[0] = r->n_nodes;
  s[1] = r->n_leaves;
  s[2] = r->depth;
  s[3] = r->n_m2l;
  s[4] = r->n_p2p;
  s[5] = r->n_marked;
  s[6] = r->K;
}
void oracle_root(const oracle_result* r, double* lo, double* side) {
  for (int a = 0; a < 3; a++) lo[a] = r->lo[a];
  *side = r->side;
}
void oracle_times(const oracle_result* r, double* t8) { memcpy(t8, r->times, sizeof(r->times)); }
void oracle_copy_keys(const oracle_result* r, uint64_t* keys, int32_t* perm) {
  if (keys) memcpy(keys, r->key, sizeof(uint64_t) * (size_t)r->n);
  if (perm) memcpy(perm, r->perm, sizeof(int32_t) * (size_t)r->n);
}
void oracle_copy_tree(const oracle_result* r, uint8_t* level, uint64_t* prefix, int32_t* begin,
                      int32_t* count, int32_t* parent, int32_t* first_child, uint8_t* n_child) {
  size_t m = (size_t)r->n_nodes;
  if (level) memcpy(level, r->level, m);
  if (prefix) memcpy(prefix, r->prefix, 8 * m);
  if (begin) memcpy(begin, r->begin, 4 * m);
  if (count) memcpy(count, r->count, 4 * m);
  if (parent) memcpy(parent, r->parent, 4 * m);
  if (first_child) memcpy(first_child, r->first_child, 4 * m);
  if (n_child) memcpy(n_child, r->n_child, m);
}
void oracle_copy_lists(const oracle_result* r, int64_t* m2l_off, int32_t* m2l_src,
                       int64_t* p2p_off, int32_t* p2p_src) {
  size_t m = (size_t)r->n_nodes + 1;
  if (!r->m2l_off) return; /* digest mode: no lists */
  if (m2l_off) memcpy(m2l_off, r->m2l_off, 8 * m);
  if (m2l_src) memcpy(m2l_src, r->m2l_src, 4 * (size_t)r->n_m2l);
  if (p2p_off) memcpy(p2p_off, r->p2p_off, 8 * m);
  if (p2p_src) memcpy(p2p_src, r->p2p_src, 4 * (size_t)r->n_p2p);
}
int oracle_copy_digests(const oracle_result* r, uint64_t* m2l_cnt, uint64_t* m2l_hash,
                        uint64_t* p2p_cnt, uint64_t* p2p_hash) {
  uint64_t* cnt[2] = {m2l_cnt, p2p_cnt};
  uint64_t* hash[2] = {m2l_hash, p2p_hash};
  for (int k = 0; k < 2; k++) {
    if (r->dcnt[k]) { /* digest mode */
      memcpy(cnt[k], r->dcnt[k], sizeof(uint64_t) * (size_t)r->n_nodes);
      memcpy(hash[k], r->dhash[k], sizeof(uint64_t) * (size_t)r->n_nodes);
      continue;
    }
    const int64_t* off = k == 0 ? r->m2l_off : r->p2p_off;
    const int32_t* src = k == 0 ? r->m2l_src : r->p2p_src;
    if (!off) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < r->n_nodes; i++) {
      uint64_t h = 0;
      for (int64_t e = off[i]; e < off[i + 1]; e++) h += digest_h(src[e]);
      cnt[k][i] = (uint64_t)(off[i + 1] - off[i]);
      hash[k][i] = h;
    }
  }
  return ORACLE_OK;
}

void oracle_copy_mark(const oracle_result* r, uint8_t* mark) {
  if (r->mark)
    memcpy(mark, r->mark, (size_t)r->n_nodes);
  else
    memset(mark, 1, (size_t)r->n_nodes);
}
void oracle_copy_expansions(const oracle_result* r, double* M, double* L) {
  size_t m = (size_t)r->n_nodes * (size_t)r->K;
  if (M && r->M) memcpy(M, r->M, 8 * m);
  if (L && r->L) memcpy(L, r->L, 8 * m);
}
void oracle_copy_result(const oracle_result* r, double* phi, double* acc) {
  if (phi && r->phi) memcpy(phi, r->phi, 8 * (size_t)r->n);
  if (acc && r->acc) memcpy(acc, r->acc, 24 * (size_t)r->n);
}

/*
 * CPU oracle for the Mamba-3 physical-frame state moments (TEST INFRASTRUCTURE).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library. It shares no code, header or constant with the HIP path.
 *
 * Sources (pages on burn-mamba's mamba3 moments module):
 *   - "backward.rs" source page, module doc "Gradient math": forward equations
 *     h~[t] = d_t h_- + sum_j L[t,j] W_j, c_t = R_t^T h~[t], m2 += c^T c, m1 += c,
 *     and the statement that d_t, L[t,j] are products of exp(da) over the tokens
 *     between (so the chunked form equals the per-token recurrence).
 *   - "recalculated.rs" source page: rotate_chunk (de-rotation R(-theta) on pairs,
 *     pairwise or half-split; left Hamilton product by Q on 4-blocks),
 *     quat_mul_prim (Hamilton product), chunk_mask (positions < valid_len).
 *
 * What is computed here is the plain definition the chunked method reaches
 * exactly: per (b,h) chain, in fp64,
 *     H_t = exp(da_t) H_{t-1} + sum_c xhat[t,c] (outer) bhat[t,c],  H_{-1} = h0
 *     C_t = H_t M_t^T     (each state row is de-rotated by the r x r matrix M_t)
 *     m2 += C_t^T C_t,  m1 += C_t   for t < V = min(valid_len, s)
 * m1 is kept per row p ([b,h,p,r]); the pages' pooled m1[b,h,r] is its sum over p.
 *
 * The backward is this file's own reverse-time adjoint of that recurrence,
 * written with explicit matrices (dM_t = dC_t^T H_t contracted with dM/dtheta or
 * dM/dQ_k), deliberately not the pages' chunkwise VJP formulas, so the two can
 * cross-check. States are re-materialised from checkpoints every CKPT tokens.
 *
 * Layouts (row-major): xhat[b,s,c,h,p], bhat[b,s,c,h,r], da[b,s,h],
 * rot[b,s,h,A] (A angles) or [b,s,h,J,4] (w,x,y,z), h0[b,h,p,r],
 * m2[b,h,r,r], m1[b,h,p,r]; gradients have the shapes of their inputs.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_ROT_NONE 0
#define ORC_ROT_PAIRWISE 1
#define ORC_ROT_HALF 2
#define ORC_ROT_QUAT 3
#define CKPT 256

typedef struct {
  int64_t b, s, c, h, p, r;
  int64_t valid_len;
  int64_t rot_kind;
  int64_t rope_dim;   /* complex modes: number of rotated coordinates (even) */
  int64_t quat_blocks;/* quaternion mode: J */
} orc_desc;

/* ---- the de-rotation matrix M_t, one block at a time -------------------- */

/* Number of rotation blocks, block size and the state coordinates of block k. */
static int64_t n_blocks(const orc_desc* d) {
  if (d->rot_kind == ORC_ROT_PAIRWISE || d->rot_kind == ORC_ROT_HALF) return d->rope_dim / 2;
  if (d->rot_kind == ORC_ROT_QUAT) return d->quat_blocks;
  return 0;
}
static int block_size(const orc_desc* d) { return d->rot_kind == ORC_ROT_QUAT ? 4 : 2; }
static void block_coords(const orc_desc* d, int64_t k, int64_t* idx) {
  if (d->rot_kind == ORC_ROT_PAIRWISE) { idx[0] = 2 * k; idx[1] = 2 * k + 1; }
  else if (d->rot_kind == ORC_ROT_HALF) { idx[0] = k; idx[1] = d->r / 2 + k; }
  else { for (int i = 0; i < 4; i++) idx[i] = 4 * k + i; }
}
/* Angle count per token in the rot tensor (complex) or quaternion count. */
static int64_t rot_stride(const orc_desc* d) {
  if (d->rot_kind == ORC_ROT_PAIRWISE || d->rot_kind == ORC_ROT_HALF) return d->rope_dim / 2;
  if (d->rot_kind == ORC_ROT_QUAT) return 4 * d->quat_blocks;
  return 0;
}

/* Fill blk (bs x bs, row-major) with block k of M_t; pr points at rot[b,t,h,:]. */
static void block_matrix(const orc_desc* d, const double* pr, int64_t k, double* blk) {
  if (d->rot_kind == ORC_ROT_QUAT) {
    /* left Hamilton matrix of Q = (w,x,y,z): (Q (x) v) = Lmat(Q) v */
    const double w = pr[4 * k], x = pr[4 * k + 1], y = pr[4 * k + 2], z = pr[4 * k + 3];
    const double m[16] = {w, -x, -y, -z,
                          x,  w, -z,  y,
                          y,  z,  w, -x,
                          z, -y,  x,  w};
    memcpy(blk, m, sizeof(m));
  } else {
    /* de-rotation R(-theta): (x,y) -> (cos x + sin y, -sin x + cos y) */
    const double th = pr[k], cs = cos(th), sn = sin(th);
    blk[0] = cs; blk[1] = sn; blk[2] = -sn; blk[3] = cs;
  }
}

/* Partial derivative of block k of M_t with respect to its parameter q
 * (q = 0 for the angle; q = 0..3 for w,x,y,z). */
static void block_dmatrix(const orc_desc* d, const double* pr, int64_t k, int q, double* g) {
  if (d->rot_kind == ORC_ROT_QUAT) {
    static const double E[4][16] = {
        {1, 0, 0, 0,  0, 1, 0, 0,  0, 0, 1, 0,  0, 0, 0, 1},
        {0, -1, 0, 0,  1, 0, 0, 0,  0, 0, 0, -1,  0, 0, 1, 0},
        {0, 0, -1, 0,  0, 0, 0, 1,  1, 0, 0, 0,  0, -1, 0, 0},
        {0, 0, 0, -1,  0, 0, -1, 0,  0, 1, 0, 0,  1, 0, 0, 0}};
    memcpy(g, E[q], sizeof(E[q]));
  } else {
    const double th = pr[k], cs = cos(th), sn = sin(th);
    g[0] = -sn; g[1] = cs; g[2] = -cs; g[3] = -sn;
  }
}

/* c_row = M_t h_row for one state row (length r). */
static void derotate_row(const orc_desc* d, const double* pr, const double* hrow, double* crow) {
  const int64_t r = d->r;
  memcpy(crow, hrow, (size_t)r * sizeof(double));
  const int64_t nb = n_blocks(d);
  const int bs = block_size(d);
  int64_t idx[4];
  double blk[16];
  for (int64_t k = 0; k < nb; k++) {
    block_coords(d, k, idx);
    block_matrix(d, pr, k, blk);
    for (int u = 0; u < bs; u++) {
      double acc = 0.0;
      for (int v = 0; v < bs; v++) acc += blk[u * bs + v] * hrow[idx[v]];
      crow[idx[u]] = acc;
    }
  }
}

/* g_row = M_t^T v_row (the transpose, applied to cotangents). */
static void derotate_row_T(const orc_desc* d, const double* pr, const double* vrow, double* grow) {
  const int64_t r = d->r;
  memcpy(grow, vrow, (size_t)r * sizeof(double));
  const int64_t nb = n_blocks(d);
  const int bs = block_size(d);
  int64_t idx[4];
  double blk[16];
  for (int64_t k = 0; k < nb; k++) {
    block_coords(d, k, idx);
    block_matrix(d, pr, k, blk);
    for (int v = 0; v < bs; v++) {
      double acc = 0.0;
      for (int u = 0; u < bs; u++) acc += blk[u * bs + v] * vrow[idx[u]];
      grow[idx[v]] = acc;
    }
  }
}

/* ---- work units: one (b,h) chain, a group of state rows [p0, p1) ---------
 * State rows evolve independently; only m2 (fwd) and d_bhat, d_rot, d_da (bwd)
 * sum over rows. Those sums go to per-unit partial buffers that are added in a
 * fixed order after all threads finish, so results do not depend on threading. */

typedef struct {
  const orc_desc* d;
  const double *xhat, *bhat, *da, *rot, *h0, *dm2, *dm1;
  double *m2, *m1, *dxhat, *dbhat, *dda, *drot, *dh0;
  const int64_t* chains;
  int64_t nchains, npg, nunits;
  double** part;         /* per-unit partial buffers */
  int64_t next;
  pthread_mutex_t mu;
} job_t;

static int64_t V_of(const orc_desc* d) { return d->valid_len < d->s ? d->valid_len : d->s; }
static void unit_rows(const job_t* J, int64_t g, int64_t* p0, int64_t* p1) {
  const int64_t p = J->d->p, per = (p + J->npg - 1) / J->npg;
  *p0 = g * per < p ? g * per : p;
  *p1 = (g + 1) * per < p ? (g + 1) * per : p;
}

/* H[rows] <- exp(da_t) H[rows] + sum_c xhat[t,c,rows] (outer) bhat[t,c]. */
static void step_state(const orc_desc* d, const double* xhat, const double* bhat, const double* da,
                       int64_t bi, int64_t hi, int64_t t, int64_t p0, int64_t p1, double* H) {
  const int64_t p = d->p, r = d->r, c = d->c, h = d->h, s = d->s, np = p1 - p0;
  const double e = exp(da[(bi * s + t) * h + hi]);
  for (int64_t i = 0; i < np * r; i++) H[i] *= e;
  for (int64_t ci = 0; ci < c; ci++) {
    const double* x = xhat + (((bi * s + t) * c + ci) * h + hi) * p;
    const double* bb = bhat + (((bi * s + t) * c + ci) * h + hi) * r;
    for (int64_t pi = p0; pi < p1; pi++) {
      const double xv = x[pi];
      double* Hr = H + (pi - p0) * r;
      for (int64_t ri = 0; ri < r; ri++) Hr[ri] += xv * bb[ri];
    }
  }
}

static void init_rows(const job_t* J, int64_t chain, int64_t p0, int64_t p1, double* H) {
  const int64_t p = J->d->p, r = J->d->r;
  if (J->h0) memcpy(H, J->h0 + (chain * p + p0) * r, (size_t)((p1 - p0) * r) * sizeof(double));
  else memset(H, 0, (size_t)((p1 - p0) * r) * sizeof(double));
}

static void fwd_unit(job_t* J, int64_t u) {
  const orc_desc* d = J->d;
  const int64_t r = d->r, h = d->h, s = d->s, p = d->p;
  const int64_t chain = J->chains[u / J->npg];
  const int64_t bi = chain / h, hi = chain % h;
  int64_t p0, p1;
  unit_rows(J, u % J->npg, &p0, &p1);
  const int64_t np = p1 - p0, V = V_of(d), rs = rot_stride(d);
  double* H = (double*)malloc((size_t)(np * r + 1) * sizeof(double));
  double* C = (double*)malloc((size_t)(np * r + 1) * sizeof(double));
  double* m2 = J->part[u];                       /* r*r partial */
  double* m1 = J->m1 + (chain * p + p0) * r;     /* disjoint rows */
  memset(m1, 0, (size_t)(np * r) * sizeof(double));
  init_rows(J, chain, p0, p1, H);
  for (int64_t t = 0; t < V; t++) {
    step_state(d, J->xhat, J->bhat, J->da, bi, hi, t, p0, p1, H);
    const double* pr = rs ? J->rot + ((bi * s + t) * h + hi) * rs : NULL;
    for (int64_t i = 0; i < np; i++) derotate_row(d, pr, H + i * r, C + i * r);
    for (int64_t i = 0; i < np; i++) {       /* m2 += C^T C over these rows */
      const double* Cr = C + i * r;
      for (int64_t a = 0; a < r; a++) {
        const double ca = Cr[a];
        double* row = m2 + a * r;
        for (int64_t v = 0; v < r; v++) row[v] += ca * Cr[v];
      }
    }
    for (int64_t i = 0; i < np * r; i++) m1[i] += C[i];
  }
  free(H);
  free(C);
}

static void bwd_unit(job_t* J, int64_t u) {
  const orc_desc* d = J->d;
  const int64_t p = d->p, r = d->r, c = d->c, h = d->h, s = d->s;
  const int64_t chain = J->chains[u / J->npg];
  const int64_t bi = chain / h, hi = chain % h;
  int64_t p0, p1;
  unit_rows(J, u % J->npg, &p0, &p1);
  const int64_t np = p1 - p0, V = V_of(d), rs = rot_stride(d), nb = n_blocks(d);
  const int bsz = block_size(d);
  const int64_t sz = np * r + 1;
  const int64_t nck = (V + CKPT - 1) / CKPT;
  /* partial layout: d_bhat [V, c, r] | d_rot [V, rs] | d_da [V] */
  double* part_db = J->part[u];
  double* part_dr = part_db + V * c * r;
  double* part_dd = part_dr + V * rs;

  double* S = (double*)malloc((size_t)(r * r) * sizeof(double));  /* dm2 + dm2^T */
  const double* dm2 = J->dm2 + chain * r * r;
  for (int64_t a = 0; a < r; a++)
    for (int64_t v = 0; v < r; v++) S[a * r + v] = dm2[a * r + v] + dm2[v * r + a];
  const double* dm1 = J->dm1 + (chain * p + p0) * r;

  double* ck = (double*)malloc((size_t)((nck > 0 ? nck : 1) * sz) * sizeof(double));
  double* H = (double*)malloc((size_t)sz * sizeof(double));
  init_rows(J, chain, p0, p1, H);
  for (int64_t t = 0; t < V; t++) {          /* ck[k] = state entering token k*CKPT */
    if (t % CKPT == 0) memcpy(ck + (t / CKPT) * sz, H, (size_t)sz * sizeof(double));
    step_state(d, J->xhat, J->bhat, J->da, bi, hi, t, p0, p1, H);
  }
  double* seg = (double*)malloc((size_t)((CKPT + 1) * sz) * sizeof(double));
  double* g = (double*)calloc((size_t)sz, sizeof(double));   /* exp(da_{t+1}) dH_{t+1} */
  double* C = (double*)malloc((size_t)sz * sizeof(double));
  double* dC = (double*)malloc((size_t)sz * sizeof(double));
  double* dH = (double*)malloc((size_t)sz * sizeof(double));
  double* tmp = (double*)malloc((size_t)r * sizeof(double));

  for (int64_t k = nck - 1; k >= 0; k--) {
    const int64_t t0 = k * CKPT, t1 = (t0 + CKPT < V) ? t0 + CKPT : V;
    memcpy(seg, ck + k * sz, (size_t)sz * sizeof(double));
    for (int64_t t = t0; t < t1; t++) {
      memcpy(seg + (t - t0 + 1) * sz, seg + (t - t0) * sz, (size_t)sz * sizeof(double));
      step_state(d, J->xhat, J->bhat, J->da, bi, hi, t, p0, p1, seg + (t - t0 + 1) * sz);
    }
    for (int64_t t = t1 - 1; t >= t0; t--) {
      const double* Hprev = seg + (t - t0) * sz;
      const double* Ht = seg + (t - t0 + 1) * sz;
      const double* pr = rs ? J->rot + ((bi * s + t) * h + hi) * rs : NULL;
      /* C_t = H_t M_t^T ; dC_t = C_t S + dm1 */
      for (int64_t i = 0; i < np; i++) derotate_row(d, pr, Ht + i * r, C + i * r);
      for (int64_t i = 0; i < np; i++) {
        const double* Cr = C + i * r;
        double* out = dC + i * r;
        for (int64_t v = 0; v < r; v++) out[v] = dm1[i * r + v];
        for (int64_t a = 0; a < r; a++) {
          const double ca = Cr[a];
          const double* Srow = S + a * r;
          for (int64_t v = 0; v < r; v++) out[v] += ca * Srow[v];
        }
      }
      /* dH = dC M_t + g  (row form: dh = M_t^T dc) */
      for (int64_t i = 0; i < np; i++) {
        derotate_row_T(d, pr, dC + i * r, tmp);
        for (int64_t v = 0; v < r; v++) dH[i * r + v] = tmp[v] + g[i * r + v];
      }
      /* rotation parameters: dM = dC^T H_t restricted to each block, contracted
       * with the block's derivative */
      if (nb > 0) {
        double* dr = part_dr + t * rs;
        int64_t idx[4];
        double dM[16], gm[16];
        for (int64_t kb = 0; kb < nb; kb++) {
          block_coords(d, kb, idx);
          for (int a = 0; a < bsz; a++)
            for (int v = 0; v < bsz; v++) {
              double acc = 0.0;
              for (int64_t i = 0; i < np; i++) acc += dC[i * r + idx[a]] * Ht[i * r + idx[v]];
              dM[a * bsz + v] = acc;
            }
          const int nq = (d->rot_kind == ORC_ROT_QUAT) ? 4 : 1;
          for (int q = 0; q < nq; q++) {
            block_dmatrix(d, pr, kb, q, gm);
            double acc = 0.0;
            for (int e = 0; e < bsz * bsz; e++) acc += dM[e] * gm[e];
            if (d->rot_kind == ORC_ROT_QUAT) dr[4 * kb + q] = acc;
            else dr[kb] = acc;
          }
        }
      }
      /* injections: d_xhat rows (disjoint) and the d_bhat partial over these rows */
      for (int64_t ci = 0; ci < c; ci++) {
        const int64_t row = ((bi * s + t) * c + ci) * h + hi;
        const double* x = J->xhat + row * p;
        const double* bb = J->bhat + row * r;
        if (J->dxhat) {
          double* dx = J->dxhat + row * p;
          for (int64_t i = 0; i < np; i++) {
            double acc = 0.0;
            for (int64_t v = 0; v < r; v++) acc += dH[i * r + v] * bb[v];
            dx[p0 + i] = acc;
          }
        }
        double* db = part_db + (t * c + ci) * r;
        for (int64_t v = 0; v < r; v++) db[v] = 0.0;
        for (int64_t i = 0; i < np; i++) {
          const double xv = x[p0 + i];
          for (int64_t v = 0; v < r; v++) db[v] += dH[i * r + v] * xv;
        }
      }
      /* decay: d_da_t = exp(da_t) <dH_t, H_{t-1}> */
      const double e = exp(J->da[(bi * s + t) * h + hi]);
      double acc = 0.0;
      for (int64_t i = 0; i < np * r; i++) acc += dH[i] * Hprev[i];
      part_dd[t] = e * acc;
      for (int64_t i = 0; i < np * r; i++) g[i] = e * dH[i];
    }
  }
  if (J->dh0) memcpy(J->dh0 + (chain * p + p0) * r, g, (size_t)(np * r) * sizeof(double));
  free(S); free(ck); free(H); free(seg); free(g); free(C); free(dC); free(dH); free(tmp);
}

/* ---- threading and reductions ------------------------------------------- */

typedef struct { job_t* J; int bwd; } worker_arg;

static void* worker(void* arg) {
  worker_arg* a = (worker_arg*)arg;
  job_t* J = a->J;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    const int64_t u = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (u >= J->nunits) break;
    if (a->bwd) bwd_unit(J, u);
    else fwd_unit(J, u);
  }
  return NULL;
}

static void run(job_t* J, int bwd, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > J->nunits) nthreads = (int)(J->nunits > 0 ? J->nunits : 1);
  pthread_mutex_init(&J->mu, NULL);
  J->next = 0;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  worker_arg wa = {J, bwd};
  for (int i = 1; i < nthreads; i++) pthread_create(&th[i], NULL, worker, &wa);
  worker(&wa);
  for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J->mu);
}

static int check_desc(const orc_desc* d) {
  if (d->b < 0 || d->s < 0 || d->c < 1 || d->h < 1 || d->p < 1 || d->r < 1) return -1;
  if (d->rot_kind == ORC_ROT_PAIRWISE || d->rot_kind == ORC_ROT_HALF) {
    if (d->rope_dim < 0 || d->rope_dim % 2 || d->rope_dim > d->r) return -1;
    if (d->rot_kind == ORC_ROT_HALF && (d->r % 2 || d->rope_dim / 2 > d->r / 2)) return -1;
  } else if (d->rot_kind == ORC_ROT_QUAT) {
    if (d->quat_blocks < 0 || 4 * d->quat_blocks > d->r) return -1;
  } else if (d->rot_kind != ORC_ROT_NONE) {
    return -1;
  }
  if (d->valid_len < 0) return -1;
  return 0;
}

static int setup(job_t* J, const int64_t* chains, int64_t nchains, int64_t npg, int64_t** all) {
  const orc_desc* d = J->d;
  *all = NULL;
  if (!chains) {
    nchains = d->b * d->h;
    *all = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nchains > 0 ? nchains : 1));
    for (int64_t i = 0; i < nchains; i++) (*all)[i] = i;
    chains = *all;
  }
  if (npg < 1) npg = 1;
  if (npg > d->p) npg = d->p;
  J->chains = chains;
  J->nchains = nchains;
  J->npg = npg;
  J->nunits = nchains * npg;
  return 0;
}

/* chains: flat (b*h + h) chain ids to compute (NULL = all); outputs of other
 * chains are left untouched. npg: state-row groups per chain (threading only;
 * results are the same for every npg up to fp64 summation order). */
int oracle_fwd(const orc_desc* d, const double* xhat, const double* bhat, const double* da,
               const double* rot, const double* h0, double* m2, double* m1,
               const int64_t* chains, int64_t nchains, int64_t npg, int nthreads) {
  if (check_desc(d)) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.d = d; J.xhat = xhat; J.bhat = bhat; J.da = da; J.rot = rot; J.h0 = h0;
  J.m2 = m2; J.m1 = m1;
  int64_t* all;
  setup(&J, chains, nchains, npg, &all);
  const int64_t r = d->r;
  J.part = (double**)malloc(sizeof(double*) * (size_t)(J.nunits + 1));
  for (int64_t u = 0; u < J.nunits; u++) J.part[u] = (double*)calloc((size_t)(r * r), sizeof(double));
  run(&J, 0, nthreads);
  for (int64_t i = 0; i < J.nchains; i++) {
    double* out = m2 + J.chains[i] * r * r;
    memset(out, 0, (size_t)(r * r) * sizeof(double));
    for (int64_t gi = 0; gi < J.npg; gi++) {
      const double* pp = J.part[i * J.npg + gi];
      for (int64_t e = 0; e < r * r; e++) out[e] += pp[e];
    }
  }
  for (int64_t u = 0; u < J.nunits; u++) free(J.part[u]);
  free(J.part);
  free(all);
  return 0;
}

/* Gradient buffers must be zero-filled by the caller: positions t >= V are
 * never written. d_rot may be NULL only when there is no rotation. */
int oracle_bwd(const orc_desc* d, const double* xhat, const double* bhat, const double* da,
               const double* rot, const double* h0, const double* dm2, const double* dm1,
               double* dxhat, double* dbhat, double* dda, double* drot, double* dh0,
               const int64_t* chains, int64_t nchains, int64_t npg, int nthreads) {
  if (check_desc(d)) return -1;
  job_t J;
  memset(&J, 0, sizeof(J));
  J.d = d; J.xhat = xhat; J.bhat = bhat; J.da = da; J.rot = rot; J.h0 = h0;
  J.dm2 = dm2; J.dm1 = dm1;
  J.dxhat = dxhat; J.dbhat = dbhat; J.dda = dda; J.drot = drot; J.dh0 = dh0;
  int64_t* all;
  setup(&J, chains, nchains, npg, &all);
  const int64_t V = V_of(d), c = d->c, r = d->r, h = d->h, s = d->s, rs = rot_stride(d);
  const int64_t psz = V * c * r + V * rs + V + 1;
  J.part = (double**)malloc(sizeof(double*) * (size_t)(J.nunits + 1));
  for (int64_t u = 0; u < J.nunits; u++) J.part[u] = (double*)calloc((size_t)psz, sizeof(double));
  run(&J, 1, nthreads);
  for (int64_t i = 0; i < J.nchains; i++) {
    const int64_t chain = J.chains[i], bi = chain / h, hi = chain % h;
    for (int64_t gi = 0; gi < J.npg; gi++) {
      const double* pdb = J.part[i * J.npg + gi];
      const double* pdr = pdb + V * c * r;
      const double* pdd = pdr + V * rs;
      for (int64_t t = 0; t < V; t++) {
        if (dbhat)
          for (int64_t ci = 0; ci < c; ci++) {
            double* db = dbhat + (((bi * s + t) * c + ci) * h + hi) * r;
            const double* src = pdb + (t * c + ci) * r;
            for (int64_t v = 0; v < r; v++) db[v] += src[v];
          }
        if (drot && rs) {
          double* dr = drot + ((bi * s + t) * h + hi) * rs;
          for (int64_t e = 0; e < rs; e++) dr[e] += pdr[t * rs + e];
        }
        if (dda) dda[(bi * s + t) * h + hi] += pdd[t];
      }
    }
  }
  for (int64_t u = 0; u < J.nunits; u++) free(J.part[u]);
  free(J.part);
  free(all);
  return 0;
}

/*
 * sinkstate_oracle.c -- plain fp64 CPU oracle for factored recurrent states.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (all citations are to "SinkState: On-the-Fly SVD of
 * Recurrent States for Efficient Hybrid LLM Serving", arXiv 2611.14246, and to
 * "Shallow Encoding Emits Deep Memories", arXiv 2611.06084):
 *
 *   state     S = sum_i sigma_i u_i v_i^T + sum_j c_j k_j w_j^T      (d_k x d_v)
 *             with factors (u_i, v_i, sigma_i) sorted by sigma, the first
 *             min(r, R) of them "active", the rest "frozen" (SinkState, 3.2
 *             Design 1), and a pad of buffered (k_j, w_j, c_j)
 *             (SinkState, 4.2 "(i) Buffering", Figure 6(b)).
 *   decode    every sigma and every pad weight is multiplied by alpha, the
 *             token's pair is appended with weight 1, and o = S^T q is read
 *             after the update (SinkState, 4.2 "(i) Buffering"; 2.1 recurrence).
 *             Scalar rule (Mamba-2): w = v.  Delta rule (Gated DeltaNet,
 *             SEED section 2 eq. (2)):  S_t = a (I - b k k^T) S_{t-1} + b k v^T,
 *             which is S_t = a S_{t-1} + k w^T with w = b (v - a S_{t-1}^T k).
 *   compact   Brand's local SVD of the active part plus the pad, merge with
 *             the frozen part, drop sigma < eps * sigma_max, re-split
 *             (SinkState, 4.2 "(ii) Top-subspace SVD", Figure 6(b) step 3).
 *   dense     states whose rank exceeds floor(d_k d_v / (d_k + d_v)) are held
 *             as a dense matrix (SinkState, 4.4 "Memory layout").
 *   init      randomized block SVD of a dense state after prefill
 *             (SinkState, 4.2 "Randomized SVD initialization after prefill").
 *   consolidate  exact SVD of the frozen part, drop sigma < eps * sigma_0
 *             (SinkState, 4.3 "Asynchronous CPU Consolidation", Figure 7(a)).
 *   fp16      optional fp16 factor storage (SEED, section 6 "Lower precision
 *             composes"): every factor vector written (initial factors,
 *             compaction and consolidation results) is rounded to binary16;
 *             sigma and the pad keep full precision.
 *   diag      optional per-channel decay (Kimi Delta Attention; SEED
 *             appendix B.1 eq. (6): S_t = (I - theta b k k^T) Lambda S_{t-1}
 *             + b k v^T with Lambda = diag(lambda_1..lambda_dk)).  Written as
 *             S_t = Lambda S_{t-1} + k w^T with w = b (v - S_{t-1}^T Lambda k)
 *             (delta rule) or w = v (scalar rule).  Applied literally: every
 *             factor u_i and every pad key is multiplied by Lambda each step
 *             (SEED Lemma 2: U+ = [Lambda U, k]); at a compaction the frozen
 *             components are renormalized (sigma_f <- sigma_f |u_f|,
 *             u_f <- u_f / |u_f|) and re-sorted before the merge.
 *
 * Decay is applied literally, every step, to every sigma and pad weight.  QR
 * is Householder, the small SVD is cyclic one-sided (Hestenes) Jacobi, both
 * written from the textbook definitions.  Storage: per state, growable heap
 * arrays; components are rows (u_i is U + i*d_k).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_SCALAR = 0, ORC_DELTA = 1 };

typedef struct {
  int R;        /* components, sigma descending; first min(r, R) active */
  int cap;      /* allocated component slots */
  double *U;    /* cap x d_k */
  double *V;    /* cap x d_v */
  double *sig;  /* cap */
  int n;        /* filled pad slots */
  double *PK;   /* K x d_k */
  double *PW;   /* K x d_v */
  double *pc;   /* K */
  int dense;
  double *S;    /* d_k x d_v row-major when dense */
  int rule;
  double eps;
  double bound;      /* open-loop error bound, SEED Prop. 3 */
  int64_t compactions;
} orc_state;

typedef struct {
  int64_t N;
  int d_k, d_v, K, r, L, promote;
  int fp16;     /* factor vectors stored in fp16: rounded whenever they are written */
  int diag;     /* per-channel decay: alpha is [N][d_k] */
  orc_state *st;
} orc_pool;

/* ------------------------------------------------------------------ */
/* small helpers                                                        */
/* ------------------------------------------------------------------ */
static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/* IEEE 754 binary16 rounding of x, round to nearest with ties to even
 * (11-bit significand; normal exponents -14..15, subnormal step 2^-24;
 * magnitudes that round to 2^16 or above become infinite).  Used for fp16
 * factor storage (SEED section 6: fp16 factors with an fp32 pad). */
double orc_round_fp16(double x) {
  if (x == 0.0 || x != x) return x;
  double a = fabs(x);
  if (a >= 65520.0) return x > 0 ? INFINITY : -INFINITY;
  int e;
  frexp(a, &e);               /* a = m 2^e, m in [0.5, 1): the leading bit is 2^(e-1) */
  int q = e - 11;             /* quantum 2^(e-1-10) */
  if (q < -24) q = -24;       /* subnormal range */
  double y = ldexp(a, -q);    /* exact: a power-of-two scaling */
  double f = floor(y), r = y - f;
  if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
  double out = ldexp(f, q);
  return x < 0 ? -out : out;
}

static void round_rows(double *A, size_t n) {
  for (size_t i = 0; i < n; ++i) A[i] = orc_round_fp16(A[i]);
}

void orc_set_factor_fp16(orc_pool *p, int on) { p->fp16 = on ? 1 : 0; }
void orc_set_diag_decay(orc_pool *p, int on) { p->diag = on ? 1 : 0; }

static int ensure_cap(orc_state *s, int need, int d_k, int d_v) {
  if (need <= s->cap) return 0;
  int cap = need + 16;
  double *U = (double *)realloc(s->U, (size_t)cap * d_k * sizeof(double));
  if (!U) return -1;
  s->U = U;
  double *V = (double *)realloc(s->V, (size_t)cap * d_v * sizeof(double));
  if (!V) return -1;
  s->V = V;
  double *g = (double *)realloc(s->sig, (size_t)cap * sizeof(double));
  if (!g) return -1;
  s->sig = g;
  s->cap = cap;
  return 0;
}

/* ------------------------------------------------------------------ */
/* Householder thin QR.  A is d x m column-major (column j at A + j*d).  */
/* Produces Q (d x p, column-major, orthonormal columns) and R (p x m,   */
/* column-major, upper trapezoidal) with p = min(d, m) and A = Q R.      */
/* Textbook reflectors H = I - 2 v v^T / (v^T v).                        */
/* ------------------------------------------------------------------ */
int orc_householder_qr(int d, int m, const double *A, double *Q, double *R) {
  int p = d < m ? d : m;
  double *W = (double *)malloc((size_t)d * m * sizeof(double));
  double *Vh = (double *)calloc((size_t)d * (p > 0 ? p : 1), sizeof(double));
  double *vn = (double *)calloc((size_t)(p > 0 ? p : 1), sizeof(double));
  if (!W || !Vh || !vn) { free(W); free(Vh); free(vn); return -1; }
  memcpy(W, A, (size_t)d * m * sizeof(double));
  for (int j = 0; j < p; ++j) {
    double *x = W + (size_t)j * d + j; /* column j, rows j.. */
    int len = d - j;
    double nx = sqrt(dot(x, x, len));
    double alpha = (x[0] >= 0.0) ? -nx : nx;
    double *v = Vh + (size_t)j * d + j;
    for (int i = 0; i < len; ++i) v[i] = x[i];
    v[0] -= alpha;
    double vv = dot(v, v, len);
    vn[j] = vv;
    if (vv == 0.0) continue; /* column already zero below the diagonal */
    for (int c = j; c < m; ++c) {
      double *col = W + (size_t)c * d + j;
      double f = 2.0 * dot(v, col, len) / vv;
      for (int i = 0; i < len; ++i) col[i] -= f * v[i];
    }
  }
  /* R: rows 0..p-1 of W, upper part */
  for (int c = 0; c < m; ++c)
    for (int i = 0; i < p; ++i) R[(size_t)c * p + i] = (i <= c) ? W[(size_t)c * d + i] : 0.0;
  /* Q = H_0 H_1 ... H_{p-1} [I_p; 0] */
  for (int c = 0; c < p; ++c)
    for (int i = 0; i < d; ++i) Q[(size_t)c * d + i] = (i == c) ? 1.0 : 0.0;
  for (int j = p - 1; j >= 0; --j) {
    if (vn[j] == 0.0) continue;
    const double *v = Vh + (size_t)j * d + j;
    int len = d - j;
    for (int c = 0; c < p; ++c) {
      double *col = Q + (size_t)c * d + j;
      double f = 2.0 * dot(v, col, len) / vn[j];
      for (int i = 0; i < len; ++i) col[i] -= f * v[i];
    }
  }
  free(W); free(Vh); free(vn);
  return p;
}

/* ------------------------------------------------------------------ */
/* One-sided (Hestenes) Jacobi SVD, cyclic pair order.                  */
/* A is rows x cols column-major.  On return: s[cols] descending,       */
/* Uo (rows x cols, column-major; zero column where s == 0) and          */
/* Vo (cols x cols, column-major, orthogonal) with A = Uo diag(s) Vo^T.   */
/* Each rotation makes columns i and j orthogonal:                      */
/*   zeta = (|a_j|^2 - |a_i|^2) / (2 a_i.a_j),                           */
/*   t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), c = 1/sqrt(1+t^2),   */
/*   [a_i a_j] <- [a_i a_j] [[c, s], [-s, c]] with s = c t.              */
/* ------------------------------------------------------------------ */
int orc_jacobi_svd(int rows, int cols, const double *A, double *Uo, double *s, double *Vo) {
  double *W = (double *)malloc((size_t)rows * cols * sizeof(double) + 8);
  double *J = (double *)malloc((size_t)cols * cols * sizeof(double) + 8);
  double *sv = (double *)malloc((size_t)cols * sizeof(double) + 8);
  int *ord = (int *)malloc((size_t)cols * sizeof(int) + 8);
  if (!W || !J || !sv || !ord) { free(W); free(J); free(sv); free(ord); return -1; }
  memcpy(W, A, (size_t)rows * cols * sizeof(double));
  for (int c = 0; c < cols; ++c)
    for (int i = 0; i < cols; ++i) J[(size_t)c * cols + i] = (i == c) ? 1.0 : 0.0;
  const double tol = 1e-15;
  int sweeps = 0;
  for (; sweeps < 100; ++sweeps) {
    int rotated = 0;
    for (int i = 0; i < cols - 1; ++i) {
      for (int j = i + 1; j < cols; ++j) {
        double *ai = W + (size_t)i * rows, *aj = W + (size_t)j * rows;
        double a = dot(ai, ai, rows), b = dot(aj, aj, rows), g = dot(ai, aj, rows);
        if (g == 0.0 || fabs(g) <= tol * sqrt(a * b)) continue;
        double zeta = (b - a) / (2.0 * g);
        double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        double c = 1.0 / sqrt(1.0 + t * t), sn = c * t;
        for (int r = 0; r < rows; ++r) {
          double x = ai[r], y = aj[r];
          ai[r] = c * x - sn * y;
          aj[r] = sn * x + c * y;
        }
        double *ji = J + (size_t)i * cols, *jj = J + (size_t)j * cols;
        for (int r = 0; r < cols; ++r) {
          double x = ji[r], y = jj[r];
          ji[r] = c * x - sn * y;
          jj[r] = sn * x + c * y;
        }
        rotated = 1;
      }
    }
    if (!rotated) break;
  }
  for (int c = 0; c < cols; ++c) {
    sv[c] = sqrt(dot(W + (size_t)c * rows, W + (size_t)c * rows, rows));
    ord[c] = c;
  }
  /* stable insertion sort, descending */
  for (int a = 1; a < cols; ++a) {
    int x = ord[a], b = a - 1;
    while (b >= 0 && sv[ord[b]] < sv[x]) { ord[b + 1] = ord[b]; --b; }
    ord[b + 1] = x;
  }
  for (int c = 0; c < cols; ++c) {
    int src = ord[c];
    s[c] = sv[src];
    for (int r = 0; r < rows; ++r)
      Uo[(size_t)c * rows + r] = sv[src] > 0.0 ? W[(size_t)src * rows + r] / sv[src] : 0.0;
    for (int r = 0; r < cols; ++r) Vo[(size_t)c * cols + r] = J[(size_t)src * cols + r];
  }
  free(W); free(J); free(sv); free(ord);
  return sweeps;
}

/* ------------------------------------------------------------------ */
/* Brand's update (SinkState 4.2 (ii)): given U_C (d_k x m), V_C        */
/* (d_v x m) column-major and weights sc[m], returns the SVD of          */
/* U_C diag(sc) V_C^T as Uo (d_k x pr), Vo (d_v x pr), so[pr], sorted.    */
/*   U_C = Q_L R_L,  V_C = Q_R R_R,  C = R_L diag(sc) R_R^T,             */
/*   C = Uh diag(so) Vh^T,  Uo = Q_L Uh,  Vo = Q_R Vh.                    */
/* Returns pr (= min(d_v, m)), or -1 on allocation failure.              */
/* ------------------------------------------------------------------ */
int orc_brand(int d_k, int d_v, int m, const double *UC, const double *VC, const double *sc,
              double *Uo, double *Vo, double *so) {
  int pl = d_k < m ? d_k : m, pr = d_v < m ? d_v : m;
  if (m == 0) return 0;
  double *QL = (double *)malloc((size_t)d_k * pl * sizeof(double));
  double *RL = (double *)malloc((size_t)pl * m * sizeof(double));
  double *QR = (double *)malloc((size_t)d_v * pr * sizeof(double));
  double *RR = (double *)malloc((size_t)pr * m * sizeof(double));
  double *C = (double *)malloc((size_t)pl * pr * sizeof(double));
  double *Uh = (double *)malloc((size_t)pl * pr * sizeof(double));
  double *Vh = (double *)malloc((size_t)pr * pr * sizeof(double));
  int ok = QL && RL && QR && RR && C && Uh && Vh;
  if (ok) {
    orc_householder_qr(d_k, m, UC, QL, RL);
    orc_householder_qr(d_v, m, VC, QR, RR);
    /* C[i][j] = sum_t RL[i][t] sc[t] RR[j][t]  (column-major: C + j*pl + i) */
    for (int j = 0; j < pr; ++j)
      for (int i = 0; i < pl; ++i) {
        double acc = 0.0;
        for (int t = 0; t < m; ++t) acc += RL[(size_t)t * pl + i] * sc[t] * RR[(size_t)t * pr + j];
        C[(size_t)j * pl + i] = acc;
      }
    if (orc_jacobi_svd(pl, pr, C, Uh, so, Vh) < 0) ok = 0;
  }
  if (ok) {
    for (int c = 0; c < pr; ++c) {
      for (int i = 0; i < d_k; ++i) {
        double acc = 0.0;
        for (int t = 0; t < pl; ++t) acc += QL[(size_t)t * d_k + i] * Uh[(size_t)c * pl + t];
        Uo[(size_t)c * d_k + i] = acc;
      }
      for (int i = 0; i < d_v; ++i) {
        double acc = 0.0;
        for (int t = 0; t < pr; ++t) acc += QR[(size_t)t * d_v + i] * Vh[(size_t)c * pr + t];
        Vo[(size_t)c * d_v + i] = acc;
      }
    }
  }
  free(QL); free(RL); free(QR); free(RR); free(C); free(Uh); free(Vh);
  return ok ? pr : -1;
}

/* ------------------------------------------------------------------ */
/* pool                                                                 */
/* ------------------------------------------------------------------ */
orc_pool *orc_create(int64_t N, int d_k, int d_v, int K, int r, int L, int promote) {
  if (N < 0 || d_k <= 0 || d_v <= 0 || K <= 0 || r <= 0) return NULL;
  orc_pool *p = (orc_pool *)calloc(1, sizeof(orc_pool));
  if (!p) return NULL;
  p->N = N; p->d_k = d_k; p->d_v = d_v; p->K = K; p->r = r;
  p->L = L < 0 ? (d_k * d_v) / (d_k + d_v) : L;
  p->promote = promote;
  p->st = (orc_state *)calloc((size_t)(N > 0 ? N : 1), sizeof(orc_state));
  if (!p->st) { free(p); return NULL; }
  for (int64_t s = 0; s < N; ++s) {
    orc_state *x = &p->st[s];
    x->PK = (double *)calloc((size_t)K * d_k, sizeof(double));
    x->PW = (double *)calloc((size_t)K * d_v, sizeof(double));
    x->pc = (double *)calloc((size_t)K, sizeof(double));
    if (!x->PK || !x->PW || !x->pc) return NULL;
  }
  return p;
}

void orc_destroy(orc_pool *p) {
  if (!p) return;
  for (int64_t s = 0; s < p->N; ++s) {
    orc_state *x = &p->st[s];
    free(x->U); free(x->V); free(x->sig); free(x->PK); free(x->PW); free(x->pc); free(x->S);
  }
  free(p->st);
  free(p);
}

int orc_dense_limit(const orc_pool *p) { return p->L; }

static int make_dense(orc_pool *p, orc_state *x) {
  int dk = p->d_k, dv = p->d_v;
  double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
  if (!S) return -1;
  for (int i = 0; i < x->R; ++i)
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) S[(size_t)a * dv + b] += x->sig[i] * x->U[(size_t)i * dk + a] * x->V[(size_t)i * dv + b];
  for (int j = 0; j < x->n; ++j)
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) S[(size_t)a * dv + b] += x->pc[j] * x->PK[(size_t)j * dk + a] * x->PW[(size_t)j * dv + b];
  free(x->S);
  x->S = S;
  x->dense = 1;
  x->R = 0;
  x->n = 0;
  return 0;
}

/* Set one state.  Components are given as rows.  With as_init set they are
 * sorted by sigma (descending, stable), and a factored state given with
 * R > L falls back to the dense form (SinkState 4.4: the dense test is made
 * once the initial factors exist).  Without it the state is loaded as given,
 * e.g. to continue from a state taken in the middle of a run: the first
 * min(r, R) components stay the active part and the rest the frozen part,
 * each sorted on its own (after a consolidation, SinkState 4.3, the frozen
 * list can start above the last active value). */
int orc_set_state(orc_pool *p, int64_t s, int rule, double eps, int R, const double *U, const double *V,
                  const double *sig, int n, const double *PK, const double *PW, const double *pc, int dense,
                  const double *S, int as_init) {
  if (!p || s < 0 || s >= p->N || R < 0 || n < 0 || n > p->K) return -1;
  int dk = p->d_k, dv = p->d_v;
  orc_state *x = &p->st[s];
  x->rule = rule;
  x->eps = eps;
  x->bound = 0.0;
  x->compactions = 0;
  free(x->S);
  x->S = NULL;
  x->dense = 0;
  x->R = 0;
  x->n = 0;
  if (dense) {
    x->S = (double *)malloc((size_t)dk * dv * sizeof(double));
    if (!x->S) return -1;
    memcpy(x->S, S, (size_t)dk * dv * sizeof(double));
    x->dense = 1;
    return 0;
  }
  if (ensure_cap(x, R, dk, dv)) return -1;
  int *ord = (int *)malloc((size_t)(R > 0 ? R : 1) * sizeof(int));
  if (!ord) return -1;
  for (int i = 0; i < R; ++i) ord[i] = i;
  int split = as_init ? R : (R < p->r ? R : p->r);
  for (int part = 0; part < 2; ++part) {
    int lo = part == 0 ? 0 : split, hi = part == 0 ? split : R;
    for (int a = lo + 1; a < hi; ++a) {
      int t = ord[a], b = a - 1;
      while (b >= lo && sig[ord[b]] < sig[t]) { ord[b + 1] = ord[b]; --b; }
      ord[b + 1] = t;
    }
  }
  for (int i = 0; i < R; ++i) {
    memcpy(x->U + (size_t)i * dk, U + (size_t)ord[i] * dk, dk * sizeof(double));
    memcpy(x->V + (size_t)i * dv, V + (size_t)ord[i] * dv, dv * sizeof(double));
    x->sig[i] = sig[ord[i]];
  }
  free(ord);
  x->R = R;
  if (p->fp16 && as_init) {  /* initial factors are written in fp16; a mid-run state is taken as given
                                (with per-channel decay its u carry the decays since the last compaction) */
    round_rows(x->U, (size_t)R * dk);
    round_rows(x->V, (size_t)R * dv);
  }
  for (int j = 0; j < n; ++j) {
    memcpy(x->PK + (size_t)j * dk, PK + (size_t)j * dk, dk * sizeof(double));
    memcpy(x->PW + (size_t)j * dv, PW + (size_t)j * dv, dv * sizeof(double));
    x->pc[j] = pc[j];
  }
  x->n = n;
  if (as_init && x->R > p->L) return make_dense(p, x);
  return 0;
}

int orc_get_sizes(const orc_pool *p, int64_t s, int *R, int *n, int *dense, int *rule, double *eps) {
  if (!p || s < 0 || s >= p->N) return -1;
  const orc_state *x = &p->st[s];
  *R = x->R; *n = x->n; *dense = x->dense; *rule = x->rule; *eps = x->eps;
  return 0;
}

/* Copies out the stored representation; pointers may be NULL to skip. */
int orc_get_state(const orc_pool *p, int64_t s, double *U, double *V, double *sig, double *PK, double *PW,
                  double *pc, double *S) {
  if (!p || s < 0 || s >= p->N) return -1;
  const orc_state *x = &p->st[s];
  int dk = p->d_k, dv = p->d_v;
  if (x->dense) {
    if (S) memcpy(S, x->S, (size_t)dk * dv * sizeof(double));
    return 0;
  }
  if (U) memcpy(U, x->U, (size_t)x->R * dk * sizeof(double));
  if (V) memcpy(V, x->V, (size_t)x->R * dv * sizeof(double));
  if (sig) memcpy(sig, x->sig, (size_t)x->R * sizeof(double));
  if (PK) memcpy(PK, x->PK, (size_t)x->n * dk * sizeof(double));
  if (PW) memcpy(PW, x->PW, (size_t)x->n * dv * sizeof(double));
  if (pc) memcpy(pc, x->pc, (size_t)x->n * sizeof(double));
  return 0;
}

double orc_get_bound(const orc_pool *p, int64_t s) { return p->st[s].bound; }
int64_t orc_get_compactions(const orc_pool *p, int64_t s) { return p->st[s].compactions; }

/* S~ as a dense d_k x d_v matrix (row-major): sum of components plus pad. */
int orc_reconstruct(const orc_pool *p, int64_t s, double *out) {
  if (!p || s < 0 || s >= p->N) return -1;
  const orc_state *x = &p->st[s];
  int dk = p->d_k, dv = p->d_v;
  if (x->dense) {
    memcpy(out, x->S, (size_t)dk * dv * sizeof(double));
    return 0;
  }
  memset(out, 0, (size_t)dk * dv * sizeof(double));
  for (int i = 0; i < x->R; ++i)
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) out[(size_t)a * dv + b] += x->sig[i] * x->U[(size_t)i * dk + a] * x->V[(size_t)i * dv + b];
  for (int j = 0; j < x->n; ++j)
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) out[(size_t)a * dv + b] += x->pc[j] * x->PK[(size_t)j * dk + a] * x->PW[(size_t)j * dv + b];
  return 0;
}

/* S~^T x from the factors and the pad (no dense matrix is formed). */
static void factored_apply_t(const orc_pool *p, const orc_state *x, const double *vec, double *out) {
  int dk = p->d_k, dv = p->d_v;
  for (int b = 0; b < dv; ++b) out[b] = 0.0;
  for (int i = 0; i < x->R; ++i) {
    double c = x->sig[i] * dot(x->U + (size_t)i * dk, vec, dk);
    for (int b = 0; b < dv; ++b) out[b] += c * x->V[(size_t)i * dv + b];
  }
  for (int j = 0; j < x->n; ++j) {
    double c = x->pc[j] * dot(x->PK + (size_t)j * dk, vec, dk);
    for (int b = 0; b < dv; ++b) out[b] += c * x->PW[(size_t)j * dv + b];
  }
}

static void dense_apply_t(const orc_pool *p, const double *S, const double *vec, double *out) {
  int dk = p->d_k, dv = p->d_v;
  for (int b = 0; b < dv; ++b) out[b] = 0.0;
  for (int a = 0; a < dk; ++a)
    for (int b = 0; b < dv; ++b) out[b] += S[(size_t)a * dv + b] * vec[a];
}

/* One decode step of one state: returns 0, or -2 if the pad is full (the
 * caller's compaction schedule missed this state). */
/* One decode step with per-channel decay lam[0..d_k-1] (Kimi Delta Attention,
 * SEED appendix B.1 eq. (6)), applied literally; tmp holds d_k doubles. */
static int decode_one_diag(orc_pool *p, orc_state *x, const double *q, const double *k, const double *v,
                           const double *lam, double beta, double *o, double *w, double *tmp) {
  int dk = p->d_k, dv = p->d_v;
  double lmax = 0.0;
  for (int a = 0; a < dk; ++a) lmax = lam[a] > lmax ? lam[a] : lmax;
  if (x->dense) {
    if (x->rule == ORC_DELTA) {
      for (int a = 0; a < dk; ++a) tmp[a] = lam[a] * k[a];
      dense_apply_t(p, x->S, tmp, w); /* S_{t-1}^T Lambda k */
      for (int b = 0; b < dv; ++b) w[b] = beta * (v[b] - w[b]);
    } else {
      for (int b = 0; b < dv; ++b) w[b] = v[b];
    }
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) x->S[(size_t)a * dv + b] = lam[a] * x->S[(size_t)a * dv + b] + k[a] * w[b];
    dense_apply_t(p, x->S, q, o);
    x->bound *= lmax;
    return 0;
  }
  if (x->n >= p->K) return -2;
  /* Lambda S~: every u_i and every pad key, channel by channel */
  for (int i = 0; i < x->R; ++i)
    for (int a = 0; a < dk; ++a) x->U[(size_t)i * dk + a] *= lam[a];
  for (int j = 0; j < x->n; ++j)
    for (int a = 0; a < dk; ++a) x->PK[(size_t)j * dk + a] *= lam[a];
  if (x->rule == ORC_DELTA) {
    factored_apply_t(p, x, k, w); /* (Lambda S~_{t-1})^T k = S~_{t-1}^T Lambda k */
    for (int b = 0; b < dv; ++b) w[b] = beta * (v[b] - w[b]);
  } else {
    for (int b = 0; b < dv; ++b) w[b] = v[b];
  }
  memcpy(x->PK + (size_t)x->n * dk, k, dk * sizeof(double));
  memcpy(x->PW + (size_t)x->n * dv, w, dv * sizeof(double));
  x->pc[x->n] = 1.0;
  x->n += 1;
  factored_apply_t(p, x, q, o);
  x->bound *= lmax;
  return 0;
}

static int decode_one(orc_pool *p, orc_state *x, const double *q, const double *k, const double *v, double alpha,
                      double beta, double *o, double *w) {
  int dk = p->d_k, dv = p->d_v;
  if (x->dense) {
    if (x->rule == ORC_DELTA) {
      dense_apply_t(p, x->S, k, w); /* S_{t-1}^T k */
      for (int b = 0; b < dv; ++b) w[b] = beta * (v[b] - alpha * w[b]);
    } else {
      for (int b = 0; b < dv; ++b) w[b] = v[b];
    }
    for (int a = 0; a < dk; ++a)
      for (int b = 0; b < dv; ++b) x->S[(size_t)a * dv + b] = alpha * x->S[(size_t)a * dv + b] + k[a] * w[b];
    dense_apply_t(p, x->S, q, o);
    x->bound *= alpha;
    return 0;
  }
  if (x->n >= p->K) return -2;
  if (x->rule == ORC_DELTA) {
    factored_apply_t(p, x, k, w); /* S~_{t-1}^T k read from the factors */
    for (int b = 0; b < dv; ++b) w[b] = beta * (v[b] - alpha * w[b]);
  } else {
    for (int b = 0; b < dv; ++b) w[b] = v[b];
  }
  for (int i = 0; i < x->R; ++i) x->sig[i] *= alpha;
  for (int j = 0; j < x->n; ++j) x->pc[j] *= alpha;
  memcpy(x->PK + (size_t)x->n * dk, k, dk * sizeof(double));
  memcpy(x->PW + (size_t)x->n * dv, w, dv * sizeof(double));
  x->pc[x->n] = 1.0;
  x->n += 1;
  factored_apply_t(p, x, q, o);
  x->bound *= alpha;
  return 0;
}

/* All states, one step.  Inputs are [N][d] row-major; beta may be NULL when
 * no state uses the delta rule; alpha is [N], or [N][d_k] in a pool with
 * per-channel decay.  Returns 0 or the number of states whose pad was already
 * full (their step is skipped). */
int64_t orc_decode(orc_pool *p, const double *q, const double *k, const double *v, const double *alpha,
                   const double *beta, double *o, int nthreads) {
  int64_t bad = 0;
  int dk = p->d_k, dv = p->d_v;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads) reduction(+ : bad)
#endif
  for (int64_t s = 0; s < p->N; ++s) {
    double w[1024], tmp[1024];
    double b = beta ? beta[s] : 0.0;
    int rc = p->diag ? decode_one_diag(p, &p->st[s], q + s * dk, k + s * dk, v + s * dv, alpha + s * dk, b,
                                       o + s * dv, w, tmp)
                     : decode_one(p, &p->st[s], q + s * dk, k + s * dk, v + s * dv, alpha[s], b, o + s * dv, w);
    if (rc) bad += 1;
  }
  (void)nthreads;
  return bad;
}

int orc_readout(const orc_pool *p, const double *q, double *o, int nthreads) {
  int dk = p->d_k, dv = p->d_v;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
  for (int64_t s = 0; s < p->N; ++s) {
    const orc_state *x = &p->st[s];
    if (x->dense)
      dense_apply_t(p, x->S, q + s * dk, o + s * dv);
    else
      factored_apply_t(p, x, q + s * dk, o + s * dv);
  }
  (void)nthreads;
  return 0;
}

/* Compaction of one state (SinkState 4.2 (ii), Figure 6(b) step 3):
 *  1. active = first min(r, R) components; frozen = the rest;
 *  2. U_C = [U_active | pad keys], V_C = [V_active | pad w's],
 *     Sigma_C = diag(sigma_active, pad weights);
 *  3. Brand: QR both sides, SVD of the small core, rotate back;
 *  4. merge with the frozen components in descending sigma order (ties:
 *     the local result first), drop sigma < eps * sigma_max and sigma = 0;
 *  5. the merged list becomes the component list (its first r are the next
 *     active part), the pad is emptied;
 *  6. with promotion on, a state left with more than L components is
 *     re-stored dense (the memory test of SinkState 4.4, applied again).
 * An empty pad leaves the state unchanged. */
/* Per-channel decay leaves the frozen u_f scaled by Lambda: give them unit
 * norm again (sigma takes the norm; a zero vector gets sigma 0 and is
 * dropped by the merge) and sort the frozen part by the new sigma,
 * descending, equal values in their stored order (insertion sort). */
static void renormalize_frozen(orc_pool *p, orc_state *x, int ra) {
  int dk = p->d_k, dv = p->d_v;
  for (int f = ra; f < x->R; ++f) {
    double *u = x->U + (size_t)f * dk;
    double nrm = sqrt(dot(u, u, dk));
    if (nrm > 0.0) {
      for (int a = 0; a < dk; ++a) u[a] /= nrm;
      x->sig[f] *= nrm;
    } else {
      x->sig[f] = 0.0;
    }
  }
  double *tu = (double *)malloc((size_t)dk * sizeof(double));
  double *tv = (double *)malloc((size_t)dv * sizeof(double));
  if (!tu || !tv) { free(tu); free(tv); return; }
  for (int f = ra + 1; f < x->R; ++f) {
    double sg = x->sig[f];
    memcpy(tu, x->U + (size_t)f * dk, dk * sizeof(double));
    memcpy(tv, x->V + (size_t)f * dv, dv * sizeof(double));
    int g = f;
    while (g > ra && x->sig[g - 1] < sg) {
      x->sig[g] = x->sig[g - 1];
      memcpy(x->U + (size_t)g * dk, x->U + (size_t)(g - 1) * dk, dk * sizeof(double));
      memcpy(x->V + (size_t)g * dv, x->V + (size_t)(g - 1) * dv, dv * sizeof(double));
      --g;
    }
    x->sig[g] = sg;
    memcpy(x->U + (size_t)g * dk, tu, dk * sizeof(double));
    memcpy(x->V + (size_t)g * dv, tv, dv * sizeof(double));
  }
  free(tu);
  free(tv);
}

static int compact_one(orc_pool *p, orc_state *x) {
  int dk = p->d_k, dv = p->d_v;
  if (x->dense || x->n == 0) return 0;
  int ra = x->R < p->r ? x->R : p->r;
  if (p->diag) renormalize_frozen(p, x, ra);
  int m = ra + x->n;
  int pr = dv < m ? dv : m;
  int nf = x->R - ra;
  int total = pr + nf;
  double *UC = (double *)malloc((size_t)dk * m * sizeof(double));
  double *VC = (double *)malloc((size_t)dv * m * sizeof(double));
  double *sc = (double *)malloc((size_t)m * sizeof(double));
  double *Ul = (double *)malloc((size_t)dk * pr * sizeof(double));
  double *Vl = (double *)malloc((size_t)dv * pr * sizeof(double));
  double *sl = (double *)malloc((size_t)pr * sizeof(double));
  double *nU = (double *)malloc((size_t)(total > 0 ? total : 1) * dk * sizeof(double));
  double *nV = (double *)malloc((size_t)(total > 0 ? total : 1) * dv * sizeof(double));
  double *ns = (double *)malloc((size_t)(total > 0 ? total : 1) * sizeof(double));
  double *E = (double *)calloc((size_t)dk * dv, sizeof(double));
  int rc = -1;
  if (!UC || !VC || !sc || !Ul || !Vl || !sl || !nU || !nV || !ns || !E) goto done;
  for (int i = 0; i < ra; ++i) {
    memcpy(UC + (size_t)i * dk, x->U + (size_t)i * dk, dk * sizeof(double));
    memcpy(VC + (size_t)i * dv, x->V + (size_t)i * dv, dv * sizeof(double));
    sc[i] = x->sig[i];
  }
  for (int j = 0; j < x->n; ++j) {
    memcpy(UC + (size_t)(ra + j) * dk, x->PK + (size_t)j * dk, dk * sizeof(double));
    memcpy(VC + (size_t)(ra + j) * dv, x->PW + (size_t)j * dv, dv * sizeof(double));
    sc[ra + j] = x->pc[j];
  }
  if (orc_brand(dk, dv, m, UC, VC, sc, Ul, Vl, sl) != pr) goto done;

  {
    /* merge two descending lists, local first on ties */
    double smax = 0.0;
    if (pr > 0) smax = sl[0];
    if (nf > 0 && x->sig[ra] > smax) smax = x->sig[ra];
    double thr = x->eps * smax;
    int a = 0, b = 0, out = 0;
    while (a < pr || b < nf) {
      int take_local;
      if (a >= pr) take_local = 0;
      else if (b >= nf) take_local = 1;
      else take_local = (sl[a] >= x->sig[ra + b]);
      const double *u, *vv;
      double sg;
      if (take_local) { u = Ul + (size_t)a * dk; vv = Vl + (size_t)a * dv; sg = sl[a]; ++a; }
      else { u = x->U + (size_t)(ra + b) * dk; vv = x->V + (size_t)(ra + b) * dv; sg = x->sig[ra + b]; ++b; }
      if (sg > 0.0 && sg >= thr) {
        memcpy(nU + (size_t)out * dk, u, dk * sizeof(double));
        memcpy(nV + (size_t)out * dv, vv, dv * sizeof(double));
        ns[out] = sg;
        ++out;
      } else {
        for (int i2 = 0; i2 < dk; ++i2)
          for (int j2 = 0; j2 < dv; ++j2) E[(size_t)i2 * dv + j2] += sg * u[i2] * vv[j2];
      }
    }
    if (ensure_cap(x, out, dk, dv)) goto done;
    if (p->fp16) {  /* factors are stored in fp16 when a compaction writes them */
      round_rows(nU, (size_t)out * dk);
      round_rows(nV, (size_t)out * dv);
    }
    memcpy(x->U, nU, (size_t)out * dk * sizeof(double));
    memcpy(x->V, nV, (size_t)out * dv * sizeof(double));
    memcpy(x->sig, ns, (size_t)out * sizeof(double));
    x->R = out;
    x->n = 0;
    x->bound += sqrt(dot(E, E, dk * dv));
    x->compactions += 1;
    if (p->promote && x->R > p->L) {
      if (make_dense(p, x)) goto done;
    }
    rc = 0;
  }
done:
  free(UC); free(VC); free(sc); free(Ul); free(Vl); free(sl); free(nU); free(nV); free(ns); free(E);
  return rc;
}

/* Compacts the listed states (all states when ids == NULL).  Returns the
 * number of failures (allocation only). */
int64_t orc_compact(orc_pool *p, const int64_t *ids, int64_t n_ids, int nthreads) {
  int64_t bad = 0;
  int64_t cnt = ids ? n_ids : p->N;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads) reduction(+ : bad)
#endif
  for (int64_t i = 0; i < cnt; ++i) {
    int64_t s = ids ? ids[i] : i;
    if (s < 0 || s >= p->N || compact_one(p, &p->st[s])) bad += 1;
  }
  (void)nthreads;
  return bad;
}

/* Consolidation of the frozen part of one state (SinkState 4.3 "Asynchronous
 * CPU Consolidation", Figure 7(a)):
 *  1. frozen = components ra..R-1 (ra = min(r, R)); the active part and the
 *     pad are not touched;
 *  2. sigma_0 is the state's largest stored singular value before the
 *     consolidation (active and frozen lists are each descending, so it is
 *     the larger of their first entries);
 *  3. exact SVD of the frozen part U_F diag(sigma_F) V_F^T (the Brand routine
 *     above applied to the frozen components alone is that SVD);
 *  4. keep the singular values >= eps * sigma_0 (and > 0), in descending
 *     order; they replace the frozen part.  The dropped part goes into the
 *     open-loop bound as its Frobenius norm.
 * A dense state, or one with no frozen component, is left unchanged.  The
 * result's frozen list is sorted on its own; its first entry may exceed the
 * last active one, as the active part is left as it was. */
static int consolidate_one(orc_pool *p, orc_state *x) {
  int dk = p->d_k, dv = p->d_v;
  if (x->dense) return 0;
  int ra = x->R < p->r ? x->R : p->r;
  int nf = x->R - ra;
  if (nf <= 0) return 0;
  int pr = dv < nf ? dv : nf;
  double *UF = (double *)malloc((size_t)dk * nf * sizeof(double));
  double *VF = (double *)malloc((size_t)dv * nf * sizeof(double));
  double *sf = (double *)malloc((size_t)nf * sizeof(double));
  double *Uo = (double *)malloc((size_t)dk * pr * sizeof(double));
  double *Vo = (double *)malloc((size_t)dv * pr * sizeof(double));
  double *so = (double *)malloc((size_t)pr * sizeof(double));
  int rc = -1;
  if (!UF || !VF || !sf || !Uo || !Vo || !so) goto done;
  memcpy(UF, x->U + (size_t)ra * dk, (size_t)nf * dk * sizeof(double));
  memcpy(VF, x->V + (size_t)ra * dv, (size_t)nf * dv * sizeof(double));
  memcpy(sf, x->sig + ra, (size_t)nf * sizeof(double));
  {
    double s0 = x->sig[ra];
    if (ra > 0 && x->sig[0] > s0) s0 = x->sig[0];
    double thr = x->eps * s0;
    if (orc_brand(dk, dv, nf, UF, VF, sf, Uo, Vo, so) != pr) goto done;
    int out = 0;
    double dropped2 = 0.0;
    for (int c = 0; c < pr; ++c) {
      if (so[c] > 0.0 && so[c] >= thr) {
        memcpy(x->U + (size_t)(ra + out) * dk, Uo + (size_t)c * dk, dk * sizeof(double));
        memcpy(x->V + (size_t)(ra + out) * dv, Vo + (size_t)c * dv, dv * sizeof(double));
        x->sig[ra + out] = so[c];
        ++out;
      } else {
        dropped2 += so[c] * so[c];
      }
    }
    x->R = ra + out;
    if (p->fp16) {
      round_rows(x->U + (size_t)ra * dk, (size_t)out * dk);
      round_rows(x->V + (size_t)ra * dv, (size_t)out * dv);
    }
    x->bound += sqrt(dropped2);
    rc = 0;
  }
done:
  free(UF); free(VF); free(sf); free(Uo); free(Vo); free(so);
  return rc;
}

/* Consolidates the listed states (all states when ids == NULL).  Returns the
 * number of failures (allocation only). */
int64_t orc_consolidate(orc_pool *p, const int64_t *ids, int64_t n_ids, int nthreads) {
  int64_t bad = 0;
  int64_t cnt = ids ? n_ids : p->N;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads) reduction(+ : bad)
#endif
  for (int64_t i = 0; i < cnt; ++i) {
    int64_t s = ids ? ids[i] : i;
    if (s < 0 || s >= p->N || consolidate_one(p, &p->st[s])) bad += 1;
  }
  (void)nthreads;
  return bad;
}

/* Staggered schedule (SinkState 4.2 "Staggered compaction across layers"):
 * a group with step offset o compacts after step t (t counted from 1) when
 * (t + o) mod K == 0.  Writes the due groups to out and returns their count. */
int orc_schedule_due(int64_t step, int K, int n_groups, const int32_t *offsets, int32_t *out) {
  int c = 0;
  for (int g = 0; g < n_groups; ++g) {
    int64_t x = (step + offsets[g]) % K;
    if (x < 0) x += K;
    if (x == 0) out[c++] = g;
  }
  return c;
}

/* ------------------------------------------------------------------ */
/* Randomized SVD initialization of a dense state, block by block       */
/* (SinkState 4.1; 4.2 "Randomized SVD initialization after prefill",   */
/* Figure 6(a); Halko et al. 2011).  The pages write the state as        */
/* H = S^T (d_v x d_k, y = H q); here S is d_k x d_v row-major.           */
/* For each block k, with the caller's Gaussian Omega_k (d_k x b):       */
/*   repeat `iters` times:  Y = H Omega (= S^T Omega),  Q = orth(Y),      */
/*                          Omega = H^T Q (= S Q);                        */
/*   block SVD of Omega = X diag(sig) W^T gives the block's components    */
/*   u = X (d_k side), v = Q W (d_v side), sig;                           */
/*   the first block's largest sig is sigma_0; components with            */
/*   sig >= eps sigma_0 and sig > 0 are kept; if any is below, no further */
/*   block is taken.  Otherwise the block is removed from the residual,   */
/*   S <- S - X diag(sig) (Q W)^T, and the next block starts from it.     */
/* Also stops after nb blocks or once `max_rank` components are kept.    */
/* orth is the Q of the Householder thin QR; the block SVD is the        */
/* one-sided Jacobi SVD above.  omega: block k at omega + k d_k b,        */
/* column-major (column c at + c d_k).  Outputs are rows: U[i] at         */
/* U + i d_k, V[i] at V + i d_v, sig[i], descending within each block.   */
/* Returns the number of components kept, or -1 on allocation failure.  */
/* ------------------------------------------------------------------ */
int orc_rsvd_init(int d_k, int d_v, const double *S, int b, int nb, int iters, const double *omega, double eps,
                  int max_rank, double *U, double *V, double *sig) {
  int R = 0, rc = -1;
  double sigma0 = 0.0;
  if (iters < 1) iters = 1;
  double *Sr = (double *)malloc((size_t)d_k * d_v * sizeof(double));
  double *Om = (double *)malloc((size_t)d_k * b * sizeof(double));  /* d_k x b, column-major */
  double *Y = (double *)malloc((size_t)d_v * b * sizeof(double));   /* d_v x b */
  double *Q = (double *)malloc((size_t)d_v * b * sizeof(double));
  double *Rq = (double *)malloc((size_t)b * b * sizeof(double));
  double *X = (double *)malloc((size_t)d_k * b * sizeof(double));
  double *W = (double *)malloc((size_t)b * b * sizeof(double));
  double *sb = (double *)malloc((size_t)b * sizeof(double));
  double *QW = (double *)malloc((size_t)d_v * b * sizeof(double));
  if (!Sr || !Om || !Y || !Q || !Rq || !X || !W || !sb || !QW || b < 1 || b > d_v || b > d_k) goto done;
  memcpy(Sr, S, (size_t)d_k * d_v * sizeof(double));
  for (int blk = 0; blk < nb && R < max_rank; ++blk) {
    memcpy(Om, omega + (size_t)blk * d_k * b, (size_t)d_k * b * sizeof(double));
    for (int it = 0; it < iters; ++it) {
      for (int c = 0; c < b; ++c) /* Y = S^T Omega */
        for (int j = 0; j < d_v; ++j) {
          double acc = 0.0;
          for (int i = 0; i < d_k; ++i) acc += Sr[(size_t)i * d_v + j] * Om[(size_t)c * d_k + i];
          Y[(size_t)c * d_v + j] = acc;
        }
      if (orc_householder_qr(d_v, b, Y, Q, Rq) < 0) goto done;
      for (int c = 0; c < b; ++c) /* Omega = S Q */
        for (int i = 0; i < d_k; ++i) {
          double acc = 0.0;
          for (int j = 0; j < d_v; ++j) acc += Sr[(size_t)i * d_v + j] * Q[(size_t)c * d_v + j];
          Om[(size_t)c * d_k + i] = acc;
        }
    }
    if (orc_jacobi_svd(d_k, b, Om, X, sb, W) < 0) goto done;
    for (int c = 0; c < b; ++c) /* v = Q W */
      for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;
        for (int t = 0; t < b; ++t) acc += Q[(size_t)t * d_v + j] * W[(size_t)c * b + t];
        QW[(size_t)c * d_v + j] = acc;
      }
    if (blk == 0) sigma0 = sb[0];
    int kept = 0;
    for (int c = 0; c < b && R < max_rank; ++c) {
      if (!(sb[c] >= eps * sigma0 && sb[c] > 0.0)) break;  /* descending: the rest are below too */
      for (int i = 0; i < d_k; ++i) U[(size_t)R * d_k + i] = X[(size_t)c * d_k + i];
      for (int j = 0; j < d_v; ++j) V[(size_t)R * d_v + j] = QW[(size_t)c * d_v + j];
      sig[R] = sb[c];
      ++R;
      ++kept;
    }
    if (kept < b) break;
    for (int c = 0; c < b; ++c) /* remove the block from the residual */
      for (int i = 0; i < d_k; ++i) {
        const double f = sb[c] * X[(size_t)c * d_k + i];
        for (int j = 0; j < d_v; ++j) Sr[(size_t)i * d_v + j] -= f * QW[(size_t)c * d_v + j];
      }
  }
  rc = R;
done:
  free(Sr); free(Om); free(Y); free(Q); free(Rq); free(X); free(W); free(sb); free(QW);
  return rc;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

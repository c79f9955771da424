/*
 * oracle_driver.c -- runs every function of the fp64 oracle (oracle/gla_oracle.c)
 * on small inputs, built together with it under AddressSanitizer and
 * UndefinedBehaviorSanitizer (the test that builds it aborts on the first
 * report). Besides memory and arithmetic safety it checks what holds between
 * the oracle's own formulations whatever the inputs:
 *   - recurrent, quadratic and chunked forms agree (every dtype, both modes,
 *     with and without a carried state, ragged chunk sizes);
 *   - the state-only call (no queries) gives the same state;
 *   - the rotary recurrent and quadratic forms agree;
 *   - the backward pass matches central differences of the forward along a
 *     random direction (plain and rotary, both modes);
 *   - the softmax anchor in causal mode with an unlimited window equals full
 *     mode for the last frame's queries;
 *   - empty sizes (B, F or T zero) run without touching memory they lack.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct orc_rope {
  int grid_h, grid_w, frame_offset, dim_t, dim_h, dim_w;
  double theta;
} orc_rope;

int gla_oracle_max_threads(void);
int gla_oracle_recurrent(int mode, int dt, const void *q, const void *k, const void *v,
                         const void *g, const double *gamma, const double *S_in,
                         const double *z_in, double *o, double *S_out, double *z_out, int B,
                         int H, int F, int T, int d, double eps, int nthreads);
int gla_oracle_quadratic(int mode, int dt, const void *q, const void *k, const void *v,
                         const void *g, const double *gamma, const double *S_in,
                         const double *z_in, double *o, double *S_out, double *z_out, int B,
                         int H, int F, int T, int d, double eps, int nthreads);
int gla_oracle_chunked(int mode, int dt, const void *q, const void *k, const void *v,
                       const void *g, const double *gamma, const double *S_in,
                       const double *z_in, double *o, double *S_out, double *z_out, int B, int H,
                       int F, int T, int d, double eps, int C, int nthreads);
int gla_oracle_rope_recurrent(int mode, int dt, const void *q, const void *k, const void *v,
                              const void *g, const double *gamma, const double *S_in,
                              const double *z_in, double *o, double *S_out, double *z_out, int B,
                              int H, int F, int T, int d, double eps, const orc_rope *rope,
                              int nthreads);
int gla_oracle_rope_quadratic(int mode, int dt, const void *q, const void *k, const void *v,
                              const void *g, const double *gamma, const double *S_in,
                              const double *z_in, double *o, int B, int H, int F, int T, int d,
                              double eps, const orc_rope *rope, int nthreads);
int gla_oracle_backward(int mode, int dt, const void *q, const void *k, const void *v,
                        const void *g, const double *gamma, const double *S_in,
                        const double *z_in, const double *dO, const double *dS_out,
                        const double *dz_out, double *dq, double *dk, double *dv, double *dg,
                        double *dgamma, double *dS_in, double *dz_in, int B, int H, int F, int T,
                        int d, double eps, const orc_rope *rope, int pos_T, int nthreads);
int gla_oracle_gdn(int dt, const void *q, const void *k, const void *v, const double *beta,
                   const double *gamma, const double *S_in, double *o, double *S_out, int B,
                   int H, int F, int T, int d, double key_scale, int nthreads);
int gla_oracle_softmax_anchor(int dt, const void *q, const void *k, const void *v,
                              const void *g, double *o, int B, int H, int Fq, int F, int T,
                              int d, int causal, int n_sink, int window, double scale,
                              int nthreads);

enum { F32 = 0, BF16 = 1, F64 = 2 };
enum { BIDIR = 0, FRAMECAUSAL = 1 };
static const int NT = 2; /* OpenMP threads */

static int failures = 0, checks = 0;
#define CHECK(cond, ...)                                            \
  do {                                                              \
    ++checks;                                                       \
    if (!(cond)) {                                                  \
      ++failures;                                                   \
      fprintf(stderr, "FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                                 \
      fprintf(stderr, "\n");                                        \
    }                                                               \
  } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* exact-size buffers (malloc(0) may be NULL: callers pass sizes that allow it) */
static double *dbuf(size_t n) {
  double *p = (double *)malloc(n ? n * sizeof(double) : 1);
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}

/* an input of n elements in dtype dt, random in [-1, 1), its exact double values in *x */
static void *tensor(int dt, size_t n, double **x) {
  *x = (double *)malloc(n ? n * sizeof(double) : 1);
  if (dt == F64) {
    double *p = (double *)malloc(n ? n * sizeof(double) : 1);
    for (size_t i = 0; i < n; ++i) (*x)[i] = p[i] = urand();
    return p;
  }
  if (dt == F32) {
    float *p = (float *)malloc(n ? n * sizeof(float) : 1);
    for (size_t i = 0; i < n; ++i) (*x)[i] = p[i] = (float)urand();
    return p;
  }
  uint16_t *p = (uint16_t *)malloc(n ? n * sizeof(uint16_t) : 1);
  for (size_t i = 0; i < n; ++i) {
    float f = (float)urand();
    uint32_t b;
    memcpy(&b, &f, 4);
    p[i] = (uint16_t)(b >> 16); /* truncation: any bf16 value will do */
    b = (uint32_t)p[i] << 16;
    memcpy(&f, &b, 4);
    (*x)[i] = f;
  }
  return p;
}

static double max_rel(const double *a, const double *b, size_t n) {
  double m = 0.0, s = 1e-300;
  for (size_t i = 0; i < n; ++i) {
    const double e = fabs(a[i] - b[i]);
    if (e > m) m = e;
    if (fabs(b[i]) > s) s = fabs(b[i]);
  }
  return m / s;
}

static void forward_forms(int dt, int mode, int B, int H, int F, int T, int d, int carry) {
  const size_t BH = (size_t)B * H, N = (size_t)F * T, n = BH * N * d;
  double *xq, *xk, *xv, *xg;
  void *q = tensor(dt, n, &xq), *k = tensor(dt, n, &xk), *v = tensor(dt, n, &xv),
       *g = tensor(dt, n, &xg);
  double *gamma = dbuf(BH * F), *S_in = dbuf(BH * d * d), *z_in = dbuf(BH * d);
  for (size_t i = 0; i < BH * F; ++i) gamma[i] = 0.6 + 0.4 * fabs(gamma[i]);
  for (size_t i = 0; i < BH * d; ++i) z_in[i] = fabs(z_in[i]);
  const double *Si = carry ? S_in : NULL, *zi = carry ? z_in : NULL;
  double *o[3], *S[4], *z[4];
  for (int r = 0; r < 4; ++r) {
    if (r < 3) o[r] = dbuf(n);
    S[r] = dbuf(BH * d * d);
    z[r] = dbuf(BH * d);
  }
  gla_oracle_recurrent(mode, dt, q, k, v, g, gamma, Si, zi, o[0], S[0], z[0], B, H, F, T, d,
                       1e-6, NT);
  gla_oracle_quadratic(mode, dt, q, k, v, g, gamma, Si, zi, o[1], S[1], z[1], B, H, F, T, d,
                       1e-6, NT);
  const int C = T > 3 ? T / 2 + 1 : 1; /* chunks that do not divide the frame */
  gla_oracle_chunked(mode, dt, q, k, v, g, gamma, Si, zi, o[2], S[2], z[2], B, H, F, T, d, 1e-6,
                     C, NT);
  gla_oracle_recurrent(mode, dt, NULL, k, v, NULL, gamma, Si, zi, NULL, S[3], z[3], B, H, F, T,
                       d, 1e-6, NT);
  for (int r = 1; r < 3; ++r) {
    CHECK(max_rel(o[r], o[0], n) < 1e-12, "dt %d mode %d F%d T%d d%d form %d: o", dt, mode, F, T,
          d, r);
    CHECK(max_rel(S[r], S[0], BH * d * d) < 1e-12, "form %d: S_out", r);
    CHECK(max_rel(z[r], z[0], BH * d) < 1e-12, "form %d: z_out", r);
  }
  CHECK(max_rel(S[3], S[0], BH * d * d) == 0.0 && max_rel(z[3], z[0], BH * d) == 0.0,
        "state-only call differs (dt %d mode %d)", dt, mode);
  for (int r = 0; r < 4; ++r) {
    if (r < 3) free(o[r]);
    free(S[r]);
    free(z[r]);
  }
  free(q); free(k); free(v); free(g); free(xq); free(xk); free(xv); free(xg);
  free(gamma); free(S_in); free(z_in);
}

static void rope_forms(int mode) {
  const int B = 1, H = 2, F = 3, T = 6, d = 8;
  const size_t BH = (size_t)B * H, N = (size_t)F * T, n = BH * N * d;
  const orc_rope rope = {2, 3, 5, 2, 2, 4, 100.0};
  double *xq, *xk, *xv, *xg;
  void *q = tensor(F64, n, &xq), *k = tensor(F64, n, &xk), *v = tensor(F64, n, &xv),
       *g = tensor(F64, n, &xg);
  double *gamma = dbuf(BH * F), *S_in = dbuf(BH * d * d), *z_in = dbuf(BH * d);
  for (size_t i = 0; i < BH * F; ++i) gamma[i] = 0.7 + 0.3 * fabs(gamma[i]);
  for (size_t i = 0; i < BH * d; ++i) z_in[i] = fabs(z_in[i]);
  double *o1 = dbuf(n), *o2 = dbuf(n), *S = dbuf(BH * d * d), *z = dbuf(BH * d);
  gla_oracle_rope_recurrent(mode, F64, q, k, v, g, gamma, S_in, z_in, o1, S, z, B, H, F, T, d,
                            1e-6, &rope, NT);
  gla_oracle_rope_quadratic(mode, F64, q, k, v, g, gamma, S_in, z_in, o2, B, H, F, T, d, 1e-6,
                            &rope, NT);
  CHECK(max_rel(o2, o1, n) < 1e-12, "rope mode %d: quadratic vs recurrent", mode);
  free(q); free(k); free(v); free(g); free(xq); free(xk); free(xv); free(xg);
  free(gamma); free(S_in); free(z_in); free(o1); free(o2); free(S); free(z);
}

/* L = <W, o> + <WS, S_out> + <Wz, z_out> (the last two in frame-causal mode) */
static double loss(int mode, const double *q, const double *k, const double *v, const double *g,
                   const double *gamma, const double *S_in, const double *z_in, const double *W,
                   const double *WS, const double *Wz, int B, int H, int F, int T, int d,
                   const orc_rope *rope) {
  const size_t BH = (size_t)B * H, n = BH * (size_t)F * T * d;
  double *o = dbuf(n), *S = dbuf(BH * d * d), *z = dbuf(BH * d);
  if (rope)
    gla_oracle_rope_recurrent(mode, F64, q, k, v, g, gamma, S_in, z_in, o, S, z, B, H, F, T, d,
                              0.1, rope, 1);
  else
    gla_oracle_recurrent(mode, F64, q, k, v, g, gamma, S_in, z_in, o, S, z, B, H, F, T, d, 0.1,
                         1);
  double L = 0.0;
  for (size_t i = 0; i < n; ++i) L += W[i] * o[i];
  if (mode == FRAMECAUSAL) {
    for (size_t i = 0; i < BH * d * d; ++i) L += WS[i] * S[i];
    for (size_t i = 0; i < BH * d; ++i) L += Wz[i] * z[i];
  }
  free(o); free(S); free(z);
  return L;
}

static void backward_vs_differences(int mode, int with_rope) {
  /* bidirectional: one frame of all N tokens (the rotary positions then take
   * the whole sequence as one frame of pos_T = N tokens) */
  const int fc = mode == FRAMECAUSAL;
  const int B = 1, H = 2, F = fc ? 3 : 1, T = fc ? 6 : 12, d = 8;
  const size_t BH = (size_t)B * H, N = (size_t)F * T, n = BH * N * d;
  const orc_rope rope = {fc ? 2 : 4, 3, 1, 2, 2, 4, 50.0};
  const orc_rope *rp = with_rope ? &rope : NULL;
  double *x[4], *gamma = dbuf(BH * F), *S_in = dbuf(BH * d * d), *z_in = dbuf(BH * d);
  for (int i = 0; i < 4; ++i) x[i] = dbuf(n);
  /* inputs away from the kink of phi at 0, decays in (0.6, 1], z_in > 0 */
  for (int i = 0; i < 3; ++i)
    for (size_t e = 0; e < n; ++e)
      if (fabs(x[i][e]) < 0.05) x[i][e] = 0.05;
  for (size_t i = 0; i < BH * F; ++i) gamma[i] = 0.6 + 0.4 * fabs(gamma[i]);
  for (size_t i = 0; i < BH * d; ++i) z_in[i] = 1.0 + fabs(z_in[i]);
  double *W = dbuf(n), *WS = dbuf(BH * d * d), *Wz = dbuf(BH * d);
  double *dx[4], *dgamma = dbuf(BH * F), *dS_in = dbuf(BH * d * d), *dz_in = dbuf(BH * d);
  for (int i = 0; i < 4; ++i) dx[i] = dbuf(n);
  gla_oracle_backward(mode, F64, x[0], x[1], x[2], x[3], fc ? gamma : NULL, fc ? S_in : NULL,
                      fc ? z_in : NULL, W, fc ? WS : NULL, fc ? Wz : NULL, dx[0], dx[1], dx[2],
                      dx[3], fc ? dgamma : NULL, fc ? dS_in : NULL, fc ? dz_in : NULL, B, H, F,
                      T, d, 0.1, rp, rope.grid_h * rope.grid_w, NT);
  /* directional derivative along a random direction of every input at once */
  double *dir[4], *dirg = dbuf(BH * F), *dirS = dbuf(BH * d * d), *dirz = dbuf(BH * d);
  for (int i = 0; i < 4; ++i) dir[i] = dbuf(n);
  double pred = 0.0;
  for (int i = 0; i < 4; ++i)
    for (size_t e = 0; e < n; ++e) pred += dir[i][e] * dx[i][e];
  if (fc) {
    for (size_t e = 0; e < BH * F; ++e) pred += dirg[e] * dgamma[e];
    for (size_t e = 0; e < BH * d * d; ++e) pred += dirS[e] * dS_in[e];
    for (size_t e = 0; e < BH * d; ++e) pred += dirz[e] * dz_in[e];
  }
  const double h = 1e-5;
  double Lpm[2];
  for (int s = 0; s < 2; ++s) {
    const double sg = s ? -h : h;
    double *y[4], *yg = dbuf(BH * F), *yS = dbuf(BH * d * d), *yz = dbuf(BH * d);
    for (int i = 0; i < 4; ++i) {
      y[i] = dbuf(n);
      for (size_t e = 0; e < n; ++e) y[i][e] = x[i][e] + sg * dir[i][e];
    }
    for (size_t e = 0; e < BH * F; ++e) yg[e] = gamma[e] + sg * dirg[e];
    for (size_t e = 0; e < BH * d * d; ++e) yS[e] = S_in[e] + sg * dirS[e];
    for (size_t e = 0; e < BH * d; ++e) yz[e] = z_in[e] + sg * dirz[e];
    Lpm[s] = loss(mode, y[0], y[1], y[2], y[3], fc ? yg : NULL, fc ? yS : NULL, fc ? yz : NULL,
                  W, WS, Wz, B, H, F, T, d, rp);
    for (int i = 0; i < 4; ++i) free(y[i]);
    free(yg); free(yS); free(yz);
  }
  const double fd = (Lpm[0] - Lpm[1]) / (2 * h);
  CHECK(fabs(fd - pred) <= 1e-6 * (1.0 + fabs(pred)),
        "backward mode %d rope %d: directional derivative %.12g, differences %.12g", mode,
        with_rope, pred, fd);
  for (int i = 0; i < 4; ++i) {
    free(x[i]); free(dx[i]); free(dir[i]);
  }
  free(gamma); free(S_in); free(z_in); free(W); free(WS); free(Wz); free(dgamma); free(dS_in);
  free(dz_in); free(dirg); free(dirS); free(dirz);
}

static void gdn_and_anchor(void) {
  const int B = 1, H = 2, F = 3, T = 5, d = 8;
  const size_t BH = (size_t)B * H, N = (size_t)F * T, n = BH * N * d;
  double *xq, *xk, *xv, *xg;
  void *q = tensor(BF16, n, &xq), *k = tensor(BF16, n, &xk), *v = tensor(BF16, n, &xv),
       *g = tensor(BF16, n, &xg);
  double *beta = dbuf(BH * N), *gamma = dbuf(BH * F), *S_in = dbuf(BH * d * d);
  double *o = dbuf(n), *S1 = dbuf(BH * d * d), *S2 = dbuf(BH * d * d);
  gla_oracle_gdn(BF16, q, k, v, beta, gamma, S_in, o, S1, B, H, F, T, d, 0.1, NT);
  gla_oracle_gdn(BF16, NULL, k, v, beta, gamma, S_in, NULL, S2, B, H, F, T, d, 0.1, NT);
  CHECK(max_rel(S2, S1, BH * d * d) == 0.0, "gdn state-only call differs");

  /* the last frame's queries see every key frame in both modes */
  const size_t nq = BH * T * d;
  double *oc = dbuf(nq), *of = dbuf(nq);
  const void *qlast = (const char *)q, *glast = (const char *)g;
  gla_oracle_softmax_anchor(BF16, qlast, k, v, glast, oc, B, H, 1, F, T, d, 1, 0, 0, 0.3, NT);
  gla_oracle_softmax_anchor(BF16, qlast, k, v, glast, of, B, H, 1, F, T, d, 0, 0, 0, 0.3, NT);
  CHECK(max_rel(oc, of, nq) == 0.0, "anchor: causal unlimited window differs from full mode");
  /* sinks and a window in causal mode, several query frames */
  double *ow = dbuf(BH * 2 * T * d);
  gla_oracle_softmax_anchor(BF16, q, k, v, g, ow, B, H, 2, F, T, d, 1, 1, 1, 0.3, NT);
  free(ow);
  free(q); free(k); free(v); free(g); free(xq); free(xk); free(xv); free(xg);
  free(beta); free(gamma); free(S_in); free(o); free(S1); free(S2); free(oc); free(of);
}

/* empty sizes: nothing to read, the state passes through (F = 0) */
static void empty_sizes(void) {
  const int d = 8;
  double *S_in = dbuf(d * d), *z_in = dbuf(d), *S = dbuf(d * d), *z = dbuf(d);
  double *o = dbuf(1), *gamma = dbuf(1);
  double *x;
  void *t = tensor(F32, 0, &x);
  gla_oracle_recurrent(FRAMECAUSAL, F32, t, t, t, t, gamma, S_in, z_in, o, S, z, 1, 1, 0, 5, d,
                       1e-6, NT);
  CHECK(max_rel(S, S_in, d * d) == 0.0 && max_rel(z, z_in, d) == 0.0, "F = 0: S_out != S_in");
  gla_oracle_quadratic(FRAMECAUSAL, F32, t, t, t, t, gamma, S_in, z_in, o, S, z, 1, 1, 0, 5, d,
                       1e-6, NT);
  CHECK(max_rel(S, S_in, d * d) == 0.0, "quadratic F = 0: S_out != S_in");
  gla_oracle_chunked(FRAMECAUSAL, F32, t, t, t, t, gamma, S_in, z_in, o, S, z, 1, 1, 0, 5, d,
                     1e-6, 2, NT);
  CHECK(max_rel(S, S_in, d * d) == 0.0, "chunked F = 0: S_out != S_in");
  gla_oracle_recurrent(BIDIR, F32, t, t, t, t, NULL, NULL, NULL, o, S, z, 1, 1, 1, 0, d, 1e-6,
                       NT);
  gla_oracle_recurrent(FRAMECAUSAL, F32, t, t, t, t, gamma, NULL, NULL, o, S, z, 0, 4, 3, 5, d,
                       1e-6, NT);
  gla_oracle_softmax_anchor(F32, t, t, t, t, o, 0, 4, 1, 3, 5, d, 1, 0, 0, 0.3, NT);
  free(S_in); free(z_in); free(S); free(z); free(o); free(gamma); free(t); free(x);
}

int main(void) {
  CHECK(gla_oracle_max_threads() >= 1, "threads");
  for (int dt = 0; dt < 3; ++dt)
    for (int mode = 0; mode < 2; ++mode) {
      forward_forms(dt, mode, 2, 2, mode == FRAMECAUSAL ? 4 : 1, 7, 16, mode == FRAMECAUSAL);
      if (mode == FRAMECAUSAL) forward_forms(dt, mode, 1, 3, 3, 5, 8, 0);
    }
  forward_forms(F64, FRAMECAUSAL, 1, 1, 1, 1, 16, 1);
  rope_forms(FRAMECAUSAL);
  rope_forms(BIDIR);
  for (int mode = 0; mode < 2; ++mode)
    for (int r = 0; r < 2; ++r) backward_vs_differences(mode, r);
  gdn_and_anchor();
  empty_sizes();
  printf("%d checks, %d failures\n", checks, failures);
  return failures ? 1 : 0;
}

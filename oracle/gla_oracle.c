/*
 * gla_oracle.c -- fp64 CPU oracle for the gated linear-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker that the GPU library is
 * compared against. It shares no code, header, table or helper with the HIP
 * library; only the test suite, the smoke check and the benchmark's CPU
 * baseline load it. The product path never calls it.
 *
 * What is computed (per batch b and head h, each an independent N x d slab):
 *
 *   phi(x)   = max(x, 0)                         ReLU feature map
 *   sigma(x) = 1 / (1 + exp(-x))                 output gate
 *
 *   frame-causal mode, tokens grouped into F frames of T tokens:
 *     S_{-1} = S_in (or 0), z_{-1} = z_in (or 0)
 *     S_f = gamma_f * S_{f-1} + sum_{t in f} phi(k_t) v_t^T      (d x d)
 *     z_f = gamma_f * z_{f-1} + sum_{t in f} phi(k_t)            (d)
 *     o_t = sigma(g_t) (.) (phi(q_t)^T S_f) / (phi(q_t)^T z_f + eps),  t in f
 *     S_out = S_{F-1}, z_out = z_{F-1}
 *
 *   bidirectional mode: one state over the whole sequence, no decay, no carry:
 *     S = sum_t phi(k_t) v_t^T, z = sum_t phi(k_t), same readout for every t.
 *
 * Sources:
 *  - "SANA-Video 2.0: Hybrid Linear Attention with Attention Residuals for
 *    Efficient Video Generation" (project page), section "Hybrid Linear-Softmax
 *    Attention": gated linear attention carries the O(N) token mixing.
 *  - "SANA-Video: Efficient Video Generation with Block Linear Diffusion
 *    Transformer" (ICLR 2026 oral, talk transcript), block KV cache passage:
 *    the linear-attention state has a fixed D x D shape independent of the
 *    sequence length, and each new block adds its K^T V contribution to the
 *    cached state (block-causal linear attention, global history).
 *  - "SANA-WM: Efficient Minute-Scale World Modeling with Hybrid Linear
 *    Diffusion Transformer" (analysis page), method components: plain
 *    cumulative linear attention has no decay and drifts at minute scale; the
 *    frame-wise variant adds decay gates to the recurrent state.
 *  The pages print neither the feature map, the gate, the normaliser nor eps;
 *  the readings taken (ReLU, sigmoid gate after normalisation, normaliser z
 *  decayed with the same gamma, eps added to the denominator, a frame's own
 *  tokens included in its state) are the plainest ones and are listed with the
 *  design notes of this repository.
 *
 * Three formulations, written independently of each other:
 *   R  recurrent: decay, then one rank-1 update per token, then the frame's
 *      readout (the whole frame is in the state before any of its outputs)
 *   Q  quadratic: o_t from the explicit weighted sum over all earlier-or-same
 *      frame tokens, A_ts = (phi(q_t).phi(k_s)) * prod_{m=frame(s)+1}^{frame(t)} gamma_m
 *   C  chunked:   per-chunk sums of phi(k)v^T, summed per frame, then the scan
 *
 * Inputs are read element by element and converted exactly to double:
 *   dtype 0 = float32, 1 = bfloat16 (stored as uint16 bit patterns),
 *   2 = float64.  gamma, S_in, z_in and all outputs are float64.
 * Layout: q, k, v, g, o are [B][H][N][d] row-major; gamma is [B][H][F];
 *   S is [B][H][d][d] (S[i][j]: i = key feature, j = value feature); z [B][H][d].
 * Parallelism: OpenMP over independent (b, h, value-column block) tasks. The
 *   columns of S and o are independent sums; splitting them across threads
 *   does not change the order of any floating-point operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };
enum { ORC_BIDIR = 0, ORC_FRAMECAUSAL = 1 };

/* exact conversion of one stored input element to double */
static double ld(const void *p, int dt, size_t i) {
  if (dt == ORC_F64) return ((const double *)p)[i];
  if (dt == ORC_F32) return (double)((const float *)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16; /* bf16 -> f32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double relu(double x) { return x > 0.0 ? x : 0.0; }
static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

int gla_oracle_max_threads(void) { return set_threads(0); }

/* ------------------------------------------------------------------------ */
/* R: recurrent form                                                         */
/* ------------------------------------------------------------------------ */
/* mode: ORC_BIDIR (F must be 1, T = N, gamma/S_in/z_in ignored) or
 * ORC_FRAMECAUSAL. q, g and o may all be NULL: then only the state is
 * produced (the block-cache commit). S_in/z_in may be NULL (zero state).
 * S_out/z_out may be NULL. Returns the number of threads used. */
int gla_oracle_recurrent(int mode, int dt, const void *q, const void *k, const void *v,
                         const void *g, const double *gamma, const double *S_in,
                         const double *z_in, double *o, double *S_out, double *z_out,
                         int B, int H, int F, int T, int d, double eps, int nthreads) {
  const int CB = 8; /* value columns per task */
  const int ncb = (d + CB - 1) / CB;
  const long ntask = (long)B * H * ncb;
  const size_t N = (size_t)F * T;
  const int used = set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < ntask; ++task) {
    const long bh = task / ncb;
    const int j0 = (int)(task % ncb) * CB;
    const int nj = (j0 + CB <= d) ? CB : d - j0;
    double *S = (double *)calloc((size_t)d * CB, sizeof(double)); /* S[i][jj] */
    double *z = (double *)calloc((size_t)d, sizeof(double));
    double *fk = (double *)malloc((size_t)d * sizeof(double));
    const size_t base = (size_t)bh * N * d;

    if (mode == ORC_FRAMECAUSAL && S_in) {
      for (int i = 0; i < d; ++i)
        for (int jj = 0; jj < nj; ++jj) S[i * CB + jj] = S_in[(size_t)bh * d * d + (size_t)i * d + j0 + jj];
    }
    if (mode == ORC_FRAMECAUSAL && z_in) {
      for (int i = 0; i < d; ++i) z[i] = z_in[(size_t)bh * d + i];
    }

    for (int f = 0; f < F; ++f) {
      if (mode == ORC_FRAMECAUSAL) {
        const double gm = gamma[(size_t)bh * F + f];
        for (int i = 0; i < d; ++i) {
          z[i] *= gm;
          for (int jj = 0; jj < nj; ++jj) S[i * CB + jj] *= gm;
        }
      }
      /* rank-1 update for every token of the frame */
      for (int t = 0; t < T; ++t) {
        const size_t row = base + ((size_t)f * T + t) * d;
        for (int i = 0; i < d; ++i) fk[i] = relu(ld(k, dt, row + i));
        for (int i = 0; i < d; ++i) {
          z[i] += fk[i];
          for (int jj = 0; jj < nj; ++jj) S[i * CB + jj] += fk[i] * ld(v, dt, row + j0 + jj);
        }
      }
      /* readout: every token of the frame sees the state including its frame */
      if (o) {
        for (int t = 0; t < T; ++t) {
          const size_t row = base + ((size_t)f * T + t) * d;
          double den = 0.0;
          for (int i = 0; i < d; ++i) den += relu(ld(q, dt, row + i)) * z[i];
          for (int jj = 0; jj < nj; ++jj) {
            double num = 0.0;
            for (int i = 0; i < d; ++i) num += relu(ld(q, dt, row + i)) * S[i * CB + jj];
            o[row + j0 + jj] = sigm(ld(g, dt, row + j0 + jj)) * num / (den + eps);
          }
        }
      }
    }

    if (S_out) {
      for (int i = 0; i < d; ++i)
        for (int jj = 0; jj < nj; ++jj) S_out[(size_t)bh * d * d + (size_t)i * d + j0 + jj] = S[i * CB + jj];
    }
    if (z_out && j0 == 0) {
      for (int i = 0; i < d; ++i) z_out[(size_t)bh * d + i] = z[i];
    }
    free(S);
    free(z);
    free(fk);
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Q: quadratic (brute-force) form                                           */
/* ------------------------------------------------------------------------ */
/* decay weight between a key in frame fs and a query in frame ft:
 *   prod_{m=fs+1}^{ft} gamma_m if fs <= ft (empty product = 1), else 0 */
static double pair_decay(const double *gm, int fs, int ft) {
  if (fs > ft) return 0.0;
  double w = 1.0;
  for (int m = fs + 1; m <= ft; ++m) w *= gm[m];
  return w;
}

/* weight of the carried-in state seen from frame ft: prod_{m=0}^{ft} gamma_m */
static double carry_decay(const double *gm, int ft) {
  double w = 1.0;
  for (int m = 0; m <= ft; ++m) w *= gm[m];
  return w;
}

int gla_oracle_quadratic(int mode, int dt, const void *q, const void *k, const void *v,
                         const void *g, const double *gamma, const double *S_in,
                         const double *z_in, double *o, double *S_out, double *z_out,
                         int B, int H, int F, int T, int d, double eps, int nthreads) {
  const size_t N = (size_t)F * T;
  const long ntask = (long)B * H * (long)N;
  const int used = set_threads(nthreads);

  /* outputs: one task per query token */
  if (o) {
#pragma omp parallel for schedule(static)
    for (long task = 0; task < ntask; ++task) {
      const long bh = task / (long)N;
      const size_t t = (size_t)(task % (long)N);
      const int ft = (int)(t / T);
      const size_t base = (size_t)bh * N * d;
      const double *gm = gamma ? gamma + (size_t)bh * F : NULL;
      double *num = (double *)calloc((size_t)d, sizeof(double));
      double den = 0.0;
      for (size_t s = 0; s < N; ++s) {
        const int fs = (int)(s / T);
        double w = (mode == ORC_BIDIR) ? 1.0 : pair_decay(gm, fs, ft);
        if (w == 0.0 && fs > ft) continue;
        double a = 0.0;
        for (int i = 0; i < d; ++i)
          a += relu(ld(q, dt, base + t * d + i)) * relu(ld(k, dt, base + s * d + i));
        a *= w;
        den += a;
        for (int j = 0; j < d; ++j) num[j] += a * ld(v, dt, base + s * d + j);
      }
      if (mode == ORC_FRAMECAUSAL && (S_in || z_in)) {
        const double c = carry_decay(gm, ft);
        for (int j = 0; j < d && S_in; ++j) {
          double acc = 0.0;
          for (int i = 0; i < d; ++i)
            acc += relu(ld(q, dt, base + t * d + i)) * S_in[(size_t)bh * d * d + (size_t)i * d + j];
          num[j] += c * acc;
        }
        if (z_in) {
          double acc = 0.0;
          for (int i = 0; i < d; ++i) acc += relu(ld(q, dt, base + t * d + i)) * z_in[(size_t)bh * d + i];
          den += c * acc;
        }
      }
      for (int j = 0; j < d; ++j)
        o[base + t * d + j] = sigm(ld(g, dt, base + t * d + j)) * num[j] / (den + eps);
      free(num);
    }
  }

  /* final state as an explicit weighted sum: S_out = sum_s w_s phi(k_s) v_s^T + c S_in */
  if (S_out || z_out) {
    const long nbh = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < nbh; ++bh) {
      const size_t base = (size_t)bh * N * d;
      const double *gm = gamma ? gamma + (size_t)bh * F : NULL;
      const int fl = F - 1;
      for (int i = 0; i < d; ++i) {
        double zi = 0.0;
        for (size_t s = 0; s < N; ++s) {
          const double w = (mode == ORC_BIDIR) ? 1.0 : pair_decay(gm, (int)(s / T), fl);
          zi += w * relu(ld(k, dt, base + s * d + i));
        }
        if (mode == ORC_FRAMECAUSAL && z_in) zi += carry_decay(gm, fl) * z_in[(size_t)bh * d + i];
        if (z_out) z_out[(size_t)bh * d + i] = zi;
        if (!S_out) continue;
        for (int j = 0; j < d; ++j) {
          double sij = 0.0;
          for (size_t s = 0; s < N; ++s) {
            const double w = (mode == ORC_BIDIR) ? 1.0 : pair_decay(gm, (int)(s / T), fl);
            sij += w * relu(ld(k, dt, base + s * d + i)) * ld(v, dt, base + s * d + j);
          }
          if (mode == ORC_FRAMECAUSAL && S_in)
            sij += carry_decay(gm, fl) * S_in[(size_t)bh * d * d + (size_t)i * d + j];
          S_out[(size_t)bh * d * d + (size_t)i * d + j] = sij;
        }
      }
    }
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* C: chunked form                                                           */
/* ------------------------------------------------------------------------ */
/* Each frame (the whole sequence in bidirectional mode) is cut into chunks of
 * C tokens, the last one possibly shorter. Per chunk: U_c = sum phi(k)v^T and
 * u_c = sum phi(k). Per frame: U_f = sum of its chunks. Then the scan
 * S_f = gamma_f S_{f-1} + U_f (bidirectional: S = U of the single frame) and
 * the readout of every token of frame f against S_f. */
int gla_oracle_chunked(int mode, int dt, const void *q, const void *k, const void *v,
                       const void *g, const double *gamma, const double *S_in,
                       const double *z_in, double *o, double *S_out, double *z_out, int B,
                       int H, int F, int T, int d, double eps, int C, int nthreads) {
  const size_t N = (size_t)F * T;
  const long nbh = (long)B * H;
  const int used = set_threads(nthreads);
  if (C < 1) C = 1;

#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const size_t base = (size_t)bh * N * d;
    const size_t dd = (size_t)d * d;
    double *Uf = (double *)malloc(dd * sizeof(double));
    double *uf = (double *)malloc((size_t)d * sizeof(double));
    double *Uc = (double *)malloc(dd * sizeof(double));
    double *uc = (double *)malloc((size_t)d * sizeof(double));
    double *S = (double *)calloc(dd, sizeof(double));
    double *z = (double *)calloc((size_t)d, sizeof(double));
    if (mode == ORC_FRAMECAUSAL && S_in) memcpy(S, S_in + (size_t)bh * dd, dd * sizeof(double));
    if (mode == ORC_FRAMECAUSAL && z_in) memcpy(z, z_in + (size_t)bh * d, (size_t)d * sizeof(double));

    for (int f = 0; f < F; ++f) {
      memset(Uf, 0, dd * sizeof(double));
      memset(uf, 0, (size_t)d * sizeof(double));
      for (int c0 = 0; c0 < T; c0 += C) {
        const int c1 = (c0 + C < T) ? c0 + C : T;
        memset(Uc, 0, dd * sizeof(double));
        memset(uc, 0, (size_t)d * sizeof(double));
        for (int t = c0; t < c1; ++t) {
          const size_t row = base + ((size_t)f * T + t) * d;
          for (int i = 0; i < d; ++i) {
            const double fk = relu(ld(k, dt, row + i));
            uc[i] += fk;
            for (int j = 0; j < d; ++j) Uc[(size_t)i * d + j] += fk * ld(v, dt, row + j);
          }
        }
        for (size_t e = 0; e < dd; ++e) Uf[e] += Uc[e];
        for (int i = 0; i < d; ++i) uf[i] += uc[i];
      }
      const double gm = (mode == ORC_FRAMECAUSAL) ? gamma[(size_t)bh * F + f] : 1.0;
      for (size_t e = 0; e < dd; ++e) S[e] = gm * S[e] + Uf[e];
      for (int i = 0; i < d; ++i) z[i] = gm * z[i] + uf[i];

      if (o) {
        for (int t = 0; t < T; ++t) {
          const size_t row = base + ((size_t)f * T + t) * d;
          double den = 0.0;
          for (int i = 0; i < d; ++i) den += relu(ld(q, dt, row + i)) * z[i];
          for (int j = 0; j < d; ++j) {
            double num = 0.0;
            for (int i = 0; i < d; ++i) num += relu(ld(q, dt, row + i)) * S[(size_t)i * d + j];
            o[row + j] = sigm(ld(g, dt, row + j)) * num / (den + eps);
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * dd, S, dd * sizeof(double));
    if (z_out) memcpy(z_out + (size_t)bh * d, z, (size_t)d * sizeof(double));
    free(Uf);
    free(uf);
    free(Uc);
    free(uc);
    free(S);
    free(z);
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Rotary (3D RoPE) variant                                                  */
/* ------------------------------------------------------------------------ */
/* The SANA-Video ICLR 2026 oral talk (passage on temporal modeling) adds 3D
 * RoPE to the linear attention; the pages do not say where it sits relative
 * to the feature map. Reading taken (RoFormer's form of rotary linear
 * attention): the numerator uses rotated features R_t phi(q_t) and R_s phi(k_s),
 * the normaliser keeps the unrotated phi(q_t) . phi(k_s), so it stays positive:
 *
 *   o_t = sigma(g_t) (.) sum_s w_ts (R_t phi(q_t))^T (R_s phi(k_s)) v_s
 *                       / (sum_s w_ts phi(q_t)^T phi(k_s) + eps)
 *
 * Token n of the call (frame f = n / T, in-frame index l = n % T) sits at
 * (t, y, x) = (frame_offset + f, l / grid_w, l % grid_w). Features are rotated
 * in adjacent pairs (2p, 2p+1); the first dim_t/2 pairs turn with t, the next
 * dim_h/2 with y, the last dim_w/2 with x. Within a section of m pairs, pair j
 * turns by angle pos * theta^(-j/m). */
typedef struct orc_rope {
  int grid_h, grid_w, frame_offset, dim_t, dim_h, dim_w;
  double theta;
} orc_rope;

/* Turns the pairs of x, the features of token n (T tokens per frame), by
 * dir times their angles: dir = +1 is R_n, dir = -1 its transpose. */
static void rope_turn(double *x, int d, int T, size_t n, const orc_rope *r, double dir) {
  const int f = (int)(n / (size_t)T);
  const int l = (int)(n % (size_t)T);
  const double pt = (double)(r->frame_offset + f);
  const double py = (double)(l / r->grid_w);
  const double px = (double)(l % r->grid_w);
  const int Pt = r->dim_t / 2, Ph = r->dim_h / 2, Pw = r->dim_w / 2;
  for (int p = 0; p < d / 2; ++p) {
    double pos;
    int j, m;
    if (p < Pt) {
      pos = pt; j = p; m = Pt;
    } else if (p < Pt + Ph) {
      pos = py; j = p - Pt; m = Ph;
    } else {
      pos = px; j = p - Pt - Ph; m = Pw;
    }
    const double ang = dir * (pos * pow(r->theta, -(double)j / (double)m));
    const double c = cos(ang), s = sin(ang);
    const double a = x[2 * p], b = x[2 * p + 1];
    x[2 * p] = a * c - b * s;
    x[2 * p + 1] = a * s + b * c;
  }
}

static void rope_rotate(double *x, int d, int T, size_t n, const orc_rope *r) {
  rope_turn(x, d, T, n, r, 1.0);
}

/* Recurrent form with rotation: the state collects rotated keys, the
 * normaliser unrotated ones. Arguments as gla_oracle_recurrent, plus the
 * rotation (rope must not be NULL; T must equal grid_h * grid_w). */
int gla_oracle_rope_recurrent(int mode, int dt, const void *q, const void *k, const void *v,
                              const void *g, const double *gamma, const double *S_in,
                              const double *z_in, double *o, double *S_out, double *z_out, int B,
                              int H, int F, int T, int d, double eps, const orc_rope *rope,
                              int nthreads) {
  const long nbh = (long)B * H;
  const size_t N = (size_t)F * T;
  const int used = set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nbh; ++bh) {
    const size_t base = (size_t)bh * N * d;
    const size_t dd = (size_t)d * d;
    double *S = (double *)calloc(dd, sizeof(double));
    double *z = (double *)calloc((size_t)d, sizeof(double));
    double *fk = (double *)malloc((size_t)d * sizeof(double));
    double *rk = (double *)malloc((size_t)d * sizeof(double));
    double *fq = (double *)malloc((size_t)d * sizeof(double));
    double *rq = (double *)malloc((size_t)d * sizeof(double));
    if (mode == ORC_FRAMECAUSAL && S_in) memcpy(S, S_in + (size_t)bh * dd, dd * sizeof(double));
    if (mode == ORC_FRAMECAUSAL && z_in) memcpy(z, z_in + (size_t)bh * d, (size_t)d * sizeof(double));
    /* bidirectional: one frame holding all tokens (positions still use T) */
    const int nframes = (mode == ORC_FRAMECAUSAL) ? F : 1;
    const size_t per = (mode == ORC_FRAMECAUSAL) ? (size_t)T : N;
    for (int f = 0; f < nframes; ++f) {
      if (mode == ORC_FRAMECAUSAL) {
        const double gm = gamma[(size_t)bh * F + f];
        for (size_t e = 0; e < dd; ++e) S[e] *= gm;
        for (int i = 0; i < d; ++i) z[i] *= gm;
      }
      for (size_t t = 0; t < per; ++t) {
        const size_t n = (size_t)f * per + t;
        const size_t row = base + n * d;
        for (int i = 0; i < d; ++i) rk[i] = fk[i] = relu(ld(k, dt, row + i));
        rope_rotate(rk, d, T, n, rope);
        for (int i = 0; i < d; ++i) {
          z[i] += fk[i];
          for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += rk[i] * ld(v, dt, row + j);
        }
      }
      if (!o) continue;
      for (size_t t = 0; t < per; ++t) {
        const size_t n = (size_t)f * per + t;
        const size_t row = base + n * d;
        for (int i = 0; i < d; ++i) rq[i] = fq[i] = relu(ld(q, dt, row + i));
        rope_rotate(rq, d, T, n, rope);
        double den = 0.0;
        for (int i = 0; i < d; ++i) den += fq[i] * z[i];
        for (int j = 0; j < d; ++j) {
          double num = 0.0;
          for (int i = 0; i < d; ++i) num += rq[i] * S[(size_t)i * d + j];
          o[row + j] = sigm(ld(g, dt, row + j)) * num / (den + eps);
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * dd, S, dd * sizeof(double));
    if (z_out) memcpy(z_out + (size_t)bh * d, z, (size_t)d * sizeof(double));
    free(S); free(z); free(fk); free(rk); free(fq); free(rq);
  }
  return used;
}

/* Quadratic form with rotation: explicit pairwise weights, no state. */
int gla_oracle_rope_quadratic(int mode, int dt, const void *q, const void *k, const void *v,
                              const void *g, const double *gamma, const double *S_in,
                              const double *z_in, double *o, int B, int H, int F, int T, int d,
                              double eps, const orc_rope *rope, int nthreads) {
  const size_t N = (size_t)F * T;
  const long ntask = (long)B * H * (long)N;
  const int used = set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (long task = 0; task < ntask; ++task) {
    const long bh = task / (long)N;
    const size_t t = (size_t)(task % (long)N);
    const int ft = (int)(t / T);
    const size_t base = (size_t)bh * N * d;
    const double *gm = gamma ? gamma + (size_t)bh * F : NULL;
    double *fq = (double *)malloc((size_t)d * sizeof(double));
    double *rq = (double *)malloc((size_t)d * sizeof(double));
    double *fk = (double *)malloc((size_t)d * sizeof(double));
    double *rk = (double *)malloc((size_t)d * sizeof(double));
    double *num = (double *)calloc((size_t)d, sizeof(double));
    double den = 0.0;
    for (int i = 0; i < d; ++i) rq[i] = fq[i] = relu(ld(q, dt, base + t * d + i));
    rope_rotate(rq, d, T, t, rope);
    for (size_t s = 0; s < N; ++s) {
      const int fs = (int)(s / T);
      const double w = (mode == ORC_BIDIR) ? 1.0 : pair_decay(gm, fs, ft);
      if (w == 0.0 && fs > ft) continue;
      for (int i = 0; i < d; ++i) rk[i] = fk[i] = relu(ld(k, dt, base + s * d + i));
      rope_rotate(rk, d, T, s, rope);
      double an = 0.0, ad = 0.0;
      for (int i = 0; i < d; ++i) {
        an += rq[i] * rk[i];
        ad += fq[i] * fk[i];
      }
      den += w * ad;
      for (int j = 0; j < d; ++j) num[j] += w * an * ld(v, dt, base + s * d + j);
    }
    if (mode == ORC_FRAMECAUSAL && S_in) {
      const double c = carry_decay(gm, ft);
      for (int j = 0; j < d; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += rq[i] * S_in[(size_t)bh * d * d + (size_t)i * d + j];
        num[j] += c * acc;
      }
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += fq[i] * z_in[(size_t)bh * d + i];
      den += c * acc;
    }
    for (int j = 0; j < d; ++j)
      o[base + t * d + j] = sigm(ld(g, dt, base + t * d + j)) * num[j] / (den + eps);
    free(fq); free(rq); free(fk); free(rk); free(num);
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Backward: gradients of the definition above                               */
/* ------------------------------------------------------------------------ */
/*
 * The pages state the forward pass only; these are the chain rule through its
 * definition, taken in reverse order of the forward steps. With
 *   h_t = num_t / (den_t + eps),  o_t = sigma(g_t) (.) h_t,
 * for a loss L whose gradients are dO = dL/do, dS_out = dL/dS_out and
 * dz_out = dL/dz_out:
 *   dg_t   = dO_t (.) h_t (.) sigma(g_t) (1 - sigma(g_t))
 *   dnum_t = dO_t (.) sigma(g_t) / (den_t + eps)
 *   dden_t = -((dO_t (.) sigma(g_t)) . h_t) / (den_t + eps)
 *   dq_t   = [q_t > 0] (.) (S_f dnum_t + dden_t z_f)              t in frame f
 *   adjoint of S_f:  Sh_f = sum_{t in f} phi(q_t) dnum_t^T + gamma_{f+1} Sh_{f+1}
 *                    (Sh_{F-1} = its frame's sum + dS_out); zh_f likewise,
 *                    with dden_t phi(q_t) and dz_out
 *   dk_t   = [k_t > 0] (.) (Sh_f v_t + zh_f),   dv_t = Sh_f^T phi(k_t)
 *   dgamma_f = <Sh_f, S_{f-1}> + <zh_f, z_{f-1}>   (Frobenius products)
 *   dS_in  = gamma_0 Sh_0,  dz_in = gamma_0 zh_0
 * The derivative of ReLU is taken as 0 at 0. Bidirectional mode is one frame
 * of all N tokens with no decay and no carried state (dgamma, dS_in, dz_in
 * are then not written).
 *
 * With rotary positions (rope != NULL; the rotary form above) the numerator
 * takes turned features a~_t = R_t phi(q_t), b~_s = R_s phi(k_s) and the
 * normaliser the unturned ones, so S_f collects b~_s v_s^T and z_f phi(k_s):
 *   dq_t = [q_t > 0] (.) (R_t^T S_f dnum_t + dden_t z_f)
 *   Sh_f collects a~_t dnum_t^T, zh_f still dden_t phi(q_t)
 *   dk_t = [k_t > 0] (.) (R_t^T Sh_f v_t + zh_f),   dv_t = Sh_f^T b~_t
 * Token n = f T + t turns by the position (n / pos_T, n % pos_T) of a frame of
 * pos_T tokens (pos_T = T in frame-causal mode; in bidirectional mode the
 * positions keep the frames of pos_T tokens while the sums run over all N).
 *
 * dO, dS_out, dz_out are float64 (dS_out/dz_out may be NULL: zero); dq, dk,
 * dv, dg are float64 [B][H][N][d]; dgamma [B][H][F]; dS_in [B][H][d][d] and
 * dz_in [B][H][d] may be NULL. OpenMP over slabs.
 */
int gla_oracle_backward(int mode, int dt, const void *q, const void *k, const void *v,
                        const void *g, const double *gamma, const double *S_in,
                        const double *z_in, const double *dO, const double *dS_out,
                        const double *dz_out, double *dq, double *dk, double *dv, double *dg,
                        double *dgamma, double *dS_in, double *dz_in, int B, int H, int F, int T,
                        int d, double eps, const orc_rope *rope, int pos_T, int nthreads) {
  const long nslab = (long)B * H;
  const size_t N = (size_t)F * T, dd = (size_t)d * d;
  const int used = set_threads(nthreads);
  const int causal = mode == ORC_FRAMECAUSAL;

#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nslab; ++bh) {
    double *S = (double *)calloc((size_t)(F + 1) * dd, sizeof(double)); /* S[f+1] = S_f */
    double *z = (double *)calloc((size_t)(F + 1) * d, sizeof(double));
    double *G = (double *)calloc((size_t)F * dd + 1, sizeof(double));   /* readout sums */
    double *gz = (double *)calloc((size_t)F * d + 1, sizeof(double));
    double *A = (double *)calloc(dd, sizeof(double));                   /* incoming adjoint */
    double *az = (double *)calloc((size_t)d, sizeof(double));
    double *Sh = (double *)malloc(dd * sizeof(double));
    double *zh = (double *)malloc((size_t)d * sizeof(double));
    double *fq = (double *)malloc((size_t)d * sizeof(double));
    double *rq = (double *)malloc((size_t)d * sizeof(double)); /* turned phi(q) (= fq without rope) */
    double *rk = (double *)malloc((size_t)d * sizeof(double)); /* turned phi(k) */
    double *u = (double *)malloc((size_t)d * sizeof(double));
    double *h = (double *)malloc((size_t)d * sizeof(double));
    double *dn = (double *)malloc((size_t)d * sizeof(double));
    const size_t base = (size_t)bh * N * d;

    /* forward states S_{-1} .. S_{F-1} */
    if (causal && S_in) memcpy(S, S_in + (size_t)bh * dd, dd * sizeof(double));
    if (causal && z_in) memcpy(z, z_in + (size_t)bh * d, (size_t)d * sizeof(double));
    for (int f = 0; f < F; ++f) {
      const double gm = causal ? gamma[(size_t)bh * F + f] : 1.0;
      double *Sc = S + (size_t)(f + 1) * dd, *zc = z + (size_t)(f + 1) * d;
      for (size_t e = 0; e < dd; ++e) Sc[e] = gm * S[(size_t)f * dd + e];
      for (int i = 0; i < d; ++i) zc[i] = gm * z[(size_t)f * d + i];
      for (int t = 0; t < T; ++t) {
        const size_t n = (size_t)f * T + t, row = base + n * d;
        for (int i = 0; i < d; ++i) rk[i] = relu(ld(k, dt, row + i));
        if (rope) rope_turn(rk, d, pos_T, n, rope, 1.0);
        for (int i = 0; i < d; ++i) {
          zc[i] += relu(ld(k, dt, row + i));
          for (int j = 0; j < d; ++j) Sc[(size_t)i * d + j] += rk[i] * ld(v, dt, row + j);
        }
      }
    }

    /* readout side: dg, dq and the per-frame sums that feed the adjoints */
    for (int f = 0; f < F; ++f) {
      const double *Sc = S + (size_t)(f + 1) * dd, *zc = z + (size_t)(f + 1) * d;
      double *Gf = G + (size_t)f * dd, *gzf = gz + (size_t)f * d;
      for (int t = 0; t < T; ++t) {
        const size_t n = (size_t)f * T + t, row = base + n * d;
        double den = 0.0;
        for (int i = 0; i < d; ++i) {
          rq[i] = fq[i] = relu(ld(q, dt, row + i));
          den += fq[i] * zc[i];
        }
        if (rope) rope_turn(rq, d, pos_T, n, rope, 1.0);
        const double inv = 1.0 / (den + eps);
        double dden = 0.0;
        for (int j = 0; j < d; ++j) {
          double num = 0.0;
          for (int i = 0; i < d; ++i) num += rq[i] * Sc[(size_t)i * d + j];
          const double sg = sigm(ld(g, dt, row + j));
          h[j] = num * inv;
          const double dh = dO[row + j] * sg;
          dg[row + j] = dO[row + j] * h[j] * sg * (1.0 - sg);
          dn[j] = dh * inv;
          dden -= dh * h[j] * inv;
        }
        for (int i = 0; i < d; ++i) {
          double acc = 0.0;
          for (int j = 0; j < d; ++j) acc += Sc[(size_t)i * d + j] * dn[j];
          u[i] = acc;
        }
        if (rope) rope_turn(u, d, pos_T, n, rope, -1.0);
        for (int i = 0; i < d; ++i) {
          dq[row + i] = ld(q, dt, row + i) > 0.0 ? u[i] + dden * zc[i] : 0.0;
          for (int j = 0; j < d; ++j) Gf[(size_t)i * d + j] += rq[i] * dn[j];
          gzf[i] += dden * fq[i];
        }
      }
    }

    /* reverse scan of the adjoints, and the key side */
    if (causal && dS_out) memcpy(A, dS_out + (size_t)bh * dd, dd * sizeof(double));
    if (causal && dz_out) memcpy(az, dz_out + (size_t)bh * d, (size_t)d * sizeof(double));
    for (int f = F - 1; f >= 0; --f) {
      for (size_t e = 0; e < dd; ++e) Sh[e] = G[(size_t)f * dd + e] + A[e];
      for (int i = 0; i < d; ++i) zh[i] = gz[(size_t)f * d + i] + az[i];
      if (causal && dgamma) {
        double s = 0.0;
        for (size_t e = 0; e < dd; ++e) s += Sh[e] * S[(size_t)f * dd + e];
        for (int i = 0; i < d; ++i) s += zh[i] * z[(size_t)f * d + i];
        dgamma[(size_t)bh * F + f] = s;
      }
      for (int t = 0; t < T; ++t) {
        const size_t n = (size_t)f * T + t, row = base + n * d;
        for (int i = 0; i < d; ++i) {
          double acc = 0.0;
          for (int j = 0; j < d; ++j) acc += Sh[(size_t)i * d + j] * ld(v, dt, row + j);
          u[i] = acc;
          rk[i] = relu(ld(k, dt, row + i));
        }
        if (rope) {
          rope_turn(u, d, pos_T, n, rope, -1.0);
          rope_turn(rk, d, pos_T, n, rope, 1.0);
        }
        for (int i = 0; i < d; ++i) dk[row + i] = ld(k, dt, row + i) > 0.0 ? u[i] + zh[i] : 0.0;
        for (int j = 0; j < d; ++j) {
          double acc = 0.0;
          for (int i = 0; i < d; ++i) acc += Sh[(size_t)i * d + j] * rk[i];
          dv[row + j] = acc;
        }
      }
      const double gm = causal ? gamma[(size_t)bh * F + f] : 1.0;
      for (size_t e = 0; e < dd; ++e) A[e] = gm * Sh[e];
      for (int i = 0; i < d; ++i) az[i] = gm * zh[i];
    }
    if (causal && dS_in) memcpy(dS_in + (size_t)bh * dd, A, dd * sizeof(double));
    if (causal && dz_in) memcpy(dz_in + (size_t)bh * d, az, (size_t)d * sizeof(double));

    free(S); free(z); free(G); free(gz); free(A); free(az); free(Sh); free(zh);
    free(fq); free(rq); free(rk); free(u); free(h); free(dn);
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Frame-wise Gated DeltaNet                                                 */
/* ------------------------------------------------------------------------ */
/*
 * The SANA-WM analysis page (method components) names its linear mixer a
 * frame-wise Gated DeltaNet: decay gates plus a delta-rule correction of the
 * recurrent state, with keys scaled by 1/sqrt(D S), the only scaling that
 * trains stably (claim checks). Reading taken: the state is updated once per
 * frame, every token of the frame measuring its prediction error against the
 * same decayed prior (a block delta rule; S = tokens per frame, which is what
 * makes the frame's summed key norms, and with them the update's contraction,
 * independent of the frame size):
 *
 *   k~_t = c k_t                     (c = key_scale, 1/sqrt(d T) by default)
 *   P_f  = gamma_f S_{f-1}           (S_{-1} = S_in or 0)
 *   e_t  = v_t - P_f^T k~_t          (t in frame f)
 *   S_f  = P_f + sum_{t in f} beta_t k~_t e_t^T
 *   o_t  = S_f^T q_t                 (every token of frame f reads S_f)
 *
 * beta [B][H][N] and gamma [B][H][F] are float64; S_in, S_out [B][H][d][d]
 * (S[i][j]: i = key feature, j = value feature). q may be NULL (state only).
 * OpenMP over slabs.
 */
int gla_oracle_gdn(int dt, const void *q, const void *k, const void *v, const double *beta,
                   const double *gamma, const double *S_in, double *o, double *S_out, int B,
                   int H, int F, int T, int d, double key_scale, int nthreads) {
  const long nslab = (long)B * H;
  const size_t N = (size_t)F * T, dd = (size_t)d * d;
  const int used = set_threads(nthreads);

#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < nslab; ++bh) {
    double *S = (double *)calloc(dd, sizeof(double));
    double *Pr = (double *)malloc(dd * sizeof(double));
    double *kt = (double *)malloc((size_t)d * sizeof(double));
    double *e = (double *)malloc((size_t)d * sizeof(double));
    const size_t base = (size_t)bh * N * d;
    if (S_in) memcpy(S, S_in + (size_t)bh * dd, dd * sizeof(double));
    for (int f = 0; f < F; ++f) {
      const double gm = gamma[(size_t)bh * F + f];
      for (size_t x = 0; x < dd; ++x) Pr[x] = gm * S[x];
      for (size_t x = 0; x < dd; ++x) S[x] = Pr[x];
      for (int t = 0; t < T; ++t) {
        const size_t row = base + ((size_t)f * T + t) * d;
        const double bt = beta[(size_t)bh * N + (size_t)f * T + t];
        for (int i = 0; i < d; ++i) kt[i] = key_scale * ld(k, dt, row + i);
        for (int j = 0; j < d; ++j) {
          double pred = 0.0;
          for (int i = 0; i < d; ++i) pred += Pr[(size_t)i * d + j] * kt[i];
          e[j] = ld(v, dt, row + j) - pred;
        }
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += bt * kt[i] * e[j];
      }
      if (q && o) {
        for (int t = 0; t < T; ++t) {
          const size_t row = base + ((size_t)f * T + t) * d;
          for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += S[(size_t)i * d + j] * ld(q, dt, row + i);
            o[row + j] = acc;
          }
        }
      }
    }
    if (S_out) memcpy(S_out + (size_t)bh * dd, S, dd * sizeof(double));
    free(S); free(Pr); free(kt); free(e);
  }
  return used;
}

/* ------------------------------------------------------------------------ */
/* Gated softmax anchor: sink frames and a local temporal window             */
/* ------------------------------------------------------------------------ */
/*
 * The SANA-Video 2.0 project page ("Hybrid Linear-Softmax Attention") puts a
 * gated-softmax anchor in one layer of every four, to restore full-rank token
 * interactions; the SANA-WM analysis page (deployment) gives the softmax
 * layers attention-sink tokens and a local temporal window, so that their
 * memory and per-chunk latency stay constant along the rollout. Neither page
 * prints the formula. Reading taken (the gate as in the linear layers):
 *
 *   o_t = sigma(g_t) (.) sum_{s in V(t)} w_ts v_s
 *   w_ts = exp(scale q_t.k_s) / sum_{s' in V(t)} exp(scale q_t.k_s')
 *
 * Keys and values are F frames of T tokens; queries (and g, o) are the tokens
 * of the last Fq of those frames: query frame j is key frame f = F - Fq + j
 * (a streaming call passes [kept frames | new frames] as keys and the new
 * frames as queries). V(t) is every key in full mode; in frame-causal mode it
 * is the tokens of key frames i with i <= f and (i < n_sink or i > f - window):
 * the sink frames plus a window of `window` frames that ends with the query's
 * own frame (window <= 0: unlimited). The query's own frame is always in V(t).
 * scale is given by the caller (the usual choice is 1/sqrt(d)). The maximum
 * score over V(t) is subtracted before exp, which leaves w unchanged.
 * q, k, v, g in the input dtype, o float64; OpenMP over (slab, query frame).
 */
static int anchor_visible(int i, int f, int causal, int n_sink, int window) {
  if (!causal) return 1;
  if (i > f) return 0;
  return i < n_sink || window <= 0 || i > f - window;
}

int gla_oracle_softmax_anchor(int dt, const void *q, const void *k, const void *v,
                              const void *g, double *o, int B, int H, int Fq, int F, int T,
                              int d, int causal, int n_sink, int window, double scale,
                              int nthreads) {
  const long nslab = (long)B * H;
  const size_t Nq = (size_t)Fq * T, Nk = (size_t)F * T;
  const int used = set_threads(nthreads);
  const long tasks = nslab * Fq;

#pragma omp parallel for schedule(dynamic, 1)
  for (long task = 0; task < tasks; ++task) {
    const long bh = task / Fq;
    const int j = (int)(task % Fq), f = F - Fq + j;
    double *w = (double *)malloc((Nk ? Nk : 1) * sizeof(double));
    double *acc = (double *)malloc((size_t)d * sizeof(double));
    for (int t = 0; t < T; ++t) {
      const size_t qrow = ((size_t)bh * Nq + (size_t)j * T + t) * d;
      double mx = -INFINITY;
      for (size_t s = 0; s < Nk; ++s) {
        if (!anchor_visible((int)(s / T), f, causal, n_sink, window)) continue;
        const size_t krow = ((size_t)bh * Nk + s) * d;
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += ld(q, dt, qrow + x) * ld(k, dt, krow + x);
        w[s] = scale * dot;
        if (w[s] > mx) mx = w[s];
      }
      double den = 0.0;
      for (int x = 0; x < d; ++x) acc[x] = 0.0;
      for (size_t s = 0; s < Nk; ++s) {
        if (!anchor_visible((int)(s / T), f, causal, n_sink, window)) continue;
        const double e = exp(w[s] - mx);
        const size_t vrow = ((size_t)bh * Nk + s) * d;
        den += e;
        for (int x = 0; x < d; ++x) acc[x] += e * ld(v, dt, vrow + x);
      }
      for (int x = 0; x < d; ++x) o[qrow + x] = sigm(ld(g, dt, qrow + x)) * acc[x] / den;
    }
    free(w);
    free(acc);
  }
  return used;
}

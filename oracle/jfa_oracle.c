/*
 * Jagged attention oracle: a plain, slow, fp64 CPU statement of what the
 * jagged attention path computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code with the GPU path.
 *
 * Sources (the pages on Meta's GEM training work):
 *  - "Meta GEM Training Efficiency: Why LLM-Scale Recommenders Need a
 *    Different Stack", section "Bottleneck move 1": Jagged Flash Attention
 *    runs on variable-length tensors with custom biases and asymmetric
 *    query/key-value lengths; GDPA replaces softmax by GELU or SiLU.
 *  - same page, FAQ "What is a jagged tensor?": values plus offsets.
 *  - same page, "Bottleneck move 1": removing padding exposes tile
 *    scheduling (the tile-list oracle below).
 *  - "GEM Training: How Meta Doubled the Efficiency ...", "Challenge 1":
 *    padding to the longest sample wastes compute, so nothing here pads.
 *  - "Meta Enhances GEM Training Efficiency ...", "Leveraging Compute
 *    Efficiency through Customized Kernels": MXFP8 attention.
 *
 * The pages give no formula.  Every formula here is standard scaled
 * dot-product attention restricted to each sample's own rows; the readings
 * taken where the pages are silent (scale, bias placement, causal alignment,
 * bucket function, GDPA 1/kv_len, dense-bias layout, tile order, split rule,
 * MXFP8 rounding) are listed in the design notes and passed in as
 * parameters.  Arithmetic is fp64, evaluated literally: no tiling, no online
 * softmax, no fused multiply-add (built with -ffp-contract=off).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t batch, heads, head_dim;
  int32_t mode;        /* 0 softmax, 1 silu, 2 gelu */
  int32_t causal;      /* 1: key j is visible to query i iff j <= i + (kv_len - q_len) */
  double scale;        /* multiplies q.k */
  int32_t normalize;   /* GDPA only: 1 divides the output by the sample's kv_len */
  int32_t bias_kind;   /* 0 none, 1 relative-position bucket table, 2 dense jagged */
  int32_t num_buckets; /* relative-position table width */
  int32_t block;       /* BlockAttention: >0 splits every sample (q_len = kv_len) into
                          consecutive blocks of this many rows that attend only within
                          themselves; 0 = full attention over the sample */
  int32_t window;      /* sliding window: >0 limits query i to keys j with
                          |i + (kv_len - q_len) - j| < window (with causal: the window keys
                          ending at its own position); 0 = no window */
} ora_problem;

/* ---------------------------------------------------------------- threads */

void ora_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int ora_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------- offsets */

/* Exclusive prefix sum of per-sample lengths: off[0] = 0, off[b+1] = off[b] + len[b].
 * Returns -1 (and stops) on a negative length. */
int ora_offsets(const int32_t* len, int32_t n, int64_t* off) {
  off[0] = 0;
  for (int32_t b = 0; b < n; ++b) {
    if (len[b] < 0) return -1;
    off[b + 1] = off[b] + (int64_t)len[b];
  }
  return 0;
}

/* Start of sample b's block in a dense jagged bias: the running sum of q_len*kv_len. */
int ora_bias_offsets(const int32_t* qlen, const int32_t* kvlen, int32_t n, int64_t* bo) {
  bo[0] = 0;
  for (int32_t b = 0; b < n; ++b) {
    if (qlen[b] < 0 || kvlen[b] < 0) return -1;
    bo[b + 1] = bo[b] + (int64_t)qlen[b] * (int64_t)kvlen[b];
  }
  return 0;
}

/* Block boundaries of BlockAttention as offsets of a refined batch: every sample of length n
 * contributes ceil(n / block) entries (its block starts, block rows apart), in sample order;
 * the remaining entries up to out[out_batch] hold the total row count (empty blocks).
 * Returns the number of blocks, or -1 when they exceed out_batch or block < 1. */
int64_t ora_block_offsets(const int64_t* off, int32_t n, int32_t block, int64_t* out,
                          int64_t out_batch) {
  if (block < 1) return -1;
  int64_t e = 0;
  for (int32_t b = 0; b < n; ++b) {
    for (int64_t start = off[b]; start < off[b + 1]; start += block) {
      if (e >= out_batch) return -1;
      out[e++] = start;
    }
  }
  for (int64_t x = e; x <= out_batch; ++x) out[x] = off[n];
  return e;
}

/* ------------------------------------------------------- relative position */

/* Bucket of a query-key distance: exact below 16, then four buckets per
 * doubling, clamped to the table width. */
int ora_relpos_bucket(int64_t delta, int32_t num_buckets) {
  if (delta < 0) delta = -delta;
  int64_t bucket;
  if (delta < 16) {
    bucket = delta;
  } else {
    int k = 0;                               /* position of the highest set bit */
    while ((delta >> (k + 1)) != 0) ++k;
    bucket = 16 + 4 * (int64_t)(k - 4) + ((delta >> (k - 2)) & 3);
  }
  if (bucket > num_buckets - 1) bucket = num_buckets - 1;
  return (int)bucket;
}

static double bias_value(const ora_problem* p, const double* bias, const int64_t* bo,
                         int64_t b, int h, int64_t i, int64_t j, int64_t n, int64_t m) {
  if (p->bias_kind == 1) {
    int64_t delta = (i + (m - n)) - j;
    return bias[(int64_t)h * p->num_buckets + ora_relpos_bucket(delta, p->num_buckets)];
  }
  if (p->bias_kind == 2) {
    return bias[(int64_t)p->heads * bo[b] + (int64_t)h * n * m + i * m + j];
  }
  return 0.0;
}

/* ------------------------------------------------------------- activations */

static double act(int mode, double x) {
  if (mode == 1) return x / (1.0 + exp(-x));                  /* SiLU */
  return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));                /* GELU, erf form */
}

static double act_grad(int mode, double x) {
  if (mode == 1) {
    double sg = 1.0 / (1.0 + exp(-x));
    return sg * (1.0 + x * (1.0 - sg));
  }
  double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
  double pdf = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
  return cdf + x * pdf;
}

/* BlockAttention ("Meta GEM Training Efficiency: ...", section "Bottleneck move 1": long
 * sequences become independent fixed-size blocks; "Meta Enhances GEM Training Efficiency ...",
 * "Exploring the Customized Kernel Library": windows in place of full attention): query i and
 * key j interact only when they fall in the same block of p->block consecutive rows. */
static int visible(const ora_problem* p, int64_t i, int64_t j, int64_t n, int64_t m) {
  if (p->block > 0 && i / p->block != j / p->block) return 0;
  /* sliding window ("GEM Training: How Meta Doubled ...", "Challenge 1": long sequences with a
   * short attention window; "Meta Enhances GEM Training Efficiency ...", "Leveraging Compute
   * Efficiency through Customized Kernels": attention over windows): the key must lie fewer
   * than `window` positions from the query's aligned position i + (m - n) */
  if (p->window > 0) {
    const int64_t dist = (i + (m - n)) - j;
    if (dist >= p->window || -dist >= p->window) return 0;
  }
  return !p->causal || j <= i + (m - n);
}

/* GDPA output weight of query i: 1 / (number of keys it attends over before masking), the
 * sample's kv_len, or with BlockAttention the length of i's block. */
static double gdpa_weight(const ora_problem* p, int64_t i, int64_t m) {
  if (!p->normalize || m <= 0) return 1.0;
  if (p->block > 0) {
    const int64_t start = (i / p->block) * p->block;
    const int64_t len = m - start < p->block ? m - start : p->block;
    return 1.0 / (double)len;
  }
  return 1.0 / (double)m;
}

static double score(const ora_problem* p, const double* q, const double* k, const double* bias,
                    const int64_t* bo, int64_t b, int h, int64_t qrow, int64_t krow,
                    int64_t i, int64_t j, int64_t n, int64_t m) {
  const int64_t H = p->heads, d = p->head_dim;
  const double* qi = q + (qrow * H + h) * d;
  const double* kj = k + (krow * H + h) * d;
  double dot = 0.0;
  for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
  return p->scale * dot + bias_value(p, bias, bo, b, h, i, j, n, m);
}

/* ---------------------------------------------------------------- forward */

/* q [Tq][H][d], k/v [Tkv][H][d], o [Tq][H][d], lse [H][Tq] (softmax only; may be NULL).
 * Rows whose query sees no key get o = 0 and lse = -inf. */
void ora_forward(const ora_problem* p, const int64_t* qo, const int64_t* ko,
                 const double* q, const double* k, const double* v, const double* bias,
                 const int64_t* bo, double* o, double* lse) {
  const int64_t B = p->batch, H = p->heads, d = p->head_dim;
  const int64_t Tq = qo[B];
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t item = 0; item < B * H; ++item) {
    const int64_t b = item / H;
    const int h = (int)(item % H);
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    double* s = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    for (int64_t i = 0; i < n; ++i) {
      double* oi = o + ((qo[b] + i) * H + h) * d;
      for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
      int64_t nvis = 0;
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        s[j] = score(p, q, k, bias, bo, b, h, qo[b] + i, ko[b] + j, i, j, n, m);
        ++nvis;
      }
      if (p->mode == 0) {
        if (nvis == 0) {
          if (lse) lse[h * Tq + qo[b] + i] = -INFINITY;
          continue;
        }
        double mx = -INFINITY;
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m) && s[j] > mx) mx = s[j];
        double l = 0.0;
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m)) l += exp(s[j] - mx);
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          const double pij = exp(s[j] - mx) / l;
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          for (int64_t c = 0; c < d; ++c) oi[c] += pij * vj[c];
        }
        if (lse) lse[h * Tq + qo[b] + i] = mx + log(l);
      } else {
        const double w = gdpa_weight(p, i, m);
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          const double pij = act(p->mode, s[j]);
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          for (int64_t c = 0; c < d; ++c) oi[c] += w * pij * vj[c];
        }
      }
    }
    free(s);
  }
}

/* --------------------------------------------------------------- backward */

/* Gradients of the scalar <O, dO>.  dq [Tq][H][d], dk/dv [Tkv][H][d] are fully written. */
void ora_backward(const ora_problem* p, const int64_t* qo, const int64_t* ko,
                  const double* q, const double* k, const double* v, const double* bias,
                  const int64_t* bo, const double* dout, double* dq, double* dk, double* dv) {
  const int64_t B = p->batch, H = p->heads, d = p->head_dim;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t item = 0; item < B * H; ++item) {
    const int64_t b = item / H;
    const int h = (int)(item % H);
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    for (int64_t i = 0; i < n; ++i)
      memset(dq + ((qo[b] + i) * H + h) * d, 0, sizeof(double) * (size_t)d);
    for (int64_t j = 0; j < m; ++j) {
      memset(dk + ((ko[b] + j) * H + h) * d, 0, sizeof(double) * (size_t)d);
      memset(dv + ((ko[b] + j) * H + h) * d, 0, sizeof(double) * (size_t)d);
    }
    double* s = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    double* pr = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    double* oi = (double*)malloc(sizeof(double) * (size_t)d);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t qrow = qo[b] + i;
      const double* qi = q + (qrow * H + h) * d;
      const double* doi = dout + (qrow * H + h) * d;
      double* dqi = dq + (qrow * H + h) * d;
      int64_t nvis = 0;
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        s[j] = score(p, q, k, bias, bo, b, h, qrow, ko[b] + j, i, j, n, m);
        ++nvis;
      }
      if (nvis == 0) continue;
      if (p->mode == 0) {
        /* P row, O row, then D = dO . O */
        double mx = -INFINITY, l = 0.0;
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m) && s[j] > mx) mx = s[j];
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m)) l += exp(s[j] - mx);
        for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          pr[j] = exp(s[j] - mx) / l;
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          for (int64_t c = 0; c < d; ++c) oi[c] += pr[j] * vj[c];
        }
        double D = 0.0;
        for (int64_t c = 0; c < d; ++c) D += doi[c] * oi[c];
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          const double* kj = k + ((ko[b] + j) * H + h) * d;
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          double* dkj = dk + ((ko[b] + j) * H + h) * d;
          double* dvj = dv + ((ko[b] + j) * H + h) * d;
          double dp = 0.0;
          for (int64_t c = 0; c < d; ++c) dp += doi[c] * vj[c];
          const double ds = pr[j] * (dp - D);
          for (int64_t c = 0; c < d; ++c) {
            dvj[c] += pr[j] * doi[c];
            dqi[c] += p->scale * ds * kj[c];
            dkj[c] += p->scale * ds * qi[c];
          }
        }
      } else {
        const double w = gdpa_weight(p, i, m);
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          const double* kj = k + ((ko[b] + j) * H + h) * d;
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          double* dkj = dk + ((ko[b] + j) * H + h) * d;
          double* dvj = dv + ((ko[b] + j) * H + h) * d;
          double dp = 0.0;
          for (int64_t c = 0; c < d; ++c) dp += doi[c] * vj[c];
          dp *= w;
          const double ds = act_grad(p->mode, s[j]) * dp;
          const double a = act(p->mode, s[j]);
          for (int64_t c = 0; c < d; ++c) {
            dvj[c] += w * a * doi[c];
            dqi[c] += p->scale * ds * kj[c];
            dkj[c] += p->scale * ds * qi[c];
          }
        }
      }
    }
    free(s);
    free(pr);
    free(oi);
  }
}

/* ------------------------------------------------ operand-rounding magnitudes */

/* Absolute-value contractions behind each output element, for bounding the error that comes
 * from rounding an operand of a product to a narrower format (relative error at most u per
 * element): the output's error from rounding P (or dS) is then at most u times
 *   cO[i]  = sum_j |P_ij| |V_j|            (GDPA: P_ij = w act(S_ij))
 *   cdV[j] = sum_i |P_ij| |dO_i|
 *   cdQ[i] = scale * sum_j |dS_ij| |K_j|
 *   cdK[j] = scale * sum_i |dS_ij| |Q_i|
 * over visible pairs, with P and dS exactly as in ora_forward / ora_backward (fp64).  Outputs
 * have the layouts of o, dv, dq, dk and are fully written; dout may be NULL (then only cO). */
void ora_abs_terms(const ora_problem* p, const int64_t* qo, const int64_t* ko,
                   const double* q, const double* k, const double* v, const double* bias,
                   const int64_t* bo, const double* dout, double* c_o, double* c_dq,
                   double* c_dk, double* c_dv) {
  const int64_t B = p->batch, H = p->heads, d = p->head_dim;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t item = 0; item < B * H; ++item) {
    const int64_t b = item / H;
    const int h = (int)(item % H);
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    for (int64_t i = 0; i < n; ++i) {
      memset(c_o + ((qo[b] + i) * H + h) * d, 0, sizeof(double) * (size_t)d);
      if (dout) memset(c_dq + ((qo[b] + i) * H + h) * d, 0, sizeof(double) * (size_t)d);
    }
    if (dout)
      for (int64_t j = 0; j < m; ++j) {
        memset(c_dk + ((ko[b] + j) * H + h) * d, 0, sizeof(double) * (size_t)d);
        memset(c_dv + ((ko[b] + j) * H + h) * d, 0, sizeof(double) * (size_t)d);
      }
    double* s = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    double* pr = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    for (int64_t i = 0; i < n; ++i) {
      const int64_t qrow = qo[b] + i;
      const double* qi = q + (qrow * H + h) * d;
      int64_t nvis = 0;
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        s[j] = score(p, q, k, bias, bo, b, h, qrow, ko[b] + j, i, j, n, m);
        ++nvis;
      }
      if (nvis == 0) continue;
      /* P row (softmax: normalised exponentials; GDPA: w act(S)) */
      double mx = -INFINITY, l = 0.0;
      const double w = gdpa_weight(p, i, m);
      if (p->mode == 0) {
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m) && s[j] > mx) mx = s[j];
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m)) l += exp(s[j] - mx);
      }
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        pr[j] = p->mode == 0 ? exp(s[j] - mx) / l : w * act(p->mode, s[j]);
      }
      double* coi = c_o + (qrow * H + h) * d;
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        const double* vj = v + ((ko[b] + j) * H + h) * d;
        for (int64_t c = 0; c < d; ++c) coi[c] += fabs(pr[j]) * fabs(vj[c]);
      }
      if (!dout) continue;
      const double* doi = dout + (qrow * H + h) * d;
      double D = 0.0;
      if (p->mode == 0) {
        /* D = dO . O with O = sum_j P_ij V_j */
        for (int64_t c = 0; c < d; ++c) {
          double oc = 0.0;
          for (int64_t j = 0; j < m; ++j)
            if (visible(p, i, j, n, m)) oc += pr[j] * v[((ko[b] + j) * H + h) * d + c];
          D += doi[c] * oc;
        }
      }
      double* cdqi = c_dq + (qrow * H + h) * d;
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        const double* kj = k + ((ko[b] + j) * H + h) * d;
        const double* vj = v + ((ko[b] + j) * H + h) * d;
        double* cdkj = c_dk + ((ko[b] + j) * H + h) * d;
        double* cdvj = c_dv + ((ko[b] + j) * H + h) * d;
        double dp = 0.0;
        for (int64_t c = 0; c < d; ++c) dp += doi[c] * vj[c];
        const double ds = p->mode == 0 ? pr[j] * (dp - D) : act_grad(p->mode, s[j]) * w * dp;
        for (int64_t c = 0; c < d; ++c) {
          cdvj[c] += fabs(pr[j]) * fabs(doi[c]);
          cdqi[c] += p->scale * fabs(ds) * fabs(kj[c]);
          cdkj[c] += p->scale * fabs(ds) * fabs(qi[c]);
        }
      }
    }
    free(s);
    free(pr);
  }
}

/* ------------------------------------------------------------ bias gradient */

/* Gradient of <O, dO> with respect to the additive bias ("Meta GEM Training Efficiency: ...",
 * section "Bottleneck move 1": custom biases, which a model trains).  The bias enters every
 * score S_ij additively, so its gradient is dS_ij = dL/dS_ij on visible pairs:
 *   softmax: dS = P (dO.V_j - D_i), D_i = dO_i.O_i;   GDPA: dS = act'(S) w (dO_i.V_j).
 * Dense bias (bias_kind 2): dbias has the bias layout, dS per element, 0 on pairs that are not
 * visible.  Relative-position table (bias_kind 1): dbias [H][num_buckets] accumulates dS over
 * every visible pair of its bucket; per-(sample, head) partials are summed over samples in
 * order, so the sum does not depend on the thread count. */
void ora_bias_grad(const ora_problem* p, const int64_t* qo, const int64_t* ko,
                   const double* q, const double* k, const double* v, const double* bias,
                   const int64_t* bo, const double* dout, double* dbias) {
  const int64_t B = p->batch, H = p->heads, d = p->head_dim, NB = p->num_buckets;
  double* part = NULL;
  if (p->bias_kind == 1) part = (double*)calloc((size_t)(B * H * NB), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t item = 0; item < B * H; ++item) {
    const int64_t b = item / H;
    const int h = (int)(item % H);
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    double* s = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m : 1));
    double* oi = (double*)malloc(sizeof(double) * (size_t)d);
    for (int64_t i = 0; i < n; ++i) {
      const int64_t qrow = qo[b] + i;
      const double* doi = dout + (qrow * H + h) * d;
      int64_t nvis = 0;
      for (int64_t j = 0; j < m; ++j) {
        if (p->bias_kind == 2) dbias[H * bo[b] + (int64_t)h * n * m + i * m + j] = 0.0;
        if (!visible(p, i, j, n, m)) continue;
        s[j] = score(p, q, k, bias, bo, b, h, qrow, ko[b] + j, i, j, n, m);
        ++nvis;
      }
      if (nvis == 0) continue;
      double mx = -INFINITY, l = 0.0, D = 0.0;
      if (p->mode == 0) {
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m) && s[j] > mx) mx = s[j];
        for (int64_t j = 0; j < m; ++j)
          if (visible(p, i, j, n, m)) l += exp(s[j] - mx);
        for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
        for (int64_t j = 0; j < m; ++j) {
          if (!visible(p, i, j, n, m)) continue;
          const double pij = exp(s[j] - mx) / l;
          const double* vj = v + ((ko[b] + j) * H + h) * d;
          for (int64_t c = 0; c < d; ++c) oi[c] += pij * vj[c];
        }
        for (int64_t c = 0; c < d; ++c) D += doi[c] * oi[c];
      }
      const double w = gdpa_weight(p, i, m);
      for (int64_t j = 0; j < m; ++j) {
        if (!visible(p, i, j, n, m)) continue;
        const double* vj = v + ((ko[b] + j) * H + h) * d;
        double dp = 0.0;
        for (int64_t c = 0; c < d; ++c) dp += doi[c] * vj[c];
        double ds;
        if (p->mode == 0) ds = exp(s[j] - mx) / l * (dp - D);
        else ds = act_grad(p->mode, s[j]) * w * dp;
        if (p->bias_kind == 2) {
          dbias[H * bo[b] + (int64_t)h * n * m + i * m + j] = ds;
        } else if (p->bias_kind == 1) {
          part[item * NB + ora_relpos_bucket((i + (m - n)) - j, p->num_buckets)] += ds;
        }
      }
    }
    free(s);
    free(oi);
  }
  if (p->bias_kind == 1) {
    for (int64_t x = 0; x < H * NB; ++x) dbias[x] = 0.0;
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < H; ++h)
        for (int64_t k2 = 0; k2 < NB; ++k2) dbias[h * NB + k2] += part[(b * H + h) * NB + k2];
    free(part);
  }
}

/* ------------------------------------------------------------- tile lists */

typedef struct {
  int32_t bm, bn;        /* forward: query rows per tile, key rows per kv step */
  int32_t slots;         /* >0: split long forward tiles for this many concurrent workers; <=0: never */
  int32_t bq_bm, bq_bn;  /* query-stationary backward: query rows per tile, key rows per step */
  int32_t bk_bn, bk_bm;  /* key-stationary backward: key rows per tile, query rows per step */
  int32_t fuse;          /* single backward pass: bit 0 for samples with one query tile, bit 1 for
                            samples with one key tile (and not one query tile) */
  int32_t window;        /* sliding window of the attention (0 = none), as in ora_problem */
} ora_sched_params;

typedef struct { int32_t b, t, lo, hi; } ora_rec;

static int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int32_t rec_cost(const ora_rec* r) { int32_t c = r->hi - r->lo; return c > 1 ? c : 1; }

/* Longest first; ties broken by sample, then tile, then first kv step. */
static int rec_cmp(const void* pa, const void* pb) {
  const ora_rec* a = (const ora_rec*)pa;
  const ora_rec* b = (const ora_rec*)pb;
  int32_t ca = rec_cost(a), cb = rec_cost(b);
  if (ca != cb) return ca > cb ? -1 : 1;
  if (a->b != b->b) return a->b < b->b ? -1 : 1;
  if (a->t != b->t) return a->t < b->t ? -1 : 1;
  if (a->lo != b->lo) return a->lo < b->lo ? -1 : 1;
  return 0;
}

/* Keys [*lo, *hi) that some query of rows [r0, r1) may see (causal, window); returns 0 when
 * there are none.  Query i sees key j iff j <= i + (m - n) (causal) and, with a window W,
 * i + (m - n) - W < j < i + (m - n) + W. */
static int kv_range(int causal, int32_t window, int64_t r0, int64_t r1, int64_t n, int64_t m,
                    int64_t* lo, int64_t* hi) {
  const int64_t dl = m - n;
  int64_t a = 0, e = m;
  if (window > 0) {
    a = r0 + dl - window + 1;
    e = r1 - 1 + dl + window;
  }
  if (causal && r1 + dl < e) e = r1 + dl;
  if (a < 0) a = 0;
  if (e > m) e = m;
  *lo = a;
  *hi = e;
  return e > a;
}

/* Queries [*lo, *hi) that may see some key of columns [c0, c1). */
static int q_range(int causal, int32_t window, int64_t c0, int64_t c1, int64_t n, int64_t m,
                   int64_t* lo, int64_t* hi) {
  const int64_t dl = m - n;
  int64_t a = 0, e = n;
  if (window > 0) {
    a = c0 - dl - window + 1;
    e = c1 - 1 - dl + window;
  }
  if (causal && c0 - dl > a) a = c0 - dl;
  if (a < 0) a = 0;
  if (e > n) e = n;
  *lo = a;
  *hi = e;
  return e > a;
}

/* Step range [*s0, *s1) of `step`-row steps covering [lo, hi), or the empty range at `empty`. */
static void step_range(int nonempty, int64_t lo, int64_t hi, int64_t step, int64_t empty,
                       int64_t* s0, int64_t* s1) {
  if (nonempty) {
    *s0 = lo / step;
    *s1 = ceil_div64(hi, step);
  } else {
    *s0 = *s1 = empty;
  }
}

/*
 * Builds the forward, combine and two backward tile lists.
 * Forward record {b, t, kb, ke}: query tile t of sample b over kv steps [kb, ke).
 * fwd_slot[w]: first partial slot of a split tile's chunk (slot base + chunk), -1 if unsplit.
 * Combine record {b, t, slot_base, n_chunks} for every split tile, in (b, t) order.
 * Query-stationary backward record {b, t, 0, n_kv_steps}; key-stationary {b, u, q_first, q_end}.
 * counts[0..3] = forward, combine, query-stationary, key-stationary record counts;
 * counts[4] = split threshold (0 when splitting is off).
 * Returns -1 on malformed offsets, -2 if a capacity is exceeded.
 */
int ora_schedule(const int64_t* qo, const int64_t* ko, int32_t B, int32_t H, int32_t causal,
                 const ora_sched_params* sp, int32_t* fwd, int32_t* fwd_slot, int32_t* comb,
                 int32_t* bq, int32_t* bk, int64_t cap, int64_t* counts) {
  if (qo[0] != 0 || ko[0] != 0) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (qo[b + 1] < qo[b] || ko[b + 1] < ko[b]) return -1;

  /* forward tiles in (b, t) order and their costs */
  int64_t ntiles = 0, sumcost = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    const int64_t nqt = ceil_div64(n, sp->bm);
    for (int64_t t = 0; t < nqt; ++t) {
      int64_t r1 = (t + 1) * sp->bm < n ? (t + 1) * sp->bm : n;
      int64_t lo, hi, s0, s1;
      const int any = kv_range(causal, sp->window, t * sp->bm, r1, n, m, &lo, &hi);
      step_range(any, lo, hi, sp->bn, 0, &s0, &s1);
      const int64_t nkv = s1 - s0;
      sumcost += nkv > 1 ? nkv : 1;
      ++ntiles;
    }
  }
  int64_t C = 0;
  if (sp->slots > 0) {
    C = ceil_div64((int64_t)H * sumcost, sp->slots);
    if (C < 8) C = 8;
  }
  ora_rec* recs = (ora_rec*)malloc(sizeof(ora_rec) * (size_t)(ntiles + 1));
  int64_t nf = 0, nc = 0, slot = 0;
  int32_t* slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)(ntiles + 1));
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    const int64_t nqt = ceil_div64(n, sp->bm);
    for (int64_t t = 0; t < nqt; ++t) {
      int64_t r1 = (t + 1) * sp->bm < n ? (t + 1) * sp->bm : n;
      int64_t lo, hi, s0, s1;
      const int any = kv_range(causal, sp->window, t * sp->bm, r1, n, m, &lo, &hi);
      step_range(any, lo, hi, sp->bn, 0, &s0, &s1);
      const int64_t nkv = s1 - s0;
      if (C > 0 && nkv > C) {
        int64_t nch = ceil_div64(nkv, C);
        if (nc >= cap) { free(recs); free(slot_of); return -2; }
        comb[4 * nc + 0] = b; comb[4 * nc + 1] = (int32_t)t;
        comb[4 * nc + 2] = (int32_t)slot; comb[4 * nc + 3] = (int32_t)nch;
        ++nc;
        for (int64_t c = 0; c < nch; ++c) {
          ora_rec r = {b, (int32_t)t, (int32_t)(s0 + c * nkv / nch),
                       (int32_t)(s0 + (c + 1) * nkv / nch)};
          recs = (ora_rec*)realloc(recs, sizeof(ora_rec) * (size_t)(nf + 1));
          slot_of = (int32_t*)realloc(slot_of, sizeof(int32_t) * (size_t)(nf + 1));
          recs[nf] = r;
          slot_of[nf] = (int32_t)(slot + c);
          ++nf;
        }
        slot += nch;
      } else {
        recs = (ora_rec*)realloc(recs, sizeof(ora_rec) * (size_t)(nf + 1));
        slot_of = (int32_t*)realloc(slot_of, sizeof(int32_t) * (size_t)(nf + 1));
        ora_rec r = {b, (int32_t)t, (int32_t)s0, (int32_t)s1};
        recs[nf] = r;
        slot_of[nf] = -1;
        ++nf;
      }
    }
  }
  if (nf > cap) { free(recs); free(slot_of); return -2; }
  /* sort (record, slot) pairs together by the record key */
  typedef struct { ora_rec r; int32_t slot; } pair_t;
  pair_t* pairs = (pair_t*)malloc(sizeof(pair_t) * (size_t)(nf + 1));
  for (int64_t w = 0; w < nf; ++w) { pairs[w].r = recs[w]; pairs[w].slot = slot_of[w]; }
  qsort(pairs, (size_t)nf, sizeof(pair_t), rec_cmp);  /* key is a total order: result unique */
  for (int64_t w = 0; w < nf; ++w) {
    fwd[4 * w + 0] = pairs[w].r.b; fwd[4 * w + 1] = pairs[w].r.t;
    fwd[4 * w + 2] = pairs[w].r.lo; fwd[4 * w + 3] = pairs[w].r.hi;
    fwd_slot[w] = pairs[w].slot;
  }
  free(pairs); free(recs); free(slot_of);

  /* backward lists */
  ora_rec* rq = (ora_rec*)malloc(sizeof(ora_rec) * 1);
  ora_rec* rk = (ora_rec*)malloc(sizeof(ora_rec) * 1);
  int64_t nq = 0, nk = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = qo[b + 1] - qo[b], m = ko[b + 1] - ko[b];
    const int64_t nqt = ceil_div64(n, sp->bq_bm);    /* query tiles of the q-stationary pass */
    const int64_t nkt = ceil_div64(m, sp->bk_bn);    /* key tiles of the kv-stationary pass */
    const int one_q = (sp->fuse & 1) && nqt == 1;
    const int one_k = (sp->fuse & 2) && !one_q && nkt == 1;
    if (!one_k) {            /* q-stationary pass: every query tile */
      for (int64_t t = 0; t < nqt; ++t) {
        int64_t r1 = (t + 1) * sp->bq_bm < n ? (t + 1) * sp->bq_bm : n;
        int64_t lo, hi, s0, s1;
        const int any = kv_range(causal, sp->window, t * sp->bq_bm, r1, n, m, &lo, &hi);
        step_range(any, lo, hi, sp->bq_bn, 0, &s0, &s1);
        /* a single pass also owns dK/dV, so it visits every key tile (unseen keys get zeros) */
        if (one_q) {
          s0 = 0;
          s1 = ceil_div64(m, sp->bq_bn);
        }
        rq = (ora_rec*)realloc(rq, sizeof(ora_rec) * (size_t)(nq + 1));
        ora_rec r = {b, (int32_t)t, (int32_t)s0, (int32_t)s1};
        rq[nq++] = r;
      }
    }
    if (!one_q) {            /* kv-stationary pass: every key tile */
      const int64_t nqs = ceil_div64(n, sp->bk_bm);
      for (int64_t u = 0; u < nkt; ++u) {
        int64_t c1 = (u + 1) * sp->bk_bn < m ? (u + 1) * sp->bk_bn : m;
        int64_t lo, hi, s0, s1;
        const int any = q_range(causal, sp->window, u * sp->bk_bn, c1, n, m, &lo, &hi);
        step_range(any, lo, hi, sp->bk_bm, nqs, &s0, &s1);
        /* a single pass also owns dQ, so it visits every query tile (unseeing queries get zeros) */
        if (one_k) {
          s0 = 0;
          s1 = nqs;
        }
        rk = (ora_rec*)realloc(rk, sizeof(ora_rec) * (size_t)(nk + 1));
        ora_rec r = {b, (int32_t)u, (int32_t)s0, (int32_t)s1};
        rk[nk++] = r;
      }
    }
  }
  if (nq > cap || nk > cap) { free(rq); free(rk); return -2; }
  qsort(rq, (size_t)nq, sizeof(ora_rec), rec_cmp);
  qsort(rk, (size_t)nk, sizeof(ora_rec), rec_cmp);
  for (int64_t w = 0; w < nq; ++w) {
    bq[4 * w + 0] = rq[w].b; bq[4 * w + 1] = rq[w].t; bq[4 * w + 2] = rq[w].lo; bq[4 * w + 3] = rq[w].hi;
  }
  for (int64_t w = 0; w < nk; ++w) {
    bk[4 * w + 0] = rk[w].b; bk[4 * w + 1] = rk[w].t; bk[4 * w + 2] = rk[w].lo; bk[4 * w + 3] = rk[w].hi;
  }
  free(rq); free(rk);
  counts[0] = nf; counts[1] = nc; counts[2] = nq; counts[3] = nk; counts[4] = C;
  return 0;
}

/* ------------------------------------------------------------------ MXFP8 */

/* Value of an E4M3 magnitude code 0..126 (sign bit clear): 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals at exponent field 0. */
double ora_e4m3_magnitude(int code) {
  const int e = (code >> 3) & 15, f = code & 7;
  if (e == 0) return ldexp((double)f / 8.0, -6);
  return ldexp(1.0 + (double)f / 8.0, e - 7);
}

/* Full decode of a byte: sign bit 7; 0x7F and 0xFF are NaN. */
double ora_e4m3_decode(int code) {
  code &= 255;
  if ((code & 127) == 127) return NAN;
  const double mag = ora_e4m3_magnitude(code & 127);
  return (code & 128) ? -mag : mag;
}

/* Nearest finite E4M3 magnitude to y >= 0 by exhaustive search; a tie goes to
 * the even code.  Values past the largest (448) saturate to it. */
static int e4m3_nearest(double y) {
  int best = 0;
  double bestd = fabs(y - ora_e4m3_magnitude(0));
  for (int c = 1; c <= 126; ++c) {
    const double dist = fabs(y - ora_e4m3_magnitude(c));
    if (dist < bestd || (dist == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      bestd = dist;
    }
  }
  return best;
}

/*
 * Microscaling FP8 (OCP MX v1.0): per 32 consecutive elements of a row, a
 * shared power-of-two scale 2^e stored as e + 127, with e = floor(log2 amax) - 8
 * (8 = largest E4M3 exponent) clamped to [-127, 127], and elements x * 2^-e
 * rounded to E4M3.  An all-zero block stores scale 127 and zero codes.
 * x [rows][d], codes [rows][d], scales [rows][d/32].
 */
int ora_mxfp8_quantize(const double* x, int64_t rows, int32_t d, uint8_t* codes, uint8_t* scales) {
  if (d % 32 != 0) return -1;
  const int32_t nblk = d / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t blk = 0; blk < nblk; ++blk) {
      const double* xb = x + r * d + blk * 32;
      uint8_t* cb = codes + r * d + blk * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs(xb[i]) > amax) amax = fabs(xb[i]);
      if (amax == 0.0) {
        scales[r * nblk + blk] = 127;
        for (int i = 0; i < 32; ++i) cb[i] = 0;
        continue;
      }
      int E;
      frexp(amax, &E);                 /* amax = f * 2^E, f in [0.5, 1): floor(log2 amax) = E - 1 */
      int e = (E - 1) - 8;
      if (e < -127) e = -127;
      if (e > 127) e = 127;
      scales[r * nblk + blk] = (uint8_t)(e + 127);
      for (int i = 0; i < 32; ++i) {
        const double y = ldexp(xb[i], -e);
        const int mag = e4m3_nearest(fabs(y));
        cb[i] = (uint8_t)(mag | (signbit(y) ? 128 : 0));
      }
    }
  }
  return 0;
}

/* codes/scales back to values: decode(code) * 2^(scale - 127). */
void ora_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t d,
                          double* x) {
  const int32_t nblk = d / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int32_t c = 0; c < d; ++c)
      x[r * d + c] = ldexp(ora_e4m3_decode(codes[r * d + c]), (int)scales[r * nblk + c / 32] - 127);
}

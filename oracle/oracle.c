/*
 * oracle.c -- plain, slow, fp64 CPU reference for the quantized MoE expert
 * forward at decode time.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The GPU library never calls it and
 * shares no code, header, table or helper with it.
 *
 * Sources (the Flash-MoE pages; titles as published):
 *  [P1] "397B MoE en MacBook: Motor Flash-MoE a 4,4 t/s" (aibit.im, Spanish)
 *  [P2] "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook
 *       Pro mit reinem C/Metal" (openclawradar.com, German)
 *  [P3] "Flash-MoE - Executando um modelo de 397 bilhoes de parametros em um
 *       notebook" (news.hada.io, Portuguese)
 *
 * What is computed, and where the pages say so:
 *  - Dequantization: weight = code * scale + bias, code an unsigned 4-bit
 *    ("nibble") or 2-bit value, with one scale and one bias per group of inputs
 *    ([P1] "2. Kernel de desquantizacion optimizado con FMA", the "before"
 *    form; [P2] "FMA-optimierter Dequant-Kernel"). The pages fix neither the
 *    group size nor its axis nor the dtype of scale and bias; the reading taken
 *    is groups of `group` consecutive input columns of one row, bf16 scale and
 *    bias. The fp64 product code*scale+bias is exact (a <=4-bit integer times an
 *    8-bit significand plus an 8-bit significand), so W is known exactly.
 *  - Matrix-vector product: y = W x, summed in ascending column order in fp64
 *    ([P2] "Metal-Compute-Shader": dequantized matrix-vector multiplication).
 *  - Expert: SwiGLU feed-forward out = down( silu(gate x) * (up x) ) with
 *    silu(z) = z / (1 + exp(-z)) ([P2] "Metal-Compute-Shader": fused SwiGLU
 *    activation; gate/up/down projections of each expert).
 *  - Routing: logits = R x, softmax over the experts, the top K by probability
 *    ([P2] "Pipeline-Leistung": softmax + top-K routing; [P2] "Technische
 *    Implementierung": 512 experts per layer, K=4 active per token plus one
 *    shared expert). The pages say nothing of renormalising or of ties; the
 *    reading taken is: order by probability descending, lower expert index
 *    first on an exact tie, and renormalise the K chosen probabilities to sum 1.
 *    softmax being strictly increasing, that order is the order of the logits,
 *    which is what is compared (fp64 probabilities far below the largest round
 *    to 0 and would tie).
 *  - Combine: out = residual + sum_k w_k E_k(x) + sigmoid(g . x) E_shared(x)
 *    ([P2] "Metal-Compute-Shader": MoE combination + residual + sigmoid gate
 *    as one fused kernel). The gate is read as a scalar sigmoid of the dot
 *    product of a learned vector g with x.
 *  - RMS scaling between layers: x = h / sqrt(mean(h^2) + eps), two stages (sum
 *    of squares, then apply) ([P2] "Metal-Compute-Shader": RMS normalization,
 *    two-stage), with no learned weight and eps = 1e-6 (reading).
 *
 * Every sum below runs in a fixed order, so the result does not depend on the
 * number of OpenMP threads (threads split output rows only).
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Thread count for the row-parallel loops (results do not depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

int orc_get_threads(void) { return omp_get_max_threads(); }

/* bf16 bit pattern -> fp64 (exact). */
double orc_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* W[r][c] = code[r][c] * scale[r][c/group] + bias[r][c/group]   (fp64, exact) */
int orc_dequant(int rows, int cols, int group, const uint8_t *codes, const uint16_t *scale,
                const uint16_t *bias, double *W) {
  if (rows < 0 || cols <= 0 || group <= 0 || cols % group) return -1;
  const int ng = cols / group;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    for (int c = 0; c < cols; ++c) {
      double s = orc_bf16(scale[(int64_t)r * ng + c / group]);
      double b = orc_bf16(bias[(int64_t)r * ng + c / group]);
      double q = (double)codes[(int64_t)r * cols + c];
      double p = q * s;
      W[(int64_t)r * cols + c] = p + b;
    }
  }
  return 0;
}

/* y[r] = sum_{c ascending} (code*scale + bias) * x[c]   -- the plain definition. */
int orc_qmatvec(int rows, int cols, int group, const uint8_t *codes, const uint16_t *scale,
                const uint16_t *bias, const double *x, double *y) {
  if (rows < 0 || cols <= 0 || group <= 0 || cols % group) return -1;
  const int ng = cols / group;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    const uint8_t *cr = codes + (int64_t)r * cols;
    double acc = 0.0;
    for (int g = 0; g < ng; ++g) {
      double s = orc_bf16(scale[(int64_t)r * ng + g]);
      double b = orc_bf16(bias[(int64_t)r * ng + g]);
      for (int j = 0; j < group; ++j) {
        int c = g * group + j;
        double w = (double)cr[c] * s;
        w = w + b;
        double t = w * x[c];
        acc = acc + t;
      }
    }
    y[r] = acc;
  }
  return 0;
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

double orc_sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

typedef struct {
  const uint8_t *codes;
  const uint16_t *scale;
  const uint16_t *bias;
} orc_qmat;

/* One SwiGLU expert: gate, up are [inter][hidden]; down is [hidden][inter].
 * h (optional, [inter]) receives silu(gate x) * (up x); out ([hidden]) the expert output. */
int orc_expert(int hidden, int inter, int group, const orc_qmat *gate, const orc_qmat *up,
               const orc_qmat *down, const double *x, double *h, double *out) {
  double *g = (double *)malloc(sizeof(double) * (size_t)inter * 3);
  if (!g) return -3;
  double *u = g + inter, *hh = g + 2 * (size_t)inter;
  int rc = orc_qmatvec(inter, hidden, group, gate->codes, gate->scale, gate->bias, x, g);
  if (!rc) rc = orc_qmatvec(inter, hidden, group, up->codes, up->scale, up->bias, x, u);
  if (!rc) {
    for (int r = 0; r < inter; ++r) hh[r] = orc_silu(g[r]) * u[r];
    if (h) memcpy(h, hh, sizeof(double) * (size_t)inter);
    rc = orc_qmatvec(hidden, inter, group, down->codes, down->scale, down->bias, hh, out);
  }
  free(g);
  return rc;
}

/* logits[e] = sum_{i ascending} R[e][i] * x[i], R fp32 [n_experts][hidden]. */
int orc_router(int n_experts, int hidden, const float *R, const double *x, double *logits) {
#pragma omp parallel for schedule(static)
  for (int e = 0; e < n_experts; ++e) {
    double acc = 0.0;
    for (int i = 0; i < hidden; ++i) {
      double t = (double)R[(int64_t)e * hidden + i] * x[i];
      acc = acc + t;
    }
    logits[e] = acc;
  }
  return 0;
}

/* p = softmax(logits); pick the k largest p (lower index first on exact ties),
 * in that order; w_j = p[idx_j] / sum of the k chosen p. prob (optional) gets p.
 * softmax is strictly increasing in each logit, so the k largest p are the k largest
 * logits; they are ranked by the logits, because in fp64 every p more than ~745
 * below the largest logit rounds to 0 and would tie with the rest. A NaN logit
 * counts as -infinity (probability 0). */
static double rank_key(double l) { return l == l ? l : -INFINITY; }

int orc_route(int n, int k, const double *logits, int32_t *idx, double *w, double *prob) {
  if (n <= 0 || k < 1 || k > n) return -1;
  double *p = (double *)malloc(sizeof(double) * (size_t)n);
  char *taken = (char *)calloc((size_t)n, 1);
  if (!p || !taken) {
    free(p);
    free(taken);
    return -3;
  }
  double m = rank_key(logits[0]);
  for (int e = 1; e < n; ++e)
    if (rank_key(logits[e]) > m) m = rank_key(logits[e]);
  double z = 0.0;
  for (int e = 0; e < n; ++e) {
    p[e] = exp(rank_key(logits[e]) - m);
    z = z + p[e];
  }
  for (int e = 0; e < n; ++e) p[e] = p[e] / z;
  /* k passes of "largest remaining logit, smallest index on a tie" */
  double sum = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < n; ++e) {
      if (taken[e]) continue;
      if (best < 0 || rank_key(logits[e]) > rank_key(logits[best])) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
    sum = sum + p[best];
  }
  for (int j = 0; j < k; ++j) w[j] = p[idx[j]] / sum;
  if (prob) memcpy(prob, p, sizeof(double) * (size_t)n);
  free(p);
  free(taken);
  return 0;
}

/* sigmoid(sum_{i ascending} g[i] * x[i]) */
double orc_shared_gate(int hidden, const float *g, const double *x) {
  double acc = 0.0;
  for (int i = 0; i < hidden; ++i) {
    double t = (double)g[i] * x[i];
    acc = acc + t;
  }
  return orc_sigmoid(acc);
}

/* One MoE layer for one token.
 * experts: n_experts entries of {gate, up, down}; only the chosen ones are read
 * (the others may hold NULL pointers). shared: {gate, up, down} of the shared expert.
 * out[i] = residual[i] + sum_j w_j * E_{idx_j}(x)[i] + sigmoid(g . x) * E_shared(x)[i].
 * Returns -2 (and fills idx, w) when a chosen expert has NULL codes. */
int orc_moe_layer(int hidden, int inter, int group, int n_experts, int k, const float *R,
                  const float *gvec, const orc_qmat *experts /* [n_experts][3] */,
                  const orc_qmat *shared /* [3] */, const double *x, const double *residual,
                  double *out, int32_t *idx, double *w, double *sigma_out) {
  double *logits = (double *)malloc(sizeof(double) * ((size_t)n_experts + (size_t)hidden));
  if (!logits) return -3;
  double *d = logits + n_experts;
  int rc = orc_router(n_experts, hidden, R, x, logits);
  if (!rc) rc = orc_route(n_experts, k, logits, idx, w, NULL);
  for (int j = 0; !rc && j < k; ++j)
    if (!experts[3 * idx[j]].codes || !experts[3 * idx[j] + 1].codes || !experts[3 * idx[j] + 2].codes)
      rc = -2;
  if (!rc) {
    double sig = orc_shared_gate(hidden, gvec, x);
    if (sigma_out) *sigma_out = sig;
    for (int i = 0; i < hidden; ++i) out[i] = residual[i];
    for (int j = 0; j < k && !rc; ++j) {
      const orc_qmat *E = experts + 3 * idx[j];
      rc = orc_expert(hidden, inter, group, E, E + 1, E + 2, x, NULL, d);
      for (int i = 0; i < hidden && !rc; ++i) out[i] = out[i] + w[j] * d[i];
    }
    if (!rc) {
      rc = orc_expert(hidden, inter, group, shared, shared + 1, shared + 2, x, NULL, d);
      for (int i = 0; i < hidden && !rc; ++i) out[i] = out[i] + sig * d[i];
    }
  }
  free(logits);
  return rc;
}

/* x = h / sqrt(sum(h^2) / n + eps): stage 1 the sum of squares, stage 2 the scaling. */
int orc_rms_scale(int n, const double *h, double eps, double *x) {
  if (n <= 0) return -1;
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss = ss + h[i] * h[i];
  double r = sqrt(ss / (double)n + eps);
  for (int i = 0; i < n; ++i) x[i] = h[i] / r;
  return 0;
}

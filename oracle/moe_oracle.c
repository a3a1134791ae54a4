/*
 * Reference oracle for one routed-expert MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the GPU
 * library.
 *
 * It is the plain definition of what the layer computes, written for a
 * reader to check by eye: full sorts, per-token loops, double-precision
 * accumulation, no blocking or fusion.
 *
 * Sources (FreeToken pages):
 *  - each token activates a subset of experts, DeepSeek-V4-Flash picks 6 of
 *    256 routed experts per layer: RTX-4090 page, "How the MoE memory
 *    hierarchy works"; llama page, "Official project overview".
 *  - experts are whole (layer, expert) entries under one logical mapping on
 *    CPU and GPU: RTX-4090 page, same section.  Caching and streaming change
 *    where weights live, never the arithmetic, so one layer's result is this
 *    function of (x, logits, weights).
 * The pages state no layer math.  Readings taken where they are silent:
 *  - gate: softmax over the k selected logits (= full softmax renormalised
 *    over the top-k); no bias, scaling factor or shared expert.
 *  - top-k order: descending logit, ties to the lower expert id, compared by
 *    value (-0 == +0).
 *  - expert FFN: SwiGLU (Shazeer 2020), h = SiLU(x Wg^T) * (x Wu^T),
 *    y = h Wd^T, SiLU(z) = z / (1 + exp(-z)); no biases.
 *  - grouping: stable counting sort by expert (order (t, j) inside an
 *    expert, experts ascending).
 *
 * Weights are given per expert as row-major matrices: wg[e], wu[e] are
 * [f][d] (row i = unit i), wd[e] is [d][f] (row o = output channel o), in
 * fp32 (dtype 0) or bf16 bit patterns (dtype 1, upcast exactly).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double elem(const void* p, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* a1: logits[t][e] = sum_c x[t][c] * wr[e][c], double sum rounded once to fp32. */
void oracle_router_logits(const float* x, const float* wr, int T, int d, int E, float* logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int c = 0; c < d; ++c) s += (double)x[(int64_t)t * d + c] * (double)wr[(int64_t)e * d + c];
      logits[(int64_t)t * E + e] = (float)s;
    }
}

typedef struct {
  float v;
  int32_t e;
} scored;

/* Order: larger logit first; equal logits (by value) -> smaller expert id first. */
static int by_logit_desc_then_id(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->e > y->e) - (x->e < y->e);
}

/* a2: ids[t][0..k) = first k experts in the order above; w = softmax over the
 * k selected logits (double). */
void oracle_route(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  scored* row = (scored*)malloc(sizeof(scored) * (size_t)E);
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      row[e].v = logits[(int64_t)t * E + e];
      row[e].e = e;
    }
    qsort(row, (size_t)E, sizeof(scored), by_logit_desc_then_id);
    const double m = (double)row[0].v;
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp((double)row[j].v - m);
    for (int j = 0; j < k; ++j) {
      ids[(int64_t)t * k + j] = row[j].e;
      w[(int64_t)t * k + j] = exp((double)row[j].v - m) / z;
    }
  }
  free(row);
}

/* a5: stable counting sort of the flat assignments a = t*k + j by expert id.
 * counts[e], offsets[e] = sum of counts below e (offsets[E] = T*k),
 * perm[p] = a for sorted position p, inv[a] = p.  Returns 0, or -1 if an id is
 * outside [0, E). */
int oracle_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                   int32_t* perm, int32_t* inv) {
  const int64_t A = (int64_t)T * k;
  if (E <= 0 || T < 0 || k < 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < A; ++a) {
    if (ids[a] < 0 || ids[a] >= E) return -1;
    counts[ids[a]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t a = 0; a < A; ++a) {
    const int32_t e = ids[a];
    const int32_t p = offsets[e] + seen[e]++;
    perm[p] = (int32_t)a;
    inv[a] = p;
  }
  free(seen);
  return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* a6 for one token row x (length d) and one expert: y (length d). */
static void expert_ffn(const void* x, int xdtype, int64_t xoff, const void* wg, const void* wu,
                       const void* wd, int wdtype, int d, int f, double* h, double* y) {
  for (int i = 0; i < f; ++i) {
    double g = 0.0, u = 0.0;
    for (int c = 0; c < d; ++c) {
      const double xc = elem(x, xdtype, xoff + c);
      g += xc * elem(wg, wdtype, (int64_t)i * d + c);
      u += xc * elem(wu, wdtype, (int64_t)i * d + c);
    }
    h[i] = silu(g) * u;
  }
  for (int o = 0; o < d; ++o) {
    double s = 0.0;
    for (int i = 0; i < f; ++i) s += h[i] * elem(wd, wdtype, (int64_t)o * f + i);
    y[o] = s;
  }
}

/* a6 for a list of assignments: y[q] = FFN_{ids[a]}(x[a / k]) for a = assign[q].
 * wg/wu/wd are indexed by expert id. */
void oracle_expert_ffn(const void* x, int xdtype, int d, int f, int k, const int32_t* ids,
                       const void* const* wg, const void* const* wu, const void* const* wd,
                       int wdtype, int n_assign, const int32_t* assign, double* y) {
#pragma omp parallel
  {
    double* h = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
    for (int q = 0; q < n_assign; ++q) {
      const int32_t a = assign[q];
      const int32_t e = ids[a];
      expert_ffn(x, xdtype, (int64_t)(a / k) * d, wg[e], wu[e], wd[e], wdtype, d, f, h,
                 y + (int64_t)q * d);
    }
    free(h);
  }
}

/* Whole layer for a list of tokens: out[q] = sum_j w[t][j] * FFN_{ids[t][j]}(x[t]),
 * j ascending, t = tokens[q].  Routes every token (ids, w written for all T).
 * The (token, j) expert FFNs are independent, so they run in parallel, 64 tokens at a time;
 * each token's weighted sum is then formed in j order.  Every output element is the same
 * arithmetic however many threads run. */
void oracle_moe_layer(const void* x, int xdtype, const float* logits, int T, int d, int E, int k,
                      int f, const void* const* wg, const void* const* wu, const void* const* wd,
                      int wdtype, int n_tok, const int32_t* tokens, int32_t* ids, double* w,
                      double* out) {
  oracle_route(logits, T, E, k, ids, w);
  enum { CHUNK = 64 };
  double* y = (double*)malloc(sizeof(double) * (size_t)CHUNK * k * d);
  for (int q0 = 0; q0 < n_tok; q0 += CHUNK) {
    const int nq = n_tok - q0 < CHUNK ? n_tok - q0 : CHUNK;
#pragma omp parallel
    {
      double* h = (double*)malloc(sizeof(double) * (size_t)f);
#pragma omp for schedule(dynamic, 1)
      for (int qj = 0; qj < nq * k; ++qj) {
        const int t = tokens[q0 + qj / k], j = qj % k;
        const int32_t e = ids[(int64_t)t * k + j];
        expert_ffn(x, xdtype, (int64_t)t * d, wg[e], wu[e], wd[e], wdtype, d, f, h,
                   y + (int64_t)qj * d);
      }
      free(h);
    }
#pragma omp parallel for schedule(static)
    for (int qq = 0; qq < nq; ++qq) {
      const int t = tokens[q0 + qq];
      double* o = out + (int64_t)(q0 + qq) * d;
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        const double wj = w[(int64_t)t * k + j];
        const double* yj = y + ((int64_t)qq * k + j) * d;
        for (int c = 0; c < d; ++c) o[c] += wj * yj[c];
      }
    }
  }
  free(y);
}

/* Thread count of the parallel loops above (benchmark baselines time 1 and all cores). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* a7 alone: out[t] = sum_j w[t][j] * yperm[inv[t*k+j]], j ascending (double). */
void oracle_combine(const double* yperm, const int32_t* inv, const double* w, int T, int k, int d,
                    double* out) {
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int j = 0; j < k; ++j)
        s += w[(int64_t)t * k + j] * yperm[(int64_t)inv[(int64_t)t * k + j] * d + c];
      out[(int64_t)t * d + c] = s;
    }
}

/*
 * Seeded, counter-based generator of synthetic inputs for the routed-MoE layer.
 *
 * This module is shared by the test oracle and by the GPU path's tests and
 * benchmark.  It holds none of the layer's arithmetic: it only produces
 * numbers (activations, weights, router logits, routing traces) from
 * (seed, tensor tag, logical index), so any element can be regenerated on its
 * own without materialising a whole tensor.
 *
 * Bits: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  The stream for (seed, tag) starts at a
 * mixed key; draw i is mix64(key + (i + 1) * golden_gamma), which is the
 * i-th output of a SplitMix64 generator seeded with that key.
 *
 * Normals: the classical "sum of twelve uniforms" (Irwin-Hall, n = 12)
 * approximation of N(0,1), computed with exact integers: twelve 16-bit
 * uniforms come from three draws, their sum S has mean 393210 and variance
 * 65536^2 - 1, and z = (2S - 786420) / 2^17 is exactly representable in fp32.
 * A tensor element with standard deviation sd is the single fp32 product
 * z * sd.  No libm call is involved, so values are bit-identical on any
 * IEEE machine.  bf16 values are the round-to-nearest-even of those fp32
 * values.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return mix64(mix64(seed + GAMMA) ^ (tag * GAMMA + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline float normal_from_key(uint64_t key, uint64_t i) {
  int64_t s = 0;
  for (int w = 0; w < 3; ++w) {
    uint64_t b = draw(key, 3 * i + (uint64_t)w);
    s += (int64_t)(b & 0xFFFF) + (int64_t)((b >> 16) & 0xFFFF) +
         (int64_t)((b >> 32) & 0xFFFF) + (int64_t)(b >> 48);
  }
  return (float)(2 * s - 786420) * (1.0f / 131072.0f);
}

static inline double uniform_from_key(uint64_t key, uint64_t i) {
  return (double)(draw(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

static inline uint16_t f32_to_bf16_rne(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t gen_u64(uint64_t seed, uint64_t tag, uint64_t i) { return draw(stream_key(seed, tag), i); }

double gen_uniform(uint64_t seed, uint64_t tag, uint64_t i) {
  return uniform_from_key(stream_key(seed, tag), i);
}

float gen_normal(uint64_t seed, uint64_t tag, uint64_t i, float sd) {
  return normal_from_key(stream_key(seed, tag), i) * sd;
}

/* n consecutive elements starting at logical index i0; dtype 0 = fp32, 1 = bf16. */
void gen_fill_normal(uint64_t seed, uint64_t tag, uint64_t i0, int64_t n, float sd, int dtype,
                     void* dst) {
  const uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    float v = normal_from_key(key, i0 + (uint64_t)j) * sd;
    if (dtype == 0)
      ((float*)dst)[j] = v;
    else
      ((uint16_t*)dst)[j] = f32_to_bf16_rne(v);
  }
}

/* nseg segments of seg_len elements: segment s covers logical indices
 * [src_i0[s], src_i0[s] + seg_len) and lands at element offset dst_off[s] of dst. */
void gen_fill_normal_segments(uint64_t seed, uint64_t tag, int64_t nseg, const uint64_t* src_i0,
                              int64_t seg_len, float sd, int dtype, void* dst,
                              const int64_t* dst_off) {
  const uint64_t key = stream_key(seed, tag);
  const int64_t chunk = 16384;
  const int64_t per_seg = (seg_len + chunk - 1) / chunk;
  const int64_t total = nseg * per_seg;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t w = 0; w < total; ++w) {
    const int64_t s = w / per_seg, c0 = (w % per_seg) * chunk;
    const int64_t c1 = c0 + chunk < seg_len ? c0 + chunk : seg_len;
    for (int64_t j = c0; j < c1; ++j) {
      float v = normal_from_key(key, src_i0[s] + (uint64_t)j) * sd;
      if (dtype == 0)
        ((float*)dst)[dst_off[s] + j] = v;
      else
        ((uint16_t*)dst)[dst_off[s] + j] = f32_to_bf16_rne(v);
    }
  }
}

/* ---- MXFP4 weights (OCP Microscaling Formats (MX) specification v1.0) ----------------
 * A block of 32 consecutive elements of a row shares one E8M0 scale X = 2^e (stored as
 * e + 127); each element is an FP4 E2M1 code (sign bit 3, exponent bits 2:1 with bias 1,
 * mantissa bit 0), whose magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Conversion of a block
 * V (the MX spec's rule): e = floor(log2(max |V_i|)) - 2 (2 = the largest E2M1 exponent),
 * clamped to [-127, 127] (e = -127 for an all-zero block); each element is V_i / X rounded
 * to nearest on the E2M1 grid, ties to the even code (mantissa bit 0), magnitudes beyond
 * 6 saturating to 6.  V_i / X is exact (X is a power of two), so every decision is exact.
 * A block's 16 code bytes hold element 2j in the low nibble of byte j and element 2j+1 in
 * the high nibble.  This is input preparation (the weights are given in MXFP4); nothing of
 * the layer is computed. */
static inline uint8_t e2m1_code(float q) {  /* q = V_i / X, |q| < 8 */
  const float a = fabsf(q);
  uint8_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return (uint8_t)(c | (q < 0.0f ? 8 : 0));
}

/* floor(log2(a)) for a finite a > 0 (exact, from the bits). */
static inline int floor_log2f(float a) {
  uint32_t u;
  memcpy(&u, &a, 4);
  const int ex = (int)((u >> 23) & 0xFF);
  if (ex != 0) return ex - 127;
  int k = -127; /* subnormal: 2^-126 * (mantissa / 2^23) */
  uint32_t m = u & 0x7FFFFF;
  while (m < 0x400000u) { m <<= 1; --k; }
  return k;
}

/* Quantise one block of 32 values: 16 code bytes and one scale byte. */
void gen_mxfp4_block(const float* v, uint8_t* codes, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = fabsf(v[i]) > amax ? fabsf(v[i]) : amax;
  int e = amax > 0.0f ? floor_log2f(amax) - 2 : -127;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  *scale = (uint8_t)(e + 127);
  const float inv = ldexpf(1.0f, -e);
  for (int j = 0; j < 16; ++j) {
    const uint8_t lo = e2m1_code(v[2 * j] * inv), hi = e2m1_code(v[2 * j + 1] * inv);
    codes[j] = (uint8_t)(lo | (hi << 4));
  }
}

/* nrows rows of K normals (row r = logical indices [row_i0[r], row_i0[r] + K), sd), each
 * quantised to MXFP4: codes of row r at codes + code_off[r] (K/2 bytes), scales at
 * scales + scale_off[r] (K/32 bytes).  K is a multiple of 32. */
void gen_fill_mxfp4_rows(uint64_t seed, uint64_t tag, int64_t nrows, const uint64_t* row_i0,
                         int64_t K, float sd, uint8_t* codes, const int64_t* code_off,
                         uint8_t* scales, const int64_t* scale_off) {
  const uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    float v[32];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = normal_from_key(key, row_i0[r] + (uint64_t)(b * 32 + i)) * sd;
      gen_mxfp4_block(v, codes + code_off[r] + b * 16, scales + scale_off[r] + b);
    }
  }
}

/* Byte offsets of block b (elements 32b .. 32b+31) of row r of an R x K MXFP4 matrix in the
 * library's tiled entry layout: tiles of 16 rows x 128 elements, row strips one after the
 * other and, inside a strip, tiles in k order (the last tile of a strip holds what is left
 * of K); inside a tile, the 16 code bytes of (row i, block q of the tile) sit at slot
 * 16 q + i, and its scale byte at the same slot of the strip's scale tile. */
static inline int64_t mx_code_off(int64_t r, int64_t b, int64_t K) {
  return (r / 16) * 8 * K + (b / 4) * 1024 + (16 * (b % 4) + r % 16) * 16;
}
static inline int64_t mx_scale_off(int64_t r, int64_t b, int64_t K) {
  return (r / 16) * (K / 2) + (b / 4) * 64 + 16 * (b % 4) + r % 16;
}

/* nmat matrices of R x K normals (matrix q: element (r, c) = logical index i0[q] + r K + c,
 * sd) quantised to MXFP4 into the tiled layout: codes at codes + code_base[q], scales at
 * scales + scale_base[q].  R is a multiple of 16 and K of 32. */
void gen_fill_mxfp4_tiled(uint64_t seed, uint64_t tag, int64_t nmat, const uint64_t* i0,
                          int64_t R, int64_t K, float sd, uint8_t* codes,
                          const int64_t* code_base, uint8_t* scales, const int64_t* scale_base) {
  const uint64_t key = stream_key(seed, tag);
#pragma omp parallel for schedule(static)
  for (int64_t qr = 0; qr < nmat * R; ++qr) {
    const int64_t q = qr / R, r = qr % R;
    float v[32];
    uint8_t blk[16];
    for (int64_t b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i)
        v[i] = normal_from_key(key, i0[q] + (uint64_t)(r * K + b * 32 + i)) * sd;
      gen_mxfp4_block(v, blk, scales + scale_base[q] + mx_scale_off(r, b, K));
      memcpy(codes + code_base[q] + mx_code_off(r, b, K), blk, 16);
    }
  }
}

typedef struct {
  uint64_t key;
  int32_t e;
} rank_item;

static int rank_cmp(const void* a, const void* b) {
  const rank_item* x = (const rank_item*)a;
  const rank_item* y = (const rank_item*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->e - y->e;
}

/* A seeded permutation of popularity ranks: rank[e] in 1..E. */
void gen_rank_perm(uint64_t seed, uint64_t tag, int E, int32_t* rank) {
  const uint64_t key = stream_key(seed, tag);
  rank_item* it = (rank_item*)malloc(sizeof(rank_item) * (size_t)E);
  for (int e = 0; e < E; ++e) {
    it[e].key = draw(key, (uint64_t)e);
    it[e].e = e;
  }
  qsort(it, (size_t)E, sizeof(rank_item), rank_cmp);
  for (int r = 0; r < E; ++r) rank[it[r].e] = r + 1;
  free(it);
}

/* Per-expert popularity bias b_e = -alpha * s * ln(rank_e) (a log-Zipf(s) tilt of
 * the router logits; alpha scales how strongly it is applied). */
void gen_zipf_bias(uint64_t seed, uint64_t tag, int E, double alpha, double s, float* bias) {
  int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  gen_rank_perm(seed, tag, E, rank);
  for (int e = 0; e < E; ++e) bias[e] = (float)(-alpha * s * log((double)rank[e]));
  free(rank);
}

static int desc_cmp(const void* a, const void* b) {
  const float x = *(const float*)a, y = *(const float*)b;
  return x > y ? -1 : (x < y ? 1 : 0);
}

/* Router logits: row t is z + bias (fp32), z ~ N(0,1) drawn at logical index
 * (a*T + t)*E + e for attempt a.  A row whose k-th and (k+1)-th largest values
 * differ by less than min_gap is redrawn with the next attempt, so the top-k
 * set is well defined.  Returns the number of redraws, or -1 if some row still
 * violates the gap after max_attempts. */
int64_t gen_routing_logits(uint64_t seed, uint64_t tag, int T, int E, int k, const float* bias,
                           double min_gap, int max_attempts, float* out) {
  const uint64_t key = stream_key(seed, tag);
  int64_t redraws = 0;
  int failed = 0;
#pragma omp parallel reduction(+ : redraws) reduction(| : failed)
  {
    float* tmp = (float*)malloc(sizeof(float) * (size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      float* row = out + (size_t)t * E;
      int ok = 0;
      for (int a = 0; a < max_attempts && !ok; ++a) {
        for (int e = 0; e < E; ++e) {
          uint64_t i = ((uint64_t)a * (uint64_t)T + (uint64_t)t) * (uint64_t)E + (uint64_t)e;
          row[e] = normal_from_key(key, i) + (bias ? bias[e] : 0.0f);
        }
        if (k >= E) {
          ok = 1;
        } else {
          memcpy(tmp, row, sizeof(float) * (size_t)E);
          qsort(tmp, (size_t)E, sizeof(float), desc_cmp);
          ok = ((double)tmp[k - 1] - (double)tmp[k]) >= min_gap;
        }
        if (!ok) redraws += 1;
      }
      if (!ok) failed |= 1;
    }
    free(tmp);
  }
  return failed ? -1 : redraws;
}

/* Multi-step decode routing trace with per-layer temporal locality.
 * For step s, layer l, token b, slot j: with probability p_stay (s > 0) the
 * token keeps the expert it had in slot j at step s-1 unless it already chose
 * it this step; otherwise it draws from a categorical Zipf(zipf_s) over a
 * per-layer popularity ranking, redrawing duplicates.  ids: [steps][L][B][k].
 * logits: [steps][L][B][E]; slot j's expert gets 10 - j + 0.5u, every other
 * expert gets N(0,1) clipped to [-4, 4], so descending-logit order reproduces
 * the slot order with a gap of at least 0.5. */
void gen_markov_routing(uint64_t seed, int steps, int L, int B, int E, int k, double p_stay,
                        double zipf_s, uint64_t tag_rank, uint64_t tag_stay, uint64_t tag_zipf,
                        uint64_t tag_chosen, uint64_t tag_noise, int32_t* ids, float* logits) {
  const uint64_t kstay = stream_key(seed, tag_stay);
  const uint64_t kzipf = stream_key(seed, tag_zipf);
  const uint64_t kch = stream_key(seed, tag_chosen);
  const uint64_t knoise = stream_key(seed, tag_noise);
  double* cdf = (double*)malloc(sizeof(double) * (size_t)E);
  int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  int32_t* by_rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)E * (size_t)L);
  double z = 0.0;
  for (int r = 0; r < E; ++r) {
    z += pow((double)(r + 1), -zipf_s);
    cdf[r] = z;
  }
  for (int r = 0; r < E; ++r) cdf[r] /= z;
  for (int l = 0; l < L; ++l) {
    gen_rank_perm(seed, tag_rank + (uint64_t)l * 0x10000ULL, E, rank);
    for (int e = 0; e < E; ++e) by_rank[(size_t)l * E + (rank[e] - 1)] = e;
  }
  for (int s = 0; s < steps; ++s) {
    for (int l = 0; l < L; ++l) {
      for (int b = 0; b < B; ++b) {
        const uint64_t row = ((uint64_t)s * L + l) * B + b;
        int32_t* cur = ids + row * (uint64_t)k;
        const int32_t* prev = s > 0 ? ids + (((uint64_t)(s - 1) * L + l) * B + b) * (uint64_t)k : 0;
        for (int j = 0; j < k; ++j) {
          int chosen = -1;
          if (prev && uniform_from_key(kstay, row * k + j) < p_stay) {
            int dup = 0;
            for (int q = 0; q < j; ++q) dup |= cur[q] == prev[j];
            if (!dup) chosen = prev[j];
          }
          for (int a = 0; chosen < 0 && a < 64; ++a) {
            double u = uniform_from_key(kzipf, (row * k + j) * 64 + a);
            int lo = 0, hi = E - 1;
            while (lo < hi) {
              int mid = (lo + hi) / 2;
              if (cdf[mid] > u) hi = mid; else lo = mid + 1;
            }
            int e = by_rank[(size_t)l * E + lo];
            int dup = 0;
            for (int q = 0; q < j; ++q) dup |= cur[q] == e;
            if (!dup) chosen = e;
          }
          for (int r = 0; chosen < 0 && r < E; ++r) { /* fallback: most popular unchosen */
            int e = by_rank[(size_t)l * E + r];
            int dup = 0;
            for (int q = 0; q < j; ++q) dup |= cur[q] == e;
            if (!dup) chosen = e;
          }
          cur[j] = chosen;
        }
        float* lg = logits + row * (uint64_t)E;
        for (int e = 0; e < E; ++e) {
          float v = normal_from_key(knoise, row * E + e);
          lg[e] = v < -4.0f ? -4.0f : (v > 4.0f ? 4.0f : v);
        }
        for (int j = 0; j < k; ++j)
          lg[cur[j]] = (float)(10.0 - j + 0.5 * uniform_from_key(kch, row * E + cur[j]));
      }
    }
  }
  free(cdf);
  free(rank);
  free(by_rank);
}

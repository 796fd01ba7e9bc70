/*
 * tq_oracle.c -- plain, slow CPU oracle for compressed-domain KV decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or load
 * this file; only tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Everything is double precision, scalar loops, no blocking and no fusion.
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fPIC -shared (no fast-math), so
 * that every floating-point operation is the IEEE operation written here.
 *
 * What it computes (sources are the five pages on TurboQuant KV compression):
 *  - sign vector: a Rademacher (+/-1) diagonal drawn from a seed ("HadamardPreconditioner",
 *    VeloxQuant "How I built" post, Stage 1). The pages name no generator; the
 *    reading taken here is SplitMix64 (Steele, Lea and Flood, OOPSLA 2014), top bit
 *    of each output selects the sign.
 *  - rotation: sign flip first, then the Walsh-Hadamard transform (same post,
 *    Stage 1 code). H is the Sylvester matrix, H[i][j] = (-1)^popcount(i & j),
 *    applied here as the dense matrix it is.
 *  - norm: the L2 norm of the vector, kept beside the codes (Stage 2 of that post;
 *    the PR's storage ratios imply a 4-byte norm).
 *  - scalar quantisation: coordinates of the rotated vector divided by the norm
 *    are N(0,1)-scaled; the index is the number of Lloyd-Max boundaries the value
 *    exceeds (VeloxQuant "optimization journey", boundary-sum step).
 *  - packing: b-bit indices written LSB-first into a byte stream, an index may
 *    straddle bytes (the "BitPackBuffer" section of the same post).
 *  - decode attention: the compressed cache is dequantised and ordinary softmax
 *    attention is taken over it (turboquant-mlx KV-cache guide: the fused kernel's
 *    output equals the expand-then-attend path).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD (-1)
#define ORC_NOMEM (-2)

/* ---------------------------------------------------------------- helpers */

static int popcount_u32(uint32_t v) {
  int c = 0;
  while (v) {
    c += (int)(v & 1u);
    v >>= 1;
  }
  return c;
}

/* Sylvester-Hadamard entry (-1)^popcount(i & j). */
static double hadamard_entry(int i, int j) {
  return (popcount_u32((uint32_t)(i & j)) & 1) ? -1.0 : 1.0;
}

static int is_pow2(int d) { return d > 0 && (d & (d - 1)) == 0; }

/* Dense d x d Hadamard matrix, row-major. */
static double* hadamard_matrix(int d) {
  double* h = (double*)malloc(sizeof(double) * (size_t)d * (size_t)d);
  if (!h) return NULL;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) h[(size_t)i * d + j] = hadamard_entry(i, j);
  return h;
}

/* y = H x, plain matrix-vector product in index order. */
static void hadamard_apply(const double* h, int d, const double* x, double* y) {
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += h[(size_t)i * d + j] * x[j];
    y[i] = acc;
  }
}

/* Sum of d = 2^k values over the canonical pairwise tree: each level adds
 * neighbouring pairs in index order. */
static double pairwise_tree_sum(const double* v, int d, double* scratch) {
  memcpy(scratch, v, sizeof(double) * (size_t)d);
  for (int w = d; w > 1; w >>= 1)
    for (int i = 0; i < w / 2; ++i) scratch[i] = scratch[2 * i] + scratch[2 * i + 1];
  return scratch[0];
}

/* Exposed for tests: the dense Hadamard matrix the oracle applies. */
int orc_hadamard(int d, double* out) {
  if (!is_pow2(d) || !out) return ORC_BAD;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) out[(size_t)i * d + j] = hadamard_entry(i, j);
  return ORC_OK;
}

/* ---------------------------------------------------------------- signs */

/* Raw SplitMix64 outputs (exposed so the generator can be pinned to its
 * published test vector). */
void orc_splitmix64(uint64_t seed, int n, uint64_t* out) {
  uint64_t state = seed;
  for (int i = 0; i < n; ++i) {
    state += 0x9E3779B97F4A7C15ULL;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    z ^= z >> 31;
    out[i] = z;
  }
}

/* Sign j is -1 when the top bit of the j-th SplitMix64 output is set. */
int orc_signs(uint64_t seed, int d, int8_t* out) {
  if (d <= 0 || !out) return ORC_BAD;
  uint64_t* raw = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)d);
  if (!raw) return ORC_NOMEM;
  orc_splitmix64(seed, d, raw);
  for (int j = 0; j < d; ++j) out[j] = (raw[j] >> 63) ? (int8_t)-1 : (int8_t)1;
  free(raw);
  return ORC_OK;
}

/* ---------------------------------------------------------------- packing */

/* Index i occupies stream bits [bits*i, bits*i + bits), bit k of the index at
 * stream bit p = bits*i + k, i.e. byte p/8, bit p%8. */
void orc_pack(int d, int bits, const int32_t* idx, uint8_t* row) {
  int nbytes = d * bits / 8;
  memset(row, 0, (size_t)nbytes);
  for (int i = 0; i < d; ++i)
    for (int k = 0; k < bits; ++k) {
      int p = bits * i + k;
      if ((idx[i] >> k) & 1) row[p / 8] |= (uint8_t)(1u << (p % 8));
    }
}

void orc_unpack(int d, int bits, const uint8_t* row, int32_t* idx) {
  for (int i = 0; i < d; ++i) {
    int32_t v = 0;
    for (int k = 0; k < bits; ++k) {
      int p = bits * i + k;
      v |= (int32_t)((row[p / 8] >> (p % 8)) & 1u) << k;
    }
    idx[i] = v;
  }
}

/* ---------------------------------------------------------------- encode */

/* Number of boundaries the value exceeds: #{k : beta_k < z}. A value equal to
 * a boundary does not exceed it and goes to the lower cell. */
static int32_t bucketize(double z, const float* boundaries, int nb) {
  int32_t c = 0;
  for (int k = 0; k < nb; ++k)
    if ((double)boundaries[k] < z) ++c;
  return c;
}

/* Exposed for tests: bucketize n values against nb fp32 boundaries. */
void orc_bucketize(const double* z, int64_t n, const float* boundaries, int nb, int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bucketize(z[i], boundaries, nb);
}

/*
 * Encode n vectors of d values (given as doubles that are exactly the fp16
 * inputs). Vector v is read from x + v*x_stride, its packed row goes to
 * codes + v*row_bytes and its norm to norms[v] (fp32, round to nearest).
 * z_out (optional, n*d doubles) receives the scaled rotated coordinates.
 */
int orc_encode(int d, int bits, const int8_t* signs, const float* boundaries,
               const double* x, int64_t n, int64_t x_stride, uint8_t* codes,
               float* norms, double* norms64, double* z_out) {
  if (!is_pow2(d) || bits < 1 || bits > 8 || (d * bits) % 8) return ORC_BAD;
  int nb = (1 << bits) - 1;
  int row_bytes = d * bits / 8;
  double* h = hadamard_matrix(d);
  double* u = (double*)malloc(sizeof(double) * (size_t)d);
  double* w = (double*)malloc(sizeof(double) * (size_t)d);
  double* sq = (double*)malloc(sizeof(double) * (size_t)d);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
  if (!h || !u || !w || !sq || !tmp || !idx) {
    free(h); free(u); free(w); free(sq); free(tmp); free(idx);
    return ORC_NOMEM;
  }
  for (int64_t v = 0; v < n; ++v) {
    const double* xv = x + v * x_stride;
    for (int j = 0; j < d; ++j) {
      u[j] = (double)signs[j] * xv[j];
      sq[j] = xv[j] * xv[j];
    }
    double nrm = sqrt(pairwise_tree_sum(sq, d, tmp));
    hadamard_apply(h, d, u, w);
    for (int i = 0; i < d; ++i) {
      double z = (nrm == 0.0) ? 0.0 : w[i] / nrm;
      if (z_out) z_out[v * d + i] = z;
      idx[i] = bucketize(z, boundaries, nb);
    }
    orc_pack(d, bits, idx, codes + v * row_bytes);
    norms[v] = (float)nrm;
    if (norms64) norms64[v] = nrm;
  }
  free(h); free(u); free(w); free(sq); free(tmp); free(idx);
  return ORC_OK;
}

/* ---------------------------------------------------------------- dequant */

/* x_hat = (norm / d) * sigma (.) (H c[idx]) for n packed rows. */
int orc_dequant(int d, int bits, const int8_t* signs, const float* centroids,
                const uint8_t* codes, const float* norms, int64_t n, double* out) {
  if (!is_pow2(d) || bits < 1 || bits > 8 || (d * bits) % 8) return ORC_BAD;
  int row_bytes = d * bits / 8;
  double* h = hadamard_matrix(d);
  double* c = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
  if (!h || !c || !y || !idx) {
    free(h); free(c); free(y); free(idx);
    return ORC_NOMEM;
  }
  for (int64_t v = 0; v < n; ++v) {
    orc_unpack(d, bits, codes + v * row_bytes, idx);
    for (int i = 0; i < d; ++i) c[i] = (double)centroids[idx[i]];
    hadamard_apply(h, d, c, y);
    double s = (double)norms[v] / (double)d;
    for (int j = 0; j < d; ++j) out[v * d + j] = s * (double)signs[j] * y[j];
  }
  free(h); free(c); free(y); free(idx);
  return ORC_OK;
}

/* ---------------------------------------------------------------- attention */

/*
 * Decode attention over the compressed cache, by its plain definition:
 * dequantise every cached K and V row of the sequence, then
 *   s_t = scale * <q, k_hat_t>,  p = softmax(s),  out = sum_t p_t v_hat_t.
 *
 * Cache layout: codes [B][Hkv][max_ctx][row_bytes], norms [B][Hkv][max_ctx].
 * q: [B][Hq][d] doubles. Query head h reads KV head h / (Hq/Hkv).
 * bh: n_bh pairs (b, h) to compute (NULL: every pair in b-major order);
 * out: n_bh x d doubles. A sequence of length 0 yields a zero row.
 */
int orc_attend(int d, int k_bits, int v_bits,
               const int8_t* k_signs, const float* k_centroids,
               const int8_t* v_signs, const float* v_centroids,
               const double* q, int batch, int n_q_heads, int n_kv_heads,
               const uint8_t* k_codes, const float* k_norms,
               const uint8_t* v_codes, const float* v_norms,
               int max_ctx, const int32_t* lengths, double scale,
               const int32_t* bh, int n_bh, double* out) {
  if (n_kv_heads <= 0 || n_q_heads % n_kv_heads) return ORC_BAD;
  int group = n_q_heads / n_kv_heads;
  int kr = d * k_bits / 8, vr = d * v_bits / 8;
  int total = bh ? n_bh : batch * n_q_heads;
  double* kh = (double*)malloc(sizeof(double) * (size_t)max_ctx * d + 8);
  double* vh = (double*)malloc(sizeof(double) * (size_t)max_ctx * d + 8);
  double* s = (double*)malloc(sizeof(double) * (size_t)max_ctx + 8);
  if (!kh || !vh || !s) {
    free(kh); free(vh); free(s);
    return ORC_NOMEM;
  }
  int cur_b = -1, cur_g = -1;
  for (int e = 0; e < total; ++e) {
    int b = bh ? bh[2 * e] : e / n_q_heads;
    int h = bh ? bh[2 * e + 1] : e % n_q_heads;
    if (b < 0 || b >= batch || h < 0 || h >= n_q_heads) {
      free(kh); free(vh); free(s);
      return ORC_BAD;
    }
    int g = h / group;
    int len = lengths[b];
    double* o = out + (size_t)e * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    if (len <= 0) continue;
    if (b != cur_b || g != cur_g) {
      size_t base = ((size_t)b * n_kv_heads + g) * (size_t)max_ctx;
      int rc = orc_dequant(d, k_bits, k_signs, k_centroids, k_codes + base * kr,
                           k_norms + base, len, kh);
      if (rc == ORC_OK)
        rc = orc_dequant(d, v_bits, v_signs, v_centroids, v_codes + base * vr,
                         v_norms + base, len, vh);
      if (rc != ORC_OK) {
        free(kh); free(vh); free(s);
        return rc;
      }
      cur_b = b;
      cur_g = g;
    }
    const double* qv = q + ((size_t)b * n_q_heads + h) * d;
    double m = -INFINITY;
    for (int t = 0; t < len; ++t) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += qv[j] * kh[(size_t)t * d + j];
      s[t] = scale * acc;
      if (s[t] > m) m = s[t];
    }
    double z = 0.0;
    for (int t = 0; t < len; ++t) {
      s[t] = exp(s[t] - m);
      z += s[t];
    }
    for (int t = 0; t < len; ++t) {
      double p = s[t] / z;
      for (int j = 0; j < d; ++j) o[j] += p * vh[(size_t)t * d + j];
    }
  }
  free(kh); free(vh); free(s);
  return ORC_OK;
}

/*
 * The same attention taken in the rotated basis, without expanding the cache:
 *   q_tilde = H (sigma_K (.) q)
 *   s_t     = scale * (nK_t / d) * sum_j q_tilde_j cK[idxK_tj]
 *   a_j     = sum_t p_t nV_t cV[idxV_tj]
 *   out     = (1/d) sigma_V (.) H a
 * Used only to show that reading K in its rotated basis gives the result of
 * the plain definition above; same argument conventions as orc_attend.
 */
int orc_attend_rotated(int d, int k_bits, int v_bits,
                       const int8_t* k_signs, const float* k_centroids,
                       const int8_t* v_signs, const float* v_centroids,
                       const double* q, int batch, int n_q_heads, int n_kv_heads,
                       const uint8_t* k_codes, const float* k_norms,
                       const uint8_t* v_codes, const float* v_norms,
                       int max_ctx, const int32_t* lengths, double scale,
                       const int32_t* bh, int n_bh, double* out) {
  if (n_kv_heads <= 0 || n_q_heads % n_kv_heads || !is_pow2(d)) return ORC_BAD;
  int group = n_q_heads / n_kv_heads;
  int kr = d * k_bits / 8, vr = d * v_bits / 8;
  int total = bh ? n_bh : batch * n_q_heads;
  double* h = hadamard_matrix(d);
  double* u = (double*)malloc(sizeof(double) * (size_t)d);
  double* qt = (double*)malloc(sizeof(double) * (size_t)d);
  double* a = (double*)malloc(sizeof(double) * (size_t)d);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
  double* s = (double*)malloc(sizeof(double) * (size_t)max_ctx + 8);
  if (!h || !u || !qt || !a || !y || !idx || !s) {
    free(h); free(u); free(qt); free(a); free(y); free(idx); free(s);
    return ORC_NOMEM;
  }
  for (int e = 0; e < total; ++e) {
    int b = bh ? bh[2 * e] : e / n_q_heads;
    int hq = bh ? bh[2 * e + 1] : e % n_q_heads;
    int g = hq / group;
    int len = lengths[b];
    double* o = out + (size_t)e * d;
    for (int j = 0; j < d; ++j) o[j] = 0.0;
    if (len <= 0) continue;
    size_t base = ((size_t)b * n_kv_heads + g) * (size_t)max_ctx;
    const double* qv = q + ((size_t)b * n_q_heads + hq) * d;
    for (int j = 0; j < d; ++j) u[j] = (double)k_signs[j] * qv[j];
    hadamard_apply(h, d, u, qt);
    double m = -INFINITY;
    for (int t = 0; t < len; ++t) {
      orc_unpack(d, k_bits, k_codes + (base + t) * kr, idx);
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += qt[j] * (double)k_centroids[idx[j]];
      s[t] = scale * ((double)k_norms[base + t] / d) * acc;
      if (s[t] > m) m = s[t];
    }
    double z = 0.0;
    for (int t = 0; t < len; ++t) {
      s[t] = exp(s[t] - m);
      z += s[t];
    }
    for (int j = 0; j < d; ++j) a[j] = 0.0;
    for (int t = 0; t < len; ++t) {
      orc_unpack(d, v_bits, v_codes + (base + t) * vr, idx);
      double wgt = s[t] / z * (double)v_norms[base + t];
      for (int j = 0; j < d; ++j) a[j] += wgt * (double)v_centroids[idx[j]];
    }
    hadamard_apply(h, d, a, y);
    for (int j = 0; j < d; ++j) o[j] = (double)v_signs[j] * y[j] / d;
  }
  free(h); free(u); free(qt); free(a); free(y); free(idx); free(s);
  return ORC_OK;
}

/* ---------------------------------------------------------------- dense rotation
 * Head dims that are not a power of two have no Walsh-Hadamard transform; the
 * pages' fallback is a dense rotation (PR #232, Known limitations: dense
 * rotation otherwise; VeloxQuant "How I built", Stage 1: the original method
 * draws the rotation as the Q factor of a Gaussian matrix). Here the rotation
 * is an input: m is d x d, row-major, equal to sqrt(d) times an orthogonal
 * matrix, so that z = m x / |x| is N(0,1)-scaled like H(sigma x) / |x|, and
 * m = H diag(sigma) reproduces the Walsh-Hadamard codec exactly.
 */

/* Pairwise tree for any count: each level adds neighbouring pairs in index
 * order and carries an odd last element up unchanged (for d = 2^k this is the
 * canonical tree above). */
static double pairwise_tree_sum_any(const double* v, int d, double* scratch) {
  memcpy(scratch, v, sizeof(double) * (size_t)d);
  for (int w = d; w > 1; w = (w + 1) / 2) {
    for (int i = 0; i < w / 2; ++i) scratch[i] = scratch[2 * i] + scratch[2 * i + 1];
    if (w & 1) scratch[w / 2] = scratch[w - 1];
  }
  return scratch[0];
}

/* y = m x: products and sums in index order, no fused multiply-add. */
static void matvec(const double* m, int d, const double* x, double* y) {
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += m[(size_t)i * d + j] * x[j];
    y[i] = acc;
  }
}

/* Exposed for tests: the any-count pairwise tree. */
double orc_tree_sum(const double* v, int d) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(d > 0 ? d : 1));
  if (!s) return NAN;
  double r = d > 0 ? pairwise_tree_sum_any(v, d, s) : 0.0;
  free(s);
  return r;
}

int orc_encode_dense(int d, int bits, const double* m, const float* boundaries,
                     const double* x, int64_t n, int64_t x_stride, uint8_t* codes,
                     float* norms, double* norms64, double* z_out) {
  if (d < 1 || bits < 1 || bits > 8 || (d * bits) % 8) return ORC_BAD;
  int nb = (1 << bits) - 1;
  int row_bytes = d * bits / 8;
  double* w = (double*)malloc(sizeof(double) * (size_t)d);
  double* sq = (double*)malloc(sizeof(double) * (size_t)d);
  double* tmp = (double*)malloc(sizeof(double) * (size_t)d);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
  if (!w || !sq || !tmp || !idx) {
    free(w); free(sq); free(tmp); free(idx);
    return ORC_NOMEM;
  }
  for (int64_t v = 0; v < n; ++v) {
    const double* xv = x + v * x_stride;
    for (int j = 0; j < d; ++j) sq[j] = xv[j] * xv[j];
    double nrm = sqrt(pairwise_tree_sum_any(sq, d, tmp));
    matvec(m, d, xv, w);
    for (int i = 0; i < d; ++i) {
      double z = (nrm == 0.0) ? 0.0 : w[i] / nrm;
      if (z_out) z_out[v * d + i] = z;
      idx[i] = bucketize(z, boundaries, nb);
    }
    orc_pack(d, bits, idx, codes + v * row_bytes);
    norms[v] = (float)nrm;
    if (norms64) norms64[v] = nrm;
  }
  free(w); free(sq); free(tmp); free(idx);
  return ORC_OK;
}

/* x_hat = (norm / d) m^T c[idx]: the inverse of z = m x / |x| when m / sqrt(d)
 * is orthogonal. */
int orc_dequant_dense(int d, int bits, const double* m, const float* centroids,
                      const uint8_t* codes, const float* norms, int64_t n, double* out) {
  if (d < 1 || bits < 1 || bits > 8 || (d * bits) % 8) return ORC_BAD;
  int row_bytes = d * bits / 8;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)d);
  if (!idx) return ORC_NOMEM;
  for (int64_t v = 0; v < n; ++v) {
    orc_unpack(d, bits, codes + v * row_bytes, idx);
    double s = (double)norms[v] / (double)d;
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += m[(size_t)i * d + j] * (double)centroids[idx[i]];
      out[v * d + j] = s * acc;
    }
  }
  free(idx);
  return ORC_OK;
}

// codec.cpp -- host-side codec construction: sign vector and Lloyd-Max tables.
//
// Built with g++ (quad precision via libquadmath); no HIP code here.
//
// Sign vector: a seeded Rademacher diagonal for the randomized Walsh-Hadamard
// rotation (VeloxQuant "How I built" post, Stage 1: Random Rotation). The pages
// do not name a generator; sign j is -1 iff the top bit of the j-th SplitMix64
// output is set (Steele, Lea, Flood, OOPSLA 2014).
//
// Codebook: the Lloyd-Max quantizer of N(0,1) with 2^bits levels (same post,
// Stage 2 and "The Core Idea"): boundaries are midpoints of neighbouring
// centroids and every centroid is the conditional mean of its cell. The
// fixed point is reached with a few plain Lloyd sweeps followed by Newton's
// method on F(c) = T(c) - c, where T is "midpoints, then conditional means".
// Cell (a, b) has mass Q(a) - Q(b) and first moment phi(a) - phi(b), so the
// Jacobian of T is tridiagonal with closed-form entries:
//   dT_i/db = phi(b) (b - T_i) / mass_i,   dT_i/da = phi(a) (T_i - a) / mass_i.
// At 256 levels the system is ill-conditioned (smallest singular value ~3e-5),
// so it is solved in __float128: tables rounded once to fp32 are then exact
// roundings of the true fixed point.
#include <quadmath.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "codec.hpp"

namespace tq {

typedef __float128 qreal;

static qreal q_phi(qreal x) {
  static const qreal inv_sqrt_2pi = 1 / sqrtq(2 * acosq(-1));
  return expq(-x * x / 2) * inv_sqrt_2pi;
}

// Upper tail Q(x) = P(X > x) = erfc(x / sqrt 2) / 2.
static qreal q_tail(qreal x) {
  static const qreal sqrt2 = sqrtq(2);
  return erfcq(x / sqrt2) / 2;
}

// P(a < X < b) with a < b; infinities are flagged by the has_* booleans.
static qreal q_mass(bool has_a, qreal a, bool has_b, qreal b) {
  if (has_a && a >= 0) return q_tail(a) - (has_b ? q_tail(b) : 0);
  if (has_b && b <= 0) return q_tail(-b) - (has_a ? q_tail(-a) : 0);
  return 1 - (has_a ? q_tail(-a) : 0) - (has_b ? q_tail(b) : 0);
}

// Conditional means of all cells for centroids c; also the partial
// derivatives of each mean with respect to its lower and upper boundary.
static void lloyd_map(const std::vector<qreal>& c, std::vector<qreal>& t,
                      std::vector<qreal>& dlo, std::vector<qreal>& dhi) {
  const int n = (int)c.size();
  for (int i = 0; i < n; ++i) {
    const bool has_a = i > 0, has_b = i < n - 1;
    const qreal a = has_a ? (c[i - 1] + c[i]) / 2 : 0;
    const qreal b = has_b ? (c[i] + c[i + 1]) / 2 : 0;
    const qreal pa = has_a ? q_phi(a) : 0;
    const qreal pb = has_b ? q_phi(b) : 0;
    const qreal mass = q_mass(has_a, a, has_b, b);
    const qreal m = (pa - pb) / mass;
    t[i] = m;
    dlo[i] = has_a ? pa * (m - a) / mass : 0;
    dhi[i] = has_b ? pb * (b - m) / mass : 0;
  }
}

static bool lloyd_max_q(int n, std::vector<qreal>& c) {
  c.assign(n, 0);
  std::vector<qreal> t(n), dlo(n), dhi(n);
  // start: levels spread over +/- (1 + 0.9 sqrt(2 ln n))
  const qreal span = 1 + (qreal)0.9 * sqrtq(2 * logq((qreal)n));
  for (int i = 0; i < n; ++i)
    c[i] = (n == 1) ? 0 : span * (2 * (qreal)i / (n - 1) - 1);
  // plain Lloyd sweeps to enter Newton's basin
  for (int it = 0; it < 400; ++it) {
    lloyd_map(c, t, dlo, dhi);
    for (int i = 0; i < n; ++i) c[i] = (t[i] - t[n - 1 - i]) / 2;
  }
  // Newton on F(c) = T(c) - c with the tridiagonal Jacobian J = dT/dc - I
  std::vector<qreal> f(n), lo(n), di(n), up(n), x(n), cp(n), dp(n);
  for (int it = 0; it < 200; ++it) {
    lloyd_map(c, t, dlo, dhi);
    qreal res = 0;
    for (int i = 0; i < n; ++i) {
      f[i] = t[i] - c[i];
      if (fabsq(f[i]) > res) res = fabsq(f[i]);
    }
    if (res < (qreal)1e-28) return true;  // quad-precision evaluation noise is ~3e-32
    for (int i = 0; i < n; ++i) {
      lo[i] = dlo[i] / 2;                    // d T_i / d c_{i-1}
      up[i] = dhi[i] / 2;                    // d T_i / d c_{i+1}
      di[i] = (dlo[i] + dhi[i]) / 2 - 1;     // d T_i / d c_i - 1
    }
    // Thomas algorithm for J x = -f
    cp[0] = up[0] / di[0];
    dp[0] = -f[0] / di[0];
    for (int i = 1; i < n; ++i) {
      const qreal m = di[i] - lo[i] * cp[i - 1];
      cp[i] = (i < n - 1) ? up[i] / m : 0;
      dp[i] = (-f[i] - lo[i] * dp[i - 1]) / m;
    }
    x[n - 1] = dp[n - 1];
    for (int i = n - 2; i >= 0; --i) x[i] = dp[i] - cp[i] * x[i + 1];
    std::vector<qreal> nc(n);
    for (int i = 0; i < n; ++i) nc[i] = c[i] + x[i];
    for (int i = 0; i < n; ++i) c[i] = (nc[i] - nc[n - 1 - i]) / 2;
  }
  return false;
}

uint64_t splitmix64_next(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ULL;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

bool build_codec(int dim, int bits, uint64_t seed, CodecTables* out) {
  std::memset(out, 0, sizeof(*out));
  out->dim = dim;
  out->bits = bits;
  out->seed = seed;
  uint64_t state = seed;
  for (int j = 0; j < dim; ++j) {
    const uint64_t z = splitmix64_next(&state);
    if (z >> 63) out->sign_bits[j >> 5] |= 1u << (j & 31);
  }
  const int n = 1 << bits;
  std::vector<qreal> c;
  if (!lloyd_max_q(n, c)) return false;
  for (int i = 0; i < n; ++i) out->centroids[i] = (float)c[i];
  for (int i = 0; i + 1 < n; ++i) out->boundaries[i] = (float)((c[i] + c[i + 1]) / 2);
  return true;
}

bool build_prod_codec(int dim, int total_bits, uint64_t seed, CodecTables* out) {
  if (!build_codec(dim, total_bits - 1, seed, out)) return false;
  out->prod = true;
  uint64_t state = seed + 1;
  for (int j = 0; j < dim; ++j) {
    const uint64_t z = splitmix64_next(&state);
    if (z >> 63) out->sketch_sign_bits[j >> 5] |= 1u << (j & 31);
  }
  return true;
}

}  // namespace tq

// encode.hip -- TurboQuant-style encode of fp16 K/V vectors on gfx950.
//
// Per vector x (d fp16 values), following the mlx-swift-lm PR's fused encode
// (rotation, codebook search and packing in one dispatch) and the VeloxQuant
// "How I built" post (Stages 1-2, "The Bit-Packing Problem"):
//   N  = |x|_2                       (fp64; squares summed over the canonical
//                                      pairwise tree, then IEEE sqrt)
//   w  = H (sigma (.) x)              (fp64 Walsh-Hadamard butterfly; exact for
//                                      fp16 input, so any stage order is exact)
//   z  = w / N                        (IEEE fp64 division; z = 0 when N = 0)
//   idx_j = #{k : beta_k < z_j}       (boundary count, the pages' boundary-sum)
//   row = idx packed LSB-first, bit k of idx_j at stream bit bits*j + k
//
// Mapping: L lanes per vector, lane s owning the E = d/L consecutive
// coordinates E*s .. E*s+E-1; a wavefront holds 64/L vectors. Two layouts:
//   wide    L = 64 (E = d/64): the most lanes per vector, for the short
//           latency-bound launches of a cache append (a few hundred vectors);
//   narrow  L = d/8 (E = 8): the least cross-lane work per coordinate, for
//           bulk encodes (prefill), where throughput decides.
// The butterfly runs its in-lane stages first, then its cross-lane stages in
// ascending lane-mask order, i.e. all stages in ascending bit order. The
// norm's tree is the in-lane pairwise sum followed by an xor butterfly with
// ascending lane masks: the canonical tree, evaluated in every lane of the
// vector (fp addition is commutative, so the partner order does not matter).
// Cross-lane exchanges are VALU operations only: DPP inside a 16-lane row for
// lane masks 1, 2, 4, 8, and the gfx950 permlane swaps for masks 16 and 32.
//
// Boundary count: up to 15 boundaries (bits <= 4) are compared linearly from
// scalar registers. Above that the count is split in two levels: 15 coarse
// boundaries (every 2^(bits-4)-th, from scalar registers) select a cell, and
// the 2^(bits-4) - 1 boundaries inside the cell are read from LDS in one round
// and compared. Both give #{k : beta_k < z} exactly because beta is sorted.
//
// Packing: lane s's E codes form a CH = E*bits-bit chunk at stream bit CH*s.
// The G = 8/gcd(CH, 8) lanes of a byte-aligned group OR their chunks together
// (DPP tree), and the group's first lane stores the group's whole bytes.
//
// Several jobs (e.g. the K and V caches of one appended token batch) share a
// launch: blockIdx.y selects the job, and the bit width is a block-uniform
// run-time switch.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.hpp"
#include "xlane.hpp"

namespace tq {

namespace {

constexpr int kWavesPerBlock = 4;
// Below this many narrow-layout wavefronts (one per SIMD) the launch is
// latency-bound and the wide layout is used.
constexpr long long kNarrowMinWaves = 1024;
// Vector indices of the last workgroup stay below 2^31.
constexpr long long kMaxEncodeVectors = 0x7fffffffLL - 64;

template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
  const uint32_t lo = xor_lane<M>((uint32_t)v);
  const uint32_t hi = xor_lane<M>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

template <int M>
__device__ __forceinline__ double xor_lane_f64(double x) {
  return __builtin_bit_cast(double, xor_lane64<M>(__builtin_bit_cast(uint64_t, x)));
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// #{k : beta_k < z} over the job's 2^BITS - 1 sorted boundaries. Above 15
// boundaries: two levels (kTwoLevel: 30 compares, one LDS round) or a binary
// search over the LDS copy (BITS dependent LDS rounds, BITS compares).
template <int BITS, bool kTwoLevel>
__device__ __forceinline__ uint32_t count_below(double z, const EncodeJob& jb,
                                                const float* s_bnd) {
  if constexpr (BITS <= 4) {
    uint32_t idx = 0;
#pragma unroll
    for (int k = 0; k < (1 << BITS) - 1; ++k) idx += ((double)jb.boundaries[k] < z) ? 1u : 0u;
    return idx;
  } else if constexpr (kTwoLevel) {
    constexpr int S = 1 << (BITS - 4);  // boundaries per coarse cell, the last one coarse
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 15; ++k) c += ((double)jb.boundaries[k * S + S - 1] < z) ? 1u : 0u;
    const float* cell = s_bnd + c * S;
    uint32_t f = 0;
#pragma unroll
    for (int i = 0; i < S - 1; ++i) f += ((double)cell[i] < z) ? 1u : 0u;
    return c * S + f;
  } else {
    uint32_t idx = 0;  // invariant: the first idx boundaries are below z
#pragma unroll
    for (int step = 1 << (BITS - 1); step > 0; step >>= 1)
      if ((double)s_bnd[idx + step - 1] < z) idx += step;
    return idx;
  }
}

// OR this lane's CH-bit chunk (stream bits CH*sub ..) into its byte-aligned
// group of G = 8/gcd(CH, 8) lanes with a DPP tree; the group's first lane
// stores the group's whole bytes at row + (sub / G) * NBY.
template <int CH>
__device__ __forceinline__ void pack_store(uint64_t chunk, int sub, uint8_t* row) {
  constexpr int G = CH % 8 == 0 ? 1 : 8 / gcd_c(CH, 8);  // lanes per byte-aligned group
  constexpr int NBY = G * CH / 8;                       // bytes a group stores
  static_assert(G * CH <= 64, "group chunk fits 64 bits");
  // after the stage with mask m, every lane whose index is a multiple of 2m
  // holds the chunks of its 2m lanes
  if constexpr (G >= 2) chunk |= xor_lane64<1>(chunk) << CH;
  if constexpr (G >= 4) chunk |= xor_lane64<2>(chunk) << (2 * CH);
  if constexpr (G >= 8) chunk |= xor_lane64<4>(chunk) << (4 * CH);
  if (sub % G == 0) {
    uint8_t* dst = row + (sub / G) * NBY;
    if constexpr (NBY % 4 == 0) {
#pragma unroll
      for (int i = 0; i < NBY / 4; ++i) ((uint32_t*)dst)[i] = (uint32_t)(chunk >> (32 * i));
    } else if constexpr (NBY % 2 == 0) {
#pragma unroll
      for (int i = 0; i < NBY / 2; ++i) ((uint16_t*)dst)[i] = (uint16_t)(chunk >> (16 * i));
    } else {
#pragma unroll
      for (int i = 0; i < NBY; ++i) dst[i] = (uint8_t)(chunk >> (8 * i));
    }
  }
}

// Sum over the canonical pairwise tree of the vector's squares: in-lane levels,
// then an xor butterfly with ascending lane masks (every lane gets the sum).
template <int E, int L>
__device__ __forceinline__ double tree_sum_sq(const double (&x)[E]) {
  double sq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sq[e] = x[e] * x[e];
#pragma unroll
  for (int w = 1; w < E; w <<= 1)
#pragma unroll
    for (int i = 0; i < E; i += 2 * w) sq[i] = sq[i] + sq[i + w];
  double s = sq[0];
  if constexpr (L > 1) s = s + xor_lane_f64<1>(s);
  if constexpr (L > 2) s = s + xor_lane_f64<2>(s);
  if constexpr (L > 4) s = s + xor_lane_f64<4>(s);
  if constexpr (L > 8) s = s + xor_lane_f64<8>(s);
  if constexpr (L > 16) s = s + xor_lane_f64<16>(s);
  if constexpr (L > 32) s = s + xor_lane_f64<32>(s);
  return s;
}

// Walsh-Hadamard butterfly over the vector: in-lane stages, then cross-lane
// stages, all in ascending order of the pair distance.
template <int E, int L>
__device__ __forceinline__ void wht_vector(double (&u)[E], int sub) {
#pragma unroll
  for (int hs = 1; hs < E; hs <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & hs) == 0) {
        const double p = u[e], q = u[e + hs];
        u[e] = p + q;
        u[e + hs] = p - q;
      }
  // partner p, own value u: the lower lane keeps u + p, the upper p - u. Both
  // are fma(u, s, p) with s = +-1: the product is exact, so the one rounding
  // is that of the sum or difference (the same bits, signed zeros included).
  auto cross = [&](auto mtag) __attribute__((always_inline)) {
    constexpr int m = decltype(mtag)::value;
    const double s = (sub & m) != 0 ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double pv = xor_lane_f64<m>(u[e]);
      u[e] = __builtin_fma(u[e], s, pv);
    }
  };
  if constexpr (L > 1) cross(std::integral_constant<int, 1>{});
  if constexpr (L > 2) cross(std::integral_constant<int, 2>{});
  if constexpr (L > 4) cross(std::integral_constant<int, 4>{});
  if constexpr (L > 8) cross(std::integral_constant<int, 8>{});
  if constexpr (L > 16) cross(std::integral_constant<int, 16>{});
  if constexpr (L > 32) cross(std::integral_constant<int, 32>{});
}

// Quantise this lane's E coordinates and store its share of the packed row.
// For a TurboQuant-Prod job also the residual rho = z - c[idx]: its norm
// (canonical tree) and the signs of H (sigma_S (.) rho), one bit per
// coordinate, set for a negative value.
template <int E, int L, int BITS>
__device__ __forceinline__ void quantize_store(const double (&u)[E], double nrm, int sub,
                                               const EncodeJob& jb, const float* s_bnd,
                                               const float* s_cen, uint32_t ssgn, uint8_t* row,
                                               uint8_t* sketch_row, float* rnorm) {
  double z[E];
  uint32_t idx[E];
  uint64_t chunk = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    z[e] = (nrm == 0.0) ? 0.0 : u[e] / nrm;
    idx[e] = count_below<BITS, (E <= 4)>(z[e], jb, s_bnd);
    chunk |= (uint64_t)idx[e] << (BITS * e);
  }
  if constexpr (BITS <= 7) {
    if (jb.prod) {  // block-uniform
      double rho[E];
#pragma unroll
      for (int e = 0; e < E; ++e) rho[e] = z[e] - (double)s_cen[idx[e]];
      const double gam = __builtin_sqrt(tree_sum_sq<E, L>(rho));
#pragma unroll
      for (int e = 0; e < E; ++e) rho[e] = ((ssgn >> e) & 1u) ? -rho[e] : rho[e];
      wht_vector<E, L>(rho, sub);
      uint64_t sk = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) sk |= (uint64_t)(rho[e] < 0.0 ? 1u : 0u) << e;
      pack_store<E>(sk, sub, sketch_row);
      if (sub == 0) *rnorm = (float)gam;
    }
  }
  pack_store<E * BITS>(chunk, sub, row);
}

template <int D, int L>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a) {
  constexpr int E = D / L;     // coordinates per lane
  constexpr int VPW = 64 / L;  // vectors per wavefront
  static_assert(L >= 8 && L <= 64 && E >= 1 && E <= 8, "layout");
  __shared__ float s_bnd[256];
  __shared__ float s_cen[128];

  const EncodeJob& jb = a.job[blockIdx.y];
  // The scalars the first vector load depends on come in one round of scalar
  // loads (the empty asm keeps the compiler from splitting it).
  int n_tok = a.n_tok, n_head = a.n_head, bits = jb.bits;
  uint32_t magic = a.head_magic, shift = a.head_shift;
  long long xs_tok = jb.xs_tok, xs_head = jb.xs_head;
  asm volatile("" : "+s"(n_tok), "+s"(n_head), "+s"(bits), "+s"(magic), "+s"(shift),
               "+s"(xs_tok), "+s"(xs_head));

  const int lane = threadIdx.x & 63;
  const int sub = lane & (L - 1);
  const int nvec = n_tok * n_head;  // < 2^31 - 64, checked on the host
  const int v = ((int)blockIdx.x * kWavesPerBlock + (int)(threadIdx.x >> 6)) * VPW + lane / L;
  const bool live = v < nvec;  // whole vectors: the L lanes of a vector agree
  // Lanes past the end read vector 0, so the load needs no branch (a branch
  // would make the compiler wait for it before the boundary copy below).
  const int vl = live ? v : 0;
  const int t = (int)(((uint64_t)(uint32_t)vl * magic) >> shift);
  const int h = vl - t * n_head;
  const __half* xv = (const __half*)jb.x + (long long)t * xs_tok + (long long)h * xs_head + E * sub;
  __half xh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xh[e] = xv[e];
  uint32_t words[D / 32];
#pragma unroll
  for (int w = 0; w < D / 32; ++w) words[w] = jb.sign.bits[w];

  const int prod = jb.prod;
  if (bits >= 5 || prod) {  // block-uniform: LDS copies of the boundaries / centroids
    static_assert(64 * kWavesPerBlock >= 255, "one boundary per thread");
    if ((int)threadIdx.x < (1 << bits) - 1) s_bnd[threadIdx.x] = jb.boundaries[threadIdx.x];
    if (prod && (int)threadIdx.x < (1 << bits))
      s_cen[threadIdx.x] = jb.boundaries[128 + threadIdx.x];
    __syncthreads();
  }
  if (!live) return;

  // signs of coordinates E*sub .. E*sub+E-1 (one word; E divides 32)
  uint32_t sw = words[0];
#pragma unroll
  for (int w = 1; w < D / 32; ++w) sw = ((E * sub) >> 5 == w) ? words[w] : sw;
  const uint32_t sgn = sw >> ((E * sub) & 31);
  double xd[E];
#pragma unroll
  for (int e = 0; e < E; ++e) xd[e] = (double)__half2float(xh[e]);

  double u[E];
#pragma unroll
  for (int e = 0; e < E; ++e) u[e] = ((sgn >> e) & 1u) ? -xd[e] : xd[e];
  // squared norm: canonical pairwise tree over x
  const double nrm = __builtin_sqrt(tree_sum_sq<E, L>(xd));
  // Walsh-Hadamard butterfly
  wht_vector<E, L>(u, sub);

  if (sub == 0) jb.norms[(long long)t * jb.ns_tok + (long long)h * jb.ns_head] = (float)nrm;
  uint8_t* row = jb.codes + (long long)t * jb.cs_tok + (long long)h * jb.cs_head;
  uint8_t* srow = nullptr;
  float* rn = nullptr;
  uint32_t ssgn = 0;
  if (prod) {
    srow = jb.sketch + (long long)t * jb.ss_tok + (long long)h * jb.ss_head;
    rn = jb.rnorms + (long long)t * jb.rs_tok + (long long)h * jb.rs_head;
    uint32_t sw2 = jb.sketch_sign.bits[0];
#pragma unroll
    for (int w = 1; w < D / 32; ++w) sw2 = ((E * sub) >> 5 == w) ? jb.sketch_sign.bits[w] : sw2;
    ssgn = sw2 >> ((E * sub) & 31);
  }
#define TQ_Q(B) quantize_store<E, L, B>(u, nrm, sub, jb, s_bnd, s_cen, ssgn, row, srow, rn)
  switch (bits) {
    case 1: TQ_Q(1); break;
    case 2: TQ_Q(2); break;
    case 3: TQ_Q(3); break;
    case 4: TQ_Q(4); break;
    case 5: TQ_Q(5); break;
    case 6: TQ_Q(6); break;
    case 7: TQ_Q(7); break;
    default: TQ_Q(8); break;
  }
#undef TQ_Q
}

template <int D, int L>
hipError_t launch_layout(EncodeArgs& a, hipStream_t stream) {
  const long long nvec = (long long)a.n_tok * a.n_head;
  const long long per_block = (long long)kWavesPerBlock * (64 / L);
  const long long blocks = (nvec + per_block - 1) / per_block;
  hipLaunchKernelGGL((encode_kernel<D, L>), dim3((unsigned)blocks, (unsigned)a.n_jobs),
                     dim3(64 * kWavesPerBlock), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(EncodeArgs& a, hipStream_t stream) {
  const long long vecs = (long long)a.n_tok * a.n_head * a.n_jobs;
  const long long narrow_waves = (vecs + (64 / (D / 8)) - 1) / (64 / (D / 8));
  if (narrow_waves < kNarrowMinWaves) return launch_layout<D, (D < 64 ? D : 64)>(a, stream);
  return launch_layout<D, D / 8>(a, stream);
}

}  // namespace

hipError_t launch_encode(int dim, EncodeArgs& args, hipStream_t stream) {
  if (args.n_jobs < 1 || args.n_jobs > kMaxEncodeJobs) return hipErrorInvalidValue;
  if (args.n_tok < 1 || args.n_head < 1 ||
      (long long)args.n_tok * args.n_head > kMaxEncodeVectors)
    return hipErrorInvalidValue;
  for (int i = 0; i < args.n_jobs; ++i)
    if (args.job[i].bits < 1 || args.job[i].bits > 8) return hipErrorInvalidValue;
  // Division by the invariant n_head through a multiply and shift (Granlund and
  // Montgomery, "Division by invariant integers using multiplication", 1994):
  // with l = ceil(log2 n_head) and m = ceil(2^(31+l) / n_head) < 2^32,
  // floor(v * m / 2^(31+l)) = floor(v / n_head) for every 0 <= v < 2^31.
  const uint64_t dv = (uint64_t)args.n_head;
  uint32_t l = 0;
  while ((1ull << l) < dv) ++l;
  args.head_shift = 31 + l;
  args.head_magic = (uint32_t)(((1ull << (31 + l)) + dv - 1) / dv);
  switch (dim) {
    case 64: return launch_dim<64>(args, stream);
    case 128: return launch_dim<128>(args, stream);
    case 256: return launch_dim<256>(args, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq

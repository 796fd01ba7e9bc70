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
// Mapping: one 64-lane wavefront per vector; lane l owns the E = d/64
// contiguous coordinates E*l .. E*l+E-1. In-lane butterfly stages first, then
// cross-lane stages through __shfl_xor (DPP / ds_swizzle). The norm's tree is
// the in-lane pairwise sum followed by an xor-butterfly with ascending lane
// masks, which is the canonical tree evaluated in every lane (fp add is
// commutative, so the partner order does not matter). Packing: lane l's E
// codes form an E*bits-bit chunk at stream offset E*bits*l; output lane w
// gathers the chunks that overlap dword w with wavefront shuffles and stores
// one dword, so a row is written with coalesced 4-byte stores.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace tq {

namespace {

constexpr int kWavesPerBlock = 4;

template <int D, int BITS>
__global__ __launch_bounds__(256) void encode_kernel(
    const __half* __restrict__ x, int n_tok, int n_head, long long xs_tok, long long xs_head,
    uint8_t* __restrict__ codes, long long cs_tok, long long cs_head, float* __restrict__ norms,
    long long ns_tok, long long ns_head, EncodeTables tabs) {
  constexpr int E = D / 64;
  constexpr int NB = (1 << BITS) - 1;
  constexpr int CHUNK = E * BITS;          // bits per lane, <= 32
  constexpr int NW = D * BITS / 32;        // output dwords per row
  constexpr bool kSearch = BITS >= 5;      // binary search in LDS above 16 levels
  __shared__ float s_bnd[kSearch ? 256 : 1];
  if (kSearch) {
    for (int i = threadIdx.x; i < NB; i += blockDim.x) s_bnd[i] = tabs.boundaries[i];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const long long nvec = (long long)n_tok * n_head;
  const long long v = (long long)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (v >= nvec) return;
  const int t = (int)(v / n_head);
  const int h = (int)(v - (long long)t * n_head);

  const __half* xv = x + (long long)t * xs_tok + (long long)h * xs_head + E * lane;
  double u[E], sq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double xe = (double)__half2float(xv[e]);
    const int j = E * lane + e;
    const bool neg = (tabs.sign.bits[j >> 5] >> (j & 31)) & 1u;
    u[e] = neg ? -xe : xe;
    sq[e] = xe * xe;
  }
  // squared norm: canonical pairwise tree
  double s;
  if constexpr (E == 1) {
    s = sq[0];
  } else if constexpr (E == 2) {
    s = sq[0] + sq[1];
  } else {
    s = (sq[0] + sq[1]) + (sq[2] + sq[3]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
  const double nrm = __builtin_sqrt(s);

  // Walsh-Hadamard butterfly, in-lane stages then cross-lane stages
#pragma unroll
  for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((e & hs) == 0) {
        const double a = u[e], b = u[e + hs];
        u[e] = a + b;
        u[e + hs] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double p = __shfl_xor(u[e], m);
      u[e] = upper ? (p - u[e]) : (u[e] + p);
    }
  }

  // boundary count and per-lane chunk of packed bits
  uint32_t chunk = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double z = (nrm == 0.0) ? 0.0 : u[e] / nrm;
    uint32_t idx = 0;
    if constexpr (kSearch) {
#pragma unroll
      for (int step = 1 << (BITS - 1); step > 0; step >>= 1)
        if ((double)s_bnd[idx + step - 1] < z) idx += step;
    } else {
#pragma unroll
      for (int k = 0; k < NB; ++k) idx += ((double)tabs.boundaries[k] < z) ? 1u : 0u;
    }
    chunk |= idx << (BITS * e);
  }

  // gather the chunks overlapping output dword w = lane
  constexpr int R = 32 / CHUNK + 2;
  const int w = lane < NW ? lane : 0;
  const int l0 = (32 * w) / CHUNK;
  uint32_t word = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int src = l0 + r;
    const uint32_t val = (uint32_t)__shfl((int)chunk, src < 64 ? src : 63);
    const int off = CHUNK * src - 32 * w;
    if (src < 64 && off < 32 && off > -CHUNK) word |= off >= 0 ? (val << off) : (val >> (-off));
  }
  if (lane < NW) {
    uint32_t* row = (uint32_t*)(codes + (long long)t * cs_tok + (long long)h * cs_head);
    row[lane] = word;
  }
  if (lane == 0) norms[(long long)t * ns_tok + (long long)h * ns_head] = (float)nrm;
}

template <int D, int BITS>
hipError_t launch_one(const void* x, int n_tok, int n_head, int64_t xs_tok, int64_t xs_head,
                      uint8_t* codes, int64_t cs_tok, int64_t cs_head, float* norms,
                      int64_t ns_tok, int64_t ns_head, const EncodeTables& tabs,
                      hipStream_t stream) {
  const long long nvec = (long long)n_tok * n_head;
  const long long blocks = (nvec + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((encode_kernel<D, BITS>), dim3((unsigned)blocks), dim3(64 * kWavesPerBlock),
                     0, stream, (const __half*)x, n_tok, n_head, (long long)xs_tok,
                     (long long)xs_head, codes, (long long)cs_tok, (long long)cs_head, norms,
                     (long long)ns_tok, (long long)ns_head, tabs);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(int bits, const void* x, int n_tok, int n_head, int64_t xs_tok,
                      int64_t xs_head, uint8_t* codes, int64_t cs_tok, int64_t cs_head,
                      float* norms, int64_t ns_tok, int64_t ns_head, const EncodeTables& tabs,
                      hipStream_t stream) {
#define TQ_ENC_CASE(B)                                                                      \
  case B:                                                                                   \
    return launch_one<D, B>(x, n_tok, n_head, xs_tok, xs_head, codes, cs_tok, cs_head,     \
                            norms, ns_tok, ns_head, tabs, stream);
  switch (bits) {
    TQ_ENC_CASE(1)
    TQ_ENC_CASE(2)
    TQ_ENC_CASE(3)
    TQ_ENC_CASE(4)
    TQ_ENC_CASE(5)
    TQ_ENC_CASE(6)
    TQ_ENC_CASE(7)
    TQ_ENC_CASE(8)
  }
#undef TQ_ENC_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_encode(int dim, int bits, const void* x, int n_tok, int n_head,
                         int64_t xs_tok, int64_t xs_head, uint8_t* codes, int64_t cs_tok,
                         int64_t cs_head, float* norms, int64_t ns_tok, int64_t ns_head,
                         const EncodeTables& tabs, hipStream_t stream) {
  switch (dim) {
    case 64:
      return launch_dim<64>(bits, x, n_tok, n_head, xs_tok, xs_head, codes, cs_tok, cs_head,
                            norms, ns_tok, ns_head, tabs, stream);
    case 128:
      return launch_dim<128>(bits, x, n_tok, n_head, xs_tok, xs_head, codes, cs_tok, cs_head,
                             norms, ns_tok, ns_head, tabs, stream);
    case 256:
      return launch_dim<256>(bits, x, n_tok, n_head, xs_tok, xs_head, codes, cs_tok, cs_head,
                             norms, ns_tok, ns_head, tabs, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq

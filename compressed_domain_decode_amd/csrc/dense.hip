// dense.hip -- codecs whose rotation is a dense matrix, for head dims with no
// Walsh-Hadamard transform (PR #232, Known limitations: power-of-2 head dims
// use the WHT, others fall back to a dense rotation; VeloxQuant "How I built",
// Stage 1: the original method's rotation is the Q factor of a Gaussian matrix).
//
// The caller supplies m (d x d, m / sqrt(d) orthogonal, d a multiple of 32 up
// to 256). With m = H diag(sigma) this is exactly the Walsh-Hadamard codec.
//
// Encode, per fp16 vector x:
//   N = sqrt(sum_j x_j^2)  fp64; pairwise tree in index order, an odd last
//                          element carried up to the next level
//   w = m x                fp64; products and sums in index order, no fused
//                          multiply-add
//   z = w / N (0 when N = 0), index = #{boundaries < z}, packed LSB-first.
// dense_encode_lds_kernel (d <= 96) holds m in LDS and takes passes of 64
// vectors, 4 x 4 output tiles per thread; dense_encode_kernel (larger d)
// reads m transposed from global memory, four vectors per wavefront.
//
// Attend (the same split / combine shape as the Walsh-Hadamard path, without
// its matrix-core scoring): q_hat = scale log2(e) / d * m_K q per query head;
// scores s = n_t q_hat . c_K[idx_t]; online softmax in base 2; the values
// accumulate p_t n^V_t c_V[idx^V_t] in the rotated basis; the combine merges
// the splits and applies the inverse rotation out = m_V^T a / d.
// dense_lt_kernel (one query head per KV head, d = 64, 96, 128 or 256; also
// for Walsh-Hadamard codec pairs of that shape, m = H diag(sigma)) keeps a
// token's work in registers, two lanes per token (four at 256);
// dense_split_kernel (other shapes) stages 64-token tiles in LDS, a lane
// scoring one token and then owning coordinates for the values.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "codec.hpp"
#include "kernels.hpp"
#include "xlane.hpp"

namespace tq {
namespace {

constexpr int kDW = 4;           // wavefronts per encode workgroup
constexpr int kDTile = 64;       // tokens per wavefront tile
constexpr int kDMaxG = 16;       // query heads per KV head
constexpr float kDLog2e = 1.4426950408889634f;
constexpr float kDNoRow = -1e30f;  // running maximum before any row (finite)

__device__ __forceinline__ void dwave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ float dwave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float dwave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Copy n dwords src -> dst (LDS) with up to 16 loads per lane in flight
// before the first store (a load-store pair per iteration would wait out one
// memory round trip per dword).
__device__ __forceinline__ void stage_rows(uint32_t* dst, const uint32_t* src, int n, int lane) {
  for (int k0 = 0; k0 < n; k0 += 64 * 16) {
    uint32_t tmp[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int k = k0 + lane + 64 * u;
      tmp[u] = k < n ? src[k] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int k = k0 + lane + 64 * u;
      if (k < n) dst[k] = tmp[u];
    }
  }
}

// Scores of one token (this lane's K row r) against the G rotated queries,
// for KB-bit codes: 32 coordinates at a time, the row's KB dwords for them in
// registers and every field at a compile-time offset, so the 32 centroid
// lookups are independent.
template <int GM, int KB>
__device__ __forceinline__ void dense_scores(const uint32_t* r, int d, int G, const float* s_q,
                                             const float* s_ck, float (&sc)[GM]) {
  for (int j0 = 0; j0 < d; j0 += 32) {
    uint32_t w[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) w[k] = r[(j0 >> 5) * KB + k];
#pragma unroll
    for (int jj = 0; jj < 32; ++jj) {
      constexpr uint32_t mask = (1u << KB) - 1u;
      const int off = jj * KB, wi = off >> 5, sh = off & 31;
      uint32_t f = w[wi] >> sh;
      if (sh + KB > 32) f |= w[wi + 1] << (32 - sh);
      const float c = s_ck[f & mask];
#pragma unroll
      for (int h = 0; h < GM; ++h)
        if (h < G) sc[h] += s_q[h * d + j0 + jj] * c;
    }
  }
}

// ---------------------------------------------------------------- encode

constexpr int kVPW = 4;  // vectors per encode wavefront: each column load of m serves all

__global__ __launch_bounds__(256) void dense_encode_kernel(DenseEncodeArgs a) {
#pragma clang fp contract(off)
  __shared__ float s_bnd[256];
  __shared__ double s_x[kDW][kVPW][kMaxDim];
  __shared__ double s_t[kDW][2][kMaxDim];
  __shared__ uint32_t s_row[kDW][kVPW][kMaxDim * 8 / 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = (1 << a.bits) - 1;
  s_bnd[threadIdx.x] = (int)threadIdx.x < nb ? a.boundaries[threadIdx.x] : 0.f;
  __syncthreads();
  const long long nvec = (long long)a.n_tok * a.n_head;
  const long long v0 = ((long long)blockIdx.x * kDW + wave) * kVPW;
  if (v0 >= nvec) return;  // whole wavefront
  const int nv = nvec - v0 < kVPW ? (int)(nvec - v0) : kVPW;
  const int d = a.dim, b = a.bits, words = d * b / 32;
  double nrm[kVPW];
#pragma unroll
  for (int u = 0; u < kVPW; ++u) {
    double* xs = s_x[wave][u];
    double* cur = s_t[wave][0];
    double* nxt = s_t[wave][1];
    if (u < nv) {
      const long long v = v0 + u, t = v / a.n_head, h = v - t * a.n_head;
      const __half* x = (const __half*)a.x + t * a.xs_tok + h * a.xs_head;
      for (int j = lane; j < d; j += 64) {
        const double xv = (double)__half2float(x[j]);
        xs[j] = xv;
        cur[j] = xv * xv;  // exact
      }
    } else {
      for (int j = lane; j < d; j += 64) xs[j] = cur[j] = 0.0;
    }
    for (int k = lane; k < words; k += 64) s_row[wave][u][k] = 0u;
    dwave_sync();
    // sum of squares: pairwise tree in index order, an odd last element carried up
    for (int w = d; w > 1; w = (w + 1) >> 1) {
      for (int i = lane; i < (w >> 1); i += 64) nxt[i] = cur[2 * i] + cur[2 * i + 1];
      if ((w & 1) && lane == 0) nxt[w >> 1] = cur[w - 1];
      dwave_sync();
      double* tmp = cur;
      cur = nxt;
      nxt = tmp;
    }
    nrm[u] = __builtin_sqrt(cur[0]);
    dwave_sync();  // the tree buffers are reused by the next vector
  }
  // w = m x for the wavefront's vectors: products and sums in index order
  double acc[kVPW][kMaxDim / 64];
#pragma unroll
  for (int u = 0; u < kVPW; ++u)
#pragma unroll
    for (int e = 0; e < kMaxDim / 64; ++e) acc[u][e] = 0.0;
#pragma unroll 4
  for (int j = 0; j < d; ++j) {  // d is a multiple of 32
    const double* col = a.mt + (size_t)j * d;
#pragma unroll
    for (int e = 0; e < kMaxDim / 64; ++e) {
      const int i = lane + 64 * e;
      if (i < d) {
        const double m = col[i];
#pragma unroll
        for (int u = 0; u < kVPW; ++u) acc[u][e] = acc[u][e] + m * s_x[wave][u][j];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kVPW; ++u) {
    if (u < nv) {
      uint32_t* srow = s_row[wave][u];
#pragma unroll
      for (int e = 0; e < kMaxDim / 64; ++e) {
        const int i = lane + 64 * e;
        if (i < d) {
          const double z = nrm[u] == 0.0 ? 0.0 : acc[u][e] / nrm[u];
          int c = 0;
          for (int s = (nb + 1) >> 1; s >= 1; s >>= 1)
            if ((double)s_bnd[c + s - 1] < z) c += s;
          // LSB-first: the code occupies stream bits i*b .. i*b + b - 1
          const int p = i * b, wi = p >> 5, sh = p & 31;
          atomicOr(&srow[wi], (uint32_t)c << sh);
          if (sh + b > 32) atomicOr(&srow[wi + 1], (uint32_t)c >> (32 - sh));
        }
      }
    }
  }
  dwave_sync();
#pragma unroll
  for (int u = 0; u < kVPW; ++u) {
    if (u < nv) {
      const long long v = v0 + u, t = v / a.n_head, h = v - t * a.n_head;
      uint32_t* row = (uint32_t*)(a.codes + t * a.cs_tok + h * a.cs_head);
      for (int k = lane; k < words; k += 64) row[k] = s_row[wave][u][k];
      if (lane == 0) a.norms[t * a.ns_tok + h * a.ns_head] = (float)nrm[u];
    }
  }
}

// Encode with the rotation staged in LDS, for head dims up to 96. The kernel
// above reads the whole transposed rotation from L2 for every four vectors;
// here a workgroup copies it into LDS once and takes passes of kEV vectors.
// Per pass: the vectors go to LDS as fp64; one thread per vector sums its
// squares over the same pairwise tree (written as a compile-time recursion
// over index ranges); each thread computes a tile of 4 vectors x 4
// coordinates of w = m x, every output's products and sums in index order
// (no fused multiply-add); then it bucketizes its 16 outputs and ORs each
// vector's four codes into that vector's LDS row, which is stored as dwords.
constexpr int kEV = 64;  // vectors per pass

template <int D>
struct EncLds {
  static constexpr int THREADS = (kEV / 4) * (D / 4);
  static constexpr int XS = D + 1;             // LDS row stride of a staged vector (doubles)
  static constexpr int WORDS = D * 8 / 32;     // dwords of a row at 8 bits (the most)
  static constexpr int PER = kEV * D / THREADS;  // staged elements per thread (16)
  static constexpr int NS = D / 32;              // 32-leaf subtrees of a norm's tree
  static constexpr size_t BYTES = sizeof(double) * ((size_t)D * D + (size_t)kEV * XS + kEV +
                                                    (size_t)kEV * NS) +
                                  sizeof(long long) * 3 * kEV +
                                  sizeof(uint32_t) * ((size_t)kEV * WORDS + 256);
};

// Sum of x_j^2 over leaves [LO, LO + SIZE) of an N-leaf pairwise tree in
// index order: a node adds its two halves, and a half that starts past the
// last leaf is absent (the level-by-level tree's odd last element carried up).
template <int N, int LO, int SIZE>
__device__ __forceinline__ double enc_tree(const double* x) {
#pragma clang fp contract(off)
  if constexpr (SIZE == 1) {
    return x[LO] * x[LO];
  } else if constexpr (LO + SIZE / 2 >= N) {
    return enc_tree<N, LO, SIZE / 2>(x);
  } else {
    return enc_tree<N, LO, SIZE / 2>(x) + enc_tree<N, LO + SIZE / 2, SIZE / 2>(x);
  }
}
constexpr int enc_pow2(int n) { return n <= 1 ? 1 : 2 * enc_pow2((n + 1) / 2); }
// The same tree above its 32-leaf subtrees, whose sums are sub[0], sub[1], ...
// (D a multiple of 32: every subtree is whole).
template <int N, int LO, int SIZE>
__device__ __forceinline__ double enc_tree_top(const double* sub) {
#pragma clang fp contract(off)
  if constexpr (SIZE == 32) {
    return sub[LO / 32];
  } else if constexpr (LO + SIZE / 2 >= N) {
    return enc_tree_top<N, LO, SIZE / 2>(sub);
  } else {
    return enc_tree_top<N, LO, SIZE / 2>(sub) + enc_tree_top<N, LO + SIZE / 2, SIZE / 2>(sub);
  }
}

template <int D>
__global__ __launch_bounds__(EncLds<D>::THREADS) void dense_encode_lds_kernel(DenseEncodeArgs a) {
#pragma clang fp contract(off)
  using E = EncLds<D>;
  extern __shared__ __attribute__((aligned(16))) double elds[];
  double* s_m = elds;                              // [j][i] = m[i][j]
  double* s_x = s_m + D * D;                       // [u][XS]
  double* s_n = s_x + kEV * E::XS;                 // [kEV] norms
  double* s_sub = s_n + kEV;                       // [kEV][NS] subtree sums of squares
  long long* s_off = (long long*)(s_sub + kEV * E::NS);  // [3][kEV] offsets of x, codes, norms
  uint32_t* s_row = (uint32_t*)(s_off + 3 * kEV);  // [kEV][WORDS]
  float* s_bnd = (float*)(s_row + kEV * E::WORDS);  // [256]
  const int tid = threadIdx.x;
  const int b = a.bits, nb = (1 << b) - 1, words = D * b / 32;
  for (int k = tid; k < D * D; k += E::THREADS) s_m[k] = a.mt[k];
  for (int k = tid; k < 256; k += E::THREADS) s_bnd[k] = k < nb ? a.boundaries[k] : 0.f;
  const long long nvec = (long long)a.n_tok * a.n_head;
  const long long npass = (nvec + kEV - 1) / kEV;
  const int uq = tid / (D / 4), iq = tid - uq * (D / 4);  // tile: vectors 4 uq.., coordinates 4 iq..
  for (long long pass = blockIdx.x; pass < npass; pass += gridDim.x) {
    const long long v0 = pass * kEV;
    const int nv = nvec - v0 < kEV ? (int)(nvec - v0) : kEV;
    // each vector's offsets, once (one thread per vector)
    if (tid < nv) {
      const long long v = v0 + tid, t = v / a.n_head, h = v - t * a.n_head;
      s_off[tid] = t * a.xs_tok + h * a.xs_head;
      s_off[kEV + tid] = t * a.cs_tok + h * a.cs_head;
      s_off[2 * kEV + tid] = t * a.ns_tok + h * a.ns_head;
    }
    for (int k = tid; k < kEV * words; k += E::THREADS) s_row[(k / words) * E::WORDS + k % words] = 0u;
    __syncthreads();
    // stage the pass's vectors (zeros past the last): all loads before any store
    {
      float xf[E::PER];
#pragma unroll
      for (int r = 0; r < E::PER; ++r) {
        const int k = tid + r * E::THREADS, u = k / D, j = k - u * D;
        xf[r] = u < nv ? __half2float(((const __half*)a.x)[s_off[u] + j]) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < E::PER; ++r) {
        const int k = tid + r * E::THREADS, u = k / D, j = k - u * D;
        s_x[u * E::XS + j] = (double)xf[r];
      }
    }
    __syncthreads();
    if (tid < kEV * E::NS) {  // one 32-leaf subtree per thread
      const int u = tid / E::NS, q = tid - u * E::NS;
      s_sub[tid] = enc_tree<32, 0, 32>(s_x + u * E::XS + 32 * q);
    }
    double w[4][4];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) w[uu][ii] = 0.0;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
      double mv[4], xv[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) mv[ii] = s_m[j * D + 4 * iq + ii];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) xv[uu] = s_x[(4 * uq + uu) * E::XS + j];
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) w[uu][ii] = w[uu][ii] + mv[ii] * xv[uu];
    }
    __syncthreads();  // subtree sums written
    // norms (the tree above the subtrees), z = w / N, and the codes: the 16
    // binary searches advance together, one boundary level at a time
    double z[4][4];
    int c[4][4];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int u = 4 * uq + uu;
      const double nrm = __builtin_sqrt(enc_tree_top<D, 0, enc_pow2(D)>(s_sub + u * E::NS));
      if (iq == 0) s_n[u] = nrm;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        z[uu][ii] = nrm == 0.0 ? 0.0 : w[uu][ii] / nrm;
        c[uu][ii] = 0;
      }
    }
    for (int st = (nb + 1) >> 1; st >= 1; st >>= 1) {
#pragma unroll
      for (int uu = 0; uu < 4; ++uu)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if ((double)s_bnd[c[uu][ii] + st - 1] < z[uu][ii]) c[uu][ii] += st;
    }
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int u = 4 * uq + uu;
      if (u < nv) {
        uint32_t pk = 0u;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) pk |= (uint32_t)c[uu][ii] << (ii * b);
        // the four codes occupy stream bits 4 iq b .. 4 iq b + 4 b - 1, LSB first
        const int p = 4 * iq * b, wi = p >> 5, sh = p & 31;
        atomicOr(&s_row[u * E::WORDS + wi], pk << sh);
        if (sh + 4 * b > 32) atomicOr(&s_row[u * E::WORDS + wi + 1], pk >> (32 - sh));
      }
    }
    __syncthreads();
    for (int k = tid; k < nv * words; k += E::THREADS) {
      const int u = k / words, kw = k - u * words;
      ((uint32_t*)(a.codes + s_off[kEV + u]))[kw] = s_row[u * E::WORDS + kw];
    }
    for (int u = tid; u < nv; u += E::THREADS) a.norms[s_off[2 * kEV + u]] = (float)s_n[u];
    __syncthreads();  // rows and vectors read before the next pass
  }
}

// ---------------------------------------------------------------- attend

// Key rotation entry m_K[i][j]. For Walsh-Hadamard codecs m = H diag(sigma)
// with H_ij = (-1)^popcount(i & j), so an entry is a sign (the combine applies
// the value rotation of such codecs by butterflies instead).
__device__ __forceinline__ double rot_k(const DenseAttendArgs& a, int i, int j) {
  if (a.wht) return ((__popc(i & j) + (a.wht_k.bits[j >> 5] >> (j & 31))) & 1) ? -1.0 : 1.0;
  return a.mt_k[(size_t)j * a.dim + i];
}

// Grid (splits, n_kv_heads, batch); nw = blockDim.x / 64 wavefronts take the
// range's 64-token tiles in turn and merge at the end; one partial
// (m, l, acc[d]) per query head and split, in base-2 units. GM and EM bound
// the query heads per KV head and the coordinates per lane (d / 64, rounded
// up) so that the per-lane arrays stay in registers; with EX the group size
// is exactly GM and the per-head loops have no run-time guard. LDS (sized at launch):
// rotated queries [G][d], the two centroid tables, running (m, l) per
// wavefront, and per wavefront a region of a.wave_stride floats holding the
// tile's staged rows (a.rows_words dwords) and weights [64][G], reused for its
// accumulators [G][d] at the merge.
template <int GM, int EM, bool EX>
__global__ __launch_bounds__(GM * EM > 8 ? 512 : 1024) void dense_split_kernel(DenseAttendArgs a) {
  extern __shared__ __attribute__((aligned(16))) float dlds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int d = a.dim, G = EX ? GM : a.group, kb = a.k_bits, vb = a.v_bits;
  float* s_q = dlds;
  float* s_ck = s_q + G * d;
  float* s_cv = s_ck + 256;
  float* s_ml = s_cv + 256;                       // [nw][2][G]
  float* s_wave = s_ml + ((nw * 2 * G + 3) & ~3);
  float* mine = s_wave + (size_t)wave * a.wave_stride;
  uint32_t* rows = (uint32_t*)mine;
  float* s_w = mine + a.rows_words;               // [64][G]
  for (int k = tid; k < 256; k += blockDim.x) {
    s_ck[k] = a.k_centroids[k];
    s_cv[k] = a.v_centroids[k];
  }
  // rotated queries of this KV head's group: q_hat_i = sum_j m_ij q_j
  const __half* qg = (const __half*)a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * d;
  for (int idx = tid; idx < G * d; idx += blockDim.x) {
    const int h = idx / d, i = idx - h * d;
    const __half* qh = qg + (size_t)h * d;
    double acc = 0.0;
#pragma unroll 8
    for (int j = 0; j < d; ++j) acc += rot_k(a, i, j) * (double)__half2float(qh[j]);
    s_q[h * d + i] = (float)(acc * (double)a.qscale);
  }
  __syncthreads();

  const int len = min(a.lengths[b], a.max_len);  // never read past the host bound
  const long long t_begin = (long long)s * a.tokens_per_split;
  const long long t_stop = t_begin + a.tokens_per_split;
  const int t_end = (int)(t_stop < len ? t_stop : (len > 0 ? len : 0));
  const int kw = d * kb / 32, vw = d * vb / 32;  // dwords per row
  const size_t row0 = ((size_t)b * a.n_kv_heads + g) * (size_t)a.max_ctx;
  const uint32_t* kbase = (const uint32_t*)a.k_codes + row0 * kw;
  const uint32_t* vbase = (const uint32_t*)a.v_codes + row0 * vw;

  // this lane's value coordinates lane + 64 e: field positions in a V row
  int v_wi[EM], v_sh[EM];
#pragma unroll
  for (int e = 0; e < EM; ++e) {
    const int p = (lane + 64 * e) * vb;
    v_wi[e] = p >> 5;
    v_sh[e] = p & 31;
  }
  const uint32_t v_mask = (1u << vb) - 1u;
  float m_run[GM], l_run[GM], acc[GM][EM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m_run[h] = kDNoRow;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EM; ++e) acc[h][e] = 0.f;
  }
  for (long long t0 = t_begin + (long long)kDTile * wave; t0 < t_end;
       t0 += (long long)kDTile * nw) {
    const int cnt = (int)(t_end - t0 < kDTile ? t_end - t0 : kDTile);
    const bool valid = lane < cnt;
    // K rows t0 .. t0 + cnt - 1 are contiguous
    const uint32_t* ksrc = kbase + (size_t)t0 * kw;
    stage_rows(rows, ksrc, cnt * kw, lane);
    const float nk = valid ? a.k_norms[row0 + t0 + lane] : 0.f;
    const float nv = valid ? a.v_norms[row0 + t0 + lane] : 0.f;
    dwave_sync();
    float sc[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) sc[h] = 0.f;
    if (valid) {
      const uint32_t* r = rows + lane * kw;
      switch (kb) {
        case 1: dense_scores<GM, 1>(r, d, G, s_q, s_ck, sc); break;
        case 2: dense_scores<GM, 2>(r, d, G, s_q, s_ck, sc); break;
        case 3: dense_scores<GM, 3>(r, d, G, s_q, s_ck, sc); break;
        case 4: dense_scores<GM, 4>(r, d, G, s_q, s_ck, sc); break;
        case 5: dense_scores<GM, 5>(r, d, G, s_q, s_ck, sc); break;
        case 6: dense_scores<GM, 6>(r, d, G, s_q, s_ck, sc); break;
        case 7: dense_scores<GM, 7>(r, d, G, s_q, s_ck, sc); break;
        default: dense_scores<GM, 8>(r, d, G, s_q, s_ck, sc); break;
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float sv = valid ? sc[h] * nk : -INFINITY;
        const float mn = fmaxf(m_run[h], dwave_max(sv));
        const float alpha = exp2f(m_run[h] - mn);
        const float p = exp2f(sv - mn);
        l_run[h] = l_run[h] * alpha + dwave_sum(p);
#pragma unroll
        for (int e = 0; e < EM; ++e) acc[h][e] *= alpha;
        m_run[h] = mn;
        s_w[lane * G + h] = p * nv;
      }
    }
    dwave_sync();  // K rows read, weights written
    const uint32_t* vsrc = vbase + (size_t)t0 * vw;
    stage_rows(rows, vsrc, cnt * vw, lane);
    dwave_sync();
#pragma unroll 4
    for (int t = 0; t < cnt; ++t) {
      const uint32_t* r = rows + t * vw;
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        if (lane + 64 * e < d) {
          uint32_t f = r[v_wi[e]] >> v_sh[e];
          if (v_sh[e] + vb > 32) f |= r[v_wi[e] + 1] << (32 - v_sh[e]);
          const float c = s_cv[f & v_mask];
#pragma unroll
          for (int h = 0; h < GM; ++h)
            if (h < G) acc[h][e] += s_w[t * G + h] * c;
        }
      }
    }
    dwave_sync();  // V rows and weights read before the next tile
  }

  // merge: each wavefront's accumulators go to its own region
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
#pragma unroll
      for (int e = 0; e < EM; ++e) {
        const int j = lane + 64 * e;
        if (j < d) mine[h * d + j] = acc[h][e];
      }
      if (lane == 0) {
        s_ml[(wave * 2) * G + h] = m_run[h];
        s_ml[(wave * 2 + 1) * G + h] = l_run[h];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * d; idx += blockDim.x) {
    const int h = idx / d, j = idx - h * d;
    float mx = s_ml[h];
    for (int w = 1; w < nw; ++w) mx = fmaxf(mx, s_ml[(w * 2) * G + h]);
    float A = 0.f, L = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float f = exp2f(s_ml[(w * 2) * G + h] - mx);
      A += s_wave[(size_t)w * a.wave_stride + h * d + j] * f;
      L += s_ml[(w * 2 + 1) * G + h] * f;
    }
    const size_t slot = ((size_t)b * a.n_q_heads + (size_t)g * G + h) * a.splits + s;
    a.pacc[slot * d + j] = A;
    if (j == 0) {
      a.pml[slot * 2] = mx;
      a.pml[slot * 2 + 1] = L;
    }
  }
}

// ------------------------------------------------ attend, one query head per KV head
//
// With one query head per KV head (multi-head attention: no group shares a
// KV row) the kernel above spends its time in dependent LDS round trips
// (staged row, then centroid, per token and coordinate) with a quarter of
// its lanes idle at head dim 96. Here everything a token needs stays in
// registers: two lanes share a token (four at head dim 256), each holding
// its part of the rotated query and of the value accumulator, and each lane
// keeps its own online softmax state (running maximum, sum) over the tokens
// it visits, so a step needs no cross-lane work beyond adding the parts'
// scores. A lane loads its part of a row straight from global memory, one
// step ahead. The lanes' states are merged once, at the end of the range:
// per wavefront by two transposing lane swaps and LDS, then across
// wavefronts.

template <int... Is, class F>
__device__ __forceinline__ void sfor_d_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <int N, class F>
__device__ __forceinline__ void sfor_d(F&& f) {
  sfor_d_impl(std::make_integer_sequence<int, N>{}, f);
}

// lanes per token: two, or four at d = 256 (a lane then holds 64 coordinates,
// as at d = 128)
template <int D>
constexpr int lt_lanes() { return D <= 128 ? 2 : 4; }
// wavefronts per workgroup: 4 per SIMD where a lane's state fits 128 VGPRs
// (d = 64), 3 where it fits 168 (d = 96), else 2
template <int D>
constexpr int lt_waves() { return D <= 64 ? 16 : D <= 96 ? 12 : 8; }
constexpr float kLtSlack = 8.f;  // the running maximum moves only when a score exceeds it by more

template <int D, int KB, int VB>
struct LtShape {
  static constexpr int P = lt_lanes<D>();                   // lanes per token
  static constexpr int STEP = 64 / P;                       // tokens per wavefront step
  static constexpr int H = D / P;                           // coordinates per lane
  static constexpr int HK = H * KB, HV = H * VB;            // bits of a lane's part of a row
  static constexpr int KW = D * KB / 32, VW = D * VB / 32;  // dwords per row
  // dwords a lane loads (with two parts the second may start inside a dword)
  // and keeps once its part is shifted down to bit 0
  static constexpr int KL = (HK % 32 + HK + 31) / 32, VL = (HV % 32 + HV + 31) / 32;
  static constexpr int KS = (HK + 31) / 32, VS = (HV + 31) / 32;
  // V codes of up to 3 bits are looked up two coordinates at a time
  static constexpr bool VP = VB <= 3;
  static constexpr int VPN = VP ? (1 << (2 * VB)) * 32 : 1;  // pair-table entries
  static constexpr int R = H / 4;   // accumulators per lane after the two swaps
  static constexpr int RP = R | 1;  // their LDS stride (odd: no bank conflicts)
  static_assert(D % 32 == 0 && H % 16 == 0, "head dim");
  // with more than two parts every part starts at a dword (no bit offset)
  static_assert(P == 2 || (HK % 32 == 0 && HV % 32 == 0), "part alignment");
};

// Bits [off, off + 32 S) of the window w (0 <= off < 32) as S dwords.
template <int L, int S>
__device__ __forceinline__ void lt_shift(const uint32_t (&w)[L], int off, uint32_t (&o)[S]) {
#pragma unroll
  for (int k = 0; k < S; ++k) o[k] = __builtin_amdgcn_alignbit(k + 1 < L ? w[k + 1] : 0u, w[k], off);
}
// Code j of a B-bit LSB-first stream held in registers (j a compile-time index).
template <int B, int S>
__device__ __forceinline__ uint32_t lt_field(const uint32_t (&w)[S], int j) {
  const int p = j * B, wi = p >> 5, sh = p & 31;
  uint32_t f = w[wi] >> sh;
  if (sh + B > 32) f |= w[wi + 1] << (32 - sh);
  return f & ((1u << B) - 1u);
}

// Sum of the two registers a lane swap returns. Each is copied to a named
// word before it is reinterpreted: a bit cast taken straight from an element
// of the returned pair compiles to a read of its first element for both.
template <class P>
__device__ __forceinline__ float swap_sum(const P& p) {
  const uint32_t x = p[0], y = p[1];
  return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// (x & m) | o in one VALU operation (written out: the compiler turns the OR
// of the disjoint terms into an add after a separate AND).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(o));
  return r;
}
// Byte offset of code j (width B, at bit j * B of the stream) in a table of
// 256-byte rows, plus the lane's slot o within its row.
template <int B, int S>
__device__ __forceinline__ uint32_t lt_row_off(const uint32_t (&w)[S], int j, uint32_t m, uint32_t o) {
  const int p = j * B, wi = p >> 5, sh = p & 31;
  if (sh + B > 32) return and_or(__builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) << 8, m, o);
  if (sh == 8) return and_or(w[wi], m, o);
  return and_or(sh > 8 ? w[wi] >> (sh - 8) : w[wi] << (8 - sh), m, o);
}
// Byte BY of x, ANDed with m, in one VALU operation (a source byte select;
// written out because the compiler folds the shifts that would lead to it
// into shift-and pairs).
template <int BY>
__device__ __forceinline__ uint32_t byte_and(uint32_t x, uint32_t m) {
  uint32_t r;
  if constexpr (BY == 0) {
    r = x & m;
  } else if constexpr (BY == 1) {
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1 src1_sel:DWORD"
        : "=v"(r) : "v"(x), "v"(m));
  } else if constexpr (BY == 2) {
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2 src1_sel:DWORD"
        : "=v"(r) : "v"(x), "v"(m));
  } else {
    static_assert(BY == 3, "byte");
    asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "=v"(r) : "v"(x), "v"(m));
  }
  return r;
}

template <int D, int KB, int VB>
struct LtRows {
  uint32_t k[LtShape<D, KB, VB>::KL];
  uint32_t v[LtShape<D, KB, VB>::VL];
  float nk, nv;
};

// Grid (splits, n_kv_heads, batch), W wavefronts; the partials have
// the layout of dense_split_kernel's, so dense_combine_kernel finishes both.
template <int D, int KB, int VB, int W>
__global__ __launch_bounds__(64 * W) void dense_lt_kernel(DenseAttendArgs a) {
  using S = LtShape<D, KB, VB>;
  constexpr int H = S::H, NT = 64 * W;
  __shared__ float s_q[D];
  __shared__ float s_ck[1 << KB], s_cv[1 << VB];
  // V pair table: entry (code, slot) = (cV[code & m], cV[code >> VB]) for
  // codes of two coordinates, copied into all 32 eight-byte bank slots so
  // that lane l reading slot l % 32 never conflicts, whatever the codes
  __shared__ float2 s_cvp[S::VPN];
  constexpr int QP = NT / D;  // threads per rotated query coordinate
  // the query rotation's partial sums and the merge's accumulators share LDS
  // (barriers separate their uses)
  constexpr int QP_BYTES = QP * D * 8, RED_BYTES = W * 64 * S::RP * 4;
  __shared__ __attribute__((aligned(16))) unsigned char s_u[QP_BYTES > RED_BYTES ? QP_BYTES : RED_BYTES];
  double (*s_qp)[D] = reinterpret_cast<double (*)[D]>(s_u);
  float (*s_red)[64][S::RP] = reinterpret_cast<float (*)[64][S::RP]>(s_u);
  __shared__ float s_ml[W][2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  constexpr int P = S::P, STEP = S::STEP;
  const int part = lane & (P - 1);  // which 1/P of the coordinates this lane holds

  // the range, and its first rows (in flight during the query rotation)
  const int len = min(a.lengths[b], a.max_len);  // never read past the host bound
  const long long t_stop = (long long)s * a.tokens_per_split + a.tokens_per_split;
  const int t_begin = s * a.tokens_per_split;
  const int t_end = (int)(t_stop < len ? t_stop : (len > 0 ? len : 0));
  const int last = t_end > 0 ? t_end - 1 : 0;  // a row that exists even for an empty range
  const size_t row0 = ((size_t)b * a.n_kv_heads + g) * (size_t)a.max_ctx;
  const uint32_t* kbase = (const uint32_t*)a.k_codes + row0 * S::KW + part * (S::HK / 32);
  const uint32_t* vbase = (const uint32_t*)a.v_codes + row0 * S::VW + part * (S::HV / 32);
  const float* kn = a.k_norms + row0;
  const float* vn = a.v_norms + row0;
  const int me = t_begin + lane / P;
  // rows of step st; tokens past the range read its last row (in bounds)
  auto load = [&](int st, LtRows<D, KB, VB>& r) {
    const int t = me + st * STEP, rr = t < t_end ? t : last;
    const uint32_t* kp = kbase + (size_t)rr * S::KW;
    const uint32_t* vp = vbase + (size_t)rr * S::VW;
#pragma unroll
    for (int k = 0; k < S::KL; ++k) r.k[k] = kp[k];
#pragma unroll
    for (int k = 0; k < S::VL; ++k) r.v[k] = vp[k];
    r.nk = kn[rr];
    r.nv = vn[rr];
  };
  LtRows<D, KB, VB> cur, nxt;
  load(wave, cur);

  for (int k = tid; k < (1 << KB); k += NT) s_ck[k] = a.k_centroids[k];
  for (int k = tid; k < (1 << VB); k += NT) s_cv[k] = a.v_centroids[k];
  if constexpr (S::VP) {
    for (int e = tid; e < S::VPN; e += NT) {
      const int c = e >> 5;
      s_cvp[e] = make_float2(a.v_centroids[c & ((1 << VB) - 1)], a.v_centroids[c >> VB]);
    }
  }
  // rotated query of this KV head's one query head, q_hat_i = sum_j m_ij q_j:
  // QP threads per coordinate sum consecutive stretches of j, then one adds
  // the partial sums in order (fp64 throughout)
  const __half* qg = (const __half*)a.q + ((size_t)b * a.n_q_heads + g) * D;
  if (tid < QP * D) {
    const int i = tid % D, part = tid / D;
    const int j0 = part * D / QP, j1 = (part + 1) * D / QP;
    double acc = 0.0;
#pragma unroll 4
    for (int j = j0; j < j1; ++j) acc += rot_k(a, i, j) * (double)__half2float(qg[j]);
    s_qp[part][i] = acc;
  }
  __syncthreads();
  if (tid < D) {
    double acc = 0.0;
#pragma unroll
    for (int p = 0; p < QP; ++p) acc += s_qp[p][tid];
    s_q[tid] = (float)(acc * (double)a.qscale);
  }
  __syncthreads();

  float qv[H], acc[H];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    qv[i] = s_q[part * H + i];
    acc[i] = 0.f;
  }
  float m = kDNoRow, l = 0.f;
  if (t_end > t_begin) {  // uniform over the workgroup
    const int koff = part * (S::HK % 32), voff = part * (S::HV % 32);
    const int steps = (t_end - t_begin + STEP - 1) / STEP;
    const uint32_t lane8 = (lane & 31) * 8;  // this lane's 8-byte slot in a pair-table row
    const uint32_t m3c = 0x3cu, mpair = ((1u << (2 * VB)) - 1u) << 8;
    // one step over the rows r of step st
    auto step = [&](LtRows<D, KB, VB>& r, int st) {
      const bool valid = me + st * STEP < t_end;
      uint32_t kw[S::KS];
      if constexpr (S::HK % 32 != 0) {
        lt_shift(r.k, koff, kw);
      } else {
#pragma unroll
        for (int k = 0; k < S::KS; ++k) kw[k] = r.k[k];
      }
      float p4[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KB == 4) {
        // code n of a dword as a table byte offset in one AND with a byte
        // select: even codes from w << 2, odd codes from w >> 2
#pragma unroll
        for (int k = 0; k < S::KS; ++k) {
          const uint32_t ea = kw[k] << 2, eb = kw[k] >> 2;
          uint32_t off[8];
          sfor_d<4>([&](auto by) {
            off[2 * by] = byte_and<by>(ea, m3c);
            off[2 * by + 1] = byte_and<by>(eb, m3c);
          });
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const float c = *(const float*)((const char*)s_ck + off[n]);
            p4[n & 3] = fmaf(qv[8 * k + n], c, p4[n & 3]);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < H; ++j) p4[j & 3] = fmaf(qv[j], s_ck[lt_field<KB>(kw, j)], p4[j & 3]);
      }
      float sk = (p4[0] + p4[1]) + (p4[2] + p4[3]);
      // the token's other parts; commutative adds leave the same sum on all
      sk += xor_lane_f32<1>(sk);
      if constexpr (P == 4) sk += xor_lane_f32<2>(sk);
      const float sc = valid ? sk * r.nk : -INFINITY;
      if (sc > m + kLtSlack) {
        const float al = exp2f(m - sc);
        l *= al;
#pragma unroll
        for (int i = 0; i < H; ++i) acc[i] *= al;
        m = sc;
      }
      const float p = exp2f(sc - m);  // at most 2^kLtSlack
      l += p;
      const float w = p * r.nv;
      uint32_t vw[S::VS];
      if constexpr (S::HV % 32 != 0) {
        lt_shift(r.v, voff, vw);
      } else {
#pragma unroll
        for (int k = 0; k < S::VS; ++k) vw[k] = r.v[k];
      }
      if constexpr (S::VP) {
#pragma unroll
        for (int i = 0; i < H / 2; ++i) {
          const uint32_t off = lt_row_off<2 * VB>(vw, i, mpair, lane8);
          const float2 e = *(const float2*)((const char*)s_cvp + off);
          acc[2 * i] = fmaf(w, e.x, acc[2 * i]);
          acc[2 * i + 1] = fmaf(w, e.y, acc[2 * i + 1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < H; ++j) acc[j] = fmaf(w, s_cv[lt_field<VB>(vw, j)], acc[j]);
      }
    };
    // two row buffers in turn: the prefetch needs no register copies
    for (int st = wave; st < steps; st += 2 * W) {
      load(st + W, nxt);  // unconditional: the prefetch has no branch
      step(cur, st);
      if (st + W >= steps) break;
      load(st + 2 * W, cur);
      step(nxt, st + W);
    }
  }

  // merge the lanes: scale to the wavefront's maximum, fold lanes l, l^16,
  // l^32, l^48 by two transposing swaps, then the rest through LDS
  float mw = m;
  mw = fmaxf(mw, xor_lane_f32<1>(mw));
  mw = fmaxf(mw, xor_lane_f32<2>(mw));
  mw = fmaxf(mw, xor_lane_f32<4>(mw));
  mw = fmaxf(mw, xor_lane_f32<8>(mw));
  mw = fmaxf(mw, xor_lane_f32<16>(mw));
  mw = fmaxf(mw, xor_lane_f32<32>(mw));
  const float f = exp2f(m - mw);  // 1 where no lane saw a token (then l and acc are 0)
  float lw = part ? 0.f : l * f;  // a token's sum is held by all of its lanes
  lw += xor_lane_f32<1>(lw);
  lw += xor_lane_f32<2>(lw);
  lw += xor_lane_f32<4>(lw);
  lw += xor_lane_f32<8>(lw);
  lw += xor_lane_f32<16>(lw);
  lw += xor_lane_f32<32>(lw);
  float r1[H / 2];
#pragma unroll
  for (int i = 0; i < H / 2; ++i) {
    // lanes below 32 end with coordinate i, the others with i + H/2
    const auto p = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, acc[i] * f),
                                                    __builtin_bit_cast(uint32_t, acc[i + H / 2] * f),
                                                    false, false);
    r1[i] = swap_sum(p);
  }
#pragma unroll
  for (int i = 0; i < S::R; ++i) {
    // rows 0 and 2 end with r1[i], rows 1 and 3 with r1[i + R]
    const auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, r1[i]),
                                                    __builtin_bit_cast(uint32_t, r1[i + S::R]),
                                                    false, false);
    s_red[wave][lane][i] = swap_sum(p);
  }
  if (lane == 0) {
    s_ml[wave][0] = mw;
    s_ml[wave][1] = lw;
  }
  __syncthreads();
  // coordinate c: part c / H, index i within it, held by the 16 / P lanes of
  // that part in row (i / (H/2), i % (H/2) / R) at slot i % R
  for (int c = tid; c < D; c += NT) {
    const int pc = c / H, i = c - pc * H;
    const int b5 = i / (H / 2), i2 = i - b5 * (H / 2), b4 = i2 / S::R, k = i2 - b4 * S::R;
    const int l0 = 32 * b5 + 16 * b4 + pc;
    float mx = s_ml[0][0];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, s_ml[w][0]);
    float A = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < 16 / P; ++u) sum += s_red[w][l0 + P * u][k];
      const float fw = exp2f(s_ml[w][0] - mx);
      A += sum * fw;
      L += s_ml[w][1] * fw;
    }
    const size_t slot = ((size_t)b * a.n_q_heads + g) * a.splits + s;
    a.pacc[slot * D + c] = A;
    if (c == 0) {
      a.pml[slot * 2] = mx;
      a.pml[slot * 2 + 1] = L;
    }
  }
}

// Grid (n_q_heads, batch), kDCombineThreads threads: merge the splits by
// log-sum-exp, then out_i = sum_j m_V[j][i] a_j / d (fp64 sums; several
// threads per output coordinate sum consecutive stretches of j, and one adds
// their partial sums in order), or for Walsh-Hadamard codecs
// out = sigma_V (.) H a / d by butterflies. Every global read that does not depend on
// another (the thread's stretch of m_V, a group of splits' partials) is
// issued before the first is used.
constexpr int kDCombineThreads = 512;
constexpr int kDMReg = 32;  // rotation entries a thread holds in registers
constexpr int kDSplitGroup = 8;  // splits whose partials are read at once
__global__ __launch_bounds__(kDCombineThreads) void dense_combine_kernel(DenseAttendArgs a) {
  constexpr int kParts = kDCombineThreads / 32;  // at most, for d = 32
  __shared__ float s_a[kMaxDim];
  __shared__ double s_part[kParts * 32];
  const int tid = threadIdx.x, h = blockIdx.x, b = blockIdx.y, d = a.dim;
  const int parts = kDCombineThreads / d;  // d <= 256: at least 2
  const bool rot = tid < parts * d;
  const int i = tid % d, part = tid / d;
  const int j0 = part * d / parts, j1 = (part + 1) * d / parts;
  double mreg[kDMReg];
#pragma unroll
  for (int k = 0; k < kDMReg; ++k)
    mreg[k] = !a.wht && rot && j0 + k < j1 ? a.m_v[(size_t)(j0 + k) * d + i] : 0.0;

  if (tid < d) {
    const size_t slot0 = ((size_t)b * a.n_q_heads + h) * a.splits;
    float mx = -INFINITY, L = 0.f, A = 0.f;
    for (int s0 = 0; s0 < a.splits; s0 += kDSplitGroup) {
      float pm[kDSplitGroup], pl[kDSplitGroup], pa[kDSplitGroup];
#pragma unroll
      for (int k = 0; k < kDSplitGroup; ++k) {
        const bool in = s0 + k < a.splits;
        const size_t sl = slot0 + (in ? s0 + k : 0);
        pm[k] = in ? a.pml[sl * 2] : -INFINITY;
        pl[k] = in ? a.pml[sl * 2 + 1] : 0.f;
        pa[k] = in ? a.pacc[sl * d + tid] : 0.f;
      }
      float nm = mx;
#pragma unroll
      for (int k = 0; k < kDSplitGroup; ++k) nm = fmaxf(nm, pm[k]);
      const float al = exp2f(mx - nm);  // 0 on the first group (split maxima are finite)
      L *= al;
      A *= al;
#pragma unroll
      for (int k = 0; k < kDSplitGroup; ++k) {
        const float f = exp2f(pm[k] - nm);
        L += pl[k] * f;
        A += pa[k] * f;
      }
      mx = nm;
    }
    s_a[tid] = L > 0.f ? A / L : 0.f;  // no visible row: a zero output
  }
  __syncthreads();
  if (a.wht) {
    // m = H diag(sigma): out_j = sigma_j (H a)_j / d (d = 64 E, E in {1, 2, 4};
    // H_ij = (-1)^popcount(i & j)). Wavefront 0 holds coordinates E lane + e
    // in registers: butterflies over the bits of e within a lane, then over
    // the bits of the lane by lane exchanges.
    if (tid < 64) {
      const int E = d / 64, lane = tid;
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = e < E ? s_a[E * lane + e] : 0.f;
      auto bfly = [](float& x, float& y) {
        const float t = x;
        x = t + y;
        y = t - y;
      };
      if (E >= 2) {
        bfly(u[0], u[1]);
        bfly(u[2], u[3]);
      }
      if (E == 4) {
        bfly(u[0], u[2]);
        bfly(u[1], u[3]);
      }
      sfor_d<6>([&](auto MI) {
        constexpr int m = 1 << MI;
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = xor_lane_f32<m>(u[e]);
          u[e] = upper ? (p - u[e]) : (u[e] + p);
        }
      });
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (e < E) {
          const int jj = E * lane + e;
          const float v = u[e] / (float)d;
          a.out[((size_t)b * a.n_q_heads + h) * d + jj] =
              ((a.wht_v.bits[jj >> 5] >> (jj & 31)) & 1u) ? -v : v;
        }
      }
    }
    return;
  }
  if (rot) {
    double o = 0.0;
#pragma unroll
    for (int k = 0; k < kDMReg; ++k)
      if (j0 + k < j1) o += mreg[k] * (double)s_a[j0 + k];
    for (int j = j0 + kDMReg; j < j1; ++j) o += a.m_v[(size_t)j * d + i] * (double)s_a[j];
    s_part[part * d + i] = o;
  }
  __syncthreads();
  for (int i = tid; i < d; i += kDCombineThreads) {
    double o = 0.0;
    for (int p = 0; p < parts; ++p) o += s_part[p * d + i];
    a.out[((size_t)b * a.n_q_heads + h) * d + i] = (float)(o / d);
  }
}

}  // namespace

template <int D>
hipError_t launch_encode_lds(const DenseEncodeArgs& a, long long nvec, hipStream_t stream) {
  const long long npass = (nvec + kEV - 1) / kEV;
  // as many workgroups as fit at once: 256 CUs, each with 160 KB of LDS
  const long long fit = 256LL * (long long)(kDenseLdsFull / EncLds<D>::BYTES);
  const int blocks = (int)(npass < fit ? npass : fit);
  hipLaunchKernelGGL(dense_encode_lds_kernel<D>, dim3(blocks), dim3(EncLds<D>::THREADS),
                     EncLds<D>::BYTES, stream, a);
  return hipGetLastError();
}

hipError_t launch_encode_dense(const DenseEncodeArgs& a, hipStream_t stream) {
  const long long nvec = (long long)a.n_tok * a.n_head;
  if (nvec <= 0) return hipSuccess;
  if (a.dim == 96) return launch_encode_lds<96>(a, nvec, stream);
  if (a.dim == 64) return launch_encode_lds<64>(a, nvec, stream);
  if (a.dim == 32) return launch_encode_lds<32>(a, nvec, stream);
  const long long per_block = (long long)kDW * kVPW;
  const long long blocks = (nvec + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dense_encode_kernel, dim3((unsigned)blocks), dim3(64 * kDW), 0, stream, a);
  return hipGetLastError();
}

constexpr size_t kDenseLdsLimit = kDenseLdsFull;

template <int GM, int EM, bool EX>
hipError_t allow_dense_lds() {
  return hipFuncSetAttribute((const void*)&dense_split_kernel<GM, EM, EX>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDenseLdsLimit);
}

template <int GM, int EM, bool EX>
hipError_t launch_dense_split(DenseAttendArgs a, int batch, hipStream_t stream) {
  constexpr int kMaxWaves = GM * EM > 8 ? 8 : 16;
  const size_t kLdsLimit = a.lds_limit < (int)kDenseLdsLimit ? (size_t)a.lds_limit
                                                               : kDenseLdsLimit;
  const int G = a.group, d = a.dim;
  const int kw = d * a.k_bits / 32, vw = d * a.v_bits / 32;
  a.rows_words = kDTile * (kw > vw ? kw : vw);
  int stride = a.rows_words + kDTile * G;
  if (stride < G * d) stride = G * d;
  a.wave_stride = (stride + 3) & ~3;
  auto bytes = [&](int nw) {
    return sizeof(float) * ((size_t)G * d + 512 + ((nw * 2 * G + 3) & ~3) +
                            (size_t)nw * a.wave_stride);
  };
  int nw = kMaxWaves;
  while (nw > 1 && bytes(nw) > kLdsLimit) nw >>= 1;
  const size_t lds = bytes(nw);
  if (lds > kLdsLimit) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dense_split_kernel<GM, EM, EX>), dim3(a.splits, a.n_kv_heads, batch),
                     dim3(64 * nw), lds, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t allow_encode_lds() {
  static_assert(EncLds<D>::BYTES <= kDenseLdsFull, "encode LDS");
  return hipFuncSetAttribute((const void*)&dense_encode_lds_kernel<D>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)EncLds<D>::BYTES);
}

hipError_t prepare_attend_dense() {
  const hipError_t e[] = {allow_encode_lds<96>(), allow_encode_lds<64>(), allow_encode_lds<32>(),allow_dense_lds<1, 2, true>(),   allow_dense_lds<1, 4, true>(),
                          allow_dense_lds<4, 2, true>(),   allow_dense_lds<4, 4, true>(),
                          allow_dense_lds<4, 2, false>(),  allow_dense_lds<4, 4, false>(),
                          allow_dense_lds<16, 2, false>(), allow_dense_lds<16, 4, false>()};
  for (const hipError_t x : e)
    if (x != hipSuccess) return x;
  return hipSuccess;
}

template <int D, int KB, int VB>
hipError_t launch_dense_lt(const DenseAttendArgs& a, int batch, hipStream_t stream) {
  constexpr int W = lt_waves<D>();
  hipLaunchKernelGGL((dense_lt_kernel<D, KB, VB, W>), dim3(a.splits, a.n_kv_heads, batch),
                     dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}
using DenseLaunch = hipError_t (*)(const DenseAttendArgs&, int, hipStream_t);
template <int D, int KB>
DenseLaunch lt_for_v(int vb) {
  switch (vb) {
    case 2: return &launch_dense_lt<D, KB, 2>;
    case 3: return &launch_dense_lt<D, KB, 3>;
    case 4: return &launch_dense_lt<D, KB, 4>;
    default: return nullptr;
  }
}
template <int D>
DenseLaunch lt_for_bits(int kb, int vb) {
  switch (kb) {
    case 2: return lt_for_v<D, 2>(vb);
    case 3: return lt_for_v<D, 3>(vb);
    case 4: return lt_for_v<D, 4>(vb);
    case 8: return lt_for_v<D, 8>(vb);
    default: return nullptr;
  }
}
// The register-held kernel's instances: one query head per KV head, head dim
// 64, 96, 128 or 256, K 2/3/4/8 and V 2/3/4 bits; the rotation dense or, at
// powers of 2, the Walsh-Hadamard codecs' H diag(sigma).
DenseLaunch find_lt(int dim, int k_bits, int v_bits, int group) {
  if (group != 1) return nullptr;
  if (dim == 64) return lt_for_bits<64>(k_bits, v_bits);
  if (dim == 96) return lt_for_bits<96>(k_bits, v_bits);
  if (dim == 128) return lt_for_bits<128>(k_bits, v_bits);
  if (dim == 256) return lt_for_bits<256>(k_bits, v_bits);
  return nullptr;
}
DenseLaunch find_dense_lt(const DenseAttendArgs& a) {
  return find_lt(a.dim, a.k_bits, a.v_bits, a.group);
}

hipError_t launch_attend_dense(const DenseAttendArgs& a, int batch, hipStream_t stream) {
  if (a.group < 1 || a.group > kDMaxG || a.dim % 32 || a.dim > kMaxDim) return hipErrorInvalidValue;
  hipError_t err;
  const bool wide = a.dim > 128;
  if (const DenseLaunch lt = find_dense_lt(a))
    err = lt(a, batch, stream);
  else if (a.group == 1)  // exact group sizes: the head loops fold away
    err = wide ? launch_dense_split<1, 4, true>(a, batch, stream)
               : launch_dense_split<1, 2, true>(a, batch, stream);
  else if (a.group == 4)
    err = wide ? launch_dense_split<4, 4, true>(a, batch, stream)
               : launch_dense_split<4, 2, true>(a, batch, stream);
  else if (a.group < 4)
    err = wide ? launch_dense_split<4, 4, false>(a, batch, stream)
               : launch_dense_split<4, 2, false>(a, batch, stream);
  else
    err = wide ? launch_dense_split<16, 4, false>(a, batch, stream)
               : launch_dense_split<16, 2, false>(a, batch, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dense_combine_kernel, dim3(a.n_q_heads, batch), dim3(kDCombineThreads), 0,
                     stream, a);
  return hipGetLastError();
}

float dense_qscale(float scale, int dim) { return scale * kDLog2e / (float)dim; }

bool dense_lt_supported(int dim, int k_bits, int v_bits, int group) {
  return find_lt(dim, k_bits, v_bits, group) != nullptr;
}

}  // namespace tq

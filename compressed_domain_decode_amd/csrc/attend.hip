// attend.hip -- decode attention straight from the packed TurboQuant cache.
//
// What is computed (the fused compressed-domain decode of the X post on
// TurboQuant in mlx-swift-lm and of the turboquant-mlx KV-cache guide, "Fused
// decode+attend"): for query head h of sequence b, over cached tokens
// t < len_b of KV head g = h / G,
//   s_t   = scale * <q, k_hat_t>,   k_hat_t = (nK_t / d) sigma_K (.) (H cK[idxK_t])
//   out   = sum_t softmax(s)_t v_hat_t
// K is never expanded: with q~ = H (sigma_K (.) q), <q, k_hat_t> equals
// (nK_t / d) <q~, cK[idxK_t]>, so scores are taken in the rotated basis; V is
// accumulated in the rotated basis as nV_t cV[idxV_t] and one inverse
// transform per head, out = (1/d) sigma_V (.) H a, finishes it.
//
// Three kernels (all on the caller's stream):
//  1. rotate_q: q^ = (scale * log2 e / d) H (sigma_K (.) q) in fp64, stored fp32.
//     Folding log2 e lets the softmax use exp2 directly.
//  2. attend_split (the hot one): grid (splits, kv heads, batch), 4 wavefronts
//     per workgroup, each wavefront streams 64-token tiles of the workgroup's
//     context range with its own online-softmax state:
//       K phase, one lane per token: the lane reads its token's packed K row,
//       looks each code up in an LDS copy of the K codebook and accumulates G
//       scores; q^ is wavefront-uniform and comes through scalar loads, so the
//       inner step is one table lookup and G FMAs per coordinate.
//       softmax: wavefront max per head (cross-lane butterfly), rescale, p.
//       V phase, lanes over coordinates: per token, the G weights p * nV_t are
//       broadcast from LDS and each lane decodes its E = d/64 codes of that
//       token's V row (staged in LDS), accumulating G x E fp32 outputs.
//     The four wavefronts merge (m, l, acc) through LDS and write one partial
//     per (batch, query head, split).
//  3. combine: log-sum-exp merge of the split partials, normalisation, inverse
//     Walsh-Hadamard transform (cross-lane butterfly), sign flip, 1/d.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "kernels.hpp"

namespace tq {

namespace {

constexpr int kTile = 64;            // tokens per wavefront tile
constexpr int kWaves = 4;            // wavefronts per workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Make this wavefront's LDS writes visible to its other lanes before reading.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- 1. rotate q

template <int D>
__global__ __launch_bounds__(64) void rotate_q_kernel(const __half* __restrict__ q,
                                                      float* __restrict__ qhat, float qscale,
                                                      SignArg sign) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const long long row = (long long)blockIdx.y * gridDim.x + blockIdx.x;  // b * Hq + h
  const __half* qv = q + row * D + E * lane;
  double u[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * lane + e;
    const double x = (double)__half2float(qv[e]);
    u[e] = ((sign.bits[j >> 5] >> (j & 31)) & 1u) ? -x : x;
  }
#pragma unroll
  for (int hs = 1; hs < E; hs <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & hs) == 0) {
        const double a = u[e], b = u[e + hs];
        u[e] = a + b;
        u[e + hs] = a - b;
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
#pragma unroll
  for (int e = 0; e < E; ++e) qhat[row * D + E * lane + e] = (float)(u[e] * (double)qscale);
}

// ---------------------------------------------------------------- 2. split attend

// Code j (0..31) of a 32-code group held in BITS consecutive dwords w[].
template <int BITS>
__device__ inline uint32_t code_at(const uint32_t* w, int j) {
  const int bit = BITS * j;
  const int lo = bit >> 5, sh = bit & 31;
  if (sh + BITS <= 32) return (w[lo] >> sh) & ((1u << BITS) - 1u);
  return __builtin_amdgcn_alignbit(w[lo + 1], w[lo], sh) & ((1u << BITS) - 1u);
}

template <int D, int BK, int BV, int G>
__global__ __launch_bounds__(256, 2) void attend_split_kernel(
    const float* __restrict__ qhat, const uint8_t* __restrict__ k_codes,
    const float* __restrict__ k_norms, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ v_norms, const int32_t* __restrict__ lengths, int n_kv_heads,
    int max_ctx, int max_len, int tokens_per_split, float* __restrict__ part_acc,
    float* __restrict__ part_ml, AttendTables tabs) {
  constexpr int E = D / 64;                 // V coordinates per lane
  constexpr int RKW = D * BK / 32;          // dwords per K row
  constexpr int RVW = D * BV / 32;          // dwords per V row
  constexpr int VSTR = RVW + 1;             // LDS stride of a staged V row
  constexpr int NK = 1 << BK, NV = 1 << BV;
  constexpr int VCH = E * BV;               // V bits per lane per token

  __shared__ float s_ck[NK];
  __shared__ float s_cv[NV];
  __shared__ uint32_t s_vrow[kWaves][kTile * VSTR];
  __shared__ float s_w[kWaves][kTile * G];
  __shared__ float s_merge[kWaves * D];
  __shared__ float s_ml[kWaves][2 * G];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int len = min(lengths[b], max_len);   // never read past the host bound
  const int t_begin = split * tokens_per_split;
  if (t_begin >= len) return;  // whole workgroup: this split is past the sequence end
  const int t_end = min(len, t_begin + tokens_per_split);

  for (int i = threadIdx.x; i < NK; i += blockDim.x) s_ck[i] = tabs.k_centroids[i];
  for (int i = threadIdx.x; i < NV; i += blockDim.x) s_cv[i] = tabs.v_centroids[i];
  __syncthreads();

  const int n_q_heads = n_kv_heads * G;
  const float* __restrict__ qh = qhat + ((long long)b * n_q_heads + (long long)g * G) * D;
  const long long kvrow0 = ((long long)b * n_kv_heads + g) * max_ctx;
  const uint32_t* __restrict__ kbase = (const uint32_t*)k_codes + kvrow0 * RKW;
  const uint32_t* __restrict__ vbase = (const uint32_t*)v_codes + kvrow0 * RVW;

  float m_run[G], l_lane[G], acc[G][E];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  // this lane's V bits within a row: [VCH*lane, VCH*lane + VCH)
  const int vbit0 = VCH * lane;
  const int vdw = vbit0 >> 5, vsh = vbit0 & 31;
  uint32_t* my_vrow = s_vrow[wave];
  float* my_w = s_w[wave];

  for (int tile = t_begin + wave * kTile; tile < t_end; tile += kWaves * kTile) {
    const int t = tile + lane;
    const bool valid = t < t_end;
    const int ntok = min(kTile, t_end - tile);

    // ---- K phase: one lane per token
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = 0.f;
    float nv = 0.f;
    if (valid) {
      const uint32_t* krow = kbase + (long long)t * RKW;
#pragma unroll
      for (int grp = 0; grp < D / 32; ++grp) {
        uint32_t w[BK];
#pragma unroll
        for (int i = 0; i < BK; ++i) w[i] = krow[grp * BK + i];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float c = s_ck[code_at<BK>(w, j)];
#pragma unroll
          for (int h = 0; h < G; ++h) sc[h] = fmaf(qh[h * D + grp * 32 + j], c, sc[h]);
        }
      }
      const float nk = k_norms[kvrow0 + t];
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] *= nk;
      nv = v_norms[kvrow0 + t];
      const uint32_t* vrow = vbase + (long long)t * RVW;
#pragma unroll
      for (int i = 0; i < RVW; ++i) my_vrow[lane * VSTR + i] = vrow[i];
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = -INFINITY;
    }

    // ---- online softmax (base 2)
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mt = wave_max(sc[h]);
      const float mn = fmaxf(m_run[h], mt);
      alpha[h] = exp2f(m_run[h] - mn);      // m_run = -inf -> 0
      const float p = valid ? exp2f(sc[h] - mn) : 0.f;
      l_lane[h] = l_lane[h] * alpha[h] + p;
      m_run[h] = mn;
      my_w[lane * G + h] = p * nv;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha[h];
    }
    wave_lds_sync();

    // ---- V phase: lanes over coordinates
    for (int tt = 0; tt < ntok; ++tt) {
      const uint32_t* vr = my_vrow + tt * VSTR;
      uint32_t bits;
      if (vsh + VCH <= 32) {
        bits = vr[vdw] >> vsh;
      } else {
        bits = __builtin_amdgcn_alignbit(vr[vdw + 1], vr[vdw], vsh);
      }
      float wt[G];
#pragma unroll
      for (int h = 0; h < G; ++h) wt[h] = my_w[tt * G + h];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float c = s_cv[(bits >> (BV * e)) & (NV - 1)];
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h][e] = fmaf(wt[h], c, acc[h][e]);
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four wavefronts and write this split's partials
  float l_w[G];
#pragma unroll
  for (int h = 0; h < G; ++h) l_w[h] = wave_sum(l_lane[h]);
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_ml[wave][2 * h] = m_run[h];
      s_ml[wave][2 * h + 1] = l_w[h];
    }
  }
  const int S = gridDim.x;
  for (int h = 0; h < G; ++h) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) s_merge[wave * D + E * lane + e] = acc[h][e];
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[w][2 * h]);
    const long long prow = ((long long)b * n_q_heads + (long long)g * G + h) * S + split;
    for (int j = threadIdx.x; j < D; j += blockDim.x) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_ml[w][2 * h];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        a = fmaf(f, s_merge[w * D + j], a);
      }
      part_acc[prow * D + j] = a;
    }
    if (threadIdx.x == 0) {
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = s_ml[w][2 * h];
        if (mw != -INFINITY) L = fmaf(exp2f(mw - M), s_ml[w][2 * h + 1], L);
      }
      part_ml[prow * 2] = M;
      part_ml[prow * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- 3. combine

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ part_acc,
                                                     const float* __restrict__ part_ml,
                                                     const int32_t* __restrict__ lengths,
                                                     int max_len, int n_q_heads, int splits,
                                                     int tokens_per_split, float* __restrict__ out,
                                                     SignArg sign) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x;
  const int h = blockIdx.x, b = blockIdx.y;
  const long long row = (long long)b * n_q_heads + h;
  const int len = min(lengths[b], max_len);
  float a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
  if (len > 0) {
    const int ns = min(splits, (len + tokens_per_split - 1) / tokens_per_split);
    const float* ml = part_ml + row * splits * 2;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float f = exp2f(ml[2 * s] - M);
      L = fmaf(f, ml[2 * s + 1], L);
      const float* pa = part_acc + (row * splits + s) * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = fmaf(f, pa[e], a[e]);
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] *= inv;
  }
  // inverse rotation: out = (1/d) sigma_V (.) H a
#pragma unroll
  for (int hs = 1; hs < E; hs <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & hs) == 0) {
        const float x = a[e], y = a[e + hs];
        a[e] = x + y;
        a[e + hs] = x - y;
      }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float p = __shfl_xor(a[e], m);
      a[e] = upper ? (p - a[e]) : (a[e] + p);
    }
  }
  const float invd = 1.f / (float)D;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = E * lane + e;
    const float v = a[e] * invd;
    out[row * D + j] = ((sign.bits[j >> 5] >> (j & 31)) & 1u) ? -v : v;
  }
}

// ---------------------------------------------------------------- dispatch

template <int D, int BK, int BV, int G>
hipError_t launch_split(const AttendPlan& plan, int batch, int n_kv_heads, const float* qhat,
                        const uint8_t* kc, const float* kn, const uint8_t* vc, const float* vn,
                        const int32_t* lengths, int max_ctx, int max_len, float* pacc,
                        float* pml, const AttendTables& tabs, hipStream_t stream) {
  hipLaunchKernelGGL((attend_split_kernel<D, BK, BV, G>),
                     dim3(plan.splits, n_kv_heads, batch), dim3(64 * kWaves), 0, stream, qhat,
                     kc, kn, vc, vn, lengths, n_kv_heads, max_ctx, max_len,
                     plan.tokens_per_split, pacc, pml, tabs);
  return hipGetLastError();
}

typedef hipError_t (*SplitFn)(const AttendPlan&, int, int, const float*, const uint8_t*,
                              const float*, const uint8_t*, const float*, const int32_t*, int,
                              int, float*, float*, const AttendTables&, hipStream_t);

struct SplitEntry {
  int d, bk, bv, g;
  SplitFn fn;
};

#define TQ_SPLIT(D, BK, BV, G) {D, BK, BV, G, &launch_split<D, BK, BV, G>}
const SplitEntry kSplitTable[] = {
    // head_dim 64
    TQ_SPLIT(64, 4, 4, 2), TQ_SPLIT(64, 3, 3, 8), TQ_SPLIT(64, 4, 4, 1), TQ_SPLIT(64, 3, 3, 4),
    TQ_SPLIT(64, 8, 3, 4), TQ_SPLIT(64, 2, 2, 2), TQ_SPLIT(64, 1, 1, 2), TQ_SPLIT(64, 5, 7, 2),
    TQ_SPLIT(64, 6, 6, 16), TQ_SPLIT(64, 8, 8, 1),
    // head_dim 128
    TQ_SPLIT(128, 4, 2, 3), TQ_SPLIT(128, 8, 3, 4), TQ_SPLIT(128, 3, 3, 4), TQ_SPLIT(128, 4, 4, 4),
    TQ_SPLIT(128, 4, 3, 4), TQ_SPLIT(128, 2, 2, 4), TQ_SPLIT(128, 8, 4, 4), TQ_SPLIT(128, 4, 4, 8),
    TQ_SPLIT(128, 8, 3, 8), TQ_SPLIT(128, 4, 2, 1), TQ_SPLIT(128, 3, 3, 2), TQ_SPLIT(128, 8, 8, 2),
    TQ_SPLIT(128, 1, 1, 4), TQ_SPLIT(128, 7, 5, 6),
    // head_dim 256
    TQ_SPLIT(256, 4, 4, 4), TQ_SPLIT(256, 8, 3, 4), TQ_SPLIT(256, 3, 3, 2), TQ_SPLIT(256, 8, 4, 1),
    TQ_SPLIT(256, 2, 2, 8),
};
#undef TQ_SPLIT

const SplitEntry* find_split(int d, int bk, int bv, int g) {
  for (const SplitEntry& e : kSplitTable)
    if (e.d == d && e.bk == bk && e.bv == bv && e.g == g) return &e;
  return nullptr;
}

}  // namespace

AttendPlan plan_attend(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len) {
  AttendPlan p{};
  // Enough workgroups to give each of the 256 CUs several to interleave, but
  // at least one full round of tiles (4 wavefronts x 64 tokens) per workgroup.
  const long long units = (long long)batch * n_kv_heads;
  const long long target_wgs = 2048;
  long long tps = ((long long)max_len * units + target_wgs - 1) / target_wgs;
  const long long round = (long long)kWaves * kTile;
  tps = ((tps + round - 1) / round) * round;
  if (tps < round) tps = round;
  p.tokens_per_split = (int)tps;
  p.splits = (int)((max_len + tps - 1) / tps);
  if (p.splits < 1) p.splits = 1;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.qhat_bytes = align((size_t)batch * n_q_heads * dim * sizeof(float));
  p.part_acc_bytes = align((size_t)batch * n_q_heads * p.splits * dim * sizeof(float));
  p.part_ml_bytes = align((size_t)batch * n_q_heads * p.splits * 2 * sizeof(float));
  p.total_bytes = p.qhat_bytes + p.part_acc_bytes + p.part_ml_bytes;
  return p;
}

bool attend_supported(int dim, int k_bits, int v_bits, int group) {
  return find_split(dim, k_bits, v_bits, group) != nullptr;
}

hipError_t launch_attend(int dim, int k_bits, int v_bits, int batch, int n_q_heads,
                         int n_kv_heads, const void* q, const SignArg& k_sign,
                         const SignArg& v_sign, const AttendTables& tabs,
                         const uint8_t* k_codes, const float* k_norms,
                         const uint8_t* v_codes, const float* v_norms, int max_ctx,
                         const int32_t* lengths, int max_len, float scale, float* out,
                         void* workspace, const AttendPlan& plan, hipEvent_t ev_before,
                         hipEvent_t ev_after, hipStream_t stream) {
  const int group = n_q_heads / n_kv_heads;
  const SplitEntry* ent = find_split(dim, k_bits, v_bits, group);
  if (!ent) return hipErrorInvalidValue;
  char* ws = (char*)workspace;
  float* qhat = (float*)ws;
  float* pacc = (float*)(ws + plan.qhat_bytes);
  float* pml = (float*)(ws + plan.qhat_bytes + plan.part_acc_bytes);
  const float qscale = scale * kLog2e / (float)dim;
  hipError_t err;
  switch (dim) {
    case 64:
      hipLaunchKernelGGL(rotate_q_kernel<64>, dim3(n_q_heads, batch), dim3(64), 0, stream,
                         (const __half*)q, qhat, qscale, k_sign);
      break;
    case 128:
      hipLaunchKernelGGL(rotate_q_kernel<128>, dim3(n_q_heads, batch), dim3(64), 0, stream,
                         (const __half*)q, qhat, qscale, k_sign);
      break;
    case 256:
      hipLaunchKernelGGL(rotate_q_kernel<256>, dim3(n_q_heads, batch), dim3(64), 0, stream,
                         (const __half*)q, qhat, qscale, k_sign);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ev_before && (err = hipEventRecord(ev_before, stream)) != hipSuccess) return err;
  err = ent->fn(plan, batch, n_kv_heads, qhat, k_codes, k_norms, v_codes, v_norms, lengths,
                max_ctx, max_len, pacc, pml, tabs, stream);
  if (err != hipSuccess) return err;
  if (ev_after && (err = hipEventRecord(ev_after, stream)) != hipSuccess) return err;
  switch (dim) {
    case 64:
      hipLaunchKernelGGL(combine_kernel<64>, dim3(n_q_heads, batch), dim3(64), 0, stream, pacc,
                         pml, lengths, max_len, n_q_heads, plan.splits, plan.tokens_per_split, out,
                         v_sign);
      break;
    case 128:
      hipLaunchKernelGGL(combine_kernel<128>, dim3(n_q_heads, batch), dim3(64), 0, stream, pacc,
                         pml, lengths, max_len, n_q_heads, plan.splits, plan.tokens_per_split, out,
                         v_sign);
      break;
    case 256:
      hipLaunchKernelGGL(combine_kernel<256>, dim3(n_q_heads, batch), dim3(64), 0, stream, pacc,
                         pml, lengths, max_len, n_q_heads, plan.splits, plan.tokens_per_split, out,
                         v_sign);
      break;
  }
  return hipGetLastError();
}

}  // namespace tq

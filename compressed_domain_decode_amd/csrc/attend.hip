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
// Two kernels on the caller's stream:
//
// 1. attend_split (the hot one). Grid (splits, kv heads, batch); each
//    workgroup owns one context range of one (sequence, KV head) and all G
//    query heads that read it; its wavefronts stream 64-token tiles.
//    Per tile, both contractions run on the fp32 matrix cores with the
//    v_mfma_f32_4x4x1 16-block instruction, while the VALU and LDS only
//    unpack codes and look centroids up:
//      scores  S[h][t] = sum_j q^[h][j] * cK[idxK[t][j]]
//              lane t holds token t's packed K row; for each coordinate j the
//              centroid it looks up is the B operand, and the A operand is
//              q^[h][j] broadcast from one 4-lane block (CBSZ/ABID), so one
//              VGPR carries q^ for 16 coordinates and lane t ends with the 4
//              heads' scores of token t.
//      softmax online softmax in base 2 (log2 e folded into q^), per head
//              running max from a cross-lane reduction; weights p * nV_t.
//      values  A[h][j] += sum_t w[h][t] * cV[idxV[t][j]]
//              lanes own coordinates. The lane holding token t stages t's
//              packed V row in LDS; per token each lane reads the two dwords
//              that hold its code(s), funnel-shifts them and looks the
//              centroid up. The 4 heads' weights are broadcast the same way
//              as q^.
//    The online softmax moves its running maximum only when a tile's
//    maximum exceeds it by more than 2^8, so the rescale is rare.
//    Centroid tables live in LDS replicated once per bank (a 256-byte row
//    per code: 32 copies of an 8-byte code-pair entry or 64 copies of a
//    4-byte entry), so a lookup is conflict-free whatever the codes; codes of
//    <= 3 bits are looked up two coordinates at a time. The query rotation q^ = (scale log2 e / d)
//    H (sigma_K (.) q) is done by every wavefront in its prologue.
//    The wavefronts merge (max, sum, accumulator) through LDS and write one
//    partial per (sequence, query head, split).
// 2. combine: log-sum-exp merge of the split partials, normalisation, inverse
//    Walsh-Hadamard transform (cross-lane butterfly), sign flip, 1/d.
#include <hip/hip_fp16.h>
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>
#include <utility>

#include "kernels.hpp"

namespace tq {

namespace {

constexpr int kTile = 64;  // tokens per wavefront tile (one per lane)
constexpr float kLog2e = 1.4426950408889634f;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

template <int... Is, class F>
__device__ __forceinline__ void sfor_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(std::make_integer_sequence<int, N>{}, f);
}

// D[v] += A[4*ABID + v] * B[lane] on a 4x4x1 block grid, the A operand of
// block ABID broadcast to all 16 blocks: lane l accumulates column l % 4 of
// its block, i.e. lane l gets A_bcast[v] * B[l] for v = 0..3.
template <int ABID>
__device__ __forceinline__ v4f mfma_bcast(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 4, ABID, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over the wavefront, returned in every lane: DPP within each 16-lane
// row (quad swaps, half-row and row mirrors), then the four row results.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
// Maximum over the wavefront of finite or -inf scores, returned in every lane:
// the same DPP pattern on an order-preserving integer key (the bits, with the
// magnitude bits flipped for negative values), so each step is one fused
// v_max_i32_dpp with no NaN quieting, and the maximum is exact.
__device__ __forceinline__ float wave_max_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  int k = b ^ ((b >> 31) & 0x7FFFFFFF);
  constexpr int kLow = (int)0x80000000;  // identity of the max for the DPP's inactive sources
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x141, 0xF, 0xF, false));  // row_half_mirror
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x140, 0xF, 0xF, false));  // row_mirror
  const int r = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
                    max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
  return __builtin_bit_cast(float, r ^ ((r >> 31) & 0x7FFFFFFF));
}
// Sum over the wavefront, returned in every lane (same DPP pattern).
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Order this wavefront's LDS writes before its following LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The F-bit field starting at bit O of the register row w (O a compile-time
// bit offset), moved so that it starts at bit 8; bits above it are garbage.
// The next register is read only when the field straddles into it.
template <int O, int F, int NW>
__device__ __forceinline__ uint32_t field_at8(const uint32_t (&w)[NW]) {
  constexpr int wi = O >> 5, sh = O & 31;
  if constexpr (sh + F > 32) {
    static_assert(wi + 1 < NW && sh > 8, "straddling field");
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh - 8);
  } else if constexpr (sh >= 8) {
    return w[wi] >> (sh - 8);
  } else {
    return w[wi] << (8 - sh);
  }
}

// Centroid tables live in LDS as one 256-byte row per code (or code pair):
// 64 copies of a 4-byte centroid, or 32 copies of an 8-byte centroid pair, so
// that every lane reads its own copy and a lookup never has a bank conflict,
// whatever the codes. A lookup address is (code << 8) | lane_offset.
template <int D_, int BK_, int BV_, int NHG_, int WAVES_>
struct CfgBase {
  static constexpr int D = D_, BK = BK_, BV = BV_, NHG = NHG_, WAVES = WAVES_;
  static constexpr int E = D / 64;                     // coordinates per lane (rotation)
  // BK == 16: raw fp16 keys (PR #232's raw-K turbo0v* schemes), scored in the
  // original basis with no lookup table and no key norm. BK == 32 + m:
  // TurboQuant-Prod keys, m-bit codes plus a D-bit residual sketch and norm.
  static constexpr bool PROD = BK > 32;
  static constexpr int KBITS = PROD ? BK - 32 : BK;    // bits of the key codes
  static constexpr bool KRAW = BK == 16;
  static constexpr bool KPAIR = !KRAW && KBITS <= 3;   // K looked up two coordinates at a time
  static constexpr bool VPAIR = BV <= 3 && D >= 128;   // V likewise
  static constexpr int KF = KPAIR ? 2 * KBITS : KBITS; // bits per K lookup
  static constexpr int SKW = PROD ? D / 32 : 1;        // sketch dwords per K row
  static constexpr int VF = VPAIR ? 2 * BV : BV;       // bits per V lookup
  static constexpr int NKL = KPAIR ? D / 2 : D;        // K lookups per token
  static constexpr int NVS = VPAIR ? D / 128 : D / 64; // V lookups per lane per token
  static constexpr int RKW = D * KBITS / 32;           // dwords per K row
  static constexpr int RVW = D * BV / 32;              // dwords per V row
  // V rows of a tile staged contiguously in LDS (row t at dword 2 + t RVW,
  // 2 dwords of padding on each side): a lane reads the two dwords around its
  // field, which may reach from the dword before the row to the dword after
  // it (a neighbouring row or padding; those bits are masked off).
  static constexpr int VT_BYTES = (1 << VF) * 256;
  static constexpr int KT_BYTES = KRAW ? 0 : (1 << KF) * 256;
  static constexpr int VS_BYTES = (kTile * RVW + 4) * 4;  // per wavefront
  static constexpr int WB_BYTES = kTile * 4 * NHG * 4;  // per wavefront: weights of a tile
  // rotated queries (and for Prod keys their sketch projections)
  static constexpr int QS_BYTES = (PROD ? 2 : 1) * 4 * NHG * D * 4;
  static constexpr int CEN_BYTES = 2 * 256 * 4;         // plain centroid tables while filling
  static constexpr int GATE_BYTES = (WAVES * 4 + 15) / 16 * 16;  // first-tile arrival flags
  static constexpr int MAIN_BYTES =
      VT_BYTES + KT_BYTES + WAVES * (VS_BYTES + WB_BYTES) + QS_BYTES + CEN_BYTES + GATE_BYTES;
  static constexpr int MERGE_BYTES = (WAVES * 4 * NHG * 2 + WAVES * 4 * NHG * D) * 4;
  static constexpr int LDS_BYTES = MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES;
  static constexpr int NACC = (VPAIR ? 2 * NVS : NVS) < 2 ? 2 : (VPAIR ? 2 * NVS : NVS);
};

constexpr int kLdsPerCU = 163840;

// Software-pipeline depths of the tile loop: K lookups per batch, tokens per
// batch of the values phase.
constexpr int kKBatch = 8;
constexpr int kVBatch = 4;

// Rough count of the VGPRs one lane holds through the tile loop: rotated
// queries, norms, value accumulators, weight and softmax state, V field
// positions, the V row being staged, plus the larger of the scores phase (the
// K row, two batches of lookups, four accumulator chains) and the values
// phase (three batches of staged dwords, two of lookups).
template <class B>
constexpr int vgpr_estimate() {
  constexpr int base = B::NHG * B::D / 16 + 2 + B::NACC * B::NHG * 4 + B::NHG * 20 + 2 * B::NVS;
  constexpr int kphase = B::RKW + 2 * kKBatch * (B::KPAIR ? 2 : 1) + 16 * B::NHG;
  constexpr int vphase = 3 * kVBatch * B::NVS * 2 + 2 * kVBatch * B::NVS * (B::VPAIR ? 2 : 1);
  constexpr int prod = B::PROD ? B::D / 32 + 1 + B::NHG * B::D / 16 + 16 * B::NHG : 0;
  return base + prod + (kphase > vphase ? kphase : vphase);
}

// Wavefronts per workgroup: as many as the LDS and the register file allow
// (16, 12, 8 or 4; 128, 168 or 256 VGPRs per lane); the centroid tables are
// shared by all of them.
template <int D, int BK, int BV, int NHG>
constexpr int cfg_waves() {
  using B = CfgBase<D, BK, BV, NHG, 4>;
  constexpr int need = vgpr_estimate<B>() + 24;  // + addresses, temporaries
  if (NHG < 4 && need <= 128 && CfgBase<D, BK, BV, NHG, 16>::LDS_BYTES <= kLdsPerCU) return 16;
  if (NHG < 4 && need <= 168 && CfgBase<D, BK, BV, NHG, 12>::LDS_BYTES <= kLdsPerCU) return 12;
  if (CfgBase<D, BK, BV, NHG, 8>::LDS_BYTES <= kLdsPerCU) return 8;
  return 4;
}
template <int D, int BK, int BV, int NHG>
struct Cfg : CfgBase<D, BK, BV, NHG, cfg_waves<D, BK, BV, NHG>()> {
  using B = CfgBase<D, BK, BV, NHG, 4>;
  static_assert(B::RVW % 2 == 0, "V rows are staged with 8-byte writes");
  static_assert(B::VT_BYTES < 65536, "K table base must fit a DS offset");
  static_assert(CfgBase<D, BK, BV, NHG, 4>::LDS_BYTES <= kLdsPerCU, "LDS budget");
};
// The same kernel with 4 wavefronts, for ranges of at most 4 tiles (short
// contexts): a 16-wavefront workgroup would leave 12 or more without a tile
// yet launch, synchronise and merge them all.
template <int D, int BK, int BV, int NHG>
struct CfgShort : CfgBase<D, BK, BV, NHG, 4> {
  static_assert(Cfg<D, BK, BV, NHG>::WAVES >= 4, "a full configuration exists");
};
constexpr int kShortTiles = 4;  // ranges up to this many tiles use the short workgroup

// One tile's worth of this lane's token: packed K and V rows and the norms.
template <class C>
struct TileRegs {
  uint32_t kw[C::RKW];
  uint32_t vw[C::RVW];
  uint32_t sk[C::SKW];  // Prod keys: sketch bits
  float nk, nv, rn;     // rn: Prod keys' residual norm
};

// TurboQuant-Prod keys: per-row sketch bits [.][Hkv][max_ctx][D/8] and residual
// norms [.][Hkv][max_ctx], the sketch signs sigma_S, and the factor taking the
// sketch projection H(sigma_S (.) H(sigma_K (.) q)) to score units
// (scale log2(e) / d * sqrt(pi/2) / d).
struct ProdArgs {
  const uint8_t* sketch;
  const float* rnorms;
  SignArg sign;
  float uscale;
};

// Rescale threshold of the online softmax (log2 units): the running maximum
// is only moved when a tile's maximum exceeds it by more than this, so
// weights stay below 2^8 and the rescale is rare.
constexpr float kRescaleSlack = 8.f;

// First tiles in flight per workgroup. Wavefronts 0 .. kGateDepth-1 request
// their first tile at once; wavefront w >= kGateDepth requests its first tile
// when the first tile of wavefront w - kGateDepth has arrived. Requested all at
// once, every tile would share the memory pipeline and arrive only near the
// end; gated, tiles arrive in order and the first ones are computed while the
// later ones stream in. The gate only orders requests: a wavefront that waited
// kGateSpins polls goes ahead anyway.
constexpr int kGateDepth = 4;
// Running maximum before a head has seen any row: finite, so a masked score
// (-inf) weighs exp2(-inf - kNoRow) = 0 without a test, and the first visible
// row always moves the maximum (its weight rescales the empty sums by 0).
constexpr float kNoRow = -1e30f;
constexpr int kGateSpins = 1 << 16;

// Flag word in LDS read and written with LDS instructions the compiler does not
// order against vector memory, so polling never waits for this wavefront's own
// outstanding row loads.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ int flag_read(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void flag_write(uint32_t addr, int v) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// s_waitcnt on the vector-memory counter only (N outstanding at most).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS only: it does not wait for the caller's
// outstanding global loads (tile rows requested before the barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <class C>
__global__ __launch_bounds__(64 * C::WAVES) void attend_split_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ k_codes,
    const float* __restrict__ k_norms, const uint8_t* __restrict__ v_codes,
    const float* __restrict__ v_norms, const int32_t* __restrict__ lengths, int n_kv_heads,
    int group, int n_qtok, int max_ctx, int max_len, int tokens_per_split, float qscale,
    float* __restrict__ part_acc, float* __restrict__ part_ml, AttendTables tabs, SignArg ksign,
    ProdArgs pa) {
  constexpr int D = C::D, NHG = C::NHG, WAVES = C::WAVES, E = C::E;
  constexpr int RKW = C::RKW, RVW = C::RVW;
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int len = min(lengths[b], max_len);  // never read past the host bound
  const int t_begin = split * tokens_per_split;
  if (t_begin >= len) return;  // whole workgroup: range past the sequence end
  const int t_end = min(len, t_begin + tokens_per_split);
  const int G = group;
  const int n_q_heads = n_kv_heads * G;
  // The workgroup serves GV = G * n_qtok virtual heads: virtual head vh is
  // query token vh / G of the sequence for query head g G + vh % G. Query
  // token i of n_qtok sees the rows before len - n_qtok + i + 1 (causal
  // multi-token decode); with one query token that is every row.
  const int GV = G * n_qtok;

  unsigned char* vt = lds;
  unsigned char* kt = lds + C::VT_BYTES;
  uint32_t* vstage = (uint32_t*)(lds + C::VT_BYTES + C::KT_BYTES + wave * C::VS_BYTES);
  float* wbuf = (float*)(lds + C::VT_BYTES + C::KT_BYTES + WAVES * C::VS_BYTES + wave * C::WB_BYTES);
  float* wq = (float*)(lds + C::VT_BYTES + C::KT_BYTES + WAVES * (C::VS_BYTES + C::WB_BYTES));
  float* cen = wq + C::QS_BYTES / 4;
  int* gate = (int*)(cen + C::CEN_BYTES / 4);

  const long long kvrow0 = ((long long)b * n_kv_heads + g) * max_ctx;
  const uint32_t* __restrict__ kbase = (const uint32_t*)k_codes + kvrow0 * RKW;
  const uint32_t* __restrict__ vbase = (const uint32_t*)v_codes + kvrow0 * RVW;
  const float* __restrict__ knb = k_norms + kvrow0;
  const float* __restrict__ vnb = v_norms + kvrow0;
  const uint32_t* __restrict__ skb = (const uint32_t*)pa.sketch + kvrow0 * C::SKW;
  const float* __restrict__ rnb = pa.rnorms + kvrow0;

  // ---- tile registers: this lane's token rows and norms. Lanes past the
  //      range end load the range's last row instead (always in bounds); their
  //      scores are masked to -inf, so the rows never contribute.
  auto load_tile = [&](int tile, TileRegs<C>& r) __attribute__((always_inline)) {
    const int t = min(tile + lane, t_end - 1);
    const uint32_t* kr = kbase + (long long)t * RKW;
    const uint32_t* vr = vbase + (long long)t * RVW;
    // written in the order they are consumed (V norm and row, staged first;
    // then K norm and row): vector loads complete in order, so the scores
    // can start on the first pieces of the K row while the rest is in flight
    r.nv = vnb[t];
    if constexpr (RVW % 4 == 0) {
#pragma unroll
      for (int i = 0; i < RVW; i += 4) {
        const uint4 x = *(const uint4*)(vr + i);
        r.vw[i] = x.x; r.vw[i + 1] = x.y; r.vw[i + 2] = x.z; r.vw[i + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RVW; i += 2) {
        const uint2 x = *(const uint2*)(vr + i);
        r.vw[i] = x.x; r.vw[i + 1] = x.y;
      }
    }
    if constexpr (C::KRAW)
      r.nk = 1.f;
    else
      r.nk = knb[t];
    if constexpr (C::PROD) {
      r.rn = rnb[t];
      const uint32_t* sr = skb + (long long)t * C::SKW;
#pragma unroll
      for (int i = 0; i < C::SKW; i += 2) {
        const uint2 x = *(const uint2*)(sr + i);
        r.sk[i] = x.x;
        r.sk[i + 1] = x.y;
      }
    }
    if constexpr (RKW % 4 == 0) {
#pragma unroll
      for (int i = 0; i < RKW; i += 4) {
        const uint4 x = *(const uint4*)(kr + i);
        r.kw[i] = x.x; r.kw[i + 1] = x.y; r.kw[i + 2] = x.z; r.kw[i + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RKW; i += 2) {
        const uint2 x = *(const uint2*)(kr + i);
        r.kw[i] = x.x; r.kw[i + 1] = x.y;
      }
    }
  };

  // ---- prologue, before any tile row is requested: fetch the centroid
  //      tables, this wavefront's query rows and the sign words, build the LDS
  //      tables and rotate the queries.
  const int nthr = 64 * WAVES;
  constexpr int kCenPer = (512 + 64 * WAVES - 1) / (64 * WAVES);
  float cenv[kCenPer];
#pragma unroll
  for (int u = 0; u < kCenPer; ++u) {
    const int i = threadIdx.x + u * nthr;
    cenv[u] = i < 256 ? tabs.v_centroids[i] : (i < 512 ? tabs.k_centroids[i - 256] : 0.f);
  }
  constexpr int kHeadsPerWave = (4 * NHG + WAVES - 1) / WAVES;  // GV <= 4 NHG
  __half qx[kHeadsPerWave][E];
#pragma unroll
  for (int r = 0; r < kHeadsPerWave; ++r) {
    const int vh = min(wave + r * WAVES, GV - 1);  // in bounds; surplus rows unused
    const int qi = vh / G;
    const __half* qrow =
        q + (((long long)b * n_qtok + qi) * n_q_heads + (long long)g * G + (vh - qi * G)) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) qx[r][e] = qrow[E * lane + e];
  }
  // sign word of this lane's coordinates E lane .. E lane + E - 1 (one word:
  // E <= 4 consecutive coordinates never straddle a 32-bit boundary)
  uint32_t sword = 0;
#pragma unroll
  for (int w = 0; w < D / 32; ++w)
    if ((E * lane) >> 5 == w) sword = ksign.bits[w];

  // ---- centroid tables: plain copies (the small loads are consumed before any
  //      tile row is requested, so these waits cover only them), then one
  //      replicated 256-byte row per code (pair)
#pragma unroll
  for (int u = 0; u < kCenPer; ++u) {
    const int i = threadIdx.x + u * nthr;
    if (i < 512) cen[i] = cenv[u];
  }
  float qf[kHeadsPerWave][E];
#pragma unroll
  for (int r = 0; r < kHeadsPerWave; ++r)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      qf[r][e] = __half2float(qx[r][e]);
      asm volatile("" : "+v"(qf[r][e]) : : "memory");  // converted here, before the tile loads
    }
  if (threadIdx.x < WAVES) gate[threadIdx.x] = 0;

  lds_barrier();
  // the ungated wavefronts request their first tile now: every wavefront's
  // small loads are done, and the rest of the prologue overlaps the transfer
  constexpr int kStride = WAVES * kTile;
  const int tile0 = t_begin + wave * kTile;
  TileRegs<C> ra;
  // a wavefront past the range end (short ranges) has no tile: it requests
  // nothing and waits for no gate (the later ones have none either)
  const bool has_tile = tile0 < t_end;
  if (wave < kGateDepth && has_tile) load_tile(tile0, ra);
  auto fill = [&](unsigned char* tab, const float* c, int bits, bool pair) {
    const int rows = 1 << (pair ? 2 * bits : bits);
    const int mask = (1 << bits) - 1;
    for (int i = threadIdx.x; i < rows * 16; i += nthr) {
      const int e = i >> 4;
      const v4f x = pair ? v4f{c[e & mask], c[e >> bits], c[e & mask], c[e >> bits]}
                         : v4f{c[e], c[e], c[e], c[e]};
      ((v4f*)tab)[i] = x;
    }
  };
  fill(vt, cen, C::BV, C::VPAIR);
  if constexpr (!C::KRAW) fill(kt, cen + 256, C::KBITS, C::KPAIR);

  // ---- rotated queries: wavefront w rotates heads w, w + WAVES, ... into LDS
#pragma unroll
  for (int r = 0; r < kHeadsPerWave; ++r) {
    const int h = wave + r * WAVES;
    if (h < GV) {
      float u[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = E * lane + e;
        const float x = qf[r][e];
        u[e] = (!C::KRAW && ((sword >> (j & 31)) & 1u)) ? -x : x;
      }
      // raw keys are scored in the original basis: no rotation
#pragma unroll
      for (int hs = 1; hs < (C::KRAW ? 1 : E); hs <<= 1)
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & hs) == 0) {
            const float a0 = u[e], a1 = u[e + hs];
            u[e] = a0 + a1;
            u[e + hs] = a0 - a1;
          }
#pragma unroll
      for (int m = 1; m < (C::KRAW ? 1 : 64); m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float p = __shfl_xor(u[e], m);
          u[e] = upper ? (p - u[e]) : (u[e] + p);
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) wq[h * D + E * lane + e] = u[e] * qscale;
      if constexpr (C::PROD) {
        // sketch projection H (sigma_S (.) q~) of the rotated query
        uint32_t pw = pa.sign.bits[0];
#pragma unroll
        for (int w = 1; w < D / 32; ++w) pw = ((E * lane) >> 5 == w) ? pa.sign.bits[w] : pw;
#pragma unroll
        for (int e = 0; e < E; ++e) u[e] = ((pw >> ((E * lane + e) & 31)) & 1u) ? -u[e] : u[e];
#pragma unroll
        for (int hs = 1; hs < E; hs <<= 1)
#pragma unroll
          for (int e = 0; e < E; ++e)
            if ((e & hs) == 0) {
              const float a0 = u[e], a1 = u[e + hs];
              u[e] = a0 + a1;
              u[e + hs] = a0 - a1;
            }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const bool upper = (lane & m) != 0;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float p = __shfl_xor(u[e], m);
            u[e] = upper ? (p - u[e]) : (u[e] + p);
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e) wq[4 * NHG * D + h * D + E * lane + e] = u[e] * pa.uscale;
      }
    }
  }
  lds_barrier();  // tables, rotated queries and gate flags ready

  // broadcast layout: lane 4c + v of VGPR Q[hg][m] holds q^[4 hg + v][16 m + c]
  float Q[NHG][D / 16];
  float U[C::PROD ? NHG : 1][C::PROD ? D / 16 : 1];  // Prod keys: sketch projections
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int h = 4 * hg + (lane & 3);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) Q[hg][m] = h < GV ? wq[h * D + 16 * m + (lane >> 2)] : 0.f;
    if constexpr (C::PROD) {
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        U[hg][m] = h < GV ? wq[4 * NHG * D + h * D + 16 * m + (lane >> 2)] : 0.f;
    }
  }

  // The gated wavefronts request their first tile once the first tile of
  // wavefront w - kGateDepth has arrived. No workgroup barrier follows until
  // the merge: a wavefront may stall in issuing vector loads while the memory
  // pipeline is full, and each one runs its tiles independently.
  if (wave >= kGateDepth && has_tile) {
    const uint32_t ga = lds_addr(gate + (wave - kGateDepth));
    for (int i = 0; i < kGateSpins && flag_read(ga) == 0; ++i) __builtin_amdgcn_s_sleep(1);
    load_tile(tile0, ra);
  }
  // this wavefront's first tile has arrived: open the gate of wavefront w + kGateDepth
  wait_vmcnt<0>();
  flag_write(lds_addr(gate + wave), 1);

  // rows [0, vlim) are visible to virtual head 4 hg + v (wavefront-uniform)
  int vlim[NHG][4];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int v = 0; v < 4; ++v) vlim[hg][v] = min(t_end, len - n_qtok + (4 * hg + v) / G + 1);

  // ---- per-wave online-softmax state
  float m_run[NHG][4];
  v4f l_run[NHG];
  v4f acc[C::NACC][NHG];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    l_run[hg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) m_run[hg][v] = kNoRow;
#pragma unroll
    for (int a = 0; a < C::NACC; ++a) acc[a][hg] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  const uint32_t koff = C::KPAIR ? (uint32_t)(lane & 31) << 3 : (uint32_t)lane << 2;
  const uint32_t voff = C::VPAIR ? (uint32_t)(lane & 31) << 3 : (uint32_t)lane << 2;
  constexpr uint32_t KMASK = ((1u << C::KF) - 1u) << 8;
  constexpr uint32_t VMASK = ((1u << C::VF) - 1u) << 8;

  // V fields of this lane: field 64k + lane of each staged row, read from bit
  // o - 8 of the padded row so the field lands at bit 8
  int vdw[C::NVS], vsh[C::NVS];
#pragma unroll
  for (int k = 0; k < C::NVS; ++k) {
    const int o = C::VF * (64 * k + lane) + 64 - 8;
    vdw[k] = o >> 5;
    vsh[k] = o & 31;
  }

  // One tile: scores, online softmax, values. `r` is consumed and refilled
  // with the wavefront's next tile as soon as its rows have been used.
  auto process = [&](int tile, TileRegs<C>& r) __attribute__((always_inline)) {

    // stage this token's V row (row `lane`, after 2 dwords of padding)
#pragma unroll
    for (int i = 0; i < RVW; i += 2)
      *(uint2*)(vstage + 2 + lane * RVW + i) = uint2{r.vw[i], r.vw[i + 1]};

    // ---- scores on the matrix cores. The lookups of batch j + 1 are issued
    //      before the products of batch j, so a batch's LDS latency hides
    //      behind the previous batch's MFMAs; four accumulator chains.
    using KLut = std::conditional_t<C::KPAIR, v2f, float>;
    v4f sc[4][NHG];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg) sc[a4][hg] = v4f{0.f, 0.f, 0.f, 0.f};
    auto k_lookup = [&](auto BI, KLut (&dst)[kKBatch]) __attribute__((always_inline)) {
      sfor<kKBatch>([&](auto II) {
        constexpr int f = BI * kKBatch + II;
        constexpr int bit = C::KF * f;
        uint32_t addr;
        if constexpr (C::KRAW) {
          // coordinate f of the raw key row: half f % 2 of dword f / 2
          dst[II] = __half2float(__builtin_bit_cast(__half, (uint16_t)(r.kw[f >> 1] >> (16 * (f & 1)))));
          return;
        } else if constexpr (C::KF == 8) {
          // whole byte: one byte permute builds (code << 8) | koff
          addr = __builtin_amdgcn_perm(r.kw[bit >> 5], koff,
                                       0x0C0C0000u | ((4u + ((bit >> 3) & 3)) << 8));
        } else {
          addr = (field_at8<bit, C::KF>(r.kw) & KMASK) | koff;
        }
        dst[II] = *(const KLut*)(kt + addr);
      });
    };
    auto k_mfma = [&](auto BI, const KLut (&src)[kKBatch]) __attribute__((always_inline)) {
      sfor<kKBatch>([&](auto II) {
        constexpr int f = BI * kKBatch + II;
        if constexpr (C::KPAIR) {
          constexpr int j0 = 2 * f, j1 = 2 * f + 1, a0 = 2 * (f % 2);
#pragma unroll
          for (int hg = 0; hg < NHG; ++hg) {
            sc[a0][hg] = mfma_bcast<j0 % 16>(Q[hg][j0 / 16], src[II].x, sc[a0][hg]);
            sc[a0 + 1][hg] = mfma_bcast<j1 % 16>(Q[hg][j1 / 16], src[II].y, sc[a0 + 1][hg]);
          }
        } else {
#pragma unroll
          for (int hg = 0; hg < NHG; ++hg)
            sc[f % 4][hg] = mfma_bcast<f % 16>(Q[hg][f / 16], src[II], sc[f % 4][hg]);
        }
      });
    };
    {
      constexpr int NKB = C::NKL / kKBatch;
      KLut lb0[kKBatch], lb1[kKBatch];
      k_lookup(std::integral_constant<int, 0>{}, lb0);
      sfor<NKB>([&](auto BI) {
        constexpr int bb = BI;
        if constexpr (bb % 2 == 0) {
          if constexpr (bb + 1 < NKB) k_lookup(std::integral_constant<int, bb + 1>{}, lb1);
          k_mfma(BI, lb0);
        } else {
          if constexpr (bb + 1 < NKB) k_lookup(std::integral_constant<int, bb + 1>{}, lb0);
          k_mfma(BI, lb1);
        }
      });
    }
    v4f s0[NHG];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) s0[hg] = (sc[0][hg] + sc[1][hg]) + (sc[2][hg] + sc[3][hg]);
    if constexpr (C::PROD) {
      // QJL correction: residual norm x sum_j sgn_j u^_j, sgn_j = -1 for a set
      // sketch bit (the bit becomes the sign of 1.0 as the MFMA operand)
      v4f kc4[4][NHG];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg) kc4[a4][hg] = v4f{0.f, 0.f, 0.f, 0.f};
      sfor<D>([&](auto JI) {
        constexpr int j = JI;
        const float sg =
            __builtin_bit_cast(float, 0x3f800000u | ((r.sk[j >> 5] << (31 - (j & 31))) & 0x80000000u));
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
          kc4[j % 4][hg] = mfma_bcast<j % 16>(U[hg][j / 16], sg, kc4[j % 4][hg]);
      });
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg)
        s0[hg] += r.rn * ((kc4[0][hg] + kc4[1][hg]) + (kc4[2][hg] + kc4[3][hg]));
    }

    const float nv_cur = r.nv;
    const float nk_cur = r.nk;
    // the rows are consumed: refill with this wavefront's next tile
    const int ahead = tile + kStride;
    if (ahead < t_end) load_tile(ahead, r);

    // ---- online softmax (base 2) with a lazily moved maximum
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const v4f s = s0[hg] * nk_cur;
      v4f w;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sv = tile + lane < vlim[hg][v] ? s[v] : -INFINITY;
        // the tile maximum exceeds m_run + slack iff some lane's score does:
        // one compare and a ballot decide it, and the maximum itself is only
        // taken then (always on a wavefront's first tile, rarely after)
        if (__ballot(sv > m_run[hg][v] + kRescaleSlack) != 0ull) {  // wavefront-uniform
          const float mt = wave_max_key(sv);
          const float alpha = __builtin_amdgcn_exp2f(m_run[hg][v] - mt);
          l_run[hg][v] *= alpha;
#pragma unroll
          for (int a = 0; a < C::NACC; ++a) acc[a][hg][v] *= alpha;
          m_run[hg][v] = mt;
        }
        const float p = __builtin_amdgcn_exp2f(sv - m_run[hg][v]);
        l_run[hg][v] += p;
        w[v] = p * nv_cur;
      }
      *(v4f*)(wbuf + (lane * NHG + hg) * 4) = w;
    }
    wave_lds_sync();

    // weights in the broadcast layout: lane 4c + v of Wr[hg][m] holds w[4 hg + v][16 m + c]
    float Wr[NHG][4];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        Wr[hg][m] = wbuf[((16 * m + (lane >> 2)) * NHG + hg) * 4 + (lane & 3)];

    // ---- values on the matrix cores, lanes over coordinates. Three stages
    //      over batches of tokens: the staged dwords around this lane's
    //      fields (two batches ahead), the centroid lookups (one batch
    //      ahead), the products.
    using VLut = std::conditional_t<C::VPAIR, v2f, float>;
    constexpr int TB = kVBatch, NTB = kTile / TB;
    auto v_stage = [&](auto JI, uint2 (&dst)[TB][C::NVS]) __attribute__((always_inline)) {
      sfor<TB>([&](auto TI) {
        constexpr int t = JI * TB + TI;
        const uint32_t* row = vstage + t * RVW;
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) dst[TI][k] = uint2{row[vdw[k]], row[vdw[k] + 1]};
      });
    };
    auto v_lookup = [&](const uint2 (&xs)[TB][C::NVS], VLut (&dst)[TB][C::NVS]) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < TB; ++tt)
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) {
          const uint32_t x = __builtin_amdgcn_alignbit(xs[tt][k].y, xs[tt][k].x, vsh[k]);
          dst[tt][k] = *(const VLut*)(vt + ((x & VMASK) | voff));
        }
    };
    auto v_mfma = [&](auto JI, const VLut (&cs)[TB][C::NVS]) __attribute__((always_inline)) {
      sfor<TB>([&](auto TI) {
        constexpr int t = JI * TB + TI;
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) {
          if constexpr (C::VPAIR) {
#pragma unroll
            for (int hg = 0; hg < NHG; ++hg) {
              acc[2 * k][hg] = mfma_bcast<t % 16>(Wr[hg][t / 16], cs[TI][k].x, acc[2 * k][hg]);
              acc[2 * k + 1][hg] = mfma_bcast<t % 16>(Wr[hg][t / 16], cs[TI][k].y, acc[2 * k + 1][hg]);
            }
          } else {
            constexpr int par = (C::NVS == 1) ? (t & 1) : 0;
#pragma unroll
            for (int hg = 0; hg < NHG; ++hg)
              acc[k + par][hg] = mfma_bcast<t % 16>(Wr[hg][t / 16], cs[TI][k], acc[k + par][hg]);
          }
        }
      });
    };
    {
      uint2 xs0[TB][C::NVS], xs1[TB][C::NVS], xs2[TB][C::NVS];
      VLut cv0[TB][C::NVS], cv1[TB][C::NVS];
      v_stage(std::integral_constant<int, 0>{}, xs0);
      v_stage(std::integral_constant<int, 1>{}, xs1);
      v_lookup(xs0, cv0);
      // batch j: stage j + 2 into xs[(j + 2) % 3], look up j + 1 from xs[(j + 1) % 3]
      // into cv[(j + 1) % 2], multiply batch j from cv[j % 2]
      sfor<NTB>([&](auto JI) {
        constexpr int j = JI;
        auto& xs_next2 = (j + 2) % 3 == 0 ? xs0 : (j + 2) % 3 == 1 ? xs1 : xs2;
        auto& xs_next1 = (j + 1) % 3 == 0 ? xs0 : (j + 1) % 3 == 1 ? xs1 : xs2;
        auto& cv_next = (j + 1) % 2 == 0 ? cv0 : cv1;
        auto& cv_cur = j % 2 == 0 ? cv0 : cv1;
        if constexpr (j + 2 < NTB) v_stage(std::integral_constant<int, j + 2>{}, xs_next2);
        if constexpr (j + 1 < NTB) v_lookup(xs_next1, cv_next);
        v_mfma(JI, cv_cur);
      });
    }
    wave_lds_sync();
  };

  // the first tile is peeled off the loop so that its register waits follow
  // the order its loads were issued in
  if (has_tile) process(tile0, ra);
  for (int tile = tile0 + kStride; tile < t_end; tile += kStride) process(tile, ra);

  // ---- merge the wavefronts of this workgroup and write the split partial:
  //      every wavefront stores its maxima, sums and unscaled accumulators,
  //      then thread (virtual head, coordinate) folds the wavefronts with the
  //      factors 2^(m_w - M), M their maximum (a wavefront that saw no row
  //      has the finite sentinel maximum, so it weighs 0 next to one that did)
  if constexpr (C::NVS == 1 && !C::VPAIR) {
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) acc[0][hg] += acc[1][hg];
  }
  __syncthreads();  // all wavefronts are done with tables and buffers
  constexpr int NV = 4 * NHG;                   // virtual-head slots per wavefront
  float* mbuf = (float*)lds;                    // [WAVES][NV] maxima
  float* lbuf = mbuf + WAVES * NV;              // [WAVES][NV] sums
  float* abuf = lbuf + WAVES * NV;              // [WAVES][NV][D] accumulators
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lsum = wave_sum(l_run[hg][v]);
      if (lane == 0) {
        mbuf[wave * NV + 4 * hg + v] = m_run[hg][v];
        lbuf[wave * NV + 4 * hg + v] = lsum;
      }
      float* dst = abuf + (wave * NV + 4 * hg + v) * D;
      if constexpr (C::VPAIR) {
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) {
          dst[2 * (64 * k + lane)] = acc[2 * k][hg][v];
          dst[2 * (64 * k + lane) + 1] = acc[2 * k + 1][hg][v];
        }
      } else {
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) dst[64 * k + lane] = acc[k][hg][v];
      }
    }
  __syncthreads();
  const int S = gridDim.x;
  for (int idx = threadIdx.x; idx < NV * D; idx += 64 * WAVES) {
    const int h = idx / D, j = idx - h * D;
    if (h >= GV) continue;
    float M = -INFINITY;
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mbuf[w * NV + h]);
    float a = 0.f, L = 0.f;
    for (int w = 0; w < WAVES; ++w) {
      const float f = exp2f(mbuf[w * NV + h] - M);
      a += f * abuf[(w * NV + h) * D + j];
      L += f * lbuf[w * NV + h];
    }
    const long long prow = (((long long)b * n_kv_heads + g) * GV + h) * S + split;
    part_acc[prow * D + j] = a;
    if (j == 0) {
      part_ml[prow * 2] = M;
      part_ml[prow * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- 2. combine

constexpr int kCombineThreads = 1024;
constexpr int kCombineUnroll = 4;  // splits per thread whose loads are in flight together
constexpr int kMaxRawRows = 4096;  // raw fp16 rows per sequence and KV head (scores in LDS)

// Raw fp16 rows attended with the packed cache: an fp16 prefix of "sink"
// tokens kept uncompressed (turboquant-mlx guide, --kv-min-tokens) or pending
// tokens not yet batch-compressed (PR #232, Design). lengths == nullptr: none.
struct RawArgs {
  const __half* q;       // [B][Hq][D], the unrotated queries
  const __half* k;       // [B][Hkv][max_raw][D]
  const __half* v;
  const int32_t* lengths;
  int max_raw;
  int n_kv_heads;
  float qscale2;         // softmax scale * log2(e): scores in the splits' base-2 units
};

// One workgroup per (sequence, query row): merges the split partials of the
// packed rows, adds the raw rows' attention when there are any, normalises and
// applies the inverse rotation to the packed part. The raw part needs none:
// its V sum is taken in the original basis and added after the rotation.
template <int D, bool kRaw>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml,
    const int32_t* __restrict__ lengths, int max_len, int n_q_heads, int group, int n_qtok,
    int splits, int tokens_per_split, float* __restrict__ out, SignArg sign, RawArgs raw) {
  constexpr int E = D / 64;
  constexpr int NG = kCombineThreads / D;  // split groups
  constexpr int U = kCombineUnroll;
  constexpr int RL = 16;                   // lanes per raw row for its score
  constexpr int RPD = D / RL;              // coordinates per lane
  __shared__ float s_acc[NG][D];
  __shared__ float s_racc[kRaw ? NG : 1][D];
  __shared__ float s_l[NG];
  __shared__ float s_m[NG];
  __shared__ float s_lr[kRaw ? NG : 1];
  __shared__ float s_raw[kRaw ? kMaxRawRows : 1];
  const int tid = threadIdx.x;
  // partial row: virtual head hx = g GV + vh of sequence b; output row: query
  // token vh / G, query head g G + vh % G
  const int hx = blockIdx.x, b = blockIdx.y;
  const int GV = group * n_qtok;
  const long long row = (long long)b * n_q_heads * n_qtok + hx;
  const int g = hx / GV, vh = hx - g * GV, qi = vh / group;
  const long long orow =
      ((long long)b * n_qtok + qi) * n_q_heads + (long long)g * group + (vh - qi * group);
  const float* ml = part_ml + row * splits * 2;
  // sign word of coordinates E lane .. E lane + E - 1 (scalar loads, early)
  uint32_t sword = 0;
#pragma unroll
  for (int w = 0; w < D / 32; ++w)
    if ((E * (tid & 63)) >> 5 == w) sword = sign.bits[w];

  // rescaled sums: thread (group grp, coordinate j) over splits s = grp mod NG,
  // U splits at a time, each group with its own running maximum. The loads
  // are issued before the sequence length arrives: slots past the valid
  // splits read in-bounds workspace and are dropped.
  const int j = tid % D, grp = tid / D;
  const float* pa = part_acc + row * splits * D + j;
  const int len = min(lengths[b], max_len);
  const int ns = len > 0 ? min(splits, (len + tokens_per_split - 1) / tokens_per_split) : 0;
  const int R = kRaw ? min(raw.lengths[b], raw.max_raw) : 0;
  float a = 0.f, L = 0.f, mg = -INFINITY;
  for (int s0 = grp; s0 < splits; s0 += NG * U) {
    float mv[U], lv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u * NG, splits - 1);
      mv[u] = ml[2 * s];
      lv[u] = ml[2 * s + 1];
      av[u] = pa[(long long)s * D];
    }
    // a split where this head saw no row has maximum -inf and is dropped
    bool ok[U];
    float mnew = mg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = s0 + u * NG < ns && mv[u] != -INFINITY;
      if (ok[u]) mnew = fmaxf(mnew, mv[u]);
    }
    if (mnew != mg) {  // mnew > mg: rescale (by 0 while mg is still -inf)
      const float r = exp2f(mg - mnew);
      a *= r;
      L *= r;
      mg = mnew;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) {
        const float f = exp2f(mv[u] - mg);
        a = fmaf(f, av[u], a);
        L = fmaf(f, lv[u], L);
      }
  }

  // raw rows: scores (RL lanes per row, 64 rows per pass) into LDS, their
  // maximum mr, then weights and the V sum in the original basis, rows
  // t = grp mod NG, U of them with their loads in flight together
  float mr = -INFINITY, ar = 0.f, Lr = 0.f;
  if (kRaw && R > 0) {
    const long long kv0 = ((long long)b * raw.n_kv_heads + g) * raw.max_raw;
    const int part = tid % RL;
    const __half* qr = raw.q + orow * D + part * RPD;
    float qv[RPD];
#pragma unroll
    for (int i = 0; i < RPD; ++i) qv[i] = __half2float(qr[i]) * raw.qscale2;
    for (int t0 = 0; t0 < R; t0 += kCombineThreads / RL) {
      const int t = t0 + tid / RL;
      const __half* kr = raw.k + (kv0 + min(t, R - 1)) * D + part * RPD;
      float sc = 0.f;
#pragma unroll
      for (int i = 0; i < RPD; ++i) sc = fmaf(qv[i], __half2float(kr[i]), sc);
#pragma unroll
      for (int m = 1; m < RL; m <<= 1) sc += __shfl_xor(sc, m);
      if (part == 0 && t < R) s_raw[t] = sc;
    }
    __syncthreads();
    for (int t = tid & 63; t < R; t += 64) mr = fmaxf(mr, s_raw[t]);
    mr = wave_max(mr);
    const __half* vcol =
        raw.v + ((long long)b * raw.n_kv_heads + g) * raw.max_raw * D + j;
    for (int t0 = grp; t0 < R; t0 += NG * 2 * U) {
      float vv[2 * U], pp[2 * U];
#pragma unroll
      for (int u = 0; u < 2 * U; ++u) {
        const int t = min(t0 + u * NG, R - 1);
        vv[u] = __half2float(vcol[(long long)t * D]);
        pp[u] = t0 + u * NG < R ? exp2f(s_raw[t] - mr) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 2 * U; ++u) {
        ar = fmaf(pp[u], vv[u], ar);
        Lr += pp[u];
      }
    }
  }
  s_acc[grp][j] = a;
  if constexpr (kRaw) s_racc[grp][j] = ar;
  if (j == 0) {
    s_m[grp] = mg;
    s_l[grp] = L;
    if constexpr (kRaw) s_lr[grp] = Lr;
  }
  __syncthreads();

  if (tid < 64) {
    const int lane = tid;
    float u[E], ur[E];
    // the groups (and the raw rows) meet at the overall maximum M
    float M = mr;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) M = fmaxf(M, s_m[g2]);
    float fg[NG];
    float Lt = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      fg[g2] = s_m[g2] == -INFINITY ? 0.f : exp2f(s_m[g2] - M);
      Lt = fmaf(fg[g2], s_l[g2], Lt);
    }
    const float fr = kRaw && mr != -INFINITY ? exp2f(mr - M) : 0.f;
    if constexpr (kRaw) {
      float lr = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) lr += s_lr[g2];
      Lt = fmaf(fr, lr, Lt);
    }
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;  // no visible row: a zero output row
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float x = 0.f, xr = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < NG; ++g2) {
        x = fmaf(fg[g2], s_acc[g2][E * lane + e], x);
        if constexpr (kRaw) xr += s_racc[g2][E * lane + e];
      }
      u[e] = Lt > 0.f ? x / Lt : 0.f;
      ur[e] = xr * fr * inv;
    }
    // inverse rotation: out = (1/d) sigma_V (.) H a
#pragma unroll
    for (int hs = 1; hs < E; hs <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((e & hs) == 0) {
          const float x0 = u[e], x1 = u[e + hs];
          u[e] = x0 + x1;
          u[e + hs] = x0 - x1;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float p = __shfl_xor(u[e], m);
        u[e] = upper ? (p - u[e]) : (u[e] + p);
      }
    }
    const float invd = 1.f / (float)D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int jj = E * lane + e;
      const float v = u[e] * invd;
      out[orow * D + jj] = (((sword >> (jj & 31)) & 1u) ? -v : v) + ur[e];
    }
  }
}

// ---------------------------------------------------------------- dispatch

template <class C>
hipError_t launch_split(const AttendPlan& plan, int batch, int n_kv_heads, int group,
                        int n_qtok, const void* q, const uint8_t* kc, const float* kn,
                        const uint8_t* vc,
                        const float* vn, const int32_t* lengths, int max_ctx, int max_len,
                        float qscale, float* pacc, float* pml, const AttendTables& tabs,
                        const SignArg& ksign, const ProdArgs& pa, hipEvent_t ev_start,
                        hipEvent_t ev_stop, hipStream_t stream) {
  const dim3 grid(plan.splits, n_kv_heads, batch), block(64 * C::WAVES);
  if (ev_start) {
    // events bound to this dispatch: they time the kernel itself, not the queue
    hipExtLaunchKernelGGL((attend_split_kernel<C>), grid, block, 0, stream, ev_start, ev_stop, 0,
                          (const __half*)q, kc, kn, vc, vn, lengths, n_kv_heads, group, n_qtok,
                          max_ctx, max_len, plan.tokens_per_split, qscale, pacc, pml, tabs,
                          ksign, pa);
  } else {
    hipLaunchKernelGGL((attend_split_kernel<C>), grid, block, 0, stream, (const __half*)q, kc, kn,
                       vc, vn, lengths, n_kv_heads, group, n_qtok, max_ctx, max_len,
                       plan.tokens_per_split, qscale, pacc, pml, tabs, ksign, pa);
  }
  return hipGetLastError();
}

typedef hipError_t (*SplitFn)(const AttendPlan&, int, int, int, int, const void*, const uint8_t*,
                              const float*, const uint8_t*, const float*, const int32_t*, int,
                              int, float, float*, float*, const AttendTables&, const SignArg&,
                              const ProdArgs&, hipEvent_t, hipEvent_t, hipStream_t);

struct SplitEntry {
  int d, bk, bv, nhg;
  SplitFn fn;
  SplitFn short_fn;  // 4-wavefront workgroups for ranges of <= kShortTiles tiles, or null
};

// Instantiated (head_dim, K bits, V bits, groups of 4 query heads). A group
// size G is served by the entry with the smallest nhg such that G <= 4 * nhg.
// TQ_SPLIT_S entries also have the short-range variant (the small-context
// workloads' configurations).
#define TQ_SPLIT(D, BK, BV, NHG) {D, BK, BV, NHG, &launch_split<Cfg<D, BK, BV, NHG>>, nullptr}
#define TQ_SPLIT_S(D, BK, BV, NHG)                                      \
  {D, BK, BV, NHG, &launch_split<Cfg<D, BK, BV, NHG>>,                  \
   &launch_split<CfgShort<D, BK, BV, NHG>>}
const SplitEntry kSplitTable[] = {
    // head_dim 64
    TQ_SPLIT_S(64, 4, 4, 1), TQ_SPLIT(64, 3, 3, 2), TQ_SPLIT(64, 3, 3, 1),
    TQ_SPLIT(64, 8, 3, 1), TQ_SPLIT(64, 2, 2, 1), TQ_SPLIT(64, 1, 1, 1),
    TQ_SPLIT(64, 5, 7, 1), TQ_SPLIT(64, 6, 6, 4), TQ_SPLIT(64, 4, 4, 2),
    TQ_SPLIT(64, 8, 3, 2), TQ_SPLIT(64, 3, 3, 4), TQ_SPLIT(64, 16, 4, 1), TQ_SPLIT(64, 16, 4, 2),
    TQ_SPLIT(64, 35, 4, 1),
    // head_dim 128
    TQ_SPLIT_S(128, 4, 2, 1), TQ_SPLIT(128, 8, 3, 1), TQ_SPLIT(128, 3, 3, 1),
    TQ_SPLIT(128, 4, 4, 1), TQ_SPLIT(128, 4, 3, 1), TQ_SPLIT(128, 2, 2, 1),
    TQ_SPLIT(128, 8, 4, 1), TQ_SPLIT(128, 4, 4, 2), TQ_SPLIT(128, 8, 3, 2),
    TQ_SPLIT(128, 1, 1, 1), TQ_SPLIT(128, 7, 5, 2),
    TQ_SPLIT(128, 3, 3, 2), TQ_SPLIT(128, 4, 2, 2),
    // four query tokens of a group of 4 (multi-token decode)
    TQ_SPLIT(128, 8, 3, 4), TQ_SPLIT(128, 3, 3, 4),
    // raw fp16 keys (turbo0v4, turbo0v2)
    TQ_SPLIT(128, 16, 4, 1), TQ_SPLIT(128, 16, 2, 1), TQ_SPLIT(128, 16, 4, 2),
    // TurboQuant-Prod keys (32 + code bits): 4-bit (3 + sketch) with 4-bit V,
    // 3-bit (2 + sketch) with 3-bit V
    TQ_SPLIT(128, 35, 4, 1), TQ_SPLIT(128, 35, 4, 2), TQ_SPLIT(128, 34, 3, 1),
    // head_dim 256
    TQ_SPLIT(256, 4, 4, 1), TQ_SPLIT(256, 8, 3, 1), TQ_SPLIT(256, 3, 3, 1),
    TQ_SPLIT(256, 8, 4, 1), TQ_SPLIT(256, 2, 2, 2),
};
#undef TQ_SPLIT
#undef TQ_SPLIT_S

const SplitEntry* find_split(int d, int bk, int bv, int group) {
  const SplitEntry* best = nullptr;
  for (const SplitEntry& e : kSplitTable)
    if (e.d == d && e.bk == bk && e.bv == bv && group <= 4 * e.nhg &&
        (!best || e.nhg < best->nhg))
      best = &e;
  return best;
}

}  // namespace

AttendPlan plan_attend(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len) {
  AttendPlan p{};
  // About one workgroup per CU (256 CUs), each range a whole number of
  // 64-token tiles: short contexts get short ranges (some wavefronts of a
  // workgroup then have no tile) rather than fewer workgroups than CUs.
  const long long units = (long long)batch * n_kv_heads;
  const long long target_wgs = 256;
  const long long quantum = kTile;
  long long tps = ((long long)max_len * units + target_wgs - 1) / target_wgs;
  tps = ((tps + quantum - 1) / quantum) * quantum;
  if (tps < quantum) tps = quantum;
  p.tokens_per_split = (int)tps;
  p.splits = (int)((max_len + tps - 1) / tps);
  if (p.splits < 1) p.splits = 1;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.qhat_bytes = 0;
  p.part_acc_bytes = align((size_t)batch * n_q_heads * p.splits * dim * sizeof(float));
  p.part_ml_bytes = align((size_t)batch * n_q_heads * p.splits * 2 * sizeof(float));
  p.total_bytes = p.part_acc_bytes + p.part_ml_bytes;
  return p;
}

bool attend_supported(int dim, int k_bits, int v_bits, int group) {
  return find_split(dim, k_bits, v_bits, group) != nullptr;
}

hipError_t launch_attend(int dim, int k_bits, int v_bits, int batch, int n_qtok, int n_q_heads,
                         int n_kv_heads, const void* q, const SignArg& k_sign,
                         const SignArg& v_sign, const AttendTables& tabs,
                         const uint8_t* k_codes, const float* k_norms,
                         const uint8_t* v_codes, const float* v_norms, int max_ctx,
                         const int32_t* lengths, int max_len, float scale, float* out,
                         void* workspace, const AttendPlan& plan, const RawSegment& raw,
                         const ProdKeys& prodk, hipEvent_t ev_before, hipEvent_t ev_after,
                         hipStream_t stream) {
  const int group = n_q_heads / n_kv_heads;
  const SplitEntry* ent = find_split(dim, k_bits, v_bits, group * n_qtok);
  if (!ent) return hipErrorInvalidValue;
  char* ws = (char*)workspace;
  float* pacc = (float*)ws;
  float* pml = (float*)(ws + plan.part_acc_bytes);
  // rotated keys carry a factor d (H H = d I); raw keys are scored as they are
  const float qscale = k_bits == 16 ? scale * kLog2e : scale * kLog2e / (float)dim;
  hipError_t err;
  ProdArgs pa;
  pa.sketch = prodk.sketch;
  pa.rnorms = prodk.rnorms;
  pa.sign = prodk.sign;
  pa.uscale = qscale * 1.2533141373155003f / (float)dim;  // sqrt(pi/2) / d
  const SplitFn fn =
      ent->short_fn && plan.tokens_per_split <= kShortTiles * kTile ? ent->short_fn : ent->fn;
  err = fn(plan, batch, n_kv_heads, group, n_qtok, q, k_codes, k_norms, v_codes, v_norms, lengths,
           max_ctx, max_len, qscale, pacc, pml, tabs, k_sign, pa, ev_before, ev_after, stream);
  if (err != hipSuccess) return err;
  if (raw.lengths && n_qtok != 1) return hipErrorInvalidValue;
  RawArgs ra;
  ra.q = (const __half*)q;
  ra.k = (const __half*)raw.k;
  ra.v = (const __half*)raw.v;
  ra.lengths = raw.lengths;
  ra.max_raw = raw.max_raw;
  ra.n_kv_heads = n_kv_heads;
  ra.qscale2 = scale * kLog2e;
  const dim3 cgrid(n_q_heads * n_qtok, batch);
  switch (dim) {
    case 64:
      if (raw.lengths)
        hipLaunchKernelGGL((combine_kernel<64, true>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      else
        hipLaunchKernelGGL((combine_kernel<64, false>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      break;
    case 128:
      if (raw.lengths)
        hipLaunchKernelGGL((combine_kernel<128, true>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      else
        hipLaunchKernelGGL((combine_kernel<128, false>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      break;
    case 256:
      if (raw.lengths)
        hipLaunchKernelGGL((combine_kernel<256, true>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      else
        hipLaunchKernelGGL((combine_kernel<256, false>), cgrid, dim3(kCombineThreads), 0, stream,
                           pacc, pml, lengths, max_len, n_q_heads, group, n_qtok, plan.splits,
                           plan.tokens_per_split, out, v_sign, ra);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tq

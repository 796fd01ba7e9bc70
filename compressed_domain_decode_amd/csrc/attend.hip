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
//    Both contractions run on the matrix cores as fp16 4x4x4 products with
//    fp32 accumulation, each fp32 operand carried as an fp16 pair hi + lo
//    (hi the nearest fp16, lo the nearest fp16 of the remainder; about 22
//    significant bits). On gfx950 the fp16 matrix instructions can execute
//    alongside VALU work, which the fp32 ones do not, so part of the
//    unpacking and table addressing overlaps the products. The 4-deep reduction of an
//    instruction is laid out as (hi_j, lo_j, hi_j', lo_j') of two
//    coordinates (scores) or two tokens (values), so a centroid entry
//    (hi, lo) read from LDS is an operand as it stands:
//      scores  S[h][t] = sum_j q^[h][j] * cK[idxK[t][j]]
//              lane t holds token t's packed K row. Per coordinate pair the
//              B operand is the two centroid entries; the A operand, broadcast
//              from one 4-lane block, is (qh_j, qh_j, qh_j', qh_j') for the
//              first product and (ql_j, 0, ql_j', 0) for the second, so the
//              sum is qh (ch + cl) + ql ch. Lane t ends with the 4 heads'
//              scores of token t.
//      softmax online softmax in base 2 (log2 e folded into q^), per head
//              running max from a cross-lane reduction; weights p * nV_t.
//      values  A[h][j] += sum_t w[h][t] * cV[idxV[t][j]]
//              lanes own coordinates. A tile's packed V rows are copied into
//              the wavefront's LDS stage by buffer loads straight to LDS;
//              per token each lane reads the two dwords
//              that hold its code(s), funnel-shifts them and looks the
//              centroid entry up; two tokens' entries form the B operand and
//              the weights, (wh_t, wh_t, wh_t', wh_t') and (wl_t, 0, wl_t', 0),
//              the broadcast A operand.
//    Scale factors (powers of two, exact) keep every fp16 half in the normal
//    range: the rotated queries of a workgroup and each codebook are scaled
//    so their largest magnitude lies in [2^13, 2^14), and the weights carry
//    2^(6 - Ev) with 2^Ev above every V norm seen so far (Ev only grows, and
//    the accumulators are rescaled when it does).
//    The online softmax moves its running maximum only when a tile's
//    maximum exceeds it by more than 2^8, so the rescale is rare.
//    Centroid tables live in LDS replicated once per bank (a 256-byte row
//    per code: 64 copies of a 4-byte entry, or 32 of an 8-byte code-pair
//    entry), so a lookup is conflict-free whatever the codes; codes of
//    <= 3 bits are looked up two coordinates at a time. The query rotation
//    q^ = (scale log2 e / d) H (sigma_K (.) q) is done in the prologue, one
//    head per worker wavefront at a time, into LDS.
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
#include "xlane.hpp"

namespace tq {

namespace {

constexpr int kTile = 64;  // tokens per wavefront tile (one per lane)
constexpr float kLog2e = 1.4426950408889634f;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef uint32_t u2v __attribute__((ext_vector_type(2)));  // two dwords, kept in registers

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
// The fp16 form: D[v] += sum_k A_bcast[v][k] * B[lane][k] over the 4 halves
// k of the operands, A taken from block ABID (lane 4 ABID + v).
template <int ABID>
__device__ __forceinline__ v4f mfma16(v4h a, v4h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 4, ABID, 0);
}
__device__ __forceinline__ v4h as_v4h(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(v4h, u2v{lo, hi});
}

// x as an fp16 pair in one dword: the low half is the nearest fp16 of x, the
// high half the nearest fp16 of what remains (x - hi is exact in fp32).
__device__ __forceinline__ uint32_t split_hl(float x) {
  const _Float16 h = (_Float16)x;
  const _Float16 l = (_Float16)(x - (float)h);
  return (uint32_t)__builtin_bit_cast(uint16_t, h) |
         ((uint32_t)__builtin_bit_cast(uint16_t, l) << 16);
}
// 2^e for e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) {
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}
// The exponent e with m * 2^e in [2^13, 2^14) for a positive finite m (0 for
// anything else), clamped to the normal range.
__device__ __forceinline__ int hl_exponent(float m) {
  if (!(m > 0.f) || !(m < INFINITY)) return 0;
  const int e = (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFF) - 127;
  return min(126, max(-126, 13 - e));
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
// Maximum over the wavefront of signed integers, returned in every lane (the
// same DPP pattern; each step one fused v_max_i32_dpp).
__device__ __forceinline__ int wave_max_int(int k) {
  constexpr int kLow = (int)0x80000000;  // identity of the max for the DPP's inactive sources
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x141, 0xF, 0xF, false));  // row_half_mirror
  k = max(k, __builtin_amdgcn_update_dpp(kLow, k, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
             max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
}
// Maximum over the wavefront of finite or -inf scores, returned in every lane:
// the integer maximum of an order-preserving key (the bits, with the
// magnitude bits flipped for negative values), exact and without NaN quieting.
__device__ __forceinline__ float wave_max_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  const int r = wave_max_int(b ^ ((b >> 31) & 0x7FFFFFFF));
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

// Centroid tables live in LDS as one 256-byte row per code (or code pair),
// so that every lane reads its own copy and a lookup never has a bank
// conflict, whatever the codes. A wave64 LDS read is served 32 lanes at a
// time over 32 banks of 4 bytes:
// - 4-byte entries (hi, lo): 64 copies, lane l at dword l;
// - K pair entries (hi, lo, hi', lo'), read as one 8-byte access into the
//   operand pair they feed: 32 interleaved copies, lane l at dwords
//   2 (l % 32) and 2 (l % 32) + 1 (8 bytes per lane fill the 32 banks twice
//   per pass, which is the access's own width, not a conflict);
// - V pair entries, read as two 4-byte accesses that feed two different
//   operands: 32 copies of the first coordinate's (hi, lo) in dwords 0..31
//   and 32 of the second's in 32..63, lane l at dwords l % 32 and
//   32 + l % 32 (interleaved, each 4-byte access would put two lanes of a
//   pass on every even or odd bank).
// A lookup address is (code << 8) | lane_offset.
constexpr int kVPad = 4;  // dwords of padding around a wavefront's staged V rows
// Fourth word of a raw buffer resource on CDNA (32-bit data format, no
// swizzle, no stride): loads past the resource's byte count read zero.
constexpr int kBufferWord3 = 0x00020000;

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
  static constexpr int NVS = VPAIR ? D / 128 : D / 64; // V lookups per lane per token
  static constexpr int RKW = D * KBITS / 32;           // dwords per K row
  static constexpr int RVW = D * BV / 32;              // dwords per V row
  // K operand registers: raw keys take 4 coordinates per product (the row's
  // own fp16 values), coded keys 2 coordinates (hi, lo each)
  static constexpr int QREG = KRAW ? D / 64 : D / 32;  // v4h registers per head group (hi or lo)
  // V rows of a tile staged contiguously in LDS (row t at dword kVPad + t RVW,
  // kVPad dwords of padding on each side), copied there from HBM by the
  // wavefront's own global-to-LDS loads: a lane reads the two dwords around
  // its field, which may reach from the dword before the row to the dword
  // after it (a neighbouring row or padding; those bits are masked off).
  static constexpr int VT_BYTES = (1 << VF) * 256;
  static constexpr int KT_BYTES = KRAW ? 0 : (1 << KF) * 256;
  static constexpr int VS_BYTES = (kTile * RVW + 2 * kVPad) * 4;  // per wavefront
  // global-to-LDS copy of a tile's V rows: 16 bytes per lane when the block
  // is a whole number of 1 KB pieces, else 4 bytes per lane
  static constexpr bool VDMA16 = RVW % 4 == 0;
  static constexpr int VDMA_OPS = VDMA16 ? RVW / 4 : RVW;
  static constexpr int WB_BYTES = kTile * 4 * NHG * 4;  // per wavefront: weights (hi, lo) of a tile
  // rotated queries (and for Prod keys their sketch projections), then one
  // maximum magnitude per virtual head
  static constexpr int QS_BYTES = (PROD ? 2 : 1) * 4 * NHG * D * 4 + 4 * NHG * 4;
  // first-tile arrival flags and the workers' tables-ready counter
  static constexpr int GATE_BYTES = ((WAVES + 1) * 4 + 15) / 16 * 16;
  // The V stages live in an LDS array of their own: the compiler then knows
  // that reads of the tables, weights and queries cannot touch rows still in
  // flight from HBM, and waits for those only before reading a stage.
  static constexpr int STAGE_BYTES = WAVES * VS_BYTES;
  static constexpr int MAIN_BYTES = VT_BYTES + KT_BYTES + WAVES * WB_BYTES + QS_BYTES + GATE_BYTES;
  static constexpr int MERGE_BYTES = (WAVES * 4 * NHG * 3 + 2 * 4 * NHG + WAVES * 4 * NHG * D) * 4;
  static constexpr int SHARED_BYTES = MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES;
  static constexpr int LDS_BYTES = SHARED_BYTES + STAGE_BYTES;  // the workgroup's whole LDS
  // value accumulators per head group and half (hi or lo weights): one per
  // coordinate a lane owns; two (even and odd token pairs) when it owns one
  static constexpr int NACC = (VPAIR ? 2 * NVS : NVS) < 2 ? 2 : (VPAIR ? 2 * NVS : NVS);
};

constexpr int kLdsPerCU = 163840;

// Software-pipeline depths of the tile loop: K coordinate pairs whose
// lookups run ahead of the products, token pairs per batch of the values
// phase.
constexpr int kKAhead = 6;
constexpr int kVBatch = 1;

// Rough count of the VGPRs one lane holds through the tile loop: query
// operands (hi and lo), norms, value accumulators, weight operands and
// softmax state, V field positions, the tile's K row, plus the larger of the
// scores phase (two batches of lookups, four accumulator chains) and the
// values phase (three batches of staged dwords, two of lookups).
template <class B>
constexpr int vgpr_estimate() {
  constexpr int base = B::NHG * B::QREG * 4 + 3 + 2 * B::NACC * B::NHG * 4 + B::NHG * 24 +
                       2 * B::NVS + B::RKW + B::SKW;
  constexpr int kphase = 2 * (kKAhead + 1) + 16 * B::NHG;
  constexpr int vphase = 3 * 2 * kVBatch * B::NVS * 2 + 2 * 2 * kVBatch * B::NVS * (B::VPAIR ? 2 : 1);
  constexpr int prod = B::PROD ? B::NHG * B::D / 16 + 16 * B::NHG : 0;
  return base + prod + (kphase > vphase ? kphase : vphase);
}

// Wavefronts per workgroup: as many as the LDS and the register file allow
// (16, 12, 8 or 4; 128, 168 or 256 VGPRs per lane); the centroid tables are
// shared by all of them.
// The estimate runs about 20 above what the compiler allocates; 148 is the
// largest value whose compiled kernel fits 128 VGPRs without spilling in the
// tile loop (the 32K-context K8/V3 configuration sits just under it).
template <int D, int BK, int BV, int NHG>
constexpr int cfg_waves() {
  using B = CfgBase<D, BK, BV, NHG, 4>;
  constexpr int need = vgpr_estimate<B>() + 16;  // + addresses, temporaries
  if (NHG < 4 && need <= 152 && CfgBase<D, BK, BV, NHG, 16>::LDS_BYTES <= kLdsPerCU) return 16;
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

// One tile's worth of this lane's token in registers: the packed K row and
// the norms (the V rows go straight to LDS).
template <class C>
struct TileRegs {
  uint32_t kw[C::RKW];
  uint32_t sk[C::SKW];  // Prod keys: sketch bits
  float nk, nv, rn;     // rn: Prod keys' residual norm
};
// Vector-memory instructions of one load_k (its vmcnt footprint).
template <class C>
constexpr int k_loads() {
  return 1 + (C::KRAW ? 0 : 1) + (C::PROD ? 1 + C::SKW / 2 : 0) +
         (C::RKW % 4 == 0 ? C::RKW / 4 : C::RKW / 2);
}

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
// Weights are p * nV * 2^(kWeightExp - Ev) < 2^(8 + kWeightExp) (p <= 2^8,
// nV < 2^Ev): below the fp16 maximum with room to spare.
constexpr int kWeightExp = 6;

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
typedef const __attribute__((address_space(3))) uint32_t lds_u32;
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

// s_waitcnt on the LDS (and scalar memory) counter only: lgkmcnt(0).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
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
  __shared__ __attribute__((aligned(16))) unsigned char lds[C::SHARED_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t vstages[C::STAGE_BYTES / 4];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  // the wavefront index is uniform: kept in a scalar register, so that the
  // tile loop's control and the stage address need no vector registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t_begin = split * tokens_per_split;
  // rows [t_begin, t_host) lie inside the cache allocation whatever the
  // device lengths are (max_len <= max_ctx)
  const int t_host = min(max_len, t_begin + tokens_per_split);
  const int G = group;
  const int n_q_heads = n_kv_heads * G;
  // The workgroup serves GV = G * n_qtok virtual heads: virtual head vh is
  // query token vh / G of the sequence for query head g G + vh % G. Query
  // token i of n_qtok sees the rows before len - n_qtok + i + 1 (causal
  // multi-token decode); with one query token that is every row.
  const int GV = G * n_qtok;

  unsigned char* vt = lds;
  unsigned char* kt = lds + C::VT_BYTES;
  uint32_t* vstage = vstages + wave * (C::VS_BYTES / 4);
  uint32_t* wbuf = (uint32_t*)(lds + C::VT_BYTES + C::KT_BYTES + wave * C::WB_BYTES);
  float* wq = (float*)(lds + C::VT_BYTES + C::KT_BYTES + WAVES * C::WB_BYTES);
  float* qmax = wq + (C::PROD ? 2 : 1) * 4 * NHG * D;  // [4 NHG] largest |q^| per virtual head
  int* gate = (int*)(qmax + 4 * NHG);

  const long long kvrow0 = ((long long)b * n_kv_heads + g) * max_ctx;
  const uint32_t* __restrict__ kbase = (const uint32_t*)k_codes + kvrow0 * RKW;
  const uint32_t* __restrict__ vbase = (const uint32_t*)v_codes + kvrow0 * RVW;
  const float* __restrict__ knb = k_norms + kvrow0;
  const float* __restrict__ vnb = v_norms + kvrow0;
  const uint32_t* __restrict__ skb = (const uint32_t*)pa.sketch + kvrow0 * C::SKW;
  const float* __restrict__ rnb = pa.rnorms + kvrow0;

  // ---- a tile's V rows: copied from HBM into this wavefront's LDS stage
  //      in their own layout (rows contiguous), each instruction a coalesced
  //      1 KB (or 256 B) piece; pieces past row `last` re-read the last
  //      valid piece (always in bounds; those rows are never used). The
  //      copies are buffer loads over a resource that spans exactly the
  //      tile's valid rows: unlike the flat-encoded global-to-LDS form they
  //      leave the compiler's count of the wavefront's other loads exact, so
  //      a wait for the next tile's K row does not also wait for these rows.
  auto load_v = [&](int tile, int last) __attribute__((always_inline)) {
    const uint32_t* src = vbase + (long long)tile * RVW;
    auto* dst = (__attribute__((address_space(3))) uint32_t*)(vstage + kVPad);
    if constexpr (C::VDMA16) {
      const int valid = (last - tile + 1) * (RVW / 4);  // 16-byte pieces
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * 16, kBufferWord3);
#pragma unroll
      for (int i = 0; i < C::VDMA_OPS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + 256 * i), 16,
            16 * min(64 * i + lane, valid - 1), 0, 0, 0);
    } else {
      const int valid = (last - tile + 1) * RVW;  // dwords
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, valid * 4, kBufferWord3);
#pragma unroll
      for (int i = 0; i < C::VDMA_OPS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(dst + 64 * i), 4,
            4 * min(64 * i + lane, valid - 1), 0, 0, 0);
    }
  };
  // ---- tile registers: this lane's token's norms and K row. Lanes past
  //      `last` load row `last` instead (always in bounds); their scores are
  //      masked to -inf and their weights are 0, so the rows never contribute.
  //      The norms and the row are requested separately: inside the tile
  //      loop the next tile's row goes out once the scores have consumed the
  //      current one, its norms once the softmax has consumed the current
  //      ones, so that no register holding a current value is also the
  //      target of a load in flight (which would cost a wait for it).
  auto load_norms = [&](int tile, int last, TileRegs<C>& r) __attribute__((always_inline)) {
    const int t = min(tile + lane, last);
    r.nv = vnb[t];
    if constexpr (C::KRAW)
      r.nk = 1.f;
    else
      r.nk = knb[t];
  };
  auto load_krow = [&](int tile, int last, TileRegs<C>& r) __attribute__((always_inline)) {
    const int t = min(tile + lane, last);
    const uint32_t* kr = kbase + (long long)t * RKW;
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
  // a first tile: V rows, norms, then the K row (vector loads complete in
  // order, so the scores can start on the first pieces of the K row while
  // the rest is in flight)
  auto load_tile = [&](int tile, int last, TileRegs<C>& r) __attribute__((always_inline)) {
    load_v(tile, last);
    load_norms(tile, last, r);
    load_krow(tile, last, r);
  };

  // ---- prologue. With more wavefronts than the gate depth, the ungated
  //      ones (0 .. kGateDepth - 1) request their first tile at once, bounded
  //      by the host's row bound (the device length is not waited for); the
  //      others ("workers") fill the LDS tables and rotate the queries while
  //      those tiles stream in. No workgroup barrier follows a tile request:
  //      a wavefront that has requested rows may stall in issuing them for as
  //      long as its CU's share of the bandwidth takes to drain what is ahead,
  //      so every wavefront instead waits for an LDS counter the workers
  //      raise when their part is written. With no more wavefronts than the
  //      gate depth every wavefront is a worker and requests its first tile
  //      once the tables are ready.
  const int nthr = 64 * WAVES;
  constexpr bool kSplitRoles = WAVES > kGateDepth;
  constexpr int kWorkers = kSplitRoles ? WAVES - kGateDepth : WAVES;
  const bool worker = !kSplitRoles || wave >= kGateDepth;
  const int widx = kSplitRoles ? wave - kGateDepth : wave;  // worker index
  const int wtid = threadIdx.x - (kSplitRoles ? 64 * kGateDepth : 0);
  constexpr int kStride = WAVES * kTile;
  const int tile0 = t_begin + wave * kTile;
  TileRegs<C> ra;
  int* ready = gate + WAVES;  // worker wavefronts whose tables and queries are written

  // table entries: 16 threads write one 256-byte row (four 16-byte copies
  // each); a worker thread's entries are wtid, wtid + 64 kWorkers, ...
  constexpr int kVRows = 1 << C::VF, kKRows = C::KRAW ? 0 : 1 << C::KF;
  constexpr int kVEnt = (kVRows * 16 + 64 * kWorkers - 1) / (64 * kWorkers);
  constexpr int kKEnt = (kKRows * 16 + 64 * kWorkers - 1) / (64 * kWorkers);
  constexpr int kHeadsPerWave = (4 * NHG + kWorkers - 1) / kWorkers;  // GV <= 4 NHG
  float vce[kVEnt][2], kce[kKEnt ? kKEnt : 1][2];
  __half qx[kHeadsPerWave][E];
  if (worker) {
    // every small load a worker needs goes out before the barrier below,
    // ahead of any tile row in the CU's memory pipeline (its loads drain
    // roughly in order at its share of the bandwidth)
    auto centroids = [&](const float* c, int bits, bool pair, int rows, float (&dst)[2], int u) {
      const int e = min(wtid + u * 64 * kWorkers, rows * 16 - 1) >> 4;  // in bounds
      const int mask = (1 << bits) - 1;
      dst[0] = c[pair ? (e & mask) : e];
      dst[1] = pair ? c[e >> bits] : 0.f;
    };
#pragma unroll
    for (int u = 0; u < kVEnt; ++u) centroids(tabs.v_centroids, C::BV, C::VPAIR, kVRows, vce[u], u);
#pragma unroll
    for (int u = 0; u < kKEnt; ++u)
      centroids(tabs.k_centroids, C::KBITS, C::KPAIR, kKRows, kce[u], u);
#pragma unroll
    for (int r = 0; r < kHeadsPerWave; ++r) {
      const int h = min(widx + r * kWorkers, GV - 1);  // in bounds; surplus rows unused
      const int qi = h / G;
      const __half* qrow =
          q + (((long long)b * n_qtok + qi) * n_q_heads + (long long)g * G + (h - qi * G)) * D;
#pragma unroll
      for (int e = 0; e < E; ++e) qx[r][e] = qrow[E * lane + e];
    }
  }
  if (threadIdx.x <= WAVES) gate[threadIdx.x] = 0;
  lds_barrier();  // flags and counter cleared; the workers' small loads issued
  if (kSplitRoles && !worker && tile0 < t_host) load_tile(tile0, t_host - 1, ra);

  if (worker) {
    // table rows of (hi, lo) entries
    // (16-byte piece i of the table: row i / 16, piece i % 16 of that row)
    auto fill = [&](unsigned char* tab, int rows, bool pair, bool halves, float cs,
                    const float (&ce)[2], int u) {
      const int i = wtid + u * 64 * kWorkers;
      if (i < rows * 16) {
        const uint32_t a = split_hl(ce[0] * cs);
        const uint32_t bb = pair ? split_hl(ce[1] * cs) : a;
        if (halves)  // pieces 0..7: the first coordinate's entry, 8..15: the second's
          ((uint4*)tab)[i] = (i & 15) < 8 ? uint4{a, a, a, a} : uint4{bb, bb, bb, bb};
        else
          ((uint4*)tab)[i] = uint4{a, bb, a, bb};
      }
    };
#pragma unroll
    for (int u = 0; u < kVEnt; ++u) fill(vt, kVRows, C::VPAIR, C::VPAIR, tabs.v_scale, vce[u], u);
#pragma unroll
    for (int u = 0; u < kKEnt; ++u) fill(kt, kKRows, C::KPAIR, false, tabs.k_scale, kce[u], u);

    // rotated queries: worker w rotates heads w, w + kWorkers, ... into LDS
    // and records each one's largest magnitude
    // sign word of this lane's coordinates E lane .. E lane + E - 1 (one word:
    // E <= 4 consecutive coordinates never straddle a 32-bit boundary)
    uint32_t sword = 0;
#pragma unroll
    for (int w = 0; w < D / 32; ++w)
      if ((E * lane) >> 5 == w) sword = ksign.bits[w];
#pragma unroll
    for (int r = 0; r < kHeadsPerWave; ++r) {
      const int h = widx + r * kWorkers;
      if (h < GV) {
        float u[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = E * lane + e;
          const float x = __half2float(qx[r][e]);
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
        if constexpr (!C::KRAW) {
          sfor<6>([&](auto MI) {
            constexpr int m = 1 << MI;
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float p = xor_lane_f32<m>(u[e]);
              u[e] = upper ? (p - u[e]) : (u[e] + p);
            }
          });
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float v = u[e] * qscale;
          wq[h * D + E * lane + e] = v;
          amax = fmaxf(amax, fabsf(v));
        }
        amax = wave_max(amax);
        if (lane == 0) qmax[h] = amax;
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
          sfor<6>([&](auto MI) {
            constexpr int m = 1 << MI;
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float p = xor_lane_f32<m>(u[e]);
              u[e] = upper ? (p - u[e]) : (u[e] + p);
            }
          });
#pragma unroll
          for (int e = 0; e < E; ++e) wq[4 * NHG * D + h * D + E * lane + e] = u[e] * pa.uscale;
        }
      }
    }
    // this wavefront's table rows and queries are written: count it
    wait_lgkmcnt0();
    if (lane == 0) __hip_atomic_fetch_add(ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  // every wavefront: wait until all workers have written their part (a
  // bounded wait: a wavefront that gives up computes with what is there)
  {
    const uint32_t ra_addr = lds_addr(ready);
    for (int i = 0; i < kGateSpins && flag_read(ra_addr) < kWorkers; ++i) __builtin_amdgcn_s_sleep(1);
  }
  if (!kSplitRoles && wave < kGateDepth && tile0 < t_host) load_tile(tile0, t_host - 1, ra);

  // the device length: a workgroup whose range starts past it has nothing
  // to do (its early rows, if requested, are drained first)
  const int len = min(lengths[b], max_len);  // never read past the host bound
  if (t_begin >= len) {
    wait_vmcnt<0>();
    return;  // whole workgroup
  }
  const int t_end = min(len, t_host);

  // one power-of-two scale for the workgroup's queries
  float qm = 0.f;
  for (int h = 0; h < GV; ++h) qm = fmaxf(qm, qmax[h]);
  const int sq = hl_exponent(qm);
  const float qs2 = exp2i(sq);
  // score units: undo the query and key-table scales
  const float kunscale = exp2i(-sq) * (C::KRAW ? 1.f : 1.f / tabs.k_scale);

  // query operands in the broadcast layout. Coded keys: lane 4c + v of
  // QH[hg][m] holds (qh_j, qh_j, qh_j', qh_j') and of QL[hg][m] (ql_j, 0,
  // ql_j', 0) for virtual head 4 hg + v and coordinates j = 32 m + 2c,
  // j' = j + 1. Raw keys: lane 4c + v holds coordinates 64 m + 4c .. + 3.
  v4h QH[NHG][C::QREG], QL[NHG][C::QREG];
  float U[C::PROD ? NHG : 1][C::PROD ? D / 16 : 1];  // Prod keys: sketch projections
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    const int h = 4 * hg + (lane & 3);
    const int c = lane >> 2;
#pragma unroll
    for (int m = 0; m < C::QREG; ++m) {
      if constexpr (C::KRAW) {
        const float4 x = h < GV ? *(const float4*)(wq + h * D + 64 * m + 4 * c)
                                : float4{0.f, 0.f, 0.f, 0.f};
        const uint32_t a0 = split_hl(x.x * qs2), a1 = split_hl(x.y * qs2);
        const uint32_t a2 = split_hl(x.z * qs2), a3 = split_hl(x.w * qs2);
        QH[hg][m] = as_v4h(__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                           __builtin_amdgcn_perm(a3, a2, 0x05040100u));
        QL[hg][m] = as_v4h(__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                           __builtin_amdgcn_perm(a3, a2, 0x07060302u));
      } else {
        const float2 x = h < GV ? *(const float2*)(wq + h * D + 32 * m + 2 * c) : float2{0.f, 0.f};
        const uint32_t a0 = split_hl(x.x * qs2), a1 = split_hl(x.y * qs2);
        QH[hg][m] = as_v4h(__builtin_amdgcn_perm(a0, a0, 0x01000100u),
                           __builtin_amdgcn_perm(a1, a1, 0x01000100u));
        QL[hg][m] = as_v4h(a0 >> 16, a1 >> 16);
      }
    }
    if constexpr (C::PROD) {
      const int hh = 4 * hg + (lane & 3);
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        U[hg][m] = hh < GV ? wq[4 * NHG * D + hh * D + 16 * m + (lane >> 2)] : 0.f;
    }
  }

  // a wavefront past the range end (short ranges) has no tile: it requests
  // nothing more and waits for no gate (the later ones have none either)
  const bool has_tile = tile0 < t_end;
  // The gated wavefronts request their first tile once the first tile of
  // wavefront w - kGateDepth has arrived. No workgroup barrier follows until
  // the merge: a wavefront may stall in issuing vector loads while the memory
  // pipeline is full, and each one runs its tiles independently.
  if (wave >= kGateDepth && has_tile) {
    const uint32_t ga = lds_addr(gate + (wave - kGateDepth));
    for (int i = 0; i < kGateSpins && flag_read(ga) == 0; ++i) __builtin_amdgcn_s_sleep(1);
    load_tile(tile0, t_end - 1, ra);
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

  // ---- per-wave online-softmax state. acc[0] collects the products with
  //      the weights' high halves, acc[LO] with their low halves.
  float m_run[NHG][4];
  v4f l_run[NHG];
  // The high- and low-half products of an operand go into one accumulator
  // (and one score chain per product parity below): the chains of the
  // accumulators, parities and head groups are enough to keep the matrix
  // unit busy. Separate chains for the two halves (HL = 2) measured no
  // faster with one head group and slower with two, and with four head
  // groups they spill. HL accumulator sets, LO the low halves' set.
  constexpr int HL = 1, LO = HL - 1;
  v4f acc[HL][C::NACC][NHG];
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg) {
    l_run[hg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) m_run[hg][v] = kNoRow;
#pragma unroll
    for (int a = 0; a < C::NACC; ++a) acc[0][a][hg] = acc[LO][a][hg] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // every V norm seen so far is below 2^ev (ev only grows)
  int ev = 0;
  bool seen = false;  // a tile has been processed (the accumulators may be nonzero)

  const uint32_t koff = C::KPAIR ? (uint32_t)(lane & 31) << 3 : (uint32_t)lane << 2;
  const uint32_t voff = C::VPAIR ? (uint32_t)(lane & 31) << 2 : (uint32_t)lane << 2;
  constexpr uint32_t KMASK = ((1u << C::KF) - 1u) << 8;
  constexpr uint32_t VMASK = ((1u << C::VF) - 1u) << 8;

  // V fields of this lane: field 64k + lane of each staged row, read from bit
  // o - 8 of the padded row so the field lands at bit 8. The two dwords
  // around it are read through separate base addresses the compiler cannot
  // relate (so it neither merges the reads into one register pair nor needs
  // an address add per row: every row is a constant offset from them), and
  // so are the two dwords of a V pair entry, each of which feeds its own
  // product.
  uint32_t va0[C::NVS], va1[C::NVS];
  int vsh[C::NVS];
#pragma unroll
  for (int k = 0; k < C::NVS; ++k) {
    const int o = C::VF * (64 * k + lane) + 32 * kVPad - 8;
    va0[k] = lds_addr(vstage) + 4 * (o >> 5);
    va1[k] = va0[k] + 4;
    asm("" : "+v"(va1[k]));
    vsh[k] = o & 31;
  }
  uint32_t voff_y = voff + 128, vmask_y = VMASK;  // opaque copies: one v_and_or per address
  asm("" : "+v"(voff_y));
  asm("" : "+s"(vmask_y));

  // One tile: scores, online softmax, values. With MORE (another tile of
  // this wavefront follows) `r` is refilled with the next tile as soon as
  // its rows have been used, and the next V rows are requested once the
  // stage has been read. MORE is a compile-time property of the call, so
  // every load of a tile is issued on one path: the compiler then counts the
  // loads in flight exactly and waits for each register only as long as it
  // must.
  auto process = [&](int tile, TileRegs<C>& r, auto MORE) __attribute__((always_inline)) {

    // ---- scores on the matrix cores: per coordinate pair (raw keys: per
    //      four coordinates) one product with the high and one with the low
    //      halves of the queries, into four accumulator chains. The lookups
    //      of batch j + 1 are issued before the products of batch j, so a
    //      batch's LDS latency hides behind the previous batch's products.
    // score chains: per parity of the product index, the high and the low
    // halves' products (one chain per parity when HL == 1)
    constexpr int SCN = 2 * HL;
    v4f sc[SCN][NHG];
#pragma unroll
    for (int a4 = 0; a4 < SCN; ++a4)
#pragma unroll
      for (int hg = 0; hg < NHG; ++hg) sc[a4][hg] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (C::KRAW) {
      // coordinates 4f .. 4f + 3 of the raw key row are dwords 2f, 2f + 1
      sfor<D / 4>([&](auto FI) {
        constexpr int f = FI;
        const v4h kb = as_v4h(r.kw[2 * f], r.kw[2 * f + 1]);
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg) {
          sc[HL * (f % 2)][hg] = mfma16<f % 16>(QH[hg][f / 16], kb, sc[HL * (f % 2)][hg]);
          sc[HL * (f % 2) + LO][hg] = mfma16<f % 16>(QL[hg][f / 16], kb, sc[HL * (f % 2) + LO][hg]);
        }
      });
    } else {
      constexpr int NKP = D / 2;  // coordinate pairs
      // rolling pipeline: the lookups of pair p + kKAhead are issued before
      // the products of pair p, so up to 2 kKAhead lookups are in flight
      u2v kl[kKAhead + 1];
      auto k_lookup = [&](auto PI) __attribute__((always_inline)) {
        constexpr int p = PI;
        u2v& dst = kl[p % (kKAhead + 1)];
        if constexpr (C::KPAIR) {
          const uint32_t addr = (field_at8<C::KF * p, C::KF>(r.kw) & KMASK) | koff;
          dst = u2v{*(const uint32_t*)(kt + addr), *(const uint32_t*)(kt + addr + 4)};
        } else {
          uint32_t a2[2];
          sfor<2>([&](auto SI) {
            constexpr int j = 2 * p + SI;
            constexpr int bit = C::KF * j;
            if constexpr (C::KF == 8) {
              // whole byte: one byte permute builds (code << 8) | koff
              a2[SI] = __builtin_amdgcn_perm(r.kw[bit >> 5], koff,
                                             0x0C0C0000u | ((4u + ((bit >> 3) & 3)) << 8));
            } else {
              a2[SI] = (field_at8<bit, C::KF>(r.kw) & KMASK) | koff;
            }
          });
          dst = u2v{*(const uint32_t*)(kt + a2[0]), *(const uint32_t*)(kt + a2[1])};
        }
      };
      auto k_mfma = [&](auto PI) __attribute__((always_inline)) {
        constexpr int p = PI;
        const u2v& src = kl[p % (kKAhead + 1)];
        const v4h kb = as_v4h(src.x, src.y);
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg) {
          sc[HL * (p % 2)][hg] = mfma16<p % 16>(QH[hg][p / 16], kb, sc[HL * (p % 2)][hg]);
          sc[HL * (p % 2) + LO][hg] = mfma16<p % 16>(QL[hg][p / 16], kb, sc[HL * (p % 2) + LO][hg]);
        }
      };
      sfor<NKP + kKAhead>([&](auto I) {
        constexpr int i = I;
        if constexpr (i < NKP) k_lookup(std::integral_constant<int, i>{});
        if constexpr (i >= kKAhead) k_mfma(std::integral_constant<int, i - kKAhead>{});
      });
    }
    v4f s0[NHG];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
      if constexpr (HL == 2)
        s0[hg] = ((sc[0][hg] + sc[1][hg]) + (sc[SCN - 2][hg] + sc[SCN - 1][hg])) * kunscale;
      else
        s0[hg] = (sc[0][hg] + sc[SCN - 1][hg]) * kunscale;
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

    // a lane past the range end holds a repeated (or, for a first tile
    // requested before the length was known, an unused) row: weight 0
    const bool live = tile + lane < t_end;
    const float nv_cur = live ? r.nv : 0.f;
    const float nk_cur = r.nk;
    // the K row is consumed: refill it with this wavefront's next tile's
    // (its norms follow after the softmax, its V rows once this tile's stage
    // has been read)
    const int ahead = tile + kStride;
    constexpr bool more = decltype(MORE)::value;
    if constexpr (more) load_krow(ahead, t_end - 1, r);

    // V norm scale: every norm below 2^ev (rare: usually the first tile only)
    if (__ballot(__builtin_bit_cast(int, nv_cur) >= ((ev + 127) << 23)) != 0ull) {
      const int mx = wave_max_int(__builtin_bit_cast(int, nv_cur));
      const int en = min(120, ((mx >> 23) & 0xFF) - 127 + 1);
      if (seen) {  // before the first tile the accumulators are zero
        const float f = exp2i(max(-126, ev - en));
#pragma unroll
        for (int hl = 0; hl < HL; ++hl)
#pragma unroll
          for (int a = 0; a < C::NACC; ++a)
#pragma unroll
            for (int hg = 0; hg < NHG; ++hg) acc[hl][a][hg] *= f;
      }
      ev = en;
    }
    seen = true;
    const float wmul = nv_cur * exp2i(kWeightExp - ev);

    // ---- online softmax (base 2) with a lazily moved maximum
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const v4f s = s0[hg] * nk_cur;
      uint32_t w[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float sv = tile + lane < vlim[hg][v] ? s[v] : -INFINITY;
        // the tile maximum exceeds m_run + slack iff some lane's score does:
        // one compare and a ballot decide it, and the maximum itself is only
        // taken then (always on a wavefront's first tile, rarely after)
        if (__ballot(sv > m_run[hg][v] + kRescaleSlack) != 0ull) {  // wavefront-uniform
          const float mt = wave_max_key(sv);
          // a head that has seen no row yet has zero sums: nothing to rescale
          if (m_run[hg][v] != kNoRow) {
            const float alpha = __builtin_amdgcn_exp2f(m_run[hg][v] - mt);
            l_run[hg][v] *= alpha;
#pragma unroll
            for (int hl = 0; hl < HL; ++hl)
#pragma unroll
              for (int a = 0; a < C::NACC; ++a) acc[hl][a][hg][v] *= alpha;
          }
          m_run[hg][v] = mt;
        }
        const float p = __builtin_amdgcn_exp2f(sv - m_run[hg][v]);
        l_run[hg][v] += p;
        w[v] = split_hl(p * wmul);
      }
      *(uint4*)(wbuf + (lane * NHG + hg) * 4) = uint4{w[0], w[1], w[2], w[3]};
    }
    if constexpr (more) load_norms(ahead, t_end - 1, r);
    wave_lds_sync();

    // this tile's V rows are in the stage: they were requested before its K
    // row, whose loads have completed (only the refill may be in flight)
    if constexpr (more)
      wait_vmcnt<k_loads<C>()>();
    else
      wait_vmcnt<0>();

    // weights in the broadcast layout: lane 4c + v of WH[hg][m] holds
    // (wh_t, wh_t, wh_t', wh_t') and of WL[hg][m] (wl_t, 0, wl_t', 0) for
    // virtual head 4 hg + v and tokens t = 2 (16 m + c), t' = t + 1
    v4h WH[NHG][2], WL[NHG][2];
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int t0 = 2 * (16 * m + (lane >> 2));
        const uint32_t x0 = wbuf[(t0 * NHG + hg) * 4 + (lane & 3)];
        const uint32_t x1 = wbuf[((t0 + 1) * NHG + hg) * 4 + (lane & 3)];
        WH[hg][m] = as_v4h(__builtin_amdgcn_perm(x0, x0, 0x01000100u),
                           __builtin_amdgcn_perm(x1, x1, 0x01000100u));
        WL[hg][m] = as_v4h(x0 >> 16, x1 >> 16);
      }

    // ---- values on the matrix cores, lanes over coordinates, two tokens
    //      per product. Three stages over batches of token pairs: the staged
    //      dwords around this lane's fields (two batches ahead), the centroid
    //      entries (one batch ahead), the products.
    // a pair entry is read as its two dwords (x: the first coordinate's
    // (hi, lo), y: the second's), each straight into the operand it feeds
    constexpr int TB = kVBatch, NTB = kTile / 2 / TB;
    // A batch's lookups: pair entries per (token pair, token, lookup) as
    // their two dwords; single entries per (token pair, lookup) as the two
    // tokens' dwords, which is the operand pair they feed (held any other
    // way, the compiler has paired them through a stack round trip).
    struct VLuts {
      std::conditional_t<C::VPAIR, u2v[TB][2][C::NVS], u2v[TB][C::NVS]> e;
    };
    auto v_stage = [&](auto JI, u2v (&dst)[TB][2][C::NVS]) __attribute__((always_inline)) {
      sfor<TB>([&](auto TI) {
        sfor<2>([&](auto SI) {
          constexpr int t = 2 * (JI * TB + TI) + SI;
#pragma unroll
          for (int k = 0; k < C::NVS; ++k)
            dst[TI][SI][k] = u2v{*(const lds_u32*)(uintptr_t)(va0[k] + 4 * t * RVW),
                                 *(const lds_u32*)(uintptr_t)(va1[k] + 4 * t * RVW)};
        });
      });
    };
    auto v_lookup = [&](const u2v (&xs)[TB][2][C::NVS], VLuts& dst) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < TB; ++tt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int k = 0; k < C::NVS; ++k) {
            const uint32_t x = __builtin_amdgcn_alignbit(xs[tt][s][k].y, xs[tt][s][k].x, vsh[k]);
            const uint32_t a = (x & VMASK) | voff;
            if constexpr (C::VPAIR) {
              dst.e[tt][s][k] = u2v{*(const uint32_t*)(vt + a),
                                    *(const uint32_t*)(vt + ((x & vmask_y) | voff_y))};
            } else {
              if (s == 0)
                dst.e[tt][k].x = *(const uint32_t*)(vt + a);
              else
                dst.e[tt][k].y = *(const uint32_t*)(vt + a);
            }
          }
    };
    auto v_mfma = [&](auto JI, const VLuts& cs) __attribute__((always_inline)) {
      sfor<TB>([&](auto TI) {
        constexpr int tp = JI * TB + TI;  // token pair
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) {
          if constexpr (C::VPAIR) {
            const v4h b0 = as_v4h(cs.e[TI][0][k].x, cs.e[TI][1][k].x);
            const v4h b1 = as_v4h(cs.e[TI][0][k].y, cs.e[TI][1][k].y);
#pragma unroll
            for (int hg = 0; hg < NHG; ++hg) {
              acc[0][2 * k][hg] = mfma16<tp % 16>(WH[hg][tp / 16], b0, acc[0][2 * k][hg]);
              acc[LO][2 * k][hg] = mfma16<tp % 16>(WL[hg][tp / 16], b0, acc[LO][2 * k][hg]);
              acc[0][2 * k + 1][hg] = mfma16<tp % 16>(WH[hg][tp / 16], b1, acc[0][2 * k + 1][hg]);
              acc[LO][2 * k + 1][hg] = mfma16<tp % 16>(WL[hg][tp / 16], b1, acc[LO][2 * k + 1][hg]);
            }
          } else {
            constexpr int par = (C::NVS == 1) ? (tp & 1) : 0;
            const v4h bv = __builtin_bit_cast(v4h, cs.e[TI][k]);
#pragma unroll
            for (int hg = 0; hg < NHG; ++hg) {
              acc[0][k + par][hg] = mfma16<tp % 16>(WH[hg][tp / 16], bv, acc[0][k + par][hg]);
              acc[LO][k + par][hg] = mfma16<tp % 16>(WL[hg][tp / 16], bv, acc[LO][k + par][hg]);
            }
          }
        }
      });
    };
    {
      u2v xs0[TB][2][C::NVS], xs1[TB][2][C::NVS], xs2[TB][2][C::NVS];
      VLuts cv0, cv1;
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
    if constexpr (more) {
      // every read of the stage has returned before it is overwritten
      wait_lgkmcnt0();
      load_v(ahead, t_end - 1);
    }
  };

  // every tile but the wavefront's last prefetches the next one
  if (has_tile) {
    int tile = tile0;
    for (; tile + kStride < t_end; tile += kStride) process(tile, ra, std::true_type{});
    process(tile, ra, std::false_type{});
  }

  // ---- merge the wavefronts of this workgroup and write the split partial:
  //      every wavefront stores its maxima, sums and accumulators (brought to
  //      true scale); one lane per virtual head then takes the maximum M
  //      over the wavefronts, their factors 2^(m_w - M) and the folded sum
  //      (a wavefront that saw no row has the finite sentinel maximum, so it
  //      weighs 0 next to one that did), and thread (virtual head,
  //      coordinate) folds the accumulators with those factors
  const float aunscale = exp2i(ev - kWeightExp) / tabs.v_scale;
  v4f accf[C::NACC][NHG];
#pragma unroll
  for (int a = 0; a < C::NACC; ++a)
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg)
      accf[a][hg] = (HL == 2 ? acc[0][a][hg] + acc[LO][a][hg] : acc[0][a][hg]) * aunscale;
  if constexpr (C::NVS == 1 && !C::VPAIR) {
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) accf[0][hg] += accf[1][hg];
  }
  __syncthreads();  // all wavefronts are done with tables and buffers
  constexpr int NV = 4 * NHG;                   // virtual-head slots per wavefront
  float* mbuf = (float*)lds;                    // [NV][WAVES] maxima
  float* lbuf = mbuf + NV * WAVES;              // [NV][WAVES] sums
  float* fbuf = lbuf + NV * WAVES;              // [NV][WAVES] factors 2^(m_w - M)
  float* tot = fbuf + NV * WAVES;               // [NV][2] M and the folded sum
  float* abuf = tot + 2 * NV;                   // [WAVES][NV][D] accumulators
#pragma unroll
  for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lsum = wave_sum(l_run[hg][v]);
      if (lane == 0) {
        mbuf[(4 * hg + v) * WAVES + wave] = m_run[hg][v];
        lbuf[(4 * hg + v) * WAVES + wave] = lsum;
      }
      float* dst = abuf + (wave * NV + 4 * hg + v) * D;
      if constexpr (C::VPAIR) {
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) {
          dst[2 * (64 * k + lane)] = accf[2 * k][hg][v];
          dst[2 * (64 * k + lane) + 1] = accf[2 * k + 1][hg][v];
        }
      } else {
#pragma unroll
        for (int k = 0; k < C::NVS; ++k) dst[64 * k + lane] = accf[k][hg][v];
      }
    }
  __syncthreads();
  if (wave == 0 && lane < GV) {
    const int h = lane;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mbuf[h * WAVES + w]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      // m_w - M <= 0: the hardware exponential (0 far below; 1 for the maximum)
      const float f = __builtin_amdgcn_exp2f(mbuf[h * WAVES + w] - M);
      fbuf[h * WAVES + w] = f;
      L += f * lbuf[h * WAVES + w];
    }
    tot[2 * h] = M;
    tot[2 * h + 1] = L;
  }
  __syncthreads();
  const int S = gridDim.x;
  // D >= 64: a wavefront's threads share one virtual head
  for (int idx = threadIdx.x; idx < NV * D; idx += 64 * WAVES) {
    const int h = idx / D, j = idx - h * D;
    if (h >= GV) continue;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) a += fbuf[h * WAVES + w] * abuf[(w * NV + h) * D + j];
    const long long prow = (((long long)b * n_kv_heads + g) * GV + h) * S + split;
    part_acc[prow * D + j] = a;
    if (j == 0) {
      part_ml[prow * 2] = tot[2 * h];
      part_ml[prow * 2 + 1] = tot[2 * h + 1];
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
  static_assert(RL == 16, "the raw-row score sums over 4 lane-xor steps");
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
    // every exponent below is <= 0 (or -inf): the hardware exponential
    if (mnew != mg) {  // mnew > mg: rescale (by 0 while mg is still -inf)
      const float r = __builtin_amdgcn_exp2f(mg - mnew);
      a *= r;
      L *= r;
      mg = mnew;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) {
        const float f = __builtin_amdgcn_exp2f(mv[u] - mg);
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
      sfor<4>([&](auto MI) { sc += xor_lane_f32<1 << MI>(sc); });
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
        pp[u] = t0 + u * NG < R ? __builtin_amdgcn_exp2f(s_raw[t] - mr) : 0.f;
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
      fg[g2] = s_m[g2] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[g2] - M);
      Lt = fmaf(fg[g2], s_l[g2], Lt);
    }
    const float fr = kRaw && mr != -INFINITY ? __builtin_amdgcn_exp2f(mr - M) : 0.f;
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
    // (cross-lane steps on DPP and permlane swaps: wavefront 0 is whole)
    sfor<6>([&](auto MI) {
      constexpr int m = 1 << MI;
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float p = xor_lane_f32<m>(u[e]);
        u[e] = upper ? (p - u[e]) : (u[e] + p);
      }
    });
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
    TQ_SPLIT(64, 35, 4, 1), TQ_SPLIT(64, 4, 2, 1), TQ_SPLIT(64, 4, 3, 1),
    TQ_SPLIT(64, 16, 2, 1),
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
    TQ_SPLIT(256, 8, 4, 1), TQ_SPLIT(256, 2, 2, 2), TQ_SPLIT(256, 4, 2, 1),
    TQ_SPLIT(256, 4, 3, 1),
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

// 2^e with max |c| * 2^e in [2^13, 2^14) (1 for an all-zero table).
float table_scale(const float* c, int n) {
  float m = 0.f;
  for (int i = 0; i < n; ++i) m = std::fmax(m, std::fabs(c[i]));
  if (!(m > 0.f) || !std::isfinite(m)) return 1.f;
  int e;
  std::frexp(m, &e);  // m = f * 2^e, f in [0.5, 1): m in [2^(e-1), 2^e)
  return std::ldexp(1.f, 14 - e);
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
  // codebook scales: powers of two taking each table's largest magnitude
  // into [2^13, 2^14), so both fp16 halves of every entry are normal numbers
  AttendTables t2 = tabs;
  const int kb = k_bits >= 32 ? k_bits - 32 : k_bits;
  t2.k_scale = k_bits == 16 ? 1.f : table_scale(tabs.k_centroids, 1 << kb);
  t2.v_scale = table_scale(tabs.v_centroids, 1 << v_bits);
  err = fn(plan, batch, n_kv_heads, group, n_qtok, q, k_codes, k_norms, v_codes, v_norms, lengths,
           max_ctx, max_len, qscale, pacc, pml, t2, k_sign, pa, ev_before, ev_after, stream);
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

// codec.hpp -- codec tables shared by the host code and the kernel launchers.
#pragma once
#include <cstdint>

namespace tq {

constexpr int kMaxDim = 256;
constexpr int kMaxLevels = 256;

// Sign vector as a bitmask (bit j set = sign -1) and fp32 Lloyd-Max tables.
// A TurboQuant-Prod key codec (prod) quantises with bits = total - 1 and adds
// a 1-bit sketch of the residual under H diag(sketch signs).
struct CodecTables {
  int dim;
  int bits;                       // Lloyd-Max bits (the MSE part for prod)
  uint64_t seed;
  uint32_t sign_bits[kMaxDim / 32];
  float centroids[kMaxLevels];
  float boundaries[kMaxLevels];   // 2^bits - 1 used
  bool prod;
  uint32_t sketch_sign_bits[kMaxDim / 32];
};

uint64_t splitmix64_next(uint64_t* state);
bool build_codec(int dim, int bits, uint64_t seed, CodecTables* out);
// total_bits in [2, 8]: (total_bits - 1)-bit Lloyd-Max part, sketch signs from
// the SplitMix64 stream of seed + 1.
bool build_prod_codec(int dim, int total_bits, uint64_t seed, CodecTables* out);

}  // namespace tq

// codec.hpp -- codec tables shared by the host code and the kernel launchers.
#pragma once
#include <cstdint>

namespace tq {

constexpr int kMaxDim = 256;
constexpr int kMaxLevels = 256;

// Sign vector as a bitmask (bit j set = sign -1) and fp32 Lloyd-Max tables.
struct CodecTables {
  int dim;
  int bits;
  uint64_t seed;
  uint32_t sign_bits[kMaxDim / 32];
  float centroids[kMaxLevels];
  float boundaries[kMaxLevels];   // 2^bits - 1 used
};

uint64_t splitmix64_next(uint64_t* state);
bool build_codec(int dim, int bits, uint64_t seed, CodecTables* out);

}  // namespace tq

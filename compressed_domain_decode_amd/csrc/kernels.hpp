// kernels.hpp -- kernel argument blocks and launcher declarations (host side).
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace tq {

// Everything a kernel needs from a codec, passed by value in the kernel
// arguments (read through the scalar cache; copied to LDS where indexed).
struct SignArg {
  uint32_t bits[8];            // bit j set: sign_j = -1
};
struct EncodeTables {
  SignArg sign;
  float boundaries[256];
};
struct AttendTables {
  float k_centroids[256];
  float v_centroids[256];
};

struct AttendPlan {
  int splits;                  // context splits per (batch, kv head)
  int tokens_per_split;        // multiple of the tile size
  size_t qhat_bytes;
  size_t part_acc_bytes;
  size_t part_ml_bytes;
  size_t total_bytes;
};

AttendPlan plan_attend(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len);

// Launchers: return hipSuccess or the launch error. Shapes are validated by
// the caller (the C ABI layer) before these are reached.
hipError_t launch_encode(int dim, int bits, const void* x, int n_tok, int n_head,
                         int64_t xs_tok, int64_t xs_head, uint8_t* codes, int64_t cs_tok,
                         int64_t cs_head, float* norms, int64_t ns_tok, int64_t ns_head,
                         const EncodeTables& tabs, hipStream_t stream);

bool attend_supported(int dim, int k_bits, int v_bits, int group);

hipError_t launch_attend(int dim, int k_bits, int v_bits, int batch, int n_q_heads,
                         int n_kv_heads, const void* q, const SignArg& k_sign,
                         const SignArg& v_sign, const AttendTables& tabs,
                         const uint8_t* k_codes, const float* k_norms,
                         const uint8_t* v_codes, const float* v_norms, int max_ctx,
                         const int32_t* lengths, int max_len, float scale, float* out,
                         void* workspace, const AttendPlan& plan, hipEvent_t ev_before,
                         hipEvent_t ev_after, hipStream_t stream);

// Plain streaming read of `bytes` (a multiple of 16) at buf (16-byte aligned).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace tq

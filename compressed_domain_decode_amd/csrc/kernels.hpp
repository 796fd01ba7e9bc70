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
// One set of n_tok x n_head vectors to encode with one codec.
struct EncodeJob {
  const void* x;               // fp16; vector (t, h) at element t*xs_tok + h*xs_head
  long long xs_tok, xs_head;
  uint8_t* codes;              // row (t, h) at byte t*cs_tok + h*cs_head (4-byte aligned)
  long long cs_tok, cs_head;
  float* norms;                // norm (t, h) at element t*ns_tok + h*ns_head
  long long ns_tok, ns_head;
  int bits;
  int prod;                    // TurboQuant-Prod keys: also the residual sketch and norm
  SignArg sign;
  float boundaries[256];       // 2^bits - 1 used; for prod, the centroids from [128]
  uint8_t* sketch;             // prod: row (t, h) at byte t*ss_tok + h*ss_head, dim/8 bytes
  long long ss_tok, ss_head;
  float* rnorms;               // prod: residual norm (t, h) at element t*rs_tok + h*rs_head
  long long rs_tok, rs_head;
  SignArg sketch_sign;
};
constexpr int kMaxEncodeJobs = 2;
struct EncodeArgs {
  int n_tok, n_head;           // n_tok * n_head < 2^31
  int n_jobs;                  // 1 .. kMaxEncodeJobs, all of the same dim
  uint32_t head_magic;         // t = (v * head_magic) >> head_shift equals v / n_head
  uint32_t head_shift;         //   for 0 <= v < 2^31 (set by launch_encode)
  int pad_;
  EncodeJob job[kMaxEncodeJobs];
};
struct AttendTables {
  float k_centroids[256];
  float v_centroids[256];
  float k_scale = 1.f, v_scale = 1.f;  // powers of two applied to the tables on the device
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

// TurboQuant-Prod keys' extra cache arrays (sketch == nullptr: plain keys):
// sketch rows [batch][n_kv_heads][max_ctx][dim/8] (16-byte aligned) and
// residual norms [batch][n_kv_heads][max_ctx]; sign: the sketch signs.
struct ProdKeys {
  const uint8_t* sketch = nullptr;
  const float* rnorms = nullptr;
  SignArg sign{};
};

// Raw fp16 rows attended together with the packed cache (lengths == nullptr:
// none). k and v are [batch][n_kv_heads][max_raw][dim], 16-byte aligned.
struct RawSegment {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* lengths = nullptr;
  int max_raw = 0;
};

// Launchers: return hipSuccess or the launch error. Shapes are validated by
// the caller (the C ABI layer) before these are reached.
// All jobs of one call go out in a single launch. Fails with
// hipErrorInvalidValue if the grid would exceed 2^31 - 1 workgroups.
hipError_t launch_encode(int dim, EncodeArgs& args, hipStream_t stream);

bool attend_supported(int dim, int k_bits, int v_bits, int group);

// k_bits: 1..8 plain codes, 16 raw fp16 keys, 32 + m TurboQuant-Prod keys with
// m-bit codes (prodk then set).
// n_qtok query tokens per sequence (q and out [batch][n_qtok][n_q_heads][dim]),
// causal among themselves; plan sized for n_q_heads * n_qtok heads.
hipError_t launch_attend(int dim, int k_bits, int v_bits, int batch, int n_qtok, int n_q_heads,
                         int n_kv_heads, const void* q, const SignArg& k_sign,
                         const SignArg& v_sign, const AttendTables& tabs,
                         const uint8_t* k_codes, const float* k_norms,
                         const uint8_t* v_codes, const float* v_norms, int max_ctx,
                         const int32_t* lengths, int max_len, float scale, float* out,
                         void* workspace, const AttendPlan& plan, const RawSegment& raw,
                         const ProdKeys& prodk, hipEvent_t ev_before, hipEvent_t ev_after,
                         hipStream_t stream);

// Two-phase cache: rows [0, rows) of each of `heads` heads copied for K and V
// (strides and row sizes in 16-byte words), and the lengths published.
struct CopyRowsArgs {
  const void* src_k;           // 16-byte aligned
  const void* src_v;
  void* dst_k;
  void* dst_v;
  long long src_head, dst_head;  // words between consecutive heads
  int row16;                     // words per row
  int rows, heads;               // rows may be 0 (lengths only)
  int batch;
  int n_packed, n_pending;
  int32_t* packed_len;
  int32_t* pending_len;
};
hipError_t launch_pending_rows(const CopyRowsArgs& a, hipStream_t stream);

// Dense-rotation codecs (head dims with no Walsh-Hadamard transform).
struct DenseEncodeArgs {
  const void* x;               // fp16; vector (t, h) at element t*xs_tok + h*xs_head
  long long xs_tok, xs_head;
  uint8_t* codes;              // row (t, h) at byte t*cs_tok + h*cs_head (4-byte aligned)
  long long cs_tok, cs_head;
  float* norms;
  long long ns_tok, ns_head;
  const double* mt;            // transposed rotation, mt[j*dim + i] = m[i][j] (device)
  int dim, bits, n_tok, n_head;
  float boundaries[256];       // 2^bits - 1 used
};
hipError_t launch_encode_dense(const DenseEncodeArgs& a, hipStream_t stream);

struct DenseAttendArgs {
  const void* q;               // fp16 [batch][n_q_heads][dim]
  const double* mt_k;          // transposed K rotation (device)
  const double* m_v;           // V rotation, row-major (device)
  // wht != 0: the rotations are H diag(sigma) of Walsh-Hadamard codecs, their
  // +-1 entries formed from these signs (mt_k and m_v unused)
  int wht;
  SignArg wht_k, wht_v;
  const uint8_t* k_codes;      // [batch][n_kv_heads][max_ctx][dim*k_bits/8], 4-byte aligned
  const float* k_norms;
  const uint8_t* v_codes;
  const float* v_norms;
  const int32_t* lengths;
  float* pacc;                 // workspace: [batch][n_q_heads][splits][dim]
  float* pml;                  //            [batch][n_q_heads][splits][2]
  float* out;                  // [batch][n_q_heads][dim]
  int dim, k_bits, v_bits, n_q_heads, n_kv_heads, group, max_ctx, splits, tokens_per_split;
  int max_len;                 // host bound of lengths (<= max_ctx); lengths are clamped to it
  int lds_limit;               // bytes of LDS a split workgroup may use
  int rows_words, wave_stride; // per-wavefront LDS region (set by the launcher)
  float qscale;                // scale * log2(e) / dim
  float k_centroids[256];      // unused entries zero
  float v_centroids[256];
};
hipError_t launch_attend_dense(const DenseAttendArgs& a, int batch, hipStream_t stream);
// Lets the dense attend kernels use up to 160 KB of LDS on the current device;
// called at codec set-up so no launch (or graph capture) makes the call.
// Launches of codecs set up without it keep lds_limit at 64 KB.
hipError_t prepare_attend_dense();
constexpr int kDenseLdsFull = 160 * 1024;
constexpr int kDenseLdsDefault = 64 * 1024;
float dense_qscale(float scale, int dim);
// True where the register-held kernel (one query head per KV head) has an
// instance for these shapes; Walsh-Hadamard codec pairs it covers are served
// by it, with m = H diag(sigma), rather than by the matrix-core kernel.
bool dense_lt_supported(int dim, int k_bits, int v_bits, int group);

// Device address of this GPU's fixed scratch array (TQ_NOALLOC_SCRATCH_BYTES
// bytes, 256-byte aligned), looked up on the first call per device.
hipError_t scratch_region(void** ptr);

// Plain streaming read of `bytes` (a multiple of 16) at buf (16-byte aligned).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_stream_read_resident(const void* buf, size_t bytes, uint32_t* sink,
                                       hipStream_t stream);

}  // namespace tq

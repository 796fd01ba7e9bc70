/*
 * tq.h -- C ABI of the compressed-domain KV decode library (MI355X, gfx950).
 *
 * The method (TurboQuant-style KV-cache compression, as described in the
 * mlx-swift-lm pull request "add TurboQuant KV cache compression", the
 * VeloxQuant "How I built" post and the turboquant-mlx KV-cache guide):
 *
 *   encode   x (fp16, d values)  ->  norm N = |x|_2 (fp32)
 *                                    codes idx_j = #{k : beta_k < z_j}, packed LSB-first
 *            where w = H (sigma (.) x), z = w / N, H the d x d Sylvester-Hadamard
 *            matrix, sigma a seeded +/-1 vector and beta the midpoints of the
 *            2^bits-level Lloyd-Max codebook c for N(0,1).
 *   attend   out = sum_t softmax_t(scale * <q, k_hat_t>) v_hat_t over the
 *            compressed cache, where x_hat = (N/d) sigma (.) (H c[idx]); computed
 *            in the rotated basis: K is scored against H (sigma_K (.) q), V is
 *            accumulated as N c[idx] and one inverse transform per head ends it.
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device memory (or host memory the device can read)
 *     owned by the caller; the library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue work on it and return without waiting.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failing call enqueues nothing. tq_last_error() then holds a message.
 *   - Codecs: dim in {64, 128, 256} and bits in [1, 8] (tq_codec_init), Prod
 *     bits in [2, 8], dense-rotation dims any multiple of 32 up to 256.
 *   - Attend coverage. n_q_heads must be a multiple of n_kv_heads with G =
 *     n_q_heads / n_kv_heads <= 16. tq_decode_attend serves every (K bits,
 *     V bits) pair of one dim: the pairs below run the matrix-core kernels,
 *     every other pair a slower kernel that forms the rotation from the
 *     codecs' signs (same results within the attend tolerance). Matrix-core
 *     instances, as (K bits, V bits) up to G query heads per KV head:
 *       dim 64:  4/4 (8), 3/3 (16), 8/3 (8), 6/6 (16), 2/2, 1/1, 5/7, 4/2, 4/3 (4)
 *       dim 128: 8/3 (16), 3/3 (16), 4/4 (8), 4/2 (8), 7/5 (8), 4/3, 2/2, 8/4,
 *                1/1 (4)
 *       dim 256: 2/2 (8), 4/4, 8/3, 3/3, 8/4, 4/2, 4/3 (4)
 *     With one query head per KV head (G = 1) at dim 64, 128 or 256 and K
 *     2/3/4/8, V 2/3/4 bits, tq_decode_attend runs a register-held kernel
 *     instead (two lanes per token, four at dim 256; the rotation formed from
 *     the signs), which is faster there than the matrix-core one.
 *     tq_decode_attend_multi (G x query tokens heads) and tq_decode_attend_mixed
 *     use these instances only; tq_decode_attend_raw_k and
 *     tq_decode_attend_prod list theirs. A request outside them returns
 *     TQ_ERR_UNSUPPORTED and enqueues nothing.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, stride or alignment    */
  TQ_ERR_UNSUPPORTED = -2, /* valid request the kernels do not cover; a      */
                           /* caller may fall back to another path           */
  TQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  TQ_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed     */
  TQ_ERR_NOMEM = -5        /* host allocation failed                          */
} tq_status;

/* Opaque codec: sign vector and fp32 Lloyd-Max tables for one (dim, bits, seed).
 * Immutable after init and shareable across threads, streams and layers (all
 * layers with the same triple share one codec, as in the PR's "shared codecs"
 * design note). A Walsh-Hadamard or Prod codec is host memory only: its tables
 * travel to the GPU inside each launch's kernel arguments, so it holds no
 * device memory and serves every device. A dense-rotation codec owns device
 * memory (its rotation) on the device that was current at
 * tq_codec_init_dense and is used on that device only. */
typedef struct tq_codec tq_codec;

/* Build a codec. dim: head dimension (64, 128 or 256; the Hadamard rotation
 * needs a power of two). bits: code width (1..8), 2^bits centroids.
 * seed: sign-vector seed; sign j is -1 iff the top bit of the j-th SplitMix64
 * output for that seed is set. The codebook is the Lloyd-Max fixed point for
 * N(0,1) (boundaries are centroid midpoints, centroids are cell conditional
 * means), solved on the host in quad precision and rounded once to fp32.
 * Errors: TQ_ERR_UNSUPPORTED for other dims/bits, TQ_ERR_INVALID_ARG for NULL out. */
tq_status tq_codec_init(int dim, int bits, uint64_t seed, tq_codec** out);

/* Free a codec (NULL is a no-op). Work already enqueued keeps its own copy of
 * the tables in its kernel arguments, so a codec may be destroyed at any time. */
void tq_codec_destroy(tq_codec* c);

/* Host copies of the codec's tables: signs[dim] (+1/-1), centroids[2^bits],
 * boundaries[2^bits - 1] (each may be NULL to skip). */
tq_status tq_codec_tables(const tq_codec* c, int8_t* signs, float* centroids,
                          float* boundaries);

/* dim, bits and seed of a codec (each pointer may be NULL). */
tq_status tq_codec_info(const tq_codec* c, int* dim, int* bits, uint64_t* seed);

/* Bytes of one packed code row: dim * bits / 8. */
int tq_row_bytes(int dim, int bits);

/*
 * Encode n_tok x n_head vectors (the PR's batch recompression of pending
 * tokens; a cache append is this call with the destination offset to the
 * append position).
 *   x_fp16: vector (t, h) starts at element t*x_stride_tok + h*x_stride_head
 *           (in fp16 elements); its dim values are contiguous.
 *   codes:  row (t, h) starts at byte t*c_stride_tok + h*c_stride_head and
 *           receives dim*bits/8 bytes; pointer and strides must be multiples of 4.
 *   norms:  norm (t, h) is written at element t*n_stride_tok + h*n_stride_head.
 * Results are bit-exact with the definition above: the rotation and norm are
 * computed in fp64 (the rotation of fp16 input is exact; the squared norm is
 * summed over the canonical pairwise tree), z = w/N in IEEE fp64, a zero
 * vector encodes to norm 0 and index 2^(bits-1)-1 everywhere.
 * n_tok == 0 or n_head == 0 enqueues nothing and returns TQ_OK.
 */
tq_status tq_encode(const tq_codec* c, const void* x_fp16, int n_tok, int n_head,
                    int64_t x_stride_tok, int64_t x_stride_head, uint8_t* codes,
                    int64_t c_stride_tok, int64_t c_stride_head, float* norms,
                    int64_t n_stride_tok, int64_t n_stride_head, void* stream);

/* One vector set of an encode call: a codec and the x / codes / norms arrays
 * with their strides, exactly as the arguments of tq_encode. */
typedef struct {
  const tq_codec* codec;
  const void* x_fp16;
  int64_t x_stride_tok, x_stride_head;
  uint8_t* codes;
  int64_t c_stride_tok, c_stride_head;
  float* norms;
  int64_t n_stride_tok, n_stride_head;
} tq_encode_job;

/*
 * Encode the K and V vectors of one appended token batch in a single launch
 * (the PR's cache update appends keys and values together; one launch instead
 * of two halves the fixed cost of a short append). k and v each describe
 * n_tok x n_head vectors with the layout, alignment and exactness rules of
 * tq_encode; their codecs must have the same dim and may differ in bits and
 * seed. Results are identical to tq_encode(k) followed by tq_encode(v). The
 * two jobs' outputs must not overlap. Errors as tq_encode, plus
 * TQ_ERR_INVALID_ARG for a NULL job or codecs of different dim.
 */
tq_status tq_encode_kv(const tq_encode_job* k, const tq_encode_job* v, int n_tok, int n_head,
                       void* stream);

/*
 * TurboQuant-Prod key codec (VeloxQuant "How I built", Stage 3 "QJL Residual
 * Correction", and its TurboQuantProd method): bits - 1 bits of Lloyd-Max
 * codes as above, plus a 1-bit sketch of the quantisation residual, so that
 * scores can be corrected. In the rotated basis z = H(sigma x) / N the residual
 * is rho = z - c[idx]; the codec stores its norm gamma = |rho| (fp32) and the
 * signs of H(sigma_S (.) rho), sigma_S the SplitMix64 signs of seed + 1 (one bit
 * per coordinate, LSB-first, set for a negative value). bits in [2, 8].
 * Prod codecs encode with tq_encode_prod and attend as K codecs with
 * tq_decode_attend_prod; the other calls reject them.
 */
tq_status tq_codec_init_prod(int dim, int bits, uint64_t seed, tq_codec** out);

/*
 * Dense-rotation codec for head dims with no Walsh-Hadamard transform (PR #232,
 * Known limitations: power-of-2 head dims use the WHT, others a dense
 * rotation; VeloxQuant "How I built", Stage 1: the original method rotates by
 * the Q factor of a Gaussian matrix). rotation: host array, dim x dim fp64,
 * row-major, equal to sqrt(dim) times an orthogonal matrix (the caller draws
 * it; only finiteness is checked). It is copied to the current device, with
 * its transpose (16 dim^2 bytes); the codec owns both until tq_codec_destroy.
 * Encode (tq_encode, tq_encode_kv with two dense codecs of one dim):
 * N = |x| summed in fp64 over a pairwise tree in index order (an odd last
 * element is carried up a level), w = rotation . x in fp64 with products and
 * sums in index order and no fused multiply-add, z = w / N, then the
 * Lloyd-Max indices and packing of tq_encode. With rotation = H diag(sigma)
 * the codes and norms equal those of tq_codec_init's codec with that sigma.
 * Attend: tq_decode_attend with dense K and V codecs (the same arguments and
 * workspace as for the Walsh-Hadamard codecs); the other attend calls and the
 * two-phase cache return TQ_ERR_UNSUPPORTED for dense codecs.
 * dim: a multiple of 32 in [32, 256] (so rows are whole dwords), else
 * TQ_ERR_UNSUPPORTED; bits in [1, 8]. TQ_ERR_INVALID_ARG for a NULL rotation
 * or a non-finite entry, TQ_ERR_HIP if the device copy or the one-time set-up
 * of the dense attend kernels (their LDS limit on the current device) fails.
 * Codec set-up, not the attend call, makes that runtime call, so attend calls
 * can be captured in a HIP graph. tq_codec_tables
 * reports signs of +1 and tq_codec_info a seed of 0 for a dense codec.
 */
tq_status tq_codec_init_dense(int dim, int bits, const double* rotation, tq_codec** out);

/* tq_encode for a Prod codec: codes (dim*(bits-1)/8 bytes per row, layout and
 * alignment as tq_encode), sketch (dim/8 bytes per row at byte
 * t*s_stride_tok + h*s_stride_head, any alignment), norms, and residual norms
 * gamma (fp32, element t*r_stride_tok + h*r_stride_head, 4-byte aligned). Codes,
 * sketch bits, norms and residual norms are bit-exact with the definition (fp64
 * throughout, butterflies in ascending stage order, canonical pairwise trees). */
tq_status tq_encode_prod(const tq_codec* c, const void* x_fp16, int n_tok, int n_head,
                         int64_t x_stride_tok, int64_t x_stride_head, uint8_t* codes,
                         int64_t c_stride_tok, int64_t c_stride_head, uint8_t* sketch,
                         int64_t s_stride_tok, int64_t s_stride_head, float* norms,
                         int64_t n_stride_tok, int64_t n_stride_head, float* rnorms,
                         int64_t r_stride_tok, int64_t r_stride_head, void* stream);

/*
 * Decode attention with TurboQuant-Prod keys (encoded by tq_encode_prod):
 * scores use the QJL-corrected estimate of <q, k>,
 *   <q, k_hat_MSE> + (N / d) sqrt(pi / 2) (gamma / d) sum_j sgn_j u_j,
 * u = H(sigma_S (.) H(sigma_K (.) q)), sgn_j = -1 where sketch bit j is set
 * (the asymmetric 1-bit JL estimate of the residual term of VeloxQuant "How I
 * built", Stage 3). Values are read through vc as in tq_decode_attend.
 *   k_codes: [batch][n_kv_heads][max_ctx][dim*(bits-1)/8], 16-byte aligned;
 *   k_sketch: [batch][n_kv_heads][max_ctx][dim/8], 16-byte aligned;
 *   k_norms, k_rnorms: [batch][n_kv_heads][max_ctx] fp32.
 * Every other argument as for tq_decode_attend. Kernels exist for dim 128 with
 * 4-bit Prod K and 4-bit V (group <= 8), 3-bit Prod K and 3-bit V (group <= 4),
 * and dim 64 with 4-bit Prod K and 4-bit V (group <= 4).
 */
tq_status tq_decode_attend_prod(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                int batch, int n_q_heads, int n_kv_heads,
                                const uint8_t* k_codes, const uint8_t* k_sketch,
                                const float* k_norms, const float* k_rnorms,
                                const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                const int32_t* lengths, int max_len, float scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes tq_decode_attend needs for this shape (the per-split
 * partial results). A pure function of its arguments; 0 on invalid input. */
size_t tq_attend_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int dim,
                                 int max_len);

/*
 * Decode attention straight from the packed cache (the fused compressed-domain
 * decode of the X post and the turboquant-mlx guide: score, softmax and inline
 * dequantisation without expanding the cache).
 *   kc, vc:     codecs of the K and V caches (same dim; bits may differ).
 *   q_fp16:     [batch][n_q_heads][dim] fp16, contiguous.
 *   k_codes:    [batch][n_kv_heads][max_ctx][dim*kc_bits/8] bytes, contiguous,
 *               16-byte aligned (v_codes likewise).
 *   k_norms:    [batch][n_kv_heads][max_ctx] fp32.  v_codes / v_norms likewise.
 *   lengths:    device int32[batch]; sequence b attends to rows [0, lengths[b]).
 *               Values are clamped to max_len on the device, so the cache is
 *               never read past max_len rows; a length <= 0 gives a zero row.
 *   max_len:    host-side upper bound of lengths, 1 <= max_len <= max_ctx; it
 *               sizes the launch.
 *   scale:      softmax scale (1/sqrt(dim) for standard attention).
 *   out:        [batch][n_q_heads][dim] fp32. Query head h reads KV head
 *               h / (n_q_heads / n_kv_heads).
 *   workspace:  device buffer of at least tq_attend_workspace_bytes(...) bytes,
 *               256-byte aligned; its contents need not be initialised. It
 *               holds one partial per (sequence, query head, split).
 * Two kernels are enqueued: split attend (the query rotation runs in its
 * prologue) and combine + inverse rotation. Every (K bits, V bits) pair of
 * one dim is served (the coverage list at the top of this header names the
 * matrix-core pairs and the one-query-head-per-KV-head shapes of the
 * register-held kernel; the others take the slower sign-formed rotation
 * kernels).
 * Results agree with softmax attention over the dequantised cache (computed
 * in fp64) to about 1e-5 absolute for unit-scale inputs, and within 2e-3 for
 * the tested workloads; sums in a different order make the low bits differ
 * from any serial evaluation.
 */
tq_status tq_decode_attend(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                           int batch, int n_q_heads, int n_kv_heads,
                           const uint8_t* k_codes, const float* k_norms,
                           const uint8_t* v_codes, const float* v_norms, int max_ctx,
                           const int32_t* lengths, int max_len, float scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * tq_decode_attend for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels, with the per-split partials in a fixed array the library
 * holds on each GPU (TQ_NOALLOC_SCRATCH_BYTES bytes in its code object, kept
 * until the process ends) instead of a caller workspace. The call allocates
 * nothing; its first call on a device looks up that device's array.
 *   Arguments as tq_decode_attend without the workspace pair; the caller still
 *   owns q, the cache, lengths and out.
 *   Errors as tq_decode_attend; TQ_ERR_UNSUPPORTED when the shape needs more
 *   than TQ_NOALLOC_SCRATCH_BYTES of partials (tq_attend_workspace_bytes of the
 *   same shape tells), TQ_ERR_HIP if the array's address cannot be found.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one device (two streams, two threads) race and must be ordered by the caller.
 * The kernels write every partial they later read, so nothing carries over
 * from the previous call. Results equal tq_decode_attend's bit for bit.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (8u << 20)
tq_status tq_decode_attend_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                   int batch, int n_q_heads, int n_kv_heads,
                                   const uint8_t* k_codes, const float* k_norms,
                                   const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                   const int32_t* lengths, int max_len, float scale, float* out,
                                   void* stream);

/*
 * Multi-token decode: n_query_tokens new query rows per sequence attend the
 * packed cache at once, causal among themselves (verifying a speculative
 * draft, or a chunk of queries; PR #232's review threads on the multi-query
 * NR0 attention path and on speculative decoding with draft tokens).
 *   q_fp16: [batch][n_query_tokens][n_q_heads][dim] fp16, contiguous.
 *   out:    [batch][n_query_tokens][n_q_heads][dim] fp32.
 *   lengths[b] counts the cache rows of sequence b including the
 *   n_query_tokens rows of the new tokens (already appended, e.g. with
 *   tq_encode_kv). Query token i sees rows [0, lengths[b] - n_query_tokens +
 *   i + 1), clamped to max_len; if that is empty its output row is zero.
 *   Every other argument is as for tq_decode_attend, with a workspace of at
 *   least tq_attend_multi_workspace_bytes(...) bytes. With n_query_tokens == 1
 *   this is tq_decode_attend.
 * Supported while (n_q_heads / n_kv_heads) * n_query_tokens <= 16 and a
 * matrix-core instance of the header's list covers that many heads per KV
 * head (TQ_ERR_UNSUPPORTED otherwise).
 */
tq_status tq_decode_attend_multi(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                 int batch, int n_query_tokens, int n_q_heads, int n_kv_heads,
                                 const uint8_t* k_codes, const float* k_norms,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes tq_decode_attend_multi needs for this shape; 0 on invalid
 * input. */
size_t tq_attend_multi_workspace_bytes(int batch, int n_query_tokens, int n_q_heads,
                                       int n_kv_heads, int dim, int max_len);

/*
 * Decode attention over the packed cache plus a segment of raw fp16 rows
 * attended together with it: an fp16 prefix of "sink" tokens kept
 * uncompressed (turboquant-mlx guide, --kv-min-tokens), or the pending tokens
 * of a two-phase cache that are not yet batch-compressed (PR #232, Design).
 * Softmax runs over the union of the packed rows [0, lengths[b]) and the raw
 * rows [0, raw_lengths[b]) (their order does not matter to one query).
 *   raw_k_fp16, raw_v_fp16: [batch][n_kv_heads][max_raw][dim] fp16,
 *       contiguous, 16-byte aligned.
 *   raw_lengths: device int32[batch]; values are clamped to max_raw on the
 *       device; <= 0 means no raw rows for that sequence.
 *   max_raw: 1 .. 4096 (TQ_ERR_UNSUPPORTED above).
 *   lengths[b] may be 0 (raw rows only); a sequence with no row at all gets
 *   a zero output row.
 * Every other argument is as for tq_decode_attend, with the same workspace
 * size (tq_attend_workspace_bytes). The same two kernels are enqueued: the
 * combine kernel also scores the raw rows and adds their part.
 */
tq_status tq_decode_attend_mixed(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                 int batch, int n_q_heads, int n_kv_heads,
                                 const uint8_t* k_codes, const float* k_norms,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, const void* raw_k_fp16,
                                 const void* raw_v_fp16, int max_raw,
                                 const int32_t* raw_lengths, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention with raw fp16 keys and packed values: PR #232's raw-K
 * schemes (turbo0v4, turbo0v2: keys at FP16, only values compressed). Scores
 * are taken from the fp16 key rows as they are; values are read through vc
 * as in tq_decode_attend.
 *   k_fp16: [batch][n_kv_heads][max_ctx][dim] fp16, contiguous, 16-byte
 *           aligned.
 *   v_codes / v_norms, lengths, max_len, scale, out, workspace: as for
 *           tq_decode_attend (workspace size tq_attend_workspace_bytes).
 * Kernels exist for dim 64 and 128 with 4-bit V (up to 8 query heads per KV
 * head) or 2-bit V (up to 4); TQ_ERR_UNSUPPORTED otherwise.
 */
tq_status tq_decode_attend_raw_k(const tq_codec* vc, const void* q_fp16, int batch,
                                 int n_q_heads, int n_kv_heads, const void* k_fp16,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Two-phase cache of one layer (PR #232, Design: keys and values stay fp16
 * until they are batch-compressed; pending tokens are accumulated and
 * encoded in batches, default 64). The cache holds packed rows [0, n_packed)
 * of every (sequence, KV head) and fp16 pending rows that follow them; rows
 * are compressed only in whole groups of group_size, so a long append (a
 * prompt) is compressed in one batch and a decode step's row waits in the
 * pending buffer until its group is full. Attention covers both parts.
 * All sequences of the batch advance together (one length per cache).
 *
 * The caller allocates every buffer and keeps it alive until
 * tq_cache_destroy; the cache object holds only host state (the two counts).
 *   k_codes, k_norms, v_codes, v_norms: packed cache, as for
 *       tq_decode_attend ([batch][n_kv_heads][max_ctx][row], 16-byte aligned).
 *   pending_k, pending_v: fp16 [batch][n_kv_heads][group_size][dim], 16-byte
 *       aligned.
 *   packed_len, pending_len: device int32[batch]; the cache writes n_packed
 *       and n_pending there (the lengths tq_decode_attend_mixed reads).
 *   group_size: 1 .. 4096; max_ctx >= 1.
 * Calls on one cache must be ordered by the caller (one stream, or events);
 * they are not thread-safe.
 */
typedef struct tq_cache tq_cache;
typedef struct {
  int batch, n_kv_heads, max_ctx, group_size;
  uint8_t* k_codes;
  float* k_norms;
  uint8_t* v_codes;
  float* v_norms;
  void* pending_k;
  void* pending_v;
  int32_t* packed_len;
  int32_t* pending_len;
} tq_cache_desc;

/* Validate desc against the codecs (plain codecs of the same dim, a dim and
 * bit widths tq_decode_attend_mixed covers) and create an empty cache. No
 * device work is enqueued. */
tq_status tq_cache_init(const tq_codec* kc, const tq_codec* vc, const tq_cache_desc* desc,
                        tq_cache** out);
void tq_cache_destroy(tq_cache* c);

/* Current counts: rows compressed and rows pending, per (sequence, KV head). */
tq_status tq_cache_state(const tq_cache* c, int* n_packed, int* n_pending);

/*
 * Append n_tok rows to every (sequence, KV head). k_fp16, v_fp16:
 * [batch][n_kv_heads][n_tok][dim] fp16, contiguous, 16-byte aligned. Every
 * whole group of group_size rows (pending rows first, then the new ones) is
 * encoded into the packed cache at n_packed with tq_encode_kv's rules (bit-
 * exact codes and norms); the remaining rows are copied to the pending
 * buffer, and both length arrays are rewritten. Enqueues on `stream`: at most
 * two encode launches, one copy and one length fill. Fails with
 * TQ_ERR_INVALID_ARG before enqueueing anything when the packed rows would
 * exceed max_ctx. n_tok == 0 does nothing.
 */
tq_status tq_cache_append(tq_cache* c, const void* k_fp16, const void* v_fp16, int n_tok,
                          void* stream);

/* Workspace bytes tq_cache_attend needs for n_q_heads query heads at any
 * fill level (0 on invalid input). */
size_t tq_cache_workspace_bytes(const tq_cache* c, int n_q_heads);

/*
 * Decode attention of q_fp16 [batch][n_q_heads][dim] over the packed and the
 * pending rows (tq_decode_attend_mixed with the cache's buffers and lengths;
 * the same result for any split of the rows between the two parts, up to
 * rounding). An empty cache gives zero output rows. out, scale, workspace as
 * for tq_decode_attend.
 */
tq_status tq_cache_attend(tq_cache* c, const void* q_fp16, int n_q_heads, float scale,
                          float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Measurement hook (per calling thread): while `before` and `after` are
 * non-NULL, each tq_decode_attend launches its split-attend kernel with the
 * hipEvent_t `before` and `after` bound to that dispatch (hipExtLaunchKernel
 * start and stop events), so hipEventElapsedTime(before, after) is the
 * kernel's own execution time. The events are created and owned by the
 * caller. Pass NULL, NULL to stop. */
tq_status tq_set_split_events(void* before, void* after);

/* Measurement aid: enqueue a plain streaming read of `bytes` bytes at the
 * device buffer buf (16-byte aligned, bytes a multiple of 16) on `stream`. It
 * reads every byte once and writes nothing in practice (at most 4 bytes at
 * sink, a caller-owned device word, for one input pattern), so its time is the
 * read bandwidth the device reaches for a transfer of that size: the measured
 * ceiling next to the nominal peak. bytes == 0 does nothing. */
tq_status tq_stream_read(const void* buf, size_t bytes, void* sink, void* stream);

/* Measurement aid, the same read by a second design: a resident grid of one
 * 1024-thread workgroup per compute unit whose threads loop over their share
 * with eight 16-byte loads in flight per pass (tq_stream_read launches one
 * 256-thread workgroup per 32 KB). Same arguments, alignment rules and
 * errors as tq_stream_read. */
tq_status tq_stream_read_resident(const void* buf, size_t bytes, void* sink, void* stream);

/* Number of context splits tq_decode_attend launches for this shape (for
 * measurement and tests); 0 on invalid input. */
int tq_attend_num_splits(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len);

/* Static text for a status code. */
const char* tq_status_string(tq_status s);

/* Detail text of the last failing call on this thread ("" if none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */

// api.cpp -- the C ABI declared in include/tq.h: argument validation, launch
// planning and error reporting. Every check runs on the host before anything
// is enqueued, so a failing call leaves the stream untouched.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "../../include/tq.h"
#include "codec.hpp"
#include "kernels.hpp"

struct tq_codec {
  tq::CodecTables tabs;
  // dense-rotation codecs: the rotation and its transpose on the device
  bool dense = false;
  double* m_dev = nullptr;
  double* mt_dev = nullptr;
};

// Host state of a two-phase cache: the caller's buffers and the two counts.
struct tq_cache {
  const tq_codec* kc;
  const tq_codec* vc;
  tq_cache_desc d;
  int n_packed = 0, n_pending = 0;
  bool lengths_published = false;  // the device length arrays hold the counts
};

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_split_before = nullptr;
thread_local hipEvent_t g_split_after = nullptr;

tq_status fail(tq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tq_status ok() {
  g_last_error.clear();
  return TQ_OK;
}

bool dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool dense_dim_ok(int d) { return d >= 32 && d <= tq::kMaxDim && d % 32 == 0; }

tq::SignArg sign_arg(const tq_codec* c) {
  tq::SignArg s;
  std::memcpy(s.bits, c->tabs.sign_bits, sizeof(s.bits));
  return s;
}

// Sketch and residual-norm outputs of a TurboQuant-Prod encode.
struct ProdOut {
  uint8_t* sketch;
  int64_t s_stride_tok, s_stride_head;
  float* rnorms;
  int64_t r_stride_tok, r_stride_head;
};

// Validate the jobs of one encode call and launch them together. `prod`
// (one entry per job, or NULL) carries the extra outputs of Prod codecs.
tq_status encode_jobs(const char* fn, const tq_encode_job* jobs, int n_jobs, int n_tok,
                      int n_head, void* stream, const ProdOut* prod = nullptr) {
  for (int i = 0; i < n_jobs; ++i) {
    const tq_encode_job& j = jobs[i];
    if (!j.codec) return fail(TQ_ERR_INVALID_ARG, "%s: codec %d is NULL", fn, i);
    if (j.codec->tabs.prod != (prod != nullptr))
      return fail(TQ_ERR_INVALID_ARG, "%s: %s codec %d (use %s)", fn,
                  j.codec->tabs.prod ? "TurboQuant-Prod" : "plain", i,
                  j.codec->tabs.prod ? "tq_encode_prod" : "tq_encode or tq_encode_kv");
    if (j.codec->tabs.dim != jobs[0].codec->tabs.dim)
      return fail(TQ_ERR_INVALID_ARG, "%s: codecs of different dim (%d, %d)", fn,
                  jobs[0].codec->tabs.dim, j.codec->tabs.dim);
    if (j.codec->dense != jobs[0].codec->dense)
      return fail(TQ_ERR_INVALID_ARG, "%s: dense-rotation and Walsh-Hadamard codecs mixed", fn);
  }
  if (n_tok < 0 || n_head < 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: negative count (n_tok %d, n_head %d)", fn, n_tok,
                n_head);
  if (n_tok == 0 || n_head == 0) return ok();
  tq::EncodeArgs args;
  std::memset(&args, 0, sizeof(args));
  args.n_tok = n_tok;
  args.n_head = n_head;
  args.n_jobs = n_jobs;
  for (int i = 0; i < n_jobs; ++i) {
    const tq_encode_job& j = jobs[i];
    if (!j.x_fp16 || !j.codes || !j.norms)
      return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer in job %d", fn, i);
    if (((uintptr_t)j.codes & 3) || (j.c_stride_tok & 3) || (j.c_stride_head & 3))
      return fail(TQ_ERR_INVALID_ARG,
                  "%s: codes pointer and strides must be multiples of 4 bytes (job %d)", fn, i);
    if (((uintptr_t)j.x_fp16 & 1) || ((uintptr_t)j.norms & 3))
      return fail(TQ_ERR_INVALID_ARG, "%s: misaligned x or norms pointer (job %d)", fn, i);
    tq::EncodeJob& e = args.job[i];
    e.x = j.x_fp16;
    e.xs_tok = j.x_stride_tok;
    e.xs_head = j.x_stride_head;
    e.codes = j.codes;
    e.cs_tok = j.c_stride_tok;
    e.cs_head = j.c_stride_head;
    e.norms = j.norms;
    e.ns_tok = j.n_stride_tok;
    e.ns_head = j.n_stride_head;
    e.bits = j.codec->tabs.bits;
    e.sign = sign_arg(j.codec);
    std::memcpy(e.boundaries, j.codec->tabs.boundaries, sizeof(float) * ((1 << e.bits) - 1));
    if (prod) {
      const ProdOut& po = prod[i];
      if (!po.sketch || !po.rnorms)
        return fail(TQ_ERR_INVALID_ARG, "%s: NULL sketch or residual-norm pointer", fn);
      if ((uintptr_t)po.rnorms & 3)
        return fail(TQ_ERR_INVALID_ARG, "%s: misaligned residual-norm pointer", fn);
      e.prod = 1;
      std::memcpy(e.boundaries + 128, j.codec->tabs.centroids, sizeof(float) * (1 << e.bits));
      e.sketch = po.sketch;
      e.ss_tok = po.s_stride_tok;
      e.ss_head = po.s_stride_head;
      e.rnorms = po.rnorms;
      e.rs_tok = po.r_stride_tok;
      e.rs_head = po.r_stride_head;
      std::memcpy(e.sketch_sign.bits, j.codec->tabs.sketch_sign_bits, sizeof(e.sketch_sign.bits));
    }
  }
  const long long nvec = (long long)n_tok * n_head;
  if (nvec > 0x7fffffffLL - 64)
    return fail(TQ_ERR_UNSUPPORTED, "%s: more than 2^31 - 65 vectors", fn);
  if (jobs[0].codec->dense) {  // one launch per job
    for (int i = 0; i < n_jobs; ++i) {
      const tq_codec* c = jobs[i].codec;
      const tq::EncodeJob& e = args.job[i];
      tq::DenseEncodeArgs da;
      std::memset(&da, 0, sizeof(da));
      da.x = e.x;
      da.xs_tok = e.xs_tok;
      da.xs_head = e.xs_head;
      da.codes = e.codes;
      da.cs_tok = e.cs_tok;
      da.cs_head = e.cs_head;
      da.norms = e.norms;
      da.ns_tok = e.ns_tok;
      da.ns_head = e.ns_head;
      da.mt = c->mt_dev;
      da.dim = c->tabs.dim;
      da.bits = c->tabs.bits;
      da.n_tok = n_tok;
      da.n_head = n_head;
      std::memcpy(da.boundaries, c->tabs.boundaries, sizeof(float) * ((1 << da.bits) - 1));
      const hipError_t err = tq::launch_encode_dense(da, (hipStream_t)stream);
      if (err != hipSuccess)
        return fail(TQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    }
    return ok();
  }
  hipError_t err = tq::launch_encode(jobs[0].codec->tabs.dim, args, (hipStream_t)stream);
  if (err != hipSuccess)
    return fail(TQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_NOMEM: return "TQ_ERR_NOMEM";
  }
  return "TQ_ERR_UNKNOWN";
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

int tq_row_bytes(int dim, int bits) {
  if (dim <= 0 || bits < 1 || bits > 8) return 0;
  return dim * bits / 8;
}

tq_status tq_codec_init(int dim, int bits, uint64_t seed, tq_codec** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_init: out is NULL");
  *out = nullptr;
  if (!dim_ok(dim))
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_init: dim %d not in {64, 128, 256}", dim);
  if (bits < 1 || bits > 8)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_init: bits %d not in [1, 8]", bits);
  tq_codec* c = new (std::nothrow) tq_codec;
  if (!c) return fail(TQ_ERR_NOMEM, "tq_codec_init: out of host memory");
  if (!tq::build_codec(dim, bits, seed, &c->tabs)) {
    delete c;
    return fail(TQ_ERR_INVALID_ARG, "tq_codec_init: Lloyd-Max solve did not converge");
  }
  *out = c;
  return ok();
}

tq_status tq_codec_init_prod(int dim, int bits, uint64_t seed, tq_codec** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codec_init_prod: out is NULL");
  *out = nullptr;
  if (!dim_ok(dim))
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_init_prod: dim %d not in {64, 128, 256}", dim);
  if (bits < 2 || bits > 8)
    return fail(TQ_ERR_UNSUPPORTED, "tq_codec_init_prod: bits %d not in [2, 8]", bits);
  tq_codec* c = new (std::nothrow) tq_codec;
  if (!c) return fail(TQ_ERR_NOMEM, "tq_codec_init_prod: out of host memory");
  if (!tq::build_prod_codec(dim, bits, seed, &c->tabs)) {
    delete c;
    return fail(TQ_ERR_INVALID_ARG, "tq_codec_init_prod: Lloyd-Max solve did not converge");
  }
  *out = c;
  return ok();
}

tq_status tq_codec_init_dense(int dim, int bits, const double* rotation, tq_codec** out) {
  const char* fn = "tq_codec_init_dense";
  if (!out) return fail(TQ_ERR_INVALID_ARG, "%s: out is NULL", fn);
  *out = nullptr;
  if (!rotation) return fail(TQ_ERR_INVALID_ARG, "%s: rotation is NULL", fn);
  if (!dense_dim_ok(dim))
    return fail(TQ_ERR_UNSUPPORTED, "%s: dim %d not a multiple of 32 in [32, 256]", fn, dim);
  if (bits < 1 || bits > 8) return fail(TQ_ERR_UNSUPPORTED, "%s: bits %d not in [1, 8]", fn, bits);
  const size_t n = (size_t)dim * dim;
  for (size_t i = 0; i < n; ++i)
    if (!(rotation[i] - rotation[i] == 0.0))
      return fail(TQ_ERR_INVALID_ARG, "%s: rotation entry %zu is not finite", fn, i);
  tq_codec* c = new (std::nothrow) tq_codec;
  if (!c) return fail(TQ_ERR_NOMEM, "%s: out of host memory", fn);
  if (!tq::build_codec(dim, bits, 0, &c->tabs)) {
    delete c;
    return fail(TQ_ERR_INVALID_ARG, "%s: Lloyd-Max solve did not converge", fn);
  }
  std::memset(c->tabs.sign_bits, 0, sizeof(c->tabs.sign_bits));  // no sign vector
  c->dense = true;
  std::string err_text;
  double* mt = new (std::nothrow) double[n];
  if (!mt) {
    delete c;
    return fail(TQ_ERR_NOMEM, "%s: out of host memory", fn);
  }
  for (int i = 0; i < dim; ++i)
    for (int j = 0; j < dim; ++j) mt[(size_t)j * dim + i] = rotation[(size_t)i * dim + j];
  hipError_t e = hipMalloc((void**)&c->m_dev, n * sizeof(double));
  if (e == hipSuccess) e = hipMalloc((void**)&c->mt_dev, n * sizeof(double));
  if (e == hipSuccess) e = hipMemcpy(c->m_dev, rotation, n * sizeof(double), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(c->mt_dev, mt, n * sizeof(double), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = tq::prepare_attend_dense();
  delete[] mt;
  if (e != hipSuccess) {
    if (c->m_dev) (void)hipFree(c->m_dev);
    if (c->mt_dev) (void)hipFree(c->mt_dev);
    delete c;
    return fail(TQ_ERR_HIP, "%s: device set-up failed: %s", fn,
                hipGetErrorString(e));
  }
  *out = c;
  return ok();
}

void tq_codec_destroy(tq_codec* c) {
  if (!c) return;
  if (c->m_dev) (void)hipFree(c->m_dev);
  if (c->mt_dev) (void)hipFree(c->mt_dev);
  delete c;
}

tq_status tq_codec_tables(const tq_codec* c, int8_t* signs, float* centroids,
                          float* boundaries) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "tq_codec_tables: codec is NULL");
  const int n = 1 << c->tabs.bits;
  if (signs)
    for (int j = 0; j < c->tabs.dim; ++j)
      signs[j] = ((c->tabs.sign_bits[j >> 5] >> (j & 31)) & 1u) ? -1 : 1;
  if (centroids) std::memcpy(centroids, c->tabs.centroids, sizeof(float) * n);
  if (boundaries) std::memcpy(boundaries, c->tabs.boundaries, sizeof(float) * (n - 1));
  return ok();
}

tq_status tq_codec_info(const tq_codec* c, int* dim, int* bits, uint64_t* seed) {
  if (!c) return fail(TQ_ERR_INVALID_ARG, "tq_codec_info: codec is NULL");
  if (dim) *dim = c->tabs.dim;
  if (bits) *bits = c->tabs.bits;
  if (seed) *seed = c->tabs.seed;
  return ok();
}

tq_status tq_encode(const tq_codec* c, const void* x_fp16, int n_tok, int n_head,
                    int64_t x_stride_tok, int64_t x_stride_head, uint8_t* codes,
                    int64_t c_stride_tok, int64_t c_stride_head, float* norms,
                    int64_t n_stride_tok, int64_t n_stride_head, void* stream) {
  const tq_encode_job job = {c,     x_fp16,       x_stride_tok, x_stride_head,
                             codes, c_stride_tok, c_stride_head, norms,
                             n_stride_tok, n_stride_head};
  return encode_jobs("tq_encode", &job, 1, n_tok, n_head, stream);
}

tq_status tq_encode_prod(const tq_codec* c, const void* x_fp16, int n_tok, int n_head,
                         int64_t x_stride_tok, int64_t x_stride_head, uint8_t* codes,
                         int64_t c_stride_tok, int64_t c_stride_head, uint8_t* sketch,
                         int64_t s_stride_tok, int64_t s_stride_head, float* norms,
                         int64_t n_stride_tok, int64_t n_stride_head, float* rnorms,
                         int64_t r_stride_tok, int64_t r_stride_head, void* stream) {
  const tq_encode_job job = {c,     x_fp16,       x_stride_tok, x_stride_head,
                             codes, c_stride_tok, c_stride_head, norms,
                             n_stride_tok, n_stride_head};
  const ProdOut po = {sketch, s_stride_tok, s_stride_head, rnorms, r_stride_tok, r_stride_head};
  return encode_jobs("tq_encode_prod", &job, 1, n_tok, n_head, stream, &po);
}

tq_status tq_encode_kv(const tq_encode_job* k, const tq_encode_job* v, int n_tok, int n_head,
                       void* stream) {
  if (!k || !v) return fail(TQ_ERR_INVALID_ARG, "tq_encode_kv: job is NULL");
  const tq_encode_job jobs[2] = {*k, *v};
  return encode_jobs("tq_encode_kv", jobs, 2, n_tok, n_head, stream);
}

tq_status tq_set_split_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(TQ_ERR_INVALID_ARG, "tq_set_split_events: give both events or neither");
  g_split_before = (hipEvent_t)before;
  g_split_after = (hipEvent_t)after;
  return ok();
}

tq_status tq_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(TQ_ERR_INVALID_ARG, "tq_stream_read: NULL buffer or sink");
  if ((uintptr_t)buf % 16 || bytes % 16 || (uintptr_t)sink % 4)
    return fail(TQ_ERR_INVALID_ARG,
                "tq_stream_read: buffer must be 16-byte aligned, bytes a multiple of 16, "
                "sink 4-byte aligned");
  const hipError_t e = tq::launch_stream_read(buf, bytes, (uint32_t*)sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TQ_ERR_HIP, "tq_stream_read: %s", hipGetErrorString(e));
  return ok();
}

tq_status tq_stream_read_resident(const void* buf, size_t bytes, void* sink, void* stream) {
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(TQ_ERR_INVALID_ARG, "tq_stream_read_resident: NULL buffer or sink");
  if ((uintptr_t)buf % 16 || bytes % 16 || (uintptr_t)sink % 4)
    return fail(TQ_ERR_INVALID_ARG,
                "tq_stream_read_resident: buffer must be 16-byte aligned, bytes a multiple of 16, "
                "sink 4-byte aligned");
  const hipError_t e =
      tq::launch_stream_read_resident(buf, bytes, (uint32_t*)sink, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TQ_ERR_HIP, "tq_stream_read_resident: %s", hipGetErrorString(e));
  return ok();
}

static bool attend_shape_ok(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len) {
  return batch > 0 && n_kv_heads > 0 && n_q_heads > 0 && n_q_heads % n_kv_heads == 0 &&
         n_q_heads / n_kv_heads <= 16 && dense_dim_ok(dim) && max_len > 0 && batch <= 65535 &&
         n_kv_heads <= 65535;
}

size_t tq_attend_workspace_bytes(int batch, int n_q_heads, int n_kv_heads, int dim,
                                 int max_len) {
  if (!attend_shape_ok(batch, n_q_heads, n_kv_heads, dim, max_len)) return 0;
  return tq::plan_attend(batch, n_q_heads, n_kv_heads, dim, max_len).total_bytes;
}

int tq_attend_num_splits(int batch, int n_q_heads, int n_kv_heads, int dim, int max_len) {
  if (!attend_shape_ok(batch, n_q_heads, n_kv_heads, dim, max_len)) return 0;
  return tq::plan_attend(batch, n_q_heads, n_kv_heads, dim, max_len).splits;
}

}  // extern "C"

namespace {

// tq_decode_attend (n_qtok == 1) and tq_decode_attend_multi share every check
// and the launch.
tq_status decode_attend(const char* fn, const tq_codec* kc, const tq_codec* vc,
                        const void* q_fp16, int batch, int n_qtok, int n_q_heads,
                        int n_kv_heads, const uint8_t* k_codes, const float* k_norms,
                        const uint8_t* v_codes, const float* v_norms, int max_ctx,
                        const int32_t* lengths, int max_len, float scale, float* out,
                        void* workspace, size_t workspace_bytes, const tq::RawSegment& raw,
                        void* stream, bool raw_k = false,
                        const tq::ProdKeys* prodk = nullptr, bool use_scratch = false) {
  // raw_k: k_codes holds fp16 key rows, there is no K codec and no key norm
  if ((!kc && !raw_k) || !vc) return fail(TQ_ERR_INVALID_ARG, "%s: codec is NULL", fn);
  if (kc && kc->tabs.prod != (prodk != nullptr))
    return fail(TQ_ERR_INVALID_ARG, "%s: %s K codec (use %s)", fn,
                kc->tabs.prod ? "TurboQuant-Prod" : "plain",
                kc->tabs.prod ? "tq_decode_attend_prod" : "a call without sketch arrays");
  if (vc->tabs.prod) return fail(TQ_ERR_INVALID_ARG, "%s: V codec is a TurboQuant-Prod codec", fn);
  if (kc && kc->tabs.dim != vc->tabs.dim)
    return fail(TQ_ERR_INVALID_ARG, "%s: K dim %d != V dim %d", fn, kc->tabs.dim,
                vc->tabs.dim);
  const int dim = vc->tabs.dim;
  const bool dense = vc->dense || (kc && kc->dense);
  if (dense && (!kc || !kc->dense || !vc->dense || n_qtok != 1 || raw.lengths))
    return fail(TQ_ERR_UNSUPPORTED,
                "%s: dense-rotation codecs are attended only by tq_decode_attend with dense "
                "K and V codecs",
                fn);
  const int k_bits = raw_k ? 16 : (prodk ? 32 + kc->tabs.bits : kc->tabs.bits);
  if (batch <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_qtok <= 0)
    return fail(TQ_ERR_INVALID_ARG,
                "%s: batch %d, query tokens %d, heads %d/%d must be positive", fn, batch,
                n_qtok, n_q_heads, n_kv_heads);
  if (n_q_heads % n_kv_heads)
    return fail(TQ_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d", fn, n_q_heads,
                n_kv_heads);
  if ((long long)(n_q_heads / n_kv_heads) * n_qtok > 16)
    return fail(TQ_ERR_UNSUPPORTED, "%s: group size %d x %d query tokens > 16", fn,
                n_q_heads / n_kv_heads, n_qtok);
  if (batch > 65535 || n_kv_heads > 65535)
    return fail(TQ_ERR_UNSUPPORTED, "%s: batch or kv heads above 65535", fn);
  if (max_len <= 0 || max_len > max_ctx)
    return fail(TQ_ERR_INVALID_ARG, "%s: need 1 <= max_len (%d) <= max_ctx (%d)", fn, max_len,
                max_ctx);
  if (!q_fp16 || !k_codes || (!k_norms && !raw_k) || !v_codes || !v_norms || !lengths || !out)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (((uintptr_t)k_codes & 15) || ((uintptr_t)v_codes & 15) || ((uintptr_t)k_norms & 3) ||
      ((uintptr_t)v_norms & 3) || ((uintptr_t)out & 3) || ((uintptr_t)lengths & 3) ||
      ((uintptr_t)q_fp16 & 1))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned pointer", fn);
  if (!(scale == scale)) return fail(TQ_ERR_INVALID_ARG, "%s: scale is NaN", fn);
  const int group = n_q_heads / n_kv_heads;
  // The caller's workspace, or (use_scratch) this device's fixed scratch
  // array, checked against what the plan needs.
  auto take_workspace = [&](size_t need) -> tq_status {
    if (use_scratch) {
      if (need > (size_t)TQ_NOALLOC_SCRATCH_BYTES)
        return fail(TQ_ERR_UNSUPPORTED,
                    "%s: this shape needs %zu bytes of scratch, more than the fixed %zu", fn,
                    need, (size_t)TQ_NOALLOC_SCRATCH_BYTES);
      void* p = nullptr;
      const hipError_t e = tq::scratch_region(&p);
      if (e != hipSuccess)
        return fail(TQ_ERR_HIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
      workspace = p;
      workspace_bytes = (size_t)TQ_NOALLOC_SCRATCH_BYTES;
      return TQ_OK;
    }
    if (!workspace || workspace_bytes < need)
      return fail(TQ_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn,
                  workspace ? workspace_bytes : (size_t)0, need);
    if ((uintptr_t)workspace & 255)
      return fail(TQ_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    return TQ_OK;
  };
  // Walsh-Hadamard codec pairs with no matrix-core instance run the dense
  // kernels with m = H diag(sigma) formed from the codecs' signs (the same
  // result as the dense codec with that matrix): every bit width pair is served
  const bool fast = !dense && tq::attend_supported(dim, k_bits, vc->tabs.bits, group * n_qtok);
  const bool wht_fallback = !dense && !fast && n_qtok == 1 && !raw.lengths && !prodk && !raw_k;
  // one query head per KV head at the register-held kernel's shapes: that
  // kernel also serves Walsh-Hadamard codec pairs (the matrix-core one would
  // carry one head in each 4-head block)
  const bool wht_lt = !dense && n_qtok == 1 && !raw.lengths && !prodk && !raw_k &&
                      tq::dense_lt_supported(dim, k_bits, vc->tabs.bits, group);
  if (dense || wht_fallback || wht_lt) {
    const tq::AttendPlan dplan = tq::plan_attend(batch, n_q_heads, n_kv_heads, dim, max_len);
    const tq_status ws = take_workspace(dplan.total_bytes);
    if (ws != TQ_OK) return ws;
    tq::DenseAttendArgs da;
    std::memset(&da, 0, sizeof(da));
    da.q = q_fp16;
    if (dense) {
      da.mt_k = kc->mt_dev;
      da.m_v = vc->m_dev;
      da.lds_limit = tq::kDenseLdsFull;  // raised at codec set-up
    } else {
      da.wht = 1;
      da.wht_k = sign_arg(kc);
      da.wht_v = sign_arg(vc);
      da.lds_limit = tq::kDenseLdsDefault;
    }
    da.k_codes = k_codes;
    da.k_norms = k_norms;
    da.v_codes = v_codes;
    da.v_norms = v_norms;
    da.lengths = lengths;
    da.pacc = (float*)workspace;
    da.pml = (float*)((char*)workspace + dplan.part_acc_bytes);
    da.out = out;
    da.dim = dim;
    da.k_bits = kc->tabs.bits;
    da.v_bits = vc->tabs.bits;
    da.n_q_heads = n_q_heads;
    da.n_kv_heads = n_kv_heads;
    da.group = group;
    da.max_ctx = max_ctx;
    da.splits = dplan.splits;
    da.tokens_per_split = dplan.tokens_per_split;
    da.max_len = max_len;
    da.qscale = tq::dense_qscale(scale, dim);
    std::memcpy(da.k_centroids, kc->tabs.centroids, sizeof(float) * (1 << da.k_bits));
    std::memcpy(da.v_centroids, vc->tabs.centroids, sizeof(float) * (1 << da.v_bits));
    const hipError_t err = tq::launch_attend_dense(da, batch, (hipStream_t)stream);
    if (err != hipSuccess)
      return fail(TQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
    return ok();
  }
  if (!fast)
    return fail(TQ_ERR_UNSUPPORTED,
                "%s: no kernel for dim %d, K %d-bit%s, V %d-bit, %d heads per KV head", fn, dim,
                prodk ? kc->tabs.bits + 1 : k_bits, prodk ? " Prod" : "", vc->tabs.bits,
                group * n_qtok);
  const tq::AttendPlan plan =
      tq::plan_attend(batch, n_q_heads * n_qtok, n_kv_heads, dim, max_len);
  if ((long long)plan.splits > 0x7fffffffLL)
    return fail(TQ_ERR_UNSUPPORTED, "%s: context too long", fn);
  const tq_status ws = take_workspace(plan.total_bytes);
  if (ws != TQ_OK) return ws;
  tq::AttendTables tabs;
  tq::SignArg ksign;
  if (raw_k) {
    std::memset(tabs.k_centroids, 0, sizeof(tabs.k_centroids));
    std::memset(&ksign, 0, sizeof(ksign));
  } else {
    std::memcpy(tabs.k_centroids, kc->tabs.centroids, sizeof(tabs.k_centroids));
    ksign = sign_arg(kc);
  }
  std::memcpy(tabs.v_centroids, vc->tabs.centroids, sizeof(tabs.v_centroids));
  hipError_t err = tq::launch_attend(dim, k_bits, vc->tabs.bits, batch, n_qtok,
                                     n_q_heads, n_kv_heads, q_fp16, ksign, sign_arg(vc),
                                     tabs, k_codes, k_norms, v_codes, v_norms, max_ctx, lengths,
                                     max_len, scale, out, workspace, plan, raw,
                                     prodk ? *prodk : tq::ProdKeys{}, g_split_before,
                                     g_split_after, (hipStream_t)stream);
  if (err != hipSuccess) return fail(TQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_decode_attend(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                           int batch, int n_q_heads, int n_kv_heads,
                           const uint8_t* k_codes, const float* k_norms,
                           const uint8_t* v_codes, const float* v_norms, int max_ctx,
                           const int32_t* lengths, int max_len, float scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return decode_attend("tq_decode_attend", kc, vc, q_fp16, batch, 1, n_q_heads, n_kv_heads,
                       k_codes, k_norms, v_codes, v_norms, max_ctx, lengths, max_len, scale,
                       out, workspace, workspace_bytes, tq::RawSegment{}, stream);
}

tq_status tq_decode_attend_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                   int batch, int n_q_heads, int n_kv_heads,
                                   const uint8_t* k_codes, const float* k_norms,
                                   const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                   const int32_t* lengths, int max_len, float scale, float* out,
                                   void* stream) {
  return decode_attend("tq_decode_attend_noalloc", kc, vc, q_fp16, batch, 1, n_q_heads,
                       n_kv_heads, k_codes, k_norms, v_codes, v_norms, max_ctx, lengths,
                       max_len, scale, out, nullptr, 0, tq::RawSegment{}, stream, false,
                       nullptr, true);
}

size_t tq_attend_multi_workspace_bytes(int batch, int n_query_tokens, int n_q_heads,
                                       int n_kv_heads, int dim, int max_len) {
  if (n_query_tokens <= 0 || (long long)n_q_heads * n_query_tokens > 0x7fffffffLL) return 0;
  if (!attend_shape_ok(batch, n_q_heads, n_kv_heads, dim, max_len)) return 0;
  return tq::plan_attend(batch, n_q_heads * n_query_tokens, n_kv_heads, dim, max_len)
      .total_bytes;
}

tq_status tq_decode_attend_multi(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                 int batch, int n_query_tokens, int n_q_heads, int n_kv_heads,
                                 const uint8_t* k_codes, const float* k_norms,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return decode_attend("tq_decode_attend_multi", kc, vc, q_fp16, batch, n_query_tokens,
                       n_q_heads, n_kv_heads, k_codes, k_norms, v_codes, v_norms, max_ctx,
                       lengths, max_len, scale, out, workspace, workspace_bytes,
                       tq::RawSegment{}, stream);
}

tq_status tq_decode_attend_prod(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                int batch, int n_q_heads, int n_kv_heads,
                                const uint8_t* k_codes, const uint8_t* k_sketch,
                                const float* k_norms, const float* k_rnorms,
                                const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                const int32_t* lengths, int max_len, float scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tq_decode_attend_prod";
  if (!kc || !kc->tabs.prod)
    return fail(TQ_ERR_INVALID_ARG, "%s: K codec must be a TurboQuant-Prod codec", fn);
  if (!k_sketch || !k_rnorms) return fail(TQ_ERR_INVALID_ARG, "%s: NULL sketch pointer", fn);
  if (((uintptr_t)k_sketch & 15) || ((uintptr_t)k_rnorms & 3))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned sketch or residual-norm pointer", fn);
  tq::ProdKeys pk;
  pk.sketch = k_sketch;
  pk.rnorms = k_rnorms;
  std::memcpy(pk.sign.bits, kc->tabs.sketch_sign_bits, sizeof(pk.sign.bits));
  return decode_attend(fn, kc, vc, q_fp16, batch, 1, n_q_heads, n_kv_heads, k_codes, k_norms,
                       v_codes, v_norms, max_ctx, lengths, max_len, scale, out, workspace,
                       workspace_bytes, tq::RawSegment{}, stream, false, &pk);
}

tq_status tq_decode_attend_raw_k(const tq_codec* vc, const void* q_fp16, int batch,
                                 int n_q_heads, int n_kv_heads, const void* k_fp16,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return decode_attend("tq_decode_attend_raw_k", nullptr, vc, q_fp16, batch, 1, n_q_heads,
                       n_kv_heads, (const uint8_t*)k_fp16, nullptr, v_codes, v_norms, max_ctx,
                       lengths, max_len, scale, out, workspace, workspace_bytes,
                       tq::RawSegment{}, stream, true);
}

tq_status tq_decode_attend_mixed(const tq_codec* kc, const tq_codec* vc, const void* q_fp16,
                                 int batch, int n_q_heads, int n_kv_heads,
                                 const uint8_t* k_codes, const float* k_norms,
                                 const uint8_t* v_codes, const float* v_norms, int max_ctx,
                                 const int32_t* lengths, int max_len, const void* raw_k_fp16,
                                 const void* raw_v_fp16, int max_raw,
                                 const int32_t* raw_lengths, float scale, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tq_decode_attend_mixed";
  if (max_raw <= 0) return fail(TQ_ERR_INVALID_ARG, "%s: max_raw %d must be positive", fn, max_raw);
  if (max_raw > 4096)
    return fail(TQ_ERR_UNSUPPORTED, "%s: max_raw %d above 4096 raw rows", fn, max_raw);
  if (!raw_k_fp16 || !raw_v_fp16 || !raw_lengths)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL raw segment pointer", fn);
  if (((uintptr_t)raw_k_fp16 & 15) || ((uintptr_t)raw_v_fp16 & 15) ||
      ((uintptr_t)raw_lengths & 3))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned raw segment pointer", fn);
  tq::RawSegment raw;
  raw.k = raw_k_fp16;
  raw.v = raw_v_fp16;
  raw.lengths = raw_lengths;
  raw.max_raw = max_raw;
  return decode_attend(fn, kc, vc, q_fp16, batch, 1, n_q_heads, n_kv_heads, k_codes, k_norms,
                       v_codes, v_norms, max_ctx, lengths, max_len, scale, out, workspace,
                       workspace_bytes, raw, stream);
}

}  // extern "C"

// ------------------------------------------------------------ two-phase cache

namespace {

// Rows [row0, row0 + n) of the fp16 array x ([heads][rows_per_head][dim]) as
// an encode job writing packed positions [pos, pos + n).
tq_encode_job cache_job(const tq_codec* c, const void* x, int rows_per_head, int row0,
                        uint8_t* codes, float* norms, int max_ctx, int pos) {
  const int dim = c->tabs.dim;
  const int64_t rb = (int64_t)dim * c->tabs.bits / 8;
  tq_encode_job j;
  j.codec = c;
  j.x_fp16 = (const uint16_t*)x + (int64_t)row0 * dim;
  j.x_stride_tok = dim;
  j.x_stride_head = (int64_t)rows_per_head * dim;
  j.codes = codes + (int64_t)pos * rb;
  j.c_stride_tok = rb;
  j.c_stride_head = (int64_t)max_ctx * rb;
  j.norms = norms + pos;
  j.n_stride_tok = 1;
  j.n_stride_head = max_ctx;
  return j;
}

// One launch: K and V rows [row0, row0 + rows) of src ([heads][src_rows][dim])
// to pending rows [dst_row0, ..) and the counts n_packed / n_pending published
// to the length arrays. The caller commits those counts to the host state only
// once this has returned TQ_OK, so a failed launch leaves host and device agreeing.
tq_status cache_move_rows(tq_cache* c, const char* fn, const void* src_k, const void* src_v,
                          int src_rows, int row0, int dst_row0, int rows, int n_packed,
                          int n_pending, void* stream) {
  const int dim = c->kc->tabs.dim;
  const int row16 = dim / 8;  // 16-byte words per fp16 row
  tq::CopyRowsArgs a;
  a.src_k = (const char*)src_k + (int64_t)row0 * dim * 2;
  a.src_v = (const char*)src_v + (int64_t)row0 * dim * 2;
  a.dst_k = (char*)c->d.pending_k + (int64_t)dst_row0 * dim * 2;
  a.dst_v = (char*)c->d.pending_v + (int64_t)dst_row0 * dim * 2;
  a.src_head = (long long)src_rows * row16;
  a.dst_head = (long long)c->d.group_size * row16;
  a.row16 = row16;
  a.rows = rows;
  a.heads = c->d.batch * c->d.n_kv_heads;
  a.batch = c->d.batch;
  a.n_packed = n_packed;
  a.n_pending = n_pending;
  a.packed_len = c->d.packed_len;
  a.pending_len = c->d.pending_len;
  hipError_t err = tq::launch_pending_rows(a, (hipStream_t)stream);
  if (err != hipSuccess) return fail(TQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(err));
  c->lengths_published = true;
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_cache_init(const tq_codec* kc, const tq_codec* vc, const tq_cache_desc* desc,
                        tq_cache** out) {
  const char* fn = "tq_cache_init";
  if (!out) return fail(TQ_ERR_INVALID_ARG, "%s: out is NULL", fn);
  *out = nullptr;
  if (!kc || !vc || !desc) return fail(TQ_ERR_INVALID_ARG, "%s: NULL codec or descriptor", fn);
  if (kc->tabs.prod || vc->tabs.prod)
    return fail(TQ_ERR_INVALID_ARG, "%s: TurboQuant-Prod codecs are not cached here", fn);
  if (kc->dense || vc->dense)
    return fail(TQ_ERR_UNSUPPORTED, "%s: dense-rotation codecs are not cached here", fn);
  if (kc->tabs.dim != vc->tabs.dim)
    return fail(TQ_ERR_INVALID_ARG, "%s: K dim %d != V dim %d", fn, kc->tabs.dim, vc->tabs.dim);
  const tq_cache_desc& d = *desc;
  if (d.batch <= 0 || d.n_kv_heads <= 0 || d.max_ctx <= 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: batch %d, kv heads %d, max_ctx %d must be positive", fn,
                d.batch, d.n_kv_heads, d.max_ctx);
  if (d.batch > 65535 || d.n_kv_heads > 65535)
    return fail(TQ_ERR_UNSUPPORTED, "%s: batch or kv heads above 65535", fn);
  if ((long long)d.batch * d.n_kv_heads > 0x7fffffffLL / 4096)
    return fail(TQ_ERR_UNSUPPORTED, "%s: too many (sequence, KV head) pairs", fn);
  if (d.group_size < 1 || d.group_size > 4096)
    return fail(TQ_ERR_INVALID_ARG, "%s: group_size %d outside 1..4096", fn, d.group_size);
  if (!d.k_codes || !d.k_norms || !d.v_codes || !d.v_norms || !d.pending_k || !d.pending_v ||
      !d.packed_len || !d.pending_len)
    return fail(TQ_ERR_INVALID_ARG, "%s: NULL buffer in the descriptor", fn);
  if (((uintptr_t)d.k_codes & 15) || ((uintptr_t)d.v_codes & 15) || ((uintptr_t)d.k_norms & 3) ||
      ((uintptr_t)d.v_norms & 3) || ((uintptr_t)d.pending_k & 15) ||
      ((uintptr_t)d.pending_v & 15) || ((uintptr_t)d.packed_len & 3) ||
      ((uintptr_t)d.pending_len & 3))
    return fail(TQ_ERR_INVALID_ARG, "%s: misaligned buffer in the descriptor", fn);
  tq_cache* c = new (std::nothrow) tq_cache;
  if (!c) return fail(TQ_ERR_NOMEM, "%s: out of host memory", fn);
  c->kc = kc;
  c->vc = vc;
  c->d = d;
  *out = c;
  return ok();
}

void tq_cache_destroy(tq_cache* c) { delete c; }

tq_status tq_cache_state(const tq_cache* c, int* n_packed, int* n_pending) {
  if (!c || !n_packed || !n_pending) return fail(TQ_ERR_INVALID_ARG, "tq_cache_state: NULL argument");
  *n_packed = c->n_packed;
  *n_pending = c->n_pending;
  return ok();
}

tq_status tq_cache_append(tq_cache* c, const void* k_fp16, const void* v_fp16, int n_tok,
                          void* stream) {
  const char* fn = "tq_cache_append";
  if (!c) return fail(TQ_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  if (n_tok < 0) return fail(TQ_ERR_INVALID_ARG, "%s: n_tok %d is negative", fn, n_tok);
  if (n_tok == 0) return ok();
  if (!k_fp16 || !v_fp16) return fail(TQ_ERR_INVALID_ARG, "%s: NULL rows", fn);
  if (((uintptr_t)k_fp16 & 15) || ((uintptr_t)v_fp16 & 15))
    return fail(TQ_ERR_INVALID_ARG, "%s: rows must be 16-byte aligned", fn);
  const tq_cache_desc& d = c->d;
  const long long G = d.group_size, P = c->n_pending;
  const long long total = P + n_tok;
  const long long groups = total / G;
  const long long new_packed = c->n_packed + groups * G;
  if (new_packed > d.max_ctx)
    return fail(TQ_ERR_INVALID_ARG, "%s: %lld packed rows would exceed max_ctx %d", fn, new_packed,
                d.max_ctx);
  const int heads = d.batch * d.n_kv_heads;
  tq_status st;
  if (groups == 0) {
    // the rows join the pending buffer
    if ((st = cache_move_rows(c, fn, k_fp16, v_fp16, n_tok, 0, (int)P, n_tok, c->n_packed,
                              (int)total, stream)) != TQ_OK)
      return st;
    c->n_pending = (int)total;
    return ok();
  }
  // whole groups: the pending rows first, then the leading new rows
  if (P > 0) {
    const tq_encode_job kj = cache_job(c->kc, d.pending_k, d.group_size, 0, d.k_codes, d.k_norms,
                                       d.max_ctx, c->n_packed);
    const tq_encode_job vj = cache_job(c->vc, d.pending_v, d.group_size, 0, d.v_codes, d.v_norms,
                                       d.max_ctx, c->n_packed);
    tq_encode_job jobs[2] = {kj, vj};
    if ((st = encode_jobs(fn, jobs, 2, (int)P, heads, stream)) != TQ_OK) return st;
  }
  const int from_new = (int)(groups * G - P);
  {
    const tq_encode_job kj = cache_job(c->kc, k_fp16, n_tok, 0, d.k_codes, d.k_norms, d.max_ctx,
                                       c->n_packed + (int)P);
    const tq_encode_job vj = cache_job(c->vc, v_fp16, n_tok, 0, d.v_codes, d.v_norms, d.max_ctx,
                                       c->n_packed + (int)P);
    tq_encode_job jobs[2] = {kj, vj};
    if ((st = encode_jobs(fn, jobs, 2, from_new, heads, stream)) != TQ_OK) return st;
  }
  // the rest of the new rows start the next pending group; the encodes above
  // wrote only rows past the published packed length, so until this launch
  // succeeds the device state still matches the old counts
  const int rest = n_tok - from_new;
  if ((st = cache_move_rows(c, fn, k_fp16, v_fp16, n_tok, from_new, 0, rest, (int)new_packed,
                            rest, stream)) != TQ_OK)
    return st;
  c->n_packed = (int)new_packed;
  c->n_pending = rest;
  return ok();
}

size_t tq_cache_workspace_bytes(const tq_cache* c, int n_q_heads) {
  if (!c) return 0;
  return tq_attend_workspace_bytes(c->d.batch, n_q_heads, c->d.n_kv_heads, c->kc->tabs.dim,
                                   c->d.max_ctx);
}

tq_status tq_cache_attend(tq_cache* c, const void* q_fp16, int n_q_heads, float scale,
                          float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tq_cache_attend";
  if (!c) return fail(TQ_ERR_INVALID_ARG, "%s: cache is NULL", fn);
  const tq_cache_desc& d = c->d;
  if (!c->lengths_published) {
    tq_status st = cache_move_rows(c, fn, d.pending_k, d.pending_v, d.group_size, 0, 0, 0,
                                   c->n_packed, c->n_pending, stream);
    if (st != TQ_OK) return st;
  }
  return tq_decode_attend_mixed(c->kc, c->vc, q_fp16, d.batch, n_q_heads, d.n_kv_heads,
                                d.k_codes, d.k_norms, d.v_codes, d.v_norms, d.max_ctx,
                                d.packed_len, c->n_packed > 0 ? c->n_packed : 1, d.pending_k,
                                d.pending_v, d.group_size, d.pending_len, scale, out, workspace,
                                workspace_bytes, stream);
}

}  // extern "C"

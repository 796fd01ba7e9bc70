/*
 * c_abi_client.c -- a plain C caller of the library, with no Python and no
 * torch: device memory from hipMalloc, the codecs, tq_encode of the K and V
 * caches and tq_decode_attend, exactly as a C program would use include/tq.h.
 * The GPU parity test writes the inputs, runs this program and checks what it
 * writes against the oracle.
 *
 *   c_abi_client IN OUT
 *
 * IN (little endian): int32 B, Hq, Hkv, d, T, k_bits, v_bits; uint64 seed;
 *   int32 lengths[B]; fp16 k[B][Hkv][T][d]; fp16 v[B][Hkv][T][d];
 *   fp16 q[B][Hq][d].
 * OUT: uint8 k_codes[B][Hkv][T][d*k_bits/8]; float k_norms[B][Hkv][T];
 *   uint8 v_codes[..]; float v_norms[..]; float out[B][Hq][d].
 * Exit status 0 on success; otherwise the failing call and tq_last_error()
 * are printed to stderr.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/tq.h"

#define CHECK_HIP(call)                                                         \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
      return 1;                                                                 \
    }                                                                           \
  } while (0)
#define CHECK_TQ(call)                                                          \
  do {                                                                          \
    tq_status s_ = (call);                                                      \
    if (s_ != TQ_OK) {                                                          \
      fprintf(stderr, "%s: %s (%s)\n", #call, tq_status_string(s_), tq_last_error()); \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

static int read_all(FILE* f, void* dst, size_t n) { return fread(dst, 1, n, f) == n ? 0 : -1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* fin = fopen(argv[1], "rb");
  if (!fin) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int32_t hdr[7];
  uint64_t seed;
  if (read_all(fin, hdr, sizeof(hdr)) || read_all(fin, &seed, sizeof(seed))) return 2;
  const int B = hdr[0], Hq = hdr[1], Hkv = hdr[2], d = hdr[3], T = hdr[4];
  const int kb = hdr[5], vb = hdr[6];
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || T <= 0 || kb <= 0 || vb <= 0) return 2;
  const size_t nkv = (size_t)B * Hkv * T, nq = (size_t)B * Hq;
  int32_t* lengths = (int32_t*)malloc(sizeof(int32_t) * B);
  uint16_t* k = (uint16_t*)malloc(2 * nkv * d);
  uint16_t* v = (uint16_t*)malloc(2 * nkv * d);
  uint16_t* q = (uint16_t*)malloc(2 * nq * d);
  if (!lengths || !k || !v || !q) return 2;
  if (read_all(fin, lengths, sizeof(int32_t) * B) || read_all(fin, k, 2 * nkv * d) ||
      read_all(fin, v, 2 * nkv * d) || read_all(fin, q, 2 * nq * d))
    return 2;
  fclose(fin);
  int max_len = 1;
  for (int b = 0; b < B; ++b) max_len = lengths[b] > max_len ? lengths[b] : max_len;

  tq_codec *kc = NULL, *vc = NULL;
  CHECK_TQ(tq_codec_init(d, kb, seed, &kc));
  CHECK_TQ(tq_codec_init(d, vb, seed, &vc));
  const int kr = tq_row_bytes(d, kb), vr = tq_row_bytes(d, vb);

  void *dk, *dv, *dq, *dout, *dlen, *ws;
  uint8_t *dkc, *dvc;
  float *dkn, *dvn;
  CHECK_HIP(hipMalloc(&dk, 2 * nkv * d));
  CHECK_HIP(hipMalloc(&dv, 2 * nkv * d));
  CHECK_HIP(hipMalloc(&dq, 2 * nq * d));
  CHECK_HIP(hipMalloc((void**)&dkc, nkv * kr));
  CHECK_HIP(hipMalloc((void**)&dvc, nkv * vr));
  CHECK_HIP(hipMalloc((void**)&dkn, sizeof(float) * nkv));
  CHECK_HIP(hipMalloc((void**)&dvn, sizeof(float) * nkv));
  CHECK_HIP(hipMalloc(&dout, sizeof(float) * nq * d));
  CHECK_HIP(hipMalloc(&dlen, sizeof(int32_t) * B));
  const size_t ws_bytes = tq_attend_workspace_bytes(B, Hq, Hkv, d, max_len);
  if (ws_bytes == 0) {
    fprintf(stderr, "tq_attend_workspace_bytes: shape rejected\n");
    return 1;
  }
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  CHECK_HIP(hipMemcpy(dk, k, 2 * nkv * d, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, v, 2 * nkv * d, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dq, q, 2 * nq * d, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dlen, lengths, sizeof(int32_t) * B, hipMemcpyHostToDevice));

  /* the caches [B][Hkv][T][row]: token t of head slot h = b*Hkv + g */
  const int nh = B * Hkv;
  CHECK_TQ(tq_encode(kc, dk, T, nh, d, (int64_t)T * d, dkc, kr, (int64_t)T * kr, dkn, 1, T, NULL));
  CHECK_TQ(tq_encode(vc, dv, T, nh, d, (int64_t)T * d, dvc, vr, (int64_t)T * vr, dvn, 1, T, NULL));
  CHECK_TQ(tq_decode_attend(kc, vc, dq, B, Hq, Hkv, dkc, dkn, dvc, dvn, T, (const int32_t*)dlen,
                            max_len, (float)(1.0 / sqrt((double)d)), (float*)dout, ws, ws_bytes,
                            NULL));
  CHECK_HIP(hipDeviceSynchronize());

  uint8_t* hkc = (uint8_t*)malloc(nkv * kr);
  uint8_t* hvc = (uint8_t*)malloc(nkv * vr);
  float* hkn = (float*)malloc(sizeof(float) * nkv);
  float* hvn = (float*)malloc(sizeof(float) * nkv);
  float* hout = (float*)malloc(sizeof(float) * nq * d);
  if (!hkc || !hvc || !hkn || !hvn || !hout) return 2;
  CHECK_HIP(hipMemcpy(hkc, dkc, nkv * kr, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hvc, dvc, nkv * vr, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hkn, dkn, sizeof(float) * nkv, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hvn, dvn, sizeof(float) * nkv, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hout, dout, sizeof(float) * nq * d, hipMemcpyDeviceToHost));
  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  fwrite(hkc, 1, nkv * kr, fo);
  fwrite(hkn, sizeof(float), nkv, fo);
  fwrite(hvc, 1, nkv * vr, fo);
  fwrite(hvn, sizeof(float), nkv, fo);
  fwrite(hout, sizeof(float), nq * d, fo);
  fclose(fo);

  tq_codec_destroy(kc);
  tq_codec_destroy(vc);
  hipFree(dk); hipFree(dv); hipFree(dq); hipFree(dkc); hipFree(dvc); hipFree(dkn);
  hipFree(dvn); hipFree(dout); hipFree(dlen); hipFree(ws);
  free(lengths); free(k); free(v); free(q); free(hkc); free(hvc); free(hkn); free(hvn);
  free(hout);
  return 0;
}

/*
 * A C caller of the library, with no Python or PyTorch in the process: it reads one
 * problem from a file, runs the one-call loss on device memory from hipMalloc and on a
 * stream of its own, runs the forward and backward halves on the same inputs, checks
 * that an invalid teacher index is refused with the outputs untouched, and writes what
 * it got.  tests/test_c_abi_gpu.py writes the problem and compares the outputs with the
 * oracle.
 *
 *   kd_driver IN OUT
 *
 * IN:  int64 magic 0x4C4B444B, dtype (KD_F32 or KD_BF16), N, d, V, K, chunk; then
 *      h [N][d] and W [V][d] (float32, or bfloat16 bit patterns), idx [N][K] int32,
 *      p [N][K] float32, mask [N] uint8.
 * OUT: one-call form: loss (float32), dh [N][d] (h's type), dW [V][d] float32,
 *      row_loss [N], row_lse [N], zg [N][K] (float32); split form: loss, dh, dW;
 *      then int32 return code of the call with a bad index, int32 1 if
 *      kd_last_error() described it, int32 1 if loss and dh were left untouched.
 * Exit status 0 when every call returned as expected, 1 on a usage or I/O error, 2 on
 * a HIP error, 3 on an unexpected library return code.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kdkl.h"

#define HIP(x)                                                                         \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      fprintf(stderr, "kd_driver: %s: %s\n", #x, hipGetErrorString(e_));               \
      exit(2);                                                                         \
    }                                                                                  \
  } while (0)

#define KD(x, want)                                                                    \
  do {                                                                                 \
    int r_ = (x);                                                                      \
    if (r_ != (want)) {                                                                \
      fprintf(stderr, "kd_driver: %s returned %d (%s), expected %d\n", #x, r_,         \
              kd_last_error(), (want));                                                \
      exit(3);                                                                         \
    }                                                                                  \
  } while (0)

static void *read_all(FILE *f, size_t bytes) {
  void *p = malloc(bytes ? bytes : 1);
  if (!p || fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "kd_driver: short input\n");
    exit(1);
  }
  return p;
}

static void *to_device(const void *host, size_t bytes) {
  void *d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void write_back(FILE *f, const void *dev, size_t bytes) {
  void *h = malloc(bytes ? bytes : 1);
  if (!h) exit(1);
  if (bytes) HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "kd_driver: write failed\n");
    exit(1);
  }
  free(h);
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: kd_driver IN OUT\n");
    return 1;
  }
  FILE *fi = fopen(argv[1], "rb");
  if (!fi) {
    perror(argv[1]);
    return 1;
  }
  int64_t hd[7];
  if (fread(hd, sizeof hd, 1, fi) != 1 || hd[0] != 0x4C4B444B) {
    fprintf(stderr, "kd_driver: not a problem file\n");
    return 1;
  }
  const int32_t dtype = (int32_t)hd[1];
  const int64_t N = hd[2], d = hd[3], V = hd[4], chunk = hd[6];
  const int32_t K = (int32_t)hd[5];
  const size_t es = dtype == KD_BF16 ? 2 : 4;
  void *h_h = read_all(fi, (size_t)N * d * es);
  void *h_W = read_all(fi, (size_t)V * d * es);
  int32_t *h_idx = (int32_t *)read_all(fi, (size_t)N * K * 4);
  void *h_p = read_all(fi, (size_t)N * K * 4);
  void *h_mask = read_all(fi, (size_t)N);
  fclose(fi);

  HIP(hipSetDevice(0));
  hipStream_t s;
  HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  void *h = to_device(h_h, (size_t)N * d * es), *W = to_device(h_W, (size_t)V * d * es);
  int32_t *idx = (int32_t *)to_device(h_idx, (size_t)N * K * 4);
  float *p = (float *)to_device(h_p, (size_t)N * K * 4);
  uint8_t *mask = (uint8_t *)to_device(h_mask, (size_t)N);
  float *loss, *dW, *row_loss, *row_lse, *zg, *loss2, *dW2, *lse2;
  void *dh, *dh2, *ws;
  HIP(hipMalloc((void **)&loss, 4));
  HIP(hipMalloc((void **)&loss2, 4));
  HIP(hipMalloc(&dh, (size_t)N * d * es + 16));
  HIP(hipMalloc(&dh2, (size_t)N * d * es + 16));
  HIP(hipMalloc((void **)&dW, (size_t)V * d * 4));
  HIP(hipMalloc((void **)&dW2, (size_t)V * d * 4));
  HIP(hipMalloc((void **)&row_loss, (size_t)N * 4 + 16));
  HIP(hipMalloc((void **)&row_lse, (size_t)N * 4 + 16));
  HIP(hipMalloc((void **)&lse2, (size_t)N * 4 + 16));
  HIP(hipMalloc((void **)&zg, (size_t)N * K * 4 + 16));
  size_t wsb = 0;
  KD(kd_workspace_bytes(N, d, V, K, chunk, dtype, &wsb), KD_OK);
  HIP(hipMalloc(&ws, wsb));

  /* one call: loss, dh, dW and the per-row outputs */
  KD(kd_chunked_kl_fwd_bwd(h, W, dtype, idx, p, mask, N, d, V, K, chunk, loss, dh, dW, row_loss,
                           row_lse, zg, ws, wsb, s),
     KD_OK);
  /* the two halves, with an upstream gradient of 1 read on the device */
  float one = 1.f, *g;
  HIP(hipMalloc((void **)&g, 4));
  HIP(hipMemcpy(g, &one, 4, hipMemcpyHostToDevice));
  KD(kd_chunked_kl_fwd(h, W, dtype, idx, p, mask, N, d, V, K, chunk, loss2, lse2, NULL, NULL, ws,
                       wsb, s),
     KD_OK);
  KD(kd_chunked_kl_bwd(h, W, dtype, idx, p, mask, N, d, V, K, chunk, lse2, g, dh2, dW2, ws, wsb,
                       s),
     KD_OK);
  HIP(hipStreamSynchronize(s));

  /* a teacher index outside [0, V): refused after validation, outputs untouched */
  const float sentinel = -12345.f;
  float *sent, *dW_bad;
  HIP(hipMalloc((void **)&sent, 4));
  HIP(hipMalloc((void **)&dW_bad, (size_t)V * d * 4));
  HIP(hipMemcpy(sent, &sentinel, 4, hipMemcpyHostToDevice));
  void *dh_before = malloc((size_t)N * d * es + 1);
  HIP(hipMemcpy(dh_before, dh, (size_t)N * d * es, hipMemcpyDeviceToHost));
  h_idx[0] = (int32_t)V;
  HIP(hipMemcpy(idx, h_idx, 4, hipMemcpyHostToDevice));
  const int32_t rc_bad = kd_chunked_kl_fwd_bwd(h, W, dtype, idx, p, mask, N, d, V, K, chunk, sent,
                                               dh, dW_bad, NULL, NULL, NULL, ws, wsb, s);
  const int32_t described = strlen(kd_last_error()) > 0 ? 1 : 0;
  HIP(hipStreamSynchronize(s));
  float sent_after = 0.f;
  HIP(hipMemcpy(&sent_after, sent, 4, hipMemcpyDeviceToHost));
  void *dh_after = malloc((size_t)N * d * es + 1);
  HIP(hipMemcpy(dh_after, dh, (size_t)N * d * es, hipMemcpyDeviceToHost));
  const int32_t untouched =
      sent_after == sentinel && memcmp(dh_before, dh_after, (size_t)N * d * es) == 0 ? 1 : 0;

  FILE *fo = fopen(argv[2], "wb");
  if (!fo) {
    perror(argv[2]);
    return 1;
  }
  write_back(fo, loss, 4);
  write_back(fo, dh, (size_t)N * d * es);
  write_back(fo, dW, (size_t)V * d * 4);
  write_back(fo, row_loss, (size_t)N * 4);
  write_back(fo, row_lse, (size_t)N * 4);
  write_back(fo, zg, (size_t)N * K * 4);
  write_back(fo, loss2, 4);
  write_back(fo, dh2, (size_t)N * d * es);
  write_back(fo, dW2, (size_t)V * d * 4);
  fwrite(&rc_bad, 4, 1, fo);
  fwrite(&described, 4, 1, fo);
  fwrite(&untouched, 4, 1, fo);
  if (fclose(fo) != 0) return 1;
  printf("kd_driver: N=%lld d=%lld V=%lld K=%d chunk=%lld dtype=%d workspace %zu bytes; "
         "bad index -> %d\n", (long long)N, (long long)d, (long long)V, K, (long long)chunk,
         dtype, wsb, rc_bad);
  return 0;
}

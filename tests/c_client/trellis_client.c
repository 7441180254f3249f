/*
 * A plain C client of the trellis C ABI (include/trellis.h), with no Python
 * or torch in the process: test infrastructure for the GPU test
 * tests/test_gpu_c_client.py.
 *
 * Usage: trellis_client IN OUT
 *   IN   int32 m, k, n, bits; then x bf16 [m, k], codes uint32 [n, k*bits/32],
 *        scales bf16 [n] (native byte order, no padding)
 *   OUT  int32 status of trellis_prefill, of trellis_decode, of a call with
 *        an unsupported m, and trellis_supported(g, m); then out bf16 [m, n]
 *        and w bf16 [n, k]
 * Device buffers come from hipMalloc; the calls run on a stream created here.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "trellis.h"

static int read_all(FILE *f, void *p, size_t bytes) { return fread(p, 1, bytes, f) == bytes; }

#define HIP_OK(call)                                                  \
  do {                                                                \
    if ((call) != hipSuccess) {                                       \
      fprintf(stderr, "%s failed at line %d\n", #call, __LINE__);     \
      return 2;                                                       \
    }                                                                 \
  } while (0)

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE *fi = fopen(argv[1], "rb");
  if (!fi) return 2;
  int32_t hdr[4];
  if (!read_all(fi, hdr, sizeof hdr)) return 2;
  const int32_t m = hdr[0], k = hdr[1], n = hdr[2], bits = hdr[3];
  const size_t xs = (size_t)m * k, cs = (size_t)n * k * bits / 32, os = (size_t)m * n, ws = (size_t)n * k;
  uint16_t *x = malloc(xs * 2), *sc = malloc((size_t)n * 2), *out = malloc(os * 2), *w = malloc(ws * 2);
  uint32_t *codes = malloc(cs * 4);
  if (!x || !sc || !out || !w || !codes) return 2;
  if (!read_all(fi, x, xs * 2) || !read_all(fi, codes, cs * 4) || !read_all(fi, sc, (size_t)n * 2)) return 2;
  fclose(fi);

  void *dx, *dc, *ds, *dout, *dw;
  HIP_OK(hipMalloc(&dx, xs * 2));
  HIP_OK(hipMalloc(&dc, cs * 4));
  HIP_OK(hipMalloc(&ds, (size_t)n * 2));
  HIP_OK(hipMalloc(&dout, os * 2));
  HIP_OK(hipMalloc(&dw, ws * 2));
  HIP_OK(hipMemcpy(dx, x, xs * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dc, codes, cs * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ds, sc, (size_t)n * 2, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  const trellis_geom g = {n, k, TRELLIS_T, TRELLIS_L, bits};
  int32_t res[4];
  res[0] = trellis_prefill(dx, m, dc, ds, g, dout, stream);
  res[1] = trellis_decode(dc, ds, g, dw, stream);
  res[2] = trellis_prefill(dx, TRELLIS_MIN_M - 1, dc, ds, g, dout, stream); /* rejected, nothing launched */
  res[3] = trellis_supported(g, m);
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(out, dout, os * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(w, dw, ws * 2, hipMemcpyDeviceToHost));
  printf("prefill: %s; decode: %s; m = %d: %s\n", trellis_status_string((trellis_status)res[0]),
         trellis_status_string((trellis_status)res[1]), TRELLIS_MIN_M - 1,
         trellis_status_string((trellis_status)res[2]));

  FILE *fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  if (fwrite(res, sizeof res, 1, fo) != 1 || fwrite(out, 2, os, fo) != os || fwrite(w, 2, ws, fo) != ws) return 2;
  fclose(fo);
  HIP_OK(hipStreamDestroy(stream));
  hipFree(dx);
  hipFree(dc);
  hipFree(ds);
  hipFree(dout);
  hipFree(dw);
  free(x);
  free(codes);
  free(sc);
  free(out);
  free(w);
  return 0;
}

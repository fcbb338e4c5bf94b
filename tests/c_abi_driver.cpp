// A C-style host program that uses libec.so through include/ec.h alone (HIP
// runtime for memory and streams; no Python, no torch).  It runs the entropy
// pass with its threshold decision and the row selection on inputs read from a
// file and writes what the library produced to another file; the GPU test
// tests/test_gpu_c_abi.py writes the inputs and checks the outputs.
//
// Input (little-endian):
//   int32 magic 0x45430001, n_rows, V, dtype (0 fp32, 1 bf16), n_decoded; float tau
//   logits   n_rows * V elements of dtype (row stride V)
//   decoded  n_decoded int32 row indices
//   int32 L, block_start, block_len, block_causal, history_cap, history_len, k, full_flag
//   uint8 is_masked[L]; int32 history[history_cap]
// Output:
//   int32 status of ec_entropy_max, of ec_select_rows, of a call with a NULL
//         logits pointer (must be EC_E_NULL), of a call with a short workspace
//         (must be EC_E_WORKSPACE)
//   float H[n_rows]; int32 argmax[n_rows]; float p1[n_rows]; float E; int32 flag
//   int32 n_sel; int32 rows[n_sel]
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ec.h"

static int fail(const char* what) {
  fprintf(stderr, "c_abi_driver: %s\n", what);
  return 1;
}

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "c_abi_driver: %s: %s\n", #x, hipGetErrorString(e_)); \
      return 1;                                                            \
    }                                                                      \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes; }

int main(int argc, char** argv) {
  if (argc != 3) return fail("usage: c_abi_driver <input> <output>");
  FILE* in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open input");
  int32_t hdr[5];
  float tau;
  if (!read_all(in, hdr, sizeof hdr) || !read_all(in, &tau, sizeof tau)) return fail("short header");
  const int32_t n_rows = hdr[1], V = hdr[2], dtype = hdr[3], n_dec = hdr[4];
  if (hdr[0] != 0x45430001 || n_rows < 1 || n_rows > 4096 || V < 1 || V > (1 << 20) ||
      (dtype != EC_F32 && dtype != EC_BF16) || n_dec < 0 || n_dec > n_rows)
    return fail("bad header");
  const size_t esz = dtype == EC_BF16 ? 2 : 4;
  const size_t lbytes = size_t(n_rows) * V * esz;
  char* logits = (char*)malloc(lbytes);
  int32_t* dec = (int32_t*)malloc(sizeof(int32_t) * (n_dec > 0 ? n_dec : 1));
  int32_t sel[8];
  if (!logits || !dec) return fail("host allocation");
  if (!read_all(in, logits, lbytes) || !read_all(in, dec, sizeof(int32_t) * n_dec) ||
      !read_all(in, sel, sizeof sel))
    return fail("short input");
  const int32_t L = sel[0], bs = sel[1], bl = sel[2], bc = sel[3], cap = sel[4], hlen = sel[5],
                k = sel[6], flag_in = sel[7];
  if (L < 1 || L > (1 << 20) || cap < 1 || cap > (1 << 20)) return fail("bad selection sizes");
  uint8_t* masked = (uint8_t*)malloc(L);
  int32_t* hist = (int32_t*)malloc(sizeof(int32_t) * cap);
  if (!masked || !hist || !read_all(in, masked, L) || !read_all(in, hist, sizeof(int32_t) * cap))
    return fail("short selection input");
  fclose(in);

  // the row stride must be a multiple of 16 bytes: pad rows on the device
  const int64_t stride = int64_t((V * esz + 15) / 16 * 16 / esz);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  char* d_logits;
  int32_t *d_dec, *d_ndec, *d_argmax, *d_flag;
  float *d_H, *d_p1, *d_E;
  const size_t ws_bytes = ec_entropy_workspace_bytes(n_rows, V);
  void* d_ws;
  HIP_OK(hipMalloc((void**)&d_logits, size_t(n_rows) * stride * esz));
  HIP_OK(hipMalloc((void**)&d_dec, sizeof(int32_t) * (n_dec > 0 ? n_dec : 1)));
  HIP_OK(hipMalloc((void**)&d_ndec, sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_H, sizeof(float) * n_rows));
  HIP_OK(hipMalloc((void**)&d_argmax, sizeof(int32_t) * n_rows));
  HIP_OK(hipMalloc((void**)&d_p1, sizeof(float) * n_rows));
  HIP_OK(hipMalloc((void**)&d_E, sizeof(float)));
  HIP_OK(hipMalloc((void**)&d_flag, sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_ws, ws_bytes > 0 ? ws_bytes : 16));
  HIP_OK(hipMemcpy2D(d_logits, stride * esz, logits, V * esz, V * esz, n_rows, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_dec, dec, sizeof(int32_t) * n_dec, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_ndec, &n_dec, sizeof(int32_t), hipMemcpyHostToDevice));

  int32_t st[4];
  st[0] = ec_entropy_max(d_logits, dtype, n_rows, V, stride, d_dec, d_ndec, n_rows, tau, d_H, d_argmax,
                         d_p1, d_E, d_flag, d_ws, ws_bytes, s);
  // argument errors are reported on the host, before anything is enqueued
  st[2] = ec_entropy_max(NULL, dtype, n_rows, V, stride, d_dec, d_ndec, n_rows, tau, d_H, d_argmax,
                         d_p1, d_E, d_flag, d_ws, ws_bytes, s);
  st[3] = ws_bytes > 0 ? ec_entropy_max(d_logits, dtype, n_rows, V, stride, d_dec, d_ndec, n_rows, tau, d_H,
                                        d_argmax, d_p1, d_E, d_flag, d_ws, ws_bytes - 1, s)
                       : EC_E_WORKSPACE;

  int32_t *d_fflag, *d_hist, *d_hlen, *d_rows, *d_nrows;
  uint8_t* d_masked;
  HIP_OK(hipMalloc((void**)&d_fflag, sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_hist, sizeof(int32_t) * cap));
  HIP_OK(hipMalloc((void**)&d_hlen, sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_rows, sizeof(int32_t) * L));
  HIP_OK(hipMalloc((void**)&d_nrows, sizeof(int32_t)));
  HIP_OK(hipMalloc((void**)&d_masked, L));
  HIP_OK(hipMemcpy(d_fflag, &flag_in, sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_hist, hist, sizeof(int32_t) * cap, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_hlen, &hlen, sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_masked, masked, L, hipMemcpyHostToDevice));
  st[1] = ec_select_rows(d_fflag, d_masked, L, bs, bl, bc, d_hist, d_hlen, cap, k, d_rows, d_nrows, s);
  HIP_OK(hipStreamSynchronize(s));

  float* H = (float*)malloc(sizeof(float) * n_rows);
  float* p1 = (float*)malloc(sizeof(float) * n_rows);
  int32_t* am = (int32_t*)malloc(sizeof(int32_t) * n_rows);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * L);
  float E = 0.f;
  int32_t flag = -1, n_sel = 0;
  if (!H || !p1 || !am || !rows) return fail("host allocation");
  HIP_OK(hipMemcpy(H, d_H, sizeof(float) * n_rows, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(am, d_argmax, sizeof(int32_t) * n_rows, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(p1, d_p1, sizeof(float) * n_rows, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&E, d_E, sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&flag, d_flag, sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&n_sel, d_nrows, sizeof(int32_t), hipMemcpyDeviceToHost));
  if (n_sel < 0 || n_sel > L) return fail("row count out of range");
  HIP_OK(hipMemcpy(rows, d_rows, sizeof(int32_t) * n_sel, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out) return fail("cannot open output");
  const bool wrote = fwrite(st, sizeof st, 1, out) == 1 &&
                     fwrite(H, sizeof(float), n_rows, out) == size_t(n_rows) &&
                     fwrite(am, sizeof(int32_t), n_rows, out) == size_t(n_rows) &&
                     fwrite(p1, sizeof(float), n_rows, out) == size_t(n_rows) &&
                     fwrite(&E, sizeof E, 1, out) == 1 && fwrite(&flag, sizeof flag, 1, out) == 1 &&
                     fwrite(&n_sel, sizeof n_sel, 1, out) == 1 &&
                     fwrite(rows, sizeof(int32_t), n_sel, out) == size_t(n_sel);
  if (fclose(out) != 0 || !wrote) return fail("cannot write output");

  void* bufs[] = {d_logits, d_dec, d_ndec, d_H, d_argmax, d_p1, d_E, d_flag, d_ws, d_fflag, d_hist,
                  d_hlen, d_rows, d_nrows, d_masked};
  for (void* b : bufs) HIP_OK(hipFree(b));
  HIP_OK(hipStreamDestroy(s));
  free(logits); free(dec); free(masked); free(hist); free(H); free(p1); free(am); free(rows);
  printf("c_abi_driver: ok (%d rows, V = %d, %d selected)\n", n_rows, V, n_sel);
  return 0;
}

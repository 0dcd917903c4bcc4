/*
 * A plain C consumer of the library's C ABI: no PyTorch, no Python, only the HIP runtime for
 * device memory and a stream.  It runs the m=1 decode path on small seeded inputs and checks
 * the results against the CPU oracle (test infrastructure; this program is a test):
 *
 *   1. producer (q8_fuse_gate.rs, module doc and `run_shape`): the fused rmsnorm_q8_1 and the
 *      two-launch chain rms_norm_f32 -> quantize_q8_1 give the same z, qs and d bytes, and
 *      the oracle's quantiser applied to the GPU's z gives the GPU's qs and d bit for bit;
 *   2. the three GEMVs (gemv_e4m3_bench.rs, THE COMPARISON and THE BLOCK-128 ARM), plain and
 *      on the matrix cores, on that q8_1 row: every output within 1e-5 of the sum of the
 *      absolute terms of the oracle;
 *   3. argument errors come back as negative codes with a message, and launch nothing.
 *
 * Inputs come from the shared seeded generators (synth), with the seeds the Python tests use.
 * Prints one line per case and "c_abi_check PASS" at the end; exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp8_gemv.h"

/* shared generators (synth/synth.c) */
void synth_f32(uint64_t seed, float *out, int64_t n);
void synth_e4m3(uint64_t seed, uint8_t *out, int64_t n);
void synth_q8_0(uint64_t seed, uint8_t *out, int64_t out_f, int64_t in_f);
void synth_grid(uint64_t seed, float *out, int64_t n);

/* oracle (oracle/oracle.c) */
int oracle_quantize_q8_1(const float *z, int nrows, int ncols, int8_t *qs, float *d);
int oracle_gemv_q8_0(const uint8_t *W, int64_t row_bytes, const int8_t *qs, const float *d,
                     int m, int in_f, int out_f, int r0, int r1, double *y, double *A);
int oracle_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                     const float *d, int m, int in_f, int out_f, int r0, int r1, double *y,
                     double *A);
int oracle_gemv_e4m3_blk128(const uint8_t *W, int64_t row_bytes, const float *grid,
                            int grid_cols, const int8_t *qs, const float *d, int m, int in_f,
                            int out_f, int r0, int r1, double *y, double *A);

#define SEED_X 0x9E3779B97F4A7C15ull
#define SEED_W 0xD1B54A32D192ED03ull
#define SEED_E4M3 0x12345678ull
#define SEED_Q8_0 0x9E3779B9ull
#define SEED_GRID 0x5BF03635ull

static int failures = 0;

#define HIP_OK(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) {                                                           \
      printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__);   \
      exit(2);                                                                        \
    }                                                                                 \
  } while (0)

static void check(int ok, const char *what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  fflush(stdout);
  if (!ok) ++failures;
}

static void *dev_alloc(size_t bytes) {
  void *p = NULL;
  HIP_OK(hipMalloc(&p, bytes));
  return p;
}

static void *host_alloc(size_t bytes) {
  void *p = malloc(bytes);
  if (!p) {
    printf("out of host memory\n");
    exit(2);
  }
  return p;
}

static uint64_t shape_seed(uint64_t base, int out_f, int in_f) {
  return base ^ (((uint64_t)out_f << 32) | (uint64_t)in_f);
}

/* |y_gpu - y| <= 1e-5 * A for every output */
static int within(const float *y, const double *y64, const double *A, int n) {
  for (int i = 0; i < n; ++i)
    if (!(fabs((double)y[i] - y64[i]) <= 1e-5 * A[i])) {
      printf("  row %d: gpu %.9g oracle %.17g bound %.3g\n", i, (double)y[i], y64[i],
             1e-5 * A[i]);
      return 0;
    }
  return 1;
}

static void run_case(int out_f, int in_f, hipStream_t s) {
  char what[160];
  const int nb = in_f / 32;
  const size_t qrow = (size_t)nb * 34;

  /* ---- producer ---- */
  float *x = host_alloc(sizeof(float) * in_f), *w = host_alloc(sizeof(float) * in_f);
  synth_f32(SEED_X ^ (uint64_t)in_f, x, in_f);
  synth_f32(SEED_W ^ (uint64_t)in_f, w, in_f);
  float *dx = dev_alloc(sizeof(float) * in_f), *dw = dev_alloc(sizeof(float) * in_f);
  float *dz1 = dev_alloc(sizeof(float) * in_f), *dz2 = dev_alloc(sizeof(float) * in_f);
  int8_t *dq1 = dev_alloc(in_f), *dq2 = dev_alloc(in_f);
  float *dd1 = dev_alloc(sizeof(float) * nb), *dd2 = dev_alloc(sizeof(float) * nb);
  HIP_OK(hipMemcpy(dx, x, sizeof(float) * in_f, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, w, sizeof(float) * in_f, hipMemcpyHostToDevice));
  int rc = rmsnorm_q8_1(dx, dw, dz1, dq1, dd1, in_f, 1, 1e-6f, s);
  if (rc == 0) rc = rms_norm_f32(dx, dw, dz2, in_f, 1, 1e-6f, s);
  if (rc == 0) rc = quantize_q8_1(dz2, dq2, dd2, 1, in_f, s);
  snprintf(what, sizeof what, "producer launches at ncols %d (rc %d: %s)", in_f, rc,
           fp8gemv_strerror(rc));
  check(rc == 0, what);
  HIP_OK(hipStreamSynchronize(s));

  float *z1 = host_alloc(sizeof(float) * in_f), *z2 = host_alloc(sizeof(float) * in_f);
  int8_t *q1 = host_alloc(in_f), *q2 = host_alloc(in_f), *qo = host_alloc(in_f);
  float *d1 = host_alloc(sizeof(float) * nb), *d2 = host_alloc(sizeof(float) * nb);
  float *dor = host_alloc(sizeof(float) * nb);
  HIP_OK(hipMemcpy(z1, dz1, sizeof(float) * in_f, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(z2, dz2, sizeof(float) * in_f, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(q1, dq1, in_f, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(q2, dq2, in_f, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(d1, dd1, sizeof(float) * nb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(d2, dd2, sizeof(float) * nb, hipMemcpyDeviceToHost));
  snprintf(what, sizeof what, "fused == chain bytes (z, qs, d) at ncols %d", in_f);
  check(!memcmp(z1, z2, sizeof(float) * in_f) && !memcmp(q1, q2, in_f) &&
            !memcmp(d1, d2, sizeof(float) * nb),
        what);
  rc = oracle_quantize_q8_1(z1, 1, in_f, qo, dor);
  snprintf(what, sizeof what, "oracle q8_1 of the GPU z == GPU qs, d at ncols %d", in_f);
  check(rc == 0 && !memcmp(qo, q1, in_f) && !memcmp(dor, d1, sizeof(float) * nb), what);

  /* ---- GEMVs on the GPU's q8_1 row ---- */
  const size_t e_bytes = (size_t)out_f * in_f, q_bytes = (size_t)out_f * qrow;
  const int gr = (out_f + 127) / 128, gc = (in_f + 127) / 128;
  uint8_t *We = host_alloc(e_bytes), *Wq = host_alloc(q_bytes);
  float *G = host_alloc(sizeof(float) * gr * gc);
  synth_e4m3(shape_seed(SEED_E4M3, out_f, in_f), We, (int64_t)e_bytes);
  synth_q8_0(shape_seed(SEED_Q8_0, out_f, in_f), Wq, out_f, in_f);
  synth_grid(shape_seed(SEED_GRID, out_f, in_f), G, (int64_t)gr * gc);
  uint8_t *dWe = dev_alloc(e_bytes), *dWq = dev_alloc(q_bytes);
  float *dG = dev_alloc(sizeof(float) * gr * gc), *dy = dev_alloc(sizeof(float) * out_f);
  HIP_OK(hipMemcpy(dWe, We, e_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dWq, Wq, q_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dG, G, sizeof(float) * gr * gc, hipMemcpyHostToDevice));
  float *y = host_alloc(sizeof(float) * out_f);
  double *y64 = host_alloc(sizeof(double) * out_f), *A = host_alloc(sizeof(double) * out_f);
  const float scale = 0.0625f;

  /* arms 0..2: the plain entry points; 3..5: the same containers on the matrix cores (*_mc) */
  for (int k = 0; k < 6; ++k) {
    const int arm = k % 3, mc = k >= 3;
    const char *name = k == 0 ? "e4m3" : k == 1 ? "blk128" : k == 2 ? "q8_0"
                     : k == 3 ? "e4m3_mc" : k == 4 ? "blk128_mc" : "q8_0_mc";
    if (arm == 0) {
      rc = (mc ? gemv_e4m3_q81_mc : gemv_e4m3_q81)(dWe, in_f, scale, dq1, dd1, dy, 1, in_f,
                                                   out_f, s);
    } else if (arm == 1) {
      rc = (mc ? gemv_e4m3_blk128_q81_mc : gemv_e4m3_blk128_q81)(dWe, in_f, dG, gc, dq1, dd1,
                                                                 dy, 1, in_f, out_f, s);
    } else {
      rc = (mc ? gemv_q8_0_q81_mc : gemv_q8_0_q81)(dWq, (int64_t)qrow, dq1, dd1, dy, 1, in_f,
                                                   out_f, s);
    }
    snprintf(what, sizeof what, "%s %dx%d launches (rc %d: %s)", name, out_f, in_f, rc,
             fp8gemv_strerror(rc));
    check(rc == 0, what);
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(y, dy, sizeof(float) * out_f, hipMemcpyDeviceToHost));
    if (arm == 0) {
      rc = oracle_gemv_e4m3(We, in_f, scale, q1, d1, 1, in_f, out_f, 0, out_f, y64, A);
    } else if (arm == 1) {
      rc = oracle_gemv_e4m3_blk128(We, in_f, G, gc, q1, d1, 1, in_f, out_f, 0, out_f, y64, A);
    } else {
      rc = oracle_gemv_q8_0(Wq, (int64_t)qrow, q1, d1, 1, in_f, out_f, 0, out_f, y64, A);
    }
    snprintf(what, sizeof what, "%s %dx%d: every output within 1e-5 of sum |terms|", name,
             out_f, in_f);
    check(rc == 0 && within(y, y64, A, out_f), what);
  }

  HIP_OK(hipFree(dx)); HIP_OK(hipFree(dw)); HIP_OK(hipFree(dz1)); HIP_OK(hipFree(dz2));
  HIP_OK(hipFree(dq1)); HIP_OK(hipFree(dq2)); HIP_OK(hipFree(dd1)); HIP_OK(hipFree(dd2));
  HIP_OK(hipFree(dWe)); HIP_OK(hipFree(dWq)); HIP_OK(hipFree(dG)); HIP_OK(hipFree(dy));
  free(x); free(w); free(z1); free(z2); free(q1); free(q2); free(qo); free(d1); free(d2);
  free(dor); free(We); free(Wq); free(G); free(y); free(y64); free(A);
}

int main(void) {
  int ndev = 0;
  HIP_OK(hipGetDeviceCount(&ndev));
  if (ndev < 1) {
    printf("no HIP device\n");
    return 2;
  }
  HIP_OK(hipSetDevice(0));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  /* argument errors: negative codes, nothing launched (no pointer is dereferenced) */
  check(gemv_e4m3_q81(NULL, 64, 1.0f, NULL, NULL, NULL, 1, 64, 8, s) == FP8GEMV_ERR_NULL,
        "NULL weights -> FP8GEMV_ERR_NULL");
  check(strlen(fp8gemv_strerror(FP8GEMV_ERR_SHAPE)) > 0, "fp8gemv_strerror has text");

  run_case(2048, 2048, s);  /* the small end-to-end configuration */
  run_case(131, 8224, s);   /* ragged rows, in_f past the first range, generic Q8_0 path */
  run_case(130, 96, s);     /* one window, partial block-128 tiles */

  HIP_OK(hipStreamDestroy(s));
  if (failures) {
    printf("c_abi_check FAIL (%d)\n", failures);
    return 1;
  }
  printf("c_abi_check PASS\n");
  return 0;
}

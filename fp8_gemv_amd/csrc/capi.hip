// C ABI of the gfx950 matvec library: argument checks on the host, then one launch on the
// caller's stream.  Nothing here allocates, synchronises or touches device memory.
#include "../../include/fp8_gemv.h"
#include "common.hpp"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int launch_rc(hipError_t e) { return e == hipSuccess ? FP8GEMV_OK : (int)e; }

inline bool bad_cols(int ncols) { return ncols < 32 || ncols % 32 != 0; }

int check_gemv_common(const void *W, const int8_t *qs, const float *d, float *y, int m,
                      int in_f, int out_f) {
  if (!W || !qs || !d || !y) return FP8GEMV_ERR_NULL;
  if (m < 1 || out_f < 1 || bad_cols(in_f)) return FP8GEMV_ERR_SHAPE;
  if (in_f > FP8GEMV_MAX_IN_F || m > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(qs, 16) || !aligned(d, 4) || !aligned(y, 4)) return FP8GEMV_ERR_ALIGN;
  return FP8GEMV_OK;
}

}  // namespace

extern "C" {

int rms_norm_f32(const float *x, const float *w, float *z, int ncols, int nrows, float eps,
                 void *stream) {
  if (!x || !w || !z) return FP8GEMV_ERR_NULL;
  if (nrows < 1 || bad_cols(ncols)) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(z, 16)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_rms_norm(x, w, z, ncols, nrows, eps, (hipStream_t)stream));
}

int quantize_q8_1(const float *z, int8_t *qs, float *d, int nrows, int ncols, void *stream) {
  if (!z || !qs || !d) return FP8GEMV_ERR_NULL;
  if (nrows < 1 || bad_cols(ncols)) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(z, 16) || !aligned(qs, 16) || !aligned(d, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_quantize_q8_1(z, qs, d, nrows, ncols, (hipStream_t)stream));
}

int rmsnorm_q8_1(const float *x, const float *w, float *z, int8_t *qs, float *d, int ncols,
                 int nrows, float eps, void *stream) {
  if (!x || !w || !qs || !d) return FP8GEMV_ERR_NULL;
  if (nrows < 1 || bad_cols(ncols)) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(x, 16) || !aligned(w, 16) || (z && !aligned(z, 16)) || !aligned(qs, 16) ||
      !aligned(d, 4))
    return FP8GEMV_ERR_ALIGN;
  return launch_rc(
      fp8gemv::launch_rmsnorm_q8_1(x, w, z, qs, d, ncols, nrows, eps, (hipStream_t)stream));
}

int silu_mul_f32(const float *gate, const float *up, float *h, int ncols, int nrows,
                 void *stream) {
  if (!gate || !up || !h) return FP8GEMV_ERR_NULL;
  if (nrows < 1 || bad_cols(ncols)) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(h, 16)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_silu_mul(gate, up, h, ncols, nrows, (hipStream_t)stream));
}

int silu_mul_q8_1(const float *gate, const float *up, float *h, int8_t *qs, float *d, int ncols,
                  int nrows, void *stream) {
  if (!gate || !up || !qs || !d) return FP8GEMV_ERR_NULL;
  if (nrows < 1 || bad_cols(ncols)) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(gate, 16) || !aligned(up, 16) || (h && !aligned(h, 16)) || !aligned(qs, 16) ||
      !aligned(d, 4))
    return FP8GEMV_ERR_ALIGN;
  return launch_rc(
      fp8gemv::launch_silu_mul_q8_1(gate, up, h, qs, d, ncols, nrows, (hipStream_t)stream));
}

namespace {
int check_gated(const float *o, const float *g, const float *w, int ncols, int head_dim,
                int nrows) {
  if (!o || !g || !w) return FP8GEMV_ERR_NULL;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256)
    return FP8GEMV_ERR_SHAPE;
  if (nrows < 1 || bad_cols(ncols) || ncols % head_dim != 0) return FP8GEMV_ERR_SHAPE;
  if (ncols > FP8GEMV_MAX_IN_F || nrows > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(o, 16) || !aligned(g, 16) || !aligned(w, 16)) return FP8GEMV_ERR_ALIGN;
  return FP8GEMV_OK;
}
}  // namespace

int gated_rms_norm_f32(const float *o, const float *g, const float *w, float *z, int ncols,
                       int head_dim, int nrows, float eps, void *stream) {
  if (!z) return FP8GEMV_ERR_NULL;
  const int rc = check_gated(o, g, w, ncols, head_dim, nrows);
  if (rc) return rc;
  if (!aligned(z, 16)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_gated_rms_norm(o, g, w, z, ncols, head_dim, nrows, eps,
                                                  (hipStream_t)stream));
}

int gated_rmsnorm_q8_1(const float *o, const float *g, const float *w, float *z, int8_t *qs,
                       float *d, int ncols, int head_dim, int nrows, float eps, void *stream) {
  if (!qs || !d) return FP8GEMV_ERR_NULL;
  const int rc = check_gated(o, g, w, ncols, head_dim, nrows);
  if (rc) return rc;
  if ((z && !aligned(z, 16)) || !aligned(qs, 16) || !aligned(d, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_gated_rmsnorm_q8_1(o, g, w, z, qs, d, ncols, head_dim, nrows,
                                                      eps, (hipStream_t)stream));
}

namespace {
int gemv_q8_0_call(const void *W, int64_t row_bytes, const int8_t *qs, const float *d, float *y,
                   int m, int in_f, int out_f, bool matrix_cores, void *stream) {
  const int rc = check_gemv_common(W, qs, d, y, m, in_f, out_f);
  if (rc) return rc;
  if (row_bytes < (int64_t)(in_f / 32) * 34) return FP8GEMV_ERR_ROW_BYTES;
  if (!aligned(W, 2) || row_bytes % 2 != 0) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_gemv_q8_0(static_cast<const uint8_t *>(W), row_bytes, qs, d,
                                             y, m, in_f, out_f, matrix_cores,
                                             (hipStream_t)stream));
}

int gemv_e4m3_call(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                   const float *d, float *y, int m, int in_f, int out_f, bool matrix_cores,
                   void *stream) {
  const int rc = check_gemv_common(W, qs, d, y, m, in_f, out_f);
  if (rc) return rc;
  if (row_bytes < in_f) return FP8GEMV_ERR_ROW_BYTES;
  if (!aligned(W, 16) || row_bytes % 16 != 0) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_gemv_e4m3(W, row_bytes, scale, nullptr, 0, false, qs, d, y, m,
                                             in_f, out_f, matrix_cores, (hipStream_t)stream));
}

int gemv_e4m3_blk128_call(const uint8_t *W, int64_t row_bytes, const float *grid, int grid_cols,
                          const int8_t *qs, const float *d, float *y, int m, int in_f,
                          int out_f, bool matrix_cores, void *stream) {
  const int rc = check_gemv_common(W, qs, d, y, m, in_f, out_f);
  if (rc) return rc;
  if (!grid) return FP8GEMV_ERR_NULL;
  if (grid_cols != (in_f + 127) / 128) return FP8GEMV_ERR_GRID;
  if (row_bytes < in_f) return FP8GEMV_ERR_ROW_BYTES;
  if (!aligned(W, 16) || row_bytes % 16 != 0 || !aligned(grid, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_gemv_e4m3(W, row_bytes, 1.0f, grid, grid_cols, true, qs, d, y,
                                             m, in_f, out_f, matrix_cores, (hipStream_t)stream));
}
}  // namespace

int gemv_q8_0_q81(const void *W, int64_t row_bytes, const int8_t *qs, const float *d, float *y,
                  int m, int in_f, int out_f, void *stream) {
  return gemv_q8_0_call(W, row_bytes, qs, d, y, m, in_f, out_f, false, stream);
}

int gemv_e4m3_q81(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                  const float *d, float *y, int m, int in_f, int out_f, void *stream) {
  return gemv_e4m3_call(W, row_bytes, scale, qs, d, y, m, in_f, out_f, false, stream);
}

int gemv_e4m3_blk128_q81(const uint8_t *W, int64_t row_bytes, const float *grid, int grid_cols,
                         const int8_t *qs, const float *d, float *y, int m, int in_f, int out_f,
                         void *stream) {
  return gemv_e4m3_blk128_call(W, row_bytes, grid, grid_cols, qs, d, y, m, in_f, out_f, false,
                               stream);
}

int gemv_q8_0_q81_mc(const void *W, int64_t row_bytes, const int8_t *qs, const float *d,
                     float *y, int m, int in_f, int out_f, void *stream) {
  return gemv_q8_0_call(W, row_bytes, qs, d, y, m, in_f, out_f, true, stream);
}

int gemv_e4m3_q81_mc(const uint8_t *W, int64_t row_bytes, float scale, const int8_t *qs,
                     const float *d, float *y, int m, int in_f, int out_f, void *stream) {
  return gemv_e4m3_call(W, row_bytes, scale, qs, d, y, m, in_f, out_f, true, stream);
}

int gemv_e4m3_blk128_q81_mc(const uint8_t *W, int64_t row_bytes, const float *grid,
                            int grid_cols, const int8_t *qs, const float *d, float *y, int m,
                            int in_f, int out_f, void *stream) {
  return gemv_e4m3_blk128_call(W, row_bytes, grid, grid_cols, qs, d, y, m, in_f, out_f, true,
                               stream);
}

namespace {
int check_requant(const uint8_t *W, int64_t row_bytes, void *Wq, int64_t q_row_bytes, int in_f,
                  int out_f) {
  if (!W || !Wq) return FP8GEMV_ERR_NULL;
  if (out_f < 1 || bad_cols(in_f)) return FP8GEMV_ERR_SHAPE;
  if (in_f > FP8GEMV_MAX_IN_F) return FP8GEMV_ERR_TOO_LARGE;
  if (row_bytes < in_f || q_row_bytes < (int64_t)(in_f / 32) * 34) return FP8GEMV_ERR_ROW_BYTES;
  if (!aligned(W, 16) || row_bytes % 16 != 0 || !aligned(Wq, 2) || q_row_bytes % 2 != 0)
    return FP8GEMV_ERR_ALIGN;
  return FP8GEMV_OK;
}
}  // namespace

int requant_e4m3_q8_0(const uint8_t *W, int64_t row_bytes, float scale, void *Wq,
                      int64_t q_row_bytes, int in_f, int out_f, void *stream) {
  const int rc = check_requant(W, row_bytes, Wq, q_row_bytes, in_f, out_f);
  if (rc) return rc;
  return launch_rc(fp8gemv::launch_requant_q8_0(W, row_bytes, scale, nullptr, 0, false, Wq,
                                                q_row_bytes, in_f, out_f, (hipStream_t)stream));
}

int requant_e4m3_blk128_q8_0(const uint8_t *W, int64_t row_bytes, const float *grid,
                             int grid_cols, void *Wq, int64_t q_row_bytes, int in_f, int out_f,
                             void *stream) {
  const int rc = check_requant(W, row_bytes, Wq, q_row_bytes, in_f, out_f);
  if (rc) return rc;
  if (!grid) return FP8GEMV_ERR_NULL;
  if (grid_cols != (in_f + 127) / 128) return FP8GEMV_ERR_GRID;
  if (!aligned(grid, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_requant_q8_0(W, row_bytes, 1.0f, grid, grid_cols, true, Wq,
                                                q_row_bytes, in_f, out_f, (hipStream_t)stream));
}

int fp8gemv_read_bytes(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
  if (!p || !sink) return FP8GEMV_ERR_NULL;
  if (bytes < 1) return FP8GEMV_ERR_SHAPE;
  if (bytes > FP8GEMV_MAX_READ_BYTES) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(p, 16) || !aligned(sink, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(fp8gemv::launch_read_bytes(p, bytes, sink, (hipStream_t)stream));
}

int fp8gemv_read_pattern(const void *p, int64_t bytes, int pattern, int64_t row_bytes,
                         uint32_t *sink, void *stream) {
  if (!p || !sink) return FP8GEMV_ERR_NULL;
  if (bytes < 1 || pattern < 0 || pattern >= FP8GEMV_READ_NUM_PATTERNS) return FP8GEMV_ERR_SHAPE;
  if (pattern == FP8GEMV_READ_ROWS_1K || pattern == FP8GEMV_READ_ROWS_816 ||
      pattern == FP8GEMV_READ_ROWS_ALIGNED || pattern == FP8GEMV_READ_LINE_WINDOWS) {
    if (row_bytes < 1024 || row_bytes > (1 << 20) || row_bytes % 16 != 0 || bytes % row_bytes != 0)
      return FP8GEMV_ERR_SHAPE;
  }
  if (bytes > FP8GEMV_MAX_READ_BYTES) return FP8GEMV_ERR_TOO_LARGE;
  if (!aligned(p, 16) || !aligned(sink, 4)) return FP8GEMV_ERR_ALIGN;
  return launch_rc(
      fp8gemv::launch_read_pattern(p, bytes, pattern, row_bytes, sink, (hipStream_t)stream));
}

int fp8gemv_gemv_launch_info(int container, const void *W, int64_t row_bytes, int m, int in_f,
                             int out_f, fp8gemv_launch_info *info) {
  if (!W || !info) return FP8GEMV_ERR_NULL;
  if (m < 1 || out_f < 1 || bad_cols(in_f)) return FP8GEMV_ERR_SHAPE;
  if (in_f > FP8GEMV_MAX_IN_F || m > FP8GEMV_MAX_M) return FP8GEMV_ERR_TOO_LARGE;
  fp8gemv::LaunchDesc r;
  const bool mc = container == FP8GEMV_Q8_0_MC || container == FP8GEMV_E4M3_MC ||
                  container == FP8GEMV_E4M3_BLK128_MC;
  if (container == FP8GEMV_Q8_0 || container == FP8GEMV_Q8_0_MC) {
    if (row_bytes < (int64_t)(in_f / 32) * 34) return FP8GEMV_ERR_ROW_BYTES;
    if (!aligned(W, 2) || row_bytes % 2 != 0) return FP8GEMV_ERR_ALIGN;
    r = fp8gemv::describe_gemv_q8_0(static_cast<const uint8_t *>(W), row_bytes, m, in_f, out_f,
                                    mc);
  } else if (container == FP8GEMV_E4M3 || container == FP8GEMV_E4M3_BLK128 ||
             container == FP8GEMV_E4M3_MC || container == FP8GEMV_E4M3_BLK128_MC) {
    if (row_bytes < in_f) return FP8GEMV_ERR_ROW_BYTES;
    if (!aligned(W, 16) || row_bytes % 16 != 0) return FP8GEMV_ERR_ALIGN;
    r = fp8gemv::describe_gemv_e4m3(
        container == FP8GEMV_E4M3_BLK128 || container == FP8GEMV_E4M3_BLK128_MC, row_bytes, m,
        in_f, out_f, mc);
  } else {
    return FP8GEMV_ERR_SHAPE;
  }
  info->grid_x = r.grid_x;
  info->grid_y = r.grid_y;
  info->workgroup_size = r.threads;
  info->lds_bytes = r.lds;
  info->kernel = r.kernel;
  info->config = r.config;
  return FP8GEMV_OK;
}

const char *fp8gemv_strerror(int rc) {
  switch (rc) {
    case FP8GEMV_OK: return "ok";
    case FP8GEMV_ERR_NULL: return "a required pointer is NULL";
    case FP8GEMV_ERR_SHAPE: return "bad shape: columns must be a positive multiple of 32, rows >= 1";
    case FP8GEMV_ERR_ROW_BYTES: return "row_bytes is below the container minimum";
    case FP8GEMV_ERR_GRID: return "grid_cols must equal ceil(in_f / 128)";
    case FP8GEMV_ERR_ALIGN: return "a pointer or row stride breaks the required alignment";
    case FP8GEMV_ERR_TOO_LARGE: return "a size exceeds the library limit";
    default: break;
  }
  if (rc > 0) return hipGetErrorString((hipError_t)rc);
  return "unknown error";
}

}  // extern "C"

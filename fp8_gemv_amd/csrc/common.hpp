// Shared device helpers and the internal launcher interface of the gfx950 matvec library.
// Everything here is written for CDNA4 wave64; there is no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemv {

constexpr int kWave = 64;
constexpr int kMaxInF = 65536;  // FP8GEMV_MAX_IN_F of the public header

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef int int4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ cross-lane sums ----
// DPP controls (GFX9 encoding).
constexpr int kQuadPerm1032 = 0xB1;  // lanes {1,0,3,2} within each quad
constexpr int kQuadPerm2301 = 0x4E;  // lanes {2,3,0,1} within each quad
constexpr int kRowRor4 = 0x124;      // rotate right by 4 within each row of 16
constexpr int kRowRor8 = 0x128;      // rotate right by 8 within each row of 16
constexpr int kWaveShr1 = 0x138;     // shift right by one lane across the whole wave
constexpr int kRowHalfMirror = 0x141;  // reverse lanes within each group of 8

// Full row and bank masks.  Every lane has a valid source for these patterns, so bound_ctrl
// changes nothing here; it is set because it lets the compiler fold the move into the
// instruction that consumes it (v_add_f32_dpp instead of v_mov_b32_dpp + v_add_f32).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over all 64 lanes.  Within each row of 16 lanes a DPP butterfly (xor 1, xor 2, then
// rotations by 4 and 8) leaves the row sum r_k in the row's first lane (16k); the four row
// sums are then added in the fixed order (r0 + r1) + (r2 + r3): v_permlane16_swap brings lane
// 16 to lane 0 and lane 48 to lane 32, v_permlane32_swap then lane 32 to lane 0.  The result
// is read from lane 0, so it is wave-uniform, and it depends only on the lane values.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kQuadPerm1032>(v);
  v += dpp_f32<kQuadPerm2301>(v);
  v += dpp_f32<kRowRor4>(v);
  v += dpp_f32<kRowRor8>(v);
  // Swapping a value with itself: element 0 keeps the even rows (lanes 0-15, 32-47) and
  // element 1 holds the odd rows moved down (lane 0 <- 16, lane 32 <- 48).
  const int iv = __builtin_bit_cast(int, v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
  // lane 0: r0 + r1; lane 32: r2 + r3
  const float t = __builtin_bit_cast(float, (int)p16[0]) + __builtin_bit_cast(float, (int)p16[1]);
  // element 0 keeps lanes 0-31, element 1 holds lanes 32-63 moved down (lane 0 <- 32)
  const int it = __builtin_bit_cast(int, t);
  const auto p32 = __builtin_amdgcn_permlane32_swap(it, it, false, false);
  // lane 0: (r0 + r1) + (r2 + r3)
  const float u = __builtin_bit_cast(float, (int)p32[0]) + __builtin_bit_cast(float, (int)p32[1]);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, u), 0));
}

// ----------------------------------------------------------------------- loads ----
// Raw buffer resource over [base, base + bytes).  Loads through it at offsets past `bytes`
// return zeros and touch no memory, so every load can be issued unconditionally: no
// branches around loads means the compiler can count outstanding loads exactly and wait
// only for the one it needs.  `base` must be wave-uniform.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, no swizzle
constexpr int kAuxNonTemporal = 2;      // "nt": streamed once, do not keep

__device__ __forceinline__ rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
// 16-byte streaming load of weight bytes: read once, never reused, so marked non-temporal.
__device__ __forceinline__ int4_t buf_load16_stream(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0,
                                                                          kAuxNonTemporal));
}
__device__ __forceinline__ int4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// The wave index as a value the compiler knows to be uniform.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

}  // namespace fp8gemv

// ------------------------------------------------------------- launch-time helpers ----
// Raise a kernel's dynamic LDS limit to `bytes` once per device (the attribute is per device).
// Thread-safe: concurrent first calls may both set it, which is harmless; the result is
// remembered only when it succeeded.
#include <atomic>
namespace fp8gemv {
constexpr int kMaxDevices = 64;
inline hipError_t set_lds_limit_once(const void *kernel, size_t bytes,
                                     std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire))
    return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices)
    done[dev].store(true, std::memory_order_release);
  return e;
}
// CUs of the current device, cached per device (256 if it cannot be read: it only sizes the
// grids of the persistent launches, and every grid size computes the same result).
inline int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
    c = 256;
  cache[dev].store(c, std::memory_order_relaxed);
  return c;
}
}  // namespace fp8gemv

// -------------------------------------------------------------- launch descriptions ----
// What a GEMV call launches, for profilers and benches: the same selection code that launches
// fills it in, so it can never disagree with the launch.
#include <cstdio>
#include <string>
namespace fp8gemv {
struct LaunchDesc {
  unsigned grid_x = 0, grid_y = 0, threads = 0, lds = 0;
  const char *kernel = "";
  const char *config = "";
};
template <class C> struct Tag { using type = C; };
// The launch configuration type's text as it appears in the demangled kernel symbol, every
// template argument written out, e.g. "Cfg<4, 1, 2, 2, 1, true, 8, 1, 1>" (static storage).
// C provides NAME and the nine parameters P0..P8 in template-argument order (P5 a bool).
template <class C> const char *config_text() {
  static const std::string text = [] {
    char b[128];
    snprintf(b, sizeof b, "%s<%d, %d, %d, %d, %d, %s, %d, %d, %d>", C::NAME, C::P0, C::P1, C::P2,
             C::P3, C::P4, C::P5 ? "true" : "false", C::P6, C::P7, C::P8);
    return std::string(b);
  }();
  return text.c_str();
}
}  // namespace fp8gemv

// --------------------------------------------------------------- internal launchers ----
// Host-side launchers, one per kernel family; arguments are validated by the C ABI layer
// before these run.  Each returns the hipError_t of the launch.
namespace fp8gemv {

hipError_t launch_rms_norm(const float *x, const float *w, float *z, int ncols, int nrows,
                           float eps, hipStream_t s);
hipError_t launch_quantize_q8_1(const float *z, int8_t *qs, float *d, int nrows, int ncols,
                                hipStream_t s);
hipError_t launch_rmsnorm_q8_1(const float *x, const float *w, float *z, int8_t *qs, float *d,
                               int ncols, int nrows, float eps, hipStream_t s);
hipError_t launch_silu_mul(const float *g, const float *u, float *h, int ncols, int nrows,
                           hipStream_t s);
hipError_t launch_gated_rms_norm(const float *o, const float *g, const float *w, float *z,
                                 int ncols, int head_dim, int nrows, float eps, hipStream_t s);
hipError_t launch_gated_rmsnorm_q8_1(const float *o, const float *g, const float *w, float *z,
                                     int8_t *qs, float *d, int ncols, int head_dim, int nrows,
                                     float eps, hipStream_t s);
hipError_t launch_silu_mul_q8_1(const float *g, const float *u, float *h, int8_t *qs, float *d,
                                int ncols, int nrows, hipStream_t s);
// matrix_cores: run the matrix-core kernel where the row layout allows it (the *_mc entry
// points); otherwise, and always for the plain entry points, the vector kernels, whose rows are
// bit-identical to m = 1 for any m.
hipError_t launch_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                            int grid_cols, bool blk128, const int8_t *qs, const float *d,
                            float *y, int m, int in_f, int out_f, bool matrix_cores,
                            hipStream_t s);
hipError_t launch_gemv_q8_0(const uint8_t *W, int64_t row_bytes, const int8_t *qs,
                            const float *d, float *y, int m, int in_f, int out_f,
                            bool matrix_cores, hipStream_t s);
LaunchDesc describe_gemv_e4m3(bool blk128, int64_t row_bytes, int m, int in_f, int out_f,
                              bool matrix_cores);
// The matrix-core kernel for several activation rows (gemv_e4m3_mfma.hip): the row layouts it
// takes.
bool gemv_e4m3_mfma_applies(int64_t row_bytes, int in_f);
hipError_t launch_gemv_e4m3_mfma(const uint8_t *W, int64_t row_bytes, float scale,
                                 const float *grid, int grid_cols, bool blk128, const int8_t *qs,
                                 const float *d, float *y, int m, int in_f, int out_f,
                                 hipStream_t s);
LaunchDesc describe_gemv_e4m3_mfma(bool blk128, int m, int in_f, int out_f);
// The matrix-core kernel for several activation rows over Q8_0 (gemv_q8_0_mfma.hip): the row
// layouts it takes.
bool gemv_q8_0_mfma_applies(const uint8_t *W, int64_t row_bytes, int in_f);
hipError_t launch_gemv_q8_0_mfma(const uint8_t *W, int64_t row_bytes, const int8_t *qs,
                                 const float *d, float *y, int m, int in_f, int out_f,
                                 hipStream_t s);
LaunchDesc describe_gemv_q8_0_mfma(int m, int in_f, int out_f);
LaunchDesc describe_gemv_q8_0(const uint8_t *W, int64_t row_bytes, int m, int in_f, int out_f,
                              bool matrix_cores);
hipError_t launch_requant_q8_0(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                               int grid_cols, bool blk128, void *Wq, int64_t q_row_bytes,
                               int in_f, int out_f, hipStream_t s);
hipError_t launch_read_bytes(const void *p, int64_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_read_pattern(const void *p, int64_t bytes, int pattern, int64_t row_bytes,
                               uint32_t *sink, hipStream_t s);

}  // namespace fp8gemv

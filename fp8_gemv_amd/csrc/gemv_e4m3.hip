// m=1 decode GEMV over raw OCP FP8 E4M3 weights, per-tensor or block-128 scaled, against a
// q8_1 activation.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc sections
// QUESTION and THE COMPARISON (the raw checkpoint e4m3 bytes are the weight stream, one byte
// per weight, row_bytes == in_f, no dequantisation pass) and THE BLOCK-128 ARM (an f32
// [ceil(out_f/128), ceil(in_f/128)] grid multiplies each 128x128 tile).
//
// gfx950 design (the page's kernel is a warp-per-row CUDA MMVQ doing cvt + fmaf; this one is
// not a translation of it):
//   * A workgroup is WAVES wave64s; each wave owns RPW consecutive weight rows.  A "window" is
//     1024 consecutive columns: lane l streams bytes [16l, 16l+16) of the window with one
//     16-byte non-temporal load per row, so every wave-wide load instruction reads 1 KiB of
//     contiguous HBM and every weight byte is fetched exactly once.  U windows x RPW rows of
//     loads are in flight per lane before any is consumed.
//   * Order of memory operations at kernel start: first the few activation loads this thread
//     stages, then the weight loads.  Loads of one wave complete in issue order, so staging
//     (which waits only for the older activation loads) overlaps the weight stream instead of
//     waiting behind it.
//   * The q8_1 activation row is staged once per workgroup in LDS as f16 (int8 is exact in
//     f16, converted with the 0x6400 exponent trick) next to its block scales -- for the
//     block-128 container the scale already times the grid value of the workgroup's
//     128-row tile (all rows of a workgroup lie in one tile).
//   * Decode: v_cvt_scalef32_pk_f16_fp8 turns two e4m3 bytes into two f16 with scale 1.0
//     (every e4m3 value, subnormals included, is exact in f16); v_dot2_f32_f16 multiplies a
//     weight pair by an activation pair and accumulates in f32 (each product is exact: 4 + 8
//     significant bits).  A lane's 16 columns lie in one q8_1 block and one 128-column tile,
//     so its 16-term partial is scaled once.
//   * At most 64 VGPRs (8 waves per SIMD): on this part occupancy, not arithmetic, decides
//     how close the stream gets to the HBM roofline.
//   * Each row's 64 lane partials are summed with a DPP butterfly + fixed-order readlanes.
// Activation rows t = blockIdx.y are independent and run identical code, so row t of an
// m-row call is bit-identical to an m=1 call on that row.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kWinCols = kWave * 16;  // 1024 columns per window

__host__ __device__ constexpr int num_windows(int in_f) { return (in_f + kWinCols - 1) / kWinCols; }

// LDS bytes for one staged activation row: f16 values then f32 block scales, whole windows.
__host__ __device__ constexpr size_t act_lds_bytes(int in_f) {
  return (size_t)num_windows(in_f) * (kWinCols * 2 + (kWinCols / 32) * 4);
}
// Plus a 32-byte sink that takes the staging writes of threads with nothing to stage, so
// that the staging code has no branches (a branch would let the compiler sink an activation
// load behind the weight loads and then wait for all of them).
constexpr size_t kSinkBytes = 32;

// int8 x4 -> two f16 pairs, exactly: after flipping the sign bit a byte u is 0..255 and the
// f16 with bits 0x6400 | u is 1024 + u; subtracting 1152 leaves the signed value.
__device__ __forceinline__ void i8x4_to_f16(uint32_t q, half2_t &lo, half2_t &hi) {
  const uint32_t u = q ^ 0x80808080u;
  const uint32_t a = (u & 0xFFu) | ((u & 0xFF00u) << 8) | 0x64006400u;
  const uint32_t b = ((u >> 16) & 0xFFu) | ((u >> 8) & 0xFF0000u) | 0x64006400u;
  const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(half2_t, a) - off;
  hi = __builtin_bit_cast(half2_t, b) - off;
}

// 16-term dot of one lane's 16 e4m3 weights (one 16-byte load) with 16 staged f16 values.
__device__ __forceinline__ float dot16(const int4_t w, const half2_t a[8]) {
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, false);
    const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, true);
    p = __builtin_amdgcn_fdot2(lo, a[2 * j], p, false);
    p = __builtin_amdgcn_fdot2(hi, a[2 * j + 1], p, false);
  }
  return p;
}

// Launch shape.  K chunks of 16 activation columns and KD block scales per thread cover the
// whole activation row: K * WAVES * 1024 >= in_f and KD * WAVES * 64 >= in_f / 32.
// DB: double-buffered window loop -- the next U windows are loaded before the current U are
// consumed, so a wave never waits with nothing in flight (rows of many windows).
template <int WAVES_, int RPW_, int U_, int K_, int KD_, bool DB_ = false, int WPE_ = 8,
          int SPLIT_ = 1>
struct Cfg {
  static constexpr int WAVES = WAVES_, RPW = RPW_, U = U_, K = K_, KD = KD_, WPE = WPE_;
  static constexpr int SPLIT = SPLIT_;  // waves sharing one group of RPW rows (split over k)
  static constexpr int ROWS = WAVES / SPLIT * RPW;  // rows per workgroup
  static constexpr bool DB = DB_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int MAX_IN_F = K * THREADS * 16;
};

template <bool BLK, class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_e4m3(const uint8_t *__restrict__ W, int64_t row_bytes, float scale,
                 const float *__restrict__ grid, int grid_cols, const int8_t *__restrict__ qs,
                 const float *__restrict__ d, float *__restrict__ y, int in_f, int out_f) {
  constexpr int RPW = C::RPW, U = C::U, K = C::K, KD = C::KD, NTH = C::THREADS;
  constexpr int SPLIT = C::SPLIT;
  static_assert(C::WAVES % SPLIT == 0 && 128 % C::ROWS == 0, "a workgroup's rows lie in one tile");
  extern __shared__ __align__(16) unsigned char lds[];
  const int nwin = num_windows(in_f);
  _Float16 *act = reinterpret_cast<_Float16 *>(lds);
  float *dsc = reinterpret_cast<float *>(lds + (size_t)nwin * kWinCols * 2);

  const int t = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int rbase = (blockIdx.x * (C::WAVES / SPLIT) + wave / SPLIT) * RPW;
  const int part = wave % SPLIT;
  const int wbeg = part * nwin / SPLIT, wend = (part + 1) * nwin / SPLIT;  // this wave's windows
  const int nb = in_f / 32;
  const rsrc_t qrs = buf_rsrc(qs + (int64_t)t * in_f, (uint32_t)in_f);
  const rsrc_t drs = buf_rsrc(d + (int64_t)t * nb, (uint32_t)nb * 4);

  // 1. this thread's share of the activation row (oldest loads; zeros past in_f).
  int4_t aq[K];
  float dv[KD];
#pragma unroll
  for (int k = 0; k < K; ++k) aq[k] = buf_load16(qrs, (uint32_t)(threadIdx.x + k * NTH) * 16);
#pragma unroll
  for (int k = 0; k < KD; ++k) dv[k] = buf_load_f32(drs, (uint32_t)(threadIdx.x + k * NTH) * 4);
  if (BLK) {
    // Grid row of this workgroup (its rows all lie in one 128-row tile); clamped so a
    // workgroup past the last row still reads inside the grid.
    const int rfirst = blockIdx.x * C::ROWS;
    const int grow = (rfirst < out_f ? rfirst : out_f - 1) / 128;
    const rsrc_t grs = buf_rsrc(grid + (int64_t)grow * grid_cols, (uint32_t)grid_cols * 4);
#pragma unroll
    for (int k = 0; k < KD; ++k) dv[k] *= buf_load_f32(grs, (uint32_t)((threadIdx.x + k * NTH) / 4) * 4);
  }

  // 2. the first batch of weight loads: one resource per row over its first in_f bytes (no
  // bytes for a row past out_f), so out-of-range windows and rows read as zeros.
  rsrc_t wrs[RPW];
  bool rok[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rok[r] = rbase + r < out_f;
    // wbeg < nwin, so wbeg * 1024 < in_f and the record count is never negative
    const int lim = in_f < wend * kWinCols ? in_f : wend * kWinCols;
    wrs[r] = buf_rsrc(W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes + (int64_t)wbeg * kWinCols,
                      rok[r] ? (uint32_t)(lim - wbeg * kWinCols) : 0u);
  }
  int4_t wv[U][RPW];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      wv[u][r] = buf_load16_stream(wrs[r], (uint32_t)(u * kWinCols + lane * 16));
  }

  // 3. stage the activation (f16) and its scales in LDS; zeros past in_f.  Threads past the
  // staged range write into the sink instead of branching around the store.
  unsigned char *sink = lds + act_lds_bytes(in_f);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int c = (threadIdx.x + k * NTH) * 16;
    half2_t h[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) i8x4_to_f16((uint32_t)aq[k][j], h[2 * j], h[2 * j + 1]);
    _Float16 *dst = c < nwin * kWinCols ? act + c : reinterpret_cast<_Float16 *>(sink);
    *reinterpret_cast<int4_t *>(dst) = *reinterpret_cast<const int4_t *>(h);
    *reinterpret_cast<int4_t *>(dst + 8) = *reinterpret_cast<const int4_t *>(h + 4);
  }
#pragma unroll
  for (int k = 0; k < KD; ++k) {
    const int b = threadIdx.x + k * NTH;
    float *dst = b < nwin * (kWinCols / 32) ? dsc + b : reinterpret_cast<float *>(sink);
    *dst = dv[k];
  }
  __syncthreads();

  // 4. stream.
  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;
  auto compute = [&](const int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int win = w0 + u;
      if (win < wend) {
        const int col = win * kWinCols + lane * 16;
        half2_t a[8];
        *reinterpret_cast<int4_t *>(a) = *reinterpret_cast<const int4_t *>(act + col);
        *reinterpret_cast<int4_t *>(a + 4) = *reinterpret_cast<const int4_t *>(act + col + 8);
        const float sc = dsc[col / 32];
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r] = fmaf(dot16(wb[u][r], a), sc, acc[r]);
      }
    }
  };
  // Loads are issued unconditionally: past the row they read zeros and no memory.
  auto load = [&](int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        wb[u][r] = buf_load16_stream(wrs[r], (uint32_t)((w0 + u - wbeg) * kWinCols + lane * 16));
    }
  };
  if constexpr (C::DB) {
    int4_t wv2[U][RPW];
    for (int w0 = wbeg; w0 < wend; w0 += 2 * U) {
      load(wv2, w0 + U);
      compute(wv, w0);
      if (w0 + U >= wend) break;
      load(wv, w0 + 2 * U);
      compute(wv2, w0 + U);
    }
  } else {
    for (int w0 = wbeg; w0 < wend; w0 += U) {
      compute(wv, w0);
      load(wv, w0 + U);
    }
  }

  if constexpr (SPLIT == 1) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float s = wave_sum(acc[r]);
      if (lane == 0 && rok[r]) y[(int64_t)t * out_f + rbase + r] = BLK ? s : s * scale;
    }
  } else {
    // the SPLIT partial sums of a row meet in LDS and are added in part order
    __shared__ float psum[C::WAVES * RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float s = wave_sum(acc[r]);
      if (lane == 0) psum[wave * RPW + r] = s;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (lane == 0 && part == 0 && rok[r]) {
        float s = psum[wave * RPW + r];
#pragma unroll
        for (int p = 1; p < SPLIT; ++p) s += psum[(wave + p) * RPW + r];
        y[(int64_t)t * out_f + rbase + r] = BLK ? s : s * scale;
      }
    }
  }
}

template <bool BLK, class C>
hipError_t launch_cfg(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                      int grid_cols, const int8_t *qs, const float *d, float *y, int m,
                      int in_f, int out_f, hipStream_t s) {
  auto kern = k_gemv_e4m3<BLK, C>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(act_lds_bytes(C::MAX_IN_F) + kSinkBytes));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 g((out_f + C::ROWS - 1) / C::ROWS, m);
  hipLaunchKernelGGL(kern, g, dim3(C::THREADS), act_lds_bytes(in_f) + kSinkBytes, s, W, row_bytes, scale,
                     grid, grid_cols, qs, d, y, in_f, out_f);
  return hipGetLastError();
}

// Shapes measured on MI355X: 4-wave workgroups with one row per wave up to in_f = 8192; 8
// waves (so that the larger LDS row still allows 32 waves per CU) up to 24576, two waves
// per row there (long rows, few of them: splitting keeps more, shorter-lived waves in
// flight; 6% faster at 5120 x 17408); 16 waves beyond.  All double-buffer their windows
// (2 to 4 per batch) and fit 64 VGPRs.
using CfgSmall = Cfg<4, 1, 2, 2, 1, true>;      // in_f <= 8192
using CfgMid = Cfg<8, 1, 3, 3, 2, true, 8, 2>;  // in_f <= 24576
using CfgLarge = Cfg<16, 1, 4, 4, 4, true>;  // in_f <= 65536
static_assert(CfgSmall::MAX_IN_F == 8192 && CfgMid::MAX_IN_F >= 24576 &&
                  CfgLarge::MAX_IN_F == kMaxInF, "activation coverage");
static_assert(CfgSmall::KD * CfgSmall::THREADS * 32 >= CfgSmall::MAX_IN_F &&
                  CfgMid::KD * CfgMid::THREADS * 32 >= CfgMid::MAX_IN_F &&
                  CfgLarge::KD * CfgLarge::THREADS * 32 >= CfgLarge::MAX_IN_F,
              "scale coverage");

template <bool BLK>
hipError_t dispatch(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                    int grid_cols, const int8_t *qs, const float *d, float *y, int m, int in_f,
                    int out_f, hipStream_t s) {
  if (in_f <= CfgSmall::MAX_IN_F)
    return launch_cfg<BLK, CfgSmall>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  if (in_f <= CfgMid::MAX_IN_F)
    return launch_cfg<BLK, CfgMid>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  return launch_cfg<BLK, CfgLarge>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
}

}  // namespace

hipError_t launch_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                            int grid_cols, bool blk128, const int8_t *qs, const float *d,
                            float *y, int m, int in_f, int out_f, hipStream_t s) {
  if (blk128) return dispatch<true>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  return dispatch<false>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
}

}  // namespace fp8gemv

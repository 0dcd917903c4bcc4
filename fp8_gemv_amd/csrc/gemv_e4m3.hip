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
//   * A workgroup is 4 wave64s; each wave owns RPW consecutive weight rows.  A "window" is
//     1024 consecutive columns: lane l streams bytes [16l, 16l+16) of the window with one
//     16-byte non-temporal load per row, so every wave-wide load instruction reads 1 KiB of
//     contiguous HBM and every weight byte is fetched exactly once.
//   * U windows x RPW rows of loads are issued before any of them is consumed, so each lane
//     keeps U*RPW 16-byte loads in flight.
//   * The q8_1 activation row is staged once per workgroup in LDS as f16 (int8 values are
//     exact in f16) plus its f32 block scales, zero-padded to whole windows.
//   * Decode: v_cvt_scalef32_pk_f16_fp8 turns two e4m3 bytes into two f16 with scale 1.0
//     (every e4m3 value, subnormals included, is exact in f16); v_dot2_f32_f16 multiplies a
//     weight pair by an activation pair and accumulates in f32 (each product is exact: 4 + 8
//     significant bits).  One lane's 16 columns lie in one q8_1 block and one 128-column
//     grid tile, so its 16-term partial is scaled once by the block scale (times the grid
//     value for block-128).
//   * Each row's 64 lane partials are summed with a DPP butterfly + fixed-order readlanes.
// Activation rows t = blockIdx.y are independent and run identical code, so row t of an
// m-row call is bit-identical to an m=1 call on that row.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kWinCols = kWave * 16;  // 1024 columns per window

__host__ __device__ constexpr int num_windows(int in_f) { return (in_f + kWinCols - 1) / kWinCols; }

// Bytes of LDS for one staged activation row: f16 values then f32 block scales.
__host__ __device__ constexpr size_t act_lds_bytes(int in_f) {
  return (size_t)num_windows(in_f) * (kWinCols * 2 + (kWinCols / 32) * 4);
}

// Stage q8_1 row t into LDS: f16 qs for columns [0, nwin*1024) and f32 d for blocks
// [0, nwin*32); entries past in_f are zero.
__device__ __forceinline__ void stage_activation(const int8_t *__restrict__ qs,
                                                 const float *__restrict__ d, int in_f,
                                                 _Float16 *act, float *dsc) {
  const int nwin = num_windows(in_f);
  const int ncols = nwin * kWinCols;
  for (int c = threadIdx.x * 16; c < ncols; c += kThreads * 16) {
    int4_t q = {0, 0, 0, 0};
    if (c < in_f) q = *reinterpret_cast<const int4_t *>(qs + c);
    _Float16 h[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) h[4 * j + b] = (_Float16)(int)(int8_t)(q[j] >> (8 * b));
    }
    *reinterpret_cast<int4_t *>(act + c) = *reinterpret_cast<const int4_t *>(h);
    *reinterpret_cast<int4_t *>(act + c + 8) = *reinterpret_cast<const int4_t *>(h + 8);
  }
  const int nb = in_f / 32;
  for (int b = threadIdx.x; b < nwin * (kWinCols / 32); b += kThreads) dsc[b] = (b < nb) ? d[b] : 0.0f;
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

template <bool BLK, int RPW, int U>
__global__ __launch_bounds__(kThreads) void k_gemv_e4m3(
    const uint8_t *__restrict__ W, int64_t row_bytes, float scale, const float *__restrict__ grid,
    int grid_cols, const int8_t *__restrict__ qs, const float *__restrict__ d,
    float *__restrict__ y, int in_f, int out_f) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int nwin = num_windows(in_f);
  _Float16 *act = reinterpret_cast<_Float16 *>(lds);
  float *dsc = reinterpret_cast<float *>(lds + (size_t)nwin * kWinCols * 2);

  const int t = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int rbase = (blockIdx.x * kWaves + wave) * RPW;

  const uint8_t *wrow[RPW];
  bool rok[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rok[r] = rbase + r < out_f;
    wrow[r] = W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes + lane * 16;
  }
  // Grid row of this wave's rows (RPW divides 128, so all of them share it); clamped so a wave
  // past the last row still reads inside the grid.
  const float *grow =
      BLK ? grid + (int64_t)((rbase < out_f ? rbase : out_f - 1) / 128) * grid_cols : nullptr;

  // Issue the first batch of weight loads before staging the activation so that HBM traffic
  // starts immediately.
  int4_t wv[U][RPW];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int col = u * kWinCols + lane * 16;
      wv[u][r] = (int4_t){0, 0, 0, 0};
      if (rok[r] && col < in_f) wv[u][r] = load_stream16(wrow[r] + u * kWinCols);
    }
  }

  stage_activation(qs + (int64_t)t * in_f, d + (int64_t)t * (in_f / 32), in_f, act, dsc);
  __syncthreads();

  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

  for (int w0 = 0; w0 < nwin; w0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int win = w0 + u;
      if (win < nwin) {
        const int col = win * kWinCols + lane * 16;
        half2_t a[8];
        *reinterpret_cast<int4_t *>(a) = *reinterpret_cast<const int4_t *>(act + col);
        *reinterpret_cast<int4_t *>(a + 4) = *reinterpret_cast<const int4_t *>(act + col + 8);
        float sc = dsc[col / 32];
        if (BLK) sc *= (col < in_f) ? grow[col / 128] : 0.0f;
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r] = fmaf(dot16(wv[u][r], a), sc, acc[r]);
      }
    }
    // Next batch.
    const int nxt = w0 + U;
    if (nxt < nwin) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const int col = (nxt + u) * kWinCols + lane * 16;
          wv[u][r] = (int4_t){0, 0, 0, 0};
          if (rok[r] && col < in_f) wv[u][r] = load_stream16(wrow[r] + (int64_t)(nxt + u) * kWinCols);
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float s = wave_sum(acc[r]);
    if (lane == 0 && rok[r]) y[(int64_t)t * out_f + rbase + r] = BLK ? s : s * scale;
  }
}

template <bool BLK, int RPW, int U>
hipError_t launch_cfg(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                      int grid_cols, const int8_t *qs, const float *d, float *y, int m,
                      int in_f, int out_f, hipStream_t s) {
  const size_t lds = act_lds_bytes(in_f);
  auto kern = k_gemv_e4m3<BLK, RPW, U>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)act_lds_bytes(kMaxInF));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int rows_per_wg = kWaves * RPW;
  const dim3 g((out_f + rows_per_wg - 1) / rows_per_wg, m);
  hipLaunchKernelGGL(kern, g, dim3(kThreads), lds, s, W, row_bytes, scale, grid, grid_cols, qs,
                     d, y, in_f, out_f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                            int grid_cols, bool blk128, const int8_t *qs, const float *d,
                            float *y, int m, int in_f, int out_f, hipStream_t s) {
  if (blk128)
    return launch_cfg<true, 2, 4>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  return launch_cfg<false, 2, 4>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
}

}  // namespace fp8gemv

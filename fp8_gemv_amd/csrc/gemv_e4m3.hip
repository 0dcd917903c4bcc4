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
//   * A workgroup is WAVES wave64s; each wave owns RPW consecutive weight rows, or, with
//     SPLIT > 1, a contiguous share of the windows of its rows (the SPLIT partial sums of a
//     row meet in LDS and are added in part order).  A "window" is 1024 consecutive
//     columns: lane l streams bytes [16l, 16l+16) of the window with one 16-byte
//     non-temporal load per row, so every wave-wide load instruction reads 1 KiB of
//     contiguous HBM and every weight byte is fetched exactly once.  U windows x RPW rows of
//     loads are in flight per lane before any is consumed (double-buffered batches).
//   * Order of memory operations at kernel start: first the few activation loads this thread
//     stages, then the weight loads.  Loads of one wave complete in issue order, so staging
//     (which waits only for the older activation loads) overlaps the weight stream instead of
//     waiting behind it.
//   * The q8_1 activation row is staged once per workgroup in LDS as f16 (int8 is exact in
//     f16, converted with the 0x6400 exponent trick; per window, the first 8 values of every
//     lane's chunk and then the last 8, so LDS reads are contiguous across the wave) next
//     to its block scales -- for the block-128 container the scale already times the grid
//     value of the workgroup's 128-row tile (all rows of a workgroup lie in one tile).
//   * Decode: v_cvt_scalef32_pk_f16_fp8 turns two e4m3 bytes into two f16 with scale 1.0
//     (every e4m3 value, subnormals included, is exact in f16); v_dot2_f32_f16 multiplies a
//     weight pair by an activation pair and accumulates in f32 (each product is exact: 4 + 8
//     significant bits).  A lane's 16 columns lie in one q8_1 block and one 128-column tile,
//     so its 16-term partial is scaled once.
//   * At most 64 VGPRs (8 waves per SIMD) for m = 1: on this part occupancy, not arithmetic,
//     decides how close the stream gets to the HBM roofline.
//   * Each row's 64 lane partials are summed with a DPP butterfly + fixed-order readlanes.
// Several activation rows (MT per workgroup, grid.y = ceil(m / MT)) share one weight pass:
// each weight chunk is decoded once and multiplied into every row with the same operations
// in the same order as for MT = 1, and every launch shape of an in_f range splits rows the
// same way, so row t of an m-row call is bit-identical to an m=1 call on that row.  The
// launches for 3 or more rows of up to 18432 columns are persistent: as many workgroups as fit
// on the device stage their activation rows once and then loop over the weight rows (each
// wave over groups of RPW rows, or, where two waves share a row, each workgroup over blocks
// of rows), so that the staging is not repeated per row group and the last groups spread over
// all CUs instead of leaving a partial round of workgroups.
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
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one CU, the most a workgroup may use

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

// One lane's 16 e4m3 weights (one 16-byte load) as 8 f16 pairs.  v_cvt_scalef32_pk_f16_fp8
// with scale 1.0 is exact: every e4m3 value, subnormals included, is an f16 normal.
__device__ __forceinline__ void decode16(const int4_t w, half2_t wh[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wh[2 * j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, false);
    wh[2 * j + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[j], 1.0f, true);
  }
}

// 16-term dot of decoded weights with 16 staged f16 activation values, accumulated in f32 in
// a fixed order (each product is exact: 4 + 8 significant bits).
__device__ __forceinline__ float dot16(const half2_t wh[8], const half2_t a[8]) {
  float p = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) p = __builtin_amdgcn_fdot2(wh[j], a[j], p, false);
  return p;
}

// Launch shape.  K chunks of 16 activation columns and KD block scales per thread cover the
// whole activation row: K * WAVES * 1024 >= in_f and KD * WAVES * 64 >= in_f / 32.
// DB: double-buffered window loop -- the next U windows are loaded before the current U are
// consumed, so a wave never waits with nothing in flight (rows of many windows).
// MT: activation rows per workgroup.  Each weight chunk is loaded and decoded once and used
// for all MT rows; every row's arithmetic is exactly the MT = 1 sequence.
template <int WAVES_, int RPW_, int U_, int K_, int KD_, bool DB_ = false, int WPE_ = 8,
          int SPLIT_ = 1, int MT_ = 1>
struct Cfg {
  static constexpr int WAVES = WAVES_, RPW = RPW_, U = U_, K = K_, KD = KD_, WPE = WPE_;
  static constexpr int SPLIT = SPLIT_;  // waves sharing one group of RPW rows (split over k)
  static constexpr int MT = MT_;
  // The launches for 4-8 staged activation rows are persistent: as many workgroups as fit on
  // the device at once, whose waves loop over row groups.  (With 2 rows the staging is cheap
  // and the launch already fills the device evenly; there the block-128 grid value, fetched
  // per window and row, cost more than the loop saved.)
  static constexpr bool PERSIST = MT_ >= 4;
  // workgroups that fit on one CU: WPE waves per SIMD, and the LDS of MT staged rows
  static constexpr int wgs_per_cu(int in_f) {
    const int by_waves = 4 * WPE_ / WAVES_;
    const int lds = (int)(MT_ * act_lds_bytes(in_f) + kSinkBytes);
    const int by_lds = (160 * 1024) / ((lds + 1023) / 1024 * 1024);
    return by_waves < by_lds ? by_waves : by_lds;
  }
  static constexpr int ROWS = WAVES / SPLIT * RPW;  // rows per workgroup
  static constexpr bool DB = DB_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int MAX_IN_F = K * THREADS * 16;
  // the template arguments, for config_text
  static constexpr const char *NAME = "Cfg";
  static constexpr int P0 = WAVES_, P1 = RPW_, P2 = U_, P3 = K_, P4 = KD_, P6 = WPE_, P7 = SPLIT_,
                       P8 = MT_;
  static constexpr bool P5 = DB_;
};

template <bool BLK, class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_e4m3(const uint8_t *__restrict__ W, int64_t row_bytes, float scale,
                 const float *__restrict__ grid, int grid_cols, const int8_t *__restrict__ qs,
                 const float *__restrict__ d, float *__restrict__ y, int m, int in_f, int out_f) {
  constexpr int RPW = C::RPW, U = C::U, K = C::K, KD = C::KD, NTH = C::THREADS, MT = C::MT;
  constexpr int SPLIT = C::SPLIT;
  static_assert(C::WAVES % SPLIT == 0 && 128 % C::ROWS == 0, "a workgroup's rows lie in one tile");
  static_assert(128 % RPW == 0, "a wave's rows lie in one tile");
  extern __shared__ __align__(16) unsigned char lds[];
  const int nwin = num_windows(in_f);
  const size_t row_lds = act_lds_bytes(in_f);  // one staged activation row

  const int t0 = blockIdx.y * MT;  // first activation row of this workgroup
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  // PERSIST: the resident workgroups stage their activation rows once and then loop over
  // units of weight rows.  With whole rows per wave (SPLIT == 1) a unit is one wave's RPW
  // rows and unit g belongs to wave g mod (waves of the grid), the waves numbered so that
  // consecutive units fall on different workgroups.  With rows split between waves a unit is
  // the workgroup's ROWS rows, taken by the workgroups in turn, so that the waves sharing a
  // row stay together.  Every row is still computed with the operations of m = 1.
  constexpr bool PERSIST = C::PERSIST;
  const int nunits = SPLIT == 1 ? (out_f + RPW - 1) / RPW : (out_f + C::ROWS - 1) / C::ROWS;
  const int ustride = SPLIT == 1 ? (int)gridDim.x * C::WAVES : (int)gridDim.x;
  int unit = SPLIT == 1 && PERSIST ? wave * (int)gridDim.x + (int)blockIdx.x : (int)blockIdx.x;
  auto rbase_of = [&](int u) {
    return SPLIT == 1 && PERSIST ? u * RPW : (u * (C::WAVES / SPLIT) + wave / SPLIT) * RPW;
  };
  int rbase = rbase_of(unit);
  const int part = wave % SPLIT;
  const int wbeg = part * nwin / SPLIT, wend = (part + 1) * nwin / SPLIT;  // this wave's windows
  const int nb = in_f / 32;

  // 1. this thread's share of the MT activation rows (oldest loads; zeros past in_f and for
  // rows past m).
  int4_t aq[MT][K];
  float dv[MT][KD];
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) {
    const bool tok = t0 + tt < m;
    const rsrc_t qrs = buf_rsrc(qs + (int64_t)(tok ? t0 + tt : 0) * in_f, tok ? (uint32_t)in_f : 0u);
    const rsrc_t drs = buf_rsrc(d + (int64_t)(tok ? t0 + tt : 0) * nb, tok ? (uint32_t)nb * 4 : 0u);
#pragma unroll
    for (int k = 0; k < K; ++k) aq[tt][k] = buf_load16(qrs, (uint32_t)(threadIdx.x + k * NTH) * 16);
#pragma unroll
    for (int k = 0; k < KD; ++k) dv[tt][k] = buf_load_f32(drs, (uint32_t)(threadIdx.x + k * NTH) * 4);
  }
  if (BLK && !PERSIST) {
    // Grid row of this workgroup (its rows all lie in one 128-row tile); clamped so a
    // workgroup past the last row still reads inside the grid.
    const int rfirst = blockIdx.x * C::ROWS;
    const int grow = (rfirst < out_f ? rfirst : out_f - 1) / 128;
    const rsrc_t grs = buf_rsrc(grid + (int64_t)grow * grid_cols, (uint32_t)grid_cols * 4);
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const float gv = buf_load_f32(grs, (uint32_t)((threadIdx.x + k * NTH) / 4) * 4);
#pragma unroll
      for (int tt = 0; tt < MT; ++tt) dv[tt][k] *= gv;
    }
  }

  // 2. the first batch of weight loads: one resource per row over this wave's windows of its
  // first in_f bytes (none for a row past out_f), so out-of-range windows read as zeros.
  rsrc_t wrs[RPW];
  bool rok[RPW];
  rsrc_t grs = buf_rsrc(grid, 0u);  // PERSIST, block-128: the grid row of the current rows
  auto setup_rows = [&]() {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      rok[r] = rbase + r < out_f;
      // wbeg < nwin, so wbeg * 1024 < in_f and the record count is never negative
      const int lim = in_f < wend * kWinCols ? in_f : wend * kWinCols;
      wrs[r] = buf_rsrc(W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes + (int64_t)wbeg * kWinCols,
                        rok[r] ? (uint32_t)(lim - wbeg * kWinCols) : 0u);
    }
    if constexpr (PERSIST && BLK) {
      // RPW divides 128, so a group's rows lie in one 128-row tile
      const bool ok = rbase < out_f;
      grs = buf_rsrc(grid + (int64_t)(ok ? rbase / 128 : 0) * grid_cols,
                     ok ? (uint32_t)grid_cols * 4 : 0u);
    }
  };
  setup_rows();
  // Loads are issued unconditionally: past the row they read zeros and no memory.  With
  // PERSIST and block-128, each window's grid value (the lane's 128-column tile, window * 8 +
  // lane / 8) comes in with the window's weights.
  auto load = [&](int4_t (&wb)[U][RPW], float (&gb)[U], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        wb[u][r] = buf_load16_stream(wrs[r], (uint32_t)((w0 + u - wbeg) * kWinCols + lane * 16));
      if constexpr (PERSIST && BLK)
        gb[u] = buf_load_f32(grs, (uint32_t)(((w0 + u) * (kWinCols / 128) + lane / 8) * 4));
      else
        gb[u] = 1.0f;
    }
  };
  int4_t wv[U][RPW];
  float gv1[U];
  load(wv, gv1, wbeg);

  // 3. stage the activation rows (f16) and their scales in LDS; zeros past in_f.  Threads
  // past the staged range write into the sink instead of branching around the store.
  unsigned char *sink = lds + MT * row_lds;
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) {
    _Float16 *act = reinterpret_cast<_Float16 *>(lds + tt * row_lds);
    float *dsc = reinterpret_cast<float *>(lds + tt * row_lds + (size_t)nwin * kWinCols * 2);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int c = (threadIdx.x + k * NTH) * 16;
      half2_t h[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) i8x4_to_f16((uint32_t)aq[tt][k][j], h[2 * j], h[2 * j + 1]);
      // Window layout: the first 8 values of all 64 lanes' chunks, then the last 8, so that
      // each of a lane's two 16-byte LDS reads is contiguous across the wave (no bank
      // conflicts).  Chunk c / 16 is lane (c / 16) % 64 of window c / 1024.
      const int base = (c / kWinCols) * kWinCols + ((c / 16) % kWave) * 8;
      _Float16 *lo = c < nwin * kWinCols ? act + base : reinterpret_cast<_Float16 *>(sink);
      _Float16 *hi = c < nwin * kWinCols ? act + base + kWinCols / 2 : reinterpret_cast<_Float16 *>(sink);
      *reinterpret_cast<int4_t *>(lo) = *reinterpret_cast<const int4_t *>(h);
      *reinterpret_cast<int4_t *>(hi) = *reinterpret_cast<const int4_t *>(h + 4);
    }
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const int b = threadIdx.x + k * NTH;
      float *dst = b < nwin * (kWinCols / 32) ? dsc + b : reinterpret_cast<float *>(sink);
      *dst = dv[tt][k];
    }
  }
  __syncthreads();

  // 4. stream.
  float acc[MT][RPW];
#pragma unroll
  for (int tt = 0; tt < MT; ++tt)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[tt][r] = 0.0f;
  auto compute = [&](const int4_t (&wb)[U][RPW], const float (&gb)[U], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int win = w0 + u;
      if (win < wend) {
        const int col = win * kWinCols + lane * 16;
        half2_t wh[RPW][8];
#pragma unroll
        for (int r = 0; r < RPW; ++r) decode16(wb[u][r], wh[r]);
        // Activation row tt's 16 values and block scale from LDS; row tt + 1 is read while
        // row tt is multiplied, so the LDS latency is not paid once per row.
        auto read_row = [&](int tt, half2_t (&a)[8], float &sc) {
          const _Float16 *act = reinterpret_cast<const _Float16 *>(lds + tt * row_lds);
          const float *dsc =
              reinterpret_cast<const float *>(lds + tt * row_lds + (size_t)nwin * kWinCols * 2);
          const int base = win * kWinCols + lane * 8;
          *reinterpret_cast<int4_t *>(a) = *reinterpret_cast<const int4_t *>(act + base);
          *reinterpret_cast<int4_t *>(a + 4) =
              *reinterpret_cast<const int4_t *>(act + base + kWinCols / 2);
          sc = dsc[col / 32];
          if constexpr (PERSIST && BLK) sc = sc * gb[u];
        };
        half2_t a[2][8];
        float sc[2];
        read_row(0, a[0], sc[0]);
#pragma unroll
        for (int tt = 0; tt < MT; ++tt) {
          if (tt + 1 < MT) read_row(tt + 1, a[(tt + 1) & 1], sc[(tt + 1) & 1]);
#pragma unroll
          for (int r = 0; r < RPW; ++r)
            acc[tt][r] = fmaf(dot16(wh[r], a[tt & 1]), sc[tt & 1], acc[tt][r]);
        }
      }
    }
  };
  int pbuf = 0;  // SPLIT > 1: the partial-sum buffer of this unit
  for (;;) {
  if constexpr (C::DB) {
    int4_t wv2[U][RPW];
    float gv2[U];
    for (int w0 = wbeg; w0 < wend; w0 += 2 * U) {
      load(wv2, gv2, w0 + U);
      compute(wv, gv1, w0);
      if (w0 + U >= wend) break;
      load(wv, gv1, w0 + 2 * U);
      compute(wv2, gv2, w0 + U);
    }
  } else {
    for (int w0 = wbeg; w0 < wend; w0 += U) {
      compute(wv, gv1, w0);
      load(wv, gv1, w0 + U);
    }
  }

  if constexpr (SPLIT == 1) {
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float s = wave_sum(acc[tt][r]);
        if (lane == 0 && rok[r] && t0 + tt < m)
          y[(int64_t)(t0 + tt) * out_f + rbase + r] = BLK ? s : s * scale;
      }
    }
  } else {
    // the SPLIT partial sums of a row meet in LDS and are added in part order; two buffers
    // used in turn, because the barrier of the next unit is the first point where every wave
    // has finished reading this one
    __shared__ float psum[2][MT][C::WAVES * RPW];
    float(*ps)[C::WAVES * RPW] = psum[pbuf];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float s = wave_sum(acc[tt][r]);
        if (lane == 0) ps[tt][wave * RPW + r] = s;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (lane == 0 && part == 0 && rok[r] && t0 + tt < m) {
          float s = ps[tt][wave * RPW + r];
#pragma unroll
          for (int p = 1; p < SPLIT; ++p) s += ps[tt][(wave + p) * RPW + r];
          y[(int64_t)(t0 + tt) * out_f + rbase + r] = BLK ? s : s * scale;
        }
      }
    }
    pbuf ^= 1;
  }
    if constexpr (!PERSIST) break;
    // the next unit of this wave (SPLIT == 1) or workgroup (SPLIT > 1), if any: uniform over
    // the wave, and over the workgroup when its waves share rows, so every wave of a
    // workgroup meets the same barriers
    unit += ustride;
    if (unit >= nunits) break;
    rbase = rbase_of(unit);
    setup_rows();
    load(wv, gv1, wbeg);
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[tt][r] = 0.0f;
  }
}

// Workgroups along x: one per ROWS rows, or for a persistent launch as many as fit on the
// device at once (at most one per WAVES row groups), so one round covers the grid.
template <class C>
unsigned grid_x_for(int out_f, int in_f) {
  if constexpr (C::PERSIST) {
    // units: groups of RPW rows (whole rows per wave) or of ROWS rows (rows split over waves)
    const int want = C::SPLIT == 1 ? ((out_f + C::RPW - 1) / C::RPW + C::WAVES - 1) / C::WAVES
                                   : (out_f + C::ROWS - 1) / C::ROWS;
    const int cap = cu_count() * C::wgs_per_cu(in_f);
    return (unsigned)(want < cap ? want : cap);
  } else {
    return (unsigned)((out_f + C::ROWS - 1) / C::ROWS);
  }
}

template <bool BLK, class C>
hipError_t launch_cfg(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                      int grid_cols, const int8_t *qs, const float *d, float *y, int m,
                      int in_f, int out_f, hipStream_t s) {
  auto kern = k_gemv_e4m3<BLK, C>;
  static std::atomic<bool> lds_set[kMaxDevices];
  // The dynamic LDS limit leaves room for the kernel's static partial-sum buffers (at most
  // 2 * MT * WAVES * RPW floats), which count against the same 160 KiB.
  const size_t want = C::MT * act_lds_bytes(C::MAX_IN_F) + kSinkBytes;
  const size_t cap = kLdsBytes - 2 * C::MT * C::WAVES * C::RPW * sizeof(float);
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void *>(kern),
                                          want < cap ? want : cap, lds_set);
  if (e != hipSuccess) return e;
  const dim3 g(grid_x_for<C>(out_f, in_f), (m + C::MT - 1) / C::MT);
  hipLaunchKernelGGL(kern, g, dim3(C::THREADS), C::MT * act_lds_bytes(in_f) + kSinkBytes, s, W,
                     row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f);
  return hipGetLastError();
}

// Shapes measured on MI355X: 4-wave workgroups with one row per wave up to in_f = 8192; 8
// waves (so that the larger LDS row still allows 32 waves per CU) up to 24576, two waves
// per row there (long rows, few of them: splitting keeps more, shorter-lived waves in
// flight; 6% faster at 5120 x 17408); 16 waves beyond.  All double-buffer their windows
// (2 to 4 per batch) and fit 64 VGPRs.
// Several activation rows (m > 1) share each weight pass: up to 8 rows per workgroup for
// in_f <= 8192, 4 up to 18432, 2 up to 24576 and 1 beyond (LDS holds one staged row per
// activation row).  Every shape
// used for one in_f range splits rows the same way (SPLIT), so each activation row is
// computed in the same order whatever m is.
using CfgSmall = Cfg<4, 1, 2, 2, 1, true>;                // in_f <= 8192, m = 1
using CfgSmallB2 = Cfg<8, 1, 2, 1, 1, true, 8, 1, 2>;     //               m = 2
using CfgSmallB4 = Cfg<8, 2, 1, 1, 1, true, 5, 1, 4>;     //               m = 3..4
using CfgSmallB8 = Cfg<16, 2, 1, 1, 1, true, 4, 1, 8>;    //               m >= 5
using CfgMid = Cfg<8, 1, 3, 3, 2, true, 8, 2>;            // in_f <= 24576, m = 1
using CfgMidB2 = Cfg<8, 1, 3, 3, 2, true, 8, 2, 2>;       //                m = 2 (and beyond 18432)
using CfgMidB4 = Cfg<8, 1, 3, 3, 2, true, 4, 2, 4>;       // in_f <= 18432, m >= 3
using CfgLarge = Cfg<16, 1, 4, 4, 4, true>;               // in_f <= 65536
static_assert(CfgSmall::MAX_IN_F == 8192 && CfgSmallB2::MAX_IN_F >= 8192 &&
                  CfgSmallB4::MAX_IN_F >= 8192 && CfgSmallB8::MAX_IN_F >= 8192 &&
                  CfgMid::MAX_IN_F >= 24576 && CfgMidB2::MAX_IN_F >= 24576 &&
                  CfgMidB4::MAX_IN_F >= 18432 &&
                  CfgLarge::MAX_IN_F == kMaxInF, "activation coverage");
static_assert(CfgSmall::KD * CfgSmall::THREADS * 32 >= CfgSmall::MAX_IN_F &&
                  CfgSmallB2::KD * CfgSmallB2::THREADS * 32 >= 8192 &&
                  CfgSmallB4::KD * CfgSmallB4::THREADS * 32 >= 8192 &&
                  CfgSmallB8::KD * CfgSmallB8::THREADS * 32 >= 8192 &&
                  CfgMid::KD * CfgMid::THREADS * 32 >= CfgMid::MAX_IN_F &&
                  CfgMidB2::KD * CfgMidB2::THREADS * 32 >= 24576 &&
                  CfgMidB4::KD * CfgMidB4::THREADS * 32 >= 18432 &&
                  CfgLarge::KD * CfgLarge::THREADS * 32 >= CfgLarge::MAX_IN_F,
              "scale coverage");
static_assert(CfgSmallB8::MT * act_lds_bytes(8192) + kSinkBytes <= kLdsBytes &&
                  CfgMidB2::MT * act_lds_bytes(24576) + kSinkBytes <= kLdsBytes &&
                  CfgMidB4::MT * act_lds_bytes(18432) + kSinkBytes +
                          2 * CfgMidB4::MT * CfgMidB4::WAVES * CfgMidB4::RPW * sizeof(float) <=
                      kLdsBytes &&
                  act_lds_bytes(kMaxInF) + kSinkBytes <= kLdsBytes,
              "staged rows fit the LDS of a workgroup");
static_assert(CfgSmall::SPLIT == CfgSmallB2::SPLIT && CfgSmall::SPLIT == CfgSmallB4::SPLIT &&
                  CfgSmall::SPLIT == CfgSmallB8::SPLIT && CfgMid::SPLIT == CfgMidB2::SPLIT &&
                  CfgMid::SPLIT == CfgMidB4::SPLIT,
              "one row split per in_f range");

// The launch shape for (m, in_f): f is called with the Tag of the chosen configuration.
template <class F>
auto with_cfg(int m, int in_f, F &&f) {
  if (in_f <= 8192) {
    if (m == 1) return f(Tag<CfgSmall>{});
    if (m == 2) return f(Tag<CfgSmallB2>{});
    if (m <= 4) return f(Tag<CfgSmallB4>{});
    return f(Tag<CfgSmallB8>{});
  }
  if (in_f <= 24576) {
    if (m == 1) return f(Tag<CfgMid>{});
    if (m >= 3 && in_f <= 18432) return f(Tag<CfgMidB4>{});
    return f(Tag<CfgMidB2>{});
  }
  return f(Tag<CfgLarge>{});
}

template <bool BLK>
hipError_t dispatch(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                    int grid_cols, const int8_t *qs, const float *d, float *y, int m, int in_f,
                    int out_f, hipStream_t s) {
  return with_cfg(m, in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    return launch_cfg<BLK, C>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  });
}

}  // namespace

hipError_t launch_gemv_e4m3(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                            int grid_cols, bool blk128, const int8_t *qs, const float *d,
                            float *y, int m, int in_f, int out_f, bool matrix_cores,
                            hipStream_t s) {
  if (matrix_cores && gemv_e4m3_mfma_applies(row_bytes, in_f))
    return launch_gemv_e4m3_mfma(W, row_bytes, scale, grid, grid_cols, blk128, qs, d, y, m, in_f,
                                 out_f, s);
  if (blk128) return dispatch<true>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  return dispatch<false>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
}

LaunchDesc describe_gemv_e4m3(bool blk128, int64_t row_bytes, int m, int in_f, int out_f,
                              bool matrix_cores) {
  if (matrix_cores && gemv_e4m3_mfma_applies(row_bytes, in_f))
    return describe_gemv_e4m3_mfma(blk128, m, in_f, out_f);
  return with_cfg(m, in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    LaunchDesc r;
    r.grid_x = grid_x_for<C>(out_f, in_f);
    r.grid_y = (unsigned)((m + C::MT - 1) / C::MT);
    r.threads = C::THREADS;
    r.lds = (unsigned)(C::MT * act_lds_bytes(in_f) + kSinkBytes);
    r.kernel = blk128 ? "k_gemv_e4m3<true" : "k_gemv_e4m3<false";
    r.config = config_text<C>();
    return r;
  });
}

}  // namespace fp8gemv

// Measurement aids: stream a byte range from HBM in one of several load patterns and do
// nothing with the data but fold it into one word.  Their durations over cold ranges give the
// achievable read time the GEMVs are compared with, and split a launch's fixed cost into its
// parts (an empty grid of the same size, one wave's single cold round trip).
//
// Every pattern issues 16-byte buffer loads whose resource covers only the range handed in, so
// no load reaches past it (out-of-range lanes read zeros and touch no memory).  The fold ends
// in a store that depends on the data and never happens in practice, which keeps the loads
// alive.
#include "../../include/fp8_gemv.h"
#include "common.hpp"

namespace fp8gemv {
namespace {

__device__ __forceinline__ uint32_t fold(const int4_t v) {
  return (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
}
__device__ __forceinline__ void keep(uint32_t x, uint32_t *sink) {
  if (x == 0x9E3779B9u && threadIdx.x % kWave == 0) sink[0] = x;
}

template <int AUX>
__device__ __forceinline__ int4_t load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// Contiguous chunks: wave w of workgroup b reads LOADS KiB starting at (b * WAVES + w) * LOADS
// KiB, all loads issued before any is consumed (LOADS loads in flight per lane).
template <int WAVES, int LOADS, int AUX, int WPE>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void k_read_chunks(const uint8_t *__restrict__ p, int64_t bytes, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x % kWave;
  const int64_t base = ((int64_t)blockIdx.x * WAVES + wave_id()) * LOADS * 1024;
  const int64_t left = bytes - base;
  const rsrc_t rs = buf_rsrc(p + (base < bytes ? base : 0),
                             left <= 0 ? 0u : (uint32_t)(left < LOADS * 1024 ? left : LOADS * 1024));
  int4_t v[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) v[u] = load16<AUX>(rs, (uint32_t)(u * 1024 + lane * 16));
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < LOADS; ++u) x ^= fold(v[u]);
  keep(x, sink);
}

// Grid sized to the resident waves: every wave strides over 4 KiB blocks (block index
// = global wave + k * total waves), the next block's loads issued before the current block is
// folded (8 loads in flight per lane).  The loop ends for every wave once its index passes
// the last block.
constexpr int kPersistWaves = 4;
constexpr int kPersistLoads = 4;
__global__ __launch_bounds__(kPersistWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_read_persistent(const uint8_t *__restrict__ p, int64_t bytes, uint32_t *__restrict__ sink) {
  constexpr int64_t kBlk = kPersistLoads * 1024;
  const int lane = threadIdx.x % kWave;
  const int64_t nblk = (bytes + kBlk - 1) / kBlk;
  const int64_t total = (int64_t)gridDim.x * kPersistWaves;
  auto rsrc = [&](int64_t b) {
    const int64_t base = b * kBlk;
    const int64_t left = bytes - base;
    return buf_rsrc(p + (b < nblk ? base : 0),
                    left <= 0 || b >= nblk ? 0u : (uint32_t)(left < kBlk ? left : kBlk));
  };
  int64_t b = (int64_t)blockIdx.x * kPersistWaves + wave_id();
  int4_t cur[kPersistLoads], nxt[kPersistLoads];
  rsrc_t rs = rsrc(b);
#pragma unroll
  for (int u = 0; u < kPersistLoads; ++u)
    cur[u] = load16<kAuxNonTemporal>(rs, (uint32_t)(u * 1024 + lane * 16));
  uint32_t x = 0;
  for (; b < nblk; b += total) {
    rs = rsrc(b + total);  // zero-length past the last block: those loads read nothing
#pragma unroll
    for (int u = 0; u < kPersistLoads; ++u)
      nxt[u] = load16<kAuxNonTemporal>(rs, (uint32_t)(u * 1024 + lane * 16));
#pragma unroll
    for (int u = 0; u < kPersistLoads; ++u) {
      x ^= fold(cur[u]);
      cur[u] = nxt[u];
    }
  }
  keep(x, sink);
}

// Rows of row_bytes, one wave per row, 4-wave workgroups, windows of WIN_LANES * 16 bytes
// (lanes past WIN_LANES load nothing), batches of 4 windows with the next batch in flight
// while the current one is folded: the load pattern of the GEMVs at m = 1 (64 lanes: the e4m3
// stream's 1 KiB windows; 51 lanes: the Q8_0 stream's 816-byte windows of three 8-block groups).
template <int WIN_LANES>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_read_rows(const uint8_t *__restrict__ p, int64_t row_bytes, int64_t rows,
                 uint32_t *__restrict__ sink) {
  constexpr int U = 4;
  constexpr int kWin = WIN_LANES * 16;
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  const bool ok = row < rows;
  const rsrc_t rs = buf_rsrc(p + (ok ? row * row_bytes : 0), ok ? (uint32_t)row_bytes : 0u);
  const uint32_t lane_off = lane < WIN_LANES ? (uint32_t)lane * 16 : 0x40000000u;
  const int nwin = (int)((row_bytes + kWin - 1) / kWin);
  int4_t a[U], b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = load16<kAuxNonTemporal>(rs, lane_off + u * kWin);
  uint32_t x = 0;
  for (int w0 = 0; w0 < nwin; w0 += 2 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = load16<kAuxNonTemporal>(rs, lane_off + (w0 + U + u) * kWin);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(a[u]);
    if (w0 + U >= nwin) break;
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = load16<kAuxNonTemporal>(rs, lane_off + (w0 + 2 * U + u) * kWin);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(b[u]);
  }
  keep(x, sink);
}

// Rows of row_bytes, one wave per row, each row read from the 128-byte line boundary at or
// before its first byte in 1 KiB windows (every wave-wide load covers 8 whole lines); the
// bytes before the row lie before its resource (negative offsets, wrapped) and read as zeros.
// Batches of 3 windows with the next batch in flight.
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_read_rows_aligned(const uint8_t *__restrict__ p, int64_t row_bytes, int64_t rows,
                         uint32_t *__restrict__ sink) {
  constexpr int U = 3;
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave_id();
  const bool ok = row < rows;
  const uint8_t *rp = p + (ok ? row * row_bytes : 0);
  const rsrc_t rs = buf_rsrc(rp, ok ? (uint32_t)row_bytes : 0u);
  const uint32_t pre = (uint32_t)(reinterpret_cast<uintptr_t>(rp) & 127u);
  const uint32_t lo = (uint32_t)lane * 16 - pre;  // wraps for the lanes before the row
  const int nwin = (int)((pre + (uint64_t)row_bytes + 1023) / 1024);
  int4_t a[U], b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = load16<kAuxNonTemporal>(rs, lo + u * 1024);
  uint32_t x = 0;
  for (int w0 = 0; w0 < nwin; w0 += 2 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) b[u] = load16<kAuxNonTemporal>(rs, lo + (w0 + U + u) * 1024);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(a[u]);
    if (w0 + U >= nwin) break;
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = load16<kAuxNonTemporal>(rs, lo + (w0 + 2 * U + u) * 1024);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(b[u]);
  }
  keep(x, sink);
}

// Line windows: a 4-wave workgroup owns R consecutive rows (R * row_bytes a multiple of 2176
// when there are R of them) and reads them as one span of 2176-byte windows (17 whole lines;
// for Q8_0 rows, 8 groups of 8 blocks), window K by wave K % 4, each as lines 0-7 and 8-15 (64
// lanes) and line 16 (8 lanes).  Batches of 2 windows with the next batch in flight.
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_read_line_windows(const uint8_t *__restrict__ p, int64_t row_bytes, int64_t rows, int R,
                         uint32_t *__restrict__ sink) {
  constexpr int U = 2;
  constexpr uint32_t kWin = 2176;
  const int lane = threadIdx.x % kWave, w = wave_id();
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int64_t nr = r0 < rows ? (rows - r0 < R ? rows - r0 : R) : 0;
  const uint32_t span = (uint32_t)(nr * row_bytes);
  const rsrc_t rs = buf_rsrc(p + (nr ? r0 * row_bytes : 0), span);
  const int nwin = (int)((span + kWin - 1) / kWin);
  const int nmine = nwin > w ? (nwin - w + 3) / 4 : 0;
  auto base = [&](int i) -> uint32_t { return i < nmine ? (uint32_t)(w + 4 * i) * kWin : 0x40000000u; };
  const uint32_t lo = (uint32_t)lane * 16, lc = lane < 8 ? 2048u + (uint32_t)lane * 16 : 0x40000000u;
  int4_t a[U][3], b[U][3];
  auto load3 = [&](int4_t (&v)[3], uint32_t bb) {
    v[0] = load16<kAuxNonTemporal>(rs, bb + lo);
    v[1] = load16<kAuxNonTemporal>(rs, bb + 1024 + lo);
    v[2] = load16<kAuxNonTemporal>(rs, bb + lc);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) load3(a[u], base(u));
  uint32_t x = 0;
  for (int w0 = 0; w0 < nmine; w0 += 2 * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) load3(b[u], base(w0 + U + u));
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(a[u][0]) ^ fold(a[u][1]) ^ fold(a[u][2]);
    if (w0 + U >= nmine) break;
#pragma unroll
    for (int u = 0; u < U; ++u) load3(a[u], base(w0 + 2 * U + u));
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= fold(b[u][0]) ^ fold(b[u][1]) ^ fold(b[u][2]);
  }
  keep(x, sink);
}

// The grid of the 8 KiB-per-wave pattern with no loads: what dispatch and drain cost alone.
__global__ __launch_bounds__(4 * kWave) void k_read_empty(int64_t bytes, uint32_t *__restrict__ sink) {
  if (bytes < 0 && threadIdx.x == 0) sink[0] = 0;  // never: bytes >= 1
}

template <class K, class... A>
hipError_t launch(K kern, unsigned grid, unsigned threads, hipStream_t s, A... args) {
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, s, args...);
  return hipGetLastError();
}

template <int WAVES, int LOADS, int AUX, int WPE>
hipError_t launch_chunks(const uint8_t *p, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t per_wg = (int64_t)WAVES * LOADS * 1024;
  return launch(k_read_chunks<WAVES, LOADS, AUX, WPE>, (unsigned)((bytes + per_wg - 1) / per_wg),
                WAVES * kWave, s, p, bytes, sink);
}

}  // namespace

hipError_t launch_read_bytes(const void *p, int64_t bytes, uint32_t *sink, hipStream_t s) {
  return launch_chunks<4, 8, kAuxNonTemporal, 8>(static_cast<const uint8_t *>(p), bytes, sink, s);
}

hipError_t launch_read_pattern(const void *pv, int64_t bytes, int pattern, int64_t row_bytes,
                               uint32_t *sink, hipStream_t s) {
  const uint8_t *p = static_cast<const uint8_t *>(pv);
  switch (pattern) {
    case FP8GEMV_READ_CHUNK8K: return launch_chunks<4, 8, kAuxNonTemporal, 8>(p, bytes, sink, s);
    case FP8GEMV_READ_CHUNK16K: return launch_chunks<4, 16, kAuxNonTemporal, 4>(p, bytes, sink, s);
    case FP8GEMV_READ_WG8: return launch_chunks<8, 8, kAuxNonTemporal, 8>(p, bytes, sink, s);
    case FP8GEMV_READ_WG16: return launch_chunks<16, 8, kAuxNonTemporal, 8>(p, bytes, sink, s);
    case FP8GEMV_READ_CACHED: return launch_chunks<4, 8, 0, 8>(p, bytes, sink, s);
    case FP8GEMV_READ_PERSISTENT: {
      // 8 waves per SIMD, 4 SIMDs per CU: 8 four-wave workgroups per CU
      const int64_t nblk = (bytes + kPersistLoads * 1024 - 1) / (kPersistLoads * 1024);
      int64_t wgs = (int64_t)cu_count() * 8;
      const int64_t need = (nblk + kPersistWaves - 1) / kPersistWaves;
      if (need < wgs) wgs = need;
      return launch(k_read_persistent, (unsigned)wgs, kPersistWaves * kWave, s, p, bytes, sink);
    }
    case FP8GEMV_READ_ROWS_1K:
    case FP8GEMV_READ_ROWS_816: {
      const int64_t rows = bytes / row_bytes;
      const unsigned grid = (unsigned)((rows + 3) / 4);
      if (pattern == FP8GEMV_READ_ROWS_1K)
        return launch(k_read_rows<64>, grid, 4 * kWave, s, p, row_bytes, rows, sink);
      return launch(k_read_rows<51>, grid, 4 * kWave, s, p, row_bytes, rows, sink);
    }
    case FP8GEMV_READ_ROWS_ALIGNED: {
      const int64_t rows = bytes / row_bytes;
      return launch(k_read_rows_aligned, (unsigned)((rows + 3) / 4), 4 * kWave, s, p, row_bytes,
                    rows, sink);
    }
    case FP8GEMV_READ_LINE_WINDOWS: {
      const int64_t rows = bytes / row_bytes;
      int64_t g = 2176, r = row_bytes;
      while (r) { const int64_t t = g % r; g = r; r = t; }  // gcd(2176, row_bytes)
      const int R = (int)(2176 / g);
      return launch(k_read_line_windows, (unsigned)((rows + R - 1) / R), 4 * kWave, s, p,
                    row_bytes, rows, R, sink);
    }
    case FP8GEMV_READ_EMPTY:
      return launch(k_read_empty, (unsigned)((bytes + 32767) / 32768), 4 * kWave, s, bytes, sink);
    case FP8GEMV_READ_ONE_WAVE:
      return launch(k_read_chunks<1, 1, kAuxNonTemporal, 8>, 1u, kWave, s, p,
                    bytes < 1024 ? bytes : (int64_t)1024, sink);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8gemv

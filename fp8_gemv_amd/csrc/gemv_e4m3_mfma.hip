// Several activation rows at once over raw OCP e4m3 weights (per-tensor or block-128 scaled),
// on the matrix cores.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc sections THE
// COMPARISON and THE BLOCK-128 ARM: the contraction of the m = 1 GEMV (e4m3 weight rows,
// row_bytes == in_f, times a q8_1 activation row), here for a few activation rows, which
// makes it a skinny product Y[m, out_f] = X[m, in_f] * W^T.
//
// Why the matrix cores: with m activation rows the vector path spends, per weight pair, one
// decode and m dot-2 instructions, and beyond m = 4 that is more than the SIMDs issue while
// the weights stream at the HBM rate (measured at 17408 x 5120: 21.6 us at m = 4, 45 us at
// m = 8).  v_mfma_f32_16x16x32_f16 does 16 x 16 x 32 products in one instruction, so the cost
// no longer grows with m: this kernel takes 26.4 us for any m from 3 to 8 at that shape, so
// it serves m >= 5.
//
// gfx950 design:
//   * A workgroup is 4 wave64s.  Each wave owns 16 consecutive weight rows (the MFMA's M
//     dimension); a workgroup owns 64 rows, which always lie in one 128-row tile of the
//     block-128 grid.  Up to 8 activation rows per workgroup (grid.y = ceil(m / 8)) are the
//     MFMA's N columns 0..7; columns 8..15 repeat them and are never stored.
//   * Weights stream in steps of 256 columns.  One wave-wide 16-byte non-temporal buffer load
//     covers 4 rows x 256 contiguous bytes (lanes 16r..16r+15 read row r), so 4 loads cover
//     the wave's 16 rows and every weight byte is fetched once.  U steps are in flight per
//     wave.  Past in_f (or past out_f) a lane's offset lies outside the buffer resource and
//     the load returns zeros without touching memory.
//   * Each step goes through a per-wave LDS relay (16 rows x 256 bytes, row pitch 288 so
//     that the fragment reads below are conflict-free) and comes back as MFMA A fragments:
//     lane (i, g) = (lane % 16, lane / 16) reads 8 bytes of row i at column 32k + 8g for the
//     step's k-th 32-column block.  v_cvt_scalef32_pk_f16_fp8 with scale 1.0 decodes them to
//     f16 exactly (every e4m3 value, subnormals included, is an f16 normal).
//   * The workgroup's 8 activation rows are staged once in LDS as int8 with the sign bit
//     flipped (u = q ^ 0x80), with their block scales (times the grid value of the
//     workgroup's tile for block-128).  A B fragment is 8 bytes of row j = lane % 16 (mod 8)
//     at the same columns; a byte permute against 0x64 makes the f16 1024 + u and one packed
//     subtraction of 1152 leaves q, exactly.
//   * One MFMA covers 32 columns, exactly one q8_1 block and a quarter of a 128-column tile,
//     so its 16 x 16 result is scaled per activation row by that block's scale.
// Numerics: each product (4 + 8 significant bits) is exact in f16 x f16; the MFMA sums a
// block's 32 products in f32; acc += D * scale with one fma, into one of 4 accumulators by
// block index mod 4, so that no f32 chain has more than in_f / 128 terms; the 4 are added in
// a fixed order at the end.  Deterministic (no atomics, every order fixed), and each output
// depends only on its own weight row and activation row, whatever m and the row's position in
// the call.  The rounding differs from the vector path's, so an m-row call on this path is not
// bit-identical to m = 1; both are within the parity tolerance of the exact result.
#include "common.hpp"

namespace fp8gemv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

constexpr int kRowsPerWave = 16;                    // the MFMA's M
constexpr int kWavesM = 4;                          // waves per workgroup
constexpr int kThreadsM = kWavesM * kWave;
constexpr int kRowsPerWg = kRowsPerWave * kWavesM;  // 64: inside one 128-row tile
constexpr int kMT = 8;                              // activation rows per workgroup
constexpr int kStep = 256;                          // columns per step
constexpr int kRelayPitch = kStep + 32;             // bytes per relay row
constexpr int kRelayBytes = kRowsPerWave * kRelayPitch;
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset past every resource used here
constexpr int kMaxInFM = 8192;              // LDS holds 8 staged rows up to this width

// Columns covered by the step loop (whole groups of U steps).
__host__ __device__ constexpr int padded_cols(int in_f, int U) {
  return (in_f + U * kStep - 1) / (U * kStep) * (U * kStep);
}
// LDS layout: 8 activation rows (int8, pitch padded_cols + 32), then 8 rows of block scales
// (f32, pitch padded_cols / 32 + 1), then one relay per wave, then a 16-byte sink that takes
// the staging stores of threads with nothing to stage (so that staging has no branches, which
// would let the compiler wait for the weight loads before staging).
__host__ __device__ constexpr int act_pitch(int in_f, int U) { return padded_cols(in_f, U) + 32; }
__host__ __device__ constexpr int scale_pitch(int in_f, int U) { return padded_cols(in_f, U) / 32 + 1; }
__host__ __device__ constexpr size_t mfma_lds_bytes(int in_f, int U) {
  return (size_t)kMT * act_pitch(in_f, U) + (size_t)kMT * scale_pitch(in_f, U) * 4 +
         (size_t)kWavesM * kRelayBytes + 16;
}

template <int U_, int WPE_>
struct MCfg {
  static constexpr int U = U_, WPE = WPE_;
};

// 8 e4m3 bytes -> 8 f16 (exact).
__device__ __forceinline__ half8_t decode8(int2_t w) {
  half8_t h;
  const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false);
  const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true);
  const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false);
  const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true);
  h[0] = a[0]; h[1] = a[1]; h[2] = b[0]; h[3] = b[1];
  h[4] = c[0]; h[5] = c[1]; h[6] = d[0]; h[7] = d[1];
  return h;
}

// 8 staged activation bytes u = q ^ 0x80 -> 8 f16 q (exact): the f16 with bits 0x6400 | u is
// 1024 + u, and 1024 + u - 1152 = q.
__device__ __forceinline__ half8_t act8(int2_t u) {
  const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  half8_t h;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    // bytes {u0, 0x64, u1, 0x64} and {u2, 0x64, u3, 0x64}
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, (uint32_t)u[i], 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, (uint32_t)u[i], 0x04030402u);
    const half2_t a = __builtin_bit_cast(half2_t, lo) - off;
    const half2_t b = __builtin_bit_cast(half2_t, hi) - off;
    h[4 * i] = a[0]; h[4 * i + 1] = a[1]; h[4 * i + 2] = b[0]; h[4 * i + 3] = b[1];
  }
  return h;
}

// The wave's LDS traffic between relay writes and fragment reads crosses lanes: keep the
// compiler from moving LDS accesses across this point (LDS operations of one wave execute in
// order, so no wait is needed).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <bool BLK, class C>
__global__ __launch_bounds__(kThreadsM) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_e4m3_mfma(const uint8_t *__restrict__ W, int64_t row_bytes, float scale,
                      const float *__restrict__ grid, int grid_cols,
                      const int8_t *__restrict__ qs, const float *__restrict__ d,
                      float *__restrict__ y, int m, int in_f, int out_f) {
  constexpr int U = C::U;
  extern __shared__ __align__(16) unsigned char lds[];
  const int P = act_pitch(in_f, U), SP = scale_pitch(in_f, U);
  unsigned char *act = lds;
  float *dsc = reinterpret_cast<float *>(lds + (size_t)kMT * P);
  unsigned char *relay = lds + (size_t)kMT * P + (size_t)kMT * SP * 4;
  unsigned char *sink = relay + kWavesM * kRelayBytes;

  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int t0 = blockIdx.y * kMT;
  const int rwg = blockIdx.x * kRowsPerWg;  // first weight row of the workgroup
  const int r0 = rwg + wave * kRowsPerWave;  // first weight row of this wave
  const int nb = in_f / 32;
  const int nsteps_pad = padded_cols(in_f, U) / kStep;

  // 1. the staging loads (oldest): activation row r's 16-byte chunks c = tid + 256 n, and
  // the block scales b = tid and tid + 256; rows past m read as zeros.
  constexpr int NC = kMaxInFM / (kThreadsM * 16);  // chunks per row per thread
  int4_t aq[kMT][NC];
  float dv[kMT][2];
#pragma unroll
  for (int r = 0; r < kMT; ++r) {
    const bool tok = t0 + r < m;
    const rsrc_t qrs = buf_rsrc(qs + (int64_t)(tok ? t0 + r : 0) * in_f, tok ? (uint32_t)in_f : 0u);
    const rsrc_t drs = buf_rsrc(d + (int64_t)(tok ? t0 + r : 0) * nb, tok ? (uint32_t)nb * 4 : 0u);
#pragma unroll
    for (int n = 0; n < NC; ++n) aq[r][n] = buf_load16(qrs, (uint32_t)(threadIdx.x + n * kThreadsM) * 16);
#pragma unroll
    for (int n = 0; n < 2; ++n) dv[r][n] = buf_load_f32(drs, (uint32_t)(threadIdx.x + n * kThreadsM) * 4);
  }
  float gv[2] = {1.0f, 1.0f};
  if (BLK) {
    // the grid row of the workgroup's tile (clamped, so a workgroup past out_f reads inside)
    const int grow = (rwg < out_f ? rwg : out_f - 1) / 128;
    const rsrc_t grs = buf_rsrc(grid + (int64_t)grow * grid_cols, (uint32_t)grid_cols * 4);
#pragma unroll
    for (int n = 0; n < 2; ++n) gv[n] = buf_load_f32(grs, (uint32_t)((threadIdx.x + n * kThreadsM) / 4) * 4);
  }

  // 2. the first U steps of weights.  The wave's rows [r0, r0 + nrw) form one resource; a
  // lane's offset is its row's offset plus its column, or past the resource where the column
  // is at or past in_f (so no lane ever reads into the next row).
  const int nrw = out_f - r0 < kRowsPerWave ? out_f - r0 : kRowsPerWave;
  const rsrc_t wrs = buf_rsrc(W + (int64_t)(nrw > 0 ? r0 : 0) * row_bytes,
                              nrw > 0 ? (uint32_t)((int64_t)(nrw - 1) * row_bytes + in_f) : 0u);
  const int lrow = lane / 16;          // row within each 4-row load
  const int lcol = (lane % 16) * 16;   // byte within the step
  uint32_t rowoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) rowoff[q] = (uint32_t)((int64_t)(4 * q + lrow) * row_bytes);
  auto load_step = [&](int4_t (&wb)[4], int s) {
    const int col = s * kStep + lcol;
    const bool in = col < in_f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wb[q] = buf_load16_stream(wrs, in ? rowoff[q] + (uint32_t)col : kPastEnd);
  };
  int4_t wv[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) load_step(wv[u], u);

  // 3. stage (waits only for the staging loads, which are older than the weight loads).
#pragma unroll
  for (int r = 0; r < kMT; ++r) {
#pragma unroll
    for (int n = 0; n < NC; ++n) {
      const int col = (threadIdx.x + n * kThreadsM) * 16;
      int4_t u = aq[r][n];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] ^= (int)0x80808080u;
      unsigned char *dst = col + 16 <= P ? act + r * P + col : sink;
      *reinterpret_cast<int4_t *>(dst) = u;
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int b = threadIdx.x + n * kThreadsM;
      float *dst = b < SP ? dsc + r * SP + b : reinterpret_cast<float *>(sink);
      *dst = BLK ? dv[r][n] * gv[n] : dv[r][n];
    }
  }
  __syncthreads();

  // 4. stream: per step, relay the 4 loads through LDS, then 8 MFMAs (one per 32-column
  // block), each result scaled per activation row and accumulated.
  unsigned char *rl = relay + wave * kRelayBytes;
  const int fi = lane % 16, fg = lane / 16;  // fragment row (A) / column (B), k-group
  const unsigned char *arow = rl + fi * kRelayPitch + 8 * fg;
  const unsigned char *brow = act + (fi % kMT) * P + 8 * fg;
  const float *srow = dsc + (fi % kMT) * SP;
  float4_t acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const int4_t (&wb)[4], int s) {
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<int4_t *>(rl + (4 * q + lrow) * kRelayPitch + lcol) = wb[q];
    wave_lds_fence();
    // all of the step's fragments first, so that one LDS latency covers the 8 MFMAs
    constexpr int KB = kStep / 32;
    int2_t wa[KB], xb[KB];
    float sc[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      wa[k] = *reinterpret_cast<const int2_t *>(arow + 32 * k);
      xb[k] = *reinterpret_cast<const int2_t *>(brow + s * kStep + 32 * k);
      sc[k] = srow[s * KB + k];
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float4_t zero = {0.f, 0.f, 0.f, 0.f};
      const float4_t dk =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(wa[k]), act8(xb[k]), zero, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[k % 4][v] = fmaf(dk[v], sc[k], acc[k % 4][v]);
    }
  };
  for (int s0 = 0; s0 < nsteps_pad; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      step(wv[u], s0 + u);
      load_step(wv[u], s0 + u + U);  // past the padded range: past the resource
    }
  }

  // 5. lane (g, j) holds D rows 4g..4g+3 of activation column j.
  const int t = t0 + fi;
  if (fi < kMT && t < m) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + 4 * fg + v;
      const float s = (acc[0][v] + acc[1][v]) + (acc[2][v] + acc[3][v]);
      if (row < out_f) y[(int64_t)t * out_f + row] = BLK ? s : s * scale;
    }
  }
}

template <bool BLK, class C>
hipError_t launch_m(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                    int grid_cols, const int8_t *qs, const float *d, float *y, int m, int in_f,
                    int out_f, hipStream_t s) {
  auto kern = k_gemv_e4m3_mfma<BLK, C>;
  static std::atomic<bool> lds_set[kMaxDevices];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void *>(kern),
                                          mfma_lds_bytes(kMaxInFM, C::U), lds_set);
  if (e != hipSuccess) return e;
  const dim3 g((out_f + kRowsPerWg - 1) / kRowsPerWg, (m + kMT - 1) / kMT);
  hipLaunchKernelGGL(kern, g, dim3(kThreadsM), mfma_lds_bytes(in_f, C::U), s, W, row_bytes,
                     scale, grid, grid_cols, qs, d, y, m, in_f, out_f);
  return hipGetLastError();
}

using MCfgDefault = MCfg<4, 2>;
static_assert(mfma_lds_bytes(kMaxInFM, MCfgDefault::U) <= 160 * 1024, "LDS of one workgroup");
static_assert(kMaxInFM % (kThreadsM * 16) == 0 && kMaxInFM / 32 <= 2 * kThreadsM - 1,
              "staging covers every activation chunk and block scale");

}  // namespace

bool gemv_e4m3_mfma_applies(int64_t row_bytes, int m, int in_f) {
  // offsets of the wave's 16 rows stay below the past-the-end offset
  return m >= 5 && in_f <= kMaxInFM && row_bytes <= ((int64_t)1 << 26);
}

hipError_t launch_gemv_e4m3_mfma(const uint8_t *W, int64_t row_bytes, float scale,
                                 const float *grid, int grid_cols, bool blk128, const int8_t *qs,
                                 const float *d, float *y, int m, int in_f, int out_f,
                                 hipStream_t s) {
  if (blk128)
    return launch_m<true, MCfgDefault>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f,
                                       out_f, s);
  return launch_m<false, MCfgDefault>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f,
                                      out_f, s);
}

LaunchDesc describe_gemv_e4m3_mfma(bool blk128, int m, int in_f, int out_f) {
  LaunchDesc r;
  r.grid_x = (unsigned)((out_f + kRowsPerWg - 1) / kRowsPerWg);
  r.grid_y = (unsigned)((m + kMT - 1) / kMT);
  r.threads = kThreadsM;
  r.lds = (unsigned)mfma_lds_bytes(in_f, MCfgDefault::U);
  r.kernel = blk128 ? "k_gemv_e4m3_mfma<true" : "k_gemv_e4m3_mfma<false";
  static const std::string text = [] {
    char b[64];
    snprintf(b, sizeof b, "MCfg<%d, %d>", MCfgDefault::U, MCfgDefault::WPE);
    return std::string(b);
  }();
  r.config = text.c_str();
  return r;
}

}  // namespace fp8gemv

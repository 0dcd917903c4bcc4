// Several activation rows at once over raw OCP e4m3 weights (per-tensor or block-128 scaled),
// on the matrix cores.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc sections THE
// COMPARISON and THE BLOCK-128 ARM: the contraction of the m = 1 GEMV (e4m3 weight rows,
// row_bytes == in_f, times a q8_1 activation row), here for a few activation rows, which
// makes it a skinny product Y[m, out_f] = X[m, in_f] * W^T.
//
// Why the matrix cores: with m activation rows the vector path spends, per weight pair, one
// decode and m dot-2 instructions, and from m = 4 on that is more than the SIMDs issue while
// the weights stream at the HBM rate (17408 x 5120: 22 us at m = 4 and 45 us at m = 8 on the
// vector path).  v_mfma_f32_16x16x32_f16 does 16 x 16 x 32 products in one instruction, so
// the cost no longer grows with m: 21 us for any m from 3 to 8 at that shape, which is why
// this kernel takes m >= 4.
//
// gfx950 design:
//   * Each wave owns 16 consecutive weight rows (the MFMA's M dimension) and a contiguous
//     share of their columns: KS waves share a row group, and their partial sums meet in LDS
//     and are added in part order.  A workgroup is 4 waves, so it owns 64 / KS rows, which
//     always lie in one 128-row tile of the block-128 grid.  Up to 8 activation rows per
//     workgroup (grid.y = ceil(m / 8)) are the MFMA's N columns 0..7; columns 8..15 read past
//     the activation buffer (zeros) and are never stored.
//   * Weights stream in steps of 1024 / R columns: one wave-wide 16-byte non-temporal buffer
//     load covers R rows x 1024 / R contiguous bytes, so 16 / R loads cover the wave's 16
//     rows, and every weight byte is fetched once.  Past in_f, past the wave's share or past
//     out_f a lane's offset lies outside the buffer resource and the load returns zeros
//     without touching memory.
//   * Each step goes through a per-wave LDS relay (16 rows, pitch chosen so that the
//     fragment reads below are conflict-free) and comes back as MFMA A fragments: lane
//     (i, g) = (lane % 16, lane / 16) reads 8 bytes of row i at column 32k + 8g for the step's
//     k-th 32-column block.  v_cvt_scalef32_pk_f16_fp8 with scale 1.0 decodes them to f16
//     exactly (every e4m3 value, subnormals included, is an f16 normal).
//   * The activation comes straight from the q8_1 rows (L2-resident): per step each wave
//     loads its 8 activation rows' 256 bytes (two 16-byte loads per lane) and the 64 block
//     scales (times the grid values for block-128) together with the step's weights, U steps
//     ahead, so the in-order load counter never makes a step wait for loads issued after its
//     own.  They go through a second small per-wave relay, from which lane (j, g) reads the B
//     fragment: 8 values of activation row j at the A fragment's columns (rows j >= 8 repeat
//     j - 8).  They are stored as q ^ 0x80; a byte permute against 0x64 gives the f16
//     1024 + (q ^ 0x80), and one packed subtraction of 1152 leaves q, exactly.  Nothing is
//     staged per workgroup, so a workgroup needs only its waves' relays and many small
//     workgroups fit a CU.
//   * One MFMA covers 32 columns, exactly one q8_1 block and a quarter of a 128-column tile,
//     so its 16 x 16 result is scaled per activation row by that block's scale (times the grid
//     value for block-128).
// Numerics: each product (4 + 8 significant bits) is exact in f16 x f16; the MFMA sums a
// block's 32 products in f32; acc += D * scale with one fma, into one of 4 accumulators by
// block index mod 4; the 4 are added in a fixed order, then the KS parts in part order.
// Deterministic (no atomics, every order fixed), and each output depends only on its own
// weight row and activation row, whatever m and the row's position in the call.  The rounding
// differs from the vector path's, so an m-row call on this path is not bit-identical to
// m = 1; both are within the parity tolerance of the exact result.
#include "common.hpp"

namespace fp8gemv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef int int2_t __attribute__((ext_vector_type(2)));

constexpr int kRowsPerWave = 16;                    // the MFMA's M
constexpr int kMT = 8;                              // activation rows per workgroup
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset past every resource used here

// A step is 16 rows x step_cols(R) columns, loaded R rows per wave-wide load.
__host__ __device__ constexpr int step_cols(int R) { return 1024 / R; }
// relay row pitch: a row starts 4 banks after the previous one, so the 16 rows' 32-byte
// fragment reads cover every bank exactly twice (the two passes a 512-byte read needs anyway)
__host__ __device__ constexpr int relay_pitch(int R) { return step_cols(R) + 16; }
// per wave: 16 weight rows, 8 activation rows, 8 x (step_cols / 32) scales
__host__ __device__ constexpr int relay_bytes(int R) {
  return (kRowsPerWave + kMT) * relay_pitch(R) + kMT * (step_cols(R) / 32) * 4;
}

// U steps in flight, WPE waves per SIMD, R rows per load, KS waves per 16-row group, WAVES
// waves per workgroup.
template <int U_, int WPE_, int R_, int KS_, int WAVES_>
struct MCfg {
  static constexpr int U = U_, WPE = WPE_, R = R_, KS = KS_, WAVES = WAVES_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int ROWS = kRowsPerWave * WAVES / KS;  // rows per workgroup
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

// 8 activation bytes u = q ^ 0x80 -> 8 f16 q (exact): the f16 with bits 0x6400 | u is
// 1024 + u, and 1024 + u - 1152 = q.
__device__ __forceinline__ half8_t act8(int2_t uu) {
  const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  half8_t h;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t u = (uint32_t)uu[i];
    // bytes {u0, 0x64, u1, 0x64} and {u2, 0x64, u3, 0x64}
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
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
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_e4m3_mfma(const uint8_t *__restrict__ W, int64_t row_bytes, float scale,
                      const float *__restrict__ grid, int grid_cols,
                      const int8_t *__restrict__ qs, const float *__restrict__ d,
                      float *__restrict__ y, int m, int in_f, int out_f) {
  constexpr int U = C::U, R = C::R, KS = C::KS;
  constexpr int SC = step_cols(R), NQ = kRowsPerWave / R, RP = relay_pitch(R), KB = SC / 32;
  static_assert(128 % C::ROWS == 0, "a workgroup's rows lie in one 128-row tile");
  static_assert(C::WAVES % KS == 0, "a workgroup holds whole row groups");
  static_assert(KB % 4 == 0, "a step covers whole 128-column tiles");
  __shared__ __align__(16) unsigned char relay[C::WAVES * relay_bytes(R)];

  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int t0 = blockIdx.y * kMT;
  const int nt = m - t0 < kMT ? m - t0 : kMT;  // activation rows of this workgroup (>= 1)
  const int rwg = blockIdx.x * C::ROWS;        // first weight row of the workgroup
  const int part = wave % KS;                  // this wave's share of the row group's steps
  const int r0 = rwg + (wave / KS) * kRowsPerWave;  // first weight row of this wave
  const int nb = in_f / 32;
  const int nsteps = (in_f + SC - 1) / SC;
  const int nmine = ((nsteps + KS - 1) / KS + U - 1) / U * U;  // whole groups of U steps
  const int sbeg = part * nmine;
  // columns past this wave's share (or past in_f) are never loaded
  const int cend = (sbeg + nmine) * SC < in_f ? (sbeg + nmine) * SC : in_f;

  // Weights: the wave's rows [r0, r0 + nrw) form one resource; a lane's offset is its row's
  // offset plus its column, or past the resource where the column is at or past cend (so no
  // lane ever reads into the next row).
  const int nrw = out_f - r0 < kRowsPerWave ? out_f - r0 : kRowsPerWave;
  const rsrc_t wrs = buf_rsrc(W + (int64_t)(nrw > 0 ? r0 : 0) * row_bytes,
                              nrw > 0 ? (uint32_t)((int64_t)(nrw - 1) * row_bytes + in_f) : 0u);
  const int lrow = lane / (kWave / R);          // row within each R-row load
  const int lcol = (lane % (kWave / R)) * 16;   // byte within the step
  uint32_t rowoff[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) rowoff[q] = (uint32_t)((int64_t)(R * q + lrow) * row_bytes);
  // Activation rows [t0, t0 + nt) and their scales; lane (j, g) reads row j (rows past nt,
  // and so the MFMA columns 8..15, read zeros).  A column past in_f reads the next row's
  // values (finite) against zero weights, or zeros after the last row.
  const int fi = lane % 16, fg = lane / 16;  // fragment row (A) / column (B), k-group
  const rsrc_t qrs = buf_rsrc(qs + (int64_t)t0 * in_f, (uint32_t)(nt * in_f));
  const rsrc_t drs = buf_rsrc(d + (int64_t)t0 * nb, (uint32_t)(nt * nb * 4));
  // lane l loads 32 bytes of activation row l / 8 at step column 32 (l % 8), and the scale
  // of that row's block l % 8 of the step
  constexpr int SPL = SC / 32 / (kWave / kMT) ;  // 32-byte pieces per lane per step (1 for R=4)
  static_assert(SC == 256, "one 32-byte activation piece per lane per step");
  const int arw = lane / kMT, apc = lane % kMT;
  const uint32_t qoff = (uint32_t)(arw * in_f + 32 * apc), doff = (uint32_t)(arw * nb + apc);
  (void)SPL;
  rsrc_t grs = buf_rsrc(grid, 0u);
  if (BLK) {
    // the grid row of the workgroup's tile (clamped, so a workgroup past out_f reads inside)
    const int grow = (rwg < out_f ? rwg : out_f - 1) / 128;
    grs = buf_rsrc(grid + (int64_t)grow * grid_cols, (uint32_t)grid_cols * 4);
  }

  struct Step {
    int4_t w[NQ];
    int4_t a[2];  // 32 activation bytes
    float sc;     // one block scale (times the grid value)
    float gv;
  };
  auto load_step = [&](Step &st, int s) {
    const int col = s * SC + lcol;
    const bool in = col < cend;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      st.w[q] = buf_load16_stream(wrs, in ? rowoff[q] + (uint32_t)col : kPastEnd);
    // this lane's block of the step; a block at or past cend reads zeros and no scale
    const int cblk = s * SC + 32 * apc;
    const bool ain = cblk < cend;
    st.a[0] = buf_load16(qrs, ain ? qoff + (uint32_t)(s * SC) : kPastEnd);
    st.a[1] = buf_load16(qrs, ain ? qoff + (uint32_t)(s * SC) + 16 : kPastEnd);
    st.sc = buf_load_f32(drs, ain ? (doff + (uint32_t)(s * KB)) * 4 : kPastEnd);
    if (BLK) st.gv = buf_load_f32(grs, ain ? (uint32_t)(cblk / 128) * 4 : kPastEnd);
  };
  Step sd[U];
#pragma unroll
  for (int u = 0; u < U; ++u) load_step(sd[u], sbeg + u);

  // Per step: relay the weight loads through LDS, then one MFMA per 32-column block, its
  // result scaled per activation row and accumulated.
  unsigned char *rl = relay + wave * relay_bytes(R);  // weights: 16 rows of pitch RP
  unsigned char *rb = rl + kRowsPerWave * RP;          // activation: 8 rows of pitch RP
  float *rs = reinterpret_cast<float *>(rb + kMT * RP);  // scales: [8][KB]
  const unsigned char *arow = rl + fi * RP + 8 * fg;
  const unsigned char *brow = rb + (fi % kMT) * RP + 8 * fg;
  const float *srow = rs + (fi % kMT) * KB;
  float4_t acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const Step &st) {
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      *reinterpret_cast<int4_t *>(rl + (R * q + lrow) * RP + lcol) = st.w[q];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int4_t u = st.a[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] ^= (int)0x80808080u;
      *reinterpret_cast<int4_t *>(rb + arw * RP + 32 * apc + 16 * h) = u;
    }
    rs[arw * KB + apc] = BLK ? st.sc * st.gv : st.sc;
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int2_t wa = *reinterpret_cast<const int2_t *>(arow + 32 * k);
      const int2_t xb = *reinterpret_cast<const int2_t *>(brow + 32 * k);
      const float sc = srow[k];
      const float4_t zero = {0.f, 0.f, 0.f, 0.f};
      const float4_t dk =
          __builtin_amdgcn_mfma_f32_16x16x32_f16(decode8(wa), act8(xb), zero, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[k % 4][v] = fmaf(dk[v], sc, acc[k % 4][v]);
    }
  };
  for (int s0 = sbeg; s0 < sbeg + nmine; s0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      step(sd[u]);
      load_step(sd[u], s0 + u + U);  // past this wave's share: past every resource
    }
  }

  // Lane (g, j) holds D rows 4g..4g+3 of activation column j.
  float4_t tot;
#pragma unroll
  for (int v = 0; v < 4; ++v) tot[v] = (acc[0][v] + acc[1][v]) + (acc[2][v] + acc[3][v]);
  if constexpr (KS > 1) {
    // the parts of a row group meet in their relays (no longer needed), added in part order
    wave_lds_fence();
    *reinterpret_cast<float4_t *>(rl + lane * 16) = tot;
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int p = 1; p < KS; ++p)
        tot += *reinterpret_cast<const float4_t *>(rl + p * relay_bytes(R) + lane * 16);
    }
  }
  const int t = t0 + fi;
  if (part == 0 && fi < kMT && t < m) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + 4 * fg + v;
      if (row < out_f) y[(int64_t)t * out_f + row] = BLK ? tot[v] : tot[v] * scale;
    }
  }
}

template <bool BLK, class C>
hipError_t launch_m(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                    int grid_cols, const int8_t *qs, const float *d, float *y, int m, int in_f,
                    int out_f, hipStream_t s) {
  const dim3 g((out_f + C::ROWS - 1) / C::ROWS, (m + kMT - 1) / kMT);
  hipLaunchKernelGGL((k_gemv_e4m3_mfma<BLK, C>), g, dim3(C::THREADS), 0, s, W, row_bytes, scale,
                     grid, grid_cols, qs, d, y, m, in_f, out_f);
  return hipGetLastError();
}

// Measured at 17408 x 5120 and 5120 x 17408 (m = 4 and 8): one step in flight, 4 waves per
// row group; rows of more than 8192 columns split 8 ways in 8-wave workgroups, so that the
// few long rows still give enough waves.
using MCfgSmall = MCfg<1, 6, 4, 4, 4>;  // in_f <= 8192
using MCfgLong = MCfg<1, 6, 4, 8, 8>;   // in_f > 8192

template <class F>
auto with_mcfg(int in_f, F &&f) {
  return in_f <= 8192 ? f(Tag<MCfgSmall>{}) : f(Tag<MCfgLong>{});
}

}  // namespace

bool gemv_e4m3_mfma_applies(int64_t row_bytes, int in_f) {
  (void)in_f;
  // offsets of the wave's 16 rows stay below the past-the-end offset
  return row_bytes <= ((int64_t)1 << 26);
}

hipError_t launch_gemv_e4m3_mfma(const uint8_t *W, int64_t row_bytes, float scale,
                                 const float *grid, int grid_cols, bool blk128, const int8_t *qs,
                                 const float *d, float *y, int m, int in_f, int out_f,
                                 hipStream_t s) {
  return with_mcfg(in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    if (blk128)
      return launch_m<true, C>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
    return launch_m<false, C>(W, row_bytes, scale, grid, grid_cols, qs, d, y, m, in_f, out_f, s);
  });
}

LaunchDesc describe_gemv_e4m3_mfma(bool blk128, int m, int in_f, int out_f) {
  return with_mcfg(in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    LaunchDesc r;
    r.grid_x = (unsigned)((out_f + C::ROWS - 1) / C::ROWS);
    r.grid_y = (unsigned)((m + kMT - 1) / kMT);
    r.threads = C::THREADS;
    r.lds = 0;  // static: the relays only
    r.kernel = blk128 ? "k_gemv_e4m3_mfma<true" : "k_gemv_e4m3_mfma<false";
    static const std::string text = [] {
      char b[64];
      snprintf(b, sizeof b, "MCfg<%d, %d, %d, %d, %d>", C::U, C::WPE, C::R, C::KS, C::WAVES);
      return std::string(b);
    }();
    r.config = text.c_str();
    return r;
  });
}

}  // namespace fp8gemv

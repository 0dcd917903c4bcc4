// Several activation rows at once over ggml Q8_0 weight rows, on the matrix cores.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc sections
// QUESTION and THE COMPARISON (arm Q8_0: 34 bytes per 32 weights, an fp16 scale then 32
// int8) and `synth_q8_0`: the contraction of the m = 1 Q8_0 GEMV, here for a few activation
// rows, which makes it a skinny product Y[m, out_f] = X[m, in_f] * W^T.
//
// y[t, r] = sum_b fp16(scale[r, b]) * d_a[t, b] * sum_{i<32} qw[r, b, i] * qs[t, 32b + i]
//
// Why the matrix cores: per weight chunk the vector path spends the integer dot products and
// the scaling once per activation row, so its cost grows with m (17408 x 5120: 16.7 us at
// m = 1, 29.6 at m = 4, 49 at m = 8).  v_mfma_i32_16x16x32_i8 forms a block's 16 x 16 exact
// integer sums in one instruction.
//
// gfx950 design (the same frame as the e4m3 matrix-core kernel):
//   * Each wave owns 16 consecutive weight rows (the MFMA's M) and a share of their columns:
//     KS waves share a row group, taking its column steps in turn (wave p: steps p, p + KS,
//     ..), so the KS waves read adjacent pieces of the same rows at about the same time and a
//     128-byte line cut between two steps is still in L2 for the second one (with contiguous
//     shares per wave, 23% more bytes came from memory than the plane holds; interleaved, 11%).
//     Their partial sums meet in LDS and are added in part order.  Up to 8 activation rows
//     per workgroup (grid.y = ceil(m / 8)) are the MFMA's N columns 0..7; columns 8..15
//     repeat them and are never stored.
//   * Weights stream in steps of one group (8 blocks = 272 bytes = 17 chunks of 16 bytes) of
//     each of the 16 rows: chunk index 64q + lane of the 16 x 17 is loaded by lane `lane` of
//     load q (5 loads, the last with 16 lanes), so 17 consecutive lanes read 272 contiguous
//     bytes of one row and every weight byte is fetched once.  Past the wave's share or past
//     out_f an offset lies outside the buffer resource and the load returns zeros.
//   * The chunks go to a per-wave LDS relay in row order (pitch 272: a row starts 4 banks
//     after the previous one).  The A fragment of block k is read straight from the raw rows:
//     lane (i, g) takes 8 quants of row i at byte 34k + 2 + 8g (aligned reads, below).  A
//     group's block k has its fp16 scale at byte 2k of chunk 2k, so the lanes that
//     load chunks 0, 2, .., 14 also convert that scale to f32 and write it to a [block][row]
//     table next to the relay (which dword and which half are fixed per lane); a lane then
//     reads the 4 scales of its output rows with one 16-byte LDS read.  Block k's quants start
//     4-byte aligned for odd k and 2 bytes past a dword for even k, so the fragment is read as
//     two aligned dwords, or as three funnel-shifted by 2 bytes: a 2-byte-aligned 8-byte LDS
//     read is legal here but cost about a fifth of the kernel's time at 5120 x 17408.
//   * The activation rows come straight from the q8_1 rows, as in the e4m3 kernel: per step
//     two 16-byte loads per lane cover 8 rows x 256 columns, plus one block scale per lane,
//     issued together with the step's weights, through a second small relay.  The int8 values
//     are the MFMA's B operand as they are.
//   * Scaling: acc += float(isum) * (fp16(scale) * d_a), one product and one fma per output,
//     into one of 4 accumulators by block index mod 4; the 4 are added in a fixed order, then
//     the KS parts in part order.
// Numerics: each block's integer sum is exact (MFMA int32), as in the vector path; the float
// operations around it are in a different (fixed) order, so an m-row call on this path is
// not bit-identical to m = 1, and each output depends only on its own weight row and
// activation row, whatever m and the row's position in the call.
#include "common.hpp"

namespace fp8gemv {
namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 16;  // the MFMA's M
constexpr int kMT = 8;            // activation rows per workgroup
constexpr int kGrpBlocks = 8;     // blocks per step
constexpr int kGrpBytes = 272;    // bytes of one row per step
constexpr int kGrpChunks = 17;
constexpr int kStepCols = 256;
constexpr int kLoads = (kRowsPerWave * kGrpChunks + kWave - 1) / kWave;  // 5
constexpr uint32_t kPastEnd = 0x80000000u;
// per-wave LDS: weight relay, activation relay, activation scales, weight scales
constexpr int kAPitch = kGrpBytes;
constexpr int kBPitch = kStepCols + 16;
constexpr int kRelayA = kRowsPerWave * kAPitch;
constexpr int kRelayB = kMT * kBPitch;
constexpr int kRelayD = kMT * kGrpBlocks * 4;
constexpr int kRelayW = kGrpBlocks * kRowsPerWave * 4;
constexpr int kRelaySink = 16;  // takes the writes of lanes with nothing to write
constexpr int kRelayBytes = kRelayA + kRelayB + kRelayD + kRelayW + kRelaySink;
static_assert(kRelayA % 16 == 0 && kRelayB % 16 == 0 && kRelayD % 16 == 0 &&
                  kRelayBytes % 16 == 0, "16-byte aligned relay parts");

// WPE waves per SIMD, KS waves per 16-row group, WAVES waves per workgroup.
template <int WPE_, int KS_, int WAVES_>
struct QMCfg {
  static constexpr int WPE = WPE_, KS = KS_, WAVES = WAVES_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int ROWS = kRowsPerWave * WAVES / KS;  // rows per workgroup
};

// The wave's LDS traffic between relay writes and reads crosses lanes: keep the compiler from
// moving LDS accesses across this point (LDS operations of one wave execute in order, so no
// wait is needed).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_q8_0_mfma(const uint8_t *__restrict__ W, int64_t row_bytes,
                      const int8_t *__restrict__ qs, const float *__restrict__ d,
                      float *__restrict__ y, int m, int in_f, int out_f) {
  constexpr int KS = C::KS;
  static_assert(C::WAVES % KS == 0, "a workgroup holds whole row groups");
  __shared__ __align__(16) unsigned char relay[C::WAVES * kRelayBytes];

  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int t0 = blockIdx.y * kMT;
  const int nt = m - t0 < kMT ? m - t0 : kMT;  // activation rows of this workgroup (>= 1)
  const int part = wave % KS;                  // this wave's share of the row group's steps
  const int r0 = blockIdx.x * C::ROWS + (wave / KS) * kRowsPerWave;  // first weight row
  const int nb = in_f / 32;
  const int ngrp = in_f / kStepCols;  // in_f % 256 == 0 on this path
  const int nmine = (ngrp + KS - 1) / KS;  // steps part, part + KS, part + 2 KS, ..

  // Weights: the wave's rows [r0, r0 + nrw) form one resource over their blocks.
  const int nrw = out_f - r0 < kRowsPerWave ? out_f - r0 : kRowsPerWave;
  const rsrc_t wrs = buf_rsrc(
      W + (int64_t)(nrw > 0 ? r0 : 0) * row_bytes,
      nrw > 0 ? (uint32_t)((int64_t)(nrw - 1) * row_bytes + (int64_t)nb * 34) : 0u);
  unsigned char *rl = relay + wave * kRelayBytes;    // weights: 16 rows of kAPitch
  unsigned char *rb = rl + kRelayA;                  // activation: 8 rows of kBPitch
  float *rd = reinterpret_cast<float *>(rb + kRelayB);  // activation scales [8][8]
  float *rw = rd + kMT * kGrpBlocks;                    // weight scales [8 blocks][16 rows]
  // load q, lane l: chunk c = 64q + l of the step's 16 x 17 (row-major), written to the
  // relay at 16c (the pitch is 17 chunks).  Lanes past the 272 chunks load nothing; their
  // writes land in the activation relay, which is written after them.  A lane whose chunk is
  // 2k (k < 8) holds the fp16 scale of block k at byte 2k (quadword k / 4, bit 16 (k % 4));
  // it writes that scale as f32 to the table, the others write to the sink.
  constexpr uint32_t kSink = kRelayA + kRelayB + kRelayD + kRelayW;
  static_assert(kAPitch == kGrpChunks * 16, "relay offset of chunk c is 16 c");
  uint32_t woff[kLoads], soff[kLoads], sbit[kLoads];
  bool shi[kLoads];
#pragma unroll
  for (int q = 0; q < kLoads; ++q) {
    const int c = kWave * q + lane;
    const bool ok = c < kRowsPerWave * kGrpChunks;
    const int row = c / kGrpChunks, ch = c % kGrpChunks;
    woff[q] = ok ? (uint32_t)((int64_t)row * row_bytes + 16 * ch) : kPastEnd;
    const bool sc = ok && ch % 2 == 0 && ch < 2 * kGrpBlocks;
    const int k = ch / 2;
    soff[q] = sc ? (uint32_t)(kRelayA + kRelayB + kRelayD + (k * kRowsPerWave + row) * 4) : kSink;
    sbit[q] = 16u * (uint32_t)(k % 4);
    shi[q] = k >= 4;
  }
  // Activation rows [t0, t0 + nt): lane l loads 32 bytes of row l / 8 at step column
  // 32 (l % 8) and the scale of that block; rows past nt read zeros.
  const rsrc_t qrs = buf_rsrc(qs + (int64_t)t0 * in_f, (uint32_t)(nt * in_f));
  const rsrc_t drs = buf_rsrc(d + (int64_t)t0 * nb, (uint32_t)(nt * nb * 4));
  const int arw = lane / kMT, apc = lane % kMT;
  const uint32_t qoff = (uint32_t)(arw * in_f + 32 * apc), doff = (uint32_t)(arw * nb + apc);

  struct Step {
    int4_t w[kLoads];
    int4_t a[2];
    float sc;
  };
  auto load_step = [&](Step &st, int s) {
    const bool in = s < ngrp;  // past the row: past every resource
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
      st.w[q] = buf_load16_stream(wrs, in && woff[q] != kPastEnd ? woff[q] + (uint32_t)(kGrpBytes * s) : kPastEnd);
    st.a[0] = buf_load16(qrs, in ? qoff + (uint32_t)(kStepCols * s) : kPastEnd);
    st.a[1] = buf_load16(qrs, in ? qoff + (uint32_t)(kStepCols * s) + 16 : kPastEnd);
    st.sc = buf_load_f32(drs, in ? (doff + (uint32_t)(kGrpBlocks * s)) * 4 : kPastEnd);
  };
  Step st;
  load_step(st, part);

  const int fi = lane % 16, fg = lane / 16;  // fragment row (A) / column (B), k-group
  const unsigned char *arow = rl + fi * kAPitch + 8 * fg;  // 8-byte aligned
  const unsigned char *brow = rb + (fi % kMT) * kBPitch + 8 * fg;
  const float *drow = rd + (fi % kMT) * kGrpBlocks;
  float4_t acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int s = part; s < part + KS * nmine; s += KS) {
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int4_t w = st.w[q];
      *reinterpret_cast<int4_t *>(rl + 16 * (kWave * q + lane)) = w;
      const uint64_t lo = (uint64_t)(uint32_t)w[0] | ((uint64_t)(uint32_t)w[1] << 32);
      const uint64_t hi = (uint64_t)(uint32_t)w[2] | ((uint64_t)(uint32_t)w[3] << 32);
      const uint16_t h = (uint16_t)((shi[q] ? hi : lo) >> sbit[q]);
      *reinterpret_cast<float *>(rl + soff[q]) = (float)__builtin_bit_cast(_Float16, h);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<int4_t *>(rb + arw * kBPitch + 32 * apc + 16 * h) = st.a[h];
    rd[arw * kGrpBlocks + apc] = st.sc;
    load_step(st, s + KS);
    wave_lds_fence();
#pragma unroll
    for (int k = 0; k < kGrpBlocks; ++k) {
      // Block k's quants start at byte 34k + 2 of the row: 4-byte aligned for odd k, 2 bytes
      // past a dword for even k.  Odd k: two aligned dwords.  Even k: three aligned dwords
      // funnel-shifted by 2 bytes (an unaligned LDS read costs more than the extra dword).
      long wa, xb;
      if (k % 2) {
        const uint32_t *a4 = reinterpret_cast<const uint32_t *>(arow + 34 * k + 2);
        wa = (long)((uint64_t)a4[0] | ((uint64_t)a4[1] << 32));
      } else {
        const uint32_t *a4 = reinterpret_cast<const uint32_t *>(arow + 34 * k);
        const uint32_t d0 = a4[0], d1 = a4[1], d2 = a4[2];
        wa = (long)((uint64_t)__builtin_amdgcn_alignbyte(d1, d0, 2) |
                    ((uint64_t)__builtin_amdgcn_alignbyte(d2, d1, 2) << 32));
      }
      __builtin_memcpy(&xb, brow + 32 * k, 8);
      const float4_t dw = *reinterpret_cast<const float4_t *>(rw + k * kRowsPerWave + 4 * fg);
      const float da = drow[k];
      const int4_t zero = {0, 0, 0, 0};
      const int4_t dk = __builtin_amdgcn_mfma_i32_16x16x32_i8(wa, xb, zero, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[k % 4][v] = fmaf((float)dk[v], dw[v] * da, acc[k % 4][v]);
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
        tot += *reinterpret_cast<const float4_t *>(rl + p * kRelayBytes + lane * 16);
    }
  }
  const int t = t0 + fi;
  if (part == 0 && fi < kMT && t < m) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = r0 + 4 * fg + v;
      if (row < out_f) y[(int64_t)t * out_f + row] = tot[v];
    }
  }
}

// Rows of up to 8192 columns: 4 waves per row group; longer rows split 8 ways in 8-wave
// workgroups, so that the few long rows still give enough waves.
using QMCfgSmall = QMCfg<5, 4, 4>;
using QMCfgLong = QMCfg<5, 8, 8>;

template <class F>
auto with_qmcfg(int in_f, F &&f) {
  return in_f <= 8192 ? f(Tag<QMCfgSmall>{}) : f(Tag<QMCfgLong>{});
}

}  // namespace

bool gemv_q8_0_mfma_applies(const uint8_t *W, int64_t row_bytes, int in_f) {
  // whole groups, 16-byte aligned rows (the chunk loads), and offsets of the wave's 16 rows
  // below the past-the-end offset
  return in_f % 256 == 0 && row_bytes % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(W) & 15) == 0 && row_bytes <= ((int64_t)1 << 26);
}

hipError_t launch_gemv_q8_0_mfma(const uint8_t *W, int64_t row_bytes, const int8_t *qs,
                                 const float *d, float *y, int m, int in_f, int out_f,
                                 hipStream_t s) {
  return with_qmcfg(in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    const dim3 g((out_f + C::ROWS - 1) / C::ROWS, (m + kMT - 1) / kMT);
    hipLaunchKernelGGL((k_gemv_q8_0_mfma<C>), g, dim3(C::THREADS), 0, s, W, row_bytes, qs, d, y,
                       m, in_f, out_f);
    return hipGetLastError();
  });
}

LaunchDesc describe_gemv_q8_0_mfma(int m, int in_f, int out_f) {
  return with_qmcfg(in_f, [&](auto tag) {
    using C = typename decltype(tag)::type;
    LaunchDesc r;
    r.grid_x = (unsigned)((out_f + C::ROWS - 1) / C::ROWS);
    r.grid_y = (unsigned)((m + kMT - 1) / kMT);
    r.threads = C::THREADS;
    r.lds = 0;  // static: the relays only
    r.kernel = "k_gemv_q8_0_mfma";
    static const std::string text = [] {
      char b[64];
      snprintf(b, sizeof b, "QMCfg<%d, %d, %d>", C::WPE, C::KS, C::WAVES);
      return std::string(b);
    }();
    r.config = text.c_str();
    return r;
  });
}

}  // namespace fp8gemv

// m=1 decode GEMV over ggml Q8_0 weight rows against a q8_1 activation.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc sections
// QUESTION and THE COMPARISON (arm Q8_0: 34 bytes per 32 weights, an fp16 scale then 32
// int8, row_bytes = in_f/32*34, the 1.0625 byte/weight floor) and `synth_q8_0` (the scale
// is little-endian at bytes 0..1 of each block).
//
// y[t, r] = sum_b fp16(scale[r, b]) * d_a[t, b] * sum_{i<32} qw[r, b, i] * qs[t, 32b + i]
//
// gfx950 design (the page's kernel is a CUDA warp-per-row MMVQ with dp4a; this one is not a
// translation of it).  The difficulty is that 34-byte blocks do not line up with 16-byte
// loads.  Fast path (in_f % 256 == 0, so every row is 17*in_f/256 whole 16-byte chunks and
// every row starts the block pattern at a chunk boundary):
//   * Lane l of a wave streams chunk 64*win + l of the row with one 16-byte non-temporal
//     load: fully coalesced, every weight byte fetched exactly once.
//   * The activation is staged in LDS "in the shape of a Q8_0 row": 34 bytes per block, two
//     zero bytes where the weight row has its fp16 scale, then the 32 qs.  A weight chunk and
//     the activation chunk at the same offset line up byte for byte, so four v_dot4_i32_i8
//     give the integer products of the chunk, and the scale bytes meet zeros.
//   * No dword mixes quantised bytes of two blocks (block boundaries are 34 bytes apart and
//     the 2-byte scale sits between them), so a chunk's four dwords split into a prefix that
//     belongs to block b0 and a suffix that belongs to b0 + 1; the two exact int32 sums are
//     scaled separately.
//   * A chunk contains at most one block scale.  The lane holding it converts it (fp16 ->
//     f32, times the activation scale d_a[b]).  The scale of a chunk's first block starts 0,
//     1 or 2 chunks earlier -- 0, 1 or 2 lanes to the left -- so it reaches the lanes that
//     need it through one or two wave-wide DPP right shifts; lanes 0 and 1 take lanes 62
//     and 63 of the previous window, carried in scalar registers.  No LDS round trip.
// Generic path (any in_f % 32 == 0): one lane per block, 2-byte loads; correct, not tuned.
// Row t = blockIdx.y of the activation runs identical code, so each activation row of an
// m-row call is bit-identical to an m=1 call on that row.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;  // generic path
constexpr int kWaves = kThreads / kWave;
constexpr int kBlkBytes = 34;

__host__ __device__ constexpr int chunks_per_row(int in_f) { return in_f / 32 * kBlkBytes / 16; }
__host__ __device__ constexpr int windows_per_row(int in_f) {
  return (chunks_per_row(in_f) + kWave - 1) / kWave;
}

// Launch shape of the fast path.  Each thread stages KQ activation blocks and KD block scales:
// KQ * WAVES * 64 >= in_f / 32 and KD * WAVES * 64 >= in_f / 32 + 2.
// DB: double-buffered window loop -- the next U windows are loaded before the current U are
// consumed, so a wave never waits with nothing in flight (rows of many windows).
template <int WAVES_, int RPW_, int U_, int KQ_, int KD_, bool DB_ = false, int WPE_ = 8,
          int SPLIT_ = 1>
struct QCfg {
  static constexpr int WAVES = WAVES_, RPW = RPW_, U = U_, KQ = KQ_, KD = KD_, WPE = WPE_;
  static constexpr int SPLIT = SPLIT_;  // waves sharing one group of RPW rows (split over k)
  static constexpr int ROWS = WAVES / SPLIT * RPW;  // rows per workgroup
  static constexpr bool DB = DB_;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int MAX_IN_F = KQ * THREADS * 32;
};

// LDS layout of the fast path: shaped activation (whole windows of 1 KiB), d_a[nb + 2].
// Last: a 48-byte sink that takes the staging writes of threads with nothing to stage, so
// that the staging code has no branches (a branch would let the compiler sink an activation
// load behind the weight loads and then wait for all of them).
constexpr size_t kSinkBytes = 48;
template <class C>
__host__ __device__ constexpr size_t fast_lds_bytes(int in_f) {
  return (size_t)windows_per_row(in_f) * 1024 + (size_t)(in_f / 32 + 2) * 4 + kSinkBytes;
}

// Wave-wide shift right by one lane (DPP wave_shr:1); lane 0 receives `in0`.
__device__ __forceinline__ float wave_shr1(float v, float in0) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, in0),
                                                               __builtin_bit_cast(int, v),
                                                               kWaveShr1, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_q8_0_fast(const uint8_t *__restrict__ W, int64_t row_bytes,
                      const int8_t *__restrict__ qs, const float *__restrict__ d,
                      float *__restrict__ y, int in_f, int out_f) {
  constexpr int RPW = C::RPW, U = C::U, KQ = C::KQ, KD = C::KD, NTH = C::THREADS;
  constexpr int SPLIT = C::SPLIT;
  static_assert(C::WAVES % SPLIT == 0, "whole row groups per workgroup");
  extern __shared__ __align__(16) unsigned char lds[];
  const int nb = in_f / 32;
  const int cpr = chunks_per_row(in_f);
  const int nwin = windows_per_row(in_f);
  uint8_t *shaped = lds;                                              // nwin * 1024 bytes
  float *dsc = reinterpret_cast<float *>(lds + (size_t)nwin * 1024);  // nb + 2
  const int t = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int rbase = (blockIdx.x * (C::WAVES / SPLIT) + wave / SPLIT) * RPW;
  const int part = wave % SPLIT;
  const int wbeg = part * nwin / SPLIT, wend = (part + 1) * nwin / SPLIT;  // this wave's windows
  const rsrc_t qrs = buf_rsrc(qs + (int64_t)t * in_f, (uint32_t)in_f);
  const rsrc_t drs = buf_rsrc(d + (int64_t)t * nb, (uint32_t)nb * 4);

  // 1. this thread's activation blocks and scales (oldest loads; zeros past the row).
  int4_t aq[KQ][2];
  float dv[KD];
#pragma unroll
  for (int k = 0; k < KQ; ++k) {
    const uint32_t off = (uint32_t)(threadIdx.x + k * NTH) * 32;
    aq[k][0] = buf_load16(qrs, off);
    aq[k][1] = buf_load16(qrs, off + 16);
  }
#pragma unroll
  for (int k = 0; k < KD; ++k) dv[k] = buf_load_f32(drs, (uint32_t)(threadIdx.x + k * NTH) * 4);

  // 2. the first batch of weight loads: one resource per row over the used bytes of this
  // wave's windows (none for a row past out_f), so chunks past them read as zeros.
  rsrc_t wrs[RPW];
  bool rok[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rok[r] = rbase + r < out_f;
    // wbeg < nwin, so 1024 * wbeg < 16 * cpr and the record count is never negative
    const int lim = cpr * 16 < wend * 1024 ? cpr * 16 : wend * 1024;
    wrs[r] = buf_rsrc(W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes + (int64_t)wbeg * 1024,
                      rok[r] ? (uint32_t)(lim - wbeg * 1024) : 0u);
  }
  // A wave that starts inside the row (wbeg > 0) also needs the block scales that lanes 62
  // and 63 of window wbeg - 1 would carry into it: those two lanes fetch the two scale bytes
  // of their chunk of that window, if it holds one (every other lane reads past the resource,
  // i.e. zero, without touching memory).
  uint32_t prev_bits[RPW];
  const int pc = (wbeg - 1) * kWave + lane;  // chunk of window wbeg - 1 (used when wbeg > 0)
  const int pb = 16 * pc / kBlkBytes;
  const int phb = pb + (16 * pc - kBlkBytes * pb != 0);
  const int phpos = kBlkBytes * phb - 16 * pc;
  const bool prev_scale = SPLIT > 1 && wbeg > 0 && lane >= kWave - 2 && phpos <= 14;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    prev_bits[r] = 0;
    if constexpr (SPLIT > 1) {
      const rsrc_t rowrs = buf_rsrc(W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes,
                                    rok[r] ? (uint32_t)cpr * 16 : 0u);
      prev_bits[r] = __builtin_amdgcn_raw_buffer_load_b16(
          rowrs, prev_scale ? (uint32_t)(16 * pc + phpos) : (uint32_t)cpr * 16, 0, 0);
    }
  }
  int4_t wv[U][RPW];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      wv[u][r] = buf_load16_stream(wrs[r], (uint32_t)(u * 1024 + lane * 16));
  }

  // 3. stage the activation in the shape of a Q8_0 row -- per block two zero bytes where the
  // weight row has its fp16 scale, then the 32 qs -- with zeros past the row, and d_a.
  {
    uint16_t *sh16 = reinterpret_cast<uint16_t *>(shaped);
    unsigned char *sink = lds + fast_lds_bytes<C>(in_f) - kSinkBytes;
#pragma unroll
    for (int k = 0; k < KQ; ++k) {
      const int b = threadIdx.x + k * NTH;
      // 2-byte aligned block start, or the sink for a thread past the last block.
      uint16_t *dst = b < nb ? sh16 + (kBlkBytes / 2) * b : reinterpret_cast<uint16_t *>(sink);
      dst[0] = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[1 + 8 * h + 2 * j] = (uint16_t)((uint32_t)aq[k][h][j] & 0xFFFFu);
          dst[2 + 8 * h + 2 * j] = (uint16_t)((uint32_t)aq[k][h][j] >> 16);
        }
      }
    }
    for (int i = (kBlkBytes / 2) * nb + threadIdx.x; i < nwin * 512; i += NTH) sh16[i] = 0;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const int b = threadIdx.x + k * NTH;
      float *dst = b < nb + 2 ? dsc + b : reinterpret_cast<float *>(sink);
      *dst = dv[k];
    }
  }
  __syncthreads();

  float acc[RPW], carry63[RPW], carry62[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    acc[r] = 0.0f;
    // the same value lanes 62 and 63 compute for window wbeg - 1 (zero at the row start)
    const float H = prev_scale ? (float)__builtin_bit_cast(_Float16, (uint16_t)prev_bits[r]) *
                                     dsc[prev_scale ? phb : 0]
                               : 0.0f;
    carry63[r] = lane_value(H, 63);
    carry62[r] = lane_value(H, 62);
  }

  auto compute = [&](const int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int win = w0 + u;
      if (win >= wend) break;
      const int c = win * kWave + lane;  // chunk index within the row
      const bool live = c < cpr;
      // Chunk geometry (the same for every row): bytes [p0, p0 + 16) of the row.
      const int p0 = 16 * c;
      const int b0 = p0 / kBlkBytes;         // block of the first byte
      const int o = p0 - kBlkBytes * b0;     // offset inside that block, even, 0..32
      const int hb = b0 + (o != 0);          // block whose scale may start in the chunk
      const int hpos = kBlkBytes * hb - p0;  // its byte offset inside the chunk
      const bool has_scale = live && hpos <= 14;
      // dwords j < nlo hold quants of b0 (or its scale); the rest belong to b0 + 1.
      const int nlo = o <= 20 ? 4 : (o <= 24 ? 3 : (o <= 28 ? 2 : 1));
      const int4_t a = *reinterpret_cast<const int4_t *>(shaped + p0);  // zero past the row
      const float da_h = dsc[live ? hb : 0];  // hb <= nb for a chunk inside the row

      // The scale that starts in this chunk (0 if none): fp16 -> f32, times d_a.  The scale of
      // b0 sits delta = 0, 1 or 2 chunks back, i.e. delta lanes to the left: one or two
      // wave-wide DPP right shifts, lanes 0 and 1 taking lanes 62 and 63 of the last window.
      const int delta = o == 0 ? 0 : (o <= 16 ? 1 : 2);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int4_t w = wb[u][r];
        const int q = hpos >> 2;
        const uint32_t dw = q == 0 ? w[0] : (q == 1 ? w[1] : (q == 2 ? w[2] : w[3]));
        const uint16_t hbits = (hpos & 2) ? (uint16_t)(dw >> 16) : (uint16_t)(dw & 0xFFFF);
        const float H = has_scale ? (float)__builtin_bit_cast(_Float16, hbits) * da_h : 0.0f;
        const float h1 = wave_shr1(H, carry63[r]);   // scale of chunk c - 1
        const float h2 = wave_shr1(h1, carry62[r]);  // scale of chunk c - 2
        carry63[r] = lane_value(H, 63);
        carry62[r] = lane_value(H, 62);
        const int t1 = __builtin_amdgcn_sdot4(w[0], a[0], 0, false);
        const int t2 = __builtin_amdgcn_sdot4(w[1], a[1], t1, false);
        const int t3 = __builtin_amdgcn_sdot4(w[2], a[2], t2, false);
        const int t4 = __builtin_amdgcn_sdot4(w[3], a[3], t3, false);
        const int s_lo = nlo == 4 ? t4 : (nlo == 3 ? t3 : (nlo == 2 ? t2 : t1));
        const int s_hi = t4 - s_lo;
        const float S0 = live ? (delta == 0 ? H : (delta == 1 ? h1 : h2)) : 0.0f;
        const float S1 = (live && nlo < 4) ? H : 0.0f;
        acc[r] = fmaf((float)s_lo, S0, acc[r]);
        acc[r] = fmaf((float)s_hi, S1, acc[r]);
      }
    }
  };
  // Loads are issued unconditionally: past the row they read zeros and no memory.
  auto load = [&](int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        wb[u][r] = buf_load16_stream(wrs[r], (uint32_t)((w0 + u - wbeg) * 1024 + lane * 16));
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
      if (lane == 0 && rok[r]) y[(int64_t)t * out_f + rbase + r] = s;
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
        y[(int64_t)t * out_f + rbase + r] = s;
      }
    }
  }
}

// Generic path: one wave per row, one lane per 34-byte block, 2-byte loads (W and row_bytes
// need only be 2-byte aligned).
__global__ __launch_bounds__(kThreads) void k_gemv_q8_0_generic(
    const uint8_t *__restrict__ W, int64_t row_bytes, const int8_t *__restrict__ qs,
    const float *__restrict__ d, float *__restrict__ y, int in_f, int out_f) {
  const int nb = in_f / 32;
  const int t = blockIdx.y;
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (row >= out_f) return;  // whole wave exits together
  const uint16_t *wr = reinterpret_cast<const uint16_t *>(W + (int64_t)row * row_bytes);
  const int8_t *qa = qs + (int64_t)t * in_f;
  const float *da = d + (int64_t)t * nb;
  float acc = 0.0f;
  for (int b = lane; b < nb; b += kWave) {
    const uint16_t *blk = wr + b * (kBlkBytes / 2);
    const uint16_t hbits = blk[0];
    int isum = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t wq = (uint32_t)blk[1 + 2 * j] | ((uint32_t)blk[2 + 2 * j] << 16);
      const int aq = *reinterpret_cast<const int *>(qa + 32 * b + 4 * j);
      isum = __builtin_amdgcn_sdot4((int)wq, aq, isum, false);
    }
    const float S = (float)__builtin_bit_cast(_Float16, hbits) * da[b];
    acc = fmaf((float)isum, S, acc);
  }
  const float s = wave_sum(acc);
  if (lane == 0) y[(int64_t)t * out_f + row] = s;
}

template <class C>
hipError_t launch_fast(const uint8_t *W, int64_t row_bytes, const int8_t *qs, const float *d,
                       float *y, int m, int in_f, int out_f, hipStream_t s) {
  auto kern = k_gemv_q8_0_fast<C>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)fast_lds_bytes<C>(C::MAX_IN_F));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 g((out_f + C::ROWS - 1) / C::ROWS, m);
  hipLaunchKernelGGL(kern, g, dim3(C::THREADS), fast_lds_bytes<C>(in_f), s, W, row_bytes, qs, d,
                     y, in_f, out_f);
  return hipGetLastError();
}

// Shapes as for the e4m3 stream: 4 waves up to in_f = 8192, 8 up to 24576, 16 beyond, with
// double-buffered batches of 3 or 4 windows (a row of in_f = 5120 is 6 windows, the last one
// partly used).  In the middle range two waves share each row (4 rows per workgroup): rows
// of 17408 columns are 19 windows, and with one wave per row a 5120-row matrix would keep
// only 20 long-lived waves per CU, unevenly spread; measured 10% faster split.
using QSmall = QCfg<4, 1, 3, 1, 2, true>;         // in_f <= 8192
using QMid = QCfg<8, 1, 4, 2, 3, true, 8, 2>;     // in_f <= 32768
using QLarge = QCfg<16, 1, 4, 2, 3, true>;  // in_f <= 65536
static_assert(QSmall::MAX_IN_F >= 8192 && QMid::MAX_IN_F >= 24576 && QLarge::MAX_IN_F == kMaxInF,
              "activation coverage of the in_f ranges dispatched to each shape");
static_assert(QSmall::KD * QSmall::THREADS >= QSmall::MAX_IN_F / 32 + 2 &&
                  QMid::KD * QMid::THREADS >= QMid::MAX_IN_F / 32 + 2 &&
                  QLarge::KD * QLarge::THREADS >= QLarge::MAX_IN_F / 32 + 2,
              "scale coverage");

}  // namespace

hipError_t launch_gemv_q8_0(const uint8_t *W, int64_t row_bytes, const int8_t *qs,
                            const float *d, float *y, int m, int in_f, int out_f, hipStream_t s) {
  const bool fast = (in_f % 256 == 0) && (row_bytes % 16 == 0) &&
                    ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
  if (fast) {
    if (in_f <= 8192) return launch_fast<QSmall>(W, row_bytes, qs, d, y, m, in_f, out_f, s);
    if (in_f <= 24576) return launch_fast<QMid>(W, row_bytes, qs, d, y, m, in_f, out_f, s);
    return launch_fast<QLarge>(W, row_bytes, qs, d, y, m, in_f, out_f, s);
  }
  const dim3 g((out_f + kWaves - 1) / kWaves, m);
  hipLaunchKernelGGL(k_gemv_q8_0_generic, g, dim3(kThreads), 0, s, W, row_bytes, qs, d, y, in_f,
                     out_f);
  return hipGetLastError();
}

}  // namespace fp8gemv

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
// loads.  Fast path (in_f % 256 == 0, W 16-byte aligned, row_bytes % 16 == 0):
//   * The block pattern repeats every 272 bytes: a "group" is 8 blocks = 17 chunks of 16
//     bytes, and every group starts on a block boundary.  A window is 3 groups (816 bytes):
//     lane l < 51 streams chunk l of the window with one 16-byte non-temporal load, so a
//     wave-wide load reads 816 contiguous bytes and every weight byte is fetched once; lanes
//     51..63 load nothing (their offsets lie past the buffer resource).
//   * Because windows start on group boundaries, everything about a lane's chunk -- where its
//     block boundary falls, whether and where it holds a block scale, which lane holds the
//     scale of its first block -- is the same in every window and every row.  It is worked
//     out once per thread, outside the stream loop; per window only the data change.
//   * The activation is staged in LDS "in the shape of a Q8_0 row": 34 bytes per block, two
//     zero bytes where the weight row has its fp16 scale, then the 32 qs.  A weight chunk and
//     the activation chunk at the same offset line up byte for byte, so four v_dot4_i32_i8
//     give the integer products of the chunk, and the scale bytes meet zeros.
//   * No dword mixes quantised bytes of two blocks (block boundaries are 34 bytes apart and
//     the 2-byte scale sits between them), so a chunk's four dwords split into a prefix that
//     belongs to block b0 and a suffix that belongs to b0 + 1; the two exact int32 sums are
//     scaled separately.
//   * A chunk holds at most one block scale.  The lane holding it extracts the two bytes with
//     v_perm_b32 (fixed selectors per lane), converts fp16 -> f32 and multiplies by d_a of
//     that block.  The scale of a chunk's first block starts 0, 1 or 2 chunks earlier in the
//     same group -- 0, 1 or 2 lanes to the left -- and reaches the lanes that need it through
//     one or two wave-wide DPP right shifts.  A window never needs a value from the previous
//     one, so a row can also be split between waves at any window.
// Generic path (any in_f % 32 == 0): one lane per block, 2-byte loads; correct, not tuned.
// Several activation rows (MT per workgroup, grid.y = ceil(m / MT)) share one weight pass:
// the scale of a weight chunk is extracted once and its dwords are split once into the parts
// of block b0 and b0 + 1; every row's integer sums are exact, so they equal the MT = 1 prefix
// sums, and its float operations are those of MT = 1 in the same order.  (With MT > 1 the
// fp16 scale of a chunk's first block is moved between lanes once per window and each row
// multiplies it by its own d_a there; that is the product the scale's own lane forms for
// MT = 1, so the bits are the same.)  Every launch shape
// of an in_f range splits rows the same way, so each activation row of an m-row call is
// bit-identical to an m=1 call on that row.  The launches for 3 or more rows of up to 24576
// columns are persistent, as in the e4m3 stream: the device's resident workgroups stage their
// activation rows once and their waves take groups of RPW weight rows in turn.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;  // generic path
constexpr int kWaves = kThreads / kWave;
constexpr int kBlkBytes = 34;
constexpr int kGrpChunks = 17;                        // 272 bytes = 8 blocks = 256 weights
constexpr int kWinLanes = 3 * kGrpChunks;             // 51 lanes stream a window
constexpr int kWinBytes = kWinLanes * 16;             // 816 bytes
constexpr int kWinBlocks = kWinBytes / kBlkBytes;     // 24 blocks
static_assert(kWinBlocks * kBlkBytes == kWinBytes, "a window is whole blocks");

// Windows of a row (fast path: in_f % 256 == 0, i.e. whole groups).
__host__ __device__ constexpr int windows_per_row(int in_f) {
  return (in_f / 256 + 2) / 3;
}

// Launch shape of the fast path.  Each thread stages KQ activation blocks and KD block scales:
// KQ * WAVES * 64 >= in_f / 32 and KD * WAVES * 64 >= in_f / 32 + 32 (the scale table is
// padded with zeros to whole windows plus one group).
// DB: double-buffered window loop -- the next U windows are loaded before the current U are
// consumed, so a wave never waits with nothing in flight (rows of many windows).
// MT: activation rows per workgroup.  Each weight chunk is loaded once and used for all MT
// rows; every row gets the same exact integer sums and the same float operations as MT = 1.
template <int WAVES_, int RPW_, int U_, int KQ_, int KD_, bool DB_ = false, int WPE_ = 8,
          int SPLIT_ = 1, int MT_ = 1>
struct QCfg {
  static constexpr int WAVES = WAVES_, RPW = RPW_, U = U_, KQ = KQ_, KD = KD_, WPE = WPE_;
  static constexpr bool DB = DB_;
  static constexpr int MT = MT_;
  static constexpr int SPLIT = SPLIT_;  // waves sharing one group of RPW rows (split over k)
  static constexpr int ROWS = WAVES / SPLIT * RPW;  // rows per workgroup
  // The launches for 3-8 activation rows are persistent: as many workgroups as fit on the
  // device at once, whose waves loop over groups of RPW rows (the staging of the MT
  // activation rows is paid once per workgroup, and the rows spread evenly over the waves).
  static constexpr bool PERSIST = MT_ >= 4 && SPLIT_ == 1;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int MAX_IN_F = KQ * THREADS * 32;
  // the template arguments, for config_text
  static constexpr const char *NAME = "QCfg";
  static constexpr int P0 = WAVES_, P1 = RPW_, P2 = U_, P3 = KQ_, P4 = KD_, P6 = WPE_,
                       P7 = SPLIT_, P8 = MT_;
  static constexpr bool P5 = DB_;
};

// LDS layout of the fast path: shaped activation (whole windows), then d_a padded with zeros
// to nwin * 24 + 8 entries.  Last: a 48-byte sink that takes the staging writes of threads
// with nothing to stage, so that the staging code has no branches (a branch would let the
// compiler sink an activation load behind the weight loads and then wait for all of them).
constexpr size_t kSinkBytes = 48;
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one CU, the most a workgroup may use
__host__ __device__ constexpr size_t dsc_entries(int in_f) {
  return (size_t)windows_per_row(in_f) * kWinBlocks + 8;
}
// One staged activation row (16-byte multiple: 816 * nwin + 4 * (24 * nwin + 8)).
__host__ __device__ constexpr size_t row_lds_bytes(int in_f) {
  return (size_t)windows_per_row(in_f) * kWinBytes + dsc_entries(in_f) * 4;
}
__host__ __device__ constexpr size_t fast_lds_bytes(int in_f, int mt) {
  return (size_t)mt * row_lds_bytes(in_f) + kSinkBytes;
}

// Wave-wide shift right by one lane (DPP wave_shr:1); lane 0 receives 0 (bound_ctrl: a lane
// whose source is out of range reads zero, so no zero has to be moved into the destination
// first).
__device__ __forceinline__ float wave_shr1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                            kWaveShr1, 0xF, 0xF, true));
}

// Signed 4 x int8 dot product plus c.  The clamp bit keeps the compiler on the three-operand
// v_dot4_i32_i8: without it the accumulator is tied to the destination (v_dot4c), and every
// partial sum that is also used on its own costs a copy.  The sums here stay far inside int32
// (at most 16 * 128 * 127 in magnitude per chunk), so the clamp never acts and the result is
// the exact integer.
__device__ __forceinline__ int dot4(int a, int b, int c) {
  return __builtin_amdgcn_sdot4(a, b, c, true);
}

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::WPE, C::WPE)))
void k_gemv_q8_0_fast(const uint8_t *__restrict__ W, int64_t row_bytes,
                      const int8_t *__restrict__ qs, const float *__restrict__ d,
                      float *__restrict__ y, int m, int in_f, int out_f) {
  constexpr int RPW = C::RPW, U = C::U, KQ = C::KQ, KD = C::KD, NTH = C::THREADS, MT = C::MT;
  constexpr int SPLIT = C::SPLIT;
  static_assert(C::WAVES % SPLIT == 0, "whole row groups per workgroup");
  extern __shared__ __align__(16) unsigned char lds[];
  const int nb = in_f / 32;
  const int row_used = nb * kBlkBytes;  // used bytes of a row (a multiple of 16)
  const int nwin = windows_per_row(in_f);
  const int ndsc = nwin * kWinBlocks + 8;
  const int row_lds = (int)row_lds_bytes(in_f);
  // activation row tt: shaped bytes at lds + tt * row_lds (nwin * 816), then ndsc scales
  const int t0 = blockIdx.y * MT;  // first activation row of this workgroup
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  // PERSIST: group g of RPW rows belongs to wave g mod (waves of the grid), numbered so that
  // consecutive groups fall on different workgroups; every row is still computed by one wave
  // with the operations of m = 1.
  constexpr bool PERSIST = C::PERSIST;
  static_assert(!PERSIST || SPLIT == 1, "a persistent wave owns whole rows");
  const int ngroups = (out_f + RPW - 1) / RPW;
  const int gstride = (int)gridDim.x * C::WAVES;
  int grp = wave * (int)gridDim.x + (int)blockIdx.x;
  int rbase = PERSIST ? grp * RPW : (blockIdx.x * (C::WAVES / SPLIT) + wave / SPLIT) * RPW;
  const int part = wave % SPLIT;
  const int wbeg = part * nwin / SPLIT, wend = (part + 1) * nwin / SPLIT;  // this wave's windows

  // 1. this thread's activation blocks and scales of the MT rows (oldest loads; zeros past
  // the row and for rows past m).
  int4_t aq[MT][KQ][2];
  float dv[MT][KD];
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) {
    const bool tok = t0 + tt < m;
    const rsrc_t qrs = buf_rsrc(qs + (int64_t)(tok ? t0 + tt : 0) * in_f, tok ? (uint32_t)in_f : 0u);
    const rsrc_t drs = buf_rsrc(d + (int64_t)(tok ? t0 + tt : 0) * nb, tok ? (uint32_t)nb * 4 : 0u);
#pragma unroll
    for (int k = 0; k < KQ; ++k) {
      const uint32_t off = (uint32_t)(threadIdx.x + k * NTH) * 32;
      aq[tt][k][0] = buf_load16(qrs, off);
      aq[tt][k][1] = buf_load16(qrs, off + 16);
    }
#pragma unroll
    for (int k = 0; k < KD; ++k)
      dv[tt][k] = buf_load_f32(drs, (uint32_t)(threadIdx.x + k * NTH) * 4);
  }

  // 2. the first batch of weight loads: one resource per row over the used bytes of this
  // wave's windows (none for a row past out_f), so chunks past them read as zeros.  Lanes
  // 51..63 use an offset past any resource.
  const uint32_t lane_off = lane < kWinLanes ? (uint32_t)lane * 16 : 0x40000000u;
  rsrc_t wrs[RPW];
  bool rok[RPW];
  auto setup_rows = [&]() {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      rok[r] = rbase + r < out_f;
      // wbeg < nwin, so 816 * wbeg < row_used and the record count is never negative
      const int lim = row_used < wend * kWinBytes ? row_used : wend * kWinBytes;
      wrs[r] = buf_rsrc(W + (int64_t)(rok[r] ? rbase + r : 0) * row_bytes + (int64_t)wbeg * kWinBytes,
                        rok[r] ? (uint32_t)(lim - wbeg * kWinBytes) : 0u);
    }
  };
  setup_rows();
  int4_t wv[U][RPW];
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      wv[u][r] = buf_load16_stream(wrs[r], lane_off + (uint32_t)(u * kWinBytes));
  }

  // 3. stage the activation in the shape of a Q8_0 row -- per block two zero bytes where the
  // weight row has its fp16 scale, then the 32 qs -- with zeros to the end of the last
  // window, and d_a with zeros past nb.
  unsigned char *sink = lds + MT * row_lds;
#pragma unroll
  for (int tt = 0; tt < MT; ++tt) {
    uint16_t *sh16 = reinterpret_cast<uint16_t *>(lds + tt * row_lds);
    float *dsc = reinterpret_cast<float *>(lds + tt * row_lds + nwin * kWinBytes);
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
          dst[1 + 8 * h + 2 * j] = (uint16_t)((uint32_t)aq[tt][k][h][j] & 0xFFFFu);
          dst[2 + 8 * h + 2 * j] = (uint16_t)((uint32_t)aq[tt][k][h][j] >> 16);
        }
      }
    }
    for (int i = (kBlkBytes / 2) * nb + threadIdx.x; i < nwin * (kWinBytes / 2); i += NTH) sh16[i] = 0;
#pragma unroll
    for (int k = 0; k < KD; ++k) {
      const int b = threadIdx.x + k * NTH;
      float *dst = b < ndsc ? dsc + b : reinterpret_cast<float *>(sink);
      *dst = dv[tt][k];
    }
  }

  // 4. this lane's chunk geometry, the same in every window: chunk r of group g of the window.
  const int gidx = lane < kWinLanes ? lane / kGrpChunks : 0;
  const int rch = lane < kWinLanes ? lane % kGrpChunks : kGrpChunks - 1;
  const int p0 = 16 * rch;                 // byte offset of the chunk in its group
  const int b0 = p0 / kBlkBytes;           // block of its first byte
  const int o = p0 - kBlkBytes * b0;       // offset inside that block, even, 0..32
  const int hb = b0 + (o != 0);            // block whose scale may start in the chunk
  const int hpos = kBlkBytes * hb - p0;    // its byte offset inside the chunk
  const bool has_scale = lane < kWinLanes && hpos <= 14;
  // v_perm_b32 selectors that move the two scale bytes to bits 0..15 from dwords 0-1 or 2-3
  // of the chunk; selector byte 0x0C yields zero, so a lane without a scale gets 0.
  const uint32_t sel_lo = has_scale && hpos < 8
                              ? 0x0C0C0000u | ((uint32_t)(hpos + 1) << 8) | (uint32_t)hpos
                              : 0x0C0C0C0Cu;
  const uint32_t sel_hi = has_scale && hpos >= 8
                              ? 0x0C0C0000u | ((uint32_t)(hpos - 7) << 8) | (uint32_t)(hpos - 8)
                              : 0x0C0C0C0Cu;
  // dwords j < nlo hold quants of b0 (or its scale); the rest belong to b0 + 1.
  const bool lo_ge2 = o <= 28, lo_ge3 = o <= 24, lo_4 = o <= 20;
  // the scale of b0 sits delta = 0, 1 or 2 lanes to the left
  const bool d0 = o == 0, d1 = o != 0 && o <= 16;
  const int dsc_lane = 8 * gidx + (has_scale ? hb : 0);  // d_a entry of the scale, per window + 24
  const int dsc_b0 = 8 * gidx + b0;                       // d_a entry of the chunk's first block
  const int lds_lane = lane < kWinLanes ? lane * 16 : 0;  // lanes 51..63 multiply zero weights
  __syncthreads();

  float acc[MT][RPW];
#pragma unroll
  for (int tt = 0; tt < MT; ++tt)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[tt][r] = 0.0f;

  auto compute = [&](const int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int win = w0 + u;
      if (win >= wend) break;
      // Per weight row: the scale bytes of the chunk (fp16 -> f32) and, for MT > 1, the
      // dwords of b0 and of b0 + 1 as two masked copies of the chunk, shared by all rows (the
      // integer sums are exact, so they equal the MT = 1 prefix sums).
      float hw[RPW];
      int4_t wlo[RPW], whi[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int4_t w = wb[u][r];
        const uint32_t hbits = __builtin_amdgcn_perm((uint32_t)w[1], (uint32_t)w[0], sel_lo) |
                               __builtin_amdgcn_perm((uint32_t)w[3], (uint32_t)w[2], sel_hi);
        hw[r] = (float)__builtin_bit_cast(_Float16, (uint16_t)hbits);
        wlo[r] = int4_t{w[0], lo_ge2 ? w[1] : 0, lo_ge3 ? w[2] : 0, lo_4 ? w[3] : 0};
        whi[r] = int4_t{0, lo_ge2 ? 0 : w[1], lo_ge3 ? 0 : w[2], lo_4 ? 0 : w[3]};
      }
      // Activation row tt's chunk and scale from LDS, read ahead of its multiply (below), so
      // the LDS latency is not paid once per row.
      auto read_row = [&](int tt, int4_t &a, float &da, float &da0) {
        const unsigned char *arow = lds + tt * row_lds;
        a = *reinterpret_cast<const int4_t *>(arow + win * kWinBytes + lds_lane);
        const float *dsc = reinterpret_cast<const float *>(arow + nwin * kWinBytes) + win * kWinBlocks;
        da = dsc[dsc_lane];
        if constexpr (MT > 1) da0 = dsc[dsc_b0];
      };
      // MT > 1: the fp16 scale of the chunk's first block is fetched from its lane once per
      // window; each row then forms the same product (scale x d_a of that block) locally.
      float hw0[RPW];
      if constexpr (MT > 1) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float g1 = wave_shr1(hw[r]);
          const float g2 = wave_shr1(g1);
          hw0[r] = d0 ? hw[r] : (d1 ? g1 : g2);
        }
      }
      // Up to 4 rows: all their chunks are read before the first is multiplied; more rows:
      // one row ahead (registers).
      constexpr int NB = MT <= 4 ? MT : 2;
      int4_t abuf[NB];
      float dbuf[NB], d0buf[NB];
#pragma unroll
      for (int j = 0; j + 1 < NB; ++j) read_row(j, abuf[j], dbuf[j], d0buf[j]);
#pragma unroll
      for (int tt = 0; tt < MT; ++tt) {
        if (tt + NB - 1 < MT)
          read_row(tt + NB - 1, abuf[(tt + NB - 1) % NB], dbuf[(tt + NB - 1) % NB],
                   d0buf[(tt + NB - 1) % NB]);
        const int4_t a = abuf[tt % NB];
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float H = hw[r] * dbuf[tt % NB];
          float h1 = 0.0f, h2 = 0.0f;
          if constexpr (MT == 1) {
            h1 = wave_shr1(H);   // scale of chunk c - 1
            h2 = wave_shr1(h1);  // scale of chunk c - 2
          }
          int s_lo, s_hi;
          if constexpr (MT == 1) {
            const int4_t w = wb[u][r];
            const int t1 = dot4(w[0], a[0], 0);
            const int t2 = dot4(w[1], a[1], t1);
            const int t3 = dot4(w[2], a[2], t2);
            const int t4 = dot4(w[3], a[3], t3);
            s_lo = lo_4 ? t4 : (lo_ge3 ? t3 : (lo_ge2 ? t2 : t1));
            s_hi = t4 - s_lo;
          } else {
            s_lo = dot4(wlo[r][0], a[0], 0);
            s_lo = dot4(wlo[r][1], a[1], s_lo);
            s_lo = dot4(wlo[r][2], a[2], s_lo);
            s_lo = dot4(wlo[r][3], a[3], s_lo);
            s_hi = dot4(whi[r][1], a[1], 0);
            s_hi = dot4(whi[r][2], a[2], s_hi);
            s_hi = dot4(whi[r][3], a[3], s_hi);
          }
          float S0;
          if constexpr (MT == 1) {
            S0 = d0 ? H : (d1 ? h1 : h2);
          } else {
            S0 = hw0[r] * d0buf[tt % NB];
          }
          acc[tt][r] = fmaf((float)s_lo, S0, acc[tt][r]);
          acc[tt][r] = fmaf((float)s_hi, H, acc[tt][r]);
        }
      }
    }
  };
  // Loads are issued unconditionally: past this wave's windows they read zeros and no memory.
  auto load = [&](int4_t (&wb)[U][RPW], int w0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        wb[u][r] = buf_load16_stream(wrs[r], lane_off + (uint32_t)((w0 + u - wbeg) * kWinBytes));
    }
  };
  for (;;) {
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
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float s = wave_sum(acc[tt][r]);
        if (lane == 0 && rok[r] && t0 + tt < m) y[(int64_t)(t0 + tt) * out_f + rbase + r] = s;
      }
    }
    if constexpr (!PERSIST) break;
    // the next group of this wave, if any (wave-uniform)
    grp += gstride;
    if (grp >= ngroups) break;
    rbase = grp * RPW;
    setup_rows();
    load(wv, wbeg);
#pragma unroll
    for (int tt = 0; tt < MT; ++tt)
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[tt][r] = 0.0f;
  } else {
    // the SPLIT partial sums of a row meet in LDS and are added in part order
    __shared__ float psum[MT][C::WAVES * RPW];
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float s = wave_sum(acc[tt][r]);
        if (lane == 0) psum[tt][wave * RPW + r] = s;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < MT; ++tt) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (lane == 0 && part == 0 && rok[r] && t0 + tt < m) {
          float s = psum[tt][wave * RPW + r];
#pragma unroll
          for (int p = 1; p < SPLIT; ++p) s += psum[tt][(wave + p) * RPW + r];
          y[(int64_t)(t0 + tt) * out_f + rbase + r] = s;
        }
      }
    }
    break;
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

// Workgroups along x: one per ROWS rows, or for a persistent launch as many as fit on the
// device at once (WPE waves per SIMD and the LDS of the staged rows; at most one per WAVES row
// groups), so one round covers the grid.
template <class C>
unsigned grid_x_for(int out_f, int in_f) {
  if constexpr (C::PERSIST) {
    const int groups = (out_f + C::RPW - 1) / C::RPW;
    const int want = (groups + C::WAVES - 1) / C::WAVES;
    const int by_waves = 4 * C::WPE / C::WAVES;
    const int lds = (int)fast_lds_bytes(in_f, C::MT);
    const int by_lds = (int)(kLdsBytes / ((lds + 1023) / 1024 * 1024));
    const int cap = cu_count() * (by_waves < by_lds ? by_waves : by_lds);
    return (unsigned)(want < cap ? want : cap);
  } else {
    return (unsigned)((out_f + C::ROWS - 1) / C::ROWS);
  }
}

template <class C>
hipError_t launch_fast(const uint8_t *W, int64_t row_bytes, const int8_t *qs, const float *d,
                       float *y, int m, int in_f, int out_f, hipStream_t s) {
  auto kern = k_gemv_q8_0_fast<C>;
  static std::atomic<bool> lds_set[kMaxDevices];
  const size_t want = fast_lds_bytes(C::MAX_IN_F, C::MT);
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void *>(kern),
                                          want < kLdsBytes ? want : kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  const dim3 g(grid_x_for<C>(out_f, in_f), (m + C::MT - 1) / C::MT);
  hipLaunchKernelGGL(kern, g, dim3(C::THREADS), fast_lds_bytes(in_f, C::MT), s, W, row_bytes, qs,
                     d, y, m, in_f, out_f);
  return hipGetLastError();
}

// Shapes measured on MI355X: one wave per row throughout, 4-wave workgroups up to in_f = 24576
// and 16 beyond, with double-buffered batches of 4 windows (a row of in_f = 5120 is 7 windows,
// the last one two groups; a row of 17408 is 23).  Unlike the e4m3 stream, the middle range
// does not split rows between waves: with 816-byte windows, one wave per row in 4-wave
// workgroups is 2-7% faster at 5120x17408, 2048x12288 and 5120x12288 than two waves per row
// in 8-wave ones.
// Several activation rows (m > 1) share each weight pass: up to 8 rows per workgroup for
// in_f <= 8192, 2 up to 24576 and 1 beyond (LDS holds one staged row per activation row).  Every shape
// used for one in_f range splits rows the same way (SPLIT), so each activation row is
// computed in the same order whatever m is.
using QSmall = QCfg<4, 1, 4, 1, 2, true>;                 // in_f <= 8192, m = 1
using QSmallB2 = QCfg<4, 1, 3, 1, 2, true, 8, 1, 2>;      //               m = 2
using QSmallB4 = QCfg<4, 1, 2, 1, 2, true, 5, 1, 4>;      //               m = 3..4
using QSmallB8 = QCfg<8, 2, 1, 1, 3, true, 4, 1, 8>;      //               m >= 5
using QMid = QCfg<4, 1, 4, 3, 4, true>;                   // in_f <= 24576, m = 1
using QMidB2 = QCfg<8, 1, 3, 2, 3, true, 8, 1, 2>;        //                m = 2
using QMidB4 = QCfg<8, 1, 3, 2, 3, true, 4, 1, 4>;        //                m >= 3
using QLarge = QCfg<16, 1, 4, 2, 3, true>;                // in_f <= 65536
static_assert(QSmall::MAX_IN_F >= 8192 && QSmallB2::MAX_IN_F >= 8192 &&
                  QSmallB4::MAX_IN_F >= 8192 && QSmallB8::MAX_IN_F >= 8192 &&
                  QMid::MAX_IN_F >= 24576 && QMidB2::MAX_IN_F >= 24576 &&
                  QMidB4::MAX_IN_F >= 24576 && QLarge::MAX_IN_F == kMaxInF,
              "activation coverage of the in_f ranges dispatched to each shape");
static_assert(QSmall::KD * QSmall::THREADS >= (int)dsc_entries(QSmall::MAX_IN_F) &&
                  QSmallB2::KD * QSmallB2::THREADS >= (int)dsc_entries(8192) &&
                  QSmallB4::KD * QSmallB4::THREADS >= (int)dsc_entries(8192) &&
                  QSmallB8::KD * QSmallB8::THREADS >= (int)dsc_entries(8192) &&
                  QMid::KD * QMid::THREADS >= (int)dsc_entries(QMid::MAX_IN_F) &&
                  QMidB2::KD * QMidB2::THREADS >= (int)dsc_entries(24576) &&
                  QMidB4::KD * QMidB4::THREADS >= (int)dsc_entries(24576) &&
                  QLarge::KD * QLarge::THREADS >= (int)dsc_entries(QLarge::MAX_IN_F),
              "scale coverage");
static_assert(fast_lds_bytes(8192, QSmallB8::MT) <= kLdsBytes &&
                  fast_lds_bytes(24576, QMidB2::MT) <= kLdsBytes &&
                  fast_lds_bytes(24576, QMidB4::MT) <= kLdsBytes &&
                  fast_lds_bytes(kMaxInF, 1) <= kLdsBytes,
              "staged rows fit the LDS of a workgroup");
static_assert(QSmall::SPLIT == QSmallB2::SPLIT && QSmall::SPLIT == QSmallB4::SPLIT &&
                  QSmall::SPLIT == QSmallB8::SPLIT && QMid::SPLIT == QMidB2::SPLIT &&
                  QMid::SPLIT == QMidB4::SPLIT,
              "one row split per in_f range");

}  // namespace

namespace {
// The launch shape for (m, in_f) on the fast path: f is called with the Tag of the chosen
// configuration.
template <class F>
auto with_cfg(int m, int in_f, F &&f) {
  if (in_f <= 8192) {
    if (m == 1) return f(Tag<QSmall>{});
    if (m == 2) return f(Tag<QSmallB2>{});
    if (m <= 4) return f(Tag<QSmallB4>{});
    return f(Tag<QSmallB8>{});
  }
  if (in_f <= 24576) {
    if (m == 1) return f(Tag<QMid>{});
    if (m == 2) return f(Tag<QMidB2>{});
    return f(Tag<QMidB4>{});
  }
  return f(Tag<QLarge>{});
}

bool fast_path(const uint8_t *W, int64_t row_bytes, int in_f) {
  return (in_f % 256 == 0) && (row_bytes % 16 == 0) &&
         ((reinterpret_cast<uintptr_t>(W) & 15) == 0);
}
}  // namespace

hipError_t launch_gemv_q8_0(const uint8_t *W, int64_t row_bytes, const int8_t *qs,
                            const float *d, float *y, int m, int in_f, int out_f,
                            bool matrix_cores, hipStream_t s) {
  if (matrix_cores && gemv_q8_0_mfma_applies(W, row_bytes, in_f))
    return launch_gemv_q8_0_mfma(W, row_bytes, qs, d, y, m, in_f, out_f, s);
  if (fast_path(W, row_bytes, in_f)) {
    return with_cfg(m, in_f, [&](auto tag) {
      using C = typename decltype(tag)::type;
      return launch_fast<C>(W, row_bytes, qs, d, y, m, in_f, out_f, s);
    });
  }
  const dim3 g((out_f + kWaves - 1) / kWaves, m);
  hipLaunchKernelGGL(k_gemv_q8_0_generic, g, dim3(kThreads), 0, s, W, row_bytes, qs, d, y, in_f,
                     out_f);
  return hipGetLastError();
}

LaunchDesc describe_gemv_q8_0(const uint8_t *W, int64_t row_bytes, int m, int in_f, int out_f,
                              bool matrix_cores) {
  if (matrix_cores && gemv_q8_0_mfma_applies(W, row_bytes, in_f))
    return describe_gemv_q8_0_mfma(m, in_f, out_f);
  if (fast_path(W, row_bytes, in_f)) {
    return with_cfg(m, in_f, [&](auto tag) {
      using C = typename decltype(tag)::type;
      LaunchDesc r;
      r.grid_x = grid_x_for<C>(out_f, in_f);
      r.grid_y = (unsigned)((m + C::MT - 1) / C::MT);
      r.threads = C::THREADS;
      r.lds = (unsigned)fast_lds_bytes(in_f, C::MT);
      r.kernel = "k_gemv_q8_0_fast";
      r.config = config_text<C>();
      return r;
    });
  }
  LaunchDesc r;
  r.grid_x = (unsigned)((out_f + kWaves - 1) / kWaves);
  r.grid_y = (unsigned)m;
  r.threads = kThreads;
  r.kernel = "k_gemv_q8_0_generic";
  return r;
}

}  // namespace fp8gemv

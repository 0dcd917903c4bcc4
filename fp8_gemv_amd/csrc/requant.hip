// Load-time requantisation of a raw e4m3 weight plane into ggml Q8_0 rows.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/gemv_e4m3_bench.rs -- module doc QUESTION (the
// ship path dequantises FP8 checkpoints to a Q8_0 slab at load: an fp16 scale then 32 int8 per
// 32 weights, 34 bytes) and THE BLOCK-128 ARM (the per-tile f32 grid of block-scaled
// checkpoints).  The page gives no formula; this takes the 32-value int8 block rule of the gate
// page's q8_1 quantiser (q8_fuse_gate.rs, the `id = 1/d` branch) with the scale stored as fp16.
// Per 32-block of row r, all in f32:
//   v_i = e4m3(W[r, 32b + i]) * S      S = scale, or grid[r / 128, b / 4]
//   d   = max_i |v_i| / 127,  id = 1 / d (0 when d == 0)
//   q_i = round(v_i * id), halves away from zero
//   out = binary16(d) (round to nearest even, little-endian), then the 32 q_i as int8
// d and id are IEEE f32 quotients (HIP's default division is correctly rounded) and the file is
// compiled without contraction, so every step rounds exactly once, as written.
//
// gfx950 design: 1 byte read, 1.0625 bytes written per weight.  One thread per block, 256
// blocks per workgroup, numbered across rows (block g is block g % nb of row g / nb), so no
// lane idles at the end of a row whatever in_f is: every wave's arithmetic is useful work.  When
// the output rows are packed (q_row_bytes = 34 nb) a workgroup's 256 * 34 output bytes are
// contiguous, so they are assembled in LDS and written back with coalesced 16-byte stores
// (2-byte stores when the start or the length is not a multiple of 16); padded output rows
// take one 2-byte store per halfword of each thread's own block.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;   // blocks per workgroup
constexpr int kBlk = 34;        // Q8_0 block bytes
typedef float float2_t __attribute__((ext_vector_type(2)));

// round(x), halves away from zero, as an int: x plus the largest float below one half, with
// x's sign, truncated.  The f32 sum reaches the next integer exactly when |frac(x)| >= 1/2 (an
// exhaustive check over every finite f32 confirms it), so this is one bit-insert, one add and
// one truncating conversion instead of roundf's compare-and-select sequence.
__device__ __forceinline__ int round_half_away(float x) {
  const float h = __builtin_bit_cast(
      float, (__builtin_bit_cast(uint32_t, x) & 0x80000000u) | 0x3EFFFFFFu);
  return (int)(x + h);
}

// How a workgroup writes its assembled blocks.
enum StoreMode : int {
  kStoreWide = 0,    // packed output rows, 16-byte aligned start and length: 16-byte stores
  kStorePacked = 1,  // packed output rows otherwise: coalesced 2-byte stores
  kStoreRows = 2,    // padded output rows: each thread stores its own block
};

template <bool BLK>
__global__ __launch_bounds__(kThreads) void k_requant_q8_0(
    const uint8_t *__restrict__ W, int64_t row_bytes, float scale, const float *__restrict__ grid,
    int grid_cols, uint8_t *__restrict__ Wq, int64_t q_row_bytes, int nb, int total,
    double inv_nb, int store_mode) {
  __shared__ __align__(16) uint16_t out16[kThreads * kBlk / 2];
  const int g0 = blockIdx.x * kThreads;
  const int g = g0 + (int)threadIdx.x;
  const bool valid = g < total;
  const int gc = valid ? g : total - 1;  // past the end: recompute the last block, store nothing
  // Row and block of gc.  The f64 product gc * fl(1/nb) is within 2^-21 of gc / nb, whose
  // fraction is a multiple of 1/nb >= 2^-11, so truncating it gives the row, or one less when
  // gc is a multiple of nb; the remainder then equals nb and one step corrects it.
  int r = (int)((double)gc * inv_nb);
  int b = gc - r * nb;
  if (b >= nb) {
    ++r;
    b -= nb;
  }

  // 32 weight bytes of block b of row r (16-byte aligned: W and row_bytes are).
  const int4_t *src =
      reinterpret_cast<const int4_t *>(W + (int64_t)r * row_bytes + (int64_t)b * 32);
  int4_t raw[2];
  raw[0] = __builtin_nontemporal_load(src);
  raw[1] = __builtin_nontemporal_load(src + 1);
  float S = scale;
  if (BLK) S = grid[(int64_t)(r / 128) * grid_cols + b / 4];

  // v_i = e4m3 * S: the decode to f32 (scale 1.0) is exact, the product rounds once.
  float v[32];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw[h][j], 1.0f, false);
      const float2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw[h][j], 1.0f, true);
      v[16 * h + 4 * j + 0] = lo[0] * S;
      v[16 * h + 4 * j + 1] = lo[1] * S;
      v[16 * h + 4 * j + 2] = hi[0] * S;
      v[16 * h + 4 * j + 3] = hi[1] * S;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float d = amax / 127.0f;
  const _Float16 d16 = (_Float16)d;

  // Assemble the block in LDS: scale, then q pairs (a block starts 2-byte aligned).
  uint16_t *dst = out16 + threadIdx.x * (kBlk / 2);
  if (valid) {
    dst[0] = __builtin_bit_cast(uint16_t, d16);
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const int q0 = round_half_away(v[i] * id);
      const int q1 = round_half_away(v[i + 1] * id);
      dst[1 + i / 2] = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
    }
  }
  __syncthreads();

  const int nblk = total - g0 < kThreads ? total - g0 : kThreads;  // blocks of this workgroup
  if (store_mode == kStoreRows) {
    if (valid) {
      uint16_t *o = reinterpret_cast<uint16_t *>(Wq + (int64_t)r * q_row_bytes + (int64_t)b * kBlk);
#pragma unroll
      for (int k = 0; k < kBlk / 2; ++k) o[k] = dst[k];
    }
    return;
  }
  // Packed rows: the workgroup's nblk * 34 output bytes are contiguous from block g0.
  uint8_t *orun = Wq + (int64_t)g0 * kBlk;
  const int nbytes = nblk * kBlk;
  if (store_mode == kStoreWide) {
    // 16-byte aligned start (g0 * 34 is a multiple of 8704) and length (nblk % 8 == 0)
    for (int c = threadIdx.x; c < nbytes / 16; c += kThreads)
      *reinterpret_cast<int4_t *>(orun + 16 * c) = reinterpret_cast<const int4_t *>(out16)[c];
  } else {
    for (int c = threadIdx.x; c < nbytes / 2; c += kThreads)
      reinterpret_cast<uint16_t *>(orun)[c] = out16[c];
  }
}

}  // namespace

hipError_t launch_requant_q8_0(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                               int grid_cols, bool blk128, void *Wq, int64_t q_row_bytes,
                               int in_f, int out_f, hipStream_t s) {
  const int nb = in_f / 32;
  // Block numbers are int: launch at most 2^30 blocks at a time, in row ranges that start on a
  // 128-row grid tile.
  int64_t rows_per = (((int64_t)1 << 30) / nb) / 128 * 128;
  if (rows_per < 128) rows_per = 128;
  const double inv_nb = 1.0 / (double)nb;
  for (int64_t r0 = 0; r0 < out_f; r0 += rows_per) {
    const int rows = (int)(out_f - r0 < rows_per ? out_f - r0 : rows_per);
    const int total = rows * nb;
    const uint8_t *w = W + r0 * row_bytes;
    uint8_t *out = static_cast<uint8_t *>(Wq) + r0 * q_row_bytes;
    int mode = kStoreRows;
    if (q_row_bytes == (int64_t)nb * kBlk)
      mode = (reinterpret_cast<uintptr_t>(out) & 15) == 0 && total % 8 == 0 ? kStoreWide
                                                                            : kStorePacked;
    const dim3 g((unsigned)((total + kThreads - 1) / kThreads));
    if (blk128)
      hipLaunchKernelGGL(k_requant_q8_0<true>, g, dim3(kThreads), 0, s, w, row_bytes, 0.0f,
                         grid + (r0 / 128) * grid_cols, grid_cols, out, q_row_bytes, nb, total,
                         inv_nb, mode);
    else
      hipLaunchKernelGGL(k_requant_q8_0<false>, g, dim3(kThreads), 0, s, w, row_bytes, scale,
                         nullptr, 0, out, q_row_bytes, nb, total, inv_nb, mode);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace fp8gemv

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
// blocks per workgroup; a workgroup's 256 * 34 output bytes are contiguous in the row, so they
// are assembled in LDS and written back with coalesced 16-byte stores when the row layout
// allows it (in_f % 256 == 0, 16-byte aligned rows), 2-byte stores otherwise.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;   // blocks per workgroup
constexpr int kBlk = 34;        // Q8_0 block bytes

template <bool BLK>
__global__ __launch_bounds__(kThreads) void k_requant_q8_0(
    const uint8_t *__restrict__ W, int64_t row_bytes, float scale, const float *__restrict__ grid,
    int grid_cols, uint8_t *__restrict__ Wq, int64_t q_row_bytes, int in_f, bool wide_store) {
  __shared__ __align__(16) uint16_t out16[kThreads * kBlk / 2];
  const int nb = in_f / 32;
  const int r = blockIdx.x;
  const int b0 = blockIdx.y * kThreads;
  const int b = b0 + threadIdx.x;
  const int nblk = nb - b0 < kThreads ? nb - b0 : kThreads;  // blocks of this workgroup

  // 32 weight bytes of block b (zeros past the row).
  const rsrc_t wrs = buf_rsrc(W + (int64_t)r * row_bytes, (uint32_t)in_f);
  int4_t raw[2];
  raw[0] = buf_load16_stream(wrs, (uint32_t)b * 32);
  raw[1] = buf_load16_stream(wrs, (uint32_t)b * 32 + 16);
  float S = scale;
  if (BLK) {
    const rsrc_t grs = buf_rsrc(grid + (int64_t)(r / 128) * grid_cols, (uint32_t)grid_cols * 4);
    S = buf_load_f32(grs, (uint32_t)(b / 4) * 4);
  }

  // v_i = e4m3 * S: the decode to f16 (scale 1.0) and to f32 are exact, the product rounds once.
  float v[32];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[h][j], 1.0f, false);
      const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[h][j], 1.0f, true);
      v[16 * h + 4 * j + 0] = (float)lo[0] * S;
      v[16 * h + 4 * j + 1] = (float)lo[1] * S;
      v[16 * h + 4 * j + 2] = (float)hi[0] * S;
      v[16 * h + 4 * j + 3] = (float)hi[1] * S;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float d = amax / 127.0f;
  const _Float16 d16 = (_Float16)d;

  // Assemble the block in LDS: scale, then q pairs (a block starts 2-byte aligned).
  uint16_t *dst = out16 + threadIdx.x * (kBlk / 2);
  if (b < nb) {
    dst[0] = __builtin_bit_cast(uint16_t, d16);
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const int q0 = (int)roundf(v[i] * id);
      const int q1 = (int)roundf(v[i + 1] * id);
      dst[1 + i / 2] = (uint16_t)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
    }
  }
  __syncthreads();

  // Write the workgroup's nblk * 34 contiguous bytes of row r.
  uint8_t *orow = Wq + (int64_t)r * q_row_bytes + (int64_t)b0 * kBlk;
  const int nbytes = nblk * kBlk;
  if (wide_store) {
    // 16-byte aligned start (b0 * 34 is a multiple of 8704) and length (nblk % 8 == 0)
    for (int c = threadIdx.x; c < nbytes / 16; c += kThreads)
      *reinterpret_cast<int4_t *>(orow + 16 * c) = reinterpret_cast<const int4_t *>(out16)[c];
  } else {
    for (int c = threadIdx.x; c < nbytes / 2; c += kThreads)
      reinterpret_cast<uint16_t *>(orow)[c] = out16[c];
  }
}

}  // namespace

hipError_t launch_requant_q8_0(const uint8_t *W, int64_t row_bytes, float scale, const float *grid,
                               int grid_cols, bool blk128, void *Wq, int64_t q_row_bytes,
                               int in_f, int out_f, hipStream_t s) {
  const int nb = in_f / 32;
  const bool wide = in_f % 256 == 0 && q_row_bytes % 16 == 0 &&
                    (reinterpret_cast<uintptr_t>(Wq) & 15) == 0;
  const dim3 g(out_f, (nb + kThreads - 1) / kThreads);
  uint8_t *out = static_cast<uint8_t *>(Wq);
  if (blk128)
    hipLaunchKernelGGL(k_requant_q8_0<true>, g, dim3(kThreads), 0, s, W, row_bytes, 0.0f, grid,
                       grid_cols, out, q_row_bytes, in_f, wide);
  else
    hipLaunchKernelGGL(k_requant_q8_0<false>, g, dim3(kThreads), 0, s, W, row_bytes, scale,
                       nullptr, 0, out, q_row_bytes, in_f, wide);
  return hipGetLastError();
}

}  // namespace fp8gemv

// The activation producer: RMSNorm of an f32 row and its q8_1 quantisation.
//
// Source: docs.rs, memra-engine 0.125.0, src/bin/q8_fuse_gate.rs -- module doc and
// `run_shape`: the two-launch chain rms_norm(x, w, z, ncols, nrows, eps) -> quantize_q8_1(z)
// and the fused one-launch producer that still writes z and must give byte-identical z, qs
// and d.  Byte identity holds here by construction: the chain kernels and the fused kernel
// call the same device functions (row_scale for the RMS factor, z_value for z, quant_group
// for a 32-block) with the same workgroup shape, and quantisation of a block depends only on
// that block's 32 values.
//
// Parallel shape: one workgroup per (1024-column slice, row).  Every workgroup of a row
// computes the row's RMS factor itself from the whole row (same function, same order, so the
// same bits everywhere) and then normalises and quantises only its slice: no inter-workgroup
// communication, and a single row is spread over ceil(ncols / 1024) CUs.
//
// Numerics (this file is compiled with -ffp-contract=off):
//   ss  = sum_j x_j^2, every square exact in f64, accumulated as a double-double and rounded
//         once to f64, so ss is the correctly rounded sum except in vanishingly rare ties;
//   s   = 1 / sqrt(ss / ncols + eps)                        (f64, IEEE div and sqrt)
//   z_j = (float)(((double)x_j * (double)w_j) * s)          (x_j * w_j is exact in f64)
//   q8_1 per 32-block in f32: d = amax / 127, id = d ? 1 / d : 0, q = roundf(z * id).
//
// The second front end, silu(gate) * up -> q8_1 (the same page's main: the MoE expert-ff
// width 1536 is the activation fusion site still on the unfused chain), follows the same
// pattern: a chain (silu_mul_f32 then quantize_q8_1) and a fused kernel sharing the device
// function h_value, byte-identical by construction.  h_value in f64, rounded once to f32:
//   h_j = (float)((g_j / (1 + exp(-g_j))) * u_j)            (g, u widened exactly to f64)
//
// The third front end, the KDA gated norm (the same page names the KDA gated-norm site at the
// KDA qkv width, 64 heads x 128 head_dim, as still on the unfused chain; no formula is given,
// the rule is the output stage of a Kimi-delta-attention layer): per head of head_dim
// columns, the RMS factor of that head only, the gain indexed inside the head, then the
// sigmoid output gate, in f64 with one rounding to f32:
//   s_h = 1 / sqrt(sum_{j in h} o_j^2 / head_dim + eps)     (double-double sum, as above)
//   z_j = (float)((((double)o_j * w_{j mod head_dim}) * s_h) * (1 / (1 + exp(-g_j))))
// A head is head_dim / 4 consecutive lanes; its sum of squares is formed per quad by DPP
// (identical bits in all four lanes) and then over the head's quads in quad order from
// uniform lane reads.  Chain (gated_rms_norm_f32 then quantize_q8_1) and fused kernel call
// the same device functions, so they are byte-identical by construction.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kThreads = 256;            // 4 waves per row
constexpr int kColsPerPass = kThreads * 4;  // each thread owns 4 consecutive columns

// Exact sum and rounding error of a + b (Knuth's TwoSum; needs no contraction).
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ void dd_add(double &hi, double &lo, double ohi, double olo) {
  double s, e;
  two_sum(hi, ohi, s, e);
  hi = s;
  lo = (lo + olo) + e;
}

// A double moved between lanes by DPP (both 32-bit halves with the same control).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double lane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// 1 / sqrt(mean(x^2) + eps) for one row, computed by the whole workgroup; every thread
// returns the same value.  `red` is LDS scratch for 2 doubles per wave.  Inlined, so that the
// loads below stay in the kernel's own instruction stream.
__device__ __forceinline__ double row_scale(const float *__restrict__ x, int ncols, float eps,
                                            double *red) {
  double hi = 0.0, lo = 0.0;
  constexpr int kBatch = 8;  // loads issued together before they are accumulated
  // Batches of kBatch loads; the next batch is issued before the current one is accumulated,
  // so a long row costs one load latency, not one per batch.  Every thread runs the same
  // number of batches, and a load past the row reads zeros through the buffer resource's
  // range check, so there is no branch around any load and the compiler waits only for the
  // batch it uses.  A zero adds nothing (TwoSum of hi and 0 is exactly hi and 0), so the sum
  // is that of the row's own elements, in the same per-thread order.
  const rsrc_t xrs = buf_rsrc(x, (uint32_t)ncols * 4);
  auto load_batch = [&](float4 (&v)[kBatch], int base) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      v[u] = __builtin_bit_cast(float4, buf_load16(xrs, (uint32_t)(base + u * kColsPerPass) * 4));
  };
  const int nbatch = (ncols + kBatch * kColsPerPass - 1) / (kBatch * kColsPerPass);
  auto accumulate = [&](const float4 (&v)[kBatch]) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float e4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double p = (double)e4[i] * (double)e4[i];
        double s, e;
        two_sum(hi, p, s, e);
        hi = s;
        lo += e;
      }
    }
  };
  // Two buffers used in turn (no register copies between batches, which would make the
  // compiler wait for the batch just issued).  Past the last batch every offset lies past
  // the row: zeros, and no memory traffic.
  const int t4 = threadIdx.x * 4;
  float4 va[kBatch], vb[kBatch];
  load_batch(va, t4);
  for (int b = 0; b < nbatch; b += 2) {
    load_batch(vb, t4 + (b + 1) * kBatch * kColsPerPass);
    accumulate(va);
    if (b + 1 >= nbatch) break;
    load_batch(va, t4 + (b + 2) * kBatch * kColsPerPass);
    accumulate(vb);
  }
  // Across the wave: DPP within each row of 16 lanes (quad swaps, then rotations by 4 and
  // 8), then the four row sums from lanes 0, 16, 32, 48 added in that fixed order.  Lanes of
  // a row may differ in the last bits after the rotations; only the fixed lanes are read.
  dd_add(hi, lo, dpp_f64<kQuadPerm1032>(hi), dpp_f64<kQuadPerm1032>(lo));
  dd_add(hi, lo, dpp_f64<kQuadPerm2301>(hi), dpp_f64<kQuadPerm2301>(lo));
  dd_add(hi, lo, dpp_f64<kRowRor4>(hi), dpp_f64<kRowRor4>(lo));
  dd_add(hi, lo, dpp_f64<kRowRor8>(hi), dpp_f64<kRowRor8>(lo));
  double whi = lane_f64(hi, 0), wlo = lane_f64(lo, 0);
  double h1 = lane_f64(hi, 16), l1 = lane_f64(lo, 16);
  double h2 = lane_f64(hi, 32), l2 = lane_f64(lo, 32);
  double h3 = lane_f64(hi, 48), l3 = lane_f64(lo, 48);
  dd_add(whi, wlo, h1, l1);
  dd_add(h2, l2, h3, l3);
  dd_add(whi, wlo, h2, l2);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    red[2 * wave] = whi;
    red[2 * wave + 1] = wlo;
  }
  __syncthreads();
  double thi = red[0], tlo = red[1];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) dd_add(thi, tlo, red[2 * w], red[2 * w + 1]);
  const double ss = thi + tlo;
  return 1.0 / sqrt(ss / (double)ncols + (double)eps);
}

__device__ __forceinline__ float z_value(float x, float w, double s) {
  return (float)(((double)x * (double)w) * s);
}

// SiLU-gated product of one column, in f64 with a single rounding to f32.
__device__ __forceinline__ float h_value(float g, float u) {
  const double gd = (double)g;
  const double sg = gd / (1.0 + exp(-gd));
  return (float)(sg * (double)u);
}

// q8_1 of one 32-block held by 8 consecutive lanes (4 values each).  All 8 lanes of a group
// must execute this together.  Returns the 4 int8 codes packed little-endian; the block
// scale is returned through d_out (same value on all 8 lanes).
__device__ __forceinline__ uint32_t quant_group(const float z[4], float &d_out) {
  float amax = fmaxf(fmaxf(fabsf(z[0]), fabsf(z[1])), fmaxf(fabsf(z[2]), fabsf(z[3])));
  // max over the 8 lanes (exact in any order): quad swaps, then the mirror within 8 lanes
  amax = fmaxf(amax, dpp_f32<kQuadPerm1032>(amax));
  amax = fmaxf(amax, dpp_f32<kQuadPerm2301>(amax));
  amax = fmaxf(amax, dpp_f32<kRowHalfMirror>(amax));
  const float d = amax / 127.0f;
  const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = (int)roundf(z[i] * id);
    packed |= (uint32_t)(uint8_t)(int8_t)q << (8 * i);
  }
  d_out = d;
  return packed;
}

// 1 / sqrt(mean over the head of o^2 + eps) for the head that holds this lane's 4 columns.
// Heads are D / 4 consecutive lanes (D in {32, 64, 128, 256}, so a head never leaves its wave);
// every lane of the wave must call this together.
template <int D>
__device__ double head_scale(const float o[4], float eps) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head_dim");
  constexpr int kQuadsPerHead = D / 16;
  constexpr int kHeadsPerWave = kWave * 4 / D;
  double hi = 0.0, lo = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double p = (double)o[i] * (double)o[i];
    double s, e;
    two_sum(hi, p, s, e);
    hi = s;
    lo += e;
  }
  // quad sums: both operands of every step are the same two values in every lane of the
  // quad (added in either order, TwoSum gives the same sum and the same exact error)
  dd_add(hi, lo, dpp_f64<kQuadPerm1032>(hi), dpp_f64<kQuadPerm1032>(lo));
  dd_add(hi, lo, dpp_f64<kQuadPerm2301>(hi), dpp_f64<kQuadPerm2301>(lo));
  const int head = (int)(threadIdx.x % kWave) / (D / 4);
  double shi = 0.0, slo = 0.0;
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    double thi = lane_f64(hi, 4 * h * kQuadsPerHead), tlo = lane_f64(lo, 4 * h * kQuadsPerHead);
#pragma unroll
    for (int k = 1; k < kQuadsPerHead; ++k)
      dd_add(thi, tlo, lane_f64(hi, 4 * (h * kQuadsPerHead + k)),
             lane_f64(lo, 4 * (h * kQuadsPerHead + k)));
    shi = head == h ? thi : shi;
    slo = head == h ? tlo : slo;
  }
  const double ss = shi + slo;
  return 1.0 / sqrt(ss / (double)D + (double)eps);
}

// Gated z of one column, in f64 with a single rounding to f32.
__device__ __forceinline__ float gated_z(float o, float w, float g, double s) {
  const double gate = 1.0 / (1.0 + exp(-(double)g));
  return (float)((((double)o * (double)w) * s) * gate);
}

// This thread's 4 columns of the gated norm (zeros, and no loads, past ncols).
template <int D>
__device__ __forceinline__ void gated_columns(const float *__restrict__ o,
                                              const float *__restrict__ g,
                                              const float *__restrict__ w, int64_t row, int j,
                                              int ncols, float eps, float z[4]) {
  float ov[4] = {0.f, 0.f, 0.f, 0.f}, gv[4] = {0.f, 0.f, 0.f, 0.f}, wv[4] = {0.f, 0.f, 0.f, 0.f};
  if (j < ncols) {
    const float4 a = *reinterpret_cast<const float4 *>(o + row * ncols + j);
    const float4 b = *reinterpret_cast<const float4 *>(g + row * ncols + j);
    const float4 c = *reinterpret_cast<const float4 *>(w + j % D);
    ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
    gv[0] = b.x; gv[1] = b.y; gv[2] = b.z; gv[3] = b.w;
    wv[0] = c.x; wv[1] = c.y; wv[2] = c.z; wv[3] = c.w;
  }
  const double s = head_scale<D>(ov, eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = gated_z(ov[i], wv[i], gv[i], s);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_gated_rms_norm(const float *__restrict__ o,
                                                             const float *__restrict__ g,
                                                             const float *__restrict__ w,
                                                             float *__restrict__ z, int ncols,
                                                             float eps) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  float zv[4];
  gated_columns<D>(o, g, w, row, j, ncols, eps, zv);
  if (j < ncols)
    *reinterpret_cast<float4 *>(z + row * ncols + j) = make_float4(zv[0], zv[1], zv[2], zv[3]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void k_gated_rmsnorm_q8_1(
    const float *__restrict__ o, const float *__restrict__ g, const float *__restrict__ w,
    float *__restrict__ z, int8_t *__restrict__ qs, float *__restrict__ d, int ncols, float eps) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  const bool live = j < ncols;  // whole 8-lane groups are live or not (ncols % 32 == 0)
  float zv[4];
  gated_columns<D>(o, g, w, row, j, ncols, eps, zv);
  if (live && z != nullptr)
    *reinterpret_cast<float4 *>(z + row * ncols + j) = make_float4(zv[0], zv[1], zv[2], zv[3]);
  float db;
  const uint32_t packed = quant_group(zv, db);
  if (live) {
    *reinterpret_cast<uint32_t *>(qs + row * ncols + j) = packed;
    if ((threadIdx.x & 7) == 0) d[row * (ncols / 32) + j / 32] = db;
  }
}

__global__ __launch_bounds__(kThreads) void k_rms_norm(const float *__restrict__ x,
                                                       const float *__restrict__ w,
                                                       float *__restrict__ z, int ncols,
                                                       float eps) {
  __shared__ double red[2 * kThreads / kWave];
  const int64_t row = blockIdx.y;
  const float *xr = x + row * ncols;
  const double s = row_scale(xr, ncols, eps, red);
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  if (j < ncols) {
    const float4 xv = *reinterpret_cast<const float4 *>(xr + j);
    const float4 wv = *reinterpret_cast<const float4 *>(w + j);
    float4 zv;
    zv.x = z_value(xv.x, wv.x, s);
    zv.y = z_value(xv.y, wv.y, s);
    zv.z = z_value(xv.z, wv.z, s);
    zv.w = z_value(xv.w, wv.w, s);
    *reinterpret_cast<float4 *>(z + row * ncols + j) = zv;
  }
}

// One workgroup per (1024-column slice, row).
__global__ __launch_bounds__(kThreads) void k_quantize_q8_1(const float *__restrict__ z,
                                                            int8_t *__restrict__ qs,
                                                            float *__restrict__ d, int ncols) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  const bool live = j < ncols;  // whole 8-lane groups are live or not (ncols % 32 == 0)
  float zv[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float4 v = *reinterpret_cast<const float4 *>(z + row * ncols + j);
    zv[0] = v.x; zv[1] = v.y; zv[2] = v.z; zv[3] = v.w;
  }
  float db;
  const uint32_t packed = quant_group(zv, db);
  if (live) {
    *reinterpret_cast<uint32_t *>(qs + row * ncols + j) = packed;
    if ((threadIdx.x & 7) == 0) d[row * (ncols / 32) + j / 32] = db;
  }
}

__global__ __launch_bounds__(kThreads) void k_rmsnorm_q8_1(const float *__restrict__ x,
                                                           const float *__restrict__ w,
                                                           float *__restrict__ z,
                                                           int8_t *__restrict__ qs,
                                                           float *__restrict__ d, int ncols,
                                                           float eps) {
  __shared__ double red[2 * kThreads / kWave];
  const int64_t row = blockIdx.y;
  const float *xr = x + row * ncols;
  const double s = row_scale(xr, ncols, eps, red);
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  const bool live = j < ncols;  // whole 8-lane groups are live or not (ncols % 32 == 0)
  float zv[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float4 xv = *reinterpret_cast<const float4 *>(xr + j);
    const float4 wv = *reinterpret_cast<const float4 *>(w + j);
    zv[0] = z_value(xv.x, wv.x, s);
    zv[1] = z_value(xv.y, wv.y, s);
    zv[2] = z_value(xv.z, wv.z, s);
    zv[3] = z_value(xv.w, wv.w, s);
    if (z != nullptr)
      *reinterpret_cast<float4 *>(z + row * ncols + j) = make_float4(zv[0], zv[1], zv[2], zv[3]);
  }
  float db;
  const uint32_t packed = quant_group(zv, db);
  if (live) {
    *reinterpret_cast<uint32_t *>(qs + row * ncols + j) = packed;
    if ((threadIdx.x & 7) == 0) d[row * (ncols / 32) + j / 32] = db;
  }
}

__global__ __launch_bounds__(kThreads) void k_silu_mul(const float *__restrict__ g,
                                                       const float *__restrict__ u,
                                                       float *__restrict__ h, int ncols) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  if (j < ncols) {
    const float4 gv = *reinterpret_cast<const float4 *>(g + row * ncols + j);
    const float4 uv = *reinterpret_cast<const float4 *>(u + row * ncols + j);
    *reinterpret_cast<float4 *>(h + row * ncols + j) =
        make_float4(h_value(gv.x, uv.x), h_value(gv.y, uv.y), h_value(gv.z, uv.z),
                    h_value(gv.w, uv.w));
  }
}

__global__ __launch_bounds__(kThreads) void k_silu_mul_q8_1(const float *__restrict__ g,
                                                            const float *__restrict__ u,
                                                            float *__restrict__ h,
                                                            int8_t *__restrict__ qs,
                                                            float *__restrict__ d, int ncols) {
  const int64_t row = blockIdx.y;
  const int j = blockIdx.x * kColsPerPass + threadIdx.x * 4;
  const bool live = j < ncols;  // whole 8-lane groups are live or not (ncols % 32 == 0)
  float hv[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    const float4 gv = *reinterpret_cast<const float4 *>(g + row * ncols + j);
    const float4 uv = *reinterpret_cast<const float4 *>(u + row * ncols + j);
    hv[0] = h_value(gv.x, uv.x);
    hv[1] = h_value(gv.y, uv.y);
    hv[2] = h_value(gv.z, uv.z);
    hv[3] = h_value(gv.w, uv.w);
    if (h != nullptr)
      *reinterpret_cast<float4 *>(h + row * ncols + j) = make_float4(hv[0], hv[1], hv[2], hv[3]);
  }
  float db;
  const uint32_t packed = quant_group(hv, db);
  if (live) {
    *reinterpret_cast<uint32_t *>(qs + row * ncols + j) = packed;
    if ((threadIdx.x & 7) == 0) d[row * (ncols / 32) + j / 32] = db;
  }
}

}  // namespace

hipError_t launch_silu_mul(const float *g, const float *u, float *h, int ncols, int nrows,
                           hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  hipLaunchKernelGGL(k_silu_mul, grid, dim3(kThreads), 0, s, g, u, h, ncols);
  return hipGetLastError();
}

hipError_t launch_silu_mul_q8_1(const float *g, const float *u, float *h, int8_t *qs, float *d,
                                int ncols, int nrows, hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  hipLaunchKernelGGL(k_silu_mul_q8_1, grid, dim3(kThreads), 0, s, g, u, h, qs, d, ncols);
  return hipGetLastError();
}

hipError_t launch_gated_rms_norm(const float *o, const float *g, const float *w, float *z,
                                 int ncols, int head_dim, int nrows, float eps, hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(k_gated_rms_norm<32>, grid, dim3(kThreads), 0, s, o, g, w, z, ncols, eps); break;
    case 64: hipLaunchKernelGGL(k_gated_rms_norm<64>, grid, dim3(kThreads), 0, s, o, g, w, z, ncols, eps); break;
    case 128: hipLaunchKernelGGL(k_gated_rms_norm<128>, grid, dim3(kThreads), 0, s, o, g, w, z, ncols, eps); break;
    case 256: hipLaunchKernelGGL(k_gated_rms_norm<256>, grid, dim3(kThreads), 0, s, o, g, w, z, ncols, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm_q8_1(const float *o, const float *g, const float *w, float *z,
                                     int8_t *qs, float *d, int ncols, int head_dim, int nrows,
                                     float eps, hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(k_gated_rmsnorm_q8_1<32>, grid, dim3(kThreads), 0, s, o, g, w, z, qs, d, ncols, eps); break;
    case 64: hipLaunchKernelGGL(k_gated_rmsnorm_q8_1<64>, grid, dim3(kThreads), 0, s, o, g, w, z, qs, d, ncols, eps); break;
    case 128: hipLaunchKernelGGL(k_gated_rmsnorm_q8_1<128>, grid, dim3(kThreads), 0, s, o, g, w, z, qs, d, ncols, eps); break;
    case 256: hipLaunchKernelGGL(k_gated_rmsnorm_q8_1<256>, grid, dim3(kThreads), 0, s, o, g, w, z, qs, d, ncols, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rms_norm(const float *x, const float *w, float *z, int ncols, int nrows,
                           float eps, hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  hipLaunchKernelGGL(k_rms_norm, grid, dim3(kThreads), 0, s, x, w, z, ncols, eps);
  return hipGetLastError();
}

hipError_t launch_quantize_q8_1(const float *z, int8_t *qs, float *d, int nrows, int ncols,
                                hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  hipLaunchKernelGGL(k_quantize_q8_1, grid, dim3(kThreads), 0, s, z, qs, d, ncols);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_q8_1(const float *x, const float *w, float *z, int8_t *qs, float *d,
                               int ncols, int nrows, float eps, hipStream_t s) {
  const dim3 grid((ncols + kColsPerPass - 1) / kColsPerPass, nrows);
  hipLaunchKernelGGL(k_rmsnorm_q8_1, grid, dim3(kThreads), 0, s, x, w, z, qs, d, ncols, eps);
  return hipGetLastError();
}

}  // namespace fp8gemv

// Measurement aid: stream a byte range from HBM the way the GEMVs stream weights (one 16-byte
// non-temporal load per lane, 1 KiB per wave-wide load, 8 loads in flight per lane, 4-wave
// workgroups, 64 VGPRs or fewer) and do nothing with the data but fold it into one word.  Its
// duration over a cold range is the achievable read time that the GEMVs are compared with.
#include "common.hpp"

namespace fp8gemv {
namespace {

constexpr int kWaves = 4;
constexpr int kLoads = 8;                        // KiB per wave
constexpr int64_t kBytesPerWg = kWaves * kLoads * 1024;

__global__ __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_read_bytes(const uint8_t *__restrict__ p, int64_t bytes, uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x % kWave;
  const int64_t base = (int64_t)blockIdx.x * kBytesPerWg + (int64_t)wave_id() * kLoads * 1024;
  const int64_t left = bytes - base;
  const rsrc_t rs = buf_rsrc(p + (base < bytes ? base : 0),
                             left <= 0 ? 0u : (uint32_t)(left < kLoads * 1024 ? left : kLoads * 1024));
  int4_t v[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) v[u] = buf_load16_stream(rs, (uint32_t)(u * 1024 + lane * 16));
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kLoads; ++u) x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  // A data-dependent store that never happens in practice keeps the loads alive.
  if (x == 0x9E3779B9u && lane == 0) sink[0] = x;
}

}  // namespace

hipError_t launch_read_bytes(const void *p, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t wgs = (bytes + kBytesPerWg - 1) / kBytesPerWg;
  hipLaunchKernelGGL(k_read_bytes, dim3((unsigned)wgs), dim3(kWaves * kWave), 0, s,
                     static_cast<const uint8_t *>(p), bytes, sink);
  return hipGetLastError();
}

}  // namespace fp8gemv

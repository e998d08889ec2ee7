// Measurement helpers: the device's CU count and clock (for the derived bf16
// MFMA peak), and a dense bf16 MFMA throughput probe that shows what the
// matrix cores sustain on given operand data under the chip's power limit.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ra.h"
#include "ra_device.h"

namespace {

constexpr int kProbeWaves = 8;        // two waves per SIMD, as in the attention kernels
constexpr int kProbeLdsBytes = 96 * 1024;  // more than half the CU's LDS: one block per CU

// Each wave loads 8 A and 8 B operand registers from `ops` (16 x 64 lanes x
// 16 bytes) once, then issues `iters` x 16 independent-chain 32x32x16 bf16
// MFMAs into four accumulators.  The first wave of block 0 records the shader
// clock (s_memtime) and the 100 MHz reference clock (s_memrealtime) around its
// loop into clocks[0..1] with a vector store.
__global__ __launch_bounds__(64 * kProbeWaves, 1) void mfma_probe_kernel(const ra::u32x4* __restrict__ ops,
                                                                         float* __restrict__ sink,
                                                                         unsigned long long* __restrict__ clocks,
                                                                         int iters) {
  __shared__ uint8_t pad[kProbeLdsBytes];
  const int lane = threadIdx.x & 63;
  ra::u32x4 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = ops[(2 * j) * 64 + lane];
    b[j] = ops[(2 * j + 1) * 64 + lane];
  }
  ra::f32x16 acc[4] = {};
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j & 3] = ra::mfma32(a[j & 7], b[(j + (j >> 3)) & 7], acc[j & 3]);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[k][i];
  pad[threadIdx.x] = (uint8_t)iters;  // keeps the LDS reservation (and so one block per CU)
  __syncthreads();
  if (pad[(threadIdx.x + 1) % (64 * kProbeWaves)] == 0xFF && iters < 0) s += 1.f;
  sink[(size_t)blockIdx.x * 64 * kProbeWaves + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = c1 - c0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

int ra_device_info(int* cu_count, int* max_clock_khz) {
  if (!cu_count || !max_clock_khz) return RA_ERR_NULL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cu_count, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, dev);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

int ra_mfma_probe(const void* operands, float* sink, unsigned long long* clocks, int blocks, int iters,
                  void* stream) {
  if (!operands || !sink || !clocks) return RA_ERR_NULL;
  if (blocks < 1 || iters < 1) return RA_ERR_SHAPE;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(64 * kProbeWaves), 0, static_cast<hipStream_t>(stream),
                     static_cast<const ra::u32x4*>(operands), sink, clocks, iters);
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

}  // extern "C"

// Row-wise kernels: the standalone log-sum-exp merge of a ring-step partial,
// the backward's per-row term D = rowsum(dO * O), and a zero fill.
#include "ra_device.h"
#include "ra_grid.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();

// One row per LPR = D/4 lanes (one float4 each); a wave covers 64/LPR rows.
// Every lane of a row reads the old lse before any lane writes the new one:
// a row lives in one wave, whose lanes execute the load before the store.
//
// With lse' = ln(e^lse + e^lse_p): o <- e^(lse-lse') o + e^(lse_p-lse') o_p
// -- the online-softmax update of partial results ("Training Long-Context
// Models Without OOM: Ring Attention", "Ring Attention Demystified").
template <int D>
__global__ __launch_bounds__(kRowThreads) void lse_merge_kernel(float* __restrict__ o, float* __restrict__ lse,
                                                                const float* __restrict__ op,
                                                                const float* __restrict__ lp, int rows) {
  constexpr int LPR = D / 4;
  // Grid-stride over rows * LPR items (up to 2^36): 64-bit indices.
  const long long n = (long long)rows * LPR;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x; gid < n; gid += stride) {
    const int row = (int)(gid / LPR), c = (int)(gid % LPR);
    const float la = lse[row], lb = lp[row];
    const float M = fmaxf(la, lb);
    float wa = 0.f, wb = 0.f, lnew = kNegInf;
    if (M != kNegInf) {
      const float ea = expf(la - M), eb = expf(lb - M);
      const float tot = ea + eb;
      lnew = M + logf(tot);
      wa = ea / tot;
      wb = eb / tot;
    }
    const size_t off = (size_t)row * D + c * 4;
    const f32x4 a = *reinterpret_cast<const f32x4*>(o + off);
    const f32x4 b = *reinterpret_cast<const f32x4*>(op + off);
    // A zero weight must not turn an inf/nan-free zero partial into nan.
    f32x4 r;
    r[0] = (wa != 0.f ? wa * a[0] : 0.f) + (wb != 0.f ? wb * b[0] : 0.f);
    r[1] = (wa != 0.f ? wa * a[1] : 0.f) + (wb != 0.f ? wb * b[1] : 0.f);
    r[2] = (wa != 0.f ? wa * a[2] : 0.f) + (wb != 0.f ? wb * b[2] : 0.f);
    r[3] = (wa != 0.f ? wa * a[3] : 0.f) + (wb != 0.f ? wb * b[3] : 0.f);
    *reinterpret_cast<f32x4*>(o + off) = r;
    // The row's lanes sit in one wave and one loop trip (LPR divides the
    // stride), and each reads lse before any of them writes it.
    if (c == 0) lse[row] = lnew;
  }
}

// out[row] = -D[row], D[row] = sum_d dO[row, d] * O[row, d]; 32 lanes per row
// (D = 128: 4 values per lane; D = 64: 2), butterfly sum over the 32 lanes.
// The key kernel starts its dP accumulators at -D, which yields dP - D with
// no vector work; the dq kernel negates it back.  Also the row's lse
// in base 2, lse * log2(e), with -inf (a row that saw no key) mapped to +inf
// so that exp2(s - lse2) is 0 for it.
template <int D>
__global__ __launch_bounds__(kRowThreads) void rowdot_kernel(const uint16_t* __restrict__ dO,
                                                             const float* __restrict__ o,
                                                             const float* __restrict__ lse,
                                                             float* __restrict__ out, float* __restrict__ lse2,
                                                             int rows) {
  constexpr int VPL = D / 32;
  // Grid-stride over rows * 32 items (up to 2^36): 64-bit indices.  The
  // stride is a multiple of 64, so a row's 32 lanes stay in one wave and the
  // wave's trip count is uniform (the butterfly needs every lane).
  const long long n = (long long)rows * 32;
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long first = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long wave_first = first & ~63LL;
  for (long long base = wave_first; base < n; base += stride) {
    const long long gid = base + (first & 63);
    const bool ok = gid < n;
    const int row = (int)(gid >> 5), c = (int)(gid & 31);
    float acc = 0.f;
    if (ok) {
      const size_t off = (size_t)row * D + c * VPL;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const uint32_t bits = (uint32_t)dO[off + i] << 16;
        acc += __builtin_bit_cast(float, bits) * o[off + i];
      }
    }
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 32);
    if (ok && c == 0) {
      out[row] = -acc;
      const float l2 = lse[row] * kLog2e;
      lse2[row] = (l2 == -__builtin_inff()) ? __builtin_inff() : l2;
    }
  }
}

__global__ __launch_bounds__(kRowThreads) void zero_kernel(float* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

}  // namespace

hipError_t launch_lse_merge(float* o, float* lse, const float* op, const float* lp, int rows, int d,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(row_grid_blocks((uint64_t)rows * (d / 4))), block(kRowThreads);
  if (d == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, o, lse, op, lp, rows);
  else if (d == 64)
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, o, lse, op, lp, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_rowdot(const uint16_t* dO, const float* o, const float* lse, float* D, float* lse2,
                             int rows, int d, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid(row_grid_blocks((uint64_t)rows * 32)), block(kRowThreads);
  if (d == 128)
    hipLaunchKernelGGL(rowdot_kernel<128>, grid, block, 0, stream, dO, o, lse, D, lse2, rows);
  else if (d == 64)
    hipLaunchKernelGGL(rowdot_kernel<64>, grid, block, 0, stream, dO, o, lse, D, lse2, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(row_grid_blocks(n)), dim3(kRowThreads), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace ra

// Backward of one ring step against one KV chunk.
//
// The pages give no backward; this is the textbook softmax-attention gradient
// with the probabilities recomputed from the final log-sum-exp of the forward
// walk (so no merge is needed in the backward):
//   P = exp(scale q k^T - lse), dP = dO v^T, dS = P (dP - D), D = rowsum(dO o),
//   dq += scale dS k,  dk += scale dS^T q,  dv += P^T dO.
//
// Two kernels per step, neither with atomics (results are deterministic):
//  * dq kernel -- a block owns 128 query rows (32 per wave, Q^T and dO^T in
//    registers as MFMA B operands, like the forward) and streams 64-key tiles
//    of K, V (row-major LDS tiles, A operands) and K^T (transposed LDS tile).
//    Scores are computed transposed (S^T = K Q^T, dP^T = V dO^T), so lse and
//    D are per-lane scalars and dS^T feeds dq^T += K^T dS^T directly.
//  * dk/dv kernel -- a block owns 128 keys of the chunk (32 per wave, K and V
//    in registers as B operands) and streams 64-query tiles of Q, dO
//    (row-major) and Q^T, dO^T (transposed).  Here S = Q K^T has a lane per
//    key, so P and dS feed dv^T += dO^T P and dk^T += Q^T dS directly; lse and
//    D of the tile's queries come from LDS.
// The price of avoiding atomics is recomputing S and dP in both kernels.
#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// Per-thread staging of one 64-token tile: item `it` holds tokens
// 4*kq .. 4*kq+3, features 8*dc .. 8*dc+7.
template <int D>
struct TileItems {
  static constexpr int kItems = (D / 8) * (kTileTokens / 4);
  static constexpr int kPerThread = (kItems + 255) / 256;
};

template <int D>
__device__ __forceinline__ void load_items(u32x4 (&r)[TileItems<D>::kPerThread][4], const uint16_t* base,
                                           int t0, int n, int tid) {
#pragma unroll
  for (int i = 0; i < TileItems<D>::kPerThread; ++i) {
    const int it = tid + i * 256;
    if (it < TileItems<D>::kItems) {
      const int dc = it % (D / 8), kq = it / (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = t0 + kq * 4 + rr;
        r[i][rr] = (tok < n) ? ld16(base + (size_t)tok * D + dc * 8) : u32x4{0, 0, 0, 0};
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void store_items_rows(uint8_t* tile, const u32x4 (&r)[TileItems<D>::kPerThread][4],
                                                 int tid) {
#pragma unroll
  for (int i = 0; i < TileItems<D>::kPerThread; ++i) {
    const int it = tid + i * 256;
    if (it < TileItems<D>::kItems) {
      const int dc = it % (D / 8), kq = it / (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *reinterpret_cast<u32x4*>(tile + row_off<D>(kq * 4 + rr, dc)) = r[i][rr];
    }
  }
}

template <int D>
__device__ __forceinline__ void store_items_tr(uint8_t* tile, const u32x4 (&r)[TileItems<D>::kPerThread][4],
                                               int tid) {
#pragma unroll
  for (int i = 0; i < TileItems<D>::kPerThread; ++i) {
    const int it = tid + i * 256;
    if (it < TileItems<D>::kItems) store_tr4x8(tile, it % (D / 8), it / (D / 8), r[i]);
  }
}

// ---------------------------------------------------------------------------
// dq kernel.
// ---------------------------------------------------------------------------
template <int D, bool DIAG>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                                     const uint16_t* __restrict__ vg, const uint16_t* __restrict__ dog,
                                                     const float* __restrict__ lseg, const float* __restrict__ Dg,
                                                     float* __restrict__ dqg, int Sq, int Sk, int n_qtiles,
                                                     int total_tiles, float scale_log2, float scale) {
  constexpr int BR = 128, BC = kTileTokens, NKS = D / 16, NDB = D / 32, NKB = BC / 32;
  constexpr int TB = BC * D * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[3 * TB];
  uint8_t* const ks = smem;
  uint8_t* const vs = smem + TB;
  uint8_t* const kts = smem + 2 * TB;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int t = xcd_remap(blockIdx.x, total_tiles);
  const int bh = t / n_qtiles;
  int qt = t - bh * n_qtiles;
  if (DIAG) qt = n_qtiles - 1 - qt;
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 32;
  const int qq = qw0 + l32;

  const uint16_t* __restrict__ kp = kg + (size_t)bh * Sk * D;
  const uint16_t* __restrict__ vp = vg + (size_t)bh * Sk * D;
  u32x4 qf[NKS], df[NKS];
  {
    const uint16_t* qrow = qg + ((size_t)bh * Sq + qq) * D;
    const uint16_t* drow = dog + ((size_t)bh * Sq + qq) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[s] = (qq < Sq) ? ld16(qrow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
      df[s] = (qq < Sq) ? ld16(drow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
  }
  float lse2 = kPosInf, Dq = 0.f;
  if (qq < Sq) {
    lse2 = lseg[(size_t)bh * Sq + qq] * kLog2e;
    if (lse2 == kNegInf) lse2 = kPosInf;  // a row that saw no key has P = 0
    Dq = Dg[(size_t)bh * Sq + qq];
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;

  u32x4 kr[TileItems<D>::kPerThread][4], vr[TileItems<D>::kPerThread][4];
  load_items<D>(kr, kp, 0, Sk, tid);
  load_items<D>(vr, vp, 0, Sk, tid);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * BC;
    __syncthreads();
    store_items_rows<D>(ks, kr, tid);
    store_items_tr<D>(kts, kr, tid);
    store_items_rows<D>(vs, vr, tid);
    __syncthreads();
    if (tile + 1 < ntiles) {
      load_items<D>(kr, kp, k0 + BC, Sk, tid);
      load_items<D>(vr, vp, k0 + BC, Sk, tid);
    }
    if (DIAG && k0 > qw0 + 31) continue;

    f32x16 s_[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s_[kb][i] = 0.f;
        dp[kb][i] = 0.f;
      }
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(ks + row_off<D>(kb * 32 + l32, s * 2 + g));
        const u32x4 va = *reinterpret_cast<const u32x4*>(vs + row_off<D>(kb * 32 + l32, s * 2 + g));
        s_[kb] = mfma32(ka, qf[s], s_[kb]);
        dp[kb] = mfma32(va, df[s], dp[kb]);
      }
    const bool need_mask = (k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s_[kb][i], scale_log2, -lse2));
        if (need_mask) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= Sk || (DIAG && key > qq)) p = 0.f;
        }
        s_[kb][i] = p * (dp[kb][i] - Dq);  // dS^T
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 b = pack8(s_[kb], 8 * h);
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma32(ld_tr(kts, db * 32 + l32, kb, h, g), b, acc[db]);
      }
  }

  if (qq < Sq) {
    float* row = dqg + ((size_t)bh * Sq + qq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = row + db * 32 + 8 * j + 4 * g;
        f32x4 val = {acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale, acc[db][4 * j + 2] * scale,
                     acc[db][4 * j + 3] * scale};
        val += *reinterpret_cast<const f32x4*>(dst);
        *reinterpret_cast<f32x4*>(dst) = val;
      }
  }
}

// ---------------------------------------------------------------------------
// dk/dv kernel.
// ---------------------------------------------------------------------------
template <int D, bool DIAG>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                                       const uint16_t* __restrict__ vg, const uint16_t* __restrict__ dog,
                                                       const float* __restrict__ lseg, const float* __restrict__ Dg,
                                                       float* __restrict__ dkg, float* __restrict__ dvg, int Sq, int Sk,
                                                       int n_ktiles, int total_tiles, float scale_log2, float scale) {
  constexpr int BK = 128, BQ = kTileTokens, NKS = D / 16, NDB = D / 32, NQB = BQ / 32;
  constexpr int TB = BQ * D * 2;
  __shared__ __attribute__((aligned(16))) uint8_t smem[4 * TB + 2 * BQ * 4];
  uint8_t* const qs = smem;
  uint8_t* const dos = smem + TB;
  uint8_t* const qts = smem + 2 * TB;
  uint8_t* const dots = smem + 3 * TB;
  float* const lse_s = reinterpret_cast<float*>(smem + 4 * TB);
  float* const d_s = lse_s + BQ;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int t = xcd_remap(blockIdx.x, total_tiles);
  const int bh = t / n_ktiles;
  const int kt = t - bh * n_ktiles;  // low key tiles see the most queries: they go first
  const int kb0 = kt * BK;
  const int kw0 = kb0 + wave * 32;
  const int kk = kw0 + l32;

  const uint16_t* __restrict__ qp = qg + (size_t)bh * Sq * D;
  const uint16_t* __restrict__ dp_ = dog + (size_t)bh * Sq * D;
  const float* __restrict__ lp = lseg + (size_t)bh * Sq;
  const float* __restrict__ Dp = Dg + (size_t)bh * Sq;

  u32x4 kf[NKS], vf[NKS];
  {
    const uint16_t* krow = kg + ((size_t)bh * Sk + kk) * D;
    const uint16_t* vrow = vg + ((size_t)bh * Sk + kk) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kf[s] = (kk < Sk) ? ld16(krow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
      vf[s] = (kk < Sk) ? ld16(vrow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dk[db][i] = 0.f;
      dv[db][i] = 0.f;
    }

  const int qstart = DIAG ? (kb0 / BQ) * BQ : 0;
  const int ntiles = (Sq > qstart) ? (Sq - qstart + BQ - 1) / BQ : 0;

  u32x4 qr[TileItems<D>::kPerThread][4], dr[TileItems<D>::kPerThread][4];
  float lr = kPosInf, dr1 = 0.f;
  auto load_q = [&](int q0) {
    load_items<D>(qr, qp, q0, Sq, tid);
    load_items<D>(dr, dp_, q0, Sq, tid);
    if (tid < BQ) {
      const int qi = q0 + tid;
      lr = kPosInf;
      dr1 = 0.f;
      if (qi < Sq) {
        lr = lp[qi] * kLog2e;
        if (lr == kNegInf) lr = kPosInf;
        dr1 = Dp[qi];
      }
    }
  };
  if (ntiles > 0) load_q(qstart);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int q0 = qstart + tile * BQ;
    __syncthreads();
    store_items_rows<D>(qs, qr, tid);
    store_items_tr<D>(qts, qr, tid);
    store_items_rows<D>(dos, dr, tid);
    store_items_tr<D>(dots, dr, tid);
    if (tid < BQ) {
      lse_s[tid] = lr;
      d_s[tid] = dr1;
    }
    __syncthreads();
    if (tile + 1 < ntiles) load_q(q0 + BQ);
    if (DIAG && q0 + BQ - 1 < kw0) continue;  // every query of the tile precedes this wave's keys

    f32x16 s_[NQB], dpv[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s_[qb][i] = 0.f;
        dpv[qb][i] = 0.f;
      }
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const u32x4 qa = *reinterpret_cast<const u32x4*>(qs + row_off<D>(qb * 32 + l32, s * 2 + g));
        const u32x4 da = *reinterpret_cast<const u32x4*>(dos + row_off<D>(qb * 32 + l32, s * 2 + g));
        s_[qb] = mfma32(qa, kf[s], s_[qb]);
        dpv[qb] = mfma32(da, vf[s], dpv[qb]);
      }
    const bool need_mask = (q0 + BQ > Sq) || (DIAG && q0 < kw0 + 31);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = qb * 32 + 8 * j + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + r0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(d_s + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          float p = fast_exp2(fmaf(s_[qb][i], scale_log2, -l4[e]));
          if (need_mask) {
            const int qi = q0 + r0 + e;
            if (qi >= Sq || (DIAG && kk > qi)) p = 0.f;
          }
          s_[qb][i] = p;
          dpv[qb][i] = p * (dpv[qb][i] - d4[e]);  // dS
        }
      }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 pb = pack8(s_[qb], 8 * h);
        const u32x4 sb = pack8(dpv[qb], 8 * h);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = mfma32(ld_tr(dots, db * 32 + l32, qb, h, g), pb, dv[db]);
          dk[db] = mfma32(ld_tr(qts, db * 32 + l32, qb, h, g), sb, dk[db]);
        }
      }
  }

  if (kk < Sk) {
    float* krow = dkg + ((size_t)bh * Sk + kk) * D;
    float* vrow = dvg + ((size_t)bh * Sk + kk) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = db * 32 + 8 * j + 4 * g;
        f32x4 a = {dk[db][4 * j] * scale, dk[db][4 * j + 1] * scale, dk[db][4 * j + 2] * scale,
                   dk[db][4 * j + 3] * scale};
        a += *reinterpret_cast<const f32x4*>(krow + off);
        *reinterpret_cast<f32x4*>(krow + off) = a;
        f32x4 b = {dv[db][4 * j], dv[db][4 * j + 1], dv[db][4 * j + 2], dv[db][4 * j + 3]};
        b += *reinterpret_cast<const f32x4*>(vrow + off);
        *reinterpret_cast<f32x4*>(vrow + off) = b;
      }
  }
}

template <int D>
hipError_t launch_dq_d(const BwdStepArgs& a, hipStream_t stream) {
  const int nq = (a.Sq + 127) / 128;
  const long long total = (long long)nq * a.BH;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  if (a.diag)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)total), dim3(256), 0, stream, a.q, a.k, a.v, a.dO,
                       a.lse, a.D, a.dq, a.Sq, a.Sk, nq, (int)total, sl2, a.scale);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)total), dim3(256), 0, stream, a.q, a.k, a.v, a.dO,
                       a.lse, a.D, a.dq, a.Sq, a.Sk, nq, (int)total, sl2, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdStepArgs& a, hipStream_t stream) {
  const int nk = (a.Sk + 127) / 128;
  const long long total = (long long)nk * a.BH;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  if (a.diag)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((unsigned)total), dim3(256), 0, stream, a.q, a.k, a.v,
                       a.dO, a.lse, a.D, a.dk, a.dv, a.Sq, a.Sk, nk, (int)total, sl2, a.scale);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((unsigned)total), dim3(256), 0, stream, a.q, a.k, a.v,
                       a.dO, a.lse, a.D, a.dk, a.dv, a.Sq, a.Sk, nk, (int)total, sl2, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq(const BwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_dq_d<128>(a, stream);
  if (a.d == 64) return launch_dq_d<64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const BwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_dkdv_d<128>(a, stream);
  if (a.d == 64) return launch_dkdv_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

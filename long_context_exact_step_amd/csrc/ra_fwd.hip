// Forward ring step: blockwise exact attention of a query block against one
// KV chunk with a fused log-sum-exp merge into the running output.
//
// Each ring step is one FlashAttention-style pass: K/V tiles are staged in
// on-chip memory and the score tile never leaves the chip; running row
// maximum and running sum of exponentials make the result exact ("Training
// Long-Context Models Without OOM: Ring Attention", "Ring Attention
// Demystified").  The epilogue folds the step's partial into the running
// (O, lse) in HBM ("Context Parallelism", 2 "Ring Attention", "How It Works",
// online softmax across steps), so only O and lse cross HBM between steps.
//
// gfx950 design.  A block is 4 waves; each wave owns NQW query rows.  The
// score tile is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// K (32 keys x 16 d) comes from LDS as the A operand, Q^T stays in registers
// as the B operand for the whole kernel.  In the accumulator a lane holds one
// query and 16 of its keys, so the softmax statistics are per-lane scalars
// (one cross-lane exchange with lane^32 per row maximum) and the probability
// registers are already the B operand of O^T += V^T P^T -- no shuffle.  V^T
// is staged in LDS, transposed in registers on the way in, with its keys
// permuted to match the accumulator's row order.  Both LDS tiles use an XOR
// swizzle of 16-byte chunks so the 32-row MFMA operand reads are free of bank
// conflicts.  The exponent base is 2 with scale*log2(e) folded into one FMA.
// The running maximum is only raised when a row's tile maximum exceeds it by
// more than 2^8 (exact: numerator and denominator share the stale maximum),
// so the O rescale is rare.
#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyTau = 8.0f;  // log2 of the largest un-rescaled probability

template <int D, int NQW>
struct FwdCfg {
  static constexpr int kThreads = 256;
  static constexpr int kWaves = 4;
  static constexpr int BR = kWaves * NQW;  // query rows per block
  static constexpr int BC = 64;            // keys per tile
  static constexpr int NCB = NQW / 32;     // 32-query column blocks per wave
  static constexpr int NKS = D / 16;       // MFMA k-steps of Q K^T
  static constexpr int NDB = D / 32;       // 32-row d blocks of O^T
  static constexpr int NKB = BC / 32;      // 32-key row blocks of S^T
  static constexpr int KCH = D / 8;        // 16-byte chunks per K row
  static constexpr int K_BYTES = BC * D * 2;
  static constexpr int V_BYTES = D * BC * 2;
  static constexpr int K_ITEMS = BC * KCH;         // 16-byte K chunks per tile
  static constexpr int KPT = K_ITEMS / kThreads;   // per thread
  static constexpr int V_ITEMS = (D / 8) * (BC / 4);  // (8 d x 4 keys) items per tile
  static constexpr int VPT = (V_ITEMS + kThreads - 1) / kThreads;
  static_assert(K_ITEMS % kThreads == 0, "K tile must split evenly");
};

template <int D, int NQW, bool DIAG, bool MERGE>
__global__ __launch_bounds__(256) void fwd_step_kernel(const uint16_t* __restrict__ qg,
                                                       const uint16_t* __restrict__ kg,
                                                       const uint16_t* __restrict__ vg,
                                                       float* __restrict__ og,
                                                       float* __restrict__ lseg, int Sq, int Sk,
                                                       int n_qtiles, int total_tiles,
                                                       float scale_log2) {
  using Cfg = FwdCfg<D, NQW>;
  constexpr int BR = Cfg::BR, BC = Cfg::BC, NCB = Cfg::NCB, NKS = Cfg::NKS;
  constexpr int NDB = Cfg::NDB, NKB = Cfg::NKB, KCH = Cfg::KCH;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::K_BYTES + Cfg::V_BYTES];
  uint8_t* const ks = smem;
  uint8_t* const vs = smem + Cfg::K_BYTES;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;

  const int t = xcd_remap(blockIdx.x, total_tiles);
  const int bh = t / n_qtiles;
  int qt = t - bh * n_qtiles;
  if (DIAG) qt = n_qtiles - 1 - qt;  // longest rows of the triangle first
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * NQW;

  const uint16_t* __restrict__ qp = qg + (size_t)bh * Sq * D;
  const uint16_t* __restrict__ kp = kg + (size_t)bh * Sk * D;
  const uint16_t* __restrict__ vp = vg + (size_t)bh * Sk * D;

  // Q^T fragments: column = query, k = 8 consecutive d values.
  u32x4 qf[NCB][NKS];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int qq = qw0 + cb * 32 + l32;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      qf[cb][s] = (qq < Sq) ? ld16(qp + (size_t)qq * D + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[NCB][NDB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[cb][db][i] = 0.f;
  float mrow[NCB], lrow[NCB];  // running max (log2 units) and this lane's partial row sum
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    mrow[cb] = kNegInf;
    lrow[cb] = 0.f;
  }

  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;

  // Register staging of the next K/V tile.
  u32x4 kr[Cfg::KPT];
  u32x4 vr[Cfg::VPT][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < Cfg::KPT; ++i) {
      const int it = tid + i * Cfg::kThreads;
      const int r = it / KCH, c = it % KCH;
      kr[i] = (k0 + r < Sk) ? ld16(kp + (size_t)(k0 + r) * D + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Cfg::VPT; ++i) {
      const int it = tid + i * Cfg::kThreads;
      if (it < Cfg::V_ITEMS) {
        const int dc = it % (D / 8), kq = it / (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = k0 + kq * 4 + rr;
          vr[i][rr] = (key < Sk) ? ld16(vp + (size_t)key * D + dc * 8) : u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < Cfg::KPT; ++i) {
      const int it = tid + i * Cfg::kThreads;
      const int r = it / KCH, c = it % KCH;
      *reinterpret_cast<u32x4*>(ks + row_off<D>(r, c)) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::VPT; ++i) {
      const int it = tid + i * Cfg::kThreads;
      if (it < Cfg::V_ITEMS) {
        const int dc = it % (D / 8), kq = it / (D / 8);
        store_tr4x8(vs, dc, kq, vr[i]);
      }
    }
  };

  load_tile(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int k0 = tile * BC;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile + 1 < ntiles) load_tile(k0 + BC);

    // Diagonal chunk: a wave whose rows all precede this tile has nothing to do.
    if (DIAG && k0 > qw0 + NQW - 1) continue;

    f32x16 sacc[NKB][NCB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][cb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(ks + row_off<D>(kb * 32 + l32, s * 2 + g));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) sacc[kb][cb] = mfma32(af, qf[cb][s], sacc[kb][cb]);
      }
    }

    const bool need_mask = (k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int qq = qw0 + cb * 32 + l32;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= Sk || (DIAG && key > qq)) sacc[kb][cb][i] = kNegInf;
          }
        }
    }

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][cb][i]);
      mx = fmaxf(mx, xor32(mx)) * scale_log2;
      if (__ballot(mx > mrow[cb] + kLazyTau) != 0) {
        const float mnew = fmaxf(mrow[cb], mx);
        const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(mrow[cb] - mnew);
        mrow[cb] = mnew;
        lrow[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[cb][db][i] *= alpha;
      }
      const float mb = (mrow[cb] == kNegInf) ? 0.f : mrow[cb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[kb][cb][i], scale_log2, -mb));
          sacc[kb][cb][i] = p;
          ls += p;
        }
      lrow[cb] += ls;
    }

#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 pb[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) pb[cb] = pack8(sacc[kb][cb], 8 * h);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 vf = ld_tr(vs, db * 32 + l32, kb, h, g);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) oacc[cb][db] = mfma32(vf, pb[cb], oacc[cb][db]);
        }
      }
    }
  }

  // Epilogue: this step's partial (oacc / l, m + log2 l) folded into (O, lse).
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = lrow[cb] + xor32(lrow[cb]);
    const int qq = qw0 + cb * 32 + l32;
    if (qq >= Sq) continue;
    const float lse_s = (lt > 0.f) ? mrow[cb] + log2f(lt) : kNegInf;  // log2 units
    float w_old = 0.f, w_step, lse_new;
    float* orow = og + ((size_t)bh * Sq + qq) * D;
    float* lp = lseg + (size_t)bh * Sq + qq;
    if (MERGE) {
      const float lold = *lp * kLog2e;
      const float M = fmaxf(lold, lse_s);
      if (M == kNegInf) {
        lse_new = kNegInf;
        w_step = 0.f;
      } else {
        const float eo = exp2f(lold - M), es = exp2f(lse_s - M);
        const float tot = eo + es;
        lse_new = M + log2f(tot);
        w_old = eo / tot;
        w_step = (lt > 0.f) ? es / tot / lt : 0.f;
      }
    } else {
      lse_new = lse_s;
      w_step = (lt > 0.f) ? 1.f / lt : 0.f;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = orow + db * 32 + 8 * j + 4 * g;
        f32x4 val = {oacc[cb][db][4 * j + 0] * w_step, oacc[cb][db][4 * j + 1] * w_step,
                     oacc[cb][db][4 * j + 2] * w_step, oacc[cb][db][4 * j + 3] * w_step};
        if (MERGE) {
          const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
          val += w_old * old;
        }
        *reinterpret_cast<f32x4*>(dst) = val;
      }
    if (g == 0) *lp = lse_new * kLn2;
  }
}

template <int D, int NQW>
hipError_t launch_cfg(const FwdStepArgs& a, hipStream_t stream) {
  using Cfg = FwdCfg<D, NQW>;
  const int n_qtiles = (a.Sq + Cfg::BR - 1) / Cfg::BR;
  const long long total = (long long)n_qtiles * a.BH;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((unsigned)total), block(Cfg::kThreads);
#define RA_FWD_LAUNCH(DIAG, MERGE)                                                          \
  hipLaunchKernelGGL((fwd_step_kernel<D, NQW, DIAG, MERGE>), grid, block, 0, stream, a.q, a.k, \
                     a.v, a.o, a.lse, a.Sq, a.Sk, n_qtiles, (int)total, sl2)
  if (a.diag) {
    if (a.merge) RA_FWD_LAUNCH(true, true);
    else RA_FWD_LAUNCH(true, false);
  } else {
    if (a.merge) RA_FWD_LAUNCH(false, true);
    else RA_FWD_LAUNCH(false, false);
  }
#undef RA_FWD_LAUNCH
  return hipGetLastError();
}

}  // namespace

#ifndef RA_FWD_NQW
#define RA_FWD_NQW 32
#endif

hipError_t launch_fwd_step(const FwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_cfg<128, RA_FWD_NQW>(a, stream);
  if (a.d == 64) return launch_cfg<64, RA_FWD_NQW>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

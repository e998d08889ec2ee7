// Forward ring step: blockwise exact attention of a query block against one
// KV chunk with a fused log-sum-exp merge into the running output.
//
// Each ring step is one FlashAttention-style pass: K/V tiles are staged in
// on-chip memory and the score tile never leaves the chip; a running row
// maximum and running sum of exponentials make the result exact ("Training
// Long-Context Models Without OOM: Ring Attention", "Ring Attention
// Demystified").  The epilogue folds the step's partial into the running
// (O, lse) in HBM ("Context Parallelism", 2 "Ring Attention", "How It Works":
// online softmax merges partial results across steps), so only O and lse
// cross HBM between steps.
//
// gfx950 design.
//  * A block is 4 waves (one per SIMD); each wave owns 64 query rows, so a
//    block covers 256 rows and every K/V byte read from LDS feeds 64 queries.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS; Q^T is the B operand and stays in registers for the whole kernel.
//    In the accumulator a lane holds one query and 16 of its keys, so the
//    softmax statistics are per-lane scalars (one lane^32 exchange per row
//    maximum), and the probabilities, packed to bf16, are already the B
//    operand of O^T += V^T P^T.  V^T's A operand comes straight from the
//    row-major V tile through ds_read_b64_tr_b16 (no transpose pass).
//  * K and V tiles (64 keys) go global -> LDS with global_load_lds
//    (no registers, no LDS store instructions); three K and two V buffers
//    give every load a whole tile of compute to land, with one block barrier
//    per tile.
//  * Software pipeline over 32-key sub-tiles: while the VALU does the
//    softmax of sub-tile u, the matrix cores already compute S^T of u+1;
//    then P V of u.
//  * exp2 with scale*log2(e) folded into one FMA; the running maximum is
//    raised only when a row's tile maximum exceeds it by more than 2^8
//    (exact: numerator and denominator share the stale maximum), so the
//    O rescale is rare.
//  * Blocks are mapped so each XCD works on one contiguous range of
//    (head, query tile) pairs (K/V lines shared in that XCD's L2); on the
//    diagonal chunk the longest query tiles go first.
#include <type_traits>

#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyTau = 8.0f;  // log2 of the largest un-rescaled probability

template <int D, int NW_, int NQW_>
struct FwdCfg {
  static constexpr int kWaves = NW_;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int NQW = NQW_;             // query rows per wave
  static constexpr int BR = kWaves * NQW;      // query rows per block
  static constexpr int BC = kTileTokens;       // keys per tile
  static constexpr int NCB = NQW / 32;         // 32-query column blocks per wave
  static constexpr int NKS = D / 16;           // MFMA k-steps of K Q^T
  static constexpr int NDB = D / 32;           // 32-row d blocks of O^T
  static constexpr int NKB = BC / 32;          // 32-key row blocks of S^T
  static constexpr int TILE = BC * D * 2;      // bytes of one K or V tile
};

template <int D, int NW_, int NQW_, bool DIAG, bool MERGE>
__global__ __launch_bounds__(64 * NW_) void fwd_step_kernel(const uint16_t* __restrict__ qg,
                                                       const uint16_t* __restrict__ kg,
                                                       const uint16_t* __restrict__ vg,
                                                       float* __restrict__ og,
                                                       float* __restrict__ lseg, int Sq, int Sk,
                                                       int n_qtiles, int total_tiles,
                                                       float scale_log2) {
  using Cfg = FwdCfg<D, NW_, NQW_>;
  constexpr int NW = Cfg::kWaves, NQW = Cfg::NQW, BR = Cfg::BR, BC = Cfg::BC, NCB = Cfg::NCB;
  constexpr int NKS = Cfg::NKS, NDB = Cfg::NDB, TILE = Cfg::TILE;
  // LDS: K tiles in buffers 0..2, V tiles in buffers 3..4 (TILE bytes each).
  // K tile T sits in K buffer T % 3 and V tile T in V buffer T % 2; the
  // main loop is unrolled by 6 so every buffer offset is an immediate.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * TILE];

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

  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;
  // Prologue loads: K(0), K(1), V(0).
  TileDma<D, NW> dma;
  dma.init(wave, lane);
  dma.load(smem, kp, 0, Sk);
  if (ntiles > 1) dma.load(smem + TILE, kp, BC, Sk);
  dma.load(smem + 3 * TILE, vp, 0, Sk);

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

  // Compute proceeds in 32-key sub-tiles u (LDS tile u/2, half u%2).
  const int nsub = (kend + 31) / 32;
  const int wsub = DIAG ? min(nsub, max(0, (min(qw0 + NQW, Sq) - 1) / 32 + 1)) : nsub;

  // Lane parts of the LDS addresses, fixed for the whole kernel: the K
  // operand chunk of k-step s (row l32, chunk 2s+g of a K tile), and the two
  // transposed-read addresses of each 32-feature block of a V tile.  Tile,
  // half and 16-token offsets are added as immediates.
  uint32_t kofs[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kofs[s] = (uint32_t)tile_off<D>(l32, 2 * s + g);
  uint32_t vaddr[NDB][2];
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
    const uint32_t vbase = lds_addr(smem) + 3 * TILE;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        vaddr[db][t] = vbase + tile_off<D>(4 * g + m + 8 * t, d >> 3) + ((d & 4) ? 8 : 0);
    }
  }

  // S^T of sub-tile HALF of K buffer KB into `acc`.
  auto scores = [&](f32x16 (&acc)[NCB], auto kbc, auto halfc) __attribute__((always_inline)) {
    constexpr int OFF = decltype(kbc)::value * TILE + decltype(halfc)::value * 32 * D * 2;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const u32x4 af = *reinterpret_cast<const u32x4*>(smem + kofs[s] + OFF);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[cb] = mfma32(af, qf[cb][s], acc[cb]);
    }
  };

  // O^T += V^T P^T for the 16 tokens h of sub-tile HALF of V buffer VB.
  auto pv = [&](const u32x4 (&pb)[NCB], auto vbc, auto halfc, auto hc) __attribute__((always_inline)) {
    constexpr int OFF = decltype(vbc)::value * TILE + (32 * decltype(halfc)::value + 16 * decltype(hc)::value) * D * 2;
    u32x4 vf[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2 lo = ds_read_tr16_off<OFF>(vaddr[db][0]);
      const u32x2 hi = ds_read_tr16_off<OFF>(vaddr[db][1]);
      vf[db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    if constexpr (NDB == 4) lds_wait(vf[0], vf[1], vf[2], vf[3]);
    else lds_wait(vf[0], vf[1]);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) oacc[cb][db] = mfma32(vf[db], pb[cb], oacc[cb][db]);
  };

  // Online softmax of sub-tile u held in `acc` (overwritten with P), then
  // O^T += V^T P^T from half HALF of V buffer VB.
  auto softmax_pv = [&](f32x16 (&acc)[NCB], int u, auto vbc, auto halfc) __attribute__((always_inline)) {
    const int k0 = u * 32;
    const bool need_mask = (k0 + 32 > Sk) || (DIAG && k0 + 31 > qw0);
    if (need_mask) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int qq = qw0 + cb * 32 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= Sk || (DIAG && key > qq)) acc[cb][i] = kNegInf;
        }
      }
    }
    u32x4 pb0[NCB], pb1[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[cb][i]);
      mx = pair_max(mx) * scale_log2;
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
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(acc[cb][i], scale_log2, -mb));
        acc[cb][i] = p;
        ls += p;
      }
      lrow[cb] += ls;
      pb0[cb] = pack8(acc[cb], 0);
      pb1[cb] = pack8(acc[cb], 8);
    }
    pv(pb0, vbc, halfc, std::integral_constant<int, 0>{});
    pv(pb1, vbc, halfc, std::integral_constant<int, 1>{});
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  f32x16 sA[NCB], sB[NCB];
  wait_vmem();
  __syncthreads();
  if (0 < wsub) scores(sA, I0{}, I0{});
  // Iteration T (T % 6 == I): at its top K(T+1) and V(T) have landed and
  // every wave is done with K(T-1) and V(T-1), whose buffers then receive
  // K(T+2) and V(T+1).  Sub-step 2T: S^T(2T+1) from the second half of K(T)
  // while the softmax and P V of 2T run; sub-step 2T+1: S^T(2T+2) from the
  // first half of K(T+1) while the softmax and P V of 2T+1 run.
  auto iteration = [&](auto ic, int T) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    using KC = std::integral_constant<int, I % 3>;
    using KN = std::integral_constant<int, (I + 1) % 3>;
    using VC = std::integral_constant<int, I % 2>;
    constexpr int KL = (I + 2) % 3, VN = (I + 1) % 2;
    wait_vmem();
    __syncthreads();
    if (T + 2 < ntiles) dma.load(smem + KL * TILE, kp, (T + 2) * BC, Sk);
    if (T + 1 < ntiles) dma.load(smem + (3 + VN) * TILE, vp, (T + 1) * BC, Sk);
    const int u0 = 2 * T, u1 = 2 * T + 1;
    if (u0 + 1 < wsub) scores(sB, KC{}, I1{});
    if (u0 < wsub) softmax_pv(sA, u0, VC{}, I0{});
    if (u1 + 1 < wsub) scores(sA, KN{}, I0{});
    if (u1 < wsub) softmax_pv(sB, u1, VC{}, I1{});
  };
  for (int T = 0; T < ntiles; T += 6) {
    iteration(std::integral_constant<int, 0>{}, T);
    if (T + 1 < ntiles) iteration(std::integral_constant<int, 1>{}, T + 1);
    if (T + 2 < ntiles) iteration(std::integral_constant<int, 2>{}, T + 2);
    if (T + 3 < ntiles) iteration(std::integral_constant<int, 3>{}, T + 3);
    if (T + 4 < ntiles) iteration(std::integral_constant<int, 4>{}, T + 4);
    if (T + 5 < ntiles) iteration(std::integral_constant<int, 5>{}, T + 5);
  }

  // Epilogue: this step's partial (oacc / l, m + log2 l) folded into (O, lse).
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = pair_sum(lrow[cb]);
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

template <int D, int NW, int NQW>
hipError_t launch_cfg(const FwdStepArgs& a, hipStream_t stream) {
  using Cfg = FwdCfg<D, NW, NQW>;
  const int n_qtiles = (a.Sq + Cfg::BR - 1) / Cfg::BR;
  const long long total = (long long)n_qtiles * a.BH;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((unsigned)total), block(Cfg::kThreads);
#define RA_FWD_LAUNCH(DIAG, MERGE)                                                                      \
  hipLaunchKernelGGL((fwd_step_kernel<D, NW, NQW, DIAG, MERGE>), grid, block, 0, stream, a.q, a.k, a.v, a.o, a.lse, \
                     a.Sq, a.Sk, n_qtiles, (int)total, sl2)
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

#ifndef RA_FWD_WAVES
#define RA_FWD_WAVES 8
#endif
#ifndef RA_FWD_ROWS_PER_WAVE
#define RA_FWD_ROWS_PER_WAVE 32
#endif

hipError_t launch_fwd_step(const FwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_cfg<128, RA_FWD_WAVES, RA_FWD_ROWS_PER_WAVE>(a, stream);
  if (a.d == 64) return launch_cfg<64, RA_FWD_WAVES, RA_FWD_ROWS_PER_WAVE>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

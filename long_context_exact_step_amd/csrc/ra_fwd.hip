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
//  * A block is 8 waves of 32 query rows (256 rows); two waves share each
//    SIMD, so one wave's softmax (VALU) overlaps the other's MFMAs.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS; Q^T is the B operand and stays in registers for the whole kernel.
//    In the accumulator a lane holds one query and 16 of its keys, so the
//    softmax statistics are per-lane scalars (one v_permlane32_swap per row
//    maximum), and the probabilities, packed to bf16, are already the B
//    operand of O^T += V^T P^T.  V^T's A operand comes straight from the
//    row-major V tile through ds_read_b64_tr_b16 (no transpose pass).
//  * K and V tiles (64 keys) go global -> LDS with global_load_lds
//    (no registers, no LDS store instructions), two buffers each, one block
//    barrier per tile; each load has a whole tile of compute to land.
//  * Software pipeline per wave: S^T of tile t+1 is computed in the same
//    basic block as the softmax of tile t, then P V of tile t.
//  * The loop is unrolled by 2 so every LDS offset is an immediate; the lane
//    parts of the LDS addresses are computed once per kernel.
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


// Epilogue: this step's partial (oacc / l, m + log2 l) of the lane's query
// row folded into the running (O, lse).
template <int D, bool MERGE>
__device__ __forceinline__ void fwd_epilogue(const f32x16 (&oacc)[D / 32], float mrow, float lrow,
                                             float* __restrict__ og, float* __restrict__ lseg, int bh, int Sq,
                                             int qq, int g) {
  constexpr int NDB = D / 32;
  const float lt = pair_sum(lrow);
  if (qq >= Sq) return;
  const float lse_s = (lt > 0.f) ? mrow + log2f(lt) : kNegInf;  // log2 units
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
      f32x4 val = {oacc[db][4 * j + 0] * w_step, oacc[db][4 * j + 1] * w_step, oacc[db][4 * j + 2] * w_step,
                   oacc[db][4 * j + 3] * w_step};
      if (MERGE) {
        const f32x4 old = *reinterpret_cast<const f32x4*>(dst);
        val += w_old * old;
      }
      *reinterpret_cast<f32x4*>(dst) = val;
    }
  if (g == 0) *lp = lse_new * kLn2;
}

// LDS reads still in flight after those of MFMA m, when the reads of MFMAs
// m+1 .. m+LA have been issued; the first NPV MFMAs take two reads each.
__host__ __device__ constexpr int reads_after(int m, int LA, int NPV, int NOP) {
  int n = 0;
  for (int k = m + 1; k <= m + LA && k < NOP; ++k) n += (k < NPV) ? 2 : 1;
  return n;
}

constexpr int kFwdWaves = 8;       // waves per block; waves w and w + 4 share a SIMD
constexpr int kFwdRowsPerWave = 32;
constexpr int kFwdLookahead = 6;   // MFMAs whose LDS operands are read ahead

// One ring step.  A block holds 256 query rows, 32 per wave, and walks the
// chunk's keys in 64-key tiles.  Per tile a wave runs two phases:
//   MFMA phase of tile t:     O^T += V^T P^T(t-1), then S^T(t) = K(t) Q^T;
//   softmax phase of tile t:  the online softmax of S^T(t) -> P^T(t) in bf16.
// Waves 4..7 run one phase behind waves 0..3, with a workgroup barrier
// between phases, so on every SIMD one wave keeps the matrix core busy while
// the other computes exponentials.  Phase 2u starts the loads of K(u+1) and
// V(u) (two buffers each); they are waited for at the end of phase 2u+1,
// before anyone reads them in phase 2u+2.
template <int D, bool DIAG, bool MERGE>
__global__ __launch_bounds__(64 * kFwdWaves) void fwd_step_kernel(const uint16_t* __restrict__ qg,
                                                                  const uint16_t* __restrict__ kg,
                                                                  const uint16_t* __restrict__ vg,
                                                                  float* __restrict__ og,
                                                                  float* __restrict__ lseg, int Sq, int Sk,
                                                                  int n_qtiles, int total_tiles,
                                                                  float scale_log2) {
  constexpr int NW = kFwdWaves, NQW = kFwdRowsPerWave, BR = NW * NQW, BC = kTileTokens;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = BC / 32, TILE = BC * D * 2, LA = kFwdLookahead;
  // LDS: K tiles in buffers 0..1, V tiles in buffers 2..3; tile t uses buffer t % 2.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const bool lead = wave < NW / 2;
  const int t = xcd_remap(blockIdx.x, total_tiles);
  const int bh = t / n_qtiles;
  int qt = t - bh * n_qtiles;
  if (DIAG) qt = n_qtiles - 1 - qt;  // longest rows of the triangle first
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * NQW;
  const int qq = qw0 + l32;
  const uint16_t* __restrict__ qp = qg + (size_t)bh * Sq * D;
  const uint16_t* __restrict__ kp = kg + (size_t)bh * Sk * D;
  const uint16_t* __restrict__ vp = vg + (size_t)bh * Sk * D;

  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR);
  const int ntiles = (kend + BC - 1) / BC;
  const int wtiles = DIAG ? min(ntiles, max(0, (min(qw0 + NQW, Sq) - 1) / BC + 1)) : ntiles;

  TileDma<D, NW, BC> dma;
  dma.init(wave, lane);
  dma.load(smem, kp, 0, Sk);
  dma.load(smem + 3 * TILE, vp, 0, Sk);  // finite data for the P = 0 product of tile 0

  u32x4 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = (qq < Sq) ? ld16(qp + (size_t)qq * D + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float mrow = kNegInf, lrow = 0.f;
  f32x16 sacc[NKB];
  u32x4 pb[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) pb[kb][0] = pb[kb][1] = u32x4{0, 0, 0, 0};

  const uint32_t base = lds_addr(smem);
  uint32_t kaddr[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kaddr[s] = base + (uint32_t)tile_off<D>(l32, 2 * s + g);
  uint32_t vaddr[NDB][2];
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        vaddr[db][tt] = base + tile_off<D>(4 * g + m + 8 * tt, d >> 3) + ((d & 4) ? 8 : 0);
    }
  }

  // MFMA phase: O^T += V^T P^T from V buffer VB, then S^T from K buffer KB
  // into sacc.  The LDS operands of the next LA MFMAs are always in flight;
  // each MFMA waits only for its own.
  auto mfma_phase = [&](auto kbc, auto vbc) __attribute__((always_inline)) {
    constexpr int KB = decltype(kbc)::value, VB = decltype(vbc)::value;
    constexpr int NPV = 4 * NDB, NOP = NPV + NKS * NKB;
    u32x2 lo[LA + 1], hi[LA + 1];
    u32x4 kq[LA + 1];
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      if constexpr (m < NPV) {
        // V^T block db for tokens 32*(gi/2) + 16*(gi%2) .. +15.
        constexpr int gi = m / NDB, db = m % NDB;
        constexpr int OFF = (2 + VB) * TILE + (32 * (gi >> 1) + 16 * (gi & 1)) * D * 2;
        lo[b] = ds_read_tr16_off<OFF>(vaddr[db][0]);
        hi[b] = ds_read_tr16_off<OFF>(vaddr[db][1]);
      } else if constexpr (m < NOP) {
        constexpr int j = m - NPV, s = j / NKB, kb = j % NKB;
        kq[b] = ds_read_b128_off<KB * TILE + kb * 32 * D * 2>(kaddr[s]);
      }
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      constexpr int N = reads_after(m, LA, NPV, NOP);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (m < NPV) {
        constexpr int gi = m / NDB, db = m % NDB;
        lgkm_wait<N>(lo[b], hi[b]);
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        oacc[db] = mfma32(a, pb[gi >> 1][gi & 1], oacc[db]);
      } else {
        constexpr int j = m - NPV, s = j / NKB, kb = j % NKB;
        lgkm_wait<N>(kq[b]);
        if constexpr (s == 0) sacc[kb] = mfma32(kq[b], qf[0], f32x16{});
        else sacc[kb] = mfma32(kq[b], qf[s], sacc[kb]);
      }
    };
    static_for<LA>(issue);
    static_for<NOP>(run);
  };

  // Softmax phase of tile tt: mask, running maximum (raised lazily), P in
  // bf16 into pb, running sum, and the rare rescale of O.
  auto softmax_phase = [&](int tt) __attribute__((always_inline)) {
    const int k0 = tt * BC;
    if ((k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= Sk || (DIAG && key > qq)) sacc[kb][i] = kNegInf;
        }
    }
    // Row maximum as a tree (short dependency chains).
    float mp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mp[j] = fmaxf(fmaxf(sacc[j >> 1][8 * (j & 1)], sacc[j >> 1][8 * (j & 1) + 1]),
                                            sacc[j >> 1][8 * (j & 1) + 2]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 3; i < 8; ++i) {
        mp[2 * kb] = fmaxf(mp[2 * kb], sacc[kb][i]);
        mp[2 * kb + 1] = fmaxf(mp[2 * kb + 1], sacc[kb][8 + i]);
      }
    float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
    mx = pair_max(mx) * scale_log2;
    const bool grow = __ballot(mx > mrow + kLazyTau) != 0;
    const float mnew = grow ? fmaxf(mrow, mx) : mrow;
    const float mb = (mnew == kNegInf) ? 0.f : mnew;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = fmaf(sacc[kb][i], scale_log2, -mb);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = fast_exp2(sacc[kb][i]);
    // Row sum with four partial sums.
    float lp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) lp[(i & 1) + 2 * kb] += sacc[kb][i];
    const float acc_l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      pb[kb][0] = pack8(sacc[kb], 0);
      pb[kb][1] = pack8(sacc[kb], 8);
    }
    if (grow) {
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(mrow - mnew);
      lrow *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    mrow = mnew;
    lrow += acc_l;
  };

  // Tile tt's MFMA phase runs for 0 <= tt <= wtiles: at tt = 0 P is still
  // zero (the V buffer it multiplies holds finite data), and at tt = wtiles the
  // score tile is computed but never used.  One code shape for every tile.
  auto mfma_tile = [&](int tt, auto kbc, auto vbc) __attribute__((always_inline)) {
    if (tt <= wtiles) mfma_phase(kbc, vbc);
  };
  auto softmax_tile = [&](int tt) __attribute__((always_inline)) {
    if (tt >= 0 && tt < wtiles) softmax_phase(tt);
  };
  // Phases 2u and 2u + 1 (u % 2 == I): K(u) sits in K buffer I and V(u-1) in
  // V buffer 1 - I; K(u+1) and V(u) are loaded into the other two.
  auto phase_pair = [&](auto ic, int u) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    using KC = std::integral_constant<int, I>;
    using VC = std::integral_constant<int, 1 - I>;
    if (u + 1 < ntiles) dma.load(smem + (1 - I) * TILE, kp, (u + 1) * BC, Sk);
    if (u < ntiles) dma.load(smem + (2 + I) * TILE, vp, u * BC, Sk);
    if (lead) mfma_tile(u, KC{}, VC{});
    else softmax_tile(u - 1);
    phase_barrier();
    if (lead) softmax_tile(u);
    else mfma_tile(u, KC{}, VC{});
    wait_vmem();
    phase_barrier();
  };

  wait_vmem();
  phase_barrier();
  for (int u = 0; u <= ntiles; u += 2) {
    phase_pair(std::integral_constant<int, 0>{}, u);
    if (u + 1 <= ntiles) phase_pair(std::integral_constant<int, 1>{}, u + 1);
  }

  fwd_epilogue<D, MERGE>(oacc, mrow, lrow, og, lseg, bh, Sq, qq, g);
}

template <int D>
hipError_t launch_cfg(const FwdStepArgs& a, hipStream_t stream) {
  constexpr int BR = kFwdWaves * kFwdRowsPerWave;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  const long long total = (long long)n_qtiles * a.BH;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((unsigned)total), block(64 * kFwdWaves);
#define RA_FWD_LAUNCH(DIAG, MERGE)                                                                         \
  hipLaunchKernelGGL((fwd_step_kernel<D, DIAG, MERGE>), grid, block, 0, stream, a.q, a.k, a.v, a.o, \
                     a.lse, a.Sq, a.Sk, n_qtiles, (int)total, sl2)
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

hipError_t launch_fwd_step(const FwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_cfg<128>(a, stream);
  if (a.d == 64) return launch_cfg<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

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


// Epilogue shared by the forward kernels: this step's partial
// (oacc / l, m + log2 l) folded into the running (O, lse) of the lane's rows.
template <int D, int NCB, bool MERGE>
__device__ __forceinline__ void fwd_epilogue(const f32x16 (&oacc)[NCB][D / 32], const float (&mrow)[NCB],
                                             const float (&lrow)[NCB], float* __restrict__ og,
                                             float* __restrict__ lseg, int bh, int Sq, int qw0, int l32, int g) {
  constexpr int NDB = D / 32;
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

// One ring step.  A block is NW waves; wave w owns NQW query rows.  Step t
// of the key loop computes S^T for the next whole 64-key tile (two 32-key
// blocks) while the online softmax of tile t runs, then O^T += V^T P^T of
// tile t.  Two K and two V buffers: K(t+2) overwrites K(t), whose last reader
// (S^T(t)) ran in the previous iteration.
template <int D, int NW_, int NQW_, bool DIAG, bool MERGE>
__global__ __launch_bounds__(64 * NW_) void fwd_step_kernel(const uint16_t* __restrict__ qg,
                                                                const uint16_t* __restrict__ kg,
                                                                const uint16_t* __restrict__ vg,
                                                                float* __restrict__ og,
                                                                float* __restrict__ lseg, int Sq, int Sk,
                                                                int n_qtiles, int total_tiles,
                                                                float scale_log2) {
  constexpr int NW = NW_, NQW = NQW_, BR = NW * NQW, BC = kTileTokens, NCB = NQW / 32;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = BC / 32, TILE = BC * D * 2;
  // LDS: K tiles in buffers 0..1, V tiles in buffers 2..3; tile t uses buffer t % 2.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE];

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
  const int wtiles = DIAG ? min(ntiles, max(0, (min(qw0 + NQW, Sq) - 1) / BC + 1)) : ntiles;

  TileDma<D, NW, BC> dma;
  dma.init(wave, lane);
  dma.load(smem, kp, 0, Sk);
  if (ntiles > 1) dma.load(smem + TILE, kp, BC, Sk);
  dma.load(smem + 2 * TILE, vp, 0, Sk);

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
  float mrow[NCB], lrow[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    mrow[cb] = kNegInf;
    lrow[cb] = 0.f;
  }

  uint32_t kofs[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kofs[s] = (uint32_t)tile_off<D>(l32, 2 * s + g);
  uint32_t vaddr[NDB][2];
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
    const uint32_t vbase = lds_addr(smem) + 2 * TILE;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        vaddr[db][tt] = vbase + tile_off<D>(4 * g + m + 8 * tt, d >> 3) + ((d & 4) ? 8 : 0);
    }
  }

  // S^T of K buffer KB (both 32-key blocks) into `acc`.
  auto scores = [&](f32x16 (&acc)[NKB][NCB], auto kbc) __attribute__((always_inline)) {
    constexpr int OFF = decltype(kbc)::value * TILE;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[kb][cb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(smem + kofs[s] + OFF + kb * 32 * D * 2);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[kb][cb] = mfma32(af, qf[cb][s], acc[kb][cb]);
      }
  };

  // O^T += V^T P^T for tokens 32*KB2 + 16*H of V buffer VB.
  auto pv = [&](const u32x4 (&pb)[NCB], auto vbc, auto kbc, auto hc) __attribute__((always_inline)) {
    constexpr int OFF =
        decltype(vbc)::value * TILE + (32 * decltype(kbc)::value + 16 * decltype(hc)::value) * D * 2;
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

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // Step t: S^T(t+1) into `nxt` from K buffer KBN while the online softmax of
  // tile t (in `cur`) runs, then O^T += V^T P^T from V buffer VB.
  auto step = [&](f32x16 (&cur)[NKB][NCB], f32x16 (&nxt)[NKB][NCB], int tile, auto kbn, auto vbc)
                  __attribute__((always_inline)) {
    if (tile >= wtiles) return;
    const int k0 = tile * BC;
    if ((k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int qq = qw0 + cb * 32 + l32;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= Sk || (DIAG && key > qq)) cur[kb][cb][i] = kNegInf;
          }
        }
    }
    scores(nxt, kbn);
    float mnew[NCB], ls[NCB];
    bool grow = false;
    u32x4 pb[NKB][2][NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, cur[kb][cb][i]);
      mx = pair_max(mx) * scale_log2;
      const bool g_cb = __ballot(mx > mrow[cb] + kLazyTau) != 0;
      grow = grow || g_cb;
      mnew[cb] = g_cb ? fmaxf(mrow[cb], mx) : mrow[cb];
      const float mb = (mnew[cb] == kNegInf) ? 0.f : mnew[cb];
      float acc_l = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(cur[kb][cb][i], scale_log2, -mb));
          cur[kb][cb][i] = p;
          acc_l += p;
        }
      ls[cb] = acc_l;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pb[kb][0][cb] = pack8(cur[kb][cb], 0);
        pb[kb][1][cb] = pack8(cur[kb][cb], 8);
      }
    }
    if (grow) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float alpha = (mnew[cb] == kNegInf) ? 1.f : fast_exp2(mrow[cb] - mnew[cb]);
        lrow[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[cb][db][i] *= alpha;
      }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      mrow[cb] = mnew[cb];
      lrow[cb] += ls[cb];
    }
    pv(pb[0][0], vbc, I0{}, I0{});
    pv(pb[0][1], vbc, I0{}, I1{});
    pv(pb[1][0], vbc, I1{}, I0{});
    pv(pb[1][1], vbc, I1{}, I1{});
  };

  f32x16 sA[NKB][NCB], sB[NKB][NCB];
  wait_vmem();
  __syncthreads();
  if (0 < wtiles) scores(sA, I0{});
  // Iteration t (t % 2 == I): at its top K(t+1) and V(t) have landed and
  // every wave is done with K(t) (read by S^T(t) last iteration) and V(t-1),
  // whose buffers then receive K(t+2) and V(t+1).
  auto iteration = [&](auto ic, int tile) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    using KN = std::integral_constant<int, (I + 1) % 2>;
    using VC = std::integral_constant<int, I>;
    wait_vmem();
    __syncthreads();
    if (tile + 2 < ntiles) dma.load(smem + I * TILE, kp, (tile + 2) * BC, Sk);
    if (tile + 1 < ntiles) dma.load(smem + (2 + (I + 1) % 2) * TILE, vp, (tile + 1) * BC, Sk);
    if constexpr (I == 0) step(sA, sB, tile, KN{}, VC{});
    else step(sB, sA, tile, KN{}, VC{});
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    iteration(I0{}, tile);
    if (tile + 1 < ntiles) iteration(I1{}, tile + 1);
  }

  fwd_epilogue<D, NCB, MERGE>(oacc, mrow, lrow, og, lseg, bh, Sq, qw0, l32, g);
}

template <int D, int NW, int NQW>
hipError_t launch_cfg(const FwdStepArgs& a, hipStream_t stream) {
  constexpr int BR = NW * NQW;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  const long long total = (long long)n_qtiles * a.BH;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((unsigned)total), block(64 * NW);
#define RA_FWD_LAUNCH(DIAG, MERGE)                                                                         \
  hipLaunchKernelGGL((fwd_step_kernel<D, NW, NQW, DIAG, MERGE>), grid, block, 0, stream, a.q, a.k, a.v, a.o, \
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

// 8 waves of 32 query rows: two waves share each SIMD, so one's softmax can
// overlap the other's MFMAs.
constexpr int kFwdWaves = 8;
constexpr int kFwdRowsPerWave = 32;

hipError_t launch_fwd_step(const FwdStepArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_cfg<128, kFwdWaves, kFwdRowsPerWave>(a, stream);
  if (a.d == 64) return launch_cfg<64, kFwdWaves, kFwdRowsPerWave>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ra

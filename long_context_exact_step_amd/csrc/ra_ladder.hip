// Ladder probe: the forward step kernel's instruction stream, rebuilt from
// the dense MFMA probe one feature at a time, to account for the distance
// between what the matrix cores sustain and what the attention kernel
// reaches (measurement helper; no page defines it).
//
// Every level runs 8 waves per CU (two per SIMD, one 128 KB block per CU,
// as the attention kernel) and issues 32 bf16 32x32x16 MFMAs per "tile" per
// wave, so every level does the same matrix work: 32 * 32768 flop per tile
// per wave.  Level L adds to level L-1:
//   0  the dense probe: four independent accumulators, register operands
//   1  the kernel's accumulator pattern: per tile 16 MFMAs into four output
//      accumulators (P V) and 16 into two score accumulators that restart
//      every tile (eight-deep chains, Q^T as the register operand)
//   2  A operands read from LDS as the kernel reads them: ds_read_b64_tr_b16
//      pairs for the P V half, ds_read_b128 for the score half, three MFMAs
//      ahead with counted waits, over four buffers per operand
//   3  the online-softmax vector work of the previous tile's scores in the
//      MFMA slots (scale, exp2, row sum, bf16 pack), its P feeding the next
//      P V half as the kernel's does
//   4  one workgroup barrier per tile
//   5  the tile loads: 1 KB direct-to-LDS buffer loads (four per wave per
//      tile) two tiles ahead, and the kernel's wait for them before the
//      barrier
// Wave 0 of block 0 records its loop's shader clocks and 100 MHz reference
// ticks, whose ratio is the clock the cores ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ra.h"
#include "ra_device.h"

namespace ra {
namespace {

constexpr int kLadWaves = 8;
constexpr int kLadD = 128;
constexpr int kLadTile = kTileTokens * kLadD * 2;  // one 64-token bf16 tile: 16 KB
constexpr int kLadBuffers = 4;                     // per operand, as the kernel
constexpr int kLadSrcTiles = 64;                   // distinct source tiles of the tile loads (1 MB)

// First softmax element issued in MFMA slot m (the kernel's spread).
__host__ __device__ constexpr int lad_first(int m, int SH, int NOP, int NEL) {
  return m <= SH ? 0 : (m >= NOP ? NEL : ((m - SH) * NEL + (NOP - SH) - 1) / (NOP - SH));
}

template <int LEVEL>
__global__ __launch_bounds__(64 * kLadWaves) void fwd_ladder_kernel(const u32x4* __restrict__ ops,
                                                                       const uint16_t* __restrict__ src,
                                                                       float* __restrict__ sink,
                                                                       unsigned long long* __restrict__ clocks,
                                                                       int iters, float c) {
  constexpr int D = kLadD, NKS = D / 16, NDB = D / 32, BC = kTileTokens, NKB = BC / 32, TILE = kLadTile;
  constexpr int NB = kLadBuffers, LA = 3, NPV = 4 * NDB, NS = NKS * NKB, NOP = NPV + NS, NEL = 16 * NKB;
  constexpr int SH = 3, VOFF = NB * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NB * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Random operand registers (level 0/1 A operands, Q^T, initial P).
  u32x4 areg[8], qf[NKS], pb[NKB][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) areg[j] = ops[j * 64 + lane];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = ops[(8 + s) * 64 + lane];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    pb[kb][0] = ops[(16 + 2 * kb) * 64 + lane];
    pb[kb][1] = ops[(17 + 2 * kb) * 64 + lane];
  }
  // Fill every LDS buffer with random tiles (plain loads and stores).
  for (int i = tid; i < 2 * NB * TILE / 16; i += 64 * kLadWaves)
    reinterpret_cast<u32x4*>(smem)[i] = reinterpret_cast<const u32x4*>(src)[i % (kLadSrcTiles * TILE / 16)];
  __syncthreads();

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  f32x16 sacc[2][NKB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[t][kb][i] = 0.f;
  float lsum = 0.f;

  // The kernel's LDS read addresses.
  const uint32_t base = lds_addr(smem);
  uint32_t kaddr[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kaddr[s] = base + VOFF + (uint32_t)tile_off<D>(l32, 2 * s + g);
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
  u32x2 lo[LA + 1], hi[LA + 1];
  u32x4 kq[LA + 1];
  auto read_pv = [&](auto mc, auto vbc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value, VB = decltype(vbc)::value, b = m % (LA + 1);
    constexpr int gi = m / NDB, db = m % NDB;
    constexpr int OFF = VB * TILE + (32 * (gi >> 1) + 16 * (gi & 1)) * D * 2;
    lo[b] = ds_read_tr16_off<OFF>(vaddr[db][0]);
    hi[b] = ds_read_tr16_off<OFF>(vaddr[db][1]);
  };
  auto read_s = [&](auto mc, auto jc, auto kbc) __attribute__((always_inline)) {
    constexpr int b = decltype(mc)::value % (LA + 1), j = decltype(jc)::value, KB = decltype(kbc)::value;
    constexpr int s = j / NKB, kb = j % NKB;
    kq[b] = ds_read_b128_off<KB * TILE + kb * 32 * D * 2>(kaddr[s]);
  };

  // Tile loads (level 5): this wave's pieces of a 16 KB tile, as the kernel.
  using Dma = TileBufDma<D, kLadWaves, BC>;
  constexpr int NPIECE = Dma::kPerWave;
  Dma dma;
  dma.init(wave, lane);

  // One tile: the 32-MFMA stream (P V from V buffer VB, scores into sn
  // from K buffer KB), with valu(m) in slot m.
  auto stream = [&](auto kbc, auto vbc, auto vbnc, f32x16(&sn)[NKB], auto&& valu) __attribute__((always_inline)) {
    auto reads_after = [](int m) {
      int n = 0;
      for (int k = m + 1; k <= m + LA; ++k) n += (k < NPV || k >= NOP) ? 2 : 1;
      return n;
    };
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (LEVEL >= 2) {
        if constexpr (m < NPV) read_pv(mc, vbc);
        else if constexpr (m < NOP) read_s(mc, std::integral_constant<int, m - NPV>{}, kbc);
        else read_pv(std::integral_constant<int, m - NOP>{}, vbnc);
      }
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (LEVEL == 0) {
        // Four independent accumulators over the output registers.
        oacc[m & 3] = mfma32(areg[m & 7], qf[(m + (m >> 3)) & 7], oacc[m & 3]);
      } else if constexpr (m < NPV) {
        constexpr int gi = m / NDB, db = m % NDB;
        u32x4 a;
        if constexpr (LEVEL >= 2) {
          lgkm_wait<reads_after(m)>(lo[b], hi[b]);
          a = u32x4{lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        } else {
          a = areg[m & 7];
        }
        oacc[db] = mfma32(a, pb[gi >> 1][gi & 1], oacc[db]);
      } else {
        constexpr int j = m - NPV, s = j / NKB, kb = j % NKB;
        u32x4 a;
        if constexpr (LEVEL >= 2) {
          lgkm_wait<reads_after(m)>(kq[b]);
          a = kq[b];
        } else {
          a = areg[(j + 3) & 7];
        }
        if constexpr (s == 0) sn[kb] = mfma32(a, qf[0], f32x16{});
        else sn[kb] = mfma32(a, qf[s], sn[kb]);
      }
      valu(mc);
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<NOP>(run);
  };

  auto tile = [&](int it, auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    // Register operands count as changed every tile, so that no level's
    // score chains (which restart every tile) can be hoisted out of the loop.
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(areg[j]));
    f32x16(&sc)[NKB] = sacc[I % 2];
    float xs[NEL], ps[NEL], l4[4] = {0.f, 0.f, 0.f, 0.f};
    auto scale_stage = [&](int e) __attribute__((always_inline)) { xs[e] = sc[e >> 4][e & 15] * c; };
    auto exp_stage = [&](int e) __attribute__((always_inline)) { ps[e] = fast_exp2(xs[e]); };
    auto sum_stage = [&](int e) __attribute__((always_inline)) {
      const int kb = e >> 4, i = e & 15;
      l4[i & 3] += ps[e];
      asm volatile("" : "+v"(l4[i & 3]));
      if (i & 1) pb[kb][i >> 3][(i & 7) >> 1] = pack_bf16(ps[e - 1], ps[e]);
    };
    auto valu = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (LEVEL >= 5) {
        constexpr int DMA_EVERY = NOP / (2 * NPIECE);
        if constexpr (m % DMA_EVERY == DMA_EVERY / 2) {
          constexpr int k = m / DMA_EVERY;
          const uint16_t* t = src + (size_t)((it * 4 + I) % kLadSrcTiles) * BC * D;
          if constexpr (k < NPIECE) dma.load_piece(k, smem + ((I + 1) % NB) * TILE, t, 0, BC);
          else dma.load_piece(k - NPIECE, smem + VOFF + ((I + 3) % NB) * TILE, t, 0, BC);
        }
      }
      if constexpr (LEVEL >= 3) {
#pragma unroll
        for (int e = lad_first(m - 2, SH, NOP, NEL); e < lad_first(m - 1, SH, NOP, NEL); ++e) sum_stage(e);
#pragma unroll
        for (int e = lad_first(m - 1, SH, NOP, NEL); e < lad_first(m, SH, NOP, NEL); ++e) exp_stage(e);
#pragma unroll
        for (int e = lad_first(m, SH, NOP, NEL); e < lad_first(m + 1, SH, NOP, NEL); ++e) scale_stage(e);
      }
    };
    stream(std::integral_constant<int, (I + 1) % NB>{}, std::integral_constant<int, (I + NB - 1) % NB>{},
           std::integral_constant<int, I>{}, sacc[1 - I % 2], valu);
    if constexpr (LEVEL >= 3) {
#pragma unroll
      for (int e = lad_first(NOP - 2, SH, NOP, NEL); e < NEL; ++e) {
        if (e >= lad_first(NOP - 1, SH, NOP, NEL)) exp_stage(e);
        sum_stage(e);
      }
      lsum += (l4[0] + l4[1]) + (l4[2] + l4[3]);
    } else {
      // The scores are not consumed below level 3; keep them computed.
      asm volatile("" ::"v"(sacc[1 - I % 2][0]), "v"(sacc[1 - I % 2][1]));
    }
    if constexpr (LEVEL >= 5) wait_vmem_but<NPIECE>();
    if constexpr (LEVEL >= 4) phase_barrier();
  };

  // The first operand reads of the first tile.
  if constexpr (LEVEL >= 2) {
    static_for<LA>([&](auto mc) __attribute__((always_inline)) {
      read_pv(mc, std::integral_constant<int, NB - 1>{});
    });
  }
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    tile(it, std::integral_constant<int, 0>{});
    tile(it, std::integral_constant<int, 1>{});
    tile(it, std::integral_constant<int, 2>{});
    tile(it, std::integral_constant<int, 3>{});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wait_vmem();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = lsum;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += oacc[db][i];
  sink[(size_t)blockIdx.x * 64 * kLadWaves + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
    clocks[0] = c1 - c0;
    clocks[1] = r1 - r0;
  }
}

// Levels 6-10: one wave per SIMD (4 waves per block), each holding 64 query
// rows as two 32-row blocks, so that every LDS operand read feeds two MFMAs
// (one per row block).  Same matrix work per block as the other levels.
// The output accumulators (128 registers) must live in AGPRs and the score
// accumulators, which the vector unit reads, in VGPRs; the products are
// written as inline assembly with those register classes, since the
// compiler otherwise puts the scores in AGPRs and copies every element out.
// Hazards the compiler cannot see in them are covered by distance: an
// output accumulator recurs every 8 MFMAs, a score chain every 4, scores
// are read a tile after they are written, and P is double-buffered.
template <int LEVEL>
struct W64Features {
  // 6: operand reads only; 7: softmax, barrier per tile, tile loads;
  // 8: softmax only; 9: softmax and barrier per tile; 10: as 7 with the
  // barrier every second tile.
  static constexpr bool kSoftmax = LEVEL >= 7;
  static constexpr int kBarrier = (LEVEL == 7 || LEVEL == 9) ? 1 : (LEVEL == 10 ? 2 : 0);
  static constexpr bool kDma = LEVEL == 7 || LEVEL == 10;
};

template <int LEVEL>
__global__ __launch_bounds__(64 * kLadWaves / 2) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_ladder_w64_kernel(const u32x4* __restrict__ ops, const uint16_t* __restrict__ src, float* __restrict__ sink,
                           unsigned long long* __restrict__ clocks, int iters, float c) {
  constexpr int NW = kLadWaves / 2, QB = 2;
  constexpr int D = kLadD, NKS = D / 16, NDB = D / 32, BC = kTileTokens, NKB = BC / 32, TILE = kLadTile;
  constexpr int NB = kLadBuffers, LA = 3, NPV = 4 * NDB, NS = NKS * NKB, NOP = NPV + NS;
  // P is double-buffered: the softmax of tile t writes pbuf[t % 2] while the
  // P V products of iteration t read pbuf[(t + 1) % 2], so no vector write
  // lands on a register an issued MFMA still reads.
  constexpr int NSLOT = QB * NOP, NEL = QB * 16 * NKB, SH = 3, VOFF = NB * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NB * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  u32x4 qf[QB][NKS], pbuf[2][QB][NKB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[qb][s] = ops[((8 + s + qb) & 15) * 64 + lane];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pbuf[t][qb][kb][0] = ops[(16 + 2 * kb) * 64 + lane];
        pbuf[t][qb][kb][1] = ops[(17 + 2 * kb) * 64 + lane];
      }
  }
  for (int i = tid; i < 2 * NB * TILE / 16; i += 64 * NW)
    reinterpret_cast<u32x4*>(smem)[i] = reinterpret_cast<const u32x4*>(src)[i % (kLadSrcTiles * TILE / 16)];
  __syncthreads();

  f32x16 oacc[QB][NDB], sacc[2][QB][NKB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][db][i] = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[t][qb][kb][i] = 0.f;
  }
  float lsum = 0.f;

  const uint32_t base = lds_addr(smem);
  uint32_t kaddr[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) kaddr[s] = base + VOFF + (uint32_t)tile_off<D>(l32, 2 * s + g);
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
  u32x2 lo[LA + 1], hi[LA + 1];
  u32x4 kq[LA + 1];
  auto read_pv = [&](auto mc, auto vbc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value, VB = decltype(vbc)::value, b = m % (LA + 1);
    constexpr int gi = m / NDB, db = m % NDB;
    constexpr int OFF = VB * TILE + (32 * (gi >> 1) + 16 * (gi & 1)) * D * 2;
    lo[b] = ds_read_tr16_off<OFF>(vaddr[db][0]);
    hi[b] = ds_read_tr16_off<OFF>(vaddr[db][1]);
  };
  auto read_s = [&](auto mc, auto jc, auto kbc) __attribute__((always_inline)) {
    constexpr int b = decltype(mc)::value % (LA + 1), j = decltype(jc)::value, KB = decltype(kbc)::value;
    constexpr int s = j / NKB, kb = j % NKB;
    kq[b] = ds_read_b128_off<KB * TILE + kb * 32 * D * 2>(kaddr[s]);
  };
  using Dma = TileBufDma<D, NW, BC>;
  constexpr int NPIECE = Dma::kPerWave;
  Dma dma;
  dma.init(wave, lane);

  // Op m: one operand read, then two MFMAs (row blocks 0 and 1); valu(2m+qb)
  // in each MFMA slot.
  auto stream = [&](auto kbc, auto vbc, auto vbnc, f32x16(&sn)[QB][NKB], u32x4(&pb)[QB][NKB][2], auto&& valu)
                    __attribute__((always_inline)) {
    auto reads_after = [](int m) {
      int n = 0;
      for (int k = m + 1; k <= m + LA; ++k) n += (k < NPV || k >= NOP) ? 2 : 1;
      return n;
    };
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NPV) read_pv(mc, vbc);
      else if constexpr (m < NOP) read_s(mc, std::integral_constant<int, m - NPV>{}, kbc);
      else read_pv(std::integral_constant<int, m - NOP>{}, vbnc);
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (m < NPV) {
        constexpr int gi = m / NDB, db = m % NDB;
        lgkm_wait<reads_after(m)>(lo[b], hi[b]);
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        static_for<QB>([&](auto qc) __attribute__((always_inline)) {
          constexpr int qb = decltype(qc)::value;
          // The output accumulators live in AGPRs (the score accumulators,
          // which the vector unit reads, in VGPRs): the product is written
          // with an AGPR accumulator constraint.  The same accumulator
          // recurs every 8 MFMAs and P was written a tile earlier.
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+a"(oacc[qb][db])
                       : "v"(a), "v"(pb[qb][gi >> 1][gi & 1]));
          valu(std::integral_constant<int, 2 * m + qb>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      } else {
        constexpr int j = m - NPV, s = j / NKB, kb = j % NKB;
        lgkm_wait<reads_after(m)>(kq[b]);
        static_for<QB>([&](auto qc) __attribute__((always_inline)) {
          constexpr int qb = decltype(qc)::value;
          // Score accumulators in VGPRs (the vector unit reads them), Q^T in
          // AGPRs as the B operand.  A chain recurs every 4 MFMAs; its scores
          // are read a tile later.
          if constexpr (s == 0)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sn[qb][kb]) : "v"(kq[b]), "a"(qf[qb][0]));
          else
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sn[qb][kb]) : "v"(kq[b]), "a"(qf[qb][s]));
          valu(std::integral_constant<int, 2 * m + qb>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    };
    static_for<NOP>(run);
  };

  auto tile = [&](int it, auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    f32x16(&sc)[QB][NKB] = sacc[I % 2];
    u32x4(&pw)[QB][NKB][2] = pbuf[I % 2];
    float xs[NEL], ps[NEL], l4[4] = {0.f, 0.f, 0.f, 0.f};
    // Element e: key group gi = e / 16 (16 keys, P register pb[qb][gi/2][gi%2]),
    // row block qb = (e / 8) % 2, j = e % 8 within the group's half.
    auto elem = [](int e, int& qb, int& kb, int& i) {
      const int gi = e >> 4;
      qb = (e >> 3) & 1;
      kb = gi >> 1;
      i = 8 * (gi & 1) + (e & 7);
    };
    auto scale_stage = [&](int e) __attribute__((always_inline)) {
      int qb, kb, i;
      elem(e, qb, kb, i);
      xs[e] = sc[qb][kb][i] * c;
    };
    auto exp_stage = [&](int e) __attribute__((always_inline)) { ps[e] = fast_exp2(xs[e]); };
    auto sum_stage = [&](int e) __attribute__((always_inline)) {
      int qb, kb, i;
      elem(e, qb, kb, i);
      l4[e & 3] += ps[e];
      asm volatile("" : "+v"(l4[e & 3]));
      if (e & 1) pw[qb][kb][i >> 3][(i & 7) >> 1] = pack_bf16(ps[e - 1], ps[e]);
    };
    using F = W64Features<LEVEL>;
    auto valu = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (F::kDma) {
        constexpr int DMA_EVERY = NSLOT / (2 * NPIECE);
        if constexpr (m % DMA_EVERY == DMA_EVERY / 2) {
          constexpr int k = m / DMA_EVERY;
          const uint16_t* t = src + (size_t)((it * 4 + I) % kLadSrcTiles) * BC * D;
          if constexpr (k < NPIECE) dma.load_piece(k, smem + ((I + 2) % NB) * TILE, t, 0, BC);
          else dma.load_piece(k - NPIECE, smem + VOFF + ((I + 3) % NB) * TILE, t, 0, BC);
        }
      }
      if constexpr (F::kSoftmax) {
#pragma unroll
        for (int e = lad_first(m - 2, SH, NSLOT, NEL); e < lad_first(m - 1, SH, NSLOT, NEL); ++e) sum_stage(e);
#pragma unroll
        for (int e = lad_first(m - 1, SH, NSLOT, NEL); e < lad_first(m, SH, NSLOT, NEL); ++e) exp_stage(e);
#pragma unroll
        for (int e = lad_first(m, SH, NSLOT, NEL); e < lad_first(m + 1, SH, NSLOT, NEL); ++e) scale_stage(e);
      }
    };
    stream(std::integral_constant<int, (I + 1) % NB>{}, std::integral_constant<int, (I + NB - 1) % NB>{},
           std::integral_constant<int, I>{}, sacc[1 - I % 2], pbuf[1 - I % 2], valu);
    if constexpr (F::kSoftmax) {
#pragma unroll
      for (int e = lad_first(NSLOT - 2, SH, NSLOT, NEL); e < NEL; ++e) {
        if (e >= lad_first(NSLOT - 1, SH, NSLOT, NEL)) exp_stage(e);
        sum_stage(e);
      }
      lsum += (l4[0] + l4[1]) + (l4[2] + l4[3]);
      if constexpr (F::kDma) wait_vmem_but<2 * NPIECE>();
      if constexpr (F::kBarrier == 1 || (F::kBarrier == 2 && (I & 1))) phase_barrier();
    } else {
      asm volatile("" ::"v"(sacc[1 - I % 2][0][0]), "v"(sacc[1 - I % 2][0][1]), "v"(sacc[1 - I % 2][1][0]),
                   "v"(sacc[1 - I % 2][1][1]));
    }
  };

  static_for<LA>([&](auto mc) __attribute__((always_inline)) { read_pv(mc, std::integral_constant<int, NB - 1>{}); });
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    tile(it, std::integral_constant<int, 0>{});
    tile(it, std::integral_constant<int, 1>{});
    tile(it, std::integral_constant<int, 2>{});
    tile(it, std::integral_constant<int, 3>{});
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wait_vmem();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = lsum;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) s += oacc[qb][db][i];
  sink[(size_t)blockIdx.x * 64 * kLadWaves + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
    clocks[0] = c1 - c0;
    clocks[1] = r1 - r0;
  }
}

}  // namespace
}  // namespace ra

extern "C" int ra_fwd_ladder_probe(int level, const void* operands, const void* tiles, float* sink,
                                   unsigned long long* clocks, int blocks, int iters, float c, void* stream) {
  if (!operands || !tiles || !sink || !clocks) return RA_ERR_NULL;
  if (level < 0 || level > 10 || blocks < 1 || iters < 1) return RA_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(64 * ra::kLadWaves);
  const auto* o = static_cast<const ra::u32x4*>(operands);
  const auto* t = static_cast<const uint16_t*>(tiles);
  switch (level) {
    case 0: hipLaunchKernelGGL(ra::fwd_ladder_kernel<0>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
    case 1: hipLaunchKernelGGL(ra::fwd_ladder_kernel<1>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
    case 2: hipLaunchKernelGGL(ra::fwd_ladder_kernel<2>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
    case 3: hipLaunchKernelGGL(ra::fwd_ladder_kernel<3>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
    case 4: hipLaunchKernelGGL(ra::fwd_ladder_kernel<4>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
    case 5: hipLaunchKernelGGL(ra::fwd_ladder_kernel<5>, grid, block, 0, st, o, t, sink, clocks, iters, c); break;
#define RA_LADDER_W64(L)                                                                                    \
  case L:                                                                                                   \
    hipLaunchKernelGGL(ra::fwd_ladder_w64_kernel<L>, grid, dim3(64 * ra::kLadWaves / 2), 0, st, o, t, sink, \
                       clocks, iters, c);                                                                   \
    break;
    RA_LADDER_W64(6)
    RA_LADDER_W64(7)
    RA_LADDER_W64(8)
    RA_LADDER_W64(9)
    RA_LADDER_W64(10)
#undef RA_LADDER_W64
    default: return RA_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? RA_OK : RA_ERR_HIP;
}

// Backward of one ring step against one KV chunk.
//
// The pages give no backward; this is the textbook softmax-attention gradient
// with the probabilities recomputed from the final log-sum-exp of the forward
// walk (so no merge is needed in the backward):
//   P = exp(scale q k^T - lse), dP = dO v^T, dS = P (dP - D), D = rowsum(dO o),
//   dq += scale dS k,  dk += scale dS^T q,  dv += P^T dO.
//
// Two launches per step, none with atomics (results are deterministic):
//  * dq kernel -- a block owns 256 query rows (32 per wave, Q^T and dO^T in
//    registers as MFMA B operands, like the forward) and streams 64-key tiles
//    of K and V (row-major LDS tiles, A operands; K^T is read from the same
//    tile through the transposing LDS read).  Scores are computed transposed
//    (S^T = K Q^T, dP^T = V dO^T), so lse and D are per-lane scalars and dS^T
//    feeds dq^T += K^T dS^T directly.
//  * key kernel -- a block owns 128 keys of the chunk; the two waves of a
//    SIMD share 32 of them, one holding K (S, P, dv) and the other V (dP, dS,
//    dk), and stream 64-query tiles of Q and dO (row-major; Q^T and dO^T
//    through the transposing read).  Here S = Q K^T has a lane per key, so P
//    and dS feed dv^T += dO^T P and dk^T += Q^T dS directly; lse and D of the
//    tile's queries are staged in LDS, and P passes from one wave to the
//    other through LDS.
// The price of avoiding atomics is recomputing S and dP in both launches:
// 14 d flop per (query, key) pair executed for the 10 d of the gradient.
#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kPosInf = __builtin_inff();

// One ds_write_b128 of v at LDS byte address addr + OFF, as inline assembly
// beside the inline-assembly reads; its completion is waited for explicitly
// (s_waitcnt lgkmcnt(0)) before the barrier after which another wave reads it.
template <int OFF>
__device__ __forceinline__ void ds_write_b128_off(uint32_t addr, const u32x4& v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF) : "memory");
}

// ---------------------------------------------------------------------------
// dq kernel.
// ---------------------------------------------------------------------------
constexpr int kDqWaves = 8;  // waves per block; waves w and w + 4 share a SIMD
constexpr int kDqRowsPerWave = 32;
constexpr int kDqLookahead = 2;  // MFMAs whose LDS operands are read ahead

// dq^T += scale K^T dS^T for one ring step.  A block holds 256 query rows,
// 32 per wave (Q^T and dO^T in registers as MFMA B operands), and walks the
// chunk's keys in 64-key tiles.  Per tile a wave runs two phases:
//   MFMA phase of tile t:  dq^T += K^T(t-1) dS^T(t-1), S^T(t) = K(t) Q^T,
//                          dP^T(t) = V(t) dO^T   (48 MFMAs at d = 128);
//   vector phase of tile t: P = exp2(S scale - lse) (masked where needed),
//                          dS = P (dP - D), packed to bf16.
// Waves 4..7 run the same code one phase behind waves 0..3 (one extra
// barrier first), with a workgroup barrier between phases, so each SIMD's
// matrix core is fed by one wave while the other does the element-wise
// work.  K^T comes straight from the row-major K tile through
// ds_read_b64_tr_b16.  LDS operands are read LA MFMAs ahead with counted
// waits.  Tiles load two ahead of use: K into four LDS buffers (a phase
// reads K(t-1) and K(t)), V into three.
template <int D, bool DIAG>
__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lse2g, const float* __restrict__ Dg,
    float* __restrict__ dqg, int Sq, int Sk, int n_qtiles, int total_tiles, float scale_log2, float scale,
    int group, int qoff) {
  constexpr int NW = kDqWaves, NQW = kDqRowsPerWave, BR = NW * NQW, BC = kTileTokens;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = BC / 32, TILE = BC * D * 2, LA = kDqLookahead;
  constexpr int NQ = 4 * NDB, NS = 2 * NKS * NKB, NOP = NQ + NS;  // dq ops, then S and dP ops
  // LDS: V tiles in buffers 0..2 at [0, 3 TILE), K tiles in buffers 0..3 at
  // [KOFF, KOFF + 4 TILE); tile j uses K buffer j % 4 and V buffer j % 3.
  // Buffer offsets are added per read at run time (the vector unit is idle
  // in the MFMA phase), so one copy of the code serves every tile.
  constexpr int KOFF = 3 * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[7 * TILE];
  auto kbuf = [&](int b) __attribute__((always_inline)) { return smem + KOFF + b * TILE; };
  auto vbuf = [&](int b) __attribute__((always_inline)) { return smem + b * TILE; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const bool lead = wave < NW / 2;  // waves 4..7 run one phase behind
  int bh, qt;
  if constexpr (DIAG) {
    // Causal: the last query tiles see the most keys; they go first.
    longest_first(blockIdx.x, total_tiles / n_qtiles, bh, qt);
    qt = n_qtiles - 1 - qt;
  } else {
    const int t = xcd_remap(blockIdx.x, total_tiles);
    bh = t / n_qtiles;
    qt = t - bh * n_qtiles;
  }
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * NQW;
  const int qq = qw0 + l32;
  // Grouped-query attention: query head row bh reads key/value head bh / group.
  const uint16_t* __restrict__ kp = kg + (size_t)(bh / group) * Sk * D;
  const uint16_t* __restrict__ vp = vg + (size_t)(bh / group) * Sk * D;

  // Causal: query row q sees keys k <= q + qoff.
  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR + qoff);
  const int ntiles = (kend + BC - 1) / BC;
  const int wtiles = DIAG ? min(ntiles, max(0, (min(qw0 + NQW, Sq) - 1 + qoff) / BC + 1)) : ntiles;
  const int lim = DIAG ? min(Sk, qq + 1 + qoff) : Sk;  // keys at or past lim are masked

  TileBufDma<D, NW, BC> dma;
  dma.init(wave, lane);
  dma.load(kbuf(0), kp, 0, Sk);
  dma.load(kbuf(1), kp, BC, Sk);
  dma.load(kbuf(3), kp, 0, Sk);  // finite data for the dS = 0 product of tile 0
  dma.load(vbuf(0), vp, 0, Sk);
  dma.load(vbuf(1), vp, BC, Sk);

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
    lse2 = lse2g[(size_t)bh * Sq + qq];  // +inf for a row that saw no key: P = 0
    Dq = Dg[(size_t)bh * Sq + qq];
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  f32x16 sacc[NKB], pacc[NKB];
  u32x4 dsb[NKB][2];  // dS^T of the last vector phase, bf16 (B operand of dq^T)
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) dsb[kb][0] = dsb[kb][1] = u32x4{0, 0, 0, 0};

  const uint32_t base = lds_addr(smem);
  uint32_t kaddr[NKS];  // row-major operand (K or V) of lane l32, chunk pair s
#pragma unroll
  for (int s = 0; s < NKS; ++s) kaddr[s] = base + KOFF + (uint32_t)tile_off<D>(l32, 2 * s + g);
  uint32_t taddr[NDB][2];  // transposed K operand
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        taddr[db][tt] = base + KOFF + tile_off<D>(4 * g + m + 8 * tt, d >> 3) + ((d & 4) ? 8 : 0);
    }
  }

  // MFMA phase: dq^T from the K buffer at byte offset kpo (previous tile)
  // and dsb, then S^T from the K buffer at kbo and dP^T from the V buffer at
  // vbo (offsets from the first buffer of each kind; the vector unit is idle
  // in this phase, so adding them per read costs nothing).
  auto mfma_phase = [&](uint32_t kpo, uint32_t kbo, uint32_t vbo, auto&& hook) __attribute__((always_inline)) {
    u32x2 lo[LA + 1], hi[LA + 1];
    u32x4 rq[LA + 1];
    auto reads_after = [](int m) {
      int n = 0;
      for (int k = m + 1; k <= m + LA && k < NOP; ++k) n += (k < NQ) ? 2 : 1;
      return n;
    };
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      if constexpr (m < NQ) {
        // K^T block db for keys 32*(gi/2) + 16*(gi%2) .. +15.
        constexpr int gi = m / NDB, db = m % NDB;
        constexpr int OFF = (32 * (gi >> 1) + 16 * (gi & 1)) * D * 2;
        lo[b] = ds_read_tr16_off<OFF>(taddr[db][0] + kpo);
        hi[b] = ds_read_tr16_off<OFF>(taddr[db][1] + kpo);
      } else if constexpr (m < NOP) {
        // s-major: S kb0, S kb1, dP kb0, dP kb1 for each chunk pair s.
        constexpr int j = m - NQ, s = j / (2 * NKB), r = j % (2 * NKB), kb = r % NKB;
        if constexpr (r < NKB) rq[b] = ds_read_b128_off<kb * 32 * D * 2>(kaddr[s] + kbo);
        else rq[b] = ds_read_b128_off<kb * 32 * D * 2>(kaddr[s] + vbo - (uint32_t)KOFF);
      }
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      constexpr int N = reads_after(m);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (m < NQ) {
        constexpr int gi = m / NDB, db = m % NDB;
        lgkm_wait<N>(lo[b], hi[b]);
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        acc[db] = mfma32(a, dsb[gi >> 1][gi & 1], acc[db]);
      } else {
        constexpr int j = m - NQ, s = j / (2 * NKB), r = j % (2 * NKB), kb = r % NKB;
        lgkm_wait<N>(rq[b]);
        if constexpr (r < NKB) {
          if constexpr (s == 0) sacc[kb] = mfma32(rq[b], qf[0], f32x16{});
          else sacc[kb] = mfma32(rq[b], qf[s], sacc[kb]);
        } else {
          if constexpr (s == 0) pacc[kb] = mfma32(rq[b], df[0], f32x16{});
          else pacc[kb] = mfma32(rq[b], df[s], pacc[kb]);
        }
      }
      hook(mc);
    };
    static_for<LA>(issue);
    static_for<NOP>(run);
  };

  // Vector phase of tile tt: dS^T = P^T (dP^T - D) into dsb.
  auto vector_phase = [&](int tt) __attribute__((always_inline)) {
    const int k0 = tt * BC;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sacc[kb][i], scale_log2, -lse2));
        sacc[kb][i] = p * (pacc[kb][i] - Dq);
      }
    // Masked tiles (the diagonal band, the ragged tail) zero the entries of
    // keys at or past the lane's limit, whatever was computed for them, in a
    // pass of their own that full tiles skip.
    if ((k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0 + qoff)) {
      const int r = lim - k0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) >= r) sacc[kb][i] = 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dsb[kb][0] = pack8(sacc[kb], 0);
      dsb[kb][1] = pack8(sacc[kb], 8);
    }
  };

  // Tile tt's MFMA phase runs for 0 <= tt <= wtiles: at tt = 0 dS is still
  // zero (the K buffer it multiplies holds finite data), and at tt = wtiles
  // only its dq part is used.  One code shape for every tile.
  // On full chunks the phase also issues tile tt + 2's loads (this wave's K
  // pieces, then its V pieces), one piece every EVERY MFMAs.  Tiles past the
  // chunk load zeros that nothing reads.  On the diagonal chunk, where waves
  // run different tile counts, the loads go out together at the start of
  // the iteration (the per-wave branch costs the spread version registers).
  constexpr int NPW = decltype(dma)::kPerWave, NPC = 2 * NPW;
  auto load_piece = [&](int j, int k) __attribute__((always_inline)) {
    if (k < NPW) dma.load_piece(k, kbuf(j & 3), kp, j * BC, Sk);
    else dma.load_piece(k - NPW, vbuf(j % 3), vp, j * BC, Sk);
  };
  auto mfma_tile = [&](int tt) __attribute__((always_inline)) {
    constexpr int EVERY = NOP / NPC;
    if (tt <= wtiles)
      mfma_phase((uint32_t)(((tt + 3) & 3) * TILE), (uint32_t)((tt & 3) * TILE), (uint32_t)((tt % 3) * TILE),
                 [&](auto mc) __attribute__((always_inline)) {
                   constexpr int m = decltype(mc)::value;
                   if constexpr (!DIAG && m % EVERY == EVERY / 2 && m / EVERY < NPC) load_piece(tt + 2, m / EVERY);
                 });
  };
  auto vector_tile = [&](int tt) __attribute__((always_inline)) {
    if (tt >= 0 && tt < wtiles) vector_phase(tt);
  };
  // Iteration u: MFMA phase of tile u (reads K(u-1), K(u), V(u)), vector
  // phase of tile u.  The MFMA phase loads tile u + 2 into the K and V
  // buffers of tiles u - 2 and u - 1, whose last readers finished in the
  // MFMA phase of tile u - 1 two phases back (for either wave group); the
  // iteration ends waiting for that load, and the barrier after the trailing
  // group's wait comes two phases before anyone reads tile u + 2.
  wait_vmem();
  phase_barrier();
  if (!lead) phase_barrier();
  for (int u = 0; u <= ntiles; ++u) {
    if (DIAG && u + 2 < ntiles) {
#pragma unroll
      for (int k = 0; k < NPC; ++k) load_piece(u + 2, k);
    }
    mfma_tile(u);
    phase_barrier();
    vector_tile(u);
    wait_vmem();
    phase_barrier();
  }
  if (lead) phase_barrier();

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
// dk/dv kernel, one pass: the two waves of a SIMD share 32 keys.
// ---------------------------------------------------------------------------
constexpr int kKvfWaves = 8;  // waves w and w + 4 share a SIMD and the same 32 keys
constexpr int kKvfKeysPerWave = 32;
constexpr int kKvfLookahead = 2;  // MFMAs whose LDS operands are read ahead

// dv^T += dO^T P and dk^T += scale Q^T dS for one ring step in one launch.
// A block holds 128 keys.  Waves w and w + 4 (one SIMD) hold the same 32
// keys and split the work:
//   wave w (S, P, dv): MFMA phase of tile t: dv^T += dO^T(t-1) P(t-1),
//     S(t) = Q(t) K^T; vector phase: P = exp2(S scale - lse) (masked), packed
//     to bf16, kept as its own B operand and written to LDS for its partner;
//   wave w + 4 (dP, dS, dk), one phase behind: MFMA phase of tile t:
//     dk^T += Q^T(t-1) dS(t-1), dP(t) = dO(t) V^T; vector phase: reads P(t)
//     (written in the phase before), dS = P (dP - D), packed to bf16.
// S is computed once per (query, key) pair in this kernel, and each wave
// holds one accumulator and one register operand (K or V), which keeps two
// waves per SIMD within the register file.  Both roles run the same MFMA phase code on runtime buffer offsets;
// only the vector phases differ.  dS is formed from the bf16 P that also
// feeds dv.  Tiles of Q and dO stream through four LDS buffers each, two
// tiles ahead; the lse and D rows of a tile sit beside them.
template <int D, bool DIAG>
__global__ __launch_bounds__(64 * kKvfWaves) void bwd_kvf_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lse2g, const float* __restrict__ Dg,
    float* __restrict__ dkg, float* __restrict__ dvg, int Sq, int Sk, int n_ktiles, int total_tiles,
    float scale_log2, float scale, int group, int qoff) {
  constexpr int NW = kKvfWaves, NKW = kKvfKeysPerWave, BK = (NW / 2) * NKW, BQ = kTileTokens;
  constexpr int NKS = D / 16, NDB = D / 32, NQB = BQ / 32, TILE = BQ * D * 2, LA = kKvfLookahead;
  constexpr int NX = 4 * NDB, NS = NKS * NQB, NOP = NX + NS;
  // LDS: Q tiles in buffers 0..3, dO tiles in buffers 0..3 at DOFF, the rows'
  // lse and D (64 floats per tile each), then one P tile per wave pair (bf16,
  // word k of lane l at k * 1024 + 16 l); tile j uses buffer j % 4.
  constexpr int DOFF = 4 * TILE, LOFF = 8 * TILE, DLOFF = LOFF + 4 * BQ * 4, POFF = DLOFF + 4 * BQ * 4;
  constexpr int PSLOT = 2 * NQB * 64 * 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[POFF + (NW / 2) * PSLOT];
  auto qbuf = [&](int b) __attribute__((always_inline)) { return smem + b * TILE; };
  auto dbuf = [&](int b) __attribute__((always_inline)) { return smem + DOFF + b * TILE; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const bool lead = wave < NW / 2;  // S, P, dv; waves 4..7 (dP, dS, dk) run one phase behind
  const int pw = wave & (NW / 2 - 1);  // key group of the wave pair
  // Key/value head row bhk (its query heads are bhk * group + [0, group)) and
  // key tile kt.  Causal: low key tiles see the most queries; they go first.
  int bhk, kt;
  if constexpr (DIAG) {
    longest_first(blockIdx.x, total_tiles / n_ktiles, bhk, kt);
  } else {
    const int t = xcd_remap(blockIdx.x, total_tiles);
    bhk = t / n_ktiles;
    kt = t - bhk * n_ktiles;
  }
  const int kb0 = kt * BK;
  const int kw0 = kb0 + pw * NKW;
  const int kk = kw0 + l32;
  // Query-side rows of the query head being walked (set per head below).
  const uint16_t* __restrict__ qp = qg;
  const uint16_t* __restrict__ dp = dog;
  const float* __restrict__ lp = lse2g;
  const float* __restrict__ Dp = Dg;

  // Query tiles qs .. ntq-1; this pair's keys see tiles from ws on (causal:
  // query q sees keys <= q + qoff).  A block whose keys no query sees skips
  // the walk and adds zero.
  const int ntq = (Sq + BQ - 1) / BQ;
  const int qs = DIAG ? min(max(0, kb0 - qoff) / BQ, ntq) : 0;
  const int ws = DIAG ? min(max(qs, max(0, kw0 - qoff) / BQ), ntq) : qs;

  TileBufDma<D, NW, BQ> dma;
  dma.init(wave, lane);
  // lse and D of tile j (rows clamped to Sq - 1) into their LDS slots: one
  // 4-byte load per lane, issued by waves 0 and 1.
  auto load_rows = [&](int j) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int row = min(j * BQ + lane, Sq - 1);
    if (wave == 0) __builtin_amdgcn_global_load_lds(lp + row, (lds_void*)(smem + LOFF + (j & 3) * BQ * 4), 4, 0, 0);
    if (wave == 1) __builtin_amdgcn_global_load_lds(Dp + row, (lds_void*)(smem + DLOFF + (j & 3) * BQ * 4), 4, 0, 0);
#else
    (void)j, (void)lp, (void)Dp;
#endif
  };
  auto load_tile = [&](int j) __attribute__((always_inline)) {
    dma.load(qbuf(j & 3), qp, j * BQ, Sq);
    dma.load(dbuf(j & 3), dp, j * BQ, Sq);
    load_rows(j);
  };
  // Piece k of tile j's loads: this wave's Q pieces, its dO pieces, then the
  // lse / D rows (waves 0 and 1).
  constexpr int NPW = decltype(dma)::kPerWave, NPC = 2 * NPW + 1;
  auto load_piece = [&](int j, int k) __attribute__((always_inline)) {
    if (k < NPW) dma.load_piece(k, qbuf(j & 3), qp, j * BQ, Sq);
    else if (k < 2 * NPW) dma.load_piece(k - NPW, dbuf(j & 3), dp, j * BQ, Sq);
    else load_rows(j);
  };

  // The register operand: K rows (S = Q K^T) or V rows (dP = dO V^T) of key kk.
  u32x4 kvf[NKS];
  {
    const uint16_t* row = (lead ? kg : vg) + ((size_t)bhk * Sk + kk) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s) kvf[s] = (kk < Sk) ? ld16(row + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  f32x16 sacc[NQB];  // S (waves 0..3) or dP (waves 4..7) of the current tile
  u32x4 yb[NQB][2];  // P or dS of the last vector phase, bf16 (B operand of the product)

  const uint32_t base = lds_addr(smem);
  // Row-major operand of the scores (Q or dO) and transposed operand of the
  // product (dO^T or Q^T), as buffer-0 addresses.
  const uint32_t roff = lead ? 0u : (uint32_t)DOFF, xoff = lead ? (uint32_t)DOFF : 0u;
  uint32_t raddr[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) raddr[s] = base + roff + (uint32_t)tile_off<D>(l32, 2 * s + g);
  uint32_t taddr[NDB][2];
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        taddr[db][tt] = base + xoff + tile_off<D>(4 * g + m + 8 * tt, d >> 3) + ((d & 4) ? 8 : 0);
    }
  }
  const uint32_t laddr = base + LOFF + (uint32_t)(4 * g) * 4;  // this lane's rows 4g .. 4g+3 of a tile's lse
  const uint32_t paddr = base + POFF + (uint32_t)(pw * PSLOT + lane * 16);

  // MFMA phase: acc from the X buffer at xo (previous tile) and yb, then the
  // scores from the buffer at bo.
  auto mfma_phase = [&](uint32_t xo, uint32_t bo, auto&& hook) __attribute__((always_inline)) {
    u32x2 lo[LA + 1], hi[LA + 1];
    u32x4 rq[LA + 1];
    auto reads_after = [](int m) {
      int n = 0;
      for (int k = m + 1; k <= m + LA && k < NOP; ++k) n += (k < NX) ? 2 : 1;
      return n;
    };
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      if constexpr (m < NX) {
        constexpr int gi = m / NDB, db = m % NDB;
        constexpr int OFF = (32 * (gi >> 1) + 16 * (gi & 1)) * D * 2;
        lo[b] = ds_read_tr16_off<OFF>(taddr[db][0] + xo);
        hi[b] = ds_read_tr16_off<OFF>(taddr[db][1] + xo);
      } else if constexpr (m < NOP) {
        constexpr int j = m - NX, s = j / NQB, qb = j % NQB;
        rq[b] = ds_read_b128_off<qb * 32 * D * 2>(raddr[s] + bo);
      }
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      constexpr int N = reads_after(m);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (m < NX) {
        constexpr int gi = m / NDB, db = m % NDB;
        lgkm_wait<N>(lo[b], hi[b]);
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        acc[db] = mfma32(a, yb[gi >> 1][gi & 1], acc[db]);
      } else {
        constexpr int j = m - NX, s = j / NQB, qb = j % NQB;
        lgkm_wait<N>(rq[b]);
        if constexpr (s == 0) sacc[qb] = mfma32(rq[b], kvf[0], f32x16{});
        else sacc[qb] = mfma32(rq[b], kvf[s], sacc[qb]);
      }
      hook(mc);
    };
    static_for<LA>(issue);
    static_for<NOP>(run);
  };

  // Vector phase of tile tt, waves 0..3: P into yb and the pair's LDS slot.
  // Row i of accumulator qb is query 32*qb + 8*(i/4) + 4g + i%4 of the tile.
  auto vector_p = [&](int tt) __attribute__((always_inline)) {
    const int q0 = tt * BQ;
    const bool masked = (q0 + BQ > Sq) || (DIAG && q0 + qoff < kw0 + NKW);
    const uint32_t lo_ = laddr + (uint32_t)((tt & 3) * BQ * 4);
    // The lse values of accumulator qb's 32 rows, four rows per read, are
    // requested together and consumed in order with counted waits.
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      u32x4 lrs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) lrs[j] = ds_read_b128_off<0>(lo_ + (qb * 32 + 8 * j) * 4);
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        lgkm_wait<3 - j>(lrs[j]);
        const u32x4 lr = lrs[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          // lse2 is +inf for a row that saw no key: P = 0.
          sacc[qb][i] = fast_exp2(fmaf(sacc[qb][i], scale_log2, -as_float(lr[e])));
        }
      });
    }
    // Masked tiles (the diagonal band, the ragged tail) zero the entries of
    // rows past the chunk or of keys after the query, in a pass of their own
    // that full tiles skip.  dS of those entries is then zero too.
    if (masked) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = q0 + qb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (qi >= Sq || (DIAG && kk > qi + qoff)) sacc[qb][i] = 0.f;
        }
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      yb[qb][0] = pack8(sacc[qb], 0);
      yb[qb][1] = pack8(sacc[qb], 8);
    }
    // Hand P to the partner wave; the writes complete before the barrier
    // after which it reads them.
    static_for<2 * NQB>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      ds_write_b128_off<k * 1024>(paddr, yb[k >> 1][k & 1]);
    });
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Vector phase of tile tt, waves 4..7: dS = P (dP - D) into yb, with P(tt)
  // from the partner's slot.
  auto vector_ds = [&](int tt) __attribute__((always_inline)) {
    const uint32_t lo_ = laddr + (uint32_t)((tt & 3) * BQ * 4);
    u32x4 pk[NQB][2];
    static_for<2 * NQB>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      pk[k >> 1][k & 1] = ds_read_b128_off<k * 1024>(paddr);
    });
    static_for<2 * NQB>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      lgkm_wait<0>(pk[k >> 1][k & 1]);
    });
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      u32x4 drs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) drs[j] = ds_read_b128_off<DLOFF - LOFF>(lo_ + (qb * 32 + 8 * j) * 4);
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        lgkm_wait<3 - j>(drs[j]);
        const u32x4 dr = drs[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * j + e;
          const uint32_t w = pk[qb][i >> 3][(i & 7) >> 1];
          const float p = as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
          sacc[qb][i] = p * (sacc[qb][i] - as_float(dr[e]));
        }
      });
    }
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      yb[qb][0] = pack8(sacc[qb], 0);
      yb[qb][1] = pack8(sacc[qb], 8);
    }
  };

  // Tile tt's MFMA phase runs for ws <= tt <= ntq: at tt = ws Y is still zero
  // (the X buffer it multiplies holds finite data), and at tt = ntq only its
  // product with the previous tile is used.  The phase of tile tt also issues
  // tile tt + 2's loads, one piece every EVERY MFMAs; a wave without that
  // phase issues them all at once.  Tiles past the last one load zeros (or
  // clamped rows) that nothing reads.  The phase runs at a raised wave
  // priority: the other wave of the SIMD is in its vector phase meanwhile
  // (for waves 4..7, the exp2-heavy one of waves 0..3), and the matrix core's
  // next instruction then issues first.
  auto mfma_tile = [&](int tt) __attribute__((always_inline)) {
    constexpr int EVERY = NOP / NPC;
    if (tt >= ws && tt <= ntq) {
      __builtin_amdgcn_s_setprio(1);
      mfma_phase((uint32_t)(((tt + 3) & 3) * TILE), (uint32_t)((tt & 3) * TILE),
                 [&](auto mc) __attribute__((always_inline)) {
                   constexpr int m = decltype(mc)::value;
                   if constexpr (m % EVERY == EVERY / 2 && m / EVERY < NPC) load_piece(tt + 2, m / EVERY);
                 });
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int k = 0; k < NPC; ++k) load_piece(tt + 2, k);
    }
  };
  auto vector_tile = [&](int tt) __attribute__((always_inline)) {
    if (tt >= ws && tt < ntq) {
      if (lead) vector_p(tt);
      else vector_ds(tt);
    }
  };
  // Grouped-query attention: the block's keys serve `group` query heads, walked
  // one after the other into the same accumulators (dk, dv sum over them).
  // The last barrier of a head's walk comes after every wave's last LDS read
  // of it, so the next head's first loads may reuse any buffer.
  for (int gh = 0; gh < group && (!DIAG || qs < ntq); ++gh) {
    const int bh = bhk * group + gh;
    qp = qg + (size_t)bh * Sq * D;
    dp = dog + (size_t)bh * Sq * D;
    lp = lse2g + (size_t)bh * Sq;
    Dp = Dg + (size_t)bh * Sq;
    load_tile(qs);
    if (qs + 1 < ntq) load_tile(qs + 1);
    // Finite data in both X buffers of the Y = 0 product of the first tile.
    dma.load(qbuf((qs + 3) & 3), qp, qs * BQ, Sq);
    dma.load(dbuf((qs + 3) & 3), dp, qs * BQ, Sq);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) yb[qb][0] = yb[qb][1] = u32x4{0, 0, 0, 0};
    // Iteration u: MFMA phase of tile u, vector phase of tile u.  Waves 4..7
    // run one phase behind, so their vector phase of tile u follows the
    // barrier after waves 0..3 wrote P(u).  The MFMA phase loads tile u + 2
    // into buffers whose last readers (tiles u - 2 and u - 1's products)
    // finished two phases back for either wave group; the iteration ends
    // waiting for that load.
    wait_vmem();
    phase_barrier();
    if (!lead) phase_barrier();
    for (int u = qs; u <= ntq; ++u) {
      mfma_tile(u);
      phase_barrier();
      vector_tile(u);
      wait_vmem();
      phase_barrier();
    }
    if (lead) phase_barrier();
  }

  if (kk < Sk) {
    float* row = (lead ? dvg : dkg) + ((size_t)bhk * Sk + kk) * D;
    const float f = lead ? 1.f : scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float* dst = row + db * 32 + 8 * j + 4 * g;
        f32x4 val = {acc[db][4 * j] * f, acc[db][4 * j + 1] * f, acc[db][4 * j + 2] * f, acc[db][4 * j + 3] * f};
        val += *reinterpret_cast<const f32x4*>(dst);
        *reinterpret_cast<f32x4*>(dst) = val;
      }
  }
}

template <int D>
hipError_t launch_dq_d(const BwdStepArgs& a, hipStream_t stream) {
  constexpr int BR = kDqWaves * kDqRowsPerWave;
  const int nq = (a.Sq + BR - 1) / BR;
  if (a.group < 1 || a.BH % a.group || a.qoff < 0 || (long long)a.Sq + a.Sk + a.qoff + 1024 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long total = (long long)nq * a.BH;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  if (a.diag)
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)total), dim3(64 * kDqWaves), 0, stream, a.q, a.k,
                       a.v, a.dO, a.lse2, a.D, a.dq, a.Sq, a.Sk, nq, (int)total, sl2, a.scale, a.group, a.qoff);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)total), dim3(64 * kDqWaves), 0, stream, a.q, a.k,
                       a.v, a.dO, a.lse2, a.D, a.dq, a.Sq, a.Sk, nq, (int)total, sl2, a.scale, a.group, a.qoff);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_d(const BwdStepArgs& a, hipStream_t stream) {
  constexpr int BK = (kKvfWaves / 2) * kKvfKeysPerWave;
  const int nk = (a.Sk + BK - 1) / BK;
  if (a.group < 1 || a.BH % a.group || a.qoff < 0 || (long long)a.Sq + a.Sk + a.qoff + 1024 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long total = (long long)nk * (a.BH / a.group);  // blocks per key/value head
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid((unsigned)total), block(64 * kKvfWaves);
  if (a.diag)
    hipLaunchKernelGGL((bwd_kvf_kernel<D, true>), grid, block, 0, stream, a.q, a.k, a.v, a.dO, a.lse2, a.D, a.dk,
                       a.dv, a.Sq, a.Sk, nk, (int)total, sl2, a.scale, a.group, a.qoff);
  else
    hipLaunchKernelGGL((bwd_kvf_kernel<D, false>), grid, block, 0, stream, a.q, a.k, a.v, a.dO, a.lse2, a.D, a.dk,
                       a.dv, a.Sq, a.Sk, nk, (int)total, sl2, a.scale, a.group, a.qoff);
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

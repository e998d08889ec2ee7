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
//  * key kernel -- a block owns 128 keys of the chunk, one wave per SIMD and
//    32 keys per wave, each wave holding its keys' K and V rows and the dk,
//    dv accumulators (in AGPRs), and streams 64-query tiles of Q and dO
//    (row-major; Q^T and dO^T through the transposing read).  Here S = Q K^T
//    has a lane per key, so P and dS feed dv^T += dO^T P and dk^T += Q^T dS
//    directly; lse2 and -D of the tile's queries are staged in LDS.
// The price of avoiding atomics is recomputing S and dP in both launches:
// 14 d flop per (query, key) pair executed for the 10 d of the gradient.
#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kPosInf = __builtin_inff();

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
  float lse2 = kPosInf, nDq = 0.f;
  if (qq < Sq) {
    lse2 = lse2g[(size_t)bh * Sq + qq];  // +inf for a row that saw no key: P = 0
    nDq = Dg[(size_t)bh * Sq + qq];      // the row pre-pass stores -D
  }
  // At d = 64 the dP^T chain starts at the lane's -D, so it yields dP^T - D
  // and the vector phase saves a subtraction per element (the vector unit
  // bounds that kernel); at d = 128 the 16 extra registers are not there.
  constexpr bool kFoldD = D == 64;
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
          if constexpr (s == 0 && kFoldD) {
            f32x16 c;
#pragma unroll
            for (int i = 0; i < 16; ++i) c[i] = nDq;
            pacc[kb] = mfma32(rq[b], df[0], c);
          } else if constexpr (s == 0) {
            pacc[kb] = mfma32(rq[b], df[0], f32x16{});
          } else {
            pacc[kb] = mfma32(rq[b], df[s], pacc[kb]);
          }
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
        sacc[kb][i] = kFoldD ? p * pacc[kb][i] : p * (pacc[kb][i] + nDq);
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
// dk/dv kernel: each wave holds 32 keys and all of their work (one wave per
// SIMD at d = 128, two at d = 64).
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;  // waves per block, 32 keys each
// MFMAs whose LDS operands are read ahead: 3 at d = 128 (a step's stream
// then covers the reads' latency; 2 left it exposed), 2 at d = 64.
template <int D>
constexpr int kKvLookahead = D == 128 ? 3 : 2;

// The bf16 MFMA D = A B + C as inline assembly with the register classes
// fixed: score accumulators in VGPRs (the vector unit reads them) with the
// key or value fragment in AGPRs, product accumulators in AGPRs.  The
// compiler, left to choose, puts every accumulator of a function that uses
// AGPRs in AGPRs and copies each score out.  Inline assembly carries no
// hazard tracking, so every use keeps its distance from the instructions
// that feed it: an accumulator recurs every second MFMA or later, a score is
// read by the vector unit in the next step (two or more MFMAs after it is
// written) or, by the mask pass, after 20 wait states, and the packed P and
// dS are read by the products one step after they are written.  A result that does not accumulate in place is early-clobber: the
// MFMA reads its sources over several passes while it writes, so its
// destination may overlap none of them.
__device__ __forceinline__ void mfma_score_first(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_score(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_score_c(f32x16& d, const u32x4& a, const u32x4& b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void mfma_product(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// s_waitcnt lgkmcnt(N) in the key kernel.  The MFMAs and the
// operand reads are volatile inline assembly, which the compiler keeps in
// order, so the wait names no operand registers (naming them would make them
// look freshly written to the hazard check, which then pads every MFMA).  It
// names the registers that ordinary code reads after it, which must not move
// above it: lse batch J (J >= 0) and, with ND, the -D rows.
template <int N, int J, bool ND>
__device__ __forceinline__ void kv_wait(u32x4 (&lr)[4], u32x4 (&nd)[4]) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  if constexpr (J >= 0 && ND)
    asm volatile("s_waitcnt lgkmcnt(%5)"
                 : "+v"(lr[J]), "+v"(nd[0]), "+v"(nd[1]), "+v"(nd[2]), "+v"(nd[3])
                 : "i"(N));
  else if constexpr (ND)
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(nd[0]), "+v"(nd[1]), "+v"(nd[2]), "+v"(nd[3]) : "i"(N));
  else if constexpr (J >= 0)
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(lr[J]) : "i"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
}

// LDS read schedule of one step of the key kernel (NKS = d/16).
// MFMA m of the step's 4 NKS: even m is score MFMA m/2 (S k-steps, then dP
// k-steps), reading one 16-byte operand; odd m is product (m-1)/2, reading
// two 8-byte transposed halves.  Operands are read LA MFMAs ahead.  Before
// the first operand reads the step reads the unit's -D rows (4 reads) and
// the lse batches that are due early; lse batch j (one read, rows of
// elements 4j .. 4j+3 of the previous unit) is issued in run(lse_run(j))
// after that run's operand reads.  Waits come in odd-even pairs: run(m),
// m even, waits for the operands of MFMAs m and m + 1.
struct KvReads {
  int nks, la, slot;  // slot: MFMA slots per element (NOP / 16)
  constexpr int nop() const { return 4 * nks; }
  constexpr int ring(int m) const { return m < nop() ? (m % 2 == 0 ? 1 : 2) : 0; }
  constexpr int lse_run(int j) const { return 4 * j * slot - la - 2; }
  constexpr int lse_at(int r) const {
    int n = 0;
    for (int j = 0; j < 4; ++j) n += lse_run(j) == r ? 1 : 0;
    return n;
  }
  constexpr int pre_lse() const {
    int n = 0;
    for (int j = 0; j < 4; ++j) n += lse_run(j) < 0 ? 1 : 0;
    return n;
  }
  // Reads issued up to the end of run(r)'s issues (r = -1: the step's
  // opening reads).
  constexpr int after_run(int r) const {
    int n = 4 + pre_lse();
    for (int m = 0; m < la; ++m) n += ring(m);
    for (int k = 0; k <= r; ++k) n += ring(k + la) + lse_at(k);
    return n;
  }
  // Position (count of reads up to and including it) of MFMA m's last
  // operand read.
  constexpr int operand_pos(int m) const {
    if (m < la) {
      int n = 4 + pre_lse();
      for (int k = 0; k <= m; ++k) n += ring(k);
      return n;
    }
    return after_run(m - la - 1) + ring(m);
  }
  constexpr int lse_pos(int j) const {
    if (lse_run(j) < 0) {
      int n = 4;
      for (int i = 0; i <= j; ++i) n += lse_run(i) < 0 ? 1 : 0;
      return n;
    }
    return after_run(lse_run(j));
  }
  constexpr int covered(int m) const { return operand_pos(m + 1 < nop() ? m + 1 : m); }
  // lgkmcnt of run(m)'s wait (m even): the reads issued after those it covers.
  constexpr int wait_count(int m) const { return after_run(m) - covered(m); }
  // The first wait that covers lse batch j.
  constexpr int first_wait(int j) const {
    for (int m = 0; m < nop(); m += 2)
      if (covered(m) >= lse_pos(j)) return m;
    return nop();
  }
  constexpr int tied(int m) const {
    int t = -1;
    for (int j = 0; j < 4; ++j)
      if (first_wait(j) == m) t = j;
    return t;
  }
  // Every lse batch is valid by slot 4j, its first use, and no two share a
  // wait; every count fits lgkmcnt.
  constexpr bool valid() const {
    for (int j = 0; j < 4; ++j) {
      if (first_wait(j) > 4 * j * slot) return false;
      for (int i = 0; i < j; ++i)
        if (first_wait(i) == first_wait(j)) return false;
    }
    for (int m = 0; m < nop(); m += 2)
      if (wait_count(m) < 0 || wait_count(m) > 15) return false;
    return true;
  }
};
static_assert(KvReads{8, kKvLookahead<128>, 2}.valid() && KvReads{4, kKvLookahead<64>, 1}.valid(),
              "key kernel read schedule");

// dv^T += dO^T P and dk^T += scale Q^T dS for one ring step in one launch.
// A block holds 128 keys, 32 per wave, 4 waves; at d = 128 a block takes a
// CU (one wave per SIMD: a wave's state needs 428 registers), at d = 64 two
// blocks share one (246 registers, 66 KB of LDS each), so that one wave's
// vector work runs beside the other's MFMAs.  A wave keeps
// its keys' K and V rows (the B operands of S = Q K^T and dP = dO V^T) and
// the dk^T and dv^T accumulators in AGPRs.  It walks the chunk's queries in
// units of 32 (half a 64-query LDS tile).  Step u, one unit's worth of
// matrix work, is a single stream of 4 d/16 MFMAs that alternates the unit's
// scores with the products of unit u-2:
//   S(u) = Q(u) K^T (d/16 k-steps), then dP(u) - D = dO(u) V^T - D (d/16
//   k-steps, the accumulator starting at the rows' -D), against
//   dv^T += dO^T(u-2) P(u-2) and dk^T += Q^T(u-2) dS(u-2) (d/8 MFMAs),
// and in the MFMA slots the vector unit turns unit u-1's scores into
// P = exp2(S scale log2(e) - lse2) and dS = P (dP - D), packed to bf16 for
// the products of step u+1.  S and dP are computed once per (query, key)
// pair, and dS uses the fp32 P.  Masked entries (the diagonal band, rows
// past the chunk, the units before and after the walk) have S set to -inf
// and dP - D to 0 between steps, so P and dS come out 0.  Q and dO tiles
// stream through four LDS buffers each, two tiles ahead, with the rows'
// lse2 and -D beside them; buffer slots are counted from the walk's first
// tile, and the tile loop is unrolled four times so that every LDS offset is
// an immediate.
template <int D, bool DIAG>
__global__ __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 1))) void bwd_kv_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
    const uint16_t* __restrict__ dog, const float* __restrict__ lse2g, const float* __restrict__ Dg,
    float* __restrict__ dkg, float* __restrict__ dvg, int Sq, int Sk, int n_ktiles, int total_tiles,
    float scale_log2, float scale, int group, int qoff) {
  constexpr int NW = kKvWaves, BK = NW * 32, BQ = kTileTokens, LA = kKvLookahead<D>;
  constexpr int NKS = D / 16, NDB = D / 32, TILE = BQ * D * 2;
  constexpr int NSC = 2 * NKS, NPR = 4 * NDB, NOP = NSC + NPR;  // MFMAs per step
  // LDS: Q tiles in buffers 0..3, dO tiles in buffers 0..3 at DOFF, then the
  // rows' lse2 and D (64 floats per tile each).
  constexpr int DOFF = 4 * TILE, LOFF = 8 * TILE, DLOFF = LOFF + 4 * BQ * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DLOFF + 4 * BQ * 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  int bhk, kt;
  if constexpr (DIAG) {
    longest_first(blockIdx.x, total_tiles / n_ktiles, bhk, kt);
  } else {
    const int t = xcd_remap(blockIdx.x, total_tiles);
    bhk = t / n_ktiles;
    kt = t - bhk * n_ktiles;
  }
  const int kb0 = kt * BK;
  const int kw0 = kb0 + wave * 32;
  const int kk = kw0 + l32;
  const uint16_t* __restrict__ qp = qg;
  const uint16_t* __restrict__ dp = dog;
  const float* __restrict__ lp = lse2g;
  const float* __restrict__ Dp = Dg;

  // Query tiles qs .. ntq-1 (causal: query q sees keys <= q + qoff); a block
  // whose keys no query sees skips the walk and adds zero.
  const int ntq = (Sq + BQ - 1) / BQ;
  const int qs = DIAG ? min(max(0, kb0 - qoff) / BQ, ntq) : 0;

  TileBufDma<D, NW, BQ> dma;
  dma.init(wave, lane);
  constexpr int NPW = decltype(dma)::kPerWave;
  // Tile j's lse2 and D rows (clamped to Sq - 1) into row slot b: one 4-byte
  // load per lane, by waves 0 and 1.
  auto load_rows = [&](int j, int b) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int row = min(j * BQ + lane, Sq - 1);
    if (wave == 0) __builtin_amdgcn_global_load_lds(lp + row, (lds_void*)(smem + LOFF + b * BQ * 4), 4, 0, 0);
    if (wave == 1) __builtin_amdgcn_global_load_lds(Dp + row, (lds_void*)(smem + DLOFF + b * BQ * 4), 4, 0, 0);
#else
    (void)j, (void)b, (void)lp, (void)Dp;
#endif
  };
  auto load_tile = [&](int j, int b) __attribute__((always_inline)) {
    load_rows(j, b);
    dma.load(smem + b * TILE, qp, j * BQ, Sq);
    dma.load(smem + DOFF + b * TILE, dp, j * BQ, Sq);
  };

  u32x4 kf[NKS], vf[NKS];
  {
    const uint16_t* krow = kg + ((size_t)bhk * Sk + kk) * D;
    const uint16_t* vrow = vg + ((size_t)bhk * Sk + kk) * D;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const u32x4 kv = (kk < Sk) ? ld16(krow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
      const u32x4 vv = (kk < Sk) ? ld16(vrow + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
      // Moved into AGPRs once: their only readers are MFMA B operands.
      asm volatile("" : "=a"(kf[s]) : "0"(kv));
      asm volatile("" : "=a"(vf[s]) : "0"(vv));
    }
  }
  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dv[db][i] = dk[db][i] = 0.f;
  // Scores of the unit being computed and of the one being turned into P
  // and dS: sd[u & 1][0] = S(u), sd[u & 1][1] = dP(u) - D.  yb[u & 1][0][k] and
  // yb[u & 1][1][k] hold unit u's P and dS, bf16, for query rows 16k..16k+15
  // of the unit (the B operands of the products).
  f32x16 sd[2][2];
  u32x4 yb[2][2][2];

  // Operand addresses (buffer 0): row-major reads of Q or dO and transposing
  // reads of Q^T or dO^T; dO's at DOFF, beyond the 16-bit offset field.
  const uint32_t base = lds_addr(smem);
  uint32_t rq[NKS], rd[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    rq[s] = base + (uint32_t)tile_off<D>(l32, 2 * s + g);
    rd[s] = rq[s] + (uint32_t)DOFF;
  }
  uint32_t tq[NDB][2], td[NDB][2];
  {
    const int m = (lane & 15) >> 2, a4 = lane & 3, half16 = (lane >> 4) & 1;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + 16 * half16 + 4 * a4;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        tq[db][tt] = base + tile_off<D>(4 * g + m + 8 * tt, d >> 3) + ((d & 4) ? 8 : 0);
        td[db][tt] = tq[db][tt] + (uint32_t)DOFF;
      }
    }
  }
  const uint32_t laddr = base + LOFF + (uint32_t)(4 * g) * 4;  // rows 4g .. 4g+3 of a tile's lse2 slot

  // Sets the masked entries of unit (t, h)'s scores: S = -inf, dP - D = 0.
  // Units at or past the last tile are masked whole.
  auto mask_unit = [&](int t, int h, f32x16(&s)[2]) __attribute__((always_inline)) {
    const int q0 = t * BQ + 32 * h;
    const bool whole = t >= ntq;
    if (whole || q0 + 32 > Sq || (DIAG && q0 + qoff < kw0 + 31)) {
      // The step's last dP MFMA issued two MFMAs back; 20 wait states make
      // its result readable by the vector unit whatever the pass count (the
      // scores are named, so nothing that reads them moves above).
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s[0]), "+v"(s[1]));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = q0 + 8 * (i >> 2) + 4 * g + (i & 3);
        if (whole || qi >= Sq || (DIAG && kk > qi + qoff)) {
          s[0][i] = -kPosInf;
          s[1][i] = 0.f;
        }
      }
    }
  };

  // Step of unit u = 2t + H, tile t in buffer R: the MFMA stream of S(u),
  // dP(u) - D and unit u-2's products; unit u-1's P and dS in its slots.  With
  // H = 0 the step also loads tile t + 2 into buffer R + 2.
  auto step = [&](auto rc, auto hc, int t) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value, H = decltype(hc)::value;
    constexpr int XB = (R + 3) & 3;                   // buffer of tile t - 1
    constexpr int EB = H ? R : XB, EH = 1 - H;        // unit u-1: its tile's buffer, its half
    constexpr KvReads RS{NKS, LA, NOP / 16};
    f32x16(&sc)[2] = sd[H];                           // written here
    f32x16(&se)[2] = sd[1 - H];                       // unit u-1, read here
    u32x4(&yp)[2][2] = yb[H];                         // unit u-2, read by the products
    u32x4(&ye)[2][2] = yb[1 - H];                     // unit u-1, written here
    u32x4 nd[4], lr[4];  // unit u's -D rows (the dP accumulator's start), unit u-1's lse2 rows
    u32x4 ra[LA + 1];
    u32x2 lo[LA + 1], hi[LA + 1];
    auto issue_lse = [&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      lr[j] = ds_read_b128_off<EB * BQ * 4 + (32 * EH + 8 * j) * 4>(laddr);
    };
    // MFMA m: even m is score MFMA m/2 (S k-steps, then dP k-steps); odd m is
    // product (m-1)/2.
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      if constexpr (m < NOP && m % 2 == 0) {
        constexpr int si = m / 2, OFF = R * TILE + H * 32 * D * 2;
        if constexpr (si < NKS) ra[b] = ds_read_b128_off<OFF>(rq[si]);
        else ra[b] = ds_read_b128_off<OFF>(rd[si - NKS]);
      } else if constexpr (m < NOP) {
        constexpr int j = m / 2, k = j / (2 * NDB), db = (j % (2 * NDB)) / 2, dkp = j & 1;
        constexpr int OFF = XB * TILE + (32 * H + 16 * k) * D * 2;
        lo[b] = ds_read_tr16_off<OFF>(dkp ? tq[db][0] : td[db][0]);
        hi[b] = ds_read_tr16_off<OFF>(dkp ? tq[db][1] : td[db][1]);
      }
    };
    // Unit u-1's elements: A(e) scales and centres S, B(e) exponentiates,
    // C(e) forms dS = P (dP - D) and packs pairs; element e's stages fall in
    // slots a(e), a(e)+1, a(e)+2, the ones past the stream after it.  Each
    // stage's results are pinned where it stands (an empty asm that takes
    // them), or the compiler sinks the arithmetic to its first use.
    float x[16], p[16], ds[16];
    auto stage_a = [&](int e) __attribute__((always_inline)) {
      x[e] = fmaf(se[0][e], scale_log2, -as_float(lr[e >> 2][e & 3]));
      asm volatile("" : "+v"(x[e]));
    };
    auto stage_b = [&](int e) __attribute__((always_inline)) {
      p[e] = fast_exp2(x[e]);
      asm volatile("" : "+v"(p[e]));
    };
    auto stage_c = [&](int e) __attribute__((always_inline)) {
      ds[e] = p[e] * se[1][e];
      if (e & 1) {
        uint32_t pp = pack_bf16(p[e - 1], p[e]), dd = pack_bf16(ds[e - 1], ds[e]);
        asm volatile("" : "+v"(pp), "+v"(dd));
        ye[0][e >> 3][(e & 7) >> 1] = pp;
        ye[1][e >> 3][(e & 7) >> 1] = dd;
      }
    };
    constexpr int SLOT_STRIDE = NOP / 16;  // 2 at d = 128, 1 at d = 64
    auto valu = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m % SLOT_STRIDE == 0 && m / SLOT_STRIDE < 16) stage_a(m / SLOT_STRIDE);
      if constexpr (m >= 1 && (m - 1) % SLOT_STRIDE == 0 && (m - 1) / SLOT_STRIDE < 16) stage_b((m - 1) / SLOT_STRIDE);
      if constexpr (m >= 2 && (m - 2) % SLOT_STRIDE == 0 && (m - 2) / SLOT_STRIDE < 16) stage_c((m - 2) / SLOT_STRIDE);
      // Tile t + 2's loads, in the first step of the tile: rows first, then
      // this wave's Q and dO pieces.
      if constexpr (H == 0) {
        constexpr int LE = NOP / (2 * NPW + 1);
        if constexpr (m % LE == 0 && m / LE < 2 * NPW + 1) {
          constexpr int k = m / LE, B2 = (R + 2) & 3;
          if constexpr (k == 0) load_rows(t + 2, B2);
          else if constexpr (k <= NPW) dma.load_piece(k - 1, smem + B2 * TILE, qp, (t + 2) * BQ, Sq);
          else dma.load_piece(k - 1 - NPW, smem + DOFF + B2 * TILE, dp, (t + 2) * BQ, Sq);
        }
      }
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      issue(std::integral_constant<int, m + LA>{});
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        if constexpr (RS.lse_run(decltype(jc)::value) == m) issue_lse(jc);
      });
      if constexpr (m % 2 == 0) kv_wait<RS.wait_count(m), RS.tied(m), m == 0>(lr, nd);
      if constexpr (m % 2 == 0) {
        constexpr int si = m / 2;
        if constexpr (si == 0) {
          mfma_score_first(sc[0], ra[b], kf[0]);
        } else if constexpr (si < NKS) {
          mfma_score(sc[0], ra[b], kf[si]);
        } else if constexpr (si == NKS) {
          // dP - D: the accumulator starts at the rows' -D.
          const f32x16 c = {as_float(nd[0][0]), as_float(nd[0][1]), as_float(nd[0][2]), as_float(nd[0][3]),
                            as_float(nd[1][0]), as_float(nd[1][1]), as_float(nd[1][2]), as_float(nd[1][3]),
                            as_float(nd[2][0]), as_float(nd[2][1]), as_float(nd[2][2]), as_float(nd[2][3]),
                            as_float(nd[3][0]), as_float(nd[3][1]), as_float(nd[3][2]), as_float(nd[3][3])};
          mfma_score_c(sc[1], ra[b], vf[0], c);
        } else {
          mfma_score(sc[1], ra[b], vf[si - NKS]);
        }
      } else {
        constexpr int j = m / 2, k = j / (2 * NDB), db = (j % (2 * NDB)) / 2, dkp = j & 1;
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        if constexpr (dkp) mfma_product(dk[db], a, yp[1][k]);
        else mfma_product(dv[db], a, yp[0][k]);
      }
      valu(mc);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Opening reads: unit u's -D rows, the early lse batches, the first
    // operands.
    static_for<4>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      nd[j] = ds_read_b128_off<DLOFF - LOFF + R * BQ * 4 + (32 * H + 8 * j) * 4>(laddr);
    });
    static_for<4>([&](auto jc) __attribute__((always_inline)) {
      if constexpr (RS.lse_run(decltype(jc)::value) < 0) issue_lse(jc);
    });
    static_for<LA>(issue);
    static_for<NOP>(run);
    // Stages past the stream.
    static_for<3>([&](auto oc) __attribute__((always_inline)) {
      constexpr int m = NOP + decltype(oc)::value;
      if constexpr ((m - 1) % SLOT_STRIDE == 0 && (m - 1) / SLOT_STRIDE < 16) stage_b((m - 1) / SLOT_STRIDE);
      if constexpr ((m - 2) % SLOT_STRIDE == 0 && (m - 2) / SLOT_STRIDE < 16) stage_c((m - 2) / SLOT_STRIDE);
    });
    mask_unit(t, H, sc);
  };
  // Tile t in buffer R: its two steps, then (once this wave's loads of the
  // tile before have landed) the barrier after which buffer R + 2 may be
  // reloaded.  Loads are issued rows first, so waiting for all but the last
  // 2 NPW covers every earlier tile's.
  auto tile = [&](auto rc, int t) __attribute__((always_inline)) {
    step(rc, std::integral_constant<int, 0>{}, t);
    step(rc, std::integral_constant<int, 1>{}, t);
    wait_vmem_but<2 * NPW>();
    phase_barrier();
  };

  // Grouped-query attention: the block's keys serve `group` query heads,
  // walked one after the other into the same accumulators.
  for (int gh = 0; gh < group && qs < ntq; ++gh) {
    const int bh = bhk * group + gh;
    qp = qg + (size_t)bh * Sq * D;
    dp = dog + (size_t)bh * Sq * D;
    lp = lse2g + (size_t)bh * Sq;
    Dp = Dg + (size_t)bh * Sq;
    // Tiles qs and qs + 1 into buffers 0 and 1; buffer 3, which the first
    // tile's products read (as tile qs - 1) and the first unit's rows come
    // from, gets tile qs as well, so that everything read there is finite.
    load_tile(qs, 0);
    load_tile(qs + 1, 1);
    load_tile(qs, 3);
    // Unit 2 qs - 1 (before the walk) is masked whole; unit 2 qs - 2's P and
    // dS are zero.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sd[1][0][i] = -kPosInf;
      sd[1][1][i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int k = 0; k < 2; ++k) yb[0][h][k] = yb[1][h][k] = u32x4{0, 0, 0, 0};
    wait_vmem();
    phase_barrier();
    // Tiles qs .. ntq; the last (past the chunk, masked whole) drains the
    // pipeline.
    for (int t = qs;;) {
      tile(std::integral_constant<int, 0>{}, t);
      if (++t > ntq) break;
      tile(std::integral_constant<int, 1>{}, t);
      if (++t > ntq) break;
      tile(std::integral_constant<int, 2>{}, t);
      if (++t > ntq) break;
      tile(std::integral_constant<int, 3>{}, t);
      if (++t > ntq) break;
    }
    wait_vmem();
    phase_barrier();
  }

  // The product accumulators are read from AGPRs well after their last MFMA;
  // the padding covers the longest MFMA-to-read distance in any case.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if (kk < Sk) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float* row = (r ? dkg : dvg) + ((size_t)bhk * Sk + kk) * D;
      const float f = r ? scale : 1.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& acc = r ? dk[db] : dv[db];
          float* dst = row + db * 32 + 8 * j + 4 * g;
          f32x4 val = {acc[4 * j] * f, acc[4 * j + 1] * f, acc[4 * j + 2] * f, acc[4 * j + 3] * f};
          val += *reinterpret_cast<const f32x4*>(dst);
          *reinterpret_cast<f32x4*>(dst) = val;
        }
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
  constexpr int BK = kKvWaves * 32;
  const int nk = (a.Sk + BK - 1) / BK;
  if (a.group < 1 || a.BH % a.group || a.qoff < 0 || (long long)a.Sq + a.Sk + a.qoff + 1024 > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long total = (long long)nk * (a.BH / a.group);  // blocks per key/value head
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  if (total == 0) return hipSuccess;
  const float sl2 = a.scale * kLog2e;
  const dim3 grid((unsigned)total), block(64 * kKvWaves);
  if (a.diag)
    hipLaunchKernelGGL((bwd_kv_kernel<D, true>), grid, block, 0, stream, a.q, a.k, a.v, a.dO, a.lse2, a.D, a.dk,
                       a.dv, a.Sq, a.Sk, nk, (int)total, sl2, a.scale, a.group, a.qoff);
  else
    hipLaunchKernelGGL((bwd_kv_kernel<D, false>), grid, block, 0, stream, a.q, a.k, a.v, a.dO, a.lse2, a.D, a.dk,
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

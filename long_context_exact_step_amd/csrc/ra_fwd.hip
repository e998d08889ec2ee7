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
//    SIMD and interleave on its matrix core.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: K (32 keys x 16 d) is the A operand read from
//    LDS; Q^T is the B operand and stays in registers for the whole kernel.
//    In the accumulator a lane holds one query and 16 of its keys, so the
//    softmax statistics are per-lane scalars (one v_permlane32_swap per row
//    maximum), and the probabilities, packed to bf16, are already the B
//    operand of O^T += V^T P^T.  V^T's A operand comes straight from the
//    row-major V tile through ds_read_b64_tr_b16 (no transpose pass).
//  * Per 64-key tile each wave issues one stream of 32 MFMAs (P V of the
//    previous tile, S^T of the next) and runs the softmax of the current
//    tile in the vector-ALU slots between them, one score per slot, each
//    score spread over three slots so no instruction waits on its own slot.
//  * LDS operands are read three MFMAs ahead with counted waits, and the
//    stream runs on across tiles.
//  * K and V tiles (64 keys) go global -> LDS with buffer loads into LDS
//    (no registers; a per-tile buffer resource, so the per-lane offsets are
//    constants and keys past the chunk read as zeros) into four buffers
//    each, two tiles ahead of use, one 1 KB piece per MFMA slot; one block
//    barrier per tile.
//  * exp2 with scale*log2(e) folded into one FMA, against the running
//    maximum; the tile maximum is only taken (and O rescaled) on the exact
//    path: a row's first tile, masked tiles, and tiles whose row sums exceed
//    2^8.
//  * Blocks are mapped so each XCD works on one contiguous range of
//    (head, query tile) pairs (K/V lines shared in that XCD's L2); on the
//    diagonal chunk the longest query tiles of every head go first.
#include <type_traits>

#include <atomic>

#include "ra_device.h"
#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyBound = 256.0f;  // largest row sum of one tile computed without a new maximum


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

// First softmax element issued in MFMA slot m when NEL elements are spread in
// order over slots SH .. NOP-1 (element e goes to slot SH + e*(NOP-SH)/NEL).
__host__ __device__ constexpr int first_element(int m, int SH, int NOP, int NEL) {
  return m <= SH ? 0 : (m >= NOP ? NEL : ((m - SH) * NEL + (NOP - SH) - 1) / (NOP - SH));
}

constexpr int kFwdWaves = 8;      // waves per block, two per SIMD
constexpr int kFwdRowsPerWave = 32;
constexpr int kFwdLookahead = 3;  // MFMAs whose LDS operands are read ahead
constexpr int kFwdBuffers = 4;    // LDS buffers per operand (K, V)

// One ring step.  A block holds 256 query rows, 32 per wave, and walks the
// chunk's keys in 64-key tiles with a three-stage software pipeline per wave.
// Iteration t issues, one MFMA per slot,
//   O^T += V^T P^T(t-1)      (16 MFMAs at d = 128; V^T read transposed)
//   S^T(t+1) = K(t+1) Q^T    (16 MFMAs)
// and, in the vector-ALU slots between those MFMAs, the online softmax of
// S^T(t) (computed one iteration earlier): about one score per MFMA slot, so
// the exponentials never wait on a matrix result and never stall the matrix
// core.  The exponentials use the running maximum as reference without
// computing the tile maximum first; a wave-uniform test on the tile's row
// sums sends the rare tile whose scores exceed the reference by more than
// 2^8 (and every row's first tile) to an exact path that takes the maximum,
// recomputes P and rescales O.
// K and V tiles arrive by direct-to-LDS loads into four buffers each, two
// tiles ahead of use, so the operands of an iteration's first MFMAs are read
// before the barrier that ends the previous one and the operand stream runs
// on across it.  One workgroup barrier per tile.
//
// WALK: the keys are tbl.n resident chunks walked in one pass (Sk = n * C),
// so the online-softmax state runs on from chunk to chunk in registers and
// no partial crosses HBM.  Key tile T is tile T % (C/64) of chunk
// T / (C/64); the chunk bases sit one per lane and are read out with
// readlane as the tile loads cross into a new chunk.
template <int D, bool DIAG, bool MERGE, bool WALK>
__device__ __forceinline__ void fwd_body(const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
                                         const uint16_t* __restrict__ vg, float* __restrict__ og,
                                         float* __restrict__ lseg, int Sq, int Sk, int n_qtiles, int total_tiles,
                                         float scale_log2, int group, int qoff, const ChunkTable& tbl,
                                         const StageCopy& stage, int unit, bool stage_now) {
  constexpr int NW = kFwdWaves, NQW = kFwdRowsPerWave, BR = NW * NQW, BC = kTileTokens;
  constexpr int NKS = D / 16, NDB = D / 32, NKB = BC / 32, TILE = BC * D * 2, LA = kFwdLookahead;
  constexpr int NB = kFwdBuffers;
  constexpr int NPV = 4 * NDB, NS = NKS * NKB, NOP = NPV + NS, NEL = 16 * NKB;
  // The ring of LA + 1 operand registers lines up with every stream.
  static_assert(NOP % (LA + 1) == 0 && NS % (LA + 1) == 0, "operand ring must divide the streams");
  static_assert(LA <= NPV, "the next iteration's first operands are PV reads");
  // Softmax element e of tile t (keys 16j .. 16j+15 for e in 8j .. 8j+7)
  // overwrites P^T(t-1) of the same keys, which the MFMAs of slots
  // NDB*j .. NDB*j+NDB-1 read; starting the elements at slot SH keeps every
  // write after the slot of the last MFMA that reads its register.
  constexpr int SH = 3;
  // LDS: V tiles in buffers 0 .. NB-1, K tiles in buffers NB .. 2NB-1 (the
  // K half starts at VOFF, folded into the K addresses so that every read
  // offset fits the 16-bit immediate); tile j uses buffer j % NB.
  constexpr int VOFF = NB * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NB * TILE];
  auto kbuf = [&](int b) __attribute__((always_inline)) { return smem + VOFF + b * TILE; };
  auto vbuf = [&](int b) __attribute__((always_inline)) { return smem + b * TILE; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const int l32 = lane & 31, g = lane >> 5;
  // The block's unit: the (head row, query tile) pair, numbered as the
  // launch maps them (see fwd_step_kernel).
  int bh, qt;
  if constexpr (DIAG) {
    // Causal: the last query tiles see the most keys; they go first.
    longest_first(unit, total_tiles / n_qtiles, bh, qt);
    qt = n_qtiles - 1 - qt;
  } else {
    bh = unit / n_qtiles;
    qt = unit - bh * n_qtiles;
  }
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * NQW;
  const int qq = qw0 + l32;
  const uint16_t* __restrict__ qp = qg + (size_t)bh * Sq * D;
  // Grouped-query attention: query head row bh reads key/value head bh / group.
  const uint16_t* __restrict__ kp = WALK ? kg : kg + (size_t)(bh / group) * Sk * D;
  const uint16_t* __restrict__ vp = WALK ? vg : vg + (size_t)(bh / group) * Sk * D;
  // Walk: chunk bases (lane c holds chunk c's), the head's offset in a
  // chunk, and the source (base, first token, tokens) of key tile T.
  [[maybe_unused]] uint64_t kchunk = 0, vchunk = 0;
  [[maybe_unused]] int tpc = 1;
  [[maybe_unused]] size_t hoff = 0;
  if constexpr (WALK) {
    tpc = tbl.C / kTileTokens;
    hoff = (size_t)(bh / group) * tbl.C * D;
#pragma unroll
    for (int i = 0; i < kMaxWalkChunks; ++i)
      if (lane == i) {
        kchunk = (uint64_t)(uintptr_t)tbl.k[i];
        vchunk = (uint64_t)(uintptr_t)tbl.v[i];
      }
  }
  auto chunk_base = [&](uint64_t table, int c) __attribute__((always_inline)) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)table, c);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(table >> 32), c);
    return reinterpret_cast<const uint16_t*>(((uint64_t)hi << 32) | lo) + hoff;
  };
  // A walk position: tile l of chunk c, its chunk's base, and the tokens
  // there (0 past the last chunk: such tiles read as zeros).
  struct WalkPos {
    int c, l, n;
    const uint16_t* base;
  };
  auto walk_pos = [&](uint64_t table, int T) __attribute__((always_inline)) {
    const int c = T / tpc;
    return WalkPos{c, T - c * tpc, c < tbl.n ? tbl.C : 0, chunk_base(table, c < tbl.n ? c : 0)};
  };
  auto walk_next = [&](uint64_t table, WalkPos& p) __attribute__((always_inline)) {
    if (++p.l == tpc) {
      p.l = 0;
      ++p.c;
      p.n = p.c < tbl.n ? tbl.C : 0;
      p.base = chunk_base(table, p.c < tbl.n ? p.c : 0);
    }
  };

  // Causal: query row q sees keys k <= q + qoff.
  int kend = Sk;
  if (DIAG) kend = min(kend, q0 + BR + qoff);
  const int ntiles = (kend + BC - 1) / BC;
  const int wtiles = DIAG ? min(ntiles, max(0, (min(qw0 + NQW, Sq) - 1 + qoff) / BC + 1)) : ntiles;
  // Keys at or past `lim` are masked for this lane's query.
  const int lim = DIAG ? min(Sk, qq + 1 + qoff) : Sk;

  // Iteration t reads K(t+1) and V(t-1); step t loads V(t+1) and K(t+3),
  // one 1 KB piece per MFMA slot in DMA_SLOT, V pieces first.  A step ends
  // waiting for all but its K pieces, which have one more step to land.
  // (Loading V a step earlier as well measured the same time and 16 % more
  // HBM traffic: the blocks of a head drift further apart in their L2 use.)
  using Dma = TileBufDma<D, NW, BC>;
  constexpr int NPIECE = Dma::kPerWave;  // pieces per tile per wave
  Dma dma;
  dma.init(wave, lane);
  [[maybe_unused]] WalkPos vpos{}, kpos{};  // walk: tiles tt + 1 (V) and tt + 3 (K) of step tt
  if constexpr (WALK) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < ntiles) {
        const WalkPos p = walk_pos(kchunk, j);
        dma.load(kbuf(j), p.base, p.l * BC, p.n);
      }
    const WalkPos v0 = walk_pos(vchunk, 0);
    dma.load(vbuf(0), v0.base, 0, v0.n);
    dma.load(vbuf(NB - 1), v0.base, 0, v0.n);  // finite data for the P = 0 product of iteration 0
    vpos = walk_pos(vchunk, 1);
    kpos = walk_pos(kchunk, 3);
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < ntiles) dma.load(kbuf(j), kp, j * BC, Sk);
    dma.load(vbuf(0), vp, 0, Sk);
    dma.load(vbuf(NB - 1), vp, 0, Sk);  // finite data for the P = 0 product of iteration 0
  }

  u32x4 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = (qq < Sq) ? ld16(qp + (size_t)qq * D + s * 16 + g * 8) : u32x4{0, 0, 0, 0};
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  // Running row sum, compensated: lrow - lcomp is the sum.  Over a long chunk
  // each tile adds far less than the sum holds, and plain fp32 accumulation
  // would drift by up to (tiles x 2^-25) of it.
  float mrow = kNegInf, lrow = 0.f, lcomp = 0.f;
  float mref = 0.f;  // exponent reference: mrow, or 0 while the row has seen no key
  // S^T of tiles t (being softmaxed) and t + 1 (being computed): sacc[t % 2].
  f32x16 sacc[2][NKB];
  // P^T in bf16: P^T(t-1) while iteration t multiplies it, overwritten in
  // place by P^T(t) as the softmax of tile t produces it.
  u32x4 pb[NKB][2];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) pb[kb][0] = pb[kb][1] = u32x4{0, 0, 0, 0};

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

  // Offset of element (kb, i) of a score accumulator from the tile's first key,
  // less 4g (the lane half's own offset).
  auto key_off = [](int kb, int i) { return 32 * kb + 8 * (i >> 2) + (i & 3); };

  // Operand registers of the MFMAs whose LDS reads are in flight; op m of any
  // stream uses ring slot m % (LA + 1).  They carry over from one stream to
  // the next.
  u32x2 lo[LA + 1], hi[LA + 1];
  u32x4 kq[LA + 1];
  // Reads of PV op m (V^T block db for tokens 32*(gi/2) + 16*(gi%2) .. +15)
  // from V buffer VB, or of S op m from K buffer KB.
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

  // One MFMA stream: PV from V buffer VB with P^T `pb` (if PV), then S^T from
  // K buffer KB into `sn`, with `valu(m)` in the slot of MFMA m.  The reads of
  // the first LA ops were issued before the stream (by the previous stream);
  // the stream's last slots issue those of the next stream, a PV from V
  // buffer VBN.  Each MFMA waits only for its own operands; sched_barrier
  // keeps every slot's instructions in their slot.
  auto mfma_stream = [&](auto pvc, auto kbc, auto vbc, auto vbnc, f32x16 (&sn)[NKB], auto&& valu)
                         __attribute__((always_inline)) {
    constexpr bool PV = decltype(pvc)::value;
    constexpr int N2 = PV ? NPV : 0, NO = N2 + NS;
    // Reads in flight after those of op m: ops m+1 .. m+LA, the ones past
    // the end being the next stream's PV ops (two reads each).
    auto reads_after = [](int m) {
      int n = 0;
      for (int k = m + 1; k <= m + LA; ++k) n += (k < N2 || k >= NO) ? 2 : 1;
      return n;
    };
    auto issue = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < N2) read_pv(mc, vbc);
      else if constexpr (m < NO) read_s(mc, std::integral_constant<int, m - N2>{}, kbc);
      else read_pv(std::integral_constant<int, m - NO>{}, vbnc);
    };
    auto run = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value, b = m % (LA + 1);
      constexpr int N = reads_after(m);
      issue(std::integral_constant<int, m + LA>{});
      if constexpr (m < N2) {
        constexpr int gi = m / NDB, db = m % NDB;
        lgkm_wait<N>(lo[b], hi[b]);
        const u32x4 a = {lo[b][0], lo[b][1], hi[b][0], hi[b][1]};
        oacc[db] = mfma32(a, pb[gi >> 1][gi & 1], oacc[db]);
      } else {
        constexpr int j = m - N2, s = j / NKB, kb = j % NKB;
        lgkm_wait<N>(kq[b]);
        if constexpr (s == 0) sn[kb] = mfma32(kq[b], qf[0], f32x16{});
        else sn[kb] = mfma32(kq[b], qf[s], sn[kb]);
      }
      valu(mc);
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<NO>(run);
  };

  // Exact path of the softmax of tile tt (rare): mask, tile maximum, P and
  // its row sums recomputed against the raised reference, O and l rescaled.
  auto softmax_exact = [&](int tt, f32x16 (&sc)[NKB]) __attribute__((always_inline)) {
    const int r = lim - tt * BC - 4 * g;
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (key_off(kb, i) >= r) sc[kb][i] = kNegInf;
        mx = fmaxf(mx, sc[kb][i]);
      }
    mx = pair_max(mx) * scale_log2;
    const float mnew = fmaxf(mrow, mx);
    const float mb = (mnew == kNegInf) ? 0.f : mnew;
    float l4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(sc[kb][i], scale_log2, -mb));
        sc[kb][i] = p;
        l4[i & 3] += p;
      }
      pb[kb][0] = pack8(sc[kb], 0);
      pb[kb][1] = pack8(sc[kb], 8);
    }
    const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(mrow - mnew);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    lrow = (lrow - lcomp) * alpha + ((l4[0] + l4[1]) + (l4[2] + l4[3]));
    lcomp = 0.f;
    mrow = mnew;
    mref = mb;
  };

  // Piece k of step tt's loads: V(tt+1) replaces V(tt-3) and K(tt+3)
  // replaces K(tt-1), both last read in iteration tt - 2 or earlier.  Loads
  // past the last tile read zeros and are never used.
  auto dma_piece = [&](int tt, auto ic, int k) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    if constexpr (WALK) {
      if (k < NPIECE) dma.load_piece(k, vbuf((I + 1) % NB), vpos.base, vpos.l * BC, vpos.n);
      else dma.load_piece(k - NPIECE, kbuf((I + 3) % NB), kpos.base, kpos.l * BC, kpos.n);
    } else {
      if (k < NPIECE) dma.load_piece(k, vbuf((I + 1) % NB), vp, (tt + 1) * BC, Sk);
      else dma.load_piece(k - NPIECE, kbuf((I + 3) % NB), kp, (tt + 3) * BC, Sk);
    }
  };
  // Iteration tt (tt % NB == I): PV(tt-1), S^T(tt+1) and the softmax of tile
  // tt.  The same code runs for tt = wtiles, where only PV(tt-1) matters: the
  // score tile and the softmax it computes there are never committed or
  // used.  Tiles that need a mask (keys past the chunk, or past the
  // diagonal) take the exact path, which applies it.
  auto iteration = [&](int tt, auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    f32x16(&sc)[NKB] = sacc[I % 2];
    const float mb = mref;
    float l4[4];
    // Each element runs as three stages in three consecutive slots (scale,
    // exp2, sum and pack), so no instruction waits on one issued in its own
    // slot.  xs / ps hold the elements between stages, by element index.
    float xs[NEL], ps[NEL];
    auto scale_stage = [&](int e) __attribute__((always_inline)) {
      xs[e] = fmaf(sc[e >> 4][e & 15], scale_log2, -mb);
    };
    auto exp_stage = [&](int e) __attribute__((always_inline)) { ps[e] = fast_exp2(xs[e]); };
    auto sum_stage = [&](int e) __attribute__((always_inline)) {
      const int kb = e >> 4, i = e & 15;
      if (e < 4) {
        l4[i & 3] = ps[e];  // elements 0..3 start the four partial sums
      } else {
        l4[i & 3] += ps[e];
        asm volatile("" : "+v"(l4[i & 3]));  // keeps the sum in this slot
      }
      if (i & 1) pb[kb][i >> 3][(i & 7) >> 1] = pack_bf16(ps[e - 1], ps[e]);
    };
    // Slots SH .. NOP-1 take the elements in order, spread evenly: slot m
    // starts elements first_element(m) .. first_element(m + 1) - 1.  The
    // step's tile loads go to evenly spaced slots.
    auto valu = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      constexpr int DMA_EVERY = NOP / (2 * NPIECE);
      if constexpr (m % DMA_EVERY == DMA_EVERY / 2) dma_piece(tt, ic, m / DMA_EVERY);
#pragma unroll
      for (int e = first_element(m - 2, SH, NOP, NEL); e < first_element(m - 1, SH, NOP, NEL); ++e) sum_stage(e);
#pragma unroll
      for (int e = first_element(m - 1, SH, NOP, NEL); e < first_element(m, SH, NOP, NEL); ++e) exp_stage(e);
#pragma unroll
      for (int e = first_element(m, SH, NOP, NEL); e < first_element(m + 1, SH, NOP, NEL); ++e) scale_stage(e);
    };
    mfma_stream(std::true_type{}, std::integral_constant<int, (I + 1) % NB>{},
                std::integral_constant<int, (I + NB - 1) % NB>{}, std::integral_constant<int, I>{},
                sacc[1 - I % 2], valu);
    // The stages still in flight after the last slot.
#pragma unroll
    for (int e = first_element(NOP - 2, SH, NOP, NEL); e < NEL; ++e) {
      if (e >= first_element(NOP - 1, SH, NOP, NEL)) exp_stage(e);
      sum_stage(e);
    }
    if (tt < wtiles) {
      const int k0 = tt * BC;
      const bool masked = (k0 + BC > Sk) || (DIAG && k0 + BC - 1 > qw0 + qoff);
      const float lt = (l4[0] + l4[1]) + (l4[2] + l4[3]);
      if (masked || __ballot(!(lt <= kLazyBound) || mrow == kNegInf) != 0) softmax_exact(tt, sc);
      else {
        const float y = lt - lcomp, sum = lrow + y;
        lcomp = (sum - lrow) - y;
        lrow = sum;
      }
    }
  };
  auto step = [&](int tt, auto ic) __attribute__((always_inline)) {
    if (tt <= wtiles) iteration(tt, ic);
    // A wave past its last tile still loads its share of the tiles.
    if (tt > wtiles) {
#pragma unroll
      for (int k = 0; k < 2 * NPIECE; ++k) dma_piece(tt, ic, k);
    }
    if constexpr (WALK) {
      walk_next(vchunk, vpos);
      walk_next(kchunk, kpos);
    }
    wait_vmem_but<NPIECE>();
    phase_barrier();
  };

  // The ring's next chunk into the idle slot (this block's share), while the
  // block's first tile loads are in flight.
  if constexpr (!WALK) {
    if (stage_now) stage_block_share<64 * NW, 8>(stage.src, stage.dst, stage.units);
  }

  // Prologue: S^T(0) once K(0) has landed (computed, harmlessly, also for a
  // wave with no rows); its stream issues iteration 0's first reads.
  wait_vmem();
  phase_barrier();
  {
    auto none = [](auto) __attribute__((always_inline)) {};
    static_for<LA>([&](auto mc) __attribute__((always_inline)) {
      read_s(mc, mc, std::integral_constant<int, 0>{});
    });
    mfma_stream(std::false_type{}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
                std::integral_constant<int, NB - 1>{}, sacc[0], none);
  }
  // Steps past ntiles only keep the barrier count uniform.
  for (int tt = 0; tt <= ntiles; tt += NB) {
    step(tt, std::integral_constant<int, 0>{});
    step(tt + 1, std::integral_constant<int, 1>{});
    step(tt + 2, std::integral_constant<int, 2>{});
    step(tt + 3, std::integral_constant<int, 3>{});
  }
  // Reads issued for an iteration that never ran, and the tile loads still
  // in flight (nothing lands in LDS once the block is done).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  wait_vmem();

  fwd_epilogue<D, MERGE>(oacc, mrow, lrow - lcomp, og, lseg, bh, Sq, qq, g);
}

// One ring step: block b takes unit xcd_remap(b) of a full chunk, or
// level-ordered unit b of the diagonal.  Block 0 first zeroes the work-queue
// counters of the next step launch (queue_next), if any.
template <int D, bool DIAG, bool MERGE>
__global__ __launch_bounds__(64 * kFwdWaves) void fwd_step_kernel(const uint16_t* __restrict__ qg,
                                                                  const uint16_t* __restrict__ kg,
                                                                  const uint16_t* __restrict__ vg,
                                                                  float* __restrict__ og,
                                                                  float* __restrict__ lseg, int Sq, int Sk,
                                                                  int n_qtiles, int total_tiles,
                                                                  float scale_log2, int group, int qoff,
                                                                  StageCopy stage, int* queue_next) {
  if (queue_next && blockIdx.x == 0 && threadIdx.x < kFwdQueueInts) queue_next[threadIdx.x] = 0;
  const ChunkTable none{};
  const int unit = DIAG ? (int)blockIdx.x : xcd_remap(blockIdx.x, total_tiles);
  fwd_body<D, DIAG, MERGE, false>(qg, kg, vg, og, lseg, Sq, Sk, n_qtiles, total_tiles, scale_log2, group, qoff,
                                  none, stage, unit, true);
}

// One full-chunk ring step on persistent blocks (one per compute unit).
// Thread 0 takes the next unit of its XCD's queue -- XCD x's queue holds the
// units that xcd_remap gives XCD x, in the same order -- and, once that
// queue is empty, of the next XCDs' in turn.  The units are equal work, but
// the XCDs do not run at equal speed, and a static split ends with the
// slowest one.  queue: kFwdQueueInts zeroed counters, one per XCD 64 bytes
// apart; queue_next as in fwd_step_kernel.
template <int D, bool MERGE>
__global__ __launch_bounds__(64 * kFwdWaves) void fwd_queue_kernel(const uint16_t* __restrict__ qg,
                                                                   const uint16_t* __restrict__ kg,
                                                                   const uint16_t* __restrict__ vg,
                                                                   float* __restrict__ og,
                                                                   float* __restrict__ lseg, int Sq, int Sk,
                                                                   int n_qtiles, int total_tiles,
                                                                   float scale_log2, int group, int qoff,
                                                                   StageCopy stage, int* queue, int* queue_next) {
  static_assert(16 * kXcds <= kFwdQueueInts, "one counter per XCD, 64 bytes apart");
  if (queue_next && blockIdx.x == 0 && threadIdx.x < kFwdQueueInts) queue_next[threadIdx.x] = 0;
  const ChunkTable none{};
  __shared__ int unit_s;
  // This wave's XCD (hardware register XCC_ID).
  const int xcd = (int)(__builtin_amdgcn_s_getreg(kHwRegXccId) % kXcds);
  const int q = total_tiles / kXcds, r = total_tiles % kXcds;
  int from = 0;  // queues xcd, xcd+1, ... before `from` are empty (thread 0)
  for (bool first = true;; first = false) {
    if (threadIdx.x == 0) {
      int t = -1;
      for (; from < kXcds; ++from) {
        const int y = (xcd + from) % kXcds;
        const int n = __hip_atomic_fetch_add(queue + 16 * y, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n < q + (y < r ? 1 : 0)) {
          t = y * q + (y < r ? y : r) + n;
          break;
        }
      }
      unit_s = t;
    }
    __syncthreads();
    const int t = unit_s;
    __syncthreads();  // every thread has read unit_s before thread 0 writes it again
    if (t < 0) {
      // A block that started after the queues ran dry (the grid need not
      // be resident all at once) still copies its share of the next chunk.
      if (first) stage_block_share<64 * kFwdWaves, 8>(stage.src, stage.dst, stage.units);
      break;
    }
    fwd_body<D, false, MERGE, false>(qg, kg, vg, og, lseg, Sq, Sk, n_qtiles, total_tiles, scale_log2, group, qoff,
                                     none, stage, t, first);
  }
}

// One pass over resident chunks (no merge: the pass sees every key).
template <int D, bool DIAG>
__global__ __launch_bounds__(64 * kFwdWaves) void fwd_walk_kernel(const uint16_t* __restrict__ qg,
                                                                  float* __restrict__ og,
                                                                  float* __restrict__ lseg, int Sq, int Sk,
                                                                  int n_qtiles, int total_tiles,
                                                                  float scale_log2, int group, int qoff,
                                                                  ChunkTable tbl) {
  const StageCopy none{};
  const int unit = DIAG ? (int)blockIdx.x : xcd_remap(blockIdx.x, total_tiles);
  fwd_body<D, DIAG, false, true>(qg, nullptr, nullptr, og, lseg, Sq, Sk, n_qtiles, total_tiles, scale_log2, group,
                                 qoff, tbl, none, unit, true);
}

constexpr int kPersistentUnitsPerCu = 4;

// Compute units of the current device, looked up once per device.
int compute_units() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return -1;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D>
hipError_t launch_cfg(const FwdStepArgs& a, hipStream_t stream) {
  constexpr int BR = kFwdWaves * kFwdRowsPerWave;
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  if (a.group < 1 || a.BH % a.group || a.qoff < 0 || (long long)a.Sq + a.qoff + BR > 0x7fffffffLL)
    return hipErrorInvalidValue;
  const long long total = (long long)n_qtiles * a.BH;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sl2 = a.scale * kLog2e;
  dim3 grid((unsigned)total), block(64 * kFwdWaves);
  if (a.walk) {
    const ChunkTable& t = *a.walk;
    if (a.merge || a.stage || t.n < 1 || t.n > kMaxWalkChunks || t.C < 1 || t.C % kTileTokens ||
        (long long)t.n * t.C != a.Sk)
      return hipErrorInvalidValue;
    if (a.diag)
      hipLaunchKernelGGL((fwd_walk_kernel<D, true>), grid, block, 0, stream, a.q, a.o, a.lse, a.Sq, a.Sk, n_qtiles,
                         (int)total, sl2, a.group, a.qoff, t);
    else
      hipLaunchKernelGGL((fwd_walk_kernel<D, false>), grid, block, 0, stream, a.q, a.o, a.lse, a.Sq, a.Sk, n_qtiles,
                         (int)total, sl2, a.group, a.qoff, t);
    return hipGetLastError();
  }
  const StageCopy stage = a.stage ? *a.stage : StageCopy{};
  // Persistent blocks only where each compute unit has several units to
  // take (kPersistentUnitsPerCu or more): with fewer, the last unit of each
  // block sets the step's length anyway, and a staging copy queued on
  // another stream would wait for CUs that the step holds throughout.
  if (a.queue && !a.diag) {
    const int ncu = compute_units();
    if (ncu <= 0) return hipErrorInvalidDevice;
    if (total >= (long long)kPersistentUnitsPerCu * ncu) {
      const dim3 pgrid((unsigned)ncu);
      if (a.merge)
        hipLaunchKernelGGL((fwd_queue_kernel<D, true>), pgrid, block, 0, stream, a.q, a.k, a.v, a.o, a.lse, a.Sq,
                           a.Sk, n_qtiles, (int)total, sl2, a.group, a.qoff, stage, a.queue, a.queue_next);
      else
        hipLaunchKernelGGL((fwd_queue_kernel<D, false>), pgrid, block, 0, stream, a.q, a.k, a.v, a.o, a.lse, a.Sq,
                           a.Sk, n_qtiles, (int)total, sl2, a.group, a.qoff, stage, a.queue, a.queue_next);
      return hipGetLastError();
    }
  }
#define RA_FWD_LAUNCH(DIAG, MERGE)                                                                         \
  hipLaunchKernelGGL((fwd_step_kernel<D, DIAG, MERGE>), grid, block, 0, stream, a.q, a.k, a.v, a.o, \
                     a.lse, a.Sq, a.Sk, n_qtiles, (int)total, sl2, a.group, a.qoff, stage, a.queue_next)
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

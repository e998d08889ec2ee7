// Device-side building blocks shared by the ring-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>
#include <utility>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;  // MI355X: 8 XCDs x 32 CUs; workgroups go round-robin over XCDs
// s_getreg operand for the XCC_ID hardware register (id 20, all 32 bits):
// the XCD the wave runs on.
constexpr int kHwRegXccId = 20 | (31 << 11);
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l holds A row l%32 and B column l%32, with k = (l/32)*8 + [0..7] (any
// k order shared by A and B gives the same product).  C/D lane l holds
// column l%32, register i = row 8*(i/4) + 4*(l/32) + i%4.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// A 32-bit pattern as float, taken by value.  __builtin_bit_cast applied to
// a vector element (v[e]) reinterprets the vector's storage from element 0
// whatever e is, so vector elements go through this scalar parameter.
__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of x over the lane pair (l, l ^ 32) with v_permlane32_swap (a
// VALU lane exchange, no LDS round trip): swapping the upper half of one copy
// with the lower half of another leaves x[l] and x[l^32] in the two results.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Logical tile for a dispatched block: gives each XCD one contiguous range of
// logical tiles, so blocks resident on one XCD share K/V lines in its L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int xcd = b % kXcds, slot = b / kXcds;
  const int q = total / kXcds, r = total % kXcds;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Block b's (head row, level) in a causal launch whose blocks shrink with the
// level: level 0 (the longest block of every head) for all n_bh head rows
// first, then level 1, and so on.  Consecutive blocks go round-robin over the
// XCDs, so every XCD receives its blocks longest first; when n_bh is a
// multiple of the XCD count, an XCD holds the same head rows at every level
// (their K/V lines stay in its L2).  Ordering the levels within each head
// only would start some heads' longest blocks near the end of the launch.
__device__ __forceinline__ void longest_first(int b, int n_bh, int& bh, int& level) {
  level = b / n_bh;
  bh = b - level * n_bh;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Eight consecutive accumulator registers (the k slots of one MFMA operand)
// packed to bf16.
__device__ __forceinline__ u32x4 pack8(const f32x16& a, int base) {
  return u32x4{pack_bf16(a[base + 0], a[base + 1]), pack_bf16(a[base + 2], a[base + 3]),
               pack_bf16(a[base + 4], a[base + 5]), pack_bf16(a[base + 6], a[base + 7])};
}

constexpr int kTileTokens = 64;  // tokens per LDS tile

// ---------------------------------------------------------------------------
// Direct-to-LDS tiles of 64 tokens (row-major, D bf16 per token).
//
// 16-byte chunk c of token row r sits at physical chunk swz<D>(r, c) of its
// row.  The XOR mask is chosen so that both reads the MFMAs need are free of
// bank conflicts:
//  * A operand of K Q^T: 32 consecutive rows, one chunk each (any 16
//    consecutive rows land in 16 distinct 16-byte bank groups);
//  * the transposing read of V (ds_read_b64_tr_b16): 4 consecutive rows x
//    4 consecutive chunks per 32 lanes, all distinct.
// XOR with a row-only mask is its own inverse, so the same function maps a
// physical slot back to its logical chunk.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (D == 128) {
    const int x = row & 15;
    return c ^ (((x & 3) << 2) | ((x >> 2) & 3));
  } else {
    const int x = (row >> 1) & 7;
    return c ^ (((x & 1) << 2) | ((x >> 1) & 3));
  }
}

template <int D>
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * (D * 2) + (swz<D>(row, c) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;

// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format,
// no swizzle, no thread-id addressing).
constexpr int kBufWord3 = 0x00020000;

// Direct-to-LDS loading of 64-token tiles with buffer loads into LDS (16
// bytes per lane, 1 KB per instruction, no registers).  Wave `wave` of NW
// issues its share of the tile's 1 KB pieces; piece p fills LDS bytes
// [1024p, 1024p+1024) of the tile in lane order, so lane l loads the global
// chunk that belongs at physical slot l of the piece.  The tile's first row
// is the buffer resource's base and the tile's rows that exist in the matrix
// (at most TOK) set its size, so the per-lane offset is the same for every
// tile (no vector arithmetic per piece), and rows past the end fail the
// buffer range check, which writes zeros to LDS instead of reading out of
// bounds.
template <int D, int NW, int TOK = kTileTokens>
struct TileBufDma {
  static constexpr int kPieces = TOK * D * 2 / 1024;
  static constexpr int kRowsPerPiece = 1024 / (D * 2);
  static constexpr int kPerWave = kPieces / NW;
  static_assert(kPieces % NW == 0, "tile pieces must split evenly over waves");
  uint32_t off[kPerWave];  // byte offset of this lane's 16 bytes from the tile's first row
  int piece0;              // first piece of this wave

  __device__ __forceinline__ void init(int wave, int lane) {
    const int rin = (lane * 16) / (D * 2);
    const int p = ((lane * 16) % (D * 2)) >> 4;
    piece0 = wave * kPerWave;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int row = (piece0 + i) * kRowsPerPiece + rin;
      off[i] = (uint32_t)(row * D * 2 + swz<D>(row, p) * 16);
    }
  }

  // This wave's piece i of tokens t0 .. t0+TOK-1 of the [n, D] bf16 matrix
  // at `mat` into `tile`; tokens at or past n read as zeros.  t0 >= 0 and
  // the arguments other than the piece index are wave-uniform.
  __device__ __forceinline__ void load_piece(int i, uint8_t* tile, const uint16_t* mat, int t0, int n) const {
#if defined(__HIP_DEVICE_COMPILE__)
    // The resource covers this tile only: its byte size stays far below the
    // 32-bit record count however long the matrix is.
    const int rows = n > t0 ? min(n - t0, TOK) : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(mat) + (size_t)t0 * D, 0, rows * (D * 2), kBufWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(tile + (piece0 + i) * 1024), 16, off[i], 0, 0, 0);
#else
    (void)i, (void)tile, (void)mat, (void)t0, (void)n;
#endif
  }

  __device__ __forceinline__ void load(uint8_t* tile, const uint16_t* mat, int t0, int n) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) load_piece(i, tile, mat, t0, n);
  }
};

// One ds_read_b64_tr_b16 at LDS byte address addr + OFF, as inline assembly:
// the compiler cannot see which LDS buffer the intrinsic form reads, so it
// would wait for every direct-to-LDS load in flight (into any buffer).  The
// result is valid only after a wait that names it (lgkm_wait).  Within each
// 16-lane group, lane 4a+b receives element b of the 64-bit rows supplied
// by lanes a, 4+a, 8+a, 12+a.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_off(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// One ds_read_b128 at LDS byte address addr + OFF, as inline assembly like
// ds_read_tr16_off (valid only after a wait that names the result).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128_off(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Waits until at most N LDS operations of this wave are outstanding.  LDS
// operations complete in issue order, so when N counts only reads issued
// after the one that produced the tied registers, those registers are valid
// afterwards; tying them orders their consumers after the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& a) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x2& a, u32x2& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// Workgroup barrier that no instruction is scheduled across, with no memory
// fence: every LDS read before it has already been waited for by its consumer,
// and LDS-DMA completion is waited for explicitly (wait_vmem) where needed.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

// s_waitcnt vmcnt(0) (global loads, including loads into LDS, complete).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Waits until at most N vector-memory operations of this wave are
// outstanding (vmcnt(N), N < 16); they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 16, "vmcnt low field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// This block's share of a staging copy: units [b*per, min((b+1)*per, n)) of
// each tensor, per = ceil(n / gridDim.x), 16 bytes per unit, UNROLL loads in
// flight per thread.  Every thread of the block calls it.
template <int NTHREADS, int UNROLL = 4>
__device__ __forceinline__ void stage_block_share(const void* const (&src)[2], void* const (&dst)[2], size_t n) {
  if (n == 0) return;
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t u0 = (size_t)blockIdx.x * per;
  const size_t u1 = u0 + per < n ? u0 + per : n;
  for (int t = 0; t < 2; ++t) {
    const u32x4* __restrict__ s = static_cast<const u32x4*>(src[t]);
    u32x4* __restrict__ d = static_cast<u32x4*>(dst[t]);
    for (size_t u = u0 + threadIdx.x; u < u1; u += (size_t)NTHREADS * UNROLL) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int k = 0; k < UNROLL; ++k)
        if (u + (size_t)k * NTHREADS < u1) v[k] = __builtin_nontemporal_load(s + u + (size_t)k * NTHREADS);
#pragma unroll
      for (int k = 0; k < UNROLL; ++k)
        if (u + (size_t)k * NTHREADS < u1) d[u + (size_t)k * NTHREADS] = v[k];
    }
  }
}

}  // namespace ra

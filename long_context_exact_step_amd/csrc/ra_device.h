// Device-side building blocks shared by the ring-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 XCDs x 32 CUs; workgroups go round-robin over XCDs
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, kWave);
}

// Logical tile for a dispatched block: gives each XCD one contiguous range of
// logical tiles, so blocks resident on one XCD share K/V lines in its L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int xcd = b % kXcds, slot = b / kXcds;
  const int q = total / kXcds, r = total % kXcds;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// LDS tiles of 64 tokens.
//
// Row-major tile: 64 token rows x D bf16, 16-byte chunk c of row r at
// row_off<D>(r, c).  The XOR swizzle puts the same chunk of 16 consecutive
// rows in 16 different bank groups, so the 32-row MFMA operand reads (one
// 16-byte chunk per lane) are conflict-free.
//
// Transposed tile: D rows (one per feature) x 64 token positions bf16, 128
// bytes per row.  Token positions are permuted within each group of 16
// (bits 2 and 3 of the index swapped) so that the 8 tokens a lane needs as
// the k slots of an MFMA operand -- rows 16h + 4g + {0..3, 8..11} of a 32x32
// accumulator -- are one contiguous 16-byte chunk: chunk 4*kb + 2*h + g of a
// row holds those tokens for 32-token block kb.
// ---------------------------------------------------------------------------
constexpr int kTileTokens = 64;

template <int D>
__device__ __forceinline__ int row_off(int r, int c) {
  if constexpr (D == 128) return r * 256 + ((c ^ (r & 15)) << 4);
  else return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}

__device__ __forceinline__ int tr_off(int d, int c) { return d * 128 + ((c ^ ((d >> 1) & 7)) << 4); }

// Writes tokens 4*kq .. 4*kq+3 (rows[rr] = features 8*dc .. 8*dc+7 of token
// 4*kq+rr) into the transposed tile.
__device__ __forceinline__ void store_tr4x8(uint8_t* ts, int dc, int kq, const u32x4 (&rows)[4]) {
  const int u = kq & 3;
  const int pos = (kq & ~3) * 4 + (((u & 1) << 1) | (u >> 1)) * 4;
  const int half = (pos & 4) ? 8 : 0;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    const int w = cc >> 1;
    uint32_t lo, hi;
    if (cc & 1) {
      lo = (rows[0][w] >> 16) | (rows[1][w] & 0xffff0000u);
      hi = (rows[2][w] >> 16) | (rows[3][w] & 0xffff0000u);
    } else {
      lo = (rows[0][w] & 0xffffu) | (rows[1][w] << 16);
      hi = (rows[2][w] & 0xffffu) | (rows[3][w] << 16);
    }
    *reinterpret_cast<u32x2*>(ts + tr_off(dc * 8 + cc, pos >> 3) + half) = u32x2{lo, hi};
  }
}

// The 16-byte operand chunk of a transposed tile: feature row d, 32-token
// block kb, half h (tokens 16h..16h+15 of the block), lane group g.
__device__ __forceinline__ u32x4 ld_tr(const uint8_t* ts, int d, int kb, int h, int g) {
  return *reinterpret_cast<const u32x4*>(ts + tr_off(d, kb * 4 + 2 * h + g));
}

// Eight consecutive accumulator registers (the k slots of one MFMA operand)
// packed to bf16.
__device__ __forceinline__ u32x4 pack8(const f32x16& a, int base) {
  return u32x4{pack_bf16(a[base + 0], a[base + 1]), pack_bf16(a[base + 2], a[base + 3]),
               pack_bf16(a[base + 4], a[base + 5]), pack_bf16(a[base + 6], a[base + 7])};
}

}  // namespace ra

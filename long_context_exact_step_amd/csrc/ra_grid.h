// Launch geometry of the row kernels (standalone merge, backward row
// pre-pass, zero fill).  Plain C++ with no HIP dependency, so the arithmetic
// can be checked on the host at the sizes the entry points accept.
//
// The kernels walk their items with a grid-stride loop, so the grid is
// capped: a launch's work-item count (blocks x threads per block) must fit
// the 32-bit grid size of the dispatch packet, and the host accepts up to
// 2^31 - 1 rows per tensor (which at 32 lanes per row is 2^36 items).
#pragma once

#include <cstdint>

namespace ra {

constexpr unsigned kRowThreads = 256;       // threads per block of every row kernel
constexpr unsigned kRowMaxBlocks = 1u << 16;  // 64K blocks: 16M work-items per launch at most

// Blocks of kRowThreads for `items` work-items (0 for none), at most
// kRowMaxBlocks; each thread then strides by blocks * kRowThreads.
constexpr unsigned row_grid_blocks(uint64_t items) {
  const uint64_t need = (items + kRowThreads - 1) / kRowThreads;
  return need < kRowMaxBlocks ? (unsigned)need : kRowMaxBlocks;
}

}  // namespace ra

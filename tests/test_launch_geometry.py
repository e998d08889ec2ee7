"""Launch geometry of the row kernels (merge, backward row pre-pass, zero
fill) at the sizes the entry points accept, checked on the host: the header
that computes it is plain C++ and is compiled here with g++.

The host accepts up to 2^31 - 1 rows per tensor; at 32 lanes per row that is
about 2^36 work-items, far past the 32-bit work-item count of one dispatch.
The kernels therefore stride over their items with a capped grid; this test
checks that every launch stays within the dispatch limits and that the
stride keeps the properties the kernels rely on (a row's lanes in one wave
and one loop trip)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_exact_step_amd", "csrc")

PROGRAM = r"""
#include <cstdio>
#include <cstdint>
#include "ra_grid.h"
int main() {
  const uint64_t max_rows = (1ull << 31) - 1;
  const uint64_t cases[] = {1, 2, 31, 32, 255, 256, 257, 1ull << 20, (1ull << 24) + 7, 1ull << 27,
                            (1ull << 27) + 1, 1ull << 32, (1ull << 32) + 1, max_rows * 16, max_rows * 32,
                            max_rows * 128};
  for (uint64_t n : cases) {
    const unsigned b = ra::row_grid_blocks(n);
    const uint64_t items = (uint64_t)b * ra::kRowThreads;
    std::printf("%llu %u %llu\n", (unsigned long long)n, b, (unsigned long long)items);
  }
  std::printf("zero %u\n", ra::row_grid_blocks(0));
  std::printf("threads %u max %u\n", ra::kRowThreads, ra::kRowMaxBlocks);
  return 0;
}
"""


@pytest.fixture(scope="module")
def geometry(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("geom")
    src, exe = d / "geom.cpp", d / "geom"
    src.write_text(PROGRAM)
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Werror", "-I" + CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines()
    rows = [tuple(int(x) for x in line.split()) for line in out if line[0].isdigit()]
    zero = int(out[-2].split()[1])
    threads, maxb = int(out[-1].split()[1]), int(out[-1].split()[3])
    return rows, zero, threads, maxb


def test_every_launch_fits_the_dispatch(geometry):
    rows, zero, threads, maxb = geometry
    assert zero == 0
    for n, blocks, items in rows:
        assert 1 <= blocks <= maxb
        assert items < 2 ** 32, f"{n} items: grid of {items} work-items overflows the dispatch"
        # Small inputs get one thread per item (no idle launch beyond a block).
        if n <= maxb * threads:
            assert blocks == -(-n // threads)


def test_stride_keeps_rows_in_one_wave_and_trip(geometry):
    rows, _, threads, _ = geometry
    assert threads % 64 == 0
    for _, blocks, items in rows:
        # Rows of 32 lanes (pre-pass) and of d/4 = 16 or 32 lanes (merge)
        # stay in one 64-lane wave and one loop trip when the stride is a
        # multiple of 64.
        assert items % 64 == 0


def test_host_limit_is_covered(geometry):
    """At the host's row limit the strided grid covers every item of the
    largest launch (merge at d = 128: 32 lanes per row; pre-pass: 32 lanes
    per row; zero fill of dq: d floats per row)."""
    rows, _, _, _ = geometry
    by_n = {n: (b, items) for n, b, items in rows}
    n = ((1 << 31) - 1) * 128
    b, items = by_n[n]
    trips = -(-n // items)
    assert trips * items >= n and (trips - 1) * items < n

// Host-only check of libecho's grid sizes (launch_shape.h) at the extreme
// sizes the header allows: no HIP, no launch.  Exits non-zero on failure.
#include <stdint.h>
#include <stdio.h>

#include "echo.h"
#include "launch_shape.h"

using namespace echo;

static int fails = 0;
#define CHECK(c)                                             \
  do {                                                       \
    if (!(c)) {                                              \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++fails;                                               \
    }                                                        \
  } while (0)

// A grid is launchable when its x dimension holds at most 2^32 - 1 work-items.
static bool launchable(uint64_t blocks) { return blocks >= 1 && blocks * kBlock <= 0xFFFFFFFFull; }

// The kernels' grid-stride loops step a 32-bit wave-step index by the grid's
// wave count; the index must not wrap before it passes the end.
static bool stride_fits(uint64_t steps, uint64_t blocks, uint64_t per_step) {
  const uint64_t nwaves = blocks * kWavesPerBlock;
  return steps + nwaves * per_step <= 0xFFFFFFFFull;
}

int main() {
  CHECK((uint64_t)kMaxBlocks * kBlock <= 0xFFFFFFFFull);
  CHECK(blocks_for(0) == 1);
  CHECK(blocks_for(1) == 1);
  CHECK(blocks_for(kWavesPerBlock) == 1);
  CHECK(blocks_for(kWavesPerBlock + 1) == 2);
  CHECK(blocks_for(~0ull) == kMaxBlocks);
  CHECK(blocks_for(1000, 7) == 7);
  CHECK(blocks_for_items(0) == 1);
  CHECK(blocks_for_items(kBlock) == 1);
  CHECK(blocks_for_items(kBlock + 1) == 2);
  CHECK(blocks_for_items(~0ull) == kMaxBlocks);

  const uint64_t n = (uint64_t)ECHO_MAX_ELEMENTS;
  const uint64_t groups = n / ECHO_GROUP;
  // stage-1 and reduce kernels: one slice (2 groups) per wave step, up to 2
  const uint64_t slices = (groups + 1) / 2;
  for (uint64_t u = 1; u <= 2; ++u) {
    const uint32_t b = blocks_for((slices + u - 1) / u);
    CHECK(launchable(b));
    CHECK(stride_fits(slices, b, u));
  }
  // exit kernel: quads of groups, 2 per wave step, grid (blocks, segments)
  for (uint32_t nseg = 1; nseg < ECHO_MAX_RANKS; ++nseg) {
    const uint64_t quads = (groups / (nseg + 1) + 3) / 4;
    const uint32_t b = blocks_for((quads + 1) / 2, kMaxBlocks / nseg);
    CHECK(launchable(b));
    CHECK(stride_fits(quads, b, 2));
  }
  // zero fill of the averages (float4 items) and the stream copy (16-byte items)
  CHECK(launchable(blocks_for_items(n / 4)));
  CHECK(launchable(blocks_for_items(((uint64_t)1 << 40) / 16)));
  if (fails) return 1;
  printf("launch shapes ok: kMaxBlocks = %u\n", kMaxBlocks);
  return 0;
}

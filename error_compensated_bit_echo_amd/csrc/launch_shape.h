// launch_shape.h -- grid sizes of libecho's launches.  Host arithmetic only
// (no HIP types), so a plain C++ program can check the limits.
#pragma once

#include <stdint.h>

#ifndef ECHO_BLOCK
#define ECHO_BLOCK 256
#endif

namespace echo {

constexpr int kBlock = ECHO_BLOCK;  // threads per workgroup (4 wavefronts)
constexpr int kWavesPerBlock = kBlock / 64;

// A launch's x dimension may hold at most 2^32 - 1 work-items (gridDim.x *
// blockDim.x), so at most this many workgroups.  Every kernel has a
// grid-stride loop, so a capped grid still covers its range.
constexpr uint32_t kMaxBlocksHip = 0xFFFFFFFFu / (uint32_t)kBlock;
#ifdef ECHO_MAX_BLOCKS
constexpr uint32_t kMaxBlocks =
    (uint32_t)ECHO_MAX_BLOCKS < kMaxBlocksHip ? (uint32_t)ECHO_MAX_BLOCKS : kMaxBlocksHip;
#else
constexpr uint32_t kMaxBlocks = kMaxBlocksHip;
#endif

// Workgroups for `wave_steps` wavefront steps: at least 1, at most `cap`.
inline uint32_t blocks_for(uint64_t wave_steps, uint32_t cap = kMaxBlocks) {
  uint64_t b = wave_steps / kWavesPerBlock + (wave_steps % kWavesPerBlock != 0);
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (uint32_t)b;
}

// Workgroups for a grid-stride loop with one item per thread.
inline uint32_t blocks_for_items(uint64_t items, uint32_t cap = kMaxBlocks) {
  uint64_t b = items / kBlock + (items % kBlock != 0);
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (uint32_t)b;
}

}  // namespace echo

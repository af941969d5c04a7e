// Launch description of the rate and pack kernels over several matrices.
#pragma once

#include "hq_internal.h"

namespace hq {

constexpr int kRateMaxItems = 8;   // matrices per launch

// Up to kRateMaxItems matrices that share the tile and the coset layout;
// block0[i] numbers matrix i's first rate / pack block, block0[n] the total.
struct RateBatch {
  int32_t n;
  int32_t pad;
  int64_t block0[kRateMaxItems + 1];
  RateLaunch it[kRateMaxItems];
};

// Rate and pack blocks of one matrix (the same for its rate and pack grids).
int64_t rate_blocks(int tile, int64_t n_tiles);
hipError_t launch_rate_batch(const RateBatch& b, hipStream_t s);

}  // namespace hq

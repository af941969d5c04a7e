// The KV dither on the 2^-24 grid, shared by the kernels that regenerate it
// (tile-128 encode and decode, attention over the compressed cache).
//
// Passage: [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice
// Quantization Pipeline ..." (subtractive dither).  w = 2^-23 h - 1 for the
// top 24 bits h of the counter hash of (seed, vector, element); the dither
// is d = w - Q_E8(w), taken exactly on the grid W = w 2^24.
#pragma once

#include "hq_device.h"
#include "hq_lanes.h"

namespace hq {
namespace {

using namespace fastlib;

// d = w - Q_E8(w) for one block, on the 2^-24 grid (W = w 2^24), exact.  The
// nearest point is decided as in e8_block_fast; with off = [coset a] 2^23 the
// coordinate's offset from its point is ((W + off) mod 2^24) - 2^23, and the
// parity flip moves one coordinate's point by one.
__device__ inline void e8_dither_block(const int32_t* W, int32_t* d24) {
  uint32_t k1[8];
#define HQ_DITHER_KEYS(i)                                         \
  {                                                               \
    const uint32_t F8 = ((uint32_t)W[i] << 3) & 0x07FFFFFFu;      \
    k1[i] = sad26<i>(F8);                                         \
  }
  HQ_DITHER_KEYS(0) HQ_DITHER_KEYS(1) HQ_DITHER_KEYS(2) HQ_DITHER_KEYS(3)
  HQ_DITHER_KEYS(4) HQ_DITHER_KEYS(5) HQ_DITHER_KEYS(6) HQ_DITHER_KEYS(7)
#undef HQ_DITHER_KEYS
  const uint32_t kmin = min3u(min3u(k1[0], k1[1], k1[2]), min3u(k1[3], k1[4], k1[5]),
                              k1[6] < k1[7] ? k1[6] : k1[7]);
  const uint32_t kmax = max3u(max3u(k1[0], k1[1], k1[2]), max3u(k1[3], k1[4], k1[5]),
                              k1[6] > k1[7] ? k1[6] : k1[7]);
  const int32_t bmin = (int32_t)(kmin >> 3), bmax = (int32_t)(kmax >> 3);
  if (bmin == 0 || bmax == kHalf) {
    int32_t z[8];
    const int c = e8_nearest(W, z);
#pragma unroll
    for (int i = 0; i < 8; ++i) d24[i] = W[i] - (shl24(z[i]) + (c ? kHalf : 0));
    return;
  }
  const uint32_t sumB =
      (((k1[0] + k1[1] + k1[2]) + (k1[3] + k1[4] + k1[5]) + (k1[6] + k1[7])) - 28u) >> 3;
  const uint32_t X = ((uint32_t)W[0] ^ (uint32_t)W[1] ^ (uint32_t)W[2]) ^
                     ((uint32_t)W[3] ^ (uint32_t)W[4] ^ (uint32_t)W[5]) ^
                     ((uint32_t)W[6] ^ (uint32_t)W[7]);
  const int odd_b = (int)((X >> 24) & 1u);
  const int odd_a = (int)(((X >> 23) ^ (X >> 24)) & 1u);
  const int32_t D = (1 << 25) - (int32_t)sumB + (odd_a ? 2 * bmin : 0) -
                    (odd_b ? (1 << 24) - 2 * bmax : 0);
  const int c = D > 0;
  const uint32_t jf = c ? (kmax & 7u) : (kmin & 7u);
  const int odd = c ? odd_b : odd_a;
  const uint32_t G0 = third_bytes(W[0], W[1], W[2], W[3]);
  const uint32_t G1 = third_bytes(W[4], W[5], W[6], W[7]);
  const uint32_t upj = (uint32_t)((((uint64_t)G1 << 32) | G0) >> (8 * jf + 7)) & 1u;
  const bool neg = ((uint32_t)c ^ upj) != 0u;   // the flipped point moves by -1
  const uint32_t off = c ? 0u : (uint32_t)kHalf;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int32_t d = (int32_t)(((uint32_t)W[i] + off) & 0xFFFFFFu) - kHalf;
    if (odd && (uint32_t)i == jf) d += neg ? kOne : -kOne;
    d24[i] = d;
  }
}

// W = w 2^24 for element e of vector vec: w = 2^-23 h - 1, h the top 24 bits
// of the counter hash (SplitMix64) of the key (seed << 40) ^ (vec << 8 | e).
//
// The vector's part is taken once.  With B = (seed << 40 ^ vec << 8) + the
// additive constant (low byte 0x15), the first state is B + e, and for
// e <= 0xEA the element moves only the low byte of it (0x15 + e, no carry).
// So the first xor-shift's high word, and every bit it brings down into the
// low word, are the vector's: x_lo = q ^ (0x15 + e), x_hi fixed, and of the
// first 64-bit product only x_lo's terms change (p = lo32(x_hi C1lo) is the
// vector's).  The last xor-shift leaves the top 24 bits unchanged, so h is
// bits 40..63 of the second product, whose high word takes three 32-bit
// products.  Bit-identical to the full hash for every e <= 0xEA (tile and
// head sizes up to 128 use e < 128).
struct DitherVec {
  uint32_t q;   // x_lo ^ (0x15 + e)
  uint32_t p;   // lo32(x_hi C1lo)
};

constexpr uint64_t kSmC1 = 0xBF58476D1CE4E5B9ull, kSmC2 = 0x94D049BB133111EBull;
constexpr uint32_t kSmC1Lo = 0x1CE4E5B9u;

__host__ __device__ inline DitherVec dither_vec(uint32_t seed, uint64_t vec) {
  const uint64_t B = (((uint64_t)seed << 40) ^ (vec << 8)) + 0x9E3779B97F4A7C15ull;
  const uint32_t bl = (uint32_t)B, bh = (uint32_t)(B >> 32);
  const uint32_t xh = bh ^ (bh >> 30);
  const uint32_t m = (bh << 2) | (bl >> 30);   // low word of B >> 30
  return DitherVec{(bl & 0xFFFFFF00u) ^ m, xh * kSmC1Lo};
}

__host__ __device__ inline int32_t dither_w(const DitherVec& k, uint32_t e) {
  const uint32_t xl = k.q ^ (0x15u + e);
  // x C1 = x_lo C1 + 2^32 x_hi C1lo; only bits 40..63 of the second product
  // are kept, so its low word is never formed
  const uint64_t z1 = (uint64_t)xl * kSmC1 + ((uint64_t)k.p << 32);
  const uint64_t z2 = z1 ^ (z1 >> 27);
  return 2 * (int32_t)((z2 * kSmC2) >> 40) - kOne;
}

}  // namespace
}  // namespace hq

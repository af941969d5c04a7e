// Encode kernels: tile load -> signs -> scale -> Walsh-Hadamard -> quantizer
// grid -> (dither) -> nearest lattice point -> strip -> Rice rate -> stores.
//
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." ideas (i) rotation, (ii) lattice, (iii) strip and
// Rice coding, (iv) KV bias correction; [ICLR abstract] "HyperQuant: A
// Near-Entropy-Optimal Lattice Quantization Pipeline ..." (E8 default,
// lossless strip, Rice, subtractive dither).
//
// Work mapping: a tile of N elements is held by G = N/16 consecutive lanes,
// 16 contiguous elements per lane (two or four 16-byte loads), so a wave
// covers 64/G whole tiles.  The first four Hadamard stages run inside a lane,
// the remaining log2(G) across the lane group.  Butterflies run in fp64 and
// are exact for bf16 tiles (every partial sum fits in 53 bits).
#include <type_traits>

#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

template <int G, typename T>
__device__ inline T group_sum(T v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, G);
  return v;
}

template <int G>
__device__ inline uint32_t group_or(uint32_t v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v |= __shfl_xor(v, m, G);
  return v;
}

template <int LAT>
struct Lat {
  static constexpr int kBlocksPerLane = 16 / LAT;
  // coset bits per lane: one per E8 block or A2 pair
  static constexpr int kCosetBits = (LAT == 8 || LAT == 2) ? kBlocksPerLane : 0;
};

// In-lane stages of the Sylvester Walsh-Hadamard transform (element bits 0-3)
// followed by cross-lane stages (element bits 4 .. 3 + log2 G).  Natural
// order: the lower element of each pair receives a + b, the upper a - b.
template <int G>
__device__ inline void fwht16(double* v, int r) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (!(i & h)) {
        double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < G; m <<= 1) {
    const bool upper = (r & m) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double p = __shfl_xor(v[i], m, G);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
}

__device__ inline uint32_t lane_sign_mask(const EncodeLaunch& a, int r) {
  const int w = r >> 1;
  uint32_t s = a.signs[0];
#pragma unroll
  for (int k = 1; k < kMaxTile / 32; ++k) s = (w == k) ? a.signs[k] : s;
  return (s >> (16 * (r & 1))) & 0xFFFFu;
}

// Quantizer input on the 2^-24 grid for 16 rotated values: U = rne(S K) of
// the exact product (A2: odd coordinates with K3); magnitudes past the clamp (kUClamp, or
// kUClamp16 for the 64-bit grid of the int16 index mode) flag an overflow.
template <int LAT, typename GI>
__device__ inline void grid_values(const double* v, double K, double K3, GI* U, uint32_t& st) {
  constexpr double kClamp = sizeof(GI) == 8 ? kUClamp16 : kUClamp;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    double q = rne_product(v[i], (LAT == 2 && (i & 1)) ? K3 : K);
    if (!(fabs(q) <= kClamp)) {
      st |= HQ_ST_OVERFLOW;
      q = (q > 0.0) ? kClamp : -kClamp;
    }
    U[i] = (GI)q;
  }
}

// Nearest point and lossless strip of this lane's 16 grid values: stored
// integers s, full coordinates crd (E8 and A2: 2p), coset bits of the
// lane's blocks (E8) or pairs (A2).
template <int LAT, typename GI>
__device__ inline void nearest_strip(const GI* U, int32_t* s, int16_t* crd, uint32_t& cbits) {
  cbits = 0;
  if constexpr (LAT == 8) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      int32_t z[8];
      const int c = e8_nearest(&U[8 * blk], z);
      cbits |= (uint32_t)c << blk;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s[8 * blk + i] = (i == 7) ? (z[i] >> 1) : z[i];
        crd[8 * blk + i] = (int16_t)(2 * z[i] + c);
      }
    }
  } else if constexpr (LAT == 4) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      int32_t z[4];
      d_round<4>(&U[4 * blk], z);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[4 * blk + i] = (i == 3) ? (z[i] >> 1) : z[i];
        crd[4 * blk + i] = (int16_t)z[i];
      }
    }
  } else if constexpr (LAT == 2) {
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      int32_t x0, x1;
      const int c = a2_nearest(U[2 * pr], U[2 * pr + 1], x0, x1);
      cbits |= (uint32_t)c << pr;
      s[2 * pr] = x0;
      s[2 * pr + 1] = x1;
      crd[2 * pr] = (int16_t)(2 * x0 + c);
      crd[2 * pr + 1] = (int16_t)(2 * x1 + c);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int32_t R;
      s[i] = rne_grid(U[i], R);
      crd[i] = (int16_t)s[i];
    }
  }
}

// Rice parameter of the tile: k = argmin sum(floor(zeta/2^k) + 1 + k), first
// minimum, over the int8 values of s (k >= 8 gives every zeta >> k = 0, so
// k = 8 dominates k = 9..15).  Flags int8 overflow; returns the payload bits
// and fills the lane's four packed index words.
template <int G, int N>
__device__ inline uint32_t rice_best(const int32_t* s, uint32_t& st, int& bk, uint32_t* packed) {
  uint32_t Lp[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) Lp[k] = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) packed[i] = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (s[i] < -128 || s[i] > 127) st |= HQ_ST_OVERFLOW;
    const int32_t s8 = (int32_t)(int8_t)s[i];
    packed[i >> 2] |= ((uint32_t)s8 & 0xFFu) << (8 * (i & 3));
    const uint32_t zz = zigzag(s8);
#pragma unroll
    for (int k = 0; k < 9; ++k) Lp[k] += zz >> k;
  }
  uint32_t best = 0xFFFFFFFFu;
  bk = 0;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    const uint32_t L = group_sum<G>(Lp[k]) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

// The same for int16 indices (zeta < 2^16, k in [0, 15]): the first minimum
// is one of kt - 1, kt, kt + 1 with kt the smallest k with S <= N 2^(k+1)
// (the argument of the int8 case; past k = 15 every zeta >> k is 0, so for
// S > N 2^16 the minimum is k = 15).  Fills the lane's eight words of packed
// int16 indices.
template <int G, int N>
__device__ inline uint32_t rice_best16(const int32_t* s, uint32_t& st, int& bk, uint32_t* packed) {
  uint32_t zz[16], S = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (s[i] < -32768 || s[i] > 32767) st |= HQ_ST_OVERFLOW;
    const int32_t s16 = (int32_t)(int16_t)s[i];
    if (i & 1) packed[i >> 1] |= (uint32_t)s16 << 16;
    else packed[i >> 1] = (uint32_t)s16 & 0xFFFFu;
    zz[i] = zigzag(s16);
    S += zz[i];
  }
  S = group_sum<G>(S);
  int kt = 0;
  while (kt < 15 && S > ((uint32_t)N << (kt + 1))) ++kt;
  uint32_t best = 0xFFFFFFFFu;
  bk = 0;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int k = kt - 1 + c;
    k = k < 0 ? 0 : (k > 15 ? 15 : k);
    uint32_t R = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) R += zz[i] & ((1u << k) - 1u);
    R = group_sum<G>(R);
    const uint32_t L = ((S - R) >> k) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

// WIDE: the int16 index mode (64-bit grid values, int16 indices; no dither,
// no rate control).
template <int LAT, int N, bool IN_BF16, bool DITHER, bool WIDE>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeLaunch a) {
  using GI = typename std::conditional<WIDE, int64_t, int32_t>::type;
  constexpr int G = N / kElemsPerLane;
  constexpr int TPB = kBlock / G;
  const int r = threadIdx.x % G;
  const int64_t tile = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
  if (tile >= a.n_tiles) return;   // whole lane groups leave together
  const int64_t e0 = tile * N + (int64_t)r * kElemsPerLane;

  // ---- load 16 contiguous elements
  double v[16];
  if constexpr (IN_BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.x) + e0);
    uint4 q[2] = {p[0], p[1]};
    const uint32_t* w = reinterpret_cast<const uint32_t*>(q);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = (double)bf16_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = (double)bf16_to_f32(w[i] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(
        static_cast<const float*>(a.x) + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 f = p[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
  uint32_t st = 0;
  double ss = 0.0;
  const uint32_t smask = lane_sign_mask(a, r);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (!isfinite(v[i])) st |= HQ_ST_NONFINITE;
    ss = fma(v[i], v[i], ss);
    if ((smask >> i) & 1u) v[i] = -v[i];
  }

  // ---- per-tile scale (auto: bf16_rne(rms * c); 1 for a zero tile)
  ss = group_sum<G>(ss);
  float delta;
  if (a.auto_scale) {
    double rms = sqrt(ss / (double)N);
    delta = bf16_round_to_f32(rms * a.c);
    if (delta == 0.0f) delta = 1.0f;
  } else {
    delta = a.scale[tile];
    if (!(delta > 0.0f) || !isfinite(delta)) st |= HQ_ST_NONFINITE;
  }
  // ---- rotation
  fwht16<G>(v, r);

  // ---- per-tile rate control: the finest bf16 scale, by bisection on its
  // bit pattern within eight binades of the automatic one, at which the
  // indices fit int8 and the tile fits the budget (every decision integer)
  if constexpr (!DITHER && !WIDE) {
    if (a.rate_control && group_or<G>(st) == 0u && ss > 0.0) {   // group-uniform
      auto feasible = [&](uint32_t code) {
        const double tq = a.sqrt_n * (double)__uint_as_float(code << 16);
        int32_t Uq[16], sq[16];
        int16_t cq[16];
        uint32_t stq = 0, cbq, pq[4];
        int bkq;
        grid_values<LAT>(v, 16777216.0 / tq, 16777216.0 / (tq * 1.7320508075688772), Uq, stq);
        nearest_strip<LAT>(Uq, sq, cq, cbq);
        const uint32_t bits = 4u + (uint32_t)(N / LAT) * (Lat<LAT>::kCosetBits > 0 ? 1u : 0u) +
                              rice_best<G, N>(sq, stq, bkq, pq);
        return (group_or<G>(stq) & HQ_ST_OVERFLOW) == 0u && bits <= a.rc_budget;
      };
      const int32_t ac = (int32_t)(__float_as_uint(delta) >> 16);
      int32_t lo = ac - kRcSpan > 0x0080 ? ac - kRcSpan : 0x0080;
      int32_t hi = ac + kRcSpan < 0x7F7F ? ac + kRcSpan : 0x7F7F;
      // probe hi first (infeasible: the tile takes hi), then the midpoints
      // (one call site, so the search inlines)
      int32_t probe = hi;
      for (bool top = true;; top = false) {
        const bool f = feasible((uint32_t)probe);
        if (top && !f) break;
        if (!top) (f ? hi : lo) = probe;
        if (hi - lo <= 1) break;
        probe = (lo + hi) / 2;
      }
      delta = __uint_as_float((uint32_t)hi << 16);
    }
  }
  const double t = a.sqrt_n * (double)delta;
  const double K = 16777216.0 / t;
  const double K3 = 16777216.0 / (t * 1.7320508075688772);

  // ---- quantizer input on the 2^-24 grid
  GI U[16];
  grid_values<LAT>(v, K, K3, U, st);

  if constexpr (DITHER && !WIDE) {
    // d = w - Q_E8(w), w = 2^-23 h - 1 with h the top 24 bits of the hash
    const uint64_t vec = (uint64_t)(a.dither_base + tile);
    int32_t W[16], Z[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint64_t j = (uint64_t)(r * kElemsPerLane + i);
      const uint64_t key = ((uint64_t)a.dither_seed << 40) ^ ((vec << 8) | j);
      const int32_t h = (int32_t)(splitmix64(key) >> 40);
      W[i] = 2 * h - kOne;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int cw = e8_nearest(&W[8 * blk], Z);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        U[8 * blk + i] += W[8 * blk + i] - (shl24(Z[i]) + (cw ? kHalf : 0));
    }
  }

  // ---- nearest point, strip, coordinates; int8 indices and the Rice parameter
  int32_t s[16];
  int16_t crd[16];
  uint32_t cbits;
  nearest_strip<LAT>(U, s, crd, cbits);
  int bk;
  uint32_t best;
  if constexpr (WIDE) {
    uint32_t packed[8];
    best = rice_best16<G, N>(s, st, bk, packed);
    uint4* ip = reinterpret_cast<uint4*>(reinterpret_cast<int16_t*>(a.idx) + e0);
    ip[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    ip[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  } else {
    uint32_t packed[4];
    best = rice_best<G, N>(s, st, bk, packed);
    *reinterpret_cast<uint4*>(a.idx + e0) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  if (a.coords != nullptr) {
    uint32_t cw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cw[i] = ((uint32_t)(uint16_t)crd[2 * i]) | ((uint32_t)(uint16_t)crd[2 * i + 1] << 16);
    uint4* cp = reinterpret_cast<uint4*>(a.coords + e0);
    cp[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    cp[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
  }

  // ---- coset words: lane r owns bits [r B, r B + B) of the tile's bit row
  constexpr int kCB = Lat<LAT>::kCosetBits;
  if constexpr (kCB > 0) {
    constexpr int kLanesPerWord = (32 / kCB < G) ? 32 / kCB : G;
    uint32_t word = cbits << ((r * kCB) & 31);
    word = group_or<kLanesPerWord>(word);
    if ((r % kLanesPerWord) == 0) {
      constexpr int kWords = (N / LAT + 31) / 32;
      a.coset[tile * kWords + (r * kCB) / 32] = word;
    }
  }
  st = group_or<G>(st);
  if (r == 0) {
    if (a.auto_scale) a.scale[tile] = delta;
    a.rice_k[tile] = (uint8_t)bk;
    a.tile_bits[tile] = 4u + (uint32_t)(N / LAT) * (kCB > 0 ? 1u : 0u) + best;
    if (st) set_status(a.status, st);
  }
}

template <int LAT, int N>
hipError_t launch_lat_n(const EncodeLaunch& a, hipStream_t s) {
  constexpr int TPB = kBlock / (N / kElemsPerLane);
  const int64_t blocks = (a.n_tiles + TPB - 1) / TPB;
  dim3 grid((unsigned)blocks), block(kBlock);
  if (a.wide) {
    if (a.dither || a.rate_control) return hipErrorInvalidValue;
    if (a.in_bf16)
      hipLaunchKernelGGL((encode_kernel<LAT, N, true, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((encode_kernel<LAT, N, false, false, true>), grid, block, 0, s, a);
  } else if (a.dither) {
    if constexpr (LAT != 8) {
      return hipErrorInvalidValue;
    } else {
      if (a.in_bf16)
        hipLaunchKernelGGL((encode_kernel<LAT, N, true, true, false>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((encode_kernel<LAT, N, false, true, false>), grid, block, 0, s, a);
    }
  } else {
    if (a.in_bf16)
      hipLaunchKernelGGL((encode_kernel<LAT, N, true, false, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((encode_kernel<LAT, N, false, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int LAT>
hipError_t launch_lat(const EncodeLaunch& a, hipStream_t s) {
  switch (a.tile) {
    case 64: return launch_lat_n<LAT, 64>(a, s);
    case 128: return launch_lat_n<LAT, 128>(a, s);
    case 256: return launch_lat_n<LAT, 256>(a, s);
    default: return launch_lat_n<LAT, 512>(a, s);
  }
}

}  // namespace

hipError_t launch_encode(const EncodeLaunch& a, hipStream_t s) {
  // (the fast E8 kernel also runs the per-tile rate control)
  if (e8_fast_encode_ok(a)) {
    EncBatch b;
    b.n = 1;
    b.pad = 0;
    b.n_groups = (a.n_tiles + 15) / 16;
    b.it[0] = EncItem{a.x, a.idx, a.scale, a.coset, a.rice_k, a.tile_bits, a.n_tiles, 0};
    for (int i = 1; i < kMaxItems; ++i) b.it[i] = b.it[0];
    return launch_encode_e8_fast(a, b, s);
  }
  if (!a.rate_control && fast128_encode_ok(a)) return launch_encode_fast128(a, s);
  switch (a.lattice) {
    case 8: return launch_lat<8>(a, s);
    case 4: return launch_lat<4>(a, s);
    case 2: return launch_lat<2>(a, s);
    default: return launch_lat<1>(a, s);
  }
}

}  // namespace hq

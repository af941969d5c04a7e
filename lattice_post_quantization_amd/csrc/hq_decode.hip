// Decode kernels: stripped indices + coset bits + scale -> lattice point ->
// inverse Walsh-Hadamard -> signs -> fp32 / bf16 weights.
//
// Passages: [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice
// Quantization Pipeline ..." (decoding is algebraic: no codebook; subtractive
// dither removed on decode); [arXiv abstract] "HyperQuant: A
// Rate-Distortion-Optimal Quantization Pipeline ..." ideas (i)-(iii).
//
// Same work mapping as the encoder: G = N/16 lanes per tile, 16 contiguous
// elements per lane.  yhat = Delta * p is exact in fp64 (p has at most a few
// significant bits beyond Delta's 8), as is the Hadamard sum, so the only
// rounding is the final 1/sqrt(n) product (exact for n = 256) and the store.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

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

__device__ inline uint32_t lane_sign_mask(const DecodeLaunch& a, int r) {
  const int w = r >> 1;
  uint32_t s = a.signs[0];
#pragma unroll
  for (int k = 1; k < kMaxTile / 32; ++k) s = (w == k) ? a.signs[k] : s;
  return (s >> (16 * (r & 1))) & 0xFFFFu;
}

// WIDE: the int16 index mode (idx holds int16 values; no dither).
template <int LAT, int N, bool OUT_BF16, bool DITHER, bool WIDE>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeLaunch a) {
  constexpr int G = N / kElemsPerLane;
  constexpr int TPB = kBlock / G;
  const int r = threadIdx.x % G;
  const int64_t tile = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
  if (tile >= a.n_tiles) return;
  const int64_t e0 = tile * N + (int64_t)r * kElemsPerLane;

  int32_t s[16];
  if constexpr (WIDE) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const int16_t*>(a.idx) + e0);
    const uint4 q0 = p[0], q1 = p[1];
    const uint32_t qw[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (int32_t)(int16_t)(qw[i >> 1] >> (16 * (i & 1)));
  } else {
    const uint4 q = *reinterpret_cast<const uint4*>(a.idx + e0);
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (int32_t)(int8_t)(qw[i >> 2] >> (8 * (i & 3)));
  }
  const double delta = (double)a.scale[tile];

  // coset bits of this lane's blocks (E8: 2 per lane, A2: 8 per lane)
  uint32_t cb = 0;
  if constexpr (LAT == 8 || LAT == 2) {
    constexpr int kCB = 16 / LAT;
    constexpr int kWords = (N / LAT + 31) / 32;
    const uint32_t w = a.coset[tile * kWords + (r * kCB) / 32];
    cb = (w >> ((r * kCB) & 31)) & ((1u << kCB) - 1u);
  }

  // ---- lattice point, scaled: yhat = Delta * p  (KV: Delta * (p - d))
  double v[16];
  if constexpr (LAT == 8) {
    int32_t P[16];   // 2p
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int c = (cb >> blk) & 1;
      int32_t par = 0;
#pragma unroll
      for (int i = 0; i < 7; ++i) par += s[8 * blk + i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int32_t z = (i == 7) ? 2 * s[8 * blk + 7] + (par & 1) : s[8 * blk + i];
        P[8 * blk + i] = 2 * z + c;
      }
    }
    if constexpr (DITHER) {
      const uint64_t vec = (uint64_t)(a.dither_base + tile);
      int32_t W[16], Z[8];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint64_t j = (uint64_t)(r * kElemsPerLane + i);
        const uint64_t key = ((uint64_t)a.dither_seed << 40) ^ ((vec << 8) | j);
        W[i] = 2 * (int32_t)(splitmix64(key) >> 40) - kOne;
      }
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int cw = e8_nearest(&W[8 * blk], Z);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // (p - d) 2^24 = P 2^23 - (W - point(w) 2^24), exact in fp64
          const int32_t d24 = W[8 * blk + i] - (shl24(Z[i]) + (cw ? kHalf : 0));
          const double pd = (double)P[8 * blk + i] * 8388608.0 - (double)d24;
          v[8 * blk + i] = delta * (pd * 5.9604644775390625e-08);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = delta * (0.5 * (double)P[i]);
    }
  } else if constexpr (LAT == 4) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int32_t par = s[4 * blk] + s[4 * blk + 1] + s[4 * blk + 2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t z = (i == 3) ? 2 * s[4 * blk + 3] + (par & 1) : s[4 * blk + i];
        v[4 * blk + i] = delta * (double)z;
      }
    }
  } else if constexpr (LAT == 2) {
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      const double h = 0.5 * (double)((cb >> pr) & 1);
      v[2 * pr] = delta * ((double)s[2 * pr] + h);
      v[2 * pr + 1] = delta * (1.7320508075688772 * ((double)s[2 * pr + 1] + h));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = delta * (double)s[i];
  }

  fwht16<G>(v, r);

  const uint32_t smask = lane_sign_mask(a, r);
  if constexpr (OUT_BF16) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double x0 = v[2 * i] * a.inv_sqrt_n, x1 = v[2 * i + 1] * a.inv_sqrt_n;
      if ((smask >> (2 * i)) & 1u) x0 = -x0;
      if ((smask >> (2 * i + 1)) & 1u) x1 = -x1;
      o[i] = f64_to_bf16(x0) | (f64_to_bf16(x1) << 16);
    }
    uint4* y = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.y) + e0);
    y[0] = make_uint4(o[0], o[1], o[2], o[3]);
    y[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    float o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double x = v[i] * a.inv_sqrt_n;
      if ((smask >> i) & 1u) x = -x;
      o[i] = (float)x;
    }
    float4* y = reinterpret_cast<float4*>(static_cast<float*>(a.y) + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}

template <int LAT, int N>
hipError_t launch_lat_n(const DecodeLaunch& a, hipStream_t s) {
  constexpr int TPB = kBlock / (N / kElemsPerLane);
  const int64_t blocks = (a.n_tiles + TPB - 1) / TPB;
  dim3 grid((unsigned)blocks), block(kBlock);
  if (a.wide) {
    if (a.dither) return hipErrorInvalidValue;
    if (a.out_bf16)
      hipLaunchKernelGGL((decode_kernel<LAT, N, true, false, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<LAT, N, false, false, true>), grid, block, 0, s, a);
  } else if (a.dither) {
    if constexpr (LAT != 8) {
      return hipErrorInvalidValue;
    } else {
      if (a.out_bf16)
        hipLaunchKernelGGL((decode_kernel<LAT, N, true, true, false>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_kernel<LAT, N, false, true, false>), grid, block, 0, s, a);
    }
  } else {
    if (a.out_bf16)
      hipLaunchKernelGGL((decode_kernel<LAT, N, true, false, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<LAT, N, false, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <int LAT>
hipError_t launch_lat(const DecodeLaunch& a, hipStream_t s) {
  switch (a.tile) {
    case 64: return launch_lat_n<LAT, 64>(a, s);
    case 128: return launch_lat_n<LAT, 128>(a, s);
    case 256: return launch_lat_n<LAT, 256>(a, s);
    default: return launch_lat_n<LAT, 512>(a, s);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t s) {
  if (e8_fast_decode_ok(a)) {
    DecBatch b;
    b.n = 1;
    b.pad = 0;
    b.n_groups = (a.n_tiles + 15) / 16;
    b.it[0] = DecItem{a.idx, a.coset, a.scale, a.y, a.n_tiles, 0};
    for (int i = 1; i < kMaxItems; ++i) b.it[i] = b.it[0];
    return launch_decode_e8_fast(a, b, s);
  }
  if (fast128_decode_ok(a)) return launch_decode_fast128(a, s);
  switch (a.lattice) {
    case 8: return launch_lat<8>(a, s);
    case 4: return launch_lat<4>(a, s);
    case 2: return launch_lat<2>(a, s);
    default: return launch_lat<1>(a, s);
  }
}

}  // namespace hq

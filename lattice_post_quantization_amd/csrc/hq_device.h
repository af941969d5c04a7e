// Device building blocks for the HyperQuant hot path on gfx950.
//
// Sources (web pages, cited by title):
//   [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal Quantization
//       Pipeline for Large Language and Diffusion Models" (arXiv abstract on
//       mlsanity.com), ideas (i)-(iv);
//   [ICLR abstract]  "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
//       Pipeline for Large Language and Diffusion Models" (acceptodds.com).
//
// Numerics.  The quantizer input u = y / Delta is formed as
// U = rne(S * 2^24 / (sqrt(n) Delta)) with S the exact (fp64) Hadamard sum, and
// every lattice decision is then taken on the integer U (units of 2^-24).
// With all decisions exact, ties break by the stated rules on every device.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

constexpr int32_t kOne = 1 << 24;    // 1.0 in quantizer-grid units
constexpr int32_t kHalf = 1 << 23;   // 0.5
// |U| is clamped here (u = +-124); rne_grid below needs |U| + 2^25 < 2^31.
constexpr double kUClamp = 2080374784.0;   // 2^31 - 2^26
// The int16 index mode holds U in 64 bits and clamps at u = +-32000, where
// every index still fits int16.
constexpr double kUClamp16 = 536870912000.0;   // 32000 2^24

// rne(x K) of the exact product x K (one rounding, ties to even), as a
// double holding the integer: the fma adds 1.5 2^52 to the exact product and
// rounds once at unit spacing.  A product of magnitude >= 2^50, far past
// every clamp, is rounded twice; it clamps the same way.
constexpr double kGridMagic = 6755399441055744.0;   // 1.5 2^52
__device__ inline double rne_product(double x, double K) {
  const double p = __dmul_rn(x, K);
  if (!(fabs(p) < 0x1p50)) return rint(p);
  return __fma_rn(x, K, kGridMagic) - kGridMagic;
}

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) applied to a
// counter key: the randomness the method draws (RHT signs, KV dither).
__host__ __device__ inline uint64_t splitmix64(uint64_t k) {
  uint64_t z = k + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline int32_t shl24(int32_t a) {
  return (int32_t)((uint32_t)a << 24);
}

// a = rne(U / 2^24) (ties to even), R = U - a 2^24, |R| <= 2^23.  GI is the
// grid's integer type: int32_t, or int64_t in the int16 index mode (a fits
// int32 either way).
template <typename GI>
__device__ inline int32_t rne_grid(GI U, int32_t& R) {
  const GI t = U + 0x7FFFFF + ((U >> 24) & 1);
  const GI a = t >> 24;
  R = (int32_t)(U - (GI)((uint64_t)(int64_t)a << 24));
  return (int32_t)a;
}

__device__ inline int32_t iabs(int32_t v) { return v < 0 ? -v : v; }

// Nearest point of D_m (m = 4 or 8) to U / 2^24: round half to even; on an
// odd coordinate sum move the first coordinate of largest residual one step
// towards U (+1 on a zero residual).  Textbook rule (Conway & Sloane 1982).
template <int M, typename GI>
__device__ inline void d_round(const GI* U, int32_t* z) {
  int32_t R[M];
  int32_t sum = 0, amax = -1, j = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    z[i] = rne_grid(U[i], R[i]);
    sum += z[i];
    int32_t A = iabs(R[i]);
    if (A > amax) { amax = A; j = i; }
  }
  if (sum & 1) {
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (i == j) z[i] += (R[i] >= 0) ? 1 : -1;
  }
}

// Nearest E8 = D8 u (D8 + 1/2) point.  Returns the coset bit c; z is in D8 and
// the point is z + c/2.  The half coset's parity fix takes the last
// coordinate of largest residual (the integer coset's, as d_round, the first).  The coset comparison |u-a|^2 <= |u-b|^2 is evaluated
// exactly in closed form: with A_i = |u_i - rne(u_i)| and B_i = 1/2 - A_i,
//   (|u-a|^2 - |u-b|^2) / 2^24 = sum A - 2^25 + [odd a](2^24 - 2 max A)
//                                 - [odd b](2^24 - 2 max B)
// in grid units (a parity fix on coordinate j changes the squared distance by
// 1 - 2|residual_j|).  Ties keep the integer coset.
template <typename GI>
__device__ inline int e8_nearest(const GI* U, int32_t* z) {
  int32_t a[8], RA[8], b[8], RB[8];
  int32_t sa = 0, sb = 0, sumA = 0, amax = -1, amin = 0x7FFFFFFF, ja = 0, jb = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = rne_grid(U[i], RA[i]);
    b[i] = rne_grid(U[i] - kHalf, RB[i]);
    sa += a[i];
    sb += b[i];
    int32_t A = iabs(RA[i]);
    sumA += A;
    if (A > amax) { amax = A; ja = i; }
    if (A <= amin) { amin = A; jb = i; }  // max |RB| = 2^23 - min |RA|, last on ties
  }
  const bool odd_a = sa & 1, odd_b = sb & 1;
  const int32_t bmax = kHalf - amin;
  const int32_t D = sumA - (1 << 25) + (odd_a ? (1 << 24) - 2 * amax : 0) -
                    (odd_b ? (1 << 24) - 2 * bmax : 0);
  const int c = D > 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int32_t va = a[i] + ((odd_a && i == ja) ? ((RA[i] >= 0) ? 1 : -1) : 0);
    int32_t vb = b[i] + ((odd_b && i == jb) ? ((RB[i] >= 0) ? 1 : -1) : 0);
    z[i] = c ? vb : va;
  }
  return c;
}

// Nearest A2 point for one pair, given U1 = grid(u1) and V2 = grid(u2/sqrt3):
// integer coset (rne, rne) vs half coset (rne(. - 1/2) + 1/2) under the
// metric diag(1, 3); ties keep the integer coset.  Returns c; (a, b) are the
// integer parts, the point is (a + c/2, sqrt3 (b + c/2)).
template <typename GI>
__device__ inline int a2_nearest(GI U1, GI V2, int32_t& a, int32_t& b) {
  int32_t r1, r2, s1, s2;
  int32_t a0 = rne_grid(U1, r1), b0 = rne_grid(V2, r2);
  int32_t a1 = rne_grid(U1 - kHalf, s1), b1 = rne_grid(V2 - kHalf, s2);
  // |r|, |s| <= 2^23: squares <= 2^46, the sums are exact in fp64
  double d0 = (double)r1 * (double)r1 + 3.0 * ((double)r2 * (double)r2);
  double d1 = (double)s1 * (double)s1 + 3.0 * ((double)s2 * (double)s2);
  int c = d1 < d0;
  a = c ? a1 : a0;
  b = c ? b1 : b0;
  return c;
}

// ----------------------------------------------------------- conversions

__device__ inline float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// fp64 -> bf16 bits, round to nearest even directly from fp64 (no double
// rounding); results below the smallest normal bf16 flush to signed zero,
// overflow gives infinity.
__device__ inline uint32_t f64_to_bf16(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(b >> 63) << 15;
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull)
    return sign | (mag > 0x7FF0000000000000ull ? 0x7FC0u : 0x7F80u);
  uint64_t r = (mag + 0xFFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
  int32_t e = (int32_t)(r >> 7) - 1023 + 127;
  if (e >= 255) return sign | 0x7F80u;
  if (e <= 0) return sign;
  return sign | ((uint32_t)e << 7) | (uint32_t)(r & 0x7Fu);
}

// Scale rule: bf16_rne(x) as an fp32 value (x > 0 finite expected).
__device__ inline float bf16_round_to_f32(double x) {
  return __uint_as_float(f64_to_bf16(x) << 16);
}

__device__ inline uint32_t zigzag(int32_t z) {
  return ((uint32_t)z << 1) ^ (uint32_t)(z >> 31);
}

__device__ inline void set_status(uint32_t* status, uint32_t bits) {
  if (status != nullptr) atomicOr(status, bits);
}

}  // namespace hq

// Device building blocks shared by the fast kernels (E8 / tile 256 weights,
// E8 / tile 128 KV vectors): cross-row lane swaps, tile reductions, the sign
// table, the exact E8 block decision on the 2^-24 grid, bytewise Rice
// helpers, bounds-checked buffer stores, and the persistent-grid sizing.
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." ideas (i)-(iii); [ICLR abstract] "HyperQuant: A
// Near-Entropy-Optimal Lattice Quantization Pipeline ...".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace fastlib {

// 1.5 * 2^52: adding it to |q| < 2^51 rounds q to an integer (ties to even)
// that sits in the low mantissa bits.
constexpr double kMagic = 6755399441055744.0;

// Raw buffer over [base, base + bytes): the hardware drops stores whose
// offset falls outside and returns zeros for such loads, which replaces
// per-lane bounds branches around the memory operations of a ragged last
// group.  Offsets are 32-bit, so each buffer covers one group.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t out_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ inline lds_void* lds_ptr(uint4* p) { return (lds_void*)p; }

__device__ inline void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t a, uint32_t b,
                               uint32_t c, uint32_t d) {
  __builtin_amdgcn_raw_buffer_store_b128((u32x4){a, b, c, d}, r, (int)off, 0, 0);
}

// Tiles of a group that exist (the last group of a matrix may be short).
__device__ inline uint32_t live_tiles(int64_t n_tiles, int64_t group) {
  const int64_t n = n_tiles - group * 16;
  return (uint32_t)(n < 16 ? n : 16);
}

// Lanes of one wave exchange data through LDS.  LDS instructions of a wave
// execute in order, so no wait is needed; the fences (no instruction at
// wavefront scope) keep the compiler from moving or reusing LDS accesses
// across the exchange.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline void swap16(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

__device__ inline void swap32(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

template <bool ROW32>
__device__ inline void swap_f64(double& a, double& b) {
  uint64_t ua = (uint64_t)__double_as_longlong(a), ub = (uint64_t)__double_as_longlong(b);
  uint32_t alo = (uint32_t)ua, ahi = (uint32_t)(ua >> 32);
  uint32_t blo = (uint32_t)ub, bhi = (uint32_t)(ub >> 32);
  if (ROW32) {
    swap32(alo, blo);
    swap32(ahi, bhi);
  } else {
    swap16(alo, blo);
    swap16(ahi, bhi);
  }
  a = __longlong_as_double((long long)(((uint64_t)ahi << 32) | alo));
  b = __longlong_as_double((long long)(((uint64_t)bhi << 32) | blo));
}

// Sum / OR of a value over the four lanes (rows) that hold one tile.
__device__ inline uint32_t tile_sum_u32(uint32_t v) {
  uint32_t a = v, b = v;
  swap16(a, b);
  v = a + b;
  a = v;
  b = v;
  swap32(a, b);
  return a + b;
}

__device__ inline uint32_t tile_or_u32(uint32_t v) {
  uint32_t a = v, b = v;
  swap16(a, b);
  v = a | b;
  a = v;
  b = v;
  swap32(a, b);
  return a | b;
}

__device__ inline double tile_sum_f64(double v) {
  double a = v, b = v;
  swap_f64<false>(a, b);
  v = a + b;
  a = v;
  b = v;
  swap_f64<true>(a, b);
  return a + b;
}

// Sign table: for row r and element pair p (elements 64 r + 2p, 64 r + 2p + 1)
// the bf16-pair XOR mask (bit 15: first element, bit 31: second).
__device__ inline void fill_sign_table(uint32_t* tab, const uint32_t* signs) {
  for (int i = threadIdx.x; i < 128; i += kBlock) {
    const int e = 2 * i;   // row r = i / 32, pair p = i % 32 -> element 64 r + 2 p = 2 i
    uint32_t w0 = signs[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) w0 = ((e >> 5) == k) ? signs[k] : w0;
    const uint32_t b0 = (w0 >> (e & 31)) & 1u, b1 = (w0 >> ((e + 1) & 31)) & 1u;
    tab[i] = (b0 << 15) | (b1 << 31);
  }
}

// ------------------------------------------------------------------ E8 block
// Nearest E8 point for one block of grid values U (units of 2^-24), exact.
// Fast path: with F_i = U_i mod 2^24, I_i = floor(U_i / 2^24), B_i = |F_i - 2^23|
// (distance to the nearest half-integer; the distance to the nearest integer
// is 2^23 - B_i), and no coordinate exactly on an integer or half-integer:
//   integer coset a_i = I_i + [F_i > 2^23], half coset b_i = I_i (+ 1/2),
//   parity fixes on the first min of B (coset a) and the last max of B
//   (coset b), coset choice by
//   D = 2^25 - sum B + [odd a] 2 min B - [odd b] (2^24 - 2 max B) > 0.
// Bit 24 of U_i is the parity of I_i and bit 23 is [F_i > 2^23], so both
// parities come from the XOR of the eight U_i.  The stored integers are
// built as bytes: the top byte of U_i is I_i; coset a adds the bit-23 bits
// and the parity flip adds +/-1 to one byte.  The bytes carry a bias of 128
// while they are added to, so no byte carries into the next (a tile without
// the overflow flag has |u_i| < 126, keeping every biased byte in 0..255).
// The last coordinate is stored halved, from U_7 + [coset a] 2^23 with its
// flip applied before halving.
// Blocks with a coordinate on an integer or half-integer need the general
// decoder (rare; same results): e8_block_fast then returns 1 and its other
// results are meaningless, and e8_block_exact gives the answer.  Both write
// the stored integers (z0..z6, floor(z7/2)) as two dwords of int8 and the
// coset bit.  The fast decision has no branch, so the blocks of a lane can
// be scheduled together and the rare search runs once, after all of them.
__device__ inline uint32_t sad_u32(uint32_t a, uint32_t b) {
  uint32_t r;
  __asm__("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// |a - 2^26| + C (C an inline constant)
template <int C>
__device__ inline uint32_t sad26(uint32_t a) {
  uint32_t r;
  __asm__("v_sad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(1u << 26), "i"(C));
  return r;
}

__device__ inline uint32_t min3u(uint32_t a, uint32_t b, uint32_t c) {
  const uint32_t m = a < b ? a : b;
  return m < c ? m : c;
}
__device__ inline uint32_t max3u(uint32_t a, uint32_t b, uint32_t c) {
  const uint32_t m = a > b ? a : b;
  return m > c ? m : c;
}

// top bytes of four dwords, in order, as one dword
__device__ inline uint32_t top_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0703u) | __builtin_amdgcn_perm(d, c, 0x07030C0Cu);
}

// byte 2 of four dwords, in order
__device__ inline uint32_t third_bytes(int32_t a, int32_t b, int32_t c, int32_t d) {
  return __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0C0C0602u) |
         __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x06020C0Cu);
}

__device__ inline uint32_t pack4(const int32_t* s);

// 8 (U mod 2^24): v_mul_u32_u24 reads only the low 24 bits of U
__device__ inline uint32_t frac8(int32_t u) {
  uint32_t r;
  __asm__("v_mul_u32_u24 %0, 8, %1" : "=v"(r) : "v"(u));
  return r;
}

__device__ inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  __asm__("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// per 16-bit half: a * b + c (mod 2^16)
__device__ inline uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  __asm__("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline uint32_t pk_add_u16(uint32_t a, uint32_t b) {
  uint32_t r;
  __asm__("v_pk_add_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ inline uint32_t e8_block_fast(const int32_t* U, uint32_t& p0, uint32_t& p1, int& cs) {
  // keys (B << 3) + i = |8F - 2^26| plus the index: their minimum is the
  // integer coset's parity coordinate (smallest B, first on ties), their
  // maximum the half coset's (largest B, last on ties)
  uint32_t k1[8];
#define HQ_E8_KEYS(i)                                             \
  {                                                               \
    const uint32_t F8 = frac8(U[i]);                              \
    k1[i] = sad26<i>(F8);                                         \
  }
  HQ_E8_KEYS(0) HQ_E8_KEYS(1) HQ_E8_KEYS(2) HQ_E8_KEYS(3)
  HQ_E8_KEYS(4) HQ_E8_KEYS(5) HQ_E8_KEYS(6) HQ_E8_KEYS(7)
#undef HQ_E8_KEYS
  const uint32_t kmin = min3u(min3u(k1[0], k1[1], k1[2]), min3u(k1[3], k1[4], k1[5]),
                              k1[6] < k1[7] ? k1[6] : k1[7]);
  const uint32_t kmax = max3u(max3u(k1[0], k1[1], k1[2]), max3u(k1[3], k1[4], k1[5]),
                              k1[6] > k1[7] ? k1[6] : k1[7]);
  // min B = 0 or max B = 2^23: a coordinate on a half-integer or an integer
  const uint32_t tie = (uint32_t)(kmin < 8u) | (uint32_t)(kmax >= (1u << 26));
  // 8 sum B = sum k1 - 28
  const uint32_t sumk = (k1[0] + k1[1] + k1[2]) + (k1[3] + k1[4] + k1[5]) + (k1[6] + k1[7]);
  const uint32_t X = xor3(xor3((uint32_t)U[0], (uint32_t)U[1], (uint32_t)U[2]),
                          xor3((uint32_t)U[3], (uint32_t)U[4], (uint32_t)U[5]),
                          (uint32_t)U[6] ^ (uint32_t)U[7]);
  const int odd_b = (int)((X >> 24) & 1u);                 // sum I odd
  const int odd_a = (int)(((X >> 23) ^ (X >> 24)) & 1u);   // sum (I + up) odd
  // 8 D = 2^28 - 8 sum B + [odd a] 16 min B - [odd b] (2^27 - 16 max B)
  const int32_t D8 = (int32_t)((1u << 28) + 28u - sumk) +
                     (odd_a ? 2 * (int32_t)(kmin & ~7u) : 0) -
                     (odd_b ? (1 << 27) - 2 * (int32_t)(kmax & ~7u) : 0);
  const int c = D8 > 0;
  const uint32_t jf = c ? (kmax & 7u) : (kmin & 7u);
  const int odd = c ? odd_b : odd_a;
  // Q: the high halves (U >> 16) of two coordinates; byte 1 of a half is I,
  // bit 7 of byte 0 is [F > 2^23]
  const uint32_t Q0 = __builtin_amdgcn_perm((uint32_t)U[1], (uint32_t)U[0], 0x07060302u);
  const uint32_t Q1 = __builtin_amdgcn_perm((uint32_t)U[3], (uint32_t)U[2], 0x07060302u);
  const uint32_t Q2 = __builtin_amdgcn_perm((uint32_t)U[5], (uint32_t)U[4], 0x07060302u);
  const uint32_t Q3 = __builtin_amdgcn_perm((uint32_t)U[7], (uint32_t)U[6], 0x07060302u);
  // byte k of Gq: byte 2 of U_{4q+k}
  const uint32_t G0 = __builtin_amdgcn_perm(Q1, Q0, 0x06040200u);
  const uint32_t G1 = __builtin_amdgcn_perm(Q3, Q2, 0x06040200u);
  const uint32_t upj = (uint32_t)((((uint64_t)G1 << 32) | G0) >> (8 * jf + 7)) & 1u;
  // Adding 0x80 to a half carries [F > 2^23] into its high byte (the
  // integer coset's rounding); 0x8000 adds the bias of 128 to the byte, so
  // the parity flip below cannot carry into a neighbour (a tile without the
  // overflow flag has |u_i| < 126, so every biased byte stays in 1..255).
  const uint32_t cadd = c ? 0x80008000u : 0x80808080u;
  const uint32_t b0 = __builtin_amdgcn_perm(pk_add_u16(Q1, cadd), pk_add_u16(Q0, cadd), 0x07050301u);
  const uint32_t b1 = __builtin_amdgcn_perm(pk_add_u16(Q3, cadd), pk_add_u16(Q2, cadd), 0x07050301u);
  // The flipped coordinate moves away from u's rounding in coset a (-1 when
  // rounded up) and towards u in coset b (+1 when u lies above the
  // half-integer).
  // +-1 at byte jf of the 8 biased bytes: one 64-bit shift-and-add of the
  // sign-extended step (no biased byte is 0, so a -1 borrows nothing)
  const int32_t step = odd ? (((uint32_t)c ^ upj) ? -1 : 1) : 0;
  const uint64_t bb = ((((uint64_t)b1 << 32) | b0) + ((uint64_t)(int64_t)step << (8u * jf)));
  constexpr uint32_t kBias = 0x80808080u;
  p0 = (uint32_t)bb ^ kBias;
  const uint32_t q1 = (uint32_t)(bb >> 32) ^ kBias;
  // the last coordinate is stored halved: floor(z7 / 2)
  p1 = __builtin_amdgcn_perm((uint32_t)((int32_t)q1 >> 25), q1, 0x04020100u);
  cs = c;
  return tie;
}

__device__ inline uint32_t pack4(const int32_t* s) {
  return ((uint32_t)s[0] & 0xFFu) | (((uint32_t)s[1] & 0xFFu) << 8) |
         (((uint32_t)s[2] & 0xFFu) << 16) | ((uint32_t)s[3] << 24);
}

__device__ inline int e8_block_exact(const int32_t* U, uint32_t& p0, uint32_t& p1) {
  int32_t z[8];
  const int c = e8_nearest(U, z);
  z[7] >>= 1;
  p0 = pack4(z);
  p1 = pack4(z + 4);
  return c;
}

// zigzag of four int8 values held in a dword, bytewise: 2z, or its
// complement for negative z.  v_perm selectors 8-11 replicate the sign bits
// of bytes 1, 3, 5, 7 of {d << 8, d}, i.e. of bytes 1, 3, 0, 2 of d.
__device__ inline uint32_t zigzag4(uint32_t d) {
  const uint32_t neg = __builtin_amdgcn_perm(d << 8, d, 0x090B080Au);
  return ((d << 1) & 0xFEFEFEFEu) ^ neg;
}

__device__ inline uint32_t byte_sum(uint32_t d, uint32_t acc) {
  return __builtin_amdgcn_sad_u8(d, 0u, acc);
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

__device__ inline s16x2 as_s16x2(uint32_t u) { return __builtin_bit_cast(s16x2, u); }
__device__ inline uint32_t as_u32(s16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// in-dword butterfly: (lo, hi) -> (lo + hi, lo - hi)
__device__ inline uint32_t half_butterfly(uint32_t x) {
  const s16x2 p = as_s16x2(x);
  const s16x2 hh = __builtin_shufflevector(p, p, 1, 1);
  const s16x2 ll = __builtin_shufflevector(p, p, 0, 0);
  return as_u32(hh * (s16x2){1, -1} + ll);
}

// Item holding global group g (items are few; the index is wave-uniform).
template <typename B>
__device__ inline int item_of(const B& b, int64_t g) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kMaxItems; ++k)
    if (k < b.n && g >= b.it[k].group0) i = k;
  return i;
}

// Item holding global group g, found from item i, which holds an earlier
// group of the same walk (groups are visited in increasing order, so the
// item only moves forward; usually one comparison).
template <typename B>
__device__ inline int item_from(const B& b, int i, int64_t g) {
  while (i + 1 < b.n && g >= b.it[i + 1].group0) ++i;
  return i;
}

inline int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Resident blocks of a kernel on the whole device (persistent grid size).
template <typename K>
inline int64_t resident_blocks(K kernel, int& cache) {
  if (cache == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    cache = per_cu;
  }
  return (int64_t)cache * device_cus();
}

inline int64_t persistent_grid(int64_t n_tiles, int64_t resident, int64_t tiles_per_group = 16) {
  const int64_t groups = (n_tiles + tiles_per_group - 1) / tiles_per_group;
  const int64_t blocks = (groups + kBlock / 64 - 1) / (kBlock / 64);
  return blocks < resident ? blocks : resident;
}


}  // namespace fastlib
}  // namespace hq

// Rice rate accounting and packing of stripped indices.
//
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." idea (iii) (near-entropy-optimal Rice coding of
// the lattice indices); [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal
// Lattice Quantization Pipeline ..." (Rice code, one itemized rate
// accounting); GitHub issue "HyperQuant ... #9", "Additional context" (a
// packed, Rice-coded lattice-index checkpoint format).
//
// Three kernels, each wave owning a contiguous span of tiles (the rate and
// pack kernels use the same partition; with the encoder's rice_k and
// tile_bits given, a rate kernel that reads only tile_bits replaces the
// first):
//   rate_kernel  per tile (16 indices per lane): zigzag bytewise, k from
//                byte sums over three candidates, tile_bits; per wave the
//                sum of ceil(tile_bits/32), per block the sums of
//                ceil(tile_bits/32) and of tile_bits, into the workspace
//                (without a workspace, the bit total is accumulated with one
//                64-bit atomic per block instead).
//   scan_kernel  one block: exclusive prefix sum of the per-block word sums,
//                and the total of the per-block bit sums.
//   pack_kernel  per tile: each lane's payload length from byte sums, an
//                exclusive scan over the tile's lanes gives its first bit;
//                the lane then writes its 16 codes into the wave's LDS copy
//                of the tile with OR operations, and the tile's lanes store
//                its words at the tile's word offset.  Tiles are word
//                aligned, so no two tiles share a word.  Only wave-level
//                synchronisation: waves never wait for each other.
#include <string.h>

#include "hq.h"
#include "hq_device.h"
#include "hq_ratebatch.h"
#include "hq_internal.h"

namespace hq {
namespace {

// The G lanes of a tile (G = 4, 8, 16 or 32) are aligned lane groups: for
// G <= 16 within one 16-lane DPP row, for G = 32 two neighbouring rows, so
// sums and scans over them use DPP moves (VALU, no LDS round trip).
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}

template <int G>
__device__ inline uint32_t row_sum(uint32_t x) {
  x += dpp<0xB1>(x);                    // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                    // quad_perm [2,3,0,1]
  if (G >= 8) x += dpp<0x141>(x);       // row_half_mirror: the other quad of the half row
  if (G >= 16) x += dpp<0x140>(x);      // row_mirror: the other half row
  if (G == 32) x += __shfl_xor(x, 16);  // the other row of the pair
  return x;
}

// Inclusive scan over the G lanes of a group (lane r of the group).
template <int G>
__device__ inline uint32_t row_incl_scan(uint32_t x, int r) {
  uint32_t v = dpp<0x111>(x);           // row_shr:1
  x += r >= 1 ? v : 0u;
  v = dpp<0x112>(x);                    // row_shr:2
  x += r >= 2 ? v : 0u;
  if (G >= 8) {
    v = dpp<0x114>(x);                  // row_shr:4
    x += r >= 4 ? v : 0u;
  }
  if (G >= 16) {
    v = dpp<0x118>(x);                  // row_shr:8
    x += r >= 8 ? v : 0u;
  }
  if (G == 32) {
    v = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += r >= 16 ? v : 0u;
  }
  return x;
}

// Zigzag of four int8 values held in a dword, bytewise: 2z, or its
// complement for negative z (v_perm selectors 8-11 replicate the sign bits of
// bytes 1, 3, 5, 7 of {d << 8, d}, i.e. of bytes 1, 3, 0, 2 of d).
__device__ inline uint32_t zigzag4(uint32_t d) {
  return ((d << 1) & 0xFEFEFEFEu) ^ __builtin_amdgcn_perm(d << 8, d, 0x090B080Au);
}

__device__ inline uint32_t byte_sum(uint32_t d, uint32_t acc) {
  return __builtin_amdgcn_sad_u8(d, 0u, acc);
}

// This lane's 16 zigzagged indices of a tile as 4 dwords of bytes.
__device__ inline void zeta4(const uint4 q, uint32_t* zz) {
  zz[0] = zigzag4(q.x);
  zz[1] = zigzag4(q.y);
  zz[2] = zigzag4(q.z);
  zz[3] = zigzag4(q.w);
}

__device__ inline uint4 load16(const int8_t* idx, int64_t e0) {
  return *reinterpret_cast<const uint4*>(idx + e0);
}

// A lane's 16 indices: 16 bytes (int8) or 32 bytes (int16 index mode).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool WIDE>
struct LaneIdx {
  uint4 q[WIDE ? 2 : 1];
};

template <bool WIDE>
__device__ inline LaneIdx<WIDE> load_lane(const int8_t* idx, int64_t e0) {
  LaneIdx<WIDE> v;
  if constexpr (WIDE) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const int16_t*>(idx) + e0);
    v.q[0] = p[0];
    v.q[1] = p[1];
  } else {
    v.q[0] = load16(idx, e0);
  }
  return v;
}

// Zigzag of the 16 int16 values of a lane, one per dword.
__device__ inline void zeta16(const LaneIdx<true>& v, uint32_t* zz) {
  const uint32_t w[8] = {v.q[0].x, v.q[0].y, v.q[0].z, v.q[0].w,
                         v.q[1].x, v.q[1].y, v.q[1].z, v.q[1].w};
#pragma unroll
  for (int i = 0; i < 16; ++i) zz[i] = zigzag((int32_t)(int16_t)(w[i >> 1] >> (16 * (i & 1))));
}

// k = argmin_k L(k), L(k) = sum floor(zeta / 2^k) + N (1 + k), first minimum.
// L is convex in k: L(k+1) - L(k) = N - D_k with D_k = sum floor((zeta + 2^k)
// / 2^(k+1)) non-increasing in k and within N/2 of S / 2^(k+1), S = sum zeta.
// With kt the smallest k with S <= N 2^(k+1), D_{kt+1} <= N and D_k > N for
// k <= kt - 2, so the first minimum is one of kt - 1, kt, kt + 1 (zeta <= 255
// keeps kt <= 7).  Sums over the tile's G lanes; returns the payload bits.
template <int G, int N>
__device__ inline uint32_t best_k(const uint32_t* zz, int& bk) {
  uint32_t S = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) S = byte_sum(zz[j], S);
  S = row_sum<G>(S);
  int kt = 0;
  while (kt < 8 && S > ((uint32_t)N << (kt + 1))) ++kt;
  uint32_t best = 0xFFFFFFFFu;
  bk = 0;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int k = kt - 1 + c;
    k = k < 0 ? 0 : (k > 8 ? 8 : k);
    const uint32_t mask = ((1u << k) - 1u) * 0x01010101u;
    uint32_t R = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) R = byte_sum(zz[j] & mask, R);
    R = row_sum<G>(R);
    const uint32_t L = ((S - R) >> k) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

// The same for int16 indices (zeta < 2^16, one per dword; k in [0, 15]; for
// S > N 2^16 every candidate clamps to k = 15, where every zeta >> k is 0 or 1
// and D_15 <= N).
template <int G, int N>
__device__ inline uint32_t best_k16(const uint32_t* zz, int& bk) {
  uint32_t S = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) S += zz[i];
  S = row_sum<G>(S);
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
    R = row_sum<G>(R);
    const uint32_t L = ((S - R) >> k) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

// Waves of the rate and pack grids, and the tiles each covers: wave w owns
// [w span, (w + 1) span), span a multiple of the TPW = 64 / G tiles one pass
// of a wave handles.
constexpr int64_t kMaxRateWaves = 8192;

template <int N>
__host__ __device__ inline int64_t rate_waves(int64_t n_tiles) {
  constexpr int TPW = 64 / (N / kElemsPerLane);
  const int64_t passes = (n_tiles + TPW - 1) / TPW;
  return passes < kMaxRateWaves ? passes : kMaxRateWaves;
}

template <int N>
__device__ inline int64_t wave_span(int64_t n_tiles) {
  constexpr int TPW = 64 / (N / kElemsPerLane);
  const int64_t passes = (n_tiles + TPW - 1) / TPW;
  const int64_t waves = rate_waves<N>(n_tiles);
  return (passes + waves - 1) / waves * TPW;
}

__device__ inline uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// A wave's word and bit totals (summed over its lanes) into the workspace:
// its word count, and its block's word and bit sums (without a workspace,
// the bit total through one 64-bit atomic per block).  Every thread of the
// block calls it.
__device__ inline void rate_sums(const RateLaunch& a, int64_t bx, uint64_t words, uint64_t bits,
                                 int64_t wave, int wl, int lane,
                                 uint64_t (*blk)[kBlock / 64]) {
  words = wave_sum_u64(words);
  bits = wave_sum_u64(bits);
  if (lane == 0) {
    if (a.wave_words != nullptr) a.wave_words[wave] = words;
    blk[0][wl] = words;
    blk[1][wl] = bits;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t w = 0, b = 0;
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i) {
      w += blk[0][i];
      b += blk[1][i];
    }
    if (a.block_words != nullptr) {
      a.block_words[bx] = w;
      a.block_bits[bx] = b;
    } else {
      atomicAdd((unsigned long long*)a.total_bits, (unsigned long long)b);
    }
  }
}

// The block's matrix in the batch (block-uniform) and its block index there.
__device__ inline int rate_item(const RateBatch& b, int64_t& bx) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kRateMaxItems; ++k)
    if (k < b.n && (int64_t)blockIdx.x >= b.block0[k]) i = k;
  bx = (int64_t)blockIdx.x - b.block0[i];
  return i;
}

template <int N, bool WIDE>
__global__ __launch_bounds__(kBlock) void rate_kernel(RateBatch bt) {
  int64_t bx;
  const RateLaunch& a = bt.it[rate_item(bt, bx)];
  constexpr int G = N / kElemsPerLane;
  constexpr int TPW = 64 / G;
  __shared__ uint64_t blk[2][kBlock / 64];
  const int lane = threadIdx.x & 63;
  const int r = lane % G;
  const int wl = threadIdx.x >> 6;
  const int64_t wave = bx * (kBlock / 64) + wl;
  // waves past the last one have an empty span (the block still syncs)
  const int64_t span = wave_span<N>(a.n_tiles);
  const int64_t first = wave < rate_waves<N>(a.n_tiles) ? wave * span : a.n_tiles;
  const int64_t end = first + span < a.n_tiles ? first + span : a.n_tiles;
  uint64_t words = 0, bits = 0;
  // the next pass's indices are loaded while this pass is computed
  auto fetch = [&](int64_t t0) {
    const int64_t tile = t0 + lane / G;
    const int64_t tl = tile < end ? tile : end - 1;   // whole groups stay convergent
    return load_lane<WIDE>(a.idx, tl * N + (int64_t)r * kElemsPerLane);
  };
  LaneIdx<WIDE> nxt;
  if (first < end) nxt = fetch(first);
  for (int64_t t0 = first; t0 < end; t0 += TPW) {
    const int64_t tile = t0 + lane / G;
    const bool live = tile < end;
    int bk;
    uint32_t pay;
    if constexpr (WIDE) {
      uint32_t zz[16];
      zeta16(nxt, zz);
      if (t0 + TPW < end) nxt = fetch(t0 + TPW);
      pay = best_k16<G, N>(zz, bk);
    } else {
      uint32_t zz[4];
      zeta4(nxt.q[0], zz);
      if (t0 + TPW < end) nxt = fetch(t0 + TPW);
      pay = best_k<G, N>(zz, bk);
    }
    const uint32_t tb = 4u + (uint32_t)a.coset_bits + pay;
    if (live && r == 0) {
      a.rice_k[tile] = (uint8_t)bk;
      a.tile_bits[tile] = tb;
      words += (tb + 31u) / 32u;
      bits += tb;
    }
  }
  rate_sums(a, bx, words, bits, wave, wl, lane, blk);
}

// Rate pass with the encoder's rice_k and tile_bits given: the same spans
// and sums, from tile_bits alone (lanes stride over the wave's tiles).
template <int N>
__global__ __launch_bounds__(kBlock) void rate_given_kernel(RateBatch bt) {
  int64_t bx;
  const RateLaunch& a = bt.it[rate_item(bt, bx)];
  __shared__ uint64_t blk[2][kBlock / 64];
  const int lane = threadIdx.x & 63;
  const int wl = threadIdx.x >> 6;
  const int64_t wave = bx * (kBlock / 64) + wl;
  const int64_t span = wave_span<N>(a.n_tiles);
  const int64_t first = wave < rate_waves<N>(a.n_tiles) ? wave * span : a.n_tiles;
  const int64_t end = first + span < a.n_tiles ? first + span : a.n_tiles;
  uint64_t words = 0, bits = 0;
  for (int64_t t = first + lane; t < end; t += 64) {
    const uint32_t tb = a.tile_bits[t];
    words += (tb + 31u) / 32u;
    bits += tb;
  }
  rate_sums(a, bx, words, bits, wave, wl, lane, blk);
}

// total_bits = 0 for the matrices whose bit totals go through atomics
__global__ void zero_totals_kernel(RateBatch bt) {
  const int i = threadIdx.x;
  if (i < bt.n && bt.it[i].block_words == nullptr) *bt.it[i].total_bits = 0;
}

// Exclusive scan of the n <= kMaxRateWaves / 4 per-block word sums in place,
// and the total of the per-block bit sums; one block, kScanPer consecutive values
// per thread (all loads issued at once), wave scans by shuffles and a scan of
// the wave totals in LDS.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 2;
static_assert(kScanThreads * kScanPer >= kMaxRateWaves / (kBlock / 64), "scan covers every rate block");

// one block per matrix with a workspace
__global__ __launch_bounds__(kScanThreads) void scan_kernel(RateBatch bt) {
  const RateLaunch& a = bt.it[blockIdx.x];
  if (a.block_words == nullptr) return;     // the whole block
  uint64_t* v = a.block_words;
  const int64_t n = bt.block0[blockIdx.x + 1] - bt.block0[blockIdx.x];
  const uint64_t* bits = a.block_bits;
  uint64_t* total_bits = a.total_bits;
  __shared__ uint64_t wtot[kScanThreads / 64];
  __shared__ uint64_t btot[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint64_t x[kScanPer];
  uint64_t s = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int64_t j = (int64_t)t * kScanPer + i;
    x[i] = j < n ? v[j] : 0;
    sb += j < n ? bits[j] : 0;
    s += x[i];
  }
  // inclusive scan over the wave, then over the wave totals
  uint64_t inc = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = __shfl_up(inc, d);
    inc += lane >= d ? y : 0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) sb += __shfl_xor(sb, m);
  if (lane == 63) wtot[w] = inc;
  if (lane == 0) btot[w] = sb;
  __syncthreads();
  uint64_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kScanThreads / 64; ++i) {
    before += i < w ? wtot[i] : 0;
    total += btot[i];
  }
  if (t == 0) *total_bits = total;
  uint64_t run = before + inc - s;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int64_t j = (int64_t)t * kScanPer + i;
    if (j < n) v[j] = run;
    run += x[i];
  }
}

// Max words one tile can need: 4 + coset bits + 9 N (k = 8 bounds the
// optimum: every zeta >> 8 is 0); int16 indices: 17 N (k = 15, zeta >> 15 <= 1).
template <int N, bool WIDE>
struct PackBound {
  static constexpr int kMaxBits = 4 + N / 2 + (WIDE ? 17 : 9) * N;
  static constexpr int kWords = (kMaxBits + 31) / 32;
};

// Bit writer over a tile's LDS words.  acc holds stream bits from bit
// position 32 * wp on; an counts them.  Full words are OR-ed out (the first
// and last words of a lane's range are shared with its neighbours).
struct BitWriter {
  uint32_t* w;
  uint64_t acc;
  uint32_t an;
  uint32_t wp;

  // nbits <= 32 bits of v (higher bits zero); an < 32 on entry and exit
  __device__ inline void put(uint32_t v, uint32_t nbits) {
    acc |= (uint64_t)v << an;
    an += nbits;
    if (an >= 32u) {
      atomicOr(&w[wp], (uint32_t)acc);
      acc >>= 32;
      an -= 32u;
      ++wp;
    }
  }
  __device__ inline void flush() {
    if (an > 0u) atomicOr(&w[wp], (uint32_t)acc);
  }
};

// LDS words of one wave: its TPW tiles of at most W words each, plus a spare
// word past the last tile (the two-word OR of a code may touch it).
template <int N, bool WIDE>
constexpr int pack_lds_words() {
  return 64 / (N / kElemsPerLane) * PackBound<N, WIDE>::kWords + 1;
}

// The same rounded up to whole 16-byte stores of all 64 lanes (the wave
// clears its words with them).
template <int N, bool WIDE>
constexpr int pack_lds_zero_passes() {
  return (pack_lds_words<N, WIDE>() + 255) / 256;
}

// Passes whose loads are in flight ahead of the one being packed.
#ifndef HQ_PACK_AHEAD
#define HQ_PACK_AHEAD 3
#endif
constexpr int kPackAhead = HQ_PACK_AHEAD;

template <int N, bool WIDE>
__global__ __launch_bounds__(kBlock) void pack_kernel(RateBatch bt) {
  int64_t bx;
  const RateLaunch& a = bt.it[rate_item(bt, bx)];
  if (a.stream == nullptr) return;          // the whole block: not packing
  constexpr int G = N / kElemsPerLane;
  constexpr int TPW = 64 / G;
  constexpr int W = PackBound<N, WIDE>::kWords;
  constexpr uint32_t kMaxK = WIDE ? 15u : 8u;   // the largest optimal k
  constexpr int kZero = pack_lds_zero_passes<N, WIDE>();
  __shared__ uint4 lds[kBlock / 64][64 * kZero];
  const int lane = threadIdx.x & 63;
  const int r = lane % G;
  const int slot = lane / G;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // the wave in the block
  const int64_t wave = bx * (kBlock / 64) + wv;
  if (wave >= rate_waves<N>(a.n_tiles)) return;   // whole waves only
  uint4* buf4 = lds[wv];
  uint32_t* buf = reinterpret_cast<uint32_t*>(buf4);
  const int64_t span = wave_span<N>(a.n_tiles);
  const int64_t first = wave * span;
  const int64_t end = first + span < a.n_tiles ? first + span : a.n_tiles;
  // first word of this pass's tiles: the block's offset, then the words of
  // the block's earlier waves
  uint64_t base = a.block_words[bx];
  for (int i = 0; i < wv; ++i) base += a.wave_words[bx * (kBlock / 64) + i];
  struct PassIn {
    LaneIdx<WIDE> q;
    uint32_t k, tb, cw0;   // cw0: the tile's first coset word
  };
  // Buffers over the wave's own tiles: 32-bit offsets, and a load past
  // them reads zeros, so every pass issues the same loads whatever its
  // place (the compiler then keeps exact wait counts for the loads in
  // flight; the values of tiles past the wave's are never used).
  constexpr uint32_t kEsz = WIDE ? 2u : 1u;
  const uint32_t nt = end > first ? (uint32_t)(end - first) : 0u;
  const auto rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(a.idx) + first * N * (int64_t)kEsz, (short)0, (int)(nt * N * kEsz), 0x00020000);
  const auto rk = __builtin_amdgcn_make_buffer_rsrc(a.rice_k + first, (short)0, (int)nt, 0x00020000);
  const auto rt = __builtin_amdgcn_make_buffer_rsrc(a.tile_bits + first, (short)0, (int)(nt * 4u), 0x00020000);
  const uint32_t cwb = 4u * (uint32_t)a.coset_words;   // coset bytes per tile
  const auto rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.coset) + (a.coset_words > 0 ? first * a.coset_words : 0), (short)0,
      (int)(nt * cwb), 0x00020000);
  auto fetch = [&](int64_t t0, PassIn& in) {
    const uint32_t lt = (uint32_t)(t0 - first) + (uint32_t)slot;   // tile, from the wave's first
    const uint32_t qo = (lt * N + (uint32_t)r * kElemsPerLane) * kEsz;
#pragma unroll
    for (int h = 0; h < (WIDE ? 2 : 1); ++h) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(qo + 16u * h), 0, 0);
      in.q.q[h] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    in.k = __builtin_amdgcn_raw_buffer_load_b8(rk, (int)lt, 0, 0);
    in.tb = __builtin_amdgcn_raw_buffer_load_b32(rt, (int)(lt * 4u), 0, 0);
    in.cw0 = __builtin_amdgcn_raw_buffer_load_b32(rc, (int)(lt * cwb), 0, 0);
  };
  auto pass = [&](const PassIn& in, int64_t t0) {
    if (t0 >= end) return;   // wave-uniform
    const int64_t tile = t0 + slot;
    const bool live = tile < end;
    const uint32_t ck = in.k, tb = live ? in.tb : 0u;
    // (given tile_bits past the tile's LDS words are clamped there; the
    // codes of such a tile are not written, see below)
    const uint32_t nwords = (tb + 31u) / 32u < (uint32_t)W ? (tb + 31u) / 32u : (uint32_t)W;
    // word offsets of the pass's tiles: group g's count sits in lane g G
    uint64_t off = base, pass_words = 0;
#pragma unroll
    for (int g = 0; g < TPW; ++g) {
      const uint32_t ng = (uint32_t)__builtin_amdgcn_readlane((int)nwords, g * G);
      off += g < slot ? ng : 0u;
      pass_words += ng;
    }
    uint32_t* tw = buf + slot * W;
    // every word of the wave's tiles (and the spare word) starts at zero
#pragma unroll
    for (int z = 0; z < kZero; ++z) buf4[64 * z + lane] = make_uint4(0u, 0u, 0u, 0u);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // every lane runs the scan (DPP moves read neighbouring lanes)
    uint32_t k = 0;
    // zigzag values: four per dword (int8) or one per dword (int16)
    uint32_t zz[WIDE ? 16 : 4];
#pragma unroll
    for (int j = 0; j < (WIDE ? 16 : 4); ++j) zz[j] = 0u;
    if (live) {
      k = ck < kMaxK ? ck : kMaxK;   // (a given k above it marks the tile corrupt below)
      if constexpr (WIDE) zeta16(in.q, zz);
      else zeta4(in.q.q[0], zz);
    }
    // The lane's codes by group of four: q per code and the bit length of
    // each group (sum of q + 1 + k).  When every group of every lane of the
    // wave spans at most 32 bits, each group is one value of at most 32
    // bits and leaves with one pair of ORs (the common case: about 17 bits
    // at 4 bps); otherwise the wave writes code by code.
    uint32_t qv[16], gl[4], gmax = 0;
    const uint32_t k1 = k + 1u;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t sl = 0;
#pragma unroll
      for (int i = 4 * g; i < 4 * g + 4; ++i) {
        const uint32_t zeta = WIDE ? zz[i] : __builtin_amdgcn_ubfe(zz[i >> 2], 8 * (i & 3), 8);
        qv[i] = zeta >> k;
        sl += qv[i] + k1;
      }
      gl[g] = sl;
      gmax = sl > gmax ? sl : gmax;
    }
    // this lane's payload bits: sum floor(zeta / 2^k) + 16 (1 + k)
    const uint32_t T = live ? (gl[0] + gl[1]) + (gl[2] + gl[3]) : 0u;
    const uint32_t pos = 4u + (uint32_t)a.coset_bits + row_incl_scan<G>(T, r) - T;
    // rice_k and tile_bits computed here always hold the codes; given ones
    // that do not (k > 8, or codes past tile_bits or past the tile's LDS
    // words) leave the lane's codes unwritten and mark the tile corrupt
    const bool fits = !a.given || (ck <= kMaxK && pos + T <= tb && tb <= 32u * (uint32_t)W);
    if (live && !fits) set_status(a.status, HQ_ST_CORRUPT);
    const bool grouped = __builtin_amdgcn_ballot_w64(live && fits && gmax > 32u) == 0;
    if (live) {
      if (r == 0) {
        // header: k (4 bits), then the coset bits (word j at bit 4 + 32 j);
        // one full coset word (E8, tile 256) without the loop
        if (a.coset_words == 0) atomicOr(tw, k);
        else if (a.coset_bits == 32) {
          atomicOr(tw, (in.cw0 << 4) | k);
          atomicOr(tw + 1, in.cw0 >> 28);
        } else
        for (int j = 0; j < a.coset_words; ++j) {
          const int nb = a.coset_bits - 32 * j;
          uint32_t cw = j == 0 ? in.cw0 : a.coset[tile * a.coset_words + j];
          if (nb < 32) cw &= (1u << nb) - 1u;
          atomicOr(tw + j, (cw << 4) | (j == 0 ? k : 0u));
          atomicOr(tw + j + 1, cw >> 28);
        }
      }
      // the lane's 16 codes are OR-ed into the tile's LDS words (a lane's
      // first and last words may be shared with its neighbours, which the
      // OR allows)
      if (fits && grouped) {
        const uint32_t rmask = (1u << k) - 1u;
        uint32_t pb = pos;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // the group's codes, each ((2 rem + 1) << q) - 1 (q ones, a zero,
          // the k low bits), at their offsets inside the group
          uint32_t c = 0, sh = 0;
#pragma unroll
          for (int i = 4 * g; i < 4 * g + 4; ++i) {
            const uint32_t zeta = WIDE ? zz[i] : __builtin_amdgcn_ubfe(zz[i >> 2], 8 * (i & 3), 8);
            c |= (((((zeta & rmask) << 1) | 1u) << qv[i]) - 1u) << sh;
            sh += qv[i] + k1;
          }
          const uint64_t v = (uint64_t)c << (pb & 31u);
          uint32_t* w = tw + (pb >> 5);
          atomicOr(w, (uint32_t)v);
          atomicOr(w + 1, (uint32_t)(v >> 32));
          pb += gl[g];
        }
      } else if (fits) {
        const uint32_t rmask = (1u << k) - 1u;
        uint32_t pb = pos;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t zeta = WIDE ? zz[i] : __builtin_amdgcn_ubfe(zz[i >> 2], 8 * (i & 3), 8);
          const uint32_t q = zeta >> k, rem = zeta & rmask, len = q + 1u + k;
          if (len <= 32u) {
            // q ones, a zero, the k low bits: ((2 rem + 1) << q) - 1, at bit
            // pb, OR-ed into the (at most two) words it touches
            const uint32_t c = (((rem << 1) | 1u) << q) - 1u;
            const uint64_t v = (uint64_t)c << (pb & 31u);
            uint32_t* w = tw + (pb >> 5);
            atomicOr(w, (uint32_t)v);
            atomicOr(w + 1, (uint32_t)(v >> 32));
          } else {
            BitWriter bw{tw, 0, pb & 31u, pb >> 5};
            uint32_t qq = q;
            while (qq > 0u) {
              const uint32_t t = qq < 32u ? qq : 32u;
              bw.put(t == 32u ? 0xFFFFFFFFu : (1u << t) - 1u, t);
              qq -= t;
            }
            bw.put(rem << 1, 1u + k);
            bw.flush();
          }
          pb += len;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (live) {
      if (r == 0) a.tile_word_offset[tile] = off;
      if (tile == a.n_tiles - 1 && r == 0) a.tile_word_offset[a.n_tiles] = off + nwords;
      if (off + nwords <= a.capacity) {
        // the pass's words are [base, base + pass_words): 32-bit offsets
        // from there (a pass holds at most 64 / G * W words)
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(a.stream + base, (short)0,
                                                          (int)(pass_words * 4u), 0x00020000);
        const uint32_t o0 = (uint32_t)(off - base);
        // a fixed count of stores (the wait counts of the loads in flight
        // stay known to the compiler)
#pragma unroll
        for (int s = 0; s < (W + G - 1) / G; ++s) {
          const uint32_t j = (uint32_t)(r + s * G);
          if (j < nwords) __builtin_amdgcn_raw_buffer_store_b32(tw[j], rs, (int)((o0 + j) * 4u), 0, 0);
        }
      } else if (r == 0) {
        set_status(a.status, HQ_ST_STREAM_FULL);
      }
    }
    base += pass_words;
    // the LDS words are rewritten by the next pass
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // the data of the next kPackAhead passes are loaded while this pass is
  // computed (a pass takes a few VGPRs; the loads are what keeps HBM
  // busy).  Slot d of the ring serves passes d, d + kPackAhead, ...: it is
  // refilled right after its pass, so no register is copied while its load
  // is in flight.
  // (the prologue issues its loads slot by slot, in the loop's order, so
  // that the waits at the loop head are the loop's own)
  PassIn ring[kPackAhead];
#pragma unroll
  for (int d = 0; d < kPackAhead; ++d) {
    fetch(first + (int64_t)d * TPW, ring[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t t0 = first; t0 < end; t0 += (int64_t)kPackAhead * TPW) {
#pragma unroll
    for (int d = 0; d < kPackAhead; ++d) {
      const int64_t t = t0 + (int64_t)d * TPW;
      pass(ring[d], t);
      fetch(t + (int64_t)kPackAhead * TPW, ring[d]);
    }
  }
}

template <int N, bool WIDE>
hipError_t launch_nw(const RateBatch& b, hipStream_t s) {
  const unsigned blocks = (unsigned)b.block0[b.n];
  bool atomics = false, given = false, pack = false;
  for (int i = 0; i < b.n; ++i) {
    atomics = atomics || b.it[i].block_words == nullptr;
    given = given || b.it[i].given;
    pack = pack || b.it[i].stream != nullptr;
  }
  if (atomics) hipLaunchKernelGGL(zero_totals_kernel, dim3(1), dim3(64), 0, s, b);
  if (given)
    hipLaunchKernelGGL(rate_given_kernel<N>, dim3(blocks), dim3(kBlock), 0, s, b);
  else
    hipLaunchKernelGGL((rate_kernel<N, WIDE>), dim3(blocks), dim3(kBlock), 0, s, b);
  hipLaunchKernelGGL(scan_kernel, dim3((unsigned)b.n), dim3(kScanThreads), 0, s, b);
  if (pack) hipLaunchKernelGGL((pack_kernel<N, WIDE>), dim3(blocks), dim3(kBlock), 0, s, b);
  return hipGetLastError();
}

// (the matrices of one launch share the index mode)
template <int N>
hipError_t launch_n(const RateBatch& b, hipStream_t s) {
  return b.it[0].wide ? launch_nw<N, true>(b, s) : launch_nw<N, false>(b, s);
}

template <int N>
int64_t blocks_n(int64_t n_tiles) {
  return (rate_waves<N>(n_tiles) + kBlock / 64 - 1) / (kBlock / 64);
}

}  // namespace

int64_t rate_blocks(int tile, int64_t n_tiles) {
  switch (tile) {
    case 64: return blocks_n<64>(n_tiles);
    case 128: return blocks_n<128>(n_tiles);
    case 256: return blocks_n<256>(n_tiles);
    default: return blocks_n<512>(n_tiles);
  }
}

// The matrices of one launch share the tile and, for a pass with given
// values, the flag (the API groups them so).
hipError_t launch_rate_batch(const RateBatch& b, hipStream_t s) {
  switch (b.it[0].tile) {
    case 64: return launch_n<64>(b, s);
    case 128: return launch_n<128>(b, s);
    case 256: return launch_n<256>(b, s);
    default: return launch_n<512>(b, s);
  }
}

hipError_t launch_rate(const RateLaunch& a, hipStream_t s) {
  RateBatch b;
  memset(&b, 0, sizeof(b));
  b.n = 1;
  b.it[0] = a;
  b.block0[0] = 0;
  b.block0[1] = rate_blocks(a.tile, a.n_tiles);
  for (int i = 1; i < kRateMaxItems; ++i) b.it[i] = a;
  for (int i = 2; i <= kRateMaxItems; ++i) b.block0[i] = b.block0[1];
  return launch_rate_batch(b, s);
}

int64_t rate_workspace_blocks(int64_t n_tiles) {
  // at most one wave per 2 tiles (tile 512), capped, in blocks of 4 waves
  int64_t w = (n_tiles + 1) / 2;
  if (w > kMaxRateWaves) w = kMaxRateWaves;
  return (w + kBlock / 64 - 1) / (kBlock / 64);
}

}  // namespace hq

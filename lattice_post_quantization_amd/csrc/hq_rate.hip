// Rice rate accounting and packing of stripped indices.
//
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." idea (iii) (near-entropy-optimal Rice coding of
// the lattice indices); [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal
// Lattice Quantization Pipeline ..." (Rice code, one itemized rate
// accounting); GitHub issue "HyperQuant ... #9", "Additional context" (a
// packed, Rice-coded lattice-index checkpoint format).
//
// Three kernels:
//   rate_kernel  per tile: zigzag, k = argmin payload, tile_bits; per block:
//                the sum of ceil(tile_bits/32) into the workspace; the total
//                bit count is accumulated with one 64-bit atomic per block.
//   scan_kernel  one block: exclusive prefix sum of the per-block word sums.
//   pack_kernel  per tile: code lengths -> in-tile exclusive scan (lanes and
//                lane groups) -> bit positions; codes are OR-ed into an LDS
//                copy of the tile's words, which is then stored at the
//                tile's word offset.  Tiles are word aligned, so no two
//                tiles share a word.
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

// Inclusive scan across a lane group of width G (Hillis-Steele on shuffles).
template <int G>
__device__ inline uint32_t group_inclusive_scan(uint32_t v, int r) {
#pragma unroll
  for (int d = 1; d < G; d <<= 1) {
    uint32_t p = __shfl_up(v, d, G);
    if (r >= d) v += p;
  }
  return v;
}

template <int N>
__device__ inline void load_zeta(const int8_t* idx, int64_t e0, uint32_t* zz) {
  const uint4 q = *reinterpret_cast<const uint4*>(idx + e0);
  const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) zz[i] = zigzag((int32_t)(int8_t)(qw[i >> 2] >> (8 * (i & 3))));
}

// k = argmin_k sum(floor(zeta/2^k) + 1 + k), first minimum; returns the payload.
template <int G, int N>
__device__ inline uint32_t best_k(const uint32_t* zz, int& bk) {
  uint32_t best = 0xFFFFFFFFu;
  bk = 0;
#pragma unroll
  for (int k = 0; k < 9; ++k) {
    uint32_t p = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) p += zz[i] >> k;
    const uint32_t L = group_sum<G>(p) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

template <int N>
__global__ __launch_bounds__(kBlock) void rate_kernel(RateLaunch a) {
  constexpr int G = N / kElemsPerLane;
  constexpr int TPB = kBlock / G;
  __shared__ uint64_t blk_words[kBlock / 64];
  __shared__ uint64_t blk_bits[kBlock / 64];
  const int r = threadIdx.x % G;
  const int64_t tile = (int64_t)blockIdx.x * TPB + threadIdx.x / G;
  uint64_t words = 0, bits = 0;
  if (tile < a.n_tiles) {
    uint32_t zz[16];
    load_zeta<N>(a.idx, tile * N + (int64_t)r * kElemsPerLane, zz);
    int bk;
    const uint32_t pay = best_k<G, N>(zz, bk);
    const uint32_t tb = 4u + (uint32_t)a.coset_bits + pay;
    if (r == 0) {
      a.rice_k[tile] = (uint8_t)bk;
      a.tile_bits[tile] = tb;
      words = (tb + 31u) / 32u;
      bits = tb;
    }
  }
  // block sums (lane 0 of each group contributes)
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    words += __shfl_xor(words, m);
    bits += __shfl_xor(bits, m);
  }
  if ((threadIdx.x & 63) == 0) {
    blk_words[threadIdx.x >> 6] = words;
    blk_bits[threadIdx.x >> 6] = bits;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t w = 0, b = 0;
    for (int i = 0; i < kBlock / 64; ++i) { w += blk_words[i]; b += blk_bits[i]; }
    if (a.block_words != nullptr) a.block_words[blockIdx.x] = w;
    atomicAdd((unsigned long long*)a.total_bits, (unsigned long long)b);
  }
}

__global__ void zero_u64_kernel(uint64_t* p) { *p = 0; }

// Exclusive scan of n values in place, one block of kBlock threads.
__global__ __launch_bounds__(kBlock) void scan_kernel(uint64_t* v, int64_t n) {
  __shared__ uint64_t part[kBlock];
  const int t = threadIdx.x;
  const int64_t chunk = (n + kBlock - 1) / kBlock;
  const int64_t lo = t * chunk;
  const int64_t hi = (lo + chunk < n) ? lo + chunk : n;
  uint64_t s = 0;
  for (int64_t i = lo; i < hi; ++i) s += v[i];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    uint64_t run = 0;
    for (int i = 0; i < kBlock; ++i) {
      uint64_t x = part[i];
      part[i] = run;
      run += x;
    }
  }
  __syncthreads();
  uint64_t run = part[t];
  for (int64_t i = lo; i < hi; ++i) {
    uint64_t x = v[i];
    v[i] = run;
    run += x;
  }
}

// Max words one tile can need: 4 + coset bits + 9 N (k = 8 bounds the optimum).
template <int N>
struct PackBound {
  static constexpr int kMaxBits = 4 + N / 2 + 9 * N;
  static constexpr int kWords = (kMaxBits + 31) / 32;
};

__device__ inline void lds_set_bits(uint32_t* w, uint32_t pos, uint32_t nbits, uint32_t value) {
  // value has nbits <= 32 significant bits, LSB first at bit position pos
  if (nbits == 0) return;
  const uint32_t wi = pos >> 5, sh = pos & 31;
  atomicOr(&w[wi], value << sh);
  if (sh + nbits > 32) atomicOr(&w[wi + 1], value >> (32 - sh));
}

__device__ inline void lds_set_ones(uint32_t* w, uint32_t pos, uint32_t count) {
  while (count > 0) {
    const uint32_t wi = pos >> 5, sh = pos & 31;
    const uint32_t take = (32 - sh < count) ? 32 - sh : count;
    const uint32_t mask = (take == 32) ? 0xFFFFFFFFu : (((1u << take) - 1u) << sh);
    atomicOr(&w[wi], mask);
    pos += take;
    count -= take;
  }
}

template <int N>
__global__ __launch_bounds__(kBlock) void pack_kernel(RateLaunch a) {
  constexpr int G = N / kElemsPerLane;
  constexpr int TPB = kBlock / G;
  constexpr int W = PackBound<N>::kWords;
  __shared__ uint32_t buf[TPB * W];
  __shared__ uint64_t toff[TPB + 1];
  const int r = threadIdx.x % G;
  const int slot = threadIdx.x / G;
  const int64_t tile0 = (int64_t)blockIdx.x * TPB;
  const int64_t tile = tile0 + slot;

  for (int i = threadIdx.x; i < TPB * W; i += kBlock) buf[i] = 0;
  if (threadIdx.x == 0) {
    // tile word offsets inside this block (serial over TPB tiles)
    uint64_t run = a.block_words[blockIdx.x];
    for (int s = 0; s < TPB; ++s) {
      toff[s] = run;
      const int64_t t = tile0 + s;
      if (t < a.n_tiles) run += (a.tile_bits[t] + 31u) / 32u;
    }
    toff[TPB] = run;
  }
  __syncthreads();
  const bool live = tile < a.n_tiles;
  uint32_t* tw = buf + slot * W;
  uint32_t tb = 0, nwords = 0;
  if (live) {
    tb = a.tile_bits[tile];
    nwords = (tb + 31u) / 32u;
    const int k = a.rice_k[tile];
    uint32_t zz[16];
    load_zeta<N>(a.idx, tile * N + (int64_t)r * kElemsPerLane, zz);
    uint32_t lens[16], lane_total = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      lens[i] = (zz[i] >> k) + 1u + (uint32_t)k;
      lane_total += lens[i];
    }
    const uint32_t incl = group_inclusive_scan<G>(lane_total, r);
    uint32_t pos = 4u + (uint32_t)a.coset_bits + incl - lane_total;
    if (r == 0) {
      lds_set_bits(tw, 0, 4, (uint32_t)k);
      for (int j = 0; j < a.coset_words; ++j) {
        const int nb = a.coset_bits - 32 * j;
        const uint32_t cw = a.coset[tile * a.coset_words + j];
        lds_set_bits(tw, 4u + 32u * j, nb < 32 ? nb : 32,
                     nb < 32 ? (cw & ((1u << nb) - 1u)) : cw);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t qv = zz[i] >> k;
      lds_set_ones(tw, pos, qv);
      if (k > 0) lds_set_bits(tw, pos + qv + 1u, (uint32_t)k, zz[i] & ((1u << k) - 1u));
      pos += lens[i];
    }
  }
  __syncthreads();
  if (live) {
    const uint64_t off = toff[slot];
    if (r == 0) a.tile_word_offset[tile] = off;
    if (tile == a.n_tiles - 1 && r == 0) a.tile_word_offset[a.n_tiles] = toff[slot] + nwords;
    if (off + nwords <= a.capacity) {
      for (uint32_t j = r; j < nwords; j += G) a.stream[off + j] = tw[j];
    } else if (r == 0) {
      set_status(a.status, HQ_ST_STREAM_FULL);
    }
  }
}

template <int N>
hipError_t launch_n(const RateLaunch& a, hipStream_t s) {
  constexpr int TPB = kBlock / (N / kElemsPerLane);
  const int64_t blocks = (a.n_tiles + TPB - 1) / TPB;
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(1), 0, s, a.total_bits);
  hipLaunchKernelGGL(rate_kernel<N>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  if (a.stream != nullptr) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kBlock), 0, s, a.block_words, blocks);
    hipLaunchKernelGGL(pack_kernel<N>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rate(const RateLaunch& a, hipStream_t s) {
  return a.tile == 256 ? launch_n<256>(a, s) : launch_n<128>(a, s);
}

int64_t rate_blocks(int64_t n_tiles, int tile) {
  const int TPB = kBlock / (tile / kElemsPerLane);
  return (n_tiles + TPB - 1) / TPB;
}

}  // namespace hq

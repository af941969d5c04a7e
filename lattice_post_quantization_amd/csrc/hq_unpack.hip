// Rice stream decoder: packed words back to stripped indices, coset words
// and Rice parameters (the inverse of the packing in hq_rate.hip).
//
// Passages: GitHub issue "HyperQuant ... #9", "Additional context" (a packed,
// Rice-coded lattice-index checkpoint format); [arXiv abstract] "HyperQuant:
// A Rate-Distortion-Optimal Quantization Pipeline ..." idea (iii) and [ICLR
// abstract] "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
// Pipeline ..." (the Rice code of the stripped indices).
//
// A Rice code is only self-delimiting front to back, so one lane decodes one
// tile: a 64-bit bit buffer is refilled a word at a time, with the next word
// loaded one refill ahead; a unary run is found with a count of trailing
// zeros of the inverted buffer.  A wave holds 64 consecutive tiles.  Decoded
// bytes go to an 8 KB LDS buffer (128 bytes of each of the 64 tiles) that is
// written back as full 128-byte lines, eight tiles per store instruction.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ inline __amdgpu_buffer_rsrc_t out_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

// Lanes of one wave exchange data through LDS; the fences only keep the
// compiler from moving or reusing LDS accesses across the exchange (LDS
// instructions of one wave execute in order).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bits of one tile's words [wp, we): b holds nb unread bits, least
// significant first; bits of b above nb are zero.
struct BitReader {
  const uint32_t* s;
  uint64_t wp, we;
  uint64_t b;
  uint32_t nb;
  uint32_t ahead;   // s[wp] when wp < we, loaded one refill early

  __device__ inline void init(const uint32_t* src, uint64_t w0, uint64_t w1) {
    s = src;
    wp = w0;
    we = w1;
    b = 0;
    nb = 0;
    ahead = w0 < w1 ? s[w0] : 0u;
  }
  // afterwards nb > 32 unless the tile's words ran out
  __device__ inline void refill() {
    if (nb <= 32u && wp < we) {
      b |= (uint64_t)ahead << nb;
      nb += 32u;
      ++wp;
      ahead = wp < we ? s[wp] : 0u;
    }
  }
  // n <= 32 bits (fewer if fewer remain; the caller checks nb first)
  __device__ inline uint32_t take(uint32_t n) {
    n = n < nb ? n : nb;
    const uint32_t v = (uint32_t)b & (n >= 32u ? 0xFFFFFFFFu : (1u << n) - 1u);
    b >>= n;
    nb -= n;
    return v;
  }
};

// One Rice code: the zigzag value, or 256 and bad set when the code runs past
// the tile or exceeds a byte.
__device__ inline uint32_t read_code(BitReader& br, uint32_t k, bool& bad) {
  br.refill();
  uint32_t q = 0;
  for (;;) {
    // first zero bit among the nb valid bits (bits above nb are zero, so
    // ~b has ones there and the count stops at nb at the latest)
    const uint64_t inv = ~br.b;
    const uint32_t z = inv == 0 ? 64u : (uint32_t)__builtin_ctzll(inv);
    if (z < br.nb) {
      q += z;
      br.b = z + 1u >= 64u ? 0 : br.b >> (z + 1u);
      br.nb -= z + 1u;
      break;
    }
    q += br.nb;
    br.b = 0;
    br.nb = 0;
    br.refill();
    if (br.nb == 0u || q > 255u) {
      bad = true;
      return 256u;
    }
  }
  br.refill();
  if (br.nb < k) {
    bad = true;
    return 256u;
  }
  const uint32_t zeta = (q << k) | br.take(k);
  if (q > 255u || zeta > 255u) {
    bad = true;
    return 256u;
  }
  return zeta;
}

// int8 index of a zigzag value (as a byte)
__device__ inline uint32_t unzigzag8(uint32_t zeta) {
  return ((zeta >> 1) ^ (0u - (zeta & 1u))) & 0xFFu;
}

template <int N>
__global__ __launch_bounds__(kBlock) void unpack_kernel(UnpackLaunch a) {
  __shared__ uint4 stage[kBlock / 64][512];   // per wave: 8 chunks of 64 tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint4* st = stage[wave];
  const int64_t wave_tile0 = ((int64_t)blockIdx.x * kBlock) + (int64_t)wave * 64;
  if (wave_tile0 >= a.n_tiles) return;   // whole waves only
  const int64_t tile = wave_tile0 + lane;
  const bool live = tile < a.n_tiles;
  const int64_t rem_tiles = a.n_tiles - wave_tile0;
  const uint32_t live_in_wave = (uint32_t)(rem_tiles < 64 ? rem_tiles : 64);

  bool bad = false;
  BitReader br;
  uint64_t w0 = 0, w1 = 0;
  if (live) {
    w0 = a.tile_word_offset[tile];
    w1 = a.tile_word_offset[tile + 1];
    if (w1 < w0) {
      bad = true;
      w1 = w0;
    }
  }
  br.init(a.stream, w0, w1);
  br.refill();
  if (br.nb < 4u) bad = true;
  const uint32_t k = br.take(4);
  for (int j = 0; j < a.coset_words; ++j) {
    const int nbits = a.coset_bits - 32 * j < 32 ? a.coset_bits - 32 * j : 32;
    br.refill();
    if (br.nb < (uint32_t)nbits) bad = true;
    const uint32_t cw = br.take((uint32_t)nbits);
    if (live) a.coset[tile * a.coset_words + j] = cw;
  }
  if (live && a.rice_k != nullptr) a.rice_k[tile] = (uint8_t)k;

  const auto rs = out_rsrc(a.idx + wave_tile0 * N, live_in_wave * (uint32_t)N);
  // writer lane L keeps chunk c of its current 128 bytes at slot
  // 8 L + ((c ^ (L >> 1)) & 7): each 16-lane group writes 16 bank groups
#pragma unroll 1
  for (int half = 0; half < N / 128; ++half) {
#pragma unroll 1
    for (int c = 0; c < 8; ++c) {
      uint32_t d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) w |= unzigzag8(read_code(br, k, bad)) << (8 * bi);
        d[j] = w;
      }
      st[8 * lane + ((c ^ (lane >> 1)) & 7)] = make_uint4(d[0], d[1], d[2], d[3]);
    }
    wave_lds_sync();
    // store instruction j: lane l writes chunk l & 7 of wave tile 8 j + l / 8
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int T = 8 * j + (lane >> 3), cc = lane & 7;
      const uint4 q = st[8 * T + ((cc ^ (T >> 1)) & 7)];
      __builtin_amdgcn_raw_buffer_store_b128((u32x4){q.x, q.y, q.z, q.w}, rs,
                                             T * N + half * 128 + 16 * cc, 0, 0);
    }
    wave_lds_sync();
  }
  if (live && bad) set_status(a.status, HQ_ST_CORRUPT);
}

}  // namespace

hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t s) {
  const int64_t blocks = (a.n_tiles + kBlock - 1) / kBlock;
  if (a.tile == 256)
    hipLaunchKernelGGL(unpack_kernel<256>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(unpack_kernel<128>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace hq

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
// fetched one refill ahead; a unary run is found with a count of trailing
// zeros of the inverted buffer.  A wave holds 64 consecutive tiles, whose
// words are contiguous: when they fit in 10 KB the wave first copies them
// into LDS with coalesced loads and decodes from there with branch-free
// refills; otherwise it reads global memory.  Decoded bytes go to a 4 KB LDS
// buffer (64 bytes of each tile) that is written back 64 contiguous bytes
// per tile, sixteen tiles per store instruction.  One launch covers up to
// eight packed matrices (a layer's projections), its waves running over
// them in order, so that small matrices together fill the GPU.
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

typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) void lds_void;

// Bits of one tile's words [wp, we): b holds nb unread bits, least
// significant first; bits of b above nb are zero; `ahead` is word wp (when
// wp < we), fetched one refill early.  FromLds: the words sit in LDS at
// lds[w - base]; else they are read from the stream in global memory.
template <bool FromLds>
struct BitReader {
  const uint32_t* s;
  const lds_u32* lds;
  uint64_t base;
  uint64_t wp, we;
  uint64_t b;
  uint32_t nb;
  uint32_t ahead;

  __device__ inline uint32_t word(uint64_t w) const {
    if constexpr (FromLds) {
      return lds[(uint32_t)(w - base)];
    } else {
      return s[w];
    }
  }
  __device__ inline void init(const uint32_t* src, const lds_u32* staged, uint64_t staged_base,
                              uint64_t w0, uint64_t w1) {
    s = src;
    lds = staged;
    base = staged_base;
    wp = w0;
    we = w1;
    b = 0;
    nb = 0;
    ahead = w0 < w1 ? word(w0) : 0u;
  }
  // afterwards nb > 32 unless the tile's words ran out
  __device__ inline void refill() {
    if constexpr (FromLds) {
      // branch-free: the read address is clamped into the tile's range
      const bool c = nb <= 32u && wp < we;
      b |= c ? (uint64_t)ahead << nb : 0;
      nb += c ? 32u : 0u;
      wp += c ? 1u : 0u;
      const uint64_t last = we > 0 ? we - 1 : 0;
      const uint32_t nxt = word(wp < we ? wp : (last > base ? last : base));
      ahead = c ? (wp < we ? nxt : 0u) : ahead;
    } else {
      if (nb <= 32u && wp < we) {
        b |= (uint64_t)ahead << nb;
        nb += 32u;
        ++wp;
        ahead = wp < we ? word(wp) : 0u;
      }
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
  // this reader stops at the tile's last word, so an overrun shows as
  // missing bits while decoding
  __device__ inline bool overran() const { return false; }
  __device__ inline bool short_of(uint32_t n) const { return nb < n; }
};

// One Rice code: the zigzag value (garbage, with bad set, when the code runs
// past the tile or exceeds a byte).
template <bool FromLds>
__device__ inline uint32_t read_code(BitReader<FromLds>& br, uint32_t k, uint32_t zmax, bool& bad) {
  br.refill();
  // first zero among the valid bits (bits above nb are zero, so ~b has ones
  // there and the count stops at nb at the latest)
  const uint64_t inv = ~br.b;
  uint32_t z = inv == 0 ? 64u : (uint32_t)__builtin_ctzll(inv);
  uint32_t q = 0;
  if (z >= br.nb) {
    // the run of ones continues past the buffer (rare): consume and refill
    for (;;) {
      q += br.nb;
      br.b = 0;
      br.nb = 0;
      br.refill();
      const uint64_t iv = ~br.b;
      z = iv == 0 ? 64u : (uint32_t)__builtin_ctzll(iv);
      if (br.nb == 0u || q > zmax) {
        bad = true;
        z = 0;
        break;
      }
      if (z < br.nb) break;
    }
  }
  q += z;
  const uint32_t used = z + 1u <= br.nb ? z + 1u : br.nb;
  br.b = used >= 64u ? 0 : br.b >> used;
  br.nb -= used;
  br.refill();
  bad |= br.nb < k;
  const uint32_t zeta = (q << k) | br.take(k);
  bad |= zeta > zmax;
  return zeta;
}

// trailing zeros of x, 32 for x = 0 (one v_ffbl and a min)
__device__ inline uint32_t ctz0(uint32_t x) { return x ? (uint32_t)__builtin_ctz(x) : 32u; }

// Tile reader over words staged in LDS, by bit position: the 64-bit window
// (lo, hi) holds words w and w + 1 of the segment, o < 32 is the position
// of the next unread bit in lo, and nxt is word w + 2 (read when the window
// moves on; reads past the staged words repeat the last one).  A code whose
// unary run and remainder lie in the 32 bits at o (every code shorter than
// 33 bits) is read from one funnel shift of the window: its run of ones
// ends at the first zero, then k remainder bits.  The window moves by at
// most one word per code.  It does not stop at the tile's last word (the
// words after it are the wave's next tiles, or the repeated last staged
// word), so a code that runs past its tile reads staged words only; overran() reports a tile whose codes used more bits than its
// words hold.  zor collects the zigzag values (one of them exceeds zmax iff
// their OR does, zmax + 1 a power of two).
struct WinReader {
  const lds_u32* lds;
  uint32_t last4;               // byte offset of the last staged word
  uint32_t w0, wend;            // the tile's words [w0, wend)
  uint32_t p;                   // byte offset of word w + 2 (w: the word of lo)
  uint32_t o;
  uint32_t lo, hi, nxt;
  uint32_t zor;
  uint32_t zor_mask;

  __device__ inline uint32_t rd(uint32_t byte_off) const {
    const uint32_t q = byte_off < last4 ? byte_off : last4;
    return *reinterpret_cast<const lds_u32*>(reinterpret_cast<const __attribute__((address_space(3))) char*>(lds) + q);
  }
  __device__ inline uint32_t word() const { return p / 4u - 2u; }
  __device__ inline void init(const lds_u32* seg, uint32_t a, uint32_t b, uint32_t n_staged) {
    lds = seg;
    last4 = 4u * (n_staged - 1u);
    w0 = a;
    wend = b;
    p = 4u * (a + 2u);
    o = 0;
    lo = rd(4u * a);
    hi = rd(4u * a + 4u);
    nxt = rd(p);
    zor = 0;
  }
  __device__ inline void refill() {}
  __device__ inline void move() {
    if (o >= 32u) {
      o -= 32u;
      lo = hi;
      hi = nxt;
      p += 4u;
      nxt = rd(p);
    }
  }
  // the window after o moved by at most 32 bits, without a branch (the
  // read repeats the current word when the window stays)
  __device__ inline void step() {
    const bool c = o >= 32u;
    o &= 31u;
    lo = c ? hi : lo;
    hi = c ? nxt : hi;
    p += c ? 4u : 0u;
    nxt = rd(p);
  }
  // n <= 32 bits
  __device__ inline uint32_t take(uint32_t n) {
    const uint32_t x = __builtin_amdgcn_alignbit(hi, lo, o);
    o += n;
    move();
    return n >= 32u ? x : x & ((1u << n) - 1u);
  }
  __device__ inline uint32_t code(uint32_t k, uint32_t zmax, bool& bad) {
    const uint32_t x = __builtin_amdgcn_alignbit(hi, lo, o);
    const uint32_t z = ctz0(~x);
    uint32_t zeta;
    if (z + 1u + k <= 32u) {
      zeta = (z << k) | __builtin_amdgcn_ubfe(x, z + 1u, k);
      o += z + 1u + k;
      move();
    } else {
      // a run of ones or a remainder past the 32 bits at o
      uint32_t q = 0;
      for (;;) {
        const uint32_t y = __builtin_amdgcn_alignbit(hi, lo, o);
        const uint32_t zz = ctz0(~y);
        q += zz;
        o += zz < 32u ? zz + 1u : 32u;
        move();
        if (zz < 32u) break;
        if (q > zmax || word() > wend) {   // corrupt: stop here
          bad = true;
          break;
        }
      }
      zeta = (q << k) | take(k);
    }
    zor |= zeta;
    return zeta;
  }
  __device__ inline bool overran() const {
    return (zor & ~zor_mask) != 0u || 32u * (word() - w0) + o > 32u * (wend - w0);
  }
  // (header bits past the tile show up in overran())
  __device__ inline bool short_of(uint32_t) const { return false; }
};

__device__ inline uint32_t next_code(WinReader& br, uint32_t k, uint32_t zmax, bool& bad) {
  return br.code(k, zmax, bad);
}
__device__ inline uint32_t next_code(BitReader<false>& br, uint32_t k, uint32_t zmax, bool& bad) {
  return read_code(br, k, zmax, bad);
}

// index of a zigzag value, as a byte (int8) or a half-word (int16)
__device__ inline uint32_t unzigzag8(uint32_t zeta) {
  return ((zeta >> 1) ^ (0u - (zeta & 1u))) & 0xFFu;
}
__device__ inline uint32_t unzigzag16(uint32_t zeta) {
  return ((zeta >> 1) ^ (0u - (zeta & 1u))) & 0xFFFFu;
}

// The same for the four zigzag bytes (two half-words) of a dword: half the
// value, complemented where it is odd (all-ones in a field from its low
// bit l: (l << width) - l).
// (v_perm selectors 8-11 replicate the sign bits of bytes 1, 3, 5, 7 of
// {src0, src1}; shifted left by 15, bit 0 of each byte or half-word lands
// on the sign bit of byte 1 or 3.)
template <bool WIDE>
__device__ inline uint32_t unzigzag_packed(uint32_t d) {
  constexpr uint32_t kHalf = WIDE ? 0x7FFF7FFFu : 0x7F7F7F7Fu;
  // int8: byte b's low bit sits at bit 7 of byte b of d << 7 (bytes 1, 3
  // of src0) and of byte b + 1 of d << 15 (bytes 1, 3 of src1)
  const uint32_t neg = WIDE ? __builtin_amdgcn_perm(0u, d << 15, 0x09090808u)
                            : __builtin_amdgcn_perm(d << 7, d << 15, 0x0B090A08u);
  return ((d >> 1) & kHalf) ^ neg;
}

// One 16-byte chunk of a tile's indices (16 int8 or 8 int16 codes), code
// by code.
template <bool WIDE, typename Reader>
__device__ inline void chunk_by_code(Reader& br, uint32_t k, uint32_t zmax, bool& bad,
                                     uint32_t* d) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = 0;
    if constexpr (WIDE) {
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) w |= unzigzag16(next_code(br, k, zmax, bad)) << (16 * hi);
    } else {
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) w |= unzigzag8(next_code(br, k, zmax, bad)) << (8 * bi);
    }
    d[j] = w;
  }
}

template <bool WIDE>
__device__ inline void next_chunk(BitReader<false>& br, uint32_t k, uint32_t zmax, bool& bad,
                                  uint32_t* d) {
  chunk_by_code<WIDE>(br, k, zmax, bad, d);
}

// raw v_ffbl_b32: the lowest set bit, 0xFFFFFFFF for 0
__device__ inline uint32_t ffbl_raw(uint32_t x) {
  uint32_t r;
  __asm__("v_ffbl_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// WinReader: the chunk's codes without a branch, on the assumption that
// every code of every lane lies in the 32 bits at its position (z + 1 + k
// <= 32 for its first zero z); a code that does not (its first zero or its
// remainder past them, or no zero: z = 0xFFFFFFFF) shows as
// max z > 31 - k, and then the whole wave reads the chunk again code by
// code from the saved window.
template <bool WIDE>
__device__ inline void next_chunk(WinReader& br, uint32_t k, uint32_t zmax, bool& bad,
                                  uint32_t* d) {
  const uint32_t so = br.o, sp = br.p, slo = br.lo, shi = br.hi, snx = br.nxt, szor = br.zor;
  constexpr int kPer = WIDE ? 2 : 4;
  const uint32_t k1 = k + 1u;
  uint32_t zmx = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t pk = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t x = __builtin_amdgcn_alignbit(br.hi, br.lo, br.o);
      const uint32_t z = ffbl_raw(~x);
      zmx = z > zmx ? z : zmx;
      const uint32_t zeta = (z << k) | __builtin_amdgcn_ubfe(x, z + 1u, k);
      br.zor |= zeta;
      pk |= zeta << ((WIDE ? 16 : 8) * i);
      br.o += z + k1;
      br.step();
    }
    d[j] = unzigzag_packed<WIDE>(pk);
  }
  if (__builtin_amdgcn_ballot_w64(zmx > 31u - k) != 0) {
    br.o = so;
    br.p = sp;
    br.lo = slo;
    br.hi = shi;
    br.nxt = snx;
    br.zor = szor;
    chunk_by_code<WIDE>(br, k, zmax, bad, d);
  }
}

constexpr int kUnpackBlock = 128;     // two waves
constexpr int kSegWords = 2560;       // staged stream words per wave (10 KB)

// Decodes this lane's tile and writes it through the wave's 4 KB LDS buffer
// (64 bytes of each tile at a time: 64 int8 or 32 int16 indices; writer lane
// L keeps chunk c at slot 4 L + ((c ^ (L >> 2)) & 3), so each 16-lane group
// writes 16 bank groups).
template <int N, bool WIDE, typename Reader>
__device__ inline void decode_tiles(const UnpackLaunch& a, const UnpackItem& it, Reader& br,
                                    int64_t tile, bool live, int64_t wave_tile0,
                                    uint32_t live_in_wave, int lane, uint4* st, bool& bad) {
  br.refill();
  bad |= br.short_of(4u);
  const uint32_t k = br.take(4);
  for (int j = 0; j < a.coset_words; ++j) {
    const int nbits = a.coset_bits - 32 * j < 32 ? a.coset_bits - 32 * j : 32;
    br.refill();
    bad |= br.short_of((uint32_t)nbits);
    const uint32_t cw = br.take((uint32_t)nbits);
    if (live) it.coset[tile * a.coset_words + j] = cw;
  }
  if (live && it.rice_k != nullptr) it.rice_k[tile] = (uint8_t)k;

  constexpr uint32_t kIdxBytes = WIDE ? 2u : 1u;
  constexpr uint32_t kZmax = WIDE ? 65535u : 255u;
  const auto rs = out_rsrc(it.idx + wave_tile0 * N * kIdxBytes, live_in_wave * (uint32_t)N * kIdxBytes);
#pragma unroll 1
  for (int part = 0; part < N * (int)kIdxBytes / 64; ++part) {
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
      uint32_t d[4];
      next_chunk<WIDE>(br, k, kZmax, bad, d);
      st[4 * lane + ((c ^ (lane >> 2)) & 3)] = make_uint4(d[0], d[1], d[2], d[3]);
    }
    wave_lds_sync();
    // store instruction j: lane l writes chunk l & 3 of wave tile 16 j + l / 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int T = 16 * j + (lane >> 2), cc = lane & 3;
      const uint4 q = st[4 * T + ((cc ^ (T >> 2)) & 3)];
      __builtin_amdgcn_raw_buffer_store_b128((u32x4){q.x, q.y, q.z, q.w}, rs,
                                             T * N * (int)kIdxBytes + part * 64 + 16 * cc, 0, 0);
    }
    wave_lds_sync();
  }
  bad |= br.overran();
}

template <int N, bool WIDE>
__global__ __launch_bounds__(kUnpackBlock) void unpack_kernel(UnpackLaunch a) {
  __shared__ uint32_t seg[kUnpackBlock / 64][kSegWords];
  __shared__ uint4 stage[kUnpackBlock / 64][256];   // per wave: 4 chunks of 64 tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the launch's waves run over its items in order, 64 tiles each
  const int64_t gw = (int64_t)blockIdx.x * (kUnpackBlock / 64) + wave;
  if (gw >= a.n_waves) return;   // whole waves only
  int item = 0;
#pragma unroll
  for (int k = 1; k < kUnpackMaxItems; ++k)
    if (k < a.n && gw >= a.it[k].wave0) item = k;
  item = __builtin_amdgcn_readfirstlane(item);
  const UnpackItem& it = a.it[item];
  const int64_t wave_tile0 = (gw - it.wave0) * 64;
  const int64_t tile = wave_tile0 + lane;
  const bool live = tile < it.n_tiles;
  const int64_t rem_tiles = it.n_tiles - wave_tile0;
  const uint32_t live_in_wave = (uint32_t)(rem_tiles < 64 ? rem_tiles : 64);

  bool bad = false;
  uint64_t w0 = 0, w1 = 0;
  if (live) {
    w0 = it.tile_word_offset[tile];
    w1 = it.tile_word_offset[tile + 1];
    if (w1 < w0) {
      bad = true;
      w1 = w0;
    }
  }
  // When every range is in order, the wave's words [first start, last end)
  // are exactly the union of its tiles' ranges; if they fit, they are staged
  // in LDS and the whole wave decodes from there.
  const uint64_t seg_base = it.tile_word_offset[wave_tile0];
  const uint64_t seg_end = it.tile_word_offset[wave_tile0 + live_in_wave];
  const bool staged = !__any(bad) && seg_end >= seg_base &&
                      seg_end - seg_base <= (uint64_t)kSegWords;   // uniform
  const lds_u32* sw = (const lds_u32*)seg[wave];
  const uint32_t nw = staged ? (uint32_t)(seg_end - seg_base) : 0u;
  if (staged) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(it.stream) + seg_base,
                                                      (short)0, (int)(nw * 4u), 0x00020000);
    for (uint32_t j = 0; j < nw; j += 64)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(seg[wave] + j), 4,
                                               (int)((j + (uint32_t)lane) * 4u), 0, 0, 0);
    // the copies land in LDS before any lane reads them
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    wave_lds_sync();
    WinReader br;
    br.init(sw, (uint32_t)(w0 - seg_base), (uint32_t)(w1 - seg_base), nw > 0 ? nw : 1u);
    br.zor_mask = WIDE ? 0xFFFFu : 0xFFu;
    decode_tiles<N, WIDE>(a, it, br, tile, live, wave_tile0, live_in_wave, lane, stage[wave], bad);
  } else {
    BitReader<false> br;
    br.init(it.stream, sw, seg_base, w0, w1);
    decode_tiles<N, WIDE>(a, it, br, tile, live, wave_tile0, live_in_wave, lane, stage[wave], bad);
  }
  if (live && bad) set_status(a.status, HQ_ST_CORRUPT);
}

template <bool WIDE>
void launch_unpack_w(const UnpackLaunch& a, int64_t blocks, hipStream_t s) {
  switch (a.tile) {
    case 64:
      hipLaunchKernelGGL((unpack_kernel<64, WIDE>), dim3((unsigned)blocks), dim3(kUnpackBlock), 0, s, a);
      break;
    case 128:
      hipLaunchKernelGGL((unpack_kernel<128, WIDE>), dim3((unsigned)blocks), dim3(kUnpackBlock), 0, s, a);
      break;
    case 256:
      hipLaunchKernelGGL((unpack_kernel<256, WIDE>), dim3((unsigned)blocks), dim3(kUnpackBlock), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((unpack_kernel<512, WIDE>), dim3((unsigned)blocks), dim3(kUnpackBlock), 0, s, a);
  }
}

}  // namespace

hipError_t launch_unpack(const UnpackLaunch& a, hipStream_t s) {
  const int64_t blocks = (a.n_waves + kUnpackBlock / 64 - 1) / (kUnpackBlock / 64);
  if (a.wide) launch_unpack_w<true>(a, blocks, s);
  else launch_unpack_w<false>(a, blocks, s);
  return hipGetLastError();
}

}  // namespace hq

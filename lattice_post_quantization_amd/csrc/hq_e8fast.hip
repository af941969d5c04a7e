// Fast path for the headline configuration: E8, tile 256, bf16 weights in,
// bf16 or fp32 weights out, no dither.  Same results as the generic kernels,
// bit for bit; laid out for gfx950.
//
// Passages: [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal
// Quantization Pipeline ..." ideas (i)-(iii); [ICLR abstract] "HyperQuant: A
// Near-Entropy-Optimal Lattice Quantization Pipeline ..." (Walsh-Hadamard
// rotation per tile, E8 by default, lossless strip, Rice code, algebraic
// decoding).
//
// Work mapping.  A wave holds 16 tiles.  Lane (t, r) = lane t + 16 r of the
// wave holds elements [64 r, 64 r + 64) of tile t, so a tile spans the four
// 16-lane rows and every lane keeps 64 elements in registers.  Element bits
// 0-5 are register bits: six Walsh-Hadamard stages run inside the lane.
// Element bits 6 and 7 are the row bits; v_permlane16_swap / v_permlane32_swap
// exchange a row bit with a register bit (one instruction per dword pair),
// after which those two stages also run in registers.  Reductions over a tile
// use the same swaps.  No LDS traffic apart from a 512-byte sign table.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_lanes.h"

namespace hq {
namespace {

using namespace fastlib;

// Coalesced store of a group's output.  Lane (t, r) holds CPL 16-byte chunks
// of tile t, chunk k at 16-byte slot s_k of its tile (tiles are 64 CPL bytes
// apart), and the wave writes them, 4 KB (256 chunks) per pass, into a 4 KB
// LDS buffer, then reads them back so that each store instruction covers
// 1 KB of contiguous output.  Chunk c of a pass sits at LDS slot
// c ^ ((c >> 4) & 15), which spreads a pass's accesses over the banks.  With
// the slots used here that position is a per-lane base XOR a constant of the
// chunk (write: wb ^ wx(k), passed in), and the read of pass slot 64 i + lane
// is at rb ^ 68 i with rb = 16 r + (t ^ r): one XOR per access.  The slots
// let a lane keep the element order its transform left: chunks land at their
// natural positions without lane exchanges.
template <int CPL, typename WX>
__device__ inline void store_group(__amdgpu_buffer_rsrc_t rs, const uint4* chunk, uint4* ost,
                                   int t, int lane, uint32_t wb, WX wx, uint32_t rb) {
  constexpr int kTilesPerPass = 256 / (4 * CPL);
#pragma unroll
  for (int h = 0; h < 16 / kTilesPerPass; ++h) {
    wave_lds_sync();
    if (t / kTilesPerPass == h) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) ost[wb ^ wx(k)] = chunk[k];
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = ost[rb ^ (68u * i)];
      store16(rs, (uint32_t)(h * 4096 + 1024 * i + 16 * lane), q.x, q.y, q.z, q.w);
    }
  }
}

__device__ inline uint32_t store_read_base(int t, int row) {
  return (uint32_t)(16 * row + (t ^ row));
}

// Staged loads.  A wave's 16 tiles are 8 KB of contiguous bf16, read with
// eight direct-to-LDS loads of 1 KB each (instruction k covers tiles 2k and
// 2k + 1, so every load is fully coalesced).  Lane l = 16 r + b of
// instruction k fetches row r, 16-byte chunk j = (b/2) ^ k of tile
// 2k + (b & 1) and the hardware stores it at LDS slot 64 k + l; lane (t, r)
// later finds chunk j of its tile at slot e0 ^ 2j, e0 = 64 (t/2) + 16 r + t,
// so each 16-lane row reads 16 different bank groups.
// With a caller-supplied scale, a ninth load brings the group's 16 scales to
// the 256 bytes after the bf16 data (lanes 16-63 repeat them).  Lane offsets
// are relative to the group's first tile; tiles past the end read as zeros.
constexpr int kEncStage = 512 + 16;   // uint4 per wave

__device__ inline void enc_prefetch(const EncItem& it, int64_t group, uint4* buf, int lane,
                                    bool scale_in) {
  const int r = lane >> 4, b = lane & 15;
  const uint32_t live = live_tiles(it.n_tiles, group);
  // bytes past the group's live tiles read as zero (their results are dropped)
  const auto rs = out_rsrc(static_cast<uint16_t*>(const_cast<void*>(it.x)) + group * 16 * 256,
                           live * 512u);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int j = (b >> 1) ^ k;
    const int off = (2 * k + (b & 1)) * 512 + r * 128 + j * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, off, 0, 0, 0);
  }
  if (scale_in)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(out_rsrc(it.scale + group * 16, live * 4u),
                                             lds_ptr(buf + 512), 4, b * 4, 0, 0, 0);
}

__device__ inline void enc_take(const uint4* buf, int t, int r, uint32_t* w, float& scale) {
  const uint32_t e0 = (uint32_t)(64 * (t >> 1) + 16 * r + t);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 q = buf[e0 ^ (2u * j)];
    w[4 * j] = q.x; w[4 * j + 1] = q.y; w[4 * j + 2] = q.z; w[4 * j + 3] = q.w;
  }
  scale = reinterpret_cast<const float*>(buf + 512)[t];
}

// Per-tile results are written by the 16 lanes of row 0; other lanes get an
// offset past the end of the buffer, which the hardware drops.
__device__ inline uint32_t row0_offset(int t, int row, int size) {
  return row == 0 ? (uint32_t)(t * size) : 0x40000000u;
}

// E8 decisions of a lane's 64 rotated values (eight blocks) at grid factor
// K: the stored integers as 16 dwords of int8 (block blk in dwords 2 blk,
// 2 blk + 1) and the coset bit of block blk at bit blk.  Grid values
// |S K| <= 124 2^24 (no tile of the wave past the clamp).  Lanes with live
// false skip the search of boundary blocks (their results are not used).
__device__ inline uint32_t e8_lane(const double* v, double K, uint32_t* packed, bool live) {
  uint32_t cb = 0, ties = 0;
  int32_t U[64];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // one rounding of the exact product: RN(S K + 1.5 2^52)
      const double m = __fma_rn(v[8 * blk + i], K, kMagic);
      U[8 * blk + i] = (int32_t)(uint32_t)(uint64_t)__double_as_longlong(m);
    }
    int c;
    ties |= e8_block_fast(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1], c) << blk;
    cb |= (uint32_t)c << blk;
  }
  if (ties && live) {
    // blocks with a coordinate exactly on a rounding boundary
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      if ((ties >> blk) & 1u) {
        const int c = e8_block_exact(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1]);
        cb = (cb & ~(1u << blk)) | ((uint32_t)c << blk);
      }
    }
  }
  return cb;
}

// Rice parameter and payload bits of the tile whose indices the four rows'
// lanes hold (16 dwords of int8 each).  k = argmin_k L(k),
// L(k) = Q_k + 256 (1 + k), Q_k = sum floor(zeta / 2^k).  L is convex:
// L(k+1) - L(k) = 256 - D_k with D_k = Q_k - Q_{k+1} = sum floor((zeta +
// 2^k) / 2^(k+1)), which falls with k, so the first minimum is the smallest
// k with D_k <= 256.  D_k lies within 128 of S / 2^(k+1) (S = sum zeta), so
// with kt the smallest k with S <= 256 * 2^(k+1): D_{kt+1} <= 256, and
// D_k > 256 for k <= kt - 2 (strictly, so no smaller k ties).  Only
// kt - 1, kt, kt + 1 remain.
// Value of the lane in the same row with the neighbouring tile index
// (lane ^ 1): the other half of a 512-element tile.
__device__ inline uint32_t pair_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

__device__ inline double pair_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = pair_u32((uint32_t)u), hi = pair_u32((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Sum over the lanes that hold one tile: the four rows of lane t for
// N = 256, and of lanes t and t ^ 1 for N = 512.
template <int N>
__device__ inline uint32_t tile_total_u32(uint32_t v) {
  v = tile_sum_u32(v);
  if constexpr (N == 512) v += pair_u32(v);
  return v;
}

template <int N>
__device__ inline uint32_t rice_tile(const uint32_t* packed, int& bk) {
  static_assert(N == 256 || N == 512, "tile 256 or 512");
  constexpr int kLog2N = N == 256 ? 8 : 9;
  uint32_t zz[16];
  uint32_t S = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    zz[q] = zigzag4(packed[q]);
    S = byte_sum(zz[q], S);
  }
  S = tile_total_u32<N>(S);
  // kt = min(8, smallest k with S <= N 2^(k + 1)); S <= 255 N
  int kt = S <= 2u * N ? 0 : 31 - kLog2N - (int)__builtin_clz(S - 1u);
  kt = kt > 8 ? 8 : kt;
  // The candidates k0, k0 + 1, k0 + 2 with k0 = min(max(kt - 1, 0), 6)
  // contain kt - 1 .. kt + 1 within [0, 8]; the extra one (k0 + 2 when
  // kt = 0, k0 when kt = 8) is never strictly better than those.
  // R_k = sum (zeta mod 2^k): R_k0 directly; with x = zeta & (3 << k0)
  // bytewise, sum x = 2^k0 (C0 + 2 C1) and popcount x = C0 + C1 (C0, C1 the
  // counts of set bits k0, k0 + 1), so R_k0+1 = R_k0 + 2^k0 C0 and
  // R_k0+2 = R_k0+1 + 2^(k0+1) C1.
  const int k0 = kt - 1 < 0 ? 0 : (kt - 1 > 6 ? 6 : kt - 1);
  const uint32_t mlo = ((1u << k0) - 1u) * 0x01010101u;
  const uint32_t m2 = (3u << k0) * 0x01010101u;
  uint32_t r0 = 0, sx = 0, cx = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    r0 = byte_sum(zz[q] & mlo, r0);
    const uint32_t x = zz[q] & m2;
    sx = byte_sum(x, sx);
    cx += (uint32_t)__builtin_popcount(x);
  }
  r0 = tile_total_u32<N>(r0);
  sx = tile_total_u32<N>(sx);
  cx = tile_total_u32<N>(cx);
  const uint32_t c1 = (sx >> k0) - cx, c0 = cx - c1;
  const uint32_t R[3] = {r0, r0 + (c0 << k0), r0 + (c0 << k0) + (c1 << (k0 + 1))};
  uint32_t best = 0xFFFFFFFFu;
  bk = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int k = k0 + j;
    const uint32_t L = ((S - R[j]) >> k) + (uint32_t)N * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }
  return best;
}

__device__ inline double tile_max_f64(double v) {
  double a = v, b = v;
  swap_f64<false>(a, b);
  v = fmax(a, b);
  a = v;
  b = v;
  swap_f64<true>(a, b);
  return fmax(a, b);
}

// Per-tile rate control (reading R7: the finest bf16 scale, by bisection on
// its bit pattern within eight binades of the automatic one, at which the
// tile's indices stay inside the grid's clamp, hence int8, and its bits fit
// floor(R n)).  The probes of every tile follow the same rule as the
// generic kernel's; a probe whose largest grid value would pass the clamp
// (rne(max|S| K) > 124 2^24, the largest of the generic kernel's clamped
// values) is infeasible without a decision.  Returns the chosen scale
// (delta unchanged for a tile that is not searched).
__device__ inline float rc_search(const EncodeLaunch& a, const double* v, double ss, float delta,
                                  bool searched) {
  double m = 0.0;
#pragma unroll
  for (int i = 0; i < 64; ++i) m = fmax(m, fabs(v[i]));
  const double vmax = tile_max_f64(m);
  const int32_t ac = (int32_t)(__float_as_uint(delta) >> 16);
  int32_t lo = ac - kRcSpan > 0x0080 ? ac - kRcSpan : 0x0080;
  int32_t hi = ac + kRcSpan < 0x7F7F ? ac + kRcSpan : 0x7F7F;
  int32_t probe = hi;
  bool top = true, active = searched && ss > 0.0;
  while (__builtin_amdgcn_ballot_w64(active) != 0) {
    const double tq = a.sqrt_n * (double)__uint_as_float((uint32_t)probe << 16);
    const double K = 16777216.0 / tq;
    // (lanes of finished tiles and of probes past the clamp decide on
    // values whose results are not used)
    const bool in_range = rne_product(vmax, K) <= kUClamp;
    uint32_t packed[16];
    (void)e8_lane(v, K, packed, active && in_range);
    int bk;
    const uint32_t bits = 4u + 32u + rice_tile<256>(packed, bk);
    const bool f = in_range && bits <= a.rc_budget;
    if (active) {
      if (top && !f) {
        active = false;
      } else {
        if (!top) (f ? hi : lo) = probe;
        if (hi - lo <= 1) active = false;
        probe = (lo + hi) / 2;
      }
      top = false;
    }
  }
  return searched && ss > 0.0 ? __uint_as_float((uint32_t)hi << 16) : delta;
}

// One group of 16 tiles held by a wave (w: this lane's 64 bf16 of its tile).
// (scale_in: the caller's scale of this lane's tile when not automatic.)
// RC: per-tile rate control (auto scales only).
// N = 512: the wave holds 8 tiles; tile t / 2 of the group is held as its
// halves t (elements 256 (t & 1) + [0, 256)), each laid out as a tile of
// 256, so the loads, the index stores and the coset words (one per half)
// are those of 16 tiles of 256; element bit 8 is the lane's t & 1, and its
// butterfly runs between lanes t and t ^ 1.
template <bool RC, int N = 256>
__device__ inline void enc_group(const EncodeLaunch& a, const EncItem& it, const uint32_t* sign_tab,
                                 int64_t group, int t, int row, const uint32_t* w, float scale_in,
                                 uint4* ost) {
  static_assert(N == 256 || (N == 512 && !RC), "tile 256, or 512 without rate control");
  const uint4* st = reinterpret_cast<const uint4*>(
      sign_tab + (N == 512 ? (4 * (t & 1) + row) : row) * 32);
  double v[64];
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint4 m = st[k];
    const uint32_t mm[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t d = w[4 * k + j] ^ mm[j];
      const double lo = (double)__uint_as_float(d << 16);
      const double hi = (double)__uint_as_float(d & 0xFFFF0000u);
      v[8 * k + 2 * j] = lo;
      v[8 * k + 2 * j + 1] = hi;
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }

  // ---- scale: bf16_rne(rms * c) (auto) or the caller's; the norm bound
  // sqrt(sum x^2)/Delta < 126 keeps every grid value in range
  ss = tile_sum_f64(ss);
  if constexpr (N == 512) ss = ss + pair_f64(ss);
  uint32_t status = 0;
  float delta;
  if (a.auto_scale) {
    delta = bf16_round_to_f32(sqrt(ss / (double)N) * a.c);
    if (delta == 0.0f) delta = 1.0f;
  } else {
    delta = scale_in;
    if (!(delta > 0.0f) || !isfinite(delta)) status |= HQ_ST_NONFINITE;
  }
  if (!isfinite(ss)) status |= HQ_ST_NONFINITE;
  // |u_i| <= sqrt(sum x^2) / Delta: below 124 no grid value reaches the clamp
  bool big = !(sqrt(ss) < 124.0 * (double)delta);
  double K = 16777216.0 / (a.sqrt_n * (double)delta);

  // ---- Walsh-Hadamard: element bits 0-5 in registers
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (!(i & h)) {
        const double x = v[i], y = v[i + h];
        v[i] = x + y;
        v[i + h] = x - y;
      }
    }
  }
  // Element bits 4, 5 (register bits 4, 5) trade places with element bits
  // 6, 7 (the row bits) through the wave's 4 KB output buffer, in eight
  // rounds of one register pair (element bits 0-3 = 2q, 2q + 1): lane (t, r)
  // sends register 2q + {0, 1} + 16 i4 + 32 i5 to row i5 + 2 i4 of its tile,
  // which keeps it as register 2q + {0, 1} + 16 r1 + 32 r0.  16-byte slot
  // (16 t + 4 (destination row) + (source row)) ^ t: the 16 lanes of a row
  // hit 16 different bank groups.  LDS instructions take no VALU slots.
  {
    const uint32_t ot = (uint32_t)t;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      wave_lds_sync();
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int i4 = x & 1, i5 = x >> 1;
        const int j = 2 * q + 16 * i4 + 32 * i5;
        const uint64_t lo = (uint64_t)__double_as_longlong(v[j]);
        const uint64_t hi = (uint64_t)__double_as_longlong(v[j + 1]);
        ost[(16 * ot + 4 * (uint32_t)(i5 + 2 * i4) + (uint32_t)row) ^ ot] =
            make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
      }
      wave_lds_sync();
#pragma unroll
      for (int src = 0; src < 4; ++src) {
        const uint4 d = ost[(16 * ot + 4 * (uint32_t)row + (uint32_t)src) ^ ot];
        const int j = 2 * q + 16 * (src >> 1) + 32 * (src & 1);
        v[j] = __longlong_as_double((long long)(((uint64_t)d.y << 32) | d.x));
        v[j + 1] = __longlong_as_double((long long)(((uint64_t)d.w << 32) | d.z));
      }
    }
    wave_lds_sync();
  }
  // butterflies on element bit 6 (register bit 5) and bit 7 (register bit 4)
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double x = v[i], y = v[i + 32];
    v[i] = x + y;
    v[i + 32] = x - y;
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (!(i & 16)) {
      const double x = v[i], y = v[i + 16];
      v[i] = x + y;
      v[i + 16] = x - y;
    }
  }
  if constexpr (N == 512) {
    // element bit 8 (the lane's t & 1): x + y in the lower half's lane,
    // x - y in the upper half's (one rounding each, as the sums)
    const double sg = (t & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = fma(v[i], sg, pair_f64(v[i]));
  }
  // Now register i holds element bits (i0 i1 i2 i3 | i4 = b7 | i5 = b6) and the
  // lane's row bits hold (r0 = b5, r1 = b4).
  if constexpr (RC) {
    delta = rc_search(a, v, ss, delta, status == 0u);
    big = !(sqrt(ss) < 124.0 * (double)delta);
    K = 16777216.0 / (a.sqrt_n * (double)delta);
  }

  // When some tile of the wave may pass the clamp, the generic encoder's
  // clamped rne(S K) replaces S (and K becomes 1).
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      double q = rne_product(v[i], K);
      if (!(fabs(q) <= kUClamp)) {
        status |= HQ_ST_OVERFLOW;
        q = (q > 0.0) ? kUClamp : -kUClamp;
      }
      v[i] = q;
    }
    K = 1.0;
  }

  // ---- quantizer input U = rne(S K) (units of 2^-24), stored integers
  uint32_t packed[16];
  const uint32_t cb = e8_lane(v, K, packed, true);
  const int r0 = row & 1, r1 = row >> 1;
  // tile block index of register block blk = b3 + 2 b4 + 4 b5 + 8 b6 + 16 b7
  uint32_t cbits = 0;
#pragma unroll
  for (int blk = 0; blk < 8; ++blk)
    cbits |= ((cb >> blk) & 1u)
             << ((blk & 1) + 2 * r1 + 4 * r0 + 8 * (blk >> 2) + 16 * ((blk >> 1) & 1));
  const uint32_t coset_word = tile_or_u32(cbits);

  // ---- Rice parameter: k = argmin_k L(k), L(k) = Q_k + 256 (1 + k),
  // Q_k = sum floor(zeta / 2^k).  L is convex: L(k+1) - L(k) = 256 - D_k with
  // D_k = Q_k - Q_{k+1} = sum floor((zeta + 2^k) / 2^(k+1)), which falls
  // with k, so the first minimum is the smallest k with D_k <= 256.  D_k lies
  // within 128 of S / 2^(k+1) (S = sum zeta), so with kt the smallest k with
  // S <= 256 * 2^(k+1): D_{kt+1} <= 256, and D_k > 256 for k <= kt - 2
  // (strictly, so no smaller k ties).  Only kt - 1, kt, kt + 1 remain.
  int bk;
  const uint32_t best = rice_tile<N>(packed, bk);

  // ---- store.  Chunk k (blocks 2k, 2k + 1: element bits 0-3 inside) has
  // element bit 7 = k bit 0, bit 6 = k bit 1, bit 5 = row bit 0 and bit 4 =
  // row bit 1, i.e. 16-byte slot 8 k0 + 4 k1 + 2 r0 + r1 of the tile.
  const uint32_t live = live_tiles(it.n_tiles, group);
  const int64_t tile0 = group * 16;
  uint4 ch[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    ch[k] = make_uint4(packed[4 * k], packed[4 * k + 1], packed[4 * k + 2], packed[4 * k + 3]);
  // pass slot c = 16 t + s_k, (c >> 4) & 15 = t: position (16 t + ((2 r0 + r1) ^ t)) ^ (8 k0 + 4 k1)
  const uint32_t wb = (uint32_t)(16 * t + ((2 * (row & 1) + (row >> 1)) ^ t));
  store_group<4>(out_rsrc(it.idx + tile0 * 256, live * 256u), ch, ost, t, row * 16 + t, wb,
                 [](int k) { return (uint32_t)(8 * (k & 1) + 4 * (k >> 1)); },
                 store_read_base(t, row));
  __builtin_amdgcn_raw_buffer_store_b32(coset_word, out_rsrc(it.coset + tile0, live * 4u),
                                        (int)row0_offset(t, row, 4), 0, 0);
  if constexpr (N == 256) {
    if (a.auto_scale)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), out_rsrc(it.scale + tile0, live * 4u),
                                            (int)row0_offset(t, row, 4), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bk, out_rsrc(it.rice_k + tile0, live),
                                         (int)row0_offset(t, row, 1), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(4u + 32u + best, out_rsrc(it.tile_bits + tile0, live * 4u),
                                          (int)row0_offset(t, row, 4), 0, 0);
  } else {
    // per-tile results of tile t / 2, from the lower half's lane of row 0
    const uint32_t lt = live / 2;
    const int64_t T0 = tile0 / 2;
    const int tr = (t & 1) ? 1 : row;
    if (a.auto_scale)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), out_rsrc(it.scale + T0, lt * 4u),
                                            (int)row0_offset(t >> 1, tr, 4), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bk, out_rsrc(it.rice_k + T0, lt),
                                         (int)row0_offset(t >> 1, tr, 1), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(4u + 64u + best, out_rsrc(it.tile_bits + T0, lt * 4u),
                                          (int)row0_offset(t >> 1, tr, 4), 0, 0);
  }
  if (status && (uint32_t)t < live) set_status(a.status, status);
}

// Persistent waves: each wave walks groups of 16 tiles with a grid-wide
// stride; the next group streams into the wave's LDS buffer while the
// current one is computed.
// The loop body ends with reading the next group from LDS, after this
// group's stores; the last iteration prefetches its own group again (an L2
// hit) so that no branch surrounds the memory operations.
// Sign table of a 512-element tile: entry i holds the bf16-pair XOR mask
// of elements 2 i, 2 i + 1 (rows of 32 entries: half h, row r at 4 h + r).
__device__ inline void fill_sign_table512(uint32_t* tab, const uint32_t* signs) {
  for (int i = threadIdx.x; i < 256; i += kBlock) {
    const int e = 2 * i;
    const uint32_t w0 = signs[e >> 5];
    const uint32_t b0 = (w0 >> (e & 31)) & 1u, b1 = (w0 >> ((e + 1) & 31)) & 1u;
    tab[i] = (b0 << 15) | (b1 << 31);
  }
}

template <bool RC, int N = 256>
__device__ __attribute__((always_inline)) inline void encode_body(const EncodeLaunch& a,
                                                                  const EncBatch& b) {
  __shared__ uint32_t sign_tab[N / 2];
  __shared__ uint4 stage[kBlock / 64][kEncStage];
  __shared__ uint4 ostage[kBlock / 64][256];
  if constexpr (N == 512)
    fill_sign_table512(sign_tab, a.signs);
  else
    fill_sign_table(sign_tab, a.signs);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, row = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* buf = stage[wave];
  const bool scale_in = !a.auto_scale;
  const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
  int64_t g = (int64_t)blockIdx.x * (kBlock / 64) + wave;
  if (g >= b.n_groups) return;
  int ic = item_of(b, g);
  uint32_t w[32];
  float sc;
  enc_prefetch(b.it[ic], g - b.it[ic].group0, buf, lane, scale_in);
  enc_take(buf, t, row, w, sc);
  for (;;) {
    // every lane's reads of the buffer complete before it is refilled
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t gn = g + stride;
    const bool more = gn < b.n_groups;   // uniform across the wave
    const int64_t gp = more ? gn : g;
    const int ip = more ? item_from(b, ic, gn) : ic;
    enc_prefetch(b.it[ip], gp - b.it[ip].group0, buf, lane, scale_in);
    enc_group<RC, N>(a, b.it[ic], sign_tab, g - b.it[ic].group0, t, row, w, sc, ostage[wave]);
    __builtin_amdgcn_sched_barrier(0);
    enc_take(buf, t, row, w, sc);
    if (!more) break;
    g = gn;
    ic = ip;
  }
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void encode_e8_fast(EncodeLaunch a, EncBatch b) {
  encode_body<false>(a, b);
}

// Tiles of 512 (auto scale): items counted in halves of 256.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void encode_e8_fast512(EncodeLaunch a, EncBatch b) {
  encode_body<false, 512>(a, b);
}

// With the per-tile rate control a lane keeps its 64 rotated values through
// every probe: one wave per SIMD, so that they stay in registers.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(1, 1))) void encode_e8_fast_rc(EncodeLaunch a, EncBatch b) {
  encode_body<true>(a, b);
}

// ------------------------------------------------------------------ decode
// Integer Hadamard on P = 2p in packed int16 pairs (2 elements per register);
// exact while sum |P| <= 32767, which every tile of encoder output satisfies
// (|P_i| stays far below that bound); otherwise the tile runs the same
// transform in fp32 (exact for |values| < 2^24).  Then
// x = s * (H P) * (Delta / 32) is exact in fp32 and rounded once to the output.

// Staged loads as in the encoder: a wave's 16 tiles are 4 KB of int8
// indices, four 1 KB direct-to-LDS loads (instruction k covers tiles 4k ..
// 4k + 3).  Lane l = 16 r + b of instruction k fetches row r, chunk
// j = (b/4) ^ k of tile 4k + (b & 3) into slot 64 k + l; lane (t, r) reads
// chunk j of its tile from slot d0 ^ 4j, d0 = 64 (t/4) + 16 r + t.
// Two more loads bring the group's coset words and scales (lanes 0-15; the
// other lanes repeat them) to the 512 bytes after the indices.
constexpr int kDecStage = 256 + 32;   // uint4 per wave

struct DecIn {
  uint32_t cw;
  float scale;
};

template <int N = 256>
__device__ inline void dec_prefetch(const DecItem& it, int64_t group, uint4* buf, int lane) {
  const int r = lane >> 4, b = lane & 15;
  const uint32_t live = live_tiles(it.n_tiles, group);
  const auto rs = out_rsrc(const_cast<int8_t*>(it.idx) + group * 16 * 256, live * 256u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = (b >> 2) ^ k;
    const int off = (4 * k + (b & 3)) * 256 + r * 64 + j * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, off, 0, 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      out_rsrc(const_cast<uint32_t*>(it.coset) + group * 16, live * 4u), lds_ptr(buf + 256), 4,
      b * 4, 0, 0, 0);
  if constexpr (N == 512) {
    // one scale per 512-tile (two halves): slot b holds the scale of tile b / 2
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        out_rsrc(const_cast<float*>(it.scale) + group * 8, live * 2u), lds_ptr(buf + 272), 4,
        (b >> 1) * 4, 0, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        out_rsrc(const_cast<float*>(it.scale) + group * 16, live * 4u), lds_ptr(buf + 272), 4,
        b * 4, 0, 0, 0);
  }
}

__device__ inline void dec_take(const uint4* buf, int t, int r, uint32_t* d, DecIn& in) {
  const uint32_t d0 = (uint32_t)(64 * (t >> 2) + 16 * r + t);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 q = buf[d0 ^ (4u * j)];
    d[4 * j] = q.x; d[4 * j + 1] = q.y; d[4 * j + 2] = q.z; d[4 * j + 3] = q.w;
  }
  in.cw = reinterpret_cast<const uint32_t*>(buf + 256)[t];
  in.scale = reinterpret_cast<const float*>(buf + 272)[t];
}

// N = 512: the group's 16 tiles are the two halves of 8 tiles of 512 (half
// h of tile T on lanes t = 2T + h), each half unstripped and transformed
// as a tile of 256; element bit 8 is then one butterfly with the value of
// the neighbouring lane (inv = fp64 1/sqrt(512)).
template <bool OUT_BF16, int N = 256>
__device__ inline void dec_group(const DecItem& it, const uint32_t* sign_tab, int64_t group, int t,
                                 int row, const uint32_t* d, const DecIn& in, uint4* ost,
                                 double inv = 0.0) {
  static_assert(N == 256 || N == 512, "tile of 256 or 512");
  const uint32_t cw = in.cw >> (8 * row);        // this lane's 8 blocks
  const float dsc = in.scale * 0.03125f;         // Delta / 32, exact

  // bound for the int16 path: sum |P| <= 4 sum|stored| + 320 (|z7| <= 2|t7| + 1).
  // For a signed byte z held as the unsigned byte u, |u - 128| = 128 - |z|,
  // so the tile's sum of |u - 128| over its 256 bytes is 32768 - sum |z|.
  uint32_t sad = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) sad = __builtin_amdgcn_sad_u8(d[q], 0x80808080u, sad);
  sad = tile_sum_u32(sad);
  // N = 512: 64 blocks, sum |P| <= 4 sum |stored| + 640; 65536 - sum |z| over 512 bytes
  if constexpr (N == 512) sad += pair_u32(sad);
  const bool small = N == 256 ? sad >= 32768u - 8111u : sad >= 65536u - 8031u;

  // ---- unstrip into P = 2z + c as int16 pairs: P2[m] = (P_2m, P_2m+1)
  uint32_t P2[32];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t d0 = d[2 * b], d1 = d[2 * b + 1];
    uint32_t x = d0 ^ (d1 & 0x00FFFFFFu);
    x ^= x >> 16;
    x ^= x >> 8;
    const uint32_t par = x & 1u;
    const uint32_t c = (cw >> b) & 1u;
    // sign-extended int16 pairs (z0,z1) (z2,z3) from d0 and (z4,z5) (z6,t7) from d1
    const uint32_t e0 = d0 << 8, e1 = d1 << 8;
    const uint32_t p01 = __builtin_amdgcn_perm(d0, e0, 0x0A050804u);
    const uint32_t p23 = __builtin_amdgcn_perm(d0, e0, 0x0B070906u);
    const uint32_t p45 = __builtin_amdgcn_perm(d1, e1, 0x0A050804u);
    const uint32_t p67 = __builtin_amdgcn_perm(d1, e1, 0x0B070906u);
    const uint32_t cc = c * 0x00010001u;
    // z7 = 2 t7 + par: P7 = 4 t7 + 2 par + c
    const uint32_t c7 = cc + (par << 17);
    P2[4 * b] = pk_mad_u16(p01, 0x00020002u, cc);
    P2[4 * b + 1] = pk_mad_u16(p23, 0x00020002u, cc);
    P2[4 * b + 2] = pk_mad_u16(p45, 0x00020002u, cc);
    P2[4 * b + 3] = pk_mad_u16(p67, 0x00040002u, c7);
  }

  float y[64];
  if (small) {
    // element bit 0: inside each dword
#pragma unroll
    for (int m = 0; m < 32; ++m) P2[m] = half_butterfly(P2[m]);
    // element bits 1-5: dword index bits 0-4
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        if (!(m & h)) {
          const s16x2 x = as_s16x2(P2[m]), z = as_s16x2(P2[m + h]);
          P2[m] = as_u32(x + z);
          P2[m + h] = as_u32(x - z);
        }
      }
    }
    // element bit 6 (row bit 0) <-> dword bit 4; element bit 7 (row bit 1) <-> dword bit 3
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      swap16(P2[m], P2[m + 16]);
      const s16x2 x = as_s16x2(P2[m]), z = as_s16x2(P2[m + 16]);
      P2[m] = as_u32(x + z);
      P2[m + 16] = as_u32(x - z);
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      if (!(m & 8)) {
        swap32(P2[m], P2[m + 8]);
        const s16x2 x = as_s16x2(P2[m]), z = as_s16x2(P2[m + 8]);
        P2[m] = as_u32(x + z);
        P2[m + 8] = as_u32(x - z);
      }
    }
    if constexpr (N == 512) {
      // element bit 8: half 0 keeps a + b, half 1 keeps a - b (its own value
      // negated plus its neighbour's); both within int16 by the bound above
      const uint32_t sg = (t & 1) ? 0xFFFFFFFFu : 0x00010001u;
#pragma unroll
      for (int m = 0; m < 32; ++m) P2[m] = pk_mad_u16(P2[m], sg, pair_u32(P2[m]));
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      y[2 * m] = (float)(short)(P2[m] & 0xFFFFu);
      y[2 * m + 1] = (float)((int32_t)P2[m] >> 16);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      y[2 * m] = (float)(short)(P2[m] & 0xFFFFu);
      y[2 * m + 1] = (float)((int32_t)P2[m] >> 16);
    }
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        if (!(i & h)) {
          const float x = y[i], z = y[i + h];
          y[i] = x + z;
          y[i + h] = x - z;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t p = __float_as_uint(y[i]), q = __float_as_uint(y[i + 32]);
      swap16(p, q);
      const float x = __uint_as_float(p), z = __uint_as_float(q);
      y[i] = x + z;
      y[i + 32] = x - z;
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (!(i & 16)) {
        uint32_t p = __float_as_uint(y[i]), q = __float_as_uint(y[i + 16]);
        swap32(p, q);
        const float x = __uint_as_float(p), z = __uint_as_float(q);
        y[i] = x + z;
        y[i + 16] = x - z;
      }
    }
    if constexpr (N == 512) {
      // exact: |sums| <= 512 (4 * 128 + 3) < 2^24
      const float sgf = (t & 1) ? -1.0f : 1.0f;
#pragma unroll
      for (int i = 0; i < 64; ++i)
        y[i] = __builtin_fmaf(y[i], sgf, __uint_as_float(pair_u32(__float_as_uint(y[i]))));
    }
  }
  // Register i now holds element bits (i0 .. i3, i4 = b7, i5 = b6); rows (b5, b4),
  // as the exact integer (H P)_e.

  // ---- x = (H P)_e Delta / 32.  fp32 output: one rounding of the exact
  // product.  bf16 output: the fp32 product is exact for a bf16-valued scale
  // (|H P| < 2^16 times 8 significant bits) of normal magnitude, and one
  // rounding to bf16 follows; a wave with any other scale (fp32 caller
  // scales, outputs that could be subnormal) rounds from the exact fp64
  // product as the generic decoder does.
  //
  // N = 512: x = fl64(((H P)_e (Delta / 2)) inv), the first product exact
  // (an fp32 scale times at most 18 bits), the rounding of the fp64 value
  // itself.  bf16 output: rounding that fp32 value to bf16 rounds x itself
  // unless the fp32 value sits exactly on a bf16 midpoint (low 16 bits
  // 0x8000): a nearer fp32 value cannot lie past a midpoint that fp32
  // represents.  A wave with such a value, or a scale outside 2^-100 ..
  // 2^100 (outputs that could leave fp32's normal range), rounds from fp64.
  const uint32_t* stab = sign_tab + (N == 512 ? 128 * (t & 1) : 0);
  const double dh = (double)in.scale * 0.5;
  if constexpr (OUT_BF16) {
    uint32_t o[32];
    if constexpr (N == 512) {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      uint32_t key = 0xFFFFFFFFu;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float f0 = (float)(((double)y[2 * m] * dh) * inv);
        const float f1 = (float)(((double)y[2 * m + 1] * dh) * inv);
        key = min(key, min((__float_as_uint(f0) << 16) + 0x80000000u,
                           (__float_as_uint(f1) << 16) + 0x80000000u));
        const bf16x2 pr = {(__bf16)f0, (__bf16)f1};
        o[m] = __builtin_bit_cast(uint32_t, pr);
      }
      const bool fast = key != 0u && in.scale >= 0x1p-100f && in.scale <= 0x1p100f;
      if (__builtin_amdgcn_ballot_w64(!fast) != 0) {
#pragma unroll
        for (int m = 0; m < 32; ++m)
          o[m] = f64_to_bf16(((double)y[2 * m] * dh) * inv) |
                 (f64_to_bf16(((double)y[2 * m + 1] * dh) * inv) << 16);
      }
    } else {
    const bool exact32 = (__float_as_uint(in.scale) & 0xFFFFu) == 0u && in.scale >= 0x1p-100f &&
                         in.scale <= 0x1p100f;
    if (__builtin_amdgcn_ballot_w64(!exact32) == 0) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 pr = {(__bf16)(y[2 * m] * dsc), (__bf16)(y[2 * m + 1] * dsc)};
        o[m] = __builtin_bit_cast(uint32_t, pr);
      }
    } else {
      const double dd = (double)in.scale * 0.03125;
#pragma unroll
      for (int m = 0; m < 32; ++m)
        o[m] = f64_to_bf16((double)y[2 * m] * dd) | (f64_to_bf16((double)y[2 * m + 1] * dd) << 16);
    }
    }
    // Chunk k = o[4k .. 4k + 3] holds element bits 0-2 inside; bit 3 = k
    // bit 0, bit 7 = k bit 1, bit 6 = k bit 2, bit 5 = row bit 0, bit 4 = row
    // bit 1: 16-byte slot k0 + 16 k1 + 8 k2 + 4 r0 + 2 r1 of the tile.  The
    // sign masks of those elements come from the sign table of the natural
    // layout (row r, chunk j covers elements 64 r + 8 j ...).
    uint4 ch[8];
    const int rs0 = 4 * (row & 1) + 2 * (row >> 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int sl = (k & 1) + 16 * ((k >> 1) & 1) + 8 * (k >> 2) + rs0;
      const uint4 sm = reinterpret_cast<const uint4*>(stab)[sl];
      ch[k] = make_uint4(o[4 * k] ^ sm.x, o[4 * k + 1] ^ sm.y, o[4 * k + 2] ^ sm.z,
                         o[4 * k + 3] ^ sm.w);
    }
    // pass slot c = 32 a + s_k (a = t mod 8), (c >> 4) & 15 = 2a + k1:
    // position (32 a + (rs0 ^ 2a)) ^ (16 k1 + 8 k2 + (k0 ^ k1))
    const int a8 = t & 7;
    const uint32_t wb = (uint32_t)(32 * a8 + (rs0 ^ (2 * a8)));
    store_group<8>(out_rsrc(static_cast<uint16_t*>(it.y) + group * 16 * 256,
                            live_tiles(it.n_tiles, group) * 512u),
                   ch, ost, t, row * 16 + t, wb, [](int k) {
                     return (uint32_t)(16 * ((k >> 1) & 1) + 8 * (k >> 2) + ((k & 1) ^ ((k >> 1) & 1)));
                   }, store_read_base(t, row));
  } else {
    uint32_t o[64];
#pragma unroll
    for (int i = 0; i < 64; ++i)
      o[i] = N == 512 ? __float_as_uint((float)(((double)y[i] * dh) * inv))
                      : __float_as_uint(y[i] * dsc);
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (!(i & 16)) swap32(o[i], o[i + 16]);
#pragma unroll
    for (int i = 0; i < 32; ++i) swap16(o[i], o[i + 32]);
    uint4 ch[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t sm = stab[row * 32 + 2 * k], sn = stab[row * 32 + 2 * k + 1];
      ch[k] = make_uint4(o[4 * k] ^ (sm << 16), o[4 * k + 1] ^ (sm & 0x80000000u),
                         o[4 * k + 2] ^ (sn << 16), o[4 * k + 3] ^ (sn & 0x80000000u));
    }
    store_group<16>(out_rsrc(static_cast<float*>(it.y) + group * 16 * 256,
                             live_tiles(it.n_tiles, group) * 1024u),
                    // pass slot c = 64 a + 16 r + k (a = t mod 4), (c >> 4) & 15 = 4a + r:
                    // position (64 a + 16 r + (4a + r)) ^ k
                    ch, ost, t, row * 16 + t,
                    (uint32_t)(64 * (t & 3) + 16 * row + 4 * (t & 3) + row),
                    [](int k) { return (uint32_t)k; }, store_read_base(t, row));
  }
}

// Persistent waves as in the encoder.  The loop body ends with reading the
// next group from LDS, after this group's stores, so the wait for the
// prefetch never includes those stores; the last iteration prefetches its
// own group again (an L2 hit) to keep the loop free of branches around
// memory operations.
template <bool OUT_BF16, int N = 256>
__global__ __launch_bounds__(kBlock) void decode_e8_fast(DecodeLaunch a, DecBatch b) {
  __shared__ uint32_t sign_tab[N / 2];
  __shared__ uint4 stage[kBlock / 64][kDecStage];
  __shared__ uint4 ostage[kBlock / 64][256];
  if constexpr (N == 512)
    fill_sign_table512(sign_tab, a.signs);
  else
    fill_sign_table(sign_tab, a.signs);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, row = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* buf = stage[wave];
  const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
  int64_t g = (int64_t)blockIdx.x * (kBlock / 64) + wave;
  if (g >= b.n_groups) return;
  int ic = item_of(b, g);
  uint32_t d[16];
  DecIn in;
  dec_prefetch<N>(b.it[ic], g - b.it[ic].group0, buf, lane);
  dec_take(buf, t, row, d, in);
  for (;;) {
    // every lane's reads of the buffer complete before it is refilled
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t gn = g + stride;
    const bool more = gn < b.n_groups;   // uniform across the wave
    const int64_t gp = more ? gn : g;
    const int ip = more ? item_from(b, ic, gn) : ic;
    dec_prefetch<N>(b.it[ip], gp - b.it[ip].group0, buf, lane);
    dec_group<OUT_BF16, N>(b.it[ic], sign_tab, g - b.it[ic].group0, t, row, d, in, ostage[wave],
                           a.inv_sqrt_n);
    __builtin_amdgcn_sched_barrier(0);
    dec_take(buf, t, row, d, in);
    if (!more) break;
    g = gn;
    ic = ip;
  }
}

// ---------------------------------------------------------------- pipeline
// One launch that encodes one batch and decodes another, independent one
// (a model streamed through the codec: layer l + 1 is encoded while layer l
// is decoded).  Encode is bound by VALU issue and leaves most of the HBM
// bandwidth unused; decode is bound by HBM and leaves most of the VALU
// unused.  Here every wave alternates: slot s = w, w + W, ... is encode
// group s (if the encode batch has it) followed by decode group s (if the
// decode batch has it), so the two waves of a SIMD are usually in different
// phases and both resources stay busy.  The next item streams into the
// wave's LDS buffer while the current one is computed, as in the separate
// kernels; the group bodies are the same functions, so the results are bit
// for bit those of the two separate launches.  The caller guarantees that
// no decode input is written by the encode.
struct PipeItem {
  int64_t slot;
  int kind;   // 0: encode group `slot`, 1: decode group `slot`, -1: none
};

// This lane's index in the wave, recomputed where it is called (an asm the
// compiler may neither hoist nor merge).
__device__ inline int opaque_lane_id() {
  int v;
  __asm__ volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

__device__ inline PipeItem pipe_first(int64_t s, int64_t ne, int64_t nd) {
  if (s < ne) return {s, 0};
  if (s < nd) return {s, 1};
  return {s, -1};
}

__device__ inline PipeItem pipe_next(PipeItem c, int64_t stride, int64_t ne, int64_t nd) {
  if (c.kind == 0 && c.slot < nd) return {c.slot, 1};
  return pipe_first(c.slot + stride, ne, nd);
}

// The encode stage (528 uint4 per wave) also holds a decode group (288).
template <bool OUT_BF16>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void codec_e8_fast(
    EncodeLaunch a, EncBatch b, DecodeLaunch ad, DecBatch bd) {
  __shared__ uint32_t sign_enc[128];
  __shared__ uint32_t sign_dec[128];
  __shared__ uint4 stage[kBlock / 64][kEncStage];
  __shared__ uint4 ostage[kBlock / 64][256];
  fill_sign_table(sign_enc, a.signs);
  fill_sign_table(sign_dec, ad.signs);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = lane & 15, row = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* buf = stage[wave];
  const bool scale_in = !a.auto_scale;
  const int64_t ne = b.n_groups, nd = bd.n_groups;
  const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
  PipeItem cur = pipe_first((int64_t)blockIdx.x * (kBlock / 64) + wave, ne, nd);
  if (cur.kind < 0) return;
  // one register set for either kind: an encode group's 32 dwords of bf16
  // pairs, or a decode group's 16 dwords of indices
  uint32_t w[32];
  float sc = 0.0f;
  DecIn din;
  int ic = cur.kind == 0 ? item_of(b, cur.slot) : item_of(bd, cur.slot);
  // the last item of each batch met so far (the walks only move forward)
  int ie = cur.kind == 0 ? ic : 0, id = cur.kind == 0 ? 0 : ic;
  if (cur.kind == 0) {
    enc_prefetch(b.it[ic], cur.slot - b.it[ic].group0, buf, lane, scale_in);
    enc_take(buf, t, row, w, sc);
  } else {
    dec_prefetch(bd.it[ic], cur.slot - bd.it[ic].group0, buf, lane);
    dec_take(buf, t, row, w, din);
  }
  for (;;) {
    // every lane's reads of the buffer complete before it is refilled
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    PipeItem nx = pipe_next(cur, stride, ne, nd);
    const bool more = nx.kind >= 0;   // uniform across the wave
    if (!more) nx = cur;              // the last item prefetches itself again
    const int ip = nx.kind == 0 ? item_from(b, ie, nx.slot) : item_from(bd, id, nx.slot);
    if (nx.kind == 0) ie = ip; else id = ip;
    // Each kind's per-lane LDS addresses are derived inside its own branch
    // from a lane id the compiler cannot hoist: kept live across the loop,
    // both kinds' addresses would not fit the register file next to an
    // encode group's working set.
    {
      const int ln = opaque_lane_id(), tt = ln & 15, rr = ln >> 4;
      if (nx.kind == 0)
        enc_prefetch(b.it[ip], nx.slot - b.it[ip].group0, buf, ln, scale_in);
      else
        dec_prefetch(bd.it[ip], nx.slot - bd.it[ip].group0, buf, ln);
      // An encode group runs at a raised wave priority: when both waves of
      // a SIMD are ready, the VALU-bound encode issues first and the
      // decode's memory-bound work fills the gaps (measured: the fused
      // launch about 5% shorter than with equal priorities).
      if (cur.kind == 0) {
        __builtin_amdgcn_s_setprio(1);
        enc_group<false>(a, b.it[ic], sign_enc, cur.slot - b.it[ic].group0, tt, rr, w, sc,
                         ostage[wave]);
        __builtin_amdgcn_s_setprio(0);
      } else
        dec_group<OUT_BF16>(bd.it[ic], sign_dec, cur.slot - bd.it[ic].group0, tt, rr, w, din,
                            ostage[wave]);
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const int ln = opaque_lane_id(), tt = ln & 15, rr = ln >> 4;
      if (nx.kind == 0)
        enc_take(buf, tt, rr, w, sc);
      else
        dec_take(buf, tt, rr, w, din);
    }
    if (!more) break;
    cur = nx;
    ic = ip;
  }
}

}  // namespace

bool e8_fast_encode_ok(const EncodeLaunch& a) {
  return a.lattice == 8 && (a.tile == 256 || (a.tile == 512 && a.auto_scale && !a.rate_control)) &&
         a.in_bf16 && !a.dither && !a.wide && a.coords == nullptr;
}

bool e8_fast_decode_ok(const DecodeLaunch& a) {
  return a.lattice == 8 && (a.tile == 256 || a.tile == 512) && !a.dither && !a.wide;
}


using namespace fastlib;

hipError_t launch_encode_e8_fast(const EncodeLaunch& a, const EncBatch& b, hipStream_t s) {
  if (a.tile == 512) {
    // the items' tiles of 512 as halves of 256, in groups of 16 halves
    EncBatch h = b;
    h.n_groups = 0;
    for (int i = 0; i < b.n; ++i) {
      h.it[i].n_tiles = 2 * b.it[i].n_tiles;
      h.it[i].group0 = h.n_groups;
      h.n_groups += (h.it[i].n_tiles + 15) / 16;
    }
    for (int i = b.n; i < kMaxItems; ++i) h.it[i] = h.it[0];
    static int occ512 = 0;
    const int64_t blocks =
        persistent_grid(h.n_groups * 16, resident_blocks(encode_e8_fast512, occ512));
    hipLaunchKernelGGL(encode_e8_fast512, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, h);
    return hipGetLastError();
  }
  if (a.rate_control) {
    static int occ_rc = 0;
    const int64_t blocks =
        persistent_grid(b.n_groups * 16, resident_blocks(encode_e8_fast_rc, occ_rc));
    hipLaunchKernelGGL(encode_e8_fast_rc, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b);
  } else {
    static int occ = 0;
    const int64_t blocks = persistent_grid(b.n_groups * 16, resident_blocks(encode_e8_fast, occ));
    hipLaunchKernelGGL(encode_e8_fast, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b);
  }
  return hipGetLastError();
}

hipError_t launch_codec_e8_fast(const EncodeLaunch& a, const EncBatch& b, const DecodeLaunch& ad,
                               const DecBatch& bd, hipStream_t s) {
  static int occ_bf16 = 0, occ_f32 = 0;
  const int64_t slots = b.n_groups > bd.n_groups ? b.n_groups : bd.n_groups;
  if (ad.out_bf16) {
    const int64_t blocks = persistent_grid(slots * 16, resident_blocks(codec_e8_fast<true>, occ_bf16));
    hipLaunchKernelGGL(codec_e8_fast<true>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b, ad, bd);
  } else {
    const int64_t blocks = persistent_grid(slots * 16, resident_blocks(codec_e8_fast<false>, occ_f32));
    hipLaunchKernelGGL(codec_e8_fast<false>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b, ad, bd);
  }
  return hipGetLastError();
}

hipError_t launch_decode_e8_fast(const DecodeLaunch& a, const DecBatch& b, hipStream_t s) {
  if (a.tile == 512) {
    // the items' tiles of 512 as halves of 256, in groups of 16 halves
    DecBatch h = b;
    h.n_groups = 0;
    for (int i = 0; i < b.n; ++i) {
      h.it[i].n_tiles = 2 * b.it[i].n_tiles;
      h.it[i].group0 = h.n_groups;
      h.n_groups += (h.it[i].n_tiles + 15) / 16;
    }
    for (int i = b.n; i < kMaxItems; ++i) h.it[i] = h.it[0];
    static int occ512_bf16 = 0, occ512_f32 = 0;
    if (a.out_bf16) {
      const int64_t blocks = persistent_grid(
          h.n_groups * 16, resident_blocks(decode_e8_fast<true, 512>, occ512_bf16));
      hipLaunchKernelGGL((decode_e8_fast<true, 512>), dim3((unsigned)blocks), dim3(kBlock), 0, s,
                         a, h);
    } else {
      const int64_t blocks = persistent_grid(
          h.n_groups * 16, resident_blocks(decode_e8_fast<false, 512>, occ512_f32));
      hipLaunchKernelGGL((decode_e8_fast<false, 512>), dim3((unsigned)blocks), dim3(kBlock), 0,
                         s, a, h);
    }
    return hipGetLastError();
  }
  static int occ_bf16 = 0, occ_f32 = 0;
  if (a.out_bf16) {
    const int64_t blocks = persistent_grid(b.n_groups * 16, resident_blocks(decode_e8_fast<true>, occ_bf16));
    hipLaunchKernelGGL(decode_e8_fast<true>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b);
  } else {
    const int64_t blocks = persistent_grid(b.n_groups * 16, resident_blocks(decode_e8_fast<false>, occ_f32));
    hipLaunchKernelGGL(decode_e8_fast<false>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b);
  }
  return hipGetLastError();
}

}  // namespace hq

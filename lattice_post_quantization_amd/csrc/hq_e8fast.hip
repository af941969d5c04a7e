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

// Coalesced store of a group's output.  Lane (t, r) holds CPL 16-byte chunks:
// chunk k lies at byte r * 16 CPL + 16 k of tile t, and tiles are
// 64 CPL bytes apart.  The wave writes them, 4 KB (256 chunks) per pass,
// into a 4 KB LDS buffer and reads them back so that each store instruction
// covers 1 KB of contiguous output.  Chunk c of a pass sits at LDS slot
// c ^ ((c >> 4) & 15), which keeps both sides free of bank conflicts.
template <int CPL>
__device__ inline void store_group(__amdgpu_buffer_rsrc_t rs, const uint4* chunk, uint4* ost,
                                   int t, int row) {
  constexpr int kTilesPerPass = 256 / (4 * CPL);
  const int lane = row * 16 + t;
#pragma unroll
  for (int h = 0; h < 16 / kTilesPerPass; ++h) {
    wave_lds_sync();
    if (t / kTilesPerPass == h) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = (t % kTilesPerPass) * 4 * CPL + row * CPL + k;
        ost[c ^ ((c >> 4) & 15)] = chunk[k];
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 64 * i + lane;
      const uint4 q = ost[c ^ ((c >> 4) & 15)];
      store16(rs, (uint32_t)(h * 4096 + 16 * c), q.x, q.y, q.z, q.w);
    }
  }
}

// Staged loads.  A wave's 16 tiles are 8 KB of contiguous bf16, read with
// eight direct-to-LDS loads of 1 KB each (instruction k covers tiles 2k and
// 2k + 1, so every load is fully coalesced).  Lane l = 16 r + b of
// instruction k fetches row r, 16-byte chunk j = (b/2 - k) mod 8 of tile
// 2k + (b & 1) and the hardware stores it at LDS slot 64 k + l; lane (t, r)
// later finds chunk j of its tile at slot 64 (t/2) + 16 r + ((t + 2j) mod 16),
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
    const int j = ((b >> 1) - k) & 7;
    const int off = (2 * k + (b & 1)) * 512 + r * 128 + j * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, off, 0, 0, 0);
  }
  if (scale_in)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(out_rsrc(it.scale + group * 16, live * 4u),
                                             lds_ptr(buf + 512), 4, b * 4, 0, 0, 0);
}

__device__ inline void enc_take(const uint4* buf, int t, int r, uint32_t* w, float& scale) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 q = buf[64 * (t >> 1) + 16 * r + ((t + 2 * j) & 15)];
    w[4 * j] = q.x; w[4 * j + 1] = q.y; w[4 * j + 2] = q.z; w[4 * j + 3] = q.w;
  }
  scale = reinterpret_cast<const float*>(buf + 512)[t];
}

// Per-tile results are written by the 16 lanes of row 0; other lanes get an
// offset past the end of the buffer, which the hardware drops.
__device__ inline uint32_t row0_offset(int t, int row, int size) {
  return row == 0 ? (uint32_t)(t * size) : 0x40000000u;
}

// One group of 16 tiles held by a wave (w: this lane's 64 bf16 of its tile).
// (scale_in: the caller's scale of this lane's tile when not automatic.)
__device__ inline void enc_group(const EncodeLaunch& a, const EncItem& it, const uint32_t* sign_tab,
                                 int64_t group, int t, int row, const uint32_t* w, float scale_in,
                                 uint4* ost) {

  const uint4* st = reinterpret_cast<const uint4*>(sign_tab + row * 32);
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
  uint32_t status = 0;
  float delta;
  if (a.auto_scale) {
    delta = bf16_round_to_f32(sqrt(ss / 256.0) * a.c);
    if (delta == 0.0f) delta = 1.0f;
  } else {
    delta = scale_in;
    if (!(delta > 0.0f) || !isfinite(delta)) status |= HQ_ST_NONFINITE;
  }
  if (!isfinite(ss)) status |= HQ_ST_NONFINITE;
  // |u_i| <= sqrt(sum x^2) / Delta: below 124 no grid value reaches the clamp
  const bool big = !(sqrt(ss) < 124.0 * (double)delta);
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
  // element bit 6 (row bit 0) <-> register bit 5, then butterfly
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    swap_f64<false>(v[i], v[i + 32]);
    const double x = v[i], y = v[i + 32];
    v[i] = x + y;
    v[i + 32] = x - y;
  }
  // element bit 7 (row bit 1) <-> register bit 4, then butterfly
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (!(i & 16)) {
      swap_f64<true>(v[i], v[i + 16]);
      const double x = v[i], y = v[i + 16];
      v[i] = x + y;
      v[i + 16] = x - y;
    }
  }
  // Now register i holds element bits (i0 i1 i2 i3 | i4 = b7 | i5 = b6) and the
  // lane's row bits hold (r0 = b5, r1 = b4).

  // When some tile of the wave may pass the clamp, the generic encoder's
  // clamped rint(S K) replaces S (and K becomes 1).
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      double q = rint(__dmul_rn(v[i], K));
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
  uint32_t cbits = 0, ties = 0;
  int32_t U[64];
  const int r0 = row & 1, r1 = row >> 1;
  // tile block index of register block blk = b3 + 2 b4 + 4 b5 + 8 b6 + 16 b7
  auto bpos = [&](int blk) {
    return (blk & 1) + 2 * r1 + 4 * r0 + 8 * (blk >> 2) + 16 * ((blk >> 1) & 1);
  };
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // two roundings, never fused: q = RN(S K), then RN(q + 1.5 2^52)
      const double m = __dadd_rn(__dmul_rn(v[8 * blk + i], K), kMagic);
      U[8 * blk + i] = (int32_t)(uint32_t)(uint64_t)__double_as_longlong(m);
    }
    int c;
    ties |= e8_block_fast(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1], c) << blk;
    cbits |= (uint32_t)c << bpos(blk);
  }
  if (ties) {
    // blocks with a coordinate exactly on a rounding boundary
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      if ((ties >> blk) & 1u) {
        const int c = e8_block_exact(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1]);
        cbits = (cbits & ~(1u << bpos(blk))) | ((uint32_t)c << bpos(blk));
      }
    }
  }
  const uint32_t coset_word = tile_or_u32(cbits);

  // ---- Rice parameter: k = argmin_k L(k), L(k) = Q_k + 256 (1 + k),
  // Q_k = sum floor(zeta / 2^k).  L is convex: L(k+1) - L(k) = 256 - D_k with
  // D_k = Q_k - Q_{k+1} = sum floor((zeta + 2^k) / 2^(k+1)), which falls
  // with k, so the first minimum is the smallest k with D_k <= 256.  D_k lies
  // within 128 of S / 2^(k+1) (S = sum zeta), so with kt the smallest k with
  // S <= 256 * 2^(k+1): D_{kt+1} <= 256, and D_k > 256 for k <= kt - 2
  // (strictly, so no smaller k ties).  Only kt - 1, kt, kt + 1 remain.
  uint32_t zz[16];
  uint32_t S = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    zz[q] = zigzag4(packed[q]);
    S = byte_sum(zz[q], S);
  }
  S = tile_sum_u32(S);
  int kt = 0;
  while (kt < 8 && S > (256u << (kt + 1))) ++kt;
  int kc[3];
  uint32_t R[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    int k = kt - 1 + j;
    kc[j] = k < 0 ? 0 : (k > 8 ? 8 : k);
    const uint32_t mask = ((1u << kc[j]) - 1u) * 0x01010101u;
    uint32_t r = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) r = byte_sum(zz[q] & mask, r);
    R[j] = r;
  }
  uint32_t best = 0xFFFFFFFFu;
  int bk = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint32_t Rk = tile_sum_u32(R[j]);
    const uint32_t L = ((S - Rk) >> kc[j]) + 256u * (uint32_t)(1 + kc[j]);
    if (L < best) { best = L; bk = kc[j]; }
  }

  // ---- restore natural element order (undo the two swaps) and store
#pragma unroll
  for (int q = 0; q < 16; ++q)
    if (!(q & 4)) swap32(packed[q], packed[q + 4]);
#pragma unroll
  for (int q = 0; q < 8; ++q) swap16(packed[q], packed[q + 8]);
  const uint32_t live = live_tiles(it.n_tiles, group);
  const int64_t tile0 = group * 16;
  uint4 ch[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    ch[k] = make_uint4(packed[4 * k], packed[4 * k + 1], packed[4 * k + 2], packed[4 * k + 3]);
  store_group<4>(out_rsrc(it.idx + tile0 * 256, live * 256u), ch, ost, t, row);
  if (a.auto_scale)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), out_rsrc(it.scale + tile0, live * 4u),
                                          (int)row0_offset(t, row, 4), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(coset_word, out_rsrc(it.coset + tile0, live * 4u),
                                        (int)row0_offset(t, row, 4), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bk, out_rsrc(it.rice_k + tile0, live),
                                       (int)row0_offset(t, row, 1), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(4u + 32u + best, out_rsrc(it.tile_bits + tile0, live * 4u),
                                        (int)row0_offset(t, row, 4), 0, 0);
  if (status && (uint32_t)t < live) set_status(a.status, status);
}

// Persistent waves: each wave walks groups of 16 tiles with a grid-wide
// stride; the next group streams into the wave's LDS buffer while the
// current one is computed.
// The loop body ends with reading the next group from LDS, after this
// group's stores; the last iteration prefetches its own group again (an L2
// hit) so that no branch surrounds the memory operations.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void encode_e8_fast(EncodeLaunch a, EncBatch b) {
  __shared__ uint32_t sign_tab[128];
  __shared__ uint4 stage[kBlock / 64][kEncStage];
  __shared__ uint4 ostage[kBlock / 64][256];
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
    const int ip = more ? item_of(b, gn) : ic;
    enc_prefetch(b.it[ip], gp - b.it[ip].group0, buf, lane, scale_in);
    enc_group(a, b.it[ic], sign_tab, g - b.it[ic].group0, t, row, w, sc, ostage[wave]);
    __builtin_amdgcn_sched_barrier(0);
    enc_take(buf, t, row, w, sc);
    if (!more) break;
    g = gn;
    ic = ip;
  }
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
// j = (b/4 - k) mod 4 of tile 4k + (b & 3) into slot 64 k + l; lane (t, r)
// reads chunk j of its tile from slot 64 (t/4) + 16 r + ((t + 4j) mod 16).
// Two more loads bring the group's coset words and scales (lanes 0-15; the
// other lanes repeat them) to the 512 bytes after the indices.
constexpr int kDecStage = 256 + 32;   // uint4 per wave

struct DecIn {
  uint32_t cw;
  float scale;
};

__device__ inline void dec_prefetch(const DecItem& it, int64_t group, uint4* buf, int lane) {
  const int r = lane >> 4, b = lane & 15;
  const uint32_t live = live_tiles(it.n_tiles, group);
  const auto rs = out_rsrc(const_cast<int8_t*>(it.idx) + group * 16 * 256, live * 256u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = ((b >> 2) - k) & 3;
    const int off = (4 * k + (b & 3)) * 256 + r * 64 + j * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, off, 0, 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      out_rsrc(const_cast<uint32_t*>(it.coset) + group * 16, live * 4u), lds_ptr(buf + 256), 4,
      b * 4, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      out_rsrc(const_cast<float*>(it.scale) + group * 16, live * 4u), lds_ptr(buf + 272), 4,
      b * 4, 0, 0, 0);
}

__device__ inline void dec_take(const uint4* buf, int t, int r, uint32_t* d, DecIn& in) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 q = buf[64 * (t >> 2) + 16 * r + ((t + 4 * j) & 15)];
    d[4 * j] = q.x; d[4 * j + 1] = q.y; d[4 * j + 2] = q.z; d[4 * j + 3] = q.w;
  }
  in.cw = reinterpret_cast<const uint32_t*>(buf + 256)[t];
  in.scale = reinterpret_cast<const float*>(buf + 272)[t];
}

template <bool OUT_BF16>
__device__ inline void dec_group(const DecItem& it, const uint32_t* sign_tab, int64_t group, int t,
                                 int row, const uint32_t* d, const DecIn& in, uint4* ost) {
  const uint32_t cw = in.cw >> (8 * row);        // this lane's 8 blocks
  const float dsc = in.scale * 0.03125f;         // Delta / 32, exact

  // bound for the int16 path: sum |P| <= 4 sum|stored| + 320 (|z7| <= 2|t7| + 1)
  uint32_t sabs = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) sabs = __builtin_amdgcn_sad_u8(d[q] ^ 0x80808080u, 0x80808080u, sabs);
  sabs = tile_sum_u32(sabs);
  const bool small = sabs <= 8111u;

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
    const s16x2 cc = (s16x2){(short)c, (short)c};
    // z7 = 2 t7 + par: P7 = 4 t7 + 2 par + c
    const s16x2 c7 = (s16x2){(short)c, (short)(c + 2 * par)};
    P2[4 * b] = as_u32(as_s16x2(p01) * (s16x2){2, 2} + cc);
    P2[4 * b + 1] = as_u32(as_s16x2(p23) * (s16x2){2, 2} + cc);
    P2[4 * b + 2] = as_u32(as_s16x2(p45) * (s16x2){2, 2} + cc);
    P2[4 * b + 3] = as_u32(as_s16x2(p67) * (s16x2){2, 4} + c7);
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
  }
  // Register i now holds element bits (i0 .. i3, i4 = b7, i5 = b6); rows (b5, b4),
  // as the exact integer (H P)_e.

  // ---- x = (H P)_e Delta / 32.  fp32 output: one rounding of the exact
  // product.  bf16 output: the fp32 product is exact for a bf16-valued scale
  // (|H P| < 2^16 times 8 significant bits) of normal magnitude, and one
  // rounding to bf16 follows; a wave with any other scale (fp32 caller
  // scales, outputs that could be subnormal) rounds from the exact fp64
  // product as the generic decoder does.
  const uint4* st = reinterpret_cast<const uint4*>(sign_tab + row * 32);
  if constexpr (OUT_BF16) {
    uint32_t o[32];
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
    // undo the swaps: dword bit 3 <-> row bit 1, dword bit 4 <-> row bit 0
#pragma unroll
    for (int m = 0; m < 32; ++m)
      if (!(m & 8)) swap32(o[m], o[m + 8]);
#pragma unroll
    for (int m = 0; m < 16; ++m) swap16(o[m], o[m + 16]);
    uint4 ch[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 sm = st[k];
      ch[k] = make_uint4(o[4 * k] ^ sm.x, o[4 * k + 1] ^ sm.y, o[4 * k + 2] ^ sm.z,
                         o[4 * k + 3] ^ sm.w);
    }
    store_group<8>(out_rsrc(static_cast<uint16_t*>(it.y) + group * 16 * 256,
                            live_tiles(it.n_tiles, group) * 512u),
                   ch, ost, t, row);
  } else {
    uint32_t o[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) o[i] = __float_as_uint(y[i] * dsc);
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (!(i & 16)) swap32(o[i], o[i + 16]);
#pragma unroll
    for (int i = 0; i < 32; ++i) swap16(o[i], o[i + 32]);
    uint4 ch[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t sm = sign_tab[row * 32 + 2 * k], sn = sign_tab[row * 32 + 2 * k + 1];
      ch[k] = make_uint4(o[4 * k] ^ (sm << 16), o[4 * k + 1] ^ (sm & 0x80000000u),
                         o[4 * k + 2] ^ (sn << 16), o[4 * k + 3] ^ (sn & 0x80000000u));
    }
    store_group<16>(out_rsrc(static_cast<float*>(it.y) + group * 16 * 256,
                             live_tiles(it.n_tiles, group) * 1024u),
                    ch, ost, t, row);
  }
}

// Persistent waves as in the encoder.  The loop body ends with reading the
// next group from LDS, after this group's stores, so the wait for the
// prefetch never includes those stores; the last iteration prefetches its
// own group again (an L2 hit) to keep the loop free of branches around
// memory operations.
template <bool OUT_BF16>
__global__ __launch_bounds__(kBlock) void decode_e8_fast(DecodeLaunch a, DecBatch b) {
  __shared__ uint32_t sign_tab[128];
  __shared__ uint4 stage[kBlock / 64][kDecStage];
  __shared__ uint4 ostage[kBlock / 64][256];
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
  dec_prefetch(b.it[ic], g - b.it[ic].group0, buf, lane);
  dec_take(buf, t, row, d, in);
  for (;;) {
    // every lane's reads of the buffer complete before it is refilled
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t gn = g + stride;
    const bool more = gn < b.n_groups;   // uniform across the wave
    const int64_t gp = more ? gn : g;
    const int ip = more ? item_of(b, gn) : ic;
    dec_prefetch(b.it[ip], gp - b.it[ip].group0, buf, lane);
    dec_group<OUT_BF16>(b.it[ic], sign_tab, g - b.it[ic].group0, t, row, d, in, ostage[wave]);
    __builtin_amdgcn_sched_barrier(0);
    dec_take(buf, t, row, d, in);
    if (!more) break;
    g = gn;
    ic = ip;
  }
}

}  // namespace

bool e8_fast_encode_ok(const EncodeLaunch& a) {
  return a.lattice == 8 && a.tile == 256 && a.in_bf16 && !a.dither && a.coords == nullptr;
}

bool e8_fast_decode_ok(const DecodeLaunch& a) {
  return a.lattice == 8 && a.tile == 256 && !a.dither;
}


using namespace fastlib;

hipError_t launch_encode_e8_fast(const EncodeLaunch& a, const EncBatch& b, hipStream_t s) {
  static int occ = 0;
  const int64_t blocks = persistent_grid(b.n_groups * 16, resident_blocks(encode_e8_fast, occ));
  hipLaunchKernelGGL(encode_e8_fast, dim3((unsigned)blocks), dim3(kBlock), 0, s, a, b);
  return hipGetLastError();
}

hipError_t launch_decode_e8_fast(const DecodeLaunch& a, const DecBatch& b, hipStream_t s) {
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

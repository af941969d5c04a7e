// Fast paths for tile 128 with bf16 input: E8 (KV vectors of head dimension
// 128, with or without the subtractive dither), D4, A2 and Z (the lattices
// of the sweep at tile 128).  bf16 or fp32 out.  Same results as the generic
// kernels, bit for bit (A2 decode, whose point has sqrt(3) coordinates:
// within fp64 rounding of them, as the generic decoder).
//
// Passages: [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice
// Quantization Pipeline ..." (per-vector rotation, E8, subtractive dither that
// keeps cached inner products unbiased, Rice code, algebraic decoding);
// [arXiv abstract] "HyperQuant: A Rate-Distortion-Optimal Quantization
// Pipeline ..." ideas (i)-(iii), idea (ii) naming D4, A2 and Z beside E8.
//
// Work mapping.  A wave holds 32 tiles: lane (t, r) = lane t + 32 r holds
// elements [64 r, 64 r + 64) of tile t, so six Walsh-Hadamard stages run in
// registers and the seventh (element bit 6 = lane bit 5) after one
// v_permlane32_swap per dword pair.  Groups of 32 tiles stream through LDS
// (coalesced direct-to-LDS loads, a swizzle keeps the reads conflict free)
// and leave through a 4 KB LDS buffer as contiguous 1 KB stores.  The dither
// w of element e of vector v is regenerated from the counter hash of
// (seed, v, e); d = w - Q_E8(w) uses the same exact block decision as the
// lattice step.
//
// Lattice decisions are taken on the integer grid values U = u 2^24 without
// branches.  With F = U mod 2^24, the top byte of
// t = U + 2^23 - 1 + [floor(U / 2^24) odd] is rne(u) (ties to even), and
// B = |F - 2^23| is u's distance to the nearest half-integer (its distance to
// the nearest integer is 2^23 - B).  A tile whose norm allows a grid value
// past the clamp of the generic encoder (|u| > 124) takes the clamped grid,
// as there, for the whole wave.
//
// Decode: the lattice points in packed int16 (always exact for D4, A2 and Z:
// sum |P| <= 20512 per tile), Hadamard in int16, one fp64 product by the
// scale and one by 1/sqrt(128), and bf16 by rounding to odd at fp32 first.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_lanes.h"
#include "hq_dither.h"

namespace hq {
namespace {

using namespace fastlib;

constexpr int kTpw = 32;   // tiles per wave
constexpr uint32_t kBias = 0x80808080u;

// coset bits of a tile of 128: one per E8 block or A2 pair
template <int LAT>
constexpr uint32_t coset_bits128() {
  return LAT == 8 ? 16u : (LAT == 2 ? 64u : 0u);
}

__device__ inline uint32_t live32(int64_t n_tiles, int64_t group) {
  const int64_t n = n_tiles - group * kTpw;
  return (uint32_t)(n < kTpw ? n : kTpw);
}

// Sum / OR over the two lanes (t, 0) and (t, 1) of a tile.
__device__ inline uint32_t pair_sum_u32(uint32_t v) {
  uint32_t a = v, b = v;
  swap32(a, b);
  return a + b;
}
__device__ inline uint32_t pair_or_u32(uint32_t v) {
  uint32_t a = v, b = v;
  swap32(a, b);
  return a | b;
}
__device__ inline double pair_sum_f64(double v) {
  double a = v, b = v;
  swap_f64<true>(a, b);
  return a + b;
}

// ------------------------------------------------- D4, A2 and Z decisions
// t = U + 2^23 - 1 + [floor(U / 2^24) odd]; its top byte is rne(U / 2^24).
__device__ inline uint32_t rne_t(int32_t U) {
  return (uint32_t)U + 0x7FFFFFu + (((uint32_t)U >> 24) & 1u);
}

// |a - 2^31| + C (C an inline constant)
template <int C>
__device__ inline uint32_t sad31(uint32_t a) {
  uint32_t r;
  __asm__("v_sad_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(0x80000000u), "i"(C));
  return r;
}

// |a - 2^23|
__device__ inline uint32_t sad23(uint32_t a) {
  uint32_t r;
  __asm__("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(a), "s"(0x00800000u));
  return r;
}

// Nearest D4 point of one block, as the stored int8 bytes (z0, z1, z2,
// floor(z3 / 2)).  Each coordinate rounds to a = rne(u); on an odd sum the
// first coordinate j of largest residual steps one towards u (down if it was
// rounded up), as in the generic D_m rule.  Residuals rank by
// 256 B_i + i = |256 F_i - 2^31| + i (one v_sad_u32; U << 8 is 256 F), so the
// minimum key is the first largest residual.  Bit 0 of byte i of
// top(t) ^ top(U) tells whether coordinate i was rounded up.  The bytes
// carry a bias of 128 while one is stepped, so no byte carries into the
// next (|u| <= 124).
__device__ inline uint32_t d4_block(const int32_t* U) {
  const uint32_t u0 = (uint32_t)U[0], u1 = (uint32_t)U[1], u2 = (uint32_t)U[2],
                 u3 = (uint32_t)U[3];
  const uint32_t t0 = rne_t(U[0]), t1 = rne_t(U[1]), t2 = rne_t(U[2]), t3 = rne_t(U[3]);
  const uint32_t k0 = sad31<0>(u0 << 8), k1 = sad31<1>(u1 << 8), k2 = sad31<2>(u2 << 8),
                 k3 = sad31<3>(u3 << 8);
  const uint32_t kmin = min3u(k0, k1, k2 < k3 ? k2 : k3);
  const uint32_t sh = (kmin & 3u) << 3;
  const uint32_t A = top_bytes(t0, t1, t2, t3);
  const uint32_t up = ((A ^ top_bytes(u0, u1, u2, u3)) >> sh) & 1u;
  const uint32_t odd = ((t0 ^ t1 ^ t2 ^ t3) >> 24) & 1u;
  const uint32_t step = (up ? 0xFFFFFFFFu : 1u) << sh;
  const uint32_t W = (A ^ kBias) + (odd ? step : 0u);
  // biased floor(z3 / 2) = floor((z3 + 128) / 2) + 64
  return ((W & 0x00FFFFFFu) | (((W >> 25) + 64u) << 24)) ^ kBias;
}

// Nearest A2 point of one pair, given U1 = grid(u1) and V2 = grid(u2 /
// sqrt3): integer coset (rne, rne) or half coset (rne(. - 1/2) + 1/2) under
// the metric diag(1, 3).  The squared distances differ by
// d_int - d_half = 2^24 (2^24 - (B1 + 3 B2)) grid units squared, so the half
// coset wins iff B1 + 3 B2 < 2^24 (a tie keeps the integer coset).  The top
// byte of U - 1 + [floor((U - 2^23) / 2^24) odd] is rne(U / 2^24 - 1/2).
// Returns c; ta, tb hold the stored integers (a, b) in their top bytes.
__device__ inline uint32_t a2_pair(int32_t U1, int32_t V2, uint32_t& ta, uint32_t& tb) {
  const uint32_t u = (uint32_t)U1, v = (uint32_t)V2;
  const uint32_t B1 = sad23(u & 0xFFFFFFu), B2 = sad23(v & 0xFFFFFFu);
  const bool c = B1 + 3u * B2 < (1u << 24);
  const uint32_t h1 = u - 1u + (((u - (uint32_t)kHalf) >> 24) & 1u);
  const uint32_t h2 = v - 1u + (((v - (uint32_t)kHalf) >> 24) & 1u);
  ta = c ? h1 : rne_t(U1);
  tb = c ? h2 : rne_t(V2);
  return c ? 1u : 0u;
}

// Grid value of one rotated coordinate: the low dword of RN(S K + 1.5 2^52)
// (one rounding of the exact product) is rne(S K) for |S K| < 2^31.
__device__ __attribute__((always_inline)) inline int32_t grid_at(double v, double K) {
  const double m = __fma_rn(v, K, kMagic);
  return (int32_t)(uint32_t)(uint64_t)__double_as_longlong(m);
}

// ------------------------------------------------------------------ encode
// Group loads: 32 tiles of 256 bytes, eight direct-to-LDS loads of 1 KB
// (instruction k covers tiles 4k .. 4k + 3).  Lane l = 16 q + b of
// instruction k fetches chunk ((4 q + b / 4) ^ (k mod 4)) of tile 4k + (b mod 4)
// into slot 64 k + l; lane (t, r) finds chunk c of its tile at slot
// 64 (t / 4) + 4 (c ^ ((t / 4) mod 4)) + (t mod 4).  A caller-supplied scale
// arrives in the 256 bytes after the data.
constexpr int kEnc128Stage = 512 + 16;

__device__ inline void enc128_prefetch(const EncodeLaunch& a, int64_t group, uint4* buf,
                                       int lane, bool scale_in) {
  const uint32_t live = live32(a.n_tiles, group);
  const auto rs = out_rsrc(static_cast<uint16_t*>(const_cast<void*>(a.x)) + group * kTpw * 128,
                           live * 256u);
  const int q = lane >> 4, b = lane & 15;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int T = 4 * k + (b & 3);
    const int c = (4 * q + (b >> 2)) ^ (k & 3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, T * 256 + c * 16, 0,
                                             0, 0);
  }
  if (scale_in)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(out_rsrc(a.scale + group * kTpw, live * 4u),
                                             lds_ptr(buf + 512), 4, (lane & 31) * 4, 0, 0, 0);
}

__device__ inline void enc128_take(const uint4* buf, int t, int r, uint32_t* w, float& scale) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * r + j;
    const int cp = c ^ ((t >> 2) & 3);
    const uint4 q = buf[64 * (t >> 2) + 4 * cp + (t & 3)];
    w[4 * j] = q.x; w[4 * j + 1] = q.y; w[4 * j + 2] = q.z; w[4 * j + 3] = q.w;
  }
  scale = reinterpret_cast<const float*>(buf + 512)[t];
}

__device__ inline uint32_t row0_off(int t, int r, int size) {
  return r == 0 ? (uint32_t)(t * size) : 0x40000000u;
}

template <int LAT, bool DITHER>
__device__ inline void enc128_group(const EncodeLaunch& a, const uint32_t* sign_tab,
                                    int64_t group, int t, int r, const uint32_t* w,
                                    float scale_in, uint4* ost) {
  const uint32_t live = live32(a.n_tiles, group);
  const int64_t tile0 = group * kTpw;
  const uint4* st = reinterpret_cast<const uint4*>(sign_tab + r * 32);
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
  ss = pair_sum_f64(ss);
  uint32_t status = 0;
  float delta;
  if (a.auto_scale) {
    delta = bf16_round_to_f32(sqrt(ss / 128.0) * a.c);
    if (delta == 0.0f) delta = 1.0f;
  } else {
    delta = scale_in;
    if (!(delta > 0.0f) || !isfinite(delta)) status |= HQ_ST_NONFINITE;
  }
  if (!isfinite(ss)) status |= HQ_ST_NONFINITE;
  // |u_i| <= sqrt(sum x^2) / Delta: below 124 no grid value reaches the clamp
  const bool big = !(sqrt(ss) < 124.0 * (double)delta);
  const double tq = a.sqrt_n * (double)delta;
  const double K = 16777216.0 / tq;
  const double K3 = (LAT == 2) ? 16777216.0 / (tq * 1.7320508075688772) : K;

  // ---- Walsh-Hadamard: element bits 0-5 in registers, bit 6 across lanes
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
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    swap_f64<true>(v[i], v[i + 32]);
    const double x = v[i], y = v[i + 32];
    v[i] = x + y;
    v[i + 32] = x - y;
  }
  // register i now holds element (i mod 32) + 32 r + 64 (i / 32)

  // ---- quantizer grid U = u 2^24 = RN(S K + 1.5 2^52) - 1.5 2^52 (one
  // rounding of the exact product), formed block by block as the decisions
  // use it.  When some tile of the wave may pass the clamp, the generic
  // encoder's clamped rne(S K) first replaces S (and K becomes 1).
  double Kq = K, K3q = K3;
  if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      double q = rne_product(v[i], (LAT == 2 && (i & 1)) ? K3 : K);
      if (!(fabs(q) <= kUClamp)) {
        status |= HQ_ST_OVERFLOW;
        q = (q > 0.0) ? kUClamp : -kUClamp;
      }
      v[i] = q;
    }
    Kq = 1.0;
    K3q = 1.0;
  }

  // ---- nearest point and strip: packed[q] holds registers 4q .. 4q + 3
  uint32_t packed[16];
  uint32_t cw0 = 0, cw1 = 0;   // this lane's coset bits in the tile's words
  if constexpr (LAT == 8) {
    uint32_t ties = 0;
    int32_t U[64];
    const uint64_t vec = (uint64_t)(a.dither_base + tile0 + t);
    // tile block index of register block blk = element / 8
    auto bpos = [&](int blk) { return (blk & 3) + 4 * r + 8 * (blk >> 2); };
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      // the block's dither first (fewer registers live across the hash)
      int32_t d24[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (DITHER) {
        uint32_t e0 = (uint32_t)(8 * (blk & 3) + 32 * r + 64 * (blk >> 2));
        asm volatile("" : "+v"(e0));   // formed per block, not held across the loop
        int32_t W[8];
        const DitherVec dk = dither_vec(a.dither_seed, vec);
#pragma unroll
        for (int i = 0; i < 8; ++i) W[i] = dither_w(dk, e0 + (uint32_t)i);
        e8_dither_block(W, d24);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) U[8 * blk + i] = grid_at(v[8 * blk + i], Kq) + d24[i];
      int c;
      const uint32_t tie = e8_block_fast(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1], c);
      if constexpr (DITHER) {
        // searched at once: the hash leaves no registers for deferring it
        if (tie) c = e8_block_exact(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1]);
      } else {
        ties |= tie << blk;
      }
      cw0 |= (uint32_t)c << bpos(blk);
    }
    if (ties) {
      // blocks with a coordinate exactly on a rounding boundary
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) {
        if ((ties >> blk) & 1u) {
          const int c = e8_block_exact(U + 8 * blk, packed[2 * blk], packed[2 * blk + 1]);
          cw0 = (cw0 & ~(1u << bpos(blk))) | ((uint32_t)c << bpos(blk));
        }
      }
    }
  } else if constexpr (LAT == 4) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int32_t U[4] = {grid_at(v[4 * q], Kq), grid_at(v[4 * q + 1], Kq),
                            grid_at(v[4 * q + 2], Kq), grid_at(v[4 * q + 3], Kq)};
      packed[q] = d4_block(U);
    }
  } else if constexpr (LAT == 2) {
    // pair m (registers 2m, 2m + 1) is tile pair (m mod 16) + 16 r + 32 (m / 16)
    uint32_t cb = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      uint32_t a0, b0, a1, b1;
      const uint32_t c0 = a2_pair(grid_at(v[4 * q], Kq), grid_at(v[4 * q + 1], K3q), a0, b0);
      const uint32_t c1 = a2_pair(grid_at(v[4 * q + 2], Kq), grid_at(v[4 * q + 3], K3q), a1, b1);
      packed[q] = top_bytes(a0, b0, a1, b1);
      cb |= (c0 << (2 * q)) | (c1 << (2 * q + 1));
    }
    cw0 = (cb & 0xFFFFu) << (16 * r);
    cw1 = (cb >> 16) << (16 * r);
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      packed[q] = top_bytes(rne_t(grid_at(v[4 * q], Kq)), rne_t(grid_at(v[4 * q + 1], Kq)),
                            rne_t(grid_at(v[4 * q + 2], Kq)), rne_t(grid_at(v[4 * q + 3], Kq)));
  }
  if constexpr (coset_bits128<LAT>() > 0) cw0 = pair_or_u32(cw0);
  if constexpr (LAT == 2) cw1 = pair_or_u32(cw1);

  // ---- Rice parameter (n = 128): first minimum among kt - 1 .. kt + 1
  uint32_t zz[16];
  uint32_t S = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    zz[q] = zigzag4(packed[q]);
    S = byte_sum(zz[q], S);
  }
  S = pair_sum_u32(S);
  int kt = 0;
  while (kt < 8 && S > (128u << (kt + 1))) ++kt;
  uint32_t best = 0xFFFFFFFFu;
  int bk = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    int k = kt - 1 + j;
    k = k < 0 ? 0 : (k > 8 ? 8 : k);
    const uint32_t mask = ((1u << k) - 1u) * 0x01010101u;
    uint32_t R = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) R = byte_sum(zz[q] & mask, R);
    R = pair_sum_u32(R);
    const uint32_t L = ((S - R) >> k) + 128u * (uint32_t)(1 + k);
    if (L < best) { best = L; bk = k; }
  }

  // ---- natural order (register bit 5 <-> lane bit 5), then stores
#pragma unroll
  for (int q = 0; q < 8; ++q) swap32(packed[q], packed[q + 8]);
  const int lane = t + 32 * r;
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 8 * t + 4 * r + k;
    ost[c ^ ((c >> 4) & 15)] = make_uint4(packed[4 * k], packed[4 * k + 1], packed[4 * k + 2],
                                          packed[4 * k + 3]);
  }
  wave_lds_sync();
  const auto rs = out_rsrc(a.idx + tile0 * 128, live * 128u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 64 * i + lane;
    const uint4 q = ost[c ^ ((c >> 4) & 15)];
    store16(rs, (uint32_t)(16 * c), q.x, q.y, q.z, q.w);
  }
  if (a.auto_scale)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(delta), out_rsrc(a.scale + tile0, live * 4u),
                                          (int)row0_off(t, r, 4), 0, 0);
  if constexpr (LAT == 8) {
    __builtin_amdgcn_raw_buffer_store_b32(cw0, out_rsrc(a.coset + tile0, live * 4u),
                                          (int)row0_off(t, r, 4), 0, 0);
  } else if constexpr (LAT == 2) {
    const auto cr = out_rsrc(a.coset + 2 * tile0, live * 8u);
    __builtin_amdgcn_raw_buffer_store_b32(cw0, cr, (int)row0_off(t, r, 8), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(cw1, cr, (int)row0_off(t, r, 8) + 4, 0, 0);
  }
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bk, out_rsrc(a.rice_k + tile0, live),
                                       (int)row0_off(t, r, 1), 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(4u + coset_bits128<LAT>() + best,
                                        out_rsrc(a.tile_bits + tile0, live * 4u),
                                        (int)row0_off(t, r, 4), 0, 0);
  if (status && (uint32_t)t < live) set_status(a.status, status);
}

// Persistent waves as in the tile-256 path: the next group streams into LDS
// while this one is computed; the last iteration prefetches its own group.
template <int LAT, bool DITHER>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void encode_fast128(EncodeLaunch a) {
  __shared__ uint32_t sign_tab[128];
  __shared__ uint4 stage[kBlock / 64][kEnc128Stage];
  __shared__ uint4 ostage[kBlock / 64][256];
  fill_sign_table(sign_tab, a.signs);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = lane & 31, r = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* buf = stage[wave];
  const bool scale_in = !a.auto_scale;
  const int64_t n_groups = (a.n_tiles + kTpw - 1) / kTpw;
  const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
  int64_t g = (int64_t)blockIdx.x * (kBlock / 64) + wave;
  if (g >= n_groups) return;
  uint32_t w[32];
  float sc;
  enc128_prefetch(a, g, buf, lane, scale_in);
  enc128_take(buf, t, r, w, sc);
  for (;;) {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t gn = g + stride;
    const bool more = gn < n_groups;
    const int64_t gp = more ? gn : g;
    enc128_prefetch(a, gp, buf, lane, scale_in);
    enc128_group<LAT, DITHER>(a, sign_tab, g, t, r, w, sc, ostage[wave]);
    __builtin_amdgcn_sched_barrier(0);
    enc128_take(buf, t, r, w, sc);
    if (!more) break;
    g = gn;
  }
}

// ------------------------------------------------------------------ decode
// Group loads: 32 tiles of 128 index bytes, four direct-to-LDS loads of 1 KB
// (instruction k covers tiles 8k .. 8k + 7): lane l fetches chunk
// (l mod 8) ^ ((T / 2) mod 8) of tile T = 8k + l / 8 into slot 64 k + l; lane
// (t, r) finds chunk c of its tile at slot 64 (t / 8) + 8 (t mod 8) +
// (c ^ ((t / 2) mod 8)).  Coset words (E8: one per tile, A2: two) and the
// scales follow, 256 bytes each.
constexpr int kDec128Stage = 256 + 32;

template <int LAT>
__device__ inline void dec128_prefetch(const DecodeLaunch& a, int64_t group, uint4* buf,
                                       int lane) {
  const uint32_t live = live32(a.n_tiles, group);
  const auto rs = out_rsrc(const_cast<int8_t*>(a.idx) + group * kTpw * 128, live * 128u);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int T = 8 * k + (lane >> 3);
    const int c = (lane & 7) ^ ((T >> 1) & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + 64 * k), 16, T * 128 + c * 16, 0,
                                             0, 0);
  }
  if constexpr (LAT == 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        out_rsrc(const_cast<uint32_t*>(a.coset) + group * kTpw, live * 4u), lds_ptr(buf + 256),
        4, (lane & 31) * 4, 0, 0, 0);
  if constexpr (LAT == 2)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        out_rsrc(const_cast<uint32_t*>(a.coset) + 2 * group * kTpw, live * 8u),
        lds_ptr(buf + 256), 4, lane * 4, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      out_rsrc(const_cast<float*>(a.scale) + group * kTpw, live * 4u), lds_ptr(buf + 272), 4,
      (lane & 31) * 4, 0, 0, 0);
}

struct Dec128In {
  uint32_t cw;      // E8: the tile's word; A2: the word of this lane's pairs
  float scale;
};

template <int LAT>
__device__ inline void dec128_take(const uint4* buf, int t, int r, uint32_t* d, Dec128In& in) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * r + j;
    const uint4 q = buf[64 * (t >> 3) + 8 * (t & 7) + (c ^ ((t >> 1) & 7))];
    d[4 * j] = q.x; d[4 * j + 1] = q.y; d[4 * j + 2] = q.z; d[4 * j + 3] = q.w;
  }
  const uint32_t* cws = reinterpret_cast<const uint32_t*>(buf + 256);
  in.cw = (LAT == 8) ? cws[t] : (LAT == 2 ? cws[2 * t + r] : 0u);
  in.scale = reinterpret_cast<const float*>(buf + 272)[t];
}

// fp32 bits of x rounded to odd (toward zero, last bit set when inexact);
// x zero or of normal fp32 magnitude.  Rounding that to bf16 (nearest even)
// rounds x itself correctly, as 24 >= 8 + 2 bits.
__device__ inline float round_odd_f32(double x) {
  const float f = (float)x;
  const double b = (double)f;
  uint32_t u = __float_as_uint(f);
  if (b != x) u = (u - (fabs(b) > fabs(x) ? 1u : 0u)) | 1u;
  return __uint_as_float(u);
}

__device__ inline uint32_t bf16x2_rto(double lo, double hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 pr = {(__bf16)round_odd_f32(lo), (__bf16)round_odd_f32(hi)};
  return __builtin_bit_cast(uint32_t, pr);
}

// In-register Hadamard of the packed int16 points over element bits 1-6
// (and bit 0 within each dword when BIT0); afterwards pair m holds elements
// 2 (m mod 16) + 32 r + 64 (m / 16), + 1.
template <bool BIT0>
__device__ __attribute__((always_inline)) inline void hadamard_i16(uint32_t* P2) {
  if constexpr (BIT0) {
#pragma unroll
    for (int m = 0; m < 32; ++m) P2[m] = half_butterfly(P2[m]);
  }
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
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    swap32(P2[m], P2[m + 16]);
    const s16x2 x = as_s16x2(P2[m]), z = as_s16x2(P2[m + 16]);
    P2[m] = as_u32(x + z);
    P2[m + 16] = as_u32(x - z);
  }
}

// Output values x = (H P) (sc) (1 / sqrt n) from the int16 points (E8:
// sc = Delta / 2, D4 and Z: Delta); A2 combines the transforms of the
// even (2a + c) and odd (2b + c) coordinates: x = (Delta / 2)(E +/- sqrt3 O).
template <int LAT>
__device__ __attribute__((always_inline)) inline void int16_values(uint32_t* P2, float scale,
                                                                   double inv, double* x) {
  hadamard_i16<LAT != 2>(P2);
  if constexpr (LAT == 2) {
    const double sc = 0.5 * (double)scale, sc3 = sc * 1.7320508075688772;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const double e = (double)(short)(P2[m] & 0xFFFFu) * sc;
      const double o = (double)((int32_t)P2[m] >> 16) * sc3;
      x[2 * m] = (e + o) * inv;
      x[2 * m + 1] = (e - o) * inv;
    }
  } else {
    const double sc = (LAT == 8 ? 0.5 : 1.0) * (double)scale;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      x[2 * m] = ((double)(short)(P2[m] & 0xFFFFu) * sc) * inv;
      x[2 * m + 1] = ((double)((int32_t)P2[m] >> 16) * sc) * inv;
    }
  }
}

template <int LAT, bool OUT_BF16, bool DITHER>
__device__ inline void dec128_group(const DecodeLaunch& a, const uint32_t* sign_tab,
                                    int64_t group, int t, int r, const uint32_t* d,
                                    const Dec128In& in, uint4* ost) {
  const uint32_t live = live32(a.n_tiles, group);
  const int64_t tile0 = group * kTpw;
  const int lane = t + 32 * r;
  const double inv = a.inv_sqrt_n;

  // ---- unstrip into int16 pairs: P2[m] = (P_2m, P_2m+1) of elements
  // 64 r + 2m, + 1 (E8: P = 2p = 2z + c; D4, Z: P = z; A2: (2a + c, 2b + c))
  uint32_t P2[32];
  if constexpr (LAT == 8) {
    const uint32_t cw = in.cw >> (8 * r);   // this lane's 8 blocks
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t d0 = d[2 * b], d1 = d[2 * b + 1];
      uint32_t x = d0 ^ (d1 & 0x00FFFFFFu);
      x ^= x >> 16;
      x ^= x >> 8;
      const uint32_t par = x & 1u;
      const uint32_t c = (cw >> b) & 1u;
      const uint32_t e0 = d0 << 8, e1 = d1 << 8;
      const uint32_t p01 = __builtin_amdgcn_perm(d0, e0, 0x0A050804u);
      const uint32_t p23 = __builtin_amdgcn_perm(d0, e0, 0x0B070906u);
      const uint32_t p45 = __builtin_amdgcn_perm(d1, e1, 0x0A050804u);
      const uint32_t p67 = __builtin_amdgcn_perm(d1, e1, 0x0B070906u);
      const s16x2 cc = (s16x2){(short)c, (short)c};
      const s16x2 c7 = (s16x2){(short)c, (short)(c + 2 * par)};
      P2[4 * b] = as_u32(as_s16x2(p01) * (s16x2){2, 2} + cc);
      P2[4 * b + 1] = as_u32(as_s16x2(p23) * (s16x2){2, 2} + cc);
      P2[4 * b + 2] = as_u32(as_s16x2(p45) * (s16x2){2, 2} + cc);
      P2[4 * b + 3] = as_u32(as_s16x2(p67) * (s16x2){2, 4} + c7);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      // dword q: elements 64 r + 4q .. + 3 (a D4 block; A2 pairs 2q, 2q + 1)
      const uint32_t d0 = d[q], e0 = d0 << 8;
      const uint32_t p01 = __builtin_amdgcn_perm(d0, e0, 0x0A050804u);
      const uint32_t p23 = __builtin_amdgcn_perm(d0, e0, 0x0B070906u);
      if constexpr (LAT == 4) {
        const uint32_t par = (d0 ^ (d0 >> 8) ^ (d0 >> 16)) & 1u;   // z0 + z1 + z2
        P2[2 * q] = p01;
        P2[2 * q + 1] = as_u32(as_s16x2(p23) * (s16x2){1, 2} + (s16x2){0, (short)par});
      } else if constexpr (LAT == 2) {
        const short c0 = (short)((in.cw >> (2 * q)) & 1u), c1 = (short)((in.cw >> (2 * q + 1)) & 1u);
        P2[2 * q] = as_u32(as_s16x2(p01) * (s16x2){2, 2} + (s16x2){c0, c0});
        P2[2 * q + 1] = as_u32(as_s16x2(p23) * (s16x2){2, 2} + (s16x2){c1, c1});
      } else {
        P2[2 * q] = p01;
        P2[2 * q + 1] = p23;
      }
    }
  }

  // ---- x = H y / sqrt(n) in registers: register i holds element
  // (i mod 32) + 32 r + 64 (i / 32)
  double x[64];
  if constexpr (LAT == 8) {
    // int16 sums are exact while sum |P| <= 4 sum |stored| + 160 <= 2^15 - 1
    bool small = false;
    if constexpr (!DITHER) {
      uint32_t sabs = 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) sabs = __builtin_amdgcn_sad_u8(d[q] ^ 0x80808080u, 0x80808080u, sabs);
      small = pair_sum_u32(sabs) <= 8151u;
    }
    if (small) {
      int16_values<8>(P2, in.scale, inv, x);
    } else {
      // fp64: y = P / 2, or with the dither y 2^24 = P 2^23 - d 2^24; the
      // values and every Hadamard sum are integers below 2^40, exact
      double sc;
      if constexpr (DITHER) {
        const uint64_t vec = (uint64_t)(a.dither_base + tile0 + t);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          int32_t W[8], d24[8];
          uint32_t e0 = (uint32_t)(64 * r + 8 * b);
          asm volatile("" : "+v"(e0));   // formed per block, not held across the loop
          const DitherVec dk = dither_vec(a.dither_seed, vec);
#pragma unroll
          for (int i = 0; i < 8; ++i) W[i] = dither_w(dk, e0 + (uint32_t)i);
          e8_dither_block(W, d24);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t pr = P2[4 * b + (i >> 1)];
            const int32_t P = (i & 1) ? ((int32_t)pr >> 16) : (int32_t)(short)(pr & 0xFFFFu);
            x[8 * b + i] = (double)P * 8388608.0 - (double)d24[i];
          }
        }
        sc = (double)in.scale * 5.9604644775390625e-08;   // Delta 2^-24, exact
      } else {
#pragma unroll
        for (int m = 0; m < 32; ++m) {
          x[2 * m] = (double)(short)(P2[m] & 0xFFFFu);
          x[2 * m + 1] = (double)((int32_t)P2[m] >> 16);
        }
        sc = 0.5 * (double)in.scale;
      }
#pragma unroll
      for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          if (!(i & h)) {
            const double p = x[i], q = x[i + h];
            x[i] = p + q;
            x[i + h] = p - q;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        swap_f64<true>(x[i], x[i + 32]);
        const double p = x[i], q = x[i + 32];
        x[i] = p + q;
        x[i + 32] = p - q;
      }
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = (x[i] * sc) * inv;
    }
  } else {
    int16_values<LAT>(P2, in.scale, inv, x);
  }

  const uint4* st = reinterpret_cast<const uint4*>(sign_tab + r * 32);
  if constexpr (OUT_BF16) {
    // rounding through fp32 holds while every value is zero or of normal
    // magnitude: scales within 2^-90 .. 2^90 (else the exact fp64 rounding)
    const bool normal = in.scale >= 0x1p-90f && in.scale <= 0x1p90f;
    uint32_t o[32];
    if (__builtin_amdgcn_ballot_w64(!normal) == 0) {
#pragma unroll
      for (int m = 0; m < 32; ++m) o[m] = bf16x2_rto(x[2 * m], x[2 * m + 1]);
    } else {
#pragma unroll
      for (int m = 0; m < 32; ++m) o[m] = f64_to_bf16(x[2 * m]) | (f64_to_bf16(x[2 * m + 1]) << 16);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) swap32(o[m], o[m + 16]);
    // lane (t, r): 8 chunks at bytes 128 r + 16 k of tile t; two passes of
    // 16 tiles through the 4 KB buffer
    const auto rs = out_rsrc(static_cast<uint16_t*>(a.y) + tile0 * 128, live * 256u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      wave_lds_sync();
      if ((t >> 4) == h) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint4 sm = st[k];
          const int c = 16 * (t & 15) + 8 * r + k;
          ost[c ^ ((c >> 4) & 15)] = make_uint4(o[4 * k] ^ sm.x, o[4 * k + 1] ^ sm.y,
                                                o[4 * k + 2] ^ sm.z, o[4 * k + 3] ^ sm.w);
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
  } else {
    uint32_t o[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) o[i] = __float_as_uint((float)x[i]);
#pragma unroll
    for (int i = 0; i < 32; ++i) swap32(o[i], o[i + 32]);
    // lane (t, r): 16 chunks at bytes 256 r + 16 k of tile t; four passes of
    // 8 tiles
    const auto rs = out_rsrc(static_cast<float*>(a.y) + tile0 * 128, live * 512u);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      wave_lds_sync();
      if ((t >> 3) == h) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t sm = sign_tab[r * 32 + 2 * k], sn = sign_tab[r * 32 + 2 * k + 1];
          const int c = 32 * (t & 7) + 16 * r + k;
          ost[c ^ ((c >> 4) & 15)] =
              make_uint4(o[4 * k] ^ (sm << 16), o[4 * k + 1] ^ (sm & 0x80000000u),
                         o[4 * k + 2] ^ (sn << 16), o[4 * k + 3] ^ (sn & 0x80000000u));
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
}

template <int LAT, bool OUT_BF16, bool DITHER>
__global__ __launch_bounds__(kBlock) void decode_fast128(DecodeLaunch a) {
  __shared__ uint32_t sign_tab[128];
  __shared__ uint4 stage[kBlock / 64][kDec128Stage];
  __shared__ uint4 ostage[kBlock / 64][256];
  fill_sign_table(sign_tab, a.signs);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = lane & 31, r = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint4* buf = stage[wave];
  const int64_t n_groups = (a.n_tiles + kTpw - 1) / kTpw;
  const int64_t stride = (int64_t)gridDim.x * (kBlock / 64);
  int64_t g = (int64_t)blockIdx.x * (kBlock / 64) + wave;
  if (g >= n_groups) return;
  uint32_t d[16];
  Dec128In in;
  dec128_prefetch<LAT>(a, g, buf, lane);
  dec128_take<LAT>(buf, t, r, d, in);
  for (;;) {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int64_t gn = g + stride;
    const bool more = gn < n_groups;
    const int64_t gp = more ? gn : g;
    dec128_prefetch<LAT>(a, gp, buf, lane);
    dec128_group<LAT, OUT_BF16, DITHER>(a, sign_tab, g, t, r, d, in, ostage[wave]);
    __builtin_amdgcn_sched_barrier(0);
    dec128_take<LAT>(buf, t, r, d, in);
    if (!more) break;
    g = gn;
  }
}

template <int LAT, bool DITHER>
hipError_t launch_enc(const EncodeLaunch& a, hipStream_t s) {
  static int occ = 0;
  const int64_t blocks =
      persistent_grid(a.n_tiles, resident_blocks(encode_fast128<LAT, DITHER>, occ), kTpw);
  hipLaunchKernelGGL((encode_fast128<LAT, DITHER>), dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int LAT, bool OUT_BF16, bool DITHER>
hipError_t launch_dec(const DecodeLaunch& a, hipStream_t s) {
  static int occ = 0;
  const int64_t blocks =
      persistent_grid(a.n_tiles, resident_blocks(decode_fast128<LAT, OUT_BF16, DITHER>, occ), kTpw);
  hipLaunchKernelGGL((decode_fast128<LAT, OUT_BF16, DITHER>), dim3((unsigned)blocks), dim3(kBlock),
                     0, s, a);
  return hipGetLastError();
}

template <int LAT>
hipError_t launch_dec_lat(const DecodeLaunch& a, hipStream_t s) {
  return a.out_bf16 ? launch_dec<LAT, true, false>(a, s) : launch_dec<LAT, false, false>(a, s);
}

}  // namespace

bool fast128_encode_ok(const EncodeLaunch& a) {
  return a.tile == 128 && a.in_bf16 && a.coords == nullptr && !a.wide &&
         (a.lattice == 8 || !a.dither);
}

bool fast128_decode_ok(const DecodeLaunch& a) {
  return a.tile == 128 && !a.wide && (a.lattice == 8 || !a.dither);
}

hipError_t launch_encode_fast128(const EncodeLaunch& a, hipStream_t s) {
  switch (a.lattice) {
    case 8: return a.dither ? launch_enc<8, true>(a, s) : launch_enc<8, false>(a, s);
    case 4: return launch_enc<4, false>(a, s);
    case 2: return launch_enc<2, false>(a, s);
    default: return launch_enc<1, false>(a, s);
  }
}

hipError_t launch_decode_fast128(const DecodeLaunch& a, hipStream_t s) {
  switch (a.lattice) {
    case 8:
      if (a.dither)
        return a.out_bf16 ? launch_dec<8, true, true>(a, s) : launch_dec<8, false, true>(a, s);
      return launch_dec_lat<8>(a, s);
    case 4: return launch_dec_lat<4>(a, s);
    case 2: return launch_dec_lat<2>(a, s);
    default: return launch_dec_lat<1>(a, s);
  }
}

}  // namespace hq

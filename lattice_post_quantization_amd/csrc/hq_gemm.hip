// Y = W X^T straight from E8 indices (tile 256) for many vectors, on the
// bf16 matrix cores: the GEMM counterpart of hq_gemv.
//
// Passages: GitHub issue "HyperQuant ... #9", "Is your feature request
// related to a problem?" (the compressed weights must serve inference);
// [ICLR abstract] "HyperQuant: A Near-Entropy-Optimal Lattice Quantization
// Pipeline ..." (algebraic decoding of the lattice indices).
//
// As in hq_gemv, tile t of row r decodes to w = s (.) H P Delta / 32 (P = 2p,
// n = 256), and H is symmetric, so w . x_t = (Delta / 32) <P, xr_t> with
// xr_t = H (s (.) x_t).  Per 256-column slice the products P xr are a plain
// matrix product of integers |P| <= 255 (exact in bf16) with the rotated
// inputs; the rotated inputs are held as two bf16 terms hi + lo (hi the
// rounding of the fp64 rotation, lo the rounding of the rest), so each slice
// is two bf16 MFMA products with fp32 accumulation, scaled by the row's
// Delta / 32 and added to the output accumulator.
//
// One launch of each kernel covers up to kGemmMaxItems matrices that share
// m (a layer's projections).
//
// split_kernel: one wave per (vector, slice) rotates in fp64 (as hq_gemv)
// and writes xh, xl [m][cols] bf16.
// gemm_kernel: a block of W waves owns 32 W rows x 32 NF vectors and a
// range of slices (a small matrix splits its slices over several blocks,
// whose partial sums sum_kernel adds in range order; the ranges depend on
// the sizes of the whole batch); per slice the
// 256 x 32 NF hi and lo inputs go through registers (loaded one slice
// ahead) into LDS in a swizzled order so that the fragment reads hit
// distinct banks (two buffers, one barrier per slice), and each wave
// decodes its 32 rows' index bytes (one E8 block per lane and step: z7 from
// the parity of z0..z6, P = 2 z + c) into bf16 A fragments and runs
// v_mfma_f32_32x32x16_bf16 over the 16 steps of the slice.  The K order
// within a slice is permuted so that a lane reads its row's bytes 16 at a
// time next to the other half's: step s, lane half h covers block
// 4 (s / 2) + 2 h + s % 2 (B uses the same permutation).  Blocks go to the
// eight XCDs in turn; the numbering puts the blocks that share a row range
// (one per 32 NF vectors) on one XCD, one after the other, so the index
// bytes they all read come from that XCD's L2 after the first.
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_lanes.h"

namespace hq {
namespace {

using namespace fastlib;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSliceK = 256;

// Matrix of the batch that holds index g of a numbering (wave-uniform).
template <typename F>
__device__ inline int item_at(const GemmBatch& b, int64_t g, F first) {
  int i = 0;
#pragma unroll
  for (int k = 1; k < kGemmMaxItems; ++k)
    if (k < b.n && g >= first(b.it[k])) i = k;
  return i;
}

// xh / xl [v][c] for c in slice t: one wave per (vector, slice), lane l
// holding elements 4 l .. 4 l + 3; fp64 butterflies as in hq_gemv's rotation.
__global__ __launch_bounds__(256) void split_kernel(GemmBatch bt) {
  __shared__ double v[4][256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t g = (int64_t)blockIdx.x * 4 + w;
  if (g >= bt.n_split) return;
  const GemmItem& a = bt.it[item_at(bt, g, [](const GemmItem& t) { return t.split0; })];
  const int64_t slices = a.cols / kSliceK;
  const int64_t vec = (g - a.split0) / slices, t = (g - a.split0) % slices;
  const int64_t c0 = vec * a.cols + t * kSliceK + 4 * lane;
  const float4 xv = *reinterpret_cast<const float4*>(a.x + c0);
  const uint32_t sg = bt.signs[lane >> 3] >> (4 * (lane & 7));
  double e[4] = {(double)xv.x, (double)xv.y, (double)xv.z, (double)xv.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if ((sg >> i) & 1u) e[i] = -e[i];
  double p = e[0], q = e[1];
  e[0] = p + q; e[1] = p - q;
  p = e[2]; q = e[3];
  e[2] = p + q; e[3] = p - q;
  p = e[0]; q = e[2];
  e[0] = p + q; e[2] = p - q;
  p = e[1]; q = e[3];
  e[1] = p + q; e[3] = p - q;
  double* vw = v[w];
#pragma unroll
  for (int hb = 1; hb < 64; hb <<= 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[4 * lane + i] = e[i];
    wave_lds_sync();
    double o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = vw[4 * (lane ^ hb) + i];
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = (lane & hb) ? o[i] - e[i] : e[i] + o[i];
  }
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = f64_to_bf16(e[i]);
    lo[i] = f64_to_bf16(e[i] - (double)__uint_as_float(hi[i] << 16));
  }
  *reinterpret_cast<uint2*>(a.xh + c0) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
  *reinterpret_cast<uint2*>(a.xl + c0) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
}

// A fragment of one E8 block: stored bytes (z0 .. z6, t7) in d0, d1 and
// coset bit c; P_i = 2 z_i + c, and P7 = 2 z7 + c = 4 t7 + 2 parity(z0 ..
// z6) + c.  Every value is an integer of magnitude <= 255: exact in bf16.
__device__ inline bf16x8 a_fragment(uint32_t d0, uint32_t d1, uint32_t c) {
  uint32_t x = d0 ^ (d1 & 0x00FFFFFFu);
  x ^= x >> 16;
  x ^= x >> 8;
  const float cf = (float)c;
  const float c7 = (float)(c + 2u * (x & 1u));
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = fmaf((float)(int32_t)(int8_t)(d0 >> (8 * i)), 2.0f, cf);
    f[4 + i] = fmaf((float)(int32_t)(int8_t)(d1 >> (8 * i)), i == 3 ? 4.0f : 2.0f,
                    i == 3 ? c7 : cf);
  }
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2));
  return __builtin_bit_cast(bf16x8, r);
}

// One 32 x 32 x 16 bf16 matrix-core product accumulated into c.
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A lane's 128 index bytes of one slice: 16 bytes (two blocks) out of every
// 32 of its row, from offset off (the two lanes of a row read neighbouring
// 16 bytes, so an instruction touches 32 B of each of 32 rows).
__device__ inline void load_a(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* d) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 32 * i), 0, 0);
    d[4 * i] = q[0]; d[4 * i + 1] = q[1]; d[4 * i + 2] = q[2]; d[4 * i + 3] = q[3];
  }
}

// NF fragments of 32 vectors; W waves of 32 rows each.
template <int NF, int W>
__global__ __launch_bounds__(64 * W, 2) void gemm_kernel(GemmBatch bt) {
  // a slice's inputs: NF x 32 vectors x 256 k, hi and lo, as 16-byte chunks;
  // chunk (j, q) of vector j sits at slot j * 32 + (q ^ (j & 31)); two
  // buffers: the next slice's inputs, loaded into registers while this
  // slice computes, are written to one while the other is read
  constexpr int kSlots = NF * 32 * 32;
  constexpr int kPerWave = kSlots / (64 * W);   // chunks per array and lane
  __shared__ uint4 bh[2][kSlots];
  __shared__ uint4 bl[2][kSlots];
  __shared__ float dsc[W][32];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, li = lane & 31;
  // the block's matrix, then (XCD, position on it) -> (row range, slice
  // range, vector block); numbers past the matrix's blocks end at once
  const int64_t g = blockIdx.x;
  const GemmItem& a = bt.it[item_at(bt, g, [](const GemmItem& t) { return t.blk0; })];
  const int64_t local = g - a.blk0;
  const int64_t vblocks = (bt.m + 32 * NF - 1) / (32 * NF);
  const int64_t rblocks = (a.rows + 32 * W - 1) / (32 * W);
  const int64_t k = local >> 3;
  const int64_t rt = (k / vblocks) * 8 + (local & 7);
  if (rt >= rblocks * a.kchunks) return;
  const int64_t chunk = rt / rblocks;
  const int64_t row0 = (rt % rblocks) * (32 * W) + 32 * w;
  const int64_t vec0 = (k % vblocks) * (32 * NF);
  const int64_t slices = a.cols / kSliceK;
  // this block's slice range
  const int64_t t_begin = chunk * a.spc;
  const int64_t t_end = t_begin + a.spc < slices ? t_begin + a.spc : slices;

  // inputs of this block's vectors (zeros past m), indices of this wave's
  // rows (zeros past rows), per-tile words and scales
  const int64_t live_vecs = bt.m - vec0 < 32 * NF ? bt.m - vec0 : 32 * NF;
  const auto xh_rs = out_rsrc(const_cast<uint16_t*>(a.xh) + vec0 * a.cols,
                              (uint32_t)(live_vecs * a.cols * 2));
  const auto xl_rs = out_rsrc(const_cast<uint16_t*>(a.xl) + vec0 * a.cols,
                              (uint32_t)(live_vecs * a.cols * 2));
  // a wave wholly past the matrix (small matrices) gets empty ranges
  const int64_t rest = a.rows - row0;
  const int64_t live_rows = rest < 0 ? 0 : (rest < 32 ? rest : 32);
  const auto idx_rs = out_rsrc(const_cast<int8_t*>(a.idx) + row0 * a.cols,
                               (uint32_t)(live_rows * a.cols));
  const auto cw_rs = out_rsrc(const_cast<uint32_t*>(a.coset) + row0 * slices,
                              (uint32_t)(live_rows * slices * 4));
  const auto sc_rs = out_rsrc(const_cast<float*>(a.scale) + row0 * slices,
                              (uint32_t)(live_rows * slices * 4));

  // chunk i of lane (w, lane) is slot 64 (kPerWave w + i) + lane
  u32x4 nh[kPerWave], nl[kPerWave];
  auto fetch = [&](int64_t t) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int S = 64 * (kPerWave * w + i) + lane;
      const int j = S >> 5, q = (S & 31) ^ (j & 31);
      const int goff = (int)((j * a.cols + t * kSliceK + 8 * q) * 2);
      nh[i] = __builtin_amdgcn_raw_buffer_load_b128(xh_rs, goff, 0, 0);
      nl[i] = __builtin_amdgcn_raw_buffer_load_b128(xl_rs, goff, 0, 0);
    }
  };
  auto put = [&](int b) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int S = 64 * (kPerWave * w + i) + lane;
      bh[b][S] = __builtin_bit_cast(uint4, nh[i]);
      bl[b][S] = __builtin_bit_cast(uint4, nl[i]);
    }
  };
  auto tile_word = [&](__amdgpu_buffer_rsrc_t rs, int64_t t) {
    return __builtin_amdgcn_raw_buffer_load_b32(rs, (int)((li * slices + t) * 4), 0, 0);
  };

  f32x16 out[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) out[f] = (f32x16){};

  // the first slice's loads
  uint32_t dn[32];
  fetch(t_begin);
  put(0);
  uint32_t cw_n = tile_word(cw_rs, t_begin), sc_n = tile_word(sc_rs, t_begin);
  load_a(idx_rs, (uint32_t)(li * a.cols + t_begin * kSliceK + 16 * h), dn);

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int b = (int)((t - t_begin) & 1);
    // this slice's inputs are in buffer b, and every wave has read the other
    // buffer's previous slice
    __syncthreads();
    const uint32_t cw = cw_n;
    const float sc = __uint_as_float(sc_n);
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = dn[i];
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < t_end) {
      fetch(t + 1);
      cw_n = tile_word(cw_rs, t + 1);
      sc_n = tile_word(sc_rs, t + 1);
      load_a(idx_rs, (uint32_t)(li * a.cols + (t + 1) * kSliceK + 16 * h), dn);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the rows' Delta / 32, for the transpose into the output layout below
    if (h == 0) dsc[w][li] = sc * 0.03125f;

    const uint4* Bh = bh[b];
    const uint4* Bl = bl[b];
    f32x16 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = (f32x16){};
    // step s covers block 4 (s / 2) + 2 h + s % 2 of this lane half; the
    // next step's inputs and A fragment are formed before this step's
    // products are issued
    uint4 cbh[NF], cbl[NF], nbh[NF], nbl[NF];
    auto ldb = [&](int s, uint4* hh, uint4* ll) {
      const int q = 4 * (s >> 1) + 2 * h + (s & 1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int j = 32 * f + li;
        const int slot = j * 32 + (q ^ (j & 31));
        hh[f] = Bh[slot];
        ll[f] = Bl[slot];
      }
    };
    auto afr = [&](int s) {
      const int q = 4 * (s >> 1) + 2 * h + (s & 1);
      return a_fragment(d[2 * s], d[2 * s + 1], (cw >> q) & 1u);
    };
    ldb(0, cbh, cbl);
    bf16x8 af = afr(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      bf16x8 afn = af;
      if (s + 1 < 16) {
        ldb(s + 1, nbh, nbl);
        afn = afr(s + 1);
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        acc[f] = mfma32(af, __builtin_bit_cast(bf16x8, cbh[f]), acc[f]);
        acc[f] = mfma32(af, __builtin_bit_cast(bf16x8, cbl[f]), acc[f]);
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        cbh[f] = nbh[f];
        cbl[f] = nbl[f];
      }
      af = afn;
    }
    if (t + 1 < t_end) put(b ^ 1);
    // ---- out += (Delta / 32) acc; register r holds row 8 (r / 4) + 4 h + r % 4
    wave_lds_sync();
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 ds = *reinterpret_cast<const float4*>(&dsc[w][8 * g4 + 4 * h]);
      const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[f][4 * g4 + r] = fmaf(dv[r], acc[f][4 * g4 + r], out[f][4 * g4 + r]);
    }
  }

  // ---- y[vec][row] (or this range's partial sums), one element per store;
  // rows past the matrix go to an offset the hardware drops
  float* dst = a.kchunks > 1 ? a.part + chunk * bt.m * a.rows : a.y;
  const auto y_rs = out_rsrc(dst + vec0 * a.rows, (uint32_t)(live_vecs * a.rows * 4));
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t j = 32 * f + li;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int64_t r0 = row0 + 8 * g4 + 4 * h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t off = r0 + r < a.rows ? (uint32_t)((j * a.rows + r0 + r) * 4) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out[f][4 * g4 + r]), y_rs, (int)off,
                                              0, 0);
      }
    }
  }
}

// Wide tiles for many vectors: a block of eight waves (two per SIMD) owns
// 256 rows x 128 vectors; wave w owns rows 32 w .. 32 w + 31 and all 128
// vectors as four 32-vector fragments, so each step (16 k) forms one A
// fragment and reads eight B fragments for eight products: half the A
// decoding per product of gemm_kernel's 32 x 64 wave tile, at the same LDS
// reads per product.  A slice is staged as four quarters of 64 k: the
// rotated inputs (128 vectors x 64 k, hi and lo), the index bytes (256 rows
// x 64 bytes) and the slice's coset words and scales are copied by
// direct-to-LDS buffer loads into one of three buffers, two quarters ahead
// of the one computed; one barrier per quarter.  The per-slice products
// accumulate exactly as in gemm_kernel (32 matrix-core accumulations per
// slice, then out += (Delta / 32) acc), so the results obey the same bound.
//
// LDS layout of a quarter: input chunk q (8 k) of vector j at slot
// 8 j + (q ^ ((j >> 1) & 7)) of its term; 16-byte chunk c of block-row r's
// 64 index bytes at slot 4 r + (c ^ ((r >> 2) & 3)): the 16 lanes that a
// 16-byte fragment read serves together hit the 16 different 16-byte bank
// groups of gfx950's 64 banks.
constexpr int kWideRows = 256;
constexpr int kWideVecs = 128;

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt
// and lgkmcnt at their no-wait values)
constexpr int kWaitVm0 = 0x0F70, kWaitVm7 = 0x0F77;

typedef uint4 WideB[2][1024];   // a quarter's inputs: [hi, lo][slot]
typedef uint4 WideA[1024 + 128];  // a quarter's index bytes [slot], then the slice's
                                  // coset words [256] and scales [256] of the block's rows

__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(GemmBatch bt) {
  // three buffers as separate objects, so that the compiler sees that a
  // quarter's fragment reads and the loads filling another buffer do not
  // overlap
  __shared__ WideB sb0, sb1, sb2;
  __shared__ WideA sa0, sa1, sa2;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int64_t g = blockIdx.x;
  const GemmItem& a = bt.it[item_at(bt, g, [](const GemmItem& t) { return t.blk0; })];
  const int64_t local = g - a.blk0;
  const int64_t vblocks = (bt.m + kWideVecs - 1) / kWideVecs;
  const int64_t rblocks = (a.rows + kWideRows - 1) / kWideRows;
  const int64_t k = local >> 3;
  const int64_t rt = (k / vblocks) * 8 + (local & 7);
  if (rt >= rblocks * a.kchunks) return;
  const int64_t chunk = rt / rblocks;
  const int64_t rowB = (rt % rblocks) * kWideRows;
  const int64_t vec0 = (k % vblocks) * kWideVecs;
  const int64_t slices = a.cols / kSliceK;
  const int64_t t_begin = chunk * a.spc;
  const int64_t t_end = t_begin + a.spc < slices ? t_begin + a.spc : slices;
  const int nq = (int)(4 * (t_end - t_begin));

  const int64_t live_vecs = bt.m - vec0 < kWideVecs ? bt.m - vec0 : kWideVecs;
  const auto xh_rs = out_rsrc(const_cast<uint16_t*>(a.xh) + vec0 * a.cols,
                              (uint32_t)(live_vecs * a.cols * 2));
  const auto xl_rs = out_rsrc(const_cast<uint16_t*>(a.xl) + vec0 * a.cols,
                              (uint32_t)(live_vecs * a.cols * 2));
  const int64_t live_block = a.rows - rowB < kWideRows ? a.rows - rowB : kWideRows;
  const auto idx_rs = out_rsrc(const_cast<int8_t*>(a.idx) + rowB * a.cols,
                               (uint32_t)(live_block * a.cols));
  // the words of block rows 64 (w % 4) .. + 63: coset words for waves 0-3,
  // scales for waves 4-7
  const int64_t wrow = rowB + 64 * (w & 3);
  const int64_t wrest = a.rows - wrow;
  const int64_t wlive = wrest < 0 ? 0 : (wrest < 64 ? wrest : 64);
  const auto wd_rs = out_rsrc(w < 4 ? (void*)(a.coset + wrow * slices) : (void*)(a.scale + wrow * slices),
                              (uint32_t)(wlive * slices * 4));

  // Loads of quarter qq (slice t_begin + qq / 4, k offset 64 (qq % 4)), 7
  // per wave, all into LDS: two 1 KB loads of each input term, two of index
  // bytes and one of words.  Quarters past the range load the last one
  // again, so every group has the same size and the waits below are fixed
  // counts.
  auto issue = [&](int qq, WideB& B, WideA& A) {
    qq = qq < nq ? qq : nq - 1;
    const int64_t t = t_begin + qq / 4;
    const int64_t kofs = t * kSliceK + 64 * (qq & 3);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int S = 128 * w + 64 * i + lane;
      const int j = S >> 3, q = (S & 7) ^ ((j >> 1) & 7);
      const int goff = (int)((j * a.cols + kofs + 8 * q) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xh_rs, lds_ptr(&B[0][128 * w + 64 * i]), 16,
                                               goff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xl_rs, lds_ptr(&B[1][128 * w + 64 * i]), 16,
                                               goff, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int S = 128 * w + 64 * i + lane;
      const int r = S >> 2, c = (S & 3) ^ ((r >> 2) & 3);
      const int goff = (int)(r * a.cols + kofs + 16 * c);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(idx_rs, lds_ptr(&A[128 * w + 64 * i]), 16, goff,
                                               0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wd_rs, lds_ptr(&A[1024 + 16 * w]), 4,
                                             (int)((lane * slices + t) * 4), 0, 0, 0);
  };

  f32x16 out[4], acc[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    out[f] = (f32x16){};
    acc[f] = (f32x16){};
  }

  // one step's eight B fragments (block q of the quarter: vector fragment f,
  // hi and lo) and its products with the A fragment af
  auto ldb = [&](const WideB& B, int q, uint4* bf) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int j = 32 * f + li;
      const int slot = 8 * j + (q ^ ((j >> 1) & 7));
      bf[2 * f] = B[0][slot];
      bf[2 * f + 1] = B[1][slot];
    }
  };
  auto products = [&](const uint4* bf, bf16x8 af) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[f] = mfma32(af, __builtin_bit_cast(bf16x8, bf[2 * f]), acc[f]);
      acc[f] = mfma32(af, __builtin_bit_cast(bf16x8, bf[2 * f + 1]), acc[f]);
    }
  };

  // quarter qq from buffers (B, A); quarter qq + 2 is loaded into (Bn, An)
  auto quarter = [&](int qq, const WideB& B, const WideA& A, WideB& Bn, WideA& An) {
    // this wave's loads of quarter qq are complete (vector memory loads
    // complete in order; only quarter qq + 1's are younger), then every
    // wave's are, and every wave has finished quarter qq - 1, whose
    // buffers quarter qq + 2 refills
    __builtin_amdgcn_s_waitcnt(kWaitVm7);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    issue(qq + 2, Bn, An);
    if (qq >= nq) return;
    const int u = qq & 3;
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(&A[1024]);
    const uint32_t cw = wl[32 * w + li];
    const int row = 32 * w + li;
    // this lane half's blocks 4 v + 2 h + {0, 1} for steps 2 v, 2 v + 1
    // (index chunk 2 v + h of its row)
    const uint4 ab0 = A[4 * row + ((0 + h) ^ ((row >> 2) & 3))];
    const uint4 ab1 = A[4 * row + ((2 + h) ^ ((row >> 2) & 3))];
    uint4 bc[8], bn[8];
    ldb(B, 2 * h, bc);
    // steps 0..3: the next step's B fragments are read, and its A fragment
    // formed, before this step's products are issued
    bf16x8 af = a_fragment(ab0.x, ab0.y, (cw >> (8 * u + 2 * h)) & 1u);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int qn = 4 * ((s + 1) >> 1) + 2 * h + ((s + 1) & 1);
      bf16x8 afn = af;
      if (s < 3) {
        ldb(B, qn, bn);
        const uint4& ab = (s + 1) < 2 ? ab0 : ab1;
        afn = a_fragment((s + 1) & 1 ? ab.z : ab.x, (s + 1) & 1 ? ab.w : ab.y,
                         (cw >> (8 * u + qn)) & 1u);
      }
      products(bc, af);
      // each product issued with one fragment read and a few of the next A
      // fragment's instructions, so that the matrix core, the LDS and the
      // VALU work side by side
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) bc[i] = bn[i];
      af = afn;
    }
    if (u == 3) {
      // ---- out += (Delta / 32) acc; acc register i holds row
      // 8 (i / 4) + 4 h + i % 4 of the wave
      const float* sl = reinterpret_cast<const float*>(wl + 256 + 32 * w);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 ds = *reinterpret_cast<const float4*>(&sl[8 * g4 + 4 * h]);
        const float dv[4] = {ds.x * 0.03125f, ds.y * 0.03125f, ds.z * 0.03125f, ds.w * 0.03125f};
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            out[f][4 * g4 + i] = fmaf(dv[i], acc[f][4 * g4 + i], out[f][4 * g4 + i]);
            acc[f][4 * g4 + i] = 0.0f;
          }
      }
    }
  };

  issue(0, sb0, sa0);
  issue(1, sb1, sa1);
  for (int q0 = 0; q0 < nq; q0 += 3) {
    quarter(q0, sb0, sa0, sb2, sa2);
    quarter(q0 + 1, sb1, sa1, sb0, sa0);
    quarter(q0 + 2, sb2, sa2, sb1, sa1);
  }
  // no load into this block's LDS may land after the block ends
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- y[vec][row] (or this range's partial sums); rows past the matrix
  // go to an offset the hardware drops (one buffer per 32-vector fragment
  // keeps the 32-bit offsets in range)
  const int64_t row0 = rowB + 32 * w;
  float* dst = a.kchunks > 1 ? a.part + chunk * bt.m * a.rows : a.y;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int64_t fv = live_vecs - 32 * f;
    const auto y_rs = out_rsrc(dst + (vec0 + 32 * f) * a.rows,
                               (uint32_t)((fv < 0 ? 0 : (fv < 32 ? fv : 32)) * a.rows * 4));
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int64_t r0 = row0 + 8 * g4 + 4 * h;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off =
            r0 + i < a.rows ? (uint32_t)((li * a.rows + r0 + i) * 4) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out[f][4 * g4 + i]), y_rs,
                                              (int)off, 0, 0);
      }
    }
  }
}

// y = the sum of the ranges' partial sums, in range order (matrices with
// more than one range)
__global__ __launch_bounds__(256) void sum_kernel(GemmBatch bt) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= bt.n_sum) return;
  // the element's matrix (lanes may differ: a plain scan)
  int k = 0;
  for (int j = 1; j < bt.n; ++j)
    if (bt.it[j].kchunks > 1 && g >= bt.it[j].sum0) k = j;
  const GemmItem& a = bt.it[k];
  const int64_t n = (int64_t)bt.m * a.rows;
  const int64_t i = g - a.sum0;
  float s = a.part[i];
  for (int64_t c = 1; c < a.kchunks; ++c) s += a.part[c * n + i];
  a.y[i] = s;
}

template <int NF, int W>
void launch_nf(const GemmBatch& b, hipStream_t s) {
  hipLaunchKernelGGL((gemm_kernel<NF, W>), dim3((unsigned)b.n_blocks), dim3(64 * W), 0, s, b);
}

// Block shapes by m: one 32-vector fragment per block for m <= 32 (4 waves
// of 32 rows, two blocks per CU); two up to m = 192 (8 waves of 32 rows,
// one block per CU: the double-buffered inputs take 128 KiB of LDS); above,
// the wide tiles (8 waves of 32 rows x 128 vectors, one block per CU),
// which measured faster from m = 256 on (a Llama-shaped layer: 328 against
// 394 us at m = 256, 618 against 684 us at m = 512) and slower below
// (264 against 219 us at m = 128).
constexpr int32_t kWideMinM = 193;
int shape_for(int32_t m) { return m <= 32 ? 1 : (m < kWideMinM ? 2 : 3); }
int64_t vecs_per_block(int shape) { return shape == 1 ? 32 : (shape == 2 ? 64 : kWideVecs); }
int64_t rows_per_block(int shape) { return shape == 1 ? 128 : 256; }
int64_t threads_per_block(int shape) { return shape == 1 ? 256 : 512; }
int64_t slots_for(int shape) { return shape == 1 ? 512 : 256; }

}  // namespace

// Slice ranges of a group: one length L (at most 16 slices) for the whole
// group, the longest that still gives every CU slot a block (512 slots of
// 4 waves, 256 of 8); a matrix with more slices than L splits them into
// ceil(slices / L) ranges of near-equal length.  Few ranges keep the
// partial sums (written and read back once) small next to the index bytes.
void gemm_plan(GemmBatch& b) {
  const int shape = shape_for(b.m);
  const int64_t vpb = vecs_per_block(shape), rpb = rows_per_block(shape);
  const int64_t vblocks = (b.m + vpb - 1) / vpb;
  const int64_t slots = slots_for(shape);
  int64_t len = 16;
  for (; len > 1; --len) {
    int64_t blocks = 0;
    for (int i = 0; i < b.n; ++i) {
      const int64_t slices = b.it[i].cols / kSliceK;
      blocks += (b.it[i].rows + rpb - 1) / rpb * vblocks * ((slices + len - 1) / len);
    }
    if (blocks >= slots) break;
  }
  for (int i = 0; i < b.n; ++i) {
    GemmItem& it = b.it[i];
    const int64_t slices = it.cols / kSliceK;
    it.kchunks = (slices + len - 1) / len;
    // at most kGemmMaxRanges ranges (longer ranges for very wide matrices)
    if (it.kchunks > kGemmMaxRanges) it.kchunks = kGemmMaxRanges;
    it.spc = (slices + it.kchunks - 1) / it.kchunks;
    it.kchunks = (slices + it.spc - 1) / it.spc;
  }
}

bool gemm_fits_launch(const GemmBatch& b) {
  const int shape = shape_for(b.m);
  const int64_t vpb = vecs_per_block(shape), rpb = rows_per_block(shape);
  const int64_t vblocks = (b.m + vpb - 1) / vpb;
  int64_t blocks = 0, split = 0, sum = 0;
  for (int i = 0; i < b.n; ++i) {
    const GemmItem& it = b.it[i];
    const int64_t tasks = (it.rows + rpb - 1) / rpb * it.kchunks;
    blocks += (tasks + 7) / 8 * 8 * vblocks;
    split += (int64_t)b.m * (it.cols / kSliceK);
    if (it.kchunks > 1) sum += (int64_t)b.m * it.rows;
  }
  // every grid below 2^32 work-items
  const int64_t lim = (int64_t)1 << 32;
  return blocks * threads_per_block(shape) < lim && (split + 3) / 4 * 256 < lim &&
         (sum + 255) / 256 * 256 < lim;
}

size_t gemm_item_workspace(const GemmItem& it, int32_t m) {
  return (size_t)4 * (size_t)m * (size_t)it.cols +
         (it.kchunks > 1 ? (size_t)4 * (size_t)it.kchunks * (size_t)m * (size_t)it.rows : 0);
}

void gemm_layout(GemmBatch& b, char* workspace) {
  const int shape = shape_for(b.m);
  const int64_t rpb = rows_per_block(shape), vpb = vecs_per_block(shape);
  const int64_t vblocks = (b.m + vpb - 1) / vpb;
  gemm_plan(b);
  b.n_blocks = b.n_split = b.n_sum = 0;
  for (int i = 0; i < b.n; ++i) {
    GemmItem& it = b.it[i];
    const size_t half = (size_t)2 * (size_t)b.m * (size_t)it.cols;
    it.xh = reinterpret_cast<uint16_t*>(workspace);
    it.xl = reinterpret_cast<uint16_t*>(workspace + half);
    it.part = it.kchunks > 1 ? reinterpret_cast<float*>(workspace + 2 * half) : nullptr;
    workspace += gemm_item_workspace(it, b.m);
    // blocks: (row ranges x slice ranges) rounded up to the eight XCDs,
    // times the vector blocks
    const int64_t tasks = (it.rows + rpb - 1) / rpb * it.kchunks;
    it.blk0 = b.n_blocks;
    it.split0 = b.n_split;
    it.sum0 = b.n_sum;
    b.n_blocks += (tasks + 7) / 8 * 8 * vblocks;
    b.n_split += (int64_t)b.m * (it.cols / kSliceK);
    if (it.kchunks > 1) b.n_sum += (int64_t)b.m * it.rows;
  }
  for (int i = b.n; i < kGemmMaxItems; ++i) b.it[i] = b.it[0];
}

hipError_t launch_gemm(const GemmBatch& b, hipStream_t s) {
  hipLaunchKernelGGL(split_kernel, dim3((unsigned)((b.n_split + 3) / 4)), dim3(256), 0, s, b);
  const int shape = shape_for(b.m);
  if (shape == 1)
    launch_nf<1, 4>(b, s);
  else if (shape == 2)
    launch_nf<2, 8>(b, s);
  else
    hipLaunchKernelGGL(gemm_wide_kernel, dim3((unsigned)b.n_blocks), dim3(512), 0, s, b);
  if (b.n_sum > 0)
    hipLaunchKernelGGL(sum_kernel, dim3((unsigned)((b.n_sum + 255) / 256)), dim3(256), 0, s, b);
  return hipGetLastError();
}

}  // namespace hq

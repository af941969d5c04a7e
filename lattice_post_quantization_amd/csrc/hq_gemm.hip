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
// split_kernel: one wave per (vector, slice) rotates in fp64 (as hq_gemv)
// and writes xh, xl [m][cols] bf16.
// gemm_kernel: a block of 4 waves owns 128 rows x 32 NF vectors and a range
// of slices (a small matrix splits its slices over several blocks, whose
// partial sums sum_kernel adds in range order); per slice
// it stages the 256 x 32 NF hi and lo inputs in LDS (direct-to-LDS loads in
// a swizzled order so that the fragment reads hit distinct banks), each wave
// decodes its 32 rows' index bytes (one E8 block per lane and step: z7 from
// the parity of z0..z6, P = 2 z + c) into bf16 A fragments and runs
// v_mfma_f32_32x32x16_bf16 over the 16 steps of the slice.  The K order
// within a slice is permuted so that a lane's 16 blocks are its row's
// contiguous 128 bytes: step s, lane half h covers block 16 h + s (B uses
// the same permutation).
#include "hq.h"
#include "hq_device.h"
#include "hq_internal.h"
#include "hq_lanes.h"

namespace hq {
namespace {

using namespace fastlib;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmRows = 128;      // rows per block (4 waves x 32)
constexpr int kSliceK = 256;

// xh / xl [v][c] for c in slice t: one wave per (vector, slice), lane l
// holding elements 4 l .. 4 l + 3; fp64 butterflies as in hq_gemv's rotation.
__global__ __launch_bounds__(256) void split_kernel(GemmLaunch a) {
  __shared__ double v[4][256];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t slices = a.cols / kSliceK;
  const int64_t g = (int64_t)blockIdx.x * 4 + w;
  if (g >= (int64_t)a.m * slices) return;
  const int64_t vec = g / slices, t = g % slices;
  const int64_t c0 = vec * a.cols + t * kSliceK + 4 * lane;
  const float4 xv = *reinterpret_cast<const float4*>(a.x + c0);
  const uint32_t sg = a.signs[lane >> 3] >> (4 * (lane & 7));
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
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)f[i];
  return r;
}

// One 32 x 32 x 16 bf16 matrix-core product accumulated into c.
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from offset goff of rs into LDS at dst + 16 lane (a
// plain function: written directly in the kernel template, the builtin keeps
// the host pass from instantiating the template's launch stub).
__device__ inline void to_lds16(__amdgpu_buffer_rsrc_t rs, uint4* dst, int goff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(dst), 16, goff, 0, 0, 0);
}

// A lane's 128 index bytes of one slice (its row, its half), from offset off.
__device__ inline void load_a(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t* d) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + 16 * i), 0, 0);
    d[4 * i] = q[0]; d[4 * i + 1] = q[1]; d[4 * i + 2] = q[2]; d[4 * i + 3] = q[3];
  }
}

template <int NF>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmLaunch a) {
  // per slice: NF fragments of 32 vectors x 256 k, hi and lo, 16-byte chunks;
  // chunk (j, q) of vector j (0 .. 32 NF) sits at slot j * 32 + (q ^ (j & 31))
  __shared__ uint4 bh[NF * 32 * 32];
  __shared__ uint4 bl[NF * 32 * 32];
  __shared__ float dsc[4][32];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, li = lane & 31;
  const int64_t row0 = (int64_t)blockIdx.x * kGemmRows + 32 * w;
  const int64_t vec0 = (int64_t)blockIdx.y * (32 * NF);
  const int64_t slices = a.cols / kSliceK;
  // this block's slice range
  const int64_t t_begin = (int64_t)blockIdx.z * a.spc;
  const int64_t t_end = t_begin + a.spc < slices ? t_begin + a.spc : slices;

  // inputs of this block's vectors (zeros past m), indices of this wave's
  // rows (zeros past rows), per-tile words and scales
  const auto xh_rs = out_rsrc(const_cast<uint16_t*>(a.xh) + vec0 * a.cols,
                              (uint32_t)((a.m - vec0 < 32 * NF ? a.m - vec0 : 32 * NF) * a.cols * 2));
  const auto xl_rs = out_rsrc(const_cast<uint16_t*>(a.xl) + vec0 * a.cols,
                              (uint32_t)((a.m - vec0 < 32 * NF ? a.m - vec0 : 32 * NF) * a.cols * 2));
  const int64_t live_rows = a.rows - row0 < 32 ? a.rows - row0 : 32;
  const auto idx_rs = out_rsrc(const_cast<int8_t*>(a.idx) + row0 * a.cols,
                               (uint32_t)(live_rows * a.cols));
  const auto cw_rs = out_rsrc(const_cast<uint32_t*>(a.coset) + row0 * slices,
                              (uint32_t)(live_rows * slices * 4));
  const auto sc_rs = out_rsrc(const_cast<float*>(a.scale) + row0 * slices,
                              (uint32_t)(live_rows * slices * 4));

  f32x16 out[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) out[f] = (f32x16){};

  uint32_t dn[32];
  load_a(idx_rs, (uint32_t)(li * a.cols + t_begin * kSliceK + 128 * h), dn);

  for (int64_t t = t_begin; t < t_end; ++t) {
    // ---- stage the slice's inputs: instruction i of wave w fills slots
    // 64 (4 NF w + i) + lane (4 NF instructions per array and wave)
    __syncthreads();   // the previous slice's fragments have been read
#pragma unroll
    for (int i = 0; i < NF * 4; ++i) {
      const int S = 64 * (NF * 4 * w + i) + lane;   // slot
      const int j = S >> 5, q = (S & 31) ^ (j & 31);
      const int goff = (int)((j * a.cols + t * kSliceK + 8 * q) * 2);
      to_lds16(xh_rs, bh + 64 * (NF * 4 * w + i), goff);
      to_lds16(xl_rs, bl + 64 * (NF * 4 * w + i), goff);
    }
    const uint32_t cw = __builtin_amdgcn_raw_buffer_load_b32(cw_rs, (int)((li * slices + t) * 4), 0, 0);
    const float sc = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(sc_rs, (int)((li * slices + t) * 4), 0, 0));
    uint32_t d[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) d[i] = dn[i];
    __builtin_amdgcn_sched_barrier(0);
    // the next slice's index bytes are the last loads issued: the wait below
    // leaves them in flight during this slice
    if (t + 1 < t_end) load_a(idx_rs, (uint32_t)(li * a.cols + (t + 1) * kSliceK + 128 * h), dn);
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < t_end)
      __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (h == 0) dsc[w][li] = sc * 0.03125f;
    __syncthreads();

    f32x16 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = (f32x16){};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t c = (cw >> (16 * h + s)) & 1u;
      const bf16x8 af = a_fragment(d[2 * s], d[2 * s + 1], c);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int j = 32 * f + li, q = 16 * h + s;
        const int slot = j * 32 + (q ^ (j & 31));
        const bf16x8 b_hi = __builtin_bit_cast(bf16x8, bh[slot]);
        const bf16x8 b_lo = __builtin_bit_cast(bf16x8, bl[slot]);
        acc[f] = mfma32(af, b_hi, acc[f]);
        acc[f] = mfma32(af, b_lo, acc[f]);
      }
    }
    // ---- out += (Delta / 32) acc; register r holds row 8 (r / 4) + 4 h + r % 4
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

  // ---- y[vec][row]: four consecutive rows per 16-byte store (dropped past
  // the matrix: rows past a.rows, vectors past m)
  // y, or this range's partial sums
  const int64_t live_vecs = a.m - vec0 < 32 * NF ? a.m - vec0 : 32 * NF;
  float* dst = a.kchunks > 1 ? a.part + (int64_t)blockIdx.z * a.m * a.rows : a.y;
  const auto y_rs = out_rsrc(dst + vec0 * a.rows, (uint32_t)(live_vecs * a.rows * 4));
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t j = 32 * f + li;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int64_t r0 = row0 + 8 * g4 + 4 * h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // rows past the matrix go to an offset the hardware drops
        const uint32_t off = r0 + r < a.rows ? (uint32_t)((j * a.rows + r0 + r) * 4) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out[f][4 * g4 + r]), y_rs, (int)off,
                                              0, 0);
      }
    }
  }
}

// y = the sum of the ranges' partial sums, in range order
__global__ __launch_bounds__(256) void sum_kernel(GemmLaunch a) {
  const int64_t n = (int64_t)a.m * a.rows;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = a.part[i];
  for (int64_t c = 1; c < a.kchunks; ++c) s += a.part[c * n + i];
  a.y[i] = s;
}

template <int NF>
void launch_nf(const GemmLaunch& a, hipStream_t s) {
  const int64_t row_blocks = (a.rows + kGemmRows - 1) / kGemmRows;
  const int64_t vec_blocks = (a.m + 32 * NF - 1) / (32 * NF);
  hipLaunchKernelGGL((gemm_kernel<NF>),
                     dim3((unsigned)row_blocks, (unsigned)vec_blocks, (unsigned)a.kchunks),
                     dim3(256), 0, s, a);
}

}  // namespace

void gemm_plan(int64_t rows, int64_t cols, int32_t m, int64_t& kchunks, int64_t& spc) {
  const int nf = m <= 32 ? 1 : 2;
  const int64_t base = ((rows + kGemmRows - 1) / kGemmRows) * ((m + 32 * nf - 1) / (32 * nf));
  const int64_t slices = cols / kSliceK;
  int64_t k = (1024 + base - 1) / base;
  k = k < 1 ? 1 : (k > slices ? slices : k);
  spc = (slices + k - 1) / k;
  kchunks = (slices + spc - 1) / spc;
}

size_t gemm_workspace(int64_t rows, int64_t cols, int32_t m) {
  int64_t kchunks, spc;
  gemm_plan(rows, cols, m, kchunks, spc);
  return (size_t)4 * (size_t)m * (size_t)cols +
         (kchunks > 1 ? (size_t)4 * (size_t)kchunks * (size_t)m * (size_t)rows : 0);
}

hipError_t launch_gemm(const GemmLaunch& a, hipStream_t s) {
  const int64_t splits = (int64_t)a.m * (a.cols / kSliceK);
  hipLaunchKernelGGL(split_kernel, dim3((unsigned)((splits + 3) / 4)), dim3(256), 0, s, a);
  if (a.m <= 32)
    launch_nf<1>(a, s);
  else
    launch_nf<2>(a, s);
  if (a.kchunks > 1) {
    const int64_t n = (int64_t)a.m * a.rows;
    hipLaunchKernelGGL(sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace hq
